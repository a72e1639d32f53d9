// CPU checks of the address helpers the GPU kernels use (moe_expert_layer_top_amd/csrc/addr.h).
#include <cstdint>
#include <cstdio>
#include <initializer_list>

#include "addr.h"

static int failures = 0;

static void expect(bool ok, const char* what) {
  if (!ok) {
    std::printf("FAILED: %s\n", what);
    ++failures;
  }
}

int main() {
  using moe::join_u32_halves;
  using moe::lane_offsets_fit_u32;
  // readfirstlane yields a signed int: a low half with bit 31 set is negative
  const int lo_neg = static_cast<int>(0x80001234u);
  expect(join_u32_halves(lo_neg, 0x7f) == 0x0000007f80001234ULL, "low half with bit 31 set");
  expect(join_u32_halves(-1, 1) == 0x00000001ffffffffULL, "low half all ones");
  expect(join_u32_halves(0, static_cast<int>(0xffff8000u)) == 0xffff800000000000ULL, "high half with bit 31 set");
  expect(join_u32_halves(0x12345678u, 0x9abcdef0u) == 0x9abcdef012345678ULL, "unsigned halves");
  // the form that once faulted, for contrast: widening the signed low half sign-extends it
  const uint64_t wrong = (static_cast<uint64_t>(0x7fu) << 32) | static_cast<uint64_t>(static_cast<int64_t>(lo_neg));
  expect(wrong != join_u32_halves(lo_neg, 0x7f), "the sign-extending form differs");
  // a typical device address of a scale tensor: every 32-bit split round-trips
  for (uint64_t a : {0x00007f2a80000000ULL, 0x00007fffffffff00ULL, 0x0000100000000004ULL}) {
    expect(join_u32_halves(static_cast<int>(static_cast<uint32_t>(a)), static_cast<int>(static_cast<uint32_t>(a >> 32))) == a,
           "address round trip");
  }
  // 32-bit lane offsets: rows * cols * bytes <= 2^32 - 1
  expect(lane_offsets_fit_u32(1, 1, 0xffffffffLL), "2^32 - 1 bytes fit");
  expect(!lane_offsets_fit_u32(1, 1, 0x100000000LL), "2^32 bytes do not");
  expect(lane_offsets_fit_u32(2, 0x7fffffffLL, 1), "2^32 - 2 bytes of bf16 fit");
  expect(!lane_offsets_fit_u32(2, 0x80000000LL, 1), "2^32 bytes of bf16 do not");
  expect(lane_offsets_fit_u32(1, (1LL << 25) - 1, 128), "2^32 - 128 bytes (H = 128) fit");
  expect(!lane_offsets_fit_u32(1, 1LL << 25, 128), "2^25 rows of 128 bytes do not");
  expect(!lane_offsets_fit_u32(2, 1LL << 18, 8192), "2^18 rows of 16 KB do not");
  expect(lane_offsets_fit_u32(2, (1LL << 18) - 1, 8192), "2^18 - 1 rows of 16 KB fit");
  expect(lane_offsets_fit_u32(2, 8192, 7168), "the 8192-token bf16 prefill fits");
  expect(lane_offsets_fit_u32(1, 16384, 7168), "the 16384-token fp8 codes fit");
  expect(!lane_offsets_fit_u32(2, 1LL << 40, 1LL << 40), "no 64-bit overflow");
  expect(lane_offsets_fit_u32(2, 0, 7168), "no rows");
  expect(!lane_offsets_fit_u32(0, 1, 1), "element size must be positive");
  if (failures) return 1;
  std::printf("all address checks passed\n");
  return 0;
}
