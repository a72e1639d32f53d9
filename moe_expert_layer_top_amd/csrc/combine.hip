// Un-permute + weighted combine, and the fp32 kernels of the MoE layer (gfx950).
//
// [R1P] = page "CANN/cann-recipes-infer: DeepSeek-R1 prefill optimization".
// [R1P §MoE deployment strategy optimization]: finalize-routing restores the
// original token order through expanded_row_idx and, in the same op, forms the
// weighted sum of the routed-expert rows plus the shared-expert output.

#include "common.h"
#include "kernels.h"

namespace moe {

// out[t] = skip[t] + sum_j w[t, j] * y[eri[t*k + j]], fp32 accumulation, one rounding.
// One thread per (token, 16-byte vector of the row): the k routed rows and the skip row
// are loaded before the first FMA (all k + 1 loads in flight per thread), then
// accumulated in slot order j = 0 .. k-1 starting from the skip value.  KC > 0 fixes
// k at compile time (fully unrolled); KC = 0 handles any k in chunks of 8.
template <bool BF16, int KC>
__global__ __launch_bounds__(256) void finalize_kernel(const uint8_t* __restrict__ y,
                                                       const uint8_t* __restrict__ skip,
                                                       const float* __restrict__ w,
                                                       const int32_t* __restrict__ eri,
                                                       uint8_t* __restrict__ out, int T, int H,
                                                       int k_rt) {
  constexpr int EB = BF16 ? 2 : 4;
  constexpr int PER = 16 / EB;  // elements per 16-byte vector
  const int k = KC > 0 ? KC : k_rt;
  const long long row_bytes = static_cast<long long>(H) * EB;
  const int nvec = static_cast<int>(row_bytes / 16);
  const long long id = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (id >= static_cast<long long>(T) * nvec) return;
  const int t = static_cast<int>(id / nvec);
  const int v = static_cast<int>(id % nvec);

  float acc[PER];
  auto unpack_add = [&](uint4 q, float wj, bool first_skip) __attribute__((always_inline)) {
    const uint32_t qw[4] = {q.x, q.y, q.z, q.w};
    if constexpr (BF16) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float lo = __uint_as_float(qw[i] << 16), hi = __uint_as_float(qw[i] & 0xffff0000u);
        if (first_skip) { acc[2 * i] = lo; acc[2 * i + 1] = hi; }
        else { acc[2 * i] = fmaf(wj, lo, acc[2 * i]); acc[2 * i + 1] = fmaf(wj, hi, acc[2 * i + 1]); }
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float f = __uint_as_float(qw[i]);
        acc[i] = first_skip ? f : fmaf(wj, f, acc[i]);
      }
    }
  };

  uint4 sv = make_uint4(0u, 0u, 0u, 0u);
  if (skip) sv = reinterpret_cast<const uint4*>(skip + t * row_bytes)[v];
  const int32_t* er = eri + static_cast<long long>(t) * k;
  const float* wr = w ? w + static_cast<long long>(t) * k : nullptr;
  constexpr int CH = KC > 0 ? KC : 8;
  bool first = true;
  for (int j0 = 0; j0 < k; j0 += CH) {
    uint4 yv[CH];
    float wv[CH];
    bool ok[CH];
#pragma unroll
    for (int jj = 0; jj < CH; ++jj) {
      const int j = j0 + jj;
      const int32_t r = j < k ? er[j] : -1;
      ok[jj] = r >= 0;
      wv[jj] = (wr && j < k) ? wr[j] : 1.0f;
      if (ok[jj]) {
        const u32x4 q = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(y + r * row_bytes) + v);
        yv[jj] = make_uint4(q.x, q.y, q.z, q.w);
      } else {
        yv[jj] = make_uint4(0u, 0u, 0u, 0u);
      }
    }
    if (first) {
      unpack_add(sv, 1.0f, true);
      first = false;
    }
#pragma unroll
    for (int jj = 0; jj < CH; ++jj)
      if (ok[jj]) unpack_add(yv[jj], wv[jj], false);
  }
  if (first) unpack_add(sv, 1.0f, true);
  uint4 o;
  if constexpr (BF16) {
    o = make_uint4(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]),
                   pack_bf16x2(acc[4], acc[5]), pack_bf16x2(acc[6], acc[7]));
  } else {
    o = make_uint4(__float_as_uint(acc[0]), __float_as_uint(acc[1]), __float_as_uint(acc[2]),
                   __float_as_uint(acc[3]));
  }
  __builtin_nontemporal_store(u32x4{o.x, o.y, o.z, o.w}, reinterpret_cast<u32x4*>(out + t * row_bytes) + v);
}

template <bool BF16>
hipError_t finalize_go(const void* y, const void* skip, const float* w, const int32_t* eri,
                       void* out, int T, int H, int k, hipStream_t st) {
  const long long n = static_cast<long long>(T) * (static_cast<long long>(H) * (BF16 ? 2 : 4) / 16);
  const unsigned grid = static_cast<unsigned>((n + 255) / 256);
  const auto* yb = static_cast<const uint8_t*>(y);
  const auto* sb = static_cast<const uint8_t*>(skip);
  auto* ob = static_cast<uint8_t*>(out);
  switch (k) {
    case 1: finalize_kernel<BF16, 1><<<grid, 256, 0, st>>>(yb, sb, w, eri, ob, T, H, k); break;
    case 2: finalize_kernel<BF16, 2><<<grid, 256, 0, st>>>(yb, sb, w, eri, ob, T, H, k); break;
    case 4: finalize_kernel<BF16, 4><<<grid, 256, 0, st>>>(yb, sb, w, eri, ob, T, H, k); break;
    case 6: finalize_kernel<BF16, 6><<<grid, 256, 0, st>>>(yb, sb, w, eri, ob, T, H, k); break;
    case 8: finalize_kernel<BF16, 8><<<grid, 256, 0, st>>>(yb, sb, w, eri, ob, T, H, k); break;
    default: finalize_kernel<BF16, 0><<<grid, 256, 0, st>>>(yb, sb, w, eri, ob, T, H, k); break;
  }
  return hipGetLastError();
}

hipError_t launch_finalize(const void* y, const void* skip, const float* w, const int32_t* eri,
                           void* out, int T, int H, int k, int act_bytes, hipStream_t st) {
  if (T == 0) return hipSuccess;
  if (static_cast<long long>(T) * H * act_bytes / 16 >= (1LL << 31) * 256LL) return hipErrorInvalidValue;
  return act_bytes == 2 ? finalize_go<true>(y, skip, w, eri, out, T, H, k, st)
                        : finalize_go<false>(y, skip, w, eri, out, T, H, k, st);
}

// ------------------------------------------------------------------ fp32 path
// The fp32 workload is a correctness-sized layer; on gfx950 the fp32 matrix and
// vector peaks are equal, so plain FMA kernels are used.  One thread per output.

// C[M, N] = A[M, K] . B[N, K]^T
__global__ __launch_bounds__(256) void gemm_nt_f32_kernel(const float* __restrict__ A,
                                                          const float* __restrict__ B,
                                                          float* __restrict__ C, int M, int N,
                                                          int K) {
  const long long id = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (id >= static_cast<long long>(M) * N) return;
  const int m = static_cast<int>(id / N), n = static_cast<int>(id % N);
  const float* a = A + static_cast<long long>(m) * K;
  const float* b = B + static_cast<long long>(n) * K;
  float s = 0.f;
  for (int kk = 0; kk < K; ++kk) s = fmaf(a[kk], b[kk], s);
  C[id] = s;
}

hipError_t launch_gemm_nt_f32(const float* A, const float* B, float* C, int M, int N, int K,
                              hipStream_t st) {
  const long long n = static_cast<long long>(M) * N;
  if (n == 0) return hipSuccess;
  gemm_nt_f32_kernel<<<static_cast<unsigned>((n + 255) / 256), 256, 0, st>>>(A, B, C, M, N, K);
  return hipGetLastError();
}

__device__ __forceinline__ int group_of_row(const int32_t* offsets, int G, int r) {
  int lo = 0, hi = G;  // offsets[lo] <= r < offsets[hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (offsets[mid] <= r) lo = mid;
    else hi = mid;
  }
  return lo;
}

// h[r, c] = silu(a[r] . W1_g[c]) * (a[r] . W3_g[c]) for rows r < offsets[G]
__global__ __launch_bounds__(256) void ffn1_f32_kernel(const float* __restrict__ a,
                                                       const int32_t* __restrict__ offsets, int G,
                                                       int R_max, const float* __restrict__ w13,
                                                       float* __restrict__ h, int H, int I) {
  const long long id = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (id >= static_cast<long long>(R_max) * I) return;
  const int r = static_cast<int>(id / I), c = static_cast<int>(id % I);
  if (offsets && r >= offsets[G]) return;
  const int g = offsets ? group_of_row(offsets, G, r) : 0;
  const float* ar = a + static_cast<long long>(r) * H;
  const float* wg = w13 + (static_cast<long long>(g) * 2 * I + c) * H;
  const float* wu = w13 + (static_cast<long long>(g) * 2 * I + I + c) * H;
  float sg = 0.f, su = 0.f;
  for (int kk = 0; kk < H; ++kk) {
    sg = fmaf(ar[kk], wg[kk], sg);
    su = fmaf(ar[kk], wu[kk], su);
  }
  h[id] = sg / (1.0f + expf(-sg)) * su;
}

// y[r, c] = h[r] . W2_g[c]
__global__ __launch_bounds__(256) void ffn2_f32_kernel(const float* __restrict__ h,
                                                       const int32_t* __restrict__ offsets, int G,
                                                       int R_max, const float* __restrict__ w2,
                                                       float* __restrict__ y, int H, int I) {
  const long long id = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (id >= static_cast<long long>(R_max) * H) return;
  const int r = static_cast<int>(id / H), c = static_cast<int>(id % H);
  if (offsets && r >= offsets[G]) return;
  const int g = offsets ? group_of_row(offsets, G, r) : 0;
  const float* hr = h + static_cast<long long>(r) * I;
  const float* wr = w2 + (static_cast<long long>(g) * H + c) * I;
  float s = 0.f;
  for (int kk = 0; kk < I; ++kk) s = fmaf(hr[kk], wr[kk], s);
  y[id] = s;
}

hipError_t launch_grouped_ffn_f32(const float* a, const int32_t* offsets, int G, int R_max,
                                  const float* w13, const float* w2, float* h, float* y, int H,
                                  int I, hipStream_t st) {
  if (R_max == 0) return hipSuccess;
  const long long n1 = static_cast<long long>(R_max) * I;
  ffn1_f32_kernel<<<static_cast<unsigned>((n1 + 255) / 256), 256, 0, st>>>(a, offsets, G, R_max,
                                                                            w13, h, H, I);
  const long long n2 = static_cast<long long>(R_max) * H;
  ffn2_f32_kernel<<<static_cast<unsigned>((n2 + 255) / 256), 256, 0, st>>>(h, offsets, G, R_max,
                                                                            w2, y, H, I);
  return hipGetLastError();
}

}  // namespace moe
