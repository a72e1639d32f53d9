// Grouped GEMM on gfx950 matrix cores for the MoE experts and the gate.
//
// [MND] = page "Lower latency and higher throughput with multi-node DeepSeek
//         deployment".  [MND §Roofline / GroupGEMM]: g groups, group i has m_i
// rows and multiplies [m_i, k] x [k, n] -> [m_i, n].  Here group g is one expert
// and its rows are a contiguous slice of the expert-sorted activations.
//
// Design (one kernel template, several tile shapes):
//   * Work unit = (expert, row slice of at most BM rows) x (N tile) x (K split).
//     The unit table is built on the device from the routed counts
//     ([MND §Quantization]: kernels read the number of tokens per expert rather
//     than sizing work by the buffer bound), so no count ever crosses to the host.
//     An expert's rows are cut into ceil(n/BM) near-equal slices, so a prefill
//     expert (n <= BM) streams its weight panel from HBM exactly once.
//   * Workgroups are dealt round-robin to the 8 XCDs.  The planner cuts the unit table
//     into one contiguous, cost-balanced chunk per XCD; an XCD's workgroups walk its
//     chunk expert by expert, N tile major inside an expert's units, so the workgroups
//     that run together share each weight panel and each unit's activation rows
//     through that XCD's L2.
//   * In the two-deep 8-wavefront tiles, wavefronts 0-3 (one per SIMD) issue all of a
//     stage's loads and 4-7 none: a wavefront stalls until the CU accepts each load,
//     and this way one wavefront per SIMD starts its MFMAs while the other issues.
//   * Operands are both K-contiguous ([out, in] weights).  Each stage moves a K slice
//     of BM activation rows and BN weight rows straight into LDS (direct-to-LDS loads,
//     an NST-deep ring, one barrier per stage), XOR-swizzled by row so the 16-byte
//     fragment reads of 8 consecutive lanes hit distinct banks.
//   * Wavefronts own 16-row tiles round-robin, so a partially filled unit spreads
//     its valid rows over all wavefronts; tiles past the unit's rows are skipped, and
//     the two-deep rings do not load activation chunks wholly past them.
//   * bf16: v_mfma_f32_16x16x32_bf16.  fp8 (e4m3): one v_mfma 16x16x128 per
//     128-wide K block, promoted into the fp32 accumulator with the 1x128
//     activation scale times the 128x128 weight scale ([MND §Quantization]:
//     activation scales vary only along K, so the promotion happens once per
//     K block).
//   * Epilogues: SwiGLU (h = silu(gate) * up, gate and up columns of the same
//     h column sit in the same lane), optional 1x128 fp8 quantization of h,
//     bf16 store (tile pairs regrouped by a lane swap into 16-byte stores), or fp32
//     split-k partials; bf16 and e4m3 rounding use gfx950's conversion instructions.

#include <type_traits>

#include "addr.h"
#include "common.h"
#include "kernels.h"
#include "plan.h"

namespace moe {

// ------------------------------------------------------------------ DMA pipeline
// Global -> LDS with global_load_lds_dwordx4 (each lane lands 16 bytes at
// lds + 16 * lane, no staging registers) into an NST-deep ring
// of stage buffers; step s waits only for its own loads (vmcnt), so NST - 1 stages of
// weight traffic are in flight per workgroup.  Stage = ROWB bytes of K for all BM
// activation rows and BN weight rows.  The ring buffers are distinct LDS objects and
// the step loop is unrolled by NST so every buffer index is a compile-time constant:
// the compiler can then see that the DMA into one buffer never aliases the fragment
// reads of another and keeps them unordered.  Prefill tiles (320 x 256) use 128-byte
// stages in a 2-deep ring: each stage then reads whole 128-byte lines of every row,
// which the L2 serves at a markedly higher rate than the 64-byte half lines of a
// deeper 64-byte ring, and that outweighs the shallower prefetch.

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  // gfx9 s_waitcnt: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[5:4] at [15:14]
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Workgroup barrier without a memory fence.  __syncthreads() also drains every
// outstanding global access (vmcnt(0)), which would empty the DMA ring at each step;
// here each wave has already waited for its own stage loads (wait_vmcnt), its LDS
// fragment reads have returned before their MFMAs, and the empty asm statements keep
// the compiler from moving memory operations across the barrier.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// 16 bytes per lane (global_load_lds_dwordx4) into lds_chunk + 16 * lane, with the
// address split into a wave-uniform 64-bit base (scalar registers) and a 32-bit per-lane
// byte offset: the per-lane address needs one VGPR and no 64-bit add.  M0 holds the LDS
// destination; the DMA is counted by vmcnt like any global load.
// NT: non-temporal (streaming) cache policy, for data read once.  m0: the LDS byte
// address of the 1 KB chunk (wave-uniform, in a scalar register).
template <bool NT = false>
__device__ __forceinline__ void dma16m(const void* base, uint32_t off, uint32_t m0) {
  if constexpr (NT) {
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1 nt"
                 :
                 : "v"(off), "s"(base), "s"(m0)
                 : "memory", "m0");
  } else {
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
                 :
                 : "v"(off), "s"(base), "s"(m0)
                 : "memory", "m0");
  }
}

// 4 bytes per lane (global_load_lds_dword) into lds_chunk + 4 * lane; base/offset form.
__device__ __forceinline__ void dma4s(const void* base, uint32_t off, uint8_t* lds_chunk) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(
      static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
          (__attribute__((address_space(3))) uint8_t*)lds_chunk)));
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dword %0, %1"
               :
               : "v"(off), "s"(base), "s"(m0)
               : "memory", "m0");
}

// 16 packed int4 codes (8 bytes: per byte, element i low nibble, element 8 + i high
// nibble) -> 16 int8 codes in element order.  Sign extension of each nibble n, per byte
// without carries between bytes: ((n ^ 8) + 0x78) ^ 0x80.
__device__ __forceinline__ i32x4 unpack_int4x16(uint2 pk) {
  constexpr uint32_t kLo = 0x0F0F0F0Fu;
  const uint32_t v[4] = {pk.x & kLo, pk.y & kLo, (pk.x >> 4) & kLo, (pk.y >> 4) & kLo};
  i32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) r[i] = static_cast<int>(((v[i] ^ 0x08080808u) + 0x78787878u) ^ 0x80808080u);
  return r;
}

template <int ROWB>
__device__ __forceinline__ int swz(int row) {
  if constexpr (ROWB >= 128) return row & 7;   // 128- and 256-byte rows: 8 rows, 8 slots
  else return (row >> 1) & 3;                  // 64-byte rows: 2 rows per 128-byte window
}

template <int WM, int WN, int TM, int TN, int EPI, bool UNIFORM, int ROWB, int NST, bool FP8,
          bool I8 = false, bool W4 = false>
__device__ __forceinline__ void gemm_dma_body(const GemmArgs& p) {
  constexpr int NT = WM * WN * 64;
  constexpr int NW = NT / 64;
  constexpr int BM = WM * TM * 16;
  constexpr int BN = WN * TN * 16;
  // Q8: int8 activations and exact int32 accumulation (W8A8, and W4A8 whose packed int4
  // weights are unpacked to int8 codes after LDS)
  constexpr bool Q8 = I8 || W4;
  constexpr int EB = (FP8 || Q8) ? 1 : 2;   // activation element bytes
  constexpr int KSTEP = ROWB / EB;       // elements per stage
  constexpr int CPR = ROWB / 16;         // 16-byte chunks per activation row
  constexpr int RPC = 64 / CPR;          // rows per 1 KB DMA (one wave instruction)
  constexpr int ROWB_B = W4 ? ROWB / 2 : ROWB;   // weight bytes per row and stage
  constexpr int CPR_B = ROWB_B / 16;
  constexpr int RPC_B = 64 / CPR_B;
  constexpr int A_LD = BM / RPC, B_LD = BN / RPC_B;
  constexpr int LD_ALL = A_LD + B_LD;
  constexpr int LMAX = (LD_ALL + NW - 1) / NW;   // DMA instructions per wave per stage
  constexpr int LREM = LD_ALL % NW;              // waves < LREM issue LMAX, others LMAX-1
  constexpr int STAGE = BM * ROWB + BN * ROWB_B;
  // Loader wavefronts.  With a two-deep ring and 8 wavefronts, waves 0..3 (one per SIMD)
  // issue every load of a stage and waves 4..7 none: a wavefront stalls until the CU
  // accepts each of its loads, so this way one wavefront per SIMD starts its MFMAs right
  // after the barrier while the other is still issuing, instead of both waiting on a
  // burst of loads.  Otherwise every wavefront issues an equal share.
  constexpr int LW = (NST == 2 && NW == 8) ? 4 : NW;
  static_assert(A_LD % LW == 0 && B_LD % LW == 0, "chunks split evenly over the loaders");
  constexpr int A_PER = A_LD / LW, B_PER = B_LD / LW;
  constexpr int LPER = A_PER + B_PER;            // DMA chunks per loader wave and stage
  static_assert(LW != NW || (LPER == LMAX && LREM == 0), "uniform per-wave DMA count");
  // Weights read by this unit alone stream through the caches non-temporally (they are
  // not read again); weights that other units of the group also read stay cacheable.
  // Packed int4 rows of a 128-element stage are 64-byte half lines: not non-temporal, so
  // that the line's other half, read one stage later, still hits.
  constexpr bool NTW_OK = !UNIFORM && ROWB_B >= 128;
  constexpr bool SWIGLU = (EPI == EPI_SWIGLU_BF16 || EPI == EPI_SWIGLU_FP8);
  // fp8: one stage = one 128-wide K block of e4m3 codes; its 1x128 activation scales and
  // the two 128x128 weight-block scales of the tile come into LDS with the stage.
  // fp8: waves 0 .. ASW-1 DMA the stage's activation scales (64 rows each), wave ASW the
  // two weight-block scales
  constexpr int ASW = (BM + 63) / 64;
  static_assert(!FP8 || (ROWB == kQBlock && (BM % 64 == 0 || BM == 32) && ASW < WM * WN && !UNIFORM),
                "fp8 tiles: one scale block per stage");
  static_assert(FP8 == (EPI == EPI_SWIGLU_FP8) || EPI == EPI_STORE_BF16 || EPI == EPI_STORE_F32,
                "epilogue matches operands");
  // I8 (W8A8): int8 codes, exact int32 accumulation, one dequantization in the epilogue
  // with the activation row's scale and the weight column's scale
  static_assert(!Q8 || (!FP8 && !UNIFORM && (EPI == EPI_SWIGLU_BF16 || EPI == EPI_STORE_BF16 ||
                                             EPI == EPI_STORE_F32)),
                "int8 operands: grouped launches with a bf16 result");
  static_assert(!W4 || ROWB == 128 || ROWB == 256, "int4 weights: 64- or 128-byte weight rows per stage");
  static_assert(BM % RPC == 0 && BN % RPC_B == 0, "tiles are whole DMA chunks");
  static_assert(NST >= 2 && NST <= 4, "ring depth");
  static_assert(!SWIGLU || TN % 2 == 0, "swiglu needs gate/up tile pairs");

  __shared__ __attribute__((aligned(1024))) uint8_t st0[STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t st1[STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t st2[NST > 2 ? STAGE : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t st3[NST > 3 ? STAGE : 16];
  // per ring slot: activation scales (64 per scale wave) and weight-block scales
  __shared__ __attribute__((aligned(16))) float sa_st[FP8 ? NST : 1][FP8 ? ASW * 64 : 1];
  __shared__ __attribute__((aligned(16))) float sb_st[FP8 ? NST : 1][FP8 ? 64 : 1];
  // fp8: the per-lane DMA offsets live in LDS and are re-read (volatile) at each issue;
  // in registers they would be spilled, and a scratch reload waits on vmcnt(0), which
  // would drain the DMAs in flight.
  // loader lanes' chunk offsets, four per 16-byte entry (one 16-byte read per four DMAs)
  constexpr int OFFG = (LPER + 3) / 4;
  __shared__ __attribute__((aligned(16))) u32x4 off_tab[FP8 ? OFFG : 1][FP8 ? LW * 64 : 1];
  __shared__ uint32_t sc_tab[FP8 ? (ASW + 1) * 64 : 1];               // scale offsets, waves 0 .. ASW

  // A workgroup computes TPW consecutive N tiles of one unit (one K split); its ring runs
  // on from one tile's K steps into the next's, so the next tile's first stage is in
  // flight while this one's epilogue stores.  Only for plain stores (the down
  // projection) of int8 / int4 operands where the ring is two deep (every wait drains the
  // counter, so the epilogue's stores cannot shift it).
  constexpr bool MULTI = !UNIFORM && Q8 && NST == 2 && (EPI == EPI_STORE_BF16 || EPI == EPI_STORE_F32);
  const int tpw = MULTI ? p.tiles_per_wg : 1;
  // tiles past the first address their weight rows by a fixed offset from the first's,
  // which needs whole tiles along N (the launcher enforces it)
  if (tpw > 1 && p.N % (SWIGLU ? BN / 2 : BN) != 0) return;
  const int bid = blockIdx.x;
  const int xcd = bid % kXcds;
  const int slot = bid / kXcds;
  const int n_grp = (p.n_tiles + tpw - 1) / tpw;
  const int per_unit = n_grp * p.splits;
  int u, rem;
  if constexpr (UNIFORM) {
    u = (slot / per_unit) * kXcds + xcd;
    rem = slot % per_unit;
  } else {
    // This XCD's chunk of the unit table, walked run by run (a run: one group's
    // consecutive units), and inside a run N tile (and split) major: the workgroups
    // that run together on the XCD share each weight panel through its L2.
    const int c0 = p.n_units[1 + xcd], c1 = p.n_units[2 + xcd];
    if (slot >= (c1 - c0) * per_unit) return;
    const Unit uq = p.units[c0 + slot / per_unit];
    plan_map_slot(slot, per_unit, c0, c1, uq.first, uq.count, &u, &rem);
  }
  const int nt0 = (rem % n_grp) * tpw;           // first N tile of this workgroup
  const int ntc = min(tpw, p.n_tiles - nt0);     // N tiles it computes
  const int split = rem / n_grp;
  Unit un;
  if constexpr (UNIFORM) {
    if (u * BM >= p.uniform_rows) return;
    un.group = 0;
    un.row0 = u * BM;
    un.rows = min(BM, p.uniform_rows - u * BM);
  } else {
    un = p.units[u];
  }
  const int rows = un.rows;
  if (rows <= 0) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar)
  const int wm = wave / WN;
  const int wn = wave % WN;
  const int mtiles = (rows + 15) >> 4;
  int jcount = mtiles > wm ? (mtiles - wm + WM - 1) / WM : 0;
  if (jcount > TM) jcount = TM;

  const int k0 = split * p.k_chunk;
  const int k1 = min(p.K, k0 + p.k_chunk);
  const int nsteps = (k1 - k0) / KSTEP;

  // Units of the alternate group (the shared expert folded into the routed launch)
  // read their own activations and weights and write their own output.
  const bool alt = !UNIFORM && un.group == p.alt_group;
  const long long lda = alt ? p.lda2 : p.lda;
  const int32_t* gather = (!UNIFORM && !alt) ? p.gather : nullptr;
  const uint8_t* a_base = (alt ? p.A2 : p.A) +
                          (gather ? 0LL : static_cast<long long>(un.row0) * lda) +
                          static_cast<long long>(k0) * EB;
  const uint8_t* b_base = (alt ? p.B2 : p.B + static_cast<long long>(un.group) * p.b_group) +
                          static_cast<long long>(k0) * EB / (W4 ? 2 : 1);
  void* const cptr = alt ? p.C2 : p.C;
  const long long ldc = alt ? p.ldc2 : p.ldc;
  bool ntb = false;   // wave-uniform: stream this unit's weights non-temporally
  if constexpr (!UNIFORM) ntb = (un.flags & kUnitSoleReader) != 0;

  // DMA plan.  Every loader wavefront issues up to A_PER activation chunks (q = wave + i *
  // LW) and B_PER weight chunks (q = wave + i * LW) per stage.  Lane -> (row q*RPC +
  // lane/CPR, physical 16-byte slot lane%CPR), which holds logical K chunk (lane%CPR) ^
  // swz(row).  Rows past the unit inside a chunk and columns past N re-load a valid row;
  // in the two-deep rings (whose waits drain the counter, so the per-wave load count may
  // vary) an activation chunk wholly past the unit's rows is not loaded and its LDS rows
  // keep stale data.  Either way those rows only feed result rows that are never stored.
  const bool loader = LW == NW || wave < LW;   // wave-uniform
  uint32_t goff[LPER];
  const int lrow = lane / CPR;
  const int lphys = lane % CPR;
  const int lrow_b = lane / CPR_B;
  const int lphys_b = lane % CPR_B;
  if (loader) {
#pragma unroll
    for (int i = 0; i < A_PER; ++i) {
      const int q = wave + i * LW;
      const int r = q * RPC + lrow;
      const int rc = r < rows ? r : rows - 1;
      const long long src = gather ? gather[un.row0 + rc] / p.gather_div : rc;
      goff[i] = static_cast<uint32_t>(src * lda + ((lphys ^ swz<ROWB>(r)) << 4));
    }
#pragma unroll
    for (int i = 0; i < B_PER; ++i) {
      const int j = (wave + i * LW) * RPC_B + lrow_b;
      int col, grow;
      if constexpr (SWIGLU) {
        constexpr int WCOLS = TN * 16, HALF = TN * 8;
        const int wn2 = j / WCOLS, jj = j % WCOLS;
        col = nt0 * (BN / 2) + wn2 * HALF + (jj % HALF);
        grow = (jj < HALF ? 0 : p.up_off) + col;
      } else {
        col = nt0 * BN + j;
        grow = col;
      }
      if (col >= p.N) grow -= col - (p.N - 1);
      goff[A_PER + i] = static_cast<uint32_t>(static_cast<long long>(grow) * p.ldb + ((lphys_b ^ swz<ROWB_B>(j)) << 4));
    }
  }

  // fp8 scale sources of this lane: wavefronts 0 .. BM/64-1 fetch the activation
  // scales of rows 64 * wave + lane, wavefront BM/64 the two weight-block scales.
  // (base: wave-uniform pointer at the first K block of the split; off: lane byte offset)
  const float* sc_base = nullptr;
  uint32_t sc_off = 0;
  if constexpr (FP8) {
    const int kb0 = k0 / kQBlock;
    if (wave < ASW) {
      // the scale row of this lane's activation row (gathered: the token's row)
      const int r = 64 * wave + lane;
      const int rc = r < rows ? r : rows - 1;
      const long long src = gather ? gather[un.row0 + rc] / p.gather_div : un.row0 + rc;
      sc_base = p.a_scale + kb0;
      sc_off = static_cast<uint32_t>(src * p.a_scale_ld * 4);
    } else {
      int blk;
      if constexpr (SWIGLU) {
        blk = (lane == 1) ? p.up_off / kQBlock + nt0 : nt0;        // gate, up block
      } else {
        const int nb = (p.N + kQBlock - 1) / kQBlock;
        blk = min(2 * nt0 + (lane == 1 ? 1 : 0), nb - 1);          // two column blocks
      }
      sc_base = p.b_scale + static_cast<long long>(un.group) * p.b_scale_group + kb0;
      sc_off = static_cast<uint32_t>(static_cast<long long>(blk) * p.b_scale_ld * 4);
    }
    // one base per wavefront (the DMA takes it in scalar registers), rebuilt from its two
    // wave-uniform 32-bit halves
    const uint64_t sb = reinterpret_cast<uint64_t>(sc_base);
    sc_base = reinterpret_cast<const float*>(
        join_u32_halves(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(sb)),
                        __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(sb >> 32))));
  }
  using vlds = volatile __attribute__((address_space(3))) uint32_t*;
  if constexpr (FP8) {
    if (loader) {
#pragma unroll
      for (int g = 0; g < OFFG; ++g)
        off_tab[g][tid] = u32x4{goff[4 * g], 4 * g + 1 < LPER ? goff[4 * g + 1] : 0u,
                                4 * g + 2 < LPER ? goff[4 * g + 2] : 0u, 4 * g + 3 < LPER ? goff[4 * g + 3] : 0u};
    }
    if (wave <= ASW) sc_tab[tid] = sc_off;
    // visible to this lane's own later reads; no other lane reads it
  }
  // (fp8 reads its offsets from the LDS table at each issue instead)
  auto lane_off_of = [&](int i) __attribute__((always_inline)) { return goff[i]; };
  // This wavefront's first 1 KB chunk of each ring buffer, as an LDS byte address
  // (wave-uniform).  Each DMA's M0 is formed from it with a compile-time offset at the
  // issue itself: the empty asm below makes the base a fresh value per issue, so the
  // compiler cannot hoist the buffers x chunks M0 values out of the loop into scalar
  // registers (it spilled them to vector lanes, inside the loop).
  auto lds_addr = [&](const uint8_t* buf) __attribute__((always_inline)) {
    return __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
        (const __attribute__((address_space(3))) uint8_t*)buf)) + wave * 1024u);
  };
  // weight rows between one N tile and the next (the offsets above address tile nt0)
  const long long tile_b = static_cast<long long>(SWIGLU ? BN / 2 : BN) * p.ldb;
  auto issue = [&](int t, int step, uint8_t* buf, int b) __attribute__((always_inline)) {
    const long long kb = static_cast<long long>(step) * ROWB;
    const uint8_t* ak = a_base + kb;   // wave-uniform bases of this K step
    const uint8_t* bk = b_base + static_cast<long long>(step) * ROWB_B;
    if constexpr (MULTI) bk += t * tile_b;
    uint32_t m0w = lds_addr(buf);
    asm volatile("" : "+s"(m0w));
    if (loader) {
      // every lane offset of this issue is read before the first DMA (fp8: from the LDS
      // table, four offsets per 16-byte read, so one wait covers them all instead of one
      // LDS round trip per DMA)
      uint32_t offs[LPER];
      if constexpr (FP8) {
        using vlds4 = volatile __attribute__((address_space(3))) u32x4*;
#pragma unroll
        for (int g = 0; g < OFFG; ++g) {
          const u32x4 o = ((vlds4)&off_tab[g][0])[tid];
          offs[4 * g] = o.x;
          if (4 * g + 1 < LPER) offs[4 * g + 1] = o.y;
          if (4 * g + 2 < LPER) offs[4 * g + 2] = o.z;
          if (4 * g + 3 < LPER) offs[4 * g + 3] = o.w;
        }
      } else {
#pragma unroll
        for (int i = 0; i < LPER; ++i) offs[i] = lane_off_of(i);
      }
#pragma unroll
      for (int i = 0; i < A_PER; ++i)   // wave-uniform test: chunk q holds a row of the unit
        if (NST != 2 || (wave + i * LW) * RPC < rows) dma16m(ak, offs[i], m0w + i * LW * 1024u);
      if (NTW_OK && ntb) {
#pragma unroll
        for (int i = 0; i < B_PER; ++i)
          dma16m<true>(bk, offs[A_PER + i], m0w + BM * ROWB + i * LW * 1024u);
      } else {
#pragma unroll
        for (int i = 0; i < B_PER; ++i)
          dma16m<false>(bk, offs[A_PER + i], m0w + BM * ROWB + i * LW * 1024u);
      }
    }
    if constexpr (FP8) {
      if (wave <= ASW) {
        const uint32_t so = ((vlds)&sc_tab[0])[tid];
        if (wave < ASW) dma4s(sc_base + step, so, reinterpret_cast<uint8_t*>(&sa_st[b][64 * wave]));
        else dma4s(sc_base + step, so, reinterpret_cast<uint8_t*>(&sb_st[b][0]));
      }
    }
  };

  f32x4 acc[TM][TN];

  const int frag_row = lane & 15;
  const int kgrp = lane >> 4;

  // int8 / int4: this lane's activation-row scales for the epilogue, loaded before the
  // main loop (gathered rows take the scale of the token they read), so nothing of the
  // gather stays live across the loop
  float sa[Q8 ? TM : 1];
  if constexpr (Q8) {
    const float* sa_base = alt ? p.a_scale2 : p.a_scale;
#pragma unroll
    for (int j = 0; j < TM; ++j) {
      const int row = 16 * (j * WM + wm) + (lane & 15);
      sa[j] = (j < jcount && row < rows)
                  ? sa_base[gather ? gather[un.row0 + row] / p.gather_div : un.row0 + row]
                  : 0.f;
    }
  }

  // One stage of MFMAs for a wavefront owning J valid 16-row tiles.  J is a
  // compile-time constant (the main loop is instantiated per row-tile count), so
  // every fragment read of a K slice is issued before its first MFMA and no
  // branch separates them.
  // Fragment rows are 16 * tile + frag_row, and the row swizzle of such a row is a
  // function of frag_row alone (tile rows are multiples of 8), so every fragment address
  // is a per-lane offset (computed once) plus a compile-time tile offset.
  auto lane_off = [&](int c) __attribute__((always_inline)) {
    return frag_row * ROWB + ((c ^ swz<ROWB>(frag_row)) << 4);
  };
  auto compute = [&](const uint8_t* buf, int b, auto Jc) __attribute__((always_inline)) {
    constexpr int J = decltype(Jc)::value;
    const uint8_t* lb = buf + BM * ROWB;
    if constexpr (FP8) {
      // one v_mfma_scale_f32_16x16x128_f8f6f4 (unit hardware scales) per tile pair and
      // K block, promoted into the fp32 accumulator with s_a(token) * s_w(column block)
      // ([MND §Quantization]: activation scales vary only along K).  Lane holds 32
      // codes of its fragment row: 16-byte chunks kgrp and kgrp + 4 of the 128-byte K
      // block (any split of K between the lanes is the same product as long as both
      // operands use it; this one reads conflict-free, where chunks 2 kgrp and 2 kgrp + 1
      // spent half the LDS cycles in bank conflicts).  Weight fragments of the TN column
      // tiles stay in registers; each row tile's activation fragment is read once and used
      // TN times.
      // One LDS pointer per operand and chunk (stage base + lane offset), made opaque so
      // that every tile's read uses it with an immediate tile offset instead of a
      // precomputed address register per tile and stage.
      using lptr = __attribute__((address_space(3))) const uint8_t*;
      lptr a_lo = (lptr)(buf + lane_off(kgrp));
      lptr a_hi = (lptr)(buf + lane_off(kgrp + 4));
      lptr b_lo = (lptr)(lb + lane_off(kgrp));
      lptr b_hi = (lptr)(lb + lane_off(kgrp + 4));
      asm volatile("" : "+v"(a_lo), "+v"(a_hi), "+v"(b_lo), "+v"(b_hi));
      auto frag = [&](lptr lo_p, lptr hi_p, int tile) __attribute__((always_inline)) {
        const u32x4 lo = *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(lo_p + tile * 16 * ROWB);
        const u32x4 hi = *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(hi_p + tile * 16 * ROWB);
        return i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      };
      // the same read, kept in program order (volatile), so that it stays in the step
      // of the pipeline below that issues it
      auto frag_v = [&](lptr lo_p, lptr hi_p, int tile) __attribute__((always_inline)) {
        using vp = volatile const __attribute__((address_space(3))) u32x4*;
        const u32x4 lo = *reinterpret_cast<vp>(lo_p + tile * 16 * ROWB);
        const u32x4 hi = *reinterpret_cast<vp>(hi_p + tile * 16 * ROWB);
        return i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      };
      i32x8 bw[TN];
      float sb[TN];
      const float sb0 = sb_st[b][0];
      const float sb1 = sb_st[b][1];
#pragma unroll
      for (int i = 0; i < TN; ++i) {
        bw[i] = frag(b_lo, b_hi, wn * TN + i);
        // SwiGLU: tiles i < TN/2 are gate columns (block 0), the rest up columns
        // (block 1); plain store: the first 128 columns of the tile are block 0
        sb[i] = SWIGLU ? (i < TN / 2 ? sb0 : sb1) : (wn * TN * 16 < kQBlock ? sb0 : sb1);
      }
      // Software pipeline over the row tiles: the MFMAs of row tile j are issued before
      // the promotion of row tile j - 1, whose products have finished by then, so no
      // MFMA waits on its own result and the promotion runs beside the next MFMAs.  The
      // scheduling barriers keep the compiler from hoisting every row tile's fragment
      // read to the top (which left no registers for separate products).
      i32x8 at = frag(a_lo, a_hi, wm);
      f32x4 prev[TN];
      float fprev[TN];
#pragma unroll
      for (int j = 0; j < J; ++j) {
        const float sa = sa_st[b][16 * (j * WM + wm) + (lane & 15)];
        f32x4 cur[TN];
#pragma unroll
        for (int i = 0; i < TN; ++i)
          cur[i] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
              bw[i], at, f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 127, 0, 127);
        if (j + 1 < J) at = frag_v(a_lo, a_hi, (j + 1) * WM + wm);
        if (j > 0) {
#pragma unroll
          for (int i = 0; i < TN; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              acc[j - 1][i][r] = fmaf(prev[i][r], fprev[i], acc[j - 1][i][r]);
              // pins the promotion (and so the MFMAs it reads) to this step: pure
              // arithmetic would otherwise sink below later reads and branches
              asm volatile("" : "+v"(acc[j - 1][i][r]));
            }
        }
#pragma unroll
        for (int i = 0; i < TN; ++i) {
          prev[i] = cur[i];
          fprev[i] = sa * sb[i];
        }
        // order within the step: each MFMA followed by one LDS read and a few of the
        // promotion FMAs, which run while the MFMA does
#pragma unroll
        for (int i = 0; i < TN; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // LDS read
          __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);   // VALU
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      if constexpr (J > 0) {
#pragma unroll
        for (int i = 0; i < TN; ++i)
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[J - 1][i][r] = fmaf(prev[i][r], fprev[i], acc[J - 1][i][r]);
      }
      return;
    }
#pragma unroll
    for (int kk = 0; kk < ROWB / 64; ++kk) {
      const int o = lane_off(kk * 4 + kgrp);
      bf16x8 bfr[TN];
      bf16x8 afr[J > 0 ? J : 1];
      if constexpr (W4) {
        // this lane's 16 elements of K are the 8 bytes at byte kk*32 + kgrp*8 of the
        // 64-byte weight row (16-byte chunk kk*2 + kgrp/2, swizzled like the DMA wrote it)
        const int ob = frag_row * ROWB_B + (((kk * 2 + (kgrp >> 1)) ^ swz<ROWB_B>(frag_row)) << 4) +
                       (kgrp & 1) * 8;
#pragma unroll
        for (int i = 0; i < TN; ++i)
          bfr[i] = __builtin_bit_cast(
              bf16x8, unpack_int4x16(*reinterpret_cast<const uint2*>(lb + (wn * TN + i) * 16 * ROWB_B + ob)));
      } else {
#pragma unroll
        for (int i = 0; i < TN; ++i)
          bfr[i] = *reinterpret_cast<const bf16x8*>(lb + (wn * TN + i) * 16 * ROWB + o);
      }
#pragma unroll
      for (int j = 0; j < J; ++j)
        afr[j] = *reinterpret_cast<const bf16x8*>(buf + (j * WM + wm) * 16 * ROWB + o);
#pragma unroll
      for (int j = 0; j < J; ++j)
#pragma unroll
        for (int i = 0; i < TN; ++i) {
          // weights as the MFMA's A operand and tokens as its B operand: the result tile is
          // [output column][token], so each lane ends up with 4 consecutive output
          // columns of one token row (stored as one 8- or 16-byte vector)
          if constexpr (Q8) {
            // the same 16 bytes per lane hold 16 int8 codes of K: one 16x16x64 MFMA
            // covers the 64-byte K slice that two bf16 steps would
            acc[j][i] = __builtin_bit_cast(
                f32x4, __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i32x4, bfr[i]),
                                                            __builtin_bit_cast(i32x4, afr[j]),
                                                            __builtin_bit_cast(i32x4, acc[j][i]), 0, 0, 0));
          } else {
            acc[j][i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bfr[i], afr[j], acc[j][i], 0, 0, 0);
          }
        }
    }
  };

  // DMA instructions this wavefront issues per stage (wave-uniform): its tile chunks
  // (LMAX, or LMAX - 1 for waves at or past LREM) plus, for fp8, one scale load on
  // waves 0 .. ASW
  constexpr int HI = FP8 ? LMAX + 1 : LMAX;
  constexpr int LO = FP8 ? LMAX : LMAX - 1;
  const bool hi = FP8 ? wave <= ASW : wave < (LREM == 0 ? NW : LREM);
  // wait until the loads of the current step landed; `later` = steps issued after it
  auto wait_step = [&](int later) __attribute__((always_inline)) {
    if (later >= NST - 2 && NST > 2) {
      if (hi) wait_vmcnt<(NST > 2 ? (NST - 2) * HI : 0)>();
      else wait_vmcnt<(NST > 2 ? (NST - 2) * LO : 0)>();
    } else if (later == 1 && NST > 3) {
      if (hi) wait_vmcnt<HI>();
      else wait_vmcnt<LO>();
    } else {
      wait_vmcnt<0>();
    }
  };

  // The ring runs on across this workgroup's N tiles when each tile's step count is a
  // whole number of ring turns (step s of every tile then lands in buffer s % NST);
  // otherwise every tile starts its own ring.
  const bool chain = MULTI && nsteps % NST == 0;
  auto buf_of = [&](int b) __attribute__((always_inline)) {
    return b == 0 ? st0 : b == 1 ? st1 : b == 2 ? st2 : st3;
  };
  auto mainloop = [&](auto Jc, int t) __attribute__((always_inline)) {
    // last step (counted over the workgroup's tiles) that is loaded by this ring
    const int last = (chain ? ntc : t + 1) * nsteps - 1;
    for (int s0 = 0; s0 < nsteps; s0 += NST) {
#pragma unroll
      for (int b = 0; b < NST; ++b) {
        const int s = s0 + b;
        if (s < nsteps) {
          const int g = t * nsteps + s;
          const int issued_after = min(last, g + NST - 2) - g;
          wait_step(issued_after);
          lds_barrier();
          // refill the buffer consumed at step s - 1 with step s + NST - 1 (of the next
          // tile once this one has none left)
          const int nb = (b + NST - 1) % NST;
          if (s + NST - 1 < nsteps) issue(t, s + NST - 1, buf_of(nb), nb);
          else if (chain && t + 1 < ntc) issue(t + 1, s + NST - 1 - nsteps, buf_of(nb), nb);
          compute(buf_of(b), b, Jc);
        }
      }
    }
  };
  for (int t = 0; t < ntc; ++t) {
  const int nt = nt0 + t;
  if (t == 0 || !chain) {
    // prologue: steps 0 .. NST-2 of this tile
#pragma unroll
    for (int b = 0; b < NST - 1; ++b) {
      if (b < nsteps) issue(t, b, buf_of(b), b);
    }
  }
#pragma unroll
  for (int j = 0; j < TM; ++j)
#pragma unroll
    for (int i = 0; i < TN; ++i) acc[j][i] = f32x4{0.f, 0.f, 0.f, 0.f};
  // jcount is wave-uniform and at most TM; every instantiation runs the same
  // sequence of barriers, so wavefronts with different counts stay in step.
  static_assert(TM <= 10, "row-tile dispatch covers TM <= 10");
  switch (jcount) {
    case 10: if constexpr (TM >= 10) mainloop(std::integral_constant<int, (TM >= 10 ? 10 : 0)>{}, t); break;
    case 9: if constexpr (TM >= 9) mainloop(std::integral_constant<int, (TM >= 9 ? 9 : 0)>{}, t); break;
    case 8: if constexpr (TM >= 8) mainloop(std::integral_constant<int, (TM >= 8 ? 8 : 0)>{}, t); break;
    case 7: if constexpr (TM >= 7) mainloop(std::integral_constant<int, (TM >= 7 ? 7 : 0)>{}, t); break;
    case 6: if constexpr (TM >= 6) mainloop(std::integral_constant<int, (TM >= 6 ? 6 : 0)>{}, t); break;
    case 5: if constexpr (TM >= 5) mainloop(std::integral_constant<int, (TM >= 5 ? 5 : 0)>{}, t); break;
    case 4: if constexpr (TM >= 4) mainloop(std::integral_constant<int, (TM >= 4 ? 4 : 0)>{}, t); break;
    case 3: if constexpr (TM >= 3) mainloop(std::integral_constant<int, (TM >= 3 ? 3 : 0)>{}, t); break;
    case 2: if constexpr (TM >= 2) mainloop(std::integral_constant<int, (TM >= 2 ? 2 : 0)>{}, t); break;
    case 1: mainloop(std::integral_constant<int, 1>{}, t); break;
    default: mainloop(std::integral_constant<int, 0>{}, t); break;
  }

  // ---- epilogue.  Transposed C fragment of a 16x16 tile: lane holds token row
  // lane & 15 and output columns 4 * (lane >> 4) + r, r = 0..3.
  // The epilogue's base values pass through an empty asm statement here, so no output
  // address can be formed before the main loop and held in registers across it.
  int row0_e = un.row0;
  long long ldc_e = ldc;
  void* cptr_e = cptr;
  asm volatile("" : "+s"(row0_e), "+s"(ldc_e), "+s"(cptr_e));
  const int crow = lane & 15;
  const int ccol4 = 4 * kgrp;
  if constexpr (Q8) {
    // W8A8 / W4A8 dequantization: value = acc (exact int32) * s_a[row] * s_w[channel], with the
    // activation scale of the unit's row and the per-output-channel weight scale
    // (units of the alternate group take its own activation and weight scales)
    constexpr int HT = TN / 2;
    const float* sw_base =
        alt ? p.b_scale2 : p.b_scale + static_cast<long long>(un.group) * p.b_scale_group;

#pragma unroll
    for (int i = 0; i < TN; ++i) {
      int col, ch;   // first output column of this lane in tile i, and its weight channel
      if constexpr (EPI == EPI_SWIGLU_BF16) {
        col = nt * (BN / 2) + wn * (TN * 8) + 16 * (i % HT) + ccol4;
        ch = (i < HT ? 0 : p.up_off) + col;
      } else {
        col = nt * BN + wn * TN * 16 + 16 * i + ccol4;
        ch = col;
      }
      float sw[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) sw[r] = col + r < p.N ? sw_base[ch + r] : 0.f;
#pragma unroll
      for (int j = 0; j < TM; ++j) {
        // whole-vector reinterpretation first, then a new float vector: the integer
        // tile is read once, before any of its lanes is overwritten
        const i32x4 iv = __builtin_bit_cast(i32x4, acc[j][i]);
        f32x4 fv;
#pragma unroll
        for (int r = 0; r < 4; ++r) fv[r] = static_cast<float>(iv[r]) * sa[j] * sw[r];
        acc[j][i] = fv;
      }
    }
  }
  if constexpr (EPI == EPI_STORE_BF16 && TN % 2 == 0) {
    // Tiles i and i + 1 in pairs: lanes kgrp and kgrp ^ 1 (lane ^ 16, the same token row)
    // swap one 4-column half, so an even kgrp holds columns 4 * kgrp .. + 7 of tile i and
    // an odd one columns 4 * (kgrp - 1) .. + 7 of tile i + 1, 16 bytes either way; a store
    // instruction then writes 64 contiguous bytes of each of its 16 rows instead of 32.
    const bool odd = (kgrp & 1) != 0;
    const int cpair = nt * BN + wn * TN * 16 + (odd ? 16 : 0) + 4 * (kgrp & ~1);
#pragma unroll
    for (int j = 0; j < TM; ++j) {
      if (j >= jcount) continue;   // wave-uniform
      const int row = 16 * (j * WM + wm) + crow;
      uint16_t* crow_p = static_cast<uint16_t*>(cptr_e) + static_cast<long long>(row0_e + row) * ldc_e;
#pragma unroll
      for (int i = 0; i < TN; i += 2) {
        const uint32_t a0 = pack_bf16x2(acc[j][i][0], acc[j][i][1]);
        const uint32_t a1 = pack_bf16x2(acc[j][i][2], acc[j][i][3]);
        const uint32_t b0 = pack_bf16x2(acc[j][i + 1][0], acc[j][i + 1][1]);
        const uint32_t b1 = pack_bf16x2(acc[j][i + 1][2], acc[j][i + 1][3]);
        // every lane takes part in the swap; the partner lane has the same row, so the
        // row test below drops both or neither
        const uint32_t r0 = __shfl_xor(odd ? a0 : b0, 16, 64);
        const uint32_t r1 = __shfl_xor(odd ? a1 : b1, 16, 64);
        if (row >= rows) continue;
        const uint4 v = odd ? make_uint4(r0, r1, b0, b1) : make_uint4(a0, a1, r0, r1);
        const int col = cpair + 16 * i;
        if (col + 7 < p.N) {
          *reinterpret_cast<uint4*>(crow_p + col) = v;
        } else {
          const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
          for (int r = 0; r < 8; ++r)
            if (col + r < p.N) crow_p[col + r] = static_cast<uint16_t>(w[r >> 1] >> (16 * (r & 1)));
        }
      }
    }
  } else if constexpr (EPI == EPI_STORE_BF16 || EPI == EPI_STORE_F32) {
#pragma unroll
    for (int j = 0; j < TM; ++j) {
      if (j >= jcount) continue;
      const int row = 16 * (j * WM + wm) + crow;
      if (row >= rows) continue;
#pragma unroll
      for (int i = 0; i < TN; ++i) {
        const int col = nt * BN + wn * TN * 16 + 16 * i + ccol4;
        const long long o = static_cast<long long>(row0_e + row) * ldc_e + col;
        // bf16 rows are 8-byte aligned (ldc is a multiple of 128); fp32 partials only
        // take the 16-byte store when the address allows it
        const long long cs = split * (alt ? p.c_split2 : p.c_split);   // split-K slice offset
        const bool vec = col + 3 < p.N &&
                         (EPI == EPI_STORE_BF16 ||
                          (reinterpret_cast<uintptr_t>(static_cast<float*>(cptr_e) + o + cs) & 15) == 0);
        if (vec) {
          if constexpr (EPI == EPI_STORE_BF16) {
            *reinterpret_cast<uint2*>(static_cast<uint16_t*>(cptr_e) + o) =
                make_uint2(pack_bf16x2(acc[j][i][0], acc[j][i][1]), pack_bf16x2(acc[j][i][2], acc[j][i][3]));
          } else {
            *reinterpret_cast<f32x4*>(static_cast<float*>(cptr_e) + o + cs) = acc[j][i];
          }
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            if (col + r >= p.N) continue;
            if constexpr (EPI == EPI_STORE_BF16) static_cast<uint16_t*>(cptr_e)[o + r] = f32_to_bf16(acc[j][i][r]);
            else static_cast<float*>(cptr_e)[o + r + cs] = acc[j][i][r];
          }
        }
      }
    }
  } else if constexpr (EPI == EPI_SWIGLU_BF16) {
    constexpr int HT = TN / 2;
#pragma unroll
    for (int j = 0; j < TM; ++j) {
      if (j >= jcount) continue;
      const int row = 16 * (j * WM + wm) + crow;
      if (row >= rows) continue;
#pragma unroll
      for (int i = 0; i < HT; ++i) {
        const int col = nt * (BN / 2) + wn * (TN * 8) + 16 * i + ccol4;
        float hv[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float g = acc[j][i][r];
          const float up = acc[j][i + HT][r];
          hv[r] = silu_fast(g) * up;
        }
        uint16_t* hp = static_cast<uint16_t*>(cptr_e) + static_cast<long long>(row0_e + row) * ldc_e + col;
        if (col + 3 < p.N) {
          *reinterpret_cast<uint2*>(hp) = make_uint2(pack_bf16x2(hv[0], hv[1]), pack_bf16x2(hv[2], hv[3]));
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (col + r < p.N) hp[r] = f32_to_bf16(hv[r]);
        }
      }
    }
  } else {
    // EPI_SWIGLU_FP8: h = silu(gate) * up, quantized per 1x128 block (the workgroup's
    // 128 h columns) with scale = amax / 448 and codes e4m3(h * 448 / amax)
    // ([MND §Quantization]: the SiLU output is block-quantized in the same kernel).
    // Row amax: lane-local over its 4 * HT values, across the four lanes of the row
    // (lane ^ 16, lane ^ 32), then across the WN wavefronts through LDS.
    constexpr int HT = TN / 2;
    static_assert(BN / 2 == kQBlock, "h tile must be one scale block");
    float* xch = reinterpret_cast<float*>(st0);   // [WN][BM] row maxima
    lds_barrier();                                 // every wavefront is done with the ring
#pragma unroll
    for (int j = 0; j < TM; ++j) {
      if (j >= jcount) continue;
      float m = 0.f;
#pragma unroll
      for (int i = 0; i < HT; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float g = acc[j][i][r];
          const float hv = silu_fast(g) * acc[j][i + HT][r];
          acc[j][i][r] = hv;
          m = fmaxf(m, fabsf(hv));
        }
      m = fmaxf(m, __shfl_xor(m, 16, 64));
      m = fmaxf(m, __shfl_xor(m, 32, 64));
      if (kgrp == 0) xch[wn * BM + 16 * (j * WM + wm) + crow] = m;
    }
    __builtin_amdgcn_s_waitcnt(0xc07f & ~(15 << 8));   // LDS writes done (lgkmcnt 0)
    lds_barrier();
#pragma unroll
    for (int j = 0; j < TM; ++j) {
      if (j >= jcount) continue;
      const int row = 16 * (j * WM + wm) + crow;
      if (row >= rows) continue;
      float amax = 0.f;
#pragma unroll
      for (int w = 0; w < WN; ++w) amax = fmaxf(amax, xch[w * BM + row]);
      const bool zero = amax == 0.f;
      const float scale = zero ? 1.0f : amax / 448.0f;
      const float inv = zero ? 0.0f : 448.0f / amax;
      uint8_t* hrow = static_cast<uint8_t*>(cptr_e) + static_cast<long long>(row0_e + row) * ldc_e;
#pragma unroll
      for (int i = 0; i < HT; ++i) {
        const int col = nt * (BN / 2) + wn * (TN * 8) + 16 * i + ccol4;
        const uint32_t q = zero ? 0u
                                : f32x4_to_e4m3(acc[j][i][0] * inv, acc[j][i][1] * inv, acc[j][i][2] * inv,
                                                acc[j][i][3] * inv);
        if (col + 3 < p.N) {
          *reinterpret_cast<uint32_t*>(hrow + col) = q;
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (col + r < p.N) hrow[col + r] = static_cast<uint8_t>(q >> (8 * r));
        }
      }
      if (wn == 0 && kgrp == 0)
        p.c_scale[static_cast<long long>(row0_e + row) * p.c_scale_ld + nt] = scale;
    }
  }
  }  // N tiles of this workgroup
}

template <int WM, int WN, int TM, int TN, int EPI, int ROWB, int NST, bool FP8, bool I8 = false,
          bool W4 = false>
__global__ __launch_bounds__(WM* WN * 64) void grouped_gemm_dma_kernel(GemmArgs p) {
  gemm_dma_body<WM, WN, TM, TN, EPI, false, ROWB, NST, FP8, I8, W4>(p);
}

template <int WM, int WN, int TM, int TN, int EPI, int ROWB, int NST>
__global__ __launch_bounds__(WM* WN * 64) void dense_gemm_dma_kernel(GemmArgs p) {
  gemm_dma_body<WM, WN, TM, TN, EPI, true, ROWB, NST, false>(p);
}

// Experts: units come from the device-built table.
// ------------------------------------------------------------------ unit planner
// One block of 1024 threads, thread g owning group g (G <= 1024, the callers' limit):
// units per group = ceil(n / BM) near-equal slices (rows rounded up to 16), prefix-summed
// over groups, then each group writes its slices.  When extra_rows > 0 there is one more
// group, index G, of extra_rows rows starting at row 0 of its own tensor (the shared
// expert folded into the routed launch).  Its n_x slices are spread evenly through the
// table -- slice i goes right before the units of group floor(i * G / n_x) -- so every
// stretch of consecutive units (the workgroups that run together) mixes the
// compute-heavy shared slices with weight-streaming routed ones.  Units past `cap` (only
// reachable if offsets[G] exceeds the rows the caller sized the workspace for) are
// dropped rather than written out of bounds.  Then the table is cut into kXcds chunks of
// consecutive units, one per XCD, of near-equal cost and at most ceil(cap / kXcds) units
// each, the most a launch sized for `cap` units gives one XCD.  A unit's cost is its
// 16-row tiles, counted as at least cost_floor rows (below that its loads, not its MFMAs,
// set its time), plus one for its prologue and epilogue; cost_floor = BM makes every unit
// cost the same.  Counts and costs are scanned together and every value stays in
// registers, so the table is written once and never read back.
static_assert(kPlanInts == 2 + kXcds, "planner count array: count + chunk bounds");
__global__ __launch_bounds__(1024) void plan_kernel(const int32_t* __restrict__ offsets, int G,
                                                    int rows_if_null, int extra_rows, int BM,
                                                    int cap, int cost_floor, Unit* __restrict__ units,
                                                    int32_t* __restrict__ n_units) {
  __shared__ int32_t wsum[16];
  __shared__ long long csum[16];
  __shared__ int32_t below[kXcds];
  if (threadIdx.x < kXcds) below[threadIdx.x] = 0;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int g = threadIdx.x;
  const int nx = plan_units_of(extra_rows, BM);
  const int per_x = nx > 0 ? plan_slice_rows(extra_rows, nx) : 0;
  int n = 0, start = 0;
  if (g < G) {
    start = offsets ? offsets[g] : 0;
    n = offsets ? offsets[g + 1] - start : rows_if_null;
  }
  const int nu = plan_units_of(n, BM);
  const int per = nu > 0 ? plan_slice_rows(n, nu) : 0;
  const int x0 = g < G ? plan_extra_upto(g - 1, nx, G) : 0;
  const int x1 = g < G ? plan_extra_upto(g, nx, G) : 0;
  auto extra_rows_of = [&](int i) { return min(per_x, extra_rows - i * per_x); };
  auto own_rows_of = [&](int i) { return min(per, n - i * per); };
  // units of groups before g: a block scan of nu
  int incl = nu;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int v = __shfl_up(incl, o, 64);
    if (lane >= o) incl += v;
  }
  if (lane == 63) wsum[w] = incl;
  __syncthreads();
  int base = incl - nu;   // routed units of groups < g
  for (int v = 0; v < w; ++v) base += wsum[v];
  int routed = 0;
  for (int v = 0; v < 16; ++v) routed += wsum[v];
  const int total = min(routed + nx, cap);
  // this thread's table entries: extras at base + x0 .. base + x1 - 1, then its own units
  // at base + x1 ..; their cost (entries past the cap are dropped and cost nothing)
  long long cg = 0;
  for (int i = x0; i < x1; ++i)
    if (base + i < cap) cg += plan_unit_cost(extra_rows_of(i), cost_floor);
  for (int i = 0; i < nu; ++i)
    if (base + x1 + i < cap) cg += plan_unit_cost(own_rows_of(i), cost_floor);
  long long cincl = cg;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const long long v = __shfl_up(cincl, o, 64);
    if (lane >= o) cincl += v;
  }
  if (lane == 63) csum[w] = cincl;
  if (g < G) {
    for (int i = x0; i < x1; ++i) {
      Unit un;
      un.group = G;
      un.row0 = i * per_x;
      un.rows = extra_rows_of(i);
      un.flags = nx == 1 ? kUnitSoleReader : 0;
      un.first = base + x0;
      un.count = x1 - x0;
      if (base + i < cap) units[base + i] = un;
    }
    for (int i = 0; i < nu; ++i) {
      Unit un;
      un.group = g;
      un.row0 = start + i * per;
      un.rows = own_rows_of(i);
      un.flags = nu == 1 ? kUnitSoleReader : 0;
      un.first = base + x1;
      un.count = nu;
      if (base + x1 + i < cap) units[base + x1 + i] = un;
    }
  }
  __syncthreads();
  long long before = cincl - cg;   // cost of the table entries before this thread's
  for (int v = 0; v < w; ++v) before += csum[v];
  long long all = 0;
  for (int v = 0; v < 16; ++v) all += csum[v];
  // units whose cost midpoint lies before x / kXcds of the total
  int cnt[kXcds] = {};
  auto count = [&](int idx, int rows) {
    if (idx >= cap) return;
    const long long c = plan_unit_cost(rows, cost_floor);
#pragma unroll
    for (int x = 1; x < kXcds; ++x) cnt[x] += plan_below(2 * before + c, x, kXcds, all) ? 1 : 0;
    before += c;
  };
  for (int i = x0; i < x1; ++i) count(base + i, extra_rows_of(i));
  for (int i = 0; i < nu; ++i) count(base + x1 + i, own_rows_of(i));
#pragma unroll
  for (int x = 1; x < kXcds; ++x) {
    int v = cnt[x];
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    if (lane == 0 && v != 0) atomicAdd(&below[x], v);
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    n_units[0] = total;
    plan_chunk_bounds(below, total, cap, kXcds, n_units + 1);
  }
}

hipError_t launch_plan(const int32_t* offsets, int G, int rows_if_null, int extra_rows, int block_m,
                       int cap, int cost_floor, Unit* units, int32_t* n_units, hipStream_t st) {
  if (G < 1 || G > 1024) return hipErrorInvalidValue;   // one group per planner thread
  plan_kernel<<<1, 1024, 0, st>>>(offsets, G, rows_if_null, extra_rows, block_m, cap, cost_floor,
                                  units, n_units);
  return hipGetLastError();
}

// ------------------------------------------------------------------ dispatch
namespace {
template <int WM, int WN, int TM, int TN, int EPI, int ROWB, int NST, bool FP8 = false, bool I8 = false,
          bool W4 = false>
hipError_t go_dma(const GemmArgs& a, int max_units, hipStream_t st) {
  constexpr int BN = WN * TN * 16;
  constexpr bool SWIGLU = EPI == EPI_SWIGLU_BF16 || EPI == EPI_SWIGLU_FP8;
  const int tpw = a.tiles_per_wg;
  if (tpw < 1) return hipErrorInvalidValue;
  // several N tiles per workgroup: grouped two-deep int8 / int4 rings with plain stores,
  // whole tiles along N
  if (tpw > 1 && (!(I8 || W4) || NST != 2 || SWIGLU || a.uniform_rows > 0 || a.N % BN != 0))
    return hipErrorInvalidValue;
  const long long per_unit = static_cast<long long>((a.n_tiles + tpw - 1) / tpw) * a.splits;
  const long long slots = (static_cast<long long>(max_units) + kXcds - 1) / kXcds;
  const long long blocks = slots * kXcds * per_unit;
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  if (a.uniform_rows > 0) {
    if constexpr (FP8 || I8 || W4) {
      return hipErrorInvalidValue;  // quantized operands come only from the grouped (routed) path
    } else {
      dense_gemm_dma_kernel<WM, WN, TM, TN, EPI, ROWB, NST>
          <<<static_cast<unsigned>(blocks), WM * WN * 64, 0, st>>>(a);
    }
  } else {
    grouped_gemm_dma_kernel<WM, WN, TM, TN, EPI, ROWB, NST, FP8, I8, W4>
        <<<static_cast<unsigned>(blocks), WM * WN * 64, 0, st>>>(a);
  }
  return hipGetLastError();
}

}  // namespace

int gemm_block_m(GemmCfg cfg, bool fp8) {
  switch (cfg) {
    case CFG_BIG: return fp8 ? 256 : 320;
    case CFG_SMALL: return 32;
    default: return 64;
  }
}

int gemm_block_n(GemmCfg) { return 256; }

int gemm_wgs_per_cu(GemmCfg, bool) {
  // LDS per workgroup against the 160 KB of a CU: every short tile holds a 120-156 KB ring
  return 1;
}

int gemm_k_step(GemmCfg cfg, bool fp8, bool i8, bool w4, int K) {
  if (fp8) return 128;                                        // one scale block per stage
  if (w4 && cfg == CFG_SMALL && K % 256 == 0) return 256;     // whole lines of packed weights
  return (i8 || w4) ? 128 : 64;                               // 128-byte rows per stage
}

hipError_t launch_gemm(GemmCfg cfg, Epilogue epi, bool fp8, const GemmArgs& a, int max_units,
                       hipStream_t st) {
  switch (cfg) {
    case CFG_BIG:
      if (fp8) {
        if (a.uniform_rows > 0) return hipErrorInvalidValue;
        // fp8 fragments are 32 bytes per lane and the promotion needs the scales next to
        // the accumulators: 256 x 256 tiles, 2 x 4 wavefronts of 128 x 64 that keep four
        // weight fragments resident and stream the activation fragments
        if (epi == EPI_SWIGLU_FP8) return go_dma<2, 4, 8, 4, EPI_SWIGLU_FP8, 128, 2, true>(a, max_units, st);
        if (epi == EPI_STORE_BF16) return go_dma<2, 4, 8, 4, EPI_STORE_BF16, 128, 2, true>(a, max_units, st);
        return hipErrorInvalidValue;
      }
      if (epi == EPI_SWIGLU_BF16) return go_dma<4, 2, 5, 8, EPI_SWIGLU_BF16, 128, 2>(a, max_units, st);
      if (epi == EPI_STORE_BF16) return go_dma<4, 2, 5, 8, EPI_STORE_BF16, 128, 2>(a, max_units, st);
      return hipErrorInvalidValue;
    case CFG_SMALL:
      if (fp8) {
        if (a.uniform_rows > 0) return hipErrorInvalidValue;
        if (epi == EPI_SWIGLU_FP8) return go_dma<1, 4, 2, 4, EPI_SWIGLU_FP8, 128, 4, true>(a, max_units, st);
        if (epi == EPI_STORE_BF16) return go_dma<1, 4, 2, 4, EPI_STORE_BF16, 128, 4, true>(a, max_units, st);
        if (epi == EPI_STORE_F32) return go_dma<1, 4, 2, 4, EPI_STORE_F32, 128, 4, true>(a, max_units, st);
        return hipErrorInvalidValue;
      }
      if (epi == EPI_SWIGLU_BF16) return go_dma<1, 4, 2, 4, EPI_SWIGLU_BF16, 128, 4>(a, max_units, st);
      if (epi == EPI_STORE_BF16) return go_dma<1, 4, 2, 4, EPI_STORE_BF16, 128, 4>(a, max_units, st);
      if (epi == EPI_STORE_F32) return go_dma<1, 4, 2, 4, EPI_STORE_F32, 128, 4>(a, max_units, st);
      return hipErrorInvalidValue;
    case CFG_GATE:
      if (epi != EPI_STORE_F32 || fp8) return hipErrorInvalidValue;
      return go_dma<1, 4, 4, 4, EPI_STORE_F32, 128, 3>(a, max_units, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_gemm_i8(GemmCfg cfg, Epilogue epi, bool w4, const GemmArgs& a, int max_units,
                          hipStream_t st) {
  if (a.uniform_rows > 0 || !a.a_scale || !a.b_scale) return hipErrorInvalidValue;
  if (a.splits < 1 || a.K % 128 || a.k_chunk % 128) return hipErrorInvalidValue;
  if (epi != EPI_SWIGLU_BF16 && epi != EPI_STORE_BF16 && epi != EPI_STORE_F32) return hipErrorInvalidValue;
  if (epi == EPI_STORE_F32 && cfg != CFG_SMALL) return hipErrorInvalidValue;
  const bool sw = epi == EPI_SWIGLU_BF16;
  if (epi == EPI_STORE_F32) {   // split-K partials of a decode-sized grouped GEMM
    if (w4 && a.K % 256 == 0 && a.k_chunk % 256 == 0)
      return go_dma<1, 4, 2, 4, EPI_STORE_F32, 256, 3, false, false, true>(a, max_units, st);
    if (w4) return go_dma<1, 4, 2, 4, EPI_STORE_F32, 128, 4, false, false, true>(a, max_units, st);
    return go_dma<1, 4, 2, 4, EPI_STORE_F32, 128, 4, false, true>(a, max_units, st);
  }
  switch (cfg) {
    case CFG_BIG:
      if (w4) {
        return sw ? go_dma<4, 2, 5, 8, EPI_SWIGLU_BF16, 128, 2, false, false, true>(a, max_units, st)
                  : go_dma<4, 2, 5, 8, EPI_STORE_BF16, 128, 2, false, false, true>(a, max_units, st);
      }
      return sw ? go_dma<4, 2, 5, 8, EPI_SWIGLU_BF16, 128, 2, false, true>(a, max_units, st)
                : go_dma<4, 2, 5, 8, EPI_STORE_BF16, 128, 2, false, true>(a, max_units, st);
    case CFG_SMALL:
      if (w4 && a.K % 256 == 0 && a.k_chunk % 256 == 0) {
        // 256-element stages: whole 128-byte lines of packed weights, 3-deep ring (40 KB stages)
        return sw ? go_dma<1, 4, 2, 4, EPI_SWIGLU_BF16, 256, 3, false, false, true>(a, max_units, st)
                  : go_dma<1, 4, 2, 4, EPI_STORE_BF16, 256, 3, false, false, true>(a, max_units, st);
      }
      if (w4) {
        return sw ? go_dma<1, 4, 2, 4, EPI_SWIGLU_BF16, 128, 4, false, false, true>(a, max_units, st)
                  : go_dma<1, 4, 2, 4, EPI_STORE_BF16, 128, 4, false, false, true>(a, max_units, st);
      }
      return sw ? go_dma<1, 4, 2, 4, EPI_SWIGLU_BF16, 128, 4, false, true>(a, max_units, st)
                : go_dma<1, 4, 2, 4, EPI_STORE_BF16, 128, 4, false, true>(a, max_units, st);
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace moe
