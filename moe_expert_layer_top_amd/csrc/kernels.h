// Internal launchers of the MoE kernels (not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kSegSlots = 1024;  // routing slots per counting-sort segment (one wavefront)

// Unit of grouped-GEMM work: rows [row0, row0 + rows) of group `group`.  The units of
// one group (and the consecutive slices of the extra group) form a run of consecutive
// table entries: `first` is the table index of the run's first unit, `count` its length.
struct Unit {
  int32_t group, row0, rows, flags, first, count;
};
// The planner's count array: [0] units in the table, [1 + x] (x = 0..kXcds) first unit
// of XCD x's chunk of the table ([1 + kXcds] = the count again).
constexpr int kPlanInts = 2 + 8;   // 8 = kXcds (checked where both are visible)
// Unit::flags bit: no other unit reads this group's weights (the weight panel is streamed
// once, with a non-temporal cache policy)
constexpr int32_t kUnitSoleReader = 1;

enum Epilogue : int {
  EPI_SWIGLU_BF16 = 0,  // h = silu(gate) * up, stored bf16
  EPI_SWIGLU_FP8 = 1,   // h quantized to e4m3 with one fp32 scale per 1x128 block
  EPI_STORE_BF16 = 2,   // C stored bf16
  EPI_STORE_F32 = 3,    // C stored fp32 (split-k partials)
};

struct GemmArgs {
  const uint8_t* A;         // activation rows
  long long lda;            // row pitch in bytes
  const float* a_scale;     // fp8: [rows, K/128]; int8: [rows] (one per row)
  long long a_scale_ld;     // floats per row (fp8)
  const uint8_t* B;         // weights of group 0
  long long ldb;            // row pitch in bytes
  long long b_group;        // bytes between groups
  const float* b_scale;     // fp8: [Brows/128, K/128] per group; int8: [Brows] per group
  long long b_scale_group;  // floats between groups
  long long b_scale_ld;     // floats per scale row (fp8)
  void* C;                  // output
  long long ldc;            // elements per output row
  long long c_split;        // elements between split-k partial outputs
  float* c_scale;           // EPI_SWIGLU_FP8: [rows, N/128]
  long long c_scale_ld;
  const Unit* units;        // device unit table (unused when uniform_rows > 0)
  const int32_t* n_units;   // device unit count and XCD chunk bounds (kPlanInts ints;
                            // unused when uniform_rows > 0)
  int uniform_rows;         // > 0: one group of this many rows cut into BM slices
  int N;                    // logical output columns
  int K;                    // reduction length in elements
  int up_off;               // swiglu: first row of the up projection (= I)
  int n_tiles;              // output tiles along N
  // N tiles each workgroup computes one after another (its load ring running on from one
  // tile into the next); > 1 only for grouped plain-store tiles with a two-deep ring, no
  // fp8, and N a whole number of tiles
  int tiles_per_wg = 1;
  int splits;               // split-k factor
  int k_chunk;              // elements of K per split (multiple of the stage depth)
  // Alternate group (bf16 and int8 DMA kernels): units whose group equals alt_group read
  // A2 (pitch lda2) and the single weight panel B2 (pitch ldb, like the primary groups),
  // and write C2 (pitch ldc2); int8 units take their scales from a_scale2 [rows] and
  // b_scale2 [Brows].  -1: none.
  // Gathered activations (DMA kernels): when set, row r of a unit of the primary groups
  // is row gather[row0 + r] / gather_div of A (x, or its per-token codes, indexed by
  // token through the slot order of the expert sort) instead of row row0 + r; fp8 and
  // int8 rows take their activation scales from the same token row of a_scale.
  const int32_t* gather = nullptr;
  int gather_div = 1;
  int alt_group = -1;
  const uint8_t* A2 = nullptr;
  long long lda2 = 0;
  const uint8_t* B2 = nullptr;
  void* C2 = nullptr;
  long long ldc2 = 0;
  const float* a_scale2 = nullptr;
  const float* b_scale2 = nullptr;
  long long c_split2 = 0;   // EPI_STORE_F32: elements between the alternate group's partials
};

enum GemmCfg : int {
  CFG_BIG = 0,    // 320 (fp8: 256) x 256 tiles, 8 wavefronts: prefill-sized groups
  CFG_SMALL = 1,  // 32 x 256 tiles, 4 wavefronts: decode-sized groups
  CFG_GATE = 2,   // 64 x 256 tiles, 4 wavefronts: gate projection
};

int gemm_block_m(GemmCfg cfg, bool fp8);
int gemm_block_n(GemmCfg cfg);
hipError_t launch_gemm(GemmCfg cfg, Epilogue epi, bool fp8, const GemmArgs& a, int max_units,
                       hipStream_t st);
// W8A8 / W4A8 grouped GEMM: int8 A, int8 B (w4: packed int4 B, ldb and b_group in bytes of
// the packed rows), per-row a_scale and per-channel b_scale, bf16 result (EPI_SWIGLU_BF16
// or EPI_STORE_BF16); the bf16 tiles (gemm_block_m(cfg, false)).
hipError_t launch_gemm_i8(GemmCfg cfg, Epilogue epi, bool w4, const GemmArgs& a, int max_units,
                          hipStream_t st);

// Builds the unit table of a grouped GEMM on the device.  `offsets` [G+1] or, when
// NULL, one group of `rows_if_null` rows; extra_rows > 0 appends group G of that many
// rows (rows counted from 0 in its own tensor).
hipError_t launch_plan(const int32_t* offsets, int G, int rows_if_null, int extra_rows, int block_m,
                       int cap, int cost_floor, Unit* units, int32_t* n_units, hipStream_t st);

// Router variant (the plain router: {0, 1, 1, 1, 1, 1.0f}); validated by the caller.
struct RouterArgs {
  int scoring = 0;       // 0 sigmoid, 1 softmax over all experts
  int renormalize = 1;
  int n_group = 1;
  int topk_group = 1;
  int group_topn = 1;
  float scale = 1.0f;
};

hipError_t launch_topk(const float* part, int splits, long long split_stride, int T, int E, int k,
                       const float* bias, float* logits_out, int32_t* idx, float* w,
                       hipStream_t st,
                       const RouterArgs& router = RouterArgs());

// counts_ws: [nseg * E] int32, seg_err: [nseg] int32 with nseg = ceil(R / kSegSlots).
// err_word is overwritten with 1 if any id fell outside [e_base, e_base + E), else 0.
hipError_t launch_routing(const int32_t* ids, long long R, int e_base, int E, int32_t* counts_ws,
                          int32_t* seg_err, int32_t* err_word, int32_t* eri, int32_t* sorted_src,
                          int32_t* tpe, int32_t* offsets, hipStream_t st);

// Writes token t's row (fp8: its 1x128 codes and scales) to rows eri[t*k .. t*k+k-1];
// eri NULL (fp8, k = 1): to row t, the per-token codes in token order.
hipError_t launch_expand(const void* x, int T, int H, int k, int act_bytes, bool quant_fp8,
                         const int32_t* eri, void* out, float* out_scale, hipStream_t st);

// int8 per-row quantization of bf16 rows (W8A8 activations).  dst_rows [rows * k] or NULL
// (in place); n_rows: device count of rows that hold data, or NULL (all).
hipError_t launch_quant_rows_i8(const void* src, int rows, int cols, int k, const int32_t* dst_rows,
                                const int32_t* n_rows, int8_t* out, float* out_scale,
                                hipStream_t st);

hipError_t launch_finalize(const void* y, const void* skip, const float* w, const int32_t* eri,
                           void* out, int T, int H, int k, int act_bytes, hipStream_t st);

// Split-K reductions over fp32 partials [S][rows][N] (slice stride split_stride floats),
// one block per row, rows >= *n_rows skipped (n_rows NULL: all rows).
// swiglu: N = 2I (gate | up) -> h [rows, I] bf16, or fp8 codes + h_scale [rows, I/128].
hipError_t launch_swiglu_reduce(const float* part, int S, long long split_stride, int rows, int I,
                                const int32_t* n_rows, void* h, bool fp8, float* h_scale,
                                hipStream_t st);
// sum: -> y [rows, N] bf16.
hipError_t launch_sum_reduce(const float* part, int S, long long split_stride, int rows, int N,
                             const int32_t* n_rows, void* y, hipStream_t st);

// Elements of K per stage of the grouped GEMM launched for (cfg, dtype, K): split-K
// slices must be whole multiples of it.
int gemm_k_step(GemmCfg cfg, bool fp8, bool i8, bool w4, int K);
// Workgroups of the grouped GEMM launched for (cfg, fp8) that one CU holds at once.
int gemm_wgs_per_cu(GemmCfg cfg, bool fp8);

// fp32 path (plain FMA kernels; fp32 matrix and vector peaks are equal on gfx950)
hipError_t launch_gemm_nt_f32(const float* A, const float* B, float* C, int M, int N, int K,
                              hipStream_t st);
// offsets == NULL: one group holding all R_max rows.
hipError_t launch_grouped_ffn_f32(const float* a, const int32_t* offsets, int G, int R_max,
                                  const float* w13, const float* w2, float* h, float* y, int H,
                                  int I, hipStream_t st);

}  // namespace moe
