// C ABI of the MoE layer: argument validation, workspace layout and the launch
// sequence of each call.  Declarations and contracts are in include/moe.h.
//
// [MND] = page "Lower latency and higher throughput with multi-node DeepSeek
//         deployment"; [R1P] = page "CANN/cann-recipes-infer: DeepSeek-R1
//         prefill optimization".

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <climits>
#include <cstdint>
#include <initializer_list>
#include <mutex>

#include "../../include/moe.h"
#include "addr.h"
#include "kernels.h"

namespace {

using moe::GemmArgs;
using moe::Unit;

constexpr size_t kAlign = 256;
static_assert(moe::kPlanInts * sizeof(int32_t) <= kAlign, "planner count array fits its slot");
constexpr int kMaxE = 1024;
constexpr int kMaxK = 64;
constexpr int kGateMaxSplits = 16;
constexpr int kSmallTileRows = 512;  // at most this many rows in all: the short tile
constexpr int kMaxFfnSplits = 8;     // split-K slices of a decode-sized expert GEMM
constexpr long long kSplitBelowWgs = 128;  // split-K only grids smaller than this
constexpr long long kCus = 256;             // MI355X compute units
constexpr int kMinSliceStages = 8;        // K stages per split-K slice, at least

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

// Tensor pointers must be 16-byte aligned (the kernels move 16-byte vectors); null
// pointers, the optional arguments, pass.
bool aligned16(std::initializer_list<const void*> ps) {
  for (const void* q : ps)
    if (reinterpret_cast<uintptr_t>(q) & 15u) return false;
  return true;
}

int elem_bytes(int dt) { return dt == MOE_F32 ? 4 : dt == MOE_BF16 ? 2 : 1; }  // int4: 1 (bound)

// int8 activations with per-row scales: W8A8 and W4A8 experts
bool q8_weights(const moe_shape* s) { return s->wt == MOE_INT8 || s->wt == MOE_INT4; }

bool dtypes_ok(const moe_shape* s) {
  if (s->act == MOE_F32) return s->wt == MOE_F32;
  if (s->act == MOE_BF16)
    return s->wt == MOE_BF16 || s->wt == MOE_FP8_E4M3 || s->wt == MOE_INT8 || s->wt == MOE_INT4;
  return false;
}

// Shape checks shared by every call (I sizes are checked by the calls that use them).
moe_status check_shape(const moe_shape* s) {
  if (!s) return MOE_EINVAL;
  if (s->T < 0 || s->H <= 0 || s->E < 1 || s->k < 1 || s->k > s->E) return MOE_EINVAL;
  if (s->act != MOE_F32 && s->act != MOE_BF16) return MOE_EUNSUPPORTED;
  if (s->wt != MOE_F32 && s->wt != MOE_BF16 && s->wt != MOE_FP8_E4M3 && s->wt != MOE_INT8 &&
      s->wt != MOE_INT4)
    return MOE_EUNSUPPORTED;
  if (!dtypes_ok(s)) return MOE_EUNSUPPORTED;
  if (s->E > kMaxE || s->k > kMaxK) return MOE_EUNSUPPORTED;
  if (s->act == MOE_F32 ? (s->H % 4) : (s->H % 128)) return MOE_EUNSUPPORTED;
  if (static_cast<long long>(s->T) * s->k > INT32_MAX / 2) return MOE_EUNSUPPORTED;
  return MOE_OK;
}

moe_status check_inter(const moe_shape* s, int I) {
  if (I <= 0) return MOE_EINVAL;
  if (s->act != MOE_F32 && I % 128) return MOE_EUNSUPPORTED;
  // weight panels are addressed with 32-bit offsets inside one expert
  if (2LL * I * s->H * elem_bytes(s->wt) >= (1LL << 31)) return MOE_EUNSUPPORTED;
  return MOE_OK;
}

// Router variant -> kernel arguments; false if it breaks the rules stated in moe.h.
bool router_args(const moe_shape* s, const moe_router* r, moe::RouterArgs* out) {
  moe::RouterArgs a;
  if (r) {
    if ((r->scoring != MOE_SCORE_SIGMOID && r->scoring != MOE_SCORE_SOFTMAX) ||
        (r->renormalize != 0 && r->renormalize != 1))
      return false;
    if (r->n_group < 1 || r->n_group > 64 || s->E % r->n_group) return false;
    const int gsz = s->E / r->n_group;
    if (r->topk_group < 1 || r->topk_group > r->n_group) return false;
    if ((r->group_topn != 1 && r->group_topn != 2) || r->group_topn > gsz) return false;
    if (static_cast<long long>(s->k) > static_cast<long long>(r->topk_group) * gsz) return false;
    if (!(r->scale > 0.0f) || !std::isfinite(r->scale)) return false;
    a.scoring = r->scoring;
    a.renormalize = r->renormalize;
    a.n_group = r->n_group;
    a.topk_group = r->topk_group;
    a.group_topn = r->group_topn;
    a.scale = r->scale;
  }
  *out = a;
  return true;
}

int nseg_of(long long R) { return static_cast<int>((R + moe::kSegSlots - 1) / moe::kSegSlots); }

// ------------------------------------------------------------------ gate split-k
struct GatePlan {
  int splits, k_chunk;
};

// The gate's 64-row tiles split K until the grid holds about one workgroup per CU (at most
// kGateMaxSplits slices): prefill keeps its partials small (c2: 2 slices, gate 0.063 ->
// 0.058 ms against 4), decode gets enough workgroups to stream x and the gate matrix.
GatePlan gate_plan(const moe_shape* s) {
  if (s->act == MOE_F32) return {1, s->H};
  const int bm = moe::gemm_block_m(moe::CFG_GATE, false);
  const int mtiles = std::max(1, (s->T + bm - 1) / bm);
  const int ksteps = s->H / 64;
  int splits = std::min(ksteps, std::max(1, static_cast<int>(kCus) / mtiles));
  splits = std::min(splits, kGateMaxSplits);
  const int steps_per = (ksteps + splits - 1) / splits;
  splits = (ksteps + steps_per - 1) / steps_per;
  return {splits, steps_per * 64};
}

// ------------------------------------------------------------------ grouped FFN plan
moe::GemmCfg ffn_cfg(int G, int R_max) {
  // decode-sized groups (a few rows each) take the short tile, prefill the tall one; so
  // do small batches in few groups (the dense shared expert at decode), which the tall
  // tile would give a handful of workgroups on a 256-CU machine
  return (G > 0 && (R_max <= 64LL * G || R_max <= kSmallTileRows)) ? moe::CFG_SMALL
                                                                    : moe::CFG_BIG;
}

// Upper bound on the units the planner writes: every group of n > 0 rows makes
// ceil(n / bm) <= n / bm + 1 units; the extra group (if any) likewise.
int max_units(moe::GemmCfg cfg, bool fp8, int G, int R_max, int extra_rows = 0) {
  const int bm = moe::gemm_block_m(cfg, fp8);
  return R_max / bm + std::min(G, R_max) + (extra_rows > 0 ? extra_rows / bm + 1 : 0);
}

// Split-K of a decode-sized grouped FFN ([MND §Quantization]: for some shapes and small
// batches split-K lowers the latency).  When the short-tile grid would leave half the
// CUs idle (units x N tiles < 128: a token or two of a model with few, narrow experts;
// DeepSeek-shaped decode keeps at least 128 workgroups per GEMM, which already stream
// the weights at HBM speed), each GEMM splits its reduction into up to
// kMaxFfnSplits slices of at least kMinSliceStages stages (so the ring's prologue and the
// partial traffic stay small against the weights a slice streams) and stores fp32
// partials, which a reduction
// kernel adds in slice order before the SwiGLU (first GEMM) or the bf16 rounding (second).
// Everything here is known on the host, so workspace sizes follow from the shape.
struct FfnSplit {
  int s1, kc1, s2, kc2;  // slices and K elements per slice of the two GEMMs
  bool on() const { return s1 > 1 || s2 > 1; }
};

int split_of(long long wgs, long long capacity, int K, int kstep, int* kc) {
  const int steps = K / kstep;
  int sp = 1;
  // as many slices as one round of resident workgroups holds: more would queue a second round
  if (wgs < kSplitBelowWgs)
    sp = static_cast<int>(std::min<long long>(kMaxFfnSplits, capacity / std::max(1LL, wgs)));
  sp = std::max(1, std::min(sp, steps / kMinSliceStages));
  const int per = (steps + sp - 1) / sp;
  sp = (steps + per - 1) / per;
  *kc = per * kstep;
  return sp;
}

// Work units of a grouped GEMM before the plan runs (a lower bound): every non-empty group
// makes one at least (one group: its row slices), plus the extra group's row slices.
long long est_units(int G, int R_max, int extra_rows, int bm) {
  return (G == 1 ? (R_max + bm - 1) / bm : std::min(G, R_max)) + (extra_rows + bm - 1) / bm;
}

FfnSplit ffn_split(const moe_shape* s, int G, int R_max, int I, int extra_rows = 0) {
  FfnSplit f{1, s->H, 1, I};
  if (s->act == MOE_F32 || G < 1 || R_max <= 0) return f;
  const moe::GemmCfg cfg = ffn_cfg(G, R_max);
  if (cfg != moe::CFG_SMALL) return f;
  const bool fp8 = s->wt == MOE_FP8_E4M3, i8 = q8_weights(s), w4 = s->wt == MOE_INT4;
  const int bm = moe::gemm_block_m(cfg, fp8), bn = moe::gemm_block_n(cfg);
  const long long units = est_units(G, R_max, extra_rows, bm);
  const long long cap = static_cast<long long>(kCus) * moe::gemm_wgs_per_cu(cfg, fp8);
  const int s1 = split_of(units * (2LL * I / bn), cap, s->H, moe::gemm_k_step(cfg, fp8, i8, w4, s->H),
                          &f.kc1);
  const int s2 = split_of(units * ((s->H + bn - 1) / bn), cap, I,
                          moe::gemm_k_step(cfg, fp8, i8, w4, I), &f.kc2);
  // each GEMM splits on its own (one unit table serves both; a GEMM that does not split
  // keeps its fused epilogue)
  f.s1 = s1;
  f.s2 = s2;
  if (s1 == 1) f.kc1 = s->H;
  if (s2 == 1) f.kc2 = I;
  return f;
}

// The shared expert's dtypes: W8A8 beside W8A8 or W4A8 routed experts ([V32 §quantization
// strategy] quantizes it W8A8 in both), else its weights are in the activation dtype.
moe_shape shared_shape(const moe_shape* s) {
  moe_shape sh = *s;
  sh.wt = q8_weights(s) ? MOE_INT8 : s->act;
  return sh;
}

// The shared expert runs inside the routed grouped-GEMM launches (as one extra group
// whose units read x and the shared weights) when it has the routed experts' shape
// and dtype: bf16 activations, bf16 or int8 weights, I_shared == I.
bool merge_shared(const moe_shape* s) {
  return s->act == MOE_BF16 && (s->wt == MOE_BF16 || s->wt == MOE_INT8) && s->I_shared == s->I;
}

// N tiles per workgroup of the unsplit down projection with tall int8 / int4 tiles: the
// ring's one stage in flight carries on across a tile boundary (the next tile's first
// stage loads while this tile's epilogue stores) and the workgroup's start-up (unit
// read, offsets, first load) is paid once per several tiles.  Four, or two, while the
// grid still holds a round of workgroups for the CUs (c6's down projection: 1.51 ->
// 1.46 ms against one tile).  The bf16 tall tiles keep one tile per workgroup: with the
// units of an expert walked N tile major on one XCD (the planner's chunks) and four
// loader wavefronts, grouping no longer pays there (c2: 2.25 ms with one tile, 2.27 with
// four, which also re-read the unit's rows of h from the last-level cache).  The gate /
// up projection keeps one tile per workgroup: there a second tile re-reads the unit's
// activation rows (14 KB each at H = 7168).  The decode tiles keep one tile per
// workgroup in both GEMMs: grouping four measured 3-7% slower (c7, c8).
int down_tiles_per_wg(moe::GemmCfg cfg, bool fp8, bool q8, long long units, int N, int bn) {
  if (cfg != moe::CFG_BIG || fp8 || !q8 || N % bn != 0) return 1;
  const long long tiles = N / bn;
  for (int t : {4, 2})
    if (units * ((tiles + t - 1) / t) >= kCus) return t;
  return 1;
}

// The first expert GEMM gathers the routed rows from the token-order activations
// through the sort's slot order, so the expanded copy is never written: x itself for
// bf16 experts, x's per-token codes (fp8 1x128 blocks, int8 rows: one quantization per
// token instead of k copies) for fp8 and W8A8 experts.  W4A8 experts keep the expanded
// rows: their 256-element stages ran slower on gathered rows (decode GEMM1 +6%).
// 32-bit row offsets: T * H * bytes per element must stay below 4 GiB.
bool gather_rows(const moe_shape* s) {
  if (s->act != MOE_BF16 || s->wt == MOE_INT4) return false;
  return moe::lane_offsets_fit_u32(s->wt == MOE_BF16 ? 2 : 1, s->T, s->H);
}

struct FfnLayout {
  size_t units, n_units, h, h_scale, hq, h2, h2_scale, h2q, part, part2, total;
};

// extra_rows > 0: room for the extra group's units and its intermediate h2 [extra_rows, I]
// (int8: with its row scales and codes).
FfnLayout ffn_layout(const moe_shape* s, int G, int R_max, int I, int extra_rows = 0) {
  FfnLayout L{};
  size_t o = 0;
  if (s->act == MOE_F32) {
    L.h = o;
    o += align_up(static_cast<size_t>(R_max) * I * 4);
    L.total = o;
    return L;
  }
  const moe::GemmCfg cfg = ffn_cfg(G, R_max);
  L.units = o;
  o += align_up(static_cast<size_t>(std::max(
                    1, max_units(cfg, s->wt == MOE_FP8_E4M3, G, R_max, extra_rows))) *
                sizeof(Unit));
  L.n_units = o;
  o += kAlign;
  L.h = o;
  const bool fp8 = s->wt == MOE_FP8_E4M3;
  const bool i8 = q8_weights(s);
  o += align_up(static_cast<size_t>(R_max) * I * (fp8 ? 1 : 2));
  L.h_scale = o;
  if (fp8) o += align_up(static_cast<size_t>(R_max) * (I / 128) * 4);
  if (i8) o += align_up(static_cast<size_t>(R_max) * 4);   // one scale per row of h
  L.hq = o;
  if (i8) o += align_up(static_cast<size_t>(R_max) * I);   // h quantized per row
  L.h2 = o;
  if (extra_rows > 0) o += align_up(static_cast<size_t>(extra_rows) * I * 2);
  L.h2_scale = o;
  if (extra_rows > 0 && i8) o += align_up(static_cast<size_t>(extra_rows) * 4);
  L.h2q = o;
  if (extra_rows > 0 && i8) o += align_up(static_cast<size_t>(extra_rows) * I);
  // split-K partials of either GEMM (the first is reduced before the second runs), and
  // of the extra group's rows
  const FfnSplit sp = ffn_split(s, G, R_max, I, extra_rows);
  const size_t per_row = 4 * std::max(static_cast<size_t>(sp.s1 > 1 ? sp.s1 : 0) * 2 * I,
                                      static_cast<size_t>(sp.s2 > 1 ? sp.s2 : 0) * s->H);
  L.part = o;
  o += align_up(static_cast<size_t>(R_max) * per_row);
  L.part2 = o;
  if (extra_rows > 0) o += align_up(static_cast<size_t>(extra_rows) * per_row);
  L.total = o;
  return L;
}

// ------------------------------------------------------------------ layer layout
struct Layout {
  size_t err, seg_err, part, logits, idx, w, counts, tpe, offsets, eri, sorted_src, ex, ex_scale,
      y, ffn, sh_out, sh_xq, sh_xs, sh_ffn, total;
};

Layout layer_layout(const moe_shape* s) {
  Layout L{};
  const size_t T = static_cast<size_t>(s->T), E = static_cast<size_t>(s->E);
  const size_t R = T * s->k, H = static_cast<size_t>(s->H);
  const GatePlan gp = gate_plan(s);
  const bool fp8 = s->wt == MOE_FP8_E4M3;
  const int ab = elem_bytes(s->act);
  size_t o = 0;
  L.err = o;           o += kAlign;
  L.seg_err = o;       o += align_up(static_cast<size_t>(std::max(1, nseg_of(R))) * 4);
  L.part = o;          o += align_up(static_cast<size_t>(gp.splits) * T * E * 4);
  L.logits = o;        o += align_up(T * E * 4);
  L.idx = o;           o += align_up(R * 4);
  L.w = o;             o += align_up(R * 4);
  L.counts = o;        o += align_up(static_cast<size_t>(std::max(1, nseg_of(R))) * E * 4);
  L.tpe = o;           o += align_up(E * 4);
  L.offsets = o;       o += align_up((E + 1) * 4);
  L.eri = o;           o += align_up(R * 4);
  L.sorted_src = o;    o += align_up(R * 4);
  const bool i8 = q8_weights(s);
  // expanded rows, or (gathered, quantized experts) the per-token codes in token order
  const bool gathered = gather_rows(s);
  const size_t qrows = gathered ? T : R;
  L.ex = o;            if (!gathered) o += align_up(R * H * (fp8 || i8 ? 1 : ab));
                       else if (fp8 || i8) o += align_up(T * H);
  L.ex_scale = o;      if (fp8) o += align_up(qrows * (H / 128) * 4);
                       if (i8) o += align_up(qrows * 4);
  L.y = o;             o += align_up(R * H * ab);
  const bool merged = merge_shared(s);
  L.ffn = o;           o += ffn_layout(s, s->E, static_cast<int>(R), s->I, merged ? s->T : 0).total;
  L.sh_out = o;        o += align_up(T * H * ab);
  // W8A8 shared expert on the second stream (or beside expanded rows): its own int8
  // codes and scales of the tokens in token order
  L.sh_xq = o;         if (i8) o += align_up(T * H);
  L.sh_xs = o;         if (i8) o += align_up(T * 4);
  const moe_shape sh = shared_shape(s);
  L.sh_ffn = o;        if (!merged) o += ffn_layout(&sh, 1, s->T, s->I_shared).total;
  L.total = o;
  return L;
}

template <typename P>
P* at(void* ws, size_t off) {
  return reinterpret_cast<P*>(static_cast<uint8_t*>(ws) + off);
}

moe_status hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_EHIP; }

// Optional event marks at launch boundaries (moe_layer_profiled).
struct Prof {
  hipEvent_t* ev = nullptr;
  int n = 0;
  hipError_t mark(int i, hipStream_t st) const {
    return (ev && i < n && ev[i]) ? hipEventRecord(ev[i], st) : hipSuccess;
  }
};

// ------------------------------------------------------------------ launch sequences
moe_status run_gate_topk(const moe_shape* s, const void* x, const void* w_gate, const float* bias,
                         float* logits, int32_t* idx, float* w, float* part, hipStream_t st,
                         const Prof& prof = Prof(), const moe::RouterArgs& router = moe::RouterArgs()) {
  const GatePlan gp = gate_plan(s);
  hipError_t e;
  if (s->act == MOE_F32) {
    e = moe::launch_gemm_nt_f32(static_cast<const float*>(x), static_cast<const float*>(w_gate),
                                part, s->T, s->E, s->H, st);
  } else {
    GemmArgs a{};
    a.A = static_cast<const uint8_t*>(x);
    a.lda = static_cast<long long>(s->H) * 2;
    a.B = static_cast<const uint8_t*>(w_gate);
    a.ldb = static_cast<long long>(s->H) * 2;
    a.b_group = 0;
    a.C = part;
    a.ldc = s->E;
    a.c_split = static_cast<long long>(s->T) * s->E;
    a.uniform_rows = s->T;
    a.N = s->E;
    a.K = s->H;
    a.n_tiles = (s->E + moe::gemm_block_n(moe::CFG_GATE) - 1) / moe::gemm_block_n(moe::CFG_GATE);
    a.splits = gp.splits;
    a.k_chunk = gp.k_chunk;
    const int bm = moe::gemm_block_m(moe::CFG_GATE, false);
    e = s->T > 0 ? moe::launch_gemm(moe::CFG_GATE, moe::EPI_STORE_F32, false, a,
                                    (s->T + bm - 1) / bm, st)
                 : hipSuccess;
  }
  if (e != hipSuccess || prof.mark(MOE_EV_GATE, st) != hipSuccess) return MOE_EHIP;
  e = moe::launch_topk(part, gp.splits, static_cast<long long>(s->T) * s->E, s->T, s->E, s->k, bias,
                       logits, idx, w, st, router);
  if (e != hipSuccess || prof.mark(MOE_EV_TOPK, st) != hipSuccess) return MOE_EHIP;
  return MOE_OK;
}

struct FfnIo {
  const void* a;
  const float* a_scale;
  const int32_t* offsets;  // NULL: one group of R_max rows
  const void* w13;
  const float* w13_scale;
  const void* w2;
  const float* w2_scale;
  void* y;
  // when set, sorted row r is row gather[r] / gather_div of `a` (x or its per-token
  // codes, or rows in any order), so the expert-sorted copy is never written
  const int32_t* gather = nullptr;
  int gather_div = 1;
};

// `alt` (bf16 only): the shared expert as group G of alt_rows rows in the same
// launches; alt->a is x [alt_rows, H], alt->w13 / alt->w2 its weights, alt->y its
// output [alt_rows, H].
moe_status run_ffn(const moe_shape* s, int G, int R_max, int I, const FfnIo& io, void* ws,
                   hipStream_t st, const Prof& prof = Prof(), int ev_plan = -1, int ev_ffn1 = -1,
                   int ev_ffn2 = -1, const FfnIo* alt = nullptr, int alt_rows = 0) {
  if (!alt) alt_rows = 0;
  if (R_max == 0 && alt_rows == 0) return MOE_OK;
  const FfnLayout L = ffn_layout(s, G, R_max, I, alt_rows);
  const int H = s->H;
  if (s->act == MOE_F32) {
    // one fused launch: its boundaries are marked as the plan (empty) and both GEMMs
    if (prof.mark(ev_plan, st) != hipSuccess) return MOE_EHIP;
    const moe_status fst = hip_status(moe::launch_grouped_ffn_f32(
        static_cast<const float*>(io.a), io.offsets, G, R_max, static_cast<const float*>(io.w13),
        static_cast<const float*>(io.w2), at<float>(ws, L.h), static_cast<float*>(io.y), H, I, st));
    if (fst != MOE_OK) return fst;
    if (prof.mark(ev_ffn1, st) != hipSuccess || prof.mark(ev_ffn2, st) != hipSuccess) return MOE_EHIP;
    return MOE_OK;
  }
  const bool fp8 = s->wt == MOE_FP8_E4M3;
  const bool i8 = q8_weights(s);
  const bool w4 = s->wt == MOE_INT4;
  if (alt_rows > 0 && (fp8 || w4)) return MOE_EUNSUPPORTED;  // bf16 / int8 panels only
  const int eb = (fp8 || i8) ? 1 : 2;
  const moe::GemmCfg cfg = ffn_cfg(G, R_max);
  const int bm = moe::gemm_block_m(cfg, fp8);
  const int bn = moe::gemm_block_n(cfg);
  const FfnSplit sp = ffn_split(s, G, R_max, I, alt_rows);
  float* part = at<float>(ws, L.part);
  float* part2 = at<float>(ws, L.part2);   // the extra group's partials
  const int32_t* n_rows = io.offsets ? io.offsets + G : nullptr;   // rows holding data
  Unit* units = at<Unit>(ws, L.units);
  int32_t* n_units = at<int32_t>(ws, L.n_units);
  // grouped rows, and the int8 kernels (which have no uniform-row form), run from a unit
  // table; a dense bf16 / fp8 FFN cuts its rows into uniform slices
  const bool planned = io.offsets || i8;
  int mu;
  if (planned) {
    mu = max_units(cfg, fp8, G, R_max, alt_rows);
    // XCD chunks balance 16-row tiles for the big tiles (their MFMAs set the time of a
    // well-filled unit) and unit counts for the short ones (their time is the weights)
    hipError_t e = moe::launch_plan(io.offsets, G, io.offsets ? 0 : R_max, alt_rows, bm,
                                    std::max(1, mu), cfg == moe::CFG_BIG ? bm / 2 : bm,
                                    units, n_units, st);
    if (e != hipSuccess) return MOE_EHIP;
  } else {
    mu = (R_max + bm - 1) / bm;
  }
  if (prof.mark(ev_plan, st) != hipSuccess) return MOE_EHIP;
  GemmArgs g1{};
  g1.A = static_cast<const uint8_t*>(io.a);
  g1.lda = static_cast<long long>(H) * eb;
  g1.a_scale = io.a_scale;
  g1.a_scale_ld = H / 128;
  g1.B = static_cast<const uint8_t*>(io.w13);
  g1.ldb = static_cast<long long>(H) * eb;
  g1.b_group = 2LL * I * H * eb;
  g1.b_scale = io.w13_scale;
  g1.b_scale_group = static_cast<long long>(2 * I / 128) * (H / 128);
  g1.b_scale_ld = H / 128;
  g1.C = at<uint8_t>(ws, L.h);
  g1.ldc = I;
  g1.c_scale = fp8 ? at<float>(ws, L.h_scale) : nullptr;
  g1.c_scale_ld = I / 128;
  g1.units = units;
  g1.n_units = n_units;
  g1.uniform_rows = planned ? 0 : R_max;
  g1.N = I;
  g1.K = H;
  g1.up_off = I;
  g1.n_tiles = I / 128;
  g1.splits = 1;
  g1.k_chunk = H;
  g1.gather = io.gather;
  g1.gather_div = io.gather_div;
  if (alt_rows > 0) {
    g1.alt_group = G;
    g1.A2 = static_cast<const uint8_t*>(alt->a);
    g1.lda2 = static_cast<long long>(H) * 2;
    g1.B2 = static_cast<const uint8_t*>(alt->w13);
    g1.C2 = at<uint8_t>(ws, L.h2);
    g1.ldc2 = I;
  }
  if (i8) {
    // W8A8: per-row activation scales, per-channel weight scales [G, 2I]; h comes out in
    // bf16 and is quantized per row (its amax spans all I columns, which no single
    // workgroup holds) before the down projection
    g1.a_scale_ld = 1;
    g1.b_scale_group = 2LL * I;
    g1.b_scale_ld = 1;
    g1.c_scale = nullptr;
    if (w4) {   // two codes per byte
      g1.ldb = H / 2;
      g1.b_group = static_cast<long long>(I) * H;
    }
    if (alt_rows > 0) {   // the int8 shared expert: its token codes and its own scales
      g1.lda2 = H;
      g1.a_scale2 = alt->a_scale;
      g1.b_scale2 = alt->w13_scale;
    }
  }
  hipError_t e;
  if (sp.s1 > 1) {
    // split-K: the stacked gate | up projection as a plain GEMM into fp32 partials, then
    // SwiGLU (and the fp8 quantization of h) over their slice-ordered sum
    GemmArgs p1 = g1;
    p1.N = 2 * I;
    p1.up_off = 0;
    p1.n_tiles = (2 * I + bn - 1) / bn;
    p1.splits = sp.s1;
    p1.k_chunk = sp.kc1;
    p1.C = part;
    p1.ldc = 2 * I;
    p1.c_split = static_cast<long long>(R_max) * 2 * I;
    p1.c_scale = nullptr;
    if (alt_rows > 0) {
      p1.C2 = part2;
      p1.ldc2 = 2 * I;
      p1.c_split2 = static_cast<long long>(alt_rows) * 2 * I;
    }
    e = i8 ? moe::launch_gemm_i8(cfg, moe::EPI_STORE_F32, w4, p1, mu, st)
           : moe::launch_gemm(cfg, moe::EPI_STORE_F32, fp8, p1, mu, st);
    if (e == hipSuccess)
      e = moe::launch_swiglu_reduce(part, sp.s1, p1.c_split, R_max, I, n_rows, at<uint8_t>(ws, L.h),
                                    fp8, fp8 ? at<float>(ws, L.h_scale) : nullptr, st);
    if (e == hipSuccess && alt_rows > 0)
      e = moe::launch_swiglu_reduce(part2, sp.s1, p1.c_split2, alt_rows, I, nullptr,
                                    at<uint8_t>(ws, L.h2), false, nullptr, st);
  } else {
    e = i8 ? moe::launch_gemm_i8(cfg, moe::EPI_SWIGLU_BF16, w4, g1, mu, st)
           : moe::launch_gemm(cfg, fp8 ? moe::EPI_SWIGLU_FP8 : moe::EPI_SWIGLU_BF16, fp8, g1, mu,
                              st);
  }
  // the ffn1 mark closes the first GEMM alone; h's int8 quantization (W8A8) is timed
  // with the down projection that consumes it
  if (e != hipSuccess || prof.mark(ev_ffn1, st) != hipSuccess) return MOE_EHIP;
  if (i8) {
    e = moe::launch_quant_rows_i8(at<uint8_t>(ws, L.h), R_max, I, 1, nullptr, n_rows,
                                  at<int8_t>(ws, L.hq), at<float>(ws, L.h_scale), st);
    if (e == hipSuccess && alt_rows > 0)
      e = moe::launch_quant_rows_i8(at<uint8_t>(ws, L.h2), alt_rows, I, 1, nullptr, nullptr,
                                    at<int8_t>(ws, L.h2q), at<float>(ws, L.h2_scale), st);
    if (e != hipSuccess) return MOE_EHIP;
  }
  GemmArgs g2 = g1;
  g2.gather = nullptr;
  g2.gather_div = 1;
  g2.A = at<uint8_t>(ws, L.h);
  g2.lda = static_cast<long long>(I) * eb;
  g2.a_scale = fp8 ? at<float>(ws, L.h_scale) : nullptr;
  g2.a_scale_ld = I / 128;
  g2.B = static_cast<const uint8_t*>(io.w2);
  g2.ldb = static_cast<long long>(I) * eb;
  g2.b_group = static_cast<long long>(H) * I * eb;
  g2.b_scale = io.w2_scale;
  g2.b_scale_group = static_cast<long long>(H / 128) * (I / 128);
  g2.b_scale_ld = I / 128;
  g2.C = io.y;
  g2.ldc = H;
  g2.c_scale = nullptr;
  g2.N = H;
  g2.K = I;
  g2.up_off = 0;
  g2.n_tiles = (H + moe::gemm_block_n(cfg) - 1) / moe::gemm_block_n(cfg);
  g2.k_chunk = I;
  if (alt_rows > 0) {
    g2.A2 = at<uint8_t>(ws, L.h2);
    g2.lda2 = static_cast<long long>(I) * 2;
    g2.B2 = static_cast<const uint8_t*>(alt->w2);
    g2.C2 = alt->y;
    g2.ldc2 = H;
  }
  if (i8) {
    g2.A = at<uint8_t>(ws, L.hq);
    g2.a_scale = at<float>(ws, L.h_scale);
    g2.a_scale_ld = 1;
    g2.b_scale_group = H;
    g2.b_scale_ld = 1;
    if (w4) {
      g2.ldb = I / 2;
      g2.b_group = static_cast<long long>(H) * I / 2;
    }
    if (alt_rows > 0) {
      g2.A2 = at<uint8_t>(ws, L.h2q);
      g2.lda2 = I;
      g2.a_scale2 = at<float>(ws, L.h2_scale);
      g2.b_scale2 = alt->w2_scale;
    }
  }
  if (sp.s2 > 1) {
    GemmArgs p2 = g2;
    p2.splits = sp.s2;
    p2.k_chunk = sp.kc2;
    p2.C = part;
    p2.ldc = H;
    p2.c_split = static_cast<long long>(R_max) * H;
    if (alt_rows > 0) {
      p2.C2 = part2;
      p2.ldc2 = H;
      p2.c_split2 = static_cast<long long>(alt_rows) * H;
    }
    e = i8 ? moe::launch_gemm_i8(cfg, moe::EPI_STORE_F32, w4, p2, mu, st)
           : moe::launch_gemm(cfg, moe::EPI_STORE_F32, fp8, p2, mu, st);
    if (e == hipSuccess) e = moe::launch_sum_reduce(part, sp.s2, p2.c_split, R_max, H, n_rows, io.y, st);
    if (e == hipSuccess && alt_rows > 0)
      e = moe::launch_sum_reduce(part2, sp.s2, p2.c_split2, alt_rows, H, nullptr, alt->y, st);
  } else {
    GemmArgs q2 = g2;
    q2.tiles_per_wg = planned ? down_tiles_per_wg(cfg, fp8, i8, est_units(G, R_max, alt_rows, bm), H, bn) : 1;
    e = i8 ? moe::launch_gemm_i8(cfg, moe::EPI_STORE_BF16, w4, q2, mu, st)
           : moe::launch_gemm(cfg, moe::EPI_STORE_BF16, fp8, q2, mu, st);
  }
  if (e != hipSuccess || prof.mark(ev_ffn2, st) != hipSuccess) return MOE_EHIP;
  return MOE_OK;
}

}  // namespace

extern "C" {

size_t moe_workspace_bytes(const moe_shape* s) {
  if (check_shape(s) != MOE_OK || check_inter(s, s->I) != MOE_OK) return 0;
  const moe_shape sh = shared_shape(s);
  if (check_inter(&sh, s->I_shared) != MOE_OK) return 0;
  return layer_layout(s).total;
}

moe_status moe_layer_plan_of(const moe_shape* s, moe_layer_plan* out) {
  if (!out) return MOE_EINVAL;
  moe_status st = check_shape(s);
  if (st != MOE_OK || (st = check_inter(s, s->I)) != MOE_OK) return st;
  const moe_shape sh = shared_shape(s);
  if ((st = check_inter(&sh, s->I_shared)) != MOE_OK) return st;
  const int R = s->T * s->k;
  const FfnSplit sp = ffn_split(s, s->E, R, s->I, merge_shared(s) ? s->T : 0);
  out->shared_merged = merge_shared(s) ? 1 : 0;
  out->rows_gathered = gather_rows(s) ? 1 : 0;
  out->ffn1_splits = sp.s1;
  out->ffn2_splits = sp.s2;
  const moe::GemmCfg cfg = ffn_cfg(s->E, R);
  const bool fp8 = s->wt == MOE_FP8_E4M3;
  out->block_m = s->act == MOE_F32 ? 0 : moe::gemm_block_m(cfg, fp8);
  out->ffn2_tiles_per_wg =
      (s->act == MOE_F32 || sp.s2 > 1)
          ? 1
          : down_tiles_per_wg(cfg, fp8, q8_weights(s), est_units(s->E, R, merge_shared(s) ? s->T : 0, out->block_m),
                              s->H, moe::gemm_block_n(cfg));
  return MOE_OK;
}

size_t moe_grouped_ffn_workspace_bytes(const moe_shape* s, int32_t G, int32_t R_max) {
  if (check_shape(s) != MOE_OK || check_inter(s, s->I) != MOE_OK || G < 1 || G > kMaxE || R_max < 0)
    return 0;
  return std::max<size_t>(ffn_layout(s, G, R_max, s->I).total, kAlign);
}

moe_status moe_gate_topk(const moe_shape* s, const void* x, const void* w_gate, const float* bias,
                         float* logits, int32_t* topk_idx, float* topk_w, void* ws,
                         size_t ws_bytes, hipStream_t stream) {
  return moe_gate_topk_ex(s, nullptr, x, w_gate, bias, logits, topk_idx, topk_w, ws, ws_bytes,
                          stream);
}

moe_status moe_gate_topk_ex(const moe_shape* s, const moe_router* router, const void* x,
                            const void* w_gate, const float* bias, float* logits,
                            int32_t* topk_idx, float* topk_w, void* ws, size_t ws_bytes,
                            hipStream_t stream) {
  moe_status st = check_shape(s);
  if (st != MOE_OK) return st;
  moe::RouterArgs ra;
  if (!router_args(s, router, &ra)) return MOE_EINVAL;
  if (s->T > 0 && (!x || !w_gate || !topk_idx || !topk_w)) return MOE_EINVAL;
  if (!ws) return MOE_EINVAL;
  if (!aligned16({x, w_gate, bias, logits, topk_idx, topk_w, ws})) return MOE_EINVAL;
  const size_t need = moe_workspace_bytes(s);
  if (need == 0) return MOE_EINVAL;
  if (ws_bytes < need) return MOE_EWORKSPACE;
  if (s->T == 0) return MOE_OK;
  const Layout L = layer_layout(s);
  // without a caller buffer the logits go to the workspace (as in moe_layer)
  return run_gate_topk(s, x, w_gate, bias, logits ? logits : at<float>(ws, L.logits), topk_idx, topk_w,
                       at<float>(ws, L.part), stream, Prof(), ra);
}

static moe_status init_routing_impl(const moe_shape* s, const void* x, const int32_t* ids,
                                    int32_t e_base, void* expanded_x, float* expanded_scale,
                                    int32_t* expanded_row_idx, int32_t* sorted_src,
                                    int32_t* tokens_per_expert, int32_t* expert_offsets, void* ws,
                                    size_t ws_bytes, hipStream_t stream, const Prof& prof,
                                    void* tok_q = nullptr, float* tok_s = nullptr);

moe_status moe_init_routing(const moe_shape* s, const void* x, const int32_t* ids, int32_t e_base,
                            void* expanded_x, float* expanded_scale, int32_t* expanded_row_idx,
                            int32_t* sorted_src, int32_t* tokens_per_expert,
                            int32_t* expert_offsets, void* ws, size_t ws_bytes,
                            hipStream_t stream) {
  return init_routing_impl(s, x, ids, e_base, expanded_x, expanded_scale, expanded_row_idx,
                           sorted_src, tokens_per_expert, expert_offsets, ws, ws_bytes, stream,
                           Prof());
}

static moe_status init_routing_impl(const moe_shape* s, const void* x, const int32_t* ids,
                                    int32_t e_base, void* expanded_x, float* expanded_scale,
                                    int32_t* expanded_row_idx, int32_t* sorted_src,
                                    int32_t* tokens_per_expert, int32_t* expert_offsets, void* ws,
                                    size_t ws_bytes, hipStream_t stream, const Prof& prof,
                                    void* tok_q, float* tok_s) {
  moe_status st = check_shape(s);
  if (st != MOE_OK) return st;
  const bool fp8 = s->wt == MOE_FP8_E4M3;
  const bool i8 = q8_weights(s);
  if (!tokens_per_expert || !expert_offsets || !ws) return MOE_EINVAL;
  if (s->T > 0 && (!ids || !expanded_row_idx)) return MOE_EINVAL;
  if (expanded_x && s->T > 0 && !x) return MOE_EINVAL;
  if (expanded_x && (fp8 || i8) && !expanded_scale) return MOE_EINVAL;
  if (!aligned16({x, ids, expanded_x, expanded_scale, expanded_row_idx, sorted_src, tokens_per_expert,
                  expert_offsets, ws, tok_q, tok_s}))
    return MOE_EINVAL;
  const size_t need = moe_workspace_bytes(s);
  if (need == 0) return MOE_EINVAL;
  if (ws_bytes < need) return MOE_EWORKSPACE;
  const Layout L = layer_layout(s);
  const long long R = static_cast<long long>(s->T) * s->k;
  hipError_t e = moe::launch_routing(ids, R, e_base, s->E, at<int32_t>(ws, L.counts),
                                     at<int32_t>(ws, L.seg_err), at<int32_t>(ws, L.err),
                                     expanded_row_idx, sorted_src, tokens_per_expert,
                                     expert_offsets, stream);
  if (e != hipSuccess || prof.mark(MOE_EV_ROUTE, stream) != hipSuccess) return MOE_EHIP;
  if (expanded_x && s->T > 0) {
    // int8 (W8A8): each token quantized once per row, its codes copied to its k rows
    e = i8 ? moe::launch_quant_rows_i8(x, s->T, s->H, s->k, expanded_row_idx, nullptr,
                                       static_cast<int8_t*>(expanded_x), expanded_scale, stream)
           : moe::launch_expand(x, s->T, s->H, s->k, elem_bytes(s->act), fp8, expanded_row_idx,
                                expanded_x, expanded_scale, stream);
    if (e != hipSuccess) return MOE_EHIP;
  }
  if (tok_q && s->T > 0) {
    // the per-token codes in token order (the layer's gathered first GEMM and its W8A8
    // shared expert read them): one quantization per token
    e = i8 ? moe::launch_quant_rows_i8(x, s->T, s->H, 1, nullptr, nullptr, static_cast<int8_t*>(tok_q),
                                       tok_s, stream)
           : moe::launch_expand(x, s->T, s->H, 1, 2, true, nullptr, tok_q, tok_s, stream);
    if (e != hipSuccess) return MOE_EHIP;
  }
  if (prof.mark(MOE_EV_EXPAND, stream) != hipSuccess) return MOE_EHIP;
  return MOE_OK;
}

moe_status moe_grouped_ffn(const moe_shape* s, int32_t G, int32_t R_max, const void* a,
                           const float* a_scale, const int32_t* group_offsets, const void* w13,
                           const float* w13_scale, const void* w2, const float* w2_scale, void* y,
                           void* ws, size_t ws_bytes, hipStream_t stream) {
  moe_status st = check_shape(s);
  if (st != MOE_OK) return st;
  if ((st = check_inter(s, s->I)) != MOE_OK) return st;
  if (G < 1 || R_max < 0) return MOE_EINVAL;
  if (G > kMaxE) return MOE_EUNSUPPORTED;
  const bool scaled = s->wt == MOE_FP8_E4M3 || q8_weights(s);
  if (!group_offsets || !ws) return MOE_EINVAL;
  if (R_max > 0 && (!a || !w13 || !w2 || !y)) return MOE_EINVAL;
  if (scaled && R_max > 0 && (!a_scale || !w13_scale || !w2_scale)) return MOE_EINVAL;
  if (!aligned16({a, a_scale, group_offsets, w13, w13_scale, w2, w2_scale, y, ws})) return MOE_EINVAL;
  if (ws_bytes < moe_grouped_ffn_workspace_bytes(s, G, R_max)) return MOE_EWORKSPACE;
  FfnIo io{a, a_scale, group_offsets, w13, w13_scale, w2, w2_scale, y};
  return run_ffn(s, G, R_max, s->I, io, ws, stream);
}

moe_status moe_grouped_ffn_gathered(const moe_shape* s, int32_t G, int32_t R_max, const void* a,
                                    int32_t a_rows, const float* a_scale, const int32_t* row_of,
                                    int32_t row_div, const int32_t* group_offsets,
                                    const void* w13, const float* w13_scale, const void* w2,
                                    const float* w2_scale, void* y, void* ws, size_t ws_bytes,
                                    hipStream_t stream) {
  moe_status st = check_shape(s);
  if (st != MOE_OK) return st;
  if ((st = check_inter(s, s->I)) != MOE_OK) return st;
  if (G < 1 || R_max < 0 || a_rows < 0 || row_div < 1) return MOE_EINVAL;
  if (G > kMaxE) return MOE_EUNSUPPORTED;
  if (s->act == MOE_F32) return MOE_EUNSUPPORTED;   // the fp32 kernels read rows in order
  const bool fp8 = s->wt == MOE_FP8_E4M3, scaled = fp8 || q8_weights(s);
  if (!moe::lane_offsets_fit_u32((fp8 || q8_weights(s)) ? 1 : 2, a_rows, s->H)) return MOE_EUNSUPPORTED;
  if (!group_offsets || !ws) return MOE_EINVAL;
  if (R_max > 0 && (!a || !row_of || !w13 || !w2 || !y)) return MOE_EINVAL;
  if (scaled && R_max > 0 && (!a_scale || !w13_scale || !w2_scale)) return MOE_EINVAL;
  if (!aligned16({a, a_scale, row_of, group_offsets, w13, w13_scale, w2, w2_scale, y, ws}))
    return MOE_EINVAL;
  if (ws_bytes < moe_grouped_ffn_workspace_bytes(s, G, R_max)) return MOE_EWORKSPACE;
  FfnIo io{a, a_scale, group_offsets, w13, w13_scale, w2, w2_scale, y};
  io.gather = row_of;
  io.gather_div = row_div;
  return run_ffn(s, G, R_max, s->I, io, ws, stream);
}

moe_status moe_finalize_routing(const moe_shape* s, const void* y, const void* skip,
                                const float* topk_w, const int32_t* expanded_row_idx, void* out,
                                hipStream_t stream) {
  moe_status st = check_shape(s);
  if (st != MOE_OK) return st;
  if (s->T == 0) return MOE_OK;
  if (!y || !expanded_row_idx || !out) return MOE_EINVAL;
  if (!aligned16({y, skip, topk_w, expanded_row_idx, out})) return MOE_EINVAL;
  return hip_status(moe::launch_finalize(y, skip, topk_w, expanded_row_idx, out, s->T, s->H, s->k,
                                         elem_bytes(s->act), stream));
}

static moe_status layer_impl(const moe_shape* s, const moe_weights* w, const void* x, void* out,
                             int32_t* topk_idx, float* topk_w, float* logits, void* ws,
                             size_t ws_bytes, hipStream_t stream, const Prof& prof,
                             hipStream_t side = nullptr, const moe_router* router = nullptr);

moe_status moe_layer(const moe_shape* s, const moe_weights* w, const void* x, void* out,
                     int32_t* topk_idx, float* topk_w, float* logits, void* ws, size_t ws_bytes,
                     hipStream_t stream) {
  return layer_impl(s, w, x, out, topk_idx, topk_w, logits, ws, ws_bytes, stream, Prof());
}

moe_status moe_layer_ex(const moe_shape* s, const moe_router* router, const moe_weights* w,
                        const void* x, void* out, int32_t* topk_idx, float* topk_w,
                        float* logits, void* ws, size_t ws_bytes, hipStream_t stream,
                        hipStream_t side) {
  return layer_impl(s, w, x, out, topk_idx, topk_w, logits, ws, ws_bytes, stream, Prof(),
                    side == stream ? nullptr : side, router);
}

moe_status moe_layer_overlap(const moe_shape* s, const moe_weights* w, const void* x, void* out,
                             int32_t* topk_idx, float* topk_w, float* logits, void* ws,
                             size_t ws_bytes, hipStream_t stream, hipStream_t side) {
  return layer_impl(s, w, x, out, topk_idx, topk_w, logits, ws, ws_bytes, stream, Prof(),
                    side == stream ? nullptr : side);
}

moe_status moe_layer_profiled(const moe_shape* s, const moe_weights* w, const void* x, void* out,
                              int32_t* topk_idx, float* topk_w, float* logits, void* ws,
                              size_t ws_bytes, hipStream_t stream, hipStream_t side,
                              hipEvent_t* events, int32_t n_events) {
  Prof p;
  p.ev = events;
  p.n = events ? n_events : 0;
  return layer_impl(s, w, x, out, topk_idx, topk_w, logits, ws, ws_bytes, stream, p,
                    side == stream ? nullptr : side);
}

// Fork/join of the shared expert onto a second stream: two events, created for this call
// and released once enqueued (a recorded event that streams still wait on is freed by the
// runtime when it completes).  Once `side` waits on the fork, the join is owed: a return
// that leaves before the layer's own join (an error in any later launch) still records the
// join on `side` and makes `stream` wait for it, so the side work never outlives the call's
// ordering on `stream` (and a capture in progress keeps both streams joined).
struct SideFork {
  hipEvent_t fork = nullptr, join = nullptr;
  hipStream_t stream = nullptr, side = nullptr;
  bool owed = false;
  hipError_t rejoin() {
    owed = false;
    hipError_t e = hipEventRecord(join, side);
    if (e == hipSuccess) e = hipStreamWaitEvent(stream, join, 0);
    return e;
  }
  ~SideFork() {
    if (owed) (void)rejoin();
    if (fork) (void)hipEventDestroy(fork);
    if (join) (void)hipEventDestroy(join);
  }
};

static moe_status layer_impl(const moe_shape* s, const moe_weights* w, const void* x, void* out,
                             int32_t* topk_idx, float* topk_w, float* logits, void* ws,
                             size_t ws_bytes, hipStream_t stream, const Prof& prof,
                             hipStream_t side, const moe_router* router) {
  moe_status st = check_shape(s);
  if (st != MOE_OK) return st;
  moe::RouterArgs ra;
  if (!router_args(s, router, &ra)) return MOE_EINVAL;
  if ((st = check_inter(s, s->I)) != MOE_OK) return st;
  if (!w || !ws) return MOE_EINVAL;
  const bool fp8 = s->wt == MOE_FP8_E4M3;
  if (s->T > 0 && (!x || !out || !w->w_gate || !w->w13 || !w->w2 || !w->sh_w13 || !w->sh_w2))
    return MOE_EINVAL;
  const bool q8 = q8_weights(s);
  if ((fp8 || q8) && (!w->w13_scale || !w->w2_scale)) return MOE_EINVAL;
  if (q8 && s->T > 0 && (!w->sh_w13_scale || !w->sh_w2_scale)) return MOE_EINVAL;
  if (!aligned16({x, out, topk_idx, topk_w, logits, ws, w->w_gate, w->w13, w->w2, w->sh_w13, w->sh_w2,
                  w->w13_scale, w->w2_scale, w->bias, w->sh_w13_scale, w->sh_w2_scale}))
    return MOE_EINVAL;
  const size_t need = moe_workspace_bytes(s);
  if (need == 0) return MOE_EINVAL;
  if (ws_bytes < need) return MOE_EWORKSPACE;
  if (s->T == 0) return MOE_OK;
  const Layout L = layer_layout(s);
  float* lg = logits ? logits : at<float>(ws, L.logits);
  int32_t* idx = topk_idx ? topk_idx : at<int32_t>(ws, L.idx);
  float* tw = topk_w ? topk_w : at<float>(ws, L.w);
  if (prof.mark(MOE_EV_START, stream) != hipSuccess) return MOE_EHIP;
  // The shared expert depends on x alone, not on the gate, the routing or the routed
  // experts ([V32 §multi-stream parallel optimization]; [MND §Computation and
  // communication overlap], Dispatch Overlap).  When it runs in launches of its own and
  // the caller gives a second stream, it starts there at once and overlaps the routing
  // kernels, which leave most of the machine idle; finalize waits for it.
  // Token-order activations of the first expert GEMM and of the W8A8 shared expert: x
  // for bf16 experts; for quantized experts the per-token codes, written once in the
  // expansion's place (gathered rows) or beside the expanded rows.  A shared expert on
  // the second stream quantizes its own copy there.
  const bool merged = merge_shared(s);
  const bool gathered = gather_rows(s);
  const bool quant_act = fp8 || q8;
  const bool forked = side && !merged;
  void* tok_q = nullptr;        // per-token codes written by the routing's expansion stage
  float* tok_s = nullptr;
  if (quant_act && gathered) {
    tok_q = at<void>(ws, L.ex);
    tok_s = at<float>(ws, L.ex_scale);
  } else if (q8 && !forked) {
    tok_q = at<void>(ws, L.sh_xq);
    tok_s = at<float>(ws, L.sh_xs);
  }
  FfnIo sio{x, nullptr, nullptr, w->sh_w13, nullptr, w->sh_w2, nullptr, at<void>(ws, L.sh_out)};
  if (q8) {
    sio.a = forked ? at<void>(ws, L.sh_xq) : tok_q;
    sio.a_scale = forked ? at<float>(ws, L.sh_xs) : tok_s;
    sio.w13_scale = w->sh_w13_scale;
    sio.w2_scale = w->sh_w2_scale;
  }
  const moe_shape sh = shared_shape(s);
  SideFork sf;
  if (forked) {
    sf.stream = stream;
    sf.side = side;
    if (hipEventCreateWithFlags(&sf.fork, hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&sf.join, hipEventDisableTiming) != hipSuccess ||
        hipEventRecord(sf.fork, stream) != hipSuccess ||
        hipStreamWaitEvent(side, sf.fork, 0) != hipSuccess)
      return MOE_EHIP;
    sf.owed = true;
    if (q8 && moe::launch_quant_rows_i8(x, s->T, s->H, 1, nullptr, nullptr, at<int8_t>(ws, L.sh_xq),
                                        at<float>(ws, L.sh_xs), side) != hipSuccess)
      return MOE_EHIP;
    st = run_ffn(&sh, 1, s->T, s->I_shared, sio, at<void>(ws, L.sh_ffn), side);
    if (st != MOE_OK) return st;
  }
  // gate + router  ([MND §Expert Parallelism], [MND §MoE Router])
  st = run_gate_topk(s, x, w->w_gate, w->bias, lg, idx, tw, at<float>(ws, L.part), stream, prof, ra);
  if (st != MOE_OK) return st;
  // first routing: sort by expert  ([R1P §MoE deployment strategy optimization]); the
  // expanded rows are written only where the first expert GEMM cannot gather them
  int32_t* eri = at<int32_t>(ws, L.eri);
  int32_t* offs = at<int32_t>(ws, L.offsets);
  int32_t* ssrc = at<int32_t>(ws, L.sorted_src);
  st = init_routing_impl(s, x, idx, 0, gathered ? nullptr : at<void>(ws, L.ex),
                         (!gathered && quant_act) ? at<float>(ws, L.ex_scale) : nullptr, eri, ssrc,
                         at<int32_t>(ws, L.tpe), offs, ws, ws_bytes, stream, prof, tok_q, tok_s);
  if (st != MOE_OK) return st;
  // routed experts as one grouped GEMM over the expert-sorted rows
  // The shared expert runs on every token ([MND §Expert Parallelism]: its output is
  // added); with the routed experts' shape it is one more group of the same launches.
  const int R = s->T * s->k;
  FfnIo io{at<void>(ws, L.ex), quant_act ? at<float>(ws, L.ex_scale) : nullptr, offs, w->w13,
           w->w13_scale, w->w2, w->w2_scale, at<void>(ws, L.y)};
  if (gathered) {
    io.a = quant_act ? tok_q : x;
    io.a_scale = quant_act ? tok_s : nullptr;
    io.gather = ssrc;
    io.gather_div = s->k;
  }
  st = run_ffn(s, s->E, R, s->I, io, at<void>(ws, L.ffn), stream, prof, MOE_EV_PLAN, MOE_EV_FFN1,
               MOE_EV_FFN2, merged ? &sio : nullptr, merged ? s->T : 0);
  if (st != MOE_OK) return st;
  if (forked) {
    if (sf.rejoin() != hipSuccess) return MOE_EHIP;
  } else if (!merged) {
    st = run_ffn(&sh, 1, s->T, s->I_shared, sio, at<void>(ws, L.sh_ffn), stream);
    if (st != MOE_OK) return st;
  }
  if (prof.mark(MOE_EV_SHARED, stream) != hipSuccess) return MOE_EHIP;
  // finalize: un-permute, weighted sum, plus the shared expert
  st = moe_finalize_routing(s, at<void>(ws, L.y), at<void>(ws, L.sh_out), tw, eri, out, stream);
  if (st != MOE_OK) return st;
  return prof.mark(MOE_EV_FINALIZE, stream) == hipSuccess ? MOE_OK : MOE_EHIP;
}

}  // extern "C"

// ------------------------------------------------------------------ static scratch
// moe_layer_static's workspace: one array per GPU, in device memory the code object
// reserves when it loads on that GPU, held until the process ends.  In host code the
// array's name is only a host-side stand-in: its device address on the current GPU comes
// from hipGetSymbolAddress, taken once per device and kept in g_scratch_ptr; only that
// address is ever handed to kernels.
static __device__ __align__(256) uint8_t scratch[MOE_STATIC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of the current GPU's scratch array (set up on its first use there).
moe_status static_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return MOE_EHIP;
  if (dev >= kMaxDevices) return MOE_EUNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOE_EHIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}
}  // namespace

extern "C" {

moe_status moe_layer_static(const moe_shape* s, const moe_weights* w, const void* x, void* out,
                            int32_t* topk_idx, float* topk_w, float* logits, hipStream_t stream) {
  moe_status st = check_shape(s);
  if (st != MOE_OK || (st = check_inter(s, s->I)) != MOE_OK) return st;
  const moe_shape sh = shared_shape(s);
  if ((st = check_inter(&sh, s->I_shared)) != MOE_OK) return st;
  // the shape's workspace must fit the fixed array: checked before any device call
  if (moe_workspace_bytes(s) > MOE_STATIC_SCRATCH_BYTES) return MOE_EWORKSPACE;
  void* ws = nullptr;
  if ((st = static_scratch(&ws)) != MOE_OK) return st;
  return layer_impl(s, w, x, out, topk_idx, topk_w, logits, ws, MOE_STATIC_SCRATCH_BYTES, stream, Prof());
}

moe_status moe_get_error(void* ws, hipStream_t stream) {
  if (!ws) return MOE_EINVAL;
  if (hipStreamSynchronize(stream) != hipSuccess) return MOE_EHIP;
  int32_t v = 0;
  if (hipMemcpy(&v, ws, sizeof(v), hipMemcpyDeviceToHost) != hipSuccess) return MOE_EHIP;
  if (hipMemset(ws, 0, sizeof(v)) != hipSuccess) return MOE_EHIP;
  return v ? MOE_EDEVICE : MOE_OK;
}

const char* moe_status_str(moe_status st) {
  switch (st) {
    case MOE_OK: return "ok";
    case MOE_EINVAL: return "invalid argument";
    case MOE_EUNSUPPORTED: return "unsupported shape or dtype";
    case MOE_EWORKSPACE: return "workspace too small";
    case MOE_EHIP: return "HIP runtime error";
    case MOE_EDEVICE: return "device-detected bad input (expert id out of range)";
  }
  return "unknown status";
}

}  // extern "C"
