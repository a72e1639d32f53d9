// Top-k router and expand-and-sort routing for the MoE layer (gfx950).
//
// [MND] = page "Lower latency and higher throughput with multi-node DeepSeek
//         deployment"; [R1P] = page "CANN/cann-recipes-infer: DeepSeek-R1
//         prefill optimization".
//
// Routing is a stable counting sort in three launches, deterministic without
// order-dependent atomics:
//   route_count   one wavefront per segment of kSegSlots consecutive slots counts
//                 the slots of each expert with ballot-built peer masks
//   route_scan    per-expert exclusive prefix over segments, then over experts
//   route_place   each wavefront replays its segment in slot order and places every
//                 slot at offsets[e] + (earlier slots of e), writing the src->dst
//                 map (expanded_row_idx) and its inverse (sorted_src)
// or, for up to 16 segments (decode batches), in one launch doing the same three passes
// in one block (route_small),
// and the copy kernel `expand_rows` reads each token row once and writes its k
// copies (optionally quantized to fp8 with one scale per 1x128 vector).

#include "common.h"
#include "kernels.h"

namespace moe {

constexpr size_t kSmallRouteLds = 60 * 1024;  // LDS bound of the single-launch routing

// ------------------------------------------------------------------ top-k router
// [MND §Expert Parallelism]: every token goes to k different routed experts whose
// outputs are weighted-summed.  [MND §MoE Router]: a sort that tracks element
// indices selects the top-k.  One wavefront per token; each lane holds
// ceil(E/64) scores; k rounds of a wave-wide (score desc, id asc) arg-max.
// The gate GEMM may have split the reduction into `splits` partial sums, added
// here in split order so the float32 logits are reproducible run to run.
// Router variants ([MND §MoE Router]: the ungrouped routing is the grouped one with
// every expert in the top-K group): group-limited candidates, softmax weights, no
// renormalization, a scaling factor.
template <int VPL>
__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ part, int splits,
                                                   long long split_stride, int T, int E, int k,
                                                   const float* __restrict__ bias,
                                                   float* __restrict__ logits_out,
                                                   int32_t* __restrict__ idx_out,
                                                   float* __restrict__ w_out, RouterArgs r) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * (blockDim.x / 64) + (threadIdx.x >> 6);
  if (t >= T) return;
  // Partial logits: every lane's VPL experts advance through the splits together, with
  // kBatch splits of each in flight at once (about 32 loads per lane), and each expert's
  // partials are added strictly in split order, so the sum does not depend on the batching.
  constexpr int kBatch = VPL >= 16 ? 2 : VPL >= 8 ? 4 : 8;
  const float* p = part + static_cast<long long>(t) * E + lane;
  float z[VPL];
#pragma unroll
  for (int v = 0; v < VPL; ++v) z[v] = v * 64 + lane < E ? p[v * 64] : -INFINITY;
  for (int s0 = 1; s0 < splits; s0 += kBatch) {
    float q[VPL][kBatch];
#pragma unroll
    for (int v = 0; v < VPL; ++v)
#pragma unroll
      for (int i = 0; i < kBatch; ++i)
        q[v][i] = (v * 64 + lane < E && s0 + i < splits)
                      ? p[(s0 + i) * split_stride + v * 64] : 0.f;
#pragma unroll
    for (int v = 0; v < VPL; ++v)
#pragma unroll
      for (int i = 0; i < kBatch; ++i)
        if (s0 + i < splits) z[v] += q[v][i];
  }
#pragma unroll
  for (int v = 0; v < VPL; ++v) {
    const int e = v * 64 + lane;
    if (e < E) {
      if (logits_out) logits_out[static_cast<long long>(t) * E + e] = z[v];
      if (bias) z[v] += bias[e];
    }
  }
  // softmax statistics over all E experts, before any candidate is masked
  float zmax = 0.f, zsum = 1.f;
  if (r.scoring == 1) {
    float m = -INFINITY;
#pragma unroll
    for (int v = 0; v < VPL; ++v)
      if (v * 64 + lane < E) m = fmaxf(m, z[v]);
    zmax = wave_max(m);
    float sum = 0.f;
#pragma unroll
    for (int v = 0; v < VPL; ++v)
      if (v * 64 + lane < E) sum += expf(z[v] - zmax);
    zsum = wave_sum(sum);
  }
  // group-limited candidates: lane g holds group g's score (its best z, plus its second
  // best when group_topn == 2, added in fp32); the topk_group best groups are kept
  // (equal scores: lower group id) and the other groups' experts leave the selection
  if (r.topk_group < r.n_group) {
    const int gsz = E / r.n_group;
    float gscore = -INFINITY;
    for (int g = 0; g < r.n_group; ++g) {
      float b1 = -INFINITY;
      int e1 = 0x7fffffff;
#pragma unroll
      for (int v = 0; v < VPL; ++v) {
        const int e = v * 64 + lane;
        if (e < E && e / gsz == g && (z[v] > b1 || (z[v] == b1 && e < e1))) {
          b1 = z[v];
          e1 = e;
        }
      }
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) {
        const float ob = __shfl_xor(b1, o, 64);
        const int oe = __shfl_xor(e1, o, 64);
        if (ob > b1 || (ob == b1 && oe < e1)) {
          b1 = ob;
          e1 = oe;
        }
      }
      float sc = b1;
      if (r.group_topn == 2) {
        float b2 = -INFINITY;
#pragma unroll
        for (int v = 0; v < VPL; ++v) {
          const int e = v * 64 + lane;
          if (e < E && e / gsz == g && e != e1) b2 = fmaxf(b2, z[v]);
        }
        sc = b1 + wave_max(b2);
      }
      if (lane == g) gscore = sc;
    }
    uint64_t kept = 0;
    for (int j = 0; j < r.topk_group; ++j) {
      const bool open = lane < r.n_group && !((kept >> lane) & 1ull);
      float bz = open ? gscore : -INFINITY;
      int bg = open ? lane : 0x7fffffff;
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) {
        const float oz = __shfl_xor(bz, o, 64);
        const int og = __shfl_xor(bg, o, 64);
        if (oz > bz || (oz == bz && og < bg)) {
          bz = oz;
          bg = og;
        }
      }
      kept |= 1ull << bg;
    }
#pragma unroll
    for (int v = 0; v < VPL; ++v) {
      const int e = v * 64 + lane;
      if (e < E && !((kept >> (e / gsz)) & 1ull)) z[v] = -INFINITY;
    }
  }
  float sel_z = 0.f;  // score of the expert this lane records (lanes 0..k-1)
  int sel_e = 0;
  for (int j = 0; j < k; ++j) {
    // local best (lower id wins ties because v ascends)
    float bz = -INFINITY;
    int be = 0x7fffffff;
#pragma unroll
    for (int v = 0; v < VPL; ++v) {
      const int e = v * 64 + lane;
      if (e < E && (z[v] > bz || (z[v] == bz && e < be))) {
        bz = z[v];
        be = e;
      }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float oz = __shfl_xor(bz, o, 64);
      const int oe = __shfl_xor(be, o, 64);
      if (oz > bz || (oz == bz && oe < be)) {
        bz = oz;
        be = oe;
      }
    }
    if (lane == j) {
      sel_z = bz;
      sel_e = be;
    }
#pragma unroll
    for (int v = 0; v < VPL; ++v)
      if (v * 64 + lane == be) z[v] = -INFINITY;  // remove the winner
  }
  // sigmoid of the selected scores, or their softmax over all experts; renormalized
  // over the k selected (the workload's router) or not; times the scaling factor
  float sg = 0.f;
  if (lane < k) sg = r.scoring == 1 ? expf(sel_z - zmax) / zsum : 1.0f / (1.0f + expf(-sel_z));
  const float tot = r.renormalize ? wave_sum(sg) : 1.0f;
  if (lane < k) {
    idx_out[static_cast<long long>(t) * k + lane] = sel_e;
    w_out[static_cast<long long>(t) * k + lane] = sg / tot * r.scale;
  }
}

hipError_t launch_topk(const float* part, int splits, long long split_stride, int T, int E, int k,
                       const float* bias, float* logits_out, int32_t* idx, float* w,
                       hipStream_t st, const RouterArgs& router) {
  if (router.n_group < 1 || router.n_group > 64 || E % router.n_group ||
      router.topk_group < 1 || router.topk_group > router.n_group)
    return hipErrorInvalidValue;
  if (T == 0) return hipSuccess;
  const dim3 block(256), grid((T + 3) / 4);
  const int vpl = (E + 63) / 64;
#define MOE_TOPK_CASE(N)                                                                   \
  case N:                                                                                  \
    topk_kernel<N><<<grid, block, 0, st>>>(part, splits, split_stride, T, E, k, bias,      \
                                           logits_out, idx, w, router);                            \
    break;
  switch (vpl) {
    MOE_TOPK_CASE(1)
    MOE_TOPK_CASE(2)
    MOE_TOPK_CASE(3)
    MOE_TOPK_CASE(4)
    MOE_TOPK_CASE(8)
    MOE_TOPK_CASE(16)
    default:
      if (vpl <= 8) {
        topk_kernel<8><<<grid, block, 0, st>>>(part, splits, split_stride, T, E, k, bias,
                                               logits_out, idx, w, router);
      } else {
        topk_kernel<16><<<grid, block, 0, st>>>(part, splits, split_stride, T, E, k, bias,
                                                logits_out, idx, w, router);
      }
  }
#undef MOE_TOPK_CASE
  return hipGetLastError();
}

// ------------------------------------------------------------------ counting sort
// Peer mask of a lane: the lanes of the wave (among `active`) holding the same key.
// Built from one ballot per key bit, so equal keys are found without atomics.
__device__ __forceinline__ uint64_t peer_mask(uint32_t key, int bits, uint64_t active) {
  uint64_t m = active;
  for (int b = 0; b < bits; ++b) {
    const bool bit = (key >> b) & 1u;
    const uint64_t bal = __ballot(bit);
    m &= bit ? bal : ~bal;
  }
  return m;
}

__device__ __forceinline__ uint32_t local_key(const int32_t* ids, long long s, long long R,
                                              int e_base, int E, int* err) {
  if (s >= R) return static_cast<uint32_t>(E);
  const int v = ids[s] - e_base;
  if (v < 0 || v >= E) {
    *err = 1;
    return static_cast<uint32_t>(E);  // sentinel: invalid slot
  }
  return static_cast<uint32_t>(v);
}

// counts[seg * E + e] = slots of expert e in segment seg.
__global__ __launch_bounds__(256) void route_count_kernel(const int32_t* __restrict__ ids,
                                                          long long R, int e_base, int E, int bits,
                                                          int32_t* __restrict__ counts,
                                                          int nseg, int32_t* __restrict__ seg_err) {
  extern __shared__ int32_t cnt_lds[];  // [4][E]
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int seg = blockIdx.x * 4 + wave;
  int32_t* cnt = cnt_lds + wave * E;
  for (int e = lane; e < E; e += 64) cnt[e] = 0;
  if (seg >= nseg) return;
  int err = 0;
  const long long s0 = static_cast<long long>(seg) * kSegSlots;
  // every key of the segment is loaded before the first ballot (all loads in flight)
  uint32_t keys[kSegSlots / 64];
#pragma unroll
  for (int it = 0; it < kSegSlots / 64; ++it) keys[it] = local_key(ids, s0 + it * 64 + lane, R, e_base, E, &err);
#pragma unroll
  for (int it = 0; it < kSegSlots / 64; ++it) {
    const long long s = s0 + it * 64 + lane;
    const uint32_t key = keys[it];
    const uint64_t active = __ballot(s < R);
    if (active == 0) break;
    const uint64_t peers = peer_mask(key, bits, active);
    const bool leader = (s < R) && key < static_cast<uint32_t>(E) &&
                        (__builtin_ctzll(peers) == lane);
    if (leader) cnt[key] += __builtin_popcountll(peers);
  }
  for (int e = lane; e < E; e += 64) counts[static_cast<long long>(seg) * E + e] = cnt[e];
  const bool any_err = __ballot(err) != 0;
  if (lane == 0) seg_err[seg] = any_err ? 1 : 0;
}

// Exclusive prefix of one value per thread over a block of 1024 threads (16 waves),
// in thread order; wsum: 16 ints of LDS.
__device__ __forceinline__ int32_t block_excl_scan1024(int32_t run, int32_t* wsum) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int32_t incl = run;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int32_t v = __shfl_up(incl, o, 64);
    if (lane >= o) incl += v;
  }
  if (lane == 63) wsum[w] = incl;
  __syncthreads();
  if (w == 0) {
    int32_t v = lane < 16 ? wsum[lane] : 0;
    int32_t inc = v;
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) {
      const int32_t u = __shfl_up(inc, o, 64);
      if (lane >= o) inc += u;
    }
    if (lane < 16) wsum[lane] = inc - v;  // exclusive wave base
  }
  __syncthreads();
  return wsum[w] + incl - run;
}

// One block: base[seg*E+e] = offsets[e] + sum_{seg'<seg} counts[seg'*E+e] (in place),
// tokens_per_expert[e] and expert_offsets[0..E].
__global__ __launch_bounds__(1024) void route_scan_kernel(int32_t* __restrict__ counts, int nseg,
                                                          int E, int32_t* __restrict__ tpe,
                                                          int32_t* __restrict__ offsets,
                                                          const int32_t* __restrict__ seg_err,
                                                          int32_t* __restrict__ err_word) {
  __shared__ int32_t wsum[16];
  __shared__ int32_t any_err;
  const int e = threadIdx.x;
  if (e == 0) any_err = 0;
  __syncthreads();
  for (int s = e; s < nseg; s += blockDim.x)
    if (seg_err[s]) any_err = 1;  // benign race: every writer stores 1
  int32_t run = 0;
  if (e < E) {
    // segment counts 16 at a time (loads in flight together), prefix in segment order
    for (int s0 = 0; s0 < nseg; s0 += 16) {
      int32_t c[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) c[i] = s0 + i < nseg ? counts[static_cast<long long>(s0 + i) * E + e] : 0;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if (s0 + i < nseg) counts[static_cast<long long>(s0 + i) * E + e] = run;
        run += c[i];
      }
    }
  }
  const int32_t excl = block_excl_scan1024(run, wsum);
  if (e == 0) *err_word = any_err;
  if (e < E) {
    tpe[e] = run;
    offsets[e] = excl;
    if (e == E - 1) offsets[E] = excl + run;
  }
  __syncthreads();
  if (e < E) {
    for (int s0 = 0; s0 < nseg; s0 += 16) {
      int32_t c[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) c[i] = s0 + i < nseg ? counts[static_cast<long long>(s0 + i) * E + e] : 0;
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (s0 + i < nseg) counts[static_cast<long long>(s0 + i) * E + e] = c[i] + excl;
    }
  }
}

__global__ __launch_bounds__(256) void route_place_kernel(const int32_t* __restrict__ ids,
                                                          long long R, int e_base, int E, int bits,
                                                          const int32_t* __restrict__ base,
                                                          int nseg, int32_t* __restrict__ eri,
                                                          int32_t* __restrict__ sorted_src) {
  extern __shared__ int32_t cnt_lds[];  // [4][E]
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int seg = blockIdx.x * 4 + wave;
  if (seg >= nseg) return;
  int32_t* cnt = cnt_lds + wave * E;
  for (int e = lane; e < E; e += 64) cnt[e] = base[static_cast<long long>(seg) * E + e];
  int err = 0;
  const long long s0 = static_cast<long long>(seg) * kSegSlots;
  uint32_t keys[kSegSlots / 64];
#pragma unroll
  for (int it = 0; it < kSegSlots / 64; ++it) keys[it] = local_key(ids, s0 + it * 64 + lane, R, e_base, E, &err);
#pragma unroll
  for (int it = 0; it < kSegSlots / 64; ++it) {
    const long long s = s0 + it * 64 + lane;
    const uint64_t active = __ballot(s < R);
    if (active == 0) break;
    const uint32_t key = keys[it];
    const uint64_t peers = peer_mask(key, bits, active);
    const bool valid = (s < R) && key < static_cast<uint32_t>(E);
    int32_t pos = -1;
    if (valid) {
      const uint64_t lower = peers & ((1ull << lane) - 1ull);
      pos = cnt[key] + __builtin_popcountll(lower);
    }
    // every lane has read cnt[] before the leaders advance it (in-order LDS within a wave)
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
    __builtin_amdgcn_wave_barrier();
    if (valid && __builtin_ctzll(peers) == lane) cnt[key] += __builtin_popcountll(peers);
    if (s < R) {
      eri[s] = pos;
      if (valid && sorted_src) sorted_src[pos] = static_cast<int32_t>(s);
    }
  }
}

// Single-launch routing for a few segments (decode batches, one rank's share): wave w of
// one 1024-thread block owns segment w (`seg` consecutive slots, a multiple of 64 up to
// kSegSlots).  Its keys stay in registers from the count to
// the placement and the per-segment counts and their prefix stay in LDS, so the three
// launches above become one; the order of the result is the same stable slot order.
__global__ __launch_bounds__(1024) void route_small_kernel(const int32_t* __restrict__ ids,
                                                           long long R, int e_base, int E, int bits,
                                                           int nseg, int seg, int32_t* __restrict__ tpe,
                                                           int32_t* __restrict__ offsets,
                                                           int32_t* __restrict__ err_word,
                                                           int32_t* __restrict__ eri,
                                                           int32_t* __restrict__ sorted_src) {
  extern __shared__ int32_t cnt_lds[];  // [nseg][E]
  __shared__ int32_t wsum[16];
  __shared__ int32_t werr[16];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const bool owner = wave < nseg;
  int32_t* cnt = cnt_lds + wave * E;
  int err = 0;
  const long long s0 = static_cast<long long>(wave) * seg;
  const int batches = seg / 64;   // 64-slot batches of this wave's segment
  uint32_t keys[kSegSlots / 64];
  if (owner) {
    for (int e = lane; e < E; e += 64) cnt[e] = 0;
#pragma unroll
    for (int it = 0; it < kSegSlots / 64; ++it)
      keys[it] = it < batches ? local_key(ids, s0 + it * 64 + lane, R, e_base, E, &err) : 0u;
#pragma unroll
    for (int it = 0; it < kSegSlots / 64; ++it) {
      if (it >= batches) break;
      const long long s = s0 + it * 64 + lane;
      const uint32_t key = keys[it];
      const uint64_t active = __ballot(s < R);
      if (active == 0) break;
      const uint64_t peers = peer_mask(key, bits, active);
      const bool leader = (s < R) && key < static_cast<uint32_t>(E) &&
                          (__builtin_ctzll(peers) == lane);
      if (leader) cnt[key] += __builtin_popcountll(peers);
    }
  }
  const bool any_err = __ballot(err) != 0;
  if (lane == 0) werr[wave] = any_err ? 1 : 0;
  __syncthreads();
  // per expert: exclusive prefix over segments, then over experts
  const int e = threadIdx.x;
  int32_t run = 0;
  if (e < E) {
    for (int w = 0; w < nseg; ++w) {
      const int32_t c = cnt_lds[w * E + e];
      cnt_lds[w * E + e] = run;
      run += c;
    }
  }
  const int32_t excl = block_excl_scan1024(run, wsum);
  if (e < E) {
    tpe[e] = run;
    offsets[e] = excl;
    if (e == E - 1) offsets[E] = excl + run;
    for (int w = 0; w < nseg; ++w) cnt_lds[w * E + e] += excl;
  }
  if (e == 0) {
    int32_t any = 0;
    for (int w = 0; w < 16; ++w) any |= werr[w];
    *err_word = any;
  }
  __syncthreads();
  if (!owner) return;
#pragma unroll
  for (int it = 0; it < kSegSlots / 64; ++it) {
    if (it >= batches) break;
    const long long s = s0 + it * 64 + lane;
    const uint64_t active = __ballot(s < R);
    if (active == 0) break;
    const uint32_t key = keys[it];
    const uint64_t peers = peer_mask(key, bits, active);
    const bool valid = (s < R) && key < static_cast<uint32_t>(E);
    int32_t pos = -1;
    if (valid) {
      const uint64_t lower = peers & ((1ull << lane) - 1ull);
      pos = cnt[key] + __builtin_popcountll(lower);
    }
    // every lane has read cnt[] before the leaders advance it (in-order LDS within a wave)
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
    __builtin_amdgcn_wave_barrier();
    if (valid && __builtin_ctzll(peers) == lane) cnt[key] += __builtin_popcountll(peers);
    if (s < R) {
      eri[s] = pos;
      if (valid && sorted_src) sorted_src[pos] = static_cast<int32_t>(s);
    }
  }
}

hipError_t launch_routing(const int32_t* ids, long long R, int e_base, int E, int32_t* counts_ws,
                          int32_t* seg_err, int32_t* err_word, int32_t* eri, int32_t* sorted_src,
                          int32_t* tpe, int32_t* offsets, hipStream_t st) {
  const int nseg = static_cast<int>((R + kSegSlots - 1) / kSegSlots);
  int bits = 0;
  while ((1 << bits) <= E) ++bits;  // keys 0..E (E = invalid sentinel)
  // up to 16 x kSegSlots slots: one launch, the slots cut into 16 near-equal segments of
  // whole 64-slot batches (one per wavefront), if their counts fit in 60 KB of LDS
  if (nseg <= 16) {
    const int seg = static_cast<int>(std::max<long long>(64, (((R + 15) / 16) + 63) / 64 * 64));
    const int nseg_s = static_cast<int>((R + seg - 1) / seg);
    const size_t small_lds = static_cast<size_t>(nseg_s) * E * sizeof(int32_t);
    if (small_lds <= kSmallRouteLds) {
      route_small_kernel<<<1, 1024, small_lds, st>>>(ids, R, e_base, E, bits, nseg_s, seg, tpe,
                                                      offsets, err_word, eri, sorted_src);
      return hipGetLastError();
    }
  }
  const size_t lds = 4 * static_cast<size_t>(E) * sizeof(int32_t);
  if (nseg > 0) {
    route_count_kernel<<<(nseg + 3) / 4, 256, lds, st>>>(ids, R, e_base, E, bits, counts_ws, nseg,
                                                          seg_err);
  }
  route_scan_kernel<<<1, 1024, 0, st>>>(counts_ws, nseg, E, tpe, offsets, seg_err, err_word);
  if (nseg > 0) {
    route_place_kernel<<<(nseg + 3) / 4, 256, lds, st>>>(ids, R, e_base, E, bits, counts_ws, nseg,
                                                          eri, sorted_src);
  }
  return hipGetLastError();
}

// ------------------------------------------------------------------ row expansion
// [R1P §MoE deployment strategy optimization]: expanded_x holds every token once
// per chosen expert, in expert order.  Scatter form: block (t) reads token row t
// once (16-byte vectors) and writes it to its k destination rows.
template <int EB>  // element bytes of x and of the expanded rows (4 = fp32, 2 = bf16)
__global__ __launch_bounds__(256) void expand_copy_kernel(const uint8_t* __restrict__ x, int H,
                                                          int k, const int32_t* __restrict__ eri,
                                                          uint8_t* __restrict__ out) {
  const int t = blockIdx.x;
  const long long row_bytes = static_cast<long long>(H) * EB;
  const int nvec = static_cast<int>(row_bytes / 16);
  const uint4* src = reinterpret_cast<const uint4*>(x + t * row_bytes);
  const int32_t* dst = eri + static_cast<long long>(t) * k;  // uniform over the block
  for (int v = threadIdx.x; v < nvec; v += blockDim.x) {
    const uint4 val = src[v];
    for (int j = 0; j < k; ++j) {
      const int32_t d = dst[j];
      if (d >= 0) reinterpret_cast<uint4*>(out + d * row_bytes)[v] = val;
    }
  }
}

// fp8 variant: [MND §Quantization] activations are quantized on the fly with one
// fp32 scale per 128-element vector.  16 lanes own one 128-element block (8 bf16
// each): amax by a 16-lane butterfly, scale = amax / 448, q = e4m3(x * (448/amax)),
// all in float32 with IEEE division.  A zero block gets scale 1 and zero codes.
__global__ __launch_bounds__(256) void expand_quant_kernel(const uint16_t* __restrict__ x, int H,
                                                           int k, const int32_t* __restrict__ eri,
                                                           uint8_t* __restrict__ out,
                                                           float* __restrict__ out_scale) {
  const int t = blockIdx.x;
  const int nblk = H / kQBlock;
  const int lane16 = threadIdx.x & 15;
  const int grp = threadIdx.x >> 4;  // 16 groups of 16 lanes per block
  // uniform over the block; NULL: the token's own row (per-token codes in token order)
  const int32_t* dst = eri ? eri + static_cast<long long>(t) * k : nullptr;
  for (int b = grp; b < nblk; b += 16) {
    const uint4 raw = reinterpret_cast<const uint4*>(x + static_cast<long long>(t) * H +
                                                     b * kQBlock)[lane16];
    float v[8];
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
#pragma unroll
    for (int o = 8; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 16));
    const bool zero = amax == 0.f;
    const float scale = zero ? 1.0f : amax / 448.0f;
    const float inv = zero ? 0.0f : 448.0f / amax;
    uint32_t lo = f32x4_to_e4m3(v[0] * inv, v[1] * inv, v[2] * inv, v[3] * inv);
    uint32_t hi = f32x4_to_e4m3(v[4] * inv, v[5] * inv, v[6] * inv, v[7] * inv);
    if (zero) lo = hi = 0;
    const uint2 q = make_uint2(lo, hi);
    for (int j = 0; j < k; ++j) {
      const int32_t d = dst ? dst[j] : t;
      if (d < 0) continue;
      reinterpret_cast<uint2*>(out + static_cast<long long>(d) * H + b * kQBlock)[lane16] = q;
      if (lane16 == 0) out_scale[static_cast<long long>(d) * nblk + b] = scale;
    }
  }
}

// Per-row int8 quantization of bf16 rows (the A8 of W8A8, [V32 §quantization
// strategy]): one block per row finds the row's amax, then writes codes
// round-half-even(x * (127 / amax)) with scale amax / 127 (a zero row: scale 1, codes 0),
// all in float32.  dst_rows [rows * k] sends row r to rows dst_rows[r*k + j] (the
// token expansion; negative entries are skipped); NULL writes row r in place of itself.
// n_rows (device, or NULL) bounds the rows that hold data.  Rows of up to 8192 columns are read from memory once: each thread
// keeps its 8-column vectors in registers between the amax and the coding pass.
constexpr int kQuantKeep = 4;  // 8-column vectors a thread keeps (256 threads: 8192 columns)

__device__ __forceinline__ float amax8_bf16(const uint4& raw, float amax) {
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
  for (int i = 0; i < 4; ++i)
    amax = fmaxf(amax, fmaxf(fabsf(__uint_as_float(w[i] << 16)),
                             fabsf(__uint_as_float(w[i] & 0xffff0000u))));
  return amax;
}

__device__ __forceinline__ uint2 codes8_i8(const uint4& raw, float inv) {
  const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
  uint32_t q[2] = {0u, 0u};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float v = __uint_as_float(i & 1 ? (w[i / 2] & 0xffff0000u) : (w[i / 2] << 16));
    const float code = fminf(fmaxf(rintf(v * inv), -127.0f), 127.0f);
    q[i / 4] |= (static_cast<uint32_t>(static_cast<int>(code)) & 0xffu) << (8 * (i % 4));
  }
  return make_uint2(q[0], q[1]);
}

__global__ __launch_bounds__(256) void quant_rows_i8_kernel(const uint16_t* __restrict__ src,
                                                            int cols, int k,
                                                            const int32_t* __restrict__ dst_rows,
                                                            const int32_t* __restrict__ n_rows,
                                                            int8_t* __restrict__ out,
                                                            float* __restrict__ out_scale) {
  __shared__ float wmax[4];
  const int r = blockIdx.x;
  if (n_rows && r >= *n_rows) return;
  const uint16_t* row = src + static_cast<long long>(r) * cols;
  float amax = 0.f;
  uint4 keep[kQuantKeep];
#pragma unroll
  for (int it = 0; it < kQuantKeep; ++it) {
    const int c = (threadIdx.x + it * 256) * 8;
    keep[it] = c < cols ? *reinterpret_cast<const uint4*>(row + c) : make_uint4(0, 0, 0, 0);
    amax = amax8_bf16(keep[it], amax);
  }
  for (int c = (threadIdx.x + kQuantKeep * 256) * 8; c < cols; c += 256 * 8)
    amax = amax8_bf16(*reinterpret_cast<const uint4*>(row + c), amax);
  amax = wave_max(amax);
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
  const bool zero = amax == 0.f;
  const float scale = zero ? 1.0f : amax / 127.0f;
  const float inv = zero ? 0.0f : 127.0f / amax;
  auto emit = [&](int c, const uint2 qq) {
    for (int j = 0; j < k; ++j) {
      const int32_t d = dst_rows ? dst_rows[static_cast<long long>(r) * k + j] : r;
      if (d < 0) continue;
      *reinterpret_cast<uint2*>(out + static_cast<long long>(d) * cols + c) = qq;
    }
  };
#pragma unroll
  for (int it = 0; it < kQuantKeep; ++it) {
    const int c = (threadIdx.x + it * 256) * 8;
    if (c < cols) emit(c, codes8_i8(keep[it], inv));
  }
  for (int c = (threadIdx.x + kQuantKeep * 256) * 8; c < cols; c += 256 * 8)
    emit(c, codes8_i8(*reinterpret_cast<const uint4*>(row + c), inv));
  if (threadIdx.x == 0) {
    for (int j = 0; j < k; ++j) {
      const int32_t d = dst_rows ? dst_rows[static_cast<long long>(r) * k + j] : r;
      if (d >= 0) out_scale[d] = scale;
    }
  }
}

hipError_t launch_quant_rows_i8(const void* src, int rows, int cols, int k, const int32_t* dst_rows,
                                const int32_t* n_rows, int8_t* out, float* out_scale,
                                hipStream_t st) {
  if (rows == 0) return hipSuccess;
  if (cols % 8) return hipErrorInvalidValue;
  quant_rows_i8_kernel<<<rows, 256, 0, st>>>(static_cast<const uint16_t*>(src), cols, k, dst_rows,
                                             n_rows, out, out_scale);
  return hipGetLastError();
}

hipError_t launch_expand(const void* x, int T, int H, int k, int act_bytes, bool quant_fp8,
                         const int32_t* eri, void* out, float* out_scale, hipStream_t st) {
  if (T == 0) return hipSuccess;
  if (!eri && (!quant_fp8 || k != 1)) return hipErrorInvalidValue;   // in place: fp8 codes only
  if (quant_fp8) {
    expand_quant_kernel<<<T, 256, 0, st>>>(static_cast<const uint16_t*>(x), H, k, eri,
                                           static_cast<uint8_t*>(out), out_scale);
  } else if (act_bytes == 2) {
    expand_copy_kernel<2><<<T, 256, 0, st>>>(static_cast<const uint8_t*>(x), H, k, eri,
                                             static_cast<uint8_t*>(out));
  } else {
    expand_copy_kernel<4><<<T, 256, 0, st>>>(static_cast<const uint8_t*>(x), H, k, eri,
                                             static_cast<uint8_t*>(out));
  }
  return hipGetLastError();
}

}  // namespace moe
