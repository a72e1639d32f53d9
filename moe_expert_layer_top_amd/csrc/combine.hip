// Un-permute + weighted combine, and the fp32 kernels of the MoE layer (gfx950).
//
// [R1P] = page "CANN/cann-recipes-infer: DeepSeek-R1 prefill optimization".
// [R1P §MoE deployment strategy optimization]: finalize-routing restores the
// original token order through expanded_row_idx and, in the same op, forms the
// weighted sum of the routed-expert rows plus the shared-expert output.
// [MND] = page "Lower latency and higher throughput with multi-node DeepSeek deployment".

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

// ------------------------------------------------------------------ split-K reductions
// A grouped GEMM whose grid would leave most CUs idle (decode batches of a few tokens)
// splits its reduction into S slices and stores fp32 partials [S][rows][N]; these
// kernels add the S partials of an element in slice order (fp32) and finish the step
// the GEMM's own epilogue would have done.  One block per row; rows at or past *n_rows
// (device count, or all rows when NULL) hold no data and are skipped.

// SwiGLU of the first expert GEMM: partial columns 0..I-1 are the gate projection,
// I..2I-1 the up projection; h = silu(g) * u, stored bf16, or (FP8) quantized per
// 1x128 block with scale = amax / 448 and codes e4m3(h * 448 / amax) ([MND §Quantization],
// the same arithmetic as the fused epilogue).  Thread t owns 4 consecutive h columns of
// each 1024-column pass; a 128-column block is 32 consecutive threads (half a wave).
template <bool FP8>
__global__ __launch_bounds__(256) void swiglu_reduce_kernel(const float* __restrict__ part, int S,
                                                            long long split_stride, int I,
                                                            const int32_t* __restrict__ n_rows,
                                                            uint8_t* __restrict__ h,
                                                            float* __restrict__ h_scale) {
  const int r = blockIdx.x;
  if (n_rows && r >= *n_rows) return;
  const float* row = part + static_cast<long long>(r) * 2 * I;
  for (int c = threadIdx.x * 4; c < I; c += 256 * 4) {
    f32x4 g = *reinterpret_cast<const f32x4*>(row + c);
    f32x4 u = *reinterpret_cast<const f32x4*>(row + I + c);
    for (int sp = 1; sp < S; ++sp) {
      const float* q = row + sp * split_stride;
      g += *reinterpret_cast<const f32x4*>(q + c);
      u += *reinterpret_cast<const f32x4*>(q + I + c);
    }
    float hv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) hv[i] = silu_fast(g[i]) * u[i];
    if constexpr (FP8) {
      float m = fmaxf(fmaxf(fabsf(hv[0]), fabsf(hv[1])), fmaxf(fabsf(hv[2]), fabsf(hv[3])));
#pragma unroll
      for (int o = 16; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 32));
      const bool zero = m == 0.f;
      const float scale = zero ? 1.0f : m / 448.0f;
      const float inv = zero ? 0.0f : 448.0f / m;
      const uint32_t q = f32x4_to_e4m3(hv[0] * inv, hv[1] * inv, hv[2] * inv, hv[3] * inv);
      *reinterpret_cast<uint32_t*>(h + static_cast<long long>(r) * I + c) = zero ? 0u : q;
      if ((threadIdx.x & 31) == 0) h_scale[static_cast<long long>(r) * (I / kQBlock) + c / kQBlock] = scale;
    } else {
      *reinterpret_cast<uint2*>(h + (static_cast<long long>(r) * I + c) * 2) =
          make_uint2(pack_bf16x2(hv[0], hv[1]), pack_bf16x2(hv[2], hv[3]));
    }
  }
}

// Plain sum of the partials, rounded once to bf16 (the second expert GEMM).
__global__ __launch_bounds__(256) void sum_reduce_kernel(const float* __restrict__ part, int S,
                                                         long long split_stride, int N,
                                                         const int32_t* __restrict__ n_rows,
                                                         uint16_t* __restrict__ y) {
  const int r = blockIdx.x;
  if (n_rows && r >= *n_rows) return;
  const float* row = part + static_cast<long long>(r) * N;
  for (int c = threadIdx.x * 4; c < N; c += 256 * 4) {
    f32x4 v = *reinterpret_cast<const f32x4*>(row + c);
    for (int sp = 1; sp < S; ++sp) v += *reinterpret_cast<const f32x4*>(row + sp * split_stride + c);
    *reinterpret_cast<uint2*>(y + static_cast<long long>(r) * N + c) =
        make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
  }
}

hipError_t launch_swiglu_reduce(const float* part, int S, long long split_stride, int rows, int I,
                                const int32_t* n_rows, void* h, bool fp8, float* h_scale,
                                hipStream_t st) {
  if (rows == 0) return hipSuccess;
  if (S < 1 || I % kQBlock || (fp8 && !h_scale)) return hipErrorInvalidValue;
  if (fp8) {
    swiglu_reduce_kernel<true><<<rows, 256, 0, st>>>(part, S, split_stride, I, n_rows,
                                                      static_cast<uint8_t*>(h), h_scale);
  } else {
    swiglu_reduce_kernel<false><<<rows, 256, 0, st>>>(part, S, split_stride, I, n_rows,
                                                       static_cast<uint8_t*>(h), nullptr);
  }
  return hipGetLastError();
}

hipError_t launch_sum_reduce(const float* part, int S, long long split_stride, int rows, int N,
                             const int32_t* n_rows, void* y, hipStream_t st) {
  if (rows == 0) return hipSuccess;
  if (S < 1 || N % 4) return hipErrorInvalidValue;
  sum_reduce_kernel<<<rows, 256, 0, st>>>(part, S, split_stride, N, n_rows,
                                          static_cast<uint16_t*>(y));
  return hipGetLastError();
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
