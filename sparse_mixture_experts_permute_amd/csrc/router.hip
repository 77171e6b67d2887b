// Router scores, top-k selection and softmax gate.
//
// logits[t][e] = sum_i x[t][i] * Wg[e][i] (+ bias[e]), then per token the k
// largest scores (ties go to the lower expert index) and
// gate_j = exp(l_j - l_0) / sum_j' exp(l_j' - l_0) over the selected scores
// ("Chapter 10 MoE", section 10.3; "Mistral 8x7B SMoE architecture deep
// dive", section 3.2).  The router is a skinny contraction and runs on the
// vector ALU in fp32 (bf16 pairs through v_dot2_f32_bf16); the matrix cores
// are kept for the expert GEMMs.
//
// Two kernels:
//  scores : partial scores over S slices of the feature dimension, each slice
//           written to its own plane of a [S][T][E] buffer; S is chosen so the
//           grid fills the GPU.  Two shapes:
//           - up to 32 experts: one wavefront per (token, slice); lanes split the
//             slice with 16-byte loads, keep all E sums in registers and reduce
//             them with a butterfly at the end (the router weights, at most
//             32 x d, stay in L2);
//           - more experts: a register-tiled VALU GEMM.  A 256-thread block owns
//             64 tokens x 64 experts x one slice; each thread keeps 4 x 4 sums
//             and streams its slice through LDS in 64-element chunks
//             (double-buffered, one barrier per chunk).
//  topk   : one wavefront per token sums the S partials in a fixed order (so
//           the scores do not depend on scheduling), adds the bias, writes the
//           scores, and runs k rounds of a wavefront arg-max and the gate.
#include "common.h"
#include "kernels.h"
#include "route_block.h"

namespace moe {

namespace {

constexpr int RS_TOK = 64, RS_EXP = 64;  // block tile
constexpr int RS_THREADS = 256;
constexpr int RS_ROWB = 128;            // bytes of a row chunk (64 bf16 / 32 fp32)
constexpr int RS_LDW = (RS_ROWB + 16) / 16;  // padded LDS row stride in uint4

template <typename T> struct RouterTraits;
template <> struct RouterTraits<float> {
  static constexpr int VEC = 4;  // elements per 16 bytes
};
template <> struct RouterTraits<bf16_t> {
  static constexpr int VEC = 8;
};

__device__ __forceinline__ float dot16b(const uint4 &a, const uint4 &b, float acc, float) {
  acc = fmaf(__uint_as_float(a.x), __uint_as_float(b.x), acc);
  acc = fmaf(__uint_as_float(a.y), __uint_as_float(b.y), acc);
  acc = fmaf(__uint_as_float(a.z), __uint_as_float(b.z), acc);
  acc = fmaf(__uint_as_float(a.w), __uint_as_float(b.w), acc);
  return acc;
}

__device__ __forceinline__ float dot16b(const uint4 &a, const uint4 &b, float acc, bf16_t) {
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_v, a.x),
                                        __builtin_bit_cast(bf16x2_v, b.x), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_v, a.y),
                                        __builtin_bit_cast(bf16x2_v, b.y), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_v, a.z),
                                        __builtin_bit_cast(bf16x2_v, b.z), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_v, a.w),
                                        __builtin_bit_cast(bf16x2_v, b.w), acc, false);
  return acc;
}

// grid: (token tiles, expert tiles, feature slices); slice s covers
// features [s*dslice, (s+1)*dslice), dslice a multiple of the chunk.
template <typename T>
__global__ __launch_bounds__(RS_THREADS, 2) void router_scores_kernel(
    const T *__restrict__ x, const T *__restrict__ Wg, int T_, int d, int E, int dslice,
    float *__restrict__ part) {
  constexpr int VEC = RouterTraits<T>::VEC;
  constexpr int CPR = RS_ROWB / 16;  // uint4 per row chunk (8)
  __shared__ uint4 xs[2][RS_TOK * RS_LDW];
  __shared__ uint4 ws[2][RS_EXP * RS_LDW];

  const int tid = threadIdx.x;
  const int t0 = blockIdx.x * RS_TOK, e0 = blockIdx.y * RS_EXP;
  const int s = blockIdx.z;
  const int tg = tid / 16, eg = tid % 16;  // 16 x 16 threads, 4 x 4 outputs each

  const uint4 *xg = reinterpret_cast<const uint4 *>(x);
  const uint4 *wgg = reinterpret_cast<const uint4 *>(Wg);
  const size_t rowq = (size_t)d / VEC;
  const size_t q0 = (size_t)s * dslice / VEC;
  const int nchunk = dslice * (int)sizeof(T) / RS_ROWB;

  // each thread stages 2 x-chunks and 2 Wg-chunks of 16 bytes per row chunk
  uint4 rx[2], rw[2];
  auto gload = [&](int c) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int idx = tid + i * RS_THREADS;  // 0..511: 64 rows x 8 uint4
      const int r = idx / CPR, q = idx % CPR;
      const size_t col = q0 + (size_t)c * CPR + q;
      rx[i] = (t0 + r < T_) ? xg[(size_t)(t0 + r) * rowq + col] : make_uint4(0, 0, 0, 0);
      rw[i] = (e0 + r < E) ? wgg[(size_t)(e0 + r) * rowq + col] : make_uint4(0, 0, 0, 0);
    }
  };
  auto lstore = [&](int b) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int idx = tid + i * RS_THREADS;
      const int r = idx / CPR, q = idx % CPR;
      xs[b][r * RS_LDW + q] = rx[i];
      ws[b][r * RS_LDW + q] = rw[i];
    }
  };

  float acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[a][j] = 0.f;

  gload(0);
  lstore(0);
  __syncthreads();
  for (int c = 0; c < nchunk; ++c) {
    const int b = c & 1;
    if (c + 1 < nchunk) gload(c + 1);
#pragma unroll 2
    for (int q = 0; q < CPR; ++q) {
      uint4 xv[4], wv[4];
#pragma unroll
      for (int a = 0; a < 4; ++a) xv[a] = xs[b][(tg * 4 + a) * RS_LDW + q];
#pragma unroll
      for (int j = 0; j < 4; ++j) wv[j] = ws[b][(eg + 16 * j) * RS_LDW + q];
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[a][j] = dot16b(xv[a], wv[j], acc[a][j], T());
    }
    if (c + 1 < nchunk) lstore(b ^ 1);
    __syncthreads();
  }

  float *out = part + (size_t)s * T_ * E;
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    const int t = t0 + tg * 4 + a;
    if (t >= T_) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = e0 + eg + 16 * j;
      if (e < E) out[(size_t)t * E + e] = acc[a][j];
    }
  }
}

// Up to 32 experts: one wavefront per (token, slice of NS*64*VEC features).
template <typename T, int EB>
__global__ __launch_bounds__(256) void router_scores_narrow_kernel(
    const T *__restrict__ x, const T *__restrict__ Wg, int T_, int d, int E, int ns,
    float *__restrict__ part) {
  constexpr int VEC = RouterTraits<T>::VEC;
  const int w = threadIdx.x / kWave, lane = lane_id();
  const int t = blockIdx.x * 4 + w;
  const int s = blockIdx.y;
  if (t >= T_) return;
  const uint4 *xg = reinterpret_cast<const uint4 *>(x);
  const uint4 *wgg = reinterpret_cast<const uint4 *>(Wg);
  const size_t rowq = (size_t)d / VEC;
  const size_t q0 = (size_t)s * ns * kWave + lane;
  float acc[EB];
#pragma unroll
  for (int e = 0; e < EB; ++e) acc[e] = 0.f;
  for (int i = 0; i < ns; ++i) {
    const size_t q = q0 + (size_t)i * kWave;
    const uint4 xv = xg[(size_t)t * rowq + q];
#pragma unroll
    for (int e = 0; e < EB; ++e)
      if (e < E) acc[e] = dot16b(xv, wgg[(size_t)e * rowq + q], acc[e], T());
  }
  float *out = part + ((size_t)s * T_ + t) * E;
#pragma unroll
  for (int e = 0; e < EB; ++e) {
    if (e < E) {
      float v = acc[e];
#pragma unroll
      for (int off = kWave / 2; off > 0; off >>= 1) v += __shfl_xor(v, off);
      if (lane == 0) out[e] = v;
    }
  }
}

// Sum of a score's S slice partials (stride apart), in slice order; the loads
// go out eight at a time so that their latencies overlap.
__device__ __forceinline__ float sum_partials(const float *__restrict__ p, size_t stride, int S) {
  float l = 0.f;
  for (int s0 = 0; s0 < S; s0 += 8) {
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = s0 + i < S ? p[(size_t)(s0 + i) * stride] : 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (s0 + i < S) l += v[i];
  }
  return l;
}

// One wavefront per token: scores (partials summed in slice order), top-k, gate.
__global__ __launch_bounds__(256) void router_topk_kernel(
    const float *__restrict__ part, int S, const float *__restrict__ bias, int T_, int E, int k,
    int gate_mode, int32_t *__restrict__ idx, float *__restrict__ gate,
    float *__restrict__ logits) {
  __shared__ float selv[4][256];
  __shared__ int seli[4][256];
  const int w = threadIdx.x / kWave, lane = lane_id();
  const int t = blockIdx.x * 4 + w;
  if (t >= T_) return;
  float v[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = lane + kWave * j;
    float l = -INFINITY;
    if (e < E) {
      l = sum_partials(part + (size_t)t * E + e, (size_t)T_ * E, S);
      if (bias) l += bias[e];
      if (logits) logits[(size_t)t * E + e] = l;
    }
    v[j] = l;
  }
  wave_topk_gate(v, E, k, gate_mode, selv[w], seli[w], idx + (size_t)t * k, gate + (size_t)t * k);
}

// Top-k, gate and the grouping of the pairs by expert for a decode step
// (T <= 4 tokens, T * k <= 64 pairs, E <= 64) in one workgroup: the launch that follows the
// score kernel (one less than top-k and permutation kernels apart).  Scores
// are summed over the slices exactly as router_topk_kernel does; the grouping
// is the stable counting sort of the pair ids under the capacity (the pairs an
// expert keeps, in pair order), by one wavefront with a lane per pair.
// Outputs as router_topk_kernel plus the permutation kernels.
__global__ __launch_bounds__(256) void topk_permute_tiny_kernel(
    const float *__restrict__ part, int S, const float *__restrict__ bias, int T_, int E, int k,
    int gate_mode, int capacity, int bm0, int bm1, float *__restrict__ logits,
    int32_t *__restrict__ idx, float *__restrict__ gate, int32_t *__restrict__ counts,
    int32_t *__restrict__ offsets, int32_t *__restrict__ perm, int32_t *__restrict__ inv,
    int32_t *__restrict__ mtiles0, int32_t *__restrict__ mtiles1,
    int32_t *__restrict__ shared_seg, int32_t *__restrict__ active, int32_t *__restrict__ zero,
    int nzero) {
  __shared__ float selv[4][64];
  __shared__ int seli[4][64];
  __shared__ int sidx[64];
  const int tid = threadIdx.x, w = tid / kWave, lane = lane_id();
  for (int i = tid; i < nzero; i += 256) zero[i] = 0;
  for (int t = w; t < T_; t += 4) {
    float v[4];
    v[0] = -INFINITY;
    if (lane < E) {
      float l = sum_partials(part + (size_t)t * E + lane, (size_t)T_ * E, S);
      if (bias) l += bias[lane];
      logits[(size_t)t * E + lane] = l;
      v[0] = l;
    }
    v[1] = v[2] = v[3] = -INFINITY;
    wave_topk_gate(v, E, k, gate_mode, selv[w], seli[w], idx + (size_t)t * k,
                   gate + (size_t)t * k);
    // lane r wrote idx[r] (k <= 64): its own store, read back in program order
    if (lane < k) sidx[t * k + lane] = idx[(size_t)t * k + lane];
  }
  __syncthreads();
  if (w != 0) return;
  wave_group_pairs(sidx, T_, E, k, capacity, bm0, bm1,
                   RouteOut{counts, offsets, perm, inv, mtiles0, mtiles1, shared_seg, active});
}

// Feature slices for the score kernels (enough work items to fill the GPU).
// Narrow kernel: a slice is ns steps of 64 lanes x 16 bytes.  Tiled kernel: a
// slice is a whole number of 128-byte chunks.
struct RouterSplit {
  bool narrow;
  int S, ns;
};
RouterSplit router_split(int T, int d, int E, int esize) {
  RouterSplit r{};
  const int vec = 16 / esize;
  r.narrow = E <= 32 && d % (kWave * vec) == 0;
  if (r.narrow) {
    const int steps = d / (kWave * vec);   // 16-byte steps per lane over the whole row
    const long long waves_per_slice = T;   // one wave per token and slice
    int S = steps;                         // finest split: one step per lane
    while (S > 1 && (steps % (S / 2) == 0) && waves_per_slice * (S / 2) >= 2048) S /= 2;
    r.S = S;
    r.ns = steps / S;
    return r;
  }
  const int chunk = RS_ROWB / esize;
  const int nchunks = d / chunk;
  const long long tiles = (long long)((T + RS_TOK - 1) / RS_TOK) * ((E + RS_EXP - 1) / RS_EXP);
  int S = 1;
  while (tiles * S < 512 && S * 2 <= nchunks && nchunks % (S * 2) == 0) S *= 2;
  r.S = S;
  r.ns = 0;
  return r;
}

template <typename T>
void launch_scores(const RouterSplit &r, const void *x, const void *Wg, int T_, int d, int E,
                   float *part, hipStream_t s) {
  if (r.narrow) {
    dim3 grid((T_ + 3) / 4, r.S);
    if (E <= 8)
      hipLaunchKernelGGL((router_scores_narrow_kernel<T, 8>), grid, dim3(256), 0, s,
                         (const T *)x, (const T *)Wg, T_, d, E, r.ns, part);
    else if (E <= 16)
      hipLaunchKernelGGL((router_scores_narrow_kernel<T, 16>), grid, dim3(256), 0, s,
                         (const T *)x, (const T *)Wg, T_, d, E, r.ns, part);
    else
      hipLaunchKernelGGL((router_scores_narrow_kernel<T, 32>), grid, dim3(256), 0, s,
                         (const T *)x, (const T *)Wg, T_, d, E, r.ns, part);
  } else {
    dim3 grid((T_ + RS_TOK - 1) / RS_TOK, (E + RS_EXP - 1) / RS_EXP, r.S);
    hipLaunchKernelGGL(router_scores_kernel<T>, grid, dim3(RS_THREADS), 0, s, (const T *)x,
                       (const T *)Wg, T_, d, E, d / r.S, part);
  }
}

}  // namespace

bool route_permute_tiny_ok(int T, int E, int k) {
  // one token per wavefront: beyond that the tokens' top-k would run in turn
  return T >= 1 && T <= 4 && E <= 64 && T * k <= 64;
}

hipError_t launch_route_permute_tiny(int dtype, const void *x, const void *Wg, const float *bias,
                                     int T, int d, int E, int k, int gate_mode, int capacity,
                                     int bm0, int bm1, float *logits, int32_t *idx, float *gate,
                                     int32_t *counts, int32_t *offsets, int32_t *perm,
                                     int32_t *inv, int32_t *mtiles0, int32_t *mtiles1,
                                     int32_t *shared_seg, int32_t *active, int32_t *zero,
                                     int nzero, float *part, hipStream_t s) {
  const int P = T * k;
  const int cap = capacity < 0 || capacity > P ? P : capacity;
  if (!zero) nzero = 0;
  const int es = dtype == 1 ? 2 : 4;
  const RouterSplit r = router_split(T, d, E, es);
  if (dtype == 1)
    launch_scores<bf16_t>(r, x, Wg, T, d, E, part, s);
  else
    launch_scores<float>(r, x, Wg, T, d, E, part, s);
  hipLaunchKernelGGL(topk_permute_tiny_kernel, dim3(1), dim3(256), 0, s, part, r.S, bias, T, E,
                     k, gate_mode, cap, bm0, bm1, logits, idx, gate, counts, offsets, perm, inv,
                     mtiles0, mtiles1, shared_seg, active, zero, nzero);
  return hipGetLastError();
}

size_t router_partial_bytes(int T, int d, int E, int esize) {
  return (size_t)router_split(T, d, E, esize).S * T * E * 4;
}

hipError_t launch_router(int dtype, const void *x, const void *Wg, const float *bias, int T,
                         int d, int E, int k, int gate_mode, int32_t *idx, float *gate,
                         float *logits, float *part, hipStream_t s) {
  const int es = dtype == 1 ? 2 : 4;
  const RouterSplit r = router_split(T, d, E, es);
  if (dtype == 1)
    launch_scores<bf16_t>(r, x, Wg, T, d, E, part, s);
  else
    launch_scores<float>(r, x, Wg, T, d, E, part, s);
  hipLaunchKernelGGL(router_topk_kernel, dim3((T + 3) / 4), dim3(256), 0, s, part, r.S, bias, T,
                     E, k, gate_mode, idx, gate, logits);
  return hipGetLastError();
}

}  // namespace moe
