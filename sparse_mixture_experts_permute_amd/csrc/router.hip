// Router scores, top-k selection and softmax gate, fused in one kernel.
//
// logits[t][e] = sum_i x[t][i] * Wg[e][i] (+ bias[e])  -- fp32 accumulate on the
// vector ALU (the router is a skinny contraction; matrix cores are kept for the
// expert GEMMs).  Then, per token, k rounds of a wavefront arg-max (ties go to
// the lower expert index) and gate_j = exp(l_j - l_0) / sum_j' exp(l_j' - l_0)
// over the selected logits ("Chapter 10 MoE", section 10.3; "Mistral 8x7B SMoE
// architecture deep dive", section 3.2).
//
// Work split: a 256-thread block owns 32 tokens and every expert.  Thread
// (tg = tid/32, eg = tid%32) accumulates tokens 4*tg..4*tg+3 against experts
// eg, eg+32, ..., so each Wg element fetched into LDS feeds 32 tokens.  The
// feature dimension is streamed through LDS in 128-byte row chunks.
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int RT_TOK = 32;      // tokens per block
constexpr int RT_THREADS = 256;
constexpr int RT_EMAX = 256;
constexpr int RT_EJ = RT_EMAX / 32;  // experts per thread at most
constexpr int RT_ROWB = 128;         // bytes of a row chunk
constexpr int RT_PADB = 16;          // LDS row padding (bytes)

template <typename T> struct RouterTraits;
template <> struct RouterTraits<float> {
  static constexpr int DC = RT_ROWB / 4;  // elements per chunk
  static constexpr int VEC = 4;           // elements per 16-byte load
};
template <> struct RouterTraits<bf16_t> {
  static constexpr int DC = RT_ROWB / 2;
  static constexpr int VEC = 8;
};

__device__ __forceinline__ float dot16b(const uint4 &a, const uint4 &b, float acc, float) {
  // fp32 x 4
  acc = fmaf(__uint_as_float(a.x), __uint_as_float(b.x), acc);
  acc = fmaf(__uint_as_float(a.y), __uint_as_float(b.y), acc);
  acc = fmaf(__uint_as_float(a.z), __uint_as_float(b.z), acc);
  acc = fmaf(__uint_as_float(a.w), __uint_as_float(b.w), acc);
  return acc;
}

__device__ __forceinline__ float dot16b(const uint4 &a, const uint4 &b, float acc, bf16_t) {
  // bf16 x 8 through the packed bf16 dot (fp32 accumulate)
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

template <typename T>
__global__ __launch_bounds__(RT_THREADS) void router_topk_kernel(
    const T *__restrict__ x, const T *__restrict__ Wg, const float *__restrict__ bias, int T_,
    int d, int E, int k, int32_t *__restrict__ idx, float *__restrict__ gate,
    float *__restrict__ logits) {
  constexpr int DC = RouterTraits<T>::DC;
  constexpr int VEC = RouterTraits<T>::VEC;
  constexpr int CPR = RT_ROWB / 16;            // 16-byte chunks per row chunk
  constexpr int LDR = (RT_ROWB + RT_PADB) / 16;  // LDS row stride in uint4
  __shared__ uint4 xs[RT_TOK * LDR];
  __shared__ uint4 ws[RT_EMAX * LDR];
  __shared__ float ls[RT_TOK][RT_EMAX + 1];
  __shared__ float selv[RT_THREADS / kWave][RT_EMAX];
  __shared__ int seli[RT_THREADS / kWave][RT_EMAX];

  const int tid = threadIdx.x;
  const int t0 = blockIdx.x * RT_TOK;
  const int tg = tid / 32, eg = tid % 32;
  const int ej = (E + 31) / 32;

  float acc[4][RT_EJ];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int j = 0; j < RT_EJ; ++j) acc[a][j] = 0.f;

  const uint4 *xg = reinterpret_cast<const uint4 *>(x);
  const uint4 *wgg = reinterpret_cast<const uint4 *>(Wg);
  const size_t rowq = (size_t)d / VEC;  // uint4 per row

  for (int c0 = 0; c0 < d; c0 += DC) {
    const size_t cq = (size_t)c0 / VEC;
    // stage x chunk: RT_TOK rows x CPR uint4 (one per thread)
    for (int i = tid; i < RT_TOK * CPR; i += RT_THREADS) {
      int r = i / CPR, q = i % CPR;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (t0 + r < T_) v = xg[(size_t)(t0 + r) * rowq + cq + q];
      xs[r * LDR + q] = v;
    }
    for (int i = tid; i < E * CPR; i += RT_THREADS) {
      int r = i / CPR, q = i % CPR;
      ws[r * LDR + q] = wgg[(size_t)r * rowq + cq + q];
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < CPR; ++q) {
      uint4 xv[4];
#pragma unroll
      for (int a = 0; a < 4; ++a) xv[a] = xs[(tg * 4 + a) * LDR + q];
#pragma unroll
      for (int j = 0; j < RT_EJ; ++j) {
        if (j < ej) {
          int e = eg + 32 * j;
          if (e < E) {
            uint4 wv = ws[e * LDR + q];
#pragma unroll
            for (int a = 0; a < 4; ++a) acc[a][j] = dot16b(xv[a], wv, acc[a][j], T());
          }
        }
      }
    }
    __syncthreads();
  }

  // scores to LDS (and to global when requested)
#pragma unroll
  for (int j = 0; j < RT_EJ; ++j) {
    int e = eg + 32 * j;
    if (j < ej && e < E) {
      float b = bias ? bias[e] : 0.f;
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        int tl = tg * 4 + a;
        float v = acc[a][j] + b;
        ls[tl][e] = v;
        if (logits && t0 + tl < T_) logits[(size_t)(t0 + tl) * E + e] = v;
      }
    }
  }
  __syncthreads();

  // top-k + gate: each wave takes 8 tokens
  const int w = tid / kWave, lane = lane_id();
  for (int tl = w * (RT_TOK / 4); tl < (w + 1) * (RT_TOK / 4); ++tl) {
    const int t = t0 + tl;
    if (t >= T_) break;
    float v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      int e = lane + kWave * j;
      v[j] = e < E ? ls[tl][e] : -INFINITY;
    }
    unsigned taken = 0;
    for (int r = 0; r < k; ++r) {
      float bv = -INFINITY;
      int bi = 0x7fffffff;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        int e = lane + kWave * j;
        if (e < E && !(taken & (1u << j)) && (bi == 0x7fffffff || v[j] > bv)) {
          bv = v[j];
          bi = e;
        }
      }
#pragma unroll
      for (int off = kWave / 2; off > 0; off >>= 1) {
        float ov = __shfl_xor(bv, off);
        int oi = __shfl_xor(bi, off);
        if (oi != 0x7fffffff && (bi == 0x7fffffff || ov > bv || (ov == bv && oi < bi))) {
          bv = ov;
          bi = oi;
        }
      }
      if ((bi & (kWave - 1)) == lane) taken |= 1u << (bi / kWave);
      if (lane == 0) {
        selv[w][r] = bv;
        seli[w][r] = bi;
      }
    }
    // lane 0's selections become visible to the whole wave
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    const float m = selv[w][0];
    float z = 0.f;
    for (int r = lane; r < k; r += kWave) z += expf(selv[w][r] - m);
#pragma unroll
    for (int off = kWave / 2; off > 0; off >>= 1) z += __shfl_xor(z, off);
    for (int r = lane; r < k; r += kWave) {
      idx[(size_t)t * k + r] = seli[w][r];
      gate[(size_t)t * k + r] = expf(selv[w][r] - m) / z;
    }
    __builtin_amdgcn_wave_barrier();
  }
}

}  // namespace

hipError_t launch_router(int dtype, const void *x, const void *Wg, const float *bias, int T,
                         int d, int E, int k, int32_t *idx, float *gate, float *logits,
                         hipStream_t s) {
  dim3 grid((T + RT_TOK - 1) / RT_TOK);
  if (dtype == 1)
    hipLaunchKernelGGL(router_topk_kernel<bf16_t>, grid, dim3(RT_THREADS), 0, s,
                       (const bf16_t *)x, (const bf16_t *)Wg, bias, T, d, E, k, idx, gate,
                       logits);
  else
    hipLaunchKernelGGL(router_topk_kernel<float>, grid, dim3(RT_THREADS), 0, s,
                       (const float *)x, (const float *)Wg, bias, T, d, E, k, idx, gate,
                       logits);
  return hipGetLastError();
}

}  // namespace moe
