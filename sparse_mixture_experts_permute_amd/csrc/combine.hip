// Gate-weighted combine back to token order:
//   y[t][:] = sum_{j<k} gate[t][j] * Yp[inv[t*k+j]][:]  (+ Ys[t][:] for the shared expert)
// A pair with inv < 0 was dropped by an expert's capacity limit and adds
// nothing.  Summed in fp32 with j ascending, written once per token with no
// atomics.  When the down projection split K into planes, Yp has nsplit planes
// whose rows are added first, in plane order; the bf16 layer's tiled down
// projection otherwise leaves Yp in bf16
// ("Chapter 10 MoE", sections 10.4 and 10.5; "Mixtral and MoE architecture",
// weighted accumulation in the MixtralMoE listing).
#include "common.h"
#include "kernels.h"

#include <algorithm>
#include <type_traits>

namespace moe {

namespace {

// Eight consecutive elements of a Yp row (fp32 or bf16), raw: two float4 or
// one uint4 of bf16 pairs; i8 counts 8-element chunks.
struct Raw8f {
  float4 a, b;
};
struct Raw8h {
  uint4 u;
};
template <typename YT> struct Raw8;
template <> struct Raw8<float> { using type = Raw8f; };
template <> struct Raw8<bf16_t> { using type = Raw8h; };

__device__ __forceinline__ Raw8f load8(const float *p, size_t i8) {
  const float4 *q = reinterpret_cast<const float4 *>(p) + 2 * i8;
  return Raw8f{q[0], q[1]};
}
__device__ __forceinline__ Raw8h load8(const bf16_t *p, size_t i8) {
  return Raw8h{reinterpret_cast<const uint4 *>(p)[i8]};
}
__device__ __forceinline__ void to_f32(const Raw8f &r, float (&v)[8]) {
  v[0] = r.a.x; v[1] = r.a.y; v[2] = r.a.z; v[3] = r.a.w;
  v[4] = r.b.x; v[5] = r.b.y; v[6] = r.b.z; v[7] = r.b.w;
}
__device__ __forceinline__ void to_f32(const Raw8h &r, float (&v)[8]) {
  const uint32_t w[4] = {r.u.x, r.u.y, r.u.z, r.u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}
__device__ __forceinline__ void store8(float *p, size_t o, const float (&v)[8]) {
  float4 *q = reinterpret_cast<float4 *>(p + o);
  q[0] = make_float4(v[0], v[1], v[2], v[3]);
  q[1] = make_float4(v[4], v[5], v[6], v[7]);
}
__device__ __forceinline__ void store8(bf16_t *p, size_t o, const float (&v)[8]) {
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    w[i] = (uint32_t)__builtin_bit_cast(uint16_t, f32_to_bf16(v[2 * i])) |
           ((uint32_t)__builtin_bit_cast(uint16_t, f32_to_bf16(v[2 * i + 1])) << 16);
  *reinterpret_cast<uint4 *>(p + o) = make_uint4(w[0], w[1], w[2], w[3]);
}

// One block per token; each thread handles 8 consecutive columns per step
// (d is a multiple of 8).  The Yp rows of J pairs at a time are all in flight
// before the sums, which still run in pair order: the loads are unconditional
// (a pair past k, or dropped, reads row 0 and is then skipped), since a load
// under a branch would be waited for before the next one is issued.  YT: Yp's
// element type (bf16 Yp has one plane).
template <int J, typename T, typename YT>
__global__ __launch_bounds__(1024) void combine_kernel(const YT *__restrict__ Yp, int nsplit,
                                                       size_t plane,
                                                       const float *__restrict__ Ys,
                                                       const int32_t *__restrict__ inv,
                                                       const float *__restrict__ gate, int k,
                                                       int d, T *__restrict__ y) {
  using R8 = typename Raw8<YT>::type;
  const int t = blockIdx.x;
  const int d8 = d / 8;
  const int32_t *tinv = inv + (size_t)t * k;
  const float *tgate = gate + (size_t)t * k;
  for (int c = threadIdx.x; c < d8; c += blockDim.x) {
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int j0 = 0; j0 < k; j0 += J) {
      int slot[J];
      R8 r[J];
#pragma unroll
      for (int u = 0; u < J; ++u) {
        const int sv = tinv[min(j0 + u, k - 1)];
        slot[u] = j0 + u < k ? sv : -1;
        r[u] = load8(Yp, (size_t)max(slot[u], 0) * d8 + c);
      }
#pragma unroll
      for (int u = 0; u < J; ++u) {
        float v[8];
        to_f32(r[u], v);
        if constexpr (std::is_same<YT, float>::value) {
          for (int sp = 1; sp < nsplit; ++sp) {
            float w[8];
            to_f32(load8(Yp + sp * plane, (size_t)max(slot[u], 0) * d8 + c), w);
#pragma unroll
            for (int i = 0; i < 8; ++i) v[i] += w[i];
          }
        }
        // no pair, or dropped by a capacity limit: acc stays as it is
        const bool use = slot[u] >= 0;
        const float g = tgate[min(j0 + u, k - 1)];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float a = fmaf(g, v[i], acc[i]);
          acc[i] = use ? a : acc[i];
        }
      }
    }
    if (Ys) {
      float v[8];
      to_f32(load8(Ys, (size_t)t * d8 + c), v);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += v[i];
    }
    store8(y, (size_t)t * d + 8 * (size_t)c, acc);
  }
}

}  // namespace

hipError_t launch_combine(int dtype, const void *Yp, int nsplit, size_t plane, const float *Ys,
                          const int32_t *inv, const float *gate, int T, int k, int d, void *y,
                          hipStream_t s, bool yp_bf16) {
  if (T <= 0) return hipSuccess;
  if ((yp_bf16 && nsplit != 1) || d % 8 || plane % 8) return hipErrorInvalidValue;
  // a thread per 8 columns, in whole waves, up to 1024 per token
  const dim3 grid(T), block(std::min(1024, (d / 8 + 63) / 64 * 64));
#define COMBINE_LAUNCH(J)                                                                    \
  if (yp_bf16)                                                                               \
    hipLaunchKernelGGL((combine_kernel<J, bf16_t, bf16_t>), grid, block, 0, s,               \
                       (const bf16_t *)Yp, 1, plane, Ys, inv, gate, k, d, (bf16_t *)y);      \
  else if (dtype == 1)                                                                       \
    hipLaunchKernelGGL((combine_kernel<J, bf16_t, float>), grid, block, 0, s,                \
                       (const float *)Yp, nsplit, plane, Ys, inv, gate, k, d, (bf16_t *)y);  \
  else                                                                                       \
    hipLaunchKernelGGL((combine_kernel<J, float, float>), grid, block, 0, s,                 \
                       (const float *)Yp, nsplit, plane, Ys, inv, gate, k, d, (float *)y)
  if (k <= 2)
    COMBINE_LAUNCH(2);
  else if (k <= 4)
    COMBINE_LAUNCH(4);
  else
    COMBINE_LAUNCH(8);
#undef COMBINE_LAUNCH
  return hipGetLastError();
}

}  // namespace moe
