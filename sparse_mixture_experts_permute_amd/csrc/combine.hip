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

namespace moe {

namespace {

// Four consecutive elements of a Yp row (fp32 or bf16) as fp32.
__device__ __forceinline__ float4 load4(const float *p, size_t i4) {
  return reinterpret_cast<const float4 *>(p)[i4];
}
__device__ __forceinline__ float4 load4(const bf16_t *p, size_t i4) {
  const uint2 u = reinterpret_cast<const uint2 *>(p)[i4];
  return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xFFFF0000u),
                     __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xFFFF0000u));
}

// One block per token; each thread handles 4 consecutive columns per step.
// YT: Yp's element type (bf16 Yp has one plane).
template <typename T, typename YT>
__global__ __launch_bounds__(256) void combine_kernel(const YT *__restrict__ Yp, int nsplit,
                                                      size_t plane,
                                                      const float *__restrict__ Ys,
                                                      const int32_t *__restrict__ inv,
                                                      const float *__restrict__ gate, int k,
                                                      int d, T *__restrict__ y) {
  const int t = blockIdx.x;
  const int d4 = d / 4;
  for (int c = threadIdx.x; c < d4; c += 256) {
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int j = 0; j < k; ++j) {
      const int slot = inv[(size_t)t * k + j];
      if (slot < 0) continue;
      const float g = gate[(size_t)t * k + j];
      const size_t row = (size_t)slot * d4 + c;
      float4 v = load4(Yp, row);
      for (int sp = 1; sp < nsplit; ++sp) {
        const float4 u = load4(Yp + sp * plane, row);
        v.x += u.x;
        v.y += u.y;
        v.z += u.z;
        v.w += u.w;
      }
      acc.x = fmaf(g, v.x, acc.x);
      acc.y = fmaf(g, v.y, acc.y);
      acc.z = fmaf(g, v.z, acc.z);
      acc.w = fmaf(g, v.w, acc.w);
    }
    if (Ys) {
      const float4 v = reinterpret_cast<const float4 *>(Ys)[(size_t)t * d4 + c];
      acc.x += v.x;
      acc.y += v.y;
      acc.z += v.z;
      acc.w += v.w;
    }
    const size_t o = (size_t)t * d + 4 * c;
    Elem<T>::store(y, o + 0, acc.x);
    Elem<T>::store(y, o + 1, acc.y);
    Elem<T>::store(y, o + 2, acc.z);
    Elem<T>::store(y, o + 3, acc.w);
  }
}

}  // namespace

hipError_t launch_combine(int dtype, const void *Yp, int nsplit, size_t plane, const float *Ys,
                          const int32_t *inv, const float *gate, int T, int k, int d, void *y,
                          hipStream_t s, bool yp_bf16) {
  if (T <= 0) return hipSuccess;
  if (yp_bf16 && nsplit != 1) return hipErrorInvalidValue;
  if (yp_bf16)
    hipLaunchKernelGGL((combine_kernel<bf16_t, bf16_t>), dim3(T), dim3(256), 0, s,
                       (const bf16_t *)Yp, 1, plane, Ys, inv, gate, k, d, (bf16_t *)y);
  else if (dtype == 1)
    hipLaunchKernelGGL((combine_kernel<bf16_t, float>), dim3(T), dim3(256), 0, s,
                       (const float *)Yp, nsplit, plane, Ys, inv, gate, k, d, (bf16_t *)y);
  else
    hipLaunchKernelGGL((combine_kernel<float, float>), dim3(T), dim3(256), 0, s,
                       (const float *)Yp, nsplit, plane, Ys, inv, gate, k, d, (float *)y);
  return hipGetLastError();
}

}  // namespace moe
