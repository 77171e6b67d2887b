// Weight-only FP8 experts: quantisation of expert weights to OCP FP8 E4M3
// ("E4M3FN": sign, 4 exponent bits with bias 7, 3 mantissa bits; exponent
// field 0 holds the subnormals m * 2^-9; no infinities; S.1111.111 is NaN;
// largest finite 448) with one scale per expert ("Mistral 8x7B SMoE
// architecture deep dive", section 5.3: quantise only the expert weights,
// keep the router in high precision, give each expert its own scale).
//
// scale[e] = amax_e / 448 rounded to fp32 (1 for an all-zero expert), amax_e
// the largest |w| of expert e; q = the nearest E4M3 value of w / scale[e]
// (quotient in fp64, ties to the even mantissa, magnitudes above 448 give
// 448; rounded by integer arithmetic on the quotient's bits).  The dequantised weight is scale[e] * decode(q).  Four launches: clear
// the per-expert maxima, reduce them (atomic max of non-negative float bits,
// which is order independent), turn them into scales, encode.
#include <cmath>

#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int Q_THREADS = 256;

template <typename T>
__device__ __forceinline__ float load_w(const T *p, size_t i);
template <>
__device__ __forceinline__ float load_w<float>(const float *p, size_t i) { return p[i]; }
template <>
__device__ __forceinline__ float load_w<bf16_t>(const bf16_t *p, size_t i) {
  return bf16_to_f32(p[i]);
}

// Nearest E4M3 code of v by integer rounding of its fp64 bit pattern.  The
// significand S (53 bits with the hidden one) times 2^(e - 52) is |v|; the
// code's quantum is 2^(e - 3) for e >= -6 and 2^-9 below (the subnormal
// step), so |v| / quantum = S / 2^sh with sh = 49 (normal range) or
// 43 - e.  The quotient r is rounded half to even from the shifted-out bits;
// then code = 8 * (e + 6) + r in the normal range (r = 16 carries into the
// next exponent by itself) and code = r below it (r = 8 is the smallest
// normal, 0x08).  Codes above 0x7E (448) saturate to 0x7E.
__device__ __forceinline__ uint8_t fp8_e4m3_encode(double v) {
  const uint64_t bits = (uint64_t)__double_as_longlong(v);
  const uint8_t sign = (uint8_t)((bits >> 56) & 0x80);
  const int bexp = (int)((bits >> 52) & 0x7FF);
  if (bexp == 0) return sign;  // zero or an fp64 subnormal (far below 2^-10)
  const int e = bexp - 1023;
  if (e > 8) return sign | 0x7E;
  const uint64_t S = (bits & ((1ull << 52) - 1)) | (1ull << 52);
  const int sh = e >= -6 ? 49 : 43 - e;
  if (sh > 53) return sign;  // below 2^-10: rounds to zero (2^-10 itself ties to 0)
  uint64_t r = S >> sh;
  const uint64_t rem = S & ((1ull << sh) - 1), half = 1ull << (sh - 1);
  if (rem > half || (rem == half && (r & 1))) ++r;
  const uint64_t code = (e >= -6 ? (uint64_t)(8 * (e + 6)) : 0ull) + r;
  return sign | (uint8_t)(code > 0x7E ? 0x7E : code);
}

__global__ void fp8_clear_kernel(float *__restrict__ amax, int E) {
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e < E) amax[e] = 0.f;
}

// grid (blocks per expert, E): block-local maximum, then one atomic per block
template <typename T>
__global__ __launch_bounds__(Q_THREADS) void fp8_amax_kernel(const T *__restrict__ W, size_t n,
                                                             float *__restrict__ amax) {
  __shared__ float red[Q_THREADS / kWave];
  const int e = blockIdx.y;
  const T *w = W + (size_t)e * n;
  float m = 0.f;
  for (size_t i = (size_t)blockIdx.x * Q_THREADS + threadIdx.x; i < n;
       i += (size_t)gridDim.x * Q_THREADS)
    m = fmaxf(m, fabsf(load_w(w, i)));
#pragma unroll
  for (int off = kWave / 2; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  if (lane_id() == 0) red[threadIdx.x / kWave] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int i = 1; i < Q_THREADS / kWave; ++i) m = fmaxf(m, red[i]);
    // non-negative floats order as their bit patterns
    atomicMax(reinterpret_cast<unsigned int *>(amax) + e, __float_as_uint(m));
  }
}

__global__ void fp8_scale_kernel(float *__restrict__ scale, int E) {
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e < E) {
    const float a = scale[e];
    scale[e] = a > 0.f ? (float)((double)a / 448.0) : 1.0f;
  }
}

template <typename T>
__global__ __launch_bounds__(Q_THREADS) void fp8_encode_kernel(const T *__restrict__ W, size_t n,
                                                               const float *__restrict__ scale,
                                                               uint8_t *__restrict__ q) {
  const int e = blockIdx.y;
  const double s = (double)scale[e];
  const T *w = W + (size_t)e * n;
  uint8_t *qe = q + (size_t)e * n;
  for (size_t i = (size_t)blockIdx.x * Q_THREADS + threadIdx.x; i < n;
       i += (size_t)gridDim.x * Q_THREADS)
    qe[i] = fp8_e4m3_encode((double)load_w(w, i) / s);
}

template <typename T>
hipError_t quantize_t(const void *W, int E, size_t n, uint8_t *q, float *scale, hipStream_t s) {
  const int eb = (E + Q_THREADS - 1) / Q_THREADS;
  // about 2048 blocks in all, at least one per expert
  const size_t per = (size_t)(2048 + E - 1) / E;
  const unsigned bx = (unsigned)std::max<size_t>(1, std::min(per, (n + Q_THREADS - 1) / Q_THREADS));
  hipLaunchKernelGGL(fp8_clear_kernel, dim3(eb), dim3(Q_THREADS), 0, s, scale, E);
  hipLaunchKernelGGL((fp8_amax_kernel<T>), dim3(bx, E), dim3(Q_THREADS), 0, s, (const T *)W, n,
                     scale);
  hipLaunchKernelGGL(fp8_scale_kernel, dim3(eb), dim3(Q_THREADS), 0, s, scale, E);
  hipLaunchKernelGGL((fp8_encode_kernel<T>), dim3(bx, E), dim3(Q_THREADS), 0, s, (const T *)W, n,
                     scale, q);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize_fp8(int dtype, const void *W, int E, size_t n, uint8_t *q,
                               float *scale, hipStream_t s) {
  if (E <= 0 || n == 0) return hipSuccess;
  return dtype == 1 ? quantize_t<bf16_t>(W, E, n, q, scale, s)
                    : quantize_t<float>(W, E, n, q, scale, s);
}

}  // namespace moe
