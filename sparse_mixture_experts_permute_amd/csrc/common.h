// Kernel-side helpers shared by the HIP sources of the MoE layer (gfx950).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef uint16_t bf16_t;  // bf16 held as its bit pattern

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_v;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_v;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4_v;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_v;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_v;

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_to_f32(bf16_t h) {
  return __uint_as_float(((uint32_t)h) << 16);
}

// Round to nearest even (the hardware conversion, v_cvt_pk_bf16_f32).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(bf16_t, (__bf16)f);
}

template <typename T> struct Elem;
template <> struct Elem<float> {
  __device__ __forceinline__ static float load(const float *p, size_t i) { return p[i]; }
  __device__ __forceinline__ static void store(float *p, size_t i, float v) { p[i] = v; }
};
template <> struct Elem<bf16_t> {
  __device__ __forceinline__ static float load(const bf16_t *p, size_t i) {
    return bf16_to_f32(p[i]);
  }
  __device__ __forceinline__ static void store(bf16_t *p, size_t i, float v) {
    p[i] = f32_to_bf16(v);
  }
};

__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & (kWave - 1)); }

// Raw buffer resource over [base, base + bytes): loads at byte offsets >= bytes
// return zeros (the hardware range check).  The last word selects 32-bit data
// format, which untyped buffer loads require.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                           0x00020000);
}

// 16 bytes per lane from a buffer (byte offset `voff` per lane) straight into
// LDS.  `lds` must be the same for every lane of the wavefront; lane l's bytes
// land at lds + 16*l.
// NT: non-temporal (streaming) cache policy, for data read once.
template <bool NT = false>
__device__ __forceinline__ void buffer_to_lds16(__amdgpu_buffer_rsrc_t r, uint32_t voff,
                                                uint4 *lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void *)lds, 16,
                                           (int)voff, 0, 0, NT ? 2 : 0);
}

// SiLU(a) = a * sigmoid(a), with the hardware exp2 and reciprocal (a few fp32
// ulp, far below the bf16 rounding of the activations or a 1e-4 fp32 tolerance).
__device__ __forceinline__ float silu(float a) {
  return a * __builtin_amdgcn_rcpf(1.0f + __expf(-a));
}

// Hidden unit of a gated expert from its two projections g = W1 x, u = W3 x:
// act 0 SiLU(g) * u (SwiGLU), act 1 sigmoid(g) * u (sigmoid-gated GLU).
__device__ __forceinline__ float gated(float g, float u, int act) {
  return act ? u * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) : silu(g) * u;
}

// First index i in [0, n) with a[i+1] > g, for non-decreasing a[0..n] with a[0] <= g.
__device__ __forceinline__ int upper_segment(const int32_t *a, int n, int g) {
  int lo = 0, hi = n;  // invariant: a[lo] <= g, answer in [lo, hi)
  while (hi - lo > 1) {
    int mid = (lo + hi) >> 1;
    if (a[mid] <= g) lo = mid; else hi = mid;
  }
  return lo;
}

}  // namespace moe
