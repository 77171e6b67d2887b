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
//           - up to 32 experts: four tokens per wavefront, 16 lanes each, which
//             split the slice with 16-byte loads, keep all E sums in registers
//             and reduce them over the 16 lanes at the end (the router weights,
//             at most 32 x d, stay in L2 and each load of them serves four
//             tokens).  With one slice (large batches) and k <= 16 this kernel
//             also runs the top-k and the gate, and there is no second kernel;
//           - more experts: a register-tiled VALU GEMM.  A 256-thread block owns
//             128 tokens x 128 experts x one slice; each thread keeps 8 x 8 sums
//             (8 LDS reads per 64 dot products) and streams its slice through
//             LDS in 64-element chunks (double-buffered, one barrier per
//             chunk).
//  topk   : one wavefront per token sums the S partials in a fixed order (so
//           the scores do not depend on scheduling), adds the bias, writes the
//           scores, and runs k rounds of a wavefront arg-max and the gate.
#include "common.h"
#include "kernels.h"
#include "route_block.h"

namespace moe {

namespace {

constexpr int RS_TOK = 128, RS_EXP = 128;  // block tile
constexpr int RS_JT = RS_TOK / 16;  // tokens per thread
constexpr int RS_JE = RS_EXP / 16;  // experts per thread
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
  const int tg = tid / 16, eg = tid % 16;  // 16 x 16 threads, RS_JT x RS_JE outputs each

  const uint4 *xg = reinterpret_cast<const uint4 *>(x);
  const uint4 *wgg = reinterpret_cast<const uint4 *>(Wg);
  const size_t rowq = (size_t)d / VEC;
  const size_t q0 = (size_t)s * dslice / VEC;
  const int nchunk = dslice * (int)sizeof(T) / RS_ROWB;

  constexpr int NX = RS_TOK * CPR / RS_THREADS, NW = RS_EXP * CPR / RS_THREADS;
  uint4 rx[NX], rw[NW];
  auto gload = [&](int c) {
#pragma unroll
    for (int i = 0; i < NX; ++i) {
      const int idx = tid + i * RS_THREADS;
      const int r = idx / CPR, q = idx % CPR;
      const size_t col = q0 + (size_t)c * CPR + q;
      rx[i] = (t0 + r < T_) ? xg[(size_t)(t0 + r) * rowq + col] : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < NW; ++i) {
      const int idx = tid + i * RS_THREADS;
      const int r = idx / CPR, q = idx % CPR;
      const size_t col = q0 + (size_t)c * CPR + q;
      rw[i] = (e0 + r < E) ? wgg[(size_t)(e0 + r) * rowq + col] : make_uint4(0, 0, 0, 0);
    }
  };
  auto lstore = [&](int b) {
#pragma unroll
    for (int i = 0; i < NX; ++i) {
      const int idx = tid + i * RS_THREADS;
      xs[b][(idx / CPR) * RS_LDW + idx % CPR] = rx[i];
    }
#pragma unroll
    for (int i = 0; i < NW; ++i) {
      const int idx = tid + i * RS_THREADS;
      ws[b][(idx / CPR) * RS_LDW + idx % CPR] = rw[i];
    }
  };

  float acc[RS_JT][RS_JE];
#pragma unroll
  for (int a = 0; a < RS_JT; ++a)
#pragma unroll
    for (int j = 0; j < RS_JE; ++j) acc[a][j] = 0.f;

  gload(0);
  lstore(0);
  __syncthreads();
  for (int c = 0; c < nchunk; ++c) {
    const int b = c & 1;
    if (c + 1 < nchunk) gload(c + 1);
#pragma unroll 2
    for (int q = 0; q < CPR; ++q) {
      uint4 xv[RS_JT], wv[RS_JE];
#pragma unroll
      for (int a = 0; a < RS_JT; ++a) xv[a] = xs[b][(tg * RS_JT + a) * RS_LDW + q];
#pragma unroll
      for (int j = 0; j < RS_JE; ++j) wv[j] = ws[b][(eg + 16 * j) * RS_LDW + q];
#pragma unroll
      for (int a = 0; a < RS_JT; ++a)
#pragma unroll
        for (int j = 0; j < RS_JE; ++j) acc[a][j] = dot16b(xv[a], wv[j], acc[a][j], T());
    }
    if (c + 1 < nchunk) lstore(b ^ 1);
    __syncthreads();
  }

  float *out = part + (size_t)s * T_ * E;
#pragma unroll
  for (int a = 0; a < RS_JT; ++a) {
    const int t = t0 + tg * RS_JT + a;
    if (t >= T_) continue;
#pragma unroll
    for (int j = 0; j < RS_JE; ++j) {
      const int e = e0 + eg + 16 * j;
      if (e < E) out[(size_t)t * E + e] = acc[a][j];
    }
  }
}

// Top-k and gate of one token from its E (<= EB) scores held by every lane of
// a group (the same rule and arithmetic as wave_topk_gate: picks by strict >
// in expert order, so ties go to the lower index; the sums run in expert or
// pick order instead of the butterfly's).  Lane j < k of the group writes pick
// j.  Returns nothing; idx / gate point at the token's k slots.
template <int EB>
__device__ __forceinline__ void group_topk_gate(const float (&v)[EB], int E, int k, int gate_mode,
                                                int li, int32_t *__restrict__ idx,
                                                float *__restrict__ gate) {
  unsigned taken = 0;
  float m = 0.f, zsel = 0.f, myv = 0.f;
  int myi = 0;
  for (int r = 0; r < k; ++r) {
    float bv = -INFINITY;
    int bi = -1;
#pragma unroll
    for (int e = 0; e < EB; ++e)
      if (e < E && !(taken & (1u << e)) && (bi < 0 || v[e] > bv)) {
        bv = v[e];
        bi = e;
      }
    taken |= 1u << bi;
    if (r == 0) m = bv;
    zsel += expf(bv - m);
    if (r == li) {
      myv = bv;
      myi = bi;
    }
  }
  if (li >= k) return;
  if (gate_mode == 3 || gate_mode == 4) {
    float zt = 0.f, s1 = 0.f;
#pragma unroll
    for (int e = 0; e < EB; ++e)
      if (e < E) {
        const float u = (v[e] - m) / ENTROPY_TAU;
        const float w = expf(u);
        zt += w;
        s1 += w * u;
      }
    const float H = logf(zt) - s1 / zt;
    const int kt = H > ENTROPY_THRESHOLD ? k : k - 1;
    const float p = expf((myv - m) / ENTROPY_TAU) / zt;
    if (gate_mode == 4) {  // see wave_topk_gate
      idx[li] = li < kt ? myi : -(myi + 2);
      gate[li] = p;
    } else {
      idx[li] = li < kt ? myi : -1;
      gate[li] = li < kt ? p : 0.f;
    }
    return;
  }
  idx[li] = myi;
  if (gate_mode == 2) {
    gate[li] = 1.0f / (1.0f + expf(-myv));
  } else if (gate_mode == 1) {
    float z = 0.f;
#pragma unroll
    for (int e = 0; e < EB; ++e)
      if (e < E) z += expf(v[e] - m);
    gate[li] = expf(myv - m) / z;
  } else {
    gate[li] = expf(myv - m) / zsel;
  }
}

// Up to 32 experts: a wavefront takes 4 tokens, 16 lanes each.  Per step the
// 16 lanes of a token read 256 contiguous bytes of its row and the same 256
// bytes of every router row; the four tokens' lanes read the same router
// addresses, which one load serves, so the router weights are read once per
// four tokens.  U steps go out together.  Slice s covers steps s*ns ..
// s*ns+ns-1 of 16 x 16 bytes; the sums are reduced over the 16 lanes.
// TOPK (one slice, k <= 16): the group then adds the bias, writes the scores
// and runs top-k and the gate itself (no partials); else slice s's sums go to
// part [S][T][E].
template <typename T, int EB, bool TOPK>
__global__ __launch_bounds__(256) void router_narrow_kernel(
    const T *__restrict__ x, const T *__restrict__ Wg, int T_, int d, int E, int ns,
    float *__restrict__ part, const float *__restrict__ bias, int k, int gate_mode,
    int32_t *__restrict__ idx, float *__restrict__ gate, float *__restrict__ logits) {
  constexpr int VEC = RouterTraits<T>::VEC;
  constexpr int U = EB <= 16 ? 2 : 1;
  const int w = threadIdx.x / kWave, lane = lane_id();
  const int li = lane & 15;
  const int t = (blockIdx.x * 4 + w) * 4 + (lane >> 4);
  const int s = blockIdx.y;
  const bool tv = t < T_;
  const uint4 *xg = reinterpret_cast<const uint4 *>(x);
  const uint4 *wgg = reinterpret_cast<const uint4 *>(Wg);
  const size_t rowq = (size_t)d / VEC;
  const size_t q0 = (size_t)s * ns * 16 + li;
  float acc[EB];
#pragma unroll
  for (int e = 0; e < EB; ++e) acc[e] = 0.f;
  for (int i = 0; i < ns; i += U) {
    uint4 xv[U], wv[U][EB];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool in = i + u < ns;
      const size_t q = q0 + (size_t)(i + u) * 16;
      xv[u] = in && tv ? xg[(size_t)t * rowq + q] : make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int e = 0; e < EB; ++e)
        wv[u][e] = in && e < E ? wgg[(size_t)e * rowq + q] : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int e = 0; e < EB; ++e) acc[e] = dot16b(xv[u], wv[u][e], acc[e], T());
  }
#pragma unroll
  for (int e = 0; e < EB; ++e)
#pragma unroll
    for (int off = 8; off > 0; off >>= 1) acc[e] += __shfl_xor(acc[e], off);
  if (!tv) return;
  if constexpr (TOPK) {
#pragma unroll
    for (int e = 0; e < EB; ++e) {
      if (bias && e < E) acc[e] += bias[e];
      if (logits && e < E && (e & 15) == li) logits[(size_t)t * E + e] = acc[e];
    }
    group_topk_gate(acc, E, k, gate_mode, li, idx + (size_t)t * k, gate + (size_t)t * k);
  } else {
    float *out = part + ((size_t)s * T_ + t) * E;
#pragma unroll
    for (int e = 0; e < EB; ++e)
      if (e < E && (e & 15) == li) out[e] = acc[e];
  }
}

// Small batches with up to 32 experts: one wavefront per token, in one
// launch.  Lane l takes the 16-byte chunks l, l + 64, ... of the token's row
// and of every router row (U steps in flight), the sums are reduced over the
// 64 lanes, and the lanes then run top-k and the gate as in the kernel above
// (lane j < k writes pick j).  Against the d-split kernel plus its top-k
// launch, this saves a launch and the partial sums' round trip.
template <typename T, int EB>
__global__ __launch_bounds__(256) void router_wave_kernel(
    const T *__restrict__ x, const T *__restrict__ Wg, int T_, int d, int E,
    const float *__restrict__ bias, int k, int gate_mode, int32_t *__restrict__ idx,
    float *__restrict__ gate, float *__restrict__ logits) {
  constexpr int VEC = RouterTraits<T>::VEC;
  constexpr int U = EB <= 8 ? 4 : EB <= 16 ? 2 : 1;
  const int lane = lane_id();
  const int t = blockIdx.x * 4 + (int)threadIdx.x / kWave;
  if (t >= T_) return;  // the whole wavefront: no barrier follows
  const int rowq = d / VEC;  // a multiple of 64
  const int nq = rowq / 64;
  const uint4 *xr = reinterpret_cast<const uint4 *>(x) + (size_t)t * rowq;
  const uint4 *wgg = reinterpret_cast<const uint4 *>(Wg);
  float acc[EB];
#pragma unroll
  for (int e = 0; e < EB; ++e) acc[e] = 0.f;
  for (int i = 0; i < nq; i += U) {
    uint4 xv[U], wv[U][EB];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool in = i + u < nq;
      const int q = (i + u) * 64 + lane;
      xv[u] = in ? xr[q] : make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int e = 0; e < EB; ++e)
        wv[u][e] = in && e < E ? wgg[(size_t)e * rowq + q] : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int e = 0; e < EB; ++e) acc[e] = dot16b(xv[u], wv[u][e], acc[e], T());
  }
#pragma unroll
  for (int e = 0; e < EB; ++e)
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) acc[e] += __shfl_xor(acc[e], off);
#pragma unroll
  for (int e = 0; e < EB; ++e) {
    if (bias && e < E) acc[e] += bias[e];
    if (logits && e < E && e == lane) logits[(size_t)t * E + e] = acc[e];
  }
  group_topk_gate(acc, E, k, gate_mode, lane, idx + (size_t)t * k, gate + (size_t)t * k);
}

// Large batches with a small router (E <= 16, E * d * size <= 64 KB, k <= 16):
// the workgroup copies the router weights into LDS once and streams 16 tokens'
// rows, four per wavefront with 16 lanes each (per step 256 contiguous bytes
// of a row), RX steps in flight and the next RX issued before the current ones
// are used; the router chunks come from LDS (the four tokens' lanes read the
// same addresses).  The sums are reduced over the 16 lanes, then the group
// adds the bias, writes the scores and runs top-k and the gate.  (More steps
// in flight, or more experts per step, and the compiler's hoisting of the LDS
// reads runs out of registers.)
template <int EB> constexpr int router_rx() { return EB <= 8 ? 4 : 2; }
template <typename T, int EB>
__global__ __launch_bounds__(256, 2) void router_lds_kernel(
    const T *__restrict__ x, const T *__restrict__ Wg, int T_, int d, int E,
    const float *__restrict__ bias, int k, int gate_mode, int32_t *__restrict__ idx,
    float *__restrict__ gate, float *__restrict__ logits) {
  constexpr int VEC = RouterTraits<T>::VEC;
  constexpr int RX = router_rx<EB>();
  extern __shared__ uint4 wl[];  // [E][d / VEC]
  const int tid = threadIdx.x, w = tid / kWave, lane = lane_id();
  const int li = lane & 15;
  const int t = (blockIdx.x * 4 + w) * 4 + (lane >> 4);
  const bool tv = t < T_;
  const int rowq = d / VEC;
  const int steps = rowq / 16;  // a multiple of 2 RX
  // a token past the end reads row 0 and writes nothing
  const uint4 *xg = reinterpret_cast<const uint4 *>(x) + (size_t)(tv ? t : 0) * rowq + li;
  // start the row's first steps before the router copy
  uint4 xa[RX], xb[RX];
#pragma unroll
  for (int u = 0; u < RX; ++u) xa[u] = xg[16 * u];
  {
    const uint4 *wgg = reinterpret_cast<const uint4 *>(Wg);
    const int nq = E * rowq;  // a multiple of 256 * 8
    for (int i0 = 0; i0 < nq; i0 += 256 * 8) {
      uint4 c[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) c[j] = wgg[i0 + j * 256 + tid];
#pragma unroll
      for (int j = 0; j < 8; ++j) wl[i0 + j * 256 + tid] = c[j];
    }
  }
  __syncthreads();
  float acc[EB];
#pragma unroll
  for (int e = 0; e < EB; ++e) acc[e] = 0.f;
  // sums past E read router row E - 1 (no branch between the LDS reads) and
  // are never used
  auto use = [&](const uint4 (&xv)[RX], int j0) {
#pragma unroll
    for (int u = 0; u < RX; ++u) {
      const int q = li + 16 * (j0 + u);
#pragma unroll
      for (int e = 0; e < EB; ++e) acc[e] = dot16b(xv[u], wl[min(e, E - 1) * rowq + q], acc[e], T());
      // one step at a time: hoisting every step's LDS reads would take more
      // registers than the loads in flight leave
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
    }
  };
  // steps is a multiple of 2 RX: xb holds steps j0 + RX .., xa the next 2 RX
  for (int j0 = 0; j0 < steps; j0 += 2 * RX) {
#pragma unroll
    for (int u = 0; u < RX; ++u) xb[u] = xg[16 * (j0 + RX + u)];
    use(xa, j0);
    if (j0 + 2 * RX < steps) {
#pragma unroll
      for (int u = 0; u < RX; ++u) xa[u] = xg[16 * (j0 + 2 * RX + u)];
    }
    use(xb, j0 + RX);
  }
#pragma unroll
  for (int e = 0; e < EB; ++e)
#pragma unroll
    for (int off = 8; off > 0; off >>= 1) acc[e] += __shfl_xor(acc[e], off);
  if (!tv) return;
#pragma unroll
  for (int e = 0; e < EB; ++e) {
    if (bias && e < E) acc[e] += bias[e];
    if (logits && e < E && (e & 15) == li) logits[(size_t)t * E + e] = acc[e];
  }
  group_topk_gate(acc, E, k, gate_mode, li, idx + (size_t)t * k, gate + (size_t)t * k);
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

// The entropy-aware routing with one k for the batch ("Mixtral 8x7B model
// architecture", section 4.1, as its listing prints it: the batch's largest
// per-token k).  The top-k kernels (gate_mode 4) leave each token's last slot
// as its expert e when the token's own k is the full k, else as -(e + 2);
// one workgroup then keeps every last slot if any token takes the full k
// (its expert restored, its probability kept), else empties them all (idx
// -1, gate 0).
__global__ __launch_bounds__(1024) void entropy_batch_kernel(int32_t *__restrict__ idx,
                                                             float *__restrict__ gate, int T_,
                                                             int k) {
  int any = 0;
  for (int t = threadIdx.x; t < T_; t += 1024) any |= idx[(size_t)t * k + k - 1] >= 0;
  any = __syncthreads_or(any);
  for (int t = threadIdx.x; t < T_; t += 1024) {
    const size_t q = (size_t)t * k + k - 1;
    const int v = idx[q];
    if (any) {
      if (v < 0) idx[q] = -v - 2;
    } else {
      idx[q] = -1;
      gate[q] = 0.f;
    }
  }
}

// Feature slices for the score kernels (enough work items to fill the GPU).
// Narrow kernel: a slice is ns steps of 16 lanes x 16 bytes per token.  Tiled
// kernel: a slice is a whole number of 128-byte chunks.
struct RouterSplit {
  bool narrow;
  int S, ns;
};
RouterSplit router_split(int T, int d, int E, int esize) {
  RouterSplit r{};
  const int vec = 16 / esize;
  r.narrow = E <= 32 && d % (16 * vec) == 0;
  if (r.narrow) {
    const int steps = d / (16 * vec);               // 16-byte steps per lane over the whole row
    const long long waves_per_slice = (T + 3) / 4;  // four tokens per wave
    int S = steps;                                  // finest split: one step per lane
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

template <typename T, bool TOPK>
void launch_narrow(const RouterSplit &r, const void *x, const void *Wg, int T_, int d, int E,
                   float *part, const float *bias, int k, int gate_mode, int32_t *idx,
                   float *gate, float *logits, hipStream_t s) {
  dim3 grid((T_ + 15) / 16, r.S);
#define RN_LAUNCH(EB)                                                                          \
  hipLaunchKernelGGL((router_narrow_kernel<T, EB, TOPK>), grid, dim3(256), 0, s, (const T *)x, \
                     (const T *)Wg, T_, d, E, r.ns, part, bias, k, gate_mode, idx, gate, logits)
  if (E <= 8)
    RN_LAUNCH(8);
  else if (E <= 16)
    RN_LAUNCH(16);
  else
    RN_LAUNCH(32);
#undef RN_LAUNCH
}

template <typename T>
void launch_scores(const RouterSplit &r, const void *x, const void *Wg, int T_, int d, int E,
                   float *part, hipStream_t s) {
  if (r.narrow) {
    launch_narrow<T, false>(r, x, Wg, T_, d, E, part, nullptr, 0, 0, nullptr, nullptr, nullptr,
                            s);
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

namespace {
hipError_t launch_router_scores_topk(int dtype, const void *x, const void *Wg, const float *bias,
                                     int T, int d, int E, int k, int gate_mode, int32_t *idx,
                                     float *gate, float *logits, float *part, hipStream_t s);
}  // namespace

hipError_t launch_router(int dtype, const void *x, const void *Wg, const float *bias, int T,
                         int d, int E, int k, int gate_mode, int32_t *idx, float *gate,
                         float *logits, float *part, hipStream_t s) {
  hipError_t e = launch_router_scores_topk(dtype, x, Wg, bias, T, d, E, k, gate_mode, idx, gate,
                                           logits, part, s);
  if (e != hipSuccess || gate_mode != 4 || T == 0) return e;
  hipLaunchKernelGGL(entropy_batch_kernel, dim3(1), dim3(1024), 0, s, idx, gate, T, k);
  return hipGetLastError();
}

namespace {
// Batches up to this many tokens route with one wavefront per token.
constexpr int ROUTER_WAVE_MAX_T = 2048;

hipError_t launch_router_scores_topk(int dtype, const void *x, const void *Wg, const float *bias,
                                     int T, int d, int E, int k, int gate_mode, int32_t *idx,
                                     float *gate, float *logits, float *part, hipStream_t s) {
  const int es = dtype == 1 ? 2 : 4;
  const RouterSplit r = router_split(T, d, E, es);
  const size_t wl_bytes = (size_t)E * d * es;
  const int rx = E <= 8 ? router_rx<8>() : router_rx<16>();
  if (E <= 16 && k <= 16 && wl_bytes <= 65536 && T >= 4096 &&
      d % (16 * (16 / es) * 2 * rx) == 0 && (wl_bytes / 16) % (256 * 8) == 0) {
    // many tokens, a router that fits LDS: one kernel, router weights in LDS
#define RL_LAUNCH(TT, EB)                                                                     \
  hipLaunchKernelGGL((router_lds_kernel<TT, EB>), dim3((T + 15) / 16), dim3(256), wl_bytes, s, \
                     (const TT *)x, (const TT *)Wg, T, d, E, bias, k, gate_mode, idx, gate, logits)
    if (dtype == 1) {
      if (E <= 8) RL_LAUNCH(bf16_t, 8); else RL_LAUNCH(bf16_t, 16);
    } else {
      if (E <= 8) RL_LAUNCH(float, 8); else RL_LAUNCH(float, 16);
    }
#undef RL_LAUNCH
    return hipGetLastError();
  }
  if (E <= 32 && k <= 16 && T <= ROUTER_WAVE_MAX_T && (d / (16 / es)) % 64 == 0) {
    // small batches: one wavefront per token, top-k in the same launch
#define RW_LAUNCH(TT, EB)                                                                       \
  hipLaunchKernelGGL((router_wave_kernel<TT, EB>), dim3((T + 3) / 4), dim3(256), 0, s,          \
                     (const TT *)x, (const TT *)Wg, T, d, E, bias, k, gate_mode, idx, gate, logits)
    if (dtype == 1) {
      if (E <= 8) RW_LAUNCH(bf16_t, 8); else if (E <= 16) RW_LAUNCH(bf16_t, 16); else RW_LAUNCH(bf16_t, 32);
    } else {
      if (E <= 8) RW_LAUNCH(float, 8); else if (E <= 16) RW_LAUNCH(float, 16); else RW_LAUNCH(float, 32);
    }
#undef RW_LAUNCH
    return hipGetLastError();
  }
  if (r.narrow && r.S == 1 && k <= 16) {
    // whole rows per wave: top-k and gate in the score kernel
    if (dtype == 1)
      launch_narrow<bf16_t, true>(r, x, Wg, T, d, E, nullptr, bias, k, gate_mode, idx, gate,
                                  logits, s);
    else
      launch_narrow<float, true>(r, x, Wg, T, d, E, nullptr, bias, k, gate_mode, idx, gate,
                                 logits, s);
    return hipGetLastError();
  }
  if (dtype == 1)
    launch_scores<bf16_t>(r, x, Wg, T, d, E, part, s);
  else
    launch_scores<float>(r, x, Wg, T, d, E, part, s);
  hipLaunchKernelGGL(router_topk_kernel, dim3((T + 3) / 4), dim3(256), 0, s, part, r.S, bias, T,
                     E, k, gate_mode, idx, gate, logits);
  return hipGetLastError();
}

}  // namespace
}  // namespace moe
