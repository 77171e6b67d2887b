// Weight-streaming grouped GEMMs for few rows per expert (decode-sized batches).
//
// Same operations as the tiled grouped GEMMs ("Mistral 8x7B SMoE architecture
// deep dive", section 3.1; "Mixtral and MoE architecture", FeedForward
// listing):
//   SWIGLU = true : H = SiLU(A W1_e^T) * (A W3_e^T)   A rows gathered from x by the permutation
//   SWIGLU = false: Y = A W2_e^T                       A = H, rows already grouped by expert
// but shaped for the regime where every weight element is used by only a few
// rows, so the layer is bound by streaming the weights of the experts that were
// hit.  A workgroup owns one (active expert, 16 output columns) pair and reads
// that weight slice exactly once: its eight wavefronts split K, each loads
// weight and activation fragments straight into registers (16 contiguous
// bytes per lane, several K chunks in flight) and runs 16x16x32 bf16 MFMAs on
// up to MB row blocks of 16; the partial sums are reduced across the waves in
// LDS, where the SiLU * mul epilogue is applied.  Experts with more than 16*MB
// rows loop over row groups (the weight slice is then read again).
//
// MFMA 16x16x32 operand layout: lane l holds A[m = l%16][k = (l/16)*8 .. +8]
// and B[k = (l/16)*8 .. +8][n = l%16]; the result holds C[m = (l/16)*4 + i][n =
// l%16] in element i.  Weights are [N][K] (K-contiguous), so B = W^T is read
// as 16 consecutive bytes of one weight row per lane.
#include <type_traits>
#include "common.h"
#include "kernels.h"
#include "route_block.h"

namespace moe {

namespace {

typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f4_v;

constexpr int SK_WAVES = 8;
constexpr int SK_THREADS = SK_WAVES * kWave;
constexpr int SK_NB = 16;  // output columns per workgroup
constexpr int SK_KC = 32;  // K per MFMA
// K chunks in flight per wave: more for the single-matrix (down) projection
template <bool SWIGLU> struct SkInFlight { static constexpr int U = SWIGLU ? 4 : 8; };

__device__ __forceinline__ uint4 ldg16(const bf16_t *p) {
  return *reinterpret_cast<const uint4 *>(p);
}

__device__ __forceinline__ f4_v mfma16(const uint4 &a, const uint4 &b, const f4_v &c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_v, a),
                                                 __builtin_bit_cast(bf16x8_v, b), c, 0, 0, 0);
}

template <bool SWIGLU, int MB>
__global__ __launch_bounds__(SK_THREADS) void skinny_gemm_kernel(
    const bf16_t *__restrict__ A, const int32_t *__restrict__ perm, int kslots,
    const bf16_t *__restrict__ B1, const bf16_t *__restrict__ B3, void *__restrict__ C,
    const int32_t *__restrict__ seg_off, const int32_t *__restrict__ active,
    const int32_t *__restrict__ nactive, int N, int K, int act) {
  constexpr int NW = SWIGLU ? 2 : 1;  // weight matrices per output
  __shared__ float red[SK_WAVES][NW * MB][4][kWave];

  const int ntn = N / SK_NB;
  const int a_idx = blockIdx.x / ntn;
  if (a_idx >= nactive[0]) return;
  const int e = active[a_idx];
  const int n0 = (blockIdx.x % ntn) * SK_NB;
  const int s0 = seg_off[e], cnt = seg_off[e + 1] - s0;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave), lane = lane_id();
  const int kper = K / SK_WAVES;  // multiple of SK_KC (checked by the host)
  const int kbeg = wave * kper + (lane >> 4) * 8;
  const int nch = kper / SK_KC;
  const size_t wrow = ((size_t)e * N + n0 + (lane & 15)) * K + kbeg;
  const bf16_t *b1p = B1 + wrow;
  const bf16_t *b3p = SWIGLU ? B3 + wrow : b1p;

  for (int rg = 0; rg < cnt; rg += 16 * MB) {
    const bf16_t *ap[MB];
#pragma unroll
    for (int rb = 0; rb < MB; ++rb) {
      const int r = min(rg + rb * 16 + (lane & 15), cnt - 1);  // rows past the end: not stored
      const int src = perm ? perm[s0 + r] / kslots : s0 + r;
      ap[rb] = A + (size_t)src * K + kbeg;
    }
    f4_v acc[NW][MB];
#pragma unroll
    for (int w = 0; w < NW; ++w)
#pragma unroll
      for (int rb = 0; rb < MB; ++rb) acc[w][rb] = f4_v{0.f, 0.f, 0.f, 0.f};

    constexpr int U = SkInFlight<SWIGLU>::U;
    for (int c = 0; c < nch; c += U) {
      uint4 bw[U][NW], av[U][MB];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int cc = min(c + u, nch - 1);  // clamped reload past the end: never used
        bw[u][0] = ldg16(b1p + cc * SK_KC);
        if (SWIGLU) bw[u][NW - 1] = ldg16(b3p + cc * SK_KC);
#pragma unroll
        for (int rb = 0; rb < MB; ++rb) av[u][rb] = ldg16(ap[rb] + cc * SK_KC);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (c + u < nch) {
#pragma unroll
          for (int rb = 0; rb < MB; ++rb)
#pragma unroll
            for (int w = 0; w < NW; ++w) acc[w][rb] = mfma16(av[u][rb], bw[u][w], acc[w][rb]);
        }
      }
    }

    // cross-wave reduction and epilogue
#pragma unroll
    for (int w = 0; w < NW; ++w)
#pragma unroll
      for (int rb = 0; rb < MB; ++rb)
#pragma unroll
        for (int i = 0; i < 4; ++i) red[wave][w * MB + rb][i][lane] = acc[w][rb][i];
    __syncthreads();
    for (int o = tid; o < MB * 4 * kWave; o += SK_THREADS) {
      const int rb = o / (4 * kWave), i = (o / kWave) % 4, l = o % kWave;
      const int r = rg + rb * 16 + (l >> 4) * 4 + i;
      if (r < cnt) {
        float s[NW];
#pragma unroll
        for (int w = 0; w < NW; ++w) {
          float t = 0.f;
#pragma unroll
          for (int v = 0; v < SK_WAVES; ++v) t += red[v][w * MB + rb][i][l];
          s[w] = t;
        }
        const size_t out = (size_t)(s0 + r) * N + n0 + (l & 15);
        if (SWIGLU)
          reinterpret_cast<bf16_t *>(C)[out] = f32_to_bf16(gated(s[0], s[NW - 1], act));
        else
          reinterpret_cast<float *>(C)[out] = s[0];
      }
    }
    __syncthreads();
  }
}

template <bool SWIGLU>
hipError_t launch_mb(int mb, int act, const void *A, const int32_t *perm, int kslots,
                     const void *B1, const void *B3, void *C, const int32_t *seg_off,
                     const int32_t *active, const int32_t *nactive, int G, int N, int K,
                     hipStream_t s) {
  dim3 grid(G * (N / SK_NB));
  const bf16_t *a = (const bf16_t *)A, *b1 = (const bf16_t *)B1, *b3 = (const bf16_t *)B3;
  if (mb <= 1)
    hipLaunchKernelGGL((skinny_gemm_kernel<SWIGLU, 1>), grid, dim3(SK_THREADS), 0, s, a, perm,
                       kslots, b1, b3, C, seg_off, active, nactive, N, K, act);
  else if (mb == 2)
    hipLaunchKernelGGL((skinny_gemm_kernel<SWIGLU, 2>), grid, dim3(SK_THREADS), 0, s, a, perm,
                       kslots, b1, b3, C, seg_off, active, nactive, N, K, act);
  else
    hipLaunchKernelGGL((skinny_gemm_kernel<SWIGLU, 4>), grid, dim3(SK_THREADS), 0, s, a, perm,
                       kslots, b1, b3, C, seg_off, active, nactive, N, K, act);
  return hipGetLastError();
}


// ---------------------------------------------------------------------------
// Vector-ALU weight streaming for experts that hold one to four rows (decode
// steps).  Each wavefront instruction reads 1 KB of ONE weight row -- eight
// whole 128-byte lines -- with a non-temporal load (the weights are read once),
// and v_dot2_f32_bf16 multiplies it with the matching slice of the expert's
// rows, which each lane keeps in registers for the whole workgroup.
//  gemv_kernel             : up to four rows; the four wavefronts split K and a
//                            workgroup walks its columns CB at a time with the
//                            next group's weights in flight while the current
//                            one is reduced (lanes by shuffles, wavefronts
//                            through LDS in a fixed order)
//  gemv_swiglu_wave_kernel : one token's SwiGLU projection after routing it,
//                            every wavefront on its own columns over all of K
//  gemv_down_token_kernel  : one token's down projection, a workgroup covering
//                            a column block of every active expert, with the
//                            combine formed in LDS
// ---------------------------------------------------------------------------
constexpr int GV_WAVES = 4;
constexpr int GV_THREADS = GV_WAVES * kWave;
constexpr int GV_CHUNK = 512;  // K elements per wavefront instruction (1 KB of bf16)

typedef unsigned int gv_u4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ldg16_stream(const bf16_t *p) {
  const gv_u4 v = __builtin_nontemporal_load(reinterpret_cast<const gv_u4 *>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
// Workgroup barrier that waits only for this wave's LDS traffic: the weight
// loads of the next group stay in flight (a __syncthreads() would wait for
// every outstanding load of the wave first).
__device__ __forceinline__ void lds_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}
__device__ __forceinline__ float dot8_bf16(const uint4 &a, const uint4 &b, float acc) {
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

// FP8 (E4M3) weights: 8 bytes (8 weights) per lane per instruction; the
// conversion to bf16 is exact, so the products are those of the dequantized
// weights up to the per-expert scale, applied to the reduced sums.
typedef unsigned int gv_u2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint2 ldg8_stream(const uint8_t *p) {
  const gv_u2 v = __builtin_nontemporal_load(reinterpret_cast<const gv_u2 *>(p));
  return make_uint2(v.x, v.y);
}
__device__ __forceinline__ uint4 gv_load(const bf16_t *p) { return ldg16_stream(p); }
__device__ __forceinline__ uint2 gv_load(const uint8_t *p) { return ldg8_stream(p); }
__device__ __forceinline__ float gv_dot(const uint4 &a, const uint4 &b, float acc) {
  return dot8_bf16(a, b, acc);
}
__device__ __forceinline__ float gv_dot(const uint4 &a, const uint2 &b, float acc) {
  // E4M3 -> bf16 is exact (3 mantissa bits into 7), two codes per conversion
  // (gfx950's scaled conversion with scale 1), then the same dot2 as the bf16
  // weights: four conversions and four dot2 per 8 weights
  const bf16x2_v w01 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(b.x, 1.0f, false);
  const bf16x2_v w23 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(b.x, 1.0f, true);
  const bf16x2_v w45 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(b.y, 1.0f, false);
  const bf16x2_v w67 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(b.y, 1.0f, true);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_v, a.x), w01, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_v, a.y), w23, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_v, a.z), w45, acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_v, a.w), w67, acc, false);
  return acc;
}

// Columns per group: the largest power of two that keeps about 16 weight
// loads (16 KB of bf16, 8 KB of FP8) per wavefront in flight (more columns
// per group were slower for FP8: the per-group reductions grow with them).
constexpr int gv_cb(int loads_per_col) {
  int cb = 1;
  while (cb * 2 * loads_per_col <= 16) cb *= 2;
  return cb;
}

// KC: 1 KB chunks per wavefront (K = GV_WAVES * KC * GV_CHUNK); R: rows per
// pass; CB: columns per group.  The workgroup owns columns c0 .. c0+cpw-1 of
// active expert blockIdx.x / (N / cpw).
//
// COMBINE (down projection): the gate-weighted combine rides along.  Outputs
// go to Yp with device-scope stores; the workgroup then counts itself in on
// its column block (cm.cnt, zero before the launch), and the last of the
// block's active experts to finish forms y[t][c] = sum_j gate[t][j] *
// Yp[inv[t*k+j]][c] for all T tokens and its columns, in the combine kernel's
// order and arithmetic, and clears the counter.
struct GemvCombine {
  const int32_t *inv;
  const float *gate;
  int T, k;
  bf16_t *y;
  int32_t *cnt;
};
// ROUTE (SwiGLU, one token): the workgroup routes the token itself before it
// streams weights.  The router scores come from a fixed split of the features
// (thread i: the 16-byte chunks i, i + 256, ...; lanes then waves summed in a
// fixed order), so every workgroup computes the same scores, top-k, gates and
// grouping; workgroup 0 also writes them out for the launches that follow.
struct RouteLds {
  float red[GV_WAVES][64];
  float logit[64], selv[64], gate[64];
  int32_t seli[64], idx[64], counts[64], perm[64], inv[64];
  int32_t offsets[65], mt0[65], mt1[65], active[65], shseg[8];
};
__device__ __forceinline__ void route_token(const bf16_t *__restrict__ x, int d,
                                            const DecodeRoute &rt, RouteLds &rs) {
  const int tid = threadIdx.x, wave = tid / kWave, lane = lane_id();
  const int E = rt.E;
  const uint4 *xq = reinterpret_cast<const uint4 *>(x);
  const uint4 *wq = reinterpret_cast<const uint4 *>(rt.Wg);
  const int rowq = d / 8;               // 16-byte chunks per row
  const int nj = d / (GV_THREADS * 8);  // chunks per thread (d is a multiple of 2048)
  constexpr int JU = 4;  // chunks whose loads go out together (one round trip up to d = 8192)
  for (int e0 = 0; e0 < E; e0 += 8) {
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.f;
    for (int j0 = 0; j0 < nj; j0 += JU) {
      uint4 xv[JU], wv[JU][8];
#pragma unroll
      for (int u = 0; u < JU; ++u) {
        const int q = tid + GV_THREADS * (j0 + u);
        const bool in = j0 + u < nj;
        xv[u] = in ? xq[q] : make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < 8; ++i)
          wv[u][i] = in && e0 + i < E ? wq[(size_t)(e0 + i) * rowq + q] : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int u = 0; u < JU; ++u)
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = dot8_bf16(xv[u], wv[u][i], acc[i]);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float v = acc[i];
#pragma unroll
      for (int off = kWave / 2; off > 0; off >>= 1) v += __shfl_xor(v, off);
      if (lane == 0 && e0 + i < E) rs.red[wave][e0 + i] = v;
    }
  }
  __syncthreads();
  if (wave == 0) {
    float v[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
    if (lane < E) {
      float l = rs.red[0][lane];
#pragma unroll
      for (int w = 1; w < GV_WAVES; ++w) l += rs.red[w][lane];
      if (rt.bias) l += rt.bias[lane];
      rs.logit[lane] = l;
      v[0] = l;
    }
    wave_topk_gate(v, E, rt.k, rt.gate_mode, rs.selv, rs.seli, rs.idx, rs.gate);
    // lane j wrote idx[j] and reads it back as pair j's expert
    wave_group_pairs(rs.idx, 1, E, rt.k, rt.capacity, rt.bm0, rt.bm1,
                     RouteOut{rs.counts, rs.offsets, rs.perm, rs.inv, rs.mt0, rs.mt1, rs.shseg,
                              rs.active});
  }
  __syncthreads();
  if (blockIdx.x == 0) {
    const int k = rt.k, kept = rs.offsets[E], na = rs.active[E];
    for (int i = tid; i < rt.nzero; i += GV_THREADS) rt.zero[i] = 0;
    if (tid < E) {
      rt.logits[tid] = rs.logit[tid];
      rt.counts[tid] = rs.counts[tid];
    }
    if (tid <= E) {
      rt.offsets[tid] = rs.offsets[tid];
      rt.mtiles0[tid] = rs.mt0[tid];
      rt.mtiles1[tid] = rs.mt1[tid];
    }
    if (tid < k) {
      rt.idx[tid] = rs.idx[tid];
      rt.gate[tid] = rs.gate[tid];
      rt.inv[tid] = rs.inv[tid];
    }
    if (tid < kept) rt.perm[tid] = rs.perm[tid];
    if (tid < na) rt.active[tid] = rs.active[tid];
    if (tid == 0) rt.active[E] = na;
    if (tid < 8) rt.shared_seg[tid] = rs.shseg[tid];
  }
}

//
// W8: FP8 weights (uint8 E4M3 codes) with per-expert scales sc1 (W1 or W2) and
// sc3 (W3).
template <bool SWIGLU, int R, int KC, bool COMBINE = false, bool W8 = false,
          bool ROUTE = false>
__global__ __launch_bounds__(GV_THREADS) void gemv_kernel(
    const bf16_t *__restrict__ A, const int32_t *__restrict__ perm, int kslots,
    const void *__restrict__ B1v, const void *__restrict__ B3v, void *__restrict__ C,
    const int32_t *__restrict__ seg_off, const int32_t *__restrict__ active,
    const int32_t *__restrict__ nactive, int N, int K, int cpw, int act, GemvCombine cm,
    const float *__restrict__ sc1, const float *__restrict__ sc3, DecodeRoute rt) {
  static_assert(!(SWIGLU && COMBINE), "the combine follows the down projection");
  static_assert(SWIGLU || !ROUTE, "a token is routed before its SwiGLU projection");
  using WT = typename std::conditional<W8, uint8_t, bf16_t>::type;  // weight element
  using WV = typename std::conditional<W8, uint2, uint4>::type;     // 8 weights
  constexpr int NW = SWIGLU ? 2 : 1;
  constexpr int CB = gv_cb(NW * KC);
  __shared__ float red[2][GV_WAVES][CB][NW][R];
  __shared__ int arrived;

  __shared__ typename std::conditional<ROUTE, RouteLds, char>::type rsh;
  if constexpr (ROUTE) {
    route_token(A, K, rt, rsh);
    seg_off = rsh.offsets;
    active = rsh.active;
    nactive = rsh.active + rt.E;
    perm = rsh.perm;
  }
  const int nblk = N / cpw;
  const int a_idx = blockIdx.x / nblk;
  if (COMBINE && nactive[0] == 0) {
    // every pair dropped: y is zero
    if (a_idx == 0)
      for (int i = threadIdx.x; i < cm.T * cpw; i += GV_THREADS)
        cm.y[(size_t)(i / cpw) * N + (blockIdx.x % nblk) * cpw + i % cpw] = 0;
    return;
  }
  if (a_idx >= nactive[0]) return;
  const int e = active[a_idx];
  const int c0 = (blockIdx.x % nblk) * cpw;
  const int s0 = seg_off[e], cnt = seg_off[e + 1] - s0;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave), lane = lane_id();
  const int kl = wave * KC * GV_CHUNK + lane * 8;  // first K element of the lane
  const WT *w1 = reinterpret_cast<const WT *>(B1v) + (size_t)e * N * K + kl;
  const WT *w3 = SWIGLU ? reinterpret_cast<const WT *>(B3v) + (size_t)e * N * K + kl : w1;
  const int ngroups = cpw / CB;

  for (int rg = 0; rg < cnt; rg += R) {
    uint4 xa[R][KC];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int row = min(rg + r, cnt - 1);  // rows past the end: duplicates, not stored
      const int src = perm ? perm[s0 + row] / kslots : s0 + row;
      const bf16_t *ap = A + (size_t)src * K + kl;
#pragma unroll
      for (int i = 0; i < KC; ++i) xa[r][i] = *reinterpret_cast<const uint4 *>(ap + i * GV_CHUNK);
    }
    WV wa[CB][NW][KC], wb[CB][NW][KC];  // two groups of weights in flight
    // Workgroups start at different groups of their columns: workgroups a
    // fixed distance apart would otherwise all read the same offsets of their
    // blocks at the same time and crowd a few HBM channels.
    const int rot = blockIdx.x % ngroups;
    auto col_of = [&](int g) { return c0 + ((g + rot) % ngroups) * CB; };
    auto load = [&](WV (&dst)[CB][NW][KC], int g) {
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) {
        const size_t ro = (size_t)(col_of(g) + cb) * K;
#pragma unroll
        for (int i = 0; i < KC; ++i) {
          dst[cb][0][i] = gv_load(w1 + ro + i * GV_CHUNK);
          if (SWIGLU) dst[cb][NW - 1][i] = gv_load(w3 + ro + i * GV_CHUNK);
        }
      }
    };
    // dot products of one group, reduced over the lanes, then over the waves
    // (red[rb]: the two groups in flight use different halves)
    auto compute = [&](const WV (&wv)[CB][NW][KC], int g, int rb) {
      float acc[CB][NW][R];
#pragma unroll
      for (int cb = 0; cb < CB; ++cb)
#pragma unroll
        for (int m = 0; m < NW; ++m)
#pragma unroll
          for (int r = 0; r < R; ++r) {
            float t = 0.f;
#pragma unroll
            for (int i = 0; i < KC; ++i) t = gv_dot(xa[r][i], wv[cb][m][i], t);
#pragma unroll
            for (int off = kWave / 2; off > 0; off >>= 1) t += __shfl_xor(t, off);
            acc[cb][m][r] = t;
          }
      if (lane == 0) {
#pragma unroll
        for (int cb = 0; cb < CB; ++cb)
#pragma unroll
          for (int m = 0; m < NW; ++m)
#pragma unroll
            for (int r = 0; r < R; ++r) red[rb][wave][cb][m][r] = acc[cb][m][r];
      }
      lds_barrier();
      if (tid < CB * R) {
        const int cb = tid / R, r = tid % R;
        if (rg + r < cnt) {
          float v[NW];
#pragma unroll
          for (int m = 0; m < NW; ++m) {
            float t = 0.f;
#pragma unroll
            for (int w = 0; w < GV_WAVES; ++w) t += red[rb][w][cb][m][r];
            v[m] = t;
          }
          if (W8) {  // the experts' scales
            v[0] *= sc1[e];
            if (SWIGLU) v[NW - 1] *= sc3[e];
          }
          const size_t out = (size_t)(s0 + rg + r) * N + col_of(g) + cb;
          if (SWIGLU)
            reinterpret_cast<bf16_t *>(C)[out] = f32_to_bf16(gated(v[0], v[NW - 1], act));
          else if (COMBINE)
            __hip_atomic_store(reinterpret_cast<float *>(C) + out, v[0], __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
          else
            reinterpret_cast<float *>(C)[out] = v[0];
        }
      }
      // red[rb] is written again two groups later, after the next barrier
    };
    // ngroups is even (the host makes cpw a multiple of 2 CB): two groups in
    // flight, no conditional loads inside the loop
    load(wa, 0);
    load(wb, 1);
    int g = 0;
    for (; g + 2 < ngroups; g += 2) {
      compute(wa, g, 0);
      load(wa, g + 2);
      compute(wb, g + 1, 1);
      load(wb, g + 3);
    }
    compute(wa, g, 0);
    compute(wb, g + 1, 1);
    lds_barrier();
  }
  if constexpr (COMBINE) {
    __builtin_amdgcn_s_waitcnt(0);  // this wave's outputs are in memory
    __syncthreads();
    const int blk = blockIdx.x % nblk;
    if (tid == 0)
      arrived = __hip_atomic_fetch_add(&cm.cnt[blk], 1, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    if (arrived != nactive[0] - 1) return;
    const float *Yp = reinterpret_cast<const float *>(C);
    for (int i = tid; i < cm.T * cpw; i += GV_THREADS) {
      const int t = i / cpw, c = c0 + i % cpw;
      float acc = 0.f;
      for (int j = 0; j < cm.k; ++j) {
        const int slot = cm.inv[(size_t)t * cm.k + j];
        if (slot < 0) continue;
        const float v = __hip_atomic_load(Yp + (size_t)slot * N + c, __ATOMIC_RELAXED,
                                          __HIP_MEMORY_SCOPE_AGENT);
        acc = fmaf(cm.gate[(size_t)t * cm.k + j], v, acc);
      }
      cm.y[(size_t)t * N + c] = f32_to_bf16(acc);
    }
    if (tid == 0)
      __hip_atomic_store(&cm.cnt[blk], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// One token's down projection with the combine inside: a workgroup owns a
// block of cw <= GT_COLS output columns for EVERY active expert, so the
// token's k outputs of a column meet in its LDS and y is formed there (no
// partial outputs leave the workgroup, no arrival counting).  The workgroup
// walks (active expert, column group) units with two groups of weights in
// flight across expert boundaries; the next expert's row of H is loaded with
// the first weights of that expert.  Per column the arithmetic is that of
// gemv_kernel (lanes by the butterfly, then waves in order, then the FP8
// scale) followed by the combine kernel's (fmaf over j ascending, dropped
// pairs skipped).
constexpr int GT_COLS = 64, GT_SLOTS = 64;
template <int KC, bool W8>
__global__ __launch_bounds__(GV_THREADS) void gemv_down_token_kernel(
    const bf16_t *__restrict__ H, const void *__restrict__ W2v,
    const int32_t *__restrict__ seg_off, const int32_t *__restrict__ active,
    const int32_t *__restrict__ nactive, int N, int K, int cw, const int32_t *__restrict__ inv,
    const float *__restrict__ gate, int k, bf16_t *__restrict__ y, const float *__restrict__ sc) {
  using WT = typename std::conditional<W8, uint8_t, bf16_t>::type;
  using WV = typename std::conditional<W8, uint2, uint4>::type;
  constexpr int CB = gv_cb(KC);
  __shared__ float red[2][GV_WAVES][CB];
  __shared__ float ys[GT_SLOTS][GT_COLS];  // [slot of H][column of the block]
  __shared__ int ex[GT_SLOTS], slot[GT_SLOTS];
  __shared__ float scl[GT_SLOTS];

  const int tid = threadIdx.x;
  const int c0 = blockIdx.x * cw;
  const int na = nactive[0];
  if (na == 0) {  // every pair dropped: y is zero
    for (int i = tid; i < cw; i += GV_THREADS) y[c0 + i] = 0;
    return;
  }
  if (tid < na) {
    const int e = active[tid];
    ex[tid] = e;
    slot[tid] = seg_off[e];
    scl[tid] = W8 ? sc[e] : 1.f;
  }
  __syncthreads();
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave), lane = lane_id();
  const int kl = wave * KC * GV_CHUNK + lane * 8;
  const WT *w0 = reinterpret_cast<const WT *>(W2v) + kl;
  const int ngroups = cw / CB;  // even
  const int units = na * ngroups;
  const int rot = blockIdx.x % ngroups;  // see gemv_kernel
  auto col_of = [&](int g) { return ((g + rot) % ngroups) * CB; };  // inside the block
  auto load = [&](WV (&dst)[CB][KC], int u) {
    const int a = u / ngroups;
    const WT *w = w0 + (size_t)ex[a] * N * K;
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      const size_t ro = (size_t)(c0 + col_of(u % ngroups) + cb) * K;
#pragma unroll
      for (int i = 0; i < KC; ++i) dst[cb][i] = gv_load(w + ro + i * GV_CHUNK);
    }
  };
  uint4 xa[KC], xn[KC];
  auto load_x = [&](uint4 (&dst)[KC], int a) {
    const bf16_t *ap = H + (size_t)slot[a] * K + kl;
#pragma unroll
    for (int i = 0; i < KC; ++i) dst[i] = *reinterpret_cast<const uint4 *>(ap + i * GV_CHUNK);
  };
  auto compute = [&](const WV (&wv)[CB][KC], int u, int rb) {
    float acc[CB];
#pragma unroll
    for (int cb = 0; cb < CB; ++cb) {
      float t = 0.f;
#pragma unroll
      for (int i = 0; i < KC; ++i) t = gv_dot(xa[i], wv[cb][i], t);
#pragma unroll
      for (int off = kWave / 2; off > 0; off >>= 1) t += __shfl_xor(t, off);
      acc[cb] = t;
    }
    if (lane == 0) {
#pragma unroll
      for (int cb = 0; cb < CB; ++cb) red[rb][wave][cb] = acc[cb];
    }
    lds_barrier();
    if (tid < CB) {
      const int a = u / ngroups;
      float v = 0.f;
#pragma unroll
      for (int w = 0; w < GV_WAVES; ++w) v += red[rb][w][tid];
      if (W8) v *= scl[a];
      ys[slot[a]][col_of(u % ngroups) + tid] = v;
    }
    // red[rb] is written again two units later, after the next barrier
  };
  WV wa[CB][KC], wb[CB][KC];
  load_x(xa, 0);
  load(wa, 0);
  load(wb, 1);
  int u = 0;
  for (; u + 2 < units; u += 2) {
    // units come in pairs of one expert (ngroups is even)
    if (u > 0 && u % ngroups == 0) {
#pragma unroll
      for (int i = 0; i < KC; ++i) xa[i] = xn[i];
    }
    compute(wa, u, 0);
    if ((u + 2) % ngroups == 0) load_x(xn, (u + 2) / ngroups);
    load(wa, u + 2);
    compute(wb, u + 1, 1);
    load(wb, u + 3);
  }
  if (u > 0 && u % ngroups == 0) {
#pragma unroll
    for (int i = 0; i < KC; ++i) xa[i] = xn[i];
  }
  compute(wa, u, 0);
  compute(wb, u + 1, 1);
  __syncthreads();
  for (int c = tid; c < cw; c += GV_THREADS) {
    float acc = 0.f;
    for (int j = 0; j < k; ++j) {
      const int s = inv[j];
      if (s < 0) continue;
      acc = fmaf(gate[j], ys[s][c], acc);
    }
    y[c0 + c] = f32_to_bf16(acc);
  }
}

// One token's SwiGLU projection (K = KF * 512) after the routing prologue,
// every wavefront on its own run of the workgroup's columns: the 64 lanes
// split K in pieces of 8 weights of KF chunks per row and reduce by the
// butterfly, with two columns' W1 and W3 rows in flight.  No wavefront waits
// for another (gemv_kernel's cross-wave reduction puts a barrier between a
// group's data and the next group's loads).  W8: FP8 codes with the
// per-expert scales applied to the reduced sums.
template <int KF, bool W8>
__global__ __launch_bounds__(GV_THREADS) void gemv_swiglu_wave_kernel(
    const bf16_t *__restrict__ x, const void *__restrict__ W1v, const void *__restrict__ W3v,
    bf16_t *__restrict__ H, int N, int K, int cpw, int act, DecodeRoute rt,
    const float *__restrict__ sc1, const float *__restrict__ sc3) {
  using WT = typename std::conditional<W8, uint8_t, bf16_t>::type;
  using WV = typename std::conditional<W8, uint2, uint4>::type;
  __shared__ RouteLds rsh;
  route_token(x, K, rt, rsh);
  const int nblk = N / cpw;
  const int a_idx = blockIdx.x / nblk;
  if (a_idx >= rsh.active[rt.E]) return;
  const int e = rsh.active[a_idx];
  const int s0 = rsh.offsets[e];
  const int tid = threadIdx.x, wave = tid / kWave, lane = lane_id();
  const int ncw = cpw / GV_WAVES;
  const int c0 = (blockIdx.x % nblk) * cpw + wave * ncw;
  uint4 xa[KF];
  const bf16_t *xp = x + (size_t)(rsh.perm[s0] / rt.k) * K + lane * 8;
#pragma unroll
  for (int i = 0; i < KF; ++i) xa[i] = *reinterpret_cast<const uint4 *>(xp + i * GV_CHUNK);
  const WT *w1 = reinterpret_cast<const WT *>(W1v) + (size_t)e * N * K + lane * 8;
  const WT *w3 = reinterpret_cast<const WT *>(W3v) + (size_t)e * N * K + lane * 8;
  const int rot = (blockIdx.x + wave) % ncw;  // spread the workgroups over HBM channels
  auto col = [&](int j) { return c0 + (j + rot) % ncw; };
  auto load = [&](WV (&dst)[2][KF], int j) {
    const size_t ro = (size_t)col(j) * K;
#pragma unroll
    for (int i = 0; i < KF; ++i) {
      dst[0][i] = gv_load(w1 + ro + i * GV_CHUNK);
      dst[1][i] = gv_load(w3 + ro + i * GV_CHUNK);
    }
  };
  auto compute = [&](const WV (&w)[2][KF], int j) {
    float g = 0.f, u = 0.f;
#pragma unroll
    for (int i = 0; i < KF; ++i) {
      g = gv_dot(xa[i], w[0][i], g);
      u = gv_dot(xa[i], w[1][i], u);
    }
#pragma unroll
    for (int off = kWave / 2; off > 0; off >>= 1) {
      g += __shfl_xor(g, off);
      u += __shfl_xor(u, off);
    }
    if (W8) {
      g *= sc1[e];
      u *= sc3[e];
    }
    if (lane == 0) H[(size_t)s0 * N + col(j)] = f32_to_bf16(gated(g, u, act));
  };
  WV wa[2][KF], wb[2][KF];
  load(wa, 0);
  load(wb, 1);
  int j = 0;
  for (; j + 2 < ncw; j += 2) {  // ncw is even
    compute(wa, j);
    load(wa, j + 2);
    compute(wb, j + 1);
    load(wb, j + 3);
  }
  compute(wa, j);
  compute(wb, j + 1);
}

// ---------------------------------------------------------------------------
// Weight streaming for [K][N] expert weights (in x out: the layer computes
// rows of A W), up to R rows per pass.  A workgroup owns one (active expert,
// block of CW output columns) pair and reads that weight slice once; its four
// wavefronts split K.  Lane l covers columns c0 + 8 * (l % LPR) .. + 7 (LPR =
// CW / 8 lanes per k-row); the KG = 64 / LPR lane groups of a wavefront take
// the consecutive 8-row pieces of a block of 8 * KG k-rows, so one
// instruction reads KG k-row segments of CW * 2 bytes that lie within 8 * KG
// rows of each other, and one 16-byte load of each row's activations serves a
// lane's eight k-rows.  The products are summed in fp32 per column; lanes that share
// columns are then reduced by the butterfly and the wavefronts through LDS,
// both in a fixed order.
// ---------------------------------------------------------------------------
// ROUTE (SwiGLU, one token): the workgroup routes the token itself first, as
// gemv_kernel's ROUTE variant does.
template <bool SWIGLU, int R, int CW, bool ROUTE = false>
__global__ __launch_bounds__(GV_THREADS) void gemv_t_kernel(
    const bf16_t *__restrict__ A, const int32_t *__restrict__ perm, int kslots,
    const bf16_t *__restrict__ B1, const bf16_t *__restrict__ B3, void *__restrict__ C,
    const int32_t *__restrict__ seg_off, const int32_t *__restrict__ active,
    const int32_t *__restrict__ nactive, int N, int K, int act, size_t plane, DecodeRoute rt) {
  static_assert(SWIGLU || !ROUTE, "a token is routed before its SwiGLU projection");
  constexpr int NW = SWIGLU ? 2 : 1;
  constexpr int LPR = CW / 8;     // lanes per k-row
  constexpr int KG = kWave / LPR; // k-rows per wavefront instruction
  __shared__ float red[GV_WAVES][NW][R][CW];
  __shared__ typename std::conditional<ROUTE, RouteLds, char>::type rsh;
  if constexpr (ROUTE) {
    route_token(A, K, rt, rsh);
    seg_off = rsh.offsets;
    active = rsh.active;
    nactive = rsh.active + rt.E;
    perm = rsh.perm;
  }
  const int nblk = N / CW;
  const int a_idx = blockIdx.x / nblk;
  if (a_idx >= nactive[0]) return;
  const int e = active[a_idx];
  const int c0 = (blockIdx.x % nblk) * CW;
  const int s0 = seg_off[e], cnt = seg_off[e + 1] - s0;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave), lane = lane_id();
  // The down projection may split K over gridDim.y workgroups (part y writes
  // its fp32 sums to plane y, the combine adds the planes in order).  The
  // wave's K range holds ng blocks of 8 * KG k-rows (a whole number: host
  // check); lane group j takes rows 8 j .. 8 j + 7 of each.
  const int Kp = K / gridDim.y;
  const int kb = blockIdx.y * Kp + wave * (Kp / GV_WAVES) + (lane / LPR) * 8;
  const int cl = c0 + (lane % LPR) * 8;
  const bf16_t *w1 = B1 + ((size_t)e * K + kb) * N + cl;
  const bf16_t *w3 = SWIGLU ? B3 + ((size_t)e * K + kb) * N + cl : w1;
  const int ng = Kp / (GV_WAVES * 8 * KG);

  for (int rg = 0; rg < cnt; rg += R) {
    const bf16_t *ap[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int row = min(rg + r, cnt - 1);  // rows past the end: duplicates, not stored
      const int src = perm ? perm[s0 + row] / kslots : s0 + row;
      ap[r] = A + (size_t)src * K + kb;
    }
    float acc[NW][R][8];
#pragma unroll
    for (int m = 0; m < NW; ++m)
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[m][r][j] = 0.f;
    uint4 wa[NW][8], wb[NW][8], xa[R], xb[R];
    auto load = [&](uint4 (&w)[NW][8], uint4 (&xv)[R], int g) {
      const size_t ro = (size_t)g * 8 * KG * N;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        w[0][i] = ldg16_stream(w1 + ro + (size_t)i * N);
        if (SWIGLU) w[NW - 1][i] = ldg16_stream(w3 + ro + (size_t)i * N);
      }
#pragma unroll
      for (int r = 0; r < R; ++r) xv[r] = *reinterpret_cast<const uint4 *>(ap[r] + g * 8 * KG);
    };
    auto compute = [&](const uint4 (&w)[NW][8], const uint4 (&xv)[R]) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
#pragma unroll
        for (int m = 0; m < NW; ++m) {
          const uint32_t wq[4] = {w[m][i].x, w[m][i].y, w[m][i].z, w[m][i].w};
          float wf[8];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            wf[2 * q] = __uint_as_float(wq[q] << 16);
            wf[2 * q + 1] = __uint_as_float(wq[q] & 0xFFFF0000u);
          }
#pragma unroll
          for (int r = 0; r < R; ++r) {
            const uint32_t xw = (&xv[r].x)[i >> 1];
            const float xs = __uint_as_float((i & 1) ? (xw & 0xFFFF0000u) : (xw << 16));
#pragma unroll
            for (int j = 0; j < 8; ++j) acc[m][r][j] = fmaf(xs, wf[j], acc[m][r][j]);
          }
        }
      }
    };
    load(wa, xa, 0);
    if (ng > 1) load(wb, xb, 1);
    int g = 0;
    for (; g + 2 < ng; g += 2) {
      compute(wa, xa);
      load(wa, xa, g + 2);
      compute(wb, xb);
      if (g + 3 < ng) load(wb, xb, g + 3);
    }
    compute(wa, xa);
    if (g + 1 < ng) compute(wb, xb);
    // lanes of one column set (same lane % LPR) hold partial sums over
    // different k-rows: butterfly over the k-row groups, then waves in order
#pragma unroll
    for (int m = 0; m < NW; ++m)
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          float v = acc[m][r][j];
#pragma unroll
          for (int off = LPR; off < kWave; off <<= 1) v += __shfl_xor(v, off);
          acc[m][r][j] = v;
        }
    if (lane < LPR) {
#pragma unroll
      for (int m = 0; m < NW; ++m)
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
          for (int j = 0; j < 8; ++j) red[wave][m][r][lane * 8 + j] = acc[m][r][j];
    }
    __syncthreads();
    for (int o = tid; o < R * CW; o += GV_THREADS) {
      const int r = o / CW, c = o % CW;
      if (rg + r < cnt) {
        float v[NW];
#pragma unroll
        for (int m = 0; m < NW; ++m) {
          float t = 0.f;
#pragma unroll
          for (int w = 0; w < GV_WAVES; ++w) t += red[w][m][r][c];
          v[m] = t;
        }
        const size_t out = (size_t)(s0 + rg + r) * N + c0 + c;
        if (SWIGLU)
          reinterpret_cast<bf16_t *>(C)[out] = f32_to_bf16(gated(v[0], v[NW - 1], act));
        else
          reinterpret_cast<float *>(C)[blockIdx.y * plane + out] = v[0];
      }
    }
    __syncthreads();
  }
}

// Column block of the [K][N] weight-streaming kernel: the widest (up to
// GVT_MAX_CW columns) that still gives GVT_MIN_WG workgroups with the K
// parts.  Wider blocks read longer runs of each k-row (128 columns: 256
// bytes), which the memory system serves better (one token's SwiGLU, 470 MB:
// 32 columns 183 us, 64 95 us, 128 79 us).
constexpr int GVT_MAX_CW = 128, GVT_MIN_WG = 128;
inline int gvt_kg(int cw) { return kWave / (cw / 8); }
inline bool gvt_fits(int cw, int N, int Kp) {
  return N % cw == 0 && Kp % (GV_WAVES * 8 * gvt_kg(cw)) == 0;
}
inline int gvt_cw(int G, int N, int Kp, int ksplit) {
  for (int cw = GVT_MAX_CW; cw >= 32; cw /= 2)
    if (gvt_fits(cw, N, Kp) && ((long long)G * (N / cw) * ksplit >= GVT_MIN_WG || cw == 32))
      return cw;
  return 0;
}

template <bool SWIGLU, int R>
hipError_t launch_gemv_t_r(int act, const void *A, const int32_t *perm, int kslots,
                           const void *B1, const void *B3, void *C, const int32_t *seg_off,
                           const int32_t *active, const int32_t *nactive, int G, int N, int K,
                           int ksplit, size_t plane, hipStream_t s) {
  const bf16_t *a = (const bf16_t *)A, *b1 = (const bf16_t *)B1, *b3 = (const bf16_t *)B3;
  if ((SWIGLU && ksplit != 1) || ksplit < 1 || K % ksplit) return hipErrorInvalidValue;
  const int cw = gvt_cw(G, N, K / ksplit, ksplit);
#define GVT_LAUNCH(CW_)                                                                       \
  hipLaunchKernelGGL((gemv_t_kernel<SWIGLU, R, CW_>), dim3(G * (N / CW_), ksplit),           \
                     dim3(GV_THREADS), 0, s, a, perm, kslots, b1, b3, C, seg_off, active,    \
                     nactive, N, K, act, plane, DecodeRoute{})
  switch (cw) {
    case 256: GVT_LAUNCH(256); break;
    case 128: GVT_LAUNCH(128); break;
    case 64: GVT_LAUNCH(64); break;
    case 32: GVT_LAUNCH(32); break;
    default: return hipErrorInvalidValue;
  }
#undef GVT_LAUNCH
  return hipGetLastError();
}

template <bool SWIGLU>
hipError_t launch_gemv_t(int rows, int act, const void *A, const int32_t *perm, int kslots,
                         const void *B1, const void *B3, void *C, const int32_t *seg_off,
                         const int32_t *active, const int32_t *nactive, int G, int N, int K,
                         int ksplit, size_t plane, hipStream_t s) {
  if (rows <= 1)
    return launch_gemv_t_r<SWIGLU, 1>(act, A, perm, kslots, B1, B3, C, seg_off, active, nactive,
                                      G, N, K, ksplit, plane, s);
  if (rows <= 2)
    return launch_gemv_t_r<SWIGLU, 2>(act, A, perm, kslots, B1, B3, C, seg_off, active, nactive,
                                      G, N, K, ksplit, plane, s);
  return launch_gemv_t_r<SWIGLU, 4>(act, A, perm, kslots, B1, B3, C, seg_off, active, nactive, G,
                                    N, K, ksplit, plane, s);
}

template <bool SWIGLU, int R, bool COMBINE = false, bool W8 = false, bool ROUTE = false>
hipError_t launch_gemv_r(int act, const void *A, const int32_t *perm, int kslots,
                         const void *B1, const void *B3, void *C, const int32_t *seg_off,
                         const int32_t *active, const int32_t *nactive, int G, int N, int K,
                         int nact, const GemvCombine &cm, const float *sc1, const float *sc3,
                         hipStream_t s, const DecodeRoute &rt = DecodeRoute{}) {
  const int kc = K / (GV_WAVES * GV_CHUNK);
  constexpr int NW = SWIGLU ? 2 : 1;
  // columns per workgroup: a power of two from two groups up to 256, with
  // about 128 workgroups per active expert (fewer, longer workgroups stream
  // best)
  int cpw = 256;
  while (cpw > 1 && 2 * (N / cpw) < 256) cpw /= 2;
  const bf16_t *a = (const bf16_t *)A;
#define GV_CASE(KC_)                                                                          \
  case KC_: {                                                                                 \
    constexpr int CB = gv_cb(NW * KC_);                                                 \
    int cw = cpw < 2 * CB ? 2 * CB : cpw;                                                     \
    if (nact > 0) {                                                                           \
      /* known active experts: as close to one workgroup per CU as N allows */                \
      for (int m = 1; 2 * CB * m <= N; ++m)                                                   \
        if (N % (2 * CB * m) == 0 && (long long)nact * (N / (2 * CB * m)) <= 256) {           \
          cw = 2 * CB * m;                                                                    \
          break;                                                                              \
        }                                                                                     \
    }                                                                                         \
    if (N % cw) return hipErrorInvalidValue;                                                  \
    if (COMBINE && N / cw > FIX_SLOTS) return hipErrorInvalidValue;                           \
    hipLaunchKernelGGL((gemv_kernel<SWIGLU, R, KC_, COMBINE, W8, ROUTE>), dim3(G * (N / cw)), \
                       dim3(GV_THREADS), 0, s, a, perm, kslots, B1, B3, C, seg_off, active,    \
                       nactive, N, K, cw, act, cm, sc1, sc3, rt);                              \
    break;                                                                                    \
  }
  switch (kc) {
    GV_CASE(1) GV_CASE(2) GV_CASE(3) GV_CASE(4) GV_CASE(5) GV_CASE(6) GV_CASE(7) GV_CASE(8)
    default: return hipErrorInvalidValue;
  }
#undef GV_CASE
  return hipGetLastError();
}

template <bool SWIGLU, bool COMBINE = false, bool W8 = false>
hipError_t launch_gemv(int rows, int act, const void *A, const int32_t *perm, int kslots,
                       const void *B1, const void *B3, void *C, const int32_t *seg_off,
                       const int32_t *active, const int32_t *nactive, int G, int N, int K,
                       int nact, const GemvCombine &cm, hipStream_t s,
                       const float *sc1 = nullptr, const float *sc3 = nullptr) {
  if (rows <= 1)
    return launch_gemv_r<SWIGLU, 1, COMBINE, W8>(act, A, perm, kslots, B1, B3, C, seg_off,
                                                 active, nactive, G, N, K, nact, cm, sc1, sc3, s);
  if (rows <= 2)
    return launch_gemv_r<SWIGLU, 2, COMBINE, W8>(act, A, perm, kslots, B1, B3, C, seg_off,
                                                 active, nactive, G, N, K, nact, cm, sc1, sc3, s);
  return launch_gemv_r<SWIGLU, 4, COMBINE, W8>(act, A, perm, kslots, B1, B3, C, seg_off, active,
                                               nactive, G, N, K, nact, cm, sc1, sc3, s);
}

}  // namespace

bool skinny_ok(int N, int K) { return N % SK_NB == 0 && K % (SK_WAVES * SK_KC) == 0; }

hipError_t launch_skinny_swiglu(int mb, int act, const void *x, const int32_t *perm, int kslots,
                                const void *W1, const void *W3, void *H,
                                const int32_t *seg_off, const int32_t *active,
                                const int32_t *nactive, int G, int N, int K, hipStream_t s) {
  return launch_mb<true>(mb, act, x, perm, kslots, W1, W3, H, seg_off, active, nactive, G, N, K,
                         s);
}

hipError_t launch_skinny_down(int mb, const void *Hin, const void *W2, float *Y,
                              const int32_t *seg_off, const int32_t *active,
                              const int32_t *nactive, int G, int N, int K, hipStream_t s) {
  return launch_mb<false>(mb, 0, Hin, nullptr, 1, W2, nullptr, Y, seg_off, active, nactive, G,
                          N, K, s);
}

bool gemv_ok(int N, int K) {
  const int kc = K / (GV_WAVES * GV_CHUNK);
  return K % (GV_WAVES * GV_CHUNK) == 0 && kc >= 1 && kc <= 8 && N % 64 == 0;
}

hipError_t launch_gemv_swiglu(int rows, int act, const void *x, const int32_t *perm, int kslots,
                              const void *W1, const void *W3, void *H, const int32_t *seg_off,
                              const int32_t *active, const int32_t *nactive, int G, int N, int K,
                              int nact, hipStream_t s) {
  return launch_gemv<true>(rows, act, x, perm, kslots, W1, W3, H, seg_off, active, nactive, G, N,
                           K, nact, GemvCombine{}, s);
}

hipError_t launch_gemv_down(int rows, const void *Hin, const void *W2, float *Y,
                            const int32_t *seg_off, const int32_t *active,
                            const int32_t *nactive, int G, int N, int K, int nact,
                            hipStream_t s) {
  return launch_gemv<false>(rows, 0, Hin, nullptr, 1, W2, nullptr, Y, seg_off, active, nactive,
                            G, N, K, nact, GemvCombine{}, s);
}

hipError_t launch_gemv_down_combine(int rows, const void *Hin, const void *W2, float *Y,
                                    const int32_t *seg_off, const int32_t *active,
                                    const int32_t *nactive, int G, int N, int K, int nact,
                                    const int32_t *inv, const float *gate, int T, int k, void *y,
                                    int32_t *cnt, hipStream_t s) {
  const GemvCombine cm{inv, gate, T, k, (bf16_t *)y, cnt};
  return launch_gemv<false, true>(rows, 0, Hin, nullptr, 1, W2, nullptr, Y, seg_off, active,
                                  nactive, G, N, K, nact, cm, s);
}

hipError_t launch_gemv_swiglu_fp8(int rows, int act, const void *x, const int32_t *perm,
                                  int kslots, const uint8_t *W1q, const uint8_t *W3q,
                                  const float *s1, const float *s3, void *H,
                                  const int32_t *seg_off, const int32_t *active,
                                  const int32_t *nactive, int G, int N, int K, int nact,
                                  hipStream_t s) {
  return launch_gemv<true, false, true>(rows, act, x, perm, kslots, W1q, W3q, H, seg_off, active,
                                        nactive, G, N, K, nact, GemvCombine{}, s, s1, s3);
}

hipError_t launch_gemv_down_combine_fp8(int rows, const void *Hin, const uint8_t *W2q,
                                        const float *s2, float *Y, const int32_t *seg_off,
                                        const int32_t *active, const int32_t *nactive, int G,
                                        int N, int K, int nact, const int32_t *inv,
                                        const float *gate, int T, int k, void *y, int32_t *cnt,
                                        hipStream_t s) {
  const GemvCombine cm{inv, gate, T, k, (bf16_t *)y, cnt};
  return launch_gemv<false, true, true>(rows, 0, Hin, nullptr, 1, W2q, nullptr, Y, seg_off,
                                        active, nactive, G, N, K, nact, cm, s, s2, nullptr);
}

bool gemv_t_ok(int N, int K) { return gvt_fits(32, N, K); }

hipError_t launch_gemv_t_swiglu(int rows, int act, const void *x, const int32_t *perm,
                                int kslots, const void *W1, const void *W3, void *H,
                                const int32_t *seg_off, const int32_t *active,
                                const int32_t *nactive, int G, int N, int K, hipStream_t s) {
  return launch_gemv_t<true>(rows, act, x, perm, kslots, W1, W3, H, seg_off, active, nactive, G,
                             N, K, 1, 0, s);
}

hipError_t launch_gemv_t_swiglu_routed(int act, const void *x, const DecodeRoute &r,
                                       const void *W1, const void *W3, void *H, int N, int K,
                                       hipStream_t s) {
  // a single token activates at most k experts: a grid for k of them (the
  // workgroups of experts past the active count return)
  const int G = r.k;
  const int cw = gvt_cw(G, N, K, 1);
  const bf16_t *a = (const bf16_t *)x, *b1 = (const bf16_t *)W1, *b3 = (const bf16_t *)W3;
#define GVTR_LAUNCH(CW_)                                                                      \
  hipLaunchKernelGGL((gemv_t_kernel<true, 1, CW_, true>), dim3(G * (N / CW_), 1),              \
                     dim3(GV_THREADS), 0, s, a, nullptr, r.k, b1, b3, H, nullptr, nullptr,     \
                     nullptr, N, K, act, (size_t)0, r)
  switch (cw) {
    case 256: GVTR_LAUNCH(256); break;
    case 128: GVTR_LAUNCH(128); break;
    case 64: GVTR_LAUNCH(64); break;
    case 32: GVTR_LAUNCH(32); break;
    default: return hipErrorInvalidValue;
  }
#undef GVTR_LAUNCH
  return hipGetLastError();
}

int gemv_t_down_splits(int G, int N, int K, int max_split) {
  // enough K parts for a workgroup per CU in the widest column blocks
  int S = 1;
  while (S * 2 <= max_split && (long long)G * (N / GVT_MAX_CW) * S < 256 && K % (S * 2) == 0 &&
         gvt_cw(G, N, K / (S * 2), S * 2) != 0)
    S *= 2;
  return S;
}

hipError_t launch_gemv_t_down(int rows, const void *Hin, const void *W2, float *Y,
                              const int32_t *seg_off, const int32_t *active,
                              const int32_t *nactive, int G, int N, int K, int ksplit,
                              size_t plane, hipStream_t s) {
  return launch_gemv_t<false>(rows, 0, Hin, nullptr, 1, W2, nullptr, Y, seg_off, active, nactive,
                              G, N, K, ksplit, plane, s);
}

bool route_fused_ok(int T, int d, int E, int k) {
  return T == 1 && E >= 1 && E <= 64 && k <= E && (long long)E * d <= 65536 &&
         d % (GV_THREADS * 8) == 0;
}

hipError_t launch_gemv_swiglu_routed(int act, const void *x, const DecodeRoute &r, const void *W1,
                                     const void *W3, const float *s1, const float *s3, void *H,
                                     int N, int K, hipStream_t s) {
  const int kf = K / GV_CHUNK;
  if (kf == 4 || kf == 8) {
    // column blocks of a multiple of 8 (an even number per wavefront), as
    // many as make one workgroup per CU over the k active experts
    int cpw = N;
    for (int m = 2 * GV_WAVES; m <= N; m += 2 * GV_WAVES)
      if (N % m == 0 && (long long)r.k * (N / m) <= 256) {
        cpw = m;
        break;
      }
    if (N % cpw || (cpw / GV_WAVES) % 2) return hipErrorInvalidValue;
    const dim3 grid(r.k * (N / cpw));
#define GW_LAUNCH(KF_, W8_)                                                                   \
  hipLaunchKernelGGL((gemv_swiglu_wave_kernel<KF_, W8_>), grid, dim3(GV_THREADS), 0, s,        \
                     (const bf16_t *)x, W1, W3, (bf16_t *)H, N, K, cpw, act, r, s1, s3)
    if (kf == 8) {
      if (s1) GW_LAUNCH(8, true); else GW_LAUNCH(8, false);
    } else {
      if (s1) GW_LAUNCH(4, true); else GW_LAUNCH(4, false);
    }
#undef GW_LAUNCH
    return hipGetLastError();
  }
  // one token: at most k experts are active, and the grid covers exactly k
  if (s1)
    return launch_gemv_r<true, 1, false, true, true>(act, x, nullptr, r.k, W1, W3, H, nullptr,
                                                     nullptr, nullptr, r.k, N, K, r.k,
                                                     GemvCombine{}, s1, s3, s, r);
  return launch_gemv_r<true, 1, false, false, true>(act, x, nullptr, r.k, W1, W3, H, nullptr,
                                                    nullptr, nullptr, r.k, N, K, r.k,
                                                    GemvCombine{}, nullptr, nullptr, s, r);
}

bool gemv_token_ok(int N, int K, int k) { return gemv_ok(N, K) && k <= GT_SLOTS; }

hipError_t launch_gemv_down_token(const void *H, const void *W2, const float *s2,
                                  const int32_t *seg_off, const int32_t *active,
                                  const int32_t *nactive, int N, int K, const int32_t *inv,
                                  const float *gate, int k, void *y, hipStream_t s) {
  if (!gemv_token_ok(N, K, k)) return hipErrorInvalidValue;
  const int kc = K / (GV_WAVES * GV_CHUNK);
#define GT_CASE(KC_)                                                                        \
  case KC_: {                                                                               \
    constexpr int CB = gv_cb(KC_);                                                          \
    /* the narrowest block (two groups) up to GT_COLS that keeps to two workgroups per CU */ \
    /* (Mixtral shape, one token, FP8 weights: 0.7-1.5 us per step off one per CU) */     \
    int cw = 2 * CB;                                                                        \
    while (N / cw > 512 && 2 * cw <= GT_COLS && N % (2 * cw) == 0) cw *= 2;                 \
    if (N % cw) return hipErrorInvalidValue;                                                \
    if (s2)                                                                                 \
      hipLaunchKernelGGL((gemv_down_token_kernel<KC_, true>), dim3(N / cw), dim3(GV_THREADS), \
                         0, s, (const bf16_t *)H, W2, seg_off, active, nactive, N, K, cw, inv, \
                         gate, k, (bf16_t *)y, s2);                                         \
    else                                                                                    \
      hipLaunchKernelGGL((gemv_down_token_kernel<KC_, false>), dim3(N / cw), dim3(GV_THREADS), \
                         0, s, (const bf16_t *)H, W2, seg_off, active, nactive, N, K, cw, inv, \
                         gate, k, (bf16_t *)y, nullptr);                                    \
    break;                                                                                  \
  }
  switch (kc) {
    GT_CASE(1) GT_CASE(2) GT_CASE(3) GT_CASE(4) GT_CASE(5) GT_CASE(6) GT_CASE(7) GT_CASE(8)
    default: return hipErrorInvalidValue;
  }
#undef GT_CASE
  return hipGetLastError();
}

}  // namespace moe
