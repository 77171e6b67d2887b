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
#include "common.h"
#include "kernels.h"

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
    const int32_t *__restrict__ nactive, int N, int K) {
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
          reinterpret_cast<bf16_t *>(C)[out] = f32_to_bf16(silu(s[0]) * s[NW - 1]);
        else
          reinterpret_cast<float *>(C)[out] = s[0];
      }
    }
    __syncthreads();
  }
}

template <bool SWIGLU>
hipError_t launch_mb(int mb, const void *A, const int32_t *perm, int kslots, const void *B1,
                     const void *B3, void *C, const int32_t *seg_off, const int32_t *active,
                     const int32_t *nactive, int G, int N, int K, hipStream_t s) {
  dim3 grid(G * (N / SK_NB));
  const bf16_t *a = (const bf16_t *)A, *b1 = (const bf16_t *)B1, *b3 = (const bf16_t *)B3;
  if (mb <= 1)
    hipLaunchKernelGGL((skinny_gemm_kernel<SWIGLU, 1>), grid, dim3(SK_THREADS), 0, s, a, perm,
                       kslots, b1, b3, C, seg_off, active, nactive, N, K);
  else if (mb == 2)
    hipLaunchKernelGGL((skinny_gemm_kernel<SWIGLU, 2>), grid, dim3(SK_THREADS), 0, s, a, perm,
                       kslots, b1, b3, C, seg_off, active, nactive, N, K);
  else
    hipLaunchKernelGGL((skinny_gemm_kernel<SWIGLU, 4>), grid, dim3(SK_THREADS), 0, s, a, perm,
                       kslots, b1, b3, C, seg_off, active, nactive, N, K);
  return hipGetLastError();
}

}  // namespace

bool skinny_ok(int N, int K) { return N % SK_NB == 0 && K % (SK_WAVES * SK_KC) == 0; }

hipError_t launch_skinny_swiglu(int mb, const void *x, const int32_t *perm, int kslots,
                                const void *W1, const void *W3, void *H,
                                const int32_t *seg_off, const int32_t *active,
                                const int32_t *nactive, int G, int N, int K, hipStream_t s) {
  return launch_mb<true>(mb, x, perm, kslots, W1, W3, H, seg_off, active, nactive, G, N, K, s);
}

hipError_t launch_skinny_down(int mb, const void *Hin, const void *W2, float *Y,
                              const int32_t *seg_off, const int32_t *active,
                              const int32_t *nactive, int G, int N, int K, hipStream_t s) {
  return launch_mb<false>(mb, Hin, nullptr, 1, W2, nullptr, Y, seg_off, active, nactive, G, N,
                          K, s);
}

}  // namespace moe
