// Grouped expert GEMMs on the gfx950 matrix cores.
//
// For each expert segment e (rows offsets[e] .. offsets[e+1]-1 of the permuted
// activations):
//   SWIGLU = true : H = SiLU(A W1_e^T) * (A W3_e^T)   (W1, W3 [E][N][K], H [rows][N])
//   SWIGLU = false: Y = A W2_e^T                       (W2 [E][N][K], Y fp32 [rows][N])
// ("Mistral 8x7B SMoE architecture deep dive", section 3.1; "Mixtral and MoE
// architecture", FeedForward listing; the fused gate/up layout of the numpy
// listing in "Trillion-parameter MoE ... 7 expert configs measured" is what
// pairing W1 and W3 tiles in one workgroup follows.)
//
// Tiling.  A workgroup of 256 threads (4 wavefronts, WM x WN) owns a BM x BNB
// tile, where BNB counts B rows: for SWIGLU the B tile interleaves 32-row
// blocks of W1 and W3 for the same output columns, so a wave holds the W1 and
// W3 accumulators of an output element in the same lane and register and the
// SiLU * mul epilogue needs no data movement.  K is streamed in BK slices
// through double-buffered LDS.  The register-staged kernel (fp32, and bf16
// with K not a multiple of 64) pads LDS rows by 16 bytes; the bf16 kernel
// with direct global->LDS loads swizzles 16-byte chunks instead.  Both keep
// the 16-byte fragment reads free of bank conflicts.
//
// Operands: both A and B are K-contiguous ([rows][K] and [N][K]), the layout
// in which every lane of a 32x32 MFMA reads 16 consecutive bytes of K.
//   bf16: v_mfma_f32_32x32x16_bf16, one per 16-wide K step.
//   fp32: v_mfma_f32_32x32x2_f32, eight per 16-wide K step; lane group g feeds
//         K indices g*8 + i to the i-th MFMA (A and B use the same order).
//
// Tile map.  mtile_off[e] is the prefix of ceil(count_e / BM) over experts;
// map_tile turns a 1-D workgroup id into (expert, m-tile, n-tile).
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

template <typename T> struct MfmaTraits;
template <> struct MfmaTraits<bf16_t> {
  static constexpr int BK = 64;  // 128 bytes of K per LDS row
  static constexpr int FRAG_U4 = 1;  // uint4 per lane per 16-wide K step
  __device__ __forceinline__ static void mma(const uint4 *a, const uint4 *b, f32x16_v &c) {
    c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_v, a[0]),
                                                __builtin_bit_cast(bf16x8_v, b[0]), c, 0, 0, 0);
  }
  __device__ __forceinline__ static void store(bf16_t *p, size_t i, float v) {
    p[i] = f32_to_bf16(v);
  }
};
template <> struct MfmaTraits<float> {
  static constexpr int BK = 32;
  static constexpr int FRAG_U4 = 2;
  __device__ __forceinline__ static void mma(const uint4 *a, const uint4 *b, f32x16_v &c) {
    const float *af = reinterpret_cast<const float *>(a);
    const float *bf = reinterpret_cast<const float *>(b);
#pragma unroll
    for (int i = 0; i < 8; ++i) c = __builtin_amdgcn_mfma_f32_32x32x2f32(af[i], bf[i], c, 0, 0, 0);
  }
  __device__ __forceinline__ static void store(float *p, size_t i, float v) { p[i] = v; }
};

constexpr int GM_THREADS = 256;
constexpr int NUM_XCD = 8;  // MI355X: 8 accelerator complex dies, each with its own L2

// Workgroup -> (expert, global m-tile, n-tile).  Workgroups are dispatched to
// the XCDs round-robin (id % 8), so each XCD gets a contiguous chunk of the
// logical tile order; the logical order is expert-major, then n-tile, with the
// expert's m-tiles fastest, so the workgroups that share a weight tile run at
// the same time on the same XCD and its L2 serves the re-reads.  The chunking
// uses the real tile count (known on the device once the permutation ran);
// the grid is launched for an upper bound plus NUM_XCD and surplus
// workgroups exit.
struct Tile {
  int e, g, n;
};
__device__ __forceinline__ bool map_tile(int hw, const int32_t *mtile_off, int G, int ntn,
                                         Tile &t) {
  const int R = ntn * mtile_off[G];
  const int R8 = (R + NUM_XCD - 1) / NUM_XCD;
  const int local = hw / NUM_XCD;
  if (local >= R8) return false;
  const int L = (hw % NUM_XCD) * R8 + local;
  if (L >= R) return false;
  const int e = upper_segment(mtile_off, G, L / ntn);
  const int rem = L - ntn * mtile_off[e];
  const int me = mtile_off[e + 1] - mtile_off[e];
  t.e = e;
  t.n = rem / me;
  t.g = mtile_off[e] + rem % me;
  return true;
}

template <typename T, int BM, int BNB, int WM, int WN, bool SWIGLU>
__global__ __launch_bounds__(GM_THREADS) void grouped_gemm_kernel(
    const T *__restrict__ A, const T *__restrict__ B1, const T *__restrict__ B3,
    void *__restrict__ C, const int32_t *__restrict__ seg_off,
    const int32_t *__restrict__ mtile_off, int G, int N, int K) {
  constexpr int BK = MfmaTraits<T>::BK;
  constexpr int ES = sizeof(T);
  constexpr int CPR = BK * ES / 16;            // 16-byte chunks per tile row (8)
  constexpr int LDW = (BK * ES + 16) / 16;     // LDS row stride in uint4 (9)
  constexpr int TM = BM / WM / 32;             // 32-row MFMA blocks per wave
  constexpr int TN = BNB / WN / 32;            // 32-col MFMA blocks per wave
  constexpr int A_CH = BM * CPR / GM_THREADS;  // A chunks per thread
  constexpr int B_CH = BNB * CPR / GM_THREADS;
  constexpr int FU = MfmaTraits<T>::FRAG_U4;
  static_assert(!SWIGLU || (TN % 2 == 0), "SwiGLU pairs W1/W3 blocks inside a wave");
  static_assert(A_CH * GM_THREADS == BM * CPR && B_CH * GM_THREADS == BNB * CPR, "tile/threads");

  __shared__ uint4 lds[2][(BM + BNB) * LDW];

  constexpr int COLS = SWIGLU ? BNB / 2 : BNB;  // output columns per tile
  Tile tile;
  if (!map_tile(blockIdx.x, mtile_off, G, (N + COLS - 1) / COLS, tile)) return;
  const int e = tile.e;
  const int row0 = seg_off[e] + (tile.g - mtile_off[e]) * BM;
  const int rows = min(BM, seg_off[e + 1] - row0);
  const int NOUT = N;  // output columns
  const int n0 = tile.n * COLS;  // first output column

  const int tid = threadIdx.x;
  const int wave = tid / kWave, lane = lane_id();
  const int wm = wave / WN, wn = wave % WN;

  // ---- global source pointers for this thread's chunks (fixed over K) ----
  const uint4 *srcA[A_CH];
  const uint4 *srcB[B_CH];
  int dstA[A_CH], dstB[B_CH];
  const size_t rowq = (size_t)K * ES / 16;
#pragma unroll
  for (int i = 0; i < A_CH; ++i) {
    int c = tid + i * GM_THREADS;
    int r = c / CPR, q = c % CPR;
    int rr = min(r, rows - 1);
    srcA[i] = reinterpret_cast<const uint4 *>(A) + (size_t)(row0 + rr) * rowq + q;
    dstA[i] = r * LDW + q;
  }
  const size_t bexp = (size_t)e * N * rowq;  // expert offset in uint4
#pragma unroll
  for (int i = 0; i < B_CH; ++i) {
    int c = tid + i * GM_THREADS;
    int r = c / CPR, q = c % CPR;
    const T *base;
    int col;
    if (SWIGLU) {
      int rb = r / 32, wnb = rb / TN, j = rb % TN;
      col = n0 + wnb * (TN / 2) * 32 + (j / 2) * 32 + (r % 32);
      base = (j & 1) ? B3 : B1;
    } else {
      col = n0 + r;
      base = B1;
    }
    col = min(col, N - 1);
    srcB[i] = reinterpret_cast<const uint4 *>(base) + bexp + (size_t)col * rowq + q;
    dstB[i] = (BM + r) * LDW + q;
  }

  f32x16_v acc[TM][TN];
#pragma unroll
  for (int a = 0; a < TM; ++a)
#pragma unroll
    for (int b = 0; b < TN; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[a][b][i] = 0.f;

  uint4 ra[A_CH], rb[B_CH];
  const int nk = K / BK;
  auto gload = [&](int kt) {
    const size_t ko = (size_t)kt * CPR;
#pragma unroll
    for (int i = 0; i < A_CH; ++i) ra[i] = srcA[i][ko];
#pragma unroll
    for (int i = 0; i < B_CH; ++i) rb[i] = srcB[i][ko];
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < A_CH; ++i) lds[buf][dstA[i]] = ra[i];
#pragma unroll
    for (int i = 0; i < B_CH; ++i) lds[buf][dstB[i]] = rb[i];
  };

  gload(0);
  lstore(0);
  __syncthreads();

  // fragment addressing inside a tile (uint4 units)
  const int frow = lane & 31;
  const int fk = (lane >> 5) * FU;  // lane group's first uint4 within a 16-wide K step

  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) gload(kt + 1);
    const uint4 *L = lds[buf];
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      const int ko = ks * 2 * FU + fk;  // 16-wide K step = 2*FU uint4
      uint4 af[TM][FU], bfr[TN][FU];
#pragma unroll
      for (int a = 0; a < TM; ++a)
#pragma unroll
        for (int u = 0; u < FU; ++u) af[a][u] = L[((wm * TM + a) * 32 + frow) * LDW + ko + u];
#pragma unroll
      for (int b = 0; b < TN; ++b)
#pragma unroll
        for (int u = 0; u < FU; ++u)
          bfr[b][u] = L[(BM + (wn * TN + b) * 32 + frow) * LDW + ko + u];
#pragma unroll
      for (int a = 0; a < TM; ++a)
#pragma unroll
        for (int b = 0; b < TN; ++b) MfmaTraits<T>::mma(af[a], bfr[b], acc[a][b]);
    }
    if (kt + 1 < nk) lstore(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue ----
  const int ccol = lane & 31;
  const int crow4 = (lane >> 5) * 4;
#pragma unroll
  for (int a = 0; a < TM; ++a) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int r = (wm * TM + a) * 32 + (i / 4) * 8 + crow4 + (i % 4);
      if (r >= rows) continue;
      const size_t orow = (size_t)(row0 + r) * NOUT;
      if (SWIGLU) {
#pragma unroll
        for (int q = 0; q < TN / 2; ++q) {
          const int col = n0 + wn * (TN / 2) * 32 + q * 32 + ccol;
          if (col < N) {
            const float h = silu(acc[a][2 * q][i]) * acc[a][2 * q + 1][i];
            MfmaTraits<T>::store(reinterpret_cast<T *>(C), orow + col, h);
          }
        }
      } else {
#pragma unroll
        for (int b = 0; b < TN; ++b) {
          const int col = n0 + (wn * TN + b) * 32 + ccol;
          if (col < N) reinterpret_cast<float *>(C)[orow + col] = acc[a][b][i];
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// bf16 variant with direct global->LDS loads (global_load_lds_dwordx4).
//
// Each wavefront instruction moves 64 x 16 bytes into 1 KB of contiguous LDS:
// 8 tile rows of 128 bytes (64 bf16 of K).  Rows are not padded; instead lane
// l of an instruction fetches global 16-byte chunk (l % 8) ^ f(row) of its row,
// with f(row) = (row >> 1) & 7, so LDS chunk c of row r holds global chunk
// c ^ f(r).  A fragment read (16 lanes, 16 consecutive rows, one global chunk)
// then touches 16 distinct 16-byte slots modulo 256 bytes: conflict-free on
// the 64 LDS banks.  Two stages of (BM + BNB) x 128 bytes, no staging
// registers.
//
// The loads are bound by how many requests a CU keeps in flight, not by the
// bandwidth of L2 or HBM, so the schedule gives each slice's loads as much
// time as the two stages allow: every wave reads ALL fragments of a slice into
// registers at the slice's start; once every wave has done so (a barrier a
// quarter of the way in), the stage is refilled with the slice two ahead, and
// those loads are spread over the next 32 MFMAs.  A load thus has about 1.75
// slices of MFMA work to land (one slice with the stage held until the end).
// ---------------------------------------------------------------------------
// Split K (down projection only): blockIdx.y picks one of gridDim.y equal K
// ranges and its fp32 partial goes to output plane blockIdx.y (plane elements
// apart); the combine adds the planes in a fixed order.
template <int BM, int BNB, bool SWIGLU>
__global__ __launch_bounds__(GM_THREADS) void grouped_gemm_dl_kernel(
    const bf16_t *__restrict__ A, const bf16_t *__restrict__ B1, const bf16_t *__restrict__ B3,
    void *__restrict__ C, const int32_t *__restrict__ seg_off,
    const int32_t *__restrict__ mtile_off, int G, int N, int K, size_t plane) {
  constexpr int WM = 2, WN = 2;
  constexpr int TM = BM / WM / 32, TN = BNB / WN / 32;
  constexpr int ROWS = BM + BNB;          // tile rows per stage (A then B)
  constexpr int STAGE_U4 = ROWS * 8;      // uint4 per stage
  static_assert(!SWIGLU || (TN % 2 == 0), "SwiGLU pairs W1/W3 blocks inside a wave");
  static_assert(BM % 32 == 0 && BNB % 32 == 0, "rows per stage must split over 4 waves");

  __shared__ uint4 st0[STAGE_U4];
  __shared__ uint4 st1[STAGE_U4];
  constexpr int COLS = SWIGLU ? BNB / 2 : BNB;
  Tile tile;
  if (!map_tile(blockIdx.x, mtile_off, G, (N + COLS - 1) / COLS, tile)) return;
  const int e = tile.e;
  const int row0 = seg_off[e] + (tile.g - mtile_off[e]) * BM;
  const int rows = min(BM, seg_off[e + 1] - row0);
  const int n0 = tile.n * COLS;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave), lane = lane_id();
  const int wm = wave / WN, wn = wave % WN;

  // Per-instruction global byte offsets (relative to uniform bases).  Wave w
  // loads A blocks w*IA .. w*IA+IA-1 and B blocks w*IB .. w*IB+IB-1 (8 rows
  // each), so whether an instruction reads A, W1 or W3 is fixed per j.
  constexpr int IA = BM / 32, IB = BNB / 32;  // instructions per wave per stage
  const int kpart = K / gridDim.y;  // K range of this split (a multiple of 64)
  const size_t kb = (size_t)blockIdx.y * kpart * 2;  // its byte offset inside a row
  const char *abase = reinterpret_cast<const char *>(A) + (size_t)row0 * K * 2 + kb;
  const size_t eoff = (size_t)e * N * K * 2 + kb;
  const char *b1base = reinterpret_cast<const char *>(B1) + eoff;
  const char *b3base = SWIGLU ? reinterpret_cast<const char *>(B3) + eoff : b1base;
  uint32_t aoff[IA], boff[IB];
  const int lrow = lane >> 3, lchunk = lane & 7;
#pragma unroll
  for (int j = 0; j < IA; ++j) {
    const int r = (wave * IA + j) * 8 + lrow;
    const int gch = lchunk ^ ((r >> 1) & 7);
    aoff[j] = (uint32_t)min(r, rows - 1) * K * 2 + gch * 16;
  }
#pragma unroll
  for (int j = 0; j < IB; ++j) {
    const int br = (wave * IB + j) * 8 + lrow;
    const int gch = lchunk ^ ((br >> 1) & 7);
    int col;
    if (SWIGLU) {
      // 32-row blocks alternate W1 / W3 for the same 32 output columns
      const int rb = br / 32, wnb = rb / TN, jj = rb % TN;
      col = n0 + wnb * (TN / 2) * 32 + (jj / 2) * 32 + (br % 32);
    } else {
      col = n0 + br;
    }
    boff[j] = (uint32_t)min(col, N - 1) * K * 2 + gch * 16;
  }
  // B block parity: block (wave*IB + j)/4 is odd (a W3 block) iff (j/4) is odd,
  // because IB is a multiple of 8
  static_assert(!SWIGLU || IB % 8 == 0, "W1/W3 choice must be fixed per instruction");
  auto issue = [&](uint4 *stage, int kt) {
    const uint32_t ko = (uint32_t)kt * 128;
#pragma unroll
    for (int j = 0; j < IA; ++j)
      global_to_lds16(abase + aoff[j] + ko, stage + (wave * IA + j) * 64);
#pragma unroll
    for (int j = 0; j < IB; ++j) {
      const char *bb = (SWIGLU && ((j / 4) & 1)) ? b3base : b1base;
      global_to_lds16(bb + boff[j] + ko, stage + BM * 8 + (wave * IB + j) * 64);
    }
  };

  f32x16_v acc[TM][TN];
#pragma unroll
  for (int a = 0; a < TM; ++a)
#pragma unroll
    for (int b = 0; b < TN; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[a][b][i] = 0.f;

  // fragment addressing: row part and the swizzled chunk of each 16-wide K step
  const int frow = lane & 31;
  const int xf = (frow >> 1) & 7;
  int cidx[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) cidx[ks] = (ks * 2 + (lane >> 5)) ^ xf;
  // fragments of one 16-wide K step
  auto rd = [&](const uint4 *stage, int ks, uint4 (&af)[TM], uint4 (&bf)[TN]) {
#pragma unroll
    for (int a = 0; a < TM; ++a) af[a] = stage[((wm * TM + a) * 32 + frow) * 8 + cidx[ks]];
#pragma unroll
    for (int b = 0; b < TN; ++b) bf[b] = stage[(BM + (wn * TN + b) * 32 + frow) * 8 + cidx[ks]];
  };
  auto mm = [&](const uint4 (&af)[TM], const uint4 (&bf)[TN]) {
#pragma unroll
    for (int a = 0; a < TM; ++a)
#pragma unroll
      for (int b = 0; b < TN; ++b)
        acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            __builtin_bit_cast(bf16x8_v, af[a]), __builtin_bit_cast(bf16x8_v, bf[b]), acc[a][b],
            0, 0, 0);
  };

  // Pipeline: a slice's fragments are all read into registers at its start,
  // so its LDS stage can be refilled (with the slice two ahead) once every
  // wave has read it, a quarter of the way into the slice; the load of a
  // slice then has about 1.75 slices of MFMA work to land instead of one.
  const int nk = kpart / 64;
  constexpr int PER = IA + IB;  // LDS-DMA instructions per wave per slice
  uint4 f0a[TM], f0b[TN], g0a[TM], g0b[TN], f1a[TM], f1b[TN], f2a[TM], f2b[TN], f3a[TM], f3b[TN];
#define SCHED_FENCE() __builtin_amdgcn_sched_barrier(0)
#define SG(m, n) __builtin_amdgcn_sched_group_barrier(m, n, 0)
#define RAW_BARRIER() do { __atomic_signal_fence(__ATOMIC_SEQ_CST); __builtin_amdgcn_s_barrier(); \
  __atomic_signal_fence(__ATOMIC_SEQ_CST); } while (0)
#define VM_WAIT(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | 0xF70)
#define LGKM_WAIT0() __builtin_amdgcn_s_waitcnt(0xC07F)
  // 32 MFMAs with one LDS-DMA issue after every second one
#define P_MM_LD() do { for (int q_ = 0; q_ < 16; ++q_) { SG(8,1); SG(0x20,1); SG(8,1); } } while (0)
  // 16 MFMAs with two LDS reads after each of the first 12
#define P_MM_RD() do { for (int q_ = 0; q_ < 12; ++q_) { SG(8,1); SG(0x100,2); } SG(8,4); } while (0)
  // body of one slice: S holds it, its K step 0 fragments are in (ca, cb);
  // S2 receives / holds the next slice, whose step 0 goes to (na, nb)
#define SLICE_BODY(S, S2, s, ca, cb, na, nb)                                   \
  do {                                                                         \
    rd(S, 1, f1a, f1b);                                                        \
    rd(S, 2, f2a, f2b);                                                        \
    rd(S, 3, f3a, f3b);                                                        \
    mm(ca, cb);                                                                \
    P_MM_RD();                                                                 \
    SCHED_FENCE();                                                             \
    LGKM_WAIT0();                                                              \
    RAW_BARRIER(); /* every wave has read S */                                 \
    issue(S, min((s) + 2, nk - 1)); /* past the end: a harmless reload */      \
    mm(f1a, f1b);                                                              \
    mm(f2a, f2b);                                                              \
    P_MM_LD();                                                                 \
    SCHED_FENCE();                                                             \
    VM_WAIT(PER);                                                              \
    RAW_BARRIER(); /* slice s+1 is in S2 */                                    \
    rd(S2, 0, na, nb); /* past the end: stale, unused */                       \
    mm(f3a, f3b);                                                              \
    SCHED_FENCE();                                                             \
  } while (0)
  issue(st0, 0);
  issue(st1, min(1, nk - 1));
  VM_WAIT(PER);
  RAW_BARRIER();
  rd(st0, 0, f0a, f0b);
  int kt = 0;
  for (; kt + 1 < nk; kt += 2) {
    SLICE_BODY(st0, st1, kt, f0a, f0b, g0a, g0b);
    SLICE_BODY(st1, st0, kt + 1, g0a, g0b, f0a, f0b);
  }
  if (kt < nk) SLICE_BODY(st0, st1, kt, f0a, f0b, g0a, g0b);
  VM_WAIT(0);
#undef SLICE_BODY
#undef P_MM_LD
#undef P_MM_RD
#undef RAW_BARRIER
#undef VM_WAIT
#undef LGKM_WAIT0
#undef SCHED_FENCE
#undef SG

  // ---- epilogue ----
  const int ccol = lane & 31;
  const int crow4 = (lane >> 5) * 4;
#pragma unroll
  for (int a = 0; a < TM; ++a) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int r = (wm * TM + a) * 32 + (i / 4) * 8 + crow4 + (i % 4);
      if (r >= rows) continue;
      const size_t orow = (size_t)(row0 + r) * N;
      if (SWIGLU) {
#pragma unroll
        for (int q = 0; q < TN / 2; ++q) {
          const int col = n0 + wn * (TN / 2) * 32 + q * 32 + ccol;
          if (col < N)
            reinterpret_cast<bf16_t *>(C)[orow + col] =
                f32_to_bf16(silu(acc[a][2 * q][i]) * acc[a][2 * q + 1][i]);
        }
      } else {
#pragma unroll
        for (int b = 0; b < TN; ++b) {
          const int col = n0 + (wn * TN + b) * 32 + ccol;
          if (col < N)
            reinterpret_cast<float *>(C)[blockIdx.y * plane + orow + col] = acc[a][b][i];
        }
      }
    }
  }
}

template <int BM, int BNB, bool SWIGLU>
hipError_t launch_dl(const void *A, const void *B1, const void *B3, void *C,
                     const int32_t *seg_off, const int32_t *mtile_off, int G, int N, int K,
                     int max_mtiles, int ksplit, size_t plane, hipStream_t s) {
  const int cols = SWIGLU ? BNB / 2 : BNB;
  dim3 grid(((N + cols - 1) / cols) * max_mtiles + NUM_XCD, ksplit);
  hipLaunchKernelGGL((grouped_gemm_dl_kernel<BM, BNB, SWIGLU>), grid, dim3(GM_THREADS), 0, s,
                     (const bf16_t *)A, (const bf16_t *)B1, (const bf16_t *)B3, C, seg_off,
                     mtile_off, G, N, K, plane);
  return hipGetLastError();
}

template <typename T, int BM, int BNB, int WM, int WN, bool SWIGLU>
hipError_t launch_one(const void *A, const void *B1, const void *B3, void *C,
                      const int32_t *seg_off, const int32_t *mtile_off, int G, int N, int K,
                      int max_mtiles, hipStream_t s) {
  const int cols = SWIGLU ? BNB / 2 : BNB;
  dim3 grid(((N + cols - 1) / cols) * max_mtiles + NUM_XCD);
  hipLaunchKernelGGL((grouped_gemm_kernel<T, BM, BNB, WM, WN, SWIGLU>), grid, dim3(GM_THREADS),
                     0, s, (const T *)A, (const T *)B1, (const T *)B3, C, seg_off, mtile_off, G,
                     N, K);
  return hipGetLastError();
}

}  // namespace

GemmPlan gemm_plan(int dtype, int d, int d_ff, int d_ff_shared, long long rows_per_expert) {
  GemmPlan p;
  const int q = 64;  // K granule of the direct-to-LDS kernel
  p.dl1 = dtype == 1 && d % q == 0;
  p.dl2 = dtype == 1 && d_ff % q == 0 && (d_ff_shared == 0 || d_ff_shared % q == 0);
  // 64-row tiles when experts hold few rows (less padding, two workgroups per CU)
  const int bm_dl = rows_per_expert <= 96 ? 64 : 256;
  p.bm1 = p.dl1 ? bm_dl : 128;
  p.bm2 = p.dl2 ? bm_dl : 128;
  return p;
}

hipError_t launch_gemm_swiglu(int dtype, bool dl, int bm, const void *A, const void *W1,
                              const void *W3, void *H, const int32_t *seg_off,
                              const int32_t *mtile_off, int G, int N, int K, int max_mtiles,
                              hipStream_t s) {
  if (max_mtiles <= 0) return hipSuccess;
  if (dl && bm == 64)
    return launch_dl<64, 256, true>(A, W1, W3, H, seg_off, mtile_off, G, N, K, max_mtiles, 1, 0,
                                    s);
  if (dl)
    return launch_dl<256, 256, true>(A, W1, W3, H, seg_off, mtile_off, G, N, K, max_mtiles, 1,
                                     0, s);
  if (dtype == 1)
    return launch_one<bf16_t, 128, 128, 2, 2, true>(A, W1, W3, H, seg_off, mtile_off, G, N, K,
                                                    max_mtiles, s);
  return launch_one<float, 128, 128, 2, 2, true>(A, W1, W3, H, seg_off, mtile_off, G, N, K,
                                                 max_mtiles, s);
}

hipError_t launch_gemm_down(int dtype, bool dl, int bm, const void *A, const void *W2, float *Y,
                            const int32_t *seg_off, const int32_t *mtile_off, int G, int N, int K,
                            int max_mtiles, int ksplit, size_t plane, hipStream_t s) {
  if (max_mtiles <= 0) return hipSuccess;
  if (dl && bm == 64)
    return launch_dl<64, 256, false>(A, W2, nullptr, Y, seg_off, mtile_off, G, N, K,
                                     max_mtiles, ksplit, plane, s);
  if (dl)
    return launch_dl<256, 256, false>(A, W2, nullptr, Y, seg_off, mtile_off, G, N, K,
                                      max_mtiles, ksplit, plane, s);
  if (dtype == 1)
    return launch_one<bf16_t, 128, 128, 2, 2, false>(A, W2, nullptr, Y, seg_off, mtile_off, G,
                                                     N, K, max_mtiles, s);
  return launch_one<float, 128, 128, 2, 2, false>(A, W2, nullptr, Y, seg_off, mtile_off, G, N,
                                                  K, max_mtiles, s);
}

}  // namespace moe
