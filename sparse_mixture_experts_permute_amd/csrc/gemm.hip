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
// map_tile turns a 1-D workgroup id into (expert, m-tile, n-tile).  The
// direct-to-LDS kernel takes expert e's rows as seg_off[e] .. seg_end[e] - 1,
// so a segment's bulk can go to 256-row tiles and a short remainder to light
// 64-row tiles of the same launch (LIGHT).  The persistent kernel also splits
// the tiles of its last round along K (plan_split).
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
  // the fragments stay in registers: each uint4 is reinterpreted as a value
  // (a float pointer into the fragment arrays would put them in scratch)
  __device__ __forceinline__ static void mma(const uint4 *a, const uint4 *b, f32x16_v &c) {
#pragma unroll
    for (int u = 0; u < FRAG_U4; ++u) {
      const f32x4_v av = __builtin_bit_cast(f32x4_v, a[u]);
      const f32x4_v bv = __builtin_bit_cast(f32x4_v, b[u]);
#pragma unroll
      for (int i = 0; i < 4; ++i) c = __builtin_amdgcn_mfma_f32_32x32x2f32(av[i], bv[i], c, 0, 0, 0);
    }
  }
  __device__ __forceinline__ static void store(float *p, size_t i, float v) { p[i] = v; }
};

constexpr int GM_THREADS = 256;
constexpr int NUM_XCD = 8;  // MI355X: 8 accelerator complex dies, each with its own L2

// Workgroup -> (expert, global m-tile, n-tile).  Workgroups are dispatched to
// the XCDs round-robin (id % 8).  The logical tile order is expert-major, then
// n-tile, with the expert's m-tiles fastest; it is cut into blocks of BS
// consecutive tiles, dealt to the XCDs in turn (block b -> XCD b % 8).  Within
// a block the workgroups sharing a weight tile or a row tile run at the same
// time on one XCD (its L2 serves the re-reads), and neighbouring blocks, which
// share the expert's rows, run at the same time on the other XCDs (the MALL
// serves those).  BS is chosen so that every XCD gets the same number of tiles
// (within one block) for the grid's CUs per XCD; surplus workgroups exit.
// Launches with light tiles (below) take each XCD's tiles from a queue instead
// (an atomic counter per XCD, tile_q): a workgroup takes the XCD's next tile
// when it finishes one, so the XCD's workgroups stay on neighbouring tiles
// however unequal the tiles' times (a full and a light tile of the same
// weight columns, tiles with the epilogue or without), and the rows or weights
// they share stay in its L2.  Walked in fixed steps, the workgroups drift
// apart over the rounds: on 256 experts at T=8192 the down GEMM read 12.1 GB
// against 7.8 GB of operands, and took 2.79 ms against 2.42 with the queue.
struct Tile {
  int e, g, n;
  int light;  // a 64-row light tile of a 256-row launch (below)
};
// Position in the logical order of the tile that workgroup slot hw takes, or
// -1 (a surplus slot).  R tiles; W workgroups walk them (a multiple of 8).
__device__ __forceinline__ int tile_order(int hw, int R, int W) {
  const int cpx = max(1, W / NUM_XCD);  // resident workgroups per XCD
  const int R8 = (R + NUM_XCD - 1) / NUM_XCD;
  const int rounds = max(1, (R8 + cpx - 1) / cpx);
  const int BS = max(1, (R + NUM_XCD * rounds - 1) / (NUM_XCD * rounds));
  const int xcd = hw % NUM_XCD, local = hw / NUM_XCD;
  const int L = ((local / BS) * NUM_XCD + xcd) * BS + local % BS;
  return L < R ? L : -1;
}
// Logical tile L -> (expert, global m-tile, n-tile): expert-major, then
// n-tile, the expert's m-tiles fastest.
__device__ __forceinline__ Tile decode_tile(int L, const int32_t *mtile_off, int G, int ntn) {
  Tile t;
  const int e = upper_segment(mtile_off, G, L / ntn);
  const int rem = L - ntn * mtile_off[e];
  const int me = mtile_off[e + 1] - mtile_off[e];
  t.e = e;
  t.n = rem / me;
  t.g = mtile_off[e] + rem % me;
  t.light = 0;
  return t;
}
// Light tiles.  A 256-row launch may also serve the few rows of an expert
// past its last full tile ("light" 64-row tiles, at most two per expert):
// expert e then has mt0[e+1] - mt0[e] full tiles followed by lt[e+1] - lt[e]
// light tiles in its m-tile order (mt0, lt: prefixes), so that a light tile
// runs next to the full tiles of the same weight columns and reads them
// through the same L2.  Combined prefix: mt0[e] + lt[e].
__device__ __forceinline__ Tile decode_tile_light(int L, const int32_t *mt0, const int32_t *lt,
                                                  int G, int ntn) {
  const int gt = L / ntn;
  int lo = 0, hi = G;  // largest e with mt0[e] + lt[e] <= gt
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (mt0[mid] + lt[mid] <= gt) lo = mid; else hi = mid;
  }
  Tile t;
  const int c0 = mt0[lo] + lt[lo];
  const int rem = L - ntn * c0;
  const int me = mt0[lo + 1] + lt[lo + 1] - c0;
  const int gl = rem % me;  // m-tile of the expert: its full tiles first
  const int full = mt0[lo + 1] - mt0[lo];
  t.e = lo;
  t.n = rem / me;
  t.light = gl >= full;
  t.g = t.light ? gl - full : mt0[lo] + gl;  // light: its index among the expert's light tiles
  return t;
}
__device__ __forceinline__ bool map_tile(int hw, const int32_t *mtile_off, int G, int ntn,
                                         Tile &t) {
  const int L = tile_order(hw, ntn * mtile_off[G], gridDim.x);
  if (L < 0) return false;
  t = decode_tile(L, mtile_off, G, ntn);
  return true;
}

// Spreading the last, partial round of a persistent launch.  With W resident
// workgroups, R tiles are q full rounds plus m = R mod W tail tiles, which
// would leave W - m workgroups idle for a whole tile.  Instead each tail tile
// is cut into S parts along K, so the tail becomes m*S shorter work units:
// units 0 .. F-1 (F = R - m) are whole tiles, units F .. F + m*S - 1 are the
// parts (part p of tail tile j is unit F + p*m + j).  Every part writes its fp32
// partial sums to a scratch slot and counts itself in; the part that arrives
// last adds all partials in part order (so the sum does not depend on timing)
// and runs the tile's epilogue.  S is a power of two dividing the K slices
// into pairs, at most 16 and with m*S <= part_cap, picked by an estimate of
// the tail's time in K slices: ceil(m*S / W) rounds of nk/S slices of MFMA
// work, 6 of fixed cost (the partial's store among them) and red10/10 per
// partial the last part reads back; a split must save 15% of the tail.
struct Split {
  int F, m, S;
};
__device__ __forceinline__ Split plan_split(int R, int W, int nk, int red10, int part_cap) {
  Split sp{R, 0, 1};
  const int m = R % W;
  if (m == 0 || m > FIX_SLOTS - TILE_Q_SLOTS) return sp;
  int best = nk * 85 / 10;  // the tail tiles run whole (a split must save 15%)
  for (int s = 2; s <= 16 && (nk / 2) % s == 0 && m * s <= part_cap; s *= 2) {
    const int cost = ((m * s + W - 1) / W) * (nk * 10 / s + 60 + red10 * s);
    if (cost < best) {
      best = cost;
      sp.S = s;
    }
  }
  if (sp.S > 1) {
    sp.F = R - m;
    sp.m = m;
  }
  return sp;
}

template <typename T, int BM, int BNB, int WM, int WN, bool SWIGLU, bool TB = false>
__global__ __launch_bounds__(GM_THREADS) void grouped_gemm_kernel(
    const T *__restrict__ A, const T *__restrict__ B1, const T *__restrict__ B3,
    void *__restrict__ C, const int32_t *__restrict__ seg_off,
    const int32_t *__restrict__ mtile_off, int G, int N, int K, int act, size_t plane) {
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
  // K planes (down projection): blockIdx.y takes one of gridDim.y equal K
  // ranges and writes its fp32 sums to output plane blockIdx.y (plane
  // elements apart); the combine adds the planes in order
  const int Kp = K / gridDim.y, kbeg = blockIdx.y * Kp;

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
    srcA[i] = reinterpret_cast<const uint4 *>(A) + (size_t)(row0 + rr) * rowq + q +
              (size_t)kbeg * ES / 16;
    dstA[i] = r * LDW + q;
  }
  const size_t bexp = (size_t)e * N * rowq;  // expert offset in uint4
  // TB ([K][N] weights): chunk c holds VE consecutive columns of k-row c / (BNB
  // / VE); it is stored transposed into the [column][K] LDS tile
  constexpr int VE = 16 / ES;  // elements per 16-byte chunk
  const size_t bstep = TB ? (size_t)BK * N / VE : (size_t)CPR;  // uint4 per K slice
#pragma unroll
  for (int i = 0; i < B_CH; ++i) {
    int c = tid + i * GM_THREADS;
    if constexpr (TB) {
      const int kk = c / (BNB / VE), r = (c % (BNB / VE)) * VE;
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
      col = min(col, N - VE);
      srcB[i] = reinterpret_cast<const uint4 *>(base + ((size_t)e * K + kbeg + kk) * N + col);
      dstB[i] = (BM + r) * LDW * VE + kk;  // in elements
      continue;
    }
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
    srcB[i] = reinterpret_cast<const uint4 *>(base) + bexp + (size_t)col * rowq + q +
              (size_t)kbeg * ES / 16;
    dstB[i] = (BM + r) * LDW + q;
  }

  f32x16_v acc[TM][TN];
#pragma unroll
  for (int a = 0; a < TM; ++a)
#pragma unroll
    for (int b = 0; b < TN; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[a][b][i] = 0.f;

  // staging registers of the next K slice, as plain vectors (uint4 arrays
  // copied through here stayed in scratch memory, which serialised every
  // slice's global loads ahead of its MFMAs)
  typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
  u32x4_t ra[A_CH], rb[B_CH];
  const int nk = Kp / BK;
  auto gload = [&](int kt) {
    const size_t ko = (size_t)kt * CPR;
#pragma unroll
    for (int i = 0; i < A_CH; ++i) ra[i] = *reinterpret_cast<const u32x4_t *>(srcA[i] + ko);
#pragma unroll
    for (int i = 0; i < B_CH; ++i)
      rb[i] = *reinterpret_cast<const u32x4_t *>(srcB[i] + (size_t)kt * bstep);
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < A_CH; ++i) *reinterpret_cast<u32x4_t *>(&lds[buf][dstA[i]]) = ra[i];
#pragma unroll
    for (int i = 0; i < B_CH; ++i) {
      if constexpr (TB) {
        T v[VE];
        __builtin_memcpy(v, &rb[i], 16);
        T *l = reinterpret_cast<T *>(lds[buf]);
#pragma unroll
        for (int u = 0; u < VE; ++u) l[dstB[i] + u * LDW * VE] = v[u];
      } else {
        *reinterpret_cast<u32x4_t *>(&lds[buf][dstB[i]]) = rb[i];
      }
    }
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
            const float h = gated(acc[a][2 * q][i], acc[a][2 * q + 1][i], act);
            MfmaTraits<T>::store(reinterpret_cast<T *>(C), orow + col, h);
          }
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

// ---------------------------------------------------------------------------
// bf16 variant with direct loads into LDS (buffer_load_dwordx4 ... lds).
//
// Each wavefront instruction moves 64 x 16 bytes into 1 KB of contiguous LDS:
// 8 tile rows of 128 bytes (64 bf16 of K).  Rows are not padded; instead lane
// l of an instruction fetches global 16-byte chunk (l % 8) ^ f(row) of its row,
// with f(row) = (row >> 1) & 7, so LDS chunk c of row r holds global chunk
// c ^ f(r).  A fragment read (16 lanes, 16 consecutive rows, one global chunk)
// then touches 16 distinct 16-byte slots modulo 256 bytes: conflict-free on
// the 64 LDS banks.  Two stages of (BM + BNB) x 128 bytes, no staging
// registers.  The buffer resources are bounded to the tile's rows of A and to
// the expert's N weight rows, so ragged tiles need no clamping.
//
// The loads are bound by how many requests a CU keeps in flight, not by the
// bandwidth of L2 or HBM, so the schedule gives each slice's loads as much
// time as the two stages allow: every wave reads ALL fragments of a slice into
// registers at the slice's start; once every wave has done so (a barrier a
// quarter of the way in), the stage is refilled with the slice two ahead, and
// those loads are spread over the remaining 48 MFMAs.  A load thus has about
// 1.75 slices of MFMA work to land (one slice with the stage held until the
// end).
//
// The kernel is persistent (one workgroup per CU, two for 64-row tiles): the
// next tile's first two slices are loaded while the current tile's epilogue
// runs.  The tiles of the last round are split along K (plan_split), so that
// every workgroup has work until the end.  A down projection with too few
// tiles for the GPU instead splits every tile's K into planes (blockIdx.y)
// that the combine adds.
// ---------------------------------------------------------------------------
// Two floats to two bf16 (round to nearest even) in one 32-bit word, low first.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2_v;
  const f32x2_v f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_v));
}

// Epilogue of one tile of the direct-to-LDS kernel.  The MFMAs take the
// weight fragment as their first operand, so each accumulator block holds the
// transposed product: lane l has token row l % 32 of the block and, in each of
// the four groups of 8 output columns, the 4 consecutive columns starting at
// 4 * (l / 32).  SwiGLU gates those 4 columns (act: the gate's activation)
// and stores them as 8 bytes of bf16; the down projection stores them as 16
// bytes of fp32 into plane blockIdx.y, or (act = 1, one plane) as 8 bytes of
// bf16.  No LDS staging, so both stages are free for the next tile's loads
// during the epilogue.
template <int BM, int BNB, bool SWIGLU, int TM, int TN, typename TA>
__device__ __forceinline__ void dl_epilogue(const TA &ta, f32x16_v (&acc)[TM][TN],
                                            void *__restrict__ C, int N, size_t plane, int act,
                                            int wave, int lane) {
  constexpr int WN = 2;
  const int wm = wave / WN, wn = wave % WN;
  const int row0 = ta.row0, rows = ta.rows, n0 = ta.n0;
  const int tr = lane & 31;          // token row inside a 32-row block
  const int cq = (lane >> 5) * 4;    // first of the lane's 4 columns in each 8-column group
  if constexpr (SWIGLU) {
    constexpr int WC = 32 * TN / 2;  // output columns per wave
#pragma unroll
    for (int a = 0; a < TM; ++a) {
      const int grow = (wm * TM + a) * 32 + tr;
      bf16_t *dst = reinterpret_cast<bf16_t *>(C) + (size_t)(row0 + grow) * N + n0 + wn * WC;
#pragma unroll
      for (int q = 0; q < TN / 2; ++q)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          float h[4];
#pragma unroll
          for (int u = 0; u < 4; ++u)
            h[u] = gated(acc[a][2 * q][g * 4 + u], acc[a][2 * q + 1][g * 4 + u], act);
          uint2 v;
          v.x = pack_bf16x2(h[0], h[1]);
          v.y = pack_bf16x2(h[2], h[3]);
          const int c = q * 32 + g * 8 + cq;
          if (grow < rows && n0 + wn * WC + c < N) *reinterpret_cast<uint2 *>(dst + c) = v;
        }
    }
  } else if (act) {
    bf16_t *out = reinterpret_cast<bf16_t *>(C);
#pragma unroll
    for (int a = 0; a < TM; ++a) {
      const int r = (wm * TM + a) * 32 + tr;
      bf16_t *dst = out + (size_t)(row0 + r) * N + n0;
#pragma unroll
      for (int b = 0; b < TN; ++b)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int c = (wn * TN + b) * 32 + g * 8 + cq;
          uint2 v;
          v.x = pack_bf16x2(acc[a][b][g * 4], acc[a][b][g * 4 + 1]);
          v.y = pack_bf16x2(acc[a][b][g * 4 + 2], acc[a][b][g * 4 + 3]);
          if (r < rows && n0 + c < N) *reinterpret_cast<uint2 *>(dst + c) = v;
        }
    }
  } else {
    float *out = reinterpret_cast<float *>(C) + blockIdx.y * plane;
#pragma unroll
    for (int a = 0; a < TM; ++a) {
      const int r = (wm * TM + a) * 32 + tr;
      float *dst = out + (size_t)(row0 + r) * N + n0;
#pragma unroll
      for (int b = 0; b < TN; ++b)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int c = (wn * TN + b) * 32 + g * 8 + cq;
          const float4 v = make_float4(acc[a][b][g * 4], acc[a][b][g * 4 + 1],
                                       acc[a][b][g * 4 + 2], acc[a][b][g * 4 + 3]);
          if (r < rows && n0 + c < N) *reinterpret_cast<float4 *>(dst + c) = v;
        }
    }
  }
}

// SPLIT: the last round's tiles may be split along K (plan_split); compiled
// only where that pays, since the split's code costs registers in every tile.
// GATHER: A is the token matrix x (a_bytes bytes) and tile row s reads x row
// gperm[s] / gk, so the grouped rows are never written out; each lane keeps
// the byte offsets of its rows for the tile (one per A instruction).
// W8: the weights are FP8 (E4M3) codes [N][K] with one scale per expert (sc1
// for W1 or W2, sc3 for W3).  They reach LDS as codes, 128 bytes of K per row
// and code stage (whole 128-byte lines; 16-byte chunk c of row r sits in slot
// c ^ ((r >> 1) & 7)), so one code stage serves two 64-wide K slices; a
// fragment read converts its 8 codes to bf16 exactly, and the epilogue
// multiplies the sums by the expert's scales.  64-row tiles only.
// LIGHT: the launch also serves light 64-row tiles (lmt: their per-expert
// prefix, lmid[e]: the row where expert e's light rows start; full tiles end
// there); a light tile's rows sit in wave row 0's first two 32-row blocks,
// whose MFMAs alone run.
template <int BM, int BNB, bool SWIGLU, bool SPLIT, bool GATHER = false, bool TB = false,
          bool W8 = false, bool LIGHT = false>
__global__ __launch_bounds__(GM_THREADS) void grouped_gemm_dl_kernel(
    const bf16_t *__restrict__ A, const bf16_t *__restrict__ B1, const bf16_t *__restrict__ B3,
    void *__restrict__ C, const int32_t *__restrict__ seg_off,
    const int32_t *__restrict__ seg_end, const int32_t *__restrict__ mtile_off, int G, int N,
    int K, size_t plane, int act, int32_t *__restrict__ fix_cnt, f32x4_v *__restrict__ fix_part,
    int part_cap, const int32_t *__restrict__ gperm, int gk, uint32_t a_bytes,
    const float *__restrict__ sc1, const float *__restrict__ sc3,
    const int32_t *__restrict__ lmid, const int32_t *__restrict__ lmt,
    int32_t *__restrict__ tile_q) {
  constexpr int WM = 2, WN = 2;
  constexpr int TM = BM / WM / 32, TN = BNB / WN / 32;
  // A rows of 128 bytes, then B rows of 128 bytes (64 for FP8 codes)
  constexpr int STAGE_U4 = BM * 8 + BNB * (W8 ? 4 : 8);  // uint4 per stage
  static_assert(!SWIGLU || (TN % 2 == 0), "SwiGLU pairs W1/W3 blocks inside a wave");
  static_assert(BM % 32 == 0 && BNB % 32 == 0, "rows per stage must split over 4 waves");
  static_assert(!TB || BNB == 256, "the [K][N] weight tile is two 128-column halves");
  static_assert(!W8 || (BM == 64 && !TB && !SPLIT), "FP8 weights: 64-row tiles of [N][K] codes");
  static_assert(!LIGHT || (BM == 256 && !SPLIT && !W8), "light tiles: 256-row launches");

  // FP8 tiles: two row stages of one 64-wide K slice and two code stages of
  // a slice pair (128 codes per weight row: a code load reads whole 128-byte
  // lines, where a load of one slice's 64 codes per row reads half-lines and
  // moves half the bytes per memory request).  Slice s reads rows ra[s % 2]
  // and half s % 2 of code stage pc[(s / 2) % 2], then refills ra[s % 2] with
  // the rows of slice s+2; an odd slice s also refills the code stage it has
  // just finished with the codes of slices s+3 and s+4, which then have two
  // and a half slices to land.  Each stage is an array of its own and fixed
  // per slice of a four-slice unrolled loop: with the stage picked at run time
  // the compiler cannot tell which stage a read touches and waits for every
  // load in flight before it.  80 KB per workgroup, two per CU.
  constexpr bool RING4 = W8;
  constexpr int A_U4 = BM * 8, P_U4 = BNB * 8;
  __shared__ uint4 st0[RING4 ? 1 : STAGE_U4];
  __shared__ uint4 st1[RING4 ? 1 : STAGE_U4];
  __shared__ uint4 ra0[RING4 ? A_U4 : 1], ra1[RING4 ? A_U4 : 1];
  __shared__ uint4 pc0[RING4 ? P_U4 : 1], pc1[RING4 ? P_U4 : 1];
  __shared__ int fix_arrived;
  __shared__ int q_next;  // LIGHT with a queue: the next tile's index in the XCD's order
  constexpr int COLS = SWIGLU ? BNB / 2 : BNB;
  const int ntn = (N + COLS - 1) / COLS;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave), lane = lane_id();
  const int wm = wave / WN, wn = wave % WN;

  // LDS-DMA instructions per wave per stage; IBP: code instructions per wave
  // per FP8 code stage (8 rows of 128 codes each)
  constexpr int IA = BM / 32, IB = BNB / 32, IBP = BNB / 32;
  constexpr int PER = IA + IB;
  // K planes (down projection of small batches): blockIdx.y takes one of
  // gridDim.y equal K ranges, its fp32 partial goes to output plane blockIdx.y
  // (plane elements apart) and the combine adds the planes in order
  const int kpl = K / gridDim.y;                          // a multiple of 128
  const uint32_t kb_pl = (uint32_t)blockIdx.y * kpl * 2;  // its byte offset in a row
  const int nk_all = kpl / 64;  // 64-wide K slices of a whole tile (even)
  // work units: whole tiles, then the parts of the tail tiles (reading a
  // partial back is bound by the latency of device-scope loads: about 10 slices)
  const int R = ntn * (LIGHT ? mtile_off[G] + lmt[G] : mtile_off[G]);
  // Workgroups in use.  64-row tiles serve weight-streaming batches, where a
  // partly used last round costs bandwidth: as many workgroups as give every
  // one the same number of tiles walk them, the rest exit (Mixtral-shaped
  // decode, 784 tiles on 512 resident workgroups: SwiGLU GEMM 0.308 -> 0.286
  // ms at 8 tokens).  Larger tiles keep the whole grid (the last-round split
  // spreads their tail).
  int Wg = gridDim.x;
  if constexpr (BM == 64) {
    const int rounds = max(1, (R + Wg - 1) / Wg);  // R may be 0 (every pair dropped)
    Wg = min((int)gridDim.x, ((R + rounds - 1) / rounds + NUM_XCD - 1) / NUM_XCD * NUM_XCD);
  }
  if ((int)blockIdx.x >= Wg) return;
  const Split sp = SPLIT && gridDim.y == 1 ? plan_split(R, Wg, nk_all, 100, part_cap)
                                           : Split{R, 0, 1};
  const int lrow = lane >> 3, lchunk = lane & 7;

  // Addressing of one tile.  A tile reads its rows of A and its columns of
  // W1 / W3 (or W2) through buffer resources bounded to the segment's rows and
  // the N rows of the expert's weight, so rows past either end read as zeros
  // (their results are not stored) and nothing is clamped.  Wave w loads A
  // blocks w*IA .. w*IA+IA-1 and B blocks w*IB .. w*IB+IB-1 (8 rows of 128
  // bytes each); lane l takes row l/8 of the block and the 16-byte chunk
  // (l % 8) ^ ((row >> 1) & 7), which only depends on the block's parity.
  const uint32_t rowb = (uint32_t)K * 2;  // bytes per row of A and B
  const uint32_t lc0 = (uint32_t)lrow * rowb + (uint32_t)((lchunk ^ (lrow >> 1)) * 16);
  const uint32_t lc1 = lc0 ^ 64u;          // chunk ^ 4 for odd blocks
  // TB ([K][N] weights): an instruction moves 4 k-rows of 128 columns (256 B
  // each) of one matrix; lane l takes k-row l / 16 and LDS chunk l % 16, which
  // holds global chunk (l % 16) ^ (4 * (row & 3)) of its row (row & 3 = l / 16)
  const uint32_t tbl = TB ? (uint32_t)(lane >> 4) * (uint32_t)N * 2u +
                                (uint32_t)(((lane & 15) ^ ((lane >> 4) << 2)) * 16)
                          : 0u;
  // W8: instruction q moves code rows 8q .. 8q+7, 128 bytes of each; lane l
  // takes row 8q + l / 8 and LDS slot l % 8, which holds chunk (l % 8) ^ x of
  // its row, x = (row >> 1) & 7 = 4 (q & 1) + l / 16 (w8l0: q even, w8l1: odd)
  const uint32_t w8l0 =
      W8 ? (uint32_t)(lane >> 3) * (uint32_t)K + (uint32_t)(((lane & 7) ^ (lane >> 4)) * 16) : 0u;
  const uint32_t w8l1 =
      W8 ? (uint32_t)(lane >> 3) * (uint32_t)K +
               (uint32_t)(((lane & 7) ^ (4 + (lane >> 4))) * 16)
         : 0u;
  struct TileAddr {
    __amdgpu_buffer_rsrc_t ra, r1, r3;
    uint32_t lc0, lc1;
    uint32_t tbl;  // TB: the lane's byte offset inside a [K][N] weight instruction
    uint32_t w8l0, w8l1;  // W8: the lane's byte offset inside an even / odd code instruction
    int e;         // the unit's expert
    uint32_t ga[GATHER ? IA : 1];  // GATHER: byte offset in x of each A instruction's row
    int row0, rows, n0;
    int light; // a light 64-row tile (LIGHT)
    int nk;    // K slices of this unit (even)
    int part;  // part of a split tail tile, or -1 for a whole tile
    int slot;  // the tail tile's index among the split ones
  };
  // work unit u -> tile and K range (false: no unit u)
  auto map_unit = [&](int u, Tile &t, TileAddr &ta) -> bool {
    if (u < sp.F || sp.S == 1) {
      const int L = tile_order(u, sp.F, Wg);
      if (L < 0) return false;
      if constexpr (LIGHT) t = decode_tile_light(L, mtile_off, lmt, G, ntn);
      else t = decode_tile(L, mtile_off, G, ntn);
      ta.nk = nk_all;
      ta.part = -1;
      ta.slot = 0;
      return true;
    }
    const int j = u - sp.F;
    if (j >= sp.m * sp.S) return false;
    ta.slot = j % sp.m;
    ta.part = j / sp.m;
    ta.nk = nk_all / sp.S;
    t = decode_tile(sp.F + ta.slot, mtile_off, G, ntn);
    return true;
  };
  auto setup = [&](const Tile &t, TileAddr &ta) {
    const int e = t.e;
    const uint32_t kb = kb_pl + (ta.part < 0 ? 0u : (uint32_t)(ta.part * ta.nk) * 128u);
    if (LIGHT && t.light) {
      ta.row0 = lmid[e] + t.g * 64;
      ta.rows = min(64, seg_end[e] - ta.row0);
    } else {
      ta.row0 = seg_off[e] + (t.g - mtile_off[e]) * BM;
      ta.rows = min(BM, (LIGHT ? lmid[e] : seg_end[e]) - ta.row0);
    }
    ta.light = LIGHT ? t.light : 0;
    ta.n0 = t.n * COLS;
    if constexpr (GATHER) {
      // the whole of x; a row past the tile's end reads at a_bytes, past the
      // buffer's range, which loads zeros
      ta.ra = make_rsrc(reinterpret_cast<const char *>(A) + kb, a_bytes - kb);
      const uint32_t cx0 = (uint32_t)((lchunk ^ (lrow >> 1)) * 16);
#pragma unroll
      for (int j = 0; j < IA; ++j) {
        const int r = (wave * IA + j) * 8 + lrow;
        const uint32_t cx = (j & 1) ? (cx0 ^ 64u) : cx0;
        ta.ga[j] = (r < ta.rows ? (uint32_t)(gperm[ta.row0 + r] / gk) * rowb : a_bytes) + cx;
      }
    } else {
      ta.ra = make_rsrc(reinterpret_cast<const char *>(A) + (size_t)ta.row0 * rowb + kb,
                        (uint32_t)ta.rows * rowb - kb);
    }
    // [N][K] weights: the unit's K range starts kb bytes into every row;
    // [K][N] weights (TB): it starts kb / 2 rows of N elements into the matrix
    // FP8 codes (W8): one byte per element, so kb / 2 bytes into every row
    const uint32_t wkb = TB ? (kb / 2) * (uint32_t)N * 2u : W8 ? kb / 2 : kb;
    const uint32_t wrow = W8 ? (uint32_t)K : rowb;  // bytes per weight row
    const size_t eoff = (size_t)e * N * wrow + wkb;
    const uint32_t wbytes = (uint32_t)N * wrow - wkb;
    ta.e = e;
    ta.r1 = make_rsrc(reinterpret_cast<const char *>(B1) + eoff, wbytes);
    ta.r3 = SWIGLU ? make_rsrc(reinterpret_cast<const char *>(B3) + eoff, wbytes) : ta.r1;
    // per-tile copies of the lane offsets: keeps the compiler from hoisting
    // every instruction's offset out of the tile loop (and spilling them)
    ta.lc0 = lc0;
    ta.lc1 = lc1;
    ta.tbl = tbl;
    ta.w8l0 = w8l0;
    ta.w8l1 = w8l1;
    asm volatile("" : "+v"(ta.lc0), "+v"(ta.lc1), "+v"(ta.tbl), "+v"(ta.w8l0), "+v"(ta.w8l1));
  };
  // B block parity: block (wave*IB + j)/4 is odd (a W3 block) iff (j/4) is odd,
  // because IB is a multiple of 8
  static_assert(W8 || !SWIGLU || IB % 8 == 0, "W1/W3 choice must be fixed per instruction");
  static_assert(IA % 2 == 0 && IB % 2 == 0, "chunk swizzle parity per instruction");
  // LDS-DMA instructions j0 <= j < j1 of one slice (A blocks first, then B)
  auto issue_part = [&](const TileAddr &ta, uint4 *stage, int kt, int j0, int j1) {
    const uint32_t ko = (uint32_t)kt * 128;
#pragma unroll
    for (int j = 0; j < IA; ++j)
      if (j >= j0 && j < j1) {
        if constexpr (GATHER) {
          buffer_to_lds16(ta.ra, ta.ga[j] + ko, stage + (wave * IA + j) * 64);
        } else {
          const uint32_t u = (uint32_t)((wave * IA + j) * 8) * rowb + ko;
          buffer_to_lds16(ta.ra, ((j & 1) ? ta.lc1 : ta.lc0) + u, stage + (wave * IA + j) * 64);
        }
      }
    if constexpr (TB) {
      // B stage: [half][k-row 0..63][128 columns]; half = matrix (W1, W3) for
      // SwiGLU, else columns n0 + 128 * half.  Instruction q = wave * IB + j
      // fills k-rows 4 * (q % 16) .. + 3 of half q / 16.
      const uint32_t kob = (uint32_t)kt * 128u * (uint32_t)N;  // 64 k-rows per slice
#pragma unroll
      for (int j = 0; j < IB; ++j) {
        if (IA + j >= j0 && IA + j < j1) {
          const int q = wave * IB + j, h = q / 16, kq = q % 16;
          const uint32_t colb = (uint32_t)(SWIGLU ? ta.n0 : ta.n0 + 128 * h) * 2u;
          buffer_to_lds16<BM == 64>((SWIGLU && h) ? ta.r3 : ta.r1,
                                    ta.tbl + kob + (uint32_t)kq * 8u * (uint32_t)N + colb,
                                    stage + BM * 8 + q * 64);
        }
      }
      return;
    }
#pragma unroll
    for (int j = 0; j < IB; ++j) {
      if (IA + j >= j0 && IA + j < j1) {
        const int br = (wave * IB + j) * 8;  // first B row of the block
        int col;
        if (SWIGLU) {
          // 32-row blocks alternate W1 / W3 for the same 32 output columns
          const int rb = br / 32, wnb = rb / TN, jj = rb % TN;
          col = ta.n0 + wnb * (TN / 2) * 32 + (jj / 2) * 32 + (br % 32);
        } else {
          col = ta.n0 + br;
        }
        const uint32_t u = (uint32_t)col * rowb + ko;
        // 64-row tiles serve small batches, where a weight tile is read by
        // one m-tile: stream it past the caches
        buffer_to_lds16<BM == 64>((SWIGLU && ((j / 4) & 1)) ? ta.r3 : ta.r1,
                                  ((j & 1) ? ta.lc1 : ta.lc0) + u,
                        stage + BM * 8 + (wave * IB + j) * 64);
      }
    }
  };
  auto issue = [&](const TileAddr &ta, uint4 *stage, int kt) { issue_part(ta, stage, kt, 0, PER); };
  // ring: rows of slice kta into sa and, when kpb >= 0, the codes of slice
  // pair kpb (K 128 kpb .. + 127) into sb; code instruction q = wave * IBP + j
  // fills code rows 8q .. 8q+7, all in one 32-row block.  Instructions j0 <= j
  // < j1 of the slice: the IA row instructions first, then the IBP code ones.
  // A slice or pair past the unit's end is loaded from past the buffer's
  // range (zeros, no memory read), which keeps every slice's load count and
  // wait the same.
  auto issue4 = [&](const TileAddr &ta, uint4 *sa, int kta, uint4 *sb, int kpb, int j0, int j1) {
    uint32_t koa = (uint32_t)kta * 128 + (kta < ta.nk ? 0u : 0x80000000u);
    uint32_t kop = (uint32_t)kpb * 128 + (2 * kpb < ta.nk ? 0u : 0x80000000u);
    asm volatile("" : "+s"(koa), "+s"(kop));
#pragma unroll
    for (int j = 0; j < IA; ++j)
      if (j >= j0 && j < j1) {
        if constexpr (GATHER) {
          buffer_to_lds16(ta.ra, ta.ga[j] + koa, sa + (wave * IA + j) * 64);
        } else {
          const uint32_t u = (uint32_t)((wave * IA + j) * 8) * rowb + koa;
          buffer_to_lds16(ta.ra, ((j & 1) ? ta.lc1 : ta.lc0) + u, sa + (wave * IA + j) * 64);
        }
      }
    if (kpb < 0) return;
#pragma unroll
    for (int j = 0; j < IBP; ++j)
      if (IA + j >= j0 && IA + j < j1) {
        const int q = wave * IBP + j, br = 8 * q;
        int col;
        bool w3 = false;
        if (SWIGLU) {
          const int rb = br / 32, wnb = rb / TN, jj = rb % TN;
          col = ta.n0 + wnb * (TN / 2) * 32 + (jj / 2) * 32 + (br % 32);
          w3 = jj & 1;
        } else {
          col = ta.n0 + br;
        }
        buffer_to_lds16<true>(w3 ? ta.r3 : ta.r1,
                              ((j & 1) ? ta.w8l1 : ta.w8l0) + (uint32_t)col * (uint32_t)K + kop,
                              sb + q * 64);
      }
  };
  // a unit's first slices: rows of slices 0 and 1, codes of pairs 0 and 1
  auto prologue4 = [&](const TileAddr &ta) {
    issue4(ta, ra0, 0, pc0, 0, 0, IA + IBP);
    issue4(ta, ra1, 1, pc1, 1, 0, IA + IBP);
  };

  f32x16_v acc[TM][TN];
  // fragment addressing: row part and the swizzled chunk of each 16-wide K step
  // (recomputed per tile from a laundered lane id, see lane_t below)
  int frow, cidx[4];
  // TB: byte offset inside the B stage of the lane's transposed read for
  // 32-column block beta of a half (its K step 0, first 4 k-rows).  Lane l of
  // group g = l / 16 (i = l % 16) addresses k-row 8 * (g / 2) + i / 4 and
  // columns 32 * beta + 16 * (g % 2) + 4 * (i % 4) .. + 3; ds_read_tr16_b64
  // then hands lane i of the group column 32 * beta + 16 * (g % 2) + i of
  // those four k-rows, which is what a 32x32x16 MFMA lane needs (column l % 32,
  // K values 8 * (l / 32) + 0..3; the next read gives + 4..7).
  int tbo[TN];
  // W8: the lane's 8 codes of chunk x (= 4 h + K step ks) sit at byte
  // w8b + 16 (x ^ w8f) of a code stage (two registers, not one per chunk)
  int w8b = 0, w8f = 0;
  auto set_frag_addr = [&](int ln) {
    frow = ln & 31;
    const int xf = (frow >> 1) & 7;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) cidx[ks] = (ks * 2 + (ln >> 5)) ^ xf;
    if constexpr (W8) {
      w8f = ((ln & 31) >> 1) & 7;
      w8b = (ln & 31) * 128 + 8 * ((ln >> 5) & 1);
    }
    if constexpr (TB) {
      // the wave's block b: SwiGLU matrix b & 1, beta 2 * wn + b / 2; down
      // half wn, beta b (the wave-dependent parts folded in here, so that a
      // read's offset is a constant beyond this per-lane value)
      const int g = (ln >> 4) & 3, i = ln & 15, r = i >> 2;
#pragma unroll
      for (int b = 0; b < TN; ++b) {
        const int m = SWIGLU ? (b & 1) : wn;
        const int be = SWIGLU ? 2 * wn + (b >> 1) : b;
        tbo[b] = BM * 128 + m * 16384 + (8 * (g >> 1) + r) * 256 +
                 ((4 * (be ^ r)) + 2 * (g & 1) + ((i & 3) >> 1)) * 16 + 8 * (i & 1);
      }
    }
  };
  set_frag_addr(lane);
  // fragments of one 16-wide K step
  auto rd = [&](const uint4 *stage, int ks, uint4 (&af)[TM], uint4 (&bf)[TN]) {
#pragma unroll
    for (int a = 0; a < TM; ++a) af[a] = stage[((wm * TM + a) * 32 + frow) * 8 + cidx[ks]];
    if constexpr (TB) {
      typedef __attribute__((address_space(3))) bf16x4_v lds_bf16x4;
      const __attribute__((address_space(3))) char *sb =
          (const __attribute__((address_space(3))) char *)stage;
#pragma unroll
      for (int b = 0; b < TN; ++b) {
        // SwiGLU: block b of wave wn is matrix b & 1, columns wn * 64 + (b / 2) * 32
        // of the half; down: half wn, columns b * 32 (folded into tbo[b])
        const int off = tbo[b] + ks * 16 * 256;
        const bf16x4_v lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)(sb + off));
        const bf16x4_v hi =
            __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)(sb + off + 4 * 256));
        const uint2 l2 = __builtin_bit_cast(uint2, lo), h2 = __builtin_bit_cast(uint2, hi);
        bf[b] = make_uint4(l2.x, l2.y, h2.x, h2.y);
      }
    } else {
#pragma unroll
      for (int b = 0; b < TN; ++b)
        bf[b] = stage[(BM + (wn * TN + b) * 32 + frow) * 8 + cidx[ks]];
    }
  };
  int rd_tag = 0;  // the slice being read (varies per slice)
  // fragments of K step ks of a slice: rows from sa, codes from half h of sb
  auto rd4 = [&](const uint4 *sa, const uint4 *sb, int h, int ks, uint4 (&af)[TM],
                 uint4 (&bf)[TN]) {
    // lane offsets through an opaque copy tied to the slice: every read is a
    // register plus a constant offset, not a register per read held across
    // the loop
    int oa = ((wm * TM * 32 + frow) * 8 + cidx[ks]) * 16, f = w8f;
    asm("" : "+v"(oa), "+v"(f) : "s"(rd_tag));
    const int ob = w8b + 16 * ((h * 4 + ks) ^ f) + wn * TN * 32 * 128;
    const char *pa = reinterpret_cast<const char *>(sa), *pb = reinterpret_cast<const char *>(sb);
#pragma unroll
    for (int a = 0; a < TM; ++a) af[a] = *reinterpret_cast<const uint4 *>(pa + oa + a * 4096);
#pragma unroll
    for (int b = 0; b < TN; ++b) {
      const uint2 q = *reinterpret_cast<const uint2 *>(pb + ob + b * 32 * 128);
      // E4M3 -> bf16 is exact; gfx950 converts two codes at a time
      bf[b] = make_uint4(
          __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q.x, 1.f, false)),
          __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q.x, 1.f, true)),
          __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q.y, 1.f, false)),
          __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(q.y, 1.f, true)));
    }
  };
  auto mm = [&](const uint4 (&af)[TM], const uint4 (&bf)[TN]) {
#pragma unroll
    for (int a = 0; a < TM; ++a)
#pragma unroll
      for (int b = 0; b < TN; ++b)
        acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            __builtin_bit_cast(bf16x8_v, bf[b]), __builtin_bit_cast(bf16x8_v, af[a]), acc[a][b],
            0, 0, 0);
  };
  // a light tile: rows 0..63, the first two 32-row blocks of wave row 0
  auto mml = [&](const uint4 (&af)[TM], const uint4 (&bf)[TN]) {
    if (wm == 0) {
#pragma unroll
      for (int a = 0; a < 2 && a < TM; ++a)
#pragma unroll
        for (int b = 0; b < TN; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              __builtin_bit_cast(bf16x8_v, bf[b]), __builtin_bit_cast(bf16x8_v, af[a]),
              acc[a][b], 0, 0, 0);
    }
  };
  uint4 f0a[TM], f0b[TN], g0a[TM], g0b[TN], f1a[TM], f1b[TN], f2a[TM], f2b[TN], f3a[TM], f3b[TN];
#define SCHED_FENCE() __builtin_amdgcn_sched_barrier(0)
#define SG(m, n) __builtin_amdgcn_sched_group_barrier(m, n, 0)
#define RAW_BARRIER() do { __atomic_signal_fence(__ATOMIC_SEQ_CST); __builtin_amdgcn_s_barrier(); \
  __atomic_signal_fence(__ATOMIC_SEQ_CST); } while (0)
#define VM_WAIT(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | 0xF70)
#define LGKM_WAIT0() __builtin_amdgcn_s_waitcnt(0xC07F)
  // LDS read instructions per 16-wide K step (a transposed B fragment takes two)
  constexpr int RDS = TM + (TB ? 2 : 1) * TN;
  // 16 MFMAs with RDS / 4 LDS reads after each of the first 12
#define P_MM_RD() do { for (int q_ = 0; q_ < 12; ++q_) { SG(8,1); SG(0x100,RDS / 4); } SG(8,4); } while (0)
  // loads of the slice two ahead: J1 of them spread over the MFMAs of K steps
  // 1 and 2, the rest over step 3 (after the wait for the next slice)
  constexpr int J1 = PER * 5 / 8;
  constexpr int J1O = (IA + IBP) / 2;  // FP8 ring: an odd slice's loads before its wait
  // the interleave patterns are written for the 256 x 256 tile
  constexpr bool FULL = TM == 4 && TN == 4 && PER == 16;
#define P_MM_LD() do { for (int q_ = 0; q_ < J1; ++q_) { SG(8,3); SG(0x20,1); } SG(8, 32 - 3 * J1); } while (0)
#define P_MM_RD_LD() do { for (int q_ = 0; q_ < PER - J1; ++q_) { SG(8,2); SG(0x100,1); SG(0x20,1); } \
  SG(0x100, RDS - (PER - J1)); SG(8, 16 - 2 * (PER - J1)); } while (0)
// ISSUE: the slice two ahead exists and is loaded into S; NEXT: a next slice
// exists (wait for it, read its first K step)
#define SLICE_BODY(S, S2, s, ca, cb, na, nb, ISSUE, NEXT, MMF, PAT)            \
  do {                                                                         \
    rd(S, 1, f1a, f1b);                                                        \
    rd(S, 2, f2a, f2b);                                                        \
    rd(S, 3, f3a, f3b);                                                        \
    MMF(ca, cb);                                                               \
    if constexpr (PAT) P_MM_RD();                                              \
    SCHED_FENCE();                                                             \
    LGKM_WAIT0();                                                              \
    RAW_BARRIER(); /* every wave has read S */                                 \
    if constexpr (ISSUE) issue_part(cur, S, (s) + 2, 0, J1);                        \
    MMF(f1a, f1b);                                                             \
    MMF(f2a, f2b);                                                             \
    if constexpr (PAT && ISSUE) P_MM_LD();                                     \
    SCHED_FENCE();                                                             \
    if constexpr (NEXT) {                                                      \
      if constexpr (ISSUE) VM_WAIT(J1); else VM_WAIT(0);                       \
      RAW_BARRIER(); /* slice s+1 is in S2 */                                  \
      rd(S2, 0, na, nb);                                                       \
    }                                                                          \
    if constexpr (ISSUE) issue_part(cur, S, (s) + 2, J1, PER);                      \
    MMF(f3a, f3b);                                                             \
    if constexpr (PAT && ISSUE && NEXT) P_MM_RD_LD();                          \
    SCHED_FENCE();                                                             \
  } while (0)

// ring slice s (rows SA, codes half H of SB; the next slice's in NA, half NH
// of NB).  Even s issues the rows of slice s+2 (IA loads, all before its
// wait); odd s also the codes of pair (s+1)/2 + 1 into SB (IA + IBP loads,
// J1O of them before its wait).  The wait for slice s+1 leaves in flight: at
// even s the codes issued by slice s-1 after the rows of slice s+1, and this
// slice's rows; at odd s this slice's first J1O loads (the codes slice s+1
// reads were issued by slice s-2).
#define R4_BODY(s, ODD, SA, SB, H, NA, NB, NH, ca, cb, na, nb)                             \
  do {                                                                                      \
    rd_tag = (s);                                                                           \
    rd4(SA, SB, H, 1, f1a, f1b);                                                            \
    rd4(SA, SB, H, 2, f2a, f2b);                                                            \
    rd4(SA, SB, H, 3, f3a, f3b);                                                            \
    mm(ca, cb);                                                                             \
    SCHED_FENCE();                                                                          \
    LGKM_WAIT0();                                                                           \
    RAW_BARRIER();                                                                          \
    if constexpr (ODD) issue4(cur, SA, (s) + 2, SB, ((s) + 1) / 2 + 1, 0, J1O);             \
    else issue4(cur, SA, (s) + 2, SB, -1, 0, IA);                                           \
    mm(f1a, f1b);                                                                           \
    mm(f2a, f2b);                                                                           \
    SCHED_FENCE();                                                                          \
    if constexpr (ODD) VM_WAIT(J1O); else VM_WAIT(IBP + IA);                                \
    RAW_BARRIER();                                                                          \
    rd4(NA, NB, NH, 0, na, nb);                                                             \
    if constexpr (ODD) issue4(cur, SA, (s) + 2, SB, ((s) + 1) / 2 + 1, J1O, IA + IBP);      \
    mm(f3a, f3b);                                                                           \
    SCHED_FENCE();                                                                          \
  } while (0)
#define R4_LAST(SA, SB, H, ca, cb)                                                          \
  do {                                                                                      \
    rd4(SA, SB, H, 1, f1a, f1b);                                                            \
    rd4(SA, SB, H, 2, f2a, f2b);                                                            \
    rd4(SA, SB, H, 3, f3a, f3b);                                                            \
    mm(ca, cb);                                                                             \
    SCHED_FENCE();                                                                          \
    LGKM_WAIT0();                                                                           \
    RAW_BARRIER();                                                                          \
    mm(f1a, f1b);                                                                           \
    mm(f2a, f2b);                                                                           \
    mm(f3a, f3b);                                                                           \
    SCHED_FENCE();                                                                          \
  } while (0)
#define R4_SLICES()                                                                         \
  do {                                                                                      \
    for (; kt + 4 < cur.nk; kt += 4) {                                                      \
      R4_BODY(kt, false, ra0, pc0, 0, ra1, pc0, 1, f0a, f0b, g0a, g0b);                     \
      R4_BODY(kt + 1, true, ra1, pc0, 1, ra0, pc1, 0, g0a, g0b, f0a, f0b);                  \
      R4_BODY(kt + 2, false, ra0, pc1, 0, ra1, pc1, 1, f0a, f0b, g0a, g0b);                 \
      R4_BODY(kt + 3, true, ra1, pc1, 1, ra0, pc0, 0, g0a, g0b, f0a, f0b);                  \
    }                                                                                       \
    /* 2 or 4 slices left, the first in stages 0 */                                         \
    R4_BODY(kt, false, ra0, pc0, 0, ra1, pc0, 1, f0a, f0b, g0a, g0b);                       \
    if (kt + 2 == cur.nk) {                                                                 \
      R4_LAST(ra1, pc0, 1, g0a, g0b);                                                       \
    } else {                                                                                \
      R4_BODY(kt + 1, true, ra1, pc0, 1, ra0, pc1, 0, g0a, g0b, f0a, f0b);                  \
      R4_BODY(kt + 2, false, ra0, pc1, 0, ra1, pc1, 1, f0a, f0b, g0a, g0b);                 \
      R4_LAST(ra1, pc1, 1, g0a, g0b);                                                       \
    }                                                                                       \
  } while (0)

  // The last part of a split tile to finish adds the partial sums of all its
  // parts into acc (false: other parts are still missing, nothing to store).
  // A tile's S partial slots hold its accumulators in lane order (float4
  // number ((wave * TM * TN + a * TN + b) * 4 + g) * 64 + lane of each slot).
  // The parts may run on different XCDs, whose L2 caches are not coherent
  // with each other, so partials are stored and loaded with device scope
  // (sc1): written through to memory, read from it.  A part's stores are
  // complete before it counts itself in, so the part that counts S - 1 finds
  // every partial in memory.
  auto fixup = [&](const TileAddr &ta) -> bool {
    constexpr uint32_t TILE_B = BM * BNB * 4;  // bytes of one partial
    constexpr int SC1 = 16;                    // cache policy: device scope
    typedef uint32_t u32x4_v __attribute__((ext_vector_type(4)));
    const __amdgpu_buffer_rsrc_t rs =
        make_rsrc(fix_part + (size_t)ta.slot * sp.S * (TILE_B / 16), (uint32_t)sp.S * TILE_B);
    const uint32_t lb = (uint32_t)(wave * TM * TN * 4 * 64 + lane) * 16;
    // the per-instruction constant goes in the scalar offset
#pragma unroll
    for (int a = 0; a < TM; ++a)
#pragma unroll
      for (int b = 0; b < TN; ++b)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x4_v v = {acc[a][b][4 * g], acc[a][b][4 * g + 1], acc[a][b][4 * g + 2],
                             acc[a][b][4 * g + 3]};
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_v, v), rs,
                                                 (uint32_t)ta.part * TILE_B + lb,
                                                 ((a * TN + b) * 4 + g) * 1024, SC1);
        }
    VM_WAIT(0);  // this wave's partial is in memory
    RAW_BARRIER();
    if (tid == 0)
      fix_arrived = __hip_atomic_fetch_add(&fix_cnt[ta.slot], 1, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    if (fix_arrived != sp.S - 1) return false;
    // acc = partial 0 + partial 1 + ... in part order (the own partial is read
    // back too); TN * 4 loads in flight per wave
    for (int q = 0; q < sp.S; ++q) {
#pragma unroll
      for (int a = 0; a < TM; ++a) {
        f32x4_v v[TN][4];
#pragma unroll
        for (int b = 0; b < TN; ++b)
#pragma unroll
          for (int g = 0; g < 4; ++g)
            v[b][g] = __builtin_bit_cast(
                f32x4_v, __builtin_amdgcn_raw_buffer_load_b128(
                             rs, (uint32_t)q * TILE_B + lb, ((a * TN + b) * 4 + g) * 1024, SC1));
#pragma unroll
        for (int b = 0; b < TN; ++b)
#pragma unroll
          for (int g = 0; g < 4; ++g)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              acc[a][b][4 * g + i] = q == 0 ? v[b][g][i] : acc[a][b][4 * g + i] + v[b][g][i];
      }
    }
    if (tid == 0)  // ready for the next launch
      __hip_atomic_store(&fix_cnt[ta.slot], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return true;
  };

  // Persistent: the workgroup walks the work units in steps of Wg (a
  // multiple of the XCD count, so it stays on its XCD's chunk), or takes them
  // from its XCD's queue (LIGHT).  The next unit's first slices are loaded
  // while the current unit's epilogue runs.
  // Queue of XCD x: tile_q[x] counts the tiles handed out (the n-th is the XCD's
  // n-th in the fixed order), tile_q[8 + x] the workgroups done; the last one
  // done puts both back to zero for the next launch.  The counter is taken
  // before the unit's last two slices, whose waits cover its latency.
  const bool dyn = LIGHT && tile_q != nullptr && gridDim.y == 1;
  const int xq = blockIdx.x % NUM_XCD;
  int q_got = 0;  // thread 0: the index taken
  auto q_take = [&]() {
    if (tid == 0)
      q_got = __hip_atomic_fetch_add(&tile_q[xq], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  };
  auto q_done = [&]() {
    if (dyn && tid == 0 &&
        __hip_atomic_fetch_add(&tile_q[NUM_XCD + xq], 1, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT) == Wg / NUM_XCD - 1) {
      __hip_atomic_store(&tile_q[xq], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(&tile_q[NUM_XCD + xq], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  };
  int hw = blockIdx.x;
  if (dyn) {
    q_take();
    if (tid == 0) q_next = q_got;
    __syncthreads();
    hw = q_next * NUM_XCD + xq;  // the unit tile_order places n-th on XCD xq
  }
  Tile tile;
  TileAddr cur;
  if (!map_unit(hw, tile, cur)) {
    q_done();
    return;
  }
  setup(tile, cur);
  if constexpr (RING4) {
    prologue4(cur);
    VM_WAIT(IA + IBP);  // rows of slice 0 and codes of pair 0 are in
    RAW_BARRIER();
    rd4(ra0, pc0, 0, 0, f0a, f0b);
  } else {
    issue(cur, st0, 0);
    issue(cur, st1, 1);
    VM_WAIT(PER);
    RAW_BARRIER();
    rd(st0, 0, f0a, f0b);
  }
  for (;;) {
    // a per-tile copy of the lane id the compiler cannot see through: lane
    // dependent addresses are then recomputed per tile instead of being hoisted
    // out of the tile loop and spilled
    int lane_t = lane;
    asm volatile("" : "+v"(lane_t));
    set_frag_addr(lane_t);
#pragma unroll
    for (int a = 0; a < TM; ++a)
#pragma unroll
      for (int b = 0; b < TN; ++b)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[a][b][i] = 0.f;
    // From here on the wait for slice s+1 lets the J1 loads of slice s+2 that
    // were issued before it stay in flight (the remaining PER - J1 come after).
    // nk is even (K is a multiple of 128 and S divides K / 128); the last pair
    // issues nothing.
    int kt = 0;
    if constexpr (RING4) {
      R4_SLICES();
    } else if (LIGHT && cur.light) {
      for (; kt + 2 < cur.nk; kt += 2) {
        SLICE_BODY(st0, st1, kt, f0a, f0b, g0a, g0b, true, true, mml, false);
        SLICE_BODY(st1, st0, kt + 1, g0a, g0b, f0a, f0b, true, true, mml, false);
      }
      if (dyn) q_take();
      SLICE_BODY(st0, st1, kt, f0a, f0b, g0a, g0b, false, true, mml, false);
      if (dyn && tid == 0) q_next = q_got;  // read after the last slice's barrier
      SLICE_BODY(st1, st0, kt + 1, g0a, g0b, f0a, f0b, false, false, mml, false);
    } else {
      for (; kt + 2 < cur.nk; kt += 2) {
        SLICE_BODY(st0, st1, kt, f0a, f0b, g0a, g0b, true, true, mm, FULL);
        SLICE_BODY(st1, st0, kt + 1, g0a, g0b, f0a, f0b, true, true, mm, FULL);
      }
      if (dyn) q_take();
      SLICE_BODY(st0, st1, kt, f0a, f0b, g0a, g0b, false, true, mm, FULL);
      if (dyn && tid == 0) q_next = q_got;
      SLICE_BODY(st1, st0, kt + 1, g0a, g0b, f0a, f0b, false, false, mm, FULL);
    }
    // Every wave is past the last barrier of the unit, so no wave reads either
    // stage any more: the next unit's first two slices are loaded while the
    // epilogue runs.
    hw = dyn ? q_next * NUM_XCD + xq : hw + Wg;
    Tile nt;
    TileAddr nxt;
    const bool more = map_unit(hw, nt, nxt);
    if (more) {
      setup(nt, nxt);
      if constexpr (RING4) {
        prologue4(nxt);
      } else {
        issue(nxt, st0, 0);
        issue(nxt, st1, 1);
      }
    }
    bool store = true;
    if constexpr (SPLIT) store = cur.part < 0 || fixup(cur);
    if constexpr (W8) {
      // the experts' scales: W1 (or W2) blocks and W3 blocks
      const float s1v = sc1[cur.e], s3v = SWIGLU ? sc3[cur.e] : s1v;
#pragma unroll
      for (int a = 0; a < TM; ++a)
#pragma unroll
        for (int b = 0; b < TN; ++b)
#pragma unroll
          for (int i = 0; i < 16; ++i) acc[a][b][i] *= (SWIGLU && (b & 1)) ? s3v : s1v;
    }
    if (store) dl_epilogue<BM, BNB, SWIGLU>(cur, acc, C, N, plane, act, wave, lane_t);
    if (!more) {
      q_done();
      break;
    }
    VM_WAIT(0);  // both slices (and the epilogue's stores) done
    RAW_BARRIER();
    if constexpr (RING4)
      rd4(ra0, pc0, 0, 0, f0a, f0b);
    else
      rd(st0, 0, f0a, f0b);
    cur = nxt;
  }
#undef SLICE_BODY
#undef R4_BODY
#undef R4_LAST
#undef R4_SLICES
#undef P_MM_LD
#undef P_MM_RD_LD
#undef P_MM_RD
#undef RAW_BARRIER
#undef VM_WAIT
#undef LGKM_WAIT0
#undef SCHED_FENCE
#undef SG
}

// Workgroups that stay resident at once: one per CU for 256-row tiles (128 KB
// of LDS), two for 64-row tiles.
int resident_wgs(int bm) {
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  if (cus[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cus[dev] = n;
  }
  return cus[dev] * (bm == 64 ? 2 : 1);
}

template <int BM, int BNB, bool SWIGLU, bool SPLIT = false, bool GATHER = false, bool TB = false,
          bool W8 = false, bool LIGHT = false>
hipError_t launch_dl(const void *A, const void *B1, const void *B3, void *C,
                     const int32_t *seg_off, const int32_t *seg_end, const int32_t *mtile_off,
                     int G, int N, int K, int ksplit, size_t plane, int act, const FixScratch &fx,
                     hipStream_t s, const int32_t *gperm = nullptr, int gk = 1,
                     uint32_t a_bytes = 0, const float *sc1 = nullptr,
                     const float *sc3 = nullptr, const int32_t *lmid = nullptr,
                     const int32_t *lmt = nullptr, int32_t *tile_q = nullptr) {
  // persistent grid: what stays resident, a multiple of the XCD count
  const int gx = (resident_wgs(BM) / ksplit + NUM_XCD - 1) / NUM_XCD * NUM_XCD;
  const size_t cap = fx.part ? fx.part_bytes / ((size_t)BM * BNB * 4) : 0;
  hipLaunchKernelGGL((grouped_gemm_dl_kernel<BM, BNB, SWIGLU, SPLIT, GATHER, TB, W8, LIGHT>),
                     dim3(gx, ksplit),
                     dim3(GM_THREADS), 0, s, (const bf16_t *)A, (const bf16_t *)B1,
                     (const bf16_t *)B3, C, seg_off, seg_end ? seg_end : seg_off + 1, mtile_off, G,
                     N, K, plane, act, fx.cnt, (f32x4_v *)fx.part,
                     (int)(cap < (size_t)FIX_SLOTS * 16 ? cap : (size_t)FIX_SLOTS * 16), gperm,
                     gk, a_bytes, sc1, sc3, lmid, lmt, tile_q);
  return hipGetLastError();
}

template <typename T, int BM, int BNB, int WM, int WN, bool SWIGLU, bool TB>
hipError_t launch_one(const void *A, const void *B1, const void *B3, void *C,
                      const int32_t *seg_off, const int32_t *mtile_off, int G, int N, int K,
                      int max_mtiles, int act, hipStream_t s, int ksplit = 1,
                      size_t plane = 0) {
  const int cols = SWIGLU ? BNB / 2 : BNB;
  if (ksplit < 1 || (SWIGLU && ksplit != 1) || K % (ksplit * MfmaTraits<T>::BK))
    return hipErrorInvalidValue;
  dim3 grid(((N + cols - 1) / cols) * max_mtiles + NUM_XCD, ksplit);
  hipLaunchKernelGGL((grouped_gemm_kernel<T, BM, BNB, WM, WN, SWIGLU, TB>), grid, dim3(GM_THREADS),
                     0, s, (const T *)A, (const T *)B1, (const T *)B3, C, seg_off, mtile_off, G,
                     N, K, act, plane);
  return hipGetLastError();
}

}  // namespace

size_t fix_part_bytes(long long tiles) {
  // a split uses at most 16 parts of each tail tile, and the kernel's own
  // estimate rules out more than two rounds of parts on 256 workgroups
  const long long parts = tiles * 16 < 512 ? tiles * 16 : 512;
  return (size_t)(parts > 0 ? parts : 0) * 256 * 256 * 4;
}

GemmPlan gemm_plan(int dtype, int d, int d_ff, int d_ff_shared, long long rows_per_expert) {
  GemmPlan p;
  const int q = 128;  // K granule of the direct-to-LDS kernel (pairs of 64-wide slices)
  p.dl1 = dtype == 1 && d % q == 0;
  p.dl2 = dtype == 1 && d_ff % q == 0 && (d_ff_shared == 0 || d_ff_shared % q == 0);
  // 64-row tiles when experts hold few rows (less padding, two workgroups per CU)
  const int bm_dl = rows_per_expert <= 96 ? 64 : 256;
  p.bm1 = p.dl1 ? bm_dl : 128;
  p.bm2 = p.dl2 ? bm_dl : 128;
  return p;
}

bool gemm_gather_ok(int dtype, bool dl, int bm, long long a_bytes) {
  return dtype == 1 && dl && (bm == 64 || bm == 256) && a_bytes + (1LL << 20) < (1LL << 31);
}

namespace {

template <bool TB>
hipError_t gemm_swiglu_t(int dtype, bool dl, int bm, int act, const void *A, const void *W1,
                         const void *W3, void *H, const int32_t *seg_off,
                         const int32_t *mtile_off, int G, int N, int K, int max_mtiles,
                         hipStream_t s, const int32_t *seg_end, const int32_t *gperm, int gk,
                         long long a_bytes, const int32_t *lmid, const int32_t *lmt,
                         int32_t *tile_q) {
  const FixScratch none{nullptr, nullptr, 0};
  if (lmt) {  // 256-row tiles with light tiles for the rows past them
    if (!dl || bm != 256 || !lmid || !seg_end) return hipErrorInvalidValue;
    if (gperm) {
      if (!gemm_gather_ok(dtype, dl, bm, a_bytes)) return hipErrorInvalidValue;
      return launch_dl<256, 256, true, false, true, TB, false, true>(
          A, W1, W3, H, seg_off, seg_end, mtile_off, G, N, K, 1, 0, act, none, s, gperm, gk,
          (uint32_t)a_bytes, nullptr, nullptr, lmid, lmt, tile_q);
    }
    return launch_dl<256, 256, true, false, false, TB, false, true>(
        A, W1, W3, H, seg_off, seg_end, mtile_off, G, N, K, 1, 0, act, none, s, nullptr, 1, 0,
        nullptr, nullptr, lmid, lmt, tile_q);
  }
  if (gperm) {
    if (!gemm_gather_ok(dtype, dl, bm, a_bytes)) return hipErrorInvalidValue;
    if (bm == 64)
      return launch_dl<64, 256, true, false, true, TB>(A, W1, W3, H, seg_off, seg_end, mtile_off,
                                                       G, N, K, 1, 0, act, none, s, gperm, gk,
                                                       (uint32_t)a_bytes);
    return launch_dl<256, 256, true, false, true, TB>(A, W1, W3, H, seg_off, seg_end, mtile_off,
                                                      G, N, K, 1, 0, act, none, s, gperm, gk,
                                                      (uint32_t)a_bytes);
  }
  if (dl && bm == 64)
    return launch_dl<64, 256, true, false, false, TB>(A, W1, W3, H, seg_off, seg_end, mtile_off,
                                                      G, N, K, 1, 0, act, none, s);
  if (dl)
    return launch_dl<256, 256, true, false, false, TB>(A, W1, W3, H, seg_off, seg_end, mtile_off,
                                                       G, N, K, 1, 0, act, none, s);
  if (seg_end) return hipErrorInvalidValue;  // the tiled kernels take whole segments
  if (dtype == 1)
    return launch_one<bf16_t, 128, 128, 2, 2, true, TB>(A, W1, W3, H, seg_off, mtile_off, G, N,
                                                        K, max_mtiles, act, s);
  return launch_one<float, 128, 128, 2, 2, true, TB>(A, W1, W3, H, seg_off, mtile_off, G, N, K,
                                                     max_mtiles, act, s);
}

template <bool TB>
hipError_t gemm_down_t(int dtype, bool dl, int bm, const void *A, const void *W2, void *Y,
                       const int32_t *seg_off, const int32_t *mtile_off, int G, int N, int K,
                       int max_mtiles, int ksplit, size_t plane, const FixScratch &fx,
                       hipStream_t s, const int32_t *seg_end, bool ybf16, const int32_t *lmid,
                       const int32_t *lmt) {
  const int yb = ybf16 ? 1 : 0;
  if (lmt) {  // 256-row tiles with light tiles for the rows past them
    if (!dl || bm != 256 || !lmid || !seg_end) return hipErrorInvalidValue;
    return launch_dl<256, 256, false, false, false, TB, false, true>(
        A, W2, nullptr, Y, seg_off, seg_end, mtile_off, G, N, K, ksplit, plane, yb, fx, s,
        nullptr, 1, 0, nullptr, nullptr, lmid, lmt,
        fx.cnt ? fx.cnt + FIX_SLOTS - TILE_Q_SLOTS : nullptr);
  }
  if (dl && bm == 64)
    return launch_dl<64, 256, false, false, false, TB>(A, W2, nullptr, Y, seg_off, seg_end,
                                                       mtile_off, G, N, K, ksplit, plane, yb,
                                                       fx, s);
  // the last-round split pays for long K only (the kernel's estimate never
  // splits below SPLIT_MIN_K)
  if (dl && ksplit == 1 && K >= SPLIT_MIN_K && fx.part)
    return launch_dl<256, 256, false, true, false, TB>(A, W2, nullptr, Y, seg_off, seg_end,
                                                       mtile_off, G, N, K, 1, 0, yb, fx, s);
  if (dl)
    return launch_dl<256, 256, false, false, false, TB>(A, W2, nullptr, Y, seg_off, seg_end,
                                                        mtile_off, G, N, K, ksplit, plane, yb,
                                                        fx, s);
  if (seg_end) return hipErrorInvalidValue;  // the tiled kernels take whole segments
  if (dtype == 1)
    return launch_one<bf16_t, 128, 128, 2, 2, false, TB>(A, W2, nullptr, Y, seg_off, mtile_off,
                                                         G, N, K, max_mtiles, 0, s, ksplit,
                                                         plane);
  return launch_one<float, 128, 128, 2, 2, false, TB>(A, W2, nullptr, Y, seg_off, mtile_off, G,
                                                      N, K, max_mtiles, 0, s, ksplit, plane);
}

}  // namespace

hipError_t launch_gemm_swiglu(int dtype, bool dl, int bm, int act, const void *A,
                              const void *W1, const void *W3, void *H, const int32_t *seg_off,
                              const int32_t *mtile_off, int G, int N, int K, int max_mtiles,
                              hipStream_t s, const int32_t *seg_end, const int32_t *gperm, int gk,
                              long long a_bytes, bool tb, const int32_t *lmid,
                              const int32_t *lmt, int32_t *tile_q) {
  if (max_mtiles <= 0) return hipSuccess;
  return tb ? gemm_swiglu_t<true>(dtype, dl, bm, act, A, W1, W3, H, seg_off, mtile_off, G, N, K,
                                  max_mtiles, s, seg_end, gperm, gk, a_bytes, lmid, lmt, tile_q)
            : gemm_swiglu_t<false>(dtype, dl, bm, act, A, W1, W3, H, seg_off, mtile_off, G, N, K,
                                   max_mtiles, s, seg_end, gperm, gk, a_bytes, lmid, lmt, tile_q);
}

hipError_t launch_gemm_swiglu_fp8(int act, const void *A, const uint8_t *W1q, const uint8_t *W3q,
                                  const float *s1, const float *s3, void *H,
                                  const int32_t *seg_off, const int32_t *mtile_off, int G, int N,
                                  int K, int max_mtiles, hipStream_t s, const int32_t *gperm,
                                  int gk, long long a_bytes) {
  if (max_mtiles <= 0) return hipSuccess;
  const FixScratch none{nullptr, nullptr, 0};
  if (K % 128) return hipErrorInvalidValue;
  if (gperm) {
    if (!gemm_gather_ok(1, true, 64, a_bytes)) return hipErrorInvalidValue;
    return launch_dl<64, 256, true, false, true, false, true>(A, W1q, W3q, H, seg_off, nullptr,
                                                              mtile_off, G, N, K, 1, 0, act, none,
                                                              s, gperm, gk, (uint32_t)a_bytes, s1,
                                                              s3);
  }
  return launch_dl<64, 256, true, false, false, false, true>(A, W1q, W3q, H, seg_off, nullptr,
                                                             mtile_off, G, N, K, 1, 0, act, none,
                                                             s, nullptr, 1, 0, s1, s3);
}

hipError_t launch_gemm_down_fp8(const void *A, const uint8_t *W2q, const float *s2, void *Y,
                                const int32_t *seg_off, const int32_t *mtile_off, int G, int N,
                                int K, int max_mtiles, int ksplit, size_t plane, hipStream_t s,
                                bool ybf16) {
  if (max_mtiles <= 0) return hipSuccess;
  if (K % (128 * ksplit) || (ybf16 && ksplit != 1)) return hipErrorInvalidValue;
  const FixScratch none{nullptr, nullptr, 0};
  return launch_dl<64, 256, false, false, false, false, true>(A, W2q, nullptr, Y, seg_off, nullptr,
                                                              mtile_off, G, N, K, ksplit, plane,
                                                              ybf16 ? 1 : 0, none, s, nullptr, 1,
                                                              0, s2, nullptr);
}

hipError_t launch_gemm_down(int dtype, bool dl, int bm, const void *A, const void *W2, void *Y,
                            const int32_t *seg_off, const int32_t *mtile_off, int G, int N, int K,
                            int max_mtiles, int ksplit, size_t plane, const FixScratch &fx,
                            hipStream_t s, const int32_t *seg_end, bool ybf16, bool tb,
                            const int32_t *lmid, const int32_t *lmt) {
  if (max_mtiles <= 0) return hipSuccess;
  if (ybf16 && (!dl || ksplit != 1)) return hipErrorInvalidValue;
  return tb ? gemm_down_t<true>(dtype, dl, bm, A, W2, Y, seg_off, mtile_off, G, N, K, max_mtiles,
                                ksplit, plane, fx, s, seg_end, ybf16, lmid, lmt)
            : gemm_down_t<false>(dtype, dl, bm, A, W2, Y, seg_off, mtile_off, G, N, K,
                                 max_mtiles, ksplit, plane, fx, s, seg_end, ybf16, lmid, lmt);
}

}  // namespace moe
