// Grouping of (token, slot) pairs by expert: histogram -> prefix scan ->
// stable scatter ("Chapter 10 MoE", section 10.4 groups an expert's tokens in
// ascending order; the numpy listing of "Trillion-parameter MoE ... 7 expert
// configs measured" builds the same per-expert row lists).
//
// The result is the stable counting sort of the flat pair ids p = t*k + j by
// expert, independent of scheduling: ranks come from block-local histograms
// plus block-prefix bases and from in-wave ballots, never from the order in
// which atomics land.
//
//   hist    : block b counts the experts of pairs [256b, 256b+256) -> blk[b][e]
//   scan    : one block turns blk[][] into per-block rank bases (1024 threads
//             over (block range, expert)), counts, offsets and the m-tile
//             prefix used by the grouped GEMM tile maps
//   scatter : block b re-reads its pairs; a pair's rank among its expert's
//             pairs is base[b][e] + (pairs of e in earlier waves of b) + (rank
//             in wave), and its slot is offsets[e] + rank
//
// Under a capacity limit ("Mistral 8x7B SMoE architecture deep dive", section
// 2.4) an expert keeps the pairs of rank < capacity (its first ones in pair
// order); counts, offsets and the tile prefixes cover the kept pairs, and a
// dropped pair gets inv = -1.
#include "common.h"
#include "kernels.h"

namespace moe {

namespace {

constexpr int PM_CHUNK = 256;  // pairs per block == threads per block

// Split tiling of an expert's c kept rows (large batches): 256-row tiles for
// the bulk and, when c runs at most 128 rows past a multiple of 256, 64-row
// tiles for that remainder, served by a second GEMM launch (a 256-row tile
// for a few rows would cost a whole tile).  main / rem: tiles of each kind;
// main_rows: rows the 256-row tiles cover.
__device__ __forceinline__ void tile_split(int c, int &main, int &rem, int &main_rows) {
  const int r = c & 255;
  if (c < 256 || r == 0 || r > 128) {
    main = (c + 255) >> 8;
    rem = 0;
    main_rows = c;
  } else {
    main = c >> 8;
    rem = (r + 63) >> 6;
    main_rows = c - r;
  }
}

__global__ __launch_bounds__(PM_CHUNK) void permute_hist_kernel(const int32_t *__restrict__ idx,
                                                                int P, int E,
                                                                int32_t *__restrict__ blk) {
  __shared__ int h[256];
  const int tid = threadIdx.x;
  if (tid < E) h[tid] = 0;
  __syncthreads();
  const int p = blockIdx.x * PM_CHUNK + tid;
  if (p < P) {
    const int e = idx[p];
    if ((unsigned)e < (unsigned)E) atomicAdd(&h[e], 1);  // out-of-range ids are not placed
  }
  __syncthreads();
  if (tid < E) blk[(size_t)blockIdx.x * E + tid] = h[tid];
}

// One block of 1024 threads.  The per-block counts blk[b][e] are summed and
// turned into rank bases by thread (q, e): expert e (of EP, E rounded up to a
// power of two) and part q of the blocks (Q = 1024 / EP contiguous parts),
// with eight loads in flight; the parts' sums give each part its starting rank
// and each expert its total.  Then threads e < 256 scan over the experts.
constexpr int SC_THREADS = 1024;
__global__ __launch_bounds__(SC_THREADS) void permute_scan_kernel(
    int32_t *__restrict__ blk, int nb, int E, int P, int T, int capacity, int bm0, int bm1,
    int32_t *__restrict__ counts, int32_t *__restrict__ offsets, int32_t *__restrict__ mtiles0,
    int32_t *__restrict__ mtiles1, int32_t *__restrict__ shared_seg,
    int32_t *__restrict__ active, int32_t *__restrict__ zero, int nzero,
    int32_t *__restrict__ mid) {
  __shared__ int s0[256], s1[256], s2[256], s3[256], tot[256];
  __shared__ int psum[SC_THREADS];
  const int tid = threadIdx.x;
  for (int i = tid; i < nzero; i += SC_THREADS) zero[i] = 0;
  int EP = 1;
  while (EP < E) EP <<= 1;
  const int Q = SC_THREADS / EP, pe = tid % EP, q = tid / EP;
  const int R = (nb + Q - 1) / Q;
  const int b0 = q * R, b1 = min(nb, b0 + R);
  int sum = 0;
  if (pe < E) {
    for (int b = b0; b < b1; b += 8) {
      int v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = b + i < b1 ? blk[(size_t)(b + i) * E + pe] : 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) sum += v[i];
    }
  }
  psum[tid] = sum;
  __syncthreads();
  if (pe < E) {
    // rank of the part's first pair among the expert's pairs, then the
    // parts' blocks get their running bases
    int run = 0;
    for (int q2 = 0; q2 < q; ++q2) run += psum[q2 * EP + pe];
    if (q == 0) {
      int t = 0;
      for (int q2 = 0; q2 < Q; ++q2) t += psum[q2 * EP + pe];
      tot[pe] = t;
    }
    for (int b = b0; b < b1; b += 8) {
      int v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = b + i < b1 ? blk[(size_t)(b + i) * E + pe] : 0;
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (b + i < b1) {
          blk[(size_t)(b + i) * E + pe] = run;
          run += v[i];
        }
    }
  }
  __syncthreads();
  const int e = tid;
  const int total = e < E ? min(tot[e], capacity) : 0;  // pairs the expert keeps
  // m-tiles: of bm0 / bm1 rows, or (mid != NULL) the split tiling's 256-row
  // and 64-row tiles
  int t0 = (total + bm0 - 1) / bm0, t1 = (total + bm1 - 1) / bm1, mrows = total;
  if (mid) tile_split(total, t0, t1, mrows);
  if (e < 256) {
    s0[e] = total;
    s1[e] = e < E ? t0 : 0;
    s2[e] = e < E ? t1 : 0;
    s3[e] = (e < E && total > 0) ? 1 : 0;
  }
  __syncthreads();
  // inclusive Hillis-Steele scans over the experts (256 entries)
  for (int off = 1; off < 256; off <<= 1) {
    int a0 = 0, a1 = 0, a2 = 0, a3 = 0;
    if (e < 256 && e >= off) {
      a0 = s0[e - off];
      a1 = s1[e - off];
      a2 = s2[e - off];
      a3 = s3[e - off];
    }
    __syncthreads();
    if (e < 256) {
      s0[e] += a0;
      s1[e] += a1;
      s2[e] += a2;
      s3[e] += a3;
    }
    __syncthreads();
  }
  // compact list of the experts that received pairs; active[E] = their number
  if (e < E && total > 0) active[s3[e] - 1] = e;
  if (e == 0) active[E] = s3[255];
  if (e < E) {
    counts[e] = total;
    offsets[e] = s0[e] - total;
    mtiles0[e] = s1[e] - t0;
    mtiles1[e] = s2[e] - t1;
    if (mid) mid[e] = s0[e] - total + mrows;
  }
  if (e == 0) {
    offsets[E] = s0[255];  // kept pairs (== P when nothing is dropped)
    mtiles0[E] = s1[255];
    mtiles1[E] = s2[255];
    // the shared expert is one segment of all T tokens
    shared_seg[0] = 0;
    shared_seg[1] = T;
    shared_seg[2] = 0;
    shared_seg[3] = (T + bm0 - 1) / bm0;
    shared_seg[4] = 0;
    shared_seg[5] = (T + bm1 - 1) / bm1;
    shared_seg[6] = 0;  // the shared expert as a one-entry active list: {0}, count 1
    shared_seg[7] = 1;
  }
}

__global__ __launch_bounds__(PM_CHUNK) void permute_scatter_kernel(
    const int32_t *__restrict__ idx, int P, int E, int capacity, const int32_t *__restrict__ base,
    const int32_t *__restrict__ offsets, int32_t *__restrict__ perm, int32_t *__restrict__ inv) {
  __shared__ int wc[PM_CHUNK / kWave][256];
  const int tid = threadIdx.x, w = tid / kWave, lane = lane_id();
  for (int i = tid; i < (PM_CHUNK / kWave) * 256; i += PM_CHUNK) (&wc[0][0])[i] = 0;
  __syncthreads();
  const int p = blockIdx.x * PM_CHUNK + tid;
  const int ev = p < P ? idx[p] : -1;
  const bool valid = (unsigned)ev < (unsigned)E;
  const int e = valid ? ev : 0;
  // lanes holding the same expert: intersect ballots over the 8 bits of e
  uint64_t same = __ballot(valid);
#pragma unroll
  for (int bit = 0; bit < 8; ++bit) {
    uint64_t ones = __ballot(valid && ((e >> bit) & 1));
    same &= ((e >> bit) & 1) ? ones : ~ones;
  }
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
  const int rank = __popcll(same & below);
  if (valid && rank == 0) wc[w][e] = __popcll(same);
  __syncthreads();
  if (valid) {
    int r = base[(size_t)blockIdx.x * E + e] + rank;
    for (int w2 = 0; w2 < w; ++w2) r += wc[w2][e];
    if (r < capacity) {
      const int pos = offsets[e] + r;
      perm[pos] = p;
      inv[p] = pos;
    } else {
      inv[p] = -1;
    }
  } else if (p < P) {
    inv[p] = -1;
  }
}

// Small batches: histogram, scan and stable scatter in one workgroup (one
// launch instead of three).  Pairs are processed in order in chunks of 1024;
// within a chunk a pair's slot is cursor[e] + (pairs of e in earlier waves of
// the chunk) + (rank among equal experts inside its wave); cursor[e] then
// advances by the chunk's count.  Same result as the three-kernel path.
constexpr int PS_THREADS = 1024;
constexpr int PS_WAVES = PS_THREADS / kWave;

__global__ __launch_bounds__(PS_THREADS) void permute_small_kernel(
    const int32_t *__restrict__ idx, int P, int E, int T, int capacity, int bm0, int bm1,
    int32_t *__restrict__ counts, int32_t *__restrict__ offsets, int32_t *__restrict__ perm,
    int32_t *__restrict__ inv, int32_t *__restrict__ mtiles0, int32_t *__restrict__ mtiles1,
    int32_t *__restrict__ shared_seg, int32_t *__restrict__ active, int32_t *__restrict__ zero,
    int nzero, int32_t *__restrict__ mid) {
  // hist: pairs per expert; koff: kept-pair offsets (scanned in place);
  // rk: rank of the next pair of each expert
  __shared__ int hist[256], koff[256], rk[256], s1[256], s2[256], s3[256];
  __shared__ int wc[PS_WAVES][256];
  const int tid = threadIdx.x, w = tid / kWave, lane = lane_id();
  for (int i = tid; i < nzero; i += PS_THREADS) zero[i] = 0;
  if (tid < 256) hist[tid] = 0;
  __syncthreads();
  for (int p = tid; p < P; p += PS_THREADS) {
    const int e = idx[p];
    if ((unsigned)e < (unsigned)E) atomicAdd(&hist[e], 1);
  }
  __syncthreads();
  if (tid < 256) {
    const int c = tid < E ? min(hist[tid], capacity) : 0;  // kept pairs
    int t0 = (c + bm0 - 1) / bm0, t1 = (c + bm1 - 1) / bm1, mrows = c;
    if (mid) tile_split(c, t0, t1, mrows);
    koff[tid] = c;
    rk[tid] = 0;
    s1[tid] = tid < E ? t0 : 0;
    s2[tid] = tid < E ? t1 : 0;
    s3[tid] = (tid < E && c > 0) ? 1 : 0;
  }
  __syncthreads();
  for (int off = 1; off < 256; off <<= 1) {  // inclusive scans over the experts
    int a0 = 0, a1 = 0, a2 = 0, a3 = 0;
    if (tid < 256 && tid >= off) {
      a0 = koff[tid - off];
      a1 = s1[tid - off];
      a2 = s2[tid - off];
      a3 = s3[tid - off];
    }
    __syncthreads();
    if (tid < 256) {
      koff[tid] += a0;
      s1[tid] += a1;
      s2[tid] += a2;
      s3[tid] += a3;
    }
    __syncthreads();
  }
  if (tid < E) {
    const int c = min(hist[tid], capacity);
    int t0 = (c + bm0 - 1) / bm0, t1 = (c + bm1 - 1) / bm1, mrows = c;
    if (mid) tile_split(c, t0, t1, mrows);
    counts[tid] = c;
    offsets[tid] = koff[tid] - c;
    mtiles0[tid] = s1[tid] - t0;
    mtiles1[tid] = s2[tid] - t1;
    if (mid) mid[tid] = koff[tid] - c + mrows;
    if (c > 0) active[s3[tid] - 1] = tid;
  }
  if (tid == 0) {
    offsets[E] = koff[255];  // inclusive scan: the number of kept pairs
    mtiles0[E] = s1[255];
    mtiles1[E] = s2[255];
    active[E] = s3[255];
    shared_seg[0] = 0;
    shared_seg[1] = T;
    shared_seg[2] = 0;
    shared_seg[3] = (T + bm0 - 1) / bm0;
    shared_seg[4] = 0;
    shared_seg[5] = (T + bm1 - 1) / bm1;
    shared_seg[6] = 0;
    shared_seg[7] = 1;
  }
  __syncthreads();
  if (tid < 256) koff[tid] -= (tid < E ? min(hist[tid], capacity) : 0);  // exclusive
  __syncthreads();
  for (int c0 = 0; c0 < P; c0 += PS_THREADS) {
    for (int i = tid; i < PS_WAVES * 256; i += PS_THREADS) (&wc[0][0])[i] = 0;
    __syncthreads();
    const int p = c0 + tid;
    const int ev = p < P ? idx[p] : -1;
    const bool valid = (unsigned)ev < (unsigned)E;
    const int e = valid ? ev : 0;
    uint64_t same = __ballot(valid);
#pragma unroll
    for (int bit = 0; bit < 8; ++bit) {
      const uint64_t ones = __ballot(valid && ((e >> bit) & 1));
      same &= ((e >> bit) & 1) ? ones : ~ones;
    }
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
    const int rank = __popcll(same & below);
    if (valid && rank == 0) wc[w][e] = __popcll(same);
    __syncthreads();
    if (valid) {
      int r = rk[e] + rank;
      for (int w2 = 0; w2 < w; ++w2) r += wc[w2][e];
      if (r < capacity) {
        const int pos = koff[e] + r;
        perm[pos] = p;
        inv[p] = pos;
      } else {
        inv[p] = -1;
      }
    } else if (p < P) {
      inv[p] = -1;
    }
    __syncthreads();
    if (tid < E) {
      int add = 0;
      for (int w2 = 0; w2 < PS_WAVES; ++w2) add += wc[w2][tid];
      rk[tid] += add;
    }
    __syncthreads();
  }
}

// Xp[s][:] = x[perm[s] / k][:]; one block copies 4 rows with 16-byte accesses.
// Rows of the placed pairs only: *placed (offsets[E]) is below P when a
// capacity limit dropped pairs.
__global__ __launch_bounds__(256) void gather_rows_kernel(const uint4 *__restrict__ x,
                                                          const int32_t *__restrict__ perm,
                                                          const int32_t *__restrict__ placed,
                                                          int k, int rowq,
                                                          uint4 *__restrict__ xp) {
  const int r0 = blockIdx.x * 4;
  const int P = *placed;
  for (int r = r0; r < r0 + 4 && r < P; ++r) {
    const size_t src = (size_t)(perm[r] / k) * rowq;
    const size_t dst = (size_t)r * rowq;
    for (int q = threadIdx.x; q < rowq; q += 256) xp[dst + q] = x[src + q];
  }
}

}  // namespace

int permute_nblocks(int P) { return (P + PM_CHUNK - 1) / PM_CHUNK; }

hipError_t launch_permute(const int32_t *idx, int T, int E, int k, int capacity, int bm0,
                          int bm1, int32_t *blk, int32_t *counts, int32_t *offsets,
                          int32_t *perm, int32_t *inv, int32_t *mtiles0, int32_t *mtiles1,
                          int32_t *shared_seg, int32_t *active, int32_t *zero, int nzero,
                          hipStream_t s, int32_t *mid) {
  const int P = T * k;
  if (!zero) nzero = 0;
  const int cap = capacity < 0 || capacity > P ? P : capacity;
  if (P <= 8 * PS_THREADS) {
    hipLaunchKernelGGL(permute_small_kernel, dim3(1), dim3(PS_THREADS), 0, s, idx, P, E, T, cap,
                       bm0, bm1, counts, offsets, perm, inv, mtiles0, mtiles1, shared_seg,
                       active, zero, nzero, mid);
    return hipGetLastError();
  }
  const int nb = permute_nblocks(P);
  hipLaunchKernelGGL(permute_hist_kernel, dim3(nb), dim3(PM_CHUNK), 0, s, idx, P, E, blk);
  hipLaunchKernelGGL(permute_scan_kernel, dim3(1), dim3(SC_THREADS), 0, s, blk, nb, E, P, T, cap,
                     bm0, bm1, counts, offsets, mtiles0, mtiles1, shared_seg, active, zero,
                     nzero, mid);
  hipLaunchKernelGGL(permute_scatter_kernel, dim3(nb), dim3(PM_CHUNK), 0, s, idx, P, E, cap, blk,
                     offsets, perm, inv);
  return hipGetLastError();
}

hipError_t launch_gather(const void *x, const int32_t *perm, const int32_t *placed, int P, int k,
                         int d, int esize, void *xp, hipStream_t s) {
  const int rowq = d * esize / 16;
  hipLaunchKernelGGL(gather_rows_kernel, dim3((P + 3) / 4), dim3(256), 0, s,
                     (const uint4 *)x, perm, placed, k, rowq, (uint4 *)xp);
  return hipGetLastError();
}

}  // namespace moe
