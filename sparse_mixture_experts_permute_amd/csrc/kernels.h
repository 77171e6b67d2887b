// Launchers of the HIP kernels (host-side declarations, internal to the library).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

size_t router_partial_bytes(int T, int d, int E, int esize);
// gate_mode: 0 softmax over the selected logits, 1 softmax over all E (no
// renormalisation), 2 sigmoid of each selected logit, 3 entropy-aware k (an
// unused slot gets idx -1, gate 0)
hipError_t launch_router(int dtype, const void *x, const void *Wg, const float *bias, int T,
                         int d, int E, int k, int gate_mode, int32_t *idx, float *gate,
                         float *logits, float *part, hipStream_t s);

// Weight-only FP8 experts: per-expert E4M3 quantisation of E matrices of n
// elements (dtype 1 bf16, 0 fp32); scale [E] out.
hipError_t launch_quantize_fp8(int dtype, const void *W, int E, size_t n, uint8_t *q,
                               float *scale, hipStream_t s);
// The weight-streaming kernels on FP8 experts (scales s1/s3/s2 [E]); the down
// projection also does the combine (launch_gemv_down_combine).
hipError_t launch_gemv_swiglu_fp8(int rows, int act, const void *x, const int32_t *perm,
                                  int kslots, const uint8_t *W1q, const uint8_t *W3q,
                                  const float *s1, const float *s3, void *H,
                                  const int32_t *seg_off, const int32_t *active,
                                  const int32_t *nactive, int G, int N, int K, int nact,
                                  hipStream_t s);
hipError_t launch_gemv_down_combine_fp8(int rows, const void *Hin, const uint8_t *W2q,
                                        const float *s2, float *Y, const int32_t *seg_off,
                                        const int32_t *active, const int32_t *nactive, int G,
                                        int N, int K, int nact, const int32_t *inv,
                                        const float *gate, int T, int k, void *y, int32_t *cnt,
                                        hipStream_t s);

// Decode steps (T <= 4, T * k <= 64 pairs, E <= 64): the router's scores, then top-k,
// gate and the grouping by expert in one more launch; outputs as
// launch_router + launch_permute (capacity as there; zero: nzero int32
// cleared on the way, may be NULL; part: the router's partial-score scratch).
bool route_permute_tiny_ok(int T, int E, int k);
hipError_t launch_route_permute_tiny(int dtype, const void *x, const void *Wg, const float *bias,
                                     int T, int d, int E, int k, int gate_mode, int capacity,
                                     int bm0, int bm1, float *logits, int32_t *idx, float *gate,
                                     int32_t *counts, int32_t *offsets, int32_t *perm,
                                     int32_t *inv, int32_t *mtiles0, int32_t *mtiles1,
                                     int32_t *shared_seg, int32_t *active, int32_t *zero,
                                     int nzero, float *part, hipStream_t s);

// A single token whose router fits every workgroup (E * d <= 65536, E <= 64):
// the SwiGLU weight-streaming kernel routes it itself.  Each of its
// workgroups computes the token's scores, top-k, gate and grouping (the same
// instructions on the same data, so all reach the same routing) and takes its
// expert from them; workgroup 0 writes the routing outputs as
// launch_route_permute_tiny does (capacity clamped to [0, k] by the caller)
// and clears `zero`.
struct DecodeRoute {
  const void *Wg;
  const float *bias;
  int E, k, gate_mode, capacity, bm0, bm1;
  float *logits;
  int32_t *idx;
  float *gate;
  int32_t *counts, *offsets, *perm, *inv, *mtiles0, *mtiles1, *shared_seg, *active;
  int32_t *zero;
  int nzero;
};
bool route_fused_ok(int T, int d, int E, int k);
// s1 / s3 NULL: bf16 W1 / W3; else FP8 codes with these per-expert scales
hipError_t launch_gemv_swiglu_routed(int act, const void *x, const DecodeRoute &r, const void *W1,
                                     const void *W3, const float *s1, const float *s3, void *H,
                                     int N, int K, hipStream_t s);

int permute_nblocks(int P);
// capacity: pairs an expert keeps (its first ones in pair order); >= T*k keeps
// all.  Dropped pairs (and ids outside [0, E)) get inv = -1.
// zero (may be NULL): nzero int32 set to 0 on the way (the GEMMs' arrival
// counters, see FixScratch).
// mid (may be NULL): split tiling (experts under 512 rows on average).
// mtiles0 is then the prefix of each expert's full 256-row tiles and mtiles1
// of its light 64-row tiles for the rows past them (at most SPLIT_REM_TILES;
// bm0 and bm1 are not used), and mid[e] the row where those rows start
// (offsets[e + 1] when there are none).
constexpr int SPLIT_REM_TILES = 2;
hipError_t launch_permute(const int32_t *idx, int T, int E, int k, int capacity, int bm0,
                          int bm1, int32_t *blk, int32_t *counts, int32_t *offsets,
                          int32_t *perm, int32_t *inv, int32_t *mtiles0, int32_t *mtiles1,
                          int32_t *shared_seg, int32_t *active, int32_t *zero, int nzero,
                          hipStream_t s, int32_t *mid = nullptr);
// xp[s] = x[perm[s] / k] for s < *placed (<= P, read on the device)
hipError_t launch_gather(const void *x, const int32_t *perm, const int32_t *placed, int P, int k,
                         int d, int esize, void *xp, hipStream_t s);

// Which grouped-GEMM kernel serves each projection, and its m-tile height.
struct GemmPlan {
  bool dl1, dl2;  // pipelined direct-to-LDS kernel for the SwiGLU / down GEMM
  int bm1, bm2;   // rows per m-tile of the SwiGLU / down GEMM
};
GemmPlan gemm_plan(int dtype, int d, int d_ff, int d_ff_shared, long long rows_per_expert);
// Scratch of the direct-to-LDS down projection (256-row tiles, K of at least
// SPLIT_MIN_K) for the tiles of its last round, which it splits along K:
// FIX_SLOTS arrival counters (zero before the launch; the kernel leaves them
// zero) and part_bytes of fp32 partial tiles (no split when part is NULL).
// Launches on one stream may share it.
constexpr int FIX_SLOTS = 1024;
// The last TILE_Q_SLOTS of those counters are the per-XCD tile queues of the
// 256-row launches with light tiles (zero before the launch, left zero).
constexpr int TILE_Q_SLOTS = 16;
constexpr int SPLIT_MIN_K = 4864;
struct FixScratch {
  int32_t *cnt;
  void *part;
  size_t part_bytes;
};
// Partial-tile bytes that let every split the kernel would choose go ahead
// for a GEMM of at most `tiles` output tiles.
size_t fix_part_bytes(long long tiles);
// act: 0 SiLU(W1 a) * (W3 a), 1 sigmoid(W1 a) * (W3 a)
// tb: the weights are [K][N] per expert (in x out, A W) instead of [N][K]
// lmid / lmt (256-row direct-to-LDS tiles only): the same launch also serves
// each expert's rows from lmid[e] to seg_end[e] as light 64-row tiles (lmt:
// their prefix over the experts) placed after its full tiles, which end at
// lmid[e]; tile_q (with lmt; NULL: fixed order): 2 * 8 counters, zero before
// the launch and left zero, through which each XCD's workgroups take its tiles
// (the down projection uses the last TILE_Q_SLOTS of fx.cnt)
// seg_end (direct-to-LDS kernel only; NULL: seg_off + 1): expert e's rows
// are seg_off[e] .. seg_end[e] - 1, with mtile_off the prefix of its tiles.
// gperm (gemm_gather_ok only): A is x itself (a_bytes bytes) and grouped row s
// is read from x row gperm[s] / gk inside the GEMM (no gathered copy).
bool gemm_gather_ok(int dtype, bool dl, int bm, long long a_bytes);
hipError_t launch_gemm_swiglu(int dtype, bool dl, int bm, int act, const void *A,
                              const void *W1, const void *W3, void *H, const int32_t *seg_off,
                              const int32_t *mtile_off, int G, int N, int K, int max_mtiles,
                              hipStream_t s, const int32_t *seg_end = nullptr,
                              const int32_t *gperm = nullptr, int gk = 1, long long a_bytes = 0,
                              bool tb = false, const int32_t *lmid = nullptr,
                              const int32_t *lmt = nullptr, int32_t *tile_q = nullptr);
// ksplit > 1 (direct-to-LDS kernel only): every tile's K is split in ksplit
// equal ranges whose fp32 partials go to planes `plane` elements apart (for
// batches with few tiles; the last-round split then stays off).
// ybf16 (direct-to-LDS kernel, one plane): Y is stored as bf16, else fp32.
hipError_t launch_gemm_down(int dtype, bool dl, int bm, const void *A, const void *W2, void *Y,
                            const int32_t *seg_off, const int32_t *mtile_off, int G, int N, int K,
                            int max_mtiles, int ksplit, size_t plane, const FixScratch &fx,
                            hipStream_t s, const int32_t *seg_end = nullptr, bool ybf16 = false,
                            bool tb = false, const int32_t *lmid = nullptr,
                            const int32_t *lmt = nullptr);

// The 64-row tiled GEMMs on FP8 (E4M3) expert weights [N][K] with per-expert
// scales (s1 / s3 / s2 [E]); arguments otherwise as launch_gemm_swiglu /
// launch_gemm_down (K a multiple of 128; the down projection's K planes each
// a multiple of 128).
hipError_t launch_gemm_swiglu_fp8(int act, const void *A, const uint8_t *W1q, const uint8_t *W3q,
                                  const float *s1, const float *s3, void *H,
                                  const int32_t *seg_off, const int32_t *mtile_off, int G, int N,
                                  int K, int max_mtiles, hipStream_t s, const int32_t *gperm,
                                  int gk, long long a_bytes);
hipError_t launch_gemm_down_fp8(const void *A, const uint8_t *W2q, const float *s2, void *Y,
                                const int32_t *seg_off, const int32_t *mtile_off, int G, int N,
                                int K, int max_mtiles, int ksplit, size_t plane, hipStream_t s,
                                bool ybf16);

// Weight-streaming grouped GEMMs for few rows per expert (bf16 only).
bool skinny_ok(int N, int K);
// vector-ALU weight streaming for experts holding at most `rows` (<= 4) rows
bool gemv_ok(int N, int K);
// nact: the number of active experts when the host knows it (a single token
// has exactly k), else 0; it sets how many workgroups share the columns
hipError_t launch_gemv_swiglu(int rows, int act, const void *x, const int32_t *perm, int kslots,
                              const void *W1, const void *W3, void *H, const int32_t *seg_off,
                              const int32_t *active, const int32_t *nactive, int G, int N, int K,
                              int nact, hipStream_t s);
hipError_t launch_gemv_down(int rows, const void *Hin, const void *W2, float *Y,
                            const int32_t *seg_off, const int32_t *active,
                            const int32_t *nactive, int G, int N, int K, int nact,
                            hipStream_t s);
// launch_gemv_down that also writes y [T][N] (bf16) as launch_combine would
// (no shared expert): the last workgroup of each column block combines the
// T tokens' k outputs.  cnt: FIX_SLOTS counters, zero before the launch (the
// kernel leaves them zero).
hipError_t launch_gemv_down_combine(int rows, const void *Hin, const void *W2, float *Y,
                                    const int32_t *seg_off, const int32_t *active,
                                    const int32_t *nactive, int G, int N, int K, int nact,
                                    const int32_t *inv, const float *gate, int T, int k, void *y,
                                    int32_t *cnt, hipStream_t s);
// One token's down projection and combine (no shared expert, k <= 64): one
// workgroup per block of output columns covers every active expert, forms y
// [N] (bf16) in LDS as launch_combine would, and writes no partial outputs.
// s2 NULL: bf16 W2; else FP8 codes with these per-expert scales.
bool gemv_token_ok(int N, int K, int k);
hipError_t launch_gemv_down_token(const void *H, const void *W2, const float *s2,
                                  const int32_t *seg_off, const int32_t *active,
                                  const int32_t *nactive, int N, int K, const int32_t *inv,
                                  const float *gate, int k, void *y, hipStream_t s);
// [K][N] (in x out) weights, up to four rows per expert per pass (more rows
// loop): vector-ALU weight streaming, H bf16 / Y fp32 as the gemv kernels
bool gemv_t_ok(int N, int K);
// one token routed inside the [K][N] SwiGLU kernel (route_fused_ok, gemv_t_ok)
hipError_t launch_gemv_t_swiglu_routed(int act, const void *x, const DecodeRoute &r,
                                       const void *W1, const void *W3, void *H, int N, int K,
                                       hipStream_t s);
hipError_t launch_gemv_t_swiglu(int rows, int act, const void *x, const int32_t *perm,
                                int kslots, const void *W1, const void *W3, void *H,
                                const int32_t *seg_off, const int32_t *active,
                                const int32_t *nactive, int G, int N, int K, hipStream_t s);
// the down projection may split K into ksplit parts (fp32 planes `plane`
// floats apart, added in order by the combine); gemv_t_down_splits: the parts
// that give every CU a workgroup, at most max_split
int gemv_t_down_splits(int G, int N, int K, int max_split);
hipError_t launch_gemv_t_down(int rows, const void *Hin, const void *W2, float *Y,
                              const int32_t *seg_off, const int32_t *active,
                              const int32_t *nactive, int G, int N, int K, int ksplit,
                              size_t plane, hipStream_t s);
hipError_t launch_skinny_swiglu(int mb, int act, const void *x, const int32_t *perm, int kslots,
                                const void *W1, const void *W3, void *H,
                                const int32_t *seg_off, const int32_t *active,
                                const int32_t *nactive, int G, int N, int K, hipStream_t s);
hipError_t launch_skinny_down(int mb, const void *Hin, const void *W2, float *Y,
                              const int32_t *seg_off, const int32_t *active,
                              const int32_t *nactive, int G, int N, int K, hipStream_t s);

// Yp holds nsplit planes of `plane` floats each (summed in order), or with
// yp_bf16 one plane of bf16; a pair with inv < 0 (dropped by a capacity
// limit) contributes nothing.
hipError_t launch_combine(int dtype, const void *Yp, int nsplit, size_t plane, const float *Ys,
                          const int32_t *inv, const float *gate, int T, int k, int d, void *y,
                          hipStream_t s, bool yp_bf16 = false);

}  // namespace moe
