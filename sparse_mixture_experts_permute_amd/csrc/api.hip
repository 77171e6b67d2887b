// C ABI of the MoE layer: argument checks, workspace layout and the launch
// sequence route -> permute -> gather -> grouped SwiGLU GEMM -> grouped down
// GEMM -> combine, all enqueued on the caller's stream with no host sync.
#include <string.h>

#include <algorithm>
#include <cmath>
#include <mutex>

#include "../../include/moe_mi355x.h"
#include "kernels.h"

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

enum Field {
  F_LOGITS, F_IDX, F_GATE, F_COUNTS, F_OFFSETS, F_PERM, F_INV, F_MT0, F_MT1, F_SHSEG, F_ACT,
  F_MID, F_FIXC, F_FIXP, F_RPART, F_BLK, F_XP, F_H, F_YP, F_HS, F_YS, F_COUNT
};

struct Layout {
  size_t off[F_COUNT];
  size_t total;
};

bool dims_ok(int T, int d, int d_ff, int E, int k, int dffs) {
  if (T < 0 || E < 1 || E > 256 || k < 1 || k > E) return false;
  if (d < 64 || d % 64 || d_ff < 64 || d_ff % 64) return false;
  if (dffs < 0 || dffs % 64) return false;
  if ((long long)T * k >= (1LL << 31)) return false;
  if ((long long)T * k * (long long)(d > d_ff ? d : d_ff) >= (1LL << 40)) return false;
  // one expert's weight matrix is addressed with 32-bit byte offsets
  if ((long long)d * d_ff >= (1LL << 31) || (long long)d * dffs >= (1LL << 31)) return false;
  return true;
}

size_t esize(int dtype) { return dtype == MOE_BF16 ? 2 : 4; }

// The kernels move tensors 16 bytes at a time (x, weights, y) and fp32 / int32
// arrays 4 bytes at a time; a null pointer passes (checked separately).
bool al16(const void *p) { return ((uintptr_t)p & 15) == 0; }
bool al4(const void *p) { return ((uintptr_t)p & 3) == 0; }

// Most output tiles a down projection that may split its last round can have
// (0: none can); sizes the scratch of that split.
long long dl_tiles(const moe::GemmPlan &plan, int T, int k, int E, int d, int d_ff, int dffs) {
  if (!plan.dl2 || plan.bm2 != 256) return 0;
  const long long P = (long long)T * k;
  long long t = 0;
  if (d_ff >= moe::SPLIT_MIN_K) t = (long long)((d + 255) / 256) * ((P + 255) / 256 + E);
  if (dffs >= moe::SPLIT_MIN_K) {
    const long long ts = (long long)((d + 255) / 256) * ((T + 255) / 256);
    t = ts > t ? ts : t;
  }
  return t;
}

int down_splits(const moe::GemmPlan &plan, int T, int k, int E, int d, int d_ff);

Layout layout(int T, int d, int d_ff, int E, int k, int dffs, int dtype) {
  Layout L;
  const moe::GemmPlan plan = moe::gemm_plan(dtype, d, d_ff, dffs, ((long long)T * k + E - 1) / E);
  const long long tiles = dl_tiles(plan, T, k, E, d, d_ff, dffs);
  const int ksplit = down_splits(plan, T, k, E, d, d_ff);
  const size_t P = (size_t)T * k, es = esize(dtype);
  const size_t nb = (size_t)moe::permute_nblocks((int)P);
  size_t sz[F_COUNT] = {};
  sz[F_LOGITS] = (size_t)T * E * 4;
  sz[F_IDX] = P * 4;
  sz[F_GATE] = P * 4;
  sz[F_COUNTS] = (size_t)E * 4;
  sz[F_OFFSETS] = (size_t)(E + 1) * 4;
  sz[F_PERM] = P * 4;
  sz[F_INV] = P * 4;
  sz[F_MT0] = (size_t)(E + 1) * 4;
  sz[F_MT1] = (size_t)(E + 1) * 4;
  sz[F_SHSEG] = 8 * 4;
  sz[F_ACT] = (size_t)(E + 1) * 4;
  sz[F_MID] = (size_t)E * 4;
  sz[F_FIXC] = (size_t)moe::FIX_SLOTS * 4;  // arrival counters (cleared by each forward)
  sz[F_FIXP] = moe::fix_part_bytes(tiles);
  sz[F_RPART] = moe::router_partial_bytes(T, d, E, (int)es);
  sz[F_BLK] = nb * E * 4;
  sz[F_XP] = P * d * es;
  sz[F_H] = P * d_ff * es;
  sz[F_YP] = (size_t)ksplit * P * d * 4;
  sz[F_HS] = (size_t)T * dffs * es;
  sz[F_YS] = dffs ? (size_t)T * d * 4 : 0;
  size_t o = 0;
  for (int f = 0; f < F_COUNT; ++f) {
    L.off[f] = o;
    o += align_up(sz[f]);
  }
  L.total = o;
  return L;
}

// Device check, cached per device id.
int device_ok() {
  static int state[64];  // 0 unknown, 1 ok, 2 bad
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return MOE_EDEVICE;
  if (dev < 64 && state[dev]) return state[dev] == 1 ? MOE_OK : MOE_EDEVICE;
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return MOE_EDEVICE;
  const bool ok = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (dev < 64) state[dev] = ok ? 1 : 2;
  return ok ? MOE_OK : MOE_EDEVICE;
}

int launched(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ELAUNCH; }

// K planes of the tiled down projection: a batch with fewer tiles than one
// round of the persistent kernel (256 workgroups of 256-row tiles, 512 of
// 64-row tiles on 256 CUs) would leave most CUs idle, so every tile's K is
// split until a round is full, and the combine adds the partial planes in a
// fixed order (cheaper there than the kernel's own last-round split, whose
// last part reads the other parts back).  From one round on, that last-round
// split serves instead.
int down_splits(const moe::GemmPlan &plan, int T, int k, int E, int d, int d_ff) {
  if (!plan.dl2) {
    // the register-staged kernel (128 x 128 tiles, two workgroups per CU):
    // K parts of a multiple of 64 until the grid covers every CU twice
    const long long P = (long long)T * k;
    const long long active = P < E ? P : E;
    const long long mt_floor = (P + 127) / 128;
    const long long wgs = (active > mt_floor ? active : mt_floor) * ((d + 127) / 128);
    int S = 1;
    while (wgs * S < 512 && S < 16 && d_ff % (64 * S * 2) == 0) S *= 2;
    return S;
  }
  const long long P = (long long)T * k;
  const long long active = P < E ? P : E;  // experts that can hold rows
  const long long mt_floor = (P + plan.bm2 - 1) / plan.bm2;
  const long long mt = active > mt_floor ? active : mt_floor;
  const long long wgs = mt * ((d + 255) / 256);
  const long long round = plan.bm2 == 64 ? 512 : 256;
  int S = 1;
  while (wgs * S < round && S < 16 && d_ff % (128 * S * 2) == 0) S *= 2;  // K parts of 128
  return S;
}

// Row blocks of 16 that one pass of the weight-streaming kernel covers.
int skinny_mb(long long rows) { return rows <= 12 ? 1 : rows <= 24 ? 2 : 4; }

// The weight-streaming kernels serve the routed experts when they average one
// row each (single-token decode: they also fold the row gather into the first
// GEMM) and the shared expert up to 64 tokens; the tiled kernels (64-row tiles
// for small batches, split K for the down projection) serve everything else.
// Up to four tokens (at most four rows on any expert) the vector-ALU kernels
// stream the weights; beyond that the matrix-core ones do.
struct SkinnyPlan {
  bool routed, shared, gemv, gemv_shared;
  int mb, mb_shared;
};
SkinnyPlan skinny_plan(int dtype, int T, int k, int E, int d, int d_ff, int dffs) {
  SkinnyPlan p{};
  if (dtype != MOE_BF16) return p;
  const long long avg = ((long long)T * k + E - 1) / E;
  p.routed = avg <= 1 && moe::skinny_ok(d_ff, d) && moe::skinny_ok(d, d_ff);
  p.gemv = p.routed && T <= 4 && moe::gemv_ok(d_ff, d) && moe::gemv_ok(d, d_ff);
  p.mb = skinny_mb(avg);
  p.shared = dffs > 0 && T <= 64 && moe::skinny_ok(dffs, d) && moe::skinny_ok(d, dffs);
  p.gemv_shared = p.shared && T <= 4 && moe::gemv_ok(dffs, d) && moe::gemv_ok(d, dffs);
  p.mb_shared = skinny_mb(T);
  return p;
}

template <typename P> P *at(void *ws, size_t off) {
  return reinterpret_cast<P *>(reinterpret_cast<char *>(ws) + off);
}

}  // namespace

extern "C" {

const char *moe_strerror(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_EINVAL:
      return "invalid argument (shape, k, E, a required NULL pointer or a misaligned tensor)";
    case MOE_EDTYPE: return "unsupported dtype (MOE_F32 or MOE_BF16)";
    case MOE_EWORKSPACE: return "workspace too small or not 256-byte aligned";
    case MOE_ELAUNCH: return "kernel launch failed";
    case MOE_EDEVICE: return "current device is not a gfx950 GPU";
    case MOE_ESCRATCH:
      return "the layer needs more scratch than moe_forward_noalloc's static array holds";
    default: return "unknown status";
  }
}

size_t moe_route_workspace_bytes(int T, int d, int E, int dtype) {
  if (dtype != MOE_F32 && dtype != MOE_BF16) return 0;
  if (T < 0 || E < 1 || E > 256 || d < 64 || d % 64) return 0;
  return align_up(moe::router_partial_bytes(T, d, E, (int)esize(dtype))) + kAlign;
}

int moe_route_ex(const void *x, const void *Wg, const float *bias, int T, int d, int E, int k,
                 int dtype, int gate_mode, int32_t *idx, float *gate, float *logits,
                 void *workspace, size_t workspace_bytes, void *stream) {
  if (dtype != MOE_F32 && dtype != MOE_BF16) return MOE_EDTYPE;
  if (gate_mode < MOE_GATE_SOFTMAX_TOPK || gate_mode > MOE_GATE_ENTROPY_BATCH) return MOE_EINVAL;
  if ((gate_mode == MOE_GATE_ENTROPY || gate_mode == MOE_GATE_ENTROPY_BATCH) && k < 2)
    return MOE_EINVAL;
  if (T < 0 || E < 1 || E > 256 || k < 1 || k > E || d < 64 || d % 64) return MOE_EINVAL;
  if ((long long)T * E >= (1LL << 31)) return MOE_EINVAL;
  if (T == 0) return MOE_OK;
  if (!x || !Wg || !idx || !gate || !workspace) return MOE_EINVAL;
  if (!al16(x) || !al16(Wg) || !al4(bias) || !al4(idx) || !al4(gate) || !al4(logits))
    return MOE_EINVAL;
  if (workspace_bytes < moe_route_workspace_bytes(T, d, E, dtype) ||
      ((uintptr_t)workspace % kAlign))
    return MOE_EWORKSPACE;
  int st = device_ok();
  if (st != MOE_OK) return st;
  return launched(moe::launch_router(dtype, x, Wg, bias, T, d, E, k, gate_mode, idx, gate,
                                     logits, (float *)workspace, (hipStream_t)stream));
}

int moe_route(const void *x, const void *Wg, const float *bias, int T, int d, int E, int k,
              int dtype, int32_t *idx, float *gate, float *logits, void *workspace,
              size_t workspace_bytes, void *stream) {
  return moe_route_ex(x, Wg, bias, T, d, E, k, dtype, MOE_GATE_SOFTMAX_TOPK, idx, gate, logits,
                      workspace, workspace_bytes, stream);
}

int moe_capacity(int T, int k, double capacity_factor) {
  if (T < 0 || k < 1 || !(capacity_factor >= 0.0)) return -1;
  const double c = std::floor(capacity_factor * (double)T);
  const long long m = (long long)k * T;
  const long long cap = c < (double)m ? (long long)c : m;
  return cap > INT32_MAX ? INT32_MAX : (int)cap;
}

int moe_capacity_mean(int T, int k, int E, double capacity_factor) {
  if (T < 0 || k < 1 || E < 1 || !(capacity_factor >= 0.0)) return -1;
  const double c = std::ceil(capacity_factor * (double)T * (double)k / (double)E);
  return c >= (double)INT32_MAX ? INT32_MAX : (int)c;
}

size_t moe_permute_workspace_bytes(int T, int E, int k) {
  if (T < 0 || E < 1 || k < 1) return 0;
  const size_t nb = (size_t)moe::permute_nblocks(T * k);
  return align_up(nb * E * 4) + 4 * align_up((size_t)(E + 1) * 4 + 32);
}

int moe_permute_ex(const int32_t *idx, int T, int E, int k, int capacity, int32_t *counts,
                   int32_t *offsets, int32_t *perm, int32_t *inv, void *workspace,
                   size_t workspace_bytes, void *stream) {
  if (T < 0 || E < 1 || E > 256 || k < 1 || k > E) return MOE_EINVAL;
  if ((long long)T * k >= (1LL << 31)) return MOE_EINVAL;
  if (T == 0) {
    if (!offsets) return MOE_EINVAL;
    // all counts and offsets are zero: nothing routed
    hipStream_t s = (hipStream_t)stream;
    if (counts && hipMemsetAsync(counts, 0, (size_t)E * 4, s) != hipSuccess) return MOE_ELAUNCH;
    return launched(hipMemsetAsync(offsets, 0, (size_t)(E + 1) * 4, s));
  }
  if (!idx || !counts || !offsets || !perm || !inv || !workspace) return MOE_EINVAL;
  if (!al4(idx) || !al4(counts) || !al4(offsets) || !al4(perm) || !al4(inv)) return MOE_EINVAL;
  if (workspace_bytes < moe_permute_workspace_bytes(T, E, k) ||
      ((uintptr_t)workspace % kAlign))
    return MOE_EWORKSPACE;
  int st = device_ok();
  if (st != MOE_OK) return st;
  const size_t nb = (size_t)moe::permute_nblocks(T * k);
  char *w = (char *)workspace;
  int32_t *blk = (int32_t *)w;
  int32_t *mt0 = (int32_t *)(w + align_up(nb * E * 4));
  int32_t *mt1 = mt0 + align_up((size_t)(E + 1) * 4 + 32) / 4;
  int32_t *sh = mt1 + align_up((size_t)(E + 1) * 4 + 32) / 4;
  int32_t *act = sh + align_up((size_t)(E + 1) * 4 + 32) / 4;
  // the m-tile prefixes are by-products here; any tile height will do
  return launched(moe::launch_permute(idx, T, E, k, capacity, 256, 256, blk, counts, offsets,
                                      perm, inv, mt0, mt1, sh, act, nullptr, 0,
                                      (hipStream_t)stream));
}

int moe_permute(const int32_t *idx, int T, int E, int k, int32_t *counts, int32_t *offsets,
                int32_t *perm, int32_t *inv, void *workspace, size_t workspace_bytes,
                void *stream) {
  return moe_permute_ex(idx, T, E, k, -1, counts, offsets, perm, inv, workspace,
                        workspace_bytes, stream);
}

size_t moe_workspace_bytes(int T, int d, int d_ff, int E, int k, int d_ff_shared, int dtype) {
  if (dtype != MOE_F32 && dtype != MOE_BF16) return 0;
  if (!dims_ok(T, d, d_ff, E, k, d_ff_shared)) return 0;
  return layout(T, d, d_ff, E, k, d_ff_shared, dtype).total;
}

int moe_workspace_offsets(int T, int d, int d_ff, int E, int k, int d_ff_shared, int dtype,
                          size_t out[MOE_WS_NFIELDS]) {
  if (dtype != MOE_F32 && dtype != MOE_BF16) return MOE_EDTYPE;
  if (!dims_ok(T, d, d_ff, E, k, d_ff_shared) || !out) return MOE_EINVAL;
  Layout L = layout(T, d, d_ff, E, k, d_ff_shared, dtype);
  const Field f[MOE_WS_NFIELDS] = {F_LOGITS, F_IDX, F_GATE, F_COUNTS, F_OFFSETS, F_PERM, F_INV};
  for (int i = 0; i < MOE_WS_NFIELDS; ++i) out[i] = L.off[f[i]];
  return MOE_OK;
}

}  // extern "C"

namespace {

// FP8 expert weights (moe_forward_fp8): codes and per-expert scales
struct Fp8Experts {
  const uint8_t *W1q, *W3q, *W2q;
  const float *s1, *s3, *s2;
};

int forward_impl(const void *x, const void *Wg, const float *bias, const void *W1,
                 const void *W3, const void *W2, const void *Ws1, const void *Ws3,
                 const void *Ws2, int d_ff_shared, int T, int E, int k, int d, int d_ff,
                 int dtype, const moe_options *opt, void *workspace, size_t workspace_bytes,
                 void *y, void *stream, void *const *events, const Fp8Experts *f8 = nullptr) {
  if (dtype != MOE_F32 && dtype != MOE_BF16) return MOE_EDTYPE;
  const moe_options o =
      opt ? *opt : moe_options{MOE_GATE_SOFTMAX_TOPK, MOE_ACT_SWIGLU, -1, MOE_LAYOUT_OUT_IN};
  if (o.weight_layout != MOE_LAYOUT_OUT_IN && o.weight_layout != MOE_LAYOUT_IN_OUT)
    return MOE_EINVAL;
  // [in][out] weights: the tiled kernels read them through transposing LDS
  // reads, few-token steps through the [K][N] weight-streaming kernel
  const bool tb = o.weight_layout == MOE_LAYOUT_IN_OUT;
  if (f8 && tb) return MOE_EINVAL;
  if (o.gate_mode < MOE_GATE_SOFTMAX_TOPK || o.gate_mode > MOE_GATE_ENTROPY_BATCH)
    return MOE_EINVAL;
  if ((o.gate_mode == MOE_GATE_ENTROPY || o.gate_mode == MOE_GATE_ENTROPY_BATCH) && k < 2)
    return MOE_EINVAL;
  // one token: the batch's largest k is the token's own
  const int gmode = o.gate_mode == MOE_GATE_ENTROPY_BATCH && T == 1 ? MOE_GATE_ENTROPY : o.gate_mode;
  if (o.activation != MOE_ACT_SWIGLU && o.activation != MOE_ACT_GLU_SIGMOID) return MOE_EINVAL;
  if (!dims_ok(T, d, d_ff, E, k, d_ff_shared)) return MOE_EINVAL;
  const bool shared = d_ff_shared > 0;
  if (shared != (Ws1 != nullptr) || shared != (Ws3 != nullptr) || shared != (Ws2 != nullptr))
    return MOE_EINVAL;
  if (T == 0) return MOE_OK;
  if (!x || !Wg || !W1 || !W3 || !W2 || !y || !workspace || x == y) return MOE_EINVAL;
  if (!al16(x) || !al16(Wg) || !al16(W1) || !al16(W3) || !al16(W2) || !al16(Ws1) ||
      !al16(Ws3) || !al16(Ws2) || !al16(y) || !al4(bias))
    return MOE_EINVAL;
  if (f8 && (!al4(f8->s1) || !al4(f8->s3) || !al4(f8->s2))) return MOE_EINVAL;
  const Layout L = layout(T, d, d_ff, E, k, d_ff_shared, dtype);
  if (workspace_bytes < L.total || ((uintptr_t)workspace % kAlign)) return MOE_EWORKSPACE;
  int st = device_ok();
  if (st != MOE_OK) return st;

  hipStream_t s = (hipStream_t)stream;
  void *ws = workspace;
  const int P = T * k;
  const moe::GemmPlan plan =
      moe::gemm_plan(dtype, d, d_ff, d_ff_shared, ((long long)T * k + E - 1) / E);
  SkinnyPlan sk = skinny_plan(dtype, T, k, E, d, d_ff, d_ff_shared);
  // FP8 experts: vector-ALU weight streaming up to four tokens, 64-row tiles
  // beyond (the caller checked that one of them applies)
  const bool f8_tiled = f8 && !(T <= 4 && moe::gemv_ok(d_ff, d) && moe::gemv_ok(d, d_ff));
  if (f8) sk.routed = sk.gemv = !f8_tiled;
  if (tb) {
    // [K][N] weights: vector-ALU streaming up to four tokens, tiles beyond
    sk.gemv = sk.gemv && moe::gemv_t_ok(d_ff, d) && moe::gemv_t_ok(d, d_ff);
    sk.routed = sk.gemv;
    sk.gemv_shared = sk.gemv_shared && moe::gemv_t_ok(d_ff_shared, d) &&
                     moe::gemv_t_ok(d, d_ff_shared);
    sk.shared = sk.gemv_shared;
  }
  // K planes of the down projection: the tiled kernel's choice; the [K][N]
  // weight-streaming kernel takes up to 4 (within the workspace's planes)
  const int ksplit =
      sk.routed ? (tb ? moe::gemv_t_down_splits(std::min(E, T * k), d, d_ff,
                                                std::min(4, down_splits(plan, T, k, E, d, d_ff)))
                      : 1)
                : down_splits(plan, T, k, E, d, d_ff);
  const size_t plane = (size_t)P * d;
  float *logits = at<float>(ws, L.off[F_LOGITS]);
  int32_t *idx = at<int32_t>(ws, L.off[F_IDX]);
  float *gate = at<float>(ws, L.off[F_GATE]);
  int32_t *counts = at<int32_t>(ws, L.off[F_COUNTS]);
  int32_t *offsets = at<int32_t>(ws, L.off[F_OFFSETS]);
  int32_t *perm = at<int32_t>(ws, L.off[F_PERM]);
  int32_t *inv = at<int32_t>(ws, L.off[F_INV]);
  int32_t *mt0 = at<int32_t>(ws, L.off[F_MT0]);
  int32_t *mt1 = at<int32_t>(ws, L.off[F_MT1]);
  int32_t *shseg = at<int32_t>(ws, L.off[F_SHSEG]);
  int32_t *act = at<int32_t>(ws, L.off[F_ACT]);
  int32_t *mid = at<int32_t>(ws, L.off[F_MID]);
  int32_t *blk = at<int32_t>(ws, L.off[F_BLK]);
  void *Xp = at<char>(ws, L.off[F_XP]);
  void *H = at<char>(ws, L.off[F_H]);
  float *Yp = at<float>(ws, L.off[F_YP]);
  void *Hs = at<char>(ws, L.off[F_HS]);
  float *Ys = at<float>(ws, L.off[F_YS]);
  int32_t *fixc = at<int32_t>(ws, L.off[F_FIXC]);
  const size_t fixp_bytes = L.off[F_FIXP + 1] - L.off[F_FIXP];
  const moe::FixScratch fx{fixc, fixp_bytes ? at<char>(ws, L.off[F_FIXP]) : nullptr, fixp_bytes};
  // single-token-scale batches without a shared expert: the down projection's
  // last workgroups also do the combine
  const bool fused_combine = sk.gemv && !shared && !tb;
  // a single token with a small router: the SwiGLU weight-streaming kernel
  // routes it itself (no score or top-k launches)
  const bool route_fused = sk.gemv && moe::route_fused_ok(T, d, E, k);
  const moe::DecodeRoute rt{Wg, bias, E, k, gmode,
                            o.capacity < 0 || o.capacity > P ? P : o.capacity,
                            plan.bm1, plan.bm2, logits, idx, gate, counts, offsets, perm, inv,
                            mt0, mt1, shseg, act, fixc, moe::FIX_SLOTS};
  // one token without a shared expert: a workgroup per column block covers
  // all its experts and forms y itself
  const bool token_down = fused_combine && T == 1 && moe::gemv_token_ok(d, d_ff, k);
  // experts a weight-streaming grid covers: at most P are active
  const int G = std::min(E, P);
  // 256-row tiles with fewer than 512 rows per expert on average: an expert's
  // rows past its last full tile, when few (up to 128), go to light 64-row
  // tiles of the same launch, placed after the expert's full tiles of the
  // same weight columns (mt0: full-tile prefix, mt1: light-tile prefix, mid:
  // where each expert's light rows start).  Measured on 256 experts at
  // T=8192: 8.50 -> 8.30 ms against a second launch for those rows (which read
  // the weights from HBM again); on Mixtral (about 2048 rows per expert) light
  // tiles in place of partly filled 256-row tiles cost more (4.67 -> 4.94 ms),
  // so that layer keeps one tile height.
  const bool split = !sk.routed && plan.dl1 && plan.dl2 && plan.bm1 == 256 && plan.bm2 == 256 &&
                     (long long)P < 512LL * E;
  // the tiled down projection of the bf16 layer leaves its outputs in bf16
  // (one plane), which halves what it writes and the combine reads
  const bool yp_bf16 = dtype == MOE_BF16 && !sk.routed && ksplit == 1 && plan.dl2;
  // 64-row tiles (and the split tiling's 256-row tiles) read their rows
  // straight from x (no gathered copy)
  const bool gather_fused = !sk.routed && plan.dl1 && (plan.bm1 == 64 || split) &&
                            moe::gemm_gather_ok(dtype, plan.dl1, plan.bm1, (long long)T * d * 2);

  hipError_t e;
  // stage boundary i: an optional timing event recorded on the stream
#define MOE_MARK(i) \
  if (events && hipEventRecord((hipEvent_t)events[i], s) != hipSuccess) goto fail;
  MOE_MARK(0);
  if (route_fused) {
    MOE_MARK(1);
  } else if (moe::route_permute_tiny_ok(T, E, k) && gmode != MOE_GATE_ENTROPY_BATCH) {
    // a small batch: scores, then top-k, gate and grouping in one more launch
    if ((e = moe::launch_route_permute_tiny(dtype, x, Wg, bias, T, d, E, k, gmode,
                                            o.capacity, plan.bm1, plan.bm2, logits, idx, gate,
                                            counts, offsets, perm, inv, mt0, mt1, shseg, act,
                                            fixc, moe::FIX_SLOTS,
                                            at<float>(ws, L.off[F_RPART]), s)))
      goto fail;
    MOE_MARK(1);
  } else {
    if ((e = moe::launch_router(dtype, x, Wg, bias, T, d, E, k, gmode, idx, gate, logits,
                                at<float>(ws, L.off[F_RPART]), s)))
      goto fail;
    MOE_MARK(1);
    if ((e = moe::launch_permute(idx, T, E, k, o.capacity, plan.bm1, plan.bm2, blk, counts,
                                 offsets, perm, inv, mt0, mt1, shseg, act, fixc, moe::FIX_SLOTS,
                                 s, split ? mid : nullptr)))
      goto fail;
  }
  MOE_MARK(2);
  if (sk.routed) {
    // few rows per expert: weight-streaming kernels; the gather rides in the first GEMM
    MOE_MARK(3);
    // a single token activates exactly k experts (fewer only under a capacity)
    const int nact = T == 1 ? k : 0;
    if ((e = route_fused && tb
                 ? moe::launch_gemv_t_swiglu_routed(o.activation, x, rt, W1, W3, H, d_ff, d, s)
             : route_fused
                 ? moe::launch_gemv_swiglu_routed(o.activation, x, rt, f8 ? f8->W1q : W1,
                                                  f8 ? f8->W3q : W3, f8 ? f8->s1 : nullptr,
                                                  f8 ? f8->s3 : nullptr, H, d_ff, d, s)
             : f8 ? moe::launch_gemv_swiglu_fp8(T, o.activation, x, perm, k, f8->W1q, f8->W3q,
                                                f8->s1, f8->s3, H, offsets, act, act + E, G,
                                                d_ff, d, nact, s)
             : tb ? moe::launch_gemv_t_swiglu(T, o.activation, x, perm, k, W1, W3, H, offsets,
                                              act, act + E, G, d_ff, d, s)
             : sk.gemv ? moe::launch_gemv_swiglu(T, o.activation, x, perm, k, W1, W3, H, offsets,
                                               act, act + E, G, d_ff, d, nact, s)
                     : moe::launch_skinny_swiglu(sk.mb, o.activation, x, perm, k, W1, W3, H,
                                                 offsets, act, act + E, E, d_ff, d, s)))
      goto fail;
    MOE_MARK(4);
    if ((e = token_down
                 ? moe::launch_gemv_down_token(H, f8 ? f8->W2q : W2, f8 ? f8->s2 : nullptr, offsets,
                                               act, act + E, d, d_ff, inv, gate, k, y, s)
             : f8 ? moe::launch_gemv_down_combine_fp8(T, H, f8->W2q, f8->s2, Yp, offsets, act,
                                                    act + E, G, d, d_ff, nact, inv, gate, T, k,
                                                    y, fixc, s)
             : fused_combine
                 ? moe::launch_gemv_down_combine(T, H, W2, Yp, offsets, act, act + E, G, d, d_ff,
                                                 nact, inv, gate, T, k, y, fixc, s)
             : tb ? moe::launch_gemv_t_down(T, H, W2, Yp, offsets, act, act + E, G, d, d_ff,
                                            ksplit, plane, s)
             : sk.gemv ? moe::launch_gemv_down(T, H, W2, Yp, offsets, act, act + E, G, d, d_ff,
                                               nact, s)
                       : moe::launch_skinny_down(sk.mb, H, W2, Yp, offsets, act, act + E, E, d,
                                                 d_ff, s)))
      goto fail;
    MOE_MARK(5);
  } else {
    if (!gather_fused &&
        (e = moe::launch_gather(x, perm, offsets + E, P, k, d, (int)esize(dtype), Xp, s)))
      goto fail;
    MOE_MARK(3);
    if (f8) {
      if ((e = moe::launch_gemm_swiglu_fp8(o.activation, gather_fused ? x : Xp, f8->W1q, f8->W3q,
                                           f8->s1, f8->s3, H, offsets, mt0, E, d_ff, d,
                                           (P + 63) / 64 + E, s, gather_fused ? perm : nullptr, k,
                                           gather_fused ? (long long)T * d * 2 : 0)))
        goto fail;
    } else if (gather_fused && split) {
      if ((e = moe::launch_gemm_swiglu(dtype, true, 256, o.activation, x, W1, W3, H, offsets, mt0,
                                       E, d_ff, d, P / 256 + 3 * E, s, offsets + 1, perm, k,
                                       (long long)T * d * 2, tb, mid, mt1,
                                       fixc + moe::FIX_SLOTS - moe::TILE_Q_SLOTS)))
        goto fail;
    } else if (gather_fused) {
      if ((e = moe::launch_gemm_swiglu(dtype, true, 64, o.activation, x, W1, W3, H, offsets, mt0,
                                       E, d_ff, d, (P + 63) / 64 + E, s, nullptr, perm, k,
                                       (long long)T * d * 2, tb)))
        goto fail;
    } else if (split) {
      if ((e = moe::launch_gemm_swiglu(dtype, true, 256, o.activation, Xp, W1, W3, H, offsets, mt0,
                                       E, d_ff, d, P / 256 + 3 * E, s, offsets + 1, nullptr, 1, 0,
                                       tb, mid, mt1, fixc + moe::FIX_SLOTS - moe::TILE_Q_SLOTS)))
        goto fail;
    } else if ((e = moe::launch_gemm_swiglu(dtype, plan.dl1, plan.bm1, o.activation, Xp, W1, W3,
                                            H, offsets, mt0, E, d_ff, d,
                                            (P + plan.bm1 - 1) / plan.bm1 + E, s, nullptr, nullptr,
                                            1, 0, tb))) {
      goto fail;
    }
    MOE_MARK(4);
    if (f8) {
      if ((e = moe::launch_gemm_down_fp8(H, f8->W2q, f8->s2, Yp, offsets, mt1, E, d, d_ff,
                                         (P + 63) / 64 + E, ksplit, plane, s, yp_bf16)))
        goto fail;
    } else if (split) {
      if ((e = moe::launch_gemm_down(dtype, true, 256, H, W2, Yp, offsets, mt0, E, d, d_ff,
                                     P / 256 + 3 * E, ksplit, plane, fx, s, offsets + 1, yp_bf16,
                                     tb, mid, mt1)))
        goto fail;
    } else if ((e = moe::launch_gemm_down(dtype, plan.dl2, plan.bm2, H, W2, Yp, offsets, mt1, E, d,
                                          d_ff, (P + plan.bm2 - 1) / plan.bm2 + E, ksplit, plane,
                                          fx, s, nullptr, yp_bf16, tb))) {
      goto fail;
    }
    MOE_MARK(5);
  }
  if (shared) {
    if (sk.gemv_shared && tb) {
      if ((e = moe::launch_gemv_t_swiglu(T, o.activation, x, nullptr, 1, Ws1, Ws3, Hs, shseg,
                                         shseg + 6, shseg + 7, 1, d_ff_shared, d, s)))
        goto fail;
      if ((e = moe::launch_gemv_t_down(T, Hs, Ws2, Ys, shseg, shseg + 6, shseg + 7, 1, d,
                                       d_ff_shared, 1, 0, s)))
        goto fail;
    } else if (sk.gemv_shared) {
      if ((e = moe::launch_gemv_swiglu(T, o.activation, x, nullptr, 1, Ws1, Ws3, Hs, shseg,
                                       shseg + 6, shseg + 7, 1, d_ff_shared, d, 1, s)))
        goto fail;
      if ((e = moe::launch_gemv_down(T, Hs, Ws2, Ys, shseg, shseg + 6, shseg + 7, 1, d,
                                     d_ff_shared, 1, s)))
        goto fail;
    } else if (sk.shared) {
      if ((e = moe::launch_skinny_swiglu(sk.mb_shared, o.activation, x, nullptr, 1, Ws1, Ws3,
                                         Hs, shseg, shseg + 6, shseg + 7, 1, d_ff_shared, d, s)))
        goto fail;
      if ((e = moe::launch_skinny_down(sk.mb_shared, Hs, Ws2, Ys, shseg, shseg + 6, shseg + 7, 1,
                                       d, d_ff_shared, s)))
        goto fail;
    } else {
      if ((e = moe::launch_gemm_swiglu(dtype, plan.dl1, plan.bm1, o.activation, x, Ws1, Ws3, Hs,
                                       shseg, shseg + 2, 1, d_ff_shared, d,
                                       (T + plan.bm1 - 1) / plan.bm1, s, nullptr, nullptr, 1, 0,
                                       tb)))
        goto fail;
      if ((e = moe::launch_gemm_down(dtype, plan.dl2, plan.bm2, Hs, Ws2, Ys, shseg, shseg + 4, 1, d,
                                     d_ff_shared, (T + plan.bm2 - 1) / plan.bm2, 1, 0, fx, s,
                                     nullptr, false, tb)))
        goto fail;
    }
  }
  MOE_MARK(6);
  if (!fused_combine &&
      (e = moe::launch_combine(dtype, Yp, ksplit, plane, shared ? Ys : nullptr, inv, gate, T, k,
                               d, y, s, yp_bf16)))
    goto fail;
  MOE_MARK(7);
#undef MOE_MARK
  return MOE_OK;
fail:
  return MOE_ELAUNCH;
}

}  // namespace

extern "C" {

int moe_forward(const void *x, const void *Wg, const float *bias, const void *W1,
                const void *W3, const void *W2, const void *Ws1, const void *Ws3,
                const void *Ws2, int d_ff_shared, int T, int E, int k, int d, int d_ff,
                int dtype, void *workspace, size_t workspace_bytes, void *y, void *stream) {
  return forward_impl(x, Wg, bias, W1, W3, W2, Ws1, Ws3, Ws2, d_ff_shared, T, E, k, d, d_ff,
                      dtype, nullptr, workspace, workspace_bytes, y, stream, nullptr);
}

int moe_forward_ex(const void *x, const void *Wg, const float *bias, const void *W1,
                   const void *W3, const void *W2, const void *Ws1, const void *Ws3,
                   const void *Ws2, int d_ff_shared, int T, int E, int k, int d, int d_ff,
                   int dtype, const moe_options *opt, void *workspace, size_t workspace_bytes,
                   void *y, void *stream) {
  return forward_impl(x, Wg, bias, W1, W3, W2, Ws1, Ws3, Ws2, d_ff_shared, T, E, k, d, d_ff,
                      dtype, opt, workspace, workspace_bytes, y, stream, nullptr);
}

int moe_forward_inout(const void *x, const void *Wg, const float *bias, const void *W1,
                      const void *W3, const void *W2, const void *Ws1, const void *Ws3,
                      const void *Ws2, int d_ff_shared, int T, int E, int k, int d, int d_ff,
                      int dtype, void *workspace, size_t workspace_bytes, void *y, void *stream) {
  const moe_options o{MOE_GATE_SOFTMAX_TOPK, MOE_ACT_SWIGLU, -1, MOE_LAYOUT_IN_OUT};
  return forward_impl(x, Wg, bias, W1, W3, W2, Ws1, Ws3, Ws2, d_ff_shared, T, E, k, d, d_ff,
                      dtype, &o, workspace, workspace_bytes, y, stream, nullptr);
}

int moe_forward_timed(const void *x, const void *Wg, const float *bias, const void *W1,
                      const void *W3, const void *W2, const void *Ws1, const void *Ws3,
                      const void *Ws2, int d_ff_shared, int T, int E, int k, int d, int d_ff,
                      int dtype, const moe_options *opt, void *workspace,
                      size_t workspace_bytes, void *y, void *stream, void *const *events) {
  if (!events) return MOE_EINVAL;
  for (int i = 0; i < MOE_NSTAGE_EVENTS; ++i)
    if (!events[i]) return MOE_EINVAL;
  return forward_impl(x, Wg, bias, W1, W3, W2, Ws1, Ws3, Ws2, d_ff_shared, T, E, k, d, d_ff,
                      dtype, opt, workspace, workspace_bytes, y, stream, events);
}

int moe_quantize_fp8(const void *W, int E, long long n, int dtype, uint8_t *q, float *scale,
                     void *stream) {
  if (dtype != MOE_F32 && dtype != MOE_BF16) return MOE_EDTYPE;
  if (E < 0 || n < 0) return MOE_EINVAL;
  if (E == 0 || n == 0) return MOE_OK;
  if (!W || !q || !scale) return MOE_EINVAL;
  int st = device_ok();
  if (st != MOE_OK) return st;
  return launched(moe::launch_quantize_fp8(dtype, W, E, (size_t)n, q, scale, (hipStream_t)stream));
}

int moe_forward_fp8(const void *x, const void *Wg, const float *bias, const uint8_t *W1q,
                    const uint8_t *W3q, const uint8_t *W2q, const float *s1, const float *s3,
                    const float *s2, int T, int E, int k, int d, int d_ff,
                    const moe_options *opt, void *workspace, size_t workspace_bytes, void *y,
                    void *stream) {
  if (T < 0 || E < 1 || k < 1 || k > E) return MOE_EINVAL;
  // up to four tokens: the weight-streaming kernels (d and d_ff multiples of
  // 2048 up to 16384); beyond: 64-row tiles (at most 96 rows per expert on
  // average, d and d_ff multiples of 128)
  const bool streamed = T <= 4 && moe::gemv_ok(d_ff, d) && moe::gemv_ok(d, d_ff);
  const long long rpe = ((long long)T * k + E - 1) / E;
  const moe::GemmPlan plan = moe::gemm_plan(MOE_BF16, d, d_ff, 0, rpe);
  const bool tiled = plan.dl1 && plan.dl2 && plan.bm1 == 64 && plan.bm2 == 64;
  if (!streamed && !tiled) return MOE_EINVAL;
  if (T > 0 && (!s1 || !s3 || !s2)) return MOE_EINVAL;
  const Fp8Experts f8{W1q, W3q, W2q, s1, s3, s2};
  return forward_impl(x, Wg, bias, W1q, W3q, W2q, nullptr, nullptr, nullptr, 0, T, E, k, d, d_ff,
                      MOE_BF16, opt, workspace, workspace_bytes, y, stream, nullptr, &f8);
}

}  // extern "C"

namespace {

// Scratch of moe_forward_noalloc: one array per GPU, allocated with the code
// object when the library is loaded on that device and held until the process
// ends.  Host code uses the per-device address from hipGetSymbolAddress, never
// the array's name (a host-side stand-in, not a device address).
constexpr size_t kNoAllocBytes = (size_t)MOE_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kNoAllocBytes];

// scratch's address on the current device (NULL if it cannot be had)
void *noalloc_scratch() {
  static std::mutex mu;
  static void *addr[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  std::lock_guard<std::mutex> g(mu);
  if (!addr[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    addr[dev] = p;
  }
  return addr[dev];
}

}  // namespace

extern "C" {

int moe_forward_noalloc(const void *x, const void *Wg, const float *bias, const void *W1,
                        const void *W3, const void *W2, const void *Ws1, const void *Ws3,
                        const void *Ws2, int d_ff_shared, int T, int E, int k, int d, int d_ff,
                        int dtype, void *y, void *stream) {
  if (dtype != MOE_F32 && dtype != MOE_BF16) return MOE_EDTYPE;
  if (!dims_ok(T, d, d_ff, E, k, d_ff_shared)) return MOE_EINVAL;
  if (T == 0) return MOE_OK;
  const size_t need = layout(T, d, d_ff, E, k, d_ff_shared, dtype).total;
  if (need > kNoAllocBytes) return MOE_ESCRATCH;
  int st = device_ok();
  if (st != MOE_OK) return st;
  void *ws = noalloc_scratch();
  if (!ws) return MOE_ELAUNCH;
  return forward_impl(x, Wg, bias, W1, W3, W2, Ws1, Ws3, Ws2, d_ff_shared, T, E, k, d, d_ff,
                      dtype, nullptr, ws, kNoAllocBytes, y, stream, nullptr);
}

}  // extern "C"
