/*
 * moe_mi355x.h -- C ABI of the sparse Mixture-of-Experts feed-forward layer
 * for AMD MI355X (gfx950).
 *
 * The layer (sources cited by page title and section):
 *   router    logits[t][e] = sum_i x[t][i] * Wg[e][i] (+ bias[e])
 *             ("Chapter 10 MoE" of LLMs-from-scratch, section 10.3;
 *              "Mistral 8x7B SMoE architecture deep dive", section 3.2)
 *   top-k     the k largest logits per token, ordered by descending logit;
 *             an exact tie goes to the lower expert index
 *   gate      softmax over the k selected logits only (sums to one)
 *             (same sections; the chapter stresses selected-only softmax)
 *   experts   FFN_e(x) = W2_e( SiLU(W1_e x) * (W3_e x) ),  SiLU(a) = a*sigmoid(a)
 *             ("Mistral 8x7B SMoE ..." section 3.1; "Mixtral and MoE
 *              architecture", FeedForward listing)
 *   combine   y[t] = sum_j gate[t][j] * FFN_{idx[t][j]}(x_t)
 *             (+ an always-on shared expert with weight 1, "Chapter 10 MoE"
 *              section 10.5)
 * Pairs are grouped by expert before the expert GEMMs ("Chapter 10 MoE"
 * section 10.4; the per-expert row lists of the "Trillion-parameter MoE ...
 * 7 expert configs measured" numpy listing): a stable counting sort of the
 * flat pair ids p = t*k + j by expert.
 *
 * Conventions for every call
 *  - All tensors are row-major and dense.  The router is Wg [E][d] (scores
 *    x Wg^T).  Expert weights come in one of two layouts (moe_options
 *    weight_layout):
 *      MOE_LAYOUT_OUT_IN (default): Linear weights [out][in]: W1 and W3
 *        [E][d_ff][d], W2 [E][d][d_ff], shared Ws1 and Ws3 [d_ff_shared][d],
 *        Ws2 [d][d_ff_shared] ("Chapter 10 MoE" and the "Mixtral and MoE
 *        architecture" listing hold nn.Linear weights);
 *      MOE_LAYOUT_IN_OUT: [in][out], the layer multiplies x W: W1 and W3
 *        [E][d][d_ff], W2 [E][d_ff][d], shared Ws1 and Ws3 [d][d_ff_shared],
 *        Ws2 [d_ff_shared][d] (the numpy forward of "Trillion-parameter MoE
 *        ... 7 expert configs measured" multiplies x @ W1[e] and h @ W2[e]).
 *    Both give the same results up to the order of fp32 additions (the tiled
 *    kernels: the same bits).
 *  - Every pointer argument is a DEVICE pointer owned by the caller; the
 *    library never allocates, frees or retains memory, and never synchronises
 *    the host with the device.
 *  - Alignment: x, the weights (and FP8 codes) and y 16 bytes; bias, scales,
 *    logits, gates and int32 arrays 4 bytes (any PyTorch allocation or row
 *    slice qualifies).  A misaligned pointer is MOE_EINVAL.
 *  - `stream` is a hipStream_t (NULL = the default stream).  All work is
 *    enqueued on it asynchronously; results are valid once the stream has
 *    reached that point.
 *  - dtype MOE_BF16: x, weights and y are bf16 (IEEE binary32 upper halves);
 *    dtype MOE_F32: all fp32.  Accumulation is always fp32.  Router logits and
 *    gates are always fp32; indices and counts are int32.
 *  - Return value: MOE_OK (0) or a negative error code (see moe_strerror).
 *    Argument errors are detected before anything is enqueued.  A fault
 *    inside a kernel is reported by the stream, not by these calls.
 *  - Shape limits: 1 <= k <= E <= 256; T >= 0 (T = 0 enqueues nothing);
 *    d and d_ff (and d_ff_shared) positive multiples of 64;
 *    T * k < 2^31 and every tensor under 2^31 elements per expert slice.
 *  - Inputs must be finite.  Calls that share a workspace on overlapping
 *    streams race.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;

enum {
    MOE_OK = 0,
    MOE_EINVAL = -1,     /* bad shape, k, E, a required NULL pointer, misalignment */
    MOE_EDTYPE = -2,     /* dtype not MOE_F32 / MOE_BF16 */
    MOE_EWORKSPACE = -3, /* workspace too small or misaligned (needs 256 B) */
    MOE_ELAUNCH = -4,    /* the HIP runtime refused a kernel launch */
    MOE_EDEVICE = -5,    /* current device is not a gfx950 GPU */
    MOE_ESCRATCH = -6    /* moe_forward_noalloc: the shape needs more than its static scratch */
};

/* Bytes of scratch moe_route needs for (T, d, E, dtype); 0 on invalid arguments. */
size_t moe_route_workspace_bytes(int T, int d, int E, int dtype);

/* Router + top-k + gate (the first two steps above).
 *   x      [T][d]   dtype          Wg [E][d] dtype
 *   bias   [E] fp32 or NULL (a per-expert logit offset, e.g. to skew routing)
 *   idx    [T][k] int32  out: selected experts, descending logit, ties -> lower e
 *   gate   [T][k] fp32   out: softmax over the selected logits
 *   logits [T][E] fp32   out (may be NULL): the router scores idx/gate came from
 *   workspace: device scratch of moe_route_workspace_bytes(T, d, E, dtype)
 *     bytes, 256-byte aligned (partial sums over slices of the d dimension,
 *     added in a fixed order, so the scores are deterministic). */
int moe_route(const void *x, const void *Wg, const float *bias, int T, int d, int E, int k,
              int dtype, int32_t *idx, float *gate, float *logits, void *workspace,
              size_t workspace_bytes, void *stream);

/* Bytes of scratch moe_permute needs for (T, E, k). */
size_t moe_permute_workspace_bytes(int T, int E, int k);

/* Grouping of the T*k (token, slot) pairs by expert (stable counting sort).
 *   idx     [T][k] int32 in, values in [0, E)
 *   counts  [E]    out: pairs routed to each expert
 *   offsets [E+1]  out: exclusive prefix sum, offsets[E] = T*k
 *   perm    [T*k]  out: perm[s] = flat pair id t*k+j placed at slot s; slots of
 *                  expert e are offsets[e]..offsets[e+1]-1 in ascending pair id
 *   inv     [T*k]  out: inv[perm[s]] = s
 * Deterministic (no atomic-order dependence).  `workspace` is device scratch of
 * moe_permute_workspace_bytes(T, E, k) bytes, 256-byte aligned. */
int moe_permute(const int32_t *idx, int T, int E, int k, int32_t *counts, int32_t *offsets,
                int32_t *perm, int32_t *inv, void *workspace, size_t workspace_bytes,
                void *stream);

/* Bytes of scratch moe_forward needs (d_ff_shared = 0: no shared expert). */
size_t moe_workspace_bytes(int T, int d, int d_ff, int E, int k, int d_ff_shared, int dtype);

/* Byte offsets inside the moe_forward workspace of the intermediates, so that
 * a caller can read them after the call:
 *   out[0] logits [T][E] f32    out[1] idx  [T][k] i32   out[2] gate [T][k] f32
 *   out[3] counts [E] i32       out[4] offsets [E+1] i32 out[5] perm [T*k] i32
 *   out[6] inv [T*k] i32
 * Returns MOE_OK or MOE_EINVAL / MOE_EDTYPE. */
#define MOE_WS_NFIELDS 7
int moe_workspace_offsets(int T, int d, int d_ff, int E, int k, int d_ff_shared, int dtype,
                          size_t out[MOE_WS_NFIELDS]);

/* The whole layer: route -> permute -> grouped SwiGLU expert GEMMs -> combine.
 *   x [T][d]; Wg [E][d]; bias [E] fp32 or NULL; W1, W3 [E][d_ff][d]; W2 [E][d][d_ff]
 *   Ws1, Ws3 [d_ff_shared][d], Ws2 [d][d_ff_shared]: the shared expert, or all
 *     NULL with d_ff_shared = 0
 *   workspace: device scratch of moe_workspace_bytes(...) bytes, 256-byte aligned
 *   y [T][d] out, dtype.  y may not alias x. */
int moe_forward(const void *x, const void *Wg, const float *bias, const void *W1,
                const void *W3, const void *W2, const void *Ws1, const void *Ws3,
                const void *Ws2, int d_ff_shared, int T, int E, int k, int d, int d_ff,
                int dtype, void *workspace, size_t workspace_bytes, void *y, void *stream);

/* moe_forward that also records a timing event on `stream` at each stage
 * boundary, for measurement.  `events` holds MOE_NSTAGE_EVENTS caller-created
 * hipEvent_t handles: [0] before the router, [1] after the router, [2] after
 * the permutation, [3] after the row gather, [4] after the SwiGLU GEMM, [5]
 * after the down GEMM, [6] after the shared expert (if any), [7] after the
 * combine.  A decode step (T <= 4, T * k <= 64, E <= 64) runs top-k and the
 * grouping in one launch: [1] and [2] then both follow it.  A single token
 * whose router has at most 65536 elements (d a multiple of 2048) is routed
 * inside the SwiGLU projection, in either weight layout: [0] to [3] then all
 * precede that kernel.  When the down projection streams [out][in] weights
 * and there is no shared expert, the combine rides in that kernel: [5], [6]
 * and [7] then all follow it.  Same results
 * and errors as moe_forward; MOE_EINVAL if `events` or any of its handles is
 * NULL.  `opt`: the variants and weight layout of moe_forward_ex (NULL: the
 * defaults). */
#define MOE_NSTAGE_EVENTS 8
struct moe_options_s; /* moe_options, defined below */
int moe_forward_timed(const void *x, const void *Wg, const float *bias, const void *W1,
                      const void *W3, const void *W2, const void *Ws1, const void *Ws3,
                      const void *Ws2, int d_ff_shared, int T, int E, int k, int d, int d_ff,
                      int dtype, const struct moe_options_s *opt, void *workspace,
                      size_t workspace_bytes, void *y, void *stream, void *const *events);

/* ------------------------------------------------------------------------
 * Variants the pages print beside the method (all optional; the calls above
 * are these with the defaults).
 *
 *   gate_mode  MOE_GATE_SOFTMAX_TOPK  softmax over the k selected logits (the
 *                                     method; default)
 *              MOE_GATE_SOFTMAX_ALL   softmax over all E logits, the selected
 *                                     entries used as they are (no
 *                                     renormalisation): the Router of "Mixtral
 *                                     8x7B model architecture", section 1.2
 *              MOE_GATE_SIGMOID       logistic sigmoid of each selected logit:
 *                                     the numpy function of "Trillion-parameter
 *                                     MoE ... 7 expert configs measured"
 *              MOE_GATE_ENTROPY       entropy-aware k ("Mixtral 8x7B model
 *                                     architecture", section 4.1): p =
 *                                     softmax(logits / 0.1) over all E; a token
 *                                     whose entropy -sum p ln p exceeds 0.8
 *                                     takes k experts, otherwise k - 1 (the
 *                                     page's 3 and 2; needs k >= 2); gates are
 *                                     the selected p as they are.  The unused
 *                                     slot holds idx -1 and gate 0 and is
 *                                     placed nowhere (inv -1).  The page takes
 *                                     the batch's largest k for every token;
 *                                     in this mode each token keeps its own
 *              MOE_GATE_ENTROPY_BATCH the same routing as the page's listing
 *                                     prints it: one k for the whole call,
 *                                     the largest per-token k (k if any
 *                                     token's entropy exceeds 0.8, else
 *                                     k - 1, in which case every token's
 *                                     last slot is empty: idx -1, gate 0);
 *                                     needs k >= 2.
 *   activation MOE_ACT_SWIGLU         W2( SiLU(W1 x) * (W3 x) )  (default)
 *              MOE_ACT_GLU_SIGMOID    W2( sigmoid(W1 x) * (W3 x) ): the same
 *                                     numpy function's gated projection (its
 *                                     fused [a | g] weight is [W3 | W1] here)
 *   weight_layout  MOE_LAYOUT_OUT_IN or MOE_LAYOUT_IN_OUT (see the
 *              conventions above); MOE_EINVAL otherwise
 *   capacity   at most `capacity` pairs per expert ("Mistral 8x7B SMoE
 *              architecture deep dive", section 2.4); an expert keeps its
 *              first pairs in pair order t*k+j (the page does not say which
 *              pairs go), a dropped pair contributes nothing and the token's
 *              other gates are not renormalised.  capacity < 0: no limit.
 * ------------------------------------------------------------------------ */
enum {
    MOE_GATE_SOFTMAX_TOPK = 0,
    MOE_GATE_SOFTMAX_ALL = 1,
    MOE_GATE_SIGMOID = 2,
    MOE_GATE_ENTROPY = 3,
    MOE_GATE_ENTROPY_BATCH = 4
};
enum { MOE_ACT_SWIGLU = 0, MOE_ACT_GLU_SIGMOID = 1 };

enum { MOE_LAYOUT_OUT_IN = 0, MOE_LAYOUT_IN_OUT = 1 };

typedef struct moe_options_s {
    int gate_mode;     /* MOE_GATE_* */
    int activation;    /* MOE_ACT_* */
    int capacity;      /* pairs per expert; < 0: no limit */
    int weight_layout; /* MOE_LAYOUT_*: expert weights [out][in] (default) or [in][out] */
} moe_options;

/* The page's capacity for a batch of T tokens: min(k*T, floor(cf*T))
 * ("Mistral 8x7B SMoE ..." section 2.4: cf = 1.2 gives 38 for T=32, k=2).
 * Host-only arithmetic; returns -1 for T < 0, k < 1 or cf < 0. */
int moe_capacity(int T, int k, double capacity_factor);

/* The capacity as cf times an expert's mean load: ceil(cf * T * k / E) (the
 * page's formula above compares cf with the batch alone, so for k >= 2 it
 * never limits an expert: an expert holds at most T pairs).  Host-only;
 * -1 for T < 0, k < 1, E < 1 or cf < 0; saturates at INT32_MAX. */
int moe_capacity_mean(int T, int k, int E, double capacity_factor);

/* moe_route with a gate variant (gate_mode as above); MOE_EINVAL for an
 * unknown mode, or an entropy-aware mode with k < 2. */
int moe_route_ex(const void *x, const void *Wg, const float *bias, int T, int d, int E, int k,
                 int dtype, int gate_mode, int32_t *idx, float *gate, float *logits,
                 void *workspace, size_t workspace_bytes, void *stream);

/* moe_permute under a per-expert capacity (< 0: no limit).  Only kept pairs
 * are placed: counts[e] = pairs kept by expert e, offsets their exclusive
 * prefix sum (offsets[E] = kept pairs), perm has offsets[E] valid entries,
 * inv[p] = -1 for a dropped pair (and for an id outside [0, E)). */
int moe_permute_ex(const int32_t *idx, int T, int E, int k, int capacity, int32_t *counts,
                   int32_t *offsets, int32_t *perm, int32_t *inv, void *workspace,
                   size_t workspace_bytes, void *stream);

/* moe_forward with expert weights in the [in][out] layout (MOE_LAYOUT_IN_OUT):
 * W1, W3 [E][d][d_ff], W2 [E][d_ff][d]; shared Ws1, Ws3 [d][d_ff_shared], Ws2
 * [d_ff_shared][d] ("Trillion-parameter MoE ... 7 expert configs measured",
 * the numpy forward: x @ W1[e], h @ W2[e]).  Everything else as moe_forward. */
int moe_forward_inout(const void *x, const void *Wg, const float *bias, const void *W1,
                      const void *W3, const void *W2, const void *Ws1, const void *Ws3,
                      const void *Ws2, int d_ff_shared, int T, int E, int k, int d, int d_ff,
                      int dtype, void *workspace, size_t workspace_bytes, void *y, void *stream);

/* moe_forward with the variants in `opt` (NULL: the defaults).  Same
 * workspace; its counts/offsets/perm/inv fields then follow moe_permute_ex. */
int moe_forward_ex(const void *x, const void *Wg, const float *bias, const void *W1,
                   const void *W3, const void *W2, const void *Ws1, const void *Ws3,
                   const void *Ws2, int d_ff_shared, int T, int E, int k, int d, int d_ff,
                   int dtype, const moe_options *opt, void *workspace, size_t workspace_bytes,
                   void *y, void *stream);

/* ------------------------------------------------------------------------
 * Weight-only FP8 experts for decode ("Mistral 8x7B SMoE architecture deep
 * dive", section 5.3: quantise only the expert weights, keep the router in
 * high precision, one scale per expert).  Format OCP FP8 E4M3 ("E4M3FN":
 * largest finite 448, no infinities).  Symmetric; an FP8 float needs no
 * zero-point.
 * ------------------------------------------------------------------------ */

/* Quantise E expert matrices of n elements each (W [E][n], dtype MOE_BF16 or
 * MOE_F32, any layout inside an expert): scale[e] = amax_e / 448 rounded to
 * fp32 (1 for an all-zero expert), amax_e the largest |w| of expert e, and
 * q[e][i] = the E4M3 code nearest to W[e][i] / scale[e] (quotient in fp64,
 * ties to the even mantissa, magnitudes above 448 give 448).  q [E][n] uint8
 * and scale [E] fp32 are device outputs; scale doubles as scratch during the
 * call.  Deterministic.  Used on W1 [E][d_ff][d], W3 and W2 [E][d][d_ff]. */
int moe_quantize_fp8(const void *W, int E, long long n, int dtype, uint8_t *q, float *scale,
                     void *stream);

/* The layer with FP8 experts: y = sum_j gate_j * W2'( act(W1' x, W3' x) ) with
 * W' = scale[e] * decode(q) (the router, activations and outputs stay bf16, as
 * does all arithmetic outside the weights: fp32 accumulation).
 *   x [T][d] bf16, Wg [E][d] bf16, bias as moe_forward; W1q, W3q [E][d_ff][d],
 *   W2q [E][d][d_ff] uint8 with scales s1, s3, s2 [E] fp32 (moe_quantize_fp8);
 *   opt: gate / activation / capacity variants as moe_forward_ex (NULL:
 *   defaults); no shared expert.
 *   workspace: moe_workspace_bytes(T, d, d_ff, E, k, 0, MOE_BF16) bytes.
 * Decode-sized batches: up to four tokens with d and d_ff multiples of 2048
 * up to 16384 (vector-ALU weight streaming), or batches averaging at most 96
 * rows per expert with d and d_ff multiples of 128 (64-row matrix-core tiles
 * that widen the codes to bf16 in LDS reads); MOE_EINVAL otherwise. */
int moe_forward_fp8(const void *x, const void *Wg, const float *bias, const uint8_t *W1q,
                    const uint8_t *W3q, const uint8_t *W2q, const float *s1, const float *s3,
                    const float *s2, int T, int E, int k, int d, int d_ff,
                    const moe_options *opt, void *workspace, size_t workspace_bytes, void *y,
                    void *stream);

/* ------------------------------------------------------------------------
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the layer
 * with its scratch in a static device array of MOE_NOALLOC_SCRATCH_BYTES
 * per GPU, which the library holds from its first use on a device until the
 * process ends.  Same arguments and results as moe_forward, without the
 * workspace; allocates and frees nothing.
 *   Returns MOE_ESCRATCH when the shape needs more scratch than the array
 *   holds, i.e. when moe_workspace_bytes for the same arguments exceeds
 *   MOE_NOALLOC_SCRATCH_BYTES (128 MiB: the Mixtral-shaped layer up to about
 *   1000 tokens, its decode steps, every 512-wide layer of 512 tokens).
 *   Every call on one GPU uses that GPU's one array: calls that overlap on a
 *   GPU (on different streams, or from different threads) race, and the
 *   intermediates of moe_workspace_offsets are not exposed.  Each call clears
 *   what its kernels need cleared; nothing depends on a previous call.
 * ------------------------------------------------------------------------ */
#define MOE_NOALLOC_SCRATCH_BYTES (128u << 20)
int moe_forward_noalloc(const void *x, const void *Wg, const float *bias, const void *W1,
                        const void *W3, const void *W2, const void *Ws1, const void *Ws3,
                        const void *Ws2, int d_ff_shared, int T, int E, int k, int d, int d_ff,
                        int dtype, void *y, void *stream);

/* Static text for a status code. */
const char *moe_strerror(int status);

#ifdef __cplusplus
}
#endif
#endif /* MOE_MI355X_H */
