/*
 * CPU oracle for the sparse Mixture-of-Experts feed-forward layer.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the plain, slow, obviously correct
 * reference that the GPU kernels are checked against.  Only the test suite,
 * the smoke entry point and the benchmark's CPU-baseline leg may load it; the
 * product path never does.  It shares no code, header or table with the HIP
 * library.
 *
 * Everything is computed in fp64 from the exact input values (fp32 inputs, or
 * bf16 bit patterns widened exactly), with plain loops in the order the
 * definitions below state.  No blocking, fusion or reordering beyond an
 * OpenMP split over independent tokens / slots.
 *
 * Sources (web pages; cited by title and section):
 *  [SMoE]  "Mistral 8x7B SMoE architecture deep dive: sparse activation and
 *          expert division of labour" (jsqmd.com news 960234), sections 2.2,
 *          3.1, 3.2.
 *  [CH10]  "Chapter 10 MoE: holding more knowledge with less compute"
 *          (LLMs-from-scratch ch.10), sections 10.1-10.5.
 *  [BENCH] "Trillion-parameter MoE activates only 4.9%: 7 expert configs
 *          measured" (m.xxqk.cn news 679798), parameter accounting paragraph
 *          and the numpy forward listing.
 *  [MIXA]  "Mixtral and MoE architecture" (astro-blog-cod.pages.dev), the
 *          MixtralMoE / FeedForward listing.
 *  [OVW]   "Mixtral 8x7B model architecture" (bjdmk.com.cn news 6109040),
 *          section 1.2 (the Router: softmax over all experts, then top-k).
 *  [SMoE] section 2.4 also states the expert capacity limit used below.
 *
 * Layouts (row-major; every weight held as a Linear weight [out][in]):
 *   x   [T][d]         Wg  [E][d]        bias [E] (fp32, optional)
 *   W1  [E][d_ff][d]   W3  [E][d_ff][d]  W2   [E][d][d_ff]
 *   Ws1 [d_ffs][d]     Ws3 [d_ffs][d]    Ws2  [d][d_ffs]   (shared expert)
 *
 * Parity status per function (pins live in the CPU test suite):
 *   orc_logits        pinned (numpy fp64 matmul)
 *   orc_topk          pinned (brute-force stable sort; constructed ties)
 *   orc_gate          pinned (closed forms; softmax-all + renormalise form)
 *   orc_count/permute pinned (bincount; numpy stable argsort)
 *   orc_swiglu_row    pinned (E=1,k=1 dense FFN via numpy matmul)
 *   orc_forward       pinned (k=E softmax-weighted sum; invariants)
 *   orc_param_count   pinned (50,331,648 stated as 50.3M on [BENCH])
 *   orc_gate_mode     pinned (torch softmax / sigmoid of the logits)
 *   act GLU_SIGMOID   pinned (dense FFN via torch; the [BENCH] fused-weight
 *                     formulation recomputed in numpy)
 *   orc_keep          pinned (brute force on tiny inputs; no-drop case)
 *   orc_capacity      pinned (the two worked numbers of [SMoE] 2.4)
 *   orc_entropy       pinned (closed forms; torch softmax + entr)
 *   orc_route_entropy pinned (per-token torch.topk of the tempered softmax)
 *   orc_route_entropy_batch pinned (torch.topk of the tempered softmax with
 *                     the batch's largest k; brute force on tiny batches)
 *   orc_fp8_decode    pinned (all 256 codes against torch.float8_e4m3fn)
 *   orc_fp8_encode    pinned (torch's float8_e4m3fn cast; brute-force nearest)
 *   orc_quantize_fp8  pinned (per-expert amax by numpy; round trip bounds)
 */
#include <math.h>
#ifdef _OPENMP
#include <omp.h>
#endif
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_F32 0
#define ORC_BF16 1
#define ORC_F64 2 /* fp64 arrays, e.g. dequantized weights */

/* Widen one stored element to double.  bf16 is the upper half of an IEEE
 * binary32, so the widening is exact. */
static double elem(const void *p, int dt, size_t i)
{
    if (dt == ORC_F64)
        return ((const double *)p)[i];
    if (dt == ORC_BF16) {
        uint32_t u = ((uint32_t)((const uint16_t *)p)[i]) << 16;
        float f;
        memcpy(&f, &u, sizeof f);
        return (double)f;
    }
    return (double)((const float *)p)[i];
}

static void row_to_double(const void *p, int dt, size_t off, int n, double *dst)
{
    for (int i = 0; i < n; ++i)
        dst[i] = elem(p, dt, off + (size_t)i);
}

static double dot(const double *a, const double *b, int n)
{
    double s = 0.0;
    for (int i = 0; i < n; ++i)
        s += a[i] * b[i];
    return s;
}

/* Router scores [SMoE 3.2; CH10 10.3; BENCH listing; MIXA listing]:
 * logits[t][e] = sum_i x[t][i] * Wg[e][i]  (+ bias[e] when given). */
void orc_logits(const void *x, const void *Wg, const float *bias, int dt,
                long T, int d, int E, double *logits)
{
    double *wg = malloc(sizeof(double) * (size_t)E * d);
    for (int e = 0; e < E; ++e)
        row_to_double(Wg, dt, (size_t)e * d, d, wg + (size_t)e * d);
#pragma omp parallel
    {
        double *xr = malloc(sizeof(double) * d);
#pragma omp for schedule(static)
        for (long t = 0; t < T; ++t) {
            row_to_double(x, dt, (size_t)t * d, d, xr);
            for (int e = 0; e < E; ++e) {
                double l = dot(xr, wg + (size_t)e * d, d);
                if (bias)
                    l += (double)bias[e];
                logits[(size_t)t * E + e] = l;
            }
        }
        free(xr);
    }
    free(wg);
}

/* Top-k selection [SMoE 2.2; CH10 10.3]: k rounds; each round takes the
 * largest logit not yet chosen, scanning experts in ascending order with a
 * strict '>' so an exact tie goes to the lower expert index.  idx[t][j] is
 * therefore ordered by descending logit.  Returns 0, or -1 on bad k. */
int orc_topk(const double *logits, long T, int E, int k, int32_t *idx)
{
    if (k < 1 || k > E)
        return -1;
    for (long t = 0; t < T; ++t) {
        const double *l = logits + (size_t)t * E;
        char *taken = calloc((size_t)E, 1);
        for (int j = 0; j < k; ++j) {
            int best = -1;
            for (int e = 0; e < E; ++e) {
                if (taken[e])
                    continue;
                if (best < 0 || l[e] > l[best])
                    best = e;
            }
            taken[best] = 1;
            idx[(size_t)t * k + j] = best;
        }
        free(taken);
    }
    return 0;
}

/* Gate weights [SMoE 3.2 step 3; CH10 10.3]: softmax over the k selected
 * logits only, so each token's gates sum to one.  Max-subtracted form:
 * gate_j = exp(l_j - l_0) / sum_j' exp(l_j' - l_0), l_0 the largest. */
void orc_gate(const double *logits, const int32_t *idx, long T, int E, int k,
              double *gate)
{
    for (long t = 0; t < T; ++t) {
        const double *l = logits + (size_t)t * E;
        const int32_t *ix = idx + (size_t)t * k;
        double m = l[ix[0]];
        double z = 0.0;
        for (int j = 0; j < k; ++j)
            z += exp(l[ix[j]] - m);
        for (int j = 0; j < k; ++j)
            gate[(size_t)t * k + j] = exp(l[ix[j]] - m) / z;
    }
}

/* Gate weights, all variants the pages print.  mode:
 *  0  softmax over the k selected logits (orc_gate above) [SMoE 3.2; CH10 10.3]
 *  1  softmax over all E logits, the selected entries taken as they are (no
 *     renormalisation, the gates sum to at most one) [OVW 1.2 Router]
 *  2  logistic sigmoid of each selected logit on its own [BENCH listing]. */
void orc_gate_mode(const double *logits, const int32_t *idx, long T, int E,
                   int k, int mode, double *gate)
{
    if (mode == 0) {
        orc_gate(logits, idx, T, E, k, gate);
        return;
    }
    for (long t = 0; t < T; ++t) {
        const double *l = logits + (size_t)t * E;
        const int32_t *ix = idx + (size_t)t * k;
        if (mode == 1) {
            double m = l[0];
            for (int e = 1; e < E; ++e)
                if (l[e] > m)
                    m = l[e];
            double zall = 0.0;
            for (int e = 0; e < E; ++e)
                zall += exp(l[e] - m);
            for (int j = 0; j < k; ++j)
                gate[(size_t)t * k + j] = exp(l[ix[j]] - m) / zall;
        } else {
            for (int j = 0; j < k; ++j)
                gate[(size_t)t * k + j] = 1.0 / (1.0 + exp(-l[ix[j]]));
        }
    }
}

/* Entropy-aware routing [OVW 4.1, the entropy-controlled strategy]: the
 * probabilities are a temperature-scaled softmax over all E scores,
 * p_e = exp(l_e / tau) / sum_e' exp(l_e' / tau) (tau = 0.1 on the page); the
 * token's entropy H = -sum_e p_e ln p_e decides its k: the larger k when
 * H > threshold (0.8 on the page), else one less (the page's 3 and 2).
 * orc_entropy: H per token, computed as ln Z - (1/Z) sum_e w_e u_e with
 * u_e = (l_e - m) / tau, w_e = exp(u_e), m the largest score, Z = sum w_e,
 * which is -sum p ln p rewritten so that p = 0 contributes 0. */
#define ORC_ENTROPY_TAU 0.1
#define ORC_ENTROPY_THRESHOLD 0.8
void orc_entropy(const double *logits, long T, int E, double tau, double *H)
{
    for (long t = 0; t < T; ++t) {
        const double *l = logits + (size_t)t * E;
        double m = l[0];
        for (int e = 1; e < E; ++e)
            if (l[e] > m)
                m = l[e];
        double z = 0.0, s1 = 0.0;
        for (int e = 0; e < E; ++e) {
            double u = (l[e] - m) / tau;
            double w = exp(u);
            z += w;
            s1 += w * u;
        }
        H[t] = log(z) - s1 / z;
    }
}

/* The routing of [OVW 4.1]: idx [T][k] holds the token's top k_t experts by
 * score (= by probability; descending, ties to the lower index), k_t = k when
 * H > threshold else k - 1, and -1 in the slot past k_t; gate [T][k] the
 * selected probabilities p_e as they are (no renormalisation; the page
 * returns the top-k values of the probabilities), 0 in an empty slot.
 * Reading: the page computes k per token but then takes the batch's largest
 * k for every token; the per-token k is used (the page's +12% compute over
 * top-2 fits only a per-token choice). */
int orc_route_entropy(const double *logits, long T, int E, int k, double tau,
                      double threshold, int32_t *idx, double *gate)
{
    if (k < 2 || k > E)
        return -1;
    double *H = malloc(sizeof(double) * (size_t)(T > 0 ? T : 1));
    orc_entropy(logits, T, E, tau, H);
    orc_topk(logits, T, E, k, idx);
    for (long t = 0; t < T; ++t) {
        const double *l = logits + (size_t)t * E;
        const int kt = H[t] > threshold ? k : k - 1;
        double m = l[0];
        for (int e = 1; e < E; ++e)
            if (l[e] > m)
                m = l[e];
        double z = 0.0;
        for (int e = 0; e < E; ++e)
            z += exp((l[e] - m) / tau);
        for (int j = 0; j < k; ++j) {
            size_t q = (size_t)t * k + j;
            if (j < kt) {
                gate[q] = exp((l[idx[q]] - m) / tau) / z;
            } else {
                idx[q] = -1;
                gate[q] = 0.0;
            }
        }
    }
    free(H);
    return 0;
}

/* The routing of [OVW 4.1] as its listing prints it: the per-token k_t as
 * above (k when H > threshold, else k - 1), then one k for the whole batch,
 * the largest k_t, so that every token keeps its top max_t k_t experts by
 * probability (descending, ties to the lower index) with the probabilities as
 * gates; the slot past that k (when it is k - 1) holds idx -1 and gate 0 for
 * every token.  Returns the batch's k, or -1 for k < 2 or k > E. */
int orc_route_entropy_batch(const double *logits, long T, int E, int k, double tau,
                            double threshold, int32_t *idx, double *gate)
{
    if (k < 2 || k > E)
        return -1;
    double *H = malloc(sizeof(double) * (size_t)(T > 0 ? T : 1));
    orc_entropy(logits, T, E, tau, H);
    int kb = k - 1;
    for (long t = 0; t < T; ++t)
        if (H[t] > threshold)
            kb = k;
    orc_topk(logits, T, E, k, idx);
    for (long t = 0; t < T; ++t) {
        const double *l = logits + (size_t)t * E;
        double m = l[0];
        for (int e = 1; e < E; ++e)
            if (l[e] > m)
                m = l[e];
        double z = 0.0;
        for (int e = 0; e < E; ++e)
            z += exp((l[e] - m) / tau);
        for (int j = 0; j < k; ++j) {
            size_t q = (size_t)t * k + j;
            if (j < kb) {
                const double w = exp((l[idx[q]] - m) / tau);
                gate[q] = w / z;
            } else {
                gate[q] = 0.0;
                idx[q] = -1; /* the slot past the batch's k */
            }
        }
    }
    free(H);
    return kb;
}

/* FP8 weights for the experts [SMoE 5.3: quantise only the expert weights,
 * keep the router in high precision, and give every expert its own scale so
 * that no error crosses experts].  Format: OCP FP8 E4M3 ("E4M3FN"): sign,
 * 4 exponent bits with bias 7, 3 mantissa bits; exponent field 0 holds the
 * subnormals m * 2^-9; no infinities; S.1111.111 is NaN; the largest finite
 * value is 1.75 * 2^8 = 448. */
double orc_fp8_decode(uint8_t c)
{
    int sign = c >> 7, e = (c >> 3) & 15, m = c & 7;
    double v;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        v = ldexp((double)m, -9);
    else
        v = ldexp(1.0 + m / 8.0, e - 7);
    return sign ? -v : v;
}

/* Nearest E4M3 value, ties to the even mantissa; magnitudes above 448 give
 * 448 (the format has no infinity).  Scales are chosen so that no weight
 * goes above 448 by more than a rounding of the scale. */
uint8_t orc_fp8_encode(double v)
{
    uint8_t sign = signbit(v) ? 0x80 : 0; /* -0 keeps its sign */
    double a = fabs(v);
    if (a >= 448.0)
        return sign | 0x7E; /* e = 15, m = 6: 448 */
    if (a < ldexp(1.0, -6)) {
        /* subnormal range: integer multiples of 2^-9 (8 * 2^-9 is the
         * smallest normal, encoded as e = 1, m = 0 by the same bits) */
        double m = rint(ldexp(a, 9)); /* rint: round half to even */
        return sign | (uint8_t)m;
    }
    int ex;
    frexp(a, &ex);       /* a = f * 2^ex, 0.5 <= f < 1 */
    int e = ex - 1;      /* a = (1 + x) * 2^e with 0 <= x < 1 */
    double m = rint((ldexp(a, -e) - 1.0) * 8.0);
    if (m == 8.0) {      /* rounded up to the next power of two */
        m = 0.0;
        e += 1;
    }
    if (e + 7 > 15 || (e + 7 == 15 && m > 6.0))
        return sign | 0x7E;
    return sign | (uint8_t)(((e + 7) << 3) | (int)m);
}

/* Weight-only FP8 experts: W holds E experts of n elements each (one matrix
 * per expert, any row layout).  scale[e] = amax_e / 448 rounded to fp32 (1 for
 * an all-zero expert), amax_e the largest |w| of the expert; q = E4M3 of
 * w / scale[e], the quotient taken in fp64.  The dequantized weight is
 * scale[e] * decode(q). */
void orc_quantize_fp8(const void *W, int dt, long E, long n, uint8_t *q, float *scale)
{
    for (long e = 0; e < E; ++e) {
        double amax = 0.0;
        for (long i = 0; i < n; ++i) {
            double a = fabs(elem(W, dt, (size_t)e * n + i));
            if (a > amax)
                amax = a;
        }
        float s = amax > 0.0 ? (float)(amax / 448.0) : 1.0f;
        scale[e] = s;
        for (long i = 0; i < n; ++i)
            q[(size_t)e * n + i] = orc_fp8_encode(elem(W, dt, (size_t)e * n + i) / (double)s);
    }
}

/* out[e][i] = scale[e] * decode(q[e][i]) (fp64, exact). */
void orc_dequant_fp8(const uint8_t *q, long E, long n, const float *scale, double *out)
{
    for (long e = 0; e < E; ++e)
        for (long i = 0; i < n; ++i)
            out[(size_t)e * n + i] = (double)scale[e] * orc_fp8_decode(q[(size_t)e * n + i]);
}

/* Expert capacity [SMoE 2.4]: an expert takes at most min(k*T, floor(cf*T))
 * of a batch's T tokens (the page's two examples: batch 32, k=2 -> min(64,
 * 1.2*32); batch 16 -> 1.2*16 = 19). */
long orc_capacity(long T, int k, double cf)
{
    long c = (long)floor(cf * (double)T);
    long m = (long)k * T;
    return c < m ? c : m;
}

/* Which pairs an expert keeps under a capacity [SMoE 2.4 states the limit but
 * not which pairs go; reading: an expert keeps its first `capacity` pairs in
 * ascending pair id p = t*k + j, i.e. earlier tokens first].  keep[p] = 1 or
 * 0.  A dropped pair contributes nothing and the token's other gates are not
 * renormalised. */
void orc_keep(const int32_t *idx, long T, int E, int k, long capacity,
              int32_t *keep)
{
    long *seen = calloc((size_t)E, sizeof(long));
    for (long p = 0; p < T * (long)k; ++p) {
        int e = idx[p];
        if (e < 0 || e >= E) { /* an empty slot (entropy-aware k) */
            keep[p] = 0;
            continue;
        }
        keep[p] = seen[e] < capacity ? 1 : 0;
        seen[e] += 1;
    }
    free(seen);
}

/* Tokens per expert [CH10 10.4 grouping by expert; BENCH listing's per-expert
 * row lists]: counts[e] = number of (token, slot) pairs routed to e;
 * offsets is the exclusive prefix sum, offsets[E] = T*k. */
void orc_count(const int32_t *idx, long T, int E, int k, int32_t *counts,
               int32_t *offsets)
{
    for (int e = 0; e < E; ++e)
        counts[e] = 0;
    for (long p = 0; p < T * (long)k; ++p)
        counts[idx[p]] += 1;
    offsets[0] = 0;
    for (int e = 0; e < E; ++e)
        offsets[e + 1] = offsets[e] + counts[e];
}

/* Grouping of pairs by expert [CH10 10.4 (nonzero / index_select); BENCH
 * listing (np.where per expert)]: both list an expert's rows in ascending
 * token order.  Flat pair id p = t*k + j; pairs are placed expert by expert,
 * ascending p inside each expert (a stable counting sort).
 * perm[s] = pair at sorted slot s; inv[p] = slot of pair p. */
void orc_permute(const int32_t *idx, long T, int E, int k,
                 const int32_t *offsets, int32_t *perm, int32_t *inv)
{
    int32_t *cursor = malloc(sizeof(int32_t) * (size_t)E);
    for (int e = 0; e < E; ++e)
        cursor[e] = offsets[e];
    for (long p = 0; p < T * (long)k; ++p) {
        int32_t s = cursor[idx[p]]++;
        perm[s] = (int32_t)p;
        inv[p] = s;
    }
    free(cursor);
}

/* One gated expert on one token: a = W1 x, c = W3 x (length dff),
 *   act 0 (SwiGLU) [SMoE 3.1; CH10 10.1; MIXA FeedForward]:
 *         h = SiLU(a) * c with SiLU(a) = a/(1+e^-a);
 *   act 1 (sigmoid GLU) [BENCH listing: the fused up projection's second half
 *         gates the first through a logistic sigmoid; here W1 is that gated
 *         half and W3 the other]: h = c / (1+e^-a);
 * out = W2 h (length d).  xr is the token row already widened to double;
 * w1/w3/w2 point at this expert's matrices, element offsets o1/o3/o2. */
static void swiglu(const double *xr, int d, int dff, const void *W1, size_t o1,
                   const void *W3, size_t o3, const void *W2, size_t o2, int dt,
                   int act, double *h, double *wrow, double *out)
{
    for (int n = 0; n < dff; ++n) {
        row_to_double(W1, dt, o1 + (size_t)n * d, d, wrow);
        double a = dot(xr, wrow, d);
        row_to_double(W3, dt, o3 + (size_t)n * d, d, wrow);
        double c = dot(xr, wrow, d);
        h[n] = act == 1 ? c / (1.0 + exp(-a)) : a / (1.0 + exp(-a)) * c;
    }
    for (int j = 0; j < d; ++j) {
        row_to_double(W2, dt, o2 + (size_t)j * dff, dff, wrow);
        out[j] = dot(h, wrow, dff);
    }
}

/* Exposed single-row expert evaluation (used by per-token sampled checks):
 * out[d] = W2_e(act(W1_e x_t, W3_e x_t)). */
void orc_swiglu_row(const void *x, int dt, long t, int d, const void *W1,
                    const void *W3, const void *W2, int e, int dff, int act,
                    double *out)
{
    int wmax = d > dff ? d : dff;
    double *xr = malloc(sizeof(double) * d);
    double *h = malloc(sizeof(double) * dff);
    double *wrow = malloc(sizeof(double) * wmax);
    row_to_double(x, dt, (size_t)t * d, d, xr);
    size_t eo = (size_t)e * dff * d;
    swiglu(xr, d, dff, W1, eo, W3, eo, W2, eo, dt, act, h, wrow, out);
    free(xr);
    free(h);
    free(wrow);
}

/* Whole layer, computed through the permutation (the pages group pairs by
 * expert before running each expert):
 *   Yp[s] = FFN_e(x_t) with p = perm[s], t = p / k, e = idx[p];
 *   y[t]  = sum_{j<k, pair kept} gate[t][j] * Yp[inv[t*k+j]]   (j ascending)
 *           + shared FFN(x_t) with weight 1 when Ws1 != NULL [CH10 10.5].
 * gate_mode (orc_gate_mode; 3: orc_route_entropy, 4: orc_route_entropy_batch,
 * both with the page's tau and threshold), act (swiglu) and capacity (orc_keep; a value
 * >= T*k drops nothing) select the variants; only kept pairs are placed, so
 * counts/offsets/perm cover the kept pairs and inv[p] = -1 for a dropped one.
 * Routing comes from `logits_in` when given (e.g. another implementation's
 * router scores), else from orc_logits.  Outputs that are non-NULL receive
 * the intermediates.  y is [T][d] in double.  Returns 0 or -1. */
int orc_forward_ex(const void *x, const void *Wg, const float *bias,
                   const void *W1, const void *W3, const void *W2,
                   const void *Ws1, const void *Ws3, const void *Ws2, int dffs,
                   long T, int E, int k, int d, int dff, int dt, int gate_mode,
                   int act, long capacity, const double *logits_in,
                   double *logits_out, int32_t *idx_out, double *gate_out,
                   int32_t *counts_out, int32_t *offsets_out,
                   int32_t *perm_out, int32_t *inv_out, double *y)
{
    if (T < 0 || E < 1 || k < 1 || k > E || d < 1 || dff < 1 || capacity < 0)
        return -1;
    long P = T * (long)k;
    double *logits = malloc(sizeof(double) * (size_t)(T > 0 ? T : 1) * E);
    if (logits_in)
        memcpy(logits, logits_in, sizeof(double) * (size_t)T * E);
    else
        orc_logits(x, Wg, bias, dt, T, d, E, logits);
    int32_t *idx = malloc(sizeof(int32_t) * (size_t)(P > 0 ? P : 1));
    double *gate = malloc(sizeof(double) * (size_t)(P > 0 ? P : 1));
    int32_t *counts = malloc(sizeof(int32_t) * (size_t)E);
    int32_t *offsets = malloc(sizeof(int32_t) * (size_t)(E + 1));
    int32_t *perm = malloc(sizeof(int32_t) * (size_t)(P > 0 ? P : 1));
    int32_t *inv = malloc(sizeof(int32_t) * (size_t)(P > 0 ? P : 1));
    int32_t *keep = malloc(sizeof(int32_t) * (size_t)(P > 0 ? P : 1));
    if (gate_mode == 3 || gate_mode == 4) {
        const int rc = gate_mode == 3
                           ? orc_route_entropy(logits, T, E, k, ORC_ENTROPY_TAU,
                                               ORC_ENTROPY_THRESHOLD, idx, gate)
                           : (orc_route_entropy_batch(logits, T, E, k, ORC_ENTROPY_TAU,
                                                      ORC_ENTROPY_THRESHOLD, idx, gate) < 0
                                  ? -1 : 0);
        if (rc != 0) {
            free(logits); free(idx); free(gate); free(counts); free(offsets);
            free(perm); free(inv); free(keep);
            return -1;
        }
    } else {
        orc_topk(logits, T, E, k, idx);
        orc_gate_mode(logits, idx, T, E, k, gate_mode, gate);
    }
    orc_keep(idx, T, E, k, capacity, keep);
    /* counts and the stable grouping over the kept pairs only */
    for (int e = 0; e < E; ++e)
        counts[e] = 0;
    for (long p = 0; p < P; ++p)
        if (keep[p])
            counts[idx[p]] += 1;
    offsets[0] = 0;
    for (int e = 0; e < E; ++e)
        offsets[e + 1] = offsets[e] + counts[e];
    {
        int32_t *cursor = malloc(sizeof(int32_t) * (size_t)E);
        for (int e = 0; e < E; ++e)
            cursor[e] = offsets[e];
        for (long p = 0; p < P; ++p) {
            if (!keep[p]) {
                inv[p] = -1;
                continue;
            }
            int32_t sl = cursor[idx[p]]++;
            perm[sl] = (int32_t)p;
            inv[p] = sl;
        }
        free(cursor);
    }
    const long nkept = offsets[E];

    double *Yp = malloc(sizeof(double) * (size_t)(P > 0 ? P : 1) * d);
    int wmax = d > dff ? d : dff;
    if (dffs > wmax)
        wmax = dffs;
#pragma omp parallel
    {
        double *xr = malloc(sizeof(double) * d);
        double *h = malloc(sizeof(double) * (dff > dffs ? dff : dffs));
        double *wrow = malloc(sizeof(double) * wmax);
#pragma omp for schedule(dynamic, 1)
        for (long s = 0; s < nkept; ++s) {
            long p = perm[s];
            long t = p / k;
            int e = idx[p];
            size_t eo = (size_t)e * dff * d;
            row_to_double(x, dt, (size_t)t * d, d, xr);
            swiglu(xr, d, dff, W1, eo, W3, eo, W2, eo, dt, act, h, wrow,
                   Yp + (size_t)s * d);
        }
#pragma omp for schedule(dynamic, 1)
        for (long t = 0; t < T; ++t) {
            double *yt = y + (size_t)t * d;
            for (int c = 0; c < d; ++c)
                yt[c] = 0.0;
            for (int j = 0; j < k; ++j) {
                int32_t sl = inv[(size_t)t * k + j];
                if (sl < 0)
                    continue; /* dropped by the capacity limit, or an empty slot */
                double g = gate[(size_t)t * k + j];
                const double *yp = Yp + (size_t)sl * d;
                for (int c = 0; c < d; ++c)
                    yt[c] += g * yp[c];
            }
            if (Ws1) {
                double *ys = malloc(sizeof(double) * d);
                row_to_double(x, dt, (size_t)t * d, d, xr);
                swiglu(xr, d, dffs, Ws1, 0, Ws3, 0, Ws2, 0, dt, act, h, wrow, ys);
                for (int c = 0; c < d; ++c)
                    yt[c] += ys[c];
                free(ys);
            }
        }
        free(xr);
        free(h);
        free(wrow);
    }

    if (logits_out)
        memcpy(logits_out, logits, sizeof(double) * (size_t)T * E);
    if (idx_out)
        memcpy(idx_out, idx, sizeof(int32_t) * (size_t)P);
    if (gate_out)
        memcpy(gate_out, gate, sizeof(double) * (size_t)P);
    if (counts_out)
        memcpy(counts_out, counts, sizeof(int32_t) * (size_t)E);
    if (offsets_out)
        memcpy(offsets_out, offsets, sizeof(int32_t) * (size_t)(E + 1));
    if (perm_out)
        memcpy(perm_out, perm, sizeof(int32_t) * (size_t)nkept);
    if (inv_out)
        memcpy(inv_out, inv, sizeof(int32_t) * (size_t)P);
    free(logits);
    free(idx);
    free(gate);
    free(counts);
    free(offsets);
    free(perm);
    free(inv);
    free(keep);
    free(Yp);
    return 0;
}

/* The method itself ("Chapter 10 MoE", section 10.3; "Mistral 8x7B SMoE
 * architecture deep dive", sections 3.1 and 3.2): softmax over the selected
 * logits, SwiGLU experts, no capacity limit. */
int orc_forward(const void *x, const void *Wg, const float *bias,
                const void *W1, const void *W3, const void *W2,
                const void *Ws1, const void *Ws3, const void *Ws2, int dffs,
                long T, int E, int k, int d, int dff, int dt,
                const double *logits_in, double *logits_out, int32_t *idx_out,
                double *gate_out, int32_t *counts_out, int32_t *offsets_out,
                int32_t *perm_out, int32_t *inv_out, double *y)
{
    return orc_forward_ex(x, Wg, bias, W1, W3, W2, Ws1, Ws3, Ws2, dffs, T, E, k,
                          d, dff, dt, 0, 0, T * (long)k, logits_in, logits_out,
                          idx_out, gate_out, counts_out, offsets_out, perm_out,
                          inv_out, y);
}

/* Output rows for a chosen list of tokens, given their routing (idx, gate
 * rows of those tokens; a zero gate marks a dropped pair): y[r] = sum_j
 * gate[r][j] * FFN_{idx[r][j]}(x_{tok[r]}) (+ shared FFN).  Each token's output depends only on its own routing, so a
 * sample of a large workload can be checked row by row. */
void orc_forward_rows(const void *x, const void *W1, const void *W3,
                      const void *W2, const void *Ws1, const void *Ws3,
                      const void *Ws2, int dffs, int k, int d, int dff, int dt,
                      int act, long nrows, const int64_t *tok,
                      const int32_t *idx, const double *gate, double *y)
{
    int wmax = d > dff ? d : dff;
    if (dffs > wmax)
        wmax = dffs;
#pragma omp parallel
    {
        double *xr = malloc(sizeof(double) * d);
        double *h = malloc(sizeof(double) * (dff > dffs ? dff : dffs));
        double *wrow = malloc(sizeof(double) * wmax);
        double *o = malloc(sizeof(double) * d);
#pragma omp for schedule(dynamic, 1)
        for (long r = 0; r < nrows; ++r) {
            double *yr = y + (size_t)r * d;
            row_to_double(x, dt, (size_t)tok[r] * d, d, xr);
            for (int c = 0; c < d; ++c)
                yr[c] = 0.0;
            for (int j = 0; j < k; ++j) {
                int e = idx[(size_t)r * k + j];
                double g = gate[(size_t)r * k + j];
                if (g == 0.0 || e < 0)
                    continue; /* dropped by a capacity limit, or an empty slot */
                size_t eo = (size_t)e * dff * d;
                swiglu(xr, d, dff, W1, eo, W3, eo, W2, eo, dt, act, h, wrow, o);
                for (int c = 0; c < d; ++c)
                    yr[c] += g * o[c];
            }
            if (Ws1) {
                swiglu(xr, d, dffs, Ws1, 0, Ws3, 0, Ws2, 0, dt, act, h, wrow, o);
                for (int c = 0; c < d; ++c)
                    yr[c] += o[c];
            }
        }
        free(xr);
        free(h);
        free(wrow);
        free(o);
    }
}

/* Parameter accounting [BENCH parameter paragraph]: a layer holds
 * 3 * d * E * d_ff expert weights (gate+up counted as two, down as one);
 * the router is not included. */
long long orc_param_count(long long d, long long E, long long dff)
{
    return 3LL * d * E * dff;
}

/* Fraction of expert parameters a token activates: k / E [BENCH parameter
 * paragraph; CH10 10.6]. */
double orc_active_fraction(int E, int k)
{
    return (double)k / (double)E;
}

/* Threads an OpenMP region of the oracle uses (for reporting CPU timings). */
int orc_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Threads for the oracle's later OpenMP regions (n >= 1; for timing it on a
 * given number of host cores). */
void orc_set_threads(int n)
{
#ifdef _OPENMP
    omp_set_num_threads(n > 0 ? n : 1);
#else
    (void)n;
#endif
}
