/*
 * oracle.c -- plain fp64 CPU oracle of the MoE layer forward.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call it: only the
 * tests, the smoke check and the bench's CPU-baseline leg load this library.
 * It shares no code, header, table or helper with the HIP library; it has its
 * own decoders for bf16, fp16 and int4 codes.  Every loop is the textbook
 * definition in double precision, parallelised (OpenMP) over the outermost
 * independent loop only, with no blocking, fusion or reordering.
 *
 * Sources ("the pages"):
 *   [P1] trdm.cn/news/527833, "Colibri：专为MoE模型优化的纯C高性能推理引擎"
 *   [P2] discosf.com/news/4731160, "Colibri不是一只蜂鸟，而是一套为前沿MoE模型量身定制的C语言推理引擎"
 *   [P3] wzjinhao.cn/news/17934, Colibri C engine walkthrough (section numbers as printed)
 *   [P4] mhpn.cn/news/2221639, "Colibri：轻量级MoE推理引擎的C语言实践"
 *   [P5] wth2jhl.online/blog/colibri-justvugg-deep-dive, "一只蜂鸟如何喂饱九头大象"
 *
 * Readings taken where the pages are silent (each also listed in the design notes):
 *   - selection is made on logits, ties go to the lower expert index, the k
 *     slots are in descending logit order;
 *   - gate weights are the softmax restricted to the k selected experts
 *     (the full softmax denominator cancels in the renormalisation);
 *   - the FFN is SwiGLU without biases: w1 = gate, w3 = up, w2 = down;
 *   - int4: symmetric codes in two's complement, 128-element groups along K,
 *     one fp16 scale per group, low nibble = even K index;
 *   - nothing is rounded: the oracle never stores an intermediate in a
 *     narrower type.
 *
 * Parity status: every function below is pinned by a CPU test against a
 * library routine, a closed form, a brute-force enumeration or an invariant
 * (k = E dense mixture, sum of gate weights, bijective dispatch, int4 = q*s).
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_F32 0
#define ORC_BF16 1
#define ORC_INT4_G128 2
#define ORC_INT4_G64 3
#define ORC_MXFP4 4
#define ORC_MXFP8 5

/* special-value conventions of the small float formats decoded below */
#define ORC_MF_IEEE 0     /* all-ones exponent: inf (zero mantissa) or NaN */
#define ORC_MF_FN 1       /* no infinities; only all-ones exponent and mantissa is NaN */
#define ORC_MF_FINITE 2   /* every code is a finite number */

#define ORC_OK 0
#define ORC_EINVAL (-1)

/* Threads the OpenMP loops below will use (reported beside CPU timings). */
int orc_num_threads(void) { return omp_get_max_threads(); }

/* Thread count for later calls (n >= 1), for timing runs at a stated count.
 * Touches no arithmetic: every loop computes the same values at any count. */
void orc_set_num_threads(int n)
{
    if (n >= 1)
        omp_set_num_threads(n);
}

/* ---------------------------------------------------------------- decoders */

/* bf16 is the upper half of an IEEE binary32 word. */
double orc_dec_bf16(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* IEEE binary16: 1 sign bit, 5 exponent bits (bias 15), 10 mantissa bits. */
double orc_dec_f16(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int ex = (h >> 10) & 0x1f;
    int man = h & 0x3ff;
    double v;
    if (ex == 0)
        v = ldexp((double)man, -24);                 /* zero and subnormals */
    else if (ex == 31)
        v = man ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + man), ex - 25);    /* (1 + man/1024) * 2^(ex-15) */
    return sign ? -v : v;
}

/* A small binary floating-point code: sign bit above ebits exponent bits
 * above mbits mantissa bits, exponent bias `bias`; exponent 0 is zero or
 * subnormal (m * 2^(1 - bias - mbits)), otherwise (2^mbits + m) *
 * 2^(e - bias - mbits).  `special` picks the format's treatment of the
 * all-ones exponent.  E4M3 of the OCP 8-bit formats is (4, 3, 7, FN); E2M1
 * of the OCP MX formats is (2, 1, 1, FINITE); IEEE binary16 is (5, 10, 15, IEEE). */
double orc_dec_minifloat(uint32_t code, int ebits, int mbits, int bias, int special)
{
    const uint32_t man = code & ((1u << mbits) - 1);
    const uint32_t ex = (code >> mbits) & ((1u << ebits) - 1);
    const int sign = (code >> (mbits + ebits)) & 1;
    const uint32_t emax = (1u << ebits) - 1;
    double v;
    if (ex == emax && special == ORC_MF_IEEE)
        v = man ? NAN : INFINITY;
    else if (ex == emax && special == ORC_MF_FN && man == (1u << mbits) - 1)
        v = NAN;
    else if (ex == 0)
        v = ldexp((double)man, 1 - bias - mbits);
    else
        v = ldexp((double)((1u << mbits) + man), (int)ex - bias - mbits);
    return sign ? -v : v;
}

/* E8M0 scale of the OCP MX formats: 2^(code - 127), code 255 is NaN. */
double orc_dec_e8m0(uint8_t code)
{
    return code == 255 ? NAN : ldexp(1.0, (int)code - 127);
}

/* One 4-bit two's-complement code from a packed byte: hi=0 low nibble. */
int orc_dec_int4(uint8_t byte, int hi)
{
    int v = hi ? (byte >> 4) & 0xf : byte & 0xf;
    return v >= 8 ? v - 16 : v;
}

static double act_at(const void *p, int dt, size_t i)
{
    if (dt == ORC_F32)
        return (double)((const float *)p)[i];
    return orc_dec_bf16(((const uint16_t *)p)[i]);
}

/* Element (row, kk) of a weight matrix stored row-major with K columns.
 * row already folds the expert index: row = e*N + n.  Quantised formats:
 * int4 codes q with one fp16 scale s per group of 128 (or 64) K elements,
 * w = q * s ([P5] §7.3); MX formats: E2M1 (two codes per byte, even K in the
 * low nibble) or E4M3 (one per byte) elements times the E8M0 scale of their
 * block of 32 K elements (the OCP microscaling formats behind the native
 * MXFP4 / FP8 checkpoints of [P5] §6). */
static double wt_at(const void *w, const void *s, int dt, size_t row, size_t K, size_t kk)
{
    if (dt == ORC_F32)
        return (double)((const float *)w)[row * K + kk];
    if (dt == ORC_BF16)
        return orc_dec_bf16(((const uint16_t *)w)[row * K + kk]);
    if (dt == ORC_INT4_G128 || dt == ORC_INT4_G64) {
        const size_t gs = dt == ORC_INT4_G128 ? 128 : 64;
        uint8_t b = ((const uint8_t *)w)[row * (K / 2) + kk / 2];
        int q = orc_dec_int4(b, (int)(kk & 1));
        double sc = orc_dec_f16(((const uint16_t *)s)[row * (K / gs) + kk / gs]);
        return (double)q * sc;
    }
    {
        const double x = orc_dec_e8m0(((const uint8_t *)s)[row * (K / 32) + kk / 32]);
        if (dt == ORC_MXFP8)
            return orc_dec_minifloat(((const uint8_t *)w)[row * K + kk], 4, 3, 7, ORC_MF_FN) * x;
        {
            uint8_t b = ((const uint8_t *)w)[row * (K / 2) + kk / 2];
            uint32_t c = (kk & 1) ? (b >> 4) & 0xf : b & 0xf;
            return orc_dec_minifloat(c, 2, 1, 1, ORC_MF_FINITE) * x;
        }
    }
}

/* ------------------------------------------------------------- router (A1) */
/* Gating network = linear layer then softmax over experts: [P1] §2.1, §3.2;
 * [P3] §3.2 (softmax(x*W + b)); [P4] §2.1 (W*x + b). */
int orc_router_logits(int T, int d, int E, int act, const void *x,
                      const float *wg, const float *b, double *logits)
{
    if (T < 0 || d <= 0 || E <= 0 || !x || !wg || !logits)
        return ORC_EINVAL;
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t) {
        for (int e = 0; e < E; ++e) {
            double acc = 0.0;
            for (int j = 0; j < d; ++j)
                acc += act_at(x, act, (size_t)t * d + j) * (double)wg[(size_t)e * d + j];
            if (b)
                acc += (double)b[e];
            logits[(size_t)t * E + e] = acc;
        }
    }
    return ORC_OK;
}

/* ------------------------------------------------------------ softmax (A2) */
/* Max-subtracted softmax over the E experts of each token: [P3] §3.2 detail 1,
 * [P1] §3.2 (subtract the maximum before exponentiating). */
int orc_softmax(int T, int E, const double *logits, double *probs)
{
    if (T < 0 || E <= 0 || !logits || !probs)
        return ORC_EINVAL;
    for (int t = 0; t < T; ++t) {
        const double *l = logits + (size_t)t * E;
        double m = l[0];
        for (int e = 1; e < E; ++e)
            if (l[e] > m)
                m = l[e];
        double s = 0.0;
        for (int e = 0; e < E; ++e)
            s += exp(l[e] - m);
        for (int e = 0; e < E; ++e)
            probs[(size_t)t * E + e] = exp(l[e] - m) / s;
    }
    return ORC_OK;
}

/* ------------------------------------------------ top-k + renormalise (A3) */
/* Take the k highest-scoring experts and renormalise their gate weights:
 * [P1] §2.1 (top-2 indices + normalised gate weights), §3.2 (maximum first,
 * then the runner-up).  Repeated selection of the first strict maximum among
 * the unchosen experts gives descending order with ties to the lower index. */
int orc_topk(int T, int E, int k, const double *logits, int32_t *idx, double *w)
{
    if (T < 0 || E <= 0 || k <= 0 || k > E || !logits || !idx)
        return ORC_EINVAL;
    for (int t = 0; t < T; ++t) {
        const double *l = logits + (size_t)t * E;
        char *chosen = (char *)calloc((size_t)E, 1);
        if (!chosen)
            return ORC_EINVAL;
        for (int j = 0; j < k; ++j) {
            int best = -1;
            for (int e = 0; e < E; ++e) {
                if (chosen[e])
                    continue;
                if (best < 0 || l[e] > l[best])
                    best = e;
            }
            chosen[best] = 1;
            idx[(size_t)t * k + j] = best;
        }
        free(chosen);
        if (w) {
            /* P[idx_j] / sum_m P[idx_m]: the full softmax denominator cancels,
             * leaving the softmax of the selected logits. */
            double m = l[idx[(size_t)t * k]];
            double s = 0.0;
            for (int j = 0; j < k; ++j)
                s += exp(l[idx[(size_t)t * k + j]] - m);
            for (int j = 0; j < k; ++j)
                w[(size_t)t * k + j] = exp(l[idx[(size_t)t * k + j]] - m) / s;
        }
    }
    return ORC_OK;
}

/* Gate weights for a given (possibly forced) expert choice. */
int orc_gate_weights(int T, int E, int k, const double *logits, const int32_t *idx, double *w)
{
    if (T < 0 || E <= 0 || k <= 0 || !logits || !idx || !w)
        return ORC_EINVAL;
    for (int t = 0; t < T; ++t) {
        const double *l = logits + (size_t)t * E;
        double m = l[idx[(size_t)t * k]];
        for (int j = 1; j < k; ++j)
            if (l[idx[(size_t)t * k + j]] > m)
                m = l[idx[(size_t)t * k + j]];
        double s = 0.0;
        for (int j = 0; j < k; ++j)
            s += exp(l[idx[(size_t)t * k + j]] - m);
        for (int j = 0; j < k; ++j)
            w[(size_t)t * k + j] = exp(l[idx[(size_t)t * k + j]] - m) / s;
    }
    return ORC_OK;
}

/* ----------------------------------------------------------- dispatch (A4) */
/* Group the T*k (token, slot) assignments by expert: per-expert histogram,
 * running offsets, then a stable placement pass (the counting sort of
 * [P2] §4.2, completed with the scatter the printed code leaves out; the
 * token_to_expert_map + expert_offset pair of [P1] §3.3).  Assignment a is
 * token a / k, slot a % k.  inv is the inverse permutation. */
int orc_dispatch(int T, int k, int E, const int32_t *idx, int32_t *counts,
                 int32_t *offsets, int32_t *perm, int32_t *inv)
{
    const int n = T * k;
    if (T < 0 || k <= 0 || E <= 0 || !idx || !counts || !offsets || !perm || !inv)
        return ORC_EINVAL;
    for (int a = 0; a < n; ++a)
        if (idx[a] < 0 || idx[a] >= E)
            return ORC_EINVAL;
    for (int e = 0; e < E; ++e)
        counts[e] = 0;
    for (int a = 0; a < n; ++a)
        counts[idx[a]] += 1;
    offsets[0] = 0;
    for (int e = 0; e < E; ++e)
        offsets[e + 1] = offsets[e] + counts[e];
    int32_t *cursor = (int32_t *)malloc(sizeof(int32_t) * (size_t)(E > 0 ? E : 1));
    if (!cursor)
        return ORC_EINVAL;
    for (int e = 0; e < E; ++e)
        cursor[e] = offsets[e];
    for (int a = 0; a < n; ++a)
        perm[cursor[idx[a]]++] = a;
    free(cursor);
    for (int p = 0; p < n; ++p)
        inv[perm[p]] = p;
    return ORC_OK;
}

/* ------------------------------------------------------ SwiGLU FFN (A5/A6) */
/* One expert applied to one activation row: h_f = silu(x . Wgate[f]) * (x . Wup[f]),
 * out_i = sum_f h_f * Wdown[i][f].  Three matrices per expert, gate/up/down
 * (w1/w3/w2), no biases: [P1] §3.1 (expert tensors packed w1, w2, w3),
 * [P1] §2.1 (per-expert FFN then weighted merge), [P3] §2.3 / §3.1.
 * Gate/up are [E][F][d], down is [E][d][F], K contiguous. */
static void swiglu_row(int d, int F, int act, int wt, const void *xrow_base, size_t xrow,
                       const void *wg, const void *wu, const void *wd,
                       const void *sg, const void *su, const void *sd,
                       int e, double *h, double *out)
{
    for (int f = 0; f < F; ++f) {
        double g = 0.0, u = 0.0;
        size_t row = (size_t)e * F + f;
        for (int j = 0; j < d; ++j) {
            double xv = act_at(xrow_base, act, xrow * d + j);
            g += xv * wt_at(wg, sg, wt, row, (size_t)d, (size_t)j);
            u += xv * wt_at(wu, su, wt, row, (size_t)d, (size_t)j);
        }
        h[f] = g / (1.0 + exp(-g)) * u;
    }
    for (int i = 0; i < d; ++i) {
        double acc = 0.0;
        size_t row = (size_t)e * d + i;
        for (int f = 0; f < F; ++f)
            acc += h[f] * wt_at(wd, sd, wt, row, (size_t)F, (size_t)f);
        out[i] = acc;
    }
}

static int wt_ok(int wt, int d, int F)
{
    if (wt == ORC_F32 || wt == ORC_BF16)
        return 1;
    if (wt == ORC_INT4_G128)
        return d % 128 == 0 && F % 128 == 0;
    if (wt == ORC_INT4_G64)
        return d % 64 == 0 && F % 64 == 0;
    return (wt == ORC_MXFP4 || wt == ORC_MXFP8) && d % 32 == 0 && F % 32 == 0;
}

/* Expert FFN over dispatched rows: row p of expert e's segment holds token
 * perm[p] / k.  Only experts with a non-empty segment touch their weights
 * ([P3] §2.3, active experts only). */
int orc_expert_ffn(int T, int d, int E, int k, int F, int act, int wt, const void *x,
                   const void *wg, const void *wu, const void *wd,
                   const void *sg, const void *su, const void *sd,
                   const int32_t *counts, const int32_t *offsets, const int32_t *perm,
                   double *y_perm)
{
    (void)counts;
    if (T < 0 || d <= 0 || E <= 0 || k <= 0 || F <= 0 || !x || !wg || !wu || !wd ||
        !offsets || !perm || !y_perm || !wt_ok(wt, d, F))
        return ORC_EINVAL;
    const int n = T * k;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int p = 0; p < n; ++p) {
        int e = 0;
        while (e < E && !(p >= offsets[e] && p < offsets[e + 1]))
            ++e;
        if (e == E) {
            bad = 1;
            continue;
        }
        double *h = (double *)malloc(sizeof(double) * (size_t)F);
        if (!h) {
            bad = 1;
            continue;
        }
        swiglu_row(d, F, act, wt, x, (size_t)(perm[p] / k), wg, wu, wd, sg, su, sd, e, h,
                   y_perm + (size_t)p * d);
        free(h);
    }
    return bad ? ORC_EINVAL : ORC_OK;
}

/* Always-on shared expert (a single expert applied to every token, weight 1). */
int orc_shared_ffn(int T, int d, int F, int act, int wt, const void *x,
                   const void *wg, const void *wu, const void *wd,
                   const void *sg, const void *su, const void *sd, double *ys)
{
    if (T < 0 || d <= 0 || F <= 0 || !x || !wg || !wu || !wd || !ys || !wt_ok(wt, d, F))
        return ORC_EINVAL;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int t = 0; t < T; ++t) {
        double *h = (double *)malloc(sizeof(double) * (size_t)F);
        if (!h) {
            bad = 1;
            continue;
        }
        swiglu_row(d, F, act, wt, x, (size_t)t, wg, wu, wd, sg, su, sd, 0, h,
                   ys + (size_t)t * d);
        free(h);
    }
    return bad ? ORC_EINVAL : ORC_OK;
}

/* ------------------------------------------------------------ combine (A8) */
/* Weighted merge back into token order ([P1] §2.1; the K-slot merge in token
 * order of [P4] §2.3):  y[t] = sum_j w[t][j] * y_perm[inv[t*k+j]] (+ ys[t])
 * (+ residual[t]), slots summed in order j = 0..k-1. */
int orc_combine(int T, int d, int k, const double *y_perm, const int32_t *inv,
                const double *w, const double *ys, const void *residual, int res_act,
                double *y)
{
    if (T < 0 || d <= 0 || k <= 0 || !y_perm || !inv || !w || !y)
        return ORC_EINVAL;
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t) {
        for (int i = 0; i < d; ++i) {
            double acc = 0.0;
            for (int j = 0; j < k; ++j)
                acc += w[(size_t)t * k + j] * y_perm[(size_t)inv[(size_t)t * k + j] * d + i];
            if (ys)
                acc += ys[(size_t)t * d + i];
            if (residual)
                acc += act_at(residual, res_act, (size_t)t * d + i);
            y[(size_t)t * d + i] = acc;
        }
    }
    return ORC_OK;
}

/* --------------------------------------------------- whole layer (A1..A8) */
/* The layer by its plain definition, token by token:
 *   y[t] = sum_j w[t][j] * SwiGLU_{idx[t][j]}(x[t]) + shared(x[t]) + residual[t].
 * forced_idx (or NULL) replaces the top-k choice; the gate weights are then
 * the renormalised softmax over the forced experts.  sel (n_sel tokens, or
 * NULL for all T) selects which output rows are computed: each token's output
 * depends only on its own row.  idx_out / w_out / logits_out may be NULL. */
int orc_layer_forward(int T, int d, int E, int k, int F, int act, int wt, const void *x,
                      const float *w_router, const float *b_router,
                      const void *wg, const void *wu, const void *wd,
                      const void *sg, const void *su, const void *sd,
                      const void *shg, const void *shu, const void *shd,
                      const void *shsg, const void *shsu, const void *shsd,
                      const void *residual, const int32_t *forced_idx,
                      int n_sel, const int32_t *sel,
                      double *y_out, int32_t *idx_out, double *w_out, double *logits_out)
{
    if (T < 0 || d <= 0 || E <= 0 || k <= 0 || k > E || F <= 0 || !x || !w_router ||
        !wg || !wu || !wd || !y_out || !wt_ok(wt, d, F))
        return ORC_EINVAL;
    const int nrows = sel ? n_sel : T;
    for (int r = 0; r < nrows; ++r)
        if (sel && (sel[r] < 0 || sel[r] >= T))
            return ORC_EINVAL;
    int bad = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : bad)
    for (int r = 0; r < nrows; ++r) {
        const int t = sel ? sel[r] : r;
        double *lg = (double *)malloc(sizeof(double) * (size_t)E);
        int32_t *id = (int32_t *)malloc(sizeof(int32_t) * (size_t)k);
        double *gw = (double *)malloc(sizeof(double) * (size_t)k);
        double *h = (double *)malloc(sizeof(double) * (size_t)F);
        double *o = (double *)malloc(sizeof(double) * (size_t)d);
        if (!lg || !id || !gw || !h || !o) {
            bad = 1;
            free(lg); free(id); free(gw); free(h); free(o);
            continue;
        }
        for (int e = 0; e < E; ++e) {
            double acc = 0.0;
            for (int j = 0; j < d; ++j)
                acc += act_at(x, act, (size_t)t * d + j) * (double)w_router[(size_t)e * d + j];
            if (b_router)
                acc += (double)b_router[e];
            lg[e] = acc;
        }
        if (forced_idx) {
            for (int j = 0; j < k; ++j) {
                id[j] = forced_idx[(size_t)t * k + j];
                if (id[j] < 0 || id[j] >= E)
                    bad = 1;
            }
            if (bad) {
                free(lg); free(id); free(gw); free(h); free(o);
                continue;
            }
            orc_gate_weights(1, E, k, lg, id, gw);
        } else {
            orc_topk(1, E, k, lg, id, gw);
        }
        double *y = y_out + (size_t)r * d;
        for (int i = 0; i < d; ++i)
            y[i] = 0.0;
        for (int j = 0; j < k; ++j) {
            swiglu_row(d, F, act, wt, x, (size_t)t, wg, wu, wd, sg, su, sd, id[j], h, o);
            for (int i = 0; i < d; ++i)
                y[i] += gw[j] * o[i];
        }
        if (shg) {
            swiglu_row(d, F, act, wt, x, (size_t)t, shg, shu, shd, shsg, shsu, shsd, 0, h, o);
            for (int i = 0; i < d; ++i)
                y[i] += o[i];
        }
        if (residual)
            for (int i = 0; i < d; ++i)
                y[i] += act_at(residual, act, (size_t)t * d + i);
        if (idx_out)
            for (int j = 0; j < k; ++j)
                idx_out[(size_t)r * k + j] = id[j];
        if (w_out)
            for (int j = 0; j < k; ++j)
                w_out[(size_t)r * k + j] = gw[j];
        if (logits_out)
            for (int e = 0; e < E; ++e)
                logits_out[(size_t)r * E + e] = lg[e];
        free(lg); free(id); free(gw); free(h); free(o);
    }
    return bad ? ORC_EINVAL : ORC_OK;
}

/* ------------------------------------- one-layer-ahead prediction score */
/* [P5] §4.2 (PILOT): the next layer's router, run one layer early, picks the
 * experts to fetch ahead; [P5] §二 quotes the share of the next layer's
 * experts it predicts.  For token t, the number of experts in both
 * pred[t][0..k) and actual[t][0..k) (each list holds k distinct experts);
 * hist[j] counts the tokens with j in common. */
int orc_topk_overlap(int T, int k, const int32_t *pred, const int32_t *actual, int32_t *hist)
{
    if (T < 0 || k <= 0 || !pred || !actual || !hist)
        return ORC_EINVAL;
    for (int j = 0; j <= k; ++j)
        hist[j] = 0;
    for (int t = 0; t < T; ++t) {
        int n = 0;
        for (int j = 0; j < k; ++j)
            for (int m = 0; m < k; ++m)
                if (pred[(size_t)t * k + j] == actual[(size_t)t * k + m]) {
                    ++n;
                    break;
                }
        hist[n] += 1;
    }
    return ORC_OK;
}

/* ------------------------------------------------------------ RMSNorm (A9) */
/* Pre-norm of the stacked workload: out = h / sqrt(mean(h^2) + eps) * gamma.
 * (The pages only name the residual around the MoE layer, [P3] §2.3; the
 * normalisation form is the stacked workload's definition.) */
int orc_rmsnorm(int T, int d, int act, const void *h, const float *gamma, double eps,
                double *out)
{
    if (T < 0 || d <= 0 || !h || !out)
        return ORC_EINVAL;
    for (int t = 0; t < T; ++t) {
        double ss = 0.0;
        for (int i = 0; i < d; ++i) {
            double v = act_at(h, act, (size_t)t * d + i);
            ss += v * v;
        }
        double r = 1.0 / sqrt(ss / d + eps);
        for (int i = 0; i < d; ++i)
            out[(size_t)t * d + i] = act_at(h, act, (size_t)t * d + i) * r *
                                     (gamma ? (double)gamma[i] : 1.0);
    }
    return ORC_OK;
}
