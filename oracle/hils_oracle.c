/*
 * hils_oracle.c -- plain fp64 CPU reference of the HiLS-Attention forward path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark may load this library.  It shares no code,
 * header, table or helper with the GPU library.
 *
 * Source: "Hierarchical Sparse Attention Done Right: Toward Infinite Context
 * Modeling" (HiLS-Attention).  Citations name the page and its section:
 *   [p1 BSA]   paper-body page, section "Block Sparse Attention" preliminaries
 *              (chunk partition, aligned window, candidate set, token logits,
 *              chunk masses, top-k selection).
 *   [p1 RQ1]   paper-body page, RQ1 (LogSumExp linearization, landmark query;
 *              every query scores all chunk summaries and retains k of them).
 *   [p1 RQ2]   paper-body page, RQ2 (hierarchical factorisation of weights).
 *   [p1 GQA]   paper-body page, implementation: GQA-aware chunk selection.
 *   [p1 Q-Cal] paper-body page, implementation: the partition estimate combines
 *              chunk-level surrogates with token-level attention mass.
 *   [p2 Eq.7], [p2 Eq.8], [p2 Eq.10]  summary page, Methodology 1 and 2.
 *
 * Everything is computed in double precision from the stored input bytes
 * (fp32 or bf16 values widen exactly).  The only roundings are the two storage
 * points of the path's outputs that later stages read back: the chunk summary
 * key k' (to the summary dtype) and the entropy bias b' (to fp32).
 *
 * Readings where the pages are silent (stated once here, used below):
 *   - token i lies in chunk floor(i/S); only complete chunks are summarised;
 *   - window left edge l_i = max(0, S*floor((i-W+1)/S)) (floor toward -inf);
 *     window = [l_i, i]; candidates C_i = {c : (c+1)*S <= l_i};
 *   - logit scale is the caller's `scale` (1/sqrt(d) by default) everywhere;
 *   - token logits use q, retrieval scores use q_hat;
 *   - GQA rank key r_c = max_h (s_hat_{h,c} - LSE_{c' in C_i} s_hat_{h,c'}),
 *     for a group of one head r_c = s_hat_c; ties go to the lower chunk index;
 *   - |C_i| <= k selects every candidate;
 *   - the window enters the normaliser at its true token-level log-mass.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ODT_F32 = 0, ODT_BF16 = 1, ODT_F64 = 2 };
enum { ORND_NONE = 0, ORND_F32 = 1, ORND_BF16 = 2 };

/* Read element i of an array of dtype dt, widened exactly to double. */
static double ld(const void* p, int dt, int64_t i) {
    if (dt == ODT_F32) return (double)((const float*)p)[i];
    if (dt == ODT_BF16) {
        uint32_t u = (uint32_t)((const uint16_t*)p)[i] << 16;
        float f;
        memcpy(&f, &u, sizeof f);
        return (double)f;
    }
    return ((const double*)p)[i];
}

/* Round a double once, to nearest with ties to even, onto the bf16 grid
 * (8 significant bits). */
static double round_bf16(double x) {
    if (x == 0.0 || !isfinite(x)) return x;
    int e;
    (void)frexp(fabs(x), &e);            /* |x| in [2^(e-1), 2^e) */
    int qe = e - 8;                      /* spacing of the bf16 grid there */
    if (qe < -133) qe = -133;            /* subnormal spacing */
    double r = nearbyint(ldexp(fabs(x), -qe));
    double y = ldexp(r, qe);
    if (y > 3.3895313892515355e38) y = INFINITY;
    return copysign(y, x);
}

static double round_to(double x, int mode) {
    if (mode == ORND_F32) return (double)(float)x;
    if (mode == ORND_BF16) return round_bf16(x);
    return x;
}

/* log(sum_j exp(x_j)) for n >= 1 values, max-shifted. */
static double lse(const double* x, int64_t n) {
    double m = -INFINITY;
    for (int64_t j = 0; j < n; ++j) if (x[j] > m) m = x[j];
    if (m == -INFINITY) return -INFINITY;
    double z = 0.0;
    for (int64_t j = 0; j < n; ++j) z += exp(x[j] - m);
    return m + log(z);
}

static int64_t floor_div(int64_t a, int64_t b) {
    int64_t q = a / b;
    if ((a % b != 0) && ((a < 0) != (b < 0))) --q;
    return q;
}

/* Threads an OpenMP region of the oracle uses (1 without OpenMP). */
int orc_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Set the number of threads later OpenMP regions use (no-op without OpenMP). */
void orc_set_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* [p1 BSA]: aligned window left edge and candidate count for position i. */
int64_t orc_window_left(int64_t i, int S, int W) {
    int64_t l = (int64_t)S * floor_div(i - (int64_t)W + 1, S);
    return l < 0 ? 0 : l;
}

int64_t orc_num_candidates(int64_t i, int S, int W) {
    return orc_window_left(i, S, W) / S;
}

/*
 * Landmark summaries, [p2 Eq.8] with [p1 RQ1] (landmark query gives q'_c).
 * For every (b, h, c) with c in [c0, c0+nc), g = h / (Hq/Hkv):
 *   s_j = scale * q'_{h,c} . k_{g,cS+j},  j = 0..S-1
 *   p = softmax(s);  k'_{h,c} = sum_j p_j k_{g,cS+j};  b'_{h,c} = -sum_j p_j log p_j
 * b' is evaluated as LSE(s) - sum_j p_j s_j, the same quantity without log(0).
 *
 * k      [B, Hkv, k_T, d]  dtype k_dt
 * ql     [B, Hq, ql_NC, d] dtype ql_dt
 * ksum   [B, Hq, ks_NC, d] doubles (rounded per ks_round)
 * bsum   [B, Hq, ks_NC]    doubles (rounded to fp32)
 */
int orc_summarize(int B, int Hq, int Hkv, int d, int S, double scale,
                  const void* k, int k_dt, int64_t k_T,
                  const void* ql, int ql_dt, int64_t ql_NC,
                  int64_t c0, int64_t nc, int ks_round,
                  double* ksum, double* bsum, int64_t ks_NC) {
    if (Hkv <= 0 || Hq % Hkv != 0 || S <= 0 || d <= 0) return -1;
    if ((c0 + nc) * S > k_T || c0 + nc > ql_NC || c0 + nc > ks_NC) return -2;
    const int G = Hq / Hkv;
    const int64_t total = (int64_t)B * Hq * nc;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t t = 0; t < total; ++t) {
        const int64_t c = c0 + t % nc;
        const int h = (int)((t / nc) % Hq);
        const int b = (int)(t / (nc * Hq));
        const int g = h / G;
        double* s = (double*)malloc(sizeof(double) * (size_t)S);
        double* p = (double*)malloc(sizeof(double) * (size_t)S);
        const int64_t qoff = (((int64_t)b * Hq + h) * ql_NC + c) * d;
        const int64_t koff = (((int64_t)b * Hkv + g) * k_T + c * S) * d;
        for (int j = 0; j < S; ++j) {
            double acc = 0.0;
            for (int e = 0; e < d; ++e) acc += ld(ql, ql_dt, qoff + e) * ld(k, k_dt, koff + (int64_t)j * d + e);
            s[j] = scale * acc;
        }
        const double L = lse(s, S);
        double ps = 0.0;
        for (int j = 0; j < S; ++j) {
            p[j] = exp(s[j] - L);
            ps += p[j] * s[j];
        }
        double* kout = ksum + (((int64_t)b * Hq + h) * ks_NC + c) * d;
        for (int e = 0; e < d; ++e) {
            double acc = 0.0;
            for (int j = 0; j < S; ++j) acc += p[j] * ld(k, k_dt, koff + (int64_t)j * d + e);
            kout[e] = round_to(acc, ks_round);
        }
        bsum[((int64_t)b * Hq + h) * ks_NC + c] = round_to(L - ps, ORND_F32);
        free(s);
        free(p);
    }
    return 0;
}

typedef struct { double r; int64_t c; } rank_entry;

/* Order: larger rank key first; equal keys -> lower chunk index first. */
static int rank_cmp(const void* a, const void* b) {
    const rank_entry* x = (const rank_entry*)a;
    const rank_entry* y = (const rank_entry*)b;
    if (x->r > y->r) return -1;
    if (x->r < y->r) return 1;
    return (x->c < y->c) ? -1 : (x->c > y->c);
}

static int cmp_i64(const void* a, const void* b) {
    int64_t x = *(const int64_t*)a, y = *(const int64_t*)b;
    return (x < y) ? -1 : (x > y);
}

/* Intra-group attention ([p1 BSA] token logits, [p2 Eq.10] first factor):
 * for keys/values rows [j0, j1) of KV head (b, g) and query vector qv:
 *   log Z = LSE_j (scale q.k_j);  o = sum_j exp(s_j - log Z) v_j. */
static double group_attend(const double* qv, int d, double scale,
                           const void* k, const void* v, int kv_dt, int64_t base,
                           int64_t j0, int64_t j1, double* s, double* o) {
    const int64_t n = j1 - j0;
    for (int64_t j = 0; j < n; ++j) {
        double acc = 0.0;
        const int64_t off = base + (j0 + j) * d;
        for (int e = 0; e < d; ++e) acc += qv[e] * ld(k, kv_dt, off + e);
        s[j] = scale * acc;
    }
    const double logZ = lse(s, n);
    for (int e = 0; e < d; ++e) o[e] = 0.0;
    for (int64_t j = 0; j < n; ++j) {
        const double w = exp(s[j] - logZ);
        const int64_t off = base + (j0 + j) * d;
        for (int e = 0; e < d; ++e) o[e] += w * ld(v, kv_dt, off + e);
    }
    return logZ;
}

/*
 * One query row per entry: (b, g, position i, row iq of the query arrays).
 * For each row and each head h of group g:
 *   s_hat_{h,c} = scale * q_hat_{h,i} . k'_{h,c} + b'_{h,c},  c in C_i     [p2 Eq.10 / p1 RQ1]
 *   Sel = top-k of the rank key over C_i (all of C_i if |C_i| <= k)      [p1 BSA, p1 GQA]
 *   per group gamma in Sel + {window}: log Z_gamma, o_gamma              [p2 Eq.10]
 *   log Zhat = LSE({s_hat_c : c in Sel} + {log Z_win})                    [p1 Q-Cal, p2 Eq.10]
 *   out = sum_c exp(s_hat_c - log Zhat) o_c + exp(log Z_win - log Zhat) o_win;  lse = log Zhat
 *
 * q, qh      [B, Hq, q_T, d]   dtype q_dt (row iq is the query of position i)
 * k, v       [B, Hkv, kv_T, d] dtype kv_dt (rows 0..i are read, nothing beyond)
 * ksum, bsum [B, Hq, ks_NC(, d)] doubles
 * forced_idx [nrows, topk] or NULL: use this selection instead of computing one
 * idx_out    [nrows, topk]       ascending chunk ids, -1 padded
 * ssel_out   [nrows, G, topk]    each head's s_hat on the selection, -inf padded
 * gap_out    [nrows]             r_(k) - r_(k+1); +inf when |C_i| <= k
 * ncand_out  [nrows]             |C_i|
 * out        [nrows, G, d], lse [nrows, G]
 * r_out      NULL or [nrows, r_stride]: the rank key of every candidate
 */
int orc_rows(int B, int Hq, int Hkv, int d, int S, int W, int topk, double scale,
             int64_t nrows, const int32_t* rb, const int32_t* rg, const int64_t* ri,
             const int64_t* rq,
             const void* q, const void* qh, int q_dt, int64_t q_T,
             const void* k, const void* v, int kv_dt, int64_t kv_T,
             const double* ksum, const double* bsum, int64_t ks_NC,
             const int32_t* forced_idx,
             int32_t* idx_out, double* ssel_out, double* gap_out, int64_t* ncand_out,
             double* out, double* lse_out, double* r_out, int64_t r_stride) {
    if (Hkv <= 0 || Hq % Hkv != 0 || topk < 0) return -1;
    const int G = Hq / Hkv;
    int err = 0;
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t t = 0; t < nrows; ++t) {
        const int b = rb[t], g = rg[t];
        const int64_t i = ri[t], iq = rq[t];
        if (b < 0 || b >= B || g < 0 || g >= Hkv || i < 0 || i >= kv_T || iq < 0 || iq >= q_T) {
#pragma omp atomic write
            err = -2;
            continue;
        }
        const int64_t lw = orc_window_left(i, S, W);
        const int64_t nc = lw / S;
        if (nc > ks_NC) {
#pragma omp atomic write
            err = -3;
            continue;
        }
        ncand_out[t] = nc;
        const int64_t nsel = nc < topk ? nc : topk;
        double* sh = (double*)malloc(sizeof(double) * (size_t)(G * (nc > 0 ? nc : 1)));
        double* qv = (double*)malloc(sizeof(double) * (size_t)d);
        int64_t* sel = (int64_t*)malloc(sizeof(int64_t) * (size_t)(topk > 0 ? topk : 1));
        /* retrieval scores of every candidate, per head */
        for (int hh = 0; hh < G; ++hh) {
            const int h = g * G + hh;
            const int64_t qo = (((int64_t)b * Hq + h) * q_T + iq) * d;
            for (int e = 0; e < d; ++e) qv[e] = ld(qh, q_dt, qo + e);
            for (int64_t c = 0; c < nc; ++c) {
                const double* kk = ksum + (((int64_t)b * Hq + h) * ks_NC + c) * d;
                double acc = 0.0;
                for (int e = 0; e < d; ++e) acc += qv[e] * kk[e];
                sh[hh * nc + c] = scale * acc + bsum[((int64_t)b * Hq + h) * ks_NC + c];
            }
        }
        /* rank keys and selection */
        double gap = INFINITY;
        if (forced_idx) {
            for (int64_t s = 0; s < nsel; ++s) {
                sel[s] = forced_idx[t * topk + s];
                if (sel[s] < 0 || sel[s] >= nc) {
#pragma omp atomic write
                    err = -4;
                    sel[s] = 0;
                }
            }
        } else if (nc > 0) {
            rank_entry* re = (rank_entry*)malloc(sizeof(rank_entry) * (size_t)nc);
            double* L = (double*)malloc(sizeof(double) * (size_t)G);
            for (int hh = 0; hh < G; ++hh) L[hh] = lse(sh + hh * nc, nc);
            for (int64_t c = 0; c < nc; ++c) {
                double r;
                if (G == 1) {
                    r = sh[c];
                } else {
                    r = -INFINITY;
                    for (int hh = 0; hh < G; ++hh) {
                        const double x = sh[hh * nc + c] - L[hh];
                        if (x > r) r = x;
                    }
                }
                re[c].r = r;
                re[c].c = c;
                if (r_out) r_out[t * r_stride + c] = r;
            }
            qsort(re, (size_t)nc, sizeof(rank_entry), rank_cmp);
            for (int64_t s = 0; s < nsel; ++s) sel[s] = re[s].c;
            if (nc > topk && topk > 0) gap = re[topk - 1].r - re[topk].r;
            free(re);
            free(L);
        }
        qsort(sel, (size_t)nsel, sizeof(int64_t), cmp_i64);
        gap_out[t] = gap;
        for (int s = 0; s < topk; ++s) idx_out[t * topk + s] = s < nsel ? (int32_t)sel[s] : -1;

        /* attention per head: window and selected chunks, then the fusion */
        const int64_t wlen = i - lw + 1;
        const int64_t smax = wlen > S ? wlen : S;
        double* s = (double*)malloc(sizeof(double) * (size_t)smax);
        double* o = (double*)malloc(sizeof(double) * (size_t)d);
        double* ow = (double*)malloc(sizeof(double) * (size_t)d);
        double* ws = (double*)malloc(sizeof(double) * (size_t)(nsel + 1));
        double* oc = (double*)malloc(sizeof(double) * (size_t)((nsel > 0 ? nsel : 1) * d));
        const int64_t kvb = ((int64_t)b * Hkv + g) * kv_T * d;
        for (int hh = 0; hh < G; ++hh) {
            const int h = g * G + hh;
            const int64_t qo = (((int64_t)b * Hq + h) * q_T + iq) * d;
            for (int e = 0; e < d; ++e) qv[e] = ld(q, q_dt, qo + e);
            const double logZw = group_attend(qv, d, scale, k, v, kv_dt, kvb, lw, i + 1, s, ow);
            for (int64_t sidx = 0; sidx < nsel; ++sidx) {
                const int64_t c = sel[sidx];
                (void)group_attend(qv, d, scale, k, v, kv_dt, kvb, c * S, c * S + S, s, oc + sidx * d);
                ws[sidx] = sh[hh * (nc > 0 ? nc : 1) + c];
                ssel_out[(t * G + hh) * topk + sidx] = ws[sidx];
            }
            for (int64_t sidx = nsel; sidx < topk; ++sidx) ssel_out[(t * G + hh) * topk + sidx] = -INFINITY;
            ws[nsel] = logZw;
            const double Lhat = lse(ws, nsel + 1);
            for (int e = 0; e < d; ++e) o[e] = exp(logZw - Lhat) * ow[e];
            for (int64_t sidx = 0; sidx < nsel; ++sidx) {
                const double w = exp(ws[sidx] - Lhat);
                for (int e = 0; e < d; ++e) o[e] += w * oc[sidx * d + e];
            }
            for (int e = 0; e < d; ++e) out[(t * G + hh) * d + e] = o[e];
            lse_out[t * G + hh] = Lhat;
        }
        free(s); free(o); free(ow); free(ws); free(oc);
        free(sh); free(qv); free(sel);
    }
    return err;
}

/*
 * Backward of the prefill forward ([p1 RQ2] and [p2 Eq.10]: the model's loss
 * reaches the landmark summaries and the calibrated query through the fused
 * weights; [p2 Eq.8] carries it on to the landmark queries and the keys).
 * The selection is held fixed (it is piecewise constant in the inputs): the
 * gradient is that of the forward with sel_idx forced.  Straight-through for
 * the storage rounding of k' (ksum holds the values the forward used).
 *
 * For each row (b, h, i) with upstream gradients g = dout, gl = dlse:
 *   w_c = exp(s_hat_c - lse), w_win = exp(log Z_win - lse)
 *   D = g . out,  D_c = g . o_c
 *   d s_hat_c = w_c (D_c - D + gl)
 *   chunk token j of c:  ds_ij = w_c p_cj (g . v_j - D_c),  dv_j += w_c p_cj g
 *   window token j:      ds_ij = a_ij (g . v_j - D + gl),    dv_j += a_ij g,
 *                        a_ij = exp(s_ij - lse)
 *   dq_i += scale sum_j ds_ij k_j,  dk_j += scale ds_ij q_i
 *   dq_hat_i += scale sum_c d s_hat_c k'_c,  dk'_c += scale d s_hat_c q_hat_i,
 *   db'_c += d s_hat_c
 * and for every summarised chunk (b, h, c), with p = softmax(s), s_j = scale q'_c . k_j:
 *   e_j = dk'_c . k_j - db'_c s_j,   ds_j = p_j (e_j - sum_l p_l e_l)
 *   dq'_c = scale sum_j ds_j k_j,    dk_j += p_j dk'_c + scale ds_j q'_c
 *
 * Arrays as in orc_summarize / orc_rows, all rows of all positions (T = q_T = kv_T):
 * sel_idx [B,Hkv,T,topk] (ascending, -1 pads), dout [B,Hq,T,d], dlse [B,Hq,T] or NULL
 * (doubles).  Outputs (doubles, overwritten): dq, dqh [B,Hq,T,d]; dk, dv [B,Hkv,T,d]
 * (dk includes the summaries' part); dks [B,Hq,NC,d]; dbs [B,Hq,NC]; dql [B,Hq,NC,d].
 */
int orc_prefill_backward(int B, int Hq, int Hkv, int d, int S, int W, int topk, double scale,
                         int64_t T, const void* q, const void* qh, const void* ql, int q_dt,
                         const void* k, const void* v, int kv_dt,
                         const double* ksum, const double* bsum, int64_t NC,
                         const int32_t* sel_idx, const double* dout, const double* dlse,
                         double* dq, double* dqh, double* dk, double* dv, double* dks,
                         double* dbs, double* dql) {
    if (Hkv <= 0 || Hq % Hkv != 0 || topk < 0 || NC != T / S) return -1;
    const int G = Hq / Hkv;
    memset(dq, 0, sizeof(double) * (size_t)(B * Hq * T * d));
    memset(dqh, 0, sizeof(double) * (size_t)(B * Hq * T * d));
    memset(dk, 0, sizeof(double) * (size_t)(B * Hkv * T * d));
    memset(dv, 0, sizeof(double) * (size_t)(B * Hkv * T * d));
    memset(dks, 0, sizeof(double) * (size_t)(B * Hq * NC * d));
    memset(dbs, 0, sizeof(double) * (size_t)(B * Hq * NC));
    memset(dql, 0, sizeof(double) * (size_t)(B * Hq * NC * d));
    int err = 0;
    /* one (b, g) per iteration: every accumulation stays inside it */
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t bg = 0; bg < (int64_t)B * Hkv; ++bg) {
        const int b = (int)(bg / Hkv), g = (int)(bg % Hkv);
        const int64_t kvb = ((int64_t)b * Hkv + g) * T * d;
        const int64_t smax = (int64_t)W + S > S ? (int64_t)W + 2 * S : 2 * S;
        double* qv = (double*)malloc(sizeof(double) * (size_t)d);
        double* gv = (double*)malloc(sizeof(double) * (size_t)d);
        double* s = (double*)malloc(sizeof(double) * (size_t)(smax > T ? smax : T + 1));
        double* oc = (double*)malloc(sizeof(double) * (size_t)d * (topk > 0 ? topk : 1));
        double* ow = (double*)malloc(sizeof(double) * (size_t)d);
        double* lz = (double*)malloc(sizeof(double) * (size_t)(topk > 0 ? topk : 1));
        double* sh = (double*)malloc(sizeof(double) * (size_t)(topk > 0 ? topk : 1));
        for (int hh = 0; hh < G; ++hh) {
            const int h = g * G + hh;
            for (int64_t i = 0; i < T; ++i) {
                const int64_t lw = orc_window_left(i, S, W);
                const int64_t nc = lw / S;
                const int64_t nsel = nc < topk ? nc : topk;
                const int64_t qo = (((int64_t)b * Hq + h) * T + i) * d;
                const int32_t* sel = sel_idx + (((int64_t)b * Hkv + g) * T + i) * topk;
                for (int e = 0; e < d; ++e) {
                    qv[e] = ld(q, q_dt, qo + e);
                    gv[e] = dout[qo + e];
                }
                const double gl = dlse ? dlse[((int64_t)b * Hq + h) * T + i] : 0.0;
                /* forward pieces */
                for (int64_t t = 0; t < nsel; ++t) {
                    const int64_t c = sel[t];
                    if (c < 0 || c >= nc) {
#pragma omp atomic write
                        err = -4;
                        continue;
                    }
                    const double* kk = ksum + (((int64_t)b * Hq + h) * NC + c) * d;
                    double acc = 0.0;
                    for (int e = 0; e < d; ++e) acc += ld(qh, q_dt, qo + e) * kk[e];
                    sh[t] = scale * acc + bsum[((int64_t)b * Hq + h) * NC + c];
                    lz[t] = group_attend(qv, d, scale, k, v, kv_dt, kvb, c * S, c * S + S, s, oc + t * d);
                }
                const double lzw = group_attend(qv, d, scale, k, v, kv_dt, kvb, lw, i + 1, s, ow);
                double lhat = lzw;
                {
                    double m = lzw;
                    for (int64_t t = 0; t < nsel; ++t) if (sh[t] > m) m = sh[t];
                    double z = exp(lzw - m);
                    for (int64_t t = 0; t < nsel; ++t) z += exp(sh[t] - m);
                    lhat = m + log(z);
                }
                const double ww = exp(lzw - lhat);
                double Dd = 0.0, Dw = 0.0;
                for (int e = 0; e < d; ++e) Dw += gv[e] * ow[e];
                Dd = ww * Dw;
                for (int64_t t = 0; t < nsel; ++t) {
                    double Dc = 0.0;
                    for (int e = 0; e < d; ++e) Dc += gv[e] * oc[t * d + e];
                    Dd += exp(sh[t] - lhat) * Dc;
                }
                /* selected chunks */
                for (int64_t t = 0; t < nsel; ++t) {
                    const int64_t c = sel[t];
                    if (c < 0 || c >= nc) continue;
                    const double wc = exp(sh[t] - lhat);
                    double Dc = 0.0;
                    for (int e = 0; e < d; ++e) Dc += gv[e] * oc[t * d + e];
                    const double dsh = wc * (Dc - Dd + gl);
                    const double* kk = ksum + (((int64_t)b * Hq + h) * NC + c) * d;
                    double* dkk = dks + (((int64_t)b * Hq + h) * NC + c) * d;
                    for (int e = 0; e < d; ++e) {
                        dqh[qo + e] += scale * dsh * kk[e];
                        dkk[e] += scale * dsh * ld(qh, q_dt, qo + e);
                    }
                    dbs[((int64_t)b * Hq + h) * NC + c] += dsh;
                    for (int64_t j = c * S; j < c * S + S; ++j) {
                        double sj = 0.0, gvj = 0.0;
                        for (int e = 0; e < d; ++e) {
                            sj += qv[e] * ld(k, kv_dt, kvb + j * d + e);
                            gvj += gv[e] * ld(v, kv_dt, kvb + j * d + e);
                        }
                        const double pj = exp(scale * sj - lz[t]);
                        const double dsj = wc * pj * (gvj - Dc);
                        for (int e = 0; e < d; ++e) {
                            dq[qo + e] += scale * dsj * ld(k, kv_dt, kvb + j * d + e);
                            dk[kvb + j * d + e] += scale * dsj * qv[e];
                            dv[kvb + j * d + e] += wc * pj * gv[e];
                        }
                    }
                }
                /* window tokens */
                for (int64_t j = lw; j <= i; ++j) {
                    double sj = 0.0, gvj = 0.0;
                    for (int e = 0; e < d; ++e) {
                        sj += qv[e] * ld(k, kv_dt, kvb + j * d + e);
                        gvj += gv[e] * ld(v, kv_dt, kvb + j * d + e);
                    }
                    const double aj = exp(scale * sj - lhat);
                    const double dsj = aj * (gvj - Dd + gl);
                    for (int e = 0; e < d; ++e) {
                        dq[qo + e] += scale * dsj * ld(k, kv_dt, kvb + j * d + e);
                        dk[kvb + j * d + e] += scale * dsj * qv[e];
                        dv[kvb + j * d + e] += aj * gv[e];
                    }
                }
            }
            /* summaries of this head: Eq. 8 backward */
            for (int64_t c = 0; c < NC; ++c) {
                const int64_t qlo = (((int64_t)b * Hq + h) * NC + c) * d;
                const double* dkc = dks + qlo;
                const double dbc = dbs[((int64_t)b * Hq + h) * NC + c];
                double* pp = s;   /* p_j, then reuse */
                double m = -INFINITY;
                double* sj = (double*)malloc(sizeof(double) * (size_t)S);
                double* ej = (double*)malloc(sizeof(double) * (size_t)S);
                for (int j = 0; j < S; ++j) {
                    double acc = 0.0;
                    for (int e = 0; e < d; ++e) acc += ld(ql, q_dt, qlo + e) * ld(k, kv_dt, kvb + (c * S + j) * d + e);
                    sj[j] = scale * acc;
                    if (sj[j] > m) m = sj[j];
                }
                double z = 0.0;
                for (int j = 0; j < S; ++j) z += exp(sj[j] - m);
                double pe = 0.0;
                for (int j = 0; j < S; ++j) {
                    pp[j] = exp(sj[j] - m) / z;
                    double acc = 0.0;
                    for (int e = 0; e < d; ++e) acc += dkc[e] * ld(k, kv_dt, kvb + (c * S + j) * d + e);
                    ej[j] = acc - dbc * sj[j];
                    pe += pp[j] * ej[j];
                }
                for (int j = 0; j < S; ++j) {
                    const double dsj = pp[j] * (ej[j] - pe);
                    for (int e = 0; e < d; ++e) {
                        dql[qlo + e] += scale * dsj * ld(k, kv_dt, kvb + (c * S + j) * d + e);
                        dk[kvb + (c * S + j) * d + e] += pp[j] * dkc[e] + scale * dsj * ld(ql, q_dt, qlo + e);
                    }
                }
                free(sj);
                free(ej);
            }
        }
        free(qv); free(gv); free(s); free(oc); free(ow); free(lz); free(sh);
    }
    return err;
}

/*
 * Naive Block Sparse Attention selection ([p1 BSA]: the chunk mass of a
 * candidate chunk is the sum of the exponentiated token logits of the query
 * against the chunk's keys; naive BSA keeps the k candidates of largest mass,
 * which needs every token logit).  For each row (b, g, i) and head h of g:
 *   log Z_{h,c} = LSE_{j in chunk c} scale * q_{h,i} . k_j,   c in C_i
 * and the selection takes the group rule of the retrieval scores with log Z in
 * place of s_hat ([p1 GQA]): r_c = log Z_c for a group of one head, else
 * r_c = max_h (log Z_{h,c} - LSE_{c'} log Z_{h,c'}); top-k by r, ties to the
 * lower chunk index; all of C_i when |C_i| <= k.
 *
 * q [B,Hq,q_T,d] (row iq is the query of position i), k [B,Hkv,kv_T,d].
 * idx_out [nrows, topk] ascending, -1 padded; gap_out [nrows] r_(k) - r_(k+1)
 * (+inf when |C_i| <= k); ncand_out [nrows]; r_out NULL or [nrows, r_stride];
 * lz_out NULL or [nrows, G, lz_stride]: log Z of every candidate per head.
 */
int orc_bsa_rows(int B, int Hq, int Hkv, int d, int S, int W, int topk, double scale,
                 int64_t nrows, const int32_t* rb, const int32_t* rg, const int64_t* ri,
                 const int64_t* rq, const void* q, int q_dt, int64_t q_T,
                 const void* k, int kv_dt, int64_t kv_T,
                 int32_t* idx_out, double* gap_out, int64_t* ncand_out,
                 double* r_out, int64_t r_stride, double* lz_out, int64_t lz_stride) {
    if (Hkv <= 0 || Hq % Hkv != 0 || topk < 0) return -1;
    const int G = Hq / Hkv;
    int err = 0;
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t t = 0; t < nrows; ++t) {
        const int b = rb[t], g = rg[t];
        const int64_t i = ri[t], iq = rq[t];
        if (b < 0 || b >= B || g < 0 || g >= Hkv || i < 0 || i >= kv_T || iq < 0 || iq >= q_T) {
#pragma omp atomic write
            err = -2;
            continue;
        }
        const int64_t nc = orc_window_left(i, S, W) / S;
        if ((r_out && nc > r_stride) || (lz_out && nc > lz_stride)) {
#pragma omp atomic write
            err = -3;
            continue;
        }
        ncand_out[t] = nc;
        const int64_t nsel = nc < topk ? nc : topk;
        double* lz = (double*)malloc(sizeof(double) * (size_t)(G * (nc > 0 ? nc : 1)));
        double* qx = (double*)malloc(sizeof(double) * (size_t)d);
        double* s = (double*)malloc(sizeof(double) * (size_t)S);
        int64_t* sel = (int64_t*)malloc(sizeof(int64_t) * (size_t)(topk > 0 ? topk : 1));
        const int64_t kvb = ((int64_t)b * Hkv + g) * kv_T * d;
        /* exact chunk masses per head */
        for (int hh = 0; hh < G; ++hh) {
            const int h = g * G + hh;
            const int64_t qo = (((int64_t)b * Hq + h) * q_T + iq) * d;
            for (int e = 0; e < d; ++e) qx[e] = ld(q, q_dt, qo + e);
            for (int64_t c = 0; c < nc; ++c) {
                for (int j = 0; j < S; ++j) {
                    double acc = 0.0;
                    const int64_t off = kvb + (c * S + j) * d;
                    for (int e = 0; e < d; ++e) acc += qx[e] * ld(k, kv_dt, off + e);
                    s[j] = scale * acc;
                }
                lz[hh * nc + c] = lse(s, S);
                if (lz_out) lz_out[(t * G + hh) * lz_stride + c] = lz[hh * nc + c];
            }
        }
        double gap = INFINITY;
        if (nc > 0) {
            rank_entry* re = (rank_entry*)malloc(sizeof(rank_entry) * (size_t)nc);
            double* L = (double*)malloc(sizeof(double) * (size_t)G);
            for (int hh = 0; hh < G; ++hh) L[hh] = lse(lz + hh * nc, nc);
            for (int64_t c = 0; c < nc; ++c) {
                double best = -INFINITY;
                if (G == 1) {
                    best = lz[c];
                } else {
                    for (int hh = 0; hh < G; ++hh) best = fmax(best, lz[hh * nc + c] - L[hh]);
                }
                re[c].r = best;
                re[c].c = c;
                if (r_out) r_out[t * r_stride + c] = best;
            }
            qsort(re, (size_t)nc, sizeof(rank_entry), rank_cmp);
            for (int64_t sidx = 0; sidx < nsel; ++sidx) sel[sidx] = re[sidx].c;
            if (nc > topk && topk > 0) gap = re[topk - 1].r - re[topk].r;
            free(re);
            free(L);
        }
        qsort(sel, (size_t)nsel, sizeof(int64_t), cmp_i64);
        gap_out[t] = gap;
        for (int sidx = 0; sidx < topk; ++sidx) idx_out[t * topk + sidx] = sidx < nsel ? (int32_t)sel[sidx] : -1;
        free(lz); free(qx); free(s); free(sel);
    }
    return err;
}

/*
 * Low-rank query calibration ([p1 Q-Cal] and the summary page's practical
 * enhancements: the retrieval query is the token query plus a rank-r correction
 * of the token's hidden state, q_hat = q + W_up W_down h).  For every b, t:
 *   z_j = sum_m w_down[j, m] h[b, t, m]                         (j < r)
 *   q_hat[b, hd, t, e] = q[b, hd, t, e] + sum_j w_up[hd, e, j] z_j
 * rounded once to `round_mode` (the stored query the scoring reads).
 * h [B, T, dm], w_down [r, dm], w_up [Hq, d, r], q [B, Hq, T, d], all of dtype dt;
 * out [B, Hq, T, d] doubles.
 */
int orc_qcal(int B, int Hq, int d, int64_t T, int dm, int r, const void* h, const void* w_down,
             const void* w_up, const void* q, int dt, int round_mode, double* out) {
    if (B < 0 || Hq < 0 || d < 0 || T < 0 || dm < 0 || r < 0) return -1;
    int err = 0;
#pragma omp parallel for schedule(static)
    for (int64_t bt = 0; bt < (int64_t)B * T; ++bt) {
        const int64_t b = bt / T, t = bt % T;
        double* z = (double*)malloc(sizeof(double) * (size_t)(r > 0 ? r : 1));
        if (!z) {
#pragma omp atomic write
            err = -2;
            continue;
        }
        for (int j = 0; j < r; ++j) {
            double acc = 0.0;
            for (int m = 0; m < dm; ++m) acc += ld(w_down, dt, (int64_t)j * dm + m) * ld(h, dt, bt * dm + m);
            z[j] = acc;
        }
        for (int hd = 0; hd < Hq; ++hd) {
            for (int e = 0; e < d; ++e) {
                double acc = 0.0;
                for (int j = 0; j < r; ++j) acc += ld(w_up, dt, ((int64_t)hd * d + e) * r + j) * z[j];
                const int64_t o = (((int64_t)b * Hq + hd) * T + t) * d + e;
                out[o] = round_to(ld(q, dt, o) + acc, round_mode);
            }
        }
        free(z);
    }
    return err;
}
