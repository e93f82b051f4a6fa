/*
 * forkgdn_oracle.c -- plain, slow fp64 CPU reference for exact state forking.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg load this file's library.  It shares no code,
 * header, table or helper with the HIP library, and the HIP library never
 * links it.
 *
 * What it computes, and from which passage:
 *
 *  - Indexing (Flide, section 3.2, the per-token request/branch/position
 *    metadata under Eq. 2): a segment's first position is its parent's first
 *    position plus its fork offset, so positions of a question continue from
 *    the end of the state it forks from.
 *
 *  - Attention (Flide, section 3.2.1, Eq. 3, generalised to deeper trees as a
 *    sequence of aliases, ForkServe item 1; the softmax attention definition
 *    of the Flex page, section 2.1, Eq. 1): every live segment s defines the
 *    isolated sequence  P(s) = history(root) + visible prefix of each ancestor
 *    + s.  A token's output is plain causal softmax attention over P(s), in
 *    fp64.  This is Proposition 3.1 taken literally: each branch equals its
 *    own isolated forward pass.
 *
 *    Two more visibility rules of the same section: a sliding-window layer
 *    of width W also requires t_x - t_y < W (positions along P(s) are the
 *    standalone positions, so the same keys are chosen); a two-way layer
 *    (a model that reads each block both ways, Flide appendix H) drops
 *    t_y <= t_x, so a row sees every token of its own segment and each
 *    ancestor's visible prefix -- the state still never reads a question.
 *
 *  - Gated DeltaNet (Flide, section 3.2.2, Eq. 4): along the same isolated
 *    sequence, token by token,
 *        S_t = a_t * S_{t-1} (I - b_t k_t k_t^T) + b_t v_t k_t^T,  o_t = S_t q_t
 *    with S in R^{dv x dk}, a zero initial state for a fresh root, and the
 *    saved fp32 state for a cached history (Flide, section 3.4).
 *
 *  - Projection (Flide, section 3.5: in a batch-invariant engine every matrix
 *    product sums each output element in one order whatever the number of
 *    rows; section 3.3.3: the last layer's products run only at the rows of
 *    the readout index buffer): the plain definition y[m][n] = sum_k
 *    x[r(m)][k] w[n][k] with r(m) an index buffer of rows, in fp64.
 *
 *  - Short causal convolution (Flide, section 3.2.2: in front of the Gated
 *    DeltaNet rule a short causal convolution mixes each token with its few
 *    predecessors, and the first tokens of a question see the last tokens
 *    of its state; section 3.4: a checkpoint keeps the convolution window):
 *    along the same isolated sequence, y_t[c] = sum_{i<W} w[c][i] x_{t-i}[c],
 *    zero before the sequence's first row.  The pages give neither the width
 *    nor an activation: here it is depthwise, linear, width W.
 *
 * Two evaluation modes give identical bits (same operations, same order):
 *   mode 0 (literal): every live leaf's whole root-to-leaf path runs as its own
 *      sequence; tokens shared by several paths are compared bit for bit, and
 *      mismatches are counted.  Segment tails that lie on no leaf path (a
 *      child forked before the parent's end) run their own path P(s).
 *   mode 1 (rows/tree): attention computes only the selected rows of each
 *      segment over P(s); GDN runs each segment once from its parent's state
 *      at the fork offset.  Used at large sizes; cross-checked against mode 0.
 *
 * Readings where the pages are silent (each listed in the design notes):
 *   GQA groups are contiguous (q head h reads kv head h / (Hq/Hkv)); GDN
 *   v-head h reads q/k head h / (Hv/Hk); a and b are given after the
 *   sigmoid; cached segments are roots or children of cached segments, and a
 *   live child of a cached segment forks at its end.
 *
 * Build: gcc -O2 -fopenmp -shared -fPIC (no -ffast-math: fp64 order matters).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* Planted mistakes for the pin suite's mutation tests (tests plant them here,
   on the CPU).  The default build defines none, so every MUT(n) is 0. */
#ifndef ORACLE_MUTANT
#define ORACLE_MUTANT 0
#endif
#define MUT(n) (ORACLE_MUTANT == (n))

#define OR_OK 0
#define OR_E_ARG -1        /* bad sizes / null pointers                          */
#define OR_E_SEG_RANGE -2  /* a token names a segment outside [0, S)             */
#define OR_E_NONCONTIG -3  /* a segment's tokens are not contiguous in the stream */
#define OR_E_PARENT -4     /* parent index out of range or self                  */
#define OR_E_CYCLE -5      /* parent chain does not reach a root                 */
#define OR_E_FORK -6       /* fork outside [0, parent length], or root fork != 0 */
#define OR_E_EMPTY -7      /* live segment with no tokens / cached with tokens   */
#define OR_E_CACHED -8     /* cached segment below a live one, or a live child of
                              a cached segment that forks before its end         */

/* ------------------------------------------------------------------------ */
/* Indexing                                                                  */
/* ------------------------------------------------------------------------ */

int or_index(int T, int S, const int *tok_seg, const int *seg_parent, const int *seg_fork,
             const int *seg_cached_len, int *seg_start, int *seg_len, int *seg_pos0,
             int *seg_depth, int *seg_root, int *tok_pos)
{
    if (T < 0 || S <= 0 || !seg_parent || !seg_fork || !seg_cached_len) return OR_E_ARG;
    if (T > 0 && !tok_seg) return OR_E_ARG;
    int *count = calloc((size_t)S, sizeof(int));
    int *first = malloc((size_t)S * sizeof(int));
    int *last = malloc((size_t)S * sizeof(int));
    int rc = OR_OK;
    for (int s = 0; s < S; ++s) { first[s] = -1; last[s] = -1; }
    for (int t = 0; t < T; ++t) {
        int s = tok_seg[t];
        if (s < 0 || s >= S) { rc = OR_E_SEG_RANGE; goto done; }
        if (first[s] < 0) first[s] = t;
        last[s] = t;
        count[s]++;
    }
    for (int s = 0; s < S; ++s) {
        int cached = seg_cached_len[s];
        if (cached < 0) { rc = OR_E_EMPTY; goto done; }
        if (cached > 0 && count[s] > 0) { rc = OR_E_EMPTY; goto done; }
        if (cached == 0 && count[s] == 0) { rc = OR_E_EMPTY; goto done; }
        if (count[s] > 0 && last[s] - first[s] + 1 != count[s]) { rc = OR_E_NONCONTIG; goto done; }
        seg_start[s] = cached ? -1 : first[s];
        seg_len[s] = cached ? cached : count[s];
    }
    for (int s = 0; s < S; ++s) {
        int p = seg_parent[s];
        if (p < -1 || p >= S || p == s) { rc = OR_E_PARENT; goto done; }
        if (p == -1) {
            if (seg_fork[s] != 0) { rc = OR_E_FORK; goto done; }
        } else {
            if (seg_fork[s] < 0 || seg_fork[s] > seg_len[p]) { rc = OR_E_FORK; goto done; }
            if (seg_cached_len[s] > 0 && seg_cached_len[p] == 0) { rc = OR_E_CACHED; goto done; }
            if (seg_cached_len[p] > 0 && seg_cached_len[s] == 0 && seg_fork[s] != seg_len[p]) {
                rc = OR_E_CACHED; goto done;
            }
        }
    }
    /* depth, root and first position by walking the parent chain */
    for (int s = 0; s < S; ++s) {
        int depth = 0, pos0 = 0, i = s;
        while (seg_parent[i] >= 0) {
            pos0 += seg_fork[i];
            i = seg_parent[i];
            if (++depth > S) { rc = OR_E_CYCLE; goto done; }
        }
        if (depth >= 4096) { rc = OR_E_CYCLE; goto done; }  /* chain arrays hold 4096 */
        seg_depth[s] = depth;
        seg_root[s] = i;
        seg_pos0[s] = pos0;
    }
    for (int t = 0; t < T; ++t) {
        int s = tok_seg[t];
        tok_pos[t] = seg_pos0[s] + (t - seg_start[s]) + MUT(8) * (seg_parent[s] >= 0);
    }
done:
    free(count); free(first); free(last);
    return rc;
}

/* ------------------------------------------------------------------------ */
/* Isolated path P(s): the list of rows (stream or history) it consists of   */
/* ------------------------------------------------------------------------ */

typedef struct {
    int L;          /* rows in the isolated sequence                       */
    int *src;       /* row r: >= 0 stream token index; < 0: -(1 + history row) */
} path_t;

/* Rows of P(s) truncated to the first `upto` rows of s itself. */
static void build_path(int s, int upto, const int *seg_parent, const int *seg_fork,
                       const int *seg_cached_len, const int *seg_start, const int *seg_pos0,
                       const int64_t *hist_off, path_t *P)
{
    int chain[4096];
    int n = 0;
    for (int i = s; i >= 0; i = seg_parent[i]) chain[n++] = i;
    P->L = seg_pos0[s] + upto;
    P->src = malloc((size_t)(P->L > 0 ? P->L : 1) * sizeof(int));
    int r = 0;
    if (MUT(2)) {
        for (int j = n - 1; j >= 1; --j)
            if (seg_cached_len[chain[j]] == 0) P->L -= seg_fork[chain[j - 1]];
    }
    for (int j = n - 1; j >= 0; --j) {
        int a = chain[j];
        int cnt = (j == 0) ? upto : seg_fork[chain[j - 1]];
        if (MUT(2) && j > 0 && seg_cached_len[a] == 0) cnt = 0;
        for (int i = 0; i < cnt; ++i) {
            if (seg_cached_len[a] > 0) P->src[r++] = -(int)(1 + hist_off[a] + i);
            else P->src[r++] = seg_start[a] + i;
        }
    }
}

static const double *row_ptr(const double *stream, const double *hist, int src, int H, int D, int h)
{
    if (src >= 0) return stream + ((size_t)src * H + h) * D;
    return hist + ((size_t)(-src - 1) * H + h) * D;
}

/* ------------------------------------------------------------------------ */
/* Attention                                                                 */
/* ------------------------------------------------------------------------ */

#define OR_RULE_CAUSAL 0   /* t_y <= t_x                                   */
#define OR_RULE_WINDOW 1   /* t_y <= t_x and t_x - t_y < window             */
#define OR_RULE_TWO_WAY 2  /* every row of the own segment; ancestors' prefixes */

/* softmax attention of row `r` of path P for q head h (kv head g) under the
   visibility rule; the row index along P is the standalone position. */
static void attend_row(const path_t *P, int r, int h, int g, int Hq, int Hkv, int d, double scale,
                       int rule, int window, const double *q, const double *k, const double *v,
                       const double *hk, const double *hv, double *o, double *sc)
{
    const double *qr = row_ptr(q, NULL, P->src[r], Hq, d, h);
    double m = -INFINITY;
    int first = 0, last = r - MUT(1);           /* keys 0..r are visible (t_y <= t_x) */
    if (rule == OR_RULE_WINDOW) {
        first = r - window + 1 - MUT(11);       /* t_x - t_y < window */
        if (first < 0) first = 0;
    } else if (rule == OR_RULE_TWO_WAY) {
        last = P->L - 1 - MUT(12);              /* the whole own segment (P ends with it) */
    }
    for (int j = 0; j < first; ++j) sc[j] = -INFINITY;
    for (int j = first; j <= last; ++j) {
        const double *kj = row_ptr(k, hk, P->src[j], Hkv, d, g);
        double s = 0.0;
        for (int x = 0; x < d; ++x) s += qr[x] * kj[x];
        s *= MUT(6) ? 1.0 : scale;
        sc[j] = s;
        if (s > m) m = s;
    }
    double den = 0.0;
    for (int x = 0; x < d; ++x) o[x] = 0.0;
    for (int j = first; j <= last; ++j) {
        double p = exp(sc[j] - m);
        den += p;
        const double *vj = row_ptr(v, hv, P->src[j], Hkv, d, g);
        for (int x = 0; x < d; ++x) o[x] += p * vj[x];
    }
    for (int x = 0; x < d; ++x) o[x] /= den;
}

int or_attention(int T, int S, const int *tok_seg, const int *seg_parent, const int *seg_fork,
                 const int *seg_cached_len, const int64_t *hist_off, int Hq, int Hkv, int d,
                 double scale, int rule, int window, const double *q, const double *k, const double *v,
                 const double *hk, const double *hv, int mode, const uint8_t *tok_sel,
                 const uint8_t *head_sel, double *out, int64_t *n_mismatch)
{
    if (Hq <= 0 || Hkv <= 0 || Hq % Hkv || d <= 0) return OR_E_ARG;
    if (rule < OR_RULE_CAUSAL || rule > OR_RULE_TWO_WAY || (rule == OR_RULE_WINDOW && window < 1)) return OR_E_ARG;
    /* under the two-way rule an ancestor's rows see their whole segment, which
       a leaf path holds only up to the fork: rows are evaluated over P(s) */
    if (rule == OR_RULE_TWO_WAY && mode == 0) return OR_E_ARG;
    int *seg_start = malloc(S * sizeof(int)), *seg_len = malloc(S * sizeof(int));
    int *seg_pos0 = malloc(S * sizeof(int)), *seg_depth = malloc(S * sizeof(int));
    int *seg_root = malloc(S * sizeof(int)), *tok_pos = malloc((T + 1) * sizeof(int));
    int rc = or_index(T, S, tok_seg, seg_parent, seg_fork, seg_cached_len, seg_start, seg_len,
                      seg_pos0, seg_depth, seg_root, tok_pos);
    int64_t mism = 0;
    if (rc) goto done;
    int G = Hq / Hkv;
    uint8_t *done_tok = calloc((size_t)T + 1, 1);

    /* which segments run their own path: mode 1 = every live segment;
       mode 0 = every live leaf, then any segment with uncovered tokens */
    int *has_child = calloc(S, sizeof(int));
    for (int s = 0; s < S; ++s) if (seg_parent[s] >= 0) has_child[seg_parent[s]] = 1;

    for (int pass = 0; pass < 2; ++pass) {
        for (int s = 0; s < S; ++s) {
            if (seg_cached_len[s] > 0) continue;
            if (mode == 0) {
                if (pass == 0 && has_child[s]) continue;
                if (pass == 1) {
                    int uncovered = 0;
                    for (int i = 0; i < seg_len[s]; ++i) uncovered |= !done_tok[seg_start[s] + i];
                    if (!uncovered) continue;
                }
            } else if (pass == 1) {
                continue;
            }
            path_t P;
            build_path(s, seg_len[s], seg_parent, seg_fork, seg_cached_len, seg_start, seg_pos0,
                       hist_off, &P);
            /* rows to compute: mode 0 = every live row of the path; mode 1 = s's rows */
            int r0 = (mode == 0) ? 0 : seg_pos0[s];
            int nrows = P.L - r0;
            int64_t local_mism = 0;
#pragma omp parallel for schedule(dynamic, 1) collapse(2) reduction(+ : local_mism)
            for (int h = 0; h < Hq; ++h) {
                for (int rr = 0; rr < nrows; ++rr) {
                    int r = r0 + rr;
                    int src = P.src[r];
                    if (src < 0) continue;                       /* history row: no output */
                    if (head_sel && !head_sel[h]) continue;
                    if (mode == 1 && tok_sel && !tok_sel[src]) continue;
                    double *sc = malloc((size_t)P.L * sizeof(double));   /* keys 0 .. P.L-1 at most */
                    double *o = malloc((size_t)d * sizeof(double));
                    int g = MUT(3) ? h % Hkv : h / G;       /* contiguous GQA groups */
                    attend_row(&P, r, h, g, Hq, Hkv, d, scale, rule, window, q, k, v, hk, hv, o, sc);
                    double *dst = out + ((size_t)src * Hq + h) * d;
                    if (done_tok[src]) {
                        if (memcmp(dst, o, (size_t)d * sizeof(double)) != 0) local_mism++;
                    } else {
                        memcpy(dst, o, (size_t)d * sizeof(double));
                    }
                    free(sc); free(o);
                }
            }
            mism += local_mism;
            for (int r = r0; r < P.L; ++r)
                if (P.src[r] >= 0) done_tok[P.src[r]] = 1;
            free(P.src);
        }
    }
    free(done_tok); free(has_child);
done:
    if (n_mismatch) *n_mismatch = mism;
    free(seg_start); free(seg_len); free(seg_pos0); free(seg_depth); free(seg_root); free(tok_pos);
    return rc;
}

/* ------------------------------------------------------------------------ */
/* Gated DeltaNet                                                            */
/* ------------------------------------------------------------------------ */

/* One step of Eq. 4 on the dv x dk state S (row-major, S[i*dk + j]):
   u = S k;  S <- a (S - b u k^T) + b v k^T;  o = S q.                         */
static void gdn_step(double *S, int dk, int dv, const double *q, const double *k,
                     const double *v, double a, double b, double *o)
{
    if (MUT(5)) {               /* planted: state used transposed (needs dv == dk) */
        double *u = calloc((size_t)dk, sizeof(double));
        for (int j = 0; j < dk; ++j)
            for (int i = 0; i < dv; ++i) u[j] += S[(size_t)i * dk + j] * k[i];
        for (int i = 0; i < dv; ++i)
            for (int j = 0; j < dk; ++j)
                S[(size_t)i * dk + j] = a * (S[(size_t)i * dk + j] - b * k[i] * u[j]) + b * v[i] * k[j];
        for (int i = 0; i < dv; ++i) {
            double acc = 0.0;
            for (int j = 0; j < dk; ++j) acc += S[(size_t)i * dk + j] * q[j];
            o[i] = acc;
        }
        free(u);
        return;
    }
    for (int i = 0; i < dv; ++i) {
        double *Si = S + (size_t)i * dk;
        double u = 0.0;
        for (int j = 0; j < dk; ++j) u += Si[j] * k[j];
        double prev = 0.0;
        if (MUT(7)) for (int j = 0; j < dk; ++j) prev += Si[j] * q[j];
        for (int j = 0; j < dk; ++j) {
            if (MUT(4)) Si[j] = a * Si[j] - b * u * k[j] + b * v[i] * k[j];
            else Si[j] = a * (Si[j] - b * u * k[j]) + b * v[i] * k[j];
        }
        double acc = 0.0;
        for (int j = 0; j < dk; ++j) acc += Si[j] * q[j];
        o[i] = MUT(7) ? prev : acc;
    }
}

int or_gdn(int T, int S, const int *tok_seg, const int *seg_parent, const int *seg_fork,
           const int *seg_cached_len, int Hk, int Hv, int dk, int dv, const double *q,
           const double *k, const double *v, const double *a, const double *b,
           const double *state_in, const int *seg_state_in, int mode, const uint8_t *head_sel,
           double *out, const int *seg_state_out, double *state_out, int64_t *n_mismatch)
{
    if (Hk <= 0 || Hv <= 0 || Hv % Hk || dk <= 0 || dv <= 0) return OR_E_ARG;
    int *seg_start = malloc(S * sizeof(int)), *seg_len = malloc(S * sizeof(int));
    int *seg_pos0 = malloc(S * sizeof(int)), *seg_depth = malloc(S * sizeof(int));
    int *seg_root = malloc(S * sizeof(int)), *tok_pos = malloc((T + 1) * sizeof(int));
    int rc = or_index(T, S, tok_seg, seg_parent, seg_fork, seg_cached_len, seg_start, seg_len,
                      seg_pos0, seg_depth, seg_root, tok_pos);
    int64_t mism = 0;
    if (rc) goto done;
    /* a cached segment that a live child reads must bring a state */
    for (int s = 0; s < S; ++s) {
        int p = seg_parent[s];
        if (seg_cached_len[s] == 0 && p >= 0 && seg_cached_len[p] > 0 && seg_state_in[p] < 0) {
            rc = OR_E_CACHED; goto done;
        }
    }
    const int R = Hv / Hk;
    const size_t SZ = (size_t)dv * dk;
    int *has_child = calloc(S, sizeof(int));
    for (int s = 0; s < S; ++s) if (seg_parent[s] >= 0) has_child[seg_parent[s]] = 1;
    int maxdepth = 0;
    for (int s = 0; s < S; ++s) if (seg_depth[s] > maxdepth) maxdepth = seg_depth[s];
    /* live children of every segment (CSR, in segment-index order) */
    int *kid_off = calloc((size_t)S + 1, sizeof(int));
    int *kids = malloc((size_t)S * sizeof(int));
    for (int s = 0; s < S; ++s)
        if (seg_parent[s] >= 0 && seg_cached_len[s] == 0) kid_off[seg_parent[s] + 1]++;
    for (int s = 0; s < S; ++s) kid_off[s + 1] += kid_off[s];
    {
        int *fill = calloc((size_t)S, sizeof(int));
        for (int s = 0; s < S; ++s) {
            int p = seg_parent[s];
            if (p >= 0 && seg_cached_len[s] == 0) kids[kid_off[p] + fill[p]++] = s;
        }
        free(fill);
    }

#pragma omp parallel for schedule(dynamic, 1) reduction(+ : mism)
    for (int h = 0; h < Hv; ++h) {
        if (head_sel && !head_sel[h]) continue;
        int g = h / R;
        double *o = malloc((size_t)dv * sizeof(double));
        uint8_t *done_tok = calloc((size_t)T + 1, 1);
        uint8_t *done_state = calloc((size_t)S, 1);
        if (mode == 0) {
            /* literal: each leaf path from its root state, then uncovered tails */
            for (int pass = 0; pass < 2; ++pass) {
                for (int s = 0; s < S; ++s) {
                    if (seg_cached_len[s] > 0) continue;
                    if (pass == 0 && has_child[s]) continue;
                    if (pass == 1) {
                        int unc = 0;
                        for (int i = 0; i < seg_len[s]; ++i) unc |= !done_tok[seg_start[s] + i];
                        if (!unc && (seg_state_out[s] < 0 || done_state[s])) continue;
                    }
                    int chain[4096], n = 0;
                    for (int i = s; i >= 0; i = seg_parent[i]) chain[n++] = i;
                    double *St = calloc(SZ, sizeof(double));
                    int j = n - 1;
                    /* skip the cached prefix of the chain; start from its saved state */
                    while (j >= 0 && seg_cached_len[chain[j]] > 0) --j;
                    if (j < n - 1) {
                        int c = chain[j + 1];
                        memcpy(St, state_in + ((size_t)seg_state_in[c] * Hv + h) * SZ, SZ * sizeof(double));
                    }
                    for (; j >= 0; --j) {
                        int sg = chain[j];
                        int cnt = (j == 0) ? seg_len[sg] : seg_fork[chain[j - 1]];
                        for (int i = 0; i < cnt; ++i) {
                            int t = seg_start[sg] + i;
                            gdn_step(St, dk, dv, q + ((size_t)t * Hk + g) * dk,
                                     k + ((size_t)t * Hk + g) * dk, v + ((size_t)t * Hv + h) * dv,
                                     a[(size_t)t * Hv + h], b[(size_t)t * Hv + h], o);
                            double *dst = out + ((size_t)t * Hv + h) * dv;
                            if (done_tok[t]) {
                                if (memcmp(dst, o, (size_t)dv * sizeof(double))) mism++;
                            } else {
                                memcpy(dst, o, (size_t)dv * sizeof(double));
                                done_tok[t] = 1;
                            }
                        }
                        if (cnt == seg_len[sg] && seg_state_out[sg] >= 0) {
                            double *dst = state_out + ((size_t)seg_state_out[sg] * Hv + h) * SZ;
                            if (done_state[sg]) {
                                if (memcmp(dst, St, SZ * sizeof(double))) mism++;
                            } else {
                                memcpy(dst, St, SZ * sizeof(double));
                                done_state[sg] = 1;
                            }
                        }
                    }
                    free(St);
                }
            }
        } else {
            /* tree: each live segment once, from its parent's state at the fork */
            double **snap = calloc(S, sizeof(double *));  /* state a child starts from */
            for (int depth = 0; depth <= maxdepth; ++depth) {
                for (int s = 0; s < S; ++s) {
                    if (seg_depth[s] != depth || seg_cached_len[s] > 0) continue;
                    double *St = calloc(SZ, sizeof(double));
                    int p = seg_parent[s];
                    if (p >= 0 && seg_cached_len[p] > 0)
                        memcpy(St, state_in + ((size_t)seg_state_in[p] * Hv + h) * SZ, SZ * sizeof(double));
                    else if (p >= 0) {
                        memcpy(St, snap[s], SZ * sizeof(double));
                        free(snap[s]); snap[s] = NULL;
                    }
                    for (int i = 0; i <= seg_len[s]; ++i) {
                        /* children forking after i tokens start from this state */
                        for (int x = kid_off[s]; x < kid_off[s + 1]; ++x) {
                            int c = kids[x];
                            if (seg_fork[c] == i) {
                                snap[c] = malloc(SZ * sizeof(double));
                                memcpy(snap[c], St, SZ * sizeof(double));
                            }
                        }
                        if (i == seg_len[s]) break;
                        int t = seg_start[s] + i;
                        gdn_step(St, dk, dv, q + ((size_t)t * Hk + g) * dk,
                                 k + ((size_t)t * Hk + g) * dk, v + ((size_t)t * Hv + h) * dv,
                                 a[(size_t)t * Hv + h], b[(size_t)t * Hv + h], o);
                        memcpy(out + ((size_t)t * Hv + h) * dv, o, (size_t)dv * sizeof(double));
                    }
                    if (seg_state_out[s] >= 0)
                        memcpy(state_out + ((size_t)seg_state_out[s] * Hv + h) * SZ, St,
                               SZ * sizeof(double));
                    free(St);
                }
            }
            for (int s = 0; s < S; ++s) free(snap[s]);
            free(snap);
        }
        free(o); free(done_tok); free(done_state);
    }
    free(has_child); free(kid_off); free(kids);
done:
    if (n_mismatch) *n_mismatch = mism;
    free(seg_start); free(seg_len); free(seg_pos0); free(seg_depth); free(seg_root); free(tok_pos);
    return rc;
}

/* ------------------------------------------------------------------------ */
/* Short causal convolution                                                  */
/* ------------------------------------------------------------------------ */

/* x [T, C] stream rows and hx [Nh, C] history rows (cached segment s owns
 * history rows hist_off[s] ..); w [C, W] with w[c][0] on the token itself and
 * w[c][i] on its i-th predecessor along P(s).  y [T, C].  For every segment
 * with a state_out slot, window_out[slot] [W-1, C] holds the inputs of the
 * last W-1 rows of P(s) (oldest first; zero where P(s) is shorter), i.e. the
 * window a continuation of s reads. */
int or_conv(int T, int S, const int *tok_seg, const int *seg_parent, const int *seg_fork,
            const int *seg_cached_len, const int64_t *hist_off, int C, int W, const double *w,
            const double *x, const double *hx, const int *seg_state_out, int n_state_out, double *y,
            double *window_out)
{
    if (C <= 0 || W <= 0) return OR_E_ARG;
    int *seg_start = malloc(S * sizeof(int)), *seg_len = malloc(S * sizeof(int));
    int *seg_pos0 = malloc(S * sizeof(int)), *seg_depth = malloc(S * sizeof(int));
    int *seg_root = malloc(S * sizeof(int)), *tok_pos = malloc((T + 1) * sizeof(int));
    int rc = or_index(T, S, tok_seg, seg_parent, seg_fork, seg_cached_len, seg_start, seg_len,
                      seg_pos0, seg_depth, seg_root, tok_pos);
    if (rc) goto done;
    for (int s = 0; s < S; ++s) {
        if (seg_cached_len[s] > 0) continue;
        path_t P;
        build_path(s, seg_len[s], seg_parent, seg_fork, seg_cached_len, seg_start, seg_pos0, hist_off, &P);
        /* planted: rows before the segment's own first row are not read */
        const int first = MUT(9) ? seg_pos0[s] : 0;
#pragma omp parallel for schedule(static)
        for (int r = seg_pos0[s]; r < P.L; ++r) {
            const int src = P.src[r];
            for (int c = 0; c < C; ++c) {
                double acc = 0.0;
                for (int i = 0; i < W; ++i) {
                    /* planted: predecessors taken one row too far back */
                    const int rr = r - i - (MUT(10) && i > 0);
                    if (rr < first) continue;
                    acc += w[(size_t)c * W + i] * row_ptr(x, hx, P.src[rr], 1, C, 0)[c];
                }
                y[(size_t)src * C + c] = acc;
            }
        }
        const int slot = seg_state_out ? seg_state_out[s] : -1;
        if (slot >= 0 && slot < n_state_out && W > 1) {
            for (int k = 0; k < W - 1; ++k) {
                const int rr = P.L - (W - 1) + k;
                for (int c = 0; c < C; ++c)
                    window_out[((size_t)slot * (W - 1) + k) * C + c] =
                        rr >= 0 ? row_ptr(x, hx, P.src[rr], 1, C, 0)[c] : 0.0;
            }
        }
        free(P.src);
    }
done:
    free(seg_start); free(seg_len); free(seg_pos0); free(seg_depth); free(seg_root); free(tok_pos);
    return rc;
}

/* ------------------------------------------------------------------------ */
/* Projection                                                                */
/* ------------------------------------------------------------------------ */

/* y [M, N] = rows of x [Mx, K] times w [N, K] transposed (w row n = output
 * feature n, as a linear layer stores it):
 *     y[m][n] = sum_{k < K} x[r][k] * w[n][k],   r = rows ? rows[m] : m,
 * summed in fp64, k ascending.  An entry rows[m] < 0 selects no row: y's row
 * m is left as it was.  An entry >= Mx is an error. */
int or_proj(int M, int Mx, int K, int N, const double *x, const int *rows, const double *w, double *y)
{
    if (M < 0 || Mx < 0 || K <= 0 || N <= 0 || !x || !w || !y) return OR_E_ARG;
    if (!rows && M > Mx) return OR_E_ARG;
    for (int m = 0; m < M; ++m)
        if (rows && rows[m] >= Mx) return OR_E_ARG;
#pragma omp parallel for schedule(static)
    for (int m = 0; m < M; ++m) {
        /* planted: the index buffer ignored */
        const int r = (rows && !MUT(14)) ? rows[m] : m;
        if (r < 0 || r >= Mx) continue;
        const double *xr = x + (size_t)r * K;
        for (int n = 0; n < N; ++n) {
            const double *wn = w + (size_t)n * K;
            double acc = 0.0;
            /* planted: the last term of the sum dropped */
            for (int k = 0; k < K - MUT(13); ++k) acc += xr[k] * wn[k];
            y[(size_t)m * N + n] = acc;
        }
    }
    return OR_OK;
}
