/*
 * mc_oracle.c -- fp64 CPU oracle for Memory Caching (MC) over a linear-attention memory.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, loads or calls this
 * file; only the test-suite, the smoke check and the benchmark's CPU-baseline leg do.
 * It shares no code, header or constant with the HIP path.
 *
 * Sources (the pages this follows; section / equation of each page):
 *   [MC]   "Memory Caching: RNNs with growing memory" (Behrouz et al.), zh-TW and ja renderings:
 *          §2 linear attention Eq. (2); §3 segmentation + per-segment recurrence Eq. (4a)/(4b)
 *          and aggregation Eq. (5); §3.1 residual memory Eq. (6)/(7); gated residual memory
 *          Eq. (8)/(9) with the context gate Eq. (10) normalised by a softmax.
 *   [EXP]  "给 RNN 装上“会增长的记忆”：解读 Google 的 Memory Caching" (gitcode explainer):
 *          §3.3 Memory Soup, §3.4 Sparse Selective Caching (router score, Top-k, online
 *          memory always kept).
 *   [MC-A] the appendix of [MC] on the MC variants, its paragraph on memory caching applied
 *          after pre-training: decoding reads an average of the cached memories, with no
 *          learned weights.
 *
 * Readings of points the pages leave open:
 *   - the memory is the unnormalised linear-attention state ([MC] §2, the Miras remark that
 *     the inner-product objective gives *unnormalised* linear attention): no 1/Z anywhere;
 *   - M = sum_r v_r phi(k_r)^T is d_v x d_k and is read as y = M phi(q) ([MC] Eq. 2, 4b);
 *   - the memory is updated with token t before token t reads it ([MC] §3: the last state
 *     is cached "after updating the memory"; Eq. 8 precedes Eq. 9);
 *   - MeanPooling(S^(i)) is the mean of the layer input x over segment i; the online
 *     segment uses the causal prefix mean over its tokens seen so far;
 *   - gamma_t = softmax over i = 0..s of <u_t, MeanPooling(S^(i))>, no temperature;
 *   - SSC: candidates are the completed segments i < s, the online segment is always kept,
 *     Top-k takes the larger score first and the lower index on ties, the softmax runs over
 *     the selected set plus the online segment;
 *   - segments have a constant length C; a trailing partial segment is the online segment.
 *
 * Conventions: every array is dense row-major fp64; token index t is 0-based; s = t / C is
 * the segment of t, j = t % C its position inside the segment.
 *   Q, K [B,H,L,dk]; V [B,H,L,dv]; U [B,H,L,dg]; X [B,xh,L,dg] with xh = 1 (shared by the
 *   heads) or xh = H (head h reads X[:,h]).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { MCO_GRM = 0, MCO_SSC = 1, MCO_RESIDUAL = 2, MCO_SOUP = 3, MCO_AVERAGE = 4 };
enum { MCO_OK = 0, MCO_EARG = 1, MCO_ENOMEM = 2 };

/* phi of [MC] Eq. (2): identity, or elu(z)+1 = z+1 for z>0, e^z otherwise. */
static double mco_phi(double z, int phi) {
    if (phi == 0) return z;
    return z > 0.0 ? z + 1.0 : exp(z);
}

/* Top-k of score[0..n-1]: repeatedly take the largest remaining score, scanning indices
 * upwards and replacing only on a strictly larger value, so equal scores keep the lower
 * index.  The chosen indices are returned in ascending order; fewer than k candidates
 * means all of them are chosen.  Returns the number chosen. */
static int mco_topk(const double* score, int n, int k, int* chosen) {
    int m = n < k ? n : k;
    char* taken = (char*)calloc((size_t)(n > 0 ? n : 1), 1);
    for (int c = 0; c < m; ++c) {
        int best = -1;
        for (int i = 0; i < n; ++i) {
            if (taken[i]) continue;
            if (best < 0 || score[i] > score[best]) best = i;
        }
        taken[best] = 1;
    }
    int w = 0;
    for (int i = 0; i < n; ++i)
        if (taken[i]) chosen[w++] = i;
    free(taken);
    return w;
}

/*
 * Prefill over a whole sequence, per (b, h), token by token ([MC] §3, Eq. 4b then Eq. 9).
 *
 * dims = {B, H, L, dk, dv, dg, C, xh, phi}.  mode: MCO_GRM (Eq. 9 with the Eq. 10 softmax
 * gate), MCO_SSC ([EXP] §3.4 with top_k), MCO_RESIDUAL (Eq. 7, every weight 1) or MCO_SOUP
 * ([EXP] §3.3: the gamma-weighted average of the memory matrices is formed first and then
 * read once).
 *
 * SWLA memory (alpha != NULL; [MC] §3.1, the sliding-window linear attention paragraph,
 * Eq. 26 with window c = 2, i.e. Eq. 28): alpha, beta, lam are [B,H,L] per-token scalars and
 * the update is M_t = alpha_t M_{t-1} + beta_t v_{t-1} phi(k_{t-1})^T + lam_t v_t phi(k_t)^T.
 * The window stays inside the segment: at a segment's first token there is no previous
 * token to write (its memory starts from zero, Eq. 4b).  The read (Eq. 29) is unchanged.
 * With alpha == NULL the update is the linear-attention one (Eq. 2).
 *
 * Segments: constant length C, or (off != NULL) the n_seg segments [off[i], off[i+1]) with
 * off[0] = 0 < off[1] < ... < off[n_seg] = L ([MC] Eq. 4b lets the segment lengths L^(s)
 * differ); C is then not read.
 * rows: ascending token indices to evaluate (NULL = all L tokens); Y [B,H,n_rows,dv].
 * Optional outputs (NULL to skip):
 *   M_out [B,H,NS,dv,dk]  state of segment i after its last token (NS = ceil(L/C) or n_seg;
 *                         a trailing partial segment stores its state after token L-1)
 *   P_out [B,xh,NS,dg]    mean of x over segment i (partial segment: over its tokens)
 *   O_on  [B,H,L,dv]      ungated online read M_t^(s) phi(q_t)  (only with rows == NULL)
 *   gamma [B,H,n_rows,NS] weights of segments 0..s (0 for segments not read)
 *   idx   [B,H,n_rows,top_k] SSC selection, ascending, -1 padded
 */
int mco_prefill(const int32_t* dims, int mode, int top_k,
                const double* Q, const double* K, const double* V, const double* U,
                const double* X, const int32_t* rows, int64_t n_rows,
                double* Y, double* M_out, double* P_out, double* O_on, double* gamma,
                int32_t* idx, int n_threads, const int32_t* off, int32_t n_seg,
                const double* alpha, const double* beta, const double* lam) {
    const int B = dims[0], H = dims[1], L = dims[2], dk = dims[3], dv = dims[4], dg = dims[5];
    const int C = dims[6], xh = dims[7], phi = dims[8];
    if (B <= 0 || H <= 0 || L <= 0 || dk <= 0 || dv <= 0 || dg <= 0) return MCO_EARG;
    if (off == NULL && C <= 0) return MCO_EARG;
    if (off != NULL) {
        if (n_seg <= 0 || off[0] != 0 || off[n_seg] != L) return MCO_EARG;
        for (int i = 0; i < n_seg; ++i)
            if (off[i + 1] <= off[i]) return MCO_EARG;
    }
    if (!(xh == 1 || xh == H)) return MCO_EARG;
    if (mode < 0 || mode > 3) return MCO_EARG;
    if (mode == MCO_SSC && top_k <= 0) return MCO_EARG;
    if (rows != NULL && O_on != NULL) return MCO_EARG;
    if (alpha != NULL && (beta == NULL || lam == NULL)) return MCO_EARG;
    const int NS = off ? n_seg : (L + C - 1) / C;
    const int64_t nr = rows ? n_rows : (int64_t)L;
    if (rows)
        for (int64_t a = 0; a < nr; ++a)
            if (rows[a] < 0 || rows[a] >= L || (a > 0 && rows[a] <= rows[a - 1])) return MCO_EARG;
#ifdef _OPENMP
    if (n_threads > 0) omp_set_num_threads(n_threads);
#else
    (void)n_threads;
#endif
    int err = MCO_OK;

#pragma omp parallel for schedule(dynamic, 1)
    for (int bh = 0; bh < B * H; ++bh) {
        const int b = bh / H, h = bh % H;
        const int hx = (xh == 1) ? 0 : h;
        const double* q = Q + (size_t)bh * L * dk;
        const double* k = K + (size_t)bh * L * dk;
        const double* v = V + (size_t)bh * L * dv;
        const double* u = U + (size_t)bh * L * dg;
        const double* x = X + ((size_t)b * xh + hx) * L * dg;

        double* Mc = (double*)calloc((size_t)NS * dv * dk, sizeof(double)); /* cached states */
        double* Pc = (double*)calloc((size_t)NS * dg, sizeof(double));      /* segment means */
        double* Mon = (double*)calloc((size_t)dv * dk, sizeof(double));     /* online state */
        double* xs = (double*)calloc((size_t)dg, sizeof(double));           /* online x sum */
        double* kh = (double*)malloc(sizeof(double) * dk);
        double* kp = (double*)malloc(sizeof(double) * dk);
        double* qh = (double*)malloc(sizeof(double) * dk);
        double* pt = (double*)malloc(sizeof(double) * dg);
        double* a = (double*)malloc(sizeof(double) * (NS + 1));
        double* g = (double*)malloc(sizeof(double) * (NS + 1));
        int* sel = (int*)malloc(sizeof(int) * (NS + 1));
        double* soup = (double*)malloc(sizeof(double) * dv * dk);
        double* tmp = (double*)malloc(sizeof(double) * dv);
        if (!Mc || !Pc || !Mon || !xs || !kh || !kp || !qh || !pt || !a || !g || !sel || !soup || !tmp) {
#pragma omp atomic write
            err = MCO_ENOMEM;
        } else {
            int64_t next = 0; /* position in rows */
            int s = 0;        /* segment of t */
            for (int t = 0; t < L; ++t) {
                if (off) {
                    while (t >= off[s + 1]) ++s;
                } else {
                    s = t / C;
                }
                const int s0 = off ? off[s] : s * C;                    /* its first token */
                const int s1 = off ? off[s + 1] : (s + 1 < NS ? (s + 1) * C : L); /* one past */
                const int j = t - s0;
                if (j == 0) { /* a new segment starts from the zero memory ([MC] Eq. 4b) */
                    memset(Mon, 0, sizeof(double) * dv * dk);
                    memset(xs, 0, sizeof(double) * dg);
                }
                for (int r = 0; r < dk; ++r) kh[r] = mco_phi(k[(size_t)t * dk + r], phi);
                if (alpha) {
                    /* SWLA, window 2 ([MC] Eq. 28): decay the memory, then write the previous
                     * token of this segment with beta_t and this token with lam_t */
                    const size_t gi = (size_t)bh * L + t;
                    for (size_t e = 0; e < (size_t)dv * dk; ++e) Mon[e] *= alpha[gi];
                    if (j > 0) {
                        for (int r = 0; r < dk; ++r) kp[r] = mco_phi(k[(size_t)(t - 1) * dk + r], phi);
                        for (int c = 0; c < dv; ++c) {
                            const double vc = beta[gi] * v[(size_t)(t - 1) * dv + c];
                            for (int r = 0; r < dk; ++r) Mon[(size_t)c * dk + r] += vc * kp[r];
                        }
                    }
                    for (int c = 0; c < dv; ++c) {
                        const double vc = lam[gi] * v[(size_t)t * dv + c];
                        for (int r = 0; r < dk; ++r) Mon[(size_t)c * dk + r] += vc * kh[r];
                    }
                } else {
                    /* memory update M_t = M_{t-1} + v_t phi(k_t)^T  ([MC] Eq. 2, Eq. 4b) */
                    for (int c = 0; c < dv; ++c) {
                        const double vc = v[(size_t)t * dv + c];
                        for (int r = 0; r < dk; ++r) Mon[(size_t)c * dk + r] += vc * kh[r];
                    }
                }
                for (int e = 0; e < dg; ++e) xs[e] += x[(size_t)t * dg + e];

                const int want_all = (rows == NULL);
                const int want = want_all || (next < nr && rows[next] == t);
                if (want) {
                    const int64_t row = want_all ? t : next;
                    for (int r = 0; r < dk; ++r) qh[r] = mco_phi(q[(size_t)t * dk + r], phi);
                    /* context gate logits ([MC] Eq. 10): <u_t, MeanPooling(S^(i))> */
                    for (int i = 0; i < s; ++i) {
                        double acc = 0.0;
                        for (int e = 0; e < dg; ++e) acc += u[(size_t)t * dg + e] * Pc[(size_t)i * dg + e];
                        a[i] = acc;
                    }
                    for (int e = 0; e < dg; ++e) pt[e] = xs[e] / (double)(j + 1);
                    {
                        double acc = 0.0;
                        for (int e = 0; e < dg; ++e) acc += u[(size_t)t * dg + e] * pt[e];
                        a[s] = acc;
                    }
                    /* which segments are read, and with what weight */
                    int nsel = 0;
                    if (mode == MCO_SSC) {
                        nsel = mco_topk(a, s, top_k, sel);
                    } else {
                        for (int i = 0; i < s; ++i) sel[i] = i;
                        nsel = s;
                    }
                    sel[nsel] = s; /* the online memory is always read */
                    if (mode == MCO_RESIDUAL) {
                        for (int c = 0; c <= nsel; ++c) g[c] = 1.0;
                    } else {
                        double mx = a[sel[0]];
                        for (int c = 1; c <= nsel; ++c) mx = fmax(mx, a[sel[c]]);
                        double z = 0.0;
                        for (int c = 0; c <= nsel; ++c) { g[c] = exp(a[sel[c]] - mx); z += g[c]; }
                        for (int c = 0; c <= nsel; ++c) g[c] /= z;
                    }
                    double* yr = Y + ((size_t)bh * nr + row) * dv;
                    if (mode == MCO_SOUP) {
                        /* soup: one matrix sum_i gamma_i M^(i), then one read */
                        for (size_t e = 0; e < (size_t)dv * dk; ++e) soup[e] = g[nsel] * Mon[e];
                        for (int c = 0; c < nsel; ++c) {
                            const double* Mi = Mc + (size_t)sel[c] * dv * dk;
                            for (size_t e = 0; e < (size_t)dv * dk; ++e) soup[e] += g[c] * Mi[e];
                        }
                        for (int c = 0; c < dv; ++c) {
                            double acc = 0.0;
                            for (int r = 0; r < dk; ++r) acc += soup[(size_t)c * dk + r] * qh[r];
                            yr[c] = acc;
                        }
                    } else {
                        /* Eq. 9: gamma^(s) M_t^(s) q_t + sum_i gamma^(i) M^(i) q_t */
                        for (int c = 0; c < dv; ++c) {
                            double acc = 0.0;
                            for (int r = 0; r < dk; ++r) acc += Mon[(size_t)c * dk + r] * qh[r];
                            yr[c] = g[nsel] * acc;
                        }
                        for (int cc = 0; cc < nsel; ++cc) {
                            const double* Mi = Mc + (size_t)sel[cc] * dv * dk;
                            for (int c = 0; c < dv; ++c) {
                                double acc = 0.0;
                                for (int r = 0; r < dk; ++r) acc += Mi[(size_t)c * dk + r] * qh[r];
                                tmp[c] = acc;
                            }
                            for (int c = 0; c < dv; ++c) yr[c] += g[cc] * tmp[c];
                        }
                    }
                    if (gamma) {
                        double* gr = gamma + ((size_t)bh * nr + row) * NS;
                        for (int i = 0; i < NS; ++i) gr[i] = 0.0;
                        for (int c = 0; c <= nsel; ++c) gr[sel[c]] = g[c];
                    }
                    if (idx && mode == MCO_SSC) {
                        int32_t* ir = idx + ((size_t)bh * nr + row) * top_k;
                        for (int c = 0; c < top_k; ++c) ir[c] = c < nsel ? sel[c] : -1;
                    }
                    if (O_on) {
                        double* orow = O_on + ((size_t)bh * L + t) * dv;
                        for (int c = 0; c < dv; ++c) {
                            double acc = 0.0;
                            for (int r = 0; r < dk; ++r) acc += Mon[(size_t)c * dk + r] * qh[r];
                            orow[c] = acc;
                        }
                    }
                    if (!want_all) ++next;
                }
                /* segment end (or end of input): cache the last state and the segment mean */
                if (t == s1 - 1 || t == L - 1) {
                    memcpy(Mc + (size_t)s * dv * dk, Mon, sizeof(double) * dv * dk);
                    for (int e = 0; e < dg; ++e) Pc[(size_t)s * dg + e] = xs[e] / (double)(j + 1);
                }
            }
            if (M_out) memcpy(M_out + (size_t)bh * NS * dv * dk, Mc, sizeof(double) * NS * dv * dk);
            if (P_out && (xh == H || h == 0))
                memcpy(P_out + ((size_t)b * xh + hx) * NS * dg, Pc, sizeof(double) * NS * dg);
        }
        free(Mc); free(Pc); free(Mon); free(xs); free(kh); free(kp); free(qh); free(pt);
        free(a); free(g); free(sel); free(soup); free(tmp);
    }
    return err;
}

/*
 * One decode step ([MC] §3 applied to one new token per sequence): for each (b, h) the
 * online memory is updated with the new token, the gate runs over the n cached segments
 * plus the online segment, and y reads all of them (Eq. 9).  When the online segment then
 * holds C tokens, its state and mean are appended to the cache and the online memory
 * restarts from zero (the segment boundary of Eq. 4b).
 *
 * dims = {B, H, dk, dv, dg, C, xh, phi}.  q,k [B,H,dk]; v [B,H,dv]; u [B,H,dg]; x [B,xh,dg].
 * In/out: M_on [B,H,dv,dk], xsum [B,xh,dg], *count (tokens already in the online segment,
 * 0..C-1 on entry), M_cache [B,H,n_cap,dv,dk], P_cache [B,xh,n_cap,dg], *n_cached.
 * Out: y [B,H,dv]; gamma (nullable) [B,H,n_cap+1] (entry n_cap is the online weight).
 * mode: MCO_GRM, MCO_RESIDUAL or MCO_AVERAGE ([MC-A]: every one of the n + 1 memories
 * weighs 1 / (n + 1); u is not read).
 */
int mco_decode_step(const int32_t* dims, int mode, const double* q, const double* k,
                    const double* v, const double* u, const double* x, double* M_on,
                    double* xsum, int32_t* count, double* M_cache, double* P_cache,
                    int32_t* n_cached, int32_t n_cap, double* y, double* gamma) {
    const int B = dims[0], H = dims[1], dk = dims[2], dv = dims[3], dg = dims[4];
    const int C = dims[5], xh = dims[6], phi = dims[7];
    if (B <= 0 || H <= 0 || dk <= 0 || dv <= 0 || dg <= 0 || C <= 0) return MCO_EARG;
    if (!(xh == 1 || xh == H)) return MCO_EARG;
    if (!(mode == MCO_GRM || mode == MCO_RESIDUAL || mode == MCO_AVERAGE)) return MCO_EARG;
    const int cnt = *count, n = *n_cached;
    if (cnt < 0 || cnt >= C || n < 0 || n > n_cap) return MCO_EARG;
    const int emit = (cnt + 1 == C);
    if (emit && n == n_cap) return MCO_EARG;

    /* new x sums: every head of a sequence sees the same updated sum */
    double* xs_new = (double*)malloc(sizeof(double) * (size_t)B * xh * dg);
    if (!xs_new) return MCO_ENOMEM;
    for (size_t e = 0; e < (size_t)B * xh * dg; ++e) xs_new[e] = xsum[e] + x[e];

    for (int bh = 0; bh < B * H; ++bh) {
        const int b = bh / H, h = bh % H;
        const int hx = (xh == 1) ? 0 : h;
        double* Mon = M_on + (size_t)bh * dv * dk;
        const double* xs = xs_new + ((size_t)b * xh + hx) * dg;
        const double* uu = u + (size_t)bh * dg;
        double kh[1024], qh[1024];
        if (dk > 1024) { free(xs_new); return MCO_EARG; }
        for (int r = 0; r < dk; ++r) {
            kh[r] = mco_phi(k[(size_t)bh * dk + r], phi);
            qh[r] = mco_phi(q[(size_t)bh * dk + r], phi);
        }
        for (int c = 0; c < dv; ++c)
            for (int r = 0; r < dk; ++r) Mon[(size_t)c * dk + r] += v[(size_t)bh * dv + c] * kh[r];
        double* a = (double*)malloc(sizeof(double) * (n + 1));
        double* g = (double*)malloc(sizeof(double) * (n + 1));
        for (int i = 0; i < n; ++i) {
            const double* Pi = P_cache + (((size_t)b * xh + hx) * n_cap + i) * dg;
            double acc = 0.0;
            for (int e = 0; e < dg; ++e) acc += uu[e] * Pi[e];
            a[i] = acc;
        }
        {
            double acc = 0.0;
            for (int e = 0; e < dg; ++e) acc += uu[e] * (xs[e] / (double)(cnt + 1));
            a[n] = acc;
        }
        if (mode == MCO_RESIDUAL) {
            for (int i = 0; i <= n; ++i) g[i] = 1.0;
        } else if (mode == MCO_AVERAGE) {
            /* [MC-A]: the plain mean over the n cached memories and the online one */
            for (int i = 0; i <= n; ++i) g[i] = 1.0 / (double)(n + 1);
        } else {
            double mx = a[0];
            for (int i = 1; i <= n; ++i) mx = fmax(mx, a[i]);
            double z = 0.0;
            for (int i = 0; i <= n; ++i) { g[i] = exp(a[i] - mx); z += g[i]; }
            for (int i = 0; i <= n; ++i) g[i] /= z;
        }
        double* yr = y + (size_t)bh * dv;
        for (int c = 0; c < dv; ++c) {
            double acc = 0.0;
            for (int r = 0; r < dk; ++r) acc += Mon[(size_t)c * dk + r] * qh[r];
            yr[c] = g[n] * acc;
        }
        for (int i = 0; i < n; ++i) {
            const double* Mi = M_cache + ((size_t)bh * n_cap + i) * dv * dk;
            for (int c = 0; c < dv; ++c) {
                double acc = 0.0;
                for (int r = 0; r < dk; ++r) acc += Mi[(size_t)c * dk + r] * qh[r];
                yr[c] += g[i] * acc;
            }
        }
        if (gamma) {
            double* gr = gamma + (size_t)bh * (n_cap + 1);
            for (int i = 0; i <= n_cap; ++i) gr[i] = 0.0;
            for (int i = 0; i < n; ++i) gr[i] = g[i];
            gr[n_cap] = g[n];
        }
        if (emit) {
            memcpy(M_cache + ((size_t)bh * n_cap + n) * dv * dk, Mon, sizeof(double) * dv * dk);
            memset(Mon, 0, sizeof(double) * dv * dk);
        }
        free(a); free(g);
    }
    for (int b = 0; b < B; ++b)
        for (int hx = 0; hx < xh; ++hx) {
            double* dst = xsum + ((size_t)b * xh + hx) * dg;
            const double* src = xs_new + ((size_t)b * xh + hx) * dg;
            if (emit) {
                double* Pn = P_cache + (((size_t)b * xh + hx) * n_cap + n) * dg;
                for (int e = 0; e < dg; ++e) Pn[e] = src[e] / (double)C;
                for (int e = 0; e < dg; ++e) dst[e] = 0.0;
            } else {
                for (int e = 0; e < dg; ++e) dst[e] = src[e];
            }
        }
    free(xs_new);
    if (emit) { *count = 0; *n_cached = n + 1; } else { *count = cnt + 1; }
    return MCO_OK;
}

/* derivative of phi ([MC] Eq. 2 feature map): 1, or 1 for z > 0 and e^z otherwise. */
static double mco_dphi(double z, int phi) {
    if (phi == 0) return 1.0;
    return z > 0.0 ? 1.0 : exp(z);
}

/*
 * Gradients of the GRM prefill with respect to its inputs: the chain rule applied to the
 * per-token definitions ([MC] Eq. 4b memories, the Eq. 10 softmax gate, the Eq. 9 read),
 * for an upstream gradient dY of Y.  With o_i = M^(i) phi(q_t) for the cached segments
 * i < s and o_s = M_t^(s) phi(q_t) for the online one, y_t = sum_i g_i o_i and
 *   dg_i = <dy_t, o_i>,  da_i = g_i (dg_i - sum_j g_j dg_j)          (softmax)
 *   du_t = sum_{i<s} da_i P_i + da_s p_t        (p_t: prefix mean of x in segment s)
 *   dP_i += da_i u_t,  dp_t = da_s u_t
 *   dphi(q_t) = sum_{i<s} g_i M^(i)^T dy_t + g_s M_t^(s)^T dy_t
 *   dM^(i) += g_i dy_t phi(q_t)^T  (i < s),  and for r <= t in segment s (the online memory
 *   holds v_r phi(k_r)^T): dv_r += g_s <phi(q_t), phi(k_r)> dy_t,
 *   dphi(k_r) += g_s <dy_t, v_r> phi(q_t).
 * Then for r in segment i: dv_r += dM^(i) phi(k_r), dphi(k_r) += dM^(i)^T v_r,
 * dx_r += dP_i / |S_i| + sum_{t >= r in segment i} dp_t / (j_t + 1); finally
 * dq = dphi(q) phi'(q), dk = dphi(k) phi'(k).
 *
 * dims = {B, H, L, dk, dv, dg, C, xh, phi} (segments of constant length C).  Inputs as for
 * mco_prefill; dY [B,H,L,dv].  Outputs dQ, dK [B,H,L,dk], dV [B,H,L,dv], dU [B,H,L,dg],
 * dX [B,xh,L,dg] (with xh = 1 the heads' contributions are summed, in head order).
 * rows (ascending, n_rows of them) restricts the work to the gradients that belong to single
 * tokens, dQ and dU [B,H,n_rows,.] at those rows; dK, dV and dX are then not written.
 */
int mco_grm_backward(const int32_t* dims, const double* Q, const double* K, const double* V,
                     const double* U, const double* X, const double* dY, double* dQ,
                     double* dK, double* dV, double* dU, double* dX, int n_threads,
                     const int32_t* rows, int64_t n_rows) {
    const int B = dims[0], H = dims[1], L = dims[2], dk = dims[3], dv = dims[4], dg = dims[5];
    const int C = dims[6], xh = dims[7], phi = dims[8];
    if (B <= 0 || H <= 0 || L <= 0 || dk <= 0 || dv <= 0 || dg <= 0 || C <= 0) return MCO_EARG;
    if (!(xh == 1 || xh == H)) return MCO_EARG;
    const int NS = (L + C - 1) / C;
    const int64_t nr = rows ? n_rows : (int64_t)L;
    if (rows)
        for (int64_t a = 0; a < nr; ++a)
            if (rows[a] < 0 || rows[a] >= L || (a > 0 && rows[a] <= rows[a - 1])) return MCO_EARG;
#ifdef _OPENMP
    if (n_threads > 0) omp_set_num_threads(n_threads);
#else
    (void)n_threads;
#endif
    double* dXh = (double*)calloc(rows ? 1 : (size_t)B * H * L * dg, sizeof(double));
    if (!dXh) return MCO_ENOMEM;
    int err = MCO_OK;

#pragma omp parallel for schedule(dynamic, 1)
    for (int bh = 0; bh < B * H; ++bh) {
        const int b = bh / H, h = bh % H;
        const int hx = (xh == 1) ? 0 : h;
        const double* q = Q + (size_t)bh * L * dk;
        const double* k = K + (size_t)bh * L * dk;
        const double* v = V + (size_t)bh * L * dv;
        const double* u = U + (size_t)bh * L * dg;
        const double* x = X + ((size_t)b * xh + hx) * L * dg;
        const double* dy = dY + (size_t)bh * L * dv;
        double* dq = dQ + (size_t)bh * nr * dk;
        double* dkk = rows ? NULL : dK + (size_t)bh * L * dk;
        double* dvv = rows ? NULL : dV + (size_t)bh * L * dv;
        double* du = dU + (size_t)bh * nr * dg;
        double* dx = rows ? NULL : dXh + (size_t)bh * L * dg;
        int64_t next = 0; /* position in rows */

        double* qh = (double*)malloc(sizeof(double) * L * dk);
        double* kh = (double*)malloc(sizeof(double) * L * dk);
        double* Mc = (double*)calloc((size_t)NS * dv * dk, sizeof(double));
        double* dMc = (double*)calloc((size_t)NS * dv * dk, sizeof(double));
        double* Pc = (double*)calloc((size_t)NS * dg, sizeof(double));
        double* dPc = (double*)calloc((size_t)NS * dg, sizeof(double));
        double* Mon = (double*)calloc((size_t)dv * dk, sizeof(double));
        double* xs = (double*)calloc((size_t)dg, sizeof(double));
        double* gs = (double*)malloc(sizeof(double) * L);        /* online weight per token */
        double* wt = (double*)calloc((size_t)L * dg, sizeof(double)); /* dp_t / (j_t + 1) */
        double* dqh = (double*)calloc((size_t)L * dk, sizeof(double));
        double* dkh = (double*)calloc((size_t)L * dk, sizeof(double));
        double* a = (double*)malloc(sizeof(double) * (NS + 1));
        double* g = (double*)malloc(sizeof(double) * (NS + 1));
        double* dgm = (double*)malloc(sizeof(double) * (NS + 1));
        double* o = (double*)malloc(sizeof(double) * (size_t)(NS + 1) * dv);
        if (!qh || !kh || !Mc || !dMc || !Pc || !dPc || !Mon || !xs || !gs || !wt || !dqh ||
            !dkh || !a || !g || !dgm || !o) {
#pragma omp atomic write
            err = MCO_ENOMEM;
        } else {
            for (size_t e = 0; e < (size_t)L * dk; ++e) {
                qh[e] = mco_phi(q[e], phi);
                kh[e] = mco_phi(k[e], phi);
            }
            /* the cached states and means (forward, [MC] Eq. 4b and Eq. 10) */
            for (int t = 0; t < L; ++t) {
                const int i = t / C;
                for (int c = 0; c < dv; ++c)
                    for (int r = 0; r < dk; ++r)
                        Mc[((size_t)i * dv + c) * dk + r] += v[(size_t)t * dv + c] * kh[(size_t)t * dk + r];
                for (int e = 0; e < dg; ++e) Pc[(size_t)i * dg + e] += x[(size_t)t * dg + e];
            }
            for (int i = 0; i < NS; ++i) {
                const int len = (i + 1 < NS ? C : L - i * C);
                for (int e = 0; e < dg; ++e) Pc[(size_t)i * dg + e] /= (double)len;
            }
            for (int t = 0; t < L; ++t) {
                const int s = t / C, j = t - s * C;
                if (j == 0) {
                    memset(Mon, 0, sizeof(double) * dv * dk);
                    memset(xs, 0, sizeof(double) * dg);
                }
                const double* kt = kh + (size_t)t * dk;
                const double* qt = qh + (size_t)t * dk;
                const double* ut = u + (size_t)t * dg;
                const double* dyt = dy + (size_t)t * dv;
                for (int c = 0; c < dv; ++c)
                    for (int r = 0; r < dk; ++r) Mon[(size_t)c * dk + r] += v[(size_t)t * dv + c] * kt[r];
                for (int e = 0; e < dg; ++e) xs[e] += x[(size_t)t * dg + e];
                int64_t row = t; /* output row of this token */
                if (rows) {
                    if (next >= nr || rows[next] != t) continue;
                    row = next++;
                }
                /* gate (forward) */
                for (int i = 0; i < s; ++i) {
                    double acc = 0.0;
                    for (int e = 0; e < dg; ++e) acc += ut[e] * Pc[(size_t)i * dg + e];
                    a[i] = acc;
                }
                {
                    double acc = 0.0;
                    for (int e = 0; e < dg; ++e) acc += ut[e] * (xs[e] / (double)(j + 1));
                    a[s] = acc;
                }
                double mx = a[0];
                for (int i = 1; i <= s; ++i) mx = fmax(mx, a[i]);
                double z = 0.0;
                for (int i = 0; i <= s; ++i) { g[i] = exp(a[i] - mx); z += g[i]; }
                for (int i = 0; i <= s; ++i) g[i] /= z;
                gs[t] = g[s];
                /* the reads o_i and their gradients dg_i */
                for (int i = 0; i <= s; ++i) {
                    const double* Mi = (i < s) ? Mc + (size_t)i * dv * dk : Mon;
                    double dgi = 0.0;
                    for (int c = 0; c < dv; ++c) {
                        double acc = 0.0;
                        for (int r = 0; r < dk; ++r) acc += Mi[(size_t)c * dk + r] * qt[r];
                        o[(size_t)i * dv + c] = acc;
                        dgi += dyt[c] * acc;
                    }
                    dgm[i] = dgi;
                }
                double D = 0.0;
                for (int i = 0; i <= s; ++i) D += g[i] * dgm[i];
                /* softmax backward, then the gate's inputs */
                for (int e = 0; e < dg; ++e) du[(size_t)row * dg + e] = 0.0;
                for (int i = 0; i <= s; ++i) {
                    const double dai = g[i] * (dgm[i] - D);
                    for (int e = 0; e < dg; ++e) {
                        const double pe = (i < s) ? Pc[(size_t)i * dg + e] : xs[e] / (double)(j + 1);
                        du[(size_t)row * dg + e] += dai * pe;
                        if (i < s)
                            dPc[(size_t)i * dg + e] += dai * ut[e];
                        else
                            wt[(size_t)t * dg + e] = dai * ut[e] / (double)(j + 1);
                    }
                }
                /* dphi(q_t) and the cached states' gradients */
                for (int i = 0; i <= s; ++i) {
                    const double* Mi = (i < s) ? Mc + (size_t)i * dv * dk : Mon;
                    for (int c = 0; c < dv; ++c)
                        for (int r = 0; r < dk; ++r)
                            dqh[(size_t)row * dk + r] += g[i] * Mi[(size_t)c * dk + r] * dyt[c];
                    if (i < s && !rows) {
                        double* dMi = dMc + (size_t)i * dv * dk;
                        for (int c = 0; c < dv; ++c)
                            for (int r = 0; r < dk; ++r) dMi[(size_t)c * dk + r] += g[i] * dyt[c] * qt[r];
                    }
                }
            }
            /* the online memory's pairs r <= t of one segment */
            for (int t = 0; t < (rows ? 0 : L); ++t) {
                const int s0 = (t / C) * C;
                const double* qt = qh + (size_t)t * dk;
                const double* dyt = dy + (size_t)t * dv;
                for (int r = s0; r <= t; ++r) {
                    double qk = 0.0, dyv = 0.0;
                    for (int e = 0; e < dk; ++e) qk += qt[e] * kh[(size_t)r * dk + e];
                    for (int c = 0; c < dv; ++c) dyv += dyt[c] * v[(size_t)r * dv + c];
                    for (int c = 0; c < dv; ++c) dvv[(size_t)r * dv + c] += gs[t] * qk * dyt[c];
                    for (int e = 0; e < dk; ++e) dkh[(size_t)r * dk + e] += gs[t] * dyv * qt[e];
                }
            }
            /* the cached states' gradients reach the tokens of their segment */
            for (int r = 0; r < (rows ? 0 : L); ++r) {
                const int i = r / C;
                const double* dMi = dMc + (size_t)i * dv * dk;
                for (int c = 0; c < dv; ++c)
                    for (int e = 0; e < dk; ++e) {
                        dvv[(size_t)r * dv + c] += dMi[(size_t)c * dk + e] * kh[(size_t)r * dk + e];
                        dkh[(size_t)r * dk + e] += dMi[(size_t)c * dk + e] * v[(size_t)r * dv + c];
                    }
            }
            /* x: segment means and the online prefix means */
            for (int i = 0; i < (rows ? 0 : NS); ++i) {
                const int r0 = i * C, r1 = (i + 1 < NS ? (i + 1) * C : L);
                for (int e = 0; e < dg; ++e) {
                    double tail = 0.0;
                    for (int r = r1 - 1; r >= r0; --r) {
                        tail += wt[(size_t)r * dg + e];
                        dx[(size_t)r * dg + e] = dPc[(size_t)i * dg + e] / (double)(r1 - r0) + tail;
                    }
                }
            }
            for (int64_t a = 0; a < nr; ++a) {
                const int t = rows ? rows[a] : (int)a;
                for (int e = 0; e < dk; ++e)
                    dq[(size_t)a * dk + e] = dqh[(size_t)a * dk + e] * mco_dphi(q[(size_t)t * dk + e], phi);
            }
            if (!rows)
                for (size_t e = 0; e < (size_t)L * dk; ++e) dkk[e] = dkh[e] * mco_dphi(k[e], phi);
        }
        free(qh); free(kh); free(Mc); free(dMc); free(Pc); free(dPc); free(Mon); free(xs);
        free(gs); free(wt); free(dqh); free(dkh); free(a); free(g); free(dgm); free(o);
    }
    if (err == MCO_OK && !rows) {
        memset(dX, 0, sizeof(double) * (size_t)B * xh * L * dg);
        for (int bh = 0; bh < B * H; ++bh) {
            const int b = bh / H, h = bh % H;
            double* dst = dX + ((size_t)b * xh + (xh == 1 ? 0 : h)) * L * dg;
            const double* src = dXh + (size_t)bh * L * dg;
            for (size_t e = 0; e < (size_t)L * dg; ++e) dst[e] += src[e];
        }
    }
    free(dXh);
    return err;
}

/* Number of threads OpenMP will use (1 without OpenMP). */
int mco_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
