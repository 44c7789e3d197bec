/*
 * oracle.c -- plain, slow, fp64 CPU reference for the bounded-generation
 * attention hot path.  TEST INFRASTRUCTURE ONLY: the tests, the smoke check
 * and the bench's CPU-baseline leg call it; the product library never does,
 * and this file shares no code, header or table with it.
 *
 * Every function follows the plain definition of what the page
 * "SLM 生成式高并发推理引擎：延迟约束下的有效吞吐优化" says is computed:
 *   - packed prefill: each sequence keeps its own valid length and only its
 *     valid tokens are computed (§1.2); the model is decoder-only (abstract),
 *     hence causal attention inside each sequence and none across sequences;
 *   - last-valid-token selection for prefill-only outputs (abstract, §1.1);
 *   - beam search: all beams of a request share one prompt K/V and keep their
 *     own short suffix K/V (§1.2); each step merges per-beam candidates with
 *     the cumulative scores and keeps a fixed number, carrying parent indices
 *     (§1.1);
 *   - the same merge taking each beam row's logits, with the row's
 *     log-softmax folded in (the next step the page's fixed beam-search
 *     node runs on the model's output, §1.1);
 *   - the prefill-only label head: the next-token logits of the target
 *     label tokens at each sequence's last valid token, then softmax, top-K
 *     and a fixed mapping (§1.1, prefill-only models).
 * Where the page is silent the readings are: GQA query head h reads KV head
 * floor(h*Hkv/Hq); softmax scale is a parameter (1/sqrt(D) in every workload);
 * the causal boundary includes the diagonal; candidate score is one IEEE fp32
 * addition cum+logprob, ranked by score descending then flat index b*V+v
 * ascending.
 *
 * bf16 values arrive as their 16-bit storage and are widened exactly.
 * Parallelism is OpenMP over independent output rows / requests only.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

static double bf16_to_f64(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* One attention row: softmax(scale * q.k_j) over the n given keys, times V.
 * keys[j] / vals[j] point at D-element bf16 rows.  out gets D doubles. */
static void attend_row(const uint16_t *q, const uint16_t *const *keys,
                       const uint16_t *const *vals, int n, int D, double scale,
                       double *score /* n scratch */, double *out)
{
    double m = -INFINITY;
    for (int j = 0; j < n; ++j) {
        double s = 0.0;
        for (int d = 0; d < D; ++d)
            s += bf16_to_f64(q[d]) * bf16_to_f64(keys[j][d]);
        score[j] = scale * s;
        if (score[j] > m)
            m = score[j];
    }
    double denom = 0.0;
    for (int j = 0; j < n; ++j) {
        score[j] = exp(score[j] - m);
        denom += score[j];
    }
    for (int d = 0; d < D; ++d) {
        double acc = 0.0;
        for (int j = 0; j < n; ++j)
            acc += score[j] * bf16_to_f64(vals[j][d]);
        out[d] = acc / denom;
    }
}

/* Sequence that holds packed token t: cu[b] <= t < cu[b+1]. */
static int seq_of_token(const int32_t *cu, int B, int64_t t)
{
    for (int b = 0; b < B; ++b)
        if (t >= cu[b] && t < cu[b + 1])
            return b;
    return -1;
}

/* Causal attention of packed token t (query head h) over its own sequence.
 * q [T,Hq,D], k/v [T,Hkv,D]; out: D doubles. */
static void prefill_row(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                        const int32_t *cu, int B, int Hq, int Hkv, int D,
                        double scale, int64_t t, int h, double *out)
{
    int b = seq_of_token(cu, B, t);
    int64_t s0 = cu[b];
    int n = (int)(t - s0) + 1;                 /* keys s0..t, diagonal included */
    int g = (int)((int64_t)h * Hkv / Hq);      /* GQA: contiguous head groups */
    const uint16_t **keys = malloc(sizeof(*keys) * (size_t)n);
    const uint16_t **vals = malloc(sizeof(*vals) * (size_t)n);
    double *score = malloc(sizeof(double) * (size_t)n);
    for (int j = 0; j < n; ++j) {
        keys[j] = k + ((s0 + j) * Hkv + g) * (int64_t)D;
        vals[j] = v + ((s0 + j) * Hkv + g) * (int64_t)D;
    }
    attend_row(q + (t * Hq + h) * (int64_t)D, keys, vals, n, D, scale, score, out);
    free(keys);
    free(vals);
    free(score);
}

/* Packed causal GQA prefill attention, every row.  out [T,Hq,D] fp64. */
int orc_prefill_attn(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                     const int32_t *cu, int B, int Hq, int Hkv, int D,
                     double scale, double *out)
{
    if (B < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || Hq % Hkv != 0)
        return 1;
    int64_t T = cu[B];
#pragma omp parallel for schedule(dynamic, 16) collapse(2)
    for (int64_t t = 0; t < T; ++t)
        for (int h = 0; h < Hq; ++h)
            prefill_row(q, k, v, cu, B, Hq, Hkv, D, scale, t, h,
                        out + (t * Hq + h) * (int64_t)D);
    return 0;
}

/* The same rows, only at the n listed (token, head) pairs.  out [n,D]. */
int orc_prefill_attn_rows(const uint16_t *q, const uint16_t *k, const uint16_t *v,
                          const int32_t *cu, int B, int Hq, int Hkv, int D,
                          double scale, const int64_t *tokens, const int32_t *heads,
                          int64_t n, double *out)
{
    if (B < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || Hq % Hkv != 0)
        return 1;
#pragma omp parallel for schedule(dynamic, 4)
    for (int64_t i = 0; i < n; ++i)
        prefill_row(q, k, v, cu, B, Hq, Hkv, D, scale, tokens[i], heads[i],
                    out + i * (int64_t)D);
    return 0;
}

/* Last valid token of every sequence: out[b,:] = hidden[cu[b+1]-1,:];
 * an empty sequence gives a zero row.  Bit copy of 16-bit storage. */
int orc_gather_last(const uint16_t *hidden, const int32_t *cu, int B, int H,
                    uint16_t *out)
{
    for (int b = 0; b < B; ++b) {
        if (cu[b + 1] > cu[b])
            memcpy(out + (int64_t)b * H, hidden + ((int64_t)cu[b + 1] - 1) * H,
                   sizeof(uint16_t) * (size_t)H);
        else
            memset(out + (int64_t)b * H, 0, sizeof(uint16_t) * (size_t)H);
    }
    return 0;
}

/* Prefill-only label head.  For sequence b, h = its last valid hidden row
 * (zero for an empty sequence); for label j, z[b,j] = h . lm[label[j]] (fp64
 * over the 16-bit-storage values); p[b,:] = softmax over the L label logits
 * (fp64, shifted by the row maximum); the K labels with the largest logits,
 * ties to the lower label index, in that order: their index j and
 * probability; with a map, class[b,k] = map[j].  hidden [T,H], lm [V,H]
 * bf16 storage; label [L] token ids. */
int orc_label_head(const uint16_t *hidden, const int32_t *cu, int B, int H,
                   const uint16_t *lm, int V, const int32_t *label, int L, int K,
                   const int32_t *map, double *logits, double *probs,
                   int32_t *top_idx, double *top_prob, int32_t *top_class)
{
    if (B < 0 || H <= 0 || V <= 0 || L <= 0 || K <= 0 || K > L)
        return 1;
    for (int j = 0; j < L; ++j)
        if (label[j] < 0 || label[j] >= V)
            return 1;
#pragma omp parallel for schedule(dynamic, 4)
    for (int b = 0; b < B; ++b) {
        const int64_t last = cu[b + 1] > cu[b] ? (int64_t)cu[b + 1] - 1 : -1;
        double *z = logits + (int64_t)b * L;
        double m = -INFINITY;
        for (int j = 0; j < L; ++j) {
            double acc = 0.0;
            if (last >= 0) {
                const uint16_t *hr = hidden + last * H, *wr = lm + (int64_t)label[j] * H;
                for (int d = 0; d < H; ++d)
                    acc += bf16_to_f64(hr[d]) * bf16_to_f64(wr[d]);
            }
            z[j] = acc;
            if (acc > m)
                m = acc;
        }
        double s = 0.0;
        for (int j = 0; j < L; ++j)
            s += exp(z[j] - m);
        for (int j = 0; j < L; ++j)
            probs[(int64_t)b * L + j] = exp(z[j] - m) / s;
        /* top K by selection: each pick is the largest logit not yet taken,
         * the lower index first among equals */
        unsigned char *taken = calloc((size_t)L, 1);
        for (int k = 0; k < K; ++k) {
            int best = -1;
            for (int j = 0; j < L; ++j)
                if (!taken[j] && (best < 0 || z[j] > z[best]))
                    best = j;
            taken[best] = 1;
            top_idx[(int64_t)b * K + k] = best;
            top_prob[(int64_t)b * K + k] = probs[(int64_t)b * L + best];
            if (top_class)
                top_class[(int64_t)b * K + k] = map ? map[best] : best;
        }
        free(taken);
    }
    return 0;
}

/* Beam decode attention over a shared prompt and per-beam suffixes.
 *   q       [NL,R,W,Hq,D]          prefix_k/v [NL,R,P,Hkv,D]
 *   sk_in/sv_in [NL,R,W,S_cap,Hkv,D]  history rows 0..hist-1, previous order
 *   k_new/v_new [NL,R,W,Hkv,D]      parent [R,W] (NULL: identity)
 * For beam j the history is the suffix of beam parent[j]; its keys are the P
 * prompt rows, the hist history rows and the new row (s = hist+1 keys of its
 * own), all visible.  out [NL,R,W,Hq,D] fp64; sk_out/sv_out rows 0..hist get
 * the history (current order) and the new row. */
int orc_beam_decode_attn(int NL, int R, int W, int P, int hist, int S_cap,
                         int Hq, int Hkv, int D, double scale,
                         const uint16_t *q, const uint16_t *prefix_k,
                         const uint16_t *prefix_v, const uint16_t *sk_in,
                         const uint16_t *sv_in, const uint16_t *k_new,
                         const uint16_t *v_new, const int32_t *parent,
                         const int32_t *prompt_cu,
                         double *out, uint16_t *sk_out, uint16_t *sv_out)
{
    if (NL <= 0 || R <= 0 || W <= 0 || P < 0 || hist < 0 || hist + 1 > S_cap ||
        Hq <= 0 || Hkv <= 0 || D <= 0 || Hq % Hkv != 0)
        return 1;
    /* Prompts of request r: rows prompt_cu[r] .. prompt_cu[r+1] of each
       layer's [prompt_cu[R], Hkv, D] block (each at most P long); without
       prompt_cu, every request has P rows ([R, P, Hkv, D] per layer). */
    if (prompt_cu) {
        if (prompt_cu[0] != 0) return 1;
        for (int r = 0; r < R; ++r)
            if (prompt_cu[r + 1] < prompt_cu[r] || prompt_cu[r + 1] - prompt_cu[r] > P) return 1;
    }
    const int64_t Tp = prompt_cu ? prompt_cu[R] : (int64_t)R * P;   /* prompt rows per layer */
    const int nkeys = P + hist + 1;
#pragma omp parallel for collapse(3) schedule(dynamic, 1)
    for (int l = 0; l < NL; ++l)
        for (int r = 0; r < R; ++r)
            for (int j = 0; j < W; ++j) {
                int src = parent ? parent[r * W + j] : j;
                const uint16_t **keys = malloc(sizeof(*keys) * (size_t)nkeys);
                const uint16_t **vals = malloc(sizeof(*vals) * (size_t)nkeys);
                double *score = malloc(sizeof(double) * (size_t)nkeys);
                for (int h = 0; h < Hq; ++h) {
                    int g = (int)((int64_t)h * Hkv / Hq);
                    int n = 0;
                    const int64_t p0 = prompt_cu ? prompt_cu[r] : (int64_t)r * P;
                    const int Pr = prompt_cu ? prompt_cu[r + 1] - prompt_cu[r] : P;
                    for (int i = 0; i < Pr; ++i) {
                        int64_t off = (((int64_t)l * Tp + p0 + i) * Hkv + g) * D;
                        keys[n] = prefix_k + off;
                        vals[n] = prefix_v + off;
                        ++n;
                    }
                    for (int i = 0; i < hist; ++i) {
                        int64_t off = (((((int64_t)l * R + r) * W + src) * S_cap + i) * Hkv + g) * D;
                        keys[n] = sk_in + off;
                        vals[n] = sv_in + off;
                        ++n;
                    }
                    int64_t noff = ((((int64_t)l * R + r) * W + j) * Hkv + g) * D;
                    keys[n] = k_new + noff;
                    vals[n] = v_new + noff;
                    ++n;
                    int64_t qoff = ((((int64_t)l * R + r) * W + j) * Hq + h) * D;
                    attend_row(q + qoff, keys, vals, n, D, scale, score, out + qoff);
                }
                /* suffix in the current beam order: history of the parent, then the new row */
                for (int i = 0; i <= hist; ++i)
                    for (int g = 0; g < Hkv; ++g) {
                        int64_t dst = (((((int64_t)l * R + r) * W + j) * S_cap + i) * Hkv + g) * D;
                        const uint16_t *ks, *vs;
                        if (i < hist) {
                            int64_t so = (((((int64_t)l * R + r) * W + src) * S_cap + i) * Hkv + g) * D;
                            ks = sk_in + so;
                            vs = sv_in + so;
                        } else {
                            int64_t so = ((((int64_t)l * R + r) * W + j) * Hkv + g) * D;
                            ks = k_new + so;
                            vs = v_new + so;
                        }
                        memcpy(sk_out + dst, ks, sizeof(uint16_t) * (size_t)D);
                        memcpy(sv_out + dst, vs, sizeof(uint16_t) * (size_t)D);
                    }
                free(keys);
                free(vals);
                free(score);
            }
    return 0;
}

/* Candidate a ranks before candidate b: higher fp32 score first, then the
 * lower flat index.  IEEE comparison, so +0 and -0 are equal scores. */
static int ranks_before(float sa, int64_t fa, float sb, int64_t fb)
{
    return sa > sb || (sa == sb && fa < fb);
}

/* Beam top-k merge.  For request r and every candidate (b,v) the score is
 * the fp32 sum cum[r,b] + lp[r,b,v]; the W first candidates in the order
 * above are written sorted: token = f mod V, parent = f div V, cum_out =
 * score, with f = b*V + v.  Kept as a sorted array of the best W seen. */
int orc_topk_merge(const float *lp, const float *cum, int R, int Win, int V,
                   int W, int32_t *tokens, int32_t *parent, float *cum_out)
{
    if (R <= 0 || Win <= 0 || V <= 0 || W <= 0 || (int64_t)W > (int64_t)Win * V)
        return 1;
#pragma omp parallel for schedule(dynamic, 1)
    for (int r = 0; r < R; ++r) {
        float *best_s = malloc(sizeof(float) * (size_t)W);
        int64_t *best_f = malloc(sizeof(int64_t) * (size_t)W);
        int count = 0;
        for (int b = 0; b < Win; ++b) {
            float c = cum[(int64_t)r * Win + b];
            for (int v = 0; v < V; ++v) {
                float s = c + lp[((int64_t)r * Win + b) * V + v];   /* one fp32 add */
                int64_t f = (int64_t)b * V + v;
                if (count == W && !ranks_before(s, f, best_s[W - 1], best_f[W - 1]))
                    continue;
                int pos = count < W ? count : W - 1;   /* slot to fill, then bubble up */
                if (count < W)
                    ++count;
                while (pos > 0 && ranks_before(s, f, best_s[pos - 1], best_f[pos - 1])) {
                    best_s[pos] = best_s[pos - 1];
                    best_f[pos] = best_f[pos - 1];
                    --pos;
                }
                best_s[pos] = s;
                best_f[pos] = f;
            }
        }
        for (int j = 0; j < W; ++j) {
            tokens[(int64_t)r * W + j] = (int32_t)(best_f[j] % V);
            parent[(int64_t)r * W + j] = (int32_t)(best_f[j] / V);
            cum_out[(int64_t)r * W + j] = best_s[j];
        }
        free(best_s);
        free(best_f);
    }
    return 0;
}

/* Beam top-k merge on logits (the merge with its log-softmax folded in).
 * For request r and beam row b: lse[r,b] = log sum_v exp(x[r,b,v]) over the
 * row's V logits (fp64, shifted by the row maximum); the log-probability of
 * (b,v) is x - lse and the candidate score is cum[r,b] + (x - lse), all in
 * fp64.  Candidates rank by score descending, then flat index f = b*V + v
 * ascending; the W first are written in that order (token = f mod V, parent
 * = f div V, score), with every row's lse.  Logits are finite or -inf, and
 * every row holds at least one finite logit. */
int orc_topk_merge_logits(const float *x, const float *cum, int R, int Win, int V,
                          int W, int32_t *tokens, int32_t *parent, double *score_out,
                          double *lse_out)
{
    if (R <= 0 || Win <= 0 || V <= 0 || W <= 0 || (int64_t)W > (int64_t)Win * V)
        return 1;
    int bad = 0;
#pragma omp parallel for schedule(static)
    for (int64_t row = 0; row < (int64_t)R * Win; ++row) {
        const float *xr = x + row * V;
        double m = -INFINITY;
        for (int v = 0; v < V; ++v)
            if ((double)xr[v] > m)
                m = xr[v];
        double s = 0.0;
        for (int v = 0; v < V; ++v)
            s += exp((double)xr[v] - m);       /* exp(-inf) = 0 */
        if (!(m > -INFINITY) || !isfinite(m) || isnan(s)) {
#pragma omp atomic write
            bad = 1;
        }
        lse_out[row] = m + log(s);
    }
    if (bad)
        return 1;
#pragma omp parallel for schedule(dynamic, 1)
    for (int r = 0; r < R; ++r) {
        double *best_s = malloc(sizeof(double) * (size_t)W);
        int64_t *best_f = malloc(sizeof(int64_t) * (size_t)W);
        int count = 0;
        for (int b = 0; b < Win; ++b) {
            const int64_t row = (int64_t)r * Win + b;
            const double c = cum[row], lse = lse_out[row];
            for (int v = 0; v < V; ++v) {
                const double s = c + ((double)x[row * V + v] - lse);
                const int64_t f = (int64_t)b * V + v;
                if (count == W && !(s > best_s[W - 1] || (s == best_s[W - 1] && f < best_f[W - 1])))
                    continue;
                int pos = count < W ? count : W - 1;
                if (count < W)
                    ++count;
                while (pos > 0 && (s > best_s[pos - 1] || (s == best_s[pos - 1] && f < best_f[pos - 1]))) {
                    best_s[pos] = best_s[pos - 1];
                    best_f[pos] = best_f[pos - 1];
                    --pos;
                }
                best_s[pos] = s;
                best_f[pos] = f;
            }
        }
        for (int j = 0; j < W; ++j) {
            tokens[(int64_t)r * W + j] = (int32_t)(best_f[j] % V);
            parent[(int64_t)r * W + j] = (int32_t)(best_f[j] / V);
            score_out[(int64_t)r * W + j] = best_s[j];
        }
        free(best_s);
        free(best_f);
    }
    return 0;
}

/* Suffix reorder after a merge: new[l,r,j,i] = old[l,r,parent[r,j],i] for
 * rows i < rows, every layer, K and V.  [NL,R,W,S_cap,Hkv,D] 16-bit storage. */
int orc_reorder_suffix(int NL, int R, int W, int rows, int S_cap, int Hkv, int D,
                       const int32_t *parent, const uint16_t *k_in,
                       const uint16_t *v_in, uint16_t *k_out, uint16_t *v_out)
{
    if (NL <= 0 || R <= 0 || W <= 0 || rows < 0 || rows > S_cap || Hkv <= 0 || D <= 0)
        return 1;
    const int64_t row = (int64_t)Hkv * D;
    for (int l = 0; l < NL; ++l)
        for (int r = 0; r < R; ++r)
            for (int j = 0; j < W; ++j) {
                int src = parent[r * W + j];
                for (int i = 0; i < rows; ++i) {
                    int64_t dst = ((((int64_t)l * R + r) * W + j) * S_cap + i) * row;
                    int64_t so = ((((int64_t)l * R + r) * W + src) * S_cap + i) * row;
                    memcpy(k_out + dst, k_in + so, sizeof(uint16_t) * (size_t)row);
                    memcpy(v_out + dst, v_in + so, sizeof(uint16_t) * (size_t)row);
                }
            }
    return 0;
}

/* Final backtrack of a fixed-step beam search into token sequences (the
 * request returns its candidate sequences: page "SLM 生成式高并发推理引擎：延迟
 * 约束下的有效吞吐优化", §1.1, beam-search form).  tokens and parent hold the
 * outputs of the n_merges merges, [n_merges, R, W] each (merge 0 takes one
 * beam in, so its parents are 0).  Beam j after the last merge emitted
 * tokens[n_merges-1][r][j] and descends from beam parent[n_merges-1][r][j] of
 * the merge before; following the parents back to merge 0 gives one token
 * per merge.  seq [R, W, n_merges]: seq[r][j][t] = the token beam j's
 * ancestor took at merge t.  A parent outside [0, W) is rejected. */
int orc_beam_backtrack(const int32_t *tokens, const int32_t *parent, int n_merges, int R,
                       int W, int32_t *seq)
{
    if (n_merges <= 0 || R <= 0 || W <= 0)
        return 1;
    for (int r = 0; r < R; ++r)
        for (int j = 0; j < W; ++j) {
            int b = j;                                  /* beam index at merge t */
            for (int t = n_merges - 1; t >= 0; --t) {
                const int64_t at = ((int64_t)t * R + r) * W + b;
                seq[((int64_t)r * W + j) * n_merges + t] = tokens[at];
                b = parent[at];
                if (t > 0 && (b < 0 || b >= W))
                    return 1;
            }
        }
    return 0;
}
