/*
 * msa_oracle.c -- plain, slow, obviously-correct CPU oracle for MiniMax Sparse
 * Attention (MSA).  TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and
 * the benchmark's CPU-baseline leg are its only callers.  The GPU library never
 * links, loads or calls it, and it shares no source with the GPU library.
 *
 * Sources (cited by page title and section):
 *   [P1] "MSA 稀疏注意力三国杀：NSA / DSA / MoBA / MSA 四方案深度对比"
 *        (ai-engineering-6yk.pages.dev), sections "第一步：粗筛", "第二步：精算",
 *        "Kernel 创新：Outer Gather Q", "附录最有意思：head 涌现的三种模式".
 *   [P3] "稀疏注意力速览（Sparse Attention，2019 ~ 2026）" (speedcell4.github.io),
 *        entry "MiniMax Sparse Attention（MSA）".
 *   [P1] also section "索引分支训练：KL 对齐" for the training functions.
 *   [P5] "稀疏注意力架构革命：2026年长上下文大模型核心技术解析" (chenxutan.com),
 *        section on standard self-attention (softmax(QK^T/sqrt(d_k))V).
 *
 * Every function works on ONE (sequence, KV-group) slice; the caller loops over
 * slices.  All arithmetic is IEEE double.  Inputs arrive already decoded from
 * their storage dtype (bf16/fp32 -> double is exact).
 *
 * Notation: N keys, block size B, nb = ceil(N/B) blocks; a query row r sits at
 * absolute position pos[r] (0-based, pos < N) and owns block bt = pos/B.
 *
 * Readings where the pages are silent (each also listed in the design notes):
 *   - the index score is the raw dot product q_I . k_I (no scale, no activation);
 *   - the block max-pool only covers keys j <= pos (causal), blocks b > bt are
 *     not scored (written as NaN here, "not written" on the GPU);
 *   - ties between equal block scores go to the lower block index;
 *   - when fewer than k blocks are eligible, all bt+1 are selected and the rest
 *     of the row is padded with -1; selections are emitted in ascending order;
 *   - the main branch scales logits by softmax_scale (1/sqrt(d) by default).
 *
 * Parity status: every function here is pinned by tests against brute force,
 * closed forms and special cases that reduce to textbook dense attention; the
 * training functions against float64 autograd, closed forms and finite differences.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* [P1 第一步：粗筛 items 1-2; P3 MSA entry: token scores first, then a max-pool inside each block]
 * out[r*nb + b] = max over keys j in block b with j <= pos[r] of
 *                 sum_c qI[r*dI + c] * kI[j*dI + c],          for b <= pos[r]/B;
 * out[r*nb + b] = NaN for b > pos[r]/B (such blocks are not eligible). */
void orc_index_scores(int64_t N, int B, int dI, int64_t nrows,
                      const double *qI, const int64_t *pos, const double *kI,
                      double *out)
{
    const int64_t nb = (N + B - 1) / B;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < nrows; ++r) {
        const int64_t p = pos[r];
        const int64_t bt = p / B;
        const double *q = qI + r * dI;
        for (int64_t b = 0; b < nb; ++b) {
            if (b > bt) { out[r * nb + b] = NAN; continue; }
            double best = -INFINITY;
            int64_t jend = (b + 1) * B - 1;
            if (jend > p) jend = p;
            for (int64_t j = b * B; j <= jend; ++j) {
                const double *kk = kI + j * dI;
                double s = 0.0;
                for (int c = 0; c < dI; ++c) s += q[c] * kk[c];
                if (s > best) best = s;
            }
            out[r * nb + b] = best;
        }
    }
}

/* [P1 第一步：粗筛 item 3 (the block of the current position is always taken, the others by score) and the closing
 *  rule of the head-pattern appendix (only the own block is forced);
 *  P3 MSA entry (each GQA group runs its own top-k over blocks and always keeps the local block of the
 *  current token)]
 * Row r: start from {own[r]}; repeatedly add the not-yet-chosen block b < own[r]
 * with the largest score, ties to the smaller b, until min(k, own[r]+1) blocks
 * are chosen.  Emit ascending, pad with -1.  scores is [nrows, nb]. */
void orc_block_topk(int64_t nb, int k, int64_t nrows, const double *scores,
                    const int64_t *own, int32_t *sel)
{
#pragma omp parallel
    {
        unsigned char *taken = (unsigned char *)calloc((size_t)nb, 1);
        int64_t *chosen = (int64_t *)malloc(sizeof(int64_t) * (size_t)k);
#pragma omp for schedule(dynamic, 64)
        for (int64_t r = 0; r < nrows; ++r) {
            const double *s = scores + r * nb;
            const int64_t bt = own[r];
            int64_t want = bt + 1 < k ? bt + 1 : k;
            memset(taken, 0, (size_t)nb);
            int n = 0;
            chosen[n++] = bt;
            taken[bt] = 1;
            while (n < want) {
                int64_t best = -1;
                for (int64_t b = 0; b < bt; ++b) {
                    if (taken[b]) continue;
                    if (best < 0 || s[b] > s[best]) best = b; /* strict: lower b keeps ties */
                }
                taken[best] = 1;
                chosen[n++] = best;
            }
            /* ascending order: insertion sort of <= k ids */
            for (int i = 1; i < n; ++i) {
                int64_t v = chosen[i];
                int j = i - 1;
                while (j >= 0 && chosen[j] > v) { chosen[j + 1] = chosen[j]; --j; }
                chosen[j + 1] = v;
            }
            for (int i = 0; i < k; ++i) sel[r * k + i] = i < n ? (int32_t)chosen[i] : -1;
        }
        free(taken);
        free(chosen);
    }
}

/* [P1 Kernel 创新：Outer Gather Q: for each block, collect every query that chose it]
 * Inverse of one slice's selection: for every block b, the list of entries
 * t*k + slot (ascending t) of query rows t whose selection holds b at `slot`.
 * offsets has nb+1 entries (offsets[0] = 0); entries has room for T*k ints.
 * Written as a two-pass counting sort so a full-size slice stays O(T*k). */
void orc_invert(int64_t T, int k, int64_t nb, const int32_t *sel,
                int64_t *offsets, int32_t *entries)
{
    int64_t *cursor = (int64_t *)calloc((size_t)nb, sizeof(int64_t));
    for (int64_t b = 0; b <= nb; ++b) offsets[b] = 0;
    for (int64_t t = 0; t < T; ++t)
        for (int i = 0; i < k; ++i) {
            int32_t b = sel[t * k + i];
            if (b >= 0) offsets[b + 1] += 1;
        }
    for (int64_t b = 0; b < nb; ++b) offsets[b + 1] += offsets[b];
    for (int64_t b = 0; b < nb; ++b) cursor[b] = offsets[b];
    for (int64_t t = 0; t < T; ++t)
        for (int i = 0; i < k; ++i) {
            int32_t b = sel[t * k + i];
            if (b >= 0) entries[cursor[b]++] = (int32_t)(t * k + i);
        }
    free(cursor);
}

/* [P1 第二步：精算: full attention only over the chosen blocks; P3 MSA entry: the main
 *  branch computes exact softmax attention on those blocks only; P5 standard formula
 *  softmax(QK^T/sqrt(d_k))V]
 * For row r and each of the G query heads of this group:
 *   J = union over valid sel[r][i] of [b*B, (b+1)*B) intersected with [0, pos[r]];
 *   out[r,h,:] = sum_{j in J} softmax_j(scale * q[r,h,:].K[j,:]) V[j,:].
 * q is [nrows, G, d]; K, V are [N, d]; sel is [nrows, k]; out is [nrows, G, d]. */
void orc_attention(int64_t N, int B, int d, int G, int k, int64_t nrows,
                   const double *q, const int64_t *pos, const int32_t *sel,
                   const double *K, const double *V, double scale, double *out)
{
    (void)N;
#pragma omp parallel
    {
        double *logit = (double *)malloc(sizeof(double) * (size_t)k * (size_t)B);
        int64_t *key = (int64_t *)malloc(sizeof(int64_t) * (size_t)k * (size_t)B);
#pragma omp for schedule(dynamic, 1)
        for (int64_t r = 0; r < nrows; ++r) {
            const int64_t p = pos[r];
            int64_t nk = 0;
            for (int i = 0; i < k; ++i) {
                int32_t b = sel[r * k + i];
                if (b < 0) continue;
                for (int64_t j = (int64_t)b * B; j < ((int64_t)b + 1) * B && j <= p; ++j) key[nk++] = j;
            }
            for (int h = 0; h < G; ++h) {
                const double *qq = q + (r * G + h) * d;
                double m = -INFINITY;
                for (int64_t a = 0; a < nk; ++a) {
                    const double *kk = K + key[a] * d;
                    double s = 0.0;
                    for (int c = 0; c < d; ++c) s += qq[c] * kk[c];
                    logit[a] = s * scale;
                    if (logit[a] > m) m = logit[a];
                }
                double l = 0.0;
                for (int64_t a = 0; a < nk; ++a) { logit[a] = exp(logit[a] - m); l += logit[a]; }
                double *o = out + (r * G + h) * d;
                for (int c = 0; c < d; ++c) o[c] = 0.0;
                for (int64_t a = 0; a < nk; ++a) {
                    const double w = logit[a] / l;
                    const double *vv = V + key[a] * d;
                    for (int c = 0; c < d; ++c) o[c] += w * vv[c];
                }
            }
        }
        free(logit);
        free(key);
    }
}

/* Partial form of the main branch, one result per selected block (the unit of
 * work of the Outer-Gather-Q order in [P1 Kernel 创新：Outer Gather Q]):
 *   lse[r,i,h] = log sum_{j in block sel[r][i], j <= pos} exp(scale q.K_j)
 *   Op[r,i,h,:] = softmax over that block alone, applied to V.
 * Slots with sel = -1 get lse = -inf and Op = 0.
 * lse is [nrows, k, G]; Op is [nrows, k, G, d]. */
void orc_attention_partials(int64_t N, int B, int d, int G, int k, int64_t nrows,
                            const double *q, const int64_t *pos, const int32_t *sel,
                            const double *K, const double *V, double scale,
                            double *lse, double *Op)
{
    (void)N;
#pragma omp parallel
    {
        double *logit = (double *)malloc(sizeof(double) * (size_t)B);
#pragma omp for schedule(dynamic, 1)
        for (int64_t r = 0; r < nrows; ++r) {
            const int64_t p = pos[r];
            for (int i = 0; i < k; ++i) {
                const int32_t b = sel[r * k + i];
                for (int h = 0; h < G; ++h) {
                    double *o = Op + ((r * k + i) * G + h) * d;
                    double *L = lse + (r * k + i) * G + h;
                    for (int c = 0; c < d; ++c) o[c] = 0.0;
                    if (b < 0) { *L = -INFINITY; continue; }
                    const double *qq = q + (r * G + h) * d;
                    int64_t j0 = (int64_t)b * B, nk = 0;
                    double m = -INFINITY;
                    for (int64_t j = j0; j < j0 + B && j <= p; ++j, ++nk) {
                        const double *kk = K + j * d;
                        double s = 0.0;
                        for (int c = 0; c < d; ++c) s += qq[c] * kk[c];
                        logit[nk] = s * scale;
                        if (logit[nk] > m) m = logit[nk];
                    }
                    double l = 0.0;
                    for (int64_t a = 0; a < nk; ++a) { logit[a] = exp(logit[a] - m); l += logit[a]; }
                    for (int64_t a = 0; a < nk; ++a) {
                        const double w = logit[a] / l;
                        const double *vv = V + (j0 + a) * d;
                        for (int c = 0; c < d; ++c) o[c] += w * vv[c];
                    }
                    *L = m + log(l);
                }
            }
        }
        free(logit);
    }
}

/* Log-sum-exp merge of per-block partials (not on the pages; it is the identity
 * softmax over a union of disjoint key sets = lse-weighted mix of the parts):
 *   Lt = log sum_i exp(lse_i);  out = sum_i exp(lse_i - Lt) * Op_i.
 * Slots with lse = -inf contribute nothing.  Shapes as in the partials. */
void orc_lse_merge(int d, int G, int k, int64_t nrows, const double *lse,
                   const double *Op, double *out)
{
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < nrows; ++r) {
        for (int h = 0; h < G; ++h) {
            double m = -INFINITY;
            for (int i = 0; i < k; ++i) {
                double L = lse[(r * k + i) * G + h];
                if (L > m) m = L;
            }
            double tot = 0.0;
            for (int i = 0; i < k; ++i) {
                double L = lse[(r * k + i) * G + h];
                if (L != -INFINITY) tot += exp(L - m);
            }
            const double Lt = m + log(tot);
            double *o = out + (r * G + h) * d;
            for (int c = 0; c < d; ++c) o[c] = 0.0;
            for (int i = 0; i < k; ++i) {
                double L = lse[(r * k + i) * G + h];
                if (L == -INFINITY) continue;
                const double w = exp(L - Lt);
                const double *src = Op + ((r * k + i) * G + h) * d;
                for (int c = 0; c < d; ++c) o[c] += w * src[c];
            }
        }
    }
}

/* ------------------------------------------------------------------ training
 * [P1 索引分支训练：KL 对齐: the index branch learns from the main branch's attention
 *  distribution through a KL divergence, and the training signal updates only the index
 *  branch (the teacher is cut from the gradient); P3 MSA entry: a KL loss
 *  pulls the index distribution toward the main branch probabilities, teacher stop-gradient]
 * Readings where the pages are silent (also in the design notes):
 *   - teacher of row r = the main branch's attention mass on each selected block,
 *     averaged over the G heads of the group (L1-normalised over the selection);
 *   - student = softmax over the same selected blocks of sigma * block score;
 *   - loss per row = KL(teacher || student); gradients are of the sum of row losses;
 *   - the max-pool passes the gradient of a block score to its arg-max key, the lowest
 *     position among equal maxima. */

/* The main branch of orc_attention, also returning for each row and head the
 * natural-log normaliser lse[r,h] = log sum_{j in J} exp(scale q.K_j), and for each
 * selected slot the teacher mass[r,i] = (1/G) sum_h sum_{j in block sel[r][i], j <= pos}
 * softmax_j (0 for a -1 slot).  lse is [nrows, G]; mass is [nrows, k]. */
void orc_attention_train(int64_t N, int B, int d, int G, int k, int64_t nrows,
                         const double *q, const int64_t *pos, const int32_t *sel,
                         const double *K, const double *V, double scale, double *out,
                         double *lse, double *mass)
{
    (void)N;
#pragma omp parallel
    {
        double *logit = (double *)malloc(sizeof(double) * (size_t)k * (size_t)B);
        int64_t *key = (int64_t *)malloc(sizeof(int64_t) * (size_t)k * (size_t)B);
        int *slot = (int *)malloc(sizeof(int) * (size_t)k * (size_t)B);
#pragma omp for schedule(dynamic, 1)
        for (int64_t r = 0; r < nrows; ++r) {
            const int64_t p = pos[r];
            int64_t nk = 0;
            for (int i = 0; i < k; ++i) {
                mass[r * k + i] = 0.0;
                int32_t b = sel[r * k + i];
                if (b < 0) continue;
                for (int64_t j = (int64_t)b * B; j < ((int64_t)b + 1) * B && j <= p; ++j) {
                    key[nk] = j;
                    slot[nk++] = i;
                }
            }
            for (int h = 0; h < G; ++h) {
                const double *qq = q + (r * G + h) * d;
                double m = -INFINITY;
                for (int64_t a = 0; a < nk; ++a) {
                    const double *kk = K + key[a] * d;
                    double s = 0.0;
                    for (int c = 0; c < d; ++c) s += qq[c] * kk[c];
                    logit[a] = s * scale;
                    if (logit[a] > m) m = logit[a];
                }
                double l = 0.0;
                for (int64_t a = 0; a < nk; ++a) { logit[a] = exp(logit[a] - m); l += logit[a]; }
                lse[r * G + h] = m + log(l);
                double *o = out + (r * G + h) * d;
                for (int c = 0; c < d; ++c) o[c] = 0.0;
                for (int64_t a = 0; a < nk; ++a) {
                    const double w = logit[a] / l;
                    const double *vv = V + key[a] * d;
                    for (int c = 0; c < d; ++c) o[c] += w * vv[c];
                    mass[r * k + slot[a]] += w / G;
                }
            }
        }
        free(logit);
        free(key);
        free(slot);
    }
}

/* Gradients of the main branch: with out as in orc_attention and an upstream gradient
 * dout [nrows, G, d], the gradients of sum_{r,h} dout[r,h,:] . out[r,h,:] with respect to
 * q [nrows, G, d], K [N, d] and V [N, d] (chain rule through the softmax):
 *   P_j = softmax_j(scale q.K_j) over J,   dP_j = dout . V_j,   D = sum_j P_j dP_j,
 *   dS_j = P_j (dP_j - D),   dq += scale sum_j dS_j K_j,
 *   dK_j += scale dS_j q,    dV_j += P_j dout.
 * dq, dK, dV are overwritten.  Serial (the K/V gradients accumulate across rows). */
void orc_attention_backward(int64_t N, int B, int d, int G, int k, int64_t nrows,
                            const double *q, const int64_t *pos, const int32_t *sel,
                            const double *K, const double *V, double scale, const double *dout,
                            double *dq, double *dK, double *dV)
{
    memset(dq, 0, sizeof(double) * (size_t)nrows * (size_t)G * (size_t)d);
    memset(dK, 0, sizeof(double) * (size_t)N * (size_t)d);
    memset(dV, 0, sizeof(double) * (size_t)N * (size_t)d);
    double *P = (double *)malloc(sizeof(double) * (size_t)k * (size_t)B);
    double *dP = (double *)malloc(sizeof(double) * (size_t)k * (size_t)B);
    int64_t *key = (int64_t *)malloc(sizeof(int64_t) * (size_t)k * (size_t)B);
    for (int64_t r = 0; r < nrows; ++r) {
        const int64_t p = pos[r];
        int64_t nk = 0;
        for (int i = 0; i < k; ++i) {
            int32_t b = sel[r * k + i];
            if (b < 0) continue;
            for (int64_t j = (int64_t)b * B; j < ((int64_t)b + 1) * B && j <= p; ++j) key[nk++] = j;
        }
        for (int h = 0; h < G; ++h) {
            const double *qq = q + (r * G + h) * d;
            const double *go = dout + (r * G + h) * d;
            double m = -INFINITY;
            for (int64_t a = 0; a < nk; ++a) {
                const double *kk = K + key[a] * d;
                double s = 0.0;
                for (int c = 0; c < d; ++c) s += qq[c] * kk[c];
                P[a] = s * scale;
                if (P[a] > m) m = P[a];
            }
            double l = 0.0;
            for (int64_t a = 0; a < nk; ++a) { P[a] = exp(P[a] - m); l += P[a]; }
            double D = 0.0;
            for (int64_t a = 0; a < nk; ++a) {
                P[a] /= l;
                const double *vv = V + key[a] * d;
                double t = 0.0;
                for (int c = 0; c < d; ++c) t += go[c] * vv[c];
                dP[a] = t;
                D += P[a] * t;
            }
            double *gq = dq + (r * G + h) * d;
            for (int64_t a = 0; a < nk; ++a) {
                const double dS = P[a] * (dP[a] - D);
                const double *kk = K + key[a] * d;
                double *gk = dK + key[a] * d;
                double *gv = dV + key[a] * d;
                for (int c = 0; c < d; ++c) {
                    gq[c] += scale * dS * kk[c];
                    gk[c] += scale * dS * qq[c];
                    gv[c] += P[a] * go[c];
                }
            }
        }
    }
    free(P);
    free(dP);
    free(key);
}

/* KL alignment of the index branch, one row at a time.  scores are the block scores
 * [nrows, nb] of orc_index_scores, mass the teacher [nrows, k] of orc_attention_train.
 * Over the valid slots i of row r (sel >= 0):
 *   pT_i = mass_i / sum mass,   pS_i = softmax_i(sigma * scores[r, sel[r][i]]),
 *   loss[r] = sum_i pT_i (log pT_i - log pS_i)   (a term with pT_i = 0 is 0),
 *   dscore[r,i] = d loss[r] / d scores[r, sel[r][i]] = sigma (pS_i - pT_i)  (teacher fixed);
 * dscore is 0 for -1 slots. */
void orc_index_kl(int64_t nb, int k, int64_t nrows, const double *scores, const int32_t *sel,
                  const double *mass, double sigma, double *loss, double *dscore)
{
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < nrows; ++r) {
        double m = -INFINITY, tm = 0.0;
        for (int i = 0; i < k; ++i) {
            const int32_t b = sel[r * k + i];
            if (b < 0) continue;
            const double z = sigma * scores[r * nb + b];
            if (z > m) m = z;
            tm += mass[r * k + i];
        }
        double l = 0.0;
        for (int i = 0; i < k; ++i) {
            const int32_t b = sel[r * k + i];
            if (b >= 0) l += exp(sigma * scores[r * nb + b] - m);
        }
        const double logl = log(l);
        double L = 0.0;
        for (int i = 0; i < k; ++i) {
            const int32_t b = sel[r * k + i];
            dscore[r * k + i] = 0.0;
            if (b < 0) continue;
            const double logpS = sigma * scores[r * nb + b] - m - logl;
            const double pT = mass[r * k + i] / tm;
            if (pT > 0.0) L += pT * (log(pT) - logpS);
            dscore[r * k + i] = sigma * (exp(logpS) - pT);
        }
        loss[r] = L;
    }
}

/* Index-branch input gradients through the causal block max-pool.  For each row r and
 * valid slot i (block b = sel[r][i]): j* = the lowest position j in [bB, min((b+1)B-1,
 * pos[r])] with the largest q_I[r] . k_I[j]; then dqI[r] += dscore[r,i] k_I[j*] and
 * dKI[j*] += dscore[r,i] q_I[r].  qI is [nrows, dI], KI [N, dI]; dqI, dKI overwritten.
 * Serial (the key gradients accumulate across rows). */
void orc_index_backward(int64_t N, int B, int dI, int k, int64_t nrows, const double *qI,
                        const int64_t *pos, const int32_t *sel, const double *KI,
                        const double *dscore, double *dqI, double *dKI)
{
    memset(dqI, 0, sizeof(double) * (size_t)nrows * (size_t)dI);
    memset(dKI, 0, sizeof(double) * (size_t)N * (size_t)dI);
    for (int64_t r = 0; r < nrows; ++r) {
        const double *qq = qI + r * dI;
        for (int i = 0; i < k; ++i) {
            const int32_t b = sel[r * k + i];
            if (b < 0) continue;
            int64_t best_j = -1;
            double best = -INFINITY;
            for (int64_t j = (int64_t)b * B; j < ((int64_t)b + 1) * B && j <= pos[r]; ++j) {
                double s = 0.0;
                for (int c = 0; c < dI; ++c) s += qq[c] * KI[j * dI + c];
                if (best_j < 0 || s > best) { best = s; best_j = j; }
            }
            if (best_j < 0) continue;
            const double g = dscore[r * k + i];
            for (int c = 0; c < dI; ++c) {
                dqI[r * dI + c] += g * KI[best_j * dI + c];
                dKI[best_j * dI + c] += g * qq[c];
            }
        }
    }
}

/* The arg-max of the max-pool where several keys may be correct: for each row r and valid
 * slot i, jbest[r,i] / best[r,i] = the lowest position holding the largest score in the
 * block (double) and that score, and cand_val[r,i] = the score at position cand[r,i]
 * (NaN if that position is outside the block's causal range).  -1 slots: jbest = -1. */
void orc_index_argmax(int64_t N, int B, int dI, int k, int64_t nrows, const double *qI,
                      const int64_t *pos, const int32_t *sel, const double *KI, const int64_t *cand,
                      int64_t *jbest, double *best, double *cand_val)
{
    (void)N;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < nrows; ++r) {
        const double *qq = qI + r * dI;
        for (int i = 0; i < k; ++i) {
            const int64_t o = r * k + i;
            const int32_t b = sel[o];
            jbest[o] = -1;
            best[o] = -INFINITY;
            cand_val[o] = NAN;
            if (b < 0) continue;
            for (int64_t j = (int64_t)b * B; j < ((int64_t)b + 1) * B && j <= pos[r]; ++j) {
                double s = 0.0;
                for (int c = 0; c < dI; ++c) s += qq[c] * KI[j * dI + c];
                if (jbest[o] < 0 || s > best[o]) { best[o] = s; jbest[o] = j; }
                if (cand != NULL && j == cand[o]) cand_val[o] = s;
            }
        }
    }
}

/* The scatter of orc_index_backward for given arg-max positions j[r,i] (-1 = none):
 * dqI[r] += dscore[r,i] k_I[j], dKI[j] += dscore[r,i] q_I[r].  Serial. */
void orc_index_backward_at(int64_t N, int dI, int k, int64_t nrows, const double *qI,
                           const int64_t *jstar, const double *KI, const double *dscore,
                           double *dqI, double *dKI)
{
    memset(dqI, 0, sizeof(double) * (size_t)nrows * (size_t)dI);
    memset(dKI, 0, sizeof(double) * (size_t)N * (size_t)dI);
    for (int64_t r = 0; r < nrows; ++r)
        for (int i = 0; i < k; ++i) {
            const int64_t j = jstar[r * k + i];
            if (j < 0) continue;
            const double g = dscore[r * k + i];
            for (int c = 0; c < dI; ++c) {
                dqI[r * dI + c] += g * KI[j * dI + c];
                dKI[j * dI + c] += g * qI[r * dI + c];
            }
        }
}

/* ------------------------------------------------------------------ token level
 * [P1 分歧一：颗粒度: DSA picks 2048 single tokens per query where MSA picks 16 blocks
 *  of 128 -- the same budget; P3 DSA entry: the lightning indexer scores every earlier
 *  token and the top-k single tokens are kept.]  Token scores are orc_index_scores with
 *  block size 1, token attention is orc_attention with block size 1; the selection differs:
 *  no token is forced (reading: the pages name no forced rule for token-level selection).
 * For each row r: the `budget` positions j <= pos[r] with the largest scores, ordered by
 * (score desc, position asc), emitted in ascending position order; when fewer than budget
 * positions are eligible all are taken; -1 pads.  scores is [nrows, N] (entries j > pos
 * are not read); out is [nrows, budget]. */
void orc_token_topk(int64_t N, int budget, int64_t nrows, const double *scores,
                    const int64_t *pos, int32_t *out)
{
#pragma omp parallel
    {
        unsigned char *taken = (unsigned char *)malloc((size_t)N);
#pragma omp for schedule(dynamic, 1)
        for (int64_t r = 0; r < nrows; ++r) {
            const double *sc = scores + r * N;
            const int64_t n = pos[r] + 1;
            memset(taken, 0, (size_t)N);
            const int64_t want = n < budget ? n : budget;
            for (int64_t c = 0; c < want; ++c) {      /* repeated arg-max, lower position on ties */
                int64_t best = -1;
                for (int64_t j = 0; j < n; ++j)
                    if (!taken[j] && (best < 0 || sc[j] > sc[best])) best = j;
                taken[best] = 1;
            }
            int32_t *o = out + r * budget;
            int64_t w = 0;
            for (int64_t j = 0; j < n; ++j)
                if (taken[j]) o[w++] = (int32_t)j;
            for (; w < budget; ++w) o[w] = -1;
        }
        free(taken);
    }
}

/* Threads OpenMP will use for the parallel loops above (reported beside timings). */
#ifdef _OPENMP
#include <omp.h>
int orc_num_threads(void) { return omp_get_max_threads(); }
#else
int orc_num_threads(void) { return 1; }
#endif
