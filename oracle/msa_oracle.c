/*
 * msa_oracle.c -- plain, slow fp64 CPU oracle for MiniMax Sparse Attention (MSA).
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, the smoke check in __graft_entry__.py
 * and the cpu_baseline leg of bench.py may load this library.  It shares no
 * code, header, table or helper with the HIP library under
 * block_sparse_attention_03_amd/csrc, and the HIP library never calls it.
 *
 * What it computes (sources, cited by page and section):
 *   [aivizor]   edge.aivizor.me news item on the MiniMax M3 serving report:
 *               the paragraph on the two MSA stages, the paragraph on the
 *               KV-Block-Major kernel (partial outputs + Log-Sum-Exp reduction)
 *               and the paragraph on MSA with paged attention in decode.
 *   [youmind]   "MiniMax M3: Como la atencion dispersa hace practicos a los
 *               agentes de largo alcance": the MSA figure caption (index branch
 *               scores KV blocks, top-k per query group) and the bullet
 *               "Costo predecible a cualquier longitud" (Bk = 128, k = 16,
 *               2048 tokens per query and GQA group).
 *   [mechatronic] "MiniMax M3: MoE de 428B con 1M de contexto en Blackwell",
 *               section "Que hace tan distinto al MiniMax M3?": attention runs
 *               on the real, uncompressed KV of the selected blocks.
 * The pages never give the scoring function.  The reading used here (and by
 * the HIP library) is: score(block) = max over the block's causally visible
 * tokens of the dot product q_idx . k_idx, idx_dim = 64; blocks after the
 * query's own block are ineligible; the query's own block is always selected;
 * ties go to the lower block index.
 *
 * Everything is computed in double precision from the exact bf16 values, with
 * plain loops in the order the definition states.  The only parallelism is an
 * OpenMP loop over independent output rows.
 *
 * Tensor layouts (all row-major, bf16 passed as raw uint16 bits):
 *   q_idx      [T, H_kv, d]          index query, one per (token, KV group)
 *   kidx_cache [P, H_idx, Bk, d]     index keys, H_idx = 1 (shared) or H_kv
 *   q          [T, H_q, D]
 *   k_cache    [P, H_kv, Bk, D]      v_cache same
 *   block_table[B, maxblk]           logical block -> physical page
 *   seq_lens   [B]                   tokens in the cache, new ones included
 *   cu_q       [B+1]                 query tokens of seq s: cu_q[s]..cu_q[s+1]-1
 * Query head h belongs to KV group h / (H_q / H_kv).
 *
 * Parity pins: scores, selection and attention are pinned in
 * tests/test_oracle.py against integer-exact brute force, an exhaustive subset
 * search, torch's scaled_dot_product_attention and closed forms.  No function
 * here is parity-unpinned.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static double bf16_to_double(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

int msa_oracle_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * Absolute position of every query token.  The n_s new tokens of sequence s
 * are the last n_s tokens of its cache, so token i of them sits at
 * p = L_s - n_s + i (in decode n_s = 1 and p = L_s - 1).
 * Returns 0, or -1 when a sequence has more queries than cache tokens.
 */
int msa_oracle_positions(int B, const int32_t *seq_lens, const int32_t *cu_q,
                         int32_t *seq_of, int32_t *pos_of)
{
    for (int s = 0; s < B; ++s) {
        int n = cu_q[s + 1] - cu_q[s];
        int L = seq_lens[s];
        if (n < 0 || n > L)
            return -1;
        for (int i = 0; i < n; ++i) {
            seq_of[cu_q[s] + i] = s;
            pos_of[cu_q[s] + i] = L - n + i;
        }
    }
    return 0;
}

/*
 * Index-branch block scores ([aivizor] two-stage paragraph, [youmind] MSA
 * figure caption).  For output row r = t*H_kv + g and block b:
 *   score = max_{j in block b, j <= p} sum_i q_idx[t,g,i] * k_idx[s, j, i]
 * and -inf for blocks after the query's own block b_loc = p / Bk.
 * Token j of sequence s lives in page block_table[s][j / Bk], slot j % Bk.
 * rows == NULL means all T*H_kv rows in order; scores is [n_rows, maxblk].
 */
void msa_oracle_index_score(int T, int H_kv, int H_idx, int d, int Bk, int maxblk,
                            const uint16_t *q_idx, const uint16_t *kidx_cache,
                            const int32_t *block_table, const int32_t *seq_of,
                            const int32_t *pos_of, long n_rows, const int64_t *rows,
                            double *scores)
{
    (void)T;
#pragma omp parallel for schedule(dynamic, 4)
    for (long r = 0; r < n_rows; ++r) {
        long row = rows ? (long)rows[r] : r;
        long t = row / H_kv;
        int g = (int)(row % H_kv);
        int s = seq_of[t];
        long p = pos_of[t];
        int ih = (H_idx == 1) ? 0 : g;
        long b_loc = p / Bk;
        const uint16_t *qv = q_idx + ((long)t * H_kv + g) * d;
        double *out = scores + r * (long)maxblk;
        for (long b = 0; b < maxblk; ++b) {
            if (b > b_loc) {
                out[b] = -INFINITY;
                continue;
            }
            long page = block_table[(long)s * maxblk + b];
            long j_end = (b + 1) * (long)Bk;
            if (j_end > p + 1)
                j_end = p + 1;
            double best = -INFINITY;
            for (long j = b * (long)Bk; j < j_end; ++j) {
                const uint16_t *kv =
                    kidx_cache + ((page * H_idx + ih) * (long)Bk + (j - b * (long)Bk)) * d;
                double dot = 0.0;
                for (int i = 0; i < d; ++i)
                    dot += bf16_to_double(qv[i]) * bf16_to_double(kv[i]);
                if (dot > best)
                    best = dot;
            }
            out[b] = best;
        }
    }
}

/* Ordering for selection: larger key first, lower block index on equal keys.
 * Keys are compared by value, so -0.0 and +0.0 are equal. */
typedef struct {
    double key;
    int32_t idx;
} cand_t;

static int cand_desc(const void *a, const void *b)
{
    const cand_t *x = (const cand_t *)a, *y = (const cand_t *)b;
    if (x->key > y->key)
        return -1;
    if (x->key < y->key)
        return 1;
    return (x->idx < y->idx) ? -1 : (x->idx > y->idx);
}

static int int_asc(const void *a, const void *b)
{
    int32_t x = *(const int32_t *)a, y = *(const int32_t *)b;
    return (x < y) ? -1 : (x > y);
}

/*
 * Top-k block selection ([youmind] bullet "Costo predecible a cualquier
 * longitud": k blocks per query and GQA group).  Candidates are blocks
 * 0..b_loc of the row; the query's own block b_loc gets key +inf so it is
 * always kept; the rest are ranked by score, ties to the lower index.  The
 * first min(k, b_loc+1) are kept, written in ascending block order, and the
 * row is padded with -1 up to k.
 * scores is [n_rows, maxblk]; b_loc is per row; sel is [n_rows, k].
 */
void msa_oracle_topk(long n_rows, int maxblk, int k, const double *scores,
                     const int32_t *b_loc, int32_t *sel)
{
#pragma omp parallel
    {
        cand_t *c = (cand_t *)malloc(sizeof(cand_t) * (size_t)(maxblk > 0 ? maxblk : 1));
        int32_t *keep = (int32_t *)malloc(sizeof(int32_t) * (size_t)(k > 0 ? k : 1));
#pragma omp for schedule(dynamic, 16)
        for (long r = 0; r < n_rows; ++r) {
            int bl = b_loc[r];
            int n = bl + 1;
            const double *sc = scores + r * (long)maxblk;
            for (int b = 0; b < n; ++b) {
                c[b].key = (b == bl) ? INFINITY : sc[b];
                c[b].idx = b;
            }
            qsort(c, (size_t)n, sizeof(cand_t), cand_desc);
            int n_sel = n < k ? n : k;
            for (int i = 0; i < n_sel; ++i)
                keep[i] = c[i].idx;
            qsort(keep, (size_t)n_sel, sizeof(int32_t), int_asc);
            int32_t *o = sel + r * (long)k;
            for (int i = 0; i < k; ++i)
                o[i] = (i < n_sel) ? keep[i] : -1;
        }
        free(c);
        free(keep);
    }
}

/*
 * Sparse attention by its plain definition ([aivizor] two-stage paragraph,
 * [mechatronic] section on what makes M3 different: dense attention over the
 * real KV of the selected blocks).  For output row r = t*H_q + h, group
 * g = h / (H_q/H_kv), the token set is the union over selected blocks b of
 * [b*Bk, min((b+1)*Bk, p+1)).  With z_j = scale * q.K_j:
 *   m = max z, w_j = exp(z_j - m), l = sum w, out = sum w_j V_j / l,
 *   lse = m + ln l  (natural log, scale included).
 * A row with an empty token set gets out = 0 and lse = -inf.
 * sel is [T, H_kv, k] (-1 entries ignored); out is [n_rows, D], lse [n_rows].
 */
void msa_oracle_attention(int T, int H_q, int H_kv, int D, int Bk, int k, int maxblk,
                          double scale, const uint16_t *q, const uint16_t *k_cache,
                          const uint16_t *v_cache, const int32_t *block_table,
                          const int32_t *seq_of, const int32_t *pos_of,
                          const int32_t *sel, long n_rows, const int64_t *rows,
                          double *out, double *lse)
{
    (void)T;
    int G = H_q / H_kv;
#pragma omp parallel
    {
        /* token j of the sequence -> attended?  Built per row as a true union. */
        long cap = (long)k * Bk;
        long *tok = (long *)malloc(sizeof(long) * (size_t)cap);
        double *z = (double *)malloc(sizeof(double) * (size_t)cap);
#pragma omp for schedule(dynamic, 4)
        for (long r = 0; r < n_rows; ++r) {
            long row = rows ? (long)rows[r] : r;
            long t = row / H_q;
            int h = (int)(row % H_q);
            int g = h / G;
            int s = seq_of[t];
            long p = pos_of[t];
            const int32_t *sr = sel + ((long)t * H_kv + g) * k;
            long n = 0;
            for (int i = 0; i < k; ++i) {
                int b = sr[i];
                if (b < 0)
                    continue;
                int dup = 0;
                for (int i2 = 0; i2 < i; ++i2)
                    if (sr[i2] == b)
                        dup = 1;
                if (dup)
                    continue;
                long j_end = ((long)b + 1) * Bk;
                if (j_end > p + 1)
                    j_end = p + 1;
                for (long j = (long)b * Bk; j < j_end; ++j)
                    tok[n++] = j;
            }
            double *o = out + r * (long)D;
            for (int c = 0; c < D; ++c)
                o[c] = 0.0;
            if (n == 0) {
                lse[r] = -INFINITY;
                continue;
            }
            const uint16_t *qv = q + ((long)t * H_q + h) * D;
            double m = -INFINITY;
            for (long a = 0; a < n; ++a) {
                long j = tok[a];
                long page = block_table[(long)s * maxblk + j / Bk];
                const uint16_t *kv = k_cache + ((page * H_kv + g) * (long)Bk + j % Bk) * D;
                double dot = 0.0;
                for (int c = 0; c < D; ++c)
                    dot += bf16_to_double(qv[c]) * bf16_to_double(kv[c]);
                z[a] = scale * dot;
                if (z[a] > m)
                    m = z[a];
            }
            double l = 0.0;
            for (long a = 0; a < n; ++a) {
                long j = tok[a];
                long page = block_table[(long)s * maxblk + j / Bk];
                const uint16_t *vv = v_cache + ((page * H_kv + g) * (long)Bk + j % Bk) * D;
                double w = exp(z[a] - m);
                l += w;
                for (int c = 0; c < D; ++c)
                    o[c] += w * bf16_to_double(vv[c]);
            }
            for (int c = 0; c < D; ++c)
                o[c] /= l;
            lse[r] = m + log(l);
        }
        free(tok);
        free(z);
    }
}

/*
 * Decode page table ([aivizor] paragraph on MSA with paged attention): the
 * KV-group dimension is flattened into the batch, row r = s*H_kv + g, and the
 * row's pages are the physical pages of its selected blocks in selection
 * order.  With the selection ascending, the query's own (partial) block comes
 * last, so the row reads like an ordinary contiguous sequence of
 *   row_len = (n_sel - 1) * Bk + (p - Bk*b_loc + 1)
 * tokens, p = L_s - 1.  Unused entries are -1.
 * sel is [B, H_kv, k]; page_table [B*H_kv, k]; row_lens [B*H_kv].
 */
void msa_oracle_page_table(int B, int H_kv, int k, int Bk, int maxblk,
                           const int32_t *sel, const int32_t *block_table,
                           const int32_t *seq_lens, int32_t *page_table,
                           int32_t *row_lens)
{
    for (int s = 0; s < B; ++s) {
        long p = (long)seq_lens[s] - 1;
        long b_loc = p / Bk;
        for (int g = 0; g < H_kv; ++g) {
            long r = (long)s * H_kv + g;
            const int32_t *sr = sel + r * k;
            int n_sel = 0;
            for (int i = 0; i < k; ++i) {
                int b = sr[i];
                page_table[r * k + i] = (b >= 0) ? block_table[(long)s * maxblk + b] : -1;
                if (b >= 0)
                    ++n_sel;
            }
            row_lens[r] = (int32_t)((long)(n_sel - 1) * Bk + (p - (long)Bk * b_loc + 1));
        }
    }
}

/*
 * Ordinary fixed-page attention over a flattened batch, the form the decode
 * page table feeds ([aivizor] paged-attention paragraph).  Row r has G query
 * heads q[r*G .. r*G+G-1] (= q[B, H_q, D] viewed as [B*H_kv, G, D]) and reads
 * group g = r % H_kv of pages page_table[r][i / Bk], slot i % Bk, for tokens
 * i < row_lens[r].  out is [R*G, D], lse [R*G].
 */
void msa_oracle_paged_attention(int R, int G, int H_kv, int D, int Bk, int pt_width,
                                double scale, const uint16_t *q, const uint16_t *k_cache,
                                const uint16_t *v_cache, const int32_t *page_table,
                                const int32_t *row_lens, double *out, double *lse)
{
#pragma omp parallel for schedule(dynamic, 1)
    for (long rh = 0; rh < (long)R * G; ++rh) {
        long r = rh / G;
        int g = (int)(r % H_kv);
        long n = row_lens[r];
        const uint16_t *qv = q + rh * D;
        double *o = out + rh * D;
        for (int c = 0; c < D; ++c)
            o[c] = 0.0;
        if (n <= 0) {
            lse[rh] = -INFINITY;
            continue;
        }
        double *z = (double *)malloc(sizeof(double) * (size_t)n);
        double m = -INFINITY;
        for (long i = 0; i < n; ++i) {
            long page = page_table[r * pt_width + i / Bk];
            const uint16_t *kv = k_cache + ((page * H_kv + g) * (long)Bk + i % Bk) * D;
            double dot = 0.0;
            for (int c = 0; c < D; ++c)
                dot += bf16_to_double(qv[c]) * bf16_to_double(kv[c]);
            z[i] = scale * dot;
            if (z[i] > m)
                m = z[i];
        }
        double l = 0.0;
        for (long i = 0; i < n; ++i) {
            long page = page_table[r * pt_width + i / Bk];
            const uint16_t *vv = v_cache + ((page * H_kv + g) * (long)Bk + i % Bk) * D;
            double w = exp(z[i] - m);
            l += w;
            for (int c = 0; c < D; ++c)
                o[c] += w * bf16_to_double(vv[c]);
        }
        for (int c = 0; c < D; ++c)
            o[c] /= l;
        lse[rh] = m + log(l);
        free(z);
    }
}

/*
 * Log-Sum-Exp reduction of partial results ([aivizor] KV-Block-Major
 * paragraph): parts (o_i, lse_i) computed over disjoint token sets combine
 * into the result over their union as
 *   lse = ln sum_i exp(lse_i),  o = sum_i exp(lse_i - lse) * o_i.
 * Parts with lse_i = -inf are empty and contribute nothing.
 * o_parts [n, parts, D], lse_parts [n, parts] -> o [n, D], lse [n].
 */
void msa_oracle_lse_merge(long n, int parts, int D, const double *o_parts,
                          const double *lse_parts, double *o, double *lse)
{
    for (long r = 0; r < n; ++r) {
        const double *lp = lse_parts + r * parts;
        double mx = -INFINITY;
        for (int i = 0; i < parts; ++i)
            if (lp[i] > mx)
                mx = lp[i];
        double *orow = o + r * D;
        for (int c = 0; c < D; ++c)
            orow[c] = 0.0;
        if (mx == -INFINITY) {
            lse[r] = -INFINITY;
            continue;
        }
        double sum = 0.0;
        for (int i = 0; i < parts; ++i)
            sum += exp(lp[i] - mx);
        double total = mx + log(sum);
        for (int i = 0; i < parts; ++i) {
            if (lp[i] == -INFINITY)
                continue;
            double w = exp(lp[i] - total);
            const double *op = o_parts + (r * parts + i) * (long)D;
            for (int c = 0; c < D; ++c)
                orow[c] += w * op[c];
        }
        lse[r] = total;
    }
}
