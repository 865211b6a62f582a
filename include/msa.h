/*
 * msa.h -- C ABI of libmsa.so: MiniMax Sparse Attention (MSA) on one MI355X.
 *
 * MSA, as the pages describe it, runs in two stages: a light index branch
 * scores the KV cache in blocks of Bk = 128 tokens and keeps the top k = 16
 * blocks per query and GQA KV group; then dense attention runs over the real
 * (uncompressed) K/V of just those blocks.  Sources, by page and section:
 *   [aivizor]     edge.aivizor.me news item on the MiniMax M3 serving report --
 *                 the paragraphs on the two MSA stages, on the KV-Block-Major
 *                 sparse-attention kernel (outer loop over KV blocks, partial
 *                 outputs, final Log-Sum-Exp reduction) and on MSA with paged
 *                 attention in decode (page table from the selected blocks,
 *                 KV-group dimension flattened into the batch).
 *   [youmind]     "MiniMax M3: Como la atencion dispersa hace practicos a los
 *                 agentes de largo alcance" -- MSA figure caption and the bullet
 *                 "Costo predecible a cualquier longitud" (Bk = 128, k = 16).
 *   [mechatronic] "MiniMax M3: MoE de 428B con 1M de contexto en Blackwell",
 *                 section on what makes M3 different (each KV block read once,
 *                 contiguously; attention on real KV).
 *   [despertar]   despertarmatinal.com page on MiniMax M2 and M3 -- the
 *                 paragraph on the multi-token prediction (MTP) modules used
 *                 for speculative decoding, and the section "MiniMax Sparse
 *                 Attention (MSA) y escalado subcuadratico entrante".
 * The pages do not give the scoring function.  This library fixes it as:
 * score(block) = max over the block's causally visible tokens of
 * q_idx . k_idx (idx_dim = 64, fp32 accumulation); blocks after the query's
 * own block are ineligible; the own block is always kept; ties go to the lower
 * block index.
 *
 * Conventions shared by every entry point
 *   - Every tensor pointer is a DEVICE pointer to contiguous row-major memory,
 *     16-byte aligned.  bf16 tensors are passed as raw 16-bit patterns.
 *   - The caller owns every buffer.  The library allocates nothing on the hot
 *     path and holds no mutable global state; calls on different streams with
 *     different buffers may run concurrently.
 *   - Each call only enqueues kernels on `stream` (a hipStream_t; NULL is the
 *     default stream) and returns without synchronising.
 *   - Host-side checks (dims, null or misaligned pointers, workspace size) run
 *     before any launch; on failure the call returns an error status, launches
 *     nothing and leaves outputs untouched.  A call with no work (num_seqs =
 *     0, or total_q = 0 for the calls that take it; msa_validate_inputs
 *     excepted) returns MSA_SUCCESS once dims and total_q pass, without
 *     looking at its pointers (they may be NULL) or launching anything.  The library never aborts, prints
 *     or throws.  Device-resident CONTENT (seq_lens, cu_q, block_table, sel,
 *     page_table, row_lens) is a precondition the caller guarantees: page
 *     indices in [0, num_pages), 1 <= seq_lens[s], 0 <= cu_q[s+1]-cu_q[s] <=
 *     seq_lens[s], block_table rows cover ceil(seq_lens[s]/Bk) blocks.
 *   - Same inputs give bit-identical outputs (no float atomics in results).
 *   - Sequences and positions: sequence s owns query tokens cu_q[s] ..
 *     cu_q[s+1]-1 (its n_s new tokens), which are the LAST n_s of its
 *     seq_lens[s] cache tokens: the i-th has absolute position
 *     p = seq_lens[s] - n_s + i and own block b_loc = p / Bk.  Their K, V and
 *     k_idx are already in the cache (msa_append_kv puts them there;
 *     msa_decode_step_append does so itself).  Decode is n_s = 1 for every
 *     sequence.
 *   - Token j of sequence s lives in page block_table[s][j / Bk], slot j % Bk.
 *   - Query head h belongs to KV group h / (H_q / H_kv).
 *   - Supported sizes: head_dim 128, idx_dim 64, block_size 128, topk 16,
 *     H_q / H_kv <= 16, num_idx_heads 1 or H_kv, max_blocks_per_seq <= 16384.
 *     Other values return MSA_ERROR_NOT_SUPPORTED.
 */
#ifndef MSA_H_
#define MSA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MSA_ABI_VERSION 1

typedef enum {
    MSA_SUCCESS = 0,
    MSA_ERROR_INVALID_VALUE = 1, /* a null/misaligned pointer or inconsistent dims */
    MSA_ERROR_NOT_SUPPORTED = 2, /* valid, but outside the sizes listed above */
    MSA_ERROR_WORKSPACE = 3,     /* workspace null or smaller than the size query */
    MSA_ERROR_LAUNCH = 4         /* the HIP runtime refused a launch */
} msa_status_t;

typedef struct {
    int32_t num_seqs;           /* B */
    int32_t num_q_heads;        /* H_q, a multiple of H_kv */
    int32_t num_kv_heads;       /* H_kv: KV groups */
    int32_t num_idx_heads;      /* H_idx: 1 = one index key per token shared by all
                                   groups; H_kv = one index key per token and group */
    int32_t head_dim;           /* D = 128 */
    int32_t idx_dim;            /* d = 64 */
    int32_t block_size;         /* Bk = 128 (also the page size) */
    int32_t topk;               /* k = 16 */
    int32_t max_blocks_per_seq; /* width of block_table and of scores */
    int32_t num_pages;          /* pages in the K/V/k_idx pools */
    float softmax_scale;        /* <= 0 selects 1/sqrt(head_dim) */
} msa_dims_t;

/*
 * Index-branch block scores ([aivizor] two-stage paragraph; [youmind] MSA
 * figure caption: the index branch scores the KV blocks).
 *   q_idx       [total_q, H_kv, 64]        bf16
 *   kidx_cache  [num_pages, H_idx, 128, 64] bf16
 *   block_table [B, max_blocks_per_seq]    int32
 *   seq_lens    [B] int32, cu_q [B+1] int32 (cu_q[0] = 0, cu_q[B] = total_q)
 *   scores      [total_q, H_kv, max_blocks_per_seq] fp32 (output)
 * scores[t,g,b] = max_{j in block b, j <= p} sum_i q_idx[t,g,i] * k_idx[j,i]
 * with fp32 accumulation, where k_idx comes from index head 0 (H_idx = 1) or
 * g (H_idx = H_kv); -inf for b > b_loc.  total_q = 0 is a no-op.
 */
msa_status_t msa_index_score(const msa_dims_t *dims, int32_t total_q, const uint16_t *q_idx,
                             const uint16_t *kidx_cache, const int32_t *block_table,
                             const int32_t *seq_lens, const int32_t *cu_q, float *scores,
                             void *stream);

/*
 * Top-k block selection per (query, KV group) ([youmind] bullet "Costo
 * predecible a cualquier longitud").  Candidates are blocks 0..b_loc; the own
 * block b_loc is always kept; the others rank by score, equal scores (with
 * -0.0 == +0.0) to the lower block index.  min(k, b_loc+1) blocks are kept.
 *   scores [total_q, H_kv, max_blocks_per_seq] fp32 (entries b > b_loc unread;
 *          NaN scores are a precondition violation)
 *   sel    [total_q, H_kv, k] int32 (output): kept blocks in ascending order,
 *          then -1 padding.
 */
msa_status_t msa_topk_blocks(const msa_dims_t *dims, int32_t total_q, const float *scores,
                             const int32_t *seq_lens, const int32_t *cu_q, int32_t *sel,
                             void *stream);

/*
 * Decode page table ([aivizor] paragraph on MSA with paged attention): the
 * KV-group dimension is flattened into the batch, row r = s*H_kv + g, and the
 * row's pages are the physical pages of its selected blocks.  Decode only:
 * one query per sequence, so sel is [B, H_kv, k] (total_q = B).
 *   page_table [B*H_kv, k] int32 (output): block_table[s][sel[s,g,i]], -1 pad
 *   row_lens   [B*H_kv]    int32 (output): (n_sel-1)*Bk + (p - Bk*b_loc + 1),
 *              p = seq_lens[s]-1: with an ascending selection the own, partial
 *              block is last, so the row reads as a contiguous sequence.
 */
msa_status_t msa_build_page_table(const msa_dims_t *dims, const int32_t *sel,
                                  const int32_t *block_table, const int32_t *seq_lens,
                                  int32_t *page_table, int32_t *row_lens, void *stream);

/*
 * Sparse decode attention over the flattened page table ([aivizor] paged-
 * attention paragraph).  Row r = s*H_kv + g holds the G = H_q/H_kv query heads
 * q[s, g*G .. g*G+G-1, :] and attends the first row_lens[r] tokens of pages
 * page_table[r][0..], group g of the K/V pools:
 *   out = softmax(scale * q K^T) V,  lse = scale-included natural-log LSE.
 *   q       [B, H_q, 128] bf16;  k_cache, v_cache [num_pages, H_kv, 128, 128] bf16
 *   out     [B, H_q, 128] bf16 (output, round-to-nearest-even)
 *   lse     [B, H_q] fp32 (output) or NULL
 *   workspace: at least msa_decode_workspace_size(dims) bytes of device
 *   memory, 256-byte aligned; no initial contents required.
 * 1 <= row_lens[r] <= k*Bk is a precondition.
 */
msa_status_t msa_sparse_attn_decode(const msa_dims_t *dims, const uint16_t *q,
                                    const uint16_t *k_cache, const uint16_t *v_cache,
                                    const int32_t *page_table, const int32_t *row_lens,
                                    uint16_t *out, float *lse, void *workspace,
                                    size_t workspace_bytes, void *stream);

/*
 * Sparse prefill attention, KV-block-major ([aivizor] KV-Block-Major
 * paragraph; [mechatronic]: each KV block read once, contiguously).  The
 * outer loop runs over (sequence, KV group, block) work items: the block's K
 * and V are staged once on chip and every (query, head) that selected the
 * block is attended against it, giving one partial (output, LSE) per
 * (query, head, selection slot); a Log-Sum-Exp reduction then merges each
 * query's partials.  The result equals softmax attention over the union of
 * the selected blocks' tokens, cut at the query position.
 *   q     [total_q, H_q, 128] bf16; sel [total_q, H_kv, k] int32 (ascending or
 *         not; -1 entries ignored; entries must be <= b_loc and unique)
 *   out   [total_q, H_q, 128] bf16 (output); lse [total_q, H_q] fp32 or NULL.
 *         A (query, group) row whose entries are all -1 attends no token:
 *         its heads get out = 0 and lse = -inf.
 *   workspace: at least msa_prefill_workspace_size(dims, total_q) bytes,
 *   256-byte aligned; no initial contents required.
 */
msa_status_t msa_sparse_attn_prefill(const msa_dims_t *dims, int32_t total_q, const uint16_t *q,
                                     const uint16_t *k_cache, const uint16_t *v_cache,
                                     const int32_t *block_table, const int32_t *seq_lens,
                                     const int32_t *cu_q, const int32_t *sel, uint16_t *out,
                                     float *lse, void *workspace, size_t workspace_bytes,
                                     void *stream);

/*
 * The whole decode layer-step in three launches (the fused form of the four
 * calls above; same results, bit for bit).  Scoring runs as in
 * msa_index_score (into the workspace, leaving the scores of blocks past each
 * row's own block unwritten, since the selection never reads them); then
 * every (row r = s*H_kv + g, page slot i) workgroup
 * makes the row's top-k selection itself from the block scores -- the same
 * deterministic rule as msa_topk_blocks -- maps its i-th selected block to a
 * physical page through block_table (the row's page table, built on chip:
 * [aivizor] paragraph on MSA with paged attention) and attends that page as
 * msa_sparse_attn_decode does; a final kernel merges each row's pages with
 * the Log-Sum-Exp rule.  One query per sequence (decode, p = seq_lens[s]-1).
 *   q_idx [B, H_kv, 64], q [B, H_q, 128]; caches, block_table, seq_lens as above
 *   out   [B, H_q, 128] bf16 (output); lse [B, H_q] fp32 or NULL
 *   sel   [B, H_kv, k] int32 (output, the selection) or NULL
 *   workspace: at least msa_decode_step_workspace_size(dims) bytes, 256-byte
 *   aligned; no initial contents required.
 */
msa_status_t msa_decode_step(const msa_dims_t *dims, const uint16_t *q_idx,
                             const uint16_t *kidx_cache, const uint16_t *q,
                             const uint16_t *k_cache, const uint16_t *v_cache,
                             const int32_t *block_table, const int32_t *seq_lens, uint16_t *out,
                             float *lse, int32_t *sel, void *workspace, size_t workspace_bytes,
                             void *stream);

/*
 * msa_decode_step for callers that cannot allocate device memory (code under
 * HIP graph capture, serving loops and harnesses that forbid allocation): the
 * same launches and results, bit for bit, with no workspace argument.  The
 * step's scratch (page partials, block scores, row lengths) is a fixed array
 * of MSA_STATIC_SCRATCH_BYTES inside the library, one per GPU, held from the
 * first call on that GPU until the process ends; the call itself allocates
 * nothing.  Arguments as msa_decode_step; the work runs on the GPU of
 * `stream`.
 *   Returns MSA_ERROR_WORKSPACE, launching nothing, when
 *   msa_decode_step_workspace_size(dims) exceeds MSA_STATIC_SCRATCH_BYTES.
 * Every call on one GPU uses that GPU's one array, which keeps the last call's
 * contents (no call depends on them): calls ordered on one stream are fine,
 * while calls that may overlap on one GPU (unordered streams) race and give
 * wrong results.
 */
#define MSA_STATIC_SCRATCH_BYTES (32u << 20)
msa_status_t msa_decode_step_noalloc(const msa_dims_t *dims, const uint16_t *q_idx,
                                     const uint16_t *kidx_cache, const uint16_t *q,
                                     const uint16_t *k_cache, const uint16_t *v_cache,
                                     const int32_t *block_table, const int32_t *seq_lens,
                                     uint16_t *out, float *lse, int32_t *sel, void *stream);

/*
 * A multi-query layer-step: a few query tokens per sequence, e.g. the draft
 * tokens of speculative decoding ([despertar] paragraph on the multi-token
 * prediction (MTP) modules used for speculative decoding), each KV block read
 * once for all of a sequence's drafts ([aivizor] KV-Block-Major paragraph).
 * Same results as msa_index_score,
 * msa_topk_blocks and msa_sparse_attn_prefill called in turn, bit for bit.
 *
 * With at most 4 queries per sequence on average, total_q x k <= 4096 and
 * max_blocks_per_seq <= 1024 it runs in three launches:
 *   - scoring, as msa_index_score;
 *   - one kernel whose (sequence, group) workgroups make the top-k selection
 *     of their sequence's queries from the scores (the rule of
 *     msa_topk_blocks), find the union of the selected blocks and attend
 *     each block once for every query that selected it;
 *   - the Log-Sum-Exp merge.
 * Otherwise it makes the three calls' own launches.
 *
 * Arguments:
 *   q_idx [total_q, H_kv, 64] and q [total_q, H_q, 128] bf16; caches,
 *         block_table, seq_lens, cu_q as for the prefill calls (query token t
 *         of sequence s at position seq_lens[s] - n_s + (t - cu_q[s]))
 *   out   [total_q, H_q, 128] bf16 (output); lse [total_q, H_q] fp32 or NULL
 *   sel   [total_q, H_kv, k] int32 (output, the selection) or NULL
 *   workspace: at least msa_multi_query_step_workspace_size(dims, total_q)
 *         bytes, 256-byte aligned; no initial contents required.
 */
msa_status_t msa_multi_query_step(const msa_dims_t *dims, int32_t total_q, const uint16_t *q_idx,
                                  const uint16_t *kidx_cache, const uint16_t *q,
                                  const uint16_t *k_cache, const uint16_t *v_cache,
                                  const int32_t *block_table, const int32_t *seq_lens,
                                  const int32_t *cu_q, uint16_t *out, float *lse, int32_t *sel,
                                  void *workspace, size_t workspace_bytes, void *stream);

/*
 * Dense GQA decode attention, the baseline MSA's decode speedup is measured/*
 * Dense GQA decode attention, the baseline MSA's decode speedup is measured
 * against ([youmind] bullet "Rapido en produccion": decode vs dense GQA with
 * the same heads): every query head of sequence s attends all seq_lens[s]
 * cached tokens of its KV group, softmax(scale * q K^T) V.  Same caches and
 * block table as the sparse path; one query per sequence at p = seq_lens[s]-1.
 *   q     [B, H_q, 128] bf16; k_cache, v_cache, block_table, seq_lens as above
 *   out   [B, H_q, 128] bf16 (output); lse [B, H_q] fp32 or NULL
 *   workspace: at least msa_dense_decode_workspace_size(dims) bytes, 256-byte
 *   aligned; no initial contents required.  seq_lens[s] >= 1.
 */
msa_status_t msa_dense_attn_decode(const msa_dims_t *dims, const uint16_t *q,
                                   const uint16_t *k_cache, const uint16_t *v_cache,
                                   const int32_t *block_table, const int32_t *seq_lens,
                                   uint16_t *out, float *lse, void *workspace,
                                   size_t workspace_bytes, void *stream);

/*
 * Dense causal prefill attention, the baseline MSA's prefill speedup is
 * measured against ([youmind] bullet "Rapido en produccion": prefill vs dense
 * GQA with the same heads): query token t of sequence s (position
 * p = seq_lens[s] - n_s + (t - cu_q[s])) attends every cached token j <= p of
 * its KV group, softmax(scale * q K^T) V.  Same caches, block table and
 * (cu_q, seq_lens) convention as msa_sparse_attn_prefill; no workspace.
 *   q     [total_q, H_q, 128] bf16
 *   out   [total_q, H_q, 128] bf16 (output); lse [total_q, H_q] fp32 or NULL
 */
msa_status_t msa_dense_attn_prefill(const msa_dims_t *dims, int32_t total_q, const uint16_t *q,
                                    const uint16_t *k_cache, const uint16_t *v_cache,
                                    const int32_t *block_table, const int32_t *seq_lens,
                                    const int32_t *cu_q, uint16_t *out, float *lse, void *stream);

/*
 * Cache append, the step before scoring ([aivizor] paragraph on MSA with paged
 * attention: the caches are paged by 128-token blocks): the i-th new token of
 * sequence s (query token t = cu_q[s] + i) sits at position
 * p = seq_lens[s] - n_s + i, i.e. page block_table[s][p / Bk], slot p % Bk,
 * and its rows are copied there -- the (cu_q, seq_lens) convention of
 * msa_sparse_attn_prefill, so decode is cu_q[s] = s.
 *   k_new, v_new [total_q, H_kv, 128] bf16; kidx_new [total_q, H_idx, 64] bf16
 *   k_cache, v_cache [num_pages, H_kv, 128, 128], kidx_cache
 *   [num_pages, H_idx, 128, 64] (updated in place: only the new tokens' slots
 *   are written)
 * The new tokens' slots must be distinct (no two tokens at one position).
 */
msa_status_t msa_append_kv(const msa_dims_t *dims, int32_t total_q, const uint16_t *k_new,
                           const uint16_t *v_new, const uint16_t *kidx_new,
                           const int32_t *block_table, const int32_t *seq_lens,
                           const int32_t *cu_q, uint16_t *k_cache, uint16_t *v_cache,
                           uint16_t *kidx_cache, void *stream);

/*
 * msa_append_kv followed by msa_decode_step, in the decode step's three
 * launches: the new token of each sequence (position seq_lens[s] - 1, so
 * seq_lens already counts it) is written into its page slot by the scoring
 * launch ([aivizor] paragraph on MSA with paged attention), which scores that
 * slot from the new index keys; the selection and attention launches then
 * read the updated caches.  Results and cache contents equal those of the two
 * calls, bit for bit.
 *   k_new, v_new [B, H_kv, 128] bf16; kidx_new [B, H_idx, 64] bf16
 *   k_cache, v_cache, kidx_cache: updated in place (only the new slots)
 *   the other arguments as msa_decode_step (same workspace size)
 * The new slots must be distinct; k_new, v_new and kidx_new must not overlap
 * the caches; and a page that receives a new token must not appear in another
 * sequence's block table in the same call (it is written while the other
 * sequences' blocks are scored: a shared prefix page must be copied first).
 */
msa_status_t msa_decode_step_append(const msa_dims_t *dims, const uint16_t *k_new,
                                    const uint16_t *v_new, const uint16_t *kidx_new,
                                    const uint16_t *q_idx, uint16_t *kidx_cache,
                                    const uint16_t *q, uint16_t *k_cache, uint16_t *v_cache,
                                    const int32_t *block_table, const int32_t *seq_lens,
                                    uint16_t *out, float *lse, int32_t *sel, void *workspace,
                                    size_t workspace_bytes, void *stream);

/*
 * Device-side check of the content preconditions listed at the top of this
 * file, for callers that want them verified (not a hot-path call): for every
 * sequence s, 1 <= seq_lens[s] <= max_blocks_per_seq*Bk; with cu_q,
 * cu_q[0] = 0, cu_q[B] = total_q and 0 <= cu_q[s+1]-cu_q[s] <= seq_lens[s];
 * block_table[s][b] in [0, num_pages) for b < ceil(seq_lens[s]/Bk).
 *   cu_q   [B+1] or NULL (decode: one query per sequence; total_q ignored)
 *   status one int32 in device memory (output): 0, or the OR of the
 *          msa_input_fault_t bits found, written on `stream`.
 * It reads only within the arrays' declared sizes, whatever their content.
 */
typedef enum {
    MSA_FAULT_SEQ_LEN = 1,     /* a sequence length below 1 or past the block table */
    MSA_FAULT_CU_Q = 2,        /* query ranges not within [0, total_q] or longer than L */
    MSA_FAULT_BLOCK_TABLE = 4  /* a used block-table entry outside [0, num_pages) */
} msa_input_fault_t;
msa_status_t msa_validate_inputs(const msa_dims_t *dims, int32_t total_q,
                                 const int32_t *block_table, const int32_t *seq_lens,
                                 const int32_t *cu_q, int32_t *status, void *stream);

/* Workspace sizes in bytes (0 for invalid dims). */
size_t msa_decode_workspace_size(const msa_dims_t *dims);
size_t msa_prefill_workspace_size(const msa_dims_t *dims, int32_t total_q);
size_t msa_decode_step_workspace_size(const msa_dims_t *dims);
size_t msa_multi_query_step_workspace_size(const msa_dims_t *dims, int32_t total_q);
size_t msa_dense_decode_workspace_size(const msa_dims_t *dims);

/* Static, human-readable name of a status code. */
const char *msa_status_string(msa_status_t status);

/* MSA_ABI_VERSION of the loaded library. */
int msa_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MSA_H_ */
