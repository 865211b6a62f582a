// msa_api.cpp -- host side of libmsa.so: argument checks and kernel launches
// behind the C ABI declared in include/msa.h.  No allocation, no global
// mutable state, no synchronisation: every call validates its scalars and
// pointers, then enqueues kernels on the caller's stream.
#include <cmath>
#include <cstdint>

#include "../../include/msa.h"
#include "msa_common.hpp"

namespace {

constexpr int kMaxBlocks = 16384;  // widest block_table / score row handled by top-k

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Validates the dims and fills the internal shape.  Returns MSA_SUCCESS or the
// status to report.
msa_status_t check_dims(const msa_dims_t* d, MsaShape* out) {
    if (!d) return MSA_ERROR_INVALID_VALUE;
    if (d->num_seqs < 0 || d->num_q_heads <= 0 || d->num_kv_heads <= 0 ||
        d->num_idx_heads <= 0 || d->max_blocks_per_seq <= 0 || d->num_pages <= 0)
        return MSA_ERROR_INVALID_VALUE;
    if (d->num_q_heads % d->num_kv_heads != 0) return MSA_ERROR_INVALID_VALUE;
    if (d->num_idx_heads != 1 && d->num_idx_heads != d->num_kv_heads) return MSA_ERROR_INVALID_VALUE;
    if (!(std::isfinite(d->softmax_scale))) return MSA_ERROR_INVALID_VALUE;
    if (d->head_dim != msa::kHeadDim || d->idx_dim != msa::kIdxDim ||
        d->block_size != msa::kBlock || d->topk != msa::kTopK)
        return MSA_ERROR_NOT_SUPPORTED;
    if (d->num_q_heads / d->num_kv_heads > msa::kMaxGroup) return MSA_ERROR_NOT_SUPPORTED;
    if (d->max_blocks_per_seq > kMaxBlocks) return MSA_ERROR_NOT_SUPPORTED;
    // grid-dimension and 32-bit index limits of the launches
    if ((int64_t)d->num_seqs * d->num_kv_heads > 65535) return MSA_ERROR_NOT_SUPPORTED;
    if ((int64_t)d->num_seqs * d->num_kv_heads * d->max_blocks_per_seq > INT32_MAX)
        return MSA_ERROR_NOT_SUPPORTED;
    out->B = d->num_seqs;
    out->Hq = d->num_q_heads;
    out->Hkv = d->num_kv_heads;
    out->Hidx = d->num_idx_heads;
    out->maxblk = d->max_blocks_per_seq;
    out->num_pages = d->num_pages;
    out->scale = d->softmax_scale > 0.f ? d->softmax_scale
                                        : 1.0f / std::sqrt(static_cast<float>(d->head_dim));
    return MSA_SUCCESS;
}

msa_status_t check_total_q(const MsaShape& s, int32_t total_q) {
    if (total_q < 0) return MSA_ERROR_INVALID_VALUE;
    // (query << 4 | slot) entries and 32-bit row counts
    if ((int64_t)total_q >= (1 << 27)) return MSA_ERROR_NOT_SUPPORTED;
    if ((int64_t)total_q * s.Hq * msa::kTopK > INT32_MAX) return MSA_ERROR_NOT_SUPPORTED;
    return MSA_SUCCESS;
}

msa_status_t launched(hipError_t e) { return e == hipSuccess ? MSA_SUCCESS : MSA_ERROR_LAUNCH; }

// Marks a decode step that runs in the library's static scratch: a tag
// compared by address, never dereferenced or passed to a kernel.
char g_static_scratch_tag;
void* const kStaticScratch = &g_static_scratch_tag;

}  // namespace

extern "C" {

msa_status_t msa_index_score(const msa_dims_t* dims, int32_t total_q, const uint16_t* q_idx,
                             const uint16_t* kidx_cache, const int32_t* block_table,
                             const int32_t* seq_lens, const int32_t* cu_q, float* scores,
                             void* stream) {
    MsaShape s;
    msa_status_t st = check_dims(dims, &s);
    if (st != MSA_SUCCESS) return st;
    if ((st = check_total_q(s, total_q)) != MSA_SUCCESS) return st;
    if (total_q == 0) return MSA_SUCCESS;  // no work: nothing read, nothing launched
    if (!q_idx || !kidx_cache || !block_table || !seq_lens || !cu_q || !scores)
        return MSA_ERROR_INVALID_VALUE;
    if (!aligned(q_idx, 16) || !aligned(kidx_cache, 16) || !aligned(block_table, 4) ||
        !aligned(seq_lens, 4) || !aligned(cu_q, 4) || !aligned(scores, 4))
        return MSA_ERROR_INVALID_VALUE;
    if ((int64_t)s.B * s.Hidx > 65535) return MSA_ERROR_NOT_SUPPORTED;
    return launched(msa_launch_index_score(s, total_q, q_idx, kidx_cache, block_table, seq_lens,
                                           cu_q, scores, static_cast<hipStream_t>(stream)));
}

msa_status_t msa_topk_blocks(const msa_dims_t* dims, int32_t total_q, const float* scores,
                             const int32_t* seq_lens, const int32_t* cu_q, int32_t* sel,
                             void* stream) {
    MsaShape s;
    msa_status_t st = check_dims(dims, &s);
    if (st != MSA_SUCCESS) return st;
    if ((st = check_total_q(s, total_q)) != MSA_SUCCESS) return st;
    if (total_q == 0) return MSA_SUCCESS;  // no work: nothing read, nothing launched
    if (!scores || !seq_lens || !cu_q || !sel) return MSA_ERROR_INVALID_VALUE;
    if (!aligned(scores, 4) || !aligned(seq_lens, 4) || !aligned(cu_q, 4) || !aligned(sel, 4))
        return MSA_ERROR_INVALID_VALUE;
    return launched(msa_launch_topk(s, total_q, scores, seq_lens, cu_q, sel,
                                    static_cast<hipStream_t>(stream)));
}

msa_status_t msa_build_page_table(const msa_dims_t* dims, const int32_t* sel,
                                  const int32_t* block_table, const int32_t* seq_lens,
                                  int32_t* page_table, int32_t* row_lens, void* stream) {
    MsaShape s;
    msa_status_t st = check_dims(dims, &s);
    if (st != MSA_SUCCESS) return st;
    if (s.B == 0) return MSA_SUCCESS;  // no work: nothing read, nothing launched
    if (!sel || !block_table || !seq_lens || !page_table || !row_lens) return MSA_ERROR_INVALID_VALUE;
    if (!aligned(sel, 4) || !aligned(block_table, 4) || !aligned(seq_lens, 4) ||
        !aligned(page_table, 4) || !aligned(row_lens, 4))
        return MSA_ERROR_INVALID_VALUE;
    return launched(msa_launch_page_table(s, sel, block_table, seq_lens, page_table, row_lens,
                                          static_cast<hipStream_t>(stream)));
}

size_t msa_decode_workspace_size(const msa_dims_t* dims) {
    MsaShape s;
    if (check_dims(dims, &s) != MSA_SUCCESS) return 0;
    return msa_decode_ws_bytes(s);
}

size_t msa_prefill_workspace_size(const msa_dims_t* dims, int32_t total_q) {
    MsaShape s;
    if (check_dims(dims, &s) != MSA_SUCCESS || check_total_q(s, total_q) != MSA_SUCCESS) return 0;
    return msa_prefill_ws_bytes(s, total_q);
}

msa_status_t msa_sparse_attn_decode(const msa_dims_t* dims, const uint16_t* q,
                                    const uint16_t* k_cache, const uint16_t* v_cache,
                                    const int32_t* page_table, const int32_t* row_lens,
                                    uint16_t* out, float* lse, void* workspace,
                                    size_t workspace_bytes, void* stream) {
    MsaShape s;
    msa_status_t st = check_dims(dims, &s);
    if (st != MSA_SUCCESS) return st;
    if (s.B == 0) return MSA_SUCCESS;  // no work: nothing read, nothing launched
    if (!q || !k_cache || !v_cache || !page_table || !row_lens || !out) return MSA_ERROR_INVALID_VALUE;
    if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) ||
        !aligned(page_table, 4) || !aligned(row_lens, 4) || !aligned(out, 16) ||
        (lse && !aligned(lse, 4)))
        return MSA_ERROR_INVALID_VALUE;
    if (!workspace || !aligned(workspace, 256) || workspace_bytes < msa_decode_ws_bytes(s))
        return MSA_ERROR_WORKSPACE;
    return launched(msa_launch_decode(s, q, k_cache, v_cache, page_table, row_lens, out, lse,
                                      workspace, static_cast<hipStream_t>(stream)));
}

msa_status_t msa_sparse_attn_prefill(const msa_dims_t* dims, int32_t total_q, const uint16_t* q,
                                     const uint16_t* k_cache, const uint16_t* v_cache,
                                     const int32_t* block_table, const int32_t* seq_lens,
                                     const int32_t* cu_q, const int32_t* sel, uint16_t* out,
                                     float* lse, void* workspace, size_t workspace_bytes,
                                     void* stream) {
    MsaShape s;
    msa_status_t st = check_dims(dims, &s);
    if (st != MSA_SUCCESS) return st;
    if ((st = check_total_q(s, total_q)) != MSA_SUCCESS) return st;
    if (total_q == 0) return MSA_SUCCESS;  // no work: nothing read, nothing launched
    if (!q || !k_cache || !v_cache || !block_table || !seq_lens || !cu_q || !sel || !out)
        return MSA_ERROR_INVALID_VALUE;
    if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) ||
        !aligned(block_table, 4) || !aligned(seq_lens, 4) || !aligned(cu_q, 4) ||
        !aligned(sel, 4) || !aligned(out, 16) || (lse && !aligned(lse, 4)))
        return MSA_ERROR_INVALID_VALUE;
    if (!workspace || !aligned(workspace, 256) ||
        workspace_bytes < msa_prefill_ws_bytes(s, total_q))
        return MSA_ERROR_WORKSPACE;
    return launched(msa_launch_prefill(s, total_q, q, k_cache, v_cache, block_table, seq_lens, cu_q,
                                       sel, out, lse, workspace, static_cast<hipStream_t>(stream)));
}

size_t msa_multi_query_step_workspace_size(const msa_dims_t* dims, int32_t total_q) {
    MsaShape s;
    if (check_dims(dims, &s) != MSA_SUCCESS || check_total_q(s, total_q) != MSA_SUCCESS) return 0;
    return msa_multi_query_ws_bytes(s, total_q);
}

msa_status_t msa_multi_query_step(const msa_dims_t* dims, int32_t total_q, const uint16_t* q_idx,
                                  const uint16_t* kidx_cache, const uint16_t* q,
                                  const uint16_t* k_cache, const uint16_t* v_cache,
                                  const int32_t* block_table, const int32_t* seq_lens,
                                  const int32_t* cu_q, uint16_t* out, float* lse, int32_t* sel,
                                  void* workspace, size_t workspace_bytes, void* stream) {
    MsaShape s;
    msa_status_t st = check_dims(dims, &s);
    if (st != MSA_SUCCESS) return st;
    if ((st = check_total_q(s, total_q)) != MSA_SUCCESS) return st;
    if (total_q == 0) return MSA_SUCCESS;  // no work: nothing read, nothing launched
    if (!q_idx || !kidx_cache || !q || !k_cache || !v_cache || !block_table || !seq_lens ||
        !cu_q || !out)
        return MSA_ERROR_INVALID_VALUE;
    if (!aligned(q_idx, 16) || !aligned(kidx_cache, 16) || !aligned(q, 16) ||
        !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(block_table, 4) ||
        !aligned(seq_lens, 4) || !aligned(cu_q, 4) || !aligned(out, 16) ||
        (lse && !aligned(lse, 4)) || (sel && !aligned(sel, 4)))
        return MSA_ERROR_INVALID_VALUE;
    if ((int64_t)s.B * s.Hidx > 65535) return MSA_ERROR_NOT_SUPPORTED;
    if (!workspace || !aligned(workspace, 256) ||
        workspace_bytes < msa_multi_query_ws_bytes(s, total_q))
        return MSA_ERROR_WORKSPACE;
    return launched(msa_launch_multi_query_step(s, total_q, q_idx, kidx_cache, q, k_cache, v_cache,
                                                block_table, seq_lens, cu_q, out, lse, sel,
                                                workspace, static_cast<hipStream_t>(stream)));
}

size_t msa_decode_step_workspace_size(const msa_dims_t* dims) {
    MsaShape s;
    if (check_dims(dims, &s) != MSA_SUCCESS) return 0;
    return msa_decode_step_ws_bytes(s);
}

// The decode step's checks and launches, with or without the cache append;
// workspace == kStaticScratch selects the library's static scratch.
static msa_status_t decode_step(const msa_dims_t* dims, const uint16_t* q_idx,
                                const uint16_t* kidx_cache, const uint16_t* q,
                                const uint16_t* k_cache, const uint16_t* v_cache,
                                const int32_t* block_table, const int32_t* seq_lens,
                                uint16_t* out, float* lse, int32_t* sel, void* workspace,
                                size_t workspace_bytes, const DecodeAppend* app, void* stream) {
    MsaShape s;
    msa_status_t st = check_dims(dims, &s);
    if (st != MSA_SUCCESS) return st;
    if (s.B == 0) return MSA_SUCCESS;  // no work: nothing read, nothing launched
    if (app && (!app->k_new || !app->v_new || !app->kidx_new || !aligned(app->k_new, 16) ||
                !aligned(app->v_new, 16) || !aligned(app->kidx_new, 16)))
        return MSA_ERROR_INVALID_VALUE;
    if (!q_idx || !kidx_cache || !q || !k_cache || !v_cache || !block_table || !seq_lens || !out)
        return MSA_ERROR_INVALID_VALUE;
    if (!aligned(q_idx, 16) || !aligned(kidx_cache, 16) || !aligned(q, 16) ||
        !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(block_table, 4) ||
        !aligned(seq_lens, 4) || !aligned(out, 16) || (lse && !aligned(lse, 4)) ||
        (sel && !aligned(sel, 4)))
        return MSA_ERROR_INVALID_VALUE;
    if ((int64_t)s.B * s.Hidx > 65535) return MSA_ERROR_NOT_SUPPORTED;
    hipStream_t hs = static_cast<hipStream_t>(stream);
    if (workspace == kStaticScratch) {
        // the library's own scratch on the stream's GPU, no caller workspace
        if (msa_decode_step_ws_bytes(s) > msa_static_scratch_bytes()) return MSA_ERROR_WORKSPACE;
        if (msa_static_scratch(hs, &workspace) != hipSuccess) return MSA_ERROR_LAUNCH;
    } else if (!workspace || !aligned(workspace, 256) ||
               workspace_bytes < msa_decode_step_ws_bytes(s)) {
        return MSA_ERROR_WORKSPACE;
    }
    return launched(msa_launch_decode_step(s, q_idx, kidx_cache, q, k_cache, v_cache, block_table,
                                           seq_lens, out, lse, sel, workspace, app, hs));
}

msa_status_t msa_decode_step(const msa_dims_t* dims, const uint16_t* q_idx,
                             const uint16_t* kidx_cache, const uint16_t* q,
                             const uint16_t* k_cache, const uint16_t* v_cache,
                             const int32_t* block_table, const int32_t* seq_lens, uint16_t* out,
                             float* lse, int32_t* sel, void* workspace, size_t workspace_bytes,
                             void* stream) {
    return decode_step(dims, q_idx, kidx_cache, q, k_cache, v_cache, block_table, seq_lens, out,
                       lse, sel, workspace, workspace_bytes, nullptr, stream);
}

msa_status_t msa_decode_step_append(const msa_dims_t* dims, const uint16_t* k_new,
                                    const uint16_t* v_new, const uint16_t* kidx_new,
                                    const uint16_t* q_idx, uint16_t* kidx_cache,
                                    const uint16_t* q, uint16_t* k_cache, uint16_t* v_cache,
                                    const int32_t* block_table, const int32_t* seq_lens,
                                    uint16_t* out, float* lse, int32_t* sel, void* workspace,
                                    size_t workspace_bytes, void* stream) {
    const DecodeAppend app{k_new, v_new, kidx_new, k_cache, v_cache, kidx_cache};
    return decode_step(dims, q_idx, kidx_cache, q, k_cache, v_cache, block_table, seq_lens, out,
                       lse, sel, workspace, workspace_bytes, &app, stream);
}

msa_status_t msa_decode_step_noalloc(const msa_dims_t* dims, const uint16_t* q_idx,
                                     const uint16_t* kidx_cache, const uint16_t* q,
                                     const uint16_t* k_cache, const uint16_t* v_cache,
                                     const int32_t* block_table, const int32_t* seq_lens,
                                     uint16_t* out, float* lse, int32_t* sel, void* stream) {
    return decode_step(dims, q_idx, kidx_cache, q, k_cache, v_cache, block_table, seq_lens, out,
                       lse, sel, kStaticScratch, 0, nullptr, stream);
}

size_t msa_dense_decode_workspace_size(const msa_dims_t* dims) {
    MsaShape s;
    if (check_dims(dims, &s) != MSA_SUCCESS) return 0;
    return msa_dense_decode_ws_bytes(s);
}

msa_status_t msa_dense_attn_decode(const msa_dims_t* dims, const uint16_t* q,
                                   const uint16_t* k_cache, const uint16_t* v_cache,
                                   const int32_t* block_table, const int32_t* seq_lens,
                                   uint16_t* out, float* lse, void* workspace,
                                   size_t workspace_bytes, void* stream) {
    MsaShape s;
    msa_status_t st = check_dims(dims, &s);
    if (st != MSA_SUCCESS) return st;
    if (s.B == 0) return MSA_SUCCESS;  // no work: nothing read, nothing launched
    if (!q || !k_cache || !v_cache || !block_table || !seq_lens || !out)
        return MSA_ERROR_INVALID_VALUE;
    if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) ||
        !aligned(block_table, 4) || !aligned(seq_lens, 4) || !aligned(out, 16) ||
        (lse && !aligned(lse, 4)))
        return MSA_ERROR_INVALID_VALUE;
    if ((int64_t)s.B * s.Hkv > 65535) return MSA_ERROR_NOT_SUPPORTED;
    if (!workspace || !aligned(workspace, 256) || workspace_bytes < msa_dense_decode_ws_bytes(s))
        return MSA_ERROR_WORKSPACE;
    return launched(msa_launch_dense_decode(s, q, k_cache, v_cache, block_table, seq_lens, out, lse,
                                            workspace, static_cast<hipStream_t>(stream)));
}

msa_status_t msa_dense_attn_prefill(const msa_dims_t* dims, int32_t total_q, const uint16_t* q,
                                    const uint16_t* k_cache, const uint16_t* v_cache,
                                    const int32_t* block_table, const int32_t* seq_lens,
                                    const int32_t* cu_q, uint16_t* out, float* lse, void* stream) {
    MsaShape s;
    msa_status_t st = check_dims(dims, &s);
    if (st != MSA_SUCCESS) return st;
    if ((st = check_total_q(s, total_q)) != MSA_SUCCESS) return st;
    if (total_q == 0) return MSA_SUCCESS;  // no work: nothing read, nothing launched
    if (!q || !k_cache || !v_cache || !block_table || !seq_lens || !cu_q || !out)
        return MSA_ERROR_INVALID_VALUE;
    if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) ||
        !aligned(block_table, 4) || !aligned(seq_lens, 4) || !aligned(cu_q, 4) ||
        !aligned(out, 16) || (lse && !aligned(lse, 4)))
        return MSA_ERROR_INVALID_VALUE;
    return launched(msa_launch_dense_prefill(s, total_q, q, k_cache, v_cache, block_table, seq_lens,
                                             cu_q, out, lse, static_cast<hipStream_t>(stream)));
}

msa_status_t msa_append_kv(const msa_dims_t* dims, int32_t total_q, const uint16_t* k_new,
                           const uint16_t* v_new, const uint16_t* kidx_new,
                           const int32_t* block_table, const int32_t* seq_lens,
                           const int32_t* cu_q, uint16_t* k_cache, uint16_t* v_cache,
                           uint16_t* kidx_cache, void* stream) {
    MsaShape s;
    msa_status_t st = check_dims(dims, &s);
    if (st != MSA_SUCCESS) return st;
    if ((st = check_total_q(s, total_q)) != MSA_SUCCESS) return st;
    if (total_q == 0) return MSA_SUCCESS;  // no work: nothing read, nothing launched
    if (!k_new || !v_new || !kidx_new || !block_table || !seq_lens || !cu_q || !k_cache ||
        !v_cache || !kidx_cache)
        return MSA_ERROR_INVALID_VALUE;
    if (!aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(kidx_new, 16) ||
        !aligned(block_table, 4) || !aligned(seq_lens, 4) || !aligned(cu_q, 4) ||
        !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(kidx_cache, 16))
        return MSA_ERROR_INVALID_VALUE;
    return launched(msa_launch_append_kv(s, total_q, k_new, v_new, kidx_new, block_table, seq_lens,
                                         cu_q, k_cache, v_cache, kidx_cache,
                                         static_cast<hipStream_t>(stream)));
}

msa_status_t msa_validate_inputs(const msa_dims_t* dims, int32_t total_q, const int32_t* block_table,
                                 const int32_t* seq_lens, const int32_t* cu_q, int32_t* status,
                                 void* stream) {
    MsaShape s;
    msa_status_t st = check_dims(dims, &s);
    if (st != MSA_SUCCESS) return st;
    if (cu_q && (st = check_total_q(s, total_q)) != MSA_SUCCESS) return st;
    if (!block_table || !seq_lens || !status) return MSA_ERROR_INVALID_VALUE;
    if (!aligned(block_table, 4) || !aligned(seq_lens, 4) || (cu_q && !aligned(cu_q, 4)) ||
        !aligned(status, 4))
        return MSA_ERROR_INVALID_VALUE;
    return launched(msa_launch_validate(s, cu_q ? total_q : s.B, block_table, seq_lens, cu_q, status,
                                        static_cast<hipStream_t>(stream)));
}

const char* msa_status_string(msa_status_t status) {
    switch (status) {
        case MSA_SUCCESS: return "MSA_SUCCESS";
        case MSA_ERROR_INVALID_VALUE: return "MSA_ERROR_INVALID_VALUE";
        case MSA_ERROR_NOT_SUPPORTED: return "MSA_ERROR_NOT_SUPPORTED";
        case MSA_ERROR_WORKSPACE: return "MSA_ERROR_WORKSPACE";
        case MSA_ERROR_LAUNCH: return "MSA_ERROR_LAUNCH";
    }
    return "MSA_ERROR_UNKNOWN";
}

int msa_abi_version(void) { return MSA_ABI_VERSION; }

}  // extern "C"
