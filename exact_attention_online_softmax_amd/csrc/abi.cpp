// abi.cpp -- the C ABI of libosm: argument validation on the host, then
// dispatch to the gfx950 kernels on the caller's stream.  Declared in
// include/osm.h, which documents every argument, layout and error code.
//
// Every check runs before any HIP call, so an error other than OSM_ERR_HIP
// means nothing was launched and no output was touched.  No C++ exception
// escapes (none is thrown here, and HIP's C API throws none).
#include <math.h>

#include "../../include/osm.h"
#include "osm_internal.h"

namespace {

inline osm_status hip_status(hipError_t e) { return e == hipSuccess ? OSM_OK : OSM_ERR_HIP; }

constexpr int64_t kMaxDecodeScores = 16384;   // heads-per-group * split_size (64 KiB of LDS)

// (batch, head) pairs are numbered with 32-bit integers inside the kernels
inline bool too_many_heads(int32_t batch, int32_t heads) { return (int64_t)batch * heads > INT32_MAX; }

inline bool misaligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15) != 0; }

}  // namespace

extern "C" {

const char *osm_status_str(osm_status status) {
    switch (status) {
        case OSM_OK: return "OSM_OK";
        case OSM_ERR_NULL: return "OSM_ERR_NULL: a required pointer is NULL";
        case OSM_ERR_SHAPE: return "OSM_ERR_SHAPE: invalid or inconsistent sizes";
        case OSM_ERR_UNSUPPORTED: return "OSM_ERR_UNSUPPORTED: dtype/head_dim/layout not implemented";
        case OSM_ERR_WORKSPACE: return "OSM_ERR_WORKSPACE: workspace missing or too small";
        case OSM_ERR_HIP: return "OSM_ERR_HIP: a HIP runtime call failed";
    }
    return "OSM_ERR_UNKNOWN";
}

osm_status osm_softmax_rows(const float *x, float *y, int64_t rows, int64_t cols, int64_t ld_x,
                            int64_t ld_y, float *row_max, float *row_sum, osm_stream stream) {
    if (rows < 0 || cols < 0 || ld_x < cols || ld_y < cols) return OSM_ERR_SHAPE;
    if (rows == 0) return OSM_OK;
    if ((!x || !y) && cols > 0) return OSM_ERR_NULL;
    if (cols == 0 && !row_max && !row_sum) return OSM_OK;
    osm::SoftmaxArgs a{x, y, rows, cols, ld_x, ld_y, row_max, row_sum};
    const osm::SoftmaxPlan p = osm::plan_softmax_rows(cols, 0);
    return hip_status(osm::launch_softmax_rows(a, p, static_cast<hipStream_t>(stream)));
}

osm_status osm_softmax_rows_twopass(const float *x, float *y, int64_t rows, int64_t cols, int64_t ld_x,
                                    int64_t ld_y, float *row_max, float *row_sum, osm_stream stream) {
    if (rows < 0 || cols < 0 || ld_x < cols || ld_y < cols) return OSM_ERR_SHAPE;
    if (rows == 0) return OSM_OK;
    if ((!x || !y) && cols > 0) return OSM_ERR_NULL;
    if (cols == 0 && !row_max && !row_sum) return OSM_OK;
    osm::SoftmaxArgs a{x, y, rows, cols, ld_x, ld_y, row_max, row_sum};
    const osm::SoftmaxPlan p = osm::plan_softmax_rows(cols, 1);
    return hip_status(osm::launch_softmax_rows(a, p, static_cast<hipStream_t>(stream)));
}

osm_status osm_attn_fwd(const void *q, const void *k, const void *v, void *o, float *lse,
                        osm_dtype dtype, int32_t batch, int32_t heads_q, int32_t heads_kv,
                        int32_t seqlen_q, int32_t seqlen_k, int32_t head_dim,
                        const int32_t *seqlens_q, const int32_t *seqlens_k, float scale,
                        int32_t causal, osm_stream stream) {
    if (batch < 1 || heads_q < 1 || heads_kv < 1 || head_dim < 1 || seqlen_q < 0 || seqlen_k < 0 ||
        heads_q % heads_kv != 0 || !(scale > 0.0f) || !isfinite(scale) || (causal != 0 && causal != 1))
        return OSM_ERR_SHAPE;
    if (dtype != OSM_BF16 || (head_dim != 128 && head_dim != 64) || too_many_heads(batch, heads_q))
        return OSM_ERR_UNSUPPORTED;
    // one head's rows of K, V, Q and O are addressed with 32-bit byte offsets
    if ((int64_t)seqlen_k * head_dim * 2 >= ((int64_t)1 << 31) ||
        (int64_t)seqlen_q * head_dim * 2 >= ((int64_t)1 << 31))
        return OSM_ERR_UNSUPPORTED;
    if (seqlen_q == 0) return OSM_OK;
    if (!q || !o || (seqlen_k > 0 && (!k || !v))) return OSM_ERR_NULL;
    // rows are read and written 16 bytes at a time
    if (misaligned16(q) || misaligned16(k) || misaligned16(v) || misaligned16(o)) return OSM_ERR_UNSUPPORTED;
    osm::AttnFwdArgs a{q, k, v, o, lse, batch, heads_q, heads_kv, seqlen_q, seqlen_k, head_dim,
                       seqlens_q, seqlens_k, scale, causal};
    return hip_status(osm::launch_attn_fwd(a, static_cast<hipStream_t>(stream)));
}

osm_status osm_attn_fwd_fp8(const void *q, const void *k, const void *v, void *o, float *lse,
                            int32_t batch, int32_t heads_q, int32_t heads_kv, int32_t seqlen_q,
                            int32_t seqlen_k, int32_t head_dim, const int32_t *seqlens_q,
                            const int32_t *seqlens_k, float scale, float v_scale, int32_t causal,
                            osm_stream stream) {
    if (batch < 1 || heads_q < 1 || heads_kv < 1 || head_dim < 1 || seqlen_q < 0 || seqlen_k < 0 ||
        heads_q % heads_kv != 0 || !(scale > 0.0f) || !isfinite(scale) || !isfinite(v_scale) ||
        (causal != 0 && causal != 1))
        return OSM_ERR_SHAPE;
    if (head_dim != 128 || too_many_heads(batch, heads_q)) return OSM_ERR_UNSUPPORTED;
    // one head's rows of K, V, Q (E4M3) and O (bf16) are addressed with 32-bit byte offsets
    if ((int64_t)seqlen_k * head_dim >= ((int64_t)1 << 31) ||
        (int64_t)seqlen_q * head_dim * 2 >= ((int64_t)1 << 31))
        return OSM_ERR_UNSUPPORTED;
    if (seqlen_q == 0) return OSM_OK;
    if (!q || !o || (seqlen_k > 0 && (!k || !v))) return OSM_ERR_NULL;
    // operands are read 16 bytes at a time
    if (misaligned16(q) || misaligned16(k) || misaligned16(v) || misaligned16(o)) return OSM_ERR_UNSUPPORTED;
    osm::AttnFwdFp8Args a{q, k, v, o, lse, batch, heads_q, heads_kv, seqlen_q, seqlen_k,
                          seqlens_q, seqlens_k, scale, v_scale, causal};
    return hip_status(osm::launch_attn_fwd_fp8(a, static_cast<hipStream_t>(stream)));
}

size_t osm_attn_bwd_workspace_bytes(int32_t batch, int32_t heads_q, int32_t seqlen_q) {
    if (batch < 1 || heads_q < 1 || seqlen_q < 0) return 0;
    return osm::attn_bwd_workspace_bytes(batch, heads_q, seqlen_q);
}

osm_status osm_attn_bwd(const void *q, const void *k, const void *v, const void *o,
                        const void *dout, const float *lse, void *dq, void *dk, void *dv,
                        osm_dtype dtype, int32_t batch, int32_t heads_q, int32_t heads_kv,
                        int32_t seqlen_q, int32_t seqlen_k, int32_t head_dim,
                        const int32_t *seqlens_q, const int32_t *seqlens_k, float scale,
                        int32_t causal, void *workspace, size_t workspace_bytes,
                        osm_stream stream) {
    if (batch < 1 || heads_q < 1 || heads_kv < 1 || head_dim < 1 || seqlen_q < 0 || seqlen_k < 0 ||
        heads_q % heads_kv != 0 || !(scale > 0.0f) || !isfinite(scale) || (causal != 0 && causal != 1))
        return OSM_ERR_SHAPE;
    if (dtype != OSM_BF16 || (head_dim != 128 && head_dim != 64) || too_many_heads(batch, heads_q))
        return OSM_ERR_UNSUPPORTED;
    // one head's rows are addressed with 32-bit byte offsets
    if ((int64_t)seqlen_k * head_dim * 2 >= ((int64_t)1 << 31) ||
        (int64_t)seqlen_q * head_dim * 2 >= ((int64_t)1 << 31))
        return OSM_ERR_UNSUPPORTED;
    if (seqlen_q == 0 && seqlen_k == 0) return OSM_OK;
    if ((seqlen_q > 0 && (!q || !o || !dout || !lse || !dq)) || (seqlen_k > 0 && (!k || !v || !dk || !dv)))
        return OSM_ERR_NULL;
    // operands are read 16 bytes at a time
    const void *ptrs[] = {q, k, v, o, dout, dq, dk, dv};
    for (const void *p : ptrs)
        if (misaligned16(p)) return OSM_ERR_UNSUPPORTED;
    const size_t need = osm::attn_bwd_workspace_bytes(batch, heads_q, seqlen_q);
    if (need > 0 && (!workspace || workspace_bytes < need || (reinterpret_cast<uintptr_t>(workspace) & 255)))
        return OSM_ERR_WORKSPACE;
    osm::AttnBwdArgs a{q, k, v, o, dout, lse, dq, dk, dv, batch, heads_q, heads_kv, seqlen_q, seqlen_k,
                       head_dim, seqlens_q, seqlens_k, scale, causal, workspace};
    return hip_status(osm::launch_attn_bwd(a, static_cast<hipStream_t>(stream)));
}

size_t osm_decode_workspace_bytes(int32_t batch, int32_t heads_q, int32_t max_seqlen_k,
                                  int32_t head_dim, int32_t split_size) {
    if (batch < 1 || heads_q < 1 || max_seqlen_k < 1 || head_dim < 1 || split_size < 1) return 0;
    return osm::decode_layout(batch, heads_q, max_seqlen_k, head_dim, split_size).total;
}

osm_status osm_attn_decode_splitkv(const void *q, const void *k_cache, const void *v_cache,
                                   void *o, float *lse, osm_dtype dtype, int32_t batch,
                                   int32_t heads_q, int32_t heads_kv, int32_t max_seqlen_k,
                                   int32_t head_dim, const int32_t *seqlens_k, float scale,
                                   int32_t split_size, void *workspace, size_t workspace_bytes,
                                   osm_stream stream) {
    if (batch < 1 || heads_q < 1 || heads_kv < 1 || max_seqlen_k < 1 || head_dim < 1 ||
        heads_q % heads_kv != 0 || !(scale > 0.0f) || !isfinite(scale) || split_size < 1)
        return OSM_ERR_SHAPE;
    const int group = heads_q / heads_kv;
    if ((dtype != OSM_F32 && dtype != OSM_BF16) || (head_dim != 64 && head_dim != 128) ||
        (group != 1 && group != 2 && group != 4 && group != 8) || split_size % 64 != 0 ||
        split_size > 8192 || (int64_t)group * split_size > kMaxDecodeScores ||
        too_many_heads(batch, heads_q))
        return OSM_ERR_UNSUPPORTED;
    if (!q || !k_cache || !v_cache || !o || !seqlens_k) return OSM_ERR_NULL;
    // rows are read 16 bytes at a time
    if (misaligned16(q) || misaligned16(k_cache) || misaligned16(v_cache)) return OSM_ERR_UNSUPPORTED;
    const osm::DecodeLayout lay = osm::decode_layout(batch, heads_q, max_seqlen_k, head_dim, split_size);
    if (lay.total == 0) return OSM_ERR_UNSUPPORTED;   // a workspace past 2^62 bytes
    if (!workspace || workspace_bytes < lay.total || (reinterpret_cast<uintptr_t>(workspace) & 255))
        return OSM_ERR_WORKSPACE;
    osm::DecodeArgs a{q, k_cache, v_cache, o, lse, dtype == OSM_BF16 ? 1 : 0, batch, heads_q,
                      heads_kv, max_seqlen_k, head_dim, seqlens_k, scale, split_size, workspace};
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = osm::launch_decode_split(a, lay, s);
    if (e != hipSuccess) return OSM_ERR_HIP;
    const char *ws = static_cast<const char *>(workspace);
    osm::MergeArgs m{reinterpret_cast<const float *>(ws + lay.off_m),
                     reinterpret_cast<const float *>(ws + lay.off_l),
                     reinterpret_cast<const float *>(ws + lay.off_o),
                     lay.rows, lay.chunks, head_dim, o, a.dtype, lse};
    return hip_status(osm::launch_merge_partials(m, s));
}

osm_status osm_attn_decode_splitkv_noalloc(const void *q, const void *k_cache, const void *v_cache,
                                           void *o, float *lse, osm_dtype dtype, int32_t batch,
                                           int32_t heads_q, int32_t heads_kv, int32_t max_seqlen_k,
                                           int32_t head_dim, const int32_t *seqlens_k, float scale,
                                           int32_t split_size, osm_stream stream) {
    if (batch < 1 || heads_q < 1 || heads_kv < 1 || max_seqlen_k < 1 || head_dim < 1 ||
        heads_q % heads_kv != 0 || !(scale > 0.0f) || !isfinite(scale) || split_size < 1)
        return OSM_ERR_SHAPE;
    const int group = heads_q / heads_kv;
    if ((dtype != OSM_F32 && dtype != OSM_BF16) || (head_dim != 64 && head_dim != 128) ||
        (group != 1 && group != 2 && group != 4 && group != 8) || split_size % 64 != 0 ||
        split_size > 8192 || (int64_t)group * split_size > kMaxDecodeScores ||
        too_many_heads(batch, heads_q))
        return OSM_ERR_UNSUPPORTED;
    if (!q || !k_cache || !v_cache || !o || !seqlens_k) return OSM_ERR_NULL;
    if (misaligned16(q) || misaligned16(k_cache) || misaligned16(v_cache)) return OSM_ERR_UNSUPPORTED;
    const osm::DecodeLayout lay = osm::decode_layout(batch, heads_q, max_seqlen_k, head_dim, split_size);
    // the partials must fit the library's scratch array (OSM_DECODE_SCRATCH_BYTES)
    if (lay.total == 0 || lay.total > osm::kDecodeScratchBytes) return OSM_ERR_WORKSPACE;
    void *workspace = nullptr;
    if (osm::decode_scratch(&workspace) != hipSuccess) return OSM_ERR_HIP;
    osm::DecodeArgs a{q, k_cache, v_cache, o, lse, dtype == OSM_BF16 ? 1 : 0, batch, heads_q,
                      heads_kv, max_seqlen_k, head_dim, seqlens_k, scale, split_size, workspace};
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (osm::launch_decode_split(a, lay, s) != hipSuccess) return OSM_ERR_HIP;
    const char *ws = static_cast<const char *>(workspace);
    osm::MergeArgs m{reinterpret_cast<const float *>(ws + lay.off_m),
                     reinterpret_cast<const float *>(ws + lay.off_l),
                     reinterpret_cast<const float *>(ws + lay.off_o),
                     lay.rows, lay.chunks, head_dim, o, a.dtype, lse};
    return hip_status(osm::launch_merge_partials(m, s));
}

osm_status osm_merge_partials(const float *part_m, const float *part_l, const float *part_o,
                              int64_t rows, int32_t num_splits, int32_t head_dim, void *o,
                              osm_dtype out_dtype, float *lse, osm_stream stream) {
    if (rows < 0 || num_splits < 1 || head_dim < 1) return OSM_ERR_SHAPE;
    if ((out_dtype != OSM_F32 && out_dtype != OSM_BF16) || head_dim > 512) return OSM_ERR_UNSUPPORTED;
    if (rows == 0) return OSM_OK;
    if (!part_m || !part_l || !part_o || !o) return OSM_ERR_NULL;
    osm::MergeArgs m{part_m, part_l, part_o, rows, num_splits, head_dim, o,
                     out_dtype == OSM_BF16 ? 1 : 0, lse};
    return hip_status(osm::launch_merge_partials(m, static_cast<hipStream_t>(stream)));
}

osm_status osm_attn_extend(const void *q, const void *k_new, const void *v_new, osm_dtype dtype,
                           int32_t batch, int32_t heads_q, int32_t heads_kv, int32_t n_new,
                           int32_t head_dim, float scale, float *state_m, float *state_l,
                           float *state_o, int32_t split_size, void *workspace,
                           size_t workspace_bytes, osm_stream stream) {
    if (batch < 1 || heads_q < 1 || heads_kv < 1 || n_new < 0 || head_dim < 1 ||
        heads_q % heads_kv != 0 || !(scale > 0.0f) || !isfinite(scale) || split_size < 1)
        return OSM_ERR_SHAPE;
    const int group = heads_q / heads_kv;
    if ((dtype != OSM_F32 && dtype != OSM_BF16) || (head_dim != 64 && head_dim != 128) ||
        (group != 1 && group != 2 && group != 4 && group != 8) || split_size % 64 != 0 ||
        split_size > 8192 || (int64_t)group * split_size > kMaxDecodeScores ||
        too_many_heads(batch, heads_q))
        return OSM_ERR_UNSUPPORTED;
    if (!state_m || !state_l || !state_o) return OSM_ERR_NULL;
    if (n_new == 0) return OSM_OK;                 // no new keys: the state is already the answer
    if (!q || !k_new || !v_new) return OSM_ERR_NULL;
    // rows are read 16 bytes at a time
    if (misaligned16(q) || misaligned16(k_new) || misaligned16(v_new)) return OSM_ERR_UNSUPPORTED;
    const osm::DecodeLayout lay = osm::decode_layout(batch, heads_q, n_new, head_dim, split_size);
    if (lay.total == 0) return OSM_ERR_UNSUPPORTED;   // a workspace past 2^62 bytes
    if (!workspace || workspace_bytes < lay.total || (reinterpret_cast<uintptr_t>(workspace) & 255))
        return OSM_ERR_WORKSPACE;
    // the new keys' pieces, summarized as in the split decode (every key valid)
    osm::DecodeArgs a{q, k_new, v_new, nullptr, nullptr, dtype == OSM_BF16 ? 1 : 0, batch, heads_q,
                      heads_kv, n_new, head_dim, nullptr, scale, split_size, workspace};
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = osm::launch_decode_split(a, lay, s);
    if (e != hipSuccess) return OSM_ERR_HIP;
    // merged with the persisted summary, back into it
    const char *ws = static_cast<const char *>(workspace);
    osm::MergeArgs m{reinterpret_cast<const float *>(ws + lay.off_m),
                     reinterpret_cast<const float *>(ws + lay.off_l),
                     reinterpret_cast<const float *>(ws + lay.off_o),
                     lay.rows, lay.chunks, head_dim, nullptr, 0, nullptr};
    m.state_m = state_m;
    m.state_l = state_l;
    m.state_o = state_o;
    return hip_status(osm::launch_merge_partials(m, s));
}

osm_status osm_merge_lse(const void *o_parts, const float *lse_parts, int64_t rows,
                         int32_t num_parts, int32_t head_dim, osm_dtype in_dtype, void *o,
                         osm_dtype out_dtype, float *lse, osm_stream stream) {
    if (rows < 0 || num_parts < 1 || head_dim < 1) return OSM_ERR_SHAPE;
    if ((in_dtype != OSM_F32 && in_dtype != OSM_BF16) || (out_dtype != OSM_F32 && out_dtype != OSM_BF16) ||
        head_dim > 1024 || (head_dim % 2 != 0 && head_dim > 512))
        return OSM_ERR_UNSUPPORTED;
    if (rows == 0) return OSM_OK;
    if (!o_parts || !lse_parts || !o) return OSM_ERR_NULL;
    // pieces and output are read and written in vectors of up to 16 bytes
    if (misaligned16(o_parts) || misaligned16(o)) return OSM_ERR_UNSUPPORTED;
    osm::MergeLseArgs m{o_parts, lse_parts, rows, num_parts, head_dim,
                        in_dtype == OSM_BF16 ? 1 : 0, out_dtype == OSM_BF16 ? 1 : 0, o, lse};
    return hip_status(osm::launch_merge_lse(m, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
