// osm_internal.h -- host-side launch interfaces between the C ABI layer and
// the kernel translation units of libosm (not installed, not part of the ABI).
// The sizes and plans (layout.cpp) are plain host code; the launchers live
// beside their kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace osm {

// ---- row softmax ----------------------------------------------------------
struct SoftmaxArgs {
    const float *x;
    float *y;
    int64_t rows, cols, ld_x, ld_y;
    float *row_max, *row_sum;
};
struct SoftmaxPlan {
    bool resident;   // row held in registers (one HBM read) vs two streaming passes
    int nv;          // float4 vectors per lane (resident)
    int threads;     // workgroup size
};
// float4 vectors per lane whose loads the streaming kernel issues together
constexpr int kSoftmaxStreamBatch = 4;
// force_variant: 0 = automatic, 1 = streaming
SoftmaxPlan plan_softmax_rows(int64_t cols, int force_variant);
hipError_t launch_softmax_rows(const SoftmaxArgs &a, const SoftmaxPlan &p, hipStream_t s);

// ---- fused attention forward ---------------------------------------------
struct AttnFwdArgs {
    const void *q, *k, *v;
    void *o;
    float *lse;
    int batch, heads_q, heads_kv, seqlen_q, seqlen_k, head_dim;
    const int32_t *seqlens_q, *seqlens_k;
    float scale;
    int causal;
};
hipError_t launch_attn_fwd(const AttnFwdArgs &a, hipStream_t s);

// ---- fused attention forward, FP8 (OCP E4M3) inputs -------------------------
struct AttnFwdFp8Args {
    const void *q, *k, *v;   // E4M3 codes
    void *o;                 // bf16
    float *lse;
    int batch, heads_q, heads_kv, seqlen_q, seqlen_k;
    const int32_t *seqlens_q, *seqlens_k;
    float scale, v_scale;
    int causal;
};
hipError_t launch_attn_fwd_fp8(const AttnFwdFp8Args &a, hipStream_t s);

// ---- attention backward ----------------------------------------------------
struct AttnBwdArgs {
    const void *q, *k, *v, *o, *dout;
    const float *lse;
    void *dq, *dk, *dv;
    int batch, heads_q, heads_kv, seqlen_q, seqlen_k, head_dim;
    const int32_t *seqlens_q, *seqlens_k;
    float scale;
    int causal;
    void *workspace;     // attn_bwd_workspace_bytes(): (lse2, D) per query row
};
// 0 when the size does not fit in 2^62 bytes
size_t attn_bwd_workspace_bytes(int64_t batch, int64_t heads_q, int64_t seqlen_q);
hipError_t launch_attn_bwd(const AttnBwdArgs &a, hipStream_t s);

// ---- split-KV decode + merge ----------------------------------------------
struct DecodeLayout {
    int64_t rows;        // batch * heads_q
    int32_t chunks;      // C = ceil(max_seqlen_k / split)
    size_t off_m, off_l, off_o, total;   // total = 0: the workspace would exceed 2^62 bytes
};
DecodeLayout decode_layout(int64_t batch, int64_t heads_q, int64_t max_seqlen_k, int64_t head_dim,
                           int64_t split);

struct DecodeArgs {
    const void *q, *k, *v;
    void *o;
    float *lse;
    int dtype;           // 0 f32, 1 bf16
    int batch, heads_q, heads_kv, max_seqlen_k, head_dim;
    const int32_t *seqlens_k;
    float scale;
    int split;
    void *workspace;
};
hipError_t launch_decode_split(const DecodeArgs &a, const DecodeLayout &lay, hipStream_t s);

// The decode workspace held by the library for callers that cannot allocate:
// kDecodeScratchBytes of device memory per GPU (a file-scope device array in
// decode.hip), shared by every call on that GPU.  decode_scratch() returns its
// address on the current device, looked up once per device.
constexpr size_t kDecodeScratchBytes = (size_t)64 << 20;
hipError_t decode_scratch(void **ptr);

struct MergeArgs {
    const float *part_m, *part_l, *part_o;
    int64_t rows;
    int num_splits, head_dim;
    void *o;
    int out_dtype;       // 0 f32, 1 bf16
    float *lse;
    // streaming extend: when set, the persisted summary [rows], [rows],
    // [rows][head_dim] joins the merge and receives the result (o, lse unused)
    float *state_m = nullptr, *state_l = nullptr, *state_o = nullptr;
};
hipError_t launch_merge_partials(const MergeArgs &a, hipStream_t s);

// ---- log-sum-exp merge of normalized results -------------------------------
struct MergeLseArgs {
    const void *o_parts;       // [num_parts][rows][head_dim]
    const float *lse_parts;    // [num_parts][rows]
    int64_t rows;
    int num_parts, head_dim;
    int in_bf16, out_bf16;     // element types of o_parts and o
    void *o;                   // [rows][head_dim]
    float *lse;                // [rows] or null
};
hipError_t launch_merge_lse(const MergeLseArgs &a, hipStream_t s);

}  // namespace osm
