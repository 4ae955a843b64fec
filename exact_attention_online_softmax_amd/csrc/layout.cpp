// layout.cpp -- host-side sizes and launch plans of libosm: the row-softmax
// plan, the decode workspace layout and the backward workspace size.  Plain
// host code with no device code and no HIP call, shared by the C ABI layer
// (which validates against these sizes) and the kernels' launchers.
#include "osm_internal.h"

namespace osm {

namespace {

constexpr unsigned __int128 kMaxBytes = (unsigned __int128)1 << 62;

inline unsigned __int128 align256(unsigned __int128 x) { return (x + 255) & ~(unsigned __int128)255; }

}  // namespace

// The row lives in registers when it fits in 16 float4 per lane of a
// workgroup of at most 1024 threads.  Rows of more than 4096 vectors take 16
// vectors per lane and the fewest threads (measured on MI355X for 32000
// columns: 512 threads x 16 vectors reaches 69% of HBM peak, 1024 x 8 59%);
// shorter rows take the smallest power-of-two workgroup that holds them.
// Longer rows, or force_variant == 1, take the streaming two-pass kernel:
// 1024 threads, or for short rows the smallest power of two (at least 64)
// whose one batch of loads covers the row.
SoftmaxPlan plan_softmax_rows(int64_t cols, int force_variant) {
    SoftmaxPlan p{};
    const int64_t nvec = (cols + 3) / 4;
    if (force_variant != 1 && nvec <= 16 * 1024) {
        p.resident = true;
        if (nvec > 4096) {
            p.nv = 16;
            p.threads = 256;
            while ((int64_t)p.threads * 16 < nvec) p.threads *= 2;
            return p;
        }
        for (int nv : {4, 8, 16}) {
            for (int t = 64; t <= 1024; t *= 2) {
                if ((int64_t)t * nv >= nvec) {
                    p.nv = nv;
                    p.threads = t;
                    return p;
                }
            }
        }
    }
    p.resident = false;
    p.nv = 0;
    p.threads = 64;
    while (p.threads < 1024 && (int64_t)p.threads * kSoftmaxStreamBatch < nvec) p.threads *= 2;
    return p;
}

// fp32 m [rows][C], l [rows][C], O~ [rows][C][head_dim], each 256-byte
// aligned, C = ceil(max_seqlen_k / split).  Sizes are formed in 128-bit
// arithmetic; a layout past 2^62 bytes has total = 0.
DecodeLayout decode_layout(int64_t batch, int64_t heads_q, int64_t max_seqlen_k, int64_t head_dim,
                           int64_t split) {
    DecodeLayout lay{};
    lay.rows = batch * heads_q;
    lay.chunks = (int32_t)((max_seqlen_k + split - 1) / split);
    const unsigned __int128 n = (unsigned __int128)lay.rows * (unsigned __int128)lay.chunks;
    const unsigned __int128 off_l = align256(n * sizeof(float));
    const unsigned __int128 off_o = off_l + align256(n * sizeof(float));
    const unsigned __int128 total = off_o + align256(n * (unsigned __int128)head_dim * sizeof(float));
    if (total > kMaxBytes) return lay;   // total = 0
    lay.off_m = 0;
    lay.off_l = (size_t)off_l;
    lay.off_o = (size_t)off_o;
    lay.total = (size_t)total;
    return lay;
}

// one float2 (lse in base-2 units, D = dO . O) per query row
size_t attn_bwd_workspace_bytes(int64_t batch, int64_t heads_q, int64_t seqlen_q) {
    const unsigned __int128 b = (unsigned __int128)batch * (unsigned __int128)heads_q *
                                (unsigned __int128)seqlen_q * 8u;
    return b > kMaxBytes ? 0 : (size_t)b;
}

}  // namespace osm
