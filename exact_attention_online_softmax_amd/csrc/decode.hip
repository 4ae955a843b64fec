// decode.hip -- split-KV decode attention and the merge of partial
// summaries, gfx950.
//
// [P1] "How does this connect to KV-cache decoding?": one new query token
// attends to a cache of raw K and V.  [P3] "Merging partial results": the
// keys of a row are split into disjoint pieces, each summarized relative to
// its own maximum by the triple (m, l, O~) = (max s, sum e^(s-m),
// sum e^(s-m) v); the merge brings two summaries to the larger maximum and
// adds, is associative and commutative, and has the empty set (-inf, 0, 0)
// as identity.  [P3] "The same merge, in log-sum-exp form" names the split
// of one query's keys over many thread blocks.
//
// decode_split: one workgroup per (piece, kv head, batch).  All query heads
// that share the kv head (grouped-query attention) are served from one read
// of the piece's K and V.  Lanes are grouped LPK = head_dim / 8 per key, each
// lane owning 8 consecutive dims, so every wave load is a contiguous run of
// whole cache rows.  Phase 1 computes the piece's scores into LDS; the
// piece maximum and sum follow; phase 2 accumulates sum p_j v_j.
// Pieces wholly past the valid length write the identity (m = -inf, l = 0).
//
// merge_partials: one workgroup per row; pieces are merged in groups of up
// to blockDim with the running-maximum rescale between groups, empty pieces
// skipped (their l and O~ are never read).  Then o = O~ / l once and
// LSE = m + log l ([P3] "From weights to outputs").
#include "osm_device.h"
#include "osm_internal.h"

namespace osm {

namespace {

constexpr int DEC_THREADS = 256;
constexpr int DEC_WAVES = DEC_THREADS / 64;

__device__ __forceinline__ int clampi(int v, int lo, int hi) { return v < lo ? lo : (v > hi ? hi : v); }

// 8 consecutive elements of a row as fp32
template <typename T> struct Row8;
template <> struct Row8<float> {
    static __device__ __forceinline__ void load(const float *p, float (&v)[8]) {
        const float4 a = *reinterpret_cast<const float4 *>(p);
        const float4 b = *reinterpret_cast<const float4 *>(p + 4);
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
        v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    }
};
template <> struct Row8<uint16_t> {
    static __device__ __forceinline__ void load(const uint16_t *p, float (&v)[8]) {
        const uint4 a = *reinterpret_cast<const uint4 *>(p);
        v[0] = bf16_lo(a.x); v[1] = bf16_hi(a.x); v[2] = bf16_lo(a.y); v[3] = bf16_hi(a.y);
        v[4] = bf16_lo(a.z); v[5] = bf16_hi(a.z); v[6] = bf16_lo(a.w); v[7] = bf16_hi(a.w);
    }
};

template <typename T, int HD, int G>
__global__ void __launch_bounds__(DEC_THREADS)
decode_split(const T *__restrict__ Q, const T *__restrict__ K, const T *__restrict__ V,
             const int32_t *__restrict__ seqlens_k, int Hq, int Hkv, int Lmax, int split,
             int chunks, float scale_log2, float *__restrict__ ws_m, float *__restrict__ ws_l,
             float *__restrict__ ws_o) {
    constexpr int LPK = HD / 8;                 // lanes per key
    constexpr int KPW = 64 / LPK;               // keys per wave step
    constexpr int KPB = KPW * DEC_WAVES;        // keys per workgroup step
    constexpr int U = 4;                        // key steps in flight per lane
    extern __shared__ float sc[];               // scores, then weights: [G][split]
    __shared__ float red_o[DEC_WAVES][G][HD];   // cross-wave partial outputs
    __shared__ float stat_m[G], stat_l[G];

    const int c = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int L = clampi(seqlens_k[b], 0, Lmax);
    const int start = c * split;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const size_t row0 = (size_t)(b * Hq + g * G);   // first query row of this group

    if (start >= L) {          // empty piece: the identity
        if (tid < G) {
            ws_m[(row0 + tid) * chunks + c] = kNegInf;
            ws_l[(row0 + tid) * chunks + c] = 0.0f;
        }
        return;
    }
    const int n = min(split, L - start);
    const int kslot = lane / LPK;               // key slot within the wave step
    const int d0 = (lane % LPK) * 8;            // this lane's 8 dims

    // the G query vectors, this lane's 8 dims
    float q[G][8];
#pragma unroll
    for (int hh = 0; hh < G; ++hh) Row8<T>::load(Q + (row0 + hh) * HD + d0, q[hh]);

    const T *Kp = K + ((size_t)(b * Hkv + g) * Lmax + start) * HD;
    const T *Vp = V + ((size_t)(b * Hkv + g) * Lmax + start) * HD;

    // ---- phase 1: scores (base-2 scaled units) --------------------------
    // U key steps per iteration: all loads are issued before any use.
    for (int k0 = 0; k0 < n; k0 += KPB * U) {
        float kv[U][8];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int kk = k0 + u * KPB + wave * KPW + kslot;
            if (kk < n) Row8<T>::load(Kp + (size_t)kk * HD + d0, kv[u]);
            else
#pragma unroll
                for (int e = 0; e < 8; ++e) kv[u][e] = 0.0f;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int kk = k0 + u * KPB + wave * KPW + kslot;
            float dot[G];
#pragma unroll
            for (int hh = 0; hh < G; ++hh) {
                float acc = 0.0f;
#pragma unroll
                for (int e = 0; e < 8; ++e) acc = fmaf(q[hh][e], kv[u][e], acc);
                dot[hh] = acc;
            }
#pragma unroll
            for (int off = LPK / 2; off >= 1; off >>= 1)
#pragma unroll
                for (int hh = 0; hh < G; ++hh) dot[hh] += __shfl_xor(dot[hh], off, 64);
            if ((lane % LPK) == 0 && kk < n)
#pragma unroll
                for (int hh = 0; hh < G; ++hh) sc[hh * split + kk] = dot[hh] * scale_log2;
        }
    }
    __syncthreads();

    // ---- piece maximum and weights, one wave per query head --------------
    for (int hh = wave; hh < G; hh += DEC_WAVES) {
        float mx = kNegInf;
        for (int j = lane; j < n; j += 64) mx = fmaxf(mx, sc[hh * split + j]);
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
        float sum = 0.0f;
        for (int j = lane; j < n; j += 64) {
            const float p = fast_exp2(sc[hh * split + j] - mx);
            sc[hh * split + j] = p;
            sum += p;
        }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) sum += __shfl_xor(sum, off, 64);
        if (lane == 0) {
            stat_m[hh] = mx;
            stat_l[hh] = sum;
        }
    }
    __syncthreads();

    // ---- phase 2: O~ = sum_j p_j v_j --------------------------------------
    float acc[G][8];
#pragma unroll
    for (int hh = 0; hh < G; ++hh)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[hh][e] = 0.0f;
    for (int k0 = 0; k0 < n; k0 += KPB * U) {
        float vv[U][8];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int kk = k0 + u * KPB + wave * KPW + kslot;
            if (kk < n) Row8<T>::load(Vp + (size_t)kk * HD + d0, vv[u]);
            else
#pragma unroll
                for (int e = 0; e < 8; ++e) vv[u][e] = 0.0f;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int kk = k0 + u * KPB + wave * KPW + kslot;
            if (kk < n) {
#pragma unroll
                for (int hh = 0; hh < G; ++hh) {
                    const float p = sc[hh * split + kk];
#pragma unroll
                    for (int e = 0; e < 8; ++e) acc[hh][e] = fmaf(p, vv[u][e], acc[hh][e]);
                }
            }
        }
    }
    // reduce over the key slots of the wave (lanes with equal lane % LPK)
#pragma unroll
    for (int off = LPK; off < 64; off <<= 1)
#pragma unroll
        for (int hh = 0; hh < G; ++hh)
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[hh][e] += __shfl_xor(acc[hh][e], off, 64);
    if (lane < LPK)
#pragma unroll
        for (int hh = 0; hh < G; ++hh)
#pragma unroll
            for (int e = 0; e < 8; ++e) red_o[wave][hh][d0 + e] = acc[hh][e];
    __syncthreads();
    for (int i = tid; i < G * HD; i += DEC_THREADS) {
        const int hh = i / HD, d = i % HD;
        float o = 0.0f;
#pragma unroll
        for (int w = 0; w < DEC_WAVES; ++w) o += red_o[w][hh][d];
        ws_o[((row0 + hh) * chunks + c) * HD + d] = o;
    }
    if (tid < G) {
        ws_m[(row0 + tid) * chunks + c] = stat_m[tid] * kLn2;    // natural-log units
        ws_l[(row0 + tid) * chunks + c] = stat_l[tid];
    }
}

// ---- merge ----------------------------------------------------------------
__global__ void __launch_bounds__(512)
merge_partials_kernel(const float *__restrict__ pm, const float *__restrict__ pl,
                      const float *__restrict__ po, int64_t rows, int C, int HD,
                      void *__restrict__ out, int out_bf16, float *__restrict__ lse) {
    __shared__ float w_s[512];
    __shared__ float red[16];
    const int tid = threadIdx.x, nt = blockDim.x;
    const int lane = tid & 63, wave = tid >> 6, nw = nt >> 6;
    for (int64_t r = blockIdx.x; r < rows; r += gridDim.x) {
        float m = kNegInf, l = 0.0f, acc = 0.0f;
        for (int c0 = 0; c0 < C; c0 += nt) {
            const int cn = min(nt, C - c0);
            // group maximum
            const float mc = (tid < cn) ? pm[r * C + c0 + tid] : kNegInf;
            float mx = mc;
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
            if (lane == 0) red[wave] = mx;
            __syncthreads();
            mx = kNegInf;
            for (int w = 0; w < nw; ++w) mx = fmaxf(mx, red[w]);
            __syncthreads();
            const float mn = fmaxf(m, mx);
            if (mn == kNegInf) continue;                      // only empty pieces so far
            // weights of this group's pieces against the new reference
            const float wc = (mc == kNegInf) ? 0.0f : exp_acc(mc - mn);
            w_s[tid] = wc;
            float lw = (wc != 0.0f) ? wc * pl[r * C + c0 + tid] : 0.0f;
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1) lw += __shfl_xor(lw, off, 64);
            if (lane == 0) red[wave] = lw;
            __syncthreads();
            float lsum = 0.0f;
            for (int w = 0; w < nw; ++w) lsum += red[w];
            const float alpha = (m == kNegInf) ? 0.0f : exp_acc(m - mn);
            l = fmaf(l, alpha, lsum);
            if (tid < HD) {
                float a = acc * alpha;
                for (int j = 0; j < cn; ++j) {
                    const float wj = w_s[j];
                    if (wj != 0.0f) a = fmaf(wj, po[(r * C + c0 + j) * HD + tid], a);
                }
                acc = a;
            }
            m = mn;
            __syncthreads();
        }
        const bool valid = (m != kNegInf) && (l > 0.0f);
        if (tid < HD) {
            const float o = valid ? acc / l : 0.0f;
            if (out_bf16) static_cast<uint16_t *>(out)[r * HD + tid] = f32_to_bf16(o);
            else static_cast<float *>(out)[r * HD + tid] = o;
        }
        if (lse && tid == 0) lse[r] = valid ? m + logf(l) : kNegInf;
    }
}

template <typename T, int HD, int G>
hipError_t launch_split(const DecodeArgs &a, const DecodeLayout &lay, hipStream_t s) {
    char *ws = static_cast<char *>(a.workspace);
    dim3 grid(lay.chunks, a.heads_kv, a.batch);
    const size_t shmem = (size_t)G * a.split * sizeof(float);
    hipLaunchKernelGGL((decode_split<T, HD, G>), grid, dim3(DEC_THREADS), shmem, s,
                       static_cast<const T *>(a.q), static_cast<const T *>(a.k),
                       static_cast<const T *>(a.v), a.seqlens_k, a.heads_q, a.heads_kv,
                       a.max_seqlen_k, a.split, lay.chunks, a.scale * kLog2e,
                       reinterpret_cast<float *>(ws + lay.off_m), reinterpret_cast<float *>(ws + lay.off_l),
                       reinterpret_cast<float *>(ws + lay.off_o));
    return hipGetLastError();
}

template <typename T, int HD>
hipError_t launch_split_g(const DecodeArgs &a, const DecodeLayout &lay, hipStream_t s) {
    switch (a.heads_q / a.heads_kv) {
        case 1: return launch_split<T, HD, 1>(a, lay, s);
        case 2: return launch_split<T, HD, 2>(a, lay, s);
        case 4: return launch_split<T, HD, 4>(a, lay, s);
        default: return launch_split<T, HD, 8>(a, lay, s);
    }
}

}  // namespace

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

DecodeLayout decode_layout(int64_t batch, int64_t heads_q, int64_t max_seqlen_k, int64_t head_dim,
                           int64_t split) {
    DecodeLayout lay{};
    lay.rows = batch * heads_q;
    lay.chunks = (int32_t)((max_seqlen_k + split - 1) / split);
    const size_t n = (size_t)lay.rows * (size_t)lay.chunks;
    lay.off_m = 0;
    lay.off_l = align256(n * sizeof(float));
    lay.off_o = lay.off_l + align256(n * sizeof(float));
    lay.total = lay.off_o + align256(n * (size_t)head_dim * sizeof(float));
    return lay;
}

hipError_t launch_decode_split(const DecodeArgs &a, const DecodeLayout &lay, hipStream_t s) {
    if (a.dtype == 1)
        return a.head_dim == 64 ? launch_split_g<uint16_t, 64>(a, lay, s)
                                : launch_split_g<uint16_t, 128>(a, lay, s);
    return a.head_dim == 64 ? launch_split_g<float, 64>(a, lay, s)
                            : launch_split_g<float, 128>(a, lay, s);
}

hipError_t launch_merge_partials(const MergeArgs &a, hipStream_t s) {
    if (a.rows == 0) return hipSuccess;
    int threads = ((a.head_dim + 63) / 64) * 64;
    if (threads < 128) threads = 128;
    const int grid = (int)(a.rows < 1048576 ? a.rows : 1048576);
    hipLaunchKernelGGL(merge_partials_kernel, dim3(grid), dim3(threads), 0, s, a.part_m, a.part_l,
                       a.part_o, a.rows, a.num_splits, a.head_dim, a.o, a.out_dtype, a.lse);
    return hipGetLastError();
}

}  // namespace osm
