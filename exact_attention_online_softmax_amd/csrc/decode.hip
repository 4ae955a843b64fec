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
// decode_split: one workgroup (4 waves) per (piece, kv head, batch).  All
// query heads that share the kv head (grouped-query attention) are served
// from one read of the piece's K and V.  Lanes are grouped LPK = head_dim/8
// per key, each lane owning 8 consecutive dims, so every wave load is a
// contiguous run of whole cache rows; the loads of a round of 64 keys are
// issued together before any is used.  Small workgroups with few registers
// keep six of them on a CU, so the loads of some overlap the arithmetic of
// others (the piece's keys are streamed in rounds rather than all held at
// once).  Phase 1 computes the piece's
// scores (bf16 dot products with v_dot2_f32_bf16, 16-lane sums with DPP row
// shifts) into LDS; the piece maximum and sum follow; phase 2 accumulates
// sum p_j v_j in fp32.
// Pieces wholly past the valid length write the identity (m = -inf, l = 0).
//
// merge_partials: one workgroup per row; the row's largest piece maximum is
// the common reference, every piece is weighted by exp(m_c - m) and added;
// an empty piece's l and O~ are loaded with the others but dropped by a
// select, so whatever they hold (NaN included) never reaches a sum.  Then
// o = O~ / l once and LSE = m + log l ([P3] "From weights to outputs").
#include <mutex>

#include "osm_device.h"
#include "osm_internal.h"

namespace osm {

// The decode workspace of osm_attn_decode_splitkv_noalloc: one copy per GPU,
// allocated by the runtime when the library's code object is loaded there and
// held until the process ends.  Host code never passes `scratch` itself to a
// kernel (on the host the name is only a stand-in): decode_scratch() looks up
// each device's own address once and every launch uses that.
static __device__ __align__(256) unsigned char scratch[kDecodeScratchBytes];

namespace {

constexpr int DEC_THREADS = 256;
constexpr int DEC_WAVES = DEC_THREADS / 64;
constexpr int DEC_ROUND = 64;       // keys whose loads are issued together

__device__ __forceinline__ int clampi(int v, int lo, int hi) { return v < lo ? lo : (v > hi ? hi : v); }

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Eight consecutive elements of a cache or query row, kept as loaded.
template <typename T> struct Row8;
template <> struct Row8<uint16_t> {        // bf16: four packed pairs
    uint4 w;
    __device__ __forceinline__ void load(const uint16_t *p) { w = *reinterpret_cast<const uint4 *>(p); }
    __device__ __forceinline__ void load_nt(const uint16_t *p) {
        typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
        const u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
        w = make_uint4(t[0], t[1], t[2], t[3]);
    }
    // sum_e q_e x_e with q, x both bf16 rows (v_dot2_f32_bf16, fp32 accumulate)
    __device__ __forceinline__ float dot(const Row8 &q) const {
        float a = 0.0f;
        a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, q.w.x), __builtin_bit_cast(bf16x2_t, w.x), a, false);
        a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, q.w.y), __builtin_bit_cast(bf16x2_t, w.y), a, false);
        a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, q.w.z), __builtin_bit_cast(bf16x2_t, w.z), a, false);
        a = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, q.w.w), __builtin_bit_cast(bf16x2_t, w.w), a, false);
        return a;
    }
    __device__ __forceinline__ void axpy(float p, float (&acc)[8]) const {
        acc[0] = fmaf(p, bf16_lo(w.x), acc[0]); acc[1] = fmaf(p, bf16_hi(w.x), acc[1]);
        acc[2] = fmaf(p, bf16_lo(w.y), acc[2]); acc[3] = fmaf(p, bf16_hi(w.y), acc[3]);
        acc[4] = fmaf(p, bf16_lo(w.z), acc[4]); acc[5] = fmaf(p, bf16_hi(w.z), acc[5]);
        acc[6] = fmaf(p, bf16_lo(w.w), acc[6]); acc[7] = fmaf(p, bf16_hi(w.w), acc[7]);
    }
};
template <> struct Row8<float> {
    float4 a, b;
    __device__ __forceinline__ void load(const float *p) {
        a = *reinterpret_cast<const float4 *>(p);
        b = *reinterpret_cast<const float4 *>(p + 4);
    }
    __device__ __forceinline__ void load_nt(const float *p) {
        typedef float f32x4 __attribute__((ext_vector_type(4)));
        const f32x4 x = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(p));
        const f32x4 y = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(p + 4));
        a = make_float4(x[0], x[1], x[2], x[3]);
        b = make_float4(y[0], y[1], y[2], y[3]);
    }
    __device__ __forceinline__ float dot(const Row8 &q) const {
        float r = q.a.x * a.x;
        r = fmaf(q.a.y, a.y, r); r = fmaf(q.a.z, a.z, r); r = fmaf(q.a.w, a.w, r);
        r = fmaf(q.b.x, b.x, r); r = fmaf(q.b.y, b.y, r); r = fmaf(q.b.z, b.z, r);
        return fmaf(q.b.w, b.w, r);
    }
    __device__ __forceinline__ void axpy(float p, float (&acc)[8]) const {
        acc[0] = fmaf(p, a.x, acc[0]); acc[1] = fmaf(p, a.y, acc[1]);
        acc[2] = fmaf(p, a.z, acc[2]); acc[3] = fmaf(p, a.w, acc[3]);
        acc[4] = fmaf(p, b.x, acc[4]); acc[5] = fmaf(p, b.y, acc[5]);
        acc[6] = fmaf(p, b.z, acc[6]); acc[7] = fmaf(p, b.w, acc[7]);
    }
};

// Sum over each group of LPK consecutive lanes (LPK = 8 or 16) with DPP
// row shifts; the total lands in the group's last lane.
template <int LPK>
__device__ __forceinline__ float group_sum(float x) {
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x111, 0xF, 0xF, true));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x112, 0xF, 0xF, true));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x114, 0xF, 0xF, true));
    if (LPK == 16)
        x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x118, 0xF, 0xF, true));
    return x;
}

// K and V rows are read with nontemporal (streaming) loads: every row is read
// exactly once.  A decode step reads a cache far larger than L2 and the MALL
// (6% faster measured); an extend call was 2x faster with them when its keys
// had been pushed out of the caches by other work, and within 3% when they
// were still on chip.
template <typename T, int HD, int G>
__global__ void __launch_bounds__(DEC_THREADS)
decode_split(const T *__restrict__ Q, const T *__restrict__ K, const T *__restrict__ V,
             const int32_t *__restrict__ seqlens_k, int Hq, int Hkv, int Lmax, int split,
             int chunks, float scale_log2, float *__restrict__ ws_m, float *__restrict__ ws_l,
             float *__restrict__ ws_o) {
    constexpr int LPK = HD / 8;                 // lanes per key
    constexpr int KPW = 64 / LPK;               // keys per wave step
    constexpr int KPB = KPW * DEC_WAVES;        // keys per workgroup step
    constexpr int R = DEC_ROUND / KPB;          // steps per round
    extern __shared__ float sc[];               // scores, then weights: [G][split]
    __shared__ float red_o[DEC_WAVES][G][HD];   // cross-wave partial outputs
    __shared__ float stat_m[G], stat_l[G];

    const int c = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
    const int L = __builtin_amdgcn_readfirstlane(seqlens_k ? clampi(seqlens_k[b], 0, Lmax) : Lmax);
    const int start = c * split;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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
    const int kbase = wave * KPW + kslot;       // key of step 0 (round-relative)

    const T *Kp = K + ((size_t)(b * Hkv + g) * Lmax + start) * HD + d0;
    const T *Vp = V + ((size_t)(b * Hkv + g) * Lmax + start) * HD + d0;

    Row8<T> q[G];
#pragma unroll
    for (int hh = 0; hh < G; ++hh) q[hh].load(Q + (row0 + hh) * HD + d0);

    // Every load of a round is issued before any is used.  Keys past n are
    // clamped to the last valid key (in bounds, finite) and never used.
    Row8<T> kr[R], vr[R];
    auto kv_load = [&](Row8<T> &r, const T *p) __attribute__((always_inline)) { r.load_nt(p); };
    const bool one_round = (n <= DEC_ROUND);
#pragma unroll
    for (int u = 0; u < R; ++u) kv_load(kr[u], Kp + (size_t)min(kbase + u * KPB, n - 1) * HD);
    if (one_round)
#pragma unroll
        for (int u = 0; u < R; ++u) kv_load(vr[u], Vp + (size_t)min(kbase + u * KPB, n - 1) * HD);

    // ---- phase 1: scores (base-2 scaled units) into LDS ------------------
    for (int r0 = 0; r0 < n; r0 += DEC_ROUND) {
        if (r0 > 0)
#pragma unroll
            for (int u = 0; u < R; ++u) kv_load(kr[u], Kp + (size_t)min(r0 + kbase + u * KPB, n - 1) * HD);
#pragma unroll
        for (int u = 0; u < R; ++u) {
            const int kk = r0 + kbase + u * KPB;
            float dot[G];
#pragma unroll
            for (int hh = 0; hh < G; ++hh) dot[hh] = group_sum<LPK>(kr[u].dot(q[hh]));
            if ((lane % LPK) == LPK - 1 && kk < n)
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
    for (int r0 = 0; r0 < n; r0 += DEC_ROUND) {
        if (!one_round)
#pragma unroll
            for (int u = 0; u < R; ++u) kv_load(vr[u], Vp + (size_t)min(r0 + kbase + u * KPB, n - 1) * HD);
#pragma unroll
        for (int u = 0; u < R; ++u) {
            const int kk = r0 + kbase + u * KPB;
            if (kk < n) {
#pragma unroll
                for (int hh = 0; hh < G; ++hh) vr[u].axpy(sc[hh * split + kk], acc[hh]);
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
// One workgroup (4 waves) per row.  The row maximum m over the pieces is
// found first, so every piece's weight exp(m_c - m) is final and the pieces
// can be accumulated in any order with no rescaling; waves take pieces
// c = wave, wave + 4, ..., lanes own NDL dims each, and the four partial sums
// are added through LDS.  Empty pieces (m_c = -inf) get weight 0 through a
// select (their l and O~ are loaded, so their memory must be valid).
constexpr int MRG_THREADS = 256;
constexpr int MRG_WAVES = MRG_THREADS / 64;

// STATE: the row's persisted summary (state_m, state_l, state_o) is one more
// piece of the merge, and the merged summary is written back to it
// unnormalized (the streaming extend) instead of o and LSE.
template <int NDL, bool STATE>
__global__ void __launch_bounds__(MRG_THREADS)
merge_partials_kernel(const float *__restrict__ pm, const float *__restrict__ pl,
                      const float *__restrict__ po, int64_t rows, int C, int HD,
                      void *__restrict__ out, int out_bf16, float *__restrict__ lse,
                      float *state_m, float *state_l, float *state_o) {
    __shared__ float red_acc[MRG_WAVES][NDL * 64];
    __shared__ float red_s[MRG_WAVES];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    for (int64_t r = blockIdx.x; r < rows; r += gridDim.x) {
        const float *pmr = pm + r * C;
        // row maximum
        float mx = kNegInf;
        for (int c = tid; c < C; c += MRG_THREADS) mx = fmaxf(mx, pmr[c]);
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
        if (lane == 0) red_s[wave] = mx;
        __syncthreads();
        mx = kNegInf;
#pragma unroll
        for (int w = 0; w < MRG_WAVES; ++w) mx = fmaxf(mx, red_s[w]);
        __syncthreads();
        const float ms = STATE ? state_m[r] : kNegInf;
        const float m = fmaxf(mx, ms);
        float acc[NDL];
#pragma unroll
        for (int k = 0; k < NDL; ++k) acc[k] = 0.0f;
        float lsum = 0.0f;
        if (m != kNegInf) {
            // Every load of a group of U pieces is issued before any weight
            // is known (one memory round trip per group); a piece with m = -inf
            // is the empty set and is dropped by a select, so whatever its l
            // and O~ slots hold never reaches the sums.
            constexpr int U = 8;
            for (int c0 = wave; c0 < C; c0 += MRG_WAVES * U) {
                float mc[U], lv[U], ov[U][NDL];
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int c = c0 + u * MRG_WAVES;
                    mc[u] = kNegInf;
                    lv[u] = 0.0f;
#pragma unroll
                    for (int k = 0; k < NDL; ++k) ov[u][k] = 0.0f;
                    if (c < C) {
                        mc[u] = pmr[c];
                        lv[u] = pl[r * C + c];
                        const float *oc = po + (r * C + c) * HD;
#pragma unroll
                        for (int k = 0; k < NDL; ++k)
                            if (lane + 64 * k < HD) ov[u][k] = oc[lane + 64 * k];
                    }
                }
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const bool live = mc[u] != kNegInf;
                    const float w = live ? exp_acc(mc[u] - m) : 0.0f;
                    lsum = live ? fmaf(w, lv[u], lsum) : lsum;
#pragma unroll
                    for (int k = 0; k < NDL; ++k) acc[k] = live ? fmaf(w, ov[u][k], acc[k]) : acc[k];
                }
            }
        }
        if (STATE && wave == 0 && ms != kNegInf) {
            // the persisted summary, weighted like any other piece
            const float w = exp_acc(ms - m);
            lsum = fmaf(w, state_l[r], lsum);
#pragma unroll
            for (int k = 0; k < NDL; ++k)
                if (lane + 64 * k < HD) acc[k] = fmaf(w, state_o[r * HD + lane + 64 * k], acc[k]);
        }
#pragma unroll
        for (int k = 0; k < NDL; ++k) red_acc[wave][lane + 64 * k] = acc[k];
        if (lane == 0) red_s[wave] = lsum;
        __syncthreads();
        float l = 0.0f;
#pragma unroll
        for (int w = 0; w < MRG_WAVES; ++w) l += red_s[w];
        if (STATE) {
            // write the merged (m, l, O~) back; every read of this row's
            // state happened before the barrier above
            for (int d = tid; d < HD; d += MRG_THREADS) {
                float o = 0.0f;
#pragma unroll
                for (int w = 0; w < MRG_WAVES; ++w) o += red_acc[w][d];
                state_o[r * HD + d] = (m == kNegInf) ? 0.0f : o;
            }
            if (tid == 0) {
                state_m[r] = m;
                state_l[r] = (m == kNegInf) ? 0.0f : l;
            }
            __syncthreads();   // red_acc / red_s are reused by the next row
            continue;
        }
        const bool valid = (m != kNegInf) && (l > 0.0f);
        const float inv = valid ? 1.0f / l : 0.0f;
        for (int d = tid; d < HD; d += MRG_THREADS) {
            float o = 0.0f;
#pragma unroll
            for (int w = 0; w < MRG_WAVES; ++w) o += red_acc[w][d];
            o *= inv;
            if (out_bf16) static_cast<uint16_t *>(out)[r * HD + d] = f32_to_bf16(o);
            else static_cast<float *>(out)[r * HD + d] = o;
        }
        if (lse && tid == 0) lse[r] = valid ? m + logf(l) : kNegInf;
        __syncthreads();   // red_acc / red_s are reused by the next row
    }
}

// Rows of at most kSmallC pieces (the streaming extend's chunks, short
// decodes): one wave per row, four rows per workgroup, and every load of a
// row (the pieces' m, l and O~, and the persisted summary) issued before any
// is used, so a row costs one memory round trip.  Empty pieces get weight 0
// through a select, as in merge_partials_kernel; the pieces are summed in
// order, then the persisted summary.
constexpr int kSmallC = 8;

template <int NDL, bool STATE>
__global__ void __launch_bounds__(MRG_THREADS)
merge_partials_small(const float *__restrict__ pm, const float *__restrict__ pl,
                     const float *__restrict__ po, int64_t rows, int C, int HD,
                     void *__restrict__ out, int out_bf16, float *__restrict__ lse,
                     float *state_m, float *state_l, float *state_o) {
    const int lane = threadIdx.x & 63;
    const int64_t r = (int64_t)blockIdx.x * MRG_WAVES + (threadIdx.x >> 6);
    if (r >= rows) return;
    float mc[kSmallC], lc[kSmallC], oc[kSmallC][NDL];
#pragma unroll
    for (int c = 0; c < kSmallC; ++c) {
        mc[c] = kNegInf;
        lc[c] = 0.0f;
#pragma unroll
        for (int k = 0; k < NDL; ++k) oc[c][k] = 0.0f;
        if (c < C) {
            mc[c] = pm[r * C + c];
            lc[c] = pl[r * C + c];
#pragma unroll
            for (int k = 0; k < NDL; ++k)
                if (lane + 64 * k < HD) oc[c][k] = po[(r * C + c) * HD + lane + 64 * k];
        }
    }
    float ms = kNegInf, ls = 0.0f, os[NDL];
#pragma unroll
    for (int k = 0; k < NDL; ++k) os[k] = 0.0f;
    if (STATE) {
        ms = state_m[r];
        ls = state_l[r];
#pragma unroll
        for (int k = 0; k < NDL; ++k)
            if (lane + 64 * k < HD) os[k] = state_o[r * HD + lane + 64 * k];
    }
    float m = ms;
#pragma unroll
    for (int c = 0; c < kSmallC; ++c) m = fmaxf(m, mc[c]);
    float acc[NDL], lsum = 0.0f;
#pragma unroll
    for (int k = 0; k < NDL; ++k) acc[k] = 0.0f;
    if (m != kNegInf) {
#pragma unroll
        for (int c = 0; c < kSmallC; ++c) {
            const bool live = mc[c] != kNegInf;
            const float w = live ? exp_acc(mc[c] - m) : 0.0f;
            lsum = live ? fmaf(w, lc[c], lsum) : lsum;
#pragma unroll
            for (int k = 0; k < NDL; ++k) acc[k] = live ? fmaf(w, oc[c][k], acc[k]) : acc[k];
        }
        if (STATE && ms != kNegInf) {
            const float w = exp_acc(ms - m);
            lsum = fmaf(w, ls, lsum);
#pragma unroll
            for (int k = 0; k < NDL; ++k) acc[k] = fmaf(w, os[k], acc[k]);
        }
    }
    if (STATE) {
        // every read of this row's summary above precedes these writes
#pragma unroll
        for (int k = 0; k < NDL; ++k)
            if (lane + 64 * k < HD) state_o[r * HD + lane + 64 * k] = (m == kNegInf) ? 0.0f : acc[k];
        if (lane == 0) {
            state_m[r] = m;
            state_l[r] = (m == kNegInf) ? 0.0f : lsum;
        }
        return;
    }
    const bool valid = (m != kNegInf) && (lsum > 0.0f);
    const float inv = valid ? 1.0f / lsum : 0.0f;
#pragma unroll
    for (int k = 0; k < NDL; ++k) {
        const int d = lane + 64 * k;
        if (d < HD) {
            const float o = acc[k] * inv;
            if (out_bf16) static_cast<uint16_t *>(out)[r * HD + d] = f32_to_bf16(o);
            else static_cast<float *>(out)[r * HD + d] = o;
        }
    }
    if (lse && lane == 0) lse[r] = valid ? m + logf(lsum) : kNegInf;
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

hipError_t decode_scratch(void **ptr) {
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void *addr[kMaxDevices] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        // with `dev` current: this device's copy of the array
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        addr[dev] = p;
    }
    *ptr = addr[dev];
    return hipSuccess;
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
    const int ndl = (a.head_dim + 63) / 64;
    const bool st = a.state_m != nullptr;
    if (a.num_splits <= kSmallC && ndl <= 2) {
        const unsigned g = (unsigned)((a.rows + MRG_WAVES - 1) / MRG_WAVES);
#define OSM_MERGE_SMALL(N, ST)                                                                           \
    hipLaunchKernelGGL((merge_partials_small<N, ST>), dim3(g), dim3(MRG_THREADS), 0, s, a.part_m, a.part_l, \
                       a.part_o, a.rows, a.num_splits, a.head_dim, a.o, a.out_dtype, a.lse, a.state_m,     \
                       a.state_l, a.state_o)
        if (st) {
            if (ndl <= 1) OSM_MERGE_SMALL(1, true);
            else OSM_MERGE_SMALL(2, true);
        } else if (ndl <= 1) OSM_MERGE_SMALL(1, false);
        else OSM_MERGE_SMALL(2, false);
#undef OSM_MERGE_SMALL
        return hipGetLastError();
    }
    const int grid = (int)(a.rows < 1048576 ? a.rows : 1048576);
#define OSM_MERGE_LAUNCH(N, ST)                                                                        \
    hipLaunchKernelGGL((merge_partials_kernel<N, ST>), dim3(grid), dim3(MRG_THREADS), 0, s, a.part_m,  \
                       a.part_l, a.part_o, a.rows, a.num_splits, a.head_dim, a.o, a.out_dtype, a.lse, \
                       a.state_m, a.state_l, a.state_o)
    if (st) {
        if (ndl <= 1) OSM_MERGE_LAUNCH(1, true);
        else OSM_MERGE_LAUNCH(2, true);
    } else if (ndl <= 1) OSM_MERGE_LAUNCH(1, false);
    else if (ndl <= 2) OSM_MERGE_LAUNCH(2, false);
    else if (ndl <= 4) OSM_MERGE_LAUNCH(4, false);
    else OSM_MERGE_LAUNCH(8, false);
#undef OSM_MERGE_LAUNCH
    return hipGetLastError();
}

}  // namespace osm
