// merge_lse.hip -- combine normalized attention results of disjoint key
// sets in log-sum-exp form, gfx950.
//
// [P3] "The same merge, in log-sum-exp form": a kernel that processed one
// piece of a row's keys returns the normalized output o together with the
// piece's log-sum-exp; two such results merge as
//   lse = log(e^lse_A + e^lse_B),  o = e^(lse_A - lse) o_A + e^(lse_B - lse) o_B,
// which is the same merge as [P3] "Merging partial results" with each piece
// already divided by its own sum.  The merge is associative, so S pieces
// combine at once: lse = M + log sum_s e^(lse_s - M) with M = max_s lse_s,
// o = sum_s e^(lse_s - lse) o_s.  A piece with lse = -inf is the empty set:
// it drops out whatever its o holds (any bits, NaN included).
//
// Rows of a power-of-two number of 16-byte vectors (head_dim 128 in bf16,
// for example) take merge_lse_rows: a row per group of lanes, several rows
// per wave, the loads of eight pieces in flight together.  Other head_dims
// take merge_lse_kernel: one wavefront per row, the pieces spread over the
// lanes for the maximum and the sum (wave reductions), then walked with the
// row's weights, each lane owning VEC consecutive dims per 64 * VEC-dim
// chunk.  fp32 accumulation; exponentials with the accurate exp_acc.
#include "osm_device.h"
#include "osm_internal.h"

namespace osm {

namespace {

constexpr int MLSE_THREADS = 256;
constexpr int MLSE_WAVES = MLSE_THREADS / 64;

template <typename T> struct Elem;
template <> struct Elem<float> {
    static __device__ __forceinline__ float get(const float *p) { return *p; }
    static __device__ __forceinline__ void get2(const float *p, float &a, float &b) {
        const float2 v = *reinterpret_cast<const float2 *>(p);
        a = v.x;
        b = v.y;
    }
    static __device__ __forceinline__ void put(float *p, float a) { *p = a; }
    static __device__ __forceinline__ void put2(float *p, float a, float b) {
        *reinterpret_cast<float2 *>(p) = make_float2(a, b);
    }
};
template <> struct Elem<uint16_t> {   // bf16 bits
    static __device__ __forceinline__ float get(const uint16_t *p) { return __uint_as_float((uint32_t)*p << 16); }
    static __device__ __forceinline__ void get2(const uint16_t *p, float &a, float &b) {
        const uint32_t w = *reinterpret_cast<const uint32_t *>(p);
        a = bf16_lo(w);
        b = bf16_hi(w);
    }
    static __device__ __forceinline__ void put(uint16_t *p, float a) { *p = f32_to_bf16(a); }
    static __device__ __forceinline__ void put2(uint16_t *p, float a, float b) {
        *reinterpret_cast<uint32_t *>(p) = pack_bf16x2(a, b);
    }
};

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) x = fmaxf(x, __shfl_xor(x, off, 64));
    return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
    return x;
}

// VEC dims per lane per chunk (2 when head_dim is even), NK chunks of 64 * VEC dims
template <typename TI, typename TO, int VEC, int NK>
__global__ void __launch_bounds__(MLSE_THREADS)
merge_lse_kernel(const TI *__restrict__ op, const float *__restrict__ lp, int64_t rows, int S,
                 int hd, TO *__restrict__ o, float *__restrict__ lse) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t part_stride = rows * hd;
    for (int64_t r = (int64_t)blockIdx.x * MLSE_WAVES + wave; r < rows; r += (int64_t)gridDim.x * MLSE_WAVES) {
        // ---- pass 1: L = M + log sum_s e^(lse_s - M) over non-empty pieces
        float mx = kNegInf;
        for (int s = lane; s < S; s += 64) mx = fmaxf(mx, lp[(int64_t)s * rows + r]);
        mx = wave_max(mx);
        TO *orow = o + r * hd;
        if (mx == kNegInf) {          // every piece empty: o = 0, lse = -inf
#pragma unroll
            for (int k = 0; k < NK; ++k)
#pragma unroll
                for (int v = 0; v < VEC; ++v) {
                    const int e = (64 * k + lane) * VEC + v;
                    if (e < hd) Elem<TO>::put(orow + e, 0.0f);
                }
            if (lse && lane == 0) lse[r] = kNegInf;
            continue;
        }
        float sum = 0.0f;
        for (int s = lane; s < S; s += 64) {
            const float l = lp[(int64_t)s * rows + r];
            if (l != kNegInf) sum += exp_acc(l - mx);
        }
        sum = wave_sum(sum);
        const float L = mx + logf(sum);

        // ---- pass 2: o = sum_s e^(lse_s - L) o_s -----------------------------
        float acc[NK][VEC];
#pragma unroll
        for (int k = 0; k < NK; ++k)
#pragma unroll
            for (int v = 0; v < VEC; ++v) acc[k][v] = 0.0f;
        const TI *base = op + r * hd;
        for (int s = 0; s < S; ++s) {
            const float l = lp[(int64_t)s * rows + r];   // the same for every lane
            if (l == kNegInf) continue;                  // empty piece: o_s not read
            const float w = exp_acc(l - L);
            const TI *prow = base + (int64_t)s * part_stride;
#pragma unroll
            for (int k = 0; k < NK; ++k) {
                const int e = (64 * k + lane) * VEC;
                if (e < hd) {
                    if (VEC == 2) {
                        float a, b;
                        Elem<TI>::get2(prow + e, a, b);
                        acc[k][0] = fmaf(w, a, acc[k][0]);
                        acc[k][VEC - 1] = fmaf(w, b, acc[k][VEC - 1]);
                    } else {
                        acc[k][0] = fmaf(w, Elem<TI>::get(prow + e), acc[k][0]);
                    }
                }
            }
        }
#pragma unroll
        for (int k = 0; k < NK; ++k) {
            const int e = (64 * k + lane) * VEC;
            if (e < hd) {
                if (VEC == 2) Elem<TO>::put2(orow + e, acc[k][0], acc[k][VEC - 1]);
                else Elem<TO>::put(orow + e, acc[k][0]);
            }
        }
        if (lse && lane == 0) lse[r] = L;
    }
}

// Fast path: each row is LPR lanes x 16 bytes of o (VE elements per lane),
// 64 / LPR rows per wave.  Up to 8 pieces: every load of a row is issued at
// once.  More pieces go in batches of 8: their lse values are
// read by every lane of the row (one cache line), their o vectors are all
// requested before any is used.  An empty piece gets weight 0 through a
// select, so whatever its o holds (NaN included) never reaches the sum.
template <typename TI, typename TO, int LPR>
__global__ void __launch_bounds__(MLSE_THREADS)
merge_lse_rows(const TI *__restrict__ op, const float *__restrict__ lp, int64_t rows, int S,
               TO *__restrict__ o, float *__restrict__ lse) {
    constexpr int VE = 16 / sizeof(TI);          // elements per lane
    constexpr int HD = LPR * VE;                 // head_dim
    constexpr int RPW = 64 / LPR;                // rows per wave
    constexpr int BATCH = 8;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int sub = lane / LPR, part = lane % LPR;
    const int64_t part_stride = rows * HD;
    const int64_t step = (int64_t)gridDim.x * MLSE_WAVES * RPW;
    for (int64_t r0 = ((int64_t)blockIdx.x * MLSE_WAVES + wave) * RPW; r0 < rows; r0 += step) {
        const int64_t r = r0 + sub;
        const bool live = r < rows;
        const int64_t rc = live ? r : rows - 1;  // rows past the end read the last row, write nothing
        const TI *base = op + rc * HD + part * VE;
        typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
        if (S <= BATCH) {
            // one memory round trip: every o vector and lse value of the row
            // is requested before any is used (each piece is read once:
            // nontemporal loads)
            uint4 x[BATCH];
            float l[BATCH];
#pragma unroll
            for (int k = 0; k < BATCH; ++k) {
                const int sk = (k < S) ? k : S - 1;
                const u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(base + (int64_t)sk * part_stride));
                x[k] = make_uint4(t[0], t[1], t[2], t[3]);
                l[k] = (k < S) ? lp[(int64_t)k * rows + rc] : kNegInf;
            }
            float mx = kNegInf;
#pragma unroll
            for (int k = 0; k < BATCH; ++k) mx = fmaxf(mx, l[k]);
            float sum = 0.0f;
#pragma unroll
            for (int k = 0; k < BATCH; ++k) sum += (l[k] == kNegInf) ? 0.0f : exp_acc(l[k] - mx);
            const float L = (mx == kNegInf) ? kNegInf : mx + logf(sum);
            float acc[VE];
#pragma unroll
            for (int e = 0; e < VE; ++e) acc[e] = 0.0f;
#pragma unroll
            for (int k = 0; k < BATCH; ++k) {
                // an empty piece (or every piece empty: L = -inf) weighs 0
                const float w = (l[k] == kNegInf) ? 0.0f : exp_acc(l[k] - L);
                float v[VE];
                if constexpr (sizeof(TI) == 2) {
                    const uint32_t q[4] = {x[k].x, x[k].y, x[k].z, x[k].w};
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        v[2 * e] = bf16_lo(q[e]);
                        v[2 * e + 1] = bf16_hi(q[e]);
                    }
                } else {
                    v[0] = __uint_as_float(x[k].x);
                    v[1] = __uint_as_float(x[k].y);
                    v[2] = __uint_as_float(x[k].z);
                    v[3] = __uint_as_float(x[k].w);
                }
#pragma unroll
                for (int e = 0; e < VE; ++e) acc[e] = (w == 0.0f) ? acc[e] : fmaf(w, v[e], acc[e]);
            }
            if (live) {
                TO *orow = o + r * HD + part * VE;
#pragma unroll
                for (int e = 0; e < VE; e += 2) Elem<TO>::put2(orow + e, acc[e], acc[e + 1]);
                if (lse && part == 0) lse[r] = L;
            }
            continue;
        }
        // ---- pass 1: M = max lse_s, then L = M + log sum_s e^(lse_s - M) ----
        float mx = kNegInf;
        for (int s0 = 0; s0 < S; s0 += BATCH) {
            float l[BATCH];
#pragma unroll
            for (int k = 0; k < BATCH; ++k) l[k] = (s0 + k < S) ? lp[(int64_t)(s0 + k) * rows + rc] : kNegInf;
#pragma unroll
            for (int k = 0; k < BATCH; ++k) mx = fmaxf(mx, l[k]);
        }
        float sum = 0.0f;
        if (mx != kNegInf)
            for (int s0 = 0; s0 < S; s0 += BATCH) {
                float l[BATCH];
#pragma unroll
                for (int k = 0; k < BATCH; ++k) l[k] = (s0 + k < S) ? lp[(int64_t)(s0 + k) * rows + rc] : kNegInf;
#pragma unroll
                for (int k = 0; k < BATCH; ++k) sum += (l[k] == kNegInf) ? 0.0f : exp_acc(l[k] - mx);
            }
        const float L = (mx == kNegInf) ? kNegInf : mx + logf(sum);
        // ---- pass 2: o = sum_s e^(lse_s - L) o_s ----------------------------
        float acc[VE];
#pragma unroll
        for (int e = 0; e < VE; ++e) acc[e] = 0.0f;
        if (mx != kNegInf)
            for (int s0 = 0; s0 < S; s0 += BATCH) {
                float w[BATCH];
                uint4 x[BATCH];
#pragma unroll
                for (int k = 0; k < BATCH; ++k) {
                    const int sk = (s0 + k < S) ? s0 + k : S - 1;
                    // each piece is read once: nontemporal (streaming) loads, 5% faster
                    const u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(base + (int64_t)sk * part_stride));
                    x[k] = make_uint4(t[0], t[1], t[2], t[3]);
                }
#pragma unroll
                for (int k = 0; k < BATCH; ++k) {
                    const float l = (s0 + k < S) ? lp[(int64_t)(s0 + k) * rows + rc] : kNegInf;
                    w[k] = (l == kNegInf) ? 0.0f : exp_acc(l - L);
                }
#pragma unroll
                for (int k = 0; k < BATCH; ++k) {
                    float v[VE];
                    if constexpr (sizeof(TI) == 2) {
                        const uint32_t q[4] = {x[k].x, x[k].y, x[k].z, x[k].w};
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            v[2 * e] = bf16_lo(q[e]);
                            v[2 * e + 1] = bf16_hi(q[e]);
                        }
                    } else {
                        v[0] = __uint_as_float(x[k].x);
                        v[1] = __uint_as_float(x[k].y);
                        v[2] = __uint_as_float(x[k].z);
                        v[3] = __uint_as_float(x[k].w);
                    }
#pragma unroll
                    for (int e = 0; e < VE; ++e) acc[e] = (w[k] == 0.0f) ? acc[e] : fmaf(w[k], v[e], acc[e]);
                }
            }
        if (live) {
            TO *orow = o + r * HD + part * VE;
#pragma unroll
            for (int e = 0; e < VE; e += 2) Elem<TO>::put2(orow + e, acc[e], acc[e + 1]);
            if (lse && part == 0) lse[r] = L;
        }
    }
}

template <typename TI, typename TO, int VEC>
hipError_t launch_typed(const MergeLseArgs &a, hipStream_t s, int grid) {
    const int nk = (a.head_dim + 64 * VEC - 1) / (64 * VEC);
    const TI *op = static_cast<const TI *>(a.o_parts);
    TO *o = static_cast<TO *>(a.o);
#define OSM_MLSE(N)                                                                               \
    hipLaunchKernelGGL((merge_lse_kernel<TI, TO, VEC, N>), dim3(grid), dim3(MLSE_THREADS), 0, s, op, \
                       a.lse_parts, a.rows, a.num_parts, a.head_dim, o, a.lse)
    if (nk <= 1) OSM_MLSE(1);
    else if (nk <= 2) OSM_MLSE(2);
    else if (nk <= 4) OSM_MLSE(4);
    else OSM_MLSE(8);
#undef OSM_MLSE
    return hipGetLastError();
}

template <typename TI, typename TO>
hipError_t launch_vec(const MergeLseArgs &a, hipStream_t s, int grid) {
    // fast path when a row is a power-of-two number (<= 64) of 16-byte vectors
    constexpr int VE = 16 / sizeof(TI);
    const int lpr = a.head_dim / VE;
    if (a.head_dim % VE == 0 && lpr <= 64 && (lpr & (lpr - 1)) == 0) {
        const int rpw = 64 / lpr;
        const int64_t want = (a.rows + (int64_t)MLSE_WAVES * rpw - 1) / ((int64_t)MLSE_WAVES * rpw);
        const int g = (int)(want < 65536 ? want : 65536);
        const TI *op = static_cast<const TI *>(a.o_parts);
        TO *o = static_cast<TO *>(a.o);
#define OSM_MLSE_ROWS(N)                                                                              \
    hipLaunchKernelGGL((merge_lse_rows<TI, TO, N>), dim3(g), dim3(MLSE_THREADS), 0, s, op, a.lse_parts, \
                       a.rows, a.num_parts, o, a.lse)
        switch (lpr) {
        case 1: OSM_MLSE_ROWS(1); break;
        case 2: OSM_MLSE_ROWS(2); break;
        case 4: OSM_MLSE_ROWS(4); break;
        case 8: OSM_MLSE_ROWS(8); break;
        case 16: OSM_MLSE_ROWS(16); break;
        case 32: OSM_MLSE_ROWS(32); break;
        default: OSM_MLSE_ROWS(64); break;
        }
#undef OSM_MLSE_ROWS
        return hipGetLastError();
    }
    return (a.head_dim % 2 == 0) ? launch_typed<TI, TO, 2>(a, s, grid) : launch_typed<TI, TO, 1>(a, s, grid);
}

}  // namespace

hipError_t launch_merge_lse(const MergeLseArgs &a, hipStream_t s) {
    if (a.rows == 0) return hipSuccess;
    const int64_t want = (a.rows + MLSE_WAVES - 1) / MLSE_WAVES;
    const int grid = (int)(want < 65536 ? want : 65536);
    if (a.in_bf16) return a.out_bf16 ? launch_vec<uint16_t, uint16_t>(a, s, grid) : launch_vec<uint16_t, float>(a, s, grid);
    return a.out_bf16 ? launch_vec<float, uint16_t>(a, s, grid) : launch_vec<float, float>(a, s, grid);
}

}  // namespace osm
