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
// it drops out and its o is never read (it may hold any bits).
//
// One wavefront per row.  Pass 1 spreads the pieces over the lanes for the
// maximum and the sum of exponentials (wave reductions); pass 2 walks the
// pieces with the row's weights, each lane owning VEC consecutive dims per
// 64 * VEC-dim chunk, so every load of a piece row is one contiguous run.
// fp32 accumulation; exponentials with the accurate exp_acc.
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
            if (l == kNegInf) continue;                  // empty piece: o_s unread
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
