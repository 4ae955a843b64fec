// softmax_rows.hip -- row softmax with the online normalizer, gfx950.
//
// [P3] "Two numbers that can be updated" / "The recurrence, and a proof that
// it is right": a running maximum m and a running sum l of exp(x - m),
// rescaled by exp(m_old - m_new) when the maximum grows; [P3] "Merging
// partial results": summaries of disjoint pieces of a row merge exactly, in
// any order.  [P3] "Three passes, and why that is a problem" counts memory
// accesses per element: safe softmax 4, the two-pass online normalizer 3.
//
// One workgroup per row.  Each lane owns a strided set of float4 vectors of
// the row (consecutive lanes read consecutive 16-byte vectors, so every wave
// load is a contiguous 1 KiB).  Two variants:
//
//  * resident (cols <= 4 * NV * blockDim): the row is read from HBM once and
//    stays in VGPRs.  Each lane summarizes its piece as (m_lane, l_lane) and
//    keeps e_i = exp(x_i - m_lane); the lane summaries are merged across the
//    wave (butterfly) and across waves (LDS); then y_i = e_i * exp(m_lane -
//    m) / l.  HBM traffic: one load and one store per element (8 B).
//
//  * streaming (any cols): pass 1 reads the row and runs the recurrence per
//    lane, one rescale per batch of four float4 vectors; lane summaries are
//    merged as above; pass 2 reads the row again and writes
//    y = exp(x - m) / l.  Memory accesses: two loads and one store per
//    element (12 B), the pages' count.  Used for rows too long to hold, and
//    for every row through osm_softmax_rows_twopass.
#include "osm_device.h"
#include "osm_internal.h"

namespace osm {

namespace {

constexpr int kMaxWaves = 16;   // blockDim <= 1024

// Merge the per-lane (m, l) of a whole workgroup; every thread gets the row's.
__device__ __forceinline__ void block_merge_ml(float &m, float &l, float *sm, float *sl) {
    wave_merge_ml(m, l);
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int nwaves = blockDim.x >> 6;
    if (lane == 0) {
        sm[wave] = m;
        sl[wave] = l;
    }
    __syncthreads();
    m = kNegInf;
    l = 0.0f;
    for (int w = 0; w < nwaves; ++w) merge_ml(m, l, sm[w], sl[w]);
    __syncthreads();   // sm/sl are reused by the next row
}

__device__ __forceinline__ float max4(float4 v) {
    return fmaxf(fmaxf(v.x, v.y), fmaxf(v.z, v.w));
}

// Load vector `vec` (elements 4*vec .. 4*vec+3) of a row; entries at or past
// `cols` read as -inf.  ALIGNED: the row start is 16-byte aligned.
template <bool ALIGNED>
__device__ __forceinline__ float4 load_vec(const float *row, int64_t vec, int64_t cols) {
    int64_t e = vec * 4;
    if (ALIGNED && e + 4 <= cols) return *reinterpret_cast<const float4 *>(row + e);
    float4 v;
    v.x = (e + 0 < cols) ? row[e + 0] : kNegInf;
    v.y = (e + 1 < cols) ? row[e + 1] : kNegInf;
    v.z = (e + 2 < cols) ? row[e + 2] : kNegInf;
    v.w = (e + 3 < cols) ? row[e + 3] : kNegInf;
    return v;
}

// The resident kernel reads each element exactly once: its loads are
// nontemporal (streaming), which measured 4% faster than cached loads.
template <bool ALIGNED>
__device__ __forceinline__ float4 load_vec_once(const float *row, int64_t vec, int64_t cols) {
    int64_t e = vec * 4;
    if (ALIGNED && e + 4 <= cols) {
        typedef float f32x4 __attribute__((ext_vector_type(4)));
        const f32x4 w = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(row + e));
        return make_float4(w[0], w[1], w[2], w[3]);
    }
    return load_vec<ALIGNED>(row, vec, cols);
}

template <bool ALIGNED>
__device__ __forceinline__ void store_vec(float *row, int64_t vec, int64_t cols, float4 v) {
    int64_t e = vec * 4;
    if (ALIGNED && e + 4 <= cols) {
        typedef float f32x4 __attribute__((ext_vector_type(4)));
        const f32x4 w = {v.x, v.y, v.z, v.w};
        __builtin_nontemporal_store(w, reinterpret_cast<f32x4 *>(row + e));
        return;
    }
    if (e + 0 < cols) row[e + 0] = v.x;
    if (e + 1 < cols) row[e + 1] = v.y;
    if (e + 2 < cols) row[e + 2] = v.z;
    if (e + 3 < cols) row[e + 3] = v.w;
}

template <int NV, bool ALIGNED>
__global__ void __launch_bounds__(1024)
softmax_rows_resident(const float *x, float *y, int64_t rows,
                      int64_t cols, int64_t ld_x, int64_t ld_y, float *__restrict__ row_max,
                      float *__restrict__ row_sum) {
    __shared__ float sm[kMaxWaves], sl[kMaxWaves];
    const int64_t nvec = (cols + 3) / 4;
    for (int64_t r = blockIdx.x; r < rows; r += gridDim.x) {
        const float *xr = x + r * ld_x;
        float4 v[NV];
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            int64_t vec = threadIdx.x + (int64_t)i * blockDim.x;
            v[i] = (vec < nvec) ? load_vec_once<ALIGNED>(xr, vec, cols)
                                : make_float4(kNegInf, kNegInf, kNegInf, kNegInf);
        }
        // this lane's piece: maximum, then e_i = exp(x_i - m_lane) and their sum
        float m_lane = kNegInf;
#pragma unroll
        for (int i = 0; i < NV; ++i) m_lane = fmaxf(m_lane, max4(v[i]));
        float l_lane = 0.0f;
        const bool empty = (m_lane == kNegInf);
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            v[i].x = empty ? 0.0f : exp_acc(v[i].x - m_lane);
            v[i].y = empty ? 0.0f : exp_acc(v[i].y - m_lane);
            v[i].z = empty ? 0.0f : exp_acc(v[i].z - m_lane);
            v[i].w = empty ? 0.0f : exp_acc(v[i].w - m_lane);
            l_lane += (v[i].x + v[i].y) + (v[i].z + v[i].w);
        }
        float m = m_lane, l = l_lane;
        block_merge_ml(m, l, sm, sl);
        // rebase this lane's numerators on the row maximum and divide once
        float w = (empty || m == kNegInf) ? 0.0f : exp_acc(m_lane - m) / l;
        float *yr = y + r * ld_y;
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            int64_t vec = threadIdx.x + (int64_t)i * blockDim.x;
            if (vec < nvec) {
                float4 o = make_float4(v[i].x * w, v[i].y * w, v[i].z * w, v[i].w * w);
                store_vec<ALIGNED>(yr, vec, cols, o);
            }
        }
        if (threadIdx.x == 0) {
            if (row_max) row_max[r] = m;
            if (row_sum) row_sum[r] = l;
        }
    }
}

// Buffer resource word 3 for raw (unformatted, unswizzled) dword access.
constexpr int kRsrcWord3 = 0x00020000;
constexpr int kAuxNontemporal = 2;   // cache-policy bit NT of a buffer access on gfx950

// The resident kernel for rows whose width is a multiple of four on 16-byte
// aligned rows: every vector is whole, so a lane's vectors are in or out of
// the row as a unit.  Loads and stores go through a buffer resource spanning
// exactly the row; its range check turns a vector past the end into a load of
// zeros and a dropped store, so there is no per-vector branch (the generic
// kernel above pays an exec-mask branch per vector and per element of a
// partial vector).  Vectors past the end are then set to -inf by a select.
// The range check covers the VGPR offset only, so each load's whole byte
// offset is carried there.
template <int NV>
__global__ void __launch_bounds__(1024)
softmax_rows_resident_whole(const float *x, float *y, int64_t rows, int64_t cols, int64_t ld_x,
                            int64_t ld_y, float *__restrict__ row_max, float *__restrict__ row_sum) {
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    __shared__ float sm[kMaxWaves], sl[kMaxWaves];
    const uint32_t bytes = (uint32_t)(cols * 4);            // <= 2^18: the plan keeps cols <= 65536
    const uint32_t off0 = threadIdx.x * 16u, step = blockDim.x * 16u;
    for (int64_t r = blockIdx.x; r < rows; r += gridDim.x) {
        const __amdgpu_buffer_rsrc_t xr =
            __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(x + r * ld_x), 0, (int)bytes, kRsrcWord3);
        float4 v[NV];
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const uint32_t off = off0 + i * step;
            const u32x4 w = __builtin_amdgcn_raw_buffer_load_b128(xr, off, 0, kAuxNontemporal);
            const bool in = off < bytes;
            v[i].x = in ? __uint_as_float(w[0]) : kNegInf;
            v[i].y = in ? __uint_as_float(w[1]) : kNegInf;
            v[i].z = in ? __uint_as_float(w[2]) : kNegInf;
            v[i].w = in ? __uint_as_float(w[3]) : kNegInf;
        }
        float m_lane = kNegInf;
#pragma unroll
        for (int i = 0; i < NV; ++i) m_lane = fmaxf(m_lane, max4(v[i]));
        // a lane with no element of the row (m_lane = -inf) gets exp_acc(NaN)
        // = 0 for each: exp_acc clamps its argument with fmaxf, which drops
        // the NaN of -inf - (-inf); no branch is needed around it
        float l_lane = 0.0f;
        const bool empty = (m_lane == kNegInf);
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            v[i].x = exp_acc(v[i].x - m_lane);
            v[i].y = exp_acc(v[i].y - m_lane);
            v[i].z = exp_acc(v[i].z - m_lane);
            v[i].w = exp_acc(v[i].w - m_lane);
            l_lane += (v[i].x + v[i].y) + (v[i].z + v[i].w);
        }
        float m = m_lane, l = l_lane;
        block_merge_ml(m, l, sm, sl);
        const float w = (empty || m == kNegInf) ? 0.0f : exp_acc(m_lane - m) / l;
        const __amdgpu_buffer_rsrc_t yr =
            __builtin_amdgcn_make_buffer_rsrc(y + r * ld_y, 0, (int)bytes, kRsrcWord3);
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const u32x4 o = {__float_as_uint(v[i].x * w), __float_as_uint(v[i].y * w),
                             __float_as_uint(v[i].z * w), __float_as_uint(v[i].w * w)};
            __builtin_amdgcn_raw_buffer_store_b128(o, yr, off0 + i * step, 0, kAuxNontemporal);
        }
        if (threadIdx.x == 0) {
            if (row_max) row_max[r] = m;
            if (row_sum) row_sum[r] = l;
        }
    }
}

// ---- the streaming two-pass kernel (any width) ------------------------------
// Pass 1 runs the recurrence of [P3] "The recurrence, and a proof that it is
// right" per lane, one batch of kStreamU vectors (4 kStreamU elements) per
// step: the batch maximum bm moves the lane's reference once, l is rescaled
// by e^(m - bm) and the batch's e^(x - bm) are added (the rescale is paid
// once per batch, not per element).  Every exponential is exp_acc of an fp32
// difference: the difference is the only rounding before the exponent, so l
// keeps about one fp32 rounding per term.  No branch is needed around an
// empty batch or a lane that has seen nothing: exp_acc maps -inf, and the
// NaN of -inf - (-inf), to 0, so such a step leaves (m, l) = (-inf, 0).
// Pass 2 reads the row again and writes y = e^(x - m) / l.
constexpr int kStreamU = kSoftmaxStreamBatch;

__device__ __forceinline__ void fold_batch(float &m, float &l, const float4 (&v)[kStreamU]) {
    float bm = m;
#pragma unroll
    for (int u = 0; u < kStreamU; ++u) bm = fmaxf(bm, max4(v[u]));
    float s = 0.0f;
#pragma unroll
    for (int u = 0; u < kStreamU; ++u)
        s += (exp_acc(v[u].x - bm) + exp_acc(v[u].y - bm)) + (exp_acc(v[u].z - bm) + exp_acc(v[u].w - bm));
    l = fmaf(l, exp_acc(m - bm), s);
    m = bm;
}

// Rows of any width and alignment (ALIGNED: 16-byte aligned rows).  Vectors
// past the row read as -inf.  Pass 1 loads are cached, so that pass 2 may
// find the row still on chip; pass 2 loads and the stores are nontemporal.
template <bool ALIGNED>
__global__ void __launch_bounds__(1024)
softmax_rows_streaming(const float *x, float *y, int64_t rows,
                       int64_t cols, int64_t ld_x, int64_t ld_y, float *__restrict__ row_max,
                       float *__restrict__ row_sum) {
    __shared__ float sm[kMaxWaves], sl[kMaxWaves];
    const int64_t nvec = (cols + 3) / 4;
    const int64_t step = (int64_t)blockDim.x * kStreamU;
    for (int64_t r = blockIdx.x; r < rows; r += gridDim.x) {
        const float *xr = x + r * ld_x;
        float m = kNegInf, l = 0.0f;
        for (int64_t v0 = threadIdx.x; v0 < nvec; v0 += step) {
            float4 v[kStreamU];
#pragma unroll
            for (int u = 0; u < kStreamU; ++u) {
                const int64_t vec = v0 + (int64_t)u * blockDim.x;
                v[u] = (vec < nvec) ? load_vec<ALIGNED>(xr, vec, cols)
                                    : make_float4(kNegInf, kNegInf, kNegInf, kNegInf);
            }
            fold_batch(m, l, v);
        }
        block_merge_ml(m, l, sm, sl);
        const float inv_l = (m == kNegInf) ? 0.0f : 1.0f / l;
        float *yr = y + r * ld_y;
        for (int64_t v0 = threadIdx.x; v0 < nvec; v0 += step) {
            float4 v[kStreamU];
#pragma unroll
            for (int u = 0; u < kStreamU; ++u) {
                const int64_t vec = v0 + (int64_t)u * blockDim.x;
                if (vec < nvec) v[u] = load_vec_once<ALIGNED>(xr, vec, cols);
            }
#pragma unroll
            for (int u = 0; u < kStreamU; ++u) {
                const int64_t vec = v0 + (int64_t)u * blockDim.x;
                if (vec < nvec) {
                    const float4 o = make_float4(exp_acc(v[u].x - m) * inv_l, exp_acc(v[u].y - m) * inv_l,
                                                 exp_acc(v[u].z - m) * inv_l, exp_acc(v[u].w - m) * inv_l);
                    store_vec<ALIGNED>(yr, vec, cols, o);
                }
            }
        }
        if (threadIdx.x == 0) {
            if (row_max) row_max[r] = m;
            if (row_sum) row_sum[r] = l;
        }
    }
}

// The streaming kernel for 16-byte aligned rows whose width is a multiple
// of four (and below 2^29 elements): loads and stores go through a buffer
// resource spanning exactly the row, so a vector past the end loads zeros
// (set to -inf by a select) and its store is dropped, with no per-vector
// branch.  Each access carries its whole byte offset in the VGPR offset,
// which is what the range check covers.
__global__ void __launch_bounds__(1024)
softmax_rows_streaming_whole(const float *x, float *y, int64_t rows, int64_t cols, int64_t ld_x,
                             int64_t ld_y, float *__restrict__ row_max, float *__restrict__ row_sum) {
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    __shared__ float sm[kMaxWaves], sl[kMaxWaves];
    const uint32_t bytes = (uint32_t)(cols * 4);
    const uint32_t stride = blockDim.x * 16u, step = stride * kStreamU;
    for (int64_t r = blockIdx.x; r < rows; r += gridDim.x) {
        const __amdgpu_buffer_rsrc_t xr =
            __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(x + r * ld_x), 0, (int)bytes, kRsrcWord3);
        float m = kNegInf, l = 0.0f;
        for (uint32_t o0 = threadIdx.x * 16u; o0 < bytes; o0 += step) {
            float4 v[kStreamU];
#pragma unroll
            for (int u = 0; u < kStreamU; ++u) {
                const uint32_t off = o0 + u * stride;
                const u32x4 w = __builtin_amdgcn_raw_buffer_load_b128(xr, off, 0, 0);
                const bool in = off < bytes;
                v[u].x = in ? __uint_as_float(w[0]) : kNegInf;
                v[u].y = in ? __uint_as_float(w[1]) : kNegInf;
                v[u].z = in ? __uint_as_float(w[2]) : kNegInf;
                v[u].w = in ? __uint_as_float(w[3]) : kNegInf;
            }
            fold_batch(m, l, v);
        }
        block_merge_ml(m, l, sm, sl);
        const float inv_l = (m == kNegInf) ? 0.0f : 1.0f / l;
        const __amdgpu_buffer_rsrc_t yr =
            __builtin_amdgcn_make_buffer_rsrc(y + r * ld_y, 0, (int)bytes, kRsrcWord3);
        for (uint32_t o0 = threadIdx.x * 16u; o0 < bytes; o0 += step) {
            u32x4 w[kStreamU];
#pragma unroll
            for (int u = 0; u < kStreamU; ++u)
                w[u] = __builtin_amdgcn_raw_buffer_load_b128(xr, o0 + u * stride, 0, kAuxNontemporal);
#pragma unroll
            for (int u = 0; u < kStreamU; ++u) {
                const u32x4 o = {__float_as_uint(exp_acc(__uint_as_float(w[u][0]) - m) * inv_l),
                                 __float_as_uint(exp_acc(__uint_as_float(w[u][1]) - m) * inv_l),
                                 __float_as_uint(exp_acc(__uint_as_float(w[u][2]) - m) * inv_l),
                                 __float_as_uint(exp_acc(__uint_as_float(w[u][3]) - m) * inv_l)};
                __builtin_amdgcn_raw_buffer_store_b128(o, yr, o0 + u * stride, 0, kAuxNontemporal);
            }
        }
        if (threadIdx.x == 0) {
            if (row_max) row_max[r] = m;
            if (row_sum) row_sum[r] = l;
        }
    }
}

// MODE 0: unaligned rows; 1: 16-byte aligned rows; 2: aligned rows of whole vectors
template <int NV, int MODE>
hipError_t launch_resident(const SoftmaxArgs &a, int threads, int grid, hipStream_t s) {
    if constexpr (MODE == 2)
        hipLaunchKernelGGL((softmax_rows_resident_whole<NV>), dim3(grid), dim3(threads), 0, s, a.x, a.y,
                           a.rows, a.cols, a.ld_x, a.ld_y, a.row_max, a.row_sum);
    else
        hipLaunchKernelGGL((softmax_rows_resident<NV, MODE == 1>), dim3(grid), dim3(threads), 0, s, a.x,
                           a.y, a.rows, a.cols, a.ld_x, a.ld_y, a.row_max, a.row_sum);
    return hipGetLastError();
}

template <int NV>
hipError_t launch_resident_mode(const SoftmaxArgs &a, int mode, int threads, int grid, hipStream_t s) {
    return mode == 2 ? launch_resident<NV, 2>(a, threads, grid, s)
         : mode == 1 ? launch_resident<NV, 1>(a, threads, grid, s)
                     : launch_resident<NV, 0>(a, threads, grid, s);
}

}  // namespace

hipError_t launch_softmax_rows(const SoftmaxArgs &a, const SoftmaxPlan &p, hipStream_t s) {
    if (a.rows == 0) return hipSuccess;
    const bool aligned = ((reinterpret_cast<uintptr_t>(a.x) | reinterpret_cast<uintptr_t>(a.y)) % 16 == 0) &&
                         (a.ld_x % 4 == 0) && (a.ld_y % 4 == 0);
    const int grid = (int)(a.rows < 1048576 ? a.rows : 1048576);
    if (p.resident) {
        // resident rows have at most 65536 columns (16 vectors x 1024 lanes)
        const int mode = !aligned ? 0 : (a.cols % 4 == 0 ? 2 : 1);
        switch (p.nv) {
            case 4: return launch_resident_mode<4>(a, mode, p.threads, grid, s);
            case 8: return launch_resident_mode<8>(a, mode, p.threads, grid, s);
            default: return launch_resident_mode<16>(a, mode, p.threads, grid, s);
        }
    }
    // whole-vector rows whose byte offsets (plus one batch) stay below 2^31
    if (aligned && a.cols % 4 == 0 && a.cols < ((int64_t)1 << 28))
        hipLaunchKernelGGL(softmax_rows_streaming_whole, dim3(grid), dim3(p.threads), 0, s, a.x, a.y,
                           a.rows, a.cols, a.ld_x, a.ld_y, a.row_max, a.row_sum);
    else if (aligned)
        hipLaunchKernelGGL((softmax_rows_streaming<true>), dim3(grid), dim3(p.threads), 0, s, a.x,
                           a.y, a.rows, a.cols, a.ld_x, a.ld_y, a.row_max, a.row_sum);
    else
        hipLaunchKernelGGL((softmax_rows_streaming<false>), dim3(grid), dim3(p.threads), 0, s, a.x,
                           a.y, a.rows, a.cols, a.ld_x, a.ld_y, a.row_max, a.row_sum);
    return hipGetLastError();
}

}  // namespace osm
