// probe.hip -- two reference kernels that measure what this chip reaches on
// plain work, reported beside the attention, softmax and decode rates as
// context for their roofline fractions (libosm_probe.so; not part of the
// osm C ABI, used by the benchmark only):
//
//  * osmprobe_copy: a streaming device copy, 16-byte buffer accesses per
//    lane, nontemporal loads and stores, one sweep of 32 KiB per workgroup.  Its
//    GB/s (bytes read + bytes written per second) is the practical HBM
//    ceiling of a read-and-write stream.
//  * osmprobe_mfma_bf16: independent chains of v_mfma_f32_32x32x16_bf16 on
//    operands loaded from a buffer (so the matrix cores see the same kind of
//    data as the attention products), four accumulators per wave, no memory
//    traffic in the loop.  Its TFLOP/s is the rate the matrix cores sustain
//    on that data under a load that does nothing else.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Workgroup w copies bytes [32768 w, 32768 (w + 1)) of the buffer: eight
// 16-byte vectors per lane through buffer resources spanning the
// workgroup's range, nontemporal loads and stores, all loads issued before
// the stores (one sweep with 32 KiB in flight).  Of the forms tried on
// MI355X (global or buffer accesses, cached or nontemporal, 8 or 16 vectors
// per lane), this one copied fastest.
constexpr int kRsrcWord3 = 0x00020000;   // raw dword access
constexpr int kAuxNontemporal = 2;

__global__ void __launch_bounds__(256) copy_nt(const u32x4 *__restrict__ src, u32x4 *__restrict__ dst) {
    const size_t base = (size_t)blockIdx.x * 2048;
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<u32x4 *>(src + base), 0, 32768, kRsrcWord3);
    const __amdgpu_buffer_rsrc_t rd = __builtin_amdgcn_make_buffer_rsrc(dst + base, 0, 32768, kRsrcWord3);
    u32x4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u)
        v[u] = __builtin_amdgcn_raw_buffer_load_b128(rs, (threadIdx.x + 256 * u) * 16, 0, kAuxNontemporal);
#pragma unroll
    for (int u = 0; u < 8; ++u)
        __builtin_amdgcn_raw_buffer_store_b128(v[u], rd, (threadIdx.x + 256 * u) * 16, 0, kAuxNontemporal);
}

// Each lane loads eight A and eight B operand fragments (16 bf16 vectors);
// iteration i of the inner loop multiplies A fragment i with B fragment
// (i + 3) % 8 into accumulator i % 4.  The sum of the accumulators is stored
// so that nothing is optimized away.
__global__ void __launch_bounds__(512) mfma_loop(const bf16x8 *__restrict__ ops, float *__restrict__ out,
                                                 int iters) {
    const size_t t = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    bf16x8 a[8], b[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = ops[t * 16 + i];
        b[i] = ops[t * 16 + 8 + i];
    }
    f32x16 acc[4] = {};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
            acc[i & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[(i + 3) & 7], acc[i & 3], 0, 0, 0);
    }
    float s = 0.0f;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) s += acc[j][e];
    out[t] = s;
}

}  // namespace

extern "C" {

// Copy `bytes` (a multiple of 32768; both pointers 16-byte aligned) from src
// to dst on `stream`, 32 KiB per workgroup of 256 threads.  Returns a
// hipError_t value (0 = launched).
int osmprobe_copy(const void *src, void *dst, size_t bytes, void *stream) {
    if (bytes % 32768 || (reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) % 16 ||
        bytes / 32768 >= (size_t)1 << 31)
        return (int)hipErrorInvalidValue;
    const unsigned grid = (unsigned)(bytes / 32768);
    if (grid == 0) return 0;
    hipLaunchKernelGGL(copy_nt, dim3(grid), dim3(256), 0, static_cast<hipStream_t>(stream),
                       static_cast<const u32x4 *>(src), static_cast<u32x4 *>(dst));
    return (int)hipGetLastError();
}

// `grid` workgroups of `threads` (256 or 512: one or two waves per SIMD)
// threads, each thread running `iters` x 8 MFMAs of 32x32x16 (32768 flops per
// wave each).  `ops` holds grid * threads * 16 bf16x8 fragments
// (grid * threads * 256 bytes); `out` grid * threads floats.
int osmprobe_mfma_bf16(const void *ops, float *out, int grid, int threads, int iters, void *stream) {
    if (grid < 1 || iters < 1 || (threads != 256 && threads != 512) || (reinterpret_cast<uintptr_t>(ops) % 16))
        return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(mfma_loop, dim3(grid), dim3(threads), 0, static_cast<hipStream_t>(stream),
                       static_cast<const bf16x8 *>(ops), out, iters);
    return (int)hipGetLastError();
}

}  // extern "C"
