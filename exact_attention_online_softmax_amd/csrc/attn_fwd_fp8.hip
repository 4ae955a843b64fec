// attn_fwd_fp8.hip -- fused exact attention forward with FP8 (OCP E4M3) Q, K
// and V on gfx950 (head_dim 128).
//
// [P3] "Precision, and what can still go wrong": kernels keep the running
// m, l and O~ in float32 even when Q, K and V are bf16 or FP8, because those
// few numbers per row decide the output's accuracy.  The computation is the
// block step of [P3] "Blocks, the bridge to FlashAttention", exactly as in
// attn_fwd.hip (running maximum with a lazy reference, rescale of O~ and l,
// one division at the end, LSE = m + log l, masks inside the tile loop);
// what changes is the precision of the two matrix products:
//  * S^T = K Q^T on v_mfma_scale_f32_32x32x64_f8f6f4 with both operands E4M3
//    and unit scales: products of E4M3 values are exact, sums are fp32.
//  * P~ = exp2(S scale log2e - m) is at most 2^8 under the lazy reference;
//    it is rounded to E4M3 (nearest even) as the B operand of
//    O~^T += V^T P~^T on the same instruction.  l sums the fp32 P~.
//  * m, l, O~ and the epilogue stay fp32; O is written as bf16, times
//    v_scale (the dequantization factor of V), and the LSE as fp32.
//
// Mapping to CDNA4:
//  * workgroup = 8 wavefronts = 256 queries, two waves per SIMD; each wave
//    owns 32 queries and holds their Q as MFMA B operands (32 bytes per lane
//    per 64-dim k-step).  The softmax VALU per MFMA clock is twice the bf16
//    kernel's (an FP8 MFMA does twice the work per clock), so the second wave
//    on the SIMD is what keeps the matrix core fed while one wave
//    exponentiates.  That leaves a wave 256 registers: 128 VGPRs and the
//    AGPRs, which hold O~ and some of the spilled values (the compiler caps
//    the VGPRs of a kernel that uses AGPRs at half); the rest, 36 bytes per
//    lane (92 on the persistent grid), goes to scratch, two reloads per tile.
//  * tiles of 64 keys (the MFMA's k for P~V): K and V tiles of 64 rows x 128
//    bytes go from HBM straight into LDS through buffer loads with LDS
//    destination (rows past Lk read as zeros), through a ring of four slots
//    loaded three tiles ahead.
//  * software pipeline: iteration j issues the score MFMAs of tile j + 1
//    while the vector ALU exponentiates tile j, then adds P~(j) V(j) to O~,
//    and last masks tile j + 1 and takes its maximum (under the P~V MFMAs),
//    so that iteration j + 1 starts with the reference decision.
//    The scores are read by the VALU, so the score MFMAs write VGPRs (the
//    compiler is told to use the VGPR form); O~ lives in the AGPRs through
//    inline assembly.
//  * key order: row c = 8 r + 4 h + u of a 32-key score block is key
//    16 h + 4 r + u of that block, so each lane half of the score accumulator
//    holds 16 consecutive keys.  P~ packs them, in order, into the B operand
//    of P~V; its A operand V^T comes from ds_read_b64_tr_b8 reads (lane j of
//    a 16-lane group receives eight consecutive rows of column j), eight keys
//    per read, in the same order.
//  * LDS rows are unpadded, 16-byte chunk c of row r in slot c ^ swz8(r),
//    swz8(r) = 2 ((r / 2) % 4) + (r / 16) % 2.  The LDS serves 256 bytes per
//    cycle; a row-wise 16-byte read serves 16 lanes at a time, a transposing
//    read 32, and each group must touch distinct slots of a 256-byte window
//    (two 128-byte rows).  The K operand's 16 lanes read rows of both
//    parities from two groups of four, and swz8 takes eight distinct values
//    over each parity's rows there; the V^T read's 32 lanes read two chunks
//    of eight consecutive rows, and swz8 / 2 takes four distinct values over
//    each parity's four rows.  Both reads are free of bank conflicts (the
//    previous swizzle left the V^T reads two-way conflicted, 33% of the LDS
//    active cycles in rocprofv3's counters).
#include "osm_device.h"
#include "osm_internal.h"

namespace osm {

namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int D = 128;            // head dim
constexpr int ROWB = D;           // bytes per E4M3 row
constexpr int NQB = 1;            // 32-query blocks per wavefront
constexpr int QW = 32 * NQB;      // queries per wavefront
constexpr int NW = 256 / QW;      // wavefronts per workgroup (two per SIMD)
constexpr int BQ = QW * NW;       // queries per workgroup
constexpr int BK = 64;            // keys per tile
constexpr int NT = 64 * NW;
constexpr int TILEB = BK * ROWB;  // bytes per K or V tile (8 KiB)
constexpr int LPW = TILEB / 1024 / NW;   // 1 KiB loads per wave per K (or V) tile
static_assert(LPW == 1, "the wait counts assume one K and one V load per wave per tile");

constexpr int kRsrcWord3 = 0x00020000;   // raw buffer, 32-bit data format
constexpr int kWaitVm0 = 0x0F70;         // s_waitcnt vmcnt(0)
constexpr int kWaitVm2 = 0x0F72;         // s_waitcnt vmcnt(2): one tile's loads in flight
constexpr int kWaitVm4 = 0x0F74;         // s_waitcnt vmcnt(4): two tiles' loads in flight
constexpr int kWaitVm6 = 0x0F76;         // s_waitcnt vmcnt(6)
constexpr int kWaitLgkm0 = 0xC07F;       // s_waitcnt lgkmcnt(0)
constexpr int kUnitScale = 127;          // E8M0 exponent of 1.0 for the MFMA's block scales

template <int N> struct Slot { static constexpr int value = N; };

__device__ __forceinline__ int clampi(int v, int lo, int hi) { return v < lo ? lo : (v > hi ? hi : v); }
__device__ __forceinline__ int rfl(int v) { return __builtin_amdgcn_readfirstlane(v); }

// a wave-uniform pointer, moved to scalar registers
__device__ __forceinline__ const uint8_t *uniform_ptr(const uint8_t *p) {
    const uint64_t u = reinterpret_cast<uint64_t>(p);
    const uint64_t lo = (uint32_t)rfl((int)(uint32_t)u), hi = (uint32_t)rfl((int)(uint32_t)(u >> 32));
    return reinterpret_cast<const uint8_t *>((hi << 32) | lo);
}

// (batch, head, KV head, first query) of a query block
struct Blk {
    int b, h, kvh, q0;
};

// chunk c of LDS row r sits in slot c ^ swz8(r); see the header comment
__device__ __forceinline__ int swz8(int r) { return (((r >> 1) & 3) << 1) | ((r >> 4) & 1); }

__device__ __forceinline__ f32x16 mfma8(const i32x8 &a, const i32x8 &b, const f32x16 &c) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, kUnitScale, 0, kUnitScale);
}

// O~^T accumulation with the accumulator pinned to AGPRs (see the header).
// The hazard recognizer does not look into inline assembly: the VALU writes
// of the B operand need wait states before the MFMA reads them.  NOP: the
// first P~V MFMA of a tile, right after the conversions that build P~; the
// others read the same P~ behind it, and A operands that come from LDS reads
// (covered by the counter waits the compiler inserts).
template <bool NOP>
__device__ __forceinline__ void mfma8_acc(f32x16 &acc, const i32x8 &a, const i32x8 &b, int sc) {
    if constexpr (NOP)
        asm("s_nop 3\n\tv_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, %0, %3, %3" : "+a"(acc) : "v"(a), "v"(b), "v"(sc));
    else
        asm("v_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, %0, %3, %3" : "+a"(acc) : "v"(a), "v"(b), "v"(sc));
}

__device__ __forceinline__ void acc_zero8(f32x16 &acc, const i32x8 &z, int sc) {
    asm volatile("s_nop 3\n\tv_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %1, 0, %2, %2" : "=a"(acc) : "v"(z), "v"(sc));
}

// Before ordinary code reads accumulators written by mfma8_acc: wait out the
// MFMA's result latency (generously: 40 wait states).
__device__ __forceinline__ void acc_settle8(f32x16 (&o)[NQB][4]) {
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7"
                 : "+a"(o[0][0]), "+a"(o[0][1]), "+a"(o[0][2]), "+a"(o[0][3]));
    if constexpr (NQB == 2)
        asm volatile("" : "+a"(o[1][0]), "+a"(o[1][1]), "+a"(o[1][2]), "+a"(o[1][3]));
}

__device__ __forceinline__ i32x2 lds_read_tr8(const uint8_t *p) {
    return __builtin_amdgcn_ds_read_tr8_b64_v2i32((i32x2 __attribute__((address_space(3))) *)(p));
}

__device__ __forceinline__ void tile_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// PERSIST: one workgroup per CU walks the blocks L = blockIdx.x, + gridDim.x,
// ... (full-length non-causal inputs, where every block has the same work).
// The next block's Q is copied into LDS (qs) while the current block runs,
// and the ring's loads past a block's padded end fetch the next block's
// first tiles, so a block starts with its Q and first tile on chip.
template <bool PERSIST>
__device__ __forceinline__ void
attn_fp8_body(const uint8_t *__restrict__ Q, const uint8_t *__restrict__ K,
              const uint8_t *__restrict__ V, uint16_t *__restrict__ O, float *__restrict__ LSE,
              int Hq, int Hkv, int Nq, int Nk, const int32_t *__restrict__ seqlens_q,
              const int32_t *__restrict__ seqlens_k, float scale_log2, float v_scale, int causal_arg,
              int nqb, int xcd_heads, int nblocks) {
    __shared__ __attribute__((aligned(1024))) uint8_t k0[TILEB], k1[TILEB], k2[TILEB], k3[TILEB];
    __shared__ __attribute__((aligned(1024))) uint8_t v0[TILEB], v1[TILEB], v2[TILEB], v3[TILEB];
    // Q of the block (PERSIST), rows swizzled like K; less aligned than the
    // slots, so that it is laid out after them
    __shared__ __attribute__((aligned(256))) uint8_t qs[PERSIST ? BQ * ROWB : 256];
    const int causal = PERSIST ? 0 : causal_arg;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = rfl(tid >> 6);
    const int g = lane >> 5, c = lane & 31;

    // ---- which (batch, head, query block) ------------------------------
    auto decode = [&](int L) __attribute__((always_inline)) -> Blk {
        int head, qrev;
        if (xcd_heads) {
            // block L runs on XCD L % 8 (a persistent grid is a multiple of
            // 8): whole heads per XCD, so the blocks of one head share its K
            // and V in that XCD's L2
            const int xcd = L & 7, slot = L >> 3;
            qrev = slot % nqb;
            head = (slot / nqb) * 8 + xcd;
        } else {
            head = L / nqb;
            qrev = L % nqb;
        }
        head = rfl(head);
        qrev = rfl(qrev);
        const int qb0 = causal ? (nqb - 1 - qrev) : qrev;     // causal: heaviest blocks first
        const int b = head / Hq, h = head % Hq;
        return {b, h, h / (Hq / Hkv), qb0 * BQ};
    };

    int L = blockIdx.x;
    bool first = true;
    for (;;) {
        const Blk cur = decode(L);
        const int Lnext = L + (int)gridDim.x;
        const bool has_next = PERSIST && rfl(Lnext < nblocks ? 1 : 0) != 0;
        const Blk nxt = decode(has_next ? Lnext : L);
        const int b = cur.b, h = cur.h, kvh = cur.kvh, q0 = cur.q0;
        const int Lq = rfl(seqlens_q ? clampi(seqlens_q[b], 0, Nq) : Nq);
        const int Lk = rfl(seqlens_k ? clampi(seqlens_k[b], 0, Nk) : Nk);

        const int qw0 = q0 + QW * wave;             // queries qw0 + 32 qb + c
        const size_t qrow0 = (size_t)(b * Hq + h) * Nq;
        const uint8_t *Kh = K + (size_t)(b * Hkv + kvh) * Nk * D;
        const uint8_t *Vh = V + (size_t)(b * Hkv + kvh) * Nk * D;

        if (!PERSIST && q0 >= Lq) {
            const int rows = min(BQ, Nq - q0);
            for (int i = tid; i < rows * (D / 8); i += NT)
                *reinterpret_cast<uint4 *>(O + (qrow0 + q0 + i / (D / 8)) * D + (i % (D / 8)) * 8) =
                    make_uint4(0, 0, 0, 0);
            if (LSE)
                for (int r = tid; r < rows; r += NT) LSE[qrow0 + q0 + r] = kNegInf;
            return;
        }

        int kend = Lk;
        if (causal) kend = min(kend, min(q0 + BQ, Lq));
        const int ntiles = (kend + BK - 1) / BK;
        int wtiles = (qw0 >= Lq) ? 0 : ntiles;
        if (causal) wtiles = min(wtiles, (qw0 + QW - 1) / BK + 1);
        int wmask = wtiles;                           // first tile that needs a mask
        if (causal) wmask = min(wmask, qw0 / BK);
        if (Lk % BK) wmask = min(wmask, Lk / BK);
        const int nend = ((ntiles + 3) / 4) * 4;

        const int unit_scale = kUnitScale;
        f32x16 oacc[NQB][4];
        {
            const i32x8 z8 = {};
#pragma unroll
            for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
                for (int dt = 0; dt < 4; ++dt) acc_zero8(oacc[qb][dt], z8, unit_scale);
        }
        // The reference only moves when a tile's maximum exceeds it by more than
        // 2^8 in weight, so every P~ is at most 2^8 (E4M3 holds up to 448).
        constexpr float kLazy = 8.0f;
        const float lazy_raw = kLazy / scale_log2;
        float m[NQB], mlim[NQB], msub[NQB], l[NQB];
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb) {
            m[qb] = kNegInf;     // reference maximum of raw scores q.k
            mlim[qb] = kNegInf;  // m + lazy_raw: tile maxima up to it keep the reference
            msub[qb] = 0.0f;     // m * scale * log2(e) (0 while m = -inf)
            l[qb] = 0.0f;        // this lane's part of the running sum
        }

        // ---- tile DMA: load i of wave w fills LDS block LPW w + i (8 rows);
        // lane l row 8 blk + l/8, slot l%8, holding global chunk slot ^ swz8(row)
        uint32_t dmo[LPW];
#pragma unroll
        for (int i = 0; i < LPW; ++i) {
            const int row = 8 * (LPW * wave + i) + (lane >> 3);
            dmo[i] = row * ROWB + (((lane & 7) ^ swz8(row)) << 4);
        }
        // loads of tile j0 / BK from K and V rows kb, vb of length len into slots kd, vd
        auto issue_at = [&](uint8_t *kd, uint8_t *vd, const uint8_t *kb, const uint8_t *vb, int j0, int len)
            __attribute__((always_inline)) {
            const int bytes = max(0, len - j0) * ROWB;   // < 2^31: the ABI bounds Nk * 128
            const __amdgpu_buffer_rsrc_t rk =
                __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(kb) + (size_t)j0 * D, 0, bytes, kRsrcWord3);
            const __amdgpu_buffer_rsrc_t rv =
                __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(vb) + (size_t)j0 * D, 0, bytes, kRsrcWord3);
#pragma unroll
            for (int i = 0; i < LPW; ++i) {
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rk, (void __attribute__((address_space(3))) *)(kd + (LPW * wave + i) * 1024), 16, dmo[i], 0, 0, 0);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rv, (void __attribute__((address_space(3))) *)(vd + (LPW * wave + i) * 1024), 16, dmo[i], 0, 0, 0);
            }
        };
        // tile t of this block
        auto issue = [&](uint8_t *kd, uint8_t *vd, int t) __attribute__((always_inline)) {
            issue_at(kd, vd, Kh, Vh, t * BK, Lk);
        };
        // tile t of the ring in the last group of four iterations: with PERSIST,
        // tile nend + i (past this block's padded end, where the ring would load
        // zeros) is tile i of the next block, if there is one.  The selects are
        // uniform, but the compiler evaluates them on the vector ALU; rfl keeps
        // the resources in scalar registers (else every load loops over lanes).
        const uint8_t *Kn = K + (size_t)(nxt.b * Hkv + nxt.kvh) * Nk * D;
        const uint8_t *Vn = V + (size_t)(nxt.b * Hkv + nxt.kvh) * Nk * D;
        auto issue_last = [&](uint8_t *kd, uint8_t *vd, int t) __attribute__((always_inline)) {
            if constexpr (!PERSIST) {
                issue(kd, vd, t);
            } else {
                const bool next = t >= nend;
                issue_at(kd, vd, uniform_ptr(next ? Kn : Kh), uniform_ptr(next ? Vn : Vh),
                         rfl((next ? t - nend : t) * BK), rfl((next && !has_next) ? 0 : Lk));
            }
        };
        // Q rows q0 .. q0 + BQ - 1 of block n into qs (PERSIST): wave w copies its
        // own 32 rows, 4 loads of 1 KiB laid out like a tile's; rows at or past
        // Nq read as zeros
        auto issue_q = [&](const Blk &n) __attribute__((always_inline)) {
            const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
                const_cast<uint8_t *>(Q) + ((size_t)(n.b * Hq + n.h) * Nq + n.q0) * D, 0,
                max(0, Nq - n.q0) * ROWB, kRsrcWord3);
#pragma unroll
            for (int i = 0; i < QW * ROWB / 1024; ++i) {
                const int blk = (QW * ROWB / 1024) * wave + i, row = 8 * blk + (lane >> 3);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (void __attribute__((address_space(3))) *)(qs + blk * 1024), 16,
                                                         row * ROWB + (((lane & 7) ^ swz8(row)) << 4), 0, 0, 0);
            }
        };
        if (PERSIST && first) {
            issue_q(cur);
            issue(k0, v0, 0);
            issue(k1, v1, 1);
            issue(k2, v2, 2);
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
        }

        // ---- Q (B operands of S^T = K Q^T): lane (g, c) holds row qw0 + 32 qb + c,
        // bytes 64 ks + 32 g .. + 31; rows at or past Lq are zero
        i32x8 qf[NQB][2];
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb) {
            const int qi = qw0 + 32 * qb + c;
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                uint4 lo = make_uint4(0, 0, 0, 0), hi = make_uint4(0, 0, 0, 0);
                if constexpr (PERSIST) {
                    // this wave's rows of qs: row 32 wave + 32 qb + c, chunks 4 ks + 2 g, + 1
                    const int row = QW * wave + 32 * qb + c, ch = 4 * ks + 2 * g;
                    lo = *reinterpret_cast<const uint4 *>(qs + row * ROWB + ((ch ^ swz8(row)) << 4));
                    hi = *reinterpret_cast<const uint4 *>(qs + row * ROWB + (((ch + 1) ^ swz8(row)) << 4));
                } else if (qi < Lq) {
                    const uint4 *src = reinterpret_cast<const uint4 *>(Q + (qrow0 + qi) * D + 64 * ks + 32 * g);
                    lo = src[0];
                    hi = src[1];
                }
                qf[qb][ks] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
            }
        }

        // K operand (rows of a 32-key block, permuted): lane (g, c) with
        // c = 8 r + 4 hh + u reads key row 16 hh + 4 r + u, chunks 4 ks + 2 g and + 1;
        // the second 32-key block is the same offsets + 32 rows
        uint32_t koff[2][2];
        {
            const int row = 16 * ((c >> 2) & 1) + 4 * (c >> 3) + (c & 3);
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
#pragma unroll
                for (int hf = 0; hf < 2; ++hf) koff[ks][hf] = row * ROWB + (((4 * ks + 2 * g + hf) ^ swz8(row)) << 4);
        }
        // V^T operand (dim rows 32 dt + c): bytes 8 e .. 8 e + 7 of lane half g are
        // keys 32 (e/2) + 16 g + 8 (e%2) + 0..7.  16-lane group t = lane/16,
        // index i = lane%16 points at key row 16 (t/2) + i/2 (+ 8 (e%2) + 32 (e/2),
        // which leave the swizzle unchanged), dims 32 dt + 16 (t%2) + 8 (i%2)
        uint32_t voff[4];
        {
            const int t = lane >> 4, i = lane & 15;
            const int row = 16 * (t >> 1) + (i >> 1);
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) voff[dt] = row * ROWB + (((2 * dt + (t & 1)) ^ swz8(row)) << 4) + 8 * (i & 1);
        }

        // S^T of one tile: s[kb][qb] element 4 r + u of lane (g, c) is key
        // 32 kb + 16 g + 4 r + u of the tile, query qw0 + 32 qb + c
        auto qk = [&](const uint8_t *kb, f32x16 (&s)[2][NQB]) __attribute__((always_inline)) {
            const f32x16 zero = {};
#pragma unroll
            for (int kbk = 0; kbk < 2; ++kbk)
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    const uint4 lo = *reinterpret_cast<const uint4 *>(kb + 32 * kbk * ROWB + koff[ks][0]);
                    const uint4 hi = *reinterpret_cast<const uint4 *>(kb + 32 * kbk * ROWB + koff[ks][1]);
                    const i32x8 a = {(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
#pragma unroll
                    for (int qb = 0; qb < NQB; ++qb) s[kbk][qb] = mfma8(a, qf[qb][ks], ks ? s[kbk][qb] : zero);
                }
        };

        auto mask = [&](f32x16 (&s)[2][NQB], int t) __attribute__((always_inline)) {
#pragma unroll
            for (int qb = 0; qb < NQB; ++qb) {
                const int qi = qw0 + 32 * qb + c;
                const int lim = (causal ? min(Lk - 1, qi) : Lk - 1) - t * BK - 16 * g;
#pragma unroll
                for (int kbk = 0; kbk < 2; ++kbk)
#pragma unroll
                    for (int i = 0; i < 16; ++i)
                        if (32 * kbk + i > lim) s[kbk][qb][i] = kNegInf;
            }
        };

        // iteration body for tile t whose scores are in s: mask, lazy reference,
        // then (one scheduling region) the scores of tile t + 1 into sn, the
        // exponentials of tile t, and O~ += P~(t) V(t)
        // mask (when tile t needs it) and tile maximum of scores s of tile t
        auto tmax = [&](f32x16 (&s)[2][NQB], int t, float (&tm)[NQB]) __attribute__((always_inline)) {
            if (t >= wmask) mask(s, t);
#pragma unroll
            for (int qb = 0; qb < NQB; ++qb) {
                float x = fmaxf(fmaxf(s[0][qb][0], s[0][qb][1]), s[1][qb][0]);
                x = fmaxf(x, s[1][qb][1]);
#pragma unroll
                for (int i = 2; i < 16; ++i) x = fmaxf(fmaxf(x, s[0][qb][i]), s[1][qb][i]);
                tm[qb] = x;     // this lane's half; lane l ^ 32 holds the other
            }
        };
        float tmc[NQB];     // this lane's half of the tile maximum of the scores whose softmax is next
        auto body = [&](const uint8_t *kn, const uint8_t *vb, int t, f32x16 (&s)[2][NQB], f32x16 (&sn)[2][NQB])
            __attribute__((always_inline)) {
            // tmc holds this lane's half of each query's tile maximum.  Every
            // lane being within m + kLazy (mlim) is the same test as every full
            // maximum being within it, so the halves are combined only when the
            // reference moves (one ballot per comparison).
            uint64_t over = 0;
#pragma unroll
            for (int qb = 0; qb < NQB; ++qb) over |= __builtin_amdgcn_ballot_w64(tmc[qb] > mlim[qb]);
            if (over != 0) {
                float tm[NQB];
#pragma unroll
                for (int qb = 0; qb < NQB; ++qb) {
                    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(tmc[qb]), __float_as_uint(tmc[qb]),
                                                                     false, false);
                    tm[qb] = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
                }
                acc_settle8(oacc);
#pragma unroll
                for (int qb = 0; qb < NQB; ++qb) {
                    const float mn = fmaxf(m[qb], tm[qb]);
                    const float alpha = (mn == kNegInf || m[qb] == mn) ? 1.0f
                                      : (m[qb] == kNegInf ? 0.0f : fast_exp2((m[qb] - mn) * scale_log2));
                    l[qb] *= alpha;
#pragma unroll
                    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
                        for (int i = 0; i < 16; ++i) oacc[qb][dt][i] *= alpha;
                    m[qb] = mn;
                    mlim[qb] = mn + lazy_raw;
                    msub[qb] = (mn == kNegInf) ? 0.0f : mn * scale_log2;
                }
            }
            qk(kn, sn);
            // P~ = exp2(S scale log2e - m scale log2e), l += row sums (four
            // partial sums), E4M3 operands: dword 4 kb + r holds elements
            // 4 r .. 4 r + 3 of block kb
            i32x8 pf[NQB];
#pragma unroll
            for (int qb = 0; qb < NQB; ++qb) {
                float rs[4];     // set by the first weight of each (0 + x would cost an add)
#pragma unroll
                for (int kbk = 0; kbk < 2; ++kbk)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        float e[4];
#pragma unroll
                        for (int u = 0; u < 4; ++u) {
                            e[u] = fast_exp2(fmaf(s[kbk][qb][4 * r + u], scale_log2, -msub[qb]));
                            rs[u] = (kbk == 0 && r == 0) ? e[u] : rs[u] + e[u];
                        }
                        // (both halves of w are written, so the register the first
                        // conversion starts from may hold anything: an empty asm
                        // names one, where a constant would cost a move)
                        int w;
                        asm volatile("" : "=v"(w));
                        w = __builtin_amdgcn_cvt_pk_fp8_f32(e[0], e[1], w, false);
                        w = __builtin_amdgcn_cvt_pk_fp8_f32(e[2], e[3], w, true);
                        pf[qb][4 * kbk + r] = w;
                    }
                l[qb] += (rs[0] + rs[1]) + (rs[2] + rs[3]);
            }
            // O~^T += V^T P~^T
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) {
                const uint8_t *base = vb + voff[dt];
                const i32x2 r0 = lds_read_tr8(base);
                const i32x2 r1 = lds_read_tr8(base + 8 * ROWB);
                const i32x2 r2 = lds_read_tr8(base + 32 * ROWB);
                const i32x2 r3 = lds_read_tr8(base + 40 * ROWB);
                const i32x8 a = {r0[0], r0[1], r1[0], r1[1], r2[0], r2[1], r3[0], r3[1]};
#pragma unroll
                for (int qb = 0; qb < NQB; ++qb) {
                    if (dt == 0 && qb == 0) mfma8_acc<true>(oacc[qb][dt], a, pf[qb], unit_scale);
                    else mfma8_acc<false>(oacc[qb][dt], a, pf[qb], unit_scale);
                }
            }
            // interleave the score MFMAs of tile t + 1 with the exponentials
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x002, 20, 0);
            }
            tmax(sn, t + 1, tmc);
        };

        auto kslot = [&](auto S) __attribute__((always_inline)) -> uint8_t * {
            constexpr int s = decltype(S)::value % 4;
            return s == 0 ? k0 : s == 1 ? k1 : s == 2 ? k2 : k3;
        };
        auto vslot = [&](auto S) __attribute__((always_inline)) -> uint8_t * {
            constexpr int s = decltype(S)::value % 4;
            return s == 0 ? v0 : s == 1 ? v1 : s == 2 ? v2 : v3;
        };
        // iteration j (slot j % 4): this wave's loads of tile j + 1 are done (tile
        // j + 2's may be in flight); the barrier publishes every wave's and frees
        // slot (j + 3) % 4 (every wave is past iteration j - 1), which receives
        // tile j + 3.  Every iteration issues exactly four loads per wave (tiles
        // past the end are zero fills), so the wait count is the same everywhere.
        // Two score buffers alternate: even iterations read sa and fill sb.
        f32x16 sa[2][NQB], sb[2][NQB];
        // With PERSIST and a next block, the 4 loads copying its Q are issued
        // after S(0) (below), behind this block's tiles 1 and 2 and the previous
        // block's O stores: tiles 1 and 2 are then followed by at least 6 memory
        // operations, and iterations 0 and 1 wait with vmcnt(6).
        auto iter = [&](auto S, auto LAST, int j) __attribute__((always_inline)) {
            constexpr int si = decltype(S)::value;
            if (PERSIST && has_next && j < 2)
                __builtin_amdgcn_s_waitcnt(kWaitVm6);
            else
                __builtin_amdgcn_s_waitcnt(kWaitVm2);
            tile_barrier();
            if constexpr (decltype(LAST)::value)
                issue_last(kslot(Slot<si + 3>{}), vslot(Slot<si + 3>{}), j + 3);
            else
                issue(kslot(Slot<si + 3>{}), vslot(Slot<si + 3>{}), j + 3);
            if (j < wtiles) {
                if constexpr (si % 2 == 0) body(kslot(Slot<si + 1>{}), vslot(S), j, sa, sb);
                else body(kslot(Slot<si + 1>{}), vslot(S), j, sb, sa);
            }
        };

        // (with PERSIST tile 0 is resident already: loaded at the start, or by
        // the previous block's last iterations, whose final wait and barrier
        // cover it)
        if (!PERSIST) {
            issue(k0, v0, 0);
            issue(k1, v1, 1);
            issue(k2, v2, 2);
            __builtin_amdgcn_s_waitcnt(kWaitVm4);       // this wave's part of tile 0
            tile_barrier();
        }
        if (wtiles > 0) {
            qk(k0, sa);
            tmax(sa, 0, tmc);
        }
        if (has_next) {
            // this wave's reads of qs are complete (its own rows only): copy the
            // next block's Q over them
            __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
            issue_q(nxt);
        }
        // the last group of four iterations is the only one that loads past
        // the padded end (tiles nend .. nend + 2)
        int j = 0;
        for (; j + 4 < nend; j += 4) {
            iter(Slot<0>{}, Slot<0>{}, j);
            iter(Slot<1>{}, Slot<0>{}, j + 1);
            iter(Slot<2>{}, Slot<0>{}, j + 2);
            iter(Slot<3>{}, Slot<0>{}, j + 3);
        }
        if (j < nend) {
            iter(Slot<0>{}, Slot<1>{}, j);
            iter(Slot<1>{}, Slot<1>{}, j + 1);
            iter(Slot<2>{}, Slot<1>{}, j + 2);
            iter(Slot<3>{}, Slot<1>{}, j + 3);
        }
        // no load outlives the last block (the next block's tiles 1 and 2 stay
        // in flight otherwise)
        if (!has_next) __builtin_amdgcn_s_waitcnt(kWaitVm0);

        // ---- epilogue: O = v_scale O~ / l, LSE = m + log l ------------------------
        acc_settle8(oacc);
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb) {
            const int qi = qw0 + 32 * qb + c;
            const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(l[qb]), __float_as_uint(l[qb]), false, false);
            const float lt = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
            const bool valid = (qi < Lq) && (lt > 0.0f);
            const float inv = valid ? v_scale / lt : 0.0f;
            if (qi < Nq) {
                uint16_t *orow = O + (qrow0 + qi) * D;
#pragma unroll
                for (int dt = 0; dt < 4; ++dt)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        uint2 w;
                        w.x = valid ? pack_bf16x2_hw(oacc[qb][dt][4 * r + 0] * inv, oacc[qb][dt][4 * r + 1] * inv) : 0u;
                        w.y = valid ? pack_bf16x2_hw(oacc[qb][dt][4 * r + 2] * inv, oacc[qb][dt][4 * r + 3] * inv) : 0u;
                        *reinterpret_cast<uint2 *>(orow + 32 * dt + 8 * r + 4 * g) = w;
                    }
                if (LSE && g == 0)
                    LSE[qrow0 + qi] = valid ? (m[qb] * scale_log2 + __log2f(lt)) * kLn2 : kNegInf;
            }
        }
        if (!has_next) break;
        L = Lnext;
        first = false;
    }   // blocks
}

#define OSM_FP8_PARAMS                                                                              \
    const uint8_t *__restrict__ Q, const uint8_t *__restrict__ K, const uint8_t *__restrict__ V,    \
        uint16_t *__restrict__ O, float *__restrict__ LSE, int Hq, int Hkv, int Nq, int Nk,         \
        const int32_t *__restrict__ seqlens_q, const int32_t *__restrict__ seqlens_k,               \
        float scale_log2, float v_scale, int causal, int nqb, int xcd_heads, int nblocks

// one query block per workgroup
__global__ void __launch_bounds__(NT, 1) attn_fwd_fp8_d128(OSM_FP8_PARAMS) {
    attn_fp8_body<false>(Q, K, V, O, LSE, Hq, Hkv, Nq, Nk, seqlens_q, seqlens_k, scale_log2, v_scale, causal,
                         nqb, xcd_heads, nblocks);
}

// one workgroup per compute unit walking several query blocks
__global__ void __launch_bounds__(NT, 1) attn_fwd_fp8_d128_persist(OSM_FP8_PARAMS) {
    attn_fp8_body<true>(Q, K, V, O, LSE, Hq, Hkv, Nq, Nk, seqlens_q, seqlens_k, scale_log2, v_scale, causal,
                        nqb, xcd_heads, nblocks);
}
#undef OSM_FP8_PARAMS

}  // namespace

hipError_t launch_attn_fwd_fp8(const AttnFwdFp8Args &a, hipStream_t s) {
    const int nqb = (a.seqlen_q + BQ - 1) / BQ;
    const int nheads = a.batch * a.heads_q;
    const int64_t blocks = (int64_t)nqb * nheads;
    if (blocks == 0) return hipSuccess;
    const int xcd_heads = (nheads % 8 == 0) ? 1 : 0;
    // full-length non-causal inputs with more blocks than compute units run
    // on a persistent grid of one workgroup per compute unit
    int cus = 0;
    if (!a.causal && !a.seqlens_q && !a.seqlens_k && a.seqlen_k > 0) {
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            cus = 0;
        cus &= ~7;   // whole XCDs' worth, so block L keeps running on XCD L % 8
    }
    const bool persist = cus > 0 && blocks > cus;
    const unsigned grid = persist ? (unsigned)cus : (unsigned)blocks;
    const uint8_t *q = static_cast<const uint8_t *>(a.q), *k = static_cast<const uint8_t *>(a.k),
                  *v = static_cast<const uint8_t *>(a.v);
    uint16_t *o = static_cast<uint16_t *>(a.o);
    if (persist)
        hipLaunchKernelGGL(attn_fwd_fp8_d128_persist, dim3(grid), dim3(NT), 0, s, q, k, v, o, a.lse, a.heads_q,
                           a.heads_kv, a.seqlen_q, a.seqlen_k, a.seqlens_q, a.seqlens_k, a.scale * kLog2e,
                           a.v_scale, a.causal, nqb, xcd_heads, (int)blocks);
    else
        hipLaunchKernelGGL(attn_fwd_fp8_d128, dim3(grid), dim3(NT), 0, s, q, k, v, o, a.lse, a.heads_q,
                           a.heads_kv, a.seqlen_q, a.seqlen_k, a.seqlens_q, a.seqlens_k, a.scale * kLog2e,
                           a.v_scale, a.causal, nqb, xcd_heads, (int)blocks);
    return hipGetLastError();
}

}  // namespace osm
