// attn_fwd.hip -- fused exact attention forward for gfx950 (bf16, head_dim 128).
//
// The block step of [P3] "Blocks, the bridge to FlashAttention": hold a block
// of queries, stream the keys and values past them a block at a time,
// compute the block of scores with a matrix product, update the per-query
// running maximum m and sum l, rescale the unnormalized output O~ by
// exp(m - m_new) and add P~ V_j; divide once at the end and emit
// LSE = m + log l ([P3] "From weights to outputs").  Masks are applied
// inside the tile loop ([P2] "Walking through it", the mask paragraph); a
// fully masked block is skipped and the -inf - (-inf) case is guarded
// ([P3] "Precision, and what can still go wrong").  Scores stay in base-2
// scaled units, log2(e) folded into the scale (same section).
//
// Mapping to CDNA4:
//  * workgroup = 8 wavefronts = 256 queries (two waves per SIMD, one
//    workgroup per CU); each wave owns 32 queries.  A K/V tile loaded into
//    LDS serves all 256 queries.
//  * both products run on v_mfma_f32_32x32x16_bf16 with fp32 accumulation.
//    The score tile is computed transposed, S^T = K Q^T, so lane l of a wave
//    holds the scores of ONE query (l % 32) against 32 of the 64 keys of the
//    tile; its partner lane l ^ 32 holds the other 32.  Row max and row sum
//    are therefore in-lane plus one cross-half exchange.
//  * the output is accumulated transposed, O~^T = V^T P~^T: P~^T is exactly
//    the fp32 score accumulator converted in place to bf16 (no data
//    movement), and lane l holds 64 of the 128 output dims of its query, so
//    the rescale by exp2(m_old - m_new) is a per-lane multiply.
//  * K and V tiles (64 keys x 128 dims) go from HBM straight into LDS with
//    global_load_lds_dwordx4 (no VGPR staging; lane i of a load writes
//    bytes 16 i .. 16 i + 15 of a 1 KiB LDS block).  Rows are unpadded and
//    XOR-swizzled at 16-byte granularity (K: slot = chunk ^ (row % 16); V:
//    slot = chunk ^ 4 (row % 4)) so that the K operand reads and the
//    transposing V reads are free of bank conflicts.
//  * ping-pong: the two waves of each SIMD belong to groups A (waves 0-3)
//    and B (waves 4-7) that run half a tile apart, separated by barriers.
//    Each wave alternates a softmax phase (vector ALU: masks, maximum,
//    exponentials, bf16 P~) and an MFMA phase (P~V of this tile, then the
//    scores of the next tile), so on every SIMD the matrix cores work for one
//    wave while the other exponentiates.  K and V are double-buffered; each
//    tile's loads are issued two phases before first use.
//  * the V^T operand is read with the gfx950 transposing LDS read
//    (ds_read_b64_tr_b16): in each 16-lane group, lane i points at
//    V[k0 + i/4][d0 + 4 (i%4) .. +3] and lane j receives V[k0 + e][d0 + j],
//    e = 0..3 -- four consecutive keys of one dim, the operand layout.
//  * rows at or past the valid length are never loaded: their loads are
//    clamped to the last valid row, so LDS only ever holds finite valid data
//    and NaN padding cannot reach an MFMA (0 * NaN = NaN); their scores are
//    masked to -inf, so they add exactly zero.
//  * the reference maximum is only raised (and O~, l rescaled) when a score
//    exceeds it by more than 2^8 in weight ([P3] "Precision, and what can
//    still go wrong": any reference that keeps the weights bounded works;
//    the running maximum is the tightest one), so after the first tiles the
//    rescale is skipped by a wave-uniform branch.
//  * blocks are ordered heaviest-first for causal masks, and each
//    (batch, head)'s query blocks are kept on one XCD (shared L2 for K/V)
//    when the head count divides evenly by 8.
#include "osm_device.h"
#include "osm_internal.h"

namespace osm {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));

constexpr int D = 128;           // head dim
constexpr int NW = 8;            // wavefronts per workgroup (two per SIMD)
constexpr int BQ = 32 * NW;      // queries per workgroup
constexpr int BK = 64;           // keys per tile
constexpr int NT = 64 * NW;      // threads per workgroup
constexpr int ROWB = D * 2;      // bytes per K/V row in LDS (unpadded)
constexpr int TILEB = BK * ROWB; // bytes per K or V tile (16 KiB)

typedef short s16x4 __attribute__((ext_vector_type(4)));

// transposing LDS read: see the header comment for the lane layout
__device__ __forceinline__ bf16x4 lds_read_tr(const uint16_t *p) {
    const s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (s16x4 __attribute__((address_space(3))) *)(p));
    return __builtin_bit_cast(bf16x4, r);
}

__device__ __forceinline__ int clampi(int v, int lo, int hi) { return v < lo ? lo : (v > hi ? hi : v); }

// Workgroup barrier without a memory fence; the empty asm statements keep
// the compiler from moving LDS accesses across it.  Callers wait for their
// own outstanding memory operations first.
__device__ __forceinline__ void tile_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

__global__ void __launch_bounds__(NT, 1)
attn_fwd_bf16_d128(const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K,
                   const uint16_t *__restrict__ V, uint16_t *__restrict__ O,
                   float *__restrict__ LSE, int B, int Hq, int Hkv, int Nq, int Nk,
                   const int32_t *__restrict__ seqlens_q, const int32_t *__restrict__ seqlens_k,
                   float scale_log2, int causal, int nqb, int xcd_heads) {
    // K buffers 0, 1 and V buffers 0, 1, 16 KiB each
    __shared__ __attribute__((aligned(1024))) uint8_t lds[4 * TILEB];

    // ---- which (batch, head, query block) ------------------------------
    const int L = blockIdx.x;
    int head, qrev;
    if (xcd_heads) {
        // hardware places block L on XCD L % 8; give every XCD whole heads
        // (head % 8 == XCD) and run one head's query blocks back to back
        // (heaviest first), so the blocks resident on an XCD share a few
        // heads' K and V in its L2.
        const int xcd = L & 7, slot = L >> 3;
        qrev = slot % nqb;
        head = (slot / nqb) * 8 + xcd;
    } else {
        head = L / nqb;
        qrev = L % nqb;
    }
    // the integer divisions above run on the vector ALU; the results are
    // uniform, so move them back to scalar registers
    head = __builtin_amdgcn_readfirstlane(head);
    qrev = __builtin_amdgcn_readfirstlane(qrev);
    const int qb = causal ? (nqb - 1 - qrev) : qrev;
    const int b = head / Hq, h = head % Hq;
    const int kvh = h / (Hq / Hkv);
    // lengths and the wave index are uniform: keep them in scalar registers
    // so that every tile-level decision is a scalar branch
    const int Lq = __builtin_amdgcn_readfirstlane(seqlens_q ? clampi(seqlens_q[b], 0, Nq) : Nq);
    const int Lk = __builtin_amdgcn_readfirstlane(seqlens_k ? clampi(seqlens_k[b], 0, Nk) : Nk);

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 5, c = lane & 31;
    // ping-pong groups: waves 0-3 (A) and 4-7 (B), one of each per SIMD.  The
    // two waves of a SIMD take adjacent 32-query blocks.
    const bool grpB = wave >= 4;
    const int q0 = qb * BQ;
    const int qw0 = q0 + 64 * (wave & 3) + (grpB ? 32 : 0);
    const int qi = qw0 + c;

    const size_t qhead = (size_t)(b * Hq + h) * Nq;
    const uint16_t *Kh = K + (size_t)(b * Hkv + kvh) * Nk * D;
    const uint16_t *Vh = V + (size_t)(b * Hkv + kvh) * Nk * D;

    if (q0 >= Lq) {
        // every row of this block is padding: O = 0, LSE = -inf
        const int rows = min(BQ, Nq - q0);
        for (int i = tid; i < rows * (D / 8); i += NT) {
            const int r = i / (D / 8), d8 = i % (D / 8);
            *reinterpret_cast<uint4 *>(O + (qhead + q0 + r) * D + d8 * 8) = make_uint4(0, 0, 0, 0);
        }
        if (LSE)
            for (int r = tid; r < rows; r += NT) LSE[qhead + q0 + r] = kNegInf;
        return;
    }

    // keys that can be visible to some query of this block
    int kend = Lk;
    if (causal) kend = min(kend, min(q0 + BQ, Lq));
    const int ntiles = (kend + BK - 1) / BK;
    // tiles this wave computes: none if all its queries are padding; with a
    // causal mask only tiles starting at or below its last query
    int wtiles = (qw0 >= Lq) ? 0 : ntiles;
    if (causal) wtiles = min(wtiles, (qw0 + 31) / BK + 1);

    // ---- Q fragment (B operand of S^T = K Q^T), kept in registers -------
    // lane l holds Q[qi][64 g + 8 ks + 0..7] for ks = 0..7
    bf16x8 qf[8];
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
        uint4 w = make_uint4(0, 0, 0, 0);
        if (qi < Lq) w = *reinterpret_cast<const uint4 *>(Q + (qhead + qi) * D + 64 * g + 8 * ks);
        qf[ks] = __builtin_bit_cast(bf16x8, w);
    }

    f32x16 oacc[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[dt][i] = 0.0f;
    f32x16 sacc[2];                     // S^T of the current tile
    bf16x8 pb[2][2];                    // P~^T of the current tile (bf16)
    float m = kNegInf;   // reference maximum of raw scores q.k for query qi
    float msub = 0.0f;   // m * scale * log2(e) (0 while m = -inf)
    float l = 0.0f;      // this lane's half of the running sum (same reference m)
    constexpr float kLazy = 8.0f;                 // allowed growth, base-2 units
    const float lazy_raw = kLazy / scale_log2;    // the same in raw score units

    // ---- direct HBM -> LDS tile loads -----------------------------------
    // K tiles are loaded by group B, V tiles by group A.  Load j (0..15) of a
    // tile writes LDS rows 4j .. 4j+3; wave w issues j = 4 i + (w % 4).  Lane
    // l fills row 4j + l/16, slot l%16, which holds global 16-byte chunk
    // (slot ^ swizzle(row)).  Rows past Lk are clamped.
    constexpr int LPT = 4;            // 1 KiB loads per wave per tile
    const int gw = wave & 3;          // wave index within its group
    int loff[LPT], lrow[LPT];
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
        const int j = 4 * i + gw;
        const int row = 4 * j + (lane >> 4);
        const int slot = lane & 15;
        lrow[i] = row;
        loff[i] = row * D + (grpB ? (slot ^ (row & 15)) : (slot ^ ((row & 3) << 2))) * 8;
    }
    auto load_tile = [&](const uint16_t *src, uint8_t *dst, int j0) __attribute__((always_inline)) {
        const uint16_t *tb = src + (size_t)j0 * D;
        const bool tail = (j0 + BK > Lk);
#pragma unroll
        for (int i = 0; i < LPT; ++i) {
            const int j = 4 * i + gw;
            int off = loff[i];
            if (tail) off += (min(j0 + lrow[i], Lk - 1) - (j0 + lrow[i])) * D;
            __builtin_amdgcn_global_load_lds(
                (const void __attribute__((address_space(1))) *)(tb + off),
                (void __attribute__((address_space(3))) *)(dst + j * 1024), 16, 0, 0);
        }
    };

    // per-lane LDS byte offsets (within a tile) of the QK A operand: row
    // 32 mt + c, chunk 8 g + ks -> slot (8 g + ks) ^ (c % 16)
    const int ka_row = c * ROWB;
    const int ka_sb = (8 * g) ^ (c & 15);
    // transposing V read: 16-lane group q = lane/16, index i = lane%16:
    // row kb + i/4 (kb a multiple of 4), dims 32 dt + 16 (q%2) + 4 (i%4) ..+3
    const int trq = lane >> 4, tri = lane & 15;
    const int tr_row = 4 * (trq >> 1) + (tri >> 2);
    const int tr_sw = (tri >> 2) << 2;                  // 4 * (row % 4)
    const int tr_half = (tri & 1) * 8;

    // S^T = K Q^T (raw scores): lane holds key 32 mt + 8 r + 4 g + u of the
    // tile in sacc[mt][4 r + u], query qi
    auto qk = [&](const uint8_t *Kb) __attribute__((always_inline)) {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int i = 0; i < 16; ++i) sacc[mt][i] = 0.0f;
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) {
                const bf16x8 a = *reinterpret_cast<const bf16x8 *>(
                    Kb + mt * 32 * ROWB + ka_row + ((ka_sb ^ ks) << 4));
                sacc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], sacc[mt], 0, 0, 0);
            }
        }
        // one operand read per MFMA, one ahead: bounded register footprint
        // (the other wave of the SIMD covers the LDS latency)
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
        for (int i = 0; i < 14; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    };

    // O~^T += V^T P~^T.  A operand, lane l, dim row 32 dt + c: keys
    // 32 mt + 16 hh + 4 g + 0..3 and + 8, the same keys in the same order as
    // the B operand's elements
    auto pv = [&](const uint8_t *Vb) __attribute__((always_inline)) {
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
            // chunk of dims 32 dt + 16 (q%2) + 4 (i%4): 4 dt + 2 (q%2) + (i%4)/2
            const int chunk = 4 * dt + 2 * (trq & 1) + ((tri & 3) >> 1);
            const int cofs = ((chunk ^ tr_sw) << 4) + tr_half;
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    const uint8_t *base = Vb + (32 * mt + 16 * hh + tr_row) * ROWB + cofs;
                    const bf16x4 lo = lds_read_tr(reinterpret_cast<const uint16_t *>(base));
                    const bf16x4 hi = lds_read_tr(reinterpret_cast<const uint16_t *>(base + 8 * ROWB));
                    const bf16x8 a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
                    oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[mt][hh], oacc[dt], 0, 0, 0);
                }
        }
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
        for (int i = 0; i < 14; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
    };

    // softmax of tile t: masks, reference maximum, P~ = exp2(S - m), l
    auto softmax = [&](int t) __attribute__((always_inline)) {
        const int j0 = t * BK;
        const bool need_mask = (j0 + BK > Lk) || (causal && j0 + BK - 1 > qw0);
        if (need_mask) {
            // key j0 + 32 mt + 8 r + 4 g + u is visible iff it is <= lim
            const int lim = (causal ? min(Lk - 1, qi) : Lk - 1) - j0 - 4 * g;
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int r = 0; r < 4; ++r)
#pragma unroll
                    for (int u = 0; u < 4; ++u)
                        if (32 * mt + 8 * r + u > lim) sacc[mt][4 * r + u] = kNegInf;
        }
        float tmax;
        {
            float mx[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int mt = k >> 1, o = (k & 1) * 8;
                mx[k] = fmaxf(fmaxf(fmaxf(sacc[mt][o + 0], sacc[mt][o + 1]), fmaxf(sacc[mt][o + 2], sacc[mt][o + 3])),
                              fmaxf(fmaxf(sacc[mt][o + 4], sacc[mt][o + 5]), fmaxf(sacc[mt][o + 6], sacc[mt][o + 7])));
            }
            tmax = fmaxf(fmaxf(mx[0], mx[1]), fmaxf(mx[2], mx[3]));
            // the other 32 keys of this query sit in lane l ^ 32
            const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(tmax),
                                                             __float_as_uint(tmax), false, false);
            tmax = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
        }
        // The reference m only moves when some lane's tile maximum exceeds it
        // by more than kLazy (base-2 units): every weight is then at most
        // 2^kLazy, far from fp32/bf16 overflow, and the final O~/l and LSE do
        // not depend on which common reference was used.  When it moves, O~
        // and l are rescaled by exp2(m_old - m_new) (0 when m_old is -inf:
        // nothing accumulated yet).
        if (!__all(tmax <= m + lazy_raw)) {
            const float mn = fmaxf(m, tmax);
            const float alpha = (mn == kNegInf || m == mn) ? 1.0f
                              : (m == kNegInf ? 0.0f : fast_exp2((m - mn) * scale_log2));
            l *= alpha;
#pragma unroll
            for (int dt = 0; dt < 4; ++dt)
#pragma unroll
                for (int i = 0; i < 16; ++i) oacc[dt][i] *= alpha;
            m = mn;
            msub = (mn == kNegInf) ? 0.0f : mn * scale_log2;
        }
        float rs[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float p = fast_exp2(fmaf(sacc[mt][i], scale_log2, -msub));
                sacc[mt][i] = p;
                rs[i & 3] += p;
            }
        l += (rs[0] + rs[1]) + (rs[2] + rs[3]);
        // P~^T as bf16 B operands: k-step (mt, hh) = s[mt][8 hh .. 8 hh + 7]
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                f32x8 f;
#pragma unroll
                for (int e = 0; e < 8; ++e) f[e] = sacc[mt][8 * hh + e];
                pb[mt][hh] = __builtin_convertvector(f, bf16x8);
            }
    };

    // ---- schedule --------------------------------------------------------
    // Phases p = 0 .. 2 ntiles, separated by barriers.  Group A runs the
    // softmax of tile t in phase 2t and the MFMAs of tile t (P~V(t), then
    // S(t+1) = K(t+1) Q^T) in phase 2t+1; group B runs one phase later.  On
    // each SIMD one wave is in its MFMA phase while the other exponentiates.
    // K(j) lives in K buffer j%2 and is read in phases 2j-1 and 2j; V(j)
    // lives in V buffer j%2 and is read in phases 2j+1 and 2j+2.
    //  * group B loads K(t+2) at the start of its softmax phase 2t+1 (the
    //    buffer's previous tile was last read in phase 2t) and waits for it
    //    at the end of that phase;
    //  * group A loads V(t+1) at the end of its MFMA phase 2t+1 (the buffer's
    //    previous tile was last read in phase 2t) and waits for it at the end
    //    of its softmax phase 2t+2.
    // No wave reads LDS while its own loads are in flight.
    uint8_t *Kbuf0 = lds, *Kbuf1 = lds + TILEB, *Vbuf0 = lds + 2 * TILEB, *Vbuf1 = lds + 3 * TILEB;

    // prologue: K(0), K(1), V(0) resident; group A computes S(0)
    if (ntiles > 0) {
        if (grpB) {
            load_tile(Kh, Kbuf0, 0);
            if (ntiles > 1) load_tile(Kh, Kbuf1, BK);
        } else {
            load_tile(Vh, Vbuf0, 0);
        }
    }
    __builtin_amdgcn_s_waitcnt(0);   // nothing in flight (Q included)
    __syncthreads();
    if (!grpB && wtiles > 0) qk(Kbuf0);

    // Each iteration k covers phases 2k and 2k+1: group A runs softmax(k)
    // then the MFMAs of tile k; group B runs the MFMAs of tile k-1 then
    // softmax(k).  The two groups run separate loops that pass the same
    // barriers (two per iteration, ntiles + 1 iterations).
    if (!grpB) {
        for (int k = 0; k <= ntiles; ++k) {
            if (k < wtiles) softmax(k);
            __builtin_amdgcn_s_waitcnt(0x0070);      // vmcnt(0) lgkmcnt(0): own V loads landed
            tile_barrier();
            if (k < wtiles) pv((k & 1) ? Vbuf1 : Vbuf0);
            if (k + 1 < wtiles) qk(((k + 1) & 1) ? Kbuf1 : Kbuf0);
            __builtin_amdgcn_s_waitcnt(0xC07F);      // lgkmcnt(0): this wave's LDS reads done
            if (k + 1 < ntiles) load_tile(Vh, ((k + 1) & 1) ? Vbuf1 : Vbuf0, (k + 1) * BK);
            tile_barrier();
        }
    } else {
        for (int k = 0; k <= ntiles; ++k) {
            const int t = k - 1;
            if (t >= 0 && t < wtiles) pv((t & 1) ? Vbuf1 : Vbuf0);
            if (t + 1 < wtiles) qk(((t + 1) & 1) ? Kbuf1 : Kbuf0);
            __builtin_amdgcn_s_waitcnt(0xC07F);      // lgkmcnt(0)
            tile_barrier();
            if (k + 2 < ntiles) load_tile(Kh, (k & 1) ? Kbuf1 : Kbuf0, (k + 2) * BK);
            if (k < wtiles) softmax(k);
            __builtin_amdgcn_s_waitcnt(0x0070);      // vmcnt(0) lgkmcnt(0): own K loads landed
            tile_barrier();
        }
    }

    // ---- epilogue: O = O~ / l once, LSE = m + log l ------------------------
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(l), __float_as_uint(l), false, false);
    const float lt = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    const bool valid = (qi < Lq) && (lt > 0.0f);
    const float inv = valid ? 1.0f / lt : 0.0f;
    if (qi < Nq) {
        uint16_t *orow = O + (qhead + qi) * D;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                uint2 w;
                w.x = pack_bf16x2(oacc[dt][4 * r + 0] * inv, oacc[dt][4 * r + 1] * inv);
                w.y = pack_bf16x2(oacc[dt][4 * r + 2] * inv, oacc[dt][4 * r + 3] * inv);
                *reinterpret_cast<uint2 *>(orow + 32 * dt + 8 * r + 4 * g) = w;
            }
        if (LSE && g == 0)
            LSE[qhead + qi] = valid ? (m * scale_log2 + __log2f(lt)) * kLn2 : kNegInf;
    }
}

}  // namespace

hipError_t launch_attn_fwd(const AttnFwdArgs &a, hipStream_t s) {
    const int nqb = (a.seqlen_q + BQ - 1) / BQ;
    const int nheads = a.batch * a.heads_q;
    const int64_t blocks = (int64_t)nqb * nheads;
    if (blocks == 0) return hipSuccess;
    const int xcd_heads = (nheads % 8 == 0) ? nheads / 8 : 0;
    hipLaunchKernelGGL(attn_fwd_bf16_d128, dim3((unsigned)blocks), dim3(NT), 0, s,
                       static_cast<const uint16_t *>(a.q), static_cast<const uint16_t *>(a.k),
                       static_cast<const uint16_t *>(a.v), static_cast<uint16_t *>(a.o), a.lse,
                       a.batch, a.heads_q, a.heads_kv, a.seqlen_q, a.seqlen_k, a.seqlens_q,
                       a.seqlens_k, a.scale * kLog2e, a.causal, nqb, xcd_heads);
    return hipGetLastError();
}

}  // namespace osm
