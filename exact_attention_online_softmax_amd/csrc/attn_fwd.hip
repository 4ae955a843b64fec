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
//  * workgroup = 4 wavefronts = 128 queries; each wave owns 32 queries.
//  * both products run on v_mfma_f32_32x32x16_bf16 with fp32 accumulation.
//    The score tile is computed transposed, S^T = K Q^T, so lane l of a wave
//    holds the scores of ONE query (l % 32) against 32 of the 64 keys of the
//    tile; its partner lane l ^ 32 holds the other 32.  Row max and row sum
//    are therefore in-lane plus one cross-half exchange.
//  * the output is accumulated transposed, O~^T = V^T P~^T: P~^T is exactly
//    the fp32 score accumulator converted in place to bf16 (no data
//    movement), and lane l holds 64 of the 128 output dims of its query, so
//    the rescale by exp2(m_old - m_new) is a per-lane multiply.
//  * K and V tiles (64 keys x 128 dims) are staged row-major in LDS, double
//    buffered: the global loads of tile t+1 are issued into registers before
//    tile t is computed and written to the other LDS buffer afterwards, so
//    one barrier per tile separates the producers from the consumers.
//  * the V^T operand is read with the gfx950 transposing LDS read
//    (ds_read_b64_tr_b16): in each 16-lane group, lane i points at
//    V[k0 + i/4][d0 + 4 (i%4) .. +3] and lane j receives V[k0 + e][d0 + j],
//    e = 0..3 -- four consecutive keys of one dim, the operand layout.
//  * keys at or past the valid length are zero-filled in LDS (never
//    loaded), so NaN padding cannot reach an MFMA (0 * NaN = NaN).
//  * the O~ rescale is skipped when the maximum of no lane in the wave
//    moved (the factor is exactly 1 then).
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
constexpr int BQ = 128;          // queries per workgroup
constexpr int BK = 64;           // keys per tile
constexpr int NT = 256;          // threads per workgroup
constexpr int KP = D + 8;        // K row pitch in LDS (bf16 elements)
constexpr int VP = D + 32;       // V row pitch in LDS (bf16 elements): 80 dwords, so the
                                 // 4 rows of one transposing read fall in distinct banks

typedef short s16x4 __attribute__((ext_vector_type(4)));

// transposing LDS read: see the header comment for the lane layout
__device__ __forceinline__ bf16x4 lds_read_tr(const uint16_t *p) {
    const s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (s16x4 __attribute__((address_space(3))) *)(p));
    return __builtin_bit_cast(bf16x4, r);
}

__device__ __forceinline__ int clampi(int v, int lo, int hi) { return v < lo ? lo : (v > hi ? hi : v); }

__global__ void __launch_bounds__(NT, 2)
attn_fwd_bf16_d128(const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K,
                   const uint16_t *__restrict__ V, uint16_t *__restrict__ O,
                   float *__restrict__ LSE, int B, int Hq, int Hkv, int Nq, int Nk,
                   const int32_t *__restrict__ seqlens_q, const int32_t *__restrict__ seqlens_k,
                   float scale_log2, int causal, int nqb, int xcd_heads) {
    __shared__ __attribute__((aligned(16))) uint16_t Ks[2][BK * KP];
    __shared__ __attribute__((aligned(16))) uint16_t Vs[2][BK * VP];

    // ---- which (batch, head, query block) ------------------------------
    const int L = blockIdx.x;
    int head, qrev;
    if (xcd_heads) {
        // hardware places block L on XCD L % 8; give every XCD whole heads
        // (head % 8 == XCD) and walk its heads' blocks heaviest-first.
        const int xcd = L & 7, slot = L >> 3;
        const int nh = xcd_heads;           // heads per XCD
        qrev = slot / nh;
        head = (slot % nh) * 8 + xcd;
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
    const int q0 = qb * BQ;
    const int qw0 = q0 + wave * 32;
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
    float m = kNegInf;   // running max of raw scores q.k for query qi
    float l = 0.0f;      // this lane's half of the running sum (same reference m)

    // global -> registers for one tile: chunk = tid + NT*i -> (key = chunk/16,
    // 8-dim slice = chunk%16).  The loads are unconditional (rows past the
    // valid length are clamped to the last valid row, always in bounds) so
    // that no branch separates their issue from their use; the rows past
    // Lk are replaced by zeros when the tile is written to LDS.
    uint4 kreg[4], vreg[4];
    auto load_tile = [&](int j0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int chunk = tid + NT * i;
            const int kj = min(j0 + (chunk >> 4), Lk - 1), d8 = chunk & 15;
            kreg[i] = *reinterpret_cast<const uint4 *>(Kh + (size_t)kj * D + d8 * 8);
            vreg[i] = *reinterpret_cast<const uint4 *>(Vh + (size_t)kj * D + d8 * 8);
        }
    };
    auto store_tile = [&](int buf, int j0) {
        const bool tail = (j0 + BK > Lk);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int chunk = tid + NT * i;
            const int key = chunk >> 4, d8 = chunk & 15;
            uint4 kw = kreg[i], vw = vreg[i];
            if (tail && j0 + key >= Lk) {
                kw = make_uint4(0, 0, 0, 0);
                vw = make_uint4(0, 0, 0, 0);
            }
            *reinterpret_cast<uint4 *>(&Ks[buf][key * KP + d8 * 8]) = kw;
            *reinterpret_cast<uint4 *>(&Vs[buf][key * VP + d8 * 8]) = vw;
        }
    };

    // transposing-read addresses (element offsets within a V buffer) for
    // this lane: 16-lane group q = lane/16, index i = lane%16
    const int trq = lane >> 4, tri = lane & 15;
    const int tr_off = (4 * (trq >> 1) + (tri >> 2)) * VP + 16 * (trq & 1) + 4 * (tri & 3);

    if (ntiles > 0) {
        load_tile(0);
        store_tile(0, 0);
    }
    // nothing is left in flight when the loop starts (Q included), so the
    // loop's first MFMAs never wait on the next tile's prefetch
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    for (int t = 0; t < ntiles; ++t) {
        const int j0 = t * BK;
        const int buf = t & 1;
        const bool more = (t + 1 < ntiles);
        if (more) load_tile(j0 + BK);      // in flight while this tile is computed

        // this wave has something visible in this tile unless the tile is
        // above its causal diagonal or all its queries are padding
        const bool active = !((causal && qw0 + 31 < j0) || qw0 >= Lq);
        if (active) {
            const uint16_t *Kb = Ks[buf];
            const uint16_t *Vb = Vs[buf];
            // ---- S^T = K Q^T (raw scores) -------------------------------
            f32x16 s[2];
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int i = 0; i < 16; ++i) s[mt][i] = 0.0f;
#pragma unroll
            for (int ks = 0; ks < 8; ++ks) {
#pragma unroll
                for (int mt = 0; mt < 2; ++mt) {
                    const bf16x8 a = *reinterpret_cast<const bf16x8 *>(&Kb[(32 * mt + c) * KP + 64 * g + 8 * ks]);
                    s[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], s[mt], 0, 0, 0);
                }
            }
            // lane holds key j0 + 32 mt + 8 r + 4 g + u in s[mt][4 r + u], query qi

            // ---- masks (only on tiles that cross the length or the diagonal)
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
                            if (32 * mt + 8 * r + u > lim) s[mt][4 * r + u] = kNegInf;
            }

            // ---- online softmax update ----------------------------------
            float tmax = kNegInf;
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int i = 0; i < 16; i += 2) tmax = fmaxf(tmax, fmaxf(s[mt][i], s[mt][i + 1]));
            tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
            const float mn = fmaxf(m, tmax);
            float alpha, msub;
            if (mn == kNegInf) {          // nothing visible yet for this query
                alpha = 1.0f;
                msub = 0.0f;
            } else {
                alpha = (m == kNegInf) ? 0.0f : fast_exp2((m - mn) * scale_log2);
                msub = mn * scale_log2;
            }
            float rs = 0.0f;
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const float p = fast_exp2(fmaf(s[mt][i], scale_log2, -msub));
                    s[mt][i] = p;
                    rs += p;
                }
            l = fmaf(l, alpha, rs);
            m = mn;
            if (!__all(alpha == 1.0f)) {
#pragma unroll
                for (int dt = 0; dt < 4; ++dt)
#pragma unroll
                    for (int i = 0; i < 16; ++i) oacc[dt][i] *= alpha;
            }

            // ---- P~^T as bf16 B operands: k-step (mt, hh) = s[mt][8 hh .. 8 hh + 7]
            bf16x8 pb[2][2];
#pragma unroll
            for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    f32x8 f;
#pragma unroll
                    for (int e = 0; e < 8; ++e) f[e] = s[mt][8 * hh + e];
                    pb[mt][hh] = __builtin_convertvector(f, bf16x8);
                }

            // ---- O~^T += V^T P~^T -----------------------------------------
            // A operand, lane l, dim row 32 dt + c: keys 32 mt + 16 hh + 4 g + 0..3
            // and + 8, the same keys in the same order as the B operand
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) {
#pragma unroll
                for (int mt = 0; mt < 2; ++mt)
#pragma unroll
                    for (int hh = 0; hh < 2; ++hh) {
                        const uint16_t *base = Vb + tr_off + (32 * mt + 16 * hh) * VP + 32 * dt;
                        const bf16x4 lo = lds_read_tr(base);
                        const bf16x4 hi = lds_read_tr(base + 8 * VP);
                        const bf16x8 a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
                        oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[mt][hh], oacc[dt], 0, 0, 0);
                    }
            }
        }
        if (more) store_tile(buf ^ 1, j0 + BK);
        __syncthreads();
    }

    // ---- epilogue: O = O~ / l once, LSE = m + log l ------------------------
    const float lt = l + __shfl_xor(l, 32, 64);
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
