// attn_bwd.hip -- attention backward for gfx950 (bf16, head_dim 128 and 64),
// with the weights rebuilt from the stored log-sum-exp.
//
// [P3] "From weights to outputs", the log-sum-exp paragraph: lse is one
// number per query, and it is all a backward pass keeps to rebuild the
// weights, y_j = exp(s_j - lse).  The pages stop there; the gradients are
// the derivative of the forward definition, by the chain rule through
// o = sum_j y_j v_j and the softmax:
//   dV = P^T dO,  dP = dO V^T,  dS = P * (dP - D)  with D_i = sum_j P_ij dP_ij,
//   dQ = scale dS K,  dK = scale dS^T Q.
// D_i equals dO_i . O_i (O_i = sum_j P_ij v_j), which is how it is computed
// here: one dot product per row instead of a pass over the row of P.
//
// Two kernels, enqueued in order on one stream:
//  * attn_bwd_dq: query-major, laid out like the forward.  A workgroup owns
//    256 queries (32 per wave, eight waves, two per SIMD; Q and dO fragments
//    and the dQ accumulators in registers) and streams K and V tiles of
//    32 keys through a ring of three LDS slots: S^T = K Q^T, dP^T = V dO^T,
//    dS^T, and dQ^T += K^T dS^T.  Before its first tile it forms, per query
//    row, D = dO . O and the log-sum-exp in base-2 units (lse2 = lse log2 e,
//    so P = exp2(s scale log2 e - lse2)), and stores (lse2, D) for the next
//    kernel.  Rows that see no key (lse = -inf) get (lse2, D) = (+inf, 0):
//    their rebuilt weights are exactly 0 and they add nothing.
//  * attn_bwd_dkdv: key-major.  A workgroup owns 256 keys of one key/value
//    head, 32 per wave, eight waves (two per SIMD, so one wave's matrix
//    products overlap the other's exponentials and LDS reads); each wave's
//    K and V stay in registers as MFMA operands and its dK, dV accumulators
//    in the AGPRs.
//    Every query row that can see those keys -- all query heads that read
//    the key/value head -- streams through LDS, 64 rows of Q and dO per
//    stage, double-buffered.  Per 32-query block: S = Q K^T and dP = dO V^T
//    on the matrix cores (one key per lane column), P = exp2(S scale log2e
//    - lse2), dS = P (dP - D), then dV^T += dO^T P and dK^T += Q^T dS, the
//    transposed operands read from LDS with ds_read_b64_tr_b16.  dK and dV
//    sum over the whole head group in registers: no atomics.
// Splitting dQ from dK/dV computes S and dP twice (7 matrix products per
// score tile instead of 5) but needs no atomic accumulation, so the result
// is deterministic.
//
// Shared with the forward's design: bf16 operands with fp32 accumulation on
// v_mfma_f32_32x32x16_bf16; tiles go from HBM straight into LDS through
// buffer loads with LDS destination, whose range check turns rows past the
// valid length into zeros (NaN padding never reaches an MFMA); LDS rows are
// XOR-swizzled at 16-byte granularity.
//
// The two kernels are templates over the head dim, instantiated for 128
// and 64: at 64 a row is 128 bytes, a k-step loop has four steps instead of
// eight and a gradient two 32-dim output tiles instead of four.
#include "osm_device.h"
#include "osm_internal.h"

namespace osm {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

// per head dim: bytes per bf16 row, 16-byte chunks per row, rows per 1 KiB
// DMA block, k-steps of 16 dims, output tiles of 32 dims
template <int HD> struct BGeo {
    static constexpr int ROWB = HD * 2, CH = ROWB / 16, RPB = 1024 / ROWB, KS = HD / 16, NDT = HD / 32;
    static constexpr int kLogCH = CH == 16 ? 4 : 3;
};
constexpr float kPosInf = __builtin_inff();

// Buffer resource word 3 for raw dword access (DATA_FORMAT = 32 bits).
constexpr int kRsrcWord3 = 0x00020000;
// s_waitcnt encodings (gfx9): vmcnt in bits 3:0 and 15:14, lgkmcnt 11:8.
constexpr int kWaitVm0 = 0x0F70;

template <int N> struct Slot { static constexpr int value = N; };

__device__ __forceinline__ int clampi(int v, int lo, int hi) { return v < lo ? lo : (v > hi ? hi : v); }
__device__ __forceinline__ int rfl(int v) { return __builtin_amdgcn_readfirstlane(v); }

// 256-byte LDS rows hold 16 chunks of 16 bytes; chunk c of row r sits in
// slot c ^ swz(r), swz(r) = 4 (r % 4) + (r / 4) % 4.  The LDS serves 256
// bytes per cycle (64 banks of 4 bytes), so a read is free of bank
// conflicts when every group of lanes served together touches distinct
// 16-byte (row-wise reads: 16 lanes) or 8-byte (transposing reads: 32
// lanes) slots of a 256-byte window.  Over 16 consecutive rows swz takes 16
// distinct values, so the row-wise 16-byte operand reads are conflict-free;
// over rows 4a .. 4a+3 its upper two bits take four distinct values, so a
// transposing read of four adjacent chunks from those rows covers four
// disjoint groups of four slots.  (The previous swizzle, a rotation of the
// row's low four bits, left the transposing reads two-way conflicted:
// rocprofv3 counted SQ_LDS_BANK_CONFLICT at 29% of the LDS active cycles.)
__device__ __forceinline__ int swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

// 128-byte rows (head dim 64) hold 8 chunks; two rows share a 256-byte
// window, so chunk c of row r lands in 16-byte bank group 8 (r % 2) + slot.
// swz64(r) = 4 ((r / 2) % 2) + (r / 4) % 4 takes 8 distinct values over the
// even rows of any 16 consecutive ones and over the odd rows, so the
// row-wise reads stay conflict-free; rows 4a and 4a + 2 (and 4a + 1, 4a + 3)
// differ in its bit 2, so a transposing read of four adjacent chunks from
// rows 4a .. 4a + 3 covers disjoint halves of each window.
__device__ __forceinline__ int swz64(int r) { return (((r >> 1) & 1) << 2) | ((r >> 2) & 3); }
template <int HD> __device__ __forceinline__ int swzh(int r) { return HD == 128 ? swz(r) : swz64(r); }

// gfx950 transposing LDS read: in each 16-lane group, lane i points at
// row k0 + i/4, columns d0 + 4 (i%4) .. +3 of a row-major bf16 tile, and
// lane j receives rows k0 .. k0+3 of column d0 + j.
__device__ __forceinline__ bf16x4 lds_read_tr(const uint8_t *p) {
    const s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (s16x4 __attribute__((address_space(3))) *)(p));
    return __builtin_bit_cast(bf16x4, r);
}

// Accumulation MFMA with the accumulator pinned to AGPRs (attn_bwd_dkdv).
// The products whose results the vector ALU reads (S, dP) write VGPRs (the
// builtins' VGPR form); dK and dV, read only at the end, fit only in the
// AGPRs, so their MFMAs are inline assembly.  (A kernel that uses AGPRs gets
// at most half of its registers as VGPRs; attn_bwd_dq, whose 64 accumulator
// registers fit beside everything else, keeps them in VGPRs and has the
// whole budget for them.)  The hazard recognizer does not look into inline
// assembly: two wait states let a VALU-written operand settle before the
// MFMA reads it.
//
// NOP: the two wait states, for the first MFMA that reads a P or dS operand
// converted just before it.  Later uses of the same operand come after that
// MFMA and the LDS reads of their own A operand, so they need none (checked
// on the generated code by the test suite).
template <bool NOP>
__device__ __forceinline__ void mfma_acc(f32x16 &acc, const bf16x8 &a, const bf16x8 &b) {
    if constexpr (NOP)
        asm("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
    else
        asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}

__device__ __forceinline__ void acc_zero(f32x16 &acc, const bf16x8 &z) {
    asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %1, 0" : "=a"(acc) : "v"(z));
}

// Before ordinary code reads accumulators written by mfma_acc: wait out the
// MFMA result latency (24 wait states; the compiler's model asks for 12).
__device__ __forceinline__ void acc_settle(f32x16 (&o)[4]) {
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+a"(o[0]), "+a"(o[1]), "+a"(o[2]), "+a"(o[3]));
}
__device__ __forceinline__ void acc_settle(f32x16 (&o)[2]) {
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+a"(o[0]), "+a"(o[1]));
}

__device__ __forceinline__ bf16x8 cat4(const bf16x4 &lo, const bf16x4 &hi) {
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

__device__ __forceinline__ bf16x8 to_bf16x8(const float *f) {
    f32x8 v;
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = f[k];
    return __builtin_convertvector(v, bf16x8);
}

// Workgroup barrier without a memory fence; callers wait for their own
// outstanding loads first.  The empty asm statements keep the compiler
// from moving LDS accesses across it.
__device__ __forceinline__ void tile_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

__device__ __forceinline__ void dma16(const __amdgpu_buffer_rsrc_t &r, uint8_t *lds, uint32_t off) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (void __attribute__((address_space(3))) *)lds, 16, off, 0, 0, 0);
}

__device__ __forceinline__ void dma4(const __amdgpu_buffer_rsrc_t &r, void *lds, uint32_t off) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (void __attribute__((address_space(3))) *)lds, 4, off, 0, 0, 0);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, bytes, kRsrcWord3);
}

// ---------------------------------------------------------------------------
// attn_bwd_dkdv
// ---------------------------------------------------------------------------
constexpr int KV_NW = 8;                       // wavefronts per workgroup (two per SIMD)
constexpr int KV_KW = 32;                      // keys per wavefront
constexpr int KV_BK = KV_KW * KV_NW;           // keys per workgroup
constexpr int KV_NT = 64 * KV_NW;
// query rows per LDS stage: 64 keeps the four stage arrays (Q and dO, two
// stages) within the first 64 KiB of LDS, where operand reads address them
// with the 16-bit immediate offset; with 128 every read of the second
// stage's arrays needed its address computed (an OR per read)
constexpr int KV_QT = 64;
template <int HD> constexpr int kKvStb = KV_QT * BGeo<HD>::ROWB;   // bytes of Q (or dO) per stage
static_assert(KV_QT % 32 == 0 && KV_QT / 32 <= KV_NW,
              "waves 0 .. KV_QT/32-1 load a stage's (lse2, D), 256 bytes each");

template <bool CAUSAL, int HD>
__global__ void __launch_bounds__(KV_NT, 1)
attn_bwd_dkdv(const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K,
              const uint16_t *__restrict__ V, const uint16_t *__restrict__ dO,
              const float2 *__restrict__ LD, uint16_t *__restrict__ dK, uint16_t *__restrict__ dV,
              int Hq, int Hkv, int Nq, int Nk, const int32_t *__restrict__ seqlens_q,
              const int32_t *__restrict__ seqlens_k, float scale_log2, float scale, int nkb,
              int xcd_heads) {
    using G = BGeo<HD>;
    constexpr int ROWB = G::ROWB, CH = G::CH, RPB = G::RPB, KS = G::KS, NDT = G::NDT;
    constexpr int KV_STB = kKvStb<HD>;
    constexpr int KV_BLK = KV_STB / 1024 / KV_NW;  // 1 KiB DMA blocks per wave per array per stage
    static_assert(KV_BLK >= 1, "every wave loads whole 1 KiB blocks of a stage");
    // two stages of Q rows, dO rows and (lse2, D)
    __shared__ __attribute__((aligned(1024))) uint8_t qs0[KV_STB], qs1[KV_STB];
    __shared__ __attribute__((aligned(1024))) uint8_t os0[KV_STB], os1[KV_STB];
    __shared__ __attribute__((aligned(1024))) float2 ls0[KV_QT], ls1[KV_QT];

    // ---- which (batch, key/value head, key block) -----------------------
    const int L = blockIdx.x;
    int head, kb;
    if (xcd_heads) {
        // block L runs on XCD L % 8: keep each head's key blocks on one XCD
        // so that they share its Q and dO in that XCD's L2
        const int xcd = L & 7, slot = L >> 3;
        kb = slot % nkb;
        head = (slot / nkb) * 8 + xcd;
    } else {
        head = L / nkb;
        kb = L % nkb;
    }
    // with a causal mask the first key blocks see the most queries: they
    // come first
    head = rfl(head);
    kb = rfl(kb);
    const int b = head / Hkv, hkv = head % Hkv;
    const int group = Hq / Hkv;
    const int Lq = rfl(seqlens_q ? clampi(seqlens_q[b], 0, Nq) : Nq);
    const int Lk = rfl(seqlens_k ? clampi(seqlens_k[b], 0, Nk) : Nk);

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = rfl(tid >> 6);
    const int g = lane >> 5, c = lane & 31;
    const int kb0 = kb * KV_BK;
    const int kw0 = kb0 + KV_KW * wave;          // this wave's first key; lane column c is key kw0 + c
    const size_t kvrow0 = (size_t)(b * Hkv + hkv) * Nk;

    if (kb0 >= Lk) {
        // every key of this block is padding: zero gradients
        const int rows = min(KV_BK, Nk - kb0);
        for (int i = tid; i < rows * (HD / 8); i += KV_NT) {
            const size_t off = (kvrow0 + kb0 + i / (HD / 8)) * HD + (i % (HD / 8)) * 8;
            *reinterpret_cast<uint4 *>(dK + off) = make_uint4(0, 0, 0, 0);
            *reinterpret_cast<uint4 *>(dV + off) = make_uint4(0, 0, 0, 0);
        }
        return;
    }

    // ---- K and V of this wave's keys, as B operands ----------------------
    // lane (g, c) holds K[kw0 + c][(HD / 2) g + 8 ks + 0..7] for k-step ks;
    // the A operands (rows of Q, dO) use the same order of the head dim
    bf16x8 kf[KS], vf[KS];
    {
        const int key = kw0 + c;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            uint4 wk = make_uint4(0, 0, 0, 0), wv = make_uint4(0, 0, 0, 0);
            if (key < Lk) {
                wk = *reinterpret_cast<const uint4 *>(K + (kvrow0 + key) * HD + (HD / 2) * g + 8 * ks);
                wv = *reinterpret_cast<const uint4 *>(V + (kvrow0 + key) * HD + (HD / 2) * g + 8 * ks);
            }
            kf[ks] = __builtin_bit_cast(bf16x8, wk);
            vf[ks] = __builtin_bit_cast(bf16x8, wv);
        }
    }
    f32x16 dka[NDT], dva[NDT];
    {
        const bf16x8 z8 = {};
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
            acc_zero(dka[dt], z8);
            acc_zero(dva[dt], z8);
        }
    }

    // ---- the query rows to visit: every head of the group, rows qbeg..Lq-1
    // (with a causal mask, queries before kb0 see none of these keys)
    const int qbeg = CAUSAL ? (kb0 / KV_QT) * KV_QT : 0;
    const int per_head = (Lq > qbeg) ? (Lq - qbeg + KV_QT - 1) / KV_QT : 0;
    const int nst = group * per_head;

    // DMA of one stage: wave w fills 1 KiB blocks KV_BLK w .. +KV_BLK-1 (RPB
    // rows each) of the Q and dO arrays, lane l row RPB blk + l/CH, slot l%CH
    // (holding global chunk slot ^ swz(row)); waves 0 .. KV_QT/32-1 also load
    // (lse2, D) of rows 32 w .. 32 w + 31.  Rows at or past Lq read as zeros: their Q
    // and dO are 0, so whatever their weight, they add nothing.
    uint32_t dmo[KV_BLK];
#pragma unroll
    for (int i = 0; i < KV_BLK; ++i) {
        const int row = RPB * (KV_BLK * wave + i) + (lane >> G::kLogCH);
        dmo[i] = row * ROWB + (((lane & (CH - 1)) ^ swzh<HD>(row)) << 4);
    }
    auto issue = [&](uint8_t *qd, uint8_t *od, float2 *ld, int st) __attribute__((always_inline)) {
        const int hq = hkv * group + st / per_head;
        const int q0 = qbeg + (st % per_head) * KV_QT;
        const size_t row0 = (size_t)(b * Hq + hq) * Nq + q0;
        const int nrows = Lq - q0;               // > 0
        const __amdgpu_buffer_rsrc_t rq = rsrc(Q + row0 * HD, nrows * ROWB);
        const __amdgpu_buffer_rsrc_t ro = rsrc(dO + row0 * HD, nrows * ROWB);
        const __amdgpu_buffer_rsrc_t rl = rsrc(LD + row0, nrows * 8);
#pragma unroll
        for (int i = 0; i < KV_BLK; ++i) dma16(rq, qd + (KV_BLK * wave + i) * 1024, dmo[i]);
#pragma unroll
        for (int i = 0; i < KV_BLK; ++i) dma16(ro, od + (KV_BLK * wave + i) * 1024, dmo[i]);
        if (wave < KV_QT / 32) dma4(rl, reinterpret_cast<uint8_t *>(ld) + 256 * wave, 256 * wave + 4 * lane);
    };

    // operand offsets within a 32-row block of a stage.  Row-wise A operand
    // (rows of Q or dO): lane (g, c) reads row c, chunk (CH / 2) g + ks.
    uint32_t aoff[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) aoff[ks] = c * ROWB + (((((CH / 2) * g) + ks) ^ swzh<HD>(c)) << 4);
    // transposed A operand (Q^T or dO^T, dim rows 32 dt + c): 16-lane group
    // t = lane/16, index i = lane%16 reads query row 4 (t/2) + i/4 (and that
    // + 8), dims 32 dt + 16 (t%2) + 4 (i%4) .. +3
    uint32_t tlo[NDT], thi[NDT];
    {
        const int t = lane >> 4, i = lane & 15;
        const int row = 4 * (t >> 1) + (i >> 2);
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
            const int chunk = 4 * dt + 2 * (t & 1) + ((i & 3) >> 1);
            tlo[dt] = row * ROWB + ((chunk ^ swzh<HD>(row)) << 4) + (i & 1) * 8;
            thi[dt] = (row + 8) * ROWB + ((chunk ^ swzh<HD>(row + 8)) << 4) + (i & 1) * 8;
        }
    }

    // one block of 32 query rows (rows 32 sb .. of the stage, first query
    // qs0): the acc element 4 r + u of lane (g, c) is query qs0 + 8 r + 4 g + u,
    // key kw0 + c
    auto block = [&](const uint8_t *qd, const uint8_t *od, const float2 *ld, int sb, int qs0)
        __attribute__((always_inline)) {
        const uint8_t *qb = qd + 32 * sb * ROWB, *ob = od + 32 * sb * ROWB;
        f32x16 s = {}, dp = {};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const bf16x8 aq = *reinterpret_cast<const bf16x8 *>(qb + aoff[ks]);
            const bf16x8 ao = *reinterpret_cast<const bf16x8 *>(ob + aoff[ks]);
            s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aq, kf[ks], s, 0, 0, 0);
            dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ao, vf[ks], dp, 0, 0, 0);
        }
        float p[16], ds[16];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float4 x0 = *reinterpret_cast<const float4 *>(ld + 32 * sb + 8 * r + 4 * g);
            const float4 x1 = *reinterpret_cast<const float4 *>(ld + 32 * sb + 8 * r + 4 * g + 2);
            const float l2[4] = {x0.x, x0.z, x1.x, x1.z};
            const float dd[4] = {x0.y, x0.w, x1.y, x1.w};
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const float e = fast_exp2(fmaf(s[4 * r + u], scale_log2, -l2[u]));
                p[4 * r + u] = e;
                ds[4 * r + u] = e * (dp[4 * r + u] - dd[u]);
            }
        }
        // causal: only a block that crosses the diagonal (some key of the
        // wave after some query of the block) has weights to zero, so the
        // selects sit behind a wave-uniform branch.  P and dS are both
        // zeroed there, which keeps every value the branch joins already
        // live in the unmasked body (80 VALU per block against 128 when
        // every block selected).
        if (CAUSAL && kw0 + 31 > qs0) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const bool after = kw0 + c > qs0 + 8 * r + 4 * g + u;
                    p[4 * r + u] = after ? 0.0f : p[4 * r + u];
                    ds[4 * r + u] = after ? 0.0f : ds[4 * r + u];
                }
        }
        bf16x8 pb[2], db[2];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            pb[hh] = to_bf16x8(p + 8 * hh);
            db[hh] = to_bf16x8(ds + 8 * hh);
        }
        // dV^T += dO^T P, dK^T += Q^T dS: k-step hh covers queries
        // 16 hh + 4 g + 0..3 and + 8, the elements 8 hh .. 8 hh + 7 above
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) {
                const bf16x8 ao = cat4(lds_read_tr(ob + 16 * hh * ROWB + tlo[dt]),
                                       lds_read_tr(ob + 16 * hh * ROWB + thi[dt]));
                const bf16x8 aq = cat4(lds_read_tr(qb + 16 * hh * ROWB + tlo[dt]),
                                       lds_read_tr(qb + 16 * hh * ROWB + thi[dt]));
                if (dt == 0) {
                    mfma_acc<true>(dva[dt], ao, pb[hh]);
                    mfma_acc<true>(dka[dt], aq, db[hh]);
                } else {
                    mfma_acc<false>(dva[dt], ao, pb[hh]);
                    mfma_acc<false>(dka[dt], aq, db[hh]);
                }
            }
    };

    // one stage: all of this wave's loads of it are done, the barrier makes
    // every wave's visible and frees the other buffers (every wave is past
    // the previous stage), which receive the next stage
    auto stage = [&](auto S, int st) __attribute__((always_inline)) {
        constexpr int s = decltype(S)::value;
        uint8_t *qd = s ? qs1 : qs0;
        uint8_t *od = s ? os1 : os0;
        float2 *ld = s ? ls1 : ls0;
        __builtin_amdgcn_s_waitcnt(kWaitVm0);
        tile_barrier();
        if (st + 1 < nst) issue(s ? qs0 : qs1, s ? os0 : os1, s ? ls0 : ls1, st + 1);
        const int q0 = qbeg + (st % per_head) * KV_QT;
#pragma unroll
        for (int sb = 0; sb < KV_QT / 32; ++sb) {
            const int qs0 = q0 + 32 * sb;
            // rows all padding, or (causal) every key after every query
            const bool skip = (qs0 >= Lq) || (CAUSAL && kw0 > qs0 + 31);
            if (!skip) block(qd, od, ld, sb, qs0);
        }
    };

    if (nst > 0) issue(qs0, os0, ls0, 0);
    for (int st = 0; st < nst; st += 2) {
        stage(Slot<0>{}, st);
        if (st + 1 < nst) stage(Slot<1>{}, st + 1);
    }

    // ---- epilogue: dK = scale dK~, dV; keys past Lk get zeros --------------
    acc_settle(dka);
    acc_settle(dva);
    const int key = kw0 + c;
    if (key < Nk) {
        const bool valid = key < Lk;
        uint16_t *dkr = dK + (kvrow0 + key) * HD;
        uint16_t *dvr = dV + (kvrow0 + key) * HD;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                uint2 wk, wv;
                wk.x = valid ? pack_bf16x2_hw(dka[dt][4 * r] * scale, dka[dt][4 * r + 1] * scale) : 0u;
                wk.y = valid ? pack_bf16x2_hw(dka[dt][4 * r + 2] * scale, dka[dt][4 * r + 3] * scale) : 0u;
                wv.x = valid ? pack_bf16x2_hw(dva[dt][4 * r], dva[dt][4 * r + 1]) : 0u;
                wv.y = valid ? pack_bf16x2_hw(dva[dt][4 * r + 2], dva[dt][4 * r + 3]) : 0u;
                *reinterpret_cast<uint2 *>(dkr + 32 * dt + 8 * r + 4 * g) = wk;
                *reinterpret_cast<uint2 *>(dvr + 32 * dt + 8 * r + 4 * g) = wv;
            }
    }
}

// ---------------------------------------------------------------------------
// attn_bwd_dq
// ---------------------------------------------------------------------------
constexpr int DQ_NQB = 1;                      // 32-query blocks per wavefront
constexpr int DQ_QW = 32 * DQ_NQB;             // queries per wavefront
constexpr int DQ_NW = 256 / DQ_QW;             // wavefronts per workgroup (two per SIMD)
constexpr int DQ_BQ = DQ_QW * DQ_NW;           // queries per workgroup
constexpr int DQ_BK = 32;                      // keys per tile
constexpr int DQ_NT = 64 * DQ_NW;
template <int HD> constexpr int kDqTileb = DQ_BK * BGeo<HD>::ROWB;   // bytes per K or V tile

template <int HD>
__global__ void __launch_bounds__(DQ_NT, 1)
attn_bwd_dq(const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K,
            const uint16_t *__restrict__ V, const uint16_t *__restrict__ O,
            const uint16_t *__restrict__ dO, const float *__restrict__ LSE,
            float2 *__restrict__ LD, uint16_t *__restrict__ dQ, int Hq, int Hkv, int Nq,
            int Nk, const int32_t *__restrict__ seqlens_q, const int32_t *__restrict__ seqlens_k,
            float scale_log2, float scale, int causal, int nqb, int xcd_heads) {
    using G = BGeo<HD>;
    constexpr int ROWB = G::ROWB, CH = G::CH, RPB = G::RPB, KS = G::KS, NDT = G::NDT;
    constexpr int DQ_TILEB = kDqTileb<HD>;
    // 1 KiB DMA blocks per K (or V) tile, and loads per wave per tile: every
    // wave loads one block of K and one of V (head dim 128), or one block of
    // K (waves 0-3) or of V (waves 4-7, head dim 64)
    constexpr int NBLK = DQ_TILEB / 1024;
    constexpr int LPT = 2 * NBLK / DQ_NW;
    static_assert(LPT >= 1 && LPT * DQ_NW == 2 * NBLK, "whole 1 KiB loads per wave per tile");
    // wait for this wave's loads of one tile, those of the next in flight
    constexpr int kWaitTile = 0x0F70 | LPT;
    // ring of three K slots and three V slots
    __shared__ __attribute__((aligned(1024))) uint8_t k0[DQ_TILEB], k1[DQ_TILEB], k2[DQ_TILEB];
    __shared__ __attribute__((aligned(1024))) uint8_t v0[DQ_TILEB], v1[DQ_TILEB], v2[DQ_TILEB];

    const int L = blockIdx.x;
    int head, qrev;
    if (xcd_heads) {
        const int xcd = L & 7, slot = L >> 3;
        qrev = slot % nqb;
        head = (slot / nqb) * 8 + xcd;
    } else {
        head = L / nqb;
        qrev = L % nqb;
    }
    head = rfl(head);
    qrev = rfl(qrev);
    // with a causal mask the last query blocks see the most keys: they come first
    const int qb0 = causal ? (nqb - 1 - qrev) : qrev;
    const int b = head / Hq, h = head % Hq;
    const int kvh = h / (Hq / Hkv);
    const int Lq = rfl(seqlens_q ? clampi(seqlens_q[b], 0, Nq) : Nq);
    const int Lk = rfl(seqlens_k ? clampi(seqlens_k[b], 0, Nk) : Nk);

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = rfl(tid >> 6);
    const int g = lane >> 5, c = lane & 31;
    const int q0 = qb0 * DQ_BQ;
    const int qw0 = q0 + DQ_QW * wave;           // queries qw0 + 32 qb + c
    const size_t qrow0 = (size_t)(b * Hq + h) * Nq;
    const uint16_t *Kh = K + (size_t)(b * Hkv + kvh) * Nk * HD;
    const uint16_t *Vh = V + (size_t)(b * Hkv + kvh) * Nk * HD;

    if (q0 >= Lq || Lk == 0) {
        // every row of this block is padding, or there is no key: dQ = 0
        const int rows = min(DQ_BQ, Nq - q0);
        for (int i = tid; i < rows * (HD / 8); i += DQ_NT)
            *reinterpret_cast<uint4 *>(dQ + (qrow0 + q0 + i / (HD / 8)) * HD + (i % (HD / 8)) * 8) =
                make_uint4(0, 0, 0, 0);
        return;
    }

    int kend = Lk;
    if (causal) kend = min(kend, min(q0 + DQ_BQ, Lq));
    const int ntiles = (kend + DQ_BK - 1) / DQ_BK;
    int wtiles = (qw0 >= Lq) ? 0 : ntiles;
    if (causal) wtiles = min(wtiles, (qw0 + DQ_QW - 1) / DQ_BK + 1);
    int wmask = wtiles;                          // first tile that needs a mask
    if (causal) wmask = min(wmask, qw0 / DQ_BK);
    if (Lk % DQ_BK) wmask = min(wmask, Lk / DQ_BK);

    // Q and dO fragments (B operands): lane (g, c) holds row qw0 + 32 qb + c,
    // dims (HD / 2) g + 8 ks + 0..7; rows at or past Lq are zero.
    // The row's D = dO . O and lse2 = lse log2 e are formed here from the
    // same fragments of dO and O (lanes c and c + 32 hold the two halves of
    // the row) and stored for attn_bwd_dkdv, which runs after this kernel.
    // A row that sees no key (lse = -inf) gets (lse2, D) = (+inf, 0): its
    // rebuilt weights are exactly 0.
    bf16x8 qf[DQ_NQB][KS], df[DQ_NQB][KS];
    uint4 wx[DQ_NQB][KS];
    float lse[DQ_NQB], l2[DQ_NQB], dd[DQ_NQB];
#pragma unroll
    for (int qb = 0; qb < DQ_NQB; ++qb) {
        const int qi = qw0 + 32 * qb + c;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            uint4 wq = make_uint4(0, 0, 0, 0), wo = make_uint4(0, 0, 0, 0);
            wx[qb][ks] = make_uint4(0, 0, 0, 0);
            if (qi < Lq) {
                wq = *reinterpret_cast<const uint4 *>(Q + (qrow0 + qi) * HD + (HD / 2) * g + 8 * ks);
                wo = *reinterpret_cast<const uint4 *>(dO + (qrow0 + qi) * HD + (HD / 2) * g + 8 * ks);
                wx[qb][ks] = *reinterpret_cast<const uint4 *>(O + (qrow0 + qi) * HD + (HD / 2) * g + 8 * ks);
            }
            qf[qb][ks] = __builtin_bit_cast(bf16x8, wq);
            df[qb][ks] = __builtin_bit_cast(bf16x8, wo);
        }
        lse[qb] = (qi < Lq) ? LSE[qrow0 + qi] : kNegInf;
    }
    f32x16 dqa[DQ_NQB][NDT];
#pragma unroll
    for (int qb = 0; qb < DQ_NQB; ++qb)
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
            for (int i = 0; i < 16; ++i) dqa[qb][dt][i] = 0.0f;

    // tile DMA: this wave fills LDS block dblk (rows RPB dblk .. + RPB - 1) of
    // a K slot and a V slot (head dim 128), or of one of them (head dim 64);
    // lane l row RPB dblk + l/CH, slot l%CH.  Rows at or past Lk read as zeros.
    const int dblk = wave % NBLK;
    const int drow = RPB * dblk + (lane >> G::kLogCH);
    const uint32_t dmo = drow * ROWB + (((lane & (CH - 1)) ^ swzh<HD>(drow)) << 4);
    auto issue = [&](uint8_t *kd, uint8_t *vd, int t) __attribute__((always_inline)) {
        const int j0 = t * DQ_BK;
        const int bytes = max(0, Lk - j0) * ROWB;
        const __amdgpu_buffer_rsrc_t rk = rsrc(Kh + (size_t)j0 * HD, bytes);
        const __amdgpu_buffer_rsrc_t rv = rsrc(Vh + (size_t)j0 * HD, bytes);
        if constexpr (LPT == 2) {
            dma16(rk, kd + dblk * 1024, dmo);
            dma16(rv, vd + dblk * 1024, dmo);
        } else {
            if (wave < NBLK) dma16(rk, kd + dblk * 1024, dmo);
            else dma16(rv, vd + dblk * 1024, dmo);
        }
    };

    // row-wise A operand (rows of K or V): lane (g, c) reads row c, chunk (CH / 2) g + ks
    uint32_t aoff[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) aoff[ks] = c * ROWB + (((((CH / 2) * g) + ks) ^ swzh<HD>(c)) << 4);
    // transposed A operand K^T (dim rows 32 dt + c): as in attn_bwd_dkdv
    uint32_t tlo[NDT], thi[NDT];
    {
        const int t = lane >> 4, i = lane & 15;
        const int row = 4 * (t >> 1) + (i >> 2);
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
            const int chunk = 4 * dt + 2 * (t & 1) + ((i & 3) >> 1);
            tlo[dt] = row * ROWB + ((chunk ^ swzh<HD>(row)) << 4) + (i & 1) * 8;
            thi[dt] = (row + 8) * ROWB + ((chunk ^ swzh<HD>(row + 8)) << 4) + (i & 1) * 8;
        }
    }

    // key 32 t + 8 r + 4 g + u is visible to query qi iff it is
    // <= min(Lk - 1, qi) (causal) or <= Lk - 1
    auto mask = [&](f32x16 (&s)[DQ_NQB], int t) __attribute__((always_inline)) {
#pragma unroll
        for (int qb = 0; qb < DQ_NQB; ++qb) {
            const int qi = qw0 + 32 * qb + c;
            const int lim = (causal ? min(Lk - 1, qi) : Lk - 1) - t * DQ_BK - 4 * g;
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int u = 0; u < 4; ++u)
                    if (8 * r + u > lim) s[qb][4 * r + u] = kNegInf;
        }
    };

    auto compute = [&](const uint8_t *kb, const uint8_t *vb, int t, bool masked) __attribute__((always_inline)) {
        const f32x16 zero = {};
        f32x16 s[DQ_NQB], dp[DQ_NQB];
        // K and V operands read DQ_RA k-steps ahead of their MFMAs (at head
        // dim 64 one: a deeper read-ahead takes the kernel past 128 VGPRs, and
        // with it two workgroups per CU)
        constexpr int DQ_RA = HD == 128 ? 3 : 1;
        bf16x8 ak[KS], av[KS];
#pragma unroll
        for (int ks = 0; ks < DQ_RA; ++ks) {
            ak[ks] = *reinterpret_cast<const bf16x8 *>(kb + aoff[ks]);
            av[ks] = *reinterpret_cast<const bf16x8 *>(vb + aoff[ks]);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            if (ks + DQ_RA < KS) {
                ak[ks + DQ_RA] = *reinterpret_cast<const bf16x8 *>(kb + aoff[ks + DQ_RA]);
                av[ks + DQ_RA] = *reinterpret_cast<const bf16x8 *>(vb + aoff[ks + DQ_RA]);
            }
#pragma unroll
            for (int qb = 0; qb < DQ_NQB; ++qb) {
                s[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ak[ks], qf[qb][ks], ks ? s[qb] : zero, 0, 0, 0);
                dp[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[ks], df[qb][ks], ks ? dp[qb] : zero, 0, 0, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        if (masked) mask(s, t);
        // dS^T = P^T (dP^T - D), P^T = exp2(S^T scale log2e - lse2): one query per lane
        bf16x8 db[DQ_NQB][2];
#pragma unroll
        for (int qb = 0; qb < DQ_NQB; ++qb) {
            float e[16];
#pragma unroll
            for (int i = 0; i < 16; ++i)
                e[i] = fast_exp2(fmaf(s[qb][i], scale_log2, -l2[qb])) * (dp[qb][i] - dd[qb]);
            db[qb][0] = to_bf16x8(e);
            db[qb][1] = to_bf16x8(e + 8);
        }
        // dQ^T += K^T dS^T: k-step hh covers keys 16 hh + 4 g + 0..3 and + 8
#pragma unroll
        for (int hh = 0; hh < 2; ++hh)
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) {
                const bf16x8 a = cat4(lds_read_tr(kb + 16 * hh * ROWB + tlo[dt]),
                                      lds_read_tr(kb + 16 * hh * ROWB + thi[dt]));
#pragma unroll
                for (int qb = 0; qb < DQ_NQB; ++qb)
                    dqa[qb][dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, db[qb][hh], dqa[qb][dt], 0, 0, 0);
            }
    };

    auto kslot = [&](auto S) __attribute__((always_inline)) -> uint8_t * {
        constexpr int s = decltype(S)::value % 3;
        return s == 0 ? k0 : s == 1 ? k1 : k2;
    };
    auto vslot = [&](auto S) __attribute__((always_inline)) -> uint8_t * {
        constexpr int s = decltype(S)::value % 3;
        return s == 0 ? v0 : s == 1 ? v1 : v2;
    };
    // iteration j (slot j % 3): this wave's loads of tile j are done (those
    // of tile j + 1 may be in flight), the barrier makes every wave's visible
    // and frees slot (j + 2) % 3, which receives tile j + 2.  Every iteration
    // issues the same LPT loads per wave (tiles past the end are zero fills),
    // so the wait count is the same everywhere.
    auto iter = [&](auto S, int j) __attribute__((always_inline)) {
        __builtin_amdgcn_s_waitcnt(kWaitTile);
        tile_barrier();
        issue(kslot(Slot<decltype(S)::value + 2>{}), vslot(Slot<decltype(S)::value + 2>{}), j + 2);
        if (j < wtiles) compute(kslot(S), vslot(S), j, j >= wmask);
    };

    issue(k0, v0, 0);
    issue(k1, v1, 1);
    // (lse2, D) of this wave's rows, under the first tiles' loads
#pragma unroll
    for (int qb = 0; qb < DQ_NQB; ++qb) {
        const int qi = qw0 + 32 * qb + c;
        float acc = 0.0f;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const uint4 o = wx[qb][ks];
            const uint4 d = __builtin_bit_cast(uint4, df[qb][ks]);
            acc = fmaf(bf16_lo(o.x), bf16_lo(d.x), acc);
            acc = fmaf(bf16_hi(o.x), bf16_hi(d.x), acc);
            acc = fmaf(bf16_lo(o.y), bf16_lo(d.y), acc);
            acc = fmaf(bf16_hi(o.y), bf16_hi(d.y), acc);
            acc = fmaf(bf16_lo(o.z), bf16_lo(d.z), acc);
            acc = fmaf(bf16_hi(o.z), bf16_hi(d.z), acc);
            acc = fmaf(bf16_lo(o.w), bf16_lo(d.w), acc);
            acc = fmaf(bf16_hi(o.w), bf16_hi(d.w), acc);
        }
        acc += __shfl_xor(acc, 32, 64);
        const bool live = lse[qb] != kNegInf;
        l2[qb] = live ? lse[qb] * kLog2e : kPosInf;
        dd[qb] = live ? acc : 0.0f;
        if (g == 0 && qi < Lq) LD[qrow0 + qi] = make_float2(l2[qb], dd[qb]);
    }
    const int nend = ((ntiles + 2) / 3) * 3;
    for (int j = 0; j < nend; j += 3) {
        iter(Slot<0>{}, j);
        iter(Slot<1>{}, j + 1);
        iter(Slot<2>{}, j + 2);
    }
    __builtin_amdgcn_s_waitcnt(kWaitVm0);       // no load outlives the kernel

    // ---- epilogue: dQ = scale dQ~; rows past Lq get zeros ------------------
#pragma unroll
    for (int qb = 0; qb < DQ_NQB; ++qb) {
        const int qi = qw0 + 32 * qb + c;
        if (qi < Nq) {
            const bool valid = qi < Lq;
            uint16_t *row = dQ + (qrow0 + qi) * HD;
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    uint2 w;
                    w.x = valid ? pack_bf16x2_hw(dqa[qb][dt][4 * r] * scale, dqa[qb][dt][4 * r + 1] * scale) : 0u;
                    w.y = valid ? pack_bf16x2_hw(dqa[qb][dt][4 * r + 2] * scale, dqa[qb][dt][4 * r + 3] * scale) : 0u;
                    *reinterpret_cast<uint2 *>(row + 32 * dt + 8 * r + 4 * g) = w;
                }
        }
    }
}

}  // namespace

namespace {

template <int HD>
hipError_t launch_bwd(const AttnBwdArgs &a, hipStream_t s) {
    const int64_t rows = (int64_t)a.batch * a.heads_q * a.seqlen_q;
    float2 *ld = static_cast<float2 *>(a.workspace);
    const uint16_t *q = static_cast<const uint16_t *>(a.q), *k = static_cast<const uint16_t *>(a.k);
    const uint16_t *v = static_cast<const uint16_t *>(a.v), *o = static_cast<const uint16_t *>(a.o);
    const uint16_t *dout = static_cast<const uint16_t *>(a.dout);
    const float scale_log2 = a.scale * kLog2e;
    // attn_bwd_dq first: it stores the (lse2, D) rows that attn_bwd_dkdv reads
    if (rows > 0) {
        const int nqb = (a.seqlen_q + DQ_BQ - 1) / DQ_BQ;
        const int nheads = a.batch * a.heads_q;
        const int xcd_heads = (nheads % 8 == 0) ? 1 : 0;
        hipLaunchKernelGGL(attn_bwd_dq<HD>, dim3((unsigned)((int64_t)nqb * nheads)), dim3(DQ_NT), 0, s, q, k, v,
                           o, dout, a.lse, ld, static_cast<uint16_t *>(a.dq), a.heads_q, a.heads_kv, a.seqlen_q,
                           a.seqlen_k, a.seqlens_q, a.seqlens_k, scale_log2, a.scale, a.causal, nqb, xcd_heads);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (a.seqlen_k > 0) {
        const int nkb = (a.seqlen_k + KV_BK - 1) / KV_BK;
        const int nheads = a.batch * a.heads_kv;
        const int xcd_heads = (nheads % 8 == 0) ? 1 : 0;
        const dim3 grid((unsigned)((int64_t)nkb * nheads));
        if (a.causal)
            hipLaunchKernelGGL((attn_bwd_dkdv<true, HD>), grid, dim3(KV_NT), 0, s, q, k, v, dout, ld,
                               static_cast<uint16_t *>(a.dk), static_cast<uint16_t *>(a.dv), a.heads_q,
                               a.heads_kv, a.seqlen_q, a.seqlen_k, a.seqlens_q, a.seqlens_k, scale_log2,
                               a.scale, nkb, xcd_heads);
        else
            hipLaunchKernelGGL((attn_bwd_dkdv<false, HD>), grid, dim3(KV_NT), 0, s, q, k, v, dout, ld,
                               static_cast<uint16_t *>(a.dk), static_cast<uint16_t *>(a.dv), a.heads_q,
                               a.heads_kv, a.seqlen_q, a.seqlen_k, a.seqlens_q, a.seqlens_k, scale_log2,
                               a.scale, nkb, xcd_heads);
        return hipGetLastError();
    }
    return hipSuccess;
}

}  // namespace

hipError_t launch_attn_bwd(const AttnBwdArgs &a, hipStream_t s) {
    return a.head_dim == 128 ? launch_bwd<128>(a, s) : launch_bwd<64>(a, s);
}

}  // namespace osm
