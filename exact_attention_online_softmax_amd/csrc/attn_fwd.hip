// attn_fwd.hip -- fused exact attention forward for gfx950 (bf16, head_dim 128 and 64).
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
//  * workgroup = 4 wavefronts = 256 queries, one wavefront per SIMD and one
//    workgroup per CU; each wave owns 64 queries as two 32-query blocks, so
//    every K or V operand read from LDS feeds two MFMAs (half the LDS traffic
//    per flop of a 32-query wave).  With one wave per SIMD each wave has 512
//    registers: the output accumulators live in the AGPRs.
//  * head dim 64 instantiates the same body (a template over the head dim)
//    with 16 MFMA steps per tile instead of 32.  A wave then fits in 256
//    registers (the Q fragments in AGPRs, which the score MFMA reads
//    directly), so two workgroups run per CU and one wave's exponentials
//    overlap the other's matrix products: per flop, the vector work is twice
//    that of head dim 128.  It runs one query block per workgroup.
//  * both products run on v_mfma_f32_32x32x16_bf16 with fp32 accumulation.
//    The score tile is computed transposed, S^T = K Q^T, so lane l holds the
//    scores of one query (l % 32) of each block against 16 of the 32 keys of
//    the tile; lane l ^ 32 holds the other 16.  Row max and row sum are
//    in-lane plus one cross-half exchange.
//  * the output is accumulated transposed, O~^T = V^T P~^T: P~^T is the fp32
//    score accumulator converted in place to bf16, and the rescale by
//    exp2(m_old - m_new) is a per-lane multiply.
//  * software pipeline inside each wave: iteration j exponentiates the
//    scores of tile j and multiplies them into O~ while the matrix cores
//    already compute the scores of tile j+1; the vector ALU work of one tile
//    and the MFMAs of the next interleave in one instruction stream.
//  * K and V tiles (32 keys x head dim: 8 KiB each at 128, 4 KiB at 64) go
//    from HBM straight into LDS with buffer_load_dwordx4 ... lds (no VGPR
//    staging; lane i of a load writes bytes 16 i .. 16 i + 15 of a 1 KiB LDS
//    block) through a ring of
//    four slots, loaded three tiles ahead.  Each slot is its own LDS object
//    and the loop is unrolled by four, so every access names its slot
//    statically: operand reads use immediate offsets, and the compiler can
//    tell that the loads in flight never alias the slots being read.
//  * rows are unpadded and XOR-swizzled at 16-byte granularity (256-byte
//    rows: K slot = chunk ^ (row % 16), V slot = chunk ^ 4 (row % 4); 128-byte
//    rows: K slot = chunk ^ ((row / 2) % 8), V slot = chunk ^ 4 ((row / 2) % 2))
//    so that the K operand reads and the transposing V reads are free of bank
//    conflicts.
//  * the V^T operand is read with the gfx950 transposing LDS read
//    (ds_read_b64_tr_b16): in each 16-lane group, lane i points at
//    V[k0 + i/4][d0 + 4 (i%4) .. +3] and lane j receives V[k0 + e][d0 + j],
//    e = 0..3 -- four consecutive keys of one dim, the operand layout.
//  * rows at or past the valid length are never read from memory: each
//    tile's loads go through a buffer resource that ends at the valid
//    length, and its range check fills those rows of LDS with zeros, so LDS
//    only ever holds finite data and NaN padding cannot reach an MFMA
//    (0 * NaN = NaN); their scores are masked to -inf, so they add exactly
//    zero.
//  * the reference is only raised (and O~, l rescaled) when a score exceeds
//    it by more than 8 in base-2 units, so every weight stays at most 2^8 and
//    the reference may sit up to that far below the running maximum.  The
//    result does not depend on the reference: a common factor cancels
//    between O~ and l ([P3] "Merging partial results": summaries relative to
//    any common reference combine exactly), and l <= 2^8 N_k keeps clear of
//    fp32 overflow.  After the first tiles the rescale is skipped by a
//    wave-uniform branch.
//  * tiles that need a mask (the causal diagonal, the ragged end) are the
//    last ones each wave visits; they run in a separate, branchy loop so the
//    main loop carries no mask code.
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
typedef short s16x4 __attribute__((ext_vector_type(4)));

constexpr int NW = 4;             // wavefronts per workgroup (one per SIMD)
constexpr int QW = 64;            // queries per wavefront (two 32-query blocks)
constexpr int BQ = QW * NW;       // queries per workgroup
constexpr int BK = 32;            // keys per tile
constexpr int NT = 64 * NW;       // threads per workgroup
constexpr int AHEAD = 3;          // tiles loaded ahead of the one being computed

// Sizes that follow from the head dim (128 or 64).
template <int HD> struct Geo {
    static constexpr int ROWB = HD * 2;             // bytes per K/V/Q row in LDS (unpadded)
    static constexpr int CH = ROWB / 16;            // 16-byte chunks per row
    static constexpr int RPB = 1024 / ROWB;         // rows per 1 KiB block of an LDS-DMA load
    static constexpr int TILEB = BK * ROWB;         // bytes per K or V tile (8 or 4 KiB)
    static constexpr int LPW = TILEB / 1024 / NW;   // 1 KiB loads per wave per K (or V) tile
    static constexpr int KS = HD / 16;              // k-steps of the score product
    static constexpr int NDT = HD / 32;             // 32-dim blocks of the output
    static constexpr int QL = QW * ROWB / 1024;     // 1 KiB loads per wave copying a block's Q
    static constexpr int STEPS = 2 * KS + 4 * NDT;  // MFMA steps of the tile body
};

// LDS swizzles at 16-byte granularity (chunk c of row r sits in slot
// c ^ sw(r)).  K and Q rows: the row-wise operand reads (16 lanes of a
// ds_read_b128, 16 rows, one chunk) hit 16 distinct 16-byte units of a
// 256-byte bank window: at 256-byte rows sw = r % 16; at 128-byte rows two
// rows share a window, so the eight rows of each parity need distinct slots,
// sw = (r / 2) % 8.  V rows: a transposing read (32 lanes, rows 4a .. 4a+3,
// four adjacent chunks, 8 bytes each) hits 32 distinct 8-byte units: at
// 256-byte rows sw = 4 (r % 4); at 128-byte rows rows r and r + 2 share a
// window half, sw = 4 ((r / 2) % 2).
template <int HD> __device__ __forceinline__ int swk(int r) { return HD == 128 ? (r & 15) : ((r >> 1) & 7); }
template <int HD> __device__ __forceinline__ int swv(int r) { return HD == 128 ? ((r & 3) << 2) : (((r >> 1) & 1) << 2); }

template <int N> struct Slot { static constexpr int value = N; };

// f(Slot<I>{}) for I = B .. E-1, each with its index as a compile-time constant
template <int B, int E, typename F> __device__ __forceinline__ void static_for(F &&f) {
    if constexpr (B < E) {
        f(Slot<B>{});
        static_for<B + 1, E>(f);
    }
}

// The 32 exponential items of a tile (n = 0..31: query block (n/8) % 2,
// element (n%8) + 8 (n/16) of that block's scores) in the order the P~V
// steps consume them, in groups g = -1 .. kGroups-1: items
// [item_lo(g), item_lo(g+1)), four in the first group, then one or two.
// (22 groups over the 32 steps of the head-dim-128 body, 9 over the 16
// steps of the head-dim-64 body: each P~ operand is converted at least one
// full step before its first P~V step)
template <int HD> constexpr int k_groups() { return HD == 128 ? 22 : 9; }
template <int HD> constexpr int item_lo(int g) { return g < 0 ? 0 : 4 + (g * 28) / k_groups<HD>(); }
constexpr int item_qb(int n) { return (n >> 3) & 1; }
constexpr int item_i(int n) { return (n & 7) + 8 * (n >> 4); }

// O~^T accumulation MFMA with its accumulator pinned to AGPRs.  Written as
// inline assembly because the compiler picks one register form for every
// MFMA of a kernel, and the score MFMAs must write VGPRs (the softmax reads
// them) while the 128 output registers per lane only fit in the AGPRs.  The
// hazard recognizer does not look inside inline assembly: an MFMA needs two
// wait states after a VALU instruction writes one of its operands.  In the
// tile body no VALU instruction writes them near the MFMA: the V^T operand
// comes straight from LDS reads, and each P~ operand is converted at least
// one full MFMA step (an MFMA and its vector work) before its first use, so
// the wait states are there without a nop.  Back-to-back accumulation into
// the same registers needs none.
__device__ __forceinline__ void mfma_acc(f32x16 &acc, const bf16x8 &a, const bf16x8 &b) {
    asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}

__device__ __forceinline__ void acc_zero(f32x16 &acc, const bf16x8 &z) {
    asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %1, 0" : "=a"(acc) : "v"(z));
}

// Before ordinary code reads accumulators written by mfma_acc: wait out the
// MFMA result latency (the compiler model asks for 12 wait states; 24 here).
template <int NDT> __device__ __forceinline__ void acc_settle(f32x16 (&o)[2][NDT]) {
    if constexpr (NDT == 4)
        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"
                     : "+a"(o[0][0]), "+a"(o[0][1]), "+a"(o[0][2]), "+a"(o[0][3]),
                       "+a"(o[1][0]), "+a"(o[1][1]), "+a"(o[1][2]), "+a"(o[1][3]));
    else
        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"
                     : "+a"(o[0][0]), "+a"(o[0][1]), "+a"(o[1][0]), "+a"(o[1][1]));
}

// transposing LDS read: see the header comment for the lane layout
__device__ __forceinline__ bf16x4 lds_read_tr(const uint8_t *p) {
    const s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (s16x4 __attribute__((address_space(3))) *)(p));
    return __builtin_bit_cast(bf16x4, r);
}

__device__ __forceinline__ int clampi(int v, int lo, int hi) { return v < lo ? lo : (v > hi ? hi : v); }

// a wave-uniform pointer, moved to scalar registers
__device__ __forceinline__ const uint16_t *uniform_ptr(const uint16_t *p) {
    const uint64_t u = reinterpret_cast<uint64_t>(p);
    const uint64_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)u);
    const uint64_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(u >> 32));
    return reinterpret_cast<const uint16_t *>((hi << 32) | lo);
}

// Workgroup barrier without a memory fence; the empty asm statements keep
// the compiler from moving LDS accesses across it.  Callers wait for their
// own outstanding memory operations first.
__device__ __forceinline__ void tile_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Buffer resource word 3 for raw (unformatted, unswizzled) dword access:
// DATA_FORMAT = 32 bits, everything else zero.
constexpr int kRsrcWord3 = 0x00020000;

// s_waitcnt encodings (gfx9): vmcnt in bits 3:0 and 15:14, expcnt 6:4,
// lgkmcnt 11:8; a field at its maximum does not wait.
constexpr int vmcnt_wait(int n) { return 0x0F70 | (n & 15) | ((n >> 4) << 14); }
constexpr int kWaitVm0 = vmcnt_wait(0);
constexpr int kWaitLgkm0 = 0xC07F; // lgkmcnt(0)
static_assert(vmcnt_wait(4) == 0x0F74 && vmcnt_wait(20) == 0x4F74, "vmcnt encoding");

// (batch, head, KV head, first query, valid query and key lengths) of a
// query block
struct Blk {
    int b, h, kvh, q0, Lq, Lk;
};

// Persistent grid with a static schedule (causal or varlen inputs): the
// schedule of one XCD's blocks is a list in LDS of entries (t << 16) | i, head
// 8 t + XCD and query block i, at most kSchedMax of them.
constexpr int kSchedMax = 2048;
constexpr int kSchedFixed = 10;     // per-block cost outside the tile loop, in tiles (measured)

// MODE 0: one query block per workgroup.
// MODE 1 and 2 (PERSIST, head dim 128): one workgroup per CU walks several
// blocks.  The Q of the next block is copied into LDS (qs) while the
// current block runs, and the last ring loads of a block fetch the first
// tiles of the next one, so a block starts with its Q and first tiles on
// chip, and no CU waits for a new workgroup to be dispatched between blocks.
//  * MODE 1: full-length non-causal inputs, where every block has the same
//    work: workgroup L takes blocks L, L + gridDim.x, ...
//  * MODE 2: causal or varlen inputs.  Every workgroup first builds its list
//    of blocks from the lengths: the XCD's heads in decreasing order of
//    their largest block; a head's blocks, heaviest first, go to the
//    least-loaded slots of the XCD (longest-processing-time-first list
//    scheduling, with costs in tiles plus a fixed cost per block), so the
//    XCD's workgroups run one or two heads at a time and share their K and V
//    in L2.  Blocks with no visible key or no valid query only write O = 0,
//    LSE = -inf; they come last, round robin over the slots.
template <int MODE, int HD>
__device__ __forceinline__ void
attn_fwd_body(const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K,
              const uint16_t *__restrict__ V, uint16_t *__restrict__ O,
              float *__restrict__ LSE, int B, int Hq, int Hkv, int Nq, int Nk,
              const int32_t *__restrict__ seqlens_q, const int32_t *__restrict__ seqlens_k,
              float scale_log2, int causal_arg, int nqb, int xcd_heads, int nblocks) {
    using G = Geo<HD>;
    constexpr int D = HD, ROWB = G::ROWB, CH = G::CH, RPB = G::RPB, TILEB = G::TILEB, LPW = G::LPW;
    constexpr int KS = G::KS, NDT = G::NDT, QL = G::QL, STEPS = G::STEPS, kGroups = k_groups<HD>();
    constexpr int kLogCH = CH == 16 ? 4 : 3;
    // tiles of this wave in flight at the top of an iteration: one; with the
    // copy of the next block's Q behind them (iterations 0 and 1), also that
    constexpr int kWaitVmTile = vmcnt_wait(2 * LPW);
    constexpr int kWaitVmQ = vmcnt_wait(2 * LPW + QL);
    // ring of four K slots and four V slots (8 KiB each at head dim 128)
    __shared__ __attribute__((aligned(1024))) uint8_t k0[TILEB], k1[TILEB], k2[TILEB], k3[TILEB];
    __shared__ __attribute__((aligned(1024))) uint8_t v0[TILEB], v1[TILEB], v2[TILEB], v3[TILEB];
    // Q of the block (PERSIST), rows swizzled like K
    // (less aligned than the slots, so that it is laid out after them and the
    // slots stay within reach of the 16-bit immediate offset of LDS reads)
    constexpr bool PERSIST = MODE != 0;
    constexpr bool SCHED = MODE == 2;
    __shared__ __attribute__((aligned(256))) uint8_t qs[PERSIST ? BQ * ROWB : 256];
    // the workgroup's block list (SCHED): entries, then (compute items, items)
    __shared__ int sched[SCHED ? kSchedMax : 1];
    __shared__ int sched_n[2];
    const int causal = MODE == 1 ? 0 : causal_arg;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 5, c = lane & 31;

    // ---- which (batch, head, query block) ------------------------------
    auto decode = [&](int L) __attribute__((always_inline)) -> Blk {
        int head, qrev;
        if (xcd_heads) {
            // hardware places block L on XCD L % 8 (a persistent grid is a
            // multiple of 8, so block L still runs on XCD L % 8); give every
            // XCD whole heads (head % 8 == XCD) and run one head's query
            // blocks back to back (heaviest first), so the blocks resident
            // on an XCD share a few heads' K and V in its L2.
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
        const int qb0 = causal ? (nqb - 1 - qrev) : qrev;
        const int b = head / Hq, h = head % Hq;
        return {b, h, h / (Hq / Hkv), qb0 * BQ, 0, 0};   // lengths: read in the block loop
    };
    // block of a schedule entry (SCHED)
    auto item_blk = [&](int e) __attribute__((always_inline)) -> Blk {
        e = __builtin_amdgcn_readfirstlane(e);
        const int head = 8 * (e >> 16) + (int)(blockIdx.x & 7);
        // the integer divisions run on the vector ALU; the results are uniform,
        // so move them back to scalar registers (a buffer resource built from
        // a vector register makes every load a loop over lanes)
        const int b = __builtin_amdgcn_readfirstlane(head / Hq), h = __builtin_amdgcn_readfirstlane(head % Hq);
        const int kvh = __builtin_amdgcn_readfirstlane(h / (Hq / Hkv));
        const int lq = __builtin_amdgcn_readfirstlane(seqlens_q ? clampi(seqlens_q[b], 0, Nq) : Nq);
        const int lk = __builtin_amdgcn_readfirstlane(seqlens_k ? clampi(seqlens_k[b], 0, Nk) : Nk);
        return {b, h, kvh, (e & 0xffff) * BQ, lq, lk};
    };
    // every row of a block that sees no key is written O = 0, LSE = -inf
    auto zero_fill = [&](const Blk &z) __attribute__((always_inline)) {
        const size_t zhead = (size_t)(z.b * Hq + z.h) * Nq;
        const int rows = min(BQ, Nq - z.q0);
        for (int i = tid; i < rows * (D / 8); i += NT) {
            const int r = i / (D / 8), d8 = i % (D / 8);
            *reinterpret_cast<uint4 *>(O + (zhead + z.q0 + r) * D + d8 * 8) = make_uint4(0, 0, 0, 0);
        }
        if (LSE)
            for (int r = tid; r < rows; r += NT) LSE[zhead + z.q0 + r] = kNegInf;
    };

    // ---- the static schedule (SCHED), built by wave 0 -------------------------
    int n_compute = 0, n_items = 0;
    if constexpr (SCHED) {
        if (wave == 0) {
            const int xcd = blockIdx.x & 7, myslot = blockIdx.x >> 3, nslots = gridDim.x >> 3;
            const int nh = xcd_heads;
            // tiles of query block i of a head with lengths (lq, lk)
            auto tiles_of = [&](int i, int lq, int lk) __attribute__((always_inline)) -> int {
                const int kend = causal ? min(lk, min((i + 1) * BQ, lq)) : lk;
                return (kend + BK - 1) / BK;
            };
            // lane t < nh: head 8 t + xcd, its lengths and its number of blocks
            // with work (none when it has no key)
            int hlq = 0, hlk = 0, hnb = 0, hcost = -1;
            if (lane < nh) {
                const int bb = (8 * lane + xcd) / Hq;
                hlq = seqlens_q ? clampi(seqlens_q[bb], 0, Nq) : Nq;
                hlk = seqlens_k ? clampi(seqlens_k[bb], 0, Nk) : Nk;
                hnb = hlk > 0 ? (hlq + BQ - 1) / BQ : 0;
                hcost = hnb > 0 ? tiles_of(hnb - 1, hlq, hlk) : 0;
            }
            // rank of each head: decreasing cost of its largest block, ties by t
            int hrank = 0;
            for (int j = 0; j < nh; ++j) {
                const int cj = __builtin_amdgcn_readlane(hcost, j);
                hrank += (cj > hcost || (cj == hcost && j < lane)) ? 1 : 0;
            }
            int load = 0;   // lane s < nslots: tiles given to slot s so far
            int n = 0;      // entries of this workgroup's list
            for (int r = 0; r < nh; ++r) {
                const int t = (int)__builtin_ctzll(__builtin_amdgcn_ballot_w64(lane < nh && hrank == r));
                const int nb = __builtin_amdgcn_readlane(hnb, t);
                const int lq = __builtin_amdgcn_readlane(hlq, t), lk = __builtin_amdgcn_readlane(hlk, t);
                // the head's blocks, heaviest first (causal: the last), in rounds
                // of nslots: the least-loaded slot (ties by slot) takes the
                // heaviest block of the round, the next one the next, ...
                for (int i0 = 0; i0 < nb; i0 += nslots) {
                    const int take = min(nslots, nb - i0);
                    const int key = lane < nslots ? load * 64 + lane : 0x7fffffff;
                    int rk = 0;
                    for (int j = 0; j < nslots; ++j) rk += (__builtin_amdgcn_readlane(key, j) < key) ? 1 : 0;
                    if (lane < nslots && rk < take) load += tiles_of(nb - 1 - (i0 + rk), lq, lk) + kSchedFixed;
                    const int mrk = __builtin_amdgcn_readlane(rk, myslot);
                    if (mrk < take) {
                        if (lane == 0) sched[n] = (t << 16) | (nb - 1 - (i0 + mrk));
                        ++n;
                    }
                }
            }
            const int ncomp = n;
            // blocks without work, numbered over the heads in rank order; the
            // slot of block number j is j % nslots
            int pj = 0;
            for (int r = 0; r < nh; ++r) {
                const int t = (int)__builtin_ctzll(__builtin_amdgcn_ballot_w64(lane < nh && hrank == r));
                const int nb = __builtin_amdgcn_readlane(hnb, t);
                const int np = nqb - nb;
                for (int i = nb + ((myslot - pj) % nslots + nslots) % nslots; i < nqb; i += nslots) {
                    if (lane == 0) sched[n] = (t << 16) | i;
                    ++n;
                }
                pj += np;
            }
            if (lane == 0) {
                sched_n[0] = ncomp;
                sched_n[1] = n;
            }
        }
        __syncthreads();
        n_compute = __builtin_amdgcn_readfirstlane(sched_n[0]);
        n_items = __builtin_amdgcn_readfirstlane(sched_n[1]);
    }

    int L = blockIdx.x;
    int item = 0;
    bool first = true;
    for (;;) {
        if (SCHED && item >= n_compute) break;
        const Blk cur = SCHED ? item_blk(sched[item]) : decode(L);
        const int Lnext = L + (int)gridDim.x;
        const bool has_next = SCHED ? (item + 1 < n_compute)
                                    : (PERSIST && __builtin_amdgcn_readfirstlane(Lnext < nblocks ? 1 : 0) != 0);
        const Blk nxt = SCHED ? (has_next ? item_blk(sched[item + 1]) : cur) : decode(has_next ? Lnext : L);
        const int b = cur.b, h = cur.h, kvh = cur.kvh, q0 = cur.q0;
        // lengths and the wave index are uniform: keep them in scalar registers
        // so that every tile-level decision is a scalar branch
        const int Lq = SCHED ? cur.Lq : __builtin_amdgcn_readfirstlane(seqlens_q ? clampi(seqlens_q[b], 0, Nq) : Nq);
        const int Lk = SCHED ? cur.Lk : __builtin_amdgcn_readfirstlane(seqlens_k ? clampi(seqlens_k[b], 0, Nk) : Nk);

        const int qw0 = q0 + QW * wave;         // first query of this wave
        // this lane's queries: qw0 + c (block 0) and qw0 + 32 + c (block 1)

        const size_t qhead = (size_t)(b * Hq + h) * Nq;
        const uint16_t *Kh = K + (size_t)(b * Hkv + kvh) * Nk * D;
        const uint16_t *Vh = V + (size_t)(b * Hkv + kvh) * Nk * D;

        if (!PERSIST && q0 >= Lq) {
            // every row of this block is padding: O = 0, LSE = -inf
            zero_fill(cur);
            return;
        }

        // keys that can be visible to some query of this block
        int kend = Lk;
        if (causal) kend = min(kend, min(q0 + BQ, Lq));
        const int ntiles = (kend + BK - 1) / BK;
        // tiles this wave computes: none if all its queries are padding; with a
        // causal mask only tiles starting at or below its last query
        int wtiles = (qw0 >= Lq) ? 0 : ntiles;
        if (causal) wtiles = min(wtiles, (qw0 + QW - 1) / BK + 1);
        // first tile that needs a mask: the causal diagonal starts at the tile
        // holding key qw0, the ragged end at the tile holding key Lk - 1
        int wfirst_mask = wtiles;
        if (causal) wfirst_mask = min(wfirst_mask, qw0 / BK);
        if (Lk % BK) wfirst_mask = min(wfirst_mask, Lk / BK);
        // iterations j whose next tile j + 1 is computed without a mask
        const int nfast = max(0, wfirst_mask - 1);
        // the loops run in whole groups of four iterations (see below)
        const int wend = (wtiles + 3) & ~3, nend = (ntiles + 3) & ~3;

        // O~^T accumulators, zeroed in the AGPRs by an MFMA of zeros (so they
        // never pass through VGPRs)
        f32x16 oacc[2][NDT];
        {
            const bf16x8 z8 = {};
#pragma unroll
            for (int qb = 0; qb < 2; ++qb)
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt) acc_zero(oacc[qb][dt], z8);
        }
        f32x16 sacc[2];          // S^T of the tile whose softmax is next
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
#pragma unroll
            for (int i = 0; i < 16; ++i) sacc[qb][i] = kNegInf;
        constexpr float kLazy = 8.0f;                 // allowed growth, base-2 units
        const float lazy_raw = kLazy / scale_log2;    // the same in raw score units
        float m[2], mlim[2], msub[2], l[2];
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            m[qb] = kNegInf;     // reference maximum of raw scores q.k
            mlim[qb] = kNegInf;  // m + lazy_raw: tile maxima up to it keep the reference
            msub[qb] = 0.0f;     // m * scale * log2(e) (0 while m = -inf)
            l[qb] = 0.0f;        // this lane's half of the running sum
        }

        // ---- direct HBM -> LDS tile loads -----------------------------------
        // Load i of wave w fills LDS block 2 w + i (rows 4 (2 w + i) .. +3) of a
        // slot; lane l fills row 4 (2 w + i) + l/16, slot l%16, which holds global
        // 16-byte chunk (slot ^ swizzle(row)).  Offsets are in bytes within a tile.
        // The loads go through a buffer resource that starts at the tile and
        // spans its rows below Lk: the range check turns rows past Lk (and every
        // row of a tile at or past Lk) into zeros without touching memory, so
        // LDS only ever holds finite data, and a load needs no branch.  The
        // buffer (MUBUF) form of the LDS DMA is used because with the global
        // (FLAT) form in flight the compiler turns every LDS operand wait into a
        // wait for all LDS reads.
        uint32_t kld[LPW], vld[LPW];
#pragma unroll
        for (int i = 0; i < LPW; ++i) {
            const int blk = LPW * wave + i;
            const int row = RPB * blk + (lane >> kLogCH);
            const int s = lane & (CH - 1);
            kld[i] = row * ROWB + ((s ^ swk<HD>(row)) << 4);
            vld[i] = row * ROWB + ((s ^ swv<HD>(row)) << 4);
        }
        struct TileRsrc {
            __amdgpu_buffer_rsrc_t k, v;
        };
        auto rsrc_at = [&](const uint16_t *kb, const uint16_t *vb, int j0, int len)
            __attribute__((always_inline)) -> TileRsrc {
            const int bytes = max(0, len - j0) * ROWB;   // < 2^31: the ABI bounds Nk * 256
            return {__builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(kb) + (size_t)j0 * D, 0, bytes, kRsrcWord3),
                    __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(vb) + (size_t)j0 * D, 0, bytes, kRsrcWord3)};
        };
        // tile t of this block; the only kind the unmasked loop loads: it stops
        // at least two iterations short of the padded end, so t < nend there
        // (t may pass ntiles, where the range check loads zeros)
        auto tile_rsrc_cur = [&](int t) __attribute__((always_inline)) -> TileRsrc {
            return rsrc_at(Kh, Vh, t * BK, Lk);
        };
        // With PERSIST, tile nend + i (past this block's padded end, where the
        // ring would load zeros) is tile i of the next block, if there is one,
        // with the next block's key length.  The compiler
        // evaluates the uniform selects of that case on the vector ALU;
        // readfirstlane keeps the resource in scalar registers, without which
        // every load would become a loop over lanes.
        const uint16_t *Kn = K + (size_t)(nxt.b * Hkv + nxt.kvh) * Nk * D;
        const uint16_t *Vn = V + (size_t)(nxt.b * Hkv + nxt.kvh) * Nk * D;
        auto tile_rsrc = [&](int t) __attribute__((always_inline)) -> TileRsrc {
            if constexpr (!PERSIST) {
                return tile_rsrc_cur(t);
            } else {
                const bool next = t >= nend;
                const uint16_t *kb = uniform_ptr(next ? Kn : Kh), *vb = uniform_ptr(next ? Vn : Vh);
                const int j0 = __builtin_amdgcn_readfirstlane((next ? t - nend : t) * BK);
                // (MODE 1: every block has the same key length)
                const int len = __builtin_amdgcn_readfirstlane((next && !has_next) ? 0 : (next && SCHED) ? nxt.Lk : Lk);
                return rsrc_at(kb, vb, j0, len);
            }
        };
        // one of the four loads (K block 0, V block 0, K block 1, V block 1) of
        // this wave's share of a tile
        auto load1 = [&](const TileRsrc &r, uint8_t *kd, uint8_t *vd, int which) __attribute__((always_inline)) {
            const int i = which >> 1, blk = LPW * wave + i;
            if (which & 1)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    r.v, (void __attribute__((address_space(3))) *)(vd + blk * 1024), 16, vld[i], 0, 0, 0);
            else
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    r.k, (void __attribute__((address_space(3))) *)(kd + blk * 1024), 16, kld[i], 0, 0, 0);
        };
        auto issue = [&](uint8_t *kd, uint8_t *vd, int t) __attribute__((always_inline)) {
            const TileRsrc r = tile_rsrc(t);
#pragma unroll
            for (int w = 0; w < 2 * LPW; ++w) load1(r, kd, vd, w);
        };

        // Q rows q0 .. q0 + BQ - 1 of block n into qs (PERSIST): wave w copies
        // its own 64 rows, 16 loads of 1 KiB laid out like a K tile's; rows at
        // or past the block's valid length read as zeros
        auto issue_q = [&](const Blk &n) __attribute__((always_inline)) {
            const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
                const_cast<uint16_t *>(Q) + ((size_t)(n.b * Hq + n.h) * Nq + n.q0) * D, 0,
                max(0, (SCHED ? n.Lq : Nq) - n.q0) * ROWB, kRsrcWord3);
#pragma unroll
            for (int i = 0; i < QL; ++i) {
                const int blk = QL * wave + i, row = RPB * blk + (lane >> kLogCH), sl = lane & (CH - 1);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (void __attribute__((address_space(3))) *)(qs + blk * 1024), 16,
                                                         row * ROWB + ((sl ^ swk<HD>(row)) << 4), 0, 0, 0);
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

        // ---- Q fragments (B operands of S^T = K Q^T), kept in registers -----
        // lane l holds Q[qw0 + 32 qb + c][64 g + 8 ks + 0..7] for ks = 0..7
        bf16x8 qf[2][KS];
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            const int qi = qw0 + 32 * qb + c;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                if constexpr (PERSIST) {
                    // this wave's rows of qs: row 64 wave + 32 qb + c, chunk 8 g + ks
                    const int row = QW * wave + 32 * qb + c;
                    qf[qb][ks] = *reinterpret_cast<const bf16x8 *>(qs + row * ROWB + ((((CH / 2) * g + ks) ^ swk<HD>(row)) << 4));
                } else {
                    uint4 w = make_uint4(0, 0, 0, 0);
                    if (qi < Lq) w = *reinterpret_cast<const uint4 *>(Q + (qhead + qi) * D + (D / 2) * g + 8 * ks);
                    qf[qb][ks] = __builtin_bit_cast(bf16x8, w);
                }
            }
        }
        // At head dim 64 a wave has 128 VGPRs (two waves per SIMD): the
        // fragments are moved into AGPRs, which the score MFMA reads directly.
        // Left in VGPRs they do not fit, and the compiler parks them in AGPRs
        // and copies each one back before every use (32 copies per tile).
        if constexpr (HD == 64) {
#pragma unroll
            for (int qb = 0; qb < 2; ++qb)
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) asm volatile("" : "+a"(qf[qb][ks]));
        }


        // per-lane LDS byte offsets (within a tile) of the QK A operand: row c,
        // chunk 8 g + ks -> slot (8 g + ks) ^ (c % 16)
        uint32_t koff[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) koff[ks] = c * ROWB + (((((CH / 2) * g) ^ swk<HD>(c)) ^ ks) << 4);
        // transposing V read: 16-lane group q = lane/16, index i = lane%16:
        // row kb + i/4 (kb a multiple of 4), dims 32 dt + 16 (q%2) + 4 (i%4) ..+3
        const int trq = lane >> 4, tri = lane & 15;
        const int tr_row = 4 * (trq >> 1) + (tri >> 2);
        const int tr_sw = swv<HD>(tr_row);
        const int tr_half = (tri & 1) * 8;
        uint32_t voff[NDT];
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
            const int chunk = 4 * dt + 2 * (trq & 1) + ((tri & 3) >> 1);
            voff[dt] = tr_row * ROWB + ((chunk ^ tr_sw) << 4) + tr_half;
        }

        // S^T = K Q^T (raw scores) of one tile: lane holds key 8 r + 4 g + u of
        // the tile in s[qb][4 r + u], query qw0 + 32 qb + c
        auto qk = [&](const uint8_t *kb, f32x16 (&s)[2]) __attribute__((always_inline)) {
            const f32x16 zero = {};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const bf16x8 a = *reinterpret_cast<const bf16x8 *>(kb + koff[ks]);
#pragma unroll
                for (int qb = 0; qb < 2; ++qb)
                    s[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[qb][ks], ks ? s[qb] : zero, 0, 0, 0);
            }
        };

        // key 32 t + 8 r + 4 g + u is visible to query q iff it is <= min(Lk-1, q)
        // (causal) or <= Lk - 1
        auto mask = [&](f32x16 (&s)[2], int t) __attribute__((always_inline)) {
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
                const int qi = qw0 + 32 * qb + c;
                const int lim = (causal ? min(Lk - 1, qi) : Lk - 1) - t * BK - 4 * g;
#pragma unroll
                for (int r = 0; r < 4; ++r)
#pragma unroll
                    for (int u = 0; u < 4; ++u)
                        if (8 * r + u > lim) s[qb][4 * r + u] = kNegInf;
            }
        };

        // tile maximum of each query (both halves of the tile)
        auto tile_max = [&](const f32x16 (&s)[2], float (&tm)[2]) __attribute__((always_inline)) {
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
                float t = fmaxf(fmaxf(s[qb][0], s[qb][1]), s[qb][2]);
#pragma unroll
                for (int i = 3; i < 15; i += 2) t = fmaxf(fmaxf(t, s[qb][i]), s[qb][i + 1]);
                t = fmaxf(t, s[qb][15]);
                const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(t), __float_as_uint(t), false, false);
                tm[qb] = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
            }
        };

        // The reference m only moves when some lane's tile maximum exceeds it by
        // more than kLazy (base-2 units): every weight is then at most 2^kLazy,
        // far from fp32/bf16 overflow, and the final O~/l and LSE do not depend
        // on which common reference was used.  When it moves, O~ and l are
        // rescaled by exp2(m_old - m_new) (0 when m_old is -inf: nothing
        // accumulated yet).
        //
        // th holds this lane's half of each query's tile maximum (lanes l and
        // l ^ 32 hold the two halves of one query's scores).  Every lane being
        // within its bound is the same test as every query's full maximum being
        // within it, so the halves are only combined when the reference moves.
        // mlim = m + kLazy in raw units, kept beside m.
        auto update_ref = [&](const float (&th)[2]) __attribute__((always_inline)) {
            // (one ballot per comparison: the compare writes the lane mask that
            // the ballot reads, with no conversion to a value and back)
            if ((__builtin_amdgcn_ballot_w64(th[0] > mlim[0]) | __builtin_amdgcn_ballot_w64(th[1] > mlim[1])) != 0) {
                acc_settle(oacc);
#pragma unroll
                for (int qb = 0; qb < 2; ++qb) {
                    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(th[qb]), __float_as_uint(th[qb]),
                                                                     false, false);
                    const float tm = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
                    const float mn = fmaxf(m[qb], tm);
                    const float alpha = (mn == kNegInf || m[qb] == mn) ? 1.0f
                                      : (m[qb] == kNegInf ? 0.0f : fast_exp2((m[qb] - mn) * scale_log2));
                    l[qb] *= alpha;
#pragma unroll
                    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
                        for (int i = 0; i < 16; ++i) oacc[qb][dt][i] *= alpha;
                    m[qb] = mn;
                    mlim[qb] = mn + lazy_raw;
                    msub[qb] = (mn == kNegInf) ? 0.0f : mn * scale_log2;
                }
            }
        };

        // slot buffers by (compile-time) index
        auto kslot = [&](auto S) __attribute__((always_inline)) -> uint8_t * {
            constexpr int s = decltype(S)::value & 3;
            return s == 0 ? k0 : s == 1 ? k1 : s == 2 ? k2 : k3;
        };
        auto vslot = [&](auto S) __attribute__((always_inline)) -> uint8_t * {
            constexpr int s = decltype(S)::value & 3;
            return s == 0 ? v0 : s == 1 ? v1 : s == 2 ? v2 : v3;
        };

        // top of iteration j: tile j + 1 resident for every wave, and every wave
        // done with iteration j - 1, whose slot (j + 3) % 4 is refilled here
        // Every iteration issues exactly four loads per wave (tiles past the end
        // are zero fills of consumed slots), so at the top of iteration j the
        // loads of tiles j+1 and j+2 are the ones in flight.
        // With PERSIST and a next block, the 16 loads copying its Q are issued
        // after S(0) (below), behind this block's tiles 1 and 2 and the previous
        // block's O stores: tiles 1 and 2 are then followed by at least 20
        // memory operations, and iterations 0 and 1 wait with vmcnt(20), so the
        // copy and the stores are not waited for there.
        auto enter = [&](int j) __attribute__((always_inline)) {
            if (PERSIST && has_next && j < 2)
                __builtin_amdgcn_s_waitcnt(kWaitVmQ);
            else
                __builtin_amdgcn_s_waitcnt(kWaitVmTile);
            tile_barrier();
        };
        auto idle = [&](auto S, int j) __attribute__((always_inline)) {
            enter(j);
            issue(kslot(Slot<decltype(S)::value + 3>{}), vslot(Slot<decltype(S)::value + 3>{}), j + AHEAD);
        };

        // Iteration j, laid out as 32 MFMA steps: steps 0-15 compute
        // S(j+1) = K(j+1) Q^T, steps 16-31 add P~(j) V(j) to O~.  The vector
        // work rides between them, software-pipelined so that no step waits on
        // a result produced in the same step: the 32 exponential items of tile j
        // go through three stages (fma, exp2, sum/convert) in consecutive steps,
        // each bf16 P~ operand ready before its P~V step; then the maximum of
        // tile j+1 as a shallow tree.  Operand reads run four or five steps
        // ahead of their MFMA.  sched_barrier keeps the compiler from regrouping
        // the steps.  With MASKED, the scores of tile j+1 are masked first.
        auto body = [&](auto S, auto MASKED, int j) __attribute__((always_inline)) {
            constexpr bool masked = decltype(MASKED)::value != 0;
            enter(j);
            const uint8_t *kb = kslot(Slot<decltype(S)::value + 1>{});
            const uint8_t *vb = vslot(S);
            uint8_t *kd = kslot(Slot<decltype(S)::value + 3>{});
            uint8_t *vd = vslot(Slot<decltype(S)::value + 3>{});
            const TileRsrc lr = masked ? tile_rsrc(j + AHEAD) : tile_rsrc_cur(j + AHEAD);
            const f32x16 zero = {};
            float e[2][16];
            float rs[2][4];      // four partial row sums per block, set by their first item
            bf16x8 pb[2][2];
            f32x16 sn[2];
            bf16x8 ka[KS];
            bf16x8 va[2][NDT];
            float px[2][6];

            // stage 0 (fma), 1 (exp2) or 2 (sum, and the bf16 operand after the
            // eighth item of an operand) of the items of group G
            auto stage = [&](auto STAGE, auto G) __attribute__((always_inline)) {
                constexpr int stg = decltype(STAGE)::value, grp = decltype(G)::value - 1;
                static_for<item_lo<HD>(grp), item_lo<HD>(grp + 1)>([&](auto N) __attribute__((always_inline)) {
                    constexpr int n = decltype(N)::value, qb = item_qb(n), i = item_i(n);
                    if constexpr (stg == 0) {
                        e[qb][i] = fmaf(sacc[qb][i], scale_log2, -msub[qb]);
                    } else if constexpr (stg == 1) {
                        e[qb][i] = fast_exp2(e[qb][i]);
                    } else {
                        // items n < 4 and 8 <= n < 12 are the first to reach rs[qb][n & 3]
                        // (starting from 0.0f would cost an add: 0 + x is not x for x = -0)
                        if constexpr (n < 16 && !(n & 4))
                            rs[qb][i & 3] = e[qb][i];
                        else
                            rs[qb][i & 3] += e[qb][i];
                        if constexpr ((n & 7) == 7) {
                            constexpr int hh = n >> 4;
                            f32x8 f;
#pragma unroll
                            for (int k = 0; k < 8; ++k) f[k] = e[qb][8 * hh + k];
                            pb[qb][hh] = __builtin_convertvector(f, bf16x8);
                        }
                    }
                });
            };
            auto rk = [&](int ks) __attribute__((always_inline)) {
                ka[ks] = *reinterpret_cast<const bf16x8 *>(kb + koff[ks]);
            };
            auto rv = [&](int hh, int dt) __attribute__((always_inline)) {
                const uint8_t *base = vb + 16 * hh * ROWB + voff[dt];
                const bf16x4 lo4 = lds_read_tr(base);
                const bf16x4 hi4 = lds_read_tr(base + 8 * ROWB);
                va[hh][dt] = __builtin_shufflevector(lo4, hi4, 0, 1, 2, 3, 4, 5, 6, 7);
            };

            rk(0);
            rk(1);
            stage(Slot<0>{}, Slot<0>{});          // fma of group -1
            __builtin_amdgcn_sched_barrier(0);
            static_for<0, STEPS>([&](auto ST) __attribute__((always_inline)) {
                constexpr int st = decltype(ST)::value;
                constexpr int SS = 2 * KS;       // score steps, then P~V steps
                if constexpr (st < SS) {
                    constexpr int ks = st >> 1, qb = st & 1;
                    sn[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[ks], qf[qb][ks], ks ? sn[qb] : zero, 0, 0, 0);
                } else {
                    constexpr int t = st - SS, hh = t / (2 * NDT), dt = (t >> 1) % NDT, qb = t & 1;
                    mfma_acc(oacc[qb][dt], va[hh][dt], pb[qb][hh]);
                }
                // this wave's loads of tile j+3, one every eight steps
                if constexpr ((st & 7) == 3) load1(lr, kd, vd, st >> 3);
                // K operand of step 2 ks is read at step 2 ks - 4
                if constexpr (st < SS - 4 && !(st & 1)) rk((st + 4) >> 1);
                // V operand of step SS + 2 NDT hh + 2 dt is read five steps earlier
                if constexpr (st >= SS - 5 && st < SS - 5 + 4 * NDT && ((st - (SS - 5)) & 1) == 0)
                    rv(((st - (SS - 5)) >> 1) / NDT, ((st - (SS - 5)) >> 1) % NDT);
                // exponential pipeline: fma of group st, exp2 of st-1, sum of st-2
                // (Slot<g + 1> names group g)
                if constexpr (st < kGroups) stage(Slot<0>{}, Slot<st + 1>{});
                if constexpr (st <= kGroups) stage(Slot<1>{}, Slot<st>{});
                if constexpr (st >= 1 && st <= kGroups + 1) stage(Slot<2>{}, Slot<st - 1>{});
                // masked iterations: mask S(j+1) once its MFMAs are done
                // (the eight (qb, r) row groups over 2 NDT steps from step SS + 1:
                // one per step at head dim 128, two at 64)
                constexpr int kMaskPer = 8 / (2 * NDT);
                if constexpr (masked && st > SS && st <= SS + 2 * NDT) {
                    constexpr int k = (st - SS - 1) * kMaskPer;
#pragma unroll
                    for (int kk = k; kk < k + kMaskPer; ++kk) {
                        const int qb = kk >> 2, r = kk & 3;
                        const int qi = qw0 + 32 * qb + c;
                        const int lim = (causal ? min(Lk - 1, qi) : Lk - 1) - (j + 1) * BK - 4 * g;
#pragma unroll
                        for (int u = 0; u < 4; ++u)
                            if (8 * r + u > lim) sn[qb][4 * r + u] = kNegInf;
                    }
                }
                // maximum of tile j+1: five independent max3 per block, then two
                // (head dim 64: k = 0..2 at step 13, 3..4 at 14, joined at 15)
                static_for<0, 5>([&](auto KK) __attribute__((always_inline)) {
                    constexpr int k = decltype(KK)::value;
                    constexpr int kst = HD == 128 ? 25 + k : (k < 3 ? 13 : 14);
                    if constexpr (st == kst) {
#pragma unroll
                        for (int qb = 0; qb < 2; ++qb)
                            px[qb][k] = fmaxf(fmaxf(sn[qb][3 * k], sn[qb][3 * k + 1]), sn[qb][3 * k + 2]);
                    }
                });
                if constexpr (st == (HD == 128 ? 30 : 15)) {
#pragma unroll
                    for (int qb = 0; qb < 2; ++qb) {
                        px[qb][0] = fmaxf(fmaxf(px[qb][0], px[qb][1]), px[qb][2]);
                        px[qb][3] = fmaxf(fmaxf(px[qb][3], px[qb][4]), sn[qb][15]);
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
            });
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
                l[qb] += (rs[qb][0] + rs[qb][1]) + (rs[qb][2] + rs[qb][3]);
                sacc[qb] = sn[qb];
            }
            float th[2];    // this lane's half of the tile maximum
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
                th[qb] = fmaxf(px[qb][0], px[qb][3]);
                // past the last tile the scores are of stale LDS data: unused
                if (masked && j + 1 >= wtiles) th[qb] = kNegInf;
            }
            update_ref(th);
        };

        // ---- prologue: tiles 0 .. AHEAD-1 in flight, S(0) and its maximum ----
        // tiles 0..2 (zero fills past the end); iteration 0 fills slot 3
        // (with PERSIST the tiles were loaded before the Q fragments were read:
        // by the block start above, or by the last iterations of the previous
        // block, whose final wait and barrier leave tile 0 resident)
        if (!PERSIST) {
            issue(k0, v0, 0);
            issue(k1, v1, 1);
            issue(k2, v2, 2);
            __builtin_amdgcn_s_waitcnt(0);   // nothing in flight (Q included)
            __syncthreads();
        }
        if (wtiles > 0) {
            qk(k0, sacc);
            if (wfirst_mask == 0) mask(sacc, 0);
            float tm[2];
            tile_max(sacc, tm);
#pragma unroll
            for (int qb = 0; qb < 2; ++qb) {
                // nothing accumulated yet: take the tile maximum as reference
                m[qb] = tm[qb];
                mlim[qb] = tm[qb] + lazy_raw;
                msub[qb] = (tm[qb] == kNegInf) ? 0.0f : tm[qb] * scale_log2;
            }
        }
        if (has_next) {
            // this wave's reads of qs are complete (its own rows only): copy the
            // next block's Q over them
            __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
            issue_q(nxt);
        }

        // ---- main loop (unrolled by the ring size), then the masked tail -----
        // Control flow never joins two versions of the accumulators that both
        // came out of MFMAs (the compiler would copy all 128 of them through
        // VGPRs): the masked loop also runs in whole groups of four, and its
        // iterations past wtiles only load and pass the barrier.  Every wave
        // passes the same barriers.
        int j = 0;
        for (; j + 4 <= nfast; j += 4) {
            body(Slot<0>{}, Slot<0>{}, j);
            body(Slot<1>{}, Slot<0>{}, j + 1);
            body(Slot<2>{}, Slot<0>{}, j + 2);
            body(Slot<3>{}, Slot<0>{}, j + 3);
        }
        for (; j < wend; j += 4) {
            body(Slot<0>{}, Slot<1>{}, j);
            if (j + 1 < wtiles) body(Slot<1>{}, Slot<1>{}, j + 1); else idle(Slot<1>{}, j + 1);
            if (j + 2 < wtiles) body(Slot<2>{}, Slot<1>{}, j + 2); else idle(Slot<2>{}, j + 2);
            if (j + 3 < wtiles) body(Slot<3>{}, Slot<1>{}, j + 3); else idle(Slot<3>{}, j + 3);
        }
        // this wave is done; keep loading and passing barriers with the others
        for (; j < nend; j += 4) {
            idle(Slot<0>{}, j);
            idle(Slot<1>{}, j + 1);
            idle(Slot<2>{}, j + 2);
            idle(Slot<3>{}, j + 3);
        }
        // no load outlives the last block (the next block's tiles 1 and 2 stay
        // in flight otherwise)
        if (!has_next) __builtin_amdgcn_s_waitcnt(kWaitVm0);

        // ---- epilogue: O = O~ / l once, LSE = m + log l ------------------------
        acc_settle(oacc);
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
            const int qi = qw0 + 32 * qb + c;
            const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(l[qb]), __float_as_uint(l[qb]), false, false);
            const float lt = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
            const bool valid = (qi < Lq) && (lt > 0.0f);
            const float inv = valid ? 1.0f / lt : 0.0f;
            if (qi < Nq) {
                uint16_t *orow = O + (qhead + qi) * D;
#pragma unroll
                for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        uint2 w;
                        w.x = valid ? pack_bf16x2_hw(oacc[qb][dt][4 * r + 0] * inv, oacc[qb][dt][4 * r + 1] * inv) : 0u;
                        w.y = valid ? pack_bf16x2_hw(oacc[qb][dt][4 * r + 2] * inv, oacc[qb][dt][4 * r + 3] * inv) : 0u;
                        *reinterpret_cast<uint2 *>(orow + 32 * dt + 8 * r + 4 * g) = w;
                    }
                if (LSE && g == 0)
                    LSE[qhead + qi] = valid ? (m[qb] * scale_log2 + __log2f(lt)) * kLn2 : kNegInf;
            }
        }
        if (!has_next) break;
        L = Lnext;
        ++item;
        first = false;
    }   // blocks
    // blocks without work (SCHED): O = 0, LSE = -inf
    if constexpr (SCHED)
        for (int k = n_compute; k < n_items; ++k) zero_fill(item_blk(sched[k]));
}

#define OSM_ATTN_FWD_PARAMS                                                                          \
    const uint16_t *__restrict__ Q, const uint16_t *__restrict__ K, const uint16_t *__restrict__ V, \
        uint16_t *__restrict__ O, float *__restrict__ LSE, int B, int Hq, int Hkv, int Nq, int Nk,   \
        const int32_t *__restrict__ seqlens_q, const int32_t *__restrict__ seqlens_k,               \
        float scale_log2, int causal, int nqb, int xcd_heads, int nblocks

// Workgroups resident per compute unit: at head dim 128 one (each wave has
// the 512 registers of its SIMD); at 64 two (a wave fits in 256 registers and
// a workgroup in 33 KiB of LDS), so that one wave's exponentials overlap the
// other's matrix products -- the vector work per MFMA is twice that of head
// dim 128.
template <int HD> constexpr int kWgPerCu = HD == 128 ? 1 : 2;

// One query block per workgroup (attn_fwd_bf16_d<HD>); at head dim 128 also
// one workgroup per compute unit walking several equal query blocks
// (_persist) or a static schedule of unequal blocks (_sched).  At head dim 64
// the two workgroups of a compute unit hide each other's block starts and
// ends, and one block per workgroup measured 6-8% faster than both
// persistent grids, so those are not built there.
#define OSM_FWD_KERNEL(HD, MODE, NAME)                                                               \
    __global__ void __launch_bounds__(NT, kWgPerCu<HD>) NAME(OSM_ATTN_FWD_PARAMS) {                  \
        attn_fwd_body<MODE, HD>(Q, K, V, O, LSE, B, Hq, Hkv, Nq, Nk, seqlens_q, seqlens_k, scale_log2, \
                                causal, nqb, xcd_heads, nblocks);                                    \
    }
OSM_FWD_KERNEL(128, 0, attn_fwd_bf16_d128)
OSM_FWD_KERNEL(128, 1, attn_fwd_bf16_d128_persist)
OSM_FWD_KERNEL(128, 2, attn_fwd_bf16_d128_sched)
OSM_FWD_KERNEL(64, 0, attn_fwd_bf16_d64)
#undef OSM_FWD_KERNEL
#undef OSM_ATTN_FWD_PARAMS

}  // namespace

hipError_t launch_attn_fwd(const AttnFwdArgs &a, hipStream_t s) {
    const int nqb = (a.seqlen_q + BQ - 1) / BQ;
    const int nheads = a.batch * a.heads_q;
    const int64_t blocks = (int64_t)nqb * nheads;
    if (blocks == 0) return hipSuccess;
    const int xcd_heads = (nheads % 8 == 0) ? nheads / 8 : 0;
    int cus = 0;
    {
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            cus = 0;
        cus &= ~7;   // whole XCDs' worth, so block L keeps running on XCD L % 8
    }
    // Head dim 128: full-length non-causal inputs with more blocks than
    // compute units run on a persistent grid of one workgroup per compute
    // unit (MODE 1); causal or varlen inputs on the scheduled persistent grid
    // (MODE 2) when each XCD's heads and its list fit the schedule's limits
    // (slots per XCD at most 64, at most kSchedMax blocks per XCD, slot loads
    // below 2^24 tiles) and an XCD has at most 32 heads: with 64 (short
    // sequences, such as 512 heads of 1024 queries) building the schedule
    // cost more than it saved, and one block per workgroup measured 12%
    // faster.  Everything else, and head dim 64, one block per workgroup
    // (MODE 0).
    const bool uniform = !a.causal && !a.seqlens_q && !a.seqlens_k && a.seqlen_k > 0;
    const int64_t per_xcd = xcd_heads ? (int64_t)xcd_heads * nqb : 0;
    const int64_t max_tiles = per_xcd * ((a.seqlen_k + BK - 1) / BK + kSchedFixed);
    int mode = 0;
    const int pgrid = cus * kWgPerCu<128>;
    if (a.head_dim == 128 && pgrid > 0 && blocks > pgrid) {
        if (uniform) mode = 1;
        else if (xcd_heads > 0 && xcd_heads <= 32 && pgrid / 8 <= 64 && per_xcd <= kSchedMax &&
                 max_tiles < ((int64_t)1 << 24))
            mode = 2;
    }
    const unsigned grid = mode ? (unsigned)pgrid : (unsigned)blocks;
    const uint16_t *q = static_cast<const uint16_t *>(a.q), *k = static_cast<const uint16_t *>(a.k),
                   *v = static_cast<const uint16_t *>(a.v);
    uint16_t *o = static_cast<uint16_t *>(a.o);
#define OSM_FWD_LAUNCH(KERNEL)                                                                         \
    hipLaunchKernelGGL(KERNEL, dim3(grid), dim3(NT), 0, s, q, k, v, o, a.lse, a.batch, a.heads_q,     \
                       a.heads_kv, a.seqlen_q, a.seqlen_k, a.seqlens_q, a.seqlens_k, a.scale * kLog2e, \
                       a.causal, nqb, xcd_heads, (int)blocks)
    if (a.head_dim == 128) {
        if (mode == 1) OSM_FWD_LAUNCH(attn_fwd_bf16_d128_persist);
        else if (mode == 2) OSM_FWD_LAUNCH(attn_fwd_bf16_d128_sched);
        else OSM_FWD_LAUNCH(attn_fwd_bf16_d128);
    } else {
        OSM_FWD_LAUNCH(attn_fwd_bf16_d64);
    }
#undef OSM_FWD_LAUNCH
    return hipGetLastError();
}

}  // namespace osm
