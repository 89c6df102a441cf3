// MFMA attention forward for gfx950 (CDNA4): the library's hot path.
//
// Method.  Standard attention S = QK^T * scale, P = softmax(S), O = PV,
// computed tile by tile so that S and P never leave the registers, with the
// online-softmax statistics of "FlashAttention: turning the quadratic
// intermediate matrices into statistics" (section 3.1): per query row a
// reference max m, the exp-sum l relative to m and the output accumulator
// relative to m; when m is replaced by a larger m', l and the accumulator are
// multiplied by 2^(m - m').  Exponentials are base 2 with the scale and
// log2(e) folded into one fp32 factor applied to the fp32 scores (inputs are
// never pre-scaled in 16-bit), and l sums the fp32 probabilities.  Partial
// results over disjoint key sets combine the same way (m = max of the two,
// each side scaled by 2^(m_side - m)), which is how the waves that share a
// row block merge their results at the end.
//
// The reference max of a row is set from the first tile's scores; later tiles
// are exponentiated against it without computing their max (any reference
// gives the same O = u / l and LSE = m + log2 l, and every row's largest
// probability is at least 1, so none underflows to a zero sum).  Only an
// overflow is wrong: when a probability passes the 16-bit range (seen as an
// inf or NaN accumulator for fp16, as an fp32 row sum past the largest bf16
// for bf16), the work-group redoes the q-tile in a safe form that moves a
// row's reference whenever a tile's max exceeds it by more than 2^8.  The row
// sums are taken in fp32 from the unrounded probabilities.  For fp16 inputs
// they also normalise the output (rounding P to fp16 moves the product by at
// most 2^-11 relative); for bf16 inputs the output is normalised by the sum
// of the probabilities as rounded for the PV product (one v_dot2 per pair),
// so that the rounding of a dominant probability cancels between numerator
// and denominator.
//
// Work decomposition.  A work-group of 4 waves owns BM = 128 query rows of
// one (batch, head) at a time and walks the keys in tiles of BN = 64 keys.
// Its waves form a 2 x 2 grid: wave w takes the 64 rows of row half w & 1
// (two 32-row blocks) against the 32 keys of key half w >> 1 of every tile,
// so each K and V fragment read from LDS feeds two products.  At the end the
// two waves of a row half merge their partial results through LDS.  d = 64:
// two work-groups per CU (256 registers per wave, 80 KiB of LDS each), so
// that each SIMD runs waves of two independent work-groups whose softmax and
// matrix products interleave; d = 128 (the accumulator alone takes 128
// registers): one work-group per CU.
//
// K and V tiles go from global memory straight into LDS (buffer_load_dwordx4
// ... lds, written as inline asm) through a ring of 5 stages, 3 tiles ahead
// of use, with one barrier per tile.  The kernel orders every fragment read
// after the copies into its stage with its own vmcnt waits and that barrier.
// The stages are separate LDS arrays and the loop is unrolled by 5, so every
// fragment address in the steady loop is a constant stage base plus one
// per-lane offset.
//
// Software pipeline.  Step j of a wave interleaves, in one instruction
// stream, the matrix products of two neighbouring tiles with the vector work
// of the tile between them: S(j+1) = Q K(j+1)^T and O += P(j-1) V(j-1) on the
// matrix cores while the softmax of S(j) runs on the vector ALUs.
//
// LDS layout.  Tiles are stored fragment-major: every 1 KiB block holds
// exactly the 64 lanes' operands of one MFMA (K) or of two transposing reads
// (V), in lane order.  Every fragment read is then one contiguous,
// bank-conflict-free access at a per-lane base plus an immediate offset, and
// each DMA instruction fills one block.
//
// Transposed products.  A wave computes S^T = K Q^T and O^T = V^T P^T with
// v_mfma_f32_32x32x16_{f16,bf16}.  In the 32x32 result layout lane l holds
// column l % 32, i.e. one query row, so every lane owns all of its row's
// scores (shared with lane l ^ 32): row maxima and sums are lane-local plus
// one v_permlane32_swap, the rescale needs no data movement, and the S^T
// accumulator already has the lane layout of the P^T operand of the second
// product (the contraction order over keys is permuted the same way on both
// operands).  V^T operands come from ds_read_b64_tr_b16, which transposes
// 16-bit data within 16-lane groups.
//
// Causal masking is bottom-right aligned (key j visible to row i iff
// j <= i + Lk - Lq): key tiles wholly above the diagonal of a q-tile are
// never loaded, and the per-key mask is applied only on tiles that straddle
// the diagonal or the key tail.  Causal q-tiles are ordered so that the work
// a CU holds at once is about the same everywhere (see the kernel entry).
//
// This header holds the kernel template; attn_fwd_mfma_d64.hip and
// attn_fwd_mfma_d128.hip instantiate it per head dimension, so that each can
// be compiled with its own code-generation options.
#pragma once
#include <algorithm>
#include <type_traits>

#include "mfma_util.hpp"

namespace mi_attn {
namespace {

constexpr int kBM = 128;     // query rows per q-tile
constexpr int kStages = 5;   // LDS ring of K/V tiles
// Safe form of the softmax: a row's reference max moves only when a tile's
// max exceeds it by more than this (log2 units).
constexpr float kGap = 8.0f;

// Fragment-major tile layout (16-bit elements; a stage holds K then V).
//   K block kb*NKS + ks (512 elements): lane l's 8 elements are
//     K[kb*32 + (l & 31)][(2*ks + (l >> 5))*8 .. +7].
//   V half-block (db*NKC + kc)*2 + r (256 elements): lane l's 4 elements are
//     V[kc*16 + 8*r + 4*(l >> 5) + ((l & 15) >> 2)][db*32 + 16*((l >> 4) & 1)
//       + 4*(l & 3) .. +3],
//   the address pattern of a ds_read_b64_tr_b16 that yields the V^T operand
//   of keys kc*16 + 8*r + 4*hi + 0..3 and columns db*32 + (l & 31).
template <int D>
struct Layout {
    static constexpr int WAVES = 4;          // waves per work-group
    static constexpr int WG_PER_CU = D == 64 ? 2 : 1;   // resident work-groups
    static constexpr int THREADS = 64 * WAVES;
    static constexpr int KQ = WAVES / 2;     // key groups of 32 keys
    static constexpr int BN = 32 * KQ;       // keys per tile
    static constexpr int NKC = BN / 16;      // 16-key chunks per tile
    static constexpr int NKS = D / 16;       // k-steps of QK^T
    static constexpr int NDB = D / 32;       // 32-column blocks of O^T
    static constexpr int ELEMS = BN * D;     // per tile and tensor
    static constexpr int BLOCKS = ELEMS / 512;   // 1 KiB DMA blocks per tensor
    static constexpr int STAGE = 2 * ELEMS;  // K + V
    static constexpr int DPW = 2 * BLOCKS / WAVES;   // DMA blocks per wave
    // merge area: per wave room for its accumulators (ACC floats per lane;
    // the merge publishes one row block of them), then the (m, l, lr) of
    // both row blocks of every wave
    static constexpr int ACC = 2 * NDB * 16;
    static constexpr int SLOTS_PER_STAGE = (STAGE * 2) / (ACC * 64 * 4);
    static_assert(SLOTS_PER_STAGE >= 1, "merge slot fits a stage");
    static_assert(WAVES / SLOTS_PER_STAGE <= kStages - 1, "merge area");
    static_assert(WAVES * 2 * 3 * 64 * 4 <= STAGE * 2, "merge statistics");
    static_assert(kStages * STAGE * 2 * WG_PER_CU <= 160 * 1024, "LDS per CU");
};

// Stage K of the LDS ring of a work-group (one array per stage: in the
// unrolled loop every stage address is a compile-time constant).
template <int D, int K>
__device__ __forceinline__ lds16_t* ring() {
    __shared__ __attribute__((aligned(16))) uint16_t r[Layout<D>::STAGE];
    return (lds16_t*)r;
}

// Philox4x32-10 (Salmon, Moraes, Dror and Shaw, "Parallel random numbers:
// as easy as 1, 2, 3", SC 2011) on counter c with key (k0, k1): each round
// multiplies words 0 and 2 by two constants and mixes the halves of the
// products with the other words and the key; the key gains the Weyl
// increments between rounds.
__device__ __forceinline__ void philox4x32_10(uint32_t (&c)[4], uint32_t k0, uint32_t k1) {
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        const uint64_t p0 = (uint64_t)c[0] * 0xD2511F53u;
        const uint64_t p1 = (uint64_t)c[2] * 0xCD9E8D57u;
        const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c[1] ^ k0;
        const uint32_t n2 = (uint32_t)(p0 >> 32) ^ c[3] ^ k1;
        c[1] = (uint32_t)p1;
        c[3] = (uint32_t)p0;
        c[0] = n0;
        c[2] = n2;
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
}

// Rows and keys of one sequence: the first query row and key in the
// tensors (packed input) and their counts.
struct SeqSpan {
    int q0, lq, k0, lk;
    int tq;                              // packed: all query rows (the LSE row stride)
};

template <int D, typename Tin, typename Tout, bool CAUSAL, bool DROP>
__device__ __forceinline__ void attend_qtile(const FwdParams& p, int qtile,
                                             int h, int b, SeqSpan span) {
    using L = Layout<D>;
    constexpr int BN = L::BN, KQ = L::KQ;
    constexpr int NKC = L::NKC, NKS = L::NKS, NDB = L::NDB;
    constexpr int DPW = L::DPW;
    constexpr int STAGES = kStages;
    constexpr int AHEAD = STAGES - 2;    // copies run AHEAD tiles ahead
    static_assert(2 * L::BLOCKS % L::WAVES == 0, "blocks per wave");
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    using I3 = std::integral_constant<int, 3>;
    using I4 = std::integral_constant<int, 4>;

    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);   // scalar
    const int kq = wave >> 1;            // key group of every tile
    const int rh = wave & 1;             // row half of the q-tile
    // Lane indices.  Derived afresh (refresh_lane) where the code after the
    // key loop starts, from the execution mask rather than the thread id, so
    // nothing derived from the lane stays live (or spilled) across the loop.
    int lane = lane_id();
    int hi = lane >> 5;                  // which half of the wave
    int col = lane & 31;                 // the query row this lane owns
    auto refresh_lane = [&]() {
        lane = lane_id();
        hi = lane >> 5;
        col = lane & 31;
    };

    const int q0 = span.q0, lq_b = span.lq, k0 = span.k0, lk_b = span.lk;
    // packed: the LSE row stride (the dropout kernels, short of registers,
    // load it in the epilogue instead of keeping it live)
    const int tq = span.tq;
    const bool packed = p.cu_q != nullptr;
    const int row0 = qtile * kBM;
    if (row0 >= lq_b) return;            // uniform over the work-group
    // kv head h / group as a multiply-high by ceil(2^32 / group): exact for
    // h and group below 2^16 (the caller's limit on hq)
    const int g = (int)(((uint64_t)(uint32_t)h * p.group_magic) >> 32);
    static_assert(sizeof(p.group_magic) == 8, "64-bit reciprocal");
    const int diag = lk_b - lq_b;        // key j visible to row i iff j <= i + diag

    const uint16_t* qg = reinterpret_cast<const uint16_t*>(p.q) +
                         (packed ? 0 : (int64_t)b * p.q_sb) +
                         (int64_t)h * p.q_sh + (int64_t)(q0 + row0) * p.q_sr;
    const uint16_t* kg = reinterpret_cast<const uint16_t*>(p.k) +
                         (packed ? 0 : (int64_t)b * p.k_sb) +
                         (int64_t)g * p.k_sh + (int64_t)k0 * p.k_sr;
    const uint16_t* vg = reinterpret_cast<const uint16_t*>(p.v) +
                         (packed ? 0 : (int64_t)b * p.v_sb) +
                         (int64_t)g * p.v_sh + (int64_t)k0 * p.v_sr;

    // Key tiles this q-tile needs: keys [0, kend) in tiles of BN.
    int kend = lk_b;
    if (CAUSAL) kend = min(kend, row0 + kBM + diag);
    const int n_kt = kend > 0 ? (kend + BN - 1) / BN : 0;

    // Q fragments (B operand of S^T = K Q^T) of the wave's two row blocks:
    // lane holds row `col` of block rb, columns ks*16 + 8*hi .. +7.
    const int wrow0 = row0 + 64 * rh;    // first row of this wave
    // This lane's row of block rb (sequence-local) and the last key it may
    // see; recomputed where needed rather than held across the key loop.
    auto qrow = [&](int rb) { return wrow0 + 32 * rb + col; };
    auto last_key = [&](int rb) {
        return CAUSAL ? min(lk_b - 1, qrow(rb) + diag) : lk_b - 1;
    };
    u32x4_t qf[2][NKS];
    // Q goes to LDS stage 3 (which no K/V copy fills before step 0) by the
    // same kind of copy as the K/V tiles, in fragment order: block
    // qb = (rh * 2 + rb) * NKS + ks holds lane l's 8 elements of row
    // 64 rh + 32 rb + (l & 31) of the q-tile, columns ks*16 + 8*(l >> 5)
    // .. +7.  Each wave copies NKS of the 4 * NKS blocks; after the first
    // barrier every wave reads the 2 * NKS blocks of its row half.  Rows
    // past the sequence end read as zeros (range of the buffer resource).
    constexpr int QPW = NKS;             // Q blocks copied per wave
    static_assert(4 * NKS * 512 <= L::STAGE, "Q area fits a stage");
    auto issue_q = [&]() {
        const int rows = min(lq_b - row0, kBM);
        const uint64_t a = reinterpret_cast<uint64_t>(qg);
        u32x4_t rs;
        rs[0] = __builtin_amdgcn_readfirstlane((uint32_t)a);
        rs[1] = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32) & 0xffffu);
        rs[2] = __builtin_amdgcn_readfirstlane((uint32_t)(rows * p.q_sr * 2));
        rs[3] = 0x00020000u;
        const int qb0 = wave * QPW;
        const uint32_t off0 = (uint32_t)((((64 * (qb0 / (2 * NKS)) + 32 * ((qb0 / NKS) & 1) +
                                             (lane & 31)) * p.q_sr) +
                                           (qb0 % NKS) * 16 + 8 * (lane >> 5)) * 2);
#pragma unroll
        for (int t = 0; t < QPW; ++t) {
            const int qb = qb0 + t;
            const int drow = 64 * (qb / (2 * NKS) - qb0 / (2 * NKS)) +
                             32 * (((qb / NKS) & 1) - ((qb0 / NKS) & 1));
            const int dcol = 16 * (qb % NKS - qb0 % NKS);
            const uint32_t delta = __builtin_amdgcn_readfirstlane(
                (uint32_t)((drow * p.q_sr + dcol) * 2));
            const uint32_t lds_addr =
                (uint32_t)reinterpret_cast<uintptr_t>(ring<D, 3>() + qb * 512);
            asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds"
                         :: "v"(off0 + delta), "s"(rs), "{m0}"(lds_addr) : "memory");
        }
    };
    auto read_q = [&]() {
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks)
                qf[rb][ks] = *reinterpret_cast<lds_u32x4_t*>(
                    ring<D, 3>() + ((rh * 2 + rb) * NKS + ks) * 512 + lane * 8);
    };

    // DMA plan of this lane: which block of a tile it fills and the byte
    // offset, from the tile's first row, of the 16 bytes it copies.  Copies
    // go through a buffer resource whose range ends with the sequence, so
    // rows past the key range read as zeros (their scores are masked anyway).
    uint32_t dma_voff[DPW];
    int dma_dst[DPW];
    int dma_delta[DPW];                  // dma_voff[t] - dma_voff[0], uniform
    const bool dma_is_v = wave * DPW >= L::BLOCKS;   // waves copy K or V
    const int64_t dma_sr = dma_is_v ? p.v_sr : p.k_sr;
    const uint16_t* dma_base = dma_is_v ? vg : kg;
#pragma unroll
    for (int t = 0; t < DPW; ++t) {
        const int blk = wave * DPW + t;   // 0 .. 2*BLOCKS-1
        const int bi = dma_is_v ? blk - L::BLOCKS : blk;
        int r, c;
        if (!dma_is_v) {                 // K block bi = kb*NKS + ks
            const int kb = bi / NKS, ks = bi % NKS;
            r = kb * 32 + (lane & 31);
            c = (2 * ks + (lane >> 5)) * 8;
        } else {                         // V half-blocks 2*bi, 2*bi + 1
            const int db = bi / NKC, kc = bi % NKC;
            const int rr = lane >> 5;    // which half-block
            const int t2 = 2 * (lane & 31);   // transposing-read lane covered
            r = kc * 16 + 8 * rr + 4 * (t2 >> 5) + ((t2 & 15) >> 2);
            c = db * 32 + 16 * ((t2 >> 4) & 1) + 4 * (t2 & 3);
        }
        dma_voff[t] = (uint32_t)(((int64_t)r * dma_sr + c) * 2);
        dma_dst[t] = (dma_is_v ? L::ELEMS : 0) + bi * 512;
    }
    // Only the first offset stays in a vector register; the others differ
    // from it by amounts that are the same for every lane of the wave.
#pragma unroll
    for (int t = 0; t < DPW; ++t)
        dma_delta[t] = __builtin_amdgcn_readfirstlane((int)(dma_voff[t] - dma_voff[0]));
    const uint32_t dma_voff0 = dma_voff[0];
    // Tiles past the last one get an empty range: their copies read nothing
    // and write zeros, so every step issues the same copies and waits for
    // the same counts.
    // Buffer resource: base address (48 bits, stride 0), range in bytes, and
    // the fourth word of a raw 32-bit buffer.
    auto tile_rsrc = [&](int kt) {
        const int rows = kt < n_kt ? min(lk_b - kt * BN, BN) : 0;
        const uint64_t a = reinterpret_cast<uint64_t>(dma_base + (int64_t)kt * BN * dma_sr);
        u32x4_t r;
        r[0] = __builtin_amdgcn_readfirstlane((uint32_t)a);
        r[1] = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32) & 0xffffu);
        r[2] = __builtin_amdgcn_readfirstlane((uint32_t)(rows * dma_sr * 2));
        r[3] = 0x00020000u;
        return r;
    };
    // The copy is written as inline asm (no result register; M0 takes the
    // LDS address), so the compiler does not track it: every read of a
    // stage is ordered after the copies into it by this kernel's own vmcnt
    // waits and the barrier that follows them -- needed anyway, since a
    // stage is filled by all waves -- and the compiler adds no wait for all
    // copies in flight where it cannot tell the stages apart.
    auto issue_part = [&](const u32x4_t& rsrc, lds16_t* stage, int t) {
        const uint32_t lds_addr = (uint32_t)reinterpret_cast<uintptr_t>(stage + dma_dst[t]);
        asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds"
                     :: "v"(dma_voff0 + (uint32_t)dma_delta[t]), "s"(rsrc), "{m0}"(lds_addr)
                     : "memory");
    };
    auto issue_tile = [&](int kt, lds16_t* stage) {
        const auto rsrc = tile_rsrc(kt);
#pragma unroll
        for (int t = 0; t < DPW; ++t) issue_part(rsrc, stage, t);
    };

    // The prologue's copies (tile 0, Q, tile 1) go out before the rest of
    // the set-up, whose instructions then overlap their latency.
    auto issue_first = [&]() {
        issue_tile(0, ring<D, 0>());
        issue_q();
        issue_tile(1, ring<D, 1>());
    };
    if (n_kt > 0) issue_first();

    const float c2 = p.scale_log2;       // |scale| * log2(e)
    float m[2], l[2], lr[2];             // per row block: reference max (log2
    f32x16_t acc[2][NDB];                // domain), this lane's exp-sums, O^T
    float nm[2];                         // -m, or 0 while m is -inf
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
        m[rb] = -__builtin_inff();
        nm[rb] = 0.0f;
        l[rb] = 0.0f;
        lr[rb] = 0.0f;                   // sum of the rounded P (bf16)
#pragma unroll
        for (int db = 0; db < NDB; ++db) acc[rb][db] = f32x16_t{};
    }

    // Pipeline registers: S(j) of both row blocks, P(j-1) and the V(j-1)
    // fragments of the wave's key group (16-key chunks c = 0, 1).  V(j-1) is
    // read in the step that uses it; the products S(j+1) of row block 0 go
    // first while it lands.
    f32x16_t s_cur[2];
    u32x4_t p_prev[2][2];
    u32x4_t vf[NDB][2];
    // bf16 only: the low part of P(j-1) when tile j-1 was a masked tile,
    // zero otherwise; only the masked steps and the last tile read it
    u32x4_t p_lo[2][2];
    auto clear_p_lo = [&]() {
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int rb = 0; rb < 2; ++rb) p_lo[rb][c] = u32x4_t{0u, 0u, 0u, 0u};
    };
#pragma unroll
    for (int c = 0; c < 2; ++c) {
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) p_prev[rb][c] = u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
        for (int db = 0; db < NDB; ++db) vf[db][c] = u32x4_t{0u, 0u, 0u, 0u};
    }
    // with dropout every step reads the low part of the previous P
    if constexpr (Mma<Tin>::kSplit && DROP) clear_p_lo();

    // Per-lane element offsets of the wave's fragments in a stage, opaque to
    // the optimiser (re-pinned after every step's barrier): every fragment
    // address is one stage array plus one variable index plus a constant,
    // and no fragment read can be hoisted above the barrier that makes its
    // stage's copies visible.
    int k_off = (kq * NKS) * 512 + lane * 8;
    int v_off = L::ELEMS + (2 * kq) * 512 + lane * 4;
    asm volatile("" : "+v"(k_off));
    asm volatile("" : "+v"(v_off));
    auto read_k = [&](const lds16_t* stage, u32x4_t (&kf)[NKS]) {
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
            kf[ks] = *reinterpret_cast<lds_u32x4_t*>(stage + k_off + ks * 512);
    };
    auto read_v = [&](const lds16_t* stage) {
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                const lds16_t* vb = stage + v_off + (db * NKC + c) * 512;
                const u32x2_t a = __builtin_bit_cast(u32x2_t, lds_read_tr(vb));
                const u32x2_t d = __builtin_bit_cast(u32x2_t, lds_read_tr(vb + 256));
                vf[db][c] = u32x4_t{a[0], a[1], d[0], d[1]};
            }
    };
    // -inf for the scores of keys past the row's last visible key; applied
    // only in steps whose tile may hold such keys for some row of the
    // work-group (causal diagonal, end of the key range).
    auto mask_cur = [&](int kt) {
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
            const int lim = last_key(rb) - (kt * BN + 32 * kq + 4 * hi);
#pragma unroll
            for (int e = 0; e < 16; ++e)
                if (8 * (e >> 2) + (e & 3) > lim) s_cur[rb][e] = -__builtin_inff();
        }
    };
    // With dropout, bf16 P is split into hi + lo on every tile: the output
    // is normalised by the fp32 sums of the probabilities before dropout,
    // so the rounding of P does not cancel as it does with the rounded sums.
    constexpr bool kSplitAll = Mma<Tin>::kSplit && DROP;
    // Dropout.  Part g4 of row block rb of tile kt holds the scores of keys
    // kt*BN + 32 kq + 4 hi + 8 g4 + i (i = 0..3).  One Philox call on counter
    // (2 (key / 16) + (key / 4) % 2, sequence row, head, sequence) gives 8
    // 16-bit halves, which decide this lane's 8 keys of a 16-key group:
    // parts g4 and g4 + 1 for even g4 (words 0, 1 and words 2, 3).
    auto drop_words = [&](int kt, int rb, int g4, uint32_t (&c)[4]) {
        c[0] = (uint32_t)(2 * (kt * (BN / 16) + 2 * kq + (g4 >> 1)) + hi);
        c[1] = (uint32_t)qrow(rb);
        c[2] = (uint32_t)h;
        c[3] = (uint32_t)b;
        philox4x32_10(c, p.seed_lo, p.seed_hi);
    };
    // key i of a part is kept iff half i of (w0, w1) is at least the
    // threshold; kept probabilities are scaled by 1 / (1 - p), dropped ones
    // are 0
    auto drop_apply = [&](uint32_t w0, uint32_t w1, float (&x)[4]) {
        const uint32_t u[4] = {w0 & 0xffffu, w0 >> 16, w1 & 0xffffu, w1 >> 16};
#pragma unroll
        for (int i = 0; i < 4; ++i) x[i] = u[i] >= p.drop_threshold ? x[i] * p.drop_scale : 0.0f;
    };
    // PV of the last tile; LO: it was a masked tile, so for bf16 its P was
    // split and the low part goes in too
    auto pv_last = [&](auto LO) {
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int rb = 0; rb < 2; ++rb) {
                    acc[rb][db] = Mma<Tin>::run(vf[db][c], p_prev[rb][c], acc[rb][db]);
                    if constexpr (Mma<Tin>::kSplit && (decltype(LO)::value || DROP))
                        acc[rb][db] = Mma<Tin>::run(vf[db][c], p_lo[rb][c], acc[rb][db]);
                }
    };

    // One pipeline step for tile j.  The matrix products of the step -- with
    // NEXT S(j+1) = Q K(j+1)^T of row block 0, then (with PV) O += P(j-1)
    // V(j-1), then S(j+1) of row block 1 -- are spread between groups of the
    // vector work of the softmax of S(j), which depends on none of them.
    // Scheduling barriers keep the order, so the wave issues a product and
    // then vector work while the matrix core runs it.
    //
    // Short form (SAFE false): p = 2^(s*c2 - m) against the references set
    // from the first tile, with no max of the tile at all.  The references
    // never need to move for accuracy: the largest probability of every row
    // is at least 1 (its first tile's max) and larger ones keep their
    // relative precision, so only an overflow (a probability past the range
    // of the 16-bit type, or of fp32) is wrong, and it leaves an inf in the
    // row sums, which only grow.  The caller checks them after the last tile
    // and redoes the q-tile in the safe form if needed.
    //
    // Safe form: every lane takes the max of its own 16 scores of a row;
    // only when some lane's max exceeds its row's reference by more than
    // kGap does the wave exchange the maxima with lane ^ 32, move the
    // references of the rows whose tile max exceeds them by more than kGap,
    // and rescale (the accumulators after this step's products).
    auto compute = [&](int j, auto NEXT, auto PV, auto MASK, auto SAFE,
                       const u32x4_t (&kf)[NKS], f32x16_t (&s_next)[2],
                       int dma_kt, lds16_t* dma_stage, const lds16_t* v_next) {
        constexpr bool next = decltype(NEXT)::value;
        constexpr bool safe = decltype(SAFE)::value;
        constexpr bool masked_tile = decltype(MASK)::value;
        // bf16 on a masked tile: this tile's P is split into hi + lo, and the
        // PV product of the previous tile also takes its lo part (zero when
        // that tile was not masked)
        constexpr bool split = Mma<Tin>::kSplit && (masked_tile || DROP);
        constexpr int NPV = decltype(PV)::value ? 2 * NDB * 2 : 0;
        constexpr int NPVT = split ? 2 * NPV : NPV;   // with the lo products
        constexpr int NQK = next ? 2 * NKS : 0;
        constexpr int NM = NPVT + NQK;
        // The vector work overlaps the matrix products better in smaller
        // pieces (about 2 products per group): the short form gives the
        // exponentials and the packing of each part groups of their own.
        // The bf16 dropout kernel at d = 64 keeps 9 groups (exponentials of
        // a part and packing of the one before in one group): there the
        // finer schedule lengthens live ranges into more spills.
        constexpr bool kFine = !(D == 64 && DROP && Mma<Tin>::kSplit);
        constexpr int kGroups = safe ? 13 : (kFine ? 17 : 9);
        // O += P(j-1) V(j-1) first: its fragments were read in the previous
        // step.  S(j+1) = Q K(j+1)^T after it, by when the K(j+1) fragments
        // read at the start of this step have landed.
        auto mfma = [&](int q) {
            if (q < NPVT) {
                const int qp = q < NPV ? q : q - NPV;
                const int c = qp / (2 * NDB), r2 = qp % (2 * NDB);
                const int db = r2 / 2, rb2 = r2 % 2;
                acc[rb2][db] = Mma<Tin>::run(vf[db][c], q < NPV ? p_prev[rb2][c] : p_lo[rb2][c],
                                             acc[rb2][db]);
            } else if (next) {
                // row blocks alternate: neighbouring products are independent
                const int qq = q - NPVT;
                const int rb2 = qq & 1, ks = qq >> 1;
                s_next[rb2] = Mma<Tin>::run(kf[ks], qf[rb2][ks],
                                            ks == 0 ? f32x16_t{} : s_next[rb2]);
            }
        };
        // V(j) for the next step's product, read into vf in the group after
        // the one that issues the last product reading vf
        constexpr int kGroupV = [] {
            int g = 0;
            while (NPVT > 0 && (g + 1) * NM / kGroups < NPVT) ++g;
            return NPVT > 0 ? g + 1 : 0;
        }();
        auto vread_at = [&](int gi) {
            if (gi == kGroupV) read_v(v_next);
        };
        // d = 64: the short form masks each part in the group that
        // exponentiates it (at d = 128 that made the compiler's register
        // allocation of the whole kernel worse: L8192 +17 %)
        constexpr bool kMaskParts = D == 64 && !safe && kFine;
        if constexpr (masked_tile && !kMaskParts) mask_cur(j);
        u32x4_t p_new[2][2];             // this tile's P; p_prev stays for PV
        u32x4_t p_lo_new[2][2];          // its low part (split only)
        // pack a pair of probabilities; with the split also their low parts
        auto pack_pair = [&](float x, float y, uint32_t& hi_out, uint32_t& lo_out) {
            hi_out = Mma<Tin>::pack(x, y);
            if constexpr (split)
                lo_out = Mma<Tin>::pack(x - Mma<Tin>::lo16(hi_out), y - Mma<Tin>::hi16(hi_out));
        };
        // The copy of tile dma_kt (NEXT only), one instruction every few
        // groups: a burst of copies from every wave at once fills the memory
        // pipeline's queue and stalls the waves behind it.
        auto dma_at = [&](int gi, const u32x4_t& rsrc) {
            if (next) {
#pragma unroll
                for (int t = 0; t < DPW; ++t)
                    if (gi == 3 + t * (kGroups - 4) / DPW) issue_part(rsrc, dma_stage, t);
            }
        };
        const auto rsrc = tile_rsrc(dma_kt);
        if constexpr (!safe) {
            // Part u (0..7) = scores 4 * (u & 3) .. +3 of row block u >> 2:
            // group 2u exponentiates and sums part u, group 2u + 1 rounds it
            // (9 groups: group g exponentiates part g and rounds part g - 1).
            // The row sums go straight into l (fp32) and, for bf16, lr.
            float pe[2][4];              // probabilities of the last two parts
            uint32_t dw[4];              // dropout words of the current part pair
#pragma unroll
            for (int gi = 0; gi < kGroups; ++gi) {
                vread_at(gi);
                // part of the exponentials in this group (-1: none), and
                // part of the packing (-1: none)
                const int ex = kFine ? ((gi & 1) == 0 && gi / 2 < 8 ? gi / 2 : -1)
                                     : (gi < 8 ? gi : -1);
                const int pk = kFine ? ((gi & 1) == 1 ? (gi - 1) / 2 : -1)
                                     : (gi >= 1 ? gi - 1 : -1);
                if (ex >= 0) {
                    const int rb = ex >> 2, e0 = 4 * (ex & 3);
                    if constexpr (masked_tile && kMaskParts) {
                        const int lim = last_key(rb) - (j * BN + 32 * kq + 4 * hi);
#pragma unroll
                        for (int e = e0; e < e0 + 4; ++e)
                            if (8 * (e >> 2) + (e & 3) > lim) s_cur[rb][e] = -__builtin_inff();
                    }
                    float* x = pe[ex & 1];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        x[i] = fast_exp2(fmaf(s_cur[rb][e0 + i], c2, nm[rb]));
                        pin(x[i]);       // computed in this group, not sunk
                    }
                    l[rb] += (x[0] + x[1]) + (x[2] + x[3]);
                    pin(l[rb]);
                }
                if (pk >= 0) {
                    const int u = pk, rb = u >> 2, c = (u >> 1) & 1, half = u & 1;
                    float (&x)[4] = pe[u & 1];
                    if constexpr (DROP) {
                        if ((u & 1) == 0) drop_words(j, rb, u & 3, dw);
                        if ((u & 1) == 0) drop_apply(dw[0], dw[1], x);
                        else drop_apply(dw[2], dw[3], x);
                    }
                    uint32_t a, d, alo = 0, dlo = 0;
                    pack_pair(x[0], x[1], a, alo);
                    pack_pair(x[2], x[3], d, dlo);
                    p_new[rb][c][2 * half] = a;
                    p_new[rb][c][2 * half + 1] = d;
                    pin(p_new[rb][c]);
                    if constexpr (split) {
                        p_lo_new[rb][c][2 * half] = alo;
                        p_lo_new[rb][c][2 * half + 1] = dlo;
                        pin(p_lo_new[rb][c]);
                    }
                    // the sums read the packed pairs where they now live
                    // (reading the pack results directly keeps a second copy)
                    if constexpr (Mma<Tin>::kNormRounded && !DROP) {
                        lr[rb] = Mma<Tin>::add_pair(p_new[rb][c][2 * half + 1],
                                                    Mma<Tin>::add_pair(p_new[rb][c][2 * half], lr[rb]));
                        if constexpr (split)
                            lr[rb] = Mma<Tin>::add_pair(
                                p_lo_new[rb][c][2 * half + 1],
                                Mma<Tin>::add_pair(p_lo_new[rb][c][2 * half], lr[rb]));
                        pin(lr[rb]);
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int q = gi * NM / kGroups; q < (gi + 1) * NM / kGroups; ++q) mfma(q);
                dma_at(gi, rsrc);
                __builtin_amdgcn_sched_barrier(0);
            }
            if (kGroupV >= kGroups) read_v(v_next);
        } else {
            float psum[2][4];
            float rsr[2][2];             // row sums of the rounded P, per chunk
            uint32_t dw[2][4];           // dropout words of each row block's part pair
            bool upd;                    // some reference moved (wave-uniform)
            float alpha[2] = {1.0f, 1.0f};
#pragma unroll
            for (int gi = 0; gi < kGroups; ++gi) {
                vread_at(gi);
                if (gi == 0) {
                    // lane maxima of both row blocks; rare reference update
                    float mt[2];
                    bool need[2];
#pragma unroll
                    for (int rb = 0; rb < 2; ++rb) {
                        const f32x16_t& x = s_cur[rb];
                        const float a0 = max2(max2(x[0], x[1]), x[2]);
                        const float a1 = max2(max2(x[3], x[4]), x[5]);
                        const float a2 = max2(max2(x[6], x[7]), x[8]);
                        const float a3 = max2(max2(x[9], x[10]), x[11]);
                        const float a4 = max2(max2(x[12], x[13]), x[14]);
                        mt[rb] = max2(max2(max2(a0, a1), a2),
                                      max2(max2(a3, a4), x[15])) * c2;
                        need[rb] = mt[rb] > m[rb] + kGap;
                    }
                    upd = __builtin_amdgcn_ballot_w64(need[0] || need[1]) != 0;
                    if (upd) {
                        asm volatile("");   // keep this a branch: rarely taken
#pragma unroll
                        for (int rb = 0; rb < 2; ++rb) {
                            const float mr = max2(mt[rb], partner(mt[rb]));
                            const bool grow = mr > m[rb] + kGap;
                            const float m_new = grow ? mr : m[rb];
                            alpha[rb] = grow ? fast_exp2(m[rb] - m_new) : 1.0f;
                            l[rb] *= alpha[rb];
                            lr[rb] *= alpha[rb];
                            m[rb] = m_new;
                            nm[rb] = m_new == -__builtin_inff() ? 0.0f : -m_new;
                        }
                    }
                } else if (gi < 9) {
                    // p = 2^(s*c2 - m) for 4 scores of row block gi & 1
                    const int rb = (gi - 1) & 1, e0 = 4 * ((gi - 1) >> 1);
                    float pe[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        pe[i] = fast_exp2(fmaf(s_cur[rb][e0 + i], c2, nm[rb]));
                        pin(pe[i]);
                        s_cur[rb][e0 + i] = pe[i];
                    }
                    psum[rb][(gi - 1) >> 1] = (pe[0] + pe[1]) + (pe[2] + pe[3]);
                    pin(psum[rb][(gi - 1) >> 1]);
                    if constexpr (DROP) {
                        const int g4 = (gi - 1) >> 1;
                        if ((g4 & 1) == 0) drop_words(j, rb, g4, dw[rb]);
                        if ((g4 & 1) == 0) drop_apply(dw[rb][0], dw[rb][1], pe);
                        else drop_apply(dw[rb][2], dw[rb][3], pe);
#pragma unroll
                        for (int i = 0; i < 4; ++i) s_cur[rb][e0 + i] = pe[i];
                    }
                } else {
                    // P^T operand of 16-key chunk c of row block rb
                    const int rb = (gi - 9) >> 1, c = (gi - 9) & 1;
                    float t0 = 0.0f, t1 = 0.0f;
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) {
                        const int e = 8 * c + 2 * jj;
                        uint32_t hv, lv = 0;
                        pack_pair(s_cur[rb][e], s_cur[rb][e + 1], hv, lv);
                        p_new[rb][c][jj] = hv;
                        if constexpr (split) p_lo_new[rb][c][jj] = lv;
                        if constexpr (Mma<Tin>::kNormRounded) {
                            float& t = (jj & 1) ? t1 : t0;
                            t = Mma<Tin>::add_pair(hv, t);
                            if constexpr (split) t = Mma<Tin>::add_pair(lv, t);
                        }
                    }
                    rsr[rb][c] = t0 + t1;
                    pin(p_new[rb][c]);
                    pin(rsr[rb][c]);
                    if constexpr (split) pin(p_lo_new[rb][c]);
                }
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int q = gi * NM / kGroups; q < (gi + 1) * NM / kGroups; ++q) mfma(q);
                dma_at(gi, rsrc);
                __builtin_amdgcn_sched_barrier(0);
            }
            if (kGroupV >= kGroups) read_v(v_next);
#pragma unroll
            for (int rb = 0; rb < 2; ++rb) {
                l[rb] += (psum[rb][0] + psum[rb][1]) + (psum[rb][2] + psum[rb][3]);
                if constexpr (Mma<Tin>::kNormRounded) lr[rb] += rsr[rb][0] + rsr[rb][1];
            }
            // the accumulators hold P(j-1) V(j-1), relative to the old
            // references, only once this step's products are in
            if (upd) {
                asm volatile("");   // keep this a branch: rarely taken
#pragma unroll
                for (int rb = 0; rb < 2; ++rb)
#pragma unroll
                    for (int db = 0; db < NDB; ++db) acc[rb][db] *= alpha[rb];
            }
        }
        // the step's results are produced here, not where they are used
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                pin(p_new[rb][c]);
                p_prev[rb][c] = p_new[rb][c];
                if constexpr (split) p_lo[rb][c] = p_lo_new[rb][c];
            }
    };

    // Stage of tile t, picked without a runtime index into the ring.
    auto stage_of = [&](int t) {
        const int sl = t % STAGES;
        lds16_t* x = ring<D, 0>();
        if (sl == 1) x = ring<D, 1>();
        if (sl == 2) x = ring<D, 2>();
        if (sl == 3) x = ring<D, 3>();
        if (sl == 4) x = ring<D, 4>();
        return x;
    };

    // Key tiles 0 .. n_full-1 need no mask for any row of the work-group:
    // they end inside the key range and, for causal inputs, at or before the
    // last key visible to the first row.
    int n_full = lk_b / BN;
    if (CAUSAL) {
        const int lim = row0 + diag + 1;
        n_full = min(n_full, lim > 0 ? lim / BN : 0);
    }

    // Step j (0 <= j <= n_kt - 2) works on tile j, which lives in stage
    // j % STAGES.  K of tile j+1 and V of tile j-1 are read here.  The stage
    // refilled here, (j + AHEAD) % STAGES = (j-2) % STAGES, was last read
    // (V of tile j-2) one step ago, and those fragments were consumed by
    // products of that step, so every wave is done with it once it reaches
    // this step's barrier.  Every step issues the copies of tile j + AHEAD
    // -- past the key range they read nothing -- so the wait at the top of a
    // step is the same constant count everywhere.
    //   steady: stage S = j % STAGES known at compile time (the loop below is
    //           unrolled by STAGES), no mask; FIRST (j == 0) has no
    //           P(j-1) V(j-1).
    //   masked: tiles at or past n_full (at most 3 per q-tile, at the end of
    //           its range) hold keys some row of the work-group must not
    //           see; stages picked at run time.  Keeping the mask out of the
    //           unrolled loop keeps the steady step's code as it is (with
    //           the mask in every step, the d = 128 step gained ~30 % more
    //           instructions, mostly copies between register files).
    auto steady = [&](int j, auto SI, auto FIRST, auto SAFE) {
        constexpr int S = decltype(SI)::value;
        constexpr bool first = decltype(FIRST)::value;
        // tile j+1 has landed once at most the copies issued after it
        // (tiles j+2 .. j+AHEAD-1) are pending
        wait_vm<(AHEAD - 2) * DPW>();
        __builtin_amdgcn_s_barrier();
        // fragment addresses are formed here each step, not kept live per
        // stage across the loop
        asm volatile("" : "+v"(k_off));
        asm volatile("" : "+v"(v_off));
        u32x4_t kf[NKS];
        read_k(ring<D, (S + 1) % STAGES>(), kf);
        f32x16_t s_new[2];
        compute(j, std::true_type(), std::integral_constant<bool, !first>(), std::false_type(),
                SAFE, kf, s_new, j + AHEAD, ring<D, (S + AHEAD) % STAGES>(), ring<D, S>());
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) s_cur[rb] = s_new[rb];
    };
    auto masked = [&](int j, auto SAFE) {
        wait_vm<(AHEAD - 2) * DPW>();
        __builtin_amdgcn_s_barrier();
        refresh_lane();
        asm volatile("" : "+v"(k_off));
        asm volatile("" : "+v"(v_off));
        u32x4_t kf[NKS];
        read_k(stage_of(j + 1), kf);
        f32x16_t s_new[2];               // (j = 0: P(j-1) = 0 and V = 0)
        compute(j, std::true_type(), std::true_type(), std::true_type(), SAFE, kf, s_new,
                j + AHEAD, stage_of(j + AHEAD), stage_of(j));
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) s_cur[rb] = s_new[rb];
    };

    // The key loop: prologue, steps, last tile.  The short form first; the
    // safe form only when the short form overflowed (see compute).
    auto run_keys = [&](auto SAFE, bool copies_issued) {
        if (n_kt > 0) {
            // prologue: copies of tile 0, Q and tile 1 in flight, then Q
            // and tile 0 landed; S(0)
            // (tile 2 only after the barrier: less traffic in flight while
            // every work-group waits for its first tile)
            if (!copies_issued) issue_first();
            static_assert(AHEAD == 3, "prologue copies");
            wait_vm<DPW>();              // tile 0 and Q in; tile 1 may be pending
            __builtin_amdgcn_s_barrier();
            issue_tile(2, ring<D, 2>());
            read_q();
            if (p.negate_q) {                // scale < 0: fold the sign into q
#pragma unroll
                for (int rb = 0; rb < 2; ++rb)
#pragma unroll
                    for (int ks = 0; ks < NKS; ++ks) qf[rb][ks] ^= 0x80008000u;
            }
            {
                u32x4_t kf[NKS];
                read_k(ring<D, 0>(), kf);
#pragma unroll
                for (int rb = 0; rb < 2; ++rb) {
                    s_cur[rb] = f32x16_t{};
#pragma unroll
                    for (int ks = 0; ks < NKS; ++ks)
                        s_cur[rb] = Mma<Tin>::run(kf[ks], qf[rb][ks], s_cur[rb]);
                }
            }
            // references from the first tile's row maxima (its masked scores
            // excluded); every step then takes the short form of the softmax
            if (n_full == 0) mask_cur(0);
#pragma unroll
            for (int rb = 0; rb < 2; ++rb) {
                const f32x16_t& x = s_cur[rb];
                const float a0 = max2(max2(x[0], x[1]), x[2]);
                const float a1 = max2(max2(x[3], x[4]), x[5]);
                const float a2 = max2(max2(x[6], x[7]), x[8]);
                const float a3 = max2(max2(x[9], x[10]), x[11]);
                const float a4 = max2(max2(x[12], x[13]), x[14]);
                const float mx = max2(max2(max2(a0, a1), a2), max2(max2(a3, a4), x[15]));
                m[rb] = max2(mx, partner(mx)) * c2;
                nm[rb] = m[rb] == -__builtin_inff() ? 0.0f : -m[rb];
            }
            static_assert(STAGES == 5, "unrolling below");
            // unmasked steps 0 .. n_un-1: step 0, then rounds of STAGES steps
            // starting at stage 1, then the remainder
            const int n_un = max(0, min(n_full, n_kt - 1));
            int j = 0;
            if (n_un >= 1) steady(j++, I0(), std::true_type(), SAFE);
            for (; j + STAGES <= n_un; j += STAGES) {
                steady(j, I1(), std::false_type(), SAFE);
                steady(j + 1, I2(), std::false_type(), SAFE);
                steady(j + 2, I3(), std::false_type(), SAFE);
                steady(j + 3, I4(), std::false_type(), SAFE);
                steady(j + 4, I0(), std::false_type(), SAFE);
            }
            // remaining unmasked steps (j < n_un), j % STAGES == 1 here
            if (j < n_un) {
                steady(j++, I1(), std::false_type(), SAFE);
                if (j < n_un) {
                    steady(j++, I2(), std::false_type(), SAFE);
                    if (j < n_un) {
                        steady(j++, I3(), std::false_type(), SAFE);
                        if (j < n_un) steady(j++, I4(), std::false_type(), SAFE);
                    }
                }
            }
            // masked steps up to n_kt - 2 (the low part of P is zero for
            // the unmasked tile before the first of them)
            if constexpr (Mma<Tin>::kSplit && !kSplitAll) clear_p_lo();
            for (; j <= n_kt - 2; ++j) masked(j, SAFE);
            // last tile jl: no copy in flight, no product S(jl+1); then its own PV
            {
                const int jl = n_kt - 1;
                wait_vm_lgkm0<0>();
                refresh_lane();
                asm volatile("" : "+v"(k_off));
                asm volatile("" : "+v"(v_off));
                u32x4_t kf_unused[NKS];
                f32x16_t s_unused[2];
                // vf holds V(jl-1) (zeros if jl = 0); compute reads V(jl)
                const lds16_t* cur = stage_of(jl);
                if (jl >= n_full) {
                    compute(jl, std::false_type(), std::true_type(), std::true_type(), SAFE,
                            kf_unused, s_unused, 0, ring<D, 0>(), cur);
                    pv_last(std::true_type());
                } else {
                    compute(jl, std::false_type(), std::true_type(), std::false_type(), SAFE,
                            kf_unused, s_unused, 0, ring<D, 0>(), cur);
                    pv_last(std::false_type());
                }
            }
        }
    };
    run_keys(std::false_type(), true);

    // Merge of the two waves that share a row half (key groups kq = 0, 1).
    // Wave kq finishes row block rb = kq of the half (all NDB column
    // blocks): it publishes in LDS only the other row block's accumulators
    // and (m, l, lr), relative to its own reference max, for its partner,
    // and takes its own share from registers:
    //   m = max(m_0, m_1),  x = x_0 2^(m_0 - m) + x_1 2^(m_1 - m).
    constexpr int SPS = L::SLOTS_PER_STAGE;
    static_assert(KQ == 2, "two key groups per row half");
    auto slot_acc = [&](int w) {
        lds16_t* base = ring<D, 0>();
        const int si = w / SPS;
        if (si == 1) base = ring<D, 1>();
        if (si == 2) base = ring<D, 2>();
        if (si == 3) base = ring<D, 3>();
        return reinterpret_cast<lds_f4_t*>(base) + (w % SPS) * (L::ACC / 4) * 64;
    };
    auto stat = [&](int w, int rb, int k) {
        return reinterpret_cast<lds_f32_t*>(ring<D, STAGES - 1>()) +
               ((w * 2 + rb) * 3 + k) * 64;
    };
    // overflow flag of wave w: a word near the end of the statistics' stage
    auto ovf_flag = [&](int w) {
        return reinterpret_cast<lds_f32_t*>(ring<D, STAGES - 1>()) + (L::STAGE / 2 - 2 - w);
    };
    static_assert(L::WAVES * 2 * 3 * 64 + L::WAVES + 1 <= L::STAGE / 2, "flags");
    // Every wave stores the partner's row block (accumulators and
    // statistics) and whether its short-form results left their range.
    auto publish = [&]() {
        __syncthreads();                 // every wave is done with the ring
        refresh_lane();
        lds_f4_t* a = slot_acc(wave);
        auto put = [&](auto RBc) {
            constexpr int rb = decltype(RBc)::value;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int gg = 0; gg < 4; ++gg)
                    a[((rb * NDB + db) * 4 + gg) * 64 + lane] =
                        f32x4_t{acc[rb][db][4 * gg], acc[rb][db][4 * gg + 1],
                                acc[rb][db][4 * gg + 2], acc[rb][db][4 * gg + 3]};
            stat(wave, rb, 0)[lane] = m[rb];
            stat(wave, rb, 1)[lane] = l[rb];
            stat(wave, rb, 2)[lane] = lr[rb];
        };
        if (kq == 0) put(I1());
        else put(I0());
        // In range: every lane's row sums below kLMax and every accumulator
        // below kAccMax in magnitude (a NaN fails both tests).  A fp16
        // probability past 65504 is inf in the P operand, which leaves an
        // inf or NaN accumulator; a long row of moderate probabilities may
        // pass 65504 in its fp32 sum without any single one overflowing.
        float amax = 0.0f;
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int i = 0; i < 16; ++i) amax = max2(amax, __builtin_fabsf(acc[rb][db][i]));
        const bool ok = l[0] < kLMax && l[1] < kLMax && amax < kAccMax;
        const bool bad = __builtin_amdgcn_ballot_w64(!ok) != 0;
        if (lane == 0) *ovf_flag(wave) = bad ? 1.0f : 0.0f;
        __syncthreads();
    };
    publish();
    bool redo = false;
#pragma unroll
    for (int w = 0; w < L::WAVES; ++w) redo |= *ovf_flag(w) != 0.0f;
    if (redo) {
        // some probability left its range: the q-tile again in the safe
        // form (the flags are read before the ring is refilled: the first
        // copy into their stage follows two barriers of the key loop)
        refresh_lane();
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
            m[rb] = -__builtin_inff();
            nm[rb] = 0.0f;
            l[rb] = 0.0f;
            lr[rb] = 0.0f;
#pragma unroll
            for (int db = 0; db < NDB; ++db) acc[rb][db] = f32x16_t{};
        }
#pragma unroll
        for (int c = 0; c < 2; ++c) {
#pragma unroll
            for (int rb = 0; rb < 2; ++rb) p_prev[rb][c] = u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
            for (int db = 0; db < NDB; ++db) vf[db][c] = u32x4_t{0u, 0u, 0u, 0u};
        }
        if constexpr (kSplitAll) clear_p_lo();
        run_keys(std::true_type(), false);
        publish();
    }

    // Merged result of one output block, relative to mu.
    struct Block {
        float mu, lf, lrf;
        f32x16_t o;
    };
    auto store = [&](const int bi, const Block& r) {
        const int rb = bi / NDB, db = bi % NDB;
        // O is normalised by the sum of the rounded P (bf16) or the fp32 sum
        // (fp16); LSE uses the fp32 sum.
        const float lt = r.lf + partner(r.lf);
        const float ln = Mma<Tin>::kNormRounded && !DROP ? r.lrf + partner(r.lrf) : lt;
        if (qrow(rb) < lq_b) {
            const float inv = ln > 0.0f ? 1.0f / ln : 0.0f;
            const int64_t orow = (packed ? 0 : (int64_t)b * p.o_sb) +
                                 (int64_t)h * p.o_sh +
                                 (int64_t)(q0 + qrow(rb)) * p.o_sr;
#pragma unroll
            for (int gg = 0; gg < 4; ++gg) {
                const int d0 = db * 32 + 8 * gg + 4 * hi;
                Epi<Tout>::store4(p.o, orow + d0, r.o[4 * gg] * inv,
                                  r.o[4 * gg + 1] * inv, r.o[4 * gg + 2] * inv,
                                  r.o[4 * gg + 3] * inv);
            }
            if (db == 0 && p.lse != nullptr && hi == 0) {
                const float lse = lt > 0.0f
                                      ? (r.mu + __log2f(lt)) * 0.69314718055994530942f
                                      : -__builtin_inff();
                const int64_t li =
                    packed ? (int64_t)h * (DROP ? p.cu_q[p.batch] : tq) + q0 + qrow(rb)
                           : ((int64_t)b * p.hq + h) * p.lq + qrow(rb);
                p.lse[li] = lse;
            }
        }
    };
    // Row block rb = kq: this wave's share from registers, the partner's
    // (key group 1 - kq) from LDS, summed key group 0 first.
    auto finish = [&](auto RBc) {
        constexpr int rb = decltype(RBc)::value;
        const int wp = rh + 2 * (1 - rb);    // the partner wave
        const float mp = stat(wp, rb, 0)[lane];
        const float mt = max2(m[rb], mp);
        const float mu = mt == -__builtin_inff() ? 0.0f : mt;
        const float fs = fast_exp2(m[rb] - mu), fp = fast_exp2(mp - mu);
        const float lp = stat(wp, rb, 1)[lane], lrp = stat(wp, rb, 2)[lane];
        // (self, partner) in key-group order
        const float f0 = rb == 0 ? fs : fp, f1 = rb == 0 ? fp : fs;
        const float l0 = rb == 0 ? l[rb] : lp, l1 = rb == 0 ? lp : l[rb];
        const float r0 = rb == 0 ? lr[rb] : lrp, r1 = rb == 0 ? lrp : lr[rb];
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
            Block r;
            r.mu = mu;
            r.lf = l0 * f0 + l1 * f1;
            r.lrf = r0 * f0 + r1 * f1;
            const lds_f4_t* a = slot_acc(wp) + ((rb * NDB + db) * 4) * 64 + lane;
#pragma unroll
            for (int gg = 0; gg < 4; ++gg) {
                const f32x4_t x = a[gg * 64];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float own = acc[rb][db][4 * gg + i];
                    const float x0 = rb == 0 ? own : x[i], x1 = rb == 0 ? x[i] : own;
                    r.o[4 * gg + i] = x0 * f0 + x1 * f1;
                }
            }
            store(rb * NDB + db, r);
        }
    };
    if (kq == 0) finish(I0());
    else finish(I1());
}

// Span of sequence b of a packed batch.
__device__ __forceinline__ SeqSpan packed_span(const FwdParams& p, int b) {
    const int q0 = p.cu_q[b], k0 = p.cu_k[b];
    return SeqSpan{q0, p.cu_q[b + 1] - q0, k0, p.cu_k[b + 1] - k0, 0};
}

// Work of a packed non-causal batch of at most 64 sequences, longest key
// range first.  Every q-tile of sequence i visits the same ck_i key tiles,
// so the (sequence, q-tile, head) items are ranked by ck_i, most first (ties
// by sequence index, then q-tile, then head), and the work-group of linear
// grid index r takes the item of rank r: the dispatcher, which hands out
// work-groups in grid order as slots free up, then works heaviest first.
// With two resident work-groups per CU, the second round of n_cu ranks is
// taken in reverse (lightest of them first), so the pair a CU holds sums to
// about the same work.  The lane of each sequence computes its rank and its
// first item; the whole work-group derives the same answer.  Returns false
// when the work-group has no item.
template <int WG_PER_CU>
__device__ __forceinline__ bool packed_item(const FwdParams& p, int& b, int& qtile, int& h,
                                            SeqSpan& span) {
    const int nb = p.batch;
    const int lane = lane_id();
    SeqSpan mine{0, 0, 0, 0, 0};
    if (lane < nb) mine = packed_span(p, lane);
    const int nq = (mine.lq + kBM - 1) / kBM;       // q-tiles of this lane's sequence
    const int ck = (mine.lk + 63) / 64;             // key tiles each of them visits
    int rank = 0;
    for (int j = 0; j < nb; ++j) {
        const int cj = __builtin_amdgcn_readlane(ck, j);
        rank += (cj > ck || (cj == ck && j < lane)) ? 1 : 0;
    }
    int first = 0, total = 0;                       // in q-tiles
    for (int j = 0; j < nb; ++j) {
        const int rj = __builtin_amdgcn_readlane(rank, j);
        const int nj = __builtin_amdgcn_readlane(nq, j);
        first += rj < rank ? nj : 0;
        total += nj;
    }
    const int heads = p.hq;
    const int n_items = total * heads;
    int r = ((int)blockIdx.z * (int)gridDim.y + (int)blockIdx.y) * (int)gridDim.x +
            (int)blockIdx.x;
    if (WG_PER_CU == 2) {
        const int lo = p.n_cu, hi2 = min(n_items, 2 * p.n_cu);
        if (r >= lo && r < hi2) r = lo + (hi2 - 1 - r);
    }
    if (r >= n_items) return false;
    const int it = r / heads;                       // q-tile rank
    h = r - it * heads;
    const uint64_t own = __builtin_amdgcn_ballot_w64(lane < nb && it >= first && it < first + nq);
    b = (int)__builtin_ctzll(own);
    qtile = it - __builtin_amdgcn_readlane(first, b);
    // all query rows: the end of the last sequence
    const int tq = __builtin_amdgcn_readlane(mine.q0 + mine.lq, nb - 1);
    span = SeqSpan{__builtin_amdgcn_readlane(mine.q0, b), __builtin_amdgcn_readlane(mine.lq, b),
                   __builtin_amdgcn_readlane(mine.k0, b), __builtin_amdgcn_readlane(mine.lk, b), tq};
    return true;
}

// Grid (x, y, z) = (query head, batch, item), dispatched x fastest, so that
// consecutive work-groups take the same item of different heads (the
// q-tiles of one head then share one XCD when the head count is a multiple
// of the XCD count).
//   non-causal: item = q-tile; packed batches of at most 64 sequences are
//     ranked by packed_item, larger ones take q-tile n-1-item.
//   causal: q-tiles heaviest first; with `pair` 1 item t covers q-tiles
//     n-1-t and t one after the other; with `pair` 2 the second round of
//     n_cu work-groups runs lightest first, so that the two work-groups a
//     CU holds (dispatched n_cu apart) sum to about the same work.
// Work-group modes: one q-tile, the causal pair (n-1-t, t), or resident
// work-groups looping over ranked q-tiles.
enum { kModeOne = 0, kModePairs = 1, kModeResident = 2 };

template <int D, typename Tin, typename Tout, bool CAUSAL, int MODE, bool DROP>
__global__ __launch_bounds__(Layout<D>::THREADS, Layout<D>::WG_PER_CU) void attn_fwd_mfma_kernel(
    FwdParams p, int n_qtiles, int pair) {
    // every argument the work-group reads, requested in one round trip
    asm volatile("" ::"s"(p.q), "s"(p.k), "s"(p.v), "s"(p.o), "s"(p.lse),
                 "s"(p.q_sh), "s"(p.k_sh), "s"(p.v_sh), "s"(p.q_sr), "s"(p.k_sr),
                 "s"(p.v_sr), "s"(p.o_sh), "s"(p.o_sr), "s"(p.lq), "s"(p.lk),
                 "s"(p.group_magic), "s"(p.scale_log2), "s"(n_qtiles), "s"(pair));
    int h = (int)blockIdx.x;
    int b = (int)blockIdx.y;
    const int item = (int)blockIdx.z;
    if constexpr (MODE == kModeOne) {
        // one q-tile per work-group: a straight-line body
        int it = item;
        // (d = 128 keeps the halves order below: this remap, even untaken,
        // changes the register allocation of its saturated kernel)
        if (D == 64 && CAUSAL && pair == 2) {
            // Causal order 2.  In grid order (head fastest, then batch, then
            // item) the work-groups rank heaviest first.  The first n_cu take
            // one slot on every CU; the dispatcher deals the next ones to
            // the second slots in the same CU order, so ranks lo .. hi-1 of
            // that round are taken in reverse -- lightest first -- and each
            // CU's pair sums to about the same work.  The reversal moves
            // blocks of 8 work-groups, which keeps every rank on the XCD
            // (grid index mod 8) of its own position.
            const uint32_t gx = gridDim.x, cols = gx * gridDim.y;
            const uint32_t lo = (uint32_t)p.n_cu;
            const uint32_t hi = min(cols * gridDim.z, 2u * lo);   // grid below 2^31 (launcher)
            const uint32_t blocks = hi > lo ? (hi - lo) >> 3 : 0u;
            const uint32_t r = (uint32_t)it * cols + (uint32_t)b * gx + (uint32_t)h;
            if (r >= lo && r - lo < 8u * blocks) {
                const uint32_t rr = lo + 8u * (blocks - 1u - ((r - lo) >> 3)) + ((r - lo) & 7u);
                it = (int)(rr / cols);
                const uint32_t col = rr - (uint32_t)it * cols;
                b = (int)(col / gx);
                h = (int)(col - (uint32_t)b * gx);
            }
        }
        int t = it;
        SeqSpan span{0, p.lq, 0, p.lk};
        // Grouped heads: the dispatcher deals consecutive work-groups to the
        // 8 XCDs in turn, so with hq a multiple of 8 the work-group of grid
        // column x runs on XCD x % 8.  Taking head (x % 8) * (hq / 8) + x / 8
        // puts hq / 8 consecutive heads -- whole kv groups when the group
        // size divides hq / 8 -- on one XCD, where they share its L2 for K
        // and V.
        if (p.hq > p.hkv && (p.hq & 7) == 0) h = (h & 7) * (p.hq >> 3) + (h >> 3);
        if (p.cu_q != nullptr) {
            if (!CAUSAL && p.batch <= 64) {
                if (!packed_item<Layout<D>::WG_PER_CU>(p, b, t, h, span)) return;
            } else {
                // highest q-tile index first: those q-tiles exist only for
                // the longest sequences, whose work-groups are the heaviest
                t = n_qtiles - 1 - it;
                span = packed_span(p, b);
                span.tq = p.cu_q[p.batch];
            }
        }
        if (CAUSAL) {
            if constexpr (D == 64) {
                t = n_qtiles - 1 - it;
            } else {
                // order 2 at d = 128: the first half of the items heaviest
                // first, the second half lightest first
                t = pair == 2 ? (item < n_qtiles / 2 ? n_qtiles - 1 - item : item - n_qtiles / 2)
                              : n_qtiles - 1 - item;
            }
        }
        attend_qtile<D, Tin, Tout, CAUSAL, DROP>(p, t, h, b, span);
    } else if constexpr (MODE == kModePairs) {
        // causal, q-tiles n-1-item and item one after the other
        int tile[2] = {n_qtiles - 1 - item, -1};
        if (item < tile[0]) tile[1] = item;
        for (int it = 0; it < 2 && tile[it] >= 0; ++it) {
            if (it > 0) __syncthreads();     // the LDS stages are reused
            // head and batch made opaque here: what the q-tile derives from
            // them is computed inside the iteration, not hoisted out of the
            // loop and kept live (spilled) across the whole key loop
            int hh = __builtin_amdgcn_readfirstlane(h), bb = __builtin_amdgcn_readfirstlane(b);
            asm volatile("" : "+s"(hh), "+s"(bb));
            SeqSpan span = SeqSpan{0, p.lq, 0, p.lk, 0};
            if (p.cu_q != nullptr) {
                span = packed_span(p, bb);
                span.tq = p.cu_q[p.batch];
            }
            attend_qtile<D, Tin, Tout, CAUSAL, DROP>(p, tile[it], hh, bb, span);
        }
    } else {
        // Resident work-groups (dense input, a 1-D grid of one work-group per
        // resident slot): the B * Hq * n q-tiles are ranked heaviest first
        // (causal: q-tile index descending, then batch and head; otherwise
        // any order), and in round k work-group w takes rank k * G + w for
        // even k and k * G + G - 1 - w for odd k, so the rounds' heavy and
        // light q-tiles pair up and every work-group gets about the same
        // key tiles in all.
        const int G = (int)gridDim.x, w = (int)blockIdx.x;
        const int bh = p.batch * p.hq;
        const int n_items = bh * n_qtiles;
        for (int k = 0; k * G < n_items; ++k) {
            const int r = k * G + ((k & 1) ? G - 1 - w : w);
            if (r >= n_items) break;
            const int qi = r / bh, hb = r - qi * bh;
            const int t = CAUSAL ? n_qtiles - 1 - qi : qi;
            if (k > 0) __syncthreads();  // the LDS stages are reused
            int hh = __builtin_amdgcn_readfirstlane(hb % p.hq);
            int bb = __builtin_amdgcn_readfirstlane(hb / p.hq);
            asm volatile("" : "+s"(hh), "+s"(bb));
            attend_qtile<D, Tin, Tout, CAUSAL, DROP>(p, t, hh, bb, SeqSpan{0, p.lq, 0, p.lk, 0});
        }
    }
}

template <int D, typename Tin, typename Tout, bool DROP>
hipError_t launch_typed(const FwdParams& p, hipStream_t stream) {
    const int n_qtiles = (p.lq + kBM - 1) / kBM;
    // causal q-tile order: with two resident work-groups per CU and a grid
    // that the device holds at once, heaviest first with the second round
    // of n_cu reversed (2: the CU's pair sums to about the same work); with
    // a larger grid or one work-group per CU, heaviest first (0: the
    // dispatcher then balances as slots free up; measured 5 % faster at
    // B4 H32 N1024, and 1 % faster than q-tile pairs at d = 128)
    const int64_t n_wg = (int64_t)p.hq * p.batch * n_qtiles;
    int pair = !p.causal ? 0
               : p.causal_pairs >= 0 ? p.causal_pairs
               : (Layout<D>::WG_PER_CU == 2 && n_wg <= 2 * (int64_t)p.n_cu ? 2 : 0);
    if (pair == 2 && n_wg >= (int64_t)1 << 31) pair = 0;   // order 2 ranks in 32 bits
    const int items = (p.causal && pair == 1) ? (n_qtiles + 1) / 2 : n_qtiles;
    // grid limits (y and z below 2^16) are checked by the caller
    const dim3 grid((unsigned)p.hq, (unsigned)p.batch, (unsigned)items);
    // resident work-groups (order 3): d = 128, dense input, no dropout
    if constexpr (D == 128 && !DROP) {
        if (p.causal_pairs == 3 && p.cu_q == nullptr) {
            const int64_t n_items = (int64_t)p.batch * p.hq * n_qtiles;
            const int slots = p.n_cu * Layout<D>::WG_PER_CU;
            const dim3 g1((unsigned)std::min<int64_t>(n_items, slots));
            if (p.causal)
                hipLaunchKernelGGL((attn_fwd_mfma_kernel<D, Tin, Tout, true, kModeResident, false>),
                                   g1, dim3(Layout<D>::THREADS), 0, stream, p, n_qtiles, 0);
            else
                hipLaunchKernelGGL((attn_fwd_mfma_kernel<D, Tin, Tout, false, kModeResident, false>),
                                   g1, dim3(Layout<D>::THREADS), 0, stream, p, n_qtiles, 0);
            return hipGetLastError();
        }
    }
    // (the dropout kernels have no q-tile-pair variant: the caller asks for
    // order 1 only through mi_attn_fwd_select, which has no dropout)
    if (!DROP && p.causal && pair == 1)
        hipLaunchKernelGGL((attn_fwd_mfma_kernel<D, Tin, Tout, true, DROP ? kModeOne : kModePairs, DROP>), grid,
                           dim3(Layout<D>::THREADS), 0, stream, p, n_qtiles, pair);
    else if (p.causal)
        hipLaunchKernelGGL((attn_fwd_mfma_kernel<D, Tin, Tout, true, kModeOne, DROP>), grid,
                           dim3(Layout<D>::THREADS), 0, stream, p, n_qtiles, pair);
    else
        hipLaunchKernelGGL((attn_fwd_mfma_kernel<D, Tin, Tout, false, kModeOne, DROP>), grid,
                           dim3(Layout<D>::THREADS), 0, stream, p, n_qtiles, 0);
    return hipGetLastError();
}

template <int D, bool DROP>
hipError_t launch_d(const FwdParams& p, int in_dtype, int out_dtype,
                    hipStream_t stream) {
    if (in_dtype == 0) {
        return out_dtype == 2 ? launch_typed<D, f16_t, float, DROP>(p, stream)
                              : launch_typed<D, f16_t, f16_t, DROP>(p, stream);
    }
    return out_dtype == 2 ? launch_typed<D, bf16_t, float, DROP>(p, stream)
                          : launch_typed<D, bf16_t, bf16_t, DROP>(p, stream);
}

}  // namespace
}  // namespace mi_attn
