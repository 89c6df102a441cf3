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
// never pre-scaled in 16-bit), and l sums the fp32 probabilities.
//
// The reference max is only replaced when a tile's max exceeds it by more
// than a gap of 8 (log2 units), and the rescale is skipped when no row of the
// wave needs it.  Any reference value gives the same O = u / l and LSE =
// m + log2 l; probabilities stay below 2^8, far inside every range, and the
// rescale of the accumulator is skipped on almost every tile.  The output is
// normalised by the sum of the probabilities as rounded for the PV product
// (one v_dot2 per pair), so that the rounding of a dominant probability
// cancels between numerator and denominator.  The log-sum-exp uses that sum
// for fp16 inputs (2^-11 relative at most) and an fp32 sum for bf16 inputs.
//
// Work decomposition.  A work-group of 4 waves owns BM = 128 query rows of one
// (batch, head) at a time; each wave owns 32 rows and walks the keys in tiles
// of BN = 64.  K and V tiles go from global memory straight into LDS
// (buffer_load_dwordx4 ... lds) through a ring of 5 stages, 3 tiles ahead of
// use, with one barrier per tile.  The stages are separate LDS arrays and the
// loop is unrolled by 5, so the compiler can see that a fragment read never
// touches a stage a copy is still landing in.
//
// Software pipeline.  Step j of a wave interleaves, in one instruction
// stream, the matrix products of two neighbouring tiles with the vector work
// of the tile between them: S(j+1) = Q K(j+1)^T and O += P(j-1) V(j-1) on the
// matrix cores while the softmax of S(j) runs on the vector ALUs.  Both
// engines are busy at once within each wave.
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
// the diagonal or the key tail.  For causal inputs a work-group may process
// q-tiles t and n-1-t one after the other, so that every work-group does the
// same amount of work.
#include <type_traits>

#include "common.hpp"

namespace mi_attn {
namespace {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kBM = 128;     // query rows per q-tile (4 waves of 32)
constexpr int kBN = 64;      // keys per tile
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kStages = 5;   // LDS ring of K/V tiles
constexpr int kAhead = 3;    // copies in flight: tiles j+1 .. j+kAhead at step j

template <typename T> struct Mma;
template <> struct Mma<f16_t> {
    static constexpr float kGap = 8.0f;   // reference-max lag allowed (log2)
    __device__ __forceinline__ static f32x16_t run(u32x4_t a, u32x4_t b,
                                                   f32x16_t c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(
            __builtin_bit_cast(half8_t, a), __builtin_bit_cast(half8_t, b), c,
            0, 0, 0);
    }
    // The row sum is taken over the rounded P (v_dot2_f32_f16 with ones):
    // fp16 rounding moves it by at most 2^-11 relative, i.e. the log-sum-exp
    // by at most 4.9e-4, and the output normalisation matches the product.
    static constexpr bool kFp32Sum = false;
    __device__ __forceinline__ static float add_pair(uint32_t pr, float c) {
        const half2_t one = {(_Float16)1.0f, (_Float16)1.0f};
        return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, pr), one, c,
                                      false);
    }
    // two fp32 -> packed 16-bit, round to nearest even (v_cvt_pk_f16_f32)
    __device__ __forceinline__ static uint32_t pack(float x, float y) {
        half2_t r;
        r[0] = (_Float16)x;
        r[1] = (_Float16)y;
        return __builtin_bit_cast(uint32_t, r);
    }
};
template <> struct Mma<bf16_t> {
    static constexpr float kGap = 8.0f;
    __device__ __forceinline__ static f32x16_t run(u32x4_t a, u32x4_t b,
                                                   f32x16_t c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            __builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
            c, 0, 0, 0);
    }
    // bf16 rounding is too coarse for the log-sum-exp: it uses an fp32 sum,
    // the output normalisation the sum of the rounded P.
    static constexpr bool kFp32Sum = true;
    // c + the two packed bf16 values (exact products with 1, fp32 sum)
    __device__ __forceinline__ static float add_pair(uint32_t pr, float c) {
        const bf16x2_t one = {(__bf16)1.0f, (__bf16)1.0f};
        return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pr),
                                               one, c, false);
    }
    // v_cvt_pk_bf16_f32, round to nearest even
    __device__ __forceinline__ static uint32_t pack(float x, float y) {
        bf16x2_t r;
        r[0] = (__bf16)x;
        r[1] = (__bf16)y;
        return __builtin_bit_cast(uint32_t, r);
    }
};

// Value of x held by lane l ^ 32.
__device__ __forceinline__ float partner(float x) {
    const uint32_t u = __builtin_bit_cast(uint32_t, x);
    auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    const uint32_t y = (threadIdx.x & 32) ? r[0] : r[1];
    return __builtin_bit_cast(float, y);
}

__device__ __forceinline__ float fast_exp2(float x) {
    return __builtin_amdgcn_exp2f(x);   // v_exp_f32; 2^-inf = 0
}

// IEEE maximum (v_maximum3_f32 when nested); no NaN canonicalisation.
__device__ __forceinline__ float max2(float a, float b) {
    return __builtin_elementwise_maximum(a, b);
}

__device__ __forceinline__ s16x4_t lds_read_tr(const uint16_t* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4_t*)(p));
}

// 16 bytes per lane from global memory into LDS at base + 16 * lane
// (base uniform over the wave).
__device__ __forceinline__ void dma16(const void* src, uint16_t* lds_base) {
    __builtin_amdgcn_global_load_lds(
        src, (__attribute__((address_space(3))) void*)(lds_base), 16, 0, 0);
}

// s_waitcnt with vmcnt <= V and lgkmcnt == 0 (gfx9 encoding: vmcnt in bits
// 3:0 and 15:14, expcnt 6:4 left at its maximum, lgkmcnt 11:8).
template <int V>
__device__ __forceinline__ void wait_vm_lgkm0() {
    static_assert(V >= 0 && V < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((V & 15) | (7 << 4) | ((V >> 4) << 14));
}
// s_waitcnt with vmcnt <= V only (expcnt and lgkmcnt at their maxima).
template <int V>
__device__ __forceinline__ void wait_vm() {
    static_assert(V >= 0 && V < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((V & 15) | (7 << 4) | (15 << 8) | ((V >> 4) << 14));
}

// Empty asm that reads and redefines x: the value must be computed before
// this point, so no optimisation sinks its computation into a later step.
__device__ __forceinline__ void pin(float& x) { asm volatile("" : "+v"(x)); }
__device__ __forceinline__ void pin(u32x4_t& x) { asm volatile("" : "+v"(x)); }

template <typename Tout> struct Epi;
template <> struct Epi<f16_t> {
    __device__ __forceinline__ static void store4(void* o, int64_t i, float a,
                                                  float b, float c, float d) {
        u32x2_t v;
        v[0] = Mma<f16_t>::pack(a, b);
        v[1] = Mma<f16_t>::pack(c, d);
        *reinterpret_cast<u32x2_t*>(reinterpret_cast<uint16_t*>(o) + i) = v;
    }
};
template <> struct Epi<bf16_t> {
    __device__ __forceinline__ static void store4(void* o, int64_t i, float a,
                                                  float b, float c, float d) {
        u32x2_t v;
        v[0] = Mma<bf16_t>::pack(a, b);
        v[1] = Mma<bf16_t>::pack(c, d);
        *reinterpret_cast<u32x2_t*>(reinterpret_cast<uint16_t*>(o) + i) = v;
    }
};
template <> struct Epi<float> {
    __device__ __forceinline__ static void store4(void* o, int64_t i, float a,
                                                  float b, float c, float d) {
        float4 v = {a, b, c, d};
        *reinterpret_cast<float4*>(reinterpret_cast<float*>(o) + i) = v;
    }
};

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
    static constexpr int NKB = kBN / 32;     // 32-key blocks per tile
    static constexpr int NKC = kBN / 16;     // 16-key chunks per tile
    static constexpr int NKS = D / 16;       // k-steps of QK^T
    static constexpr int NDB = D / 32;       // 32-column blocks of O^T
    static constexpr int ELEMS = kBN * D;    // per tile and tensor
    static constexpr int BLOCKS = ELEMS / 512;   // 1 KiB DMA blocks per tensor
    static constexpr int STAGE = 2 * ELEMS;  // K + V
    static constexpr int DPW = 2 * BLOCKS / kWaves;   // DMA blocks per wave
};

template <int D>
struct Stages {
    uint16_t* s[kStages];
};

template <int D, typename Tin, typename Tout, bool CAUSAL>
__device__ __forceinline__ void attend_qtile(const FwdParams& p, int qtile,
                                             int h, int b, const Stages<D>& st) {
    using L = Layout<D>;
    constexpr int NKB = L::NKB, NKC = L::NKC, NKS = L::NKS, NDB = L::NDB;
    constexpr int DPW = L::DPW;
    static_assert(2 * L::BLOCKS % kWaves == 0, "blocks per wave");

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // scalar
    const int hi = lane >> 5;            // which half of the wave
    const int col = lane & 31;           // the query row this lane owns

    int q0 = 0, lq_b = p.lq, k0 = 0, lk_b = p.lk;
    const bool packed = p.cu_q != nullptr;
    if (packed) {
        q0 = p.cu_q[b];
        lq_b = p.cu_q[b + 1] - q0;
        k0 = p.cu_k[b];
        lk_b = p.cu_k[b + 1] - k0;
    }
    const int row0 = qtile * kBM;
    if (row0 >= lq_b) return;            // uniform over the work-group
    const int g = h / p.group;
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

    // Key tiles this q-tile needs.
    int kend = lk_b;
    if (CAUSAL) kend = min(kend, row0 + kBM + diag);
    const int n_kt = kend > 0 ? (kend + kBN - 1) / kBN : 0;

    // Q fragment (B operand of S^T = K Q^T): lane holds row `col`, columns
    // ks*16 + 8*hi .. +7.
    const int wrow0 = row0 + 32 * wave;  // first row of this wave
    const int qrow = wrow0 + col;        // this lane's row (sequence-local)
    const bool row_ok = qrow < lq_b;
    u32x4_t qf[NKS];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
        u32x4_t x = {0u, 0u, 0u, 0u};
        if (row_ok)
            x = *reinterpret_cast<const u32x4_t*>(
                qg + (int64_t)(32 * wave + col) * p.q_sr + ks * 16 + 8 * hi);
        if (p.negate_q) x ^= 0x80008000u;   // scale < 0: fold the sign into q
        qf[ks] = x;
    }

    // DMA plan of this lane: which block of a tile it fills and the byte
    // offset, from the tile's first row, of the 16 bytes it copies.  Copies
    // go through a buffer resource whose range ends with the sequence, so
    // rows past the key range read as zeros (their scores are masked anyway).
    uint32_t dma_voff[DPW];
    int dma_dst[DPW];
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
    auto issue_tile = [&](int kt, uint16_t* stage) {
        const int rows = min(lk_b - kt * kBN, kBN);
        const auto rsrc = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(dma_base + (int64_t)kt * kBN * dma_sr), (short)0,
            (int)(rows * dma_sr * 2), 0x00020000);
#pragma unroll
        for (int t = 0; t < DPW; ++t)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rsrc, (__attribute__((address_space(3))) void*)(stage + dma_dst[t]),
                16, dma_voff[t], 0, 0, 0);
    };

    const float c2 = p.scale_log2;       // |scale| * log2(e)
    float m = -__builtin_inff();         // reference max, log2 domain
    float l = 0.0f;                      // this lane's half of the exp-sum
    float lr = 0.0f;                     // same over the rounded P
    f32x16_t acc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) acc[db] = f32x16_t{};
    const int my_last_key = CAUSAL ? min(lk_b - 1, qrow + diag) : lk_b - 1;

    // Pipeline registers: scores of the current tile, probabilities and V
    // fragments of the previous tile.
    f32x16_t s_cur[NKB];
    u32x4_t p_prev[NKC];
    u32x4_t vf[NDB][NKC];
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) p_prev[kc] = u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc) vf[db][kc] = u32x4_t{0u, 0u, 0u, 0u};

    auto read_k = [&](const uint16_t* stage, u32x4_t (&kf)[NKB][NKS]) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks)
                kf[kb][ks] = *reinterpret_cast<const u32x4_t*>(
                    stage + (kb * NKS + ks) * 512 + lane * 8);
    };
    auto read_v = [&](const uint16_t* stage) {
        const uint16_t* vl = stage + L::ELEMS;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int kc = 0; kc < NKC; ++kc) {
                const uint16_t* vb = vl + (db * NKC + kc) * 512 + lane * 4;
                const u32x2_t a = __builtin_bit_cast(u32x2_t, lds_read_tr(vb));
                const u32x2_t c = __builtin_bit_cast(u32x2_t, lds_read_tr(vb + 256));
                vf[db][kc] = u32x4_t{a[0], a[1], c[0], c[1]};
            }
    };
    auto mask_cur = [&](int kt) {
        const int kstart = kt * kBN;
        const bool need_mask = (kstart + kBN > lk_b) ||
                               (CAUSAL && kstart + kBN - 1 > wrow0 + diag);
        if (need_mask) {
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int key =
                        kstart + kb * 32 + 8 * (e >> 2) + 4 * hi + (e & 3);
                    if (key > my_last_key) s_cur[kb][e] = -__builtin_inff();
                }
        }
    };
    auto pv_prev = [&]() {
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc)
#pragma unroll
            for (int db = 0; db < NDB; ++db)
                acc[db] = Mma<Tin>::run(vf[db][kc], p_prev[kc], acc[db]);
    };

    // One pipeline step for tile j (its scores are in s_cur).  The softmax
    // of tile j is cut into kGroups groups of vector instructions; the
    // matrix products of the step (first O += P(j-1) V(j-1), whose operands
    // are ready, then with NEXT S(j+1) = Q K(j+1)^T, whose K fragments were
    // just requested) are spread between the groups.  Scheduling barriers
    // keep this order, so the wave issues a product and then vector work
    // while the matrix core runs it.
    auto compute = [&](int j, auto NEXT, const u32x4_t (&kf_next)[NKB][NKS],
                       f32x16_t (&s_next)[NKB]) {
        constexpr bool next = decltype(NEXT)::value;
        constexpr int NPV = NDB * NKC;
        constexpr int NQK = next ? NKB * NKS : 0;
        constexpr int NM = NPV + NQK;
        constexpr int kGroups = 18;
        static_assert(NKB == 2, "groups below assume 64-key tiles");
        mask_cur(j);
        float mxg[4];
        float m_new = m, m_use = 0.0f;
        bool grow = false;
        float psum[8];
        float rs = 0.0f;
        float rsr = 0.0f;     // row sum of the rounded P
        u32x4_t p_new[NKC];   // this tile's P; p_prev stays for the products
#pragma unroll
        for (int gi = 0; gi < kGroups; ++gi) {
            if (gi < 4) {
                // partial max over 8 scores
                const int kb = gi >> 1, e0 = 8 * (gi & 1);
                float x = max2(s_cur[kb][e0], s_cur[kb][e0 + 1]);
#pragma unroll
                for (int e = e0 + 2; e < e0 + 8; e += 2)
                    x = max2(x, max2(s_cur[kb][e], s_cur[kb][e + 1]));
                mxg[gi] = x;
            } else if (gi == 4) {
                // tile max of the row (with lane ^ 32), reference update
                float mx = max2(max2(mxg[0], mxg[1]), max2(mxg[2], mxg[3]));
                mx = max2(mx, partner(mx));
                const float mt = mx * c2;
                grow = mt > m + Mma<Tin>::kGap;      // false if all -inf
                m_new = grow ? mt : m;
                m_use = m_new == -__builtin_inff() ? 0.0f : m_new;
            } else if (gi < 13) {
                // p = 2^(s*c2 - m) for 4 scores, fp32
                const int e4 = gi - 5;               // 0..7
                const int kb = e4 >> 2, e0 = 4 * (e4 & 3);
                float pe[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    pe[i] = fast_exp2(fmaf(s_cur[kb][e0 + i], c2, -m_use));
                    s_cur[kb][e0 + i] = pe[i];
                }
                if (Mma<Tin>::kFp32Sum)
                    psum[e4] = (pe[0] + pe[1]) + (pe[2] + pe[3]);
            } else if (gi == 13) {
                if (Mma<Tin>::kFp32Sum)
                    rs = ((psum[0] + psum[1]) + (psum[2] + psum[3])) +
                         ((psum[4] + psum[5]) + (psum[6] + psum[7]));
            } else {
                // P^T operand of 16-key chunk kc: elements 8*(kc&1) .. +7 of
                // s_cur[kc/2], rounded to the input type
                const int kc = gi - 14;
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const int e = 8 * (kc & 1) + 2 * jj;
                    p_new[kc][jj] =
                        Mma<Tin>::pack(s_cur[kc >> 1][e], s_cur[kc >> 1][e + 1]);
                    rsr = Mma<Tin>::add_pair(p_new[kc][jj], rsr);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int q = gi * NM / kGroups; q < (gi + 1) * NM / kGroups; ++q) {
                if (q < NPV) {
                    const int kc = q / NDB, db = q % NDB;
                    acc[db] = Mma<Tin>::run(vf[db][kc], p_prev[kc], acc[db]);
                } else if (next) {
                    const int qq = q - NPV;
                    const int ks = qq / NKB, kb = qq % NKB;
                    s_next[kb] = Mma<Tin>::run(kf_next[kb][ks], qf[ks],
                                               ks == 0 ? f32x16_t{} : s_next[kb]);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        // the step's results are produced here, not where they are used
#pragma unroll
        for (int kc = 0; kc < NKC; ++kc) {
            pin(p_new[kc]);
            p_prev[kc] = p_new[kc];
        }
        if (Mma<Tin>::kFp32Sum) pin(rs);
        pin(rsr);
        pin(m_new);
        // rescale the accumulator (after the previous tile's product) when
        // the reference max moved for some row of the wave
        if (__builtin_amdgcn_ballot_w64(grow) != 0) {
            asm volatile("");   // keep this a branch: it is rarely taken
            const float alpha = grow ? fast_exp2(m - m_new) : 1.0f;
            l *= alpha;
            lr *= alpha;
#pragma unroll
            for (int db = 0; db < NDB; ++db) acc[db] *= alpha;
        }
        m = m_new;
        l += rs;
        lr += rsr;
    };

    // Steady step j (0 <= j < n_kt - 1) on stage S = j % kStages: wait for
    // tile j+1, refill stage (j+3) % kStages = (j-2) % kStages with tile j+3,
    // then compute.  Tile t always lives in stage t % kStages.  The refilled
    // stage was last read (V of tile j-2) at the end of step j-2 and those
    // values were consumed by products of step j-1, so every wave is done
    // with it once it reaches this step's barrier: no LDS wait is needed.
    auto steady = [&](int j, auto SI) {
        constexpr int S = decltype(SI)::value;
        // tile j+1 has landed once at most the copies of tile j+2 are pending
        if (j + 2 < n_kt) wait_vm<DPW>();
        else wait_vm<0>();
        __builtin_amdgcn_s_barrier();
        if (j + kAhead < n_kt)
            issue_tile(j + kAhead, st.s[(S + kAhead) % kStages]);
        u32x4_t kf[NKB][NKS];
        read_k(st.s[(S + 1) % kStages], kf);
        f32x16_t s_next[NKB];
        compute(j, std::integral_constant<bool, true>(), kf, s_next);
        read_v(st.s[S]);
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) s_cur[kb] = s_next[kb];
    };
    // Last step j = n_kt - 1 on stage S: no next tile, no barrier needed.
    auto last = [&](int j, auto SI) {
        constexpr int S = decltype(SI)::value;
        wait_vm_lgkm0<0>();
        u32x4_t kf_unused[NKB][NKS];
        f32x16_t s_unused[NKB];
        compute(j, std::integral_constant<bool, false>(), kf_unused, s_unused);
        read_v(st.s[S]);
        pv_prev();
    };
    static_assert(kStages == 5 && kAhead == 3, "unrolling below");

    if (n_kt > 0) {
        // prologue: tiles 0 .. kAhead-1 in flight, wait for tile 0
#pragma unroll
        for (int t = 0; t < kAhead; ++t)
            if (t < n_kt) issue_tile(t, st.s[t]);
        if (n_kt >= 3) wait_vm<2 * DPW>();
        else if (n_kt == 2) wait_vm<DPW>();
        else wait_vm<0>();
        __builtin_amdgcn_s_barrier();
        {
            u32x4_t kf[NKB][NKS];
            read_k(st.s[0], kf);
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) s_cur[kb] = f32x16_t{};
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb)
                    s_cur[kb] = Mma<Tin>::run(kf[kb][ks], qf[ks], s_cur[kb]);
        }
        using I0 = std::integral_constant<int, 0>;
        using I1 = std::integral_constant<int, 1>;
        using I2 = std::integral_constant<int, 2>;
        using I3 = std::integral_constant<int, 3>;
        using I4 = std::integral_constant<int, 4>;
        int j = 0;
        for (; j + kStages <= n_kt - 1; j += kStages) {
            steady(j, I0());
            steady(j + 1, I1());
            steady(j + 2, I2());
            steady(j + 3, I3());
            steady(j + 4, I4());
        }
        // remaining steady steps, then the last step (stage j % kStages)
        if (j < n_kt - 1) {
            steady(j++, I0());
            if (j < n_kt - 1) {
                steady(j++, I1());
                if (j < n_kt - 1) {
                    steady(j++, I2());
                    if (j < n_kt - 1) steady(j++, I3());
                }
            }
        }
        switch (j % kStages) {
            case 0: last(j, I0()); break;
            case 1: last(j, I1()); break;
            case 2: last(j, I2()); break;
            case 3: last(j, I3()); break;
            default: last(j, I4()); break;
        }
    }

    // Epilogue: O = acc / l, LSE = ln(2) * (m + log2 l).
    // O is normalised by the sum of the rounded P, LSE uses the fp32 sum
    // where there is one.
    const float ln = lr + partner(lr);
    const float lt = Mma<Tin>::kFp32Sum ? l + partner(l) : ln;
    if (row_ok) {
        const float inv = ln > 0.0f ? 1.0f / ln : 0.0f;
        const int64_t orow = (packed ? 0 : (int64_t)b * p.o_sb) +
                             (int64_t)h * p.o_sh + (int64_t)(q0 + qrow) * p.o_sr;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int gg = 0; gg < 4; ++gg) {
                const int d0 = db * 32 + 8 * gg + 4 * hi;
                Epi<Tout>::store4(p.o, orow + d0, acc[db][4 * gg] * inv,
                                  acc[db][4 * gg + 1] * inv,
                                  acc[db][4 * gg + 2] * inv,
                                  acc[db][4 * gg + 3] * inv);
            }
        if (p.lse != nullptr && hi == 0) {
            const float lse = lt > 0.0f
                                  ? (m + __log2f(lt)) * 0.69314718055994530942f
                                  : -__builtin_inff();
            const int64_t li = packed ? (int64_t)h * p.cu_q[p.batch] + q0 + qrow
                                      : ((int64_t)b * p.hq + h) * p.lq + qrow;
            p.lse[li] = lse;
        }
    }
}

// Grid: blockIdx.x = item * (hq * batch) + (batch, head) index, so that
// consecutive work-groups take the same item of different heads.  Items are
// q-tiles, heaviest first for causal inputs.  With `pair` (causal only) item t
// covers q-tiles n-1-t and t, which together see n+1 key tiles; the middle
// tile of an odd count runs alone.
template <int D, typename Tin, typename Tout, bool CAUSAL>
__global__ __launch_bounds__(kThreads, D == 64 ? 2 : 1) void attn_fwd_mfma_kernel(
    FwdParams p, int n_qtiles, int pair) {
    __shared__ __attribute__((aligned(16))) uint16_t st0[Layout<D>::STAGE];
    __shared__ __attribute__((aligned(16))) uint16_t st1[Layout<D>::STAGE];
    __shared__ __attribute__((aligned(16))) uint16_t st2[Layout<D>::STAGE];
    __shared__ __attribute__((aligned(16))) uint16_t st3[Layout<D>::STAGE];
    __shared__ __attribute__((aligned(16))) uint16_t st4[Layout<D>::STAGE];
    const Stages<D> st{{st0, st1, st2, st3, st4}};
    const int bh_count = p.hq * p.batch;
    const int item = (int)blockIdx.x / bh_count;
    const int bh = (int)blockIdx.x - item * bh_count;
    const int h = bh % p.hq;
    const int b = bh / p.hq;
    if (CAUSAL && pair == 2) {
        // first half of the grid heaviest-first, second half lightest-first:
        // work-groups i and i + grid/2, which the dispatcher tends to place on
        // the same CU, then see n+1 key tiles together
        const int half = n_qtiles / 2;
        const int qtile = item < half ? n_qtiles - 1 - item : item - half;
        attend_qtile<D, Tin, Tout, CAUSAL>(p, qtile, h, b, st);
    } else if (CAUSAL) {
        const int hi_tile = n_qtiles - 1 - item;
        attend_qtile<D, Tin, Tout, CAUSAL>(p, hi_tile, h, b, st);
        if (pair && item < hi_tile) {
            __syncthreads();             // the LDS stages are reused
            attend_qtile<D, Tin, Tout, CAUSAL>(p, item, h, b, st);
        }
    } else {
        attend_qtile<D, Tin, Tout, CAUSAL>(p, item, h, b, st);
    }
}

template <int D, typename Tin, typename Tout>
hipError_t launch_typed(const FwdParams& p, hipStream_t stream) {
    const int n_qtiles = (p.lq + kBM - 1) / kBM;
    const int pair = p.causal ? p.causal_pairs : 0;
    const int items = pair == 1 ? (n_qtiles + 1) / 2 : n_qtiles;
    const int64_t blocks = (int64_t)items * p.hq * p.batch;
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    if (p.causal)
        hipLaunchKernelGGL((attn_fwd_mfma_kernel<D, Tin, Tout, true>),
                           dim3((unsigned)blocks), dim3(kThreads), 0, stream, p,
                           n_qtiles, pair);
    else
        hipLaunchKernelGGL((attn_fwd_mfma_kernel<D, Tin, Tout, false>),
                           dim3((unsigned)blocks), dim3(kThreads), 0, stream, p,
                           n_qtiles, 0);
    return hipGetLastError();
}

template <int D>
hipError_t launch_d(const FwdParams& p, int in_dtype, int out_dtype,
                    hipStream_t stream) {
    if (in_dtype == 0) {
        return out_dtype == 2 ? launch_typed<D, f16_t, float>(p, stream)
                              : launch_typed<D, f16_t, f16_t>(p, stream);
    }
    return out_dtype == 2 ? launch_typed<D, bf16_t, float>(p, stream)
                          : launch_typed<D, bf16_t, bf16_t>(p, stream);
}

}  // namespace

hipError_t launch_mfma(const FwdParams& p, int in_dtype, int out_dtype,
                       int head_dim, hipStream_t stream) {
    return head_dim == 64 ? launch_d<64>(p, in_dtype, out_dtype, stream)
                          : launch_d<128>(p, in_dtype, out_dtype, stream);
}

}  // namespace mi_attn
