// MFMA attention forward for gfx950 (CDNA4): the library's hot path.
//
// Method.  Standard attention S = QK^T * scale, P = softmax(S), O = PV,
// computed tile by tile so that S and P never leave the registers, with the
// online-softmax statistics of "FlashAttention: turning the quadratic
// intermediate matrices into statistics" (section 3.1): per query row a
// running max m, the exp-sum l relative to m and the output accumulator
// relative to m; when m grows, l and the accumulator are multiplied by
// alpha = 2^(m_old - m_new).  Exponentials are base 2 with the scale and
// log2(e) folded into one fp32 factor applied to the fp32 scores (the inputs
// are never pre-scaled in 16-bit), and l sums the fp32 probabilities.
//
// Work decomposition.  One work-group of 4 waves owns BM = 128 query rows of
// one (batch, head); each wave owns 32 rows.  The key loop walks BN = 64 keys
// at a time; K and V tiles are staged in LDS, double buffered (the global
// loads of tile j+1 are in flight while tile j is computed).
//
// Transposed products.  The wave computes S^T = K Q^T and O^T = V^T P^T with
// v_mfma_f32_32x32x16_{f16,bf16}.  In the 32x32 result layout lane l holds
// column l % 32, i.e. one query row, so every lane owns all of its row's
// scores (shared with lane l ^ 32): row maxima and sums are lane-local plus
// one v_permlane32_swap, the rescale by alpha needs no data movement, and the
// S^T accumulator already has the lane layout of the P^T operand of the
// second product (the contraction order over keys is permuted consistently
// on both operands).  V stays row-major in LDS; the V^T operand is read with
// ds_read_b64_tr_b16, which transposes 16-bit data within 16-lane groups.
//
// Causal masking is bottom-right aligned (key j visible to row i iff
// j <= i + Lk - Lq): key tiles wholly above the diagonal are never loaded,
// waves whose rows see none of a tile skip its arithmetic, and the per-key
// mask is applied only on tiles that straddle the diagonal or the key tail.
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

constexpr int kBM = 128;    // query rows per work-group
constexpr int kBN = 64;     // keys per iteration
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;

template <typename T> struct Mma;
template <> struct Mma<f16_t> {
    __device__ __forceinline__ static f32x16_t run(u32x4_t a, u32x4_t b,
                                                   f32x16_t c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(
            __builtin_bit_cast(half8_t, a), __builtin_bit_cast(half8_t, b), c,
            0, 0, 0);
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
    __device__ __forceinline__ static f32x16_t run(u32x4_t a, u32x4_t b,
                                                   f32x16_t c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            __builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
            c, 0, 0, 0);
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
    return __builtin_amdgcn_exp2f(x);   // v_exp_f32; exp2(-inf) = 0
}

__device__ __forceinline__ s16x4_t lds_read_tr(const uint16_t* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4_t*)(p));
}

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

template <int D, typename Tin, typename Tout, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 2) void attn_fwd_mfma_kernel(
    FwdParams p, int n_qtiles) {
    constexpr int RS = D + 8;            // LDS row stride (halves), padded
    constexpr int KCH = D / 8;           // 16-byte chunks per row
    constexpr int LOADS = kBN * KCH / kThreads;   // chunks per thread per tile
    constexpr int NKB = kBN / 32;        // 32-key blocks per tile
    constexpr int NKC = kBN / 16;        // 16-key chunks per tile
    constexpr int NKS = D / 16;          // k-steps of the QK^T product
    constexpr int NDB = D / 32;          // 32-column blocks of O^T
    static_assert(kBN * KCH % kThreads == 0, "tile load must split evenly");

    __shared__ __attribute__((aligned(16))) uint16_t lds_k[2][kBN * RS];
    __shared__ __attribute__((aligned(16))) uint16_t lds_v[2][kBN * RS];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int hi = lane >> 5;            // which half of the wave
    const int col = lane & 31;           // the query row this lane owns

    // Heavy-first order: consecutive work-groups take the same q-tile index
    // of different (batch, head) pairs, starting from the last (for causal,
    // the most expensive) q-tile.
    const int bh_count = p.hq * p.batch;
    const int qt_i = (int)blockIdx.x / bh_count;
    const int bh = (int)blockIdx.x - qt_i * bh_count;
    const int h = bh % p.hq;
    const int b = bh / p.hq;
    const int qtile = CAUSAL ? (n_qtiles - 1 - qt_i) : qt_i;

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

    // Key tiles this work-group needs.
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

    // Staging of K/V tiles: thread chunk c = tid + kThreads*i is row c / KCH,
    // columns (c % KCH) * 8 .. +7.
    u32x4_t kst[LOADS], vst[LOADS];
    auto load_tile = [&](int kt) {
#pragma unroll
        for (int i = 0; i < LOADS; ++i) {
            const int c = tid + kThreads * i;
            const int r = c / KCH;
            const int cc = (c % KCH) * 8;
            const int key = kt * kBN + r;
            u32x4_t kx = {0u, 0u, 0u, 0u}, vx = {0u, 0u, 0u, 0u};
            if (key < lk_b) {
                kx = *reinterpret_cast<const u32x4_t*>(kg + (int64_t)key * p.k_sr + cc);
                vx = *reinterpret_cast<const u32x4_t*>(vg + (int64_t)key * p.v_sr + cc);
            }
            kst[i] = kx;
            vst[i] = vx;
        }
    };
    auto store_tile = [&](int buf) {
#pragma unroll
        for (int i = 0; i < LOADS; ++i) {
            const int c = tid + kThreads * i;
            const int r = c / KCH;
            const int cc = (c % KCH) * 8;
            *reinterpret_cast<u32x4_t*>(&lds_k[buf][r * RS + cc]) = kst[i];
            *reinterpret_cast<u32x4_t*>(&lds_v[buf][r * RS + cc]) = vst[i];
        }
    };

    const float c2 = p.scale_log2;       // |scale| * log2(e)
    float m = -__builtin_inff();         // running max, log2 domain
    float l = 0.0f;                      // this lane's half of the exp-sum
    f32x16_t acc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) acc[db] = f32x16_t{};

    if (n_kt > 0) {
        load_tile(0);
        store_tile(0);
    }
    __syncthreads();

    // Last key this wave's rows can see (causal) and whether it has rows.
    const bool wave_has_rows = wrow0 < lq_b;
    const int wave_last_key = CAUSAL ? wrow0 + 31 + diag : lk_b - 1;
    const int my_last_key = CAUSAL ? min(lk_b - 1, qrow + diag) : lk_b - 1;

    for (int kt = 0; kt < n_kt; ++kt) {
        const int buf = kt & 1;
        const bool more = kt + 1 < n_kt;
        if (more) load_tile(kt + 1);

        const int kstart = kt * kBN;
        if (wave_has_rows && kstart <= wave_last_key) {
            const uint16_t* kl = lds_k[buf];
            const uint16_t* vl = lds_v[buf];

            // S^T = K Q^T for the tile: s[kb][4*gg + r] is key
            // kb*32 + 8*gg + 4*hi + r of row `col`.
            f32x16_t s[NKB];
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
                s[kb] = f32x16_t{};
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks) {
                    const u32x4_t a = *reinterpret_cast<const u32x4_t*>(
                        kl + (kb * 32 + col) * RS + ks * 16 + 8 * hi);
                    s[kb] = Mma<Tin>::run(a, qf[ks], s[kb]);
                }
            }

            // Mask keys past the sequence end or above the diagonal.
            const bool need_mask =
                (kstart + kBN > lk_b) ||
                (CAUSAL && kstart + kBN - 1 > wrow0 + diag);
            if (need_mask) {
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        const int key =
                            kstart + kb * 32 + 8 * (e >> 2) + 4 * hi + (e & 3);
                        if (key > my_last_key) s[kb][e] = -__builtin_inff();
                    }
            }

            // Row max over the tile (lane-local, then with lane ^ 32).
            float mx = s[0][0];
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[kb][e]);
            mx = fmaxf(mx, partner(mx));
            const float m_new = fmaxf(m, mx * c2);
            const float m_use = m_new == -__builtin_inff() ? 0.0f : m_new;
            const float alpha = fast_exp2(m - m_use);
            m = m_new;

            // p = 2^(s*c2 - m) in fp32; l sums the fp32 values.
            float rs = 0.0f;
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const float pe = fast_exp2(fmaf(s[kb][e], c2, -m_use));
                    s[kb][e] = pe;
                    rs += pe;
                }
            l = fmaf(l, alpha, rs);
#pragma unroll
            for (int db = 0; db < NDB; ++db) acc[db] *= alpha;

            // P^T operand for each 16-key chunk: elements 8*(kc&1) .. +7 of
            // s[kc/2], rounded to the input type.
            u32x4_t pf[NKC];
#pragma unroll
            for (int kc = 0; kc < NKC; ++kc) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int e = 8 * (kc & 1) + 2 * j;
                    pf[kc][j] = Mma<Tin>::pack(s[kc >> 1][e], s[kc >> 1][e + 1]);
                }
            }

            // O^T += V^T P^T.  The V^T operand of chunk kc, block db: two
            // transposing reads covering keys kc*16 + 8*r + 4*hi + 0..3.
            const int lg = lane & 15;
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
#pragma unroll
                for (int kc = 0; kc < NKC; ++kc) {
                    const uint16_t* base =
                        vl + (kc * 16 + 4 * hi + (lg >> 2)) * RS + db * 32 +
                        16 * ((lane >> 4) & 1) + 4 * (lg & 3);
                    const s16x4_t lo = lds_read_tr(base);
                    const s16x4_t up = lds_read_tr(base + 8 * RS);
                    u32x4_t a;
                    a[0] = __builtin_bit_cast(uint32_t, (short __attribute__((ext_vector_type(2)))){lo[0], lo[1]});
                    a[1] = __builtin_bit_cast(uint32_t, (short __attribute__((ext_vector_type(2)))){lo[2], lo[3]});
                    a[2] = __builtin_bit_cast(uint32_t, (short __attribute__((ext_vector_type(2)))){up[0], up[1]});
                    a[3] = __builtin_bit_cast(uint32_t, (short __attribute__((ext_vector_type(2)))){up[2], up[3]});
                    acc[db] = Mma<Tin>::run(a, pf[kc], acc[db]);
                }
            }
        }

        if (more) store_tile(buf ^ 1);
        __syncthreads();
    }

    // Epilogue: O = acc / l, LSE = ln(2) * (m + log2 l).
    const float lt = l + partner(l);
    if (!row_ok) return;
    const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
    const int64_t orow = (packed ? 0 : (int64_t)b * p.o_sb) + (int64_t)h * p.o_sh +
                         (int64_t)(q0 + qrow) * p.o_sr;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int gg = 0; gg < 4; ++gg) {
            const int d0 = db * 32 + 8 * gg + 4 * hi;
            Epi<Tout>::store4(p.o, orow + d0, acc[db][4 * gg] * inv,
                              acc[db][4 * gg + 1] * inv, acc[db][4 * gg + 2] * inv,
                              acc[db][4 * gg + 3] * inv);
        }
    if (p.lse != nullptr && hi == 0) {
        const float lse = lt > 0.0f ? (m + __log2f(lt)) * 0.69314718055994530942f
                                    : -__builtin_inff();
        const int64_t li = packed ? (int64_t)h * p.cu_q[p.batch] + q0 + qrow
                                  : ((int64_t)b * p.hq + h) * p.lq + qrow;
        p.lse[li] = lse;
    }
}

template <int D, typename Tin, typename Tout>
hipError_t launch_typed(const FwdParams& p, hipStream_t stream) {
    const int n_qtiles = (p.lq + kBM - 1) / kBM;
    const int64_t blocks = (int64_t)n_qtiles * p.hq * p.batch;
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    if (p.causal)
        hipLaunchKernelGGL((attn_fwd_mfma_kernel<D, Tin, Tout, true>),
                           dim3((unsigned)blocks), dim3(kThreads), 0, stream, p,
                           n_qtiles);
    else
        hipLaunchKernelGGL((attn_fwd_mfma_kernel<D, Tin, Tout, false>),
                           dim3((unsigned)blocks), dim3(kThreads), 0, stream, p,
                           n_qtiles);
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
