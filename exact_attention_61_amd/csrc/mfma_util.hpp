// Building blocks shared by libmi_attn's gfx950 MFMA kernels: operand types,
// the 32x32x16 f16/bf16 matrix product with its rounding rules for P, lane
// helpers, LDS access types, wait-count helpers and output stores.
#pragma once
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


template <typename T> struct Mma;

// P is rounded to the input type for the PV product; the log-sum-exp always
// uses the fp32 sum of the unrounded probabilities.  (A sum of the rounded
// fp16 values, one v_dot2 per pair, would take half the instructions, but
// its error is not bounded for long rows: a probability in the fp16
// subnormal range keeps only an absolute precision of 2^-25, and many such
// terms rounding alike can move the sum by more than the LSE tolerance.)
//
// fp16 keeps 11 significant bits: O is normalised by the same fp32 sum, and
// the rounding of P moves the product by at most 2^-11 relative.
//
// bf16 keeps 8, too coarse on its own in two situations.  (1) One key
// dominates a row from a tile after the first: its probability, rounded,
// would carry ~2^-9 relative error into O.  O is therefore normalised by the
// sum of the probabilities as rounded (kNormRounded, one v_dot2 per pair),
// so the rounding of a dominant probability cancels between numerator and
// denominator.  (2) A row sees only a few keys: then each rounded
// probability moves O by up to ~2^-9 of a value, on top of the output's own
// bf16 rounding.  Every row with fewer than BN visible keys has all of them
// in the masked tiles at the end of its range, so on those tiles (and only
// there) bf16 splits P into hi = bf16(p) and lo = bf16(p - hi) and runs the
// PV product twice (kSplit); hi + lo carries 16 significant bits.
template <> struct Mma<f16_t> {
    __device__ __forceinline__ static f32x16_t run(u32x4_t a, u32x4_t b,
                                                   f32x16_t c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(
            __builtin_bit_cast(half8_t, a), __builtin_bit_cast(half8_t, b), c,
            0, 0, 0);
    }
    static constexpr bool kSplit = false;
    static constexpr bool kNormRounded = false;
    __device__ __forceinline__ static float add_pair(uint32_t pr, float c) {
        const half2_t one = {(_Float16)1.0f, (_Float16)1.0f};
        return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, pr), one, c, false);
    }
    // two fp32 -> packed 16-bit, round to nearest even (v_cvt_pk_f16_f32)
    __device__ __forceinline__ static uint32_t pack(float x, float y) {
        half2_t r;
        r[0] = (_Float16)x;
        r[1] = (_Float16)y;
        return __builtin_bit_cast(uint32_t, r);
    }
    __device__ __forceinline__ static float lo16(uint32_t p) {
        return (float)__builtin_bit_cast(_Float16, (uint16_t)p);
    }
    __device__ __forceinline__ static float hi16(uint32_t p) {
        return (float)__builtin_bit_cast(_Float16, (uint16_t)(p >> 16));
    }
};
template <> struct Mma<bf16_t> {
    __device__ __forceinline__ static f32x16_t run(u32x4_t a, u32x4_t b,
                                                   f32x16_t c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            __builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
            c, 0, 0, 0);
    }
    static constexpr bool kSplit = true;
    static constexpr bool kNormRounded = true;
    // c + the two packed bf16 values (exact products with 1, fp32 sum)
    __device__ __forceinline__ static float add_pair(uint32_t pr, float c) {
        const bf16x2_t one = {(__bf16)1.0f, (__bf16)1.0f};
        return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pr), one, c, false);
    }
    // v_cvt_pk_bf16_f32, round to nearest even
    __device__ __forceinline__ static uint32_t pack(float x, float y) {
        bf16x2_t r;
        r[0] = (__bf16)x;
        r[1] = (__bf16)y;
        return __builtin_bit_cast(uint32_t, r);
    }
    // the two packed bf16 values back in fp32 (exact: bf16 is the upper
    // half of an fp32)
    __device__ __forceinline__ static float lo16(uint32_t p) {
        return __builtin_bit_cast(float, p << 16);
    }
    __device__ __forceinline__ static float hi16(uint32_t p) {
        return __builtin_bit_cast(float, p & 0xffff0000u);
    }
};
// Largest per-lane row sum the short form accepts, and the largest
// accumulator magnitude; past either the q-tile is redone in the safe form.
// Row sums below 2^100 keep every probability far from the top of the bf16
// and fp32 ranges, and accumulators below 2^126 keep the merge of two key
// halves (a sum of two terms, each scaled by at most 1) finite.
constexpr float kLMax = 1.2676506e30f;    // 2^100
constexpr float kAccMax = 8.507059e37f;   // 2^126

// Lane index 0..63 from the execution mask (all lanes active), computed anew
// at every call: the asm is volatile, so the optimiser neither merges two
// calls nor keeps one result alive across a loop.
__device__ __forceinline__ int lane_id() {
    int x;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(x));
    return x;
}

// Value of x held by lane l ^ 32.
__device__ __forceinline__ float partner(float x) {
    const uint32_t u = __builtin_bit_cast(uint32_t, x);
    auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    const uint32_t y = (lane_id() & 32) ? r[0] : r[1];
    return __builtin_bit_cast(float, y);
}

__device__ __forceinline__ float fast_exp2(float x) {
    return __builtin_amdgcn_exp2f(x);   // v_exp_f32; 2^-inf = 0
}

// IEEE maximum (v_maximum3_f32 when nested); no NaN canonicalisation.
__device__ __forceinline__ float max2(float a, float b) {
    return __builtin_elementwise_maximum(a, b);
}

// Pointers into LDS keep their address space through selects and phis.
typedef __attribute__((address_space(3))) uint16_t lds16_t;
typedef __attribute__((address_space(3))) const u32x4_t lds_u32x4_t;
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) f32x4_t lds_f4_t;
typedef __attribute__((address_space(3))) float lds_f32_t;

__device__ __forceinline__ s16x4_t lds_read_tr(const lds16_t* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4_t*)(p));
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

}  // namespace
}  // namespace mi_attn
