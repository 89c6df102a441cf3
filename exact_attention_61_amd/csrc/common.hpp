// Shared definitions of libmi_attn's kernels and host launcher (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mi_attn {

// Everything a forward kernel needs, passed by value as the kernel argument.
// Offsets are in elements.  For packed variable-length input the batch
// strides are unused and row r of sequence b lives at row cu[b] + r.
struct FwdParams {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    float* lse;                 // may be null
    const int32_t* cu_q;        // null for dense input
    const int32_t* cu_k;
    int64_t q_sb, q_sh, q_sr;
    int64_t k_sb, k_sh, k_sr;
    int64_t v_sb, v_sh, v_sr;
    int64_t o_sb, o_sh, o_sr;
    uint64_t group_magic;            // ceil(2^32 / (hq / hkv)): kv head of query
                                     // head h = (h * group_magic) >> 32
    int32_t batch, hq, hkv;
    int32_t lq, lk;                  // dense lengths, or the packed maxima
    float scale_log2;                // |scale| * log2(e), in fp32
    int32_t negate_q;                // 1 when scale < 0 (fold the sign into q)
    int32_t causal;
    int32_t causal_pairs;            // causal q-tile order (0, 1, 2; -1 default)
    int32_t n_cu;                    // compute units of the device
    // dropout on P (the dropout kernels only): a key is kept iff its 16-bit
    // half of a Philox word is at least drop_threshold = floor(p * 2^16);
    // kept probabilities are multiplied by drop_scale = 1 / (1 - p)
    uint32_t drop_threshold;
    float drop_scale;
    uint32_t seed_lo, seed_hi;       // the Philox key
};

// Parameters of the decode kernel (attn_decode.hip): a few query rows per
// sequence against a long key/value cache, split along the keys.  Offsets
// are in elements; tensors are dense [B, H, L, d] views through strides.
struct DecParams {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    float* lse;                      // may be null
    const int32_t* seqlens_k;        // per-sequence key counts (<= lk), or null
    int64_t q_sb, q_sh, q_sr;
    int64_t k_sb, k_sh, k_sr;
    int64_t v_sb, v_sh, v_sr;
    int64_t o_sb, o_sh, o_sr;
    int32_t batch, hq, hkv, lq, lk;
    int32_t group;                   // hq / hkv query heads per kv head
    int32_t hpg;                     // query heads per work-group (hpg * lq <= 32)
    int32_t nqg;                     // query groups per kv head, ceil(group / hpg)
    int32_t splits;                  // key splits per query group
    int32_t chunk;                   // keys per split, a multiple of 128
    float scale_log2;                // |scale| * log2(e)
    int32_t negate_q;                // 1 when scale < 0
    int32_t causal;                  // bottom-right: j <= i + Lk_b - Lq
    float* part_o;                   // [B, Hq, Lq, splits, d] partial outputs
    float* part_ml;                  // [B, Hq, Lq, splits, 2] (m in log2, l)
};

// Parameters of the rotary-embedding kernel (rotary.hip).  x is rotated in
// place; row t of sequence b sits at position offset + offsets[b] + t.
// Pair k (k < rotary_dim / 2) turns by position * freq_pi[k] half-turns
// (freq_pi[k] = base^(-2k / rotary_dim) / pi, computed in double on the host).
struct RopeParams {
    void* x;
    void* x2;                        // a second tensor (K) with the same rows, or null
    const int32_t* cu_seqlens;       // packed x [T, H, d], or null (dense)
    const int32_t* offsets;          // per-sequence position offsets, or null
    int64_t sb, sh, sr;              // element strides (batch unused when packed)
    int64_t sb2, sh2, sr2;           // those of x2
    int32_t batch, heads, seqlen;    // seqlen: rows per sequence (packed: the maximum)
    int32_t heads2;                  // heads of x2 (0 without it)
    int32_t rotary_dim;              // a multiple of 16, <= head dim
    int32_t interleaved;             // 0: pairs (k, k + rd/2); 1: pairs (2k, 2k + 1)
    int64_t offset;
    double freq_pi[128];
};

// Storage tags for the element types (16-bit values are kept as raw bits).
struct f16_t { uint16_t bits; };
struct bf16_t { uint16_t bits; };

__device__ __forceinline__ float to_f32(f16_t x) {
    return (float)__builtin_bit_cast(_Float16, x.bits);
}
__device__ __forceinline__ float to_f32(bf16_t x) {
    return __builtin_bit_cast(float, (uint32_t)x.bits << 16);
}
__device__ __forceinline__ float to_f32(float x) { return x; }

// fp32 -> fp16, round to nearest even (v_cvt_f16_f32).
__device__ __forceinline__ uint16_t f32_to_f16_bits(float x) {
    return __builtin_bit_cast(uint16_t, (_Float16)x);
}

// fp32 -> bf16, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
    uint32_t u = __builtin_bit_cast(uint32_t, x);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

template <typename T> struct OutStore;
template <> struct OutStore<f16_t> {
    __device__ __forceinline__ static void put(void* base, int64_t i, float x) {
        reinterpret_cast<uint16_t*>(base)[i] = f32_to_f16_bits(x);
    }
};
template <> struct OutStore<bf16_t> {
    __device__ __forceinline__ static void put(void* base, int64_t i, float x) {
        reinterpret_cast<uint16_t*>(base)[i] = f32_to_bf16_bits(x);
    }
};
template <> struct OutStore<float> {
    __device__ __forceinline__ static void put(void* base, int64_t i, float x) {
        reinterpret_cast<float*>(base)[i] = x;
    }
};

// Host-side launchers, one per kernel family.  They only launch: every
// argument was validated by the caller.  Return the hipGetLastError() code.
hipError_t launch_simple(const FwdParams& p, int in_dtype, int out_dtype,
                         int head_dim, hipStream_t stream);
hipError_t launch_mfma_d64(const FwdParams& p, int in_dtype, int out_dtype,
                          hipStream_t stream);
hipError_t launch_mfma_d128(const FwdParams& p, int in_dtype, int out_dtype,
                           hipStream_t stream);
hipError_t launch_mfma_drop_d64(const FwdParams& p, int in_dtype, int out_dtype,
                                hipStream_t stream);
hipError_t launch_mfma_drop_d128(const FwdParams& p, int in_dtype, int out_dtype,
                                 hipStream_t stream);
hipError_t launch_decode(const DecParams& p, int in_dtype, int out_dtype, int head_dim,
                         hipStream_t stream);
hipError_t launch_rotary(const RopeParams& p, int dtype, hipStream_t stream);

}  // namespace mi_attn
