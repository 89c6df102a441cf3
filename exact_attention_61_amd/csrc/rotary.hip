// Rotary position embedding, in place, for gfx950.
//
// The "Training integration" tutorial (section 4) applies the rotary
// embedding to Q and K before attention: a rotary dimension, a base
// frequency, the GPT-NeoX layout (feature k pairs with k + rd/2) or the GPT-J
// layout (2k with 2k + 1), and, with a KV cache (section 4.3), positions that
// start at the cache length.  Pair k of a row at position p is turned by the
// angle p * base^(-2k/rd): (x, y) -> (x cos a - y sin a, x sin a + y cos a);
// features past rd are left as they are.
//
// The pass is bound by HBM traffic (each rotated element read and written
// once).  A thread owns 8 pairs of one position in 4 heads (grid z picks
// the heads; with a second tensor, Q then K, both in one launch): it issues
// the 16-byte loads of its pairs, forms the 8 angles while they are in
// flight -- in double, reduced to [0, 2) half-turns before the
// single-precision sine and cosine, so positions in the millions keep full
// accuracy -- and rotates the pairs.  (Non-temporal loads and stores were
// measured: faster on a 40 MiB Q+K rotated again and again, slower on
// 160 MiB; plain ones are kept.)
#include "common.hpp"

namespace mi_attn {
namespace {

constexpr int kRopeThreads = 256;
constexpr int kRopeHeadBatch = 4;

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

template <typename T> struct Elem;
template <> struct Elem<f16_t> {
    __device__ __forceinline__ static float get(uint32_t w, int hi) {
        return (float)__builtin_bit_cast(_Float16, (uint16_t)(hi ? w >> 16 : w & 0xffffu));
    }
    __device__ __forceinline__ static uint32_t put(float a, float b) {
        return (uint32_t)f32_to_f16_bits(a) | ((uint32_t)f32_to_f16_bits(b) << 16);
    }
};
template <> struct Elem<bf16_t> {
    __device__ __forceinline__ static float get(uint32_t w, int hi) {
        return __builtin_bit_cast(float, hi ? (w & 0xffff0000u) : (w << 16));
    }
    __device__ __forceinline__ static uint32_t put(float a, float b) {
        return (uint32_t)f32_to_bf16_bits(a) | ((uint32_t)f32_to_bf16_bits(b) << 16);
    }
};

// element e (0..7) of a 16-byte chunk
template <typename T>
__device__ __forceinline__ float chunk_elem(const u32x4_t& c, int e) {
    return Elem<T>::get(c[e >> 1], e & 1);
}

template <typename T, bool INTERLEAVED>
__global__ __launch_bounds__(kRopeThreads) void rotary_kernel(RopeParams p) {
    const int units = p.rotary_dim / 16;             // threads per row position
    const int64_t u = (int64_t)blockIdx.x * kRopeThreads + threadIdx.x;
    const int b = (int)blockIdx.y;
    const int64_t t = u / units;
    const int c = (int)(u - t * units);              // pairs 8c .. 8c + 7
    int64_t row0 = 0;                                // first row of the sequence
    int len = p.seqlen;
    if (p.cu_seqlens != nullptr) {
        row0 = p.cu_seqlens[b];
        len = p.cu_seqlens[b + 1] - (int)row0;
    }
    if (t >= len) return;
    const int64_t pos = p.offset + (p.offsets != nullptr ? p.offsets[b] : 0) + t;

    // grid z: the head groups of x, then those of x2
    const int zx = (p.heads + kRopeHeadBatch - 1) / kRopeHeadBatch;
    const bool second = (int)blockIdx.z >= zx;
    const int h0 = ((int)blockIdx.z - (second ? zx : 0)) * kRopeHeadBatch;
    const int heads = second ? p.heads2 : p.heads;
    const int64_t sb = second ? p.sb2 : p.sb, sh = second ? p.sh2 : p.sh,
                  sr = second ? p.sr2 : p.sr;

    // the two 16-byte chunks of this thread: NeoX features 8c.. and
    // rd/2 + 8c..; GPT-J features 16c.. and 16c + 8..
    const int f0 = INTERLEAVED ? 16 * c : 8 * c;
    const int f1 = INTERLEAVED ? 16 * c + 8 : p.rotary_dim / 2 + 8 * c;
    uint16_t* base = reinterpret_cast<uint16_t*>(second ? p.x2 : p.x) +
                     (p.cu_seqlens != nullptr ? 0 : (int64_t)b * sb) + (row0 + t) * sr;

    // loads first: the angles below are computed while they are in flight
    u32x4_t a[kRopeHeadBatch], d[kRopeHeadBatch];
#pragma unroll
    for (int i = 0; i < kRopeHeadBatch; ++i) {
        if (h0 + i < heads) {
            const uint16_t* r = base + (int64_t)(h0 + i) * sh;
            a[i] = *reinterpret_cast<const u32x4_t*>(r + f0);
            d[i] = *reinterpret_cast<const u32x4_t*>(r + f1);
        }
    }

    float cs[8], sn[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const double ang = (double)pos * p.freq_pi[8 * c + j];   // half-turns
        const double r = ang - 2.0 * __builtin_floor(ang * 0.5);  // in [0, 2)
        sincospif((float)r, &sn[j], &cs[j]);
    }

#pragma unroll
    for (int i = 0; i < kRopeHeadBatch; ++i) {
        if (h0 + i >= heads) continue;
        float x[8], y[8];               // pair j = (x[j], y[j])
        if (INTERLEAVED) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                x[j] = chunk_elem<T>(a[i], 2 * j);
                y[j] = chunk_elem<T>(a[i], 2 * j + 1);
                x[4 + j] = chunk_elem<T>(d[i], 2 * j);
                y[4 + j] = chunk_elem<T>(d[i], 2 * j + 1);
            }
        } else {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                x[j] = chunk_elem<T>(a[i], j);
                y[j] = chunk_elem<T>(d[i], j);
            }
        }
        float xr[8], yr[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            xr[j] = x[j] * cs[j] - y[j] * sn[j];
            yr[j] = x[j] * sn[j] + y[j] * cs[j];
        }
        u32x4_t oa, od;
        if (INTERLEAVED) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                oa[j] = Elem<T>::put(xr[j], yr[j]);
                od[j] = Elem<T>::put(xr[4 + j], yr[4 + j]);
            }
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                oa[j] = Elem<T>::put(xr[2 * j], xr[2 * j + 1]);
                od[j] = Elem<T>::put(yr[2 * j], yr[2 * j + 1]);
            }
        }
        uint16_t* r = base + (int64_t)(h0 + i) * sh;
        *reinterpret_cast<u32x4_t*>(r + f0) = oa;
        *reinterpret_cast<u32x4_t*>(r + f1) = od;
    }
}

template <typename T>
hipError_t launch_rotary_t(const RopeParams& p, hipStream_t stream) {
    const int64_t units = (int64_t)p.seqlen * (p.rotary_dim / 16);
    const int z = (p.heads + kRopeHeadBatch - 1) / kRopeHeadBatch +
                  (p.heads2 + kRopeHeadBatch - 1) / kRopeHeadBatch;
    const dim3 grid((unsigned)((units + kRopeThreads - 1) / kRopeThreads), (unsigned)p.batch,
                    (unsigned)z);
    if (p.interleaved)
        hipLaunchKernelGGL((rotary_kernel<T, true>), grid, dim3(kRopeThreads), 0, stream, p);
    else
        hipLaunchKernelGGL((rotary_kernel<T, false>), grid, dim3(kRopeThreads), 0, stream, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_rotary(const RopeParams& p, int dtype, hipStream_t stream) {
    return dtype == 0 ? launch_rotary_t<f16_t>(p, stream) : launch_rotary_t<bf16_t>(p, stream);
}

}  // namespace mi_attn
