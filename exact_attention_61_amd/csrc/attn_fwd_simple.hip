// Scalar (non-MFMA) attention forward for gfx950: one lane per query row.
//
// It walks the keys in order and keeps, per query row, the running maximum m,
// the exp-sum l taken relative to m and the output accumulator taken relative
// to m; whenever m grows both are multiplied by r = 2^(m_old - m_new) (the
// online softmax of section 3.1 of "FlashAttention: turning the quadratic
// intermediate matrices into statistics", with base-2 exponentials and the
// scale folded into the log2(e) factor).  Keys are staged through LDS in
// tiles of KT rows, converted to fp32.
//
// This kernel is the plain reference point of the library: it serves every
// supported shape, and the MFMA kernel is checked against the same oracle.
#include "common.hpp"

namespace mi_attn {
namespace {

constexpr int kRows = 64;   // query rows per work-group = one wave64
constexpr int kKeys = 32;   // keys per LDS tile

template <int D, typename Tin, typename Tout>
__global__ __launch_bounds__(kRows) void attn_fwd_simple_kernel(FwdParams p) {
    __shared__ float ks[kKeys][D + 1];
    __shared__ float vs[kKeys][D + 1];

    const int tile = blockIdx.x;
    const int h = blockIdx.y;
    const int b = blockIdx.z;
    int q0 = 0, lq_b = p.lq, k0 = 0, lk_b = p.lk;
    if (p.cu_q != nullptr) {
        q0 = p.cu_q[b];
        lq_b = p.cu_q[b + 1] - q0;
        k0 = p.cu_k[b];
        lk_b = p.cu_k[b + 1] - k0;
    }
    const int row0 = tile * kRows;
    if (row0 >= lq_b) return;                       // uniform over the block
    const int r = row0 + (int)threadIdx.x;
    const bool row_ok = r < lq_b;
    const int g = h / (p.hq / p.hkv);
    const bool packed = p.cu_q != nullptr;

    const Tin* qp = reinterpret_cast<const Tin*>(p.q) +
                    (packed ? 0 : (int64_t)b * p.q_sb) + (int64_t)h * p.q_sh +
                    (int64_t)(q0 + (row_ok ? r : row0)) * p.q_sr;
    const Tin* kp = reinterpret_cast<const Tin*>(p.k) +
                    (packed ? 0 : (int64_t)b * p.k_sb) + (int64_t)g * p.k_sh +
                    (int64_t)k0 * p.k_sr;
    const Tin* vp = reinterpret_cast<const Tin*>(p.v) +
                    (packed ? 0 : (int64_t)b * p.v_sb) + (int64_t)g * p.v_sh +
                    (int64_t)k0 * p.v_sr;

    float qr[D], acc[D];
    const float sgn = p.negate_q ? -1.0f : 1.0f;
#pragma unroll
    for (int c = 0; c < D; ++c) {
        qr[c] = sgn * to_f32(qp[c]);
        acc[c] = 0.0f;
    }
    float m = -__builtin_inff();
    float l = 0.0f;

    // Last key any row of this tile may see.
    int kend = lk_b;
    if (p.causal) {
        const int last = (row0 + kRows - 1) + lk_b - lq_b;   // inclusive
        kend = min(kend, last + 1);
    }
    const int my_last = p.causal ? r + lk_b - lq_b : lk_b - 1;

    for (int kt = 0; kt < kend; kt += kKeys) {
        __syncthreads();
        for (int e = threadIdx.x; e < kKeys * D; e += kRows) {
            const int j = e / D, c = e % D;
            const bool in = kt + j < lk_b;
            ks[j][c] = in ? to_f32(kp[(int64_t)(kt + j) * p.k_sr + c]) : 0.0f;
            vs[j][c] = in ? to_f32(vp[(int64_t)(kt + j) * p.v_sr + c]) : 0.0f;
        }
        __syncthreads();
        const int nk = min(kKeys, kend - kt);
        for (int j = 0; j < nk; ++j) {
            const int key = kt + j;
            if (!row_ok || key > my_last) continue;
            float s = 0.0f;
#pragma unroll
            for (int c = 0; c < D; ++c) s = fmaf(qr[c], ks[j][c], s);
            const float t = s * p.scale_log2;             // log2 domain
            const float m_new = fmaxf(m, t);
            const float rscl = exp2f(m - m_new);          // 0 on the first key
            const float pj = exp2f(t - m_new);
            l = l * rscl + pj;
#pragma unroll
            for (int c = 0; c < D; ++c) acc[c] = fmaf(acc[c], rscl, pj * vs[j][c]);
            m = m_new;
        }
    }

    if (!row_ok) return;
    const int64_t orow = (packed ? 0 : (int64_t)b * p.o_sb) +
                         (int64_t)h * p.o_sh + (int64_t)(q0 + r) * p.o_sr;
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
#pragma unroll
    for (int c = 0; c < D; ++c) OutStore<Tout>::put(p.o, orow + c, acc[c] * inv);
    if (p.lse != nullptr) {
        const float lse = l > 0.0f ? (m + log2f(l)) * 0.69314718055994530942f
                                   : -__builtin_inff();
        int64_t li;
        if (packed) {
            li = (int64_t)h * p.cu_q[p.batch] + q0 + r;
        } else {
            li = ((int64_t)b * p.hq + h) * p.lq + r;
        }
        p.lse[li] = lse;
    }
}

template <int D, typename Tin, typename Tout>
hipError_t launch_typed(const FwdParams& p, hipStream_t stream) {
    const dim3 grid((p.lq + kRows - 1) / kRows, p.hq, p.batch);
    hipLaunchKernelGGL((attn_fwd_simple_kernel<D, Tin, Tout>), grid, dim3(kRows),
                       0, stream, p);
    return hipGetLastError();
}

template <int D>
hipError_t launch_d(const FwdParams& p, int in_dtype, int out_dtype,
                    hipStream_t stream) {
    // dtype codes: 0 = f16, 1 = bf16, 2 = f32 (validated by the caller)
    if (in_dtype == 0) {
        return out_dtype == 2 ? launch_typed<D, f16_t, float>(p, stream)
                              : launch_typed<D, f16_t, f16_t>(p, stream);
    }
    return out_dtype == 2 ? launch_typed<D, bf16_t, float>(p, stream)
                          : launch_typed<D, bf16_t, bf16_t>(p, stream);
}

}  // namespace

hipError_t launch_simple(const FwdParams& p, int in_dtype, int out_dtype,
                         int head_dim, hipStream_t stream) {
    return head_dim == 64 ? launch_d<64>(p, in_dtype, out_dtype, stream)
                          : launch_d<128>(p, in_dtype, out_dtype, stream);
}

}  // namespace mi_attn
