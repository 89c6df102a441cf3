// Decode attention for gfx950: a few new query rows per sequence (Lq <= 32)
// against a long key/value cache, split along the keys across work-groups
// and merged by log-sum-exp.
//
// The new queries sit after the cached keys ("Training integration"
// tutorial, section 4.3: with a KV cache the rotary offset of the new tokens
// is the cache length), so the causal rule is bottom-right: query i of Lq
// sees keys j <= i + Lk_b - Lq.  Partial results over disjoint key ranges
// combine exactly as the online-softmax statistics of "FlashAttention:
// turning the quadratic intermediate matrices into statistics" (section 3.1,
// worked example 5-6): m = max of the parts, each part's exp-sum and output
// scaled by 2^(m_part - m).
//
// Work split.  One work-group = (batch b, kv head g, query group, key split
// s).  A query group packs heads g*G .. of the kv head's G query heads times
// the Lq positions into one block of at most 32 rows (row r = head * Lq +
// position), so each K/V element is read from memory once for all of them.
// The 4 waves of the work-group take the split's 32-key tiles in turn, each
// wave with its own LDS staging ring (no work-group barrier in the key
// loop): S^T = K Q^T and O^T = V^T P^T on v_mfma_f32_32x32x16, V^T operands
// from ds_read_b64_tr_b16.  The path is bound by the K/V stream from HBM, so
// the softmax keeps the exact running max per tile (P <= 1) and, for bf16,
// always splits P into hi + lo for the PV product.
//
// After the key loop the 4 waves merge through LDS.  With one split the
// work-group writes O and LSE; otherwise it writes its normalised partial
// output and (m, l) per row to the workspace, and a second kernel on the same
// stream merges the splits of every row and writes O and LSE.  (Merging in
// the last split to arrive needs a device-scope release and acquire around an
// arrival counter; with eight L2s those fences and the atomic cost ~30 us per
// launch, more than the whole merge kernel.)
#include <type_traits>

#include "../../include/mi_attn.h"
#include "mfma_util.hpp"

namespace mi_attn {

namespace {

constexpr int kDecWaves = 4;
constexpr int kDecThreads = 64 * kDecWaves;
constexpr int kDecTileKeys = 32;             // keys per wave-tile
constexpr int kDecRows = 32;                 // query rows per work-group

template <int D>
struct DecLayout {
    static constexpr int NKS = D / 16;       // k-steps of QK^T
    static constexpr int NDB = D / 32;       // 32-column blocks of O^T
    static constexpr int KEL = kDecTileKeys * D;   // elements of a K (or V) tile
    static constexpr int STAGE = 2 * KEL;    // K + V, 16-bit elements
    static constexpr int NSTG = D == 64 ? 4 : 2;   // stages per wave
    static constexpr int CPT = NKS + 2 * NDB;      // copy instructions per tile
    static constexpr int WAVE_LDS = NSTG * STAGE;  // elements per wave
    static_assert(kDecWaves * WAVE_LDS * 2 <= 160 * 1024, "LDS per CU");
    // merge area: per wave NDB x 16 x 64 floats of O^T, then (m, l) rows
    static constexpr int MERGE_ACC = NDB * 16 * 64;
    static_assert(kDecWaves * (MERGE_ACC + 2 * 64) * 4 <= kDecWaves * WAVE_LDS * 2,
                  "merge area fits the staging rings");
};

// One LDS array for the work-group; wave w uses elements [w * WAVE_LDS, ...).
template <int D>
__device__ __forceinline__ lds16_t* dec_lds() {
    __shared__ __attribute__((aligned(16))) uint16_t r[kDecWaves * DecLayout<D>::WAVE_LDS];
    return (lds16_t*)r;
}

template <int D, typename Tin, typename Tout>
__global__ __launch_bounds__(kDecThreads, 1) void attn_decode_kernel(DecParams p) {
    using L = DecLayout<D>;
    constexpr int NKS = L::NKS, NDB = L::NDB, NSTG = L::NSTG, CPT = L::CPT;

    const int split = (int)blockIdx.x;
    const int g = (int)blockIdx.y / p.nqg;               // kv head
    const int qg = (int)blockIdx.y - g * p.nqg;          // query group of the kv head
    const int b = (int)blockIdx.z;
    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    int lane = lane_id();
    int hi = lane >> 5;
    int col = lane & 31;                 // the query row of this lane (within the block)

    const int lk_b = p.seqlens_k != nullptr ? p.seqlens_k[b] : p.lk;
    const int h0 = g * p.group + qg * p.hpg;             // first query head of the group
    const int nh = min(p.hpg, p.group - qg * p.hpg);     // heads in this group
    const int rows = nh * p.lq;                          // valid rows (<= 32)
    const int diag = lk_b - p.lq;        // key j visible to position i iff j <= i + diag

    // this split's keys [kbeg, kend): the last row sees keys < lk_b
    const int kbeg = split * p.chunk;
    const int kend = max(kbeg, min(lk_b, kbeg + p.chunk));
    const int ntiles = (kend - kbeg + kDecTileKeys - 1) / kDecTileKeys;

    const uint16_t* kg = reinterpret_cast<const uint16_t*>(p.k) + (int64_t)b * p.k_sb +
                         (int64_t)g * p.k_sh + (int64_t)kbeg * p.k_sr;
    const uint16_t* vg = reinterpret_cast<const uint16_t*>(p.v) + (int64_t)b * p.v_sb +
                         (int64_t)g * p.v_sh + (int64_t)kbeg * p.v_sr;

    // Q fragments (B operand of S^T = K Q^T): lane holds row `col` (head
    // h0 + col / Lq, position col % Lq), columns (2 ks + hi) * 8 .. +7;
    // rows past the group read as zero
    u32x4_t qf[NKS];
    {
        const bool valid = col < rows;
        const int hl = valid ? col / p.lq : 0;
        const int pos = valid ? col - hl * p.lq : 0;
        const uint16_t* qrow = reinterpret_cast<const uint16_t*>(p.q) + (int64_t)b * p.q_sb +
                               (int64_t)(h0 + hl) * p.q_sh + (int64_t)pos * p.q_sr;
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            qf[ks] = valid ? *reinterpret_cast<const u32x4_t*>(qrow + (2 * ks + hi) * 8)
                           : u32x4_t{0u, 0u, 0u, 0u};
            if (p.negate_q) qf[ks] ^= 0x80008000u;
        }
    }
    // last visible key of this lane's row (split-relative: keys past it are
    // masked); padding rows see no key
    const int lastk = [&]() {
        if (col >= rows) return -1;
        const int pos = col % p.lq;
        const int last = p.causal ? min(lk_b - 1, pos + diag) : lk_b - 1;
        return last - kbeg;
    }();

    // ---- the wave's staging ring and copy plan -------------------------------
    lds16_t* ring = dec_lds<D>() + wave * L::WAVE_LDS;
    uint32_t voff[CPT];                  // byte offset of the lane's 16 bytes
    int dst[CPT];                        // element offset in a stage
#pragma unroll
    for (int t = 0; t < CPT; ++t) {
        int r, c;
        int64_t sr;
        if (t < NKS) {                   // K block ks = t
            r = lane & 31;
            c = (2 * t + (lane >> 5)) * 8;
            sr = p.k_sr;
            dst[t] = t * 512;
        } else {                         // V block bi = db * 2 + chunk
            const int bi = t - NKS;
            const int db = bi >> 1, kc = bi & 1;
            const int rr = lane >> 5;
            const int t2 = 2 * (lane & 31);
            r = kc * 16 + 8 * rr + 4 * (t2 >> 5) + ((t2 & 15) >> 2);
            c = db * 32 + 16 * ((t2 >> 4) & 1) + 4 * (t2 & 3);
            sr = p.v_sr;
            dst[t] = L::KEL + bi * 512;
        }
        voff[t] = (uint32_t)(((int64_t)r * sr + c) * 2);
    }
    auto rsrc_of = [&](const uint16_t* base, int64_t sr, int kt) {
        const int nrows = kt < ntiles ? min(kend - kbeg - kt * kDecTileKeys, kDecTileKeys) : 0;
        const uint64_t a = reinterpret_cast<uint64_t>(base + (int64_t)kt * kDecTileKeys * sr);
        u32x4_t r;
        r[0] = __builtin_amdgcn_readfirstlane((uint32_t)a);
        r[1] = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32) & 0xffffu);
        r[2] = __builtin_amdgcn_readfirstlane((uint32_t)(nrows * sr * 2));
        r[3] = 0x00020000u;
        return r;
    };
    // copies of tile kt (a tile past the split reads nothing and writes
    // zeros, so every iteration issues the same copies)
    auto issue = [&](int kt, lds16_t* st) {
        const u32x4_t rk = rsrc_of(kg, p.k_sr, kt);
        const u32x4_t rv = rsrc_of(vg, p.v_sr, kt);
#pragma unroll
        for (int t = 0; t < CPT; ++t) {
            const uint32_t lds_addr = (uint32_t)reinterpret_cast<uintptr_t>(st + dst[t]);
            if (t < NKS)
                asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds"
                             :: "v"(voff[t]), "s"(rk), "{m0}"(lds_addr) : "memory");
            else
                asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds"
                             :: "v"(voff[t]), "s"(rv), "{m0}"(lds_addr) : "memory");
        }
    };
    auto stage_at = [&](int i) { return ring + (i % NSTG) * L::STAGE; };

    // ---- the key loop: wave w takes tiles w, w + 4, ... -----------------------
    float m = -__builtin_inff(), l = 0.0f;
    f32x16_t acc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) acc[db] = f32x16_t{};
    const float c2 = p.scale_log2;
    const int nmine = ntiles > wave ? (ntiles - wave + kDecWaves - 1) / kDecWaves : 0;
#pragma unroll
    for (int i = 0; i < NSTG; ++i) issue(wave + i * kDecWaves, stage_at(i));
    for (int i = 0; i < nmine; ++i) {
        const int kt = wave + i * kDecWaves;
        // tile i landed: at most the copies of the NSTG-1 tiles after it pending
        wait_vm<(NSTG - 1) * CPT>();
        const lds16_t* st = stage_at(i);
        u32x4_t kf[NKS];
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
            kf[ks] = *reinterpret_cast<lds_u32x4_t*>(st + ks * 512 + lane * 8);
        u32x4_t vf[NDB][2];
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                const lds16_t* vb = st + L::KEL + (db * 2 + c) * 512 + lane * 4;
                const u32x2_t a = __builtin_bit_cast(u32x2_t, lds_read_tr(vb));
                const u32x2_t d = __builtin_bit_cast(u32x2_t, lds_read_tr(vb + 256));
                vf[db][c] = u32x4_t{a[0], a[1], d[0], d[1]};
            }
        f32x16_t s = f32x16_t{};
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) s = Mma<Tin>::run(kf[ks], qf[ks], s);
        // the fragments are in registers: the stage may be refilled
        wait_vm_lgkm0<63>();
        issue(kt + NSTG * kDecWaves, const_cast<lds16_t*>(st));
        // mask keys past the row's last visible key (and the split's end)
        const int lim = lastk - (kt * kDecTileKeys + 4 * hi);
#pragma unroll
        for (int e = 0; e < 16; ++e)
            if (8 * (e >> 2) + (e & 3) > lim) s[e] = -__builtin_inff();
        // exact running max
        float mx = s[0];
#pragma unroll
        for (int e = 1; e < 16; ++e) mx = max2(mx, s[e]);
        const float mt = max2(mx, partner(mx)) * c2;
        const float m_new = max2(m, mt);
        const float nm = m_new == -__builtin_inff() ? 0.0f : -m_new;
        const float alpha = m_new == -__builtin_inff() ? 1.0f : fast_exp2(m - m_new);
        m = m_new;
        l *= alpha;
#pragma unroll
        for (int db = 0; db < NDB; ++db) acc[db] *= alpha;
        u32x4_t ph[2], pl[2];
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int e = 8 * c + 2 * jj;
                const float x0 = fast_exp2(fmaf(s[e], c2, nm));
                const float x1 = fast_exp2(fmaf(s[e + 1], c2, nm));
                l += x0 + x1;
                const uint32_t hv = Mma<Tin>::pack(x0, x1);
                ph[c][jj] = hv;
                pl[c][jj] = Mma<Tin>::kSplit
                                ? Mma<Tin>::pack(x0 - Mma<Tin>::lo16(hv), x1 - Mma<Tin>::hi16(hv))
                                : 0u;
            }
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int c = 0; c < 2; ++c) {
                acc[db] = Mma<Tin>::run(vf[db][c], ph[c], acc[db]);
                if constexpr (Mma<Tin>::kSplit) acc[db] = Mma<Tin>::run(vf[db][c], pl[c], acc[db]);
            }
    }
    // every copy of this wave (including the empty tail copies) has landed
    wait_vm_lgkm0<0>();
    l = l + partner(l);                  // both halves of the row's keys
    __syncthreads();                     // every wave is done with its ring

    // ---- merge of the 4 waves through LDS ---------------------------------------
    lds_f32_t* mbase = reinterpret_cast<lds_f32_t*>(dec_lds<D>());
    auto macc = [&](int w) { return mbase + w * (L::MERGE_ACC + 128); };
    {
        lds_f32_t* a = macc(wave);
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int e = 0; e < 16; ++e) a[(db * 16 + e) * 64 + lane] = acc[db][e];
        a[L::MERGE_ACC + lane] = m;
        if (lane < 32) a[L::MERGE_ACC + 64 + lane] = l;
    }
    __syncthreads();
    // wave w combines column blocks db = w, w + 4, ... of every row
    float ms[kDecWaves], ls[kDecWaves];
    float M = -__builtin_inff();
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w) {
        ms[w] = macc(w)[L::MERGE_ACC + lane];
        ls[w] = macc(w)[L::MERGE_ACC + 64 + col];
        M = max2(M, ms[w]);
    }
    const float mu = M == -__builtin_inff() ? 0.0f : M;
    float Lsum = 0.0f, f[kDecWaves];
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w) {
        f[w] = fast_exp2(ms[w] - mu);
        Lsum += ls[w] * f[w];
    }
    const float inv = Lsum > 0.0f ? 1.0f / Lsum : 0.0f;
    const bool row_ok = col < rows;
    const int hl = row_ok ? col / p.lq : 0;
    const int pos = row_ok ? col - hl * p.lq : 0;
    const int hq = h0 + hl;
    const int64_t row_id = ((int64_t)b * p.hq + hq) * p.lq + pos;   // [B, Hq, Lq]
    for (int db = wave; db < NDB; db += kDecWaves) {
        f32x16_t o = f32x16_t{};
#pragma unroll
        for (int w = 0; w < kDecWaves; ++w) {
            const lds_f32_t* a = macc(w);
#pragma unroll
            for (int e = 0; e < 16; ++e) o[e] = fmaf(a[(db * 16 + e) * 64 + lane], f[w], o[e]);
        }
        o *= inv;                        // the work-group's normalised output
        if (!row_ok) continue;
        if (p.splits == 1) {
            const int64_t orow = (int64_t)b * p.o_sb + (int64_t)hq * p.o_sh + (int64_t)pos * p.o_sr;
#pragma unroll
            for (int gg = 0; gg < 4; ++gg) {
                const int d0 = db * 32 + 8 * gg + 4 * hi;
                Epi<Tout>::store4(p.o, orow + d0, o[4 * gg], o[4 * gg + 1], o[4 * gg + 2],
                                  o[4 * gg + 3]);
            }
        } else {
            float* po = p.part_o + (row_id * p.splits + split) * D;
#pragma unroll
            for (int gg = 0; gg < 4; ++gg) {
                const int d0 = db * 32 + 8 * gg + 4 * hi;
                *reinterpret_cast<f32x4_t*>(po + d0) =
                    f32x4_t{o[4 * gg], o[4 * gg + 1], o[4 * gg + 2], o[4 * gg + 3]};
            }
        }
    }
    if (p.splits == 1) {
        if (wave == 0 && row_ok && hi == 0 && p.lse != nullptr)
            p.lse[row_id] = Lsum > 0.0f ? (mu + __log2f(Lsum)) * 0.69314718055994530942f
                                        : -__builtin_inff();
        return;
    }
    if (wave == 0 && row_ok && hi == 0) {
        float* pm = p.part_ml + (row_id * p.splits + split) * 2;
        pm[0] = M;                       // log2 domain, -inf for a row with no key here
        pm[1] = Lsum;
    }
}

// Merge of the splits of one row per wave: m = max of the parts, each part's
// exp-sum and normalised output weighted by l_s 2^(m_s - m) (the combination
// rule of the online softmax, as across work-groups).  Lane j holds columns
// j, j + 64, ... of the row.
constexpr int kCombineRows = 4;          // rows (waves) per work-group
constexpr int kCombineUnrolled = 8;      // split counts merged with all loads up front

template <int D, typename Tout>
__global__ __launch_bounds__(64 * kCombineRows) void attn_decode_combine_kernel(DecParams p) {
    constexpr int CPL = D / 64;          // columns per lane
    const int64_t rows = (int64_t)p.batch * p.hq * p.lq;
    const int64_t rid = (int64_t)blockIdx.x * kCombineRows + (threadIdx.x >> 6);
    if (rid >= rows) return;
    const int lane = (int)threadIdx.x & 63;
    const int pos = (int)(rid % p.lq);
    const int64_t bh = rid / p.lq;
    const int hq = (int)(bh % p.hq), b = (int)(bh / p.hq);
    const float* pm = p.part_ml + rid * p.splits * 2;
    const float* po = p.part_o + rid * p.splits * D + lane;
    float M = -__builtin_inff(), L = 0.0f;
    float o[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) o[c] = 0.0f;
    if (p.splits <= kCombineUnrolled) {
        // every load of the row issued at once (the partials come from
        // other XCDs' writes, a round trip to the fabric each): one round
        // trip instead of one for (m, l) and another for the outputs
        float ms[kCombineUnrolled], ls[kCombineUnrolled], os[kCombineUnrolled][CPL];
#pragma unroll
        for (int s = 0; s < kCombineUnrolled; ++s) {
            ms[s] = -__builtin_inff();
            ls[s] = 0.0f;
#pragma unroll
            for (int c = 0; c < CPL; ++c) os[s][c] = 0.0f;
            if (s < p.splits) {
                ms[s] = pm[2 * s];
                ls[s] = pm[2 * s + 1];
#pragma unroll
                for (int c = 0; c < CPL; ++c) os[s][c] = po[s * D + 64 * c];
            }
        }
#pragma unroll
        for (int s = 0; s < kCombineUnrolled; ++s) M = max2(M, ms[s]);
        const float mu = M == -__builtin_inff() ? 0.0f : M;
#pragma unroll
        for (int s = 0; s < kCombineUnrolled; ++s) {
            if (s < p.splits) {
                const float w = ls[s] * fast_exp2(ms[s] - mu);
                L += w;
#pragma unroll
                for (int c = 0; c < CPL; ++c) o[c] = fmaf(os[s][c], w, o[c]);
            }
        }
    } else {
        for (int s = 0; s < p.splits; ++s) M = max2(M, pm[2 * s]);
        const float mu = M == -__builtin_inff() ? 0.0f : M;
        for (int s = 0; s < p.splits; ++s) {
            const float w = pm[2 * s + 1] * fast_exp2(pm[2 * s] - mu);
            L += w;
#pragma unroll
            for (int c = 0; c < CPL; ++c) o[c] = fmaf(po[s * D + 64 * c], w, o[c]);
        }
    }
    const float mu = M == -__builtin_inff() ? 0.0f : M;
    const float inv = L > 0.0f ? 1.0f / L : 0.0f;
    const int64_t orow = (int64_t)b * p.o_sb + (int64_t)hq * p.o_sh + (int64_t)pos * p.o_sr;
#pragma unroll
    for (int c = 0; c < CPL; ++c) OutStore<Tout>::put(p.o, orow + lane + 64 * c, o[c] * inv);
    if (lane == 0 && p.lse != nullptr)
        p.lse[rid] = L > 0.0f ? (mu + __log2f(L)) * 0.69314718055994530942f : -__builtin_inff();
}

template <int D, typename Tin, typename Tout>
hipError_t launch_decode_typed(const DecParams& p, hipStream_t stream) {
    const dim3 grid((unsigned)p.splits, (unsigned)(p.hkv * p.nqg), (unsigned)p.batch);
    hipLaunchKernelGGL((attn_decode_kernel<D, Tin, Tout>), grid, dim3(kDecThreads), 0, stream, p);
    if (p.splits > 1) {
        const int64_t rows = (int64_t)p.batch * p.hq * p.lq;
        const dim3 g2((unsigned)((rows + kCombineRows - 1) / kCombineRows));
        hipLaunchKernelGGL((attn_decode_combine_kernel<D, Tout>), g2, dim3(64 * kCombineRows), 0,
                           stream, p);
    }
    return hipGetLastError();
}

template <int D>
hipError_t launch_decode_d(const DecParams& p, int in_dtype, int out_dtype, hipStream_t stream) {
    if (in_dtype == 0)
        return out_dtype == 2 ? launch_decode_typed<D, f16_t, float>(p, stream)
                              : launch_decode_typed<D, f16_t, f16_t>(p, stream);
    return out_dtype == 2 ? launch_decode_typed<D, bf16_t, float>(p, stream)
                          : launch_decode_typed<D, bf16_t, bf16_t>(p, stream);
}

}  // namespace

hipError_t launch_decode(const DecParams& p, int in_dtype, int out_dtype, int head_dim,
                         hipStream_t stream) {
    return head_dim == 64 ? launch_decode_d<64>(p, in_dtype, out_dtype, stream)
                          : launch_decode_d<128>(p, in_dtype, out_dtype, stream);
}

}  // namespace mi_attn
