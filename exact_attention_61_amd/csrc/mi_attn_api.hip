// Host side of libmi_attn: the C ABI declared in include/mi_attn.h.
//
// Every argument is validated before the first HIP call, so a rejected call
// enqueues nothing and touches no output.  Validation mirrors the input
// checks of the pages' fused-dense binding (dtype, contiguity and shape
// checks before any launch, an error code instead of a crash) and the
// training tutorial's constraints (Hkv divides Hq, head_dim a multiple of 8).
#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstddef>
#include <cstdint>
#include <mutex>

#include "../../include/mi_attn.h"
#include "common.hpp"

namespace {

thread_local int32_t g_last_hip_error = 0;

constexpr int64_t kMaxRowStride = int64_t(1) << 24;   // elements
constexpr int32_t kMaxQueryRows = 65535 * 128;        // 65535 q-tiles of 128 rows

bool aligned16(const void* p) {
    return (reinterpret_cast<uintptr_t>(p) & 15u) == 0;
}

bool stride_ok(const mi_attn_strides_t& s) {
    return s.batch >= 0 && s.head >= 0 && s.row >= 0 && s.batch % 8 == 0 &&
           s.head % 8 == 0 && s.row % 8 == 0;
}

mi_attn_strides_t default_strides(bool packed, int64_t heads, int64_t rows,
                                  int64_t d) {
    if (packed) return mi_attn_strides_t{0, d, heads * d};
    return mi_attn_strides_t{heads * rows * d, rows * d, d};
}

// Compute units of the current device (a scheduling hint for the kernels;
// any positive value gives the same results).  Cached per device.
static int current_device_cus() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int n = cache[dev].load(std::memory_order_relaxed);
    if (n > 0) return n;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
        n = 256;
    cache[dev].store(n, std::memory_order_relaxed);
    return n;
}

// Validation and launch shared by mi_attn_fwd and mi_attn_fwd_select.
mi_attn_status_t forward(const void* q, const void* k, const void* v,
                         void* o, float* lse, mi_attn_dtype_t in_dtype,
                         mi_attn_dtype_t out_dtype, int32_t batch,
                         int32_t hq, int32_t hkv, int32_t lq, int32_t lk,
                         int32_t head_dim, const mi_attn_strides_t* q_strides,
                         const mi_attn_strides_t* k_strides,
                         const mi_attn_strides_t* v_strides,
                         const mi_attn_strides_t* o_strides,
                         const int32_t* cu_seqlens_q,
                         const int32_t* cu_seqlens_k, float scale,
                         int32_t causal, struct ihipStream_t* stream,
                         int32_t kernel, int32_t causal_order,
                         double dropout_p = 0.0, uint64_t seed = 0) {
    if (!(dropout_p >= 0.0 && dropout_p < 1.0)) return MI_ATTN_ERR_ARG;   // NaN too
    if (kernel != MI_ATTN_KERNEL_MFMA && kernel != MI_ATTN_KERNEL_SCALAR)
        return MI_ATTN_ERR_ARG;
    if (causal_order < -1 || causal_order > 3) return MI_ATTN_ERR_ARG;
    if (in_dtype != MI_ATTN_F16 && in_dtype != MI_ATTN_BF16)
        return MI_ATTN_ERR_DTYPE;
    if (out_dtype != in_dtype && out_dtype != MI_ATTN_F32)
        return MI_ATTN_ERR_DTYPE;
    if (batch < 0 || lq < 0 || lk < 0 || hq < 1 || hkv < 1 || hq % hkv != 0)
        return MI_ATTN_ERR_SHAPE;
    // Launch-size limits: the grid is (query head, batch, 128-row q-tile),
    // at most 65535 along each axis.
    if (hq > 65535 || batch > 65535 || lq > kMaxQueryRows) return MI_ATTN_ERR_SHAPE;
    if (head_dim != 64 && head_dim != 128) return MI_ATTN_ERR_UNSUPPORTED;
    if (!std::isfinite(scale)) return MI_ATTN_ERR_ARG;
    if (causal != 0 && causal != 1) return MI_ATTN_ERR_ARG;
    const bool packed = cu_seqlens_q != nullptr;
    if (packed != (cu_seqlens_k != nullptr)) return MI_ATTN_ERR_ARG;
    if (batch == 0 || lq == 0) return MI_ATTN_OK;   // nothing to compute
    // K and V may be absent only when a dense call has no key rows at all.
    const bool no_keys = !packed && lk == 0;
    if (q == nullptr || o == nullptr ||
        (!no_keys && (k == nullptr || v == nullptr)))
        return MI_ATTN_ERR_NULL;

    const mi_attn_strides_t qs =
        q_strides ? *q_strides : default_strides(packed, hq, lq, head_dim);
    const mi_attn_strides_t ks =
        k_strides ? *k_strides : default_strides(packed, hkv, lk, head_dim);
    const mi_attn_strides_t vs =
        v_strides ? *v_strides : default_strides(packed, hkv, lk, head_dim);
    const mi_attn_strides_t os =
        o_strides ? *o_strides : default_strides(packed, hq, lq, head_dim);
    if (!stride_ok(qs) || !stride_ok(ks) || !stride_ok(vs) || !stride_ok(os))
        return MI_ATTN_ERR_LAYOUT;
    // Q, K and V tiles are fetched with 32-bit offsets from a tile's first row.
    if (qs.row >= kMaxRowStride || ks.row >= kMaxRowStride || vs.row >= kMaxRowStride)
        return MI_ATTN_ERR_LAYOUT;
    // Rows may not overlap: the tile copies read each row's head_dim
    // elements from a range that ends with the last row, so a Q, K or V row
    // stride below head_dim (for instance 0, an expanded view) would read
    // the wrong elements, and overlapping O rows would be written by several
    // lanes.  A tensor with a single row (dense Lq or Lk == 1) may have any
    // row stride.
    {
        const bool one_q = !packed && lq == 1;
        const bool one_k = !packed && lk <= 1;
        if ((!one_q && (qs.row < head_dim || os.row < head_dim)) ||
            (!one_k && (ks.row < head_dim || vs.row < head_dim)))
            return MI_ATTN_ERR_LAYOUT;
    }
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) ||
        (lse != nullptr && (reinterpret_cast<uintptr_t>(lse) & 3u) != 0))
        return MI_ATTN_ERR_LAYOUT;

    mi_attn::FwdParams p{};
    p.q = q;
    p.k = k;
    p.v = v;
    p.o = o;
    p.lse = lse;
    p.cu_q = cu_seqlens_q;
    p.cu_k = cu_seqlens_k;
    p.q_sb = qs.batch; p.q_sh = qs.head; p.q_sr = qs.row;
    p.k_sb = ks.batch; p.k_sh = ks.head; p.k_sr = ks.row;
    p.v_sb = vs.batch; p.v_sh = vs.head; p.v_sr = vs.row;
    p.o_sb = os.batch; p.o_sh = os.head; p.o_sr = os.row;
    p.batch = batch;
    p.hq = hq;
    p.hkv = hkv;
    // kv head = h / group, taken in the kernel as (h * ceil(2^32 / group))
    // >> 32, exact for h and group below 2^16 (hq <= 65535 above)
    {
        const uint64_t grp = (uint64_t)(hq / hkv);
        p.group_magic = ((uint64_t(1) << 32) + grp - 1) / grp;
    }
    p.lq = lq;
    p.lk = lk;
    // |scale| * log2(e), floored at 1e-30 so that a masked score (-inf) times
    // the factor stays -inf; a smaller factor changes no visible score.
    p.scale_log2 = (float)std::fmax(
        std::fabs((double)scale) * 1.4426950408889634074, 1e-30);
    p.negate_q = scale < 0.0f ? 1 : 0;
    p.causal = causal;
    p.causal_pairs = causal_order;
    p.n_cu = current_device_cus();
    // dropout: keep a key iff its 16-bit Philox half >= floor(p * 2^16); kept
    // probabilities are scaled by 1 / (1 - p)
    const bool drop = dropout_p > 0.0;
    p.drop_threshold = (uint32_t)std::floor(dropout_p * 65536.0);
    p.drop_scale = (float)(1.0 / (1.0 - dropout_p));
    p.seed_lo = (uint32_t)(seed & 0xffffffffu);
    p.seed_hi = (uint32_t)(seed >> 32);

    const hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    hipError_t err;
    if (kernel == MI_ATTN_KERNEL_SCALAR)
        err = mi_attn::launch_simple(p, (int)in_dtype, (int)out_dtype, head_dim, st);
    else if (drop)
        err = head_dim == 64 ? mi_attn::launch_mfma_drop_d64(p, (int)in_dtype, (int)out_dtype, st)
                             : mi_attn::launch_mfma_drop_d128(p, (int)in_dtype, (int)out_dtype, st);
    else if (head_dim == 64)
        err = mi_attn::launch_mfma_d64(p, (int)in_dtype, (int)out_dtype, st);
    else
        err = mi_attn::launch_mfma_d128(p, (int)in_dtype, (int)out_dtype, st);
    if (err != hipSuccess) {
        g_last_hip_error = (int32_t)err;
        return MI_ATTN_ERR_HIP;
    }
    return MI_ATTN_OK;
}

// ---------------------------------------------------------------------------
// Decode: work split and workspace layout
// ---------------------------------------------------------------------------

constexpr int kDecMaxRows = 32;          // query rows per decode work-group
constexpr int kDecMaxLq = 32;
constexpr int kDecChunkAlign = 128;      // keys: 4 waves x 32-key tiles
constexpr int kCUs = 256;                // MI355X compute units

struct DecodePlan {
    int32_t hpg, nqg, splits, chunk;
    size_t off_ml, bytes;                // workspace layout (bytes == 0: none)
};

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// The split count: the caller's, or enough splits for about one work-group
// per CU, each with at least 256 keys.
DecodePlan decode_plan(int32_t batch, int32_t hq, int32_t hkv, int32_t lq, int32_t lk,
                       int32_t head_dim, int32_t num_splits) {
    DecodePlan pl{};
    const int32_t group = hq / hkv;
    pl.hpg = std::max(1, std::min(group, kDecMaxRows / std::max(1, lq)));
    pl.nqg = (group + pl.hpg - 1) / pl.hpg;
    const int64_t groups = (int64_t)batch * hkv * pl.nqg;
    const int32_t max_splits = std::max(1, (lk + 255) / 256);
    int32_t s = num_splits;
    if (s <= 0) {
        s = (int32_t)std::max<int64_t>(1, (kCUs + groups - 1) / std::max<int64_t>(1, groups));
        s = std::min(s, max_splits);
    }
    s = std::min(s, std::max(1, (lk + kDecChunkAlign - 1) / kDecChunkAlign));
    pl.splits = std::max(1, s);
    const int32_t per = (lk + pl.splits - 1) / pl.splits;
    pl.chunk = std::max(kDecChunkAlign,
                        (per + kDecChunkAlign - 1) / kDecChunkAlign * kDecChunkAlign);
    // splits whose keys all lie past lk would do nothing: drop them
    pl.splits = std::max(1, std::min(pl.splits, (lk + pl.chunk - 1) / pl.chunk));
    if (pl.splits == 1) return pl;
    const size_t rows = (size_t)batch * hq * lq * pl.splits;
    pl.off_ml = align256(rows * head_dim * 4);
    pl.bytes = pl.off_ml + align256(rows * 2 * 4);
    return pl;
}

// ---------------------------------------------------------------------------
// Static scratch of mi_attn_decode_noalloc: a file-scope device array, one
// copy per GPU, reached through the address hipGetSymbolAddress gives on that
// device (the array's name is only a host-side stand-in).  It holds the
// partial results of one call (the workspace layout); nothing in it has to
// start at any value.
// ---------------------------------------------------------------------------

constexpr size_t kScratchBytes = size_t(8) << 20;           // 8 MiB per GPU
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

struct ScratchSlot {
    std::once_flag once;
    char* ptr = nullptr;
    hipError_t err = hipSuccess;
};
ScratchSlot g_scratch[kMaxDevices];

// The scratch address on the current device, looked up on the first call
// for the device.
hipError_t scratch_on_current_device(char** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    ScratchSlot& slot = g_scratch[dev];
    std::call_once(slot.once, [&]() {
        void* ptr = nullptr;
        slot.err = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (slot.err == hipSuccess) slot.ptr = static_cast<char*>(ptr);
    });
    *out = slot.ptr;
    return slot.err;
}

bool fits_scratch(const DecodePlan& pl) { return pl.bytes <= kScratchBytes; }

// Validation and launch of the decode path.  `workspace` (bytes) holds the
// partial results of the splits (no state is kept between calls).
mi_attn_status_t decode(const void* q, const void* k, const void* v, void* o, float* lse,
                        mi_attn_dtype_t in_dtype, mi_attn_dtype_t out_dtype, int32_t batch,
                        int32_t hq, int32_t hkv, int32_t lq, int32_t lk, int32_t head_dim,
                        const mi_attn_strides_t* q_strides, const mi_attn_strides_t* k_strides,
                        const mi_attn_strides_t* v_strides, const mi_attn_strides_t* o_strides,
                        const int32_t* seqlens_k, float scale, int32_t causal,
                        int32_t num_splits, void* workspace, size_t workspace_bytes,
                        struct ihipStream_t* stream, bool use_scratch = false) {
    if (in_dtype != MI_ATTN_F16 && in_dtype != MI_ATTN_BF16) return MI_ATTN_ERR_DTYPE;
    if (out_dtype != in_dtype && out_dtype != MI_ATTN_F32) return MI_ATTN_ERR_DTYPE;
    if (batch < 0 || lq < 0 || lk < 0 || hq < 1 || hkv < 1 || hq % hkv != 0)
        return MI_ATTN_ERR_SHAPE;
    if (lq > kDecMaxLq || hq > 65535 || batch > 65535) return MI_ATTN_ERR_SHAPE;
    if (head_dim != 64 && head_dim != 128) return MI_ATTN_ERR_UNSUPPORTED;
    if (!std::isfinite(scale)) return MI_ATTN_ERR_ARG;
    if (causal != 0 && causal != 1) return MI_ATTN_ERR_ARG;
    if (num_splits < 0 || num_splits > 65535) return MI_ATTN_ERR_ARG;
    if (batch == 0 || lq == 0) return MI_ATTN_OK;
    const bool no_keys = lk == 0;
    if (q == nullptr || o == nullptr || (!no_keys && (k == nullptr || v == nullptr)))
        return MI_ATTN_ERR_NULL;
    const mi_attn_strides_t qs = q_strides ? *q_strides : default_strides(false, hq, lq, head_dim);
    const mi_attn_strides_t ks = k_strides ? *k_strides : default_strides(false, hkv, lk, head_dim);
    const mi_attn_strides_t vs = v_strides ? *v_strides : default_strides(false, hkv, lk, head_dim);
    const mi_attn_strides_t os = o_strides ? *o_strides : default_strides(false, hq, lq, head_dim);
    if (!stride_ok(qs) || !stride_ok(ks) || !stride_ok(vs) || !stride_ok(os))
        return MI_ATTN_ERR_LAYOUT;
    if (ks.row >= kMaxRowStride || vs.row >= kMaxRowStride) return MI_ATTN_ERR_LAYOUT;
    if ((lq > 1 && (qs.row < head_dim || os.row < head_dim)) ||
        (lk > 1 && (ks.row < head_dim || vs.row < head_dim)))
        return MI_ATTN_ERR_LAYOUT;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) ||
        (lse != nullptr && (reinterpret_cast<uintptr_t>(lse) & 3u) != 0))
        return MI_ATTN_ERR_LAYOUT;
    const DecodePlan pl = decode_plan(batch, hq, hkv, lq, lk, head_dim, num_splits);
    if ((int64_t)hkv * pl.nqg > 65535) return MI_ATTN_ERR_SHAPE;
    if (use_scratch) {
        if (pl.bytes > 0 && !fits_scratch(pl)) return MI_ATTN_ERR_WORKSPACE;
    } else if (pl.bytes > 0) {
        if (workspace == nullptr) return MI_ATTN_ERR_NULL;
        if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return MI_ATTN_ERR_LAYOUT;
        if (workspace_bytes < pl.bytes) return MI_ATTN_ERR_WORKSPACE;
    }
    // the static scratch of this device (set up on the first call)
    char* scratch_base = nullptr;
    if (use_scratch && pl.bytes > 0) {
        const hipError_t e = scratch_on_current_device(&scratch_base);
        if (e != hipSuccess) {
            g_last_hip_error = (int32_t)e;
            return MI_ATTN_ERR_HIP;
        }
    }

    mi_attn::DecParams p{};
    p.q = q; p.k = k; p.v = v; p.o = o; p.lse = lse;
    p.seqlens_k = seqlens_k;
    p.q_sb = qs.batch; p.q_sh = qs.head; p.q_sr = qs.row;
    p.k_sb = ks.batch; p.k_sh = ks.head; p.k_sr = ks.row;
    p.v_sb = vs.batch; p.v_sh = vs.head; p.v_sr = vs.row;
    p.o_sb = os.batch; p.o_sh = os.head; p.o_sr = os.row;
    p.batch = batch; p.hq = hq; p.hkv = hkv; p.lq = lq; p.lk = lk;
    p.group = hq / hkv;
    p.hpg = pl.hpg;
    p.nqg = pl.nqg;
    p.splits = pl.splits;
    p.chunk = pl.chunk;
    p.scale_log2 = (float)std::fmax(std::fabs((double)scale) * 1.4426950408889634074, 1e-30);
    p.negate_q = scale < 0.0f ? 1 : 0;
    p.causal = causal;
    if (pl.bytes > 0) {
        char* ws = use_scratch ? scratch_base : static_cast<char*>(workspace);
        p.part_o = reinterpret_cast<float*>(ws);
        p.part_ml = reinterpret_cast<float*>(ws + pl.off_ml);
    }
    const hipError_t err = mi_attn::launch_decode(p, (int)in_dtype, (int)out_dtype, head_dim,
                                                  reinterpret_cast<hipStream_t>(stream));
    if (err != hipSuccess) {
        g_last_hip_error = (int32_t)err;
        return MI_ATTN_ERR_HIP;
    }
    return MI_ATTN_OK;
}

}  // namespace

namespace {

// Rotary embedding of x (and of x2 with heads2 > 0, the same rows and
// positions) in one launch; the checks of mi_attn_rotary and
// mi_attn_rotary_qk in their documented order.
mi_attn_status_t rotary(void* x, void* x2, mi_attn_dtype_t dtype, int32_t batch, int32_t heads,
                        int32_t heads2, int32_t seqlen, int32_t head_dim,
                        const mi_attn_strides_t* strides, const mi_attn_strides_t* strides2,
                        const int32_t* cu_seqlens, const int32_t* position_offsets,
                        int64_t position_offset, int32_t rotary_dim, double base,
                        int32_t interleaved, struct ihipStream_t* stream) {
    if (dtype != MI_ATTN_F16 && dtype != MI_ATTN_BF16) return MI_ATTN_ERR_DTYPE;
    if (batch < 0 || heads < 1 || heads2 < 0 || seqlen < 0 || head_dim < 1)
        return MI_ATTN_ERR_SHAPE;
    // grid y (batch) and z (groups of 4 heads of each tensor)
    if (batch > 65535 || (heads + 3) / 4 + (heads2 + 3) / 4 > 65535) return MI_ATTN_ERR_SHAPE;
    if (rotary_dim < 16 || rotary_dim % 16 != 0 || rotary_dim > head_dim || rotary_dim > 256)
        return MI_ATTN_ERR_UNSUPPORTED;
    if (!std::isfinite(base) || base <= 0.0) return MI_ATTN_ERR_ARG;
    if (interleaved != 0 && interleaved != 1) return MI_ATTN_ERR_ARG;
    if (batch == 0 || seqlen == 0) return MI_ATTN_OK;
    const bool two = heads2 > 0;
    if (x == nullptr || (two && x2 == nullptr)) return MI_ATTN_ERR_NULL;
    const bool packed = cu_seqlens != nullptr;
    const mi_attn_strides_t xs = strides ? *strides : default_strides(packed, heads, seqlen, head_dim);
    const mi_attn_strides_t xs2 =
        strides2 ? *strides2 : default_strides(packed, heads2, seqlen, head_dim);
    if (!stride_ok(xs) || !aligned16(x)) return MI_ATTN_ERR_LAYOUT;
    if (two && (!stride_ok(xs2) || !aligned16(x2) || x2 == x)) return MI_ATTN_ERR_LAYOUT;
    // rows and heads may not overlap (a thread writes its features of every head)
    if ((seqlen > 1 || packed) && (xs.row < head_dim || (two && xs2.row < head_dim)))
        return MI_ATTN_ERR_LAYOUT;
    if ((heads > 1 && xs.head < head_dim) || (heads2 > 1 && xs2.head < head_dim))
        return MI_ATTN_ERR_LAYOUT;

    mi_attn::RopeParams p{};
    p.x = x;
    p.x2 = two ? x2 : nullptr;
    p.cu_seqlens = cu_seqlens;
    p.offsets = position_offsets;
    p.sb = xs.batch; p.sh = xs.head; p.sr = xs.row;
    p.sb2 = xs2.batch; p.sh2 = xs2.head; p.sr2 = xs2.row;
    p.batch = batch;
    p.heads = heads;
    p.heads2 = two ? heads2 : 0;
    p.seqlen = seqlen;
    p.rotary_dim = rotary_dim;
    p.interleaved = interleaved;
    p.offset = position_offset;
    // pair k turns by base^(-2k / rd) radians per position, i.e.
    // base^(-2k / rd) / pi half-turns
    const double lb = std::log(base);
    for (int k2 = 0; k2 < rotary_dim / 2; ++k2)
        p.freq_pi[k2] = std::exp(-2.0 * k2 / rotary_dim * lb) / 3.14159265358979323846;
    const hipError_t err = mi_attn::launch_rotary(p, (int)dtype, reinterpret_cast<hipStream_t>(stream));
    if (err != hipSuccess) {
        g_last_hip_error = (int32_t)err;
        return MI_ATTN_ERR_HIP;
    }
    return MI_ATTN_OK;
}

}  // namespace

extern "C" {

size_t mi_attn_decode_workspace_size(int32_t batch, int32_t hq, int32_t hkv, int32_t lq,
                                     int32_t lk, int32_t head_dim, int32_t num_splits) {
    if (batch <= 0 || hq < 1 || hkv < 1 || hq % hkv != 0 || lq <= 0 || lq > kDecMaxLq ||
        lk < 0 || (head_dim != 64 && head_dim != 128) || num_splits < 0)
        return 0;
    return decode_plan(batch, hq, hkv, lq, lk, head_dim, num_splits).bytes;
}

int32_t mi_attn_decode_splits(int32_t batch, int32_t hq, int32_t hkv, int32_t lq, int32_t lk,
                              int32_t head_dim, int32_t num_splits) {
    if (batch <= 0 || hq < 1 || hkv < 1 || hq % hkv != 0 || lq <= 0 || lq > kDecMaxLq ||
        lk < 0 || (head_dim != 64 && head_dim != 128) || num_splits < 0)
        return 0;
    return decode_plan(batch, hq, hkv, lq, lk, head_dim, num_splits).splits;
}

mi_attn_status_t mi_attn_decode_noalloc(const void* q, const void* k, const void* v,
                                        void* o, float* lse, mi_attn_dtype_t in_dtype,
                                        mi_attn_dtype_t out_dtype, int32_t batch, int32_t hq,
                                        int32_t hkv, int32_t lq, int32_t lk, int32_t head_dim,
                                        const mi_attn_strides_t* q_strides,
                                        const mi_attn_strides_t* k_strides,
                                        const mi_attn_strides_t* v_strides,
                                        const mi_attn_strides_t* o_strides,
                                        const int32_t* seqlens_k, float scale, int32_t causal,
                                        int32_t num_splits, struct ihipStream_t* stream) {
    return decode(q, k, v, o, lse, in_dtype, out_dtype, batch, hq, hkv, lq, lk, head_dim,
                  q_strides, k_strides, v_strides, o_strides, seqlens_k, scale, causal,
                  num_splits, nullptr, 0, stream, true);
}

size_t mi_attn_decode_noalloc_max_bytes(void) { return kScratchBytes; }

mi_attn_status_t mi_attn_decode(const void* q, const void* k, const void* v, void* o,
                                float* lse, mi_attn_dtype_t in_dtype,
                                mi_attn_dtype_t out_dtype, int32_t batch, int32_t hq,
                                int32_t hkv, int32_t lq, int32_t lk, int32_t head_dim,
                                const mi_attn_strides_t* q_strides,
                                const mi_attn_strides_t* k_strides,
                                const mi_attn_strides_t* v_strides,
                                const mi_attn_strides_t* o_strides,
                                const int32_t* seqlens_k, float scale, int32_t causal,
                                int32_t num_splits, void* workspace, size_t workspace_bytes,
                                struct ihipStream_t* stream) {
    return decode(q, k, v, o, lse, in_dtype, out_dtype, batch, hq, hkv, lq, lk, head_dim,
                  q_strides, k_strides, v_strides, o_strides, seqlens_k, scale, causal,
                  num_splits, workspace, workspace_bytes, stream);
}

mi_attn_status_t mi_attn_fwd(const void* q, const void* k, const void* v,
                             void* o, float* lse, mi_attn_dtype_t in_dtype,
                             mi_attn_dtype_t out_dtype, int32_t batch,
                             int32_t hq, int32_t hkv, int32_t lq, int32_t lk,
                             int32_t head_dim, const mi_attn_strides_t* q_strides,
                             const mi_attn_strides_t* k_strides,
                             const mi_attn_strides_t* v_strides,
                             const mi_attn_strides_t* o_strides,
                             const int32_t* cu_seqlens_q,
                             const int32_t* cu_seqlens_k, float scale,
                             int32_t causal, struct ihipStream_t* stream) {
    return forward(q, k, v, o, lse, in_dtype, out_dtype, batch, hq, hkv, lq, lk,
                   head_dim, q_strides, k_strides, v_strides, o_strides,
                   cu_seqlens_q, cu_seqlens_k, scale, causal, stream,
                   MI_ATTN_KERNEL_MFMA, -1);
}

mi_attn_status_t mi_attn_fwd_select(const void* q, const void* k, const void* v,
                                    void* o, float* lse, mi_attn_dtype_t in_dtype,
                                    mi_attn_dtype_t out_dtype, int32_t batch,
                                    int32_t hq, int32_t hkv, int32_t lq, int32_t lk,
                                    int32_t head_dim,
                                    const mi_attn_strides_t* q_strides,
                                    const mi_attn_strides_t* k_strides,
                                    const mi_attn_strides_t* v_strides,
                                    const mi_attn_strides_t* o_strides,
                                    const int32_t* cu_seqlens_q,
                                    const int32_t* cu_seqlens_k, float scale,
                                    int32_t causal, struct ihipStream_t* stream,
                                    mi_attn_kernel_t kernel, int32_t causal_order) {
    return forward(q, k, v, o, lse, in_dtype, out_dtype, batch, hq, hkv, lq, lk,
                   head_dim, q_strides, k_strides, v_strides, o_strides,
                   cu_seqlens_q, cu_seqlens_k, scale, causal, stream,
                   (int32_t)kernel, causal_order);
}

mi_attn_status_t mi_attn_fwd_dropout(const void* q, const void* k, const void* v,
                                     void* o, float* lse, mi_attn_dtype_t in_dtype,
                                     mi_attn_dtype_t out_dtype, int32_t batch,
                                     int32_t hq, int32_t hkv, int32_t lq, int32_t lk,
                                     int32_t head_dim, const mi_attn_strides_t* q_strides,
                                     const mi_attn_strides_t* k_strides,
                                     const mi_attn_strides_t* v_strides,
                                     const mi_attn_strides_t* o_strides,
                                     const int32_t* cu_seqlens_q,
                                     const int32_t* cu_seqlens_k, float scale,
                                     int32_t causal, double dropout_p, uint64_t seed,
                                     struct ihipStream_t* stream) {
    return forward(q, k, v, o, lse, in_dtype, out_dtype, batch, hq, hkv, lq, lk,
                   head_dim, q_strides, k_strides, v_strides, o_strides,
                   cu_seqlens_q, cu_seqlens_k, scale, causal, stream,
                   MI_ATTN_KERNEL_MFMA, -1, dropout_p, seed);
}

mi_attn_status_t mi_attn_rotary(void* x, mi_attn_dtype_t dtype, int32_t batch,
                                int32_t heads, int32_t seqlen, int32_t head_dim,
                                const mi_attn_strides_t* strides, const int32_t* cu_seqlens,
                                const int32_t* position_offsets, int64_t position_offset,
                                int32_t rotary_dim, double base, int32_t interleaved,
                                struct ihipStream_t* stream) {
    return rotary(x, nullptr, dtype, batch, heads, 0, seqlen, head_dim, strides, nullptr,
                  cu_seqlens, position_offsets, position_offset, rotary_dim, base, interleaved,
                  stream);
}

mi_attn_status_t mi_attn_rotary_qk(void* q, void* k, mi_attn_dtype_t dtype, int32_t batch,
                                   int32_t hq, int32_t hkv, int32_t seqlen, int32_t head_dim,
                                   const mi_attn_strides_t* q_strides,
                                   const mi_attn_strides_t* k_strides,
                                   const int32_t* cu_seqlens, const int32_t* position_offsets,
                                   int64_t position_offset, int32_t rotary_dim, double base,
                                   int32_t interleaved, struct ihipStream_t* stream) {
    if (hkv < 1) return dtype != MI_ATTN_F16 && dtype != MI_ATTN_BF16 ? MI_ATTN_ERR_DTYPE
                                                                      : MI_ATTN_ERR_SHAPE;
    return rotary(q, k, dtype, batch, hq, hkv, seqlen, head_dim, q_strides, k_strides,
                  cu_seqlens, position_offsets, position_offset, rotary_dim, base, interleaved,
                  stream);
}

const char* mi_attn_status_string(mi_attn_status_t status) {
    switch (status) {
        case MI_ATTN_OK: return "MI_ATTN_OK: success";
        case MI_ATTN_ERR_NULL: return "MI_ATTN_ERR_NULL: q, k, v or o is NULL";
        case MI_ATTN_ERR_SHAPE:
            return "MI_ATTN_ERR_SHAPE: negative size, Hq/Hkv < 1, Hq not a "
                   "multiple of Hkv, or size beyond the launch limits";
        case MI_ATTN_ERR_LAYOUT:
            return "MI_ATTN_ERR_LAYOUT: pointer not 16-byte aligned, stride "
                   "negative / not a multiple of 8 elements, or a row stride "
                   "below head_dim";
        case MI_ATTN_ERR_DTYPE:
            return "MI_ATTN_ERR_DTYPE: inputs must be F16 or BF16 and the "
                   "output the input type or F32";
        case MI_ATTN_ERR_UNSUPPORTED:
            return "MI_ATTN_ERR_UNSUPPORTED: head_dim must be 64 or 128";
        case MI_ATTN_ERR_ARG:
            return "MI_ATTN_ERR_ARG: scale not finite, causal not 0/1, only "
                   "one cu_seqlens pointer given, or an unknown kernel / order";
        case MI_ATTN_ERR_HIP: return "MI_ATTN_ERR_HIP: kernel launch failed";
        case MI_ATTN_ERR_WORKSPACE:
            return "MI_ATTN_ERR_WORKSPACE: workspace smaller than "
                   "mi_attn_decode_workspace_size()";
    }
    return "unknown mi_attn status";
}

int32_t mi_attn_version(void) { return MI_ATTN_ABI_VERSION; }

int32_t mi_attn_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"
