/*
 * mi_attn.h — C ABI of libmi_attn, an exact attention forward pass for
 * AMD Instinct MI355X (gfx950).
 *
 * What the call computes.  For every batch entry b and query head h, with
 * key/value head g = floor(h / (Hq / Hkv)):
 *
 *     S[i, j] = scale * sum_c Q[b, h, i, c] * K[b, g, j, c]
 *     P[i, :] = softmax over the keys j visible to query i
 *     O[b, h, i, :] = sum_j P[i, j] * V[b, g, j, :]
 *     LSE[b, h, i]  = ln sum_j exp(S[i, j])            (visible j only)
 *
 * This is standard attention as stated on the fusion/compiler notes page
 * ("FlashAttention: turning the quadratic intermediate matrices into
 * statistics", clxhxhhr.top post 5544, section 3), computed tile by tile with
 * the online-softmax statistics of its section 3.1 (running max m, rescaled
 * exp-sum l, rescaled output accumulator), so no Lq x Lk score or probability
 * matrix is ever written to memory.  The interface follows the training
 * integration tutorial (inference.lei6393.com, sections 2.2-2.5 and 8.5):
 * causal masking, grouped-query attention with Hkv dividing Hq, cross
 * attention with Lq != Lk, packed variable-length batches in place of a
 * key padding mask, and a default scale of 1/sqrt(head_dim) (applied by the
 * Python binding; this C call always takes the scale explicitly).
 *
 * Visibility.  Key j of a sequence is visible to query i of the same sequence
 * iff j < Lk_b and, when causal != 0, j <= i + Lk_b - Lq_b (bottom-right
 * alignment: with Lq == Lk this is j <= i).  A query row with no visible key
 * gets O = 0 and LSE = -inf.
 *
 * Ownership and threading.  The caller owns every buffer.  The library never
 * allocates, frees or keeps a pointer past the call, holds no mutable global
 * state and may be called from several threads at once.  The work is
 * enqueued on `stream` on the current HIP device and the call returns at
 * once; buffers must stay alive until that stream work is done.
 */
#ifndef MI_ATTN_H
#define MI_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MI_ATTN_ABI_VERSION 1

#if defined(__GNUC__) || defined(__clang__)
#define MI_ATTN_API __attribute__((visibility("default")))
#else
#define MI_ATTN_API
#endif

/* Return codes.  Every argument is checked on the host before any HIP call;
 * on any error nothing is enqueued and o / lse are left untouched. */
typedef enum mi_attn_status {
    MI_ATTN_OK = 0,
    MI_ATTN_ERR_NULL = 1,        /* q, k, v or o is NULL where rows exist     */
    MI_ATTN_ERR_SHAPE = 2,       /* negative size, Hq or Hkv < 1,
                                    Hq % Hkv != 0, Hq or B above 65535, or
                                    lq above 65535 * 128 = 8388480          */
    MI_ATTN_ERR_LAYOUT = 3,      /* pointer not 16-byte aligned, stride not a
                                    multiple of 8 elements or negative, a
                                    Q/K/V row stride of 2^24 elements or more,
                                    or a row stride below head_dim in a
                                    tensor with more than one row            */
    MI_ATTN_ERR_DTYPE = 4,       /* in dtype not F16/BF16, or out dtype not
                                    the in dtype or F32                       */
    MI_ATTN_ERR_UNSUPPORTED = 5, /* head_dim not 64 or 128                    */
    MI_ATTN_ERR_ARG = 6,         /* scale not finite, causal not 0/1, only
                                    one of the cu_seqlens pointers given, or
                                    (mi_attn_fwd_select) an unknown kernel or
                                    causal order                              */
    MI_ATTN_ERR_HIP = 7,         /* the kernel launch failed (the HIP error
                                    is kept per thread, see below)            */
    MI_ATTN_ERR_WORKSPACE = 8    /* mi_attn_decode: workspace smaller than
                                    mi_attn_decode_workspace_size()           */
} mi_attn_status_t;

/* Element types. */
typedef enum mi_attn_dtype {
    MI_ATTN_F16 = 0,
    MI_ATTN_BF16 = 1,
    MI_ATTN_F32 = 2
} mi_attn_dtype_t;

/* Element strides of a 4-D view [batch, head, row, column]; the column
 * stride is always 1.  Dense [B, H, L, d] contiguous is
 * {H*L*d, L*d, d}; [B, L, H, d] (sequence-major) is {L*H*d, d, H*d}.
 * For packed variable-length tensors [T, H, d] only head and row are used
 * (row = token) and batch is ignored: {0, d, H*d} when contiguous. */
typedef struct mi_attn_strides {
    int64_t batch;
    int64_t head;
    int64_t row;
} mi_attn_strides_t;

struct ihipStream_t;   /* hipStream_t; NULL is the default stream */

/*
 * mi_attn_fwd — O = softmax(scale * Q K^T, masked) V and LSE, forward only.
 *
 * q, k, v   device pointers, element type in_dtype.
 *           Dense:  q [B, Hq, Lq, d], k and v [B, Hkv, Lk, d] as strided views.
 *           Packed: q [Tq, Hq, d], k and v [Tk, Hkv, d]; sequence b owns
 *           query rows cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1 and key rows
 *           cu_seqlens_k[b] .. cu_seqlens_k[b+1]-1.
 * o         device pointer, element type out_dtype, same shape as q (head_dim
 *           columns), written through o_strides.
 * lse       device pointer to float, or NULL to skip it.  Dense: contiguous
 *           [B, Hq, Lq].  Packed: contiguous [Hq, Tq] with Tq =
 *           cu_seqlens_q[B].  Natural log, scale included.
 * in_dtype  MI_ATTN_F16 or MI_ATTN_BF16 (q, k and v alike).
 * out_dtype in_dtype or MI_ATTN_F32 (rounded to nearest even from fp32).
 * batch     B >= 0.  B == 0 (or Lq == 0) is a no-op that returns MI_ATTN_OK
 *           once the dtypes and sizes are valid; the pointers may then be
 *           NULL.  k and v may also be NULL for a dense call with Lk == 0.
 * hq, hkv   query and key/value heads, hkv >= 1, hq a multiple of hkv.
 * lq, lk    dense: sequence lengths (>= 0); packed: the longest query / key
 *           sequence (max_seqlen), used to size the launch.  lq <= 8388480
 *           (65535 tiles of 128 query rows).
 * head_dim  64 or 128.
 * *_strides element strides (see mi_attn_strides_t); NULL means contiguous
 *           ([B, H, L, d] dense, [T, H, d] packed).  Strides must be >= 0 and
 *           multiples of 8, Q, K and V row strides below 2^24 elements, and
 *           every row stride at least head_dim (rows may not overlap) unless
 *           the dense tensor has a single row; base pointers must be 16-byte
 *           aligned.
 * cu_seqlens_q, cu_seqlens_k  device int32 arrays of B + 1 offsets, both NULL
 *           (dense) or both set (packed).  Their contents are not checked:
 *           the caller guarantees cu[0] = 0, non-decreasing, every length
 *           <= lq (resp. lk), and rows inside the tensors.
 * scale     multiplies Q K^T; any finite value.
 * causal    0 or 1 (bottom-right aligned, see above).
 * stream    HIP stream to enqueue on.
 *
 * Returns MI_ATTN_OK once the kernel is enqueued.  Faults inside the kernel
 * show up at the caller's next synchronisation, as with any HIP launch.
 */
MI_ATTN_API mi_attn_status_t mi_attn_fwd(const void* q, const void* k, const void* v,
                             void* o, float* lse,
                             mi_attn_dtype_t in_dtype, mi_attn_dtype_t out_dtype,
                             int32_t batch, int32_t hq, int32_t hkv,
                             int32_t lq, int32_t lk, int32_t head_dim,
                             const mi_attn_strides_t* q_strides,
                             const mi_attn_strides_t* k_strides,
                             const mi_attn_strides_t* v_strides,
                             const mi_attn_strides_t* o_strides,
                             const int32_t* cu_seqlens_q,
                             const int32_t* cu_seqlens_k,
                             float scale, int32_t causal,
                             struct ihipStream_t* stream);

/* Kernels mi_attn_fwd_select can run. */
typedef enum mi_attn_kernel {
    MI_ATTN_KERNEL_MFMA = 0,    /* the matrix-core kernel mi_attn_fwd runs   */
    MI_ATTN_KERNEL_SCALAR = 1   /* scalar fp32 kernel, one lane per query
                                   row: an independent second implementation
                                   for cross-checks, far slower              */
} mi_attn_kernel_t;

/*
 * mi_attn_fwd_select — mi_attn_fwd with the kernel and, for causal inputs,
 * the order of the query tiles chosen by the caller.  For tests and
 * diagnostics: every choice computes the same function as mi_attn_fwd
 * (bit-identical results are not promised across kernels).
 *
 * kernel        MI_ATTN_KERNEL_MFMA or MI_ATTN_KERNEL_SCALAR.
 * causal_order  MFMA kernel, causal inputs only (ignored otherwise):
 *               -1 the library's default for the head dimension;
 *                0 one query tile per work-group, heaviest first;
 *                1 query tiles t and n-1-t in one work-group;
 *                2 one query tile per work-group; head_dim 64: heaviest
 *                  first, except that the second round of as many
 *                  work-groups as the device has CUs runs lightest first
 *                  (in blocks of 8); head_dim 128: the first half of the
 *                  grid heaviest first and the second half lightest first;
 *                3 (head_dim 128, dense inputs, causal or not) resident
 *                  work-groups, one per slot the device holds at once,
 *                  each looping over query tiles ranked heaviest first and
 *                  dealt in a snake order (the fusion notes, section 5.4,
 *                  persistent kernels); other inputs take the default.
 * Other arguments, validation, ownership and errors as for mi_attn_fwd; an
 * unknown kernel or order returns MI_ATTN_ERR_ARG with nothing enqueued.
 */
MI_ATTN_API mi_attn_status_t mi_attn_fwd_select(const void* q, const void* k, const void* v,
                             void* o, float* lse,
                             mi_attn_dtype_t in_dtype, mi_attn_dtype_t out_dtype,
                             int32_t batch, int32_t hq, int32_t hkv,
                             int32_t lq, int32_t lk, int32_t head_dim,
                             const mi_attn_strides_t* q_strides,
                             const mi_attn_strides_t* k_strides,
                             const mi_attn_strides_t* v_strides,
                             const mi_attn_strides_t* o_strides,
                             const int32_t* cu_seqlens_q,
                             const int32_t* cu_seqlens_k,
                             float scale, int32_t causal,
                             struct ihipStream_t* stream,
                             mi_attn_kernel_t kernel, int32_t causal_order);

/*
 * mi_attn_decode — the same operation for a few new query rows per sequence
 * against a long key/value cache, with the keys split across work-groups
 * and the partial results merged by log-sum-exp.
 *
 * The new queries follow the cached keys (the training-integration
 * tutorial, section 4.3: with a KV cache the new tokens' positions start at
 * the cache length), so with causal = 1 query row i of Lq sees keys
 * j <= i + Lk_b - Lq (bottom-right, as for mi_attn_fwd); causal = 0 sees all
 * Lk_b keys.  A split's partial (m, l, output) over its keys combines with
 * the others by the rule of the fusion notes, section 3.1: m = max over the
 * parts, each part's exp-sum and output scaled by exp(m_part - m).
 *
 * q, o      dense [B, Hq, Lq, d] views (strides as for mi_attn_fwd), Lq <= 32.
 * k, v      the cache, dense [B, Hkv, Lk, d] views.
 * lse       [B, Hq, Lq] contiguous fp32, or NULL.
 * seqlens_k device int32 [B]: keys of sequence b are rows 0 .. seqlens_k[b]-1
 *           of its cache (each <= lk, not checked); NULL means lk for all.
 * num_splits  key splits per (sequence, kv head): 0 lets the library choose
 *           (about one work-group per CU, at least 256 keys per split);
 *           otherwise at most 65535, and capped so every split has keys.
 * workspace, workspace_bytes  device memory of at least
 *           mi_attn_decode_workspace_size(...) bytes, 256-byte aligned, or
 *           NULL when that size is 0 (a single split).  It holds the partial
 *           results of the splits, which a second kernel on the same stream
 *           merges; its contents need no initial value and nothing is kept
 *           between calls.  Calls that share one workspace must not overlap
 *           in time.
 * Other arguments, ownership, validation and errors as for mi_attn_fwd;
 * Lq above 32 returns MI_ATTN_ERR_SHAPE, a NULL or short workspace
 * MI_ATTN_ERR_NULL / MI_ATTN_ERR_WORKSPACE, a workspace not 256-byte
 * aligned MI_ATTN_ERR_LAYOUT.
 */
MI_ATTN_API mi_attn_status_t mi_attn_decode(const void* q, const void* k, const void* v,
                             void* o, float* lse,
                             mi_attn_dtype_t in_dtype, mi_attn_dtype_t out_dtype,
                             int32_t batch, int32_t hq, int32_t hkv,
                             int32_t lq, int32_t lk, int32_t head_dim,
                             const mi_attn_strides_t* q_strides,
                             const mi_attn_strides_t* k_strides,
                             const mi_attn_strides_t* v_strides,
                             const mi_attn_strides_t* o_strides,
                             const int32_t* seqlens_k,
                             float scale, int32_t causal, int32_t num_splits,
                             void* workspace, size_t workspace_bytes,
                             struct ihipStream_t* stream);

/*
 * mi_attn_decode_noalloc — mi_attn_decode for callers that cannot allocate
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the partial results live in a static device array of the
 * library, 8 MiB per GPU, held until the process ends.  It calls no
 * hipMalloc, hipFree or other allocating routine.
 *
 * Sizes whose partial results need more than
 * mi_attn_decode_noalloc_max_bytes() (8 MiB) return MI_ATTN_ERR_WORKSPACE
 * before any HIP call.  The array needs no initial value.  All calls on one
 * GPU share the array:
 * calls that overlap in time on one GPU (other streams, other threads)
 * race and give wrong results.  Arguments otherwise as for mi_attn_decode.
 */
MI_ATTN_API mi_attn_status_t mi_attn_decode_noalloc(const void* q, const void* k,
                             const void* v, void* o, float* lse,
                             mi_attn_dtype_t in_dtype, mi_attn_dtype_t out_dtype,
                             int32_t batch, int32_t hq, int32_t hkv,
                             int32_t lq, int32_t lk, int32_t head_dim,
                             const mi_attn_strides_t* q_strides,
                             const mi_attn_strides_t* k_strides,
                             const mi_attn_strides_t* v_strides,
                             const mi_attn_strides_t* o_strides,
                             const int32_t* seqlens_k,
                             float scale, int32_t causal, int32_t num_splits,
                             struct ihipStream_t* stream);
MI_ATTN_API size_t mi_attn_decode_noalloc_max_bytes(void);

/* Bytes of workspace mi_attn_decode needs for these sizes (0: none), and
 * the number of key splits it will use; both 0 for invalid sizes. */
MI_ATTN_API size_t mi_attn_decode_workspace_size(int32_t batch, int32_t hq, int32_t hkv,
                                                 int32_t lq, int32_t lk, int32_t head_dim,
                                                 int32_t num_splits);
MI_ATTN_API int32_t mi_attn_decode_splits(int32_t batch, int32_t hq, int32_t hkv,
                                          int32_t lq, int32_t lk, int32_t head_dim,
                                          int32_t num_splits);

/*
 * mi_attn_fwd_dropout -- mi_attn_fwd with dropout on the probabilities.
 *
 * The "Training integration" tutorial, sections 2.1 and 8.2: the attention
 * module takes a dropout probability for training (0.1 in its BERT-style
 * example) and 0 for inference.  Each probability P[i, j] of the softmax is
 * kept with probability 1 - dropout_p and then scaled by 1 / (1 - dropout_p),
 * or set to 0; O = (P * M) V with that mask and scale.  lse is the
 * log-sum-exp of the softmax itself (dropout acts after the normalisation).
 *
 * The mask: Philox4x32-10 (Salmon, Moraes, Dror and Shaw, "Parallel random
 * numbers: as easy as 1, 2, 3", SC 2011) with key (seed & 0xffffffff,
 * seed >> 32) on counter (2 (j / 16) + (j / 4) % 2, i, h, b) -- key j,
 * query row i within its sequence, query head h, batch entry (packed:
 * sequence) b.  The four output words are read as eight 16-bit halves (half
 * 2m = low 16 bits of word m, half 2m + 1 = its high 16 bits); key j takes
 * half 4 ((j / 8) % 2) + j % 4 and is kept iff that half is at least
 * floor(dropout_p * 2^16) (dropout_p is resolved to 2^-16).  The same
 * (seed, b, h, i, j) always gives the same decision, whatever the layout or
 * the launch.
 *
 * Every other argument, layout, ownership and error rule is that of
 * mi_attn_fwd.  dropout_p outside [0, 1) (or NaN) returns MI_ATTN_ERR_ARG
 * before any HIP call; dropout_p = 0 runs mi_attn_fwd.
 */
MI_ATTN_API mi_attn_status_t mi_attn_fwd_dropout(const void* q, const void* k, const void* v,
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
                             int32_t causal, double dropout_p, uint64_t seed,
                             struct ihipStream_t* stream);

/*
 * mi_attn_rotary -- rotary position embedding of Q or K, in place.
 *
 * The "Training integration" tutorial, section 4 (4.1-4.3): the rotary
 * embedding applied to Q and K before attention, with a rotary dimension, a
 * base frequency (10000 in the tutorial), the GPT-NeoX layout or the GPT-J
 * layout, and a position offset for generation with a KV cache (the new
 * tokens' positions start at the cache length).  Pair k (k < rotary_dim/2) of
 * a row at position p turns by a = p * base^(-2k / rotary_dim):
 * (x, y) -> (x cos a - y sin a, x sin a + y cos a).  interleaved = 0
 * (GPT-NeoX): pair k is features (k, k + rotary_dim/2); interleaved = 1
 * (GPT-J): features (2k, 2k + 1).  Features rotary_dim .. head_dim-1 are
 * not touched.  The xPos scaling of section 4.4 is not provided.
 *
 * x          dense [batch, heads, seqlen, head_dim] through strides (NULL:
 *            contiguous), or packed [T, heads, head_dim] when cu_seqlens
 *            (device int32 [batch + 1]) is given; seqlen is then the longest
 *            sequence.  F16 or BF16; rotated in fp32 and rounded back to
 *            nearest even.
 * positions  row t of sequence b sits at position_offset +
 *            position_offsets[b] + t (position_offsets: device int32
 *            [batch], or NULL for 0).
 * rotary_dim a multiple of 16, at most head_dim and 256.
 * stream     hipStream_t to enqueue on (NULL: default stream).
 *
 * Ownership: the caller owns x, cu_seqlens and position_offsets; nothing is
 * retained.  Errors: a dtype other than F16/BF16 -> MI_ATTN_ERR_DTYPE; a
 * negative size, batch > 65535 or heads > 4 * 65535 -> MI_ATTN_ERR_SHAPE; an unsupported
 * rotary_dim -> MI_ATTN_ERR_UNSUPPORTED; base not finite and positive or
 * interleaved not 0/1 -> MI_ATTN_ERR_ARG; x not 16-byte aligned, strides
 * not multiples of 8 elements, or rows/heads that overlap ->
 * MI_ATTN_ERR_LAYOUT; all checked before any HIP call.  batch or seqlen 0
 * is a no-op.
 */
MI_ATTN_API mi_attn_status_t mi_attn_rotary(void* x, mi_attn_dtype_t dtype, int32_t batch,
                                            int32_t heads, int32_t seqlen, int32_t head_dim,
                                            const mi_attn_strides_t* strides,
                                            const int32_t* cu_seqlens,
                                            const int32_t* position_offsets,
                                            int64_t position_offset, int32_t rotary_dim,
                                            double base, int32_t interleaved,
                                            struct ihipStream_t* stream);

/*
 * mi_attn_rotary_qk -- mi_attn_rotary of Q and K together, in one launch.
 *
 * The same tutorial section applies the embedding to both Q and K at the
 * same positions.  q is [batch, hq, seqlen, head_dim] and k is [batch, hkv,
 * seqlen, head_dim] (each through its own strides, NULL: contiguous), or
 * both packed [T, hq | hkv, head_dim] with the shared cu_seqlens; positions,
 * rotary_dim, base and interleaved as for mi_attn_rotary, and the result is
 * that of mi_attn_rotary on q and then on k.  q and k must not overlap in
 * memory (q == k is rejected with MI_ATTN_ERR_LAYOUT).  hkv < 1 ->
 * MI_ATTN_ERR_SHAPE; every other check, ownership and error rule as for
 * mi_attn_rotary, applied to both tensors.
 */
MI_ATTN_API mi_attn_status_t mi_attn_rotary_qk(void* q, void* k, mi_attn_dtype_t dtype,
                                               int32_t batch, int32_t hq, int32_t hkv,
                                               int32_t seqlen, int32_t head_dim,
                                               const mi_attn_strides_t* q_strides,
                                               const mi_attn_strides_t* k_strides,
                                               const int32_t* cu_seqlens,
                                               const int32_t* position_offsets,
                                               int64_t position_offset, int32_t rotary_dim,
                                               double base, int32_t interleaved,
                                               struct ihipStream_t* stream);

/* Static, human-readable text for a status code (never NULL). */
MI_ATTN_API const char* mi_attn_status_string(mi_attn_status_t status);

/* MI_ATTN_ABI_VERSION of the loaded library. */
MI_ATTN_API int32_t mi_attn_version(void);

/* The hipError_t of the last MI_ATTN_ERR_HIP returned on this thread, 0 if
 * none. */
MI_ATTN_API int32_t mi_attn_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MI_ATTN_H */
