/*
 * iq.h -- C ABI of libiq: IsoQuant 3-bit KV compression and decode attention
 * computed directly on the packed codes, for AMD MI355X (gfx950).
 *
 * Method: "RotaryQuant: Fitting 120B MoE Models on Consumer Hardware via
 * Fused Compressed-Space Attention" (arXiv 2608.08081), Abstract.  Each
 * key/value head vector (d = 128) goes through a Walsh-Hadamard transform,
 * then a block-diagonal SO(4) rotation (256 stored parameters per head),
 * then 3-bit scalar quantization; attention then runs on the packed 3-bit
 * tensors without materialising full-precision KV.
 *
 * Conventions (all entry points):
 *   - Return IQ_OK (0) or a negative IQ_E* code; iq_last_error() then holds
 *     a message (thread-local, valid until the next call on that thread).
 *   - Pointers are DEVICE pointers unless the argument is marked "host".
 *     All device buffers are owned by the caller; the library never
 *     allocates, frees or synchronises inside these calls.
 *   - Work is enqueued on `stream` (a hipStream_t passed as void*; NULL is
 *     the default stream) and is complete when the stream reaches it.
 *   - Every argument is validated before anything is launched, so an error
 *     return other than IQ_EHIP means nothing was enqueued.  A HIP error left
 *     pending by earlier, unrelated work is cleared before the launches.
 *   - head_dim must be 128 and bits must be 3 (IQ_EUNSUPPORTED otherwise).
 *
 * Data layouts (the pages only say "packed 3-bit tensors"; these are this
 * library's readings):
 *   rotation params  float[.][32][8] per head: block b acts on coordinates
 *                    4b..4b+3 as v -> qL * v * conj(qR) (Hamilton product,
 *                    components (w,x,y,z)), params[b][0:4] = qL,
 *                    params[b][4:8] = qR.  Quaternions are normalised before
 *                    use.  The rotation is R = blockdiag(M_b) * H with H the
 *                    normalised Sylvester Walsh-Hadamard matrix.
 *   quantizer        x' = R x; s = max|x'| / 3.5 (fp32, one per vector);
 *                    code = clamp(floor(x'/s + 4), 0, 7); level s*(c-3.5);
 *                    a zero vector gives s = 0 and all codes 4.
 *   code record      48 bytes per vector, one little-endian bit stream:
 *                    bit b of the code of coordinate i is stream bit 3i + b,
 *                    and byte k holds stream bits 8k..8k+7 (bit 8k + m is
 *                    bit m of byte k).  Bytes 3g..3g+2 hold the codes of
 *                    coordinates 8g..8g+7 as sum_j c_(8g+j) * 8^j.
 *   KV cache         codes uint8[n_seq][n_heads][cache_cap][48] and scales
 *                    float[n_seq][n_heads][cache_cap], contiguous.
 */
#ifndef IQ_H
#define IQ_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  IQ_OK = 0,
  IQ_EINVAL = -1,        /* null pointer, bad count, stride or shape */
  IQ_EUNSUPPORTED = -2,  /* head_dim != 128, bits != 3, unknown dtype */
  IQ_EWORKSPACE = -3,    /* workspace missing or smaller than required */
  IQ_EHIP = -4           /* a HIP runtime call or kernel launch failed; kernels of the call
                            enqueued before the failing launch may still run, and the
                            call's outputs are then undefined */
};

enum { IQ_F32 = 0, IQ_BF16 = 1 };

/* Record formats: the pages' 3-bit uniform codes and variants with the same rotation (see
 * iq_quantize_kv_format).  Record size 16 * bits bytes. */
enum {
  IQ_FMT_U3 = 0,    /* 3-bit uniform mid-rise, s = max|x'| / 3.5 (the default), 48 bytes */
  IQ_FMT_U2 = 1,    /* 2-bit uniform mid-rise, s = max|x'| / 1.5, 32 bytes */
  IQ_FMT_U4 = 2,    /* 4-bit uniform mid-rise, s = max|x'| / 7.5, 64 bytes */
  IQ_FMT_LM3 = 3,   /* 3-bit Lloyd-Max levels of a unit Gaussian scaled by the RMS, 48 bytes */
  IQ_FMT_A3 = 4     /* 3-bit asymmetric: 8 levels from the vector's min to its max, 48 bytes,
                       and two fp32 per vector (step, min) in the scales arrays */
};

#define IQ_HEAD_DIM 128
#define IQ_BITS 3
#define IQ_RECORD_BYTES 48
#define IQ_ROT_PARAMS 256

/* Message describing the last error on the calling thread ("" if none). */
const char* iq_last_error(void);

/*
 * iq_make_rotation -- draw rotation parameters (host only, no GPU work).
 * Source: Abstract (each head stores 256 rotation parameters).  How the parameters
 * are drawn is not stated; this draws each block's left and right
 * quaternions uniformly on the 3-sphere: SplitMix64 (Steele, Lea, Flood
 * 2014) outputs z_i = mix(seed + (i+1)*0x9E3779B97F4A7C15) give uniforms
 * v = (z >> 11) * 2^-52 - 1 on [-1, 1); Marsaglia's 1972 method turns them
 * into a point on S^3 (x1,x2 with s1 = x1^2+x2^2 < 1; x3,x4 with
 * 0 < s2 = x3^2+x4^2 < 1; then (x1, x2, x3 f, x4 f), f = sqrt((1-s1)/s2)),
 * in the order head, block, qL then qR; components rounded to fp32.
 *   seed         any 64-bit value; the output is a pure function of it.
 *   n_heads      >= 1.
 *   params_host  host buffer of n_heads*256 floats, [n_heads][32][8].
 * Errors: IQ_EINVAL for n_heads < 1 or a NULL buffer.
 */
int iq_make_rotation(uint64_t seed, int32_t n_heads, float* params_host);

/*
 * iq_quantize_kv -- rotate, 3-bit quantize and pack K and/or V vectors into
 * the KV cache.  Source: Abstract (WHT, then block-diagonal SO(4), then
 * 3-bit scalar quantization; packed 3-bit tensors).
 *   k, v         input vectors, dtype IQ_F32 or IQ_BF16, element (s,h,t,i)
 *                at k[s*stride_seq + h*stride_head + t*stride_tok + i]
 *                (strides in elements, coordinates i contiguous).  Either k
 *                or v may be NULL, and that side is skipped (its code and
 *                scale pointers may then be NULL too).
 *   n_seq        sequences (or layers) >= 1; n_heads >= 1; n_tokens >= 0
 *                (0 is a no-op).
 *   rot          params of (s,h) at rot + s*rot_stride_seq + h*256 (floats);
 *                rot_stride_seq = 0 shares one set of heads across s.
 *                K and V of a head share its rotation.
 *   k_codes ...  cache arrays [n_seq][n_heads][cache_cap][48] / [...][cache_cap];
 *                token t is written at cache position tok_offset + t.
 *   cache_cap    >= tok_offset + n_tokens.
 * Errors: IQ_EINVAL (NULL where required, non-positive sizes, negative
 * strides or offset, tok_offset + n_tokens > cache_cap, misaligned input
 * pointers or strides that are not multiples of 8 elements for bf16 / 4
 * for f32), IQ_EUNSUPPORTED, IQ_EHIP.
 */
int iq_quantize_kv(const void* k, const void* v, int32_t dtype,
                   int64_t n_seq, int32_t n_heads, int64_t n_tokens,
                   int64_t stride_seq, int64_t stride_head, int64_t stride_tok,
                   const float* rot, int64_t rot_stride_seq,
                   uint8_t* k_codes, float* k_scales,
                   uint8_t* v_codes, float* v_scales,
                   int64_t cache_cap, int64_t tok_offset,
                   int32_t head_dim, int32_t bits, void* stream);

/*
 * iq_quantize_kv_format -- iq_quantize_kv for any record format IQ_FMT_*.
 * Source: Abstract (rotation, then scalar quantization with one scale per
 * vector, packed); the 2- and 4-bit and Lloyd-Max variants are readings that
 * keep the rotation and change the scalar quantizer:
 *   IQ_FMT_U2 / IQ_FMT_U4  s = max|x'| / (2^(b-1) - 1/2),
 *                          code = clamp(floor(x'/s + 2^(b-1)), 0, 2^b - 1),
 *                          level s * (code - (2^b - 1)/2);
 *   IQ_FMT_LM3             sigma = |x'| / sqrt(128) (stored as the scale), the
 *                          code of the nearest of the levels +-0.2451,
 *                          +-0.7560, +-1.344, +-2.152 (J. Max's Lloyd-Max
 *                          quantizer of a unit Gaussian) to x'/sigma, ties up;
 *                          level sigma * L[code]; sigma = 0 gives code 4;
 *   IQ_FMT_A3              the asymmetric alternative: m = min x', M = max x',
 *                          s = (M - m) / 7, code = clamp(floor((x' - m)/s + 1/2),
 *                          0, 7), level m + s * code; M = m gives s = 0 and
 *                          code 0.  (s, m) are stored as two floats per vector:
 *                          scales float[n_seq][n_heads][cache_cap][2], 8-byte
 *                          aligned.
 * Records are one little-endian bit stream of b bits per code (bit j of the
 * code of coordinate i is stream bit b*i + j): codes uint8[n_seq][n_heads]
 * [cache_cap][16*b].  IQ_FMT_U3 is exactly iq_quantize_kv.  4-bit codes must
 * be 8-byte aligned.  Other arguments and errors as iq_quantize_kv, with
 * format in place of bits (IQ_EUNSUPPORTED for an unknown format).
 */
int iq_quantize_kv_format(const void* k, const void* v, int32_t dtype,
                          int64_t n_seq, int32_t n_heads, int64_t n_tokens,
                          int64_t stride_seq, int64_t stride_head, int64_t stride_tok,
                          const float* rot, int64_t rot_stride_seq,
                          uint8_t* k_codes, float* k_scales,
                          uint8_t* v_codes, float* v_scales,
                          int64_t cache_cap, int64_t tok_offset,
                          int32_t head_dim, int32_t format, void* stream);

/*
 * iq_decode_workspace_bytes -- device workspace that iq_decode_attention
 * (and iq_decode_attention_append, and iq_decode_attention_multi with batch
 * times n_q_tokens as batch) needs with these sizes on the current device:
 * the split plan (chunk size and each sequence's first chunk) and the
 * split-K partial results.  Source: Abstract (attention computed on the
 * packed tensors); splitting the context over work-groups and merging their
 * partial softmax results is this library's way of running that attention
 * on a whole GPU.  The kernels choose the chunk size on the device from the
 * sequence lengths, so that the batch's chunks fill a fixed number of rounds
 * of work-groups per (KV head, group of up to 8 query heads): the bound
 * depends only on these sizes (n_kv_heads sets the number of such columns)
 * and the device's compute-unit count.  Negative IQ_E* code on invalid sizes.
 */
int64_t iq_decode_workspace_bytes(int32_t batch, int32_t n_q_heads,
                                  int32_t n_kv_heads, int64_t cache_cap);

/*
 * iq_decode_attention -- one decode step of attention computed on the
 * packed cache.  Source: Abstract (attention runs on the packed 3-bit
 * tensors; no full-precision K/V is ever formed).  The
 * query is rotated into the compressed space, codes are turned into
 * numbers only in registers, softmax is online and split over the
 * sequence, V is accumulated in rotated space and rotated back once per
 * (output row, chunk) partial, never per token.
 *   q            [batch][n_q_heads][128], q_dtype IQ_F32 or IQ_BF16,
 *                16-byte aligned.
 *   k_*, v_*     the cache written by iq_quantize_kv, [batch][n_kv_heads]
 *                [cache_cap][48] codes and [batch][n_kv_heads][cache_cap]
 *                scales.
 *   rot          params of (b,g) at rot + b*rot_stride_batch + g*256;
 *                rot_stride_batch = 0 shares them across the batch (a
 *                layer-stacked call passes n_kv_heads*256).
 *   seq_lens     device int32[batch], 0 <= len <= cache_cap; NULL means
 *                every sequence has cache_cap tokens.  Positions >= len are
 *                never read into the result.
 *   query head h attends with KV head h / (n_q_heads / n_kv_heads).
 *   sm_scale     softmax scale; <= 0 selects 1/sqrt(128).
 *   out          float [batch][n_q_heads][128]; a sequence with len 0 gets
 *                zeros.
 *   workspace    device buffer of at least iq_decode_workspace_bytes(...)
 *                bytes, 256-byte aligned, used only during the call.
 * Errors: IQ_EINVAL (NULL pointers, sizes < 1, n_q_heads % n_kv_heads != 0,
 * cache_cap > 83886016 (= 0xF0000000 / 48 - 64), negative stride, misaligned
 * pointers: q 16 bytes, the rest 4), IQ_EWORKSPACE,
 * IQ_EUNSUPPORTED, IQ_EHIP.
 */
int iq_decode_attention(const void* q, int32_t q_dtype,
                        const uint8_t* k_codes, const float* k_scales,
                        const uint8_t* v_codes, const float* v_scales,
                        const float* rot, int64_t rot_stride_batch,
                        const int32_t* seq_lens,
                        int32_t batch, int32_t n_q_heads, int32_t n_kv_heads,
                        int64_t cache_cap, float sm_scale, float* out,
                        void* workspace, int64_t workspace_bytes,
                        int32_t head_dim, int32_t bits, void* stream);

/*
 * iq_decode_attention_noalloc -- iq_decode_attention for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  It takes no workspace: the split plan and
 * the split-K partials live in a device array of IQ_NOALLOC_SCRATCH_BYTES
 * inside the library, one per device, which holds it until the process ends.
 * The call itself allocates and frees nothing.
 *   Arguments, kernels and results as iq_decode_attention (the output is the
 *   same bit for bit), without workspace and workspace_bytes.
 *   Every call on a device shares that device's array: calls that overlap
 *   on one device (on other streams or from other host threads) race and give
 *   undefined results.  Nothing in the array needs clearing between calls.
 * Errors: as iq_decode_attention; IQ_EWORKSPACE when the sizes need more than
 * IQ_NOALLOC_SCRATCH_BYTES (plan head plus 520 bytes per query head per work
 * item of the split: e.g. 48 stacked 32K layers of 32 query heads need about
 * 3.2 MB), IQ_EHIP when the array's device address cannot be looked up.
 */
#define IQ_NOALLOC_SCRATCH_BYTES (8 << 20)
int iq_decode_attention_noalloc(const void* q, int32_t q_dtype,
                                const uint8_t* k_codes, const float* k_scales,
                                const uint8_t* v_codes, const float* v_scales,
                                const float* rot, int64_t rot_stride_batch,
                                const int32_t* seq_lens,
                                int32_t batch, int32_t n_q_heads, int32_t n_kv_heads,
                                int64_t cache_cap, float sm_scale, float* out,
                                int32_t head_dim, int32_t bits, void* stream);

/*
 * iq_decode_attention_format -- iq_decode_attention on a cache written by
 * iq_quantize_kv_format with the same format (codes [batch][n_kv_heads]
 * [cache_cap][16*b]).  Source: Abstract (attention on the packed tensors).
 * IQ_FMT_U3 runs the same kernels as iq_decode_attention; the other formats
 * run variants of its matrix-core kernel (IQ_FMT_LM3 through tables of its
 * levels) with the same split of the context and the same combine.
 * IQ_FMT_A3 scales are (s, m) pairs, float[batch][n_kv_heads][cache_cap][2],
 * 8-byte aligned.  IQ_FMT_U4 allows cache_cap <= 62914432 (= 0xF0000000 / 64
 * - 64).  Other arguments and errors as
 * iq_decode_attention, with format in place of bits.
 */
int iq_decode_attention_format(const void* q, int32_t q_dtype,
                               const uint8_t* k_codes, const float* k_scales,
                               const uint8_t* v_codes, const float* v_scales,
                               const float* rot, int64_t rot_stride_batch,
                               const int32_t* seq_lens,
                               int32_t batch, int32_t n_q_heads, int32_t n_kv_heads,
                               int64_t cache_cap, float sm_scale, float* out,
                               void* workspace, int64_t workspace_bytes,
                               int32_t head_dim, int32_t format, void* stream);

/*
 * iq_decode_attention_multi -- attention of n_q_tokens new query tokens per
 * sequence on the packed cache (chunked prefill, or checking several drafted
 * tokens at once).  Source: Abstract (attention computed on the packed 3-bit
 * tensors); several query tokens per step is this library's extension.
 *   q, out       [batch][n_q_tokens][n_q_heads][128] (q as in
 *                iq_decode_attention; out float).
 *   seq_lens     as in iq_decode_attention: the cached tokens of sequence b,
 *                including its n_q_tokens new ones, which are the last
 *                n_q_tokens positions (written to the cache beforehand, e.g.
 *                by iq_quantize_kv).  NULL means cache_cap.
 *   Query token i of sequence b sits at position L - n_q_tokens + i
 *   (L = seq_lens[b]) and attends to positions 0 .. L - n_q_tokens + i
 *   (causal); a token whose position is below 0 gets zeros.
 *   workspace    at least iq_decode_workspace_bytes(batch * n_q_tokens,
 *                n_q_heads, n_kv_heads, cache_cap) bytes, 256-byte aligned.
 *   Other arguments as in iq_decode_attention; n_q_tokens = 1 is exactly
 *   iq_decode_attention.
 * Errors: as iq_decode_attention; IQ_EINVAL also for n_q_tokens < 1 or
 * batch * n_q_tokens > 65535.
 */
int iq_decode_attention_multi(const void* q, int32_t q_dtype, int32_t n_q_tokens,
                              const uint8_t* k_codes, const float* k_scales,
                              const uint8_t* v_codes, const float* v_scales,
                              const float* rot, int64_t rot_stride_batch,
                              const int32_t* seq_lens,
                              int32_t batch, int32_t n_q_heads, int32_t n_kv_heads,
                              int64_t cache_cap, float sm_scale, float* out,
                              void* workspace, int64_t workspace_bytes,
                              int32_t head_dim, int32_t bits, void* stream);

/*
 * iq_decode_attention_append -- one decode step with the step's new token
 * appended in the same launch.  Source: Abstract (quantised KV written as
 * packed 3-bit tensors, attention computed on them).  For every sequence b
 * and KV head g, the new key and value vectors k_new[b][g], v_new[b][g] are
 * rotated, quantised and written into the cache at token positions[b]
 * (exactly as iq_quantize_kv would), and attention then covers tokens
 * 0 .. positions[b], the new one included.  The result equals
 * iq_quantize_kv of that token followed by iq_decode_attention with
 * seq_lens = positions + 1.
 *   k_new, v_new   [batch][n_kv_heads][128], new_dtype IQ_F32 or IQ_BF16,
 *                  element strides new_stride_seq and new_stride_head (the
 *                  128 coordinates contiguous), 16-byte aligned with strides
 *                  a multiple of 16 bytes.
 *   positions      device int32[batch], ragged: each sequence has its own.
 *                  A position outside [0, cache_cap) skips the sequence:
 *                  nothing is written and its output rows are zeros.
 *   k_codes ...    the cache (written at the new positions, read below them).
 *   other arguments as in iq_decode_attention; the workspace size is the
 *   same (iq_decode_workspace_bytes).
 * Errors: as iq_decode_attention, plus IQ_EINVAL for NULL k_new / v_new /
 * positions, negative or misaligned strides; IQ_EUNSUPPORTED for an
 * unknown new_dtype.
 */
int iq_decode_attention_append(const void* q, int32_t q_dtype,
                               const void* k_new, const void* v_new, int32_t new_dtype,
                               int64_t new_stride_seq, int64_t new_stride_head,
                               const int32_t* positions,
                               uint8_t* k_codes, float* k_scales,
                               uint8_t* v_codes, float* v_scales,
                               const float* rot, int64_t rot_stride_batch,
                               int32_t batch, int32_t n_q_heads, int32_t n_kv_heads,
                               int64_t cache_cap, float sm_scale, float* out,
                               void* workspace, int64_t workspace_bytes,
                               int32_t head_dim, int32_t bits, void* stream);

/*
 * Isotropy diagnostics.  Source: Abstract (the Walsh-Hadamard transform
 * followed by block-diagonal SO(4) rotations is applied so that every
 * vector's coordinates look alike before 3-bit scalar quantization with one
 * scale per vector).  These calls measure that effect for the method's
 * transform and the variants it is compared with.
 */
enum {
  IQ_T_NONE = 0,      /* y = x */
  IQ_T_WHT = 1,       /* y = H x (normalised Sylvester Walsh-Hadamard) */
  IQ_T_SO4 = 2,       /* y = blockdiag(M_b) x (the SO(4) blocks alone) */
  IQ_T_WHT_SO4 = 3,   /* y = blockdiag(M_b) H x (the method's rotation) */
  IQ_T_DENSE = 4      /* y = T x with a caller-given 128x128 matrix T */
};
enum { IQ_N_STATS = 260 };

/*
 * iq_isotropy_workspace_bytes -- device workspace iq_isotropy_stats needs
 * for these sizes (partial sums of every 256 tokens).  Negative IQ_E* code
 * on invalid sizes.
 */
int64_t iq_isotropy_workspace_bytes(int64_t n_seq, int32_t n_heads, int64_t n_tokens);

/*
 * iq_isotropy_stats -- statistics of y = T x over the tokens of every
 * (sequence, head).
 *   x            [n_seq][n_heads][n_tokens][128] (element strides; the last
 *                dimension contiguous), dtype IQ_F32 or IQ_BF16, 16-byte
 *                aligned with strides a multiple of 16 bytes.
 *   transform    IQ_T_*.
 *   rot          SO(4) params of (s,h) at rot + s*rot_stride_seq + h*256
 *                (IQ_T_SO4, IQ_T_WHT_SO4; otherwise unused and may be NULL).
 *   dense        row-major T of (s,h) at dense + s*dense_stride_seq +
 *                h*16384 (IQ_T_DENSE; otherwise unused and may be NULL).
 *   stats        double [n_seq][n_heads][IQ_N_STATS]:
 *                  [0:128]   kurtosis m4/m2^2 of each coordinate of y over
 *                            the tokens (population central moments);
 *                  [128:256] variance m2 of each coordinate;
 *                  [256]     kurtosis of each vector's 128 entries, averaged
 *                            over the tokens;
 *                  [257]     3-bit quantization error of y (the quantizer
 *                            above), sum |y - y_hat|^2 / sum |y|^2;
 *                  [258]     peak-to-average power ratio 128 max_i y_i^2 /
 *                            |y|^2, averaged over the nonzero vectors;
 *                  [259]     n_tokens.
 *                A variance at most 1e-9 times the mean square of the same
 *                values counts as zero, and its kurtosis is reported as 0;
 *                a zero denominator gives 0; n_tokens = 0 gives all zeros.
 *   workspace    device buffer of at least iq_isotropy_workspace_bytes(...)
 *                bytes, 256-byte aligned, used only during the call.
 * Errors: IQ_EINVAL (NULL pointers, sizes out of range, negative strides,
 * misalignment, a missing rot or dense for the transform), IQ_EUNSUPPORTED
 * (dtype or transform), IQ_EWORKSPACE, IQ_EHIP.
 */
int iq_isotropy_stats(const void* x, int32_t dtype, int64_t n_seq, int32_t n_heads, int64_t n_tokens,
                      int64_t stride_seq, int64_t stride_head, int64_t stride_tok,
                      int32_t transform, const float* rot, int64_t rot_stride_seq,
                      const float* dense, int64_t dense_stride_seq,
                      double* stats, void* workspace, int64_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* IQ_H */
