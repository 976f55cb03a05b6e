// C-ABI entry points of libiq: argument validation, then kernel launches on
// the caller's stream.  Declarations and documentation: include/iq.h.
#include <cstdarg>
#include <cstdio>

#include "iq.h"
#include "iq_internal.h"

namespace iq {

static thread_local char g_err[512] = "";

void set_error(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
}

void clear_error() { g_err[0] = '\0'; }

}  // namespace iq

namespace {

bool aligned(const void* p, uintptr_t n) { return (reinterpret_cast<uintptr_t>(p) % n) == 0; }

int check_dims(const char* fn, int32_t head_dim, int32_t bits) {
  if (head_dim != IQ_HEAD_DIM) {
    iq::set_error("%s: head_dim must be 128 (got %d)", fn, head_dim);
    return IQ_EUNSUPPORTED;
  }
  if (bits != IQ_BITS) {
    iq::set_error("%s: bits must be 3 (got %d)", fn, bits);
    return IQ_EUNSUPPORTED;
  }
  return IQ_OK;
}

}  // namespace

extern "C" const char* iq_last_error(void) { return iq::g_err; }

namespace {

int check_format(const char* fn, int32_t head_dim, int32_t format) {
  if (head_dim != IQ_HEAD_DIM) {
    iq::set_error("%s: head_dim must be 128 (got %d)", fn, head_dim);
    return IQ_EUNSUPPORTED;
  }
  if (format < IQ_FMT_U3 || format > IQ_FMT_A3) {
    iq::set_error("%s: unknown record format %d", fn, format);
    return IQ_EUNSUPPORTED;
  }
  return IQ_OK;
}

int quantize_impl(const char* fn, const void* k, const void* v, int32_t dtype, int64_t n_seq, int32_t n_heads,
                  int64_t n_tokens, int64_t stride_seq, int64_t stride_head, int64_t stride_tok, const float* rot,
                  int64_t rot_stride_seq, uint8_t* k_codes, float* k_scales, uint8_t* v_codes, float* v_scales,
                  int64_t cache_cap, int64_t tok_offset, int32_t format, void* stream);

}  // namespace

extern "C" int iq_quantize_kv(const void* k, const void* v, int32_t dtype, int64_t n_seq, int32_t n_heads,
                              int64_t n_tokens, int64_t stride_seq, int64_t stride_head, int64_t stride_tok,
                              const float* rot, int64_t rot_stride_seq, uint8_t* k_codes, float* k_scales,
                              uint8_t* v_codes, float* v_scales, int64_t cache_cap, int64_t tok_offset,
                              int32_t head_dim, int32_t bits, void* stream) {
  static const char* fn = "iq_quantize_kv";
  iq::clear_error();
  const int rc = check_dims(fn, head_dim, bits);
  if (rc) return rc;
  return quantize_impl(fn, k, v, dtype, n_seq, n_heads, n_tokens, stride_seq, stride_head, stride_tok, rot,
                       rot_stride_seq, k_codes, k_scales, v_codes, v_scales, cache_cap, tok_offset, IQ_FMT_U3, stream);
}

extern "C" int iq_quantize_kv_format(const void* k, const void* v, int32_t dtype, int64_t n_seq, int32_t n_heads,
                                     int64_t n_tokens, int64_t stride_seq, int64_t stride_head, int64_t stride_tok,
                                     const float* rot, int64_t rot_stride_seq, uint8_t* k_codes, float* k_scales,
                                     uint8_t* v_codes, float* v_scales, int64_t cache_cap, int64_t tok_offset,
                                     int32_t head_dim, int32_t format, void* stream) {
  static const char* fn = "iq_quantize_kv_format";
  iq::clear_error();
  const int rc = check_format(fn, head_dim, format);
  if (rc) return rc;
  return quantize_impl(fn, k, v, dtype, n_seq, n_heads, n_tokens, stride_seq, stride_head, stride_tok, rot,
                       rot_stride_seq, k_codes, k_scales, v_codes, v_scales, cache_cap, tok_offset, format, stream);
}

namespace {

int quantize_impl(const char* fn, const void* k, const void* v, int32_t dtype, int64_t n_seq, int32_t n_heads,
                  int64_t n_tokens, int64_t stride_seq, int64_t stride_head, int64_t stride_tok, const float* rot,
                  int64_t rot_stride_seq, uint8_t* k_codes, float* k_scales, uint8_t* v_codes, float* v_scales,
                  int64_t cache_cap, int64_t tok_offset, int32_t format, void* stream) {
  if (dtype != IQ_F32 && dtype != IQ_BF16) {
    iq::set_error("%s: unknown dtype %d", fn, dtype);
    return IQ_EUNSUPPORTED;
  }
  if (n_seq < 1 || n_seq > 65535 || n_heads < 1 || n_heads > 65535 || n_tokens < 0) {
    iq::set_error("%s: need 1 <= n_seq <= 65535, 1 <= n_heads <= 65535, n_tokens >= 0", fn);
    return IQ_EINVAL;
  }
  if (n_tokens == 0) return IQ_OK;   // nothing to do (empty inputs may have NULL data pointers)
  if (format == IQ_FMT_U4 && ((k && !aligned(k_codes, 8)) || (v && !aligned(v_codes, 8)))) {
    iq::set_error("%s: 4-bit records need 8-byte aligned codes", fn);
    return IQ_EINVAL;
  }
  if (format == IQ_FMT_A3 && ((k && !aligned(k_scales, 8)) || (v && !aligned(v_scales, 8)))) {
    iq::set_error("%s: asymmetric (s, m) scale pairs need 8-byte alignment", fn);
    return IQ_EINVAL;
  }
  if (k == nullptr && v == nullptr) {
    iq::set_error("%s: k and v are both NULL", fn);
    return IQ_EINVAL;
  }
  if ((k && (!k_codes || !k_scales)) || (v && (!v_codes || !v_scales))) {
    iq::set_error("%s: codes/scales output missing for a side that has input", fn);
    return IQ_EINVAL;
  }
  if (rot == nullptr || rot_stride_seq < 0 || stride_seq < 0 || stride_head < 0 || stride_tok < 0) {
    iq::set_error("%s: rot is NULL or a stride is negative", fn);
    return IQ_EINVAL;
  }
  // (n_tokens > cache_cap - tok_offset cannot overflow once 0 <= tok_offset <= cache_cap)
  if (cache_cap < 1 || tok_offset < 0 || tok_offset > cache_cap || n_tokens > cache_cap - tok_offset) {
    iq::set_error("%s: need cache_cap >= 1, tok_offset >= 0, tok_offset + n_tokens <= cache_cap", fn);
    return IQ_EINVAL;
  }
  const int64_t vec_align = dtype == IQ_BF16 ? 8 : 4;   // 16 bytes
  if ((stride_seq % vec_align) || (stride_head % vec_align) || (stride_tok % vec_align) ||
      (k && !aligned(k, 16)) || (v && !aligned(v, 16))) {
    iq::set_error("%s: inputs must be 16-byte aligned with strides a multiple of 16 bytes", fn);
    return IQ_EINVAL;
  }
  if ((k && (!aligned(k_codes, 4) || !aligned(k_scales, 4))) || (v && (!aligned(v_codes, 4) || !aligned(v_scales, 4))) ||
      !aligned(rot, 4)) {
    iq::set_error("%s: codes, scales and rot must be 4-byte aligned", fn);
    return IQ_EINVAL;
  }
  iq::QuantizeLaunch a{};
  a.side[0] = {k, k ? k_codes : nullptr, k ? k_scales : nullptr};
  a.side[1] = {v, v ? v_codes : nullptr, v ? v_scales : nullptr};
  a.bf16 = dtype == IQ_BF16;
  a.n_seq = n_seq;
  a.n_heads = n_heads;
  a.n_tokens = n_tokens;
  a.stride_seq = stride_seq;
  a.stride_head = stride_head;
  a.stride_tok = stride_tok;
  a.rot = rot;
  a.rot_stride_seq = rot_stride_seq;
  a.cache_cap = cache_cap;
  a.tok_offset = tok_offset;
  (void)hipGetLastError();   // an earlier call's error is not this call's
  const hipError_t err = iq::launch_quantize_format(a, format, static_cast<hipStream_t>(stream));
  if (err != hipSuccess) {
    iq::set_error("%s: launch failed: %s", fn, hipGetErrorString(err));
    return IQ_EHIP;
  }
  return IQ_OK;
}

}  // namespace

namespace {

// The decode kernels address one (sequence, KV head)'s codes through a buffer resource with a
// 32-bit byte range and mark blocks that must not be read with the offset 0xF0000000, which has
// to lie past every slice: cache_cap * 48 stays below it with a 64-token margin (83,886,016
// tokens).
constexpr int64_t kMaxCacheCap = 0xF0000000ll / 48 - 64;
constexpr int64_t kMaxCacheCapU4 = 0xF0000000ll / 64 - 64;   // 62,914,432 tokens

int check_decode_sizes(const char* fn, int32_t batch, int32_t n_q_heads, int32_t n_kv_heads, int64_t cache_cap) {
  if (batch < 1 || batch > 65535 || n_q_heads < 1 || n_kv_heads < 1 || cache_cap < 1) {
    iq::set_error("%s: need 1 <= batch <= 65535, n_q_heads >= 1, n_kv_heads >= 1, cache_cap >= 1", fn);
    return IQ_EINVAL;
  }
  if (n_q_heads % n_kv_heads != 0) {
    iq::set_error("%s: n_q_heads (%d) must be a multiple of n_kv_heads (%d)", fn, n_q_heads, n_kv_heads);
    return IQ_EINVAL;
  }
  const int64_t gy = (int64_t)n_kv_heads * ((n_q_heads / n_kv_heads + 7) / 8);
  if (gy > 65535 || (int64_t)batch * n_q_heads > 0x7FFFFFFF || cache_cap > kMaxCacheCap) {
    iq::set_error("%s: sizes exceed the launch limits", fn);
    return IQ_EINVAL;
  }
  return IQ_OK;
}

}  // namespace

extern "C" int64_t iq_decode_workspace_bytes(int32_t batch, int32_t n_q_heads, int32_t n_kv_heads,
                                             int64_t cache_cap) {
  iq::clear_error();
  const int rc = check_decode_sizes("iq_decode_workspace_bytes", batch, n_q_heads, n_kv_heads, cache_cap);
  if (rc) return rc;
  return iq::decode_geometry(batch, n_q_heads, n_kv_heads, cache_cap).workspace_bytes;
}

namespace iq {

// iq_decode_attention (q_tokens = 1) and iq_decode_attention_multi: the batch's q_tokens query
// tokens per sequence run as batch * q_tokens sequences of the kernels that share their cache.
// scratch_call: the workspace is the library's own scratch of workspace_bytes bytes
// (iq_decode_attention_noalloc, one query token): it must hold what this call's kernels use.
int decode_entry(const char* fn, const void* q, int32_t q_dtype, int32_t q_tokens, const uint8_t* k_codes,
                 const float* k_scales, const uint8_t* v_codes, const float* v_scales, const float* rot,
                 int64_t rot_stride_batch, const int32_t* seq_lens, int32_t batch, int32_t n_q_heads,
                 int32_t n_kv_heads, int64_t cache_cap, float sm_scale, float* out, void* workspace,
                 int64_t workspace_bytes, int32_t format, void* stream, bool scratch_call) {
  int rc = IQ_OK;
  if (q_dtype != IQ_F32 && q_dtype != IQ_BF16) {
    iq::set_error("%s: unknown q_dtype %d", fn, q_dtype);
    return IQ_EUNSUPPORTED;
  }
  if (q_tokens < 1 || q_tokens > 65535 || (int64_t)batch * q_tokens > 65535) {
    iq::set_error("%s: need 1 <= n_q_tokens and batch * n_q_tokens <= 65535", fn);
    return IQ_EINVAL;
  }
  rc = check_decode_sizes(fn, batch * q_tokens, n_q_heads, n_kv_heads, cache_cap);
  if (rc) return rc;
  if (!q || !k_codes || !k_scales || !v_codes || !v_scales || !rot || !out) {
    iq::set_error("%s: a required pointer is NULL", fn);
    return IQ_EINVAL;
  }
  if (format == IQ_FMT_U4 && (!aligned(k_codes, 8) || !aligned(v_codes, 8))) {
    iq::set_error("%s: 4-bit records need 8-byte aligned codes", fn);
    return IQ_EINVAL;
  }
  if (format == IQ_FMT_A3 && (!aligned(k_scales, 8) || !aligned(v_scales, 8))) {
    iq::set_error("%s: asymmetric (s, m) scale pairs need 8-byte alignment", fn);
    return IQ_EINVAL;
  }
  // 64-byte records: the kernel's buffer offsets reach cache_cap * 64 (same 64-token margin)
  if (format == IQ_FMT_U4 && cache_cap > kMaxCacheCapU4) {
    iq::set_error("%s: 4-bit records allow cache_cap <= %lld", fn, (long long)kMaxCacheCapU4);
    return IQ_EINVAL;
  }
  if (rot_stride_batch < 0) {
    iq::set_error("%s: rot_stride_batch must be >= 0", fn);
    return IQ_EINVAL;
  }
  if (!aligned(k_codes, 4) || !aligned(v_codes, 4) || !aligned(k_scales, 4) || !aligned(v_scales, 4) ||
      !aligned(rot, 4) || !aligned(out, 4) || !aligned(q, 16) ||
      (seq_lens && !aligned(seq_lens, 4))) {
    iq::set_error("%s: misaligned pointer", fn);
    return IQ_EINVAL;
  }
  const iq::DecodeGeometry geo = iq::decode_geometry(batch * q_tokens, n_q_heads, n_kv_heads, cache_cap);
  if (scratch_call) {
    const int64_t need = iq::decode_single_bytes(geo, n_q_heads);
    if (q_tokens != 1 || need > workspace_bytes) {
      iq::set_error("%s: these sizes need %lld bytes of scratch, more than the library's %lld", fn,
                    (long long)need, (long long)workspace_bytes);
      return IQ_EWORKSPACE;
    }
  } else if (!workspace || workspace_bytes < geo.workspace_bytes || !aligned(workspace, 256)) {
    iq::set_error("%s: workspace must be 256-byte aligned and hold %lld bytes (got %lld)", fn,
                  (long long)geo.workspace_bytes, (long long)workspace_bytes);
    return IQ_EWORKSPACE;
  }
  iq::DecodeLaunch a{};
  a.q = q;
  a.q_bf16 = q_dtype == IQ_BF16;
  a.k_codes = k_codes;
  a.k_scales = k_scales;
  a.v_codes = v_codes;
  a.v_scales = v_scales;
  a.rot = rot;
  a.rot_stride_batch = rot_stride_batch;
  a.seq_lens = seq_lens;
  a.batch = batch;
  a.q_tokens = q_tokens;
  a.format = format;
  a.n_q_heads = n_q_heads;
  a.n_kv_heads = n_kv_heads;
  a.cache_cap = cache_cap;
  a.sm_scale = sm_scale;
  a.out = out;
  a.workspace = workspace;
  (void)hipGetLastError();   // an earlier call's error is not this call's
  const hipError_t err = iq::launch_decode(a, geo, static_cast<hipStream_t>(stream));
  if (err != hipSuccess) {
    iq::set_error("%s: launch failed: %s", fn, hipGetErrorString(err));
    return IQ_EHIP;
  }
  return IQ_OK;
}

}  // namespace iq

extern "C" int iq_decode_attention(const void* q, int32_t q_dtype, const uint8_t* k_codes, const float* k_scales,
                                   const uint8_t* v_codes, const float* v_scales, const float* rot,
                                   int64_t rot_stride_batch, const int32_t* seq_lens, int32_t batch,
                                   int32_t n_q_heads, int32_t n_kv_heads, int64_t cache_cap, float sm_scale,
                                   float* out, void* workspace, int64_t workspace_bytes, int32_t head_dim,
                                   int32_t bits, void* stream) {
  static const char* fn = "iq_decode_attention";
  iq::clear_error();
  const int rc = check_dims(fn, head_dim, bits);
  if (rc) return rc;
  return iq::decode_entry(fn, q, q_dtype, 1, k_codes, k_scales, v_codes, v_scales, rot, rot_stride_batch, seq_lens,
                          batch, n_q_heads, n_kv_heads, cache_cap, sm_scale, out, workspace, workspace_bytes, IQ_FMT_U3,
                          stream, false);
}

extern "C" int iq_decode_attention_format(const void* q, int32_t q_dtype, const uint8_t* k_codes,
                                          const float* k_scales, const uint8_t* v_codes, const float* v_scales,
                                          const float* rot, int64_t rot_stride_batch, const int32_t* seq_lens,
                                          int32_t batch, int32_t n_q_heads, int32_t n_kv_heads, int64_t cache_cap,
                                          float sm_scale, float* out, void* workspace, int64_t workspace_bytes,
                                          int32_t head_dim, int32_t format, void* stream) {
  static const char* fn = "iq_decode_attention_format";
  iq::clear_error();
  const int rc = check_format(fn, head_dim, format);
  if (rc) return rc;
  return iq::decode_entry(fn, q, q_dtype, 1, k_codes, k_scales, v_codes, v_scales, rot, rot_stride_batch, seq_lens,
                          batch, n_q_heads, n_kv_heads, cache_cap, sm_scale, out, workspace, workspace_bytes, format,
                          stream, false);
}

extern "C" int iq_decode_attention_multi(const void* q, int32_t q_dtype, int32_t n_q_tokens,
                                         const uint8_t* k_codes, const float* k_scales, const uint8_t* v_codes,
                                         const float* v_scales, const float* rot, int64_t rot_stride_batch,
                                         const int32_t* seq_lens, int32_t batch, int32_t n_q_heads,
                                         int32_t n_kv_heads, int64_t cache_cap, float sm_scale, float* out,
                                         void* workspace, int64_t workspace_bytes, int32_t head_dim, int32_t bits,
                                         void* stream) {
  static const char* fn = "iq_decode_attention_multi";
  iq::clear_error();
  const int rc = check_dims(fn, head_dim, bits);
  if (rc) return rc;
  return iq::decode_entry(fn, q, q_dtype, n_q_tokens, k_codes, k_scales, v_codes, v_scales, rot, rot_stride_batch,
                          seq_lens, batch, n_q_heads, n_kv_heads, cache_cap, sm_scale, out, workspace, workspace_bytes,
                          IQ_FMT_U3, stream, false);
}

extern "C" int iq_decode_attention_append(const void* q, int32_t q_dtype, const void* k_new, const void* v_new,
                                          int32_t new_dtype, int64_t new_stride_seq, int64_t new_stride_head,
                                          const int32_t* positions, uint8_t* k_codes, float* k_scales,
                                          uint8_t* v_codes, float* v_scales, const float* rot,
                                          int64_t rot_stride_batch, int32_t batch, int32_t n_q_heads,
                                          int32_t n_kv_heads, int64_t cache_cap, float sm_scale, float* out,
                                          void* workspace, int64_t workspace_bytes, int32_t head_dim, int32_t bits,
                                          void* stream) {
  static const char* fn = "iq_decode_attention_append";
  iq::clear_error();
  int rc = check_dims(fn, head_dim, bits);
  if (rc) return rc;
  if ((q_dtype != IQ_F32 && q_dtype != IQ_BF16) || (new_dtype != IQ_F32 && new_dtype != IQ_BF16)) {
    iq::set_error("%s: unknown dtype (q %d, new %d)", fn, q_dtype, new_dtype);
    return IQ_EUNSUPPORTED;
  }
  rc = check_decode_sizes(fn, batch, n_q_heads, n_kv_heads, cache_cap);
  if (rc) return rc;
  if (!q || !k_new || !v_new || !positions || !k_codes || !k_scales || !v_codes || !v_scales || !rot || !out) {
    iq::set_error("%s: a required pointer is NULL", fn);
    return IQ_EINVAL;
  }
  if (rot_stride_batch < 0 || new_stride_seq < 0 || new_stride_head < 0) {
    iq::set_error("%s: strides must be >= 0", fn);
    return IQ_EINVAL;
  }
  const int64_t vec_align = new_dtype == IQ_BF16 ? 8 : 4;   // 16 bytes
  if (!aligned(k_new, 16) || !aligned(v_new, 16) || (new_stride_seq % vec_align) || (new_stride_head % vec_align)) {
    iq::set_error("%s: k_new and v_new must be 16-byte aligned with strides a multiple of 16 bytes", fn);
    return IQ_EINVAL;
  }
  if (!aligned(k_codes, 4) || !aligned(v_codes, 4) || !aligned(k_scales, 4) || !aligned(v_scales, 4) ||
      !aligned(rot, 4) || !aligned(out, 4) || !aligned(q, 16) || !aligned(positions, 4)) {
    iq::set_error("%s: misaligned pointer", fn);
    return IQ_EINVAL;
  }
  const iq::DecodeGeometry geo = iq::decode_geometry(batch, n_q_heads, n_kv_heads, cache_cap);
  if (!workspace || workspace_bytes < geo.workspace_bytes || !aligned(workspace, 256)) {
    iq::set_error("%s: workspace must be 256-byte aligned and hold %lld bytes (got %lld)", fn,
                  (long long)geo.workspace_bytes, (long long)workspace_bytes);
    return IQ_EWORKSPACE;
  }
  iq::DecodeLaunch a{};
  a.q = q;
  a.q_bf16 = q_dtype == IQ_BF16;
  a.k_codes = k_codes;
  a.k_scales = k_scales;
  a.v_codes = v_codes;
  a.v_scales = v_scales;
  a.rot = rot;
  a.rot_stride_batch = rot_stride_batch;
  a.seq_lens = nullptr;
  a.batch = batch;
  a.q_tokens = 1;
  a.n_q_heads = n_q_heads;
  a.n_kv_heads = n_kv_heads;
  a.cache_cap = cache_cap;
  a.sm_scale = sm_scale;
  a.out = out;
  a.workspace = workspace;
  a.positions = positions;
  a.k_new = k_new;
  a.v_new = v_new;
  a.new_bf16 = new_dtype == IQ_BF16;
  a.new_stride_seq = new_stride_seq;
  a.new_stride_head = new_stride_head;
  (void)hipGetLastError();   // an earlier call's error is not this call's
  const hipError_t err = iq::launch_decode(a, geo, static_cast<hipStream_t>(stream));
  if (err != hipSuccess) {
    iq::set_error("%s: launch failed: %s", fn, hipGetErrorString(err));
    return IQ_EHIP;
  }
  return IQ_OK;
}

extern "C" int64_t iq_isotropy_workspace_bytes(int64_t n_seq, int32_t n_heads, int64_t n_tokens) {
  iq::clear_error();
  if (n_seq < 1 || n_seq > 65535 || n_heads < 1 || n_heads > 65535 || n_tokens < 0 || n_tokens > (int64_t)1 << 40) {
    iq::set_error("iq_isotropy_workspace_bytes: need 1 <= n_seq, n_heads <= 65535 and 0 <= n_tokens <= 2^40");
    return IQ_EINVAL;
  }
  return iq::diag_workspace_bytes(n_seq, n_heads, n_tokens);
}

extern "C" int iq_isotropy_stats(const void* x, int32_t dtype, int64_t n_seq, int32_t n_heads, int64_t n_tokens,
                                 int64_t stride_seq, int64_t stride_head, int64_t stride_tok, int32_t transform,
                                 const float* rot, int64_t rot_stride_seq, const float* dense,
                                 int64_t dense_stride_seq, double* stats, void* workspace, int64_t workspace_bytes,
                                 void* stream) {
  static const char* fn = "iq_isotropy_stats";
  iq::clear_error();
  if (dtype != IQ_F32 && dtype != IQ_BF16) {
    iq::set_error("%s: unknown dtype %d", fn, dtype);
    return IQ_EUNSUPPORTED;
  }
  if (transform < IQ_T_NONE || transform > IQ_T_DENSE) {
    iq::set_error("%s: unknown transform %d", fn, transform);
    return IQ_EUNSUPPORTED;
  }
  if (n_seq < 1 || n_seq > 65535 || n_heads < 1 || n_heads > 65535 || n_tokens < 0 || n_tokens > (int64_t)1 << 40) {
    iq::set_error("%s: need 1 <= n_seq, n_heads <= 65535 and 0 <= n_tokens <= 2^40", fn);
    return IQ_EINVAL;
  }
  if (stats == nullptr || !aligned(stats, 8)) {
    iq::set_error("%s: stats is NULL or not 8-byte aligned", fn);
    return IQ_EINVAL;
  }
  if (n_tokens > 0 && x == nullptr) {
    iq::set_error("%s: x is NULL", fn);
    return IQ_EINVAL;
  }
  if ((transform == IQ_T_SO4 || transform == IQ_T_WHT_SO4) && (rot == nullptr || rot_stride_seq < 0 || !aligned(rot, 4))) {
    iq::set_error("%s: this transform needs rot (4-byte aligned, rot_stride_seq >= 0)", fn);
    return IQ_EINVAL;
  }
  if (transform == IQ_T_DENSE && (dense == nullptr || dense_stride_seq < 0 || !aligned(dense, 4))) {
    iq::set_error("%s: IQ_T_DENSE needs dense (4-byte aligned, dense_stride_seq >= 0)", fn);
    return IQ_EINVAL;
  }
  if (stride_seq < 0 || stride_head < 0 || stride_tok < 0) {
    iq::set_error("%s: a stride is negative", fn);
    return IQ_EINVAL;
  }
  const int64_t vec_align = dtype == IQ_BF16 ? 8 : 4;   // 16 bytes
  if ((stride_seq % vec_align) || (stride_head % vec_align) || (stride_tok % vec_align) || (x && !aligned(x, 16))) {
    iq::set_error("%s: x must be 16-byte aligned with strides a multiple of 16 bytes", fn);
    return IQ_EINVAL;
  }
  const int64_t need = iq::diag_workspace_bytes(n_seq, n_heads, n_tokens);
  if (!workspace || workspace_bytes < need || !aligned(workspace, 256)) {
    iq::set_error("%s: workspace must be 256-byte aligned and hold %lld bytes (got %lld)", fn, (long long)need,
                  (long long)workspace_bytes);
    return IQ_EWORKSPACE;
  }
  iq::DiagLaunch a{};
  a.x = x;
  a.bf16 = dtype == IQ_BF16;
  a.n_seq = n_seq;
  a.n_heads = n_heads;
  a.n_tokens = n_tokens;
  a.stride_seq = stride_seq;
  a.stride_head = stride_head;
  a.stride_tok = stride_tok;
  a.mode = transform;
  a.rot = rot;
  a.rot_stride_seq = rot_stride_seq;
  a.dense = dense;
  a.dense_stride_seq = dense_stride_seq;
  a.stats = stats;
  a.workspace = workspace;
  (void)hipGetLastError();   // an earlier call's error is not this call's
  const hipError_t err = iq::launch_diag(a, static_cast<hipStream_t>(stream));
  if (err != hipSuccess) {
    iq::set_error("%s: launch failed: %s", fn, hipGetErrorString(err));
    return IQ_EHIP;
  }
  return IQ_OK;
}
