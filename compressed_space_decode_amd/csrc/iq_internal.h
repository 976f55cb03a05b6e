// Internal interface between the C-ABI entry points and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace iq {

void set_error(const char* fmt, ...) __attribute__((format(printf, 1, 2)));
void clear_error();

// One side (K or V) of a quantize call.
struct QuantSide {
  const void* src;      // input vectors (bf16 bits or f32)
  uint8_t* codes;       // [n_seq][n_heads][cap][48]
  float* scales;        // [n_seq][n_heads][cap]
};

struct QuantizeLaunch {
  QuantSide side[2];    // K, V (src == nullptr: side skipped)
  int bf16;
  int64_t n_seq;
  int n_heads;
  int64_t n_tokens;
  int64_t stride_seq, stride_head, stride_tok;   // elements
  const float* rot;
  int64_t rot_stride_seq;                        // floats
  int64_t cache_cap, tok_offset;
};

hipError_t launch_quantize(const QuantizeLaunch& a, hipStream_t stream);
// Record format IQ_FMT_* (IQ_FMT_U3 is launch_quantize).
hipError_t launch_quantize_format(const QuantizeLaunch& a, int format, hipStream_t stream);

// Isotropy statistics of one set of vectors after a transform (iq_isotropy_stats).
struct DiagLaunch {
  const void* x;
  int bf16;
  int64_t n_seq;
  int n_heads;
  int64_t n_tokens;
  int64_t stride_seq, stride_head, stride_tok;   // elements
  int mode;                                      // IQ_T_*
  const float* rot;
  int64_t rot_stride_seq;                        // floats
  const float* dense;
  int64_t dense_stride_seq;                      // floats
  double* stats;                                 // [n_seq][n_heads][IQ_N_STATS]
  void* workspace;
};

int64_t diag_workspace_bytes(int64_t n_seq, int n_heads, int64_t n_tokens);
hipError_t launch_diag(const DiagLaunch& a, hipStream_t stream);

struct DecodeLaunch {
  const void* q;
  int q_bf16;
  const uint8_t* k_codes;
  const float* k_scales;
  const uint8_t* v_codes;
  const float* v_scales;
  const float* rot;
  int64_t rot_stride_batch;
  const int32_t* seq_lens;
  int batch, n_q_heads, n_kv_heads;
  int q_tokens;          // query tokens per sequence (q, out: [batch][q_tokens][n_q_heads][128])
  int format;            // record format IQ_FMT_* of the cache (IQ_FMT_U3: the fast kernels)
  int64_t cache_cap;
  float sm_scale;
  float* out;
  void* workspace;
  // Fused append (iq_decode_attention_append): when positions is not NULL, sequence b's new
  // K/V vectors are quantised into the cache at positions[b] and the lengths are positions + 1
  // (seq_lens is then unused).
  const int32_t* positions;
  const void* k_new;
  const void* v_new;
  int new_bf16;
  int64_t new_stride_seq, new_stride_head;   // elements
};

// Split-K geometry shared by the workspace query and the launch.
struct DecodeGeometry {
  int head_groups;    // ceil(G / 8): query heads are processed 8 at a time
  int target;         // chunks per (KV head, head group) column the kernels aim for
  int x_max;          // grid width: most (sequence, chunk) pairs per column
  int guess_per_seq;  // chunks per sequence when every length is cap (>= 1)
  int64_t plan_bytes; // workspace head: chunk size and first chunk of each sequence
  int64_t workspace_bytes;
};

DecodeGeometry decode_geometry(int batch, int n_q_heads, int n_kv_heads, int64_t cache_cap);

hipError_t launch_decode(const DecodeLaunch& a, const DecodeGeometry& geo, hipStream_t stream);

// Bytes of the workspace that one single-token call with this geometry uses: the plan head and
// x_max partial rows per query head (the workspace query adds room for several query tokens).
inline int64_t decode_single_bytes(const DecodeGeometry& geo, int n_q_heads) {
  return geo.plan_bytes + (int64_t)geo.x_max * n_q_heads * (128 + 2) * 4;
}

// Validation and launch shared by the decode entry points (iq_api.hip).  scratch_call: workspace is
// the library's own scratch of workspace_bytes bytes, which must hold what the call uses.
int decode_entry(const char* fn, const void* q, int32_t q_dtype, int32_t q_tokens, const uint8_t* k_codes,
                 const float* k_scales, const uint8_t* v_codes, const float* v_scales, const float* rot,
                 int64_t rot_stride_batch, const int32_t* seq_lens, int32_t batch, int32_t n_q_heads,
                 int32_t n_kv_heads, int64_t cache_cap, float sm_scale, float* out, void* workspace,
                 int64_t workspace_bytes, int32_t format, void* stream, bool scratch_call);

}  // namespace iq
