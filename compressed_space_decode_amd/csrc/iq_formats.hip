// Quantizer variants with the same rotation: 2- and 4-bit uniform codes and
// the 8-level Lloyd-Max codebook with an RMS scale.
//
// Method: "RotaryQuant: Fitting 120B MoE Models on Consumer Hardware via Fused
// Compressed-Space Attention" (arXiv 2608.08081), Abstract: Walsh-Hadamard
// transform and block-diagonal SO(4) rotation, then scalar quantization of
// every coordinate with one scale per vector, stored packed.  The pages use
// 3 bits; these formats change only the scalar quantizer:
//   IQ_FMT_U2, IQ_FMT_U4  uniform mid-rise, 2^b levels, s = max|x'| / (2^(b-1) - 1/2),
//                         code = clamp(floor(x'/s + 2^(b-1)), 0, 2^b - 1);
//   IQ_FMT_LM3            the Lloyd-Max levels of a unit Gaussian as J. Max printed them
//                         (+-0.2451, +-0.7560, +-1.344, +-2.152), scaled by the RMS
//                         sigma = |x'| / sqrt(128); the code of the nearest level (ties up);
//   IQ_FMT_A3             asymmetric (min/max, as in the KIVI-style schemes the pages cite):
//                         m = min x', s = (max x' - m) / 7, code = clamp(floor((x' - m)/s
//                         + 1/2), 0, 7), level m + s code; (s, m) stored per vector.
// Records: one little-endian bit stream of b bits per code, 16 b bytes.
//
// Work split as in the 3-bit quantize kernel: 8 lanes per vector, lane e holds
// chunk c = chunk_of(e), coordinates 16c..16c+15, i.e. the 2b bytes 2b*c .. 2b*c +
// 2b - 1 of the record.
#include "iq.h"
#include "iq_internal.h"
#include "iq_vector.h"

namespace iq {
namespace {

constexpr int kThreads = 256;
constexpr int kVecPerStep = kThreads / 8;
constexpr int kTokPerGroup = 256;

// Max's 8 levels, ascending, and the midpoints between consecutive levels.
constexpr float kLM[8] = {-2.152f, -1.344f, -0.7560f, -0.2451f, 0.2451f, 0.7560f, 1.344f, 2.152f};

__device__ __forceinline__ float max8(float v) {
  v = fmaxf(v, vec::dpp_xor1(v));
  v = fmaxf(v, vec::dpp_xor2(v));
  return fmaxf(v, vec::dpp_mirror8(v));
}
__device__ __forceinline__ float min8(float v) {
  v = fminf(v, vec::dpp_xor1(v));
  v = fminf(v, vec::dpp_xor2(v));
  return fminf(v, vec::dpp_mirror8(v));
}
__device__ __forceinline__ float sum8(float v) {
  v += vec::dpp_xor1(v);
  v += vec::dpp_xor2(v);
  return v + vec::dpp_mirror8(v);
}

// Codes of the lane's 16 rotated values; returns the vector's scale (s or sigma) and, for the
// asymmetric format, its minimum m.
template <int kFmt>
__device__ __forceinline__ float2 codes16(const float y[16], unsigned c[16]) {
  if constexpr (kFmt == IQ_FMT_A3) {
    float mn = y[0], mx = y[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) {
      mn = fminf(mn, y[i]);
      mx = fmaxf(mx, y[i]);
    }
    mn = min8(mn);
    mx = max8(mx);
    const float range = mx - mn;
    const float rcp = range > 0.f ? 7.f / range : 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i)   // the argument lies in [0.5, 7.5]: truncation is the floor
      c[i] = min(__float2uint_rz(fmaf(y[i] - mn, rcp, 0.5f)), 7u);
    return make_float2(range / 7.f, mn);
  } else if constexpr (kFmt == IQ_FMT_LM3) {
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) ss = fmaf(y[i], y[i], ss);
    const float sigma = sqrtf(sum8(ss) * (1.f / 128.f));
    const float r = sigma > 0.f ? 1.f / sigma : 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float u = y[i] * r;
      unsigned k = 0;
#pragma unroll
      for (int t = 0; t < 7; ++t) k += u >= 0.5f * (kLM[t] + kLM[t + 1]) ? 1u : 0u;
      c[i] = sigma > 0.f ? k : 4u;
    }
    return make_float2(sigma, 0.f);
  } else {
    constexpr int b = kFmt == IQ_FMT_U2 ? 2 : 4;
    constexpr float half = (float)(1 << (b - 1));
    constexpr float top = (float)((1 << b) - 1);
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(y[i]));
    amax = max8(amax);
    const float rcp = amax > 0.f ? (half - 0.5f) / amax : 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i)   // u in [0.5, 2^b - 0.5]: truncation is the floor, clamp the top only
      c[i] = min(__float2uint_rz(fmaf(y[i], rcp, half)), (unsigned)top);
    return make_float2(amax / (half - 0.5f), 0.f);
  }
}

template <bool kBF16, int kFmt>
__global__ __launch_bounds__(kThreads) void quantize_format_kernel(QuantizeLaunch a) {
  constexpr int kBits = kFmt == IQ_FMT_U2 ? 2 : kFmt == IQ_FMT_U4 ? 4 : 3;   // LM3, A3: 3
  constexpr int kRec = 16 * kBits;
  __shared__ float mats[32][16];
  const int s = blockIdx.z;
  const int h = blockIdx.y;
  const int64_t t_begin = (int64_t)blockIdx.x * kTokPerGroup;
  const int tid = threadIdx.x;
  if (tid < 32)
    vec::build_folded_block(a.rot + (int64_t)s * a.rot_stride_seq + (int64_t)h * 256 + tid * 8, mats[tid],
                            vec::chunk_sign(tid >> 2));
  __syncthreads();
  const int lane = tid & 63;
  const int c = vec::chunk_of(lane & 7);   // coordinates 16c..16c+15
  const int vsub = (tid >> 6) * 8 + (lane >> 3);
  float F[4][16];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int i = 0; i < 16; ++i) F[j][i] = mats[4 * c + j][i];

  const int64_t n_steps = (min((int64_t)kTokPerGroup, a.n_tokens - t_begin) + kVecPerStep - 1) / kVecPerStep;
  // (step, side) items with the next input loaded after the current one is unpacked, as in the
  // 3-bit quantize kernel
  const bool two = a.side[0].src != nullptr && a.side[1].src != nullptr;
  const QuantSide sa = a.side[0].src != nullptr ? a.side[0] : a.side[1];   // even items
  const QuantSide sb = a.side[1].src != nullptr ? a.side[1] : a.side[0];   // odd items
  const int64_t n_items = two ? 2 * n_steps : n_steps;
  constexpr int kElem = kBF16 ? 2 : 4;
  const int64_t in_step = (int64_t)kVecPerStep * a.stride_tok * kElem;
  int64_t tok = t_begin + vsub;
  const int64_t off_first =
      ((int64_t)s * a.stride_seq + (int64_t)h * a.stride_head + 16 * c + t_begin * a.stride_tok) * kElem;
  int64_t off = off_first + (int64_t)vsub * a.stride_tok * kElem;
  const int64_t rec0 = ((int64_t)s * a.n_heads + h) * a.cache_cap + a.tok_offset;
  vec::Raw16<kBF16> raw;
  vec::load_raw16<kBF16>(static_cast<const char*>(sa.src) + (tok < a.n_tokens ? off : off_first), raw);
#pragma unroll 1
  for (int64_t i = 0; i < n_items; ++i) {
    const bool odd = two && (i & 1);
    const bool adv = !two || odd;
    const int64_t tok_n = adv ? tok + kVecPerStep : tok;
    const int64_t off_n = adv ? off + in_step : off;
    float x[16], y[16];
    vec::unpack16<kBF16>(raw, x);
    __builtin_amdgcn_sched_barrier(0);
    const bool more = i + 1 < n_items && tok_n < a.n_tokens;
    vec::load_raw16<kBF16>(static_cast<const char*>(two && !odd ? sb.src : sa.src) + (more ? off_n : off_first), raw);
    __builtin_amdgcn_sched_barrier(0);
    vec::rotate8(x, F, c, y);
    unsigned q[16];
    const float2 scale = codes16<kFmt>(y, q);
    const bool valid = tok < a.n_tokens;
    const int64_t rec = rec0 + tok;
    uint8_t* dst = (odd ? sb.codes : sa.codes) + rec * kRec;
    if constexpr (kBits == 2) {
      unsigned w = 0;
#pragma unroll
      for (int k = 0; k < 16; ++k) w |= q[k] << (2 * k);
      if (valid) reinterpret_cast<unsigned*>(dst)[c] = w;
    } else if constexpr (kBits == 4) {
      unsigned w0 = 0, w1 = 0;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        w0 |= q[k] << (4 * k);
        w1 |= q[8 + k] << (4 * k);
      }
      if (valid) reinterpret_cast<uint2*>(dst)[c] = make_uint2(w0, w1);
    } else {
      unsigned g0 = 0, g1 = 0, w[3];
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        g0 |= q[k] << (3 * k);
        g1 |= q[8 + k] << (3 * k);
      }
      vec::quarter_words(g0, g1, w);          // every lane runs it (cross-lane move)
      if (valid && (c & 1) == 0) {
        unsigned* d = reinterpret_cast<unsigned*>(dst + 12 * (c >> 1));
        d[0] = w[0];
        d[1] = w[1];
        d[2] = w[2];
      }
    }
    if (valid && c == 0) {
      float* scales = odd ? sb.scales : sa.scales;
      if constexpr (kFmt == IQ_FMT_A3)
        reinterpret_cast<float2*>(scales)[rec] = scale;
      else
        scales[rec] = scale.x;
    }
    tok = tok_n;
    off = off_n;
  }
}

template <bool kBF16>
void launch_format(int fmt, dim3 grid, hipStream_t stream, const QuantizeLaunch& a) {
  if (fmt == IQ_FMT_U2)
    hipLaunchKernelGGL((quantize_format_kernel<kBF16, IQ_FMT_U2>), grid, dim3(kThreads), 0, stream, a);
  else if (fmt == IQ_FMT_U4)
    hipLaunchKernelGGL((quantize_format_kernel<kBF16, IQ_FMT_U4>), grid, dim3(kThreads), 0, stream, a);
  else if (fmt == IQ_FMT_LM3)
    hipLaunchKernelGGL((quantize_format_kernel<kBF16, IQ_FMT_LM3>), grid, dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL((quantize_format_kernel<kBF16, IQ_FMT_A3>), grid, dim3(kThreads), 0, stream, a);
}

}  // namespace

hipError_t launch_quantize_format(const QuantizeLaunch& a, int format, hipStream_t stream) {
  if (format == IQ_FMT_U3) return launch_quantize(a, stream);
  const dim3 grid((unsigned)((a.n_tokens + kTokPerGroup - 1) / kTokPerGroup), (unsigned)a.n_heads, (unsigned)a.n_seq);
  if (a.bf16)
    launch_format<true>(format, grid, stream, a);
  else
    launch_format<false>(format, grid, stream, a);
  return hipGetLastError();
}

}  // namespace iq
