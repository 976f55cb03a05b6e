// Quantize/pack kernel: Walsh-Hadamard transform, block-diagonal SO(4)
// rotation, 3-bit scalar quantization with a per-vector scale, and packing
// into 48-byte records.
//
// Method: "RotaryQuant: Fitting 120B MoE Models on Consumer Hardware via Fused
// Compressed-Space Attention" (arXiv 2608.08081), Abstract.
//
// Work split: 8 lanes per 128-vector, lane e holds coordinates 16e..16e+15.
// The Hadamard stages of stride 16, 32 and 64 pair lanes (e^1, e^2, e^4) and
// run through cross-lane moves; the stages of stride 8 and 4 stay inside a
// lane; the stages of stride 2 and 1 act inside aligned blocks of four and
// are folded, together with the 1/sqrt(128) normalisation, into the 4x4 SO(4)
// blocks (H_128 = (I_32 (x) H_4)(H_32 (x) I_4)).  A work-group (4 waves, 32
// vectors per step) owns one (sequence, head) pair and a range of tokens, so
// its 32 folded blocks are built once and each lane keeps its four blocks
// (64 floats) in registers.
#include "iq_internal.h"
#include "iq_vector.h"

namespace iq {
namespace {

constexpr int kThreads = 256;
constexpr int kVecPerStep = kThreads / 8;   // 32 vectors per work-group step
constexpr int kTokPerGroup = 256;           // tokens per work-group

using vec::build_folded_block;
using vec::load16;

template <bool kBF16>
__global__ __launch_bounds__(kThreads) void quantize_kernel(QuantizeLaunch a) {
  __shared__ float mats[32][16];
  const int s = blockIdx.z;
  const int h = blockIdx.y;
  const int64_t t_begin = (int64_t)blockIdx.x * kTokPerGroup;
  const int tid = threadIdx.x;

  if (tid < 32) {
    const float* p = a.rot + (int64_t)s * a.rot_stride_seq + (int64_t)h * 256 + tid * 8;
    build_folded_block(p, mats[tid]);
  }
  __syncthreads();

  const int lane = tid & 63;
  const int e = lane & 7;                         // coordinates 16e..16e+15
  const int vsub = (tid >> 6) * 8 + (lane >> 3);  // vector slot in a step
  float F[4][16];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int i = 0; i < 16; ++i) F[j][i] = mats[4 * e + j][i];
  const int hh = e & 1;                           // odd lanes pass their two groups to lane e-1
  const int quarter = e >> 1;

  for (int step = 0; step < kTokPerGroup / kVecPerStep; ++step) {
    const int64_t t0 = t_begin + (int64_t)step * kVecPerStep;
    if (t0 >= a.n_tokens) break;                  // uniform over the work-group
    const int64_t t = t0 + vsub;
    const bool valid = t < a.n_tokens;
#pragma unroll
    for (int sd = 0; sd < 2; ++sd) {
      const QuantSide side = a.side[sd];
      if (side.src == nullptr) continue;          // uniform
      float x[16];
      load16<kBF16>(side.src, (int64_t)s * a.stride_seq + (int64_t)h * a.stride_head + t * a.stride_tok + 16 * e,
                    valid, x);
      unsigned g0, g1, w[3];
      const float scale = vec::quantize8(x, F, e, g0, g1);
      vec::quarter_words(g0, g1, w);
      if (valid) {
        const int64_t rec = ((int64_t)s * a.n_heads + h) * a.cache_cap + a.tok_offset + t;
        if (hh == 0) {
          unsigned* dst = reinterpret_cast<unsigned*>(side.codes + rec * 48 + 12 * quarter);
          dst[0] = w[0];
          dst[1] = w[1];
          dst[2] = w[2];
        }
        if (e == 0) side.scales[rec] = scale;
      }
    }
  }
}

}  // namespace

hipError_t launch_quantize(const QuantizeLaunch& a, hipStream_t stream) {
  if (a.n_tokens == 0) return hipSuccess;
  const dim3 grid((unsigned)((a.n_tokens + kTokPerGroup - 1) / kTokPerGroup), (unsigned)a.n_heads,
                  (unsigned)a.n_seq);
  if (a.bf16)
    hipLaunchKernelGGL(quantize_kernel<true>, grid, dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(quantize_kernel<false>, grid, dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace iq
