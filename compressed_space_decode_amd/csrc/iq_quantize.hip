// Quantize/pack kernel: Walsh-Hadamard transform, block-diagonal SO(4)
// rotation, 3-bit scalar quantization with a per-vector scale, and packing
// into 48-byte records.
//
// Method: "RotaryQuant: Fitting 120B MoE Models on Consumer Hardware via Fused
// Compressed-Space Attention" (arXiv 2608.08081), Abstract.
//
// Work split: 8 lanes per 128-vector, lane e holds the 16 coordinates of
// chunk chunk_of(e) (order 0 1 2 3 7 6 5 4).  The Hadamard stages of stride 16,
// 32 and 64 pair chunks c^1, c^2, c^4 and run as multiply-adds with a DPP
// operand; the stages of stride 8 and 4 stay inside a lane; the stages of
// stride 2 and 1 act inside aligned blocks of four and are folded, together
// with the 1/sqrt(128) normalisation, into the 4x4 SO(4) blocks (H_128 = (I_32 (x) H_4)(H_32 (x) I_4)).  A work-group (4 waves, 32
// vectors per step) owns one (sequence, head) pair and a range of tokens, so
// its 32 folded blocks are built once and each lane keeps its four blocks
// (64 floats) in registers.  Each vector's input is loaded one vector ahead.
#include "iq_internal.h"
#include "iq_vector.h"

namespace iq {
namespace {

constexpr int kThreads = 256;
constexpr int kVecPerStep = kThreads / 8;   // 32 vectors per work-group step
constexpr int kTokPerGroup = 256;           // tokens per work-group

using vec::Raw16;

template <bool kBF16>
__global__ __launch_bounds__(kThreads) void quantize_kernel(QuantizeLaunch a) {
  __shared__ float mats[32][16];
  const int s = blockIdx.z;
  const int h = blockIdx.y;
  const int64_t t_begin = (int64_t)blockIdx.x * kTokPerGroup;
  const int tid = threadIdx.x;

  if (tid < 32) {
    const float* p = a.rot + (int64_t)s * a.rot_stride_seq + (int64_t)h * 256 + tid * 8;
    vec::build_folded_block(p, mats[tid], vec::chunk_sign(tid >> 2));
  }
  __syncthreads();

  const int lane = tid & 63;
  const int c = vec::chunk_of(lane & 7);          // coordinates 16c..16c+15
  const int vsub = (tid >> 6) * 8 + (lane >> 3);  // vector slot in a step
  float F[4][16];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int i = 0; i < 16; ++i) F[j][i] = mats[4 * c + j][i];
  const int hh = c & 1;                           // odd chunks pass their two groups to chunk c-1
  const int quarter = c >> 1;

  const int64_t n_steps = (min((int64_t)kTokPerGroup, a.n_tokens - t_begin) + kVecPerStep - 1) / kVecPerStep;
  // Items are (step, side) pairs, K then V of each step, or one side only; the input of the next
  // item is loaded before the current one is rotated.  At least one side is present, and K and V
  // share their strides.
  const bool two = a.side[0].src != nullptr && a.side[1].src != nullptr;
  const QuantSide sa = a.side[0].src != nullptr ? a.side[0] : a.side[1];   // even items
  const QuantSide sb = a.side[1].src != nullptr ? a.side[1] : a.side[0];   // odd items
  const int64_t n_items = two ? 2 * n_steps : n_steps;
  constexpr int kElem = kBF16 ? 2 : 4;
  const int64_t in_step = (int64_t)kVecPerStep * a.stride_tok * kElem;   // bytes per step
  int64_t tok = t_begin + vsub;                                           // token of item i
  // Lanes past the last token load the work-group's first token instead (never stored).
  const int64_t off_first =
      ((int64_t)s * a.stride_seq + (int64_t)h * a.stride_head + 16 * c + t_begin * a.stride_tok) * kElem;
  int64_t off = off_first + (int64_t)vsub * a.stride_tok * kElem;
  const int64_t rec0 = ((int64_t)s * a.n_heads + h) * a.cache_cap + a.tok_offset;
  Raw16<kBF16> raw;
  vec::load_raw16<kBF16>(static_cast<const char*>(sa.src) + (tok < a.n_tokens ? off : off_first), raw);
#pragma unroll 1
  for (int64_t i = 0; i < n_items; ++i) {
    const bool odd = two && (i & 1);
    const bool adv = !two || odd;                 // the next item belongs to the next step
    const int64_t tok_n = adv ? tok + kVecPerStep : tok;
    const int64_t off_n = adv ? off + in_step : off;
    float x[16];
    vec::unpack16<kBF16>(raw, x);
    __builtin_amdgcn_sched_barrier(0);            // unpack first: the next load reuses raw's registers
    // (after the last item this loads the first token again, unused: no branch around the load)
    const bool more = i + 1 < n_items && tok_n < a.n_tokens;
    vec::load_raw16<kBF16>(static_cast<const char*>(two && !odd ? sb.src : sa.src) + (more ? off_n : off_first), raw);
    __builtin_amdgcn_sched_barrier(0);            // and issued before the rotation
    unsigned g0, g1, w[3];
    const float scale = vec::quantize8(x, F, c, g0, g1);
    vec::quarter_words(g0, g1, w);
    if (tok < a.n_tokens) {
      const int64_t rec = rec0 + tok;
      if (hh == 0) {
        unsigned* dst = reinterpret_cast<unsigned*>((odd ? sb.codes : sa.codes) + rec * 48 + 12 * quarter);
        dst[0] = w[0];
        dst[1] = w[1];
        dst[2] = w[2];
      }
      if (c == 0) (odd ? sb.scales : sa.scales)[rec] = scale;
    }
    tok = tok_n;
    off = off_n;
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
