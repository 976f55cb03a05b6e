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

namespace iq {
namespace {

constexpr int kThreads = 256;
constexpr int kVecPerStep = kThreads / 8;   // 32 vectors per work-group step
constexpr int kTokPerGroup = 256;           // tokens per work-group

__device__ __forceinline__ float dpp_xor1(float x) {   // quad_perm [1,0,3,2]
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, false));
}
__device__ __forceinline__ float dpp_xor2(float x) {   // quad_perm [2,3,0,1]
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, false));
}
__device__ __forceinline__ float swz_xor4(float x) {   // bitmask swizzle, xor 4
  return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), (4 << 10) | 0x1F));
}
__device__ __forceinline__ unsigned dpp_xor1_u(unsigned x) {
  return (unsigned)__builtin_amdgcn_mov_dpp((int)x, 0xB1, 0xF, 0xF, false);
}

// Folded block b: F = M_b * H_4 / sqrt(128), M_b = L(qL) * Rm(conj(qR)).
__device__ void build_folded_block(const float* p, float* out16) {
  float l0 = p[0], l1 = p[1], l2 = p[2], l3 = p[3];
  float r0 = p[4], r1 = p[5], r2 = p[6], r3 = p[7];
  const float nl = 1.0f / sqrtf(l0 * l0 + l1 * l1 + l2 * l2 + l3 * l3);
  const float nr = 1.0f / sqrtf(r0 * r0 + r1 * r1 + r2 * r2 + r3 * r3);
  l0 *= nl; l1 *= nl; l2 *= nl; l3 *= nl;
  r0 *= nr; r1 *= nr; r2 *= nr; r3 *= nr;
  const float L[4][4] = {{l0, -l1, -l2, -l3}, {l1, l0, -l3, l2}, {l2, l3, l0, -l1}, {l3, -l2, l1, l0}};
  const float C[4][4] = {{r0, r1, r2, r3}, {-r1, r0, -r3, r2}, {-r2, r3, r0, -r1}, {-r3, -r2, r1, r0}};
  float M[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float acc = 0.f;
#pragma unroll
      for (int m = 0; m < 4; ++m) acc = fmaf(L[i][m], C[m][j], acc);
      M[i][j] = acc;
    }
  const float inv = 0.08838834764831845f;   // 1/sqrt(128)
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float acc = 0.f;
#pragma unroll
      for (int k = 0; k < 4; ++k) acc += (__builtin_popcount(k & j) & 1) ? -M[i][k] : M[i][k];
      out16[i * 4 + j] = acc * inv;
    }
}

template <bool kBF16>
__device__ __forceinline__ void load16(const void* base, int64_t elem_off, bool valid, float x[16]) {
  if (!valid) {
#pragma unroll
    for (int i = 0; i < 16; ++i) x[i] = 0.f;
    return;
  }
  if constexpr (kBF16) {
    const uint4* p = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + elem_off);
    const uint4 a = p[0], b = p[1];
    const unsigned w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      x[2 * i] = __uint_as_float(w[i] << 16);
      x[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  } else {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(base) + elem_off);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float4 v = p[i];
      x[4 * i] = v.x; x[4 * i + 1] = v.y; x[4 * i + 2] = v.z; x[4 * i + 3] = v.w;
    }
  }
}

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
  // Cross-lane butterfly: new = partner + sg * mine gives (lower + upper) on the
  // lower lane and (lower - upper) on the upper lane.
  const float sg1 = (e & 1) ? -1.f : 1.f;
  const float sg2 = (e & 2) ? -1.f : 1.f;
  const float sg4 = (e & 4) ? -1.f : 1.f;
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
      // Hadamard stages of stride 16, 32, 64 (partner lanes e^1, e^2, e^4).
#pragma unroll
      for (int i = 0; i < 16; ++i) x[i] = fmaf(sg1, x[i], dpp_xor1(x[i]));
#pragma unroll
      for (int i = 0; i < 16; ++i) x[i] = fmaf(sg2, x[i], dpp_xor2(x[i]));
#pragma unroll
      for (int i = 0; i < 16; ++i) x[i] = fmaf(sg4, x[i], swz_xor4(x[i]));
      // Stages of stride 8 and 4 inside the lane.
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float u = x[i], v = x[i + 8];
        x[i] = u + v;
        x[i + 8] = u - v;
      }
#pragma unroll
      for (int blk = 0; blk < 16; blk += 8)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float u = x[blk + i], v = x[blk + i + 4];
          x[blk + i] = u + v;
          x[blk + i + 4] = u - v;
        }
      // Folded 4x4 blocks (stride-2/1 stages, SO(4) rotation, 1/sqrt(128)).
      float y[16];
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float acc = F[j][4 * r] * x[4 * j];
          acc = fmaf(F[j][4 * r + 1], x[4 * j + 1], acc);
          acc = fmaf(F[j][4 * r + 2], x[4 * j + 2], acc);
          acc = fmaf(F[j][4 * r + 3], x[4 * j + 3], acc);
          y[4 * j + r] = acc;
        }
      // Per-vector scale: absmax over the 8 lanes of the vector.
      float amax = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(y[i]));
      amax = fmaxf(amax, dpp_xor1(amax));
      amax = fmaxf(amax, dpp_xor2(amax));
      amax = fmaxf(amax, swz_xor4(amax));
      const float scale = amax / 3.5f;
      const float rcp = amax > 0.f ? 3.5f / amax : 0.f;
      unsigned c[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float u = floorf(fmaf(y[i], rcp, 4.0f));
        c[i] = (unsigned)fminf(fmaxf(u, 0.f), 7.f);
      }
      // Pack: the record is one little-endian bit stream with code i at bits 3i..3i+2, so this
      // lane's 16 codes are the 6 bytes 6e..6e+5, two 24-bit groups of 8 codes.  Even lanes
      // take their odd neighbour's groups and store the 12-byte quarter e/2.
      unsigned g0 = 0, g1 = 0;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        g0 |= c[k] << (3 * k);
        g1 |= c[8 + k] << (3 * k);
      }
      const unsigned g2 = dpp_xor1_u(g0), g3 = dpp_xor1_u(g1);
      if (valid) {
        const int64_t rec = ((int64_t)s * a.n_heads + h) * a.cache_cap + a.tok_offset + t;
        if (hh == 0) {
          unsigned* dst = reinterpret_cast<unsigned*>(side.codes + rec * 48 + 12 * quarter);
          dst[0] = g0 | (g1 << 24);
          dst[1] = (g1 >> 8) | (g2 << 16);
          dst[2] = (g2 >> 16) | (g3 << 8);
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
