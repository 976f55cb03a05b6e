// Device code shared by the quantize and decode kernels: the cross-lane moves
// of the lane-parallel Walsh-Hadamard transform, the folded SO(4) blocks, and
// the quantisation of one 128-vector held by 8 consecutive lanes.
//
// Method: "RotaryQuant: Fitting 120B MoE Models on Consumer Hardware via Fused
// Compressed-Space Attention" (arXiv 2608.08081), Abstract: Walsh-Hadamard
// transform, block-diagonal SO(4) rotation, 3-bit scalar quantisation, packed
// 3-bit tensors.
#ifndef IQ_VECTOR_H
#define IQ_VECTOR_H

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace iq {
namespace vec {

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

// SO(4) block b as a row-major 4x4 matrix: M_b = L(qL) * Rm(conj(qR)) with the quaternions
// normalised first (the block acts as v -> qL v conj(qR) on coordinates 4b..4b+3).
__device__ inline void build_so4_block(const float* p, float* out16) {
  float l0 = p[0], l1 = p[1], l2 = p[2], l3 = p[3];
  float r0 = p[4], r1 = p[5], r2 = p[6], r3 = p[7];
  const float nl = 1.0f / sqrtf(l0 * l0 + l1 * l1 + l2 * l2 + l3 * l3);
  const float nr = 1.0f / sqrtf(r0 * r0 + r1 * r1 + r2 * r2 + r3 * r3);
  l0 *= nl; l1 *= nl; l2 *= nl; l3 *= nl;
  r0 *= nr; r1 *= nr; r2 *= nr; r3 *= nr;
  const float L[4][4] = {{l0, -l1, -l2, -l3}, {l1, l0, -l3, l2}, {l2, l3, l0, -l1}, {l3, -l2, l1, l0}};
  const float C[4][4] = {{r0, r1, r2, r3}, {-r1, r0, -r3, r2}, {-r2, r3, r0, -r1}, {-r3, -r2, r1, r0}};
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float acc = 0.f;
#pragma unroll
      for (int m = 0; m < 4; ++m) acc = fmaf(L[i][m], C[m][j], acc);
      out16[i * 4 + j] = acc;
    }
}

// Folded block b: F = M_b * H_4 / sqrt(128), M_b = L(qL) * Rm(conj(qR)) with the quaternions
// normalised first.  H_128 = (I_32 (x) H_4)(H_32 (x) I_4), so the two finest Hadamard stages act
// inside the aligned blocks of four and fold into them.
__device__ inline void build_folded_block(const float* p, float* out16) {
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

// Loads coordinates elem_off .. elem_off+15 of a vector (16-byte aligned), fp32 or bf16; zeros
// when !valid.
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

// The rotation y = R x of one 128-vector held by 8 consecutive lanes (lane e = lane & 7 holds
// coordinates 16e..16e+15 in x; F holds its folded blocks 4e..4e+3).  Every lane of the wave must
// run it (cross-lane moves); x is overwritten.
__device__ __forceinline__ void rotate8(float x[16], const float (&F)[4][16], int e, float y[16]) {
  // Cross-lane butterfly: new = partner + sg * mine gives (lower + upper) on the lower lane and
  // (lower - upper) on the upper lane.  Hadamard stages of stride 16, 32, 64 (partners e^1, ^2, ^4).
  const float sg1 = (e & 1) ? -1.f : 1.f;
  const float sg2 = (e & 2) ? -1.f : 1.f;
  const float sg4 = (e & 4) ? -1.f : 1.f;
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
}

// Quantises one 128-vector held by 8 consecutive lanes (lane e = lane & 7 holds coordinates
// 16e..16e+15 in x, and F holds its folded blocks 4e..4e+3).  Every lane of the wave must run
// it (cross-lane moves).  Returns the vector's scale and this lane's two 24-bit code groups:
// codes of coordinates 16e..16e+7 and 16e+8..16e+15, code j of a group at bits 3j..3j+2, i.e.
// bytes 6e..6e+5 of the record (one little-endian bit stream, code i at bits 3i..3i+2).
__device__ __forceinline__ float quantize8(float x[16], const float (&F)[4][16], int e, unsigned& g0, unsigned& g1) {
  float y[16];
  rotate8(x, F, e, y);
  // Per-vector scale: absmax over the 8 lanes of the vector.
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(y[i]));
  amax = fmaxf(amax, dpp_xor1(amax));
  amax = fmaxf(amax, dpp_xor2(amax));
  amax = fmaxf(amax, swz_xor4(amax));
  const float rcp = amax > 0.f ? 3.5f / amax : 0.f;
  // u = y / s + 4 lies in [0.5, 7.5] (up to rounding), so the conversion's truncation is the
  // floor and only the top needs clamping (a negative u would convert to 0)
  unsigned c[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) c[i] = min(__float2uint_rz(fmaf(y[i], rcp, 4.0f)), 7u);
  g0 = 0;
  g1 = 0;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    g0 |= c[k] << (3 * k);
    g1 |= c[8 + k] << (3 * k);
  }
  return amax / 3.5f;
}

// The 12-byte quarter e/2 of the record, as three little-endian words, for an even lane e from
// its own groups and its odd neighbour's (every lane must run it; odd lanes' results are unused).
__device__ __forceinline__ void quarter_words(unsigned g0, unsigned g1, unsigned w[3]) {
  const unsigned g2 = dpp_xor1_u(g0), g3 = dpp_xor1_u(g1);
  w[0] = g0 | (g1 << 24);
  w[1] = (g1 >> 8) | (g2 << 16);
  w[2] = (g2 >> 16) | (g3 << 8);
}

}  // namespace vec
}  // namespace iq

#endif  // IQ_VECTOR_H
