// Device code shared by the quantize and decode kernels: the cross-lane moves
// of the lane-parallel Walsh-Hadamard transform, the folded SO(4) blocks, and
// the quantisation of one 128-vector held by 8 consecutive lanes.
//
// Lane layout of a vector: lane e (= lane & 7) holds the 16 coordinates
// 16 c .. 16 c + 15 of chunk c = chunk_of(e), i.e. chunks 0 1 2 3 7 6 5 4.  With
// that order the quad moves pair chunks c, c ^ 1 and c, c ^ 2, and the mirror
// move inside 8 lanes (DPP row_half_mirror, lane e <-> 7 - e) pairs c, c ^ 4, so
// all three cross-lane Hadamard stages are DPP operands.
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
__device__ __forceinline__ float dpp_mirror8(float x) {   // row_half_mirror: lane e <-> 7 - e in 8
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x141, 0xF, 0xF, false));
}
__device__ __forceinline__ unsigned dpp_xor1_u(unsigned x) {
  return (unsigned)__builtin_amdgcn_mov_dpp((int)x, 0xB1, 0xF, 0xF, false);
}

// Chunk of 16 coordinates held by lane e of a vector's 8 lanes (order 0 1 2 3 7 6 5 4).
__device__ __forceinline__ int chunk_of(int e) { return (e & 4) ? e ^ 3 : e; }

// Sign that the fused butterflies of rotate8 leave on the values of chunk c: (-1)^popcount(c).
__device__ __forceinline__ float chunk_sign(int c) {
  return (__builtin_popcount(c) & 1) ? -1.f : 1.f;
}

// x[i] += sg * (x[i] of the partner lane) for the 16 values, the partner given by the DPP
// control CTRL: one v_fmac_f32 with a DPP source per value (the compiler would emit a DPP move and
// a separate multiply-add).  The leading s_nop gives the wait states that a DPP read of a VGPR
// needs after a VALU or EXEC write of it.
#define IQ_FMAC_DPP16(x, sg, CTRL)                                                               \
  asm("s_nop 4\n\t"                                                                              \
      "v_fmac_f32_dpp %0, %0, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                       \
      "v_fmac_f32_dpp %1, %1, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                       \
      "v_fmac_f32_dpp %2, %2, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                       \
      "v_fmac_f32_dpp %3, %3, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                       \
      "v_fmac_f32_dpp %4, %4, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                       \
      "v_fmac_f32_dpp %5, %5, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                       \
      "v_fmac_f32_dpp %6, %6, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                       \
      "v_fmac_f32_dpp %7, %7, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                       \
      "v_fmac_f32_dpp %8, %8, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                       \
      "v_fmac_f32_dpp %9, %9, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                       \
      "v_fmac_f32_dpp %10, %10, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                     \
      "v_fmac_f32_dpp %11, %11, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                     \
      "v_fmac_f32_dpp %12, %12, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                     \
      "v_fmac_f32_dpp %13, %13, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                     \
      "v_fmac_f32_dpp %14, %14, %16 " CTRL " row_mask:0xf bank_mask:0xf\n\t"                     \
      "v_fmac_f32_dpp %15, %15, %16 " CTRL " row_mask:0xf bank_mask:0xf"                           \
      : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]), "+v"(x[4]), "+v"(x[5]), "+v"(x[6]),        \
        "+v"(x[7]), "+v"(x[8]), "+v"(x[9]), "+v"(x[10]), "+v"(x[11]), "+v"(x[12]), "+v"(x[13]),   \
        "+v"(x[14]), "+v"(x[15])                                                                 \
      : "v"(sg))

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
// inside the aligned blocks of four and fold into them.  The block is multiplied by sign, which
// rotate8 expects to be chunk_sign(b / 4).
__device__ inline void build_folded_block(const float* p, float* out16, float sign) {
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
  const float inv = 0.08838834764831845f * sign;   // 1/sqrt(128)
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

// 16 coordinates of a vector as loaded: 32 bytes of bf16 or 64 bytes of fp32.
template <bool kBF16> struct Raw16 { uint4 w[2]; };
template <> struct Raw16<false> { uint4 w[4]; };

// Loads the 16 coordinates at p (16-byte aligned).
template <bool kBF16>
__device__ __forceinline__ void load_raw16(const void* p, Raw16<kBF16>& r) {
  const uint4* q = static_cast<const uint4*>(p);
#pragma unroll
  for (int i = 0; i < (kBF16 ? 2 : 4); ++i) r.w[i] = q[i];
}

template <bool kBF16>
__device__ __forceinline__ void unpack16(const Raw16<kBF16>& r, float x[16]) {
#pragma unroll
  for (int i = 0; i < (kBF16 ? 2 : 4); ++i) {
    const unsigned w[4] = {r.w[i].x, r.w[i].y, r.w[i].z, r.w[i].w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if constexpr (kBF16) {
        x[8 * i + 2 * j] = __uint_as_float(w[j] << 16);
        x[8 * i + 2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
      } else {
        x[4 * i + j] = __uint_as_float(w[j]);
      }
    }
  }
}

// Coordinates elem_off .. elem_off+15 of a vector (16-byte aligned), as floats; zeros when !valid.
template <bool kBF16>
__device__ __forceinline__ void load16(const void* base, int64_t elem_off, bool valid, float x[16]) {
  Raw16<kBF16> r;
#pragma unroll
  for (int i = 0; i < (kBF16 ? 2 : 4); ++i) r.w[i] = make_uint4(0u, 0u, 0u, 0u);
  if (valid) load_raw16<kBF16>(static_cast<const char*>(base) + elem_off * (kBF16 ? 2 : 4), r);
  unpack16<kBF16>(r, x);
}

// The rotation y = R x of one 128-vector held by 8 consecutive lanes (lane e = lane & 7 holds
// chunk c = chunk_of(e), coordinates 16c..16c+15, in x; F holds its folded blocks 4c..4c+3 times
// chunk_sign(c)).  Every lane of the wave must run it (cross-lane moves); x is overwritten.
__device__ __forceinline__ void rotate8(float x[16], const float (&F)[4][16], int c, float y[16]) {
  // Hadamard stages of stride 16, 32, 64 (chunk partners c^1, c^2, c^4), each as
  // mine + sg * partner with sg = -1 on the lane whose chunk has the stage's bit set: the lower
  // lane gets lower + upper, the upper lane minus (lower - upper).  Partners always carry the same
  // sign, so after the three stages chunk c holds chunk_sign(c) times its values, and F takes the
  // sign back out.
  const float sg1 = (c & 1) ? -1.f : 1.f;
  const float sg2 = (c & 2) ? -1.f : 1.f;
  const float sg4 = (c & 4) ? -1.f : 1.f;
  IQ_FMAC_DPP16(x, sg1, "quad_perm:[1,0,3,2]");
  IQ_FMAC_DPP16(x, sg2, "quad_perm:[2,3,0,1]");
  IQ_FMAC_DPP16(x, sg4, "row_half_mirror");
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

// Quantises one 128-vector held by 8 consecutive lanes (lane e = lane & 7 holds chunk
// c = chunk_of(e), coordinates 16c..16c+15, in x, and F as for rotate8).  Every lane of the wave
// must run it (cross-lane moves).  Returns the vector's scale and this lane's two 24-bit code
// groups: codes of coordinates 16c..16c+7 and 16c+8..16c+15, code j of a group at bits 3j..3j+2,
// i.e. bytes 6c..6c+5 of the record (one little-endian bit stream, code i at bits 3i..3i+2).
__device__ __forceinline__ float quantize8(float x[16], const float (&F)[4][16], int c, unsigned& g0, unsigned& g1) {
  float y[16];
  rotate8(x, F, c, y);
  // Per-vector scale: absmax over the 8 lanes of the vector.
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(y[i]));
  amax = fmaxf(amax, dpp_xor1(amax));
  amax = fmaxf(amax, dpp_xor2(amax));
  amax = fmaxf(amax, dpp_mirror8(amax));
  // 3.5 / amax from the hardware reciprocal (1 ulp): it moves u by under 1e-6, far inside the
  // one-level tolerance at the thresholds.  Capped at the largest float, so that a vector whose
  // absmax is below about 1e-38 still gives |u - 4| <= 3.5.
  const float rcp = amax > 0.f ? fminf(3.5f * __builtin_amdgcn_rcpf(amax), 3.4028235e38f) : 0.f;
  // u = y / s + 4 lies in [0.5, 7.5] up to rounding (or is NaN, which converts to 0), so the
  // conversion's truncation is the floor and every code fits its 3 bits
  unsigned q[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) q[i] = __float2uint_rz(fmaf(y[i], rcp, 4.0f));
  g0 = q[0];
  g1 = q[8];
#pragma unroll
  for (int k = 1; k < 8; ++k) {
    g0 |= q[k] << (3 * k);
    g1 |= q[8 + k] << (3 * k);
  }
  return amax * (1.0f / 3.5f);
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
