// Isotropy diagnostics: statistics of the K or V vectors after the method's
// rotation and after its variants.
//
// Method: "RotaryQuant: Fitting 120B MoE Models on Consumer Hardware via Fused
// Compressed-Space Attention" (arXiv 2608.08081), Abstract: the Walsh-Hadamard
// transform followed by block-diagonal SO(4) rotations is applied so that the
// coordinates of every vector look alike (outlier energy spread over all 128)
// before 3-bit scalar quantization with one scale per vector.  These kernels
// measure that for no transform, the WHT alone, the SO(4) blocks alone, the
// method, and a dense 128x128 rotation:
//   * per coordinate, across the tokens: variance and kurtosis m4 / m2^2;
//   * per vector: kurtosis of its 128 entries, 3-bit quantization error and
//     energy, peak-to-average power ratio 128 max y^2 / |y|^2.
// A variance at most 1e-9 times the mean square of the same values counts as
// zero and its kurtosis is reported as 0.
//
// Kernel 1 (diag_partial_kernel): 8 lanes per vector (lane e holds the 16
// coordinates of chunk c = chunk_of(e), in the order 0 1 2 3 7 6 5 4, so that
// every cross-lane Hadamard stage is a DPP operand), 32 vectors per step, one
// work-group per
// (sequence, head, 256 tokens).  The per-coordinate raw moments of
// d = y - y_ref are summed, with y_ref the head's first transformed token, so
// that a coordinate that never changes gives exactly zero; the per-vector
// moments are taken about the vector's own mean (two passes over registers).
// The dense transform runs on the matrix cores for the work-group's 32
// vectors of a step (dense_step), the others on the vector units.
// Each work-group writes fp32 sums for its 256 tokens.
// Kernel 2 (diag_finalize_kernel): one work-group per (sequence, head) adds
// the partial sums in fp64 (two threads per coordinate, independent
// accumulators) and forms the statistics.
#include "iq_internal.h"
#include "iq_vector.h"

namespace iq {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kVecPerStep = kThreads / 8;   // 32 vectors per work-group step
constexpr int kTok = 256;                   // tokens per work-group (one partial)
constexpr int kScalars = 8;                 // per partial: kurtosis sum, error, energy, PAPR sum, nonzero count
constexpr int kPartFloats = 4 * 128 + kScalars;
constexpr float kInvSqrt128 = 0.08838834764831845f;
constexpr double kZeroVar = 1e-9;

enum : int { kNone = 0, kWht = 1, kSo4 = 2, kWhtSo4 = 3, kDense = 4 };

using vec::dpp_xor1;
using vec::dpp_xor2;
using vec::dpp_mirror8;

__device__ __forceinline__ float sum8(float v) {      // over the 8 lanes of a vector
  v += dpp_xor1(v);
  v += dpp_xor2(v);
  return v + dpp_mirror8(v);
}
__device__ __forceinline__ float max8(float v) {
  v = fmaxf(v, dpp_xor1(v));
  v = fmaxf(v, dpp_xor2(v));
  return fmaxf(v, dpp_mirror8(v));
}

// Normalised Walsh-Hadamard transform (Sylvester order) of the vector held by 8 lanes (chunk c in
// this lane): strides 16, 32, 64 pair chunks c^1, c^2, c^4 through fused DPP multiply-adds, which
// leave chunk c with (-1)^popcount(c) times its values (taken out with the 1/sqrt(128)); strides
// 8..1 stay in the lane.
__device__ __forceinline__ void wht8(float x[16], int c) {
  const float sg1 = (c & 1) ? -1.f : 1.f, sg2 = (c & 2) ? -1.f : 1.f, sg4 = (c & 4) ? -1.f : 1.f;
  IQ_FMAC_DPP16(x, sg1, "quad_perm:[1,0,3,2]");
  IQ_FMAC_DPP16(x, sg2, "quad_perm:[2,3,0,1]");
  IQ_FMAC_DPP16(x, sg4, "row_half_mirror");
#pragma unroll
  for (int h = 8; h >= 1; h >>= 1)
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if ((i & h) == 0) {
        const float u = x[i], v = x[i + h];
        x[i] = u + v;
        x[i + h] = u - v;
      }
  const float scale = kInvSqrt128 * vec::chunk_sign(c);
#pragma unroll
  for (int i = 0; i < 16; ++i) x[i] *= scale;
}

struct DiagArgs {
  const void* x;
  int64_t n_tokens;
  int n_heads;
  int64_t stride_seq, stride_head, stride_tok;   // elements
  const float* rot;
  int64_t rot_stride_seq;                        // floats
  const float* dense;
  int64_t dense_stride_seq;                      // floats
  float* part;                                   // per (sequence, head): y_ref [128], then n_chunks partials
  int n_chunks;
  double* stats;                                 // [n_seq][n_heads][260]
};

// y = T x for this lane's 16 coordinates (chunk c), for every transform but the dense one.
// M: the lane's SO(4) blocks 4c..4c+3 (row-major 4x4).
template <int kMode>
__device__ __forceinline__ void transform(float x[16], float y[16], int c, const float (&M)[4][16]) {
  if constexpr (kMode == kWht || kMode == kWhtSo4) wht8(x, c);
  if constexpr (kMode == kSo4 || kMode == kWhtSo4) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float acc = M[j][4 * r] * x[4 * j];
        acc = fmaf(M[j][4 * r + 1], x[4 * j + 1], acc);
        acc = fmaf(M[j][4 * r + 2], x[4 * j + 2], acc);
        acc = fmaf(M[j][4 * r + 3], x[4 * j + 3], acc);
        y[4 * j + r] = acc;
      }
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) y[i] = x[i];
  }
}

// ---- the dense transform on the matrix cores ----
// Y = X T^T for the work-group's 32 vectors (rows) on v_mfma_f32_16x16x32_f16: wave w computes
// output coordinates 32w..32w+31 (two 16-wide tiles) for both 16-vector row tiles.  Operands are
// split into fp16 hi and lo parts (22 bits each) and the products hi*hi + hi*lo + lo*hi are
// summed in fp32.  Each vector is scaled by a power of two to an absmax in [1/2, 1) before the
// split, so any fp32 range fits fp16, and scaled back on the output.
typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
constexpr int kXs = 132;                      // padded LDS row (floats): rows start 4 banks apart

struct DenseOperand {                         // B fragments T[i][j] for this wave's output tiles
  half8 hi[2][4], lo[2][4];                   // [tile][32-coordinate step]
};

// Lane (n, g4) of wave w holds T[32w + 16 nt + n][32 ks + 8 g4 .. + 7] for tile nt and step ks.
__device__ __forceinline__ void load_dense_operand(const float* T, int wave, int lane, DenseOperand& b) {
  const int n = lane & 15, g4 = lane >> 4;
#pragma unroll
  for (int nt = 0; nt < 2; ++nt)
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const float* row = T + (int64_t)(32 * wave + 16 * nt + n) * 128 + 32 * ks + 8 * g4;
      half8 h, l;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float v = row[e];
        const _Float16 hv = (_Float16)v;
        h[e] = hv;
        l[e] = (_Float16)(v - (float)hv);
      }
      b.hi[nt][ks] = h;
      b.lo[nt][ks] = l;
    }
}

// y = T x for the 32 vectors of a step (lane: vector slot vsub, chunk c).  Every thread of the
// work-group must call it (barriers).  xs, ys: [32][kXs] staging; xe: [32] exponents.
__device__ __forceinline__ void dense_step(const float x[16], float y[16], int c, int vsub, int wave, int lane,
                                           const DenseOperand& b, float (*xs)[kXs], float (*ys)[kXs], int* xe) {
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(x[i]));
  amax = max8(amax);
  int ex = 0;
  if (amax > 0.f) frexpf(amax, &ex);           // amax < 2^ex
  const float down = ldexpf(1.f, -ex);
#pragma unroll
  for (int i = 0; i < 16; ++i) xs[vsub][16 * c + i] = x[i] * down;
  if (c == 0) xe[vsub] = ex;
  __syncthreads();
  const int n = lane & 15, g4 = lane >> 4;
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) {
    half8 ah[4], al[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const float* src = &xs[16 * mt + n][32 * ks + 8 * g4];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float v = src[e];
        const _Float16 hv = (_Float16)v;
        ah[ks][e] = hv;
        al[ks][e] = (_Float16)(v - (float)hv);
      }
    }
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah[ks], b.hi[nt][ks], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah[ks], b.lo[nt][ks], acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(al[ks], b.hi[nt][ks], acc, 0, 0, 0);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {             // row 4 g4 + r of the tile: vector 16 mt + 4 g4 + r
        const int v = 16 * mt + 4 * g4 + r;
        ys[v][32 * wave + 16 * nt + n] = ldexpf(acc[r], xe[v]);
      }
    }
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 16; ++i) y[i] = ys[vsub][16 * c + i];
}

template <bool kBF16, int kMode>
__global__ __launch_bounds__(kThreads) void diag_partial_kernel(DiagArgs a) {
  constexpr bool kBlocks = kMode == kSo4 || kMode == kWhtSo4;
  constexpr bool kD = kMode == kDense;
  __shared__ float mats[kBlocks ? 32 : 1][16];
  __shared__ __attribute__((aligned(16))) float xs[kD ? kVecPerStep : 1][kXs];
  __shared__ __attribute__((aligned(16))) float ys[kD ? kVecPerStep : 1][kXs];
  __shared__ int xe[kD ? kVecPerStep : 1];
  __shared__ float ref[128];
  __shared__ float red[kWaves][8][64];
  __shared__ float red_s[kWaves][kScalars];

  const int s = blockIdx.z, h = blockIdx.y, chunk = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c = vec::chunk_of(lane & 7);             // coordinates 16c..16c+15
  const int vsub = wave * 8 + (lane >> 3);           // vector slot within a step
  const int64_t head = (int64_t)s * a.n_heads + h;
  const int64_t base = (int64_t)s * a.stride_seq + (int64_t)h * a.stride_head;

  if constexpr (kBlocks) {
    if (tid < 32) vec::build_so4_block(a.rot + (int64_t)s * a.rot_stride_seq + (int64_t)h * 256 + tid * 8, mats[tid]);
  }
  DenseOperand bop;
  if constexpr (kD) load_dense_operand(a.dense + (int64_t)s * a.dense_stride_seq + (int64_t)h * 128 * 128, wave, lane, bop);
  __syncthreads();
  float M[4][16];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int i = 0; i < 16; ++i) M[j][i] = kBlocks ? mats[kBlocks ? 4 * c + j : 0][i] : 0.f;

  // the reference: the head's first token, transformed by wave 0 (vector slot 0); the dense
  // transform runs it in every slot of one step (all threads take part in its barriers)
  if (kD || wave == 0) {
    float x[16], y[16];
    vec::load16<kBF16>(a.x, base + 16 * c, true, x);
    if constexpr (kD)
      dense_step(x, y, c, vsub, wave, lane, bop, xs, ys, xe);
    else
      transform<kMode>(x, y, c, M);
    if (wave == 0 && lane < 8) {
#pragma unroll
      for (int i = 0; i < 16; ++i) ref[16 * c + i] = y[i];
      if (chunk == 0) {
#pragma unroll
        for (int i = 0; i < 16; ++i) a.part[head * (128 + (int64_t)a.n_chunks * kPartFloats) + 16 * c + i] = y[i];
      }
    }
  }
  __syncthreads();
  float yref[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) yref[i] = ref[16 * c + i];

  float S1[16], S2[16], S3[16], S4[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) S1[i] = S2[i] = S3[i] = S4[i] = 0.f;
  float acc_kv = 0.f, acc_err = 0.f, acc_en = 0.f, acc_papr = 0.f, acc_nz = 0.f;

  const int64_t t_begin = (int64_t)chunk * kTok;
  for (int step = 0; step < kTok / kVecPerStep; ++step) {
    const int64_t t0 = t_begin + (int64_t)step * kVecPerStep;
    if (t0 >= a.n_tokens) break;                      // uniform over the work-group
    const int64_t t = t0 + vsub;
    const bool valid = t < a.n_tokens;
    float x[16], y[16];
    vec::load16<kBF16>(a.x, base + t * a.stride_tok + 16 * c, valid, x);
    if constexpr (kD)
      dense_step(x, y, c, vsub, wave, lane, bop, xs, ys, xe);
    else
      transform<kMode>(x, y, c, M);
    // per coordinate, about the reference
    const float vm = valid ? 1.f : 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float d = (y[i] - yref[i]) * vm;
      const float d2 = d * d;
      S1[i] += d;
      S2[i] += d2;
      S3[i] = fmaf(d2, d, S3[i]);
      S4[i] = fmaf(d2, d2, S4[i]);
    }
    // per vector (invalid slots hold zeros and add nothing)
    float amax = 0.f, sy = 0.f, en = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      amax = fmaxf(amax, fabsf(y[i]));
      sy += y[i];
      en = fmaf(y[i], y[i], en);
    }
    amax = max8(amax);
    const float mean = sum8(sy) * (1.f / 128.f);
    en = sum8(en);
    const float rcp = amax > 0.f ? 3.5f / amax : 0.f;
    const float sc = amax / 3.5f;
    float c2 = 0.f, c4 = 0.f, err = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float c = y[i] - mean;
      c2 = fmaf(c, c, c2);
      c4 = fmaf(c * c, c * c, c4);
      const float code = fminf(fmaxf(floorf(fmaf(y[i], rcp, 4.f)), 0.f), 7.f);
      const float q = y[i] - sc * (code - 3.5f);
      err = fmaf(q, q, err);
    }
    c2 = sum8(c2) * (1.f / 128.f);
    c4 = sum8(c4) * (1.f / 128.f);
    err = sum8(err);
    if (c == 0 && valid) {
      acc_kv += c2 > (float)kZeroVar * en * (1.f / 128.f) ? c4 / (c2 * c2) : 0.f;
      acc_err += err;
      acc_en += en;
      if (en > 0.f) {
        acc_papr += 128.f * amax * amax / en;
        acc_nz += 1.f;
      }
    }
  }

  // ---- reduce over the 8 vector slots of each wave (lanes e, e+8, ..., e+56), then the waves
#pragma unroll
  for (int m = 8; m < 64; m <<= 1) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      S1[i] += __shfl_xor(S1[i], m, 64);
      S2[i] += __shfl_xor(S2[i], m, 64);
      S3[i] += __shfl_xor(S3[i], m, 64);
      S4[i] += __shfl_xor(S4[i], m, 64);
    }
    acc_kv += __shfl_xor(acc_kv, m, 64);
    acc_err += __shfl_xor(acc_err, m, 64);
    acc_en += __shfl_xor(acc_en, m, 64);
    acc_papr += __shfl_xor(acc_papr, m, 64);
    acc_nz += __shfl_xor(acc_nz, m, 64);
  }
  if (lane < 8) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      red[wave][c][i] = S1[i];
      red[wave][c][16 + i] = S2[i];
      red[wave][c][32 + i] = S3[i];
      red[wave][c][48 + i] = S4[i];
    }
  }
  if (lane == 0) {
    red_s[wave][0] = acc_kv;
    red_s[wave][1] = acc_err;
    red_s[wave][2] = acc_en;
    red_s[wave][3] = acc_papr;
    red_s[wave][4] = acc_nz;
  }
  __syncthreads();
  float* out = a.part + head * (128 + (int64_t)a.n_chunks * kPartFloats) + 128 + (int64_t)chunk * kPartFloats;
  for (int idx = tid; idx < 4 * 128; idx += kThreads) {   // out[m * 128 + i]: moment m + 1 of coordinate i
    const int m = idx >> 7, i = idx & 127;
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) v += red[w][i >> 4][16 * m + (i & 15)];
    out[idx] = v;
  }
  if (tid < kScalars) {
    float v = 0.f;
    if (tid < 5) {
#pragma unroll
      for (int w = 0; w < kWaves; ++w) v += red_s[w][tid];
    }
    out[4 * 128 + tid] = v;
  }
}

// One work-group (256 threads: two per coordinate, each adding half of the partials with four
// independent accumulators) per (sequence, head).
__global__ __launch_bounds__(256) void diag_finalize_kernel(DiagArgs a) {
  __shared__ double half_sums[4][128];
  __shared__ double scal[2][5];
  const int s = blockIdx.y, h = blockIdx.x, tid = threadIdx.x, i = tid & 127, part = tid >> 7;
  const int64_t head = (int64_t)s * a.n_heads + h;
  double* st = a.stats + head * 260;
  const double n = (double)a.n_tokens;
  if (a.n_tokens == 0) {
    if (part == 0) {
      st[i] = 0.0;
      st[128 + i] = 0.0;
      if (i < 4) st[256 + i] = 0.0;
    }
    return;
  }
  const float* p = a.part + head * (128 + (int64_t)a.n_chunks * kPartFloats);
  const int c_begin = part * ((a.n_chunks + 1) / 2), c_end = part ? a.n_chunks : (a.n_chunks + 1) / 2;
  double S[4][4] = {};                                // [accumulator][moment]
  int c = c_begin;
  for (; c + 4 <= c_end; c += 4) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const float* q = p + 128 + (int64_t)(c + u) * kPartFloats;
#pragma unroll
      for (int m = 0; m < 4; ++m) S[u][m] += q[128 * m + i];
    }
  }
  for (; c < c_end; ++c) {
    const float* q = p + 128 + (int64_t)c * kPartFloats;
#pragma unroll
    for (int m = 0; m < 4; ++m) S[0][m] += q[128 * m + i];
  }
  if (i < 5) {                                        // the scalars: kurtosis sum, error, energy, PAPR sum, nonzero
    double v = 0.0;
    for (int cc = c_begin; cc < c_end; ++cc) v += p[128 + (int64_t)cc * kPartFloats + 4 * 128 + i];
    scal[part][i] = v;
  }
  if (part == 1) {
#pragma unroll
    for (int m = 0; m < 4; ++m) half_sums[m][i] = (S[0][m] + S[1][m]) + (S[2][m] + S[3][m]);
  }
  __syncthreads();
  if (part == 1) return;
  double M[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) M[m] = ((S[0][m] + S[1][m]) + (S[2][m] + S[3][m])) + half_sums[m][i];
  const double mu = M[0] / n;                         // mean of d = y - y_ref
  double m2 = M[1] / n - mu * mu;
  const double m4 = M[3] / n - 4.0 * mu * (M[2] / n) + 6.0 * mu * mu * (M[1] / n) - 3.0 * mu * mu * mu * mu;
  if (m2 < 0.0) m2 = 0.0;
  const double ym = mu + (double)p[i];                // mean of y
  const double mean_sq = m2 + ym * ym;
  st[i] = m2 > kZeroVar * mean_sq ? m4 / (m2 * m2) : 0.0;
  st[128 + i] = m2;
  if (i == 0) {
    double sc[5];
#pragma unroll
    for (int k = 0; k < 5; ++k) sc[k] = scal[0][k] + scal[1][k];
    st[256] = sc[0] / n;
    st[257] = sc[2] > 0.0 ? sc[1] / sc[2] : 0.0;
    st[258] = sc[4] > 0.0 ? sc[3] / sc[4] : 0.0;
    st[259] = n;
  }
}

template <bool kBF16>
void launch_partial(int mode, dim3 grid, hipStream_t stream, const DiagArgs& k) {
  switch (mode) {
    case kNone: hipLaunchKernelGGL((diag_partial_kernel<kBF16, kNone>), grid, dim3(kThreads), 0, stream, k); break;
    case kWht: hipLaunchKernelGGL((diag_partial_kernel<kBF16, kWht>), grid, dim3(kThreads), 0, stream, k); break;
    case kSo4: hipLaunchKernelGGL((diag_partial_kernel<kBF16, kSo4>), grid, dim3(kThreads), 0, stream, k); break;
    case kWhtSo4: hipLaunchKernelGGL((diag_partial_kernel<kBF16, kWhtSo4>), grid, dim3(kThreads), 0, stream, k); break;
    default: hipLaunchKernelGGL((diag_partial_kernel<kBF16, kDense>), grid, dim3(kThreads), 0, stream, k); break;
  }
}

}  // namespace

int64_t diag_workspace_bytes(int64_t n_seq, int n_heads, int64_t n_tokens) {
  const int64_t chunks = (n_tokens + kTok - 1) / kTok;
  return n_seq * n_heads * (128 + chunks * kPartFloats) * 4 + 256;
}

hipError_t launch_diag(const DiagLaunch& a, hipStream_t stream) {
  DiagArgs k{};
  k.x = a.x;
  k.n_tokens = a.n_tokens;
  k.n_heads = a.n_heads;
  k.stride_seq = a.stride_seq;
  k.stride_head = a.stride_head;
  k.stride_tok = a.stride_tok;
  k.rot = a.rot;
  k.rot_stride_seq = a.rot_stride_seq;
  k.dense = a.dense;
  k.dense_stride_seq = a.dense_stride_seq;
  k.part = static_cast<float*>(a.workspace);
  k.n_chunks = (int)((a.n_tokens + kTok - 1) / kTok);
  k.stats = a.stats;
  if (k.n_chunks > 0) {
    const dim3 grid((unsigned)k.n_chunks, (unsigned)a.n_heads, (unsigned)a.n_seq);
    if (a.bf16)
      launch_partial<true>(a.mode, grid, stream, k);
    else
      launch_partial<false>(a.mode, grid, stream, k);
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  hipLaunchKernelGGL(diag_finalize_kernel, dim3((unsigned)a.n_heads, (unsigned)a.n_seq), dim3(256), 0, stream, k);
  return hipGetLastError();
}

}  // namespace iq
