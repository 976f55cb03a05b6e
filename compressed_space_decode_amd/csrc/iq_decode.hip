// Decode attention computed directly on packed 3-bit K/V.
//
// Method: "RotaryQuant: Fitting 120B MoE Models on Consumer Hardware via Fused
// Compressed-Space Attention" (arXiv 2608.08081), Abstract: attention runs on
// the packed 3-bit tensors without materialising full-precision KV.
// Because R is orthogonal, q.k_hat = (Rq).(s (c - 3.5)): the query is rotated
// once, V levels are summed in rotated space, and R^T is applied once per
// output row.
//
// Kernel 1 (decode_split_kernel), one work-group of 4 waves per (sequence,
// KV head, group of up to 8 query heads, chunk of tokens):
//   * set-up: rotate the group's queries (WHT in LDS, then SO(4) blocks) and
//     lay them out as the fp16 B operand of the QK product, hi and lo parts
//     (q = hi + lo) in separate columns so the product carries ~22 bits;
//   * each wave walks 32-token blocks.  A lane loads 12 bytes (one quarter of
//     a record) of one token; one AND per pair of codes turns them into fp16
//     numbers c * 2^(p-24) (subnormals, handled exactly by the matrix cores),
//     the power 2^-p being folded into the query operand;
//   * S^T[token][head,part] = codes x q' via v_mfma_f32_16x16x32_f16, online
//     softmax in base 2, P'' = p s_V (scaled) split hi/lo in fp16;
//   * V codes of the block are unpacked the same way into LDS ([token][slot]
//     rows) and read back transposed with ds_read_b64_tr_b16 as the B
//     operand of O[head,part][slot] += P'' x V;
//   * the 4 waves merge in LDS and write one (max, sum, o') partial.
// Kernel 2 (combine_kernel), one work-group per (sequence, query head):
//   log-sum-exp merge of the chunk partials, then o = R^T o' (transposed SO(4)
//   blocks followed by the WHT).
#include "iq_internal.h"

namespace iq {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef short short4v __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kBlock = 32;          // tokens per wave step
constexpr int kRowHalves = 136;     // fp16 elements per LDS V row (128 + 8 padding)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kPScale = 4096.f;   // P'' = p * (s_V / sigma) * 4096 keeps fp16 lo parts normal

// Coordinate (within a quarter) held by extraction slot s: the 16 words that
// one quarter unpacks into carry coordinate (s >> 1) of half (s & 1).
__device__ __forceinline__ int slot_coord(int s) { return 16 * (s & 1) + (s >> 1); }
// Power of two carried by the fp16 value of slot s (field position p: value = c * 2^(p-24)).
__device__ __forceinline__ int slot_pow(int s) {
  const int d = s >> 1;
  if (d == 15) return 0;
  const int j = d % 5;
  return j == 0 ? 0 : j == 1 ? 3 : j == 2 ? 6 : j == 3 ? 0 : 3;
}

// Unpack one quarter (three 32-bit words) into 16 words of fp16 pairs.
// Word W_k pairs field j of half 0 (low 16 bits) with field j of half 1.
__device__ __forceinline__ void unpack_quarter(unsigned w0, unsigned w1, unsigned w2, unsigned o[16]) {
  const unsigned w[3] = {w0, w1, w2};
#pragma unroll
  for (int k = 0; k < 3; ++k) {
    o[5 * k + 0] = w[k] & 0x00070007u;
    o[5 * k + 1] = w[k] & 0x00380038u;
    o[5 * k + 2] = w[k] & 0x01C001C0u;
    const unsigned sh = w[k] >> 9;
    o[5 * k + 3] = sh & 0x00070007u;
    o[5 * k + 4] = sh & 0x00380038u;
  }
  o[15] = ((w0 >> 15) & 0x00010001u) | ((w1 >> 14) & 0x00020002u) | ((w2 >> 13) & 0x00040004u);
}

__device__ __forceinline__ half8 as_half8(unsigned a, unsigned b, unsigned c, unsigned d) {
  typedef unsigned u4 __attribute__((ext_vector_type(4)));
  u4 v = {a, b, c, d};
  return __builtin_bit_cast(half8, v);
}

__device__ __forceinline__ float wave_xor(float x, int m) { return __shfl_xor(x, m, 64); }

struct DecodeKArgs {
  const void* q;
  int q_bf16;
  const uint8_t* kc;
  const float* ks;
  const uint8_t* vc;
  const float* vs;
  const float* rot;
  int64_t rot_stride_b;
  const int32_t* seq_lens;
  int Hq, Hkv, G, head_groups;
  int64_t cap;
  int chunk, n_chunks;
  float sm_log2;          // softmax scale times log2(e)
  float* part_o;          // [B][Hq][n_chunks][128]
  float* part_ml;         // [B][Hq][n_chunks][2]  (max in log2 units, sum)
};

struct SetupSmem {
  float qr[8][128];       // query rows, rotated in place
  float mats[32][16];     // SO(4) blocks M_b
  float red[kThreads];
};
struct MergeSmem {
  float o[kWaves][8][128];
  float m[kWaves][8];
  float l[kWaves][8];
};
struct LoopSmem {
  _Float16 v[kWaves][kBlock][kRowHalves];
  float sc[kWaves][64];
};
union DecodeSmem {
  SetupSmem setup;
  MergeSmem merge;
  LoopSmem loop;
};

__device__ void build_block(const float* p, float* out16) {
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

__global__ __launch_bounds__(kThreads) void decode_split_kernel(DecodeKArgs a) {
  __shared__ DecodeSmem sm;
  const int chunk_id = blockIdx.x;
  const int g = blockIdx.y / a.head_groups;
  const int hg = blockIdx.y % a.head_groups;
  const int b = blockIdx.z;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;

  int64_t len = a.cap;
  if (a.seq_lens) {
    const int64_t l = a.seq_lens[b];
    len = l < 0 ? 0 : (l > a.cap ? a.cap : l);
  }
  const int64_t tok0 = (int64_t)chunk_id * a.chunk;
  if (tok0 >= len) return;                                   // uniform
  const int64_t tok_end = (tok0 + a.chunk < len) ? tok0 + a.chunk : len;
  const int h0 = g * a.G + hg * 8;
  const int nh = (a.G - hg * 8) < 8 ? (a.G - hg * 8) : 8;
  const int64_t kv = (int64_t)b * a.Hkv + g;
  const float* rot = a.rot + b * a.rot_stride_b + (int64_t)g * 256;

  // ---------------- set-up: rotate queries, build operands ----------------
  if (tid < 32) build_block(rot + tid * 8, sm.setup.mats[tid]);
  {
    const int i = tid >> 5;              // query row 0..7
    const int d4 = (tid & 31) * 4;
    float v[4] = {0.f, 0.f, 0.f, 0.f};
    if (i < nh) {
      const int64_t off = ((int64_t)b * a.Hq + h0 + i) * 128 + d4;
      if (a.q_bf16) {
        const uint16_t* qp = static_cast<const uint16_t*>(a.q) + off;
#pragma unroll
        for (int u = 0; u < 4; ++u) v[u] = __uint_as_float((unsigned)qp[u] << 16);
      } else {
        const float* qp = static_cast<const float*>(a.q) + off;
#pragma unroll
        for (int u = 0; u < 4; ++u) v[u] = qp[u];
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) sm.setup.qr[i][d4 + u] = v[u];
  }
  __syncthreads();
  // Unnormalised Sylvester WHT of each row: 7 butterfly stages, 512 pairs per stage.
  for (int m = 1; m < 128; m <<= 1) {
#pragma unroll
    for (int rep = 0; rep < 2; ++rep) {
      const int pidx = tid + rep * kThreads;    // pair index 0..511
      const int row = pidx >> 6;
      const int p = pidx & 63;
      const int lo = ((p / m) * 2 * m) + (p % m);
      const float u = sm.setup.qr[row][lo], w = sm.setup.qr[row][lo + m];
      sm.setup.qr[row][lo] = u + w;
      sm.setup.qr[row][lo + m] = u - w;
    }
    __syncthreads();
  }
  // SO(4) blocks and 1/sqrt(128): thread (row i, block bb).
  float amax_local;
  {
    const int i = tid >> 5, bb = tid & 31;
    const float* M = sm.setup.mats[bb];
    const float y0 = sm.setup.qr[i][4 * bb], y1 = sm.setup.qr[i][4 * bb + 1];
    const float y2 = sm.setup.qr[i][4 * bb + 2], y3 = sm.setup.qr[i][4 * bb + 3];
    float r[4];
#pragma unroll
    for (int rr = 0; rr < 4; ++rr)
      r[rr] = (M[4 * rr] * y0 + M[4 * rr + 1] * y1 + M[4 * rr + 2] * y2 + M[4 * rr + 3] * y3) *
              0.08838834764831845f;
    __syncthreads();
    amax_local = 0.f;
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      sm.setup.qr[i][4 * bb + rr] = r[rr];
      amax_local = fmaxf(amax_local, fabsf(r[rr]));
    }
  }
  // sigma = max V scale over the chunk (keeps P'' <= 4096 in fp16).
  float vmax_local = 0.f;
  for (int64_t t = tok0 + tid; t < tok_end; t += kThreads) vmax_local = fmaxf(vmax_local, a.vs[kv * a.cap + t]);
  sm.setup.red[tid] = fmaxf(amax_local, 0.f);
  __syncthreads();
  for (int st = kThreads / 2; st > 0; st >>= 1) {
    if (tid < st) sm.setup.red[tid] = fmaxf(sm.setup.red[tid], sm.setup.red[tid + st]);
    __syncthreads();
  }
  const float qamax = sm.setup.red[0];
  __syncthreads();
  sm.setup.red[tid] = vmax_local;
  __syncthreads();
  for (int st = kThreads / 2; st > 0; st >>= 1) {
    if (tid < st) sm.setup.red[tid] = fmaxf(sm.setup.red[tid], sm.setup.red[tid + st]);
    __syncthreads();
  }
  const float sigma = sm.setup.red[0] > 0.f ? sm.setup.red[0] : 1.f;
  // Query operand scaling 2^E keeps the largest |q'| * 2^E near 2^14 in fp16.
  int E = 0;
  if (qamax > 0.f) {
    int ex;
    frexpf(qamax, &ex);                // qamax in [2^(ex-1), 2^ex)
    E = 14 - ex;
  }
  // B operand of the QK product: lane = (column n = head + 8*part, quarter g4).
  const int n = lane & 15;
  const int g4 = lane >> 4;
  const int head = n & 7;
  const int part = n >> 3;
  half8 qop[4];
  float qsum = 0.f;                    // sum over coordinates of q' for this lane's head
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    _Float16 hv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int s = 8 * kb + e;
      const float qv = sm.setup.qr[head][32 * g4 + slot_coord(s)];
      const float v = ldexpf(qv, E - slot_pow(s));
      const _Float16 hi = (_Float16)v;
      hv[e] = part ? (_Float16)(v - (float)hi) : hi;
      qsum += qv;
    }
    qop[kb] = half8{hv[0], hv[1], hv[2], hv[3], hv[4], hv[5], hv[6], hv[7]};
  }
  // qsum so far covers this lane's quarter; add the other three quarters.
  qsum += wave_xor(qsum, 16);
  qsum += wave_xor(qsum, 32);
  __syncthreads();                     // set-up smem is reused by the loop below

  // z2 = log2(e) * sm * s_K * (q'.c - 3.5 sum q'), with q'.c = raw * 2^(24-E).
  const float c1 = a.sm_log2 * ldexpf(1.f, 24 - E);
  const float c2 = a.sm_log2 * 3.5f * qsum;
  const float pmul = kPScale / sigma;

  floatx4 O[8];
#pragma unroll
  for (int nt = 0; nt < 8; ++nt) O[nt] = floatx4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY;             // running max (log2 units) of this lane's head
  float l_run = 0.f;                   // sum of p
  float ls_run = 0.f;                  // sum of the P'' values fed to the PV product (own part)

  const uint8_t* kbase = a.kc + kv * a.cap * 48;
  const uint8_t* vbase = a.vc + kv * a.cap * 48;
  const float* ksb = a.ks + kv * a.cap;
  const float* vsb = a.vs + kv * a.cap;
  _Float16(*vrow)[kRowHalves] = sm.loop.v[wave];
  float* sc = sm.loop.sc[wave];

  for (int64_t t0 = tok0 + (int64_t)wave * kBlock; t0 < tok_end; t0 += (int64_t)kWaves * kBlock) {
    // ---- loads ----
    unsigned kw[2][3], vw[2][3];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      int64_t t = t0 + 16 * tt + n;
      if (t >= a.cap) t = a.cap - 1;
      const unsigned* kp = reinterpret_cast<const unsigned*>(kbase + t * 48 + 12 * g4);
      const unsigned* vp = reinterpret_cast<const unsigned*>(vbase + t * 48 + 12 * g4);
      kw[tt][0] = kp[0]; kw[tt][1] = kp[1]; kw[tt][2] = kp[2];
      vw[tt][0] = vp[0]; vw[tt][1] = vp[1]; vw[tt][2] = vp[2];
    }
    {
      int64_t t = t0 + (lane & 31);
      if (t >= a.cap) t = a.cap - 1;
      sc[lane] = (lane < 32) ? ksb[t] : vsb[t];
    }
    // ---- QK: S^T[token][head,part] ----
    floatx4 S[2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      unsigned u[16];
      unpack_quarter(kw[tt][0], kw[tt][1], kw[tt][2], u);
      floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_half8(u[4 * kb], u[4 * kb + 1], u[4 * kb + 2], u[4 * kb + 3]),
                                                    qop[kb], acc, 0, 0, 0);
      S[tt] = acc;
    }
    // ---- scores (this lane: head, tokens 4*g4 + r of each 16-token tile) ----
    float z[8], sv[8];
    float bmax = -INFINITY;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float raw = S[tt][r] + __shfl_xor(S[tt][r], 8, 64);   // hi + lo columns
        const int tl = 16 * tt + 4 * g4 + r;                          // token within block
        const float sk = sc[tl];
        sv[4 * tt + r] = sc[32 + tl];
        float zz = sk * fmaf(raw, c1, -c2);
        if (t0 + tl >= tok_end) zz = -INFINITY;
        z[4 * tt + r] = zz;
        bmax = fmaxf(bmax, zz);
      }
    bmax = fmaxf(bmax, wave_xor(bmax, 16));
    bmax = fmaxf(bmax, wave_xor(bmax, 32));
    const float m_new = fmaxf(m_run, bmax);
    if (__any(m_new > m_run)) {
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);   // 0 when m_run = -inf
      l_run *= alpha;
      ls_run *= alpha;
      // O rows are (head, part) = 4*g4 + r; fetch alpha of head (4*g4 + r) & 7.
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float ar = __shfl(alpha, ((4 * g4 + r) & 7), 64);
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) O[nt][r] *= ar;
      }
      m_run = m_new;
    }
    // ---- probabilities and the A operand of PV ----
    _Float16 ph[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float p = __builtin_amdgcn_exp2f(z[j] - m_run);
      l_run += p;
      const float pp = p * sv[j] * pmul;
      const _Float16 hi = (_Float16)pp;
      const _Float16 val = part ? (_Float16)(pp - (float)hi) : hi;
      ph[j] = val;
      ls_run += (float)val;
    }
    const half8 pop = half8{ph[0], ph[1], ph[2], ph[3], ph[4], ph[5], ph[6], ph[7]};
    // ---- V: unpack to LDS rows [token][slot], read back transposed ----
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      unsigned u[16];
      unpack_quarter(vw[tt][0], vw[tt][1], vw[tt][2], u);
      uint4* dst = reinterpret_cast<uint4*>(&vrow[16 * tt + n][32 * g4]);
      dst[0] = make_uint4(u[0], u[1], u[2], u[3]);
      dst[1] = make_uint4(u[4], u[5], u[6], u[7]);
      dst[2] = make_uint4(u[8], u[9], u[10], u[11]);
      dst[3] = make_uint4(u[12], u[13], u[14], u[15]);
    }
    __builtin_amdgcn_wave_barrier();
    // Transposed read: lane (g4, i) points at row 4*g4 + i/4 (+16), column 4*(i%4).
    const int trow = 4 * g4 + (n >> 2);
    const int tcol = 4 * (n & 3);
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) {
      typedef __attribute__((address_space(3))) short4v* lds_s4;
      const short4v lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4)(&vrow[trow][16 * nt + tcol]));
      const short4v hi4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4)(&vrow[16 + trow][16 * nt + tcol]));
      typedef short short8v __attribute__((ext_vector_type(8)));
      const short8v both = {lo4[0], lo4[1], lo4[2], lo4[3], hi4[0], hi4[1], hi4[2], hi4[3]};
      O[nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pop, __builtin_bit_cast(half8, both), O[nt], 0, 0, 0);
    }
    __builtin_amdgcn_wave_barrier();
  }

  // ---------------- per-wave results ----------------
  // l: the two part lanes hold identical p; count part 0 only, then sum quarters.
  float l_tot = part ? 0.f : l_run;
  l_tot += wave_xor(l_tot, 8);
  l_tot += wave_xor(l_tot, 16);
  l_tot += wave_xor(l_tot, 32);
  float ls_tot = ls_run;               // hi (part 0) + lo (part 1) over all quarters
  ls_tot += wave_xor(ls_tot, 8);
  ls_tot += wave_xor(ls_tot, 16);
  ls_tot += wave_xor(ls_tot, 32);
  // O: rows 4*g4 + r, g4 < 2 hold the hi part, g4 >= 2 the lo part of head 4*(g4&1) + r.
  floatx4 Of[8];
#pragma unroll
  for (int nt = 0; nt < 8; ++nt)
#pragma unroll
    for (int r = 0; r < 4; ++r) Of[nt][r] = O[nt][r] + __shfl_xor(O[nt][r], 32, 64);
  __syncthreads();                     // loop smem -> merge smem
  if (lane < 8) {
    sm.merge.m[wave][lane] = m_run;    // lane h holds head h (column n = h)
    sm.merge.l[wave][lane] = l_tot;
  }
  // Each lane of g4 < 2 writes o' for heads 4*g4 + r and slot 16*nt + n.
  // o'[coord] = sigma/4096 * (O * 2^(24 - p) - 3.5 * ls), ls taken from lane (head).
  {
    float lsr[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) lsr[r] = __shfl(ls_tot, (4 * (g4 & 1) + r), 64);
    if (g4 < 2) {
      const float back = sigma / kPScale;
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) {
        const int slot = 16 * nt + n;          // dim-slot: quarter slot/32, extraction slot slot%32
        const int qd = slot >> 5, s = slot & 31;
        const int coord = 32 * qd + slot_coord(s);
        const float up = ldexpf(1.f, 24 - slot_pow(s));
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int hrow = 4 * g4 + r;
          sm.merge.o[wave][hrow][coord] = back * fmaf(Of[nt][r], up, -3.5f * lsr[r]);
        }
      }
    }
  }
  __syncthreads();
  // ---------------- merge the 4 waves, write the chunk partial ----------------
  for (int idx = tid; idx < nh * 128; idx += kThreads) {
    const int hrow = idx >> 7, d = idx & 127;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, sm.merge.m[w][hrow]);
    float L = 0.f, acc = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float mw = sm.merge.m[w][hrow];
      const float f = (mw == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mw - M);
      L += f * sm.merge.l[w][hrow];
      acc += f * sm.merge.o[w][hrow][d];
    }
    const int64_t pidx = ((int64_t)b * a.Hq + h0 + hrow) * a.n_chunks + chunk_id;
    a.part_o[pidx * 128 + d] = acc;
    if (d == 0) {
      a.part_ml[pidx * 2] = M;
      a.part_ml[pidx * 2 + 1] = L;
    }
  }
}

struct CombineArgs {
  const float* part_o;
  const float* part_ml;
  const float* rot;
  int64_t rot_stride_b;
  const int32_t* seq_lens;
  int Hq, G;
  int64_t cap;
  int chunk, n_chunks;
  float* out;
};

__global__ __launch_bounds__(128) void combine_kernel(CombineArgs a) {
  __shared__ float y[128];
  __shared__ float mats[32][16];
  const int bh = blockIdx.x;
  const int b = bh / a.Hq, h = bh % a.Hq;
  const int g = h / a.G;
  const int d = threadIdx.x;
  int64_t len = a.cap;
  if (a.seq_lens) {
    const int64_t l = a.seq_lens[b];
    len = l < 0 ? 0 : (l > a.cap ? a.cap : l);
  }
  float* outp = a.out + (int64_t)bh * 128;
  if (len == 0) {
    outp[d] = 0.f;
    return;
  }
  const int nvalid = (int)((len + a.chunk - 1) / a.chunk);
  const float* ml = a.part_ml + (int64_t)bh * a.n_chunks * 2;
  const float* po = a.part_o + (int64_t)bh * a.n_chunks * 128;
  float M = -INFINITY;
  for (int c = 0; c < nvalid; ++c) M = fmaxf(M, ml[2 * c]);
  float L = 0.f, acc = 0.f;
  for (int c = 0; c < nvalid; ++c) {
    const float f = __builtin_amdgcn_exp2f(ml[2 * c] - M);
    L += f * ml[2 * c + 1];
    acc += f * po[(int64_t)c * 128 + d];
  }
  const float* rot = a.rot + b * a.rot_stride_b + (int64_t)g * 256;
  if (d < 32) build_block(rot + d * 8, mats[d]);
  y[d] = acc / L;
  __syncthreads();
  // Transposed blocks: z[4bb + i] = sum_k M_bb[k][i] o'[4bb + k].
  const int bb = d >> 2, i = d & 3;
  const float* M4 = mats[bb];
  const float zi = M4[i] * y[4 * bb] + M4[4 + i] * y[4 * bb + 1] + M4[8 + i] * y[4 * bb + 2] +
                   M4[12 + i] * y[4 * bb + 3];
  __syncthreads();
  y[d] = zi;
  __syncthreads();
  for (int m = 1; m < 128; m <<= 1) {
    const float self = y[d], other = y[d ^ m];
    __syncthreads();
    y[d] = (d & m) ? (other - self) : (self + other);
    __syncthreads();
  }
  outp[d] = y[d] * 0.08838834764831845f;
}

}  // namespace

DecodeGeometry decode_geometry(int batch, int n_q_heads, int n_kv_heads, int64_t cache_cap) {
  DecodeGeometry geo{};
  const int G = n_q_heads / n_kv_heads;
  geo.head_groups = (G + 7) / 8;
  // Aim for ~2048 work-groups; chunks are a power-of-two multiple of 128 tokens in [128, 2048].
  const int64_t units = (int64_t)batch * n_kv_heads * geo.head_groups;
  const int64_t want = (units * cache_cap + 2047) / 2048;
  int chunk = 128;
  while (chunk < 2048 && chunk < want) chunk <<= 1;
  geo.chunk = chunk;
  geo.n_chunks = (int)((cache_cap + chunk - 1) / chunk);
  const int64_t parts = (int64_t)batch * n_q_heads * geo.n_chunks;
  geo.workspace_bytes = parts * 128 * 4 + parts * 2 * 4 + 256;
  return geo;
}

hipError_t launch_decode(const DecodeLaunch& a, const DecodeGeometry& geo, hipStream_t stream) {
  const int G = a.n_q_heads / a.n_kv_heads;
  const int64_t parts = (int64_t)a.batch * a.n_q_heads * geo.n_chunks;
  float* part_o = static_cast<float*>(a.workspace);
  float* part_ml = part_o + parts * 128;
  const float sm = a.sm_scale > 0.f ? a.sm_scale : 0.08838834764831845f;

  DecodeKArgs k{};
  k.q = a.q;
  k.q_bf16 = a.q_bf16;
  k.kc = a.k_codes;
  k.ks = a.k_scales;
  k.vc = a.v_codes;
  k.vs = a.v_scales;
  k.rot = a.rot;
  k.rot_stride_b = a.rot_stride_batch;
  k.seq_lens = a.seq_lens;
  k.Hq = a.n_q_heads;
  k.Hkv = a.n_kv_heads;
  k.G = G;
  k.head_groups = geo.head_groups;
  k.cap = a.cache_cap;
  k.chunk = geo.chunk;
  k.n_chunks = geo.n_chunks;
  k.sm_log2 = sm * kLog2e;
  k.part_o = part_o;
  k.part_ml = part_ml;
  const dim3 grid1((unsigned)geo.n_chunks, (unsigned)(a.n_kv_heads * geo.head_groups), (unsigned)a.batch);
  hipLaunchKernelGGL(decode_split_kernel, grid1, dim3(kThreads), 0, stream, k);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;

  CombineArgs c{};
  c.part_o = part_o;
  c.part_ml = part_ml;
  c.rot = a.rot;
  c.rot_stride_b = a.rot_stride_batch;
  c.seq_lens = a.seq_lens;
  c.Hq = a.n_q_heads;
  c.G = G;
  c.cap = a.cache_cap;
  c.chunk = geo.chunk;
  c.n_chunks = geo.n_chunks;
  c.out = a.out;
  hipLaunchKernelGGL(combine_kernel, dim3((unsigned)(a.batch * a.n_q_heads)), dim3(128), 0, stream, c);
  return hipGetLastError();
}

}  // namespace iq
