// Decode attention computed directly on packed 3-bit K/V.
//
// Method: "RotaryQuant: Fitting 120B MoE Models on Consumer Hardware via Fused
// Compressed-Space Attention" (arXiv 2608.08081), Abstract: attention runs on
// the packed 3-bit tensors without materialising full-precision KV.
// Because R is orthogonal, q.k_hat = (Rq).(s (c - 3.5)): the query is rotated
// once, V levels are summed in rotated space, and R^T is applied once per
// (output row, chunk) partial, never per token.
//
// Record layout: one little-endian bit stream, code i at bits 3i..3i+2, so
// bytes 3g..3g+2 hold the codes of coordinates 8g..8g+7 (group g).
//
// Kernel 1 (decode_split_kernel): one work-group of 4 waves per (KV head,
// group of up to 8 query heads, (sequence, chunk of tokens) pair).  The chunk
// size is chosen on the device from the sequence lengths so that one round of
// work-groups covers the whole batch, ragged or not (plan_chunks).  Each wave
// works on its own, with no work-group barrier until the final merge:
//   * set-up (all four waves, shared through LDS): one thread per (query head,
//     SO(4) block) rotates 4 coordinates (H_4 in the thread, five cross-lane
//     Hadamard stages through DPP / swizzle, then its 4x4 block); wave w then
//     lays out K slots 8w .. 8w+7 of the fp16 A operand of the QK product, hi
//     and lo parts (q = hi + lo) in rows 2h and 2h+1, so the product carries
//     ~22 bits;
//   * with the fused append, wave 1 of the work-group whose chunk holds the
//     new token rotates, quantises and stores its K and V records first;
//   * loop over 32-token blocks with three blocks in flight: a buffer is
//     refilled three blocks ahead as soon as its codes are unpacked;
//   * codes become fp16 operands with byte permutes that pick 32-bit windows
//     and one AND per pair of codes: a field at bit p of a 16-bit half is the fp16
//     subnormal c * 2^(p-24) (p <= 7), multiplied exactly by the matrix cores;
//     the 2^-p is folded into the other operand or undone at the end;
//   * K: a lane loads one 12-byte quarter (4 groups) of one token, the B
//     operand of S[head, part][token] = q' x codes (v_mfma_f32_16x16x32_f16);
//     hi and lo rows are summed in-lane; online softmax in base 2;
//   * lazy online softmax: the running max moves only when a score passes it
//     by more than 8 (log2 units), so p <= 256; P'' = p * s_V * 16 / vlim
//     (vlim a running power of two above every V scale seen) is split hi/lo
//     in fp16 and transposed through LDS into the A operand of the PV product;
//   * V: lanes load 12-byte quarters like K (16 tokens x 4 quarters per load,
//     768 contiguous bytes), chosen so that a 4x4 transpose inside each quad of
//     lanes (two DPP exchange rounds) leaves lane (n, g4) with group n of its 8
//     tokens: exactly the B operand column n of O[head, part][coordinate 8n + j]
//     += P'' x V for the 8 tiles j.  V never passes through LDS;
//   * the 4 waves merge in LDS; each thread takes 4 coordinates of the merged
//     o' back through its transposed SO(4) block and the Hadamard (R^T is
//     linear, so the chunk partials can be rotated before they are merged)
//     and the work-group writes one (max, sum, R^T o') partial.
// The same kernel reads the record variants (template parameter kFmt): 4-bit and 2-bit uniform
// codes (fields at bits <= 6 and <= 8 of a half are exact fp16 subnormals too; other unpack
// masks, byte windows and slot maps), the asymmetric 3-bit format (the same records, an (s, m)
// pair per token: q'.(m + s c) = s (q'.c) + m sum(q'), and sum p m_V is added to every output
// coordinate) and the Lloyd-Max 3-bit format (the same records; its levels are not uniform, so
// each code enters as four exact subnormal planes, c, c & 6, c & 4 and parity(c), whose products
// are combined with fixed coefficients into the level's).
// Kernel 1b (decode_multi_kernel), several query tokens per sequence: the
// same loop for a group of two consecutive query tokens, each block's codes
// unpacked once and multiplied by both tokens' operands, each token with its
// own causal length and online softmax.
// Kernel 2 (combine_kernel): one work-group per (sequence, query head):
// log-sum-exp merge of the chunk partials, already in output coordinates.
#include "iq.h"
#include "iq_internal.h"
#include "iq_vector.h"

namespace iq {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef short short4v __attribute__((ext_vector_type(4)));
typedef short short8v __attribute__((ext_vector_type(8)));
typedef unsigned uint4v __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kBlock = 32;          // tokens per wave step
constexpr int kWavesPerSimd = 3;    // occupancy the split kernel is built for (register budget)
constexpr int kMaxSplitGroupsPerCU = kWavesPerSimd;   // most resident split work-groups per compute
                                                      // unit (one wave of each per SIMD), any format
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kHeadroom = 8.f;    // log2 units a score may exceed the running max before a rescale
constexpr float kPScale = 16.f;     // P'' = p s_V 16 / vlim <= 2^8 * 16 = 4096 (fp16 hi and lo parts in range)
constexpr float kInvSqrtD = 0.08838834764831845f;   // 1/sqrt(128)
constexpr int kMaxChunks = 1024;    // most chunks of one sequence (the combine's LDS weights)
constexpr int kFewChunks = 16;      // rows with at most this many chunks merge in registers
constexpr int kMidChunks = 64;      // above kPreloadFrom and up to this many: partials preloaded,
constexpr int kPreloadFrom = 32;    // weights through LDS

// Field j (0..7) of a 24-bit group is taken from byte window j / 3 (bytes 0-1, 1-2 or 2-3 of the
// group) at bit position field_pos(j) <= 7 of each 16-bit half.
__device__ __forceinline__ constexpr int field_pos(int j) {
  return j < 3 ? 3 * j : j < 6 ? 3 * j - 8 : 3 * j - 16;
}
__device__ __forceinline__ constexpr unsigned field_mask(int j) { return 0x00070007u << field_pos(j); }

// K slot s (0..31) of a quarter: fp16 word s/2 of the unpacked quarter, half s%2.  Words 0..7 pair
// groups 0 and 1 of the quarter (field = word), words 8..15 groups 2 and 3.
__device__ __forceinline__ int slot_coord(int s) { return 8 * (2 * (s >> 4) + (s & 1)) + ((s >> 1) & 7); }
__device__ __forceinline__ int slot_pow(int s) { return field_pos((s >> 1) & 7); }

// Unpack one 12-byte quarter (groups 0..3, little-endian words w0..w2) into 16 words of fp16
// pairs: word 8P + j holds field j of group 2P (low half) and of group 2P + 1 (high half).
// Window j / 3 of group pair P holds field j of both groups at field_pos(j) of its 16-bit halves.
__device__ __forceinline__ void quarter_windows(unsigned w0, unsigned w1, unsigned w2, unsigned (&win)[2][3]) {
  // __builtin_amdgcn_perm(hi, lo, sel): selector bytes 0-3 pick bytes of lo, 4-7 bytes of hi.
  win[0][0] = __builtin_amdgcn_perm(w1, w0, 0x04030100u);    // bytes 0,1 | 3,4
  win[0][1] = __builtin_amdgcn_perm(w1, w0, 0x05040201u);    // bytes 1,2 | 4,5
  win[0][2] = __builtin_amdgcn_perm(w1, w0, 0x06050302u);    // bytes 2,3 | 5,6
  win[1][0] = __builtin_amdgcn_perm(w2, w1, 0x06050302u);    // bytes 6,7 | 9,10
  win[1][1] = __builtin_amdgcn_perm(w2, w1, 0x07060403u);    // bytes 7,8 | 10,11
  win[1][2] = __builtin_amdgcn_perm(w2, w1, 0x07070404u);    // byte 8 | byte 11 (upper bytes unused)
}
__device__ __forceinline__ void unpack_quarter(unsigned w0, unsigned w1, unsigned w2, unsigned o[16]) {
  unsigned win[2][3];
  quarter_windows(w0, w1, w2, win);
#pragma unroll
  for (int P = 0; P < 2; ++P)
#pragma unroll
    for (int j = 0; j < 8; ++j) o[8 * P + j] = win[P][j / 3] & field_mask(j);
}

// Max's 8-level Lloyd-Max quantizer for a unit Gaussian (J. Max, 1960), levels of codes 0..7.
constexpr float kLmLevels[8] = {-2.152f, -1.344f, -0.7560f, -0.2451f, 0.2451f, 0.7560f, 1.344f, 2.152f};
// Every function of a 3-bit code c that is odd about the middle of the code range, plus a constant,
// is a combination of c, c & 6, c & 4 and the parity of c: the odd functions of the three bits
// form a 4-dimensional space spanned by the bits and their parity.  Max's levels are symmetric
// about 0 (level 7 - c = -level c), so
//   level(c) = k0 c + k1 (c & 6) + k2 (c & 4) + k3 parity(c) - A0   for all eight codes,
// with A0 = -level 0 and k0..k3 from codes 1, 2, 3 and 4.  Each plane is an exact subnormal operand
// like a uniform code, so the products stay on the matrix cores.
constexpr float kLmA0 = -kLmLevels[0];
constexpr float kLmK0 = 0.5f * ((kLmLevels[1] - kLmLevels[0]) + (kLmLevels[3] - kLmLevels[2]));
constexpr float kLmK3 = 0.5f * ((kLmLevels[1] - kLmLevels[0]) - (kLmLevels[3] - kLmLevels[2]));
constexpr float kLmK1 = 0.5f * (kLmLevels[2] - kLmLevels[0] - 2.f * kLmK0 - kLmK3);
constexpr float kLmK2 = 0.25f * (kLmLevels[4] - kLmLevels[0] - 4.f * kLmK0 - 4.f * kLmK1 - kLmK3);
// the other planes' coefficients relative to the first
constexpr float kLmR[4] = {1.f, kLmK1 / kLmK0, kLmK2 / kLmK0, kLmK3 / kLmK0};
constexpr float lm_level_of(int c) {
  return kLmK0 * c + kLmK1 * (c & 6) + kLmK2 * (c & 4) + kLmK3 * (((c >> 2) ^ (c >> 1) ^ c) & 1) - kLmA0;
}
constexpr bool lm_planes_exact() {
  for (int c = 0; c < 8; ++c) {
    const float d = lm_level_of(c) - kLmLevels[c];
    if (d > 1e-6f || d < -1e-6f) return false;
  }
  return true;
}
static_assert(lm_planes_exact(), "the four planes reproduce every Lloyd-Max level");
// Record geometry of the formats the matrix-core kernel reads: 3-bit (U3, and A3 with the same
// records), 4-bit and 2-bit uniform.  A quarter is the 32 coordinates 32 g4 .. 32 g4 + 31 of a
// record, kQW dwords; a group is 8 coordinates.
template <int kFmt>
struct Fmt {
  static constexpr int kBits = kFmt == IQ_FMT_U4 ? 4 : kFmt == IQ_FMT_U2 ? 2 : 3;
  static constexpr int kRec = 16 * kBits;             // record bytes
  static constexpr int kQW = kBits;                   // dwords of a quarter (4 kBits bytes)
  static constexpr bool kAsym = kFmt == IQ_FMT_A3;
  // Lloyd-Max levels are not uniform: each code enters as four subnormal operand planes (above),
  // whose products are combined with the planes' relative coefficients kLmR
  static constexpr bool kLloydMax = kFmt == IQ_FMT_LM3;
  static constexpr int kPlanes = kLloydMax ? 4 : 1;
  static constexpr int kSub = 24;                     // operand exponent offset undone in the scores
  // level(c) = kGain (sum over planes e of kLmR[e] plane_e(c)) - kCenter; a uniform code is its own
  // single plane (kGain 1, kCenter the middle of the code range)
  static constexpr float kCenter = kFmt == IQ_FMT_U4 ? 7.5f : kFmt == IQ_FMT_U2 ? 1.5f : kFmt == IQ_FMT_LM3 ? kLmA0 : 3.5f;
  static constexpr float kGain = kFmt == IQ_FMT_LM3 ? kLmK0 : 1.f;
};


// The four planes of one window word w (two codes at bits pos..pos+2 of each 16-bit half) given its
// parity fold f = w ^ (w >> 1) ^ (w >> 2): the codes, the codes & 6, the codes & 4 and their parities,
// each at the codes' bit position (so one query operand serves all four).
__device__ __forceinline__ void planes_of(unsigned w, unsigned f, int pos, unsigned (&o)[4]) {
  o[0] = w & (0x00070007u << pos);
  o[1] = w & (0x00060006u << pos);
  o[2] = w & (0x00040004u << pos);
  o[3] = f & (0x00010001u << pos);
}
__device__ __forceinline__ unsigned parity_fold(unsigned w) { return w ^ (w >> 1) ^ (w >> 2); }
// K slot s (0..31) of a quarter: the coordinate it holds and the bit position of its field.
//  3-bit: as slot_coord / slot_pow.
//  4-bit: word w = s/2 holds (dword w/4 = group w/4) & 0x000F000F or & 0x00F000F0, unshifted (w%4 <
//         2) or shifted right 8 bits: coordinates t and t + 4 of the group (t = w%4) at bit 4 (t%2).
//  2-bit: word w holds dword w/8 (16 coordinates) & (0x00030003 << 2t) for t = w%8 <= 4, else the
//         dword shifted right 8 bits & (0x00030003 << 2(t-4)): coordinates t and t + 8.
template <int kFmt>
__device__ __forceinline__ int slot_coord_f(int s) {
  const int w = s >> 1;
  if constexpr (Fmt<kFmt>::kBits == 3) return slot_coord(s);
  else if constexpr (Fmt<kFmt>::kBits == 4) return 8 * (w >> 2) + (w & 3) + 4 * (s & 1);
  else return 16 * (w >> 3) + (w & 7) + 8 * (s & 1);
}
template <int kFmt>
__device__ __forceinline__ int slot_pow_f(int s) {
  const int t = (s >> 1) & 7;
  if constexpr (Fmt<kFmt>::kBits == 3) return slot_pow(s);
  else if constexpr (Fmt<kFmt>::kBits == 4) return 4 * (t & 1);
  else return t <= 4 ? 2 * t : 2 * (t - 4);
}

// Unpacks one K quarter into the 16 fp16-pair words of the 4 QK products (words 4kb..4kb+3).
template <int kFmt>
__device__ __forceinline__ void unpack_k(const unsigned (&w)[Fmt<kFmt>::kQW], unsigned o[16]) {
  if constexpr (Fmt<kFmt>::kBits == 3) {
    unpack_quarter(w[0], w[1], w[2], o);
  } else if constexpr (Fmt<kFmt>::kBits == 4) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const unsigned h = w[k] >> 8;
      o[4 * k] = w[k] & 0x000F000Fu;
      o[4 * k + 1] = w[k] & 0x00F000F0u;
      o[4 * k + 2] = h & 0x000F000Fu;
      o[4 * k + 3] = h & 0x00F000F0u;
    }
  } else {
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const unsigned h = w[k] >> 8;
#pragma unroll
      for (int t = 0; t < 8; ++t) o[8 * k + t] = t <= 4 ? w[k] & (0x00030003u << (2 * t)) : h & (0x00030003u << (2 * (t - 4)));
    }
  }
}

// V operand of the PV product for output field j (coordinate 8n + j): which byte window of a token
// pair holds it, at which bit position, under which mask.
template <int kFmt>
struct VField {
  static constexpr int kWin = Fmt<kFmt>::kBits == 3 ? 3 : Fmt<kFmt>::kBits == 4 ? 4 : 2;   // windows per pair
  __device__ __forceinline__ static constexpr int win(int j) {
    return Fmt<kFmt>::kBits == 3 ? j / 3 : Fmt<kFmt>::kBits == 4 ? j / 2 : (j <= 4 ? 0 : 1);
  }
  __device__ __forceinline__ static constexpr int pos(int j) {
    return Fmt<kFmt>::kBits == 3 ? field_pos(j) : Fmt<kFmt>::kBits == 4 ? 4 * (j & 1) : (j <= 4 ? 2 * j : 2 * (j - 4));
  }
  __device__ __forceinline__ static constexpr unsigned mask(int j) {
    return Fmt<kFmt>::kBits == 3 ? field_mask(j) : Fmt<kFmt>::kBits == 4 ? 0x000F000Fu << pos(j) : 0x00030003u << pos(j);
  }
};

__device__ __forceinline__ half8 as_half8(unsigned a, unsigned b, unsigned c, unsigned d) {
  uint4v v = {a, b, c, d};
  return __builtin_bit_cast(half8, v);
}

__device__ __forceinline__ float dpp_xor1(float x) {   // quad_perm [1,0,3,2]
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, false));
}
__device__ __forceinline__ float dpp_xor2(float x) {   // quad_perm [2,3,0,1]
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, false));
}
__device__ __forceinline__ float swz_xor4(float x) {   // bitmask swizzle, xor 4
  return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), (4 << 10) | 0x1F));
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
  int batch, Hq, Hkv, G, head_groups;   // batch: work-item sequences (see LenSource)
  int q_tokens;           // query tokens per cached sequence
  int q_group;            // query tokens per work-item sequence (1, or the multi-token kernel's kQ)
  int n_groups;           // work-item sequences per cached sequence: ceil(q_tokens / q_group)
  int64_t cap;
  int target;             // most (sequence, chunk) pairs per (KV head, head group) column
  float sm_log2;          // softmax scale times log2(e)
  int* plan;              // [0]: chunk size; [64 + b]: index of sequence b's first chunk
  int x_max;              // partial rows per query head: work items per column (times kQ in the
                          // multi-token kernel, whose work item x writes rows x kQ + i)
  int guess_per_seq;      // chunks per sequence when every length is cap (a guess, see below)
  float* part_o;          // [Hq][x_max][128], x = index of the (sequence, chunk) pair
  float* part_ml;         // [Hq][x_max][2]  (max in log2 units, sum)
  // fused append (positions != NULL): new token of sequence b written at positions[b]
  const int32_t* positions;
  const void* k_new;
  const void* v_new;
  int new_bf16;
  int64_t new_stride_seq, new_stride_head;
};

// ---------------- split of the context into chunks ----------------
// The sequences' lengths decide the chunk size, so that ragged batches fill the GPU as evenly as
// full ones: every work-group computes the same plan from the lengths (no extra launch, no host
// round trip).  Chunks are multiples of 128 tokens (one step of the 4 waves), at least 256.
struct LenSource {
  const int32_t* positions;   // fused append: length = position + 1 (0 outside the cache)
  const int32_t* seq_lens;    // else the given lengths clamped to [0, cap]; NULL: every length cap
  int cap, batch;
  // Several query tokens per cached sequence (causal: they are its last q_tokens positions, token t
  // sees len - (q_tokens - 1 - t) of them): sequence i is group i % n_groups of cache i / n_groups,
  // the group holding tokens q_group (i % n_groups) .. q_group (i % n_groups + 1) - 1, and its
  // length is that of its last token.  q_group = 1: one sequence per token.
  int q_tokens, q_group, n_groups;
};

// The stored value for sequence i (a position or a length; 0 when there is none), then its length.
__device__ __forceinline__ int len_raw(const LenSource& s, int i) {
  const int32_t* src = s.positions ? s.positions : s.seq_lens;
  if (src == nullptr || i >= s.batch) return 0;
  return src[s.n_groups > 1 ? i / s.n_groups : i];
}
__device__ __forceinline__ int len_of(const LenSource& s, int i, int raw) {
  if (i >= s.batch) return 0;
  if (s.positions) return (raw >= 0 && raw < s.cap) ? raw + 1 : 0;
  int l = s.seq_lens ? (raw < 0 ? 0 : (raw > s.cap ? s.cap : raw)) : s.cap;
  if (s.q_tokens > 1) {                          // causal: the last q_tokens positions are the queries
    const int later = s.q_tokens - (i % s.n_groups + 1) * s.q_group;   // tokens after the group
    if (later > 0) l -= later;
    if (l < 0) l = 0;
  }
  return l;
}
__device__ __forceinline__ int len_at(const LenSource& s, int i) { return len_of(s, i, len_raw(s, i)); }

__device__ __forceinline__ long long chunk_round(long long v) {   // up to a multiple of 128, >= 256
  v = (v + 127) / 128 * 128;
  return v < 256 ? 256 : v;
}

// Inclusive prefix sum over the 64 lanes: row shifts 1, 2, 4, 8 scan each row of 16 lanes, then
// row_bcast:15 adds row 0's total into rows 1 and 3 and row_bcast:31 adds rows 0-1 into rows 2-3.
// Lanes without a source take the `old` operand, 0.
__device__ __forceinline__ int wave_scan_add(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, false);   // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, false);   // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, false);   // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, false);   // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);   // row_bcast:15, rows 1 and 3
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);   // row_bcast:31, rows 2 and 3
  return x;
}
// Running maximum of non-negative values in the same pattern; lane 63 holds the wave's maximum.
__device__ __forceinline__ int wave_scan_max(int x) {
  x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, false));
  x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, false));
  x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, false));
  x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, false));
  x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false));
  x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false));
  return x;
}
__device__ __forceinline__ int lane63(int x) { return __builtin_amdgcn_readlane(x, 63); }

// Sum over sequences of ceil(len / c).  `l0` is this lane's length of sequences 0..63.
__device__ __forceinline__ long long count_chunks(const LenSource& s, int l0, int c, int lane) {
  long long n = 0;
  for (int base = 0; base < s.batch; base += 64) {
    const int l = base == 0 ? l0 : len_at(s, base + lane);
    n += lane63(wave_scan_add((l + c - 1) / c));
  }
  return n;
}

struct ChunkPlan {
  int chunk;    // tokens per chunk
  int b;        // sequence of work item x (-1: x is past the last chunk)
  int j;        // chunk of that sequence
  int len;      // its length
};

// Work item x of a plan with chunk size c: chunk x - first(b) of the sequence b with
// first(b) <= x < first(b + 1), chunks numbered sequence by sequence.  `incl` is the inclusive scan
// of this lane's chunk count n over the 64 sequences base..base+63 (plus the earlier ones).
__device__ __forceinline__ bool locate(ChunkPlan& p, int base, int batch, int x, int incl, int n, int l) {
  const unsigned long long mask = __ballot(incl > x);
  if (!mask) return false;
  const int f = __builtin_ctzll(mask);
  if (base + f < batch) {
    p.b = base + f;
    p.j = x - __builtin_amdgcn_readlane(incl - n, f);
    p.len = __builtin_amdgcn_readlane(l, f);
  }
  return true;
}

// The smallest chunk size c (within the rounding above) whose number of chunks, summed over the
// sequences, is at most `target`, so one round of work-groups covers the batch; then the
// sequence and chunk of work item x.  Wave-uniform; every wave of the work-group computes it.
// Bounds used: sum ceil(l / c) <= 128 units / c + nz (units = sum ceil(l / 128), nz = sequences
// with tokens), so c >= 128 units / (target - nz) meets the target when target > nz; otherwise
// one chunk per sequence.
__device__ ChunkPlan plan_chunks(const LenSource& s, int l0, int target, int x, int lane) {
  ChunkPlan p{256, -1, -1, 0};
  if (s.batch <= 64) {                 // one sequence per lane; 32-bit (units <= 64 * 2^20)
    const int units = lane63(wave_scan_add((l0 + 127) >> 7));
    const int nz = __builtin_popcountll(__ballot(l0 > 0));
    const int cmax = (int)chunk_round(lane63(wave_scan_max(l0)));
    const int q = (int)(((unsigned)units + target - 1) / (unsigned)target);
    int c = q >= (cmax >> 7) ? cmax : (int)chunk_round((long long)q * 128);
    int n = (l0 + c - 1) / c;
    int incl = wave_scan_add(n);
    if (lane63(incl) > target) {       // too many chunks: search between the bounds
      if (target > nz) {
        int lo = c;
        const unsigned qh = ((unsigned)units + (target - nz) - 1) / (unsigned)(target - nz);
        int hi = qh >= (unsigned)(cmax >> 7) ? cmax : (int)chunk_round((long long)qh * 128);
        while (hi - lo > 128) {
          const int mid = lo + (hi - lo) / 256 * 128;
          if (lane63(wave_scan_add((l0 + mid - 1) / mid)) <= target) hi = mid; else lo = mid;
        }
        c = hi;
      } else {
        c = cmax;
      }
      n = (l0 + c - 1) / c;
      incl = wave_scan_add(n);
    }
    p.chunk = c;
    locate(p, 0, s.batch, x, incl, n, l0);
    return p;
  }
  // any batch size: 64 sequences per pass, 64-bit sums
  long long units = 0;
  int nz = 0, maxl = 0;
  for (int base = 0; base < s.batch; base += 64) {
    const int l = base == 0 ? l0 : len_at(s, base + lane);
    units += lane63(wave_scan_add((l + 127) >> 7));
    nz += __builtin_popcountll(__ballot(l > 0));
    maxl = max(maxl, lane63(wave_scan_max(l)));
  }
  const long long cmax = chunk_round(maxl);
  long long c = chunk_round((units + target - 1) / target * 128);
  if (c < cmax && count_chunks(s, l0, (int)c, lane) > target) {
    if (target > nz) {
      long long lo = c, hi = chunk_round((units + (target - nz) - 1) / (target - nz) * 128);
      if (hi > cmax) hi = cmax;
      while (hi - lo > 128) {
        const long long mid = lo + (hi - lo) / 256 * 128;
        if (count_chunks(s, l0, (int)mid, lane) <= target) hi = mid; else lo = mid;
      }
      c = hi;
    } else {
      c = cmax;
    }
  }
  if (c > cmax) c = cmax;
  p.chunk = (int)c;
  int offset = 0;
  for (int base = 0; base < s.batch; base += 64) {
    const int l = base == 0 ? l0 : len_at(s, base + lane);
    const int n = (l + p.chunk - 1) / p.chunk;
    const int incl = wave_scan_add(n) + offset;
    if (locate(p, base, s.batch, x, incl, n, l)) return p;
    offset = lane63(incl);
  }
  return p;
}

template <int kW>
struct MergeSmemT {
  float o[kW][8][128];
  float m[kW][8];
  float l[kW][8];
};
using MergeSmem = MergeSmemT<kWaves>;
// Per-wave loop staging: the P'' block [32 tokens][16 (head, part)] fp16 (32-byte rows) and the
// block's K/V scales.
constexpr int kPRow = 32;
template <int kP>
struct WaveLoopSmemT {
  char p[kP][kBlock * kPRow];   // one staging block per operand plane
  float sc[64];           // the block's K scales (lanes 0-31) and V scales (lanes 32-63)
  float mn[64];           // asymmetric format: the matching minima m
};
// Computed once per work-group: the rotated queries, the sum of q' and the operand exponent E of
// each head.  Shares storage with the loop staging (a barrier separates them).
struct SetupSmem {
  float qrot[8][128];
  float qsum[8];
  int E[8];
};
template <int kW, int kP>
union DecodeSmemU {
  WaveLoopSmemT<kP> loop[kW];
  SetupSmem setup;
};
// The QK A operand in lane order (the same for every wave), built once and read from LDS for
// every block, which keeps 16 registers per lane free for a second block in flight.  The merge
// area has its own storage, so a wave writes its results as soon as its loop ends, while other
// waves still use their loop staging.
template <int kW, int kP>
struct DecodeSmem {
  uint4v qop[4][64];
  float blk[32][16];      // the KV head's SO(4) blocks, for the inverse rotation of the partials
  MergeSmemT<kW> merge;
  DecodeSmemU<kW, kP> u;
};

__device__ __forceinline__ void build_block(const float* p, float* out16) {
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

// Token order of the PV product: K slot e of row group g4 is token 4*g4 + e (e < 4) or
// 16 + 4*g4 + e - 4 (e >= 4) of the block, for both operands.
__device__ __forceinline__ constexpr int pv_token(int g4, int e) { return e < 4 ? 4 * g4 + e : 12 + 4 * g4 + e; }

template <int kQW>
struct BlockData {
  unsigned kw[2][kQW];    // K quarter g4 of tokens n and 16 + n
  unsigned vw[2][kQW];    // V quarter (lane >> 2) & 3 of tokens 16t + 4 g4 + (lane & 3), t = 0, 1
  unsigned ksc, vsc;      // K and V scale bits of token n (row groups 0, 2) or 16 + n (1, 3);
                          // asymmetric format: this lane's (s, m) pair, of K (lanes 0-31) or V
};

// Per-lane constant byte offsets within a 32-token block.
struct LaneOffsets {
  unsigned kcode;         // byte offset of this lane's K quarter (token n; token 16 + n is 16 records on)
  unsigned vcode;         // byte offset of this lane's V quarter (token 4 g4 + (lane & 3); t = 1: 16 records on)
  unsigned scale;         // byte offset of this lane's scale (token n or 16 + n)
  bool vside;             // lanes 32-63: the V scale (asymmetric format: the V (s, m) pair)
};

// Raw buffer resources over one (sequence, KV head)'s codes and scales.  Every access puts its
// whole offset in the range-checked part of the address, so one past the end of the slice reads
// zeros without reaching memory (a partial last block needs no clamping: those tokens are masked
// out of the softmax anyway).
struct CacheBuffers {
  __amdgpu_buffer_rsrc_t kc, vc, ks, vs;
};

constexpr int kBufferConfig = 0x00020000;   // raw (untyped) buffer, 32-bit data format

// Byte range of a buffer resource over `cap` records of `rec` bytes.  The product is formed in
// unsigned arithmetic: at the largest accepted capacity it exceeds INT_MAX (but stays below
// 0xF0000000), and the resource field takes its 32-bit pattern.
__device__ __forceinline__ int range_bytes(int cap, int rec) { return (int)((unsigned)cap * (unsigned)rec); }

// Block base for a block that is not to be read: beyond every slice (capacity times the record
// size is validated to stay below it), so its loads return zeros without reaching memory.
constexpr unsigned kNoBlock = 0xF0000000u;

// Cache policy of every load of the packed cache (codes and scales) in the split kernel:
// non-temporal.  A decode call reads each record once, and a model's layers together stream far
// more than the 256 MB last-level cache between two reads of one layer: loads that allocate
// normally keep evicting lines for data that is not read again in time.  The hint took the
// 48-layer step (654 MB) from 123 to 112 us on the same box.  The records still come through the
// caches, so a record appended by the same work-group is read back.  A single call whose records
// fit the last-level cache, replayed back to back, loses its hits across calls with the hint (the
// 16-sequence ragged batch, 182 MB: 41.2 against 38.7 us), which a model with more layers than
// one would not see.  The multi-token kernel keeps the default policy: several token groups read
// each record within one call, and their re-reads hit the caches (Q = 16 on the 48-layer cache:
// 0.88 ms, 0.92 ms with the hint).
constexpr int kRecordLoadPolicy = 2;   // the NT bit of the cache-policy operand
constexpr int kSharedLoadPolicy = 0;   // default caching

// Keeps v in a register as an opaque value, so per-load constants added to it stay immediate
// offsets instead of becoming separate loop-invariant registers.
__device__ __forceinline__ unsigned opaque(unsigned v) {
  asm volatile("" : "+v"(v));
  return v;
}

// Issues the loads of the block at token t0, or, if t0 is not below tok_end, loads that read
// zeros without a memory access.  The whole offset is in the range-checked part of the buffer
// address (vector offset plus immediate), so tokens past the end of the slice read as zeros too.
// Loads one quarter (kQW dwords) at byte offset off of buffer r.
template <int kQW, int kPolicy>
__device__ __forceinline__ void load_quarter(unsigned (&w)[kQW], __amdgpu_buffer_rsrc_t r, unsigned off) {
  if constexpr (kQW == 3) {
    typedef unsigned u3v __attribute__((ext_vector_type(3)));
    const u3v q = __builtin_amdgcn_raw_buffer_load_b96(r, off, 0, kPolicy);
    w[0] = q.x; w[1] = q.y; w[2] = q.z;
  } else if constexpr (kQW == 4) {
    typedef unsigned u4v __attribute__((ext_vector_type(4)));
    const u4v q = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kPolicy);
    w[0] = q.x; w[1] = q.y; w[2] = q.z; w[3] = q.w;
  } else {
    typedef unsigned u2v __attribute__((ext_vector_type(2)));
    const u2v q = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, kPolicy);
    w[0] = q.x; w[1] = q.y;
  }
}

template <int kFmt, int kPolicy = kRecordLoadPolicy>
__device__ __forceinline__ void load_block(BlockData<Fmt<kFmt>::kQW>& d, const CacheBuffers& cb, int t0, int tok_end,
                                           const LaneOffsets& lo) {
  constexpr bool kAsym = Fmt<kFmt>::kAsym;
  constexpr unsigned kRec = Fmt<kFmt>::kRec;
  const bool in = t0 < tok_end;                                      // uniform
  const unsigned base = in ? (unsigned)t0 * kRec : kNoBlock;
  const unsigned ko = opaque(lo.kcode + base), vo = opaque(lo.vcode + base);
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) load_quarter<Fmt<kFmt>::kQW, kPolicy>(d.kw[tt], cb.kc, ko + 16 * kRec * tt);
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) load_quarter<Fmt<kFmt>::kQW, kPolicy>(d.vw[tt], cb.vc, vo + 16 * kRec * tt);
  if constexpr (kAsym) {
    // each lane loads the (s, m) pair it stages, under an exec mask: K in lanes 0-31, V in 32-63
    typedef unsigned u2v __attribute__((ext_vector_type(2)));
    const unsigned so = 2 * lo.scale + (in ? (unsigned)t0 * 8u : kNoBlock);
    u2v sm;
    if (lo.vside)
      sm = __builtin_amdgcn_raw_buffer_load_b64(cb.vs, so, 0, kPolicy);
    else
      sm = __builtin_amdgcn_raw_buffer_load_b64(cb.ks, so, 0, kPolicy);
    d.ksc = sm.x;
    d.vsc = sm.y;
  } else {
    // Both scale loads run in every lane (keeps the resources uniform); the block's consumer picks
    // one, so nothing here waits for the loads.
    const unsigned so = lo.scale + (in ? (unsigned)t0 * 4u : kNoBlock);
    d.ksc = __builtin_amdgcn_raw_buffer_load_b32(cb.ks, so, 0, kPolicy);
    d.vsc = __builtin_amdgcn_raw_buffer_load_b32(cb.vs, so, 0, kPolicy);
  }
}

// Running state of one wave's online softmax.  Lane (n, g4) owns heads 2*g4 and 2*g4+1.
struct WaveState {
  floatx4 O[8];           // O[j][(head, part)][n]: coordinate 8n + j, rows 4*g4 + r = (head 2*g4 + r/2, part r%2)
  float m_run[2];         // running max (log2 units), uniform over the 16 lanes of a row group
  float thr[2];           // m_run + kHeadroom: a score above it moves the running max
  float l_run[2];         // sum of p over this lane's tokens
  float ls_run[2];        // sum of P'' over this lane's tokens (asymmetric format: sum of p m_V)
  int vexp;               // vlim = 2^vexp is above every V scale seen; -200: none yet
  float vlim;             // 2^vexp (0 before the first block)
  float pmul;             // kPScale / vlim
};

__device__ __forceinline__ float row_max(float x) {   // max over the 16 lanes of a row (DPP row_ror)
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xF, 0xF, true)));
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x124, 0xF, 0xF, true)));
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x122, 0xF, 0xF, true)));
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x121, 0xF, 0xF, true)));
  return x;
}
__device__ __forceinline__ float row_sum(float x) {   // sum over the 16 lanes of a row
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xF, 0xF, true));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x124, 0xF, 0xF, true));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x122, 0xF, 0xF, true));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x121, 0xF, 0xF, true));
  return x;
}

typedef __attribute__((address_space(3))) short4v* lds_s4;

// 4x4 transpose of words inside each quad of lanes: lane x (= lane & 3) ends with g[c] equal to
// the g[x] that lane c of its quad held (two exchange rounds: partners x ^ 1, then x ^ 2).
__device__ __forceinline__ unsigned dpp_xor1_u(unsigned x) {
  return (unsigned)__builtin_amdgcn_mov_dpp((int)x, 0xB1, 0xF, 0xF, false);
}
__device__ __forceinline__ unsigned dpp_xor2_u(unsigned x) {
  return (unsigned)__builtin_amdgcn_mov_dpp((int)x, 0x4E, 0xF, 0xF, false);
}
__device__ __forceinline__ void quad_transpose(unsigned g[4], int lane) {
  (void)lane;
  // Each round is four v_cndmask_b32 with a DPP source: dst = (lane keeps) ? own : partner's
  // other register.  Round 1 (partner lane ^ 1): even lanes keep g[0], g[2] and take the partner's
  // g[0], g[2] into g[1], g[3]; odd lanes the reverse.  Round 2 (partner lane ^ 2) does the same
  // for the register pairs (0, 2) and (1, 3).  The masks go through VCC; the s_nop gives the DPP
  // reads their wait states after the VALU writes of the sources.
  const unsigned long long even = 0x5555555555555555ull, lower = 0x3333333333333333ull;
  unsigned h[4];
  asm("s_mov_b64 vcc, %8\n\t"
      "s_nop 1\n\t"
      "v_cndmask_b32_dpp %0, %5, %4, vcc quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
      "v_cndmask_b32_dpp %2, %7, %6, vcc quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
      "s_not_b64 vcc, vcc\n\t"
      "s_nop 0\n\t"
      "v_cndmask_b32_dpp %1, %4, %5, vcc quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t"
      "v_cndmask_b32_dpp %3, %6, %7, vcc quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf"
      : "=&v"(h[0]), "=&v"(h[1]), "=&v"(h[2]), "=&v"(h[3])
      : "v"(g[0]), "v"(g[1]), "v"(g[2]), "v"(g[3]), "s"(even)
      : "vcc");
  asm("s_mov_b64 vcc, %8\n\t"
      "s_nop 1\n\t"
      "v_cndmask_b32_dpp %0, %6, %4, vcc quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
      "v_cndmask_b32_dpp %1, %7, %5, vcc quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
      "s_not_b64 vcc, vcc\n\t"
      "s_nop 0\n\t"
      "v_cndmask_b32_dpp %2, %4, %6, vcc quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t"
      "v_cndmask_b32_dpp %3, %5, %7, vcc quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf"
      : "=&v"(g[0]), "=&v"(g[1]), "=&v"(g[2]), "=&v"(g[3])
      : "v"(h[0]), "v"(h[1]), "v"(h[2]), "v"(h[3]), "s"(lower)
      : "vcc");
}


// Sets the wave's issue priority from its progress through its chunk: 3 below 70% of the chunk,
// 2 below 90%, 1 below 97.5%, 0 after.  At equal priority a SIMD's arbiter prefers older waves,
// so the first work-group resident on a compute unit would run ahead and the last one would
// stream alone at the end with one wave per SIMD; dropping the priority of the waves that are
// further along keeps the work-groups of a compute unit in step.  (done, span: tokens, uniform.)
__device__ __forceinline__ void progress_priority(int done, int span) {
  const long long d = done, s = span;
  if (10 * d < 7 * s)
    __builtin_amdgcn_s_setprio(3);
  else if (10 * d < 9 * s)
    __builtin_amdgcn_s_setprio(2);
  else if (40 * d < 39 * s)
    __builtin_amdgcn_s_setprio(1);
  else
    __builtin_amdgcn_s_setprio(0);
}

// Processes the block in `cur` (`rem` valid tokens), then refills `cur` with the block at
// t_refill as soon as the current codes are unpacked; the refill loads are unconditional (zeros
// past the chunk), so the wait for a buffer at the top of a block leaves newer loads in flight.
template <bool kRefill, int kFmt>
__device__ __forceinline__ void process_block(BlockData<Fmt<kFmt>::kQW>& cur, int rem, int t_refill, int tok_end,
                                              const CacheBuffers& cb, const LaneOffsets& lo, bool vscale,
                                              WaveState& st, const uint4v (&qop)[4][64], const float (&c1)[2],
                                              const float (&c2)[2], WaveLoopSmemT<Fmt<kFmt>::kPlanes>& ws, int lane,
                                              int n, int g4, unsigned pwr, unsigned prd) {
  constexpr bool kAsym = Fmt<kFmt>::kAsym;
  constexpr int kP = Fmt<kFmt>::kPlanes;
  if constexpr (kAsym) {
    ws.sc[lane] = __uint_as_float(cur.ksc);
    ws.mn[lane] = __uint_as_float(cur.vsc);
  } else {
    ws.sc[lane] = __uint_as_float(vscale ? cur.vsc : cur.ksc);
  }
  // ---- QK: S[(head, part)][token] = q' x codes, tile tt = tokens 16*tt + column ----
  floatx4 S[2];
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    if constexpr (Fmt<kFmt>::kLloydMax) {
      // each plane on the same query operand into its own accumulator, then combined with the
      // planes' coefficients relative to the first (the first's goes into the score scale)
      unsigned win[2][3], fold[2][3];
      quarter_windows(cur.kw[tt][0], cur.kw[tt][1], cur.kw[tt][2], win);
#pragma unroll
      for (int P = 0; P < 2; ++P)
#pragma unroll
        for (int k = 0; k < 3; ++k) fold[P][k] = parity_fold(win[P][k]);
      floatx4 acc[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {             // words 4 kb .. 4 kb + 3 of unpack_quarter's order
        unsigned pl[4][4];                          // [word][plane]
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int w = 4 * kb + i, P = w >> 3, j = w & 7;
          planes_of(win[P][j / 3], fold[P][j / 3], field_pos(j), pl[i]);
        }
        const half8 qa = __builtin_bit_cast(half8, qop[kb][lane]);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          acc[e] = __builtin_amdgcn_mfma_f32_16x16x32_f16(qa, as_half8(pl[0][e], pl[1][e], pl[2][e], pl[3][e]),
                                                          acc[e], 0, 0, 0);
      }
      S[tt] = acc[0] + kLmR[1] * acc[1] + kLmR[2] * acc[2] + kLmR[3] * acc[3];
    } else {
      unsigned u[16];
      unpack_k<kFmt>(cur.kw[tt], u);
      floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, qop[kb][lane]),
                                                    as_half8(u[4 * kb], u[4 * kb + 1], u[4 * kb + 2], u[4 * kb + 3]),
                                                    acc, 0, 0, 0);
      S[tt] = acc;
    }
  }
  // ---- V: each lane holds quarter y = (lane >> 2) & 3 (groups 4y..4y+3) of the tokens
  //      16t + 4 g4 + x, x = lane & 3; a 4x4 transpose inside each quad of lanes leaves lane x with
  //      group 4y + x = n of the quad's four tokens, in token order: B operand column n in the
  //      token order of the PV product.  Then the byte windows of each token pair (3-bit: bytes
  //      0-1, 1-2, 2-3 of the group; 4-bit: byte b of each token's group in bytes 0 and 2; 2-bit:
  //      the two groups side by side, and that shifted right 8 bits). ----
  constexpr int kWin = VField<kFmt>::kWin;
  unsigned vwin[4][kWin];
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    unsigned gq[4];                                                  // group k from byte 0
    if constexpr (Fmt<kFmt>::kBits == 3) {
      gq[0] = cur.vw[tt][0];
      gq[1] = __builtin_amdgcn_alignbyte(cur.vw[tt][1], cur.vw[tt][0], 3);
      gq[2] = __builtin_amdgcn_alignbyte(cur.vw[tt][2], cur.vw[tt][1], 2);
      gq[3] = cur.vw[tt][2] >> 8;
    } else if constexpr (Fmt<kFmt>::kBits == 4) {
#pragma unroll
      for (int k = 0; k < 4; ++k) gq[k] = cur.vw[tt][k];
    } else {                                                         // upper halves unused
      gq[0] = cur.vw[tt][0];
      gq[1] = cur.vw[tt][0] >> 16;
      gq[2] = cur.vw[tt][1];
      gq[3] = cur.vw[tt][1] >> 16;
    }
    quad_transpose(gq, lane);
#pragma unroll
    for (int p = 0; p < 2; ++p) {                                    // tokens 2p and 2p + 1 of the quad
      unsigned* vw = vwin[2 * tt + p];
      if constexpr (Fmt<kFmt>::kBits == 3) {
        vw[0] = __builtin_amdgcn_perm(gq[2 * p + 1], gq[2 * p], 0x05040100u);   // bytes 0-1
        vw[1] = __builtin_amdgcn_perm(gq[2 * p + 1], gq[2 * p], 0x06050201u);   // bytes 1-2
        vw[2] = __builtin_amdgcn_perm(gq[2 * p + 1], gq[2 * p], 0x07060302u);   // bytes 2-3
      } else if constexpr (Fmt<kFmt>::kBits == 4) {
#pragma unroll
        for (int b = 0; b < 4; ++b)                                   // byte b of each, upper bytes zero
          vw[b] = __builtin_amdgcn_perm(gq[2 * p + 1], gq[2 * p], 0x0C000C00u | ((4u + b) << 16) | (unsigned)b);
      } else {
        vw[0] = __builtin_amdgcn_perm(gq[2 * p + 1], gq[2 * p], 0x05040100u);
        vw[1] = vw[0] >> 8;
      }
    }
  }
  // ---- the codes are in registers now: refill the buffer.  The scheduling barrier keeps the
  //      loads behind the last reads of the old contents, so they land in the same registers
  //      (no copies, and no waits for them, at the loop back-edge). ----
  if (kRefill) {
    __builtin_amdgcn_sched_barrier(0);
    load_block<kFmt>(cur, cb, t_refill, tok_end, lo);
  }
  // ---- scores: heads 2*g4 + j, tokens n (tile 0) and 16 + n (tile 1) ----
  const float sk0 = ws.sc[n], sk1 = ws.sc[16 + n];
  float sv0 = ws.sc[32 + n], sv1 = ws.sc[48 + n];
  float z[2][2];
  float mv[2] = {0.f, 0.f};                                   // asymmetric format: V minima
  if constexpr (kAsym) {
    // q'.(m + s c) = s (q'.c) + m sum(q'): c2[j] is log2(e) sm sum(q') of head 2*g4 + j
    const float mk0 = ws.mn[n], mk1 = ws.mn[16 + n];
    mv[0] = ws.mn[32 + n];
    mv[1] = ws.mn[48 + n];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      z[j][0] = fmaf(sk0 * c1[j], S[0][2 * j] + S[0][2 * j + 1], mk0 * c2[j]);
      z[j][1] = fmaf(sk1 * c1[j], S[1][2 * j] + S[1][2 * j + 1], mk1 * c2[j]);
    }
  } else {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      z[j][0] = sk0 * fmaf(S[0][2 * j] + S[0][2 * j + 1], c1[j], -c2[j]);
      z[j][1] = sk1 * fmaf(S[1][2 * j] + S[1][2 * j + 1], c1[j], -c2[j]);
    }
  }
  if (rem < kBlock) {                                         // last, partial block only
    if (n >= rem) { z[0][0] = z[1][0] = -INFINITY; sv0 = 0.f; }
    if (16 + n >= rem) { z[0][1] = z[1][1] = -INFINITY; sv1 = 0.f; }
  }
  // Lazy rescaling: the running max only moves when a score exceeds it by more than kHeadroom
  // (so p <= 2^kHeadroom), or when a V scale reaches the running power-of-two bound.
  const float svmax = fmaxf(sv0, sv1);
  const bool grow_l = (fmaxf(z[0][0], z[0][1]) > st.thr[0]) | (fmaxf(z[1][0], z[1][1]) > st.thr[1]) |
                      (svmax >= st.vlim);
  if (__any(grow_l)) {
    const float vmax = row_max(svmax);                         // same in every row: wave-uniform
    float ratio = 1.f;
    if (vmax >= st.vlim) {
      int ex;
      frexpf(vmax, &ex);                                       // vmax < 2^ex
      ex = ex < -60 ? -60 : ex;
      ratio = st.vexp == -200 ? 0.f : ldexpf(1.f, st.vexp - ex);
      st.vexp = ex;
      st.vlim = ldexpf(1.f, ex);
      st.pmul = ldexpf(kPScale, -ex);
    }
    float f[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const float m_new = fmaxf(st.m_run[j], row_max(fmaxf(z[j][0], z[j][1])));
      const float alpha = __builtin_amdgcn_exp2f(st.m_run[j] - m_new);   // 0 when m_run = -inf
      st.l_run[j] *= alpha;
      st.ls_run[j] *= kAsym ? alpha : alpha * ratio;
      st.m_run[j] = m_new;
      st.thr[j] = m_new + kHeadroom;
      f[j] = alpha * ratio;
    }
    // whole accumulator tuples (rows 0-1: head 2 g4, rows 2-3: head 2 g4 + 1)
    const floatx4 fv = {f[0], f[0], f[1], f[1]};
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) st.O[nt] *= fv;
  }
  // ---- probabilities; P'' = p s_V 16 / vlim split hi/lo into the P staging rows ----
  const float svm[2] = {sv0 * st.pmul, sv1 * st.pmul};
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    float pp[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const float p = __builtin_amdgcn_exp2f(z[j][tt] - st.m_run[j]);
      st.l_run[j] += p;
      pp[j] = p * svm[tt];
      st.ls_run[j] = kAsym ? fmaf(p, mv[tt], st.ls_run[j]) : st.ls_run[j] + pp[j];
    }
    // plane e stages P'' times its coefficient relative to the first plane's
#pragma unroll
    for (int e = 0; e < kP; ++e) {
      _Float16 h4[4];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const float v = e == 0 ? pp[j] : pp[j] * kLmR[e];
        const _Float16 hi = (_Float16)v;
        h4[2 * j] = hi;
        h4[2 * j + 1] = (_Float16)(v - (float)hi);
      }
      *reinterpret_cast<short4v*>(ws.p[e] + pwr + 16 * kPRow * tt) = __builtin_bit_cast(short4v, h4);
    }
  }
  __builtin_amdgcn_wave_barrier();
  // ---- PV: A = P'' (rows (head, part)) read transposed, B = V field j of the token pairs ----
  half8 pop[kP];
#pragma unroll
  for (int e = 0; e < kP; ++e) {
    const short4v pa = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4)(ws.p[e] + prd));
    const short4v pb = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4)(ws.p[e] + prd + 16 * kPRow));
    pop[e] = __builtin_bit_cast(half8, short8v{pa[0], pa[1], pa[2], pa[3], pb[0], pb[1], pb[2], pb[3]});
  }
  unsigned vfold[4][kWin];                                          // parity folds (planes only)
  if constexpr (Fmt<kFmt>::kLloydMax) {
#pragma unroll
    for (int p = 0; p < 4; ++p)
#pragma unroll
      for (int k = 0; k < kWin; ++k) vfold[p][k] = parity_fold(vwin[p][k]);
  }
  // (planes: plane-major, so consecutive products go to different accumulators)
#pragma unroll
  for (int e = 0; e < kP; ++e)
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int wj = VField<kFmt>::win(j);
      unsigned bw[4];
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        if constexpr (Fmt<kFmt>::kLloydMax) {
          unsigned pl[4];
          planes_of(vwin[p][wj], vfold[p][wj], VField<kFmt>::pos(j), pl);
          bw[p] = pl[e];
        } else {
          bw[p] = vwin[p][wj] & VField<kFmt>::mask(j);
        }
      }
      st.O[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pop[e], as_half8(bw[0], bw[1], bw[2], bw[3]), st.O[j], 0, 0, 0);
    }
  __builtin_amdgcn_wave_barrier();
}

// The set-up loads of thread (head row hr = tid / 32, SO(4) block kq = tid % 32) for sequence b:
// query coordinates 4 kq .. 4 kq + 3 of head h0 + hr (raw bf16 pairs in q.x, q.y, or fp32 words)
// and the 8 rotation parameters of block kq.
struct SetupLoads {
  uint4 q;
  float r[8];
};
__device__ __forceinline__ SetupLoads load_setup(const DecodeKArgs& a, int b, int g, int h0, int nh, int tid) {
  SetupLoads v;
  const int hr = tid >> 5, kq = tid & 31;
  const int bc = a.q_tokens > 1 ? b / a.q_tokens : b;          // the cache (and rotation) of sequence b
  const int64_t off = ((int64_t)b * a.Hq + h0 + (hr < nh ? hr : 0)) * 128 + 4 * kq;
  if (a.q_bf16) {
    const uint2 w = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(a.q) + off);
    v.q = make_uint4(w.x, w.y, 0u, 0u);
  } else {
    v.q = *reinterpret_cast<const uint4*>(static_cast<const float*>(a.q) + off);
  }
  const float* rq = a.rot + bc * a.rot_stride_b + (int64_t)g * 256 + kq * 8;
#pragma unroll
  for (int i = 0; i < 8; ++i) v.r[i] = rq[i];
  return v;
}

__device__ __forceinline__ float dpp_ror8(float x) {   // row_ror:8 = lane ^ 8 within a row of 16
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x128, 0xF, 0xF, false));
}
__device__ __forceinline__ float swz_xor16(float x) {  // bitmask swizzle, xor 16 (within 32 lanes)
  return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), (16 << 10) | 0x1F));
}
// x ^ m partner within the 32 lanes of a half-wave, m = 1, 2, 4, 8, 16.
template <int kM>
__device__ __forceinline__ float xor32(float x) {
  if constexpr (kM == 1) return dpp_xor1(x);
  else if constexpr (kM == 2) return dpp_xor2(x);
  else if constexpr (kM == 4) return swz_xor4(x);
  else if constexpr (kM == 8) return dpp_ror8(x);
  else return swz_xor16(x);
}
// One cross-lane Hadamard stage over bit log2(kM) of the block index kq: the lane with that bit
// set takes partner - mine, the other mine + partner.
template <int kM>
__device__ __forceinline__ void hadamard_stage(float (&x)[4], int kq) {
  const float sg = (kq & kM) ? -1.f : 1.f;
#pragma unroll
  for (int r = 0; r < 4; ++r) x[r] = fmaf(sg, x[r], xor32<kM>(x[r]));
}
// o = R^T o' = H (blockdiag M_b^T) o' / sqrt(128) for the 32 threads of a half-wave, thread kq holding
// coordinates 4 kq .. 4 kq + 3 of one row and M = its SO(4) block (row-major): the transposed block,
// then H_128 = H_32 (x) H_4 as in the query set-up (H_4 inside the thread, five cross-lane stages).
// Every lane of the wave must take part (cross-lane moves).
__device__ __forceinline__ void unrotate4(float (&x)[4], const float* M, int kq) {
  float z[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) z[c] = M[c] * x[0] + M[4 + c] * x[1] + M[8 + c] * x[2] + M[12 + c] * x[3];
  const float a0 = z[0] + z[1], a1 = z[0] - z[1], a2 = z[2] + z[3], a3 = z[2] - z[3];
  x[0] = a0 + a2;
  x[1] = a1 + a3;
  x[2] = a0 - a2;
  x[3] = a1 - a3;
  hadamard_stage<1>(x, kq);
  hadamard_stage<2>(x, kq);
  hadamard_stage<4>(x, kq);
  hadamard_stage<8>(x, kq);
  hadamard_stage<16>(x, kq);
#pragma unroll
  for (int r = 0; r < 4; ++r) x[r] *= kInvSqrtD;
}

// kFmt: IQ_FMT_U3 (the pages' records; the only one with the fused append), IQ_FMT_A3 (the same
// records, an (s, m) pair per token), IQ_FMT_U4 or IQ_FMT_U2.
// Waves per SIMD each format's kernel is built for (its register budget: 3 -> 168 VGPRs); the host
// sizes the plan for as many resident work-groups per compute unit.  Measured at 48 layers: four
// waves per SIMD (128 VGPRs) made U3 spill and run 167 us against 127 us, and U2 (no spills) 117
// against 114 us; U4 runs at 155 us with three against 170 us with two.
template <int kFmt>
constexpr int split_waves_per_simd() { return kWavesPerSimd; }

// kW: waves per work-group.  4 (the grid fills three work-groups per compute unit), or 8 for a grid
// of at most one work-group per compute unit (a single short sequence): the chunk's blocks are
// spread over twice the waves, two per SIMD, so each wave's chain of dependent blocks is half as
// long.  Waves 0-3 do the set-up and the final rotation in either case.
template <bool kAppend, int kFmt, int kW>
__global__ __launch_bounds__(64 * kW)
__attribute__((amdgpu_waves_per_eu(kW == kWaves ? split_waves_per_simd<kFmt>() : 2)))
void decode_split_kernel(DecodeKArgs a) {
  static_assert(kW == kWaves || kW == 2 * kWaves, "four or eight waves");
  constexpr bool kAsym = Fmt<kFmt>::kAsym;
  constexpr int kRec = Fmt<kFmt>::kRec;
  __shared__ DecodeSmem<kW, Fmt<kFmt>::kPlanes> sm;
  // blockIdx.x: (KV head, head group) column, so consecutive work-groups take the columns of one
  // work item (measured slightly faster than the transposed order)
  const int x = blockIdx.y;          // (sequence, chunk) pair
  const int g = blockIdx.x / a.head_groups;
  const int hg = blockIdx.x % a.head_groups;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: block bases stay scalar

  // Token indices are 32-bit and a sequence's codes fit one buffer resource (the capacity is
  // validated: cap * record bytes < 0xF0000000): uniform token arithmetic stays on the scalar unit.
  const int cap = (int)a.cap;
  const int h0 = g * a.G + hg * 8;
  const int nh = (a.G - hg * 8) < 8 ? (a.G - hg * 8) : 8;
  // Wave 0's set-up loads are issued before the plan is known, for the sequence that work item x
  // belongs to when every length is cap (the common case), and issued again only if the plan
  // says otherwise: the query and rotation loads then overlap the plan.
  // (the lengths are loaded first: memory loads complete in order, so the plan then waits for
  // them alone)
  const LenSource src{kAppend ? a.positions : nullptr, a.seq_lens, cap, a.batch, a.q_tokens, 1, a.q_tokens};
  const int raw0 = len_raw(src, lane);                       // sequences 0..63
  int b_guess = x / a.guess_per_seq;
  if (b_guess > a.batch - 1) b_guess = a.batch - 1;
  // (every thread rotates one SO(4) block of one query head)
  SetupLoads sl = load_setup(a, b_guess, g, h0, nh, tid);
  const int l0 = len_of(src, lane, raw0);
  const ChunkPlan plan = plan_chunks(src, l0, a.target, x, lane);
  if (plan.b < 0) return;                                    // uniform: past the last chunk
  const int b = plan.b;
  if (b != b_guess) sl = load_setup(a, b, g, h0, nh, tid);   // uniform
  const int len = plan.len;          // > 0
  // the combine reads the plan from here
  if (tid == 0 && blockIdx.x == 0) {
    if (x == 0) a.plan[0] = plan.chunk;
    if (plan.j == 0) a.plan[64 + b] = x;
  }
  // fused append: the new token sits at len - 1 (a position outside the cache gave length 0)
  const int pos = kAppend ? len - 1 : -1;
  const int tok0 = plan.j * plan.chunk;
  if (tok0 >= len) return;                                   // uniform; never taken
  const int tok_end = (tok0 + plan.chunk < len) ? tok0 + plan.chunk : len;
  const int bc = a.q_tokens > 1 ? b / a.q_tokens : b;        // cache of sequence b (uniform)
  const int64_t kv = (int64_t)bc * a.Hkv + g;
  const float* rot = a.rot + bc * a.rot_stride_b + (int64_t)g * 256;

  CacheBuffers cb;
  cb.kc = __builtin_amdgcn_make_buffer_rsrc((void*)(a.kc + kv * a.cap * kRec), (short)0, range_bytes(cap, kRec), kBufferConfig);
  cb.vc = __builtin_amdgcn_make_buffer_rsrc((void*)(a.vc + kv * a.cap * kRec), (short)0, range_bytes(cap, kRec), kBufferConfig);
  constexpr int kSW = kAsym ? 2 : 1;                         // fp32 per token in the scale arrays
  cb.ks = __builtin_amdgcn_make_buffer_rsrc((void*)(a.ks + kv * a.cap * kSW), (short)0, range_bytes(cap, 4 * kSW), kBufferConfig);
  cb.vs = __builtin_amdgcn_make_buffer_rsrc((void*)(a.vs + kv * a.cap * kSW), (short)0, range_bytes(cap, 4 * kSW), kBufferConfig);
  const int n = lane & 15;          // MFMA column: token within a 16-token tile / V group
  const int g4 = lane >> 4;         // row group: quarter of the K record; heads 2*g4, 2*g4+1
  LaneOffsets lo;
  lo.kcode = (unsigned)(n * kRec + kRec / 4 * g4);
  lo.vcode = (unsigned)(kRec * (4 * g4 + (lane & 3)) + kRec / 4 * ((lane >> 2) & 3));
  lo.scale = (unsigned)(4 * (n + 16 * (g4 & 1)));
  const bool vscale = g4 >= 2;
  lo.vside = vscale;

  const int step = kW * kBlock;
  int t0 = tok0 + wave * kBlock;
  // The first blocks of every wave are loaded now, so that they stream while the queries are
  // rotated: three in a grid of at most one work-group per compute unit (eight waves; one 32K
  // layer 11.88 -> 11.55 us, gqa8k 10.27 -> 9.98 us, same box), two otherwise (the third there
  // made the 48-layer step 0.6 us slower).  In the work-group that appends a token to one of those
  // blocks these loads read zeros without a memory access (an end of 0), and the blocks are loaded
  // after the append.
  constexpr int kEarly = kW == 2 * kWaves ? 3 : 2;
  const bool reload = kAppend && pos >= tok0 && pos < tok0 + kEarly * step;   // uniform
  BlockData<Fmt<kFmt>::kQW> buf, buf2, buf3;
  load_block<kFmt>(buf, cb, t0, reload ? 0 : tok_end, lo);
  load_block<kFmt>(buf2, cb, t0 + step, reload ? 0 : tok_end, lo);
  if constexpr (kEarly == 3) load_block<kFmt>(buf3, cb, t0 + 2 * step, reload ? 0 : tok_end, lo);

  // ---------------- set-up (all waves): rotate the queries ----------------
  // Thread (head row hr, block kq) holds coordinates 4 kq .. 4 kq + 3 of its head.  H_128 =
  // (I_32 x H_4)(H_32 x I_4): H_4 inside the thread, then five butterfly stages across the 32
  // lanes of the head, then SO(4) block kq and the 1/sqrt(128).
  SetupSmem& ss = sm.u.setup;
  if (wave < kWaves) {               // uniform: threads 0..255, one per (head, block)
    const int hr = tid >> 5, kq = tid & 31;
    float xq[4];
    if (a.q_bf16) {
      xq[0] = __uint_as_float(sl.q.x << 16);
      xq[1] = __uint_as_float(sl.q.x & 0xFFFF0000u);
      xq[2] = __uint_as_float(sl.q.y << 16);
      xq[3] = __uint_as_float(sl.q.y & 0xFFFF0000u);
    } else {
      xq[0] = __uint_as_float(sl.q.x);
      xq[1] = __uint_as_float(sl.q.y);
      xq[2] = __uint_as_float(sl.q.z);
      xq[3] = __uint_as_float(sl.q.w);
    }
    if (hr >= nh) xq[0] = xq[1] = xq[2] = xq[3] = 0.f;
    {
      const float a0 = xq[0] + xq[1], a1 = xq[0] - xq[1], a2 = xq[2] + xq[3], a3 = xq[2] - xq[3];
      xq[0] = a0 + a2;
      xq[1] = a1 + a3;
      xq[2] = a0 - a2;
      xq[3] = a1 - a3;
    }
    hadamard_stage<1>(xq, kq);
    hadamard_stage<2>(xq, kq);
    hadamard_stage<4>(xq, kq);
    hadamard_stage<8>(xq, kq);
    hadamard_stage<16>(xq, kq);
    float Mb[16];
    build_block(sl.r, Mb);
    if (hr == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        *reinterpret_cast<float4*>(&sm.blk[kq][4 * i]) = make_float4(Mb[4 * i], Mb[4 * i + 1], Mb[4 * i + 2], Mb[4 * i + 3]);
    }
    float y[4], qamax = 0.f, qs = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      y[r] = (Mb[4 * r] * xq[0] + Mb[4 * r + 1] * xq[1] + Mb[4 * r + 2] * xq[2] + Mb[4 * r + 3] * xq[3]) * kInvSqrtD;
      qamax = fmaxf(qamax, fabsf(y[r]));
      qs += y[r];
    }
    *reinterpret_cast<float4*>(&ss.qrot[hr][4 * kq]) = make_float4(y[0], y[1], y[2], y[3]);
    // per head: the sum of q' and the operand exponent E (largest |q'| 2^E in [2^13, 2^14))
    qamax = fmaxf(qamax, xor32<1>(qamax));
    qamax = fmaxf(qamax, xor32<2>(qamax));
    qamax = fmaxf(qamax, xor32<4>(qamax));
    qamax = fmaxf(qamax, xor32<8>(qamax));
    qamax = fmaxf(qamax, xor32<16>(qamax));
    qs += xor32<1>(qs);
    qs += xor32<2>(qs);
    qs += xor32<4>(qs);
    qs += xor32<8>(qs);
    qs += xor32<16>(qs);
    if (kq == 0) {
      int E = 0;
      if (qamax > 0.f) {
        int ex;
        frexpf(qamax, &ex);
        E = 14 - ex;
      }
      ss.qsum[hr] = qs;
      ss.E[hr] = E;
    }
  }
  // ---------------- fused append (wave 1 of the chunk that holds the new token) ----------------
  // The new K (lanes 0-7) and V (lanes 8-15) vectors of this KV head are rotated, quantised and
  // packed as by the quantize kernel and stored into the cache.  The barrier below makes the
  // stores visible to the whole work-group, and every load of the cache is issued after it.
  if (kAppend && pos >= tok0 && pos < tok_end && wave == 1) {
    const int side = (lane >> 3) & 1, c = vec::chunk_of(lane & 7);
    float* fold = &sm.merge.o[2][0][0];     // [32][16] folded blocks (the merge area is free until the end)
    if (lane < 32) vec::build_folded_block(rot + lane * 8, fold + lane * 16, vec::chunk_sign(lane >> 2));
    __builtin_amdgcn_wave_barrier();
    const float (&F)[4][16] = *reinterpret_cast<const float(*)[4][16]>(fold + 64 * c);
    float x[16];
    const void* src = side ? a.v_new : a.k_new;
    const int64_t off = (int64_t)b * a.new_stride_seq + (int64_t)g * a.new_stride_head + 16 * c;
    if (a.new_bf16)
      vec::load16<true>(src, off, lane < 16, x);
    else
      vec::load16<false>(src, off, lane < 16, x);
    unsigned g0, g1, w[3];
    const float scale = vec::quantize8(x, F, c, g0, g1);
    vec::quarter_words(g0, g1, w);
    if (lane < 16) {
      const int64_t rec = kv * a.cap + pos;
      if ((c & 1) == 0) {
        unsigned* dst = reinterpret_cast<unsigned*>(const_cast<uint8_t*>(side ? a.vc : a.kc) + rec * 48 + 6 * c);
#pragma unroll
        for (int i = 0; i < 3; ++i) dst[i] = w[i];
      }
      if (c == 0) const_cast<float*>(side ? a.vs : a.ks)[rec] = scale;
    }
  }
  __syncthreads();
  // A operand of the QK product, built by wave w for K slots 8w .. 8w + 7 of every lane: lane row
  // n = (head n/2, part n%2), K slots of quarter g4.
  if (wave < kWaves) {               // uniform
    const int kb = wave, head = n >> 1, part = n & 1;
    const int Eh = ss.E[head];
    _Float16 hv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int sl8 = 8 * kb + e;
      const float v = ldexpf(ss.qrot[head][32 * g4 + slot_coord_f<kFmt>(sl8)], Eh - slot_pow_f<kFmt>(sl8));
      const _Float16 hi = (_Float16)v;
      hv[e] = part ? (_Float16)(v - (float)hi) : hi;
    }
    sm.qop[kb][lane] = __builtin_bit_cast(uint4v, half8{hv[0], hv[1], hv[2], hv[3], hv[4], hv[5], hv[6], hv[7]});
  }
  const int E0 = ss.E[2 * g4], E1 = ss.E[2 * g4 + 1];
  const float qsum0 = ss.qsum[2 * g4], qsum1 = ss.qsum[2 * g4 + 1];
  __syncthreads();                   // the operand is complete; the set-up area is staging space from here on
  WaveLoopSmemT<Fmt<kFmt>::kPlanes>& ws = sm.u.loop[wave];

  // z2 = log2(e) * sm * s_K * (q'.c - 3.5 sum q'), with q'.c = raw * 2^(24-E) for each head's E.
  // (Lloyd-Max: the first plane's coefficient kGain scales the combined planes)
  const float c1[2] = {a.sm_log2 * Fmt<kFmt>::kGain * ldexpf(1.f, Fmt<kFmt>::kSub - E0),
                       a.sm_log2 * Fmt<kFmt>::kGain * ldexpf(1.f, Fmt<kFmt>::kSub - E1)};
  // (asymmetric format: c2 = log2(e) sm sum q', the coefficient of the minimum m_K)
  constexpr float kC = kAsym ? 1.f : Fmt<kFmt>::kCenter;
  const float c2[2] = {a.sm_log2 * kC * qsum0, a.sm_log2 * kC * qsum1};
  // LDS addresses: this lane's P'' writes (token n of each tile, rows 4*g4..4*g4+3) and its
  // transposed P'' reads (token row 4*g4 + n/4, piece n%4; tile 1 is 16 rows further).
  const unsigned pwr = (unsigned)(n * kPRow + 8 * g4);
  const unsigned prd = (unsigned)((4 * g4 + (n >> 2)) * kPRow + 8 * (n & 3));

  WaveState st;
#pragma unroll
  for (int nt = 0; nt < 8; ++nt) st.O[nt] = floatx4{0.f, 0.f, 0.f, 0.f};
  st.m_run[0] = st.m_run[1] = -INFINITY;
  st.thr[0] = st.thr[1] = -INFINITY;
  st.l_run[0] = st.l_run[1] = 0.f;
  st.ls_run[0] = st.ls_run[1] = 0.f;
  st.vexp = -200;
  st.vlim = 0.f;                     // the first block always rescales
  st.pmul = 0.f;

  if (reload) {                      // uniform; the barriers above ordered it after the append
    load_block<kFmt>(buf, cb, t0, tok_end, lo);
    load_block<kFmt>(buf2, cb, t0 + step, tok_end, lo);
    if constexpr (kEarly == 3) load_block<kFmt>(buf3, cb, t0 + 2 * step, tok_end, lo);
  }
  // Three buffers: the first two are refilled three blocks ahead once their codes are unpacked;
  // the third is loaded at the top of each round of three blocks after the first.  So the buffers
  // carried around the loop were refilled one or two blocks before its back-edge, never just
  // before it.
  bool top_load = kEarly == 2;
  while (t0 < tok_end) {            // uniform
    progress_priority(t0 - tok0, tok_end - tok0);
    if (top_load) load_block<kFmt>(buf3, cb, t0 + 2 * step, tok_end, lo);
    top_load = true;
    process_block<true, kFmt>(buf, min(tok_end - t0, kBlock), t0 + 3 * step, tok_end, cb, lo, vscale, st, sm.qop, c1, c2,
                        ws, lane, n, g4, pwr, prd);
    t0 += step;
    if (t0 >= tok_end) break;
    process_block<true, kFmt>(buf2, min(tok_end - t0, kBlock), t0 + 3 * step, tok_end, cb, lo, vscale, st, sm.qop, c1, c2,
                        ws, lane, n, g4, pwr, prd);
    t0 += step;
    if (t0 >= tok_end) break;
    process_block<false, kFmt>(buf3, min(tok_end - t0, kBlock), 0, tok_end, cb, lo, vscale, st, sm.qop, c1, c2, ws, lane,
                         n, g4, pwr, prd);
    t0 += step;
  }

  // ---------------- per-wave results ----------------
  float l_tot[2], ls_tot[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    l_tot[j] = row_sum(st.l_run[j]);
    ls_tot[j] = row_sum(st.ls_run[j]);
  }
  if (n == 0) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      sm.merge.m[wave][2 * g4 + j] = st.m_run[j];
      sm.merge.l[wave][2 * g4 + j] = l_tot[j];
    }
  }
  // o'[coord] = vlim/16 * (kGain O 2^(24 - p) - kCenter ls), O = hi row + lo row; tile j column n is
  // coordinate 8n + j, taken at bit position field_pos(j).  The wave's 4 KB of the merge area holds
  // them lane-major as float4 [i][lane]: i = 2 j + h is head row 2 g4 + j, coordinates 8n + 4h ..
  // 8n + 4h + 3 (128-bit writes that no two lanes share a bank for; written per coordinate into
  // [row][coord] the lanes of a row group collided eight ways).
  {
    const float back = ldexpf(1.f / kPScale, st.vexp);
    float4* ow = reinterpret_cast<float4*>(&sm.merge.o[wave][0][0]);
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        float v[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int j8 = 4 * h + t;
          const float up = Fmt<kFmt>::kGain * (float)(1 << (Fmt<kFmt>::kSub - VField<kFmt>::pos(j8)));
          v[t] = kAsym ? fmaf(back * up, st.O[j8][2 * j] + st.O[j8][2 * j + 1], ls_tot[j])
                       : back * fmaf(st.O[j8][2 * j] + st.O[j8][2 * j + 1], up, -Fmt<kFmt>::kCenter * ls_tot[j]);
        }
        ow[(2 * j + h) * 64 + lane] = make_float4(v[0], v[1], v[2], v[3]);
      }
  }
  __syncthreads();
  // ---------------- merge the 4 waves, rotate back, write the chunk partial ----------------
  // Thread (head row hr, block kq): coordinates 4 kq .. 4 kq + 3.  R^T is linear, so the partial
  // rows carry R^T o' and the combine's weighted sum needs no rotation.
  if (wave < kWaves) {               // uniform: threads 0..255
    const int hr = tid >> 5, kq = tid & 31;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kW; ++w) M = fmaxf(M, sm.merge.m[w][hr]);
    float L = 0.f, o[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < kW; ++w) {
      const float mw = sm.merge.m[w][hr];
      const float f = (mw == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mw - M);
      L += f * sm.merge.l[w][hr];
      // coordinates 4 kq .. 4 kq + 3 of head row hr: lane (kq / 2, hr / 2), float4 2 (hr % 2) + kq % 2
      const float4 v = reinterpret_cast<const float4*>(&sm.merge.o[w][0][0])[(2 * (hr & 1) + (kq & 1)) * 64 +
                                                                               (kq >> 1) + 16 * (hr >> 1)];
      o[0] += f * v.x;
      o[1] += f * v.y;
      o[2] += f * v.z;
      o[3] += f * v.w;
    }
    unrotate4(o, sm.blk[kq], kq);
    if (hr < nh) {
      const int64_t pidx = (int64_t)(h0 + hr) * a.x_max + x;
      *reinterpret_cast<float4*>(a.part_o + pidx * 128 + 4 * kq) = make_float4(o[0], o[1], o[2], o[3]);
      if (kq == 0) {
        a.part_ml[pidx * 2] = M;
        a.part_ml[pidx * 2 + 1] = L;
      }
    }
  }
}

// ---------------- several query tokens per work-group ----------------
// With several query tokens per cached sequence (iq_decode_attention_multi) the kernel above would
// read and unpack every block once per token.  Here a work item is a chunk of a group of kMultiQ
// consecutive query tokens: each 32-token block's K and V codes are unpacked once and multiplied by
// every token's operands, and each token keeps its own online softmax; the V scale bound is shared.
// Wave w rotates token w's queries.  3-bit records, no append.  The tokens go in pairs: the 16 rows
// of a product are (token, query head) of two tokens, and the hi and lo parts of q' and of P'' are
// the two halves of its K dimension (two products into one accumulator), so a token's accumulators
// take 16 registers.  Four tokens per group fill the 256 registers of two waves per SIMD.
constexpr int kMultiQ = 4;                    // tokens per group (one per wave at set-up), even
constexpr int kMultiWavesPerSimd = 2;
constexpr int kMultiRounds = 3;               // work items per column: three rounds of work-groups
constexpr int kMultiRoundsOneGroup = 2;       // two when each sequence has one group of tokens
constexpr float kNoMax = -1e30f;              // running max before any score: finite, so a token
                                              // with nothing to attend to in a chunk gets p = 0
struct MultiLoopSmem {
  char p[kMultiQ / 2][2][kBlock * kPRow];     // P'' staging of each token pair: hi parts, lo parts
  float sc[64];
};
struct MultiSetupSmem {
  float qrot[kWaves][8][128];
  float qsum[kWaves][8];
  int E[kWaves];
};
union MultiSmemU {
  MergeSmem merge;
  MultiLoopSmem loop[kWaves];
  MultiSetupSmem setup;
};
struct MultiSmem {
  uint4v qop[kMultiQ / 2][2][4][64];          // QK A operand of each token pair: hi parts, lo parts
  float blk[32][16];                          // the KV head's SO(4) blocks (set-up and the partials)
  MultiSmemU u;
};

// Lane (n, g4) of a token pair's tile holds rows 4 g4 + r, r = 0..3: token 2 pair + g4 / 2, query
// head 4 (g4 % 2) + r.
template <int kP>
struct MultiState {
  floatx4 O[kP][8];       // O[pair][j]: rows (token, head), column n = coordinate 8n + j
  float m_run[kP][4], thr[kP][4], l_run[kP][4], ls_run[kP][4];   // per row r of the lane
  int vexp;
  float vlim, pmul;
};

// fp16 hi and lo parts of s p_i for four values: hi_i = fp16(s p_i), lo_i = fp16(s p_i - hi_i), each
// rounded once from the exact product by a mixed-precision FMA; hi = {hi_0 | hi_1 << 16, hi_2 | hi_3 << 16},
// lo likewise (the compiler splits these with two more instructions per value).  A half written here
// is read two instructions later at the earliest; the leading s_nop covers a transcendental result
// read at once.
__device__ __forceinline__ void split_hi_lo4(float s, const float (&p)[4], unsigned (&hi)[2], unsigned (&lo)[2]) {
  asm("s_nop 0\n\t"
      "v_fma_mixlo_f16 %0, %4, %5, 0\n\t"
      "v_fma_mixlo_f16 %1, %4, %7, 0\n\t"
      "v_fma_mixlo_f16 %2, %4, %5, -%0 op_sel_hi:[0,0,1]\n\t"
      "v_fma_mixlo_f16 %3, %4, %7, -%1 op_sel_hi:[0,0,1]\n\t"
      "v_fma_mixhi_f16 %0, %4, %6, 0\n\t"
      "v_fma_mixhi_f16 %1, %4, %8, 0\n\t"
      "v_fma_mixhi_f16 %2, %4, %6, -%0 op_sel:[0,0,1] op_sel_hi:[0,0,1]\n\t"
      "v_fma_mixhi_f16 %3, %4, %8, -%1 op_sel:[0,0,1] op_sel_hi:[0,0,1]"
      : "=&v"(hi[0]), "=&v"(hi[1]), "=&v"(lo[0]), "=&v"(lo[1])
      : "v"(s), "v"(p[0]), "v"(p[1]), "v"(p[2]), "v"(p[3]));
}

// process_block for kP token pairs (3-bit records).  A pair's 16 rows are (token, head), and the hi
// and lo parts of q' (QK) and of P'' (PV) are the two halves of each product's K dimension: two
// products into one accumulator.  lim[p]: the lane's token of pair p attends to the block's tokens
// below lim[p].  A token the group does not have runs too, with lim = the chunk start: every score
// is masked, so its p and its products are zero (straight-line code, no per-token branches).
template <bool kRefill, int kP>
__device__ __forceinline__ void process_block_multi(BlockData<3>& cur, int t0, int tok_end, const int (&lim)[kP],
                                                    int t_refill, const CacheBuffers& cb,
                                                    const LaneOffsets& lo, bool vscale, MultiState<kP>& st,
                                                    const uint4v (&qop)[kMultiQ / 2][2][4][64],
                                                    const float (&c1)[kP], const float (&c2)[kP][4],
                                                    MultiLoopSmem& ws, int lane, int n, unsigned pwr, unsigned prd) {
  constexpr int kFmt = IQ_FMT_U3;
  ws.sc[lane] = __uint_as_float(vscale ? cur.vsc : cur.ksc);
  // ---- QK of every pair on the same unpacked codes ----
  floatx4 S[kP][2];
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    unsigned u[16];
    unpack_k<kFmt>(cur.kw[tt], u);
    half8 kb[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) kb[k] = as_half8(u[4 * k], u[4 * k + 1], u[4 * k + 2], u[4 * k + 3]);
#pragma unroll
    for (int p = 0; p < kP; ++p) {
      floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k = 0; k < 4; ++k)
#pragma unroll
        for (int part = 0; part < 2; ++part)
          acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, qop[p][part][k][lane]), kb[k], acc,
                                                      0, 0, 0);
      S[p][tt] = acc;
    }
  }
  // ---- V byte windows, as in process_block ----
  unsigned vwin[4][3];
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    unsigned gq[4];
    gq[0] = cur.vw[tt][0];
    gq[1] = __builtin_amdgcn_alignbyte(cur.vw[tt][1], cur.vw[tt][0], 3);
    gq[2] = __builtin_amdgcn_alignbyte(cur.vw[tt][2], cur.vw[tt][1], 2);
    gq[3] = cur.vw[tt][2] >> 8;
    quad_transpose(gq, lane);
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      unsigned* vw = vwin[2 * tt + p];
      vw[0] = __builtin_amdgcn_perm(gq[2 * p + 1], gq[2 * p], 0x05040100u);
      vw[1] = __builtin_amdgcn_perm(gq[2 * p + 1], gq[2 * p], 0x06050201u);
      vw[2] = __builtin_amdgcn_perm(gq[2 * p + 1], gq[2 * p], 0x07060302u);
    }
  }
  if (kRefill) {
    __builtin_amdgcn_sched_barrier(0);
    load_block<kFmt, kSharedLoadPolicy>(cur, cb, t_refill, tok_end, lo);
  }
  // ---- scores; tokens past the chunk carry no V scale, tokens past lim[p] no score ----
  const float sk0 = ws.sc[n], sk1 = ws.sc[16 + n];
  float sv0 = ws.sc[32 + n], sv1 = ws.sc[48 + n];
  const int rem = tok_end - t0;
  if (n >= rem) sv0 = 0.f;
  if (16 + n >= rem) sv1 = 0.f;
  // The mask is one additive bias per (pair, tile): a lane's four rows of a pair are one token.
  float z[kP][4][2];
#pragma unroll
  for (int p = 0; p < kP; ++p) {
    const int ri = lim[p] - t0;
    const float b0 = n < ri ? 0.f : -INFINITY, b1 = 16 + n < ri ? 0.f : -INFINITY;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      z[p][r][0] = fmaf(sk0, fmaf(S[p][0][r], c1[p], -c2[p][r]), b0);
      z[p][r][1] = fmaf(sk1, fmaf(S[p][1][r], c1[p], -c2[p][r]), b1);
    }
  }
  const float svmax = fmaxf(sv0, sv1);
  bool grow = svmax >= st.vlim;
#pragma unroll
  for (int p = 0; p < kP; ++p)
#pragma unroll
    for (int r = 0; r < 4; ++r) grow |= fmaxf(z[p][r][0], z[p][r][1]) > st.thr[p][r];
  if (__any(grow)) {
    const float vmax = row_max(svmax);
    float ratio = 1.f;
    if (vmax >= st.vlim) {
      int ex;
      frexpf(vmax, &ex);
      ex = ex < -60 ? -60 : ex;
      ratio = st.vexp == -200 ? 0.f : ldexpf(1.f, st.vexp - ex);
      st.vexp = ex;
      st.vlim = ldexpf(1.f, ex);
      st.pmul = ldexpf(kPScale, -ex);
    }
#pragma unroll
    for (int p = 0; p < kP; ++p) {
      float f[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float m_new = fmaxf(st.m_run[p][r], row_max(fmaxf(z[p][r][0], z[p][r][1])));
        const float alpha = __builtin_amdgcn_exp2f(st.m_run[p][r] - m_new);
        st.l_run[p][r] *= alpha;
        st.ls_run[p][r] *= alpha * ratio;
        st.m_run[p][r] = m_new;
        st.thr[p][r] = m_new + kHeadroom;
        f[r] = alpha * ratio;
      }
      // whole accumulator tuples: no copies of them on the path without a rescale
      const floatx4 fv = {f[0], f[1], f[2], f[3]};
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) st.O[p][nt] *= fv;
    }
  }
  // ---- P'' of each pair, its hi and lo parts staged apart and read back transposed ----
  const float svm[2] = {sv0 * st.pmul, sv1 * st.pmul};
#pragma unroll
  for (int p = 0; p < kP; ++p) {
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      float pr[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        pr[r] = __builtin_amdgcn_exp2f(z[p][r][tt] - st.m_run[p][r]);
        st.l_run[p][r] += pr[r];
        st.ls_run[p][r] = fmaf(pr[r], svm[tt], st.ls_run[p][r]);
      }
      unsigned hh[2], hl[2];
      split_hi_lo4(svm[tt], pr, hh, hl);
      *reinterpret_cast<uint2*>(ws.p[p][0] + pwr + 16 * kPRow * tt) = make_uint2(hh[0], hh[1]);
      *reinterpret_cast<uint2*>(ws.p[p][1] + pwr + 16 * kPRow * tt) = make_uint2(hl[0], hl[1]);
    }
  }
  __builtin_amdgcn_wave_barrier();
  half8 pop[kP][2];
#pragma unroll
  for (int p = 0; p < kP; ++p)
#pragma unroll
    for (int part = 0; part < 2; ++part) {
      const short4v pa = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4)(ws.p[p][part] + prd));
      const short4v pb = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4)(ws.p[p][part] + prd + 16 * kPRow));
      pop[p][part] = __builtin_bit_cast(half8, short8v{pa[0], pa[1], pa[2], pa[3], pb[0], pb[1], pb[2], pb[3]});
    }
  // ---- PV on the shared V windows: fields two at a time, so a field's hi and lo products are
  //      not back to back ----
#pragma unroll
  for (int j = 0; j < 8; j += 2) {
    half8 vb[2];
#pragma unroll
    for (int d = 0; d < 2; ++d) {
      const unsigned m = VField<kFmt>::mask(j + d);
      const int wj = VField<kFmt>::win(j + d);
      vb[d] = as_half8(vwin[0][wj] & m, vwin[1][wj] & m, vwin[2][wj] & m, vwin[3][wj] & m);
    }
#pragma unroll
    for (int part = 0; part < 2; ++part)
#pragma unroll
      for (int p = 0; p < kP; ++p)
#pragma unroll
        for (int d = 0; d < 2; ++d)
          st.O[p][j + d] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pop[p][part], vb[d], st.O[p][j + d], 0, 0, 0);
  }
  __builtin_amdgcn_wave_barrier();
}

template <int kQ>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(kMultiWavesPerSimd, kMultiWavesPerSimd)))
void decode_multi_kernel(DecodeKArgs a) {
  static_assert(kQ <= kMultiQ && kQ <= kWaves && kQ % 2 == 0, "one token per set-up wave, pairs of tokens");
  constexpr int kP = kQ / 2;
  constexpr int kFmt = IQ_FMT_U3;
  constexpr int kRec = 48;
  __shared__ MultiSmem sm;
  const int x = blockIdx.y;          // (group sequence, chunk) pair
  const int g = blockIdx.x / a.head_groups;
  const int hg = blockIdx.x % a.head_groups;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int cap = (int)a.cap;
  const int h0 = g * a.G + hg * 8;
  const int nh = (a.G - hg * 8) < 8 ? (a.G - hg * 8) : 8;
  // work-item sequence b: group b % n_groups (tokens kQ (b % n_groups) ...) of cache b / n_groups,
  // with the length of its last token
  const LenSource src{nullptr, a.seq_lens, cap, a.batch, a.q_tokens, kQ, a.n_groups};
  const int l0 = len_at(src, lane);
  const ChunkPlan plan = plan_chunks(src, l0, a.target, x, lane);
  if (plan.b < 0) return;                                    // uniform: past the last chunk
  const int b = plan.b;
  const int len = plan.len;          // > 0
  if (tid == 0 && blockIdx.x == 0) {
    if (x == 0) a.plan[0] = plan.chunk;
    if (plan.j == 0) a.plan[64 + b] = x;
  }
  const int tok0 = plan.j * plan.chunk;
  if (tok0 >= len) return;                                   // uniform; never taken
  const int tok_end = (tok0 + plan.chunk < len) ? tok0 + plan.chunk : len;
  const int bc = b / a.n_groups;
  const int t_first = (b % a.n_groups) * kQ;                 // the group's first query token
  const int nq = (a.q_tokens - t_first) < kQ ? (a.q_tokens - t_first) : kQ;   // its tokens (uniform)
  int lim[kQ];                       // token i (length len - (nq - 1 - i)) attends below lim[i]
#pragma unroll
  for (int i = 0; i < kQ; ++i) {
    const int li = len - (nq - 1 - i);
    lim[i] = i < nq ? (li < tok_end ? li : tok_end) : tok0;
  }
  const int64_t kv = (int64_t)bc * a.Hkv + g;
  const float* rot = a.rot + bc * a.rot_stride_b + (int64_t)g * 256;

  CacheBuffers cb;
  cb.kc = __builtin_amdgcn_make_buffer_rsrc((void*)(a.kc + kv * a.cap * kRec), (short)0, range_bytes(cap, kRec), kBufferConfig);
  cb.vc = __builtin_amdgcn_make_buffer_rsrc((void*)(a.vc + kv * a.cap * kRec), (short)0, range_bytes(cap, kRec), kBufferConfig);
  cb.ks = __builtin_amdgcn_make_buffer_rsrc((void*)(a.ks + kv * a.cap), (short)0, range_bytes(cap, 4), kBufferConfig);
  cb.vs = __builtin_amdgcn_make_buffer_rsrc((void*)(a.vs + kv * a.cap), (short)0, range_bytes(cap, 4), kBufferConfig);
  const int n = lane & 15;
  const int g4 = lane >> 4;
  LaneOffsets lo;
  lo.kcode = (unsigned)(n * kRec + kRec / 4 * g4);
  lo.vcode = (unsigned)(kRec * (4 * g4 + (lane & 3)) + kRec / 4 * ((lane >> 2) & 3));
  lo.scale = (unsigned)(4 * (n + 16 * (g4 & 1)));
  const bool vscale = g4 >= 2;
  lo.vside = vscale;

  const int step = kWaves * kBlock;
  int t0 = tok0 + wave * kBlock;
  BlockData<3> buf, buf2, buf3;
  load_block<kFmt, kSharedLoadPolicy>(buf, cb, t0, tok_end, lo);
  load_block<kFmt, kSharedLoadPolicy>(buf2, cb, t0 + step, tok_end, lo);

  // ---------------- set-up: wave w rotates query token t_first + w ----------------
  MultiSetupSmem& ss = sm.u.setup;
  if (lane < 8) build_block(rot + (8 * wave + lane) * 8, sm.blk[8 * wave + lane]);
  __syncthreads();
  if (wave < nq) {                                           // uniform
    const int qi = lane >> 3, qe = lane & 7;                 // head row, 16-coordinate slice
    const bool have = qi < nh;
    const int64_t off = (((int64_t)bc * a.q_tokens + t_first + wave) * a.Hq + h0 + (have ? qi : 0)) * 128 + 16 * qe;
    float xq[16];
    if (a.q_bf16) {
      const uint4* qp = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.q) + off);
      const uint4 q0 = qp[0], q1 = qp[1];
      const unsigned w[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        xq[2 * i] = __uint_as_float(w[i] << 16);
        xq[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
      }
    } else {
      const float4* qp = reinterpret_cast<const float4*>(static_cast<const float*>(a.q) + off);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float4 v = qp[i];
        xq[4 * i] = v.x; xq[4 * i + 1] = v.y; xq[4 * i + 2] = v.z; xq[4 * i + 3] = v.w;
      }
    }
    if (!have) {
#pragma unroll
      for (int i = 0; i < 16; ++i) xq[i] = 0.f;
    }
    {
      // Sylvester Hadamard (unnormalised), as in the single-token set-up
      const float sg1 = (qe & 1) ? -1.f : 1.f, sg2 = (qe & 2) ? -1.f : 1.f, sg4 = (qe & 4) ? -1.f : 1.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) xq[i] = fmaf(sg1, xq[i], dpp_xor1(xq[i]));
#pragma unroll
      for (int i = 0; i < 16; ++i) xq[i] = fmaf(sg2, xq[i], dpp_xor2(xq[i]));
#pragma unroll
      for (int i = 0; i < 16; ++i) xq[i] = fmaf(sg4, xq[i], swz_xor4(xq[i]));
#pragma unroll
      for (int m = 8; m >= 1; m >>= 1)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if ((i & m) == 0) {
            const float u = xq[i], v = xq[i + m];
            xq[i] = u + v;
            xq[i + m] = u - v;
          }
    }
    float qamax = 0.f, qs = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float* M = sm.blk[4 * qe + j];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float y = (M[4 * r] * xq[4 * j] + M[4 * r + 1] * xq[4 * j + 1] + M[4 * r + 2] * xq[4 * j + 2] +
                         M[4 * r + 3] * xq[4 * j + 3]) * kInvSqrtD;
        ss.qrot[wave][qi][16 * qe + 4 * j + r] = y;
        qamax = fmaxf(qamax, fabsf(y));
        qs += y;
      }
    }
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) qamax = fmaxf(qamax, wave_xor(qamax, m));
    qs += dpp_xor1(qs);
    qs += dpp_xor2(qs);
    qs += swz_xor4(qs);
    int E = 0;
    if (qamax > 0.f) {
      int ex;
      frexpf(qamax, &ex);
      E = 14 - ex;
    }
    if (qe == 0) ss.qsum[wave][qi] = qs;
    if (lane == 0) ss.E[wave] = E;
  }
  __syncthreads();
  // A operands: wave 2 p + part builds part (hi or lo) of pair p, lane row n = (token 2 p + n / 8,
  // head n % 8), K slots of quarter g4; tokens the group does not have get zeros
  if (wave < 2 * kP) {               // uniform
    const int pr = wave >> 1, part = wave & 1;
    const int tok = 2 * pr + (n >> 3), head = n & 7;
    const bool have = tok < nq;
    const int Et = have ? ss.E[tok] : 0;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      _Float16 hv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int sl = 8 * kb + e;
        const float v = have ? ldexpf(ss.qrot[tok][head][32 * g4 + slot_coord_f<kFmt>(sl)], Et - slot_pow_f<kFmt>(sl))
                             : 0.f;
        const _Float16 hi = (_Float16)v;
        hv[e] = part ? (_Float16)(v - (float)hi) : hi;
      }
      sm.qop[pr][part][kb][lane] =
          __builtin_bit_cast(uint4v, half8{hv[0], hv[1], hv[2], hv[3], hv[4], hv[5], hv[6], hv[7]});
    }
  }
  // this lane's rows of pair p belong to token 2 p + g4 / 2, query heads 4 (g4 % 2) + r
  float c1[kP], c2[kP][4];
  int lim_l[kP];
#pragma unroll
  for (int p = 0; p < kP; ++p) {
    const int tok = 2 * p + (g4 >> 1);
    const bool in = tok < nq;
    c1[p] = in ? a.sm_log2 * ldexpf(1.f, 24 - ss.E[tok]) : 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) c2[p][r] = in ? a.sm_log2 * 3.5f * ss.qsum[tok][4 * (g4 & 1) + r] : 0.f;
    lim_l[p] = (g4 & 2) ? lim[2 * p + 1] : lim[2 * p];
  }
  __syncthreads();                   // the operands are complete; the set-up area is staging space from here on
  MultiLoopSmem& ws = sm.u.loop[wave];
  const unsigned pwr = (unsigned)(n * kPRow + 8 * g4);
  const unsigned prd = (unsigned)((4 * g4 + (n >> 2)) * kPRow + 8 * (n & 3));

  MultiState<kP> st;
#pragma unroll
  for (int p = 0; p < kP; ++p) {
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) st.O[p][nt] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      st.m_run[p][r] = kNoMax;
      st.thr[p][r] = kNoMax;
      st.l_run[p][r] = 0.f;
      st.ls_run[p][r] = 0.f;
    }
  }
  st.vexp = -200;
  st.vlim = 0.f;                     // the first block always rescales
  st.pmul = 0.f;

  while (t0 < tok_end) {            // uniform
    progress_priority(t0 - tok0, tok_end - tok0);
    load_block<kFmt, kSharedLoadPolicy>(buf3, cb, t0 + 2 * step, tok_end, lo);
    process_block_multi<true, kP>(buf, t0, tok_end, lim_l, t0 + 3 * step, cb, lo, vscale, st, sm.qop, c1, c2, ws,
                                  lane, n, pwr, prd);
    t0 += step;
    if (t0 >= tok_end) break;
    process_block_multi<true, kP>(buf2, t0, tok_end, lim_l, t0 + 3 * step, cb, lo, vscale, st, sm.qop, c1, c2, ws,
                                  lane, n, pwr, prd);
    t0 += step;
    if (t0 >= tok_end) break;
    process_block_multi<false, kP>(buf3, t0, tok_end, lim_l, 0, cb, lo, vscale, st, sm.qop, c1, c2, ws, lane, n,
                                   pwr, prd);
    t0 += step;
  }

  // ---------------- per-token results: merge the 4 waves, write the token's partial row ----------------
  const float back = ldexpf(1.f / kPScale, st.vexp);
  __syncthreads();                     // every wave is done with the loop smem
#pragma unroll
  for (int i = 0; i < kQ; ++i) {
    if (i >= nq) continue;             // uniform
    const int p = i >> 1;
    float l_tot[4], ls_tot[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      l_tot[r] = row_sum(st.l_run[p][r]);
      ls_tot[r] = row_sum(st.ls_run[p][r]);
    }
    if ((g4 >> 1) == (i & 1)) {        // the lanes holding token i's rows: query heads 4 (g4 % 2) + r
      const int h4 = 4 * (g4 & 1);
      if (n == 0) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          sm.u.merge.m[wave][h4 + r] = st.m_run[p][r];
          sm.u.merge.l[wave][h4 + r] = l_tot[r];
        }
      }
#pragma unroll
      for (int j8 = 0; j8 < 8; ++j8) {
        const int coord = 8 * n + j8;
        const float up = (float)(1 << (24 - VField<kFmt>::pos(j8)));
#pragma unroll
        for (int r = 0; r < 4; ++r)
          sm.u.merge.o[wave][h4 + r][coord] = back * fmaf(st.O[p][j8][r], up, -3.5f * ls_tot[r]);
      }
    }
    __syncthreads();
    {                                  // as in the single-token kernel: merge, rotate back, write
      const int hr = tid >> 5, kq = tid & 31;
      float M = kNoMax;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) M = fmaxf(M, sm.u.merge.m[w][hr]);
      float L = 0.f, o[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float f = __builtin_amdgcn_exp2f(sm.u.merge.m[w][hr] - M);
        L += f * sm.u.merge.l[w][hr];
        const float4 v = *reinterpret_cast<const float4*>(&sm.u.merge.o[w][hr][4 * kq]);
        o[0] += f * v.x;
        o[1] += f * v.y;
        o[2] += f * v.z;
        o[3] += f * v.w;
      }
      unrotate4(o, sm.blk[kq], kq);
      if (hr < nh) {
        const int64_t pidx = (int64_t)(h0 + hr) * a.x_max + (int64_t)x * kQ + i;
        *reinterpret_cast<float4*>(a.part_o + pidx * 128 + 4 * kq) = make_float4(o[0], o[1], o[2], o[3]);
        if (kq == 0) {
          a.part_ml[pidx * 2] = M;
          a.part_ml[pidx * 2 + 1] = L;
        }
      }
    }
    __syncthreads();
  }
}

struct CombineArgs {
  const float* part_o;
  const float* part_ml;
  const int* plan;              // written by the split kernel: chunk size, first chunk per sequence
  const int32_t* seq_lens;
  const int32_t* positions;     // fused append: lengths are positions + 1 (seq_lens unused)
  int Hq, G;
  int q_tokens;                 // as in the split kernel
  int q_group;                  // 1, or the multi-token kernel's kQ: the partial rows of query token t
  int n_groups;                 // of a sequence are x kQ + t % kQ for the work items x of its group
  int64_t cap;
  int x_max;                    // partial rows per query head
  int guess_per_seq;            // chunks per sequence when every length is cap (the split kernel's guess)
  float* out;
};

// One sequence with one query token: its chunks are partial rows 0 .. nvalid - 1 of every query head
// (x_max <= kMidChunks of them), so every load (the rows and their (max, sum) pairs) is issued at
// once, unconditionally, before the length and the chunk size arrive: rows past x_max repeat the
// last row, and rows past nvalid are loaded but not used.  Each wave reduces the (max, sum) pairs
// itself: no weights through LDS.  An empty sequence gets zeros.
__device__ __forceinline__ void combine_one_sequence(const CombineArgs& a, int h, float* outp, int tid) {
  const int lane = tid & 63;
  const int nr = a.x_max;
  const float* po = a.part_o + (int64_t)h * nr * 128 + tid;
  float om[kMidChunks];
#pragma unroll
  for (int c = 0; c < kMidChunks; ++c) om[c] = po[(int64_t)min(c, nr - 1) * 128];
  const float2 mlv = reinterpret_cast<const float2*>(a.part_ml)[(int64_t)h * nr + min(lane, nr - 1)];
  const int chunk = a.plan[0];
  const int len = len_at(LenSource{a.positions, a.seq_lens, (int)a.cap, 1, 1, 1, 1}, 0);
  const int nvalid = len > 0 ? min((len + chunk - 1) / chunk, nr) : 0;
  const float m = lane < nvalid ? mlv.x : -INFINITY;
  float M = m;
#pragma unroll
  for (int sft = 1; sft < 64; sft <<= 1) M = fmaxf(M, wave_xor(M, sft));
  const float e = lane < nvalid ? __builtin_amdgcn_exp2f(m - M) : 0.f;
  float L = e * mlv.y;
#pragma unroll
  for (int sft = 1; sft < 64; sft <<= 1) L += wave_xor(L, sft);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < kMidChunks; ++c) {           // rows past nvalid may hold anything: selected out
    const float w = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(e), c));
    acc[c & 7] = fmaf(w, c < nvalid ? om[c] : 0.f, acc[c & 7]);
  }
  const float sum = ((acc[0] + acc[1]) + (acc[2] + acc[3])) + ((acc[4] + acc[5]) + (acc[6] + acc[7]));
  outp[tid] = nvalid > 0 ? sum / L : 0.f;
}

// Several sequences of one query token, at most kN chunks each when every length is cap: the rows
// of sequence b under that guess (b gps .. b gps + gps - 1) and their (max, sum) pairs are loaded
// together with the plan and the length, and used when the plan agrees (one round trip instead
// of two).  Returns false (nothing written) when the plan differs.
template <int kN>
__device__ __forceinline__ bool combine_guessed(const CombineArgs& a, int b, int h, float* outp, int tid) {
  const int gps = a.guess_per_seq, x0g = b * gps;
  const int64_t hrow = (int64_t)h * a.x_max;
  float mv[kN], lv[kN], ov[kN];
#pragma unroll
  for (int c = 0; c < kN; ++c) {
    const int64_t row = hrow + min(x0g + min(c, gps - 1), a.x_max - 1);   // in range; unused past nvalid
    const float2 v = reinterpret_cast<const float2*>(a.part_ml)[row];
    mv[c] = v.x;
    lv[c] = v.y;
    ov[c] = a.part_o[row * 128 + tid];
  }
  const int chunk = a.plan[0];
  const int x0 = a.plan[64 + b];
  const int len = len_at(LenSource{a.positions, a.seq_lens, (int)a.cap, (int)gridDim.x / a.Hq, 1, 1, 1}, b);
  if (len == 0) {                       // an empty sequence attends to nothing
    outp[tid] = 0.f;
    return true;
  }
  const int nvalid = (len + chunk - 1) / chunk;
  if (x0 != x0g || nvalid > gps) return false;   // uniform
  float M = -INFINITY;
#pragma unroll
  for (int c = 0; c < kN; ++c) M = c < nvalid ? fmaxf(M, mv[c]) : M;
  float L = 0.f, acc = 0.f;
#pragma unroll
  for (int c = 0; c < kN; ++c)
    if (c < nvalid) {                   // uniform; rows past it may hold anything
      const float w = __builtin_amdgcn_exp2f(mv[c] - M);
      L = fmaf(w, lv[c], L);
      acc = fmaf(w, ov[c], acc);
    }
  outp[tid] = acc / L;
  return true;
}

// One work-group (2 waves) per (sequence, query head): log-sum-exp merge of the chunk partials with
// one output coordinate per thread and independent loads.  The partial rows are already rotated
// back (R^T o', by the kernels that write them), so the merged row is the output.
__global__ __launch_bounds__(128) void combine_kernel(CombineArgs a) {
  __shared__ float wgt[kMaxChunks];
  __shared__ float inv_l;
  const int b = blockIdx.x / a.Hq, h = blockIdx.x % a.Hq;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (a.q_tokens == 1 && (int)gridDim.x == a.Hq && a.x_max <= kMidChunks) {   // uniform
    combine_one_sequence(a, h, a.out + (int64_t)h * 128, tid);
    return;
  }
  // Several sequences of one query token, at most kFewChunks chunks each when every length is cap:
  // the guessed rows first (combine_guessed, as many loads as the guess has rows, rounded up to 4,
  // 8 or 16); otherwise the general path below loads the right rows.
  if (a.q_tokens == 1 && a.guess_per_seq <= kFewChunks) {   // uniform
    float* outp = a.out + ((int64_t)b * a.Hq + h) * 128;
    bool done;
    if (a.guess_per_seq <= 4)
      done = combine_guessed<4>(a, b, h, outp, tid);
    else if (a.guess_per_seq <= 8)
      done = combine_guessed<8>(a, b, h, outp, tid);
    else
      done = combine_guessed<kFewChunks>(a, b, h, outp, tid);
    if (done) return;                   // uniform
  }
  // the plan is read together with the length (both entries exist for every sequence; they are
  // used only when the sequence has tokens, and then the split kernel wrote them)
  // output row b is query token b % q_tokens of cache b / q_tokens; its chunks are the work items
  // of work-item sequence sq, partial rows x rs + ri (rs = 1, ri = 0 with one token per sequence)
  const int bc = a.q_tokens > 1 ? b / a.q_tokens : b;
  const int tq = a.q_tokens > 1 ? b % a.q_tokens : 0;
  const int sq = bc * a.n_groups + tq / a.q_group, rs = a.q_group, ri = tq % a.q_group;
  const int chunk = a.plan[0];
  const int x0 = a.plan[64 + sq];
  const int len =
      len_at(LenSource{a.positions, a.seq_lens, (int)a.cap, (int)gridDim.x / a.Hq, a.q_tokens, 1, a.q_tokens}, b);
  float* outp = a.out + ((int64_t)b * a.Hq + h) * 128;
  if (len == 0) {                       // an empty sequence attends to nothing
    outp[tid] = 0.f;
    return;
  }
  int nvalid = (len + chunk - 1) / chunk;         // <= kMaxChunks and x0 + nvalid <= x_max / rs by
  nvalid = min(nvalid, min(kMaxChunks, a.x_max / rs - x0));   // the plan; the bound keeps every read in range
  const int64_t first = (int64_t)h * a.x_max + (int64_t)x0 * rs + ri;   // partial row of chunk 0; chunk c
  const float* ml = a.part_ml + first * 2;                             // is rs rows further
  // rows with kPreloadFrom < chunks <= kMidChunks: this thread's partials are loaded now, together
  // with the weights' loads below, and kept in registers (with fewer chunks the extra registers
  // measured slower than the loads after the barrier)
  float om[kMidChunks];
  const bool preload = nvalid > kPreloadFrom && nvalid <= kMidChunks;   // uniform
  if (preload) {
    const float* po = a.part_o + first * 128 + tid;
#pragma unroll
    for (int c = 0; c < kMidChunks; ++c)
      if (c < nvalid) om[c] = po[(int64_t)c * rs * 128];   // uniform branches
  }
  if (nvalid <= kFewChunks) {           // uniform: every thread loads all (max, sum) pairs and its partials at once
    const float* po = a.part_o + first * 128 + tid;
    float mv[kFewChunks], lv[kFewChunks], ov[kFewChunks];
#pragma unroll
    for (int c = 0; c < kFewChunks; ++c) {
      const int cc = (c < nvalid ? c : nvalid - 1) * rs;   // in range; weight 0 below
      mv[c] = ml[2 * cc];
      lv[c] = ml[2 * cc + 1];
      ov[c] = po[(int64_t)cc * 128];
    }
    float M = -INFINITY;
#pragma unroll
    for (int c = 0; c < kFewChunks; ++c) M = c < nvalid ? fmaxf(M, mv[c]) : M;
    float L = 0.f, acc = 0.f;
#pragma unroll
    for (int c = 0; c < kFewChunks; ++c) {
      const float w = c < nvalid ? __builtin_amdgcn_exp2f(mv[c] - M) : 0.f;
      L = fmaf(w, lv[c], L);
      acc = fmaf(w, ov[c], acc);
    }
    outp[tid] = acc / L;
    return;
  }
  if (wave == 0) {                      // weights 2^(m_c - M) and 1/L
    float M = -INFINITY;
    for (int c = lane; c < nvalid; c += 64) M = fmaxf(M, ml[2 * c * rs]);
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) M = fmaxf(M, wave_xor(M, m));
    float L = 0.f;
    for (int c = lane; c < nvalid; c += 64) {
      const float e = __builtin_amdgcn_exp2f(ml[2 * c * rs] - M);
      wgt[c] = e;
      L = fmaf(e, ml[2 * c * rs + 1], L);
    }
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) L += wave_xor(L, m);
    if (lane == 0) inv_l = 1.f / L;
  }
  if (preload) {
    __syncthreads();
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < kMidChunks; ++c)
      if (c < nvalid) acc[c & 7] = fmaf(wgt[c], om[c], acc[c & 7]);
    outp[tid] = (((acc[0] + acc[1]) + (acc[2] + acc[3])) + ((acc[4] + acc[5]) + (acc[6] + acc[7]))) * inv_l;
  } else {                              // nvalid > kFewChunks
    __syncthreads();
    const float* po = a.part_o + first * 128 + tid;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    int c = 0;
    for (; c + 8 <= nvalid; c += 8) {
#pragma unroll
      for (int u = 0; u < 8; ++u) acc[u] = fmaf(wgt[c + u], po[(int64_t)(c + u) * rs * 128], acc[u]);
    }
    for (; c < nvalid; ++c) acc[0] = fmaf(wgt[c], po[(int64_t)c * rs * 128], acc[0]);
    outp[tid] = (((acc[0] + acc[1]) + (acc[2] + acc[3])) + ((acc[4] + acc[5]) + (acc[6] + acc[7]))) * inv_l;
  }
}

}  // namespace

namespace {

// Compute units of the current device (cached; 256, the MI355X count, if it cannot be queried).
int device_cu_count() {
  static int cached = 0;
  if (cached == 0) {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && cus > 0)
      cached = cus;
    else
      cached = 256;
  }
  return cached;
}

}  // namespace

// Work items per (KV head, head group) column for one round of the split kernel at `groups_per_cu`
// resident work-groups per compute unit.  The kernels pick the chunk size from the lengths so that
// the batch's chunks number at most this many per column (or one per sequence when the batch has
// more sequences than that).
int64_t split_target(int batch, int64_t cache_cap, int64_t columns, int groups_per_cu) {
  int64_t target = groups_per_cu * (int64_t)device_cu_count() / columns;
  // never more work items than the batch can have chunks (256 tokens at least)
  const int64_t most = (int64_t)batch * ((cache_cap + 255) / 256);
  if (target > most) target = most;
  // A small problem (under 512 tokens per work item at this target) runs one work-group per
  // compute unit: the per-work-group set-up outweighs the extra parallelism (one 32K layer:
  // 15.9 us with 512-token chunks against 19.0 us with 256-token ones, same box)
  const int64_t per_cu = device_cu_count() / columns;
  if ((int64_t)batch * cache_cap < 512 * target && target > per_cu) target = per_cu;
  if (target < 1) target = 1;
  if (target > kMaxChunks) target = kMaxChunks;
  return target;
}

// Chunks per sequence when every length is cap, by the kernels' first estimate of the chunk size
// for this target (the kernels use it to start their set-up loads early; the combine to load the
// rows of the guessed plan).
int guess_chunks_per_seq(int batch, int64_t cache_cap, int64_t target) {
  const int64_t units = (int64_t)batch * ((cache_cap + 127) / 128);
  int64_t c = (units + target - 1) / target * 128;
  const int64_t cmax = (cache_cap + 127) / 128 * 128 < 256 ? 256 : (cache_cap + 127) / 128 * 128;
  if (c < 256) c = 256;
  if (c > cmax) c = cmax;
  return (int)((cache_cap + c - 1) / c);
}

// Resident split-kernel work-groups per compute unit (= waves per SIMD) of each record format.
int split_groups_per_cu(int format) {
  switch (format) {
    case IQ_FMT_U2: return split_waves_per_simd<IQ_FMT_U2>();
    case IQ_FMT_U4: return split_waves_per_simd<IQ_FMT_U4>();
    case IQ_FMT_LM3: return split_waves_per_simd<IQ_FMT_LM3>();
    case IQ_FMT_A3: return split_waves_per_simd<IQ_FMT_A3>();
    default: return split_waves_per_simd<IQ_FMT_U3>();
  }
}

DecodeGeometry decode_geometry(int batch, int n_q_heads, int n_kv_heads, int64_t cache_cap) {
  DecodeGeometry geo{};
  const int G = n_q_heads / n_kv_heads;
  geo.head_groups = (G + 7) / 8;
  // One round of work-groups per (KV head, head group) column; x_max = max(target, batch) work
  // items per column.
  const int64_t columns = (int64_t)n_kv_heads * geo.head_groups;
  // the partial rows are sized for the split kernel with the most work-groups per compute unit
  const int64_t target = split_target(batch, cache_cap, columns, kMaxSplitGroupsPerCU);
  geo.target = (int)target;
  geo.x_max = (int)(target > batch ? target : batch);
  geo.guess_per_seq = guess_chunks_per_seq(batch, cache_cap, target);
  geo.plan_bytes = 256 + ((int64_t)batch * 4 + 255) / 256 * 256;
  // partial rows per query head: x_max, or, when batch counts the query tokens of
  // iq_decode_attention_multi (B sequences of Q >= 2 tokens), kMultiQ rows for each work item of the
  // multi-token kernel: its target, or one per group of kMultiQ tokens
  // (B ceil(Q / kMultiQ) kMultiQ <= B Q + B (kMultiQ - 1) <= B Q (kMultiQ + 1) / 2, as B <= B Q / 2)
  int64_t rows = geo.x_max;
  const int64_t multi_target = (int64_t)kMultiRounds * kMultiWavesPerSimd * device_cu_count() / columns;
  if (kMultiQ * multi_target > rows) rows = kMultiQ * multi_target;
  const int64_t multi_groups = ((int64_t)batch * (kMultiQ + 1) + 1) / 2;
  if (multi_groups > rows) rows = multi_groups;
  const int64_t parts = rows * n_q_heads;
  geo.workspace_bytes = geo.plan_bytes + parts * 128 * 4 + parts * 2 * 4;
  return geo;
}

hipError_t launch_decode(const DecodeLaunch& a, const DecodeGeometry& geo, hipStream_t stream) {
  const int G = a.n_q_heads / a.n_kv_heads;
  const int64_t parts = (int64_t)geo.x_max * a.n_q_heads;
  int* plan = static_cast<int*>(a.workspace);
  float* part_o = reinterpret_cast<float*>(static_cast<char*>(a.workspace) + geo.plan_bytes);
  float* part_ml = part_o + parts * 128;
  const float sm = a.sm_scale > 0.f ? a.sm_scale : kInvSqrtD;

  DecodeKArgs k{};
  k.q_group = 1;
  k.n_groups = a.q_tokens;
  k.q = a.q;
  k.q_bf16 = a.q_bf16;
  k.kc = a.k_codes;
  k.ks = a.k_scales;
  k.vc = a.v_codes;
  k.vs = a.v_scales;
  k.rot = a.rot;
  k.rot_stride_b = a.rot_stride_batch;
  const int vb = a.batch * a.q_tokens;           // work-item sequences
  k.seq_lens = a.seq_lens;
  k.batch = vb;
  k.q_tokens = a.q_tokens;
  k.Hq = a.n_q_heads;
  k.Hkv = a.n_kv_heads;
  k.G = G;
  k.head_groups = geo.head_groups;
  k.cap = a.cache_cap;
  // the plan fills one round of work-groups: 4-bit records run two per compute unit, not three
  // the plan fills one round of work-groups at the format's residency
  const int64_t columns_s = (int64_t)a.n_kv_heads * geo.head_groups;
  const int64_t target_f = split_target(vb, a.cache_cap, columns_s, split_groups_per_cu(a.format));
  k.target = (int)target_f;
  k.sm_log2 = sm * kLog2e;
  k.plan = plan;
  k.x_max = geo.x_max;
  k.guess_per_seq = guess_chunks_per_seq(vb, a.cache_cap, target_f);
  k.part_o = part_o;
  k.part_ml = part_ml;
  k.positions = a.positions;
  k.k_new = a.k_new;
  k.v_new = a.v_new;
  k.new_bf16 = a.new_bf16;
  k.new_stride_seq = a.new_stride_seq;
  k.new_stride_head = a.new_stride_head;
  // (x_max, the partial rows' stride, covers every format's work items)
  const dim3 grid1((unsigned)(a.n_kv_heads * geo.head_groups), (unsigned)(target_f > vb ? target_f : vb), 1u);
  // several query tokens (3-bit records): groups of kMultiQ tokens share each block's unpacked
  // codes; partial rows x kMultiQ + i.  The plan aims at three rounds of work-groups (two when each
  // sequence has one group): with one chunk per (sequence, token group) a single round left compute
  // units idle.
  const bool multi = a.q_tokens > 1 && a.format == IQ_FMT_U3 && a.positions == nullptr;
  int xg = 0;
  if (multi) {
    const int ng = (a.q_tokens + kMultiQ - 1) / kMultiQ;
    const int64_t vbg = (int64_t)a.batch * ng;
    const int64_t columns = (int64_t)a.n_kv_heads * geo.head_groups;
    // (one group per sequence, Q = 4 at 48 layers: 0.273-0.278 ms with two rounds, 0.282-0.284 with
    // three; Q = 16: 0.85-0.87 ms with three, 0.90 with two)
    const int rounds = ng == 1 ? kMultiRoundsOneGroup : kMultiRounds;
    int64_t tg = (int64_t)rounds * kMultiWavesPerSimd * device_cu_count() / columns;
    const int64_t most = vbg * ((a.cache_cap + 255) / 256);
    if (tg > most) tg = most;
    if (tg > kMaxChunks) tg = kMaxChunks;
    if (tg < 1) tg = 1;
    xg = (int)(tg > vbg ? tg : vbg);
    k.batch = (int)vbg;
    k.q_group = kMultiQ;
    k.n_groups = ng;
    k.target = (int)tg;
    k.x_max = xg * kMultiQ;
    part_ml = part_o + (int64_t)k.x_max * a.n_q_heads * 128;
    k.part_ml = part_ml;
    hipLaunchKernelGGL((decode_multi_kernel<kMultiQ>), dim3((unsigned)columns, (unsigned)xg, 1u), dim3(kThreads), 0,
                       stream, k);
  } else if (a.format == IQ_FMT_U2)
    hipLaunchKernelGGL((decode_split_kernel<false, IQ_FMT_U2, kWaves>), grid1, dim3(kThreads), 0, stream, k);
  else if (a.format == IQ_FMT_U4)
    hipLaunchKernelGGL((decode_split_kernel<false, IQ_FMT_U4, kWaves>), grid1, dim3(kThreads), 0, stream, k);
  else if (a.format == IQ_FMT_LM3)
    hipLaunchKernelGGL((decode_split_kernel<false, IQ_FMT_LM3, kWaves>), grid1, dim3(kThreads), 0, stream, k);
  else if (a.format == IQ_FMT_A3)
    hipLaunchKernelGGL((decode_split_kernel<false, IQ_FMT_A3, kWaves>), grid1, dim3(kThreads), 0, stream, k);
  else {
    // 3-bit records: eight waves per work-group when the grid is at most one work-group per
    // compute unit (the set-up and the block chain of one short sequence are the critical path)
    const bool wide = (int64_t)grid1.x * grid1.y <= device_cu_count();
    if (a.positions && wide)
      hipLaunchKernelGGL((decode_split_kernel<true, IQ_FMT_U3, 2 * kWaves>), grid1, dim3(2 * kThreads), 0, stream, k);
    else if (a.positions)
      hipLaunchKernelGGL((decode_split_kernel<true, IQ_FMT_U3, kWaves>), grid1, dim3(kThreads), 0, stream, k);
    else if (wide)
      hipLaunchKernelGGL((decode_split_kernel<false, IQ_FMT_U3, 2 * kWaves>), grid1, dim3(2 * kThreads), 0, stream, k);
    else
      hipLaunchKernelGGL((decode_split_kernel<false, IQ_FMT_U3, kWaves>), grid1, dim3(kThreads), 0, stream, k);
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;

  CombineArgs c{};
  c.part_o = part_o;
  c.part_ml = part_ml;
  c.plan = plan;
  c.seq_lens = a.seq_lens;
  c.positions = a.positions;
  c.Hq = a.n_q_heads;
  c.G = G;
  c.q_tokens = a.q_tokens;
  c.q_group = multi ? kMultiQ : 1;
  c.n_groups = multi ? (a.q_tokens + kMultiQ - 1) / kMultiQ : a.q_tokens;
  c.cap = a.cache_cap;
  c.x_max = multi ? xg * kMultiQ : geo.x_max;
  c.guess_per_seq = k.guess_per_seq;
  c.out = a.out;
  hipLaunchKernelGGL(combine_kernel, dim3((unsigned)(vb * a.n_q_heads)), dim3(128), 0, stream, c);
  return hipGetLastError();
}

}  // namespace iq
