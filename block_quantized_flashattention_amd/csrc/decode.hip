// Decode attention: one query token per sequence and query head against an
// INT8 or packed INT4 KV cache with block or per-token scales (gfx950).
//
// What it computes ([Ascend-INT8] INT8-operator section 3: the decode KV
// cache is stored as INT8 and attention reads it without writing a
// dequantized copy; [FA-INT8/INT4] INT4 layer for the INT4 codes):
//   o_bh = sum_{j < L_b} softmax_j(softmax_scale * q_bh . (sk_j Kc_j)) * sv_j Vc_j
//
// Design (HBM-bound: every valid cache byte is read once, for all the query
// heads that share it):
//   * A workgroup of four wavefronts owns one (batch, KV head, 1024-token
//     chunk) and serves every query head of that KV head (up to 16): each K
//     and V row is read from HBM once for all of them. Each wavefront owns 256
//     consecutive tokens, walked in steps of 32, with its own softmax state;
//     the four merge through LDS at the end. Chunks past a sequence's length
//     exit at once. A second small kernel merges the chunks' partial (max,
//     sum, o) by log-sum-exp; a sequence that fits one chunk is written
//     directly.
//   * Scores on the matrix unit: S^T [16 tokens x 16 heads] = K Q^T with
//     v_mfma_f32_16x16x32 (fp16; bf16 for a bf16 query; an fp32 query is split
//     into a high and a low bf16 part, two products). Lane l supplies token
//     l%16 of a 16-token block and its channels [g D/4, (g+1) D/4), g = l/16,
//     loaded straight from the cache (one or two 16-byte loads). The sum over
//     channels does not depend on which channel sits in which operand slot, so
//     the query operand uses the same slot assignment (packed INT4 keeps the
//     nibble-pair order of its fp16 conversion). Codes become exact fp16 or
//     bf16 in registers.
//   * Softmax on the MFMA output layout: lane l holds head l%16 and tokens
//     4g..4g+3 of each block, so a head's maximum over a step is the maximum
//     of the lane's 8 values and two exchanges across lane groups. The
//     reference maximum moves only when a score exceeds it by more than
//     kSlack (probabilities stay below 2^kSlack, well inside fp16).
//   * P.V on the matrix unit: O^T [16 channels x 16 heads] += V^T P^T per
//     16-channel block, summed over the step's 32 tokens. The probabilities
//     are already in operand layout (slot i of lane group g is token 4g + i of
//     the first block for i < 4, token 16 + 4g + i - 4 of the second for
//     i >= 4); V is staged transposed through LDS with its tokens in that
//     order, four tokens of one channel per 8-byte write, so each lane's
//     operand is one 16-byte read. The V scale is folded into P as
//     p_j sv_j / sv_ref, sv_ref the largest V scale the wavefront has seen
//     (o is scaled down when it grows, as when the reference max moves).
//   * Loads go out in batches of 32 rows of 128 bytes (one 32-token step of
//     INT8 with D = 128, two of packed INT4): 8 KB per wavefront. The next
//     batch is in flight while one is computed, and the first two are
//     requested before the query is read. A wavefront walks an even number
//     of batches (a trailing batch past its tokens is fully masked), so the
//     loop carries no branch around its loads.
#include <mutex>
#include <type_traits>

#include "qfa_device.h"
#include "qfa_launch.h"

namespace qfa {
namespace {

// Split-K partials of qfa_decode_noalloc, for callers that cannot allocate.
// Each device holds its own copy from library load until the process ends.
// Host code must never pass this name to a kernel (on the host it is only a
// stand-in): decode_scratch() looks up each device's address once.
static __device__ __align__(256) float scratch[kDecodeScratchBytes / sizeof(float)];

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kGWaves = 4;
constexpr int kGWaveTokens = kDecodeChunk / kGWaves;  // 256
constexpr int kStep = 32;                              // tokens per step
constexpr int kVtStride = kStep + 8;                   // fp16 per staged V^T row (16-byte rows)
constexpr float kSlack = 8.0f;

// Query dtype handling: fp16 MFMA, bf16 MFMA, or an fp32 query as two bf16 parts.
enum QMode { Q_F16 = 0, Q_BF16 = 1, Q_F32 = 2 };

struct DecParams {
  const void* q;
  const uint8_t* k;
  const uint8_t* v;
  const void* ks;
  const void* vs;
  const int32_t* lens;
  void* out;
  float* ws;
  int Hq, Hkv, group, S_max, max_splits;
  long c_row, c_head, c_batch;  // byte strides of the caches
  long q_head, q_batch;         // element strides of q and out
  int kv_block, nkblk, kv_scale_f16, q_dtype, out_dtype;
  float scale_log2;
  // Every sequence in max_splits chunks of equal length, so no workgroup of
  // the grid is empty (grouped heads, and one head per KV head with the INT8
  // cache); else ceil(L / kDecodeChunk) chunks of kDecodeChunk tokens.
  int all_splits;
};

__device__ __forceinline__ void store_out(void* out, long i, float v, int dt) {
  if (dt == QFA_F32) ((float*)out)[i] = v;
  else if (dt == QFA_F16) ((uint16_t*)out)[i] = (uint16_t)f32_to_f16_bits(v);
  else ((uint16_t*)out)[i] = (uint16_t)f32_to_bf16_bits(v);
}

// Raw buffer resource over [base, base + bytes): loads past the end return
// zero. The last word is the gfx9 default (32-bit data format, no swizzle).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const uint8_t* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base), (short)0, bytes, 0x00020000);
}

// BYTES (4, 8, 16, or 32 as two loads) at byte offset `off` of a buffer.
template <int BYTES>
__device__ __forceinline__ void bload(uint32_t* dst, __amdgpu_buffer_rsrc_t rs, int off) {
  if constexpr (BYTES == 32) {
    bload<16>(dst, rs, off);
    bload<16>(dst + 4, rs, off + 16);
  } else if constexpr (BYTES == 16) {
    const auto r = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0);
    dst[0] = r[0]; dst[1] = r[1]; dst[2] = r[2]; dst[3] = r[3];
  } else if constexpr (BYTES == 8) {
    const auto r = __builtin_amdgcn_raw_buffer_load_b64(rs, off, 0, 0);
    dst[0] = r[0]; dst[1] = r[1];
  } else {
    dst[0] = __builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, 0);
  }
}

// A scale as loaded: the fp16 bits or the fp32 value, one load each, kept
// untouched until the value is used. Any operation on a loaded value makes
// the compiler wait for that load (and, counting in order, for every load
// issued before it); two 16-bit halves combined into one register right
// after the next batch's loads were issued waited for the whole batch in the
// middle of the current step.
template <bool F16S>
struct ScaleT {
  using type = typename std::conditional<F16S, uint16_t, float>::type;
};
template <bool F16S>
__device__ __forceinline__ typename ScaleT<F16S>::type raw_scale(const void* p, long idx) {
  return ((const typename ScaleT<F16S>::type*)p)[idx];
}
template <bool F16S>
__device__ __forceinline__ float scale_value(typename ScaleT<F16S>::type r) {
  if constexpr (F16S) return (float)__builtin_bit_cast(_Float16, r);
  else return r;
}

// Four signed bytes as two exact fp16 pairs (1024 + (byte ^ 0x80) - 1152).
template <bool OFF = false>
__device__ __forceinline__ void i8x4_to_h(uint32_t w, f16x2& lo, f16x2& hi) {
  const uint32_t u = w ^ 0x80808080u;
  lo = __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(0x64646464u, u, 0x05010400u));
  hi = __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(0x64646464u, u, 0x07030602u));
  if constexpr (!OFF) {
    const f16x2 bias = {(_Float16)1152.0f, (_Float16)1152.0f};
    lo = lo - bias;
    hi = hi - bias;
  }
}

// The fp16 offset of a code left in offset form (OFF): 1152 + code (INT8),
// 1032 + code (INT4), both exact.
template <bool INT4>
constexpr float kCodeOffset = INT4 ? 1032.0f : 1152.0f;

// Nibbles at bits s..s+3 and 16+s..19+s of w, whose sign bits were already
// flipped, as the fp16 pair 1032 + code (exact).
__device__ __forceinline__ f16x2 i4_pair_h(uint32_t wflip, int s) {
  return __builtin_bit_cast(f16x2, ((wflip >> s) & 0x000F000Fu) | 0x64006400u);
}

// Element i of a bf16 pair vector from the bf16 bits of two exact values.
__device__ __forceinline__ uint32_t bf16_pair(float a, float b) {
  // a and b are small integers (codes): their fp32 bits end in 16 zero bits.
  return __builtin_amdgcn_perm(__float_as_uint(b), __float_as_uint(a), 0x07060302u);
}

// K operand of k-step j from the lane's K words (D/4 channels of one token).
// fp16: INT8 channels in order; INT4 in the nibble-pair order
// (d, d+4, d+1, d+5, d+2, d+6, d+3, d+7) of one word. bf16: channels in order.
// OFF: the codes in offset form (kCodeOffset + code).
template <bool INT4, bool OFF = false>
__device__ __forceinline__ f16x8 k_operand_f16(const uint32_t* kw, int j) {
  f16x8 r;
  if constexpr (!INT4) {
    f16x2 a, b, c, d;
    i8x4_to_h<OFF>(kw[2 * j], a, b);
    i8x4_to_h<OFF>(kw[2 * j + 1], c, d);
    r = (f16x8){a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
  } else {
    const uint32_t w = kw[j] ^ 0x88888888u;
    f16x2 a = i4_pair_h(w, 0), b = i4_pair_h(w, 4), c = i4_pair_h(w, 8), d = i4_pair_h(w, 12);
    if constexpr (!OFF) {
      const f16x2 bias = {(_Float16)1032.0f, (_Float16)1032.0f};
      a = a - bias;
      b = b - bias;
      c = c - bias;
      d = d - bias;
    }
    r = (f16x8){a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
  }
  return r;
}
// Code u - off as a float, exactly: u (at most 8 bits) goes into the low
// mantissa bits of 2^23, and 2^23 + off is subtracted. No integer-to-float
// conversion: the compiler rewrote a sign-extract plus conversion into an
// unsigned conversion of the sign-extended byte, which is wrong for
// negative codes.
__device__ __forceinline__ float code_f32(uint32_t u, float off) {
  return __uint_as_float(0x4B000000u | u) - (8388608.0f + off);
}

template <bool INT4>
__device__ __forceinline__ bf16x8 k_operand_bf16(const uint32_t* kw, int j) {
  uint32_t u[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    float a, b;
    if constexpr (!INT4) {
      const uint32_t w = kw[2 * j + e / 2] ^ 0x80808080u;
      const int s = 16 * (e & 1);
      a = code_f32((w >> s) & 0xFFu, 128.0f);
      b = code_f32((w >> (s + 8)) & 0xFFu, 128.0f);
    } else {
      const uint32_t w = kw[j] ^ 0x88888888u;
      a = code_f32((w >> (8 * e)) & 0xFu, 8.0f);
      b = code_f32((w >> (8 * e + 4)) & 0xFu, 8.0f);
    }
    u[e] = bf16_pair(a, b);
  }
  return __builtin_bit_cast(bf16x8, (i32x4){(int)u[0], (int)u[1], (int)u[2], (int)u[3]});
}

// Channel offset (within the lane's D/4 channels) of slot i of k-step j.
template <bool INT4, int QM>
__device__ __forceinline__ int slot_channel(int j, int i) {
  if constexpr (INT4 && QM == Q_F16) return 8 * j + (i >> 1) + 4 * (i & 1);
  return 8 * j + i;
}

template <int D, bool INT4>
struct DecGeo {
  static constexpr int kRowBytes = INT4 ? D / 2 : D;
  static constexpr int kKBytes = kRowBytes / 4;  // per lane and 16-token block
  static constexpr int kKWords = kKBytes / 4;
  static constexpr int kVBytes = kRowBytes / 8;  // per lane and token (D/8 channels)
  static constexpr int kVWords = kVBytes / 4;
  static constexpr int kKSteps = D / 32;         // MFMA k-steps per 16-token block
  static constexpr int kCB = D / 16;             // 16-channel blocks of O
  // 32-token steps per load batch: a batch always carries 32 rows of 128
  // bytes (8 KB per wavefront in flight), whatever the row size.
  static constexpr int kSub = 128 / kRowBytes;
};

// One load batch: the codes of kSub steps (and, with block scales, each
// step's K and V scale).
template <int D, bool INT4, bool F16S>
struct StepRegs {
  static constexpr int kSub = DecGeo<D, INT4>::kSub;
  uint32_t k[kSub][2][DecGeo<D, INT4>::kKWords];
  uint32_t v[kSub][4][DecGeo<D, INT4>::kVWords];
  typename ScaleT<F16S>::type ks[kSub], vs[kSub];
};

// Stage this lane's 4 tokens x D/8 channels of V (codes) into the wavefront's
// V^T buffer as fp16: channel c of the lane's group, tokens in operand order.
template <int D, bool INT4, bool OFF = false>
__device__ __forceinline__ void stage_v(const uint32_t (&v)[4][DecGeo<D, INT4>::kVWords],
                                        _Float16* vt, int c0, int pos0) {
  using G = DecGeo<D, INT4>;
#pragma unroll
  for (int k = 0; k < G::kVWords; ++k) {
    if constexpr (!INT4) {
      // Channels 4k..4k+3: transpose the 4x4 bytes (tokens x channels), then
      // convert each channel's token pairs.
      const uint32_t d01l = __builtin_amdgcn_perm(v[1][k], v[0][k], 0x05010400u);
      const uint32_t d01h = __builtin_amdgcn_perm(v[1][k], v[0][k], 0x07030602u);
      const uint32_t d23l = __builtin_amdgcn_perm(v[3][k], v[2][k], 0x05010400u);
      const uint32_t d23h = __builtin_amdgcn_perm(v[3][k], v[2][k], 0x07030602u);
      f16x2 a0, a1, b0, b1, c0h, c1h, e0, e1;
      i8x4_to_h<OFF>(d01l, a0, a1);   // channel 4k: tokens 0,1 | channel 4k+1: tokens 0,1
      i8x4_to_h<OFF>(d23l, b0, b1);   // the same, tokens 2,3
      i8x4_to_h<OFF>(d01h, c0h, c1h); // channels 4k+2, 4k+3: tokens 0,1
      i8x4_to_h<OFF>(d23h, e0, e1);   // tokens 2,3
      const int c = c0 + 4 * k;
      *(f16x4*)(vt + (c + 0) * kVtStride + pos0) = (f16x4){a0[0], a0[1], b0[0], b0[1]};
      *(f16x4*)(vt + (c + 1) * kVtStride + pos0) = (f16x4){a1[0], a1[1], b1[0], b1[1]};
      *(f16x4*)(vt + (c + 2) * kVtStride + pos0) = (f16x4){c0h[0], c0h[1], e0[0], e0[1]};
      *(f16x4*)(vt + (c + 3) * kVtStride + pos0) = (f16x4){c1h[0], c1h[1], e1[0], e1[1]};
    } else {
      // Channels 8k..8k+7: nibble pairs (c, c+4) per token, then token pairs.
      uint32_t w[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) w[t] = v[t][k] ^ 0x88888888u;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        uint32_t x[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) x[t] = __builtin_bit_cast(uint32_t, i4_pair_h(w[t], 4 * s));
        f16x2 lo01 = __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(x[1], x[0], 0x05040100u));
        f16x2 lo23 = __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(x[3], x[2], 0x05040100u));
        f16x2 hi01 = __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(x[1], x[0], 0x07060302u));
        f16x2 hi23 = __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(x[3], x[2], 0x07060302u));
        if constexpr (!OFF) {
          const f16x2 bias = {(_Float16)1032.0f, (_Float16)1032.0f};
          lo01 = lo01 - bias;
          lo23 = lo23 - bias;
          hi01 = hi01 - bias;
          hi23 = hi23 - bias;
        }
        const int c = c0 + 8 * k + s;  // shift 4s: channel s and s + 4 of the word
        *(f16x4*)(vt + c * kVtStride + pos0) = (f16x4){lo01[0], lo01[1], lo23[0], lo23[1]};
        *(f16x4*)(vt + (c + 4) * kVtStride + pos0) = (f16x4){hi01[0], hi01[1], hi23[0], hi23[1]};
      }
    }
  }
}

// Three workgroups per CU (at most 168 VGPRs); the fp32 query, which keeps
// two bf16 operand sets, two (it would spill at three).
template <int D, bool INT4, int QM, bool BS, bool F16S>
__global__ __launch_bounds__(64 * kGWaves, QM == Q_F32 ? 2 : 3) void decode_gqa_kernel(DecParams p) {
  using G = DecGeo<D, INT4>;
  using Regs = StepRegs<D, INT4, F16S>;
  // Per wavefront: V^T [D][kVtStride] fp16. After the loop the same bytes
  // hold the merge of the four wavefronts: o [4][16][D], m [4][16], l [4][16].
  __shared__ __attribute__((aligned(16))) _Float16 vt_all[kGWaves * D * kVtStride];
  static_assert(kGWaves * 16 * (D + 2) * 4 <= (int)sizeof(vt_all), "merge area");

  const int split = blockIdx.x;
  const int kvh = blockIdx.y;
  const int b = blockIdx.z;
  const int L = min(max(p.lens[b], 1), p.S_max);
  const int nsplit = p.all_splits ? p.max_splits : (L + kDecodeChunk - 1) / kDecodeChunk;
  if (split >= nsplit) return;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int g = lane >> 4;   // lane group: channels [g D/4, (g+1) D/4) of K, tokens 4g.. of S^T
  const int n = lane & 15;   // token of a K block (A operand); head of S^T, P^T and O^T
  const int grp = p.group;
  _Float16* vt = vt_all + wave * D * kVtStride;

  constexpr int kSub = G::kSub;
  constexpr int kBatch = kStep * kSub;  // tokens per load batch
  // Every sequence in max_splits chunks of equal length (starts at multiples
  // of kStep) and equal wavefront shares (multiples of kStep, so block
  // scales stay uniform over a step): a workgroup's duration follows its
  // length and none is empty (as in the single-head kernel).
  const int cs = (int)((long)split * L / nsplit) / kStep * kStep;
  const int ce = split + 1 == nsplit ? L : (int)((long)(split + 1) * L / nsplit) / kStep * kStep;
  const int pw = ((ce - cs + kGWaves - 1) / kGWaves + kStep - 1) / kStep * kStep;
  const int t_begin = __builtin_amdgcn_readfirstlane(min(cs + wave * pw, ce));
  const int t_end = min(t_begin + pw, ce);
  const int nbatch = t_begin < t_end ? (t_end - t_begin + kBatch - 1) / kBatch : 0;
  const long sbase = ((long)b * p.Hkv + kvh) * p.nkblk;

  // Rows [0, L) of this (batch, KV head) through buffer resources: rows at or
  // past L read as zero (their scores are masked). Offsets stay below 2^31
  // (the host checks (S_max + chunk) * row stride).
  // This wavefront's rows [t_begin, t_end): rows past t_end read as zero.
  const long cbase = (long)b * p.c_batch + (long)kvh * p.c_head + (long)t_begin * p.c_row;
  const int span = max(t_end - t_begin - 1, 0) * (int)p.c_row + G::kRowBytes;
  const auto krs = rows_rsrc(p.k + cbase, span);
  const auto vrs = rows_rsrc(p.v + cbase, span);
  const int crow = (int)p.c_row;
  const int tq = lane >> 3, cg = lane & 7;  // V staging: tokens 4tq..4tq+3, channel group cg
  const int pos0 = tq < 4 ? 8 * tq : 8 * (tq - 4) + 4;

  auto issue = [&](Regs& r, int s) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < kSub; ++u) {
      const int t0 = t_begin + kBatch * s + kStep * u;
      if constexpr (BS) {
        const long blk = sbase + min(t0, L - 1) / p.kv_block;
        r.ks[u] = raw_scale<F16S>(p.ks, blk);
        r.vs[u] = raw_scale<F16S>(p.vs, blk);
      }
#pragma unroll
      for (int tb = 0; tb < 2; ++tb)
        bload<G::kKBytes>(r.k[u][tb], krs, (t0 - t_begin + 16 * tb + n) * crow + g * G::kKBytes);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        bload<G::kVBytes>(r.v[u][i], vrs, (t0 - t_begin + 4 * tq + i) * crow + cg * G::kVBytes);
    }
  };

  // The first two load batches go out before anything else is read.
  Regs ra, rb;
  if (nbatch > 0) {
    issue(ra, 0);
    issue(rb, min(1, nbatch - 1));
  }

  // Query operand (B of S^T = K Q^T): head n of this KV head's group, the
  // channels of this lane's slots; zero for heads past the group.
  const bool hvalid = n < grp;
  const long qoff = (long)b * p.q_batch + (long)(kvh * grp + (hvalid ? n : 0)) * p.q_head + g * (D / 4);
  f16x8 qh[G::kKSteps];
  bf16x8 qb[G::kKSteps], qb2[G::kKSteps];
#pragma unroll
  for (int j = 0; j < G::kKSteps; ++j) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int d = slot_channel<INT4, QM>(j, i);
      if constexpr (QM == Q_F16) {
        const uint16_t bits = ((const uint16_t*)p.q)[qoff + d];
        qh[j][i] = hvalid ? __builtin_bit_cast(_Float16, bits) : (_Float16)0.0f;
      } else if constexpr (QM == Q_BF16) {
        const uint16_t bits = ((const uint16_t*)p.q)[qoff + d];
        qb[j][i] = __builtin_bit_cast(__bf16, (uint16_t)(hvalid ? bits : 0));
      } else {
        const float x = hvalid ? ((const float*)p.q)[qoff + d] : 0.0f;
        const uint32_t hi = f32_to_bf16_bits(x);
        const float rest = x - __uint_as_float(hi << 16);
        qb[j][i] = __builtin_bit_cast(__bf16, (uint16_t)hi);
        qb2[j][i] = __builtin_bit_cast(__bf16, (uint16_t)f32_to_bf16_bits(rest));
      }
    }
  }

  // fp16 query: the K and V operands keep the codes in offset form
  // (kCodeOffset + code, exact), which saves a subtraction per code pair;
  // the offset's share of a score, kCodeOffset * sum(q) for head n, and of
  // O, kCodeOffset times the sum of the fp16 weights, are removed afterwards.
  constexpr bool kOffs = QM == Q_F16;
  constexpr float kCO = kCodeOffset<INT4>;
  float offq = 0.0f;
  if constexpr (kOffs) {
    float qs = 0.0f;
#pragma unroll
    for (int j = 0; j < G::kKSteps; ++j)
#pragma unroll
      for (int i = 0; i < 8; ++i) qs += (float)qh[j][i];
    qs += __shfl_xor(qs, 16);
    qs += __shfl_xor(qs, 32);
    offq = kCO * qs;
  }
  float wsum = 0.0f;  // (kOffs) this lane's sum of the fp16 weights of head n, in o's units

  f32x4 o[G::kCB];
#pragma unroll
  for (int cb = 0; cb < G::kCB; ++cb) o[cb] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
  float m_ref = -INFINITY;  // reference max of head n (log2 units), same in the 4 lane groups
  float l_sum = 0.0f;       // this lane's part of head n's sum, in units of exp2(-m_ref)
  // V scale o is expressed in: the largest V scale seen so far (o is scaled
  // down when a larger one arrives), so the fp16 weights p sv / sv_ref stay
  // at most 2^kSlack.
  float sv_ref = 0.0f;
  float inv_ref = 0.0f;  // 1 / sv_ref (0 while sv_ref is 0), updated when sv_ref changes

  auto step = [&](const Regs& r, int u, int t0) __attribute__((always_inline)) {
    stage_v<D, INT4, kOffs>(r.v[u], vt, cg * (D / 8), pos0);

    // Scores: two 16-token blocks.
    f32x4 sacc[2];
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
      sacc[tb] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int j = 0; j < G::kKSteps; ++j) {
        if constexpr (QM == Q_F16) {
          sacc[tb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(k_operand_f16<INT4, kOffs>(r.k[u][tb], j),
                                                            qh[j], sacc[tb], 0, 0, 0);
        } else {
          const bf16x8 ka = k_operand_bf16<INT4>(r.k[u][tb], j);
          sacc[tb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qb[j], sacc[tb], 0, 0, 0);
          if constexpr (QM == Q_F32)
            sacc[tb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qb2[j], sacc[tb], 0, 0, 0);
        }
      }
    }

    // Scaled, masked scores of this lane (y[4 tb + i] is token t0 + 16 tb +
    // 4g + i) and their V scales.
    float y[8], sv[8];
    const float ck_blk = BS ? scale_value<F16S>(r.ks[u]) * p.scale_log2 : 0.0f;
    const float ckoff = -offq * ck_blk;  // block scales: the offset's share, scaled
    const float sv_blk = BS ? scale_value<F16S>(r.vs[u]) : 0.0f;
    float sv_max = sv_blk;
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = t0 + 16 * tb + 4 * g + i;
        float ck = ck_blk, svt = sv_blk;
        if constexpr (!BS) {
          const long blk = sbase + min(t, L - 1) / p.kv_block;
          ck = scale_value<F16S>(raw_scale<F16S>(p.ks, blk)) * p.scale_log2;
          svt = scale_value<F16S>(raw_scale<F16S>(p.vs, blk));
          sv_max = fmaxf(sv_max, t < t_end ? svt : 0.0f);
        }
        const float yv = BS ? __builtin_fmaf(sacc[tb][i], ck, ckoff) : (sacc[tb][i] - offq) * ck;
        y[4 * tb + i] = t < t_end ? yv : -INFINITY;
        sv[4 * tb + i] = svt;
      }
    if constexpr (!BS) {
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) sv_max = fmaxf(sv_max, __shfl_xor(sv_max, off));
    } else {
      sv_max = t0 < t_end ? sv_max : 0.0f;
    }
    float mx = y[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) mx = fmaxf(mx, y[i]);
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    // Lazy rescale, decided for the whole wavefront: a new reference max, or
    // a larger V scale (sv_max is uniform over the wavefront).
    const bool need = mx > m_ref + kSlack;
    if (__builtin_amdgcn_ballot_w64(need) || sv_max > sv_ref) {
      const float m_new = need ? mx : m_ref;
      const float sv_new = fmaxf(sv_ref, sv_max);
      // 0 on the first step (m_ref = -inf, sv_ref = 0)
      const float alpha = sv_ref > 0.0f ? __builtin_amdgcn_exp2f(m_ref - m_new) * (sv_ref / sv_new) : 0.0f;
      const float lalpha = m_new == m_ref ? 1.0f : __builtin_amdgcn_exp2f(m_ref - m_new);
#pragma unroll
      for (int cb = 0; cb < G::kCB; ++cb) o[cb] *= alpha;
      wsum *= alpha;
      l_sum *= lalpha;
      m_ref = m_new;
      if (sv_new != sv_ref) inv_ref = 1.0f / sv_new;  // sv_new > 0 here
      sv_ref = sv_new;
    }
    const float mref = m_ref == -INFINITY ? 0.0f : m_ref;
    f16x8 pb;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float pr = __builtin_amdgcn_exp2f(y[i] - mref);
      l_sum += pr;
      pb[i] = (_Float16)(pr * (sv[i] * inv_ref));
    }
    if constexpr (kOffs) {
      const f16x2 one = {(_Float16)1.0f, (_Float16)1.0f};
#pragma unroll
      for (int i = 0; i < 8; i += 2)
        wsum = __builtin_amdgcn_fdot2((f16x2){pb[i], pb[i + 1]}, one, wsum, false);
    }

    // P.V: the staged V^T rows of this lane's channels, tokens in slot order.
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int cb = 0; cb < G::kCB; ++cb) {
      const f16x8 a = *(const f16x8*)(vt + (cb * 16 + n) * kVtStride + 8 * g);
      o[cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, pb, o[cb], 0, 0, 0);
    }
    __builtin_amdgcn_wave_barrier();
  };
  auto compute = [&](const Regs& r, int s) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < kSub; ++u) {
      step(r, u, t_begin + kBatch * s + kStep * u);
      // one step's conversions at a time: interleaving two spills
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // An even number of batches; a trailing batch past the tokens is fully
  // masked and its loads repeat the last batch's rows. While one batch is
  // computed the next is in flight.
  const int nbatch2 = (nbatch + 1) & ~1;
  // The fences keep every use of a batch after the issue of the next one:
  // the scheduler otherwise moved the start of a batch's work above the
  // following issue, leaving nothing in flight while the batch was awaited.
  for (int s = 0; s < nbatch2; s += 2) {
    compute(ra, s);
    issue(ra, min(s + 2, nbatch - 1));
    __builtin_amdgcn_sched_barrier(0);
    compute(rb, s + 1);
    issue(rb, min(s + 3, nbatch - 1));
    __builtin_amdgcn_sched_barrier(0);
  }

  l_sum += __shfl_xor(l_sum, 16);
  l_sum += __shfl_xor(l_sum, 32);
  if constexpr (kOffs) {
    wsum += __shfl_xor(wsum, 16);
    wsum += __shfl_xor(wsum, 32);
#pragma unroll
    for (int cb = 0; cb < G::kCB; ++cb) o[cb] -= kCO * wsum;
  }

  // Merge the four wavefronts (o in V-scale units: times sv_ref).
  __syncthreads();
  float* mo = (float*)vt_all;            // [4][16][D]
  float* mm = mo + kGWaves * 16 * D;   // [4][16]
  float* ml = mm + kGWaves * 16;       // [4][16]
#pragma unroll
  for (int cb = 0; cb < G::kCB; ++cb)
    *(f32x4*)(mo + (wave * 16 + n) * D + cb * 16 + 4 * g) = o[cb] * sv_ref;
  if (g == 0) {
    mm[wave * 16 + n] = m_ref;
    ml[wave * 16 + n] = l_sum;
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < grp * D; idx += 64 * kGWaves) {
    const int hn = idx / D, c = idx % D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kGWaves; ++w) M = fmaxf(M, mm[w * 16 + hn]);
    float lsum = 0.0f, acc = 0.0f;
#pragma unroll
    for (int w = 0; w < kGWaves; ++w) {
      const float mw = mm[w * 16 + hn];
      const float cw = mw == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(mw - M);
      lsum += ml[w * 16 + hn] * cw;
      acc += mo[(w * 16 + hn) * D + c] * cw;
    }
    const int h = kvh * grp + hn;
    if (nsplit == 1) {
      store_out(p.out, (long)b * p.q_batch + (long)h * p.q_head + c, acc / lsum, p.out_dtype);
    } else {
      float* part = p.ws + (((long)b * p.Hq + h) * p.max_splits + split) * (D + 2);
      part[c] = acc;
      if (c == 0) {
        part[D] = M;
        part[D + 1] = lsum;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// One query head per KV head (no GQA sharing to exploit): dot products on the
// vector unit, which for a single head reads the cache at a higher rate than
// the matrix-unit kernel below.
// ---------------------------------------------------------------------------

constexpr int kSWaves = 8;
constexpr int kSWaveTokens = kDecodeChunk / kSWaves;  // 128
constexpr int kSLoadGroup = 4;                         // loads issued together

template <int LPT>
__device__ __forceinline__ float lane_group_sum(float v) {
  // quad_perm [1,0,3,2] and [2,3,0,1]: partners at lane xor 1 and xor 2.
  v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, true));
  if constexpr (LPT >= 4)
    v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, true));
  if constexpr (LPT >= 8)  // row_half_mirror: lane i <-> 7-i within each 8 lanes
    v += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x141, 0xF, 0xF, true));
  return v;
}

// The nibbles at bits 0-3 and 16-19 of w (two's-complement codes) as an fp16
// pair 1032 + code, exact: flip the sign bit, keep the nibbles, set the
// exponent of 1024.
__device__ __forceinline__ uint32_t i4_pair_bits(uint32_t w) {
  return ((w ^ 0x00080008u) & 0x000F000Fu) | 0x64006400u;
}

// Offset codes (code + 128, or code + 8 for INT4) of one 16-byte chunk as floats.
template <bool INT4>
__device__ __forceinline__ void chunk_to_f32(const uint4& w, float* f) {
  const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
  if constexpr (!INT4) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t u = ww[i] ^ 0x80808080u;
      f[4 * i + 0] = (float)(u & 0xFFu);
      f[4 * i + 1] = (float)((u >> 8) & 0xFFu);
      f[4 * i + 2] = (float)((u >> 16) & 0xFFu);
      f[4 * i + 3] = (float)(u >> 24);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t u = ww[i] ^ 0x88888888u;
      const uint32_t lo = u & 0x0F0F0F0Fu, hi = (u >> 4) & 0x0F0F0F0Fu;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        f[8 * i + 2 * j] = (float)((lo >> (8 * j)) & 0xFFu);
        f[8 * i + 2 * j + 1] = (float)((hi >> (8 * j)) & 0xFFu);
      }
    }
  }
}

// Sums v[0..N) over the lanes that differ only in the lane bits OFF, 2*OFF,
// ..., 32, leaving each lane one slice of the sums: every step halves the
// values a lane holds, sending one half to its partner and adding the half it
// receives (a reduce-scatter; log2(64/OFF) steps, N - N*OFF/64 exchanges).
// The lane then holds the sums of channels scatter_base(lane) + [0, N*OFF/64).
template <int OFF, int N>
__device__ __forceinline__ void sum_scatter(float* v, int lane) {
  if constexpr (OFF < 64) {
    constexpr int H = N / 2;
    const bool up = (lane & OFF) != 0;
#pragma unroll
    for (int i = 0; i < H; ++i) {
      const float send = up ? v[i] : v[i + H];
      const float keep = up ? v[i + H] : v[i];
      v[i] = keep + __shfl_xor(send, OFF);
    }
    sum_scatter<OFF * 2, H>(v, lane);
  }
}
template <int OFF, int N>
__device__ __forceinline__ int scatter_base(int lane) {
  if constexpr (OFF < 64) {
    return ((lane & OFF) ? N / 2 : 0) + scatter_base<OFF * 2, N / 2>(lane);
  } else {
    return 0;
  }
}

// Packed INT4 with an fp16 query and block scales asks for six wavefronts per
// SIMD, i.e. three workgroups per CU (at most 80 VGPRs): its rows are half as
// long, so more of them must be in flight to cover the HBM latency.
template <int D, bool INT4, bool QF16, bool BLOCK_SCALE>
__global__ __launch_bounds__(64 * kSWaves, INT4 && QF16 && BLOCK_SCALE ? 6 : 2)
void decode_mha_kernel(DecParams p) {
  constexpr int kRowBytes = INT4 ? D / 2 : D;
  constexpr int LPT = kRowBytes / 16;        // lanes per token
  constexpr int EPL = INT4 ? 32 : 16;        // channels per lane
  constexpr int TPS = 64 / LPT;              // tokens per wavefront load
  constexpr int NSUB = kSWaveTokens / TPS;    // loads per lane per wavefront chunk
  constexpr int NG = NSUB / kSLoadGroup;
  constexpr float kOff = INT4 ? 8.0f : 128.0f;
  static_assert(NSUB % kSLoadGroup == 0, "load groups");
  constexpr int NF = EPL / (64 / LPT);  // channels per lane after the token-group reduction
  static_assert(NF >= 1 && EPL % (64 / LPT) == 0, "reduce-scatter");
  __shared__ float red_m[kSWaves], red_l[kSWaves];
  __shared__ float red_o[kSWaves][D];

  const int split = blockIdx.x;
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  const int L = min(max(p.lens[b], 1), p.S_max);
  const int nsplit = (!INT4 && p.all_splits) ? p.max_splits : (L + kDecodeChunk - 1) / kDecodeChunk;
  if (split >= nsplit) return;
  const int kvh = h / p.group;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int tg = lane / LPT;  // token within a load
  const int dc = lane % LPT;  // channel chunk
  const int d0 = dc * EPL;

  // This lane's query channels: fp16 pairs for the dot2 path, else floats.
  // The loads are issued here and used only after the first keys are
  // requested, and the dtype is decided once, outside the loads (a
  // per-element switch between dependent conversions serialized the loads'
  // latencies).
  const long qoff = (long)b * p.q_batch + (long)h * p.q_head;
  f16x2 qh[EPL / 2];
  float qf[EPL];
  float qsum = 0.0f;
  uint32_t qw[QF16 ? EPL / 2 : 1];
  if constexpr (QF16) {
    const uint32_t* qp = (const uint32_t*)((const uint16_t*)p.q + qoff + d0);
#pragma unroll
    for (int i = 0; i < EPL / 2; ++i) qw[i] = qp[i];
  } else if (p.q_dtype == QFA_F32) {
#pragma unroll
    for (int e = 0; e < EPL; ++e) qf[e] = ((const float*)p.q)[qoff + d0 + e];
  } else {
#pragma unroll
    for (int e = 0; e < EPL; ++e) qf[e] = bf16_bits_to_f32(((const uint16_t*)p.q)[qoff + d0 + e]);
  }
  // Packed INT4 keys are read as channel pairs (e, e + 4) of each group of 8
  // (the nibbles one shift-and-mask isolates); INT8 keys as (2e, 2e + 1).
  constexpr bool kI4H = INT4 && QF16;
  auto prep_q = [&]() {
    if constexpr (QF16) {
#pragma unroll
      for (int i = 0; i < EPL / 2; ++i) {
        qsum += f16_bits_to_f32(qw[i] & 0xFFFFu);
        qsum += f16_bits_to_f32(qw[i] >> 16);
      }
#pragma unroll
      for (int e = 0; e < EPL / 2; ++e) {
        if constexpr (kI4H) {
          // Channels c and c + 4 (c = 8(e/4) + e%4) share the half of dwords c/2 and c/2 + 2.
          const int c0 = 8 * (e / 4) + (e % 4);
          const uint32_t sel = (c0 & 1) ? 0x07060302u : 0x05040100u;
          qh[e] = __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(qw[c0 / 2 + 2], qw[c0 / 2], sel));
        } else {
          qh[e] = __builtin_bit_cast(f16x2, qw[e]);
        }
      }
    } else {
#pragma unroll
      for (int e = 0; e < EPL; ++e) qsum += qf[e];
    }
  };

  const long cbase = (long)b * p.c_batch + (long)kvh * p.c_head;
  const long sbase = ((long)b * p.Hkv + kvh) * p.nkblk;

  // INT8 cache (kBal): every sequence is split into max_splits chunks of
  // equal length (at most kDecodeChunk, as max_splits covers S_max) and each
  // wavefront takes an equal share of its chunk (at most kSWaveTokens), so a
  // workgroup's duration follows its length and no workgroup of the grid is
  // empty. With fixed 1024-token chunks the last, partial chunk of every
  // sequence left wavefronts idle for a whole chunk's time and the chunks
  // past a sequence's end left workgroups empty (measured on the ragged
  // decode workload: 5.2 TB/s, against 6.05 TB/s with every sequence at full
  // length). The packed INT4 cache keeps fixed chunks: the per-token
  // block-scale handling an equal share needs cost it more than the balance
  // gained.
  constexpr bool kBal = !INT4;
  int t_begin, t_end;
  if constexpr (kBal) {
    const int cs = (int)((long)split * L / nsplit), ce = (int)((long)(split + 1) * L / nsplit);
    const int pw = (ce - cs + kSWaves - 1) / kSWaves;
    // One value per wavefront (scalar, so the buffer resources below are too).
    t_begin = __builtin_amdgcn_readfirstlane(cs + wave * pw);
    t_end = min(t_begin + pw, ce);
  } else {
    t_begin = split * kDecodeChunk + wave * kSWaveTokens;
    t_end = min(t_begin + kSWaveTokens, L);
  }
  const int t_last = t_end - 1;

  float m_blk = -INFINITY, l_blk = 0.0f, wsum = 0.0f;
  float o[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) o[e] = 0.0f;
  // Block scales: a wavefront's tokens (at most kSWaveTokens <= kv_block)
  // lie in block b0 and, with kBal, possibly the next from (b0 + 1) kv_block
  // on. The K scales go into the score factors; the V scales, with kBal, as
  // ratios to the larger of the two (sv_ref) in each token's weight, O being
  // kept in units of sv_ref; otherwise sv_ref is the one block's V scale.
  float csk0 = 0.0f, csk1 = 0.0f, rv0 = 1.0f, rv1 = 1.0f, sv_ref = 1.0f;
  int dnd = 0;  // lane's tokens t_begin + tg + j TPS lie in block b0 while j TPS < dnd

  if (t_begin < t_end) {
    // ---- scores: sc[j] for token t_begin + j*TPS + tg (log2 units) ----
    float sc[NSUB];
    uint4 kw[2][kSLoadGroup];
    // This wavefront's rows of the (batch, KV head) through buffer resources
    // (kBal: [t_begin, t_end); else [t_begin, L)): one 32-bit offset per lane
    // (the host keeps every offset below 2^31), and rows past the end read as
    // zero without a memory access, so no clamp is needed (their scores are
    // masked).
    const int t0 = kBal ? t_begin : 0;  // first row of the resources (uniform)
    const long wbase = cbase + (long)t0 * p.c_row;
    const int span = ((kBal ? t_end : L) - t0 - 1) * (int)p.c_row + kRowBytes;
    const auto krs = rows_rsrc(p.k + wbase, span);
    const auto vrs = rows_rsrc(p.v + wbase, span);
    const int loff = (t_begin - t0 + tg) * (int)p.c_row + dc * 16;
    auto bload = [&](__amdgpu_buffer_rsrc_t rs, int j) {
      const auto r = __builtin_amdgcn_raw_buffer_load_b128(rs, loff + j * TPS * (int)p.c_row, 0, 0);
      return make_uint4(r[0], r[1], r[2], r[3]);
    };
    auto kload = [&](uint4* dst, int g) {
#pragma unroll
      for (int i = 0; i < kSLoadGroup; ++i) dst[i] = bload(krs, g * kSLoadGroup + i);
    };
    uint4 vw[2][kSLoadGroup];
    auto vload = [&](uint4* dst, int g) {
#pragma unroll
      for (int i = 0; i < kSLoadGroup; ++i) dst[i] = bload(vrs, g * kSLoadGroup + i);
    };
    kload(kw[0], 0);
    if constexpr (BLOCK_SCALE && kBal) {
      const int b0 = t_begin / p.kv_block;
      const int b1 = min(b0 + 1, p.nkblk - 1);
      dnd = (b0 + 1) * p.kv_block - (t_begin + tg);
      const float sk0 = load_scale(p.ks, sbase + b0, p.kv_scale_f16);
      const float sk1 = load_scale(p.ks, sbase + b1, p.kv_scale_f16);
      const float sv0 = load_scale(p.vs, sbase + b0, p.kv_scale_f16);
      const float sv1 = load_scale(p.vs, sbase + b1, p.kv_scale_f16);
      csk0 = p.scale_log2 * sk0;
      csk1 = p.scale_log2 * sk1;
      sv_ref = fmaxf(fabsf(sv0), fabsf(sv1));
      const float inv = sv_ref > 0.0f ? 1.0f / sv_ref : 0.0f;
      rv0 = sv0 * inv;
      rv1 = sv1 * inv;
    } else if constexpr (BLOCK_SCALE) {
      csk0 = p.scale_log2 * load_scale(p.ks, sbase + t_begin / p.kv_block, p.kv_scale_f16);
      sv_ref = load_scale(p.vs, sbase + t_begin / p.kv_block, p.kv_scale_f16);
    }
    prep_q();
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      if (g + 1 < NG) kload(kw[(g + 1) & 1], g + 1);
      else vload(vw[0], 0);  // first V group, in flight while the last keys are scored
#pragma unroll
      for (int i = 0; i < kSLoadGroup; ++i) {
        const int j = g * kSLoadGroup + i;
        const uint4 w = kw[g & 1][i];
        float acc;
        if constexpr (QF16) {
          f16x2 kh[EPL / 2];
          if constexpr (INT4) {
            // Channel pairs (8i + s, 8i + s + 4) as fp16 1032 + code, exact;
            // the 1032 * sum(q) this adds is removed once per token below.
            const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
              for (int sft = 0; sft < 4; ++sft)
                kh[4 * i + sft] = __builtin_bit_cast(f16x2, i4_pair_bits(ww[i] >> (4 * sft)));
          } else {
            i8x4_to_h(w.x, kh[0], kh[1]);
            i8x4_to_h(w.y, kh[2], kh[3]);
            i8x4_to_h(w.z, kh[4], kh[5]);
            i8x4_to_h(w.w, kh[6], kh[7]);
          }
          float a0 = 0.0f, a1 = 0.0f;
#pragma unroll
          for (int e = 0; e < EPL / 2; e += 2) {
            a0 = __builtin_amdgcn_fdot2(qh[e], kh[e], a0, false);
            a1 = __builtin_amdgcn_fdot2(qh[e + 1], kh[e + 1], a1, false);
          }
          acc = a0 + a1;
          if constexpr (INT4) acc = __builtin_fmaf(-1032.0f, qsum, acc);
        } else {
          float f[EPL];
          chunk_to_f32<INT4>(w, f);
          acc = -kOff * qsum;
#pragma unroll
          for (int e = 0; e < EPL; ++e) acc = __builtin_fmaf(qf[e], f[e], acc);
        }
        acc = lane_group_sum<LPT>(acc);
        const int t = t_begin + j * TPS + tg;
        float c;
        if constexpr (BLOCK_SCALE && kBal) {
          c = j * TPS < dnd ? csk0 : csk1;
        } else if constexpr (BLOCK_SCALE) {
          c = csk0;
        } else {
          c = p.scale_log2 * load_scale(p.ks, sbase + min(t, t_last) / p.kv_block, p.kv_scale_f16);
        }
        sc[j] = t < t_end ? acc * c : -INFINITY;
        m_blk = fmaxf(m_blk, sc[j]);
      }
    }
#pragma unroll
    for (int off = LPT; off < 64; off <<= 1) m_blk = fmaxf(m_blk, __shfl_xor(m_blk, off));

    // ---- values ----
    float lp[2] = {0.0f, 0.0f};
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      if (g + 1 < NG) vload(vw[(g + 1) & 1], g + 1);
      if constexpr (kI4H) {
        // Two tokens at a time: each channel's codes of tokens j and j + 1
        // form one fp16 pair (1032 + code), dotted with the two weights in
        // fp16; the sums of those same fp16 weights remove the offset.
        static_assert(kSLoadGroup % 2 == 0, "token pairs");
        const f16x2 one = {(_Float16)1.0f, (_Float16)1.0f};
#pragma unroll
        for (int i = 0; i < kSLoadGroup; i += 2) {
          const int j = g * kSLoadGroup + i;
          const float pa = __builtin_amdgcn_exp2f(sc[j] - m_blk);  // 0 for masked tokens
          const float pb = __builtin_amdgcn_exp2f(sc[j + 1] - m_blk);
          float wa = pa, wb = pb;
          if constexpr (!BLOCK_SCALE) {
            const int ta = min(t_begin + j * TPS + tg, t_last);
            const int tb = min(t_begin + (j + 1) * TPS + tg, t_last);
            wa *= load_scale(p.vs, sbase + ta / p.kv_block, p.kv_scale_f16);
            wb *= load_scale(p.vs, sbase + tb / p.kv_block, p.kv_scale_f16);
          }
          const f16x2 wp = {(_Float16)wa, (_Float16)wb};
          if constexpr (BLOCK_SCALE) {
            lp[(i >> 1) & 1] = __builtin_amdgcn_fdot2(wp, one, lp[(i >> 1) & 1], false);
          } else {
            lp[(i >> 1) & 1] += pa + pb;
            wsum = __builtin_amdgcn_fdot2(wp, one, wsum, false);
          }
          const uint4 va = vw[g & 1][i], vb = vw[g & 1][i + 1];
          const uint32_t wa4[4] = {va.x, va.y, va.z, va.w}, wb4[4] = {vb.x, vb.y, vb.z, vb.w};
#pragma unroll
          for (int d = 0; d < 4; ++d) {
            // Bytes 0-1 (2-3) of token j then of token j + 1: channel 8d + c
            // (8d + 4 + c) sits in bits 0-3 (token j) and 16-19 (token j + 1)
            // after a shift.
            const uint32_t r0 = __builtin_amdgcn_perm(wb4[d], wa4[d], 0x05040100u);
            const uint32_t r1 = __builtin_amdgcn_perm(wb4[d], wa4[d], 0x07060302u);
#pragma unroll
            for (int c = 0; c < 4; ++c) {
              const uint32_t sft = (c & 1) * 4 + (c >> 1) * 8;
              o[8 * d + c] = __builtin_amdgcn_fdot2(
                  wp, __builtin_bit_cast(f16x2, i4_pair_bits(r0 >> sft)), o[8 * d + c], false);
              o[8 * d + 4 + c] = __builtin_amdgcn_fdot2(
                  wp, __builtin_bit_cast(f16x2, i4_pair_bits(r1 >> sft)), o[8 * d + 4 + c], false);
            }
          }
        }
      } else {
#pragma unroll
        for (int i = 0; i < kSLoadGroup; ++i) {
          const int j = g * kSLoadGroup + i;
          const float pr = __builtin_amdgcn_exp2f(sc[j] - m_blk);  // 0 for masked tokens
          lp[i & 1] += pr;
          float wt = pr;
          if constexpr (BLOCK_SCALE && kBal) {
            wt *= j * TPS < dnd ? rv0 : rv1;
          } else if constexpr (!BLOCK_SCALE) {
            const int t = min(t_begin + j * TPS + tg, t_last);
            wt *= load_scale(p.vs, sbase + t / p.kv_block, p.kv_scale_f16);
          }
          wsum += wt;
          float f[EPL];
          chunk_to_f32<INT4>(vw[g & 1][i], f);
#pragma unroll
          for (int e = 0; e < EPL; ++e) o[e] = __builtin_fmaf(wt, f[e], o[e]);
        }
      }
    }
    l_blk = lp[0] + lp[1];
    if constexpr (kI4H && BLOCK_SCALE) wsum = l_blk;
    // Sum the token groups: lanes with the same channel chunk.
#pragma unroll
    for (int off = LPT; off < 64; off <<= 1) {
      l_blk += __shfl_xor(l_blk, off);
      wsum += __shfl_xor(wsum, off);
    }
    sum_scatter<LPT, EPL>(o, lane);
    constexpr float kOffV = kI4H ? 1032.0f : kOff;
#pragma unroll
    for (int e = 0; e < NF; ++e) o[e] = (o[e] - kOffV * wsum) * sv_ref;
  }

  // Merge the wavefronts of the workgroup.
  if (lane == 0) {
    red_m[wave] = m_blk;
    red_l[wave] = l_blk;
  }
  {
    const int base = scatter_base<LPT, EPL>(lane);
#pragma unroll
    for (int e = 0; e < NF; ++e) red_o[wave][d0 + base + e] = o[e];
  }
  __syncthreads();
  if (wave != 0) return;
  float M = red_m[0];
#pragma unroll
  for (int w = 1; w < kSWaves; ++w) M = fmaxf(M, red_m[w]);
  float c[kSWaves];
  float Lsum = 0.0f;
#pragma unroll
  for (int w = 0; w < kSWaves; ++w) {
    c[w] = red_m[w] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(red_m[w] - M);
    Lsum += red_l[w] * c[w];
  }
  const long obase = (long)b * p.q_batch + (long)h * p.q_head;
  if (nsplit == 1) {
    const float inv = 1.0f / Lsum;
    for (int d = lane; d < D; d += 64) {
      float acc = 0.0f;
#pragma unroll
      for (int w = 0; w < kSWaves; ++w) acc += red_o[w][d] * c[w];
      store_out(p.out, obase + d, acc * inv, p.out_dtype);
    }
    return;
  }
  float* part = p.ws + (((long)b * p.Hq + h) * p.max_splits + split) * (D + 2);
  for (int d = lane; d < D; d += 64) {
    float acc = 0.0f;
#pragma unroll
    for (int w = 0; w < kSWaves; ++w) acc += red_o[w][d] * c[w];
    part[d] = acc;
  }
  if (lane == 0) {
    part[D] = M;
    part[D + 1] = Lsum;
  }
}

// Log-sum-exp merge of the chunk partials of one (batch, head) per wavefront.
// Lane s reads chunk s's (max, sum) for up to 64 chunks at a time, so those
// loads are issued together; the weighted sums then read each chunk's o with
// its weight taken from the lane that holds it.
template <int D>
__global__ __launch_bounds__(64) void decode_reduce_kernel(DecParams p) {
  const int h = blockIdx.x;
  const int b = blockIdx.y;
  const int lane = threadIdx.x;
  const int L = min(max(p.lens[b], 1), p.S_max);
  const int nsplit = p.all_splits ? p.max_splits : (L + kDecodeChunk - 1) / kDecodeChunk;
  if (nsplit <= 1) return;
  const float* part = p.ws + ((long)b * p.Hq + h) * p.max_splits * (D + 2);
  float M = -INFINITY;
  for (int s0 = 0; s0 < nsplit; s0 += 64)
    if (s0 + lane < nsplit) M = fmaxf(M, part[(s0 + lane) * (D + 2) + D]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
  float Lsum = 0.0f;
  float acc[D / 64];
#pragma unroll
  for (int i = 0; i < D / 64; ++i) acc[i] = 0.0f;
  for (int s0 = 0; s0 < nsplit; s0 += 64) {
    float c = 0.0f, lw = 0.0f;
    if (s0 + lane < nsplit) {
      const float* ps = part + (s0 + lane) * (D + 2);
      const float ms = ps[D];
      c = ms == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(ms - M);
      lw = ps[D + 1] * c;
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) lw += __shfl_xor(lw, off);
    Lsum += lw;
    // Four chunks per step, their loads issued together; past the last chunk
    // the index is clamped and the weight is zero (lanes >= n hold c = 0).
    const int n = min(64, nsplit - s0);
    for (int j = 0; j < n; j += 4) {
      float v[4][D / 64], cj[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float* ps = part + min(s0 + j + u, nsplit - 1) * (D + 2);
        cj[u] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(c), min(j + u, 63)));
#pragma unroll
        for (int i = 0; i < D / 64; ++i) v[u][i] = ps[lane + 64 * i];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int i = 0; i < D / 64; ++i) acc[i] += v[u][i] * cj[u];
    }
  }
  const float inv = 1.0f / Lsum;
  const long obase = (long)b * p.q_batch + (long)h * p.q_head;
#pragma unroll
  for (int i = 0; i < D / 64; ++i) store_out(p.out, obase + lane + 64 * i, acc[i] * inv, p.out_dtype);
}

template <int D, bool INT4, bool QF16, bool BS>
hipError_t launch_mha(const DecParams& p, int B, hipStream_t st) {
  decode_mha_kernel<D, INT4, QF16, BS><<<dim3(p.max_splits, p.Hq, B), 64 * kSWaves, 0, st>>>(p);
  return hipGetLastError();
}

template <int D, bool INT4, int QM, bool BS>
hipError_t launch_gqa(const DecParams& p, int B, hipStream_t st) {
  const dim3 grid(p.max_splits, p.Hkv, B);
  if (p.kv_scale_f16) decode_gqa_kernel<D, INT4, QM, BS, true><<<grid, 64 * kGWaves, 0, st>>>(p);
  else decode_gqa_kernel<D, INT4, QM, BS, false><<<grid, 64 * kGWaves, 0, st>>>(p);
  return hipGetLastError();
}

template <int D, bool INT4>
hipError_t launch_dec(const DecParams& p, int B, hipStream_t st) {
  hipError_t e;
  if (p.group == 1) {
    // Block scales: a wavefront's tokens (at most 128) span at most two blocks.
    const bool bs = p.kv_block % kSWaveTokens == 0;
    if (p.q_dtype == QFA_F16)
      e = bs ? launch_mha<D, INT4, true, true>(p, B, st) : launch_mha<D, INT4, true, false>(p, B, st);
    else
      e = bs ? launch_mha<D, INT4, false, true>(p, B, st) : launch_mha<D, INT4, false, false>(p, B, st);
  } else {
    // Block scales are uniform over a 32-token step (steps start at multiples of 32).
    const bool bs = p.kv_block % kStep == 0;
    if (p.q_dtype == QFA_F16)
      e = bs ? launch_gqa<D, INT4, Q_F16, true>(p, B, st) : launch_gqa<D, INT4, Q_F16, false>(p, B, st);
    else if (p.q_dtype == QFA_BF16)
      e = bs ? launch_gqa<D, INT4, Q_BF16, true>(p, B, st) : launch_gqa<D, INT4, Q_BF16, false>(p, B, st);
    else
      e = bs ? launch_gqa<D, INT4, Q_F32, true>(p, B, st) : launch_gqa<D, INT4, Q_F32, false>(p, B, st);
  }
  if (e != hipSuccess) return e;
  if (p.max_splits > 1) {
    decode_reduce_kernel<D><<<dim3(p.Hq, B), 64, 0, st>>>(p);
    e = hipGetLastError();
  }
  return e;
}

}  // namespace

hipError_t decode_scratch(hipStream_t stream, void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    // The symbol's address is per device: look it up with that device current.
    int cur = -1;
    e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) {
      const hipError_t r = hipSetDevice(cur);
      if (e == hipSuccess) e = r;
    }
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

size_t decode_workspace_bytes(int B, int Hq, int S_max, int D) {
  const long splits = (S_max + kDecodeChunk - 1) / kDecodeChunk;
  return (size_t)B * Hq * splits * (D + 2) * sizeof(float);
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
  DecParams p;
  p.q = a.q;
  p.k = (const uint8_t*)a.k;
  p.v = (const uint8_t*)a.v;
  p.ks = a.ks;
  p.vs = a.vs;
  p.lens = a.lens;
  p.out = a.out;
  p.ws = (float*)a.workspace;
  p.Hq = a.Hq;
  p.Hkv = a.Hkv;
  p.group = a.Hq / a.Hkv;
  p.S_max = a.S_max;
  p.max_splits = (a.S_max + kDecodeChunk - 1) / kDecodeChunk;
  const long rb = a.kv_qtype == QFA_INT4 ? a.D / 2 : a.D;
  const ix::Strides cs = ix::strides(a.layout == QFA_BSND, a.Hkv, a.S_max, rb);
  p.c_row = cs.row;
  p.c_head = cs.head;
  p.c_batch = cs.batch;
  p.q_head = a.D;
  p.q_batch = (long)a.Hq * a.D;
  p.kv_block = a.kv_block;
  p.nkblk = (a.S_max + a.kv_block - 1) / a.kv_block;
  p.kv_scale_f16 = a.kv_scale_dtype == QFA_F16;
  p.q_dtype = a.q_dtype;
  p.out_dtype = a.out_dtype;
  p.scale_log2 = a.softmax_scale * kLog2e;
  const bool int4 = a.kv_qtype == QFA_INT4;
  p.all_splits = p.group > 1 || !int4;
  if (a.D == 64) return int4 ? launch_dec<64, true>(p, a.B, stream) : launch_dec<64, false>(p, a.B, stream);
  return int4 ? launch_dec<128, true>(p, a.B, stream) : launch_dec<128, false>(p, a.B, stream);
}

}  // namespace qfa
