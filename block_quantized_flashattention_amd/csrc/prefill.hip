// Prefill attention forward on block-quantized codes (gfx950).
//
// What it computes ([Ascend-INT8] INT8-operator sections 1-2; [MindIE-SD] FA
// quantization, "FP8 Attention"; [FA-INT8/INT4] INT8 and INT4 layers):
//   x_ij = softmax_scale * sq_i * sk_j * (Qc_i . Kc_j)     low-bit dot, wide accumulation
//   o_i  = sum_j softmax_j(x_ij) * sv_j * Vc_j             online softmax, P.V on MFMA
//
// Design:
//   * A workgroup of 8 wavefronts (one per CU; 2 per SIMD) owns 256
//     (query row, query head) pairs of one (batch, KV head): hpw query heads
//     of the KV head (hpw = the largest power of two <= 8 dividing the GQA
//     group) times 256/hpw consecutive rows. Each wavefront owns 32 rows of
//     one head, and one staged K/V tile feeds all of them: under GQA every
//     K/V tile is loaded, unpacked and converted once for up to 8 heads.
//   * Two groups of four wavefronts, A (waves 0-3) and B (waves 4-7), run in
//     anti-phase, one of each on every SIMD: in each phase one group issues
//     the matrix work of a tile (S(t+1) = K Q^T and O += P(t) V(t)) while the
//     other computes a tile's softmax on the vector unit; a barrier ends each
//     phase and the groups swap. Matrix instructions of one wavefront run
//     concurrently with vector instructions of the other, so the matrix unit
//     and the vector unit are both kept busy rather than idling whenever the
//     two wavefronts of a SIMD happen to be in the same kind of work.
//   * The matrix-phase group also stages the next K and V tiles: codes are
//     loaded into registers two phases ahead and written to LDS (K as bytes,
//     INT4 as the offset codes code + 8 with the Q channels permuted to match
//     and the offset's share of the dot product taken off the accumulator's
//     start value; V transposed and converted exactly to fp16), and the next
//     tiles' loads are issued. The matrix-phase wavefront runs at a raised
//     issue priority.
//   * Scores are formed transposed, S^T = K . Q^T, with
//     v_mfma_i32_32x32x32_i8 (INT8 Q/K; INT4 K widened) or
//     v_mfma_f32_32x32x64_f8f6f4 (FP8 e4m3 Q/K). Each lane then holds one
//     query row and 16 of every 32 keys, so row max and row sum are register
//     reductions plus one exchange between the lane halves, and the fp16
//     probabilities land directly in the B-operand layout of
//     O^T += V^T . P^T on v_mfma_f32_32x32x16_f16: P never goes through LDS.
//   * Scale fold: with one K/V scale per tile, INT8 scores are read from an
//     integer accumulator started at a bit pattern that makes the sum a float
//     (see kBiasBits), and each probability costs one FMA and one exp2. O is
//     kept in units of the current V block scale and rescaled when it
//     changes. With per-key scales (INT4 K/V, one scale per token) the
//     integer dot product (read off the same biased accumulator with one
//     subtraction, exact) is multiplied by the key's scale
//     (staged beside the tile; each lane loads its 32 keys' scales into
//     registers at the end of its matrix phase), and the V scale goes into the
//     staged V: code * sv_j / sv_ref in fp16, sv_ref the running maximum V
//     scale, so O is kept in units of sv_ref.
//   * The running row max is raised only when a tile's max exceeds it by more
//     than the slack (log2 units), so the O rescale is skipped on most tiles;
//     the probabilities stay below 2^slack (exact softmax; fp16 holds them
//     with its full precision).
//   * Row sums add the fp16-rounded probabilities with v_dot2_f32_f16, i.e.
//     exactly the weights the P.V product uses.
//   * Causal: tiles past the workgroup's last row are never loaded (the
//     workgroup's wavefronts walk its tiles together; one whose rows all lie
//     above a tile masks all of its keys); the mask is a compile-time variant
//     used only on tiles that cross a wavefront's diagonal or the end of the
//     keys. Work is ordered longest first.
//   * XCD-aware order: workgroup ids are dealt round-robin to the 8 XCDs, so
//     all work of one (batch, KV head) runs on one XCD and its K/V codes stay
//     in that XCD's L2.
//   * fp8 P.V variant (e4m3 Q/K/V with block scales, qfa_fwd_lowp): V is
//     staged as raw e4m3 bytes in the operand's key order and the
//     probabilities are rounded to e4m3, one v_mfma_scale_f32_32x32x64_f8f6f4
//     per 32-channel block per tile. Each row also accumulates a bound on
//     sum p^2; a row with too few effective keys flags its work item, and the
//     same workgroup then recomputes the item with the fp16 product (the fp16
//     kernel's code), so only flagged items pay for the fallback and their
//     recomputation overlaps with the rest of the grid.
#include <type_traits>

#include "qfa_device.h"
#include "qfa_index.h"
#include "qfa_launch.h"

namespace qfa {
namespace {

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kPairs = ix::kFwdPairs;  // (row, head) pairs per workgroup
constexpr int kBN = ix::kFwdBN;        // keys per tile
constexpr int kScaleRing = 4;     // tiles of scales in flight (a power of two)
constexpr float kRescaleSlack = 12.0f;
// With per-key scales the fp16 weight is p * sv_j / sv_ref <= p; the smaller
// slack keeps the weights and their row sums well inside fp16.
constexpr float kRescaleSlackTok = 8.0f;
// fp8 P.V (e4m3 probabilities): a slack of 8 keeps them at most 256, below
// the format's 448.
constexpr float kRescaleSlackLp = 8.0f;
// fp8 P.V accuracy gate: a row keeps its fp8 result when its effective number
// of keys, bounded below by l^2 / S (S = sum over tiles of the tile's largest
// probability times the tile's sum, at least sum p^2), is at least this.
constexpr float kNeffMin = 256.0f;
// Bytes per staged e4m3 V^T row (64 keys and 16 bytes of padding).
constexpr int kV8Stride = 64 + 16;

struct FwdParams {
  const uint8_t* q;
  const void* qs;
  const uint8_t* k;
  const void* ks;
  const uint8_t* v;
  const void* vs;
  void* out;
  int B, Hq, Hkv, Sq, Sk, group;
  int hpw, rph, n_rb, n_hg;     // heads per workgroup, rows per head, row blocks, head groups
  long q_row, q_head, q_batch;  // byte strides of Q codes
  long k_row, k_head, k_batch;  // byte strides of K codes
  long v_row, v_head, v_batch;  // byte strides of V codes
  long o_row, o_head, o_batch;  // element strides of out
  int q_block, kv_block, nqblk, nkblk;
  int q_scale_f16, kv_scale_f16;
  int out_dtype;
  float scale_log2;  // softmax_scale * log2(e)
  int xcd_order;     // 1: XCD-grouped workgroup order
  // fp8 P.V forward: one byte per (workgroup, wavefront), 1 where a row
  // failed the accuracy gate. Unused by the fp16 forward.
  uint8_t* flags;
};

// LDS of one workgroup, as separate arrays so that the compiler can tell the
// buffers apart (a tile's operand reads and the next tile's staging writes
// then need no ordering): K tiles [64 keys][D + 16 pad] bytes; V tiles held
// transposed, [D][64 + 8 pad] fp16, keys permuted in groups of 16 (see vt_pos)
// so that each lane's MFMA operand is one 16-byte read; a ring of per-tile
// scales (K and V scale per key with per-key scales, else slot 0, and the V
// scale O is expressed in while the tile is processed); the fp16/bf16 output
// staged per wavefront for coalesced row stores.
template <int D>
struct Geo {
  static constexpr int kKStride = D + 16;
  static constexpr int kVStride = kBN + 8;
  static constexpr int kKBytes = kBN * kKStride;
  static constexpr int kVElems = D * kVStride;
  static constexpr int kOutStride = D + 8;
};
struct ScaleRing {
  float ks[kScaleRing][kBN];   // per key: K scale
  float vs[kScaleRing][kBN];   // per key: V scale / running maximum V scale
  float vref[kScaleRing];      // the V scale O is expressed in
};

// Position of key `key` (0..kBN-1) inside a staged V^T row: groups of 4 keys
// are reordered inside each group of 16 as [0-3, 8-11, 4-7, 12-15].
__device__ __forceinline__ int vt_pos(int key) {
  const int g = key >> 4, a = (key >> 2) & 3, i = key & 3;
  return g * 16 + ((((a & 1) << 1) | (a >> 1)) << 2) + i;
}

// Byte position of key `key` (0..63) in a staged e4m3 V^T row for the fp8
// P.V product: the 64 keys in the 32x32x64 operand's slot order, lane half h
// (key bit 2) holding slots 32h + 16 kb + 4 ((key >> 3) & 3) + (key & 3) with
// kb = key >> 5, the order in which a lane holds its scores.
__device__ __forceinline__ int vt8_pos(int key) {
  return 32 * ((key >> 2) & 1) + 16 * (key >> 5) + 4 * ((key >> 3) & 3) + (key & 3);
}

// Eight packed two's-complement nibbles of `w` (element 2k in the low nibble
// of byte k) as offset bytes, code + 8 in 0..15 (the nibble with its sign bit
// flipped): elements 0, 2, 4, 6 in the first dword, 1, 3, 5, 7 in the second.
// Staged K channels are therefore in the order [0 2 4 6 1 3 5 7] within every
// group of 8; the Q operand is permuted the same way (q_k4_order), and the
// offset adds 8 * sum(Q codes) to each dot product, which the accumulator's
// start value takes off again.
__device__ __forceinline__ uint2 unpack_int4x8_offset(uint32_t w) {
  const uint32_t lo = (w & 0x0F0F0F0Fu) ^ 0x08080808u;
  const uint32_t hi = ((w >> 4) & 0x0F0F0F0Fu) ^ 0x08080808u;
  return make_uint2(lo, hi);
}

// Q bytes of every group of 8 channels put in the order [0 2 4 6 1 3 5 7].
__device__ __forceinline__ i32x4 q_k4_order(i32x4 q) {
  const uint32_t a0 = q[0], a1 = q[1], b0 = q[2], b1 = q[3];
  return (i32x4){(int)__builtin_amdgcn_perm(a1, a0, 0x06040200u), (int)__builtin_amdgcn_perm(a1, a0, 0x07050301u),
                 (int)__builtin_amdgcn_perm(b1, b0, 0x06040200u), (int)__builtin_amdgcn_perm(b1, b0, 0x07050301u)};
}

// Bytes 0 and 1 of `u` (signed codes) as an exact fp16 pair: the byte with
// its sign bit flipped goes into the mantissa of 1024, and 1152 is subtracted.
__device__ __forceinline__ f16x2 i8pair_to_h(uint32_t u, uint32_t sel) {
  const f16x2 bias = {(_Float16)1152.0f, (_Float16)1152.0f};
  return __builtin_bit_cast(f16x2, __builtin_amdgcn_perm(0x64646464u, u ^ 0x80808080u, sel)) - bias;
}

// The nibbles at bits 0-3 and 16-19 of w (two's-complement codes) as an exact
// fp16 pair: flip the sign bit, place the nibbles under the exponent of 1024
// (1032 + code), subtract 1032.
__device__ __forceinline__ f16x2 i4pair_to_h(uint32_t w) {
  const f16x2 bias = {(_Float16)1032.0f, (_Float16)1032.0f};
  return __builtin_bit_cast(f16x2, ((w ^ 0x00080008u) & 0x000F000Fu) | 0x64006400u) - bias;
}

// Code types of K and V handled by one kernel instance.
enum KVMode { KV_I8_I8 = 0, KV_I4_I4 = 1, KV_I8_I4 = 2, KV_F8_F8 = 3 };
template <int M> struct KVTypes;
template <> struct KVTypes<KV_I8_I8> { static constexpr int K = QFA_INT8, V = QFA_INT8; };
template <> struct KVTypes<KV_I4_I4> { static constexpr int K = QFA_INT4, V = QFA_INT4; };
template <> struct KVTypes<KV_I8_I4> { static constexpr int K = QFA_INT8, V = QFA_INT4; };
template <> struct KVTypes<KV_F8_F8> { static constexpr int K = QFA_FP8_E4M3, V = QFA_FP8_E4M3; };

// Staging geometry (one unit per thread and tile):
//   K: key tid / 8, eighth tid % 8 of its row: D/8 staged bytes (D/16 source
//      bytes for INT4).
//   V: keys 2 (tid % 32) and 2 (tid % 32) + 1, channels (tid / 32) * D/16 +
//      [0, D/16): D/16 source bytes (D/32 for INT4) per key.
// Threads of group A (tid < 256) hold keys 0-31 of K and channels 0..D/2-1 of
// V; group B the rest, so each group stages half of every tile.
template <int D, int KQT, int VQT>
struct Stage {
  static constexpr int kKSrc = ix::fwd_k_src(D, KQT == QFA_INT4);  // bytes
  static constexpr int kVCh = D / 16;                               // channels per key
  static constexpr int kVSrc = ix::fwd_v_src(D, VQT == QFA_INT4);  // bytes per key
  uint32_t k[kKSrc / 4];
  uint32_t v[2][kVSrc / 4 > 0 ? kVSrc / 4 : 1];
};

template <int N>
__device__ __forceinline__ void load_words(uint32_t (&w)[N], const uint8_t* p) {
  if constexpr (N == 4) {
    const uint4 x = *(const uint4*)p;
    w[0] = x.x; w[1] = x.y; w[2] = x.z; w[3] = x.w;
  } else if constexpr (N == 2) {
    const uint2 x = *(const uint2*)p;
    w[0] = x.x; w[1] = x.y;
  } else {
    w[0] = *(const uint32_t*)p;
  }
}

// Issue the loads of this thread's K and V units of a tile. Keys past the end
// are clamped to the last key (finite codes, masked scores). Nothing reads the
// registers before the matching stage_tile, two phases later.
template <int D, int KQT, int VQT>
__device__ __forceinline__ void fetch_tile(Stage<D, KQT, VQT>& f, const FwdParams& p,
                                           const uint8_t* kbase, const uint8_t* vbase, int kn0,
                                           int vn0) {
  using S = Stage<D, KQT, VQT>;
  const int tid = threadIdx.x;
  load_words(f.k, kbase + ix::fwd_k_offset(ix::fwd_k_key(kn0, tid, p.Sk), (uint32_t)p.k_row, tid,
                                            S::kKSrc));
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const uint8_t* src = vbase + ix::fwd_v_offset(ix::fwd_v_key(vn0, tid, r, p.Sk),
                                                  (uint32_t)p.v_row, tid, S::kVSrc);
    if constexpr (S::kVSrc >= 4) {
      load_words(f.v[r], src);
    } else {
      f.v[r][0] = *(const uint16_t*)src;  // D = 64 INT4: 2 bytes per key
    }
  }
}

template <int D, int KQT, int VQT>
__device__ __forceinline__ void stage_k(uint8_t* kbuf, const Stage<D, KQT, VQT>& f) {
  const int tid = threadIdx.x;
  uint8_t* dst = kbuf + (tid / 8) * Geo<D>::kKStride + (tid % 8) * (D / 8);
  if constexpr (KQT == QFA_INT4) {
    if constexpr (D == 128) {
      const uint2 a = unpack_int4x8_offset(f.k[0]), b = unpack_int4x8_offset(f.k[1]);
      *(uint4*)dst = make_uint4(a.x, a.y, b.x, b.y);
    } else {
      const uint2 a = unpack_int4x8_offset(f.k[0]);
      *(uint2*)dst = a;
    }
  } else if constexpr (D == 128) {
    *(uint4*)dst = make_uint4(f.k[0], f.k[1], f.k[2], f.k[3]);
  } else {
    *(uint2*)dst = make_uint2(f.k[0], f.k[1]);
  }
}

// V^T: channel c of keys (2kp, 2kp+1) as one fp16 pair (exact for INT8, INT4
// and e4m3 codes).
// With per-key scales (vsn != nullptr) each key's values are multiplied by
// its V scale over the running maximum V scale, vsn[key] <= 1, in fp16.
template <int D, int KQT, int VQT>
__device__ __forceinline__ void stage_v(_Float16* vbuf, const Stage<D, KQT, VQT>& f,
                                        const float* vsn) {
  using S = Stage<D, KQT, VQT>;
  const int tid = threadIdx.x;
  const int kp = tid % 32, cg = tid / 32;
  _Float16* base = vbuf + (cg * S::kVCh) * Geo<D>::kVStride + vt_pos(2 * kp);
  f16x2 vscale = {(_Float16)1.0f, (_Float16)1.0f};
  if (vsn) {
    const f32x2 v2 = *(const f32x2*)(vsn + 2 * kp);
    vscale = (f16x2){(_Float16)v2[0], (_Float16)v2[1]};
  }
  auto put = [&](int c, f16x2 h) __attribute__((always_inline)) {
    if (vsn) h = h * vscale;
    *(f16x2*)(base + c * Geo<D>::kVStride) = h;
  };
  if constexpr (VQT == QFA_INT4) {
    // Nibble c of key a (b) sits in byte c/2 of its word(s). Bytes j, j+1 of
    // both keys are gathered (a in bits 0-15, b in 16-31). With its sign bit
    // flipped a nibble is code + 8; a low nibble (bits 0-3) goes under the
    // fp16 exponent of 1024 (1032 + code), a high nibble stays in bits 4-7,
    // the mantissa bits of weight 1 under the exponent of 64 (72 + code):
    // both exact, no shift for the high nibble.
    const f16x2 b_lo = {(_Float16)1032.0f, (_Float16)1032.0f};
    const f16x2 b_hi = {(_Float16)72.0f, (_Float16)72.0f};
    auto lo_h = [&](uint32_t w) __attribute__((always_inline)) {
      return __builtin_bit_cast(f16x2, ((w ^ 0x00080008u) & 0x000F000Fu) | 0x64006400u) - b_lo;
    };
    auto hi_h = [&](uint32_t w) __attribute__((always_inline)) {
      return __builtin_bit_cast(f16x2, ((w ^ 0x00800080u) & 0x00F000F0u) | 0x54005400u) - b_hi;
    };
#pragma unroll
    for (int w = 0; w < (S::kVSrc + 3) / 4; ++w) {
      const uint32_t a = f.v[0][w], b = f.v[1][w];
#pragma unroll
      for (int j = 0; j < (S::kVSrc >= 4 ? 4 : S::kVSrc); j += 2) {
        // bytes j, j+1 of a in bytes 0-1, of b in bytes 2-3
        const uint32_t sel = (j == 0) ? 0x05040100u : 0x07060302u;
        const uint32_t u = __builtin_amdgcn_perm(b, a, sel);
        const uint32_t u8 = u >> 8;  // byte j+1 of each key in the low byte
        const int c0 = 8 * w + 2 * j;
        put(c0 + 0, lo_h(u));
        put(c0 + 1, hi_h(u));
        put(c0 + 2, lo_h(u8));
        put(c0 + 3, hi_h(u8));
      }
    }
  } else if constexpr (VQT == QFA_FP8_E4M3) {
#pragma unroll
    for (int w = 0; w < S::kVSrc / 4; ++w) {
      const uint32_t a = f.v[0][w], b = f.v[1][w];
      const uint32_t lo = __builtin_amdgcn_perm(b, a, 0x05010400u);  // a0 b0 a1 b1
      const uint32_t hi = __builtin_amdgcn_perm(b, a, 0x07030602u);  // a2 b2 a3 b3
      put(4 * w + 0, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, false));
      put(4 * w + 1, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, true));
      put(4 * w + 2, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, false));
      put(4 * w + 3, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, true));
    }
  } else {
#pragma unroll
    for (int w = 0; w < S::kVSrc / 4; ++w) {
      const uint32_t a = f.v[0][w], b = f.v[1][w];
      const uint32_t lo = __builtin_amdgcn_perm(b, a, 0x05010400u);  // a0 b0 a1 b1
      const uint32_t hi = __builtin_amdgcn_perm(b, a, 0x07030602u);  // a2 b2 a3 b3
      put(4 * w + 0, i8pair_to_h(lo, 0x05010400u));
      put(4 * w + 1, i8pair_to_h(lo, 0x07030602u));
      put(4 * w + 2, i8pair_to_h(hi, 0x05010400u));
      put(4 * w + 3, i8pair_to_h(hi, 0x07030602u));
    }
  }
}

// e4m3 V^T for the fp8 P.V product: the raw codes of keys (2kp, 2kp+1),
// which sit at adjacent positions, as one 2-byte write per channel.
template <int D, int KQT, int VQT>
__device__ __forceinline__ void stage_v8(uint8_t* vbuf, const Stage<D, KQT, VQT>& f) {
  using S = Stage<D, KQT, VQT>;
  static_assert(VQT == QFA_FP8_E4M3, "fp8 P.V takes e4m3 V");
  const int tid = threadIdx.x;
  const int kp = tid % 32, cg = tid / 32;
  uint8_t* base = vbuf + (cg * S::kVCh) * kV8Stride + vt8_pos(2 * kp);
#pragma unroll
  for (int w = 0; w < S::kVSrc / 4; ++w) {
    const uint32_t a = f.v[0][w], b = f.v[1][w];
    const uint32_t lo = __builtin_amdgcn_perm(b, a, 0x05010400u);  // a0 b0 a1 b1
    const uint32_t hi = __builtin_amdgcn_perm(b, a, 0x07030602u);  // a2 b2 a3 b3
    *(uint16_t*)(base + (4 * w + 0) * kV8Stride) = (uint16_t)lo;
    *(uint16_t*)(base + (4 * w + 1) * kV8Stride) = (uint16_t)(lo >> 16);
    *(uint16_t*)(base + (4 * w + 2) * kV8Stride) = (uint16_t)hi;
    *(uint16_t*)(base + (4 * w + 3) * kV8Stride) = (uint16_t)(hi >> 16);
  }
}

// Scales of one tile, handled by wavefront 0 (lane = key): loaded a tile
// ahead, then written to the ring slot of the tile. With per-key scales the V
// scales are divided by the running maximum V scale `vref` (carried by the
// wavefront across tiles), which is also stored for the tile.
// The raw bits of this lane's K and V scale (fp16: the low half; fp32: both
// halves). They are converted only when staged, a tile later: converting
// them at load time would make the wavefront wait for the load.
struct ScaleRegs {
  uint32_t klo, khi, vlo, vhi;
};

__device__ __forceinline__ void fetch_scales(ScaleRegs& r, const FwdParams& p, long sbase, int n0,
                                             bool tok) {
  // The block relative to the (batch, KV head)'s first, as a 32-bit offset
  // from a uniform base.
  const long g = ix::fwd_kv_scale_block(0, n0, (int)(threadIdx.x & 63), p.Sk, p.kv_block, tok);
  // Two 16-bit loads per scale, neither past the scale's own bytes.
  long i0, i1;
  ix::scale_halves(g, p.kv_scale_f16, i0, i1);
  const long base = 2 * (p.kv_scale_f16 ? sbase : 2 * sbase);  // bytes
  const uint8_t* ks = (const uint8_t*)p.ks + base;
  const uint8_t* vs = (const uint8_t*)p.vs + base;
  const uint32_t o0 = 2 * (uint32_t)i0, o1 = 2 * (uint32_t)i1;
  r.klo = *(const uint16_t*)(ks + o0);
  r.khi = *(const uint16_t*)(ks + o1);
  r.vlo = *(const uint16_t*)(vs + o0);
  r.vhi = *(const uint16_t*)(vs + o1);
}

// Largest |v| over the wavefront, in every lane. Magnitudes of floats order
// as their bit patterns, so the maximum is taken on integers: DPP exchanges
// inside each row of 16 lanes (lane i ^ 1, i ^ 2, then the mirrored lane of
// its 8 and of its 16), then the four row results read as scalars. No LDS
// round trip.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, 0xF, 0xF, false);
}
__device__ __forceinline__ float wave_max_abs(float v) {
  uint32_t m = __float_as_uint(v) & 0x7FFFFFFFu;
  m = max(m, dpp_u32<0xB1>(m));   // quad_perm [1, 0, 3, 2]
  m = max(m, dpp_u32<0x4E>(m));   // quad_perm [2, 3, 0, 1]
  m = max(m, dpp_u32<0x141>(m));  // row_half_mirror
  m = max(m, dpp_u32<0x140>(m));  // row_mirror
  const uint32_t r0 = __builtin_amdgcn_readlane(m, 0), r1 = __builtin_amdgcn_readlane(m, 16);
  const uint32_t r2 = __builtin_amdgcn_readlane(m, 32), r3 = __builtin_amdgcn_readlane(m, 48);
  return __uint_as_float(max(max(r0, r1), max(r2, r3)));
}

// With per-key scales each key's K scale is staged (the score is the dot
// product times it) and its V scale as the ratio to the running maximum V
// scale; with block scales the tile's K scale and V scale.
template <bool TOK>
__device__ __forceinline__ void stage_scales(ScaleRing& sm, int slot, const ScaleRegs& r,
                                             bool f16, float& vref_run) {
  const int lane = threadIdx.x & 63;
  const float ks = f16 ? f16_bits_to_f32(r.klo) : __uint_as_float(r.klo | (r.khi << 16));
  const float vs = f16 ? f16_bits_to_f32(r.vlo) : __uint_as_float(r.vlo | (r.vhi << 16));
  if constexpr (TOK) {
    sm.ks[slot][lane] = ks;
    // V scales are magnitudes (amax / qmax); the largest |scale| keeps every
    // ratio within [-1, 1] whatever the caller passes.
    vref_run = fmaxf(vref_run, wave_max_abs(vs));
    // The ratio goes into fp16 (the staged V), so the hardware reciprocal
    // (1 ulp) is ample.
    sm.vs[slot][lane] = vref_run > 0.0f ? vs * __builtin_amdgcn_rcpf(vref_run) : 0.0f;
    if (lane == 0) sm.vref[slot] = vref_run;
  } else {
    sm.ks[slot][lane] = ks;
    if (lane == 0) sm.vref[slot] = vs;
  }
}

template <int D, bool FP8>
struct QK {
  static constexpr int kSlice = FP8 ? 32 : 16;  // operand bytes per lane per MFMA
  static constexpr int kSteps = D / (2 * kSlice);
  typedef typename std::conditional<FP8, i32x8, i32x4>::type Op;
  typedef typename std::conditional<FP8, f32x16, i32x16>::type Acc;
  static __device__ __forceinline__ Acc mma(const Op& a, const Op& b, const Acc& c) {
    if constexpr (FP8) {
      return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
    } else {
      return __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c, 0, 0, 0);
    }
  }
  static __device__ __forceinline__ Op load(const uint8_t* p) {
    if constexpr (FP8) {
      const i32x4 lo = *(const i32x4*)p;
      const i32x4 hi = *(const i32x4*)(p + 16);
      return (i32x8){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    } else {
      return *(const i32x4*)p;
    }
  }
};

// Key offset (within the tile) of accumulator register r of 32-key block kb
// for lane half 0 (lane half 1 holds keys 4 further): MFMA 32x32 result rows
// 8*(r/4) + 4*half + r%4.
__device__ __forceinline__ constexpr int key_of(int kb, int r) { return kb * 32 + 8 * (r >> 2) + (r & 3); }

// One work item of the forward, computed by the whole workgroup in the LDS
// buffers passed in. LPV: P.V on the fp8 matrix unit (e4m3 V and
// probabilities, block scales only), with the per-row accuracy gate written to
// p.flags; returns true, without writing any output, when a row of the work
// item failed the gate. The fp16 path writes the output and returns false.
template <int D, int KVM, bool CAUSAL, bool TOK, bool LPV>
__device__ __forceinline__ bool fwd_item(const FwdParams& p, uint8_t* kbuf0, uint8_t* kbuf1,
                                         _Float16* vbuf0, _Float16* vbuf1, ScaleRing& sc,
                                         uint16_t* obuf) {
  constexpr bool FP8 = KVM == KV_F8_F8;
  static_assert(!LPV || (FP8 && !TOK), "fp8 P.V: e4m3 V with block scales");
  constexpr int KQT = KVTypes<KVM>::K, VQT = KVTypes<KVM>::V;
  constexpr bool kK4 = KQT == QFA_INT4;  // K staged as offset codes (unpack_int4x8_offset)
  using T = QK<D, FP8>;
  using Op = typename T::Op;
  using Acc = typename T::Acc;
  using St = Stage<D, KQT, VQT>;
  using G = Geo<D>;
  constexpr int kDB = D / 32;  // 32-channel blocks of the output
  constexpr int kNK = 2 * T::kSteps;  // K operand reads (and QK MFMAs) per tile
  constexpr int kNV = LPV ? kDB : 4 * kDB;  // PV MFMAs per tile
  constexpr int kVR = LPV ? 2 : 1;          // 16-byte V operand reads per PV MFMA
  // INT8 scores with one scale per tile: the integer accumulator starts at
  // the bit pattern kBiasBits of the float kBiasInt * 2^-26, so
  // 'kBiasBits + dot' is the bit pattern of the float (kBiasInt + dot) * 2^-26
  // exactly as long as the sum stays in that binade, i.e.
  // -2292099 <= dot < 6096509, which any 8-bit codes with D <= 128 satisfy
  // (|dot| <= 128 * 128 * 128). The scores then need no integer-to-float
  // conversion, and their max is a float max. With per-key scales each score
  // is multiplied by its key's scale anyway: the accumulator starts at the
  // same bias and x - kBiasInt 2^-26 = dot 2^-26 (exact, one subtraction,
  // cheaper than an integer-to-float conversion) is scaled by the key's
  // scale, the 2^26 going into the row's factor: one constant per key
  // instead of two.
  constexpr bool kBiasAcc = !FP8 && !TOK;
  // INT8 products start from bias_acc (the float bias and/or the INT4 K
  // offset correction); otherwise from zero.
  constexpr bool kTokBias = !FP8 && TOK;  // per-key scales on the biased accumulator
  constexpr bool kStartAcc = kBiasAcc || kK4 || kTokBias;
  constexpr uint32_t kBiasBits = 0x3E22F983u;
  constexpr int kBiasInt = 10680707;  // 2^23 + 0x22F983
  static_assert(D <= 128, "biased INT8 scores need |dot| < 2^21");
  constexpr float kSlack = TOK ? kRescaleSlackTok : (LPV ? kRescaleSlackLp : kRescaleSlack);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int grp = wave >> 2;   // 0: group A, 1: group B
  const int half = lane >> 5;  // lane half: keys 4*half + {0..3} of every 8
  const int col = lane & 31;   // query row of this lane within the wavefront

  // Work item: (batch, KV head, head group, row block).
  const ix::FwdItem it = ix::fwd_item(blockIdx.x, p.B, p.Hkv, p.n_hg, p.n_rb, p.xcd_order, CAUSAL);
  const int b = it.b, kvh = it.kvh;
  const int h = ix::fwd_head(it, p.group, p.hpw, wave);
  const int m0 = it.rb * p.rph;
  const int qrow = ix::fwd_row(it, p.rph, p.hpw, wave, lane);
  const int wrow0 = qrow - col;
  const bool qvalid = qrow < p.Sq;

  // Q slice of this lane (B operand of S^T = K . Q^T), kept in registers.
  Op qop[T::kSteps];
  {
    const uint8_t* qp = p.q + (long)b * p.q_batch + (long)h * p.q_head + (long)ix::fwd_read_row(qrow, p.Sq) * p.q_row;
#pragma unroll
    for (int s = 0; s < T::kSteps; ++s) {
      qop[s] = T::load(qp + s * 2 * T::kSlice + half * T::kSlice);
      if (!qvalid) qop[s] = (Op){};
      if constexpr (kK4) qop[s] = q_k4_order(qop[s]);
    }
  }
  const float sq = load_scale(p.qs, ((long)b * p.Hq + h) * p.nqblk + ix::fwd_read_row(qrow, p.Sq) / p.q_block,
                              p.q_scale_f16);
  const float cq = qvalid ? sq * p.scale_log2 : 0.0f;

  const uint8_t* kbase = p.k + (long)b * p.k_batch + (long)kvh * p.k_head;
  const uint8_t* vbase = p.v + (long)b * p.v_batch + (long)kvh * p.v_head;
  const long sbase = ((long)b * p.Hkv + kvh) * p.nkblk;

  // The accumulator start of the INT8 scores, kept in registers (an opaque
  // copy, so the compiler does not rebuild the splat for every use): the
  // float bias with block scales, and with offset INT4 K codes minus
  // 8 * (sum of the row's Q codes over both lane halves).
  int bias0 = (kBiasAcc || kTokBias) ? (int)kBiasBits : 0;
  if constexpr (kK4) {
    int qsum = 0;
#pragma unroll
    for (int s = 0; s < T::kSteps; ++s)
#pragma unroll
      for (int i = 0; i < 4; ++i) qsum = __builtin_amdgcn_sdot4(qop[s][i], 0x01010101, qsum, false);
    qsum += __shfl_xor(qsum, 32);
    bias0 -= 8 * qsum;
  }
  i32x16 bias_acc;
#pragma unroll
  for (int i = 0; i < 16; ++i) bias_acc[i] = bias0;
  if constexpr (kStartAcc) asm volatile("" : "+v"(bias_acc));

  f32x16 o[kDB];
#pragma unroll
  for (int i = 0; i < kDB; ++i) o[i] = (f32x16){};
  float m_run = -INFINITY;  // reference row max (log2 units)
  float l_run = 0.0f;       // row sum of this lane half, in units of exp2(-m_run)
  float s_run = 0.0f;       // (fp8 P.V) sum over tiles of max p times the tile's sum, units exp2(-2 m_run)
  float sv_cur = 0.0f;      // V scale O is expressed in
  float vref_run = 0.0f;    // (wavefront 0, per-key scales) running max V scale

  const int n_end = ix::fwd_key_end(CAUSAL, p.Sk, m0, p.rph);
  const int ntiles = ix::fwd_tiles(n_end);
  const int last_tile = ntiles - 1;
  // Keys beyond this offset from the tile start are masked for this lane.
  const int lim_base = (CAUSAL ? min(qrow, p.Sk - 1) : p.Sk - 1) - 4 * half;
  auto tile_n0 = [&](int t) __attribute__((always_inline)) { return ix::fwd_tile_n0(t, last_tile); };

  Acc sacc[2];
  f16x8 pb[2][2];  // P^T operand: [32-key block][16-key half]
  uint32_t pb8[8];  // fp8 P.V: the P^T operand, 32 e4m3 probabilities (slot 4w + byte)
  St pf;
  ScaleRegs sr;
  // Uniform scales of the tile whose softmax comes next, read during the
  // preceding matrix phase (a read at the start of the softmax phase would
  // queue behind the other group's operand reads).
  float tile_ks = 0.0f, tile_vref = 0.0f;
  // K scales of this lane's 32 keys of that tile (per-key scales), read at
  // the end of the matrix phase: read in the softmax phase they would wait
  // behind the other group's operand reads.
  f32x4 key_s[2][4];

  // Matrix phase for tile index t, with K_t in kb and V_{t-1} in vb (PV when
  // the template flag says so): operand reads, the staging of the registers
  // fetched two phases ago (K_{t+1} into kst, V_t into vst, scales of tile t+1
  // into the ring) and the loads of the next tiles, then S(t) = K_t Q^T and
  // O += P(t-1) V(t-1). Staging and loads happen unconditionally: past the
  // last tile they rewrite buffers nobody reads again with clamped tiles.
  auto mphase = [&](int t, const uint8_t* kb, const _Float16* vb, uint8_t* kst, _Float16* vst,
                    auto with_pv) __attribute__((always_inline)) {
    constexpr bool PV = decltype(with_pv)::value;
    // Operand stream: kNR 16-byte LDS reads (K operands, then V operands),
    // kNM matrix instructions. A ring of kDepth registers keeps kDepth reads
    // in flight ahead of the instruction that consumes them; the order is
    // pinned with scheduling fences so that each read has several matrix
    // instructions' time to arrive.
    constexpr int kKR = FP8 ? 2 : 1;              // reads per QK instruction
    constexpr int kNR = kKR * kNK + (PV ? kVR * kNV : 0);
    constexpr int kNM = kNK + (PV ? kNV : 0);
    constexpr int kDepth = 8;
    tile_ks = sc.ks[t % kScaleRing][0];
    tile_vref = sc.vref[t % kScaleRing];
    const uint8_t* kaddr = kb + col * G::kKStride + half * T::kSlice;
    const _Float16* vaddr = vb + col * G::kVStride + half * 8;
    const uint8_t* vaddr8 = (const uint8_t*)vb + col * kV8Stride + half * 32;
    // P.V comes first, so that the probabilities are dead before the new
    // scores are written (the two can share registers). Read r: V operands
    // (16-key group-major), then K operands in MFMA order (step-major, the
    // two 32-key blocks interleaved).
    constexpr int kNVM = PV ? kNV : 0;    // PV instructions
    constexpr int kNVR = kVR * kNVM;      // their reads
    auto rd = [&](int r) __attribute__((always_inline)) -> i32x4 {
      if (r < kNVR) {
        if constexpr (LPV) {
          // rows of 32 channels, lane half h: bytes [32h, 32h + 32)
          const int db = r / 2, part = r % 2;
          return *(const i32x4*)(vaddr8 + db * 32 * kV8Stride + part * 16);
        }
        const int g = r / kDB, db = r % kDB;
        return *(const i32x4*)(vaddr + db * 32 * G::kVStride + g * 16);
      }
      const int m = (r - kNVR) / kKR, part = (r - kNVR) % kKR;
      const int s = m / 2, kb2 = m % 2;
      return *(const i32x4*)(kaddr + kb2 * 32 * G::kKStride + s * 2 * T::kSlice + part * 16);
    };
    i32x4 ring[kDepth];
#pragma unroll
    for (int r = 0; r < kDepth; ++r) ring[r] = rd(r);
    __builtin_amdgcn_sched_barrier(0);
    // Reads consumed by instructions 0..m.
    auto consumed = [](int m) constexpr {
      return m < kNVM ? (m + 1) * kVR : kNVR + (m + 1 - kNVM) * kKR;
    };
#pragma unroll
    for (int m = 0; m < kNM; ++m) {
      // first read of this instruction
      const int r0 = m < kNVM ? m * kVR : kNVR + (m - kNVM) * kKR;
      if (m < kNVM) {
        if constexpr (PV && LPV) {
          const i32x4 lo = ring[r0 % kDepth], hi = ring[(r0 + 1) % kDepth];
          const i32x8 va = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          const i32x8 pa = {(int)pb8[0], (int)pb8[1], (int)pb8[2], (int)pb8[3],
                            (int)pb8[4], (int)pb8[5], (int)pb8[6], (int)pb8[7]};
          o[m] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(va, pa, o[m], 0, 0, 0, 0, 0, 0);
        } else if constexpr (PV) {
          const int g = m / kDB, db = m % kDB;
          o[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, ring[r0 % kDepth]),
                                                         pb[g >> 1][g & 1], o[db], 0, 0, 0);
        }
      } else {
        const int s = (m - kNVM) / 2, kb2 = (m - kNVM) % 2;
        Op a;
        if constexpr (FP8) {
          const i32x4 lo = ring[r0 % kDepth], hi = ring[(r0 + 1) % kDepth];
          a = (Op){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        } else {
          a = ring[r0 % kDepth];
        }
        if (s == 0) {
          if constexpr (kStartAcc) sacc[kb2] = T::mma(a, qop[0], bias_acc);
          else sacc[kb2] = T::mma(a, qop[0], (Acc){});
        } else {
          sacc[kb2] = T::mma(a, qop[s], sacc[kb2]);
        }
      }
      // Refill the slots this instruction freed.
      const int from = min(kNR, kDepth + (m ? consumed(m - 1) : 0));
      const int to = min(kNR, kDepth + consumed(m));
#pragma unroll
      for (int r = from; r < to; ++r) ring[r % kDepth] = rd(r);
      if (m + 4 < kNM) __builtin_amdgcn_sched_barrier(0);
    }
    // Staging of the next tiles and their loads; the compiler may interleave
    // this vector work with the last matrix instructions.
    stage_k<D, KQT, VQT>(kst, pf);
    if constexpr (LPV) stage_v8<D, KQT, VQT>((uint8_t*)vst, pf);
    else stage_v<D, KQT, VQT>(vst, pf, TOK ? sc.vs[t % kScaleRing] : nullptr);
    if (wave == 0) stage_scales<TOK>(sc, (t + 1) % kScaleRing, sr, p.kv_scale_f16, vref_run);
    fetch_tile<D, KQT, VQT>(pf, p, kbase, vbase, tile_n0(t + 2), tile_n0(t + 1));
    if (wave == 0) fetch_scales(sr, p, sbase, tile_n0(t + 2), TOK);
    if constexpr (TOK) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int rg = 0; rg < 4; ++rg)
          key_s[kb][rg] = *(const f32x4*)(sc.ks[t % kScaleRing] + kb * 32 + 8 * rg + 4 * half);
    }
  };

  // Softmax of the scores of tile t (in sacc) into pb and the running
  // statistics; mask_c: compile-time switch for tiles that need the mask
  // (a wavefront whose rows all lie above the tile masks every key).
  auto softmax = [&](int t, auto mask_c) __attribute__((always_inline)) {
    constexpr bool MASK = decltype(mask_c)::value;
    const int lim = lim_base - t * kBN;  // masked iff key_of(kb, r) > lim
    const f16x2 one = {(_Float16)1.0f, (_Float16)1.0f};
    float ls[4] = {0.0f, 0.0f, 0.0f, 0.0f};  // independent partial row sums
    if constexpr (!TOK) {
      // A zero Q or K scale makes every score of the row 0; the floor keeps
      // -inf (masked) times the factor from giving NaN and changes no
      // probability at fp32 precision.
      const float ck = fmaxf(cq * tile_ks, 1e-30f);
      const float sv_t = tile_vref;
      float x[2][16];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          if constexpr (kBiasAcc) x[kb][r] = __int_as_float(sacc[kb][r]);
          else x[kb][r] = sacc[kb][r];
          // Causal: masked keys are real keys and must not raise the max.
          if constexpr (MASK && CAUSAL) x[kb][r] = key_of(kb, r) > lim ? -INFINITY : x[kb][r];
        }
      float mc[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mc[r & 3] = fmaxf(mc[r & 3], x[kb][r]);
      const float mx = fmaxf(fmaxf(mc[0], mc[1]), fmaxf(mc[2], mc[3]));
      // Max of this lane half in log2 units; (x - kBiasInt 2^-26) 2^26 is the
      // integer dot product, exactly.
      const float mt = mx == -INFINITY ? -INFINITY
                       : kBiasAcc ? (mx - __int_as_float(kBiasBits)) * (ck * 67108864.0f)
                                  : mx * ck;
      // A zero V scale (all-zero V block) keeps O's unit.
      const bool sv_change = sv_t > 0.0f && sv_t != sv_cur;
      if (__any(mt > m_run + kSlack) || sv_change) {
        const float mrow = fmaxf(mt, __shfl_xor(mt, 32));
        const float m_new = mrow > m_run + kSlack ? fmaxf(m_run, mrow) : m_run;
        const float alpha = (m_run == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(m_run - m_new);
        const float sv_new = sv_t > 0.0f ? sv_t : (sv_cur > 0.0f ? sv_cur : 1.0f);
        const float f = sv_cur > 0.0f ? alpha * (sv_cur / sv_new) : 0.0f;
        l_run *= alpha;
        if constexpr (LPV) s_run *= alpha * alpha;
#pragma unroll
        for (int i = 0; i < kDB; ++i) o[i] *= f;
        m_run = m_new;
        sv_cur = sv_new;
      }
      float msub = (m_run == -INFINITY) ? 0.0f : -m_run;
      float c = ck;
      if constexpr (kBiasAcc) {
        // x = (kBiasInt + dot) 2^-26: scale by ck 2^26 and fold the offset
        // into the subtrahend (one rounding, below one unit of dot).
        msub = __builtin_fmaf(-(float)kBiasInt, ck, msub);
        c = ck * 67108864.0f;
      }
      if constexpr (LPV) {
        // e4m3 probabilities in operand slot order (slot 16 kb + r); the row
        // sum from the unrounded values. Gate statistic: the lane half's keys
        // fall into four classes (r % 4) of 8; the sum over classes of the
        // class's largest probability times its sum bounds sum p^2.
        float lt[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; r += 2) {
            float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(x[kb][r], c, msub));
            float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(x[kb][r + 1], c, msub));
            if constexpr (MASK && !CAUSAL) {
              if (key_of(kb, r) > lim) p0 = 0.0f;
              if (key_of(kb, r + 1) > lim) p1 = 0.0f;
            }
            lt[r & 3] += p0;
            lt[(r + 1) & 3] += p1;
            const int slot = 16 * kb + r;
            if (slot & 2) pb8[slot >> 2] = __builtin_amdgcn_cvt_pk_fp8_f32(p0, p1, pb8[slot >> 2], true);
            else pb8[slot >> 2] = __builtin_amdgcn_cvt_pk_fp8_f32(p0, p1, pb8[slot >> 2], false);
          }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          // mc[i] is the class's largest score (before the scale), masked
          // keys included only as -inf
          const float pm = mc[i] == -INFINITY ? 0.0f
                                              : __builtin_amdgcn_exp2f(__builtin_fmaf(mc[i], c, msub));
          s_run = __builtin_fmaf(pm, lt[i], s_run);
        }
        l_run += (lt[0] + lt[1]) + (lt[2] + lt[3]);
        return;
      }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          const float a0 = __builtin_fmaf(x[kb][r], c, msub);
          const float a1 = __builtin_fmaf(x[kb][r + 1], c, msub);
          f16x2 h2 = {(_Float16)__builtin_amdgcn_exp2f(a0), (_Float16)__builtin_amdgcn_exp2f(a1)};
          if constexpr (MASK && !CAUSAL) {
            // Keys past the end were loaded as copies of the last key: they
            // leave the max unchanged, and their probabilities are dropped.
            if (key_of(kb, r) > lim) h2[0] = (_Float16)0.0f;
            if (key_of(kb, r + 1) > lim) h2[1] = (_Float16)0.0f;
          }
          ls[(r >> 1) & 3] = __builtin_amdgcn_fdot2(h2, one, ls[(r >> 1) & 3], false);
          pb[kb][r >> 3][r & 7] = h2[0];
          pb[kb][r >> 3][(r & 7) + 1] = h2[1];
        }
    } else {
      // Per-key scales: y_j = sk_j dot_j (the dot product exact, one rounding
      // in the product; INT8 y_j carries a factor 2^-26, taken back in cqe)
      // and the score in log2 units is cq y_j. The V scales are folded into the staged V
      // (code * sv_j / sv_ref), so the weights are the probabilities
      // themselves and O is kept in units of sv_ref, which only grows.
      const float vr = tile_vref;
      if (vr != sv_cur && vr > 0.0f) {
        const float f = sv_cur > 0.0f ? sv_cur / vr : 0.0f;
#pragma unroll
        for (int i = 0; i < kDB; ++i) o[i] *= f;
        sv_cur = vr;
      }
      // A zero Q scale makes every score of the row 0; the floor keeps -inf
      // (masked) times it from giving NaN.
      const float cqe = fmaxf(cq, 1e-30f) * (kTokBias ? 67108864.0f : 1.0f);
      float y[2][16];
      float mc[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
          const f32x4 a4 = key_s[kb][rg];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int r = 4 * rg + i;
            // x - B = dot 2^-26 exactly (the 2^26 is folded into cqe).
            float yv = kTokBias ? (__int_as_float(sacc[kb][r]) - __int_as_float(kBiasBits)) * a4[i]
                                : (float)sacc[kb][r] * a4[i];
            if constexpr (MASK && CAUSAL) yv = key_of(kb, r) > lim ? -INFINITY : yv;
            y[kb][r] = yv;
            mc[i] = fmaxf(mc[i], yv);
          }
        }
      const float my = fmaxf(fmaxf(mc[0], mc[1]), fmaxf(mc[2], mc[3]));
      const float mt = my * cqe;
      if (__any(mt > m_run + kSlack)) {
        const float mrow = fmaxf(mt, __shfl_xor(mt, 32));
        const float m_new = mrow > m_run + kSlack ? fmaxf(m_run, mrow) : m_run;
        const float alpha = (m_run == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(m_run - m_new);
        l_run *= alpha;
#pragma unroll
        for (int i = 0; i < kDB; ++i) o[i] *= alpha;
        m_run = m_new;
      }
      const float msub = (m_run == -INFINITY) ? 0.0f : -m_run;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
          const float a0 = __builtin_fmaf(y[kb][r], cqe, msub);
          const float a1 = __builtin_fmaf(y[kb][r + 1], cqe, msub);
          f16x2 h2 = {(_Float16)__builtin_amdgcn_exp2f(a0), (_Float16)__builtin_amdgcn_exp2f(a1)};
          if constexpr (MASK && !CAUSAL) {
            if (key_of(kb, r) > lim) h2[0] = (_Float16)0.0f;
            if (key_of(kb, r + 1) > lim) h2[1] = (_Float16)0.0f;
          }
          ls[(r >> 1) & 3] = __builtin_amdgcn_fdot2(h2, one, ls[(r >> 1) & 3], false);
          pb[kb][r >> 3][r & 7] = h2[0];
          pb[kb][r >> 3][(r & 7) + 1] = h2[1];
        }
    }
    l_run += (ls[0] + ls[1]) + (ls[2] + ls[3]);
  };
  auto vphase = [&](int t) __attribute__((always_inline)) {
    const int n0 = t * kBN;
    // The mask is needed only on tiles crossing this wavefront's diagonal
    // (causal) and on a ragged last tile.
    const bool m = (n0 + kBN > p.Sk) || (CAUSAL && n0 + kBN - 1 > wrow0);
    if (m) softmax(t, std::true_type());
    else softmax(t, std::false_type());
  };

  // Prologue: K_0 and the scales of tile 0 staged; V buffer 1 (read as
  // "V_{-1}" by the first matrix phase, with zero probabilities) cleared;
  // K_1, V_0 and the scales of tile 1 in registers.
#pragma unroll
  for (int i = 0; i < 2; ++i) pb[i][0] = pb[i][1] = (f16x8){};
#pragma unroll
  for (int i = 0; i < 8; ++i) pb8[i] = 0;
  fetch_tile<D, KQT, VQT>(pf, p, kbase, vbase, 0, 0);
  if (wave == 0) fetch_scales(sr, p, sbase, 0, TOK);
  for (int i = tid; i < G::kVElems / 8; i += kThreads) ((uint4*)vbuf1)[i] = make_uint4(0, 0, 0, 0);
  stage_k<D, KQT, VQT>(kbuf0, pf);
  if (wave == 0) stage_scales<TOK>(sc, 0, sr, p.kv_scale_f16, vref_run);
  fetch_tile<D, KQT, VQT>(pf, p, kbase, vbase, tile_n0(1), 0);
  if (wave == 0) fetch_scales(sr, p, sbase, tile_n0(1), TOK);
  __syncthreads();

  // Each wavefront walks M_0, V_0, M_1, V_1, ..., V_{T-1}, M_T (M_t: matrix
  // work of tile t and staging; V_t: softmax of tile t), one element per
  // phase with a barrier after each; group B runs one phase behind group A,
  // so on every SIMD one wavefront is in a matrix phase while the other is
  // in a softmax phase. K_t sits in K buffer t % 2, V_{t-1} in V buffer
  // (t-1) % 2; M_t stages K_{t+1} and V_t into the other buffers.
  const int nphase = 2 * ntiles + 2;
  for (int i = 0; i < nphase; ++i) {
    const int j = i - grp;  // this wavefront's element
    if (j >= 0 && j <= 2 * ntiles) {
      const int tt = j >> 1;
      if ((j & 1) == 0) {
        const bool odd = tt & 1;
        // The matrix-phase wavefront issues ahead of the softmax wavefront
        // sharing its SIMD: its matrix instructions are the longer chain.
        __builtin_amdgcn_s_setprio(1);
        mphase(tt, odd ? kbuf1 : kbuf0, odd ? vbuf0 : vbuf1, odd ? kbuf0 : kbuf1,
               odd ? vbuf1 : vbuf0, std::true_type());
        __builtin_amdgcn_s_setprio(0);
      } else {
        vphase(tt);
      }
    }
    __syncthreads();
  }

  // Epilogue: lane holds row qrow, channels 32*db + 8*(r/4) + 4*half + (r%4).
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if constexpr (LPV) {
    // Accuracy gate: flag the wavefront when a row's effective number of keys
    // may be below kNeffMin; if any wavefront is flagged, the workgroup
    // writes nothing here and recomputes the whole item with the fp16 product.
    const float s_tot = s_run + __shfl_xor(s_run, 32);
    const bool fail = qvalid && !(l_tot * l_tot >= kNeffMin * s_tot);
    const bool any = __builtin_amdgcn_ballot_w64(fail) != 0;
    if (lane == 0) p.flags[(long)blockIdx.x * kWaves + wave] = any ? 1 : 0;
    if (__syncthreads_or(fail)) return true;
  }
  const float inv = sv_cur / l_tot;
  const long hbase = (long)b * p.o_batch + (long)h * p.o_head;
  if (p.out_dtype != QFA_F32) {
    // 16-bit output goes through LDS, one 32-row region per wavefront, and
    // leaves with 16-byte stores along the rows.
    constexpr int kOS = G::kOutStride;
    uint16_t* so = obuf + wave * 32 * kOS;
#pragma unroll
    for (int db = 0; db < kDB; ++db) {
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int d0 = db * 32 + 8 * rg + 4 * half;
        const float v0 = o[db][4 * rg] * inv, v1 = o[db][4 * rg + 1] * inv;
        const float v2 = o[db][4 * rg + 2] * inv, v3 = o[db][4 * rg + 3] * inv;
        uint32_t w0, w1;
        if (p.out_dtype == QFA_F16) {
          w0 = __builtin_bit_cast(uint32_t, (f16x2){(_Float16)v0, (_Float16)v1});
          w1 = __builtin_bit_cast(uint32_t, (f16x2){(_Float16)v2, (_Float16)v3});
        } else {
          w0 = f32_to_bf16_bits(v0) | (f32_to_bf16_bits(v1) << 16);
          w1 = f32_to_bf16_bits(v2) | (f32_to_bf16_bits(v3) << 16);
        }
        *(uint2*)(so + col * kOS + d0) = make_uint2(w0, w1);
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    constexpr int kCPR = D / 8;  // 16-byte chunks per row
#pragma unroll
    for (int q = lane; q < 32 * kCPR; q += 64) {
      const int row = q / kCPR, c = q % kCPR;
      if (wrow0 + row < p.Sq)
        *(uint4*)((uint16_t*)p.out + hbase + (long)(wrow0 + row) * p.o_row + c * 8) =
            *(const uint4*)(so + row * kOS + c * 8);
    }
    return false;
  }
  if (!qvalid) return false;
  const long obase = hbase + (long)qrow * p.o_row;
#pragma unroll
  for (int db = 0; db < kDB; ++db) {
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      const int d0 = db * 32 + 8 * rg + 4 * half;
      *(f32x4*)((float*)p.out + obase + d0) =
          (f32x4){o[db][4 * rg] * inv, o[db][4 * rg + 1] * inv, o[db][4 * rg + 2] * inv,
                  o[db][4 * rg + 3] * inv};
    }
  }
  return false;
}

// The forward kernel: one work item per workgroup. With LPV the item is first
// computed with the fp8 P.V product; a workgroup whose gate flagged a row
// recomputes the item at once with the fp16 product, exactly as the fp16
// kernel does, so the fallback costs only the flagged items' own time and
// overlaps with the rest of the grid.
template <int D, int KVM, bool CAUSAL, bool TOK, bool LPV>
__global__ __launch_bounds__(kThreads, 1) void fwd_kernel(FwdParams p) {
  using G = Geo<D>;
  __shared__ __align__(16) uint8_t kbuf0[G::kKBytes];
  __shared__ __align__(16) uint8_t kbuf1[G::kKBytes];
  __shared__ __align__(16) _Float16 vbuf0[G::kVElems];
  __shared__ __align__(16) _Float16 vbuf1[G::kVElems];
  __shared__ __align__(16) ScaleRing sc;
  __shared__ __align__(16) uint16_t obuf[kWaves * 32 * G::kOutStride];
  if constexpr (LPV) {
    if (!fwd_item<D, KVM, CAUSAL, TOK, true>(p, kbuf0, kbuf1, vbuf0, vbuf1, sc, obuf)) return;
    // Every wavefront has left the fp8 pass's last barrier (the gate's
    // reduction is one), so its LDS buffers are free.
    fwd_item<D, KVM, CAUSAL, TOK, false>(p, kbuf0, kbuf1, vbuf0, vbuf1, sc, obuf);
  } else {
    fwd_item<D, KVM, CAUSAL, TOK, false>(p, kbuf0, kbuf1, vbuf0, vbuf1, sc, obuf);
  }
}

template <int D, int KVM>
hipError_t launch_kv(const FwdParams& p, int grid, bool causal, bool tok, hipStream_t st) {
  if (causal) {
    if (tok) fwd_kernel<D, KVM, true, true, false><<<grid, kThreads, 0, st>>>(p);
    else fwd_kernel<D, KVM, true, false, false><<<grid, kThreads, 0, st>>>(p);
  } else {
    if (tok) fwd_kernel<D, KVM, false, true, false><<<grid, kThreads, 0, st>>>(p);
    else fwd_kernel<D, KVM, false, false, false><<<grid, kThreads, 0, st>>>(p);
  }
  return hipGetLastError();
}

// fp8 P.V forward with the in-kernel fp16 fallback; writes every work item's
// flags.
template <int D>
hipError_t launch_lowp(const FwdParams& p, int grid, bool causal, hipStream_t st) {
  if (causal) fwd_kernel<D, KV_F8_F8, true, false, true><<<grid, kThreads, 0, st>>>(p);
  else fwd_kernel<D, KV_F8_F8, false, false, true><<<grid, kThreads, 0, st>>>(p);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const FwdParams& p, int kvm, int grid, bool causal, bool tok, hipStream_t st) {
  switch (kvm) {
    case KV_I8_I8: return launch_kv<D, KV_I8_I8>(p, grid, causal, tok, st);
    case KV_I4_I4: return launch_kv<D, KV_I4_I4>(p, grid, causal, tok, st);
    case KV_I8_I4: return launch_kv<D, KV_I8_I4>(p, grid, causal, tok, st);
    case KV_F8_F8: return launch_kv<D, KV_F8_F8>(p, grid, causal, tok, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

// Kernel parameters of one forward call (shape checked by the C ABI).
static void fwd_params(const FwdArgs& a, FwdParams& p, ix::FwdShape& f) {
  p.q = (const uint8_t*)a.q;
  p.qs = a.qs;
  p.k = (const uint8_t*)a.k;
  p.ks = a.ks;
  p.v = (const uint8_t*)a.v;
  p.vs = a.vs;
  p.out = a.out;
  p.B = a.B;
  p.Hq = a.Hq;
  p.Hkv = a.Hkv;
  p.Sq = a.Sq;
  p.Sk = a.Sk;
  f = ix::fwd_shape(a.B, a.Hq, a.Hkv, a.Sq, a.Sk, a.D, a.layout == QFA_BSND, a.k_qtype == QFA_INT4,
                    a.v_qtype == QFA_INT4, a.q_block, a.kv_block);
  p.group = f.group;
  p.hpw = f.hpw;
  p.rph = f.rph;
  p.n_hg = f.n_hg;
  p.n_rb = f.n_rb;
  p.q_row = f.q.row; p.q_head = f.q.head; p.q_batch = f.q.batch;
  p.k_row = f.k.row; p.k_head = f.k.head; p.k_batch = f.k.batch;
  p.v_row = f.v.row; p.v_head = f.v.head; p.v_batch = f.v.batch;
  p.o_row = f.q.row; p.o_head = f.q.head; p.o_batch = f.q.batch;  // out: Q's shape, D per row
  p.q_block = a.q_block;
  p.kv_block = a.kv_block;
  p.nqblk = f.nqblk;
  p.nkblk = f.nkblk;
  p.q_scale_f16 = a.q_scale_dtype == QFA_F16;
  p.kv_scale_f16 = a.kv_scale_dtype == QFA_F16;
  p.out_dtype = a.out_dtype;
  p.scale_log2 = a.softmax_scale * kLog2e;
  p.xcd_order = f.xcd_order;
  p.flags = nullptr;
}

hipError_t launch_fwd(const FwdArgs& a, hipStream_t stream) {
  FwdParams p;
  ix::FwdShape f;
  fwd_params(a, p, f);
  const long grid = f.grid;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
  // Per-key scales unless every tile lies inside one scale block.
  const bool tok = f.per_key;
  int kvm = -1;
  if (a.q_qtype == QFA_FP8_E4M3 && a.k_qtype == QFA_FP8_E4M3 && a.v_qtype == QFA_FP8_E4M3) kvm = KV_F8_F8;
  if (a.q_qtype == QFA_INT8 && a.k_qtype == QFA_INT8 && a.v_qtype == QFA_INT8) kvm = KV_I8_I8;
  if (a.q_qtype == QFA_INT8 && a.k_qtype == QFA_INT4 && a.v_qtype == QFA_INT4) kvm = KV_I4_I4;
  if (a.q_qtype == QFA_INT8 && a.k_qtype == QFA_INT8 && a.v_qtype == QFA_INT4) kvm = KV_I8_I4;
  if (kvm < 0) return hipErrorInvalidValue;
  if (a.D == 64) return launch_d<64>(p, kvm, (int)grid, a.causal, tok, stream);
  return launch_d<128>(p, kvm, (int)grid, a.causal, tok, stream);
}

size_t fwd_lowp_workspace_bytes(int B, int Hq, int Hkv, int Sq) {
  const ix::FwdShape f = ix::fwd_shape(B, Hq, Hkv, Sq, 1, 128, false, false, false, 1, 1);
  return (size_t)f.grid * kWaves;
}

hipError_t launch_fwd_lowp(const FwdArgs& a, void* flags, hipStream_t stream) {
  FwdParams p;
  ix::FwdShape f;
  fwd_params(a, p, f);
  if (f.grid > 0x7FFFFFFF || f.per_key || a.q_qtype != QFA_FP8_E4M3 ||
      a.k_qtype != QFA_FP8_E4M3 || a.v_qtype != QFA_FP8_E4M3)
    return hipErrorInvalidValue;
  p.flags = (uint8_t*)flags;
  if (a.D == 64) return launch_lowp<64>(p, (int)f.grid, a.causal, stream);
  return launch_lowp<128>(p, (int)f.grid, a.causal, stream);
}

}  // namespace qfa
