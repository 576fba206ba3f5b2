// Prefill attention forward on block-quantized codes (gfx950).
//
// What it computes ([Ascend-INT8] INT8-operator sections 1-2; [MindIE-SD] FA
// quantization, "FP8 Attention"; [FA-INT8/INT4] INT8 and INT4 layers):
//   x_ij = softmax_scale * sq_i * sk_j * (Qc_i . Kc_j)     low-bit dot, wide accumulation
//   o_i  = sum_j softmax_j(x_ij) * sv_j * Vc_j             online softmax, P.V on MFMA
//
// Design:
//   * A workgroup of 4 wavefronts owns 128 query rows of one (batch, head);
//     each wavefront owns 32 rows. Two workgroups share a CU (at most 256
//     registers per lane), so one's softmax arithmetic overlaps the other's
//     matrix work. Key tiles of 64 rows are double-buffered in LDS, K one tile
//     ahead of V; each tile's codes are loaded into registers a step before
//     they are staged, so a load has a step of compute to arrive; one barrier
//     per tile.
//   * Scores are formed transposed, S^T = K . Q^T, with
//     v_mfma_i32_32x32x32_i8 (INT8 Q/K; INT4 K is widened to INT8 while it is
//     staged) or v_mfma_f32_32x32x64_f8f6f4 (FP8 e4m3 Q/K). In the MFMA result
//     layout each lane then holds one query row and 16 of every 32 keys, so
//     row max and row sum are register reductions plus one exchange between
//     the lane halves, and the probabilities are already in the register
//     layout of the B operand of O^T += V^T . P^T on v_mfma_f32_32x32x16_f16:
//     P never goes through LDS.
//   * V is staged transposed ([channel][key], fp16): INT8, INT4 and e4m3 codes
//     are exact in fp16 and are converted once per workgroup. Keys are
//     permuted inside each group of 16 so that every lane reads its operand
//     slice with one 16-byte LDS read.
//   * Scale fold: with one K scale per tile, the row max is taken on the raw
//     scores (INT8: the biased accumulator read as floats, see kBiasAcc) and
//     each probability costs one FMA and one exp2:
//     p = exp2(dot * (sq * sk * softmax_scale * log2 e) - m). The V block
//     scale is folded into the accumulator (O is kept in units of the current
//     V scale and rescaled when it changes). With per-token scales (INT4 K/V)
//     each score and probability takes one more multiply.
//   * The running row max is only raised when a tile's max exceeds it by more
//     than 12 (log2 units; 8 with per-key scales, whose fp16 weights carry the
//     V scale), so the O rescale is skipped on most tiles; the probabilities
//     stay below 2^12 (exact softmax; fp16 holds them with its full 11-bit
//     precision, far below its 65504 limit).
//   * Row sums add the fp16-rounded probabilities with v_dot2_f32_f16, i.e.
//     exactly the weights the P.V product uses.
//   * One step per key tile: the max of tile t and the rare rescale, then
//     (INT8 with one scale per tile) one straight-line block holding S(t+1)
//     on the matrix unit, the exponentials of tile t, the staging of the next
//     tiles and P(t) V(t). FP8 and per-token scales issue S(t+1) in a block
//     of its own before the softmax (measured faster for them).
//   * Causal: tiles past a workgroup's last row are skipped and the mask is a
//     compile-time variant used only on tiles crossing a wavefront's diagonal
//     (in the straight-line INT8 step, a wavefront whose rows all lie above a
//     tile runs it fully masked rather than branching around it; the other
//     paths skip it). Work is ordered longest first.
//   * XCD-aware order: workgroup ids are dealt round-robin to the 8 XCDs, so
//     all query heads and row blocks of one (batch, KV head) are given ids on
//     the same XCD and its K/V codes stay in that XCD's L2.
//   * Epilogue: a lane holds 64 channels of one row, so direct stores would
//     touch 32 rows per instruction; fp16/bf16 output is staged in LDS per
//     wavefront and written with 16-byte stores along the rows.
#include <type_traits>

#include "qfa_device.h"
#include "qfa_launch.h"

namespace qfa {
namespace {

constexpr int kNW = 4;            // wavefronts per workgroup
constexpr int kThreads = 64 * kNW;
constexpr int kBM = 32 * kNW;     // query rows per workgroup
constexpr int kBN = 64;           // keys per tile
constexpr int kXcds = 8;
constexpr float kRescaleSlack = 12.0f;
// With per-key V scales the fp16 weight is p * sv; the smaller slack keeps it
// below 2^8 * sv, far from the fp16 limit for any plausible V scale.
constexpr float kRescaleSlackTok = 8.0f;

struct FwdParams {
  const uint8_t* q;
  const void* qs;
  const uint8_t* k;
  const void* ks;
  const uint8_t* v;
  const void* vs;
  void* out;
  int B, Hq, Hkv, Sq, Sk, group;
  long q_row, q_head, q_batch;  // byte strides of Q codes
  long k_row, k_head, k_batch;  // byte strides of K codes
  long v_row, v_head, v_batch;  // byte strides of V codes
  long o_row, o_head, o_batch;  // element strides of out
  int q_block, kv_block, nqblk, nkblk;
  int q_scale_f16, kv_scale_f16;
  int k_qtype, v_qtype, out_dtype;
  float scale_log2;  // softmax_scale * log2(e)
  int n_mblocks;
  int xcd_order;     // 1: XCD-grouped workgroup order
};

template <int D>
struct KStage {
  static constexpr int kStride = D + 16;    // bytes per staged K row
  uint8_t k[kBN * kStride];
};
template <int D>
struct VStage {
  static constexpr int kStride = kBN + 8;   // fp16 elements per staged V^T row
  _Float16 vt[D * kStride];
  float ksc[kBN];                           // K and V scales of the same tile's keys
  float vsc[kBN];
};

// Position of key `key` (0..kBN-1) inside a staged V^T row: groups of 4 keys
// are reordered inside each group of 16 as [0-3, 8-11, 4-7, 12-15].
__device__ __forceinline__ int vt_pos(int key) {
  const int g = key >> 4, a = (key >> 2) & 3, i = key & 3;
  return g * 16 + ((((a & 1) << 1) | (a >> 1)) << 2) + i;
}

// Sign-extend eight packed two's-complement nibbles of `w` (element 2k in the
// low nibble of byte k) into eight int8 bytes, returned as two dwords.
__device__ __forceinline__ uint2 unpack_int4x8(uint32_t w) {
  uint32_t lo = w & 0x0F0F0F0Fu;         // elements 0,2,4,6
  uint32_t hi = (w >> 4) & 0x0F0F0F0Fu;  // elements 1,3,5,7
  lo |= (lo & 0x08080808u) * 0x1Eu;      // copy bit 3 into bits 4..7
  hi |= (hi & 0x08080808u) * 0x1Eu;
  const uint32_t o0 = __builtin_amdgcn_perm(hi, lo, 0x05010400u);
  const uint32_t o1 = __builtin_amdgcn_perm(hi, lo, 0x07030602u);
  return make_uint2(o0, o1);
}

// Four signed bytes of `w` as two packed fp16 pairs (exact): the byte is
// placed in the mantissa of 1024 + (byte ^ 0x80) and 1152 is subtracted.
__device__ __forceinline__ void i8x4_to_h(uint32_t w, f16x2& lo, f16x2& hi) {
  const uint32_t u = w ^ 0x80808080u;
  const uint32_t a = __builtin_amdgcn_perm(0x64646464u, u, 0x05010400u);  // bytes 0,1
  const uint32_t b = __builtin_amdgcn_perm(0x64646464u, u, 0x07030602u);  // bytes 2,3
  const f16x2 bias = {(_Float16)1152.0f, (_Float16)1152.0f};
  lo = __builtin_bit_cast(f16x2, a) - bias;
  hi = __builtin_bit_cast(f16x2, b) - bias;
}

// Code types of K and V handled by one kernel instance.
enum KVMode { KV_I8_I8 = 0, KV_I4_I4 = 1, KV_I8_I4 = 2, KV_F8_F8 = 3 };
template <int M> struct KVTypes;
template <> struct KVTypes<KV_I8_I8> { static constexpr int K = QFA_INT8, V = QFA_INT8; };
template <> struct KVTypes<KV_I4_I4> { static constexpr int K = QFA_INT4, V = QFA_INT4; };
template <> struct KVTypes<KV_I8_I4> { static constexpr int K = QFA_INT8, V = QFA_INT4; };
template <> struct KVTypes<KV_F8_F8> { static constexpr int K = QFA_FP8_E4M3, V = QFA_FP8_E4M3; };

// Registers holding one prefetched tile of K and V codes (and scales) for this thread.
struct Prefetch {
  uint4 k[kBN * 128 / 16 / kThreads];
  uint2 v[4];
  uint32_t ks, vs;  // raw dwords holding this thread's key's scales
  uint32_t shift;   // bit offset of an fp16 scale inside its dword
};

__device__ __forceinline__ float scale_from_bits(uint32_t bits, bool f16) {
  return f16 ? f16_bits_to_f32(bits) : __uint_as_float(bits);
}

// Issue the loads of one tile's codes and scales into registers. Every load is
// unconditional (keys past the end are clamped to the last key, whose codes
// are finite and whose scores are masked) and nothing reads the loaded values
// before store_tile, so the loads stay in flight across the compute of the
// tiles in between. In-head offsets are 32-bit (checked on the host).
template <int D, int KQT, int VQT>
__device__ __forceinline__ void fetch_tile(Prefetch& f, const FwdParams& p, const uint8_t* kbase,
                                           const uint8_t* vbase, long sbase, int kn0, int vn0) {
  const int tid = threadIdx.x;
  const int last = p.Sk - 1;
  int n0 = kn0;
  const uint32_t krow = (uint32_t)p.k_row, vrow = (uint32_t)p.v_row;
  constexpr int kChunks = kBN * D / 16;  // 16 codes per chunk
  static_assert(kChunks % kThreads == 0, "K chunks per thread");
#pragma unroll
  for (int i = 0; i < kChunks / kThreads; ++i) {
    const int c = tid + i * kThreads;
    const uint32_t key = (uint32_t)min(n0 + c / (D / 16), last);
    const uint32_t col = (uint32_t)(c % (D / 16)) * 16u;
    if constexpr (KQT == QFA_INT4) {
      const uint2 w = *(const uint2*)(kbase + (key * krow + col / 2u));
      f.k[i] = make_uint4(w.x, w.y, 0u, 0u);
    } else {
      f.k[i] = *(const uint4*)(kbase + (key * krow + col));
    }
  }
  // V: 4 keys x 8 channels per thread (threads past the last unit repeat a unit).
  n0 = vn0;
  constexpr int kUnits = (kBN / 4) * (D / 8);
  const int u = tid % kUnits;
  const int kg = u % (kBN / 4), dg = u / (kBN / 4);
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const uint32_t key = (uint32_t)min(n0 + kg * 4 + r, last);
    if constexpr (VQT == QFA_INT4) {
      f.v[r] = make_uint2(*(const uint32_t*)(vbase + (key * vrow + (uint32_t)dg * 4u)), 0u);
    } else {
      f.v[r] = *(const uint2*)(vbase + (key * vrow + (uint32_t)dg * 8u));
    }
  }
  // Scale of this thread's key (slot 0 alone is read when one scale covers the
  // tile), as the aligned dword holding it, for either scale type.
  const int key = min(n0 + (tid % kBN), last);
  const long g = sbase + (p.kv_block == 1 ? key : key / p.kv_block);
  const long widx = p.kv_scale_f16 ? (g >> 1) : g;
  f.shift = p.kv_scale_f16 ? (uint32_t)(g & 1) * 16u : 0u;
  f.ks = ((const uint32_t*)p.ks)[widx];
  f.vs = ((const uint32_t*)p.vs)[widx];
}

template <int D, int KQT>
__device__ __forceinline__ void store_k(KStage<D>& st, const Prefetch& f) {
  const int tid = threadIdx.x;
  constexpr int kChunks = kBN * D / 16;
#pragma unroll
  for (int i = 0; i < kChunks / kThreads; ++i) {
    const int c = tid + i * kThreads;
    const int key = c / (D / 16);
    const int col = (c % (D / 16)) * 16;
    uint4 w = f.k[i];
    if constexpr (KQT == QFA_INT4) {
      const uint2 a = unpack_int4x8(w.x), b = unpack_int4x8(w.y);
      w = make_uint4(a.x, a.y, b.x, b.y);
    }
    *(uint4*)(st.k + key * KStage<D>::kStride + col) = w;
  }
}

template <int D, int VQT>
__device__ __forceinline__ void store_v(VStage<D>& st, const Prefetch& f, bool scale_f16) {
  const int tid = threadIdx.x;
  constexpr int kUnits = (kBN / 4) * (D / 8);
  if (kUnits >= kThreads || tid < kUnits) {
    const int kg = tid % (kBN / 4), dg = tid / (kBN / 4);
    const int pos = vt_pos(kg * 4);
    if constexpr (VQT == QFA_INT8) {
      // Transpose bytes first: one permute gathers channels (c, c+1) of two
      // keys, so each conversion yields a key pair of one channel, which is
      // what the transposed store needs.
#pragma unroll
      for (int d = 0; d < 2; ++d) {
        f16x2 pr[2][4];  // [key pair][channel 4d + i]
#pragma unroll
        for (int kp = 0; kp < 2; ++kp) {
          const uint32_t wa = d ? f.v[2 * kp].y : f.v[2 * kp].x;
          const uint32_t wb = d ? f.v[2 * kp + 1].y : f.v[2 * kp + 1].x;
          i8x4_to_h(__builtin_amdgcn_perm(wb, wa, 0x05010400u), pr[kp][0], pr[kp][1]);
          i8x4_to_h(__builtin_amdgcn_perm(wb, wa, 0x07030602u), pr[kp][2], pr[kp][3]);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const f16x4 col = {pr[0][i][0], pr[0][i][1], pr[1][i][0], pr[1][i][1]};
          *(f16x4*)(st.vt + (dg * 8 + 4 * d + i) * VStage<D>::kStride + pos) = col;
        }
      }
    } else {
    f16x2 val[4][4];  // [key][channel pair]
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      uint2 w = f.v[r];
      if constexpr (VQT == QFA_INT4) w = unpack_int4x8(w.x);
      if constexpr (VQT == QFA_FP8_E4M3) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const uint32_t ww = j ? w.y : w.x;
          const f32x2 a = __builtin_amdgcn_cvt_pk_f32_fp8((int)ww, false);
          const f32x2 b = __builtin_amdgcn_cvt_pk_f32_fp8((int)ww, true);
          val[r][2 * j] = (f16x2){(_Float16)a[0], (_Float16)a[1]};
          val[r][2 * j + 1] = (f16x2){(_Float16)b[0], (_Float16)b[1]};
        }
      } else {
        i8x4_to_h(w.x, val[r][0], val[r][1]);
        i8x4_to_h(w.y, val[r][2], val[r][3]);
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int j = e >> 1, s = e & 1;
      f16x4 col = {val[0][j][s], val[1][j][s], val[2][j][s], val[3][j][s]};
      *(f16x4*)(st.vt + (dg * 8 + e) * VStage<D>::kStride + pos) = col;
    }
    }
  }
  // Every thread holds the scales of key tid % kBN; the copies write equal
  // values, which keeps this store free of a branch.
  const uint32_t mask = scale_f16 ? 0xFFFFu : 0xFFFFFFFFu;
  st.ksc[tid % kBN] = scale_from_bits((f.ks >> f.shift) & mask, scale_f16);
  st.vsc[tid % kBN] = scale_from_bits((f.vs >> f.shift) & mask, scale_f16);
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
  // a . b plus an accumulator that starts at 0x3E22F983 in every element,
  // given as the inline constant 1/(2 pi) (INT8 only; the compiler does not
  // fold a splat into that operand). The result is only read as the
  // accumulator of the next matrix instruction of the same kind, which needs
  // no wait states; the leading s_nop covers a vector write of a or b just
  // before, which the hazard check cannot see through the asm.
  static __device__ __forceinline__ Acc mma_biased(const Op& a, const Op& b) {
    Acc r;
    asm("s_nop 2\n\tv_mfma_i32_32x32x32_i8 %0, %1, %2, 0x3e22f983" : "=&v"(r) : "v"(a), "v"(b));
    return r;
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

// Key offset (within the tile) of accumulator register r of 32-key block kb,
// for the lane half `half`: MFMA 32x32 result rows 8*(r/4) + 4*half + r%4.
__device__ __forceinline__ constexpr int key_of(int kb, int r) { return kb * 32 + 8 * (r >> 2) + (r & 3); }

// RAGGED (non-causal only): Sk is not a multiple of the tile, so the last tile
// needs the end-of-keys mask; otherwise no tile does and the mask is compiled out.
template <int D, int KVM, bool CAUSAL, bool TOK, bool RAGGED>
__global__ __launch_bounds__(kThreads, 2) void fwd_kernel(FwdParams p) {
  constexpr bool FP8 = KVM == KV_F8_F8;
  constexpr int KQT = KVTypes<KVM>::K, VQT = KVTypes<KVM>::V;
  using T = QK<D, FP8>;
  using Op = typename T::Op;
  using Acc = typename T::Acc;
  constexpr int kDB = D / 32;  // 32-channel blocks of the output
  // INT8 scores with one scale per tile: the integer accumulator starts at the
  // bit pattern kBiasBits of the float kBiasInt * 2^-26 (the inline constant
  // 1/(2 pi) of the matrix instruction), so 'kBiasBits + dot' is the bit
  // pattern of the float (kBiasInt + dot) * 2^-26 exactly as long as the sum
  // stays in that binade, i.e. -2292099 <= dot < 6096509, which any 8-bit
  // codes with D <= 128 satisfy (|dot| <= 128 * 128 * 128). The scores then
  // need no integer-to-float conversion, and their max is a float max.
  constexpr bool kBiasAcc = !FP8 && !TOK;
  constexpr uint32_t kBiasBits = 0x3E22F983u;
  constexpr int kBiasInt = 10680707;  // 2^23 + 0x22F983
  static_assert(D <= 128, "biased INT8 scores need |dot| < 2^21");
  __shared__ KStage<D> kst[2];
  __shared__ VStage<D> vst[2];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int half = lane >> 5;  // lane half: keys 4*half + {0..3} of every 8
  const int col = lane & 31;   // query row of this lane within the wavefront

  // Work item of this workgroup.
  int mb, h, b;
  {
    const int id = blockIdx.x;
    const int G = p.group;
    const int ngroups = p.B * p.Hkv;
    int mrank, gidx, hig;
    if (p.xcd_order) {
      const int xcd = id % kXcds, k = id / kXcds;
      const int per_rank = (ngroups / kXcds) * G;
      mrank = k / per_rank;
      const int rem = k % per_rank;
      gidx = (rem / G) * kXcds + xcd;
      hig = rem % G;
    } else {
      const int per_rank = ngroups * G;
      mrank = id / per_rank;
      const int rem = id % per_rank;
      gidx = rem / G;
      hig = rem % G;
    }
    mb = CAUSAL ? p.n_mblocks - 1 - mrank : mrank;
    b = gidx / p.Hkv;
    h = (gidx % p.Hkv) * G + hig;
  }
  const int kvh = h / p.group;
  const int m0 = mb * kBM;
  const int wrow0 = m0 + wave * 32;
  const int qrow = wrow0 + col;
  const bool qvalid = qrow < p.Sq;

  // Q slice of this lane (B operand of S^T = K . Q^T), kept in registers.
  Op qop[T::kSteps];
  {
    const uint8_t* qp = p.q + (long)b * p.q_batch + (long)h * p.q_head + (long)qrow * p.q_row;
#pragma unroll
    for (int s = 0; s < T::kSteps; ++s) {
      qop[s] = (Op){};
      if (qvalid) qop[s] = T::load(qp + s * 2 * T::kSlice + half * T::kSlice);
    }
  }
  const float sq = qvalid ? load_scale(p.qs, ((long)b * p.Hq + h) * p.nqblk + qrow / p.q_block,
                                       p.q_scale_f16)
                          : 0.0f;
  const float cq = sq * p.scale_log2;

  const uint8_t* kbase = p.k + (long)b * p.k_batch + (long)kvh * p.k_head;
  const uint8_t* vbase = p.v + (long)b * p.v_batch + (long)kvh * p.v_head;
  const long sbase = ((long)b * p.Hkv + kvh) * p.nkblk;

  f32x16 o[kDB];
#pragma unroll
  for (int i = 0; i < kDB; ++i) o[i] = (f32x16){};
  float m_run = -INFINITY;  // reference row max (log2 units)
  float l_run = 0.0f;       // row sum of this lane half, in units of exp2(-m_run)
  float sv_cur = 0.0f;      // V scale O is expressed in (one scale per tile)

  const int n_end = CAUSAL ? min(p.Sk, m0 + kBM) : p.Sk;
  const int ntiles = (n_end + kBN - 1) / kBN;
  // Keys beyond this offset from the tile start are masked for this lane
  // (causal diagonal or end of the keys), per lane half.
  const int lim_base = (CAUSAL ? min(qrow, p.Sk - 1) : p.Sk - 1) - 4 * half;
  auto wave_active = [&](int t) { return !CAUSAL || t * kBN <= wrow0 + 31; };

  // S^T tile t = K_t . Q^T from K buffer t % 2 (two 32-key blocks).
  auto qk = [&](Acc* sacc, const KStage<D>& ks) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const uint8_t* krow = ks.k + (kb * 32 + col) * KStage<D>::kStride + half * T::kSlice;
      if constexpr (kBiasAcc) {
        sacc[kb] = T::mma_biased(T::load(krow), qop[0]);
      } else {
        sacc[kb] = T::mma(T::load(krow), qop[0], (Acc){});
      }
#pragma unroll
      for (int s = 1; s < T::kSteps; ++s)
        sacc[kb] = T::mma(T::load(krow + s * 2 * T::kSlice), qop[s], sacc[kb]);
    }
  };

  // One-scale-per-tile softmax in two parts. tile_max converts the scores of
  // a tile, takes their max and applies the lazy O rescale (a rare, uniform
  // branch); tile_exp forms the fp16 probabilities in the B-operand layout of
  // P.V and their row sums. Returns the score multiplier of the tile.
  auto tile_max = [&](const Acc* sacc, const VStage<D>& vs, float (&x)[2][16], auto mask_c,
                      bool rt_mask, int lim) -> float {
    const bool need_mask = decltype(mask_c)::value || rt_mask;
    const float ck = cq * vs.ksc[0];
    const float sv_t = vs.vsc[0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int v = sacc[kb][r];
        x[kb][r] = kBiasAcc ? __int_as_float(v) : (float)v;
      }
    // Tile max as four independent chains (short dependency depth).
    float mc[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
    if (need_mask) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          mc[r & 3] = fmaxf(mc[r & 3], key_of(kb, r) > lim ? -INFINITY : x[kb][r]);
    } else {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mc[r & 3] = fmaxf(mc[r & 3], x[kb][r]);
    }
    const float mx = fmaxf(fmaxf(mc[0], mc[1]), fmaxf(mc[2], mc[3]));
    // Max of this lane half; the row max over both halves is only formed when
    // some row needs a rescale (or the V scale changes), which is rare.
    // (x - kBiasInt * 2^-26) * 2^26 is the integer dot product, exactly.
    const float mt = mx == -INFINITY ? -INFINITY
                     : kBiasAcc ? (mx - __int_as_float(kBiasBits)) * (ck * 67108864.0f)
                                : mx * ck;  // ck >= 0
    const float sv_eff = sv_t > 0.0f ? sv_t : (sv_cur > 0.0f ? sv_cur : 1.0f);
    if (__any(mt > m_run + kRescaleSlack) || sv_eff != sv_cur) {
      const float mrow = fmaxf(mt, __shfl_xor(mt, 32));
      const float m_new = mrow > m_run + kRescaleSlack ? fmaxf(m_run, mrow) : m_run;
      const float alpha = (m_run == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(m_run - m_new);
      const float f = sv_cur > 0.0f ? alpha * (sv_cur / sv_eff) : 0.0f;
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < kDB; ++i) o[i] *= f;
      m_run = m_new;
      sv_cur = sv_eff;
    }
    return ck;
  };
  auto tile_exp = [&](const float (&x)[2][16], float ck, f16x8 (&pb)[2][2], auto mask_c,
                      bool rt_mask, int lim) {
    const bool need_mask = decltype(mask_c)::value || rt_mask;
    float msub = (m_run == -INFINITY) ? 0.0f : -m_run;
    if constexpr (kBiasAcc) {
      // x = (kBiasInt + dot) * 2^-26: scale by ck * 2^26 and fold the offset
      // into the subtrahend (one rounding, an error below one unit of dot).
      msub = __builtin_fmaf(-(float)kBiasInt, ck, msub);
      ck *= 67108864.0f;
    }
    const f16x2 one = {(_Float16)1.0f, (_Float16)1.0f};
    float ls[4] = {0.0f, 0.0f, 0.0f, 0.0f};  // independent partial row sums
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        float a0 = __builtin_fmaf(x[kb][r], ck, msub);
        float a1 = __builtin_fmaf(x[kb][r + 1], ck, msub);
        if (need_mask) {
          a0 = key_of(kb, r) > lim ? -INFINITY : a0;
          a1 = key_of(kb, r + 1) > lim ? -INFINITY : a1;
        }
        const f16x2 h2 = {(_Float16)__builtin_amdgcn_exp2f(a0),
                          (_Float16)__builtin_amdgcn_exp2f(a1)};
        ls[(r >> 1) & 3] = __builtin_amdgcn_fdot2(h2, one, ls[(r >> 1) & 3], false);
        pb[kb][r >> 3][r & 7] = h2[0];
        pb[kb][r >> 3][(r & 7) + 1] = h2[1];
      }
    l_run += (ls[0] + ls[1]) + (ls[2] + ls[3]);
  };
  // O^T += V_t^T . P_t^T; consecutive matrix instructions update different
  // output blocks.
  auto tile_pv = [&](const f16x8 (&pb)[2][2], const VStage<D>& vs) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
#pragma unroll
      for (int db = 0; db < kDB; ++db) {
        const _Float16* vrow = vs.vt + (db * 32 + col) * VStage<D>::kStride + half * 8;
        const f16x8 a = *(const f16x8*)(vrow + g * 16);
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, pb[g >> 1][g & 1], o[db], 0, 0, 0);
      }
    }
  };

  // Softmax of tile t and O^T += V_t^T . P_t^T (V and scales from V buffer t % 2).
  // The mask (causal diagonal or end of the keys) is a compile-time switch
  // for causal attention, so its many unmasked tiles carry no per-element
  // compare and select; without causality only a ragged last tile is masked
  // and a runtime flag (cheaper in registers there) selects it.
  auto softmax_pv = [&](const Acc* sacc, const VStage<D>& vs, int t, auto mask_c, bool rt_mask) {
    const int n0 = t * kBN;
    const bool need_mask = decltype(mask_c)::value || rt_mask;
    const int lim = lim_base - n0;  // masked iff key_of(kb, r) > lim
    f16x8 pb[2][2];
    if constexpr (!TOK) {
      float x[2][16];
      const float ck = tile_max(sacc, vs, x, mask_c, rt_mask, lim);
      tile_exp(x, ck, pb, mask_c, rt_mask, lim);
    } else {
      // Per-key scales (e.g. INT4 K/V with one scale per token).
      float x[2][16];
      float mc[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
          const f32x4 s4 = *(const f32x4*)(vs.ksc + kb * 32 + 8 * rg + 4 * half);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int r = 4 * rg + i;
            float xv = (float)sacc[kb][r] * (cq * s4[i]);
            if (need_mask) xv = key_of(kb, r) > lim ? -INFINITY : xv;
            x[kb][r] = xv;
            mc[i] = fmaxf(mc[i], xv);
          }
        }
      const float mt = fmaxf(fmaxf(mc[0], mc[1]), fmaxf(mc[2], mc[3]));
      if (__any(mt > m_run + kRescaleSlackTok)) {
        const float mrow = fmaxf(mt, __shfl_xor(mt, 32));
        const float m_new = mrow > m_run + kRescaleSlackTok ? fmaxf(m_run, mrow) : m_run;
        const float alpha = (m_run == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(m_run - m_new);
        l_run *= alpha;
#pragma unroll
        for (int i = 0; i < kDB; ++i) o[i] *= alpha;
        m_run = m_new;
      }
      const float msub = (m_run == -INFINITY) ? 0.0f : m_run;
      float ls[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
          const f32x4 v4 = *(const f32x4*)(vs.vsc + kb * 32 + 8 * rg + 4 * half);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int r = 4 * rg + i;
            const float pr = __builtin_amdgcn_exp2f(x[kb][r] - msub);
            ls[i] += pr;
            pb[kb][r >> 3][r & 7] = (_Float16)(pr * v4[i]);
          }
        }
      l_run += (ls[0] + ls[1]) + (ls[2] + ls[3]);
    }
    tile_pv(pb, vs);
  };

  // Pipeline: K runs one tile ahead of V. Step t issues S(t+1) = K_{t+1} Q^T on
  // the matrix unit, computes the softmax of S(t) on the vector unit meanwhile,
  // issues P(t) V_t, then writes the prefetched K_{t+2} and V_{t+1} (loaded
  // during the previous step) to the buffers freed by the last barrier.
  const int last_tile = ntiles - 1;
  auto tile_n0 = [&](int t) { return min(t, last_tile) * kBN; };
  Prefetch pf;
  fetch_tile<D, KQT, VQT>(pf, p, kbase, vbase, sbase, 0, 0);
  store_k<D, KQT>(kst[0], pf);
  store_v<D, VQT>(vst[0], pf, p.kv_scale_f16);
  fetch_tile<D, KQT, VQT>(pf, p, kbase, vbase, sbase, tile_n0(1), tile_n0(1));
  store_k<D, KQT>(kst[1], pf);
  fetch_tile<D, KQT, VQT>(pf, p, kbase, vbase, sbase, tile_n0(2), tile_n0(1));
  __syncthreads();

  Acc sa[2], sb[2];
  if (wave_active(0)) qk(sa, kst[0]);
  // One step with one scale per tile. After the max and the rare rescale,
  // S(t+1), the exponentials of tile t, the staging of the next tiles and
  // P(t) V(t) form one straight-line block, which leaves the compiler free to
  // interleave the matrix instructions with the vector work. S(t+1) is also
  // formed when tile t is the last one (from the clamped tile already staged;
  // the result is not used), and every wavefront runs every step (a step whose
  // keys all lie beyond a wavefront's rows is fully masked and adds nothing),
  // so the loop has no data-dependent paths besides the rescale.
  auto steady_step = [&](const int t, Acc* scur, Acc* snext, auto par, auto mask_c, bool rt_mask) {
    constexpr int PAR = decltype(par)::value;  // t % 2
    const int lim = lim_base - t * kBN;
    float x[2][16];
    f16x8 pb[2][2];
    const float ck = tile_max(scur, vst[PAR], x, mask_c, rt_mask, lim);
    qk(snext, kst[PAR ^ 1]);
    tile_exp(x, ck, pb, mask_c, rt_mask, lim);
    // K_{t+2} into K buffer t % 2 and V_{t+1} into V buffer (t+1) % 2, both
    // last read in step t-1, while P(t) V(t) runs.
    store_k<D, KQT>(kst[PAR], pf);
    store_v<D, VQT>(vst[PAR ^ 1], pf, p.kv_scale_f16);
    tile_pv(pb, vst[PAR]);
  };
  auto step = [&](const int t, Acc* scur, Acc* snext, auto par) {
    constexpr int PAR = decltype(par)::value;  // t % 2
    if constexpr (!TOK && !FP8) {
      const int n0 = t * kBN;
      // Masked: the causal diagonal, keys past the end, or a wavefront whose
      // rows all lie above the tile (every key masked, so the tile adds
      // nothing and the step runs the same instructions as the others).
      const bool m = (n0 + kBN > p.Sk) || (CAUSAL && n0 + kBN - 1 > wrow0);
      if constexpr (CAUSAL) {
        if (m) steady_step(t, scur, snext, par, std::true_type(), false);
        else steady_step(t, scur, snext, par, std::false_type(), false);
      } else {
        steady_step(t, scur, snext, par, std::false_type(), RAGGED && m);
      }
    } else {
      // Per-key scales and FP8 (measured faster this way): wavefronts skip the
      // tiles beyond their rows, and S(t+1) is a block of its own.
      if (t + 1 < ntiles && wave_active(t + 1)) qk(snext, kst[PAR ^ 1]);
      if (wave_active(t)) {
        const int n0 = t * kBN;
        const bool m = (n0 + kBN > p.Sk) || (CAUSAL && n0 + kBN - 1 > wrow0);
        if constexpr (CAUSAL) {
          if (m) softmax_pv(scur, vst[PAR], t, std::true_type(), false);
          else softmax_pv(scur, vst[PAR], t, std::false_type(), false);
        } else {
          softmax_pv(scur, vst[PAR], t, std::false_type(), RAGGED && m);
        }
      }
      // K_{t+2} into K buffer t % 2 (K_t was last read in step t-1) and
      // V_{t+1} into V buffer (t+1) % 2 (V_{t-1} was last read in step t-1).
      store_k<D, KQT>(kst[PAR], pf);
      store_v<D, VQT>(vst[PAR ^ 1], pf, p.kv_scale_f16);
    }
    __syncthreads();
    fetch_tile<D, KQT, VQT>(pf, p, kbase, vbase, sbase, tile_n0(t + 3), tile_n0(t + 2));
  };
  for (int t = 0; t < ntiles; t += 2) {
    step(t, sa, sb, std::integral_constant<int, 0>());
    if (t + 1 < ntiles) step(t + 1, sb, sa, std::integral_constant<int, 1>());
  }

  // Epilogue: lane holds row qrow, channels 32*db + 8*(r/4) + 4*half + (r%4).
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = (TOK ? 1.0f : sv_cur) / l_tot;
  if (p.out_dtype != QFA_F32) {
    // 16-bit output goes through LDS (the V buffers: every wavefront passed
    // the last step's barrier after its last read of them), one 32-row region
    // per wavefront, and leaves with 16-byte stores along the rows.
    constexpr int kOS = D + 8;  // 16-bit elements per staged row
    uint16_t* so = reinterpret_cast<uint16_t*>(&vst[0]) + wave * 32 * kOS;
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
    __syncthreads();
    const long hbase = (long)b * p.o_batch + (long)h * p.o_head;
    constexpr int kCPR = D / 8;  // 16-byte chunks per row
#pragma unroll
    for (int q = lane; q < 32 * kCPR; q += 64) {
      const int row = q / kCPR, c = q % kCPR;
      if (wrow0 + row < p.Sq)
        *(uint4*)((uint16_t*)p.out + hbase + (long)(wrow0 + row) * p.o_row + c * 8) =
            *(const uint4*)(so + row * kOS + c * 8);
    }
    return;
  }
  if (!qvalid) return;
  const long obase = (long)b * p.o_batch + (long)h * p.o_head + (long)qrow * p.o_row;
#pragma unroll
  for (int db = 0; db < kDB; ++db) {
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      const int d0 = db * 32 + 8 * rg + 4 * half;
      const float v0 = o[db][4 * rg] * inv, v1 = o[db][4 * rg + 1] * inv;
      const float v2 = o[db][4 * rg + 2] * inv, v3 = o[db][4 * rg + 3] * inv;
      if (p.out_dtype == QFA_F32) {
        *(f32x4*)((float*)p.out + obase + d0) = (f32x4){v0, v1, v2, v3};
      } else if (p.out_dtype == QFA_F16) {
        *(f16x4*)((_Float16*)p.out + obase + d0) =
            (f16x4){(_Float16)v0, (_Float16)v1, (_Float16)v2, (_Float16)v3};
      } else {
        const uint32_t w0 = f32_to_bf16_bits(v0) | (f32_to_bf16_bits(v1) << 16);
        const uint32_t w1 = f32_to_bf16_bits(v2) | (f32_to_bf16_bits(v3) << 16);
        *(uint2*)((uint16_t*)p.out + obase + d0) = make_uint2(w0, w1);
      }
    }
  }
}

template <int D, int KVM>
hipError_t launch_kv(const FwdParams& p, int grid, bool causal, bool tok, hipStream_t st) {
  const bool ragged = (p.Sk % kBN) != 0;
  if (causal) {
    if (tok) fwd_kernel<D, KVM, true, true, false><<<grid, kThreads, 0, st>>>(p);
    else fwd_kernel<D, KVM, true, false, false><<<grid, kThreads, 0, st>>>(p);
  } else if (ragged) {
    if (tok) fwd_kernel<D, KVM, false, true, true><<<grid, kThreads, 0, st>>>(p);
    else fwd_kernel<D, KVM, false, false, true><<<grid, kThreads, 0, st>>>(p);
  } else {
    if (tok) fwd_kernel<D, KVM, false, true, false><<<grid, kThreads, 0, st>>>(p);
    else fwd_kernel<D, KVM, false, false, false><<<grid, kThreads, 0, st>>>(p);
  }
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

hipError_t launch_fwd(const FwdArgs& a, hipStream_t stream) {
  FwdParams p;
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
  p.group = a.Hq / a.Hkv;
  const long kD = a.k_qtype == QFA_INT4 ? a.D / 2 : a.D;
  const long vD = a.v_qtype == QFA_INT4 ? a.D / 2 : a.D;
  if (a.layout == QFA_BNSD) {
    p.q_row = a.D; p.q_head = (long)a.Sq * a.D;
    p.k_row = kD; p.k_head = (long)a.Sk * kD;
    p.v_row = vD; p.v_head = (long)a.Sk * vD;
    p.o_row = a.D; p.o_head = (long)a.Sq * a.D;
  } else {
    p.q_row = (long)a.Hq * a.D; p.q_head = a.D;
    p.k_row = (long)a.Hkv * kD; p.k_head = kD;
    p.v_row = (long)a.Hkv * vD; p.v_head = vD;
    p.o_row = (long)a.Hq * a.D; p.o_head = a.D;
  }
  p.q_batch = (long)a.Hq * a.Sq * a.D;
  p.k_batch = (long)a.Hkv * a.Sk * kD;
  p.v_batch = (long)a.Hkv * a.Sk * vD;
  p.o_batch = (long)a.Hq * a.Sq * a.D;
  p.q_block = a.q_block;
  p.kv_block = a.kv_block;
  p.nqblk = (a.Sq + a.q_block - 1) / a.q_block;
  p.nkblk = (a.Sk + a.kv_block - 1) / a.kv_block;
  p.q_scale_f16 = a.q_scale_dtype == QFA_F16;
  p.kv_scale_f16 = a.kv_scale_dtype == QFA_F16;
  p.k_qtype = a.k_qtype;
  p.v_qtype = a.v_qtype;
  p.out_dtype = a.out_dtype;
  p.scale_log2 = a.softmax_scale * kLog2e;
  p.n_mblocks = (a.Sq + kBM - 1) / kBM;
  p.xcd_order = ((long)a.B * a.Hkv) % kXcds == 0;
  const long grid = (long)p.n_mblocks * a.B * a.Hq;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
  // Per-key scales unless every tile lies inside one scale block.
  const bool tok = (a.kv_block % kBN) != 0;
  int kvm = -1;
  if (a.q_qtype == QFA_FP8_E4M3 && a.k_qtype == QFA_FP8_E4M3 && a.v_qtype == QFA_FP8_E4M3) kvm = KV_F8_F8;
  if (a.q_qtype == QFA_INT8 && a.k_qtype == QFA_INT8 && a.v_qtype == QFA_INT8) kvm = KV_I8_I8;
  if (a.q_qtype == QFA_INT8 && a.k_qtype == QFA_INT4 && a.v_qtype == QFA_INT4) kvm = KV_I4_I4;
  if (a.q_qtype == QFA_INT8 && a.k_qtype == QFA_INT8 && a.v_qtype == QFA_INT4) kvm = KV_I8_I4;
  if (kvm < 0) return hipErrorInvalidValue;
  if (a.D == 64) return launch_d<64>(p, kvm, (int)grid, a.causal, tok, stream);
  return launch_d<128>(p, kvm, (int)grid, a.causal, tok, stream);
}

}  // namespace qfa
