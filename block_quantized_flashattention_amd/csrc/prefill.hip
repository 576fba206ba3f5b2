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
//     matrix work. Key tiles of 64 rows are double-buffered in LDS: the next
//     tile's codes are fetched into registers while the current one is
//     computed, then written to the free buffer; one barrier per tile.
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
//   * Scale fold: with one K scale per tile, the row max is taken on the
//     integer dot products and each probability costs one FMA and one exp2:
//     p = exp2(dot * (sq * sk * softmax_scale * log2 e) - m). The V block
//     scale is folded into the accumulator (O is kept in units of the current
//     V scale and rescaled when it changes). With per-token scales (INT4 K/V)
//     each score and probability takes one more multiply.
//   * The running row max is only raised when a tile's max exceeds it by more
//     than 8 (log2 units), so the O rescale is skipped on most tiles; the
//     probabilities stay below 2^8 (exact softmax, fp16-safe).
//   * Row sums add the fp16-rounded probabilities with v_dot2_f32_f16, i.e.
//     exactly the weights the P.V product uses.
//   * Causal: tiles past a workgroup's last row are skipped, wavefronts skip
//     tiles entirely above their rows, and the mask is applied per element
//     only on tiles crossing the diagonal. Work is ordered longest first.
//   * XCD-aware order: workgroup ids are dealt round-robin to the 8 XCDs, so
//     all query heads and row blocks of one (batch, KV head) are given ids on
//     the same XCD and its K/V codes stay in that XCD's L2.
#include "qfa_device.h"
#include "qfa_launch.h"

namespace qfa {
namespace {

constexpr int kNW = 4;            // wavefronts per workgroup
constexpr int kThreads = 64 * kNW;
constexpr int kBM = 32 * kNW;     // query rows per workgroup
constexpr int kBN = 64;           // keys per tile
constexpr int kXcds = 8;
constexpr float kRescaleSlack = 8.0f;

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
struct Stage {
  static constexpr int kKStride = D + 16;   // bytes per staged K row
  static constexpr int kVStride = kBN + 8;  // fp16 elements per staged V^T row
  uint8_t k[kBN * kKStride];
  _Float16 vt[D * kVStride];
  float ksc[kBN];
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

// Registers holding one prefetched tile of K and V codes for this thread.
struct Prefetch {
  uint4 k[2];
  uint2 v[4];
  float ks, vs;
};

template <int D>
__device__ __forceinline__ void fetch_tile(Prefetch& f, const FwdParams& p, const uint8_t* kbase,
                                           const uint8_t* vbase, long sbase, int n0) {
  const int tid = threadIdx.x;
  // K: 16-byte chunks of codes (8-byte chunks of packed INT4).
  constexpr int kChunks = kBN * D / 16;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int c = tid + i * kThreads;
    f.k[i] = make_uint4(0u, 0u, 0u, 0u);
    if (c < kChunks) {
      const int key = c / (D / 16);
      const int col = (c % (D / 16)) * 16;
      if (n0 + key < p.Sk) {
        if (p.k_qtype == QFA_INT4) {
          const uint2 w = *(const uint2*)(kbase + (long)(n0 + key) * p.k_row + col / 2);
          f.k[i] = make_uint4(w.x, w.y, 0u, 0u);
        } else {
          f.k[i] = *(const uint4*)(kbase + (long)(n0 + key) * p.k_row + col);
        }
      }
    }
  }
  // V: 4 keys x 8 channels per thread.
  constexpr int kUnits = (kBN / 4) * (D / 8);
  const int kg = tid % (kBN / 4), dg = tid / (kBN / 4);
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    f.v[r] = make_uint2(0u, 0u);
    const int key = n0 + kg * 4 + r;
    if (tid < kUnits && key < p.Sk) {
      const uint8_t* src = vbase + (long)key * p.v_row;
      if (p.v_qtype == QFA_INT4) f.v[r].x = *(const uint32_t*)(src + dg * 4);
      else f.v[r] = *(const uint2*)(src + dg * 8);
    }
  }
  f.ks = f.vs = 0.0f;
  if (tid < kBN && n0 + tid < p.Sk && (p.kv_block % kBN) != 0) {
    const long si = sbase + (n0 + tid) / p.kv_block;
    f.ks = load_scale(p.ks, si, p.kv_scale_f16);
    f.vs = load_scale(p.vs, si, p.kv_scale_f16);
  }
}

template <int D>
__device__ __forceinline__ void store_tile(Stage<D>& st, const Prefetch& f, const FwdParams& p) {
  const int tid = threadIdx.x;
  constexpr int kChunks = kBN * D / 16;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int c = tid + i * kThreads;
    if (c < kChunks) {
      const int key = c / (D / 16);
      const int col = (c % (D / 16)) * 16;
      uint4 w = f.k[i];
      if (p.k_qtype == QFA_INT4) {
        const uint2 a = unpack_int4x8(w.x), b = unpack_int4x8(w.y);
        w = make_uint4(a.x, a.y, b.x, b.y);
      }
      *(uint4*)(st.k + key * Stage<D>::kKStride + col) = w;
    }
  }
  constexpr int kUnits = (kBN / 4) * (D / 8);
  if (tid < kUnits) {
    const int kg = tid % (kBN / 4), dg = tid / (kBN / 4);
    f16x2 val[4][4];  // [key][channel pair]
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      uint2 w = f.v[r];
      if (p.v_qtype == QFA_INT4) w = unpack_int4x8(w.x);
      if (p.v_qtype == QFA_FP8_E4M3) {
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
    const int pos = vt_pos(kg * 4);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int j = e >> 1, s = e & 1;
      f16x4 col = {val[0][j][s], val[1][j][s], val[2][j][s], val[3][j][s]};
      *(f16x4*)(st.vt + (dg * 8 + e) * Stage<D>::kVStride + pos) = col;
    }
  }
  if (tid < kBN) {
    st.ksc[tid] = f.ks;
    st.vsc[tid] = f.vs;
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

template <int D, bool FP8, bool CAUSAL, bool TOK>
__global__ __launch_bounds__(kThreads, 2) void fwd_kernel(FwdParams p) {
  using T = QK<D, FP8>;
  using Op = typename T::Op;
  using Acc = typename T::Acc;
  constexpr int kDB = D / 32;  // 32-channel blocks of the output
  __shared__ Stage<D> stage[2];

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
  float sv_cur = 0.0f;      // V scale O is expressed in (per-tile scales)

  const int n_end = CAUSAL ? min(p.Sk, m0 + kBM) : p.Sk;
  const int ntiles = (n_end + kBN - 1) / kBN;

  Prefetch pf;
  fetch_tile<D>(pf, p, kbase, vbase, sbase, 0);
  store_tile<D>(stage[0], pf, p);
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int n0 = t * kBN;
    const Stage<D>& st = stage[t & 1];
    const bool more = t + 1 < ntiles;
    if (more) fetch_tile<D>(pf, p, kbase, vbase, sbase, n0 + kBN);

    const bool wave_active = !CAUSAL || n0 <= wrow0 + 31;
    if (wave_active) {
      // S^T tile: two 32-key blocks.
      Acc sacc[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        sacc[kb] = (Acc){};
        const uint8_t* krow = st.k + (kb * 32 + col) * Stage<D>::kKStride + half * T::kSlice;
#pragma unroll
        for (int s = 0; s < T::kSteps; ++s) sacc[kb] = T::mma(T::load(krow + s * 2 * T::kSlice), qop[s], sacc[kb]);
      }

      const bool need_mask = (n0 + kBN > p.Sk) || (CAUSAL && n0 + kBN - 1 > wrow0);
      float x[2][16];
      float mt;
      float sv_t = 1.0f;
      if constexpr (!TOK) {
        // One K and one V scale for the whole tile.
        const long si = sbase + n0 / p.kv_block;
        const float ck = cq * load_scale(p.ks, si, p.kv_scale_f16);
        sv_t = load_scale(p.vs, si, p.kv_scale_f16);
        // Masked keys (bit kb*16+r) only occur on tiles crossing the diagonal or the end.
        uint32_t mbits = 0;
        if (need_mask) {
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int key = n0 + kb * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
              if (key >= p.Sk || (CAUSAL && key > qrow)) mbits |= 1u << (kb * 16 + r);
            }
        }
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            x[kb][r] = (float)sacc[kb][r];
            mx = fmaxf(mx, (mbits >> (kb * 16 + r)) & 1u ? -INFINITY : x[kb][r]);
          }
        mt = mx == -INFINITY ? -INFINITY : mx * ck;  // ck >= 0: the max commutes with it
        mt = fmaxf(mt, __shfl_xor(mt, 32));
        // Rescale when the max grew past the slack or the V scale changed.
        const float sv_eff = sv_t > 0.0f ? sv_t : (sv_cur > 0.0f ? sv_cur : 1.0f);
        const bool need = mt > m_run + kRescaleSlack;
        if (__any(need) || sv_eff != sv_cur) {
          const float m_new = need ? fmaxf(m_run, mt) : m_run;
          const float alpha = (m_run == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(m_run - m_new);
          const float f = sv_cur > 0.0f ? alpha * (sv_cur / sv_eff) : 0.0f;
          l_run *= alpha;
#pragma unroll
          for (int i = 0; i < kDB; ++i) o[i] *= f;
          m_run = m_new;
          sv_cur = sv_eff;
        }
        const float msub = (m_run == -INFINITY) ? 0.0f : -m_run;
        // Probabilities as the B operand of O^T += V^T . P^T.
        f16x8 pb[2][2];
        const f16x2 one = {(_Float16)1.0f, (_Float16)1.0f};
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; r += 2) {
            float a0 = __builtin_fmaf(x[kb][r], ck, msub);
            float a1 = __builtin_fmaf(x[kb][r + 1], ck, msub);
            if (need_mask) {
              if ((mbits >> (kb * 16 + r)) & 1u) a0 = -INFINITY;
              if ((mbits >> (kb * 16 + r + 1)) & 1u) a1 = -INFINITY;
            }
            const float p0 = __builtin_amdgcn_exp2f(a0);
            const float p1 = __builtin_amdgcn_exp2f(a1);
            const f16x2 h2 = {(_Float16)p0, (_Float16)p1};
            l_run = __builtin_amdgcn_fdot2(h2, one, l_run, false);
            pb[kb][r >> 3][r & 7] = h2[0];
            pb[kb][r >> 3][(r & 7) + 1] = h2[1];
          }
#pragma unroll
        for (int db = 0; db < kDB; ++db) {
          const _Float16* vrow = st.vt + (db * 32 + col) * Stage<D>::kVStride + half * 8;
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const f16x8 a = *(const f16x8*)(vrow + g * 16);
            o[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, pb[g >> 1][g & 1], o[db], 0, 0, 0);
          }
        }
      } else {
        // Per-key scales (e.g. INT4 K/V with one scale per token).
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int rg = 0; rg < 4; ++rg) {
            const int kl = kb * 32 + 8 * rg + 4 * half;
            const f32x4 s4 = *(const f32x4*)(st.ksc + kl);
#pragma unroll
            for (int i = 0; i < 4; ++i) x[kb][4 * rg + i] = (float)sacc[kb][4 * rg + i] * (cq * s4[i]);
          }
        if (need_mask) {
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int key = n0 + kb * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
              if (key >= p.Sk || (CAUSAL && key > qrow)) x[kb][r] = -INFINITY;
            }
        }
        mt = x[0][0];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) mt = fmaxf(mt, x[kb][r]);
        mt = fmaxf(mt, __shfl_xor(mt, 32));
        const bool need = mt > m_run + kRescaleSlack;
        if (__any(need)) {
          const float m_new = fmaxf(m_run, mt);
          const float alpha = (m_run == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(m_run - m_new);
          l_run *= alpha;
#pragma unroll
          for (int i = 0; i < kDB; ++i) o[i] *= alpha;
          m_run = m_new;
        }
        const float msub = (m_run == -INFINITY) ? 0.0f : m_run;
        f16x8 pb[2][2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int rg = 0; rg < 4; ++rg) {
            const int kl = kb * 32 + 8 * rg + 4 * half;
            const f32x4 v4 = *(const f32x4*)(st.vsc + kl);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int r = 4 * rg + i;
              const float pr = __builtin_amdgcn_exp2f(x[kb][r] - msub);
              l_run += pr;
              pb[kb][r >> 3][r & 7] = (_Float16)(pr * v4[i]);
            }
          }
#pragma unroll
        for (int db = 0; db < kDB; ++db) {
          const _Float16* vrow = st.vt + (db * 32 + col) * Stage<D>::kVStride + half * 8;
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const f16x8 a = *(const f16x8*)(vrow + g * 16);
            o[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, pb[g >> 1][g & 1], o[db], 0, 0, 0);
          }
        }
      }
    }
    if (more) store_tile<D>(stage[(t + 1) & 1], pf, p);
    __syncthreads();
  }

  // Epilogue: lane holds row qrow, channels 32*db + 8*(r/4) + 4*half + (r%4).
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (!qvalid) return;
  const float inv = (TOK ? 1.0f : sv_cur) / l_tot;
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

template <int D, bool FP8>
hipError_t launch_d(const FwdParams& p, int grid, bool causal, bool tok, hipStream_t st) {
  if (causal) {
    if (tok) fwd_kernel<D, FP8, true, true><<<grid, kThreads, 0, st>>>(p);
    else fwd_kernel<D, FP8, true, false><<<grid, kThreads, 0, st>>>(p);
  } else {
    if (tok) fwd_kernel<D, FP8, false, true><<<grid, kThreads, 0, st>>>(p);
    else fwd_kernel<D, FP8, false, false><<<grid, kThreads, 0, st>>>(p);
  }
  return hipGetLastError();
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
  const bool fp8 = a.q_qtype == QFA_FP8_E4M3;
  if (a.D == 64) {
    return fp8 ? launch_d<64, true>(p, (int)grid, a.causal, tok, stream)
               : launch_d<64, false>(p, (int)grid, a.causal, tok, stream);
  }
  return fp8 ? launch_d<128, true>(p, (int)grid, a.causal, tok, stream)
             : launch_d<128, false>(p, (int)grid, a.causal, tok, stream);
}

}  // namespace qfa
