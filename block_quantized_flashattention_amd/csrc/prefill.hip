// Prefill attention forward on block-quantized codes (gfx950).
//
// What it computes ([Ascend-INT8] INT8-operator sections 1-2; [MindIE-SD] FA
// quantization, "FP8 Attention"; [FA-INT8/INT4] INT8 and INT4 layers):
//   x_ij = softmax_scale * sq_i * sk_j * (Qc_i . Kc_j)     low-bit dot, wide accumulation
//   o_i  = sum_j softmax_j(x_ij) * sv_j * Vc_j             online softmax, P.V on MFMA
//
// Design:
//   * A workgroup owns 32*NW query rows of one (batch, head); each wavefront
//     owns 32 rows. Key tiles of BLOCK_N rows stream through LDS.
//   * Scores are formed transposed, S^T = K . Q^T, with
//     v_mfma_i32_32x32x32_i8 (INT8 Q/K; INT4 K is widened to INT8 while it is
//     staged) or v_mfma_f32_32x32x64_f8f6f4 (FP8 e4m3 Q/K). In the MFMA result
//     layout each lane then holds one query row and 16 of the 32 keys, so
//     row max and row sum are register reductions plus one exchange between
//     the two lane halves, and the probabilities are already in the register
//     layout of the B operand of the P.V product (O^T = V^T . P^T) on
//     v_mfma_f32_32x32x16_f16: P never goes through LDS.
//   * V is staged into LDS transposed ([d][key], fp16), its codes converted
//     once per workgroup (INT8, INT4 and e4m3 values are exact in fp16).
//     Keys are permuted inside each group of 16 so that every lane reads its
//     A-operand slice with one 16-byte LDS read.
//   * Scale fold: one multiply per score by sq_i * sk_j * softmax_scale *
//     log2(e); scores then go through exp2. sv_j multiplies the probability
//     before its fp16 rounding; the row sum uses the unscaled probability.
//   * The running row max is only raised when a tile's max exceeds it by more
//     than 8 (in log2 units), so the O rescale is skipped on most tiles; the
//     probabilities stay below 2^8 and the result is unchanged.
//   * Causal: key tiles past the workgroup's last row are skipped; the mask is
//     applied per element only on tiles that cross the diagonal. Workgroups
//     with the most tiles are launched first.
#include "qfa_device.h"
#include "qfa_launch.h"

namespace qfa {
namespace {

constexpr int kNW = 4;            // wavefronts per workgroup
constexpr int kBM = 32 * kNW;     // query rows per workgroup
constexpr int kBN = 64;           // keys per tile
constexpr float kRescaleSlack = 8.0f;

struct FwdParams {
  const uint8_t* q;
  const void* qs;
  const uint8_t* k;
  const void* ks;
  const uint8_t* v;
  const void* vs;
  void* out;
  int Hq, Hkv, Sq, Sk, group;
  long q_row, q_head, q_batch;  // byte strides of Q codes
  long k_row, k_head, k_batch;  // byte strides of K codes
  long v_row, v_head, v_batch;  // byte strides of V codes
  long o_row, o_head, o_batch;  // element strides of out
  int q_block, kv_block, nqblk, nkblk;
  int q_scale_f16, kv_scale_f16;
  int k_qtype, v_qtype, out_dtype;
  float scale_log2;  // softmax_scale * log2(e)
  int n_mblocks;
};

template <int D>
struct Smem {
  static constexpr int kKStride = D + 16;         // bytes per staged K row
  static constexpr int kVStride = kBN + 8;        // fp16 elements per staged V^T row
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

// Sign-extend eight packed two's-complement nibbles of `w` (element 2k low)
// into eight int8 bytes returned as two dwords.
__device__ __forceinline__ uint2 unpack_int4x8(uint32_t w) {
  uint32_t lo = w & 0x0F0F0F0Fu;         // elements 0,2,4,6
  uint32_t hi = (w >> 4) & 0x0F0F0F0Fu;  // elements 1,3,5,7
  lo |= (lo & 0x08080808u) * 0x1Eu;      // copy bit 3 into bits 4..7
  hi |= (hi & 0x08080808u) * 0x1Eu;
  // interleave: out0 = [lo.b0, hi.b0, lo.b1, hi.b1], out1 = [lo.b2, hi.b2, lo.b3, hi.b3]
  const uint32_t o0 = __builtin_amdgcn_perm(hi, lo, 0x05010400u);
  const uint32_t o1 = __builtin_amdgcn_perm(hi, lo, 0x07030602u);
  return make_uint2(o0, o1);
}

__device__ __forceinline__ _Float16 i8_to_h(uint32_t byte) {
  return (_Float16)(float)(int8_t)(uint8_t)byte;
}

// Stage one K tile (codes as bytes; INT4 widened to INT8) into LDS.
template <int D>
__device__ __forceinline__ void stage_k(Smem<D>& sm, const FwdParams& p, const uint8_t* kbase,
                                        int n0) {
  const int tid = threadIdx.x;
  if (p.k_qtype == QFA_INT4) {
    constexpr int kChunks = kBN * D / 16;  // 16 codes (8 bytes) per chunk
#pragma unroll
    for (int c = tid; c < kChunks; c += 64 * kNW) {
      const int key = c / (D / 16);
      const int col = (c % (D / 16)) * 16;
      uint2 w = make_uint2(0u, 0u);
      if (n0 + key < p.Sk) w = *(const uint2*)(kbase + (long)(n0 + key) * p.k_row + col / 2);
      const uint2 a = unpack_int4x8(w.x), b = unpack_int4x8(w.y);
      *(uint4*)(sm.k + key * Smem<D>::kKStride + col) = make_uint4(a.x, a.y, b.x, b.y);
    }
  } else {
    constexpr int kChunks = kBN * D / 16;
#pragma unroll
    for (int c = tid; c < kChunks; c += 64 * kNW) {
      const int key = c / (D / 16);
      const int col = (c % (D / 16)) * 16;
      uint4 w = make_uint4(0u, 0u, 0u, 0u);
      if (n0 + key < p.Sk) w = *(const uint4*)(kbase + (long)(n0 + key) * p.k_row + col);
      *(uint4*)(sm.k + key * Smem<D>::kKStride + col) = w;
    }
  }
}

// Stage one V tile transposed into LDS as fp16: each thread converts 4 keys x 8 channels.
template <int D>
__device__ __forceinline__ void stage_v(Smem<D>& sm, const FwdParams& p, const uint8_t* vbase,
                                        int n0) {
  constexpr int kUnits = (kBN / 4) * (D / 8);
  for (int u = threadIdx.x; u < kUnits; u += 64 * kNW) {
    const int kg = u % (kBN / 4);
    const int dg = u / (kBN / 4);
    const int key0 = kg * 4;
    _Float16 val[4][8];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int key = n0 + key0 + r;
      const bool ok = key < p.Sk;
      const uint8_t* src = vbase + (long)key * p.v_row;
      if (p.v_qtype == QFA_INT4) {
        const uint32_t w = ok ? *(const uint32_t*)(src + dg * 4) : 0u;
        const uint2 b = unpack_int4x8(w);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          val[r][e] = i8_to_h((b.x >> (8 * e)) & 0xFF);
          val[r][4 + e] = i8_to_h((b.y >> (8 * e)) & 0xFF);
        }
      } else {
        const uint2 w = ok ? *(const uint2*)(src + dg * 8) : make_uint2(0u, 0u);
        if (p.v_qtype == QFA_INT8) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            val[r][e] = i8_to_h((w.x >> (8 * e)) & 0xFF);
            val[r][4 + e] = i8_to_h((w.y >> (8 * e)) & 0xFF);
          }
        } else {
          const f32x2 a0 = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.x, false);
          const f32x2 a1 = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.x, true);
          const f32x2 a2 = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.y, false);
          const f32x2 a3 = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.y, true);
          val[r][0] = (_Float16)a0[0]; val[r][1] = (_Float16)a0[1];
          val[r][2] = (_Float16)a1[0]; val[r][3] = (_Float16)a1[1];
          val[r][4] = (_Float16)a2[0]; val[r][5] = (_Float16)a2[1];
          val[r][6] = (_Float16)a3[0]; val[r][7] = (_Float16)a3[1];
        }
      }
    }
    const int pos = vt_pos(key0);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      f16x4 col = {val[0][e], val[1][e], val[2][e], val[3][e]};
      *(f16x4*)(sm.vt + (dg * 8 + e) * Smem<D>::kVStride + pos) = col;
    }
  }
}

template <int D, bool FP8>
struct QK {
  // Bytes of one MFMA operand slice per lane and the number of MFMAs over D.
  static constexpr int kSlice = FP8 ? 32 : 16;
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
};

template <int D, bool FP8, bool CAUSAL, bool TOK_SCALE>
__global__ __launch_bounds__(64 * kNW) void fwd_kernel(FwdParams p) {
  using T = QK<D, FP8>;
  using Op = typename T::Op;
  using Acc = typename T::Acc;
  constexpr int kDB = D / 32;  // 32-channel blocks of the output
  __shared__ Smem<D> sm;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int half = lane >> 5;   // which half of the 32-key MFMA rows this lane holds
  const int col = lane & 31;    // query column of this lane
  const int mb = CAUSAL ? (p.n_mblocks - 1 - (int)blockIdx.x) : (int)blockIdx.x;
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  const int kvh = h / p.group;
  const int m0 = mb * kBM;
  const int qrow = m0 + wave * 32 + col;
  const bool qvalid = qrow < p.Sq;

  // Q slice of this lane (B operand of S^T = K . Q^T), kept in registers.
  Op qop[T::kSteps];
  {
    const uint8_t* qp = p.q + (long)b * p.q_batch + (long)h * p.q_head + (long)qrow * p.q_row;
#pragma unroll
    for (int s = 0; s < T::kSteps; ++s) {
      const int off = s * 2 * T::kSlice + half * T::kSlice;
      if constexpr (FP8) {
        i32x8 v = {0, 0, 0, 0, 0, 0, 0, 0};
        if (qvalid) {
          const i32x4 lo = *(const i32x4*)(qp + off);
          const i32x4 hi = *(const i32x4*)(qp + off + 16);
          v = (i32x8){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        }
        qop[s] = v;
      } else {
        i32x4 v = {0, 0, 0, 0};
        if (qvalid) v = *(const i32x4*)(qp + off);
        qop[s] = v;
      }
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
  float m_run = -INFINITY;
  float l_run = 0.0f;

  const int n_end = CAUSAL ? min(p.Sk, m0 + kBM) : p.Sk;
  for (int n0 = 0; n0 < n_end; n0 += kBN) {
    __syncthreads();
    stage_k<D>(sm, p, kbase, n0);
    stage_v<D>(sm, p, vbase, n0);
    if constexpr (TOK_SCALE) {
      for (int t = threadIdx.x; t < kBN; t += 64 * kNW) {
        const int key = n0 + t;
        const bool ok = key < p.Sk;
        sm.ksc[t] = ok ? load_scale(p.ks, sbase + key / p.kv_block, p.kv_scale_f16) : 0.0f;
        const float sv = ok ? load_scale(p.vs, sbase + key / p.kv_block, p.kv_scale_f16) : 0.0f;
        sm.vsc[t] = sv;
      }
    }
    __syncthreads();

    // S^T tile: two 32-key blocks.
    Acc sacc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      sacc[kb] = (Acc){};
      const uint8_t* krow = sm.k + (kb * 32 + col) * Smem<D>::kKStride;
#pragma unroll
      for (int s = 0; s < T::kSteps; ++s) {
        const int off = s * 2 * T::kSlice + half * T::kSlice;
        Op kop;
        if constexpr (FP8) {
          const i32x4 lo = *(const i32x4*)(krow + off);
          const i32x4 hi = *(const i32x4*)(krow + off + 16);
          kop = (i32x8){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        } else {
          kop = *(const i32x4*)(krow + off);
        }
        sacc[kb] = T::mma(kop, qop[s], sacc[kb]);
      }
    }

    // Scale fold and mask: x in log2 units.
    float x[2][16];
    float ck_tile = 0.0f;
    if constexpr (!TOK_SCALE) ck_tile = cq * load_scale(p.ks, sbase + n0 / p.kv_block, p.kv_scale_f16);
    const bool need_mask = (n0 + kBN > p.Sk) || (CAUSAL && n0 + kBN - 1 > m0);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kl = kb * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
        const float c = TOK_SCALE ? cq * sm.ksc[kl] : ck_tile;
        x[kb][r] = (float)sacc[kb][r] * c;
        if (need_mask) {
          const int key = n0 + kl;
          if (key >= p.Sk || (CAUSAL && key > qrow)) x[kb][r] = -INFINITY;
        }
      }
    }
    float mt = x[0][0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mt = fmaxf(mt, x[kb][r]);
    mt = fmaxf(mt, __shfl_xor(mt, 32));

    const bool need = mt > m_run + kRescaleSlack;
    if (__any(need)) {
      const float m_new = fmaxf(m_run, mt);
      const float alpha = (m_run == -INFINITY) ? 0.0f : exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < kDB; ++i) o[i] *= alpha;
      m_run = m_new;
    }
    const float msub = (m_run == -INFINITY) ? 0.0f : m_run;

    // Probabilities (fp16, sv folded in) as the B operand of O^T += V^T . P^T.
    f16x8 pb[2][2];
    float sv_tile = 0.0f;
    if constexpr (!TOK_SCALE) {
      sv_tile = load_scale(p.vs, sbase + n0 / p.kv_block, p.kv_scale_f16);
    }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float pr = exp2f(x[kb][r] - msub);
        l_run += pr;
        const int kl = kb * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
        const float sv = TOK_SCALE ? sm.vsc[kl] : sv_tile;
        pb[kb][r >> 3][r & 7] = (_Float16)(pr * sv);
      }
    }

#pragma unroll
    for (int db = 0; db < kDB; ++db) {
      const _Float16* vrow = sm.vt + (db * 32 + col) * Smem<D>::kVStride;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f16x8 a = *(const f16x8*)(vrow + g * 16 + half * 8);
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, pb[g >> 1][g & 1], o[db], 0, 0, 0);
      }
    }
  }

  // Epilogue: O^T lane layout -> row qrow, channels 32*db + 8*(r/4) + 4*half + (r%4).
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (!qvalid) return;
  const float inv = 1.0f / l_tot;
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
hipError_t launch_d(const FwdParams& p, dim3 grid, bool causal, bool tok, hipStream_t st) {
  const dim3 block(64 * kNW);
  if (causal) {
    if (tok) fwd_kernel<D, FP8, true, true><<<grid, block, 0, st>>>(p);
    else fwd_kernel<D, FP8, true, false><<<grid, block, 0, st>>>(p);
  } else {
    if (tok) fwd_kernel<D, FP8, false, true><<<grid, block, 0, st>>>(p);
    else fwd_kernel<D, FP8, false, false><<<grid, block, 0, st>>>(p);
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
  const dim3 grid(p.n_mblocks, a.Hq, a.B);
  const bool tok = (a.kv_block % kBN) != 0;
  const bool fp8 = a.q_qtype == QFA_FP8_E4M3;
  if (a.D == 64) {
    return fp8 ? launch_d<64, true>(p, grid, a.causal, tok, stream)
               : launch_d<64, false>(p, grid, a.causal, tok, stream);
  }
  return fp8 ? launch_d<128, true>(p, grid, a.causal, tok, stream)
             : launch_d<128, false>(p, grid, a.causal, tok, stream);
}

}  // namespace qfa
