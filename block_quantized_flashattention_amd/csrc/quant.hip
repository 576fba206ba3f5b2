// Block quantizer: symmetric per-block amax scales and INT8 / FP8 e4m3fn /
// packed INT4 codes.
//
// Arithmetic ([Ascend-INT8] section "对称量化 vs 非对称量化"; [MindIE-SD] FA
// quantization, block-quant step; [OT-Quant] sections 5.1-5.2):
//   amax = max |x| over R rows x D channels of one (batch, head)
//   s    = fl32(amax / qmax), optionally rounded to fp16; codes use the stored s
//   code = clamp(rne(fl32(x / s)))  (INT8 / INT4), e4m3fn(rne(clamp(x / s)))  (FP8)
//
// Design (HBM-bound: one read of x, one write of codes):
//   * A team of T = 2^k threads (up to 512) owns one block; each thread
//     holds about four (at most 16) chunks of 8 consecutive channels in
//     registers, so x is read from HBM once and many blocks are in flight per
//     CU. Larger blocks take a two-pass path (the second read mostly hits L2).
//     (Measured on Q/K/V of a 32-head, 4096-token fp16 attention: teams of
//     up to 512 threads beat 256 and 1024, and 2 or 8 target chunks.)
//   * Several tensors (Q, K, V) can share one launch, the workgroups of each
//     in a contiguous range, so the loads of one block overlap the reduction
//     and stores of others across the whole chip.
//   * amax is reduced on the raw bit patterns (|x| ordered as an unsigned
//     integer), across the team with lane shuffles and, for teams wider than
//     a wavefront, through LDS.
//   * The quotient fl32(x / s) is formed with a reciprocal r = 1/s (correctly
//     rounded, once per block) and two FMA residual corrections. With r the
//     nearest float to 1/s, the first correction makes the estimate faithful
//     and the second makes it the correctly rounded quotient (Markstein's
//     theorem on FMA-based division), provided the residuals do not
//     underflow. That holds for s in [2^-60, 2^100] whenever the quotient can
//     reach a nonzero code; other scales take the plain IEEE division.
//   * FP8 codes use the gfx950 converter to OCP e4m3 (nearest-even) after
//     clamping to +-448.
#include <algorithm>

#include "qfa_device.h"
#include "qfa_launch.h"

namespace qfa {
namespace {

struct QuantParams {
  const char* x;
  char* codes;
  void* scales;
  int N, S, D, R, nblk;
  long x_row, x_head, x_batch;  // element strides of x
  long c_row, c_head, c_batch;  // byte strides of codes
  int scale_f16;
  int team_log2;
  int chunks;      // chunks of 8 channels per thread
  int step_rows;   // (T*8) / D
  int step_cols;   // (T*8) % D
  long total_blocks;
};

template <int IN>
struct In;
template <>
struct In<QFA_F32> {
  static constexpr int kBytes = 4;
  struct Raw { uint4 a, b; };
  static __device__ __forceinline__ Raw load(const char* p) {
    Raw r;
    r.a = *(const uint4*)p;
    r.b = *(const uint4*)(p + 16);
    return r;
  }
  static __device__ __forceinline__ uint32_t absmax(const Raw& r) {
    uint32_t m = max(r.a.x & 0x7FFFFFFFu, r.a.y & 0x7FFFFFFFu);
    m = max(m, max(r.a.z & 0x7FFFFFFFu, r.a.w & 0x7FFFFFFFu));
    m = max(m, max(r.b.x & 0x7FFFFFFFu, r.b.y & 0x7FFFFFFFu));
    return max(m, max(r.b.z & 0x7FFFFFFFu, r.b.w & 0x7FFFFFFFu));
  }
  static __device__ __forceinline__ float amax_value(uint32_t bits) { return __uint_as_float(bits); }
  static __device__ __forceinline__ void to_f32(const Raw& r, float* f) {
    f[0] = __uint_as_float(r.a.x); f[1] = __uint_as_float(r.a.y);
    f[2] = __uint_as_float(r.a.z); f[3] = __uint_as_float(r.a.w);
    f[4] = __uint_as_float(r.b.x); f[5] = __uint_as_float(r.b.y);
    f[6] = __uint_as_float(r.b.z); f[7] = __uint_as_float(r.b.w);
  }
};

template <int IN>
struct In16 {
  static constexpr int kBytes = 2;
  struct Raw { uint4 a; };
  static __device__ __forceinline__ Raw load(const char* p) { return Raw{*(const uint4*)p}; }
  static __device__ __forceinline__ uint32_t m2(uint32_t w) {
    return max(w & 0x7FFFu, (w >> 16) & 0x7FFFu);
  }
  static __device__ __forceinline__ uint32_t absmax(const Raw& r) {
    return max(max(m2(r.a.x), m2(r.a.y)), max(m2(r.a.z), m2(r.a.w)));
  }
  static __device__ __forceinline__ float cvt(uint32_t h) {
    return IN == QFA_F16 ? f16_bits_to_f32(h) : bf16_bits_to_f32(h);
  }
  static __device__ __forceinline__ float amax_value(uint32_t bits) { return cvt(bits); }
  static __device__ __forceinline__ void to_f32(const Raw& r, float* f) {
    const uint32_t w[4] = {r.a.x, r.a.y, r.a.z, r.a.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = cvt(w[i] & 0xFFFFu);
      f[2 * i + 1] = cvt(w[i] >> 16);
    }
  }
};
template <>
struct In<QFA_F16> : In16<QFA_F16> {};
template <>
struct In<QFA_BF16> : In16<QFA_BF16> {};

// fl32(x / s) given r = fl32(1 / s). KEEP_ZERO_SIGN restores the sign of an
// exact zero quotient, which the FMA corrections turn into +0 (e4m3 encodes -0).
template <bool KEEP_ZERO_SIGN>
__device__ __forceinline__ float quotient(float x, float s, float r, bool fast) {
  if (!fast) return x / s;
  float q = x * r;
  float e = __builtin_fmaf(-q, s, x);
  q = __builtin_fmaf(e, r, q);
  e = __builtin_fmaf(-q, s, x);
  q = __builtin_fmaf(e, r, q);
  return KEEP_ZERO_SIGN ? __builtin_copysignf(q, x) : q;
}

template <int QT>
struct Enc;
template <>
struct Enc<QFA_INT8> {
  static constexpr float kQmax = 127.0f;
  static constexpr int kBytesPerChunk = 8;
  static __device__ __forceinline__ uint2 encode(const float* t) {
    uint32_t w[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      uint32_t acc = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float n = __builtin_amdgcn_fmed3f(__builtin_rintf(t[4 * j + i]), -128.0f, 127.0f);
        acc |= ((uint32_t)(int)n & 0xFFu) << (8 * i);
      }
      w[j] = acc;
    }
    return make_uint2(w[0], w[1]);
  }
};
template <>
struct Enc<QFA_FP8_E4M3> {
  static constexpr float kQmax = 448.0f;
  static constexpr int kBytesPerChunk = 8;
  static __device__ __forceinline__ uint2 encode(const float* t) {
    float c[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) c[i] = __builtin_amdgcn_fmed3f(t[i], -448.0f, 448.0f);
    int w0 = __builtin_amdgcn_cvt_pk_fp8_f32(c[0], c[1], 0, false);
    w0 = __builtin_amdgcn_cvt_pk_fp8_f32(c[2], c[3], w0, true);
    int w1 = __builtin_amdgcn_cvt_pk_fp8_f32(c[4], c[5], 0, false);
    w1 = __builtin_amdgcn_cvt_pk_fp8_f32(c[6], c[7], w1, true);
    return make_uint2((uint32_t)w0, (uint32_t)w1);
  }
};
template <>
struct Enc<QFA_INT4> {
  static constexpr float kQmax = 7.0f;
  static constexpr int kBytesPerChunk = 4;
  static __device__ __forceinline__ uint32_t encode(const float* t) {
    uint32_t acc = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float n = __builtin_amdgcn_fmed3f(__builtin_rintf(t[i]), -8.0f, 7.0f);
      acc |= ((uint32_t)(int)n & 0xFu) << (4 * i);
    }
    return acc;
  }
};

template <int QT>
__device__ __forceinline__ void store_codes(char* p, const float* t, bool zero) {
  if constexpr (QT == QFA_INT4) {
    *(uint32_t*)p = zero ? 0u : Enc<QT>::encode(t);
  } else {
    *(uint2*)p = zero ? make_uint2(0u, 0u) : Enc<QT>::encode(t);
  }
}

constexpr int kPassGroup = 4;  // chunk loads issued together in the two-pass path

// Team-wide max of an unsigned value. Teams wider than a wavefront go through
// LDS; every thread of the workgroup must call this (it may hold a barrier).
__device__ __forceinline__ uint32_t team_max(uint32_t m, int team_log2, uint32_t* lds) {
  const int T = 1 << team_log2;
  const int width = T < 64 ? T : 64;
  for (int off = width >> 1; off >= 1; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off));
  if (T <= 64) return m;
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) lds[wave] = m;
  __syncthreads();
  const int waves_per_team = T >> 6;
  const int first = (wave / waves_per_team) * waves_per_team;
  uint32_t r = 0;
  for (int w = 0; w < waves_per_team; ++w) r = max(r, lds[first + w]);
  return r;
}

// Blocks of workgroup `wg` of one tensor (blockDim / 2^team_log2 blocks per workgroup).
template <int IN, int QT, int CH, bool TWO_PASS>
__device__ __forceinline__ void quant_blocks(const QuantParams& p, long wg, uint32_t* lds) {
  using I = In<IN>;
  using E = Enc<QT>;
  const int T = 1 << p.team_log2;
  const int team = threadIdx.x >> p.team_log2;
  const int lt = threadIdx.x & (T - 1);
  const long gb = wg * ((int)blockDim.x >> p.team_log2) + team;
  const bool active = gb < p.total_blocks;
  const long g = active ? gb : 0;
  const int r = (int)(g % p.nblk);
  const long bn = g / p.nblk;
  const int n = (int)(bn % p.N);
  const int b = (int)(bn / p.N);
  const int row0 = r * p.R;
  const int rows = active ? min(p.R, p.S - row0) : 0;
  const char* xb = p.x + ((long)b * p.x_batch + (long)n * p.x_head + (long)row0 * p.x_row) * I::kBytes;
  char* cb = p.codes + (long)b * p.c_batch + (long)n * p.c_head + (long)row0 * p.c_row;
  const int code_div = QT == QFA_INT4 ? 2 : 1;

  // Chunk k of this thread covers channels [d, d+8) of block row `row`.
  int row0_t = (lt * 8) / p.D;
  int col0_t = (lt * 8) - row0_t * p.D;

  uint32_t amax_bits = 0;
  typename I::Raw raw[TWO_PASS ? 1 : CH];
  if constexpr (!TWO_PASS) {
    // All CH loads are issued before any is used: a chunk past the block
    // reads the block's first chunk instead (always in range) and is left
    // out of the max. Loads inside a branch that also used them made the
    // compiler wait for each one before issuing the next.
    int row = row0_t, col = col0_t;
    bool ok[CH];
#pragma unroll
    for (int k = 0; k < CH; ++k) {
      ok[k] = k < p.chunks && row < rows;
      const long off = ok[k] ? (long)row * p.x_row + col : 0L;
      raw[k] = I::load(xb + off * I::kBytes);
      row += p.step_rows;
      col += p.step_cols;
      if (col >= p.D) { col -= p.D; ++row; }
    }
#pragma unroll
    for (int k = 0; k < CH; ++k) amax_bits = max(amax_bits, ok[k] ? I::absmax(raw[k]) : 0u);
  } else {
    // Blocks too large for registers: two passes over x, each issuing
    // kPassGroup chunk loads together (past the block: the first chunk,
    // left out).
    int row = row0_t, col = col0_t;
    for (int k0 = 0; k0 < p.chunks && row < rows; k0 += kPassGroup) {
      typename I::Raw rg[kPassGroup];
      bool ok[kPassGroup];
#pragma unroll
      for (int u = 0; u < kPassGroup; ++u) {
        ok[u] = k0 + u < p.chunks && row < rows;
        rg[u] = I::load(xb + (ok[u] ? (long)row * p.x_row + col : 0L) * I::kBytes);
        row += p.step_rows;
        col += p.step_cols;
        if (col >= p.D) { col -= p.D; ++row; }
      }
#pragma unroll
      for (int u = 0; u < kPassGroup; ++u) amax_bits = max(amax_bits, ok[u] ? I::absmax(rg[u]) : 0u);
    }
  }
  amax_bits = team_max(amax_bits, p.team_log2, lds);
  if (!active) return;

  const float amax = I::amax_value(amax_bits);
  float s = amax / E::kQmax;
  if (p.scale_f16) s = (float)(_Float16)s;
  if (lt == 0) {
    const long si = ((long)b * p.N + n) * p.nblk + r;
    if (p.scale_f16) ((uint16_t*)p.scales)[si] = (uint16_t)f32_to_f16_bits(s);
    else ((float*)p.scales)[si] = s;
  }
  const bool zero = !(s != 0.0f);
  const bool fast = s >= 0x1p-60f && s <= 0x1p100f;
  const float rcp = fast ? 1.0f / s : 0.0f;

  if constexpr (!TWO_PASS) {
    int row = row0_t, col = col0_t;
#pragma unroll
    for (int k = 0; k < CH; ++k) {
      if (k < p.chunks && row < rows) {
        float f[8], t[8];
        I::to_f32(raw[k], f);
#pragma unroll
        for (int i = 0; i < 8; ++i) t[i] = quotient<QT == QFA_FP8_E4M3>(f[i], s, rcp, fast);
        store_codes<QT>(cb + (long)row * p.c_row + col / code_div, t, zero);
      }
      row += p.step_rows;
      col += p.step_cols;
      if (col >= p.D) { col -= p.D; ++row; }
    }
  } else {
    int row = row0_t, col = col0_t;
    for (int k0 = 0; k0 < p.chunks && row < rows; k0 += kPassGroup) {
      typename I::Raw rg[kPassGroup];
      int rr[kPassGroup], cc[kPassGroup];
      bool ok[kPassGroup];
#pragma unroll
      for (int u = 0; u < kPassGroup; ++u) {
        ok[u] = k0 + u < p.chunks && row < rows;
        rr[u] = row;
        cc[u] = col;
        rg[u] = I::load(xb + (ok[u] ? (long)row * p.x_row + col : 0L) * I::kBytes);
        row += p.step_rows;
        col += p.step_cols;
        if (col >= p.D) { col -= p.D; ++row; }
      }
#pragma unroll
      for (int u = 0; u < kPassGroup; ++u) {
        if (!ok[u]) continue;
        float f[8], t[8];
        I::to_f32(rg[u], f);
#pragma unroll
        for (int i = 0; i < 8; ++i) t[i] = quotient<QT == QFA_FP8_E4M3>(f[i], s, rcp, fast);
        store_codes<QT>(cb + (long)rr[u] * p.c_row + cc[u] / code_div, t, zero);
      }
    }
  }
}

constexpr int kMaxTeam = 512;      // threads per block team (and per workgroup)
constexpr int kTargetChunks = 4;   // chunks of 8 channels per thread, when the team allows

// Up to kMaxJobs tensors of one input type and code type per launch: the
// workgroups of job j are [start[j], start[j+1]). Launching several tensors
// together (Q, K and V) gives the chip enough blocks that one workgroup's
// loads overlap another's reduction and stores.
constexpr int kMaxJobs = 4;
struct MultiParams {
  QuantParams job[kMaxJobs];
  long start[kMaxJobs];
  int njobs;
};

template <int IN, int QT, int CH, bool TWO_PASS>
__global__ __launch_bounds__(kMaxTeam) void block_quant_kernel(MultiParams mp) {
  __shared__ uint32_t lds[kMaxTeam / 64];
  const long bid = blockIdx.x;
  // Job of this workgroup, selected with uniform (scalar) moves only.
  QuantParams p = mp.job[0];
  long wg = bid;
#pragma unroll
  for (int j = 1; j < kMaxJobs; ++j) {
    if (j < mp.njobs && bid >= mp.start[j]) {
      p = mp.job[j];
      wg = bid - mp.start[j];
    }
  }
  quant_blocks<IN, QT, CH, TWO_PASS>(p, wg, lds);
}

// Registers per thread: the single-pass path keeps up to 16 chunks of 8
// channels (8 for fp32 inputs); the chunk count is rounded up to a power of
// two. 0: the two-pass path.
int chunk_class(int chunks, int x_dtype) {
  if (chunks > (x_dtype == QFA_F32 ? 8 : 16)) return 0;
  int c = 1;
  while (c < chunks) c <<= 1;
  return c;
}

template <int IN, int QT>
hipError_t launch_typed(const MultiParams& mp, int cls, long grid, int threads, hipStream_t stream) {
  switch (cls) {
    case 1: block_quant_kernel<IN, QT, 1, false><<<grid, threads, 0, stream>>>(mp); break;
    case 2: block_quant_kernel<IN, QT, 2, false><<<grid, threads, 0, stream>>>(mp); break;
    case 4: block_quant_kernel<IN, QT, 4, false><<<grid, threads, 0, stream>>>(mp); break;
    case 8: block_quant_kernel<IN, QT, 8, false><<<grid, threads, 0, stream>>>(mp); break;
    case 16:
      if constexpr (IN != QFA_F32) block_quant_kernel<IN, QT, 16, false><<<grid, threads, 0, stream>>>(mp);
      break;
    default: block_quant_kernel<IN, QT, 1, true><<<grid, threads, 0, stream>>>(mp); break;
  }
  return hipGetLastError();
}

template <int IN>
hipError_t launch_in(const MultiParams& mp, int qtype, int cls, long grid, int threads,
                     hipStream_t stream) {
  switch (qtype) {
    case QFA_INT8: return launch_typed<IN, QFA_INT8>(mp, cls, grid, threads, stream);
    case QFA_FP8_E4M3: return launch_typed<IN, QFA_FP8_E4M3>(mp, cls, grid, threads, stream);
    default: return launch_typed<IN, QFA_INT4>(mp, cls, grid, threads, stream);
  }
}

// Kernel parameters and workgroup count of one tensor.
long prepare(const QuantArgs& a, QuantParams& p) {

  p.x = (const char*)a.x;
  p.codes = (char*)a.codes;
  p.scales = a.scales;
  p.N = a.N;
  p.S = a.S;
  p.D = a.D;
  p.R = a.block_rows;
  p.nblk = (a.S + a.block_rows - 1) / a.block_rows;
  const long cD = a.qtype == QFA_INT4 ? a.D / 2 : a.D;
  if (a.layout == QFA_BNSD) {
    p.x_row = a.D;
    p.x_head = (long)a.S * a.D;
    p.c_row = cD;
    p.c_head = (long)a.S * cD;
  } else {
    p.x_row = (long)a.N * a.D;
    p.x_head = a.D;
    p.c_row = (long)a.N * cD;
    p.c_head = cD;
  }
  p.x_batch = (long)a.N * a.S * a.D;
  p.c_batch = (long)a.N * a.S * cD;
  p.scale_f16 = a.scale_dtype == QFA_F16;
  // Team size: the power of two giving each thread about kTargetChunks
  // chunks (more threads in flight per block), capped at kMaxTeam.
  const long chunks_total = ((long)p.R * a.D) / 8;
  const long want = (chunks_total + kTargetChunks - 1) / kTargetChunks;
  int tl = 0;
  while ((1L << tl) < want && (1L << tl) < kMaxTeam) ++tl;
  p.team_log2 = tl;
  const long T = 1L << tl;
  p.chunks = (int)((chunks_total + T - 1) / T);
  p.step_rows = (int)((T * 8) / a.D);
  p.step_cols = (int)((T * 8) % a.D);
  p.total_blocks = (long)a.B * a.N * p.nblk;
  return p.total_blocks;
}


// ---- Fused rotation and block quantization -------------------------------
// y[row][i] = round16(sum_k x[row][k] * w[i][k]) with x and w in the same
// 16-bit type (bf16 or fp16) and round16 the nearest-even rounding back to
// that type, then the block quantizer above on y ([MindIE-SD] FP8 attention
// pipeline: rotate Q and K, then block-quantize; the rotation is given as
// w = R^T so that y = x . R). The product runs on the matrix unit as
// Y^T = W . X^T (v_mfma_f32_32x32x16_{bf16,f16}): W (D x D) is staged in LDS
// once per workgroup, each lane feeds one row of x straight from memory as
// the B operand, and each lane ends up holding 16 output channels of one row
// (4 runs of 4 consecutive channels), which it scales and writes as 4-byte
// code groups into LDS (over W, once every wavefront is done with it); the
// block's rows then leave with coalesced 16-byte stores. One workgroup owns
// one block of R rows (R a multiple of 32, at most 256): 4 wavefronts for
// R <= 128, else 8, each with one 32-row tile.

struct RotParams {
  const uint16_t* x;
  const uint16_t* w;
  char* codes;
  void* scales;
  int N, S, R, nblk;
  long x_row, x_head, x_batch;  // element strides of x
  long c_row, c_head, c_batch;  // byte strides of codes
  int scale_f16;
  int c16;  // codes and row stride 16-byte aligned
};

constexpr int kRotWaves = 4;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

template <bool BF16>
__device__ __forceinline__ f32x16 mma16(const i32x4& a, const i32x4& b, const f32x16& c) {
  if constexpr (BF16) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
}

// Round to the 16-bit input type and back (the value y takes before quantization).
template <bool BF16>
__device__ __forceinline__ float round16(float f) {
  if constexpr (BF16) return bf16_bits_to_f32(f32_to_bf16_bits(f));
  return (float)(_Float16)f;
}

// Four consecutive codes as one dword.
template <int QT>
__device__ __forceinline__ uint32_t encode4(const float* t) {
  if constexpr (QT == QFA_FP8_E4M3) {
    const float c0 = __builtin_amdgcn_fmed3f(t[0], -448.0f, 448.0f);
    const float c1 = __builtin_amdgcn_fmed3f(t[1], -448.0f, 448.0f);
    const float c2 = __builtin_amdgcn_fmed3f(t[2], -448.0f, 448.0f);
    const float c3 = __builtin_amdgcn_fmed3f(t[3], -448.0f, 448.0f);
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(c0, c1, 0, false);
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c2, c3, w, true);
  } else {
    uint32_t acc = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float n = __builtin_amdgcn_fmed3f(__builtin_rintf(t[i]), -128.0f, 127.0f);
      acc |= ((uint32_t)(int)n & 0xFFu) << (8 * i);
    }
    return acc;
  }
}

// W = 1 or 2 groups of 4 wavefronts, at most 128 VGPRs (four waves per SIMD:
// four 4-wave or two 8-wave workgroups per CU). At this budget the D = 128
// bf16 8-wave and fp16 4-wave kernels keep one value in scratch (one 4-byte
// store and three reloads, in straight-line code); a budget without the
// spill leaves one 8-wave workgroup per CU and measured 14% slower.
template <int D, bool BF16, int QT, int W>
__global__ __launch_bounds__(64 * kRotWaves * W, 4) void rot_quant_kernel(RotParams p) {
  constexpr int NW = kRotWaves * W;  // wavefronts: one 32-row tile each
  constexpr int kStride = D + 8;       // 16-bit elements per staged row of W
  constexpr int kIB = D / 32;          // 32-channel output blocks
  constexpr int kKS = D / 16;          // k steps of 16
  constexpr float kQmax = QT == QFA_FP8_E4M3 ? 448.0f : 127.0f;
  constexpr int kCS = D + 4;            // bytes per row of the staged codes
  constexpr int kWsElems = D * kStride > 256 * kCS / 2 ? D * kStride : 256 * kCS / 2;
  __shared__ __align__(16) uint16_t ws[kWsElems];
  __shared__ uint32_t red[NW];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int half = lane >> 5;
  const int col = lane & 31;  // row of x within a 32-row tile
  const long blk = blockIdx.x;
  const int r = (int)(blk % p.nblk);
  const long bn = blk / p.nblk;
  const int n = (int)(bn % p.N);
  const long b = bn / p.N;
  const int row0 = r * p.R;
  const int rows = min(p.R, p.S - row0);

  // Stage W (row-major, rows padded) with 16-byte copies, all requested
  // before the first is written.
  static_assert(D * D / 8 % (64 * NW) == 0, "W chunks per thread");
#pragma unroll
  for (int n = 0; n < D * D / 8 / (64 * NW); ++n) {
    const int c = threadIdx.x + n * 64 * NW;
    const int i = c / (D / 8), k8 = (c % (D / 8)) * 8;
    *(uint4*)(ws + i * kStride + k8) = *(const uint4*)(p.w + (long)i * D + k8);
  }
  __syncthreads();

  const uint16_t* xb = p.x + b * p.x_batch + (long)n * p.x_head + (long)row0 * p.x_row;
  f32x16 acc[1][kIB];
  uint32_t amax_bits = 0;
#pragma unroll
  for (int tt = 0; tt < 1; ++tt) {
    const int tile = wave + NW * tt;
    const int trow = tile * 32 + col;  // this lane's row within the block
    const bool valid = tile * 32 < rows && trow < rows;
    // B operands: 8 channels of this lane's row per k step (zero past the block).
    // Rows past the block load row 0 (always in range) and are zeroed after
    // the load, so no branch holds the loads back.
    i32x4 xo[kKS];
    const long xrow = valid ? (long)trow * p.x_row : 0L;
#pragma unroll
    for (int s = 0; s < kKS; ++s) xo[s] = *(const i32x4*)(xb + xrow + 16 * s + 8 * half);
#pragma unroll
    for (int s = 0; s < kKS; ++s) xo[s] = valid ? xo[s] : (i32x4){};
#pragma unroll
    for (int ib = 0; ib < kIB; ++ib) {
      acc[tt][ib] = (f32x16){};
      const uint16_t* wrow = ws + (ib * 32 + col) * kStride + 8 * half;
#pragma unroll
      for (int s = 0; s < kKS; ++s)
        acc[tt][ib] = mma16<BF16>(*(const i32x4*)(wrow + 16 * s), xo[s], acc[tt][ib]);
    }
#pragma unroll
    for (int ib = 0; ib < kIB; ++ib)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float y = round16<BF16>(acc[tt][ib][e]);
        acc[tt][ib][e] = y;
        amax_bits = max(amax_bits, __float_as_uint(y) & 0x7FFFFFFFu);
      }
  }
  // Block amax: wavefront shuffles, then the four wavefronts through LDS.
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) amax_bits = max(amax_bits, (uint32_t)__shfl_xor((int)amax_bits, off));
  if (lane == 0) red[wave] = amax_bits;
  __syncthreads();
  amax_bits = red[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) amax_bits = max(amax_bits, red[w]);

  const float amax = __uint_as_float(amax_bits);
  float sc = amax / kQmax;
  if (p.scale_f16) sc = (float)(_Float16)sc;
  if (threadIdx.x == 0) {
    const long si = bn * p.nblk + r;
    if (p.scale_f16) ((uint16_t*)p.scales)[si] = (uint16_t)f32_to_f16_bits(sc);
    else ((float*)p.scales)[si] = sc;
  }
  const bool zero = !(sc != 0.0f);
  const bool fast = sc >= 0x1p-60f && sc <= 0x1p100f;
  const float rcp = fast ? 1.0f / sc : 0.0f;
  char* cb = p.codes + b * p.c_batch + (long)n * p.c_head + (long)row0 * p.c_row;
  // The codes go through LDS (W is no longer read: every wavefront passed the
  // barrier above after its last matrix instruction), rows padded to D + 4
  // bytes so that the 32 rows of a wavefront's 4-byte writes hit distinct
  // banks; then each row is written with 16-byte (or 4-byte) coalesced stores.
  uint8_t* cs = (uint8_t*)ws;
  // The row and lane half are derived again from the thread index (through
  // an opaque copy, so the compiler does not keep the earlier values live
  // across the matrix instructions: under the 128-register cap that cost a
  // spill).
  int tid2 = threadIdx.x;
  asm volatile("" : "+v"(tid2));
  const int half2 = (tid2 >> 5) & 1;
#pragma unroll
  for (int tt = 0; tt < 1; ++tt) {
    const int trow = ((tid2 >> 6) + NW * tt) * 32 + (tid2 & 31);
    if (trow >= rows) continue;
#pragma unroll
    for (int ib = 0; ib < kIB; ++ib)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        // Accumulator registers 4g..4g+3: channels ib*32 + 8g + 4*half + 0..3.
        float t[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) t[i] = quotient<QT == QFA_FP8_E4M3>(acc[tt][ib][4 * g + i], sc, rcp, fast);
        *(uint32_t*)(cs + trow * kCS + ib * 32 + 8 * g + 4 * half2) = zero ? 0u : encode4<QT>(t);
      }
  }
  __syncthreads();
  if (p.c16) {
    for (int q = threadIdx.x; q < rows * (D / 16); q += 64 * NW) {
      const int row = q / (D / 16), c = q % (D / 16);
      const uint32_t* src = (const uint32_t*)(cs + row * kCS + c * 16);
      *(uint4*)(cb + (long)row * p.c_row + c * 16) = make_uint4(src[0], src[1], src[2], src[3]);
    }
  } else {
    for (int q = threadIdx.x; q < rows * (D / 4); q += 64 * NW) {
      const int row = q / (D / 4), c = q % (D / 4);
      *(uint32_t*)(cb + (long)row * p.c_row + c * 4) = *(const uint32_t*)(cs + row * kCS + c * 4);
    }
  }
}

template <int D, bool BF16, int QT>
hipError_t launch_rot_w(const RotParams& p, long grid, int w, hipStream_t st) {
  if (w == 1) rot_quant_kernel<D, BF16, QT, 1><<<grid, 64 * kRotWaves, 0, st>>>(p);
  else rot_quant_kernel<D, BF16, QT, 2><<<grid, 128 * kRotWaves, 0, st>>>(p);
  return hipGetLastError();
}

template <int D, bool BF16>
hipError_t launch_rot_qt(const RotParams& p, int qtype, long grid, int w, hipStream_t st) {
  if (qtype == QFA_FP8_E4M3) return launch_rot_w<D, BF16, QFA_FP8_E4M3>(p, grid, w, st);
  return launch_rot_w<D, BF16, QFA_INT8>(p, grid, w, st);
}

// ---- Appending one token to a quantized KV cache -------------------------
// One workgroup per (batch, KV head) and cache puts the new row at position p
// of the sequence into block r = p / R (with a second cache, the K and V rows
// of a decode step in one launch: workgroups B*H.. take the second). When the block already has rows, a nonzero
// scale s and fl32(max|x| / s) <= qmax (or x is all zero), only the new row is
// quantized, with s. Otherwise the block is requantized as a whole: its old
// rows' values fl32(code * s) and the new row get a new scale from their
// amax and new codes (rows past p are not touched).

struct AppendParams {
  const void* x;  // [B, H, D]
  const int32_t* pos;
  char* codes;
  void* scales;
  const void* x2;  // second cache (workgroups BH..2 BH - 1), or null
  char* codes2;
  void* scales2;
  int BH;          // B * H: workgroups per cache
  int H, S_max, D, R, nblk;
  long c_row, c_head, c_batch;  // byte strides of codes
  int x_dtype, scale_f16;
};

constexpr int kAppendThreads = 256;
constexpr int kAppendUnroll = 8;   // old code bytes per thread requested together

__device__ __forceinline__ float load_value(const void* x, long i, int dt) {
  // One dword load (for 16-bit types, the aligned dword that holds the
  // element) and selects: no branch around the load, so the compiler need
  // not wait for it where the paths merge.
  const long off = dt == QFA_F32 ? i * 4 : i * 2;
  const int mis = dt == QFA_F32 ? 0 : (int)(((uintptr_t)x + (uintptr_t)off) & 2u);
  const uint32_t w = *(const uint32_t*)((const char*)x + (off - mis));
  const uint32_t h = (w >> (8 * mis)) & 0xFFFFu;
  const float f16 = f16_bits_to_f32(h), b16 = bf16_bits_to_f32(h);
  return dt == QFA_F32 ? __uint_as_float(w) : dt == QFA_F16 ? f16 : b16;
}

// Workgroup max of an unsigned value (every thread calls it; one barrier pair).
__device__ __forceinline__ uint32_t wg_max(uint32_t m, uint32_t* red) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off));
  __syncthreads();  // red may still be read from a previous call
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  uint32_t r = 0;
#pragma unroll
  for (int w = 0; w < kAppendThreads / 64; ++w) r = max(r, red[w]);
  return r;
}

template <int QT>
__device__ __forceinline__ uint32_t code_bits(float t) {
  constexpr float lo = QT == QFA_INT4 ? -8.0f : -128.0f, hi = QT == QFA_INT4 ? 7.0f : 127.0f;
  return (uint32_t)(int)__builtin_amdgcn_fmed3f(__builtin_rintf(t), lo, hi) & (QT == QFA_INT4 ? 0xFu : 0xFFu);
}

template <int QT>
__device__ __forceinline__ int code_value(uint32_t bits) {
  return QT == QFA_INT4 ? (int)(bits << 28) >> 28 : (int)(bits << 24) >> 24;
}

template <int QT>
__global__ __launch_bounds__(kAppendThreads) void kv_append_kernel(AppendParams p) {
  constexpr int kPer = QT == QFA_INT4 ? 2 : 1;  // channels per code byte
  constexpr float kQmax = QT == QFA_INT4 ? 7.0f : 127.0f;
  __shared__ uint32_t red[kAppendThreads / 64];
  // Which cache this workgroup updates (uniform selects, no branch).
  const bool second = (int)blockIdx.x >= p.BH;
  const int bh = second ? (int)blockIdx.x - p.BH : (int)blockIdx.x;
  const void* x = second ? p.x2 : p.x;
  char* codes = second ? p.codes2 : p.codes;
  void* scales = second ? p.scales2 : p.scales;
  const int b = bh / p.H, h = bh % p.H;
  const int pp = p.pos[b];
  if (pp < 0 || pp >= p.S_max) return;  // the whole workgroup leaves
  const int r = pp / p.R, row0 = r * p.R, nold = pp - row0;
  const int tid = threadIdx.x;
  const int nbytes = p.D / kPer;  // code bytes per row

  // The block's stored scale, requested with the new row (used only when the
  // block already has rows).
  const long si = (long)bh * p.nblk + r;
  const float s_stored = load_scale(scales, si, p.scale_f16);
  // The new row: this thread's code byte holds channels kPer*tid .. + kPer-1.
  float xv[kPer];
  uint32_t ax = 0;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    xv[j] = 0.0f;
    if (tid < nbytes) xv[j] = load_value(x, ((long)b * p.H + h) * p.D + kPer * tid + j, p.x_dtype);
    ax = max(ax, __float_as_uint(xv[j]) & 0x7FFFFFFFu);
  }
  ax = wg_max(ax, red);
  const float amax_x = __uint_as_float(ax);
  const float s_old = nold == 0 ? 0.0f : s_stored;
  bool fits = false;
  if (nold > 0) fits = s_old > 0.0f ? amax_x / s_old <= kQmax : amax_x == 0.0f;
  char* cb = codes + (long)b * p.c_batch + (long)h * p.c_head;

  float s = s_old;
  if (!fits) {
    // amax of the old rows' values: fl32(max|code| * s_old), fl32 being monotonic.
    // kAppendUnroll bytes per thread and step are requested together; past
    // the last byte the index is clamped (a repeated byte leaves the max).
    uint32_t mc = 0;
    const int total = nold * nbytes;
    for (int e0 = tid; e0 < total; e0 += kAppendUnroll * kAppendThreads) {
      uint32_t by[kAppendUnroll];
#pragma unroll
      for (int u = 0; u < kAppendUnroll; ++u) {
        const int e = min(e0 + u * kAppendThreads, total - 1);
        by[u] = (uint8_t)cb[(long)(row0 + e / nbytes) * p.c_row + e % nbytes];
      }
#pragma unroll
      for (int u = 0; u < kAppendUnroll; ++u)
#pragma unroll
        for (int j = 0; j < kPer; ++j) mc = max(mc, (uint32_t)abs(code_value<QT>(by[u] >> (4 * j))));
    }
    mc = wg_max(mc, red);
    const float amax = fmaxf(amax_x, nold > 0 ? (float)mc * s_old : 0.0f);
    s = amax / kQmax;
    if (p.scale_f16) s = (float)(_Float16)s;
    if (tid == 0) {
      if (p.scale_f16) ((uint16_t*)scales)[si] = (uint16_t)f32_to_f16_bits(s);
      else ((float*)scales)[si] = s;
    }
  }
  const bool zero = !(s != 0.0f);
  const bool fast = s >= 0x1p-60f && s <= 0x1p100f;
  const float rcp = fast ? 1.0f / s : 0.0f;
  if (!fits) {
    // Requantize the old rows in place (each byte read and written by one
    // thread; kAppendUnroll bytes per thread and step requested together).
    const int total = nold * nbytes;
    for (int e0 = tid; e0 < total; e0 += kAppendUnroll * kAppendThreads) {
      uint32_t by[kAppendUnroll];
#pragma unroll
      for (int u = 0; u < kAppendUnroll; ++u) {
        const int e = min(e0 + u * kAppendThreads, total - 1);
        by[u] = (uint8_t)cb[(long)(row0 + e / nbytes) * p.c_row + e % nbytes];
      }
#pragma unroll
      for (int u = 0; u < kAppendUnroll; ++u) {
        const int e = e0 + u * kAppendThreads;
        if (e >= total) break;
        uint32_t out = 0;
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
          const float v = (float)code_value<QT>(by[u] >> (4 * j)) * s_old;
          out |= (zero ? 0u : code_bits<QT>(quotient<false>(v, s, rcp, fast))) << (4 * j);
        }
        cb[(long)(row0 + e / nbytes) * p.c_row + e % nbytes] = (char)out;
      }
    }
  }
  if (tid < nbytes) {
    uint32_t out = 0;
#pragma unroll
    for (int j = 0; j < kPer; ++j)
      out |= (zero ? 0u : code_bits<QT>(quotient<false>(xv[j], s, rcp, fast))) << (4 * j);
    cb[(long)pp * p.c_row + tid] = (char)out;
  }
}
}  // namespace

hipError_t launch_block_quant_multi(const QuantArgs* a, int n, hipStream_t stream) {
  // Group the tensors by (input type, code type, single or two-pass) in order
  // of first appearance; each group goes out in launches of up to kMaxJobs.
  if (n > 64) return hipErrorInvalidValue;
  QuantParams prm[64];
  bool done[64];
  for (int i = 0; i < n; ++i) done[i] = prepare(a[i], prm[i]) == 0;
  for (int i = 0; i < n; ++i) {
    if (done[i]) continue;
    const int xd = a[i].x_dtype;
    const bool two_pass = chunk_class(prm[i].chunks, xd) == 0;
    int sel[kMaxJobs], ns = 0, cls = 1, threads = 256;
    for (int j = i; j < n && ns < kMaxJobs; ++j) {
      if (done[j] || a[j].x_dtype != a[i].x_dtype || a[j].qtype != a[i].qtype ||
          (chunk_class(prm[j].chunks, xd) == 0) != two_pass)
        continue;
      sel[ns++] = j;
      done[j] = true;
      cls = two_pass ? 0 : std::max(cls, chunk_class(prm[j].chunks, xd));
      threads = std::max(threads, 1 << prm[j].team_log2);
    }
    MultiParams mp{};
    long grid = 0;
    for (int k = 0; k < ns; ++k) {
      const QuantParams& pj = prm[sel[k]];
      const long teams_per_wg = threads >> pj.team_log2;
      mp.job[k] = pj;
      mp.start[k] = grid;
      grid += (pj.total_blocks + teams_per_wg - 1) / teams_per_wg;
    }
    mp.njobs = ns;
    if (grid > 0x7FFFFFFFL) return hipErrorInvalidValue;
    hipError_t e;
    switch (a[i].x_dtype) {
      case QFA_F32: e = launch_in<QFA_F32>(mp, a[i].qtype, cls, grid, threads, stream); break;
      case QFA_F16: e = launch_in<QFA_F16>(mp, a[i].qtype, cls, grid, threads, stream); break;
      default: e = launch_in<QFA_BF16>(mp, a[i].qtype, cls, grid, threads, stream); break;
    }
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_block_quant(const QuantArgs& a, hipStream_t stream) {
  return launch_block_quant_multi(&a, 1, stream);
}


hipError_t launch_kv_append(const AppendArgs& a, hipStream_t stream) {
  AppendParams p{};
  p.x = a.x;
  p.pos = a.positions;
  p.codes = (char*)a.codes;
  p.scales = a.scales;
  p.x2 = a.x2;
  p.codes2 = (char*)a.codes2;
  p.scales2 = a.scales2;
  p.H = a.H;
  p.S_max = a.S_max;
  p.D = a.D;
  p.R = a.kv_block;
  p.nblk = (a.S_max + a.kv_block - 1) / a.kv_block;
  const long cD = a.qtype == QFA_INT4 ? a.D / 2 : a.D;
  if (a.layout == QFA_BNSD) {
    p.c_row = cD;
    p.c_head = (long)a.S_max * cD;
  } else {
    p.c_row = (long)a.H * cD;
    p.c_head = cD;
  }
  p.c_batch = (long)a.H * a.S_max * cD;
  p.x_dtype = a.x_dtype;
  p.scale_f16 = a.scale_dtype == QFA_F16;
  const long bh = (long)a.B * a.H;
  const long grid = a.x2 ? 2 * bh : bh;
  if (grid == 0) return hipSuccess;
  if (grid > 0x7FFFFFFFL) return hipErrorInvalidValue;
  p.BH = (int)bh;
  if (a.qtype == QFA_INT4) kv_append_kernel<QFA_INT4><<<grid, kAppendThreads, 0, stream>>>(p);
  else kv_append_kernel<QFA_INT8><<<grid, kAppendThreads, 0, stream>>>(p);
  return hipGetLastError();
}

hipError_t launch_rotate_block_quant(const RotQuantArgs& a, hipStream_t stream) {
  RotParams p{};
  p.x = (const uint16_t*)a.x;
  p.w = (const uint16_t*)a.w;
  p.codes = (char*)a.codes;
  p.scales = a.scales;
  p.N = a.N;
  p.S = a.S;
  p.R = a.block_rows;
  p.nblk = (a.S + a.block_rows - 1) / a.block_rows;
  if (a.layout == QFA_BNSD) {
    p.x_row = a.D;
    p.x_head = (long)a.S * a.D;
    p.c_row = a.D;
    p.c_head = (long)a.S * a.D;
  } else {
    p.x_row = (long)a.N * a.D;
    p.x_head = a.D;
    p.c_row = (long)a.N * a.D;
    p.c_head = a.D;
  }
  p.x_batch = (long)a.N * a.S * a.D;
  p.c_batch = (long)a.N * a.S * a.D;
  p.scale_f16 = a.scale_dtype == QFA_F16;
  p.c16 = ((uintptr_t)a.codes % 16 == 0) && (p.c_row % 16 == 0) && (p.c_head % 16 == 0) && (p.c_batch % 16 == 0);
  const long grid = (long)a.B * a.N * p.nblk;
  if (grid == 0) return hipSuccess;
  if (grid > 0x7FFFFFFFL) return hipErrorInvalidValue;
  const int w = a.block_rows > 32 * kRotWaves ? 2 : 1;  // groups of 4 wavefronts
  const bool bf = a.x_dtype == QFA_BF16;
  if (a.D == 64) {
    return bf ? launch_rot_qt<64, true>(p, a.qtype, grid, w, stream)
              : launch_rot_qt<64, false>(p, a.qtype, grid, w, stream);
  }
  return bf ? launch_rot_qt<128, true>(p, a.qtype, grid, w, stream)
            : launch_rot_qt<128, false>(p, a.qtype, grid, w, stream);
}

}  // namespace qfa
