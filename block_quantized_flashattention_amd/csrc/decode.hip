// Decode attention: one query token per sequence against an INT8 or packed
// INT4 KV cache with block scales (gfx950).
//
// What it computes ([Ascend-INT8] INT8-operator section 3: the decode KV
// cache is stored as INT8 and attention reads it without writing a
// dequantized copy; [FA-INT8/INT4] INT4 layer for the INT4 codes):
//   o_bh = sum_{j < L_b} softmax_j(softmax_scale * q_bh . (sk_j Kc_j)) * sv_j Vc_j
//
// Design (HBM-bound: every valid cache byte is read once):
//   * Split-K: a workgroup of 8 wavefronts owns one (batch, query head,
//     1024-token chunk); each wavefront owns 128 consecutive tokens (short
//     per-wavefront score arrays keep the registers low, so more wavefronts
//     are resident per SIMD to cover the HBM latency). Chunks
//     past a sequence's length exit at once. A second small kernel merges the
//     chunks' partial (max, sum, o) by log-sum-exp; a sequence that fits one
//     chunk is written directly.
//   * Lane geometry: a 16-byte load per lane, LPT = row_bytes/16 lanes per
//     token, so one wavefront load covers 64/LPT consecutive tokens; loads are
//     issued four at a time ahead of their use.
//   * Two passes per 128 tokens: all scores first (a per-lane partial dot
//     product, then a DPP butterfly over the LPT lanes of the token), their
//     max, then exp2 and the V accumulation. The first V loads are issued
//     while the last keys are scored, so their latency overlaps that work.
//     Every lane accumulates o for its own channels over its own tokens; the
//     token groups are then summed by a reduce-scatter across the lanes (each
//     exchange halves what a lane holds), which leaves every lane a slice of
//     the channel sums to write.
//   * With an fp16 query, INT8 K codes are converted exactly to packed fp16
//     (the byte goes into the mantissa of 1024 + byte) and dotted with
//     v_dot2_f32_f16 (fp32 accumulation); V codes are converted with the
//     unsigned-byte converter after flipping the sign bit (code + 128) and
//     accumulated in fp32. Packed INT4, which carries twice the codes per
//     byte, stays in fp16 pairs for both: one shift and mask put a nibble
//     pair under the exponent of 1024 (1032 + code, exact); keys pair
//     channels e and e + 4 of each group of 8 (the query is paired the same
//     way) and drop 1032 * sum(q) once per token; values pair one channel of
//     two tokens against the two fp16 weights and drop 1032 times the sum of
//     those weights once per output channel. With an fp32/bf16 query the
//     codes go to fp32 (offset 128 or 8, removed once per channel).
//   * When one scale block covers a wavefront's 128 tokens (block size a
//     multiple of 128), its K and V scales are two scalar loads.
#include <mutex>

#include "qfa_device.h"
#include "qfa_launch.h"

namespace qfa {
namespace {

// Split-K partials of qfa_decode_noalloc, for callers that cannot allocate.
// Each device holds its own copy from library load until the process ends.
// Host code must never pass this name to a kernel (on the host it is only a
// stand-in): decode_scratch() looks up each device's address once.
static __device__ __align__(256) float scratch[kDecodeScratchBytes / sizeof(float)];

constexpr int kDecWaves = 8;
constexpr int kWaveTokens = kDecodeChunk / kDecWaves;  // 128
constexpr int kGroup = 4;                              // loads issued together

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
};

__device__ __forceinline__ void store_out(void* out, long i, float v, int dt) {
  if (dt == QFA_F32) ((float*)out)[i] = v;
  else if (dt == QFA_F16) ((uint16_t*)out)[i] = (uint16_t)f32_to_f16_bits(v);
  else ((uint16_t*)out)[i] = (uint16_t)f32_to_bf16_bits(v);
}

// Sum over groups of LPT consecutive lanes (LPT in {2, 4, 8}) with DPP moves.
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

// Four signed bytes as two exact fp16 pairs (1024 + (byte ^ 0x80) - 1152).
__device__ __forceinline__ void i8x4_to_h(uint32_t w, f16x2& lo, f16x2& hi) {
  const uint32_t u = w ^ 0x80808080u;
  const uint32_t a = __builtin_amdgcn_perm(0x64646464u, u, 0x05010400u);
  const uint32_t b = __builtin_amdgcn_perm(0x64646464u, u, 0x07030602u);
  const f16x2 bias = {(_Float16)1152.0f, (_Float16)1152.0f};
  lo = __builtin_bit_cast(f16x2, a) - bias;
  hi = __builtin_bit_cast(f16x2, b) - bias;
}

// The nibbles at bits 0-3 and 16-19 of w (two's-complement codes) as an fp16
// pair 1032 + code, exact: flip the sign bit, keep the nibbles, set the
// exponent of 1024.
__device__ __forceinline__ uint32_t i4_pair_h(uint32_t w) {
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

// Raw buffer resource over [base, base + bytes): loads past the end return
// zero. The last word is the gfx9 default (32-bit data format, no swizzle).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const uint8_t* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base), (short)0, bytes, 0x00020000);
}

// Packed INT4 with an fp16 query and block scales asks for six wavefronts per
// SIMD, i.e. three workgroups per CU (at most 80 VGPRs): its rows are half as
// long, so more of them must be in flight to cover the HBM latency.
template <int D, bool INT4, bool QF16, bool BLOCK_SCALE>
__global__ __launch_bounds__(64 * kDecWaves, INT4 && QF16 && BLOCK_SCALE ? 6 : 2)
void decode_split_kernel(DecParams p) {
  constexpr int kRowBytes = INT4 ? D / 2 : D;
  constexpr int LPT = kRowBytes / 16;        // lanes per token
  constexpr int EPL = INT4 ? 32 : 16;        // channels per lane
  constexpr int TPS = 64 / LPT;              // tokens per wavefront load
  constexpr int NSUB = kWaveTokens / TPS;    // loads per lane per wavefront chunk
  constexpr int NG = NSUB / kGroup;
  constexpr float kOff = INT4 ? 8.0f : 128.0f;
  static_assert(NSUB % kGroup == 0, "load groups");
  constexpr int NF = EPL / (64 / LPT);  // channels per lane after the token-group reduction
  static_assert(NF >= 1 && EPL % (64 / LPT) == 0, "reduce-scatter");
  __shared__ float red_m[kDecWaves], red_l[kDecWaves];
  __shared__ float red_o[kDecWaves][D];

  const int split = blockIdx.x;
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  const int L = min(max(p.lens[b], 1), p.S_max);
  const int nsplit = (L + kDecodeChunk - 1) / kDecodeChunk;
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

  const int t_begin = split * kDecodeChunk + wave * kWaveTokens;
  const int t_end = min(t_begin + kWaveTokens, L);
  const int t_last = t_end - 1;

  float m_blk = -INFINITY, l_blk = 0.0f, wsum = 0.0f;
  float o[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) o[e] = 0.0f;
  float sk_blk = 1.0f, sv_blk = 1.0f;

  if (t_begin < t_end) {
    // ---- scores: sc[j] for token t_begin + j*TPS + tg (log2 units) ----
    float sc[NSUB];
    uint4 kw[2][kGroup];
    // Rows [0, L) of this (batch, KV head) through buffer resources: one
    // 32-bit offset per lane (the host keeps every offset below 2^31), and
    // rows at or past L read as zero, so no clamp is needed (their scores
    // are masked).
    const int span = (L - 1) * (int)p.c_row + kRowBytes;
    const auto krs = rows_rsrc(p.k + cbase, span);
    const auto vrs = rows_rsrc(p.v + cbase, span);
    const int loff = (t_begin + tg) * (int)p.c_row + dc * 16;
    auto bload = [&](__amdgpu_buffer_rsrc_t rs, int j) {
      const auto r = __builtin_amdgcn_raw_buffer_load_b128(rs, loff + j * TPS * (int)p.c_row, 0, 0);
      return make_uint4(r[0], r[1], r[2], r[3]);
    };
    auto kload = [&](uint4* dst, int g) {
#pragma unroll
      for (int i = 0; i < kGroup; ++i) dst[i] = bload(krs, g * kGroup + i);
    };
    uint4 vw[2][kGroup];
    auto vload = [&](uint4* dst, int g) {
#pragma unroll
      for (int i = 0; i < kGroup; ++i) dst[i] = bload(vrs, g * kGroup + i);
    };
    kload(kw[0], 0);
    if constexpr (BLOCK_SCALE) {
      sk_blk = load_scale(p.ks, sbase + t_begin / p.kv_block, p.kv_scale_f16);
      sv_blk = load_scale(p.vs, sbase + t_begin / p.kv_block, p.kv_scale_f16);
    }
    prep_q();
    const float csk = p.scale_log2 * sk_blk;
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      if (g + 1 < NG) kload(kw[(g + 1) & 1], g + 1);
      else vload(vw[0], 0);  // first V group, in flight while the last keys are scored
#pragma unroll
      for (int i = 0; i < kGroup; ++i) {
        const int j = g * kGroup + i;
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
                kh[4 * i + sft] = __builtin_bit_cast(f16x2, i4_pair_h(ww[i] >> (4 * sft)));
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
        float c = csk;
        if constexpr (!BLOCK_SCALE) {
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
        static_assert(kGroup % 2 == 0, "token pairs");
        const f16x2 one = {(_Float16)1.0f, (_Float16)1.0f};
#pragma unroll
        for (int i = 0; i < kGroup; i += 2) {
          const int j = g * kGroup + i;
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
                  wp, __builtin_bit_cast(f16x2, i4_pair_h(r0 >> sft)), o[8 * d + c], false);
              o[8 * d + 4 + c] = __builtin_amdgcn_fdot2(
                  wp, __builtin_bit_cast(f16x2, i4_pair_h(r1 >> sft)), o[8 * d + 4 + c], false);
            }
          }
        }
      } else {
#pragma unroll
        for (int i = 0; i < kGroup; ++i) {
          const int j = g * kGroup + i;
          const float pr = __builtin_amdgcn_exp2f(sc[j] - m_blk);  // 0 for masked tokens
          lp[i & 1] += pr;
          float wt = pr;
          if constexpr (!BLOCK_SCALE) {
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
    for (int e = 0; e < NF; ++e) o[e] = (o[e] - kOffV * wsum) * sv_blk;
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
  for (int w = 1; w < kDecWaves; ++w) M = fmaxf(M, red_m[w]);
  float c[kDecWaves];
  float Lsum = 0.0f;
#pragma unroll
  for (int w = 0; w < kDecWaves; ++w) {
    c[w] = red_m[w] == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(red_m[w] - M);
    Lsum += red_l[w] * c[w];
  }
  const long obase = (long)b * p.q_batch + (long)h * p.q_head;
  if (nsplit == 1) {
    const float inv = 1.0f / Lsum;
    for (int d = lane; d < D; d += 64) {
      float acc = 0.0f;
#pragma unroll
      for (int w = 0; w < kDecWaves; ++w) acc += red_o[w][d] * c[w];
      store_out(p.out, obase + d, acc * inv, p.out_dtype);
    }
    return;
  }
  float* part = p.ws + (((long)b * p.Hq + h) * p.max_splits + split) * (D + 2);
  for (int d = lane; d < D; d += 64) {
    float acc = 0.0f;
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w) acc += red_o[w][d] * c[w];
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
  const int nsplit = (L + kDecodeChunk - 1) / kDecodeChunk;
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
hipError_t launch_dec4(const DecParams& p, int B, hipStream_t st) {
  decode_split_kernel<D, INT4, QF16, BS><<<dim3(p.max_splits, p.Hq, B), 64 * kDecWaves, 0, st>>>(p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (p.max_splits > 1) {
    decode_reduce_kernel<D><<<dim3(p.Hq, B), 64, 0, st>>>(p);
    e = hipGetLastError();
  }
  return e;
}

template <int D, bool INT4>
hipError_t launch_dec(const DecParams& p, int B, hipStream_t st) {
  const bool qf16 = p.q_dtype == QFA_F16;
  const bool bs = p.kv_block % kWaveTokens == 0;
  if (qf16) return bs ? launch_dec4<D, INT4, true, true>(p, B, st) : launch_dec4<D, INT4, true, false>(p, B, st);
  return bs ? launch_dec4<D, INT4, false, true>(p, B, st) : launch_dec4<D, INT4, false, false>(p, B, st);
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
  if (a.layout == QFA_BNSD) {
    p.c_row = rb;
    p.c_head = (long)a.S_max * rb;
  } else {
    p.c_row = (long)a.Hkv * rb;
    p.c_head = rb;
  }
  p.c_batch = (long)a.Hkv * a.S_max * rb;
  p.q_head = a.D;
  p.q_batch = (long)a.Hq * a.D;
  p.kv_block = a.kv_block;
  p.nkblk = (a.S_max + a.kv_block - 1) / a.kv_block;
  p.kv_scale_f16 = a.kv_scale_dtype == QFA_F16;
  p.q_dtype = a.q_dtype;
  p.out_dtype = a.out_dtype;
  p.scale_log2 = a.softmax_scale * kLog2e;
  const bool int4 = a.kv_qtype == QFA_INT4;
  if (a.D == 64) return int4 ? launch_dec<64, true>(p, a.B, stream) : launch_dec<64, false>(p, a.B, stream);
  return int4 ? launch_dec<128, true>(p, a.B, stream) : launch_dec<128, false>(p, a.B, stream);
}

}  // namespace qfa
