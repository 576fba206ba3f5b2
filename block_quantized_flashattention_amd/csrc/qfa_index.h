// Work decomposition and address arithmetic of the attention kernels, written
// once and compiled both for the device (the kernels) and for the host (the
// launchers, and a check that enumerates every address a launch forms and
// tests it against the extent of its tensor).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define QFA_HD __host__ __device__ __forceinline__

namespace qfa {
namespace ix {

constexpr int kFwdPairs = 256;  // (query row, head) pairs per forward workgroup
constexpr int kFwdBN = 64;      // keys per forward tile
constexpr int kFwdThreads = 512;
constexpr int kFwdWaves = 8;
constexpr int kXcds = 8;        // chiplets the hardware deals workgroups over, round robin

QFA_HD int imin(int a, int b) { return a < b ? a : b; }

// Byte (or element) strides of one tensor of H heads and S rows of `row`
// units, BNSD or BSND.
struct Strides {
  long row, head, batch;
};
QFA_HD Strides strides(bool bsnd, int H, int S, long row) {
  return bsnd ? Strides{(long)H * row, row, (long)S * H * row}
              : Strides{row, (long)S * row, (long)H * S * row};
}

// Forward: query heads per workgroup, the largest power of two <= 8 dividing
// the GQA group (they share every K/V tile); each takes kFwdPairs / hpw rows.
QFA_HD int fwd_heads_per_wg(int group) {
  int hpw = 1;
  while (hpw < 8 && group % (2 * hpw) == 0) hpw *= 2;
  return hpw;
}

// Launch geometry of one forward call, derived from the problem alone.
struct FwdShape {
  int group, hpw, rph, n_hg, n_rb, nqblk, nkblk;
  bool xcd_order;  // B * Hkv a multiple of the chiplet count
  bool per_key;    // per-key scales: the K/V block size does not cover whole tiles
  long grid;       // workgroups
  Strides q, k, v; // code strides in bytes (Q and the output share q's, in elements)
};
QFA_HD FwdShape fwd_shape(int B, int Hq, int Hkv, int Sq, int Sk, int D, bool bsnd, bool k_int4,
                          bool v_int4, int q_block, int kv_block) {
  FwdShape f;
  f.group = Hq / Hkv;
  f.hpw = fwd_heads_per_wg(f.group);
  f.rph = kFwdPairs / f.hpw;
  f.n_hg = f.group / f.hpw;
  f.n_rb = (Sq + f.rph - 1) / f.rph;
  f.nqblk = (Sq + q_block - 1) / q_block;
  f.nkblk = (Sk + kv_block - 1) / kv_block;
  f.xcd_order = ((long)B * Hkv) % kXcds == 0;
  f.per_key = kv_block % kFwdBN != 0;
  f.grid = (long)f.n_rb * B * Hkv * f.n_hg;
  f.q = strides(bsnd, Hq, Sq, D);
  f.k = strides(bsnd, Hkv, Sk, k_int4 ? D / 2 : D);
  f.v = strides(bsnd, Hkv, Sk, v_int4 ? D / 2 : D);
  return f;
}

// The work item of workgroup `id`: (batch, KV head, head group, row block).
// Row blocks go longest first under the causal mask. With xcd_order (B * Hkv
// a multiple of 8), the workgroups of one (batch, KV head) stay on one chiplet
// (the hardware deals consecutive ids to the chiplets in turn), so that its
// K/V tiles are read from one L2.
struct FwdItem {
  int b, kvh, hg, rb;
};
QFA_HD FwdItem fwd_item(int id, int B, int Hkv, int n_hg, int n_rb, bool xcd_order, bool causal) {
  const int ngroups = B * Hkv;
  int rank, gidx, hg;
  if (xcd_order) {
    const int xcd = id % kXcds, k = id / kXcds;
    const int per_rank = (ngroups / kXcds) * n_hg;
    rank = k / per_rank;
    const int rem = k % per_rank;
    gidx = (rem / n_hg) * kXcds + xcd;
    hg = rem % n_hg;
  } else {
    const int per_rank = ngroups * n_hg;
    rank = id / per_rank;
    const int rem = id % per_rank;
    gidx = rem / n_hg;
    hg = rem % n_hg;
  }
  return FwdItem{gidx / Hkv, gidx % Hkv, hg, causal ? n_rb - 1 - rank : rank};
}

// Query head and row of lane `lane` of wavefront `wave` (32 rows per
// wavefront, lanes l and l + 32 share a row).
QFA_HD int fwd_head(const FwdItem& it, int group, int hpw, int wave) {
  return it.kvh * group + it.hg * hpw + wave % hpw;
}
QFA_HD int fwd_row(const FwdItem& it, int rph, int hpw, int wave, int lane) {
  return it.rb * rph + 32 * (wave / hpw) + (lane & 31);
}
// Rows past the end read row Sq - 1 (their results are discarded).
QFA_HD int fwd_read_row(int qrow, int Sq) { return imin(qrow, Sq - 1); }

// Keys a row block reads: all, or under the causal mask up to its last row.
QFA_HD int fwd_key_end(bool causal, int Sk, int m0, int rph) {
  return causal ? imin(Sk, m0 + rph) : Sk;
}
QFA_HD int fwd_tiles(int n_end) { return (n_end + kFwdBN - 1) / kFwdBN; }
// First key of tile t; the prefetch runs two tiles ahead and reads the last
// tile again past the end.
QFA_HD int fwd_tile_n0(int t, int last_tile) { return imin(t, last_tile) * kFwdBN; }

// Key rows staged by thread tid for the tile at n0, clamped to the last key:
// K: key tid / 8 (eighth tid % 8 of its row); V: keys 2 (tid % 32) + r.
QFA_HD uint32_t fwd_k_key(int n0, int tid, int Sk) { return (uint32_t)imin(n0 + tid / 8, Sk - 1); }
QFA_HD uint32_t fwd_v_key(int n0, int tid, int r, int Sk) {
  return (uint32_t)imin(n0 + 2 * (tid % 32) + r, Sk - 1);
}
// Source bytes of one staging unit: a K unit is an eighth of a key row, a V
// unit D/16 channels of one key (INT4 codes: half as many bytes).
constexpr QFA_HD int fwd_k_src(int D, bool k_int4) { return k_int4 ? D / 16 : D / 8; }
constexpr QFA_HD int fwd_v_src(int D, bool v_int4) { return v_int4 ? D / 32 : D / 16; }

// Byte offsets, within one (batch, KV head), of those source bytes: k_src
// bytes per K unit, v_src bytes per V unit (channel group tid / 32).
QFA_HD uint32_t fwd_k_offset(uint32_t key, uint32_t k_row, int tid, int k_src) {
  return key * k_row + (uint32_t)(tid % 8) * (uint32_t)k_src;
}
QFA_HD uint32_t fwd_v_offset(uint32_t key, uint32_t v_row, int tid, int v_src) {
  return key * v_row + (uint32_t)(tid / 32) * (uint32_t)v_src;
}

// Scale block read by lane `lane` for the tile at n0: with per-key scales
// (a block size that does not cover whole tiles) the block of key n0 + lane
// (clamped to the last key), else the one block holding the tile.
QFA_HD long fwd_kv_scale_block(long sbase, int n0, int lane, int Sk, int kv_block, bool per_key) {
  if (!per_key) return sbase + n0 / kv_block;
  const int key = imin(n0 + lane, Sk - 1);
  return sbase + (kv_block == 1 ? key : key / kv_block);
}

// The two 16-bit elements a scale is read as: for fp16 the scale itself
// twice, for fp32 its low and high halves. Neither lies past the scale.
QFA_HD void scale_halves(long block, bool f16, long& i0, long& i1) {
  i0 = f16 ? block : 2 * block;
  i1 = f16 ? block : 2 * block + 1;
}

}  // namespace ix
}  // namespace qfa
