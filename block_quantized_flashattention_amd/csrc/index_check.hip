// Host-side check of the attention forward's address arithmetic: for one
// problem shape, walk every workgroup of the launch, every thread and every
// tile it fetches (prefetches past the end included), form each code and
// scale address with the kernel's own index functions, and test it against
// the extent of its tensor. Also checks that every (batch, head, query row)
// is computed by exactly one lane pair. Built as its own host-only library;
// nothing here runs on the GPU.
#include <stdint.h>
#include <stdio.h>

#include <vector>

#include "qfa_index.h"

namespace {

// Kinds of violation, reported as a bit mask.
enum : int {
  kQCodes = 1, kKCodes = 2, kVCodes = 4, kQScales = 8, kKVScales = 16, kOut = 32,
  kCoverage = 64, kWorkItem = 128
};

struct Report {
  long violations = 0;
  int kinds = 0;
  char* msg;
  int msg_len;
  template <typename... A>
  void fail(int kind, const char* fmt, A... a) {
    kinds |= kind;
    if (violations++ == 0 && msg && msg_len > 0) snprintf(msg, msg_len, fmt, a...);
  }
};

}  // namespace

// Returns the number of out-of-range addresses and coverage errors (0: all
// in range, every output row computed once), or -1 for a shape the forward
// does not take. Each tensor's extent is taken `shrink` bytes (or 16-bit
// scale elements) short of its true size: with shrink = 1 every tensor whose
// last byte some thread reads shows up. `kinds` (may be null) receives the
// mask of violated kinds, `msg` (may be null) the first violation.
extern "C" __attribute__((visibility("default"))) long qfa_ixcheck_fwd(
    int B, int Hq, int Hkv, int Sq, int Sk, int D, int bsnd, int k_int4, int v_int4, int q_block,
    int kv_block, int q_scale_f16, int kv_scale_f16, int causal, int shrink, int* kinds, char* msg,
    int msg_len) {
  using namespace qfa::ix;
  if (B < 1 || Hkv < 1 || Hq % Hkv || Sq < 1 || Sk < 1 || (D != 64 && D != 128) || q_block < 1 ||
      kv_block < 1 || (causal && Sq != Sk))
    return -1;
  Report rep{0, 0, msg, msg_len};
  const FwdShape f = fwd_shape(B, Hq, Hkv, Sq, Sk, D, bsnd, k_int4, v_int4, q_block, kv_block);
  const long q_bytes = (long)B * Hq * Sq * D - shrink;
  const long o_elems = (long)B * Hq * Sq * D - shrink;
  const long k_bytes = (long)B * Hkv * Sk * (k_int4 ? D / 2 : D) - shrink;
  const long v_bytes = (long)B * Hkv * Sk * (v_int4 ? D / 2 : D) - shrink;
  const long qs_elems16 = (long)B * Hq * f.nqblk * (q_scale_f16 ? 1 : 2) - shrink;
  const long kvs_elems16 = (long)B * Hkv * f.nkblk * (kv_scale_f16 ? 1 : 2) - shrink;
  const int k_src = fwd_k_src(D, k_int4), v_src = fwd_v_src(D, v_int4);
  if (f.grid > 0x7FFFFFFF) return -1;
  std::vector<uint8_t> seen((size_t)B * Hq * Sq, 0);

  for (int id = 0; id < (int)f.grid; ++id) {
    const FwdItem it = fwd_item(id, B, Hkv, f.n_hg, f.n_rb, f.xcd_order, causal);
    if (it.b < 0 || it.b >= B || it.kvh < 0 || it.kvh >= Hkv || it.hg < 0 || it.hg >= f.n_hg ||
        it.rb < 0 || it.rb >= f.n_rb) {
      rep.fail(kWorkItem, "workgroup %d: work item (%d, %d, %d, %d) out of range", id, it.b, it.kvh, it.hg,
               it.rb);
      continue;
    }
    // Query rows: code bytes [row start, + D), the scale of the row's block,
    // output rows (written for rows < Sq only).
    for (int wave = 0; wave < kFwdWaves; ++wave) {
      const int h = fwd_head(it, f.group, f.hpw, wave);
      if (h < it.kvh * f.group || h >= (it.kvh + 1) * f.group)
        rep.fail(kWorkItem, "workgroup %d wave %d: head %d outside KV head %d's group", id, wave, h, it.kvh);
      for (int lane = 0; lane < 64; ++lane) {
        const int qrow = fwd_row(it, f.rph, f.hpw, wave, lane);
        const int rr = fwd_read_row(qrow, Sq);
        const long qo = (long)it.b * f.q.batch + (long)h * f.q.head + (long)rr * f.q.row;
        if (qo < 0 || qo + D > q_bytes) rep.fail(kQCodes, "Q codes: byte %ld + %d of %ld", qo, D, q_bytes);
        long i0, i1;
        scale_halves(((long)it.b * Hq + h) * f.nqblk + rr / q_block, q_scale_f16, i0, i1);
        if (i0 < 0 || i1 >= qs_elems16) rep.fail(kQScales, "Q scales: element %ld of %ld", i1, qs_elems16);
        if (qrow < Sq && lane < 32) {
          uint8_t& c = seen[((size_t)it.b * Hq + h) * Sq + qrow];
          if (c++) rep.fail(kCoverage, "row %d of head %d (batch %d) computed twice", qrow, h, it.b);
          const long oo = (long)it.b * f.q.batch + (long)h * f.q.head + (long)qrow * f.q.row;
          if (oo < 0 || oo + D > o_elems) rep.fail(kOut, "output: element %ld of %ld", oo + D, o_elems);
        }
      }
    }
    // Key tiles: the loop fetches tiles 0 .. ntiles + 1 (two ahead).
    const int m0 = it.rb * f.rph;
    const int ntiles = fwd_tiles(fwd_key_end(causal, Sk, m0, f.rph));
    const int last_tile = ntiles - 1;
    const long kbase = (long)it.b * f.k.batch + (long)it.kvh * f.k.head;
    const long vbase = (long)it.b * f.v.batch + (long)it.kvh * f.v.head;
    const long sbase = ((long)it.b * Hkv + it.kvh) * f.nkblk;
    for (int t = 0; t <= ntiles + 1; ++t) {
      const int n0 = fwd_tile_n0(t, last_tile);
      for (int tid = 0; tid < kFwdThreads; ++tid) {
        const long ko = kbase + fwd_k_offset(fwd_k_key(n0, tid, Sk), (uint32_t)f.k.row, tid, k_src);
        if (ko < 0 || ko + k_src > k_bytes)
          rep.fail(kKCodes, "K codes: tile %d thread %d byte %ld + %d of %ld", t, tid, ko, k_src, k_bytes);
        for (int r = 0; r < 2; ++r) {
          const long vo =
              vbase + fwd_v_offset(fwd_v_key(n0, tid, r, Sk), (uint32_t)f.v.row, tid, v_src);
          if (vo < 0 || vo + v_src > v_bytes)
            rep.fail(kVCodes, "V codes: tile %d thread %d byte %ld + %d of %ld", t, tid, vo, v_src, v_bytes);
        }
      }
      for (int lane = 0; lane < 64; ++lane) {
        long i0, i1;
        scale_halves(fwd_kv_scale_block(sbase, n0, lane, Sk, kv_block, f.per_key), kv_scale_f16,
                     i0, i1);
        if (i0 < 0 || i1 >= kvs_elems16)
          rep.fail(kKVScales, "K/V scales: tile %d lane %d element %ld of %ld", t, lane, i1, kvs_elems16);
      }
    }
  }
  for (size_t i = 0; i < seen.size(); ++i)
    if (!seen[i]) {
      rep.fail(kCoverage, "row %ld of head %ld (batch %ld) not computed", (long)(i % Sq),
               (long)(i / Sq % Hq), (long)(i / Sq / Hq));
      break;
    }
  if (kinds) *kinds = rep.kinds;
  return rep.violations;
}

// The forward's work decomposition for a launch of this shape: for workgroup
// `id`, out[0..3] = (batch, first query head, number of heads, first row) and
// out[4] = rows per head. Returns the number of workgroups, or -1 for a shape
// the forward does not take.
extern "C" __attribute__((visibility("default"))) long qfa_ixcheck_fwd_item(
    int B, int Hq, int Hkv, int Sq, int causal, int id, int* out) {
  using namespace qfa::ix;
  if (B < 1 || Hkv < 1 || Hq % Hkv || Sq < 1) return -1;
  const FwdShape f = fwd_shape(B, Hq, Hkv, Sq, Sq, 128, false, false, false, 1, 1);
  if (id < 0 || id >= f.grid) return f.grid;
  const FwdItem it = fwd_item(id, B, Hkv, f.n_hg, f.n_rb, f.xcd_order, causal);
  out[0] = it.b;
  out[1] = fwd_head(it, f.group, f.hpw, 0);
  out[2] = f.hpw;
  out[3] = it.rb * f.rph;
  out[4] = f.rph;
  return f.grid;
}
