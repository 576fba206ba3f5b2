// C ABI of libqfa: argument validation and dispatch to the kernel launchers.
// Every check runs on the host before any HIP call, so an invalid call
// returns its status without touching the device.
#include <stdint.h>

#include "qfa.h"
#include "qfa_launch.h"

namespace {

bool valid_float(int t) { return t == QFA_F32 || t == QFA_F16 || t == QFA_BF16; }
bool valid_qtype(int t) { return t == QFA_INT8 || t == QFA_FP8_E4M3 || t == QFA_INT4; }
bool valid_layout(int t) { return t == QFA_BNSD || t == QFA_BSND; }
bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

int from_hip(hipError_t e) { return e == hipSuccess ? QFA_OK : QFA_ERR_HIP; }

// Validation shared by the single and multi-tensor quantizer entry points.
int check_quant(const void* x, int x_dtype, int B, int N, int S, int D, int layout,
                int block_rows, int qtype, const void* codes, const void* scales,
                int scale_dtype) {
  if (!valid_float(x_dtype) || !valid_layout(layout) || !valid_qtype(qtype) ||
      (scale_dtype != QFA_F32 && scale_dtype != QFA_F16))
    return QFA_ERR_ENUM;
  if (B < 0 || N < 0 || S < 0 || D < 8 || D > 1024 || D % 8 != 0 || block_rows < 1)
    return QFA_ERR_SHAPE;
  if ((long)B * N * S == 0) return QFA_OK;
  if (!x || !codes || !scales) return QFA_ERR_NULL;
  if (!aligned(x, 16) || !aligned(codes, qtype == QFA_INT4 ? 4 : 8) ||
      !aligned(scales, scale_dtype == QFA_F16 ? 2 : 4))
    return QFA_ERR_UNSUPPORTED;
  return QFA_OK;
}


}  // namespace

extern "C" {

int qfa_version(void) { return 100; }

const char* qfa_status_string(int status) {
  switch (status) {
    case QFA_OK: return "ok";
    case QFA_ERR_NULL: return "a required pointer is NULL";
    case QFA_ERR_SHAPE: return "a size is out of range or inconsistent";
    case QFA_ERR_ENUM: return "an enumeration value is unknown";
    case QFA_ERR_UNSUPPORTED: return "valid combination not implemented by this build";
    case QFA_ERR_WORKSPACE: return "decode workspace missing or too small";
    case QFA_ERR_HIP: return "HIP runtime error at launch";
    case QFA_ERR_SCRATCH: return "request exceeds the library's static decode scratch";
    default: return "unknown status";
  }
}


int qfa_block_quant(const void* x, int x_dtype, int B, int N, int S, int D, int layout,
                    int block_rows, int qtype, void* codes, void* scales, int scale_dtype,
                    void* stream) {
  const int st = check_quant(x, x_dtype, B, N, S, D, layout, block_rows, qtype, codes, scales,
                             scale_dtype);
  if (st != QFA_OK || (long)B * N * S == 0) return st;
  qfa::QuantArgs a{x, x_dtype, B, N, S, D, layout, block_rows, qtype, codes, scales, scale_dtype};
  return from_hip(qfa::launch_block_quant(a, (hipStream_t)stream));
}

int qfa_block_quant_multi(const qfa_quant_job* jobs, int njobs, void* stream) {
  if (njobs < 0 || njobs > QFA_MAX_QUANT_JOBS) return QFA_ERR_SHAPE;
  if (njobs == 0) return QFA_OK;
  if (!jobs) return QFA_ERR_NULL;
  qfa::QuantArgs a[QFA_MAX_QUANT_JOBS];
  int n = 0;
  for (int i = 0; i < njobs; ++i) {
    const qfa_quant_job& j = jobs[i];
    const int st = check_quant(j.x, j.x_dtype, j.B, j.N, j.S, j.D, j.layout, j.block_rows,
                               j.qtype, j.codes, j.scales, j.scale_dtype);
    if (st != QFA_OK) return st;
    if ((long)j.B * j.N * j.S == 0) continue;
    a[n++] = qfa::QuantArgs{j.x, j.x_dtype, j.B, j.N, j.S, j.D, j.layout, j.block_rows, j.qtype,
                            j.codes, j.scales, j.scale_dtype};
  }
  if (n == 0) return QFA_OK;
  return from_hip(qfa::launch_block_quant_multi(a, n, (hipStream_t)stream));
}

int qfa_rotate_block_quant(const void* x, int x_dtype, const void* w, int B, int N, int S, int D,
                           int layout, int block_rows, int qtype, void* codes, void* scales,
                           int scale_dtype, void* stream) {
  const int st = check_quant(x, x_dtype, B, N, S, D, layout, block_rows, qtype, codes, scales,
                             scale_dtype);
  if (st != QFA_OK) return st;
  if ((x_dtype != QFA_F16 && x_dtype != QFA_BF16) || (D != 64 && D != 128) ||
      qtype == QFA_INT4 || block_rows % 32 != 0 || block_rows > 256)
    return QFA_ERR_UNSUPPORTED;
  if ((long)B * N * S == 0) return QFA_OK;
  if (!w) return QFA_ERR_NULL;
  if (!aligned(w, 16) || !aligned(codes, 4)) return QFA_ERR_UNSUPPORTED;
  qfa::RotQuantArgs a{x, x_dtype, w, B, N, S, D, layout, block_rows, qtype, codes, scales,
                      scale_dtype};
  return from_hip(qfa::launch_rotate_block_quant(a, (hipStream_t)stream));
}

// Checks of one cache's arguments for qfa_kv_append and qfa_kv_append_kv;
// QFA_OK with *empty set when B * H == 0 (nothing to launch).
static int kv_append_check(const void* x, int x_dtype, const int32_t* positions, void* codes,
                           void* scales, int B, int H, int S_max, int D, int layout, int kv_block,
                           int qtype, int scale_dtype, bool* empty) {
  *empty = false;
  if (!valid_float(x_dtype) || !valid_layout(layout) || !valid_qtype(qtype) ||
      (scale_dtype != QFA_F32 && scale_dtype != QFA_F16))
    return QFA_ERR_ENUM;
  if (B < 0 || H < 0 || S_max < 1 || D < 8 || D % 8 != 0 || kv_block < 1) return QFA_ERR_SHAPE;
  if (qtype == QFA_FP8_E4M3 || D > (qtype == QFA_INT4 ? 512 : 256)) return QFA_ERR_UNSUPPORTED;
  if ((long)B * H == 0) {
    *empty = true;
    return QFA_OK;
  }
  if (!x || !positions || !codes || !scales) return QFA_ERR_NULL;
  if (!aligned(x, x_dtype == QFA_F32 ? 4 : 2) || !aligned(positions, 4) ||
      !aligned(scales, scale_dtype == QFA_F16 ? 2 : 4))
    return QFA_ERR_UNSUPPORTED;
  return QFA_OK;
}

int qfa_kv_append(const void* x, int x_dtype, const int32_t* positions, void* codes, void* scales,
                  int B, int H, int S_max, int D, int layout, int kv_block, int qtype,
                  int scale_dtype, void* stream) {
  bool empty;
  const int st = kv_append_check(x, x_dtype, positions, codes, scales, B, H, S_max, D, layout,
                                 kv_block, qtype, scale_dtype, &empty);
  if (st != QFA_OK || empty) return st;
  qfa::AppendArgs a{x, x_dtype, positions, codes, scales, B, H, S_max, D, layout, kv_block, qtype,
                    scale_dtype, nullptr, nullptr, nullptr};
  return from_hip(qfa::launch_kv_append(a, (hipStream_t)stream));
}

int qfa_kv_append_kv(const void* xk, const void* xv, int x_dtype, const int32_t* positions,
                     void* k_codes, void* k_scales, void* v_codes, void* v_scales, int B, int H,
                     int S_max, int D, int layout, int kv_block, int qtype, int scale_dtype,
                     void* stream) {
  bool empty;
  int st = kv_append_check(xk, x_dtype, positions, k_codes, k_scales, B, H, S_max, D, layout,
                           kv_block, qtype, scale_dtype, &empty);
  if (st != QFA_OK || empty) return st;
  st = kv_append_check(xv, x_dtype, positions, v_codes, v_scales, B, H, S_max, D, layout,
                       kv_block, qtype, scale_dtype, &empty);
  if (st != QFA_OK) return st;
  qfa::AppendArgs a{xk, x_dtype, positions, k_codes, k_scales, B, H, S_max, D, layout, kv_block,
                    qtype, scale_dtype, xv, v_codes, v_scales};
  return from_hip(qfa::launch_kv_append(a, (hipStream_t)stream));
}

// Validation shared by the two forward entry points; QFA_OK with *empty set
// when there is nothing to compute.
static int check_fwd(const void* q_codes, const void* q_scales, int q_qtype, int q_block,
                     int q_scale_dtype, const void* k_codes, const void* k_scales, int k_qtype,
                     const void* v_codes, const void* v_scales, int v_qtype, int kv_block,
                     int kv_scale_dtype, int B, int Hq, int Hkv, int Sq, int Sk, int D,
                     int layout, int causal, float softmax_scale, const void* out,
                     int out_dtype, bool* empty) {
  *empty = false;
  if (!valid_qtype(q_qtype) || !valid_qtype(k_qtype) || !valid_qtype(v_qtype) ||
      !valid_layout(layout) || !valid_float(out_dtype) ||
      (q_scale_dtype != QFA_F32 && q_scale_dtype != QFA_F16) ||
      (kv_scale_dtype != QFA_F32 && kv_scale_dtype != QFA_F16))
    return QFA_ERR_ENUM;
  if (B < 0 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || Sq < 0 || Sk < 0 || q_block < 1 ||
      kv_block < 1 || (causal != 0 && causal != 1))
    return QFA_ERR_SHAPE;
  if (D != 64 && D != 128) return QFA_ERR_UNSUPPORTED;
  if (causal && Sq != Sk) return QFA_ERR_UNSUPPORTED;
  if (B == 0 || Sq == 0) {
    *empty = true;
    return QFA_OK;
  }
  if (Sk < 1) return QFA_ERR_SHAPE;
  if (!(softmax_scale == softmax_scale) || softmax_scale < 0.0f || softmax_scale > 3.0e38f)
    return QFA_ERR_SHAPE;
  // Compiled code-type combinations (Q, K, V).
  const bool ok_types =
      (q_qtype == QFA_INT8 && k_qtype == QFA_INT8 && v_qtype == QFA_INT8) ||
      (q_qtype == QFA_INT8 && k_qtype == QFA_INT4 && v_qtype == QFA_INT4) ||
      (q_qtype == QFA_INT8 && k_qtype == QFA_INT8 && v_qtype == QFA_INT4) ||
      (q_qtype == QFA_FP8_E4M3 && k_qtype == QFA_FP8_E4M3 && v_qtype == QFA_FP8_E4M3);
  if (!ok_types) return QFA_ERR_UNSUPPORTED;
  if (!q_codes || !q_scales || !k_codes || !k_scales || !v_codes || !v_scales || !out)
    return QFA_ERR_NULL;
  // The kernel addresses K/V rows of one head with 32-bit offsets.
  const long kv_row_bytes = (long)(layout == QFA_BSND ? Hkv : 1) * D;
  if ((long)Sk * kv_row_bytes >= (1L << 32)) return QFA_ERR_UNSUPPORTED;
  if (!aligned(q_codes, 16) || !aligned(k_codes, 16) || !aligned(v_codes, 16) ||
      !aligned(out, 16) || !aligned(q_scales, 4) || !aligned(k_scales, 4) || !aligned(v_scales, 4))
    return QFA_ERR_UNSUPPORTED;
  return QFA_OK;
}

int qfa_fwd(const void* q_codes, const void* q_scales, int q_qtype, int q_block,
            int q_scale_dtype, const void* k_codes, const void* k_scales, int k_qtype,
            const void* v_codes, const void* v_scales, int v_qtype, int kv_block,
            int kv_scale_dtype, int B, int Hq, int Hkv, int Sq, int Sk, int D, int layout,
            int causal, float softmax_scale, void* out, int out_dtype, void* stream) {
  bool empty = false;
  const int st = check_fwd(q_codes, q_scales, q_qtype, q_block, q_scale_dtype, k_codes, k_scales,
                           k_qtype, v_codes, v_scales, v_qtype, kv_block, kv_scale_dtype, B, Hq,
                           Hkv, Sq, Sk, D, layout, causal, softmax_scale, out, out_dtype, &empty);
  if (st != QFA_OK || empty) return st;
  qfa::FwdArgs a{q_codes, q_scales, q_qtype, q_block, q_scale_dtype, k_codes, k_scales, k_qtype,
                 v_codes, v_scales, v_qtype, kv_block, kv_scale_dtype, B, Hq, Hkv, Sq, Sk, D,
                 layout, causal, softmax_scale, out, out_dtype};
  return from_hip(qfa::launch_fwd(a, (hipStream_t)stream));
}

size_t qfa_fwd_lowp_workspace_bytes(int B, int Hq, int Hkv, int Sq) {
  if (B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || Sq < 1) return 0;
  return qfa::fwd_lowp_workspace_bytes(B, Hq, Hkv, Sq);
}

int qfa_fwd_lowp(const void* q_codes, const void* q_scales, int q_qtype, int q_block,
                 int q_scale_dtype, const void* k_codes, const void* k_scales, int k_qtype,
                 const void* v_codes, const void* v_scales, int v_qtype, int kv_block,
                 int kv_scale_dtype, int B, int Hq, int Hkv, int Sq, int Sk, int D, int layout,
                 int causal, float softmax_scale, void* out, int out_dtype, void* workspace,
                 size_t workspace_bytes, void* stream) {
  bool empty = false;
  const int st = check_fwd(q_codes, q_scales, q_qtype, q_block, q_scale_dtype, k_codes, k_scales,
                           k_qtype, v_codes, v_scales, v_qtype, kv_block, kv_scale_dtype, B, Hq,
                           Hkv, Sq, Sk, D, layout, causal, softmax_scale, out, out_dtype, &empty);
  if (st != QFA_OK || empty) return st;
  // e4m3 Q/K/V with block scales: K/V blocks covering whole 64-key tiles.
  if (q_qtype != QFA_FP8_E4M3 || kv_block % 64 != 0) return QFA_ERR_UNSUPPORTED;
  const size_t need = qfa::fwd_lowp_workspace_bytes(B, Hq, Hkv, Sq);
  if (!workspace || workspace_bytes < need) return QFA_ERR_WORKSPACE;
  if (!aligned(workspace, 8)) return QFA_ERR_UNSUPPORTED;
  qfa::FwdArgs a{q_codes, q_scales, q_qtype, q_block, q_scale_dtype, k_codes, k_scales, k_qtype,
                 v_codes, v_scales, v_qtype, kv_block, kv_scale_dtype, B, Hq, Hkv, Sq, Sk, D,
                 layout, causal, softmax_scale, out, out_dtype};
  return from_hip(qfa::launch_fwd_lowp(a, workspace, (hipStream_t)stream));
}

size_t qfa_decode_workspace_bytes(int B, int Hq, int S_max, int D) {
  if (B < 1 || Hq < 1 || S_max < 1 || (D != 64 && D != 128)) return 0;
  return qfa::decode_workspace_bytes(B, Hq, S_max, D);
}

// Validation shared by the two decode entry points; on QFA_OK, *need holds the
// bytes of split-K partials the call will write.
static int check_decode(const void* q, int q_dtype, int B, int Hq, int Hkv, int D,
                        const void* k_cache, const void* v_cache, const void* k_scales,
                        const void* v_scales, int kv_qtype, int kv_block, int kv_scale_dtype,
                        int S_max, int layout, const int32_t* seq_lens, float softmax_scale,
                        const void* out, int out_dtype, size_t* need) {
  *need = 0;
  if (!valid_float(q_dtype) || !valid_float(out_dtype) || !valid_qtype(kv_qtype) ||
      !valid_layout(layout) || (kv_scale_dtype != QFA_F32 && kv_scale_dtype != QFA_F16))
    return QFA_ERR_ENUM;
  if (B < 0 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || S_max < 1 || kv_block < 1)
    return QFA_ERR_SHAPE;
  if (D != 64 && D != 128) return QFA_ERR_UNSUPPORTED;
  if (kv_qtype == QFA_FP8_E4M3) return QFA_ERR_UNSUPPORTED;
  if (Hq / Hkv > 16) return QFA_ERR_UNSUPPORTED;
  // The kernel addresses the rows of one (batch, KV head) with 32-bit offsets.
  const long row_stride = (layout == QFA_BNSD ? 1L : (long)Hkv) * (kv_qtype == QFA_INT4 ? D / 2 : D);
  if (((long)S_max + qfa::kDecodeChunk) * row_stride > INT32_MAX) return QFA_ERR_UNSUPPORTED;
  if (B == 0) return QFA_OK;
  if (!(softmax_scale == softmax_scale) || softmax_scale < 0.0f || softmax_scale > 3.0e38f)
    return QFA_ERR_SHAPE;
  if (!q || !k_cache || !v_cache || !k_scales || !v_scales || !seq_lens || !out)
    return QFA_ERR_NULL;
  if (!aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(q, 4) || !aligned(out, 4) ||
      !aligned(seq_lens, 4))
    return QFA_ERR_UNSUPPORTED;
  // Partials are written only when a sequence spans more than one chunk.
  *need = S_max > qfa::kDecodeChunk ? qfa::decode_workspace_bytes(B, Hq, S_max, D) : 0;
  return QFA_OK;
}

int qfa_decode(const void* q, int q_dtype, int B, int Hq, int Hkv, int D, const void* k_cache,
               const void* v_cache, const void* k_scales, const void* v_scales, int kv_qtype,
               int kv_block, int kv_scale_dtype, int S_max, int layout, const int32_t* seq_lens,
               float softmax_scale, void* out, int out_dtype, void* workspace,
               size_t workspace_bytes, void* stream) {
  size_t need = 0;
  const int st = check_decode(q, q_dtype, B, Hq, Hkv, D, k_cache, v_cache, k_scales, v_scales,
                              kv_qtype, kv_block, kv_scale_dtype, S_max, layout, seq_lens,
                              softmax_scale, out, out_dtype, &need);
  if (st != QFA_OK || B == 0) return st;
  if (need > 0 && (!workspace || workspace_bytes < need)) return QFA_ERR_WORKSPACE;
  if (!aligned(workspace, 16)) return QFA_ERR_UNSUPPORTED;
  qfa::DecodeArgs a{q, q_dtype, B, Hq, Hkv, D, k_cache, v_cache, k_scales, v_scales, kv_qtype,
                    kv_block, kv_scale_dtype, S_max, layout, seq_lens, softmax_scale, out,
                    out_dtype, workspace};
  return from_hip(qfa::launch_decode(a, (hipStream_t)stream));
}

size_t qfa_decode_noalloc_max_bytes(void) { return qfa::kDecodeScratchBytes; }

int qfa_decode_noalloc(const void* q, int q_dtype, int B, int Hq, int Hkv, int D,
                       const void* k_cache, const void* v_cache, const void* k_scales,
                       const void* v_scales, int kv_qtype, int kv_block, int kv_scale_dtype,
                       int S_max, int layout, const int32_t* seq_lens, float softmax_scale,
                       void* out, int out_dtype, void* stream) {
  size_t need = 0;
  const int st = check_decode(q, q_dtype, B, Hq, Hkv, D, k_cache, v_cache, k_scales, v_scales,
                              kv_qtype, kv_block, kv_scale_dtype, S_max, layout, seq_lens,
                              softmax_scale, out, out_dtype, &need);
  if (st != QFA_OK || B == 0) return st;
  if (need > qfa::kDecodeScratchBytes) return QFA_ERR_SCRATCH;
  void* ws = nullptr;
  const hipError_t e = qfa::decode_scratch((hipStream_t)stream, &ws);
  if (e != hipSuccess) return QFA_ERR_HIP;
  qfa::DecodeArgs a{q, q_dtype, B, Hq, Hkv, D, k_cache, v_cache, k_scales, v_scales, kv_qtype,
                    kv_block, kv_scale_dtype, S_max, layout, seq_lens, softmax_scale, out,
                    out_dtype, ws};
  return from_hip(qfa::launch_decode(a, (hipStream_t)stream));
}

}  // extern "C"
