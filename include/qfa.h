/*
 * qfa.h -- C ABI of libqfa.so: block-quantized FlashAttention on AMD Instinct
 * MI355X (gfx950).
 *
 * Pages cited (titles shortened):
 *   [FA-INT8/INT4]  "FlashAttention INT8/INT4 quantization" blog post on the
 *                   ops-transformer library (hwcomputing.csdn.net/6a140ce2...).
 *   [OT-Quant]      ops-transformer INT8/INT4 quantized-inference article
 *                   (2048ai.net/6989721354...).
 *   [Ascend-INT8]   "INT8 量化算子：让大模型在昇腾NPU上减肥不掉肉"
 *                   (hwcomputing.csdn.net/6a0dcc10...).
 *   [MindIE-SD]     MindIE-SD quantization feature doc, FA quantization part
 *                   (gitcode.com/Ascend/MindIE-SD, docs/zh/features/quantization.md).
 *
 * Conventions shared by every call:
 *   - Tensor pointers are DEVICE pointers owned by the caller. The library
 *     never frees or keeps them; it allocates no device memory.
 *   - Every call is asynchronous on `stream` (a hipStream_t; NULL means the
 *     default stream). Arguments are validated on the host before any launch;
 *     an invalid call returns a nonzero status and launches nothing.
 *   - A kernel-launch failure returns QFA_ERR_HIP. Faults inside a kernel
 *     surface at the caller's next synchronisation with the stream.
 *   - Enumerations are passed as int. Sizes are elements unless stated.
 *   - Layouts: QFA_BNSD is [batch, heads, seq, dim]; QFA_BSND is
 *     [batch, seq, heads, dim]; both dense, dim fastest. INT4 codes hold two
 *     codes per byte, so their innermost extent is dim/2 bytes.
 *   - A "block" is `block_rows` consecutive sequence rows times all `dim`
 *     channels of one (batch, head); the last block of a sequence may be short.
 *   - The library holds no mutable global state and calls are reentrant,
 *     with one exception: qfa_decode_noalloc works in a static per-device
 *     scratch array (see there).
 */
#ifndef QFA_H
#define QFA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#ifndef QFA_API
#define QFA_API __attribute__((visibility("default")))
#endif

typedef enum {
  QFA_OK = 0,
  QFA_ERR_NULL = 1,         /* a required pointer is NULL */
  QFA_ERR_SHAPE = 2,        /* a size is out of range or inconsistent */
  QFA_ERR_ENUM = 3,         /* an enumeration value is unknown */
  QFA_ERR_UNSUPPORTED = 4,  /* a valid combination this build does not implement */
  QFA_ERR_WORKSPACE = 5,    /* decode workspace missing or too small */
  QFA_ERR_HIP = 6,          /* the HIP runtime reported an error at launch */
  QFA_ERR_SCRATCH = 7       /* qfa_decode_noalloc: the call needs more than the static scratch */
} qfa_status;

typedef enum { QFA_F32 = 0, QFA_F16 = 1, QFA_BF16 = 2 } qfa_float;
typedef enum { QFA_INT8 = 0, QFA_FP8_E4M3 = 1, QFA_INT4 = 2 } qfa_qtype;
typedef enum { QFA_BNSD = 0, QFA_BSND = 1 } qfa_layout;

/* Library version as 10000*major + 100*minor + patch. */
QFA_API int qfa_version(void);

/* Static, NUL-terminated description of a status code (never NULL). */
QFA_API const char* qfa_status_string(int status);

/*
 * qfa_block_quant -- symmetric per-block amax quantization.
 *
 * Defined by [Ascend-INT8] section "对称量化 vs 非对称量化" (scale =
 * max(abs(x))/127, code = round(x/scale) clamped to [-128, 127], zero point
 * 0), [MindIE-SD] FA quantization "块量化" (dynamic block quantization to
 * float8_e4m3fn, Q block 128 rows, K/V block 256 rows) and [OT-Quant]
 * sections 5.1-5.2 (INT4 groups with one FP16 scale, two codes per byte,
 * element 2k in the low nibble).
 *
 * For each block: amax = max|x| (x upcast to fp32), s = fl32(amax / qmax) with
 * qmax = 127 (INT8), 448 (FP8 e4m3fn), 7 (INT4); if scale_dtype is QFA_F16, s
 * is rounded to fp16 (nearest-even) and the codes use that rounded value.
 * t = fl32(x / s) (correctly rounded), then
 *   INT8: clamp(rne(t), -128, 127);  INT4: clamp(rne(t), -8, 7), packed;
 *   FP8 : OCP e4m3fn of clamp(t, -448, 448), nearest-even, sign kept.
 * A block whose stored scale is 0 gets all-zero codes.
 *
 *   x          [B,N,S,D] or [B,S,N,D] (layout), dtype x_dtype (F32/F16/BF16).
 *   codes      same layout; int8 / e4m3 bytes: D bytes per row; INT4: D/2.
 *   scales     [B, N, ceil(S/block_rows)] of scale_dtype (F32 or F16).
 * Limits: B,N,S >= 0 (an empty tensor launches nothing); 8 <= D <= 1024 and
 * D % 8 == 0; block_rows >= 1. Inputs must be finite.
 */
QFA_API int qfa_block_quant(const void* x, int x_dtype, int B, int N, int S, int D, int layout,
                    int block_rows, int qtype, void* codes, void* scales, int scale_dtype,
                    void* stream);

/*
 * qfa_block_quant_multi -- qfa_block_quant on several tensors in as few
 * launches as possible (the Q, K and V of one attention call).
 *
 * Same arithmetic as qfa_block_quant (see there): the codes and scales of
 * every job are bit-identical to those of one qfa_block_quant call with the
 * job's arguments. Jobs with the same x_dtype and qtype share one kernel
 * launch (up to four per launch), which lets the blocks of one tensor
 * overlap the loads of another.
 *
 *   jobs   host array of njobs descriptors (read during the call only).
 *   njobs  0 <= njobs <= QFA_MAX_QUANT_JOBS.
 * Every job is validated as by qfa_block_quant before anything is launched;
 * the first failing job's status is returned and nothing runs. The output
 * buffers of one job must not overlap the input or outputs of another.
 */
#define QFA_MAX_QUANT_JOBS 16
typedef struct qfa_quant_job {
  const void* x;     /* [B,N,S,D] or [B,S,N,D], x_dtype */
  int x_dtype;
  int B, N, S, D;
  int layout;
  int block_rows;
  int qtype;
  void* codes;       /* same layout; INT4: D/2 bytes per row */
  void* scales;      /* [B, N, ceil(S/block_rows)], scale_dtype */
  int scale_dtype;
} qfa_quant_job;

QFA_API int qfa_block_quant_multi(const qfa_quant_job* jobs, int njobs, void* stream);

/*
 * qfa_rotate_block_quant -- rotate, then block-quantize, in one pass
 * ([MindIE-SD] FP8 attention pipeline: Q and K are multiplied by an
 * orthogonal matrix before the dynamic block quantization, which spreads
 * channel outliers; the rotation is applied here inside the quantizer so the
 * rotated tensor never goes to memory).
 *
 *   y[.., row, i] = round16(sum_k x[.., row, k] * w[i][k])
 *
 * i.e. y = x . w^T (pass w = R^T to apply y = x . R), with the sum in fp32 on
 * the matrix unit and round16 the nearest-even rounding to x's 16-bit type;
 * then y is quantized exactly as qfa_block_quant quantizes a tensor of that
 * type (same blocks, scales and codes).
 *
 *   x          [B,N,S,D] or [B,S,N,D] (layout), dtype x_dtype: F16 or BF16.
 *   w          [D][D] row-major, same dtype as x, device memory, 16-byte aligned.
 *   codes      same layout as x, D bytes per row (INT8 or e4m3 codes).
 *   scales     [B, N, ceil(S/block_rows)] of scale_dtype (F32 or F16).
 * Limits: as qfa_block_quant, plus D in {64, 128}, block_rows a multiple of
 * 32 and at most 256, qtype INT8 or FP8_E4M3 (otherwise QFA_ERR_UNSUPPORTED).
 * Ownership and errors as qfa_block_quant; w is read only.
 */
/*
 * qfa_kv_append -- quantize one new row per sequence into an INT8 or packed
 * INT4 KV cache ([Ascend-INT8] section 3: decode keeps the KV cache
 * quantized, so each new key and value row is quantized into it).
 *
 * Row positions[b] of sequence b (for every KV head) receives x[b, h, :].
 * In its block r = positions[b] / kv_block, with old rows r*kv_block ..
 * positions[b]-1:
 *   - if the block has old rows, a nonzero scale s and fl32(max|x| / s) <=
 *     qmax (or x is all zero), x is quantized with s (as qfa_block_quant
 *     quantizes with a given scale) and nothing else changes;
 *   - otherwise the block is requantized: the old rows' values fl32(code * s)
 *     and x get a new scale fl32(amax / qmax) (rounded to fp16 for fp16
 *     scales) and new codes, written in place. Rows after positions[b] are
 *     never touched.
 *
 *   x          [B, H, D] of x_dtype (F32/F16/BF16), device memory.
 *   positions  [B] int32, device memory; a position outside [0, S_max)
 *              leaves that sequence unchanged.
 *   codes      cache [B,H,S_max,D] or [B,S_max,H,D] (layout), INT8 bytes or
 *              packed INT4 (D/2 bytes per row), updated in place.
 *   scales     [B, H, ceil(S_max/kv_block)] of scale_dtype, updated in place.
 * Limits: B,H >= 0; S_max >= 1; D % 8 == 0, 8 <= D <= 256 (INT8) or 512
 * (INT4); kv_block >= 1; qtype INT8 or INT4 (FP8: QFA_ERR_UNSUPPORTED).
 * Two calls that touch the same block must be ordered on one stream.
 */
QFA_API int qfa_kv_append(const void* x, int x_dtype, const int32_t* positions, void* codes,
                          void* scales, int B, int H, int S_max, int D, int layout, int kv_block,
                          int qtype, int scale_dtype, void* stream);

/*
 * qfa_kv_append_kv -- qfa_kv_append on the K cache and the V cache of one
 * decode step in a single launch ([Ascend-INT8] section 3, as qfa_kv_append):
 * row positions[b] of sequence b receives xk[b, h, :] in (k_codes, k_scales)
 * and xv[b, h, :] in (v_codes, v_scales), each cache updated exactly as
 * qfa_kv_append updates it (byte-identical to two calls). Both caches have
 * the sizes, layout, code type and scale type given; they must not overlap.
 * Arguments, limits and error codes as qfa_kv_append, checked for the K
 * arguments first, then for the V ones; nothing is launched on an error.
 */
QFA_API int qfa_kv_append_kv(const void* xk, const void* xv, int x_dtype,
                             const int32_t* positions, void* k_codes, void* k_scales,
                             void* v_codes, void* v_scales, int B, int H, int S_max, int D,
                             int layout, int kv_block, int qtype, int scale_dtype, void* stream);

QFA_API int qfa_rotate_block_quant(const void* x, int x_dtype, const void* w, int B, int N, int S,
                                   int D, int layout, int block_rows, int qtype, void* codes,
                                   void* scales, int scale_dtype, void* stream);

/*
 * qfa_fwd -- prefill attention forward run on block-quantized codes.
 *
 * Computes, for query row i of head h and key row j of KV head
 * h / (Hq/Hkv) (grouped-query attention),
 *     x_ij = softmax_scale * (sq_i * q_i) . (sk_j * k_j)
 *     o_i  = sum_j softmax_j(x_ij) * (sv_j * v_j)
 * with j <= i kept when `causal` (Sq == Sk required), where q, k, v are the
 * codes and sq, sk, sv their block scales: the low-bit products are formed
 * directly on the codes with wide accumulation and the scales are applied to
 * the products ([Ascend-INT8] INT8-operator section 1: INT8 x INT8 -> INT32,
 * one conversion at the output; section 2: scales kept on chip), then online
 * softmax and P.V ([MindIE-SD] FA quantization, "FP8 Attention": the
 * attention runs on FP8 codes and the output returns to the original
 * precision; [FA-INT8/INT4] INT8 and INT4 layers, with INT4 widened to INT8
 * before the product).
 *
 *   q_codes    [B,Hq,Sq,D] (layout); k_codes, v_codes [B,Hkv,Sk,D] (D/2 bytes for INT4).
 *              Code types (q, k, v): (INT8, INT8, INT8), (INT8, INT4, INT4),
 *              (INT8, INT8, INT4) or (FP8_E4M3, FP8_E4M3, FP8_E4M3); others
 *              return QFA_ERR_UNSUPPORTED.
 *   q_scales   [B,Hq,ceil(Sq/q_block)], q_scale_dtype F32/F16.
 *   k_scales, v_scales [B,Hkv,ceil(Sk/kv_block)], kv_scale_dtype F32/F16.
 *   out        [B,Hq,Sq,D] (same layout as q), out_dtype F32/F16/BF16.
 * Limits: D in {64, 128}; Hq % Hkv == 0; Sk >= 1 when Sq >= 1; q_block and
 * kv_block >= 1; finite scales; code pointers and out 16-byte aligned, scales
 * 4-byte aligned (else QFA_ERR_UNSUPPORTED). Sq == 0 returns QFA_OK without a
 * launch. The output of a row whose scores are all equal to -inf cannot occur
 * (every row keeps at least key 0).
 */
QFA_API int qfa_fwd(const void* q_codes, const void* q_scales, int q_qtype, int q_block,
            int q_scale_dtype, const void* k_codes, const void* k_scales, int k_qtype,
            const void* v_codes, const void* v_scales, int v_qtype, int kv_block,
            int kv_scale_dtype, int B, int Hq, int Hkv, int Sq, int Sk, int D, int layout,
            int causal, float softmax_scale, void* out, int out_dtype, void* stream);

/*
 * qfa_fwd_lowp_workspace_bytes -- bytes of device workspace qfa_fwd_lowp needs
 * for these sizes (one flag byte per work item and wavefront). Returns 0 for
 * invalid sizes.
 */
QFA_API size_t qfa_fwd_lowp_workspace_bytes(int B, int Hq, int Hkv, int Sq);

/*
 * qfa_fwd_lowp -- qfa_fwd with the P.V product on the fp8 matrix unit, for
 * e4m3 Q/K/V ([MindIE-SD] FA quantization, "FP8 Attention": the attention is
 * computed in the FP8 domain). The probabilities are rounded to e4m3 and
 * multiplied with the e4m3 V codes at twice the fp16 rate; the softmax, its
 * row sums and the V scales stay in fp32.
 *
 * Accuracy gate: rounding each probability to e4m3 (relative error at most
 * 2^-4) perturbs a row's output by about 0.03 * sqrt(sum p^2) / sum p times the
 * spread of its V values, which is small only when many keys carry the row.
 * Each row bounds its effective number of keys (sum p)^2 / sum p^2 from below
 * by l^2 / S, S = the sum over 64-key tiles of the tile's largest probability
 * times the tile's sum; a row with l^2 / S < 256 ("peaky": a few keys
 * dominate) flags its work item, and the workgroup that computed the item
 * recomputes it at once exactly as qfa_fwd does (fp16 P.V) before writing any
 * of it, in the same launch. The output of a flagged work item is therefore
 * bit-identical to qfa_fwd's, and a flag costs only that item's second pass.
 *
 * Arguments as qfa_fwd, plus
 *   workspace  device buffer of at least qfa_fwd_lowp_workspace_bytes(B,Hq,Hkv,Sq)
 *              bytes, 8-byte aligned, owned by the caller; on return (after the
 *              stream has run the call) byte 8*w + v is 1 when wavefront v of work
 *              item w fell back to the fp16 product, else 0. Every byte is written.
 * Supported: q, k and v all FP8_E4M3 with kv_block a multiple of 64 (block
 * scales); other code types or per-key scales return QFA_ERR_UNSUPPORTED, a
 * missing or short workspace QFA_ERR_WORKSPACE. Calls that share a workspace
 * must not overlap.
 */
QFA_API int qfa_fwd_lowp(const void* q_codes, const void* q_scales, int q_qtype, int q_block,
                 int q_scale_dtype, const void* k_codes, const void* k_scales, int k_qtype,
                 const void* v_codes, const void* v_scales, int v_qtype, int kv_block,
                 int kv_scale_dtype, int B, int Hq, int Hkv, int Sq, int Sk, int D, int layout,
                 int causal, float softmax_scale, void* out, int out_dtype, void* workspace,
                 size_t workspace_bytes, void* stream);

/*
 * qfa_decode_workspace_bytes -- bytes of device workspace qfa_decode needs for
 * these sizes (split-K partial results). Returns 0 for invalid sizes.
 */
QFA_API size_t qfa_decode_workspace_bytes(int B, int Hq, int S_max, int D);

/*
 * qfa_decode -- one query token per sequence against a quantized KV cache.
 *
 * The cache holds K/V as INT8 (or INT4) codes with block scales, and attention
 * is computed on the codes without writing a dequantized cache
 * ([Ascend-INT8] INT8-operator section 3, KV cache quantized to INT8 for
 * decode, attention computed directly on INT8; [FA-INT8/INT4] INT4 layer for
 * the INT4 codes). The query is used unquantized.
 *     o_bh = sum_{j < seq_lens[b]} softmax_j(softmax_scale * q_bh . (sk_j k_j)) * (sv_j v_j)
 *
 *   q          [B,Hq,1,D] (BNSD; for BSND the same bytes as [B,1,Hq,D]), q_dtype F16/BF16/F32.
 *   k_cache, v_cache [B,Hkv,S_max,D or D/2] (layout), kv_qtype INT8 or INT4.
 *   k_scales, v_scales [B,Hkv,ceil(S_max/kv_block)], kv_scale_dtype F16/F32.
 *   seq_lens   device int32 [B], each in [1, S_max] (values outside are clamped
 *              to that range by the kernel).
 *   out        [B,Hq,1,D], out_dtype F16/BF16/F32.
 *   workspace  device buffer of at least qfa_decode_workspace_bytes(B,Hq,S_max,D)
 *              bytes; its contents on entry do not matter. Calls that share a
 *              workspace must be ordered on one stream.
 * Limits: D in {64, 128}; Hq % Hkv == 0; 1 <= Hq/Hkv <= 16;
 * (S_max + 1024) * row_stride < 2^31, where row_stride is the bytes between
 * consecutive tokens of one head (D, or D/2 for INT4; times Hkv in BSND).
 * Outside these limits the call returns QFA_ERR_UNSUPPORTED.
 */
QFA_API int qfa_decode(const void* q, int q_dtype, int B, int Hq, int Hkv, int D, const void* k_cache,
               const void* v_cache, const void* k_scales, const void* v_scales, int kv_qtype,
               int kv_block, int kv_scale_dtype, int S_max, int layout, const int32_t* seq_lens,
               float softmax_scale, void* out, int out_dtype, void* workspace,
               size_t workspace_bytes, void* stream);

/*
 * qfa_decode_noalloc -- qfa_decode without a workspace argument, for callers
 * that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation).
 *
 * Same arguments, arithmetic, kernels and results as qfa_decode (bit for bit),
 * except that the split-K partials go to a static device array of
 * qfa_decode_noalloc_max_bytes() bytes (8 MiB) that the library holds on each
 * GPU it runs on until the process ends. The call allocates nothing: on its
 * first use on a device it only looks up that device's copy of the array.
 * A call that needs more partial space than the array holds
 * (qfa_decode_workspace_bytes(B, Hq, S_max, D) > the maximum, when S_max >
 * 1024) returns QFA_ERR_SCRATCH and launches nothing; with D = 128 the limit
 * is B * Hq * ceil(S_max / 1024) <= 16131 (e.g. B=32, Hq=32, S_max up to
 * 15360). The array's contents on entry do not matter (every partial read is
 * written first by the same call). All calls on one GPU share the array:
 * calls that may overlap on one GPU (different streams, or host threads
 * without ordering) race and must be serialized by the caller.
 */
QFA_API size_t qfa_decode_noalloc_max_bytes(void);
QFA_API int qfa_decode_noalloc(const void* q, int q_dtype, int B, int Hq, int Hkv, int D,
                               const void* k_cache, const void* v_cache, const void* k_scales,
                               const void* v_scales, int kv_qtype, int kv_block,
                               int kv_scale_dtype, int S_max, int layout,
                               const int32_t* seq_lens, float softmax_scale, void* out,
                               int out_dtype, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* QFA_H */
