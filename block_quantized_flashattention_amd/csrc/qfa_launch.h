// Host-side launcher declarations shared by the C ABI (api.hip) and the kernel
// translation units. Every launcher assumes its arguments were validated by
// the C ABI and returns hipSuccess or the launch error.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "qfa.h"

namespace qfa {

struct QuantArgs {
  const void* x;
  int x_dtype;
  int B, N, S, D;
  int layout;
  int block_rows;
  int qtype;
  void* codes;
  void* scales;
  int scale_dtype;
};

hipError_t launch_block_quant(const QuantArgs& a, hipStream_t stream);
// Several tensors, grouped by input and code type into shared launches.
hipError_t launch_block_quant_multi(const QuantArgs* a, int n, hipStream_t stream);

// Fused rotation + block quantization (16-bit x and w, INT8 or FP8 codes).
struct RotQuantArgs {
  const void* x;
  int x_dtype;
  const void* w;
  int B, N, S, D;
  int layout;
  int block_rows;
  int qtype;
  void* codes;
  void* scales;
  int scale_dtype;
};

hipError_t launch_rotate_block_quant(const RotQuantArgs& a, hipStream_t stream);

// One new row per sequence into a quantized KV cache (INT8 or packed INT4).
struct AppendArgs {
  const void* x;
  int x_dtype;
  const int32_t* positions;
  void* codes;
  void* scales;
  int B, H, S_max, D;
  int layout;
  int kv_block;
  int qtype;
  int scale_dtype;
  // A second cache updated in the same launch (the V row of a decode step),
  // same sizes and types; x2 null for one cache.
  const void* x2;
  void* codes2;
  void* scales2;
};

hipError_t launch_kv_append(const AppendArgs& a, hipStream_t stream);

struct FwdArgs {
  const void* q;
  const void* qs;
  int q_qtype, q_block, q_scale_dtype;
  const void* k;
  const void* ks;
  int k_qtype;
  const void* v;
  const void* vs;
  int v_qtype;
  int kv_block, kv_scale_dtype;
  int B, Hq, Hkv, Sq, Sk, D, layout, causal;
  float softmax_scale;
  void* out;
  int out_dtype;
};

// Returns hipErrorInvalidValue for a combination without a compiled kernel.
hipError_t launch_fwd(const FwdArgs& a, hipStream_t stream);
// The forward with P.V on the fp8 matrix unit (e4m3 Q/K/V with block
// scales): one launch that writes one flag byte per (workgroup, wavefront)
// to `flags` (fwd_lowp_workspace_bytes of them); a workgroup with a flagged
// wavefront recomputes its work item with the fp16 product before it exits.
size_t fwd_lowp_workspace_bytes(int B, int Hq, int Hkv, int Sq);
hipError_t launch_fwd_lowp(const FwdArgs& a, void* flags, hipStream_t stream);

struct DecodeArgs {
  const void* q;
  int q_dtype;
  int B, Hq, Hkv, D;
  const void* k;
  const void* v;
  const void* ks;
  const void* vs;
  int kv_qtype, kv_block, kv_scale_dtype, S_max, layout;
  const int32_t* lens;
  float softmax_scale;
  void* out;
  int out_dtype;
  void* workspace;
};

// Token chunk handled by one split of the decode kernel.
constexpr int kDecodeChunk = 1024;

size_t decode_workspace_bytes(int B, int Hq, int S_max, int D);
hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream);

// Size of the library's static decode scratch (qfa_decode_noalloc).
constexpr size_t kDecodeScratchBytes = size_t(8) << 20;
// Device address of that scratch on the device `stream` runs on (looked up
// once per device, then cached); never allocates.
hipError_t decode_scratch(hipStream_t stream, void** ptr);

}  // namespace qfa
