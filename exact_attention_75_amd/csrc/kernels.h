// kernels.h -- internal interface between the C-ABI host layer and the HIP
// kernels (not part of the public ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tile_sched.h"

namespace attn {

constexpr int kBlockMMin = 128;  // smallest query block any kernel uses

struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  const int32_t* cu_seqlens;  // varlen offsets (device) or nullptr
  int B, Hq, Hkv, Sq, Sk;
  int group;                  // Hq / Hkv
  int q_tok_stride;           // elements between consecutive tokens of q / o (Hq * d)
  int kv_tok_stride;          // elements between consecutive tokens of k / v (Hkv * d)
  long long q_batch_stride;   // elements between batches of q / o (Sq * Hq * d)
  long long kv_batch_stride;  // elements between batches of k / v (Sk * Hkv * d)
  float scale_log2;           // scale * log2(e)
  TileMap tm;                 // dense tile order
  int grid;                   // workgroups launched
};

struct Fp8FwdParams {
  const uint8_t* q8;          // [B, Sq, Hq, 128]
  const uint8_t* k8;          // [B, Sk, Hkv, 128]
  const uint8_t* v8t;         // [B, Hkv, 128, Sk]
  const float* q_descale;     // [B, Hq, ceil(Sq/128)]
  const float* k_descale;     // [B, Hkv, ceil(Sk/128)]
  const float* v_descale;     // [B, Hkv, ceil(Sk/128)]
  void* o;                    // bf16 [B, Sq, Hq, 128]
  float* lse;                 // [B, Hq, Sq] or nullptr
  int B, Hq, Hkv, Sq, Sk;
  int group;
  float scale_log2;
  TileMap tm;
  int grid;
};

struct PrepassParams {
  const float* x;             // [B, S, H, d]
  uint8_t* x8;                // [B, S, H, d] or [B, H, d, S]
  float* descale;             // [B, H, ceil(S/128)]
  const float* signs;         // d signs or nullptr
  int B, S, H, d;
  int transpose_out;
};

// Query rows per workgroup of the bf16/fp16 forward for this configuration.
int fwd_block_m(int dtype, int d, int varlen);
// Query rows per workgroup of the fp8 forward.
int fwd_fp8_block_m();

// Returns hipSuccess or the launch error.
hipError_t launch_fwd(const FwdParams& p, int dtype, int d, int causal, int varlen, hipStream_t s);
// d = 128 dense bf16/fp16 with 256-row blocks, one wave per SIMD.
hipError_t launch_fwd_wide(const FwdParams& p, int dtype, int causal, hipStream_t s);
hipError_t launch_fwd_fp8(const Fp8FwdParams& p, int causal, hipStream_t s);
hipError_t launch_prepass(const PrepassParams& p, hipStream_t s);

}  // namespace attn
