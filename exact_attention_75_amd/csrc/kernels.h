// kernels.h -- internal interface between the C-ABI host layer and the HIP
// kernels (not part of the public ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tile_sched.h"

namespace attn {

constexpr int kBlockMMin = 128;  // smallest query block any kernel uses

// Optional features of the 4-wave forward kernel (bit flags)
constexpr int kFeatSoftcap = 1;  // scores capped: cap tanh(scale s / cap)
constexpr int kFeatVCol = 2;     // V given column-major [B, Hkv, D, Sk]

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
  // split-KV partials (launch_fwd_split): key ranges of split_keys keys
  int splits = 1;
  int split_keys = 0;
  float* o_part = nullptr;    // [splits, B, Sq, Hq, D] fp32
  float* lse_part = nullptr;  // [splits, B, Hq, Sq] fp32
  // PackGQA (dense, 128-row blocks): tm runs over (B, Hkv, Sq * group) and a
  // tile's rows are (position, head of the group) pairs
  int pack = 0;
  // optional features (kFeat* flags; dense, 128-row blocks, no split/pack)
  int feat = 0;
  float softcap_a = 0.f;      // cap / scale
  float softcap_b2 = 0.f;     // 2 scale log2(e) / cap
};

constexpr int kCombineMaxSplits = 256;   // most partials attn_combine merges per row

struct CombineParams {
  const float* o_part;        // [splits, B, Sq, Hq, d]
  const float* lse_part;      // [splits, B, Hq, Sq]
  void* o;                    // [B, Sq, Hq, d] in the output type
  float* lse;                 // [B, Hq, Sq] or nullptr
  int splits, B, Hq, Sq, d;
};

struct BwdParams {
  const void* q;              // [B, Sq, Hq, D]
  const void* k;              // [B, Sk, Hkv, D]
  const void* v;              // [B, Sk, Hkv, D]
  const void* o;              // [B, Sq, Hq, D] forward output
  const void* dout;           // [B, Sq, Hq, D] gradient of o
  const float* lse;           // [B, Hq, Sq] forward LSE (natural log)
  const float* dlse;          // [B, Hq, Sq] gradient of lse, or nullptr
  void* dq;                   // [B, Sq, Hq, D]
  void* dk;                   // [B, Sk, Hkv, D]
  void* dv;                   // [B, Sk, Hkv, D]
  float2* stats;              // [B, Hq, Sq_pad] ([Hq, T] varlen): (LSE log2 e, or +inf for -inf; delta)
  const int32_t* cu_seqlens;  // varlen offsets (device) or nullptr; then B = sequences, Sq = Sk = T
  int B, Hq, Hkv, Sq, Sk;
  int Sq_pad;                 // Sq rounded up to 32 (rows past Sq: (+inf, 0))
  int group;
  float scale;
  float scale_log2;           // scale * log2(e)
  TileMap tm;                 // dQ tiles (128 query rows)
  int grid_dq;
  int grid_dkdv;
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

// One tensor of the fp8 prepass: x [B, S, H, d] fp32 -> codes x8 ([B, S, H, d],
// or [B, H, d, S] when transpose) and scales descale [B, H, ceil(S/128)].
struct PrepassSeg {
  const float* x;
  uint8_t* x8;
  float* descale;
  const float* signs;         // d signs (device) for the rotation, or nullptr
  int default_signs;          // non-zero: rotate with the built-in default signs (signs ignored)
  int B, S, H;
  int transpose;
  int blocks;                 // B * H * ceil(S / 128): workgroups of this tensor
};
// Up to three tensors in one launch (Q, K and V^T for the fp8 forward):
// workgroup i belongs to segment s when first[s] <= i < first[s] + seg[s].blocks.
struct PrepassParams {
  PrepassSeg seg[3];
  int nseg;
  int d;
};

// splitmix64 (Steele, Lea, Flood 2014): the output for counter value x
// (state x * golden gamma, then the published mixing constants)
constexpr uint64_t splitmix64(uint64_t x) {
  uint64_t z = x * 0x9E3779B97F4A7C15ULL;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}
// Default sign i of the Hadamard rotation: the top bit of
// splitmix64((55 << 32) + i + 1) gives -1, else +1.
constexpr float default_sign(int i) {
  return (splitmix64((55ULL << 32) + (uint64_t)i + 1) >> 63) ? -1.f : 1.f;
}

// Query rows per workgroup of the bf16/fp16 forward for this configuration.
int fwd_block_m(int dtype, int d, int varlen);
// Query rows per workgroup of the fp8 forward.
int fwd_fp8_block_m();

// Returns hipSuccess or the launch error.  p.pack selects the PackGQA
// variant (128-row blocks) for dense inputs.
hipError_t launch_fwd(const FwdParams& p, int dtype, int d, int causal, int varlen, hipStream_t s);
// d = 128 dense bf16/fp16 with 256-row blocks, one wave per SIMD.
hipError_t launch_fwd_wide(const FwdParams& p, int dtype, int causal, hipStream_t s);
// Split-KV partials with the 4-wave kernel (dense, d in {64, 128}, optionally
// PackGQA); grid = splits x tiles, split index slowest.
hipError_t launch_fwd_split(const FwdParams& p, int dtype, int d, int causal, hipStream_t s);
// Merge of split-KV partials into O (dtype 0 bf16, 1 fp16) and LSE.
hipError_t launch_combine(const CombineParams& p, int dtype, hipStream_t s);
hipError_t launch_fwd_fp8(const Fp8FwdParams& p, int causal, hipStream_t s);
// Backward: statistics preprocess, dK/dV (parallel over key blocks), dQ
// (parallel over query blocks); dense bf16/fp16, d in {64, 128}.
hipError_t launch_bwd(const BwdParams& p, int dtype, int d, int causal, int varlen, hipStream_t s);
// dK, dV of the backward alone (the statistics must already be written)
hipError_t launch_bwd_dkdv(const BwdParams& p, int dtype, int d, int causal, int varlen, hipStream_t s);
// dQ of the backward alone (the statistics must already be written)
hipError_t launch_bwd_dq(const BwdParams& p, int dtype, int d, int causal, int varlen, hipStream_t s);
constexpr int kBwdBlockN = 128;   // keys per dK/dV workgroup
constexpr int kBwdBlockM = 128;   // query rows per dQ workgroup
hipError_t launch_prepass(const PrepassParams& p, hipStream_t s);
// shader-clock and wall-clock deltas of one lane over `ticks` wall-clock ticks
hipError_t launch_clock_probe(unsigned long long* out, long long ticks, hipStream_t s);

}  // namespace attn
