// attn_api.cpp -- the C ABI declared in include/attn.h: argument validation,
// tile planning, dispatch over the kernel variants, the fp8 workspace and
// error reporting.  Validation and planning touch no HIP state, so every
// error path returns before anything is enqueued.
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "../../include/attn.h"
#include "kernels.h"

namespace {

thread_local char g_hip_msg[256] = "";

int hip_fail(hipError_t e) {
  snprintf(g_hip_msg, sizeof g_hip_msg, "HIP error %d: %s", (int)e, hipGetErrorString(e));
  return ATTN_ERR_HIP;
}

constexpr long long kMax32 = 0x7fffffffLL;

int check_common(int B, int Hq, int Hkv, int Sq, int Sk, int d, float scale) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Sq <= 0 || Sk <= 0) return ATTN_ERR_SHAPE;
  if (d != 64 && d != 128) return ATTN_ERR_HEADDIM;
  if (Hq % Hkv != 0) return ATTN_ERR_GQA;
  if (!isfinite(scale) || !(scale > 0.f)) return ATTN_ERR_ARG;
  // per-tensor element counts and in-kernel 32-bit row offsets
  if ((long long)Sq * Hq * d > kMax32 || (long long)Sk * Hkv * d > kMax32) return ATTN_ERR_SIZE;
  if ((long long)B * Hq * ((Sq + attn::kBlockMMin - 1) / attn::kBlockMMin) > kMax32) return ATTN_ERR_SIZE;
  return ATTN_OK;
}

// --- workspaces: lazily grown device buffers, one per (use, device) -------
// kWsFp8 holds the quantised operands of attn_fwd's fp8 types, kWsSplit the
// split-KV partials; separate buffers, so the two paths never share memory.
constexpr int kMaxDevices = 64;
enum { kWsFp8 = 0, kWsSplit = 1, kWsKinds = 2 };
struct Workspace {
  void* ptr = nullptr;
  size_t bytes = 0;
};
Workspace g_ws[kWsKinds][kMaxDevices];
std::mutex g_ws_mu;

int workspace(int kind, size_t bytes, void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e);
  if (dev < 0 || dev >= kMaxDevices) return ATTN_ERR_ARG;
  std::lock_guard<std::mutex> lk(g_ws_mu);
  Workspace& w = g_ws[kind][dev];
  if (w.bytes < bytes) {
    if (w.ptr) {
      // the old buffer may still be in use by enqueued work
      e = hipDeviceSynchronize();
      if (e != hipSuccess) return hip_fail(e);
      (void)hipFree(w.ptr);
      w.ptr = nullptr;
      w.bytes = 0;
    }
    e = hipMalloc(&w.ptr, bytes);
    if (e != hipSuccess) {
      w.ptr = nullptr;
      return ATTN_ERR_NOMEM;
    }
    w.bytes = bytes;
  }
  *out = w.ptr;
  return ATTN_OK;
}

// Split-KV plan.  The key axis is cut into `splits` ranges of `split_keys`
// keys (a multiple of the 64-key tile); the last range may be shorter, none
// is empty.  num_splits > 0 asks for that many (fewer when Sk has fewer
// 64-key tiles); num_splits == 0 picks enough to give the chip about four
// 128-row workgroups per CU (two resident at a time), without cutting a range
// below 256 keys.
constexpr int kMaxSplits = 256;
constexpr int kSplitBlockM = 128;   // query rows per workgroup of the split kernel
int split_plan(int B, int Hq, int Sq, int Sk, int num_splits, int* splits, int* split_keys) {
  if (num_splits < 0 || num_splits > kMaxSplits) return ATTN_ERR_ARG;
  const long long tiles = (long long)B * Hq * ((Sq + kSplitBlockM - 1) / kSplitBlockM);
  const int kt = (Sk + 63) / 64;   // 64-key tiles
  int want = num_splits;
  if (want == 0) {
    constexpr long long kTarget = 4 * 256;
    const long long by_tiles = (kTarget + tiles - 1) / tiles;
    const int by_keys = (Sk + 255) / 256;
    want = (int)(by_tiles < by_keys ? by_tiles : by_keys);
    if (want > 64) want = 64;
    if (want < 1) want = 1;
  }
  if (want > kt) want = kt;
  const int per = (kt + want - 1) / want;   // tiles per range
  *split_keys = per * 64;
  *splits = (Sk + per * 64 - 1) / (per * 64);
  if (tiles * *splits > kMax32) return ATTN_ERR_SIZE;
  return ATTN_OK;
}

uint64_t splitmix64(uint64_t x) {
  uint64_t z = x * 0x9E3779B97F4A7C15ULL;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

// device copy of the default sign vector, per device
float* g_signs[kMaxDevices] = {};

}  // namespace

extern "C" {

const char* attn_strerror(int code) {
  switch (code) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_NULL: return "a required pointer is NULL";
    case ATTN_ERR_SHAPE: return "invalid shape (non-positive size, or varlen with Sq != Sk)";
    case ATTN_ERR_HEADDIM: return "unsupported head dimension (64 or 128; fp8 needs 128)";
    case ATTN_ERR_GQA: return "Hq must be a multiple of Hkv";
    case ATTN_ERR_DTYPE: return "unknown or unsupported dtype for this call";
    case ATTN_ERR_ARG: return "invalid argument (scale must be finite and > 0, or unsupported combination)";
    case ATTN_ERR_NOMEM: return "device workspace allocation failed";
    case ATTN_ERR_HIP: return g_hip_msg[0] ? g_hip_msg : "HIP runtime error";
    case ATTN_ERR_SIZE: return "problem too large for 32-bit in-kernel indexing";
    default: return "unknown status code";
  }
}

int attn_default_signs(float* signs_host, int n) {
  if (!signs_host) return ATTN_ERR_NULL;
  if (n <= 0 || n > 128) return ATTN_ERR_SHAPE;
  for (int i = 0; i < n; ++i)
    signs_host[i] = (splitmix64((55ULL << 32) + (uint64_t)i + 1) >> 63) ? -1.f : 1.f;
  return ATTN_OK;
}

int attn_grid_size(int B, int Hq, int Sq, int d, int dtype, int* grid_out, int* block_m_out) {
  if (!grid_out || !block_m_out) return ATTN_ERR_NULL;
  if (B <= 0 || Hq <= 0 || Sq <= 0) return ATTN_ERR_SHAPE;
  if (dtype < ATTN_BF16 || dtype > ATTN_FP8_E4M3_HADAMARD) return ATTN_ERR_DTYPE;
  const int bm = dtype >= ATTN_FP8_E4M3 ? attn::fwd_fp8_block_m() : attn::fwd_block_m(dtype, d, 0);
  *block_m_out = bm;
  *grid_out = B * Hq * ((Sq + bm - 1) / bm);
  return ATTN_OK;
}

int attn_tile_of(int p, int B, int Hq, int Hkv, int Sq, int block_m, int causal, int* b_out,
                 int* h_out, int* m_out) {
  if (!b_out || !h_out || !m_out) return ATTN_ERR_NULL;
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Sq <= 0 || block_m <= 0 || Hq % Hkv) return ATTN_ERR_SHAPE;
  attn::TileMap tm = attn::make_tile_map(B, Hq, Hkv, Sq, block_m, causal);
  if (p < 0 || p >= tm.ntiles) return ATTN_ERR_SHAPE;
  attn::tile_decode(tm, p, *b_out, *h_out, *m_out);
  return ATTN_OK;
}

int attn_fwd_fp8(const uint8_t* q8, const uint8_t* k8, const uint8_t* v8t, const float* q_descale,
                 const float* k_descale, const float* v_descale, void* o, float* lse, int B, int Hq,
                 int Hkv, int Sq, int Sk, int d, float scale, int causal, void* stream) {
  if (!q8 || !k8 || !v8t || !q_descale || !k_descale || !v_descale || !o) return ATTN_ERR_NULL;
  int rc = check_common(B, Hq, Hkv, Sq, Sk, d, scale);
  if (rc) return rc;
  if (d != 128) return ATTN_ERR_HEADDIM;
  if (Sk % 16 != 0) return ATTN_ERR_SHAPE;   // 16-byte aligned rows of V^T
  attn::Fp8FwdParams p{};
  p.q8 = q8;
  p.k8 = k8;
  p.v8t = v8t;
  p.q_descale = q_descale;
  p.k_descale = k_descale;
  p.v_descale = v_descale;
  p.o = o;
  p.lse = lse;
  p.B = B;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.Sq = Sq;
  p.Sk = Sk;
  p.group = Hq / Hkv;
  p.scale_log2 = scale * 1.4426950408889634f;
  p.tm = attn::make_tile_map(B, Hq, Hkv, Sq, attn::fwd_fp8_block_m(), causal);
  p.grid = p.tm.ntiles;
  hipError_t e = attn::launch_fwd_fp8(p, causal, (hipStream_t)stream);
  return e == hipSuccess ? ATTN_OK : hip_fail(e);
}

int attn_fp8_prepass(const float* x, uint8_t* x8, float* descale, int B, int S, int H, int d,
                     int transpose_out, const float* signs, void* stream) {
  if (!x || !x8 || !descale) return ATTN_ERR_NULL;
  if (B <= 0 || S <= 0 || H <= 0) return ATTN_ERR_SHAPE;
  if (d != 128) return ATTN_ERR_HEADDIM;
  if ((long long)B * S * H * d > kMax32 * 2) return ATTN_ERR_SIZE;
  attn::PrepassParams p{};
  p.x = x;
  p.x8 = x8;
  p.descale = descale;
  p.signs = signs;
  p.B = B;
  p.S = S;
  p.H = H;
  p.d = d;
  p.transpose_out = transpose_out ? 1 : 0;
  hipError_t e = attn::launch_prepass(p, (hipStream_t)stream);
  return e == hipSuccess ? ATTN_OK : hip_fail(e);
}

int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv,
             int Sq, int Sk, int d, float scale, int causal, const int32_t* cu_seqlens, int dtype,
             void* stream) {
  if (!q || !k || !v || !o) return ATTN_ERR_NULL;
  if (dtype < ATTN_BF16 || dtype > ATTN_FP8_E4M3_HADAMARD) return ATTN_ERR_DTYPE;
  const bool varlen = cu_seqlens != nullptr;
  if (varlen) {
    if (B <= 0) return ATTN_ERR_SHAPE;
    if (Sq != Sk) return ATTN_ERR_SHAPE;
  }
  int rc = check_common(varlen ? 1 : B, Hq, Hkv, Sq, Sk, d, scale);
  if (rc) return rc;
  hipStream_t s = (hipStream_t)stream;

  if (dtype == ATTN_FP8_E4M3 || dtype == ATTN_FP8_E4M3_HADAMARD) {
    if (varlen) return ATTN_ERR_ARG;
    if (d != 128) return ATTN_ERR_HEADDIM;
    if (Sk % 16 != 0) return ATTN_ERR_SHAPE;
    const long long nbq = (Sq + 127) / 128, nbk = (Sk + 127) / 128;
    const size_t qb = (size_t)B * Sq * Hq * d, kb = (size_t)B * Sk * Hkv * d;
    auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
    const size_t sq_b = al(sizeof(float) * B * Hq * nbq), sk_b = al(sizeof(float) * B * Hkv * nbk);
    const size_t total = al(qb) + 2 * al(kb) + sq_b + 2 * sk_b;
    void* ws = nullptr;
    rc = workspace(kWsFp8, total, &ws);
    if (rc) return rc;
    uint8_t* base = (uint8_t*)ws;
    uint8_t* q8 = base;
    uint8_t* k8 = q8 + al(qb);
    uint8_t* v8t = k8 + al(kb);
    float* qs = (float*)(v8t + al(kb));
    float* ks = (float*)((uint8_t*)qs + sq_b);
    float* vs = (float*)((uint8_t*)ks + sk_b);
    const float* sg = nullptr;
    if (dtype == ATTN_FP8_E4M3_HADAMARD) {
      int dev = 0;
      hipError_t e = hipGetDevice(&dev);
      if (e != hipSuccess) return hip_fail(e);
      if (dev < 0 || dev >= kMaxDevices) return ATTN_ERR_ARG;
      std::lock_guard<std::mutex> lk(g_ws_mu);
      if (!g_signs[dev]) {
        float hs[128];
        attn_default_signs(hs, 128);
        float* dp = nullptr;
        e = hipMalloc(&dp, sizeof hs);
        if (e != hipSuccess) return ATTN_ERR_NOMEM;
        e = hipMemcpy(dp, hs, sizeof hs, hipMemcpyHostToDevice);
        if (e != hipSuccess) {
          (void)hipFree(dp);
          return hip_fail(e);
        }
        g_signs[dev] = dp;
      }
      sg = g_signs[dev];
    }
    rc = attn_fp8_prepass((const float*)q, q8, qs, B, Sq, Hq, d, 0, sg, stream);
    if (!rc) rc = attn_fp8_prepass((const float*)k, k8, ks, B, Sk, Hkv, d, 0, sg, stream);
    if (!rc) rc = attn_fp8_prepass((const float*)v, v8t, vs, B, Sk, Hkv, d, 1, nullptr, stream);
    if (!rc) rc = attn_fwd_fp8(q8, k8, v8t, qs, ks, vs, o, lse, B, Hq, Hkv, Sq, Sk, d, scale, causal, stream);
    return rc;
  }

  attn::FwdParams p{};
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  p.cu_seqlens = cu_seqlens;
  p.B = B;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.Sq = Sq;
  p.Sk = Sk;
  p.group = Hq / Hkv;
  p.q_tok_stride = Hq * d;
  p.kv_tok_stride = Hkv * d;
  p.q_batch_stride = (long long)Sq * Hq * d;
  p.kv_batch_stride = (long long)Sk * Hkv * d;
  p.scale_log2 = scale * 1.4426950408889634f;
  if (varlen) {
    // one tile per (head, query block of a sequence); the number of blocks is
    // at most ceil(T / BM) + (number of sequences), the rest exit at once
    const int bm = attn::fwd_block_m(dtype, d, 1);
    const long long nb = (Sq + bm - 1) / bm + B;
    if (nb * Hq > kMax32) return ATTN_ERR_SIZE;
    p.grid = (int)(nb * Hq);
  } else {
    p.tm = attn::make_tile_map(B, Hq, Hkv, Sq, attn::fwd_block_m(dtype, d, 0), causal);
    p.grid = p.tm.ntiles;
  }
  hipError_t e = attn::launch_fwd(p, dtype, d, causal, varlen ? 1 : 0, s);
  return e == hipSuccess ? ATTN_OK : hip_fail(e);
}

int attn_split_plan(int B, int Hq, int Sq, int Sk, int num_splits, int* splits_out,
                    int* split_keys_out) {
  if (!splits_out || !split_keys_out) return ATTN_ERR_NULL;
  if (B <= 0 || Hq <= 0 || Sq <= 0 || Sk <= 0) return ATTN_ERR_SHAPE;
  return split_plan(B, Hq, Sq, Sk, num_splits, splits_out, split_keys_out);
}

int attn_combine(const float* o_part, const float* lse_part, void* o, float* lse, int splits, int B,
                 int Hq, int Sq, int d, int dtype, void* stream) {
  if (!o_part || !lse_part || !o) return ATTN_ERR_NULL;
  if (splits <= 0 || B <= 0 || Hq <= 0 || Sq <= 0) return ATTN_ERR_SHAPE;
  if (d != 64 && d != 128) return ATTN_ERR_HEADDIM;
  if (dtype != ATTN_BF16 && dtype != ATTN_FP16) return ATTN_ERR_DTYPE;
  if ((long long)B * Sq * Hq * (d / 4) > kMax32 * 64LL) return ATTN_ERR_SIZE;
  attn::CombineParams p{};
  p.o_part = o_part;
  p.lse_part = lse_part;
  p.o = o;
  p.lse = lse;
  p.splits = splits;
  p.B = B;
  p.Hq = Hq;
  p.Sq = Sq;
  p.d = d;
  hipError_t e = attn::launch_combine(p, dtype, (hipStream_t)stream);
  return e == hipSuccess ? ATTN_OK : hip_fail(e);
}

int attn_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq,
                     int Hkv, int Sq, int Sk, int d, float scale, int causal, int num_splits, int dtype,
                     void* stream) {
  if (!q || !k || !v || !o) return ATTN_ERR_NULL;
  if (dtype != ATTN_BF16 && dtype != ATTN_FP16) return ATTN_ERR_DTYPE;
  int rc = check_common(B, Hq, Hkv, Sq, Sk, d, scale);
  if (rc) return rc;
  int splits = 0, split_keys = 0;
  rc = split_plan(B, Hq, Sq, Sk, num_splits, &splits, &split_keys);
  if (rc) return rc;
  if (splits == 1)   // one range: the plain forward computes the same thing
    return attn_fwd(q, k, v, o, lse, B, Hq, Hkv, Sq, Sk, d, scale, causal, nullptr, dtype, stream);
  const size_t rows = (size_t)B * Sq * Hq;
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  const size_t ob = al(sizeof(float) * splits * rows * d), lb = al(sizeof(float) * splits * rows);
  void* ws = nullptr;
  rc = workspace(kWsSplit, ob + lb, &ws);
  if (rc) return rc;
  attn::FwdParams p{};
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  p.cu_seqlens = nullptr;
  p.B = B;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.Sq = Sq;
  p.Sk = Sk;
  p.group = Hq / Hkv;
  p.q_tok_stride = Hq * d;
  p.kv_tok_stride = Hkv * d;
  p.q_batch_stride = (long long)Sq * Hq * d;
  p.kv_batch_stride = (long long)Sk * Hkv * d;
  p.scale_log2 = scale * 1.4426950408889634f;
  p.tm = attn::make_tile_map(B, Hq, Hkv, Sq, kSplitBlockM, causal);
  p.splits = splits;
  p.split_keys = split_keys;
  p.o_part = (float*)ws;
  p.lse_part = (float*)((uint8_t*)ws + ob);
  p.grid = p.tm.ntiles * splits;
  hipError_t e = attn::launch_fwd_split(p, dtype, d, causal, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e);
  return attn_combine(p.o_part, p.lse_part, o, lse, splits, B, Hq, Sq, d, dtype, stream);
}

void attn_release(void) {
  std::lock_guard<std::mutex> lk(g_ws_mu);
  int cur = 0;
  if (hipGetDevice(&cur) != hipSuccess) return;
  for (int dev = 0; dev < kMaxDevices; ++dev) {
    bool any = g_signs[dev] != nullptr;
    for (int k = 0; k < kWsKinds; ++k) any = any || g_ws[k][dev].ptr != nullptr;
    if (!any) continue;
    if (hipSetDevice(dev) != hipSuccess) continue;
    (void)hipDeviceSynchronize();
    for (int k = 0; k < kWsKinds; ++k) {
      if (g_ws[k][dev].ptr) (void)hipFree(g_ws[k][dev].ptr);
      g_ws[k][dev] = Workspace{};
    }
    if (g_signs[dev]) (void)hipFree(g_signs[dev]);
    g_signs[dev] = nullptr;
  }
  (void)hipSetDevice(cur);
}

}  // extern "C"
