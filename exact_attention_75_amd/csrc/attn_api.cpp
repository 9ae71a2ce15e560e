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

// --- failure injection (attn_test_fail_next): one armed code per thread --
thread_local int g_fail_next = 0;

// A launch is about to be enqueued: hipSuccess, or the simulated launch
// failure that attn_test_fail_next(ATTN_ERR_HIP) armed (then nothing runs).
hipError_t launch_gate() {
  if (g_fail_next != ATTN_ERR_HIP) return hipSuccess;
  g_fail_next = 0;
  return hipErrorLaunchFailure;
}

// --- workspaces: lazily grown device buffers, one per (use, device) -------
// kWsFp8 holds the quantised operands of attn_fwd's fp8 types, kWsSplit the
// split-KV partials, kWsBwd the backward's per-row statistics; separate
// buffers, so the paths never share memory.  Growth is stream-ordered: the
// old buffer is released with hipFreeAsync on the calling stream (after the
// work already queued there) and the new one taken with hipMallocAsync, so
// no call waits for the device.  Work queued on another stream that still
// uses the old buffer is not waited for: calls that share a workspace on
// different streams must not overlap (the header states it).
constexpr int kMaxDevices = 64;
enum { kWsFp8 = 0, kWsSplit = 1, kWsBwd = 2, kWsKinds = 3 };
struct Workspace {
  void* ptr = nullptr;
  size_t bytes = 0;
};
Workspace g_ws[kWsKinds][kMaxDevices];
std::mutex g_ws_mu;

int workspace(int kind, size_t bytes, hipStream_t s, void** out) {
  if (g_fail_next == ATTN_ERR_NOMEM) {
    g_fail_next = 0;
    return ATTN_ERR_NOMEM;
  }
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e);
  if (dev < 0 || dev >= kMaxDevices) return ATTN_ERR_ARG;
  std::lock_guard<std::mutex> lk(g_ws_mu);
  Workspace& w = g_ws[kind][dev];
  if (w.bytes < bytes) {
    if (w.ptr) {
      e = hipFreeAsync(w.ptr, s);
      if (e != hipSuccess) return hip_fail(e);
      w.ptr = nullptr;
      w.bytes = 0;
    }
    e = hipMallocAsync(&w.ptr, bytes, s);
    if (e != hipSuccess) {
      w.ptr = nullptr;
      (void)hipGetLastError();
      return e == hipErrorOutOfMemory ? ATTN_ERR_NOMEM : hip_fail(e);
    }
    w.bytes = bytes;
  }
  *out = w.ptr;
  return ATTN_OK;
}

constexpr int kMaxSplits = attn::kCombineMaxSplits;
constexpr int kSplitBlockM = 128;   // query rows per workgroup of the split / packed kernel
constexpr long long kAutoSplitGrid = 128;   // attn_fwd considers split-KV below this many workgroups
constexpr int kAutoSplitMinKeys = 4096;     // ... and from this many keys (shorter: the combine launch costs more)
// PackGQA (one tile holds the rows of every query head of a KV group) needs
// the group size to divide the 128-row block.  Automatic choice: pack when it
// gives strictly fewer 128-row tiles, i.e. when the unpacked tiles would be
// mostly empty (few query positions, as in decoding).
bool pack_allowed(int Hq, int Hkv) {
  const int g = Hq / Hkv;
  return g > 1 && kSplitBlockM % g == 0;
}
int pack_choice(int pack_gqa, int Hq, int Hkv, int Sq, int* pack) {
  const int g = Hq / Hkv;
  if (pack_gqa < -1 || pack_gqa > 1) return ATTN_ERR_ARG;
  if (pack_gqa == 1 && g > 1 && !pack_allowed(Hq, Hkv)) return ATTN_ERR_ARG;
  if (pack_gqa == -1) {
    const long long packed = ((long long)Sq * g + kSplitBlockM - 1) / kSplitBlockM;
    const long long unpacked = (long long)g * ((Sq + kSplitBlockM - 1) / kSplitBlockM);
    *pack = pack_allowed(Hq, Hkv) && packed < unpacked;
  } else {
    *pack = pack_gqa == 1 && g > 1;
  }
  return ATTN_OK;
}
// 128-row tiles of a dense problem, packed or not
long long dense_tiles(int B, int Hq, int Hkv, int Sq, int pack) {
  if (pack) return (long long)B * Hkv * (((long long)Sq * (Hq / Hkv) + kSplitBlockM - 1) / kSplitBlockM);
  return (long long)B * Hq * ((Sq + kSplitBlockM - 1) / kSplitBlockM);
}

// Split-KV plan over `tiles` 128-row tiles.  The key axis is cut into
// `splits` ranges of `split_keys` keys (a multiple of the 64-key tile); the
// last range may be shorter, none is empty.  num_splits > 0 asks for that
// many (fewer when Sk has fewer 64-key tiles).  num_splits == 0 models the
// time as (waves of workgroups over the device's resident slots) x (work of
// one workgroup: its share of the keys plus a fixed cost worth 128 keys) and
// takes the cheapest count, the smallest on ties, with ranges of at least
// 256 keys and at most 64 ranges.  Slots: 256 CUs (MI355X) times one
// (d = 128) or two (d = 64) workgroups of the 4-wave kernel.  At d = 128 two
// workgroups fit in a CU's LDS, but the count of one matches what the decode
// shape measures best (8 ranges 43.8 us against 16 ranges 49.8 us).
int split_plan(long long tiles, int Sk, int d, int num_splits, int* splits, int* split_keys) {
  if (num_splits < 0 || num_splits > kMaxSplits) return ATTN_ERR_ARG;
  const int kt = (Sk + 63) / 64;   // 64-key tiles
  int want = num_splits;
  if (want == 0) {
    const long long slots = 256LL * (d == 128 ? 1 : 2);
    int cap = (Sk + 255) / 256;
    if (cap > 64) cap = 64;
    want = 1;
    double best = 0.0;
    for (int n = 1; n <= cap; ++n) {
      const long long waves = (tiles * n + slots - 1) / slots;
      const double cost = (double)waves * ((double)Sk / n + 128.0);
      if (n == 1 || cost < best) {
        best = cost;
        want = n;
      }
    }
  }
  if (want > kt) want = kt;
  const int per = (kt + want - 1) / want;   // tiles per range
  *split_keys = per * 64;
  *splits = (Sk + per * 64 - 1) / (per * 64);
  if (tiles * *splits > kMax32) return ATTN_ERR_SIZE;
  return ATTN_OK;
}

void fill_params(attn::FwdParams& p, const void* q, const void* k, const void* v, void* o, float* lse, int B,
                 int Hq, int Hkv, int Sq, int Sk, int d, float scale) {
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
}

// Bytes of split-KV partials for `rows` query rows: O_p then LSE_p, each
// 256-byte aligned.
size_t split_partials_bytes(int splits, size_t rows, int d, size_t* o_bytes) {
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  *o_bytes = al(sizeof(float) * splits * rows * d);
  return *o_bytes + al(sizeof(float) * splits * rows);
}

// --- the fixed scratch of attn_fwd_splitkv_noalloc ------------------------
// A file-scope device array: every GPU the library runs on holds its own
// copy for the life of the process.  Host code never uses the array's name
// as an address (on the host it is only a stand-in): the device address is
// taken once per device with hipGetSymbolAddress and kept in g_scratch.
constexpr size_t kScratchBytes = (size_t)ATTN_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
void* g_scratch[kMaxDevices] = {};

int scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e);
  if (dev < 0 || dev >= kMaxDevices) return ATTN_ERR_ARG;
  std::lock_guard<std::mutex> lk(g_ws_mu);
  if (!g_scratch[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr) return hip_fail(e != hipSuccess ? e : hipErrorInvalidSymbol);
    g_scratch[dev] = ptr;
  }
  *out = g_scratch[dev];
  return ATTN_OK;
}

// Dense bf16/fp16 forward after validation: the plain kernels (splits == 1)
// or split-KV partials and their combine, with or without PackGQA.  The
// partials go to `fixed` when it is given (it holds at least their bytes),
// else to the lazily grown workspace.
int fwd16_dense(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv, int Sq,
                int Sk, int d, float scale, int causal, int pack, int splits, int split_keys, int dtype,
                hipStream_t s, void* fixed = nullptr) {
  attn::FwdParams p{};
  fill_params(p, q, k, v, o, lse, B, Hq, Hkv, Sq, Sk, d, scale);
  p.pack = pack;
  const int g = Hq / Hkv;
  const int bm = (pack || splits > 1) ? kSplitBlockM : attn::fwd_block_m(dtype, d, 0);
  p.tm = pack ? attn::make_tile_map(B, Hkv, Hkv, Sq * g, bm, causal) : attn::make_tile_map(B, Hq, Hkv, Sq, bm, causal);
  if (splits <= 1) {
    p.grid = p.tm.ntiles;
    hipError_t e = launch_gate();
    if (e == hipSuccess) e = attn::launch_fwd(p, dtype, d, causal, 0, s);
    return e == hipSuccess ? ATTN_OK : hip_fail(e);
  }
  size_t ob = 0;
  const size_t bytes = split_partials_bytes(splits, (size_t)B * Sq * Hq, d, &ob);
  void* ws = fixed;
  if (!ws) {
    int rc = workspace(kWsSplit, bytes, s, &ws);
    if (rc) return rc;
  }
  p.splits = splits;
  p.split_keys = split_keys;
  p.o_part = (float*)ws;
  p.lse_part = (float*)((uint8_t*)ws + ob);
  p.grid = p.tm.ntiles * splits;
  hipError_t e = launch_gate();
  if (e == hipSuccess) e = attn::launch_fwd_split(p, dtype, d, causal, s);
  if (e != hipSuccess) return hip_fail(e);
  return attn_combine(p.o_part, p.lse_part, o, lse, splits, B, Hq, Sq, d, dtype, s);
}

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
    case ATTN_ERR_SCRATCH: return "split-KV partials exceed the fixed scratch of attn_fwd_splitkv_noalloc";
    default: return "unknown status code";
  }
}

int attn_default_signs(float* signs_host, int n) {
  if (!signs_host) return ATTN_ERR_NULL;
  if (n <= 0 || n > 128) return ATTN_ERR_SHAPE;
  for (int i = 0; i < n; ++i) signs_host[i] = attn::default_sign(i);
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
  hipError_t e = launch_gate();
  if (e == hipSuccess) e = attn::launch_fwd_fp8(p, causal, (hipStream_t)stream);
  return e == hipSuccess ? ATTN_OK : hip_fail(e);
}

namespace {
attn::PrepassSeg prepass_seg(const float* x, uint8_t* x8, float* descale, int B, int S, int H, int transpose,
                             const float* signs, int default_signs) {
  attn::PrepassSeg g{};
  g.x = x;
  g.x8 = x8;
  g.descale = descale;
  g.signs = signs;
  g.default_signs = default_signs;
  g.B = B;
  g.S = S;
  g.H = H;
  g.transpose = transpose ? 1 : 0;
  g.blocks = B * H * ((S + 127) / 128);
  return g;
}
}  // namespace

int attn_fp8_prepass(const float* x, uint8_t* x8, float* descale, int B, int S, int H, int d,
                     int transpose_out, const float* signs, void* stream) {
  if (!x || !x8 || !descale) return ATTN_ERR_NULL;
  if (B <= 0 || S <= 0 || H <= 0) return ATTN_ERR_SHAPE;
  if (d != 128) return ATTN_ERR_HEADDIM;
  if ((long long)B * S * H * d > kMax32 * 2) return ATTN_ERR_SIZE;
  attn::PrepassParams p{};
  p.seg[0] = prepass_seg(x, x8, descale, B, S, H, transpose_out, signs, 0);
  p.nseg = 1;
  p.d = d;
  hipError_t e = launch_gate();
  if (e == hipSuccess) e = attn::launch_prepass(p, (hipStream_t)stream);
  return e == hipSuccess ? ATTN_OK : hip_fail(e);
}

int attn_fp8_prepass_qkv(const float* q, const float* k, const float* v, uint8_t* q8, uint8_t* k8, uint8_t* v8t,
                         float* q_descale, float* k_descale, float* v_descale, int B, int Hq, int Hkv, int Sq,
                         int Sk, int d, const float* signs, void* stream) {
  if (!q || !k || !v || !q8 || !k8 || !v8t || !q_descale || !k_descale || !v_descale) return ATTN_ERR_NULL;
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Sq <= 0 || Sk <= 0) return ATTN_ERR_SHAPE;
  if (d != 128) return ATTN_ERR_HEADDIM;
  if ((long long)B * Sq * Hq * d > kMax32 * 2 || (long long)B * Sk * Hkv * d > kMax32 * 2) return ATTN_ERR_SIZE;
  if ((long long)B * Hq * ((Sq + 127) / 128) + 2LL * B * Hkv * ((Sk + 127) / 128) > kMax32) return ATTN_ERR_SIZE;
  attn::PrepassParams p{};
  p.seg[0] = prepass_seg(q, q8, q_descale, B, Sq, Hq, 0, signs, 0);
  p.seg[1] = prepass_seg(k, k8, k_descale, B, Sk, Hkv, 0, signs, 0);
  p.seg[2] = prepass_seg(v, v8t, v_descale, B, Sk, Hkv, 1, nullptr, 0);
  p.nseg = 3;
  p.d = d;
  hipError_t e = launch_gate();
  if (e == hipSuccess) e = attn::launch_prepass(p, (hipStream_t)stream);
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
    rc = workspace(kWsFp8, total, s, &ws);
    if (rc) return rc;
    uint8_t* base = (uint8_t*)ws;
    uint8_t* q8 = base;
    uint8_t* k8 = q8 + al(qb);
    uint8_t* v8t = k8 + al(kb);
    float* qs = (float*)(v8t + al(kb));
    float* ks = (float*)((uint8_t*)qs + sq_b);
    float* vs = (float*)((uint8_t*)ks + sk_b);
    // one launch quantises Q, K and V^T; the Hadamard type rotates Q and K
    // with the default signs, which the prepass kernel holds in constant memory
    const int rot = dtype == ATTN_FP8_E4M3_HADAMARD ? 1 : 0;
    attn::PrepassParams pp{};
    pp.seg[0] = prepass_seg((const float*)q, q8, qs, B, Sq, Hq, 0, nullptr, rot);
    pp.seg[1] = prepass_seg((const float*)k, k8, ks, B, Sk, Hkv, 0, nullptr, rot);
    pp.seg[2] = prepass_seg((const float*)v, v8t, vs, B, Sk, Hkv, 1, nullptr, 0);
    pp.nseg = 3;
    pp.d = d;
    hipError_t e = launch_gate();
    if (e == hipSuccess) e = attn::launch_prepass(pp, s);
    rc = e == hipSuccess ? ATTN_OK : hip_fail(e);
    if (!rc) rc = attn_fwd_fp8(q8, k8, v8t, qs, ks, vs, o, lse, B, Hq, Hkv, Sq, Sk, d, scale, causal, stream);
    return rc;
  }

  if (!varlen) {
    int pack = 0;
    rc = pack_choice(-1, Hq, Hkv, Sq, &pack);
    if (rc) return rc;
    // Few query blocks over long keys (decoding): when the plain launch
    // would occupy under half the CUs and there are at least 4096 keys, cut
    // the key axis as attn_fwd_splitkv does if its planner finds that faster.
    const long long plain = pack ? dense_tiles(B, Hq, Hkv, Sq, 1)
                                 : (long long)B * Hq * ((Sq + attn::fwd_block_m(dtype, d, 0) - 1) /
                                                        attn::fwd_block_m(dtype, d, 0));
    int splits = 1, split_keys = 0;
    if (plain < kAutoSplitGrid && Sk >= kAutoSplitMinKeys) {
      rc = split_plan(dense_tiles(B, Hq, Hkv, Sq, pack), Sk, d, 0, &splits, &split_keys);
      if (rc) return rc;
    }
    return fwd16_dense(q, k, v, o, lse, B, Hq, Hkv, Sq, Sk, d, scale, causal, pack, splits, split_keys, dtype, s);
  }
  attn::FwdParams p{};
  fill_params(p, q, k, v, o, lse, B, Hq, Hkv, Sq, Sk, d, scale);
  p.cu_seqlens = cu_seqlens;
  // one tile per (head, query block of a sequence); the number of blocks is
  // at most ceil(T / BM) + (number of sequences), the rest exit at once
  const int bm = attn::fwd_block_m(dtype, d, 1);
  const long long nb = (Sq + bm - 1) / bm + B;
  if (nb * Hq > kMax32) return ATTN_ERR_SIZE;
  p.grid = (int)(nb * Hq);
  hipError_t e = launch_gate();
  if (e == hipSuccess) e = attn::launch_fwd(p, dtype, d, causal, 1, s);
  return e == hipSuccess ? ATTN_OK : hip_fail(e);
}

int attn_split_plan(int B, int Hq, int Hkv, int Sq, int Sk, int d, int num_splits, int pack_gqa, int* splits_out,
                    int* split_keys_out, int* pack_out) {
  if (!splits_out || !split_keys_out || !pack_out) return ATTN_ERR_NULL;
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Sq <= 0 || Sk <= 0) return ATTN_ERR_SHAPE;
  if (d != 64 && d != 128) return ATTN_ERR_HEADDIM;
  if (Hq % Hkv) return ATTN_ERR_GQA;
  int rc = pack_choice(pack_gqa, Hq, Hkv, Sq, pack_out);
  if (rc) return rc;
  return split_plan(dense_tiles(B, Hq, Hkv, Sq, *pack_out), Sk, d, num_splits, splits_out, split_keys_out);
}

int attn_combine(const float* o_part, const float* lse_part, void* o, float* lse, int splits, int B,
                 int Hq, int Sq, int d, int dtype, void* stream) {
  if (!o_part || !lse_part || !o) return ATTN_ERR_NULL;
  if (splits <= 0 || B <= 0 || Hq <= 0 || Sq <= 0) return ATTN_ERR_SHAPE;
  if (splits > attn::kCombineMaxSplits) return ATTN_ERR_ARG;
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
  hipError_t e = launch_gate();
  if (e == hipSuccess) e = attn::launch_combine(p, dtype, (hipStream_t)stream);
  return e == hipSuccess ? ATTN_OK : hip_fail(e);
}

int attn_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq,
                     int Hkv, int Sq, int Sk, int d, float scale, int causal, int num_splits, int pack_gqa,
                     int dtype, void* stream) {
  if (!q || !k || !v || !o) return ATTN_ERR_NULL;
  if (dtype != ATTN_BF16 && dtype != ATTN_FP16) return ATTN_ERR_DTYPE;
  int rc = check_common(B, Hq, Hkv, Sq, Sk, d, scale);
  if (rc) return rc;
  int pack = 0, splits = 0, split_keys = 0;
  rc = pack_choice(pack_gqa, Hq, Hkv, Sq, &pack);
  if (rc) return rc;
  rc = split_plan(dense_tiles(B, Hq, Hkv, Sq, pack), Sk, d, num_splits, &splits, &split_keys);
  if (rc) return rc;
  return fwd16_dense(q, k, v, o, lse, B, Hq, Hkv, Sq, Sk, d, scale, causal, pack, splits, split_keys, dtype,
                     (hipStream_t)stream);
}

int attn_fwd_splitkv_noalloc(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq,
                             int Hkv, int Sq, int Sk, int d, float scale, int causal, int num_splits, int pack_gqa,
                             int dtype, void* stream) {
  if (!q || !k || !v || !o) return ATTN_ERR_NULL;
  if (dtype != ATTN_BF16 && dtype != ATTN_FP16) return ATTN_ERR_DTYPE;
  int rc = check_common(B, Hq, Hkv, Sq, Sk, d, scale);
  if (rc) return rc;
  int pack = 0, splits = 0, split_keys = 0;
  rc = pack_choice(pack_gqa, Hq, Hkv, Sq, &pack);
  if (rc) return rc;
  rc = split_plan(dense_tiles(B, Hq, Hkv, Sq, pack), Sk, d, num_splits, &splits, &split_keys);
  if (rc) return rc;
  void* fixed = nullptr;
  if (splits > 1) {
    size_t ob = 0;
    if (split_partials_bytes(splits, (size_t)B * Sq * Hq, d, &ob) > kScratchBytes) return ATTN_ERR_SCRATCH;
    rc = scratch_address(&fixed);
    if (rc) return rc;
  }
  return fwd16_dense(q, k, v, o, lse, B, Hq, Hkv, Sq, Sk, d, scale, causal, pack, splits, split_keys, dtype,
                     (hipStream_t)stream, fixed);
}

int attn_fwd_ext(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv,
                 int Sq, int Sk, int d, float scale, int causal, const int32_t* cu_seqlens, int dtype,
                 float softcap, int v_colmajor, void* stream) {
  if (!isfinite(softcap) || softcap < 0.f) return ATTN_ERR_ARG;
  if (softcap == 0.f && !v_colmajor)
    return attn_fwd(q, k, v, o, lse, B, Hq, Hkv, Sq, Sk, d, scale, causal, cu_seqlens, dtype, stream);
  if (!q || !k || !v || !o) return ATTN_ERR_NULL;
  if (dtype < ATTN_BF16 || dtype > ATTN_FP8_E4M3_HADAMARD) return ATTN_ERR_DTYPE;
  if (dtype != ATTN_BF16 && dtype != ATTN_FP16) return ATTN_ERR_ARG;   // features: 16-bit types only
  if (cu_seqlens) return ATTN_ERR_ARG;                                  // features: dense only
  int rc = check_common(B, Hq, Hkv, Sq, Sk, d, scale);
  if (rc) return rc;
  if (v_colmajor && Sk % 8 != 0) return ATTN_ERR_SHAPE;                 // 16-byte aligned rows of V^T
  attn::FwdParams p{};
  fill_params(p, q, k, v, o, lse, B, Hq, Hkv, Sq, Sk, d, scale);
  p.feat = (softcap > 0.f ? attn::kFeatSoftcap : 0) | (v_colmajor ? attn::kFeatVCol : 0);
  if (softcap > 0.f) {
    p.softcap_a = softcap / scale;
    p.softcap_b2 = 2.f * scale * 1.4426950408889634f / softcap;
  }
  p.tm = attn::make_tile_map(B, Hq, Hkv, Sq, kSplitBlockM, causal);
  p.grid = p.tm.ntiles;
  hipError_t e = launch_gate();
  if (e == hipSuccess) e = attn::launch_fwd(p, dtype, d, causal, 0, (hipStream_t)stream);
  return e == hipSuccess ? ATTN_OK : hip_fail(e);
}

int attn_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
             const float* dlse, void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int Sq, int Sk, int d,
             float scale, int causal, const int32_t* cu_seqlens, int dtype, void* stream) {
  if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv) return ATTN_ERR_NULL;
  if (dtype != ATTN_BF16 && dtype != ATTN_FP16) return ATTN_ERR_DTYPE;
  const bool varlen = cu_seqlens != nullptr;
  if (varlen) {
    if (B <= 0) return ATTN_ERR_SHAPE;
    if (Sq != Sk) return ATTN_ERR_SHAPE;
  }
  int rc = check_common(varlen ? 1 : B, Hq, Hkv, Sq, Sk, d, scale);
  if (rc) return rc;
  // dK/dV workgroups: (batch, KV head, 128 keys); varlen: at most
  // ceil(T / 128) + (number of sequences) key blocks per KV head
  const long long nkb = varlen ? (Sk + attn::kBwdBlockN - 1) / attn::kBwdBlockN + B
                               : (long long)B * ((Sk + attn::kBwdBlockN - 1) / attn::kBwdBlockN);
  const long long nqb = varlen ? (Sq + attn::kBwdBlockM - 1) / attn::kBwdBlockM + B : 0;
  if ((long long)Hkv * nkb > kMax32 || (long long)Hq * nqb > kMax32) return ATTN_ERR_SIZE;
  const int sq_pad = varlen ? Sq : (Sq + 31) / 32 * 32;
  void* ws = nullptr;
  // (+32 spare pairs: the varlen dK/dV kernel reads its 32 rows of a step
  // from one address, past the last token on the last head)
  rc = workspace(kWsBwd, sizeof(float) * 2 * ((size_t)(varlen ? 1 : B) * Hq * sq_pad + 32), (hipStream_t)stream, &ws);
  if (rc) return rc;
  attn::BwdParams p{};
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.dout = dout;
  p.lse = lse;
  p.dlse = dlse;
  p.dq = dq;
  p.dk = dk;
  p.dv = dv;
  p.stats = (float2*)ws;
  p.cu_seqlens = cu_seqlens;
  p.B = B;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.Sq = Sq;
  p.Sk = Sk;
  p.Sq_pad = sq_pad;
  p.group = Hq / Hkv;
  p.scale = scale;
  p.scale_log2 = scale * 1.4426950408889634f;
  if (varlen) {
    p.grid_dq = (int)(Hq * nqb);
  } else {
    p.tm = attn::make_tile_map(B, Hq, Hkv, Sq, attn::kBwdBlockM, causal);
    p.grid_dq = p.tm.ntiles;
  }
  p.grid_dkdv = (int)(Hkv * nkb);
  hipError_t e = launch_gate();
  if (e == hipSuccess) e = attn::launch_bwd(p, dtype, d, causal, varlen ? 1 : 0, (hipStream_t)stream);
  return e == hipSuccess ? ATTN_OK : hip_fail(e);
}

int attn_clock_probe(unsigned long long* out, int wall_ticks, int* wall_khz, void* stream) {
  if (!out || !wall_khz) return ATTN_ERR_NULL;
  if (wall_ticks <= 0) return ATTN_ERR_ARG;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(wall_khz, hipDeviceAttributeWallClockRate, dev);
  if (e == hipSuccess) e = launch_gate();
  if (e == hipSuccess) e = attn::launch_clock_probe(out, wall_ticks, (hipStream_t)stream);
  return e == hipSuccess ? ATTN_OK : hip_fail(e);
}

int attn_test_fail_next(int code) {
  if (code != 0 && code != ATTN_ERR_NOMEM && code != ATTN_ERR_HIP) return ATTN_ERR_ARG;
  g_fail_next = code;
  return ATTN_OK;
}

void attn_release(void) {
  std::lock_guard<std::mutex> lk(g_ws_mu);
  int cur = 0;
  if (hipGetDevice(&cur) != hipSuccess) return;
  for (int dev = 0; dev < kMaxDevices; ++dev) {
    bool any = false;
    for (int k = 0; k < kWsKinds; ++k) any = any || g_ws[k][dev].ptr != nullptr;
    if (!any) continue;
    if (hipSetDevice(dev) != hipSuccess) continue;
    (void)hipDeviceSynchronize();
    for (int k = 0; k < kWsKinds; ++k) {
      if (g_ws[k][dev].ptr) (void)hipFreeAsync(g_ws[k][dev].ptr, nullptr);
      g_ws[k][dev] = Workspace{};
    }
    (void)hipDeviceSynchronize();
  }
  (void)hipSetDevice(cur);
}

}  // extern "C"
