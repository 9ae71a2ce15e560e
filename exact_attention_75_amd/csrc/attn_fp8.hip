// attn_fp8.hip -- fp8 (OCP E4M3) path of the attention forward for gfx950.
//
// Two kernels:
//  * prepass_kernel: per (batch, head, block of 128 rows) -- optional signed
//    128-point Hadamard rotation of each row in fp32, the block's amax, the
//    fp32 scale s = amax / 448 (1 for an all-zero block), and the codes
//    E4M3(clip(x / s, -448, 448)) with round-to-nearest-even.  This is the
//    per-block scaling and incoherence processing of "FlashAttention-3 Deep
//    Dive" (mojostudio.in), section 4; 448 is that section's clip bound and
//    the format's largest finite value.  The codes are written row-major, or
//    transposed (token index innermost) for V, whose second-GEMM operand
//    wants the key index contiguous.
//  * fwd_fp8_kernel: the fused forward with both GEMMs on the fp8 MFMA
//    (v_mfma_scale_f32_32x32x64_f8f6f4, fp32 accumulation).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <type_traits>

#include "kernel_common.h"
#include "kernels.h"

namespace attn {

int fwd_fp8_block_m() { return 128; }

// ============================================================================
// prepass
// ============================================================================
//
// One workgroup of 256 threads per block of 128 rows of one (batch, head) of
// one tensor; a launch covers up to three tensors (segments), so the Q, K and
// V^T of the fp8 forward are quantised in one launch.  Three block paths:
//  * row-major codes, no rotation: coalesced loads (in each load, lanes 0-31
//    read one 512-byte row and lanes 32-63 another), 128-byte code rows out;
//  * transposed codes (V^T), no rotation: the same coalesced loads, each lane
//    keeping 16 consecutive rows of its 4 channels, a byte transpose in
//    registers (v_perm) and in LDS, and 128-byte code rows of V^T out;
//  * rotation: thread t owns row t/2, channels 64 (t % 2) .. +63, in
//    registers; the rotation's last butterfly stage (distance 64) pairs the
//    two threads of a row, neighbouring lanes.

__device__ __forceinline__ float lane_xor1(float x) {
  // value of lane l ^ 1 (DPP quad permutation [1, 0, 3, 2])
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, false));
}

// The default sign vector, generated at compile time: the rotation of
// attn_fwd's Hadamard type reads it from constant memory, so no call has to
// copy it to the device first.
struct SignTable {
  float v[128];
};
constexpr SignTable make_default_signs() {
  SignTable t{};
  for (int i = 0; i < 128; ++i) t.v[i] = default_sign(i);
  return t;
}
__constant__ SignTable kDefaultSigns = make_default_signs();

// Streaming accesses: every input element is read once and every code
// written once, so the coalesced paths load and all paths store through the
// non-temporal path (no cache allocation; measured 8-12% faster on the
// c3fp8 / c5 tensors, where the one-launch prepass then moves its bytes as
// fast as a plain device copy).
typedef float nf4 __attribute__((ext_vector_type(4)));
typedef unsigned nu4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ float4 load_stream(const float* p) {
  const nf4 t = __builtin_nontemporal_load((const nf4*)p);
  return make_float4(t[0], t[1], t[2], t[3]);
}
__device__ __forceinline__ void store_stream(uint8_t* p, nu4 v) { __builtin_nontemporal_store(v, (nu4*)p); }

// correctly rounded v / s (Markstein: q0 within one ulp of the quotient, the
// remainder v - q0 s exact in one FMA, one more FMA q0 + r inv rounds to the
// nearest quotient; a subnormal quotient may be one ulp off, which no E4M3
// code resolves: they all map to zero), then clipped to the E4M3 range
__device__ __forceinline__ float quot_clip(float v, float s, float inv) {
  const float q0 = v * inv;
  const float r = __builtin_fmaf(-q0, s, v);
  return fminf(fmaxf(__builtin_fmaf(r, inv, q0), -448.0f), 448.0f);
}

// block amax of the workgroup: per-lane value -> every thread
__device__ __forceinline__ float block_amax(float am, float* red, int tid) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) am = fmaxf(am, __shfl_xor(am, off));
  if ((tid & 63) == 0) red[tid >> 6] = am;
  __syncthreads();
  return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

__global__ void __launch_bounds__(256) prepass_kernel(PrepassParams pp) {
  constexpr int ROWS = 128, D = 128, HALF = 64;
  // this workgroup's segment and block
  int si = 0, local = blockIdx.x;
  while (si + 1 < pp.nseg && local >= pp.seg[si].blocks) {
    local -= pp.seg[si].blocks;
    ++si;
  }
  const PrepassSeg g = pp.seg[si];
  const int nblk = (g.S + ROWS - 1) / ROWS;
  const int blk = local % nblk;
  const int h = (local / nblk) % g.H;
  const int b = local / (nblk * g.H);
  const int tid = threadIdx.x;
  const int row0 = blk * ROWS;
  const int nrows = min(ROWS, g.S - row0);
  const int lane = tid & 63, w = tid >> 6;

  __shared__ float red[4];
  // transposed codes; a 176-byte row stride spreads the 16-byte writes of
  // neighbouring channels over the banks
  __shared__ __attribute__((aligned(16))) uint8_t tT[D][ROWS + 48];

  const float* signs = g.default_signs ? kDefaultSigns.v : g.signs;
  if (signs == nullptr) {
    // coalesced: lane half hl of wave w reads rows 32 w + 16 hl + k (k-th
    // load) for transposed output, 32 w + 2 k + hl for row-major output, 4
    // channels c4 .. c4 + 3 each
    const int hl = lane >> 5;
    const int c4 = 4 * (lane & 31);
    auto row_of = [&](int k) { return g.transpose ? 32 * w + 16 * hl + k : 32 * w + 2 * k + hl; };
    float4 xv[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int rr = row_of(k);
      if (rr < nrows) {
        const long long ri = ((long long)b * g.S + row0 + rr) * g.H + h;
        xv[k] = load_stream(g.x + ri * D + c4);
      } else {
        xv[k] = make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
    float am = 0.f;
#pragma unroll
    for (int k = 0; k < 16; ++k)
      am = fmaxf(fmaxf(am, fmaxf(fabsf(xv[k].x), fabsf(xv[k].y))), fmaxf(fabsf(xv[k].z), fabsf(xv[k].w)));
    am = block_amax(am, red, tid);
    const float s = am > 0.f ? am / 448.0f : 1.0f;
    if (tid == 0) g.descale[((long long)b * g.H + h) * nblk + blk] = s;
    const float inv = 1.0f / s;
    uint32_t code[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      int c = __builtin_amdgcn_cvt_pk_fp8_f32(quot_clip(xv[k].x, s, inv), quot_clip(xv[k].y, s, inv), 0, false);
      code[k] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(quot_clip(xv[k].z, s, inv), quot_clip(xv[k].w, s, inv),
                                                         c, true);
    }
    if (!g.transpose) {
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const int rr = row_of(k);
        if (rr < nrows) {
          const long long ri = ((long long)b * g.S + row0 + rr) * g.H + h;
          __builtin_nontemporal_store(code[k], (uint32_t*)(g.x8 + ri * D + c4));
        }
      }
      return;
    }
    // byte transpose of 4 rows x 4 channels at a time: col[j] holds channel
    // c4 + j of rows 4 i .. 4 i + 3 (v_perm picks bytes of {S0, S1}, S1 low)
    uint32_t col[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t c0 = code[4 * i], c1 = code[4 * i + 1], c2 = code[4 * i + 2], c3 = code[4 * i + 3];
      const uint32_t lo01 = __builtin_amdgcn_perm(c1, c0, 0x05010400u);   // c0.0 c1.0 c0.1 c1.1
      const uint32_t hi01 = __builtin_amdgcn_perm(c1, c0, 0x07030602u);   // c0.2 c1.2 c0.3 c1.3
      const uint32_t lo23 = __builtin_amdgcn_perm(c3, c2, 0x05010400u);
      const uint32_t hi23 = __builtin_amdgcn_perm(c3, c2, 0x07030602u);
      col[0][i] = __builtin_amdgcn_perm(lo23, lo01, 0x05040100u);
      col[1][i] = __builtin_amdgcn_perm(lo23, lo01, 0x07060302u);
      col[2][i] = __builtin_amdgcn_perm(hi23, hi01, 0x05040100u);
      col[3][i] = __builtin_amdgcn_perm(hi23, hi01, 0x07060302u);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
      *(uint4*)(&tT[c4 + j][32 * w + 16 * hl]) = make_uint4(col[j][0], col[j][1], col[j][2], col[j][3]);
  } else {
    // ---- rotation: the thread's 64 channels of row r
    const int r = tid >> 1, half = tid & 1;
    const bool live = r < nrows;
    float x[HALF];
    const long long rowidx = ((long long)b * g.S + row0 + r) * g.H + h;
    const float* src = g.x + rowidx * D + half * HALF;
    if (live) {
#pragma unroll
      for (int i = 0; i < HALF; i += 4) {
        // cached loads: a lane reads 256 contiguous bytes across these 16
        // loads while a load instruction touches 64 separate 16-byte pieces,
        // so each cache line serves several instructions (streaming loads,
        // which do not allocate, fetched the lines again: twice as slow)
        const float4 v = *(const float4*)(src + i);
        x[i] = v.x;
        x[i + 1] = v.y;
        x[i + 2] = v.z;
        x[i + 3] = v.w;
      }
    } else {
#pragma unroll
      for (int i = 0; i < HALF; ++i) x[i] = 0.f;
    }
    // x <- (x * signs) H_128 / sqrt(128), in fp32
#pragma unroll
    for (int i = 0; i < HALF; ++i) x[i] *= signs[half * HALF + i];
#pragma unroll
    for (int len = 1; len < HALF; len <<= 1)
#pragma unroll
      for (int i = 0; i < HALF; ++i)
        if ((i & len) == 0) {
          const float a = x[i], c = x[i + len];
          x[i] = a + c;
          x[i + len] = a - c;
        }
    // distance-64 stage across the two threads of the row
#pragma unroll
    for (int i = 0; i < HALF; ++i) {
      const float other = lane_xor1(x[i]);
      x[i] = half == 0 ? x[i] + other : other - x[i];
    }
    const float norm = 0.08838834764831845f;   // 1 / sqrt(128)
#pragma unroll
    for (int i = 0; i < HALF; ++i) x[i] *= norm;
    float am = 0.f;
#pragma unroll
    for (int i = 0; i < HALF; ++i) am = fmaxf(am, fabsf(x[i]));
    am = block_amax(am, red, tid);
    const float s = am > 0.f ? am / 448.0f : 1.0f;
    if (tid == 0) g.descale[((long long)b * g.H + h) * nblk + blk] = s;
    const float inv = 1.0f / s;
    uint32_t q[HALF / 4];
#pragma unroll
    for (int i = 0; i < HALF; i += 4) {
      int c = __builtin_amdgcn_cvt_pk_fp8_f32(quot_clip(x[i], s, inv), quot_clip(x[i + 1], s, inv), 0, false);
      q[i / 4] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(quot_clip(x[i + 2], s, inv), quot_clip(x[i + 3], s, inv),
                                                          c, true);
    }
    if (!g.transpose) {
      if (live) {
        uint8_t* dst = g.x8 + rowidx * D + half * HALF;
#pragma unroll
        for (int i = 0; i < HALF / 16; ++i)
          store_stream(dst + 16 * i, nu4{q[4 * i], q[4 * i + 1], q[4 * i + 2], q[4 * i + 3]});
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < HALF; ++i) tT[half * HALF + i][r] = (uint8_t)(q[i >> 2] >> (8 * (i & 3)));
  }

  // ---- transposed output [B, H, d, S]: 8 consecutive lanes write one
  // channel's 128 bytes of the block
  __syncthreads();
  const long long plane = ((long long)b * g.H + h) * D;
  if (nrows == ROWS && (g.S & 15) == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = 32 * i + (tid >> 3), piece = tid & 7;
      store_stream(g.x8 + (plane + c) * g.S + row0 + 16 * piece, *(const nu4*)(&tT[c][16 * piece]));
    }
  } else {
    for (int i = tid; i < D * nrows; i += 256) {
      const int c = i / nrows, t = i % nrows;
      g.x8[(plane + c) * g.S + row0 + t] = tT[c][t];
    }
  }
}

hipError_t launch_prepass(const PrepassParams& p, hipStream_t s) {
  long long grid = 0;
  for (int i = 0; i < p.nseg; ++i) grid += p.seg[i].blocks;
  hipLaunchKernelGGL(prepass_kernel, dim3((unsigned)grid), dim3(256), 0, s, p);
  return hipGetLastError();
}

// ============================================================================
// fp8 forward
// ============================================================================
//
// A workgroup of 4 waves owns 128 query rows (one Q scale block), each wave
// 32 rows; three workgroups share a CU (three waves per SIMD: the kernel is
// held to 168 registers, for which the Q block sits in LDS, 48 KiB with the
// K/V stages, and is read again per tile).  Tiles of 64 keys (half a K/V
// scale block).  Per tile and wave:
//   S^T = K Q^T  : 2 blocks of 32 keys x 2 k-steps of 64 channels, on
//                  v_mfma_scale_f32_32x32x64_f8f6f4 (E8M0 operand scales = 1)
//   O^T += V^T P^T: one MFMA per 32 output channels, K = the tile's 64 keys.
// Key rows of block b are fed in the order pi_b(r) = 32*bit2(r) + 16 b +
// 4*(r >> 3) + (r & 3), which makes the 16 accumulator elements of lane half
// h in block b the keys 32 h + 16 b + 0..15: the lane's 32 probabilities are
// then the 32 consecutive keys the second MFMA's B operand wants, and V^T
// (token index innermost, from the prepass) gives the A operand as plain
// 32-byte LDS reads.
//
// Scales: scores are sq * sk_t * (Q~ K~^T) (sq per 128 query rows, sk_t per
// 128 keys), folded into the exp2 argument.  O accumulates in one unit for
// every V block: sv_ref / 2^4, sv_ref the largest V block scale among the
// blocks the workgroup's rows can see.  The ratio sv_t / sv_ref of the
// tile's V block (log2 lv <= 0) is split as lv = e + f with the integer
// e = ceil(lv) <= 0 and f in (-1, 0]: 2^e is the MFMA's E8M0 scale of the
// V operand (exact, any size), and only 2^f enters the probabilities,
// P' = 2^(4 + f) exp2(c s - m), m a lazily updated running max.  So P' does
// not shrink with the V block ratio: a block whose scale is far below the
// largest keeps its probabilities in the normal E4M3 range (folding the
// whole ratio into P' sent them to subnormals or zero, and rows that see
// only such blocks lost their output).
// No per-tile row max is taken: a tile's P' are computed against the
// current m and their sum over the lane's 32 keys, which bounds each of
// them, is checked against PMAX = 448 (the largest E4M3 value).  Only when
// some lane exceeds it (or m is not set yet) does m move to 4 above the
// tile's row max, with O and l rescaled and the tile's P' recomputed; O is
// otherwise never rescaled.  The row sum is taken over the fp32 values and
// converted to l's units with 2^(-4 - f) per tile.  The factor 2^4 keeps a
// lane's sum of 32 P' well under 448 when the max is current (a factor 2^6
// put the typical sum near 300 on N(0,1) scores, and the rare path ran on a
// large share of the tiles).

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x16 mma_fp8(const i32x8& a, const i32x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}
// the same product with the A operand scaled by 2^(a_scale - 127) (E8M0)
__device__ __forceinline__ f32x16 mma_fp8_sa(const i32x8& a, const i32x8& b, const f32x16& c, int a_scale) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, a_scale, 0, 127);
}

// K tile row r (128 bytes = 8 chunks): chunk c stored at c ^ swz_k8(r)
__device__ __forceinline__ int swz_k8(int r) { return ((r >> 1) & 3) | ((r >> 3) & 4); }
// V^T tile row r (64 bytes = 4 chunks): chunk c stored at c ^ swz_v8(r)
__device__ __forceinline__ int swz_v8(int r) { return (r >> 2) & 3; }
// key of MFMA row r in block b of a 64-key tile
__device__ __forceinline__ int key_perm8(int r, int b) { return 32 * ((r >> 2) & 1) + 16 * b + 4 * (r >> 3) + (r & 3); }

template <bool CAUSAL>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3, 3)))
fwd_fp8_kernel(Fp8FwdParams p) {
  constexpr int NW = 4, BM = 128, BN = 64, D = 128;
  constexpr int KROW = D;               // bytes per K row
  constexpr int VROW = BN;              // bytes per V^T row (keys of a tile)
  constexpr int TILE = BN * KROW;       // 8 KiB, same for V^T (D * VROW)
  constexpr int LOADS = TILE / 16 / (NW * 64);   // DMA instructions per wave per tensor
  constexpr float NEG_INF = -__builtin_inff();
  constexpr float POFF = 4.0f;          // log2 of P' for a probability of 1 at the running max
  constexpr float PMAX = 448.0f;        // bound on a lane's share of a tile's sum of P' (E4M3 max)
  __shared__ __attribute__((aligned(16))) char smem[4 * TILE + BM * D];   // [K0 | K1 | V0 | V1 | Q]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5;
  const int l32 = lane & 31;

  int b, hq, mblk;
  tile_decode(p.tm, blockIdx.x, b, hq, mblk);
  const int hkv = hq / p.group;
  const int q_len = p.Sq, kv_len = p.Sk;
  const int nbq = (p.Sq + 127) / 128, nbk = (p.Sk + 127) / 128;
  const int qs = p.Hq * D, ks = p.Hkv * D;
  const uint8_t* Qp = p.q8 + (long long)b * p.Sq * qs + hq * D;
  const uint8_t* Kp = p.k8 + (long long)b * p.Sk * ks + hkv * D;
  const uint8_t* Vt = p.v8t + ((long long)b * p.Hkv + hkv) * D * p.Sk;
  const float* ksc = p.k_descale + ((long long)b * p.Hkv + hkv) * nbk;
  const float* vsc = p.v_descale + ((long long)b * p.Hkv + hkv) * nbk;
  const float sq = p.q_descale[((long long)b * p.Hq + hq) * nbq + mblk];

  const int q0 = mblk * BM;
  const int qw = q0 + wave * 32;
  const int q_hi = q0 + BM < q_len ? q0 + BM : q_len;
  const int kv_end = CAUSAL ? (kv_len < q_hi ? kv_len : q_hi) : kv_len;
  const int ntile = (kv_end + BN - 1) / BN;
  // O's unit: the largest V block scale among the blocks these rows see
  // (uniform loads)
  float sv_max = 0.f;
  for (int i = 0; i < (kv_end + 127) / 128; ++i) sv_max = fmaxf(sv_max, vsc[i]);
  const float lsv_max = log2f(sv_max);
  const int qi = qw + l32;

  // Q block in LDS (its 16 registers per lane would cost the third wave per
  // SIMD): this wave's 32 rows, copied by its own loads (the first tile's
  // wait covers them), chunk c of row r at c ^ ((r >> 1) & 7) so that the 16
  // rows one read cycle serves hit 16 different bank groups; rows past the
  // end read as zeros
  {
    uint32_t qdma[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int pos = i * 64 + lane;
      const int r = pos >> 3, c = pos & 7;
      qdma[i] = (uint32_t)(r * qs + ((c ^ ((r >> 1) & 7)) << 4));
    }
    const uint32_t qbytes = qw < q_len ? (uint32_t)(q_len - qw) * (uint32_t)qs : 0u;
    copy_rows_to_lds<4>((const void*)(Qp + (long long)(qw < q_len ? qw : 0) * qs), qbytes, smem + 4 * TILE + wave * 4096, qdma);
  }
  // lane's Q operand of k-step kk: query qi, channels 64 kk + 32 h .. +31
  int qoff[2];
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) qoff[kk] = 4 * TILE + (wave * 32 + l32) * D + (((4 * kk + 2 * h) ^ ((l32 >> 1) & 7)) << 4);

  // K / V^T copies (direct to LDS, swizzled through the fetch addresses)
  uint32_t kdma[LOADS], vdma[LOADS];
#pragma unroll
  for (int i = 0; i < LOADS; ++i) {
    const int pos = (wave * LOADS + i) * 64 + lane;
    const int kr = pos >> 3, kc = pos & 7;
    kdma[i] = (uint32_t)(kr * ks + ((kc ^ swz_k8(kr)) << 4));
    const int vr = pos >> 2, vc = pos & 3;
    vdma[i] = (uint32_t)(vr * p.Sk + ((vc ^ swz_v8(vr)) << 4));
  }
  auto issue = [&](int t, int stage) {
    const int j0 = t * BN;
    copy_rows_to_lds<LOADS>((const void*)(Kp + (long long)j0 * ks), (uint32_t)(kv_len - j0) * (uint32_t)ks,
                            smem + stage * TILE + wave * LOADS * 1024, kdma);
    copy_rows_to_lds<LOADS>((const void*)(Vt + j0), (uint32_t)(D * p.Sk - j0),
                            smem + (2 + stage) * TILE + wave * LOADS * 1024, vdma);
  };

  // per-lane LDS read offsets
  int koff[2][2];   // [block][kk]: key row pi_b(l32), chunks 4 kk + 2 h (+1)
#pragma unroll
  for (int bb = 0; bb < 2; ++bb)
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int r = key_perm8(l32, bb);
      koff[bb][kk] = r * KROW + (((4 * kk + 2 * h) ^ swz_k8(r)) << 4);
    }
  int voff[4];      // [db]: V^T row 32 db + l32, chunks 2 h (+1)
#pragma unroll
  for (int db = 0; db < 4; ++db) {
    const int r = 32 * db + l32;
    voff[db] = r * VROW + (((2 * h) ^ swz_v8(r)) << 4);
  }
  // The second chunk of each 32-byte read (K, V^T and Q): chunk 2h + 1 sits
  // at the first one's position XOR 1 (the swizzle acts on the whole chunk
  // index, and 2h has bit 0 clear), i.e. at byte offset XOR 16; one XOR per
  // read instead of a second register of offsets.
  f32x16 o[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) o[db] = f32x16{};
  float m_run = NEG_INF, l_run = 0.f;
  const float cbase = p.scale_log2 * sq;

  const int n_w = CAUSAL ? min(ntile, (qw + 31) / BN + 1) : ntile;

  float msub = 0.f;
  // factors of the current 128-key scale block, shared by the two tiles of
  // an unrolled pair (t even, t + 1): formed in the first of them
  float c = 0.f, lv = 0.f;
  int vscale = 127;
  // One key tile: barrier, the next tile's copies, and -- for tiles this
  // wave computes -- S, the probabilities, the sum check and PV.  STAGE is
  // t % 2, a constant, so every LDS read is a per-lane base plus an
  // immediate offset.
  auto step = [&](int t, auto stage_tag) {
    constexpr int STAGE = decltype(stage_tag)::value;
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    if (t + 1 < ntile) issue(t + 1, STAGE ^ 1);
    if (t >= n_w) return;
    const char* Ks = smem + STAGE * TILE;
    const char* Vs = smem + (2 + STAGE) * TILE;
    const int j0 = t * BN;
    if constexpr (STAGE == 0) {
      // block scales by scalar loads (a vector load would queue behind the
      // copies in flight and make the tile wait for them)
      c = cbase * ((const __attribute__((address_space(4))) float*)ksc)[j0 >> 7];
      // V block ratio 2^lv = 2^(e + f): 2^e as the E8M0 scale of V (clamped
      // at the format's 2^-127), 2^f in P'
      const float lv_all = log2f(((const __attribute__((address_space(4))) float*)vsc)[j0 >> 7]) - lsv_max;
      vscale = max(0, 127 + (int)ceilf(lv_all));
      lv = lv_all - (float)(vscale - 127);   // (-1, 0] unless clamped
    }

    // ---- S^T = K Q^T.  Each MFMA group runs at raised wave priority: the
    // other wave on this SIMD (another workgroup's) is then mostly in its
    // softmax, and its vector instructions fill the cycles of these MFMAs
    // instead of holding them back (at equal priority the older wave wins
    // the issue arbitration whatever it issues).
    i32x8 qf[2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const i32x4 lo = *(const i32x4*)(smem + qoff[kk]);
      const i32x4 hi = *(const i32x4*)(smem + (qoff[kk] ^ 16));
      qf[kk] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    }
    f32x16 s[2];
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int bb = 0; bb < 2; ++bb) {
      s[bb] = f32x16{};
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const i32x4 lo = *(const i32x4*)(Ks + koff[bb][kk]);
        const i32x4 hi = *(const i32x4*)(Ks + (koff[bb][kk] ^ 16));
        s[bb] = mma_fp8(__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7), qf[kk], s[bb]);
      }
    }
    __builtin_amdgcn_s_setprio(0);
    // ---- mask: element i of block bb is key j0 + 32 h + 16 bb + i
    const bool edge = (j0 + BN > kv_len) || (CAUSAL && j0 + BN - 1 > qw);
    if (edge) {
#pragma unroll
      for (int bb = 0; bb < 2; ++bb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = j0 + 32 * h + 16 * bb + i;
          const bool dead = (key >= kv_len) || (CAUSAL && key > qi);
          s[bb][i] = dead ? NEG_INF : s[bb][i];
        }
    }
    // ---- P' = 2^(4 + f) exp2(c s - m) -> E4M3 against the current max (lv
    // holds f); row sum over the fp32 values
    float rs;
    i32x8 pk;
    auto probs = [&]() {
      const float off = POFF + lv - msub;
      rs = 0.f;
#pragma unroll
      for (int w = 0; w < 8; ++w) {
        float e[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int k = 4 * w + j;           // 0..31: block k / 16, element k % 16
          e[j] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[k >> 4][k & 15], c, off));
          rs += e[j];
        }
        int v = __builtin_amdgcn_cvt_pk_fp8_f32(e[0], e[1], 0, false);
        pk[w] = __builtin_amdgcn_cvt_pk_fp8_f32(e[2], e[3], v, true);
      }
    };
    probs();
    // ---- the lane's sum bounds each of its probabilities: unless some
    // lane's exceeds PMAX (or is not finite), or the row has no max yet, the
    // tile is done.  Otherwise (rare) the max moves to the tile's row max, O
    // and l are rescaled and the probabilities recomputed.
    if (__builtin_amdgcn_ballot_w64(!(rs <= PMAX) || m_run == NEG_INF) != 0) {
      asm volatile("" ::: "memory");   // keep the rare path a branch
      float mx = NEG_INF;
#pragma unroll
      for (int bb = 0; bb < 2; ++bb)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[bb][i]);
      mx = fmaxf(mx, wave_half_swap(mx));
      // the new max sits 4 (log2 units) above the tile's row max: a max that
      // creeps up over the next tiles then stays within the bound instead of
      // taking this branch again (P' at the row max is 2^0 instead of 2^4;
      // the reference point cancels in O and l either way)
      const float m_new = fmaxf(m_run, mx * c + 4.f);
      const float alpha = (m_new == m_run) ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
#pragma unroll
      for (int db = 0; db < 4; ++db) o[db] *= alpha;
      l_run *= alpha;
      m_run = m_new;
      msub = (m_run == NEG_INF) ? 0.f : m_run;
      probs();
    }
    l_run += rs * __builtin_amdgcn_exp2f(-POFF - lv);
    // ---- O^T += V^T P'^T
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const i32x4 lo = *(const i32x4*)(Vs + voff[db]);
      const i32x4 hi = *(const i32x4*)(Vs + (voff[db] ^ 16));
      o[db] = mma_fp8_sa(__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7), pk, o[db], vscale);
    }
    __builtin_amdgcn_s_setprio(0);
  };
  typedef std::integral_constant<int, 0> S0;
  typedef std::integral_constant<int, 1> S1;
  issue(0, 0);
  int t = 0;
  for (; t + 2 <= ntile; t += 2) {
    step(t, S0{});
    step(t + 1, S1{});
  }
  if (t < ntile) step(t, S0{});

  // ---- epilogue: O = O_acc sv_max / (2^4 l) (bf16), LSE = ln2 (m + log2 l)
  const float l_tot = l_run + wave_half_swap(l_run);
  if (qi < q_len) {
    const float scl = l_tot > 0.f ? sv_max / (__builtin_amdgcn_exp2f(POFF) * l_tot) : 0.f;
    __bf16* orow = (__bf16*)p.o + ((long long)b * p.Sq + qi) * qs + hq * D;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        typedef __bf16 bf4 __attribute__((ext_vector_type(4)));
        bf4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = (__bf16)(o[db][4 * g + e] * scl);
        *(bf4*)(orow + 32 * db + 8 * g + 4 * h) = w;
      }
    if (p.lse != nullptr && h == 0) {
      const float lse = l_tot > 0.f ? (m_run + log2f(l_tot)) * 0.69314718055994530942f : NEG_INF;
      p.lse[((long long)b * p.Hq + hq) * p.Sq + qi] = lse;
    }
  }
}

hipError_t launch_fwd_fp8(const Fp8FwdParams& p, int causal, hipStream_t s) {
  if (causal) hipLaunchKernelGGL(fwd_fp8_kernel<true>, dim3(p.grid), dim3(256), 0, s, p);
  else hipLaunchKernelGGL(fwd_fp8_kernel<false>, dim3(p.grid), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace attn
