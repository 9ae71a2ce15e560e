/*
 * attn.h -- C ABI of the MI355X (gfx950) fused exact-attention forward.
 *
 * The operation is exact attention, O = softmax(scale * Q K^T + mask) V, as
 * written at the top of "FlashAttention-3 Deep Dive" (mojostudio.in,
 * introduction), computed tile by tile with a streaming softmax so that the
 * Sq x Sk score matrix never reaches device memory ("flash-attention-3",
 * ai.thesatyajit.com, opening section: tile the computation and keep a running
 * softmax).  Alongside O the library writes the per-row log-sum-exp
 * LSE_i = log sum_j exp(scale * q_i . k_j + mask_ij) (natural log, scale
 * included), the softmax statistic listed in the Hopper tag page
 * (l1-ca0.github.io, contents entry 4.6).
 *
 * Conventions shared by every entry point
 *   - All tensor pointers are DEVICE pointers owned by the caller; the
 *     library never frees or retains them.  They must stay valid until the
 *     stream has executed the enqueued work.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Every call is asynchronous: it validates its arguments on the host,
 *     enqueues kernels on `stream` and returns; results are ready after the
 *     stream is synchronised.  No call blocks or copies host<->device
 *     (attn_release, which frees the workspaces, is the one call that waits
 *     for the device).
 *   - Library-owned workspaces (the fp8 operands of attn_fwd's fp8 types,
 *     the split-KV partials, the backward's row statistics; one buffer per
 *     use and device) grow stream-ordered: a call that needs a larger buffer
 *     frees the old one with hipFreeAsync on its own stream (after the work
 *     queued there) and allocates the new one with hipMallocAsync.  So calls
 *     that use the same workspace from different streams of one device, or
 *     from several host threads, must not overlap: the caller orders them
 *     (one stream, or events between the streams).
 *   - Return value 0 (ATTN_OK) on success, a negative ATTN_ERR_* code on
 *     failure.  Validation happens before anything is enqueued, so a call
 *     that returns an error has written nothing.  Nothing throws or aborts
 *     across the ABI; attn_strerror() turns a code into text (for
 *     ATTN_ERR_HIP it includes the HIP runtime's message of the last failure).
 *   - Layouts are contiguous, innermost dimension last, tokens-major (the
 *     (batch, seqlen, heads, headdim) layout of the benchmark on the
 *     "Lecture 9 -- Hopper / FlashAttention-3 / FlashAttention-4" page,
 *     "Benchmark task").
 *   - Grouped-query attention: query head h reads key/value head
 *     h / (Hq / Hkv) (consecutive groups; Hq must be a multiple of Hkv).
 *   - Causal masking hides key j from query i when j > i (indices local to
 *     the sequence; top-left aligned when Sq != Sk).
 *   - A query row that sees no key gets O = 0 and LSE = -inf.
 */
#ifndef ATTN_H_
#define ATTN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types.  ATTN_BF16 / ATTN_FP16: q, k, v and o all hold that type.
 * ATTN_FP8_E4M3 / ATTN_FP8_E4M3_HADAMARD: q, k, v hold fp32 values; the
 * library quantises them to OCP E4M3 with one fp32 scale per 128 rows of one
 * (batch, head) -- the per-block scaling of "FlashAttention-3 Deep Dive",
 * section 4 -- optionally after the signed 128-point Hadamard rotation of Q
 * and K (same section, incoherence processing), runs both GEMMs in fp8 with
 * fp32 accumulation, and writes o as bf16. */
enum attn_dtype {
  ATTN_BF16 = 0,
  ATTN_FP16 = 1,
  ATTN_FP8_E4M3 = 2,
  ATTN_FP8_E4M3_HADAMARD = 3
};

enum attn_status {
  ATTN_OK = 0,
  ATTN_ERR_NULL = -1,     /* a required pointer is NULL                        */
  ATTN_ERR_SHAPE = -2,    /* non-positive B/Hq/Hkv/Sq/Sk, varlen with Sq != Sk */
  ATTN_ERR_HEADDIM = -3,  /* d not supported (64 or 128; 128 for fp8)          */
  ATTN_ERR_GQA = -4,      /* Hq not a multiple of Hkv                          */
  ATTN_ERR_DTYPE = -5,    /* unknown dtype, or dtype not valid for the call    */
  ATTN_ERR_ARG = -6,      /* scale not finite or not > 0; unsupported combo    */
  ATTN_ERR_NOMEM = -7,    /* workspace allocation failed                       */
  ATTN_ERR_HIP = -8,      /* a HIP runtime call or kernel launch failed        */
  ATTN_ERR_SIZE = -9,     /* a size or index would overflow 32-bit addressing  */
  ATTN_ERR_SCRATCH = -10  /* attn_fwd_splitkv_noalloc: partials exceed its scratch */
};

/*
 * attn_fwd -- fused attention forward.
 *
 * Dense (cu_seqlens == NULL):
 *   q [B, Sq, Hq, d], k and v [B, Sk, Hkv, d], o [B, Sq, Hq, d],
 *   lse [B, Hq, Sq] (fp32).
 * Varlen (cu_seqlens != NULL): B is the number of sequences and
 *   Sq == Sk == T, the total number of packed tokens.  cu_seqlens is a DEVICE
 *   array of B + 1 int32 offsets with cu[0] = 0, cu[B] = T, non-decreasing;
 *   sequence s owns tokens [cu[s], cu[s+1]) of q, k and v, and attends only
 *   within itself ("FlashAttention-3 Deep Dive", FAQ on ragged batches).
 *   q [T, Hq, d], k and v [T, Hkv, d], o [T, Hq, d], lse [Hq, T].
 *   The offsets are read on the device and are not validated (reading them on
 *   the host would need a synchronisation).  Varlen needs dtype bf16/fp16.
 * scale: multiplies Q K^T before the softmax; must be finite and > 0
 *   (1/sqrt(d) gives the formula's 1/sqrt(d_k)).
 * causal: non-zero hides key j from query i when j > i.
 * bf16/fp16 dense calls with GQA and few query positions use PackGQA (see
 *   attn_fwd_splitkv); the result does not depend on that choice.  When the
 *   plain launch would hold fewer than 128 workgroups and Sk >= 4096 (few
 *   query blocks over a long key cache, e.g. decoding), the call runs attn_fwd_splitkv's
 *   plan (num_splits = 0) and, if that plan cuts the keys, its split-KV
 *   partials and combine: O and LSE agree with the plain path to rounding,
 *   and the call then uses the split-KV workspace (shared with
 *   attn_fwd_splitkv; such calls on different streams of one device must
 *   not overlap).
 * dtype: an attn_dtype.  For the fp8 types q, k, v are fp32 and o is bf16;
 *   the quantised copies live in a library-owned, lazily grown device
 *   workspace (released by attn_release; fp8 calls on different streams of
 *   one device share it and must not overlap); the Hadamard variant uses the
 *   library's default sign vector (attn_default_signs), compiled into the
 *   library's device code.  fp8 needs d == 128
 *   and Sk a multiple of 16, and no cu_seqlens.
 * lse may be NULL when the caller does not want it.
 */
int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
             int B, int Hq, int Hkv, int Sq, int Sk, int d, float scale, int causal,
             const int32_t* cu_seqlens, int dtype, void* stream);

/*
 * attn_fp8_prepass -- per-block fp8 quantisation ("FlashAttention-3 Deep
 * Dive", section 4: per-block scaling and the Hadamard rotation).
 *
 * x [B, S, H, d] fp32 (device).  For every (b, h) and every block of 128
 * consecutive rows (the last block may be shorter):
 *   optional rotation  x <- (x * signs) H_d / sqrt(d)   (signs: d device
 *                      floats of +-1; NULL = no rotation), in fp32;
 *   s = amax / 448 over the block's rows and all d channels (s = 1 when the
 *   block is all zero); code = E4M3(clip(x / s, -448, 448)), round to
 *   nearest even.
 * Outputs (device, caller-owned):
 *   x8: uint8 codes, [B, S, H, d] when transpose_out == 0, or
 *       [B, H, d, S] (token index innermost) when transpose_out != 0;
 *   descale: fp32 [B, H, ceil(S / 128)], the scales s (dequantised value =
 *       decode(code) * s).
 * d must be 128 (the rotation is the 128-point transform).
 */
int attn_fp8_prepass(const float* x, uint8_t* x8, float* descale, int B, int S, int H, int d,
                     int transpose_out, const float* signs, void* stream);

/*
 * attn_fp8_prepass_qkv -- attn_fp8_prepass of Q, K and V in one launch, in
 * the layouts attn_fwd_fp8 takes: q [B, Sq, Hq, d] -> q8 [B, Sq, Hq, d] and
 * q_descale [B, Hq, ceil(Sq/128)]; k [B, Sk, Hkv, d] -> k8 [B, Sk, Hkv, d]
 * and k_descale [B, Hkv, ceil(Sk/128)]; v [B, Sk, Hkv, d] -> v8t
 * [B, Hkv, d, Sk] (token index innermost) and v_descale [B, Hkv,
 * ceil(Sk/128)].  signs (d device floats, or NULL) rotate Q and K as in
 * attn_fp8_prepass; V is never rotated ("FlashAttention-3 Deep Dive",
 * section 4: the rotation of Q and K leaves Q K^T unchanged).  The codes and
 * scales are those the three single calls write.  All pointers device and
 * caller-owned; d must be 128.  Returns ATTN_OK, ATTN_ERR_NULL,
 * ATTN_ERR_SHAPE, ATTN_ERR_HEADDIM, ATTN_ERR_SIZE or ATTN_ERR_HIP.
 */
int attn_fp8_prepass_qkv(const float* q, const float* k, const float* v, uint8_t* q8, uint8_t* k8,
                         uint8_t* v8t, float* q_descale, float* k_descale, float* v_descale, int B,
                         int Hq, int Hkv, int Sq, int Sk, int d, const float* signs, void* stream);

/*
 * attn_fwd_fp8 -- fused attention forward on pre-quantised E4M3 operands,
 * fp32 accumulation in both GEMMs, bf16 output.
 *   q8 [B, Sq, Hq, d] codes, k8 [B, Sk, Hkv, d] codes,
 *   v8t [B, Hkv, d, Sk] codes (token index innermost: the K-major operand
 *       the second GEMM wants, written by attn_fp8_prepass with
 *       transpose_out = 1),
 *   q_descale [B, Hq, ceil(Sq/128)], k_descale and v_descale
 *       [B, Hkv, ceil(Sk/128)] fp32 block scales,
 *   o [B, Sq, Hq, d] bf16, lse [B, Hq, Sq] fp32 (may be NULL).
 * d must be 128 and Sk a multiple of 16 (16-byte aligned rows of v8t);
 * dense only (no cu_seqlens).
 */
int attn_fwd_fp8(const uint8_t* q8, const uint8_t* k8, const uint8_t* v8t,
                 const float* q_descale, const float* k_descale, const float* v_descale,
                 void* o, float* lse, int B, int Hq, int Hkv, int Sq, int Sk, int d,
                 float scale, int causal, void* stream);

/*
 * attn_fwd_ext -- attn_fwd with two options of the 16-bit forward
 * ("FlashAttention-3 Deep Dive": the API surface lists attention
 * softcapping; the FP8 layout discussion the V_colmajor input).
 *
 * softcap: 0 = off; > 0 replaces every score s = scale q.k by
 *   softcap * tanh(s / softcap) before the causal mask and the softmax (the
 *   LSE is that of the capped scores).  Must be finite and >= 0.
 * v_colmajor: 0 = v as in attn_fwd; non-zero = v given column-major,
 *   [B, Hkv, d, Sk] (key index innermost), which the kernel reads as the
 *   second GEMM's operand without transposing.  Needs Sk % 8 == 0 (16-byte
 *   aligned rows).
 * With both options off the call is attn_fwd.  With either on: dense
 * (cu_seqlens NULL) and dtype ATTN_BF16 / ATTN_FP16 only (else
 * ATTN_ERR_ARG).  Column-major V alone at d = 128 runs the one-wave-per-SIMD
 * kernel of attn_fwd (its V tile then comes straight from the column-major
 * layout); softcap, and d = 64, run 128-row tiles of the 4-wave kernel.
 * Other arguments,
 * layouts and errors as attn_fwd.
 */
int attn_fwd_ext(const void* q, const void* k, const void* v, void* o, float* lse,
                 int B, int Hq, int Hkv, int Sq, int Sk, int d, float scale, int causal,
                 const int32_t* cu_seqlens, int dtype, float softcap, int v_colmajor,
                 void* stream);

/*
 * attn_fwd_splitkv -- the dense bf16/fp16 forward of attn_fwd with the key
 * axis cut into ranges (split-KV, "flash-decoding": the Hopper tag page,
 * l1-ca0.github.io, contents 10 and 10.2.1).  Each (query tile, key range)
 * pair is one workgroup that writes the normalised partial output O_p of its
 * range and its log-sum-exp LSE_p in fp32; attn_combine then merges the
 * ranges (block-combine of the streaming softmax, same page, contents 3.2.1).
 * The result equals attn_fwd's up to rounding.  It pays off when the tiles
 * of the plain forward are too few to fill the device: few query rows
 * (decoding), few heads, long keys.
 *
 * Arguments, layouts and causal semantics as for attn_fwd (dense only, no
 * cu_seqlens); dtype ATTN_BF16 or ATTN_FP16.
 * num_splits: the number of key ranges wanted (0 = chosen by the library,
 *   see attn_split_plan; at most 256).  The plan rounds range lengths up to
 *   multiples of 64 keys, so fewer ranges may result; with one range no
 *   partials are written and the kernels of attn_fwd run.
 * pack_gqa: PackGQA ("FlashAttention-3 Deep Dive" API surface, the
 *   pack_gqa option; Hopper tag page, contents 11): the query rows of all
 *   Hq / Hkv heads that share a KV head go into one 128-row tile, row
 *   position * (Hq / Hkv) + head-in-group, so that few query positions still
 *   fill a tile and each K/V tile is read once per group.  -1 = automatic
 *   (packed when that gives fewer tiles, e.g. decoding), 0 = off, 1 = on
 *   (needs Hq / Hkv to divide 128, else ATTN_ERR_ARG; a no-op without GQA).
 *   attn_fwd makes the automatic choice.
 * The partials live in a library-owned, lazily grown device workspace
 * (splits * B * Sq * Hq * (d + 1) floats; released by attn_release).  Calls
 * on different streams of one device share it and must not overlap.
 * lse may be NULL.
 */
int attn_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse,
                     int B, int Hq, int Hkv, int Sq, int Sk, int d, float scale, int causal,
                     int num_splits, int pack_gqa, int dtype, void* stream);

/* Bytes of the fixed device scratch of attn_fwd_splitkv_noalloc (per GPU). */
#define ATTN_NOALLOC_SCRATCH_BYTES (16u << 20)

/*
 * attn_fwd_splitkv_noalloc -- attn_fwd_splitkv for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving
 * loops (decoding), harnesses that forbid hipMalloc.  Same arguments, plan
 * (attn_split_plan) and result as attn_fwd_splitkv; the caller still passes
 * q, k, v, o and lse.  The split-KV partials go to a fixed device array of
 * ATTN_NOALLOC_SCRATCH_BYTES (16 MiB) compiled into the library, one per
 * GPU, held until the process ends, instead of the lazily grown workspace:
 * the call never allocates or frees memory.  The partials of a plan take
 * splits * B * Sq * Hq * (d + 1) floats (two parts, each rounded up to 256
 * bytes); a plan that needs more returns ATTN_ERR_SCRATCH and enqueues
 * nothing (e.g. the decode shape B=4 Hq=32 Sq=1 d=128 with 8 ranges takes
 * 129 KiB).  With one range no partials are written.  Every call on a GPU
 * shares that GPU's array and leaves its partials there; each call writes
 * every partial it reads, so nothing needs clearing, but calls that overlap
 * on one GPU (different streams, threads) race on it and must be ordered by
 * the caller.  The array's device address is looked up once per device on
 * the first call there (hipGetSymbolAddress).
 */
int attn_fwd_splitkv_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                             int B, int Hq, int Hkv, int Sq, int Sk, int d, float scale, int causal,
                             int num_splits, int pack_gqa, int dtype, void* stream);

/*
 * attn_split_plan -- the plan attn_fwd_splitkv follows for these arguments:
 * writes the number of key ranges, the keys per range (a multiple of 64; the
 * last range holds the rest, no range is empty) and whether the tiles are
 * packed (PackGQA, 0 or 1).  num_splits == 0 weighs the rounds of
 * workgroups the device runs (256 CUs; one 128-row workgroup per CU with
 * d = 128, two with d = 64) against the keys each workgroup covers plus a
 * fixed cost per workgroup worth 128 keys, and takes the cheapest count
 * (ranges of >= 256 keys, at most 64).  Returns ATTN_OK, ATTN_ERR_NULL,
 * ATTN_ERR_SHAPE, ATTN_ERR_GQA, ATTN_ERR_HEADDIM, ATTN_ERR_ARG (num_splits
 * < 0 or > 256; pack_gqa not in {-1, 0, 1}, or 1 with a group size that
 * does not divide 128) or ATTN_ERR_SIZE.
 */
int attn_split_plan(int B, int Hq, int Hkv, int Sq, int Sk, int d, int num_splits, int pack_gqa,
                    int* splits_out, int* split_keys_out, int* pack_out);

/*
 * attn_combine -- merge of split-KV partials (the Hopper tag page,
 * contents 10.2.1, with the block-combine of contents 3.2.1):
 *   m = max_p LSE_p,  w_p = exp(LSE_p - m),
 *   LSE = m + log sum_p w_p,  O = sum_p w_p O_p / sum_p w_p.
 * A partial with LSE_p = -inf (its range held no visible key) contributes
 * nothing; a row whose partials are all -inf gets O = 0 and LSE = -inf.
 *   o_part   [splits, B, Sq, Hq, d] fp32, each O_p already normalised,
 *   lse_part [splits, B, Hq, Sq] fp32 (natural log, scale included),
 *   o        [B, Sq, Hq, d] in dtype (ATTN_BF16 / ATTN_FP16), rounded to
 *            nearest even,
 *   lse      [B, Hq, Sq] fp32, may be NULL.
 * All device pointers, caller-owned.  d must be 64 or 128; 1 <= splits <= 256
 * (more gives ATTN_ERR_ARG).  The O_p of a partial whose LSE_p is -inf is
 * never used and may hold anything.
 */
int attn_combine(const float* o_part, const float* lse_part, void* o, float* lse, int splits,
                 int B, int Hq, int Sq, int d, int dtype, void* stream);

/*
 * attn_bwd -- attention backward (bf16 / fp16, dense or varlen, d = 64 or 128).
 *
 * Gradients of O = softmax(scale Q K^T + mask) V (and of LSE when dlse is
 * given), by the chain rule listed in the Hopper tag page (l1-ca0.github.io,
 * contents 7.1): P is recomputed from the forward's LSE,
 *   dV = P^T dO,  dP = dO V^T,  delta_i = dO_i . O_i - dlse_i,
 *   dS = P (dP - delta),  dQ = scale dS K,  dK = scale dS^T Q,
 * with dK, dV of a KV head summed over the Hq / Hkv query heads that read it.
 *   q, o, dout [B, Sq, Hq, d] and k, v [B, Sk, Hkv, d] in dtype
 *     (o and lse as written by attn_fwd for these q, k, v, scale, causal);
 *   lse [B, Hq, Sq] fp32; dlse [B, Hq, Sq] fp32 or NULL (no LSE gradient);
 *   dq [B, Sq, Hq, d], dk and dv [B, Sk, Hkv, d] in dtype, written whole
 *     (keys no query sees get zero gradients).
 * Varlen (cu_seqlens != NULL): as for attn_fwd -- B sequences packed along
 *   the token axis, Sq == Sk == T; q, o, dout, dq [T, Hq, d], k, v, dk, dv
 *   [T, Hkv, d], lse and dlse [Hq, T]; sequences do not see each other.
 * Deterministic: no atomics; dQ has its own kernel.  A per-row fp32
 * statistics array (2 * B * Hq * ceil(Sq / 32) * 32 floats; varlen 2 * Hq * T)
 * lives in a library-owned,
 * lazily grown workspace (released by attn_release); calls on different
 * streams of one device share it and must not overlap.  Same validation and
 * error codes as attn_fwd (dtype ATTN_BF16 or ATTN_FP16).
 */
int attn_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
             const void* dout, const float* dlse, void* dq, void* dk, void* dv,
             int B, int Hq, int Hkv, int Sq, int Sk, int d, float scale, int causal,
             const int32_t* cu_seqlens, int dtype, void* stream);

/* The library's default Hadamard sign vector used by ATTN_FP8_E4M3_HADAMARD:
 * writes n (<= 128) host floats of +-1, sign i being the top bit of the
 * splitmix64 output for counter (55 << 32) + i + 1.  Returns ATTN_OK, or
 * ATTN_ERR_NULL / ATTN_ERR_SHAPE. */
int attn_default_signs(float* signs_host, int n);

/* Tile order of the forward kernel's scheduler, evaluated on the host (for
 * inspection and tests): for workgroup index p of a dense launch, writes the
 * (batch, query head, query block) it processes.  block_m is the number of
 * query rows per tile.  (The head-packed layout of dense d = 128 inputs with a
 * group Hq / Hkv that is a multiple of 4 is this order for Hq / 4 "heads" and
 * block_m = 64: entry h stands for query heads 4 h .. 4 h + 3.)  Returns
 * ATTN_OK or ATTN_ERR_SHAPE / ATTN_ERR_NULL. */
int attn_tile_of(int p, int B, int Hq, int Hkv, int Sq, int block_m, int causal,
                 int* b_out, int* h_out, int* m_out);

/* Number of workgroups a dense launch uses, and query rows per tile, for
 * the layout of one query head per tile.  (Dense d = 128 inputs whose group
 * Hq / Hkv is a multiple of 4 run tiles of 64 rows of four heads instead,
 * B * (Hq / 4) * ceil(Sq / 64) of them, on at most one workgroup per
 * compute unit: with more tiles than compute units each workgroup runs
 * several in turn.  This call, having no Hkv, does not report that layout.) */
int attn_grid_size(int B, int Hq, int Sq, int d, int dtype, int* grid_out, int* block_m_out);

/* Human-readable text for a status code. */
const char* attn_strerror(int code);

/* Frees the library's workspaces (fp8 operands, split-KV partials, backward
 * statistics) on every device that has them.  Waits for each such device to
 * finish its queued work first (hipDeviceSynchronize). */
void attn_release(void);

/* Measurement aid: the shader clock of one compute unit while other work
 * runs.  Enqueues one wave that spins for wall_ticks ticks of the device's
 * constant-rate wall clock (hipDeviceAttributeWallClockRate, written to
 * *wall_khz on the host) and writes to out (2 device uint64) the shader-clock
 * and wall-clock deltas it saw: clock = out[0] / out[1] * wall_khz kHz.
 * Run it on a second stream beside the kernel being measured (the wave
 * takes one SIMD of one compute unit while it spins).  Returns ATTN_OK,
 * ATTN_ERR_NULL, ATTN_ERR_ARG or ATTN_ERR_HIP. */
int attn_clock_probe(unsigned long long* out, int wall_ticks, int* wall_khz, void* stream);

/* Failure injection for tests of the error paths (the failures a host-only
 * test cannot otherwise produce).  Arms a one-shot failure for the calling
 * thread: after attn_test_fail_next(ATTN_ERR_NOMEM) the next workspace
 * allocation fails as if the device were out of memory (the call returns
 * ATTN_ERR_NOMEM); after attn_test_fail_next(ATTN_ERR_HIP) the next kernel
 * launch reports a launch failure instead of running (ATTN_ERR_HIP, with the
 * text in attn_strerror).  Either way nothing is enqueued.  0 disarms.
 * Returns ATTN_OK, or ATTN_ERR_ARG for any other code. */
int attn_test_fail_next(int code);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_H_ */
