/*
 * sage.h -- C ABI of the MI355X (gfx950) SageAttention-style quantized attention forward.
 *
 * The operation: O = softmax(sm_scale * Q K^T [+ causal mask]) V, computed as
 *   1. smoothing: subtract from K its per-channel mean over all tokens of each
 *      (batch, kv-head) -- softmax is unchanged because q.mean is constant along a
 *      row (SageAttention project README, "Current Features": INT8 quantization
 *      and smoothing for QK^T);
 *   2. INT8 quantisation of Q and of smoothed K, one fp32 scale per 64-token block
 *      (same section; "varying granularities");
 *   3. INT8 x INT8 -> INT32 scores on the matrix cores, dequantised with the two
 *      block scales, online base-2 softmax over 64-key blocks;
 *   4. P.V with P and V in FP16 or FP8-e4m3 (README "Current Features": FP8
 *      quantization for PV; "Available APIs": the qk_int8_pv_fp16 / pv_fp8 kernels
 *      and pv_accum_dtype), accumulated in fp32 or in two levels (README: two-level
 *      accumulation strategy for PV);
 * with q/k/v in FP16/BF16, tensor layout HND (batch, heads, seq, dim) or NHD
 * (batch, seq, heads, dim), is_causal, sm_scale (SDPA semantics, default
 * 1/sqrt(head_dim) -- qwbw.cn one-line integration article), grouped-query
 * attention with num_qo_heads a multiple of num_kv_heads (same article), and head
 * dims other than 64/128/256 zero-padded (same article, pad_qkv paragraph).
 *
 * Conventions for every call:
 *  - All tensor pointers are DEVICE pointers owned by the caller.  The library
 *    allocates nothing, keeps no state between calls other than a per-device
 *    architecture check, never synchronises the stream, and is re-entrant.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Work is only
 *    enqueued; asynchronous faults surface at the caller's next synchronisation.
 *  - Arguments are validated before any HIP call: on error nothing is written and
 *    no kernel is launched; sage_last_error_detail() explains the failure.
 *  - Shapes: B batch, H_qo query heads, H_kv kv heads, Nq / Nkv sequence lengths,
 *    D true head dim (1..256).  Dp = 64, 128 or 256: the smallest of them >= D,
 *    NB(N) = ceil(N / 64), N_pad(N) = 64 * NB(N).  Query head h reads kv head
 *    h / (H_qo / H_kv).
 *  - Every padding element of an output buffer (tokens >= N, channels >= D) is
 *    written with zero, so outputs are deterministic bytes.
 *  - Layouts of the quantised intermediates (all row-major, innermost last):
 *      q_i8     int8   [B][H_qo][N_pad(Nq)][Dp]
 *      q_scale  float  [B][H_qo][NB(Nq)]
 *      k_i8     int8   [B][H_kv][N_pad(Nkv)][Dp]      (smoothed K)
 *      k_scale  float  [B][H_kv][NB(Nkv)]
 *      k_mean   float  [B][H_kv][D]
 *      v_hat    fp16 or e4m3 bytes [B][H_kv][NB(Nkv)][Dp][64]
 *               (each 64-key block stored channel-major: element (c, t) of block
 *               j holds token 64*j + t of channel c)
 *      v_scale  float  [B][H_kv][Dp]                   (FP8 mode only)
 */
#ifndef SAGE_H_
#define SAGE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SAGE_ABI_VERSION 6

typedef enum sage_status {
    SAGE_OK = 0,
    SAGE_ERR_INVALID_ARG = 1, /* null pointer, non-positive size, bad enum, H_qo % H_kv != 0, bad sm_scale */
    SAGE_ERR_UNSUPPORTED = 2, /* D > 256, SAGE_ACC_FP16, size overflow */
    SAGE_ERR_WORKSPACE = 3,   /* workspace pointer NULL or smaller than required */
    SAGE_ERR_DEVICE = 4,      /* no HIP device, or the current device is not gfx950 */
    SAGE_ERR_HIP = 5          /* a kernel launch failed (hipGetLastError) */
} sage_status;

typedef enum sage_dtype { SAGE_FP16 = 0, SAGE_BF16 = 1 } sage_dtype;
typedef enum sage_layout { SAGE_HND = 0, SAGE_NHD = 1 } sage_layout;
typedef enum sage_pv { SAGE_PV_FP16 = 0, SAGE_PV_FP8 = 1 } sage_pv;
/* PV accumulation (README "Available APIs", pv_accum_dtype; "Current Features":
 * two-level accumulation for FP8 P.V):
 *   SAGE_ACC_FP32        fp32 single level: the matrix instruction adds each tile's
 *                        products to the fp32 output accumulator;
 *   SAGE_ACC_FP16_FP32   the pages' "fp32+fp16" two-level mode, an ALIAS of SAGE_ACC_FP32
 *                        on gfx950: the two-level strategy keeps a reduced-precision inner
 *                        accumulator of the tensor cores from losing bits by adding short
 *                        runs into fp32; the gfx950 FP8/FP16 matrix instructions accumulate
 *                        straight into an fp32 operand, so single-level fp32 already gives
 *                        every level fp32 precision;
 *   SAGE_ACC_FP16        fp16 single level: not offered (SAGE_ERR_UNSUPPORTED; the gfx950
 *                        FP16/FP8 matrix instructions accumulate in fp32);
 *   SAGE_ACC_FP16_FP32_SPLIT  the literal two-level form: each 64-key tile's products in fresh
 *                        fp32 accumulators, folded into the output accumulator with vector
 *                        adds (64 more vector instructions per tile; block granularity only).
 *                        Its fp32 accumulator rounds differently from SAGE_ACC_FP32's, so
 *                        outputs may differ from it by one output ulp.
 */
typedef enum sage_accum {
    SAGE_ACC_FP32 = 0,
    SAGE_ACC_FP16_FP32 = 1,
    SAGE_ACC_FP16 = 2,
    SAGE_ACC_FP16_FP32_SPLIT = 3
} sage_accum;
/* Q/K quantisation granularity (README "Current Features": varying granularities).
 * SAGE_GRAN_BLOCK: one scale per 64 tokens for Q and for K (the layouts above).
 * SAGE_GRAN_THREAD: the finer "per-thread" quantisation of README "Project Updates"
 * (v2.0.1), read for gfx950 as the groups each lane owns in the score MFMA: one Q
 * scale per token, one K scale per 32 keys.  Scale layouts then:
 *   q_scale  float [B][H_qo][N_pad(Nq)]        (per token, padding rows 0)
 *   k_scale  float [B][H_kv][NB(Nkv)][2]       (keys 64j .. 64j+31, 64j+32 .. 64j+63)
 * and for packed batches q_scale [H_qo][rows(total_q)], k_scale [H_kv][slots(total_kv)][2].
 * The codes are still per element (x * inv rounded), every other step unchanged. */
typedef enum sage_qk_gran { SAGE_GRAN_BLOCK = 0, SAGE_GRAN_THREAD = 1 } sage_qk_gran;

int sage_abi_version(void);
const char* sage_status_string(sage_status s);
/* Thread-local text describing the last failure of a call made on this thread. */
const char* sage_last_error_detail(void);

/* Dp for a head dim (64, 128 or 256), 0 when D is outside 1..256. */
int sage_padded_dim(int D);
/* NB(N) = ceil(N / 64). */
int sage_num_blocks(int N);

/* Workspace of sage_quant_qk: fp64 per-block channel partial sums of K,
 * B * H_kv * NB(Nkv) * D * 8 bytes.  0 for invalid sizes. */
size_t sage_quant_qk_workspace_bytes(int B, int H_kv, int Nkv, int D);

/*
 * Smoothing + INT8 quantisation of Q and K (steps 1-2 above).
 *   q: [B,H_qo,Nq,D] (HND) or [B,Nq,H_qo,D] (NHD), k likewise with H_kv, Nkv;
 *      both fp16 or bf16 (`dtype`), contiguous.
 *   K mean, per (b, kv head, channel c): fp64 sum over each 64-token block in
 *   ascending token order, fp64 sum of those block sums in ascending block order,
 *   fp64 division by Nkv, one rounding to fp32 -> k_mean.
 *   Per 64-token block of Q, and of y = fp32(K - k_mean): amax = max|y| over the
 *   block's real tokens and channels, scale = fp32(amax / 127), inv = fp32(127 /
 *   amax), code = clamp(round_half_even(fp32(y * inv)), -127, 127); an all-zero
 *   block gets scale 0 and codes 0.
 *   Outputs: q_i8, q_scale, k_i8, k_scale, k_mean (layouts above).
 *   workspace: device buffer of at least sage_quant_qk_workspace_bytes(...) bytes,
 *   contents on entry ignored and on exit unspecified.
 */
sage_status sage_quant_qk(const void* q, const void* k, sage_dtype dtype, sage_layout layout, int B, int H_qo,
                          int H_kv, int Nq, int Nkv, int D, int8_t* q_i8, float* q_scale, int8_t* k_i8,
                          float* k_scale, float* k_mean, void* workspace, size_t workspace_bytes, void* stream);

/* Workspace of sage_quant_v: B * H_kv * Dp * 4 bytes in FP8 mode (per-channel amax), 0 in FP16 mode. */
size_t sage_quant_v_workspace_bytes(int B, int H_kv, int D, sage_pv pv);

/*
 * The P.V operand (step 4 above).
 *   v: [B,H_kv,Nkv,D] (HND) or [B,Nkv,H_kv,D] (NHD), fp16 or bf16, contiguous.
 *   SAGE_PV_FP16: v_hat = fp16(v) (round half even, saturating at +-65504);
 *                 v_scale and workspace are ignored (may be NULL).
 *   SAGE_PV_FP8:  per (b, kv head, channel c) over all Nkv tokens: amax = max|v|,
 *                 v_scale = fp32(amax / 448), inv = fp32(448 / amax),
 *                 v_hat = e4m3fn(fp32(v * inv)) (round half even, saturating at
 *                 +-448); an all-zero channel gets scale 0 and codes 0.
 *   v_hat layout above (2 bytes per element in FP16 mode, 1 in FP8 mode).
 */
sage_status sage_quant_v(const void* v, sage_dtype dtype, sage_layout layout, int B, int H_kv, int Nkv, int D,
                         sage_pv pv, void* v_hat, float* v_scale, void* workspace, size_t workspace_bytes,
                         void* stream);

/* Workspace of sage_quant_qkv: the fp64 K block sums of sage_quant_qk
 * (B * H_kv * NB(Nkv) * D * 8 bytes), plus in FP8 mode per-block V channel maxima
 * (B * H_kv * NB(Nkv) * Dp * 4) and per-channel V maxima (B * H_kv * Dp * 4).
 * 0 for invalid sizes or pv. */
size_t sage_quant_qkv_workspace_bytes(int B, int H_kv, int Nkv, int D, sage_pv pv);

/*
 * sage_quant_qk and sage_quant_v in one call: the same outputs, bit for bit, in four
 * kernel launches instead of six or seven (Q quantisation and the K/V statistics
 * stream in one grid; then the K means and V maxima; then K and V quantisation).  At
 * head dims up to 128 it takes three: FP16 P.V casts V in the first grid, FP8 P.V writes
 * the K and V codes in one grid.  Sequences of at most 32 blocks need one launch fewer.
 *   q, k, v, dtype, layout, shapes: as sage_quant_qk and sage_quant_v.
 *   Outputs: q_i8, q_scale, k_i8, k_scale, k_mean, v_hat, v_scale (v_scale only in
 *   FP8 mode, may be NULL otherwise).
 *   gran: SAGE_GRAN_BLOCK (the outputs of the two calls) or SAGE_GRAN_THREAD (per-token
 *   Q scales and per-32-key K scales, layouts at sage_qk_gran; attention then goes
 *   through sage_attn_fwd_g with the same gran).
 *   workspace: at least sage_quant_qkv_workspace_bytes(...) bytes, 8-byte aligned,
 *   contents on entry ignored and on exit unspecified.
 */
sage_status sage_quant_qkv(const void* q, const void* k, const void* v, sage_dtype dtype, sage_layout layout, int B,
                           int H_qo, int H_kv, int Nq, int Nkv, int D, sage_pv pv, sage_qk_gran gran, int8_t* q_i8,
                           float* q_scale, int8_t* k_i8, float* k_scale, float* k_mean, void* v_hat, float* v_scale,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * sage_quant_qkv for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the same arguments
 * and outputs, bit for bit, without the workspace -- its kernels use a static device
 * array of sage_quant_qkv_noalloc_max_bytes() bytes (32 MiB) that each GPU the library
 * runs on holds until the process ends.  The call allocates and frees nothing.
 *   Limit: sizes whose sage_quant_qkv_workspace_bytes(...) exceeds that maximum return
 *   SAGE_ERR_UNSUPPORTED before any HIP call (for example B=4, H_kv=32, D=128 FP8
 *   fits up to Nkv = 10880; larger problems use sage_quant_qkv).
 *   Concurrency: every call on one GPU shares that GPU's array.  Calls that may overlap
 *   on one GPU (different streams, or threads without ordering) race and give wrong
 *   outputs; calls ordered on one stream are safe.  Nothing in the array has to start
 *   at zero, and a call leaves the previous call's contents overwritten.
 */
size_t sage_quant_qkv_noalloc_max_bytes(void);
sage_status sage_quant_qkv_noalloc(const void* q, const void* k, const void* v, sage_dtype dtype, sage_layout layout,
                                   int B, int H_qo, int H_kv, int Nq, int Nkv, int D, sage_pv pv, sage_qk_gran gran,
                                   int8_t* q_i8, float* q_scale, int8_t* k_i8, float* k_scale, float* k_mean,
                                   void* v_hat, float* v_scale, void* stream);

/*
 * The K and V part of sage_quant_qkv alone (K mean, INT8 codes and block scales of the
 * smoothed K, V^ and v_scale; SageAttention README, "Current Features"), for use with
 * sage_attn_fwd_fused_q, which quantises Q itself.  Block granularity, dense batches.
 *   Arguments, layouts, workspace (sage_quant_qkv_workspace_bytes(B, H_kv, Nkv, D, pv)
 *   bytes, 8-byte aligned, contents ignored) and errors as sage_quant_qkv, without the
 *   Q tensors; results bit-identical to that call's K and V outputs.
 */
sage_status sage_quant_kv(const void* k, const void* v, sage_dtype dtype, sage_layout layout, int B, int H_kv, int Nkv,
                          int D, sage_pv pv, int8_t* k_i8, float* k_scale, float* k_mean, void* v_hat, float* v_scale,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * Attention on the quantised operands (step 3-4 above).
 *   Reads q_i8/q_scale/k_i8/k_scale/v_hat/v_scale as produced by the two calls
 *   above (v_scale only in FP8 mode, may be NULL otherwise).
 *   out: [B,H_qo,Nq,D] (HND) or [B,Nq,H_qo,D] (NHD) in out_dtype; every element
 *   is written.
 *   is_causal: key j is visible to query i iff j <= i + Nkv - Nq (the diagonal
 *   aligned to the bottom-right corner: with Nq < Nkv the queries are the last Nq
 *   positions of the keys' sequence; README "Project Updates" allows q and k/v of
 *   different lengths).  A query that sees no key (Nq > Nkv, i < Nq - Nkv) gets an
 *   output row of zeros.
 *   sm_scale: finite and > 0 (callers pass 1/sqrt(D) for SDPA semantics).
 *   accum: SAGE_ACC_FP32, SAGE_ACC_FP16_FP32 or SAGE_ACC_FP16_FP32_SPLIT.
 */
sage_status sage_attn_fwd(const int8_t* q_i8, const float* q_scale, const int8_t* k_i8, const float* k_scale,
                          const void* v_hat, const float* v_scale, void* out, sage_dtype out_dtype,
                          sage_layout out_layout, int B, int H_qo, int H_kv, int Nq, int Nkv, int D, int is_causal,
                          float sm_scale, sage_pv pv, sage_accum accum, void* stream);

/* sage_attn_fwd on operands quantised with granularity `gran` (sage_quant_qkv):
 * each score is dequantised with its query's and its key's own scale.
 * sage_attn_fwd(...) is sage_attn_fwd_g(..., SAGE_GRAN_BLOCK, stream). */
sage_status sage_attn_fwd_g(const int8_t* q_i8, const float* q_scale, const int8_t* k_i8, const float* k_scale,
                            const void* v_hat, const float* v_scale, void* out, sage_dtype out_dtype,
                            sage_layout out_layout, int B, int H_qo, int H_kv, int Nq, int Nkv, int D, int is_causal,
                            float sm_scale, sage_pv pv, sage_accum accum, sage_qk_gran gran, void* stream);

/*
 * Key-range splits for launches that leave the chip idle (few heads and short query
 * ranges: B=1 H=8 N=2048 gives 128 workgroups for 256 CUs).  The key tiles of every
 * 128-query tile are split into num_splits ranges of equal tile count; each range runs
 * the online softmax of sage_attn_fwd on its own (its own running maximum, from -inf)
 * and leaves its own output o_s = O_s / l_s (fp16: |o_s| is bounded by the largest
 * |v^|, an fp16 value), running maximum m_s and row sum l_s (fp32) in the workspace; a
 * second kernel combines them, o = sum_s w_s o_s / sum_s w_s with w_s = 2^(m_s - M) l_s
 * and M = max_s m_s, and writes out as sage_attn_fwd does.  This is the same
 * attention with the softmax state merged once more (the merge the online softmax
 * already does between key tiles); P's roundings are then taken relative to each
 * range's running maximum, which moves FP16 P by at most one fp16 rounding (the output
 * stays within the parity bar), but would move FP8 P codes by up to a binade, so the
 * splits are offered with SAGE_PV_FP16 only (SAGE_ERR_UNSUPPORTED otherwise).
 *   Arguments: those of sage_attn_fwd (block granularity), plus num_splits (1 = plain
 *   sage_attn_fwd, workspace ignored; at most 64) and a device workspace of at least
 *   sage_attn_fwd_split_workspace_bytes(B, H_qo, Nq, D, num_splits) bytes, 16-byte
 *   aligned, contents on entry ignored and on exit unspecified.
 *   sage_attn_fwd_split_choice gives the library's pick for a shape: 1 (no split) unless
 *   pv is SAGE_PV_FP16 and the unsplit launch has fewer than 384 workgroups; then enough
 *   splits for about two workgroups per CU, each of at least four key tiles.
 */
int sage_attn_fwd_split_choice(int B, int H_qo, int Nq, int Nkv, int D, int is_causal, sage_pv pv);
size_t sage_attn_fwd_split_workspace_bytes(int B, int H_qo, int Nq, int D, int num_splits);
sage_status sage_attn_fwd_split(const int8_t* q_i8, const float* q_scale, const int8_t* k_i8, const float* k_scale,
                                const void* v_hat, const float* v_scale, void* out, sage_dtype out_dtype,
                                sage_layout out_layout, int B, int H_qo, int H_kv, int Nq, int Nkv, int D,
                                int is_causal, float sm_scale, sage_pv pv, sage_accum accum, int num_splits,
                                void* workspace, size_t workspace_bytes, void* stream);

/*
 * Attention with the Q quantisation done in the attention kernel itself: the same
 * scheme as sage_quant_qkv + sage_attn_fwd (block granularity; SageAttention README,
 * "Current Features"), but each workgroup reads its 128 queries in fp16 / bf16 and
 * quantises them per 64-token block in its prologue (the block quantiser's arithmetic,
 * so the codes and scales are bit-identical to sage_quant_qkv's), so the INT8 Q codes
 * never go through HBM.  The output is bit-identical to sage_attn_fwd's on those codes.
 *   q: fp16 / bf16 (dtype), layout HND or NHD, dense, 16-byte aligned; the output takes
 *   q's dtype and layout.  k_i8 / k_scale / v_hat / v_scale as from sage_quant_kv (or
 *   sage_quant_qkv).  q_i8_out [B][H_qo][N_pad][Dp] (16-byte aligned) and q_scale_out
 *   [B][H_qo][NB], both optional (null: not written), receive the codes and scales the
 *   kernel formed.  accum SAGE_ACC_FP16_FP32_SPLIT: SAGE_ERR_UNSUPPORTED; other errors as
 *   sage_attn_fwd.
 */
sage_status sage_attn_fwd_fused_q(const void* q, sage_dtype dtype, sage_layout layout, const int8_t* k_i8,
                                  const float* k_scale, const void* v_hat, const float* v_scale, void* out, int B,
                                  int H_qo, int H_kv, int Nq, int Nkv, int D, int is_causal, float sm_scale, sage_pv pv,
                                  sage_accum accum, int8_t* q_i8_out, float* q_scale_out, void* stream);

/*
 * Debug dump of INT32 score tiles through the attention kernel's own operand
 * path: the K^ tile arrives by the same direct-to-LDS loads and swizzle, and the
 * scores come from the same matrix-instruction sequence and accumulator form (at
 * head dims up to 128 the accumulators start at a fixed bias, taken off again as an
 * integer before the write), in the MFMA operand order of the given PV mode.
 *   tiles: device int32 [T][4] = (b, h_qo, q_block, k_block), each in range.
 *   out:   device int32 [T][64][64]; out[t][i][j] = sum_c q_i8[b,h,64*qb+i,c] *
 *          k_i8[b,h_kv,64*kb+j,c] (padding rows/columns give 0).
 */
sage_status sage_debug_qk_int32(const int8_t* q_i8, const int8_t* k_i8, int B, int H_qo, int H_kv, int Nq, int Nkv,
                                int D, sage_pv pv, const int32_t* tiles, int T, int32_t* out, void* stream);

/* ---------------------------------------------------------------------------
 * Variable-length batches (README "Available APIs": sageattn_varlen, several
 * sequences of different lengths in one call; "Project Updates": q and k/v of
 * different lengths).  The tokens of the B sequences are packed along one axis:
 *   q [total_q][H_qo][D], k and v [total_kv][H_kv][D], out [total_q][H_qo][D],
 *   all contiguous; cu_seqlens_q / cu_seqlens_kv are DEVICE int32 [B + 1] prefix
 *   sums (cu[0] = 0, non-decreasing, cu[B] = total): sequence b holds tokens
 *   cu[b] .. cu[b+1]-1.  max_seqlen_q / max_seqlen_kv (host) bound every sequence's
 *   length and size the launch grids.
 * The batch is the dense operation above applied to every sequence on its own:
 * its own K mean, block scales and V scales, causal aligned per sequence; a
 * sequence without keys gives zeros.  The kernels clamp what they read from
 * cu_seqlens into [0, total] and to max_seqlen, so inconsistent prefix sums give
 * wrong numbers but no access outside the buffers.
 * Layouts of the quantised intermediates: per (kv) head, sage_varlen_rows(total, B)
 * = total + 64*B rows of Dp elements and sage_varlen_slots(total, B) =
 * ceil(rows / 64) block slots; sequence b's 64-token block j occupies rows
 * R_b + 64*j .. R_b + 64*j + 63, R_b = cu[b] + 64*b (rows past the sequence's end
 * written with zero), and slot floor(R_b / 64) + j:
 *   q_i8     int8   [H_qo][rows(total_q)][Dp]     q_scale  float [H_qo][slots(total_q)]
 *   k_i8     int8   [H_kv][rows(total_kv)][Dp]    k_scale  float [H_kv][slots(total_kv)]
 *   k_mean   float  [B][H_kv][D]
 *   v_hat    fp16 or e4m3 [H_kv][slots(total_kv)][Dp][64] (blocks channel-major)
 *   v_scale  float  [B][H_kv][Dp]                  (FP8 mode only)
 * Rows and slots between two sequences' blocks are not written.
 */
int64_t sage_varlen_rows(int total, int B);
int64_t sage_varlen_slots(int total, int B);

/* Workspace of sage_quant_qk_varlen: H_kv * slots(total_kv, B) * D * 8 bytes (fp64
 * block partial sums of K).  sage_quant_v_varlen takes sage_quant_v_workspace_bytes. */
size_t sage_quant_qk_varlen_workspace_bytes(int B, int H_kv, int total_kv, int D);

/* sage_quant_qk on a packed batch: per sequence, the K mean over its own tokens and
 * the 64-token blocks counted from its first token (arithmetic as sage_quant_qk). */
sage_status sage_quant_qk_varlen(const void* q, const void* k, sage_dtype dtype, const int32_t* cu_seqlens_q,
                                 const int32_t* cu_seqlens_kv, int B, int H_qo, int H_kv, int total_q, int total_kv,
                                 int max_seqlen_q, int max_seqlen_kv, int D, int8_t* q_i8, float* q_scale,
                                 int8_t* k_i8, float* k_scale, float* k_mean, void* workspace, size_t workspace_bytes,
                                 void* stream);

/* sage_quant_v on a packed batch: in FP8 mode the per-channel scale of each sequence
 * comes from that sequence's tokens alone. */
sage_status sage_quant_v_varlen(const void* v, sage_dtype dtype, const int32_t* cu_seqlens_kv, int B, int H_kv,
                                int total_kv, int max_seqlen_kv, int D, sage_pv pv, void* v_hat, float* v_scale,
                                void* workspace, size_t workspace_bytes, void* stream);

/* Workspace of sage_quant_qkv_varlen: as sage_quant_qkv_workspace_bytes with
 * H_kv * slots(total_kv, B) block slots in place of B * H_kv * NB(Nkv). */
size_t sage_quant_qkv_varlen_workspace_bytes(int B, int H_kv, int total_kv, int D, sage_pv pv);

/* sage_quant_qk_varlen and sage_quant_v_varlen in one call (outputs bit for bit the
 * same; the fused launch sequence of sage_quant_qkv). */
sage_status sage_quant_qkv_varlen(const void* q, const void* k, const void* v, sage_dtype dtype,
                                  const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_kv, int B, int H_qo, int H_kv,
                                  int total_q, int total_kv, int max_seqlen_q, int max_seqlen_kv, int D, sage_pv pv,
                                  sage_qk_gran gran, int8_t* q_i8, float* q_scale, int8_t* k_i8, float* k_scale,
                                  float* k_mean, void* v_hat, float* v_scale, void* workspace, size_t workspace_bytes,
                                  void* stream);

/* sage_attn_fwd on a packed batch (causal per sequence as in sage_attn_fwd);
 * out [total_q][H_qo][D] in out_dtype, every element written. */
sage_status sage_attn_fwd_varlen(const int8_t* q_i8, const float* q_scale, const int8_t* k_i8, const float* k_scale,
                                 const void* v_hat, const float* v_scale, void* out, sage_dtype out_dtype,
                                 const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_kv, int B, int H_qo, int H_kv,
                                 int total_q, int total_kv, int max_seqlen_q, int max_seqlen_kv, int D, int is_causal,
                                 float sm_scale, sage_pv pv, sage_accum accum, void* stream);

/* sage_attn_fwd_varlen with a quantisation granularity (as sage_attn_fwd_g). */
sage_status sage_attn_fwd_varlen_g(const int8_t* q_i8, const float* q_scale, const int8_t* k_i8, const float* k_scale,
                                   const void* v_hat, const float* v_scale, void* out, sage_dtype out_dtype,
                                   const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_kv, int B, int H_qo,
                                   int H_kv, int total_q, int total_kv, int max_seqlen_q, int max_seqlen_kv, int D,
                                   int is_causal, float sm_scale, sage_pv pv, sage_accum accum, sage_qk_gran gran,
                                   void* stream);

/* Packed-batch forms of sage_quant_kv and sage_attn_fwd_fused_q (block granularity):
 * K and V quantised as sage_quant_qkv_varlen does (workspace
 * sage_quant_qkv_varlen_workspace_bytes(B, H_kv, total_kv, D, pv)), and attention that
 * quantises each sequence's Q (q [total_q][H_qo][D] in fp16 / bf16, 16-byte aligned) in
 * its prologue; out [total_q][H_qo][D] in q's dtype.  q_i8_out [H_qo][rows][Dp] and
 * q_scale_out [H_qo][slots] (rows, slots of total_q), both optional, receive the codes
 * and scales, which equal sage_quant_qkv_varlen's bit for bit, as does the output
 * sage_attn_fwd_varlen's.  Errors as the calls they mirror. */
sage_status sage_quant_kv_varlen(const void* k, const void* v, sage_dtype dtype, const int32_t* cu_seqlens_kv, int B,
                                 int H_kv, int total_kv, int max_seqlen_kv, int D, sage_pv pv, int8_t* k_i8,
                                 float* k_scale, float* k_mean, void* v_hat, float* v_scale, void* workspace,
                                 size_t workspace_bytes, void* stream);
sage_status sage_attn_fwd_varlen_fused_q(const void* q, sage_dtype dtype, const int32_t* cu_seqlens_q,
                                         const int32_t* cu_seqlens_kv, const int8_t* k_i8, const float* k_scale,
                                         const void* v_hat, const float* v_scale, void* out, int B, int H_qo, int H_kv,
                                         int total_q, int total_kv, int max_seqlen_q, int max_seqlen_kv, int D,
                                         int is_causal, float sm_scale, sage_pv pv, sage_accum accum, int8_t* q_i8_out,
                                         float* q_scale_out, void* stream);

/* ---- Microscaling FP4 (MXFP4) variant ---------------------------------------------
 * The SageAttention README names a microscaling FP4 attention for inference
 * ("SageAttention3: Microscaling FP4 Attention", project updates and citations) and
 * gives only that title.  These calls take the OCP Microscaling (MX) v1.0 MXFP4 format
 * that gfx950's scaled matrix instructions read, on both products of the scheme above
 * (K smoothing and the online base-2 softmax over 64-key blocks unchanged):
 *   - a block of 32 consecutive elements along a contraction axis shares the scale
 *     X = 2^E, E = floor(log2 amax) - 2 held to [-126, 127] (an all-zero block: -126),
 *     stored as the E8M0 byte E + 127;
 *   - each element is e2m1(x / X): round to nearest even, saturating at 6, sign kept;
 *     a 4-bit code (sign bit 8 | index in {0, .5, 1, 1.5, 2, 3, 4, 6}); two per byte,
 *     element 2t in the low nibble of byte t;
 *   - Q and smoothed K are blocked along the channels of each token, V along the
 *     tokens of each channel, P along 32 consecutive keys (after the softmax step, with
 *     p = 2^(s2 - m) and the row sum l over unquantised p).
 * Scores: S = sum of dequantised Q * K products (scales applied inside the matrix
 * instruction, fp32), s2 = fp32(S * fp32(sm_scale * log2 e)), t = s2 - m in fp32, so
 * the row maximum has p = 1 exactly.  Head dims up to 256 (Dp = 64, 128 or 256, as
 * above); dense batches here, packed ones below.  Layouts (row-major, innermost last):
 *   q4      uint8 [B][H_qo][N_pad(Nq)][Dp/2]      q4_exp  uint8 [B][H_qo][N_pad(Nq)][Dp/32]
 *   k4      uint8 [B][H_kv][N_pad(Nkv)][Dp/2]     k4_exp  uint8 [B][H_kv][N_pad(Nkv)][Dp/32]
 *   k_mean  float [B][H_kv][D]
 *   v4      uint8 [B][H_kv][NB(Nkv)][Dp][32]      (per 64-token block, channel-major:
 *                                                   byte t of channel c = tokens 2t, 2t+1)
 *   v4_exp  uint8 [B][H_kv][NB(Nkv)][2][32][Dp/32] (block j, token half g, channel
 *                                                   32 u + i at [g][i][u])
 * Padding (tokens >= N, channels >= D) holds zero codes and the exponent byte 1. */

/* Workspace of sage_quant_mxfp4: B * H_kv * NB(Nkv) * D * 8 bytes (fp64 K block
 * channel sums); 0 for invalid sizes. */
size_t sage_quant_mxfp4_workspace_bytes(int B, int H_kv, int Nkv, int D);

/* K mean, then MXFP4 codes and exponents of Q, smoothed K and V (layouts above).
 * q, k, v: fp16/bf16 in `layout` (as sage_quant_qk / sage_quant_v).  Code buffers
 * 16-byte aligned; workspace at least sage_quant_mxfp4_workspace_bytes(...) bytes,
 * 8-byte aligned, overwritten.  D > 256: SAGE_ERR_UNSUPPORTED. */
sage_status sage_quant_mxfp4(const void* q, const void* k, const void* v, sage_dtype dtype, sage_layout layout, int B,
                             int H_qo, int H_kv, int Nq, int Nkv, int D, uint8_t* q4, uint8_t* q4_exp, uint8_t* k4,
                             uint8_t* k4_exp, float* k_mean, uint8_t* v4, uint8_t* v4_exp, void* workspace,
                             size_t workspace_bytes, void* stream);

/* Attention forward on the outputs of sage_quant_mxfp4: out in out_dtype and
 * out_layout ([B][H_qo][Nq][D] or [B][Nq][H_qo][D]), every element written; causal
 * aligned to the bottom-right corner as in sage_attn_fwd; a query that sees no key
 * gives zeros.  sm_scale finite and > 0.  D > 256: SAGE_ERR_UNSUPPORTED. */
sage_status sage_attn_fwd_mxfp4(const uint8_t* q4, const uint8_t* q4_exp, const uint8_t* k4, const uint8_t* k4_exp,
                                const uint8_t* v4, const uint8_t* v4_exp, void* out, sage_dtype out_dtype,
                                sage_layout out_layout, int B, int H_qo, int H_kv, int Nq, int Nkv, int D,
                                int is_causal, float sm_scale, void* stream);

/*
 * The MXFP4 variant with Q quantised inside the attention kernel (the same scheme as
 * sage_quant_mxfp4 + sage_attn_fwd_mxfp4; SageAttention README, "Project Updates"):
 * sage_quant_mxfp4_kv writes the K mean and the codes and exponents of the smoothed K
 * and of V only (arguments, layouts, workspace and errors as sage_quant_mxfp4 without the
 * Q tensors; results bit-identical), and sage_attn_fwd_mxfp4_fused_q reads q in fp16 /
 * bf16 (dtype; layout HND or NHD, dense, 16-byte aligned; the output takes q's dtype and
 * layout): every lane quantises the 32-channel blocks of its own query that it holds as
 * matrix-instruction operands, in the arithmetic of sage_quant_mxfp4, so codes,
 * exponents and output are bit-identical to the separate calls.  q4_out [B][H_qo][N_pad]
 * [Dp/2] (16-byte aligned) and q4_exp_out [B][H_qo][N_pad][Dp/32], both optional (null:
 * not written), receive the codes and exponent bytes the kernel formed.
 */
sage_status sage_quant_mxfp4_kv(const void* k, const void* v, sage_dtype dtype, sage_layout layout, int B, int H_kv,
                                int Nkv, int D, uint8_t* k4, uint8_t* k4_exp, float* k_mean, uint8_t* v4,
                                uint8_t* v4_exp, void* workspace, size_t workspace_bytes, void* stream);
sage_status sage_attn_fwd_mxfp4_fused_q(const void* q, sage_dtype dtype, sage_layout layout, const uint8_t* k4,
                                        const uint8_t* k4_exp, const uint8_t* v4, const uint8_t* v4_exp, void* out,
                                        int B, int H_qo, int H_kv, int Nq, int Nkv, int D, int is_causal,
                                        float sm_scale, uint8_t* q4_out, uint8_t* q4_exp_out, void* stream);

/* The MXFP4 calls on a packed batch (README "Available APIs", sageattn_varlen; the dense
 * scheme per sequence, as for the INT8 calls): q (total_q, H_qo, D), k and v
 * (total_kv, H_kv, D), cu_seqlens as for sage_quant_qk_varlen.  Rows and slots per head
 * as there: q4 [H_qo][rows(total_q)][Dp/2], q4_exp [H_qo][rows(total_q)][Dp/32],
 * k4 / k4_exp likewise over H_kv and total_kv, v4 [H_kv][slots(total_kv)][Dp][32],
 * v4_exp [H_kv][slots(total_kv)][2][32][Dp/32], k_mean [B][H_kv][D]; out
 * [total_q][H_qo][D].  Workspace: H_kv * slots(total_kv) * D * 8 bytes. */
size_t sage_quant_mxfp4_varlen_workspace_bytes(int B, int H_kv, int total_kv, int D);
sage_status sage_quant_mxfp4_varlen(const void* q, const void* k, const void* v, sage_dtype dtype,
                                    const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_kv, int B, int H_qo,
                                    int H_kv, int total_q, int total_kv, int max_seqlen_q, int max_seqlen_kv, int D,
                                    uint8_t* q4, uint8_t* q4_exp, uint8_t* k4, uint8_t* k4_exp, float* k_mean,
                                    uint8_t* v4, uint8_t* v4_exp, void* workspace, size_t workspace_bytes,
                                    void* stream);
sage_status sage_attn_fwd_mxfp4_varlen(const uint8_t* q4, const uint8_t* q4_exp, const uint8_t* k4,
                                       const uint8_t* k4_exp, const uint8_t* v4, const uint8_t* v4_exp, void* out,
                                       sage_dtype out_dtype, const int32_t* cu_seqlens_q,
                                       const int32_t* cu_seqlens_kv, int B, int H_qo, int H_kv, int total_q,
                                       int total_kv, int max_seqlen_q, int max_seqlen_kv, int D, int is_causal,
                                       float sm_scale, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SAGE_H_ */
