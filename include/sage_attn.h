/*
 * sage_attn.h -- C ABI of an MI355X (gfx950) library for SageAttention-style
 * quantized attention: O = softmax(sm_scale * Q K^T + mask) V computed tile by
 * tile with online softmax, after mean-smoothing of K (and of Q on the 4-bit
 * path) and per-block low-bit quantization of Q and K; P and V are quantized
 * for the PV product; an 8-bit backward produces dQ, dK, dV.
 *
 * Sources of the operation (web pages on SageAttention):
 *   - the problem is plug-and-play attention on q, k, v with a causal flag
 *     (SageAttention3 abstract; "compatible with FlashAttention" in the
 *     SageAttention contributions, reply to reviewer wwcu W1);
 *   - online softmax and FlashAttention tiling (SageAttention review thread,
 *     reply to reviewer xY6z Q3; deferred normalisation, reply to xY6z Q2);
 *   - smoothing K, INT8 QK^T, per-block granularity (reply to wwcu W1;
 *     SageAttn-B, reply to xY6z W1-(2), Q1);
 *   - P~ and V in FP8, smoothing Q, two-level P~V accumulation (SageAttention2
 *     abstract); microscaling FP4 attention and 8-bit forward + backward
 *     (SageAttention3 abstract).
 *
 * Conventions for every entry point:
 *   - Tensors are contiguous [B, H, N, d] (token-major per head), d in {64,128},
 *     N >= 1 (queries and keys share N), all device pointers 16-byte aligned.
 *   - Causal masking is top-left aligned: query i sees keys j <= i.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Every call is
 *     asynchronous on that stream; the caller synchronizes.
 *   - The caller owns every buffer it passes; the library keeps no pointer
 *     past the call.
 *   - All argument checks run on the host before anything is launched.  On an
 *     error nothing is launched, outputs are untouched, and sage_last_error()
 *     (thread-local) describes the problem.  Device faults surface at the
 *     caller's next synchronization.  No C++ exception crosses this boundary.
 *   - NaN or Inf inputs are not errors; they propagate into the affected
 *     scales and rows.
 */
#ifndef SAGE_ATTN_H
#define SAGE_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SAGE_ABI_VERSION 2

/* Environment (debugging only; no effect on results): SAGE_LOG=1 prints one line on stderr per
 * entry-point call (problem, status, error text); SAGE_DEBUG_LDS_PAD=<bytes> adds dynamic LDS
 * to the fused forward and backward launches, lowering how many workgroups share a CU (a
 * result that changed with it would reveal an LDS race); SAGE_FAULT_INJECT=alloc makes the
 * allocating entry point fail its allocation. */

typedef enum {
    SAGE_OK = 0,
    SAGE_ERR_INVALID_ARG = 1,   /* null pointer, bad size, bad scale, misaligned pointer */
    SAGE_ERR_UNSUPPORTED = 2,   /* valid request the library does not implement (d, format pair) */
    SAGE_ERR_WORKSPACE = 3,     /* workspace or quant buffer smaller than required */
    SAGE_ERR_OUT_OF_MEMORY = 4, /* internal device allocation failed */
    SAGE_ERR_HIP = 5            /* a HIP runtime call or kernel launch failed */
} sage_status;

/* Element formats.  INT8: symmetric +-127 codes with one fp32 step per 64-token
 * block.  FP8: OCP E4M3FN.  MXFP4: OCP MX, E2M1 elements in 32-element blocks
 * sharing an E8M0 (power-of-two) scale.  MXFP8: OCP MX with E4M3 elements
 * (scale floor(log2 amax) - 8, elements saturated at 448); as pv_fmt it keeps
 * P~ in FP8 with the static x448 scale (SageAttention3 abstract: microscaling
 * FP4 attention, with 8-bit V as the higher-precision fallback).  F16 (as
 * pv_fmt, with INT8 QK): the 16-bit P~V fallback of the original SageAttention
 * (INT8 QK^T with FP16 P and V, review thread, reply to reviewer wwcu W1): P~ and
 * V rounded to IEEE fp16 (RNE, overflow to infinity), fp32 accumulation -- the
 * matrix cores have no fp16-accumulating form.  INT8_TOKEN (as qk_fmt): INT8
 * codes with finer steps -- one per query token and one per 32 keys -- the
 * granularity each lane's scores share in the fused kernel (the finer
 * SageAttention-T / thread-level variants, review thread accuracy table in the
 * reply to tyTT W1, SageAttention2 abstract).  MXFP4_QBLOCK (as qk_fmt): MXFP4
 * with Q smoothed by the mean of each 128-query block instead of the whole
 * sequence (the pages leave the form of "smooth Q" open, SageAttention2
 * abstract); the removed part returns as dS = mu_q(block) . K_s per block and
 * key.  On packed sequences the blocks start at each sequence's first query. */
enum { SAGE_FMT_INT8 = 1, SAGE_FMT_FP8 = 2, SAGE_FMT_MXFP4 = 3, SAGE_FMT_MXFP8 = 4, SAGE_FMT_F16 = 5,
       SAGE_FMT_INT8_TOKEN = 6, SAGE_FMT_MXFP4_QBLOCK = 7 };

/* I/O element types of Q, K, V, O, dO, dQ, dK, dV. */
enum { SAGE_DT_BF16 = 0, SAGE_DT_F16 = 1 };

/* Supported (qk_fmt, pv_fmt) pairs: (INT8, FP8), (INT8, F16), (INT8_TOKEN, FP8),
 * (INT8_TOKEN, F16), (MXFP4 or MXFP4_QBLOCK, FP8 or MXFP4 or MXFP8). */
typedef struct {
    int B, H, N, d;      /* B, H, N >= 1 with B*H <= 65535, N <= 2^30 and B*H*(N+128)*d <= 2^40;
                            d is 64 or 128 */
    int causal;          /* 0 or 1 */
    float sm_scale;      /* finite, > 0; typically 1/sqrt(d) */
    int io_dtype;        /* SAGE_DT_* */
    int qk_fmt, pv_fmt;  /* SAGE_FMT_* */
} sage_problem;

/*
 * Byte offsets of each part inside a quantized buffer (see sage_quantize).
 * Let BH = B*H, Np = N rounded up to a multiple of 128 (padding tokens carry
 * zero codes), nb = Np/64.
 *   mu_k      fp32 [BH, d]     channel mean of K over all N tokens
 *   mu_q      fp32 [BH, d]     channel mean of Q (MXFP4 QK only; MXFP4_QBLOCK:
 *             [BH, Np/128, d], the mean of each 128-query block, followed by the
 *             same means in fp64 as [BH, Np/128 rounded up to 16, d], zero-padded:
 *             scratch of the dS step)
 *   q_codes   INT8: int8 [BH, Np, d];  MXFP4: packed E2M1 [BH, Np, d/2] of
 *             Q - mu_q, element 2i in the low nibble of byte i
 *   q_scales  INT8: fp32 [BH, nb] step of each 64-token block; INT8_TOKEN:
 *             fp32 [BH, Np] step of each token;
 *             MXFP4: E8M0 bytes [BH, Np, d/32] per token per 32 channels
 *   k_codes, k_scales   the same for K - mu_k (INT8_TOKEN: fp32 [BH, Np/32], a step
 *             per 32 keys)
 *   v_codes   FP8 and MXFP8 V: E4M3 codes tiled [BH, Np/64, d, 64] (64 tokens
 *             of one channel contiguous);  MXFP4 V: packed E2M1 [BH, Np/64, d, 32];
 *             F16 V: fp16 tiled [BH, Np/64, d, 64]
 *   v_scales  FP8 V: fp32 [BH, d] per-channel step;  MXFP4 and MXFP8 V: E8M0
 *             bytes [BH, Np/32, d] per 32-token group per channel
 *   delta_s   fp32 [BH, Np]    mu_q . (k_t - mu_k), added to every score (MXFP4 QK;
 *             MXFP4_QBLOCK: [BH, Np/128, Np], one row per query block)
 *   lse_corr  fp32 [BH, N]     sm_scale * q_t . mu_k, added to the LSE only
 *   stats     fp64 / uint32 per-chunk partials of the smoothing statistics, then (packed
 *             sequences) the batch's table of (sequence, 64-token block) pairs (scratch)
 */
typedef struct {
    size_t mu_k, mu_q, q_codes, q_scales, k_codes, k_scales, v_codes, v_scales,
           delta_s, lse_corr, stats, total;
} sage_quant_layout;

/*
 * Forward attention, bf16 I/O, the one-call form: smoothing of K (and Q on the
 * MXFP4 path), per-block quantization, then the tiled online-softmax loop with
 * P~V in the chosen format and the normalisation after the last tile.
 * Passages: plug-and-play quantized attention on q, k, v with a causal flag
 * (SageAttention3 abstract); smoothing K and INT8 QK^T (review thread, reply to
 * reviewer wwcu W1); online softmax over K tiles and normalisation once at the
 * end (reply to reviewer xY6z, Q3 and Q2); FP8 P~V with two-level accumulation
 * and smoothing Q (SageAttention2 abstract); microscaled FP4 (SageAttention3
 * abstract).
 *   q, k, v   device bf16 [B,H,N,d], read only, owned by the caller
 *   o         device bf16 [B,H,N,d], written
 *   causal    0 or 1 (top-left aligned); sm_scale finite and > 0
 *   qk_fmt, pv_fmt   a supported SAGE_FMT_* pair
 * Takes its scratch (the quantized buffer) with hipMallocAsync / hipFreeAsync
 * on `stream` (stream-ordered, so calls on different streams are independent).
 * Errors: INVALID_ARG (null or misaligned pointer, bad size or scale),
 * UNSUPPORTED (d or format pair), OUT_OF_MEMORY (the scratch), HIP (a launch).
 */
sage_status sage_attn_fwd(const void *q, const void *k, const void *v, void *o,
                          int B, int H, int N, int d, int causal, float sm_scale,
                          int qk_fmt, int pv_fmt, void *stream);

/*
 * The one-call forward for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  Same arguments, kernels and
 * results as sage_attn_fwd, but the quantized buffer lives in a fixed array of 64 MiB that the
 * library holds on each GPU it runs on until the process ends (found on the first call on a
 * device); the call allocates and frees nothing.  Problems whose quantized buffer exceeds
 * 64 MiB (sage_quant_size) return SAGE_ERR_WORKSPACE without launching.  Every call on one GPU
 * uses that GPU's array, so calls that overlap on one GPU (other streams, other threads) race;
 * calls on one stream are ordered.  Errors: as sage_attn_fwd, with WORKSPACE for the size and
 * HIP if the array's address cannot be found.
 */
sage_status sage_attn_fwd_noalloc(const void *q, const void *k, const void *v, void *o,
                                  int B, int H, int N, int d, int causal, float sm_scale,
                                  int qk_fmt, int pv_fmt, void *stream);

/*
 * Size and layout of the quantized buffer for `p` (the codes, steps and
 * smoothing terms of the prologue: per-block INT8 steps, review thread, reply
 * to reviewer xY6z W1-(2); MX blocks of 32 with E8M0 scales, SageAttention3
 * abstract and the TetraJet abstract's per-group microscaling).  Host only:
 * writes *bytes and, when layout is not NULL, the byte offsets of every part.
 * Errors: INVALID_ARG (null bytes or a bad problem), UNSUPPORTED.
 */
sage_status sage_quant_size(const sage_problem *p, size_t *bytes, sage_quant_layout *layout);

/*
 * Smoothing + quantization prologue: the per-channel mean of K over the tokens
 * (smoothing K, review thread, reply to reviewer wwcu W1; smoothing Q on the
 * 4-bit path, SageAttention2 abstract), per-block INT8 or MXFP4 codes of Q and
 * K, FP8 (or MX, or fp16) V, and the terms smoothing removes (dS added to the
 * scores, the row shift added to the LSE).
 *   q, k, v     device [B,H,N,d] in p->io_dtype, read only
 *   quant_buf   device, quant_bytes >= sage_quant_size's bytes, written as
 *               sage_quant_layout describes; owned by the caller, who may keep it
 *               and pass it to sage_attn_fwd_quantized
 * Errors: INVALID_ARG, UNSUPPORTED, WORKSPACE (quant_bytes too small), HIP.
 */
sage_status sage_quantize(const void *q, const void *k, const void *v, const sage_problem *p,
                          void *quant_buf, size_t quant_bytes, void *stream);

/*
 * Fused attention on a buffer written by sage_quantize for the same problem:
 * QK^T on INT8 or microscaled FP4 codes with the dequantization folded into the
 * softmax scale, online softmax over 64-key tiles (review thread, reply to
 * reviewer xY6z Q3), P~ quantized for the P~V product with fp32 accumulation
 * across tiles (two-level accumulation, SageAttention2 abstract), O / l after
 * the last tile (reply to xY6z Q2).
 *   quant_buf   device, read only (quant_bytes as sage_quant_size gives)
 *   o           device [B,H,N,d] in p->io_dtype, written
 *   lse         device fp32 [B,H,N] or NULL: natural-log log-sum-exp of the
 *               true, unsmoothed scaled scores
 * Errors: INVALID_ARG, UNSUPPORTED, WORKSPACE, HIP.
 */
sage_status sage_attn_fwd_quantized(const void *quant_buf, size_t quant_bytes, const sage_problem *p,
                                    void *o, float *lse, void *stream);

/* Workspace bytes needed by sage_attn_fwd_ex (the quantized buffer of sage_quant_size).
 * Host only.  Errors: INVALID_ARG, UNSUPPORTED. */
sage_status sage_attn_fwd_ws_size(const sage_problem *p, size_t *bytes);

/*
 * Forward with caller workspace: sage_quantize into ws, then
 * sage_attn_fwd_quantized (the same passages).  bf16 or fp16 I/O as
 * p->io_dtype; q, k, v read only; o written; lse device fp32 [B,H,N] or NULL;
 * ws device, ws_bytes >= sage_attn_fwd_ws_size, owned by the caller.  Launches
 * kernels only (no allocation, no memset), so a HIP graph may capture it.
 * Errors: INVALID_ARG, UNSUPPORTED, WORKSPACE, HIP.
 */
sage_status sage_attn_fwd_ex(const sage_problem *p, const void *q, const void *k, const void *v,
                             void *o, float *lse, void *ws, size_t ws_bytes, void *stream);

/* Workspace bytes needed by sage_attn_bwd.  Host only.  Errors: INVALID_ARG, UNSUPPORTED. */
sage_status sage_attn_bwd_ws_size(const sage_problem *p, size_t *bytes);

/*
 * 8-bit backward: dQ, dK, dV of softmax attention with every product on 8-bit
 * matrix cores (8-bit attention for training, forward and backward,
 * SageAttention3 abstract; SageBwd, SageAttention2++ related-papers page).
 * q, k, v, o, dout: device [B,H,N,d] (bf16 or fp16 as p->io_dtype; o is the
 * forward output), read only; lse: device fp32 [B,H,N] from the forward;
 * dq, dk, dv: device outputs [B,H,N,d], written.  p->qk_fmt must be INT8 and
 * p->pv_fmt FP8 (other pairs: SAGE_ERR_UNSUPPORTED); d is 64 or 128.  ws: device
 * workspace of at least sage_attn_bwd_ws_size bytes (the forward's quantized
 * buffer followed by the backward's operand tiles).
 */
sage_status sage_attn_bwd(const sage_problem *p, const void *q, const void *k, const void *v,
                          const void *o, const void *dout, const float *lse,
                          void *dq, void *dk, void *dv, void *ws, size_t ws_bytes, void *stream);

/*
 * sage_attn_bwd for a training step that ran the forward through sage_attn_fwd_ex (or
 * sage_quantize) with this workspace: the first sage_quant_size(p) bytes of ws must still hold
 * the quantized buffer that call wrote for this problem and these q and k (unchanged since), and
 * the Q/K quantization -- codes, steps, mu_k, LSE term, the forward's own -- is reused instead
 * of recomputed (the SageAttention3 abstract's 8-bit forward and backward as one training step).
 * Arguments, sizes (ws at least sage_attn_bwd_ws_size bytes) and errors as sage_attn_bwd; a
 * buffer that does not hold that quantization gives unspecified gradients, but every access
 * stays inside ws and the tensors.
 */
sage_status sage_attn_bwd_after_fwd(const sage_problem *p, const void *q, const void *k, const void *v,
                                    const void *o, const void *dout, const float *lse,
                                    void *dq, void *dk, void *dv, void *ws, size_t ws_bytes, void *stream);

/*
 * Packed variable-length sequences with grouped KV heads: the sageattn_varlen
 * entry named on the SageAttention3 code-link page, in FlashAttention's
 * cu_seqlens convention (the implementation builds on FlashAttention: review
 * thread, reply to reviewer wwcu W1).
 *   q, o           device [total_q, H, d]: the rows of all sequences back to back
 *   k, v           device [total_k, H_kv, d]
 *   cu_seqlens_q,  device int32 [B+1], non-decreasing, [0] = 0, [B] = total_q
 *   cu_seqlens_k   (total_k): sequence b is rows [cu[b], cu[b+1]); query and key
 *                  lengths may differ
 *   lse            device fp32 [H, total_q] or NULL
 * Query head h reads KV head h / (H / H_kv).  Every sequence is quantized on its
 * own (K mean and V channel steps per sequence and KV head, 64-token INT8 blocks
 * inside the sequence; MXFP4_QBLOCK: 128-query blocks from the sequence's first
 * query, with workspace for a dS strip of min(max_seqlen_k, total_k) keys per block
 * slot, about H * (total_q / 128 + B) * min(max_seqlen_k, total_k) floats).  Causal masking is top-left aligned per sequence (query
 * i sees keys j <= i).  A query with no key (an empty key sequence) gets a zero
 * output and LSE -inf.  max_seqlen_q / max_seqlen_k bound every sequence's
 * length (host values, as FlashAttention takes them; bounds above total_q /
 * total_k are clamped to them); the kernels clamp the
 * device offsets to [0, total] and the lengths to the bounds, so malformed
 * offsets give unspecified values but no access outside the tensors.
 * total_q = 0 returns SAGE_OK without launching; k and v may be NULL when
 * total_k = 0.  ws: device workspace of at least sage_varlen_ws_size bytes.
 */
typedef struct {
    int B;                  /* sequences */
    int H, H_kv;            /* query heads, key/value heads (H % H_kv == 0) */
    int d;
    int causal;             /* 0 or 1 */
    float sm_scale;         /* finite, > 0 */
    int io_dtype;           /* SAGE_DT_* */
    int qk_fmt, pv_fmt;     /* SAGE_FMT_*, the same pairs as sage_problem */
    int total_q, total_k;   /* rows of q and of k / v */
    int max_seqlen_q, max_seqlen_k;
} sage_varlen_problem;

/* Workspace bytes needed by sage_attn_varlen_fwd.  Host only.  Errors: INVALID_ARG, UNSUPPORTED. */
sage_status sage_varlen_ws_size(const sage_varlen_problem *p, size_t *bytes);

sage_status sage_attn_varlen_fwd(const sage_varlen_problem *p, const void *q, const void *k, const void *v,
                                 const int *cu_seqlens_q, const int *cu_seqlens_k, void *o, float *lse,
                                 void *ws, size_t ws_bytes, void *stream);

/* Status text, the calling thread's last error message (empty when none; valid until the
 * thread's next call into the library) and SAGE_ABI_VERSION.  Host only, never fail. */
const char *sage_status_string(sage_status s);
const char *sage_last_error(void);
int sage_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SAGE_ATTN_H */
