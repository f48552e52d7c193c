/*
 * attn.h - C ABI of the MI355X (gfx950) fused attention forward library.
 *
 * Two operations:
 *
 *   attn_fwd           O = softmax(Q K^T * scale [+ mask]) V for a batch of
 *                      sequences (prefill), computed tile by tile with an online
 *                      softmax so the score matrix never reaches memory.
 *   attn_decode_paged  the same for one query token per sequence over a paged
 *                      KV cache, split along the keys across workgroups and
 *                      merged with an LSE-weighted combine.
 *   attn_fwd_paged     chunked prefill: a chunk of new query tokens per
 *                      sequence attends to that sequence's keys in the same
 *                      paged KV cache.
 *   attn_bwd           the gradients of attn_fwd (dense batches).
 *
 * The operation is the softmax attention of the page "Agent 帮我写 CUDA：一个
 * Softmax Attention 算子的开发全记录" (section 二, reference baseline and the
 * note on D; section 四, the online-softmax recurrence that lets the score
 * matrix stay on chip). The variants (causal, sliding window, tanh softcap,
 * grouped-query heads, ragged batches, paged KV, split-KV decode, fp8 KV) are
 * the scenario axes of "Ask, Don't Equip: Question-Driven Coding Agents for
 * Deep Kernel Optimization", section 研究动机. Where those pages only name a
 * variant, this header states the definition used.
 *
 * Conventions for every entry point:
 *  - All tensor pointers are DEVICE pointers (HIP device memory) owned by the
 *    caller. The library never allocates, frees or synchronises; it only
 *    enqueues kernels on `stream` (a hipStream_t; NULL = the null stream) and
 *    returns. Buffers must stay valid until the stream has passed the work.
 *  - Every argument check is done on the host, synchronously, before any HIP
 *    call; a failed check enqueues nothing and returns a non-zero status, with
 *    a detail string available from attn_last_error_message() (thread-local).
 *  - Contents of device-resident index arrays (cu_seqlens, block_table,
 *    seq_lens) are trusted: the library does not read them on the host.
 *  - Every base pointer and every stride in bytes of the token / head / batch
 *    dimensions must be a multiple of 16 bytes (128-bit loads); the head_dim
 *    dimension must be contiguous (stride 1).
 */
#ifndef ATTN_H_
#define ATTN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ATTN_SUCCESS = 0,
  ATTN_ERROR_INVALID_VALUE = 1,      /* null pointer, bad size, bad stride, bad combination */
  ATTN_ERROR_NOT_SUPPORTED = 2,      /* head_dim / dtype / alignment outside what is built */
  ATTN_ERROR_WORKSPACE_TOO_SMALL = 3,
  ATTN_ERROR_LAUNCH_FAILED = 4       /* the HIP runtime reported an error at launch */
} attn_status_t;

typedef enum {
  ATTN_F32 = 0,
  ATTN_F16 = 1,
  ATTN_BF16 = 2,
  ATTN_FP8_E4M3 = 3 /* OCP E4M3 ("e4m3fn"): bias 7, max 448, S.1111.111 = NaN, no inf */
} attn_dtype_t;

/* ---------------------------------------------------------------- prefill ---- */

typedef struct {
  int32_t batch;         /* B >= 1 (ragged: number of sequences) */
  int32_t num_q_heads;   /* Hq >= 1 */
  int32_t num_kv_heads;  /* Hkv >= 1, Hq % Hkv == 0; query head h reads KV head h / (Hq/Hkv) */
  int32_t seqlen_q;      /* dense: Nq; ragged: an upper bound of every sequence's query length */
  int32_t seqlen_k;      /* dense: Nk; ragged: an upper bound of every sequence's key length */
  int32_t head_dim;      /* D: 32, 64, 128 (F32); 32, 64, 96, 128, 192, 256 (F16, BF16); 128 (FP8_E4M3) */
  int32_t dtype;         /* attn_dtype_t: ATTN_F32, ATTN_F16 or ATTN_BF16, shared by Q, K, V, O;
                            or ATTN_FP8_E4M3 for Q, K, V with O in BF16 (dense batches) */
  int32_t causal;        /* 0/1. Bottom-right aligned: key j allowed for query i iff j <= i + (Nk - Nq) */
  int32_t window;        /* <= 0: off. W > 0 (requires causal): also j > i + (Nk - Nq) - W,
                            i.e. the W most recent keys, the diagonal included */
  float softmax_scale;   /* <= 0: 1/sqrt(D) computed in double and rounded once to float */
  float softcap;         /* <= 0: off. c > 0: s <- c * tanh(s / c) on the scaled score, before the mask */
  /* Strides in ELEMENTS for the [batch, head, token] dimensions of q, k, v, o
   * (head_dim is contiguous). Ragged batches ignore the batch stride: token t
   * of the packed [T, H, D] tensor is at t * stride[2] + h * stride[1]. */
  int64_t q_stride[3];
  int64_t k_stride[3];
  int64_t v_stride[3];
  int64_t o_stride[3];
  /* Ragged batches: both NULL (dense) or both set. Device int32 arrays of
   * length batch + 1, non-decreasing, starting at 0: sequence b owns query
   * tokens [cu_seqlens_q[b], cu_seqlens_q[b+1]) and key tokens
   * [cu_seqlens_k[b], cu_seqlens_k[b+1]); sequences are independent and the
   * mask offset is Nk_b - Nq_b. Every length must be <= seqlen_q / seqlen_k. */
  const int32_t *cu_seqlens_q;
  const int32_t *cu_seqlens_k;
  /* Attention sink: NULL (none) or a device float32 [Hq] of per query head logits
   * sigma_h (natural-log units). Each row's softmax denominator gains e^sigma_h, a
   * score with no value: O = sum_j e^{s_j} V_j / (e^sigma_h + sum_j e^{s_j}) and
   * LSE = ln(e^sigma_h + sum_j e^{s_j}); a row with no allowed key gets O = 0 and
   * LSE = sigma_h. ("attention-sink" in the masks of the feature surface named by
   * "Ask, Don't Equip", section 研究动机; the definition is the per-head sink logit.) */
  const float *sinks;
  /* FP8_E4M3 inputs only: one scale per tensor, value = code * scale (finite, > 0; ignored
   * for the other dtypes). Q and K's scales multiply the scores, V's the output.
   * (fp8 inputs: "Ask, Don't Equip", section 研究动机; the per-tensor scale is the
   * reading taken.) */
  float q_scale, k_scale, v_scale;
} attn_fwd_args_t;

/*
 * attn_fwd - fused attention forward (prefill).
 *
 *   q   [B, Hq, Nq, D] (or ragged [T, Hq, D]) in args->dtype
 *   k,v [B, Hkv, Nk, D] (or ragged [Tk, Hkv, D]) in args->dtype
 *   o   same layout as q (strides o_stride), written in args->dtype (BF16 for FP8_E4M3
 *       inputs; strides are in elements of each tensor's own type)
 *   lse nullable, float32, natural-log log-sum-exp of each row's final scores:
 *       dense [B, Hq, Nq] contiguous; ragged [Hq, T] contiguous.
 *       A row with no allowed key gets O = 0 and LSE = -inf.
 *
 * Accumulation is float32 throughout; Q K^T and P V run on the matrix cores
 * (bf16/f16 inputs: P is rounded to the input type before P V; fp8 inputs: P is
 * rounded to e4m3 and both products run on the fp8 matrix cores).
 */
attn_status_t attn_fwd(const attn_fwd_args_t *args, const void *q, const void *k, const void *v,
                       void *o, float *lse, void *stream);

/* ------------------------------------------------- chunked prefill (paged) ---- */

typedef struct {
  int32_t num_seqs;          /* S >= 1 */
  int32_t num_q_heads;       /* Hq */
  int32_t num_kv_heads;      /* Hkv, Hq % Hkv == 0 */
  int32_t head_dim;          /* D in {32, 64, 96, 128, 192, 256} */
  int32_t page_size;         /* tokens per page; must be 16 */
  int32_t max_pages_per_seq; /* row length of block_table */
  int32_t num_pages;         /* pages in each cache (rows of k_cache / v_cache) */
  int32_t max_seqlen_q;      /* host-known upper bound of every chunk's query count; sizes the grid */
  int32_t dtype;             /* ATTN_F16 or ATTN_BF16: Q, both caches and O */
  int32_t causal;            /* 0/1, bottom-right aligned as for attn_fwd */
  int32_t window;            /* as for attn_fwd (requires causal) */
  float softmax_scale;       /* <= 0: 1/sqrt(D) as for attn_fwd */
  float softcap;             /* as for attn_fwd */
  const float *sinks;        /* NULL or device float32 [Hq], as for attn_fwd */
} attn_fwd_paged_args_t;

/*
 * attn_fwd_paged - chunked prefill over a paged KV cache ("分块 prefill" over paged KV,
 * scenario axes of "Ask, Don't Equip: Question-Driven Coding Agents for Deep Kernel
 * Optimization", section 研究动机, which names the case without defining it). Reading
 * used: sequence s already holds seq_lens_k[s] = Nk_s keys in the cache, the last
 * Nq_s of them being the chunk's own tokens; its Nq_s queries are positions
 * Nk_s - Nq_s ... Nk_s - 1, so causal masking is bottom-right aligned (offset
 * Nk_s - Nq_s), exactly as a ragged attn_fwd over the gathered keys.
 *
 *   q            [T, Hq, D] contiguous (packed chunks), dtype
 *   k_cache,
 *   v_cache      [num_pages, page_size, Hkv, D] contiguous, dtype; token t of sequence s
 *                lives in page block_table[s * max_pages_per_seq + t / page_size], slot
 *                t % page_size (the decode layout)
 *   block_table  device int32 [S, max_pages_per_seq], entries in [0, num_pages)
 *   cu_seqlens_q device int32 [S + 1], non-decreasing from 0: chunk s owns query rows
 *                [cu_seqlens_q[s], cu_seqlens_q[s+1]), at most max_seqlen_q of them
 *   seq_lens_k   device int32 [S], 0 <= Nk_s <= max_pages_per_seq * page_size
 *   o            [T, Hq, D] contiguous, dtype
 *   lse          nullable float32 [Hq, T], natural log; a row with no allowed key
 *                gets O = 0 and LSE = -inf
 *   workspace    nullable device buffer, 256-byte aligned, of at least
 *                attn_fwd_paged_workspace_size(args) bytes when that size is non-zero.
 *                Given one (head_dim 128), the call first copies each sequence's pages
 *                of K and V into the workspace (one slot of max_pages_per_seq * page_size
 *                tokens per sequence) and then runs the ragged prefill kernel on the
 *                copy, the faster route; without one, a single kernel reads the pages
 *                in place. Both give the same mathematical result (rounding may differ).
 *
 * The kernels clamp page ids to [0, num_pages) and key counts to the table row, so
 * out-of-range device indices give wrong values, never an access outside the cache.
 */
attn_status_t attn_fwd_paged(const attn_fwd_paged_args_t *args, const void *q, const void *k_cache,
                             const void *v_cache, const int32_t *block_table,
                             const int32_t *cu_seqlens_q, const int32_t *seq_lens_k, void *o,
                             float *lse, void *workspace, size_t workspace_bytes, void *stream);

/* Bytes of workspace attn_fwd_paged can use for these args: 0 when there is no
 * gathered route for them (head_dim other than 128) or on bad args. */
size_t attn_fwd_paged_workspace_size(const attn_fwd_paged_args_t *args);

/* ---------------------------------------------------------------- backward ---- */

typedef struct {
  int32_t batch;         /* B >= 1 */
  int32_t num_q_heads;   /* Hq */
  int32_t num_kv_heads;  /* Hkv, Hq % Hkv == 0 */
  int32_t seqlen_q;      /* Nq >= 0 (0: nothing to do) */
  int32_t seqlen_k;      /* Nk >= 1 */
  int32_t head_dim;      /* D in {64, 128} */
  int32_t dtype;         /* ATTN_F16 or ATTN_BF16, every tensor but lse */
  int32_t causal;        /* as for attn_fwd */
  int32_t window;        /* as for attn_fwd */
  float softmax_scale;   /* as for attn_fwd */
  float softcap;         /* as for attn_fwd */
} attn_bwd_args_t;

/* Bytes of workspace attn_bwd needs (0 on bad args): two floats per query row, then room
 * for four float32 partial sums each of dK and dV (one per chunk of the queries; a call
 * uses one to four chunks), then one int32 per 128-key block and chunk for the order in
 * which that work runs. The size does not depend on causal, window or softcap. */
size_t attn_bwd_workspace_size(const attn_bwd_args_t *args);

/*
 * attn_bwd - gradients of attn_fwd (dense batches): given dL/dO, writes dL/dQ, dL/dK,
 * dL/dV. The backward pass is named as the next step by "Ask, Don't Equip" (section
 * 局限与改进) and not defined there; these are the derivatives of the forward definition:
 * with P rebuilt from the scores and the forward's LSE,
 *   dV = P^T dO, dP = dO V^T, dS = P (dP - rowsum(dO O)) * scale (times 1 - tanh^2 of
 *   the capped argument under a softcap), dQ = dS K, dK = dS^T Q,
 * and query heads that share a KV head add their dK and dV. A forward with a sink gives
 * an LSE that includes it, and the same formulas hold (the sink's own gradient is not
 * computed).
 *
 *   q, o, dout, dq  [B, Hq, Nq, D] contiguous, dtype (o and lse from attn_fwd)
 *   k, v, dk, dv    [B, Hkv, Nk, D] contiguous, dtype
 *   lse             float32 [B, Hq, Nq], natural log, as attn_fwd writes it
 *   workspace       device buffer of attn_bwd_workspace_size(args) bytes, 16-byte aligned
 * Accumulation is float32; P and dS are rounded to dtype for their products. dk and dv
 * are written whole (no accumulation into the caller's buffers); the results are repeatable
 * bit for bit.
 */
attn_status_t attn_bwd(const attn_bwd_args_t *args, const void *q, const void *k, const void *v, const void *o,
                       const void *dout, const float *lse, void *dq, void *dk, void *dv, void *workspace,
                       size_t workspace_bytes, void *stream);

/* ----------------------------------------------------------------- decode ---- */

typedef struct {
  int32_t num_seqs;          /* S >= 1 */
  int32_t num_q_heads;       /* Hq */
  int32_t num_kv_heads;      /* Hkv, Hq % Hkv == 0 (any group size: more than 16 query heads per
                                KV head take 16-head tiles in pairs); Hkv * ceil(Hq/Hkv / 16) <= 65535 */
  int32_t head_dim;          /* D == 128 */
  int32_t page_size;         /* tokens per page; must be 16 */
  int32_t max_pages_per_seq; /* row length of block_table */
  int32_t max_seq_len;       /* host-known upper bound of seq_lens[]; sizes the split grid */
  int32_t q_dtype;           /* ATTN_BF16 or ATTN_F16; O has q_dtype */
  int32_t kv_dtype;          /* ATTN_BF16, ATTN_F16 or ATTN_FP8_E4M3 */
  float softmax_scale;       /* <= 0: 1/sqrt(D) as for attn_fwd */
  int32_t num_splits;        /* 0: the library plans the split length; n > 0: split_len =
                                ceil(max_seq_len / n) rounded up to a whole page, capped at
                                4096 tokens (the longest split the kernel handles) */
  const float *sinks;        /* NULL or device float32 [Hq], as for attn_fwd */
} attn_decode_args_t;

/* Split plan: every sequence s is cut into ceil(seq_lens[s] / split_len)
 * pieces of split_len tokens (a multiple of page_size, at most 4096);
 * max_splits = ceil(max_seq_len / split_len). Deterministic function of the
 * args and, for fp8 KV with at most 16 query heads per KV head and an even
 * Hkv (one workgroup per split and sequence), of the current device's
 * compute-unit count (256 when no device is visible). */
attn_status_t attn_decode_plan(const attn_decode_args_t *args, int32_t *split_len,
                               int32_t *max_splits);

/* Bytes of workspace attn_decode_paged needs for these args (0 on bad args). */
size_t attn_decode_paged_workspace_size(const attn_decode_args_t *args);

/*
 * attn_decode_paged - one query token per sequence over a paged KV cache.
 *
 *   q            [S, Hq, D] contiguous, q_dtype
 *   k_cache,
 *   v_cache      [num_pages, page_size, Hkv, D] contiguous, kv_dtype. Token t of
 *                sequence s lives in page block_table[s * max_pages_per_seq + t / page_size],
 *                slot t % page_size.
 *   k_scale,
 *   v_scale      device float32 [Hkv], required iff kv_dtype == ATTN_FP8_E4M3, else NULL:
 *                the value of a stored code c of KV head g is c * scale[g]
 *   block_table  device int32 [S, max_pages_per_seq]
 *   seq_lens     device int32 [S], 1 <= seq_lens[s] <= max_seq_len; the query attends
 *                to all seq_lens[s] cached keys (the current token included)
 *   o            [S, Hq, D] contiguous, q_dtype
 *   lse          nullable float32 [S, Hq], natural log
 *   workspace    device buffer of at least attn_decode_paged_workspace_size(args) bytes,
 *                16-byte aligned; holds the per-split partial results
 */
attn_status_t attn_decode_paged(const attn_decode_args_t *args, const void *q, const void *k_cache,
                                const void *v_cache, const float *k_scale, const float *v_scale,
                                const int32_t *block_table, const int32_t *seq_lens, void *o,
                                float *lse, void *workspace, size_t workspace_bytes, void *stream);

/*
 * attn_decode_paged_noalloc - attn_decode_paged for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same arguments, results and kernels, without the workspace. The
 * per-split partial results go to a scratch array built into the library, one copy per
 * GPU, which the process holds until it ends; no call allocates or frees anything.
 *
 *   Limit: attn_decode_paged_workspace_size(args) must not exceed
 *          ATTN_DECODE_NOALLOC_MAX_WORKSPACE bytes (64 MiB); larger calls return
 *          ATTN_ERROR_WORKSPACE_TOO_SMALL and enqueue nothing. The 64-sequence,
 *          32768-token, Hq = 32 decode needs 34 MB.
 *   Sharing: every call on one GPU uses that GPU's one scratch array, so calls that can
 *          overlap on one GPU (on different streams, or from several host threads without
 *          ordering) race and may return wrong results. Calls on one stream are ordered
 *          and safe. The array keeps the last call's contents; nothing in it needs to
 *          start at zero (every partial a call reads is written by the same call).
 *   Set-up: the first call on a device looks up the array's address on that device
 *          (the device current at the call) and keeps it; a failure there returns
 *          ATTN_ERROR_LAUNCH_FAILED.
 */
#define ATTN_DECODE_NOALLOC_MAX_WORKSPACE ((size_t)64 << 20)
attn_status_t attn_decode_paged_noalloc(const attn_decode_args_t *args, const void *q, const void *k_cache,
                                        const void *v_cache, const float *k_scale, const float *v_scale,
                                        const int32_t *block_table, const int32_t *seq_lens, void *o,
                                        float *lse, void *stream);

/* ---------------------------------------------------------- measurement ---- */
/*
 * Probes for the two figures a roofline needs, measured on this machine rather than
 * taken from the specification (clocks are not locked): the roofline of the page
 * "Agent 帮我写 CUDA：一个 Softmax Attention 算子的开发全记录" (section 七: arithmetic
 * intensity against a ridge point = compute peak / memory bandwidth). Same conventions
 * as above: device pointers, enqueue only, host-side checks.
 *
 * attn_probe_mfma: `workgroups` workgroups of 4 waves (one per SIMD), each wave issuing
 *   32 * iters back-to-back v_mfma_f32_32x32x16_bf16 products in two independent chains
 *   (32768 FLOP each: FLOPs = workgroups * 4 * 32 * iters * 32768).
 *   operands   device uint32 [256 * 8]: thread t takes its A operand bits from
 *              operands[8t .. 8t+3] and its B operand bits from [8t+4 .. 8t+7] (the power
 *              the matrix cores draw, and so the clock they hold, depends on these bits)
 *   valu_mix   0: products only; 1: beside each product the vector work of the attention
 *              loop (one exp2, one fp32 add, half a pack to bf16)
 *   clocks     device uint64 [2 * workgroups]: per workgroup, the shader-clock cycles and
 *              the 100 MHz reference ticks its first wave spent in the product loop
 *   sink       device float [256 * workgroups], written (keeps the products live)
 *
 * attn_probe_hbm_read: `workgroups` workgroups stream `bytes` of `buf` (workgroup w reads
 *   the w-th contiguous slice) with 16-byte nontemporal loads and write one uint32 each to
 *   sink [workgroups]. bytes must be a non-zero multiple of 32768 * workgroups.
 *
 * attn_flush_caches: writes zeros over `bytes` of `buf` (16-byte aligned, a multiple of 16),
 *   so that with bytes above the last-level cache size (L2 4 MiB per XCD, 256 MiB
 *   Infinity Cache on MI355X) a following launch starts with cold caches.
 */
attn_status_t attn_probe_mfma(const uint32_t *operands, int32_t workgroups, int32_t iters, int32_t valu_mix,
                              uint64_t *clocks, float *sink, void *stream);
attn_status_t attn_probe_hbm_read(const void *buf, size_t bytes, int32_t workgroups, uint32_t *sink,
                                  void *stream);
attn_status_t attn_flush_caches(void *buf, size_t bytes, void *stream);

/* ------------------------------------------------------------------ misc ---- */

const char *attn_status_string(attn_status_t status);
const char *attn_last_error_message(void);
/* Library ABI version (major * 100 + minor). */
int32_t attn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_H_ */
