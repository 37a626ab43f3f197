/*
 * exact_attn.h — C ABI of the exact, IO-aware attention forward library for
 * AMD Instinct MI355X (gfx950).
 *
 * The operation is softmax attention, O = softmax(scale * Q K^T + mask) V, as
 * defined on the "Attention Is the Bottleneck" page (samanvya.dev), section
 * "What attention costs".  It is evaluated tile by tile with an online
 * softmax (a running row maximum and row sum, with the partial output
 * rescaled whenever the maximum grows), as that page describes in
 * "FlashAttention: same math, different IO", so no N x N score matrix is ever
 * written to device memory.  The result equals the plain definition up to
 * floating-point rounding order.
 *
 * Conventions for every entry point
 *   - All tensor pointers are DEVICE pointers owned by the caller.  The
 *     library allocates nothing and keeps no per-call state.
 *   - Work is enqueued asynchronously on `stream` (0 = the null stream); no
 *     entry point synchronises the host.
 *   - Arguments are checked before any HIP call; a failing check returns an
 *     error status and enqueues nothing.  The contents of device-resident
 *     index arrays (document offsets, block tables, sequence lengths) are a
 *     caller contract and are not checked.
 *   - Tensors are dense and row-major with the head dimension fastest, and
 *     every base pointer must be 16-byte aligned.
 *   - Return value: an attn_status.  attn_status_string() turns it into
 *     text; for ATTN_ERR_HIP it also reports the HIP error of the failing
 *     launch on the calling thread.
 */
#ifndef EXACT_ATTN_H
#define EXACT_ATTN_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    ATTN_OK = 0,
    ATTN_ERR_INVALID_ARGUMENT = 1,    /* null pointer, negative size, bad mask field ... */
    ATTN_ERR_UNSUPPORTED = 2,         /* valid request the library does not implement (e.g. d) */
    ATTN_ERR_WORKSPACE_TOO_SMALL = 3, /* decode workspace below attn_paged_decode_workspace_size */
    ATTN_ERR_HIP = 4                  /* a HIP launch failed; see attn_status_string */
} attn_status;

typedef enum { ATTN_DTYPE_F32 = 0, ATTN_DTYPE_BF16 = 1 } attn_dtype;

/*
 * Masks.  Query row i of a sequence stands at key position pos = i + (Nk - Nq)
 * (bottom-right alignment, so a single decoding query sees its whole cache).
 *   NONE            every key is visible.
 *   CAUSAL          key j is visible iff j <= pos ("Attention and matrix
 *                   kernels" page, How it works: causal masks).
 *   SLIDING_WINDOW  key j is visible iff 0 <= pos - j < window, i.e. the
 *                   `window` latest positions including the query's own
 *                   ("Attention Is the Bottleneck", Sliding windows and
 *                   local:global layers).  window >= 1.
 *   DOCUMENT        causal inside packed documents: key j is visible iff
 *                   j <= pos and j lies in the same document as pos
 *                   ("Attention and matrix kernels", document masks).
 *                   doc_offsets is a DEVICE int32 array of num_docs + 1
 *                   strictly increasing entries, doc_offsets[0] = 0 and
 *                   doc_offsets[num_docs] = Nk; document t holds key
 *                   positions [doc_offsets[t], doc_offsets[t+1]).  The same
 *                   offsets apply to every batch element.
 * A query row that sees no key gets O = 0 and LSE = -inf.
 *
 * Sinks ("Attention Is the Bottleneck", Sliding windows and local:global
 * layers), two optional extensions:
 *   sink_tokens     SLIDING_WINDOW only (0 elsewhere): keys 0 .. sink_tokens-1
 *                   stay visible to every query at or past them, besides the
 *                   window (StreamingLLM's sink tokens).  >= 0.
 *   sink_logits     NULL, or a DEVICE float32 array of Hq entries, 4-byte
 *                   aligned: a learned sink per query head (as in gpt-oss).
 *                   Each row's softmax gets one more entry with that logit
 *                   (on the scale of scale * q.k, natural units) and a zero
 *                   value: O = sum_j e^{s_j} v_j / (sum_j e^{s_j} + e^{sink}),
 *                   LSE = ln(sum_j e^{s_j} + e^{sink}); a row that sees no key
 *                   gets O = 0 and LSE = sink.
 *
 * Score modifications ("Attention and matrix kernels", How it works: the
 * FlexAttention entry names score modifications as one family of variants;
 * the page names none in particular, and these two are the menu this library
 * offers).  Both act on s = scale * q.k before the mask, in this order:
 *   softcap         > 0: s becomes softcap * tanh(s / softcap), which bounds
 *                   every score by softcap.  0: off.  Finite, >= 0.
 *   alibi_slopes    NULL, or a DEVICE float32 array of Hq entries, 4-byte
 *                   aligned: s gets slope[h] * (j - pos) added, a linear
 *                   penalty on the distance from the query's position pos to
 *                   key j (pos = i + Nk - Nq, as for the causal mask).
 * Supported by attn_fwd (both dtypes), attn_paged_prefill, attn_paged_decode
 * (as two arguments of its own) and attn_bwd (which differentiates through
 * both: the cap contributes 1 - tanh^2 to dS).  Sink logits are not modified.
 */
typedef enum {
    ATTN_MASK_NONE = 0,
    ATTN_MASK_CAUSAL = 1,
    ATTN_MASK_SLIDING_WINDOW = 2,
    ATTN_MASK_DOCUMENT = 3
} attn_mask_kind;

typedef struct {
    int32_t kind;               /* an attn_mask_kind */
    int32_t window;             /* SLIDING_WINDOW only: W >= 1 */
    const int32_t* doc_offsets; /* DOCUMENT only: device pointer, num_docs + 1 entries */
    int32_t num_docs;           /* DOCUMENT only: >= 1 */
    int32_t sink_tokens;        /* SLIDING_WINDOW only: sink tokens kept visible, >= 0 */
    const float* sink_logits;   /* NULL or device [Hq]: learned sink logit per query head */
    float softcap;              /* > 0: scores become softcap * tanh(score / softcap); 0: off */
    const float* alibi_slopes;  /* NULL or device [Hq]: score += slope * (key - query position) */
    int32_t soft_exp2;          /* attn_fwd only, a performance option: 0 (the default) takes every
                                   softmax weight's 2^x from the hardware exponential; 2 or 4 take
                                   that many of each lane's 8 weights per 16-key block (a quarter
                                   or half) from a software 2^x on the FMA units instead (see
                                   below).  The other entry points ignore it. */
} attn_mask;

/*
 * attn_fwd — attention forward for a batch of prompts (prefill).
 *
 *   q    [B, Hq,  Nq, d]  dtype          read only
 *   k    [B, Hkv, Nk, d]  dtype          read only
 *   v    [B, Hkv, Nk, d]  dtype          read only
 *   o    [B, Hq,  Nq, d]  dtype          written in full
 *   lse  [B, Hq,  Nq]     float32        natural-log log-sum-exp of each row's
 *                                        scaled visible scores (the saved
 *                                        softmax statistic the "Attention Is
 *                                        the Bottleneck" page names for the
 *                                        backward pass); may be NULL.
 *
 * Grouped-query heads (MQA and GQA section of the same page): Hq must be a
 * multiple of Hkv and query head h reads KV head h / (Hq / Hkv).
 * `scale` multiplies Q K^T before the mask; pass 1/sqrt(d) for the usual
 * attention.  d must be 64 or 128.  Sizes of 0 are accepted and enqueue
 * nothing.  bf16 inputs produce a bf16 output rounded to nearest-even; the
 * softmax statistics and accumulators are float32 in both dtypes.
 */
int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
             int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale,
             attn_mask mask, int dtype, hipStream_t stream);
/*
 * mask.soft_exp2 (FlashAttention-4's software exponential, "Attention Is the
 * Bottleneck", FlashAttention-4 section): 2^x as 2^rint(x) times a degree-4
 * polynomial of the remainder, relative error at most 2.7e-6.  Supported for
 * bf16, d = 128 and no score modifications (ATTN_ERR_UNSUPPORTED otherwise);
 * values other than 0, 2 and 4 are ATTN_ERR_INVALID_ARGUMENT.  On MI355X it is
 * measured 8-17 % slower than the hardware exponential, which is why 0 is the
 * default.
 */

/*
 * attn_paged_decode_workspace_size — bytes of scratch device memory that
 * attn_paged_decode needs for these sizes (the per-split partial outputs and
 * log-sum-exps that its combine pass merges).  Returns 0 for invalid sizes.
 */
size_t attn_paged_decode_workspace_size(int num_seqs, int Hq, int d, int max_seq_len);

/*
 * attn_paged_decode — one new token per sequence attends to that sequence's
 * paged KV cache (paged-attention kernels, "Attention and matrix kernels"
 * page; Paging and prefix sharing, "Attention Is the Bottleneck").  The KV
 * sequence of each (sequence, KV head) is split into chunks that are
 * attended in parallel and then merged with a log-sum-exp combine
 * (Flash-Decoding section of the same page).
 *
 *   q            [num_seqs, Hq, d]                       bf16, read only
 *   k_pages      [num_pages, Hkv, page_size, d]          bf16, read only
 *   v_pages      [num_pages, Hkv, page_size, d]          bf16, read only
 *   block_table  [num_seqs, max_pages_per_seq]           int32; entry p of a
 *                sequence is the physical page holding its tokens
 *                [p*page_size, (p+1)*page_size)
 *   seq_lens     [num_seqs]                              int32, 0 <= len <= max_seq_len
 *   o            [num_seqs, Hq, d]                       bf16, written in full
 *   lse          [num_seqs, Hq]                          float32 natural-log LSE; may be NULL
 *   sink_logits  NULL or device float32 [Hq]: learned sink per query head
 *                (see the sinks paragraph above the mask struct)
 *   softcap,     the score modifications, as in attn_mask (0 / NULL: off);
 *   alibi_slopes the query's position is seq_len - 1
 *   workspace    device scratch of at least
 *                attn_paged_decode_workspace_size(num_seqs, Hq, d, max_seq_len)
 *                bytes, 16-byte aligned; its contents on entry do not matter.
 *
 * The query is the newest token, so it sees all seq_len cached keys.  Page
 * slots past seq_len are never read into the result (they may hold any bit
 * pattern, NaN included).  A sequence with seq_len = 0 gets O = 0 and
 * LSE = -inf.  page_size must be 16, d must be 128 or 64, Hq a multiple of
 * Hkv, max_pages_per_seq * page_size >= max_seq_len.  A seq_lens entry
 * outside [0, max_seq_len] breaks the caller contract; the kernels clamp it
 * to that range, so nothing is read outside the block-table row or the
 * workspace (the result is then that of the clamped length).  The workspace
 * must not be shared by calls that may run concurrently.
 */
int attn_paged_decode(const void* q, const void* k_pages, const void* v_pages,
                      const int32_t* block_table, const int32_t* seq_lens,
                      void* o, float* lse,
                      int num_seqs, int Hq, int Hkv, int d, int page_size,
                      int max_pages_per_seq, int max_seq_len, float scale, const float* sink_logits,
                      float softcap, const float* alibi_slopes,
                      void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * attn_paged_decode_noalloc — attn_paged_decode for callers that cannot
 * allocate device memory or bring a workspace: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc.  Same arguments and
 * result as attn_paged_decode (same kernels), minus the workspace: the
 * partials go to a device array of ATTN_NOALLOC_SCRATCH_BYTES that the
 * library holds on each GPU it runs on until the process ends.  The call
 * allocates nothing; its first call on a device looks up that device's
 * array address once.
 *
 * Limit: attn_paged_decode_workspace_size(num_seqs, Hq, d, max_seq_len) must
 * not exceed ATTN_NOALLOC_SCRATCH_BYTES (64 MiB: e.g. 64 sequences x 32
 * query heads x 32K keys at d = 128 need 33.8 MB), else
 * ATTN_ERR_WORKSPACE_TOO_SMALL and nothing runs.  Every call on one GPU uses
 * the same array: calls that may overlap on one GPU (other streams, other
 * threads) race and must be ordered by the caller.  The array needs no
 * clearing between calls (each call writes every partial it reads).
 */
#define ATTN_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int attn_paged_decode_noalloc(const void* q, const void* k_pages, const void* v_pages,
                              const int32_t* block_table, const int32_t* seq_lens,
                              void* o, float* lse,
                              int num_seqs, int Hq, int Hkv, int d, int page_size,
                              int max_pages_per_seq, int max_seq_len, float scale, const float* sink_logits,
                              float softcap, const float* alibi_slopes, hipStream_t stream);

/*
 * attn_paged_prefill — chunked prefill over the paged KV cache: each
 * sequence appends a chunk of new tokens and those tokens attend to the
 * sequence's whole cache, read through its block table.  This is the serving
 * pattern that pairs a tiled attention kernel with KV paging (the
 * FlashAttention serving-value question page, Real-world examples; paged
 * kernels on the "Attention and matrix kernels" page).
 *
 *   q            [total_q, Hq, d]                        bf16, read only;
 *                token-major: row t is token t of the concatenated chunks
 *   k_pages      [num_pages, Hkv, page_size, d]          bf16, read only
 *   v_pages      [num_pages, Hkv, page_size, d]          bf16, read only
 *   block_table  [num_seqs, max_pages_per_seq]           int32 (as for decode)
 *   seq_lens     [num_seqs]                              int32: cached tokens of
 *                each sequence, the chunk's own tokens included
 *   q_offsets    [num_seqs + 1]                          int32, nondecreasing,
 *                q_offsets[0] = 0: chunk s is rows q_offsets[s] .. q_offsets[s+1]-1
 *   o            [total_q, Hq, d]                        bf16, written in full
 *   lse          [total_q, Hq]                           float32 natural-log LSE; may be NULL
 *
 * Query i of chunk s (Nq_s = q_offsets[s+1] - q_offsets[s] tokens) stands at
 * key position i + seq_lens[s] - Nq_s, the bottom-right alignment of the mask
 * definitions above; mask NONE, CAUSAL or SLIDING_WINDOW applies within each
 * sequence (DOCUMENT returns ATTN_ERR_UNSUPPORTED).  Page slots past seq_len
 * are never read into the result (any bit pattern, NaN included).  Rows with
 * no visible key (a chunk longer than its cache, seq_len = 0) get O = 0 and
 * LSE = -inf.  Caller contract (not checked, like all device-resident index
 * data): Nq_s <= max_q_len, seq_lens[s] <= max_seq_len <= max_pages_per_seq *
 * page_size.  A seq_lens entry outside [0, max_seq_len] is clamped to that
 * range, so the block-table reads stay inside the sequence's row; rows of a
 * chunk past max_q_len are not written.  page_size must be 16, d 128 or 64,
 * Hq a multiple of Hkv.
 */
int attn_paged_prefill(const void* q, const void* k_pages, const void* v_pages,
                       const int32_t* block_table, const int32_t* seq_lens, const int32_t* q_offsets,
                       void* o, float* lse,
                       int num_seqs, int Hq, int Hkv, int d, int page_size,
                       int max_pages_per_seq, int max_seq_len, int max_q_len, float scale,
                       attn_mask mask, hipStream_t stream);

/*
 * attn_bwd_workspace_size — bytes of scratch device memory attn_bwd needs
 * (four per-row statistics of 4 bytes).  Returns 0 for invalid sizes.
 */
size_t attn_bwd_workspace_size(int B, int Hq, int Nq);

/*
 * attn_bwd — gradients of attn_fwd by recomputation from its saved
 * statistic: the forward keeps only O and the per-row LSE, and the backward
 * recomputes the probabilities tile by tile ("Attention Is the Bottleneck",
 * FlashAttention-2 section).  With P = exp(scale Q K^T + mask - LSE),
 * D = rowsum(dO o O) and dS = P o (dO V^T - D):
 *   dq = scale dS K,  dk = scale dS^T Q,  dv = P^T dO,
 * dk and dv summed over the query heads of each KV head's group, and, with
 * learned sink logits, dsink[h] = -sum over rows of P_sink D.
 *
 *   q, o, dout   [B, Hq, Nq, d]   bf16, read only (o and lse from attn_fwd
 *                                 with the same arguments)
 *   k, v         [B, Hkv, Nk, d]  bf16, read only
 *   lse          [B, Hq, Nq]      float32, read only
 *   dq           [B, Hq, Nq, d]   bf16, written in full
 *   dk, dv       [B, Hkv, Nk, d]  bf16, written in full (0 for keys no row sees)
 *   dsink        NULL or [Hq] float32, written when mask.sink_logits is given
 *   workspace    device scratch of at least attn_bwd_workspace_size(B, Hq, Nq)
 *                bytes, 16-byte aligned; not to be shared by concurrent calls
 *
 * Every mask kind and both sink forms apply as in attn_fwd.  This build
 * supports d = 64 or 128 (else ATTN_ERR_UNSUPPORTED) with dtype BF16 (the fast
 * path) or F32 (a full-precision checking path; every tensor above that is
 * "bf16" is then float32, gradients included).
 */
int attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
             const float* lse, void* dq, void* dk, void* dv, float* dsink,
             int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale, attn_mask mask, int dtype,
             void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Text for a status code (static storage; for ATTN_ERR_HIP, thread-local). */
const char* attn_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* EXACT_ATTN_H */
