/*
 * attn.h - C ABI of the MI355X (gfx950) fused softmax-attention library.
 *
 * Operation (all entry points):
 *     O = softmax(scale * Q K^T + mask) V,   LSE_i = ln sum_j exp(scale * q_i . k_j)
 * computed in one fused pass per query tile: the streaming softmax state
 * (running max m, running sum l, accumulator acc) is a monoid, so key blocks
 * and split-KV partials may be folded in any grouping.  Source: the page
 * "Não escreva kernels, derive-os", section "Aprofundamento", first paragraph
 * (flash attention from the online softmax seen as a monoid) and FAQ entry
 * "O que o Tang propõe de diferente?" (fusion, flash attention and the
 * backward obtained by rewriting); the page "Tang Project Derives GPU Kernels
 * via IR ...", section "Details" (monoid reductions; causal forward passes;
 * decode at 16-48 concurrent streams).  The pages print no formula: the
 * definition above is the textbook softmax attention.
 *
 * Conventions shared by every entry point
 *   Layout   q, o, dout, dq : [B, Hq,  Nq, d]  contiguous, d fastest
 *            k, v, dk, dv   : [B, Hkv, Nk, d]  contiguous, d fastest
 *            lse            : [B, Hq,  Nq]     fp32, natural log
 *   Heads    query head h reads kv head h / (Hq / Hkv)  (grouped-query)
 *   Causal   key j is visible to query i iff j <= i + (Nk - Nq)
 *            (bottom-right alignment; a single decode query sees every key)
 *   Empty    a query row with no visible key gets O = 0, LSE = -inf and
 *            zero gradients
 *   Types    dtype selects the element type of q, k, v, o and dout;
 *            accumulation is fp32; lse and all gradients are fp32
 *   Sizes    d must be 64 or 128; Hq % Hkv == 0; B, Nq, Nk >= 0; scale > 0
 *            and finite; Nq, Nk <= ATTN_MAX_SEQ; B * Hq <= 2^20 and
 *            B * Hq * ceil(Nq / 32) < 2^31, for attn_bwd also
 *            B * Hkv * ceil(Nk / 32) < 2^31 (the launch grids' 32-bit
 *            workgroup counts)
 *   Memory   every pointer is a device pointer owned by the caller; the
 *            library never allocates, frees or synchronises.  Inputs are
 *            read only; outputs are fully overwritten.  Workspaces are
 *            caller-provided scratch sized by the *_workspace_bytes calls.
 *   Streams  stream is a hipStream_t (NULL = the default stream); each call
 *            enqueues its kernels on it and returns without waiting.
 *   Errors   every argument check runs on the host before any HIP call and
 *            returns a status; a failed launch returns ATTN_ERR_HIP.  Device
 *            faults surface at the caller's next synchronisation.  NaN or
 *            Inf inputs propagate and are not checked.  A call whose outputs
 *            are empty (B, Hq or Nq zero) returns ATTN_OK and launches nothing.
 */
#ifndef ATTN_MI355X_H
#define ATTN_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Longest sequence (Nq, Nk, packed totals): one head's rows of q, k or v
 * then span at most 2^22 * 128 * 2 bytes = 1 GiB, so the kernels' 32-bit
 * buffer offsets never overflow. */
#define ATTN_MAX_SEQ (1 << 22)

typedef enum {
  ATTN_OK = 0,
  ATTN_ERR_INVALID = 1,     /* null pointer, negative size, Hq % Hkv != 0, bad scale or dtype */
  ATTN_ERR_UNSUPPORTED = 2, /* valid but not built: d not in {64,128}, size above the limits, dtype */
  ATTN_ERR_WORKSPACE = 3,   /* workspace pointer missing or smaller than required */
  ATTN_ERR_HIP = 4,         /* a kernel launch failed */
  ATTN_ERR_SCRATCH = 5      /* the allocation-free decode needs more than ATTN_DECODE_SCRATCH_BYTES */
} attn_status;

typedef enum { ATTN_F32 = 0, ATTN_BF16 = 1 } attn_dtype;

/*
 * Forward prefill.  q [B,Hq,Nq,d], k/v [B,Hkv,Nk,d] -> o [B,Hq,Nq,d] (dtype),
 * lse [B,Hq,Nq] fp32 (may be NULL when not needed).  dtype ATTN_BF16 runs the
 * contractions on bf16 MFMA; ATTN_F32 on fp32 MFMA.  Causal key blocks that
 * no query of a tile can see are neither loaded nor computed.
 *   Source   "Não escreva kernels, derive-os", section "Aprofundamento",
 *            first paragraph: flash attention as a fusion obtained once the
 *            streaming softmax is seen as a reduction under a monoid; the
 *            key tiles of a query tile are folded left to right in that
 *            monoid, in one pass.  "Tang Project Derives GPU Kernels via IR
 *            ...", section "Details": causal forward passes and the 44k-token
 *            prefill.
 *   Sizes    ATTN_F32 is a correctness path (one wave per workgroup, no
 *            pipelining): use it for small problems; ATTN_BF16 is the
 *            throughput path.
 */
attn_status attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t Hq,
                     int64_t Hkv, int64_t Nq, int64_t Nk, int64_t d, float scale, int causal, attn_dtype dtype,
                     void* stream);

/*
 * Forward prefill over a packed batch of variable-length sequences, and
 * chunked prefill of new tokens against a KV history (the engine setting of
 * the page "Tang Project Derives GPU Kernels via IR ...", section "Details":
 * long prefills and many concurrent streams of unequal length).  Sequence s
 * owns query rows [cu_seqlens_q[s], cu_seqlens_q[s+1]) and key rows
 * [cu_seqlens_k[s], cu_seqlens_k[s+1]); its queries attend to its own keys
 * only, with the causal rule above applied per sequence (Lk_s - Lq_s is the
 * length of its history).
 *   Layout   q, o : [Hq, total_q, d];  k, v : [Hkv, total_k, d];
 *            lse  : [Hq, total_q] fp32 (may be NULL)
 *   Offsets  cu_seqlens_q / cu_seqlens_k: device int32 arrays of n_seqs + 1
 *            non-decreasing entries from 0 to total_q / total_k.  They are
 *            read on the device only (the host never waits for them);
 *            entries outside [0, total] are clamped, so no access leaves the
 *            tensors.
 *   Grid     max_seqlen_q must be at least every sequence's query length:
 *            query rows past it are not written.
 *   Types    ATTN_BF16 only (ATTN_F32 returns ATTN_ERR_UNSUPPORTED).
 *   Sizes    n_seqs >= 0; total_q, total_k, max_seqlen_q <= ATTN_MAX_SEQ;
 *            the other rules above.
 */
attn_status attn_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                            const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int64_t n_seqs,
                            int64_t total_q, int64_t total_k, int64_t max_seqlen_q, int64_t Hq, int64_t Hkv,
                            int64_t d, float scale, int causal, attn_dtype dtype, void* stream);

/*
 * Packed variable-length forward over a paged K/V cache: attn_fwd_varlen's
 * queries (q, o packed [Hq, total_q, d]; lse [Hq, total_q], may be NULL;
 * cu_seqlens_q as there) against keys held in pages as serving engines keep
 * their cache, e.g. a chunked prefill whose new tokens' K and V have been
 * appended to the cache.  "Tang Project Derives GPU Kernels via IR ..."
 * (section "Details") measures the engine on a long prefill and on decode at
 * many concurrent streams of unequal length.
 *   Cache    k_cache, v_cache: bf16 [num_pages, Hkv, page_size, d];
 *            page_size a multiple of 64 (ATTN_ERR_UNSUPPORTED otherwise).
 *   Table    block_table: device int32 [n_seqs, max_pages]; key j of
 *            sequence s is slot j % page_size of page block_table[s *
 *            max_pages + j / page_size]; page ids outside [0, num_pages) are
 *            clamped into it (no access leaves the cache).
 *   Keys     seq_lens_k: device int32 [n_seqs], clamped to [0,
 *            min(max_seqlen_k, max_pages * page_size)]; keys past a
 *            sequence's length are never read.  Causal is bottom-right per
 *            sequence, as in attn_fwd_varlen.
 *   Sizes    max_seqlen_q must be at least every sequence's query length;
 *            max_seqlen_k at least every seq_lens_k entry; max_pages *
 *            page_size <= ATTN_MAX_SEQ; ATTN_BF16 only.
 */
attn_status attn_fwd_varlen_paged(const void* q, const void* k_cache, const void* v_cache, const int32_t* block_table,
                                  void* o, float* lse, const int32_t* cu_seqlens_q, const int32_t* seq_lens_k,
                                  int64_t n_seqs, int64_t total_q, int64_t max_seqlen_q, int64_t max_seqlen_k,
                                  int64_t Hq, int64_t Hkv, int64_t d, int64_t num_pages, int64_t page_size,
                                  int64_t max_pages, float scale, int causal, void* stream);

/*
 * Split-KV decode: one query token per stream (Nq must be 1) against a KV
 * history of Nk keys.  Each kv head's keys are cut into num_splits chunks
 * (0 = automatic plan); every chunk yields a partial state (m, l, acc) for the
 * Hq/Hkv query heads that share the kv head, written to the workspace, and a
 * merge kernel folds the partials with the monoid rule and writes o (dtype)
 * and lse (fp32, may be NULL).  With one chunk the single kernel writes o and
 * lse and no workspace is used.  Only ATTN_BF16 is built.  causal is accepted
 * and has no effect (a single bottom-right-aligned query sees every key).
 * attn_decode_num_splits returns the automatic plan: the power of two (1 to
 * 64) that minimises a cost model of the decode (per-workgroup streaming rate,
 * whole-device HBM rate, cost of each extra chunk and of the merge launch),
 * so a chunk per (stream, kv head) from about 160 (stream, kv head) pairs up.
 * attn_decode_workspace_bytes(..., num_splits) is enough for this entry point,
 * for attn_decode_splitkv_fp8 (whose plan models the FP8 kernel) and for
 * attn_decode_paged (Nk = its max_seq_len) at the same num_splits.
 *   Source   the merge is the online-softmax monoid of "Não escreva kernels,
 *            derive-os" (section "Aprofundamento", first paragraph): any
 *            grouping of the chunks gives the same state up to rounding.
 *            "Tang Project Derives GPU Kernels via IR ..." (section
 *            "Details") measures decode at 16-48 concurrent streams and ties
 *            an accuracy miss to the split granularity.
 *   Workspace [B, Hq, S, d] fp32 accumulators then [B, Hq, S, 2] fp32
 *            (m in log2 units, l), each 256-byte aligned; owned by the
 *            caller, not read across calls; NULL is accepted when the plan
 *            has one chunk (attn_decode_workspace_bytes returns 0).
 */
int attn_decode_num_splits(int64_t B, int64_t Hq, int64_t Hkv, int64_t Nk, int64_t d);
size_t attn_decode_workspace_bytes(int64_t B, int64_t Hq, int64_t Hkv, int64_t Nk, int64_t d, int num_splits);
attn_status attn_decode_splitkv(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B,
                                int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t d, float scale, int causal,
                                int num_splits, void* workspace, size_t workspace_bytes, attn_dtype dtype,
                                void* stream);

/*
 * attn_decode_splitkv for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same arguments without the workspace, the same kernels,
 * split plan and bits.  The partial states live in a fixed device array of
 * ATTN_DECODE_SCRATCH_BYTES that the library holds on each GPU it runs on
 * until the process ends; the call allocates and frees nothing.  A plan
 * whose partial states exceed it (attn_decode_noalloc_scratch_bytes, the same
 * as attn_decode_workspace_bytes of the bf16 plan) returns ATTN_ERR_SCRATCH
 * before any HIP call.  Every call on one GPU shares its array, so calls
 * that overlap on one GPU race: order them on one stream (or wait between
 * streams).  Nothing in the array needs to start at zero.
 */
#define ATTN_DECODE_SCRATCH_BYTES ((size_t)8 << 20)
size_t attn_decode_noalloc_scratch_bytes(int64_t B, int64_t Hq, int64_t Hkv, int64_t Nk, int64_t d, int num_splits);
attn_status attn_decode_splitkv_noalloc(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B,
                                        int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t d, float scale,
                                        int causal, int num_splits, attn_dtype dtype, void* stream);

/*
 * Split-KV decode in one launch.  Same arguments, rules and result as
 * attn_decode_splitkv for the same num_splits (the same kernels and the same
 * fold, so the same bits), but no merge kernel: each chunk's workgroup publishes its partial state
 * and counts itself in for its (stream, kv head) with a device atomic, and
 * the last one to arrive folds every chunk's state and writes o and lse.
 * It folds the chunks in index order whichever finishes last, so the result
 * does not depend on timing.  The fold is the online-softmax monoid of "Não
 * escreva kernels, derive-os" (section "Aprofundamento"); "Tang Project
 * Derives GPU Kernels via IR ..." (section "Details") ties decode accuracy to
 * the split granularity.
 *   Workspace attn_decode_fused_workspace_bytes bytes (0 when the plan has
 *             one chunk: then no workspace is read), 4-byte aligned
 *             (ATTN_ERR_INVALID otherwise).  Its first 64 KiB hold the
 *             arrival counts, one per (stream, kv head), so B * Hkv <= 16384
 *             when the plan has more than one chunk (ATTN_ERR_UNSUPPORTED
 *             otherwise); the partial states follow.  The counts must be zero
 *             before the first call on that memory (allocate it zeroed);
 *             every call that completes leaves them zero, so the workspace
 *             serves later calls of any size that fits.  Calls that share a
 *             workspace must not run concurrently (stream order suffices),
 *             and memory used by another entry point must be zeroed again
 *             before it serves this one.
 */
/* The automatic plan of this entry point: attn_decode_num_splits's model
 * without the merge launch, so it may split where the two-launch path does not. */
int attn_decode_fused_num_splits(int64_t B, int64_t Hq, int64_t Hkv, int64_t Nk, int64_t d);
size_t attn_decode_fused_workspace_bytes(int64_t B, int64_t Hq, int64_t Hkv, int64_t Nk, int64_t d, int num_splits);
attn_status attn_decode_splitkv_fused(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B,
                                      int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t d, float scale,
                                      int causal, int num_splits, void* workspace, size_t workspace_bytes,
                                      attn_dtype dtype, void* stream);

/*
 * Split-KV decode over a paged KV cache, each stream with its own length.
 * The decode of attn_decode_splitkv (one query token per stream, all of the
 * stream's keys visible), with the cache held in pages as serving engines
 * keep it: the second page ("Tang Project Derives GPU Kernels via IR ...",
 * section "Details") measures decode over 16-48 concurrent streams.
 *   Cache    k_cache, v_cache: bf16 [num_pages, Hkv, page_size, d]; a page
 *            holds page_size consecutive keys of every kv head.  page_size
 *            must be a multiple of 32 (ATTN_ERR_UNSUPPORTED otherwise).
 *   Table    block_table: device int32 [B, max_pages]; key j of stream b is
 *            slot j % page_size of page block_table[b * max_pages + j /
 *            page_size].  Page ids outside [0, num_pages) are clamped into
 *            it, so no access leaves the cache (the result is then wrong).
 *   Lengths  seq_lens: device int32 [B]; stream b has seq_lens[b] keys,
 *            clamped to [0, min(max_seq_len, max_pages * page_size)].  Keys
 *            past a stream's length are never read, so unused slots and
 *            pages may hold anything.  max_seq_len (host) must be at least
 *            every seq_lens entry; it sizes the split plan and the
 *            workspace, attn_decode_workspace_bytes(B, Hq, Hkv, max_seq_len,
 *            d, num_splits), which also covers this entry point's
 *            automatic plan: attn_decode_splitkv's, raised to chunks of at
 *            most 4096 keys and, with fewer (stream, kv head) pairs than
 *            the 256 CUs, to enough chunks of at least 1024 keys to give
 *            each CU one.  The (stream, chunk) items start longest first
 *            (ordered on the device from seq_lens), so unequal lengths need
 *            no further split.  A stream with no keys gets O = 0, LSE = -inf.
 *   Other    q, o bf16 [B, Hq, 1, d]; lse fp32 [B, Hq] (may be NULL);
 *            max_pages * page_size <= ATTN_MAX_SEQ; every other rule as
 *            attn_decode_splitkv.
 */
attn_status attn_decode_paged(const void* q, const void* k_cache, const void* v_cache, const int32_t* block_table,
                              const int32_t* seq_lens, void* o, float* lse, int64_t B, int64_t Hq, int64_t Hkv,
                              int64_t d, int64_t num_pages, int64_t page_size, int64_t max_pages,
                              int64_t max_seq_len, float scale, int num_splits, void* workspace,
                              size_t workspace_bytes, void* stream);

/*
 * The paged decode in one launch: attn_decode_paged's arguments, rules and
 * result for the same num_splits (the same kernel and fold, so the same
 * bits), with the chunks merged as attn_decode_splitkv_fused merges them:
 * the last chunk of each (stream, kv head) to finish folds the others' states
 * in index order and writes o and lse, so no merge kernel is launched.
 *   Workspace attn_decode_paged_fused_workspace_bytes bytes (0 when the plan
 *             has one chunk), 4-byte aligned (ATTN_ERR_INVALID otherwise);
 *             its first 64 KiB hold the arrival counts, one per (stream, kv
 *             head), so B * Hkv <= 16384 when the plan has more than one
 *             chunk (ATTN_ERR_UNSUPPORTED otherwise), and the partial states
 *             follow.  The counts must be zero before the first call on that
 *             memory; every call that completes leaves them zero.  Calls
 *             that share a workspace must not run concurrently (stream order
 *             suffices), and memory used by another entry point must be
 *             zeroed again before it serves this one.
 *   Plan     attn_decode_paged's rules on the single-launch model, which
 *             has no merge launch to pay for and so may split more.
 */
size_t attn_decode_paged_fused_workspace_bytes(int64_t B, int64_t Hq, int64_t Hkv, int64_t max_seq_len, int64_t d,
                                               int num_splits);
attn_status attn_decode_paged_fused(const void* q, const void* k_cache, const void* v_cache,
                                    const int32_t* block_table, const int32_t* seq_lens, void* o, float* lse,
                                    int64_t B, int64_t Hq, int64_t Hkv, int64_t d, int64_t num_pages,
                                    int64_t page_size, int64_t max_pages, int64_t max_seq_len, float scale,
                                    int num_splits, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Split-KV decode over an FP8 KV cache: k and v hold OCP FP8 E4M3 codes
 * (1 byte per element, [B,Hkv,Nk,d]; 0x7F / 0xFF are NaN and propagate), and
 * kv head h's values are k_scale[h] * code and v_scale[h] * code (k_scale,
 * v_scale: device fp32 arrays of Hkv scales shared by the batch).  q and o
 * are bf16 [B,Hq,1,d]; lse fp32 [B,Hq] (may be NULL).  The codes are widened
 * to bf16 exactly on the GPU and the scales enter in fp32, so the result is
 * attn_decode_splitkv's on the dequantized cache; only the KV traffic halves.
 * Workspace as attn_decode_workspace_bytes; every other rule as
 * attn_decode_splitkv.  FP8 KV caches are what the second page's fastest
 * compared engine serves ("Tang Project Derives GPU Kernels via IR ...",
 * section "Details").
 */
attn_status attn_decode_splitkv_fp8(const void* q, const void* k, const void* v, const float* k_scale,
                                    const float* v_scale, void* o, float* lse, int64_t B, int64_t Hq, int64_t Hkv,
                                    int64_t Nq, int64_t Nk, int64_t d, float scale, int num_splits, void* workspace,
                                    size_t workspace_bytes, void* stream);

/*
 * Backward from the saved log-sum-exp.  Inputs q, k, v, o, dout (dtype) and
 * lse (fp32, as written by attn_fwd with the same arguments); outputs dq
 * [B,Hq,Nq,d], dk and dv [B,Hkv,Nk,d], all fp32 and fully overwritten (dk and
 * dv sum over the query heads that share a kv head).  The workspace holds one
 * 8-byte record per query row, (LSE * log2 e, D_i = dO_i . O_i), with the rows
 * of each head padded to a multiple of 128.  Only ATTN_BF16 is built.
 *   Source   "Não escreva kernels, derive-os", FAQ entry "O que o Tang propõe
 *            de diferente?": the backward is obtained by rewriting the same
 *            fused expression; section "Aprofundamento", third paragraph: a
 *            fused bf16 backward missed an fp32 tolerance, so the gradients
 *            are accumulated and written in fp32 here.  The pages print no
 *            formula: with P = exp(scale Q K^T - LSE) (masked),
 *            dV = P^T dO, dS = P o (dO V^T - rowsum(dO o O)), dQ = scale dS K,
 *            dK = scale dS^T Q, the textbook gradient of softmax attention.
 *   Result   deterministic: every gradient element has one writer, so
 *            repeated calls give the same bits.
 */
size_t attn_bwd_workspace_bytes(int64_t B, int64_t Hq, int64_t Nq, int64_t d);
attn_status attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                     float* dq, float* dk, float* dv, int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk,
                     int64_t d, float scale, int causal, void* workspace, size_t workspace_bytes, attn_dtype dtype,
                     void* stream);

/*
 * attn_bwd with bf16 gradients: dq [B,Hq,Nq,d] and dk, dv [B,Hkv,Nk,d] are
 * bf16, each element the fp32 value attn_bwd writes for the same arguments
 * rounded to nearest even (the same kernels; only the final stores differ),
 * so the gradient traffic halves for callers whose parameters are bf16.  The
 * first page ("Não escreva kernels, derive-os", section "Aprofundamento",
 * third paragraph) reports that its fused bf16 backward missed an fp32
 * tolerance; here the accumulation stays fp32 and only the output is
 * rounded, which adds at most half a bf16 ulp of each gradient (2^-9 of its
 * magnitude).  Workspace, ownership, errors and every other rule as attn_bwd.
 */
attn_status attn_bwd_bf16_grads(const void* q, const void* k, const void* v, const void* o, const void* dout,
                                const float* lse, void* dq, void* dk, void* dv, int64_t B, int64_t Hq, int64_t Hkv,
                                int64_t Nq, int64_t Nk, int64_t d, float scale, int causal, void* workspace,
                                size_t workspace_bytes, attn_dtype dtype, void* stream);

/* Static, human-readable text for a status code. */
const char* attn_strerror(attn_status status);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_MI355X_H */
