// Internal interface between the C ABI (attn_abi.cpp) and the kernel files.
// Arguments arrive here already validated: d in {64, 128}, Hq % Hkv == 0,
// every size positive and at most ATTN_MAX_SEQ, pointers non-null where needed.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace attn {

struct FwdProblem {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;  // may be null
  int64_t B, Hq, Hkv, Nq, Nk, d;
  float scale;
  int causal;
  bool bf16;
  // packed variable-length batch (bf16 only), null for a dense one: B is
  // the number of sequences, Nq the longest query length (it sizes the
  // grid), cu_q / cu_k the [B + 1] device offsets of each sequence's rows in
  // the [H, tot_q or tot_k, d] tensors
  const int32_t* cu_q = nullptr;
  const int32_t* cu_k = nullptr;
  int64_t tot_q = 0, tot_k = 0;
  // packed batch over a paged K/V cache (with cu_q; cu_k unused): k, v are
  // [num_pages, Hkv, page, d] with page a multiple of 64; block_table
  // [B, max_pages] int32; seq_lens_k [B] int32 keys per sequence; Nk is the
  // longest
  bool paged = false;
  const int32_t* block_table = nullptr;
  const int32_t* seq_lens_k = nullptr;
  int64_t page = 0, max_pages = 0, num_pages = 0;
};
hipError_t launch_fwd(const FwdProblem& p, hipStream_t s);

struct DecodeProblem {
  const void* q;  // [B, Hq, 1, d] bf16
  const void* k;  // [B, Hkv, Nk, d] bf16
  const void* v;
  void* o;        // [B, Hq, 1, d] bf16
  float* lse;     // [B, Hq] fp32, may be null
  int64_t B, Hq, Hkv, Nk, d;
  float scale;
  int num_splits;  // >= 1, already resolved
  int chunk;       // keys per split, a multiple of the kernel's key tile
  float* part_acc; // [B, Hq, num_splits, d] fp32 (unused when num_splits == 1)
  float* part_ml;  // [B, Hq, num_splits, 2] fp32 (running max in log2 units, sum)
  // FP8 KV cache (null for bf16 k, v): OCP E4M3 codes [B, Hkv, Nk, d] and a
  // fp32 scale per kv head for each of K and V
  const uint8_t* k8 = nullptr;
  const uint8_t* v8 = nullptr;
  const float* k_scale = nullptr;
  const float* v_scale = nullptr;
  // single launch (null: a second kernel merges the splits): [B * Hkv]
  // arrival counts, zero on entry; the last split of each (stream, kv head)
  // to finish merges them and returns its count to zero
  unsigned* counters = nullptr;
  // paged KV cache (bf16; null block_table for a dense one): k, v are
  // [num_pages, Hkv, page, d] with page a multiple of kDecodeTile; block_table
  // [B, max_pages] int32 page ids, seq_lens [B] int32 keys per stream; Nk is
  // the longest stream (it sizes the split plan)
  const int32_t* block_table = nullptr;
  const int32_t* seq_lens = nullptr;
  int64_t page = 0, max_pages = 0, num_pages = 0;
};
// Keys per decode tile; split chunks are whole multiples of it.
constexpr int kDecodeTile = 32;
hipError_t launch_decode(const DecodeProblem& p, hipStream_t s);
// Bytes of the decode's fixed device scratch (the allocation-free entry
// point's partial states); ATTN_DECODE_SCRATCH_BYTES in attn.h.
constexpr size_t kDecodeScratchBytes = (size_t)8 << 20;
// Device address of the current device's copy of that scratch (looked up
// once per device).
hipError_t decode_scratch(void** ptr);

struct BwdProblem {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;
  void* dq;      // fp32, or bf16 when grad_bf16
  void* dk;
  void* dv;
  float* stats;  // workspace: [B, Hq, bwd_record_rows(Nq)] x 2 fp32 (LSE * log2 e, D)
  int64_t B, Hq, Hkv, Nq, Nk, d;
  float scale;
  int causal;
  int grad_bf16;
};
// Rows of backward row records per head: Nq rounded up to 128.
inline int64_t bwd_record_rows(int64_t Nq) { return (Nq + 127) / 128 * 128; }
hipError_t launch_bwd(const BwdProblem& p, hipStream_t s);

}  // namespace attn
