// C ABI of the attention library: argument validation (host only, before any
// HIP call), the split-KV plan, workspace layout and kernel dispatch.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>

#include "../../include/attn.h"
#include "kernels.h"

namespace {

constexpr int kNumCUs = 256;  // MI355X compute units (the decode split plan counts waves of workgroups)

bool dims_ok(int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk) {
  return B >= 0 && Hq >= 1 && Hkv >= 1 && Nq >= 0 && Nk >= 0 && Hq % Hkv == 0;
}

bool scale_ok(float s) { return std::isfinite(s) && s > 0.0f; }

// Common checks; returns ATTN_OK when the call may proceed.
attn_status check_common(int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t d, float scale,
                         attn_dtype dtype) {
  if (!dims_ok(B, Hq, Hkv, Nq, Nk)) return ATTN_ERR_INVALID;
  if (!scale_ok(scale)) return ATTN_ERR_INVALID;
  if (dtype != ATTN_F32 && dtype != ATTN_BF16) return ATTN_ERR_INVALID;
  if (d != 64 && d != 128) return ATTN_ERR_UNSUPPORTED;
  if (Nq > ATTN_MAX_SEQ || Nk > ATTN_MAX_SEQ) return ATTN_ERR_UNSUPPORTED;
  // grid sizes must fit in 32-bit workgroup counts: no kernel takes fewer
  // than 32 query rows per workgroup (the backward's key grid is bounded in
  // attn_bwd)
  if (B * Hq > (int64_t)1 << 20) return ATTN_ERR_UNSUPPORTED;
  if (B * Hq * ((Nq + 31) / 32) >= (int64_t)1 << 31) return ATTN_ERR_UNSUPPORTED;
  return ATTN_OK;
}

struct SplitPlan {
  int splits;
  int chunk;
};

// Choose the number of key chunks per (b, kv head) from a cost model of the
// decode, with constants fitted on MI355X at d = 128 to the measured time of
// every split count (1..64) at 1..48 streams x 512..16384 keys, both entry
// points, K/V streamed with the non-temporal load policy (the fit minimises
// the summed time of the picks; the points it changed were then re-measured
// against the earlier plan in a second job):
//   - a bf16 workgroup streams its chunk at ~80 keys/us after ~3 us of
//     start-up, and the workgroups of a launch run in waves of one per CU;
//     the FP8 kernel (two workgroups per CU, half the bytes per key, the
//     codes widened in registers) keeps its own calibration, ~85 keys/us
//     after ~2 us;
//   - the whole decode reads at most ~6.5 TB/s;
//   - each extra chunk costs ~0.5 us in the fold, and the two-launch path a
//     further ~6 us (FP8: ~4 us) for the merge launch;
//   - a cache the unsplit plan streams in less than ~10 us (FP8: ~15 us) is
//     not split: the call's launch and synchronisation dominate it (FP8, one
//     stream of 1024 keys: 12.9 us unsplit, 16.1 us in four chunks).
// Candidates are 1, 2, 4, ... chunks of at least one key tile, at most 64;
// a larger count must beat the smaller by 5 % (the model's resolution).
// Splitting pays only where too few workgroups would stream the cache: from
// 20 streams x 8 kv heads up a bf16 cache takes one chunk per (b, kv head).
SplitPlan plan_splits(int64_t B, int64_t Hkv, int64_t Nk, int64_t d, int requested, bool fused, bool fp8) {
  const int tile = attn::kDecodeTile;
  const int64_t tiles = Nk > 0 ? (Nk + tile - 1) / tile : 1;
  int s;
  if (requested > 0) {
    s = requested;
  } else {
    constexpr double kHbmBytesPerUs = 6.5e6, kFoldUsPerSplit = 0.5;
    const double keys_per_us = fp8 ? 85.0 : 80.0;
    const double wg_start_us = fp8 ? 2.0 : 3.0;
    const double merge_launch_us = fp8 ? 4.0 : 6.0;
    const double call_floor_us = fp8 ? 15.0 : 10.0;
    const double slots = kNumCUs * (fp8 ? 2.0 : 1.0);
    const double units = (double)(B * Hkv);
    const double key_bytes = 2.0 * (double)d * (fp8 ? 1.0 : 2.0);  // K and V
    const double hbm_us = units * (double)Nk * key_bytes / kHbmBytesPerUs;
    double best = 0.0;
    s = 1;
    for (int64_t c = 1; c <= std::min<int64_t>(tiles, 64); c *= 2) {
      const double chunk_keys = (double)(((tiles + c - 1) / c) * tile);
      const double waves = std::ceil(units * (double)c / slots);
      double t = std::max(waves * (wg_start_us + chunk_keys / keys_per_us), hbm_us);
      if (c > 1) t += kFoldUsPerSplit * (double)c + (fused ? 0.0 : merge_launch_us);
      if (c == 1 || t < 0.95 * best) {
        best = t;
        s = (int)c;
      }
      if (c == 1 && t < call_floor_us) break;
    }
  }
  if (s > tiles) s = (int)tiles;
  int64_t chunk = ((tiles + s - 1) / s) * tile;
  int eff = Nk > 0 ? (int)((Nk + chunk - 1) / chunk) : 1;
  return {eff, (int)chunk};
}

// The paged decode's plan.  Its kernel starts the longest (stream, chunk)
// items first, so unequal lengths alone need no split; the cost model, which
// takes every stream at the longest length, then gets two floors measured at
// 8..48 streams of 64..16384 keys: chunks of at most 4096 keys (48 streams of
// 8192 keys: 260 us in two chunks against 278 in one; of 1024..12288: 205 in
// three against 222), but no split into chunks of 2048 keys or fewer where
// the streams fill the CUs (48 of 512..4096: 92.7 us unsplit, 101.9 in two);
// and with fewer (stream, kv head) pairs than CUs, enough chunks of at least
// 1024 keys to give each CU one (16 streams of 512..4096: 42.7 us in two
// chunks against 51.9 in one).
SplitPlan paged_plan(int64_t B, int64_t Hkv, int64_t max_seq_len, int64_t d, int requested, bool fused = false) {
  if (requested == 0) {
    int64_t s = plan_splits(B, Hkv, max_seq_len, d, 0, fused, false).splits;
    s = std::max<int64_t>(s, max_seq_len / 4096);
    const int64_t pairs = B * Hkv;
    if (pairs > 0 && pairs < kNumCUs)
      s = std::max<int64_t>(s, std::min<int64_t>((kNumCUs + pairs - 1) / pairs, max_seq_len / 1024));
    requested = (int)std::min<int64_t>(s, 64);
  }
  return plan_splits(B, Hkv, max_seq_len, d, requested, fused, false);
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// The single-launch decode's arrival counts: a fixed region at the start of
// its workspace, one 4-byte count per (stream, kv head), so that no call's
// partial states ever overlap a count another call may use.
constexpr size_t kDecodeCountBytes = 65536;
constexpr int64_t kDecodeMaxPairs = (int64_t)(kDecodeCountBytes / sizeof(unsigned));

}  // namespace

extern "C" {

const char* attn_strerror(attn_status status) {
  switch (status) {
    case ATTN_OK:
      return "ok";
    case ATTN_ERR_INVALID:
      return "invalid argument";
    case ATTN_ERR_UNSUPPORTED:
      return "unsupported configuration";
    case ATTN_ERR_WORKSPACE:
      return "workspace missing or too small";
    case ATTN_ERR_HIP:
      return "HIP launch failed";
    case ATTN_ERR_SCRATCH:
      return "the split plan needs more than the fixed scratch of the allocation-free entry point";
  }
  return "unknown status";
}

attn_status attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B, int64_t Hq,
                     int64_t Hkv, int64_t Nq, int64_t Nk, int64_t d, float scale, int causal, attn_dtype dtype,
                     void* stream) {
  attn_status st = check_common(B, Hq, Hkv, Nq, Nk, d, scale, dtype);
  if (st != ATTN_OK) return st;
  if (B == 0 || Nq == 0) return ATTN_OK;
  if (!q || !o || (Nk > 0 && (!k || !v))) return ATTN_ERR_INVALID;
  attn::FwdProblem p{q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale, causal ? 1 : 0, dtype == ATTN_BF16};
  return attn::launch_fwd(p, (hipStream_t)stream) == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

attn_status attn_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                            const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int64_t n_seqs,
                            int64_t total_q, int64_t total_k, int64_t max_seqlen_q, int64_t Hq, int64_t Hkv,
                            int64_t d, float scale, int causal, attn_dtype dtype, void* stream) {
  if (n_seqs < 0 || total_q < 0 || total_k < 0 || max_seqlen_q < 0) return ATTN_ERR_INVALID;
  attn_status st = check_common(n_seqs, Hq, Hkv, max_seqlen_q, total_k, d, scale, dtype);
  if (st != ATTN_OK) return st;
  if (total_q > ATTN_MAX_SEQ) return ATTN_ERR_UNSUPPORTED;
  if (dtype != ATTN_BF16) return ATTN_ERR_UNSUPPORTED;
  if (n_seqs == 0 || total_q == 0 || max_seqlen_q == 0) return ATTN_OK;
  if (!q || !o || !cu_seqlens_q || !cu_seqlens_k || (total_k > 0 && (!k || !v))) return ATTN_ERR_INVALID;
  attn::FwdProblem p{q, k, v, o, lse, n_seqs, Hq, Hkv, max_seqlen_q, total_k, d, scale, causal ? 1 : 0, true};
  p.cu_q = cu_seqlens_q;
  p.cu_k = cu_seqlens_k;
  p.tot_q = total_q;
  p.tot_k = total_k;
  return attn::launch_fwd(p, (hipStream_t)stream) == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

attn_status attn_fwd_varlen_paged(const void* q, const void* k_cache, const void* v_cache, const int32_t* block_table,
                                  void* o, float* lse, const int32_t* cu_seqlens_q, const int32_t* seq_lens_k,
                                  int64_t n_seqs, int64_t total_q, int64_t max_seqlen_q, int64_t max_seqlen_k,
                                  int64_t Hq, int64_t Hkv, int64_t d, int64_t num_pages, int64_t page_size,
                                  int64_t max_pages, float scale, int causal, void* stream) {
  if (n_seqs < 0 || total_q < 0 || max_seqlen_q < 0 || max_seqlen_k < 0 || num_pages < 0 || page_size < 0 ||
      max_pages < 0)
    return ATTN_ERR_INVALID;
  attn_status st = check_common(n_seqs, Hq, Hkv, max_seqlen_q, max_seqlen_k, d, scale, ATTN_BF16);
  if (st != ATTN_OK) return st;
  if (total_q > ATTN_MAX_SEQ) return ATTN_ERR_UNSUPPORTED;
  if (page_size == 0 || page_size % 64 != 0) return ATTN_ERR_UNSUPPORTED;
  if (max_pages > ATTN_MAX_SEQ / page_size) return ATTN_ERR_UNSUPPORTED;
  if (n_seqs == 0 || total_q == 0 || max_seqlen_q == 0) return ATTN_OK;
  if (!q || !o || !cu_seqlens_q || !seq_lens_k) return ATTN_ERR_INVALID;
  if (max_seqlen_k > 0 && (!k_cache || !v_cache || !block_table || num_pages == 0 || max_pages == 0))
    return ATTN_ERR_INVALID;
  attn::FwdProblem p{q, k_cache, v_cache, o, lse, n_seqs, Hq, Hkv, max_seqlen_q, max_seqlen_k, d, scale,
                     causal ? 1 : 0, true};
  p.cu_q = cu_seqlens_q;
  p.tot_q = total_q;
  p.paged = true;
  // with max_seqlen_k = 0 every sequence is clamped to no keys and neither
  // the table nor the cache is read
  p.block_table = block_table;
  p.seq_lens_k = seq_lens_k;
  p.page = page_size;
  p.max_pages = max_pages;
  p.num_pages = num_pages;
  return attn::launch_fwd(p, (hipStream_t)stream) == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

int attn_decode_num_splits(int64_t B, int64_t Hq, int64_t Hkv, int64_t Nk, int64_t d) {
  if (!dims_ok(B, Hq, Hkv, 1, Nk) || (d != 64 && d != 128)) return -1;
  return plan_splits(B, Hkv, Nk, d, 0, false, false).splits;
}

int attn_decode_fused_num_splits(int64_t B, int64_t Hq, int64_t Hkv, int64_t Nk, int64_t d) {
  if (!dims_ok(B, Hq, Hkv, 1, Nk) || (d != 64 && d != 128)) return -1;
  return plan_splits(B, Hkv, Nk, d, 0, true, false).splits;
}

}  // extern "C"

namespace {

// Bytes of the partial states (m, l, acc) of a split plan; 0 for one chunk.
size_t partial_bytes(int64_t B, int64_t Hq, int64_t Hkv, int64_t d, const SplitPlan& sp) {
  if (sp.splits <= 1) return 0;
  const size_t rows = (size_t)B * Hq * sp.splits;
  return align256(rows * d * sizeof(float)) + align256(rows * 2 * sizeof(float));
}

}  // namespace

extern "C" {

size_t attn_decode_workspace_bytes(int64_t B, int64_t Hq, int64_t Hkv, int64_t Nk, int64_t d, int num_splits) {
  if (!dims_ok(B, Hq, Hkv, 1, Nk) || (d != 64 && d != 128) || num_splits < 0) return 0;
  // enough for the bf16, FP8 and paged entry points' plans
  static_assert(attn::kDecodeScratchBytes == ATTN_DECODE_SCRATCH_BYTES, "one scratch size");
  return std::max({partial_bytes(B, Hq, Hkv, d, plan_splits(B, Hkv, Nk, d, num_splits, false, false)),
                   partial_bytes(B, Hq, Hkv, d, plan_splits(B, Hkv, Nk, d, num_splits, false, true)),
                   partial_bytes(B, Hq, Hkv, d, paged_plan(B, Hkv, Nk, d, num_splits))});
}

size_t attn_decode_fused_workspace_bytes(int64_t B, int64_t Hq, int64_t Hkv, int64_t Nk, int64_t d, int num_splits) {
  if (!dims_ok(B, Hq, Hkv, 1, Nk) || (d != 64 && d != 128) || num_splits < 0) return 0;
  const size_t parts = partial_bytes(B, Hq, Hkv, d, plan_splits(B, Hkv, Nk, d, num_splits, true, false));
  if (parts == 0) return 0;
  return kDecodeCountBytes + parts;
}

size_t attn_decode_paged_fused_workspace_bytes(int64_t B, int64_t Hq, int64_t Hkv, int64_t max_seq_len, int64_t d,
                                               int num_splits) {
  if (!dims_ok(B, Hq, Hkv, 1, max_seq_len) || (d != 64 && d != 128) || num_splits < 0) return 0;
  const size_t parts = partial_bytes(B, Hq, Hkv, d, paged_plan(B, Hkv, max_seq_len, d, num_splits, true));
  if (parts == 0) return 0;
  return kDecodeCountBytes + parts;
}

}  // extern "C"

namespace {

attn_status decode_common(const void* q, const void* k, const void* v, const float* k_scale, const float* v_scale,
                          bool fp8, bool fused, void* o, float* lse, int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk,
                          int64_t d, float scale, int num_splits, void* workspace, size_t workspace_bytes,
                          attn_dtype dtype, void* stream, bool use_scratch = false) {
  attn_status st = check_common(B, Hq, Hkv, Nq, Nk, d, scale, dtype);
  if (st != ATTN_OK) return st;
  if (num_splits < 0) return ATTN_ERR_INVALID;
  if (Nq != 1 && !(Nq == 0 || B == 0)) return ATTN_ERR_INVALID;
  if (dtype != ATTN_BF16) return ATTN_ERR_UNSUPPORTED;
  if (Hq / Hkv > 32) return ATTN_ERR_UNSUPPORTED;
  if (B == 0 || Nq == 0) return ATTN_OK;
  if (!q || !o || (Nk > 0 && (!k || !v))) return ATTN_ERR_INVALID;
  if (fp8 && Nk > 0 && (!k_scale || !v_scale)) return ATTN_ERR_INVALID;
  SplitPlan sp = plan_splits(B, Hkv, Nk, d, num_splits, fused, fp8);
  attn::DecodeProblem p{};
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  p.B = B;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.Nk = Nk;
  p.d = d;
  p.scale = scale;
  p.num_splits = sp.splits;
  p.chunk = sp.chunk;
  if (sp.splits > 1) {
    const size_t need = (fused ? kDecodeCountBytes : 0) + partial_bytes(B, Hq, Hkv, d, sp);
    if (use_scratch) {
      // the library's fixed device scratch instead of a caller workspace
      if (need > ATTN_DECODE_SCRATCH_BYTES) return ATTN_ERR_SCRATCH;
      if (attn::decode_scratch(&workspace) != hipSuccess) return ATTN_ERR_HIP;
      workspace_bytes = ATTN_DECODE_SCRATCH_BYTES;
    }
    if (workspace == nullptr || workspace_bytes < need) return ATTN_ERR_WORKSPACE;
    // the arrival counts take device atomics: 4-byte alignment
    if (fused && ((uintptr_t)workspace & 3) != 0) return ATTN_ERR_INVALID;
    char* ws = (char*)workspace;
    if (fused) {
      if (B * Hkv > kDecodeMaxPairs) return ATTN_ERR_UNSUPPORTED;
      p.counters = (unsigned*)ws;
      ws += kDecodeCountBytes;
    }
    const size_t rows = (size_t)B * Hq * sp.splits;
    p.part_acc = (float*)ws;
    p.part_ml = (float*)(ws + align256(rows * d * sizeof(float)));
  }
  if (fp8 && Nk > 0) {
    p.k8 = (const uint8_t*)k;
    p.v8 = (const uint8_t*)v;
    p.k_scale = k_scale;
    p.v_scale = v_scale;
  }
  return attn::launch_decode(p, (hipStream_t)stream) == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

}  // namespace

extern "C" {

attn_status attn_decode_splitkv(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B,
                                int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t d, float scale, int causal,
                                int num_splits, void* workspace, size_t workspace_bytes, attn_dtype dtype,
                                void* stream) {
  (void)causal;  // one bottom-right-aligned query sees every key
  return decode_common(q, k, v, nullptr, nullptr, false, false, o, lse, B, Hq, Hkv, Nq, Nk, d, scale, num_splits, workspace,
                       workspace_bytes, dtype, stream);
}

attn_status attn_decode_splitkv_noalloc(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B,
                                        int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t d, float scale,
                                        int causal, int num_splits, attn_dtype dtype, void* stream) {
  (void)causal;
  return decode_common(q, k, v, nullptr, nullptr, false, false, o, lse, B, Hq, Hkv, Nq, Nk, d, scale, num_splits,
                       nullptr, 0, dtype, stream, true);
}

size_t attn_decode_noalloc_scratch_bytes(int64_t B, int64_t Hq, int64_t Hkv, int64_t Nk, int64_t d, int num_splits) {
  if (!dims_ok(B, Hq, Hkv, 1, Nk) || (d != 64 && d != 128) || num_splits < 0) return 0;
  return partial_bytes(B, Hq, Hkv, d, plan_splits(B, Hkv, Nk, d, num_splits, false, false));
}

attn_status attn_decode_splitkv_fused(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B,
                                      int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk, int64_t d, float scale,
                                      int causal, int num_splits, void* workspace, size_t workspace_bytes,
                                      attn_dtype dtype, void* stream) {
  (void)causal;
  return decode_common(q, k, v, nullptr, nullptr, false, true, o, lse, B, Hq, Hkv, Nq, Nk, d, scale, num_splits,
                       workspace, workspace_bytes, dtype, stream);
}

}  // extern "C"

namespace {

attn_status paged_common(const void* q, const void* k_cache, const void* v_cache, const int32_t* block_table,
                         const int32_t* seq_lens, void* o, float* lse, int64_t B, int64_t Hq, int64_t Hkv, int64_t d,
                         int64_t num_pages, int64_t page_size, int64_t max_pages, int64_t max_seq_len, float scale,
                         int num_splits, void* workspace, size_t workspace_bytes, void* stream, bool fused) {
  if (num_pages < 0 || page_size < 0 || max_pages < 0 || max_seq_len < 0) return ATTN_ERR_INVALID;
  attn_status st = check_common(B, Hq, Hkv, 1, max_seq_len, d, scale, ATTN_BF16);
  if (st != ATTN_OK) return st;
  if (num_splits < 0) return ATTN_ERR_INVALID;
  if (page_size == 0 || page_size % attn::kDecodeTile != 0) return ATTN_ERR_UNSUPPORTED;
  if (max_pages > ATTN_MAX_SEQ / page_size) return ATTN_ERR_UNSUPPORTED;
  if (Hq / Hkv > 32) return ATTN_ERR_UNSUPPORTED;
  if (B == 0) return ATTN_OK;
  if (!q || !o || !seq_lens) return ATTN_ERR_INVALID;
  // keys can be read only if there are pages to read them from
  if (max_seq_len > 0 && (max_pages == 0 || num_pages == 0 || !k_cache || !v_cache || !block_table))
    return ATTN_ERR_INVALID;
  SplitPlan sp = paged_plan(B, Hkv, max_seq_len, d, num_splits, fused);
  attn::DecodeProblem p{};
  p.q = q;
  p.k = k_cache;
  p.v = v_cache;
  p.o = o;
  p.lse = lse;
  p.B = B;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.Nk = max_seq_len;
  p.d = d;
  p.scale = scale;
  p.num_splits = sp.splits;
  p.chunk = sp.chunk;
  if (sp.splits > 1) {
    const size_t need = (fused ? kDecodeCountBytes : 0) + partial_bytes(B, Hq, Hkv, d, sp);
    if (workspace == nullptr || workspace_bytes < need) return ATTN_ERR_WORKSPACE;
    // the arrival counts take device atomics: 4-byte alignment
    if (fused && ((uintptr_t)workspace & 3) != 0) return ATTN_ERR_INVALID;
    char* ws = (char*)workspace;
    if (fused) {
      if (B * Hkv > kDecodeMaxPairs) return ATTN_ERR_UNSUPPORTED;
      p.counters = (unsigned*)ws;
      ws += kDecodeCountBytes;
    }
    const size_t rows = (size_t)B * Hq * sp.splits;
    p.part_acc = (float*)ws;
    p.part_ml = (float*)(ws + align256(rows * d * sizeof(float)));
  }
  if (max_seq_len > 0) {
    p.block_table = block_table;
    p.seq_lens = seq_lens;
    p.page = page_size;
    p.max_pages = max_pages;
    p.num_pages = num_pages;
  } else {
    // no keys at all: the dense kernel with Nk = 0 writes O = 0, LSE = -inf
    p.k = p.v = nullptr;
  }
  return attn::launch_decode(p, (hipStream_t)stream) == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

}  // namespace

extern "C" {

attn_status attn_decode_paged(const void* q, const void* k_cache, const void* v_cache, const int32_t* block_table,
                              const int32_t* seq_lens, void* o, float* lse, int64_t B, int64_t Hq, int64_t Hkv,
                              int64_t d, int64_t num_pages, int64_t page_size, int64_t max_pages,
                              int64_t max_seq_len, float scale, int num_splits, void* workspace,
                              size_t workspace_bytes, void* stream) {
  return paged_common(q, k_cache, v_cache, block_table, seq_lens, o, lse, B, Hq, Hkv, d, num_pages, page_size,
                      max_pages, max_seq_len, scale, num_splits, workspace, workspace_bytes, stream, false);
}

attn_status attn_decode_paged_fused(const void* q, const void* k_cache, const void* v_cache,
                                    const int32_t* block_table, const int32_t* seq_lens, void* o, float* lse,
                                    int64_t B, int64_t Hq, int64_t Hkv, int64_t d, int64_t num_pages,
                                    int64_t page_size, int64_t max_pages, int64_t max_seq_len, float scale,
                                    int num_splits, void* workspace, size_t workspace_bytes, void* stream) {
  return paged_common(q, k_cache, v_cache, block_table, seq_lens, o, lse, B, Hq, Hkv, d, num_pages, page_size,
                      max_pages, max_seq_len, scale, num_splits, workspace, workspace_bytes, stream, true);
}

attn_status attn_decode_splitkv_fp8(const void* q, const void* k, const void* v, const float* k_scale,
                                    const float* v_scale, void* o, float* lse, int64_t B, int64_t Hq, int64_t Hkv,
                                    int64_t Nq, int64_t Nk, int64_t d, float scale, int num_splits, void* workspace,
                                    size_t workspace_bytes, void* stream) {
  return decode_common(q, k, v, k_scale, v_scale, true, false, o, lse, B, Hq, Hkv, Nq, Nk, d, scale, num_splits, workspace,
                       workspace_bytes, ATTN_BF16, stream);
}

size_t attn_bwd_workspace_bytes(int64_t B, int64_t Hq, int64_t Nq, int64_t d) {
  if (B < 0 || Hq < 1 || Nq < 0 || (d != 64 && d != 128)) return 0;
  return align256((size_t)B * Hq * attn::bwd_record_rows(Nq) * 2 * sizeof(float));
}

}  // extern "C"

static attn_status bwd_common(const void* q, const void* k, const void* v, const void* o, const void* dout,
                              const float* lse, void* dq, void* dk, void* dv, int grad_bf16, int64_t B, int64_t Hq,
                              int64_t Hkv, int64_t Nq, int64_t Nk, int64_t d, float scale, int causal,
                              void* workspace, size_t workspace_bytes, attn_dtype dtype, void* stream) {
  attn_status st = check_common(B, Hq, Hkv, Nq, Nk, d, scale, dtype);
  if (st != ATTN_OK) return st;
  if (dtype != ATTN_BF16) return ATTN_ERR_UNSUPPORTED;
  // the dK/dV grid: 128 keys of one kv head per workgroup
  if (B * Hkv * ((Nk + 31) / 32) >= (int64_t)1 << 31) return ATTN_ERR_UNSUPPORTED;
  if (B == 0 || (Nq == 0 && Nk == 0)) return ATTN_OK;
  if (Nq > 0 && (!q || !o || !dout || !lse || !dq)) return ATTN_ERR_INVALID;
  if (Nk > 0 && (!k || !v || !dk || !dv)) return ATTN_ERR_INVALID;
  const size_t need = attn_bwd_workspace_bytes(B, Hq, Nq, d);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return ATTN_ERR_WORKSPACE;
  attn::BwdProblem p{};
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.dout = dout;
  p.lse = lse;
  p.dq = dq;
  p.dk = dk;
  p.dv = dv;
  p.stats = (float*)workspace;
  p.B = B;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.Nq = Nq;
  p.Nk = Nk;
  p.d = d;
  p.scale = scale;
  p.causal = causal ? 1 : 0;
  p.grad_bf16 = grad_bf16;
  return attn::launch_bwd(p, (hipStream_t)stream) == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

extern "C" {

attn_status attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                     float* dq, float* dk, float* dv, int64_t B, int64_t Hq, int64_t Hkv, int64_t Nq, int64_t Nk,
                     int64_t d, float scale, int causal, void* workspace, size_t workspace_bytes, attn_dtype dtype,
                     void* stream) {
  return bwd_common(q, k, v, o, dout, lse, dq, dk, dv, 0, B, Hq, Hkv, Nq, Nk, d, scale, causal, workspace,
                    workspace_bytes, dtype, stream);
}

attn_status attn_bwd_bf16_grads(const void* q, const void* k, const void* v, const void* o, const void* dout,
                                const float* lse, void* dq, void* dk, void* dv, int64_t B, int64_t Hq, int64_t Hkv,
                                int64_t Nq, int64_t Nk, int64_t d, float scale, int causal, void* workspace,
                                size_t workspace_bytes, attn_dtype dtype, void* stream) {
  return bwd_common(q, k, v, o, dout, lse, dq, dk, dv, 1, B, Hq, Hkv, Nq, Nk, d, scale, causal, workspace,
                    workspace_bytes, dtype, stream);
}

}  // extern "C"
