// Split-KV decode kernels for gfx950.
//
// One query token per stream.  A kv head's Nk keys are cut into num_splits
// chunks; workgroup (b, kv head, split) streams its chunk of K and V from HBM
// exactly once and serves all g = Hq / Hkv query heads that share the kv head
// (grouped-query packing: the g queries are the columns of one MFMA tile, so
// the bytes read do not grow with g).  The four waves of a workgroup take
// 32-key tiles in turn, each through its own pair of LDS buffers filled by
// direct-to-LDS buffer loads, and each keeps its own online-softmax state
// (m, l, acc).  At the end the four states are folded with the monoid rule
// through LDS; the result is either the final output (one split) or a partial
// state written to the workspace, and a merge kernel folds the splits:
//
//   M = max_s m_s,  L = sum_s l_s 2^(m_s - M),  acc = sum_s acc_s 2^(m_s - M),
//   O = acc / L,    LSE = (M + log2 L) ln 2,
//
// with a split whose m_s = -inf contributing nothing.  The fold is the
// online-softmax monoid of "Não escreva kernels, derive-os" (section
// "Aprofundamento", first paragraph); the decode setting with 1 to 48
// concurrent streams is the one "Tang Project Derives GPU Kernels via IR ..."
// reports in its "Details" section.  Regrouping a monoid fold does not change
// its value, so any split count gives the same result up to rounding.
#include <mutex>

#include "device_common.hpp"
#include "kernels.h"

namespace attn {

namespace {

constexpr float kTau = 8.0f;
// waves per workgroup of the FP8 decode kernel (the bf16 kernel takes 2 or 4
// by grid size)
#ifndef ATTN_DECODE_WAVES
#define ATTN_DECODE_WAVES 4
#endif
constexpr int kWaves = ATTN_DECODE_WAVES;
// LDS stages per wave of the FP8 kernel.  Two stages (64 KB of tiles, so two
// workgroups share a CU) measured faster than three or four (one workgroup
// per CU, more tiles in flight per wave) at 48 x 4096, 16 x 4096 and 48 x 2048.
#ifndef ATTN_DECODE_FP8_STAGES
#define ATTN_DECODE_FP8_STAGES 2
#endif

struct DecArgs {
  const __bf16* q;
  const __bf16* k;
  const __bf16* v;
  __bf16* o;
  float* lse;
  float* part_acc;
  float* part_ml;
  int B, Hq, Hkv, Nk, g;
  int S, chunk, n_wgs;
  float c;
  // FP8 KV cache: k8, v8 hold OCP E4M3 codes; kv head h's values are
  // k_scale[h] * code and v_scale[h] * code
  const uint8_t* k8;
  const uint8_t* v8;
  const float* k_scale;
  const float* v_scale;
  // single-launch mode (null: a merge kernel folds the splits): one arrival
  // count per (stream, kv head), zero on entry and left zero on exit
  unsigned* counters;
  // paged KV cache (null for a dense one): k, v are [num_pages, Hkv, page, D];
  // key j of stream b sits in slot j % page of page block_table[b][j / page];
  // stream b has seq_lens[b] keys (Nk is the longest)
  const int* block_table;
  const int* seq_lens;
  int page, max_pages, num_pages;
};

// The partial states are written and, in single-launch mode, read back by
// workgroups on other XCDs, whose L2 caches are not coherent with each
// other.  Device-scope relaxed accesses keep them coherent per access (the
// store writes through to memory, the load fetches from it) instead of a
// device-scope fence, which writes back or invalidates a whole L2 (measured:
// the fences doubled the 48 x 4096 decode).
__device__ __forceinline__ void store_agent(float* p, float x) {
  __hip_atomic_store(p, x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_agent(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Fold the num_splits partial states of row (b, query head) for output
// column col and write O (and LSE from column 0).  The merge kernel and the
// single-launch path share it, so both give the same bits.  AGENT: the
// states were written by this same launch on other XCDs (device-scope
// loads); otherwise by an earlier kernel (plain loads, which may hit L2).
// Up to kFoldBatch splits are loaded all at once (one memory round trip
// instead of one for the maxima and another for the sums); more splits take
// the two unrolled loops.  Either way the fold is the same sequence of
// operations, so the bits do not depend on the path.
constexpr int kFoldBatch = 8;
template <int D, bool AGENT>
__device__ __forceinline__ void fold_split_states(const DecArgs& a, size_t row, int col) {
  auto ld = [](const float* p) { return AGENT ? load_agent(p) : *p; };
  const float* ml = a.part_ml + row * a.S * 2;
  const float* pa = a.part_acc + row * a.S * D + col;
  float M = kNegInf;
  float L = 0.0f, A = 0.0f;
  if (a.S <= kFoldBatch) {
    float m[kFoldBatch], l[kFoldBatch], x[kFoldBatch];
#pragma unroll
    for (int s = 0; s < kFoldBatch; s++) {
      m[s] = kNegInf;
      l[s] = x[s] = 0.0f;
      if (s < a.S) {
        m[s] = ld(ml + 2 * s);
        l[s] = ld(ml + 2 * s + 1);
        x[s] = ld(pa + (size_t)s * D);
      }
    }
#pragma unroll
    for (int s = 0; s < kFoldBatch; s++)
      if (s < a.S) M = fmaxf(M, m[s]);
#pragma unroll
    for (int s = 0; s < kFoldBatch; s++) {
      if (s < a.S) {
        const float f = (m[s] == kNegInf) ? 0.0f : fast_exp2(m[s] - M);
        L += f * l[s];
        A += f * x[s];
      }
    }
  } else {
#pragma unroll 8
    for (int s = 0; s < a.S; s++) M = fmaxf(M, ld(ml + 2 * s));
#pragma unroll 8
    for (int s = 0; s < a.S; s++) {
      const float ms = ld(ml + 2 * s);
      const float f = (ms == kNegInf) ? 0.0f : fast_exp2(ms - M);
      L += f * ld(ml + 2 * s + 1);
      A += f * ld(pa + (size_t)s * D);
    }
  }
  const float inv = L > 0.0f ? 1.0f / L : 0.0f;
  a.o[row * D + col] = to_bf16(A * inv);
  if (col == 0 && a.lse != nullptr) a.lse[row] = L > 0.0f ? (M + __log2f(L)) * kLn2 : kNegInf;
}

// Single-launch split-KV: called by every thread of a workgroup once it has
// issued its partial state's (write-through) stores.  Each thread waits for
// its stores to complete, then the workgroup counts itself in for its
// (stream, kv head) with a device-scope atomic; the workgroup that arrives
// last (every other split's stores completed before that split counted in)
// folds all splits of its g query rows, reading them from memory, and returns
// the count to zero for the next call.
template <int D>
__device__ void merge_if_last(const DecArgs& a, int b, int kvh, int pair) {
  __shared__ unsigned s_last;
  wait_vmem();
  __syncthreads();
  if (threadIdx.x == 0) s_last = atomicAdd(a.counters + pair, 1u) == (unsigned)(a.S - 1) ? 1u : 0u;
  __syncthreads();
  if (s_last == 0u) return;
  const int total = a.g * D;
  for (int e = threadIdx.x; e < total; e += blockDim.x) {
    const int qh = e / D, col = e % D;
    fold_split_states<D, true>(a, (size_t)b * a.Hq + kvh * a.g + qh, col);
  }
  if (threadIdx.x == 0) atomicExch(a.counters + pair, 0u);
}

// Paged caches: the streams differ in length, so the launch order follows each
// (stream, chunk) item's own weight, longest first (lpt_place), instead of the
// dense grid's (stream, kv head, chunk) order, where a long stream's chunks
// could start last and run alone at the end.  Chunk s of a stream of L keys
// holds clamp(L - s chunk, 0, chunk) keys and weighs its 32-key tiles, so the
// chunks of weight >= w are a stream's first ones; the Hkv heads of an item
// take consecutive launch indices.  Empty chunks come last and only store an
// empty state for the merge.
__device__ __forceinline__ void paged_decode_item(const DecArgs& a, int rank, int& b, int& kvh, int& split) {
  const int lim = min(a.Nk, a.max_pages * a.page);
  auto size = [&](int s) -> int2 { return make_int2(min(max(a.seq_lens[s], 0), lim), 0); };
  auto count = [&](int2 sz, int w) -> int {
    if (w <= 0) return a.S;
    const int y = (w - 1) * kDecodeTile;  // weight >= w  <=>  more than y keys
    if (y >= a.chunk || sz.x <= y) return 0;
    return min(a.S, (sz.x - y + a.chunk - 1) / a.chunk);
  };
  int2 sz;
  int c_lo, c_lo1, k;
  lpt_place<4>(a.B, a.Hkv, rank, a.chunk / kDecodeTile + 2, size, count, b, sz, c_lo, c_lo1, k, kvh);
  split = c_lo1 + k;
}

template <int D, bool PAGED, int NWV>
__global__ __launch_bounds__(NWV * 64, 1) void decode_partial_kernel(DecArgs a) {
  constexpr int BN = kDecodeTile;
  constexpr int TILE_BYTES = BN * D * 2;
  constexpr int STAGE = 2 * TILE_BYTES;  // K then V
  constexpr int CPR = D / 8;
  constexpr int LOADS = BN * CPR / 64;   // per lane per tile, one wave loads its own tile
  static_assert(BN == 32, "one 32-key MFMA block per tile");
  // per wave: two stages.  One LDS object per stage, each holding every
  // wave's tile of that stage, so that the compiler can tell the prefetch
  // into one stage from the reads of the other (1-2 % faster than one array
  // with per-wave offsets); stage 0 also holds the final fold.
  constexpr int FOLD = NWV * 32 * D * 4 + 2 * NWV * 32 * 4;
  constexpr int ST0 = NWV * STAGE > FOLD ? NWV * STAGE : FOLD;
  __shared__ __attribute__((aligned(1024))) char stg0[ST0];
  __shared__ __attribute__((aligned(1024))) char stg1[NWV * STAGE];
  char* const smem = stg0;

  const int lane = threadIdx.x & 63;
  const int wave = wave_id();
  const int h32 = lane >> 5;
  const int l32 = lane & 31;

  int split, pair;
  if constexpr (PAGED) {
    int bi, hi;
    paged_decode_item(a, (int)blockIdx.x, bi, hi, split);
    pair = bi * a.Hkv + hi;
  } else {
    const int work = xcd_remap(blockIdx.x, a.n_wgs);
    split = work % a.S;
    pair = work / a.S;
  }
  const int b = pair / a.Hkv;
  const int kvh = pair % a.Hkv;

  // this stream's keys: all Nk, or (paged) its own length, clamped to the
  // block table's reach
  int nk_b = a.Nk;
  if constexpr (PAGED) nk_b = min(max(a.seq_lens[b], 0), min(a.Nk, a.max_pages * a.page));
  const int k0 = split * a.chunk;
  const int k1 = min(nk_b, k0 + a.chunk);
  const int n_tiles = k1 > k0 ? (k1 - k0 + BN - 1) / BN : 0;
  const int my_tiles = n_tiles > wave ? (n_tiles - wave + NWV - 1) / NWV : 0;

  const size_t kv_head = ((size_t)b * a.Hkv + kvh) * (size_t)a.Nk * D;
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(a.k + (PAGED ? 0 : kv_head), (uint32_t)a.Nk * D * 2);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(a.v + (PAGED ? 0 : kv_head), (uint32_t)a.Nk * D * 2);
  const size_t q_grp = ((size_t)b * a.Hq + (size_t)kvh * a.g) * D;  // the g query rows of this kv head
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(a.q + q_grp, (uint32_t)a.g * D * 2);

  char* const w0 = stg0 + wave * STAGE;
  char* const w1 = stg1 + wave * STAGE;

  // paged: the page ids of this chunk's first 64 pages, one per lane, loaded
  // once so that a tile's address needs no memory round trip
  int pg_first = 0, pg_lane = 0;
  if constexpr (PAGED) {
    pg_first = k0 / a.page;
    const int npg = k1 > k0 ? (k1 - 1) / a.page - pg_first + 1 : 0;
    if (lane < npg) pg_lane = a.block_table[(size_t)b * a.max_pages + pg_first + lane];
  }

  auto issue = [&](int i, char* kt, char* vt) {
    const int j0 = k0 + (wave + NWV * i) * BN;
    __amdgpu_buffer_rsrc_t tk = rk, tv = rv;
    int row0 = j0;
    if constexpr (PAGED) {
      // one 32-key tile lies in one page (page is a multiple of 32); rows
      // past this stream's keys read as zeros, and a page id outside the
      // cache is clamped into it
      const int pi = j0 / a.page - pg_first;
      const int id = pi < 64 ? __builtin_amdgcn_readlane(pg_lane, pi)
                             : a.block_table[(size_t)b * a.max_pages + j0 / a.page];
      const int pg = min(max(id, 0), a.num_pages - 1);
      const size_t base = (((size_t)pg * a.Hkv + kvh) * a.page + (j0 % a.page)) * D;
      const uint32_t bytes = (uint32_t)min(BN, k1 - j0) * D * 2;
      tk = make_rsrc(a.k + base, bytes);
      tv = make_rsrc(a.v + base, bytes);
      row0 = 0;
    }
#pragma unroll
    for (int n = 0; n < LOADS; n++) {
      const int p = n * 64 + lane;
      const int r = p / CPR;
      const int cc = (p % CPR) ^ swz<D>(r);
      const uint32_t src = (uint32_t)(((row0 + r) * D + cc * 8) * 2);
      buf_load_lds16_stream(tk, src, (lds_void*)(kt + n * 1024));
      buf_load_lds16_stream(tv, src, (lds_void*)(vt + n * 1024));
    }
  };

  if (my_tiles > 0) issue(0, w0, w0 + TILE_BYTES);

  // query fragments: column l32 is query head kvh*g + l32 (zero beyond g)
  bf16x8 qf[D / 16];
#pragma unroll
  for (int s = 0; s < D / 16; s++)
    qf[s] = __builtin_bit_cast(bf16x8, buf_load16(rq, (uint32_t)((l32 * D + 16 * s + 8 * h32) * 2)));

  f32x16 acc[D / 32];
#pragma unroll
  for (int cb = 0; cb < D / 32; cb++) acc[cb] = f32x16{};
  float m_run = kNegInf, l_run = 0.0f;
  const int swl = swz<D>(l32);

  auto compute = [&](int i, const char* kt, const char* vt) {
    const int j0 = k0 + (wave + NWV * i) * BN;
    f32x16 st = f32x16{};
#pragma unroll
    for (int s = 0; s < D / 16; s++) {
      const bf16x8 kf = *(const bf16x8*)(kt + l32 * (D * 2) + (((2 * s + h32) ^ swl) << 4));
      st = mfma32(kf, qf[s], st);
    }
    if (j0 + BN > k1) {
#pragma unroll
      for (int r = 0; r < 16; r++) {
        const int j = j0 + 8 * (r >> 2) + 4 * h32 + (r & 3);
        if (j >= k1) st[r] = kNegInf;
      }
    }
    float mx = kNegInf;
#pragma unroll
    for (int r = 0; r < 16; r++) mx = fmaxf(mx, st[r]);
    mx = halves_max(mx) * a.c;
    const bool grow = mx > m_run + kTau;
    if (__builtin_amdgcn_ballot_w64(grow)) {
      // lanes that do not grow keep their state (alpha = 1; their m_run may
      // still be -inf); a growing lane with m_run = -inf gets alpha = 0
      const float alpha = grow ? fast_exp2(m_run - mx) : 1.0f;
      m_run = grow ? mx : m_run;
      l_run *= alpha;
#pragma unroll
      for (int cb = 0; cb < D / 32; cb++)
#pragma unroll
        for (int r = 0; r < 16; r++) acc[cb][r] *= alpha;
    }
    const float m_use = (m_run == kNegInf) ? 0.0f : m_run;
#pragma unroll
    for (int r = 0; r < 16; r++) {
      st[r] = fast_exp2(__builtin_fmaf(st[r], a.c, -m_use));
      l_run += st[r];
    }
#pragma unroll
    for (int hf = 0; hf < 2; hf++) {
      bf16x8 pb;
#pragma unroll
      for (int e = 0; e < 8; e++) pb[e] = to_bf16(st[8 * hf + e]);
      const int vr = 16 * hf + 4 * h32 + ((lane & 15) >> 2);
#pragma unroll
      for (int cb = 0; cb < D / 32; cb++) {
        const int vc = cb * 32 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
        const s16x4 lo = ds_read_tr16(vt + tile_off<D>(vr, vc));
        const s16x4 hi = ds_read_tr16(vt + tile_off<D>(vr + 8, vc));
        acc[cb] = mfma32(join_bf16(lo, hi), pb, acc[cb]);
      }
    }
  };

  // one step: prefetch this wave's next tile into the other stage, compute the
  // current one (restrict: the prefetch never writes what the step reads)
  auto step = [&](int i, const char* __restrict__ kc, const char* __restrict__ vc, char* __restrict__ kn,
                  char* __restrict__ vn) {
    wait_vmem();
    if (i + 1 < my_tiles) issue(i + 1, kn, vn);
    compute(i, kc, vc);
  };
  for (int i = 0; i < my_tiles; i += 2) {
    step(i, w0, w0 + TILE_BYTES, w1, w1 + TILE_BYTES);
    if (i + 1 >= my_tiles) break;
    step(i + 1, w1, w1 + TILE_BYTES, w0, w0 + TILE_BYTES);
  }

  // ---- fold the wave states: the monoid rule, through LDS
  const float l_tot = halves_sum(l_run);
  __syncthreads();  // every wave is done with its tile buffers
  float* f_acc = (float*)smem;  // [NWV][g][D]
  float* f_m = f_acc + NWV * 32 * D;  // [NWV][32]
  float* f_l = f_m + NWV * 32;  // [NWV][32]
  if (l32 < a.g) {
#pragma unroll
    for (int cb = 0; cb < D / 32; cb++)
#pragma unroll
      for (int r = 0; r < 16; r++)
        f_acc[(wave * 32 + l32) * D + cb * 32 + 8 * (r >> 2) + 4 * h32 + (r & 3)] = acc[cb][r];
    if (h32 == 0) {
      f_m[wave * 32 + l32] = m_run;
      f_l[wave * 32 + l32] = l_tot;
    }
  }
  __syncthreads();
  const int total = a.g * D;
  for (int e = threadIdx.x; e < total; e += NWV * 64) {
    const int qh = e / D, col = e % D;
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < NWV; w++) M = fmaxf(M, f_m[w * 32 + qh]);
    float L = 0.0f, A = 0.0f;
#pragma unroll
    for (int w = 0; w < NWV; w++) {
      const float mw = f_m[w * 32 + qh];
      const float f = (mw == kNegInf) ? 0.0f : fast_exp2(mw - M);
      L += f * f_l[w * 32 + qh];
      A += f * f_acc[(w * 32 + qh) * D + col];
    }
    const int hq = kvh * a.g + qh;
    const size_t row = (size_t)b * a.Hq + hq;
    if (a.S == 1) {
      a.o[row * D + col] = to_bf16(L > 0.0f ? A / L : 0.0f);
      if (col == 0 && a.lse != nullptr) a.lse[row] = L > 0.0f ? (M + __log2f(L)) * kLn2 : kNegInf;
    } else {
      store_agent(a.part_acc + (row * a.S + split) * D + col, A);
      if (col == 0) {
        store_agent(a.part_ml + (row * a.S + split) * 2 + 0, M);
        store_agent(a.part_ml + (row * a.S + split) * 2 + 1, L);
      }
    }
  }
  if (a.S > 1 && a.counters != nullptr) merge_if_last<D>(a, b, kvh, pair);
}

// ---------------------------------------------------------------------------
// Split-KV decode over an FP8 (OCP E4M3) KV cache with a scale per kv head.
// Same decomposition and fold as the bf16 kernel; K and V move HBM -> LDS as
// bytes (half the traffic) through a ring of LDS stages per wave, and are
// widened to bf16 in registers
// just before the MFMAs, which is exact.  The K scale folds into the exponent
// scale and the V scale into the accumulator, so the arithmetic after the
// loads is the bf16 kernel's.
//   K (A operand of S^T = K Q^T): lane l reads bytes 16 s + 8 h .. +8 of key
//   row l % 32 (h = l / 32).
//   V^T (A operand of O^T += V^T P^T): one transposed byte read per MFMA; the
//   rows each lane addresses are chosen so that the keys land in the order
//   P^T uses (key slot 8 h + b of a 16-key half is key 4 h + b % 4 + 8 (b / 4)).
// LDS tiles are [32 keys][D bytes] with 16-byte chunk c of row r stored at
// chunk c ^ (r % (D / 16)).
template <int D>
__global__ __launch_bounds__(kWaves * 64, 1) void decode_partial_fp8_kernel(DecArgs a) {
  constexpr int BN = kDecodeTile;
  constexpr int TILE = BN * D;           // bytes of one K or V tile
  constexpr int NST = ATTN_DECODE_FP8_STAGES;  // stages per wave
  constexpr int STAGE = 2 * TILE;        // K then V
  constexpr int CPR = D / 16;            // 16-byte chunks per row
  constexpr int LOADS = BN * CPR / 64;   // per lane per K (or V) tile
  constexpr int VMT = 2 * LOADS;         // loads per wave per tile
  static_assert(BN == 32, "one 32-key MFMA block per tile");
  static_assert(LOADS * 64 == BN * CPR, "tile must split evenly over a wave");
  constexpr int FOLD = kWaves * 32 * D * 4 + 2 * kWaves * 32 * 4;  // the fold's area, reusing the tiles'
  constexpr int SMEM = kWaves * NST * STAGE > FOLD ? kWaves * NST * STAGE : FOLD;
  __shared__ __attribute__((aligned(1024))) char smem[SMEM];

  const int lane = threadIdx.x & 63;
  const int wave = wave_id();
  const int h32 = lane >> 5;
  const int l32 = lane & 31;

  const int work = xcd_remap(blockIdx.x, a.n_wgs);
  const int split = work % a.S;
  const int pair = work / a.S;
  const int b = pair / a.Hkv;
  const int kvh = pair % a.Hkv;

  const int k0 = split * a.chunk;
  const int k1 = min(a.Nk, k0 + a.chunk);
  const int n_tiles = k1 > k0 ? (k1 - k0 + BN - 1) / BN : 0;
  const int my_tiles = n_tiles > wave ? (n_tiles - wave + kWaves - 1) / kWaves : 0;

  const size_t kv_head = ((size_t)b * a.Hkv + kvh) * (size_t)a.Nk * D;
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(a.k8 + kv_head, (uint32_t)a.Nk * D);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(a.v8 + kv_head, (uint32_t)a.Nk * D);
  const size_t q_grp = ((size_t)b * a.Hq + (size_t)kvh * a.g) * D;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(a.q + q_grp, (uint32_t)a.g * D * 2);
  const float c = a.c * a.k_scale[kvh];
  const float vscale = a.v_scale[kvh];

  char* wbase = smem + wave * NST * STAGE;
  auto stage_of = [&](int i) { return wbase + (i % NST) * STAGE; };

  auto issue = [&](int i) {
    char* kt = stage_of(i);
    char* vt = kt + TILE;
    const int j0 = k0 + (wave + kWaves * i) * BN;
#pragma unroll
    for (int n = 0; n < LOADS; n++) {
      const int p = n * 64 + lane;
      const int r = p / CPR;
      const int cc = (p % CPR) ^ (r % CPR);
      const uint32_t src = (uint32_t)((j0 + r) * D + cc * 16);
      buf_load_lds16_stream(rk, src, (lds_void*)(kt + n * 1024));
      buf_load_lds16_stream(rv, src, (lds_void*)(vt + n * 1024));
    }
  };

  // tile 0, this wave's queries, then the other tiles in flight: each wait
  // below counts only tile loads issued after the tile it waits for
  if (my_tiles > 0) issue(0);
  bf16x8 qf[D / 16];
#pragma unroll
  for (int s = 0; s < D / 16; s++)
    qf[s] = __builtin_bit_cast(bf16x8, buf_load16(rq, (uint32_t)((l32 * D + 16 * s + 8 * h32) * 2)));
  for (int i = 1; i < NST - 1 && i < my_tiles; i++) issue(i);

  f32x16 acc[D / 32];
#pragma unroll
  for (int cb = 0; cb < D / 32; cb++) acc[cb] = f32x16{};
  float m_run = kNegInf, l_run = 0.0f;

  // lane-constant byte offsets: K (row l32, chunk s, half h32); V^T (rows and
  // columns of the transposed read for 16-key half hf and d block cb)
  const int g16 = lane >> 4, u = lane & 15;
  auto k_off = [&](int s) { return l32 * D + (((s ^ (l32 % CPR)) << 4)) + 8 * h32; };
  auto v_off = [&](int hf, int cb) {
    const int row = 16 * hf + 4 * (g16 >> 1) + ((u >> 1) & 3) + 8 * (u >> 3);
    const int chunk = 2 * cb + (g16 & 1);
    return row * D + ((chunk ^ (row % CPR)) << 4) + 8 * (u & 1);
  };

  auto compute = [&](int i, const char* kt, const char* vt) {
    const int j0 = k0 + (wave + kWaves * i) * BN;
    f32x16 st = f32x16{};
#pragma unroll
    for (int s = 0; s < D / 16; s++) {
      const i32x2 w = *(const i32x2*)(kt + k_off(s));
      st = mfma32(fp8x8_to_bf16(w), qf[s], st);
    }
    if (j0 + BN > k1) {
#pragma unroll
      for (int r = 0; r < 16; r++) {
        const int j = j0 + 8 * (r >> 2) + 4 * h32 + (r & 3);
        if (j >= k1) st[r] = kNegInf;
      }
    }
    float mx = kNegInf;
#pragma unroll
    for (int r = 0; r < 16; r++) mx = fmaxf(mx, st[r]);
    mx = halves_max(mx) * c;
    const bool grow = mx > m_run + kTau;
    if (__builtin_amdgcn_ballot_w64(grow)) {
      const float alpha = grow ? fast_exp2(m_run - mx) : 1.0f;
      m_run = grow ? mx : m_run;
      l_run *= alpha;
#pragma unroll
      for (int cb = 0; cb < D / 32; cb++)
#pragma unroll
        for (int r = 0; r < 16; r++) acc[cb][r] *= alpha;
    }
    const float m_use = (m_run == kNegInf) ? 0.0f : m_run;
#pragma unroll
    for (int r = 0; r < 16; r++) {
      st[r] = fast_exp2(__builtin_fmaf(st[r], c, -m_use));
      l_run += st[r];
    }
#pragma unroll
    for (int hf = 0; hf < 2; hf++) {
      bf16x8 pb;
#pragma unroll
      for (int e = 0; e < 8; e++) pb[e] = to_bf16(st[8 * hf + e]);
#pragma unroll
      for (int cb = 0; cb < D / 32; cb++)
        acc[cb] = mfma32(fp8x8_to_bf16(ds_read_tr8(vt + v_off(hf, cb))), pb, acc[cb]);
    }
  };

  for (int i = 0; i < my_tiles; i++) {
    const int ahead = min(NST - 2, my_tiles - 1 - i);  // younger tiles already in flight
    if (ahead >= 2)
      wait_vmem_n<2 * VMT>();
    else if (ahead == 1)
      wait_vmem_n<VMT>();
    else
      wait_vmem();
    // the stage of tile i + NST - 1 was tile i - 1's, whose reads are done
    if (i + NST - 1 < my_tiles) issue(i + NST - 1);
    const char* kt = stage_of(i);
    compute(i, kt, kt + TILE);
  }
#pragma unroll
  for (int cb = 0; cb < D / 32; cb++)
#pragma unroll
    for (int r = 0; r < 16; r++) acc[cb][r] *= vscale;

  // ---- fold the wave states: the monoid rule, through LDS
  const float l_tot = halves_sum(l_run);
  __syncthreads();  // every wave is done with its tile buffers
  float* f_acc = (float*)smem;           // [kWaves][32][D]
  float* f_m = f_acc + kWaves * 32 * D;  // [kWaves][32]
  float* f_l = f_m + kWaves * 32;        // [kWaves][32]
  if (l32 < a.g) {
#pragma unroll
    for (int cb = 0; cb < D / 32; cb++)
#pragma unroll
      for (int r = 0; r < 16; r++)
        f_acc[(wave * 32 + l32) * D + cb * 32 + 8 * (r >> 2) + 4 * h32 + (r & 3)] = acc[cb][r];
    if (h32 == 0) {
      f_m[wave * 32 + l32] = m_run;
      f_l[wave * 32 + l32] = l_tot;
    }
  }
  __syncthreads();
  const int total = a.g * D;
  for (int e = threadIdx.x; e < total; e += kWaves * 64) {
    const int qh = e / D, col = e % D;
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < kWaves; w++) M = fmaxf(M, f_m[w * 32 + qh]);
    float L = 0.0f, A = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; w++) {
      const float mw = f_m[w * 32 + qh];
      const float f = (mw == kNegInf) ? 0.0f : fast_exp2(mw - M);
      L += f * f_l[w * 32 + qh];
      A += f * f_acc[(w * 32 + qh) * D + col];
    }
    const int hq = kvh * a.g + qh;
    const size_t row = (size_t)b * a.Hq + hq;
    if (a.S == 1) {
      a.o[row * D + col] = to_bf16(L > 0.0f ? A / L : 0.0f);
      if (col == 0 && a.lse != nullptr) a.lse[row] = L > 0.0f ? (M + __log2f(L)) * kLn2 : kNegInf;
    } else {
      store_agent(a.part_acc + (row * a.S + split) * D + col, A);
      if (col == 0) {
        store_agent(a.part_ml + (row * a.S + split) * 2 + 0, M);
        store_agent(a.part_ml + (row * a.S + split) * 2 + 1, L);
      }
    }
  }
  if (a.S > 1 && a.counters != nullptr) merge_if_last<D>(a, b, kvh, pair);
}

// Fold num_splits partial states per (b, query head).  One wave per row.
template <int D>
__global__ __launch_bounds__(256) void decode_merge_kernel(DecArgs a) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= a.B * a.Hq) return;
#pragma unroll
  for (int e = 0; e < D / 64; e++) fold_split_states<D, false>(a, (size_t)row, e * 64 + lane);
}

template <int D>
hipError_t launch(const DecodeProblem& p, hipStream_t s) {
  DecArgs a;
  a.q = (const __bf16*)p.q;
  a.k = (const __bf16*)p.k;
  a.v = (const __bf16*)p.v;
  a.o = (__bf16*)p.o;
  a.lse = p.lse;
  a.part_acc = p.part_acc;
  a.part_ml = p.part_ml;
  a.B = (int)p.B;
  a.Hq = (int)p.Hq;
  a.Hkv = (int)p.Hkv;
  a.Nk = (int)p.Nk;
  a.g = a.Hq / a.Hkv;
  a.S = p.num_splits;
  a.chunk = p.chunk;
  a.n_wgs = a.B * a.Hkv * a.S;
  a.c = p.scale * kLog2e;
  a.k8 = p.k8;
  a.v8 = p.v8;
  a.k_scale = p.k_scale;
  a.v_scale = p.v_scale;
  a.counters = p.counters;
  a.block_table = p.block_table;
  a.seq_lens = p.seq_lens;
  a.page = (int)p.page;
  a.max_pages = (int)p.max_pages;
  a.num_pages = (int)p.num_pages;
  // Dense bf16 caches: 4-wave workgroups (one per CU) while the grid fits the
  // 256 CUs; beyond that 2-wave workgroups, two per CU, so that the whole
  // grid starts at once instead of in one and a half rounds (48 streams x 8
  // kv heads: 2-10 % faster at 512..4096 keys; 2-wave workgroups on a grid of
  // at most 256 leave half the CU slots empty and measured 2-16 % slower).
  // Paged caches keep 4 waves: their streams differ in length, the longest
  // chunks (launched first) decide the end, and a 2-wave workgroup streams a
  // chunk at half the rate (48 streams of 512..4096 keys: 103.9 against 92.7
  // us in one chunk, 96.8 in two).
  const bool two = a.n_wgs > 256;
  if (p.block_table != nullptr) {
    hipLaunchKernelGGL((decode_partial_kernel<D, true, 4>), dim3(a.n_wgs), dim3(256), 0, s, a);
  } else if (p.k8 != nullptr) {
    hipLaunchKernelGGL((decode_partial_fp8_kernel<D>), dim3(a.n_wgs), dim3(kWaves * 64), 0, s, a);
  } else if (two) {
    hipLaunchKernelGGL((decode_partial_kernel<D, false, 2>), dim3(a.n_wgs), dim3(128), 0, s, a);
  } else {
    hipLaunchKernelGGL((decode_partial_kernel<D, false, 4>), dim3(a.n_wgs), dim3(256), 0, s, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.S == 1 || a.counters != nullptr) return e;
  const int rows = a.B * a.Hq;
  hipLaunchKernelGGL((decode_merge_kernel<D>), dim3((rows + 3) / 4), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

// Fixed scratch for the decode entry point that allocates nothing: the
// partial states of its split plan live here instead of in a caller
// workspace.  Each GPU the library runs on holds its own copy until the
// process ends, and every call on that GPU shares it, so calls that overlap
// on one GPU race (stream order keeps them apart).  Host code never uses the
// array's name as an address: decode_scratch() looks the device address up.
static __device__ __attribute__((aligned(256))) char scratch[kDecodeScratchBytes];

hipError_t launch_decode(const DecodeProblem& p, hipStream_t s) {
  return p.d == 128 ? launch<128>(p, s) : launch<64>(p, s);
}

hipError_t decode_scratch(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    // once per device, with that device current: each device's copy of the
    // array sits at its own address
    void* a = nullptr;
    e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = a;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

}  // namespace attn
