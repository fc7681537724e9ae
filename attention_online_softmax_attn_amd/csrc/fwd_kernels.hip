// Forward prefill kernels for gfx950.
//
// One workgroup owns BM = 32 * NW consecutive query rows of one query head;
// each wave owns 32 of them.  Key/value tiles of BN rows stream HBM -> LDS by
// direct-to-LDS buffer loads into two alternating buffers, so the loads of
// tile t+1 overlap the MFMA work of tile t.  Per tile and wave:
//
//   S^T = K Q^T  on v_mfma_f32_32x32x16_bf16 (keys are the M dimension, so a
//                lane holds 16 keys of one query and the softmax statistics of
//                that query stay lane-local; the other 16 keys of the same
//                32-key block sit in lane ^ 32)
//   online softmax: m' = max(m, rowmax * c), p = 2^(s c - m'), l' = l 2^(m - m') + sum p
//                (c = scale * log2 e; the max needs one permlane32 swap, the
//                sum stays per lane until the epilogue)
//   O^T += V^T P^T  on the same MFMA; P^T goes from the accumulator layout to
//                the B operand without leaving registers (the key order inside
//                the contraction is permuted identically on both operands)
//                and V^T is read with the LDS transpose read.
//
// The running state (m, l, acc) is the monoid of the online softmax ("Não
// escreva kernels, derive-os", section "Aprofundamento", first paragraph);
// the fold over key tiles is its left fold.  Causal key tiles above a
// workgroup's diagonal are never loaded; a wave skips the MFMA work of tiles
// above its own diagonal; only tiles crossing a diagonal (or the end of the
// keys) are masked elementwise.  The rescale of acc is skipped while the row
// maximum has grown by less than kTau (log2 units): the final acc / l and
// LSE = (m + log2 l) ln 2 are exact for any m used consistently.
#include <type_traits>

#include "device_common.hpp"
#include "kernels.h"

namespace attn {

namespace {

constexpr float kTau = 8.0f;

struct FwdArgs {
  const __bf16* q;
  const __bf16* k;
  const __bf16* v;
  __bf16* o;
  float* lse;
  int B, Hq, Hkv, Nq, Nk, g;
  int n_qtiles, n_wgs;
  // 1: the whole grid is resident at once (two workgroups per CU): the first
  // half of each XCD's dispatch order takes the heaviest tiles first and the
  // second half the lightest first, so that the tiles a CU starts with tend
  // to add up evenly (1.7-2.5 % faster at N = 2048; the dispatcher does not
  // place the two halves slot by slot, or the gain would be larger)
  int snake;
  float c;  // scale * log2(e)
  // packed variable-length batch (null for a dense one): sequence b holds
  // query rows [cu_q[b], cu_q[b+1]) of q, o and lse and key rows
  // [cu_k[b], cu_k[b+1]) of k and v; every head is [tot_q or tot_k, D]
  const int* cu_q;
  const int* cu_k;
  int tot_q, tot_k;
  // paged K, V (with cu_q): [num_pages, Hkv, page, D]; key j of sequence b
  // is slot j % page of page block_table[b][j / page]; sequence b has
  // seq_lens_k[b] keys (cu_k unused)
  const int* block_table;
  const int* seq_lens_k;
  int page, max_pages, num_pages;
};

// Launch index -> the index lpt_order ranks: within each XCD (launch index
// mod 8) the first half of the dispatch order keeps the heaviest-first
// ranks and the second half takes the remaining ranks lightest first.  A
// bijection on [0, n) for n a multiple of 8.
__device__ __forceinline__ int snake_pid(int pid, int n, int on) {
  if (!on) return pid;
  const int T = n / 8, half = (T + 1) / 2, x = pid % 8, t = pid / 8;
  return x + 8 * (t < half ? t : T - 1 - (t - half));
}

// 1: causal query tiles end at the last query row (tile t of T covers rows
// Lq - BM (T - t) .. Lq - BM (T - 1 - t) - 1), so that the rows a ragged
// length leaves over pad the first tile, which streams the fewest keys, not
// the last, which streams them all.  Rows before 0 are padding: their Q row
// is row 0's, their mask row 0's, and they are never stored.  Each stored
// row sees the same key tiles in the same order either way.
// 1: the two-group kernel stores O through LDS, four whole rows per store
// instruction, instead of 16-byte pieces of 32 rows (0); 2: the same with
// non-temporal stores
#ifndef ATTN_FWD_O_STAGE
#define ATTN_FWD_O_STAGE 1
#endif
#ifndef ATTN_FWD_END_ALIGN
#define ATTN_FWD_END_ALIGN 1
#endif
constexpr bool kEndAlign = ATTN_FWD_END_ALIGN != 0;

// first query row of tile qt of a slice of Nq rows
template <int BM, bool CAUSAL>
__device__ __forceinline__ int qtile_row0(int qt, int Nq) {
  if constexpr (CAUSAL && kEndAlign) return Nq - ((Nq + BM - 1) / BM - qt) * BM;
  return qt * BM;
}

// Packed variable-length batch: the work item (sequence, query tile, query
// head) of launch index `rank` in a longest-first order, computed by every
// wave from the sequence offsets alone (no workspace, no host round trip).
// An item's weight is the number of BN-key tiles its workgroup streams, the
// kernel's own count: when causal, with tile t of T ending at row e_t
// (qtile_row0), W(s, t) = ceil(min(Lk, e_t + Lk - Lq) / BN) (at least 0), which
// is ceil((Lk - BM (T - 1 - t)) / BN) for end-aligned tiles; ceil(Lk / BN)
// otherwise.  It does not decrease with t, so for a threshold w the items of
// sequence s with W >= w are its last c_s(w) tiles, c_s(w) in closed form, and
// the weight of rank r is found by a binary search on w over sum_s c_s(w);
// ties go in (sequence, tile) order.
// Within an item the Hq heads take consecutive ranks, kv head first
// (j -> kv head j % Hkv), so that the dispatcher, which sends launch index i
// to XCD i % 8, keeps the query heads of one kv head together when Hkv is 8.
// Returns false for a rank past the last item.
template <int BM, int BN, bool CAUSAL, bool PAGED>
__device__ bool varlen_item(const FwdArgs& a, int rank, int& s_out, int& qt_out, int& h_out) {
  // the kernel's own clamped per-sequence sizes (Lq, Lk)
  auto size = [&](int s) -> int2 {
    const int q1 = min(a.cu_q[s + 1], a.tot_q), q0 = max(0, min(a.cu_q[s], q1));
    if constexpr (PAGED) {
      return make_int2(q1 - q0, min(max(a.seq_lens_k[s], 0), min(a.Nk, a.max_pages * a.page)));
    } else {
      const int k1 = min(a.cu_k[s + 1], a.tot_k), k0 = max(0, min(a.cu_k[s], k1));
      return make_int2(q1 - q0, k1 - k0);
    }
  };
  // items of one sequence whose weight is at least w
  auto count = [&](int2 sz, int w) -> int {
    const int lq = sz.x, lk = sz.y;
    const int n = (lq + BM - 1) / BM;
    if (w <= 0) return n;
    const int x = (w - 1) * BN;  // W >= w  <=>  the streamed keys exceed x
    if (lk <= x) return 0;
    if (!CAUSAL) return n;
    if constexpr (kEndAlign) return min(n, (lk - x + BM - 1) / BM);  // tile n - 1 - j streams Lk - BM j keys
    const int t = x - (lk - lq);  // need min((qt + 1) BM, Lq) > t
    if (lq <= t) return 0;
    return n - (t < 0 ? 0 : t / BM);
  };
  int2 sz;
  int c_lo, c_lo1, k, j;
  if (!lpt_place<4>(a.B, a.Hq, rank, a.Nk / BN + 2, size, count, s_out, sz, c_lo, c_lo1, k, j)) return false;
  // the items of weight >= w are a sequence's last count(w) tiles
  qt_out = (sz.x + BM - 1) / BM - c_lo + k;
  // within an item the Hq heads take consecutive ranks, kv head first
  const int g = a.Hq / a.Hkv;
  h_out = (j % a.Hkv) * g + j / a.Hkv;
  return true;
}

template <int D, int NW, int BN, bool CAUSAL, bool PAGED = false>
__global__ __launch_bounds__(NW * 64, 8 / NW) void fwd_bf16_kernel(FwdArgs a) {
  constexpr int BM = NW * 32;
  constexpr int TILE_BYTES = BN * D * 2;       // one K or V tile
  constexpr int CPR = D / 8;                   // 16-byte chunks per row
  constexpr int LOADS = BN * CPR / (64 * NW);  // direct-to-LDS loads per thread per tile
  constexpr int KS = 64;                       // keys per sub-tile (the unit of S, softmax and PV)
  constexpr int KB = KS / 32;                  // 32-key blocks per sub-tile
  static_assert(LOADS * 64 * NW == BN * CPR, "tile must split evenly over the workgroup");
  static_assert(BN % KS == 0, "BN must be a multiple of 64");
  // the paged cache's pages are whole multiples of 64 keys (checked by the C
  // ABI), so a 64-key tile never straddles two pages; a larger tile could
  static_assert(!PAGED || BN == 64, "paged key tiles must be 64 keys");
  static_assert(TILE_BYTES <= 65536, "LDS offsets must fit the 16-bit immediate");

  // Two stages of one K and one V tile each; tile t uses stage t % 2.  Every
  // tile buffer is its own LDS object: the compiler then proves that the
  // prefetch into one stage does not alias the reads of the other (with
  // offsets into one array it waits for the prefetch in flight before the
  // transposed V reads).  Reads address K through koff and V through voff;
  // the sub-tile, key block and row half go into the instructions' immediate
  // offset.
  __shared__ __attribute__((aligned(1024))) char k_st0[TILE_BYTES], k_st1[TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char v_st0[TILE_BYTES], v_st1[TILE_BYTES];

  const int lane = threadIdx.x & 63;
  const int wave = wave_id();
  const int h32 = lane >> 5;
  const int l32 = lane & 31;

  // ---- work decomposition.  Dense: (b, kv head) pair, then q tile
  // (descending when causal) and head in group.  Packed batch: the
  // sequences differ in length, so the launch order follows each item's
  // own weight, longest first (varlen_item).
  int qt, hq, b, kvh;
  if (a.cu_q != nullptr) {
    if (!varlen_item<BM, BN, CAUSAL, PAGED>(a, (int)blockIdx.x, b, qt, hq)) return;
    kvh = hq / a.g;
  } else {
    const WorkItem wi = lpt_order(snake_pid(blockIdx.x, a.n_wgs, a.snake), a.B * a.Hkv, a.g * a.n_qtiles);
    const int rem = wi.sub;
    qt = CAUSAL ? (a.n_qtiles - 1 - rem / a.g) : (rem / a.g);
    hq = (wi.pair % a.Hkv) * a.g + rem % a.g;
    b = wi.pair / a.Hkv;
    kvh = wi.pair % a.Hkv;
  }

  // this (batch or sequence, head) slice: its sizes and element offsets
  int Nq = a.Nq, Nk = a.Nk;
  size_t q_head, kv_head, lse_row;
  if (a.cu_q != nullptr) {
    // clamped, so that offsets that do not describe a packed batch cannot
    // take a load outside q, k or v
    const int q1 = min(a.cu_q[b + 1], a.tot_q), q0 = max(0, min(a.cu_q[b], q1));
    Nq = q1 - q0;
    q_head = ((size_t)hq * a.tot_q + q0) * D;
    lse_row = (size_t)hq * a.tot_q + q0;
    if constexpr (PAGED) {
      Nk = min(max(a.seq_lens_k[b], 0), min(a.Nk, a.max_pages * a.page));
      kv_head = 0;
    } else {
      const int k1 = min(a.cu_k[b + 1], a.tot_k), k0 = max(0, min(a.cu_k[b], k1));
      Nk = k1 - k0;
      kv_head = ((size_t)kvh * a.tot_k + k0) * D;
    }
  } else {
    q_head = ((size_t)b * a.Hq + hq) * (size_t)Nq * D;
    kv_head = ((size_t)b * a.Hkv + kvh) * (size_t)Nk * D;
    lse_row = ((size_t)b * a.Hq + hq) * (size_t)Nq;
  }
  const int i0 = qtile_row0<BM, CAUSAL>(qt, Nq);
  const int qw0 = i0 + wave * 32;
  // rows before 0 pad the first tile: they take row 0's Q and mask
  constexpr bool LEAD_PAD = CAUSAL && kEndAlign;
  auto lo_row = [](int r) { return LEAD_PAD ? max(r, 0) : r; };
  if (i0 >= Nq) return;  // the whole workgroup: a tile past this sequence's queries
  const int off = Nk - Nq;  // causal: key j visible to query i iff j <= i + off

  const __amdgpu_buffer_rsrc_t rq = make_rsrc(a.q + q_head, (uint32_t)Nq * D * 2);
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(a.k + kv_head, (uint32_t)Nk * D * 2);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(a.v + kv_head, (uint32_t)Nk * D * 2);

  int kend = Nk;
  if (CAUSAL) {
    int last_row = min(i0 + BM, Nq) - 1;
    kend = min(Nk, last_row + off + 1);
  }
  const int n_tiles = kend > 0 ? (kend + BN - 1) / BN : 0;

  // paged: the page ids of the first 64 pages, one per lane, loaded once so
  // that a tile's address needs no memory round trip
  int pg_lane = 0;
  if constexpr (PAGED) {
    if (lane < (kend + a.page - 1) / a.page) pg_lane = a.block_table[(size_t)b * a.max_pages + lane];
  }

  // ---- issue the direct-to-LDS loads of tile t into the K/V buffers kt, vt
  auto issue = [&](int t, char* kt, char* vt) {
    const int j0 = t * BN;
    __amdgpu_buffer_rsrc_t tk = rk, tv = rv;
    int row0 = j0;
    if constexpr (PAGED) {
      // a tile lies in one page (page is a multiple of BN); rows past the
      // sequence's keys read as zeros, and a page id outside the cache is
      // clamped into it
      const int pi = j0 / a.page;
      const int id = pi < 64 ? __builtin_amdgcn_readlane(pg_lane, pi)
                             : a.block_table[(size_t)b * a.max_pages + pi];
      const int pg = min(max(id, 0), a.num_pages - 1);
      const size_t base = (((size_t)pg * a.Hkv + kvh) * a.page + (j0 % a.page)) * D;
      const uint32_t bytes = (uint32_t)min(BN, Nk - j0) * D * 2;
      tk = make_rsrc(a.k + base, bytes);
      tv = make_rsrc(a.v + base, bytes);
      row0 = 0;
    }
#pragma unroll
    for (int n = 0; n < LOADS; n++) {
      const int slab = n * NW + wave;  // 64 consecutive 16-byte LDS chunks
      const int p = slab * 64 + lane;
      const int r = p / CPR;
      const int c = (p % CPR) ^ swz<D>(r);
      const uint32_t src = (uint32_t)(((row0 + r) * D + c * 8) * 2);
      buf_load_lds16(tk, src, (lds_void*)(kt + slab * 1024));
      buf_load_lds16(tv, src, (lds_void*)(vt + slab * 1024));
    }
  };

  if (n_tiles > 0) issue(0, k_st0, v_st0);

  // ---- Q fragments (B operand of S^T = K Q^T): row qw0 + l32, dims 16s + 8h .. +8
  bf16x8 qf[D / 16];
#pragma unroll
  for (int s = 0; s < D / 16; s++) {
    const uint32_t src = (uint32_t)((lo_row(qw0 + l32) * D + 16 * s + 8 * h32) * 2);
    qf[s] = __builtin_bit_cast(bf16x8, buf_load16(rq, src));
  }

  // ---- lane-constant LDS byte offsets inside a K or V tile.  The buffer, the
  // 32-key block and the 16-row half only add multiples of 16 rows, which
  // leave the swizzle unchanged, so they go into the instructions' immediate
  // offsets and the tile loop does no address arithmetic.
  const int swl = swz<D>(l32);
  int koff[D / 16];  // A operand of S^T: key row l32, column chunk 2s + h
#pragma unroll
  for (int s = 0; s < D / 16; s++) koff[s] = l32 * (D * 2) + (((2 * s + h32) ^ swl) << 4);
  int voff[D / 32][2];  // transposed V reads: rows 4h + (lane%16)/4 (+8), columns of block cb
#pragma unroll
  for (int cb = 0; cb < D / 32; cb++)
#pragma unroll
    for (int lh = 0; lh < 2; lh++)
      voff[cb][lh] = tile_off<D>(4 * h32 + ((lane & 15) >> 2) + 8 * lh, cb * 32 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3));

  f32x16 acc[D / 32];
#pragma unroll
  for (int cb = 0; cb < D / 32; cb++) acc[cb] = f32x16{};
  float m_run = kNegInf;  // log2-domain running max used for the exponentials
  float l_run = 0.0f;     // this lane's share of the running sum
  const int qi = qw0 + l32;

  // one 64-key sub-tile at key offset 64 * SUB of tile t, whose K and V sit
  // in kcur and vcur
  auto compute_sub = [&](int t, auto sub, const char* __restrict__ kcur, const char* __restrict__ vcur) {
    constexpr int SUB = decltype(sub)::value;
    const char* kt = kcur + SUB * KS * (D * 2);
    const char* vt = vcur + SUB * KS * (D * 2);
    const int j0 = t * BN + SUB * KS;
    // wave-level classification of the sub-tile
    if (j0 >= Nk || qw0 >= Nq || (LEAD_PAD && qw0 + 31 < 0)) return;  // past the keys, or a wave of padding rows
    bool need_mask = (j0 + KS > Nk);
    if (CAUSAL) {
      if (j0 > qw0 + 31 + off) return;               // nothing visible to this wave
      if (j0 + KS - 1 > qw0 + off) need_mask = true;  // crosses this wave's diagonal
    }
    // S^T = K Q^T
    f32x16 st[KB];
#pragma unroll
    for (int kb = 0; kb < KB; kb++) st[kb] = f32x16{};
#pragma unroll
    for (int s = 0; s < D / 16; s++) {
#pragma unroll
      for (int kb = 0; kb < KB; kb++) {
        const bf16x8 kf = *(const bf16x8*)(kt + koff[s] + kb * 32 * (D * 2));
        st[kb] = mfma32(kf, qf[s], st[kb]);
      }
    }
    if (need_mask) {
      // key j = j0 + 4h + c (c = kb*32 + 8(r/4) + r%4, a constant per
      // element) is visible iff j < Nk and, causal, j <= qi + off: one lane
      // bound lim on c, so each element costs one compare with a constant
      const int lim = (CAUSAL ? min(Nk, lo_row(qi) + off + 1) : Nk) - j0 - 4 * h32;
#pragma unroll
      for (int kb = 0; kb < KB; kb++)
#pragma unroll
        for (int r = 0; r < 16; r++)
          if (!(kb * 32 + 8 * (r >> 2) + (r & 3) < lim)) st[kb][r] = kNegInf;
    }
    // online softmax.  P goes to bf16 (the MFMA operand); the row sum adds the
    // fp32 values (a sum of the bf16 values would move LSE by up to 2^-9 on
    // short rows).  Fast path: once every row of the wave has a
    // running max, exponentiate against it directly and accept the tile if no
    // lane's sum exceeds 2^16 (so no P exceeds it either); only otherwise take
    // the row max and rescale (the exact slow path below).
    bf16x8 pb[KB][2];
    float psum = 0.0f;
    bool fast = __builtin_amdgcn_ballot_w64(m_run == kNegInf) == 0;
    if (fast) {
#pragma unroll
      for (int kb = 0; kb < KB; kb++)
#pragma unroll
        for (int hf = 0; hf < 2; hf++) {
#pragma unroll
          for (int e = 0; e < 8; e++) {
            const float p = fast_exp2(__builtin_fmaf(st[kb][8 * hf + e], a.c, -m_run));
            pb[kb][hf][e] = to_bf16(p);
            psum += p;
          }
        }
      fast = __builtin_amdgcn_ballot_w64(!(psum <= 65536.0f)) == 0;
    }
    if (!fast) {
      float mx = kNegInf;
#pragma unroll
      for (int kb = 0; kb < KB; kb++)
#pragma unroll
        for (int r = 0; r < 16; r++) mx = fmaxf(mx, st[kb][r]);
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
      psum = 0.0f;
#pragma unroll
      for (int kb = 0; kb < KB; kb++)
#pragma unroll
        for (int hf = 0; hf < 2; hf++) {
#pragma unroll
          for (int e = 0; e < 8; e++) {
            const float p = fast_exp2(__builtin_fmaf(st[kb][8 * hf + e], a.c, -m_use));
            pb[kb][hf][e] = to_bf16(p);
            psum += p;
          }
        }
    }
    l_run += psum;
    // O^T += V^T P^T, 16 keys per MFMA
#pragma unroll
    for (int kb = 0; kb < KB; kb++)
#pragma unroll
      for (int hf = 0; hf < 2; hf++) {
        const char* vk = vt + (kb * 32 + 16 * hf) * (D * 2);
#pragma unroll
        for (int cb = 0; cb < D / 32; cb++) {
          const s16x4 lo = ds_read_tr16(vk + voff[cb][0]);
          const s16x4 hi = ds_read_tr16(vk + voff[cb][1]);
          acc[cb] = mfma32(join_bf16(lo, hi), pb[kb][hf], acc[cb]);
        }
      }
  };

  auto compute = [&](int t, const char* __restrict__ kcur, const char* __restrict__ vcur) {
    compute_sub(t, std::integral_constant<int, 0>{}, kcur, vcur);
    if constexpr (BN / KS > 1) compute_sub(t, std::integral_constant<int, 1>{}, kcur, vcur);
    static_assert(BN / KS <= 2, "at most two sub-tiles");
  };

  // ---- one pipeline step: wait until tile t has landed, barrier, prefetch
  // tile t+1 into the other stage, compute tile t.  kc, vc: the K and V
  // tiles of this step's stage; kn, vn: the other stage.
  auto step = [&](int t, const char* __restrict__ kc, const char* __restrict__ vc, char* __restrict__ kn,
                  char* __restrict__ vn) {
    wait_vmem();
    __syncthreads();
    if (t + 1 < n_tiles) issue(t + 1, kn, vn);
    compute(t, kc, vc);
  };
  for (int t = 0; t < n_tiles; t += 2) {
    step(t, k_st0, v_st0, k_st1, v_st1);
    if (t + 1 >= n_tiles) break;
    step(t + 1, k_st1, v_st1, k_st0, v_st0);
  }

  // ---- epilogue: O = acc / l, LSE = (m + log2 l) ln 2
  const float l_tot = halves_sum(l_run);
  const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
  if ((!LEAD_PAD || qi >= 0) && qi < Nq) {
    __bf16* orow = a.o + q_head + (size_t)qi * D;
#pragma unroll
    for (int cb = 0; cb < D / 32; cb++)
#pragma unroll
      for (int g4 = 0; g4 < 4; g4++) {
        bf16x4 w;
#pragma unroll
        for (int e = 0; e < 4; e++) w[e] = to_bf16(acc[cb][4 * g4 + e] * inv);
        *(bf16x4*)(orow + cb * 32 + 8 * g4 + 4 * h32) = w;
      }
    if (a.lse != nullptr && h32 == 0) {
      a.lse[lse_row + qi] = l_tot > 0.0f ? (m_run + __log2f(l_tot)) * kLn2 : kNegInf;
    }
  }
}

// ---------------------------------------------------------------------------
// fp32 forward.  Same decomposition with one wave per workgroup (32 query
// rows) and 32-key tiles staged through LDS; contractions on
// v_mfma_f32_32x32x2_f32, so scores, P and the accumulator stay fp32.
struct FwdArgsF32 {
  const float* q;
  const float* k;
  const float* v;
  float* o;
  float* lse;
  int B, Hq, Hkv, Nq, Nk, g;
  int n_qtiles, n_wgs;
  float c;
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(64) void fwd_f32_kernel(FwdArgsF32 a) {
  constexpr int BN = 32;
  constexpr int LD = D + 1;  // padded row pitch (floats)
  __shared__ float kt[BN * LD];
  __shared__ float vt[BN * LD];
  const int lane = threadIdx.x;
  const int h32 = lane >> 5;
  const int l32 = lane & 31;

  const WorkItem wi = lpt_order(blockIdx.x, a.B * a.Hkv, a.g * a.n_qtiles);
  const int pair = wi.pair;
  const int rem = wi.sub;
  const int qt = CAUSAL ? (a.n_qtiles - 1 - rem / a.g) : (rem / a.g);
  const int hq = (pair % a.Hkv) * a.g + rem % a.g;
  const int b = pair / a.Hkv;
  const int kvh = pair % a.Hkv;
  const int qw0 = qt * 32;
  const int off = a.Nk - a.Nq;
  const int qi = qw0 + l32;

  const float* qh = a.q + ((size_t)b * a.Hq + hq) * (size_t)a.Nq * D;
  const float* kh = a.k + ((size_t)b * a.Hkv + kvh) * (size_t)a.Nk * D;
  const float* vh = a.v + ((size_t)b * a.Hkv + kvh) * (size_t)a.Nk * D;

  int kend = a.Nk;
  if (CAUSAL) kend = min(a.Nk, min(qw0 + 32, a.Nq) - 1 + off + 1);
  const int n_tiles = kend > 0 ? (kend + BN - 1) / BN : 0;

  // Q fragment s: row qi, dim 2s + h
  float qf[D / 2];
#pragma unroll
  for (int s = 0; s < D / 2; s++) qf[s] = qi < a.Nq ? qh[(size_t)qi * D + 2 * s + h32] : 0.0f;

  f32x16 acc[D / 32];
#pragma unroll
  for (int cb = 0; cb < D / 32; cb++) acc[cb] = f32x16{};
  float m_run = kNegInf, l_run = 0.0f;

  for (int t = 0; t < n_tiles; t++) {
    const int j0 = t * BN;
    __syncthreads();
    for (int e = lane; e < BN * D; e += 64) {
      const int r = e / D, cc = e % D;
      const bool in = j0 + r < a.Nk;
      kt[r * LD + cc] = in ? kh[(size_t)(j0 + r) * D + cc] : 0.0f;
      vt[r * LD + cc] = in ? vh[(size_t)(j0 + r) * D + cc] : 0.0f;
    }
    __syncthreads();
    f32x16 st = f32x16{};
#pragma unroll
    for (int s = 0; s < D / 2; s++) st = mfma32_f32(kt[l32 * LD + 2 * s + h32], qf[s], st);
#pragma unroll
    for (int r = 0; r < 16; r++) {
      const int j = j0 + 8 * (r >> 2) + 4 * h32 + (r & 3);
      bool ok = j < a.Nk;
      if (CAUSAL) ok = ok && (j <= qi + off);
      if (!ok) st[r] = kNegInf;
    }
    float mx = kNegInf;
#pragma unroll
    for (int r = 0; r < 16; r++) mx = fmaxf(mx, st[r]);
    mx = halves_max(mx) * a.c;
    const float m_new = fmaxf(m_run, mx);
    if (m_new > m_run) {
      const float alpha = fast_exp2(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int cb = 0; cb < D / 32; cb++)
#pragma unroll
        for (int r = 0; r < 16; r++) acc[cb][r] *= alpha;
      m_run = m_new;
    }
    const float m_use = (m_run == kNegInf) ? 0.0f : m_run;
#pragma unroll
    for (int r = 0; r < 16; r++) {
      st[r] = fast_exp2(__builtin_fmaf(st[r], a.c, -m_use));
      l_run += st[r];
    }
    // O^T += V^T P^T: MFMA r contracts over keys (8(r/4) + r%4) and (8(r/4) + 4 + r%4)
#pragma unroll
    for (int r = 0; r < 16; r++) {
      const int key = 8 * (r >> 2) + 4 * h32 + (r & 3);
#pragma unroll
      for (int cb = 0; cb < D / 32; cb++) acc[cb] = mfma32_f32(vt[key * LD + cb * 32 + l32], st[r], acc[cb]);
    }
  }
  const float l_tot = halves_sum(l_run);
  const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
  if (qi < a.Nq) {
    float* orow = a.o + ((size_t)b * a.Hq + hq) * (size_t)a.Nq * D + (size_t)qi * D;
#pragma unroll
    for (int cb = 0; cb < D / 32; cb++)
#pragma unroll
      for (int r = 0; r < 16; r++) orow[cb * 32 + 8 * (r >> 2) + 4 * h32 + (r & 3)] = acc[cb][r] * inv;
    if (a.lse != nullptr && h32 == 0)
      a.lse[((size_t)b * a.Hq + hq) * a.Nq + qi] = l_tot > 0.0f ? (m_run + __log2f(l_tot)) * kLn2 : kNegInf;
  }
}

// ---------------------------------------------------------------------------
// Dense forward in two alternating wave groups (8 waves, 256 query rows).
// Per 64-key tile a wave has 32 MFMAs (S^T = K Q^T and O^T += V^T P^T) and
// the softmax between them, ~3.5 VALU instructions per MFMA, one of them an
// exponential.  A SIMD hosts one wave of each group (waves w and w + 4), and
// the groups run in anti-phase, separated by a workgroup barrier at every
// phase boundary: while one wave of a SIMD issues only MFMAs (the P V of the
// previous tile and the S^T of this one), its partner issues only the VALU
// work of its softmax, so the exponentials of one wave execute under the
// contractions of the other instead of after them.  Per tile and group:
//
//   MFMA phase (tile t):  O^T += V(t-1)^T P(t-1)^T,  S^T(t) = K(t) Q^T
//   VALU phase (tile t):  mask, online softmax of S^T(t) -> P(t)
//
// Group 0 runs MFMA(t) in phase 2t and VALU(t) in phase 2t + 1; group 1 one
// phase later.  K(t) and V(t - 1) are read in phases 2t (group 0) and 2t + 1
// (group 1).  The loads are issued by the group entering its VALU phase, so
// that the group entering its MFMA phase starts its contractions at once
// (all eight waves issuing at the phase start held the MFMA group ~650
// cycles): group 1 loads K(t + 1) at the start of phase 2t and group 0 loads
// V(t + 1) at the start of phase 2t + 1, each into the buffer the tile three
// before it left (three K and three V buffers).  Results are the same bits
// as fwd_bf16_kernel: the per-tile arithmetic and its order are unchanged,
// only the interleaving of the two groups differs.
//
// ATTN_FWD_PP_GROUPS 1: the MFMA phase's operand reads are scheduled two
// contractions ahead of their MFMAs (scheduling groups; the compiler's own
// order measured 3-8 % slower)
#ifndef ATTN_FWD_PP_GROUPS
#define ATTN_FWD_PP_GROUPS 1
#endif
template <int D, bool CAUSAL, bool VARLEN = false, bool PAGED = false>
__global__ __launch_bounds__(512, 1) void fwd_pp_kernel(FwdArgs a) {
  constexpr int NW = 8, BM = NW * 32, BN = 64, KB = 2;
  constexpr int TILE_BYTES = BN * D * 2;
  constexpr int CPR = D / 8;
  constexpr int LOADS = BN * CPR / (64 * NW);
  static_assert(LOADS * 64 * NW == BN * CPR, "tile must split evenly over the workgroup");
  static_assert(!PAGED || VARLEN, "the paged layout comes with a packed batch");
  __shared__ __attribute__((aligned(1024))) char k_st0[TILE_BYTES], k_st1[TILE_BYTES], k_st2[TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char v_st0[TILE_BYTES], v_st1[TILE_BYTES], v_st2[TILE_BYTES];

  const int lane = threadIdx.x & 63;
  const int wave = wave_id();
  const int grp = wave >> 2;  // waves w and w + 4 share a SIMD
  const int h32 = lane >> 5;
  const int l32 = lane & 31;

  // work item and this (batch or sequence, head) slice, as in fwd_bf16_kernel
  int qt, hq, b, kvh;
  if constexpr (VARLEN) {
    if (!varlen_item<BM, BN, CAUSAL, PAGED>(a, (int)blockIdx.x, b, qt, hq)) return;
    kvh = hq / a.g;
  } else {
    const WorkItem wi = lpt_order(blockIdx.x, a.B * a.Hkv, a.g * a.n_qtiles);
    const int rem = wi.sub;
    qt = CAUSAL ? (a.n_qtiles - 1 - rem / a.g) : (rem / a.g);
    hq = (wi.pair % a.Hkv) * a.g + rem % a.g;
    b = wi.pair / a.Hkv;
    kvh = wi.pair % a.Hkv;
  }
  int Nq = a.Nq, Nk = a.Nk;
  size_t q_head, kv_head, lse_row;
  if constexpr (VARLEN) {
    // clamped, so that offsets that do not describe a packed batch cannot
    // take a load outside q, k or v
    const int q1 = min(a.cu_q[b + 1], a.tot_q), q0 = max(0, min(a.cu_q[b], q1));
    Nq = q1 - q0;
    q_head = ((size_t)hq * a.tot_q + q0) * D;
    lse_row = (size_t)hq * a.tot_q + q0;
    if constexpr (PAGED) {
      Nk = min(max(a.seq_lens_k[b], 0), min(a.Nk, a.max_pages * a.page));
      kv_head = 0;
    } else {
      const int k1 = min(a.cu_k[b + 1], a.tot_k), k0 = max(0, min(a.cu_k[b], k1));
      Nk = k1 - k0;
      kv_head = ((size_t)kvh * a.tot_k + k0) * D;
    }
  } else {
    q_head = ((size_t)b * a.Hq + hq) * (size_t)Nq * D;
    kv_head = ((size_t)b * a.Hkv + kvh) * (size_t)Nk * D;
    lse_row = ((size_t)b * a.Hq + hq) * (size_t)Nq;
  }
  const int i0 = qtile_row0<BM, CAUSAL>(qt, Nq);
  const int qw0 = i0 + wave * 32;
  // rows before 0 pad the first tile: they take row 0's Q and mask
  constexpr bool LEAD_PAD = CAUSAL && kEndAlign;
  auto lo_row = [](int r) { return LEAD_PAD ? max(r, 0) : r; };
  if (VARLEN && i0 >= Nq) return;  // the whole workgroup: a tile past this sequence's queries
  const int off = Nk - Nq;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(a.q + q_head, (uint32_t)Nq * D * 2);
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(a.k + kv_head, (uint32_t)Nk * D * 2);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(a.v + kv_head, (uint32_t)Nk * D * 2);
  int kend = Nk;
  if (CAUSAL) kend = min(Nk, min(i0 + BM, Nq) - 1 + off + 1);
  const int n = kend > 0 ? (kend + BN - 1) / BN : 0;

  // paged: the page ids of the first 64 pages, one per lane
  int pg_lane = 0;
  if constexpr (PAGED) {
    if (lane < (kend + a.page - 1) / a.page) pg_lane = a.block_table[(size_t)b * a.max_pages + lane];
  }
  // the buffer and first row that tile t of K (or V) is loaded from; a paged
  // tile lies in one page (pages are whole multiples of 64 keys), rows past
  // the sequence's keys read as zeros and a page id outside the cache is
  // clamped into it
  auto tile_src = [&](int t, bool is_v, int& row0) __attribute__((always_inline)) {
    if constexpr (PAGED) {
      const int j0 = t * BN;
      const int pi = j0 / a.page;
      const int id = pi < 64 ? __builtin_amdgcn_readlane(pg_lane, pi) : a.block_table[(size_t)b * a.max_pages + pi];
      const int pg = min(max(id, 0), a.num_pages - 1);
      const size_t base = (((size_t)pg * a.Hkv + kvh) * a.page + (j0 % a.page)) * D;
      row0 = 0;
      return make_rsrc((is_v ? a.v : a.k) + base, (uint32_t)min(BN, Nk - j0) * D * 2);
    } else {
      row0 = t * BN;
      return is_v ? rv : rk;
    }
  };
  auto issue1 = [&](int t, char* dst, bool is_v) __attribute__((always_inline)) {
    int row0;
    const __amdgpu_buffer_rsrc_t r = tile_src(t, is_v, row0);
#pragma unroll
    for (int m = 0; m < LOADS; m++) {
      const int slab = m * NW + wave;
      const int p = slab * 64 + lane;
      const int row = p / CPR;
      const int c = (p % CPR) ^ swz<D>(row);
      buf_load_lds16(r, (uint32_t)(((row0 + row) * D + c * 8) * 2), (lds_void*)(dst + slab * 1024));
    }
  };
  // a K (or V) tile loaded by the four waves of one group
  auto issue4 = [&](int t, char* dst, bool is_v) __attribute__((always_inline)) {
    int row0;
    const __amdgpu_buffer_rsrc_t r = tile_src(t, is_v, row0);
#pragma unroll
    for (int m = 0; m < 2 * LOADS; m++) {
      const int slab = m * (NW / 2) + (wave & 3);
      const int p = slab * 64 + lane;
      const int row = p / CPR;
      const int c = (p % CPR) ^ swz<D>(row);
      buf_load_lds16(r, (uint32_t)(((row0 + row) * D + c * 8) * 2), (lds_void*)(dst + slab * 1024));
    }
  };
  if (n > 0) issue1(0, k_st0, false);
  if (n > 0 && grp == 0) issue4(0, v_st0, true);

  bf16x8 qf[D / 16];
#pragma unroll
  for (int s = 0; s < D / 16; s++)
    qf[s] = __builtin_bit_cast(bf16x8, buf_load16(rq, (uint32_t)((lo_row(qw0 + l32) * D + 16 * s + 8 * h32) * 2)));
  // Q, K(0) and V(0) complete here, so that no later counted wait has to
  // cover the Q registers
  wait_vmem();

  const int swl = swz<D>(l32);
  int koff[D / 16];
#pragma unroll
  for (int s = 0; s < D / 16; s++) koff[s] = l32 * (D * 2) + (((2 * s + h32) ^ swl) << 4);
  int voff[D / 32][2];
#pragma unroll
  for (int cb = 0; cb < D / 32; cb++)
#pragma unroll
    for (int lh = 0; lh < 2; lh++)
      voff[cb][lh] = tile_off<D>(4 * h32 + ((lane & 15) >> 2) + 8 * lh, cb * 32 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3));

  f32x16 acc[D / 32];
#pragma unroll
  for (int cb = 0; cb < D / 32; cb++) acc[cb] = f32x16{};
  float m_run = kNegInf, l_run = 0.0f;
  const int qi = qw0 + l32;
  f32x16 st[KB];      // S^T of the tile between its MFMA and VALU phases
  bf16x8 pb[KB][2];   // P of the tile between its VALU phase and the next MFMA phase

  // the tiles this wave computes, 0 .. n_vis - 1: up to its last row's
  // diagonal when causal, and none for a wave whose 32 rows all lie past the
  // last query (the ragged tile's padding), which takes part in the loads and
  // barriers only
  int n_vis = n;
  if (CAUSAL) {
    const int x = qw0 + 31 + off;  // tile t is visible iff t * BN <= x
    n_vis = x < 0 ? 0 : min(n, x / BN + 1);
  }
  if (qw0 >= Nq || (LEAD_PAD && qw0 + 31 < 0)) n_vis = 0;
  auto visible = [&](int t) __attribute__((always_inline)) { return t >= 0 && t < n_vis; };
  // MFMA phase of tile t: P V of tile t - 1 (V in vp), S^T of tile t (K in kc)
  auto mfma_phase = [&](int t, const char* __restrict__ kc, const char* __restrict__ vp)
                        __attribute__((always_inline)) {
    if (visible(t - 1)) {
#pragma unroll
      for (int kb = 0; kb < KB; kb++)
#pragma unroll
        for (int hf = 0; hf < 2; hf++) {
          const char* vk = vp + (kb * 32 + 16 * hf) * (D * 2);
#pragma unroll
          for (int cb = 0; cb < D / 32; cb++) {
            const s16x4 lo = ds_read_tr16(vk + voff[cb][0]);
            const s16x4 hi = ds_read_tr16(vk + voff[cb][1]);
            acc[cb] = mfma32(join_bf16(lo, hi), pb[kb][hf], acc[cb]);
          }
        }
#if ATTN_FWD_PP_GROUPS
      // operand reads run two contractions ahead of their MFMAs, not all
      // hoisted to the top (which would hold 64 more registers)
      __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
#pragma unroll
      for (int i = 0; i < 2 * KB * (D / 32) - 3; i++) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 3, 0);
#endif
    }
    // P dies before S^T is born: the two never hold registers at once
    __builtin_amdgcn_sched_barrier(0);
    if (visible(t)) {
#pragma unroll
      for (int kb = 0; kb < KB; kb++) st[kb] = f32x16{};
#pragma unroll
      for (int s = 0; s < D / 16; s++)
#pragma unroll
        for (int kb = 0; kb < KB; kb++)
          st[kb] = mfma32(*(const bf16x8*)(kc + koff[s] + kb * 32 * (D * 2)), qf[s], st[kb]);
#if ATTN_FWD_PP_GROUPS
      __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
#pragma unroll
      for (int i = 0; i < KB * (D / 16) - 3; i++) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 3, 0);
#endif
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  // VALU phase of tile t: the online softmax of fwd_bf16_kernel, on st -> pb
  auto valu_phase = [&](int t) __attribute__((always_inline)) {
    if (!visible(t)) return;
    const int j0 = t * BN;
    bool need_mask = (j0 + BN > Nk);
    if (CAUSAL && j0 + BN - 1 > qw0 + off) need_mask = true;
    if (need_mask) {
      const int lim = (CAUSAL ? min(Nk, lo_row(qi) + off + 1) : Nk) - j0 - 4 * h32;
#pragma unroll
      for (int kb = 0; kb < KB; kb++)
#pragma unroll
        for (int r = 0; r < 16; r++)
          if (!(kb * 32 + 8 * (r >> 2) + (r & 3) < lim)) st[kb][r] = kNegInf;
    }
    float psum = 0.0f;
    bool fast = __builtin_amdgcn_ballot_w64(m_run == kNegInf) == 0;
    if (fast) {
#pragma unroll
      for (int kb = 0; kb < KB; kb++)
#pragma unroll
        for (int hf = 0; hf < 2; hf++)
#pragma unroll
          for (int e = 0; e < 8; e++) {
            const float p = fast_exp2(__builtin_fmaf(st[kb][8 * hf + e], a.c, -m_run));
            pb[kb][hf][e] = to_bf16(p);
            psum += p;
          }
      fast = __builtin_amdgcn_ballot_w64(!(psum <= 65536.0f)) == 0;
    }
    if (!fast) {
      float mx = kNegInf;
#pragma unroll
      for (int kb = 0; kb < KB; kb++)
#pragma unroll
        for (int r = 0; r < 16; r++) mx = fmaxf(mx, st[kb][r]);
      mx = halves_max(mx) * a.c;
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
      psum = 0.0f;
#pragma unroll
      for (int kb = 0; kb < KB; kb++)
#pragma unroll
        for (int hf = 0; hf < 2; hf++)
#pragma unroll
          for (int e = 0; e < 8; e++) {
            const float p = fast_exp2(__builtin_fmaf(st[kb][8 * hf + e], a.c, -m_use));
            pb[kb][hf][e] = to_bf16(p);
            psum += p;
          }
    }
    l_run += psum;
  };
  // Tile t takes phases 2t and 2t + 1.  Each group loads in its VALU
  // phases, so that the MFMA group never waits to issue loads: group 1
  // issues K(t + 1) at the start of phase 2t (needed at phase 2t + 2) and
  // group 0 issues V(t + 1) at the start of phase 2t + 1 (needed at phase
  // 2t + 4), each into the buffer the tile three before it left.  At the
  // start of phase 2t group 1 waits for all its loads (K(t)) and group 0 for
  // all but V(t) (so V(t - 1) has landed), then the barrier publishes them.
  // Each group runs its own loop (the same barriers in the same number), so
  // that the register allocator sees one group's phase order at a time.
  if (grp == 0) {
    auto tile = [&](int t, const char* __restrict__ kc, const char* __restrict__ vp, char* __restrict__ vn)
                    __attribute__((always_inline)) {
      if (t >= 1 && t < n)
        wait_vmem_n<2 * LOADS>();  // V(t) may still be in flight
      else
        wait_vmem();
      barrier_nofence();  // phase 2t
      mfma_phase(t, kc, vp);
      barrier_nofence();  // phase 2t + 1
      if (t + 1 < n) issue4(t + 1, vn, true);
      valu_phase(t);
    };
    for (int t = 0; t <= n; t += 3) {
      tile(t, k_st0, v_st2, v_st1);
      if (t + 1 > n) break;
      tile(t + 1, k_st1, v_st0, v_st2);
      if (t + 2 > n) break;
      tile(t + 2, k_st2, v_st1, v_st0);
    }
  } else {
    auto tile = [&](int t, const char* __restrict__ kc, const char* __restrict__ vp, char* __restrict__ kn)
                    __attribute__((always_inline)) {
      wait_vmem();
      barrier_nofence();  // phase 2t
      if (t + 1 < n) issue4(t + 1, kn, false);
      valu_phase(t - 1);
      barrier_nofence();  // phase 2t + 1
      mfma_phase(t, kc, vp);
    };
    for (int t = 0; t <= n; t += 3) {
      tile(t, k_st0, v_st2, k_st1);
      if (t + 1 > n) break;
      tile(t + 1, k_st1, v_st0, k_st2);
      if (t + 2 > n) break;
      tile(t + 2, k_st2, v_st1, k_st0);
    }
  }

  const float l_tot = halves_sum(l_run);
  const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
#if ATTN_FWD_O_STAGE
  // O through LDS: each wave writes its 32 rows into the (now free) K/V
  // buffers, two waves per buffer, and stores them back four whole rows per
  // instruction instead of 16-byte pieces of 32 rows
  static_assert(2 * 32 * D * 2 <= TILE_BYTES, "two waves' rows per buffer");
  __syncthreads();  // every wave is done with the K/V buffers
  char* const obuf = ((wave >> 1) == 0 ? k_st0 : (wave >> 1) == 1 ? k_st1 : (wave >> 1) == 2 ? k_st2 : v_st0) +
                     (wave & 1) * (32 * D * 2);
#pragma unroll
  for (int cb = 0; cb < D / 32; cb++)
#pragma unroll
    for (int g4 = 0; g4 < 4; g4++) {
      bf16x4 w;
#pragma unroll
      for (int e = 0; e < 4; e++) w[e] = to_bf16(acc[cb][4 * g4 + e] * inv);
      *(bf16x4*)(obuf + tile_off<D>(l32, cb * 32 + 8 * g4 + 4 * h32)) = w;
    }
  __syncthreads();
  constexpr int CPR_O = D / 8;  // 16-byte chunks per row
#pragma unroll
  for (int i = 0; i < 32 * CPR_O / 64; i++) {
    const int p = i * 64 + lane;
    const int r = p / CPR_O, ch = p % CPR_O;
    const int row = qw0 + r;
    const i32x4 val = *(const i32x4*)(obuf + r * (D * 2) + ((ch ^ swz<D>(r)) << 4));
    if ((!LEAD_PAD || row >= 0) && row < Nq) {
      i32x4* dst = (i32x4*)(a.o + q_head + (size_t)row * D + ch * 8);
#if ATTN_FWD_O_STAGE == 2
      __builtin_nontemporal_store(val, dst);
#else
      *dst = val;
#endif
    }
  }
  if ((!LEAD_PAD || qi >= 0) && qi < Nq && a.lse != nullptr && h32 == 0)
    a.lse[lse_row + qi] = l_tot > 0.0f ? (m_run + __log2f(l_tot)) * kLn2 : kNegInf;
#else
  if ((!LEAD_PAD || qi >= 0) && qi < Nq) {
    __bf16* orow = a.o + q_head + (size_t)qi * D;
#pragma unroll
    for (int cb = 0; cb < D / 32; cb++)
#pragma unroll
      for (int g4 = 0; g4 < 4; g4++) {
        bf16x4 w;
#pragma unroll
        for (int e = 0; e < 4; e++) w[e] = to_bf16(acc[cb][4 * g4 + e] * inv);
        *(bf16x4*)(orow + cb * 32 + 8 * g4 + 4 * h32) = w;
      }
    if (a.lse != nullptr && h32 == 0) a.lse[lse_row + qi] = l_tot > 0.0f ? (m_run + __log2f(l_tot)) * kLn2 : kNegInf;
  }
#endif
}

template <int D, bool CAUSAL, bool VARLEN = false, bool PAGED = false>
hipError_t launch_pp(const FwdProblem& p, hipStream_t s) {
  FwdArgs a{};
  a.q = (const __bf16*)p.q;
  a.k = (const __bf16*)p.k;
  a.v = (const __bf16*)p.v;
  a.o = (__bf16*)p.o;
  a.lse = p.lse;
  a.B = (int)p.B;
  a.Hq = (int)p.Hq;
  a.Hkv = (int)p.Hkv;
  a.Nq = (int)p.Nq;
  a.Nk = (int)p.Nk;
  a.g = a.Hq / a.Hkv;
  a.n_qtiles = (a.Nq + 255) / 256;
  a.n_wgs = a.B * a.Hq * a.n_qtiles;
  a.c = p.scale * kLog2e;
  a.cu_q = p.cu_q;
  a.cu_k = p.cu_k;
  a.tot_q = (int)p.tot_q;
  a.tot_k = (int)p.tot_k;
  a.block_table = p.block_table;
  a.seq_lens_k = p.seq_lens_k;
  a.page = (int)p.page;
  a.max_pages = (int)p.max_pages;
  a.num_pages = (int)p.num_pages;
  hipLaunchKernelGGL((fwd_pp_kernel<D, CAUSAL, VARLEN, PAGED>), dim3(a.n_wgs), dim3(512), 0, s, a);
  return hipGetLastError();
}

template <int D, int NW, int BN, bool CAUSAL, bool PAGED = false>
hipError_t launch_bf16(const FwdProblem& p, hipStream_t s) {
  FwdArgs a{};
  a.q = (const __bf16*)p.q;
  a.k = (const __bf16*)p.k;
  a.v = (const __bf16*)p.v;
  a.o = (__bf16*)p.o;
  a.lse = p.lse;
  a.B = (int)p.B;
  a.Hq = (int)p.Hq;
  a.Hkv = (int)p.Hkv;
  a.Nq = (int)p.Nq;
  a.Nk = (int)p.Nk;
  a.g = a.Hq / a.Hkv;
  a.n_qtiles = (a.Nq + NW * 32 - 1) / (NW * 32);
  a.n_wgs = a.B * a.Hq * a.n_qtiles;
  a.snake = (CAUSAL && NW == 4 && p.cu_q == nullptr && (a.B * a.Hkv) % 8 == 0 && a.n_wgs <= 2 * 256) ? 1 : 0;
  a.c = p.scale * kLog2e;
  a.cu_q = p.cu_q;
  a.cu_k = p.cu_k;
  a.tot_q = (int)p.tot_q;
  a.tot_k = (int)p.tot_k;
  a.block_table = p.block_table;
  a.seq_lens_k = p.seq_lens_k;
  a.page = (int)p.page;
  a.max_pages = (int)p.max_pages;
  a.num_pages = (int)p.num_pages;
  hipLaunchKernelGGL((fwd_bf16_kernel<D, NW, BN, CAUSAL, PAGED>), dim3(a.n_wgs), dim3(NW * 64), 0, s, a);
  return hipGetLastError();
}

template <int D, bool CAUSAL>
hipError_t launch_f32(const FwdProblem& p, hipStream_t s) {
  FwdArgsF32 a;
  a.q = (const float*)p.q;
  a.k = (const float*)p.k;
  a.v = (const float*)p.v;
  a.o = (float*)p.o;
  a.lse = p.lse;
  a.B = (int)p.B;
  a.Hq = (int)p.Hq;
  a.Hkv = (int)p.Hkv;
  a.Nq = (int)p.Nq;
  a.Nk = (int)p.Nk;
  a.g = a.Hq / a.Hkv;
  a.n_qtiles = (a.Nq + 31) / 32;
  a.n_wgs = a.B * a.Hq * a.n_qtiles;
  a.c = p.scale * kLog2e;
  hipLaunchKernelGGL((fwd_f32_kernel<D, CAUSAL>), dim3(a.n_wgs), dim3(64), 0, s, a);
  return hipGetLastError();
}

}  // namespace

#ifndef ATTN_FWD_BIG_NW
#define ATTN_FWD_BIG_NW 8
#endif
#ifndef ATTN_FWD_BIG_BN
#define ATTN_FWD_BIG_BN 64
#endif
// 1: dense problems with 8-wave workgroups run the two-group kernel
#ifndef ATTN_FWD_PP
#define ATTN_FWD_PP 1
#endif
// causal dense problems take 8-wave workgroups from this many 256-row tiles
// (non-causal ones from half as many)
#ifndef ATTN_FWD_DENSE_MIN_BIG
#define ATTN_FWD_DENSE_MIN_BIG (2 * 256)
#endif
// packed batches take 8-wave workgroups from this many 256-row tiles
#ifndef ATTN_FWD_PACKED_MIN_BIG
#define ATTN_FWD_PACKED_MIN_BIG (8 * 256)
#endif

hipError_t launch_fwd(const FwdProblem& p, hipStream_t s) {
  const bool causal = p.causal != 0;
  if (p.paged) {
    // packed batch over a paged K/V cache (bf16)
    constexpr int NWB = ATTN_FWD_BIG_NW, BNB = ATTN_FWD_BIG_BN;
    const bool big = p.B * p.Hq * ((p.Nq + NWB * 32 - 1) / (NWB * 32)) >= ATTN_FWD_PACKED_MIN_BIG;
    if (ATTN_FWD_PP && big) {
      if (p.d == 128) return causal ? launch_pp<128, true, true, true>(p, s) : launch_pp<128, false, true, true>(p, s);
      return causal ? launch_pp<64, true, true, true>(p, s) : launch_pp<64, false, true, true>(p, s);
    }
    if (p.d == 128) {
      if (big)
        return causal ? launch_bf16<128, NWB, BNB, true, true>(p, s) : launch_bf16<128, NWB, BNB, false, true>(p, s);
      return causal ? launch_bf16<128, 4, 64, true, true>(p, s) : launch_bf16<128, 4, 64, false, true>(p, s);
    }
    if (big) return causal ? launch_bf16<64, NWB, BNB, true, true>(p, s) : launch_bf16<64, NWB, BNB, false, true>(p, s);
    return causal ? launch_bf16<64, 4, 64, true, true>(p, s) : launch_bf16<64, 4, 64, false, true>(p, s);
  }
  if (p.bf16) {
    // 8 waves (256 query rows) per workgroup, which share each K/V tile (half
    // the tile loads and barriers per query row of the 4-wave configuration),
    // run as the two-group kernel (fwd_pp_kernel; the one-group
    // fwd_bf16_kernel<.., 8, ..> only with ATTN_FWD_PP=0).  Causal dense
    // problems take them once there are at least two such workgroups per CU
    // over the launch (the one-group kernel measured 3-8 % faster than 4
    // waves at N = 4096 and 8192, 32 heads; with one per CU, N = 2048, 32
    // heads, 14 % slower, and the two-group kernel 5-20 % slower), where
    // 4-wave workgroups, two per CU, fill the machine instead.  Packed
    // batches, whose grid counts every sequence at the longest one's length,
    // keep 4 waves up to 8 per CU (8 waves measured 9 % slower on 4 sequences
    // of 600..2048 tokens, equal on 8).
    constexpr int NWB = ATTN_FWD_BIG_NW, BNB = ATTN_FWD_BIG_BN;
    // a non-causal grid of equal workgroups fills the machine with one
    // two-group workgroup per CU (10 % faster at N = 2048, 32 heads, 256
    // such tiles); causal ones, whose workgroups differ up to 16-fold, need
    // two per CU over the launch for the longest-first order to even out
    const int64_t min_big = p.cu_q != nullptr ? ATTN_FWD_PACKED_MIN_BIG
                            : (causal || !ATTN_FWD_PP) ? ATTN_FWD_DENSE_MIN_BIG : ATTN_FWD_DENSE_MIN_BIG / 2;
    const bool big = p.B * p.Hq * ((p.Nq + NWB * 32 - 1) / (NWB * 32)) >= min_big;
    if (ATTN_FWD_PP && big && p.cu_q == nullptr) {
      if (p.d == 128) return causal ? launch_pp<128, true>(p, s) : launch_pp<128, false>(p, s);
      return causal ? launch_pp<64, true>(p, s) : launch_pp<64, false>(p, s);
    }
    if (ATTN_FWD_PP && big) {
      if (p.d == 128) return causal ? launch_pp<128, true, true>(p, s) : launch_pp<128, false, true>(p, s);
      return causal ? launch_pp<64, true, true>(p, s) : launch_pp<64, false, true>(p, s);
    }
    if (p.d == 128) {
      if (big) return causal ? launch_bf16<128, NWB, BNB, true>(p, s) : launch_bf16<128, NWB, BNB, false>(p, s);
      return causal ? launch_bf16<128, 4, 64, true>(p, s) : launch_bf16<128, 4, 64, false>(p, s);
    }
    if (big) return causal ? launch_bf16<64, NWB, BNB, true>(p, s) : launch_bf16<64, NWB, BNB, false>(p, s);
    return causal ? launch_bf16<64, 4, 64, true>(p, s) : launch_bf16<64, 4, 64, false>(p, s);
  }
  if (p.d == 128) return causal ? launch_f32<128, true>(p, s) : launch_f32<128, false>(p, s);
  return causal ? launch_f32<64, true>(p, s) : launch_f32<64, false>(p, s);
}

}  // namespace attn
