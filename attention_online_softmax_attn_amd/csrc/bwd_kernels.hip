// Backward kernels of softmax attention on gfx950, part 1: dK, dV and the
// backward's launch sequence (the formulas and the kernel split are stated in
// bwd_common.hpp).
#include <type_traits>

#include "bwd_common.hpp"

namespace attn {

namespace {

using bwd::BwdArgs;

// ---------------------------------------------------------------------------
// dK, dV.  Each wave owns 32 keys; a query tile of BQ rows is processed in
// 32-row blocks.
template <int D, int NW, int BQ, bool CAUSAL, bool G16>
__global__ __launch_bounds__(NW * 64, ATTN_BWD_KV_OCC) void bwd_dkdv_kernel(BwdArgs a) {
  constexpr int TILE = BQ * D * 2;  // bytes of one Q or dO tile
  constexpr int STAGE = 2 * TILE + 1024;  // Q, dO, row records (BQ * 8 <= 1024 bytes)
  constexpr int NS = ATTN_BWD_STAGES;     // query tiles in flight
  static_assert(NS == 2 || NS == 3, "two or three stages");
  constexpr int CPR = D / 8;
  constexpr int LOADS = BQ * CPR / (64 * NW);
  constexpr int VM_PER_TILE = 2 * LOADS + 1;  // vector-memory loads per wave per tile
  constexpr int NB = BQ / 32;  // 32-row blocks per tile
  static_assert(LOADS * 64 * NW == BQ * CPR, "tile must split evenly");
  static_assert(BQ % 32 == 0 && BQ * 8 <= 1024, "BQ must be 32, 64, 96 or 128");
  __shared__ __attribute__((aligned(1024))) char smem[NS * STAGE];  // per stage: [Q | dO | records]

  const int lane = threadIdx.x & 63;
  // the per-lane form on purpose: with the wave index made uniform the
  // compiler specialises this kernel's branches and needs ~80 more registers
  // (spilling in the non-causal instantiation)
  const int wave = threadIdx.x >> 6;
  const int h32 = lane >> 5;
  const int l32 = lane & 31;

  // causal: early key tiles are seen by the most queries, so they go first
  const WorkItem wi = lpt_order(blockIdx.x, a.B * a.Hkv, a.n_tiles);
  const int kt = wi.sub;
  const int pair = wi.pair;
  const int b = pair / a.Hkv;
  const int kvh = pair % a.Hkv;
  const int j0 = kt * (NW * 32);
  const int jw = j0 + wave * 32;  // this wave's first key
  const int jl = jw + l32;        // this lane's key (N index of S and dP)
  const int off = a.Nk - a.Nq;

  const size_t kv_head = ((size_t)b * a.Hkv + kvh) * (size_t)a.Nk * D;
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(a.k + kv_head, (uint32_t)a.Nk * D * 2);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(a.v + kv_head, (uint32_t)a.Nk * D * 2);

  // K and V as B operands: key jl, dims 16s + 8h .. +8
  bf16x8 kf[D / 16], vf[D / 16];
#pragma unroll
  for (int s = 0; s < D / 16; s++) {
    const uint32_t src = (uint32_t)((jl * D + 16 * s + 8 * h32) * 2);
    kf[s] = __builtin_bit_cast(bf16x8, buf_load16(rk, src));
    vf[s] = __builtin_bit_cast(bf16x8, buf_load16(rv, src));
  }

  f32x16 dk_acc[D / 32], dv_acc[D / 32];
#pragma unroll
  for (int cb = 0; cb < D / 32; cb++) {
    dk_acc[cb] = f32x16{};
    dv_acc[cb] = f32x16{};
  }

  // query tiles that can see any key of this workgroup
  int qt_first = 0;
  if (CAUSAL) qt_first = max(0, j0 - off) / BQ;
  const int nqt = (a.Nq + BQ - 1) / BQ;
  const int per_head = nqt > qt_first ? nqt - qt_first : 0;
  const int n_iter = per_head * a.g;
  const int swl = swz<D>(l32);

  auto head_of = [&](int it) { return kvh * a.g + it / per_head; };
  auto qtile_of = [&](int it) { return qt_first + it % per_head; };

  auto issue = [&](int it, char* st_l) {
    const int hq = head_of(it);
    const int i0 = qtile_of(it) * BQ;
    const size_t q_row0 = ((size_t)b * a.Hq + hq) * (size_t)a.Nq;
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(a.q + q_row0 * D, (uint32_t)a.Nq * D * 2);
    const __amdgpu_buffer_rsrc_t rd = make_rsrc(a.dout + q_row0 * D, (uint32_t)a.Nq * D * 2);
#pragma unroll
    for (int n = 0; n < LOADS; n++) {
      const int slab = n * NW + wave;
      const int p = slab * 64 + lane;
      const int r = p / CPR;
      const int cc = (p % CPR) ^ swz<D>(r);
      const uint32_t src = (uint32_t)(((i0 + r) * D + cc * 8) * 2);
      buf_load_lds16(rq, src, (lds_void*)(st_l + slab * 1024));
      buf_load_lds16(rd, src, (lds_void*)(st_l + TILE + slab * 1024));
    }
    {
      // row records of rows i0 .. i0 + 127 (the first BQ are used); rows past
      // nq_pad read as zeros, rows past Nq are masked.  Every wave loads the
      // same 1 KB (identical bytes), so every wave issues the same number of
      // loads per tile and can wait for an older tile by count.
      const size_t rec0 = ((size_t)b * a.Hq + hq) * (size_t)a.nq_pad;
      const __amdgpu_buffer_rsrc_t rs = make_rsrc(a.stats + 2 * rec0, (uint32_t)a.nq_pad * 8);
      buf_load_lds16(rs, (uint32_t)(i0 * 8 + lane * 16), (lds_void*)(st_l + 2 * TILE));
    }
  };

  // ---- hand-ordered pipeline over the 32-row blocks of one tile.  Round nb
  // (nb = -1 .. NB) issues the contractions S/dP of block nb + 1 and dV/dK of
  // block nb - 1, alternating one of each kind per slot, and spreads the P/dS
  // arithmetic of block nb over the slots, so that with one wave per SIMD the
  // VALU work runs while the matrix core is busy.  Each slot also issues the
  // LDS reads of the contraction LEAD slots ahead (across round boundaries)
  // and, in the first slots of a round, the row records the next round
  // needs, so a contraction rarely waits for its operands.  The scheduling
  // barriers between slots keep the compiler from regrouping the slots.
  auto run_tile = [&](const char* st_l, int i0, auto maskc) {
    constexpr bool MASK = decltype(maskc)::value;
    constexpr int SK = D / 16;     // contraction steps of S (and of dP); also dV (and dK) MFMAs per block
    constexpr int NSLOT = 4 * SK;  // slots per round
    constexpr int NG = (NB + 2) * NSLOT;
    constexpr int LEAD = ATTN_BWD_LEAD;
    static_assert(LEAD < NSLOT, "reads run at most one round ahead");
    constexpr int CBN = D / 32;
    constexpr int PER = NSLOT / 16;  // slots per P/dS element
    const char* qt_l = st_l;
    const char* dt_l = st_l + TILE;
    const float* rec = (const float*)(st_l + 2 * TILE);
    // mask of this lane's key jl over the rows i0 + 4h + c of the tile:
    // visible iff lo <= c < hi with hi = Nq - i0 - 4h and, when causal,
    // lo = jl - off - i0 - 4h (a key past Nk sees no row)
    int m_lo = 0;
    uint32_t m_span = 0;
    if (MASK) {
      const int base = i0 + 4 * h32;
      const int hi = a.Nq - base;
      int lo = CAUSAL ? jl - off - base : -(1 << 30);
      if (jl >= a.Nk) lo = 1 << 30;
      m_lo = lo;
      m_span = hi > lo ? (uint32_t)(hi - lo) : 0u;
    }
    f32x16 sa[2], da[2];
    bf16x8 pa[2], sb[2];
    bf16x8 qa[SK], oa[SK];
    bf16x8 dob[2][CBN], qb[2][CBN];
    f32x4 rx[8];  // row records of the block in P/dS: part q holds rows 8(q/2) + 4h + 2(q%2) .. +1

    // slot k of round nb: kind k % 4 (0: S, 1: dV, 2: dP, 3: dK), step k / 4
    auto read_slot = [&](int nb, int k) {
      const int st = k >> 2, kind = k & 3;
      if ((kind == 0 || kind == 2) && nb + 1 < NB) {
        const int off_b = (32 * (nb + 1) + l32) * (D * 2) + (((2 * st + h32) ^ swl) << 4);
        if (kind == 0)
          qa[st] = *(const bf16x8*)(qt_l + off_b);
        else
          oa[st] = *(const bf16x8*)(dt_l + off_b);
      }
      if ((kind == 1 || kind == 3) && nb >= 1) {
        const int hf = st / CBN, cb = st % CBN;
        const int tr = 32 * (nb - 1) + 16 * hf + 4 * h32 + ((lane & 15) >> 2);
        const int tc = cb * 32 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
        const int o1 = tile_off<D>(tr, tc), o2 = tile_off<D>(tr + 8, tc);
        if (kind == 1)
          dob[hf][cb] = join_bf16(ds_read_tr16(dt_l + o1), ds_read_tr16(dt_l + o2));
        else
          qb[hf][cb] = join_bf16(ds_read_tr16(qt_l + o1), ds_read_tr16(qt_l + o2));
      }
    };
    auto read_global = [&](int g) { read_slot(g / NSLOT - 1, g % NSLOT); };
    auto read_rec = [&](int nb, int q) {
      const int rl = 32 * nb + 8 * (q >> 1) + 4 * h32 + 2 * (q & 1);
      rx[q] = *(const f32x4*)(rec + 2 * rl);
    };
    // part q of the records is first used at slot PER * (4 (q/2) + 2 (q%2))
    // of a round; it is read REC_LEAD slots earlier (in the previous round
    // when that is negative), so only a few parts are live at a time
    constexpr int REC_LEAD = ATTN_BWD_REC_LEAD;
    auto rec_first = [](int q) { return PER * (4 * (q >> 1) + 2 * (q & 1)); };
    auto mfma_slot = [&](int nb, int k) {
      const int st = k >> 2, kind = k & 3;
      const int nxt = (nb + 1) & 1;
      if (kind == 0 && nb + 1 < NB) sa[nxt] = mfma32(qa[st], kf[st], st == 0 ? f32x16{} : sa[nxt]);
      if (kind == 2 && nb + 1 < NB) da[nxt] = mfma32(oa[st], vf[st], st == 0 ? f32x16{} : da[nxt]);
      if ((kind == 1 || kind == 3) && nb >= 1) {
        const int hf = st / CBN, cb = st % CBN;
        if (kind == 1)
          dv_acc[cb] = mfma32(pa[hf], dob[hf][cb], dv_acc[cb]);
        else
          dk_acc[cb] = mfma32(sb[hf], qb[hf][cb], dk_acc[cb]);
      }
    };
    // P and dS of element r of block nb (row 8(r/4) + 4h + r%4)
    auto pds_elem = [&](int nb, int r) {
      const int cur = nb & 1;
      const int r4 = r >> 2, e = r & 3;
      const f32x4 x = rx[2 * r4 + (e >> 1)];
      const float l2 = x[2 * (e & 1)], dd = x[2 * (e & 1) + 1];
      float p = fast_exp2(__builtin_fmaf(sa[cur][r], a.c, -l2));
      float ds = p * (da[cur][r] - dd);
      if (MASK) {
        // row i0 + 4h + c is visible to key jl iff lo <= c < lo + span;
        // selects, not products: a padding row's record may hold anything
        const int c = 32 * nb + 8 * r4 + e;
        const bool ok = (uint32_t)(c - m_lo) < m_span;
        p = ok ? p : 0.0f;
        ds = ok ? ds : 0.0f;
      }
      sa[cur][r] = p;
      da[cur][r] = ds;
    };
    auto pack_half = [&](int nb, int hf) {
      const int cur = nb & 1;
#pragma unroll
      for (int e = 0; e < 8; e++) {
        pa[hf][e] = to_bf16(sa[cur][8 * hf + e]);
        sb[hf][e] = to_bf16(da[cur][8 * hf + e]);
      }
    };

#pragma unroll
    for (int g = 0; g < LEAD; g++) read_global(g);
#pragma unroll
    for (int nb = -1; nb <= NB; nb++) {
      const bool has_pds = nb >= 0 && nb < NB;
#pragma unroll
      for (int k = 0; k < NSLOT; k++) {
        const int g = (nb + 1) * NSLOT + k;
        if (g + LEAD < NG) read_global(g + LEAD);
#pragma unroll
        for (int q = 0; q < 8; q++) {
          const int t = rec_first(q) - REC_LEAD;
          if (t >= 0 && k == t && has_pds) read_rec(nb, q);
          if (t < 0 && k == NSLOT + t && nb + 1 < NB) read_rec(nb + 1, q);
        }
        mfma_slot(nb, k);
        if (has_pds && k % PER == 0) pds_elem(nb, k / PER);
        // the dV/dK contractions of half 0 have all been issued before slot 4 CBN
        if (has_pds && k == 4 * CBN) pack_half(nb, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (has_pds) pack_half(nb, 1);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  auto compute = [&](int it, const char* st_l) {
    const int i0 = qtile_of(it) * BQ;
    if (CAUSAL && i0 + BQ - 1 + off < jw) return;  // no query of the tile sees this wave's keys
    const bool need_mask = (i0 + BQ > a.Nq) || (jw + 32 > a.Nk) || (CAUSAL && i0 + off < jw + 31);
    if (need_mask)
      run_tile(st_l, i0, std::true_type{});
    else
      run_tile(st_l, i0, std::false_type{});
  };

  // One step: wait until tile it has landed (with NS = 3, tile it + 1 may
  // still be in flight), barrier, prefetch tile it + NS - 1 into the stage
  // that tile it - 1 used, compute tile it.  Restrict: the prefetch never
  // writes the stage being read.
  auto step = [&](int it, const char* __restrict__ cur, char* __restrict__ nxt) {
    if (NS == 3 && it + 1 < n_iter)
      wait_vmem_n<VM_PER_TILE>();
    else
      wait_vmem();
    barrier_nofence();
    if (it + NS - 1 < n_iter) issue(it + NS - 1, nxt);
    compute(it, cur);
  };
  char* const s0 = smem;
  char* const s1 = smem + STAGE;
  char* const s2 = smem + (NS - 1) * STAGE;  // = s1 when NS == 2
  if (n_iter > 0) issue(0, s0);
  if (NS == 3 && n_iter > 1) issue(1, s1);
  if (NS == 3) {
    for (int it = 0; it < n_iter; it += 3) {
      step(it, s0, s2);
      if (it + 1 >= n_iter) break;
      step(it + 1, s1, s0);
      if (it + 2 >= n_iter) break;
      step(it + 2, s2, s1);
    }
  } else {
    for (int it = 0; it < n_iter; it += 2) {
      step(it, s0, s1);
      if (it + 1 >= n_iter) break;
      step(it + 1, s1, s0);
    }
  }

  // dV, dK accumulators: lane holds dim cb*32 + l32 of keys jw + 8(r/4) + 4h + r%4
#pragma unroll
  for (int r = 0; r < 16; r++) {
    const int j = jw + 8 * (r >> 2) + 4 * h32 + (r & 3);
    if (j < a.Nk) {
#pragma unroll
      for (int cb = 0; cb < D / 32; cb++) {
        const size_t at = kv_head + (size_t)j * D + cb * 32 + l32;
        if constexpr (G16) {
          ((__bf16*)a.dk)[at] = to_bf16(dk_acc[cb][r] * a.scale);
          ((__bf16*)a.dv)[at] = to_bf16(dv_acc[cb][r]);
        } else {
          a.dk[at] = dk_acc[cb][r] * a.scale;
          a.dv[at] = dv_acc[cb][r];
        }
      }
    }
  }
}

template <int D, bool CAUSAL>
hipError_t launch(const BwdProblem& p, hipStream_t s) {
  constexpr int NW = 4;
  BwdArgs a;
  a.q = (const __bf16*)p.q;
  a.k = (const __bf16*)p.k;
  a.v = (const __bf16*)p.v;
  a.o = (const __bf16*)p.o;
  a.dout = (const __bf16*)p.dout;
  a.lse = p.lse;
  a.dq = (float*)p.dq;
  a.dk = (float*)p.dk;
  a.dv = (float*)p.dv;
  a.grad_bf16 = p.grad_bf16;
  a.stats = p.stats;
  a.nq_pad = (int)bwd_record_rows(p.Nq);
  a.B = (int)p.B;
  a.Hq = (int)p.Hq;
  a.Hkv = (int)p.Hkv;
  a.Nq = (int)p.Nq;
  a.Nk = (int)p.Nk;
  a.g = a.Hq / a.Hkv;
  a.c = p.scale * kLog2e;
  a.scale = p.scale;
  // dQ first: it also writes the row records the dK/dV kernel reads
  const int rows = a.B * a.Hq * a.Nq;
  if (rows > 0) {
    hipError_t e = bwd::launch_dq(a, D, CAUSAL, s);
    if (e != hipSuccess) return e;
  }
  if (a.Nk > 0) {
    BwdArgs kv = a;
    kv.n_tiles = (a.Nk + NW * 32 - 1) / (NW * 32);
    kv.n_wgs = a.B * a.Hkv * kv.n_tiles;
    if (a.grad_bf16)
      hipLaunchKernelGGL((bwd_dkdv_kernel<D, NW, ATTN_BWD_BQ, CAUSAL, true>), dim3(kv.n_wgs), dim3(NW * 64), 0, s, kv);
    else
      hipLaunchKernelGGL((bwd_dkdv_kernel<D, NW, ATTN_BWD_BQ, CAUSAL, false>), dim3(kv.n_wgs), dim3(NW * 64), 0, s, kv);
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace

hipError_t launch_bwd(const BwdProblem& p, hipStream_t s) {
  const bool causal = p.causal != 0;
  if (p.d == 128) return causal ? launch<128, true>(p, s) : launch<128, false>(p, s);
  return causal ? launch<64, true>(p, s) : launch<64, false>(p, s);
}

}  // namespace attn
