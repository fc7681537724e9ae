// Backward kernels of softmax attention on gfx950, part 2: dQ and the row
// records (the formulas and the kernel split are stated in bwd_common.hpp).
// Built with the default machine scheduler; the dK/dV file uses the
// ILP-maximising one.
#include <type_traits>

#include "bwd_common.hpp"

// 1: grids of 8-wave dQ workgroups run the two-group kernel
// (bwd_dq_pp_kernel; the one-group bwd_dq_kernel<.., 8, ..> only with 0)
#ifndef ATTN_BWD_DQ_PP
#define ATTN_BWD_DQ_PP 1
#endif
// 1: the two-group kernel's operand reads run three contractions ahead of
// their MFMAs (scheduling groups; the compiler's own order measured ~3 %
// slower on the dQ kernel)
#ifndef ATTN_BWD_DQ_PP_GROUPS
#define ATTN_BWD_DQ_PP_GROUPS 1
#endif

namespace attn {
namespace bwd {

namespace {

// ---------------------------------------------------------------------------
// dQ, two waves per SIMD.  The forward kernel's organisation: NW waves of 32
// query rows each share 64-key K/V tiles double-buffered in LDS (direct-to-LDS
// loads, buffers at compile-time offsets, lane-constant LDS offsets with the
// buffer, key block and row half in the immediate), and each wave works one
// 32-key block at a time so that fragments, accumulators and the block's
// S^T / dP^T fit the 256 registers a wave has when two share a SIMD; the SIMD
// then overlaps one wave's exponentials with the other's MFMAs.
template <int D, int NW, bool CAUSAL, bool G16>
__global__ __launch_bounds__(NW * 64, 8 / NW) void bwd_dq_kernel(BwdArgs a) {
  constexpr int BN = 64;
  constexpr int TILE = BN * D * 2;            // one K or V tile
  constexpr int CPR = D / 8;
  constexpr int LOADS = BN * CPR / (64 * NW);  // direct-to-LDS loads per thread per K (or V) tile
  constexpr int KB = BN / 32;
  static_assert(LOADS * 64 * NW == BN * CPR, "tile must split evenly");
  static_assert(4 * TILE <= 65536, "LDS offsets must fit the 16-bit immediate");
  __shared__ __attribute__((aligned(1024))) char smem[4 * TILE];  // [K0 | K1 | V0 | V1]

  const int lane = threadIdx.x & 63;
  const int wave = wave_id();
  const int h32 = lane >> 5;
  const int l32 = lane & 31;

  const WorkItem wi = lpt_order(blockIdx.x, a.B * a.Hkv, a.g * a.n_tiles);
  const int pair = wi.pair;
  const int rem = wi.sub;
  const int qt = CAUSAL ? (a.n_tiles - 1 - rem / a.g) : (rem / a.g);
  const int hq = (pair % a.Hkv) * a.g + rem % a.g;
  const int b = pair / a.Hkv;
  const int kvh = pair % a.Hkv;
  const int i0 = qt * NW * 32;
  const int qw0 = i0 + wave * 32;
  const int qi = qw0 + l32;
  const int off = a.Nk - a.Nq;

  const size_t q_row0 = ((size_t)b * a.Hq + hq) * (size_t)a.Nq;
  const size_t kv_head = ((size_t)b * a.Hkv + kvh) * (size_t)a.Nk * D;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(a.q + q_row0 * D, (uint32_t)a.Nq * D * 2);
  const __amdgpu_buffer_rsrc_t rd = make_rsrc(a.dout + q_row0 * D, (uint32_t)a.Nq * D * 2);
  const __amdgpu_buffer_rsrc_t ro = make_rsrc(a.o + q_row0 * D, (uint32_t)a.Nq * D * 2);
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(a.k + kv_head, (uint32_t)a.Nk * D * 2);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(a.v + kv_head, (uint32_t)a.Nk * D * 2);

  int kend = a.Nk;
  if (CAUSAL) kend = min(a.Nk, min(i0 + NW * 32, a.Nq) - 1 + off + 1);
  const int n_kt = kend > 0 ? (kend + BN - 1) / BN : 0;

  auto issue = [&](int t, char* kt_l, char* vt_l) __attribute__((always_inline)) {
    const int j0 = t * BN;
#pragma unroll
    for (int n = 0; n < LOADS; n++) {
      const int slab = n * NW + wave;
      const int p = slab * 64 + lane;
      const int r = p / CPR;
      const int cc = (p % CPR) ^ swz<D>(r);
      const uint32_t src = (uint32_t)(((j0 + r) * D + cc * 8) * 2);
      buf_load_lds16(rk, src, (lds_void*)(kt_l + slab * 1024));
      buf_load_lds16(rv, src, (lds_void*)(vt_l + slab * 1024));
    }
  };
  if (n_kt > 0) issue(0, smem, smem + 2 * TILE);

  bf16x8 qf[D / 16], df[D / 16];
#pragma unroll
  for (int s = 0; s < D / 16; s++) {
    const uint32_t src = (uint32_t)((qi * D + 16 * s + 8 * h32) * 2);
    qf[s] = __builtin_bit_cast(bf16x8, buf_load16(rq, src));
    df[s] = __builtin_bit_cast(bf16x8, buf_load16(rd, src));
  }
  const bool q_in = qi < a.Nq;
  // this row's record: LSE in log2 units (+inf for a row with no visible
  // key, so that all its P are 0) and D = dO . O, each lane summing its half
  // of the row and its partner lane the other.  Used here, and stored for the
  // dK/dV kernel, which runs after this one.
  float dpart = 0.0f;
#pragma unroll
  for (int s = 0; s < D / 16; s++) {
    const uint32_t src = (uint32_t)((qi * D + 16 * s + 8 * h32) * 2);
    const bf16x8 ov = __builtin_bit_cast(bf16x8, buf_load16(ro, src));
#pragma unroll
    for (int e = 0; e < 8; e++) dpart = __builtin_fmaf((float)df[s][e], (float)ov[e], dpart);
  }
  const float dsum = halves_sum(dpart);
  const float lse_q = q_in ? a.lse[q_row0 + qi] : 0.0f;
  const float l2q = (lse_q == kNegInf) ? __builtin_inff() : lse_q * kLog2e;
  const float ddq = q_in ? dsum : 0.0f;
  if (q_in && h32 == 0) {
    const size_t rec = ((size_t)b * a.Hq + hq) * (size_t)a.nq_pad + qi;
    a.stats[2 * rec] = l2q;
    a.stats[2 * rec + 1] = ddq;
  }

  // lane-constant LDS offsets: rows l32, chunk 2s + h of a K (or V) tile for
  // the A operands of S^T and dP^T; transposed K reads for the A operand of
  // dQ^T (rows 4h + (lane%16)/4 (+8), columns of block cb)
  const int swl = swz<D>(l32);
  int aoff[D / 16];
#pragma unroll
  for (int s = 0; s < D / 16; s++) aoff[s] = l32 * (D * 2) + (((2 * s + h32) ^ swl) << 4);
  int toff[D / 32][2];
#pragma unroll
  for (int cb = 0; cb < D / 32; cb++)
#pragma unroll
    for (int lh = 0; lh < 2; lh++)
      toff[cb][lh] = tile_off<D>(4 * h32 + ((lane & 15) >> 2) + 8 * lh, cb * 32 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3));

  f32x16 acc[D / 32];
#pragma unroll
  for (int cb = 0; cb < D / 32; cb++) acc[cb] = f32x16{};

  // one 32-key block kb of tile t, whose K and V sit in kcur and vcur
  auto block = [&](int t, auto kbc, const char* __restrict__ kcur, const char* __restrict__ vcur)
                   __attribute__((always_inline)) {
    constexpr int kb = decltype(kbc)::value;
    const int j0 = t * BN + kb * 32;
    if (CAUSAL && j0 > qw0 + 31 + off) return;  // no key of the block visible to this wave
    if (qw0 >= a.Nq) return;                     // a wave of padding rows
    const bool need_mask = (j0 + 32 > a.Nk) || (qw0 + 32 > a.Nq) || (CAUSAL && j0 + 31 > qw0 + off);
    const char* kt = kcur + kb * 32 * (D * 2);
    const char* vt = vcur + kb * 32 * (D * 2);
    // S^T = K Q^T and dP^T = V dO^T: keys on M, this wave's queries on N
    f32x16 st = f32x16{}, dpt = f32x16{};
#pragma unroll
    for (int s = 0; s < D / 16; s++) {
      st = mfma32(*(const bf16x8*)(kt + aoff[s]), qf[s], st);
      dpt = mfma32(*(const bf16x8*)(vt + aoff[s]), df[s], dpt);
    }
    // dS^T = P^T o (dP^T - D); keys j0 + 4h + c, c = 8(r/4) + r%4.  Key j is
    // visible iff the row exists, j < Nk and, causal, j <= qi + off: one lane
    // bound lim on c, so a masked element costs one compare with a constant
    const int lim = q_in ? (CAUSAL ? min(a.Nk, qi + off + 1) : a.Nk) - j0 - 4 * h32 : 0;
#pragma unroll
    for (int r = 0; r < 16; r++) {
      const float p = fast_exp2(__builtin_fmaf(st[r], a.c, -l2q));
      float ds = p * (dpt[r] - ddq);
      if (need_mask) ds = (8 * (r >> 2) + (r & 3) < lim) ? ds : 0.0f;
      dpt[r] = ds;
    }
    // dQ^T += K^T dS^T, 16 keys per MFMA (K read transposed)
#pragma unroll
    for (int hf = 0; hf < 2; hf++) {
      bf16x8 sb;
#pragma unroll
      for (int e = 0; e < 8; e++) sb[e] = to_bf16(dpt[8 * hf + e]);
      const char* kk = kt + 16 * hf * (D * 2);
#pragma unroll
      for (int cb = 0; cb < D / 32; cb++) {
        const bf16x8 ka = join_bf16(ds_read_tr16(kk + toff[cb][0]), ds_read_tr16(kk + toff[cb][1]));
        acc[cb] = mfma32(ka, sb, acc[cb]);
      }
    }
  };
  auto compute = [&](int t, const char* __restrict__ kcur, const char* __restrict__ vcur)
                     __attribute__((always_inline)) {
    block(t, std::integral_constant<int, 0>{}, kcur, vcur);
    // keep the two blocks apart: overlapping them would need a second set of
    // S^T / dP^T registers, more than a wave has at two waves per SIMD
    __builtin_amdgcn_sched_barrier(0);
    block(t, std::integral_constant<int, 1>{}, kcur, vcur);
    static_assert(KB == 2, "two 32-key blocks per tile");
  };

  // the restrict qualifiers tell the compiler the prefetch does not write
  // the stage being read; without them it waits for the prefetch before the
  // transposed K reads
  auto step = [&](int t, const char* __restrict__ kc, const char* __restrict__ vc, char* __restrict__ kn,
                  char* __restrict__ vn) __attribute__((always_inline)) {
    wait_vmem();
    __syncthreads();
    if (t + 1 < n_kt) issue(t + 1, kn, vn);
    compute(t, kc, vc);
  };
  for (int t = 0; t < n_kt; t += 2) {
    step(t, smem, smem + 2 * TILE, smem + TILE, smem + 3 * TILE);
    if (t + 1 >= n_kt) break;
    step(t + 1, smem + TILE, smem + 3 * TILE, smem, smem + 2 * TILE);
  }

  if (q_in) {
    // lane holds dims cb*32 + 8 g4 + 4h .. +3 of row qi
#pragma unroll
    for (int cb = 0; cb < D / 32; cb++)
#pragma unroll
      for (int g4 = 0; g4 < 4; g4++) {
        f32x4 w;
#pragma unroll
        for (int e = 0; e < 4; e++) w[e] = acc[cb][4 * g4 + e] * a.scale;
        const size_t at = (q_row0 + qi) * D + cb * 32 + 8 * g4 + 4 * h32;
        if constexpr (G16)
          *(bf16x4*)((__bf16*)a.dq + at) = bf16x4{to_bf16(w[0]), to_bf16(w[1]), to_bf16(w[2]), to_bf16(w[3])};
        else
          *(f32x4*)(a.dq + at) = w;
      }
  }
}

// ---------------------------------------------------------------------------
// dQ in two alternating wave groups (8 waves, 256 query rows; waves w and
// w + 4 share a SIMD), one 64-key tile per phase:
//
//   MFMA phase (tile t):  dQ^T += K(t-1)^T dS^T(t-1),  S^T(t), dP^T(t)
//   VALU phase (tile t):  dS^T(t) = P^T o (dP^T - D), masked, bf16
//
// Group 0 runs MFMA(t) in phase 2t and VALU(t) in phase 2t + 1, group 1 one
// phase later, with a workgroup barrier at every phase boundary.  Group 1
// loads K(t + 1) and V(t + 1) at the start of phase 2t (its VALU phase) into
// the buffers tile t - 2 left (three of each) and waits for them before
// phase 2t + 2.  Per 32-key half the arithmetic and its order are those of
// bwd_dq_kernel, so dQ is the same bits.
template <int D, bool CAUSAL, bool G16>
__global__ __launch_bounds__(512, 1) void bwd_dq_pp_kernel(BwdArgs a) {
  constexpr int NW = 8, BN = 64;
  constexpr int TILE = BN * D * 2;
  constexpr int CPR = D / 8;
  constexpr int LOADS = BN * CPR / (64 * 4);  // loads per wave of group 1 per K (or V) tile
  constexpr int BLK = 32 * (D * 2);            // bytes of one 32-key half of a tile
  static_assert(LOADS * 64 * 4 == BN * CPR, "tile must split evenly");
  __shared__ __attribute__((aligned(1024))) char k_st0[TILE], k_st1[TILE], k_st2[TILE];
  __shared__ __attribute__((aligned(1024))) char v_st0[TILE], v_st1[TILE], v_st2[TILE];

  const int lane = threadIdx.x & 63;
  const int wave = wave_id();
  const int grp = wave >> 2;
  const int h32 = lane >> 5;
  const int l32 = lane & 31;

  const WorkItem wi = lpt_order(blockIdx.x, a.B * a.Hkv, a.g * a.n_tiles);
  const int pair = wi.pair;
  const int rem = wi.sub;
  const int qt = CAUSAL ? (a.n_tiles - 1 - rem / a.g) : (rem / a.g);
  const int hq = (pair % a.Hkv) * a.g + rem % a.g;
  const int b = pair / a.Hkv;
  const int kvh = pair % a.Hkv;
  const int i0 = qt * NW * 32;
  const int qw0 = i0 + wave * 32;
  const int qi = qw0 + l32;
  const int off = a.Nk - a.Nq;

  const size_t q_row0 = ((size_t)b * a.Hq + hq) * (size_t)a.Nq;
  const size_t kv_head = ((size_t)b * a.Hkv + kvh) * (size_t)a.Nk * D;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(a.q + q_row0 * D, (uint32_t)a.Nq * D * 2);
  const __amdgpu_buffer_rsrc_t rd = make_rsrc(a.dout + q_row0 * D, (uint32_t)a.Nq * D * 2);
  const __amdgpu_buffer_rsrc_t ro = make_rsrc(a.o + q_row0 * D, (uint32_t)a.Nq * D * 2);
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(a.k + kv_head, (uint32_t)a.Nk * D * 2);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(a.v + kv_head, (uint32_t)a.Nk * D * 2);

  int kend = a.Nk;
  if (CAUSAL) kend = min(a.Nk, min(i0 + NW * 32, a.Nq) - 1 + off + 1);
  const int n = kend > 0 ? (kend + BN - 1) / BN : 0;

  // K (or V) tile t by all waves (issue1) or by the four waves of group 1
  auto issue1 = [&](int t, char* dst, __amdgpu_buffer_rsrc_t r) __attribute__((always_inline)) {
#pragma unroll
    for (int m = 0; m < LOADS / 2; m++) {
      const int slab = m * NW + wave;
      const int p = slab * 64 + lane;
      const int row = p / CPR;
      const int c = (p % CPR) ^ swz<D>(row);
      buf_load_lds16(r, (uint32_t)(((t * BN + row) * D + c * 8) * 2), (lds_void*)(dst + slab * 1024));
    }
  };
  auto issue4 = [&](int t, char* dst, __amdgpu_buffer_rsrc_t r) __attribute__((always_inline)) {
#pragma unroll
    for (int m = 0; m < LOADS; m++) {
      const int slab = m * 4 + (wave & 3);
      const int p = slab * 64 + lane;
      const int row = p / CPR;
      const int c = (p % CPR) ^ swz<D>(row);
      buf_load_lds16(r, (uint32_t)(((t * BN + row) * D + c * 8) * 2), (lds_void*)(dst + slab * 1024));
    }
  };
  if (n > 0) {
    issue1(0, k_st0, rk);
    issue1(0, v_st0, rv);
  }

  bf16x8 qf[D / 16], df[D / 16];
#pragma unroll
  for (int s = 0; s < D / 16; s++) {
    const uint32_t src = (uint32_t)((qi * D + 16 * s + 8 * h32) * 2);
    qf[s] = __builtin_bit_cast(bf16x8, buf_load16(rq, src));
    df[s] = __builtin_bit_cast(bf16x8, buf_load16(rd, src));
  }
  const bool q_in = qi < a.Nq;
  // the row record, as in bwd_dq_kernel
  float dpart = 0.0f;
#pragma unroll
  for (int s = 0; s < D / 16; s++) {
    const uint32_t src = (uint32_t)((qi * D + 16 * s + 8 * h32) * 2);
    const bf16x8 ov = __builtin_bit_cast(bf16x8, buf_load16(ro, src));
#pragma unroll
    for (int e = 0; e < 8; e++) dpart = __builtin_fmaf((float)df[s][e], (float)ov[e], dpart);
  }
  const float dsum = halves_sum(dpart);
  const float lse_q = q_in ? a.lse[q_row0 + qi] : 0.0f;
  const float l2q = (lse_q == kNegInf) ? __builtin_inff() : lse_q * kLog2e;
  const float ddq = q_in ? dsum : 0.0f;
  if (q_in && h32 == 0) {
    const size_t rec = ((size_t)b * a.Hq + hq) * (size_t)a.nq_pad + qi;
    a.stats[2 * rec] = l2q;
    a.stats[2 * rec + 1] = ddq;
  }
  // K(0), V(0) and the fragments complete here, so that no later wait has to
  // cover the fragment registers
  wait_vmem();

  const int swl = swz<D>(l32);
  int aoff[D / 16];
#pragma unroll
  for (int s = 0; s < D / 16; s++) aoff[s] = l32 * (D * 2) + (((2 * s + h32) ^ swl) << 4);
  int toff[D / 32][2];
#pragma unroll
  for (int cb = 0; cb < D / 32; cb++)
#pragma unroll
    for (int lh = 0; lh < 2; lh++)
      toff[cb][lh] = tile_off<D>(4 * h32 + ((lane & 15) >> 2) + 8 * lh, cb * 32 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3));

  f32x16 acc[D / 32];
#pragma unroll
  for (int cb = 0; cb < D / 32; cb++) acc[cb] = f32x16{};
  f32x16 st[2], dpt[2];  // S^T, dP^T of a tile's two halves between its MFMA and VALU phases
  bf16x8 sb[2][2];       // dS^T of the two halves between the VALU phase and the next MFMA phase

  // half kb of tile t has keys this wave's rows see: halves 0 .. n_vis - 1
  // (up to the last row's diagonal when causal; none for a wave whose rows
  // all lie past the last query)
  int n_vis = 2 * n;
  if (CAUSAL) {
    const int x = qw0 + 31 + off;  // half h is visible iff 32 h <= x
    n_vis = x < 0 ? 0 : min(2 * n, x / 32 + 1);
  }
  if (qw0 >= a.Nq) n_vis = 0;
  auto visible = [&](int t, int kb) __attribute__((always_inline)) { return t >= 0 && 2 * t + kb < n_vis; };
  // MFMA phase of tile t: dQ of tile t - 1 (K in kp), S^T and dP^T of tile t
  // (K, V in kc, vc)
  auto mfma_phase = [&](int t, const char* __restrict__ kp, const char* __restrict__ kc,
                        const char* __restrict__ vc) __attribute__((always_inline)) {
#pragma unroll
    for (int kb = 0; kb < 2; kb++) {
      if (visible(t - 1, kb)) {
#pragma unroll
        for (int hf = 0; hf < 2; hf++) {
          const char* kk = kp + kb * BLK + 16 * hf * (D * 2);
#pragma unroll
          for (int cb = 0; cb < D / 32; cb++) {
            const bf16x8 ka = join_bf16(ds_read_tr16(kk + toff[cb][0]), ds_read_tr16(kk + toff[cb][1]));
            acc[cb] = mfma32(ka, sb[kb][hf], acc[cb]);
          }
        }
#if ATTN_BWD_DQ_PP_GROUPS
        // operand reads three contractions ahead of their MFMAs
        __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
#pragma unroll
        for (int i = 0; i < 2 * (D / 32) - 3; i++) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 3, 0);
#endif
      }
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int kb = 0; kb < 2; kb++) {
      if (visible(t, kb)) {
        st[kb] = f32x16{};
        dpt[kb] = f32x16{};
#pragma unroll
        for (int s = 0; s < D / 16; s++) {
          st[kb] = mfma32(*(const bf16x8*)(kc + kb * BLK + aoff[s]), qf[s], st[kb]);
          dpt[kb] = mfma32(*(const bf16x8*)(vc + kb * BLK + aoff[s]), df[s], dpt[kb]);
        }
#if ATTN_BWD_DQ_PP_GROUPS
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
        for (int i = 0; i < 2 * (D / 16) - 4; i++) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
#endif
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // VALU phase of tile t: dS^T = P^T o (dP^T - D), masked, as bf16
  auto valu_phase = [&](int t) __attribute__((always_inline)) {
#pragma unroll
    for (int kb = 0; kb < 2; kb++) {
      if (!visible(t, kb)) continue;
      const int j0 = t * BN + kb * 32;
      const bool need_mask = (j0 + 32 > a.Nk) || (qw0 + 32 > a.Nq) || (CAUSAL && j0 + 31 > qw0 + off);
      const int lim = q_in ? (CAUSAL ? min(a.Nk, qi + off + 1) : a.Nk) - j0 - 4 * h32 : 0;
#pragma unroll
      for (int r = 0; r < 16; r++) {
        const float p = fast_exp2(__builtin_fmaf(st[kb][r], a.c, -l2q));
        float ds = p * (dpt[kb][r] - ddq);
        if (need_mask) ds = (8 * (r >> 2) + (r & 3) < lim) ? ds : 0.0f;
        dpt[kb][r] = ds;
      }
#pragma unroll
      for (int hf = 0; hf < 2; hf++)
#pragma unroll
        for (int e = 0; e < 8; e++) sb[kb][hf][e] = to_bf16(dpt[kb][8 * hf + e]);
    }
  };
  // Both groups pass the same barriers; each runs its own loop so that the
  // register allocator sees one phase order at a time.
  if (grp == 0) {
    auto tile = [&](int t, const char* __restrict__ kp, const char* __restrict__ kc, const char* __restrict__ vc)
                    __attribute__((always_inline)) {
      barrier_nofence();  // phase 2t
      mfma_phase(t, kp, kc, vc);
      barrier_nofence();  // phase 2t + 1
      valu_phase(t);
    };
    for (int t = 0; t <= n; t += 3) {
      tile(t, k_st2, k_st0, v_st0);
      if (t + 1 > n) break;
      tile(t + 1, k_st0, k_st1, v_st1);
      if (t + 2 > n) break;
      tile(t + 2, k_st1, k_st2, v_st2);
    }
  } else {
    auto tile = [&](int t, const char* __restrict__ kp, const char* __restrict__ kc, const char* __restrict__ vc,
                    char* __restrict__ kn, char* __restrict__ vn) __attribute__((always_inline)) {
      wait_vmem();        // K(t), V(t), loaded at the start of phase 2t - 2
      barrier_nofence();  // phase 2t
      if (t + 1 < n) {
        issue4(t + 1, kn, rk);
        issue4(t + 1, vn, rv);
      }
      valu_phase(t - 1);
      barrier_nofence();  // phase 2t + 1
      mfma_phase(t, kp, kc, vc);
    };
    for (int t = 0; t <= n; t += 3) {
      tile(t, k_st2, k_st0, v_st0, k_st1, v_st1);
      if (t + 1 > n) break;
      tile(t + 1, k_st0, k_st1, v_st1, k_st2, v_st2);
      if (t + 2 > n) break;
      tile(t + 2, k_st1, k_st2, v_st2, k_st0, v_st0);
    }
  }

  if (q_in) {
#pragma unroll
    for (int cb = 0; cb < D / 32; cb++)
#pragma unroll
      for (int g4 = 0; g4 < 4; g4++) {
        f32x4 w;
#pragma unroll
        for (int e = 0; e < 4; e++) w[e] = acc[cb][4 * g4 + e] * a.scale;
        const size_t at = (q_row0 + qi) * D + cb * 32 + 8 * g4 + 4 * h32;
        if constexpr (G16)
          *(bf16x4*)((__bf16*)a.dq + at) = bf16x4{to_bf16(w[0]), to_bf16(w[1]), to_bf16(w[2]), to_bf16(w[3])};
        else
          *(f32x4*)(a.dq + at) = w;
      }
  }
}

template <int D, bool CAUSAL, int NW>
hipError_t launch_nw(const BwdArgs& a, hipStream_t s) {
  BwdArgs qa = a;
  qa.n_tiles = (a.Nq + NW * 32 - 1) / (NW * 32);
  qa.n_wgs = a.B * a.Hq * qa.n_tiles;
  if (a.grad_bf16)
    hipLaunchKernelGGL((bwd_dq_kernel<D, NW, CAUSAL, true>), dim3(qa.n_wgs), dim3(NW * 64), 0, s, qa);
  else
    hipLaunchKernelGGL((bwd_dq_kernel<D, NW, CAUSAL, false>), dim3(qa.n_wgs), dim3(NW * 64), 0, s, qa);
  return hipGetLastError();
}

template <int D, bool CAUSAL>
hipError_t launch_t(const BwdArgs& a, hipStream_t s) {
  // 8 waves (256 rows) per workgroup when that still gives two workgroups per
  // CU over the launch (the forward's rule; ~1 % faster at 4 x 16 heads x
  // 2048), run as the two-group kernel (dQ kernel 3-5 % faster than the
  // one-group 8-wave kernel at 4 x 16 heads x 2048, d = 64 and 128)
  const bool big = (int64_t)a.B * a.Hq * ((a.Nq + 255) / 256) >= 2 * 256;
  if (big && ATTN_BWD_DQ_PP) {
    BwdArgs qa = a;
    qa.n_tiles = (a.Nq + 255) / 256;
    qa.n_wgs = a.B * a.Hq * qa.n_tiles;
    if (a.grad_bf16)
      hipLaunchKernelGGL((bwd_dq_pp_kernel<D, CAUSAL, true>), dim3(qa.n_wgs), dim3(512), 0, s, qa);
    else
      hipLaunchKernelGGL((bwd_dq_pp_kernel<D, CAUSAL, false>), dim3(qa.n_wgs), dim3(512), 0, s, qa);
    return hipGetLastError();
  }
  return big ? launch_nw<D, CAUSAL, 8>(a, s) : launch_nw<D, CAUSAL, 4>(a, s);
}

}  // namespace

hipError_t launch_dq(const BwdArgs& a, int d, bool causal, hipStream_t s) {
  if (d == 128) return causal ? launch_t<128, true>(a, s) : launch_t<128, false>(a, s);
  return causal ? launch_t<64, true>(a, s) : launch_t<64, false>(a, s);
}

}  // namespace bwd
}  // namespace attn
