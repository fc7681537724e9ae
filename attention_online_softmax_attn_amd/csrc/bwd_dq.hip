// Backward kernels of softmax attention on gfx950, part 2: dQ (the formulas
// and the kernel split are stated in bwd_common.hpp).  Built with the default
// machine scheduler; the dK/dV file uses the ILP-maximising one.
#include "bwd_common.hpp"

namespace attn {
namespace bwd {

namespace {

// ---------------------------------------------------------------------------
// dQ.  Each wave owns 32 query rows; key tiles of BN keys stream through LDS
// and are processed in 32-key blocks.
template <int D, int NW, int BN, bool CAUSAL>
__global__ __launch_bounds__(NW * 64, ATTN_BWD_Q_OCC) void bwd_dq_kernel(BwdArgs a) {
  constexpr int TILE = BN * D * 2;
  constexpr int CPR = D / 8;
  constexpr int LOADS = BN * CPR / (64 * NW);
  constexpr int KB = BN / 32;
  static_assert(LOADS * 64 * NW == BN * CPR, "tile must split evenly");
  __shared__ __attribute__((aligned(1024))) char smem[4 * TILE];  // [K0 | V0 | K1 | V1]

  const int lane = threadIdx.x & 63;
  const int wave = wave_id();
  const int h32 = lane >> 5;
  const int l32 = lane & 31;

  const int work = xcd_remap(blockIdx.x, a.n_wgs);
  const int per_pair = a.g * a.n_tiles;
  const int pair = work / per_pair;
  const int rem = work % per_pair;
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
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(a.k + kv_head, (uint32_t)a.Nk * D * 2);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(a.v + kv_head, (uint32_t)a.Nk * D * 2);

  int kend = a.Nk;
  if (CAUSAL) kend = min(a.Nk, min(i0 + NW * 32, a.Nq) - 1 + off + 1);
  const int n_kt = kend > 0 ? (kend + BN - 1) / BN : 0;

  auto issue = [&](int t, char* kt_l, char* vt_l) {
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
  if (n_kt > 0) issue(0, smem, smem + TILE);

  bf16x8 qf[D / 16], df[D / 16];
#pragma unroll
  for (int s = 0; s < D / 16; s++) {
    const uint32_t src = (uint32_t)((qi * D + 16 * s + 8 * h32) * 2);
    qf[s] = __builtin_bit_cast(bf16x8, buf_load16(rq, src));
    df[s] = __builtin_bit_cast(bf16x8, buf_load16(rd, src));
  }
  const bool q_in = qi < a.Nq;
  const size_t rec = ((size_t)b * a.Hq + hq) * (size_t)a.nq_pad + qi;
  const float l2q = q_in ? a.stats[2 * rec] : 0.0f;
  const float ddq = q_in ? a.stats[2 * rec + 1] : 0.0f;

  f32x16 acc[D / 32];
#pragma unroll
  for (int cb = 0; cb < D / 32; cb++) acc[cb] = f32x16{};
  const int swl = swz<D>(l32);

  // S^T and dP^T of 32-key block kb: keys on M, this wave's queries on N
  // (fragments read ahead of the contractions, as in the dK/dV kernel)
  auto sdp = [&](const char* kt_l, const char* vt_l, int kb, f32x16& st, f32x16& dpt) {
    st = f32x16{};
    dpt = f32x16{};
    if (ATTN_BWD_PIPE) {
      bf16x8 ka[D / 16], va[D / 16];
#pragma unroll
      for (int s = 0; s < D / 16; s++) {
        const int off_b = (kb * 32 + l32) * (D * 2) + (((2 * s + h32) ^ swl) << 4);
        ka[s] = *(const bf16x8*)(kt_l + off_b);
        va[s] = *(const bf16x8*)(vt_l + off_b);
      }
#pragma unroll
      for (int s = 0; s < D / 16; s++) {
        st = mfma32(ka[s], qf[s], st);
        dpt = mfma32(va[s], df[s], dpt);
      }
    } else {
#pragma unroll
      for (int s = 0; s < D / 16; s++) {
        const int off_b = (kb * 32 + l32) * (D * 2) + (((2 * s + h32) ^ swl) << 4);
        st = mfma32(*(const bf16x8*)(kt_l + off_b), qf[s], st);
        dpt = mfma32(*(const bf16x8*)(vt_l + off_b), df[s], dpt);
      }
    }
  };
  // dS^T = P^T o (dP^T - D) into dpt; keys j0 + 32 kb + 8(r/4) + 4h + r%4
  auto pds = [&](int j0, int kb, bool mask, const f32x16& st, f32x16& dpt) {
#pragma unroll
    for (int r = 0; r < 16; r++) {
      float p = fast_exp2(__builtin_fmaf(st[r], a.c, -l2q));
      if (mask) {
        const int j = j0 + kb * 32 + 8 * (r >> 2) + 4 * h32 + (r & 3);
        bool ok = q_in && (j < a.Nk);
        if (CAUSAL) ok = ok && (j <= qi + off);
        p = ok ? p : 0.0f;
      }
      dpt[r] = p * (dpt[r] - ddq);
    }
  };
  // dQ^T += K^T dS^T over the 32 keys of block kb
  auto dqk = [&](const char* kt_l, int kb, const f32x16& dpt) {
#pragma unroll
    for (int hf = 0; hf < 2; hf++) {
      const int kr = kb * 32 + 16 * hf + 4 * h32 + ((lane & 15) >> 2);
      bf16x8 ka[D / 32];
#pragma unroll
      for (int cb = 0; cb < D / 32; cb++) {
        const int kc = cb * 32 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
        ka[cb] = join_bf16(ds_read_tr16(kt_l + tile_off<D>(kr, kc)), ds_read_tr16(kt_l + tile_off<D>(kr + 8, kc)));
      }
      bf16x8 sb;
#pragma unroll
      for (int e = 0; e < 8; e++) sb[e] = to_bf16(dpt[8 * hf + e]);
#pragma unroll
      for (int cb = 0; cb < D / 32; cb++) acc[cb] = mfma32(ka[cb], sb, acc[cb]);
    }
  };

  auto compute = [&](int t, const char* kt_l, const char* vt_l) {
    const int j0 = t * BN;
    if (CAUSAL && j0 > qw0 + 31 + off) return;
    const bool need_mask = (j0 + BN > a.Nk) || (qw0 + 32 > a.Nq) || (CAUSAL && j0 + BN - 1 > qw0 + off);
    if (!need_mask && !ATTN_BWD_PIPE) {
#pragma unroll
      for (int kb = 0; kb < KB; kb++) {
        f32x16 st, dpt;
        sdp(kt_l, vt_l, kb, st, dpt);
        pds(j0, kb, false, st, dpt);
        dqk(kt_l, kb, dpt);
      }
    } else if (!need_mask) {
      f32x16 st[2], dpt[2];
      sdp(kt_l, vt_l, 0, st[0], dpt[0]);
#pragma unroll
      for (int kb = 0; kb < KB; kb++) {
        if (kb + 1 < KB) sdp(kt_l, vt_l, kb + 1, st[(kb + 1) & 1], dpt[(kb + 1) & 1]);
        pds(j0, kb, false, st[kb & 1], dpt[kb & 1]);
        dqk(kt_l, kb, dpt[kb & 1]);
      }
    } else {
#pragma unroll
      for (int kb = 0; kb < KB; kb++) {
        if (CAUSAL && j0 + 32 * kb > qw0 + 31 + off) continue;
        f32x16 st, dpt;
        sdp(kt_l, vt_l, kb, st, dpt);
        pds(j0, kb, true, st, dpt);
        dqk(kt_l, kb, dpt);
      }
    }
  };

  auto step = [&](int t, const char* __restrict__ kc, const char* __restrict__ vc, char* __restrict__ kn,
                  char* __restrict__ vn) {
    wait_vmem();
    __syncthreads();
    if (t + 1 < n_kt) issue(t + 1, kn, vn);
    compute(t, kc, vc);
  };
  char* const b0 = smem;
  char* const b1 = smem + 2 * TILE;
  for (int t = 0; t < n_kt; t += 2) {
    step(t, b0, b0 + TILE, b1, b1 + TILE);
    if (t + 1 >= n_kt) break;
    step(t + 1, b1, b1 + TILE, b0, b0 + TILE);
  }

  if (q_in) {
    float* row = a.dq + (q_row0 + qi) * D;
#pragma unroll
    for (int cb = 0; cb < D / 32; cb++)
#pragma unroll
      for (int g4 = 0; g4 < 4; g4++) {
        f32x4 w;
#pragma unroll
        for (int e = 0; e < 4; e++) w[e] = acc[cb][4 * g4 + e] * a.scale;
        *(f32x4*)(row + cb * 32 + 8 * g4 + 4 * h32) = w;
      }
  }
}

template <int D, bool CAUSAL>
hipError_t launch_t(const BwdArgs& a, hipStream_t s) {
  constexpr int NW = 4;
  BwdArgs qa = a;
  qa.n_tiles = (a.Nq + NW * 32 - 1) / (NW * 32);
  qa.n_wgs = a.B * a.Hq * qa.n_tiles;
  hipLaunchKernelGGL((bwd_dq_kernel<D, NW, ATTN_BWD_DQ_BN, CAUSAL>), dim3(qa.n_wgs), dim3(NW * 64), 0, s, qa);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_dq(const BwdArgs& a, int d, bool causal, hipStream_t s) {
  if (d == 128) return causal ? launch_t<128, true>(a, s) : launch_t<128, false>(a, s);
  return causal ? launch_t<64, true>(a, s) : launch_t<64, false>(a, s);
}

}  // namespace bwd
}  // namespace attn
