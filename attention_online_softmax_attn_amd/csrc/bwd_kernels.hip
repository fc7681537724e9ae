// Backward kernels for gfx950: gradients of softmax attention from the saved
// log-sum-exp.  With s = scale * Q K^T, P = exp(s - LSE), the gradient of O
// with respect to its inputs is
//
//   dV = P^T dO,   dP = dO V^T,   D_i = rowsum(dO o O)_i,   dS = P o (dP - D),
//   dQ = scale * dS K,   dK = scale * dS^T Q,
//
// (the identity sum_j P_ij dP_ij = dO_i . O_i gives D without a pass over
// keys).  "Não escreva kernels, derive-os" (FAQ entry "O que o Tang propõe de
// diferente?") obtains its backward by rewriting and notes in "Aprofundamento"
// (third paragraph) that a fused bf16 backward missed an fp32 tolerance; this
// build keeps bf16 MFMA operands with fp32 accumulation and writes fp32
// gradients.
//
// Three kernels, no atomics (every output element has one writer):
//   bwd_pre   D_i = dO_i . O_i                              (one pass over O, dO)
//   bwd_dkdv  workgroup = (b, kv head, 32*NW keys).  K and V fragments stay in
//             registers; for every query head of the group and every query
//             tile that can see the keys, Q and dO stream through LDS.
//             S = Q K^T and dP = dO V^T put keys on the MFMA N dimension, so
//             P and dS come out with one key per lane and feed
//             dV += P^T dO and dK += dS^T Q straight from registers, with dO
//             and Q read transposed from LDS.
//   bwd_dq    workgroup = (b, query head, 32*NW queries), the forward's
//             layout: S^T = K Q^T and dP^T = V dO^T keep one query per lane;
//             dQ^T += K^T dS^T reads K transposed from LDS.
#include "device_common.hpp"
#include "kernels.h"

namespace attn {

namespace {

struct BwdArgs {
  const __bf16* q;
  const __bf16* k;
  const __bf16* v;
  const __bf16* o;
  const __bf16* dout;
  const float* lse;
  float* dq;
  float* dk;
  float* dv;
  float* delta;
  int B, Hq, Hkv, Nq, Nk, g;
  int n_tiles, n_wgs;
  float c;      // scale * log2(e)
  float scale;
};

// D_i = dO_i . O_i: 16 lanes per row, 8 elements per lane (d = 128) or 4 (d = 64)
template <int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(BwdArgs a) {
  constexpr int EPL = D / 16;
  const int rows = a.B * a.Hq * a.Nq;
  const int row = blockIdx.x * 16 + (threadIdx.x >> 4);
  const int sub = threadIdx.x & 15;
  float s = 0.0f;
  if (row < rows) {
    const __bf16* o = a.o + (size_t)row * D + sub * EPL;
    const __bf16* g = a.dout + (size_t)row * D + sub * EPL;
#pragma unroll
    for (int e = 0; e < EPL; e++) s += (float)o[e] * (float)g[e];
  }
#pragma unroll
  for (int w = 8; w >= 1; w >>= 1) s += __shfl_xor(s, w, 16);
  if (row < rows && sub == 0) a.delta[row] = s;
}

template <int D, int NW, bool CAUSAL>
__global__ __launch_bounds__(NW * 64, 1) void bwd_dkdv_kernel(BwdArgs a) {
  constexpr int BQ = 32;                 // queries per tile
  constexpr int TILE = BQ * D * 2;       // bytes of one Q or dO tile
  constexpr int CPR = D / 8;
  constexpr int LOADS = BQ * CPR / (64 * NW);
  static_assert(LOADS * 64 * NW == BQ * CPR, "tile must split evenly");
  __shared__ __attribute__((aligned(1024))) char smem[4 * TILE];  // [Q0 | dO0 | Q1 | dO1]

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int h32 = lane >> 5;
  const int l32 = lane & 31;

  const int work = xcd_remap(blockIdx.x, a.n_wgs);
  const int kt = work % a.n_tiles;  // causal: early key tiles are seen by the most queries, so they go first
  const int pair = work / a.n_tiles;
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

  auto issue = [&](int it, char* qt_l, char* dt_l) {
    const int hq = head_of(it);
    const int i0 = qtile_of(it) * BQ;
    const size_t q_head = ((size_t)b * a.Hq + hq) * (size_t)a.Nq * D;
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(a.q + q_head, (uint32_t)a.Nq * D * 2);
    const __amdgpu_buffer_rsrc_t rd = make_rsrc(a.dout + q_head, (uint32_t)a.Nq * D * 2);
#pragma unroll
    for (int n = 0; n < LOADS; n++) {
      const int slab = n * NW + wave;
      const int p = slab * 64 + lane;
      const int r = p / CPR;
      const int cc = (p % CPR) ^ swz<D>(r);
      const uint32_t src = (uint32_t)(((i0 + r) * D + cc * 8) * 2);
      buf_load_lds16(rq, src, (lds_void*)(qt_l + slab * 1024));
      buf_load_lds16(rd, src, (lds_void*)(dt_l + slab * 1024));
    }
  };

  auto compute = [&](int it, const char* qt_l, const char* dt_l) {
    const int hq = head_of(it);
    const int i0 = qtile_of(it) * BQ;
    if (CAUSAL && i0 + BQ - 1 + off < jw) return;  // no query of the tile sees this wave's keys
    const bool need_mask = (i0 + BQ > a.Nq) || (jw + 32 > a.Nk) || (CAUSAL && i0 + off < jw + 31);
    // per-row statistics for rows 8(r/4) + 4h + r%4: LSE (log2 units) and D
    const size_t rbase = ((size_t)b * a.Hq + hq) * a.Nq;
    float l2[16], dd[16];
#pragma unroll
    for (int r4 = 0; r4 < 4; r4++) {
#pragma unroll
      for (int e = 0; e < 4; e++) {
        const int i = i0 + 8 * r4 + 4 * h32 + e;
        const bool in = i < a.Nq;
        l2[4 * r4 + e] = in ? a.lse[rbase + i] * kLog2e : 0.0f;
        dd[4 * r4 + e] = in ? a.delta[rbase + i] : 0.0f;
      }
    }
    // S = Q K^T and dP = dO V^T (queries are M, this wave's keys are N)
    f32x16 s_acc = f32x16{}, dp_acc = f32x16{};
#pragma unroll
    for (int s = 0; s < D / 16; s++) {
      const int off_b = l32 * (D * 2) + (((2 * s + h32) ^ swl) << 4);
      const bf16x8 qa = *(const bf16x8*)(qt_l + off_b);
      const bf16x8 da = *(const bf16x8*)(dt_l + off_b);
      s_acc = mfma32(qa, kf[s], s_acc);
      dp_acc = mfma32(da, vf[s], dp_acc);
    }
    // P and dS (P = 0 where the key is not visible, the row is padding, or the key is past Nk)
#pragma unroll
    for (int r = 0; r < 16; r++) {
      float p = fast_exp2(__builtin_fmaf(s_acc[r], a.c, -l2[r]));
      if (need_mask) {
        const int i = i0 + 8 * (r >> 2) + 4 * h32 + (r & 3);
        bool ok = (i < a.Nq) && (jl < a.Nk);
        if (CAUSAL) ok = ok && (jl <= i + off);
        if (!ok) p = 0.0f;
      }
      s_acc[r] = p;
      dp_acc[r] = p * (dp_acc[r] - dd[r]);
    }
    // dV += P^T dO, dK += dS^T Q: 16 queries per MFMA, dO and Q read transposed
#pragma unroll
    for (int hf = 0; hf < 2; hf++) {
      bf16x8 pa, sa;
#pragma unroll
      for (int e = 0; e < 8; e++) {
        pa[e] = to_bf16(s_acc[8 * hf + e]);
        sa[e] = to_bf16(dp_acc[8 * hf + e]);
      }
      const int tr = 16 * hf + 4 * h32 + ((lane & 15) >> 2);
#pragma unroll
      for (int cb = 0; cb < D / 32; cb++) {
        const int tc = cb * 32 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
        const int o1 = tile_off<D>(tr, tc), o2 = tile_off<D>(tr + 8, tc);
        const bf16x8 dob = join_bf16(ds_read_tr16(dt_l + o1), ds_read_tr16(dt_l + o2));
        const bf16x8 qb = join_bf16(ds_read_tr16(qt_l + o1), ds_read_tr16(qt_l + o2));
        dv_acc[cb] = mfma32(pa, dob, dv_acc[cb]);
        dk_acc[cb] = mfma32(sa, qb, dk_acc[cb]);
      }
    }
  };

  auto step = [&](int it, const char* __restrict__ qc, const char* __restrict__ dc, char* __restrict__ qn,
                  char* __restrict__ dn) {
    wait_vmem();
    __syncthreads();
    if (it + 1 < n_iter) issue(it + 1, qn, dn);
    compute(it, qc, dc);
  };
  char* const b0 = smem;
  char* const b1 = smem + 2 * TILE;
  if (n_iter > 0) issue(0, b0, b0 + TILE);
  for (int it = 0; it < n_iter; it += 2) {
    step(it, b0, b0 + TILE, b1, b1 + TILE);
    if (it + 1 >= n_iter) break;
    step(it + 1, b1, b1 + TILE, b0, b0 + TILE);
  }

  // dV, dK accumulators: lane holds dim cb*32 + l32 of keys jw + 8(r/4) + 4h + r%4
  float* dkh = a.dk + kv_head;
  float* dvh = a.dv + kv_head;
#pragma unroll
  for (int r = 0; r < 16; r++) {
    const int j = jw + 8 * (r >> 2) + 4 * h32 + (r & 3);
    if (j < a.Nk) {
#pragma unroll
      for (int cb = 0; cb < D / 32; cb++) {
        dkh[(size_t)j * D + cb * 32 + l32] = dk_acc[cb][r] * a.scale;
        dvh[(size_t)j * D + cb * 32 + l32] = dv_acc[cb][r];
      }
    }
  }
}

template <int D, int NW, bool CAUSAL>
__global__ __launch_bounds__(NW * 64, 1) void bwd_dq_kernel(BwdArgs a) {
  constexpr int BN = 64;
  constexpr int TILE = BN * D * 2;
  constexpr int CPR = D / 8;
  constexpr int LOADS = BN * CPR / (64 * NW);
  static_assert(LOADS * 64 * NW == BN * CPR, "tile must split evenly");
  __shared__ __attribute__((aligned(1024))) char smem[4 * TILE];  // [K0 | V0 | K1 | V1]

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
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

  const size_t q_head = ((size_t)b * a.Hq + hq) * (size_t)a.Nq * D;
  const size_t kv_head = ((size_t)b * a.Hkv + kvh) * (size_t)a.Nk * D;
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(a.q + q_head, (uint32_t)a.Nq * D * 2);
  const __amdgpu_buffer_rsrc_t rd = make_rsrc(a.dout + q_head, (uint32_t)a.Nq * D * 2);
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
  const float l2q = q_in ? a.lse[((size_t)b * a.Hq + hq) * a.Nq + qi] * kLog2e : 0.0f;
  const float ddq = q_in ? a.delta[((size_t)b * a.Hq + hq) * a.Nq + qi] : 0.0f;

  f32x16 acc[D / 32];
#pragma unroll
  for (int cb = 0; cb < D / 32; cb++) acc[cb] = f32x16{};
  const int swl = swz<D>(l32);

  auto compute = [&](int t, const char* kt_l, const char* vt_l) {
    const int j0 = t * BN;
    if (CAUSAL && j0 > qw0 + 31 + off) return;
    const bool need_mask = (j0 + BN > a.Nk) || !q_in || (CAUSAL && j0 + BN - 1 > qw0 + off) ||
                           (qw0 + 32 > a.Nq);
    f32x16 st[BN / 32], dpt[BN / 32];
#pragma unroll
    for (int kb = 0; kb < BN / 32; kb++) {
      st[kb] = f32x16{};
      dpt[kb] = f32x16{};
    }
#pragma unroll
    for (int s = 0; s < D / 16; s++) {
#pragma unroll
      for (int kb = 0; kb < BN / 32; kb++) {
        const int off_b = (kb * 32 + l32) * (D * 2) + (((2 * s + h32) ^ swl) << 4);
        st[kb] = mfma32(*(const bf16x8*)(kt_l + off_b), qf[s], st[kb]);
        dpt[kb] = mfma32(*(const bf16x8*)(vt_l + off_b), df[s], dpt[kb]);
      }
    }
#pragma unroll
    for (int kb = 0; kb < BN / 32; kb++)
#pragma unroll
      for (int r = 0; r < 16; r++) {
        float p = fast_exp2(__builtin_fmaf(st[kb][r], a.c, -l2q));
        if (need_mask) {
          const int j = j0 + kb * 32 + 8 * (r >> 2) + 4 * h32 + (r & 3);
          bool ok = q_in && (j < a.Nk);
          if (CAUSAL) ok = ok && (j <= qi + off);
          if (!ok) p = 0.0f;
        }
        dpt[kb][r] = p * (dpt[kb][r] - ddq);
      }
    // dQ^T += K^T dS^T
#pragma unroll
    for (int kb = 0; kb < BN / 32; kb++)
#pragma unroll
      for (int hf = 0; hf < 2; hf++) {
        bf16x8 sb;
#pragma unroll
        for (int e = 0; e < 8; e++) sb[e] = to_bf16(dpt[kb][8 * hf + e]);
        const int kr = kb * 32 + 16 * hf + 4 * h32 + ((lane & 15) >> 2);
#pragma unroll
        for (int cb = 0; cb < D / 32; cb++) {
          const int kc = cb * 32 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
          const bf16x8 ka = join_bf16(ds_read_tr16(kt_l + tile_off<D>(kr, kc)), ds_read_tr16(kt_l + tile_off<D>(kr + 8, kc)));
          acc[cb] = mfma32(ka, sb, acc[cb]);
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
    float* row = a.dq + q_head + (size_t)qi * D;
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
hipError_t launch(const BwdProblem& p, hipStream_t s) {
  constexpr int NW = 4;
  BwdArgs a;
  a.q = (const __bf16*)p.q;
  a.k = (const __bf16*)p.k;
  a.v = (const __bf16*)p.v;
  a.o = (const __bf16*)p.o;
  a.dout = (const __bf16*)p.dout;
  a.lse = p.lse;
  a.dq = p.dq;
  a.dk = p.dk;
  a.dv = p.dv;
  a.delta = p.delta;
  a.B = (int)p.B;
  a.Hq = (int)p.Hq;
  a.Hkv = (int)p.Hkv;
  a.Nq = (int)p.Nq;
  a.Nk = (int)p.Nk;
  a.g = a.Hq / a.Hkv;
  a.c = p.scale * kLog2e;
  a.scale = p.scale;
  const int rows = a.B * a.Hq * a.Nq;
  if (rows > 0) {
    hipLaunchKernelGGL((bwd_pre_kernel<D>), dim3((rows + 15) / 16), dim3(256), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (a.Nk > 0) {
    BwdArgs kv = a;
    kv.n_tiles = (a.Nk + NW * 32 - 1) / (NW * 32);
    kv.n_wgs = a.B * a.Hkv * kv.n_tiles;
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, NW, CAUSAL>), dim3(kv.n_wgs), dim3(NW * 64), 0, s, kv);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (rows > 0) {
    BwdArgs qa = a;
    qa.n_tiles = (a.Nq + NW * 32 - 1) / (NW * 32);
    qa.n_wgs = a.B * a.Hq * qa.n_tiles;
    hipLaunchKernelGGL((bwd_dq_kernel<D, NW, CAUSAL>), dim3(qa.n_wgs), dim3(NW * 64), 0, s, qa);
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
