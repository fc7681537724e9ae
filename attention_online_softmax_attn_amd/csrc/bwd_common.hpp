// Backward of softmax attention on gfx950, shared definitions.  Gradients
// from the saved log-sum-exp.  With s = scale * Q K^T, P = exp(s - LSE), the gradient of O
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
// Two kernels, no atomics (every output element has one writer):
//   bwd_dq    workgroup = (b, query head, 32*NW queries), the forward's
//             layout: S^T = K Q^T and dP^T = V dO^T keep one query per lane;
//             dQ^T += K^T dS^T reads K transposed from LDS.  It first forms
//             each of its rows' record (LSE * log2 e, D_i = dO_i . O_i) from
//             the fragments it loads anyway, uses it, and stores it in the
//             workspace (one 8-byte record per row) for:
//   bwd_dkdv  workgroup = (b, kv head, 32*NW keys), launched after bwd_dq.
//             K and V fragments stay in registers; for every query head of
//             the group and every query tile that can see the keys, Q, dO and
//             the row records stream through a ring of LDS stages
//             (direct-to-LDS loads, the next tile prefetched while the
//             current one is computed).  S = Q K^T and dP = dO V^T put keys on
//             the MFMA N dimension, so P and dS come out with one key per lane
//             and feed dV += P^T dO and dK += dS^T Q straight from registers,
//             with dO and Q read transposed from LDS.
//
// The dK/dV kernel runs one wave per SIMD (its K, V fragments and dK, dV
// accumulators exceed half the register file), so its softmax-gradient VALU
// work is overlapped with MFMA work inside each wave: the 32-row blocks are
// software-pipelined two deep (S/dP of block i+1 and dV/dK of block i-1 run
// on the matrix core while the VALU turns S/dP of block i into P/dS), with
// the instruction order fixed slot by slot.  The dQ kernel fits two waves
// per SIMD, which overlap each other.
#pragma once

#include "device_common.hpp"
#include "kernels.h"

// Workgroups per CU the register allocation must allow (1: the kernel may use
// the whole register file, one wave per SIMD).
#ifndef ATTN_BWD_KV_OCC
#define ATTN_BWD_KV_OCC 1
#endif

// dK/dV pipeline: LDS reads are issued this many contraction slots ahead
#ifndef ATTN_BWD_LEAD
#define ATTN_BWD_LEAD 8
#endif
// dK/dV pipeline: row records are read this many slots before first use
#ifndef ATTN_BWD_REC_LEAD
#define ATTN_BWD_REC_LEAD 6
#endif

#ifndef ATTN_BWD_BQ
#define ATTN_BWD_BQ 64
#endif

// Pipeline depth of the dK/dV kernel: query tiles in flight (the tile being
// computed plus the prefetched ones).  Three stages (two tiles ahead) were
// measured no faster than two at B=4 H=16 N=2048.
#ifndef ATTN_BWD_STAGES
#define ATTN_BWD_STAGES 2
#endif

namespace attn {
namespace bwd {

struct BwdArgs {
  const __bf16* q;
  const __bf16* k;
  const __bf16* v;
  const __bf16* o;
  const __bf16* dout;
  const float* lse;
  float* dq;     // fp32 gradients, or bf16 ones (the same addresses as __bf16*) when grad_bf16
  float* dk;
  float* dv;
  float* stats;  // [B, Hq, nq_pad] x (LSE * log2 e, D)
  int B, Hq, Hkv, Nq, Nk, g;
  int nq_pad;    // record rows per head: Nq rounded up to 128, so that the
                 // 16-byte loads of records never straddle the end of a head
  int n_tiles, n_wgs;
  float c;      // scale * log2(e)
  float scale;
  int grad_bf16;  // 1: dq, dk, dv are bf16, each the fp32 result rounded to nearest even
};

// dQ for every query row; d is 64 or 128 (bwd_dq.hip)
hipError_t launch_dq(const BwdArgs& a, int d, bool causal, hipStream_t s);

}  // namespace bwd
}  // namespace attn

