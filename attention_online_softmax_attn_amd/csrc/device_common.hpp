// Device primitives for gfx950 (MI355X): MFMA fragments, LDS tile layout,
// buffer loads (global and direct-to-LDS), wave64 cross-half reductions.
//
// Lane layouts used throughout (wave64, lane = 0..63, half h = lane / 32):
//   v_mfma_f32_32x32x16_bf16  A[m][k]: lane holds row m = lane%32, k = 8h..8h+7
//                             B[k][n]: lane holds col n = lane%32, k = 8h..8h+7
//                             C[m][n]: lane holds col n = lane%32, 16 rows
//                                      m = 8(r/4) + 4h + r%4, r = 0..15
//   v_mfma_f32_32x32x2_f32    A: row lane%32, k = h;  B: col lane%32, k = h;  C as above
//   ds_read_b64_tr_b16        within each 16-lane group, lane t receives
//                             element t%4 of the 8-byte words addressed by the
//                             group's lanes 4e + t/4, e = 0..3.  With provider
//                             lane t pointing at row r0 + t/4, column c0 + 4(t%4)
//                             of a row-major bf16 tile, lane t receives rows
//                             r0..r0+3 of column c0 + t: a transposed read.
//   v_permlane32_swap         exchanges the upper half of its first operand
//                             with the lower half of its second, so with both
//                             operands equal lane l receives lane l^32's value
//                             in the second result (l < 32) or the first (l >= 32).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4;
typedef __attribute__((__vector_size__(4 * sizeof(int)))) int i32x4;
typedef __attribute__((__vector_size__(2 * sizeof(int)))) int i32x2;
typedef __attribute__((address_space(3))) void lds_void;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();

// Buffer resource over [base, base + bytes); loads past the end return zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ i32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}

// 16 bytes from global byte offset `off` into LDS at lds_base + 16 * lane.
// lds_base must be wave-uniform.
__device__ __forceinline__ void buf_load_lds16(__amdgpu_buffer_rsrc_t r, uint32_t off, lds_void* lds_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds_base, 16, off, 0, 0, 0);
}
// The same with the non-temporal cache policy (the `nt` bit), for data that
// one launch reads exactly once: the split-KV decode's K/V stream measured
// 11 % faster with it at 48 x 4096 and 48 x 2048 (124 vs 139 us, 63 vs 71 us)
// and 6 % at 16 x 4096.  Data that other workgroups read again (the
// forward's and backward's K/V, Q and dO tiles) keeps the default policy.
__device__ __forceinline__ void buf_load_lds16_stream(__amdgpu_buffer_rsrc_t r, uint32_t off, lds_void* lds_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds_base, 16, off, 0, 0, 2);
}

// Wait until this wave's outstanding vector-memory loads (including direct-to-LDS
// loads) have completed; expcnt and lgkmcnt are left unconstrained.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }
// Workgroup barrier without the release/acquire fences of __syncthreads()
// (the release fence waits for every outstanding load, including prefetches
// of later tiles).  The caller must already have waited (wait_vmem /
// wait_vmem_n) for the direct-to-LDS loads whose data the barrier publishes.
// The empty asm statements keep the compiler from moving memory accesses
// across the barrier.
__device__ __forceinline__ void barrier_nofence() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Wait until at most N of this wave's vector-memory loads are outstanding
// (loads complete in issue order for this count); N < 64.
template <int N>
__device__ __forceinline__ void wait_vmem_n() {
  static_assert(N >= 0 && N < 64, "vmcnt is a 6-bit field");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32_f32(float a, float b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ s16x4 ds_read_tr16(const char* lds_byte_ptr) {
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_s16x4*)(__attribute__((address_space(3))) char*)(lds_byte_ptr));
}

// Transposed 8-bit LDS read.  Within each group of 16 lanes, lane t receives
// byte (t % 8) of the 8-byte words addressed by lanes 2b + t / 8 of the group,
// b = 0 .. 7, as its bytes b (measured on gfx950).
__device__ __forceinline__ i32x2 ds_read_tr8(const char* lds_byte_ptr) {
  typedef __attribute__((address_space(3))) i32x2 lds_i32x2;
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2*)(__attribute__((address_space(3))) char*)(lds_byte_ptr));
}

// Eight OCP FP8 E4M3 values (bytes 0..7 of w) -> bf16, exactly (every E4M3
// value is a bf16 value; gfx950's conversion decodes the OCP format, measured
// on all 256 codes).
__device__ __forceinline__ bf16x8 fp8x8_to_bf16(i32x2 w) {
  typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
  const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[0], 1.0f, false);
  const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[0], 1.0f, true);
  const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[1], 1.0f, false);
  const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[1], 1.0f, true);
  return bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

__device__ __forceinline__ bf16x8 join_bf16(s16x4 lo, s16x4 hi) {
  typedef __attribute__((__vector_size__(8 * sizeof(short)))) short s16x8;
  s16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, v);
}

// x from lane l ^ 32.  After the swap the first result holds the partner's
// value in the upper half and the second holds it in the lower half; the
// select keeps both results live (folding them into one is wrong).
__device__ __forceinline__ float partner32(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  const bool lower = (threadIdx.x & 32) == 0;
  return __builtin_bit_cast(float, lower ? r[1] : r[0]);
}
// max / sum of x over lanes l and l ^ 32
__device__ __forceinline__ float halves_max(float x) { return fmaxf(x, partner32(x)); }
__device__ __forceinline__ float halves_sum(float x) { return x + partner32(x); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Index of this wave in its workgroup, as a wave-uniform (scalar) value, so
// that index arithmetic and branches derived from it stay on the scalar unit.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }


// fp32 -> bf16, round to nearest even (inputs here are finite or +-0).
__device__ __forceinline__ __bf16 to_bf16(float x) { return (__bf16)x; }

// 16-byte chunk swizzle of a row-major bf16 tile with rows of D elements.
// Logical chunk c of row r is stored at chunk c ^ swz(r).  For D = 128 the
// XOR spreads 16 consecutive rows over all 16 chunk positions (b128 reads of
// one column chunk) and sends rows r..r+3 of an aligned 4-chunk group to 4
// different groups (transposed b64 reads); D = 64 does the same over 8 chunks
// and row pairs.
template <int D>
__device__ __forceinline__ int swz(int r) {
  if constexpr (D == 128) {
    return ((r & 3) << 2) | ((r >> 2) & 3);
  } else {
    return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
  }
}

// Byte offset of element (r, c) in a swizzled [rows][D] bf16 tile.
template <int D>
__device__ __forceinline__ int tile_off(int r, int c) {
  return r * (D * 2) + ((((c >> 3) ^ swz<D>(r))) << 4) + ((c & 7) << 1);
}

// Map a launch index to a logical work index so that the workgroups the
// dispatcher sends to one XCD (launch index mod 8) get a contiguous range of
// logical indices.  A bijection on [0, n).
__device__ __forceinline__ int xcd_remap(int pid, int n) {
  constexpr int kXcd = 8;
  int q = n / kXcd, rem = n % kXcd;
  int x = pid % kXcd, t = pid / kXcd;
  int start = x < rem ? x * (q + 1) : rem * (q + 1) + (x - rem) * q;
  return start + t;
}

__device__ __forceinline__ int wave_sum(int x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return __builtin_amdgcn_readfirstlane(x);
}

__device__ __forceinline__ int wave_incl_scan(int x, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  return x;
}

// Longest-first placement of work items of unequal size, computed by every
// wave from per-sequence sizes on the device (no workspace, no host round
// trip).  Sequence s has size(s) (one or two numbers) and count(size, w)
// items of weight at least w: a count that does not increase with w, is the
// sequence's whole item count at w = 0 and 0 at w = w_end.  Ranks go to the
// items heaviest first, ties in sequence order, each item taking n_heads
// consecutive ranks; the weight of rank r is found by a binary search on w
// over the summed counts.  Rank `rank` is placed on sequence s_out (whose
// size comes back in size_out) as the k_out-th, in the sequence's own order,
// of its items of weight exactly w, where c_lo = count(size, w) and c_lo1 =
// count(size, w + 1), and on head slot j_out.  The sizes of the first
// kCached * 64 sequences stay in registers.  Returns false for a rank past
// the last item.
template <int kCached, class Size, class Count>
__device__ bool lpt_place(int n_seqs, int n_heads, int rank, int w_end, Size size, Count count, int& s_out,
                          int2& size_out, int& c_lo, int& c_lo1, int& k_out, int& j_out) {
  const int lane = threadIdx.x & 63;
  int2 sz_c[kCached];
#pragma unroll
  for (int c = 0; c < kCached; c++) {
    sz_c[c] = make_int2(0, 0);
    const int s = c * 64 + lane;
    if (s < n_seqs) sz_c[c] = size(s);
  }
  auto get = [&](int c) -> int2 {
    if (c < kCached) {
      // constant-indexed copies, so that the array stays in registers
      int2 v = sz_c[0];
#pragma unroll
      for (int i = 1; i < kCached; i++)
        if (c == i) v = sz_c[i];
      return v;
    }
    return c * 64 + lane < n_seqs ? size(c * 64 + lane) : make_int2(0, 0);
  };
  const int chunks = (n_seqs + 63) / 64;
  auto total = [&](int w) -> int {
    int c_sum = 0;
    for (int c = 0; c < chunks; c++) c_sum += count(get(c), w);
    return wave_sum(c_sum);
  };
  if (rank >= total(0) * n_heads) return false;
  // the largest w whose items (times heads) outnumber rank
  int lo = 0, hi = w_end;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (total(mid) * n_heads > rank) lo = mid;
    else hi = mid;
  }
  const int r2 = rank - total(lo + 1) * n_heads;  // index among the items of weight exactly lo
  const int u = r2 / n_heads;
  j_out = r2 % n_heads;
  int before = 0;
  for (int c = 0; c < chunks; c++) {
    const int2 sz = get(c);
    const int cw = count(sz, lo), cw1 = count(sz, lo + 1);
    const int e = cw - cw1;
    const int incl = wave_incl_scan(e, lane);
    const int excl = incl - e;
    const bool hit = e > 0 && before + excl <= u && u < before + incl;
    const uint64_t m = __builtin_amdgcn_ballot_w64(hit);
    if (m != 0) {
      const int src = (int)__builtin_ctzll(m);
      s_out = c * 64 + src;
      size_out = make_int2(__builtin_amdgcn_readlane(sz.x, src), __builtin_amdgcn_readlane(sz.y, src));
      c_lo = __builtin_amdgcn_readlane(cw, src);
      c_lo1 = __builtin_amdgcn_readlane(cw1, src);
      k_out = u - before - __builtin_amdgcn_readlane(excl, src);
      return true;
    }
    before += __builtin_amdgcn_readlane(incl, 63);
  }
  return false;  // not reached: the counts above place every rank
}

// Launch index -> (pair, sub) for a grid of n_pairs * per_pair workgroups
// whose sub 0 is the heaviest item of a pair and later subs are lighter.  The
// dispatcher sends workgroup pid to XCD pid % 8 and starts the workgroups of
// one XCD in order of pid / 8.  When the pairs split evenly over the XCDs,
// XCD x takes pairs [x P/8, (x+1) P/8) (the workgroups of a pair share their
// K/V or Q/dO reads in that XCD's L2) and starts them heaviest sub first
// across all its pairs; otherwise the whole grid goes heaviest sub first.
// Heaviest-first keeps long workgroups from starting last and running alone
// at the end of a launch.  A bijection on [0, n_pairs * per_pair).
struct WorkItem {
  int pair, sub;
};
__device__ __forceinline__ WorkItem lpt_order(int pid, int n_pairs, int per_pair) {
  constexpr int kXcd = 8;
  if (n_pairs % kXcd == 0) {
    const int ppx = n_pairs / kXcd;
    const int x = pid % kXcd, t = pid / kXcd;
    return {x * ppx + t % ppx, t / ppx};
  }
  return {pid % n_pairs, pid / n_pairs};
}

}  // namespace attn
