// common.hpp -- device helpers shared by the gfx950 kernels of libsparse_attn.
//
// Lane layouts used throughout (wave64, verified on gfx950):
//   v_mfma_f32_32x32x16_bf16: A lane l holds A[l%32][8*(l/32)+s], s=0..7;
//       B lane l holds B[8*(l/32)+s][l%32]; C lane l holds
//       C[8*(j/4) + 4*(l/32) + j%4][l%32], j=0..15.
//   v_mfma_f32_16x16x32_bf16: A lane l holds A[l%16][8*(l/16)+s];
//       B[8*(l/16)+s][l%16]; C lane l holds C[4*(l/16)+j][l%16], j=0..3.
//   v_mfma_f32_16x16x16bf16_1k: A[l%16][4*(l/16)+s], B[4*(l/16)+s][l%16], s=0..3.
//   v_mfma_f32_32x32x2f32 / 16x16x4f32: one fp32 per lane, k index = l/32 or l/16.
//   ds_read_b64_tr_b16: inside each group of 16 lanes, lane t receives
//       element (t%4) of the 4-element chunk addressed by lane 4*j + t/4, j=0..3.
//       With lanes 4j..4j+3 pointing at row r_j, columns c0 + 4*(lane%4), lane t
//       gets [row r_j][c0 + t] for j = 0..3: a transposed fragment.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sa {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short short4v __attribute__((ext_vector_type(4)));
typedef short short8v __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) short4v lds_short4v;
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// 16-byte global load marked non-temporal: for data read exactly once (decode
// cache rows), so it does not displace reusable lines from L2 and the
// last-level cache.
__device__ __forceinline__ u32x4 load_once16(const void *p) {
  return __builtin_nontemporal_load((const u32x4 *)p);
}

// Running-max sentinel: finite, so exp2(sentinel - x) is 0 and sentinel - sentinel is 0.
constexpr float kNegBig = -1.0e30f;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float bf16_to_f32(unsigned short u) {
  return __uint_as_float(((unsigned int)u) << 16);
}

// fp32 -> bf16 with round-to-nearest-even (finite inputs; NaN stays NaN).
__device__ __forceinline__ unsigned short f32_to_bf16_bits(float f) {
  unsigned int u = __float_as_uint(f);
  if ((u & 0x7f800000u) == 0x7f800000u) return (unsigned short)((u >> 16) | ((u & 0xffffu) ? 0x40u : 0u));
  u += 0x7fffu + ((u >> 16) & 1u);
  return (unsigned short)(u >> 16);
}

// Four fp32 values rounded to bf16 (RNE, NaN stays NaN) by the hardware
// conversion v_cvt_pk_bf16_f32, packed as four consecutive bf16.  Checked bit
// for bit against f32_to_bf16_bits on gfx950 (ties, denormals, infinities).
__device__ __forceinline__ uint2 pack_bf16x4(float a, float b, float c, float d) {
  const bf16x2 lo = {(bf16)a, (bf16)b}, hi = {(bf16)c, (bf16)d};
  return make_uint2(__builtin_bit_cast(unsigned, lo), __builtin_bit_cast(unsigned, hi));
}

// Two transposed 4-element reads joined into one 8-element MFMA operand.  Whole
// vectors are reinterpreted (no per-element extraction).
__device__ __forceinline__ bf16x8 join_bf16x8(short4v lo, short4v hi) {
  const short8v v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ bf16x4 as_bf16x4(short4v x) { return __builtin_bit_cast(bf16x4, x); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

template <typename T>
__device__ __forceinline__ float to_f32(T x);
template <>
__device__ __forceinline__ float to_f32<float>(float x) { return x; }
template <>
__device__ __forceinline__ float to_f32<bf16>(bf16 x) {
  return bf16_to_f32(__builtin_bit_cast(unsigned short, x));
}

__device__ __forceinline__ float wave_shfl_xor(float v, int mask) {
  return __shfl_xor(v, mask, 64);
}

// XCD-aware remap of a 1-D grid: hardware hands consecutive workgroup ids to the
// 8 XCDs round-robin; this returns a logical id such that each XCD receives one
// contiguous range of logical ids (neighbouring tiles share its L2).
__device__ __forceinline__ int xcd_remap(int bid, int total) {
  const int per = total / 8, rem = total % 8;
  const int xcd = bid % 8, idx = bid / 8;
  return (xcd < rem) ? xcd * (per + 1) + idx : rem * (per + 1) + (xcd - rem) * per + idx;
}

// Key range [key_lo(i), key_hi(i)] of query i (mode numbers as in kernels.hpp):
//   0 pi-Attention window / 1 window:  [max(0, i-k), i]
//   2 ECP paired half-segments:        [max(0, (floor(i/s)-1)*s), i]
//   3 two-sided window:                [max(0, i-k), min(N-1, i+k)]
//   4 s-Split disjoint segments:       [floor(i/s)*s, i]
//   5 ECP pair without causal mask:    [max(0, (floor(i/s)-1)*s), min(N-1, (floor(i/s)+1)*s - 1)]
// Both ends are non-decreasing in i.
__device__ __forceinline__ int key_lo(int i, int mode, int k_win, int seg) {
  if (mode == 2 || mode == 5) {
    const int lo = (i / seg - 1) * seg;
    return lo > 0 ? lo : 0;
  }
  if (mode == 4) return (i / seg) * seg;
  const int lo = i - k_win;
  return lo > 0 ? lo : 0;
}

__device__ __forceinline__ int key_hi(int i, int N, int mode, int k_win, int seg) {
  long long hi = i;
  if (mode == 3) hi = (long long)i + k_win;
  else if (mode == 5) hi = ((long long)(i / seg) + 1) * seg - 1;
  return hi < N - 1 ? (int)hi : N - 1;
}

__device__ __forceinline__ float half_swap_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float half_swap_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// 16-byte row chunks from the 32x32 MFMA C layout.  There the wave half h
// (lane >> 5) holds elements 4h..4h+3 of every 8-element group of a row.  For
// two groups lo, hi (four bf16 each, as uint2), half_regroup returns in half 0
// the whole group lo and in half 1 the whole group hi (one v_permlane32_swap
// per dword: half 0's hi part and half 1's lo part change places).  It is its
// own inverse: half_ungroup takes a 16-byte chunk loaded that way back to the
// C layout.  Both halves of a lane pair must be active.
__device__ __forceinline__ uint4 half_regroup(uint2 lo, uint2 hi) {
  const auto a = __builtin_amdgcn_permlane32_swap(lo.x, hi.x, false, false);
  const auto b = __builtin_amdgcn_permlane32_swap(lo.y, hi.y, false, false);
  return make_uint4(a[0], b[0], a[1], b[1]);
}

__device__ __forceinline__ void half_ungroup(uint4 u, uint2 &lo, uint2 &hi) {
  const auto a = __builtin_amdgcn_permlane32_swap(u.x, u.z, false, false);
  const auto b = __builtin_amdgcn_permlane32_swap(u.y, u.w, false, false);
  lo = make_uint2(a[0], b[0]);
  hi = make_uint2(a[1], b[1]);
}

// The same for the 16x16 C layout, where lane row G (lane >> 4) holds elements
// 4G..4G+3 of each 16-element block: for blocks x (even) and y (odd) of one
// 32-element span, rows 0 and 1 exchange (x of row 1, y of row 0) and so do
// rows 2 and 3 (one v_permlane16_swap per dword).  Row G then holds the 8
// consecutive elements starting at 8 (G >> 1) + 16 (G & 1) of the span.
__device__ __forceinline__ uint4 row_regroup(uint2 x, uint2 y) {
  const auto a = __builtin_amdgcn_permlane16_swap(x.x, y.x, false, false);
  const auto b = __builtin_amdgcn_permlane16_swap(x.y, y.y, false, false);
  return make_uint4(a[0], b[0], a[1], b[1]);
}

// ---------------------------------------------------------------------------
// Row-major bf16 tiles (64 rows) go from HBM straight into LDS
// (global_load_lds_dwordx4: no staging registers), rows unpadded with the
// 16-byte chunks of row r permuted by chunk ^ swz(r).  swz makes both LDS read
// patterns conflict-free:
//  * MFMA row-fragment reads (16 lanes = 16 consecutive rows, one chunk each)
//    need swz to be a bijection on rows of equal bank offset;
//  * transposed reads (32 lanes = 4 consecutive rows x 4 chunks) need the
//    4 rows' 4-chunk groups to land on disjoint banks.
// d = 64 (128-byte rows, two rows per bank sweep): swz(r) = (r1 << 2) | r3r2;
// d = 128 (256-byte rows): swz(r) = (r1r0 << 2) | r3r2.
// ---------------------------------------------------------------------------
template <int D>
__device__ __forceinline__ int tile_swz(int r) {
  if constexpr (D == 64) return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
  else return ((r & 3) << 2) | ((r >> 2) & 3);
}

// One 16-byte direct-to-LDS load per lane: lane L's bytes land at
// lds_base + 16 * L.  Issued through inline asm so that the compiler does not
// wait for it before unrelated LDS reads; the caller waits (vmcnt) itself.
__device__ __forceinline__ void dma16(const void *gbase, unsigned voff, unsigned lds_base) {
  // m0 (the LDS destination) is an operand bound to that register, so the
  // compiler writes it and knows it changed; the s_nop covers the m0-write ->
  // LDS-DMA hazard, which the compiler cannot see inside the asm.
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(gbase), "{m0}"(lds_base)
               : "memory");
}

// 4 bytes per lane to LDS address lds_base + 4 * lane.
__device__ __forceinline__ void dma4(const void *gbase, unsigned voff, unsigned lds_base) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dword %0, %1"
               :
               : "v"(voff), "s"(gbase), "{m0}"(lds_base)
               : "memory");
}

__device__ __forceinline__ void wait_dma() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// ---------------------------------------------------------------------------
// Gate network on the query (pi-Attention section 2 item 3: a light per-token,
// per-head network produces the gate alpha).  Two layers with a ReLU hidden
// layer of width H <= 32:
//   z = sum_u w2[u] * relu(<w1[u], q> + b1[u]) + b2,   alpha = sigmoid(z).
// The hidden pre-activations are one more matrix product on the query
// fragments a kernel already holds as the B operand of its score MFMAs (the
// first-layer rows take the place of key rows).  The fp32 weights enter as
// two bf16 parts, w1 = hi + lo, so the product keeps ~16 significant bits of
// each weight; the query is bf16 already.
// ---------------------------------------------------------------------------
struct GateMlp {
  const float *w1, *b1, *w2, *b2;   // [H][D], [H], [H], [1] of one head
  int H;
};

// The network of head hg: first layer [H][D], biases [H], output weights [H], bias.
__device__ __forceinline__ GateMlp make_gate(const float *w1, const float *b1, const float *w2, const float *b2, int H,
                                             int hg, int D) {
  GateMlp g;
  g.H = H;
  g.w1 = w1 + (size_t)hg * H * D;
  g.b1 = b1 + (size_t)hg * H;
  g.w2 = w2 + (size_t)hg * H;
  g.b2 = b2 + hg;
  return g;
}

// w = hi + lo with hi, lo bf16: hi by the hardware conversion, lo the
// rounded residual (x - hi is exact in fp32), ~16 significant bits in all.
__device__ __forceinline__ void split_bf16x8(const f32x4 &a, const f32x4 &b, bf16x8 &hi, bf16x8 &lo) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float x = e < 4 ? a[e] : b[e - 4];
    hi[e] = (bf16)x;
    lo[e] = (bf16)(x - (float)hi[e]);
  }
}

// Sum over four hidden units u0..u0+3 of w2[u] relu(z[u] + b1[u]) (units >= H
// contribute nothing); one 16-byte load each for b1 and w2 when all four exist
// and both addresses are 16-byte aligned.
__device__ __forceinline__ float gate_out4(const GateMlp &g, int u0, float z0, float z1, float z2, float z3, float s) {
  if (u0 + 4 <= g.H && ((((uintptr_t)(g.b1 + u0)) | ((uintptr_t)(g.w2 + u0))) & 15) == 0) {
    const f32x4 b = *(const f32x4 *)(g.b1 + u0), w = *(const f32x4 *)(g.w2 + u0);
    s = fmaf(w[0], fmaxf(z0 + b[0], 0.f), s);
    s = fmaf(w[1], fmaxf(z1 + b[1], 0.f), s);
    s = fmaf(w[2], fmaxf(z2 + b[2], 0.f), s);
    return fmaf(w[3], fmaxf(z3 + b[3], 0.f), s);
  }
  const float zz[4] = {z0, z1, z2, z3};
#pragma unroll
  for (int e = 0; e < 4; ++e)
    if (u0 + e < g.H) s = fmaf(g.w2[u0 + e], fmaxf(zz[e] + g.b1[u0 + e], 0.f), s);
  return s;
}

// Lanes in the v_mfma_f32_32x32x16_bf16 layout of the prefill: lane (c, h)
// holds q[16 kk + 8 h .. +7] of query c in qf[kk].  The first layer's rows
// are prepared once (hidden unit c of lane (c, h), bf16 hi/lo parts) and
// reused for any number of 32-query blocks.
template <int D>
struct GateRows32 {
  bf16x8 hi[D / 16], lo[D / 16];
};

template <int D>
__device__ __forceinline__ GateRows32<D> gate_rows_32(const GateMlp &g, int lane) {
  const int u = lane & 31, h = lane >> 5;
  GateRows32<D> r;
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) {
    f32x4 a = f32x4{}, b = f32x4{};
    if (u < g.H) {
      const float *w = g.w1 + (size_t)u * D + 16 * kk + 8 * h;
      a = *(const f32x4 *)w;
      b = *(const f32x4 *)(w + 4);
    }
    split_bf16x8(a, b, r.hi[kk], r.lo[kk]);
  }
  return r;
}

// z for query c (the same in both lanes of the query).
template <int D>
__device__ __forceinline__ float gate_mlp_logit_32(const bf16x8 (&qf)[D / 16], const GateRows32<D> &r,
                                                   const GateMlp &g, int lane) {
  const int h = lane >> 5;
  f32x16 z = f32x16{};
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) {
    z = __builtin_amdgcn_mfma_f32_32x32x16_bf16(r.hi[kk], qf[kk], z, 0, 0, 0);
    z = __builtin_amdgcn_mfma_f32_32x32x16_bf16(r.lo[kk], qf[kk], z, 0, 0, 0);
  }
  // register j of lane (c, h): hidden unit 8 (j / 4) + 4 h + j % 4 of query c
  float s = 0.f;
#pragma unroll
  for (int a4 = 0; a4 < 4; ++a4) s = gate_out4(g, 8 * a4 + 4 * h, z[4 * a4], z[4 * a4 + 1], z[4 * a4 + 2], z[4 * a4 + 3], s);
  return half_swap_sum(s) + g.b2[0];
}

// fp32 prefill layout (v_mfma_f32_32x32x2f32): lane (c, h) holds q[2 kk + h].
template <int D>
__device__ __forceinline__ float gate_mlp_logit_32_f32(const float (&qf)[D / 2], const GateMlp &g, int lane) {
  const int u = lane & 31, h = lane >> 5;
  f32x16 z = f32x16{};
#pragma unroll
  for (int kk = 0; kk < D / 2; ++kk) {
    const float a = u < g.H ? g.w1[(size_t)u * D + 2 * kk + h] : 0.f;
    z = __builtin_amdgcn_mfma_f32_32x32x2f32(a, qf[kk], z, 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int a4 = 0; a4 < 4; ++a4) s = gate_out4(g, 8 * a4 + 4 * h, z[4 * a4], z[4 * a4 + 1], z[4 * a4 + 2], z[4 * a4 + 3], s);
  return half_swap_sum(s) + g.b2[0];
}

// Lanes in the v_mfma_f32_16x16x32_bf16 layout of the skip pass and the
// decode: lane (G, t) = (lane / 16, lane % 16) holds q[32 kk + 8 G .. +7] of
// query column t in qf[kk].  Applies ONE head's network to every column and
// returns z of column t (the same in its four lane groups): the product pairs
// every first-layer row with every column, so a caller whose columns belong
// to different heads calls it once per head and keeps that head's columns.
template <int D>
__device__ __forceinline__ float gate_mlp_logit_16(const bf16x8 (&qf)[D / 32], const GateMlp &g, int lane) {
  const int G = lane >> 4, t = lane & 15;
  float s = 0.f;
#pragma unroll
  for (int blk = 0; blk < 2; ++blk) {
    if (blk == 1 && g.H <= 16) break;
    // A operand: hidden unit 16 blk + t (this lane's row), dims 32 kk + 8 G .. +7
    f32x4 z = f32x4{};
    const int u = 16 * blk + t;
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk) {
      f32x4 a = f32x4{}, b = f32x4{};
      if (u < g.H) {
        const float *w = g.w1 + (size_t)u * D + 32 * kk + 8 * G;
        a = *(const f32x4 *)w;
        b = *(const f32x4 *)(w + 4);
      }
      bf16x8 hi, lo;
      split_bf16x8(a, b, hi, lo);
      z = __builtin_amdgcn_mfma_f32_16x16x32_bf16(hi, qf[kk], z, 0, 0, 0);
      z = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lo, qf[kk], z, 0, 0, 0);
    }
    // register j of lane (G, t): hidden unit 16 blk + 4 G + j of column t
    s = gate_out4(g, 16 * blk + 4 * G, z[0], z[1], z[2], z[3], s);
  }
  s += wave_shfl_xor(s, 16);
  s += wave_shfl_xor(s, 32);
  return s + g.b2[0];
}

}  // namespace sa
