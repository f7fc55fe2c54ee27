// Device-side building blocks for the gfx950 attention kernels: vector types,
// the bf16 MFMA wrapper, LDS fragment readers and the workgroup -> tile maps.
//
// MFMA v_mfma_f32_32x32x16_bf16 register layout (checked on the device):
//   A (32 x 16): lane l holds row l%32, eight k values selected by l/32
//   B (16 x 32): lane l holds column l%32, the same eight k values
//   C (32 x 32): lane l, register r holds row (r/4)*8 + (l/32)*4 + r%4,
//                column l%32
// A C tile therefore gives each lane one column and 16 rows; the kernels keep
// that register -> row map as the k order when such a tile is reused as an
// operand (the k order only has to agree between A and B).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef __bf16 bf16;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4;
typedef __attribute__((__vector_size__(8 * sizeof(short)))) short s16x8;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

__device__ __forceinline__ bf16x8 zero_bf16x8() {
  bf16x8 z;
#pragma unroll
  for (int i = 0; i < 8; ++i) z[i] = (bf16)0.f;
  return z;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Wait for every outstanding vector-memory load (s_waitcnt vmcnt(0); expcnt and
// lgkmcnt left alone). Issued once after the register-resident operand loads so
// that no load is still pending on any path into a main loop; otherwise the
// compiler keeps a conservative vmcnt wait inside the loop that also drains
// the next tile's prefetch every iteration.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Max / sum of x over lanes l and l ^ 32 (v_permlane32_swap: no LDS round trip).
__device__ __forceinline__ float xhalf_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xhalf_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Row fragment from an LDS tile stored row-major with `stride` elements per row:
// lane l gets tile[row0 + l%32][col0 + (l/32)*8 .. +7] (one 16-byte read).
__device__ __forceinline__ bf16x8 frag_row(const bf16* tile, int stride, int row0, int col0, int lane) {
  return *reinterpret_cast<const bf16x8*>(tile + (row0 + (lane & 31)) * stride + col0 + ((lane >> 5) << 3));
}

// Transposed fragment: lane l gets tile[row0 + (e/4)*8 + (l/32)*4 + e%4][col0 + l%32]
// for e = 0..7, i.e. the k order of a C tile's registers. Two ds_read_b64_tr_b16:
// in each 16-lane group, lane t's value e comes from the 8-byte chunk addressed by
// lane 4e + t/4, element t%4; each lane therefore addresses row (l/32)*4 + (l%16)/4
// and columns ((l/16)%2)*16 + (l%4)*4 .. +3.
__device__ __forceinline__ bf16x8 frag_tr(const bf16* tile, int stride, int row0, int col0, int lane) {
  const int s = lane & 15;
  const int r = row0 + ((lane >> 5) << 2) + (s >> 2);
  const int c = col0 + (((lane >> 4) & 1) << 4) + ((s & 3) << 2);
  const bf16* p = tile + r * stride + c;
  s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
  s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + 8 * stride));
  s16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, v);
}

typedef float f32x2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));

// Eight consecutive C-tile registers (r0 .. r0+7) rounded (RNE) to a bf16
// operand: four v_cvt_pk_bf16_f32, one per register pair.
__device__ __forceinline__ bf16x8 pack8(const f32x16& c, int r0) {
  const bf16x2v p0 = __builtin_convertvector((f32x2v){c[r0 + 0], c[r0 + 1]}, bf16x2v);
  const bf16x2v p1 = __builtin_convertvector((f32x2v){c[r0 + 2], c[r0 + 3]}, bf16x2v);
  const bf16x2v p2 = __builtin_convertvector((f32x2v){c[r0 + 4], c[r0 + 5]}, bf16x2v);
  const bf16x2v p3 = __builtin_convertvector((f32x2v){c[r0 + 6], c[r0 + 7]}, bf16x2v);
  return (bf16x8){p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
}

// Offset of C-tile register r's row (or column) from the lane's base row
// (r/4)*8 + r%4; the lane's base adds (lane/32)*4.
__device__ __forceinline__ constexpr int creg_off(int r) { return ((r >> 2) << 3) + (r & 3); }

// Query-block tiles (forward, dQ): grid = nqb * B * Hq workgroups. Longest
// causal rows first (largest q block first). When the kv groups split evenly
// over the 8 XCDs (workgroups are dealt round-robin, bid % 8 picks the XCD), the
// query heads of one kv group stay on one XCD so their K/V reads share its L2.
__device__ __forceinline__ void decode_qblock(int bid, int nqb, int B, int Hq, int Hkv, int& qb, int& b, int& h) {
  const int G = Hq / Hkv;
  const int units = B * Hkv;
  if ((units & 7) == 0) {
    const int xcd = bid & 7, slot = bid >> 3;
    const int upx = units >> 3;
    const int per_qb = upx * G;
    const int qd = slot / per_qb, rem = slot - qd * per_qb;
    qb = nqb - 1 - qd;
    const int unit = xcd * upx + rem / G;
    b = unit / Hkv;
    h = (unit - b * Hkv) * G + rem % G;
  } else {
    const int per = B * Hq;
    const int qd = bid / per, rem = bid - qd * per;
    qb = nqb - 1 - qd;
    b = rem / Hq;
    h = rem - b * Hq;
  }
}

// Key-block tiles (dK/dV): grid = nkb * B * Hkv. A key block's work grows with
// the number of query rows below it, so blocks are dispatched longest first
// (key block 0 first). With `pair_ends`, the second half of the dispatch order
// walks the key blocks from the far end instead, so that when two workgroups
// share a CU from the start, a long block tends to pair with a short one. kv
// groups are pinned to XCDs as for query blocks.
__device__ __forceinline__ void decode_kblock(int bid, int nkb, int B, int Hkv, bool pair_ends, int& kb, int& b,
                                              int& hkv) {
  const int units = B * Hkv;
  int unit, ks;
  if ((units & 7) == 0) {
    const int xcd = bid & 7, slot = bid >> 3;
    const int upx = units >> 3;
    ks = slot / upx;
    unit = xcd * upx + (slot - ks * upx);
  } else {
    ks = bid / units;
    unit = bid - ks * units;
  }
  const int half = (nkb + 1) >> 1;
  kb = (!pair_ends || ks < half) ? ks : nkb - 1 - (ks - half);
  b = unit / Hkv;
  hkv = unit - b * Hkv;
}

__device__ __forceinline__ int valid_len(const int32_t* seqlens, int b, int S) {
  if (!seqlens) return S;
  int L = seqlens[b];
  return L < 0 ? 0 : (L > S ? S : L);
}

}  // namespace attn
