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

// Eight consecutive C-tile registers (r0 .. r0+7) rounded to a bf16 operand.
__device__ __forceinline__ bf16x8 pack8(const f32x16& c, int r0) {
  bf16x8 v;
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = (bf16)c[r0 + e];
  return v;
}

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

// Key-block tiles (dK/dV): grid = nkb * B * Hkv. Longest first = the first key
// block (it sees every query row); kv groups pinned to XCDs as above.
__device__ __forceinline__ void decode_kblock(int bid, int B, int Hkv, int& kb, int& b, int& hkv) {
  const int units = B * Hkv;
  int unit;
  if ((units & 7) == 0) {
    const int xcd = bid & 7, slot = bid >> 3;
    const int upx = units >> 3;
    kb = slot / upx;
    unit = xcd * upx + (slot - kb * upx);
  } else {
    kb = bid / units;
    unit = bid - kb * units;
  }
  b = unit / Hkv;
  hkv = unit - b * Hkv;
}

__device__ __forceinline__ int valid_len(const int32_t* seqlens, int b, int S) {
  if (!seqlens) return S;
  int L = seqlens[b];
  return L < 0 ? 0 : (L > S ? S : L);
}

}  // namespace attn
