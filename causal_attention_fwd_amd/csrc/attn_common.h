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
// Index of the calling wave in its workgroup, in a scalar register: the
// compiler cannot tell that threadIdx.x / 64 is uniform, and a buffer resource
// derived from it would otherwise live in VGPRs, wrapping each buffer
// instruction in a readfirstlane loop.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

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

// LDS tile layout. Rows of D bf16 are cut into 16-byte chunks (CH = D/8 per
// row) and grouped by 8 rows into blocks of D*16 bytes plus 128 bytes of
// padding. Inside a block the chunks are stored chunk-major: chunk c of the
// block's row x (0..7) sits in 16-byte slot c*8 + (x ^ h(c)), h(c) = 4*((c/2)%2).
//  * Every 64 consecutive slots (1 KB) are 8 rows x 8 chunks, i.e. 8 row
//    segments of 128 contiguous bytes in global memory: one direct-to-LDS wave
//    load (lane i -> slot i) per KB, coalesced.
//  * Row fragments (16 consecutive rows, one chunk each, per 16 lanes): 8 rows
//    fill 128 contiguous bytes and the next 8 start one block later, which the
//    padding shifts by 128 bytes mod 256: all 64 banks once.
//  * Transposed fragments (4 rows x 2 chunks per 16 lanes; the next 16 lanes
//    two chunks further): the two halves use row slots 0-3 and 4-7 thanks to
//    h, so 32 lanes cover all 64 banks once.
//  * For row offsets that are multiples of 8 and column offsets that are
//    multiples of 16 an address is a lane term (one of two, picked by the
//    column offset) plus a constant, so the unrolled loops need few address
//    registers.
template <int D>
struct TileLayout {
  static constexpr int kBlockElems = D * 8 + 64;  // 8 rows + 128 bytes of padding
  template <int R>
  static constexpr int elems() {
    static_assert(R % 8 == 0, "tiles hold whole 8-row blocks");
    return R / 8 * kBlockElems;
  }
};

// Row fragment: lane l gets tile[row0 + l%32][col0 + (l/32)*8 .. +7] (one
// 16-byte read). row0 % 8 == 0, col0 % 16 == 0.
template <int D>
__device__ __forceinline__ bf16x8 frag_row(const bf16* tile, int row0, int col0, int lane) {
  constexpr int BE = TileLayout<D>::kBlockElems;
  const int h = ((col0 >> 4) & 1) << 2;
  const int c = (col0 >> 3) + (lane >> 5);
  const int off = ((row0 >> 3) + ((lane & 31) >> 3)) * BE + (c * 8 + ((lane & 7) ^ h)) * 8;
  return *reinterpret_cast<const bf16x8*>(tile + off);
}

// Transposed fragment: lane l gets tile[row0 + (e/4)*8 + (l/32)*4 + e%4][col0 + l%32]
// for e = 0..7, i.e. the k order of a C tile's registers. Two ds_read_b64_tr_b16:
// in each 16-lane group, lane t's value e comes from the 8-byte piece addressed
// by lane 4e + t/4, element t%4; each lane therefore addresses row
// (l/32)*4 + (l%16)/4 (and 8 more) and columns ((l/16)%2)*16 + (l%4)*4 .. +3.
// row0 % 8 == 0, col0 % 16 == 0.
template <int D>
__device__ __forceinline__ bf16x8 frag_tr(const bf16* tile, int row0, int col0, int lane) {
  constexpr int BE = TileLayout<D>::kBlockElems;
  const int s = lane & 15;
  const int b4 = (lane >> 4) & 1;
  const int c = (col0 >> 3) + 2 * b4 + ((s & 3) >> 1);   // chunk
  const int h = (((col0 >> 4) + b4) & 1) << 2;            // h(c): c/2 = col0/16 + b4
  const int x = (((lane >> 5) << 2) + (s >> 2)) ^ h;      // row within the block, swizzled
  // both addresses from the tile base: written as the first plus one block,
  // the second read lost track of its LDS array in the compiler, which then
  // waited for every in-flight tile copy before it
  const int lo_off = (c * 8 + x) * 8 + (s & 1) * 4;
  s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(tile + (row0 >> 3) * BE + lo_off));
  s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(tile + ((row0 >> 3) + 1) * BE + lo_off));
  s16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, v);
}

typedef __attribute__((address_space(3))) void lds_void;

// Direct global -> LDS load of rows [row0, row0 + R) of one (sequence, head)
// slice of a [B, S, H, D] tensor (row_stride elements between rows) into a
// tile of the layout above, with buffer_load_dwordx4 ... lds: each wave
// instruction fills one KB of slots, lane i landing in slot i, so lane i
// fetches the chunk the layout puts there. The buffer resource starts at row0
// and ends after the last row below L, so rows at or past L arrive as zeros
// (the hardware range check) and every offset stays below R * row_stride * 2
// bytes. No VGPRs hold the data; completion is tracked by vmcnt (wait_vmem)
// and made visible to the other waves by a barrier.
template <int R, int D, int NWAVES>
__device__ __forceinline__ void tile_load_lds(const bf16* base, int64_t row_stride, int row0, int L, bf16* tile,
                                              int wave, int lane) {
  constexpr int KB_PER_BLOCK = D / 64;           // 1 KB pieces per 8-row block
  constexpr int NKB = R / 8 * KB_PER_BLOCK;      // wave instructions per tile
  static_assert(NKB % NWAVES == 0, "tile must split evenly over the waves");
  // the descriptor is uniform; readfirstlane keeps it in SGPRs whatever
  // register class the compiler picked for its inputs (a descriptor in VGPRs
  // would wrap every load in a readfirstlane loop)
  const int rows = min(L - row0, R);
  const int bytes = __builtin_amdgcn_readfirstlane(rows > 0 ? ((rows - 1) * (int)row_stride + D) * 2 : 0);
  const uint64_t addr = reinterpret_cast<uint64_t>(base + (int64_t)row0 * row_stride);
  const uint64_t addr_u = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(addr >> 32)) << 32) |
                          (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)addr);
  const __amdgpu_buffer_rsrc_t rsrc =
      __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(addr_u), (short)0, bytes, 0x00020000);
#pragma unroll
  for (int j = 0; j < NKB / NWAVES; ++j) {
    const int kb = wave * (NKB / NWAVES) + j;
    const int blk = kb / KB_PER_BLOCK;
    const int c = (kb % KB_PER_BLOCK) * 8 + (lane >> 3);
    const int row = blk * 8 + ((lane & 7) ^ (((c >> 1) & 1) << 2));
    const int voff = (int)(row * row_stride + c * 8) * 2;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)(tile + blk * TileLayout<D>::kBlockElems +
                                                               (kb % KB_PER_BLOCK) * 512),
                                             16, voff, 0, 0, 0);
  }
}

// Two-stage pipeline over n tiles held in two LDS buffers (distinct arrays, so
// the compiler can tell the buffer being filled from the one being read and
// needs no vmcnt wait before the reads): the fetch of tile t+1 is in flight
// while tile t is computed. fetch(t, buf) issues the loads, land(t, buf) runs
// once they have arrived (for data staged through registers), compute(t, buf)
// reads the tile; the barrier after each compute publishes the next tile and
// frees the one just read.
// tile_pipeline_start issues the first tile's loads; a kernel calls it as
// soon as the tile can be addressed, so that they travel while it finishes its
// prologue, and then runs the rest with started = true.
template <class Buf, class Fetch>
__device__ __forceinline__ void tile_pipeline_start(int n, const Buf& b0, Fetch&& fetch) {
  if (n > 0) fetch(0, b0);
}
template <class Buf, class Fetch, class Land, class Compute>
__device__ __forceinline__ void tile_pipeline(int n, const Buf& b0, const Buf& b1, Fetch&& fetch, Land&& land,
                                              Compute&& compute, bool started = false) {
  if (!started && n > 0) fetch(0, b0);
  wait_vmem();
  if (n > 0) land(0, b0);
  __syncthreads();
  for (int t = 0; t < n; t += 2) {
    const bool more1 = t + 1 < n;
    if (more1) fetch(t + 1, b1);
    compute(t, b0);
    wait_vmem();
    if (more1) land(t + 1, b1);
    __syncthreads();
    if (!more1) break;
    const bool more2 = t + 2 < n;
    if (more2) fetch(t + 2, b0);
    compute(t + 1, b1);
    wait_vmem();
    if (more2) land(t + 2, b0);
    __syncthreads();
  }
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

// Key-block tiles (dK/dV): grid = B * Hkv units of nkb * parts workgroups;
// returns the workgroup's unit (b, hkv) and its slot within the unit (slots
// are dispatched in order, so a unit's first key blocks, the longest under the
// causal mask, go first). kv groups are pinned to XCDs as for query blocks.
__device__ __forceinline__ void decode_kunit(int bid, int B, int Hkv, int& slot, int& b, int& hkv) {
  const int units = B * Hkv;
  int unit;
  if ((units & 7) == 0) {
    const int xcd = bid & 7, xs = bid >> 3;
    const int upx = units >> 3;
    slot = xs / upx;
    unit = xcd * upx + (xs - slot * upx);
  } else {
    slot = bid / units;
    unit = bid - slot * units;
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
