// gfx950 kernels for fused causal (or bidirectional) attention: forward,
// backward preprocess, backward dK/dV and backward dQ (optionally computing the
// preprocess's D itself), the rotary-embedding pre-pass, and decode attention
// against a key/value cache (split over waves, then merged). Every kernel
// addresses tensor rows through (sequence, position, head) strides.
//
// The method ("Axis", Zyora Labs page, feature list): flash attention forward
// and backward on matrix cores in which the attention probabilities never reach
// device memory; bf16 storage, fp32 accumulation. Grouped kv heads follow the
// "AxiomLM" page ("Key Features": grouped-query attention). The formulas are in
// include/attn.h.
//
// Design (CDNA4-specific, not taken from the pages' CUDA/WMMA kernels):
//  * every product runs on v_mfma_f32_32x32x16_bf16 with fp32 accumulators;
//  * the forward and dQ passes compute S^T = K Q^T so that each lane owns one
//    query row: row max/sum need a single cross-lane step (lane l <-> l+32), the
//    row statistics (m, l, LSE, D) are per-lane scalars, and P^T / dS^T already
//    sit in the B-operand layout of the next product (O^T = V^T P^T,
//    dQ^T = K^T dS^T) without any shuffle;
//  * the dK/dV pass computes S = Q K^T so that each lane owns one key column and
//    P / dS feed dV^T = dO^T P and dK^T = Q^T dS as B operands directly;
//  * the transposed A operands (V^T, K^T, dO^T, Q^T) come from row-major LDS tiles
//    through the gfx950 transposing LDS read (ds_read_b64_tr_b16);
//  * K/V (or Q/dO) tiles stream from global memory straight into LDS
//    (buffer_load ... lds), double-buffered, one barrier per tile;
//  * tiles entirely above the causal diagonal or past a sequence's valid length
//    are never loaded or computed; the mask is applied only on tiles that need it
//    (bidirectional attention, causal = 0, skips and masks only the padding);
//  * the softmax runs in base 2 with scale*log2(e) folded into one multiply;
//    LSE is exported as a natural log.
#include <algorithm>
#include <cmath>
#include <mutex>

#include "attn_common.h"
#include "attn_launch.h"

namespace attn {

struct FwdArgs {
  const bf16* q;
  const bf16* k;
  const bf16* v;
  bf16* o;
  float* lse;
  const int32_t* seqlens;
  int B, S, Hq, Hkv, nqb;
  float scale;
  int causal;  // 1: keys j <= i only; 0: every key of the valid prefix
  Strides sq, skv, so;  // Q; K and V; O (elements per sequence, position, head)
};

struct PreArgs {
  const bf16* o;
  const bf16* d_o;
  float* delta;
  const int32_t* seqlens;
  int B, S, Hq;
  int64_t rows;  // B * Hq * S
  Strides so;    // O and dO
};

// Rotary position embedding ("AxiomLM" PyPI page, "Key Features" and "8.
// Standalone Modern Architectural Modules"): pair (2i, 2i+1) of a query or key
// at position p is rotated by the angle p * theta_i, theta_i = base^(-2i/d).
// phi_i = theta_i / (2 pi) (revolutions per position) comes from the host in
// fp64, so the angle is reduced to [0, 1) revolutions exactly enough for any
// position before the hardware sine and cosine (which take revolutions).
struct RopeFreq {
  double phi[64];  // i < d/2
};

__device__ __forceinline__ void rope_cos_sin(double phi, int p, float& cs, float& sn) {
  const double x = (double)p * phi;
  const float rev = (float)(x - __builtin_floor(x));
  cs = __builtin_amdgcn_cosf(rev);
  sn = __builtin_amdgcn_sinf(rev);
}

// The adjoint rotation (by -p*theta) of four consecutive elements of one row,
// d = d0 + 4g .. d0 + 4g + 3 (d0 a multiple of 8, the same for every lane;
// g = 0 or 1 per lane): pairs (d, d+1) and (d+2, d+3).
__device__ __forceinline__ void rope_adjoint4(const RopeFreq& rf, int d0, int g, int p, float (&x)[4]) {
#pragma unroll
  for (int pr = 0; pr < 2; ++pr) {
    float cs, sn;
    const double phi = g ? rf.phi[d0 / 2 + 2 + pr] : rf.phi[d0 / 2 + pr];
    rope_cos_sin(phi, p, cs, sn);
    const float x0 = x[2 * pr], x1 = x[2 * pr + 1];
    x[2 * pr] = x0 * cs + x1 * sn;
    x[2 * pr + 1] = x1 * cs - x0 * sn;
  }
}

struct BwdArgs {
  const bf16* q;
  const bf16* k;
  const bf16* v;
  const bf16* d_o;
  const float* lse;
  const float* delta;
  bf16* dq;
  bf16* dk;
  bf16* dv;
  const int32_t* seqlens;
  int B, S, Hq, Hkv, nblk;
  float scale;
  int causal;  // 1: keys j <= i only; 0: every key of the valid prefix
  int rope;    // 1: q and k are rotated; dQ and dK leave through the adjoint
  RopeFreq rf;
  Strides sq, skv, so;  // Q; K, V, dK, dV; O, dO, dQ
  // dQ pass only: when o is set, D = rowsum(dO * O) is computed from O and
  // the dO rows the pass loads anyway, used, and written to delta_out (the
  // preprocess folded in); delta is then not read
  const bf16* o;
  float* delta_out;
  // dK/dV pass only: with parts > 1 the (head, query tile) iterations of each
  // key block are split into `parts` contiguous ranges, one workgroup each,
  // whose unscaled fp32 dK and dV partial sums go to part_dk / part_dv
  // ([part, B, S, Hkv, d], dense) for dkdv_reduce_kernel to add up
  int parts;
  float* part_dk;
  float* part_dv;
};

constexpr int kThreads = 256;  // four waves, one per SIMD

// LDS fragment read-ahead, in product steps: scheduling groups put the reads
// of step i + PF beside the products of step i, so that a product does not
// wait for a read issued just before it. 0 leaves the order to the compiler:
// the d=64 dQ pass (three waves per SIMD) has no registers to spare for it,
// and the d=64 forward measured the same either way.
constexpr int kDkdvReadAhead = 4;
template <int D>
constexpr int kDqReadAhead = D == 128 ? 2 : 0;
template <int D>
constexpr int kFwdReadAhead = D == 128 ? 2 : 0;
// instruction classes of __builtin_amdgcn_sched_group_barrier
constexpr int kSchedMfma = 0x008, kSchedDsRead = 0x100;

// Wave priority 1 while a wave issues its first run of MFMAs, so that the pipe
// is refilled promptly while a sibling wave on the same SIMD runs VALU work;
// back to 0 afterwards.
__device__ __forceinline__ void prio_mfma() { __builtin_amdgcn_s_setprio(1); }
__device__ __forceinline__ void prio_base() { __builtin_amdgcn_s_setprio(0); }

// One stage of a K/V (or Q/dO) tile pipeline: two swizzled LDS tiles, and the
// stage's index for side data kept in indexed arrays.
struct KVBuf {
  bf16* k;
  bf16* v;
  int idx;
};

// ----------------------------------------------------------------------------
// Forward. One workgroup of W waves = one (sequence, query head, block of
// 32*NT*W query rows); wave w owns rows [q0 + 32*NT*w, +32*NT). Loop over 64-row
// K/V tiles up to the block's last row. OCC waves per SIMD (register budget
// 512/OCC).
//
// Online softmax with a lazily refreshed reference: each row keeps the maximum
// it last rescaled to (mu). A tile's exponents use mu unless the row maximum
// has grown by more than 2^8 (in base-2 units), in which case the accumulator
// and running sum are rescaled to the new maximum. Exponents therefore stay
// <= 2^8, well inside fp32 and bf16 range, and the rescale almost never runs
// once the first tile has set mu. O = acc / l and LSE = mu*scale + ln l use the
// same mu, so the result is exact whatever mu is.
// ----------------------------------------------------------------------------
template <int D, int NT>
struct FwdState {
  bf16x8 qf[NT][D / 16];
  f32x16 oacc[D / 32][NT];
  float mu[NT], lsum[NT];
};

// One 64-key tile for one wave. MASK: keys past min(row, L-1) are excluded;
// lim[t] = min(i, L-1) - j0 - (lane/32)*4 for the lane's row i of n-tile t
// (causal), L-1 - j0 - (lane/32)*4 (bidirectional).
template <int D, int NT, bool MASK>
__device__ __forceinline__ void fwd_tile(FwdState<D, NT>& st, const bf16* Ks, const bf16* Vs, int lane, float c,
                                         const int (&lim)[NT]) {
  constexpr int KK = D / 16, DT = D / 32;
  constexpr float kHeadroom = 8.f;  // log2 of the largest exponent allowed before a rescale
  f32x16 s[2][NT];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int t = 0; t < NT; ++t) s[mt][t] = zero16();
  constexpr int NS = 2 * KK;  // step i = (kk, mt) = (i / 2, i % 2)
  bf16x8 kf[NS];
#pragma unroll
  for (int i = 0; i < NS; ++i) kf[i] = frag_row<D>(Ks, (i & 1) * 32, (i >> 1) * 16, lane);
#pragma unroll
  for (int i = 0; i < NS; ++i)
#pragma unroll
    for (int t = 0; t < NT; ++t) s[i & 1][t] = mfma32(kf[i], st.qf[t][i >> 1], s[i & 1][t]);
  if constexpr (kFwdReadAhead<D> > 0) {
    constexpr int PF = kFwdReadAhead<D>;
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, PF, 0);
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, NT, 0);
      if (i + PF < NS) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
    }
  }
  if (MASK) {
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (mt * 32 + creg_off(r) > lim[t]) s[mt][t][r] = kNegInf;
  }
  float alpha[NT];
  bool rescale = false;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    float mx = kNegInf;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[mt][t][r]);
    mx = xhalf_max(mx);
    // (mx - mu) * c is NaN (no refresh) when both are -inf
    const bool refresh = (mx - st.mu[t]) * c > kHeadroom;
    alpha[t] = refresh ? fast_exp2((st.mu[t] - mx) * c) : 1.f;
    rescale |= refresh;
    st.mu[t] = refresh ? mx : st.mu[t];
    const float mc = st.mu[t] == kNegInf ? 0.f : st.mu[t] * c;
    float ls = 0.f;  // fp32 sum of the unrounded probabilities (LSE needs it)
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = fast_exp2(__builtin_fmaf(s[mt][t][r], c, -mc));
        s[mt][t][r] = p;
        ls += p;
      }
    st.lsum[t] = st.lsum[t] * alpha[t] + ls;
  }
  if (__ballot(rescale)) {
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) st.oacc[dt][t][r] *= alpha[t];
  }
  bf16x8 pb[4][NT];
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int t = 0; t < NT; ++t) pb[u][t] = pack8(s[u >> 1][t], (u & 1) * 8);
  constexpr int NT2 = 4 * DT;  // step i = (dt, u) = (i / 4, i % 4)
  bf16x8 vf[NT2];
#pragma unroll
  for (int i = 0; i < NT2; ++i) vf[i] = frag_tr<D>(Vs, (i & 3) * 16, (i >> 2) * 32, lane);
#pragma unroll
  for (int i = 0; i < NT2; ++i)
#pragma unroll
    for (int t = 0; t < NT; ++t) st.oacc[i >> 2][t] = mfma32(vf[i], pb[i & 3][t], st.oacc[i >> 2][t]);
  if constexpr (kFwdReadAhead<D> > 0) {
    constexpr int PF = kFwdReadAhead<D>;
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2 * PF, 1);
#pragma unroll
    for (int i = 0; i < NT2; ++i) {
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, NT, 1);
      if (i + PF < NT2) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 1);
    }
  }
}

// Merge slot for the state of key group k (1 .. KS-1) of row wave `wave` in a
// key-split workgroup: NREG floats per lane, [register][lane], packed into the
// four tile arrays, which are free after the pipeline's last barrier.
template <int NREG, int KVT>
__device__ __forceinline__ float* merge_slot(bf16* a0, bf16* a1, bf16* a2, bf16* a3, int k, int wave, int WR,
                                             int lane) {
  constexpr int PER = (KVT / 2) / (NREG * 64);  // slots per array (KVT bf16 = KVT / 2 floats)
  static_assert(PER >= 1, "merge slot");
  const int wi = (k - 1) * WR + wave;
  bf16* arr = wi / PER == 0 ? a0 : wi / PER == 1 ? a1 : wi / PER == 2 ? a2 : a3;
  return reinterpret_cast<float*>(arr) + (wi % PER) * NREG * 64 + lane;
}

// KS = 2 (small grids): the workgroup's waves form two halves over the same
// query rows; each pipeline step brings two 64-key tiles, the first half of
// the waves takes the even tiles, the second half the odd ones, and at the
// end the second half hands its softmax state (reference maximum, partial
// row sums, unnormalised O) through LDS to the first, which merges the two
// by log-sum-exp. Half as many steps per block, twice the waves.
template <int D, int NT, int OCC, int W, int KS = 1>
__global__ __launch_bounds__(64 * W) __attribute__((amdgpu_waves_per_eu(OCC, OCC)))
void fwd_kernel(FwdArgs a) {
  constexpr int BN = 64;
  constexpr int WR = W / KS;  // waves per key half (each owns 32*NT query rows)
  constexpr int BM = WR * 32 * NT;
  constexpr int KK = D / 16;
  constexpr int DT = D / 32;
  constexpr int KVT = TileLayout<D>::template elems<KS * BN>();
  static_assert(KS == 1 || KS == 2 || KS == 4, "key split");
  __shared__ __attribute__((aligned(16))) bf16 sK0[KVT], sV0[KVT], sK1[KVT], sV1[KVT];

  const int lane = threadIdx.x & 63;
  const int wave_all = threadIdx.x >> 6;
  const int wave = wave_all % WR;   // row wave
  const int kh = wave_all / WR;     // key half
  const int g = lane >> 5;
  const int l32 = lane & 31;

  int qb, b, h;
  decode_qblock(blockIdx.x, a.nqb, a.B, a.Hq, a.Hkv, qb, b, h);
  const int S = a.S;
  const int L = valid_len(a.seqlens, b, S);
  const int hkv = h / (a.Hq / a.Hkv);
  const int64_t qs = a.sq.s;   // elements between consecutive positions
  const int64_t ks = a.skv.s;
  const int64_t os = a.so.s;
  const bf16* Qb = a.q + b * a.sq.b + h * a.sq.h;
  const bf16* Kb = a.k + b * a.skv.b + hkv * a.skv.h;
  const bf16* Vb = a.v + b * a.skv.b + hkv * a.skv.h;
  bf16* Ob = a.o + b * a.so.b + h * a.so.h;
  float* LSEb = a.lse + ((int64_t)b * a.Hq + h) * S;

  const int q0 = qb * BM;
  const int qw = q0 + wave * 32 * NT;
  // causal: key tiles up to the block's last row; bidirectional: all of them
  const int kend = a.causal ? min(q0 + BM, L) : L;
  const int ntiles = (q0 < L) ? (kend - 1) / (KS * BN) + 1 : 0;  // pipeline steps of KS tiles
  const int wave_last = min(qw + 32 * NT, L) - 1;  // < qw when the wave is all padding
  const int key_last = a.causal ? wave_last : (wave_last < qw ? -1 : L - 1);  // last key a row of the wave sees
  const float c = a.scale * kLog2e;

  FwdState<D, NT> st;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int row = qw + t * 32 + l32;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
      st.qf[t][kk] = row < L ? *reinterpret_cast<const bf16x8*>(Qb + (int64_t)row * qs + kk * 16 + g * 8)
                             : zero_bf16x8();
    st.mu[t] = kNegInf;
    st.lsum[t] = 0.f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) st.oacc[dt][t] = zero16();
  }
  // (no wait here: the pipeline's first wait covers these loads and the
  // first K/V tile, which is issued before it, so the two latencies overlap)

  const KVBuf b0{sK0, sV0, 0}, b1{sK1, sV1, 1};
  auto fetch = [&](int kt, const KVBuf& buf) {
    tile_load_lds<KS * BN, D, W>(Kb, ks, kt * KS * BN, L, buf.k, wave_all, lane);
    tile_load_lds<KS * BN, D, W>(Vb, ks, kt * KS * BN, L, buf.v, wave_all, lane);
  };
  auto compute = [&](int kt, const KVBuf& buf) {
    const int j0 = (kt * KS + kh) * BN;
    if (j0 > key_last) return;
    // this half's 64-key tile: rows kh*64.. of the step's tile
    const bf16* Ks = buf.k + kh * TileLayout<D>::template elems<BN>();
    const bf16* Vs = buf.v + kh * TileLayout<D>::template elems<BN>();
    if ((a.causal && j0 + BN - 1 > qw) || (j0 + BN > L)) {
      int lim[NT];
#pragma unroll
      for (int t = 0; t < NT; ++t) lim[t] = (a.causal ? min(qw + t * 32 + l32, L - 1) : L - 1) - j0 - g * 4;
      fwd_tile<D, NT, true>(st, Ks, Vs, lane, c, lim);
    } else {
      const int lim[NT] = {};
      fwd_tile<D, NT, false>(st, Ks, Vs, lane, c, lim);
    }
  };
  tile_pipeline(ntiles, b0, b1, fetch, [](int, const KVBuf&) {}, compute);

  if constexpr (KS > 1) {
    // key groups 1 .. KS-1 hand their softmax state (oacc, then mu and the
    // partial row sums) to group 0 over the same rows, which merges them one
    // by one by log-sum-exp
    constexpr int NREG = DT * NT * 16 + 2 * NT;
    static_assert((KS - 1) * WR <= 4 * ((KVT / 2) / (NREG * 64)), "merge buffers");
    if (kh > 0) {
      float* red = merge_slot<NREG, KVT>(sK0, sV0, sK1, sV1, kh, wave, WR, lane);
#pragma unroll
      for (int t = 0; t < NT; ++t) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int r = 0; r < 16; ++r) red[((t * DT + dt) * 16 + r) * 64] = st.oacc[dt][t][r];
        red[(DT * NT * 16 + 2 * t) * 64] = st.mu[t];
        red[(DT * NT * 16 + 2 * t + 1) * 64] = st.lsum[t];
      }
    }
    __syncthreads();
    if (kh > 0) return;
#pragma unroll
    for (int k = 1; k < KS; ++k) {
      const float* red = merge_slot<NREG, KVT>(sK0, sV0, sK1, sV1, k, wave, WR, lane);
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const float mu_b = red[(DT * NT * 16 + 2 * t) * 64];
        const float ls_b = red[(DT * NT * 16 + 2 * t + 1) * 64];
        const float mu = fmaxf(st.mu[t], mu_b);
        // a group that saw no key has mu = -inf and nothing accumulated
        const float fa = mu == kNegInf ? 1.f : fast_exp2((st.mu[t] - mu) * c);
        const float fb = mu == kNegInf ? 0.f : fast_exp2((mu_b - mu) * c);
        st.lsum[t] = st.lsum[t] * fa + ls_b * fb;
        st.mu[t] = mu;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            st.oacc[dt][t][r] = st.oacc[dt][t][r] * fa + red[((t * DT + dt) * 16 + r) * 64] * fb;
      }
    }
  }

  // Epilogue: O = acc / l (bf16), LSE = mu*scale + ln l; padded rows 0 / -inf.
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int i = qw + t * 32 + l32;
    const float lt = xhalf_sum(st.lsum[t]);
    if (i < S) {
      const bool valid = i < L;
      const float inv = valid ? 1.f / lt : 0.f;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          bf16x4 ov;
#pragma unroll
          for (int e = 0; e < 4; ++e) ov[e] = (bf16)(st.oacc[dt][t][rr * 4 + e] * inv);
          *reinterpret_cast<bf16x4*>(Ob + (int64_t)i * os + dt * 32 + rr * 8 + g * 4) = ov;
        }
      if (g == 0) LSEb[i] = valid ? (st.mu[t] * c + __log2f(lt)) * kLn2 : kNegInf;
    }
  }
}

// ----------------------------------------------------------------------------
// Preprocess: D = rowsum(dO * O). D/8 lanes per row, 16 bytes per lane. Rows are
// walked in D's own [B, Hq, S] order so each wave writes a contiguous run of D
// (the O/dO rows it reads are whole 128/256-byte segments either way).
// ----------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(kThreads) void preprocess_kernel(PreArgs a) {
  constexpr int LPR = D / 8;  // lanes per row
  const int64_t r = (int64_t)blockIdx.x * (kThreads / LPR) + threadIdx.x / LPR;  // index into D
  const int part = threadIdx.x % LPR;
  float acc = 0.f;
  int s = 0, b = 0;
  if (r < a.rows) {
    s = (int)(r % a.S);
    const int64_t bh = r / a.S;
    const int h = (int)(bh % a.Hq);
    b = (int)(bh / a.Hq);
    const int64_t off = b * a.so.b + s * a.so.s + h * a.so.h + part * 8;
    const bf16x8 o = *reinterpret_cast<const bf16x8*>(a.o + off);
    const bf16x8 d = *reinterpret_cast<const bf16x8*>(a.d_o + off);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc += (float)o[e] * (float)d[e];
  }
#pragma unroll
  for (int off = LPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if (r < a.rows && part == 0) a.delta[r] = s < valid_len(a.seqlens, b, a.S) ? acc : 0.f;
}

// ----------------------------------------------------------------------------
// Backward dK/dV. One workgroup = one (sequence, kv head, block of 128*NTJ key
// rows); wave w owns key rows [j0 + 32*NTJ*w, +32*NTJ), keeps its K and V rows
// as B operands in registers and dK^T, dV^T accumulators. Loop over the query
// heads of the group and, for each, over 64-row query tiles from the diagonal
// to the valid length.
// ----------------------------------------------------------------------------
template <int D, int NTJ>
struct DkdvState {
  bf16x8 kf[NTJ][D / 16], vf[NTJ][D / 16];
  f32x16 dk[D / 32][NTJ], dv[D / 32][NTJ];
};

// One 64-row query tile for one wave. MASK: query row i of register (m2, r)
// takes part only if lo[t] <= m2*32 + creg_off(r) <= hi[t] (causal, and both
// positions inside the valid length).
template <int D, int NTJ, bool MASK>
__device__ __forceinline__ void dkdv_tile(DkdvState<D, NTJ>& st, const bf16* Qs, const bf16* dOs, const float* lse2,
                                          const float* ndl, int lane, float c, const int (&lo)[NTJ],
                                          const int (&hi)[NTJ]) {
  constexpr int KK = D / 16, DT = D / 32;
  const int g = lane >> 5;
  // dP starts from -D (row i of register rr*4 + e is m2*32 + rr*8 + g*4 + e,
  // four consecutive rows per 16-byte read), so that the accumulator ends as
  // dP - D and dS = P (dP - D) is one multiply
  f32x16 s[2][NTJ], dp[2][NTJ];
#pragma unroll
  for (int m2 = 0; m2 < 2; ++m2) {
    f32x16 nd;
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const float4 d4 = *reinterpret_cast<const float4*>(ndl + m2 * 32 + rr * 8 + g * 4);
      nd[rr * 4 + 0] = d4.x;
      nd[rr * 4 + 1] = d4.y;
      nd[rr * 4 + 2] = d4.z;
      nd[rr * 4 + 3] = d4.w;
    }
#pragma unroll
    for (int t = 0; t < NTJ; ++t) {
      s[m2][t] = zero16();
      dp[m2][t] = nd;
    }
  }
  // S and dP: step i = (m2, kk) = (i / KK, i % KK) takes one Q and one dO
  // fragment: the first half of the query rows (m2 = 0) is done after KK
  // steps, so its softmax can start while the second half's products run.
  // The reads run PF steps ahead of the products that use them, so that a
  // product never waits for a read issued just before it.
  constexpr int NS = 2 * KK;
  bf16x8 aq[NS], ad[NS];
  // d=128 (one wave per SIMD, registers to spare): the tile's 64 LSE values
  // are read here, so that the softmax below never waits on LDS for them
  float4 l2all[2][4];
  if constexpr (D == 128) {
#pragma unroll
    for (int m2 = 0; m2 < 2; ++m2)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) l2all[m2][rr] = *reinterpret_cast<const float4*>(lse2 + m2 * 32 + rr * 8 + g * 4);
  }
  prio_mfma();
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    aq[i] = frag_row<D>(Qs, (i / KK) * 32, (i % KK) * 16, lane);
    ad[i] = frag_row<D>(dOs, (i / KK) * 32, (i % KK) * 16, lane);
  }
#pragma unroll
  for (int i = 0; i < NS; ++i)
#pragma unroll
    for (int t = 0; t < NTJ; ++t) {
      s[i / KK][t] = mfma32(aq[i], st.kf[t][i % KK], s[i / KK][t]);
      dp[i / KK][t] = mfma32(ad[i], st.vf[t][i % KK], dp[i / KK][t]);
    }
  if constexpr (kDkdvReadAhead > 0) {
    constexpr int PF = kDkdvReadAhead;
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2 * PF, 0);
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 2 * NTJ, 0);
      if (i + PF < NS) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 0);
    }
  }
  prio_base();
  // P = exp2(S*c - LSE*log2e), dS = P (dP - D); rows m2*32 + rr*8 + g*4 + e of
  // the lane's registers rr*4 + e, read four at a time
#pragma unroll
  for (int m2 = 0; m2 < 2; ++m2)
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int il0 = m2 * 32 + rr * 8 + g * 4;
      float4 l2;
      if constexpr (D == 128) l2 = l2all[m2][rr];
      else l2 = *reinterpret_cast<const float4*>(lse2 + il0);
      const float l2v[4] = {l2.x, l2.y, l2.z, l2.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = rr * 4 + e;
#pragma unroll
        for (int t = 0; t < NTJ; ++t) {
          float p = fast_exp2(__builtin_fmaf(s[m2][t][r], c, -l2v[e]));
          if (MASK) {
            const int off = m2 * 32 + rr * 8 + e;
            if (off < lo[t] || off > hi[t]) p = 0.f;
          }
          dp[m2][t][r] = p * dp[m2][t][r];
          s[m2][t][r] = p;
        }
      }
    }
  bf16x8 pb[4][NTJ], sb[4][NTJ];
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int t = 0; t < NTJ; ++t) {
      pb[u][t] = pack8(s[u >> 1][t], (u & 1) * 8);
      sb[u][t] = pack8(dp[u >> 1][t], (u & 1) * 8);
    }
  // dV and dK: step i = (u, ct) = (i / DT, i % DT), two transposed fragments
  // (two reads each), the same read-ahead; the first half's query rows (u =
  // 0, 1) come first, so these products can start while the second half's
  // softmax still runs
  constexpr int NT2 = 4 * DT;
  bf16x8 tdo[NT2], tq[NT2];
#pragma unroll
  for (int i = 0; i < NT2; ++i) {
    tdo[i] = frag_tr<D>(dOs, (i / DT) * 16, (i % DT) * 32, lane);
    tq[i] = frag_tr<D>(Qs, (i / DT) * 16, (i % DT) * 32, lane);
  }
#pragma unroll
  for (int i = 0; i < NT2; ++i)
#pragma unroll
    for (int t = 0; t < NTJ; ++t) {
      st.dv[i % DT][t] = mfma32(tdo[i], pb[i / DT][t], st.dv[i % DT][t]);
      st.dk[i % DT][t] = mfma32(tq[i], sb[i / DT][t], st.dk[i % DT][t]);
    }
  if constexpr (kDkdvReadAhead > 0) {
    constexpr int PF = kDkdvReadAhead;
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 4 * PF, 1);
#pragma unroll
    for (int i = 0; i < NT2; ++i) {
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 2 * NTJ, 1);
      if (i + PF < NT2) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 4, 1);
    }
  }
}

// (head, query tile) of a dK/dV block's iteration it (0 .. nq*G - 1).
// down: the query tiles from the last one down to the block's first, each for
// every head of the group in turn. The blocks of a kv group that run at the
// same time (on one XCD) then read the same Q and dO tiles at the same step
// and its L2 serves them; walking up from each block's own diagonal they read
// different tiles (longseq's d=128 dK/dV fetched 9.9 GB from HBM per launch,
// 2.1 GB walking down, 2 % faster). The d=64 pass keeps the upward walk,
// each head's tiles from the diagonal up: walking down cut llama1b's fetch
// from 159 to 138 MB but not its time (0.4 % slower), and with a split it
// would put every head's masked diagonal tile in a block's last part.
__device__ __forceinline__ void dkdv_trip(int it, int nq, int G, int qt0, bool down, int& hh, int& qt) {
  if (down) {
    const int r = it / G;
    hh = it - r * G;
    qt = qt0 + nq - 1 - r;
  } else {
    hh = it / nq;
    qt = qt0 + (it - hh * nq);
  }
}

// Key block, part and part count of a dK/dV workgroup from its slot in its
// unit (dkdv_part_base gives the deal). Without a split and with pair_ends,
// the second half of the slots walks the key blocks from the far end, so that
// when two workgroups share a CU from the start a long block tends to pair
// with a short one.
__device__ __forceinline__ void dkdv_slot(int slot, int nkb, int parts, int S, int causal, bool pair_ends, int& kb,
                                          int& part, int& nparts) {
  if (parts == 1) {
    const int half = (nkb + 1) >> 1;
    kb = (!pair_ends || slot < half) ? slot : nkb - 1 - (slot - half);
    part = 0;
    nparts = 1;
    return;
  }
  int lo = 0, hi = nkb - 1;  // the last key block whose first slot is <= slot
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (dkdv_part_base(mid, nkb, parts, S, causal) <= slot)
      lo = mid;
    else
      hi = mid - 1;
  }
  kb = lo;
  const int first = dkdv_part_base(kb, nkb, parts, S, causal);
  part = slot - first;
  nparts = dkdv_part_base(kb + 1, nkb, parts, S, causal) - first;
}

// GROUPS = 1: four waves. GROUPS = 2: eight waves in two groups of four that
// own the same key rows and split the (head, query tile) sequence by parity;
// their partial dK/dV are summed through LDS at the end. With two groups each
// SIMD keeps two waves busy for the whole block, however long it is.
template <int D, int NTJ, int OCC, int GROUPS>
__global__ __launch_bounds__(kThreads * GROUPS) __attribute__((amdgpu_waves_per_eu(OCC, OCC)))
void bwd_dkdv_kernel(BwdArgs a) {
  constexpr int BMQ = 64;
  constexpr int BN = 4 * 32 * NTJ;
  constexpr int KK = D / 16;
  constexpr int DT = D / 32;
  constexpr int TILE = TileLayout<D>::template elems<BMQ>();
  // [group] tiles; Q and dO of the two pipeline stages live in distinct arrays
  __shared__ __attribute__((aligned(16))) bf16 sQ0[GROUPS * TILE], sO0[GROUPS * TILE], sQ1[GROUPS * TILE],
      sO1[GROUPS * TILE];
  __shared__ __attribute__((aligned(16))) float sstat[GROUPS][2][2][BMQ];  // [group][buf][LSE*log2e, -D]

  // a compile-time 0 with one group: the stage buffers are then the arrays
  // themselves, and the compiler can tell the tile being read from the one
  // the next tile's copy is landing in (otherwise it waits for that copy in
  // the middle of the tile)
  const int grp = GROUPS == 1 ? 0 : wave_id() >> 2;
  const int swave = wave_id() & 3;  // wave within the group, in a scalar register
  const int gtid = threadIdx.x & (kThreads - 1);
  const int lane = threadIdx.x & 63;
  const int wave = gtid >> 6;
  const int g = lane >> 5;
  const int l32 = lane & 31;

  int slot, b, hkv, kb, part, nparts;
  decode_kunit(blockIdx.x, a.B, a.Hkv, slot, b, hkv);
  dkdv_slot(slot, a.nblk, a.parts, a.S, a.causal, GROUPS == 1, kb, part, nparts);
  const int S = a.S;
  const int L = valid_len(a.seqlens, b, S);
  const int G = a.Hq / a.Hkv;
  const int64_t qs = a.sq.s;
  const int64_t os = a.so.s;
  const int64_t ks = a.skv.s;
  const bf16* Kb = a.k + b * a.skv.b + hkv * a.skv.h;
  const bf16* Vb = a.v + b * a.skv.b + hkv * a.skv.h;

  const int j0 = kb * BN;
  const int jw = j0 + wave * 32 * NTJ;
  const float c = a.scale * kLog2e;

  DkdvState<D, NTJ> st;
#pragma unroll
  for (int t = 0; t < NTJ; ++t) {
    const int j = jw + t * 32 + l32;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      const int64_t off = (int64_t)j * ks + kk * 16 + g * 8;
      st.kf[t][kk] = j < L ? *reinterpret_cast<const bf16x8*>(Kb + off) : zero_bf16x8();
      st.vf[t][kk] = j < L ? *reinterpret_cast<const bf16x8*>(Vb + off) : zero_bf16x8();
    }
#pragma unroll
    for (int ct = 0; ct < DT; ++ct) {
      st.dk[ct][t] = zero16();
      st.dv[ct][t] = zero16();
    }
  }

  const int qt0 = a.causal ? j0 / BMQ : 0;  // first query tile with rows at or below the block
  const int nq = (j0 < L) ? (L - 1) / BMQ - qt0 + 1 : 0;  // query tiles per head
  const int iters = nq * G;                               // (head, query tile) pairs
  // this workgroup's share of them: [it_lo, it_hi)
  // (an unsplit block, the usual case, takes all of them without the 64-bit
  // divisions, which cost a few hundred scalar instructions per workgroup)
  const int it_lo = nparts == 1 ? 0 : (int)((int64_t)part * iters / nparts);
  const int it_hi = nparts == 1 ? iters : (int)((int64_t)(part + 1) * iters / nparts);
  const int trips = (it_hi - it_lo + GROUPS - 1) / GROUPS;  // this group does it = it_lo + trip*GROUPS + grp

  float st_reg = 0.f;  // wave 0 of a group carries LSE, wave 1 D
  const KVBuf b0{sQ0 + grp * TILE, sO0 + grp * TILE, 0}, b1{sQ1 + grp * TILE, sO1 + grp * TILE, 1};
  // This group handles (head, query tile) pair it = it_lo + trip * GROUPS +
  // grp: head hh = it / nq, query tile qt0 + it % nq. The pipeline fetches
  // trip t + 1 and computes trip t, each in increasing order, so each keeps a
  // cursor that steps GROUPS pairs per call instead of dividing per tile, and
  // carries the offsets of the tile's first row in Q, dO and the LSE / D rows
  // (no per-tile 64-bit products).
  struct Cursor {
    int r;                // query tile - qt0
    int64_t qoff, ooff;   // elements to row (qt0 + r) * BMQ of head hkv*G + hh in Q, in dO
    int64_t soff;         // index of that row in LSE / D
  };
  const int it_first = it_lo + grp;
  const int nq1 = nq > 0 ? nq : 1;  // nq = 0 only when there are no trips
  const int hh_first = it_first / nq1;
  Cursor cur_f;
  cur_f.r = it_first - hh_first * nq1;
  {
    const int h = hkv * G + hh_first;
    const int64_t row = (int64_t)(qt0 + cur_f.r) * BMQ;
    cur_f.qoff = b * a.sq.b + h * a.sq.h + row * qs;
    cur_f.ooff = b * a.so.b + h * a.so.h + row * os;
    cur_f.soff = ((int64_t)b * a.Hq + h) * S + row;
  }
  Cursor cur_c = cur_f;
  // trips of this group that hold a pair (it < it_hi), computed once: behind
  // the empty asm the compiler keeps the value instead of recomputing the
  // 64-bit divisions of it_lo and it_hi at every use inside the loop
  int my_trips = max(0, (it_hi - it_first + GROUPS - 1) / GROUPS);
  asm volatile("" : "+s"(my_trips));
  // per step GROUPS tiles down the same head; past its last tile, back nq
  // tiles and on to the next head
  const int64_t q_step = (int64_t)GROUPS * BMQ * qs, o_step = (int64_t)GROUPS * BMQ * os;
  const int64_t q_wrap = a.sq.h - (int64_t)nq1 * BMQ * qs, o_wrap = a.so.h - (int64_t)nq1 * BMQ * os;
  const int64_t s_wrap = (int64_t)S - (int64_t)nq1 * BMQ;
  auto step = [&](Cursor& cu) {
    cu.r += GROUPS;
    cu.qoff += q_step;
    cu.ooff += o_step;
    cu.soff += GROUPS * BMQ;
    while (cu.r >= nq1) {
      cu.r -= nq1;
      cu.qoff += q_wrap;
      cu.ooff += o_wrap;
      cu.soff += s_wrap;
    }
  };
  auto fetch = [&](int trip, const KVBuf& buf) {
    if (trip >= my_trips) return;
    const int i0 = (qt0 + cur_f.r) * BMQ;
    if (swave < 2) {
      // raw value only: any arithmetic on it here would make the compiler wait
      // for this load before the tile's compute. Wave 0 of the group loads
      // LSE, wave 1 D; the choice is made on the scalar wave index (a
      // per-lane choice between the two pointers is compiled into a vector
      // load of the pointer from the argument block, waited for at once)
      const float* src = swave == 0 ? a.lse : a.delta;
      st_reg = 0.f;
      if (i0 + lane < L) st_reg = src[cur_f.soff + lane];
    }
    // the copies start at the tile's first row: rows at or past L - i0 are zeros
    tile_load_lds<BMQ, D, 4>(a.q + cur_f.qoff, qs, 0, L - i0, buf.k, wave, lane);
    tile_load_lds<BMQ, D, 4>(a.d_o + cur_f.ooff, os, 0, L - i0, buf.v, wave, lane);
    step(cur_f);
  };
  auto land = [&](int trip, const KVBuf& buf) {
    if (trip < my_trips && swave < 2) sstat[grp][buf.idx][swave][lane] = swave == 0 ? st_reg * kLog2e : -st_reg;
  };
  auto compute = [&](int trip, const KVBuf& buf) {
    if (trip >= my_trips) return;
    const int i0 = (qt0 + cur_c.r) * BMQ;
    step(cur_c);
    // skip when every query row of the tile is above this wave's key rows, or
    // the wave's keys are all padding
    if ((a.causal && i0 + BMQ - 1 < jw) || jw >= L) return;
    const float* ls = sstat[grp][buf.idx][0];
    const float* ds = sstat[grp][buf.idx][1];
    if ((a.causal && i0 < jw + 32 * NTJ - 1) || (i0 + BMQ > L) || (jw + 32 * NTJ > L)) {
      int lo[NTJ], hi[NTJ];
#pragma unroll
      for (int t = 0; t < NTJ; ++t) {
        const int j = jw + t * 32 + l32;
        lo[t] = a.causal ? j - i0 - g * 4 : -(1 << 30);  // causal: i >= j
        hi[t] = (j < L) ? L - 1 - i0 - g * 4 : -1;  // i < L, and no rows when j >= L
      }
      dkdv_tile<D, NTJ, true>(st, buf.k, buf.v, ls, ds, lane, c, lo, hi);
    } else {
      const int lo[NTJ] = {}, hi[NTJ] = {};
      dkdv_tile<D, NTJ, false>(st, buf.k, buf.v, ls, ds, lane, c, lo, hi);
    }
  };
  // the first Q/dO tile travels together with the K/V fragment loads above:
  // one wait covers both
  tile_pipeline_start(trips, b0, fetch);
  wait_vmem();
  tile_pipeline(trips, b0, b1, fetch, land, compute, /*started=*/true);

  if constexpr (GROUPS == 2) {
    // group 1 hands its partial sums to group 0 through LDS (the tile buffers
    // are free after the loop's last barrier): wave w writes [register][lane]
    // floats into the w-th tile array
    constexpr int NREG = 2 * DT * NTJ * 16;
    static_assert(NREG * 64 * sizeof(float) <= sizeof(sQ0), "reduction buffer");
    bf16* const arr = wave == 0 ? sQ0 : wave == 1 ? sO0 : wave == 2 ? sQ1 : sO1;
    float* red = reinterpret_cast<float*>(arr) + lane;
    if (grp == 1) {
#pragma unroll
      for (int ct = 0; ct < DT; ++ct)
#pragma unroll
        for (int t = 0; t < NTJ; ++t)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            red[(((ct * NTJ + t) * 2 + 0) * 16 + r) * 64] = st.dk[ct][t][r];
            red[(((ct * NTJ + t) * 2 + 1) * 16 + r) * 64] = st.dv[ct][t][r];
          }
    }
    __syncthreads();
    if (grp == 1) return;
#pragma unroll
    for (int ct = 0; ct < DT; ++ct)
#pragma unroll
      for (int t = 0; t < NTJ; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          st.dk[ct][t][r] += red[(((ct * NTJ + t) * 2 + 0) * 16 + r) * 64];
          st.dv[ct][t][r] += red[(((ct * NTJ + t) * 2 + 1) * 16 + r) * 64];
        }
  }

  if (a.parts > 1) {
    // split: this part's unscaled fp32 sums for the valid key rows; the
    // reduce pass adds the parts, scales dK, rotates back and converts
    const int64_t prow = ((int64_t)part * a.B + b) * S;
#pragma unroll
    for (int t = 0; t < NTJ; ++t) {
      const int j = jw + t * 32 + l32;
      if (j < L) {
        float* pk = a.part_dk + ((prow + j) * a.Hkv + hkv) * D;
        float* pv = a.part_dv + ((prow + j) * a.Hkv + hkv) * D;
#pragma unroll
        for (int ct = 0; ct < DT; ++ct)
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) {
            const int c0 = ct * 32 + rr * 8 + g * 4;
            *reinterpret_cast<float4*>(pk + c0) = make_float4(st.dk[ct][t][rr * 4 + 0], st.dk[ct][t][rr * 4 + 1],
                                                              st.dk[ct][t][rr * 4 + 2], st.dk[ct][t][rr * 4 + 3]);
            *reinterpret_cast<float4*>(pv + c0) = make_float4(st.dv[ct][t][rr * 4 + 0], st.dv[ct][t][rr * 4 + 1],
                                                              st.dv[ct][t][rr * 4 + 2], st.dv[ct][t][rr * 4 + 3]);
          }
      }
    }
    return;
  }

  // Epilogue: dK = scale * dK^T, dV = dV^T transposed back; lane owns key row j.
  bf16* dKb = a.dk + b * a.skv.b + hkv * a.skv.h;
  bf16* dVb = a.dv + b * a.skv.b + hkv * a.skv.h;
#pragma unroll
  for (int t = 0; t < NTJ; ++t) {
    const int j = jw + t * 32 + l32;
    if (j < S) {
      const bool valid = j < L;
#pragma unroll
      for (int ct = 0; ct < DT; ++ct)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          bf16x4 kv4, vv4;
          float kx[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) kx[e] = st.dk[ct][t][rr * 4 + e] * a.scale;
          if (a.rope) rope_adjoint4(a.rf, ct * 32 + rr * 8, g, j, kx);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            kv4[e] = (bf16)(valid ? kx[e] : 0.f);
            vv4[e] = (bf16)(valid ? st.dv[ct][t][rr * 4 + e] : 0.f);
          }
          const int64_t off = (int64_t)j * ks + ct * 32 + rr * 8 + g * 4;
          *reinterpret_cast<bf16x4*>(dKb + off) = kv4;
          *reinterpret_cast<bf16x4*>(dVb + off) = vv4;
        }
    }
  }
}

// ----------------------------------------------------------------------------
// Backward dK/dV with each key slice's work split over two waves of one SIMD
// by role (d = 128, where one wave doing all of it needs 424 registers and so
// runs alone on its SIMD). Eight waves per 128-key block: for key rows
// [j0 + 32w, +32), wave w (the P wave) holds K and accumulates dV^T, wave
// w + 4 (the dS wave, on the same SIMD) holds V and accumulates dK^T. Each
// (head, query tile) takes two phases between barriers: first the P wave forms
// S^T = K Q^T and P = exp2(S c - LSE log2e) and leaves P in LDS (fp32, the
// lane's registers in order) while the dS wave forms dP^T = V dO^T - D; then
// the P wave adds P^T dO to dV^T while the dS wave forms dS = P (dP - D) from
// that P and adds dS^T Q to dK^T. The products and the softmax are those of
// dkdv_tile, term for term; each wave runs half of them, and the two waves of
// a SIMD interleave.
// ----------------------------------------------------------------------------

// LDS reads run this many product steps ahead in the role split's tiles (at
// d=128: 8 measured 2 % faster than 4, 12 or 16 slower; 0 and 2 as 4).
constexpr int kRoleReadAhead = 8;

// The P wave's share of one 64-row query tile, first part: S and P (written
// to pout, and packed to bf16 in pb for the dV product).
template <int D, bool MASK>
__device__ __forceinline__ void dkdv_p_scores(const bf16x8 (&kf)[D / 16], const bf16* Qs, const float* lse2,
                                              float* pout, int lane, float c, int lo, int hi, bf16x8 (&pb)[4]) {
  constexpr int KK = D / 16;
  const int g = lane >> 5;
  f32x16 s[2] = {zero16(), zero16()};
  constexpr int NS = 2 * KK;  // step i = (kk, m2) = (i / 2, i % 2)
  bf16x8 aq[NS];
  prio_mfma();
#pragma unroll
  for (int i = 0; i < NS; ++i) aq[i] = frag_row<D>(Qs, (i & 1) * 32, (i >> 1) * 16, lane);
#pragma unroll
  for (int i = 0; i < NS; ++i) s[i & 1] = mfma32(aq[i], kf[i >> 1], s[i & 1]);
  if constexpr (kRoleReadAhead > 0) {
    constexpr int PF = kRoleReadAhead;
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, PF, 0);
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
      if (i + PF < NS) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
    }
  }
  prio_base();
  // P = exp2(S*c - LSE*log2e); rows m2*32 + rr*8 + g*4 + e of registers rr*4 + e
#pragma unroll
  for (int m2 = 0; m2 < 2; ++m2)
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const float4 l2 = *reinterpret_cast<const float4*>(lse2 + m2 * 32 + rr * 8 + g * 4);
      const float l2v[4] = {l2.x, l2.y, l2.z, l2.w};
      float pv[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float p = fast_exp2(__builtin_fmaf(s[m2][rr * 4 + e], c, -l2v[e]));
        if (MASK) {
          const int off = m2 * 32 + rr * 8 + e;
          if (off < lo || off > hi) p = 0.f;
        }
        s[m2][rr * 4 + e] = p;
        pv[e] = p;
      }
      *reinterpret_cast<float4*>(pout + ((m2 * 4 + rr) * 64 + lane) * 4) = make_float4(pv[0], pv[1], pv[2], pv[3]);
    }
#pragma unroll
  for (int u = 0; u < 4; ++u) pb[u] = pack8(s[u >> 1], (u & 1) * 8);
}

// Second part, common to masked and interior tiles (so that dV^T stays in one
// set of registers): dV^T += P^T dO.
template <int D>
__device__ __forceinline__ void dkdv_p_dv(f32x16 (&dv)[D / 32], const bf16* dOs, const bf16x8 (&pb)[4], int lane) {
  constexpr int DT = D / 32;
  constexpr int NT2 = 4 * DT;  // step i = (ct, u) = (i / 4, i % 4)
  bf16x8 tdo[NT2];
#pragma unroll
  for (int i = 0; i < NT2; ++i) tdo[i] = frag_tr<D>(dOs, (i & 3) * 16, (i >> 2) * 32, lane);
#pragma unroll
  for (int i = 0; i < NT2; ++i) dv[i >> 2] = mfma32(tdo[i], pb[i & 3], dv[i >> 2]);
  if constexpr (kRoleReadAhead > 0) {
    constexpr int PF = kRoleReadAhead;
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2 * PF, 1);
#pragma unroll
    for (int i = 0; i < NT2; ++i) {
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 1);
      if (i + PF < NT2) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 1);
    }
  }
}

// The dS wave's first phase: dP^T - D (the accumulators start from -D).
template <int D>
__device__ __forceinline__ void dkdv_ds_dp(const bf16x8 (&vf)[D / 16], const bf16* dOs, const float* ndl, int lane,
                                           f32x16 (&dp)[2]) {
  constexpr int KK = D / 16;
  const int g = lane >> 5;
#pragma unroll
  for (int m2 = 0; m2 < 2; ++m2)
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const float4 d4 = *reinterpret_cast<const float4*>(ndl + m2 * 32 + rr * 8 + g * 4);
      dp[m2][rr * 4 + 0] = d4.x;
      dp[m2][rr * 4 + 1] = d4.y;
      dp[m2][rr * 4 + 2] = d4.z;
      dp[m2][rr * 4 + 3] = d4.w;
    }
  constexpr int NS = 2 * KK;
  bf16x8 ad[NS];
  prio_mfma();
#pragma unroll
  for (int i = 0; i < NS; ++i) ad[i] = frag_row<D>(dOs, (i & 1) * 32, (i >> 1) * 16, lane);
#pragma unroll
  for (int i = 0; i < NS; ++i) dp[i & 1] = mfma32(ad[i], vf[i >> 1], dp[i & 1]);
  if constexpr (kRoleReadAhead > 0) {
    constexpr int PF = kRoleReadAhead;
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, PF, 0);
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
      if (i + PF < NS) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
    }
  }
  prio_base();
}

// The dS wave's second phase: dS = P (dP - D) with P from pin (zero where the
// P wave masked it), then dK^T += dS^T Q.
template <int D>
__device__ __forceinline__ void dkdv_ds_dk(f32x16 (&dk)[D / 32], const bf16* Qs, const float* pin, int lane,
                                           f32x16 (&dp)[2]) {
  constexpr int DT = D / 32;
#pragma unroll
  for (int m2 = 0; m2 < 2; ++m2)
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const float4 p4 = *reinterpret_cast<const float4*>(pin + ((m2 * 4 + rr) * 64 + lane) * 4);
      dp[m2][rr * 4 + 0] *= p4.x;
      dp[m2][rr * 4 + 1] *= p4.y;
      dp[m2][rr * 4 + 2] *= p4.z;
      dp[m2][rr * 4 + 3] *= p4.w;
    }
  bf16x8 sb[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) sb[u] = pack8(dp[u >> 1], (u & 1) * 8);
  constexpr int NT2 = 4 * DT;
  bf16x8 tq[NT2];
#pragma unroll
  for (int i = 0; i < NT2; ++i) tq[i] = frag_tr<D>(Qs, (i & 3) * 16, (i >> 2) * 32, lane);
#pragma unroll
  for (int i = 0; i < NT2; ++i) dk[i >> 2] = mfma32(tq[i], sb[i & 3], dk[i >> 2]);
  if constexpr (kRoleReadAhead > 0) {
    constexpr int PF = kRoleReadAhead;
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2 * PF, 1);
#pragma unroll
    for (int i = 0; i < NT2; ++i) {
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 1);
      if (i + PF < NT2) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 1);
    }
  }
}

template <int D>
__global__ __launch_bounds__(8 * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
void bwd_dkdv_roles_kernel(BwdArgs a) {
  constexpr int BMQ = 64;
  constexpr int BN = 128;
  constexpr int KK = D / 16;
  constexpr int DT = D / 32;
  constexpr int TILE = TileLayout<D>::template elems<BMQ>();
  // two stages of the Q and dO tiles, each its own array
  __shared__ __attribute__((aligned(16))) bf16 sQ0[TILE], sO0[TILE], sQ1[TILE], sO1[TILE];
  // P of the four P waves: [key slice][(m2, rr)][lane][4]
  __shared__ __attribute__((aligned(16))) float sP[4][8 * 64 * 4];
  __shared__ __attribute__((aligned(16))) float sstat[2][2][BMQ];  // [stage][LSE*log2e, -D]

  const int wid = wave_id();      // scalar
  const bool ds_role = wid >= 4;  // waves 4..7: dS waves
  const int kw = wid & 3;         // key slice
  const int lane = threadIdx.x & 63;
  const int g = lane >> 5;
  const int l32 = lane & 31;

  int slot, b, hkv, kb, part, nparts;
  decode_kunit(blockIdx.x, a.B, a.Hkv, slot, b, hkv);
  dkdv_slot(slot, a.nblk, a.parts, a.S, a.causal, false, kb, part, nparts);
  const int S = a.S;
  const int L = valid_len(a.seqlens, b, S);
  const int G = a.Hq / a.Hkv;
  const int64_t qs = a.sq.s;
  const int64_t os = a.so.s;
  const int64_t ks = a.skv.s;

  const int j0 = kb * BN;
  const int jw = j0 + kw * 32;
  const int j = jw + l32;  // the lane's key row
  const float c = a.scale * kLog2e;

  // the P wave keeps K rows, the dS wave V rows (B operands of S^T and dP^T)
  const bf16* KVb = (ds_role ? a.v : a.k) + b * a.skv.b + hkv * a.skv.h;
  bf16x8 kv[KK];
  f32x16 acc[DT];  // dV^T (P wave) or dK^T (dS wave)
#pragma unroll
  for (int kk = 0; kk < KK; ++kk)
    kv[kk] = j < L ? *reinterpret_cast<const bf16x8*>(KVb + (int64_t)j * ks + kk * 16 + g * 8) : zero_bf16x8();
#pragma unroll
  for (int ct = 0; ct < DT; ++ct) acc[ct] = zero16();

  const int qt0 = a.causal ? j0 / BMQ : 0;  // first query tile with rows at or below the block
  const int nq = (j0 < L) ? (L - 1) / BMQ - qt0 + 1 : 0;  // query tiles per head
  const int iters = nq * G;                               // (head, query tile) pairs
  const int it_lo = nparts == 1 ? 0 : (int)((int64_t)part * iters / nparts);
  const int it_hi = nparts == 1 ? iters : (int)((int64_t)(part + 1) * iters / nparts);
  const int trips = it_hi - it_lo;

  float st_reg = 0.f;  // wave 0 carries LSE, wave 1 D
  auto fetch = [&](int t, const KVBuf& buf) {
    const int it = it_lo + t;
    int hh, qt;
    dkdv_trip(it, nq, G, qt0, a.parts == 1, hh, qt);
    const int h = hkv * G + hh;
    if (wid < 2) {
      // raw value only (arithmetic here would make the compiler wait for the
      // load before the step's compute); the pointer is chosen on the scalar
      // wave index
      const int i = qt * BMQ + lane;
      const float* src = wid == 0 ? a.lse : a.delta;
      st_reg = 0.f;
      if (i < L) st_reg = src[((int64_t)b * a.Hq + h) * S + i];
    }
    const bf16* Qb = a.q + b * a.sq.b + h * a.sq.h;
    const bf16* dOb = a.d_o + b * a.so.b + h * a.so.h;
    tile_load_lds<BMQ, D, 8>(Qb, qs, qt * BMQ, L, buf.k, wid, lane);
    tile_load_lds<BMQ, D, 8>(dOb, os, qt * BMQ, L, buf.v, wid, lane);
  };
  auto land = [&](int t, const KVBuf& buf) {
    if (t < trips && wid < 2) sstat[buf.idx][wid][lane] = wid == 0 ? st_reg * kLog2e : -st_reg;
  };
  // 0: the tile has no (key, query) pair of this slice; 1: masked; 2: interior
  auto kind = [&](int t, int& i0) {
    const int it = it_lo + t;
    int hh, qt;
    dkdv_trip(it, nq, G, qt0, a.parts == 1, hh, qt);
    i0 = qt * BMQ;
    if ((a.causal && i0 + BMQ - 1 < jw) || jw >= L) return 0;
    return ((a.causal && i0 < jw + 31) || (i0 + BMQ > L) || (jw + 32 > L)) ? 1 : 2;
  };
  float* const pslot = &sP[kw][0];
  // the barrier between the phases publishes P only: it waits for the wave's
  // own LDS accesses (lgkmcnt) and leaves the next tile's copy in flight, which
  // __syncthreads() (a workgroup fence) would drain; the compiler fences keep
  // memory operations on their side of it
  auto phase_barrier = []() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  auto compute_p = [&](int t, const KVBuf& buf) {
    int i0;
    const int kd = kind(t, i0);
    bf16x8 pb[4];
    if (kd == 1) {
      const int lo = a.causal ? j - i0 - g * 4 : -(1 << 30);  // causal: i >= j
      const int hi = (j < L) ? L - 1 - i0 - g * 4 : -1;       // i < L, and no rows when j >= L
      dkdv_p_scores<D, true>(kv, buf.k, sstat[buf.idx][0], pslot, lane, c, lo, hi, pb);
    } else if (kd == 2) {
      dkdv_p_scores<D, false>(kv, buf.k, sstat[buf.idx][0], pslot, lane, c, 0, 0, pb);
    }
    phase_barrier();  // P is in LDS for the partner
    if (kd != 0) dkdv_p_dv<D>(acc, buf.v, pb, lane);
  };
  auto compute_ds = [&](int t, const KVBuf& buf) {
    int i0;
    const int kd = kind(t, i0);
    f32x16 dp[2];
    if (kd != 0) dkdv_ds_dp<D>(kv, buf.v, sstat[buf.idx][1], lane, dp);
    phase_barrier();  // the partner's P is in LDS
    if (kd != 0) dkdv_ds_dk<D>(acc, buf.k, pslot, lane, dp);
  };
  // each role runs its own copy of the pipeline loop (same steps, same
  // barriers), so that its accumulators stay in one set of registers
  KVBuf b0{sQ0, sO0, 0}, b1{sQ1, sO1, 1};
  // the first tile travels together with the K or V rows above: one wait
  tile_pipeline_start(trips, b0, fetch);
  wait_vmem();
  if (ds_role)
    tile_pipeline(trips, b0, b1, fetch, land, compute_ds, /*started=*/true);
  else
    tile_pipeline(trips, b0, b1, fetch, land, compute_p, /*started=*/true);

  if (a.parts > 1) {
    // this part's unscaled fp32 sums for the valid key rows (dV from the P
    // waves, dK from the dS waves); the reduce pass adds the parts
    if (j < L) {
      const int64_t prow = ((int64_t)part * a.B + b) * S;
      float* dst = (ds_role ? a.part_dk : a.part_dv) + ((prow + j) * a.Hkv + hkv) * D;
#pragma unroll
      for (int ct = 0; ct < DT; ++ct)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr)
          *reinterpret_cast<float4*>(dst + ct * 32 + rr * 8 + g * 4) =
              make_float4(acc[ct][rr * 4 + 0], acc[ct][rr * 4 + 1], acc[ct][rr * 4 + 2], acc[ct][rr * 4 + 3]);
    }
    return;
  }

  // Epilogue: dK = scale * dK^T (and the rotation's adjoint), dV = dV^T,
  // transposed back; the lane owns key row j; padded rows get zeros
  if (j < S) {
    const bool valid = j < L;
    bf16* dst = (ds_role ? a.dk : a.dv) + b * a.skv.b + hkv * a.skv.h;
#pragma unroll
    for (int ct = 0; ct < DT; ++ct)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        float x[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = acc[ct][rr * 4 + e];
        if (ds_role) {
#pragma unroll
          for (int e = 0; e < 4; ++e) x[e] *= a.scale;
          if (a.rope) rope_adjoint4(a.rf, ct * 32 + rr * 8, g, j, x);
        }
        bf16x4 o4;
#pragma unroll
        for (int e = 0; e < 4; ++e) o4[e] = (bf16)(valid ? x[e] : 0.f);
        *reinterpret_cast<bf16x4*>(dst + (int64_t)j * ks + ct * 32 + rr * 8 + g * 4) = o4;
      }
  }
}

// ----------------------------------------------------------------------------
// dK/dV reduce (split dK/dV pass only): dK = scale * sum_p part_dk[p], dV =
// sum_p part_dv[p] over the parts in a fixed order (deterministic), the
// rotation's adjoint applied to dK, rounded to bf16 and written through the
// K strides; padded key rows (j >= L) get zeros. One thread per 4 consecutive
// elements of a (sequence, position, kv head) row.
// ----------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(kThreads) void dkdv_reduce_kernel(BwdArgs a) {
  constexpr int C4 = D / 4;
  const int64_t tid = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const int64_t total = (int64_t)a.B * a.S * a.Hkv * C4;
  if (tid >= total) return;
  const int c4 = (int)(tid % C4);
  const int64_t row = tid / C4;  // (b * S + j) * Hkv + hkv
  const int hkv = (int)(row % a.Hkv);
  const int64_t bj = row / a.Hkv;
  const int j = (int)(bj % a.S);
  const int b = (int)(bj / a.S);
  const int L = valid_len(a.seqlens, b, a.S);
  float kx[4] = {0.f, 0.f, 0.f, 0.f}, vx[4] = {0.f, 0.f, 0.f, 0.f};
  if (j < L) {
    const int64_t pstride = (int64_t)a.B * a.S * a.Hkv * D;
    const int64_t off = row * D + c4 * 4;
    const int kb = j / 128;  // the row's key block and the parts it was split into
    const int nparts = dkdv_part_base(kb + 1, a.nblk, a.parts, a.S, a.causal) -
                       dkdv_part_base(kb, a.nblk, a.parts, a.S, a.causal);
    for (int p = 0; p < nparts; ++p) {
      const float4 k4 = *reinterpret_cast<const float4*>(a.part_dk + p * pstride + off);
      const float4 v4 = *reinterpret_cast<const float4*>(a.part_dv + p * pstride + off);
      kx[0] += k4.x; kx[1] += k4.y; kx[2] += k4.z; kx[3] += k4.w;
      vx[0] += v4.x; vx[1] += v4.y; vx[2] += v4.z; vx[3] += v4.w;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) kx[e] *= a.scale;
    // pairs (d, d+1), (d+2, d+3) with d = c4 * 4 = d0 + 4g
    if (a.rope) rope_adjoint4(a.rf, (c4 * 4) & ~7, c4 & 1, j, kx);
  }
  bf16x4 k4b, v4b;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    k4b[e] = (bf16)kx[e];
    v4b[e] = (bf16)vx[e];
  }
  const int64_t o = b * a.skv.b + (int64_t)j * a.skv.s + hkv * a.skv.h + c4 * 4;
  *reinterpret_cast<bf16x4*>(a.dk + o) = k4b;
  *reinterpret_cast<bf16x4*>(a.dv + o) = v4b;
}

// ----------------------------------------------------------------------------
// Backward dQ. Same tiling as the forward: one workgroup per (sequence, query
// head, query block); recompute S^T and dP^T per 64-row K/V tile, then
// dQ^T += K^T dS^T. The dP^T accumulator starts from -D (one MFMA of a ones
// column against -D as a bf16 pair hi + lo, |hi + lo + D| <= 2^-16 |D|), so
// dS = P (dP - D) costs one multiply per element.
// ----------------------------------------------------------------------------
template <int D, int NT>
struct DqState {
  bf16x8 qf[NT][D / 16], df[NT][D / 16];
  float l2[NT], dd[NT];
  f32x16 acc[D / 32][NT];
  // -D as a rank-one term of the dP^T product: a column of ones (A) against
  // -D split into a bf16 pair hi + lo (B, k = 0 and 1 of the lane's query)
  bf16x8 ones, nd[NT];
};

// One 64-key tile for one wave. MASK: key register offset must be <= lim[t]
// (lim < 0 excludes the whole row).
template <int D, int NT, bool MASK>
__device__ __forceinline__ void dq_tile(DqState<D, NT>& st, const bf16* Ks, const bf16* Vs, int lane, float c,
                                        const int (&lim)[NT]) {
  constexpr int KK = D / 16, DT = D / 32;
  f32x16 s[2][NT], dp[2][NT];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      s[mt][t] = zero16();
      dp[mt][t] = mfma32(st.ones, st.nd[t], zero16());  // every row: -D of the lane's query
    }
  // step i = (kk, mt) = (i / 2, i % 2): one K and one V fragment, read
  // ahead of the products as in the dK/dV tile
  constexpr int NS = 2 * KK;
  bf16x8 ak[NS], av[NS];
  prio_mfma();
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    ak[i] = frag_row<D>(Ks, (i & 1) * 32, (i >> 1) * 16, lane);
    av[i] = frag_row<D>(Vs, (i & 1) * 32, (i >> 1) * 16, lane);
  }
#pragma unroll
  for (int i = 0; i < NS; ++i)
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      s[i & 1][t] = mfma32(ak[i], st.qf[t][i >> 1], s[i & 1][t]);
      dp[i & 1][t] = mfma32(av[i], st.df[t][i >> 1], dp[i & 1][t]);
    }
  if constexpr (kDqReadAhead<D> > 0) {
    constexpr int PF = kDqReadAhead<D>;
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2 * PF, 0);
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 2 * NT, 0);
      if (i + PF < NS) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 0);
    }
  }
  prio_base();
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float p = fast_exp2(__builtin_fmaf(s[mt][t][r], c, -st.l2[t]));
        if (MASK && mt * 32 + creg_off(r) > lim[t]) p = 0.f;
        dp[mt][t][r] = p * dp[mt][t][r];  // dS = P (dP - D)
      }
  bf16x8 sb[4][NT];
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int t = 0; t < NT; ++t) sb[u][t] = pack8(dp[u >> 1][t], (u & 1) * 8);
  constexpr int NT2 = 4 * DT;
  bf16x8 tk[NT2];
#pragma unroll
  for (int i = 0; i < NT2; ++i) tk[i] = frag_tr<D>(Ks, (i & 3) * 16, (i >> 2) * 32, lane);
#pragma unroll
  for (int i = 0; i < NT2; ++i)
#pragma unroll
    for (int t = 0; t < NT; ++t) st.acc[i >> 2][t] = mfma32(tk[i], sb[i & 3][t], st.acc[i >> 2][t]);
  if constexpr (kDqReadAhead<D> > 0) {
    constexpr int PF = kDqReadAhead<D>;
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2 * PF, 1);
#pragma unroll
    for (int i = 0; i < NT2; ++i) {
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, NT, 1);
      if (i + PF < NT2) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 1);
    }
  }
}

// KS = 2 (small grids): as in the forward, two halves of the workgroup's
// waves take the even and the odd 64-key tiles of the same query rows; the
// odd half's dQ sums are added to the even half's through LDS at the end.
template <int D, int NT, int OCC, int W, int KS = 1>
__global__ __launch_bounds__(64 * W) __attribute__((amdgpu_waves_per_eu(OCC, OCC)))
void bwd_dq_kernel(BwdArgs a) {
  constexpr int BN = 64;
  constexpr int WR = W / KS;  // waves per key half (each owns 32*NT query rows)
  constexpr int BM = WR * 32 * NT;
  constexpr int KK = D / 16;
  constexpr int DT = D / 32;
  constexpr int KVT = TileLayout<D>::template elems<KS * BN>();
  static_assert(KS == 1 || KS == 2 || KS == 4, "key split");
  __shared__ __attribute__((aligned(16))) bf16 sK0[KVT], sV0[KVT], sK1[KVT], sV1[KVT];

  const int lane = threadIdx.x & 63;
  const int wave_all = threadIdx.x >> 6;
  const int wave = wave_all % WR;   // row wave
  const int kh = wave_all / WR;     // key half
  const int g = lane >> 5;
  const int l32 = lane & 31;

  int qb, b, h;
  decode_qblock(blockIdx.x, a.nblk, a.B, a.Hq, a.Hkv, qb, b, h);
  const int S = a.S;
  const int L = valid_len(a.seqlens, b, S);
  const int hkv = h / (a.Hq / a.Hkv);
  const int64_t qs = a.sq.s;
  const int64_t os = a.so.s;
  const int64_t ks = a.skv.s;
  const bf16* Qb = a.q + b * a.sq.b + h * a.sq.h;
  const bf16* dOb = a.d_o + b * a.so.b + h * a.so.h;
  const bf16* Kb = a.k + b * a.skv.b + hkv * a.skv.h;
  const bf16* Vb = a.v + b * a.skv.b + hkv * a.skv.h;
  const float* LSEb = a.lse + ((int64_t)b * a.Hq + h) * S;
  const float* Db = a.delta + ((int64_t)b * a.Hq + h) * S;
  bf16* dQb = a.dq + b * a.so.b + h * a.so.h;

  const int q0 = qb * BM;
  const int qw = q0 + wave * 32 * NT;
  const int kend = a.causal ? min(q0 + BM, L) : L;
  const int ntiles = (q0 < L) ? (kend - 1) / (KS * BN) + 1 : 0;  // pipeline steps of KS tiles
  const int wave_last = min(qw + 32 * NT, L) - 1;
  const int key_last = a.causal ? wave_last : (wave_last < qw ? -1 : L - 1);
  const float c = a.scale * kLog2e;

  // K/V tiles stream straight into LDS (no staging registers), double-buffered.
  const KVBuf b0{sK0, sV0, 0}, b1{sK1, sV1, 1};
  auto fetch = [&](int kt, const KVBuf& buf) {
    tile_load_lds<KS * BN, D, W>(Kb, ks, kt * KS * BN, L, buf.k, wave_all, lane);
    tile_load_lds<KS * BN, D, W>(Vb, ks, kt * KS * BN, L, buf.v, wave_all, lane);
  };
  // the first K/V tile is issued before the row loads below, so that its copy
  // travels while they land and the prologue does its arithmetic on them
  tile_pipeline_start(ntiles, b0, fetch);

  DqState<D, NT> st;
  st.ones = zero_bf16x8();
  if (g == 0) {
    st.ones[0] = (bf16)1.f;
    st.ones[1] = (bf16)1.f;
  }
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int row = qw + t * 32 + l32;
    const bool valid = row < L;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      const int64_t col = kk * 16 + g * 8;
      st.qf[t][kk] = valid ? *reinterpret_cast<const bf16x8*>(Qb + (int64_t)row * qs + col) : zero_bf16x8();
      st.df[t][kk] = valid ? *reinterpret_cast<const bf16x8*>(dOb + (int64_t)row * os + col) : zero_bf16x8();
    }
    st.l2[t] = valid ? LSEb[row] * kLog2e : 0.f;
    if (a.o) {
      // D from the bf16 O and dO rows: this lane holds half of each row's
      // elements (16-element chunks split over the lane halves)
      const bf16* Orow = a.o + b * a.so.b + h * a.so.h + (int64_t)row * os;
      float part = 0.f;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        const bf16x8 ov = valid ? *reinterpret_cast<const bf16x8*>(Orow + kk * 16 + g * 8) : zero_bf16x8();
#pragma unroll
        for (int e = 0; e < 8; ++e) part += (float)ov[e] * (float)st.df[t][kk][e];
      }
      const float dsum = xhalf_sum(part);
      st.dd[t] = valid ? dsum : 0.f;
      if (g == 0 && kh == 0 && row < S) a.delta_out[((int64_t)b * a.Hq + h) * S + row] = valid ? dsum : 0.f;
    } else {
      st.dd[t] = valid ? Db[row] : 0.f;
    }
    {
      const float nd = -st.dd[t];
      const bf16 hi = (bf16)nd;
      const bf16 lo = (bf16)(nd - (float)hi);
      bf16x8 v = zero_bf16x8();
      if (g == 0) {
        v[0] = hi;
        v[1] = lo;
      }
      st.nd[t] = v;
    }
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) st.acc[dt][t] = zero16();
  }
  wait_vmem();

  auto compute = [&](int kt, const KVBuf& buf) {
    const int j0 = (kt * KS + kh) * BN;
    if (j0 > key_last) return;
    const bf16* Ks = buf.k + kh * TileLayout<D>::template elems<BN>();
    const bf16* Vs = buf.v + kh * TileLayout<D>::template elems<BN>();
    if ((a.causal && j0 + BN - 1 > qw) || (j0 + BN > L) || (qw + 32 * NT > L)) {
      int lim[NT];
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const int i = qw + t * 32 + l32;
        lim[t] = i < L ? (a.causal ? i : L - 1) - j0 - g * 4 : -1;
      }
      dq_tile<D, NT, true>(st, Ks, Vs, lane, c, lim);
    } else {
      const int lim[NT] = {};
      dq_tile<D, NT, false>(st, Ks, Vs, lane, c, lim);
    }
  };
  tile_pipeline(ntiles, b0, b1, fetch, [](int, const KVBuf&) {}, compute, /*started=*/true);

  if constexpr (KS > 1) {
    // key groups 1 .. KS-1 add their dQ sums to group 0's through LDS
    constexpr int NREG = DT * NT * 16;
    static_assert((KS - 1) * WR <= 4 * ((KVT / 2) / (NREG * 64)), "reduction buffers");
    if (kh > 0) {
      float* red = merge_slot<NREG, KVT>(sK0, sV0, sK1, sV1, kh, wave, WR, lane);
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int r = 0; r < 16; ++r) red[((t * DT + dt) * 16 + r) * 64] = st.acc[dt][t][r];
    }
    __syncthreads();
    if (kh > 0) return;
#pragma unroll
    for (int k = 1; k < KS; ++k) {
      const float* red = merge_slot<NREG, KVT>(sK0, sV0, sK1, sV1, k, wave, WR, lane);
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int r = 0; r < 16; ++r) st.acc[dt][t][r] += red[((t * DT + dt) * 16 + r) * 64];
    }
  }

#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int i = qw + t * 32 + l32;
    if (i < S) {
      const bool valid = i < L;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          bf16x4 ov;
          float qx[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) qx[e] = st.acc[dt][t][rr * 4 + e] * a.scale;
          if (a.rope) rope_adjoint4(a.rf, dt * 32 + rr * 8, g, i, qx);
#pragma unroll
          for (int e = 0; e < 4; ++e) ov[e] = (bf16)(valid ? qx[e] : 0.f);
          *reinterpret_cast<bf16x4*>(dQb + (int64_t)i * os + dt * 32 + rr * 8 + g * 4) = ov;
        }
    }
  }
}

// ----------------------------------------------------------------------------
// RoPE pre-pass: q_rot, k_rot = the rotated q and k, once per step (HBM-bound:
// every element read and written once). The forward and both backward passes
// then read the rotated tensors; the backward passes take dQ and dK back
// through the adjoint in their epilogues. One wave per (sequence, position):
// its D/2 (cos, sin) pairs are computed once into LDS, then each lane rotates
// 8 consecutive elements (16 bytes, four pairs) at a time, walking the rows of
// every q head, then every k head, of that position.
// ----------------------------------------------------------------------------
struct RopeArgs {
  const bf16* q;
  const bf16* k;
  bf16* qr;
  bf16* kr;
  int S, Hq, Hkv;
  RopeFreq rf;
  Strides sq, skv;  // q and q_rot; k and k_rot
};

template <int D>
__global__ __launch_bounds__(64) void rope_kernel(RopeArgs a) {
  constexpr int CPR = D / 8;  // 16-byte chunks per row
  __shared__ float2 cs_tab[D / 2];
  const int lane = threadIdx.x;
  const int b = blockIdx.x / a.S;
  const int p = blockIdx.x - b * a.S;
  if (lane < D / 2) {
    float cs, sn;
    rope_cos_sin(a.rf.phi[lane], p, cs, sn);
    cs_tab[lane] = make_float2(cs, sn);
  }
  __syncthreads();
  const int nq = a.Hq * CPR, n = (a.Hq + a.Hkv) * CPR;
  for (int i = lane; i < n; i += 64) {
    const bool isq = i < nq;
    const int ih = isq ? i : i - nq;
    const int h = ih / CPR, c = ih % CPR;
    const Strides& st = isq ? a.sq : a.skv;
    const int64_t off = (int64_t)b * st.b + (int64_t)p * st.s + (int64_t)h * st.h + c * 8;
    const bf16x8 x = *reinterpret_cast<const bf16x8*>((isq ? a.q : a.k) + off);
    bf16x8 y;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float2 t = cs_tab[c * 4 + e];
      const float x0 = (float)x[2 * e], x1 = (float)x[2 * e + 1];
      y[2 * e] = (bf16)(x0 * t.x - x1 * t.y);
      y[2 * e + 1] = (bf16)(x0 * t.y + x1 * t.x);
    }
    *reinterpret_cast<bf16x8*>((isq ? a.qr : a.kr) + off) = y;
  }
}

// ----------------------------------------------------------------------------
// Decode. Sq new queries per sequence (the last Sq cached positions) against a
// [B, Smax, Hkv, d] key/value cache. The R = G*Sq query rows of a kv head (row
// r: head r / Sq of the group, new query r % Sq) are cut into RB blocks of 32
// MFMA rows; a unit is one (sequence, kv head, row block). The valid 64-key
// tiles of all units, laid end to end (sequence-major, then kv head, then row
// block), are dealt out evenly
// to the W one-wave workgroups of the grid: wave w takes tiles
// [floor(w*T/W), floor((w+1)*T/W)) of the T in total, so every wave streams
// the same number of bytes whatever the mix of cache lengths. A wave's range
// may cross units; for each unit it touches it runs the forward's tile
// routine over its share of that unit's tiles and writes a normalised fp32
// partial O and its LSE to slot w + u. The (wave, unit) pairs form a
// staircase (a later wave never returns to an earlier unit), so w + u never
// repeats and W + U - 1 slots suffice. The merge kernel combines the partials
// of each query row by log-sum-exp. The work is bound by streaming the cache
// from HBM.
// ----------------------------------------------------------------------------
struct DecArgs {
  const bf16* q;
  const bf16* k;
  const bf16* v;
  const int32_t* lens;
  int* hdr;       // hdr[0] = T, the number of valid tiles over all units
  int2* uinfo;    // per unit: first and last wave holding a partial of it
  float* ws_o;    // [slots, RU, D]
  float* ws_lse;  // [slots, RU]
  bf16* o;        // [B, Sq, Hq, D]
  float* lse;     // [B, Hq, Sq]
  int B, Sq, Smax, Hq, Hkv, W;
  int RB, RU;     // row blocks per kv head; partial rows per slot (R if RB = 1, else 32)
  float scale;
  int rope;       // 1: query t is rotated at position L - Sq + t before use
  RopeFreq rf;
  Strides sq, skv, so;  // q; the k and v caches; o
};

// Valid 64-key tiles of each unit of sequence b.
__device__ __forceinline__ int dec_tiles(const DecArgs& a, int b) {
  return (valid_len(a.lens, b, a.Smax) + 63) >> 6;
}

// First tile of wave w (wave w owns [dec_start(w), dec_start(w + 1))).
__device__ __forceinline__ int dec_start(int w, int T, int W) {
  return (int)(((int64_t)w * T) / W);
}

__device__ __forceinline__ int wave_sum_i(int x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

__device__ __forceinline__ int wave_scan_incl_i(int x, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  return x;
}

// One unit's share of a wave: local tiles [s0, s1) of unit (b, hkv, rb),
// partial result to slot `slot`.
template <int D, int STAGES>
__device__ __forceinline__ void decode_segment(const DecArgs& a, int b, int hkv, int rb, int s0, int s1,
                                               int64_t slot, bf16* sK0, bf16* sV0, bf16* sK1, bf16* sV1,
                                               int lane) {
  constexpr int BN = 64;
  constexpr int KK = D / 16;
  constexpr int DT = D / 32;
  const int g = lane >> 5;
  const int G = a.Hq / a.Hkv;
  const int R = G * a.Sq;
  const int L = valid_len(a.lens, b, a.Smax);
  const int64_t ks = a.skv.s;
  const bf16* Kb = a.k + b * a.skv.b + hkv * a.skv.h;
  const bf16* Vb = a.v + b * a.skv.b + hkv * a.skv.h;

  // the lane's query row rr = 32*rb + r: head hkv*G + rr / Sq, new query
  // t = rr % Sq at cache position L - Sq + t, which sees keys 0 .. L - Sq + t
  const int r = lane & 31;
  const int rr = rb * 32 + r;
  const bool row_ok = rr < R;
  const int hh = row_ok ? rr / a.Sq : 0;
  const int t = row_ok ? rr - hh * a.Sq : 0;
  const int h = hkv * G + hh;
  const int jmax = row_ok ? L - a.Sq + t : -1;  // last visible key (< 0: none)

  FwdState<D, 1> st;
  const bf16* qrow = a.q + b * a.sq.b + t * a.sq.s + h * a.sq.h;
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) {
    bf16x8 qv = row_ok ? *reinterpret_cast<const bf16x8*>(qrow + kk * 16 + g * 8) : zero_bf16x8();
    if (a.rope) {
      // pairs kk*8 + 4g + e of the lane's 8 elements, rotated at the query's
      // position in fp32 and rounded to bf16: the fragment is a bf16 MFMA
      // operand (the training path stores its rotated queries in bf16 too)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float cs, sn;
        rope_cos_sin(g ? a.rf.phi[kk * 8 + 4 + e] : a.rf.phi[kk * 8 + e], L - a.Sq + t, cs, sn);
        const float x0 = (float)qv[2 * e], x1 = (float)qv[2 * e + 1];
        qv[2 * e] = (bf16)(x0 * cs - x1 * sn);
        qv[2 * e + 1] = (bf16)(x0 * sn + x1 * cs);
      }
    }
    st.qf[0][kk] = qv;
  }
  st.mu[0] = kNegInf;
  st.lsum[0] = 0.f;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) st.oacc[dt][0] = zero16();
  wait_vmem();

  const float c = a.scale * kLog2e;
  const int k0 = s0 * BN;                   // the segment's first key
  const int kend = min(s1 * BN, L);         // and one past its last
  const int ntiles = s1 - s0;
  const int first_last = L - a.Sq;          // smallest last-visible key of the rows
  const KVBuf b0{sK0, sV0, 0}, b1{sK1, sV1, 1};
  auto fetch = [&](int kt, const KVBuf& buf) {
    tile_load_lds<BN, D, 1>(Kb, ks, k0 + kt * BN, kend, buf.k, 0, lane);
    tile_load_lds<BN, D, 1>(Vb, ks, k0 + kt * BN, kend, buf.v, 0, lane);
  };
  auto compute = [&](int kt, const KVBuf& buf) {
    const int j0 = k0 + kt * BN;
    if (j0 + BN - 1 > first_last || j0 + BN > kend) {
      const int lim[1] = {min(jmax, kend - 1) - j0 - g * 4};
      fwd_tile<D, 1, true>(st, buf.k, buf.v, lane, c, lim);
    } else {
      const int lim[1] = {};
      fwd_tile<D, 1, false>(st, buf.k, buf.v, lane, c, lim);
    }
  };
  if constexpr (STAGES == 2) {
    tile_pipeline(ntiles, b0, b1, fetch, [](int, const KVBuf&) {}, compute);
  } else {
    // one stage: the wave waits for each tile; the other waves on the SIMD
    // (twice as many fit in LDS) keep HBM busy meanwhile
    for (int kt = 0; kt < ntiles; ++kt) {
      fetch(kt, b0);
      wait_vmem();
      __syncthreads();
      compute(kt, b0);
      __syncthreads();
    }
  }

  // partial result: O / l (fp32) and LSE = mu*scale + ln l
  const float lt = xhalf_sum(st.lsum[0]);
  if (row_ok) {
    const int64_t prow = slot * a.RU + r;
    const bool any = lt > 0.f;
    const float inv = any ? 1.f / lt : 0.f;
    float* wo = a.ws_o + prow * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        float4 ov;
        ov.x = st.oacc[dt][0][rr * 4 + 0] * inv;
        ov.y = st.oacc[dt][0][rr * 4 + 1] * inv;
        ov.z = st.oacc[dt][0][rr * 4 + 2] * inv;
        ov.w = st.oacc[dt][0][rr * 4 + 3] * inv;
        *reinterpret_cast<float4*>(wo + dt * 32 + rr * 8 + g * 4) = ov;
      }
    if (g == 0) a.ws_lse[prow] = any ? (st.mu[0] * c + __log2f(lt)) * kLn2 : kNegInf;
  }
}

template <int D, int OCC, int STAGES>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(OCC, OCC)))
void decode_split_kernel(DecArgs a) {
  constexpr int KVT = TileLayout<D>::template elems<64>();
  __shared__ __attribute__((aligned(16))) bf16 sK0[KVT], sV0[KVT];
  __shared__ __attribute__((aligned(16))) bf16 sK1[STAGES == 2 ? KVT : 8], sV1[STAGES == 2 ? KVT : 8];
  const int lane = threadIdx.x;
  const int w = blockIdx.x;

  const int HU = a.Hkv * a.RB;  // units per sequence
  // T: valid tiles over all units (every wave counts them; wave 0 publishes)
  int part = 0;
  for (int b = lane; b < a.B; b += 64) part += dec_tiles(a, b) * HU;
  const int T = wave_sum_i(part);
  if (w == 0 && lane == 0) a.hdr[0] = T;
  int tb = dec_start(w, T, a.W);
  const int te = dec_start(w + 1, T, a.W);
  if (tb >= te) return;

  // the sequence holding tile tb: the first whose inclusive tile prefix exceeds it
  int b = -1, before = 0;  // before: tiles of the sequences ahead of b
  for (int base = 0; base < a.B; base += 64) {
    const int x = base + lane < a.B ? dec_tiles(a, base + lane) * HU : 0;
    const int incl = wave_scan_incl_i(x, lane) + before;
    const uint64_t hit = __ballot(incl > tb);
    if (hit) {
      const int f = __builtin_ctzll(hit);
      b = base + f;
      before = __shfl(incl - x, f, 64);
      break;
    }
    before = __shfl(incl, 63, 64);
  }
  if (b < 0) return;  // unreachable while tb < T

  int nt = dec_tiles(a, b);  // > 0: sequence b holds tile tb
  int hu = (tb - before) / nt;  // unit of the sequence: kv head hu / RB, row block hu % RB
  int ustart = before + hu * nt;
  for (;;) {
    const int64_t u = (int64_t)b * HU + hu;
    const int s0 = tb - ustart;
    const int s1 = min(te, ustart + nt) - ustart;
    decode_segment<D, STAGES>(a, b, hu / a.RB, hu % a.RB, s0, s1, w + u, sK0, sV0, sK1, sV1, lane);
    if (lane == 0) {
      if (s0 == 0) a.uinfo[u].x = w;
      if (s1 == nt) a.uinfo[u].y = w;
    }
    tb = ustart + s1;
    if (tb >= te) break;
    ustart += nt;
    if (++hu == HU) {  // next sequence with a non-empty cache
      hu = 0;
      do {
        ++b;
      } while (b < a.B && (nt = dec_tiles(a, b)) == 0);
      if (b >= a.B) break;  // unreachable while tb < T
    }
  }
}

// Merge: one wave per (sequence, head, new query); LSE = ln sum_s exp(LSE_s),
// O = sum_s exp(LSE_s - LSE) O_s over the unit's partials, rounded to bf16.
// The weights are computed with lanes over partials, the sum with lanes over
// d (eight partials' loads in flight at a time). A sequence with an empty
// cache has no partials: O = 0, LSE = -inf.
template <int D>
__global__ __launch_bounds__(kThreads) void decode_merge_kernel(DecArgs a) {
  constexpr int PER = D / 64;  // elements per lane
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);  // (b * Hq + h) * Sq + t
  const int64_t rows = (int64_t)a.B * a.Hq * a.Sq;
  if (row >= rows) return;
  const int t = (int)(row % a.Sq);
  const int64_t bh = row / a.Sq;
  const int h = (int)(bh % a.Hq);
  const int b = (int)(bh / a.Hq);
  const int G = a.Hq / a.Hkv;
  const int hkv = h / G;
  const int rr = (h - hkv * G) * a.Sq + t;  // row within the kv head's rows
  const int r = rr & 31;
  const int64_t u = ((int64_t)b * a.Hkv + hkv) * a.RB + (rr >> 5);
  const int R = a.RU;  // partial rows per slot
  float m = kNegInf;
  float acc[PER] = {};
  float den = 0.f;
  if (dec_tiles(a, b) > 0) {
    const int T = a.hdr[0];
    const int2 ui = a.uinfo[u];
    const int n = ui.y - ui.x + 1;
    // waves between the first and the last that own no tile wrote nothing
    auto has = [&](int i) {
      const int w = ui.x + i;
      return i < n && dec_start(w, T, a.W) < dec_start(w + 1, T, a.W);
    };
    for (int i0 = 0; i0 < n; i0 += 64)
      if (has(i0 + lane)) m = fmaxf(m, a.ws_lse[(ui.x + i0 + lane + u) * R + r]);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
    if (m != kNegInf) {
      for (int i0 = 0; i0 < n; i0 += 64) {
        const float wt = has(i0 + lane) ? __expf(a.ws_lse[(ui.x + i0 + lane + u) * R + r] - m) : 0.f;
        den += wt;  // 0 for a partial that saw no key
        const int cnt = min(64, n - i0);
        for (int j = 0; j < cnt; j += 8) {
          float x[8][PER], wj[8];
#pragma unroll
          for (int jj = 0; jj < 8; ++jj) {
            const int jx = j + jj < cnt ? j + jj : 0;
            wj[jj] = j + jj < cnt ? __shfl(wt, jx, 64) : 0.f;
            const float* wo = a.ws_o + ((ui.x + i0 + jx + u) * R + r) * D;
#pragma unroll
            for (int e = 0; e < PER; ++e) x[jj][e] = wo[e * 64 + lane];
          }
#pragma unroll
          for (int jj = 0; jj < 8; ++jj)
#pragma unroll
            for (int e = 0; e < PER; ++e) acc[e] += wj[jj] > 0.f ? wj[jj] * x[jj][e] : 0.f;
        }
      }
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) den += __shfl_xor(den, o, 64);
    }
  }
  bf16* orow = a.o + b * a.so.b + t * a.so.s + h * a.so.h;
  const float inv = den > 0.f ? 1.f / den : 0.f;
#pragma unroll
  for (int e = 0; e < PER; ++e) orow[e * 64 + lane] = (bf16)(acc[e] * inv);
  if (lane == 0) a.lse[bh * a.Sq + t] = den > 0.f ? m + __logf(den) : kNegInf;
}

namespace {

// Per head dimension: 32-row tiles per wave (NT: query rows in the forward and
// dQ passes; the dK/dV pass always gives each wave 32 key rows), waves per
// SIMD (OCC: the register budget per wave is 512 / OCC) and waves per
// workgroup of the forward and dQ passes (W: the waves of a workgroup share
// each K/V tile loaded into LDS). The *_SMALL configurations (64-row query
// blocks) are used when the default blocks would leave CUs without work.
template <int D> struct Tiles;
template <> struct Tiles<64> {
  static constexpr int FWD_NT = 2, FWD_OCC = 2, FWD_W = 4;   // 256-row blocks
  static constexpr int DQ_NT = 1, DQ_OCC = 3, DQ_W = 4;      // 128-row blocks
  static constexpr int DKDV_NTJ = 1, DKDV_OCC = 2, DKDV_GROUPS = 2;
};
template <> struct Tiles<128> {
  static constexpr int FWD_NT = 1, FWD_OCC = 2, FWD_W = 8;   // 256-row blocks
  static constexpr int DQ_NT = 1, DQ_OCC = 2, DQ_W = 4;      // 128-row blocks
  static constexpr int DKDV_NTJ = 1, DKDV_OCC = 1, DKDV_GROUPS = 1;
};
// Small-grid configurations (forward and dQ): 64-row blocks of four waves
// whose two halves take alternate 64-key tiles of each 128-key pipeline step.
// (Four key groups of two waves each at d=64 shorten the longest block's chain
// but need 144 KB of LDS, one block per CU, and measured slower.)
// Two waves per SIMD (two blocks per CU), so at most 256 registers per wave.
struct Small { static constexpr int NT = 1, W = 4, KS = 2, OCC = 2; };

inline int cdiv(int a, int b) { return (a + b - 1) / b; }

// phi_i = base^(-2i/d) / (2 pi) in fp64; zeros when base is 0 (no rotation)
RopeFreq rope_freq_d(float base, int d) {
  RopeFreq rf{};
  if (base > 0.f)
    for (int i = 0; i < d / 2; ++i) rf.phi[i] = std::pow((double)base, -2.0 * i / d) / (2.0 * 3.14159265358979323846);
  return rf;
}

template <typename Args>
hipError_t launch(const void* fn, int64_t grid, Args args, hipStream_t stream, int threads = kThreads) {
  if (grid <= 0) return hipSuccess;
  void* kargs[] = {&args};
  return hipLaunchKernel(fn, dim3((unsigned)grid), dim3(threads), kargs, 0, stream);
}

// phi_i = base^(-2i/d) / (2 pi), in fp64 (zeros when RoPE is off)
RopeFreq rope_freq(const Problem& pr) { return rope_freq_d(pr.rope_base, pr.d); }

// Workgroups that fill the chip once: 256 CUs, each holding this many
// workgroups of the default forward / dQ configuration at once.
constexpr int64_t kCUs = 256;

template <int D>
hipError_t fwd_d(const Problem& pr, const void* q, const void* k, const void* v, void* o, float* lse,
                 hipStream_t stream) {
  constexpr int NT = Tiles<D>::FWD_NT, W = Tiles<D>::FWD_W, OCC = Tiles<D>::FWD_OCC;
  FwdArgs a{(const bf16*)q, (const bf16*)k, (const bf16*)v, (bf16*)o, lse, pr.seqlens,
            pr.B, pr.S, pr.Hq, pr.Hkv, cdiv(pr.S, 32 * NT * W), pr.scale, pr.causal, pr.sq, pr.skv, pr.so};
  const int64_t wgs = (int64_t)a.nqb * pr.B * pr.Hq;
  if (wgs >= kCUs * (4 * OCC / W))
    return launch((const void*)&fwd_kernel<D, NT, OCC, W>, wgs, a, stream, 64 * W);
  a.nqb = cdiv(pr.S, 32 * Small::NT * (Small::W / Small::KS));
  return launch((const void*)&fwd_kernel<D, Small::NT, Small::OCC, Small::W, Small::KS>, (int64_t)a.nqb * pr.B * pr.Hq, a,
                stream, 64 * Small::W);
}

template <int D>
hipError_t pre_d(const Problem& pr, const void* o, const void* d_o, float* delta, hipStream_t stream) {
  PreArgs a{(const bf16*)o, (const bf16*)d_o, delta, pr.seqlens, pr.B, pr.S, pr.Hq,
            (int64_t)pr.B * pr.S * pr.Hq, pr.so};
  constexpr int rows_per_block = kThreads / (D / 8);
  return launch((const void*)&preprocess_kernel<D>, (a.rows + rows_per_block - 1) / rows_per_block, a, stream);
}

template <int D>
hipError_t dkdv_d(const Problem& pr, const void* q, const void* k, const void* v, const void* d_o,
                  const float* lse, const float* delta, void* dk, void* dv, void* workspace, hipStream_t stream) {
  constexpr int NTJ = Tiles<D>::DKDV_NTJ;
  const int parts = dkdv_parts(pr);
  static_assert(128 * NTJ == 128, "the split's deal and the reduce pass assume 128-key blocks");
  const size_t part_elems = (size_t)pr.B * pr.S * pr.Hkv * D * dkdv_max_parts(pr);
  float* part_dk = parts > 1 ? reinterpret_cast<float*>(workspace) : nullptr;
  float* part_dv = parts > 1 ? part_dk + part_elems : nullptr;
  BwdArgs a{(const bf16*)q, (const bf16*)k, (const bf16*)v, (const bf16*)d_o, lse, delta,
            nullptr, (bf16*)dk, (bf16*)dv, pr.seqlens, pr.B, pr.S, pr.Hq, pr.Hkv,
            cdiv(pr.S, 128 * NTJ), pr.scale, pr.causal, pr.rope_base > 0.f, rope_freq(pr), pr.sq, pr.skv, pr.so,
            nullptr, nullptr, parts, part_dk, part_dv};
  constexpr int GR = Tiles<D>::DKDV_GROUPS;
  hipError_t e;
  if constexpr (D == 128)
    e = launch((const void*)&bwd_dkdv_roles_kernel<D>, (int64_t)a.nblk * parts * pr.B * pr.Hkv, a, stream, 8 * 64);
  else
    e = launch((const void*)&bwd_dkdv_kernel<D, NTJ, Tiles<D>::DKDV_OCC, GR>, (int64_t)a.nblk * parts * pr.B * pr.Hkv,
               a, stream, kThreads * GR);
  if (e != hipSuccess || parts == 1) return e;
  const int64_t threads = (int64_t)pr.B * pr.S * pr.Hkv * (D / 4);
  return launch((const void*)&dkdv_reduce_kernel<D>, (threads + kThreads - 1) / kThreads, a, stream);
}

template <int D>
hipError_t dq_d(const Problem& pr, const void* q, const void* k, const void* v, const void* d_o,
                const float* lse, const float* delta, void* dq, const void* o, float* delta_out,
                hipStream_t stream) {
  constexpr int NT = Tiles<D>::DQ_NT, W = Tiles<D>::DQ_W, OCC = Tiles<D>::DQ_OCC;
  BwdArgs a{(const bf16*)q, (const bf16*)k, (const bf16*)v, (const bf16*)d_o, lse, delta,
            (bf16*)dq, nullptr, nullptr, pr.seqlens, pr.B, pr.S, pr.Hq, pr.Hkv,
            cdiv(pr.S, 32 * NT * W), pr.scale, pr.causal, pr.rope_base > 0.f, rope_freq(pr), pr.sq, pr.skv, pr.so,
            (const bf16*)o, delta_out, 1, nullptr, nullptr};
  const int64_t wgs = (int64_t)a.nblk * pr.B * pr.Hq;
  if (wgs >= kCUs * (4 * OCC / W))
    return launch((const void*)&bwd_dq_kernel<D, NT, OCC, W>, wgs, a, stream, 64 * W);
  a.nblk = cdiv(pr.S, 32 * Small::NT * (Small::W / Small::KS));
  return launch((const void*)&bwd_dq_kernel<D, Small::NT, Small::OCC, Small::W, Small::KS>, (int64_t)a.nblk * pr.B * pr.Hq,
                a, stream, 64 * Small::W);
}

template <int D>
hipError_t rope_d(const Problem& pr, const void* q, const void* k, void* qr, void* kr, hipStream_t stream) {
  RopeArgs a{(const bf16*)q, (const bf16*)k, (bf16*)qr, (bf16*)kr, pr.S, pr.Hq, pr.Hkv, rope_freq(pr), pr.sq, pr.skv};
  return launch((const void*)&rope_kernel<D>, (int64_t)pr.B * pr.S, a, stream, 64);
}

}  // namespace

hipError_t launch_rope(const Problem& pr, const void* q, const void* k, void* q_rot, void* k_rot,
                       hipStream_t stream) {
  return pr.d == 64 ? rope_d<64>(pr, q, k, q_rot, k_rot, stream) : rope_d<128>(pr, q, k, q_rot, k_rot, stream);
}

hipError_t launch_fwd(const Problem& pr, const void* q, const void* k, const void* v, void* o, float* lse,
                      hipStream_t stream) {
  return pr.d == 64 ? fwd_d<64>(pr, q, k, v, o, lse, stream) : fwd_d<128>(pr, q, k, v, o, lse, stream);
}

hipError_t launch_preprocess(const Problem& pr, const void* o, const void* d_o, float* delta, hipStream_t stream) {
  return pr.d == 64 ? pre_d<64>(pr, o, d_o, delta, stream) : pre_d<128>(pr, o, d_o, delta, stream);
}

hipError_t launch_bwd_dkdv(const Problem& pr, const void* q, const void* k, const void* v, const void* d_o,
                           const float* lse, const float* delta, void* dk, void* dv, void* workspace,
                           hipStream_t stream) {
  return pr.d == 64 ? dkdv_d<64>(pr, q, k, v, d_o, lse, delta, dk, dv, workspace, stream)
                    : dkdv_d<128>(pr, q, k, v, d_o, lse, delta, dk, dv, workspace, stream);
}

hipError_t launch_bwd_dq(const Problem& pr, const void* q, const void* k, const void* v, const void* d_o,
                         const float* lse, const float* delta, void* dq, hipStream_t stream) {
  return pr.d == 64 ? dq_d<64>(pr, q, k, v, d_o, lse, delta, dq, nullptr, nullptr, stream)
                    : dq_d<128>(pr, q, k, v, d_o, lse, delta, dq, nullptr, nullptr, stream);
}

hipError_t launch_bwd_dq_with_delta(const Problem& pr, const void* q, const void* k, const void* v,
                                    const void* o, const void* d_o, const float* lse, float* delta, void* dq,
                                    hipStream_t stream) {
  return pr.d == 64 ? dq_d<64>(pr, q, k, v, d_o, lse, nullptr, dq, o, delta, stream)
                    : dq_d<128>(pr, q, k, v, d_o, lse, nullptr, dq, o, delta, stream);
}


// Scratch of the allocation-free decode entry point: one copy per GPU, alive
// until the process ends. Host code never passes `scratch` itself to a kernel
// (on the host it names a stand-in, not device memory): it uses the address
// hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) unsigned char scratch[kDecodeScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t decode_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t launch_decode(const DecodeProblem& pr, const DecodePlan& plan, const void* q, const void* k_cache,
                         const void* v_cache, void* o, float* lse, void* workspace, hipStream_t stream) {
  char* ws = reinterpret_cast<char*>(workspace);
  DecArgs a{(const bf16*)q, (const bf16*)k_cache, (const bf16*)v_cache, pr.cache_lens,
            reinterpret_cast<int*>(ws), reinterpret_cast<int2*>(ws + plan.off_uinfo),
            reinterpret_cast<float*>(ws + plan.off_o), reinterpret_cast<float*>(ws + plan.off_lse),
            (bf16*)o, lse, pr.B, pr.Sq, pr.Smax, pr.Hq, pr.Hkv, plan.waves, plan.rb, plan.ru, pr.scale,
            pr.rope_base > 0.f, rope_freq_d(pr.rope_base, pr.d), pr.sq, pr.skv, pr.so};
  const int64_t merge_blocks = ((int64_t)pr.B * pr.Hq * pr.Sq + 3) / 4;
  hipError_t e;
  if (pr.d == 64) {
    e = launch((const void*)&decode_split_kernel<64, 2, kDecodeStages>, plan.waves, a, stream, 64);
    if (e == hipSuccess) e = launch((const void*)&decode_merge_kernel<64>, merge_blocks, a, stream);
  } else {
    e = launch((const void*)&decode_split_kernel<128, 1, kDecodeStages>, plan.waves, a, stream, 64);
    if (e == hipSuccess) e = launch((const void*)&decode_merge_kernel<128>, merge_blocks, a, stream);
  }
  return e;
}

}  // namespace attn
