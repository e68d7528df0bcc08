// Pieces shared by the Lizard attention forward kernels: LDS geometry, chunk
// staging, the triangular MFMA operands of the in-sub-chunk gate sums, and the
// feature-map products.  The method and the decay bookkeeping are described
// at the top of fwd.hip.
#pragma once
#include "common.hpp"
#include "internal.hpp"

namespace lz {

constexpr int CH = 64;            // chunk length
constexpr float SPAN_MAX = 80.f;  // max |log-decay| across one 16-token sub-chunk for the
                                  // mid-reference MFMA path (e^80 ~ 5.5e34 < fp32/bf16 max)
constexpr float NEG_BIG = -1.0e30f;
constexpr float FAST_SPAN = 60.f; // max |log-decay| across a whole chunk for the chunk-start
                                  // reference (keys carry e^{+60} at most, queries e^{-60})
// The state pass and the self-started walk drop the chunks that reach their segment's end decayed
// below e^{-SKIP_LOG} in every feature.  With features in (0, 1] a dropped token's term is below
// e^{-16} ~ 1.1e-7 of the largest term a token can add to the same feature row, and the chunks
// further back decay geometrically, so what is dropped stays about four orders of magnitude below
// bf16 rounding of the output (e^{-40}, then e^{-24}, made the second segment's walk longer: 5%
// and 2% of the forward on the Llama-3-8B-shaped layer, for no change the output can hold).
constexpr float SKIP_LOG = 16.f;
// The same cutoff for a feature map whose values are not bounded by one: the Hedgehog map's
// features lie in [e^{-LOGIT_MAX}, e^{LOGIT_MAX}] under its documented logit bound, so a chunk is
// dropped only once its largest possible term, decayed, is below e^{-SKIP_LOG} times the smallest
// possible term of the same feature row: suffix < -(SKIP_LOG + 2 LOGIT_MAX).
constexpr float HH_LOGIT_MAX = 80.f;
template <bool HH> __host__ __device__ constexpr float skip_log() {
  return HH ? SKIP_LOG + 2.f * HH_LOGIT_MAX : SKIP_LOG;
}
constexpr int LDS_LIMIT = 160 * 1024;
constexpr int WIN_BATCH = 8;      // key tiles per online-softmax batch in the window
constexpr int KT_META = -(1 << 28);  // window tile list: the meta tile
constexpr int KT_NONE = -(1 << 29);  // window tile list: no tile

// a mod m in [0, m) for negative a too (chunk indices of the window history are < 0)
__device__ __forceinline__ int pmod(int a, int m) {
  const int r = a % m;
  return r < 0 ? r + m : r;
}

// Row strides.  gfx950 serves 16-byte LDS reads of an MFMA fragment (16 rows x 4
// column groups) without bank conflicts when the row stride is an odd multiple of
// 32 bytes, and 8-byte reads when it is an odd multiple of 16 bytes (measured).
// Rows read 16 bytes at a time (W^T, keys, meta keys, log gamma^T) take the wide
// stride when the layout fits (WIDE), rows read 8 bytes at a time the narrow one.
template <typename T, int D, int DV, bool WIDE> struct FwdGeom {
  static constexpr int PADE = 16 / (int)sizeof(T);            // 16 bytes
  static constexpr int PADW = (WIDE ? 32 : 16) / (int)sizeof(T);
  static constexpr int LDW = D + PADW;   // rows of D elements, 16-byte reads
  static constexpr int LDB = D + PADE;   // rows of D elements, 8-byte reads
  static constexpr int LDC = CH + PADE;  // rows of 64 tokens, 8-byte reads
  static constexpr int LDG = CH + PADW;  // rows of 64 tokens, 16-byte reads
  static constexpr int LDM = 16 + PADE;  // rows of 16 meta tokens
  static constexpr int SZ_W = D * LDW * (int)sizeof(T);
  static constexpr int SZ_VT = DV * LDC * (int)sizeof(T);
  static constexpr int SZ_KR = CH * LDW * (int)sizeof(T);
  // keys decayed to their sub-chunk end [s][f], overlaid on log gamma^T [f][s]
  static constexpr int SZ_KOWN = (CH * LDB > D * LDG ? CH * LDB : D * LDG) * (int)sizeof(T);
  static constexpr int SZ_SUB = 4 * D * (int)sizeof(float);  // one [4][D] fp32 table
  static constexpr int SZ_SBF = DV * LDB * (int)sizeof(T);
  static constexpr int SZ_TVT = DV * LDM * (int)sizeof(T);
  static constexpr int SZ_TK = 16 * LDW * (int)sizeof(T);
};

// Byte offsets of the LDS regions for one launch (computed on the host).
template <typename T, int D, int DV, bool WIDE>
static FwdLds make_lds(bool state_only, bool shared_w, int nr, int kr) {
  using Gm = FwdGeom<T, D, DV, WIDE>;
  FwdLds l{};
  int o = 0;
  l.wk = o; o += Gm::SZ_W;
  l.wq = (state_only || shared_w) ? l.wk : o;
  if (!(state_only || shared_w)) o += Gm::SZ_W;
  l.vt = o; o += nr * Gm::SZ_VT;
  l.kr = o; o += kr * Gm::SZ_KR;
  l.kown = o; o += Gm::SZ_KOWN;
  l.tot = o; o += Gm::SZ_SUB;   // tot_J[f]
  l.p7 = o; o += Gm::SZ_SUB;    // p7_J[f]
  l.etot = o; o += Gm::SZ_SUB;  // e^{tot_J}
  if (!state_only) {
    l.enp7 = o; o += Gm::SZ_SUB;  // e^{-p7_J}
    l.enr8 = o; o += Gm::SZ_SUB;  // e^{p7_J - tot_J}
    l.sbf = o; o += Gm::SZ_SBF;
    l.tvt = o; o += Gm::SZ_TVT;
    l.tk = o; o += Gm::SZ_TK;
  }
  l.total = o;
  return l;
}

// W_phi [d][f] row-major in global -> W^T [f][d] in LDS (row stride LDW).
template <typename T, int D, int LDW, int NT = 256>
__device__ __forceinline__ void load_wT(T *dst, const T *src, int tid) {
  for (int idx = tid; idx < D * (D / 8); idx += NT) {
    const int dd = idx / (D / 8), f0 = (idx % (D / 8)) * 8;
    float x[8];
    load8f(src + (size_t)dd * D + f0, x);
#pragma unroll
    for (int j = 0; j < 8; ++j) dst[(f0 + j) * LDW + dd] = from_f<T>(x[j]);
  }
}

// Per-thread share of one chunk: keys (row-major), values and log gamma
// (both stored transposed, token pairs 2*tp, 2*tp+1 x 8 columns).  The 32
// token pairs of one 8-column group sit in one half-wave, so the transposed
// 4-byte stores of a wave cover all 64 LDS banks.
template <typename T, int D, int DV> struct ChunkRegs {
  static constexpr int KFR = CH * D / 8 / 256;      // 8-element pieces of k per thread
  static constexpr int LFR = (CH / 2) * (D / 8) / 256;  // token-pair pieces of log gamma
  Frag<T> k[KFR];
  Frag<T> v[2];
  Frag<T> lg[LFR][2];
};

template <typename T, int D, int DV>
__device__ __forceinline__ void load_chunk(ChunkRegs<T, D, DV> &r, const T *Kh, const T *Vh, const T *LGh,
                                           int c0, int L, int dv0, bool with_v, int tid) {
  static_assert(DV == 64, "value block of 64 columns");
#pragma unroll
  for (int j = 0; j < ChunkRegs<T, D, DV>::KFR; ++j) {
    const int idx = tid + 256 * j;
    const int row = idx / (D / 8), c8 = idx % (D / 8);
    r.k[j] = (c0 + row < L) ? load8(Kh + (size_t)(c0 + row) * D + 8 * c8) : frag_zero<T>();
  }
  if (with_v) {
    const int dq = tid / 32, tp = tid % 32;  // one 8-column group per half-wave: conflict-free stores
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int t = c0 + 2 * tp + h;
      r.v[h] = (t < L) ? load8(Vh + (size_t)t * D + dv0 + 8 * dq) : frag_zero<T>();
    }
  }
#pragma unroll
  for (int j = 0; j < ChunkRegs<T, D, DV>::LFR; ++j) {
    const int idx = tid + 256 * j;
    const int fq = idx / 32, tp = idx % 32;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int t = c0 + 2 * tp + h;
      r.lg[j][h] = (t < L) ? load8(LGh + (size_t)t * D + 8 * fq) : frag_zero<T>();
    }
  }
}

template <typename T, int D, int DV, int LDW>
__device__ __forceinline__ void store_keys(const ChunkRegs<T, D, DV> &r, T *sK, int tid) {
#pragma unroll
  for (int j = 0; j < ChunkRegs<T, D, DV>::KFR; ++j) {
    const int idx = tid + 256 * j;
    const int row = idx / (D / 8), c8 = idx % (D / 8);
    T *dst = sK + row * LDW + 8 * c8;
    if constexpr (sizeof(T) == 2) {
      *reinterpret_cast<bf16x8 *>(dst) = r.k[j].v;
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) dst[e] = r.k[j].v[e];
    }
  }
}

// Two tokens x 8 columns -> transposed [col][token] (token pair adjacent).
template <typename T, int LDC>
__device__ __forceinline__ void store_pairT(const Frag<T> &a, const Frag<T> &b, T *dst) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    T *d = dst + e * LDC;
    if constexpr (sizeof(T) == 2) {
      bf16 pair[2] = {a.v[e], b.v[e]};
      *reinterpret_cast<uint32_t *>(d) = *reinterpret_cast<const uint32_t *>(pair);
    } else {
      d[0] = a.v[e];
      d[1] = b.v[e];
    }
  }
}

template <typename T, int D, int DV, int LDC>
__device__ __forceinline__ void store_values(const ChunkRegs<T, D, DV> &r, T *sVt, int tid) {
  const int dq = tid / 32, tp = tid % 32;
  store_pairT<T, LDC>(r.v[0], r.v[1], sVt + (8 * dq) * LDC + 2 * tp);
}

// The value share of load_chunk / store_values on its own (same thread mapping).
template <typename T, int D, int DV>
__device__ __forceinline__ void load_values(Frag<T> (&v)[2], const T *Vh, int c0, int L, int dv0, int tid) {
  const int dq = tid / 32, tp = tid % 32;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int t = c0 + 2 * tp + h;
    v[h] = (t < L) ? load8(Vh + (size_t)t * D + dv0 + 8 * dq) : frag_zero<T>();
  }
}
template <typename T, int LDC>
__device__ __forceinline__ void store_values2(const Frag<T> (&v)[2], T *sVt, int tid) {
  const int dq = tid / 32, tp = tid % 32;
  store_pairT<T, LDC>(v[0], v[1], sVt + (8 * dq) * LDC + 2 * tp);
}

template <typename T, int D, int DV, int LDC>
__device__ __forceinline__ void store_lgT(const ChunkRegs<T, D, DV> &r, T *sLgT, int tid) {
#pragma unroll
  for (int j = 0; j < ChunkRegs<T, D, DV>::LFR; ++j) {
    const int idx = tid + 256 * j;
    const int fq = idx / 32, tp = idx % 32;
    store_pairT<T, LDC>(r.lg[j][0], r.lg[j][1], sLgT + (8 * fq) * LDC + 2 * tp);
  }
}

// Constant B operand of the prefix / exclusive-suffix sums over the 16 rows of
// a sub-chunk: lane (t = r16, kq) holds B[s = 8kq + j][t].
template <typename T>
__device__ __forceinline__ Frag<T> tri_frag(int r16, int g4, bool prefix) {
  float x[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int s = 8 * g4 + j;
    x[j] = (s < 16 && (prefix ? (s <= r16) : (s > r16))) ? 1.f : 0.f;
  }
  return frag_from<T>(x);
}

// Constant B operand of the inclusive prefix over the whole chunk for the rows of
// sub-chunk I: K-step ks covers chunk rows s = 32 ks + 8 kq + j, and lane
// (t = r16, kq) holds B[s][t] = (s <= 16 I + t).
template <typename T>
__device__ __forceinline__ Frag<T> tri64_frag(int r16, int g4, int I, int ks) {
  float x[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) x[j] = (32 * ks + 8 * g4 + j <= 16 * I + r16) ? 1.f : 0.f;
  return frag_from<T>(x);
}

// 8 fp32 table values for the operand slots of K-step js (features
// 32js + 4g4 + 0..3 and 32js + 16 + 4g4 + 0..3).
__device__ __forceinline__ void tab8(const float *row, int js, int g4, float (&x)[8]) {
  const f32x4 a = *reinterpret_cast<const f32x4 *>(row + 32 * js + 4 * g4);
  const f32x4 b = *reinterpret_cast<const f32x4 *>(row + 32 * js + 16 + 4 * g4);
#pragma unroll
  for (int i = 0; i < 4; ++i) { x[i] = a[i]; x[4 + i] = b[i]; }
}

template <int NFT>
__device__ __forceinline__ void softmax_rows(const f32x4 (&z)[NFT], float (&phi)[NFT][4]) {
  float zm = NEG_BIG;
#pragma unroll
  for (int ft = 0; ft < NFT; ++ft)
#pragma unroll
    for (int i = 0; i < 4; ++i) zm = fmaxf(zm, z[ft][i]);
  zm = wave_max_cols(zm);
  const float zm2 = -zm * LOG2E;
  float zs = 0.f;
#pragma unroll
  for (int ft = 0; ft < NFT; ++ft)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      phi[ft][i] = exp2_fast(__builtin_fmaf(z[ft][i], LOG2E, zm2));
      zs += phi[ft][i];
    }
  zs = wave_sum_cols(zs);
  const float inv = 1.f / zs;
#pragma unroll
  for (int ft = 0; ft < NFT; ++ft)
#pragma unroll
    for (int i = 0; i < 4; ++i) phi[ft][i] *= inv;
}

// z^T[f][t] = sum_d W[d][f] x[t][d] for the wave's 16 rows (W^T in LDS).
template <typename T, int D, int LDW>
__device__ __forceinline__ void feature_logits(const T *sW, const Frag<T> (&xf)[D / 32], int r16, int g4,
                                               f32x4 (&z)[D / 16]) {
#pragma unroll
  for (int ft = 0; ft < D / 16; ++ft) {
    z[ft] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < D / 32; ++j) z[ft] = mma(load8(sW + (16 * ft + r16) * LDW + 32 * j + 8 * g4), xf[j], z[ft]);
  }
}

// Same for two inputs against one W (each W fragment read once, two MFMA chains).
template <typename T, int D, int LDW>
__device__ __forceinline__ void feature_logits2(const T *sW, const Frag<T> (&xa)[D / 32], const Frag<T> (&xb)[D / 32],
                                                int r16, int g4, f32x4 (&za)[D / 16], f32x4 (&zb)[D / 16]) {
#pragma unroll
  for (int ft = 0; ft < D / 16; ++ft) {
    za[ft] = f32x4{0.f, 0.f, 0.f, 0.f};
    zb[ft] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < D / 32; ++j) {
      const Frag<T> w = load8(sW + (16 * ft + r16) * LDW + 32 * j + 8 * g4);
      za[ft] = mma(w, xa[j], za[ft]);
      zb[ft] = mma(w, xb[j], zb[ft]);
    }
  }
}

// True when every feature's log decay over the whole chunk is at most FAST_SPAN
// in magnitude (sTot holds the four sub-chunk sums); the same value in every
// wave of the workgroup.
template <int D>
__device__ __forceinline__ bool chunk_is_mild(const float *sTot, int lane) {
  float m = 0.f;
#pragma unroll
  for (int q = 0; q < D / 64; ++q) {
    const int f = lane + 64 * q;
    m = fmaxf(m, -(sTot[f] + sTot[D + f] + sTot[2 * D + f] + sTot[3 * D + f]));
  }
  return wave_max_all(m) <= FAST_SPAN;
}

// Same test when the table holds prefix sums from the chunk start (row 3 = the
// chunk total), as in the whole-head kernel.
template <int D>
__device__ __forceinline__ bool chunk_is_mild_c(const float *sC, int lane) {
  float m = 0.f;
#pragma unroll
  for (int q = 0; q < D / 64; ++q) m = fmaxf(m, -sC[3 * D + lane + 64 * q]);
  return wave_max_all(m) <= FAST_SPAN;
}

// Role-split forward (fwd_split.hip): 8 waves per workgroup.
template <typename T, int D, int DV, bool WIDE>
hipError_t launch_fwd_split(const FwdParams &p, hipStream_t stream);

}  // namespace lz
