// Lizard attention backward: gradients of a loss L through the forward (softmax or Hedgehog
// feature map, gated linear attention, anchor window, merge) given dL/dy.
//
// Decomposition (every kernel here; the host sequence is launch_bwd at the end):
//   1. bwd_phi_kernel       phi_q = fmap(q W_q), phi_k = fmap(k W_k) into the workspace.
//   2. bwd_f_kernel         role F (workgroups of four waves, one 16-feature tile each, D / 64
//                           workgroups per batch and query head): forward over 16-token steps
//                           with its columns of the state S in registers:
//                               dphi_q[t] = mix * S_t dy_t
//                           bwd_v_kernel, role V (workgroups of D / 32 waves, one wave per 16-column
//                           tile of v, two workgroups per batch and key/value head, the step's
//                           decayed operands shared in LDS): backward over the steps with its
//                           columns of dL/dS in registers:
//                               dv_gla[s] = mix * dS_s^T phi_k[s]
//   3. bwd_r_kernel         role R (workgroups as role F, per batch and key/value head): backward
//                           with its rows of dL/dS:  dphi_k[s] = mix * dS_s v_s, and the log-gate
//                           gradient dlg_j = sum_{t >= j} (sum_g phi_q phi_q-grad - phi_k phi_k-grad)
//   4. bwd_win_q_kernel     window softmax statistics, dq of the window, meta-token gradients.
//   5. bwd_win_k_kernel     dk of the window; dv = role V's part + the window's.
//   6. bwd_fb_kernel        feature-map backward, dq = dz_q W_q^T (+ window part), dk likewise,
//                           dW partial sums.
//   7. bwd_reduce_kernel    dW and dT from their partial sums.
//
// The sweeps run one wave per SIMD and take 256 short steps per sequence of 4096, so the latency of
// a step's loads is what bounds them unless it is hidden: each step's inputs are loaded several
// steps ahead into a ring of register sets (the step loop is unrolled over the ring, so every set
// keeps fixed registers; a set is refilled once the step that used it no longer needs it), column
// values are packed into operands only in the step that uses them (packing next to the load would
// wait for every load in flight), and roles F and R load each step's tiles once per workgroup and
// share them through LDS.

// Where the recurrence lives.  S_t = diag(gamma_t) S_{t-1} + phi_k(k_t) v_t^T and y_t = phi_q^T S_t
// (papernotes.org summary, "key designs", Gated Linear Attention item).  Inside a 16-token step
// with p_t the log-gate prefix from the step start (inclusive) and P its total,
//   S_t = diag(e^{p_t}) S_in + sum_{s <= t} diag(e^{p_t - p_s}) phi_k[s] v_s^T.
// A step is "mild" when P >= -60 for the features a wave handles: the exponentials then split
// into e^{p_t} <= 1 and e^{-p_s} <= e^60 factors on the MFMA operands.  Otherwise the in-step
// products are taken per element in fp32 (e.g. gamma ~ 0).  Every state update uses e^{P - p_s}
// <= 1 and needs no split.
//
// Precision: roles F and R compute with products of about 16 significant bits (the hi / lo
// bf16 split of mmx_ft and its kin; fp32 MFMAs for fp32 inputs): the log-gate gradient is a sum
// over the whole sequence of terms whose total is exactly zero, so their errors must stay far
// below bf16 rounding.  The feature maps are kept in fp32 for the same reason.
//
// MFMA conventions (common.hpp): x32 fragments for contractions over d; K = 16 fragments (F4) for
// contractions over the 16 tokens of a step: lane (r, kq) holds A[m = r][k = 4kq + j] and
// B[k = 4kq + j][n = r], j = 0..3, and the accumulator D[m = 4kq + i][n = r].  "Interleaved" rows:
// slot j of lane group kq in K-step ks holds column 32 ks + 16 (j >> 2) + 4 kq + (j & 3), the order
// in which an accumulator tile pair (16 dt.. , 16 dt + 16..) lists its rows, so that accumulators
// of the states serve as MFMA operands straight from registers.
#include "fwd_common.hpp"

namespace lz {
// Rows past the end of a sequence store their (never read) results here, so that every store is
// issued unconditionally.
__device__ __align__(16) float g_bwd_sink[2 * 128];
namespace bwd {

constexpr int TS = 16;              // tokens per sweep step / window tile
constexpr float MILD_SPAN = 60.f;   // -P at most this for the split exponentials
constexpr int QPW = 32;             // query tiles per wave in the window-q kernel
constexpr int NB = 5;               // key tiles of a band the window-q kernel loads at once
constexpr int FB_CHUNKS = 32;       // 64-row chunks per block of the feature-map backward
constexpr int NPF = 4;              // ring of step loads in the sweeps

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

template <typename T> struct F4;
template <> struct F4<bf16> { bf16x4 v; };
template <> struct F4<float> { float v[4]; };

template <typename T> __device__ __forceinline__ F4<T> f4_from(const float (&x)[4]) {
  F4<T> f;
#pragma unroll
  for (int j = 0; j < 4; ++j) f.v[j] = from_f<T>(x[j]);
  return f;
}
template <typename T> __device__ __forceinline__ float f4_at(const F4<T> &f, int j) { return to_f(f.v[j]); }

__device__ __forceinline__ f32x4 mma16(const F4<bf16> &a, const F4<bf16> &b, f32x4 c) {
  typedef short s4 __attribute__((ext_vector_type(4)));
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s4, a.v), __builtin_bit_cast(s4, b.v), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma16(const F4<float> &a, const F4<float> &b, f32x4 c) {
#pragma unroll
  for (int j = 0; j < 4; ++j) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[j], b.v[j], c, 0, 0, 0);
  return c;
}
// fp32 operands regardless of T (exact sums of fp32 values)
__device__ __forceinline__ f32x4 mma16_f32(const float (&a)[4], const float (&b)[4], f32x4 c) {
#pragma unroll
  for (int j = 0; j < 4; ++j) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[j], b[j], c, 0, 0, 0);
  return c;
}

// Rows r0 .. r0+3 of column c0 + (lane % 16) of a row-major tile in LDS (ld elements per row,
// a multiple of 4; c0 a multiple of 4).  bf16: one transposed read (ds_read_b64_tr_b16: lane m of
// each group of 16 reads 4 elements of row r0 + m / 4 from column c0 + 4 (m % 4), lane i receives
// column c0 + i of the 4 rows).
template <typename T> __device__ __forceinline__ F4<T> lds_col4(const T *tile, int ld, int r0, int c0) {
  const int m = threadIdx.x & 15;
  F4<T> f;
  if constexpr (sizeof(T) == 2) {
    typedef short s4 __attribute__((ext_vector_type(4)));
    const T *src = tile + (r0 + (m >> 2)) * ld + c0 + 4 * (m & 3);
    const s4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s4 *)(src));
    f.v = __builtin_bit_cast(bf16x4, x);
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) f.v[j] = tile[(r0 + j) * ld + c0 + m];
  }
  return f;
}

// Interleaved row fragment of K-step ks from row `row` of a [rows][D] tensor (zero when !ok).
template <typename T> __device__ __forceinline__ Frag<T> row_il(const T *base, int ks, int kq, bool ok) {
  if (!ok) return frag_zero<T>();
  return load4x2(base + 32 * ks + 4 * kq, base + 32 * ks + 16 + 4 * kq);
}
// The same fragment written into a row-major LDS tile row (natural column order).
template <typename T> __device__ __forceinline__ void store_il(T *row, const Frag<T> &f, int ks, int kq) {
  if constexpr (sizeof(T) == 2) {
    bf16x4 a, b;
#pragma unroll
    for (int j = 0; j < 4; ++j) { a[j] = f.v[j]; b[j] = f.v[4 + j]; }
    *reinterpret_cast<bf16x4 *>(row + 32 * ks + 4 * kq) = a;
    *reinterpret_cast<bf16x4 *>(row + 32 * ks + 16 + 4 * kq) = b;
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) { row[32 * ks + 4 * kq + j] = f.v[j]; row[32 * ks + 16 + 4 * kq + j] = f.v[4 + j]; }
  }
}
// Natural row fragment (columns 32 ks + 8 kq .. + 7) of row `row`.
template <typename T> __device__ __forceinline__ Frag<T> row_nat(const T *base, int ks, int kq, bool ok) {
  return ok ? load8(base + 32 * ks + 8 * kq) : frag_zero<T>();
}
// Column fragment: rows r0 + j (j = 0..3, zero at or beyond L) of column `col`.
template <typename T> __device__ __forceinline__ F4<T> col_g(const T *base, int D, int r0, int col, int L) {
  F4<T> f;
#pragma unroll
  for (int j = 0; j < 4; ++j) f.v[j] = (r0 + j < L) ? base[(size_t)(r0 + j) * D + col] : from_f<T>(0.f);
  return f;
}
// The same column values loaded ahead of their use: rows clamped into [0, L), each value in a
// register of its own (a 2-byte value zero-extended), so that nothing packs them, and with that
// waits for every load in flight, until the step that uses them; col_use then gives the operand,
// zero at rows at or beyond L.
template <typename T> struct Col4 {
  using R = typename std::conditional<sizeof(T) == 2, uint32_t, float>::type;
  R x[4];
};
template <typename T> __device__ __forceinline__ Col4<T> col_ld(const T *base, int D, int r0, int col, int L) {
  Col4<T> c;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const size_t off = (size_t)min(r0 + j, L - 1) * D + col;
    if constexpr (sizeof(T) == 2) c.x[j] = *reinterpret_cast<const uint16_t *>(base + off);
    else c.x[j] = base[off];
  }
  return c;
}
// Four consecutive elements as one load.
template <typename T> __device__ __forceinline__ F4<T> ld_f4(const T *src) {
  F4<T> f;
  if constexpr (sizeof(T) == 2) {
    f.v = *reinterpret_cast<const bf16x4 *>(src);
  } else {
    const f32x4 x = *reinterpret_cast<const f32x4 *>(src);
#pragma unroll
    for (int j = 0; j < 4; ++j) f.v[j] = x[j];
  }
  return f;
}
// Four consecutive elements as one LDS (or global) write, and a zero operand.
template <typename T> __device__ __forceinline__ void store_f4(T *dst, const F4<T> &f) {
  if constexpr (sizeof(T) == 2) *reinterpret_cast<bf16x4 *>(dst) = f.v;
  else *reinterpret_cast<f32x4 *>(dst) = f32x4{f.v[0], f.v[1], f.v[2], f.v[3]};
}
template <typename T> __device__ __forceinline__ F4<T> f4_zero() {
  F4<T> f;
#pragma unroll
  for (int j = 0; j < 4; ++j) f.v[j] = from_f<T>(0.f);
  return f;
}
// Keeps the compiler from moving work on a fragment loaded ahead up to its load.
template <typename T> __device__ __forceinline__ void opaque_frag(Frag<T> &f) {
  if constexpr (sizeof(T) == 2) {
    asm volatile("" : "+v"(f.v));
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) asm volatile("" : "+v"(f.v[j]));
  }
}
template <typename T> __device__ __forceinline__ F4<T> col_use(const Col4<T> &c, int r0, int L) {
  F4<T> f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if constexpr (sizeof(T) == 2) f.v[j] = __builtin_bit_cast(T, (uint16_t)((r0 + j < L) ? c.x[j] : 0u));
    else f.v[j] = (r0 + j < L) ? c.x[j] : 0.f;
  }
  return f;
}
__device__ __forceinline__ void colf_g(const float *base, int D, int r0, int col, int L, float (&x)[4]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) x[j] = (r0 + j < L) ? base[(size_t)(r0 + j) * D + col] : 0.f;
}

// Conversions between operand types.
template <typename T> __device__ __forceinline__ Frag<float> to32(const Frag<T> &f) {
  Frag<float> o;
#pragma unroll
  for (int j = 0; j < 8; ++j) o.v[j] = to_f(f.v[j]);
  return o;
}
template <typename T> __device__ __forceinline__ F4<float> to32(const F4<T> &f) {
  F4<float> o;
#pragma unroll
  for (int j = 0; j < 4; ++j) o.v[j] = to_f(f.v[j]);
  return o;
}
template <typename T> __device__ __forceinline__ Frag<T> from32(const Frag<float> &f) {
  float x[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) x[j] = f.v[j];
  return frag_from<T>(x);
}

// Products where one or both operands are fp32 values that a bf16 operand would round too coarsely
// (the sweeps' states and decayed feature maps: the log-gate gradient sums products of the sweeps'
// outputs over whole sequences, and those sums cancel to zero overall).  With T = bf16 an fp32
// value x is split into hi = bf16(x) and lo = bf16(x - hi), about 16 significant bits: one fp32
// operand against an exact T operand takes two MFMAs, two fp32 operands three (the lo * lo term is
// below 2^-16 of the product).  With T = fp32 the products are fp32 MFMAs.
__device__ __forceinline__ bf16 hi_bf16(float x) { return (bf16)x; }
__device__ __forceinline__ bf16 lo_bf16(float x) { return (bf16)(x - (float)(bf16)x); }
template <typename T> __device__ __forceinline__ f32x4 mmx_ft(const float (&a)[8], const Frag<T> &b, f32x4 c) {
  if constexpr (sizeof(T) == 2) {
    Frag<bf16> h, l;
#pragma unroll
    for (int j = 0; j < 8; ++j) { h.v[j] = hi_bf16(a[j]); l.v[j] = lo_bf16(a[j]); }
    return mma(l, b, mma(h, b, c));
  } else {
    return mma(frag_from<float>(a), b, c);
  }
}
template <typename T> __device__ __forceinline__ f32x4 mmx_tf(const Frag<T> &a, const float (&b)[8], f32x4 c) {
  if constexpr (sizeof(T) == 2) {
    Frag<bf16> h, l;
#pragma unroll
    for (int j = 0; j < 8; ++j) { h.v[j] = hi_bf16(b[j]); l.v[j] = lo_bf16(b[j]); }
    return mma(a, l, mma(a, h, c));
  } else {
    return mma(a, frag_from<float>(b), c);
  }
}
template <typename T> __device__ __forceinline__ f32x4 m16_tf(const F4<T> &a, const float (&b)[4], f32x4 c) {
  if constexpr (sizeof(T) == 2) {
    F4<bf16> h, l;
#pragma unroll
    for (int j = 0; j < 4; ++j) { h.v[j] = hi_bf16(b[j]); l.v[j] = lo_bf16(b[j]); }
    return mma16(a, l, mma16(a, h, c));
  } else {
    return mma16(a, f4_from<float>(b), c);
  }
}
template <typename T> __device__ __forceinline__ f32x4 m16_ff(const float (&a)[4], const float (&b)[4], f32x4 c) {
  if constexpr (sizeof(T) == 2) {
    F4<bf16> ah, al, bh, bl;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      ah.v[j] = hi_bf16(a[j]); al.v[j] = lo_bf16(a[j]);
      bh.v[j] = hi_bf16(b[j]); bl.v[j] = lo_bf16(b[j]);
    }
    return mma16(al, bh, mma16(ah, bl, mma16(ah, bh, c)));
  } else {
    return mma16(f4_from<float>(a), f4_from<float>(b), c);
  }
}

// Constant triangles of the in-step prefix sums: lane (r, kq) slot j -> (4 kq + j <= r).
template <typename T> __device__ __forceinline__ F4<T> tri_le(int r, int kq) {
  float x[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) x[j] = (4 * kq + j <= r) ? 1.f : 0.f;
  return f4_from<T>(x);
}

}  // namespace bwd

using namespace bwd;

// ======================================================================== 1. feature maps
// One workgroup of four waves per PHI_ROWS rows of q (blocks < nq) or k: phi = softmax(x W) or
// exp(xW) (+) exp(-xW), stored in fp32 (the log-gate gradient sums products of phi with its
// gradient over the whole sequence, and those sums cancel to zero overall: their terms need fp32
// accuracy); W^T staged in LDS once per workgroup, each wave's next 16 rows loaded while the
// current ones are mapped.
constexpr int PHI_ROWS = 256;
template <typename T, int D, bool HH>
__global__ __launch_bounds__(256) void bwd_phi_kernel(BwdParams p) {
  constexpr int NFT = D / 16, KS = D / 32, LDW = D + 16 / (int)sizeof(T);
  constexpr int FC = HH ? D / 2 : D;
  __shared__ __align__(16) T sW[D * LDW];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, r = lane & 15, kq = lane >> 4;
  const int nblk = (p.L + PHI_ROWS - 1) / PHI_ROWS;
  const int nq = p.B * p.Hq * nblk;
  const bool qside = (int)blockIdx.x < nq;
  const int bid = qside ? blockIdx.x : blockIdx.x - nq;
  const int H = qside ? p.Hq : p.Hkv;
  const int bh = bid / nblk, r0 = (bid % nblk) * PHI_ROWS, r1 = min(p.L, r0 + PHI_ROWS);
  const int h = bh % H;
  const T *Wsrc = reinterpret_cast<const T *>(qside ? p.wq : p.wk) + (size_t)h * p.w_stride;
  const T *X = reinterpret_cast<const T *>(qside ? p.q : p.k) + (size_t)bh * p.L * D;
  float *PH = (qside ? p.phq : p.phk) + (size_t)bh * p.L * D;
  // W[i][c] -> sW[c][i] (and -W -> sW[FC + c][i]): the lanes of a wave take consecutive rows i
  // (pairs of rows for 2-byte types, one 4-byte word per lane and column), so a wave's writes to a
  // row of sW fall in distinct banks; every load is issued before the first write
  constexpr int RPI = sizeof(T) == 2 ? 2 : 1;
  constexpr int NR = D / RPI, NI = NR * (FC / 8), IT = (NI + 255) / 256;
  Frag<T> wa[IT][RPI];
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int idx = min(tid + 256 * it, NI - 1);
    const int i0 = RPI * (idx % NR), f0 = 8 * (idx / NR);
#pragma unroll
    for (int u = 0; u < RPI; ++u) wa[it][u] = load8(Wsrc + (size_t)(i0 + u) * FC + f0);
  }
  Frag<T> xf[KS];
  {
    const int t = r0 + 16 * w + r;
#pragma unroll
    for (int j = 0; j < KS; ++j) xf[j] = row_nat(X + (size_t)t * D, j, kq, t < r1);
  }
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int idx = tid + 256 * it;
    if (NI % 256 == 0 || idx < NI) {
      const int i0 = RPI * (idx % NR), f0 = 8 * (idx / NR);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if constexpr (RPI == 2) {
          T pair[2] = {wa[it][0].v[j], wa[it][1].v[j]};
          const uint32_t u = *reinterpret_cast<const uint32_t *>(pair);
          *reinterpret_cast<uint32_t *>(sW + (f0 + j) * LDW + i0) = u;
          if constexpr (HH) *reinterpret_cast<uint32_t *>(sW + (FC + f0 + j) * LDW + i0) = u ^ 0x80008000u;
        } else {
          sW[(f0 + j) * LDW + i0] = wa[it][0].v[j];
          if constexpr (HH) sW[(FC + f0 + j) * LDW + i0] = -wa[it][0].v[j];
        }
      }
    }
  }
  __syncthreads();
  for (int c0 = r0; c0 < r1; c0 += 64) {
    const int t = c0 + 16 * w + r;
    Frag<T> xn[KS];  // the wave's next rows in flight
#pragma unroll
    for (int j = 0; j < KS; ++j) xn[j] = row_nat(X + (size_t)(t + 64) * D, j, kq, t + 64 < r1);
    f32x4 z[NFT];
    feature_logits<T, D, LDW>(sW, xf, r, kq, z);  // z^T[f][t]: lane (t = r, kq) holds f = 16 ft + 4 kq + i
    float ph[NFT][4];
    if constexpr (HH) {
#pragma unroll
      for (int ft = 0; ft < NFT; ++ft)
#pragma unroll
        for (int i = 0; i < 4; ++i) ph[ft][i] = __expf(z[ft][i]);
    } else {
      softmax_rows<NFT>(z, ph);
    }
    if (t < r1) {
#pragma unroll
      for (int ft = 0; ft < NFT; ++ft)
        *reinterpret_cast<f32x4 *>(PH + (size_t)t * D + 16 * ft + 4 * kq) = f32x4{ph[ft][0], ph[ft][1], ph[ft][2], ph[ft][3]};
    }
#pragma unroll
    for (int j = 0; j < KS; ++j) xf[j] = xn[j];
  }
}

// ======================================================================== 2/3. sweeps
// Wave-private LDS tiles of a step: T rows of 16 tokens (8-byte aligned transposed reads), and
// fp32 tables of the exact path (16 tokens x the features the wave handles).
// Role R: dphi_k for the features of key/value head hk and dlg of those features, backward over
// the steps with the workgroup's rows of dL/dS in registers (four waves, one 16-feature tile each,
// D / 64 workgroups per head, 8 launch slots apart).  As in role F, each step's tiles -- v and
// the first query head's dy rows, log gamma, phi_k and that head's phi_q and dphi_q rows of the
// workgroup's 64 features -- are loaded once per workgroup NPF steps ahead and shared through two
// LDS buffers (dynamic shared memory: LdsR2 exceeds the static limit).  Further query heads of a
// group are loaded into the step's buffer when the previous head is done with it.
template <typename T, int D> struct LdsR2 {
  static constexpr int LD = D + 16 / (int)sizeof(T);
  static constexpr int LDG = 64 + 16 / (int)sizeof(T);
  static constexpr int LDP = 68;
  static constexpr int LDF = 20;
  T v[2][TS * LD], dy[2][TS * LD], lg[2][TS * LDG];
  float pk[2][TS * LDP], pq[2][TS * LDP], dq[2][TS * LDP];
  float pf[4][TS * LDF], ph1[4][TS * LDF], ph2[4][TS * LDF], dd[4][TS * 17];  // per wave: exact path
};

template <typename T, int D>
__global__ __launch_bounds__(256, 1) void bwd_r_kernel(BwdParams p) {
  using SM = LdsR2<T, D>;
  constexpr int NDT = D / 16, NKS = D / 32, LD = SM::LD, LDG = SM::LDG, LDP = SM::LDP, LDF = SM::LDF;
  constexpr int NH = D / 64;
  constexpr int RP = D * (int)sizeof(T) / 16;
  constexpr int NPC = TS * RP;
  extern __shared__ __attribute__((aligned(16))) char smem_r[];
  SM &sm = *reinterpret_cast<SM *>(smem_r);
  const int tid = threadIdx.x, lane = tid & 63, r = lane & 15, kq = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int x = blockIdx.x;
  const int bh = NH == 2 ? (x >> 4) * 8 + (x & 7) : x, half = NH == 2 ? (x >> 3) & 1 : 0;
  if (bh >= p.B * p.Hkv) return;  // padding of the launch to whole XCD pairs
  const int b = bh / p.Hkv, hk = bh % p.Hkv;
  const int L = p.L, G = p.G, fw = 64 * half, f0 = fw + 16 * w;
  const size_t kvo = (size_t)bh * L * D;
  const T *V = reinterpret_cast<const T *>(p.v) + kvo;
  const T *LG = reinterpret_cast<const T *>(p.lg) + kvo;
  const float *PK = p.phk + kvo;
  float *DPK = p.dphk + kvo;
  T *DLG = reinterpret_cast<T *>(p.dlg) + kvo;
  float *pfw = sm.pf[w], *ph1w = sm.ph1[w], *ph2w = sm.ph2[w], *ddw = sm.dd[w];
  auto qoff = [&](int g) { return ((size_t)b * p.Hq + hk * G + g) * L * D; };
  f32x4 dS[NDT];  // dS^T[dv = 16 dt + 4 kq + i][f = f0 + r]
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) dS[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  const F4<T> tri = tri_le<T>(r, kq);
  float ufs[4];  // U[t][t'] = (t' >= t): lane (t = r, kq) slot j -> (4 kq + j >= r)
#pragma unroll
  for (int j = 0; j < 4; ++j) ufs[j] = (4 * kq + j >= r) ? 1.f : 0.f;
  float rsum = 0.f;  // dlg of feature f0 + r summed over the later steps
  const int nstep = (L + TS - 1) / TS;
  const int prow = tid / RP, pcol = (tid % RP) * (16 / (int)sizeof(T));
  const int grow = tid / 16, gcol = 4 * (tid % 16);
  struct HeadPre {
    u32x4 dy;
    f32x4 pq, dq;
  };
  struct Pre {
    u32x4 v;
    F4<T> lg;
    f32x4 pk;
    HeadPre h;
  };
  auto load_head = [&](HeadPre &hp, int c0, int g) {  // rows clamped into the sequence
    const size_t qo = qoff(g);
    // (unconditional, as in role F: threads past the tile load a duplicate piece, not stored)
    hp.dy = *reinterpret_cast<const u32x4 *>(reinterpret_cast<const T *>(p.dy) + qo +
                                               (size_t)min(c0 + prow % TS, L - 1) * D + pcol);
    const size_t og = qo + (size_t)min(c0 + grow, L - 1) * D + fw + gcol;
    hp.pq = *reinterpret_cast<const f32x4 *>(p.phq + og);
    hp.dq = *reinterpret_cast<const f32x4 *>(p.dphq + og);
  };
  auto load_pre = [&](Pre &pr, int st) {
    const int c0 = max(st, 0) * TS;
    pr.v = *reinterpret_cast<const u32x4 *>(V + (size_t)min(c0 + prow % TS, L - 1) * D + pcol);
    const size_t og = (size_t)min(c0 + grow, L - 1) * D + fw + gcol;
    if constexpr (sizeof(T) == 2) {
      pr.lg.v = *reinterpret_cast<const bf16x4 *>(LG + og);
    } else {
      const f32x4 t = *reinterpret_cast<const f32x4 *>(LG + og);
#pragma unroll
      for (int j = 0; j < 4; ++j) pr.lg.v[j] = t[j];
    }
    pr.pk = *reinterpret_cast<const f32x4 *>(PK + og);
    load_head(pr.h, c0, 0);
  };
  // rows at or beyond L: no decay and no features (zeros), so they add nothing anywhere
  auto store_head = [&](const HeadPre &hp, int buf, int c0) {
    if (tid < NPC) *reinterpret_cast<u32x4 *>(sm.dy[buf] + prow * LD + pcol) = hp.dy;
    const bool in = c0 + grow < L;
    float *q = sm.pq[buf] + grow * LDP + gcol, *d = sm.dq[buf] + grow * LDP + gcol;
    *reinterpret_cast<f32x4 *>(q) = in ? hp.pq : f32x4{0.f, 0.f, 0.f, 0.f};
    *reinterpret_cast<f32x4 *>(d) = in ? hp.dq : f32x4{0.f, 0.f, 0.f, 0.f};
  };
  auto store_pre = [&](const Pre &pr, int buf, int c0) {
    if (tid < NPC) *reinterpret_cast<u32x4 *>(sm.v[buf] + prow * LD + pcol) = pr.v;
    const bool in = c0 + grow < L;
    T *g = sm.lg[buf] + grow * LDG + gcol;
    float *k = sm.pk[buf] + grow * LDP + gcol;
    store_f4(g, in ? pr.lg : f4_zero<T>());
    *reinterpret_cast<f32x4 *>(k) = in ? pr.pk : f32x4{0.f, 0.f, 0.f, 0.f};
    store_head(pr.h, buf, c0);
  };
  auto step = [&](Pre &pr, int buf, int st) {
    const int c0 = st * TS;
    store_pre(pr, buf, c0);
    load_pre(pr, st - NPF);  // this ring slot's registers are free now
    __syncthreads();         // the step's tiles visible
    const T *tv = sm.v[buf] + r * LD;
    Frag<T> vf[NKS];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) vf[ks] = load4x2(tv + 32 * ks + 4 * kq, tv + 32 * ks + 16 + 4 * kq);
    const F4<T> lgc = lds_col4(sm.lg[buf], LDG, 4 * kq, 16 * w);
    F4<float> pkc;
#pragma unroll
    for (int j = 0; j < 4; ++j) pkc.v[j] = sm.pk[buf][(4 * kq + j) * LDP + 16 * w + r];
    const f32x4 pK = mma16(tri, lgc, f32x4{0.f, 0.f, 0.f, 0.f});  // lane (f0 + r, kq): s = 4 kq + i
    const float Pf = __shfl(pK[3], 48 + r);
    const bool mild = wave_max_all(-Pf) <= MILD_SPAN;
    // ---- inter: X[s][f] = sum_dv v_s[dv] dS[f][dv] (lane (f0 + r, kq): s = 4 kq + i)
    f32x4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      float xs[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) xs[j] = dS[2 * ks + (j >> 2)][j & 3];
      o = mmx_tf<T>(vf[ks], xs, o);
    }
    const float eP = __expf(Pf);
    if (mild) {
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] *= eP;  // times e^{-p_s} below: e^{P - p_s} in all
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) pfw[(4 * kq + i) * LDF + r] = pK[i];
    }
    float gq[4] = {0.f, 0.f, 0.f, 0.f};  // sum_g phi_q dphi_q at (t = 4 kq + i, f0 + r)
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) dS[dt][i] *= eP;
    for (int g = 0; g < G; ++g) {
      if (g > 0) {  // this head's tiles into the step's buffer, once every wave is done with the last
        HeadPre hp;
        load_head(hp, c0, g);
        __syncthreads();
        store_head(hp, buf, c0);
        __syncthreads();
      }
      const T *ty = sm.dy[buf] + r * LD;
      Frag<T> dyf[NKS];
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) dyf[ks] = load4x2(ty + 32 * ks + 4 * kq, ty + 32 * ks + 16 + 4 * kq);
      F4<float> pqc, dqc;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        pqc.v[j] = sm.pq[buf][(4 * kq + j) * LDP + 16 * w + r];
        dqc.v[j] = sm.dq[buf][(4 * kq + j) * LDP + 16 * w + r];
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) gq[j] += f4_at(pqc, j) * f4_at(dqc, j);
      // E[t][s] = dy_t . v_s (lane (s = r, kq): t = 4 kq + i), masked to t >= s
      f32x4 e = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) e = mma(dyf[ks], vf[ks], e);
#pragma unroll
      for (int i = 0; i < 4; ++i) e[i] = (4 * kq + i >= r) ? e[i] : 0.f;
      // Qt[t][f] = phi_q[t][f] e^{p_t[f]} (lane (f0 + r, kq): t = 4 kq + j)
      float qt[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) qt[j] = f4_at(pqc, j) * __expf(pK[j]);
      if (mild) {
        float ea[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) ea[i] = e[i];
        // sum_t E[t][s] Qt[t][f]; times e^{-p_s} below
        o = m16_ff<T>(ea, qt, o);
      } else {
        // exact: sum_{t >= s} E[t][s] phi_q[t][f] e^{p_t[f] - p_s[f]}, one exponent per term,
        // summed over the group's query heads in ph2 (the wave's own tables)
#pragma unroll
        for (int i = 0; i < 4; ++i) ph1w[(4 * kq + i) * LDF + r] = f4_at(pqc, i);
#pragma unroll
        for (int i = 0; i < 4; ++i) ddw[(4 * kq + i) * 17 + r] = e[i];
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int s2 = 4 * kq + i;
          float xx = 0.f;
          for (int t = s2; t < TS; ++t)
            xx += ddw[t * 17 + s2] * ph1w[t * LDF + r] * __expf(pfw[t * LDF + r] - pfw[s2 * LDF + r]);
          ph2w[s2 * LDF + r] = (g == 0 ? 0.f : ph2w[s2 * LDF + r]) + xx;
        }
        __builtin_amdgcn_wave_barrier();
      }
      // dS^T[dv][f] += sum_t dy_t[dv] Qt[t][f]
      F4<T> dyt[NDT];  // (every fragment read before the first product)
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) dyt[dt] = lds_col4(sm.dy[buf], LD, 4 * kq, 16 * dt);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) dS[dt] = m16_tf<T>(dyt[dt], qt, dS[dt]);
    }
    // ---- dphi_k[s][f] = mix e^{-p_s} (e^{P} X + sum_g intra)   (lane (f0 + r, kq): s = 4 kq + i)
    float dpk[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (mild) {
        dpk[i] = p.mix * o[i] * __expf(-pK[i]);
      } else {  // o: the unscaled inter term
        dpk[i] = p.mix * (o[i] * __expf(Pf - pK[i]) + ph2w[(4 * kq + i) * LDF + r]);
      }
    }
    // ---- dlg: db[t][f] = sum_g phi_q dphi_q - phi_k dphi_k; reverse cumsum in the step (fp32 MFMA)
    float db[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) db[i] = gq[i] - f4_at(pkc, i) * dpk[i];
    const f32x4 cs = mma16_f32(ufs, db, f32x4{0.f, 0.f, 0.f, 0.f});  // lane (f0 + r, kq): t = 4 kq + i
    const float tot = __shfl(cs[0], r);                              // t = 0: the step's total
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int s2 = c0 + 4 * kq + i;
      const bool in = s2 < L;  // (rows past the end: the sink)
      (in ? DPK + (size_t)s2 * D : g_bwd_sink)[f0 + r] = dpk[i];
      (in ? DLG + (size_t)s2 * D : reinterpret_cast<T *>(g_bwd_sink + 128))[f0 + r] = from_f<T>(cs[i] + rsum);
    }
    rsum += tot;
  };
  // steps st = nstep - 1 - k for k = 0, 1, ..: ring slot k % NPF, LDS buffer k % 2
  static_assert(NPF % 2 == 0, "ring slot and LDS buffer parities must agree");
  Pre ring[NPF];
#pragma unroll
  for (int u = 0; u < NPF; ++u) load_pre(ring[u], nstep - 1 - u);
  int k = 0;
  for (; k + NPF <= nstep; k += NPF) {
#pragma unroll
    for (int u = 0; u < NPF; ++u) step(ring[u], u & 1, nstep - 1 - (k + u));
  }
#pragma unroll
  for (int u = 0; u < NPF; ++u)
    if (k + u < nstep) step(ring[u], u & 1, nstep - 1 - (k + u));
}

// Role F: dphi_q for the features of query head hq (see the top of the file).  Workgroups of four
// waves, one 16-feature tile each (D / 64 workgroups per head, 8 launch slots apart: one XCD).
// Each step's tiles -- dy and v rows (all D columns), log gamma and phi_k rows (the workgroup's 64
// features) -- are loaded once per workgroup with 16-byte loads, NPF steps ahead into registers,
// and written into one of two LDS buffers at the step's start; every wave reads its operands
// there.  One barrier per step: a buffer is rewritten two steps after it was read, and every wave
// has passed the barrier between.
template <typename T, int D> struct LdsF2 {
  static constexpr int LD = D + 16 / (int)sizeof(T);  // T rows of dy and v
  static constexpr int LDG = 64 + 16 / (int)sizeof(T); // T rows of log gamma (64 features)
  static constexpr int LDP = 68;                       // fp32 rows of phi_k (64 features)
  static constexpr int LDF = 20;
  T dy[2][TS * LD], v[2][TS * LD], lg[2][TS * LDG];
  float pk[2][TS * LDP];
  float pf[4][TS * LDF], ph1[4][TS * LDF];  // per wave: exact-path tables
};

template <typename T, int D>
__global__ __launch_bounds__(256, 1) void bwd_f_kernel(BwdParams p) {
  using SM = LdsF2<T, D>;
  constexpr int NDT = D / 16, NKS = D / 32, LD = SM::LD, LDG = SM::LDG, LDP = SM::LDP, LDF = SM::LDF;
  constexpr int NH = D / 64;                      // workgroups per head
  constexpr int RP = D * (int)sizeof(T) / 16;     // 16-byte pieces per dy / v row
  constexpr int NPC = TS * RP;                    // pieces per tile (<= 256)
  __shared__ SM sm;
  const int tid = threadIdx.x, lane = tid & 63, r = lane & 15, kq = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int x = blockIdx.x;
  const int bh = NH == 2 ? (x >> 4) * 8 + (x & 7) : x, half = NH == 2 ? (x >> 3) & 1 : 0;
  if (bh >= p.B * p.Hq) return;  // padding of the launch to whole XCD pairs
  const int b = bh / p.Hq, hq = bh % p.Hq;
  const int L = p.L, hk = hq / p.G, fw = 64 * half, f0 = fw + 16 * w;
  const size_t kvo = ((size_t)b * p.Hkv + hk) * L * D, qo = ((size_t)b * p.Hq + hq) * L * D;
  const T *V = reinterpret_cast<const T *>(p.v) + kvo;
  const T *LG = reinterpret_cast<const T *>(p.lg) + kvo;
  const float *PK = p.phk + kvo;
  const T *DY = reinterpret_cast<const T *>(p.dy) + qo;
  float *DPQ = p.dphq + qo;
  float *pfw = sm.pf[w], *ph1w = sm.ph1[w];
  f32x4 S[NDT];  // S^T[dv = 16 dt + 4 kq + i][f = f0 + r]
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) S[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  const F4<T> tri = tri_le<T>(r, kq);
  // this thread's pieces of a step: dy and v piece tid (row tid / RP), and four log gamma and
  // phi_k values (row tid / 16, features fw + 4 (tid % 16) ..)
  const int prow = tid / RP, pcol = (tid % RP) * (16 / (int)sizeof(T));
  const int grow = tid / 16, gcol = 4 * (tid % 16);
  struct Pre {
    u32x4 dy, v;
    F4<T> lg;
    f32x4 pk;
  };
  auto load_pre = [&](Pre &pr, int c0) {  // rows clamped into the sequence
    // (every thread loads, those past the tile a duplicate piece that is not stored: a load
    // under a condition would leave the compiler unsure it was issued, and it would then wait
    // for later loads as well before using earlier ones)
    const size_t o = (size_t)min(c0 + prow % TS, L - 1) * D + pcol;
    pr.dy = *reinterpret_cast<const u32x4 *>(DY + o);
    pr.v = *reinterpret_cast<const u32x4 *>(V + o);
    const size_t og = (size_t)min(c0 + grow, L - 1) * D + fw + gcol;
    if constexpr (sizeof(T) == 2) {
      pr.lg.v = *reinterpret_cast<const bf16x4 *>(LG + og);
    } else {
      const f32x4 t = *reinterpret_cast<const f32x4 *>(LG + og);
#pragma unroll
      for (int j = 0; j < 4; ++j) pr.lg.v[j] = t[j];
    }
    pr.pk = *reinterpret_cast<const f32x4 *>(PK + og);
  };
  auto store_pre = [&](const Pre &pr, int buf, int c0) {  // rows at or beyond L: no decay, no phi_k
    if (tid < NPC) {
      *reinterpret_cast<u32x4 *>(sm.dy[buf] + prow * LD + pcol) = pr.dy;
      *reinterpret_cast<u32x4 *>(sm.v[buf] + prow * LD + pcol) = pr.v;
    }
    const bool in = c0 + grow < L;
    T *g = sm.lg[buf] + grow * LDG + gcol;
    float *k = sm.pk[buf] + grow * LDP + gcol;
    store_f4(g, in ? pr.lg : f4_zero<T>());
    *reinterpret_cast<f32x4 *>(k) = in ? pr.pk : f32x4{0.f, 0.f, 0.f, 0.f};
  };
  auto step = [&](Pre &pr, int buf, int c0) {
    store_pre(pr, buf, c0);
    load_pre(pr, c0 + NPF * TS);  // this ring slot's registers are free now
    __syncthreads();              // the step's tiles visible
    const bool rok = c0 + r < L;
    const T *ty = sm.dy[buf] + r * LD, *tv = sm.v[buf] + r * LD;
    Frag<T> dyf[NKS], vf[NKS];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      dyf[ks] = load4x2(ty + 32 * ks + 4 * kq, ty + 32 * ks + 16 + 4 * kq);
      vf[ks] = load4x2(tv + 32 * ks + 4 * kq, tv + 32 * ks + 16 + 4 * kq);
    }
    const F4<T> lgc = lds_col4(sm.lg[buf], LDG, 4 * kq, 16 * w);  // rows 4 kq + j, feature f0 + r
    F4<float> pkc;
#pragma unroll
    for (int j = 0; j < 4; ++j) pkc.v[j] = sm.pk[buf][(4 * kq + j) * LDP + 16 * w + r];
    // ---- prefix sums: pK (lane (f = f0 + r, kq): s = 4 kq + i), pQ (lane (t = r, kq): f = f0 + 4 kq + i)
    const f32x4 pK = mma16(tri, lgc, f32x4{0.f, 0.f, 0.f, 0.f});
    const f32x4 pQ = mma16(lgc, tri, f32x4{0.f, 0.f, 0.f, 0.f});
    const float Pf = __shfl(pK[3], 48 + r);  // chunk total of feature f0 + r
    const bool mild = wave_max_all(-Pf) <= MILD_SPAN;
    // ---- D^T[s][t] = v_s . dy_t (lane (t = r, kq): s = 4 kq + i), masked to s <= t
    f32x4 dT = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) dT = mma(vf[ks], dyf[ks], dT);
#pragma unroll
    for (int i = 0; i < 4; ++i) dT[i] = (4 * kq + i <= r) ? dT[i] : 0.f;
    // ---- inter: Out^T[f][t] = sum_dv S[f][dv] dy_t[dv]
    f32x4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      float xs[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) xs[j] = S[2 * ks + (j >> 2)][j & 3];
      o = mmx_ft<T>(xs, dyf[ks], o);
    }
    if (mild) {
      float kt[4], dm[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        kt[j] = f4_at(pkc, j) * __expf(-pK[j]);
        dm[j] = dT[j];
      }
      o = m16_ff<T>(kt, dm, o);
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] *= __expf(pQ[i]);
    } else {
      // exact: o = e^{p_t} o_inter + sum_{s <= t} D[t][s] phi_k[s][f] e^{p_t[f] - p_s[f]} (the
      // wave's own tables: a wave barrier orders its writes before its reads)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pfw[(4 * kq + i) * LDF + r] = pK[i];
        ph1w[(4 * kq + i) * LDF + r] = f4_at(pkc, i);
      }
      __builtin_amdgcn_wave_barrier();
      float dts[16];
#pragma unroll
      for (int s2 = 0; s2 < 16; ++s2) dts[s2] = __shfl(dT[s2 & 3], r + 16 * (s2 >> 2));
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int fl = 4 * kq + i;
        float a = o[i] * __expf(pQ[i]);
        for (int s2 = 0; s2 <= r; ++s2) a += dts[s2] * ph1w[s2 * LDF + fl] * __expf(pQ[i] - pfw[s2 * LDF + fl]);
        o[i] = a;
      }
      __builtin_amdgcn_wave_barrier();
    }
    {  // (rows past the end into the sink: stores under a condition make the compiler's waits for
       // the load ring conservative)
      float *dst = rok ? DPQ + (size_t)(c0 + r) * D : g_bwd_sink;
      *reinterpret_cast<f32x4 *>(dst + f0 + 4 * kq) = f32x4{p.mix * o[0], p.mix * o[1], p.mix * o[2], p.mix * o[3]};
    }
    // ---- state: S^T = e^{P} S^T + V^T Kbar, Kbar[s][f] = phi_k[s][f] e^{P - p_s[f]}
    float kb[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) kb[j] = f4_at(pkc, j) * __expf(Pf - pK[j]);
    const float eP = __expf(Pf);
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) S[dt][i] *= eP;
      S[dt] = m16_tf<T>(lds_col4(sm.v[buf], LD, 4 * kq, 16 * dt), kb, S[dt]);
    }
  };
  // steps c0 = 0, TS, ..: ring slot (c0 / TS) % NPF, LDS buffer (c0 / TS) % 2
  static_assert(NPF % 2 == 0, "ring slot and LDS buffer parities must agree");
  Pre ring[NPF];
#pragma unroll
  for (int u = 0; u < NPF; ++u) load_pre(ring[u], u * TS);
  int c00 = 0;
  for (; c00 + NPF * TS <= L; c00 += NPF * TS) {
#pragma unroll
    for (int u = 0; u < NPF; ++u) step(ring[u], u & 1, c00 + u * TS);
  }
#pragma unroll
  for (int u = 0; u < NPF; ++u)  // the last 1 .. NPF steps (a ragged tail can leave NPF)
    if (c00 + u * TS < L) step(ring[u], u & 1, c00 + u * TS);
}

// Role V: dv_gla[s] = mix dS_s^T phi_k-part for value columns of key/value head hk, summed over its
// query heads, backward over the 16-token steps with dL/dS for the wave's 16 value columns in
// registers:  dv[s] = sum_f Kbar[s][f] dS[f] + sum_{t >= s} A[t][s] dy_t,  then
// dS <- diag(e^P) dS + Qtil^T dY  with Kbar = phi_k e^{P - p_s}, Qtil = phi_q e^{p_t} and, on a mild
// step, A = Qtil Ktil^T, Ktil = phi_k e^{-p_s} (otherwise A per element in fp32).
// Every value column needs the same decayed operands, so the waves of a workgroup share them: the
// NW = D / 32 waves take value tiles h NW + w of one (batch, key/value head), h = 0, 1 the two
// workgroups of the head (8 launch slots apart: one XCD, so the second reads the head's inputs from
// L2), and wave w builds the operands for features 32 w .. 32 w + 31 of every step into LDS.
template <typename T, int D> struct LdsV2 {
  static constexpr int NW = D / 32;
  static constexpr int LD = D + 8;   // T rows of the shared operands (natural feature order)
  static constexpr int LDL = 40;     // T rows of a wave's log-gamma slice (32 features)
  static constexpr int LDX = 36;     // fp32 rows of a wave's exact-path slice
  T kb[TS * LD], kt[TS * LD], qt[TS * LD];  // Kbar, Ktil, Qtil of the step [token][feature]
  float ep[D];                              // e^{P[f]}
  float span[NW];                           // per slice: max over its features of -P
  T lg[NW][TS * LDL];                       // per wave: log gamma of its slice
  float xp[NW][TS * LDX], xq[NW][TS * LDX], xk[NW][TS * LDX];  // per wave: p, phi_q, phi_k (exact path)
  float part[NW][TS * 17];                  // exact path: per slice, partial A[t][s]
};

template <typename T, int D>
__global__ __launch_bounds__(64 * (D / 32)) void bwd_v_kernel(BwdParams p) {
  using S = LdsV2<T, D>;
  constexpr int NW = S::NW, NFT = D / 16, NKS = D / 32, LD = S::LD, LDL = S::LDL, LDX = S::LDX;
  __shared__ S sm;
  const int tid = threadIdx.x, lane = tid & 63, r = lane & 15, kq = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int bh = (blockIdx.x >> 4) * 8 + (blockIdx.x & 7), half = (blockIdx.x >> 3) & 1;
  if (bh >= p.B * p.Hkv) return;  // padding of the launch to whole XCD pairs
  const int hk = bh % p.Hkv, b = bh / p.Hkv;
  const int L = p.L, G = p.G, dv0 = 16 * (half * NW + w);
  const size_t kvo = (size_t)bh * L * D;
  const T *LG = reinterpret_cast<const T *>(p.lg) + kvo;
  const float *PK = p.phk + kvo;
  float *DVG = p.dvg + kvo;
  T *lgs = sm.lg[w];
  float *xp = sm.xp[w], *xq = sm.xq[w], *xk = sm.xk[w];
  f32x4 dS[NFT];  // dS[f = 16 ft + 4 kq + i][dv = dv0 + r]
#pragma unroll
  for (int ft = 0; ft < NFT; ++ft) dS[ft] = f32x4{0.f, 0.f, 0.f, 0.f};
  const F4<T> tri = tri_le<T>(r, kq);
  auto qrow = [&](int g) { return ((size_t)b * p.Hq + hk * G + g) * L * D; };
  // A step's loads: the slice rows (token c0 + r, features 32 w + slot) of log gamma, phi_k and the
  // first query head's phi_q, and this wave's dy column of that head; rows clamped into the
  // sequence (zeroed at use where that matters).  A ring of NPF register sets, each refilled at
  // the end of the step that used it (the loop below is unrolled NPF times).
  struct Buf {
    Frag<T> lg;
    Frag<float> pk, pq;
    Col4<T> dy;
  };
  auto load_step = [&](Buf &bf, int st) {
    const int c0 = max(st, 0) * TS;
    const size_t row = (size_t)min(c0 + r, L - 1) * D;
    bf.lg = row_il(LG + row, w, kq, true);
    bf.pk = row_il(PK + row, w, kq, true);
    bf.pq = row_il(p.phq + qrow(0) + row, w, kq, true);
    bf.dy = col_ld(reinterpret_cast<const T *>(p.dy) + qrow(0), D, c0 + 4 * kq, dv0 + r, L);
  };
  auto load_head = [&](int c0, Frag<float> &pqf, F4<T> &dyc, int g) {
    pqf = row_il(p.phq + qrow(g) + (size_t)(c0 + r) * D, w, kq, c0 + r < L);
    dyc = col_g(reinterpret_cast<const T *>(p.dy) + qrow(g), D, c0 + 4 * kq, dv0 + r, L);
  };
  const int nstep = (L + TS - 1) / TS;
  auto step = [&](Buf &bf, int st) {
    const int c0 = st * TS;
    const bool rok = c0 + r < L;
    // (opaque here, so that the packing and zeroing below stay in this step instead of following
    // the loads, where they would wait for every load in flight)
#pragma unroll
    for (int j = 0; j < 4; ++j) asm volatile("" : "+v"(bf.dy.x[j]));
    opaque_frag(bf.lg);
    opaque_frag(bf.pk);
    opaque_frag(bf.pq);
    F4<T> dyc = col_use(bf.dy, c0 + 4 * kq, L);
    Frag<T> lgf = bf.lg;
    Frag<float> pkf = bf.pk, pqf = bf.pq;
    if (!rok) {  // rows beyond the sequence: no decay, no features
      lgf = frag_zero<T>();
      pkf = frag_zero<float>();
      pqf = frag_zero<float>();
    }
    // ---- the slice's prefix sums (lane (t = r, kq): feature 32 w + 16 h + 4 kq + i) and totals
    store_il(lgs + r * LDL, lgf, 0, kq);
    __builtin_amdgcn_wave_barrier();
    f32x4 pq[2];
    float P[2][4];
    float spn = 0.f;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      pq[h] = mma16(lds_col4(lgs, LDL, 4 * kq, 16 * h), tri, f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        P[h][i] = __shfl(pq[h][i], 15 + 16 * kq);
        spn = fmaxf(spn, -P[h][i]);
      }
    }
    spn = wave_max_all(spn);
    // ---- the slice's operands: Kbar = phi_k e^{P - p}, Ktil = phi_k e^{-p} (used on mild steps
    //      only, where -p <= 60), Qtil = phi_q e^{p} of the first query head, e^{P}; exact-path rows
    {
      float kb[8], kt[8], qt[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int h = j >> 2, i = j & 3;
        const float pv = pq[h][i];
        kb[j] = pkf.v[j] * __expf(P[h][i] - pv);
        kt[j] = pkf.v[j] * __expf(fminf(-pv, MILD_SPAN));
        qt[j] = pqf.v[j] * __expf(pv);
      }
      store_il(sm.kb + r * LD, frag_from<T>(kb), w, kq);
      store_il(sm.kt + r * LD, frag_from<T>(kt), w, kq);
      store_il(sm.qt + r * LD, frag_from<T>(qt), w, kq);
      if (r == 0) {
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int i = 0; i < 4; ++i) sm.ep[32 * w + 16 * h + 4 * kq + i] = __expf(P[h][i]);
      }
      if (lane == 0) sm.span[w] = spn;
    }
    __syncthreads();  // B1: the step's operands visible
    float spall = 0.f;
#pragma unroll
    for (int u = 0; u < NW; ++u) spall = fmaxf(spall, sm.span[u]);
    const bool mild = spall <= MILD_SPAN;
    // ---- inter: dV[s][dv] = sum_f Kbar[s][f] dS[f][dv]  (lane (dv = dv0 + r, kq): s = 4 kq + i)
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      float sb[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) sb[j] = dS[2 * ks + (j >> 2)][j & 3];
      const T *kr = sm.kb + r * LD + 32 * ks + 4 * kq;
      acc = mma(load4x2(kr, kr + 16), frag_from<T>(sb), acc);
    }
    for (int g = 0; g < G; ++g) {
      if (g > 0) {  // this head's Qtil (the previous head's reads ended at its last barrier)
        Frag<float> pqg;
        load_head(c0, pqg, dyc, g);
        float qt[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          qt[j] = pqg.v[j] * __expf(pq[j >> 2][j & 3]);
          xq[r * LDX + 16 * (j >> 2) + 4 * kq + (j & 3)] = pqg.v[j];
        }
        store_il(sm.qt + r * LD, frag_from<T>(qt), w, kq);
        __syncthreads();  // this head's Qtil visible
      }
      // A[t][s] (lane (s = r, kq): t = 4 kq + i), masked to t >= s
      f32x4 a = {0.f, 0.f, 0.f, 0.f};
      if (mild) {
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          const T *qr = sm.qt + r * LD + 32 * ks + 4 * kq, *kr = sm.kt + r * LD + 32 * ks + 4 * kq;
          a = mma(load4x2(qr, qr + 16), load4x2(kr, kr + 16), a);
        }
      } else {
        // exact: A[t][s] = sum_f phi_q[t][f] phi_k[s][f] e^{p_t[f] - p_s[f]}, each wave over its slice
        // (its rows of p, phi_k and phi_q in the wave's own tables, written here: mild steps, the
        // common case, need none of them)
        if (g == 0) {
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const int col = 16 * (j >> 2) + 4 * kq + (j & 3);
            xp[r * LDX + col] = pq[j >> 2][j & 3];
            xk[r * LDX + col] = pkf.v[j];
            xq[r * LDX + col] = pqf.v[j];
          }
        }
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int t = 4 * kq + i;
          float x = 0.f;
          if (t >= r)
            for (int f = 0; f < 32; ++f)
              x += xq[t * LDX + f] * xk[r * LDX + f] * __expf(xp[t * LDX + f] - xp[r * LDX + f]);
          sm.part[w][t * 17 + r] = x;
        }
        __syncthreads();  // the slices' partial scores visible
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float x = 0.f;
#pragma unroll
          for (int u = 0; u < NW; ++u) x += sm.part[u][(4 * kq + i) * 17 + r];
          a[i] = x;
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = (4 * kq + i >= r) ? a[i] : 0.f;
      // dV[s][dv] += sum_t A[t][s] dy_t[dv]
      {
        float x[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) x[i] = a[i];
        acc = mma16(f4_from<T>(x), dyc, acc);
      }
      // dS: decay to the step start (once), then + Qtil^T dY of this head
      if (g == 0) {
#pragma unroll
        for (int ft = 0; ft < NFT; ++ft) {
          const f32x4 e = *reinterpret_cast<const f32x4 *>(sm.ep + 16 * ft + 4 * kq);
#pragma unroll
          for (int i = 0; i < 4; ++i) dS[ft][i] *= e[i];
        }
      }
      // (every fragment read before the first product: one read per product waited for each)
      F4<T> qtf[NFT];
#pragma unroll
      for (int ft = 0; ft < NFT; ++ft) qtf[ft] = lds_col4(sm.qt, LD, 4 * kq, 16 * ft);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int ft = 0; ft < NFT; ++ft) dS[ft] = mma16(qtf[ft], dyc, dS[ft]);
      __syncthreads();  // B2: the step's (head's) operands read before they are rewritten
    }
    // store dV (lane (dv = dv0 + r, kq): s = c0 + 4 kq + i)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int s2 = c0 + 4 * kq + i;
      float *dst = s2 < L ? DVG + (size_t)s2 * D : g_bwd_sink;  // (rows past the end: the sink)
      dst[dv0 + r] = p.mix * acc[i];
    }
    load_step(bf, st - NPF);
  };
  // steps st = nstep - 1 - k for k = 0, 1, ..; ring slot k % NPF
  Buf ring[NPF];
#pragma unroll
  for (int u = 0; u < NPF; ++u) load_step(ring[u], nstep - 1 - u);
  int k = 0;
  for (; k + NPF <= nstep; k += NPF) {
#pragma unroll
    for (int u = 0; u < NPF; ++u) step(ring[u], nstep - 1 - (k + u));
  }
#pragma unroll
  for (int u = 0; u < NPF; ++u)
    if (k + u < nstep) step(ring[u], nstep - 1 - (k + u));
}

// ======================================================================== 4. window, query side
// One wave per (batch, query head, run of QPW 16-query tiles).  Per tile: online max / sum over the
// meta tile and the key tiles of the band, then D_t = sum_j p dp, ds = p (dp - D_t),
// dq_t = scale sum_j ds K_j; the meta keys' and values' gradients accumulate over the run.
// Logit layout: lane (t = r, kq) holds s[j = 16 u + 4 kq + i][t].
template <typename T, int D> struct WinQLds {
  static constexpr int LD = D + 8;
  T k[TS * LD];    // the key tile (or meta keys), rows
  T q[TS * LD];    // the query tile, rows
  T dy[TS * LD];   // (1 - mix) dy of the query tile, rows
  T pm[TS * 20];   // meta probabilities [m][t]
  T dm[TS * 20];   // meta ds [m][t]
  f32x4 cache[6][2][64];  // per lane: logits and dots of the first 6 tiles of a query row
};

template <typename T, int D>
__global__ __launch_bounds__(64) void bwd_win_q_kernel(BwdParams p) {
  constexpr int NDT = D / 16, KS = D / 32, LD = WinQLds<T, D>::LD;
  __shared__ WinQLds<T, D> sm;
  const int lane = threadIdx.x & 63, r = lane & 15, kq = lane >> 4;
  const int L = p.L, W = p.W, M = p.M;
  const int ntile = (L + TS - 1) / TS, nrun = (ntile + QPW - 1) / QPW;
  const int bh = blockIdx.x / nrun, run = blockIdx.x % nrun;
  const int b = bh / p.Hq, hq = bh % p.Hq, hk = hq / p.G;
  const size_t kvo = ((size_t)b * p.Hkv + hk) * L * D, qo = (size_t)bh * L * D;
  const T *K = reinterpret_cast<const T *>(p.k) + kvo;
  const T *V = reinterpret_cast<const T *>(p.v) + kvo;
  const T *Q = reinterpret_cast<const T *>(p.q) + qo;
  const T *DY = reinterpret_cast<const T *>(p.dy) + qo;
  const T *TK = reinterpret_cast<const T *>(p.tk) + (size_t)hk * M * D;
  const T *TV = reinterpret_cast<const T *>(p.tv) + (size_t)hk * M * D;
  const float sl = p.scale, wmix = 1.f - p.mix;
  f32x4 dtk[NDT], dtv[NDT];  // meta gradients (m = 4 kq + i, e = 16 et + r)
#pragma unroll
  for (int et = 0; et < NDT; ++et) { dtk[et] = f32x4{0.f, 0.f, 0.f, 0.f}; dtv[et] = f32x4{0.f, 0.f, 0.f, 0.f}; }
  Frag<T> tkf[KS], tvf[KS];  // meta keys / values as rows m = r
#pragma unroll
  for (int j = 0; j < KS; ++j) {
    tkf[j] = row_nat(TK + (size_t)r * D, j, kq, r < M);
    tvf[j] = row_nat(TV + (size_t)r * D, j, kq, r < M);
  }
  for (int qt = run * QPW; qt < min(ntile, (run + 1) * QPW); ++qt) {
    const int t0 = qt * TS, t = t0 + r;
    const bool tok = t < L;
    const int jlo = max(0, t0 - W + 1), ulo = jlo / TS, uhi = qt;
    // Loads first, all in flight together: the query and dy rows, then (when the band has at most
    // NB key tiles) every key and value tile of the band, rows clamped into the sequence (rows at
    // or beyond L are masked or weighted by zero).  A band of more tiles loads each as it goes.
    const bool batched = uhi - ulo + 1 <= NB;
    Frag<T> qf[KS], dyf[KS];
#pragma unroll
    for (int j = 0; j < KS; ++j) {
      qf[j] = row_nat(Q + (size_t)t * D, j, kq, tok);
      dyf[j] = row_nat(DY + (size_t)t * D, j, kq, tok);
    }
    Frag<T> kb[NB][KS], vb[NB][KS];
    if (batched) {
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        const size_t jr = (size_t)min(TS * min(ulo + i, uhi) + r, L - 1) * D;
#pragma unroll
        for (int j = 0; j < KS; ++j) {
          kb[i][j] = load8(K + jr + 32 * j + 8 * kq);
          vb[i][j] = load8(V + jr + 32 * j + 8 * kq);
        }
      }
    }
#pragma unroll
    for (int j = 0; j < KS; ++j) {
      float x[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = wmix * to_f(dyf[j].v[e]);
      dyf[j] = frag_from<T>(x);
      *reinterpret_cast<Frag<T> *>(sm.q + r * LD + 32 * j + 8 * kq) = qf[j];
      *reinterpret_cast<Frag<T> *>(sm.dy + r * LD + 32 * j + 8 * kq) = dyf[j];
    }
    // logits of tile u (u = -1: meta) from its key fragments, masked
    auto logits_f = [&](int u, const Frag<T> (&kf)[KS], f32x4 &s) {
      s = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < KS; ++j) s = mma(kf[j], qf[j], s);
      if (u < 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) s[i] = (4 * kq + i < M) ? s[i] * sl : -1.0e30f;
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int jj = TS * u + 4 * kq + i;
          s[i] = (jj <= t && jj > t - W && jj < L) ? s[i] * sl : -1.0e30f;
        }
      }
    };
    auto dots_f = [&](const Frag<T> (&vf)[KS], f32x4 &dp) {  // dp[j][t] = v_j . dy_w[t]
      dp = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < KS; ++j) dp = mma(vf[j], dyf[j], dp);
    };
    auto load_tile = [&](const T *X, int u, Frag<T> (&f)[KS]) {  // key or value tile u, rows r
      const int jr = TS * u + r;
#pragma unroll
      for (int j = 0; j < KS; ++j) f[j] = row_nat(X + (size_t)jr * D, j, kq, jr < L);
    };
    // tiles of the row: k = 0 the meta tile, k >= 1 key tile ulo + k - 1; the first NC tiles keep
    // their logits and dots (in lane-private LDS) for the second pass
    constexpr int NC = 6;
    static_assert(NB + 1 <= NC, "a batched band's tiles all keep their logits and dots");
    const int ntl = 2 + uhi - ulo;
    auto tile_of = [&](int k) { return k == 0 ? -1 : ulo + k - 1; };
    // pass 1 (online): row max, sum of e^{s - max}, and sum of e^{s - max} dp, rescaled as the max grows
    float mx = -1.0e30f, sum = 0.f, dnum = 0.f;
    auto online = [&](const f32x4 &sv, const f32x4 &dv) {
      float m2 = fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3]));
      m2 = fmaxf(mx, wave_max_cols(m2));
      const float al = __expf(mx - m2);
      sum *= al;
      dnum *= al;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float e = (sv[i] > -1.0e29f) ? __expf(sv[i] - m2) : 0.f;
        sum += e;
        dnum += e * dv[i];
      }
      mx = m2;
    };
    auto pass1 = [&](int k, const Frag<T> (&kf)[KS], const Frag<T> (&vf)[KS]) {
      f32x4 sv, dv;
      logits_f(tile_of(k), kf, sv);
      dots_f(vf, dv);
      online(sv, dv);
      if (k < NC) {
        sm.cache[k][0][lane] = sv;
        sm.cache[k][1][lane] = dv;
      }
    };
    pass1(0, tkf, tvf);
    if (batched) {
#pragma unroll
      for (int k = 1; k <= NB; ++k)
        if (k < ntl) pass1(k, kb[k - 1], vb[k - 1]);
    } else {
      for (int k = 1; k < ntl; ++k) {
        Frag<T> kf[KS], vf[KS];
        load_tile(K, tile_of(k), kf);
        load_tile(V, tile_of(k), vf);
        pass1(k, kf, vf);
      }
    }
    sum = wave_sum_cols(sum);
    const float inv = 1.f / sum;
    const float dsum = wave_sum_cols(dnum) * inv;  // D_t = sum_j p dp
    if (tok) {
      float *st = p.wstat + ((size_t)bh * L + t) * 4;
      if (kq == 0) *reinterpret_cast<f32x4 *>(st) = f32x4{mx, inv, dsum, 0.f};
    }
    // pass 2: ds, dq, meta gradients
    f32x4 dq[NDT];  // lane (e = 16 et + r, kq): t = 4 kq + i
#pragma unroll
    for (int et = 0; et < NDT; ++et) dq[et] = f32x4{0.f, 0.f, 0.f, 0.f};
    auto backprop = [&](int u, const f32x4 &sv, const f32x4 &dv, const Frag<T> (&kf)[KS]) {
      float pr[4], ds[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pr[i] = (sv[i] > -1.0e29f) ? __expf(sv[i] - mx) * inv : 0.f;
        ds[i] = pr[i] * (dv[i] - dsum);
      }
      // the key tile's rows into LDS for the transposed operand
#pragma unroll
      for (int j = 0; j < KS; ++j) *reinterpret_cast<Frag<T> *>(sm.k + r * LD + 32 * j + 8 * kq) = kf[j];
      __syncthreads();
      // dq[t][e] += scale sum_j ds[t][j] K[j][e]: A = ds (lane (t = r, kq): j = 4 kq + i)
      const F4<T> dsa = f4_from<T>(ds);
#pragma unroll
      for (int et = 0; et < NDT; ++et) dq[et] = mma16(dsa, lds_col4(sm.k, LD, 4 * kq, 16 * et), dq[et]);
      if (u < 0 && M > 0) {
        // meta: dTk[m][e] += scale sum_t ds[m][t] q_t[e], dTv[m][e] += sum_t p[m][t] dyw_t[e]
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          sm.dm[(4 * kq + i) * 20 + r] = from_f<T>(ds[i]);
          sm.pm[(4 * kq + i) * 20 + r] = from_f<T>(pr[i]);
        }
        __syncthreads();
        F4<T> da, pa;  // rows m = r, t = 4 kq + j
#pragma unroll
        for (int j = 0; j < 4; ++j) { da.v[j] = sm.dm[r * 20 + 4 * kq + j]; pa.v[j] = sm.pm[r * 20 + 4 * kq + j]; }
#pragma unroll
        for (int et = 0; et < NDT; ++et) {
          dtk[et] = mma16(da, lds_col4(sm.q, LD, 4 * kq, 16 * et), dtk[et]);
          dtv[et] = mma16(pa, lds_col4(sm.dy, LD, 4 * kq, 16 * et), dtv[et]);
        }
      }
      __syncthreads();
    };
    backprop(-1, sm.cache[0][0][lane], sm.cache[0][1][lane], tkf);
    if (batched) {
#pragma unroll
      for (int k = 1; k <= NB; ++k)
        if (k < ntl) backprop(tile_of(k), sm.cache[k][0][lane], sm.cache[k][1][lane], kb[k - 1]);
    } else {
      for (int k = 1; k < ntl; ++k) {
        f32x4 sv, dv;
        Frag<T> kf[KS];
        load_tile(K, tile_of(k), kf);
        if (k < NC) {
          sv = sm.cache[k][0][lane];
          dv = sm.cache[k][1][lane];
        } else {
          Frag<T> vf[KS];
          load_tile(V, tile_of(k), vf);
          logits_f(tile_of(k), kf, sv);
          dots_f(vf, dv);
        }
        backprop(tile_of(k), sv, dv, kf);
      }
    }
    T *DQW = reinterpret_cast<T *>(p.dqw) + qo;  // the window part, in the input type
#pragma unroll
    for (int et = 0; et < NDT; ++et)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tt = t0 + 4 * kq + i;
        if (tt < L) DQW[(size_t)tt * D + 16 * et + r] = from_f<T>(sl * dq[et][i]);
      }
  }
  if (M > 0) {
    float *PT = p.dtk_part + (size_t)blockIdx.x * 16 * D;
    float *PV = p.dtv_part + (size_t)blockIdx.x * 16 * D;
#pragma unroll
    for (int et = 0; et < NDT; ++et)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        PT[(4 * kq + i) * D + 16 * et + r] = sl * dtk[et][i];
        PV[(4 * kq + i) * D + 16 * et + r] = dtv[et][i];
      }
  }
}

// ======================================================================== 5. window, key side
// Workgroups of four waves per (batch, key/value head, run of four 16-key tiles), wave w taking
// key tile 4 run + w: for every query head of the group and every query tile that sees these keys,
// p from the stored statistics, ds = p (dp - D_t), then dk_j += scale sum_t ds[t][j] q_t and
// dv_j += sum_t p[t][j] dyw_t.  The query tiles the run's keys see (eight for W <= 65) are loaded
// once per workgroup -- query rows, (1 - mix) dy rows and statistics, every load in flight
// together -- into LDS, where every wave reads its operands; a longer band goes in windows of
// eight tiles.
// Logit layout: lane (j = r, kq) holds s[t = 16 u + 4 kq + i][j].
constexpr int WKQ = 8;  // query tiles per window of the window-k kernel
template <typename T, int D> struct WinKLds {
  static constexpr int LD = D + 16 / (int)sizeof(T);
  T q[WKQ][TS * LD], dy[WKQ][TS * LD];
  f32x4 st[WKQ][TS];  // (max, 1 / sum, D_t) of the window's query rows
};

template <typename T, int D>
__global__ __launch_bounds__(256) void bwd_win_k_kernel(BwdParams p) {
  using SM = WinKLds<T, D>;
  constexpr int NDT = D / 16, KS = D / 32, LD = SM::LD;
  constexpr int RP = D * (int)sizeof(T) / 16;      // 16-byte pieces per row
  constexpr int EP = 16 / (int)sizeof(T);          // elements per piece
  constexpr int NPW = WKQ * TS * RP;               // pieces per window and tensor
  static_assert(NPW % 256 == 0, "pieces per thread");
  constexpr int PPT = NPW / 256;
  extern __shared__ __attribute__((aligned(16))) char smem_k[];
  SM &sm = *reinterpret_cast<SM *>(smem_k);
  const int tid = threadIdx.x, lane = tid & 63, r = lane & 15, kq = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int L = p.L, W = p.W, G = p.G;
  const int ntile = (L + TS - 1) / TS, nrun = (ntile + 3) / 4;
  const int bh = blockIdx.x / nrun, run = blockIdx.x % nrun;
  const int b = bh / p.Hkv, hk = bh % p.Hkv;
  const size_t kvo = (size_t)bh * L * D;
  const T *K = reinterpret_cast<const T *>(p.k) + kvo;
  const T *V = reinterpret_cast<const T *>(p.v) + kvo;
  const int kt = 4 * run + w, j0 = kt * TS, j = j0 + r;
  const bool kin = kt < ntile;  // waves past the last key tile take part in the loads and barriers
  Frag<T> kf[KS], vf[KS];
#pragma unroll
  for (int x = 0; x < KS; ++x) {
    kf[x] = row_nat(K + (size_t)j * D, x, kq, j < L);
    vf[x] = row_nat(V + (size_t)j * D, x, kq, j < L);
  }
  const float sl = p.scale, wmix = 1.f - p.mix;
  f32x4 dk[NDT], dv[NDT];  // lane (e = 16 et + r, kq): j = 4 kq + i
#pragma unroll
  for (int et = 0; et < NDT; ++et) { dk[et] = f32x4{0.f, 0.f, 0.f, 0.f}; dv[et] = f32x4{0.f, 0.f, 0.f, 0.f}; }
  const int uhi = min(ntile - 1, (j0 + TS - 1 + W - 1) / TS);  // this wave's last query tile
  const int k0 = 4 * run;                                       // the run's first key tile
  const int uend = min(ntile - 1, (min(4 * run + 3, ntile - 1) * TS + TS - 1 + W - 1) / TS);
  for (int g = 0; g < G; ++g) {
    const int hq = hk * G + g;
    const size_t qo = ((size_t)b * p.Hq + hq) * L * D;
    const T *Q = reinterpret_cast<const T *>(p.q) + qo;
    const T *DY = reinterpret_cast<const T *>(p.dy) + qo;
    const float *ST = p.wstat + ((size_t)b * p.Hq + hq) * L * 4;
    for (int u0 = k0; u0 <= uend; u0 += WKQ) {
      // the window's query tiles u0 .. u0 + WKQ - 1 into LDS, rows clamped into the sequence
      u32x4 qa[PPT], da[PPT];
      f32x4 sa = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < PPT; ++i) {
        const int pc = tid + 256 * i, row = pc / RP, col = (pc % RP) * EP;
        const size_t o = (size_t)min(u0 * TS + row, L - 1) * D + col;
        qa[i] = *reinterpret_cast<const u32x4 *>(Q + o);
        da[i] = *reinterpret_cast<const u32x4 *>(DY + o);
      }
      if (tid < WKQ * TS) sa = *reinterpret_cast<const f32x4 *>(ST + (size_t)min(u0 * TS + tid, L - 1) * 4);
      __syncthreads();  // the previous window's tiles are no longer read
#pragma unroll
      for (int i = 0; i < PPT; ++i) {
        const int pc = tid + 256 * i, row = pc / RP, col = (pc % RP) * EP;
        T *qd = sm.q[row / TS] + (row % TS) * LD + col, *dd = sm.dy[row / TS] + (row % TS) * LD + col;
        *reinterpret_cast<u32x4 *>(qd) = qa[i];
        const T *dsrc = reinterpret_cast<const T *>(&da[i]);
        T sc[EP];
#pragma unroll
        for (int e = 0; e < EP; ++e) sc[e] = from_f<T>(wmix * to_f(dsrc[e]));
        *reinterpret_cast<u32x4 *>(dd) = *reinterpret_cast<const u32x4 *>(sc);
      }
      if (tid < WKQ * TS) sm.st[tid / TS][tid % TS] = sa;
      __syncthreads();  // the window's tiles visible
      if (kin) {
        for (int u = max(u0, kt); u <= min(u0 + WKQ - 1, uhi); ++u) {
          const T *tq = sm.q[u - u0], *tdy = sm.dy[u - u0];
          Frag<T> qf[KS], dyf[KS];
#pragma unroll
          for (int x = 0; x < KS; ++x) {
            qf[x] = load8(tq + r * LD + 32 * x + 8 * kq);
            dyf[x] = load8(tdy + r * LD + 32 * x + 8 * kq);
          }
          f32x4 s = {0.f, 0.f, 0.f, 0.f}, dp = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int x = 0; x < KS; ++x) {
            s = mma(qf[x], kf[x], s);   // s[t][j]: lane (j = r, kq) t = 4 kq + i
            dp = mma(dyf[x], vf[x], dp);
          }
          float ds[4], pr[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int t = u * TS + 4 * kq + i;
            const bool ok = t < L && j < L && j <= t && j > t - W;
            const f32x4 stt = sm.st[u - u0][4 * kq + i];
            pr[i] = ok ? __expf(s[i] * sl - stt[0]) * stt[1] : 0.f;
            ds[i] = pr[i] * (dp[i] - (ok ? stt[2] : 0.f));
          }
          const F4<T> dsa = f4_from<T>(ds), pa = f4_from<T>(pr);
#pragma unroll
          for (int et = 0; et < NDT; ++et) {
            dk[et] = mma16(dsa, lds_col4(tq, LD, 4 * kq, 16 * et), dk[et]);
            dv[et] = mma16(pa, lds_col4(tdy, LD, 4 * kq, 16 * et), dv[et]);
          }
        }
      }
    }
  }
  if (!kin) return;
  // dk's window part for the feature-map backward; dv = the recurrence's part (role V, already in
  // the workspace) + the window's, final here
  T *DKW = reinterpret_cast<T *>(p.dkw) + kvo;  // the window part, in the input type
  const float *DVG = p.dvg + kvo;
  T *DV = reinterpret_cast<T *>(p.dvo) + kvo;
  float g4[NDT][4];
#pragma unroll
  for (int et = 0; et < NDT; ++et)
#pragma unroll
    for (int i = 0; i < 4; ++i) g4[et][i] = DVG[(size_t)min(j0 + 4 * kq + i, L - 1) * D + 16 * et + r];
#pragma unroll
  for (int et = 0; et < NDT; ++et)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int jj = j0 + 4 * kq + i;
      if (jj < L) {
        DKW[(size_t)jj * D + 16 * et + r] = from_f<T>(sl * dk[et][i]);
        DV[(size_t)jj * D + 16 * et + r] = from_f<T>(g4[et][i] + dv[et][i]);
      }
    }
}

// ======================================================================== 6. feature-map backward
// One block (4 waves) per (batch, head, run of FB_CHUNKS 64-row chunks) of the query side (first
// B*Hq*nsplit blocks) or the key side.  Per chunk: dz = phi (dphi - <phi, dphi>) (softmax) or
// phi_j dphi_j - phi_{h+j} dphi_{h+j} (Hedgehog), dx = dz W^T + window part; the dW partial sum
// sum_t x_t^T dz_t accumulates over the run in registers (wave w: rows 16 (NIT w) .. of W) and is
// written per block.
template <typename T, int D, bool HH>
__global__ __launch_bounds__(256) void bwd_fb_kernel(BwdParams p) {
  constexpr int KS = D / 32, FC = HH ? D / 2 : D, NCT = FC / 16, NIT = D / 64, LDW = FC + 16 / (int)sizeof(T);
  constexpr int LDX = D + 8, LDZ = FC + 8;
  __shared__ __align__(16) T sW[D * LDW];   // W [i][c] rows
  __shared__ __align__(16) T sX[64 * LDX];  // x rows of the chunk
  __shared__ __align__(16) T sZ[64 * LDZ];  // dz rows of the chunk
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, r = lane & 15, kq = lane >> 4;
  const int L = p.L;
  const int nsplit = (L + 64 * FB_CHUNKS - 1) / (64 * FB_CHUNKS);
  const bool qside = (int)blockIdx.x < p.B * p.Hq * nsplit;
  const int bid = qside ? blockIdx.x : blockIdx.x - p.B * p.Hq * nsplit;
  const int bh = bid / nsplit, split = bid % nsplit;
  const int H = qside ? p.Hq : p.Hkv, h = bh % H;
  const T *Wsrc = reinterpret_cast<const T *>(qside ? p.wq : p.wk) + (size_t)h * p.w_stride;
  for (int idx = tid; idx < D * FC; idx += 256) sW[(idx / FC) * LDW + idx % FC] = Wsrc[idx];
  const size_t o = (size_t)bh * L * D;
  const T *X = reinterpret_cast<const T *>(qside ? p.q : p.k) + o;
  const float *PH = (qside ? p.phq : p.phk) + o;
  const float *DPH = (qside ? p.dphq : p.dphk) + o;
  const T *DXW = reinterpret_cast<const T *>(qside ? p.dqw : p.dkw) + o;
  T *DX = reinterpret_cast<T *>(qside ? p.dq : p.dk) + o;
  f32x4 dw[NIT][NCT];  // dW[i = 16 (NIT w + it) + 4 kq + ii][c = 16 ct + r]
#pragma unroll
  for (int it = 0; it < NIT; ++it)
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) dw[it][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
  __syncthreads();
  for (int c0 = 64 * FB_CHUNKS * split; c0 < min(L, 64 * FB_CHUNKS * (split + 1)); c0 += 64) {
    const int t = c0 + 16 * w + r;
    const bool tok = t < L;
    // the window part of dx for row t (four consecutive columns per lane and 16-column tile), its
    // loads issued first so that they are in flight while dz and its products are computed
    F4<T> xw[D / 16];
#pragma unroll
    for (int it = 0; it < D / 16; ++it) xw[it] = ld_f4(DXW + (size_t)min(t, L - 1) * D + 16 * it + 4 * kq);
    // phi and dphi of row t, natural columns 32 ks + 8 kq .. + 7
    float ph[KS][8], dph[KS][8];
    float dot = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const Frag<float> f = row_nat(PH + (size_t)t * D, ks, kq, tok);
      const Frag<float> df = row_nat(DPH + (size_t)t * D, ks, kq, tok);
      const Frag<T> xf = row_nat(X + (size_t)t * D, ks, kq, tok);
      *reinterpret_cast<Frag<T> *>(sX + (16 * w + r) * LDX + 32 * ks + 8 * kq) = xf;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        ph[ks][e] = f.v[e];
        dph[ks][e] = df.v[e];
        dot += ph[ks][e] * dph[ks][e];
      }
    }
    // dz rows (natural columns of W's FC columns)
    Frag<T> dzf[FC / 32];
    if constexpr (HH) {
#pragma unroll
      for (int ks = 0; ks < FC / 32; ++ks) {
        float z[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) z[e] = ph[ks][e] * dph[ks][e] - ph[ks + FC / 32][e] * dph[ks + FC / 32][e];
        dzf[ks] = frag_from<T>(z);
      }
    } else {
      dot = wave_sum_cols(dot);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        float z[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) z[e] = ph[ks][e] * (dph[ks][e] - dot);
        dzf[ks] = frag_from<T>(z);
      }
    }
#pragma unroll
    for (int ks = 0; ks < FC / 32; ++ks) *reinterpret_cast<Frag<T> *>(sZ + (16 * w + r) * LDZ + 32 * ks + 8 * kq) = dzf[ks];
    // dx[t][i] = sum_c W[i][c] dz[t][c] (lane (t = 16 w + r, kq): i = 16 it + 4 kq + ii, four
    // consecutive columns of row t per lane: one 8-byte store, one 16-byte load of the window part)
#pragma unroll
    for (int it = 0; it < D / 16; ++it) {
      f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < FC / 32; ++ks) a = mma(load8(sW + (16 * it + r) * LDW + 32 * ks + 8 * kq), dzf[ks], a);
      if (tok) {
        const size_t off = (size_t)t * D + 16 * it + 4 * kq;
        store4<T>(DX + off, a[0] + f4_at(xw[it], 0), a[1] + f4_at(xw[it], 1), a[2] + f4_at(xw[it], 2),
                  a[3] + f4_at(xw[it], 3));
      }
    }
    __syncthreads();  // x and dz rows of the chunk staged
    // dW[i][c] += sum_t x[t][i] dz[t][c]: K = 64 rows in 16-row steps
#pragma unroll
    for (int k4 = 0; k4 < 4; ++k4) {
      F4<T> za[NCT];
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) za[ct] = lds_col4(sZ, LDZ, 16 * k4 + 4 * kq, 16 * ct);
#pragma unroll
      for (int it = 0; it < NIT; ++it) {
        const F4<T> xa = lds_col4(sX, LDX, 16 * k4 + 4 * kq, 16 * (NIT * w + it));
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) dw[it][ct] = mma16(xa, za[ct], dw[it][ct]);
      }
    }
    __syncthreads();
  }
  float *part = p.dw_part + (size_t)blockIdx.x * D * FC;
#pragma unroll
  for (int it = 0; it < NIT; ++it)
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) part[(size_t)(16 * (NIT * w + it) + 4 * kq + ii) * FC + 16 * ct + r] = dw[it][ct][ii];
}

// The same for bf16 inputs, with phi recomputed from x and W_phi instead of read in fp32 (a quarter
// less traffic): the logits taken transposed, z^T = W^T x^T, with the A operand read from W's rows
// in LDS by transposed reads and x as the B operand as loaded, so that lane (r, kq) holds row r's
// features 16 c + 4 kq + i; dphi is loaded in that order, and dz enters dx = dz W^T with K in the
// interleaved order (the W rows read in two 8-byte pieces to match).  The feature map repeats
// bwd_phi_kernel's arithmetic: fp32 logits from the same bf16 products, max subtracted, one
// normaliser.
template <int D, bool HH>
__global__ __launch_bounds__(256) void bwd_fb_b16_kernel(BwdParams p) {
  using T = bf16;
  constexpr int KS = D / 32, FC = HH ? D / 2 : D, NCT = FC / 16, NC = D / 16, NIT = D / 64;
  constexpr int LDW = FC + 8, LDX = D + 8, LDZ = FC + 8;  // 8-byte reads: odd multiples of 16 bytes
  __shared__ __align__(16) T sW[D * LDW];   // W [i][c] rows
  __shared__ __align__(16) T sX[64 * LDX];  // x rows of the chunk
  __shared__ __align__(16) T sZ[64 * LDZ];  // dz rows of the chunk
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, r = lane & 15, kq = lane >> 4;
  const int L = p.L;
  const int nsplit = (L + 64 * FB_CHUNKS - 1) / (64 * FB_CHUNKS);
  const bool qside = (int)blockIdx.x < p.B * p.Hq * nsplit;
  const int bid = qside ? blockIdx.x : blockIdx.x - p.B * p.Hq * nsplit;
  const int bh = bid / nsplit, split = bid % nsplit;
  const int H = qside ? p.Hq : p.Hkv, h = bh % H;
  const T *Wsrc = reinterpret_cast<const T *>(qside ? p.wq : p.wk) + (size_t)h * p.w_stride;
  for (int idx = tid; idx < D * FC / 8; idx += 256)
    *reinterpret_cast<Frag<T> *>(sW + (idx / (FC / 8)) * LDW + 8 * (idx % (FC / 8))) = load8(Wsrc + 8 * (size_t)idx);
  const size_t o = (size_t)bh * L * D;
  const T *X = reinterpret_cast<const T *>(qside ? p.q : p.k) + o;
  const float *DPH = (qside ? p.dphq : p.dphk) + o;
  const T *DXW = reinterpret_cast<const T *>(qside ? p.dqw : p.dkw) + o;
  T *DX = reinterpret_cast<T *>(qside ? p.dq : p.dk) + o;
  f32x4 dw[NIT][NCT];  // dW[i = 16 (NIT w + it) + 4 kq + ii][c = 16 ct + r]
#pragma unroll
  for (int it = 0; it < NIT; ++it)
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) dw[it][ct] = f32x4{0.f, 0.f, 0.f, 0.f};
  __syncthreads();
  for (int c0 = 64 * FB_CHUNKS * split; c0 < min(L, 64 * FB_CHUNKS * (split + 1)); c0 += 64) {
    const int t = c0 + 16 * w + r;
    const bool tok = t < L;
    const size_t trow = (size_t)min(t, L - 1) * D;
    // the window part of dx, x and dphi of row t (clamped into the sequence; zeroed below past it)
    F4<T> xw[D / 16];
#pragma unroll
    for (int it = 0; it < D / 16; ++it) xw[it] = ld_f4(DXW + trow + 16 * it + 4 * kq);
    Frag<T> xf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) xf[ks] = tok ? load8(X + trow + 32 * ks + 8 * kq) : frag_zero<T>();
    f32x4 dpv[NC];  // dphi[t][16 c + 4 kq + i]
#pragma unroll
    for (int c = 0; c < NC; ++c) dpv[c] = *reinterpret_cast<const f32x4 *>(DPH + trow + 16 * c + 4 * kq);
    // logits: z[c][i] = (x W)[t][16 c + 4 kq + i]
    f32x4 z[NCT];
#pragma unroll
    for (int c = 0; c < NCT; ++c) {
      f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const F4<T> lo = lds_col4(sW, LDW, 32 * ks + 8 * kq, 16 * c), hi = lds_col4(sW, LDW, 32 * ks + 8 * kq + 4, 16 * c);
        Frag<T> wa;
        wa.v = __builtin_shufflevector(lo.v, hi.v, 0, 1, 2, 3, 4, 5, 6, 7);
        a = mma(wa, xf[ks], a);
      }
      z[c] = a;
    }
    // dz of row t, features 16 c + 4 kq + i (zero past the sequence)
    float dz[NCT][4];
    if constexpr (HH) {
#pragma unroll
      for (int c = 0; c < NCT; ++c)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          dz[c][i] = exp2_fast(z[c][i] * LOG2E) * dpv[c][i] - exp2_fast(-z[c][i] * LOG2E) * dpv[NCT + c][i];
    } else {
      float m = z[0][0];
#pragma unroll
      for (int c = 0; c < NCT; ++c)
#pragma unroll
        for (int i = 0; i < 4; ++i) m = fmaxf(m, z[c][i]);
      const float zm2 = -wave_max_cols(m) * LOG2E;
      float ph[NCT][4], sum = 0.f;
#pragma unroll
      for (int c = 0; c < NCT; ++c)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          ph[c][i] = exp2_fast(__builtin_fmaf(z[c][i], LOG2E, zm2));
          sum += ph[c][i];
        }
      const float inv = 1.f / wave_sum_cols(sum);
      float dot = 0.f;
#pragma unroll
      for (int c = 0; c < NCT; ++c)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          ph[c][i] *= inv;
          dot += ph[c][i] * dpv[c][i];
        }
      dot = wave_sum_cols(dot);
#pragma unroll
      for (int c = 0; c < NCT; ++c)
#pragma unroll
        for (int i = 0; i < 4; ++i) dz[c][i] = ph[c][i] * (dpv[c][i] - dot);
    }
    if (!tok) {
#pragma unroll
      for (int c = 0; c < NCT; ++c)
#pragma unroll
        for (int i = 0; i < 4; ++i) dz[c][i] = 0.f;
    }
    // dz operands in the interleaved K order (slots 0..3: tile 2 ks, 4..7: tile 2 ks + 1), and the
    // dz rows into LDS in natural order for dW
    Frag<T> dzf[FC / 32];
#pragma unroll
    for (int ks = 0; ks < FC / 32; ++ks) {
      float y[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        y[i] = dz[2 * ks][i];
        y[4 + i] = dz[2 * ks + 1][i];
      }
      dzf[ks] = frag_from<T>(y);
    }
#pragma unroll
    for (int c = 0; c < NCT; ++c) store4<T>(sZ + (16 * w + r) * LDZ + 16 * c + 4 * kq, dz[c][0], dz[c][1], dz[c][2], dz[c][3]);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) *reinterpret_cast<Frag<T> *>(sX + (16 * w + r) * LDX + 32 * ks + 8 * kq) = xf[ks];
    // dx[t][i] = sum_c W[i][c] dz[t][c] (lane (t = 16 w + r, kq): i = 16 it + 4 kq + ii)
#pragma unroll
    for (int it = 0; it < D / 16; ++it) {
      f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < FC / 32; ++ks) {
        const T *wr = sW + (16 * it + r) * LDW + 32 * ks + 4 * kq;
        a = mma(load4x2(wr, wr + 16), dzf[ks], a);
      }
      if (tok) {
        const size_t off = (size_t)t * D + 16 * it + 4 * kq;
        store4<T>(DX + off, a[0] + f4_at(xw[it], 0), a[1] + f4_at(xw[it], 1), a[2] + f4_at(xw[it], 2),
                  a[3] + f4_at(xw[it], 3));
      }
    }
    __syncthreads();  // x and dz rows of the chunk staged
    // dW[i][c] += sum_t x[t][i] dz[t][c]: K = 64 rows in 16-row steps
#pragma unroll
    for (int k4 = 0; k4 < 4; ++k4) {
      F4<T> za[NCT];
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) za[ct] = lds_col4(sZ, LDZ, 16 * k4 + 4 * kq, 16 * ct);
#pragma unroll
      for (int it = 0; it < NIT; ++it) {
        const F4<T> xa = lds_col4(sX, LDX, 16 * k4 + 4 * kq, 16 * (NIT * w + it));
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) dw[it][ct] = mma16(xa, za[ct], dw[it][ct]);
      }
    }
    __syncthreads();
  }
  float *part = p.dw_part + (size_t)blockIdx.x * D * FC;
#pragma unroll
  for (int it = 0; it < NIT; ++it)
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) part[(size_t)(16 * (NIT * w + it) + 4 * kq + ii) * FC + 16 * ct + r] = dw[it][ct][ii];
}

// ======================================================================== 7. reductions
// dW_q (and dW_k): sum of the per-block partials over the heads that share a matrix, in two stages
// with a fixed order (deterministic): stage 0 sums the partials of group g (partial index % RG == g)
// into tmp[g], stage 1 sums tmp over the groups.  dT_k, dT_v (stage 1): sum of the window-q
// partials of the key/value head's query heads.
constexpr int RG = 32;
__global__ __launch_bounds__(256) void bwd_reduce_kernel(BwdParams p, int D, int FC, int stage) {
  const size_t wsz = (size_t)D * FC;
  const int nwq = p.w_stride ? p.Hq : 1, nwk = p.w_stride ? p.Hkv : 1;
  const size_t nw = (size_t)(nwq + nwk) * wsz;
  const int ntile = (p.L + TS - 1) / TS, nrun = (ntile + QPW - 1) / QPW;
  const int nsplit = (p.L + 64 * FB_CHUNKS - 1) / (64 * FB_CHUNKS);
  const size_t nt = p.M > 0 ? (size_t)p.Hkv * p.M * D : 0;
  if (stage == 0) {
    const size_t x = (size_t)blockIdx.x * 256 + threadIdx.x;
    const int grp = blockIdx.y;
    if (x >= nw) return;
    const bool qs = x < (size_t)nwq * wsz;
    const size_t y = qs ? x : x - (size_t)nwq * wsz;
    const int mat = (int)(y / wsz);
    const size_t e = y % wsz;
    const int H = qs ? p.Hq : p.Hkv;
    const size_t base = qs ? 0 : (size_t)p.B * p.Hq * nsplit;
    const int hlo = p.w_stride ? mat : 0, per = p.w_stride ? 1 : H;  // heads that share the matrix
    // The partials of this output element in the order (batch, head, split), index idx; group grp
    // sums those with idx % RG == grp in increasing idx, four loads in flight at a time.
    const int total = p.B * per * nsplit;
    auto part = [&](int idx) {
      const int sp = idx % nsplit, bh = idx / nsplit, b = bh / per, h = hlo + bh % per;
      return p.dw_part[(base + ((size_t)b * H + h) * nsplit + sp) * wsz + e];
    };
    float acc = 0.f;
    int idx = grp;
    for (; idx + 3 * RG < total; idx += 4 * RG) {
      float v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) v[u] = part(idx + u * RG);
#pragma unroll
      for (int u = 0; u < 4; ++u) acc += v[u];
    }
    for (; idx < total; idx += RG) acc += part(idx);
    p.dw_tmp[(size_t)grp * nw + x] = acc;
    return;
  }
  for (size_t x = (size_t)blockIdx.x * 256 + threadIdx.x; x < nw + 2 * nt; x += (size_t)gridDim.x * 256) {
    if (x < nw) {
      float acc = 0.f;
      for (int g = 0; g < RG; ++g) acc += p.dw_tmp[(size_t)g * nw + x];
      if (x < (size_t)nwq * wsz) p.dwq[x] = acc;
      else p.dwk[x - (size_t)nwq * wsz] = acc;
    } else {
      const size_t y = x - nw;
      const bool kpart = y < nt;
      const size_t z = kpart ? y : y - nt;
      const int hk = (int)(z / ((size_t)p.M * D));
      const int m = (int)(z / D % p.M), e = (int)(z % D);
      float acc = 0.f;
      for (int b = 0; b < p.B; ++b)
        for (int g = 0; g < p.G; ++g)
          for (int run = 0; run < nrun; ++run) {
            const size_t blk = ((size_t)b * p.Hq + hk * p.G + g) * nrun + run;
            acc += (kpart ? p.dtk_part : p.dtv_part)[(blk * 16 + m) * D + e];
          }
      (kpart ? p.dtk : p.dtv)[z] = acc;
    }
  }
}

// ======================================================================== host side
size_t bwd_workspace_layout(int B, int Hq, int Hkv, int L, int d, int M, int dtype_bf16, BwdWs *ws) {
  (void)dtype_bf16;  // every workspace array is fp32
  const size_t nq = (size_t)B * Hq * L * d, nk = (size_t)B * Hkv * L * d;
  const int ntile = (L + TS - 1) / TS, nrun = (ntile + QPW - 1) / QPW;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += (bytes + 255) & ~(size_t)255;
    return o;
  };
  BwdWs w{};
  w.phq = take(nq * 4);
  w.phk = take(nk * 4);
  w.dphq = take(nq * 4);
  w.dphk = take(nk * 4);
  w.dvg = take(nk * 4);
  w.dqw = take(nq * 4);
  w.dkw = take(nk * 4);
  w.dvw = take(0);  // (unused: the window-key kernel finishes dv)
  w.wstat = take((size_t)B * Hq * L * 16);
  const int nsplit = (L + 64 * FB_CHUNKS - 1) / (64 * FB_CHUNKS);
  w.dw_part = take((size_t)(B * Hq + B * Hkv) * nsplit * d * d * 4);
  const size_t ntp = M > 0 ? (size_t)B * Hq * nrun * 16 * d * 4 : 0;
  w.dtk_part = take(ntp);
  w.dtv_part = take(ntp);
  w.dw_tmp = take((size_t)RG * (Hq + Hkv) * d * d * 4);  // (per-head W_phi: the larger layout)
  if (ws) *ws = w;
  return off;
}

template <typename T, int D>
static hipError_t launch_bwd_t(const BwdParams &p, hipStream_t st) {
  const int nphi = (p.L + PHI_ROWS - 1) / PHI_ROWS;
  if (p.hh) hipLaunchKernelGGL((bwd_phi_kernel<T, D, true>), dim3((p.B * p.Hq + p.B * p.Hkv) * nphi), dim3(256), 0, st, p);
  else hipLaunchKernelGGL((bwd_phi_kernel<T, D, false>), dim3((p.B * p.Hq + p.B * p.Hkv) * nphi), dim3(256), 0, st, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int fgrid = D == 128 ? (p.B * p.Hq + 7) / 8 * 16 : p.B * p.Hq;
  hipLaunchKernelGGL((bwd_f_kernel<T, D>), dim3(fgrid), dim3(256), 0, st, p);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_v_kernel<T, D>), dim3((p.B * p.Hkv + 7) / 8 * 16), dim3(64 * (D / 32)), 0, st, p);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int ntile = (p.L + TS - 1) / TS, nrun = (ntile + QPW - 1) / QPW;
  hipLaunchKernelGGL((bwd_win_q_kernel<T, D>), dim3(p.B * p.Hq * nrun), dim3(64), 0, st, p);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  {
    const void *rk = reinterpret_cast<const void *>(bwd_r_kernel<T, D>);
    if ((e = hipFuncSetAttribute(rk, hipFuncAttributeMaxDynamicSharedMemorySize, (int)sizeof(LdsR2<T, D>))) != hipSuccess)
      return e;
    const int rgrid = D == 128 ? (p.B * p.Hkv + 7) / 8 * 16 : p.B * p.Hkv;
    hipLaunchKernelGGL((bwd_r_kernel<T, D>), dim3(rgrid), dim3(256), sizeof(LdsR2<T, D>), st, p);
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  {
    const void *kk = reinterpret_cast<const void *>(bwd_win_k_kernel<T, D>);
    if ((e = hipFuncSetAttribute(kk, hipFuncAttributeMaxDynamicSharedMemorySize, (int)sizeof(WinKLds<T, D>))) != hipSuccess)
      return e;
    hipLaunchKernelGGL((bwd_win_k_kernel<T, D>), dim3(p.B * p.Hkv * ((ntile + 3) / 4)), dim3(256), sizeof(WinKLds<T, D>), st, p);
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int nsplit = (p.L + 64 * FB_CHUNKS - 1) / (64 * FB_CHUNKS);
  const dim3 fbgrid((p.B * p.Hq + p.B * p.Hkv) * nsplit);
  if constexpr (sizeof(T) == 2) {
    if (p.hh) hipLaunchKernelGGL((bwd_fb_b16_kernel<D, true>), fbgrid, dim3(256), 0, st, p);
    else hipLaunchKernelGGL((bwd_fb_b16_kernel<D, false>), fbgrid, dim3(256), 0, st, p);
  } else {
    if (p.hh) hipLaunchKernelGGL((bwd_fb_kernel<T, D, true>), fbgrid, dim3(256), 0, st, p);
    else hipLaunchKernelGGL((bwd_fb_kernel<T, D, false>), fbgrid, dim3(256), 0, st, p);
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int FC = p.hh ? D / 2 : D;
  const size_t nw = (size_t)((p.w_stride ? p.Hq : 1) + (p.w_stride ? p.Hkv : 1)) * D * FC;
  hipLaunchKernelGGL(bwd_reduce_kernel, dim3((unsigned)((nw + 255) / 256), RG), dim3(256), 0, st, p, D, FC, 0);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(bwd_reduce_kernel, dim3(512), dim3(256), 0, st, p, D, FC, 1);
  return hipGetLastError();
}

hipError_t launch_bwd(const BwdParams &p, int dtype_bf16, int d, hipStream_t stream) {
  if (dtype_bf16) {
    if (d == 64) return launch_bwd_t<bf16, 64>(p, stream);
    if (d == 128) return launch_bwd_t<bf16, 128>(p, stream);
  } else {
    if (d == 64) return launch_bwd_t<float, 64>(p, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace lz
