// Lizard attention forward for gfx950: chunkwise gated linear attention plus
// anchor-window softmax plus weighted merge, fused in one kernel.
//
// Method (Lizard: An Efficient Linearization Framework for LLMs):
//   global branch  S_i = diag(gamma_i) S_{i-1} + phi_k(k_i) v_i^T,
//                  y_gla_i = phi_q(q_i)^T S_i             (papernotes.org
//                  summary, "key designs", Gated Linear Attention item);
//   local branch   softmax over [q.T_k ; q.k_j, i-W < j <= i] applied to
//                  [T_v ; v_j]                            (same, Anchor Window
//                  Attention item);
//   merge          y = mix y_gla + (1-mix) y_win          (same, "overall
//                  framework").
// The arXiv page's Method section observes that the cumulative gate product
// underflows in low precision and moves it into log space so the work becomes
// dense matrix products; this kernel keeps that idea but not the page's
// formulation.  Per 64-token chunk the log gate is summed inside the chunk only
// (chunk-local, fp32), and every exponential that multiplies an MFMA operand is
// taken relative to a reference point inside the chunk so that it is <= 1:
//
//   b_t   = sum of log gamma over chunk tokens 0..t (16-token sub-chunk I,
//           local sum bl_t, sub-chunk totals tot_J)
//   intra (s <= t, s in sub-chunk J < I):  phi_q(t) e^{bl_t} . e^{sum_{J<J'<I} tot_J'}
//           . phi_k(s) e^{tot_J - bl_s}                       (all factors <= 1)
//   intra (s <= t in the same sub-chunk):  reference at the sub-chunk's 8th
//           token; exact per-element fallback when the sub-chunk's decay span
//           is too large for that (e.g. gamma = 0).
//   inter:  phi_q(t) e^{b_t} . S_chunk_start
//   state:  S <- diag(e^{b_63}) S + sum_s phi_k(s) e^{b_63 - b_s} v_s^T
//
// Work split: one workgroup (4 waves) per (batch, key/value head, 64-column
// block of the value dimension, sequence segment).  Wave I owns query/key rows
// 16I..16I+15 of every chunk for the feature maps, the intra-chunk and
// inter-chunk products and the window; for the state update the four waves
// split S by rows of the key dimension.  The state is fp32 in registers; a
// copy in the operand dtype sits in LDS for the inter-chunk product.
// Segments after the first start from a state assembled from the per-segment
// end states that fwd_state_kernel (the same code with everything but the
// state update switched off) leaves in the workspace.
#include "common.hpp"
#include "internal.hpp"

namespace lz {

constexpr int CH = 64;          // chunk length
constexpr float SPAN_MAX = 80.f;  // max |log-decay| across one 16-token sub-chunk for the
                                  // mid-reference MFMA path (e^80 ~ 5.5e34 < fp32/bf16 max)
constexpr float NEG_BIG = -1.0e30f;

template <typename T, int D, int DV, int NR, bool STATE_ONLY> struct FwdLayout {
  static constexpr int PADE = 16 / (int)sizeof(T);
  static constexpr int LDW = D + PADE;   // rows of D elements
  static constexpr int LDC = CH + PADE;  // rows of 64 tokens
  static constexpr int LDM = 16 + PADE;  // rows of 16 meta tokens
  static constexpr size_t SZ_W = (size_t)D * LDW * sizeof(T);
  static constexpr size_t SZ_VT = (size_t)DV * LDC * sizeof(T);
  static constexpr size_t SZ_KOWN = (size_t)CH * LDW * sizeof(T);
  static constexpr size_t SZ_KST = (size_t)D * LDC * sizeof(T);
  static constexpr size_t SZ_SBF = (size_t)DV * LDW * sizeof(T);
  static constexpr size_t SZ_TOT = (size_t)4 * D * sizeof(float);
  static constexpr size_t SZ_TVT = (size_t)DV * LDM * sizeof(T);
  static constexpr size_t OFF_WK = 0;
  static constexpr size_t OFF_WQ = OFF_WK + SZ_W;
  static constexpr size_t OFF_VT = OFF_WQ + (STATE_ONLY ? 0 : SZ_W);
  static constexpr size_t OFF_KST = OFF_VT + NR * SZ_VT;
  static constexpr size_t OFF_TOT = OFF_KST + SZ_KST;
  static constexpr size_t OFF_KOWN = OFF_TOT + SZ_TOT;
  static constexpr size_t OFF_SBF = OFF_KOWN + (STATE_ONLY ? 0 : SZ_KOWN);
  static constexpr size_t OFF_TVT = OFF_SBF + (STATE_ONLY ? 0 : SZ_SBF);
  static constexpr size_t TOTAL = OFF_TVT + (STATE_ONLY ? 0 : SZ_TVT);
};

// W_phi [d][f] row-major in global -> W^T [f][d] in LDS (row stride LDW).
template <typename T, int D, int LDW>
__device__ __forceinline__ void load_wT(T *dst, const T *src) {
  for (int idx = threadIdx.x; idx < D * (D / 8); idx += 256) {
    const int dd = idx / (D / 8), f0 = (idx % (D / 8)) * 8;
    float x[8];
    load8f(src + (size_t)dd * D + f0, x);
#pragma unroll
    for (int j = 0; j < 8; ++j) dst[(f0 + j) * LDW + dd] = from_f<T>(x[j]);
  }
}

// V rows c0..c0+63 (columns dv0..dv0+DV-1) -> V^T [dv][token] in LDS; rows past L are zero.
template <typename T, int D, int DV, int LDC>
__device__ __forceinline__ void load_vT(T *dst, const T *vh, int c0, int L, int dv0) {
  for (int idx = threadIdx.x; idx < (CH / 2) * (DV / 8); idx += 256) {
    const int tp = idx / (DV / 8), dq = idx % (DV / 8);
    const int t0 = 2 * tp;
    float a[8], b[8];
    if (c0 + t0 < L) load8f(vh + (size_t)(c0 + t0) * D + dv0 + 8 * dq, a);
    else {
#pragma unroll
      for (int j = 0; j < 8; ++j) a[j] = 0.f;
    }
    if (c0 + t0 + 1 < L) load8f(vh + (size_t)(c0 + t0 + 1) * D + dv0 + 8 * dq, b);
    else {
#pragma unroll
      for (int j = 0; j < 8; ++j) b[j] = 0.f;
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      dst[(8 * dq + j) * LDC + t0] = from_f<T>(a[j]);
      dst[(8 * dq + j) * LDC + t0 + 1] = from_f<T>(b[j]);
    }
  }
}

template <typename T, int D, int DV, int NR, bool STATE_ONLY>
__global__ __launch_bounds__(256, 1) void fwd_kernel(FwdParams p) {
  using Lay = FwdLayout<T, D, DV, NR, STATE_ONLY>;
  constexpr int NFT = D / 16;   // 16-row tiles of the feature dimension
  constexpr int KS = D / 32;    // K = 32 steps over d (or over features)
  constexpr int NDT = DV / 16;  // 16-column tiles of this block's value columns
  constexpr int FTW = NFT / 4;  // feature tiles of S owned by each wave
  constexpr int LDW = Lay::LDW, LDC = Lay::LDC, LDM = Lay::LDM;
  static_assert(NFT % 4 == 0, "d must be a multiple of 64");

  __shared__ __attribute__((aligned(16))) char smem[Lay::TOTAL];
  T *sWk = reinterpret_cast<T *>(smem + Lay::OFF_WK);
  T *sWq = reinterpret_cast<T *>(smem + Lay::OFF_WQ);
  T *sVt = reinterpret_cast<T *>(smem + Lay::OFF_VT);
  T *sKSt = reinterpret_cast<T *>(smem + Lay::OFF_KST);
  float *sTot = reinterpret_cast<float *>(smem + Lay::OFF_TOT);
  T *sKown = reinterpret_cast<T *>(smem + Lay::OFF_KOWN);
  T *sSbf = reinterpret_cast<T *>(smem + Lay::OFF_SBF);
  T *sTvT = reinterpret_cast<T *>(smem + Lay::OFF_TVT);

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int r16 = lane & 15, g4 = lane >> 4;

  // ---- block -> (group, value block), keeping a group's value blocks on one XCD
  const int bid = blockIdx.x;
  const int xcd = bid & 7, slot = bid >> 3;
  const int grp = (slot / p.ndvb) * 8 + xcd;
  const int dvb = slot % p.ndvb;
  if (grp >= p.ngroups) return;
  const int nsegw = STATE_ONLY ? p.nseg - 1 : p.nseg;
  const int seg = grp % nsegw;
  const int bh = grp / nsegw;
  const int b = bh / p.Hkv, kvh = bh % p.Hkv;
  const int L = p.L, G = p.G;
  const int dv0 = dvb * DV;
  const int c_begin = seg * p.cps;
  const int c_end = min(p.nchunks, c_begin + p.cps);

  const size_t kv_off = ((size_t)b * p.Hkv + kvh) * (size_t)L * D;
  const T *Kh = reinterpret_cast<const T *>(p.k) + kv_off;
  const T *Vh = reinterpret_cast<const T *>(p.v) + kv_off;
  const T *LGh = reinterpret_cast<const T *>(p.lg) + kv_off;
  const T *Wk = reinterpret_cast<const T *>(p.wk) + (size_t)kvh * p.w_stride;

  // ---- prologue
  load_wT<T, D, LDW>(sWk, Wk);
  if constexpr (!STATE_ONLY) {
    load_wT<T, D, LDW>(sWq, reinterpret_cast<const T *>(p.wq) + (size_t)(kvh * G) * p.w_stride);
    const T *Tv = reinterpret_cast<const T *>(p.tv);
    for (int idx = tid; idx < DV * 16; idx += 256) {
      const int dv = idx / 16, m = idx % 16;
      sTvT[dv * LDM + m] = (m < p.M) ? Tv[((size_t)kvh * p.M + m) * D + dv0 + dv] : from_f<T>(0.f);
    }
    // previous chunks needed by the window of this segment's first chunk
    for (int cc = max(0, c_begin - (NR - 1)); cc < c_begin; ++cc)
      load_vT<T, D, DV, LDC>(sVt + (cc % NR) * (DV * LDC), Vh, cc * CH, L, dv0);
  }

  // S owned by this wave: feature tiles wv*FTW .. +FTW-1, all value tiles.
  // S[ft][dt][i] = S[16*(wv*FTW+ft) + 4*g4 + i][dv0 + 16*dt + r16]
  f32x4 S[FTW][NDT];
#pragma unroll
  for (int ft = 0; ft < FTW; ++ft)
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) S[ft][dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  const size_t st_per_grp = (size_t)D * DV;
  if constexpr (!STATE_ONLY) {
    // start state of this segment: S = sum_j diag(prod of later decays) E_j
    for (int j = 0; j < seg; ++j) {
      const float *E = p.ws_state + ((((size_t)b * p.Hkv + kvh) * p.ndvb + dvb) * (p.nseg - 1) + j) * st_per_grp;
      const float *Dj = p.ws_decay + (((size_t)b * p.Hkv + kvh) * (p.nseg - 1) + j) * D;
#pragma unroll
      for (int ft = 0; ft < FTW; ++ft) {
        float e[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) e[i] = __expf(Dj[16 * (wv * FTW + ft) + 4 * g4 + i]);
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          const f32x4 x = *reinterpret_cast<const f32x4 *>(E + (((size_t)(wv * FTW + ft) * NDT + dt) * 64 + lane) * 4);
#pragma unroll
          for (int i = 0; i < 4; ++i) S[ft][dt][i] = e[i] * S[ft][dt][i] + x[i];
        }
      }
    }
    // operand copy S^T [dv][f]
#pragma unroll
    for (int ft = 0; ft < FTW; ++ft)
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
        store4<T>(sSbf + (16 * dt + r16) * LDW + 16 * (wv * FTW + ft) + 4 * g4, S[ft][dt][0], S[ft][dt][1],
                  S[ft][dt][2], S[ft][dt][3]);
  }
  float dsum = 0.f;  // state-only: running sum of log gamma for feature tid
  __syncthreads();

  const int I = wv;  // sub-chunk owned by this wave
  const float mix = p.mix, scale = p.scale;

  for (int c = c_begin; c < c_end; ++c) {
    const int c0 = c * CH;
    const int cur = (c % NR) * (DV * LDC);
    // ---- V of this chunk -> ring slot
    load_vT<T, D, DV, LDC>(sVt + cur, Vh, c0, L, dv0);

    // ---- own rows: keys (B-operand fragments over d) and log gamma
    const int pos = c0 + 16 * I + r16;
    const bool valid = pos < L;
    Frag<T> kf[KS];
#pragma unroll
    for (int j = 0; j < KS; ++j)
      kf[j] = valid ? load8(Kh + (size_t)pos * D + 32 * j + 8 * g4) : frag_zero<T>();
    float bl[NFT][4];  // log gamma -> local inclusive cumsum within the sub-chunk
#pragma unroll
    for (int ft = 0; ft < NFT; ++ft) {
      if (valid) load4f(LGh + (size_t)pos * D + 16 * ft + 4 * g4, bl[ft]);
      else {
#pragma unroll
        for (int i = 0; i < 4; ++i) bl[ft][i] = 0.f;
      }
    }
#pragma unroll
    for (int ft = 0; ft < NFT; ++ft)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float x = bl[ft][i];
#pragma unroll
        for (int dd = 1; dd < 16; dd <<= 1) {
          const float y = __shfl_up(x, dd, 16);
          if (r16 >= dd) x += y;
        }
        bl[ft][i] = x;
      }
    float tot[NFT][4];  // this sub-chunk's total, broadcast from its last row
#pragma unroll
    for (int ft = 0; ft < NFT; ++ft)
#pragma unroll
      for (int i = 0; i < 4; ++i) tot[ft][i] = __shfl(bl[ft][i], 16 * g4 + 15);
    if (r16 == 15) {
#pragma unroll
      for (int ft = 0; ft < NFT; ++ft)
#pragma unroll
        for (int i = 0; i < 4; ++i) sTot[I * D + 16 * ft + 4 * g4 + i] = bl[ft][i];
    }

    // ---- phi_k for own rows: z^T[f][t] = sum_d W[d][f] k[t][d]
    float phik[NFT][4];
    {
      f32x4 z[NFT];
#pragma unroll
      for (int ft = 0; ft < NFT; ++ft) {
        z[ft] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < KS; ++j) z[ft] = mma(load8(sWk + (16 * ft + r16) * LDW + 32 * j + 8 * g4), kf[j], z[ft]);
      }
      float zm = NEG_BIG;
#pragma unroll
      for (int ft = 0; ft < NFT; ++ft)
#pragma unroll
        for (int i = 0; i < 4; ++i) zm = fmaxf(zm, z[ft][i]);
      zm = wave_max_cols(zm);
      float zs = 0.f;
#pragma unroll
      for (int ft = 0; ft < NFT; ++ft)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          phik[ft][i] = __expf(z[ft][i] - zm);
          zs += phik[ft][i];
        }
      zs = wave_sum_cols(zs);
      const float inv = 1.f / zs;
#pragma unroll
      for (int ft = 0; ft < NFT; ++ft)
#pragma unroll
        for (int i = 0; i < 4; ++i) phik[ft][i] *= inv;
    }

    // ---- keys relative to the end of their own sub-chunk (<= 1) -> LDS [s][f]
    Frag<T> kmid[KS];
    bool safe = true;
    if constexpr (!STATE_ONLY) {
#pragma unroll
      for (int ft = 0; ft < NFT; ++ft) {
        float o[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = phik[ft][i] * __expf(tot[ft][i] - bl[ft][i]);
        store4<T>(sKown + (16 * I + r16) * LDW + 16 * ft + 4 * g4, o[0], o[1], o[2], o[3]);
      }
      // diagonal block operands, reference at row 7 of the sub-chunk
      float span = 0.f;
#pragma unroll
      for (int ft = 0; ft < NFT; ++ft)
#pragma unroll
        for (int i = 0; i < 4; ++i) span = fmaxf(span, -tot[ft][i]);
      span = wave_max_all(span);
      safe = span <= SPAN_MAX;
#pragma unroll
      for (int js = 0; js < KS; ++js) {
        float x[8];
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
          const int ft = 2 * js + (jj >> 2), i = jj & 3;
          const float b7 = __shfl(bl[ft][i], 16 * g4 + 7);
          x[jj] = safe ? phik[ft][i] * __expf(b7 - bl[ft][i]) : 0.f;
        }
        kmid[js] = frag_from<T>(x);
      }
    }
    __syncthreads();  // B1: sub-chunk totals (and own-sub-chunk keys) visible

    // ---- chunk prefix sums for own features: pre = sum_{J<I} tot_J, btot = sum_J tot_J
    float pre[NFT][4], btot[NFT][4];
#pragma unroll
    for (int ft = 0; ft < NFT; ++ft)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int f = 16 * ft + 4 * g4 + i;
        float a = 0.f, s = 0.f;
#pragma unroll
        for (int J = 0; J < 4; ++J) {
          const float x = sTot[J * D + f];
          if (J < I) a += x;
          s += x;
        }
        pre[ft][i] = a;
        btot[ft][i] = s;
      }
    if constexpr (STATE_ONLY) {
      if (tid < D) {
#pragma unroll
        for (int J = 0; J < 4; ++J) dsum += sTot[J * D + tid];
      }
    }
    // keys decayed to the chunk end (<= 1) -> LDS [f][s]
#pragma unroll
    for (int ft = 0; ft < NFT; ++ft)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        sKSt[(16 * ft + 4 * g4 + i) * LDC + 16 * I + r16] =
            from_f<T>(phik[ft][i] * __expf(btot[ft][i] - pre[ft][i] - bl[ft][i]));
    __syncthreads();  // B2: keys for the intra products and the state update visible

    if constexpr (!STATE_ONLY) {
      for (int g = 0; g < G; ++g) {
        const int hq = kvh * G + g;
        if (p.per_head_q && G > 1) {  // a different W_phi_q for every query head
          __syncthreads();
          load_wT<T, D, LDW>(sWq, reinterpret_cast<const T *>(p.wq) + (size_t)hq * p.w_stride);
          __syncthreads();
        }
        const T *Qh = reinterpret_cast<const T *>(p.q) + ((size_t)b * p.Hq + hq) * (size_t)L * D;
        Frag<T> qf[KS];
#pragma unroll
        for (int j = 0; j < KS; ++j)
          qf[j] = valid ? load8(Qh + (size_t)pos * D + 32 * j + 8 * g4) : frag_zero<T>();

        // phi_q for own rows, then q~ = phi_q e^{bl} (<= 1)
        float qo[NFT][4], phiq[NFT][4];
        {
          f32x4 z[NFT];
#pragma unroll
          for (int ft = 0; ft < NFT; ++ft) {
            z[ft] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < KS; ++j) z[ft] = mma(load8(sWq + (16 * ft + r16) * LDW + 32 * j + 8 * g4), qf[j], z[ft]);
          }
          float zm = NEG_BIG;
#pragma unroll
          for (int ft = 0; ft < NFT; ++ft)
#pragma unroll
            for (int i = 0; i < 4; ++i) zm = fmaxf(zm, z[ft][i]);
          zm = wave_max_cols(zm);
          float zs = 0.f;
#pragma unroll
          for (int ft = 0; ft < NFT; ++ft)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              phiq[ft][i] = __expf(z[ft][i] - zm);
              zs += phiq[ft][i];
            }
          zs = wave_sum_cols(zs);
          const float inv = 1.f / zs;
#pragma unroll
          for (int ft = 0; ft < NFT; ++ft)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              phiq[ft][i] *= inv;
              qo[ft][i] = phiq[ft][i] * __expf(bl[ft][i]);
            }
        }

        // ---- intra-chunk scores A^T[s][t] for key sub-chunks J <= I
        f32x4 at[4];
#pragma unroll
        for (int J = 0; J < 4; ++J) at[J] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int J = 0; J < 3; ++J) {
          if (J < I) {
            // factor e^{sum_{J<J'<I} tot_J'} joins the two references
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int js = 0; js < KS; ++js) {
              float x[8];
#pragma unroll
              for (int jj = 0; jj < 8; ++jj) {
                const int ft = 2 * js + (jj >> 2), i = jj & 3;
                const int f = 16 * ft + 4 * g4 + i;
                float gap = 0.f;
#pragma unroll
                for (int J2 = 0; J2 < 3; ++J2)
                  if (J2 > J && J2 < I) gap += sTot[J2 * D + f];
                x[jj] = qo[ft][i] * __expf(gap);
              }
              const T *kr = sKown + (16 * J + r16) * LDW + 32 * js + 4 * g4;
              acc = mma(load4x2(kr, kr + 16), frag_from<T>(x), acc);
            }
            at[J] = acc;
          }
        }
        {
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
          if (safe) {
#pragma unroll
            for (int js = 0; js < KS; ++js) {
              float x[8];
#pragma unroll
              for (int jj = 0; jj < 8; ++jj) {
                const int ft = 2 * js + (jj >> 2), i = jj & 3;
                const float b7 = __shfl(bl[ft][i], 16 * g4 + 7);
                x[jj] = phiq[ft][i] * __expf(bl[ft][i] - b7);
              }
              acc = mma(kmid[js], frag_from<T>(x), acc);
            }
          } else {
            // exact: A[t][s] = sum_f phi_q[t][f] phi_k[s][f] e^{bl_t[f] - bl_s[f]}
#pragma unroll 1
            for (int s2 = 0; s2 < 16; ++s2) {
              float part = 0.f;
#pragma unroll
              for (int ft = 0; ft < NFT; ++ft)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                  const float pk = __shfl(phik[ft][i], 16 * g4 + s2);
                  const float bs = __shfl(bl[ft][i], 16 * g4 + s2);
                  const float term = phiq[ft][i] * pk * __expf(bl[ft][i] - bs);
                  part += (s2 <= r16) ? term : 0.f;
                }
              part = wave_sum_cols(part);
#pragma unroll
              for (int i = 0; i < 4; ++i)
                if ((s2 >> 2) == g4 && (s2 & 3) == i) acc[i] = part;
            }
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[i] = (4 * g4 + i <= r16) ? acc[i] : 0.f;
#pragma unroll
          for (int J = 0; J < 4; ++J)
            if (J == I) at[J] = acc;  // compile-time index keeps at[] in registers
        }

        // ---- Y^T = V^T A^T (intra) + S^T q~int^T (inter); lane holds Y^T[dv][t]
        f32x4 yacc[NDT];
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) yacc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int J0 = 0; J0 < 4; J0 += 2) {
          if (J0 <= I) {
            const bool has1 = (J0 + 1) <= I;
            float x[8];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              x[i] = at[J0][i];
              x[4 + i] = has1 ? at[J0 + 1][i] : 0.f;
            }
            const Frag<T> bf = frag_from<T>(x);
            const int J1 = has1 ? J0 + 1 : J0;
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) {
              const T *vr = sVt + cur + (16 * dt + r16) * LDC + 4 * g4;
              yacc[dt] = mma(load4x2(vr + 16 * J0, vr + 16 * J1), bf, yacc[dt]);
            }
          }
        }
        {
#pragma unroll
          for (int js = 0; js < KS; ++js) {
            float x[8];
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) {
              const int ft = 2 * js + (jj >> 2), i = jj & 3;
              x[jj] = qo[ft][i] * __expf(pre[ft][i]);
            }
            const Frag<T> bf = frag_from<T>(x);
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) {
              const T *sr = sSbf + (16 * dt + r16) * LDW + 32 * js + 4 * g4;
              yacc[dt] = mma(load4x2(sr, sr + 16), bf, yacc[dt]);
            }
          }
        }

        // ---- anchor window: meta keys + keys j with pos-W < j <= pos, online softmax
        f32x4 ywin[NDT];
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) ywin[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
        float m_run = NEG_BIG, l_run = 0.f;
        const int kt_hi = (c0 >> 4) + I;
        const int lo_key = c0 + 16 * I - p.W + 1;
        const int kt_lo = lo_key <= 0 ? 0 : (lo_key >> 4);
        // tile list: u = -1 is the meta tile (if M > 0), then kt_lo..kt_hi
        const int u_first = (p.M > 0) ? -1 : 0;
        const int n_tiles = (kt_hi - kt_lo + 1) - u_first;
        const T *Tk = reinterpret_cast<const T *>(p.tk);
        for (int u0 = 0; u0 < n_tiles; u0 += 4) {
          f32x4 lt[4];
          int kts[4];
#pragma unroll
          for (int uu = 0; uu < 4; ++uu) {
            const int u = u0 + uu;
            lt[uu] = f32x4{NEG_BIG, NEG_BIG, NEG_BIG, NEG_BIG};
            kts[uu] = -2;  // none
            if (u < n_tiles) {
              const int kt = (u + u_first < 0) ? -1 : kt_lo + u + u_first;
              kts[uu] = kt;
              f32x4 acc = {0.f, 0.f, 0.f, 0.f};
              if (kt < 0) {
                const bool mv = r16 < p.M;
#pragma unroll
                for (int j = 0; j < KS; ++j) {
                  const Frag<T> a = mv ? load8(Tk + ((size_t)kvh * p.M + r16) * D + 32 * j + 8 * g4) : frag_zero<T>();
                  acc = mma(a, qf[j], acc);
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) lt[uu][i] = (4 * g4 + i < p.M) ? acc[i] * scale : NEG_BIG;
              } else {
                const int key = 16 * kt + r16;
                const bool kv = key < L;
#pragma unroll
                for (int j = 0; j < KS; ++j) {
                  const Frag<T> a = kv ? load8(Kh + (size_t)key * D + 32 * j + 8 * g4) : frag_zero<T>();
                  acc = mma(a, qf[j], acc);
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                  const int kj = 16 * kt + 4 * g4 + i;
                  lt[uu][i] = (kj <= pos && kj > pos - p.W) ? acc[i] * scale : NEG_BIG;
                }
              }
            }
          }
          float bm = NEG_BIG;
#pragma unroll
          for (int uu = 0; uu < 4; ++uu)
#pragma unroll
            for (int i = 0; i < 4; ++i) bm = fmaxf(bm, lt[uu][i]);
          bm = wave_max_cols(bm);
          const float m_new = fmaxf(m_run, bm);
          const float alpha = __expf(m_run - m_new);
          l_run *= alpha;
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
            for (int i = 0; i < 4; ++i) ywin[dt][i] *= alpha;
          m_run = m_new;
          float pv[4][4];
#pragma unroll
          for (int uu = 0; uu < 4; ++uu)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              pv[uu][i] = (lt[uu][i] > 0.5f * NEG_BIG) ? __expf(lt[uu][i] - m_new) : 0.f;
              l_run += pv[uu][i];
            }
          // P V: pairs of tiles form one K = 32 step
#pragma unroll
          for (int pr = 0; pr < 2; ++pr) {
            const int ua = 2 * pr, ub = 2 * pr + 1;
            if (kts[ua] == -2) continue;
            float x[8];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              x[i] = pv[ua][i];
              x[4 + i] = (kts[ub] == -2) ? 0.f : pv[ub][i];
            }
            const Frag<T> bf = frag_from<T>(x);
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) {
              const int dvl = 16 * dt + r16;
              float av[8];
#pragma unroll
              for (int half = 0; half < 2; ++half) {
                const int kt = kts[half ? ub : ua];
                if (kt == -2) {
#pragma unroll
                  for (int i = 0; i < 4; ++i) av[4 * half + i] = 0.f;
                } else if (kt == -1) {
                  float t4[4];
                  load4f(sTvT + dvl * LDM + 4 * g4, t4);
#pragma unroll
                  for (int i = 0; i < 4; ++i) av[4 * half + i] = t4[i];
                } else if ((kt >> 2) > c - NR) {
                  float t4[4];
                  load4f(sVt + ((kt >> 2) % NR) * (DV * LDC) + dvl * LDC + 16 * (kt & 3) + 4 * g4, t4);
#pragma unroll
                  for (int i = 0; i < 4; ++i) av[4 * half + i] = t4[i];
                } else {
                  // key tile older than the LDS ring: gather from global memory
#pragma unroll
                  for (int i = 0; i < 4; ++i) {
                    const int key = 16 * kt + 4 * g4 + i;
                    av[4 * half + i] = (key < L) ? to_f(Vh[(size_t)key * D + dv0 + dvl]) : 0.f;
                  }
                }
              }
              ywin[dt] = mma(frag_from<T>(av), bf, ywin[dt]);
            }
          }
        }
        const float l_tot = wave_sum_cols(l_run);
        const float wscale = (1.f - mix) / l_tot;

        // ---- merge and store (lane holds Y^T[dv0 + 16 dt + 4 g4 + i][pos])
        if (valid) {
          T *O = reinterpret_cast<T *>(p.out) + (((size_t)b * p.Hq + hq) * (size_t)L + pos) * D + dv0;
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt) {
            float o[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) o[i] = mix * yacc[dt][i] + wscale * ywin[dt][i];
            store4<T>(O + 16 * dt + 4 * g4, o[0], o[1], o[2], o[3]);
          }
        }
      }  // g
    }
    __syncthreads();  // B3: all reads of the state copy and this chunk's keys done

    // ---- state update on owned rows: S = diag(e^{btot}) S + KSt^T V
#pragma unroll
    for (int ft = 0; ft < FTW; ++ft) {
      const int fr = 16 * (wv * FTW + ft);
      float e[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int f = fr + 4 * g4 + i;
        float s = 0.f;
#pragma unroll
        for (int J = 0; J < 4; ++J) s += sTot[J * D + f];
        e[i] = __expf(s);
      }
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) S[ft][dt][i] *= e[i];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
          S[ft][dt] = mma(load8(sKSt + (fr + r16) * LDC + 32 * ks + 8 * g4),
                          load8(sVt + cur + (16 * dt + r16) * LDC + 32 * ks + 8 * g4), S[ft][dt]);
        if constexpr (!STATE_ONLY)
          store4<T>(sSbf + (16 * dt + r16) * LDW + fr + 4 * g4, S[ft][dt][0], S[ft][dt][1], S[ft][dt][2],
                    S[ft][dt][3]);
      }
    }
    __syncthreads();  // B4: new state copy visible; LDS buffers free for the next chunk
  }

  if constexpr (STATE_ONLY) {
    float *E = p.ws_state + ((((size_t)b * p.Hkv + kvh) * p.ndvb + dvb) * (p.nseg - 1) + seg) * st_per_grp;
#pragma unroll
    for (int ft = 0; ft < FTW; ++ft)
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
        *reinterpret_cast<f32x4 *>(E + (((size_t)(wv * FTW + ft) * NDT + dt) * 64 + lane) * 4) = S[ft][dt];
    if (dvb == 0 && tid < D) p.ws_decay[(((size_t)b * p.Hkv + kvh) * (p.nseg - 1) + seg) * D + tid] = dsum;
  }
}

// ---------------------------------------------------------------- host side
template <typename T, int D, int DV, int NR>
static hipError_t launch_fwd_t(const FwdParams &prm, int nseg, hipStream_t stream) {
  FwdParams p = prm;
  if (nseg > 1) {
    p.ngroups = p.B * p.Hkv * (nseg - 1);
    const int grid = ((p.ngroups + 7) / 8) * 8 * p.ndvb;
    hipLaunchKernelGGL((fwd_kernel<T, D, DV, 1, true>), dim3(grid), dim3(256), 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  p.ngroups = p.B * p.Hkv * nseg;
  const int grid = ((p.ngroups + 7) / 8) * 8 * p.ndvb;
  hipLaunchKernelGGL((fwd_kernel<T, D, DV, NR, false>), dim3(grid), dim3(256), 0, stream, p);
  return hipGetLastError();
}

template <typename T, int D, int DV>
static hipError_t launch_fwd_nr(const FwdParams &p, int nseg, hipStream_t stream) {
  if (p.nring <= 2) return launch_fwd_t<T, D, DV, 2>(p, nseg, stream);
  return launch_fwd_t<T, D, DV, 3>(p, nseg, stream);
}

hipError_t launch_fwd(const FwdParams &p, int dtype_bf16, int d, hipStream_t stream) {
  if (dtype_bf16) {
    if (d == 64) return launch_fwd_nr<bf16, 64, 64>(p, p.nseg, stream);
    if (d == 128) return launch_fwd_nr<bf16, 128, 64>(p, p.nseg, stream);
  } else {
    if (d == 64) return launch_fwd_nr<float, 64, 64>(p, p.nseg, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace lz
