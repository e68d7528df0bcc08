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
// formulation.  The log gate is summed inside each 16-token sub-chunk only, in
// fp32, and every exponential that multiplies an MFMA operand is taken relative
// to a reference point inside the chunk so that it stays in range:
//
//   per sub-chunk I (rows t = 0..15):  p_t = sum_{s<=t} lg_s (prefix),
//       r_t = sum_{s>t} lg_s (suffix), tot = p_15, p7 = p_7
//   keys    ko_s  = phi_k(s) e^{r_s}           (decay to the sub-chunk end, <= 1)
//   queries qo_t  = phi_q(t) e^{p_t}           (decay from the sub-chunk start, <= 1)
//   intra, key sub-chunk J < I:   qo_t . ko_s . prod_{J<J'<I} e^{tot_J'}
//   intra, same sub-chunk (s<=t): (qo_t e^{-p7}) . (ko_s e^{p7-tot}), both
//         within e^{+-span}; exact per-element fallback if the span of the
//         sub-chunk's log decay exceeds SPAN_MAX (e.g. gamma = 0)
//   inter:  qo_t prod_{J<I} e^{tot_J} . S_chunk_start
//   state:  S <- diag(prod_J e^{tot_J}) S + sum_s ko_s prod_{J'>J(s)} e^{tot_J'} v_s^T
// The per-element exponentials are the four above (phi_k, phi_q, e^{r}, e^{p});
// all per-feature factors come from small tables built once per chunk.  The
// prefix and suffix sums are MFMA products with constant triangular 0/1
// matrices (exact: bf16 inputs, fp32 accumulation).
//
// Work split: one workgroup (4 waves) per (batch, key/value head, 64-column
// block of the value dimension, sequence segment).  Wave I owns query/key rows
// 16I..16I+15 of every chunk for the feature maps, the intra-chunk and
// inter-chunk products and the window; for the state update the four waves
// split S by rows of the key dimension.  The state is fp32 in registers; a
// copy in the operand dtype sits in LDS for the inter-chunk product.
//
// Memory pipeline: the next chunk's k, v and log gamma are loaded into
// registers at the top of the current chunk (q after the query loop) and
// written to LDS at the top of the next one.  Keys and values of the last
// few chunks stay in LDS rings, so the window reads no global memory.
// Segments after the first start from a state assembled from the per-segment
// end states that the state-only variant of this kernel leaves in the
// workspace.
#include <cstdlib>
#include <cstring>

#include "fwd_common.hpp"

namespace lz {

template <typename T, int D, int DV, bool STATE_ONLY, bool WIDE>
__global__ __launch_bounds__(256, 1) void fwd_kernel(FwdParams p) {
  using Gm = FwdGeom<T, D, DV, WIDE>;
  constexpr int NFT = D / 16;   // 16-row tiles of the feature dimension
  constexpr int KS = D / 32;    // K = 32 steps over d (or over features)
  constexpr int NDT = DV / 16;  // 16-column tiles of this block's value columns
  constexpr int FTW = NFT / 4;  // feature tiles of S owned by each wave
  constexpr int LDW = Gm::LDW, LDB = Gm::LDB, LDC = Gm::LDC, LDG = Gm::LDG, LDM = Gm::LDM;
  static_assert(NFT % 4 == 0, "d must be a multiple of 64");

  extern __shared__ __attribute__((aligned(16))) char smem[];
  const FwdLds &ly = p.lds;
  T *sWk = reinterpret_cast<T *>(smem + ly.wk);
  T *sWq = reinterpret_cast<T *>(smem + ly.wq);
  T *sVt = reinterpret_cast<T *>(smem + ly.vt);
  T *sKr = reinterpret_cast<T *>(smem + ly.kr);
  T *sKown = reinterpret_cast<T *>(smem + ly.kown);
  T *sLgT = sKown;  // log gamma^T [f][s], dead before the keys are written
  float *sTot = reinterpret_cast<float *>(smem + ly.tot);
  float *sP7 = reinterpret_cast<float *>(smem + ly.p7);
  float *sETot = reinterpret_cast<float *>(smem + ly.etot);
  float *sENP7 = reinterpret_cast<float *>(smem + ly.enp7);
  float *sENR8 = reinterpret_cast<float *>(smem + ly.enr8);
  T *sSbf = reinterpret_cast<T *>(smem + ly.sbf);
  T *sTvT = reinterpret_cast<T *>(smem + ly.tvt);
  T *sTk = reinterpret_cast<T *>(smem + ly.tk);
  const int NR = p.nring, KR = p.kring;

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
  // window history before the first token (continuation of earlier tokens)
  const size_t hist_off = ((size_t)b * p.Hkv + kvh) * (size_t)p.hist_rows * D;
  const T *Hk = reinterpret_cast<const T *>(p.hist_k) + hist_off;
  const T *Hv = reinterpret_cast<const T *>(p.hist_v) + hist_off;
  const int hist_avail = p.pos ? min(p.pos[b], p.W - 1) : 0;  // history tokens the window may see
  const T *Wk = reinterpret_cast<const T *>(p.wk) + (size_t)kvh * p.w_stride;
  const T *Qbase = reinterpret_cast<const T *>(p.q);

  // ---- prologue
  load_wT<T, D, LDW>(sWk, Wk, tid);
  if constexpr (!STATE_ONLY) {
    if (ly.wq != ly.wk)
      load_wT<T, D, LDW>(sWq, reinterpret_cast<const T *>(p.wq) + (size_t)(kvh * G) * p.w_stride, tid);
    const T *Tv = reinterpret_cast<const T *>(p.tv);
    const T *Tk = reinterpret_cast<const T *>(p.tk);
    for (int idx = tid; idx < DV * 16; idx += 256) {
      const int dv = idx / 16, m = idx % 16;
      sTvT[dv * LDM + m] = (m < p.M) ? Tv[((size_t)kvh * p.M + m) * D + dv0 + dv] : from_f<T>(0.f);
    }
    for (int idx = tid; idx < 16 * D; idx += 256) {
      const int m = idx / D, e = idx % D;
      sTk[m * LDW + e] = (m < p.M) ? Tk[((size_t)kvh * p.M + m) * D + e] : from_f<T>(0.f);
    }
    // rings start as zeros: a masked window slot (probability 0) must not meet a NaN pattern
    {
      uint4 *vz = reinterpret_cast<uint4 *>(smem + ly.vt);
      const int nz = (ly.kown - ly.vt) / 16;  // value ring and key ring are contiguous
      for (int idx = tid; idx < nz; idx += 256) vz[idx] = uint4{0u, 0u, 0u, 0u};
    }
    __syncthreads();
    // earlier chunks reached by the window of this segment's first chunk
    const int R = max(NR, KR);
    for (int cc = max(-(p.hist_rows / CH), c_begin - (R - 1)); cc < c_begin; ++cc) {
      ChunkRegs<T, D, DV> pre;
      if (cc >= 0)
        load_chunk<T, D, DV>(pre, Kh, Vh, LGh, cc * CH, L, dv0, true, tid);
      else  // history rows (the log gamma slot is not used)
        load_chunk<T, D, DV>(pre, Hk, Hv, Hk, p.hist_rows + cc * CH, p.hist_rows, dv0, true, tid);
      if (cc > c_begin - KR) store_keys<T, D, DV, LDW>(pre, sKr + pmod(cc, KR) * (CH * LDW), tid);
      if (cc > c_begin - NR) store_values<T, D, DV, LDC>(pre, sVt + pmod(cc, NR) * (DV * LDC), tid);
    }
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
    if (p.state_in) {  // continuation: the state after the earlier tokens
      const float *Si = p.state_in + ((size_t)b * p.Hkv + kvh) * D * D;
#pragma unroll
      for (int ft = 0; ft < FTW; ++ft)
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            S[ft][dt][i] = Si[(size_t)(16 * (wv * FTW + ft) + 4 * g4 + i) * D + dv0 + 16 * dt + r16];
    }
    // start state of this segment: S = diag(prod of all earlier decays) S_in
    //                                  + sum_j diag(prod of later decays) E_j
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
  }
  float dsum = 0.f;  // state-only: running sum of log gamma for feature tid

  const int I = wv;  // sub-chunk owned by this wave
  const float mix = p.mix, scale = p.scale;
  const bool win_fast = (p.W <= CH + 1) && KR >= 2 && NR >= 2;
  // fast window: bit 4u+i set when slot (tile u, row 4 g4 + i) is inside the window of this
  // lane's query (u = 0 meta; band tile u: kj - pos = 16u - 80 + 4 g4 + i - r16)
  uint32_t wmask = 0;
#pragma unroll
  for (int u = 0; u < 6; ++u)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int dk = 16 * u - 80 + 4 * g4 + i - r16;
      const bool in = (u == 0) ? (4 * g4 + i < p.M) : (dk <= 0 && dk > -p.W);
      wmask |= (in ? 1u : 0u) << (4 * u + i);
    }
  // the first chunk: band slots before the first token hold history (valid only for
  // the last hist_avail tokens; band tile u < 5 - I lies in the previous chunk)
  uint32_t wmask0 = wmask;
#pragma unroll
  for (int u = 1; u < 5; ++u)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rt = I - 5 + u;
      if (rt < 0 && 16 * rt + 4 * g4 + i < -hist_avail) wmask0 &= ~(1u << (4 * u + i));
    }
  const Frag<T> tri_pre = tri_frag<T>(r16, g4, true);
  const Frag<T> tri_suf = tri_frag<T>(r16, g4, false);

  // first chunk's data into registers
  ChunkRegs<T, D, DV> pf;
  Frag<T> pfq[KS];
  load_chunk<T, D, DV>(pf, Kh, Vh, LGh, c_begin * CH, L, dv0, true, tid);
  if constexpr (!STATE_ONLY) {
    const int pos0 = c_begin * CH + 16 * I + r16;
    const T *Q0 = Qbase + ((size_t)b * p.Hq + kvh * G) * (size_t)L * D;
#pragma unroll
    for (int j = 0; j < KS; ++j) pfq[j] = (pos0 < L) ? load8(Q0 + (size_t)pos0 * D + 32 * j + 8 * g4) : frag_zero<T>();
  }
  __syncthreads();  // prologue LDS writes complete
  if constexpr (!STATE_ONLY) {
    // operand copy S^T [dv][f]
#pragma unroll
    for (int ft = 0; ft < FTW; ++ft)
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
        store4<T>(sSbf + (16 * dt + r16) * LDB + 16 * (wv * FTW + ft) + 4 * g4, S[ft][dt][0], S[ft][dt][1],
                  S[ft][dt][2], S[ft][dt][3]);
  }

  for (int c = c_begin; c < c_end; ++c) {
    const int c0 = c * CH;
    const int kcur = (c % KR) * (CH * LDW);
    const int cur = (c % NR) * (DV * LDC);
    const int kprev = ((c + KR - 1) % KR) * (CH * LDW);  // used only when KR >= 2
    const int vprev = ((c + NR - 1) % NR) * (DV * LDC);
    // ---- this chunk's keys, values, log gamma (loaded one chunk ahead) -> LDS
    store_keys<T, D, DV, LDW>(pf, sKr + kcur, tid);
    store_values<T, D, DV, LDC>(pf, sVt + cur, tid);
    store_lgT<T, D, DV, LDG>(pf, sLgT, tid);
    Frag<T> qf[KS];
    if constexpr (!STATE_ONLY) {
#pragma unroll
      for (int j = 0; j < KS; ++j) qf[j] = pfq[j];
    }
    // ---- state-only variant: next chunk in flight during this one (the full kernel issues
    //      it after the query loop, where fewer registers are live)
    if constexpr (STATE_ONLY) {
      if (c + 1 < c_end) load_chunk<T, D, DV>(pf, Kh, Vh, LGh, c0 + CH, L, dv0, true, tid);
    }
    __syncthreads();  // B0: this chunk in LDS

    const int pos = c0 + 16 * I + r16;
    const bool valid = pos < L;
    // ---- prefix / exclusive suffix sums of log gamma within the sub-chunk (MFMA with 0/1 matrices)
    float pfx[NFT][4], sfx[NFT][4];
#pragma unroll
    for (int ft = 0; ft < NFT; ++ft) {
      const Frag<T> a = (g4 < 2) ? load8(sLgT + (16 * ft + r16) * LDG + 16 * I + 8 * g4) : frag_zero<T>();
      const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
      const f32x4 pp = mma(a, tri_pre, zero);
      const f32x4 ss = mma(a, tri_suf, zero);
#pragma unroll
      for (int i = 0; i < 4; ++i) { pfx[ft][i] = pp[i]; sfx[ft][i] = ss[i]; }
    }
    if (r16 == 15 || r16 == 7) {
      float *dst = (r16 == 15 ? sTot : sP7) + I * D + 4 * g4;
#pragma unroll
      for (int ft = 0; ft < NFT; ++ft)
        *reinterpret_cast<f32x4 *>(dst + 16 * ft) = f32x4{pfx[ft][0], pfx[ft][1], pfx[ft][2], pfx[ft][3]};
    }

    // ---- phi_k for own rows (keys decayed to the sub-chunk end); phi_q of the first query
    //      head (queries decayed from the sub-chunk start), sharing W reads when W_phi is shared
    float ko[NFT][4];
    float qo[NFT][4];
    {
      Frag<T> kf[KS];
#pragma unroll
      for (int j = 0; j < KS; ++j) kf[j] = load8(sKr + kcur + (16 * I + r16) * LDW + 32 * j + 8 * g4);
      f32x4 z[NFT];
      if constexpr (STATE_ONLY) {
        feature_logits<T, D, LDW>(sWk, kf, r16, g4, z);
      } else {
        f32x4 zq[NFT];
        if (ly.wq == ly.wk) {
          feature_logits2<T, D, LDW>(sWk, kf, qf, r16, g4, z, zq);
        } else {
          feature_logits<T, D, LDW>(sWk, kf, r16, g4, z);
          feature_logits<T, D, LDW>(sWq, qf, r16, g4, zq);
        }
        softmax_rows<NFT>(zq, qo);
#pragma unroll
        for (int ft = 0; ft < NFT; ++ft)
#pragma unroll
          for (int i = 0; i < 4; ++i) qo[ft][i] *= __expf(pfx[ft][i]);
      }
      softmax_rows<NFT>(z, ko);
#pragma unroll
      for (int ft = 0; ft < NFT; ++ft)
#pragma unroll
        for (int i = 0; i < 4; ++i) ko[ft][i] *= __expf(sfx[ft][i]);
    }
    bool safe = true;
    if constexpr (!STATE_ONLY) {
      float span = 0.f;  // -tot = -(prefix + suffix) at any row
#pragma unroll
      for (int ft = 0; ft < NFT; ++ft)
#pragma unroll
        for (int i = 0; i < 4; ++i) span = fmaxf(span, -(pfx[ft][i] + sfx[ft][i]));
      safe = wave_max_all(span) <= SPAN_MAX;
    }
    __syncthreads();  // B1: sub-chunk totals visible, log gamma^T consumed

    // ---- per-feature tables for this chunk; decayed keys -> LDS [s][f]
    {
      constexpr int PER = 4 / (256 / D);  // sub-chunks handled per thread
      const int f = tid % D, j0 = (tid / D) * PER;
#pragma unroll
      for (int jj = 0; jj < PER; ++jj) {
        const int J = j0 + jj;
        const float tt = sTot[J * D + f];
        sETot[J * D + f] = __expf(tt);
        if constexpr (STATE_ONLY) {
          dsum += tt;
        } else {
          const float p7 = sP7[J * D + f];
          sENP7[J * D + f] = __expf(-p7);
          sENR8[J * D + f] = __expf(p7 - tt);
        }
      }
    }
#pragma unroll
    for (int ft = 0; ft < NFT; ++ft)
      store4<T>(sKown + (16 * I + r16) * LDB + 16 * ft + 4 * g4, ko[ft][0], ko[ft][1], ko[ft][2], ko[ft][3]);
    __syncthreads();  // B2: tables and keys visible

    if constexpr (!STATE_ONLY) {
      // diagonal-block key operand: ko e^{p7 - tot} (reference at row 7)
      Frag<T> kmid[KS];
      if (safe) {
#pragma unroll
        for (int js = 0; js < KS; ++js) {
          float t8[8], x[8];
          tab8(sENR8 + I * D, js, g4, t8);
#pragma unroll
          for (int jj = 0; jj < 8; ++jj) x[jj] = ko[2 * js + (jj >> 2)][jj & 3] * t8[jj];
          kmid[js] = frag_from<T>(x);
        }
      }

      for (int g = 0; g < G; ++g) {
        const int hq = kvh * G + g;
        if (p.per_head_q && G > 1) {  // a different W_phi_q for every query head
          __syncthreads();
          load_wT<T, D, LDW>(sWq, reinterpret_cast<const T *>(p.wq) + (size_t)hq * p.w_stride, tid);
          __syncthreads();
        }
        const T *Qh = Qbase + ((size_t)b * p.Hq + hq) * (size_t)L * D;
        if (g > 0) {
          // later query heads: phi_q here, qo = phi_q e^{prefix} (<= 1)
#pragma unroll
          for (int j = 0; j < KS; ++j)
            qf[j] = valid ? load8(Qh + (size_t)pos * D + 32 * j + 8 * g4) : frag_zero<T>();
          f32x4 z[NFT];
          feature_logits<T, D, LDW>(sWq, qf, r16, g4, z);
          softmax_rows<NFT>(z, qo);
#pragma unroll
          for (int ft = 0; ft < NFT; ++ft)
#pragma unroll
            for (int i = 0; i < 4; ++i) qo[ft][i] *= __expf(pfx[ft][i]);
        }

        // ---- intra-chunk scores A^T[s][t] for key sub-chunks J <= I
        f32x4 at[4];
#pragma unroll
        for (int J = 0; J < 4; ++J) at[J] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int J = 0; J < 3; ++J) {
          if (J < I) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int js = 0; js < KS; ++js) {
              float x[8];
#pragma unroll
              for (int jj = 0; jj < 8; ++jj) x[jj] = qo[2 * js + (jj >> 2)][jj & 3];
              // prod_{J<J'<I} e^{tot_J'} joins the two references
#pragma unroll
              for (int J2 = 1; J2 < 3; ++J2) {
                if (J2 > J && J2 < I) {
                  float t8[8];
                  tab8(sETot + J2 * D, js, g4, t8);
#pragma unroll
                  for (int jj = 0; jj < 8; ++jj) x[jj] *= t8[jj];
                }
              }
              const T *kr = sKown + (16 * J + r16) * LDB + 32 * js + 4 * g4;
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
              float t8[8], x[8];
              tab8(sENP7 + I * D, js, g4, t8);
#pragma unroll
              for (int jj = 0; jj < 8; ++jj) x[jj] = qo[2 * js + (jj >> 2)][jj & 3] * t8[jj];
              acc = mma(kmid[js], frag_from<T>(x), acc);
            }
          } else {
            // exact: A[t][s] = sum_f phi_q[t][f] phi_k[s][f] e^{p_t[f] - p_s[f]}, with phi
            // recomputed in fp32 (rare path: a sub-chunk whose log decay spans > SPAN_MAX)
            float phk[NFT][4], phq[NFT][4];
            {
              Frag<T> kf[KS];
#pragma unroll
              for (int j = 0; j < KS; ++j) kf[j] = load8(sKr + kcur + (16 * I + r16) * LDW + 32 * j + 8 * g4);
              f32x4 z[NFT];
              feature_logits<T, D, LDW>(sWk, kf, r16, g4, z);
              softmax_rows<NFT>(z, phk);
              feature_logits<T, D, LDW>(sWq, qf, r16, g4, z);
              softmax_rows<NFT>(z, phq);
            }
#pragma unroll 1
            for (int s2 = 0; s2 < 16; ++s2) {
              float part = 0.f;
#pragma unroll
              for (int ft = 0; ft < NFT; ++ft)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                  const float pk = __shfl(phk[ft][i], 16 * g4 + s2);
                  const float bs = __shfl(pfx[ft][i], 16 * g4 + s2);
                  const float term = phq[ft][i] * pk * __expf(pfx[ft][i] - bs);
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
#pragma unroll
        for (int js = 0; js < KS; ++js) {
          float x[8];
#pragma unroll
          for (int jj = 0; jj < 8; ++jj) x[jj] = qo[2 * js + (jj >> 2)][jj & 3];
          // prod_{J<I} e^{tot_J}: decay from the chunk start to the sub-chunk start
#pragma unroll
          for (int J2 = 0; J2 < 3; ++J2) {
            if (J2 < I) {
              float t8[8];
              tab8(sETot + J2 * D, js, g4, t8);
#pragma unroll
              for (int jj = 0; jj < 8; ++jj) x[jj] *= t8[jj];
            }
          }
          const Frag<T> bf = frag_from<T>(x);
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt) {
            const T *sr = sSbf + (16 * dt + r16) * LDB + 32 * js + 4 * g4;
            yacc[dt] = mma(load4x2(sr, sr + 16), bf, yacc[dt]);
          }
        }

        // ---- anchor window: meta keys + keys j with pos-W < j <= pos
        f32x4 ywin[NDT];
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) ywin[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
        float l_run = 0.f;
        if (win_fast) {
          // W <= 65 and two chunks of keys/values in the rings: exactly the meta tile and the
          // five 16-key tiles ending at this sub-chunk, one softmax pass.  Band tile u (1..5)
          // starts at chunk-relative row 16 (I - 5 + u); kj - pos = 16u - 80 + 4 g4 + i - r16.
          f32x4 lt[6];
          {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < KS; ++j) acc = mma(load8(sTk + r16 * LDW + 32 * j + 8 * g4), qf[j], acc);
#pragma unroll
            for (int i = 0; i < 4; ++i) lt[0][i] = ((wmask >> i) & 1u) ? acc[i] * scale : NEG_BIG;
          }
#pragma unroll
          for (int u = 1; u < 6; ++u) {
            const int rt = I - 5 + u;  // chunk-relative tile, < 0: previous chunk
            const T *kr = sKr + (rt < 0 ? kprev + (rt + 4) * 16 * LDW : kcur + rt * 16 * LDW) + r16 * LDW + 8 * g4;
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < KS; ++j) acc = mma(load8(kr + 32 * j), qf[j], acc);
            const uint32_t mu = (c == 0 ? wmask0 : wmask) >> (4 * u);
#pragma unroll
            for (int i = 0; i < 4; ++i) lt[u][i] = ((mu >> i) & 1u) ? acc[i] * scale : NEG_BIG;
          }
          float bm = NEG_BIG;
#pragma unroll
          for (int u = 0; u < 6; ++u)
#pragma unroll
            for (int i = 0; i < 4; ++i) bm = fmaxf(bm, lt[u][i]);
          bm = wave_max_cols(bm);
#pragma unroll
          for (int pr = 0; pr < 3; ++pr) {
            float x[8];
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const float pv = __expf(lt[2 * pr + h][i] - bm);  // masked: exp(-1e30) = 0
                x[4 * h + i] = pv;
                l_run += pv;
              }
            const Frag<T> bf = frag_from<T>(x);
            const int ua = 2 * pr, ub = 2 * pr + 1;
            const int rta = I - 5 + ua, rtb = I - 5 + ub;
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt) {
              const int dvl = 16 * dt + r16;
              const T *pa = (ua == 0) ? sTvT + dvl * LDM + 4 * g4
                                      : sVt + (rta < 0 ? vprev + 16 * (rta + 4) : cur + 16 * rta) + dvl * LDC + 4 * g4;
              const T *pb = sVt + (rtb < 0 ? vprev + 16 * (rtb + 4) : cur + 16 * rtb) + dvl * LDC + 4 * g4;
              ywin[dt] = mma(load4x2(pa, pb), bf, ywin[dt]);
            }
          }
        } else {
          // general window: batches of key tiles with an online softmax
          float m_run = NEG_BIG;
          const int kt_hi = (c0 >> 4) + I;
          const int lo_key = c0 + 16 * I - p.W + 1;
          const int kt_lo = max(lo_key >> 4, -((hist_avail + 15) >> 4));
        const int kj_floor = max(pos - p.W, -hist_avail - 1);  // keys above: window and history
          // tile list: u = -1 is the meta tile (if M > 0), then kt_lo..kt_hi
          const int u_first = (p.M > 0) ? -1 : 0;
          const int n_tiles = (kt_hi - kt_lo + 1) - u_first;
          for (int u0 = 0; u0 < n_tiles; u0 += WIN_BATCH) {
            f32x4 lt[WIN_BATCH];
#pragma unroll
            for (int uu = 0; uu < WIN_BATCH; ++uu) {
              const int u = u0 + uu;
              lt[uu] = f32x4{NEG_BIG, NEG_BIG, NEG_BIG, NEG_BIG};
              if (u < n_tiles) {
                const int kt = (u + u_first < 0) ? KT_META : kt_lo + u + u_first;
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
                if (kt == KT_META) {
#pragma unroll
                  for (int j = 0; j < KS; ++j) acc = mma(load8(sTk + r16 * LDW + 32 * j + 8 * g4), qf[j], acc);
#pragma unroll
                  for (int i = 0; i < 4; ++i) lt[uu][i] = (4 * g4 + i < p.M) ? acc[i] * scale : NEG_BIG;
                } else {
                  const int kc = kt >> 2;
                  if (kc > c - KR) {
                    const T *kr = sKr + pmod(kc, KR) * (CH * LDW) + (16 * (kt & 3) + r16) * LDW + 8 * g4;
#pragma unroll
                    for (int j = 0; j < KS; ++j) acc = mma(load8(kr + 32 * j), qf[j], acc);
                  } else {
                    // key tile older than the LDS ring: global memory
                    const int key = 16 * kt + r16;

                    const bool kv = key < L && key >= -hist_avail;

                    const T *krow = (kt >= 0 ? Kh : Hk + (size_t)p.hist_rows * D) + (ptrdiff_t)key * D;  // tiles never straddle 0
#pragma unroll
                    for (int j = 0; j < KS; ++j) {
                      const Frag<T> a = kv ? load8(krow + 32 * j + 8 * g4) : frag_zero<T>();
                      acc = mma(a, qf[j], acc);
                    }
                  }
#pragma unroll
                  for (int i = 0; i < 4; ++i) {
                    const int kj = 16 * kt + 4 * g4 + i;
                    lt[uu][i] = (kj <= pos && kj > kj_floor) ? acc[i] * scale : NEG_BIG;
                  }
                }
              }
            }
            float bm = NEG_BIG;
#pragma unroll
            for (int uu = 0; uu < WIN_BATCH; ++uu)
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
            // P V: pairs of tiles form one K = 32 step
#pragma unroll
            for (int pr = 0; pr < WIN_BATCH / 2; ++pr) {
              const int ua = u0 + 2 * pr, ub = ua + 1;
              if (ua >= n_tiles) continue;
              float x[8];
#pragma unroll
              for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                  const float l = lt[2 * pr + h][i];
                  const float pv = (l > 0.5f * NEG_BIG) ? __expf(l - m_new) : 0.f;
                  x[4 * h + i] = pv;
                  l_run += pv;
                }
              const Frag<T> bf = frag_from<T>(x);
              const int kta = (ua + u_first < 0) ? KT_META : kt_lo + ua + u_first;
              const int ktb = (ub >= n_tiles) ? KT_NONE : kt_lo + ub + u_first;
              const bool ring_a = kta != KT_META && (kta >> 2) > c - NR;
              const bool ring_b = ktb != KT_NONE && (ktb >> 2) > c - NR;
#pragma unroll
              for (int dt = 0; dt < NDT; ++dt) {
                const int dvl = 16 * dt + r16;
                const T *pa = (kta == KT_META) ? sTvT + dvl * LDM + 4 * g4
                                        : sVt + pmod(kta >> 2, NR) * (DV * LDC) + dvl * LDC + 16 * (kta & 3) + 4 * g4;
                const T *pb = (ktb == KT_NONE) ? pa : sVt + pmod(ktb >> 2, NR) * (DV * LDC) + dvl * LDC + 16 * (ktb & 3) + 4 * g4;
                Frag<T> af;
                if ((kta == KT_META || ring_a) && (ktb == KT_NONE || ring_b)) {
                  af = load4x2(pa, pb);  // slots of a missing second tile meet P = 0
                } else {
                  // a value tile older than the LDS ring: gather from global memory
                  float av[8];
#pragma unroll
                  for (int h = 0; h < 2; ++h) {
                    const int kt = h ? ktb : kta;
                    const bool inring = h ? ring_b : ring_a;
                    if (kt == KT_NONE) {
#pragma unroll
                      for (int i = 0; i < 4; ++i) av[4 * h + i] = 0.f;
                    } else if (kt == KT_META || inring) {
                      float t4[4];
                      load4f(h ? pb : pa, t4);
#pragma unroll
                      for (int i = 0; i < 4; ++i) av[4 * h + i] = t4[i];
                    } else {
#pragma unroll
                      for (int i = 0; i < 4; ++i) {
                        const int key = 16 * kt + 4 * g4 + i;
                        av[4 * h + i] = (key < L && key >= -hist_avail)
                        ? to_f((kt >= 0 ? Vh : Hv + (size_t)p.hist_rows * D)[(ptrdiff_t)key * D + dv0 + dvl])
                        : 0.f;
                      }
                    }
                  }
                  af = frag_from<T>(av);
                }
                ywin[dt] = mma(af, bf, ywin[dt]);
              }
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
      // next chunk's keys, values, log gamma and first query head in flight during the state update
      if (c + 1 < c_end) {
        load_chunk<T, D, DV>(pf, Kh, Vh, LGh, c0 + CH, L, dv0, true, tid);
        const int pn = pos + CH;
        const T *Q0 = Qbase + ((size_t)b * p.Hq + kvh * G) * (size_t)L * D;
#pragma unroll
        for (int j = 0; j < KS; ++j) pfq[j] = (pn < L) ? load8(Q0 + (size_t)pn * D + 32 * j + 8 * g4) : frag_zero<T>();
      }
    }
    __syncthreads();  // B3: all reads of the state copy done

    // ---- state update on owned rows: S = diag(prod_J e^{tot_J}) S + sum_s KSt[s] v_s^T with
    //      KSt[s][f] = ko[s][f] prod_{J' > J(s)} e^{tot_J'}[f] gathered from LDS
#pragma unroll
    for (int ft = 0; ft < FTW; ++ft) {
      const int fr = 16 * (wv * FTW + ft);
      float e[4] = {1.f, 1.f, 1.f, 1.f};
#pragma unroll
      for (int J = 0; J < 4; ++J) {
        const f32x4 t = *reinterpret_cast<const f32x4 *>(sETot + J * D + fr + 4 * g4);
#pragma unroll
        for (int i = 0; i < 4; ++i) e[i] *= t[i];
      }
      float et[4];
#pragma unroll
      for (int J = 0; J < 4; ++J) et[J] = sETot[J * D + fr + r16];
      Frag<T> ka[2];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const int J = 2 * ks + (g4 >> 1);  // rows 32ks + 8g4 .. +7 lie in sub-chunk J
        float fac = 1.f;
#pragma unroll
        for (int J2 = 1; J2 < 4; ++J2)
          if (J2 > J) fac *= et[J2];
        float x[8];
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) x[jj] = to_f(sKown[(32 * ks + 8 * g4 + jj) * LDB + fr + r16]) * fac;
        ka[ks] = frag_from<T>(x);
      }
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) S[ft][dt][i] *= e[i];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
          S[ft][dt] = mma(ka[ks], load8(sVt + cur + (16 * dt + r16) * LDC + 32 * ks + 8 * g4), S[ft][dt]);
        if constexpr (!STATE_ONLY)
          store4<T>(sSbf + (16 * dt + r16) * LDB + fr + 4 * g4, S[ft][dt][0], S[ft][dt][1], S[ft][dt][2],
                    S[ft][dt][3]);
      }
    }
    __syncthreads();  // B4: new state copy visible; LDS buffers free for the next chunk
  }

  if constexpr (!STATE_ONLY) {
    if (p.state_out && seg == p.nseg - 1) {  // the state after the last token
      float *So = p.state_out + ((size_t)b * p.Hkv + kvh) * D * D;
#pragma unroll
      for (int ft = 0; ft < FTW; ++ft)
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            So[(size_t)(16 * (wv * FTW + ft) + 4 * g4 + i) * D + dv0 + 16 * dt + r16] = S[ft][dt][i];
    }
  }
  if constexpr (STATE_ONLY) {
    float *E = p.ws_state + ((((size_t)b * p.Hkv + kvh) * p.ndvb + dvb) * (p.nseg - 1) + seg) * st_per_grp;
#pragma unroll
    for (int ft = 0; ft < FTW; ++ft)
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
        *reinterpret_cast<f32x4 *>(E + (((size_t)(wv * FTW + ft) * NDT + dt) * 64 + lane) * 4) = S[ft][dt];
    // thread tid accumulated features tid % D for sub-chunks of its quarter/half; combine
    __shared__ float sDs[256];
    sDs[tid] = dsum;
    __syncthreads();
    if (dvb == 0 && tid < D) {
      float s = 0.f;
      for (int h = 0; h < 256 / D; ++h) s += sDs[tid + h * D];
      p.ws_decay[(((size_t)b * p.Hkv + kvh) * (p.nseg - 1) + seg) * D + tid] = s;
    }
  }
}

// ---------------------------------------------------------------- host side
template <typename T, int D, int DV, bool STATE_ONLY, bool WIDE>
static hipError_t launch_one(const FwdParams &p, hipStream_t stream) {
  const int grid = ((p.ngroups + 7) / 8) * 8 * p.ndvb;
  auto kern = fwd_kernel<T, D, DV, STATE_ONLY, WIDE>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, p.lds.total);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(256), p.lds.total, stream, p);
  return hipGetLastError();
}

// Deepest value / key rings that fit in LDS (tiles older than a ring are read from
// global memory); false when no layout fits.
template <typename T, int D, int DV, bool WIDE>
static bool plan_rings(FwdParams &p, bool shared_w) {
  for (int nr = p.nring; nr >= 2; --nr)
    for (int kr = nr; kr >= 1; --kr) {
      const FwdLds l = make_lds<T, D, DV, WIDE>(false, shared_w, nr, kr);
      if (l.total <= LDS_LIMIT) {
        p.lds = l;
        p.nring = nr;
        p.kring = kr;
        return true;
      }
    }
  return false;
}

template <typename T, int D, int DV, bool WIDE>
static hipError_t launch_fwd_w(const FwdParams &prm, bool shared_w, hipStream_t stream) {
  FwdParams p = prm;
  if (p.full) {
    p.ngroups = p.B * p.Hkv * p.nseg;
    return launch_fwd_full(p, stream);
  }
  if (p.nseg > 1) {
    FwdParams s = p;
    s.ngroups = p.B * p.Hkv * (p.nseg - 1);
    s.nring = 1;
    s.kring = 1;
    s.lds = make_lds<T, D, DV, WIDE>(true, shared_w, 1, 1);
    hipError_t e = launch_one<T, D, DV, true, WIDE>(s, stream);
    if (e != hipSuccess) return e;
  }
  p.ngroups = p.B * p.Hkv * p.nseg;
  if (!plan_rings<T, D, DV, WIDE>(p, shared_w)) return hipErrorInvalidConfiguration;
  // The role-split kernel serves one query head per key/value head; grouped query heads
  // (whose per-head work would fall on the query waves alone) run on the 4-wave kernel.
  if (!p.force_4wave && p.G == 1) return launch_fwd_split<T, D, DV, WIDE>(p, stream);
  return launch_one<T, D, DV, false, WIDE>(p, stream);
}

// The wide row stride when the full-depth rings fit with it, else the narrow one.
template <typename T, int D, int DV>
static hipError_t launch_fwd_t(const FwdParams &prm, hipStream_t stream) {
  const bool shared_w = (prm.wq == prm.wk) && prm.w_stride == 0;
  FwdParams probe = prm;
  const bool wide = plan_rings<T, D, DV, true>(probe, shared_w) && probe.nring == prm.nring && probe.kring == prm.nring;
  return wide ? launch_fwd_w<T, D, DV, true>(prm, shared_w, stream) : launch_fwd_w<T, D, DV, false>(prm, shared_w, stream);
}

hipError_t launch_fwd(const FwdParams &p, int dtype_bf16, int d, hipStream_t stream) {
  if (dtype_bf16) {
    if (d == 64) return launch_fwd_t<bf16, 64, 64>(p, stream);
    if (d == 128) return launch_fwd_t<bf16, 128, 64>(p, stream);
  } else {
    if (d == 64) return launch_fwd_t<float, 64, 64>(p, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace lz
