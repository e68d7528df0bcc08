// Lizard attention decode step for gfx950: one new token per sequence.
//
// Per (sequence n, key/value head hk), the arithmetic of one recurrent step
// (Lizard: An Efficient Linearization Framework for LLMs, papernotes.org
// summary, "key designs": Gated Linear Attention and Anchor Window Attention
// items; the arXiv page's Preliminaries note that the recurrent form gives
// constant-memory generation):
//   S <- diag(gamma_t) S + phi_k(k_t) v_t^T            (fp32 state, in place)
//   y_gla = phi_q(q_t)^T S                               (every query head of hk)
//   ring[pos % W] <- (k_t, v_t)
//   y_win = softmax over M meta keys + min(pos+1, W) ring keys
//   out = mix y_gla + (1-mix) y_win
//
// Two kernels:
//   decode_phi   every feature map of the step as one small GEMM on the matrix
//                cores: rows are the new keys (per key/value head) and queries
//                (per query head) of 64 sequences, times W_phi staged in LDS
//                (bf16: as stored, the operand read transposed; fp32:
//                transposed when staged), then the softmax over features (or
//                the Hedgehog map's exponential).  fp32 results go to the
//                workspace.
//   decode_step  one workgroup per (sequence, key/value head), bound by HBM
//                traffic.  It issues its loads in the order it consumes them
//                -- the per-token vectors and meta tokens, the ring
//                keys/values, then its fp32 state rows -- because the memory
//                counter retires loads in order: the window branch then runs
//                while the state is still in flight.  Then it decays and
//                updates the state, writes it back, reads out phi_q^T S and
//                merges.  The last workgroup of a
//                sequence to finish (a counter in the workspace, cleared by
//                decode_phi) advances pos: by then every workgroup of that
//                sequence has read it.
#include "common.hpp"
#include "internal.hpp"

namespace lz {

constexpr int DEC_MAXG = 2;   // query heads per key/value head per pass (grouped heads; four spilled)
constexpr int DEC_MAXW = 256; // ring length limit
constexpr int DEC_MAXM = 16;
constexpr int DEC_RKEYS = 64; // ring keys per logits pass (4 lanes per key)
constexpr int DEC_ROWS = 64;  // sequences per decode_phi workgroup
constexpr float DEC_NEG = -1.0e30f;

// Keeps the compiler from converting a fragment to fp32 ahead of its use
// (which would double the registers it occupies across the head loop).
template <typename T> __device__ __forceinline__ void opaque(Frag<T> &f) {
  if constexpr (sizeof(T) == 2) {
    asm volatile("" : "+v"(f.v));
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) asm volatile("" : "+v"(f.v[j]));
  }
}

// grid (ceil(N / 64), Hkv + Hq): y < Hkv is the key side of key/value head y,
// otherwise query head y - Hkv.  Wave w owns rows 16w .. 16w+15 of the tile.
// HH: the Hedgehog map, phi(x) = exp(xW) (+) exp(-xW) with W_phi [D][D/2] (W^T staged with its
// negation below it, so the logits of the D features are (xW, -xW)); no normalisation.
template <typename T, int D, bool HH>
__global__ __launch_bounds__(256) void decode_phi_kernel(DecParams p) {
  constexpr int LDW = D + 16 / (int)sizeof(T);  // padded row of W^T (elements)
  constexpr int NC = D / 16;                    // 16-column output tiles
  constexpr int KS = D / 32;                    // K = 32 steps
  __shared__ __align__(16) T wt[D * LDW];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int r = lane & 15, kq = lane >> 4;
  const int Hkv = p.Hkv, Hq = p.Hq, G = p.G, N = p.N;
  const int hs = blockIdx.y;
  const bool key = hs < Hkv;
  const int h = key ? hs : hs - Hkv;
  const int n0 = blockIdx.x * DEC_ROWS;

  if (hs == 0 && tid < DEC_ROWS && n0 + tid < N) p.ws_count[n0 + tid] = 0;

  const T *Wsrc = reinterpret_cast<const T *>(key ? p.wk : p.wq) + (size_t)h * p.w_stride;
  constexpr int FC = HH ? D / 2 : D;  // columns of W_phi
  // W[i][f] -> wt[f][i] (and -W -> wt[FC + f][i]).  The lanes of a wave take consecutive rows i
  // (pairs of rows for 2-byte types, so that each lane writes one 4-byte word per feature): a
  // wave's writes to a row of wt fall in distinct banks.  Every load below is issued before the
  // first LDS write.
  constexpr int RP = sizeof(T) == 2 ? 2 : 1;  // rows of W per item
  constexpr int NR = D / RP;                  // row items
  constexpr int NI = NR * (FC / 8);           // (row item, 8-column group) items
  constexpr int IT = (NI + 255) / 256;
  Frag<T> wa[IT][RP];
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int idx = min(tid + 256 * it, NI - 1);
    const int i0 = RP * (idx % NR), f0 = 8 * (idx / NR);
#pragma unroll
    for (int u = 0; u < RP; ++u) wa[it][u] = load8(Wsrc + (size_t)(i0 + u) * FC + f0);
  }

  // A fragments straight from global: row n = n0 + 16*wv + r
  const int n = min(n0 + 16 * wv + r, N - 1);
  const T *X = reinterpret_cast<const T *>(key ? p.k : p.q) + ((size_t)n * (key ? Hkv : Hq) + h) * D;
  Frag<T> a[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) a[s] = load8(X + 32 * s + 8 * kq);  // rows past N: clamped, not stored

#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int idx = tid + 256 * it;
    if (NI % 256 == 0 || idx < NI) {
      const int i0 = RP * (idx % NR), f0 = 8 * (idx / NR);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if constexpr (RP == 2) {
          T pair[2] = {wa[it][0].v[j], wa[it][1].v[j]};
          const uint32_t u = *reinterpret_cast<const uint32_t *>(pair);
          *reinterpret_cast<uint32_t *>(wt + (f0 + j) * LDW + i0) = u;
          if constexpr (HH) *reinterpret_cast<uint32_t *>(wt + (FC + f0 + j) * LDW + i0) = u ^ 0x80008000u;
        } else {
          wt[(f0 + j) * LDW + i0] = wa[it][0].v[j];
          if constexpr (HH) wt[(FC + f0 + j) * LDW + i0] = -wa[it][0].v[j];
        }
      }
    }
  }
  __syncthreads();

  f32x4 acc[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KS; ++s) acc[c] = mma(a[s], load8(wt + (16 * c + r) * LDW + 32 * s + 8 * kq), acc[c]);
  }

  // lane (r, kq) holds z[row 16wv + 4kq + i][feature 16c + r]; softmax over features
  const int hk = key ? h : h / G;
  const int sub = key ? 0 : 1 + h % G;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float inv = 1.f;
    if constexpr (HH) {
#pragma unroll
      for (int c = 0; c < NC; ++c) acc[c][i] = __expf(acc[c][i]);
    } else {
      float m = DEC_NEG;
#pragma unroll
      for (int c = 0; c < NC; ++c) m = fmaxf(m, acc[c][i]);
      m = row_max16(m);  // over the 16 lanes of the row (DPP, no LDS round trip)
      float s = 0.f;
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        acc[c][i] = __expf(acc[c][i] - m);
        s += acc[c][i];
      }
      inv = 1.f / row_sum16(s);
    }
    const int nr = n0 + 16 * wv + 4 * kq + i;
    if (nr < N) {
      float *dst = p.ws_phi + (((size_t)nr * Hkv + hk) * (1 + G) + sub) * D;
#pragma unroll
      for (int c = 0; c < NC; ++c) dst[16 * c + r] = acc[c][i] * inv;
    }
  }
}

// decode_phi for 16-bit inputs: W_phi staged in LDS as it is stored ([D][FC] rows, plain 16-byte
// copies) and the logits computed transposed, z^T = W_phi^T x^T: the MFMA's A operand (feature m,
// input dims k) comes from W's rows by transposing LDS reads (ds_read_b64_tr_b16: in a group of 16
// lanes, lane m reads 4 values of row m / 4 at column 4 (m % 4), and lane i receives column i of
// the 4 rows), and its B operand is the raw rows x as loaded.  Lane (r, kq) then holds row r's
// features 16 c + 4 kq + i, i = 0..3: the softmax reduces over the lane's 32 values and the 4
// lanes of the row, and each lane stores its features 16 bytes at a time.  The Hedgehog map's
// second half, exp(-xW), is the negation of the same logits (negating W negates every product
// exactly).
template <int D, bool HH>
__global__ __launch_bounds__(256) void decode_phi_b16_kernel(DecParams p) {
  using T = bf16;
  typedef short v4s __attribute__((ext_vector_type(4)));
  constexpr int FC = HH ? D / 2 : D;  // columns of W_phi
  constexpr int LDR = FC + 16;        // LDS row stride (elements): 32 bytes past a multiple of 256
  constexpr int NCL = FC / 16;        // 16-feature tiles of logits
  constexpr int KS = D / 32;          // K = 32 steps
  constexpr int NP = D * FC / 8;      // 16-byte pieces of W
  static_assert(NP % 256 == 0, "pieces per thread");
  constexpr int IT = NP / 256;
  __shared__ __align__(16) T wl[D * LDR];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int r = lane & 15, kq = lane >> 4;
  const int Hkv = p.Hkv, Hq = p.Hq, G = p.G, N = p.N;
  const int hs = blockIdx.y;
  const bool key = hs < Hkv;
  const int h = key ? hs : hs - Hkv;
  const int n0 = blockIdx.x * DEC_ROWS;

  if (hs == 0 && tid < DEC_ROWS && n0 + tid < N) p.ws_count[n0 + tid] = 0;

  const T *Wsrc = reinterpret_cast<const T *>(key ? p.wk : p.wq) + (size_t)h * p.w_stride;
  Frag<T> wa[IT];
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int idx = tid + 256 * it;
    wa[it] = load8(Wsrc + (size_t)(idx / (FC / 8)) * FC + 8 * (idx % (FC / 8)));
  }
  // B operands straight from global: row n = n0 + 16 wv + r (rows past N clamped, not stored)
  const int n = min(n0 + 16 * wv + r, N - 1);
  const T *X = reinterpret_cast<const T *>(key ? p.k : p.q) + ((size_t)n * (key ? Hkv : Hq) + h) * D;
  Frag<T> x[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) x[s] = load8(X + 32 * s + 8 * kq);
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int idx = tid + 256 * it;
    *reinterpret_cast<bf16x8 *>(wl + (idx / (FC / 8)) * LDR + 8 * (idx % (FC / 8))) = wa[it].v;
  }
  __syncthreads();

  // acc[c][i] = z[row r][feature 16 c + 4 kq + i]
  // (the operands of tile c + 1 are read while tile c is multiplied)
  typedef unsigned int u2 __attribute__((ext_vector_type(2)));
  typedef unsigned int u4 __attribute__((ext_vector_type(4)));
  const T *wsrc = wl + (8 * kq + (r >> 2)) * LDR + 4 * (r & 3);
  auto wtile = [&](int c, Frag<T> (&a)[KS]) {
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const T *src = wsrc + 32 * s * LDR + 16 * c;
      const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s *)(src));
      const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s *)(src + 4 * LDR));
      const u2 l2 = __builtin_bit_cast(u2, lo), h2 = __builtin_bit_cast(u2, hi);
      a[s].v = __builtin_bit_cast(bf16x8, u4{l2.x, l2.y, h2.x, h2.y});
    }
  };
  f32x4 acc[NCL];
  Frag<T> wa2[2][KS];
  wtile(0, wa2[0]);
#pragma unroll
  for (int c = 0; c < NCL; ++c) {
    if (c + 1 < NCL) wtile(c + 1, wa2[(c + 1) & 1]);
    acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KS; ++s) acc[c] = mma(wa2[c & 1][s], x[s], acc[c]);
  }

  constexpr int NC = D / 16;  // feature tiles of phi
  float ph[NC][4];
  if constexpr (HH) {
#pragma unroll
    for (int c = 0; c < NCL; ++c)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        ph[c][i] = __expf(acc[c][i]);
        ph[NCL + c][i] = __expf(-acc[c][i]);
      }
  } else {
    float m = DEC_NEG;
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int i = 0; i < 4; ++i) m = fmaxf(m, acc[c][i]);
    m = wave_max_cols(m);
    float sum = 0.f;
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        ph[c][i] = __expf(acc[c][i] - m);
        sum += ph[c][i];
      }
    const float inv = 1.f / wave_sum_cols(sum);
#pragma unroll
    for (int c = 0; c < NC; ++c)
#pragma unroll
      for (int i = 0; i < 4; ++i) ph[c][i] *= inv;
  }
  const int hk = key ? h : h / G;
  const int sub = key ? 0 : 1 + h % G;
  const int nr = n0 + 16 * wv + r;
  if (nr < N) {
    float *dst = p.ws_phi + (((size_t)nr * Hkv + hk) * (1 + G) + sub) * D + 4 * kq;
#pragma unroll
    for (int c = 0; c < NC; ++c) *reinterpret_cast<f32x4 *>(dst + 16 * c) = f32x4{ph[c][0], ph[c][1], ph[c][2], ph[c][3]};
  }
}

// x summed over the lanes that share lane % O (O = 8, 16 or 32), in the order of an xor
// butterfly over O, 2 O, ..; every lane gets the same bits.
template <int O> __device__ __forceinline__ float sum_lanes_mod(float x) {
  static_assert(O == 8 || O == 16 || O == 32, "lane stride");
  if constexpr (O == 8) x += __shfl_xor(x, 8);
  if constexpr (O <= 16) x = pair16_sum(x);
  return pair32_sum(x);
}

template <typename T, int D, int GM>  // GM: query heads per pass (1 or DEC_MAXG)
__global__ __launch_bounds__(256, 2) void decode_step_kernel(DecParams p) {
  constexpr int C4 = D / 4;     // float4 columns per state row
  constexpr int RG = 256 / C4;  // row groups of the state
  constexpr int RPT = D / RG;   // state rows per thread
  constexpr int F8 = D / 8;     // 8-column pieces of a row
  constexpr int JG = 256 / F8;  // ring slot groups for 8-column work
  constexpr int QD = D / 4;     // quarter row (window logits: 4 lanes per key)
  constexpr int VPT = DEC_RKEYS / JG;  // value pieces per thread loaded up front
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int G = p.G, Hq = p.Hq, Hkv = p.Hkv, W = p.W, M = p.M;
  const int n = blockIdx.x / Hkv, hk = blockIdx.x % Hkv;
  const size_t nh = (size_t)n * Hkv + hk;

  __shared__ float sx[GM][D];        // raw queries of the pass
  __shared__ float sk[D], sv[D], sgam[D], sphik[D];
  __shared__ float sphq[GM][D];
  __shared__ float sy[GM][D];        // y_win of the pass
  __shared__ float sred[4][GM][D];   // per-wave partial sums
  __shared__ float slog[GM][DEC_MAXM + DEC_MAXW];
  __shared__ __align__(16) T stk[DEC_MAXM * D], stv[DEC_MAXM * D];  // meta keys / values

  const T *Q = reinterpret_cast<const T *>(p.q);
  const T *K = reinterpret_cast<const T *>(p.k);
  const T *V = reinterpret_cast<const T *>(p.v);
  const T *LG = reinterpret_cast<const T *>(p.lg);
  const T *Tk = reinterpret_cast<const T *>(p.tk);
  const T *Tv = reinterpret_cast<const T *>(p.tv);
  T *RK = reinterpret_cast<T *>(p.win_k);
  T *RV = reinterpret_cast<T *>(p.win_v);
  T *OUT = reinterpret_cast<T *>(p.out);
  const float *phi = p.ws_phi + nh * (size_t)(1 + G) * D;

  const int pn = p.pos[n];
  const int slot = pn % W;
  const int nvalid = min(pn + 1, W);
  const size_t rbase = nh * (size_t)W * D;
  float *St = p.state + nh * D * D;
  const int c4 = tid % C4, rg = tid / C4;  // state columns 4*c4 .., rows rg, rg+RG, ...

  // Every load below is unconditional, from an index clamped into bounds (a
  // conditional load becomes a branch that waits for all loads before it);
  // lanes whose index was clamped ignore what they read.
  // ---- 1. per-token vectors (thread tid < D owns element tid) and meta tokens
  const int gp0 = min(GM, G);
  const int te = tid % D;
  const float xk = to_f(K[nh * D + te]);
  const float xv = to_f(V[nh * D + te]);
  const float xg = to_f(LG[nh * D + te]);
  const float xpk = phi[te];
  float xq[GM], xpq[GM];
#pragma unroll
  for (int u = 0; u < GM; ++u) {
    const int uu = min(u, gp0 - 1);
    xq[u] = to_f(Q[((size_t)n * Hq + hk * G + uu) * D + te]);
    xpq[u] = phi[(size_t)(1 + uu) * D + te];
  }
  // meta tokens: thread tid < M * F8 takes row tid / F8, columns 8 * (tid % F8) ..
  const size_t toff = (size_t)hk * M * D + 8 * (size_t)min(tid, max(M * F8 - 1, 0));
  const Frag<T> tkf = load8(M > 0 ? Tk + toff : K);
  const Frag<T> tvf = load8(M > 0 ? Tv + toff : K);
  // ---- 2. ring key quarter and value pieces
  const int kq = tid / 4, kpart = tid % 4;  // ring slot kq (+ multiples of 64), dims kpart*QD ..
  Frag<T> kfr[QD / 8];
#pragma unroll
  for (int e8 = 0; e8 < QD / 8; ++e8)
    kfr[e8] = load8(RK + rbase + (size_t)min(kq, W - 1) * D + kpart * QD + 8 * e8);
  const int f8 = tid % F8, jg = tid / F8;   // value columns 8*f8 .., ring slots jg, jg+JG, ...
  Frag<T> vfr[VPT];
#pragma unroll
  for (int m = 0; m < VPT; ++m) vfr[m] = load8(RV + rbase + (size_t)min(jg + JG * m, W - 1) * D + 8 * f8);
  // ---- 3. the state rows
  f32x4 x[RPT];
#pragma unroll
  for (int rr = 0; rr < RPT; ++rr)
    x[rr] = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(St + (size_t)(rg + RG * rr) * D + 4 * c4));

  // LDS copies, written by every thread (duplicates carry equal values), so no
  // branch pulls the loads above down past the state loads
  sk[te] = xk;
  sv[te] = xv;
  sgam[te] = __expf(xg);
  sphik[te] = xpk;
  {
    const int tp = min(tid, max(M * F8 - 1, 0));
    *reinterpret_cast<Frag<T> *>(stk + 8 * tp) = tkf;
    *reinterpret_cast<Frag<T> *>(stv + 8 * tp) = tvf;
  }

  for (int g0 = 0; g0 < (GM == 1 ? 1 : G); g0 += GM) {  // GM = 1 runs only for G = 1
    const int gp = min(GM, G - g0);
    const bool first = (g0 == 0);
    if (first) {
#pragma unroll
      for (int u = 0; u < GM; ++u) {
        sx[u][te] = (u < gp0) ? xq[u] : 0.f;
        sphq[u][te] = (u < gp0) ? xpq[u] : 0.f;
      }
    } else {
      for (int idx = tid; idx < GM * D; idx += 256) {
        const int u = idx / D, e = idx % D;
        const bool on = u < gp;
        sx[u][e] = on ? to_f(Q[((size_t)n * Hq + hk * G + g0 + u) * D + e]) : 0.f;
        sphq[u][e] = on ? phi[(size_t)(1 + g0 + u) * D + e] : 0.f;
      }
    }
    __syncthreads();

    // ---- window logits over ring slots: slot jb + kq, quarter kpart (first pass from registers)
    for (int jb = 0; jb < W; jb += DEC_RKEYS) {
      const int jj = jb + kq;
      const bool in = jj < W;
      const int age = in ? ((slot - jj) % W + W) % W : W;  // pn - (token in slot jj)
      const bool ok = in && age < nvalid;
      float acc[GM];
#pragma unroll
      for (int u = 0; u < GM; ++u) acc[u] = 0.f;
      if (ok) {
#pragma unroll
        for (int e8 = 0; e8 < QD / 8; ++e8) {
          const int e0 = kpart * QD + 8 * e8;
          float kv8[8];
          if (jj == slot) {
#pragma unroll
            for (int t = 0; t < 8; ++t) kv8[t] = sk[e0 + t];
          } else if (jb == 0) {
            Frag<T> kk = kfr[e8];
            opaque(kk);
#pragma unroll
            for (int t = 0; t < 8; ++t) kv8[t] = to_f(kk.v[t]);
          } else {
            load8f(RK + rbase + (size_t)jj * D + e0, kv8);
          }
#pragma unroll
          for (int u = 0; u < GM; ++u)
#pragma unroll
            for (int t = 0; t < 8; ++t) acc[u] += sx[u][e0 + t] * kv8[t];
        }
      }
#pragma unroll
      for (int u = 0; u < GM; ++u) {
        acc[u] += dpp_f<DPP_XOR1>(acc[u]);
        acc[u] += dpp_f<DPP_XOR2>(acc[u]);
      }
      if (in && kpart == 0)
        for (int u = 0; u < gp; ++u) slog[u][M + jj] = ok ? acc[u] * p.scale : DEC_NEG;
    }
    for (int idx = tid; idx < gp * M; idx += 256) {  // meta keys
      const int u = idx / M, m = idx % M;
      float a = 0.f;
      for (int e = 0; e < D; ++e) a += sx[u][e] * to_f(stk[m * D + e]);
      slog[u][m] = a * p.scale;
    }
    __syncthreads();
    for (int u = wv; u < gp; u += 4) {  // softmax per head (one wave per head)
      float m = DEC_NEG;
      for (int j = lane; j < M + W; j += 64) m = fmaxf(m, slog[u][j]);
      m = wave_max_all(m);
      float sum = 0.f;
      for (int j = lane; j < M + W; j += 64) {
        const float ex = __expf(slog[u][j] - m);  // masked entries: exp(-1e30) = 0
        slog[u][j] = ex;
        sum += ex;
      }
      sum = wave_sum_cols(row_sum16(sum));
      const float inv = 1.f / sum;
      for (int j = lane; j < M + W; j += 64) slog[u][j] *= inv;
    }
    __syncthreads();

    // ---- y_win over ring slots: thread (f8, jg) sums slots jg, jg+JG, ... for columns 8*f8 ..
    {
      float acc[GM][8];
#pragma unroll
      for (int u = 0; u < GM; ++u)
#pragma unroll
        for (int t = 0; t < 8; ++t) acc[u][t] = 0.f;
#pragma unroll
      for (int m = 0; m < VPT; ++m) {  // slots whose values are already in registers
        const int j = jg + JG * m;
        if (j < W) {
          float vv[8];
          Frag<T> vk = vfr[m];
          opaque(vk);
#pragma unroll
          for (int t = 0; t < 8; ++t) vv[t] = (j == slot) ? sv[8 * f8 + t] : to_f(vk.v[t]);
#pragma unroll
          for (int u = 0; u < GM; ++u) {
            const float pj = slog[u][M + j];
#pragma unroll
            for (int t = 0; t < 8; ++t) acc[u][t] += pj * vv[t];
          }
        }
      }
      for (int j = jg + JG * VPT; j < W; j += JG) {  // longer rings
        float vv[8];
        if (j == slot) {
#pragma unroll
          for (int t = 0; t < 8; ++t) vv[t] = sv[8 * f8 + t];
        } else {
          load8f(RV + rbase + (size_t)j * D + 8 * f8, vv);
        }
#pragma unroll
        for (int u = 0; u < GM; ++u) {
          const float pj = slog[u][M + j];
#pragma unroll
          for (int t = 0; t < 8; ++t) acc[u][t] += pj * vv[t];
        }
      }
#pragma unroll
      for (int u = 0; u < GM; ++u)
#pragma unroll
        for (int t = 0; t < 8; ++t)
          acc[u][t] = sum_lanes_mod<F8>(acc[u][t]);
      if (lane < F8) {
#pragma unroll
        for (int u = 0; u < GM; ++u)
#pragma unroll
          for (int t = 0; t < 8; ++t) sred[wv][u][8 * f8 + t] = acc[u][t];
      }
    }

    // ---- state: S = diag(gamma) S + phi_k v^T (first pass), partial y = phi_q^T S
    if (first) {
      const float v0 = sv[4 * c4], v1 = sv[4 * c4 + 1], v2 = sv[4 * c4 + 2], v3 = sv[4 * c4 + 3];
#pragma unroll
      for (int rr = 0; rr < RPT; ++rr) {
        const int f = rg + RG * rr;
        const float gm = sgam[f], pk = sphik[f];
        x[rr][0] = gm * x[rr][0] + pk * v0;
        x[rr][1] = gm * x[rr][1] + pk * v1;
        x[rr][2] = gm * x[rr][2] + pk * v2;
        x[rr][3] = gm * x[rr][3] + pk * v3;
        __builtin_nontemporal_store(x[rr], reinterpret_cast<f32x4 *>(St + (size_t)f * D + 4 * c4));
      }
    }
    float yp[GM][4];
#pragma unroll
    for (int u = 0; u < GM; ++u) {
#pragma unroll
      for (int i = 0; i < 4; ++i) yp[u][i] = 0.f;
#pragma unroll
      for (int rr = 0; rr < RPT; ++rr) {
        const float pq = sphq[u][rg + RG * rr];  // zero for u >= gp
#pragma unroll
        for (int i = 0; i < 4; ++i) yp[u][i] += pq * x[rr][i];
      }
    }
#pragma unroll
    for (int u = 0; u < GM; ++u)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        yp[u][i] = sum_lanes_mod<C4>(yp[u][i]);
    __syncthreads();  // y_win partials complete
    for (int idx = tid; idx < gp * D; idx += 256) {  // y_win = ring part + meta values
      const int u = idx / D, e = idx % D;
      float w = sred[0][u][e] + sred[1][u][e] + sred[2][u][e] + sred[3][u][e];
      for (int m = 0; m < M; ++m) w += slog[u][m] * to_f(stv[m * D + e]);
      sy[u][e] = w;
    }
    __syncthreads();
    if (lane < C4) {
#pragma unroll
      for (int u = 0; u < GM; ++u)
#pragma unroll
        for (int i = 0; i < 4; ++i) sred[wv][u][4 * c4 + i] = yp[u][i];
    }
    __syncthreads();
    for (int idx = tid; idx < gp * D; idx += 256) {
      const int u = idx / D, e = idx % D;
      const float a = sred[0][u][e] + sred[1][u][e] + sred[2][u][e] + sred[3][u][e];
      OUT[((size_t)n * Hq + hk * G + g0 + u) * D + e] = from_f<T>(p.mix * a + (1.f - p.mix) * sy[u][e]);
    }
    __syncthreads();
  }
  if (tid < D) {
    RK[rbase + (size_t)slot * D + tid] = K[nh * D + tid];
    RV[rbase + (size_t)slot * D + tid] = V[nh * D + tid];
  }
  if (tid == 0) {
    // Every wave consumed its read of pos[n] before the last barrier, so a
    // relaxed count is enough (a device-scope fence here would write back and
    // invalidate this XCD's L2 once per workgroup).
    if (__hip_atomic_fetch_add(p.ws_count + n, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == Hkv - 1)
      p.pos[n] = pn + 1;
  }
}

template <typename T, int D>
static hipError_t launch_dec_t(const DecParams &p, hipStream_t stream) {
  const dim3 pgrid((p.N + DEC_ROWS - 1) / DEC_ROWS, p.Hkv + p.Hq);
  if constexpr (sizeof(T) == 2) {
    if (p.hh) hipLaunchKernelGGL((decode_phi_b16_kernel<D, true>), pgrid, dim3(256), 0, stream, p);
    else hipLaunchKernelGGL((decode_phi_b16_kernel<D, false>), pgrid, dim3(256), 0, stream, p);
  } else {
    if (p.hh) hipLaunchKernelGGL((decode_phi_kernel<T, D, true>), pgrid, dim3(256), 0, stream, p);
    else hipLaunchKernelGGL((decode_phi_kernel<T, D, false>), pgrid, dim3(256), 0, stream, p);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (p.G == 1)
    hipLaunchKernelGGL((decode_step_kernel<T, D, 1>), dim3(p.N * p.Hkv), dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL((decode_step_kernel<T, D, DEC_MAXG>), dim3(p.N * p.Hkv), dim3(256), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_decode(const DecParams &p, int dtype_bf16, int d, hipStream_t stream) {
  if (dtype_bf16) {
    if (d == 64) return launch_dec_t<bf16, 64>(p, stream);
    if (d == 128) return launch_dec_t<bf16, 128>(p, stream);
  } else {
    if (d == 64) return launch_dec_t<float, 64>(p, stream);
  }
  return hipErrorInvalidValue;
}

int decode_max_window() { return DEC_MAXW; }

size_t decode_workspace_bytes(int N, int Hq, int Hkv, int d) {
  return ((size_t)N * Hkv * (1 + Hq / Hkv) * d + (size_t)N) * sizeof(float);
}

}  // namespace lz
