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
// The step is bound by HBM traffic on the state (2*d*d*4 bytes per (sequence,
// head), read and written once) and the ring (2*W*d elements read).  One
// workgroup per (sequence, key/value head).  Every independent load is issued
// at the top -- the thread's rows of the state, its 16-byte pieces of the ring
// keys and values -- so the whole step costs about one memory round trip; the
// feature maps (W_phi from L2, one pass for phi_k and all phi_q) run while
// those loads are in flight.  Partial sums are reduced inside each wave with
// shuffles before meeting in LDS.  The position counter is advanced by a
// separate kernel once every head has read it.
#include "common.hpp"
#include "internal.hpp"

namespace lz {

constexpr int DEC_MAXG = 4;   // query heads per key/value head per pass (grouped heads)
constexpr int DEC_MAXW = 256; // ring length limit
constexpr int DEC_MAXM = 16;
constexpr int DEC_RKEYS = 64; // ring keys per logits pass (4 lanes per key)
constexpr float DEC_NEG = -1.0e30f;

template <typename T, int D, int GM>  // GM: query heads per pass (1 or DEC_MAXG)
__global__ __launch_bounds__(256, 2) void decode_kernel(DecParams p) {
  constexpr int C4 = D / 4;     // float4 columns per state row
  constexpr int RG = 256 / C4;  // row groups of the state
  constexpr int RPT = D / RG;   // state rows per thread
  constexpr int F8 = D / 8;     // 8-column pieces of a row
  constexpr int JG = 256 / F8;  // key / row groups for 8-column work
  constexpr int QD = D / 4;     // quarter row (window logits: 4 lanes per key)
  constexpr int NV = GM + 1;
  constexpr int VPT = DEC_RKEYS / JG;  // value pieces per thread loaded up front
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int G = p.G, Hq = p.Hq, Hkv = p.Hkv, W = p.W, M = p.M;
  const int n = blockIdx.x / Hkv, hk = blockIdx.x % Hkv;
  const size_t nh = (size_t)n * Hkv + hk;

  __shared__ float sx[NV][D];        // queries (0..3) and the raw key (4); later y_win per head
  __shared__ float sphi[NV][D];      // phi_q per head, phi_k
  __shared__ float sgam[D], sv[D];
  __shared__ float sred[4][NV][D];   // per-wave partial sums (feature maps, y_win, y_gla)
  __shared__ float slog[GM][DEC_MAXM + DEC_MAXW];

  const T *Q = reinterpret_cast<const T *>(p.q);
  const T *K = reinterpret_cast<const T *>(p.k);
  const T *V = reinterpret_cast<const T *>(p.v);
  const T *LG = reinterpret_cast<const T *>(p.lg);
  const T *Wq = reinterpret_cast<const T *>(p.wq);
  const T *Wk = reinterpret_cast<const T *>(p.wk) + (size_t)hk * p.w_stride;
  const T *Tk = reinterpret_cast<const T *>(p.tk);
  const T *Tv = reinterpret_cast<const T *>(p.tv);
  T *RK = reinterpret_cast<T *>(p.win_k);
  T *RV = reinterpret_cast<T *>(p.win_v);
  T *OUT = reinterpret_cast<T *>(p.out);
  const bool shared_w = (p.wq == p.wk) && p.w_stride == 0;

  const int pn = p.pos[n];
  const int slot = pn % W;
  const int nvalid = min(pn + 1, W);
  const size_t rbase = nh * (size_t)W * D;
  float *St = p.state + nh * D * D;
  const int c4 = tid % C4, rg = tid / C4;

  // ---- loads in flight from here on: state rows, ring key quarter, ring value pieces
  f32x4 x[RPT];
#pragma unroll
  for (int rr = 0; rr < RPT; ++rr)
    x[rr] = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(St + (size_t)(rg + RG * rr) * D + 4 * c4));
  const int kq = tid / 4, kpart = tid % 4;  // ring slot kq (+ multiples of 64), dims kpart*QD ..
  Frag<T> kfr[QD / 8];
#pragma unroll
  for (int e8 = 0; e8 < QD / 8; ++e8)
    kfr[e8] = (kq < W) ? load8(RK + rbase + (size_t)kq * D + kpart * QD + 8 * e8) : frag_zero<T>();
  const int f8 = tid % F8, jg = tid / F8;   // value columns 8*f8 .., ring slots jg, jg+JG, ...
  Frag<T> vfr[VPT];
#pragma unroll
  for (int m = 0; m < VPT; ++m) {
    const int j = jg + JG * m;
    vfr[m] = (j < W) ? load8(RV + rbase + (size_t)j * D + 8 * f8) : frag_zero<T>();
  }

  for (int e = tid; e < D; e += 256) {
    const size_t o = nh * D + e;
    sx[GM][e] = to_f(K[o]);
    sgam[e] = __expf(to_f(LG[o]));
    sv[e] = to_f(V[o]);
  }

  for (int g0 = 0; g0 < G; g0 += GM) {
    const int gp = min(GM, G - g0);
    const bool first = (g0 == 0);
    for (int idx = tid; idx < GM * D; idx += 256) {
      const int u = idx / D, e = idx % D;
      sx[u][e] = (u < gp) ? to_f(Q[((size_t)n * Hq + hk * G + g0 + u) * D + e]) : 0.f;
    }
    __syncthreads();

    // ---- feature maps: z[v][f] = sum_i x_v[i] W[i][f]; thread (f8, jg) sums rows jg, jg+JG, ...
    {
      float z[NV][8];
#pragma unroll
      for (int v = 0; v < NV; ++v)
#pragma unroll
        for (int j = 0; j < 8; ++j) z[v][j] = 0.f;
#pragma unroll 2
      for (int i = jg; i < D; i += JG) {
        float wk8[8];
        if (first) {
          load8f(Wk + (size_t)i * D + 8 * f8, wk8);
          const float xi = sx[GM][i];
#pragma unroll
          for (int j = 0; j < 8; ++j) z[GM][j] += xi * wk8[j];
        }
#pragma unroll
        for (int u = 0; u < GM; ++u) {
          if (u < gp) {
            float w8[8];
            if (shared_w && first) {
#pragma unroll
              for (int j = 0; j < 8; ++j) w8[j] = wk8[j];
            } else {
              load8f(Wq + (size_t)(hk * G + g0 + u) * p.w_stride + (size_t)i * D + 8 * f8, w8);
            }
            const float xi = sx[u][i];
#pragma unroll
            for (int j = 0; j < 8; ++j) z[u][j] += xi * w8[j];
          }
        }
      }
      // the 64/F8 row groups of a wave, then the 4 waves in LDS
#pragma unroll
      for (int v = 0; v < NV; ++v)
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
          for (int o = F8; o < 64; o <<= 1) z[v][j] += __shfl_xor(z[v][j], o);
      if (lane < F8) {
#pragma unroll
        for (int v = 0; v < NV; ++v)
#pragma unroll
          for (int j = 0; j < 8; ++j) sred[wv][v][8 * f8 + j] = z[v][j];
      }
      __syncthreads();
      // softmax over features: wave w handles vectors w, w+4
      for (int v = wv; v < NV; v += 4) {
        if (v == GM ? !first : v >= gp) continue;
        float zz[D / 64];
        float m = DEC_NEG;
#pragma unroll
        for (int q = 0; q < D / 64; ++q) {
          const int f = lane + 64 * q;
          zz[q] = sred[0][v][f] + sred[1][v][f] + sred[2][v][f] + sred[3][v][f];
          m = fmaxf(m, zz[q]);
        }
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) m = fmaxf(m, __shfl_xor(m, o));
        float s = 0.f;
#pragma unroll
        for (int q = 0; q < D / 64; ++q) {
          zz[q] = __expf(zz[q] - m);
          s += zz[q];
        }
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) s += __shfl_xor(s, o);
        const float inv = 1.f / s;
#pragma unroll
        for (int q = 0; q < D / 64; ++q) sphi[v][lane + 64 * q] = zz[q] * inv;
      }
    }

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
            for (int t = 0; t < 8; ++t) kv8[t] = sx[GM][e0 + t];
          } else if (jb == 0) {
#pragma unroll
            for (int t = 0; t < 8; ++t) kv8[t] = to_f(kfr[e8].v[t]);
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
        acc[u] += __shfl_xor(acc[u], 1);
        acc[u] += __shfl_xor(acc[u], 2);
      }
      if (in && kpart == 0)
        for (int u = 0; u < gp; ++u) slog[u][M + jj] = ok ? acc[u] * p.scale : DEC_NEG;
    }
    // meta keys: thread (u, m), full dot product (T_k from L2)
    for (int idx = tid; idx < gp * M; idx += 256) {
      const int u = idx / M, m = idx % M;
      const T *kr = Tk + ((size_t)hk * M + m) * D;
      float a = 0.f;
      for (int e8 = 0; e8 < D; e8 += 8) {
        float kv8[8];
        load8f(kr + e8, kv8);
#pragma unroll
        for (int t = 0; t < 8; ++t) a += sx[u][e8 + t] * kv8[t];
      }
      slog[u][m] = a * p.scale;
    }
    __syncthreads();
    // softmax per head (one wave per head)
    for (int u = wv; u < gp; u += 4) {
      float m = DEC_NEG;
      for (int j = lane; j < M + W; j += 64) m = fmaxf(m, slog[u][j]);
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) m = fmaxf(m, __shfl_xor(m, o));
      float sum = 0.f;
      for (int j = lane; j < M + W; j += 64) {
        const float ex = __expf(slog[u][j] - m);  // masked entries: exp(-1e30) = 0
        slog[u][j] = ex;
        sum += ex;
      }
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) sum += __shfl_xor(sum, o);
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
#pragma unroll
          for (int t = 0; t < 8; ++t) vv[t] = (j == slot) ? sv[8 * f8 + t] : to_f(vfr[m].v[t]);
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
#pragma unroll
          for (int o = F8; o < 64; o <<= 1) acc[u][t] += __shfl_xor(acc[u][t], o);
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
        const float gm = sgam[f], pk = sphi[GM][f];
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
      if (u < gp) {
#pragma unroll
        for (int rr = 0; rr < RPT; ++rr) {
          const float pq = sphi[u][rg + RG * rr];
#pragma unroll
          for (int i = 0; i < 4; ++i) yp[u][i] += pq * x[rr][i];
        }
      }
    }
#pragma unroll
    for (int u = 0; u < GM; ++u)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int o = C4; o < 64; o <<= 1) yp[u][i] += __shfl_xor(yp[u][i], o);
    __syncthreads();  // y_win partials complete
    // y_win per head (ring part + meta values) -> sx (the raw queries are no longer needed)
    for (int idx = tid; idx < gp * D; idx += 256) {
      const int u = idx / D, e = idx % D;
      float w = sred[0][u][e] + sred[1][u][e] + sred[2][u][e] + sred[3][u][e];
      for (int m = 0; m < M; ++m) w += slog[u][m] * to_f(Tv[((size_t)hk * M + m) * D + e]);
      sx[u][e] = w;
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
      OUT[((size_t)n * Hq + hk * G + g0 + u) * D + e] = from_f<T>(p.mix * a + (1.f - p.mix) * sx[u][e]);
    }
    __syncthreads();
  }
  if (tid < D) {
    RK[rbase + (size_t)slot * D + tid] = K[nh * D + tid];
    RV[rbase + (size_t)slot * D + tid] = V[nh * D + tid];
  }
}

__global__ void decode_advance_pos(int32_t *pos, int N) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < N) pos[i] += 1;
}

template <typename T, int D>
static hipError_t launch_dec_t(const DecParams &p, hipStream_t stream) {
  if (p.G == 1)
    hipLaunchKernelGGL((decode_kernel<T, D, 1>), dim3(p.N * p.Hkv), dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL((decode_kernel<T, D, DEC_MAXG>), dim3(p.N * p.Hkv), dim3(256), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_advance_pos, dim3((p.N + 255) / 256), dim3(256), 0, stream, p.pos, p.N);
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

}  // namespace lz
