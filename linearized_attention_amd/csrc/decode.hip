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
// head), read and written once).  Each thread streams its rows of float4
// columns with all loads issued before any use.  Workgroup: 256 threads for
// DEC_NS sequences of one key/value head, so the feature-map weights are read
// once per DEC_NS sequences.  The position counter is advanced by a separate
// kernel once every head has read it.
#include "common.hpp"
#include "internal.hpp"

namespace lz {

constexpr int DEC_NS = 4;     // sequences per workgroup
constexpr int DEC_MAXG = 4;   // query heads per key/value head per pass
constexpr int DEC_MAXW = 256; // ring length limit (logit buffer)
constexpr int DEC_MAXM = 16;
constexpr float DEC_NEG = -1.0e30f;

template <typename T, int D>
__global__ __launch_bounds__(256) void decode_kernel(DecParams p) {
  constexpr int C4 = D / 4;     // float4 columns per state row
  constexpr int RG = 256 / C4;  // row groups
  constexpr int RPT = D / RG;   // rows per thread
  constexpr int NPART = 256 / D;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int G = p.G, Hq = p.Hq, Hkv = p.Hkv, W = p.W, M = p.M;
  const int nblk = (p.N + DEC_NS - 1) / DEC_NS;
  const int hk = blockIdx.x / nblk;
  const int n0 = (blockIdx.x % nblk) * DEC_NS;
  const int ns = min(DEC_NS, p.N - n0);

  __shared__ float sq[DEC_NS][DEC_MAXG][D];    // raw queries
  __shared__ float sphq[DEC_NS][DEC_MAXG][D];  // phi_q
  __shared__ float skr[DEC_NS][D];             // raw key
  __shared__ float sphk[DEC_NS][D];            // phi_k
  __shared__ float sgam[DEC_NS][D];
  __shared__ float sv[DEC_NS][D];
  __shared__ float sy[RG][DEC_MAXG][D];        // partial y_gla per row group
  __shared__ float sygla[DEC_MAXG][D];
  __shared__ float slog[DEC_MAXG][DEC_MAXM + DEC_MAXW];
  __shared__ float sred[NPART][DEC_MAXG][D];
  __shared__ int spos[DEC_NS];

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

  if (tid < DEC_NS) spos[tid] = (tid < ns) ? p.pos[n0 + tid] : 0;
  for (int idx = tid; idx < DEC_NS * D; idx += 256) {
    const int s = idx / D, e = idx % D;
    float kk = 0.f, gm = 1.f, vv = 0.f;
    if (s < ns) {
      const size_t o = ((size_t)(n0 + s) * Hkv + hk) * D + e;
      kk = to_f(K[o]);
      gm = __expf(to_f(LG[o]));
      vv = to_f(V[o]);
    }
    skr[s][e] = kk;
    sgam[s][e] = gm;
    sv[s][e] = vv;
  }

  for (int g0 = 0; g0 < G; g0 += DEC_MAXG) {
    const int gp = min(DEC_MAXG, G - g0);
    const bool first = (g0 == 0);
    for (int idx = tid; idx < DEC_NS * DEC_MAXG * D; idx += 256) {
      const int s = idx / (DEC_MAXG * D), u = (idx / D) % DEC_MAXG, e = idx % D;
      float x = 0.f;
      if (s < ns && u < gp) x = to_f(Q[((size_t)(n0 + s) * Hq + hk * G + g0 + u) * D + e]);
      sq[s][u][e] = x;
    }
    __syncthreads();
    // ---- feature maps z = x W; job 0 = key side (first pass), job 1 + u = query head u
    {
      const int f = tid % D, part = tid / D;
      for (int job = part; job < 1 + gp; job += NPART) {
        if (job == 0 && !first) continue;
        float z[DEC_NS];
#pragma unroll
        for (int s = 0; s < DEC_NS; ++s) z[s] = 0.f;
        if (job == 0) {
          for (int i = 0; i < D; ++i) {
            const float w = to_f(Wk[(size_t)i * D + f]);
#pragma unroll
            for (int s = 0; s < DEC_NS; ++s) z[s] += skr[s][i] * w;
          }
#pragma unroll
          for (int s = 0; s < DEC_NS; ++s) sphk[s][f] = z[s];
        } else {
          const int u = job - 1;
          const T *Wm = Wq + (size_t)(hk * G + g0 + u) * p.w_stride;
          for (int i = 0; i < D; ++i) {
            const float w = to_f(Wm[(size_t)i * D + f]);
#pragma unroll
            for (int s = 0; s < DEC_NS; ++s) z[s] += sq[s][u][i] * w;
          }
#pragma unroll
          for (int s = 0; s < DEC_NS; ++s) sphq[s][u][f] = z[s];
        }
      }
    }
    __syncthreads();
    // softmax over features, one wave per vector
    for (int vec = wv; vec < DEC_NS * (1 + DEC_MAXG); vec += 4) {
      const int s = vec / (1 + DEC_MAXG), u = vec % (1 + DEC_MAXG);
      if (u == 0 ? !first : (u - 1) >= gp) continue;
      float *row = (u == 0) ? sphk[s] : sphq[s][u - 1];
      float m = DEC_NEG;
      for (int e = lane; e < D; e += 64) m = fmaxf(m, row[e]);
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) m = fmaxf(m, __shfl_xor(m, o));
      float sum = 0.f;
      for (int e = lane; e < D; e += 64) sum += __expf(row[e] - m);
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) sum += __shfl_xor(sum, o);
      const float inv = 1.f / sum;
      for (int e = lane; e < D; e += 64) row[e] = __expf(row[e] - m) * inv;
    }
    __syncthreads();

    for (int s = 0; s < ns; ++s) {
      const int n = n0 + s;
      const int pn = spos[s];
      const int slot = pn % W;
      const size_t nh = (size_t)n * Hkv + hk;
      const size_t rbase = nh * (size_t)W * D;
      // ---- state stream: S = diag(gamma) S + phi_k v^T (first pass), partial y = phi_q^T S
      {
        float *St = p.state + nh * D * D;
        const int c4 = tid % C4, rg = tid / C4;
        f32x4 x[RPT];
#pragma unroll
        for (int rr = 0; rr < RPT; ++rr)
          x[rr] = *reinterpret_cast<const f32x4 *>(St + (size_t)(rg + RG * rr) * D + 4 * c4);
        if (first) {
          const float v0 = sv[s][4 * c4], v1 = sv[s][4 * c4 + 1], v2 = sv[s][4 * c4 + 2], v3 = sv[s][4 * c4 + 3];
#pragma unroll
          for (int rr = 0; rr < RPT; ++rr) {
            const int f = rg + RG * rr;
            const float gm = sgam[s][f], pk = sphk[s][f];
            x[rr][0] = gm * x[rr][0] + pk * v0;
            x[rr][1] = gm * x[rr][1] + pk * v1;
            x[rr][2] = gm * x[rr][2] + pk * v2;
            x[rr][3] = gm * x[rr][3] + pk * v3;
            *reinterpret_cast<f32x4 *>(St + (size_t)f * D + 4 * c4) = x[rr];
          }
        }
        for (int u = 0; u < gp; ++u) {
          float y0 = 0.f, y1 = 0.f, y2 = 0.f, y3 = 0.f;
#pragma unroll
          for (int rr = 0; rr < RPT; ++rr) {
            const float pq = sphq[s][u][rg + RG * rr];
            y0 += pq * x[rr][0];
            y1 += pq * x[rr][1];
            y2 += pq * x[rr][2];
            y3 += pq * x[rr][3];
          }
          sy[rg][u][4 * c4] = y0;
          sy[rg][u][4 * c4 + 1] = y1;
          sy[rg][u][4 * c4 + 2] = y2;
          sy[rg][u][4 * c4 + 3] = y3;
        }
      }
      // ---- window logits: 4 lanes per key, each a quarter of d; keys 0..M-1 meta, then ring slots
      for (int jb = 0; jb < M + W; jb += 64) {
        const int j = jb + tid / 4, part = tid % 4;
        const bool in = j < M + W;
        bool ok = false;
        const T *kr = nullptr;
        const float *kl = nullptr;
        if (in) {
          if (j < M) {
            ok = true;
            kr = Tk + ((size_t)hk * M + j) * D;
          } else {
            const int jj = j - M;
            const int age = ((slot - jj) % W + W) % W;  // pn - (token in slot jj)
            ok = age <= pn;
            if (jj == slot) kl = skr[s];
            else kr = RK + rbase + (size_t)jj * D;
          }
        }
        float acc[DEC_MAXG];
#pragma unroll
        for (int u = 0; u < DEC_MAXG; ++u) acc[u] = 0.f;
        if (ok) {
          constexpr int QD = D / 4;
#pragma unroll
          for (int e8 = 0; e8 < QD; e8 += 8) {
            float kv8[8];
            const int e0 = part * QD + e8;
            if (kl) {
#pragma unroll
              for (int t = 0; t < 8; ++t) kv8[t] = kl[e0 + t];
            } else {
              load8f(kr + e0, kv8);
            }
#pragma unroll
            for (int u = 0; u < DEC_MAXG; ++u)
#pragma unroll
              for (int t = 0; t < 8; ++t) acc[u] += sq[s][u][e0 + t] * kv8[t];
          }
        }
#pragma unroll
        for (int u = 0; u < DEC_MAXG; ++u) {
          acc[u] += __shfl_xor(acc[u], 1);
          acc[u] += __shfl_xor(acc[u], 2);
        }
        if (in && part == 0)
          for (int u = 0; u < gp; ++u) slog[u][j] = ok ? acc[u] * p.scale : DEC_NEG;
      }
      __syncthreads();
      // reduce partial y_gla; softmax per head (one wave per head)
      for (int idx = tid; idx < gp * D; idx += 256) {
        const int u = idx / D, e = idx % D;
        float a = 0.f;
#pragma unroll
        for (int r = 0; r < RG; ++r) a += sy[r][u][e];
        sygla[u][e] = a;
      }
      for (int u = wv; u < gp; u += 4) {
        float m = DEC_NEG;
        for (int j = lane; j < M + W; j += 64) m = fmaxf(m, slog[u][j]);
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) m = fmaxf(m, __shfl_xor(m, o));
        float sum = 0.f;
        for (int j = lane; j < M + W; j += 64) {
          const float l = slog[u][j];
          const float ex = (l > 0.5f * DEC_NEG) ? __expf(l - m) : 0.f;
          slog[u][j] = ex;
          sum += ex;
        }
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) sum += __shfl_xor(sum, o);
        const float inv = 1.f / sum;
        for (int j = lane; j < M + W; j += 64) slog[u][j] *= inv;
      }
      __syncthreads();
      // ---- y_win = P [T_v ; ring V]: thread (e, part) sums keys j = part (mod NPART)
      {
        const int e = tid % D, part = tid / D;
        float acc[DEC_MAXG];
#pragma unroll
        for (int u = 0; u < DEC_MAXG; ++u) acc[u] = 0.f;
        for (int j = part; j < M + W; j += NPART) {
          float vv;
          if (j < M) vv = to_f(Tv[((size_t)hk * M + j) * D + e]);
          else if (j - M == slot) vv = sv[s][e];
          else vv = to_f(RV[rbase + (size_t)(j - M) * D + e]);
#pragma unroll
          for (int u = 0; u < DEC_MAXG; ++u) acc[u] += slog[u][j] * vv;
        }
        for (int u = 0; u < gp; ++u) sred[part][u][e] = acc[u];
      }
      __syncthreads();
      for (int idx = tid; idx < gp * D; idx += 256) {
        const int u = idx / D, e = idx % D;
        float a = 0.f;
#pragma unroll
        for (int pp = 0; pp < NPART; ++pp) a += sred[pp][u][e];
        const float y = p.mix * sygla[u][e] + (1.f - p.mix) * a;
        OUT[((size_t)n * Hq + hk * G + g0 + u) * D + e] = from_f<T>(y);
      }
      if (first && tid < D) {
        RK[rbase + (size_t)slot * D + tid] = from_f<T>(skr[s][tid]);
        RV[rbase + (size_t)slot * D + tid] = from_f<T>(sv[s][tid]);
      }
      __syncthreads();
    }
  }
}

__global__ void decode_advance_pos(int32_t *pos, int N) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < N) pos[i] += 1;
}

template <typename T, int D>
static hipError_t launch_dec_t(const DecParams &p, hipStream_t stream) {
  const int nblk = (p.N + DEC_NS - 1) / DEC_NS;
  hipLaunchKernelGGL((decode_kernel<T, D>), dim3(nblk * p.Hkv), dim3(256), 0, stream, p);
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
