// Gated-linear-attention forward alone (the global branch of Lizard attention, no window), in two
// forms of the intra-chunk product, for measuring the reparameterization the Lizard paper
// proposes against the standard chunked algorithm on the same hardware (arXiv page, Method:
// the standard parallel form needs its per-element decays in fp32, which keeps it off the
// matrix cores; Efficiency paragraph: the reparameterized kernel's forward is reported 32-36%
// faster than the standard one).
//
//   y_t = sum_{s <= t} sum_f phi_q[t][f] phi_k[s][f] e^{b_t[f] - b_s[f]} v_s,
//   b the cumulative log gate (papernotes.org summary, "key designs", Gated Linear Attention).
//
// Both forms run the same chunk loop: one workgroup of 4 waves per (batch, query head), 64-token
// chunks, wave I owning query rows 16 I .. 16 I + 15 of the chunk and rows 32 I .. 32 I + 31 of
// the d x d state; the inter-chunk product and the state update are identical.  They differ in
// the intra-chunk scores A[t][s] for s <= t in the chunk:
//   MODE 0, standard ("secondary chunking"): 16-token sub-chunks; a block of key sub-chunk J below
//     the query sub-chunk I uses sub-chunk references (queries e^{p_t - C_J}, keys e^{C_J - p_s},
//     both <= 1) on MFMA; the diagonal blocks are formed element by element in fp32 on the VALU,
//     one exponential per (t, s, f).
//   MODE 1, absorbed: every decay refers to the chunk start (queries e^{p_t} <= 1, keys e^{-p_s}),
//     so the whole masked 64 x 64 product ((Q~ K~^T) (.) M) V runs on MFMA; a chunk whose log decay
//     exceeds 60 in some feature (e^{-p_s} would overflow the operand range) takes MODE 0's
//     arithmetic instead.
// p_t is the log-gate prefix from the chunk start through t, C_J its value at the end of
// sub-chunk J, P the chunk total.  bf16 operands, fp32 accumulation, the softmax feature map over
// d features with one W_phi for queries, keys and heads, d = 128.
#include "fwd_common.hpp"

namespace lz {
namespace gla {

constexpr int D = 128, NFT = 8, KS = 4;
constexpr int LDW = 136;  // rows of 128 bf16 + 16 bytes
constexpr int LDV = 72;   // rows of 64 tokens + 16 bytes
constexpr int LDP = 132;  // fp32 rows of 128 features + 16 bytes

// LDS regions of a workgroup that owns DVB value columns.
template <int DVB> struct Geo {
  static constexpr int OFF_W = 0;                              // W_phi^T [f][d]
  static constexpr int OFF_VT = OFF_W + D * LDW * 2;           // v^T [dv][s]
  static constexpr int OFF_LGT = OFF_VT + DVB * LDV * 2;       // log gamma^T [f][s]; then keys~ [s][f]
  static constexpr int SZ_LGT = (D * LDV > CH * LDW ? D * LDV : CH * LDW) * 2;
  static constexpr int OFF_S = OFF_LGT + SZ_LGT;               // S^T copy [dv][f]
  static constexpr int OFF_PK = OFF_S + DVB * LDW * 2;         // phi_k [s][f] (diagonal blocks)
  static constexpr int OFF_P = OFF_PK + CH * LDW * 2;          // p [s][f] fp32 (diagonal blocks)
  static constexpr int OFF_TAB = OFF_P + CH * LDP * 4;         // C_J [4][f] fp32
  static constexpr int BYTES = OFF_TAB + 4 * D * 4;
  static_assert(BYTES <= LDS_LIMIT, "GLA layout exceeds LDS");
};

// Rows r0 .. r0+3 of column c0 + (lane % 16) of a row-major bf16 LDS tile (transposed read;
// each 16-lane row of the wave takes its own r0).
__device__ __forceinline__ bf16x4 col4(const bf16 *tile, int ld, int r0, int c0) {
  typedef short s4 __attribute__((ext_vector_type(4)));
  const int m = threadIdx.x & 15;
  const bf16 *src = tile + (r0 + (m >> 2)) * ld + c0 + 4 * (m & 3);
  const s4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s4 *)(src));
  return __builtin_bit_cast(bf16x4, x);
}

// Operand of K-step js from per-row fp32 values in accumulator order (lane (r, kq) holds
// f = 16 ft + 4 kq + i): slot j carries feature 32 js + 16 (j >> 2) + 4 kq + (j & 3), the order in
// which the keys' LDS rows are read (two 8-byte pieces 16 features apart).
__device__ __forceinline__ Frag<bf16> il_frag(const float (&x)[NFT][4], int js) {
  float y[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) y[j] = x[2 * js + (j >> 2)][j & 3];
  return frag_from<bf16>(y);
}

}  // namespace gla

// One workgroup per (batch, query head, block of DVB value columns); when there are two blocks,
// blocks 8 apart in launch order (the same XCD) take the two halves of one head, so the second
// reads q, k and log gamma from that XCD's L2.
template <int MODE, int DVB>
__global__ __launch_bounds__(256, 1) void gla_fwd_kernel(GlaParams p) {
  using namespace gla;
  using T = bf16;
  using G = Geo<DVB>;
  constexpr int NDT = DVB / 16, NVF = DVB / 32;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  T *sW = reinterpret_cast<T *>(smem + G::OFF_W);
  T *sVt = reinterpret_cast<T *>(smem + G::OFF_VT);
  T *sLgT = reinterpret_cast<T *>(smem + G::OFF_LGT);
  T *sKt = sLgT;  // decayed keys [s][f], written once the prefix sums have read log gamma^T
  T *sS = reinterpret_cast<T *>(smem + G::OFF_S);
  T *sPk = reinterpret_cast<T *>(smem + G::OFF_PK);
  float *sP = reinterpret_cast<float *>(smem + G::OFF_P);
  float *sTab = reinterpret_cast<float *>(smem + G::OFF_TAB);
  const int tid = threadIdx.x, lane = tid & 63, r = lane & 15, kq = lane >> 4;
  const int I = __builtin_amdgcn_readfirstlane(tid >> 6);
  int bh = blockIdx.x, dv0 = 0;
  if constexpr (DVB < D) {
    bh = (blockIdx.x >> 4) * 8 + (blockIdx.x & 7);
    dv0 = ((blockIdx.x >> 3) & 1) * DVB;
  }
  if (bh >= p.B * p.Hq) return;  // padding of the launch to whole XCD pairs
  const int b = bh / p.Hq, hq = bh % p.Hq, hk = hq / (p.Hq / p.Hkv);
  const int L = p.L;
  const size_t kvo = ((size_t)b * p.Hkv + hk) * L * D, qo = (size_t)bh * L * D;
  const T *Q = reinterpret_cast<const T *>(p.q) + qo;
  const T *K = reinterpret_cast<const T *>(p.k) + kvo;
  const T *V = reinterpret_cast<const T *>(p.v) + kvo + dv0;
  const T *LG = reinterpret_cast<const T *>(p.lg) + kvo;
  T *O = reinterpret_cast<T *>(p.out) + qo + dv0;

  load_wT<T, D, LDW>(sW, reinterpret_cast<const T *>(p.w), tid);
  f32x4 S[2][NDT];  // S[f = 32 I + 16 ft + 4 kq + i][dv = 16 dt + r]
#pragma unroll
  for (int ft = 0; ft < 2; ++ft)
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) S[ft][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int idx = tid; idx < DVB * LDW; idx += 256) sS[idx] = from_f<T>(0.f);
  const Frag<T> tri_c0 = tri64_frag<T>(r, kq, I, 0), tri_c1 = tri64_frag<T>(r, kq, I, 1);

  // this wave's 16 rows of a chunk in fragment order (lane (t = r, kq): columns 32 j + 8 kq ..)
  auto load_rows = [&](const T *X, auto &f, int c0) {
    constexpr int nf = sizeof(f) / sizeof(f[0]);
    const int t = c0 + 16 * I + r;
#pragma unroll
    for (int j = 0; j < nf; ++j) f[j] = (t < L) ? load8(X + (size_t)t * D + 32 * j + 8 * kq) : frag_zero<T>();
  };
  Frag<T> qf[KS], kf[KS], vfr[NVF], lfr[KS];
  load_rows(Q, qf, 0);
  load_rows(K, kf, 0);
  load_rows(V, vfr, 0);
  load_rows(LG, lfr, 0);
  __syncthreads();

  for (int c0 = 0; c0 < L; c0 += CH) {
    // ---- stage v^T and log gamma^T of the chunk (the wave's 16 rows, transposed)
    {
      const int s = 16 * I + r;
#pragma unroll
      for (int j = 0; j < NVF; ++j)
#pragma unroll
        for (int e = 0; e < 8; ++e) sVt[(32 * j + 8 * kq + e) * LDV + s] = vfr[j].v[e];
#pragma unroll
      for (int j = 0; j < KS; ++j)
#pragma unroll
        for (int e = 0; e < 8; ++e) sLgT[(32 * j + 8 * kq + e) * LDV + s] = lfr[j].v[e];
    }
    Frag<T> qc[KS], kc[KS];
#pragma unroll
    for (int j = 0; j < KS; ++j) {
      qc[j] = qf[j];
      kc[j] = kf[j];
    }
    if (c0 + CH < L) {  // the next chunk's rows in flight during this one
      load_rows(Q, qf, c0 + CH);
      load_rows(K, kf, c0 + CH);
      load_rows(V, vfr, c0 + CH);
      load_rows(LG, lfr, c0 + CH);
    }
    __syncthreads();  // B1: v^T and log gamma^T staged
    // ---- prefix sums p_t of the wave's rows (lane (t = r, kq): f = 16 ft + 4 kq + i); C_I
    float pc[NFT][4];
#pragma unroll
    for (int ft = 0; ft < NFT; ++ft) {
      f32x4 cc = mma(load8(sLgT + (16 * ft + r) * LDV + 8 * kq), tri_c0, f32x4{0.f, 0.f, 0.f, 0.f});
      cc = mma(load8(sLgT + (16 * ft + r) * LDV + 32 + 8 * kq), tri_c1, cc);
#pragma unroll
      for (int i = 0; i < 4; ++i) pc[ft][i] = cc[i];
    }
    if (r == 15) {
#pragma unroll
      for (int ft = 0; ft < NFT; ++ft)
        *reinterpret_cast<f32x4 *>(sTab + I * D + 16 * ft + 4 * kq) =
            f32x4{pc[ft][0], pc[ft][1], pc[ft][2], pc[ft][3]};
    }
    // ---- feature maps of the wave's rows
    float phq[NFT][4], phk[NFT][4];
    {
      f32x4 z[NFT];
      feature_logits<T, D, LDW>(sW, qc, r, kq, z);
      softmax_rows<NFT>(z, phq);
      feature_logits<T, D, LDW>(sW, kc, r, kq, z);
      softmax_rows<NFT>(z, phk);
    }
    __syncthreads();  // B2: sub-chunk ends visible; log gamma^T read
    const bool absorbed = (MODE == 1) && chunk_is_mild_c<D>(sTab, lane);
    // ---- keys~ of the wave's rows -> sKt (absorbed: e^{-p_s}; standard: e^{C_I - p_s} <= 1),
    //      and the diagonal-block tables
#pragma unroll
    for (int ft = 0; ft < NFT; ++ft) {
      const f32x4 cI = *reinterpret_cast<const f32x4 *>(sTab + I * D + 16 * ft + 4 * kq);
      float kt[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) kt[i] = phk[ft][i] * __expf(absorbed ? -pc[ft][i] : cI[i] - pc[ft][i]);
      store4<T>(sKt + (16 * I + r) * LDW + 16 * ft + 4 * kq, kt[0], kt[1], kt[2], kt[3]);
      if (!absorbed) {
        store4<T>(sPk + (16 * I + r) * LDW + 16 * ft + 4 * kq, phk[ft][0], phk[ft][1], phk[ft][2], phk[ft][3]);
        *reinterpret_cast<f32x4 *>(sP + (16 * I + r) * LDP + 16 * ft + 4 * kq) =
            f32x4{pc[ft][0], pc[ft][1], pc[ft][2], pc[ft][3]};
      }
    }
    __syncthreads();  // B3: keys~ and tables visible
    // ---- queries~: absorbed phi_q e^{p_t}; standard phi_q e^{p_t - C_{I-1}} (C_{-1} = 0); both <= 1
    float qx[NFT][4];
#pragma unroll
    for (int ft = 0; ft < NFT; ++ft) {
      f32x4 ref = {0.f, 0.f, 0.f, 0.f};
      if (!absorbed && I > 0) ref = *reinterpret_cast<const f32x4 *>(sTab + (I - 1) * D + 16 * ft + 4 * kq);
#pragma unroll
      for (int i = 0; i < 4; ++i) qx[ft][i] = phq[ft][i] * __expf(pc[ft][i] - ref[i]);
    }
    // scores A^T[s][t] of key sub-chunk J against the wave's queries (lane (t = r, kq) gets
    // s = 16 J + 4 kq + i), queries scaled per feature by fac
    auto scores = [&](int J, const float (&fac)[NFT][4]) {
      f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int js = 0; js < KS; ++js) {
        float y[NFT][4];
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int i = 0; i < 4; ++i) y[2 * js + u][i] = qx[2 * js + u][i] * fac[2 * js + u][i];
        const T *kr = sKt + (16 * J + r) * LDW + 32 * js + 4 * kq;
        a = mma(load4x2(kr, kr + 16), il_frag(y, js), a);
      }
      return a;
    };
    f32x4 sc[4];
#pragma unroll
    for (int J = 0; J < 4; ++J) sc[J] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (absorbed) {
      float one[NFT][4];
#pragma unroll
      for (int ft = 0; ft < NFT; ++ft)
#pragma unroll
        for (int i = 0; i < 4; ++i) one[ft][i] = 1.f;
#pragma unroll
      for (int J = 0; J < 4; ++J)
        if (J <= I) sc[J] = scores(J, one);
    } else {
      // blocks J < I: a further query factor e^{C_{I-1} - C_J} <= 1
#pragma unroll
      for (int J = 0; J < 3; ++J) {
        if (J < I) {
          float fac[NFT][4];
#pragma unroll
          for (int ft = 0; ft < NFT; ++ft) {
            const f32x4 a = *reinterpret_cast<const f32x4 *>(sTab + (I - 1) * D + 16 * ft + 4 * kq);
            const f32x4 c = *reinterpret_cast<const f32x4 *>(sTab + J * D + 16 * ft + 4 * kq);
#pragma unroll
            for (int i = 0; i < 4; ++i) fac[ft][i] = __expf(a[i] - c[i]);
          }
          sc[J] = scores(J, fac);
        }
      }
      // diagonal block element by element in fp32: A[t][s] = sum_f phi_q phi_k e^{p_t - p_s}
      float part[16];
#pragma unroll
      for (int s = 0; s < 16; ++s) {
        const int sr = 16 * I + s;
        float acc = 0.f;
        if (s <= r) {
#pragma unroll
          for (int ft = 0; ft < NFT; ++ft) {
            float pk[4];
            load4f(sPk + sr * LDW + 16 * ft + 4 * kq, pk);
            const f32x4 ps = *reinterpret_cast<const f32x4 *>(sP + sr * LDP + 16 * ft + 4 * kq);
#pragma unroll
            for (int i = 0; i < 4; ++i) acc += phq[ft][i] * pk[i] * __expf(pc[ft][i] - ps[i]);
          }
        }
        part[s] = wave_sum_cols(acc);
      }
      f32x4 dg;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float v = 0.f;
#pragma unroll
        for (int s = 0; s < 16; ++s) v = (s == 4 * kq + i) ? part[s] : v;
        dg[i] = v;
      }
#pragma unroll
      for (int J = 0; J < 4; ++J)
        if (J == I) sc[J] = dg;
    }
    // causal mask of the diagonal block
#pragma unroll
    for (int J = 0; J < 4; ++J)
      if (J == I) {
#pragma unroll
        for (int i = 0; i < 4; ++i) sc[J][i] = (4 * kq + i <= r) ? sc[J][i] : 0.f;
      }
    // ---- Y^T = V^T A^T over key sub-chunk pairs (K-step m: tokens 32 m + 16 (j >> 2) + 4 kq + (j & 3))
    f32x4 acc[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      if (2 * m <= I) {
        float x[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          x[i] = sc[2 * m][i];
          x[4 + i] = sc[2 * m + 1][i];
        }
        const Frag<T> af = frag_from<T>(x);
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          const T *vr = sVt + (16 * dt + r) * LDV + 32 * m + 4 * kq;
          acc[dt] = mma(load4x2(vr, vr + 16), af, acc[dt]);
        }
      }
    }
    // ---- inter: Y^T += S^T (phi_q e^{p_t})^T, S the state at the chunk start
    {
      float qi[NFT][4];
#pragma unroll
      for (int ft = 0; ft < NFT; ++ft) {
        f32x4 ref = {0.f, 0.f, 0.f, 0.f};
        if (!absorbed && I > 0) ref = *reinterpret_cast<const f32x4 *>(sTab + (I - 1) * D + 16 * ft + 4 * kq);
#pragma unroll
        for (int i = 0; i < 4; ++i) qi[ft][i] = qx[ft][i] * __expf(ref[i]);
      }
#pragma unroll
      for (int js = 0; js < KS; ++js) {
        const Frag<T> qb = il_frag(qi, js);
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          const T *sr = sS + (16 * dt + r) * LDW + 32 * js + 4 * kq;
          acc[dt] = mma(load4x2(sr, sr + 16), qb, acc[dt]);
        }
      }
    }
    {
      const int t = c0 + 16 * I + r;
      if (t < L) {
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
          store4<T>(O + (size_t)t * D + 16 * dt + 4 * kq, acc[dt][0], acc[dt][1], acc[dt][2], acc[dt][3]);
      }
    }
    __syncthreads();  // B4: the chunk's reads of the state copy done
    // ---- state: S = e^{P} S + Kbar^T V with Kbar = keys~ e^{P} (absorbed) or keys~ e^{P - C_J}
    {
      const float *P3 = sTab + 3 * D;
#pragma unroll
      for (int ft = 0; ft < 2; ++ft) {
        const int fr = 32 * I + 16 * ft;
        const f32x4 P4 = *reinterpret_cast<const f32x4 *>(P3 + fr + 4 * kq);
        float e4[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) e4[i] = __expf(P4[i]);
        const float Pr = P3[fr + r];
        Frag<T> ka[2];  // K-step ks: tokens 32 ks + 8 kq + j, all in sub-chunk 2 ks + kq / 2
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const bf16x4 lo = col4(sKt, LDW, 32 * ks + 8 * kq, fr);
          const bf16x4 hi = col4(sKt, LDW, 32 * ks + 8 * kq + 4, fr);
          const int J = 2 * ks + (kq >> 1);
          const float fac = __expf(absorbed ? Pr : Pr - sTab[J * D + fr + r]);
          float x[8];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            x[j] = to_f(lo[j]) * fac;
            x[4 + j] = to_f(hi[j]) * fac;
          }
          ka[ks] = frag_from<T>(x);
        }
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
#pragma unroll
          for (int i = 0; i < 4; ++i) S[ft][dt][i] *= e4[i];
#pragma unroll
          for (int ks = 0; ks < 2; ++ks)
            S[ft][dt] = mma(ka[ks], load8(sVt + (16 * dt + r) * LDV + 32 * ks + 8 * kq), S[ft][dt]);
        }
      }
    }
    __syncthreads();  // B5: keys~, values and the gate table read
    // state copy S^T [dv][f] for the next chunk's inter product
#pragma unroll
    for (int ft = 0; ft < 2; ++ft)
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
        store4<T>(sS + (16 * dt + r) * LDW + 32 * I + 16 * ft + 4 * kq, S[ft][dt][0], S[ft][dt][1], S[ft][dt][2],
                  S[ft][dt][3]);
  }
}

hipError_t launch_gla(const GlaParams &p, hipStream_t stream) {
  constexpr int DVB = 64;
  using G = gla::Geo<DVB>;
  const int nbh = p.B * p.Hq;
  const int grid = (nbh + 7) / 8 * 16;  // two value halves per head, heads in groups of 8
  const void *kern = p.mode ? reinterpret_cast<const void *>(gla_fwd_kernel<1, DVB>)
                            : reinterpret_cast<const void *>(gla_fwd_kernel<0, DVB>);
  hipError_t e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, G::BYTES);
  if (e != hipSuccess) return e;
  if (p.mode)
    hipLaunchKernelGGL((gla_fwd_kernel<1, DVB>), dim3(grid), dim3(256), G::BYTES, stream, p);
  else
    hipLaunchKernelGGL((gla_fwd_kernel<0, DVB>), dim3(grid), dim3(256), G::BYTES, stream, p);
  return hipGetLastError();
}

}  // namespace lz
