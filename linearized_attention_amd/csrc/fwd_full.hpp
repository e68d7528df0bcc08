// Layout constants and feature-map pieces of the whole-head forward (bf16, d = 128), shared by
// its kernels (fwd_full.hip) and the pass that computes the query feature maps on their own when
// the query side's W_phi differs from the key side's (fwd_phiq.hip).
#pragma once
#include "fwd_common.hpp"

namespace lz {
namespace full {

constexpr int D = 128, NFT = 8, KS = 4, NDT = 8, FTW = 2;
constexpr int LDW = 144;  // rows of 128 elements (288 bytes)
constexpr int LDWW = 144; // W_phi^T rows (288 bytes)
constexpr int LDQ = 144;  // decayed-query rows (288 bytes)
constexpr int LDV = 80;   // rows of 64 tokens (160 bytes)
constexpr int LDM = 16;   // rows of 16 meta tokens (32 bytes, 8-byte reads)
constexpr int OFF_W = 0;                        // W_phi^T [f][d]
constexpr int OFF_K = OFF_W + D * LDWW * 2;     // keys of the chunk [s][d]
constexpr int OFF_VT = OFF_K + CH * LDW * 2;    // v^T [dv][token, interleaved]
constexpr int OFF_KT = OFF_VT + D * LDV * 2;    // decayed keys [s][f, interleaved] / log gamma^T [f][s]
constexpr int SZ_KT = (CH * LDW > D * LDV ? CH * LDW : D * LDV) * 2;
constexpr int OFF_SB = OFF_KT + SZ_KT;          // S^T copy [dv][f, interleaved]
constexpr int OFF_Q = OFF_SB + D * LDW * 2;     // decayed queries [t][f, interleaved]
constexpr int OFF_TAB = OFF_Q + CH * LDQ * 2;   // prefix ends C_J, [4][128] fp32
constexpr int OFF_TK = OFF_TAB + 4 * D * 4;     // meta keys [16][d]
constexpr int OFF_TV = OFF_TK + 16 * LDW * 2;   // meta values^T [dv][16]
constexpr int OFF_FLAG = OFF_TV + D * LDM * 2;  // per query wave: bit k = chunk c_begin + k needs
constexpr int FLAG_WORDS = 32;                  // the exact diagonal block (segments of at most 1024 chunks)
constexpr int LDS_BYTES = OFF_FLAG + 4 * FLAG_WORDS * 4;
static_assert(LDS_BYTES <= LDS_LIMIT, "whole-head layout exceeds LDS");

// position of element e (0..31) of a 32-element group in the interleaved layout
__device__ __forceinline__ int ipos(int e) { return (e & 3) | ((e >> 4) << 2) | (((e >> 2) & 3) << 3); }
// token of slot j (0..7) of lane group kq in a 32-wide interleaved operand
__device__ __forceinline__ int islot(int kq, int j) { return 16 * (j >> 2) + 4 * kq + (j & 3); }

}  // namespace full

// W_phi^T [f][d] into LDS (row stride LDWW) from W_phi [d][f] in global memory, by NT threads:
// each thread takes row pairs (d, d + 1) x 8 features, all its loads in flight before the
// transposed 4-byte stores of the pairs.  HH (Hedgehog map): W_phi is [d][D/2], and rows
// D/2 + f receive -W_phi^T (a sign flip, exact in bf16), so that the logits of the D features
// are (xW, -xW).
template <int NT, bool HH = false>
__device__ __forceinline__ void load_wT_pairs(bf16 *dst, const bf16 *src, int tid) {
  using namespace full;
  constexpr int FC = HH ? D / 2 : D;  // columns of W_phi
  constexpr int IT = (D / 2) * (FC / 8) / NT;
  static_assert(IT * NT == (D / 2) * (FC / 8), "thread count must divide the row pairs");
  Frag<bf16> a[IT], b[IT];
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int idx = tid + it * NT, dd = 2 * (idx / (FC / 8)), f0 = (idx % (FC / 8)) * 8;
    a[it] = load8(src + (size_t)dd * FC + f0);
    b[it] = load8(src + (size_t)(dd + 1) * FC + f0);
  }
#pragma unroll
  for (int it = 0; it < IT; ++it) {
    const int idx = tid + it * NT, dd = 2 * (idx / (FC / 8)), f0 = (idx % (FC / 8)) * 8;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      bf16 pair[2] = {a[it].v[j], b[it].v[j]};
      const uint32_t u = *reinterpret_cast<const uint32_t *>(pair);
      *reinterpret_cast<uint32_t *>(dst + (f0 + j) * LDWW + dd) = u;
      if constexpr (HH) *reinterpret_cast<uint32_t *>(dst + (FC + f0 + j) * LDWW + dd) = u ^ 0x80008000u;
    }
  }
}

// The feature map of the wave's rows from their logits z: softmax over the D features (max
// subtracted), or for the Hedgehog map (logits (xW, -xW)) the plain exponential.
template <bool HH, int NFT>
__device__ __forceinline__ void feature_map_rows(const f32x4 (&z)[NFT], float (&phi)[NFT][4]) {
  if constexpr (HH) {
#pragma unroll
    for (int ft = 0; ft < NFT; ++ft)
#pragma unroll
      for (int i = 0; i < 4; ++i) phi[ft][i] = exp2_fast(z[ft][i] * LOG2E);
  } else {
    // softmax over the D features of the row (4 lanes x NFT x 4 values): max and sum as trees
    // rather than one chain through all NFT x 4 values
    float mt[NFT], st[NFT];
#pragma unroll
    for (int ft = 0; ft < NFT; ++ft) mt[ft] = fmaxf(fmaxf(z[ft][0], z[ft][1]), fmaxf(z[ft][2], z[ft][3]));
#pragma unroll
    for (int w = NFT / 2; w >= 1; w /= 2)
#pragma unroll
      for (int ft = 0; ft < w; ++ft) mt[ft] = fmaxf(mt[ft], mt[ft + w]);
    const float zm2 = -wave_max_cols(mt[0]) * LOG2E;
#pragma unroll
    for (int ft = 0; ft < NFT; ++ft) {
#pragma unroll
      for (int i = 0; i < 4; ++i) phi[ft][i] = exp2_fast(__builtin_fmaf(z[ft][i], LOG2E, zm2));
      st[ft] = (phi[ft][0] + phi[ft][1]) + (phi[ft][2] + phi[ft][3]);
    }
#pragma unroll
    for (int w = NFT / 2; w >= 1; w /= 2)
#pragma unroll
      for (int ft = 0; ft < w; ++ft) st[ft] += st[ft + w];
    const float inv = 1.f / wave_sum_cols(st[0]);
#pragma unroll
    for (int ft = 0; ft < NFT; ++ft)
#pragma unroll
      for (int i = 0; i < 4; ++i) phi[ft][i] *= inv;
  }
}


}  // namespace lz
