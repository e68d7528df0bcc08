// The query side of the whole-head forward when its W_phi differs from the key side's (separate
// matrices for queries and keys, or one per head): fwd_full_kernel<.., QPHI = true> keeps the key
// side's W_phi^T in LDS (there is no room for a second one) and reads the query side's MFMA
// operands from a fragment-ordered copy in global memory, where it stays in the L2 cache; the
// wide-window variant reads the query feature maps, computed by a pass of their own, instead.
#include "fwd_full.hpp"

namespace lz {

// One copy of D x D bf16 per query head (or one in all): fragment (ft, j) of lane l is the 16-byte
// piece W_phi_q^T[16 ft + l % 16][32 j + 8 (l / 16) .. + 7], stored at ((ft * KS + j) * 64 + l) * 16
// bytes, so that one wave's operand is one contiguous kilobyte.  The values are those the key side
// stages in LDS (load_wT_pairs: W^T, and for the Hedgehog map the rows of -W below, the sign flipped
// on the bits), so the query logits are the same products in the same order as with one shared
// matrix.  One thread per piece: eight 2-byte loads down a column of W, one 16-byte store (a copy is
// 2048 pieces, eight workgroups).
template <bool HH>
__global__ __launch_bounds__(256) void fwd_full_wq_frag_kernel(FwdParams p) {
  using namespace full;
  constexpr int FC = HH ? D / 2 : D;  // columns of W_phi
  constexpr int NPC = NFT * KS * 64;  // pieces of one copy
  const int idx = blockIdx.x * 256 + threadIdx.x;
  const int h = idx / NPC, pc = idx % NPC;
  const int l = pc & 63, fj = pc >> 6, ft = fj / KS, j = fj % KS;
  const int f = 16 * ft + (l & 15), i0 = 32 * j + 8 * (l >> 4);
  const bool neg = HH && f >= FC;
  const uint16_t *src = reinterpret_cast<const uint16_t *>(p.wq) + (size_t)h * p.w_stride + (neg ? f - FC : f);
  uint16_t x[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) x[e] = src[(size_t)(i0 + e) * FC] ^ (neg ? 0x8000u : 0u);
  uint32_t w[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) w[e] = (uint32_t)x[2 * e] | ((uint32_t)x[2 * e + 1] << 16);
  *reinterpret_cast<uint4 *>(reinterpret_cast<char *>(p.ws_wq) + (size_t)idx * 16) = make_uint4(w[0], w[1], w[2], w[3]);
}

hipError_t launch_fwd_full_wq_frag(const FwdParams &p, hipStream_t stream) {
  constexpr int kPieces = full::NFT * full::KS * 64;
  const int copies = p.per_head_q ? p.Hq : 1;
  if (p.hh) hipLaunchKernelGGL(fwd_full_wq_frag_kernel<true>, dim3(copies * kPieces / 256), dim3(256), 0, stream, p);
  else hipLaunchKernelGGL(fwd_full_wq_frag_kernel<false>, dim3(copies * kPieces / 256), dim3(256), 0, stream, p);
  return hipGetLastError();
}

// For the wide-window variant (W > 65), whose registers hold window group Z through the query feature
// map: phi_q = the feature map of q W_phi_q for every query row, bf16, written over the output rows,
// where fwd_full_kernel<true, .., QPHI> reads each row before it writes the row's output.  The features
// of a row are stored in the interleaved order of the kernel's LDS rows (within each group of 32,
// feature 16 h + 4 g + i at position 8 g + 4 h + i), so that a lane moves one 16-byte piece per
// K-step both ways.  The same products in the same order, the same map and one bf16 rounding as
// in the query waves' own computation, so a call whose separate matrices hold equal values matches
// the shared-matrix call bit for bit.  One workgroup of eight waves per (batch, query head,
// PHIQ_ROWS rows), W_phi_q^T staged in LDS once.
constexpr int PHIQ_ROWS = 1024;
template <bool HH>
__global__ __launch_bounds__(512) void fwd_full_phiq_kernel(FwdParams p) {
  using namespace full;
  using T = bf16;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  T *sW = reinterpret_cast<T *>(smem);
  const int tid = threadIdx.x, lane = tid & 63, r16 = lane & 15, g4 = lane >> 4;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nblk = (p.L + PHIQ_ROWS - 1) / PHIQ_ROWS;
  const int bh = blockIdx.x / nblk, blk = blockIdx.x % nblk;
  const int hq = bh % p.Hq;
  const T *Q = reinterpret_cast<const T *>(p.q) + (size_t)bh * p.L * D;
  T *O = reinterpret_cast<T *>(p.out) + (size_t)bh * p.L * D;
  load_wT_pairs<512, HH>(sW, reinterpret_cast<const T *>(p.wq) + (size_t)hq * p.w_stride, tid);
  __syncthreads();
  const int r1 = min(p.L, (blk + 1) * PHIQ_ROWS);
  auto load = [&](Frag<T> (&f)[KS], int t) {
#pragma unroll
    for (int j = 0; j < KS; ++j) f[j] = (t < r1) ? load8(Q + (size_t)t * D + 32 * j + 8 * g4) : frag_zero<T>();
  };
  Frag<T> x[KS], xn[KS];
  const int first = blk * PHIQ_ROWS + 16 * wv;
  load(x, first + r16);
  for (int base = first; base < r1; base += 128) {
    load(xn, base + 128 + r16);  // the wave's next rows in flight
    f32x4 z[NFT];
    float ph[NFT][4];
    // (an opaque offset keeps the W_phi^T reads in the loop: hoisted, they would need 128
    // registers for the whole matrix)
    int w0 = 0;
    asm volatile("" : "+v"(w0));
    feature_logits<T, D, LDWW>(sW + w0, x, r16, g4, z);
    feature_map_rows<HH>(z, ph);
    const int t = base + r16;
    if (t < r1) {
#pragma unroll
      for (int js = 0; js < KS; ++js) {
        float y[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          y[i] = ph[2 * js][i];
          y[4 + i] = ph[2 * js + 1][i];
        }
        *reinterpret_cast<bf16x8 *>(O + (size_t)t * D + 32 * js + 8 * g4) = frag_from<T>(y).v;
      }
    }
#pragma unroll
    for (int j = 0; j < KS; ++j) x[j] = xn[j];
  }
}

hipError_t launch_fwd_full_phiq(const FwdParams &p, hipStream_t stream) {
  constexpr int kLds = full::D * full::LDWW * 2;
  const void *kern = p.hh ? reinterpret_cast<const void *>(fwd_full_phiq_kernel<true>)
                          : reinterpret_cast<const void *>(fwd_full_phiq_kernel<false>);
  hipError_t e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, kLds);
  if (e != hipSuccess) return e;
  const dim3 grid(p.B * p.Hq * ((p.L + PHIQ_ROWS - 1) / PHIQ_ROWS));
  if (p.hh) hipLaunchKernelGGL(fwd_full_phiq_kernel<true>, grid, dim3(512), kLds, stream, p);
  else hipLaunchKernelGGL(fwd_full_phiq_kernel<false>, grid, dim3(512), kLds, stream, p);
  return hipGetLastError();
}

}  // namespace lz
