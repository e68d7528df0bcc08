// Forward as a continuation of earlier tokens: the small kernels around the
// forward that connect it to the decode step's state and ring.
//
// The recurrence carries everything before the first new token in S (the
// global branch) and in the last W - 1 keys/values (the window); see the
// recurrent form in the arXiv page's Preliminaries and the two branches in the
// papernotes.org summary's "key designs".  A forward over tokens
// pos .. pos+L-1 that starts from that S and that window history gives the
// same outputs as one forward over all pos + L tokens.
//
//   hist_stage  copies the window history out of the caller's ring (token t in
//               slot t % W) into rows ordered by position: row hist_rows - j
//               holds token pos - j for j <= min(pos, W - 1), other rows zero.
//   ring_out    writes the ring after the call: every slot holds the newest
//               token t < pos + L with t % W == slot (a new token, or the old
//               entry when fewer than W new tokens arrived).
//   pos_advance pos += L, after every other kernel has read pos.
// Rows are copied in 16-byte pieces (d * element size is a multiple of 16).
#include "common.hpp"
#include "internal.hpp"

namespace lz {

__global__ __launch_bounds__(256) void hist_stage_kernel(const uint4 *ring_k, const uint4 *ring_v, uint4 *hist_k,
                                                         uint4 *hist_v, const int32_t *pos, int Hkv, int W,
                                                         int hist_rows, int row16, long long total) {
  const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= total) return;
  const int piece = (int)(idx % row16);
  const long long rowi = idx / row16;                 // (b, hk, r)
  const int r = (int)(rowi % hist_rows);
  const long long bh = rowi / hist_rows;              // b * Hkv + hk
  const int b = (int)(bh / Hkv);
  const int rel = r - hist_rows;                      // -hist_rows .. -1
  const int avail = min(pos[b], W - 1);
  uint4 kv = {0u, 0u, 0u, 0u}, vv = {0u, 0u, 0u, 0u};
  if (-rel <= avail) {
    const int slot = (pos[b] + rel) % W;              // pos + rel >= 0 here
    const long long src = (bh * W + slot) * row16 + piece;
    kv = ring_k[src];
    vv = ring_v[src];
  }
  hist_k[idx] = kv;
  hist_v[idx] = vv;
}

__global__ __launch_bounds__(256) void ring_out_kernel(const uint4 *k, const uint4 *v, const uint4 *ring_k_in,
                                                       const uint4 *ring_v_in, uint4 *ring_k_out, uint4 *ring_v_out,
                                                       const int32_t *pos, int Hkv, int L, int W, int row16,
                                                       long long total) {
  const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= total) return;
  const int piece = (int)(idx % row16);
  const long long sloti = idx / row16;                // (b, hk, slot)
  const int slot = (int)(sloti % W);
  const long long bh = sloti / W;
  const int b = (int)(bh / Hkv);
  const int p0 = pos ? pos[b] : 0;
  const int last = p0 + L - 1;                        // newest token
  const int t = last - ((last - slot) % W + W) % W;
  uint4 kv = {0u, 0u, 0u, 0u}, vv = {0u, 0u, 0u, 0u};
  if (t >= p0) {                                      // a token of this call
    const long long src = (bh * L + (t - p0)) * row16 + piece;
    kv = k[src];
    vv = v[src];
  } else if (t >= 0 && ring_k_in) {                   // an earlier token still in the window
    if (ring_k_in == ring_k_out) return;              // in place: already there
    kv = ring_k_in[idx];
    vv = ring_v_in[idx];
  }
  ring_k_out[idx] = kv;
  ring_v_out[idx] = vv;
}

__global__ void pos_advance_kernel(int32_t *pos, int B, int L) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < B) pos[i] += L;
}

hipError_t launch_hist_stage(const FwdParams &p, const void *ring_k, const void *ring_v, int d, int esize,
                             hipStream_t stream) {
  const int row16 = d * esize / 16;
  const long long total = (long long)p.B * p.Hkv * p.hist_rows * row16;
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL(hist_stage_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream,
                     static_cast<const uint4 *>(ring_k), static_cast<const uint4 *>(ring_v),
                     (uint4 *)const_cast<void *>(p.hist_k), (uint4 *)const_cast<void *>(p.hist_v), p.pos, p.Hkv,
                     p.W, p.hist_rows, row16, total);
  return hipGetLastError();
}

hipError_t launch_ring_out(const FwdParams &p, const void *ring_k_in, const void *ring_v_in, void *ring_k_out,
                           void *ring_v_out, int32_t *pos, int d, int esize, hipStream_t stream) {
  const int row16 = d * esize / 16;
  if (ring_k_out) {
    const long long total = (long long)p.B * p.Hkv * p.W * row16;
    hipLaunchKernelGGL(ring_out_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, stream,
                       static_cast<const uint4 *>(p.k), static_cast<const uint4 *>(p.v),
                       static_cast<const uint4 *>(ring_k_in), static_cast<const uint4 *>(ring_v_in),
                       static_cast<uint4 *>(ring_k_out), static_cast<uint4 *>(ring_v_out), pos, p.Hkv, p.L, p.W,
                       row16, total);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (pos) {
    hipLaunchKernelGGL(pos_advance_kernel, dim3((p.B + 255) / 256), dim3(256), 0, stream, pos, p.B, p.L);
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace lz
