// Internal launch interface between the C-ABI host code and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lz {

// Byte offsets of the forward kernel's LDS regions (dynamic shared memory).
struct FwdLds {
  int wk, wq, vt, kr, kown, tot, p7, etot, enp7, enr8, sbf, tvt, tk, total;
};

struct FwdParams {
  const void *q, *k, *v, *lg, *wq, *wk, *tk, *tv;
  void *out;
  float *ws_state;  // per-segment end states, fp32, fragment order
  float *ws_decay;  // per-segment sums of log gamma, [B][Hkv][nseg-1][d]
  // continuation of earlier tokens (all optional): start state [B][Hkv][d][d] fp32, the
  // window history [B][Hkv][hist_rows][d] (row hist_rows - j holds the token j places
  // before the first one; staged from the caller's ring), its valid length per sequence
  // min(pos[b], W - 1), and the final state [B][Hkv][d][d]
  const float *state_in;
  float *state_out;
  const void *hist_k, *hist_v;
  const int32_t *pos;
  int hist_rows;
  int64_t w_stride;
  int B, Hq, Hkv, L, W, M, G;
  int nchunks, nseg, cps, ndvb, nring, kring, ngroups;
  FwdLds lds;
  int per_head_q;
  int force_4wave;  // value-block path: the 4-wave kernel also for one query head per KV head
  int full;  // whole-head kernel (fwd_full.hip)
  int sss;   // whole-head kernel: state-pass pieces per segment (divides cps)
  int hh;    // whole-head kernel: Hedgehog feature map (W_phi [d][d/2]) instead of the softmax
  int qphi;  // whole-head kernel: the query side's W_phi differs from the key side's (separate or
             // per-head matrices); its W_phi^T is read from ws_wq in MFMA fragment order (W > 65:
             // phi_q from a pass of its own, in the output rows)
  void *ws_wq;  // qphi: one W_phi_q^T copy of D x D bf16 per query head (per_head_q) or one in all
  int split; // whole-head kernel, two segments: > 0 puts the second segment's start at this chunk
             // plus a shift and has its workgroups walk the chunks before it (no state pass)
  int split_shift;  // the shift: < 0 estimated from the gates in the kernel, else this many chunks
  int split_max;    // largest shift allowed
  float mix, scale;
};

hipError_t launch_fwd(const FwdParams &p, int dtype_bf16, int d, hipStream_t stream);
// whole-head forward kernel (bf16, d = 128, shared W_phi, one query head per key/value
// head, W <= 65); the state pass of launch_fwd runs first when the sequence is segmented
hipError_t launch_fwd_full(const FwdParams &p, hipStream_t stream);
// before it when p.qphi: the query side's W_phi^T in MFMA fragment order into p.ws_wq
hipError_t launch_fwd_full_wq_frag(const FwdParams &p, hipStream_t stream);
// before it when p.qphi and W > 65: the query feature maps, written into the output rows
hipError_t launch_fwd_full_phiq(const FwdParams &p, hipStream_t stream);
// before the forward: window history rows from the caller's ring; after it: the ring of
// the last W tokens and pos += L
hipError_t launch_hist_stage(const FwdParams &p, const void *ring_k, const void *ring_v, int d, int esize,
                             hipStream_t stream);
hipError_t launch_ring_out(const FwdParams &p, const void *ring_k_in, const void *ring_v_in, void *ring_k_out,
                           void *ring_v_out, int32_t *pos, int d, int esize, hipStream_t stream);

struct DecParams {
  float *state;
  void *win_k, *win_v;
  int32_t *pos;
  const void *q, *k, *v, *lg, *wq, *wk, *tk, *tv;
  void *out;
  float *ws_phi;   // [N][Hkv][1+G][d]: phi_k, then phi_q of each grouped query head
  int *ws_count;   // [N]: workgroups of the step that have read pos[n]
  int64_t w_stride;
  int N, Hq, Hkv, W, M, G;
  int hh;  // Hedgehog feature map (W_phi [d][d/2]) instead of the softmax
  float mix, scale;
};

hipError_t launch_decode(const DecParams &p, int dtype_bf16, int d, hipStream_t stream);

}  // namespace lz

namespace lz {
int decode_max_window();
size_t decode_workspace_bytes(int N, int Hq, int Hkv, int d);

// Backward pass (bwd.hip).  Inputs as the forward's plus dy; outputs dq [B,Hq,L,d], dk, dvo,
// dlg [B,Hkv,L,d] in the input type, dwq / dwk (shaped like W_phi) and dtk / dtv [Hkv,M,d] in fp32.
// The workspace holds the feature maps, the fp32 feature-map gradients, the window parts and the
// partial sums (offsets from bwd_workspace_layout).
struct BwdParams {
  const void *q, *k, *v, *lg, *wq, *wk, *tk, *tv, *dy;
  void *dq, *dk, *dvo, *dlg;
  float *dwq, *dwk, *dtk, *dtv;
  float *phq, *phk;  // feature maps, fp32
  float *dphq, *dphk, *dvg, *dqw, *dkw, *dvw, *wstat, *dw_part, *dtk_part, *dtv_part, *dw_tmp;
  int64_t w_stride;  // elements between heads' W_phi; 0: one shared matrix
  int B, Hq, Hkv, L, W, M, G;
  int hh;            // Hedgehog feature map (W_phi [d][d/2])
  float mix, scale;
};
struct BwdWs {
  size_t phq, phk, dphq, dphk, dvg, dqw, dkw, dvw, wstat, dw_part, dtk_part, dtv_part, dw_tmp;
};
size_t bwd_workspace_layout(int B, int Hq, int Hkv, int L, int d, int M, int dtype_bf16, BwdWs *ws);
hipError_t launch_bwd(const BwdParams &p, int dtype_bf16, int d, hipStream_t stream);
}

namespace lz {
// Gated-linear-attention forward alone (gla.hip): bf16, d = 128, one W_phi [d][d] for queries,
// keys and heads, the softmax feature map.  mode 0: standard secondary-chunked form with fp32
// diagonal blocks; mode 1: chunk-start reference with the whole intra-chunk product on MFMA.
struct GlaParams {
  const void *q, *k, *v, *lg, *w;
  void *out;
  int B, Hq, Hkv, L;
  int mode;
};
hipError_t launch_gla(const GlaParams &p, hipStream_t stream);
}
