/*
 * lizard_attn.h -- C ABI of liblizard_attn.so: Lizard attention on AMD
 * MI355X (gfx950), forward over whole sequences and a one-token decode step.
 *
 * What is computed (for every batch entry b and query head h, with key/value
 * head hk = h / (Hq/Hkv)):
 *
 *   phi_q(x) = softmax over features of (x . W_phi_q[h])   (likewise phi_k
 *   with W_phi_k[hk]); softmax over the d features, max subtracted.
 *
 *   Global branch -- gated linear attention.  With the per-key-dimension gate
 *   gamma_i = exp(log_gamma_i) (d values per token, one per row of the d x d
 *   state):
 *       S_i = diag(gamma_i) S_{i-1} + phi_k(k_i) v_i^T,    S_{-1} = 0
 *       y_gla_i = phi_q(q_i)^T S_i
 *   ("Lizard: An Efficient Linearization Framework for Large Language
 *   Models", papernotes.org summary, section "key designs", Gated Linear
 *   Attention item; the arXiv page's Method section explains why the gate is
 *   handled in log space.)
 *
 *   Local branch -- anchor window attention.  One softmax over the M
 *   meta-memory keys and the W most recent keys (token i included):
 *       y_win_i = softmax([scale q_i.T_k[hk,m] ; scale q_i.k_j]) . [T_v ; v_j],
 *       m < M, max(0, i-W+1) <= j <= i
 *   (same summary, "key designs", Anchor Window Attention item.)
 *
 *   Output: y_i = mix * y_gla_i + (1 - mix) * y_win_i (same summary, "overall
 *   framework": the two branch outputs are combined with weights).
 *
 * Conventions shared by every entry point:
 *   - All tensor arguments are DEVICE pointers to contiguous row-major
 *     arrays, 16-byte aligned, in the element type given by `dtype`
 *     (except where a type is spelled out).  The caller owns every buffer.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Calls only
 *     enqueue work on it and return; nothing synchronises the host unless the
 *     option "debug_sync" is set (lizard_set_option, or LIZARD_DEBUG_SYNC=1 in
 *     the environment when the library is loaded).
 *   - The library allocates no device memory.  Scratch space comes from the
 *     caller's `workspace` argument.
 *   - Errors are reported only through the return value.  On any status other
 *     than LIZARD_OK nothing has been launched and no output was written
 *     (LIZARD_ERR_HIP: a launch or HIP call failed; work enqueued before the
 *     failure may have run).  lizard_last_error() returns a thread-local text
 *     with the detail.  Device-side faults surface at the caller's next
 *     synchronisation as HIP errors.
 *   - Preconditions not checked on the device: inputs are finite;
 *     log_gamma <= 0 (gamma in (0,1]; use a large finite negative value such
 *     as -1e4 for gamma = 0, never -inf); outputs do not alias inputs.
 *   - Supported head dimensions: d = 64 or 128 for bf16, d = 64 for fp32.
 *     The feature dimension equals d for both feature maps (the softmax map
 *     above, and the Hedgehog map of the *_hedgehog entry points, whose
 *     W_phi is [d, d/2]).  Meta tokens: 0 <= M <= 16.
 */
#ifndef LIZARD_ATTN_H
#define LIZARD_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  LIZARD_OK = 0,
  LIZARD_ERR_INVALID_ARG = 1, /* null pointer, bad size, misaligned pointer */
  LIZARD_ERR_UNSUPPORTED = 2, /* valid request this build has no kernel for  */
  LIZARD_ERR_WORKSPACE = 3,   /* workspace missing or too small              */
  LIZARD_ERR_HIP = 4          /* a HIP runtime call or a launch failed       */
} lizard_status;

typedef enum { LIZARD_F32 = 0, LIZARD_BF16 = 1 } lizard_dtype;

/*
 * Forward over whole sequences.
 *   q          [B, Hq, L, d]     queries
 *   k, v       [B, Hkv, L, d]    keys, values
 *   log_gamma  [B, Hkv, L, d]    log of the gate, one value per key dimension
 *   w_phi_q    query-side feature-map weights [d, d] for head h at
 *              w_phi_q + h * w_phi_head_stride elements (stride 0: one matrix
 *              for every head; otherwise at least d * d elements and a
 *              multiple of 16 bytes, so that every matrix is 16-byte aligned);
 *              w_phi_k likewise, indexed by key/value head
 *   t_k, t_v   [Hkv, M, d]       meta-memory keys / values (may be NULL if M = 0)
 *   out        [B, Hq, L, d]     written
 *   Hq must be a multiple of Hkv.  B = 0 or L = 0 is an empty problem: OK,
 *   nothing launched.  `scale` multiplies the window logits (1/sqrt(d) gives
 *   standard scaled dot-product attention); it must be finite.  `mix` weighs
 *   the global branch and 1 - mix the window: finite and >= 0 (mix > 1 is
 *   allowed and gives the window a negative weight), else
 *   LIZARD_ERR_INVALID_ARG.
 *   workspace  device scratch of at least lizard_attn_fwd_workspace_bytes()
 *              bytes for the same shapes (may be NULL when that is 0); its
 *              contents on entry do not matter and are clobbered.
 */
lizard_status lizard_attn_fwd(const void *q, const void *k, const void *v,
                              const void *log_gamma, const void *w_phi_q,
                              const void *w_phi_k, int64_t w_phi_head_stride,
                              const void *t_k, const void *t_v, void *out,
                              int B, int Hq, int Hkv, int L, int d, int W,
                              int M, float mix, float scale,
                              lizard_dtype dtype, void *workspace,
                              size_t workspace_bytes, void *stream);

/* Workspace bytes lizard_attn_fwd needs for these shapes (0 if none).  It
 * also covers lizard_attn_fwd_hedgehog. */
size_t lizard_attn_fwd_workspace_bytes(int B, int Hq, int Hkv, int L, int d,
                                       int W, lizard_dtype dtype);

/*
 * Forward with the Lizard paper's own feature map, the Hedgehog map
 *   phi(x) = exp(x . W_phi) (+) exp(-x . W_phi)
 * (the two halves concatenated, exp(xW) first, no normalisation; arXiv page,
 * Method section, the hardware-efficient reparameterization paragraph), in
 * place of the softmax over features.  W_phi is [d, d/2], so that the
 * feature dimension -- the rows of the state and the entries of log_gamma per
 * token -- is d: feature f < d/2 is exp((xW)_f), feature d/2 + f is
 * exp(-(xW)_f).  Everything else as in lizard_attn_fwd, with the same
 * workspace: W_phi shared, separate for queries and keys, or one per head
 * (w_phi_head_stride >= d * d/2 elements).  Built for bf16, d = 128 and
 * W <= 129; other requests return LIZARD_ERR_UNSUPPORTED.  Precondition, not
 * checked: the logits x . W_phi stay within about +-80, where exp is finite in
 * fp32.
 */
lizard_status lizard_attn_fwd_hedgehog(const void *q, const void *k,
                                       const void *v, const void *log_gamma,
                                       const void *w_phi_q, const void *w_phi_k,
                                       int64_t w_phi_head_stride,
                                       const void *t_k, const void *t_v,
                                       void *out, int B, int Hq, int Hkv,
                                       int L, int d, int W, int M, float mix,
                                       float scale, lizard_dtype dtype,
                                       void *workspace, size_t workspace_bytes,
                                       void *stream);

/*
 * Forward as a continuation (chunked prefill feeding decode): the L new tokens
 * of sequence b follow pos[b] earlier ones, whose effect arrives as the state
 * and ring the decode step uses (the recurrent form of the method: arXiv page,
 * Preliminaries; both branches: papernotes.org summary, "key designs").  The
 * outputs equal those of one forward over all pos[b] + L tokens.  Arguments as
 * in lizard_attn_fwd, plus (each may be NULL):
 *   state_in   [B, Hkv, d, d] fp32: S after the earlier tokens (NULL: zero).
 *   win_k_in, win_v_in [B, Hkv, W, d]: ring of the earlier keys / values,
 *              token t in slot t % W (as lizard_attn_decode keeps it).  Both or
 *              neither; require pos.  NULL: the window sees no earlier token.
 *   pos        [B] int32 on the device: earlier tokens per sequence; advanced by
 *              L at the end, after every read.
 *   state_out  [B, Hkv, d, d] fp32: S after the last new token.  Must not be
 *              state_in.
 *   win_k_out, win_v_out [B, Hkv, W, d]: the ring after the call (may be the
 *              ring in, updated in place).  Both or neither.
 *   workspace  at least lizard_attn_fwd_ext_workspace_bytes() bytes: the
 *              forward's own scratch plus the staged window history.
 * Calls on one stream run in order; state, rings and pos of a call must not be
 * touched by another stream meanwhile.  L = 0 launches nothing.
 */
lizard_status lizard_attn_fwd_ext(const void *q, const void *k, const void *v,
                                  const void *log_gamma, const void *w_phi_q,
                                  const void *w_phi_k, int64_t w_phi_head_stride,
                                  const void *t_k, const void *t_v, void *out,
                                  int B, int Hq, int Hkv, int L, int d, int W,
                                  int M, float mix, float scale,
                                  lizard_dtype dtype, const float *state_in,
                                  const void *win_k_in, const void *win_v_in,
                                  int32_t *pos, float *state_out,
                                  void *win_k_out, void *win_v_out,
                                  void *workspace, size_t workspace_bytes,
                                  void *stream);

/* Workspace bytes lizard_attn_fwd_ext needs for these shapes (ring in given). */
size_t lizard_attn_fwd_ext_workspace_bytes(int B, int Hq, int Hkv, int L,
                                           int d, int W, lizard_dtype dtype);

/*
 * One decode step: every sequence n takes one new token, in place.  This is the
 * recurrent (constant-memory) form of the same attention: the global branch
 * carries its d x d state from token to token (arXiv page, Preliminaries, the
 * recurrent view of linear attention; Experiments, "Generation Efficiency":
 * memory and throughput stay constant with the length generated), and the
 * window keeps only its last W keys and values (papernotes.org summary, "key
 * designs", Anchor Window Attention item).
 *   state       [N, Hkv, d, d] float32 (always fp32), the S matrix of the
 *               global branch; row f is key dimension f.  Updated.
 *   win_k, win_v [N, Hkv, W, d] ring buffers of the last W keys / values; the
 *               token with index t sits in slot t % W.  The new token is
 *               written into slot pos[n] % W.  Updated.
 *   pos         [N] int32: tokens already seen by sequence n (the index of the
 *               new token); slots beyond pos[n] are ignored while
 *               pos[n] + 1 < W.  Incremented by one.
 *   q [N, Hq, d]; k, v, log_gamma [N, Hkv, d]; out [N, Hq, d] (written)
 *   w_phi_q, w_phi_k, w_phi_head_stride, t_k, t_v, M, mix, scale: as in the
 *   forward (the same ranges of mix and scale).  The per-token arithmetic is the forward's: decay, add, read out;
 *   then a softmax over the M meta keys and the min(pos+1, W) newest keys.
 *   Running L steps from a zero state, pos = 0, reproduces the forward on
 *   those L tokens.
 *   workspace   device scratch of at least lizard_attn_decode_workspace_bytes()
 *               bytes (16-byte aligned), clobbered: the step's feature maps
 *               pass through it between its two kernels, with one counter per
 *               sequence.
 *   Calls on one stream run in order; calls on different streams that share
 *   state, rings, pos or workspace race.  A call launches two kernels and makes
 *   no other device call (no allocation, no memset, no synchronisation unless
 *   the debug option asks for one), so a run of steps can be captured in one
 *   HIP graph and replayed; pos advances on the device, so each replay takes
 *   the next steps.
 */
lizard_status lizard_attn_decode(float *state, void *win_k, void *win_v,
                                 int32_t *pos, const void *q, const void *k,
                                 const void *v, const void *log_gamma,
                                 const void *w_phi_q, const void *w_phi_k,
                                 int64_t w_phi_head_stride, const void *t_k,
                                 const void *t_v, void *out, int N, int Hq,
                                 int Hkv, int d, int W, int M, float mix,
                                 float scale, lizard_dtype dtype,
                                 void *workspace, size_t workspace_bytes,
                                 void *stream);

/* Workspace bytes lizard_attn_decode needs: 4 * (N*Hkv*(1 + Hq/Hkv)*d + N);
 * 0 for an empty or invalid shape. */
size_t lizard_attn_decode_workspace_bytes(int N, int Hq, int Hkv, int d,
                                          lizard_dtype dtype);

/*
 * One decode step with the Hedgehog feature map (see lizard_attn_fwd_hedgehog):
 * W_phi is [d, d/2] per matrix (w_phi_head_stride = 0, or at least d*d/2
 * elements between heads' matrices), the state's rows are the d features
 * exp(xW) (+) exp(-xW).  Everything else, the workspace included, as in
 * lizard_attn_decode, for the same dtypes and head dimensions.  Running L
 * steps from a zero state reproduces lizard_attn_fwd_hedgehog on those tokens.
 */
lizard_status lizard_attn_decode_hedgehog(float *state, void *win_k,
                                          void *win_v, int32_t *pos,
                                          const void *q, const void *k,
                                          const void *v, const void *log_gamma,
                                          const void *w_phi_q,
                                          const void *w_phi_k,
                                          int64_t w_phi_head_stride,
                                          const void *t_k, const void *t_v,
                                          void *out, int N, int Hq, int Hkv,
                                          int d, int W, int M, float mix,
                                          float scale, lizard_dtype dtype,
                                          void *workspace,
                                          size_t workspace_bytes, void *stream);

/*
 * Backward pass of lizard_attn_fwd: given dy = dL/dy [B, Hq, L, d] for a scalar
 * loss L, the gradients of L with respect to every input of the forward.  The
 * pages train the feature maps, the gate and the meta-memory tokens (arXiv
 * page, Experiments: the first training stage; the Introduction's +32%
 * figure is a training-throughput number), which needs these gradients.
 * Inputs q, k, v, log_gamma, w_phi_q, w_phi_k, w_phi_head_stride, t_k, t_v, W,
 * M, mix, scale, dtype exactly as given to the forward; w_phi_head_stride must
 * be 0 (one matrix for every head) or d*d (one per head).  Outputs (device
 * pointers, overwritten):
 *   dq [B, Hq, L, d]; dk, dv, dlog_gamma [B, Hkv, L, d]   in `dtype`
 *   dw_phi_q, dw_phi_k   fp32, shaped like w_phi_q / w_phi_k ([d, d], or
 *                        [Hq, d, d] / [Hkv, d, d] per head).  They are kept
 *                        apart even when one matrix serves both sides (pass the
 *                        same pointer twice to the forward): its gradient is
 *                        then dw_phi_q + dw_phi_k.
 *   dt_k, dt_v [Hkv, M, d] fp32 (may be NULL when M = 0)
 * The window keys' and values' gradients sum over the query heads of their
 * group, as do the meta tokens' and the key side's feature-map gradients.
 * Built for the forward's dtypes and head dimensions (bf16 d = 64 or 128, fp32
 * d = 64), any W, M <= 16, any grouping.  workspace: at least
 * lizard_attn_bwd_workspace_bytes() bytes (16-byte aligned), clobbered.
 * B = 0 or L = 0 launches nothing and writes nothing.
 */
lizard_status lizard_attn_bwd(const void *q, const void *k, const void *v,
                              const void *log_gamma, const void *w_phi_q,
                              const void *w_phi_k, int64_t w_phi_head_stride,
                              const void *t_k, const void *t_v, const void *dy,
                              void *dq, void *dk, void *dv, void *dlog_gamma,
                              float *dw_phi_q, float *dw_phi_k, float *dt_k,
                              float *dt_v, int B, int Hq, int Hkv, int L, int d,
                              int W, int M, float mix, float scale,
                              lizard_dtype dtype, void *workspace,
                              size_t workspace_bytes, void *stream);

/* Workspace bytes lizard_attn_bwd (and lizard_attn_bwd_hedgehog) needs: about
 * 24 * B * (Hq + Hkv) * L * d bytes (the feature maps, fp32 feature-map and
 * window gradients) plus partial sums; 0 for an empty or invalid shape. */
size_t lizard_attn_bwd_workspace_bytes(int B, int Hq, int Hkv, int L, int d,
                                       int M, lizard_dtype dtype);

/*
 * Backward pass of lizard_attn_fwd_hedgehog (the Hedgehog map exp(xW) (+)
 * exp(-xW), W_phi [d, d/2]): arguments as lizard_attn_bwd, with dw_phi_q /
 * dw_phi_k shaped like the [d, d/2] (or per-head [H, d, d/2]) matrices and
 * w_phi_head_stride 0 or d*d/2.  Unlike the Hedgehog forward it takes separate
 * and per-head matrices, every built dtype and head dimension, and any W.
 */
lizard_status lizard_attn_bwd_hedgehog(const void *q, const void *k,
                                       const void *v, const void *log_gamma,
                                       const void *w_phi_q, const void *w_phi_k,
                                       int64_t w_phi_head_stride,
                                       const void *t_k, const void *t_v,
                                       const void *dy, void *dq, void *dk,
                                       void *dv, void *dlog_gamma,
                                       float *dw_phi_q, float *dw_phi_k,
                                       float *dt_k, float *dt_v, int B, int Hq,
                                       int Hkv, int L, int d, int W, int M,
                                       float mix, float scale,
                                       lizard_dtype dtype, void *workspace,
                                       size_t workspace_bytes, void *stream);

/*
 * lizard_attn_decode without a workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  Arguments and results as lizard_attn_decode (softmax
 * feature map).  The step's scratch (4 * (N*Hkv*(1 + Hq/Hkv)*d + N) bytes: the
 * feature maps and one counter per sequence) lives in a static device array of
 * 32 MiB that each GPU the library runs on holds until the process ends; the
 * call allocates nothing.  Shapes that need more scratch return
 * LIZARD_ERR_UNSUPPORTED (e.g. N = 256, Hq = Hkv = 32, d = 128 needs 8.4 MB;
 * N*Hkv*(1 + Hq/Hkv)*d must stay below about 8.3 million).  Every call on one
 * GPU uses that GPU's one array: calls that overlap on a GPU (different
 * streams, or host threads) race and give wrong results; calls in order on one
 * stream are safe.  The scratch needs no clearing between calls (the step's
 * first kernel resets its counters).
 */
lizard_status lizard_attn_decode_noalloc(float *state, void *win_k, void *win_v,
                                         int32_t *pos, const void *q,
                                         const void *k, const void *v,
                                         const void *log_gamma,
                                         const void *w_phi_q,
                                         const void *w_phi_k,
                                         int64_t w_phi_head_stride,
                                         const void *t_k, const void *t_v,
                                         void *out, int N, int Hq, int Hkv,
                                         int d, int W, int M, float mix,
                                         float scale, lizard_dtype dtype,
                                         void *stream);

/* Static text for a status code. */
const char *lizard_status_string(lizard_status s);

/* Thread-local detail of the last non-OK status returned on this thread. */
const char *lizard_last_error(void);

/* Library version string, e.g. "lizard_attn 0.2.0 gfx950". */
const char *lizard_version(void);

/*
 * Tuning and test options of the forward's launch plan (process-wide; they do
 * not change any result beyond rounding):
 *   "debug_sync"      1: synchronise the stream after every call (errors then
 *                     surface at the call).
 *   "fwd_kernel"      0: kernel chosen by shape; 1: the role-split value-block
 *                     kernel; 2: the 4-wave value-block kernel.
 *   "fwd_segments"    0: segments per sequence chosen by shape; n > 0: n.
 *   "fwd_split_shift" with two segments: n >= 0 chunks moved to the first
 *                     segment; a negative value runs the state pass instead of
 *                     the self-started second segment; -1000000 (the start
 *                     value): the shift is estimated from the gates.
 * Start values come from the environment when the library is loaded
 * (LIZARD_DEBUG_SYNC, LIZARD_FWD_KERNEL=split|4wave, LIZARD_FWD_SEGMENTS,
 * LIZARD_FWD_SPLIT_SHIFT).  Calls read the options when they start; changing
 * one while another thread is inside a call affects that call or the next.
 * Unknown names or out-of-range values return LIZARD_ERR_INVALID_ARG.
 */
lizard_status lizard_set_option(const char *name, int value);
/* Current value of an option (0 for an unknown name). */
int lizard_get_option(const char *name);

/*
 * The global (gated-linear-attention) branch alone, for measuring the Lizard
 * paper's reparameterization against the standard chunked algorithm on the
 * same hardware (arXiv page, Method: the standard parallel form keeps its
 * per-element decays in fp32 and so off the matrix cores; Efficiency: the
 * reparameterized forward is reported 32-36% faster):
 *   out_t = sum_{s <= t} sum_f phi(q_t)_f phi(k_s)_f
 *           exp(sum_{s < u <= t} log_gamma_u,f) v_s,
 * the recurrence h_t = gamma_t (.) h_{t-1} + phi(k_t) v_t^T, out_t = phi(q_t)^T h_t
 * of lizard_attn_fwd without the window (its output at mix = 1).
 *   q [B, Hq, L, d]; k, v, log_gamma [B, Hkv, L, d]; out [B, Hq, L, d]
 *   w_phi      [d, d], one matrix for queries, keys and heads; the softmax
 *              over features of x . W_phi
 *   mode       0: standard -- 16-token sub-chunks; blocks below the diagonal
 *              on bf16 matrix products with decays referred to sub-chunk
 *              ends (all factors <= 1), the diagonal blocks element by element
 *              in fp32, one exponential per (query, key, feature);
 *              1: reparameterized -- decays referred to the 64-token chunk
 *              start, the whole masked intra-chunk product on bf16 matrix
 *              products (a chunk whose log decay passes 60 in some feature is
 *              done the standard way).
 * Built for bf16 and d = 128 only (else LIZARD_ERR_UNSUPPORTED); Hq a multiple
 * of Hkv; all pointers device memory, 16-byte aligned, owned by the caller;
 * no workspace.  B = 0 or L = 0: OK, nothing launched.
 */
lizard_status lizard_gla_fwd(const void *q, const void *k, const void *v,
                             const void *log_gamma, const void *w_phi,
                             void *out, int B, int Hq, int Hkv, int L, int d,
                             int mode, lizard_dtype dtype, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* LIZARD_ATTN_H */
