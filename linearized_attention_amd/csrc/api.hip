// C-ABI entry points of liblizard_attn.so: argument validation, launch plan,
// dispatch to the gfx950 kernels.  Declared and documented in
// include/lizard_attn.h.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <atomic>
#include <cmath>
#include <mutex>

#include "../../include/lizard_attn.h"
#include "internal.hpp"

namespace {

thread_local char g_err[512] = "";

lizard_status fail(lizard_status s, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Tuning and test options.  Their start values come from the environment, read once when the
// library is loaded (LIZARD_DEBUG_SYNC=1, LIZARD_FWD_KERNEL=split|4wave, LIZARD_FWD_SEGMENTS=n,
// LIZARD_FWD_SPLIT_SHIFT=n); lizard_set_option() changes them afterwards.  Calls only read them.
struct Options {
  std::atomic<int> debug_sync{0};
  std::atomic<int> fwd_kernel{0};   // 0: chosen by shape, 1: role-split, 2: 4-wave
  std::atomic<int> segments{0};     // 0: chosen by shape, else this many segments
  std::atomic<int> split_shift{kShiftAuto};  // kShiftAuto: estimated; < 0: no self-started split
  static constexpr int kShiftAuto = -1000000;
  Options() {
    if (const char *e = getenv("LIZARD_DEBUG_SYNC")) debug_sync = (e[0] == '1');
    if (const char *e = getenv("LIZARD_FWD_KERNEL")) fwd_kernel = kernel_code(e);
    if (const char *e = getenv("LIZARD_FWD_SEGMENTS")) segments = atoi(e) > 0 ? atoi(e) : 0;
    if (const char *e = getenv("LIZARD_FWD_SPLIT_SHIFT")) split_shift = atoi(e);
  }
  static int kernel_code(const char *e) {
    if (strcmp(e, "split") == 0) return 1;
    if (strcmp(e, "4wave") == 0) return 2;
    return 0;
  }
};
Options g_opt;

bool debug_sync() { return g_opt.debug_sync.load(std::memory_order_relaxed) != 0; }

lizard_status finish(hipError_t e, hipStream_t stream) {
  if (e == hipSuccess && debug_sync()) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return fail(LIZARD_ERR_HIP, "HIP error: %s", hipGetErrorString(e));
  return LIZARD_OK;
}

bool supported_d(int d, lizard_dtype dt) { return dt == LIZARD_BF16 ? (d == 64 || d == 128) : d == 64; }

constexpr int kChunk = 64;
constexpr int kDV = 64;       // value columns per workgroup
constexpr int kMaxMeta = 16;
constexpr int kTargetBlocks = 256;
constexpr int kStateBlocks = 256;  // state-pass pieces (two 80 KB workgroups fit a CU; with
                                    // the decayed chunks left out, 256 timed better than 512)
constexpr int kMaxFullCps = 1024;   // chunks per segment the whole-head kernel's LDS flags cover

struct FwdPlan {
  int nchunks, nseg, cps, ndvb, nring;
  int sss;  // whole-head kernel: state-pass pieces per segment
  size_t ws_state_bytes, ws_decay_bytes;
};

size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

// Sequence segments are added until there are about 256 workgroups (one per
// (batch, head, segment) for the whole-head kernel, one per (batch, head, 64-column
// value block, segment) otherwise); the option "fwd_segments" overrides the count for tests
// and tuning.  The segment end states are kept per 64-column
// value block in either case (the state pass works per block).
FwdPlan make_plan(int B, int Hq, int Hkv, int L, int d, int W, bool full) {
  FwdPlan p{};
  p.nchunks = (L + kChunk - 1) / kChunk;
  p.ndvb = d / kDV;
  const long base = full ? (long)B * Hq : (long)B * Hkv * p.ndvb;
  long nseg = (kTargetBlocks + base - 1) / base;
  if (const int v = g_opt.segments.load(std::memory_order_relaxed)) nseg = v;
  if (full && nseg < (p.nchunks + kMaxFullCps - 1) / kMaxFullCps) nseg = (p.nchunks + kMaxFullCps - 1) / kMaxFullCps;
  if (nseg > p.nchunks) nseg = p.nchunks;
  if (nseg < 1) nseg = 1;
  p.cps = (int)((p.nchunks + nseg - 1) / nseg);
  p.nseg = (p.nchunks + p.cps - 1) / p.cps;
  p.nring = (W - 1 <= kChunk) ? 2 : 3;
  if (p.nseg > 1) {
    p.ws_state_bytes = (size_t)B * Hkv * p.ndvb * (p.nseg - 1) * (size_t)d * kDV * sizeof(float);
    p.ws_decay_bytes = align256((size_t)B * Hkv * (p.nseg - 1) * (size_t)d * sizeof(float));
  }
  p.sss = 1;
  if (full && p.nseg > 1) {
    // the state pass (all chunks before the last segment) in about kStateBlocks pieces
    long ss = kStateBlocks / ((long)B * Hkv * (p.nseg - 1));
    if (ss < 1) ss = 1;
    if (ss > p.cps) ss = p.cps;
    while (p.cps % ss) --ss;
    p.sss = (int)ss;
    p.ws_state_bytes = (size_t)B * Hkv * (p.nseg - 1) * p.sss * (size_t)d * d * sizeof(float);
    p.ws_decay_bytes = align256((size_t)B * Hkv * (p.nseg - 1) * p.sss * (size_t)d * sizeof(float));
  }
  return p;
}

size_t plan_bytes(const FwdPlan &p) { return p.ws_state_bytes + p.ws_decay_bytes; }

// The whole-head kernel serves bf16 at d = 128 with W <= 129, any grouping of query heads and
// any W_phi arrangement (the option "fwd_kernel" = 1 or 2 selects the value-block kernels
// instead, for tests and A/B timing).
bool use_full_kernel(int d, int W, lizard_dtype dtype) {
  if (g_opt.fwd_kernel.load(std::memory_order_relaxed) != 0) return false;
  return dtype == LIZARD_BF16 && d == 128 && W <= 2 * kChunk + 1;
}

// Whether the query side needs a W_phi of its own on the whole-head path: separate matrices, or
// per-head ones with grouped query heads (with G = 1 and one pointer, query head h and key/value
// head h use the same matrix).
bool query_w_differs(const void *wq, const void *wk, int64_t w_stride, int G) {
  return wq != wk || (w_stride != 0 && G > 1);
}

// The whole-head kernel's workspace: its plan's segment states, then (when the query side's
// W_phi differs from the key side's) one fragment-ordered W_phi_q^T copy of d x d bf16 per query
// head, at the next 256-byte boundary.
size_t full_ws_bytes(const FwdPlan &plan, int Hq, int d, bool qphi) {
  return qphi ? align256(plan_bytes(plan)) + align256((size_t)Hq * d * d * 2) : plan_bytes(plan);
}

// Workspace for either plan (the caller does not say whether W_phi is shared).
size_t seg_workspace_bytes(int B, int Hq, int Hkv, int L, int d, int W, lizard_dtype dtype) {
  const size_t sa = plan_bytes(make_plan(B, Hq, Hkv, L, d, W, false));
  const bool maybe_full = use_full_kernel(d, W, dtype);
  const size_t sb = maybe_full ? full_ws_bytes(make_plan(B, Hq, Hkv, L, d, W, true), Hq, d, true) : 0;
  return sa > sb ? sa : sb;
}

// State import/export of a continuation call (all optional; see lizard_attn_fwd_ext).
struct FwdExt {
  const float *state_in = nullptr;
  const void *win_k_in = nullptr, *win_v_in = nullptr;
  int32_t *pos = nullptr;
  float *state_out = nullptr;
  void *win_k_out = nullptr, *win_v_out = nullptr;
};

// Rows of window history a continuation stages: W - 1 rounded up to whole chunks.
int hist_rows_for(int W) { return W > 1 ? ((W - 1 + kChunk - 1) / kChunk) * kChunk : 0; }

size_t ext_hist_bytes(int B, int Hkv, int d, int W, lizard_dtype dtype) {
  const size_t es = dtype == LIZARD_BF16 ? 2 : 4;
  return align256((size_t)B * Hkv * hist_rows_for(W) * d * es);
}

lizard_status fwd_impl(const void *q, const void *k, const void *v, const void *log_gamma, const void *w_phi_q,
                       const void *w_phi_k, int64_t w_phi_head_stride, const void *t_k, const void *t_v, void *out,
                       int B, int Hq, int Hkv, int L, int d, int W, int M, float mix, float scale,
                       lizard_dtype dtype, void *workspace, size_t workspace_bytes, void *stream,
                       const FwdExt *ext, bool hedgehog = false) {
  if (dtype != LIZARD_F32 && dtype != LIZARD_BF16) return fail(LIZARD_ERR_INVALID_ARG, "unknown dtype %d", (int)dtype);
  if (B < 0 || L < 0) return fail(LIZARD_ERR_INVALID_ARG, "B=%d and L=%d must be >= 0", B, L);
  if (Hq < 1 || Hkv < 1 || d < 1 || W < 1 || M < 0)
    return fail(LIZARD_ERR_INVALID_ARG, "need Hq, Hkv, d, W >= 1 and M >= 0 (got Hq=%d Hkv=%d d=%d W=%d M=%d)", Hq,
                Hkv, d, W, M);
  if (Hq % Hkv != 0) return fail(LIZARD_ERR_INVALID_ARG, "Hq=%d is not a multiple of Hkv=%d", Hq, Hkv);
  if (w_phi_head_stride < 0) return fail(LIZARD_ERR_INVALID_ARG, "negative w_phi_head_stride");
  if (!(std::isfinite(mix) && mix >= 0.f) || !std::isfinite(scale))
    return fail(LIZARD_ERR_INVALID_ARG, "mix=%g must be finite and >= 0, scale=%g finite", (double)mix, (double)scale);
  if (!supported_d(d, dtype))
    return fail(LIZARD_ERR_UNSUPPORTED, "head dim d=%d not built for %s", d, dtype == LIZARD_BF16 ? "bf16" : "fp32");
  if (M > kMaxMeta) return fail(LIZARD_ERR_UNSUPPORTED, "M=%d meta tokens (at most %d)", M, kMaxMeta);
  const int64_t wsize = (int64_t)d * (hedgehog ? d / 2 : d);  // elements of one W_phi
  if (w_phi_head_stride != 0 && w_phi_head_stride < wsize)
    return fail(LIZARD_ERR_INVALID_ARG, "w_phi_head_stride=%lld overlaps matrices of %lld elements",
                (long long)w_phi_head_stride, (long long)wsize);
  if (w_phi_head_stride * (dtype == LIZARD_BF16 ? 2 : 4) % 16 != 0)
    return fail(LIZARD_ERR_INVALID_ARG, "w_phi_head_stride=%lld elements leaves a matrix off 16-byte alignment",
                (long long)w_phi_head_stride);
  if (hedgehog && !use_full_kernel(d, W, dtype))
    return fail(LIZARD_ERR_UNSUPPORTED, "the Hedgehog map is built for bf16, d = 128, W <= %d", 2 * kChunk + 1);
  if (B == 0 || L == 0) return LIZARD_OK;  // empty problem
  if (!q || !k || !v || !log_gamma || !w_phi_q || !w_phi_k || !out)
    return fail(LIZARD_ERR_INVALID_ARG, "null tensor pointer");
  if (M > 0 && (!t_k || !t_v)) return fail(LIZARD_ERR_INVALID_ARG, "t_k/t_v null with M=%d", M);
  const void *ptrs[] = {q, k, v, log_gamma, w_phi_q, w_phi_k, out, t_k, t_v};
  for (const void *ptr : ptrs)
    if (ptr && !aligned16(ptr)) return fail(LIZARD_ERR_INVALID_ARG, "tensor pointer %p not 16-byte aligned", ptr);
  if ((int64_t)B * Hq * L > (int64_t)1 << 40) return fail(LIZARD_ERR_INVALID_ARG, "problem too large");

  const bool history = ext && ext->pos && ext->win_k_in;  // window keys before the first token
  if (ext) {
    if ((ext->win_k_in == nullptr) != (ext->win_v_in == nullptr) ||
        (ext->win_k_out == nullptr) != (ext->win_v_out == nullptr))
      return fail(LIZARD_ERR_INVALID_ARG, "ring keys and values must be given together");
    if (ext->win_k_in && !ext->pos) return fail(LIZARD_ERR_INVALID_ARG, "a ring in needs pos");
    if (ext->state_out && ext->state_out == ext->state_in)
      return fail(LIZARD_ERR_INVALID_ARG, "state_out must not be state_in");
    const void *eptrs[] = {ext->state_in, ext->win_k_in, ext->win_v_in, ext->state_out, ext->win_k_out,
                           ext->win_v_out};
    for (const void *ptr : eptrs)
      if (ptr && !aligned16(ptr)) return fail(LIZARD_ERR_INVALID_ARG, "tensor pointer %p not 16-byte aligned", ptr);
    if (ext->pos && (reinterpret_cast<uintptr_t>(ext->pos) & 3u))
      return fail(LIZARD_ERR_INVALID_ARG, "pos not 4-byte aligned");
  }
  const bool full = use_full_kernel(d, W, dtype);
  const FwdPlan plan = make_plan(B, Hq, Hkv, L, d, W, full);
  const bool qphi = full && query_w_differs(w_phi_q, w_phi_k, w_phi_head_stride, Hq / Hkv);
  const size_t seg_bytes = full ? full_ws_bytes(plan, Hq, d, qphi) : plan_bytes(plan);
  const size_t hist_bytes = history ? ext_hist_bytes(B, Hkv, d, W, dtype) : 0;
  const size_t need = (hist_bytes ? align256(seg_bytes) : seg_bytes) + 2 * hist_bytes;
  if (need > 0) {
    if (!workspace || workspace_bytes < need)
      return fail(LIZARD_ERR_WORKSPACE, "workspace of %zu bytes needed, got %zu", need,
                  workspace ? workspace_bytes : (size_t)0);
    if (!aligned16(workspace)) return fail(LIZARD_ERR_INVALID_ARG, "workspace not 16-byte aligned");
  }

  lz::FwdParams p{};
  p.q = q; p.k = k; p.v = v; p.lg = log_gamma; p.wq = w_phi_q; p.wk = w_phi_k;
  p.tk = t_k; p.tv = t_v; p.out = out;
  p.ws_state = need ? static_cast<float *>(workspace) : nullptr;
  p.ws_decay = need ? reinterpret_cast<float *>(static_cast<char *>(workspace) + plan.ws_state_bytes) : nullptr;
  p.w_stride = w_phi_head_stride;
  p.B = B; p.Hq = Hq; p.Hkv = Hkv; p.L = L; p.W = W; p.M = M; p.G = Hq / Hkv;
  p.nchunks = plan.nchunks; p.nseg = plan.nseg; p.cps = plan.cps; p.ndvb = plan.ndvb; p.nring = plan.nring;
  p.per_head_q = w_phi_head_stride != 0;
  p.full = full ? 1 : 0;
  p.force_4wave = g_opt.fwd_kernel.load(std::memory_order_relaxed) == 2 ? 1 : 0;
  p.sss = plan.sss;
  p.hh = hedgehog ? 1 : 0;
  p.qphi = qphi ? 1 : 0;
  p.ws_wq = qphi ? static_cast<char *>(workspace) + align256(plan_bytes(plan)) : nullptr;
  // Two segments on the whole-head path: the second one's workgroups walk the chunks before it
  // themselves (no state pass), and the first segment takes a few chunks more to even out the
  // walk.  Not with a start state or window history (the walk starts from zero at chunk 0).
  // The shift is estimated in the kernel from the gates (the option "fwd_split_shift" = n >= 0
  // fixes it at n chunks; a negative value turns the split off: state pass instead).
  p.split = 0;
  const int shift_opt = g_opt.split_shift.load(std::memory_order_relaxed);
  const bool shift_auto = shift_opt == Options::kShiftAuto;
  const int shift_fixed = shift_auto ? -1 : shift_opt;
  if (full && plan.nseg == 2 && !(ext && (ext->state_in || history)) && (shift_auto || shift_fixed >= 0) &&
      plan.cps < plan.nchunks && plan.cps <= kMaxFullCps) {
    int smax = plan.cps / 4;
    if (smax > plan.nchunks - 1 - plan.cps) smax = plan.nchunks - 1 - plan.cps;
    if (smax > kMaxFullCps - plan.cps) smax = kMaxFullCps - plan.cps;
    p.split = plan.cps;
    p.split_shift = shift_fixed;
    p.split_max = smax;
  }
  p.mix = mix; p.scale = scale;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int esize = dtype == LIZARD_BF16 ? 2 : 4;
  if (ext) {
    p.state_in = ext->state_in;
    p.state_out = ext->state_out;
    p.pos = history ? ext->pos : nullptr;  // the forward reads pos only to bound the history
    if (history) {
      char *h = static_cast<char *>(workspace) + align256(seg_bytes);
      p.hist_k = h;
      p.hist_v = h + hist_bytes;
      p.hist_rows = hist_rows_for(W);
      hipError_t e = lz::launch_hist_stage(p, ext->win_k_in, ext->win_v_in, d, esize, st);
      if (e != hipSuccess) return finish(e, st);
    }
  }
  hipError_t e = lz::launch_fwd(p, dtype == LIZARD_BF16, d, st);
  if (e == hipSuccess && ext && (ext->win_k_out || ext->pos))
    e = lz::launch_ring_out(p, ext->win_k_in, ext->win_v_in, ext->win_k_out, ext->win_v_out, ext->pos, d, esize, st);
  return finish(e, st);
}

}  // namespace

extern "C" {

const char *lizard_status_string(lizard_status s) {
  switch (s) {
    case LIZARD_OK: return "ok";
    case LIZARD_ERR_INVALID_ARG: return "invalid argument";
    case LIZARD_ERR_UNSUPPORTED: return "unsupported configuration";
    case LIZARD_ERR_WORKSPACE: return "workspace missing or too small";
    case LIZARD_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char *lizard_last_error(void) { return g_err; }

const char *lizard_version(void) { return "lizard_attn 0.2.0 gfx950"; }

lizard_status lizard_set_option(const char *name, int value) {
  if (!name) return fail(LIZARD_ERR_INVALID_ARG, "null option name");
  if (strcmp(name, "debug_sync") == 0) {
    g_opt.debug_sync = value != 0;
  } else if (strcmp(name, "fwd_kernel") == 0) {
    if (value < 0 || value > 2) return fail(LIZARD_ERR_INVALID_ARG, "fwd_kernel=%d (0, 1 or 2)", value);
    g_opt.fwd_kernel = value;
  } else if (strcmp(name, "fwd_segments") == 0) {
    if (value < 0) return fail(LIZARD_ERR_INVALID_ARG, "fwd_segments=%d must be >= 0", value);
    g_opt.segments = value;
  } else if (strcmp(name, "fwd_split_shift") == 0) {
    g_opt.split_shift = value;
  } else {
    return fail(LIZARD_ERR_INVALID_ARG, "unknown option '%s'", name);
  }
  return LIZARD_OK;
}

int lizard_get_option(const char *name) {
  if (!name) return 0;
  if (strcmp(name, "debug_sync") == 0) return g_opt.debug_sync;
  if (strcmp(name, "fwd_kernel") == 0) return g_opt.fwd_kernel;
  if (strcmp(name, "fwd_segments") == 0) return g_opt.segments;
  if (strcmp(name, "fwd_split_shift") == 0) return g_opt.split_shift;
  return 0;
}

size_t lizard_attn_fwd_workspace_bytes(int B, int Hq, int Hkv, int L, int d, int W, lizard_dtype dtype) {
  (void)Hq;
  (void)dtype;
  if (B <= 0 || L <= 0 || Hkv <= 0 || d <= 0 || d % kDV != 0) return 0;
  return seg_workspace_bytes(B, Hq, Hkv, L, d, W < 1 ? 1 : W, dtype);
}

lizard_status lizard_attn_fwd(const void *q, const void *k, const void *v, const void *log_gamma,
                              const void *w_phi_q, const void *w_phi_k, int64_t w_phi_head_stride,
                              const void *t_k, const void *t_v, void *out, int B, int Hq, int Hkv, int L,
                              int d, int W, int M, float mix, float scale, lizard_dtype dtype,
                              void *workspace, size_t workspace_bytes, void *stream) {
  return fwd_impl(q, k, v, log_gamma, w_phi_q, w_phi_k, w_phi_head_stride, t_k, t_v, out, B, Hq, Hkv, L, d, W, M,
                  mix, scale, dtype, workspace, workspace_bytes, stream, nullptr);
}

lizard_status lizard_attn_fwd_hedgehog(const void *q, const void *k, const void *v, const void *log_gamma,
                                       const void *w_phi_q, const void *w_phi_k, int64_t w_phi_head_stride,
                                       const void *t_k, const void *t_v, void *out, int B, int Hq, int Hkv, int L,
                                       int d, int W, int M, float mix, float scale, lizard_dtype dtype,
                                       void *workspace, size_t workspace_bytes, void *stream) {
  return fwd_impl(q, k, v, log_gamma, w_phi_q, w_phi_k, w_phi_head_stride, t_k, t_v, out, B, Hq, Hkv, L, d, W, M,
                  mix, scale, dtype, workspace, workspace_bytes, stream, nullptr, true);
}

size_t lizard_attn_fwd_ext_workspace_bytes(int B, int Hq, int Hkv, int L, int d, int W, lizard_dtype dtype) {
  (void)Hq;
  if (B <= 0 || L <= 0 || Hkv <= 0 || d <= 0 || d % kDV != 0) return 0;
  const size_t seg = seg_workspace_bytes(B, Hq, Hkv, L, d, W < 1 ? 1 : W, dtype);
  const size_t hist = ext_hist_bytes(B, Hkv, d, W < 1 ? 1 : W, dtype);
  return hist ? align256(seg) + 2 * hist : seg;
}

lizard_status lizard_attn_fwd_ext(const void *q, const void *k, const void *v, const void *log_gamma,
                                  const void *w_phi_q, const void *w_phi_k, int64_t w_phi_head_stride,
                                  const void *t_k, const void *t_v, void *out, int B, int Hq, int Hkv, int L,
                                  int d, int W, int M, float mix, float scale, lizard_dtype dtype,
                                  const float *state_in, const void *win_k_in, const void *win_v_in,
                                  int32_t *pos, float *state_out, void *win_k_out, void *win_v_out,
                                  void *workspace, size_t workspace_bytes, void *stream) {
  FwdExt ext;
  ext.state_in = state_in;
  ext.win_k_in = win_k_in;
  ext.win_v_in = win_v_in;
  ext.pos = pos;
  ext.state_out = state_out;
  ext.win_k_out = win_k_out;
  ext.win_v_out = win_v_out;
  return fwd_impl(q, k, v, log_gamma, w_phi_q, w_phi_k, w_phi_head_stride, t_k, t_v, out, B, Hq, Hkv, L, d, W, M,
                  mix, scale, dtype, workspace, workspace_bytes, stream, &ext);
}

size_t lizard_attn_decode_workspace_bytes(int N, int Hq, int Hkv, int d, lizard_dtype dtype) {
  (void)dtype;
  if (N <= 0 || Hq <= 0 || Hkv <= 0 || d <= 0 || Hq % Hkv != 0) return 0;
  return lz::decode_workspace_bytes(N, Hq, Hkv, d);
}

// Scratch of lizard_attn_decode_noalloc: the step's feature maps and per-sequence counters (what
// lizard_attn_decode keeps in the caller's workspace), in a static device array.  Every GPU the
// library runs on holds its own copy at its own address until the process ends; host code
// reaches it only through that address (the array's name is a host-side stand-in).
constexpr size_t kDecodeScratchBytes = (size_t)32 << 20;
static __device__ __align__(256) unsigned char scratch[kDecodeScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// Device address of the scratch on the stream's GPU, looked up once per device
// (hipGetSymbolAddress with that device current).
lizard_status scratch_for_stream(hipStream_t st, void **out) {
  int dev = -1;
  hipError_t e = st ? hipStreamGetDevice(st, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return fail(LIZARD_ERR_HIP, "HIP error: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(LIZARD_ERR_UNSUPPORTED, "device %d (at most %d)", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    int cur = -1;
    if ((e = hipGetDevice(&cur)) != hipSuccess) return fail(LIZARD_ERR_HIP, "HIP error: %s", hipGetErrorString(e));
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess)
      return fail(LIZARD_ERR_HIP, "HIP error: %s", hipGetErrorString(e));
    void *ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (cur != dev) {
      const hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess || !ptr)
      return fail(LIZARD_ERR_HIP, "scratch address on device %d: %s", dev, hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return LIZARD_OK;
}

static lizard_status decode_impl(float *state, void *win_k, void *win_v, int32_t *pos, const void *q, const void *k,
                                 const void *v, const void *log_gamma, const void *w_phi_q, const void *w_phi_k,
                                 int64_t w_phi_head_stride, const void *t_k, const void *t_v, void *out, int N, int Hq,
                                 int Hkv, int d, int W, int M, float mix, float scale, lizard_dtype dtype,
                                 void *workspace, size_t workspace_bytes, void *stream, bool hedgehog,
                                 bool static_scratch = false) {
  if (dtype != LIZARD_F32 && dtype != LIZARD_BF16) return fail(LIZARD_ERR_INVALID_ARG, "unknown dtype %d", (int)dtype);
  if (N < 0) return fail(LIZARD_ERR_INVALID_ARG, "N=%d must be >= 0", N);
  if (Hq < 1 || Hkv < 1 || d < 1 || W < 1 || M < 0)
    return fail(LIZARD_ERR_INVALID_ARG, "need Hq, Hkv, d, W >= 1 and M >= 0 (got Hq=%d Hkv=%d d=%d W=%d M=%d)", Hq,
                Hkv, d, W, M);
  if (Hq % Hkv != 0) return fail(LIZARD_ERR_INVALID_ARG, "Hq=%d is not a multiple of Hkv=%d", Hq, Hkv);
  if (w_phi_head_stride < 0) return fail(LIZARD_ERR_INVALID_ARG, "negative w_phi_head_stride");
  if (!(std::isfinite(mix) && mix >= 0.f) || !std::isfinite(scale))
    return fail(LIZARD_ERR_INVALID_ARG, "mix=%g must be finite and >= 0, scale=%g finite", (double)mix, (double)scale);
  if (!supported_d(d, dtype))
    return fail(LIZARD_ERR_UNSUPPORTED, "head dim d=%d not built for %s", d, dtype == LIZARD_BF16 ? "bf16" : "fp32");
  if (M > kMaxMeta) return fail(LIZARD_ERR_UNSUPPORTED, "M=%d meta tokens (at most %d)", M, kMaxMeta);
  if (W > lz::decode_max_window())
    return fail(LIZARD_ERR_UNSUPPORTED, "decode window W=%d (at most %d)", W, lz::decode_max_window());
  const int64_t wsize = (int64_t)d * (hedgehog ? d / 2 : d);  // elements of one W_phi
  if (w_phi_head_stride != 0 && w_phi_head_stride < wsize)
    return fail(LIZARD_ERR_INVALID_ARG, "w_phi_head_stride=%lld overlaps matrices of %lld elements",
                (long long)w_phi_head_stride, (long long)wsize);
  if (w_phi_head_stride * (dtype == LIZARD_BF16 ? 2 : 4) % 16 != 0)
    return fail(LIZARD_ERR_INVALID_ARG, "w_phi_head_stride=%lld elements leaves a matrix off 16-byte alignment",
                (long long)w_phi_head_stride);
  if (N == 0) return LIZARD_OK;
  if (!state || !win_k || !win_v || !pos || !q || !k || !v || !log_gamma || !w_phi_q || !w_phi_k || !out)
    return fail(LIZARD_ERR_INVALID_ARG, "null tensor pointer");
  if (M > 0 && (!t_k || !t_v)) return fail(LIZARD_ERR_INVALID_ARG, "t_k/t_v null with M=%d", M);
  const void *ptrs[] = {state, win_k, win_v, q, k, v, log_gamma, w_phi_q, w_phi_k, out, t_k, t_v};
  for (const void *ptr : ptrs)
    if (ptr && !aligned16(ptr)) return fail(LIZARD_ERR_INVALID_ARG, "tensor pointer %p not 16-byte aligned", ptr);
  if (reinterpret_cast<uintptr_t>(pos) & 3u) return fail(LIZARD_ERR_INVALID_ARG, "pos not 4-byte aligned");
  const size_t need = lz::decode_workspace_bytes(N, Hq, Hkv, d);
  if (static_scratch) {
    if (need > kDecodeScratchBytes)
      return fail(LIZARD_ERR_UNSUPPORTED,
                  "lizard_attn_decode_noalloc: N=%d, Hkv=%d, Hq/Hkv=%d, d=%d need %zu bytes of scratch; the static "
                  "scratch holds %zu (use lizard_attn_decode with a workspace)", N, Hkv, Hq / Hkv, d, need,
                  kDecodeScratchBytes);
    const lizard_status s = scratch_for_stream(static_cast<hipStream_t>(stream), &workspace);
    if (s != LIZARD_OK) return s;
    workspace_bytes = kDecodeScratchBytes;
  }
  if (!workspace || workspace_bytes < need)
    return fail(LIZARD_ERR_WORKSPACE, "workspace of %zu bytes needed, got %zu", need,
                workspace ? workspace_bytes : (size_t)0);
  if (!aligned16(workspace)) return fail(LIZARD_ERR_INVALID_ARG, "workspace not 16-byte aligned");

  lz::DecParams p{};
  p.state = state; p.win_k = win_k; p.win_v = win_v; p.pos = pos;
  p.q = q; p.k = k; p.v = v; p.lg = log_gamma; p.wq = w_phi_q; p.wk = w_phi_k; p.tk = t_k; p.tv = t_v;
  p.out = out; p.w_stride = w_phi_head_stride;
  p.ws_phi = static_cast<float *>(workspace);
  p.ws_count = reinterpret_cast<int *>(p.ws_phi + (size_t)N * Hq * d + (size_t)N * Hkv * d);  // after phi
  p.N = N; p.Hq = Hq; p.Hkv = Hkv; p.W = W; p.M = M; p.G = Hq / Hkv; p.mix = mix; p.scale = scale;
  p.hh = hedgehog ? 1 : 0;
  hipStream_t st = static_cast<hipStream_t>(stream);
  return finish(lz::launch_decode(p, dtype == LIZARD_BF16, d, st), st);
}

lizard_status lizard_attn_decode(float *state, void *win_k, void *win_v, int32_t *pos, const void *q, const void *k,
                                 const void *v, const void *log_gamma, const void *w_phi_q, const void *w_phi_k,
                                 int64_t w_phi_head_stride, const void *t_k, const void *t_v, void *out, int N, int Hq,
                                 int Hkv, int d, int W, int M, float mix, float scale, lizard_dtype dtype,
                                 void *workspace, size_t workspace_bytes, void *stream) {
  return decode_impl(state, win_k, win_v, pos, q, k, v, log_gamma, w_phi_q, w_phi_k, w_phi_head_stride, t_k, t_v,
                     out, N, Hq, Hkv, d, W, M, mix, scale, dtype, workspace, workspace_bytes, stream, false);
}

lizard_status lizard_attn_decode_hedgehog(float *state, void *win_k, void *win_v, int32_t *pos, const void *q,
                                          const void *k, const void *v, const void *log_gamma, const void *w_phi_q,
                                          const void *w_phi_k, int64_t w_phi_head_stride, const void *t_k,
                                          const void *t_v, void *out, int N, int Hq, int Hkv, int d, int W, int M,
                                          float mix, float scale, lizard_dtype dtype, void *workspace,
                                          size_t workspace_bytes, void *stream) {
  return decode_impl(state, win_k, win_v, pos, q, k, v, log_gamma, w_phi_q, w_phi_k, w_phi_head_stride, t_k, t_v,
                     out, N, Hq, Hkv, d, W, M, mix, scale, dtype, workspace, workspace_bytes, stream, true);
}

size_t lizard_attn_bwd_workspace_bytes(int B, int Hq, int Hkv, int L, int d, int M, lizard_dtype dtype) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || L <= 0 || d <= 0 || M < 0 || Hq % Hkv != 0) return 0;
  return lz::bwd_workspace_layout(B, Hq, Hkv, L, d, M, dtype == LIZARD_BF16, nullptr);
}

static lizard_status bwd_impl(const void *q, const void *k, const void *v, const void *log_gamma,
                              const void *w_phi_q, const void *w_phi_k, int64_t w_phi_head_stride, const void *t_k,
                              const void *t_v, const void *dy, void *dq, void *dk, void *dv, void *dlog_gamma,
                              float *dw_phi_q, float *dw_phi_k, float *dt_k, float *dt_v, int B, int Hq, int Hkv,
                              int L, int d, int W, int M, float mix, float scale, lizard_dtype dtype,
                              void *workspace, size_t workspace_bytes, void *stream, bool hedgehog) {
  if (dtype != LIZARD_F32 && dtype != LIZARD_BF16) return fail(LIZARD_ERR_INVALID_ARG, "unknown dtype %d", (int)dtype);
  if (B < 0 || L < 0) return fail(LIZARD_ERR_INVALID_ARG, "B=%d and L=%d must be >= 0", B, L);
  if (Hq < 1 || Hkv < 1 || d < 1 || W < 1 || M < 0)
    return fail(LIZARD_ERR_INVALID_ARG, "need Hq, Hkv, d, W >= 1 and M >= 0 (got Hq=%d Hkv=%d d=%d W=%d M=%d)", Hq,
                Hkv, d, W, M);
  if (Hq % Hkv != 0) return fail(LIZARD_ERR_INVALID_ARG, "Hq=%d is not a multiple of Hkv=%d", Hq, Hkv);
  if (!(std::isfinite(mix) && mix >= 0.f) || !std::isfinite(scale))
    return fail(LIZARD_ERR_INVALID_ARG, "mix=%g must be finite and >= 0, scale=%g finite", (double)mix, (double)scale);
  if (!supported_d(d, dtype))
    return fail(LIZARD_ERR_UNSUPPORTED, "head dim d=%d not built for %s", d, dtype == LIZARD_BF16 ? "bf16" : "fp32");
  if (M > kMaxMeta) return fail(LIZARD_ERR_UNSUPPORTED, "M=%d meta tokens (at most %d)", M, kMaxMeta);
  const int64_t wsize = (int64_t)d * (hedgehog ? d / 2 : d);
  if (w_phi_head_stride != 0 && w_phi_head_stride != wsize)
    return fail(LIZARD_ERR_INVALID_ARG, "w_phi_head_stride=%lld: 0 (shared) or %lld (one matrix per head)",
                (long long)w_phi_head_stride, (long long)wsize);
  if ((int64_t)B * Hq * L > (int64_t)1 << 34) return fail(LIZARD_ERR_INVALID_ARG, "problem too large");
  if (B == 0 || L == 0) return LIZARD_OK;  // empty problem: nothing is written
  if (!q || !k || !v || !log_gamma || !w_phi_q || !w_phi_k || !dy || !dq || !dk || !dv || !dlog_gamma ||
      !dw_phi_q || !dw_phi_k)
    return fail(LIZARD_ERR_INVALID_ARG, "null tensor pointer");
  if (M > 0 && (!t_k || !t_v || !dt_k || !dt_v)) return fail(LIZARD_ERR_INVALID_ARG, "t_k/t_v/dt_k/dt_v null with M=%d", M);
  const void *ptrs[] = {q, k, v, log_gamma, w_phi_q, w_phi_k, t_k, t_v, dy, dq, dk, dv, dlog_gamma,
                        dw_phi_q, dw_phi_k, dt_k, dt_v};
  for (const void *ptr : ptrs)
    if (ptr && !aligned16(ptr)) return fail(LIZARD_ERR_INVALID_ARG, "tensor pointer %p not 16-byte aligned", ptr);
  lz::BwdWs ws{};
  const size_t need = lz::bwd_workspace_layout(B, Hq, Hkv, L, d, M, dtype == LIZARD_BF16, &ws);
  if (!workspace || workspace_bytes < need)
    return fail(LIZARD_ERR_WORKSPACE, "workspace of %zu bytes needed, got %zu", need,
                workspace ? workspace_bytes : (size_t)0);
  if (!aligned16(workspace)) return fail(LIZARD_ERR_INVALID_ARG, "workspace not 16-byte aligned");
  char *w = static_cast<char *>(workspace);
  lz::BwdParams p{};
  p.q = q; p.k = k; p.v = v; p.lg = log_gamma; p.wq = w_phi_q; p.wk = w_phi_k; p.tk = t_k; p.tv = t_v; p.dy = dy;
  p.dq = dq; p.dk = dk; p.dvo = dv; p.dlg = dlog_gamma;
  p.dwq = dw_phi_q; p.dwk = dw_phi_k; p.dtk = dt_k; p.dtv = dt_v;
  p.phq = reinterpret_cast<float *>(w + ws.phq); p.phk = reinterpret_cast<float *>(w + ws.phk);
  p.dphq = reinterpret_cast<float *>(w + ws.dphq); p.dphk = reinterpret_cast<float *>(w + ws.dphk);
  p.dvg = reinterpret_cast<float *>(w + ws.dvg); p.dqw = reinterpret_cast<float *>(w + ws.dqw);
  p.dkw = reinterpret_cast<float *>(w + ws.dkw); p.dvw = reinterpret_cast<float *>(w + ws.dvw);
  p.wstat = reinterpret_cast<float *>(w + ws.wstat); p.dw_part = reinterpret_cast<float *>(w + ws.dw_part);
  p.dtk_part = reinterpret_cast<float *>(w + ws.dtk_part); p.dtv_part = reinterpret_cast<float *>(w + ws.dtv_part);
  p.dw_tmp = reinterpret_cast<float *>(w + ws.dw_tmp);
  p.w_stride = w_phi_head_stride;
  p.B = B; p.Hq = Hq; p.Hkv = Hkv; p.L = L; p.W = W; p.M = M; p.G = Hq / Hkv;
  p.hh = hedgehog ? 1 : 0;
  p.mix = mix; p.scale = scale;
  hipStream_t st = static_cast<hipStream_t>(stream);
  return finish(lz::launch_bwd(p, dtype == LIZARD_BF16, d, st), st);
}

lizard_status lizard_attn_bwd(const void *q, const void *k, const void *v, const void *log_gamma,
                              const void *w_phi_q, const void *w_phi_k, int64_t w_phi_head_stride, const void *t_k,
                              const void *t_v, const void *dy, void *dq, void *dk, void *dv, void *dlog_gamma,
                              float *dw_phi_q, float *dw_phi_k, float *dt_k, float *dt_v, int B, int Hq, int Hkv,
                              int L, int d, int W, int M, float mix, float scale, lizard_dtype dtype,
                              void *workspace, size_t workspace_bytes, void *stream) {
  return bwd_impl(q, k, v, log_gamma, w_phi_q, w_phi_k, w_phi_head_stride, t_k, t_v, dy, dq, dk, dv, dlog_gamma,
                  dw_phi_q, dw_phi_k, dt_k, dt_v, B, Hq, Hkv, L, d, W, M, mix, scale, dtype, workspace,
                  workspace_bytes, stream, false);
}

lizard_status lizard_attn_bwd_hedgehog(const void *q, const void *k, const void *v, const void *log_gamma,
                                       const void *w_phi_q, const void *w_phi_k, int64_t w_phi_head_stride,
                                       const void *t_k, const void *t_v, const void *dy, void *dq, void *dk,
                                       void *dv, void *dlog_gamma, float *dw_phi_q, float *dw_phi_k, float *dt_k,
                                       float *dt_v, int B, int Hq, int Hkv, int L, int d, int W, int M, float mix,
                                       float scale, lizard_dtype dtype, void *workspace, size_t workspace_bytes,
                                       void *stream) {
  return bwd_impl(q, k, v, log_gamma, w_phi_q, w_phi_k, w_phi_head_stride, t_k, t_v, dy, dq, dk, dv, dlog_gamma,
                  dw_phi_q, dw_phi_k, dt_k, dt_v, B, Hq, Hkv, L, d, W, M, mix, scale, dtype, workspace,
                  workspace_bytes, stream, true);
}

lizard_status lizard_gla_fwd(const void *q, const void *k, const void *v, const void *log_gamma, const void *w_phi,
                             void *out, int B, int Hq, int Hkv, int L, int d, int mode, lizard_dtype dtype,
                             void *stream) {
  if (dtype != LIZARD_F32 && dtype != LIZARD_BF16) return fail(LIZARD_ERR_INVALID_ARG, "unknown dtype %d", (int)dtype);
  if (B < 0 || L < 0) return fail(LIZARD_ERR_INVALID_ARG, "B=%d and L=%d must be >= 0", B, L);
  if (Hq < 1 || Hkv < 1 || d < 1)
    return fail(LIZARD_ERR_INVALID_ARG, "need Hq, Hkv, d >= 1 (got Hq=%d Hkv=%d d=%d)", Hq, Hkv, d);
  if (Hq % Hkv != 0) return fail(LIZARD_ERR_INVALID_ARG, "Hq=%d is not a multiple of Hkv=%d", Hq, Hkv);
  if (mode != 0 && mode != 1) return fail(LIZARD_ERR_INVALID_ARG, "mode=%d (0 standard, 1 reparameterized)", mode);
  if (dtype != LIZARD_BF16 || d != 128)
    return fail(LIZARD_ERR_UNSUPPORTED, "GLA forward built for bf16, d=128 (got %s, d=%d)",
                dtype == LIZARD_BF16 ? "bf16" : "fp32", d);
  if ((int64_t)B * Hq * L > (int64_t)1 << 40) return fail(LIZARD_ERR_INVALID_ARG, "problem too large");
  if (B == 0 || L == 0) return LIZARD_OK;
  if (!q || !k || !v || !log_gamma || !w_phi || !out) return fail(LIZARD_ERR_INVALID_ARG, "null tensor pointer");
  const void *ptrs[] = {q, k, v, log_gamma, w_phi, out};
  for (const void *ptr : ptrs)
    if (!aligned16(ptr)) return fail(LIZARD_ERR_INVALID_ARG, "tensor pointer %p not 16-byte aligned", ptr);
  lz::GlaParams p{};
  p.q = q; p.k = k; p.v = v; p.lg = log_gamma; p.w = w_phi; p.out = out;
  p.B = B; p.Hq = Hq; p.Hkv = Hkv; p.L = L; p.mode = mode;
  hipStream_t st = static_cast<hipStream_t>(stream);
  return finish(lz::launch_gla(p, st), st);
}

lizard_status lizard_attn_decode_noalloc(float *state, void *win_k, void *win_v, int32_t *pos, const void *q,
                                         const void *k, const void *v, const void *log_gamma, const void *w_phi_q,
                                         const void *w_phi_k, int64_t w_phi_head_stride, const void *t_k,
                                         const void *t_v, void *out, int N, int Hq, int Hkv, int d, int W, int M,
                                         float mix, float scale, lizard_dtype dtype, void *stream) {
  return decode_impl(state, win_k, win_v, pos, q, k, v, log_gamma, w_phi_q, w_phi_k, w_phi_head_stride, t_k, t_v,
                     out, N, Hq, Hkv, d, W, M, mix, scale, dtype, nullptr, 0, stream, false, true);
}

}  // extern "C"
