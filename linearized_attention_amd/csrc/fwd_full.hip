// Lizard attention forward, whole-head variant (bf16, d = 128, window W <= 129, one
// W_phi for queries and keys): one workgroup per (batch, query head, sequence
// segment) computes all 128 value columns, so the feature maps, the gate sums,
// the window logits and the intra-chunk scores are computed once per head
// instead of once per 64-column value block.  With grouped query heads the G
// workgroups of a key/value head each run its key side (on one XCD, so k, v and
// log gamma come from L2 after the first read).
//
// The arithmetic is that of the role-split kernel (fwd_split.hip), with the
// decay references of fwd.hip: a chunk whose log decay stays within FAST_SPAN
// for every feature refers all decays to the chunk start, other chunks use
// 16-token sub-chunk references.  What changes is the work split and the LDS
// layout:
//
//   key waves (4..7), sub-chunk I = wave - 4: stage the chunk's keys (in MFMA
//     fragment order, straight from the loads) and log gamma^T; gate prefix
//     sums and the choice of decay references; phi_k and the decayed keys; the
//     decay of phi_q in LDS; the state update for feature rows 32I..32I+31 of S
//     (fp32 registers, all 128 value columns) and the bf16 copy of S^T that the
//     query waves read.
//   query waves (0..3), sub-chunk I = wave: stage v^T; phi_q (while the key
//     waves stage); the window; the intra- and inter-chunk products, the merge
//     and the stores for rows 16I..16I+15 and all 128 value columns.
//
// Only the current chunk's keys and values are in LDS (a second chunk would not
// fit next to W_phi^T and the state copy).  The window of a query row is split in
// groups combined by an online softmax: the meta tokens and the previous chunk's
// keys (group X, computed at the top of the chunk while the previous chunk is
// still in LDS), and the current chunk's keys (group Y).  A window of more than
// 65 keys also reaches into the chunk two back (group Z): that part is computed
// at the top of the previous chunk, when the chunk two back is the one in LDS,
// for the next chunk's queries, and carried in registers as a partial softmax.
//
// Operand layouts: within every 32-element group along a contraction, element
// e = 16h + 4q + i is stored at position 8q + 4h + i ("interleaved").  An MFMA
// accumulator holds 4 consecutive rows of two 16-row tiles in each lane, and the
// interleaved layout turns the matching operand read into one 16-byte LDS read.
// It is used for the features of the decayed keys and of the state copy, and for
// the tokens of v^T.  Row strides are odd multiples of 32 bytes, which gfx950
// serves without bank conflicts for 16-byte fragment reads.
//
// A sequence may be split into segments (one workgroup each) to fill the chip.  A segment's start
// state comes from the state pass (fwd_full_state_kernel, three or more segments), or, for the
// second of two segments, from a backward walk over the chunks before it that its own workgroup
// runs first (walk_pipe); the first segment then takes a few chunks more (split_shift).
#include <type_traits>

#include "fwd_full.hpp"

namespace lz {

// Rows past the end of a sequence store their outputs (never read) here: one row, shared by all.
__device__ __align__(16) unsigned short g_fwd_sink[full::D];

// Exact diagonal-block scores for a sub-chunk whose log decay spans more than
// SPAN_MAX (e.g. gamma ~ 0): A[t][s] = mix sum_f phi_q[t][f] phi_k[s][f] e^{p_t[f] - p_s[f]}
// in fp32, p the log-gamma prefix inside the sub-chunk, phi recomputed from q and the
// keys.  Lane (t = lane % 16, g = lane / 16) returns s = 4g .. 4g+3.
// Wq (QPHI): the query side's W_phi [d][D or D/2] in global memory when it differs from the key
// side's W_phi^T in LDS; its W^T fragments are gathered element by element (a rare path).
template <bool HH, bool QPHI>
__device__ __forceinline__ f32x4 exact_diag_scores(const bf16 *sW, const bf16 *Wq, const bf16 *Kh, const bf16 *LGh,
                                                 const bf16 *Qh, int c0, int I, int L, float mix) {
  using namespace full;
  using T = bf16;
  const int lane = threadIdx.x & 63, r16 = lane & 15, g4 = lane >> 4;
  const Frag<T> tri_pre = tri_frag<T>(r16, g4, true);
  Frag<T> kfr[KS], qfr[KS];
  const int t0 = c0 + 16 * I + r16;
#pragma unroll
  for (int j = 0; j < KS; ++j) {
    kfr[j] = (t0 < L) ? load8(Kh + (size_t)t0 * D + 32 * j + 8 * g4) : frag_zero<T>();
    qfr[j] = (t0 < L) ? load8(Qh + (size_t)t0 * D + 32 * j + 8 * g4) : frag_zero<T>();
  }
  auto logits_ft = [&](const Frag<T>(&x)[KS], int ft) {
    f32x4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < KS; ++j) z = mma(load8(sW + (16 * ft + r16) * LDWW + 32 * j + 8 * g4), x[j], z);
    return z;
  };
  // query logits: W_phi^T in LDS, or (QPHI) W_phi_q^T[f][d] = W_q[d][f] gathered, with the
  // Hedgehog map's rows D/2 + f taking -W_q[d][f]
  auto logits_q = [&](int ft) {
    if constexpr (!QPHI) {
      return logits_ft(qfr, ft);
    } else {
      constexpr int FC = HH ? D / 2 : D;
      const int f = 16 * ft + r16;
      const bool neg = HH && f >= FC;
      const int col = neg ? f - FC : f;
      f32x4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < KS; ++j) {
        Frag<T> w;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const T x = Wq[(size_t)(32 * j + 8 * g4 + e) * FC + col];
          w.v[e] = neg ? -x : x;
        }
        z = mma(w, qfr[j], z);
      }
      return z;
    }
  };
  // loop over the feature tiles (kept rolled with the gathered query weights, whose unrolled
  // loads would not fit the registers)
  auto for_ft = [&](auto body) {
    if constexpr (QPHI) {
#pragma unroll 1
      for (int ft = 0; ft < NFT; ++ft) body(ft);
    } else {
      for (int ft = 0; ft < NFT; ++ft) body(ft);
    }
  };
  // softmax map: max and normaliser per row; the Hedgehog map is the plain exponential
  float mq = 0.f, mk = 0.f, iq = 1.f, ik = 1.f;
  if constexpr (!HH) {
    mq = NEG_BIG;
    mk = NEG_BIG;
    for_ft([&](int ft) {
      const f32x4 zq = logits_q(ft), zk = logits_ft(kfr, ft);
#pragma unroll
      for (int i = 0; i < 4; ++i) { mq = fmaxf(mq, zq[i]); mk = fmaxf(mk, zk[i]); }
    });
    mq = wave_max_cols(mq);
    mk = wave_max_cols(mk);
    float sq = 0.f, sk = 0.f;
    for_ft([&](int ft) {
      const f32x4 zq = logits_q(ft), zk = logits_ft(kfr, ft);
#pragma unroll
      for (int i = 0; i < 4; ++i) { sq += __expf(zq[i] - mq); sk += __expf(zk[i] - mk); }
    });
    iq = 1.f / wave_sum_cols(sq);
    ik = 1.f / wave_sum_cols(sk);
  }
  float part[16];
#pragma unroll
  for (int s2 = 0; s2 < 16; ++s2) part[s2] = 0.f;
  for_ft([&](int ft) {
    const f32x4 zq = logits_q(ft), zk = logits_ft(kfr, ft);
    float x[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int t = c0 + 16 * I + 8 * g4 + j;
      x[j] = (g4 < 2 && t < L) ? to_f(LGh[(size_t)t * D + 16 * ft + r16]) : 0.f;
    }
    const f32x4 px = mma(frag_from<T>(x), tri_pre, f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float phq = __expf(zq[i] - mq) * iq, phk = __expf(zk[i] - mk) * ik;
#pragma unroll
      for (int s2 = 0; s2 < 16; ++s2) {
        const float pk = __shfl(phk, 16 * g4 + s2);
        const float bs = __shfl(px[i], 16 * g4 + s2);
        part[s2] += (s2 <= r16) ? phq * pk * __expf(px[i] - bs) : 0.f;
      }
    }
  });
  f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s2 = 0; s2 < 16; ++s2) {
    const float v = wave_sum_cols(part[s2]);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if ((s2 >> 2) == g4 && (s2 & 3) == i) a[i] = v * mix;
  }
  return a;
}

// y_t += mix sum_{s<=t} A[t][s] v_s over the 16 rows of sub-chunk I of the chunk at c0, with A
// the exact diagonal-block scores: read-modify-write of rows this wave stored (same-wave
// ordering makes the stores visible to the loads).
template <bool HH, bool QPHI>
__device__ __forceinline__ void exact_diag_fixup(const bf16 *sW, const bf16 *Wq, const bf16 *Kh, const bf16 *Vh,
                                                 const bf16 *LGh, const bf16 *Qh, bf16 *Oh, int c0, int I, int L,
                                                 float mix) {
  using namespace full;
  using T = bf16;
  const int lane = threadIdx.x & 63, r16 = lane & 15, g4 = lane >> 4;
  const f32x4 a = exact_diag_scores<HH, QPHI>(sW, Wq, Kh, LGh, Qh, c0, I, L, mix);
  // lane (t, g) holds A[t][4g + i]; y_t[dv] += sum_s A[t][s] v_s[dv] for dv = 32g .. 32g+31
  float arow[16];
#pragma unroll
  for (int s2 = 0; s2 < 16; ++s2) {
    const float v = __shfl(a[s2 & 3], 16 * (s2 >> 2) + r16);
    arow[s2] = (s2 <= r16) ? v : 0.f;
  }
  const int t = c0 + 16 * I + r16;
  if (t >= L) return;
  T *O = Oh + (size_t)t * D + 32 * g4;
#pragma unroll 1
  for (int q8 = 0; q8 < 4; ++q8) {
    float y[8];
    load8f(O + 8 * q8, y);
#pragma unroll
    for (int s2 = 0; s2 < 16; ++s2) {
      const int sr = c0 + 16 * I + s2;
      if (sr < L) {
        float v8[8];
        load8f(Vh + (size_t)sr * D + 32 * g4 + 8 * q8, v8);
#pragma unroll
        for (int e = 0; e < 8; ++e) y[e] += arow[s2] * v8[e];
      }
    }
    store4<T>(O + 8 * q8, y[0], y[1], y[2], y[3]);
    store4<T>(O + 8 * q8 + 4, y[4], y[5], y[6], y[7]);
  }
}

// Feature logits of the wave's 16 rows against W_phi^T in LDS, with the W_phi^T fragments of
// feature tile ft + 1 loaded while tile ft is multiplied (the compiler otherwise waits for each
// fragment right before its products).
__device__ __forceinline__ void feature_logits_pipe(const bf16 *sW, const Frag<bf16> (&xa)[full::KS], int r16, int g4,
                                                    f32x4 (&za)[full::NFT]) {
  using namespace full;
  const bf16 *wrow = sW + r16 * LDWW + 8 * g4;
  Frag<bf16> w[2][KS];
#pragma unroll
  for (int j = 0; j < KS; ++j) w[0][j] = load8(wrow + 32 * j);
#pragma unroll
  for (int ft = 0; ft < NFT; ++ft) {
    if (ft + 1 < NFT) {
#pragma unroll
      for (int j = 0; j < KS; ++j) w[(ft + 1) & 1][j] = load8(wrow + 16 * (ft + 1) * LDWW + 32 * j);
    }
    f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < KS; ++j) a = mma(w[ft & 1][j], xa[j], a);
    za[ft] = a;
  }
}

// The state update's A operand, decayed keys^T: feature 32 I + 16 ft + r16 for the 8 tokens of
// lane group g4 in K-step ks (slots 0..3: tokens 32 ks + 4 g4 + j, slots 4..7: the same + 16), from
// sKt rows (tokens, interleaved features) by two transposed LDS reads (ds_read_b64_tr_b16): in a
// group of 16 lanes, lane m reads the 4 features 32 I + 16 ft + 4 (m % 4) .. + 3 (contiguous in the
// interleaved order) of token 32 ks + 4 g4 + m / 4, and lane i receives feature i of the 4 tokens
// that lanes 4 j + i / 4 read (j = 0..3).
__device__ __forceinline__ void keysT_tr(const bf16 *sKt, int I, int ft, int ks, int r16, int g4, float (&x)[8]) {
  using namespace full;
  typedef short v4s __attribute__((ext_vector_type(4)));
  const bf16 *src = sKt + (32 * ks + 4 * g4 + (r16 >> 2)) * LDW + 32 * I + 8 * (r16 & 3) + 4 * ft;
  const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s *)(src));
  const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s *)(src + 16 * LDW));
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    x[j] = __uint_as_float((uint32_t)(uint16_t)lo[j] << 16);
    x[4 + j] = __uint_as_float((uint32_t)(uint16_t)hi[j] << 16);
  }
}

// Chunks the first of two segments takes beyond the even split at chunk b, so that both end
// together.  The second segment first walks back from its start until every feature has decayed
// by e^{-skip_log}, about n = skip_log / r chunks for the slowest feature's log decay r per
// chunk (at most b).  Measured on MI355X, the walk with its set-up costs about 6 + 3.2 n us and
// a chunk of the main loop 6.5 us, so the first segment takes (6 + 3.2 n) / 13 chunks more (fitted
// over gates whose walks last 1, 7, 14 and all chunks).  r comes from the
// last four chunks before b: wave w < 4 sums chunk b - 1 - w per feature into part[w][D]
// (shared memory), and after the barrier that follows every wave reads the four rows and
// reduces them the same way.  Every workgroup of the head runs this on the same data with the
// same code, so the two segments agree without communicating.
__device__ __forceinline__ void split_shift_part(const bf16 *LGh, int b, int wv, int lane, float *part) {
  using namespace full;
  const int c = b - 1 - wv;
  if (wv >= 4 || c < 0) return;
  const int fg = lane & 15, tg = lane >> 4;  // features 8 fg .. 8 fg + 7 of tokens tg + 4 i
  float a[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll 1
  for (int i0 = 0; i0 < 16; i0 += 4) {  // four rows in flight at a time (few registers here)
    Frag<bf16> x[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = load8(LGh + (size_t)(c * CH + tg + 4 * (i0 + i)) * D + 8 * fg);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < 8; ++e) a[e] += to_f(x[i].v[e]);
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float t = wave_sum_cols(a[e]);
    if (tg == 0) part[wv * D + 8 * fg + e] = t;
  }
}
template <bool HH>
__device__ __forceinline__ int split_shift(const float *part, int b, int lane) {
  using namespace full;
  const int nc = b < 4 ? b : 4;
  float r = 1.0e30f;  // the slowest feature's log decay per chunk (log gamma <= 0)
#pragma unroll
  for (int q = 0; q < D / 64; ++q) {
    float a = 0.f;
    for (int w = 0; w < nc; ++w) a += part[w * D + lane + 64 * q];
    r = fminf(r, -a);
  }
  r = -wave_max_all(-r) / (float)nc;
  const float n = fminf(skip_log<HH>() / fmaxf(r, 1.0e-6f), (float)b);
  return (int)((6.f + 3.2f * n) / 13.f + 0.5f);
}

// The backward walk of the segment state pass (see fwd_full_state_kernel below).
// LDS of one backward walk: W_phi^T (staged and visible before the walk starts, or staged by
// the stage_w callback the walk runs after its first loads), v^T, the log gamma^T / decayed key
// rows, the prefix table, the suffix sums [2][D] and four vote words.
struct WalkLds {
  const bf16 *sW;
  bf16 *sVt, *sKt;
  float *sTot, *sSuf;
  int *sVote;
};

// Backward walk over the chunks [b0, b1) of one head (b1 - b0 full chunks), piece pp of sss:
// adds the chunks c with (b1 - 1 - c) % sss == pp, decayed to b1, to S (which it zeroes first).
// WORKER threads wt = 0..255 are four waves (sub-chunk I = wt / 64) that do the work; the other
// threads of the workgroup (WORKER = false) only take part in its barriers.  Returns whether the
// walk stopped before b0; the workers wt < D hold in suf the log-gate sum of the chunks walked.
// Ends with a barrier: the LDS it used is free for the caller.
template <bool HH, bool WORKER, typename StageW>
__device__ __forceinline__ bool walk_back(const WalkLds &lds, const bf16 *Kh, const bf16 *Vh, const bf16 *LGh,
                                          int b0, int b1, int pp, int sss, int wt, f32x4 (&S)[full::FTW][full::NDT],
                                          float &suf, StageW stage_w) {
  using namespace full;
  using T = bf16;
  const bf16 *sW = lds.sW;
  T *sVt = lds.sVt, *sKt = lds.sKt, *sLgT = lds.sKt;
  float *sTot = lds.sTot, *sSuf = lds.sSuf;
  int *sVote = lds.sVote;
  const int lane = wt & 63, I = wt >> 6;
  const int r16 = lane & 15, g4 = lane >> 4;
  auto own = [&](int c) { return (b1 - 1 - c) % sss == pp; };

  auto load_k = [&](Frag<T> (&kf)[KS], int c0) {
    // lane offsets rebuilt here from a lane id the compiler cannot hoist (a per-lane row
    // pointer kept across the loop was spilled, and its reload waits for the loads in flight)
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const T *src = Kh + (size_t)(c0 + 16 * I + (ln & 15)) * D;
#pragma unroll
    for (int j = 0; j < KS; ++j) kf[j] = load8(src + 32 * j + 8 * (ln >> 4));
  };
  // values and log gamma, token pairs tp = wt % 32, 8-column groups wt / 32 + 8 gsel (4 per thread)
  // (offsets from an opaque copy of wt, for the reason given in load_k)
  auto load_pairs = [&](Frag<T> (&f)[2][2], const T *base, int c0) {
    int w = wt;
    asm volatile("" : "+v"(w));
    const int tp = w & 31;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int gsel = 0; gsel < 2; ++gsel) f[gsel][h] = load8(base + (size_t)(c0 + 2 * tp + h) * D + 8 * ((w >> 5) + 8 * gsel));
  };
  Frag<T> kf[KS], vf[2][2], lf[2][2];
  int c = b1 - 1;
  if constexpr (WORKER) {
    load_pairs(lf, LGh, c * CH);
    load_k(kf, (c - pp) * CH);  // this piece's first chunk (sss <= b1 - b0)
    load_pairs(vf, Vh, (c - pp) * CH);
  }
  stage_w();  // overlaps the first loads
#pragma unroll
  for (int ft = 0; ft < FTW; ++ft)
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) S[ft][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  suf = 0.f;  // thread wt < D: log-gate sum of feature wt over the chunks walked so far
  if (WORKER && wt < D) sSuf[wt] = 0.f;
  const Frag<T> tri_c0 = tri64_frag<T>(r16, g4, I, 0), tri_c1 = tri64_frag<T>(r16, g4, I, 1);
  bool stopped = false;
  __syncthreads();

  for (int par = 0;; par ^= 1, --c) {
    const bool mine = own(c);
    float ko[NFT][4];
    if (WORKER && mine) {
      f32x4 z[NFT];
      feature_logits_pipe(sW, kf, r16, g4, z);
      feature_map_rows<HH>(z, ko);
    }
    if constexpr (WORKER) {
      const int tp = wt & 31;
      const int vpos = (2 * tp & 32) | ipos(2 * tp & 31);
#pragma unroll
      for (int gsel = 0; gsel < 2; ++gsel) {
        const int gq = (wt >> 5) + 8 * gsel;
        if (mine) store_pairT<T, LDV>(vf[gsel][0], vf[gsel][1], sVt + (8 * gq) * LDV + vpos);
        store_pairT<T, LDV>(lf[gsel][0], lf[gsel][1], sLgT + (8 * gq) * LDV + 2 * tp);
      }
      // in flight from here: the log gates of the next chunk back, the keys and values of this
      // piece's next chunk (sss chunks back: the walk's cheap chunks in between hide the loads)
      if (c > b0) load_pairs(lf, LGh, (c - 1) * CH);
      if (mine && c - sss >= b0) {
        load_k(kf, (c - sss) * CH);
        load_pairs(vf, Vh, (c - sss) * CH);
      }
    }
    __syncthreads();
    float pc[NFT][4];
    if constexpr (WORKER) {
#pragma unroll
      for (int ft = 0; ft < NFT; ++ft) {
        f32x4 cc = mma(load8(sLgT + (16 * ft + r16) * LDV + 8 * g4), tri_c0, f32x4{0.f, 0.f, 0.f, 0.f});
        cc = mma(load8(sLgT + (16 * ft + r16) * LDV + 32 + 8 * g4), tri_c1, cc);
#pragma unroll
        for (int i = 0; i < 4; ++i) pc[ft][i] = cc[i];
      }
      if (r16 == 15) {
#pragma unroll
        for (int ft = 0; ft < NFT; ++ft)
          *reinterpret_cast<f32x4 *>(sTot + I * D + 16 * ft + 4 * g4) = f32x4{pc[ft][0], pc[ft][1], pc[ft][2], pc[ft][3]};
      }
    }
    __syncthreads();
    bool mild = false;
    if constexpr (WORKER) {
      // suffix through this chunk, for the next chunk back; stop once every feature is below
      if (wt < D) {
        suf += sTot[3 * D + wt];
        sSuf[(par ^ 1) * D + wt] = suf;
        const bool below = __all(suf < -skip_log<HH>());
        if (lane == 0) sVote[I] = below;
      }
      mild = mine && chunk_is_mild_c<D>(sTot, lane);
      if (mine) {
        // decayed keys: mild chunk e^{-p_t} (chunk-start reference), else e^{C_I - p_t}
        if (mild) {
#pragma unroll
          for (int ft = 0; ft < NFT; ++ft)
#pragma unroll
            for (int i = 0; i < 4; ++i) ko[ft][i] *= exp2_fast(-pc[ft][i] * LOG2E);
        } else {
#pragma unroll
          for (int ft = 0; ft < NFT; ++ft) {
            const f32x4 t = *reinterpret_cast<const f32x4 *>(sTot + I * D + 16 * ft + 4 * g4);
#pragma unroll
            for (int i = 0; i < 4; ++i) ko[ft][i] *= __expf(t[i] - pc[ft][i]);
          }
        }
#pragma unroll
        for (int ft = 0; ft < NFT; ++ft) {
          const int fpos = 32 * (ft >> 1) + 8 * g4 + 4 * (ft & 1);
          store4<T>(sKt + (16 * I + r16) * LDW + fpos, ko[ft][0], ko[ft][1], ko[ft][2], ko[ft][3]);
        }
      }
    }
    __syncthreads();
    const bool stop = sVote[0] && sVote[1];
    if (WORKER && mine) {
      // S += sum_t k~_t e^{s + ...} v_t^T: key factors e^{s + C_3} (mild) or e^{s + C_3 - C_J}
      // for sub-chunk J, s = the suffix after this chunk (feature of the key row)
      Frag<T> ka[FTW][2];
#pragma unroll
      for (int ft = 0; ft < FTW; ++ft) {
        const int fr = 16 * (2 * I + ft);
        float fac[2][2];
        const float c3s = sTot[3 * D + fr + r16] + sSuf[par * D + fr + r16];
#pragma unroll
        for (int J = 0; J < 4; ++J) fac[J >> 1][J & 1] = __expf(mild ? c3s : c3s - sTot[J * D + fr + r16]);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          float x[8];
          keysT_tr(sKt, I, ft, ks, r16, g4, x);
#pragma unroll
          for (int jj = 0; jj < 8; ++jj) x[jj] *= fac[ks][jj >> 2];
          ka[ft][ks] = frag_from<T>(x);
        }
      }
      // each v^T fragment serves both feature tiles; the next value tile's are loaded ahead
      const T *vrow = sVt + r16 * LDV + 8 * g4;
      Frag<T> vb[2][2];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) vb[0][ks] = load8(vrow + 32 * ks);
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        if (dt + 1 < NDT) {
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) vb[(dt + 1) & 1][ks] = load8(vrow + 16 * (dt + 1) * LDV + 32 * ks);
        }
#pragma unroll
        for (int ft = 0; ft < FTW; ++ft)
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) S[ft][dt] = mma(ka[ft][ks], vb[dt & 1][ks], S[ft][dt]);
      }
    }
    if (stop || c == b0) {
      stopped = stop && c > b0;
      break;
    }
    if (mine) __syncthreads();  // keys and values read before the next chunk is staged (the
                                // other chunks' LDS reads all came before the last barrier)
  }
  __syncthreads();
  return stopped;
}

// The same walk over [0, b1) for the workgroup of a self-started segment, split between its two
// roles and pipelined by one chunk: the query waves (Q, wt = tid) stage chunk c, take its feature
// map, prefix sums, suffix and decayed keys, while the key waves (K, wt = tid - 256) add chunk
// c + 1, whose results sit in the other of two LDS buffers, to S.  Three barriers per chunk; K
// adds the last chunk after the loop.  S as in walk_back (in the key waves only).
struct PipeLds {
  const bf16 *sW;
  bf16 *sVt0, *sVt1, *sKt0, *sKt1;  // the two buffers (named, not indexed: an indexed pointer
  float *sTot0, *sTot1, *sSuf;      // array would live in scratch memory)
  int *sVote;
  __device__ bf16 *vt(int b) const { return b ? sVt1 : sVt0; }
  __device__ bf16 *kt(int b) const { return b ? sKt1 : sKt0; }
  __device__ float *tot(int b) const { return b ? sTot1 : sTot0; }
};
template <bool HH, bool QROLE>
__device__ __forceinline__ void walk_pipe(const PipeLds &lds, const bf16 *Kh, const bf16 *Vh, const bf16 *LGh,
                                          int b1, int wt, f32x4 (&S)[full::FTW][full::NDT]) {
  using namespace full;
  using T = bf16;
  const int lane = wt & 63, I = wt >> 6;
  const int r16 = lane & 15, g4 = lane >> 4;
  auto load_k = [&](Frag<T> (&kf)[KS], int c0) {
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const T *src = Kh + (size_t)(c0 + 16 * I + (ln & 15)) * D;
#pragma unroll
    for (int j = 0; j < KS; ++j) kf[j] = load8(src + 32 * j + 8 * (ln >> 4));
  };
  auto load_pairs = [&](Frag<T> (&f)[2][2], const T *base, int c0) {
    int w = wt;
    asm volatile("" : "+v"(w));
    const int tp = w & 31;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int gsel = 0; gsel < 2; ++gsel) f[gsel][h] = load8(base + (size_t)(c0 + 2 * tp + h) * D + 8 * ((w >> 5) + 8 * gsel));
  };
  // K: S += chunk c's decayed keys^T (buffer bj) times its v^T, keys scaled by e^{s_c + C_3 (- C_J)}
  auto add_chunk = [&](int bj) {
    const T *sKt = lds.kt(bj), *sVt = lds.vt(bj);
    const float *sTot = lds.tot(bj), *suf_c = lds.sSuf + bj * D;
    const bool mild = chunk_is_mild_c<D>(sTot, lane);
    Frag<T> ka[FTW][2];
#pragma unroll
    for (int ft = 0; ft < FTW; ++ft) {
      const int fr = 16 * (2 * I + ft);
      float fac[2][2];
      const float c3s = sTot[3 * D + fr + r16] + suf_c[fr + r16];
#pragma unroll
      for (int J = 0; J < 4; ++J) fac[J >> 1][J & 1] = __expf(mild ? c3s : c3s - sTot[J * D + fr + r16]);
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        float x[8];
        keysT_tr(sKt, I, ft, ks, r16, g4, x);
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) x[jj] *= fac[ks][jj >> 2];
        ka[ft][ks] = frag_from<T>(x);
      }
    }
    const T *vrow = sVt + r16 * LDV + 8 * g4;
    Frag<T> vb[2][2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) vb[0][ks] = load8(vrow + 32 * ks);
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      if (dt + 1 < NDT) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) vb[(dt + 1) & 1][ks] = load8(vrow + 16 * (dt + 1) * LDV + 32 * ks);
      }
#pragma unroll
      for (int ft = 0; ft < FTW; ++ft)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) S[ft][dt] = mma(ka[ft][ks], vb[dt & 1][ks], S[ft][dt]);
    }
  };

  Frag<T> kf[KS], vf[2][2], lf[2][2];
  float suf = 0.f;  // Q, wt < D: log-gate sum of feature wt over the chunks walked so far
  int c = b1 - 1;
  if constexpr (QROLE) {
    load_pairs(lf, LGh, c * CH);
    load_k(kf, c * CH);
    load_pairs(vf, Vh, c * CH);
    if (wt < D) lds.sSuf[wt] = 0.f;  // s of the last chunk (buffer 0)
  } else {
#pragma unroll
    for (int ft = 0; ft < FTW; ++ft)
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) S[ft][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const Frag<T> tri_c0 = tri64_frag<T>(r16, g4, I, 0), tri_c1 = tri64_frag<T>(r16, g4, I, 1);
  __syncthreads();
  for (int j = 0;; ++j, --c) {
    const int bj = j & 1;
    float ko[NFT][4];
    if constexpr (QROLE) {
      T *sKt = lds.kt(bj), *sVt = lds.vt(bj);
      {
        f32x4 z[NFT];
        feature_logits_pipe(lds.sW, kf, r16, g4, z);
        feature_map_rows<HH>(z, ko);
      }
      const int tp = wt & 31;
      const int vpos = (2 * tp & 32) | ipos(2 * tp & 31);
#pragma unroll
      for (int gsel = 0; gsel < 2; ++gsel) {
        const int gq = (wt >> 5) + 8 * gsel;
        store_pairT<T, LDV>(vf[gsel][0], vf[gsel][1], sVt + (8 * gq) * LDV + vpos);
        store_pairT<T, LDV>(lf[gsel][0], lf[gsel][1], sKt + (8 * gq) * LDV + 2 * tp);  // log gamma^T
      }
      if (c > 0) {
        load_pairs(lf, LGh, (c - 1) * CH);
        load_k(kf, (c - 1) * CH);
        load_pairs(vf, Vh, (c - 1) * CH);
      }
    } else {
      if (j > 0) add_chunk(bj ^ 1);  // the previous (later) chunk
    }
    __syncthreads();  // W1: log gamma^T and v^T of chunk c staged
    float pc[NFT][4];
    if constexpr (QROLE) {
      const T *sLgT = lds.kt(bj);
      float *sTot = lds.tot(bj);
#pragma unroll
      for (int ft = 0; ft < NFT; ++ft) {
        f32x4 cc = mma(load8(sLgT + (16 * ft + r16) * LDV + 8 * g4), tri_c0, f32x4{0.f, 0.f, 0.f, 0.f});
        cc = mma(load8(sLgT + (16 * ft + r16) * LDV + 32 + 8 * g4), tri_c1, cc);
#pragma unroll
        for (int i = 0; i < 4; ++i) pc[ft][i] = cc[i];
      }
      if (r16 == 15) {
#pragma unroll
        for (int ft = 0; ft < NFT; ++ft)
          *reinterpret_cast<f32x4 *>(sTot + I * D + 16 * ft + 4 * g4) = f32x4{pc[ft][0], pc[ft][1], pc[ft][2], pc[ft][3]};
      }
    }
    __syncthreads();  // W2: prefix ends of chunk c visible
    if constexpr (QROLE) {
      const float *sTot = lds.tot(bj);
      T *sKt = lds.kt(bj);
      if (wt < D) {  // suffix through chunk c: s of the next chunk back (other buffer's slot)
        suf += sTot[3 * D + wt];
        lds.sSuf[(bj ^ 1) * D + wt] = suf;
        const bool below = __all(suf < -skip_log<HH>());
        if (lane == 0) lds.sVote[I] = below;
      }
      if (chunk_is_mild_c<D>(sTot, lane)) {
#pragma unroll
        for (int ft = 0; ft < NFT; ++ft)
#pragma unroll
          for (int i = 0; i < 4; ++i) ko[ft][i] *= exp2_fast(-pc[ft][i] * LOG2E);
      } else {
#pragma unroll
        for (int ft = 0; ft < NFT; ++ft) {
          const f32x4 t = *reinterpret_cast<const f32x4 *>(sTot + I * D + 16 * ft + 4 * g4);
#pragma unroll
          for (int i = 0; i < 4; ++i) ko[ft][i] *= __expf(t[i] - pc[ft][i]);
        }
      }
#pragma unroll
      for (int ft = 0; ft < NFT; ++ft) {
        const int fpos = 32 * (ft >> 1) + 8 * g4 + 4 * (ft & 1);
        store4<T>(sKt + (16 * I + r16) * LDW + fpos, ko[ft][0], ko[ft][1], ko[ft][2], ko[ft][3]);
      }
    }
    __syncthreads();  // W3: decayed keys, suffix and votes of chunk c visible
    const bool stop = lds.sVote[0] && lds.sVote[1];
    if (stop || c == 0) {
      if constexpr (!QROLE) add_chunk(bj);
      break;
    }
  }
  __syncthreads();
}

// ZW: windows of 66..129 keys, which reach into the chunk two back (window group Z).
// QPHI: the query side's W_phi differs from the key side's (separate or per-head matrices): W_phi^T
// in LDS is the key side's (of this key/value head), and the query waves read their operands from
// the copy fwd_full_wq_frag_kernel wrote in fragment order (with ZW: the query feature maps that
// fwd_full_phiq_kernel wrote into the output rows).
template <bool ZW, bool HH, bool QPHI>
__global__ __launch_bounds__(512, 1) void fwd_full_kernel(FwdParams p) {
  using namespace full;
  using T = bf16;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  T *sW = reinterpret_cast<T *>(smem + OFF_W);
  T *sK = reinterpret_cast<T *>(smem + OFF_K);
  T *sVt = reinterpret_cast<T *>(smem + OFF_VT);
  T *sKt = reinterpret_cast<T *>(smem + OFF_KT);
  T *sLgT = sKt;  // log gamma^T, dead before the decayed keys are written
  T *sSb = reinterpret_cast<T *>(smem + OFF_SB);
  T *sQ = reinterpret_cast<T *>(smem + OFF_Q);
  float *sTot = reinterpret_cast<float *>(smem + OFF_TAB);  // C_J: prefix from the chunk start to the end of J
  T *sTk = reinterpret_cast<T *>(smem + OFF_TK);
  T *sTvT = reinterpret_cast<T *>(smem + OFF_TV);
  uint32_t *sFlag = reinterpret_cast<uint32_t *>(smem + OFF_FLAG);
  // A self-started segment walks the chunks before it (walk_pipe) in two LDS buffers: the
  // regions of the chunk loop, and copies of them in the S^T-copy and decayed-query rows (unused
  // until the loop), where the suffix sums, votes and the split estimate follow.
  constexpr int SC_VT = 0, SC_KT = SC_VT + D * LDV * 2, SC_TAB = SC_KT + SZ_KT;
  constexpr int SC_SUF = SC_TAB + 4 * D * 4, SC_VOTE = SC_SUF + 2 * D * 4, SC_PART = SC_VOTE + 64;
  static_assert(OFF_Q == OFF_SB + D * LDW * 2, "scratch spans the S^T copy and the decayed queries");
  static_assert(SC_PART + 4 * D * 4 <= D * LDW * 2 + CH * LDQ * 2, "walk scratch exceeds its rows");
  char *scr = smem + OFF_SB;
  const PipeLds plds{sW, sVt, reinterpret_cast<T *>(scr + SC_VT), sKt, reinterpret_cast<T *>(scr + SC_KT),
                     sTot, reinterpret_cast<float *>(scr + SC_TAB), reinterpret_cast<float *>(scr + SC_SUF),
                     reinterpret_cast<int *>(scr + SC_VOTE)};

  // lane id from mbcnt and the wave index as a scalar: both can be rebuilt anywhere, so the
  // register allocator recomputes lane-derived values instead of keeping (or spilling) them
  const int tid = threadIdx.x, lane = __lane_id();
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r16 = lane & 15, g4 = lane >> 4;
  const bool key_wave = wv >= 4;
  const int I = wv & 3;

  // block -> (batch, key/value head, segment) group and query head g of the group; the G
  // blocks of a group are 8 apart, so they run on one XCD and share its L2 for k, v, log gamma
  const int G = p.G;
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int grp = (slot / G) * 8 + xcd, g = slot % G;
  if (grp >= p.ngroups) return;
  const int seg = grp % p.nseg;
  const int bh = grp / p.nseg;
  const int b = bh / p.Hkv, kvh = bh % p.Hkv;
  const int hq = kvh * G + g;
  const int L = p.L;

  const size_t kv_off = ((size_t)b * p.Hkv + kvh) * (size_t)L * D;
  const T *Kh = reinterpret_cast<const T *>(p.k) + kv_off;
  const T *Vh = reinterpret_cast<const T *>(p.v) + kv_off;
  const T *LGh = reinterpret_cast<const T *>(p.lg) + kv_off;
  const T *Qh = reinterpret_cast<const T *>(p.q) + ((size_t)b * p.Hq + hq) * (size_t)L * D;
  T *Oh = reinterpret_cast<T *>(p.out) + ((size_t)b * p.Hq + hq) * (size_t)L * D;
  const size_t hist_off = ((size_t)b * p.Hkv + kvh) * (size_t)p.hist_rows * D;
  const T *Hk = reinterpret_cast<const T *>(p.hist_k) + hist_off;
  const T *Hv = reinterpret_cast<const T *>(p.hist_v) + hist_off;
  const int hist_avail = p.pos ? min(p.pos[b], p.W - 1) : 0;  // history tokens the window may see
  // key / value row x of the sequence (x < 0: history), zero outside [-hist_avail.., L)
  auto krow = [&](int x) -> const T * { return x >= 0 ? Kh + (size_t)x * D : Hk + (ptrdiff_t)(p.hist_rows + x) * D; };
  auto vrow = [&](int x) -> const T * { return x >= 0 ? Vh + (size_t)x * D : Hv + (ptrdiff_t)(p.hist_rows + x) * D; };
  auto row_ok = [&](int x) { return x < L && (x >= 0 || (p.hist_rows > 0 && x >= -p.hist_rows)); };

  // p.split > 0: two segments, the second starting at chunk p.split + shift and walking the
  // chunks before it for its start state (no state pass).  The shift is computed here from the
  // gates, by every workgroup of the head alike, so both segments agree on it.
  int bsplit = 0;
  if (p.split) {
    float *part = reinterpret_cast<float *>(scr + SC_PART);
    if (p.split_shift < 0) split_shift_part(LGh, p.split, wv, lane, part);
    __syncthreads();
    const int sh = p.split_shift >= 0 ? p.split_shift : split_shift<HH>(part, p.split, lane);
    bsplit = p.split + min(sh, p.split_max);
  }
  const int c_begin = p.split ? (seg ? bsplit : 0) : seg * p.cps;
  const int c_end = p.split ? (seg ? p.nchunks : bsplit) : min(p.nchunks, c_begin + p.cps);
  const bool self_start = p.split && seg == 1;

  // ---- staging helpers
  // keys of rows c0 + 16I .. +15 in fragment order (lane (r, q): row r, d = 32j + 8q .. +7)
  auto load_kfrag = [&](Frag<T> (&kf)[KS], int c0) {
    const int x = c0 + 16 * I + r16;
    const bool ok = row_ok(x);
    const T *src = krow(ok ? x : 0);
#pragma unroll
    for (int j = 0; j < KS; ++j) kf[j] = ok ? load8(src + 32 * j + 8 * g4) : frag_zero<T>();
  };
  auto store_kfrag = [&](const Frag<T> (&kf)[KS]) {
#pragma unroll
    for (int j = 0; j < KS; ++j) *reinterpret_cast<bf16x8 *>(sK + (16 * I + r16) * LDW + 32 * j + 8 * g4) = kf[j].v;
  };
  // values: thread t (of 256) takes token pairs tp = t % 32 and 8-column groups t / 32, t / 32 + 8;
  // each half-wave writes one column group, so the transposed 4-byte stores spread over the banks
  auto load_vpairs = [&](Frag<T> (&vf)[2][2], int c0, int t) {
    const int tp = t & 31;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int x = c0 + 2 * tp + h;
      const bool ok = row_ok(x);
      const T *src = vrow(ok ? x : 0);
#pragma unroll
      for (int gsel = 0; gsel < 2; ++gsel) {
        const int gq = (t >> 5) + 8 * gsel;
        vf[gsel][h] = ok ? load8(src + 8 * gq) : frag_zero<T>();
      }
    }
  };
  auto store_vpairs = [&](const Frag<T> (&vf)[2][2], int t) {
    const int tp = t & 31;
    const int pos = (2 * tp & 32) | ipos(2 * tp & 31);  // token pairs stay adjacent
#pragma unroll
    for (int gsel = 0; gsel < 2; ++gsel) {
      const int gq = (t >> 5) + 8 * gsel;
      store_pairT<T, LDV>(vf[gsel][0], vf[gsel][1], sVt + (8 * gq) * LDV + pos);
    }
  };
  // log gamma^T [f][s] (natural token order): token pairs tp = t % 32, 8-feature groups t / 32, + 8
  auto load_lgpairs = [&](Frag<T> (&lf)[2][2], int c0, int t) {
    const int tp = t & 31;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int x = c0 + 2 * tp + h;
      const bool ok = x < L;
#pragma unroll
      for (int gsel = 0; gsel < 2; ++gsel) {
        const int fq = (t >> 5) + 8 * gsel;
        lf[gsel][h] = ok ? load8(LGh + (size_t)x * D + 8 * fq) : frag_zero<T>();
      }
    }
  };
  auto store_lgpairs = [&](const Frag<T> (&lf)[2][2], int t) {
    const int tp = t & 31;
#pragma unroll
    for (int gsel = 0; gsel < 2; ++gsel) {
      const int fq = (t >> 5) + 8 * gsel;
      store_pairT<T, LDV>(lf[gsel][0], lf[gsel][1], sLgT + (8 * fq) * LDV + 2 * tp);
    }
  };

  // queries of rows c0 + 16I .. +15 in fragment order
  auto load_q = [&](Frag<T> (&f)[KS], int c0) {
    const int t = c0 + 16 * I + r16;
    const unsigned off = (unsigned)(t * D + 8 * g4);
#pragma unroll
    for (int j = 0; j < KS; ++j) f[j] = (t < L) ? load8(Qh + off + 32 * j) : frag_zero<T>();
  };
  // Loads inside the chunk loop (rows >= 0): a uniform base and a 32-bit per-lane offset
  // recomputed from the lane id each time, so no 64-bit lane addresses are held (or spilled)
  // across the loop; a reloaded spill would also wait for every load in flight.
  // (a chunk that lies inside the sequence, every chunk but a ragged last one, skips the
  // per-lane bounds checks and the exec-mask branches they cost)
  auto kfrag_in = [&](Frag<T> (&kf)[KS], int c0, int ln) {
    const int x = c0 + 16 * I + (ln & 15);
    const unsigned off = (unsigned)(x * D + 8 * (ln >> 4));
    if (c0 + CH <= L) {
#pragma unroll
      for (int j = 0; j < KS; ++j) kf[j] = load8(Kh + off + 32 * j);
    } else {
#pragma unroll
      for (int j = 0; j < KS; ++j) kf[j] = (x < L) ? load8(Kh + off + 32 * j) : frag_zero<T>();
    }
  };
  auto q_in = [&](Frag<T> (&f)[KS], int c0, int ln) {
    const int t = c0 + 16 * I + (ln & 15);
    const unsigned off = (unsigned)(t * D + 8 * (ln >> 4));
    if (c0 + CH <= L) {
#pragma unroll
      for (int j = 0; j < KS; ++j) f[j] = load8(Qh + off + 32 * j);
    } else {
#pragma unroll
      for (int j = 0; j < KS; ++j) f[j] = (t < L) ? load8(Qh + off + 32 * j) : frag_zero<T>();
    }
  };
  // token pairs (2 tp, 2 tp + 1) x 8-column groups t / 32 and t / 32 + 8 of a [L][D] tensor
  auto pairs_in = [&](Frag<T> (&f)[2][2], const T *base, int c0, int t) {
    const int tp = t & 31;
    const bool inside = c0 + CH <= L;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int x = c0 + 2 * tp + h;
#pragma unroll
      for (int gsel = 0; gsel < 2; ++gsel) {
        const unsigned off = (unsigned)(x * D + 8 * ((t >> 5) + 8 * gsel));
        f[gsel][h] = (inside || x < L) ? load8(base + off) : frag_zero<T>();
      }
    }
  };
  const float mix = p.mix, log2_mix = __log2f(p.mix);

  // ---- prologue: weights, meta tokens, the chunk before the first one
  {
    const T *Wk = reinterpret_cast<const T *>(p.wk) + (size_t)kvh * p.w_stride;
    load_wT_pairs<512, HH>(sW, Wk, tid);
    const T *Tv = reinterpret_cast<const T *>(p.tv);
    const T *Tk = reinterpret_cast<const T *>(p.tk);
    for (int idx = tid; idx < D * 16; idx += 512) {
      const int dv = idx / 16, m = idx % 16;
      sTvT[dv * LDM + m] = (m < p.M) ? Tv[((size_t)kvh * p.M + m) * D + dv] : from_f<T>(0.f);
    }
    for (int idx = tid; idx < 16 * D; idx += 512) {
      const int m = idx / D, e = idx % D;
      sTk[m * LDW + e] = (m < p.M) ? Tk[((size_t)kvh * p.M + m) * D + e] : from_f<T>(0.f);
    }
    for (int idx = tid; idx < 4 * FLAG_WORDS; idx += 512) sFlag[idx] = 0u;
  }
  // The chunks before the first one (history or the end of the previous segment; zeros if
  // none) are staged by the roles below: keys by the key waves, values by the query waves.

  if (key_wave) {
    // ======================================================= key waves
    const int kt = tid - 256;
    // S rows owned: feature tiles 2I, 2I+1; S[ft][dt][i] = S[16(2I+ft) + 4g4 + i][16dt + r16]
    f32x4 S[FTW][NDT];
    if (self_start) walk_pipe<HH, false>(plds, Kh, Vh, LGh, c_begin, kt, S);  // the state at the split
    {
      Frag<T> kf[KS];
      if constexpr (ZW) {
        load_kfrag(kf, (c_begin - 2) * CH);
        store_kfrag(kf);
        __syncthreads();  // Z0: the chunk two back staged
        __syncthreads();  // Z1: the query waves' group Z of the first chunk done
      }
      load_kfrag(kf, (c_begin - 1) * CH);
      store_kfrag(kf);
    }
    if (!self_start) {
#pragma unroll
    for (int ft = 0; ft < FTW; ++ft)
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) S[ft][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (p.state_in) {
      const float *Si = p.state_in + ((size_t)b * p.Hkv + kvh) * D * D;
#pragma unroll
      for (int ft = 0; ft < FTW; ++ft)
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
          for (int i = 0; i < 4; ++i) S[ft][dt][i] = Si[(size_t)(16 * (2 * I + ft) + 4 * g4 + i) * D + 16 * dt + r16];
    }
    // segment start: S = e^{D_j} S + E_j over the earlier segments (end states and log-gate
    // sums of fwd_full_state_kernel, E in this kernel's fragment order)
    const int nstate = (p.nseg - 1) * p.sss;  // state-pass pieces per head (p.sss per segment)
    for (int j = 0; j < seg * p.sss; ++j) {
      const size_t sj = (size_t)bh * nstate + j;
      const float *Dj = p.ws_decay + sj * D;
      const float *E = p.ws_state + sj * (size_t)(D * D);
#pragma unroll
      for (int ft = 0; ft < FTW; ++ft) {
        float e[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) e[i] = __expf(Dj[16 * (2 * I + ft) + 4 * g4 + i]);
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          const f32x4 x = *reinterpret_cast<const f32x4 *>(E + ((size_t)((2 * I + ft) * NDT + dt) * 64 + lane) * 4);
#pragma unroll
          for (int i = 0; i < 4; ++i) S[ft][dt][i] = e[i] * S[ft][dt][i] + x[i];
        }
      }
    }
    }
    const Frag<T> tri_c0 = tri64_frag<T>(r16, g4, I, 0), tri_c1 = tri64_frag<T>(r16, g4, I, 1);
    Frag<T> kf[KS], kf_next[KS];
    Frag<T> lf[2][2];
    load_kfrag(kf, c_begin * CH);
    load_lgpairs(lf, c_begin * CH, kt);
    // S^T copy of the start state
    auto publish = [&]() {
#pragma unroll
      for (int ft = 0; ft < FTW; ++ft) {
        const int fpos = 32 * I + 8 * g4 + 4 * ft;  // interleaved position of feature 16(2I+ft) + 4g4
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
          store4<T>(sSb + (16 * dt + r16) * LDW + fpos, S[ft][dt][0], S[ft][dt][1], S[ft][dt][2], S[ft][dt][3]);
      }
    };
    publish();
    __syncthreads();  // P: prologue LDS writes complete

    for (int c = c_begin; c < c_end; ++c) {
      const int c0 = c * CH;
      // ---- P0: phi_k of this chunk's rows (keys from registers); the query waves read the
      //      previous chunk's keys and values from LDS meanwhile
      float ko[NFT][4];
      {
        f32x4 z[NFT];
        feature_logits_pipe(sW, kf, r16, g4, z);
        feature_map_rows<HH>(z, ko);
      }
      // finish the feature map here: left to itself the compiler sinks the softmax past the
      // barrier into the next phase
#pragma unroll
      for (int ft = 0; ft < NFT; ++ft)
#pragma unroll
        for (int i = 0; i < 4; ++i) pin(ko[ft][i]);
      __syncthreads();  // B0: the previous chunk's LDS is dead
      // ---- P1: stage this chunk's keys and log gamma^T; publish S_c; next chunk in flight (the
      //      query waves compute phi_q meanwhile)
      store_kfrag(kf);
      store_lgpairs(lf, kt);
      if (c > c_begin) publish();
      if (c + 1 < c_end) {
        int ln = lane;
        asm volatile("" : "+v"(ln));
        kfrag_in(kf_next, c0 + CH, ln);
        pairs_in(lf, LGh, c0 + CH, ln + 64 * (wv - 4));
      }
      __syncthreads();  // B1
      // ---- P2: prefix sums from the chunk start for this sub-chunk's rows
      // (LDS addresses from a lane id the compiler cannot hoist: kept across the loop they
      // would be spilled, and a reloaded spill waits for the loads in flight)
      int ln2 = lane;
      asm volatile("" : "+v"(ln2));
      const T *lgrow = sLgT + (ln2 & 15) * LDV + 8 * (ln2 >> 4);
      const float *tabcol = sTot + 4 * (ln2 >> 4);  // + J * D + 16 ft: C_J of features 16 ft + 4 g4 ..
      // pc: prefix from the chunk start; the chunk totals (all-ones operand, the same products
      // as row 15 of sub-chunk 3) decide the references here, before the tables are shared
      float pc[NFT][4];
      float span_c = 0.f;
      {
        Frag<T> ones;
#pragma unroll
        for (int j = 0; j < 8; ++j) ones.v[j] = from_f<T>(1.f);
#pragma unroll
        for (int ft = 0; ft < NFT; ++ft) {
          const Frag<T> a0 = load8(lgrow + 16 * ft * LDV), a1 = load8(lgrow + 16 * ft * LDV + 32);
          f32x4 cc = mma(a0, tri_c0, f32x4{0.f, 0.f, 0.f, 0.f});
          cc = mma(a1, tri_c1, cc);
          f32x4 tt = mma(a0, ones, f32x4{0.f, 0.f, 0.f, 0.f});
          tt = mma(a1, ones, tt);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            pc[ft][i] = cc[i];
            span_c = fmaxf(span_c, -tt[i]);
          }
        }
      }
      const bool mild = wave_max_all(span_c) <= FAST_SPAN;
      if (r16 == 15) {
#pragma unroll
        for (int ft = 0; ft < NFT; ++ft)
          *reinterpret_cast<f32x4 *>(sTot + I * D + 16 * ft + 4 * g4) = f32x4{pc[ft][0], pc[ft][1], pc[ft][2], pc[ft][3]};
      }
      // decayed queries with the merge weight, in place.  Mild chunk: mix e^{p_t} phi_q
      // (chunk-start reference).  Otherwise mix e^{p_t - C_{I-1}} phi_q (sub-chunk start, the
      // prefix inside sub-chunk I from a masked triangle); the query waves apply the factors
      // between sub-chunks.  Both are at most mix.
      {
        float px[NFT][4];
        if (mild) {
#pragma unroll
          for (int ft = 0; ft < NFT; ++ft)
#pragma unroll
            for (int i = 0; i < 4; ++i) px[ft][i] = pc[ft][i];
        } else {
          float x[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const int sr = 32 * (I >> 1) + 8 * g4 + j;
            x[j] = (sr >= 16 * I && sr <= 16 * I + r16) ? 1.f : 0.f;
          }
          const Frag<T> tri_sub = frag_from<T>(x);
#pragma unroll
          for (int ft = 0; ft < NFT; ++ft) {
            const f32x4 cc = mma(load8(lgrow + 16 * ft * LDV + 32 * (I >> 1)), tri_sub, f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
            for (int i = 0; i < 4; ++i) px[ft][i] = cc[i];
          }
        }
#pragma unroll
        for (int js = 0; js < KS; ++js) {
          T *qp = sQ + (16 * I + r16) * LDQ + 32 * js + 8 * g4;
          const Frag<T> ph = load8(qp);
          float x[8];
#pragma unroll
          for (int jj = 0; jj < 8; ++jj) {
            const int ft = 2 * js + (jj >> 2), i = jj & 3;
            x[jj] = to_f(ph.v[jj]) * exp2_fast(__builtin_fmaf(px[ft][i], LOG2E, log2_mix));
          }
          *reinterpret_cast<bf16x8 *>(qp) = frag_from<T>(x).v;
        }
      }
      __syncthreads();  // B2: sub-chunk prefix ends and decayed queries visible; log gamma^T dead
      // ---- P3: decayed keys -> LDS (interleaved features).  Mild: keys carry e^{-p_s}.
      //      Otherwise e^{C_I - p_s} (decay to the sub-chunk end).
      if (mild) {
#pragma unroll
        for (int ft = 0; ft < NFT; ++ft)
#pragma unroll
          for (int i = 0; i < 4; ++i) ko[ft][i] *= exp2_fast(-pc[ft][i] * LOG2E);
      } else {
#pragma unroll
        for (int ft = 0; ft < NFT; ++ft) {
          const f32x4 t = *reinterpret_cast<const f32x4 *>(tabcol + I * D + 16 * ft);
#pragma unroll
          for (int i = 0; i < 4; ++i) ko[ft][i] *= __expf(t[i] - pc[ft][i]);
        }
      }
#pragma unroll
      for (int ft = 0; ft < NFT; ++ft) {
        const int fpos = 32 * (ft >> 1) + 8 * g4 + 4 * (ft & 1);
        store4<T>(sKt + (16 * I + r16) * LDW + fpos, ko[ft][0], ko[ft][1], ko[ft][2], ko[ft][3]);
      }
      __syncthreads();  // B3: decayed keys visible
      // ---- P4: S = diag(e^{B_c}) S + sum_s k~_s e^{...} v_s^T.  K = 32 steps run over the
      //      interleaved token order of v^T; slot j of lane group g4 is token 32ks + islot(g4, j)
      {
        Frag<T> ka[FTW][2];  // [ft][ks]: decayed keys^T of feature tile 2I + ft, tokens of K-step ks
        float e[FTW][4];     // row decay e^{B_c} = e^{C_3}
#pragma unroll
        for (int ft = 0; ft < FTW; ++ft) {
          const int fr = 16 * (2 * I + ft);
          // key factors e^{C_3} (mild: keys carry e^{-p_s}) or e^{C_3 - C_J} (keys carry e^{C_J - p_s})
          float fac[2][2];  // [ks][half]: factor of the keys of sub-chunk 2ks + half
          const f32x4 c3 = *reinterpret_cast<const f32x4 *>(sTot + 3 * D + fr + 4 * g4);
#pragma unroll
          for (int i = 0; i < 4; ++i) e[ft][i] = __expf(c3[i]);
          const float c3r = sTot[3 * D + fr + r16];
#pragma unroll
          for (int J = 0; J < 4; ++J) fac[J >> 1][J & 1] = __expf(mild ? c3r : c3r - sTot[J * D + fr + r16]);
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) {
            float x[8];
            keysT_tr(sKt, I, ft, ks, r16, g4, x);
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) x[jj] *= fac[ks][jj >> 2];
            ka[ft][ks] = frag_from<T>(x);
          }
        }
        // each v^T fragment serves both feature tiles; the next value tile's fragments are
        // loaded while this one is multiplied
        const T *vrow = sVt + r16 * LDV + 8 * g4;
        Frag<T> vb[2][2];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) vb[0][ks] = load8(vrow + 32 * ks);
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          if (dt + 1 < NDT) {
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) vb[(dt + 1) & 1][ks] = load8(vrow + 16 * (dt + 1) * LDV + 32 * ks);
          }
#pragma unroll
          for (int ft = 0; ft < FTW; ++ft) {
#pragma unroll
            for (int i = 0; i < 4; ++i) S[ft][dt][i] *= e[ft][i];
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) S[ft][dt] = mma(ka[ft][ks], vb[dt & 1][ks], S[ft][dt]);
          }
        }
      }
#pragma unroll
      for (int j = 0; j < KS; ++j) kf[j] = kf_next[j];
    }
    if (p.state_out && seg == p.nseg - 1 && g == 0) {
      float *So = p.state_out + ((size_t)b * p.Hkv + kvh) * D * D;
#pragma unroll
      for (int ft = 0; ft < FTW; ++ft)
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
          for (int i = 0; i < 4; ++i) So[(size_t)(16 * (2 * I + ft) + 4 * g4 + i) * D + 16 * dt + r16] = S[ft][dt][i];
    }
  } else {
    // ======================================================= query waves
    if (self_start) {  // the query waves' part of the walk to the split
      f32x4 Sd[FTW][NDT];
      walk_pipe<HH, true>(plds, Kh, Vh, LGh, c_begin, tid, Sd);
    }
    const float sl2 = p.scale * LOG2E;  // window logits in base 2
    // Window group Z (ZW only): the keys of the chunk two back, tiles I..3, for the queries qz of
    // the chunk at cz0.  It runs at the top of the chunk before (the chunk two back is then the
    // previous chunk, still in LDS) and is carried into group X as (az, mz, lz): unnormalised
    // probabilities times values, the base-2 max per query row, this lane's part of the sum.
    auto window_z = [&](const Frag<T> (&qz)[KS], int cz0, f32x4 (&az)[NDT], float &mz, float &lz) {
      // mask offsets from a lane id the compiler cannot hoist out of the chunk loop (kept
      // across it they were spilled)
      int lnz = lane;
      asm volatile("" : "+v"(lnz));
      const int kminz = max(cz0 + 16 * I + (lnz & 15) - p.W + 1, -hist_avail);
      const int kz0 = cz0 - 2 * CH + 4 * (lnz >> 4);
      f32x4 lt[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        lt[u] = f32x4{NEG_BIG, NEG_BIG, NEG_BIG, NEG_BIG};
        if (u >= I) {
          f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int j = 0; j < KS; ++j) a = mma(load8(sK + (16 * u + r16) * LDW + 32 * j + 8 * g4), qz[j], a);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            lt[u][i] = (kz0 + 16 * u + i >= kminz) ? a[i] * sl2 : NEG_BIG;
          }
        }
      }
      float m = -1.0e20f, l = 0.f;
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int i = 0; i < 4; ++i) m = fmaxf(m, lt[u][i]);
      m = wave_max_cols(m);
      Frag<T> pp[2];
#pragma unroll
      for (int pr = 0; pr < 2; ++pr) {
        float x[8];
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float pv = exp2_fast(lt[2 * pr + h][i] - m);  // masked: 0
            x[4 * h + i] = pv;
            l += pv;
          }
        pp[pr] = frag_from<T>(x);
      }
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int pr = 0; pr < 2; ++pr)
          if (2 * pr + 1 >= I) a = mma(load8(sVt + (16 * dt + r16) * LDV + 32 * pr + 8 * g4), pp[pr], a);
        az[dt] = a;
      }
      mz = m;
      lz = l;
    };
    Frag<T> qf[KS], qf_next[KS], qf_next2[KS];
    Frag<T> vf[2][2];
    f32x4 accz[NDT];
    float m_z = -1.0e20f, l_z = 0.f;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) accz[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    load_q(qf, c_begin * CH);
    if constexpr (ZW) {
      load_vpairs(vf, (c_begin - 2) * CH, tid);
      store_vpairs(vf, tid);
      __syncthreads();  // Z0
      window_z(qf, c_begin * CH, accz, m_z, l_z);
      __syncthreads();  // Z1
      load_q(qf_next, (c_begin + 1) * CH);
    }
    load_vpairs(vf, (c_begin - 1) * CH, tid);
    store_vpairs(vf, tid);
    load_vpairs(vf, c_begin * CH, tid);
    bool unsafe_seen = false;
    // QPHI: the query logits' W_phi_q^T operands come from the fragment-ordered copy in global
    // memory (one kilobyte per wave and operand, L2-resident): feature tiles 0..2 are loaded
    // before B0 and each later tile three tiles ahead, in a ring of four.
    // QPASS (the wide-window variant, which carries group Z through here and has no registers for
    // that ring): this wave's phi_q rows of chunk c, which a pass of their own wrote into the
    // output rows (read here before P4 of chunk c overwrites them), in the interleaved feature
    // order of the LDS rows, loaded at the top of the chunk.
    constexpr bool QPASS = QPHI && ZW, QGLOBAL = QPHI && !ZW;
    const __amdgpu_buffer_rsrc_t wq_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        QGLOBAL ? static_cast<void *>(reinterpret_cast<T *>(p.ws_wq) + (size_t)(p.per_head_q ? hq : 0) * D * D)
                : nullptr,
        (short)0, QGLOBAL ? D * D * (int)sizeof(T) : 0, BUF_RSRC_WORD3);
    constexpr int NWQ = QGLOBAL ? 4 : 1;
    Frag<T> wqf[NWQ][KS];
    auto wq_tile = [&](int ft) {
      if constexpr (QGLOBAL) {
#pragma unroll
        for (int j = 0; j < KS; ++j) wqf[ft % NWQ][j] = buffer_load8<T>(wq_rsrc, 16 * (int)lane, 1024 * (ft * KS + j));
      }
    };
    Frag<T> pq[QPASS ? KS : 1];
    auto load_pq = [&](int c0q) {
      if constexpr (QPASS) {
        const int t = c0q + 16 * I + r16;
        const T *src = Oh + (size_t)(t < L ? t : 0) * D + 8 * g4;
#pragma unroll
        for (int js = 0; js < KS; ++js) pq[js] = t < L ? load8(src + 32 * js) : frag_zero<T>();
      }
    };
    __syncthreads();  // P

    for (int c = c_begin; c < c_end; ++c) {
      const int c0 = c * CH;
      const int pos = c0 + 16 * I + r16;  // query row of this lane's column
      const bool valid = pos < L;

      // lowest key index the window of this row may use
      const int kmin = max(pos - p.W + 1, -hist_avail);
      load_pq(c0);

      // ---- P0: window group X (meta tokens and the previous chunk's keys, still in LDS: tiles
      //      I..3, all four with ZW) in base-2 logits, merged with group Z; unnormalised
      //      probabilities times values into acc.  Then (ZW) group Z of the next chunk.
      f32x4 acc[NDT];
      float m_x = m_z, l_run = 0.f;
      {
        f32x4 lt[5];  // 0: meta; 1 + u: previous-chunk tile u
        {
          f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int j = 0; j < KS; ++j) a = mma(load8(sTk + r16 * LDW + 32 * j + 8 * g4), qf[j], a);
#pragma unroll
          for (int i = 0; i < 4; ++i) lt[0][i] = (4 * g4 + i < p.M) ? a[i] * sl2 : NEG_BIG;
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          lt[1 + u] = f32x4{NEG_BIG, NEG_BIG, NEG_BIG, NEG_BIG};
          if (ZW || u >= I) {
            f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < KS; ++j) a = mma(load8(sK + (16 * u + r16) * LDW + 32 * j + 8 * g4), qf[j], a);
            // (wave-uniform, the wide-window variant) every key of the tile in every row's window:
            // no per-element mask (the narrow variant timed no better without its masks)
            if (ZW && c0 - CH + 16 * u >= -hist_avail && p.W >= 16 * (I - u) + 80) {
#pragma unroll
              for (int i = 0; i < 4; ++i) lt[1 + u][i] = a[i] * sl2;
            } else {
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const int kj = c0 - CH + 16 * u + 4 * g4 + i;
                lt[1 + u][i] = (kj >= kmin) ? a[i] * sl2 : NEG_BIG;
              }
            }
          }
        }
#pragma unroll
        for (int u = 0; u < 5; ++u)
#pragma unroll
          for (int i = 0; i < 4; ++i) m_x = fmaxf(m_x, lt[u][i]);
        m_x = wave_max_cols(m_x);
        const float alpha_z = exp2_fast(m_z - m_x);  // group Z rescaled to the joint max
        l_run = l_z * alpha_z;
        Frag<T> pm, pp[2];
        {
          float x[8];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            x[i] = exp2_fast(lt[0][i] - m_x);
            l_run += x[i];
            x[4 + i] = 0.f;
          }
          pm = frag_from<T>(x);
        }
#pragma unroll
        for (int pr = 0; pr < 2; ++pr) {
          float x[8];
#pragma unroll
          for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float pv = exp2_fast(lt[1 + 2 * pr + h][i] - m_x);  // masked: 0
              x[4 * h + i] = pv;
              l_run += pv;
            }
          pp[pr] = frag_from<T>(x);
        }
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          const int dvl = 16 * dt + r16;
          const T *tv = sTvT + dvl * LDM + 4 * g4;
          f32x4 a0 = {0.f, 0.f, 0.f, 0.f};
          if constexpr (ZW) {
#pragma unroll
            for (int i = 0; i < 4; ++i) a0[i] = accz[dt][i] * alpha_z;
          }
          f32x4 a = mma(load4x2(tv, tv), pm, a0);  // slots 4..7 meet P = 0
#pragma unroll
          for (int pr = 0; pr < 2; ++pr)
            if (ZW || 2 * pr + 1 >= I) a = mma(load8(sVt + dvl * LDV + 32 * pr + 8 * g4), pp[pr], a);
          acc[dt] = a;
        }
      }
      if constexpr (ZW) {
        if (c + 1 < c_end) window_z(qf_next, c0 + CH, accz, m_z, l_z);
      }
      if constexpr (QGLOBAL) {
        wq_tile(0);
        wq_tile(1);
        wq_tile(2);
      }
      __syncthreads();  // B0
      // ---- P1: stage this chunk's values; phi_q of this wave's rows into LDS (the key waves
      //      decay it in place)
      store_vpairs(vf, tid);
      if constexpr (QPASS) {
#pragma unroll
        for (int js = 0; js < KS; ++js) *reinterpret_cast<bf16x8 *>(sQ + (16 * I + r16) * LDQ + 32 * js + 8 * g4) = pq[js].v;
      } else {
        f32x4 zq[NFT];
        float qo[NFT][4];
        if constexpr (QGLOBAL) {
#pragma unroll
          for (int ft = 0; ft < NFT; ++ft) {
            if (ft + 3 < NFT) wq_tile(ft + 3);
            f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < KS; ++j) a = mma(wqf[ft % NWQ][j], qf[j], a);
            zq[ft] = a;
          }
        }
        // (the wide-window variant carries group Z through here: no registers for prefetching)
        else if constexpr (ZW) feature_logits<T, D, LDWW>(sW, qf, r16, g4, zq);
        else feature_logits_pipe(sW, qf, r16, g4, zq);
        feature_map_rows<HH>(zq, qo);
#pragma unroll
        for (int ft = 0; ft < NFT; ++ft) {  // interleaved features
          const int fpos = 32 * (ft >> 1) + 8 * g4 + 4 * (ft & 1);
          store4<T>(sQ + (16 * I + r16) * LDQ + fpos, qo[ft][0], qo[ft][1], qo[ft][2], qo[ft][3]);
        }
      }
      __syncthreads();  // B1
      // ---- P2: window group Y (this chunk's keys 0..I); the key waves compute the decayed queries
      Frag<T> qcf[KS];  // query operand of the intra and inter products (f-interleaved K = 32 slices)
      {
        f32x4 lt[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          lt[u] = f32x4{NEG_BIG, NEG_BIG, NEG_BIG, NEG_BIG};
          if (u <= I) {
            f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < KS; ++j) a = mma(load8(sK + (16 * u + r16) * LDW + 32 * j + 8 * g4), qf[j], a);
            // (wave-uniform, the wide-window variant) a tile before the diagonal inside every row's
            // window: no mask
            if (ZW && u < I && p.W >= 16 * (I - u) + 16) {
#pragma unroll
              for (int i = 0; i < 4; ++i) lt[u][i] = a[i] * sl2;
            } else {
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const int kj = c0 + 16 * u + 4 * g4 + i;
                lt[u][i] = (kj <= pos && kj >= kmin) ? a[i] * sl2 : NEG_BIG;
              }
            }
          }
        }
        float m_y = m_x;
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int i = 0; i < 4; ++i) m_y = fmaxf(m_y, lt[u][i]);
        m_y = wave_max_cols(m_y);  // >= m_x; the diagonal key is always in the window
        const float alpha = exp2_fast(m_x - m_y);
        l_run *= alpha;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[dt][i] *= alpha;
        Frag<T> pp[2];
#pragma unroll
        for (int pr = 0; pr < 2; ++pr) {
          float x[8];
#pragma unroll
          for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float pv = exp2_fast(lt[2 * pr + h][i] - m_y);
              x[4 * h + i] = pv;
              l_run += pv;
            }
          pp[pr] = frag_from<T>(x);
        }
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          const int dvl = 16 * dt + r16;
#pragma unroll
          for (int pr = 0; pr < 2; ++pr)
            if (2 * pr <= I) acc[dt] = mma(load8(sVt + dvl * LDV + 32 * pr + 8 * g4), pp[pr], acc[dt]);
        }
      }
      __syncthreads();  // B2: sub-chunk prefix ends visible
      const bool mild = chunk_is_mild_c<D>(sTot, lane);
      // general case: the diagonal block on the sub-chunk references needs the log decay across
      // sub-chunk I, C_{I-1} - C_I, within SPAN_MAX for every feature
      bool safe = true;
      if (!mild) {
        float span = 0.f;
        int ln = lane;  // (table addresses from an opaque lane id: kept across the loop, spilled)
        asm volatile("" : "+v"(ln));
#pragma unroll
        for (int q = 0; q < D / 64; ++q) {
          const int f = ln + 64 * q;
          span = fmaxf(span, (I > 0 ? sTot[(I - 1) * D + f] : 0.f) - sTot[I * D + f]);
        }
        safe = wave_max_all(span) <= SPAN_MAX;
      }
      // Products decayed out (sub-chunk references only): once every feature has decayed below
      // e^{-skip} between a key's sub-chunk end and the start of sub-chunk I - 1, every term of
      // the block is below that fraction of its undecayed size (p_t - p_s <= C_{I-1} - C_J), the
      // cutoff of the state pass; likewise the state's product once C_{I-1} is below -skip in
      // every feature.  far_s: the inter-chunk product; far0, far1: key sub-chunks 0, 1 (J <= I - 2).
      // C_J decreases with J, so far1 implies far0 and far0 implies far_s.
      bool far_s = false, far0 = false, far1 = false;
      if (!mild && I > 0) {
        float ms = -INFINITY, m0 = -INFINITY, m1 = -INFINITY;
        int ln = lane;
        asm volatile("" : "+v"(ln));
#pragma unroll
        for (int q = 0; q < D / 64; ++q) {
          const int f = ln + 64 * q;
          const float cim1 = sTot[(I - 1) * D + f];
          ms = fmaxf(ms, cim1);
          m0 = fmaxf(m0, cim1 - sTot[f]);
          m1 = fmaxf(m1, cim1 - sTot[D + f]);
        }
        far_s = wave_max_all(ms) < -skip_log<HH>();
        far0 = I >= 2 && wave_max_all(m0) < -skip_log<HH>();
        far1 = I >= 3 && wave_max_all(m1) < -skip_log<HH>();
      }
      // sub-chunks whose diagonal block needs the exact products (added after the chunk loop)
      const bool unsafe = !safe;
      unsafe_seen |= unsafe;
      if (unsafe && lane == 0) sFlag[I * FLAG_WORDS + ((c - c_begin) >> 5)] |= 1u << ((c - c_begin) & 31);
      // next chunk's values and queries in flight from here (later than the key waves' loads:
      // fewer registers live through the feature map and the window)
      if (c + 1 < c_end) {
        int ln = lane;
        asm volatile("" : "+v"(ln));
        pairs_in(vf, Vh, c0 + CH, ln + 64 * wv);
        if constexpr (ZW) q_in(qf_next2, c0 + 2 * CH, ln);
        else q_in(qf_next, c0 + CH, ln);
      }
      // ---- P3: window output normalised and scaled for the merge; for strong-decay chunks the
      //      inter-chunk product (decayed queries and prefix ends are visible since B2, the state
      //      copy since B1)
      {
        const float ws = (1.f - mix) / wave_sum_cols(l_run);
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[dt][i] *= ws;
      }
      // Y^T += S^T qop^T over the 32 S^T fragments, four loaded ahead of their products
      auto inter = [&](const Frag<T> (&qop)[KS]) {
        const T *srow = sSb + r16 * LDW + 8 * g4;
        Frag<T> sb[2][4];
#pragma unroll
        for (int u = 0; u < 4; ++u) sb[0][u] = load8(srow + 16 * u * LDW);
#pragma unroll
        for (int st = 0; st < 2 * KS; ++st) {  // step st: K-step st / 2, value tiles 4 (st % 2) ..
          if (st + 1 < 2 * KS) {
            const int js1 = (st + 1) >> 1, dh1 = (st + 1) & 1;
#pragma unroll
            for (int u = 0; u < 4; ++u) sb[(st + 1) & 1][u] = load8(srow + 16 * (4 * dh1 + u) * LDW + 32 * js1);
          }
          const int js = st >> 1, dh = st & 1;
#pragma unroll
          for (int u = 0; u < 4; ++u) acc[4 * dh + u] = mma(sb[st & 1][u], qop[js], acc[4 * dh + u]);
        }
      };
#pragma unroll
      for (int js = 0; js < KS; ++js) qcf[js] = load8(sQ + (16 * I + r16) * LDQ + 32 * js + 8 * g4);
      if (mild || ZW) {
        // (mild chunks: the inter product stays with the intra products after B3, where it
        // timed better; the wide-window variant has no registers to spare here)
      } else if (I == 0) {
        inter(qcf);
      } else if (!far_s) {
        // sub-chunk references: the queries carry e^{p_t - C_{I-1}}; the state needs e^{p_t}
        Frag<T> qs[KS];
#pragma unroll
        for (int js = 0; js < KS; ++js) {
          float x[8], c8[8];
          tab8(sTot + (I - 1) * D, js, g4, c8);
#pragma unroll
          for (int jj = 0; jj < 8; ++jj) x[jj] = to_f(qcf[js].v[jj]) * __expf(c8[jj]);
          qs[js] = frag_from<T>(x);
        }
        inter(qs);
      }
      __syncthreads();  // B3: decayed keys and tables visible
      // ---- P4: intra- and inter-chunk products onto the window output, store
      auto finish = [&](auto mild_tag) {
        constexpr bool MILD = decltype(mild_tag)::value;
        if constexpr (MILD) {
          // intra-chunk scores A^T[s][t] of key sub-chunk J (masked to s <= t on the diagonal)
          auto score = [&](int J) -> f32x4 {
            f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int js = 0; js < KS; ++js) a = mma(load8(sKt + (16 * J + r16) * LDW + 32 * js + 8 * g4), qcf[js], a);
            if (J == I) {
#pragma unroll
              for (int i = 0; i < 4; ++i) a[i] = (4 * g4 + i <= r16) ? a[i] : 0.f;
            }
            return a;
          };
          // Y^T += V^T A^T over key sub-chunk pairs (2m, 2m+1), interleaved in v^T
#pragma unroll
          for (int m = 0; m < 2; ++m) {
            if (2 * m <= I) {
              const f32x4 a0 = score(2 * m);
              const f32x4 a1 = (2 * m + 1 <= I) ? score(2 * m + 1) : f32x4{0.f, 0.f, 0.f, 0.f};
              float x[8];
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                x[i] = a0[i];
                x[4 + i] = a1[i];
              }
              const Frag<T> bf = frag_from<T>(x);
#pragma unroll
              for (int dt = 0; dt < NDT; ++dt)
                acc[dt] = mma(load8(sVt + (16 * dt + r16) * LDV + 32 * m + 8 * g4), bf, acc[dt]);
            }
          }
          // Y^T += S^T q~^T (state at the chunk start; interleaved features)
          inter(qcf);
        } else {
          // Sub-chunk references (a chunk whose log decay exceeds FAST_SPAN): queries carry
          // e^{p_t - C_{I-1}}, keys e^{C_J - p_s}.  Key sub-chunk J < I - 1 meets the factor
          // e^{C_{I-1} - C_J} <= 1 on the query operand, the diagonal block e^{C_{I-1} - C_I}
          // (at most e^{SPAN_MAX}) on the key operand, the state e^{C_{I-1}}.
          // The query operand of K-step js times e^{C_{hi-1} - C_{lo-1}} (C_{-1} = 0)
          auto qscaled = [&](int js, int lo, int hi) {
            float x[8], a8[8], b8[8];
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) { a8[jj] = 0.f; b8[jj] = 0.f; }
            if (hi > 0) tab8(sTot + (hi - 1) * D, js, g4, a8);
            if (lo > 0) tab8(sTot + (lo - 1) * D, js, g4, b8);
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) x[jj] = to_f(qcf[js].v[jj]) * __expf(a8[jj] - b8[jj]);
            return frag_from<T>(x);
          };
          // scores of the key sub-chunk pair (2m, 2m + 1), then one product with their v^T
#pragma unroll 1
          for (int m = 0; 2 * m <= I; ++m) {
            if (m == 0 && far1) continue;  // key sub-chunks 0 and 1 both decayed out (I = 3)
            f32x4 sc[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              const int J = 2 * m + h;
              f32x4 a = {0.f, 0.f, 0.f, 0.f};
              if (J + 1 == I) {
#pragma unroll
                for (int js = 0; js < KS; ++js) a = mma(load8(sKt + (16 * J + r16) * LDW + 32 * js + 8 * g4), qcf[js], a);
              } else if (J < I && !(J == 0 && far0)) {
#pragma unroll
                for (int js = 0; js < KS; ++js)
                  a = mma(load8(sKt + (16 * J + r16) * LDW + 32 * js + 8 * g4), qscaled(js, J + 1, I), a);
              } else if (J == I && safe) {
#pragma unroll
                for (int js = 0; js < KS; ++js) {
                  float c8[8], cp8[8], kv[8];
                  const Frag<T> kk = load8(sKt + (16 * I + r16) * LDW + 32 * js + 8 * g4);
                  tab8(sTot + I * D, js, g4, c8);
#pragma unroll
                  for (int jj = 0; jj < 8; ++jj) cp8[jj] = 0.f;
                  if (I > 0) tab8(sTot + (I - 1) * D, js, g4, cp8);
#pragma unroll
                  for (int jj = 0; jj < 8; ++jj) kv[jj] = to_f(kk.v[jj]) * __expf(cp8[jj] - c8[jj]);
                  a = mma(frag_from<T>(kv), qcf[js], a);
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) a[i] = (4 * g4 + i <= r16) ? a[i] : 0.f;
              }
              // (an unsafe diagonal block stays zero: its exact products are added after the loop)
              sc[h] = a;
            }
            float x[8];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              x[i] = sc[0][i];
              x[4 + i] = sc[1][i];
            }
            const Frag<T> bf = frag_from<T>(x);
#pragma unroll
            for (int dt = 0; dt < NDT; ++dt)
              acc[dt] = mma(load8(sVt + (16 * dt + r16) * LDV + 32 * m + 8 * g4), bf, acc[dt]);
          }
          if (ZW && !far_s) {  // the inter-chunk product (the other variant ran it before B3)
#pragma unroll
            for (int js = 0; js < KS; ++js) {
              const Frag<T> bf = I > 0 ? qscaled(js, 0, I) : qcf[js];
#pragma unroll
              for (int dt = 0; dt < NDT; ++dt)
                acc[dt] = mma(load8(sSb + (16 * dt + r16) * LDW + 32 * js + 8 * g4), bf, acc[dt]);
            }
          }
        }
        {  // unconditional stores (rows past the end into a sink): under a condition the compiler
           // could not count them, and the next chunk's first use of a prefetched load waited for
           // every store of this one
          T *O = valid ? Oh + (size_t)pos * D : reinterpret_cast<T *>(g_fwd_sink);
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt) store4<T>(O + 16 * dt + 4 * g4, acc[dt][0], acc[dt][1], acc[dt][2], acc[dt][3]);
        }
      };
      if (mild) finish(std::true_type{});
      else finish(std::false_type{});
#pragma unroll
      for (int j = 0; j < KS; ++j) {
        qf[j] = qf_next[j];
        if constexpr (ZW) qf_next[j] = qf_next2[j];
      }
    }
    // Exact diagonal blocks of this wave's flagged sub-chunks, added to the rows it stored
    // (few registers are live after the loop)
    if (unsafe_seen) {
      for (int c = c_begin; c < c_end; ++c) {
        if (!((sFlag[I * FLAG_WORDS + ((c - c_begin) >> 5)] >> ((c - c_begin) & 31)) & 1u)) continue;
        const T *Wq = QPHI ? reinterpret_cast<const T *>(p.wq) + (size_t)hq * p.w_stride : nullptr;
        exact_diag_fixup<HH, QPHI>(sW, Wq, Kh, Vh, LGh, Qh, Oh, c * CH, I, L, mix);
      }
    }
  }
}

// State pass of a segmented sequence: every segment but the last is a block of chunks
// [b0, b1), split into p.sss pieces.  Piece pp of a block walks the block backwards from its
// end, keeps the log-gate sums of the chunks after the current one (the suffix s), and adds the
// chunks c with (b1 - 1 - c) % p.sss == pp decayed to the block end:
//   E_pp = sum_c diag(e^{s_c}) sum_{t in c} diag(e^{C(c) - p_t}) phi_k(k_t) v_t^T,
// where p_t is the prefix sum inside chunk c through t and C(c) its total.  The pieces of a block
// thus add up to the block's state from S = 0 (the recurrence is linear in the added terms).
// Piece 0 also carries the block's log-gate sum D, the others D = 0, so that the whole-head
// kernel's fold S = e^{D_j} S + E_j over the pieces in order gives every segment its start state.
// Once the suffix is below -SKIP_LOG in every feature, the chunks before reach the block end
// decayed by less than e^{-SKIP_LOG} (about 1e-7 of their size, far below what the bf16 output
// can hold): the walk stops there, and piece 0 sets D = NEG_BIG, dropping the state carried in.
// With the Hedgehog map (features up to e^{HH_LOGIT_MAX}, not bounded by one) the cutoff is
// -(SKIP_LOG + 2 HH_LOGIT_MAX), which bounds a dropped term relative to the smallest term any
// token of the same feature row can add (skip_log).
// Every piece reads the log gates of all the chunks it walks (the suffix) and the keys and
// values of its own.  Four waves, each the key side of one sub-chunk, with the arithmetic of
// the key waves above; 80 KB of LDS, so two workgroups share a CU.  The pieces of a block run
// 8 workgroups apart, on one XCD, and share its L2 for the log gates they all read.
//
// The same walk, split between the two roles of the whole-head kernel (walk_pipe), starts the
// second of two segments there without a state pass (fwd_full_kernel, p.split).
namespace full {
constexpr int ST_OFF_W = 0;
constexpr int ST_OFF_VT = ST_OFF_W + D * LDWW * 2;
constexpr int ST_OFF_KT = ST_OFF_VT + D * LDV * 2;
constexpr int ST_OFF_TAB = ST_OFF_KT + SZ_KT;
constexpr int ST_OFF_SUF = ST_OFF_TAB + 4 * D * 4;  // [2][D] suffix sums (alternating chunks)
constexpr int ST_OFF_VOTE = ST_OFF_SUF + 2 * D * 4;
constexpr int ST_LDS_BYTES = ST_OFF_VOTE + 16;
static_assert(2 * ST_LDS_BYTES <= LDS_LIMIT, "state pass: two workgroups per CU");
}  // namespace full

template <bool HH>
__global__ __launch_bounds__(256, 2) void fwd_full_state_kernel(FwdParams p) {
  using namespace full;
  using T = bf16;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  T *sW = reinterpret_cast<T *>(smem + ST_OFF_W);
  const WalkLds lds{sW, reinterpret_cast<T *>(smem + ST_OFF_VT), reinterpret_cast<T *>(smem + ST_OFF_KT),
                    reinterpret_cast<float *>(smem + ST_OFF_TAB), reinterpret_cast<float *>(smem + ST_OFF_SUF),
                    reinterpret_cast<int *>(smem + ST_OFF_VOTE)};
  const int tid = threadIdx.x, lane = tid & 63, I = tid >> 6;
  const int sss = p.sss;
  const int nblk = p.B * p.Hkv * (p.nseg - 1);  // blocks: every segment but the last, per head
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
  const int bg = (slot / sss) * 8 + xcd, pp = slot % sss;
  if (bg >= nblk) return;
  const int bh = bg / (p.nseg - 1), blk = bg % (p.nseg - 1);
  const int grp = bg * sss + pp;  // workspace slot: piece pp of block blk of head bh
  const size_t kv_off = (size_t)bh * (size_t)p.L * D;
  const T *Kh = reinterpret_cast<const T *>(p.k) + kv_off;
  const T *Vh = reinterpret_cast<const T *>(p.v) + kv_off;
  const T *LGh = reinterpret_cast<const T *>(p.lg) + kv_off;
  const int b0 = blk * p.cps, b1 = b0 + p.cps;  // never the last segment: full chunks
  f32x4 S[FTW][NDT];
  float suf;
  const bool stopped = walk_back<HH, true>(lds, Kh, Vh, LGh, b0, b1, pp, sss, tid, S, suf, [&]() {
    load_wT_pairs<256, HH>(sW, reinterpret_cast<const T *>(p.wk) + (size_t)(bh % p.Hkv) * p.w_stride, tid);
  });
  float *E = p.ws_state + (size_t)grp * (D * D);
#pragma unroll
  for (int ft = 0; ft < FTW; ++ft)
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
      *reinterpret_cast<f32x4 *>(E + ((size_t)((2 * I + ft) * NDT + dt) * 64 + lane) * 4) = S[ft][dt];
  if (tid < D) p.ws_decay[(size_t)grp * D + tid] = pp > 0 ? 0.f : (stopped ? NEG_BIG : suf);
}

template <bool ZW, bool HH, bool QPHI>
static hipError_t launch_main(const FwdParams &p, hipStream_t stream) {
  const void *kern = reinterpret_cast<const void *>(fwd_full_kernel<ZW, HH, QPHI>);
  hipError_t e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, full::LDS_BYTES);
  if (e != hipSuccess) return e;
  const dim3 grid(((p.ngroups + 7) / 8) * 8 * p.G);
  hipLaunchKernelGGL((fwd_full_kernel<ZW, HH, QPHI>), grid, dim3(512), full::LDS_BYTES, stream, p);
  return hipGetLastError();
}

template <bool HH>
static hipError_t launch_fwd_full_t(const FwdParams &p, hipStream_t stream) {
  hipError_t e;
  if (p.nseg > 1 && !p.split) {
    e = hipFuncSetAttribute(reinterpret_cast<const void *>(fwd_full_state_kernel<HH>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, full::ST_LDS_BYTES);
    if (e != hipSuccess) return e;
    const int nblk = p.B * p.Hkv * (p.nseg - 1);  // pieces of a block 8 workgroups apart
    hipLaunchKernelGGL(fwd_full_state_kernel<HH>, dim3(((nblk + 7) / 8) * 8 * p.sss), dim3(256), full::ST_LDS_BYTES,
                       stream, p);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  const bool zw = p.W > CH + 1;
  if (p.qphi && (e = zw ? launch_fwd_full_phiq(p, stream) : launch_fwd_full_wq_frag(p, stream)) != hipSuccess)
    return e;
  return zw ? (p.qphi ? launch_main<true, HH, true>(p, stream) : launch_main<true, HH, false>(p, stream))
            : (p.qphi ? launch_main<false, HH, true>(p, stream) : launch_main<false, HH, false>(p, stream));
}

hipError_t launch_fwd_full(const FwdParams &p, hipStream_t stream) {
  return p.hh ? launch_fwd_full_t<true>(p, stream) : launch_fwd_full_t<false>(p, stream);
}

}  // namespace lz
