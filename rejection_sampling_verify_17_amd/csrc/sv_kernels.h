// Verification kernels, dense path (no top-k filter).
//
// The rule judges drafts left to right and discards everything after the
// first rejection, so rows after it need not be read.  Positions are walked
// in windows [w0, w1): one position each for large batches, all of them at
// once when the whole input is small and extra launches would dominate.
//
//   k_rows (launch 0)  statistics of rows 0..w1-1 of every sequence: partial
//                      base-2 softmax statistics (R, S) of each draft and
//                      target row, one vocabulary chunk per work item, and the
//                      two logits at the drafted token; clears the counters of
//                      the launches to come.
//   k_rows (launch 1)  a fixed number of blocks per sequence; wave 0 of each
//                      judges that first window (lane l merges row pair l's
//                      partials, evaluates q(t)/p(t) in registers and draws u;
//                      a ballot finds the first rejection; one block writes
//                      the outputs), then the block takes its share of what
//                      the judgement leaves: a statistics chunk of the next
//                      window, or a chunk of the sampled row (the residual
//                      max(0, q - p) of the rejected row, or the bonus row
//                      gamma).
//   k_rows (launch i)  a grid sized to the chip walks the two lists, sampling
//                      items (Gumbel-max winner over one chunk of a row,
//                      VALU-bound) first, then statistics items of window i
//                      (memory-bound), so both kinds share every compute unit.
//   From launch 1 on, the block that finishes a sequence's last statistics
//   item judges the window at once and appends the sequence to the lists of
//   the next launch; the block that finishes a sampled row's last chunk
//   writes the token.
//
// Blocks of one launch talk only through per-sequence counters: an item's
// results are written with stores that bypass the (per-die, mutually
// non-coherent) L2 caches, the writer waits until they are performed, then
// increments the counter atomically; the block whose increment completes the
// count reads them back with loads that bypass the L2 as well.  No block ever
// waits for another, and no fence (on this GPU a write-back and invalidation of
// the whole L2) is needed.  Lists are appended with atomic slot counters and
// read by the next launch; three sets rotate (read, append, clear).
//
// The rule is that of page "스펙큘러티브 디코딩 — 작은 모델이 먼저 쓰고 큰 모델이
// 검사한다" (blog.mna-game.duckdns.org post 46), §1, and page "추측 디코딩: 큰 모델을
// 빠르게 돌리는 법" (ai-trend.me), section "어떻게 작동하나".
#pragma once

#include "sv_device.h"

namespace sv {

constexpr int kThreads = 256;
constexpr int kJudgeWaves = 16;          // sequences judged side by side per k_judge block
constexpr int kBonusRow = 0x10000;       // sampling-list flag: sample the bonus row
constexpr int kMaxSampleChunks = 8;      // chunks a sampled row is split into at most (each finishes with atomics on the row's counters)

// Per-sequence state of the top-k path between launches: w >= 0 means
// "alive up to position w"; anything else means done.
constexpr int kDone = -1;
constexpr int kInvalid = -2;

struct Args {
  const void *target;      // [B][gamma+1][V]
  const void *draft;       // [B][gamma][V]
  const int32_t *tokens;   // [B][gamma]
  int32_t B, gamma, V, top_k;
  float top_p;             // nucleus mass (1: off); only with 0 < top_k <= 1024
  float c;                 // log2(e) / T
  uint32_t key0, key1;     // Philox key = seed
  uint64_t seq_offset;
  int32_t *out_tokens;     // [B][gamma+1]
  int32_t *n_accepted;     // [B]
  float *token_probs;      // [B][gamma][2] or null
  float *accept_ur;        // [B][gamma][2] or null
  // workspace, dense path
  float4 *part;            // [B][gamma][nch_max] {Rp, Sp, Rq, Sq}
  float2 *ztok;            // [B][gamma] draft and target logit at the drafted token
  int2 *slist;             // [3][B] sampling lists {b, row | kBonusRow}
  float4 *sst;             // [3][B] statistics of the sampled row pair
  int32_t *tlist;          // [3][B] statistics lists: sequences alive for the next window
  int32_t *lcnt;           // [3][2] list lengths {sampling, statistics}
  int32_t *icnt;           // [B] statistics items of the current window finished
  int32_t *pcnt;           // [B] sampling chunks finished
  unsigned long long *pbest;  // [B] best packed key of the sampled row so far (0 = none)
  int32_t nch;             // statistics: vocabulary chunks per row in launch 0
  int32_t nch_max;         // statistics: chunks per row at most (stride of part)
  int32_t nvec;            // statistics: 16-byte vectors per row (any alignment)
  int32_t ngb;             // sampling: group blocks (16 bytes of entries) per row
  int32_t cs_max;          // sampling: chunks per row at most
  // both paths
  int32_t *nseq;           // [B] n, or -1 for an invalid sequence
  // top-k path
  int32_t *state;          // [2][B] alternating halves by launch parity
  uint4 *rowinfo;          // [B][2*gamma] {thr lo, thr hi, R bits, S bits}
  int2 *lists;             // [B][2*gamma][K] (index, logit bits) or null
  int32_t klist;           // K when lists are kept, else 0
  // arg-max mode (temperature 0)
  unsigned long long *gpart;  // [B][gamma+1][gstride] packed arg-max key per chunk
  int32_t gstride;            // chunks per row at most
  // draft sampling
  int32_t *drafted;           // [B][gamma] drawn draft tokens
  int32_t argmax;             // 1: temperature 0 (the first largest logit)
};

__device__ __forceinline__ uint32_t seq_of(const Args &a, int b) {
  return (uint32_t)(a.seq_offset + (uint64_t)b);
}

template <int DT>
__device__ __forceinline__ const void *target_row(const Args &a, int b, int j) {
  return (const char *)a.target + ((size_t)b * (a.gamma + 1) + j) * (size_t)a.V * Elem<DT>::kSize;
}
template <int DT>
__device__ __forceinline__ const void *draft_row(const Args &a, int b, int j) {
  return (const char *)a.draft + ((size_t)b * a.gamma + j) * (size_t)a.V * Elem<DT>::kSize;
}

// Whole row of outputs for an invalid sequence (wave-cooperative).
__device__ __forceinline__ void write_invalid(const Args &a, int b, int lane) {
  const int gamma = a.gamma;
  int32_t *out = a.out_tokens + (size_t)b * (gamma + 1);
  for (int i = lane; i <= gamma; i += kWave) out[i] = -1;
  if (lane == 0) {
    a.n_accepted[b] = -1;
    a.nseq[b] = -1;
  }
}

// Prefix, padding and n of a judged sequence (wave-cooperative; the sampled
// slot n is written by the pick step).
__device__ __forceinline__ void write_judged(const Args &a, int b, int lane, int n) {
  const int gamma = a.gamma;
  int32_t *out = a.out_tokens + (size_t)b * (gamma + 1);
  for (int i = lane; i <= gamma; i += kWave) {
    if (i < n) out[i] = a.tokens[(size_t)b * gamma + i];
    else if (i > n) out[i] = -1;
  }
  if (lane == 0) {
    a.n_accepted[b] = n;
    a.nseq[b] = n;
  }
}

// Diagnostics of a judged position (NaN-filled first for every position, so
// positions after the first rejection stay NaN).
__device__ __forceinline__ void write_diag(const Args &a, int b, int j, float pt, float qt, float u, float ratio) {
  const size_t i = ((size_t)b * a.gamma + j) * 2;
  if (a.token_probs) {
    a.token_probs[i] = pt;
    a.token_probs[i + 1] = qt;
  }
  if (a.accept_ur) {
    a.accept_ur[i] = u;
    a.accept_ur[i + 1] = ratio;
  }
}

// Are all drafted tokens of sequence b in [0, V)?  (one wave)
__device__ __forceinline__ bool tokens_valid(const Args &a, int b, int lane) {
  bool ok = true;
  for (int j = lane; j < a.gamma; j += kWave) {
    const int t = a.tokens[(size_t)b * a.gamma + j];
    ok = ok && (t >= 0) && (t < a.V);
  }
  return __ballot(!ok) == 0ull;
}

// Keep-decision of draft t at one position from its stored logits and the two
// rows' statistics: keep iff q(t) > 0 and (p(t) = 0 or u < q(t)/p(t)).
// q(t)/p(t) = 2^(c (zq - zp) - (Rq - Rp)) * Sp / Sq: the large terms cancel
// before rounding (Rq - Rp is an exact integer difference).
struct Judged {
  bool accept;
  float u, ratio, pt, qt;
};
__device__ __forceinline__ Judged judge_one(const Args &a, uint32_t seq, int j, float zp, float zq, bool pzero,
                                            bool qzero, float Rp, float Sp, float Rq, float Sq) {
  Judged r;
  const Philox4 blk = stream_block(a.key0, a.key1, seq, (uint32_t)j, 0u, PURPOSE_ACCEPT);
  r.u = accept_uniform(blk.w[0]);
  if (qzero) r.ratio = 0.0f;
  else if (pzero) r.ratio = INFINITY;
  else r.ratio = __builtin_amdgcn_exp2f(a.c * (zq - zp) - (Rq - Rp)) * (Sp / Sq);
  r.accept = !qzero && (pzero || r.u < r.ratio);
  r.pt = pzero ? 0.0f : __builtin_amdgcn_exp2f(fmaf(zp, a.c, -Rp)) / Sp;
  r.qt = qzero ? 0.0f : __builtin_amdgcn_exp2f(fmaf(zq, a.c, -Rq)) / Sq;
  return r;
}

// ---------------------------------------------------------------------------
// Communication between blocks of one launch
// ---------------------------------------------------------------------------

// Agent-scope relaxed atomic loads and stores: they bypass the L2 of the die
// the block runs on, so a block on another die sees the value.
__device__ __forceinline__ void store_coherent(float *p, float v) {
  __hip_atomic_store((uint32_t *)p, __float_as_uint(v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_coherent(const float *p) {
  return __uint_as_float(__hip_atomic_load((uint32_t *)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}
__device__ __forceinline__ void store_coherent(float4 *p, float4 v) {
  float *f = (float *)p;
  store_coherent(f, v.x);
  store_coherent(f + 1, v.y);
  store_coherent(f + 2, v.z);
  store_coherent(f + 3, v.w);
}
__device__ __forceinline__ float4 load_coherent(const float4 *p) {
  const float *f = (const float *)p;
  return make_float4(load_coherent(f), load_coherent(f + 1), load_coherent(f + 2), load_coherent(f + 3));
}

// Waits until every memory operation this wave issued is performed (vmcnt,
// expcnt and lgkmcnt all zero).  Results published with agent-scope atomic
// stores are then visible to every block of the agent, and a counter bumped
// after this wait can announce them: the agent-scope release sequence of the
// LLVM AMDGPU memory model for gfx942/gfx950 is an L2 write-back followed by
// this same wait before the releasing operation; the write-back is not
// needed here because everything published was itself stored with the
// agent-coherent bit.  The empty asm statements keep the compiler from
// moving memory accesses across the wait (the builtin itself is not a
// memory barrier to the compiler).
__device__ __forceinline__ void wait_performed() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0);
  asm volatile("" ::: "memory");
}

// ---------------------------------------------------------------------------
// Work items
// ---------------------------------------------------------------------------

// Rescale (R, S) so that R >= m c (m: the largest logit about to be added).
__device__ __forceinline__ void raise_ref(float &R, float &S, float m, float c) {
  const float mc = m * c;
  if (mc > R) {
    const float Rn = ceilf(mc);
    S = (R == -INFINITY) ? 0.0f : scale_pow2(S, R - Rn);
    R = Rn;
  }
}

// Fold vectors [u0, u0 + FU) of one row into (R, S), S 2^R being the sum of
// 2^(z c) so far, R an integer that only rises.  R need not bound the
// largest z c: fp32 keeps its relative precision at any scale, so a fold
// sums its terms 2^(z c - R) against the R it finds (one fma, exp2 and add
// per entry, no maximum).  Only when R is still unset, or the fold's terms
// pass 2^64 (an entry more than 64 above R), is R raised to the fold's
// ceil(max z c), S rescaled by that exact power of two and the fold summed
// again.  Every term then stays at most 2^64 and S below 2^82 for rows of up
// to 2^17 folds per thread; partial sums merge by exact powers of two as
// before, and readers form 2^(z c - R) / S alike.
template <int FU, int U, int NE>
__device__ __forceinline__ void fold_vecs(float &R, float &S, const float (&z)[U][NE], int u0, float c) {
  float s = 0.0f;
  if (R != -INFINITY) {
#pragma unroll
    for (int u = u0; u < u0 + FU; ++u)
#pragma unroll
      for (int e = 0; e < NE; ++e) s += __builtin_amdgcn_exp2f(fmaf(z[u][e], c, -R));
  }
  if (R == -INFINITY || !(s <= 0x1p64f)) {
    float m = z[u0][0];
#pragma unroll
    for (int u = u0; u < u0 + FU; ++u)
#pragma unroll
      for (int e = 0; e < NE; ++e) m = fmaxf(m, z[u][e]);
    raise_ref(R, S, m, c);
    s = 0.0f;
    if (R != -INFINITY) {
#pragma unroll
      for (int u = u0; u < u0 + FU; ++u)
#pragma unroll
        for (int e = 0; e < NE; ++e) s += __builtin_amdgcn_exp2f(fmaf(z[u][e], c, -R));
    }
  }
  S += s;
}

// Partial statistics of draft row j and target row j over vectors [v0, v1);
// the chunk whose vectors hold the drafted token also records its two logits.
// Each step loads U vectors of each row and folds them 8 entries at a time;
// entries outside the row or the chunk (only in edge steps) are masked to
// -inf first.  The drafted token and its logits are loaded only after the
// first step's vectors: vector loads complete in order, so loading them
// first would hold the wave back by two memory round trips before its stream
// starts.  The token index is a scalar load (counted apart from vector loads),
// waited for only where it is first used.
template <int DT>
__device__ float4 chunk_stats(const Args &a, int b, int j, int v0, int v1) {
  constexpr int NE = Elem<DT>::kVec;
  constexpr int U = 2;                // vectors in flight per row per thread
  constexpr int FU = NE == 4 ? 2 : 1;  // vectors per fold (8 entries)
  const Row<DT> P(draft_row<DT>(a, b, j), a.V);
  const Row<DT> Q(target_row<DT>(a, b, j), a.V);
  const int V = a.V;
  const float c = a.c;
  // vectors [ilo, ihi) hold no entry outside the row in either row
  const int ilo = (max(P.s, Q.s) + NE - 1) / NE;
  const int ihi = min((V + P.s) / NE, (V + Q.s) / NE);
  float Rp = -INFINITY, Sp = 0.0f, Rq = -INFINITY, Sq = 0.0f;
  const int t = a.tokens[(size_t)b * a.gamma + j];  // b, j uniform: a scalar load
  bool capp = false, capq = false;
  float zpt = 0.0f, zqt = 0.0f;
  bool first = true;
  for (int base = v0 + (int)threadIdx.x; base < v1; base += kThreads * U) {
    float zp[U][NE], zq[U][NE];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int iv = base + u * kThreads;
      P.load_vec(iv, zp[u]);  // past the row: zeros or neighbours, masked below
      Q.load_vec(iv, zq[u]);
    }
    if (first) {
      first = false;
      const bool tv = t >= 0 && t < V;
      capp = tv && threadIdx.x == 0 && (t + P.s) / NE >= v0 && (t + P.s) / NE < v1;
      capq = tv && threadIdx.x == 0 && (t + Q.s) / NE >= v0 && (t + Q.s) / NE < v1;
      if (capp) zpt = P.load_one(t);
      if (capq) zqt = Q.load_one(t);
    }
    const int top = base + (U - 1) * kThreads;
    const bool edge = base < ilo || top >= ihi || top >= v1;
#pragma unroll
    for (int u0 = 0; u0 < U; u0 += FU) {
      if (edge) {
#pragma unroll
        for (int u = u0; u < u0 + FU; ++u) {
          const int iv = base + u * kThreads;
          const int e0p = iv * NE - P.s, e0q = iv * NE - Q.s;  // entry of element 0
#pragma unroll
          for (int e = 0; e < NE; ++e) {
            if (iv >= v1 || e0p + e < 0 || e0p + e >= V) zp[u][e] = -INFINITY;
            if (iv >= v1 || e0q + e < 0 || e0q + e >= V) zq[u][e] = -INFINITY;
          }
        }
      }
      fold_vecs<FU>(Rp, Sp, zp, u0, c);
      fold_vecs<FU>(Rq, Sq, zq, u0, c);
    }
  }
  float *zt = (float *)(a.ztok + (size_t)b * a.gamma + j);
  if (capp) store_coherent(zt, zpt);
  if (capq) store_coherent(zt + 1, zqt);
  block_merge_stats2<kThreads>(Rp, Sp, Rq, Sq);
  return make_float4(Rp, Sp, Rq, Sq);
}

// Residual weight max(0, q_v - p_v) as the GPU can resolve it.  q_v and p_v
// come from fp32 softmax sums whose rounding depends on how a row's entries
// fall into 16-byte vectors (its address), so two identical rows can differ
// in the last bits; a difference at or below 2^-16 of q_v (under the 1e-5
// resolution the results are held to) is rounding, not residual mass, and
// counts as zero.  An all-zero residual then falls back to q, as it does in
// exact arithmetic.  The products are rounded before the subtraction (no
// FMA contraction), so identical statistics give exactly zero.
__device__ __forceinline__ float residual_weight(float qv, float pv) {
#pragma clang fp contract(off)
  const float r = qv - pv;
  return r > qv * 0x1p-16f ? r : 0.0f;
}
__device__ __forceinline__ float residual_weight(float eq, float invSq, float ep, float invSp) {
#pragma clang fp contract(off)
  const float qv = eq * invSq;
  const float pv = ep * invSp;
  return residual_weight(qv, pv);
}

// Gumbel-max winner over group blocks [g0, g1) of row `pos`: the residual
// weights max(0, q - p) (statistics st of that row pair) when RESID, else the
// bonus row (weights q).  Residual key r / E2 (the exponential race, monotone
// in ln r - ln E), compared inside a thread as r * E2' > r' * E2 so no
// reciprocal is needed; bonus key z c - log2 E2 (monotone in ln q - ln E).
// Each thread walks its entries in increasing index, so a strict comparison
// keeps the smaller index among equal keys; the block reduction does the same
// on the packed key.  exp2(-inf) = 0 gives masked logits zero weight.
template <int DT, bool RESID, bool X3 = false>
__device__ unsigned long long chunk_winner(const Args &a, int b, int pos, float4 st, int g0, int g1) {
  constexpr int NE = Elem<DT>::kVec;
  constexpr int U = NE == 4 ? 2 : 1;  // group blocks in flight per thread (8 entries)
  const uint32_t seq = seq_of(a, b);
  const float c = a.c;
  const Row<DT> Q(target_row<DT>(a, b, pos), a.V);
  const Row<DT> P(draft_row<DT>(a, b, RESID ? pos : 0), a.V);
  const float invSp = 1.0f / st.y, invSq = 1.0f / st.w;
  const uint32_t lim = (uint32_t)min(a.V, g1 * NE);  // entries at or past lim are masked
  const PhiloxStream ps(a.key0, a.key1, seq, (uint32_t)pos, PURPOSE_SAMPLE);
  float bestk = -INFINITY;        // bonus: best key
  float bestr = 0.0f, bestE = 1.0f;  // residual: best r / E2 as a fraction
  uint32_t besti = 0xFFFFFFFFu;  // none
  for (int base = g0 + (int)threadIdx.x; base < g1; base += kThreads * U) {
    float zq[U][NE], zp[U][NE];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      Q.load_block(base + u * kThreads, zq[u]);  // past the chunk: masked below
      if (RESID) P.load_block(base + u * kThreads, zp[u]);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int gb = base + u * kThreads;
#pragma unroll
      for (int g = 0; g < NE / 4; ++g) {
        const uint32_t group = (uint32_t)(gb * (NE / 4) + g);
        const Philox4 blk = ps.template block<X3>(group);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t idx = group * 4u + (uint32_t)e;
          const float E2 = exp2_variate(blk.w[e]);
          bool take;
          if (RESID) {
            const float r = residual_weight(__builtin_amdgcn_exp2f(fmaf(zq[u][g * 4 + e], c, -st.z)), invSq,
                                            __builtin_amdgcn_exp2f(fmaf(zp[u][g * 4 + e], c, -st.x)), invSp);
            take = idx < lim && r * bestE > bestr * E2;  // r / E2 > bestr / bestE (and r > 0)
            bestr = take ? r : bestr;
            bestE = take ? E2 : bestE;
          } else {
            const float key = fmaf(zq[u][g * 4 + e], c, -__builtin_amdgcn_logf(E2));
            take = idx < lim && key > bestk;
            bestk = take ? key : bestk;
          }
          besti = take ? idx : besti;
        }
      }
    }
  }
  if (RESID) bestk = bestr / bestE;
  const unsigned long long best = besti == 0xFFFFFFFFu ? 0ull : pack_key(bestk, besti);
  return block_max_u64<kThreads>(best);
}

// ---------------------------------------------------------------------------
// Judging a window: one wave per sequence.  Positions [p0, w0) have their
// statistics; the next window starts at w0 (w0 = gamma: none left).
// mode: -1 nothing to do, 0 statistics of the next window, 1 residual of
// `row`, 2 bonus row.  Every load is issued up front (one memory round trip):
// the lane's drafted token, the logits at the token and the partial
// statistics, spread over the lanes.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int pow2_at_least(int x) {
  int g = 1;
  while (g < x) g <<= 1;
  return g;
}

template <int DT>
__device__ void judge_window(const Args &a, int b, int lane, int p0, int w0, int nch, bool first, bool write,
                             int &mode, int &row, float4 &st) {
  const int gamma = a.gamma;
  const int nj = w0 - p0;
  mode = -1;
  row = 0;
  st = make_float4(0.f, 1.f, 0.f, 1.f);
  const int tok = lane < gamma ? a.tokens[(size_t)b * gamma + lane] : 0;
  const bool act = lane < nj;
  const int jpos = p0 + (act ? lane : 0);
  const float *zt = (const float *)(a.ztok + (size_t)b * gamma + jpos);
  const float zp = load_coherent(zt), zq = load_coherent(zt + 1);
  // merged statistics of position p0 + lane: gs lanes per position and pass
  const int gs = nch >= kWave ? kWave : pow2_at_least(nch);
  const int ppp = kWave / gs;
  float Rp = -INFINITY, Sp = 0.0f, Rq = -INFINITY, Sq = 0.0f;
  for (int q0 = 0; q0 < nj; q0 += ppp) {
    const int myq = q0 + lane / gs;
    float rp = -INFINITY, sp = 0.0f, rq = -INFINITY, sq = 0.0f;
    if (myq < nj) {
      const float4 *pp = a.part + ((size_t)b * gamma + p0 + myq) * a.nch_max;
      for (int ch = lane % gs; ch < nch; ch += gs) {
        const float4 v = load_coherent(pp + ch);
        merge_stats(rp, sp, v.x, v.y);
        merge_stats(rq, sq, v.z, v.w);
      }
    }
    for (int off = gs / 2; off > 0; off >>= 1) {
      const float rp2 = __shfl_xor(rp, off, kWave), sp2 = __shfl_xor(sp, off, kWave);
      const float rq2 = __shfl_xor(rq, off, kWave), sq2 = __shfl_xor(sq, off, kWave);
      merge_stats(rp, sp, rp2, sp2);
      merge_stats(rq, sq, rq2, sq2);
    }
    const bool mine = lane >= q0 && lane < q0 + ppp;
    const int src = mine ? (lane - q0) * gs : 0;
    const float xrp = __shfl(rp, src, kWave), xsp = __shfl(sp, src, kWave);
    const float xrq = __shfl(rq, src, kWave), xsq = __shfl(sq, src, kWave);
    if (mine) {
      Rp = xrp;
      Sp = xsp;
      Rq = xrq;
      Sq = xsq;
    }
  }
  if (first) {
    // (launch 0 has filled the diagnostics with NaN)
    const bool ok = __ballot(lane < gamma && (tok < 0 || tok >= a.V)) == 0ull;
    if (!ok) {
      if (write) write_invalid(a, b, lane);
      return;
    }
  }
  // lane l judges position p0 + l; a ballot of the accept bits finds the
  // first rejection
  Judged jr{};
  if (act) jr = judge_one(a, seq_of(a, b), jpos, zp, zq, zp == -INFINITY, zq == -INFINITY, Rp, Sp, Rq, Sq);
  const unsigned long long mask = __ballot(act && jr.accept);
  const int k = (mask == ~0ull) ? kWave : __builtin_ctzll(~mask);  // first clear bit
  if (write && act && lane <= k) write_diag(a, b, jpos, jr.pt, jr.qt, jr.u, jr.ratio);
  int n;
  if (k < nj) {
    n = p0 + k;
    mode = 1;
    st = make_float4(__shfl(Rp, k, kWave), __shfl(Sp, k, kWave), __shfl(Rq, k, kWave), __shfl(Sq, k, kWave));
  } else if (w0 == gamma) {
    n = gamma;
    mode = 2;
  } else {
    mode = 0;
    return;
  }
  row = n;
  if (!write) return;
  // outputs: the accepted prefix, -1 after the sampled slot n (written by
  // the block that finishes the sampled row)
  int32_t *out = a.out_tokens + (size_t)b * (gamma + 1);
  for (int i = lane; i <= gamma; i += kWave) {
    if (i < n) out[i] = tok;  // i < n <= gamma, so i == lane
    else if (i > n) out[i] = -1;
  }
  if (lane == 0) {
    a.n_accepted[b] = n;
    a.nseq[b] = n;
  }
}

// List set of launch i (three rotate: read by launch i, appended by launch
// i - 1, cleared by launch i - 2).
__device__ __forceinline__ int list_set(int launch) { return launch % 3; }

// Append sequence b to the lists of list set li (one thread).
__device__ __forceinline__ void append(const Args &a, int li, int mode, int b, int row, float4 st) {
  int32_t *cnt = a.lcnt + 2 * li;
  // every sequence is appended at most once per set, so slot < B; the test
  // only keeps a broken invariant from writing out of bounds
  if (mode >= 1) {
    const int slot = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (slot < a.B) {
      a.slist[(size_t)li * a.B + slot] = make_int2(b, row | (mode == 2 ? kBonusRow : 0));
      a.sst[(size_t)li * a.B + slot] = st;
    }
  } else if (mode == 0) {
    const int slot = __hip_atomic_fetch_add(cnt + 1, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (slot < a.B) a.tlist[(size_t)li * a.B + slot] = b;
  }
}

// First judgement (window [0, w0) of every sequence, measured by launch 0)
// when a statistics window follows: one wave per sequence; the sequence goes
// on a list of set 1 for launch 1.  A block reserves its list slots with one
// atomic per list.
template <int DT>
__global__ __launch_bounds__(kJudgeWaves *kWave) void k_judge(Args a, int w0) {
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int b = blockIdx.x * kJudgeWaves + wave;
  __shared__ int sh_mode[kJudgeWaves], sh_row[kJudgeWaves];
  __shared__ float4 sh_st[kJudgeWaves];
  int mode = -1, row = 0;
  float4 st = make_float4(0.f, 1.f, 0.f, 1.f);
  if (b < a.B) judge_window<DT>(a, b, lane, 0, w0, a.nch, true, true, mode, row, st);
  if (lane == 0) {
    sh_mode[wave] = mode;
    sh_row[wave] = row;
    sh_st[wave] = st;
  }
  __syncthreads();
  if (wave == 0) {
    const int m = lane < kJudgeWaves ? sh_mode[lane] : -1;
    const unsigned long long ms = __ballot(m >= 1), mt = __ballot(m == 0);
    const unsigned long long below = (1ull << lane) - 1ull;
    const int li = list_set(1);
    int32_t *cnt = a.lcnt + 2 * li;
    int bs = 0, bt = 0;
    if (lane == 0) {
      if (ms) bs = __hip_atomic_fetch_add(cnt, __popcll(ms), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (mt) bt = __hip_atomic_fetch_add(cnt + 1, __popcll(mt), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    bs = __shfl(bs, 0, kWave);
    bt = __shfl(bt, 0, kWave);
    const int bl = blockIdx.x * kJudgeWaves + lane;
    if (m >= 1) {
      const int slot = bs + __popcll(ms & below);
      a.slist[(size_t)li * a.B + slot] = make_int2(bl, sh_row[lane] | (m == 2 ? kBonusRow : 0));
      a.sst[(size_t)li * a.B + slot] = sh_st[lane];
    }
    if (m == 0) a.tlist[(size_t)li * a.B + bt + __popcll(mt & below)] = bl;
  }
}

// ---------------------------------------------------------------------------
// Row work
// ---------------------------------------------------------------------------

// Values every thread of the block holds alike, moved to scalar registers
// (row addresses and buffer descriptors built from them stay scalar).
__device__ __forceinline__ int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ float uni(float x) {
  return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(x)));
}

// Launch 0 (MODE 0): statistics of rows [w0, w1) of every sequence; also
// clears the per-sequence counters of the launches to come.  When launch 0
// read every position (w0 = gamma), launch 1 runs in MODE 1: kb blocks per
// sequence; wave 0 of each judges the sequence (one block writes the
// outputs), then the block draws chunk `slot` of the sampled row (cs1
// chunks); kb = cs1 and nch1 = 0 then, though the code also takes statistics
// chunks of rows [w0, w1) (nch1 per row).  Otherwise k_judge judges the first
// window and every later launch runs in MODE 2: the lists of set i: sampling
// items, then statistics items of rows [w0, w1); the last launch (w0 = w1 =
// gamma: sampling items only) runs as MODE 3, the same code compiled without
// the statistics and judging parts.  A block takes its items in rounds of
// up to kQueue; each item's result goes out at once (partial statistics by
// coherent store, chunk winner kept in LDS), and at the end of a round the
// block finishes all its items together: winners folded into the row's best
// key, per-sequence counters advanced, and for every sequence whose window or
// sampled row it completed, the judgement (window) or the token (row).
template <int DT, int MODE>
__global__ __launch_bounds__(kThreads, 8) void k_rows(Args a, int launch, int w0, int w1, int kb, int nch1,
                                                     int cs1) {
  constexpr int kQueue = 64;
  __shared__ int sh_nq;
  __shared__ int q_b[kQueue], q_row[kQueue];  // row >= 0: sampled row; -1: statistics item
  __shared__ int q_fin[kQueue];               // 1: finished the sequence's window or row
  __shared__ unsigned long long q_w[kQueue];  // chunk winner, then the row's best key
  __shared__ int sh_mode, sh_row;
  __shared__ float4 sh_st;
  const int li = list_set(launch);
  // launch 0 clears the sets k_judge (1) and launch 1 (2) append to; launch
  // i >= 1 the set launch i + 1 appends to
  if (blockIdx.x == 0 && threadIdx.x < (MODE == 0 ? 4 : 2))
    a.lcnt[2 * list_set(launch + (MODE == 0 ? 1 : 2)) + threadIdx.x] = 0;
  if (threadIdx.x == 0) sh_nq = 0;
  // MODE 3: the last launch, which only samples (no window left to read);
  // without the statistics and judging code it has the registers for the
  // one-instruction three-way XORs of Philox
  const int dw = MODE == 3 ? 0 : w1 - w0;
  int nch, cs, per_stat;
  if (MODE == 1) {
    // one item per block, after the block's own judgement of window [0, w0)
    nch = nch1;
    cs = cs1;
    per_stat = dw * nch;
    const int b = blockIdx.x / kb, slot = blockIdx.x - b * kb;
    if (threadIdx.x < kWave) {
      int mode = -1, row = 0;
      float4 st = make_float4(0.f, 1.f, 0.f, 1.f);
      if (b < a.B) judge_window<DT>(a, b, threadIdx.x, 0, w0, a.nch, true, slot == 0, mode, row, st);
      if (threadIdx.x == 0) {
        sh_mode = mode;
        sh_row = row;
        sh_st = st;
      }
    }
    __syncthreads();
    const int mode = sh_mode, row = sh_row;
    if (mode == 0 && slot < per_stat) {
      const int r = slot / nch, ch = slot - r * nch;
      const int j = w0 + r;
      const int cv = (a.nvec + nch - 1) / nch;
      const int v0 = ch * cv;
      const float4 pst = chunk_stats<DT>(a, b, j, v0, min(a.nvec, v0 + cv));
      if (threadIdx.x == 0) {
        store_coherent(a.part + ((size_t)b * a.gamma + j) * a.nch_max + ch, pst);
        sh_nq = 1;
        q_b[0] = b;
        q_row[0] = -1;
      }
    } else if (mode >= 1 && slot < cs) {
      const int gper = (a.ngb + cs - 1) / cs;
      const int g0 = slot * gper, g1 = min(a.ngb, g0 + gper);
      const float4 st = make_float4(uni(sh_st.x), uni(sh_st.y), uni(sh_st.z), uni(sh_st.w));
      // (this launch has the registers for the one-instruction XORs)
      const unsigned long long w = mode == 2
          ? chunk_winner<DT, false, true>(a, b, row, make_float4(0.f, 1.f, 0.f, 1.f), g0, g1)
          : chunk_winner<DT, true, true>(a, b, row, st, g0, g1);
      if (threadIdx.x == 0) {
        sh_nq = 1;
        q_b[0] = b;
        q_row[0] = row;
        q_w[0] = w;
      }
    }
  }
  // Chunks per row in later launches: the grid is shared between the row
  // pairs to read (statistics) and the rows to sample, the same number of
  // blocks per row pair for both kinds, so that every block takes one item and
  // all finish about together (sampling chunks are capped: past a few per
  // row, more blocks only add fixed costs).
  int n_samp = 0, n_stat = a.B;
  if (MODE >= 2) {
    n_samp = min(max(uni(a.lcnt[2 * li]), 0), a.B);
    n_stat = min(max(uni(a.lcnt[2 * li + 1]), 0), a.B);
    const int G = (int)gridDim.x;
    const int rows = n_stat * dw;
    const int per_pair = max(1, G / max(1, rows + n_samp));
    nch = min(a.nch_max, per_pair);
    cs = n_samp > 0 ? max(1, min(a.cs_max, (G - rows * nch) / n_samp)) : 1;
    per_stat = dw * nch;
  } else if (MODE == 0) {
    nch = a.nch;  // fixed: the first judgement reads these chunks
    cs = 1;
    per_stat = dw * nch;
  }
  const long long s_items = MODE >= 2 ? (long long)n_samp * cs : 0;
  const long long total = MODE == 1 ? 0 : s_items + (long long)n_stat * per_stat;
  const long long round = (long long)kQueue * gridDim.x;
  // (a MODE 1 block passes once, with no item to take, to finish the one it has)
  for (long long k0 = blockIdx.x; k0 < total || (MODE == 1 && k0 == (long long)blockIdx.x); k0 += round) {
    const long long kend = min(total, k0 + round);
    for (long long k = k0; k < kend; k += gridDim.x) {
      if (MODE >= 2 && k < s_items) {
        const int l = (int)(k / cs);
        const int ch = (int)(k - (long long)l * cs);
        const int2 e = a.slist[(size_t)li * a.B + l];
        const int b = uni(e.x), ey = uni(e.y), row = ey & 0xFFFF;
        if ((unsigned)b >= (unsigned)a.B || row > a.gamma) continue;  // never taken: entries come from append()
        const int gper = (a.ngb + cs - 1) / cs;
        const int g0 = ch * gper, g1 = min(a.ngb, g0 + gper);
        unsigned long long w;
        if (ey & kBonusRow) {
          w = chunk_winner<DT, false, MODE == 3>(a, b, row, make_float4(0.f, 1.f, 0.f, 1.f), g0, g1);
        } else {
          const float4 st = a.sst[(size_t)li * a.B + l];
          w = chunk_winner<DT, true, MODE == 3>(a, b, row, make_float4(uni(st.x), uni(st.y), uni(st.z), uni(st.w)),
                                                g0, g1);
        }
        if (threadIdx.x == 0) {
          const int q = sh_nq++;
          q_b[q] = b;
          q_row[q] = row;
          q_w[q] = w;
        }
      } else if (MODE != 3) {
        const long long k2 = k - s_items;
        const int l = (int)(k2 / per_stat);
        const int rc = (int)(k2 - (long long)l * per_stat);
        const int r = rc / nch, ch = rc - r * nch;
        const int b = MODE == 0 ? l : uni(a.tlist[(size_t)li * a.B + l]);
        if ((unsigned)b >= (unsigned)a.B) continue;  // never taken: entries come from append()
        const int j = w0 + r;
        if (MODE == 0 && r == 0 && ch == 0 && threadIdx.x == 0) {
          // counters of the launches to come (read there after this launch
          // ends), and diagnostics NaN for every position until one is judged
          a.icnt[b] = 0;
          a.pcnt[b] = 0;
          a.pbest[b] = 0ull;
          for (int k = 0; k < a.gamma; ++k) write_diag(a, b, k, NAN, NAN, NAN, NAN);
        }
        const int cv = (a.nvec + nch - 1) / nch;
        const int v0 = ch * cv;
        const float4 pst = chunk_stats<DT>(a, b, j, v0, min(a.nvec, v0 + cv));
        if (threadIdx.x == 0) {
          store_coherent(a.part + ((size_t)b * a.gamma + j) * a.nch_max + ch, pst);
          if (MODE >= 2) {
            const int q = sh_nq++;
            q_b[q] = b;
            q_row[q] = -1;
          }
        }
      }
    }
    if (MODE == 0) continue;
    // finish the round's items, one thread each
    __syncthreads();
    const int nq = sh_nq;
    const int t = threadIdx.x;
    if (t < nq && q_row[t] >= 0)
      __hip_atomic_fetch_max(a.pbest + q_b[t], q_w[t], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    wait_performed();  // every wave: its coherent stores and maxima are performed
    __syncthreads();
    if (t < nq) {
      const int b = q_b[t];
      const bool samp = q_row[t] >= 0;
      const int old = __hip_atomic_fetch_add(samp ? a.pcnt + b : a.icnt + b, 1, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT);
      const bool fin = old == (samp ? cs : per_stat) - 1;
      q_fin[t] = fin;
      if (fin && samp) {
        const unsigned long long best =
            __hip_atomic_fetch_max(a.pbest + b, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        q_w[t] = best;
        if (best != 0ull) a.out_tokens[(size_t)b * (a.gamma + 1) + q_row[t]] = (int32_t)packed_index(best);
      }
    }
    __syncthreads();
    // judgements of completed windows, one wave each
    for (int q = threadIdx.x / kWave; MODE != 3 && q < nq; q += kThreads / kWave) {
      if (!q_fin[q] || q_row[q] >= 0) continue;
      const int b = q_b[q];
      int mode, row;
      float4 st;
      judge_window<DT>(a, b, threadIdx.x % kWave, w0, w1, nch, false, true, mode, row, st);
      if (threadIdx.x % kWave == 0) {
        // every item of this window is counted: the counter starts over for the next
        if (mode == 0) __hip_atomic_store(a.icnt + b, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        append(a, list_set(launch + 1), mode, b, row, st);
      }
    }
    // an empty residual (reachable only through rounding): sample q_row
    for (int q = 0; q < nq; ++q) {
      if (!q_fin[q] || q_row[q] < 0 || q_w[q] != 0ull) continue;
      const int b = uni(q_b[q]), row = uni(q_row[q]);
      const unsigned long long best = chunk_winner<DT, false>(a, b, row, make_float4(0.f, 1.f, 0.f, 1.f), 0, a.ngb);
      if (threadIdx.x == 0) a.out_tokens[(size_t)b * (a.gamma + 1) + row] = (int32_t)packed_index(best);
    }
    __syncthreads();
    if (threadIdx.x == 0) sh_nq = 0;
    __syncthreads();
  }
}

}  // namespace sv
