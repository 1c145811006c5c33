// Verification kernels, dense path (no top-k filter).
//
// The rule judges drafts left to right and discards everything after the
// first rejection, so rows after it need not be read.  Launches walk the
// positions in windows [w0, w1) (one position each for large batches, all of
// them at once when the whole input is small and launches would dominate):
//
//   k_step(first window)  every sequence: partial base-2 softmax statistics
//                   (R, S) of draft and target rows w0..w1-1, one vocabulary
//                   chunk per block.
//   k_step(next windows)  every block of a sequence still alive first judges
//                   the previous window itself (wave 0: lane l merges row pair
//                   l's partials, evaluates q(t)/p(t) in registers and draws
//                   u; a ballot finds the first rejection), then, on its chunk:
//                     all accepted, window left:  statistics of its row;
//                     all accepted, none left:    Gumbel-max winner over
//                                                 target row gamma (bonus);
//                     rejected at n:              Gumbel-max winner over the
//                                                 residual max(0, q - p) of row n.
//                   Memory-bound statistics of live sequences and VALU-bound
//                   sampling of finished ones share each launch.
//   k_pick          one wave per sequence: the best chunk winner is the token.
//
// A per-sequence state (double-buffered by launch index parity, so blocks of
// one launch read what the previous launch wrote) says whether the sequence
// is alive at the window start.  Blocks never signal each other inside a launch:
// results cross launch boundaries only (on this GPU an agent-scope fence is a
// write-back and invalidation of the whole L2, far too dear to pay per block).
//
// The rule is that of page "스펙큘러티브 디코딩 — 작은 모델이 먼저 쓰고 큰 모델이
// 검사한다" (blog.mna-game.duckdns.org post 46), §1, and page "추측 디코딩: 큰 모델을
// 빠르게 돌리는 법" (ai-trend.me), section "어떻게 작동하나".
#pragma once

#include "sv_device.h"

namespace sv {

constexpr int kThreads = 256;

// Per-sequence state between launches: w >= 0 means "alive: every position
// before the last window accepted and the last window's statistics written,
// up to row w"; anything else means done.
constexpr int kDone = -1;
constexpr int kInvalid = -2;

struct Args {
  const void *target;      // [B][gamma+1][V]
  const void *draft;       // [B][gamma][V]
  const int32_t *tokens;   // [B][gamma]
  int32_t B, gamma, V, top_k;
  float c;                 // log2(e) / T
  uint32_t key0, key1;     // Philox key = seed
  uint64_t seq_offset;
  int32_t *out_tokens;     // [B][gamma+1]
  int32_t *n_accepted;     // [B]
  float *token_probs;      // [B][gamma][2] or null
  float *accept_ur;        // [B][gamma][2] or null
  // workspace
  float4 *part;            // [B][gamma][nch] {Rp, Sp, Rq, Sq}
  unsigned long long *bestpart;  // [B][nchw] chunk winners (0 = none)
  int32_t *nseq;           // [B] n, or -1 for an invalid sequence
  int32_t *state;          // [2][B] launch-parity double buffer
  int32_t nch;             // statistics: vocabulary chunks per row
  int32_t nvec, cv;        // statistics: 16-byte vectors per row (any alignment), per chunk
  int32_t nchw;            // sampling: vocabulary chunks of the sampled row
  int32_t ngb, cv2;        // sampling: group blocks per row, per chunk
  // top-k path
  uint4 *rowinfo;          // [B][2*gamma] {thr lo, thr hi, R bits, S bits}
  int2 *lists;             // [B][2*gamma][K] (index, logit bits) or null
  int32_t klist;           // K when lists are kept, else 0
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

// Are all drafted tokens of sequence b in [0, V)?  (wave 0)
__device__ __forceinline__ bool tokens_valid(const Args &a, int b) {
  const int lane = threadIdx.x;
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
// Block pieces
// ---------------------------------------------------------------------------

// Partial statistics of draft row j and target row j over vectors [v0, v1).
template <int DT>
__device__ float4 chunk_stats(const Args &a, int b, int j, int v0, int v1) {
  constexpr int NE = Elem<DT>::kVec;
  constexpr int U = 4;  // vectors in flight per row per thread
  const Row<DT> P(draft_row<DT>(a, b, j), a.V);
  const Row<DT> Q(target_row<DT>(a, b, j), a.V);
  const int V = a.V;
  const float c = a.c;
  float Rp = -INFINITY, Sp = 0.0f, Rq = -INFINITY, Sq = 0.0f;
  for (int base = v0 + (int)threadIdx.x; base < v1; base += kThreads * U) {
    float zp[U][NE], zq[U][NE];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int iv = base + u * kThreads;
      P.load_vec(iv, zp[u]);  // past the row: zeros or neighbours, masked below
      Q.load_vec(iv, zq[u]);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int iv = base + u * kThreads;
      const int ep = iv * NE - P.s, eq = iv * NE - Q.s;  // entry of element 0
      if (iv >= v1 || ep < 0 || eq < 0 || ep + NE > V || eq + NE > V) {
#pragma unroll
        for (int e = 0; e < NE; ++e) {
          if (iv >= v1 || ep + e < 0 || ep + e >= V) zp[u][e] = -INFINITY;
          if (iv >= v1 || eq + e < 0 || eq + e >= V) zq[u][e] = -INFINITY;
        }
      }
      accumulate<NE>(Rp, Sp, zp[u], c);
      accumulate<NE>(Rq, Sq, zq[u], c);
    }
  }
  block_merge_stats2<kThreads>(Rp, Sp, Rq, Sq);
  return make_float4(Rp, Sp, Rq, Sq);
}

// Gumbel-max winner of group blocks [g0, g1) of row `pos`: residual weights
// q - p (statistics st of that row pair) when `residual`, else the bonus row
// (weights q).  Residual key r / E2 (the exponential race, monotone in
// ln r - ln E); bonus key z c - log2 E2 (monotone in ln q - ln E).
template <int DT>
__device__ unsigned long long chunk_winner(const Args &a, int b, int pos, bool residual, float4 st, int g0,
                                           int g1) {
  constexpr int NE = Elem<DT>::kVec;
  const uint32_t seq = seq_of(a, b);
  const float c = a.c;
  const int V = a.V;
  const Row<DT> Q(target_row<DT>(a, b, pos), V);
  const Row<DT> P(draft_row<DT>(a, b, residual ? pos : 0), V);
  const float invSp = 1.0f / st.y, invSq = 1.0f / st.w;
  constexpr int U = 2;  // group blocks in flight per thread
  unsigned long long best = 0ull;
  for (int base = g0 + (int)threadIdx.x; base < g1; base += kThreads * U) {
    float zq[U][NE], zp[U][NE];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      Q.load_block(base + u * kThreads, zq[u]);  // past the chunk: masked below
      if (residual) P.load_block(base + u * kThreads, zp[u]);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int gb = base + u * kThreads;
      if (gb >= g1) continue;
#pragma unroll
      for (int g = 0; g < NE / 4; ++g) {
        float w[4];
        bool any = false;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int idx = gb * NE + g * 4 + e;
          const float zqe = zq[u][g * 4 + e];
          if (residual) {
            const float qv = (zqe == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(fmaf(zqe, c, -st.z)) * invSq;
            const float zpe = zp[u][g * 4 + e];
            const float pv = (zpe == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(fmaf(zpe, c, -st.x)) * invSp;
            w[e] = (idx < V) ? qv - pv : 0.0f;
            any |= w[e] > 0.0f;
          } else {
            w[e] = (idx < V && zqe != -INFINITY) ? zqe : -INFINITY;
            any |= w[e] != -INFINITY;
          }
        }
        if (!any) continue;
        const uint32_t group = (uint32_t)(gb * (NE / 4) + g);
        const Philox4 blk = stream_block(a.key0, a.key1, seq, (uint32_t)pos, group, PURPOSE_SAMPLE);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t idx = group * 4u + (uint32_t)e;
          unsigned long long k = 0ull;
          if (residual) {
            if (w[e] > 0.0f) k = pack_key(w[e] * __builtin_amdgcn_rcpf(exp2_variate(blk.w[e])), idx);
          } else {
            if (w[e] != -INFINITY)
              k = pack_key(fmaf(w[e], c, -__builtin_amdgcn_logf(exp2_variate(blk.w[e]))), idx);
          }
          best = k > best ? k : best;
        }
      }
    }
  }
  return block_max_u64<kThreads>(best);
}

// ---------------------------------------------------------------------------
// One launch per window of positions (see the top of this file).  A launch
// judges the previous window [p0, w0) and computes statistics of the rows of
// its own window [w0, w1) (w0 = w1 = gamma: the last launch, judge only).
// Blocks per sequence: max(dw x nch, nchw), dw = max(1, w1 - w0).  For
// statistics block (r, ch) handles chunk ch of row w0 + r; for sampling block
// ch handles chunk ch of the sampled row; blocks beyond that count exit.
// ---------------------------------------------------------------------------
template <int DT>
__global__ __launch_bounds__(kThreads) void k_step(Args a, int launch, int p0, int w0, int w1) {
  const int dw = w1 > w0 ? w1 - w0 : 1;
  const int per_seq = max(dw * a.nch, a.nchw);
  const int b = blockIdx.x / per_seq;
  const int rem = blockIdx.x - b * per_seq;
  const int gamma = a.gamma;
  const bool lead = rem == 0;  // writes the sequence's outputs and state
  int32_t *state_in = a.state + (size_t)((launch + 1) & 1) * a.B;
  int32_t *state_out = a.state + (size_t)(launch & 1) * a.B;

  __shared__ int sh_mode;   // 0 statistics, 1 residual, 2 bonus, -1 nothing
  __shared__ int sh_row;    // row to sample (residual)
  __shared__ float4 sh_st;
  if (threadIdx.x < kWave) {
    const int lane = threadIdx.x;
    int mode = 0, row = 0;
    float4 st = make_float4(0.f, 1.f, 0.f, 1.f);
    if (w0 == 0) {
      if (!tokens_valid(a, b)) {
        mode = -1;
        if (lead) {
          write_invalid(a, b, lane);
          for (int k = lane; k < gamma; k += kWave) write_diag(a, b, k, NAN, NAN, NAN, NAN);
          if (lane == 0) state_out[b] = kInvalid;
        }
      } else if (lead) {
        for (int k = lane; k < gamma; k += kWave) write_diag(a, b, k, NAN, NAN, NAN, NAN);
        if (lane == 0) state_out[b] = w1;
      }
    } else {
      const int s = state_in[b];
      if (s != w0) {
        mode = -1;  // finished (or invalid) before this window
        if (lead && lane == 0) state_out[b] = s;
      } else {
        // judge positions p0..w0-1: lane l merges the partial statistics of
        // row pair p0 + l, evaluates its ratio and draws its u; a ballot of
        // the accept bits finds the first rejection
        const int nj = w0 - p0;
        const bool act = lane < nj;
        const int jpos = p0 + (act ? lane : 0);
        float Rp = -INFINITY, Sp = 0.0f, Rq = -INFINITY, Sq = 0.0f;
        bool accept = false;
        if (act) {
          const float4 *pp = a.part + ((size_t)b * gamma + jpos) * a.nch;
          for (int k = 0; k < a.nch; ++k) {
            const float4 v = pp[k];
            merge_stats(Rp, Sp, v.x, v.y);
            merge_stats(Rq, Sq, v.z, v.w);
          }
          const int t = a.tokens[(size_t)b * gamma + jpos];
          const float zp = Row<DT>(draft_row<DT>(a, b, jpos), a.V).load_one(t);
          const float zq = Row<DT>(target_row<DT>(a, b, jpos), a.V).load_one(t);
          const Judged jr =
              judge_one(a, seq_of(a, b), jpos, zp, zq, zp == -INFINITY, zq == -INFINITY, Rp, Sp, Rq, Sq);
          accept = jr.accept;
          if (lead) write_diag(a, b, jpos, jr.pt, jr.qt, jr.u, jr.ratio);
        }
        const unsigned long long mask = __ballot(act && accept);
        const int k = (mask == ~0ull) ? kWave : __builtin_ctzll(~mask);  // first clear bit
        if (lead && act && lane > k) write_diag(a, b, jpos, NAN, NAN, NAN, NAN);  // judged after the rejection
        if (k < nj) {
          mode = 1;
          row = p0 + k;
          st = make_float4(__shfl(Rp, k, kWave), __shfl(Sp, k, kWave), __shfl(Rq, k, kWave), __shfl(Sq, k, kWave));
          if (lead) write_judged(a, b, lane, row);
          if (lead && lane == 0) state_out[b] = kDone;
        } else if (w0 == gamma) {
          mode = 2;
          row = gamma;
          if (lead) write_judged(a, b, lane, gamma);
          if (lead && lane == 0) state_out[b] = kDone;
        } else if (lead && lane == 0) {
          state_out[b] = w1;
        }
      }
    }
    if (lane == 0) {
      sh_mode = mode;
      sh_row = row;
      sh_st = st;
    }
  }
  __syncthreads();
  const int mode = sh_mode;
  if (mode < 0) return;
  if (mode == 0) {
    if (rem >= dw * a.nch) return;
    const int r = rem / a.nch;
    const int ch = rem - r * a.nch;
    const int j = w0 + r;
    const int v0 = ch * a.cv;
    const float4 pst = chunk_stats<DT>(a, b, j, v0, min(a.nvec, v0 + a.cv));
    if (threadIdx.x == 0) a.part[((size_t)b * gamma + j) * a.nch + ch] = pst;
  } else {
    if (rem >= a.nchw) return;
    const int g0 = rem * a.cv2;
    const unsigned long long w = chunk_winner<DT>(a, b, sh_row, mode == 1, sh_st, g0, min(a.ngb, g0 + a.cv2));
    if (threadIdx.x == 0) a.bestpart[(size_t)b * a.nchw + rem] = w;
  }
}

// ---------------------------------------------------------------------------
// Pick: one wave per sequence.  The largest chunk winner is the token; if the
// residual was empty (reachable only through rounding), q_n is sampled instead
// by the same wave.
// ---------------------------------------------------------------------------
template <int DT>
__global__ __launch_bounds__(kThreads) void k_pick(Args a) {
  const int lane = threadIdx.x % kWave;
  const int b = blockIdx.x * (kThreads / kWave) + (int)threadIdx.x / kWave;
  if (b >= a.B) return;
  const int n = a.nseq[b];
  if (n < 0 || n > a.gamma) return;
  unsigned long long best = 0ull;
  for (int i = lane; i < a.nchw; i += kWave) {
    const unsigned long long k = a.bestpart[(size_t)b * a.nchw + i];
    best = k > best ? k : best;
  }
  best = wave_max_u64(best);
  if (best == 0ull) {
    const Row<DT> Q(target_row<DT>(a, b, n), a.V);
    const uint32_t seq = seq_of(a, b);
    for (int v = lane; v < a.V; v += kWave) {
      const float z = Q.load_one(v);
      if (z == -INFINITY) continue;
      const Philox4 blk = stream_block(a.key0, a.key1, seq, (uint32_t)n, (uint32_t)v >> 2, PURPOSE_SAMPLE);
      const float E = exp2_variate(word_of(blk, (uint32_t)v & 3u));
      const unsigned long long k = pack_key(fmaf(z, a.c, -__builtin_amdgcn_logf(E)), (uint32_t)v);
      best = k > best ? k : best;
    }
    best = wave_max_u64(best);
  }
  if (lane == 0) a.out_tokens[(size_t)b * (a.gamma + 1) + n] = (int32_t)packed_index(best);
}

}  // namespace sv
