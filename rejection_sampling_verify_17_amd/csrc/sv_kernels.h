// Verification kernels, dense path (no top-k filter).
//
//   k_stats   one block per (row pair, vocabulary chunk): streams draft row j and
//             target row j of a sequence and writes partial base-2 softmax
//             statistics (R, S) of both.
//   k_sample  one block per (sequence, vocabulary chunk).  Its first wave
//             merges the sequence's partials, evaluates every acceptance ratio
//             in registers and ballots the accept bits to find the first
//             rejection n (each block of the sequence does this small step
//             itself, so no block waits on another).  The block then draws the
//             Gumbel-max winner of its chunk: over the residual max(0, q_n - p_n),
//             or over target row gamma when every draft was kept.
//   k_pick    one wave per sequence: the best chunk winner is the token.
//
// Blocks never signal each other inside a kernel: results cross kernel
// boundaries only (on this GPU an agent-scope fence is a write-back and
// invalidation of the whole L2, far too dear to pay per block).
//
// The rule is that of page "스펙큘러티브 디코딩 — 작은 모델이 먼저 쓰고 큰 모델이
// 검사한다" (blog.mna-game.duckdns.org post 46), §1, and page "추측 디코딩: 큰 모델을
// 빠르게 돌리는 법" (ai-trend.me), section "어떻게 작동하나".
#pragma once

#include "sv_device.h"

namespace sv {

constexpr int kThreads = 256;

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
  float4 *part;            // [B*gamma*nch] {Rp, Sp, Rq, Sq}
  unsigned long long *bestpart;  // [B*nch2] chunk winners (0 = none)
  int32_t *nseq;           // [B] n, or -1 for an invalid sequence
  int32_t nvec, nch, cv;   // pass 1: vectors per row (any alignment), chunks, vectors per chunk
  int32_t ngb, nch2, cv2;  // pass 2: group blocks per row, chunks, group blocks per chunk
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

__device__ __forceinline__ void write_invalid(const Args &a, int b, int lane) {
  const int gamma = a.gamma;
  int32_t *out = a.out_tokens + (size_t)b * (gamma + 1);
  for (int i = lane; i <= gamma; i += kWave) out[i] = -1;
  if (lane == 0) {
    a.n_accepted[b] = -1;
    a.nseq[b] = -1;
  }
  for (int j = lane; j < gamma; j += kWave) {
    if (a.token_probs) {
      a.token_probs[((size_t)b * gamma + j) * 2 + 0] = NAN;
      a.token_probs[((size_t)b * gamma + j) * 2 + 1] = NAN;
    }
    if (a.accept_ur) {
      a.accept_ur[((size_t)b * gamma + j) * 2 + 0] = NAN;
      a.accept_ur[((size_t)b * gamma + j) * 2 + 1] = NAN;
    }
  }
}

// Prefix, padding and n of a judged sequence (the sampled slot n is written
// by the pick step).
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

// Ballot result -> first rejected position (gamma if all gamma accepted).
__device__ __forceinline__ int first_rejection(unsigned long long mask, int gamma) {
  const int n = (mask == ~0ull) ? kWave : __builtin_ctzll(~mask);
  return n < gamma ? n : gamma;
}

// ---------------------------------------------------------------------------
// Pass 1: partial softmax statistics of draft row j and target row j.
// ---------------------------------------------------------------------------
template <int DT>
__global__ __launch_bounds__(kThreads) void k_stats(Args a) {
  constexpr int NE = Elem<DT>::kVec;
  constexpr int U = 4;  // vectors in flight per row per thread
  const int tile = blockIdx.x;
  const int row = tile / a.nch;
  const int ch = tile - row * a.nch;
  const int b = row / a.gamma;
  const int j = row - b * a.gamma;

  const Row<DT> P(draft_row<DT>(a, b, j), a.V);
  const Row<DT> Q(target_row<DT>(a, b, j), a.V);
  const int v0 = ch * a.cv;
  const int v1 = min(a.nvec, v0 + a.cv);
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
      const int ep = iv * NE - P.s, eq = iv * NE - Q.s;  // entry of lane 0
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
  if (threadIdx.x == 0) a.part[tile] = make_float4(Rp, Sp, Rq, Sq);
}

// ---------------------------------------------------------------------------
// Judging a sequence (wave 0 of a block).  Lane j holds position j: it merges
// that position's partial statistics, evaluates q_j(t_j) / p_j(t_j) and draws
// u_j; a 64-wide ballot of the accept bits gives the first rejection n.
// Returns n (or -1 for an invalid sequence) in every lane; `st` receives the
// statistics of row n in every lane.  Writes the outputs if `write`.
// ---------------------------------------------------------------------------
template <int DT>
__device__ int judge_dense(const Args &a, int b, bool write, float4 &st) {
  const int lane = threadIdx.x;
  const int gamma = a.gamma;
  const bool active = lane < gamma;
  const uint32_t seq = seq_of(a, b);

  float Rp = -INFINITY, Sp = 0.0f, Rq = -INFINITY, Sq = 0.0f;
  int t = 0;
  bool ok = true;
  if (active) {
    const float4 *pp = a.part + ((size_t)b * gamma + lane) * a.nch;
    for (int c = 0; c < a.nch; ++c) {
      const float4 v = pp[c];
      merge_stats(Rp, Sp, v.x, v.y);
      merge_stats(Rq, Sq, v.z, v.w);
    }
    t = a.tokens[(size_t)b * gamma + lane];
    ok = (t >= 0) && (t < a.V);
  }
  if (__ballot(active && !ok) != 0ull) {
    if (write) write_invalid(a, b, lane);
    return -1;
  }

  bool accept = false;
  if (active) {
    const float zp = Row<DT>(draft_row<DT>(a, b, lane), a.V).load_one(t);
    const float zq = Row<DT>(target_row<DT>(a, b, lane), a.V).load_one(t);
    const Philox4 blk = stream_block(a.key0, a.key1, seq, (uint32_t)lane, 0u, PURPOSE_ACCEPT);
    const float u = accept_uniform(blk.w[0]);
    const bool qzero = (zq == -INFINITY);
    const bool pzero = (zp == -INFINITY);
    // q(t)/p(t) = 2^(c (zq - zp) - (Rq - Rp)) * Sp / Sq: the large terms cancel
    // before rounding (Rq - Rp is an exact integer difference).
    float ratio;
    if (qzero) ratio = 0.0f;
    else if (pzero) ratio = INFINITY;
    else ratio = __builtin_amdgcn_exp2f(a.c * (zq - zp) - (Rq - Rp)) * (Sp / Sq);
    accept = !qzero && (pzero || u < ratio);
    if (write && a.token_probs) {
      const float pt = pzero ? 0.0f : __builtin_amdgcn_exp2f(fmaf(zp, a.c, -Rp)) / Sp;
      const float qt = qzero ? 0.0f : __builtin_amdgcn_exp2f(fmaf(zq, a.c, -Rq)) / Sq;
      a.token_probs[((size_t)b * gamma + lane) * 2 + 0] = pt;
      a.token_probs[((size_t)b * gamma + lane) * 2 + 1] = qt;
    }
    if (write && a.accept_ur) {
      a.accept_ur[((size_t)b * gamma + lane) * 2 + 0] = u;
      a.accept_ur[((size_t)b * gamma + lane) * 2 + 1] = ratio;
    }
  }
  const int n = first_rejection(__ballot(active && accept), gamma);
  // statistics of row n, from lane n (unused when n == gamma)
  const int src = n < gamma ? n : 0;
  st = make_float4(__shfl(Rp, src, kWave), __shfl(Sp, src, kWave), __shfl(Rq, src, kWave),
                   __shfl(Sq, src, kWave));
  if (write) write_judged(a, b, lane, n);
  return n;
}

// ---------------------------------------------------------------------------
// Pass 2: judge, then the Gumbel-max winner of one vocabulary chunk of the row
// to sample.  Residual key r_v / E_v (the exponential race, monotone in
// ln r_v - ln E_v); bonus key z_v c - log2 E2_v (monotone in ln q_v - ln E_v).
// ---------------------------------------------------------------------------
template <int DT>
__global__ __launch_bounds__(kThreads) void k_sample(Args a) {
  constexpr int NE = Elem<DT>::kVec;
  const int tile = blockIdx.x;
  const int b = tile / a.nch2;
  const int ch = tile - b * a.nch2;
  const int gamma = a.gamma;

  __shared__ float4 sh_st;
  __shared__ int sh_n;
  if (threadIdx.x < kWave) {
    float4 st;
    const int n = judge_dense<DT>(a, b, ch == 0, st);
    if (threadIdx.x == 0) {
      sh_n = n;
      sh_st = st;
    }
  }
  __syncthreads();
  const int n = sh_n;
  if (n < 0) return;
  const float4 st = sh_st;
  const bool residual = n < gamma;
  const uint32_t seq = seq_of(a, b);
  const float c = a.c;
  const int V = a.V;

  const Row<DT> Q(target_row<DT>(a, b, n), V);
  const Row<DT> P(draft_row<DT>(a, b, residual ? n : 0), V);
  const float invSp = 1.0f / st.y, invSq = 1.0f / st.w;

  const int g0 = ch * a.cv2;
  const int g1 = min(a.ngb, g0 + a.cv2);
  unsigned long long best = 0ull;
  for (int gb = g0 + (int)threadIdx.x; gb < g1; gb += kThreads) {
    float zq[NE], zp[NE];
    Q.load_block(gb, zq);
    if (residual) P.load_block(gb, zp);
#pragma unroll
    for (int g = 0; g < NE / 4; ++g) {
      float w[4];
      bool any = false;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int idx = gb * NE + g * 4 + e;
        const float zqe = zq[g * 4 + e];
        if (residual) {
          const float qv = (zqe == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(fmaf(zqe, c, -st.z)) * invSq;
          const float zpe = zp[g * 4 + e];
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
      const Philox4 blk = stream_block(a.key0, a.key1, seq, (uint32_t)n, group, PURPOSE_SAMPLE);
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
  best = block_max_u64<kThreads>(best);
  if (threadIdx.x == 0) a.bestpart[tile] = best;
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
  for (int i = lane; i < a.nch2; i += kWave) {
    const unsigned long long k = a.bestpart[(size_t)b * a.nch2 + i];
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
      const float E = exp2_variate(blk.w[v & 3]);
      const unsigned long long k = pack_key(fmaf(z, a.c, -__builtin_amdgcn_logf(E)), (uint32_t)v);
      best = k > best ? k : best;
    }
    best = wave_max_u64(best);
  }
  if (lane == 0) a.out_tokens[(size_t)b * (a.gamma + 1) + n] = (int32_t)packed_index(best);
}

}  // namespace sv
