// Verification kernels, dense path (no top-k filter).
//
//   k_stats   one block per (row pair, vocabulary chunk): streams draft row j and
//             target row j of a sequence, producing partial base-2 softmax
//             statistics (R, S) for both.  The last block of a sequence merges
//             the partials, evaluates every acceptance ratio in registers,
//             ballots the accept bits and finds the first rejection.
//   k_sample  one block per (sequence, vocabulary chunk) over the row chosen by
//             the first rejection: Gumbel-max over the residual max(0, q - p),
//             or over the target's row gamma when every draft was kept.  The
//             last block of a sequence writes the sampled token.
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
  float4 *seqstat;         // [B] stats of the row to resample
  int32_t *nseq;           // [B] n (or -1)
  unsigned int *cnt1;      // [B]
  unsigned int *cnt2;      // [B]
  unsigned long long *best;  // [B]
  int32_t nch, cv;         // pass-1 chunks per row, vectors per chunk
  int32_t nch2, cv2;       // pass-2 chunks per row, vectors per chunk
  // top-k path
  uint4 *rowinfo;          // [B][2*gamma+1] {thr lo, thr hi, R bits, S bits}
  int2 *lists;             // [B][2*gamma+1][K] (index, logit bits) or null
  unsigned int *cnt3;      // [B]
  int32_t klist;           // K when lists are kept, else 0
};

__device__ __forceinline__ uint32_t seq_of(const Args &a, int b) {
  return (uint32_t)(a.seq_offset + (uint64_t)b);
}

__device__ __forceinline__ size_t esz_of(int dt) { return dt == DT_BF16 ? 2 : 4; }

template <int DT>
__device__ __forceinline__ const void *target_row(const Args &a, int b, int j) {
  return (const char *)a.target + ((size_t)b * (a.gamma + 1) + j) * (size_t)a.V * Elem<DT>::kSize;
}
template <int DT>
__device__ __forceinline__ const void *draft_row(const Args &a, int b, int j) {
  return (const char *)a.draft + ((size_t)b * a.gamma + j) * (size_t)a.V * Elem<DT>::kSize;
}

// ---------------------------------------------------------------------------
// Sequence finalisation after pass 1 (one block, wave 0 does the work).
// Lane j holds position j: it merges that position's partial statistics,
// evaluates q_j(t_j) / p_j(t_j) and draws u_j; a 64-wide ballot of the accept
// bits gives the first rejection n.
// ---------------------------------------------------------------------------
template <int DT>
__device__ void finalize_dense(const Args &a, int b) {
  if (threadIdx.x >= kWave) return;
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
  const bool invalid = __ballot(active && !ok) != 0ull;
  int32_t *out = a.out_tokens + (size_t)b * (gamma + 1);
  if (invalid) {
    for (int i = lane; i <= gamma; i += kWave) out[i] = -1;
    if (lane == 0) {
      a.n_accepted[b] = -1;
      a.nseq[b] = -1;
      a.cnt1[b] = 0u;
    }
    if (active) {
      if (a.token_probs) {
        a.token_probs[((size_t)b * gamma + lane) * 2 + 0] = NAN;
        a.token_probs[((size_t)b * gamma + lane) * 2 + 1] = NAN;
      }
      if (a.accept_ur) {
        a.accept_ur[((size_t)b * gamma + lane) * 2 + 0] = NAN;
        a.accept_ur[((size_t)b * gamma + lane) * 2 + 1] = NAN;
      }
    }
    return;
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
    if (a.token_probs) {
      const float pt = pzero ? 0.0f : __builtin_amdgcn_exp2f(fmaf(zp, a.c, -Rp)) / Sp;
      const float qt = qzero ? 0.0f : __builtin_amdgcn_exp2f(fmaf(zq, a.c, -Rq)) / Sq;
      a.token_probs[((size_t)b * gamma + lane) * 2 + 0] = pt;
      a.token_probs[((size_t)b * gamma + lane) * 2 + 1] = qt;
    }
    if (a.accept_ur) {
      a.accept_ur[((size_t)b * gamma + lane) * 2 + 0] = u;
      a.accept_ur[((size_t)b * gamma + lane) * 2 + 1] = ratio;
    }
  }
  const unsigned long long mask = __ballot(active && accept);
  // first position whose accept bit is clear; gamma when all gamma are set
  const int n = (mask == ~0ull) ? kWave : __builtin_ctzll(~mask);
  const int nn = n < gamma ? n : gamma;

  if (active && lane == nn) a.seqstat[b] = make_float4(Rp, Sp, Rq, Sq);
  for (int i = lane; i <= gamma; i += kWave) {
    if (i < nn) out[i] = a.tokens[(size_t)b * gamma + i];
    else if (i > nn) out[i] = -1;
  }
  if (lane == 0) {
    a.n_accepted[b] = nn;
    a.nseq[b] = nn;
    a.cnt1[b] = 0u;
  }
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
  const int nvec = (a.V + NE - 1) / NE;
  const int v0 = ch * a.cv;
  const int v1 = min(nvec, v0 + a.cv);
  const float c = a.c;

  float Rp = -INFINITY, Sp = 0.0f, Rq = -INFINITY, Sq = 0.0f;
  for (int base = v0 + (int)threadIdx.x; base < v1; base += kThreads * U) {
    float zp[U][NE], zq[U][NE];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int iv = base + u * kThreads;
      if (iv < v1) {
        P.load_vec(iv, zp[u]);
        Q.load_vec(iv, zq[u]);
      } else {
#pragma unroll
        for (int e = 0; e < NE; ++e) zp[u][e] = zq[u][e] = -INFINITY;
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int iv = base + u * kThreads;
      if ((iv + 1) * NE > a.V) {  // the row's tail vector: mask entries >= V
#pragma unroll
        for (int e = 0; e < NE; ++e)
          if (iv * NE + e >= a.V) zp[u][e] = zq[u][e] = -INFINITY;
      }
      accumulate<NE>(Rp, Sp, zp[u], c);
      accumulate<NE>(Rq, Sq, zq[u], c);
    }
  }
  block_merge_stats2<kThreads>(Rp, Sp, Rq, Sq);
  if (threadIdx.x == 0) a.part[tile] = make_float4(Rp, Sp, Rq, Sq);
  if (arrive_last(&a.cnt1[b], (unsigned int)(a.gamma * a.nch))) finalize_dense<DT>(a, b);
}

// ---------------------------------------------------------------------------
// Gumbel-max pieces.  Residual: weight r_v = q_v - p_v > 0, key r_v / E_v (the
// exponential race, monotone in ln r_v - ln E_v).  Bonus: key z_v c - log2 E_v
// (monotone in ln q_v - ln E_v).
// ---------------------------------------------------------------------------
template <int DT>
__device__ unsigned long long sample_fallback_q(const Args &a, int b, int pos, const Row<DT> &Q);

template <int DT>
__global__ __launch_bounds__(kThreads) void k_sample(Args a) {
  constexpr int NE = Elem<DT>::kVec;
  const int tile = blockIdx.x;
  const int b = tile / a.nch2;
  const int ch = tile - b * a.nch2;
  const int n = a.nseq[b];
  if (n < 0) return;  // invalid sequence: already written
  const int gamma = a.gamma;
  const bool residual = n < gamma;
  const uint32_t seq = seq_of(a, b);
  const float c = a.c;

  const Row<DT> Q(target_row<DT>(a, b, n), a.V);
  const Row<DT> P(draft_row<DT>(a, b, residual ? n : 0), a.V);
  const float4 st = residual ? a.seqstat[b] : make_float4(0.f, 1.f, 0.f, 1.f);
  const float invSp = 1.0f / st.y, invSq = 1.0f / st.w;

  const int nvec = (a.V + NE - 1) / NE;
  const int v0 = ch * a.cv2;
  const int v1 = min(nvec, v0 + a.cv2);
  unsigned long long best = 0ull;
  for (int iv = v0 + (int)threadIdx.x; iv < v1; iv += kThreads) {
    float zq[NE], zp[NE];
    Q.load_vec(iv, zq);
    if (residual) P.load_vec(iv, zp);
#pragma unroll
    for (int g = 0; g < NE / 4; ++g) {
      float w[4];
      bool any = false;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int idx = iv * NE + g * 4 + e;
        const float zqe = zq[g * 4 + e];
        if (residual) {
          const float qv = (zqe == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(fmaf(zqe, c, -st.z)) * invSq;
          const float zpe = zp[g * 4 + e];
          const float pv = (zpe == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(fmaf(zpe, c, -st.x)) * invSp;
          w[e] = (idx < a.V) ? qv - pv : 0.0f;
          any |= w[e] > 0.0f;
        } else {
          w[e] = (idx < a.V && zqe != -INFINITY) ? zqe : -INFINITY;
          any |= w[e] != -INFINITY;
        }
      }
      if (!any) continue;
      const uint32_t group = (uint32_t)(iv * (NE / 4) + g);
      const Philox4 blk = stream_block(a.key0, a.key1, seq, (uint32_t)n, group, PURPOSE_SAMPLE);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t idx = group * 4u + (uint32_t)e;
        unsigned long long k = 0ull;
        if (residual) {
          if (w[e] > 0.0f) k = pack_key(w[e] / exponential_variate(blk.w[e]), idx);
        } else {
          if (w[e] != -INFINITY)
            k = pack_key(fmaf(w[e], c, -__builtin_amdgcn_logf(exponential_variate(blk.w[e]))), idx);
        }
        best = k > best ? k : best;
      }
    }
  }
  best = block_max_u64<kThreads>(best);
  if (threadIdx.x == 0 && best != 0ull) atomicMax(&a.best[b], best);
  if (arrive_last(&a.cnt2[b], (unsigned int)a.nch2)) {
    __shared__ unsigned long long fin;
    if (threadIdx.x == 0) fin = atomicAdd(&a.best[b], 0ull);
    __syncthreads();
    unsigned long long k = fin;
    if (k == 0ull) k = sample_fallback_q<DT>(a, b, n, Q);  // empty residual: sample q_n
    if (threadIdx.x == 0) {
      a.out_tokens[(size_t)b * (gamma + 1) + n] = (int32_t)packed_index(k);
      a.best[b] = 0ull;
      a.cnt2[b] = 0u;
    }
  }
}

// Gumbel-max over a whole target row by one block (rare path).
template <int DT>
__device__ unsigned long long sample_fallback_q(const Args &a, int b, int pos, const Row<DT> &Q) {
  const uint32_t seq = seq_of(a, b);
  unsigned long long best = 0ull;
  for (int v = threadIdx.x; v < a.V; v += kThreads) {
    const float z = Q.load_one(v);
    if (z == -INFINITY) continue;
    const Philox4 blk = stream_block(a.key0, a.key1, seq, (uint32_t)pos, (uint32_t)v >> 2, PURPOSE_SAMPLE);
    const float E = exponential_variate(blk.w[v & 3]);
    const unsigned long long k = pack_key(fmaf(z, a.c, -__builtin_amdgcn_logf(E)), (uint32_t)v);
    best = k > best ? k : best;
  }
  return block_max_u64<kThreads>(best);
}

// Zero-fill (workspace initialisation).
__global__ void k_zero(u32x4 *p, size_t n16, uint32_t *tail, size_t ntail) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n16) p[i] = u32x4{0u, 0u, 0u, 0u};
  if (i < ntail) tail[i] = 0u;
}

}  // namespace sv
