// Verification in the arg-max mode (temperature 0).
//
// At temperature 0 each distribution is the point mass on its row's largest
// logit, the smaller vocabulary index among equal logits (page "추측 디코딩: 큰
// 모델을 빠르게 돌리는 법" (ai-trend.me), section "어떻게 작동하나": arg-max
// decoding is sampling from an adjusted distribution).  The rule of page
// "스펙큘러티브 디코딩 — 작은 모델이 먼저 쓰고 큰 모델이 검사한다" §1 then needs no
// random number and no draft row: q_j(t_j) > 0 only for t_j = argmax q_j and
// p_j(t_j) is 0 or 1, so draft j is kept iff t_j = argmax q_j.  At the first
// rejected position n the residual max(0, q_n - p_n) is the point mass on
// argmax q_n, or empty when argmax p_n = argmax q_n, and then q_n itself is
// sampled: the same token.  With all gamma kept the bonus is argmax q_gamma.
// So the token after the kept prefix is always the arg-max of the target row
// at that position, and every target row is read at most once.
//
// Target rows 0..gamma are walked in windows [0, 1), [1, 3), [3, 7), [7, 15),
// ... (a window that would leave one row over runs to row gamma, the bonus
// row, and the last window always ends there); k_greedy_step(window)
// runs nch blocks per row of the window for every sequence.  Each block first
// judges the previous window of its sequence (wave 0, lane l: row p0 + l's
// arg-max merged from the chunk keys of the previous launch, compared with the
// drafted token; row gamma always ends the sequence; a ballot finds the first
// mismatch).  If the sequence is still alive, the block writes the packed
// arg-max key of its chunk; the lead block writes the per-sequence state and,
// when the sequence ended, its outputs.  A last launch without rows only
// judges.  Windows after the one that holds a sequence's first mismatch are
// never read for it.  The first launch has nothing to judge: it reads row 0
// of every sequence at once and checks the drafted tokens afterwards.
//
// Key of entry v: (orderable(z) << 32) | (2^32 - 1 - v), so the u64 maximum is
// the largest logit with the smallest index among equals; -0 counts as +0, as
// in an ordinary floating-point comparison.
#pragma once

#include "sv_kernels.h"

namespace sv {

constexpr int kGreedyThreads = 512;
constexpr int kGreedyU = 4;  // 16-byte vectors in flight per thread

// Arg-max key of target row j of sequence b over vectors [v0, v1).  Each
// thread keeps the largest vector maximum it has seen (strictly larger only,
// so its earliest vector wins among equals) and afterwards finds the first
// entry of that vector equal to it.  Entries outside the row are masked to
// -inf; a chunk with nothing but -inf returns 0 (no key).
template <int DT>
__device__ unsigned long long chunk_argmax(const Args &a, int b, int j, int v0, int v1) {
  constexpr int NE = Elem<DT>::kVec;
  constexpr int U = kGreedyU;
  const Row<DT> Q(target_row<DT>(a, b, j), a.V);
  const int V = a.V;
  const int ilo = (Q.s + NE - 1) / NE;  // vectors [ilo, ihi) lie inside the row
  const int ihi = (V + Q.s) / NE;
  float bestz = -INFINITY;
  int bestv = -1;
  for (int base = v0 + (int)threadIdx.x; base < v1; base += kGreedyThreads * U) {
    float z[U][NE];
#pragma unroll
    for (int u = 0; u < U; ++u) Q.load_vec(base + u * kGreedyThreads, z[u]);
    const int top = base + (U - 1) * kGreedyThreads;
    const bool edge = base < ilo || top >= ihi || top >= v1;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int iv = base + u * kGreedyThreads;
      if (edge) {
        const int e0 = iv * NE - Q.s;
#pragma unroll
        for (int e = 0; e < NE; ++e)
          if (iv >= v1 || e0 + e < 0 || e0 + e >= V) z[u][e] = -INFINITY;
      }
      float m = z[u][0];
#pragma unroll
      for (int e = 1; e < NE; ++e) m = fmaxf(m, z[u][e]);
      const bool take = m > bestz;
      bestz = take ? m : bestz;
      bestv = take ? iv : bestv;
    }
  }
  unsigned long long key = 0ull;
  if (bestv >= 0) {
    float z[NE];
    Q.load_vec(bestv, z);
    const int e0 = bestv * NE - Q.s;
    int idx = -1;
#pragma unroll
    for (int e = NE - 1; e >= 0; --e)  // the first in-row entry equal to the maximum
      if (e0 + e >= 0 && e0 + e < V && z[e] == bestz) idx = e0 + e;
    const float zc = bestz == 0.0f ? 0.0f : bestz;  // -0 -> +0
    key = pack_key(zc, (uint32_t)idx);
  }
  return block_max_u64<kGreedyThreads>(key);
}

// Token of a merged key (0: a row of -inf only, outside the documented
// inputs; index 0, as a scan that keeps the first of equal maxima gives).
__device__ __forceinline__ int32_t key_token(unsigned long long k) {
  return k == 0ull ? 0 : (int32_t)packed_index(k);
}

// One launch of the arg-max mode.  Rows [w0, w1) of every sequence (none in
// the last launch), nch chunks per row; the previous window [p0, w0) was
// measured with nch_prev chunks per row.  Grid: B * max(1, w1 - w0) * nch.
template <int DT>
__global__ __launch_bounds__(kGreedyThreads) void k_greedy_step(Args a, int launch, int p0, int w0, int w1,
                                                              int nch, int nch_prev) {
  __shared__ int sh_alive;
  const int gamma = a.gamma;
  const int rows = w1 - w0;
  const int per_seq = rows > 0 ? rows * nch : 1;
  const int b = blockIdx.x / per_seq;
  const int rc = blockIdx.x - b * per_seq;
  const bool lead = rc == 0;
  const int lane = threadIdx.x % kWave;
  if (b >= a.B) return;  // never taken: the grid is B * per_seq
  int32_t *state = a.state;
  int32_t *out = a.out_tokens + (size_t)b * (gamma + 1);
  if (launch == 0) {
    // every sequence is read first (row 0 of an invalid sequence is read
    // for nothing); the drafted tokens are checked after, so no wave waits
    // for them before its stream starts
    const int cv = (a.nvec + nch - 1) / nch;
    const int v0 = rc * cv;  // window [0, 1): rc is the chunk
    const unsigned long long key = chunk_argmax<DT>(a, b, 0, v0, min(a.nvec, v0 + cv));
    if (threadIdx.x == 0) a.gpart[(size_t)b * (gamma + 1) * a.gstride + rc] = key;
    if (lead && threadIdx.x < kWave) {
      const bool ok = tokens_valid(a, b, lane);
      for (int k = lane; k < gamma; k += kWave) write_diag(a, b, k, NAN, NAN, NAN, NAN);
      if (!ok) write_invalid(a, b, lane);
      if (lane == 0) state[b] = ok ? 1 : 0;  // half 0: launch 0
    }
    return;
  }
  if (threadIdx.x < kWave) {
    int alive = state[(size_t)((launch - 1) & 1) * a.B + b] > 0;
    if (alive) {
      // lane l: row p0 + l of the previous window
      const int nj = w0 - p0;
      const int j = p0 + lane;
      unsigned long long key = 0ull;
      int tok = -1;
      if (lane < nj) {
        const unsigned long long *kp = a.gpart + ((size_t)b * (gamma + 1) + j) * a.gstride;
        for (int c = 0; c < nch_prev; ++c) {
          const unsigned long long k = kp[c];
          key = k > key ? k : key;
        }
        if (j < gamma) tok = a.tokens[(size_t)b * gamma + j];
      }
      const int am = key_token(key);
      const unsigned long long miss = __ballot(lane < nj && (j == gamma || tok != am));
      if (miss != 0ull) {
        const int k = __builtin_ctzll(miss);
        const int n = p0 + k;
        const int token = __shfl(am, k, kWave);
        alive = 0;
        if (lead) {
          for (int i = lane; i <= gamma; i += kWave) {
            if (i < n) out[i] = a.tokens[(size_t)b * gamma + i];
            else if (i == n) out[i] = token;
            else out[i] = -1;
          }
          if (lane == 0) {
            a.n_accepted[b] = n;
            a.nseq[b] = n;
          }
        }
      }
    }
    if (lead && lane == 0) state[(size_t)(launch & 1) * a.B + b] = alive ? 1 : 0;
    if (threadIdx.x == 0) sh_alive = alive;
  }
  __syncthreads();
  if (!sh_alive || rows <= 0) return;
  const int r = rc / nch, ch = rc - r * nch;
  const int j = w0 + r;
  const int cv = (a.nvec + nch - 1) / nch;
  const int v0 = ch * cv;
  const unsigned long long key = chunk_argmax<DT>(a, b, j, v0, min(a.nvec, v0 + cv));
  if (threadIdx.x == 0) a.gpart[((size_t)b * (gamma + 1) + j) * a.gstride + ch] = key;
}

}  // namespace sv
