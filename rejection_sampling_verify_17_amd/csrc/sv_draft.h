// The two ends of a speculative step around verification: drawing the draft
// tokens, and counting how many of them a step kept.
//
// Page "추측 디코딩: 큰 모델을 빠르게 돌리는 법" (ai-trend.me), section "어떻게
// 작동하나": the small model first proposes gamma tokens, each drawn from its
// own adjusted distribution (temperature, top-k, arg-max), and only then does
// the large model verify them.
//
// k_draft_sample: one block per draft row (b, j).  Token j of sequence b is
// drawn from p_j = softmax(topk(z) / T) by Gumbel-max on Philox words of
// purpose 2 (DRAFT) at (seq = seq_offset + b, pos = j, v): the arg-max over the
// kept entries of z_v c - log2 E2_v, which orders like ln p_v - ln E_v
// (E2 = E / ln 2, the exponential variate in base 2); ties go to the smaller
// index.  Without top-k every entry is kept and the row is read once, in
// groups of four entries that share one Philox block; with top-k the exact
// K-th largest key comes from the top-k path's select (then the nucleus cut,
// when on) and only the kept entries draw variates.  T = 0 (arg-max mode):
// the first largest logit.
//
// k_accept_hist: one block counts n_accepted into gamma + 2 bins.
#pragma once

#include "sv_topk.h"

namespace sv {

// RADIX: the nucleus without top-k or over more than kTopkThreads kept
// entries (see topk_row).
template <int DT, bool RADIX>
__global__ __launch_bounds__(kTopkThreads) void k_draft_sample(Args a) {
  __shared__ TopkShared sh;
  const int row = blockIdx.x;  // b * gamma + j
  const int b = row / a.gamma, j = row - b * a.gamma;
  if (b >= a.B) return;  // never taken: the grid is B * gamma
  const Row<DT> P(draft_row<DT>(a, b, j), a.V);
  const StreamRow<DT> src(P, a.V);
  const uint32_t seq = seq_of(a, b);
  unsigned long long best = 0ull;
  if (a.argmax) {
    // arg-max mode: the first largest logit
    src.for_each([&](float z, int v) {
      const unsigned long long k = entry_key(z == 0.0f ? 0.0f : z, (uint32_t)v);  // -0 counts as +0
      best = k > best ? k : best;
    });
  } else if (a.top_k > 0 || a.top_p < 1.0f) {
    // kept set: the exact top-K threshold (every entry without top-k), raised
    // by the nucleus cut when on
    const TopkRow sel = topk_row<RADIX>(sh, src, a.top_k, a.c, a.top_p, nullptr, a.V);
    auto consider = [&](float z, uint32_t v) {
      if (z == -INFINITY || entry_key(z, v) < sel.thr) return;
      const Philox4 blk = stream_block(a.key0, a.key1, seq, (uint32_t)j, v >> 2, PURPOSE_DRAFT);
      const float E = exp2_variate(word_of(blk, v & 3u));
      const unsigned long long k = pack_key(fmaf(z, a.c, -__builtin_amdgcn_logf(E)), v);
      best = k > best ? k : best;
    };
    if (sel.in_lds) {
      for (unsigned int i = threadIdx.x; i < sel.ncand; i += kTopkThreads) {
        const unsigned long long key = sh.cand[i];
        consider(from_orderable((uint32_t)(key >> 32)), 0xFFFFFFFFu - (uint32_t)(key & 0xFFFFFFFFull));
      }
    } else {
      // a kept set too large for LDS: the dense Gumbel pass over the row,
      // one Philox block per four entries, entries outside the set skipped
      const PhiloxStream ps(a.key0, a.key1, seq, (uint32_t)j, PURPOSE_DRAFT);
      best = gumbel_dense_row<DT, kTopkThreads, true>(P, a.V, a.c, ps, 0, a.ngb, sel.thr);
    }
  } else {
    const PhiloxStream ps(a.key0, a.key1, seq, (uint32_t)j, PURPOSE_DRAFT);
    best = gumbel_dense_row<DT, kTopkThreads, false, true>(P, a.V, a.c, ps, 0, a.ngb);
  }
  best = block_max_u64_sh<kTopkThreads>(best, sh.red_u);
  if (threadIdx.x == 0) a.drafted[row] = best == 0ull ? 0 : (int32_t)packed_index(best);
}

// Counts of n_accepted: hist[0] sequences flagged invalid (n < 0, or n >
// gamma, which no call writes), hist[1 + i] sequences with n = i.
__global__ __launch_bounds__(256) void k_accept_hist(const int32_t *n, int B, int gamma, int32_t *hist) {
  __shared__ int cnt[66];  // gamma <= 64
  for (int i = threadIdx.x; i < gamma + 2; i += 256) cnt[i] = 0;
  __syncthreads();
  for (int b = threadIdx.x; b < B; b += 256) {
    const int v = n[b];
    atomicAdd(&cnt[(v < 0 || v > gamma) ? 0 : v + 1], 1);
  }
  __syncthreads();
  for (int i = threadIdx.x; i < gamma + 2; i += 256) hist[i] = cnt[i];
}

}  // namespace sv
