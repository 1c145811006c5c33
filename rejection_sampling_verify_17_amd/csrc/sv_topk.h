// Verification kernels with the top-k filter (0 < K < V).
//
// Top-k keeps exactly the K entries of a row with the largest raw logit; among
// equal logits the smaller vocabulary index is kept.  Every entry gets the
// 64-bit key  (orderable(z) << 32) | (2^32 - 1 - v),  unique per row and
// ordered like "larger logit, then smaller index"; the kept set is the K
// largest keys, i.e. all keys >= the K-th largest ("threshold").
//
// The drafts are judged left to right; positions are walked in windows
// [0, 1), [1, 3), [3, 7), [7, 15), ... (a window that would leave a single
// position over runs to gamma) and k_topk_step(window) runs one block per row
// of the window (draft and target rows of every position):
//   first window   each block selects its row: threshold by an LDS radix
//                  select, base-2 softmax statistics (R, S) over the kept
//                  entries and, for small K, the kept list.
//   later windows  every block of a sequence alive at the previous window
//                  first judges it (wave 0, lane l: position p0 + l,
//                  membership of t in both kept sets, ratio in registers,
//                  Philox u; a ballot finds the first rejection); all kept:
//                  each selects its row of the new window; rejected at n: the
//                  lead block draws the replacement from the residual over
//                  the target row's kept list of position n; all kept and no
//                  window left: the lead block selects target row gamma and
//                  draws the bonus token over its kept entries.  The deciding
//                  block writes the token itself.
// With low acceptance few sequences reach the wide windows, and a launch over
// few rows costs about as much as one over many.
//
// Selection: a lower bound L on the K-th largest logit comes from the
// per-thread maxima (K threads each own an entry >= their maximum's K-th
// largest, so at least K entries are >= L); entries >= L are gathered into LDS
// and the exact K-th largest key is selected among them.  If more than kCap
// entries pass the bound (heavy ties), the select runs over the row itself.
//
// Page "추측 디코딩: 큰 모델을 빠르게 돌리는 법" (ai-trend.me), section
// "어떻게 작동하나": top-k sampling reduces to sampling from an adjusted
// distribution, which this filter builds for both p and q.
#pragma once

#include "sv_kernels.h"

namespace sv {

constexpr int kTopkThreads = 1024;
constexpr int kCap = 2048;  // candidate entries held in LDS

struct TopkShared {
  unsigned long long cand[kCap];
  unsigned int hist[256];
  unsigned int tmax[kTopkThreads];
  unsigned int ncand;
  unsigned int nkept;
  unsigned int nhot;
  unsigned long long sel_prefix;
  unsigned int sel_k;
  int sel_done;
  float red_f[kTopkThreads / kWave];
  unsigned long long red_u[kTopkThreads / kWave];
  unsigned long long red_low[kTopkThreads / kWave];  // nucleus cut: mass of the entries it leaves out of its histograms
  int bcast_n;
  unsigned long long srt[kTopkThreads];  // nucleus cut: the kept keys, sorted
  int cut;
  float cut_sum;
};

// -0 is keyed as +0: equal logits, so the smaller index ranks first, as in an
// ordinary floating-point comparison.
__device__ __forceinline__ unsigned long long entry_key(float z, uint32_t v) {
  const float zc = z == 0.0f ? 0.0f : z;
  return ((unsigned long long)orderable(zc) << 32) | (unsigned long long)(0xFFFFFFFFu - v);
}

// Radix select, most significant byte first: the K-th largest (1-based, with
// multiplicity) of the keys `src` enumerates, over bits [lo, hi) (multiples of
// 8; bits >= hi are equal across all keys).  If at some byte exactly the
// remaining rank's worth of keys share the prefix, it stops early with the low
// bits cleared: every key that shares the prefix is then within the K largest,
// so among the keys `src` enumerates (when unique) "key >= result" still selects
// exactly the K largest.  Keys outside that set may also pass the cleared
// threshold, so callers that test other keys need the exact K-th largest.
// NT threads; Sh provides hist[256], sel_prefix, sel_k, sel_done in LDS.
template <int NT, class Sh, class Src>
__device__ __forceinline__ unsigned long long radix_select(Sh &sh, const Src &src, unsigned int K, int hi, int lo) {
  const int tid = threadIdx.x;
  unsigned long long prefix = 0ull, mask = 0ull;
  unsigned int k = K;
  for (int shift = hi - 8; shift >= lo; shift -= 8) {
    for (int i = tid; i < 256; i += NT) sh.hist[i] = 0u;
    __syncthreads();
    src.for_each([&](unsigned long long key) {
      if ((key & mask) == prefix) atomicAdd(&sh.hist[(unsigned int)(key >> shift) & 255u], 1u);
    });
    __syncthreads();
    if (tid < kWave) {
      const int lane = tid;
      const unsigned int h0 = sh.hist[4 * lane], h1 = sh.hist[4 * lane + 1];
      const unsigned int h2 = sh.hist[4 * lane + 2], h3 = sh.hist[4 * lane + 3];
      const unsigned int s = h0 + h1 + h2 + h3;
      // inclusive suffix sum over lanes (higher lanes hold higher digits)
      unsigned int incl = s;
#pragma unroll
      for (int off = 1; off < kWave; off <<= 1) {
        const unsigned int y = __shfl_down(incl, off, kWave);
        if (lane + off < kWave) incl += y;
      }
      const unsigned int above = incl - s;  // keys with a digit in a higher lane
      if (above < k && k <= incl) {
        // this lane's four digits, highest first
        const unsigned int a3 = above, a2 = a3 + h3, a1 = a2 + h2, a0 = a1 + h1;
        int i;
        unsigned int ab, h;
        if (a3 + h3 >= k) { i = 3; ab = a3; h = h3; }
        else if (a2 + h2 >= k) { i = 2; ab = a2; h = h2; }
        else if (a1 + h1 >= k) { i = 1; ab = a1; h = h1; }
        else { i = 0; ab = a0; h = h0; }
        sh.sel_prefix = (unsigned long long)(4 * lane + i);
        sh.sel_k = k - ab;
        sh.sel_done = (h == k - ab);
      }
    }
    __syncthreads();
    const unsigned long long d = sh.sel_prefix;
    k = sh.sel_k;
    const int done = sh.sel_done;
    __syncthreads();
    prefix |= d << shift;
    mask |= 255ull << shift;
    if (done) break;
  }
  return prefix;
}

template <int NT> struct LdsKeys {
  const unsigned long long *keys;
  unsigned int n;
  template <class F> __device__ __forceinline__ void for_each(F f) const {
    for (unsigned int i = threadIdx.x; i < n; i += NT) f(keys[i]);
  }
};

template <int NT> struct LdsMax32 {  // per-thread maxima as 32-bit keys in the high word
  const unsigned int *m;
  template <class F> __device__ __forceinline__ void for_each(F f) const {
    for (unsigned int i = threadIdx.x; i < (unsigned int)NT; i += NT) f((unsigned long long)m[i] << 32);
  }
};

// Entry source for a row of V logits: for_each(f) calls f(z, v) once for every
// entry of the row (any order), kU 16-byte loads in flight per thread.
template <int DT> struct StreamRow {
  static constexpr int NE = Elem<DT>::kVec;
  static constexpr int kU = 2;
  static constexpr int kUCut = 8;  // loads in flight in the passes of the mass-weighted nucleus cut (one block per compute unit there)
  const Row<DT> &row;
  int e0, e1;  // entries [e0, e1) of the row
  __device__ __forceinline__ StreamRow(const Row<DT> &r, int V) : row(r), e0(0), e1(V) {}
  __device__ __forceinline__ StreamRow(const Row<DT> &r, int lo, int hi) : row(r), e0(lo), e1(hi) {}
  __device__ __forceinline__ int iv0() const { return (e0 + row.s) / NE; }          // vector holding entry e0
  __device__ __forceinline__ int iv1() const { return (e1 - 1 + row.s) / NE + 1; }  // one past the vector holding e1 - 1
  // Vectors thread t visits in for_each: iv0 + t + kTopkThreads i, i < this.
  __device__ __forceinline__ int vectors_per_thread() const {
    return (iv1() - iv0() + kTopkThreads - 1) / kTopkThreads;
  }
  // f(z, v) for the entries of the i-th vector thread t visits in for_each.
  template <class F> __device__ __forceinline__ void for_vector_of(int t, int i, F f) const {
    const int iv = iv0() + t + kTopkThreads * i;
    if (iv >= iv1()) return;
    float z[NE];
    decode<DT>(row.raw(iv), z);
    const int ev = iv * NE - row.s;
#pragma unroll
    for (int e = 0; e < NE; ++e) {
      const int v = ev + e;
      if (v >= e0 && v < e1) f(z[e], v);
    }
  }
  template <class F> __device__ __forceinline__ void for_each(F f) const { for_each_u<kU>(f); }
  // The same with U loads in flight per thread.
  template <int U, class F> __device__ __forceinline__ void for_each_u(F f) const {
    const int iv0 = this->iv0(), iv1 = this->iv1();
    for (int base = iv0 + (int)threadIdx.x; base < iv1; base += kTopkThreads * U) {
      u32x4 d[U];
#pragma unroll
      for (int u = 0; u < U; ++u) d[u] = row.raw(base + u * kTopkThreads);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float z[NE];
        decode<DT>(d[u], z);
        const int ev = (base + u * kTopkThreads) * NE - row.s;
        if (ev >= e0 && ev + NE <= e1) {  // the whole vector is inside (no test per entry)
#pragma unroll
          for (int e = 0; e < NE; ++e) f(z[e], ev + e);
        } else {
#pragma unroll
          for (int e = 0; e < NE; ++e) {
            const int v = ev + e;
            if (v >= e0 && v < e1 && base + u * kTopkThreads < iv1) f(z[e], v);
          }
        }
      }
    }
  }
};

// Keys of every entry of a source.
template <class Src> struct SrcKeys {
  const Src &src;
  template <class F> __device__ __forceinline__ void for_each(F f) const {
    src.for_each([&](float z, int v) { f(entry_key(z, (uint32_t)v)); });
  }
};

// Result of selecting a row: the threshold key and the base-2 statistics over
// the kept entries.  If `list` is given (K <= klist), the kept entries are
// written there as (index, logit bits) in no particular order.
struct TopkRow {
  unsigned long long thr;
  float R, S;
  bool in_lds;          // kept entries are among sh.cand[0..ncand) (else scan the row)
  unsigned int ncand;
};

// Exact threshold of a top-K select over the entries `src` enumerates: the
// K-th largest key (K <= number of entries).  Leaves the candidates in LDS
// (sh.cand[0..ncand) when in_lds; otherwise they are the source's entries).
struct Selected {
  unsigned long long thr;
  bool in_lds;
  unsigned int ncand;
  bool one_wave;  // K <= ncand <= 64 candidates in LDS: thr not computed, one wave finishes the row
};

template <class Src>
__device__ __forceinline__ Selected select_threshold(TopkShared &sh, const Src &src, int K) {
  const int tid = threadIdx.x;

  // Phase A: per-thread maximum logit (a float max per entry).
  float zmax = -INFINITY;
  bool any = false;
  src.for_each([&](float z, int) {
    zmax = fmaxf(zmax, z);
    any = true;
  });
  sh.tmax[tid] = any ? orderable(zmax) : 0u;  // 0: no entry (every real key is > 0)
  if (tid == 0) { sh.ncand = 0u; sh.nkept = 0u; sh.nhot = 0u; }
  __syncthreads();

  // Phase B: lower bound L = K-th largest per-thread maximum: K threads own an
  // entry >= L each, so the K-th largest logit of the row is >= L.
  // The select may clear low bits of L (still a lower bound as an integer).
  // Every bound at or below orderable(-inf), including 0 (fewer than K
  // threads hold entries), admits every entry: cleared bits there would not
  // decode to a float.
  unsigned int L = 0u;
  if (K <= kTopkThreads) L = (unsigned int)(radix_select<kTopkThreads>(sh, LdsMax32<kTopkThreads>{sh.tmax}, (unsigned)K, 64, 32) >> 32);
  const bool take_all = L <= orderable(-INFINITY);
  const float Lf = take_all ? -INFINITY : from_orderable(L);

  // Phase C (a second pass): gather every entry with logit >= L into LDS as
  // its 64-bit key (-0 also passes a +0 bound, which only adds a candidate).
  // Such an entry lies at or below its thread's maximum, so only the vectors
  // of threads whose maximum reaches L (about K threads) are read again, all
  // of them at once: the block deals them out one vector per thread.
  auto gather = [&](float z, int v) {
    if (take_all || z >= Lf) {
      const unsigned int slot = atomicAdd(&sh.ncand, 1u);
      if (slot < (unsigned int)kCap) sh.cand[slot] = entry_key(z, (uint32_t)v);
    }
  };
  if (take_all) {
    src.for_each(gather);
  } else {
    // the per-thread maxima are read; their array now lists those threads
    if (any && zmax >= Lf) sh.tmax[atomicAdd(&sh.nhot, 1u)] = (unsigned int)tid;
    __syncthreads();
    const int per = src.vectors_per_thread();
    const int nvis = (int)sh.nhot * per;
    for (int i = tid; i < nvis; i += kTopkThreads) src.for_vector_of((int)sh.tmax[i / per], i % per, gather);
  }
  __syncthreads();
  const unsigned int ncand = sh.ncand;
  // fewer than K candidates cannot happen with a true lower bound; should it,
  // the select runs over the row itself rather than over too few keys
  const bool in_lds = ncand <= (unsigned int)kCap && ncand >= (unsigned int)K;
  // a wave can sort this few candidates in registers (topk_row finishes)
  if (in_lds && ncand <= (unsigned int)kWave && (int)ncand >= K) return Selected{0ull, true, ncand, true};

  // Phase D: threshold among the candidates.
  unsigned long long thr;
  if (in_lds) thr = radix_select<kTopkThreads>(sh, LdsKeys<kTopkThreads>{sh.cand, ncand}, (unsigned)K, 64, 0);
  else thr = radix_select<kTopkThreads>(sh, SrcKeys<Src>{src}, (unsigned)K, 64, 0);
  // The select may stop with the low bits of `thr` cleared; that separates
  // the K kept entries from the other candidates but not from every entry of
  // the row, so the threshold is made exact: the smallest kept key.
  unsigned long long kmin = ~0ull;
  auto visit = [&](unsigned long long key) {
    if (key >= thr) kmin = key < kmin ? key : kmin;
  };
  if (in_lds) LdsKeys<kTopkThreads>{sh.cand, ncand}.for_each(visit);
  else SrcKeys<Src>{src}.for_each(visit);
  kmin = ~wave_max_u64(~kmin);
  if ((threadIdx.x % kWave) == 0) sh.red_u[threadIdx.x / kWave] = kmin;
  __syncthreads();
  kmin = sh.red_u[0];
  for (int i = 1; i < kTopkThreads / kWave; ++i) kmin = sh.red_u[i] < kmin ? sh.red_u[i] : kmin;
  __syncthreads();
  return Selected{kmin, in_lds, ncand, false};
}

// Base-2 softmax statistics over the kept entries (keys >= thr) of a key set;
// writes the kept entries to `list` when given.  FIXED: the keys sit in LDS in
// the order the gather's atomics handed out slots, which varies from run to
// run, so S is summed in 64-bit fixed point (every weight 2^(z c - R) is in
// (0, 1] and at most kCap of them are kept: scale 2^40, truncation below
// 2^-29 of S >= 1/2 in all) and the sum does not depend on that order.  A row
// scan visits its entries in a fixed order and sums in fp32.
template <bool FIXED, class Keys>
__device__ __forceinline__ TopkRow kept_stats(TopkShared &sh, const Keys &keys, unsigned long long thr, float c,
                                              int2 *list, int K) {
  const int tid = threadIdx.x;
  if (tid == 0) sh.nkept = 0u;
  float zmax = -INFINITY;
  keys.for_each([&](unsigned long long key) {
    if (key >= thr) zmax = fmaxf(zmax, from_orderable((uint32_t)(key >> 32)));
  });
  zmax = wave_max_f(zmax);
  if ((tid % kWave) == 0) sh.red_f[tid / kWave] = zmax;
  __syncthreads();
  zmax = sh.red_f[0];
  for (int i = 1; i < kTopkThreads / kWave; ++i) zmax = fmaxf(zmax, sh.red_f[i]);
  __syncthreads();
  const float R = (zmax == -INFINITY) ? -INFINITY : ceilf(zmax * c);
  float S = 0.0f;
  unsigned long long Sfix = 0ull;
  keys.for_each([&](unsigned long long key) {
    if (key >= thr) {
      const float z = from_orderable((uint32_t)(key >> 32));
      if (z != -INFINITY) {
        const float e = __builtin_amdgcn_exp2f(fmaf(z, c, -R));
        if (FIXED) Sfix += (unsigned long long)(e * 0x1p40f);
        else S += e;
      }
      if (list) {
        const unsigned int slot = atomicAdd(&sh.nkept, 1u);  // exactly K kept entries
        if (slot < (unsigned int)K)
          list[slot] = make_int2((int)(0xFFFFFFFFu - (uint32_t)(key & 0xFFFFFFFFull)), (int)__float_as_uint(z));
      }
    }
  });
  if (FIXED) {
#pragma unroll
    for (int off = kWave / 2; off > 0; off >>= 1) Sfix += __shfl_xor(Sfix, off, kWave);
    if ((tid % kWave) == 0) sh.red_u[tid / kWave] = Sfix;
    __syncthreads();
    Sfix = 0ull;
    for (int i = 0; i < kTopkThreads / kWave; ++i) Sfix += sh.red_u[i];
    S = (float)Sfix * 0x1p-40f;
  } else {
    S = wave_sum_f(S);
    if ((tid % kWave) == 0) sh.red_f[tid / kWave] = S;
    __syncthreads();
    S = 0.0f;
    for (int i = 0; i < kTopkThreads / kWave; ++i) S += sh.red_f[i];
  }
  __syncthreads();
  return TopkRow{thr, R, S, false, 0u};
}

// Nucleus cut (top-p) of a selected row: the kept entries (keys >= r.thr, K
// of them, K <= kTopkThreads) are sorted in the top-k order (larger logit,
// then smaller index), their base-2 weights 2^(z c - R) summed as a prefix,
// and the row keeps the shortest prefix whose mass reaches P of the total:
// the threshold rises to that prefix's last key and S becomes its sum (R
// still bounds every kept logit).  Every reader of the row tests keys
// against the threshold, so nothing else changes.
template <class Keys>
__device__ __forceinline__ void nucleus_cut(TopkShared &sh, const Keys &keys, float c, float P, TopkRow &r) {
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  if (tid == 0) {
    sh.nkept = 0u;
    sh.cut = kTopkThreads;
  }
  __syncthreads();
  keys.for_each([&](unsigned long long key) {
    if (key >= r.thr) {
      const unsigned int slot = atomicAdd(&sh.nkept, 1u);
      if (slot < (unsigned int)kTopkThreads) sh.srt[slot] = key;
    }
  });
  __syncthreads();
  const int n = (int)min(sh.nkept, (unsigned int)kTopkThreads);
  if (n <= kWave) {
    // up to 64 kept entries: wave 0 sorts them in registers (bitonic, by
    // shuffles) and scans them, with no block barrier in between
    if (wave == 0) {
      unsigned long long x = lane < n ? sh.srt[lane] : 0ull;  // 0 is below every real key
#pragma unroll
      for (int size = 2; size <= kWave; size <<= 1) {
#pragma unroll
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
          const unsigned long long y = __shfl_xor(x, stride, kWave);
          const bool desc = (lane & size) == 0, lower = (lane & stride) == 0;
          x = (lower == desc) ? (x > y ? x : y) : (x < y ? x : y);
        }
      }
      float e = 0.0f;
      if (lane < n) {
        const float z = from_orderable((uint32_t)(x >> 32));
        if (z != -INFINITY) e = __builtin_amdgcn_exp2f(fmaf(z, c, -r.R));
      }
      float s = e;
#pragma unroll
      for (int off = 1; off < kWave; off <<= 1) {
        const float y = __shfl_up(s, off, kWave);
        if (lane >= off) s += y;
      }
      const float total = __shfl(s, kWave - 1, kWave);
      const unsigned long long hit = __ballot(lane < n && s >= P * total);
      if (hit != 0ull) {
        const int m = __builtin_ctzll(hit);
        const unsigned long long km = __shfl(x, m, kWave);
        const float sm = __shfl(s, m, kWave);
        if (lane == 0) {
          sh.cut = m;
          sh.srt[0] = km;
          sh.cut_sum = sm;
        }
      }
    }
    __syncthreads();
    if (sh.cut < n) {
      r.thr = sh.srt[0];
      r.S = sh.cut_sum;
    }
    __syncthreads();
    return;
  }
  if (tid >= n) sh.srt[tid] = 0ull;  // below every real key: sorts last
  __syncthreads();
  // bitonic sort of the kTopkThreads keys, descending, one per thread
  for (int size = 2; size <= kTopkThreads; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      const int partner = tid ^ stride;
      if (partner > tid) {
        const unsigned long long x = sh.srt[tid], y = sh.srt[partner];
        const bool swap = ((tid & size) == 0) ? (x < y) : (x > y);
        if (swap) {
          sh.srt[tid] = y;
          sh.srt[partner] = x;
        }
      }
      __syncthreads();
    }
  }
  // inclusive prefix sum of the weights in that order
  float e = 0.0f;
  if (tid < n) {
    const float z = from_orderable((uint32_t)(sh.srt[tid] >> 32));
    if (z != -INFINITY) e = __builtin_amdgcn_exp2f(fmaf(z, c, -r.R));
  }
  float s = e;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const float y = __shfl_up(s, off, kWave);
    if (lane >= off) s += y;
  }
  if (lane == kWave - 1) sh.red_f[wave] = s;
  __syncthreads();
  float below = 0.0f, total = 0.0f;
  for (int w = 0; w < kTopkThreads / kWave; ++w) {
    if (w < wave) below += sh.red_f[w];
    total += sh.red_f[w];
  }
  const float cum = below + s;
  // the first entry whose prefix reaches P of the total
  const unsigned long long hit = __ballot(tid < n && cum >= P * total);
  if (lane == 0 && hit != 0ull) atomicMin(&sh.cut, wave * kWave + __builtin_ctzll(hit));
  __syncthreads();
  const int m = sh.cut;
  if (tid == m) sh.cut_sum = cum;
  __syncthreads();
  if (m < n) {
    r.thr = sh.srt[m];
    r.S = sh.cut_sum;
  }
  __syncthreads();
}

// Rows whose candidates fit one wave (K <= ncand <= 64): wave 0 sorts them
// in registers (bitonic network by shuffles, descending); the K-th key is the
// exact threshold, R comes from the first (largest) logit, S is the sum of
// the first K weights, the first K entries go to the list, and the nucleus
// cut, when on, is a prefix sum over the same lanes.  No block barrier but
// the final broadcast.
__device__ __forceinline__ TopkRow topk_one_wave(TopkShared &sh, unsigned int ncand, int K, float c, float top_p,
                                                 int2 *list) {
  const int tid = threadIdx.x, lane = tid % kWave;
  if (tid < kWave) {
    unsigned long long x = lane < (int)ncand ? sh.cand[lane] : 0ull;  // 0 is below every real key
#pragma unroll
    for (int size = 2; size <= kWave; size <<= 1) {
#pragma unroll
      for (int stride = size >> 1; stride > 0; stride >>= 1) {
        const unsigned long long y = __shfl_xor(x, stride, kWave);
        const bool desc = (lane & size) == 0, lower = (lane & stride) == 0;
        x = (lower == desc) ? (x > y ? x : y) : (x < y ? x : y);
      }
    }
    const float z = from_orderable((uint32_t)(x >> 32));
    const float zmax = __shfl(z, 0, kWave);
    const float R = (zmax == -INFINITY) ? -INFINITY : ceilf(zmax * c);
    const bool kept = lane < K;
    const float e = (kept && z != -INFINITY) ? __builtin_amdgcn_exp2f(fmaf(z, c, -R)) : 0.0f;
    if (list && kept) list[lane] = make_int2((int)(0xFFFFFFFFu - (uint32_t)(x & 0xFFFFFFFFull)), (int)__float_as_uint(z));
    // prefix sums of the kept weights in the sorted order
    float s = e;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const float y = __shfl_up(s, off, kWave);
      if (lane >= off) s += y;
    }
    int m = K - 1;
    if (top_p > 0.0f && top_p < 1.0f) {
      const float total = __shfl(s, K - 1, kWave);
      const unsigned long long hit = __ballot(kept && s >= top_p * total);
      if (hit != 0ull) m = __builtin_ctzll(hit);
    }
    const unsigned long long thr = __shfl(x, m, kWave);
    const float S = __shfl(s, m, kWave);
    if (lane == 0) {
      sh.srt[0] = thr;
      sh.cut_sum = S;
      sh.red_f[0] = R;
    }
  }
  __syncthreads();
  const TopkRow r{sh.srt[0], sh.red_f[0], sh.cut_sum, true, ncand};
  __syncthreads();
  return r;
}

// ---------------------------------------------------------------------------
// Nucleus cut over a large kept set (no top-k, or K > kTopkThreads): the kept
// entries are not sorted; the cut is found by a radix select weighted by
// mass.  Masses are 64-bit fixed point, 2^(z c - R) 2^fb with fb = 62 - (bits
// of V), so the total of at most V weights <= 1 stays below 2^62 and sums do
// not depend on the order atomics arrive in.  Three passes over the row fix
// the 32-bit logit key of the entry whose cumulative mass (in the top-k order:
// larger logit first) first reaches P of the total: each histograms the
// masses of the kept entries that share the digits fixed so far by the next
// 11, 11, 10 bits and keeps the digit where the cumulative mass from the top
// crosses the target.  Among the entries with that logit (equal weights w),
// the first k by index are kept, k = ceil((target - mass above) / w): a
// radix select over their indices gives the exact threshold key.
// ---------------------------------------------------------------------------
constexpr int kMassBins = kCap;  // the candidate buffer holds the mass histogram

__device__ __forceinline__ unsigned long long mass_fix(float z, float c, float R, float scale) {
  if (z == -INFINITY) return 0ull;
  return (unsigned long long)(__builtin_amdgcn_exp2f(fmaf(z, c, -R)) * scale);
}

// Keys of a source's entries whose logit key (high word) is hw and whose key
// is at least thr: the ties at the nucleus cut.
template <class Src> struct TieKeys {
  const Src &src;
  uint32_t hw;
  unsigned long long thr;
  template <class F> __device__ __forceinline__ void for_each(F f) const {
    src.template for_each_u<Src::kUCut>([&](float z, int v) {
      const unsigned long long k = entry_key(z, (uint32_t)v);
      if ((uint32_t)(k >> 32) == hw && k >= thr) f(k);
    });
  }
};

// Exact K-th largest key of a key set whose bits >= hi agree (K <= its size).
template <class Keys>
__device__ __forceinline__ unsigned long long exact_kth(TopkShared &sh, const Keys &keys, unsigned int K, int hi,
                                                        unsigned long long high) {
  const unsigned long long t = high | radix_select<kTopkThreads>(sh, keys, K, hi, 0);
  unsigned long long kmin = ~0ull;
  keys.for_each([&](unsigned long long key) {
    if (key >= t) kmin = key < kmin ? key : kmin;
  });
  kmin = ~wave_max_u64(~kmin);
  if ((threadIdx.x % kWave) == 0) sh.red_u[threadIdx.x / kWave] = kmin;
  __syncthreads();
  kmin = sh.red_u[0];
  for (int i = 1; i < kTopkThreads / kWave; ++i) kmin = sh.red_u[i] < kmin ? sh.red_u[i] : kmin;
  __syncthreads();
  return kmin;
}

// R of a row with every entry kept: the reference ceil(max z c).
template <class Src>
__device__ __forceinline__ float row_reference(TopkShared &sh, const Src &src, float c) {
  float zmax = -INFINITY;
  src.template for_each_u<Src::kUCut>([&](float z, int) { zmax = fmaxf(zmax, z); });
  zmax = wave_max_f(zmax);
  if ((threadIdx.x % kWave) == 0) sh.red_f[threadIdx.x / kWave] = zmax;
  __syncthreads();
  zmax = sh.red_f[0];
  for (int i = 1; i < kTopkThreads / kWave; ++i) zmax = fmaxf(zmax, sh.red_f[i]);
  __syncthreads();
  return zmax == -INFINITY ? -INFINITY : ceilf(zmax * c);
}

template <class Src>
__device__ void nucleus_cut_radix(TopkShared &sh, const Src &src, int V, float c, float P, TopkRow &r) {
  const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
  const int fb = 62 - (32 - __builtin_clz((unsigned)V));
  const float scale = ldexpf(1.0f, fb);
  const unsigned long long thr0 = r.thr;
  const float R = r.R;
  unsigned long long *mass = sh.cand;
  unsigned long long prefix = 0ull, pmask = 0ull;  // key bits fixed so far
  unsigned long long above = 0ull;                 // mass of kept keys above them
  unsigned long long target = 0ull;                // P of the total mass, rounded up
  // bf16 logits fill only the top 16 bits of their float: the low 16 bits of
  // the key's high word are then 0 (z >= 0) or all ones (z < 0, complemented
  // by orderable), fixed by the sign bit that pass 0 fixes; the last digit is
  // known without a pass
  constexpr int kPasses = Src::NE == 8 ? 2 : 3;
  // Entries with z c - R < -T weigh under 2^(fb - T) each, so together under
  // V 2^(fb - T) <= (1 - P) 2^fb / 4, at most (1 - P) / 2 of the total (the
  // largest entry alone weighs at least 2^(fb - 1)): the cumulative mass from
  // the top reaches P of the total before them.  Their mass only joins the
  // total (summed in registers, exact), and no pass puts them in a histogram,
  // which spares the LDS atomics of most of a long-tailed row.
  const float T = ceilf(log2f(2.0f * (float)V / (1.0f - P))) + 1.0f;
  unsigned long long low = 0ull;
#pragma unroll 1
  for (int pass = 0; pass < kPasses; ++pass) {
    // digits of the key's high word: bits [53, 64), [42, 53), [32, 42)
    const int shift = pass == 0 ? 53 : (pass == 1 ? 42 : 32);
    const int nb = pass < 2 ? 2048 : 1024;
    const unsigned long long dmask = (unsigned long long)(nb - 1);
    for (int i = tid; i < kMassBins; i += kTopkThreads) mass[i] = 0ull;
    __syncthreads();
    src.template for_each_u<Src::kUCut>([&](float z, int v) {
      const unsigned long long key = entry_key(z, (uint32_t)v);
      if (key >= thr0 && (key & pmask) == prefix) {
        const unsigned long long w = mass_fix(z, c, R, scale);
        if (fmaf(z, c, -R) < -T) {
          if (pass == 0) low += w;
        } else if (w) {
          atomicAdd(&mass[(unsigned)((key >> shift) & dmask)], w);
        }
      }
    });
    if (pass == 0) {
#pragma unroll
      for (int off = kWave / 2; off > 0; off >>= 1) low += __shfl_xor(low, off, kWave);
      if (lane == 0) sh.red_low[wave] = low;
    }
    __syncthreads();
    // thread t owns digits nb-1-2t and nb-2-2t (descending); inclusive scan
    const int dh = nb - 1 - 2 * tid, dl = dh - 1;
    const unsigned long long mh = dh >= 0 ? mass[dh] : 0ull, ml = dl >= 0 ? mass[dl] : 0ull;
    unsigned long long incl = mh + ml;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const unsigned long long y = __shfl_up(incl, off, kWave);
      if (lane >= off) incl += y;
    }
    if (lane == kWave - 1) sh.red_u[wave] = incl;
    if (tid == 0) sh.bcast_n = -1;
    __syncthreads();
    unsigned long long before = 0ull, total = 0ull;
    for (int w = 0; w < kTopkThreads / kWave; ++w) {
      if (w < wave) before += sh.red_u[w];
      total += sh.red_u[w];
      if (pass == 0) total += sh.red_low[w];
    }
    if (pass == 0) {
      // the cumulative mass must reach P of the total: an integer target; the
      // row stays valid (uncut) should no crossing be found below
      unsigned long long t = (unsigned long long)ceil((double)P * (double)total);
      target = t < 1ull ? 1ull : (t > total ? total : t);
      r.S = (float)total * ldexpf(1.0f, -fb);
    }
    const unsigned long long a0 = above + before + incl - (mh + ml);  // mass of the digits above dh
    if (dh >= 0 && a0 < target && a0 + mh >= target) {
      sh.bcast_n = dh;
      sh.sel_prefix = a0;
    } else if (dl >= 0 && a0 + mh < target && a0 + mh + ml >= target) {
      sh.bcast_n = dl;
      sh.sel_prefix = a0 + mh;
    }
    __syncthreads();
    const int d = sh.bcast_n;
    const unsigned long long ab = sh.sel_prefix;
    __syncthreads();
    if (d < 0) return;  // no crossing (cannot happen: the target lies within the kept mass); keep the row as is
    prefix |= (unsigned long long)d << shift;
    pmask |= dmask << shift;
    above = ab;
  }
  if (kPasses == 2) {
    const unsigned long long low = (prefix >> 63) ? 0ull : 0x3FFull;  // key bit 63 set: z >= 0
    prefix |= low << 32;
    pmask |= 0x3FFull << 32;
  }
  // every kept entry with logit key hw weighs w; the first k by index are kept
  const uint32_t hw = (uint32_t)(prefix >> 32);
  const unsigned long long w = mass_fix(from_orderable(hw), c, R, scale);
  if (w == 0ull) return;
  const unsigned long long need = target - above;
  unsigned long long k = (need + w - 1ull) / w;
  if (tid == 0) sh.ncand = 0u;
  __syncthreads();
  const TieKeys<Src> ties{src, hw, thr0};
  ties.for_each([&](unsigned long long key) {
    const unsigned int slot = atomicAdd(&sh.ncand, 1u);
    if (slot < (unsigned int)kCap) sh.cand[slot] = key;
  });
  __syncthreads();
  const unsigned int n = sh.ncand;
  __syncthreads();
  if (n == 0u) return;
  if (k > n) k = n;
  const unsigned long long high = (unsigned long long)hw << 32;
  const unsigned long long thr = n <= (unsigned int)kCap
      ? exact_kth(sh, LdsKeys<kTopkThreads>{sh.cand, n}, (unsigned int)k, 32, high)
      : exact_kth(sh, ties, (unsigned int)k, 32, high);
  r.thr = thr;
  r.S = (float)(above + k * w) * ldexpf(1.0f, -fb);
  r.in_lds = false;
}

// Kept set of a row: the top-K (0 < K < V; K <= 0: every entry), then the
// nucleus cut when 0 < top_p < 1.  Exact threshold, statistics over the kept
// entries, and the top-K list when given (K <= kTopkThreads).  RADIX compiles
// in the mass-weighted cut that sets without top-k (K <= 0) or larger than
// kTopkThreads need; it takes many registers, so kernels without it keep two
// 1024-thread blocks per compute unit.  Without RADIX the caller guarantees
// 0 < K and, with the nucleus on, K <= kTopkThreads.
template <bool RADIX, class Src>
__device__ __forceinline__ TopkRow topk_row(TopkShared &sh, const Src &src, int K, float c, float top_p,
                                            int2 *list, int V) {
  const bool nucleus = top_p > 0.0f && top_p < 1.0f;
  if (RADIX && K <= 0) {
    // no top-k: every entry is kept before the cut (callers come here only
    // with the nucleus on; without it the statistics are those of the row)
    TopkRow r{0ull, row_reference(sh, src, c), 0.0f, false, 0u};
    if (nucleus) nucleus_cut_radix(sh, src, V, c, top_p, r);
    return r;
  }
  const Selected sel = select_threshold(sh, src, K);
  if (sel.one_wave) return topk_one_wave(sh, sel.ncand, K, c, top_p, list);
  TopkRow r = sel.in_lds ? kept_stats<true>(sh, LdsKeys<kTopkThreads>{sh.cand, sel.ncand}, sel.thr, c, list, K)
                         : kept_stats<false>(sh, SrcKeys<Src>{src}, sel.thr, c, list, K);
  r.in_lds = sel.in_lds;
  r.ncand = sel.ncand;
  if (nucleus) {
    if (K > kTopkThreads) {
      if constexpr (RADIX) nucleus_cut_radix(sh, src, V, c, top_p, r);
    } else if (sel.in_lds) nucleus_cut(sh, LdsKeys<kTopkThreads>{sh.cand, sel.ncand}, c, top_p, r);
    else nucleus_cut(sh, SrcKeys<Src>{src}, c, top_p, r);
  }
  return r;
}


__device__ __forceinline__ uint4 pack_rowinfo(const TopkRow &r) {
  return make_uint4((uint32_t)(r.thr & 0xFFFFFFFFull), (uint32_t)(r.thr >> 32), __float_as_uint(r.R),
                    __float_as_uint(r.S));
}
__device__ __forceinline__ TopkRow unpack_rowinfo(uint4 u) {
  return TopkRow{((unsigned long long)u.y << 32) | u.x, __uint_as_float(u.z), __uint_as_float(u.w), false, 0u};
}

// p or q of entry (z, v) under a selected row's statistics: 0 outside the kept set.
__device__ __forceinline__ float kept_prob(const TopkRow &r, float z, uint32_t v, float c) {
  if (entry_key(z, v) < r.thr || z == -INFINITY) return 0.0f;
  return __builtin_amdgcn_exp2f(fmaf(z, c, -r.R)) / r.S;
}

template <int NT>
__device__ __forceinline__ unsigned long long block_max_u64_sh(unsigned long long x, unsigned long long *red) {
  x = wave_max_u64(x);
  if ((threadIdx.x % kWave) == 0) red[threadIdx.x / kWave] = x;
  __syncthreads();
  x = red[0];
  for (int i = 1; i < NT / kWave; ++i) x = red[i] > x ? red[i] : x;
  __syncthreads();
  return x;
}

// Gumbel-max over group blocks [g0, g1) of a row, over every entry or
// (MASKED) the entries whose key is at least thr: key z c - log2 E2 with
// words of `ps`, one Philox block per four entries.  Each thread walks its entries in
// increasing index with a strict comparison (smaller index among equal keys).
template <int DT, int NT, bool MASKED = false, bool X3 = false>
__device__ __forceinline__ unsigned long long gumbel_dense_row(const Row<DT> &R, int V, float c,
                                                             const PhiloxStream &ps, int g0, int g1,
                                                             unsigned long long thr = 0ull) {
  constexpr int NE = Elem<DT>::kVec;
  float bestk = -INFINITY;
  uint32_t besti = 0xFFFFFFFFu;  // none
  for (int gb = g0 + (int)threadIdx.x; gb < g1; gb += NT) {
    float z[NE];
    R.load_block(gb, z);  // entries NE gb .. NE gb + NE - 1; past the row: masked below
#pragma unroll
    for (int g = 0; g < NE / 4; ++g) {
      const uint32_t group = (uint32_t)(gb * (NE / 4) + g);
      const Philox4 blk = ps.template block<X3>(group);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t idx = group * 4u + (uint32_t)e;
        const float key = fmaf(z[g * 4 + e], c, -__builtin_amdgcn_logf(exp2_variate(blk.w[e])));
        const bool kept = !MASKED || entry_key(z[g * 4 + e], idx) >= thr;
        const bool take = idx < (uint32_t)V && kept && key > bestk;
        bestk = take ? key : bestk;
        besti = take ? idx : besti;
      }
    }
  }
  return besti == 0xFFFFFFFFu ? 0ull : pack_key(bestk, besti);
}

// Bonus key of kept entry (z, v) at position pos: z c - log2 E2_v, monotone in
// ln q_v - ln E_v; 0 for entries outside the kept set.
__device__ __forceinline__ unsigned long long bonus_key(const Args &a, uint32_t seq, int pos,
                                                       const TopkRow &qr, float z, uint32_t v) {
  if (z == -INFINITY || entry_key(z, v) < qr.thr) return 0ull;
  const Philox4 blk = stream_block(a.key0, a.key1, seq, (uint32_t)pos, v >> 2, PURPOSE_SAMPLE);
  const float E = exp2_variate(word_of(blk, v & 3u));
  return pack_key(fmaf(z, a.c, -__builtin_amdgcn_logf(E)), v);
}

// Gumbel-max over the kept entries of target row `pos` (weights q): the bonus
// token, or the replacement when the residual is empty.  The kept entries come
// from `list` (K entries), from the LDS candidates of a row just selected, or
// from a scan of the row with the threshold.
template <int DT>
__device__ __forceinline__ unsigned long long gumbel_over_kept_q(TopkShared &sh, const Args &a, int b, int pos,
                                                 const TopkRow &qr, const int2 *list, const Row<DT> &Q) {
  const uint32_t seq = seq_of(a, b);
  unsigned long long best = 0ull;
  auto consider = [&](float z, uint32_t v) {
    const unsigned long long k = bonus_key(a, seq, pos, qr, z, v);
    best = k > best ? k : best;
  };
  if (list) {
    for (int i = threadIdx.x; i < a.top_k; i += kTopkThreads)
      consider(__int_as_float(list[i].y), (uint32_t)list[i].x);
  } else if (qr.in_lds) {
    for (unsigned int i = threadIdx.x; i < qr.ncand; i += kTopkThreads) {
      const unsigned long long key = sh.cand[i];
      consider(from_orderable((uint32_t)(key >> 32)), 0xFFFFFFFFu - (uint32_t)(key & 0xFFFFFFFFull));
    }
  } else {
    for (int v = threadIdx.x; v < a.V; v += kTopkThreads) consider(Q.load_one(v), (uint32_t)v);
  }
  return block_max_u64_sh<kTopkThreads>(best, sh.red_u);
}

// Residual draw at rejected position n: weights max(0, q_n - p_n) over the
// target row's kept entries (outside them q_n = 0 and the weight is 0).
template <int DT>
__device__ __forceinline__ unsigned long long gumbel_residual_topk(TopkShared &sh, const Args &a, int b, int n,
                                                   const TopkRow &pr, const TopkRow &qr, const int2 *qlist,
                                                   const Row<DT> &P, const Row<DT> &Q) {
  const uint32_t seq = seq_of(a, b);
  const float c = a.c;
  unsigned long long best = 0ull;
  auto consider = [&](float zq, uint32_t v) {
    const float qv = kept_prob(qr, zq, v, c);
    if (qv <= 0.0f) return;
    const float pv = kept_prob(pr, P.load_one((int)v), v, c);
    const float r = residual_weight(qv, pv);
    if (!(r > 0.0f)) return;
    const Philox4 blk = stream_block(a.key0, a.key1, seq, (uint32_t)n, v >> 2, PURPOSE_SAMPLE);
    const unsigned long long k = pack_key(r * __builtin_amdgcn_rcpf(exp2_variate(word_of(blk, v & 3u))), v);
    best = k > best ? k : best;
  };
  if (qlist) {
    for (int i = threadIdx.x; i < a.top_k; i += kTopkThreads)
      consider(__int_as_float(qlist[i].y), (uint32_t)qlist[i].x);
  } else {
    for (int v = threadIdx.x; v < a.V; v += kTopkThreads) consider(Q.load_one(v), (uint32_t)v);
  }
  return block_max_u64_sh<kTopkThreads>(best, sh.red_u);
}

// rowinfo / lists slot of a sequence's rows: draft j -> j, target j -> gamma + j.
__device__ __forceinline__ size_t slot_of(const Args &a, int b, int s) {
  return (size_t)b * (2 * a.gamma) + s;
}

// Judge position j of sequence b against its selected rows (every lane of
// wave 0 computes the same result).
// Top-k of one global row.
template <int DT, bool RADIX>
__device__ __forceinline__ TopkRow select_row(TopkShared &sh, const Row<DT> &row, int V, int K, float c, float top_p,
                                              int2 *list) {
  const StreamRow<DT> src(row, V);
  return topk_row<RADIX>(sh, src, K, c, top_p, list, V);
}

template <int DT>
__device__ __forceinline__ Judged judge_topk(const Args &a, int b, int j) {
  const int gamma = a.gamma;
  const TopkRow pr = unpack_rowinfo(a.rowinfo[slot_of(a, b, j)]);
  const TopkRow qr = unpack_rowinfo(a.rowinfo[slot_of(a, b, gamma + j)]);
  const int t = a.tokens[(size_t)b * gamma + j];
  const float zp = Row<DT>(draft_row<DT>(a, b, j), a.V).load_one(t);
  const float zq = Row<DT>(target_row<DT>(a, b, j), a.V).load_one(t);
  const bool qzero = zq == -INFINITY || entry_key(zq, (uint32_t)t) < qr.thr;
  const bool pzero = zp == -INFINITY || entry_key(zp, (uint32_t)t) < pr.thr;
  return judge_one(a, seq_of(a, b), j, zp, zq, pzero, qzero, pr.R, pr.S, qr.R, qr.S);
}

// One launch per window [w0, w1) of positions (w0 = w1 = gamma: judge and
// sample only).  Blocks per sequence: 2 (w1 - w0), at least 1; block
// (rp, r) selects row w0 + rp of the draft (r = 0) or the target (r = 1), and
// block 0 leads (writes the outputs, draws the token).  Every block first
// judges the previous window [p0, w0) of its sequence (wave 0, lane l:
// position p0 + l; a ballot finds the first rejection).
// Two blocks per compute unit (eight waves per SIMD) keep enough rows in
// flight; RADIX: the nucleus without top-k or over more than kTopkThreads
// kept entries (see topk_row).
template <int DT, bool RADIX>
__global__ __launch_bounds__(kTopkThreads, RADIX ? 4 : 8) void k_topk_step(Args a, int launch, int p0, int w0, int w1) {
  __shared__ TopkShared sh;
  const int dw = w1 - w0;
  const int per_seq = dw > 0 ? 2 * dw : 1;
  const int b = blockIdx.x / per_seq;
  const int rem = blockIdx.x - b * per_seq;
  const int rp = rem >> 1, r = rem & 1;  // r: 0 draft row (block 0 leads), 1 target row
  const bool lead = rem == 0;
  const int gamma = a.gamma;
  int32_t *state_in = a.state + (size_t)((launch + 1) & 1) * a.B;
  int32_t *state_out = a.state + (size_t)(launch & 1) * a.B;

  if (threadIdx.x < kWave) {
    const int lane = threadIdx.x;
    int mode = 0;  // 0 select a row of the window, 1 residual at row n, 2 bonus, -1 nothing
    int n = 0;
    if (w0 == 0) {
      if (!tokens_valid(a, b, lane)) {
        mode = -1;
        if (lead) {
          write_invalid(a, b, lane);
          for (int k = lane; k < gamma; k += kWave) write_diag(a, b, k, NAN, NAN, NAN, NAN);
          if (lane == 0) state_out[b] = kInvalid;
        }
      } else if (lead) {
        for (int k = lane; k < gamma; k += kWave) write_diag(a, b, k, NAN, NAN, NAN, NAN);
        if (lane == 0) state_out[b] = 0;
      }
    } else {
      const int s = state_in[b];
      if (s != p0) {
        mode = -1;
        if (lead && lane == 0) state_out[b] = s;
      } else {
        const int nj = w0 - p0;
        const bool act = lane < nj;
        Judged jr{};
        if (act) jr = judge_topk<DT>(a, b, p0 + lane);
        const unsigned long long mask = __ballot(act && jr.accept);
        const int k = (mask == ~0ull) ? kWave : __builtin_ctzll(~mask);  // first clear bit
        if (lead && act && lane <= k) write_diag(a, b, p0 + lane, jr.pt, jr.qt, jr.u, jr.ratio);
        if (k < nj) {
          n = p0 + k;
          mode = lead ? 1 : -1;
          if (lead) write_judged(a, b, lane, n);
          if (lead && lane == 0) state_out[b] = kDone;
        } else if (w0 == gamma) {
          mode = lead ? 2 : -1;
          if (lead) write_judged(a, b, lane, gamma);
          if (lead && lane == 0) state_out[b] = kDone;
        } else if (lead && lane == 0) {
          state_out[b] = w0;
        }
      }
    }
    if (lane == 0) {
      sh.bcast_n = mode;
      sh.sel_k = (unsigned)n;
    }
  }
  __syncthreads();
  const int mode = sh.bcast_n;
  const int n = (int)sh.sel_k;
  __syncthreads();
  if (mode < 0) return;
  const int j = w0 + rp;  // the row to select in mode 0
  int32_t *out = a.out_tokens + (size_t)b * (gamma + 1);
  if (mode == 0) {
    const int slot = r == 0 ? j : gamma + j;
    const void *ptr = r == 0 ? draft_row<DT>(a, b, j) : target_row<DT>(a, b, j);
    const Row<DT> row(ptr, a.V);
    int2 *list = a.lists ? a.lists + slot_of(a, b, slot) * (size_t)a.klist : nullptr;
    const TopkRow tr = select_row<DT, RADIX>(sh, row, a.V, a.top_k, a.c, a.top_p, list);
    if (threadIdx.x == 0) a.rowinfo[slot_of(a, b, slot)] = pack_rowinfo(tr);
  } else if (mode == 1) {
    const TopkRow pr = unpack_rowinfo(a.rowinfo[slot_of(a, b, n)]);
    const TopkRow qr = unpack_rowinfo(a.rowinfo[slot_of(a, b, gamma + n)]);
    const int2 *qlist = a.lists ? a.lists + slot_of(a, b, gamma + n) * (size_t)a.klist : nullptr;
    const Row<DT> P(draft_row<DT>(a, b, n), a.V);
    const Row<DT> Q(target_row<DT>(a, b, n), a.V);
    unsigned long long k = gumbel_residual_topk<DT>(sh, a, b, n, pr, qr, qlist, P, Q);
    if (k == 0ull) k = gumbel_over_kept_q<DT>(sh, a, b, n, qr, qlist, Q);
    if (threadIdx.x == 0) out[n] = (int32_t)packed_index(k);
  } else {
    // every draft kept: top-k of target row gamma, then the bonus draw (a
    // nucleus kept set from the mass-weighted cut: the dense Gumbel pass over
    // the row, entries outside the set skipped)
    const Row<DT> Q(target_row<DT>(a, b, gamma), a.V);
    const TopkRow qr = select_row<DT, RADIX>(sh, Q, a.V, a.top_k, a.c, a.top_p, nullptr);
    unsigned long long k;
    if (!RADIX || qr.in_lds) {
      k = gumbel_over_kept_q<DT>(sh, a, b, gamma, qr, nullptr, Q);
    } else {
      const PhiloxStream ps(a.key0, a.key1, seq_of(a, b), (uint32_t)gamma, PURPOSE_SAMPLE);
      k = block_max_u64_sh<kTopkThreads>(gumbel_dense_row<DT, kTopkThreads, true>(Q, a.V, a.c, ps, 0, a.ngb, qr.thr),
                                         sh.red_u);
    }
    if (threadIdx.x == 0) out[gamma] = (int32_t)packed_index(k);
  }
}

}  // namespace sv
