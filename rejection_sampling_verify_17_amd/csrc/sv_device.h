// Device primitives for the verification kernels (gfx950, wave64).
//
// Philox4x32-10, the two variates drawn from it, logit decoding, bounds-checked
// buffer loads and wave/block reductions.  Nothing here is shared with the
// CPU oracle; the two are written separately from the same published
// definitions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sv {

constexpr int kWave = 64;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

enum { DT_F32 = 0, DT_BF16 = 1 };
enum { PURPOSE_ACCEPT = 0u, PURPOSE_SAMPLE = 1u, PURPOSE_DRAFT = 2u };

// ---------------------------------------------------------------------------
// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as easy
// as 1, 2, 3", SC'11).  Per round: multiply counter words 0 and 2 by the two
// round multipliers, keep both halves of each 64-bit product, and rebuild the
// counter from them and the key; the key then advances by the two Weyl
// increments.  Ten rounds.
// ---------------------------------------------------------------------------
struct Philox4 {
  uint32_t w[4];
};

// a ^ b ^ c in one instruction (gfx950's three-input bit operation; the
// table 0x96 is 1 where an odd number of the three inputs are 1).
__device__ __forceinline__ uint32_t xor3(uint32_t a, uint32_t b, uint32_t c) {
  return __builtin_amdgcn_bitop3_b32(a, b, c, 0x96);
}

// Rounds FIRST .. 9 of Philox4x32-10 from the words and keys of round FIRST.
// X3: each round's two three-way XORs as one instruction each (fewer
// instructions, but the operation takes its operands in vector registers,
// which costs registers a kernel near its budget may not have).
template <int FIRST, bool X3 = false>
__device__ __forceinline__ Philox4 philox_rounds(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                                 uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int round = FIRST; round < 10; ++round) {
    const uint32_t mA = 0xD2511F53u, mB = 0xCD9E8D57u;
    // one v_mad_u64_u32 gives both halves of each product
    uint64_t pA, pB, ccA, ccB;
    asm("v_mad_u64_u32 %0, %1, %2, %3, 0" : "=v"(pA), "=s"(ccA) : "s"(mA), "v"(c0));
    asm("v_mad_u64_u32 %0, %1, %2, %3, 0" : "=v"(pB), "=s"(ccB) : "s"(mB), "v"(c2));
    const uint32_t hiA = (uint32_t)(pA >> 32), loA = (uint32_t)pA;
    const uint32_t hiB = (uint32_t)(pB >> 32), loB = (uint32_t)pB;
    const uint32_t n0 = X3 ? xor3(hiB, c1, k0) : hiB ^ c1 ^ k0;
    const uint32_t n2 = X3 ? xor3(hiA, c3, k1) : hiA ^ c3 ^ k1;
    c0 = n0;
    c1 = loB;
    c2 = n2;
    c3 = loA;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  Philox4 r;
  r.w[0] = c0;
  r.w[1] = c1;
  r.w[2] = c2;
  r.w[3] = c3;
  return r;
}

__device__ __forceinline__ Philox4 philox(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                          uint32_t k0, uint32_t k1) {
  return philox_rounds<0>(c0, c1, c2, c3, k0, k1);
}

// The blocks of one (seq, pos, purpose) stream, group by group: only the
// group word varies, so the first-round product of the seq word and the
// second-round product of the first word are the same for every group and
// are formed once (18 instead of 20 lane-wise products per block, same bits).
struct PhiloxStream {
  uint32_t k0, k1, purpose;
  uint32_t w0, lo_b0;    // second-round words 0 and 1
  uint32_t hi_a1, lo_a1;  // second-round product of word 0
  __device__ __forceinline__ PhiloxStream(uint32_t key0, uint32_t key1, uint32_t seq, uint32_t pos, uint32_t pur)
      : k0(key0), k1(key1), purpose(pur) {
    const uint64_t pb0 = (uint64_t)0xCD9E8D57u * seq;
    lo_b0 = (uint32_t)pb0;
    w0 = (uint32_t)(pb0 >> 32) ^ pos ^ key0;
    const uint64_t pa1 = (uint64_t)0xD2511F53u * w0;
    hi_a1 = (uint32_t)(pa1 >> 32);
    lo_a1 = (uint32_t)pa1;
  }
  template <bool X3 = false> __device__ __forceinline__ Philox4 block(uint32_t group) const {
    uint64_t pA, pB, cc;
    asm("v_mad_u64_u32 %0, %1, %2, %3, 0" : "=v"(pA), "=s"(cc) : "s"(0xD2511F53u), "v"(group));
    const uint32_t hi_a0 = (uint32_t)(pA >> 32), lo_a0 = (uint32_t)pA;
    const uint32_t c2 = hi_a0 ^ purpose ^ k1;  // first round done: words (w0, lo_b0, c2, lo_a0)
    asm("v_mad_u64_u32 %0, %1, %2, %3, 0" : "=v"(pB), "=s"(cc) : "s"(0xCD9E8D57u), "v"(c2));
    const uint32_t n0 = (uint32_t)(pB >> 32) ^ lo_b0 ^ (k0 + 0x9E3779B9u);
    const uint32_t n2 = hi_a1 ^ lo_a0 ^ (k1 + 0xBB67AE85u);
    // second round done: words (n0, lo(pB), n2, lo_a1), keys advanced twice
    return philox_rounds<2, X3>(n0, (uint32_t)pB, n2, lo_a1, k0 + 2u * 0x9E3779B9u, k1 + 2u * 0xBB67AE85u);
  }
};

// The four words of vocabulary group g (entries 4g .. 4g+3) at (seq, pos, purpose).
__device__ __forceinline__ Philox4 stream_block(uint32_t k0, uint32_t k1, uint32_t seq, uint32_t pos,
                                                uint32_t group, uint32_t purpose) {
  return philox(group, pos, seq, purpose, k0, k1);
}

// Word i (0..3, run-time) of a block, by selects (no indexed private memory).
__device__ __forceinline__ uint32_t word_of(const Philox4 &b, uint32_t i) {
  const uint32_t lo = (i & 1u) ? b.w[1] : b.w[0];
  const uint32_t hi = (i & 1u) ? b.w[3] : b.w[2];
  return (i & 2u) ? hi : lo;
}

// Acceptance uniform: top 24 bits of the word times 2^-24, in [0, 1); exact in fp32.
__device__ __forceinline__ float accept_uniform(uint32_t w) {
  return (float)(w >> 8) * 0x1p-24f;
}

// Exponential variate in base 2: E2 = -log2 U = E / ln 2, with E = -ln U the
// exponential variate and U = (2 (w >> 9) + 1) 2^-24 (an odd multiple of 2^-24
// inside (0, 1), exact in fp32).  Scaling every E of an arg-max by the same
// 1/ln 2 leaves the arg-max unchanged: r / E2 orders like r / E, and
// z c - log2 E2 = (ln q - ln E) / ln 2 + const.  The native log2 (v_log_f32)
// is within 1 ulp of log2 U for every one of the 2^23 possible U, including
// U -> 1 where E is smallest and the key largest.
__device__ __forceinline__ float exp2_variate(uint32_t w) {
  const float U = (float)(2u * (w >> 9) + 1u) * 0x1p-24f;
  return -__builtin_amdgcn_logf(U);
}

// Order-preserving map of a float onto uint32 (larger float -> larger integer).
__device__ __forceinline__ uint32_t orderable(float f) {
  const uint32_t b = __float_as_uint(f);
  return b ^ ((uint32_t)((int32_t)b >> 31) | 0x80000000u);
}
__device__ __forceinline__ float from_orderable(uint32_t u) {
  const uint32_t b = (u & 0x80000000u) ? (u ^ 0x80000000u) : ~u;
  return __uint_as_float(b);
}

// Key of entry v for an arg-max with ties to the smaller index.
__device__ __forceinline__ unsigned long long pack_key(float key, uint32_t v) {
  return ((unsigned long long)orderable(key) << 32) | (unsigned long long)(0xFFFFFFFFu - v);
}
__device__ __forceinline__ uint32_t packed_index(unsigned long long k) {
  return 0xFFFFFFFFu - (uint32_t)(k & 0xFFFFFFFFull);
}

// ---------------------------------------------------------------------------
// Logits
// ---------------------------------------------------------------------------
template <int DT> struct Elem;
template <> struct Elem<DT_F32> {
  static constexpr int kSize = 4;  // bytes per logit
  static constexpr int kVec = 4;   // logits per 16-byte load
};
template <> struct Elem<DT_BF16> {
  static constexpr int kSize = 2;
  static constexpr int kVec = 8;
};

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

template <int DT>
__device__ __forceinline__ void decode(const u32x4 v, float (&z)[Elem<DT>::kVec]) {
  if constexpr (DT == DT_F32) {
    z[0] = __uint_as_float(v.x);
    z[1] = __uint_as_float(v.y);
    z[2] = __uint_as_float(v.z);
    z[3] = __uint_as_float(v.w);
  } else {
    z[0] = bf16_lo(v.x); z[1] = bf16_hi(v.x);
    z[2] = bf16_lo(v.y); z[3] = bf16_hi(v.y);
    z[4] = bf16_lo(v.z); z[5] = bf16_hi(v.z);
    z[6] = bf16_lo(v.w); z[7] = bf16_hi(v.w);
  }
}

// A row of V logits read through a buffer resource with 16-byte-aligned loads.
// The resource starts at the row's address rounded down to 16 bytes, so the
// row sits `s` entries into its first vector: vector iv holds entries
// [NE*iv - s, NE*iv - s + NE).  The few bytes before the row share a 16-byte
// block (hence a page) with its first entry, so reading them is always safe;
// the range ends at the row's last 4-byte word and loads beyond it return
// zeros without touching memory.  Callers mask entries outside [0, V).
template <int DT> struct Row {
  static constexpr int NE = Elem<DT>::kVec;
  static constexpr int ESZ = Elem<DT>::kSize;
  __amdgpu_buffer_rsrc_t rsrc;
  int s;  // entries of the first vector that precede the row

  __device__ __forceinline__ Row(const void *p, int V) {
    const uintptr_t addr = (uintptr_t)p;
    const uintptr_t a16 = addr & ~(uintptr_t)15;
    s = (int)((addr - a16) / ESZ);
    const uint32_t bytes = ((uint32_t)(addr - a16) + (uint32_t)V * ESZ + 3u) & ~3u;
    rsrc = __builtin_amdgcn_make_buffer_rsrc((void *)a16, (short)0, (int)bytes, 0x00020000);
  }

  // vectors covering the row
  __device__ __forceinline__ int nvec(int V) const { return (s + V + NE - 1) / NE; }

  __device__ __forceinline__ u32x4 raw(int iv) const {
    return __builtin_amdgcn_raw_buffer_load_b128(rsrc, iv * 16, 0, 0);
  }

  // Vector iv: z[e] is entry NE*iv + e - s.
  __device__ __forceinline__ void load_vec(int iv, float (&z)[NE]) const { decode<DT>(raw(iv), z); }

  // Entries [NE*g, NE*g + NE) in order (a "group block": NE/4 Philox groups).
  // When the row starts on a 4-byte boundary (always for fp32, for bf16 when
  // s is even) one 16-byte load at a 4-byte-aligned offset reads them;
  // otherwise they are assembled from vectors g and g+1 with a funnel shift.
  __device__ __forceinline__ void load_block(int g, float (&z)[NE]) const {
    if (((s * ESZ) & 3) == 0) {
      decode<DT>(__builtin_amdgcn_raw_buffer_load_b128(rsrc, g * 16 + s * ESZ, 0, 0), z);
      return;
    }
    const u32x4 A = raw(g), B = raw(g + 1);
    const uint32_t d[8] = {A.x, A.y, A.z, A.w, B.x, B.y, B.z, B.w};
    const int sb = s * ESZ;           // byte shift, 1..15
    const int q = sb >> 2, r = sb & 3;  // whole words, then bytes (0 or 2)
    uint32_t w[5];
#pragma unroll
    for (int i = 0; i < 5; ++i) {
      const uint32_t a0 = d[i], a1 = d[i + 1], a2 = d[i + 2], a3 = d[i + 3];
      w[i] = q == 0 ? a0 : q == 1 ? a1 : q == 2 ? a2 : a3;
    }
    u32x4 o;
    o.x = r ? __builtin_amdgcn_alignbyte(w[1], w[0], (uint32_t)r) : w[0];
    o.y = r ? __builtin_amdgcn_alignbyte(w[2], w[1], (uint32_t)r) : w[1];
    o.z = r ? __builtin_amdgcn_alignbyte(w[3], w[2], (uint32_t)r) : w[2];
    o.w = r ? __builtin_amdgcn_alignbyte(w[4], w[3], (uint32_t)r) : w[3];
    decode<DT>(o, z);
  }

  __device__ __forceinline__ float load_one(int v) const {
    if constexpr (DT == DT_F32) {
      return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rsrc, (v + s) * 4, 0, 0));
    } else {
      const uint16_t h = __builtin_amdgcn_raw_buffer_load_b16(rsrc, (v + s) * 2, 0, 0);
      return __uint_as_float((uint32_t)h << 16);
    }
  }
};

// ---------------------------------------------------------------------------
// Softmax statistics in base 2.  A row's (R, S) means
//   S = sum_v 2^(z_v c - R),  c = log2(e) / T,
// with R an integer-valued float >= max z_v c (rounded), so merging two
// partial sums rescales by an exact power of two.  R = -inf, S = 0: empty.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float scale_pow2(float S, float dR) {
  // S * 2^dR for integer-valued dR <= 0
  return ldexpf(S, (int)fmaxf(dR, -1000.0f));
}

__device__ __forceinline__ void merge_stats(float &R, float &S, float R2, float S2) {
  const float Rn = fmaxf(R, R2);
  if (Rn == -INFINITY) {
    R = Rn;
    S = 0.0f;
    return;
  }
  const float a = (R == -INFINITY) ? 0.0f : scale_pow2(S, R - Rn);
  const float b = (R2 == -INFINITY) ? 0.0f : scale_pow2(S2, R2 - Rn);
  R = Rn;
  S = a + b;
}

// ---------------------------------------------------------------------------
// Reductions
// ---------------------------------------------------------------------------
__device__ __forceinline__ void wave_merge_stats(float &R, float &S) {
#pragma unroll
  for (int off = kWave / 2; off > 0; off >>= 1) {
    const float R2 = __shfl_xor(R, off, kWave);
    const float S2 = __shfl_xor(S, off, kWave);
    merge_stats(R, S, R2, S2);
  }
}

__device__ __forceinline__ unsigned long long wave_max_u64(unsigned long long x) {
#pragma unroll
  for (int off = kWave / 2; off > 0; off >>= 1) {
    const unsigned long long y = __shfl_xor(x, off, kWave);
    x = y > x ? y : x;
  }
  return x;
}

__device__ __forceinline__ float wave_max_f(float x) {
#pragma unroll
  for (int off = kWave / 2; off > 0; off >>= 1) x = fmaxf(x, __shfl_xor(x, off, kWave));
  return x;
}

__device__ __forceinline__ float wave_sum_f(float x) {
#pragma unroll
  for (int off = kWave / 2; off > 0; off >>= 1) x += __shfl_xor(x, off, kWave);
  return x;
}

__device__ __forceinline__ int wave_sum_i(int x) {
#pragma unroll
  for (int off = kWave / 2; off > 0; off >>= 1) x += __shfl_xor(x, off, kWave);
  return x;
}

// Block-wide merge of two (R, S) pairs; the result is valid in every thread.
template <int NT>
__device__ __forceinline__ void block_merge_stats2(float &R1, float &S1, float &R2, float &S2) {
  constexpr int NW = NT / kWave;
  __shared__ float sh[4][NW];
  wave_merge_stats(R1, S1);
  wave_merge_stats(R2, S2);
  const int lane = threadIdx.x % kWave, w = threadIdx.x / kWave;
  if (lane == 0) {
    sh[0][w] = R1; sh[1][w] = S1; sh[2][w] = R2; sh[3][w] = S2;
  }
  __syncthreads();
  R1 = sh[0][0]; S1 = sh[1][0]; R2 = sh[2][0]; S2 = sh[3][0];
#pragma unroll
  for (int i = 1; i < NW; ++i) {
    merge_stats(R1, S1, sh[0][i], sh[1][i]);
    merge_stats(R2, S2, sh[2][i], sh[3][i]);
  }
  __syncthreads();
}

template <int NT>
__device__ __forceinline__ unsigned long long block_max_u64(unsigned long long x) {
  constexpr int NW = NT / kWave;
  __shared__ unsigned long long sh[NW];
  x = wave_max_u64(x);
  const int lane = threadIdx.x % kWave, w = threadIdx.x / kWave;
  if (lane == 0) sh[w] = x;
  __syncthreads();
  x = sh[0];
#pragma unroll
  for (int i = 1; i < NW; ++i) x = sh[i] > x ? sh[i] : x;
  __syncthreads();
  return x;
}

}  // namespace sv
