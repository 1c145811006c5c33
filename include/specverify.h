/*
 * specverify — batched speculative-sampling verification on one MI355X (gfx950).
 *
 * C ABI: plain pointers and sizes, no C++ or framework types.  All compute runs
 * in HIP kernels of this library, enqueued on the caller's stream.
 *
 * The operation (one verification step over B independent sequences):
 *   For each sequence b, the target scored gamma+1 positions (logits
 *   target_logits[b][0..gamma][V]) and the draft scored gamma positions
 *   (draft_logits[b][0..gamma-1][V]) and emitted draft_tokens[b][0..gamma-1].
 *   Both sets of logits become distributions by temperature and top-k:
 *   q_j = softmax(topk(target[b][j]) / T), p_j = softmax(topk(draft[b][j]) / T)
 *   (page "추측 디코딩: 큰 모델을 빠르게 돌리는 법", ai-trend.me, section
 *   "어떻게 작동하나": temperature and top-k sampling are ordinary sampling from
 *   adjusted distributions).  Draft t_j is kept with probability
 *   min(1, q_j(t_j) / p_j(t_j)), judged left to right; the first rejected
 *   position n is replaced by a draw from max(0, q_n - p_n) normalised, and
 *   if all gamma are kept one more token is drawn from q_gamma (page
 *   "스펙큘러티브 디코딩 — 작은 모델이 먼저 쓰고 큰 모델이 검사한다",
 *   blog.mna-game.duckdns.org post 46, §1 for the rule, §3 for "accepted + 1"
 *   tokens per step; page ai-trend.me, "어떻게 작동하나", for the scan order,
 *   the discarded tail and the bonus token).
 *
 * Conventions fixed by this library where the pages are silent:
 *   - top-k keeps exactly K entries with the largest raw logit, the smaller
 *     vocabulary index on equal logits; top_k <= 0 or >= V turns it off.
 *     It applies to every row of both inputs, the bonus row included.
 *   - acceptance: keep iff q(t) > 0 and (p(t) == 0 or u < q(t)/p(t)), where
 *     u = (w >> 8) * 2^-24 and w is the Philox4x32-10 word (below) at
 *     (seq, pos = j, v = 0, purpose 0).
 *   - the replacement and the bonus token are Gumbel-max draws: the arg-max
 *     over the support of ln(weight_v) - ln(E_v), E_v = -ln U_v,
 *     U_v = (2 * (w >> 9) + 1) * 2^-24, w the word at (seq, pos, v,
 *     purpose 1), pos = the sampled row; ties go to the smaller v.  An empty
 *     residual (only reachable through rounding) falls back to q_n.
 *   - Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11) with key
 *     (seed mod 2^32, seed >> 32), counter (v >> 2, pos, seq mod 2^32,
 *     purpose); the word is output (v mod 4).  seq = seq_offset + b.
 *   - top_p in (0, 1) is nucleus sampling (page ai-trend.me, "어떻게 작동하나"):
 *     after temperature and top-k (if on), a row keeps its entries in the
 *     top-k order (larger logit, then smaller index) until their probability
 *     mass reaches top_p (the entry that reaches it is kept), renormalised;
 *     both p and q, with or without top-k.  top_p <= 0 or >= 1 turns it off.
 *     The cut is computed in finite precision (fp32 prefix sums for kept
 *     sets of up to 1024 entries, 64-bit fixed-point masses otherwise):
 *     where the mass of a prefix lies within rounding of top_p, the kept set
 *     can differ from an exact computation.
 *   - the residual max(0, q_n - p_n) is formed from fp32 probabilities; a
 *     difference at or below 2^-16 of q_n(v) is taken as zero (it is within
 *     the rounding of the two rows' softmax sums), so identical rows give an
 *     empty residual and the draw falls back to q_n.
 *   - temperature 0 is the arg-max mode (page ai-trend.me, "어떻게 작동하나":
 *     arg-max decoding is sampling from an adjusted distribution): every
 *     distribution is the point mass on its row's largest logit, the smaller
 *     index among equal logits (-0 equals +0).  The rule above then keeps
 *     draft j iff t_j = argmax q_j, and the token after the kept prefix is
 *     argmax q_n (the residual's only entry, or q_n itself when the residual
 *     is empty) or argmax q_gamma.  Draft logits are not read, no random
 *     number is drawn, top_k changes nothing, and token_probs / accept_ur of
 *     sv_verify_debug are all NaN.
 *   Results are repeatable bit for bit: the same arguments on the same
 *   device give the same outputs.  The random numbers depend only on (seed,
 *   seq_offset + b, position, v), so a sub-batch called with the matching
 *   seq_offset draws exactly what the full batch draws.  The softmax sums are
 *   fp32, and without top-k a row's sum is split into chunks whose number
 *   follows the batch size and the device's compute-unit count; a different
 *   batch size can therefore round p(t), q(t) differently in the last bits,
 *   which changes a decision only where the acceptance uniform lies within
 *   that rounding of q(t)/p(t) or two Gumbel keys are that close.
 *
 * Layouts: row-major, contiguous.
 *   target_logits [B][gamma+1][V], draft_logits [B][gamma][V], both of dtype
 *   `dtype` (SV_F32: IEEE binary32; SV_BF16: bfloat16 as 16-bit patterns);
 *   logits must be finite or -inf and every row must keep a finite logit.
 *   draft_tokens [B][gamma] int32.
 *   out_tokens [B][gamma+1] int32: drafts 0..n-1, the sampled token at n,
 *   -1 after it.  n_accepted [B] int32: n in [0, gamma]; a sequence with a
 *   drafted token outside [0, V) gets n_accepted = -1 and a row of -1.
 *
 * Ownership: the caller allocates every buffer (device memory of the current
 * HIP device, or memory the device can address).  The library allocates
 * nothing and keeps no state between calls beyond the workspace contents
 * (sv_verify_noalloc's workspace is a fixed buffer inside the library).
 *
 * Workspace: sv_workspace_bytes() bytes of device memory, 256-byte aligned.
 * Its contents before a call do not matter (each call first clears the part
 * it counts in), and one workspace may serve calls of any shape in turn.  One
 * workspace serves one call at a time: calls that overlap (different streams,
 * same workspace) race.
 *
 * Errors: argument errors return SV_EINVAL before anything is enqueued
 * (null pointer, B < 1, gamma not in [1, 64], V < 2 or V > 2^28, temperature
 * not finite or < 0, top_p NaN, unknown dtype, a logits pointer not aligned
 * to its element size, workspace too small or misaligned, a grid that would
 * not fit 32 bits).  A failed launch returns
 * SV_EHIP.  Calls never synchronise.
 */
#ifndef SPECVERIFY_H
#define SPECVERIFY_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__)
#define SV_API __attribute__((visibility("default")))
#else
#define SV_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { SV_F32 = 0, SV_BF16 = 1 } sv_dtype;
typedef enum { SV_OK = 0, SV_EINVAL = 1, SV_EHIP = 2 } sv_status;

/* Bytes of device workspace sv_verify needs for this shape, at any temperature
 * (0 on bad shape). */
SV_API size_t sv_workspace_bytes(int32_t B, int32_t gamma, int32_t V, int32_t top_k, int32_t dtype);

/* One verification step; see the top of this file.  All pointers are device
 * pointers; `stream` is a hipStream_t (NULL = default stream). */
SV_API sv_status sv_verify(const void *target_logits, const void *draft_logits,
                    const int32_t *draft_tokens,
                    int32_t B, int32_t gamma, int32_t V, int32_t dtype,
                    float temperature, int32_t top_k, float top_p,
                    uint64_t seed, uint64_t seq_offset,
                    int32_t *out_tokens, int32_t *n_accepted,
                    void *workspace, size_t workspace_bytes, void *stream);

/* sv_verify without a workspace argument, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation.  The workspace is a buffer inside the library,
 * SV_NOALLOC_WORKSPACE_BYTES of device memory on each GPU the library runs on,
 * held until the process ends; its address is looked up once per device on
 * the first call made with that device current.  Same arguments (minus the
 * workspace), kernels and results as sv_verify.  SV_EINVAL, before anything
 * is enqueued, when sv_workspace_bytes() of the shape exceeds
 * SV_NOALLOC_WORKSPACE_BYTES (for example top_k = 1024 at B = 256, gamma = 8),
 * and for every argument error of sv_verify; SV_EHIP when the buffer's
 * address cannot be obtained or a launch fails.  Nothing is allocated.  Every
 * call on one GPU uses that GPU's single buffer: calls that overlap on one
 * GPU (different streams, or host threads enqueueing at once) race; calls
 * enqueued one after another on one stream do not.  Each call clears what it
 * counts in before use, so the buffer's earlier contents do not matter. */
#define SV_NOALLOC_WORKSPACE_BYTES ((size_t)32 << 20)
SV_API sv_status sv_verify_noalloc(const void *target_logits, const void *draft_logits,
                            const int32_t *draft_tokens,
                            int32_t B, int32_t gamma, int32_t V, int32_t dtype,
                            float temperature, int32_t top_k, float top_p,
                            uint64_t seed, uint64_t seq_offset,
                            int32_t *out_tokens, int32_t *n_accepted, void *stream);

/* sv_verify plus per-position diagnostics for tests (device outputs, either
 * may be NULL):
 *   token_probs [B][gamma][2] float: p_j(t_j), q_j(t_j) for every judged
 *     position j (0 .. n_accepted, below gamma);
 *   accept_ur [B][gamma][2] float: the acceptance uniform u_j and the ratio
 *     q_j(t_j)/p_j(t_j) (+inf when p_j(t_j) = 0, 0 when q_j(t_j) = 0) for
 *     every judged position j.
 *   Positions after the first rejection are not judged (their rows need not
 *   be read) and hold NaN in both arrays; so does every position of an
 *   invalid sequence and, in the arg-max mode, every position. */
SV_API sv_status sv_verify_debug(const void *target_logits, const void *draft_logits,
                          const int32_t *draft_tokens,
                          int32_t B, int32_t gamma, int32_t V, int32_t dtype,
                          float temperature, int32_t top_k, float top_p,
                          uint64_t seed, uint64_t seq_offset,
                          int32_t *out_tokens, int32_t *n_accepted,
                          void *workspace, size_t workspace_bytes, void *stream,
                          float *token_probs, float *accept_ur);

/* sv_verify that also records caller-created hipEvent_t handles on `stream`
 * around each kernel it enqueues, for per-kernel timing: events[2i] before
 * and events[2i+1] after launch i.  `n_events` is the array length; launches
 * beyond n_events/2 are not bracketed.  *n_launches receives the number of
 * kernels enqueued (may be NULL).  Same results as sv_verify. */
SV_API sv_status sv_verify_timed(const void *target_logits, const void *draft_logits,
                          const int32_t *draft_tokens,
                          int32_t B, int32_t gamma, int32_t V, int32_t dtype,
                          float temperature, int32_t top_k, float top_p,
                          uint64_t seed, uint64_t seq_offset,
                          int32_t *out_tokens, int32_t *n_accepted,
                          void *workspace, size_t workspace_bytes, void *stream,
                          void *const *events, int32_t n_events, int32_t *n_launches);

/* Name of kernel launch i of a call with these arguments (for matching event
 * timings to profiler rows); NULL past the last launch. */
SV_API const char *sv_launch_name(int32_t B, int32_t gamma, int32_t V, int32_t dtype,
                           int32_t top_k, float top_p, float temperature, int32_t i);

/* Draft tokens for a verification step: token j of sequence b drawn on the
 * GPU from the draft row's adjusted distribution p_j = softmax(topk(z) / T)
 * (the same temperature, top-k, top-p and arg-max conventions as sv_verify), the
 * step the small model takes before the large one verifies (page ai-trend.me,
 * section "어떻게 작동하나").  The draw is Gumbel-max: the arg-max over the kept
 * entries of ln p_v - ln E_v, E_v = -ln U_v, U_v = (2 * (w >> 9) + 1) * 2^-24,
 * w the Philox4x32-10 word at (seq = seq_offset + b, pos = j, v, purpose 2);
 * ties go to the smaller v.  At temperature 0 the token is the row's first
 * largest logit.
 *   draft_logits [B][gamma][V] of dtype `dtype` (device); draft_tokens
 *   [B][gamma] int32 (device, caller-owned).  No workspace; nothing is
 *   allocated.  Errors: SV_EINVAL for null pointers, a bad shape or dtype,
 *   temperature not finite or < 0, top_p NaN, misaligned pointers; SV_EHIP
 *   for a failed launch.  Enqueued on
 *   `stream`, never synchronises. */
SV_API sv_status sv_draft_sample(const void *draft_logits, int32_t B, int32_t gamma, int32_t V, int32_t dtype,
                          float temperature, int32_t top_k, float top_p, uint64_t seed, uint64_t seq_offset,
                          int32_t *draft_tokens, void *stream);

/* Acceptance counts of a step: hist[0] = sequences flagged invalid
 * (n_accepted < 0; values above gamma, which sv_verify never writes, are
 * counted there too), hist[1 + i] = sequences with n_accepted = i, i in
 * [0, gamma].  n_accepted [B] and hist [gamma + 2] are int32 device buffers
 * (hist caller-owned, fully overwritten).  SV_EINVAL for null or misaligned
 * pointers, B < 1 or gamma not in [1, 64]; SV_EHIP for a failed launch. */
SV_API sv_status sv_accept_histogram(const int32_t *n_accepted, int32_t B, int32_t gamma, int32_t *hist,
                              void *stream);

/* Measurement aids (not part of a verification step).
 *
 * sv_probe_read: reads `bytes` (a multiple of 16 is read; the rest ignored)
 * of device memory at x (16-byte aligned) once, `grid` blocks of 256 threads
 * each streaming a contiguous slab with four 16-byte loads in flight per
 * thread, and writes one float per block to out [grid] (device).  With
 * nontemporal != 0 the loads carry the non-temporal (streaming) cache hint.
 * Timing it gives the read rate a plain kernel reaches on this GPU, the
 * context the verification kernels' rates are read against.
 *
 * sv_probe_variates: out[i] (device, n floats) = the exponential variate in
 * base 2 that the samplers derive from Philox word w = (first + i) << 9, i.e.
 * -log2(U) for U = (2 (first + i) + 1) 2^-24, computed by the same device
 * code; first + n <= 2^23 covers every possible U.
 *
 * sv_probe_math: out[i] = the native exp2 (op 0) or log2 (op 1) the kernels
 * use, of x[i] (device arrays of n floats).
 *
 * All three: SV_EINVAL for null or misaligned pointers and out-of-range
 * sizes, SV_EHIP for a failed launch; enqueued on `stream`. */
SV_API sv_status sv_probe_read(const void *x, size_t bytes, float *out, int32_t grid, int32_t nontemporal,
                               void *stream);
SV_API sv_status sv_probe_variates(uint32_t first, int32_t n, float *out, void *stream);
SV_API sv_status sv_probe_math(const float *x, int32_t n, int32_t op, float *out, void *stream);

/* The hipError_t behind the last SV_EHIP that sv_verify (any variant),
 * sv_draft_sample or sv_accept_histogram returned on the calling host thread
 * (hipSuccess if none). */
SV_API int32_t sv_last_hip_error(void);

/* Human-readable status. */
SV_API const char *sv_status_string(sv_status s);

/* Library version string. */
SV_API const char *sv_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SPECVERIFY_H */
