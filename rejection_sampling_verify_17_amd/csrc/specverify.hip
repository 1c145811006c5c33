// C ABI of the verification library: argument checks, workspace layout,
// launch geometry.  The operation and every convention are documented in
// include/specverify.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstring>

#include "specverify.h"
#include "sv_draft.h"
#include "sv_greedy.h"
#include "sv_kernels.h"
#include "sv_topk.h"

namespace {

using namespace sv;

constexpr int kMaxGamma = 64;           // one wave ballots all positions
constexpr int kMaxV = 1 << 28;          // byte offsets of a row fit 32 bits
constexpr int kListMax = 1024;          // top-k lists kept up to this K
constexpr double kSmallRows = 256e6;    // bytes of all rows below which one launch reads them all
constexpr int kSlotsPerCU = 8;          // resident k_rows blocks per compute unit
constexpr size_t kAlign = 256;
constexpr int kMaxDevices = 64;
// Workspace of sv_verify_noalloc: a buffer inside the library, one per GPU the
// library runs on (each device holds its own copy of this array).  Host code
// never uses the array's name as an address: the device address comes from
// hipGetSymbolAddress, per device.
constexpr size_t kStaticWorkspace = SV_NOALLOC_WORKSPACE_BYTES;
__device__ __align__(256) unsigned char scratch[kStaticWorkspace];

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// The HIP error behind the last SV_EHIP this host thread received.
thread_local hipError_t g_last_hip_error = hipSuccess;
bool launch_ok() {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) g_last_hip_error = e;
  return e == hipSuccess;
}

// Compute units of the current device (queried once per device).
int compute_units() {
  static std::atomic<int> cached[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) dev = -1;
  if (dev >= 0) {
    const int c = cached[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev < 0 ? 0 : dev) != hipSuccess || n <= 0)
    n = 256;
  if (dev >= 0) cached[dev].store(n, std::memory_order_relaxed);
  return n;
}

constexpr int kMaxWindows = 9;  // windows [0,1), [1,3), [3,7), ... over at most 65 rows

struct Plan {
  bool topk, greedy;
  bool radix;  // top-k path with the mass-weighted nucleus cut (no top-k, or K > kListMax)
  int window;  // positions whose statistics one launch computes (dense path)
  int nch, nch_max, nvec, ngb, cs_max, klist;
  // arg-max mode: windows [gw0, gw1) of target rows with gnch chunks per row
  int nwin, gw0[kMaxWindows], gw1[kMaxWindows], gnch[kMaxWindows], gstride;
  size_t off_part, off_ztok, off_slist, off_sst, off_tlist, off_lcnt, off_icnt, off_pcnt, off_pbest;
  size_t off_nseq, off_state, off_rowinfo, off_lists, off_gpart;
  size_t total;
};

bool shape_ok(int32_t B, int32_t gamma, int32_t V, int32_t dtype) {
  return B >= 1 && gamma >= 1 && gamma <= kMaxGamma && V >= 2 && V <= kMaxV &&
         (dtype == SV_F32 || dtype == SV_BF16);
}

// `resident`: k_rows blocks resident at once (the grid of a launch).
// `greedy`: the arg-max mode (temperature 0), where top-k changes nothing.
// End of the window that starts at w0 < n when positions 0..n-1 are walked
// in windows [0, 1), [1, 3), [3, 7), [7, 15), ... (each twice the last); a
// window that would leave one position over runs to n.  With low acceptance
// few sequences reach the later windows, and a launch over few rows costs
// about the same as one over many, so fewer launches win.
int window_end(int n, int w0) {
  if (w0 == 0) return 1;
  const int w1 = 2 * w0 + 1;
  return n - w1 <= 1 ? n : w1;
}

// `nucleus`: top-p on (0 < top_p < 1, temperature > 0): the kept sets are cut
// per row, so the rows go through the top-k path even without top-k.
Plan make_plan(int32_t B, int32_t gamma, int32_t V, int32_t top_k, int32_t dtype, bool greedy, bool nucleus = false,
               int resident = 2048) {
  Plan p{};
  const int ne = dtype == SV_BF16 ? 8 : 4;
  p.nvec = (V + 2 * ne - 2) / ne;  // vectors covering a row at any 16-byte offset
  p.ngb = (V + ne - 1) / ne;       // group blocks of ne entries
  p.greedy = greedy;
  const bool has_k = top_k > 0 && top_k < V;
  p.topk = !greedy && (has_k || nucleus);
  p.klist = (p.topk && has_k && top_k <= kListMax) ? top_k : 0;
  p.radix = p.topk && nucleus && !(has_k && top_k <= kListMax);
  if (greedy) {
    // every thread keeps at least kGreedyU vectors; a launch gets about one
    // block per resident slot (dead sequences' blocks return at once)
    p.gstride = std::max(1, p.nvec / (kGreedyThreads * kGreedyU));
    for (int w0 = 0; w0 <= gamma; ++p.nwin) {
      const int w1 = window_end(gamma + 1, w0);
      const long long rows = (long long)B * (w1 - w0);
      p.gw0[p.nwin] = w0;
      p.gw1[p.nwin] = w1;
      p.gnch[p.nwin] = (int)std::max(1LL, std::min<long long>(p.gstride, (resident + rows - 1) / rows));
      w0 = w1;
    }
  } else if (!p.topk) {
    // Reading rows past the first rejection costs bytes; every extra launch
    // costs a fixed ~10 us.  When all rows together are small, one launch
    // reads them all; otherwise one position per launch.
    const double all_rows = 2.0 * B * gamma * (double)V * (dtype == SV_BF16 ? 2 : 4);
    p.window = all_rows <= kSmallRows ? gamma : 1;
    // launch 0: at most one statistics item per resident block, so no block
    // takes a second one while others idle; every thread keeps at least two
    // vectors
    const int max_ch = std::max(1, p.nvec / (2 * kThreads));
    const int rows = B * p.window;
    p.nch_max = max_ch;
    p.nch = std::max(1, std::min(resident / rows, max_ch));
    // a sampled row is split so that every thread keeps at least one group block
    p.cs_max = std::max(1, std::min(kMaxSampleChunks, p.ngb / kThreads));
  }
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off = align_up(off + bytes); return o; };
  // Nothing here is read before this call writes it: the workspace needs no
  // initialisation and may serve calls of any shape in turn.
  const size_t dense = (p.topk || p.greedy) ? 0 : 1;
  p.off_part = take(dense * B * gamma * p.nch_max * sizeof(float4));
  p.off_ztok = take(dense * B * gamma * sizeof(float2));
  p.off_slist = take(dense * 3 * B * sizeof(int2));
  p.off_sst = take(dense * 3 * B * sizeof(float4));
  p.off_tlist = take(dense * 3 * B * sizeof(int32_t));
  p.off_lcnt = take(dense * 3 * 2 * sizeof(int32_t));
  p.off_icnt = take(dense * B * sizeof(int32_t));
  p.off_pcnt = take(dense * B * sizeof(int32_t));
  p.off_pbest = take(dense * B * sizeof(unsigned long long));
  p.off_nseq = take((size_t)B * sizeof(int32_t));
  p.off_state = take((p.topk || p.greedy) ? 2 * (size_t)B * sizeof(int32_t) : 0);
  const size_t slots = (size_t)B * (2 * gamma);
  p.off_rowinfo = take(p.topk ? slots * sizeof(uint4) : 0);
  p.off_lists = take(p.klist ? slots * (size_t)p.klist * sizeof(int2) : 0);
  p.off_gpart = take(p.greedy ? (size_t)B * (gamma + 1) * p.gstride * sizeof(unsigned long long) : 0);
  p.total = off;
  return p;
}

// One workspace size serves every temperature and top-p.
size_t workspace_total(int32_t B, int32_t gamma, int32_t V, int32_t top_k, int32_t dtype) {
  return std::max({make_plan(B, gamma, V, top_k, dtype, false).total,
                   make_plan(B, gamma, V, top_k, dtype, true).total,
                   make_plan(B, gamma, V, top_k, dtype, false, true).total});
}


template <int DT>
struct Launches {
  // Dense: k_rows for the first window, k_rows that judges it in every block
  // and reads the next window, then k_rows per further window and once more
  // to sample.  Top-k: position 0, the other positions, then the judgement
  // and draw.  Arg-max: windows of target rows, then the judgement.
  static sv_status run(const Args &a, const Plan &p, hipStream_t stream, void *const *events, int n_events,
                       int *n_launches) {
    int li = 0;
    auto before = [&]() {
      if (events && 2 * li < n_events) (void)hipEventRecord((hipEvent_t)events[2 * li], stream);
    };
    auto after = [&]() -> bool {
      if (events && 2 * li + 1 < n_events) (void)hipEventRecord((hipEvent_t)events[2 * li + 1], stream);
      ++li;
      return launch_ok();
    };
    bool ok = true;
    if (p.greedy) {
      // one launch per window of target rows, then one that judges the last
      int p0 = 0, nprev = 1;
      for (int L = 0; L <= p.nwin; ++L) {
        const int w0 = L < p.nwin ? p.gw0[L] : a.gamma + 1;
        const int w1 = L < p.nwin ? p.gw1[L] : a.gamma + 1;
        const int nch = L < p.nwin ? p.gnch[L] : 1;
        const long long grid = (long long)a.B * std::max(1, w1 - w0) * nch;
        before();
        hipLaunchKernelGGL(k_greedy_step<DT>, dim3((unsigned)grid), dim3(kGreedyThreads), 0, stream, a, L, p0, w0,
                           w1, nch, nprev);
        ok = ok && after();
        p0 = w0;
        nprev = nch;
      }
    } else if (!p.topk) {
      const int slots = kSlotsPerCU * compute_units();
      auto grid = [&](long long items) { return (unsigned)std::max(1LL, std::min<long long>(slots, items)); };
      int w0 = std::min(a.gamma, p.window);
      before();
      hipLaunchKernelGGL((k_rows<DT, 0>), dim3(grid((long long)a.B * w0 * p.nch)), dim3(kThreads), 0, stream, a, 0, 0,
                         w0, 0, 0, 0);
      ok = ok && after();
      // Every position read at once: each block of launch 1 judges its
      // sequence itself, then draws its chunk of the sampled row (saves a
      // launch).  Otherwise k_judge judges the first window and lists the
      // work of launch 1: a judgement in every block would hold back the
      // statistics stream of the next window, which costs more than the
      // launch.
      const bool judge_in_block = w0 == a.gamma;
      if (!judge_in_block) {
        before();
        hipLaunchKernelGGL(k_judge<DT>, dim3((a.B + kJudgeWaves - 1) / kJudgeWaves), dim3(kJudgeWaves * kWave), 0,
                           stream, a, w0);
        ok = ok && after();
      }
      for (int launch = 1;; ++launch) {
        const int w1 = std::min(a.gamma, w0 + p.window);
        before();
        if (launch == 1 && judge_in_block) {
          // kb blocks per sequence, each judges, then draws one chunk
          const int cs1 = std::max(1, std::min(p.cs_max, slots / a.B));
          hipLaunchKernelGGL((k_rows<DT, 1>), dim3((unsigned)((long long)a.B * cs1)), dim3(kThreads), 0, stream, a,
                             1, w0, w1, cs1, 0, cs1);
        } else {
          const long long items = (long long)a.B * std::max((w1 - w0) * p.nch_max, p.cs_max);
          if (w0 == a.gamma)  // sampling only
            hipLaunchKernelGGL((k_rows<DT, 3>), dim3(grid(items)), dim3(kThreads), 0, stream, a, launch, w0, w1, 0,
                               0, 0);
          else
            hipLaunchKernelGGL((k_rows<DT, 2>), dim3(grid(items)), dim3(kThreads), 0, stream, a, launch, w0, w1, 0,
                               0, 0);
        }
        ok = ok && after();
        if (w0 == a.gamma) break;
        w0 = w1;
      }
    } else {
      // one launch per window, then one that judges the last window
      const int G = a.gamma;
      int launch = 0, p0 = 0, w0 = 0;
      while (true) {
        const int w1 = w0 < G ? window_end(G, w0) : G;
        const int per_seq = w1 > w0 ? 2 * (w1 - w0) : 1;
        before();
        if (p.radix)
          hipLaunchKernelGGL((k_topk_step<DT, true>), dim3(a.B * per_seq), dim3(kTopkThreads), 0, stream, a, launch,
                             p0, w0, w1);
        else
          hipLaunchKernelGGL((k_topk_step<DT, false>), dim3(a.B * per_seq), dim3(kTopkThreads), 0, stream, a, launch,
                             p0, w0, w1);
        ++launch;
        ok = ok && after();
        if (w0 == G) break;
        p0 = w0;
        w0 = w1;
      }
    }
    if (n_launches) *n_launches = li;
    return ok ? SV_OK : SV_EHIP;
  }
};

// Every workspace pointer the kernels of the chosen path dereference is set
// (a pointer left null for one path would otherwise fault on the GPU).
bool pointers_set(const Args &a, const Plan &p) {
  if (!a.nseq) return false;
  if (p.greedy) return a.state && a.gpart && a.gstride >= 1;
  if (p.topk) return a.state && a.rowinfo && (p.klist == 0 || a.lists);
  return a.part && a.ztok && a.slist && a.sst && a.tlist && a.lcnt && a.icnt && a.pcnt && a.pbest && a.nch >= 1 &&
         a.nch_max >= a.nch && a.cs_max >= 1;
}

sv_status verify_impl(const void *target, const void *draft, const int32_t *tokens, int32_t B, int32_t gamma,
                      int32_t V, int32_t dtype, float temperature, int32_t top_k, float top_p, uint64_t seed,
                      uint64_t seq_offset, int32_t *out_tokens, int32_t *n_accepted, void *workspace,
                      size_t workspace_bytes, void *stream, float *token_probs, float *accept_ur,
                      void *const *events, int32_t n_events, int32_t *n_launches) {
  if (n_launches) *n_launches = 0;
  if (!target || !draft || !tokens || !out_tokens || !n_accepted || !workspace) return SV_EINVAL;
  if (!shape_ok(B, gamma, V, dtype)) return SV_EINVAL;
  if (!std::isfinite(temperature) || !(temperature >= 0.0f)) return SV_EINVAL;  // 0: arg-max mode
  const bool greedy = temperature == 0.0f;
  // nucleus: 0 < top_p < 1 (else off), with or without top-k (the arg-max
  // mode ignores both)
  if (std::isnan(top_p)) return SV_EINVAL;
  const bool nucleus = !greedy && top_p > 0.0f && top_p < 1.0f;
  const uintptr_t elem = dtype == SV_BF16 ? 2 : 4;
  if (((uintptr_t)target % elem) || ((uintptr_t)draft % elem)) return SV_EINVAL;
  if (((uintptr_t)tokens % 4) || ((uintptr_t)out_tokens % 4) || ((uintptr_t)n_accepted % 4)) return SV_EINVAL;
  if ((uintptr_t)workspace % kAlign) return SV_EINVAL;
  const Plan p = make_plan(B, gamma, V, top_k, dtype, greedy, nucleus, kSlotsPerCU * compute_units());
  if (workspace_bytes < p.total) return SV_EINVAL;
  // overflow guards for grids that scale with B: the arg-max grid (B * rows
  // * chunks blocks) and the top-k grid (B * 2 * window blocks, window <= gamma)
  if (greedy && (long long)B * (gamma + 1) * p.gstride > 0x7FFFFFFFLL) return SV_EINVAL;
  if (p.topk && (long long)B * 2 * gamma > 0x7FFFFFFFLL) return SV_EINVAL;
  if (events && n_events < 0) return SV_EINVAL;

  char *ws = (char *)workspace;
  Args a{};
  a.target = target;
  a.draft = draft;
  a.tokens = tokens;
  a.B = B;
  a.gamma = gamma;
  a.V = V;
  a.top_k = (p.topk && top_k > 0 && top_k < V) ? top_k : 0;  // 0 on the top-k path: every entry, then the cut
  a.top_p = nucleus ? top_p : 1.0f;
  a.c = greedy ? 0.0f : (float)(1.4426950408889634 / (double)temperature);
  a.key0 = (uint32_t)seed;
  a.key1 = (uint32_t)(seed >> 32);
  a.seq_offset = seq_offset;
  a.out_tokens = out_tokens;
  a.n_accepted = n_accepted;
  a.token_probs = token_probs;
  a.accept_ur = accept_ur;
  a.part = (float4 *)(ws + p.off_part);
  a.ztok = (float2 *)(ws + p.off_ztok);
  a.slist = (int2 *)(ws + p.off_slist);
  a.sst = (float4 *)(ws + p.off_sst);
  a.tlist = (int32_t *)(ws + p.off_tlist);
  a.lcnt = (int32_t *)(ws + p.off_lcnt);
  a.icnt = (int32_t *)(ws + p.off_icnt);
  a.pcnt = (int32_t *)(ws + p.off_pcnt);
  a.pbest = (unsigned long long *)(ws + p.off_pbest);
  a.nch = p.nch;
  a.nch_max = p.nch_max;
  a.nvec = p.nvec;
  a.ngb = p.ngb;
  a.cs_max = p.cs_max;
  a.nseq = (int32_t *)(ws + p.off_nseq);
  a.state = (p.topk || p.greedy) ? (int32_t *)(ws + p.off_state) : nullptr;
  a.rowinfo = p.topk ? (uint4 *)(ws + p.off_rowinfo) : nullptr;
  a.lists = p.klist ? (int2 *)(ws + p.off_lists) : nullptr;
  a.klist = p.klist;
  a.gpart = p.greedy ? (unsigned long long *)(ws + p.off_gpart) : nullptr;
  a.gstride = p.gstride;

  if (!pointers_set(a, p)) return SV_EINVAL;

  (void)hipGetLastError();  // start from a clean error state
  hipStream_t s = (hipStream_t)stream;
  if (dtype == SV_BF16) return Launches<DT_BF16>::run(a, p, s, events, n_events, n_launches);
  return Launches<DT_F32>::run(a, p, s, events, n_events, n_launches);
}

// Device address of `scratch` on the current device: looked up on the first
// call on that device (with it current) and kept per device; null on failure.
void *noalloc_workspace() {
  static std::atomic<void *> addr[kMaxDevices];
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  void *p = addr[dev].load(std::memory_order_acquire);
  if (p) return p;
  const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (e != hipSuccess || !p) {
    g_last_hip_error = e != hipSuccess ? e : hipErrorInvalidSymbol;
    return nullptr;
  }
  addr[dev].store(p, std::memory_order_release);
  return p;
}

}  // namespace

extern "C" {

size_t sv_workspace_bytes(int32_t B, int32_t gamma, int32_t V, int32_t top_k, int32_t dtype) {
  if (!shape_ok(B, gamma, V, dtype)) return 0;
  return workspace_total(B, gamma, V, top_k, dtype);
}

sv_status sv_verify(const void *target_logits, const void *draft_logits, const int32_t *draft_tokens, int32_t B,
                    int32_t gamma, int32_t V, int32_t dtype, float temperature, int32_t top_k, float top_p,
                    uint64_t seed, uint64_t seq_offset, int32_t *out_tokens, int32_t *n_accepted, void *workspace,
                    size_t workspace_bytes, void *stream) {
  return verify_impl(target_logits, draft_logits, draft_tokens, B, gamma, V, dtype, temperature, top_k, top_p, seed,
                     seq_offset, out_tokens, n_accepted, workspace, workspace_bytes, stream, nullptr, nullptr,
                     nullptr, 0, nullptr);
}

sv_status sv_verify_noalloc(const void *target_logits, const void *draft_logits, const int32_t *draft_tokens,
                            int32_t B, int32_t gamma, int32_t V, int32_t dtype, float temperature, int32_t top_k,
                            float top_p, uint64_t seed, uint64_t seq_offset, int32_t *out_tokens,
                            int32_t *n_accepted, void *stream) {
  // shape and size first, so an oversized shape is refused before any HIP call
  if (!shape_ok(B, gamma, V, dtype)) return SV_EINVAL;
  if (workspace_total(B, gamma, V, top_k, dtype) > kStaticWorkspace) return SV_EINVAL;
  void *ws = noalloc_workspace();
  if (!ws) return SV_EHIP;
  return verify_impl(target_logits, draft_logits, draft_tokens, B, gamma, V, dtype, temperature, top_k, top_p, seed,
                     seq_offset, out_tokens, n_accepted, ws, kStaticWorkspace, stream, nullptr, nullptr, nullptr, 0,
                     nullptr);
}

sv_status sv_verify_debug(const void *target_logits, const void *draft_logits, const int32_t *draft_tokens,
                          int32_t B, int32_t gamma, int32_t V, int32_t dtype, float temperature, int32_t top_k,
                          float top_p, uint64_t seed, uint64_t seq_offset, int32_t *out_tokens, int32_t *n_accepted,
                          void *workspace, size_t workspace_bytes, void *stream, float *token_probs,
                          float *accept_ur) {
  return verify_impl(target_logits, draft_logits, draft_tokens, B, gamma, V, dtype, temperature, top_k, top_p, seed,
                     seq_offset, out_tokens, n_accepted, workspace, workspace_bytes, stream, token_probs,
                     accept_ur, nullptr, 0, nullptr);
}

sv_status sv_verify_timed(const void *target_logits, const void *draft_logits, const int32_t *draft_tokens,
                          int32_t B, int32_t gamma, int32_t V, int32_t dtype, float temperature, int32_t top_k,
                          float top_p, uint64_t seed, uint64_t seq_offset, int32_t *out_tokens, int32_t *n_accepted,
                          void *workspace, size_t workspace_bytes, void *stream, void *const *events,
                          int32_t n_events, int32_t *n_launches) {
  return verify_impl(target_logits, draft_logits, draft_tokens, B, gamma, V, dtype, temperature, top_k, top_p, seed,
                     seq_offset, out_tokens, n_accepted, workspace, workspace_bytes, stream, nullptr, nullptr,
                     events, n_events, n_launches);
}

const char *sv_launch_name(int32_t B, int32_t gamma, int32_t V, int32_t dtype, int32_t top_k, float top_p,
                           float temperature, int32_t i) {
  if (!shape_ok(B, gamma, V, dtype)) return nullptr;
  const bool greedy = temperature == 0.0f;
  const Plan p = make_plan(B, gamma, V, top_k, dtype, greedy, !greedy && top_p > 0.0f && top_p < 1.0f);
  if (i < 0) return nullptr;
  if (p.greedy) return i <= p.nwin ? "k_greedy_step" : nullptr;
  if (p.topk) {
    int launches = 1;  // one per window, then the judgement
    for (int w0 = 0; w0 < gamma; ++launches) w0 = window_end(gamma, w0);
    return i < launches ? "k_topk_step" : nullptr;
  }
  // k_rows for the first window, k_judge unless that window holds every
  // position, then one k_rows per further window and one to sample
  const int rows_after = (gamma + p.window - 1) / p.window;
  if (p.window >= gamma) return i < 2 ? "k_rows" : nullptr;
  if (i == 0) return "k_rows";
  if (i == 1) return "k_judge";
  return i < 2 + rows_after ? "k_rows" : nullptr;
}

sv_status sv_draft_sample(const void *draft_logits, int32_t B, int32_t gamma, int32_t V, int32_t dtype,
                          float temperature, int32_t top_k, float top_p, uint64_t seed, uint64_t seq_offset,
                          int32_t *draft_tokens, void *stream) {
  if (!draft_logits || !draft_tokens) return SV_EINVAL;
  if (!shape_ok(B, gamma, V, dtype)) return SV_EINVAL;
  if (!std::isfinite(temperature) || !(temperature >= 0.0f)) return SV_EINVAL;
  if (std::isnan(top_p)) return SV_EINVAL;
  const bool nucleus = temperature != 0.0f && top_p > 0.0f && top_p < 1.0f;
  const uintptr_t elem = dtype == SV_BF16 ? 2 : 4;
  if (((uintptr_t)draft_logits % elem) || ((uintptr_t)draft_tokens % 4)) return SV_EINVAL;
  if ((long long)B * gamma > 0x7FFFFFFFLL) return SV_EINVAL;
  const bool argmax = temperature == 0.0f;
  Args a{};
  a.draft = draft_logits;
  a.B = B;
  a.gamma = gamma;
  a.V = V;
  a.top_k = (!argmax && top_k > 0 && top_k < V) ? top_k : 0;
  a.top_p = nucleus ? top_p : 1.0f;
  a.c = argmax ? 0.0f : (float)(1.4426950408889634 / (double)temperature);
  a.argmax = argmax ? 1 : 0;
  a.key0 = (uint32_t)seed;
  a.key1 = (uint32_t)(seed >> 32);
  a.seq_offset = seq_offset;
  a.ngb = (V + (int)(16 / elem) - 1) / (int)(16 / elem);
  a.drafted = draft_tokens;
  (void)hipGetLastError();
  hipStream_t s = (hipStream_t)stream;
  const dim3 grid((unsigned)(B * gamma));
  const bool radix = nucleus && !(a.top_k > 0 && a.top_k <= kListMax);
  if (dtype == SV_BF16) {
    if (radix) hipLaunchKernelGGL((k_draft_sample<DT_BF16, true>), grid, dim3(kTopkThreads), 0, s, a);
    else hipLaunchKernelGGL((k_draft_sample<DT_BF16, false>), grid, dim3(kTopkThreads), 0, s, a);
  } else {
    if (radix) hipLaunchKernelGGL((k_draft_sample<DT_F32, true>), grid, dim3(kTopkThreads), 0, s, a);
    else hipLaunchKernelGGL((k_draft_sample<DT_F32, false>), grid, dim3(kTopkThreads), 0, s, a);
  }
  return launch_ok() ? SV_OK : SV_EHIP;
}

sv_status sv_accept_histogram(const int32_t *n_accepted, int32_t B, int32_t gamma, int32_t *hist, void *stream) {
  if (!n_accepted || !hist || B < 1 || gamma < 1 || gamma > kMaxGamma) return SV_EINVAL;
  if (((uintptr_t)n_accepted % 4) || ((uintptr_t)hist % 4)) return SV_EINVAL;
  (void)hipGetLastError();
  hipLaunchKernelGGL(k_accept_hist, dim3(1), dim3(256), 0, (hipStream_t)stream, n_accepted, B, gamma, hist);
  return launch_ok() ? SV_OK : SV_EHIP;
}

const char *sv_status_string(sv_status s) {
  switch (s) {
    case SV_OK: return "ok";
    case SV_EINVAL: return "invalid argument";
    case SV_EHIP: return "HIP launch failure";
  }
  return "unknown status";
}

int32_t sv_last_hip_error(void) { return (int32_t)g_last_hip_error; }

const char *sv_version(void) { return "specverify 0.1 (gfx950)"; }

}  // extern "C"
