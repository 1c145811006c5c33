"""Edge cases of the rule on the GPU, against the oracle (bar: tests/parity.py).

* Drafted tokens the draft gives no mass (p(t) = 0, q(t) > 0: always kept),
  tokens the target gives no mass (q(t) = 0: always rejected), and both at
  once on identical rows, where the residual max(0, q - p) is empty and the
  replacement comes from q (the fallback reading R6).  Page "스펙큘러티브 디코딩
  — 작은 모델이 먼저 쓰고 큰 모델이 검사한다" §1 gives the rule; the zero cases are
  the readings R3 and R6.  Built both with -inf logits and with tokens outside
  a top-k set, on the dense path (one launch of all positions, and one
  position per launch), on the top-k path, in fp32 and bf16.
* Top-k rows whose lower bound on the K-th logit falls among all -inf
  entries (a whole 16-byte vector of -inf in a row where exactly K threads
  hold entries), for verification and draft sampling.
* -0 and +0 at the top-k threshold and inside the nucleus: equal logits, so
  the smaller index ranks first.
* Repeated calls are bit-identical (acceptance uniforms, ratios,
  probabilities, outputs), on the top-k path with lists in registers and in
  LDS.
"""
import sys

import numpy as np
import pytest

import parity as PT
from oracle import oracle as O
from workloads import synth as I

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _check(rep, label):
    s = rep.summary()
    _say(label, s)
    assert rep.ok(), f"{label}: {s}"
    assert rep.mismatches == 0, f"{label}: {s}"


def zero_prob_workload(rng, B, gamma, V, top_k=0, bf16=False, sigma=0.4, frac=0.5):
    """Target N(0, 2^2), draft = target + N(0, sigma^2), tokens drawn from the
    draft; then about `frac` of the positions get one of three edits:
      1  p(t) = 0 < q(t): the draft's logit at t is -inf (no top-k) or below
         the draft's K-th largest while t stays in the target's top-K;
      2  q(t) = 0 < p(t): the same on the target side;
      3  p(t) = q(t) = 0 on identical rows: the draft row becomes a copy of the
         target row and t is dropped from both, so the residual is empty.
    Returns the workload and the edit kinds [B, gamma]."""
    t = rng.normal(0, 2, (B, gamma + 1, V)).astype(np.float32)
    d = (t[:, :gamma] + rng.normal(0, sigma, (B, gamma, V))).astype(np.float32)
    tok = I.sample_rows(d.reshape(-1, V), 1.0, top_k, rng).reshape(B, gamma)
    kind = np.where(rng.random((B, gamma)) < frac, rng.integers(1, 4, (B, gamma)), 0)
    for b in range(B):
        for j in range(gamma):
            k = kind[b, j]
            if k == 0:
                continue
            if k == 3:
                d[b, j] = t[b, j]
            v = int(tok[b, j])
            if top_k:
                # t outside one or both kept sets, inside the other
                lo_t, lo_d = t[b, j].min() - 1.0, d[b, j].min() - 1.0
                hi_t, hi_d = t[b, j].max() + 1.0, d[b, j].max() + 1.0
                if k == 1:
                    t[b, j, v], d[b, j, v] = hi_t, lo_d
                elif k == 2:
                    t[b, j, v], d[b, j, v] = lo_t, hi_d
                else:
                    t[b, j, v] = d[b, j, v] = lo_t
            else:
                if k in (1, 3):
                    d[b, j, v] = -np.inf
                if k in (2, 3):
                    t[b, j, v] = -np.inf
    if bf16:
        t, d = I.f32_to_bf16_bits(t), I.f32_to_bf16_bits(d)
    return I.from_arrays(t, d, tok, top_k=top_k), kind


ZERO_CASES = [("dense-f32", 0, False, 48, 4, 3000),
              ("dense-bf16", 0, True, 48, 4, 3001),
              ("topk-f32", 20, False, 48, 4, 3000),
              ("topk-bf16", 20, True, 48, 4, 3001),
              ("topk-K200-f32", 200, False, 24, 3, 5000)]


@pytest.mark.parametrize("name,K,bf16,B,gamma,V", ZERO_CASES, ids=[c[0] for c in ZERO_CASES])
def test_zero_probability_tokens(name, K, bf16, B, gamma, V):
    rng = np.random.default_rng(606 + K + bf16)
    w, kind = zero_prob_workload(rng, B, gamma, V, top_k=K, bf16=bf16)
    _say(f"case zero-prob {name} B={B} gamma={gamma} V={V} K={K} kinds={np.bincount(kind.ravel(), minlength=4)}")
    tensors = PT.to_device(w)
    fallback = 0
    for seed in (41, 42):
        g = PT.run_gpu(w, seed, tensors=tensors)
        _check(PT.compare(w, seed, g), f"zero-prob {name} seed {seed}")
        res = O.verify(w.target, w.draft, w.tokens, w.temperature, w.top_k, seed=seed)
        fallback += int(np.sum(res.flags & 1))
        # the edits decide the judged positions whatever the uniforms
        for b in range(B):
            n = int(res.n_accepted[b])
            for j in range(min(n + 1, gamma)):
                if kind[b, j] == 1:
                    assert j < n, (b, j)          # p(t) = 0 < q(t): kept
                elif kind[b, j] in (2, 3):
                    assert j == n, (b, j)         # q(t) = 0: rejected here
    _say(f"{name}: empty residuals (q sampled instead) {fallback}")
    assert fallback > 0


def test_zero_probability_one_position_per_launch():
    """The same edits on inputs large enough (537 MB of rows) that the dense
    path judges one position per launch."""
    import rejection_sampling_verify_17_amd as S
    rng = np.random.default_rng(707)
    w, kind = zero_prob_workload(rng, 64, 8, 131072, sigma=0.3, frac=0.25)
    assert S.launch_names(w.B, w.gamma, w.V, S.SV_F32, 0)[:2] == ["k_rows", "k_judge"]
    _say(f"case zero-prob window-1 B={w.B} gamma={w.gamma} V={w.V} kinds={np.bincount(kind.ravel(), minlength=4)}")
    tensors = PT.to_device(w)
    g = PT.run_gpu(w, 43, tensors=tensors)
    _check(PT.compare(w, 43, g), "zero-prob window-1")
    res = O.verify(w.target, w.draft, w.tokens, w.temperature, w.top_k, seed=43)
    _say(f"window-1: empty residuals {int(np.sum(res.flags & 1))}, n histogram "
         f"{np.bincount(g.n_accepted, minlength=w.gamma + 1).tolist()}")
    assert int(np.sum(res.flags & 1)) > 0


def masked_vector_rows(rng, B, gamma, V, K, bf16, vectors):
    """Rows where exactly K threads of a 1024-thread row block hold entries
    (V = K 16-byte vectors) and some whole vectors are -inf."""
    ne = 8 if bf16 else 4
    t = rng.normal(0, 2, (B, gamma + 1, V)).astype(np.float32)
    d = (t[:, :gamma] + rng.normal(0, 1, (B, gamma, V))).astype(np.float32)
    for iv in vectors:
        t[:, :, iv * ne:(iv + 1) * ne] = -np.inf
        d[:, :, iv * ne:(iv + 1) * ne] = -np.inf
    tok = I.sample_rows(d.reshape(-1, V), 1.0, K, rng).reshape(B, gamma)
    if bf16:
        t, d = I.f32_to_bf16_bits(t), I.f32_to_bf16_bits(d)
    return I.from_arrays(t, d, tok, top_k=K)


MASKED = [("f32-V256-K64", False, 256, 64, [5]),
          ("f32-V256-K64-three", False, 256, 64, [0, 31, 63]),
          ("bf16-V256-K32", True, 256, 32, [1]),
          ("bf16-V256-K32-two", True, 256, 32, [0, 17]),
          ("f32-V256-K60", False, 256, 60, [2, 3])]


@pytest.mark.parametrize("name,bf16,V,K,vectors", MASKED, ids=[m[0] for m in MASKED])
def test_topk_bound_among_neg_inf(name, bf16, V, K, vectors):
    import torch
    import rejection_sampling_verify_17_amd as S
    rng = np.random.default_rng(808 + K + len(vectors))
    w = masked_vector_rows(rng, 16, 3, V, K, bf16, vectors)
    _say(f"case masked-vector {name} B={w.B} gamma={w.gamma} V={V} K={K} vectors={vectors}")
    for seed in (51, 52):
        g = PT.run_gpu(w, seed)
        _check(PT.compare(w, seed, g), f"masked-vector {name} seed {seed}")
        assert np.all(g.n_accepted >= 0) and np.all(g.out_tokens[np.arange(w.B), g.n_accepted] >= 0)
    # draft sampling over the same rows
    drf = PT.to_device(w)[1]
    got = S.draft_sample(drf, w.temperature, w.top_k, seed=53).cpu().numpy()
    torch.cuda.synchronize()
    want, gap = O.draft_sample(w.draft, w.temperature, w.top_k, seed=53)
    ok = (got == want) | (gap < PT.KNIFE)
    assert ok.all(), f"draft draws differ at {np.argwhere(~ok)[:5].tolist()}"


def signed_zero_workload(rng, B, gamma, V, K, top_p, bf16):
    """Integer logits in [-2, 2] with about half of the zeros stored as -0.0;
    K falls among the zeros for most rows."""
    def rows(shape):
        z = rng.integers(-2, 3, shape).astype(np.float32)
        neg = (z == 0) & (rng.random(shape) < 0.5)
        z[neg] = -0.0
        return z
    t = rows((B, gamma + 1, V))
    d = rows((B, gamma, V))
    tok = I.sample_rows(d.reshape(-1, V), 1.0, K, rng, top_p=top_p).reshape(B, gamma)
    if bf16:
        t, d = I.f32_to_bf16_bits(t), I.f32_to_bf16_bits(d)
    return I.from_arrays(t, d, tok, top_k=K, top_p=top_p)


# integer logits in [-2, 2]: about 2/5 of a row is positive and 1/5 zero, so
# K between 0.4 V and 0.6 V puts the K-th largest among the zeros; P = 0.97
# after such a K puts the nucleus cut among them too
SIGNED = [("f32-K50", False, 100, 50, 1.0), ("bf16-K50", True, 100, 50, 1.0),
          ("f32-K50-P0.97", False, 100, 50, 0.97), ("bf16-K55-P0.97", True, 100, 55, 0.97),
          ("f32-V1000-K500", False, 1000, 500, 1.0)]


@pytest.mark.parametrize("name,bf16,V,K,P", SIGNED, ids=[s[0] for s in SIGNED])
def test_signed_zero_at_threshold(name, bf16, V, K, P):
    import torch
    import rejection_sampling_verify_17_amd as S
    rng = np.random.default_rng(909 + K)
    w = signed_zero_workload(rng, 12, 3, V, K, P, bf16)
    z = I.logits_f32(w.target)
    above = (z > 0).sum(axis=2)
    zeros = (z == 0).sum(axis=2)
    at_zero = np.mean((above < K) & (above + zeros >= K))
    _say(f"case signed-zero {name} K={K} P={P}: threshold among the zeros in {at_zero:.2f} of target rows")
    assert at_zero > 0.5
    for seed in (61, 62):
        g = PT.run_gpu(w, seed)
        _check(PT.compare(w, seed, g), f"signed-zero {name} seed {seed}")
    got = S.draft_sample(PT.to_device(w)[1], w.temperature, w.top_k, seed=63, top_p=w.top_p).cpu().numpy()
    torch.cuda.synchronize()
    want, gap, margin = O.draft_sample(w.draft, w.temperature, w.top_k, seed=63, top_p=w.top_p, with_margin=True)
    ok = (got == want) | (gap < PT.KNIFE) | (margin < PT.KNIFE)
    assert ok.all(), f"draft draws differ at {np.argwhere(~ok)[:5].tolist()}"


REPEAT = [("c3", None, 0), ("c3", 64, 200), ("c2", 16, 0)]


@pytest.mark.parametrize("name,B,K", REPEAT, ids=[f"{r[0]}-K{r[2] or 'spec'}" for r in REPEAT])
def test_repeat_calls_bit_identical(name, B, K):
    """Same arguments twice: outputs and every diagnostic bit for bit (the
    top-k statistics over LDS candidates are summed in fixed point, so the
    order the gather's atomics hand out slots does not matter)."""
    w = I.make(name, B=B) if not K else I.make(name, B=B, top_k=K)
    _say(f"case repeat {name} B={w.B} K={w.top_k}")
    t = PT.to_device(w)
    a = PT.run_gpu(w, 71, tensors=t)
    for _ in range(2):
        b = PT.run_gpu(w, 71, tensors=t)
        assert np.array_equal(a.out_tokens, b.out_tokens) and np.array_equal(a.n_accepted, b.n_accepted)
        assert np.array_equal(a.token_probs.view(np.uint32), b.token_probs.view(np.uint32))
        assert np.array_equal(a.accept_ur.view(np.uint32), b.accept_ur.view(np.uint32))
    if K:
        _check(PT.compare(w, 71, a), f"repeat {name} K={K}")
