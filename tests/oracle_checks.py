"""Checks that pin the oracle to what the pages and the mathematics fix.

Each check raises AssertionError on failure.  They are plain functions so
that tests/test_oracle_pins.py can run them on the oracle as built and
tests/test_oracle_mutants.py can run them on deliberately broken copies of it
(showing that a plausible mistake fails at least one of them).

The rule being pinned is that of page "speculative decoding: the small model
writes first, the big model checks" (blog.mna-game.duckdns.org, post 46), §1:
keep drafted t with probability min(1, q(t)/p(t)), else draw from
max(0, q - p) normalised; and of page "speculative decoding: running a big
model fast" (ai-trend.me), section "how it works": left-to-right judging,
first rejection replaced, a bonus token from the target's row gamma when all
drafts are kept, temperature / top-k as adjusted distributions.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
from scipy import stats

from oracle import oracle as O
from workloads import synth as I

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
LN2_T = float(np.float32(1.0 / math.log(2.0)))   # temperature turning log2 logits into probabilities


# ---------------------------------------------------------------------------
# helpers
# ---------------------------------------------------------------------------
def log2_logits(probs) -> np.ndarray:
    """float32 logits whose softmax at T = 1/ln 2 is `probs` (0 -> -inf)."""
    p = np.asarray(probs, dtype=np.float64)
    with np.errstate(divide="ignore"):
        z = np.where(p > 0, np.log2(np.where(p > 0, p, 1.0)), -np.inf)
    return z.astype(np.float32)


def chi2_pvalue(counts: np.ndarray, probs: np.ndarray) -> float:
    """Pearson chi-square of counts against probs, pooling cells with expected < 5."""
    counts = np.asarray(counts, dtype=np.float64)
    n = counts.sum()
    exp = np.asarray(probs, dtype=np.float64) * n
    assert np.all(counts[exp == 0] == 0), "mass on a zero-probability cell"
    order = np.argsort(exp)
    c_cells, e_cells = [], []
    acc_c = acc_e = 0.0
    for i in order:
        if exp[i] == 0:
            continue
        acc_c += counts[i]
        acc_e += exp[i]
        if acc_e >= 5.0:
            c_cells.append(acc_c)
            e_cells.append(acc_e)
            acc_c = acc_e = 0.0
    if acc_e > 0 and e_cells:
        c_cells[-1] += acc_c
        e_cells[-1] += acc_e
    c_cells = np.array(c_cells)
    e_cells = np.array(e_cells)
    if len(c_cells) < 2:
        return 1.0
    chi2 = float(((c_cells - e_cells) ** 2 / e_cells).sum())
    return float(stats.chi2.sf(chi2, len(c_cells) - 1))


def tv(a, b) -> float:
    return 0.5 * float(np.abs(np.asarray(a, np.float64) - np.asarray(b, np.float64)).sum())


def replicated(q_rows: np.ndarray, p_rows: np.ndarray, B: int, rng: np.random.Generator,
               temperature: float, top_k: int = 0, top_p: float = 1.0):
    """B sequences that all carry the same rows: target q_rows [gamma+1, V], draft
    p_rows [gamma, V] (float32 logits); drafted tokens drawn from the oracle's p_j."""
    g1, V = q_rows.shape
    gamma = g1 - 1
    target = np.ascontiguousarray(np.broadcast_to(q_rows, (B, g1, V)), dtype=np.float32)
    draft = np.ascontiguousarray(np.broadcast_to(p_rows, (B, gamma, V)), dtype=np.float32)
    tokens = np.empty((B, gamma), dtype=np.int32)
    for j in range(gamma):
        pj = O.row_probs(p_rows[j], temperature, top_k, top_p)
        tokens[:, j] = rng.choice(V, size=B, p=pj / pj.sum())
    return target, draft, tokens


# ---------------------------------------------------------------------------
# Philox: cross-check against rocRAND's engine, run from its source header
# ---------------------------------------------------------------------------
def check_philox_vs_rocrand(rr, n: int = 4096, seed: int = 7):
    rng = np.random.default_rng(seed)
    ctr = rng.integers(0, 2**32, size=(n, 4), dtype=np.uint64).astype(np.uint32)
    # the helper reaches counter words 0-1 through an offset counted in 32-bit
    # outputs (a 64-bit integer), so word 1 stays below 2^30 here
    ctr[:, 1] >>= 2
    key = rng.integers(0, 2**32, size=(n, 2), dtype=np.uint64).astype(np.uint32)
    ctr[0] = 0
    key[0] = 0
    ctr[1] = [0xFFFFFFFF, 0x3FFFFFFF, 0xFFFFFFFF, 0xFFFFFFFF]
    key[1] = 0xFFFFFFFF
    ref = np.zeros((n, 4), dtype=np.uint32)
    rr.rr_philox_many(ctr.ctypes.data, key.ctypes.data, ref.ctypes.data, n)
    mine = np.stack([O.philox(ctr[i], key[i]) for i in range(n)])
    bad = np.nonzero(np.any(mine != ref, axis=1))[0]
    assert bad.size == 0, f"{bad.size} Philox blocks differ from rocRAND, first at {bad[:3]}"


def check_word_layout():
    """A word is output (v mod 4) of the block at counter (v/4, pos, seq, purpose)."""
    seed, seq, pos = 0x0123456789ABCDEF, 77, 5
    for v in (0, 1, 2, 3, 4, 9, 1023):
        for purpose in (O.ACCEPT, O.SAMPLE):
            blk = O.philox([v >> 2, pos, seq, purpose], [seed & 0xFFFFFFFF, seed >> 32])
            assert O.word(seed, seq, pos, v, purpose) == int(blk[v & 3])


def check_variates():
    """24-bit acceptance uniform in [0, 1); exponential of an odd multiple of 2^-24."""
    assert O.uniform_accept(0) == 0.0
    assert O.uniform_accept(0xFFFFFFFF) == 1.0 - 2.0 ** -24
    assert O.uniform_accept(0x000000FF) == 0.0          # low 8 bits are dropped
    assert O.uniform_accept(0x00000100) == 2.0 ** -24
    assert math.isclose(O.exponential(0), 24.0 * math.log(2.0), rel_tol=1e-15)
    assert math.isclose(O.exponential(0xFFFFFFFF), -math.log1p(-2.0 ** -24), rel_tol=1e-9)
    # mean of E over many words is 1 (Exp(1)), within 5 sigma
    ws = [O.word(3, s, 0, 0, O.SAMPLE) for s in range(20000)]
    e = np.array([O.exponential(w) for w in ws])
    assert abs(e.mean() - 1.0) < 5.0 / math.sqrt(len(e))


# ---------------------------------------------------------------------------
# The rule on worked examples (golden fixture, hand-derived from the formula)
# ---------------------------------------------------------------------------
def check_golden_examples():
    with open(os.path.join(GOLDEN, "rule_worked_examples.json")) as f:
        ex = json.load(f)["examples"]
    for e in ex:
        p = O.row_probs(log2_logits(e["p"]), LN2_T)
        q = O.row_probs(log2_logits(e["q"]), LN2_T)
        np.testing.assert_allclose(p, e["p"], atol=1e-7, err_msg=e["name"])
        np.testing.assert_allclose(q, e["q"], atol=1e-7, err_msg=e["name"])
        acc = np.array([O.accept_count(p[t], q[t]) / 2.0 ** 24 for t in range(4)])
        want = np.array(e["accept_prob_per_token"])
        drafted = np.asarray(e["p"]) > 0
        np.testing.assert_allclose(acc[drafted], want[drafted], atol=2e-7, err_msg=e["name"])
        assert abs(float((p * acc).sum()) - e["accept_prob"]) < 2e-7, e["name"]
        r, empty = O.residual(q, p)
        assert not empty
        np.testing.assert_allclose(r / r.sum(), e["residual"], atol=1e-7, err_msg=e["name"])


def check_golden_adjusted():
    """Hand-worked top-k, nucleus and arg-max distributions (tests/golden)."""
    with open(os.path.join(GOLDEN, "adjusted_distributions.json")) as f:
        ex = json.load(f)["examples"]
    for e in ex:
        if "probs" in e:
            z, T = log2_logits(e["probs"]), LN2_T
        else:
            z, T = np.asarray(e["logits"], dtype=np.float32), e["temperature"]
        got = O.row_probs(z, T, e["top_k"], e["top_p"])
        np.testing.assert_allclose(got, e["expected"], atol=1e-7, err_msg=e["name"])


def check_golden_token_probs():
    """Hand-worked p_j(t_j), q_j(t_j) (tests/golden/token_probs.json): the
    values the GPU's probabilities are compared against."""
    with open(os.path.join(GOLDEN, "token_probs.json")) as f:
        cases = json.load(f)["cases"]

    def rows(x):
        return np.asarray([[-np.inf if v == "ninf" else v for v in r] for r in x], dtype=np.float32)[None]

    for c in cases:
        T = LN2_T if c["temperature"] == "1/ln2" else float(c["temperature"])
        tok = np.asarray([c["tokens"]], dtype=np.int32)
        pt, qt = O.token_probs(rows(c["target"]), rows(c["draft"]), tok, T, c["top_k"])
        np.testing.assert_allclose(pt[0], c["p"], rtol=1e-6, atol=0, err_msg=c["name"] + " (p)")
        np.testing.assert_allclose(qt[0], c["q"], rtol=1e-6, atol=0, err_msg=c["name"] + " (q)")


# ---------------------------------------------------------------------------
# P1: exact enumeration at V = 4, gamma = 1 — the output distribution is q
# ---------------------------------------------------------------------------
def enumeration_cases():
    rng = np.random.default_rng(11)
    cases = {
        "random": (rng.normal(0, 2, 4), rng.normal(0, 2, 4)),
        "p equals q": (np.array([0.3, -1.0, 2.0, 0.5]),) * 2,
        "disjoint supports": (np.array([1.0, 0.2, -np.inf, -np.inf]), np.array([-np.inf, -np.inf, 0.1, 0.7])),
        "one-hot q": (np.array([0.5, 1.0, -0.3, 0.0]), np.array([-np.inf, 2.0, -np.inf, -np.inf])),
        "one-hot p": (np.array([-np.inf, -np.inf, 3.0, -np.inf]), np.array([0.1, -0.4, 0.9, 1.3])),
    }
    return {k: (np.asarray(a, np.float32), np.asarray(b, np.float32)) for k, (a, b) in cases.items()}


def check_enumeration_v4():
    """For each t: c_t = #{k in [0, 2^24): accept(k 2^-24, p(t), q(t))} by brute force.
    P(out = x) = p(x) c_x / 2^24 + (sum_t p(t) (1 - c_t / 2^24)) r(x) / sum r.
    Claim of the page: this equals q exactly; bound 2^-22 covers the 24-bit u."""
    for name, (zp, zq) in enumeration_cases().items():
        p = O.row_probs(zp, 1.0)
        q = O.row_probs(zq, 1.0)
        c = np.array([O.accept_count(p[t], q[t]) for t in range(4)], dtype=np.float64) / 2.0 ** 24
        reject_mass = float((p * (1.0 - c)).sum())
        r, empty = O.residual(q, p)
        resid = r / r.sum() if r.sum() > 0 else np.zeros(4)
        out = p * c + reject_mass * resid
        err = float(np.abs(out - q).max())
        assert err <= 2.0 ** -22, f"{name}: |P(out) - q|_inf = {err}"
        # P2 exactly: P(accept) = sum_v min(p, q) = 1 - TV(p, q)
        pacc = float((p * c).sum())
        assert abs(pacc - np.minimum(p, q).sum()) <= 2.0 ** -22, name
        assert abs(pacc - (1.0 - tv(p, q))) <= 2.0 ** -22, name


# ---------------------------------------------------------------------------
# P2 / P3: the whole step, Monte-Carlo, against closed forms
# ---------------------------------------------------------------------------
def check_accept_rate_and_n_distribution(B: int = 400_000, seed: int = 21):
    """Rows independent of earlier tokens => acceptances are independent
    Bernoulli(alpha_j), alpha_j = sum_v min(p_j, q_j).  Then
    P(n = i) = prod_{j<i} alpha_j (1 - alpha_i), P(n = gamma) = prod alpha_j,
    E[n] = sum_{i=1..gamma} prod_{j<i} alpha_j."""
    rng = np.random.default_rng(seed)
    gamma, V = 4, 8
    zq = rng.normal(0, 1.5, (gamma + 1, V)).astype(np.float32)
    zp = (zq[:gamma] + rng.normal(0, 1.0, (gamma, V))).astype(np.float32)
    target, draft, tokens = replicated(zq, zp, B, rng, 1.0)
    res = O.verify(target, draft, tokens, 1.0, 0, seed=1234)
    alpha = np.array([np.minimum(O.row_probs(zp[j], 1.0), O.row_probs(zq[j], 1.0)).sum()
                      for j in range(gamma)])
    pn = np.array([np.prod(alpha[:i]) * (1 - alpha[i]) for i in range(gamma)] + [np.prod(alpha)])
    counts = np.bincount(res.n_accepted, minlength=gamma + 1)
    pv = chi2_pvalue(counts, pn)
    assert pv > 1e-6, f"distribution of n: chi2 p = {pv}, counts {counts}, expected {pn * B}"
    en = sum(np.prod(alpha[:i]) for i in range(1, gamma + 1))
    sd = res.n_accepted.std() / math.sqrt(B)
    assert abs(res.n_accepted.mean() - en) < 4 * sd, (res.n_accepted.mean(), en)
    # first-position acceptance rate equals 1 - TV(p_0, q_0)
    acc0 = float((res.n_accepted > 0).mean())
    a0 = 1.0 - tv(O.row_probs(zp[0], 1.0), O.row_probs(zq[0], 1.0))
    assert abs(acc0 - a0) < 4 * math.sqrt(a0 * (1 - a0) / B), (acc0, a0)


def check_output_is_q(B: int = 200_000, seed: int = 5, temperature: float = 0.9, top_k: int = 0,
                      top_p: float = 1.0):
    """gamma = 1: the committed first token is distributed as q_0 (the page's
    claim that the rule is exact, not approximate)."""
    rng = np.random.default_rng(seed)
    V = 8
    zq = rng.normal(0, 1.5, (2, V)).astype(np.float32)
    zp = rng.normal(0, 1.5, (1, V)).astype(np.float32)
    target, draft, tokens = replicated(zq, zp, B, rng, temperature, top_k, top_p)
    res = O.verify(target, draft, tokens, temperature, top_k, seed=99, top_p=top_p)
    q0 = O.row_probs(zq[0], temperature, top_k, top_p)
    counts = np.bincount(res.out_tokens[:, 0], minlength=V)
    pv = chi2_pvalue(counts, q0)
    assert pv > 1e-6, f"first token vs q0: chi2 p = {pv}; counts {counts}; q0*B {q0 * B}"


# ---------------------------------------------------------------------------
# P4: the 60,000-draw total-variation test at the most divergent position
# ---------------------------------------------------------------------------
def direct_tv_threshold(q: np.ndarray, n: int = 60_000, runs: int = 200, seed: int = 17) -> float:
    """99th percentile of TV(empirical, q) over `runs` direct samples of n draws
    from q — the noise floor of sampling straight from the target."""
    rng = np.random.default_rng(seed)
    counts = rng.multinomial(n, q / q.sum(), size=runs)
    tvs = 0.5 * np.abs(counts / n - q[None, :]).sum(axis=1)
    return float(np.percentile(tvs, 99))


def check_60k_tv(w, seed: int = 3000, n: int = 60_000):
    """Workload c0 (B=1, gamma=4, V=256): pick j* = argmax_j TV(p_j, q_j), verify
    60,000 independent one-draft sequences at that position, and require
    TV(empirical first token, q_j*) <= the direct-sampling p99 noise."""
    from workloads import synth as I
    tvs = [tv(O.row_probs(w.draft[0, j], w.temperature, w.top_k),
              O.row_probs(w.target[0, j], w.temperature, w.top_k)) for j in range(w.gamma)]
    jstar = int(np.argmax(tvs))
    rep = I.replicate_position(w, 0, jstar, n, seed=seed + 1)
    res = O.verify(rep.target, rep.draft, rep.tokens, w.temperature, w.top_k, seed=seed)
    q = O.row_probs(w.target[0, jstar], w.temperature, w.top_k)
    counts = np.bincount(res.out_tokens[:, 0], minlength=w.V)
    got = tv(counts / n, q)
    thr = direct_tv_threshold(q, n)
    assert got <= thr, f"TV(speculative, q) = {got:.5f} > direct-sampling p99 {thr:.5f}"
    pv = chi2_pvalue(counts, q)
    assert pv > 1e-4, f"chi2 p = {pv}"
    return {"jstar": jstar, "tv_draft": tvs[jstar], "tv_spec": got, "tv_direct_p99": thr, "chi2_p": pv}


# ---------------------------------------------------------------------------
# P5: special cases with no dependence on the random streams
# ---------------------------------------------------------------------------
def check_special_cases(seed: int = 8):
    rng = np.random.default_rng(seed)
    V, gamma, B = 16, 3, 2000
    zq = rng.normal(0, 2, (gamma + 1, V)).astype(np.float32)
    # (a) p == q: every draft kept, so n = gamma; the bonus token follows q_gamma
    target, draft, tokens = replicated(zq, zq[:gamma].copy(), B, rng, 1.0)
    res = O.verify(target, draft, tokens, 1.0, 0, seed=5)
    assert np.all(res.n_accepted == gamma)
    assert np.array_equal(res.out_tokens[:, :gamma], tokens)
    qg = O.row_probs(zq[gamma], 1.0)
    big = replicated(zq, zq[:gamma].copy(), 100_000, rng, 1.0)
    res_big = O.verify(*big, 1.0, 0, seed=6)
    pv = chi2_pvalue(np.bincount(res_big.out_tokens[:, gamma], minlength=V), qg)
    assert pv > 1e-6, f"bonus token vs q_gamma: p = {pv}"
    # (b) drafted token outside the target's top-k: q(t) = 0 -> rejected at once
    zq2 = np.tile(np.arange(V, dtype=np.float32), (gamma + 1, 1))          # argmax V-1
    zp2 = np.tile(np.arange(V, dtype=np.float32)[::-1].copy(), (gamma, 1))  # argmax 0
    tgt = np.broadcast_to(zq2, (4, gamma + 1, V)).copy()
    drf = np.broadcast_to(zp2, (4, gamma, V)).copy()
    tok = np.zeros((4, gamma), dtype=np.int32)                               # t = 0 = argmax p
    res = O.verify(tgt, drf, tok, 1.0, 2, seed=1)                            # q keeps {V-2, V-1}
    assert np.all(res.n_accepted == 0)
    # (c) top-k = 1 is greedy verification: accept iff argmax p == argmax q,
    #     and the replacement is argmax q
    res = O.verify(tgt, drf, tok, 1.0, 1, seed=2)
    assert np.all(res.n_accepted == 0) and np.all(res.out_tokens[:, 0] == V - 1)
    same = np.broadcast_to(zq2[:gamma], (4, gamma, V)).copy()
    tok_same = np.full((4, gamma), V - 1, dtype=np.int32)
    res = O.verify(tgt, same, tok_same, 1.0, 1, seed=3)
    assert np.all(res.n_accepted == gamma) and np.all(res.out_tokens[:, gamma] == V - 1)
    # (d) constant logits -> exactly uniform; huge temperature -> uniform
    assert np.all(O.row_probs(np.full(256, 1.25, np.float32), 0.7) == 1.0 / 256)
    np.testing.assert_allclose(O.row_probs(rng.normal(0, 3, 64).astype(np.float32), 1e30),
                               1.0 / 64, rtol=1e-12)


# ---------------------------------------------------------------------------
# P6: Gumbel-max sampler against the multinomial it claims to draw from
# ---------------------------------------------------------------------------
def check_gumbel_sampler(n: int = 1_000_000):
    for V, seed in ((4, 1), (256, 2)):
        rng = np.random.default_rng(seed)
        w = rng.random(V) ** 3
        w[rng.random(V) < 0.25] = 0.0
        w[0] = max(w[0], 0.01)
        draws = O.gumbel_sample_many(w, seed=seed + 40, seq0=0, n=n, pos=3)
        counts = np.bincount(draws, minlength=V)
        pv = chi2_pvalue(counts, w / w.sum())
        assert pv > 1e-6, f"V={V}: Gumbel sampler chi2 p = {pv}"


# ---------------------------------------------------------------------------
# P8: softmax with temperature and top-k against library routines
# ---------------------------------------------------------------------------
def check_row_probs_vs_torch():
    import torch
    rng = np.random.default_rng(4)
    for V, T in ((10, 1.0), (1000, 0.7), (32000, 1.3)):
        z = rng.normal(0, 3, V).astype(np.float32)
        want = torch.softmax(torch.from_numpy(z).double() / float(np.float32(T)), dim=0).numpy()
        got = O.row_probs(z, T)
        np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-300)


def check_topk_vs_stable_sort():
    """Kept set = first K of a stable descending sort (ties -> smaller index)."""
    rng = np.random.default_rng(12)
    for V, K in ((50, 7), (1000, 50), (300, 299), (64, 1)):
        z = rng.integers(-3, 4, V).astype(np.float32)        # many ties on purpose
        keep = np.argsort(-z.astype(np.float64), kind="stable")[:K]
        got = O.row_probs(z, 1.0, K)
        assert set(np.nonzero(got > 0)[0].tolist()) == set(keep.tolist()), (V, K)
        e = np.exp(z[keep].astype(np.float64) - z[keep].max())
        np.testing.assert_allclose(got[keep], e / e.sum(), rtol=1e-12)
    # bf16 storage decodes exactly: 0x3F80 = 1.0, 0xC000 = -2.0
    zb = np.array([0x3F80, 0xC000, 0x0000, 0x3F80], dtype=np.uint16)
    zf = np.array([1.0, -2.0, 0.0, 1.0], dtype=np.float32)
    np.testing.assert_array_equal(O.row_probs(zb, 1.0, 2), O.row_probs(zf, 1.0, 2))


# ---------------------------------------------------------------------------
# Output structure ([SDB] §3: a step commits accepted + 1 tokens, 1..gamma+1)
# ---------------------------------------------------------------------------
def check_output_structure(w, res):
    B, gamma = w.tokens.shape
    n = res.n_accepted
    for b in range(B):
        if n[b] < 0:
            assert np.all(res.out_tokens[b] == -1)
            continue
        assert 0 <= n[b] <= gamma
        assert np.array_equal(res.out_tokens[b, :n[b]], w.tokens[b, :n[b]])
        assert 0 <= res.out_tokens[b, n[b]] < w.V
        assert np.all(res.out_tokens[b, n[b] + 1:] == -1)


# ---------------------------------------------------------------------------
# Arg-max mode (temperature 0, reading R9 of the oracle)
# ---------------------------------------------------------------------------
def check_greedy(seed: int = 31):
    """T = 0: every distribution is the point mass on its row's first largest
    logit.  Then q_j(t_j) > 0 only for t_j = argmax q_j and p_j(t_j) is 0 or 1,
    so the rule keeps draft j iff t_j = argmax q_j; the residual at the first
    rejection is the point mass on argmax q_n (or empty, falling back to q_n),
    and the bonus is argmax q_gamma.  Stated here with numpy's first-occurrence
    arg-max, independently of the oracle's code; the draft rows and the seed
    change nothing."""
    rng = np.random.default_rng(seed)
    for V, gamma, B, dtype in ((9, 4, 600, np.float32), (300, 6, 300, np.float32), (64, 3, 300, np.uint16)):
        zq = rng.integers(-4, 5, (B, gamma + 1, V)).astype(np.float32)   # many tied maxima
        zp = rng.integers(-4, 5, (B, gamma, V)).astype(np.float32)
        a = np.argmax(zq, axis=2)                                        # first occurrence
        tok = np.where(rng.random((B, gamma)) < 0.8, a[:, :gamma], rng.integers(0, V, (B, gamma)))
        tok = tok.astype(np.int32)
        if dtype == np.uint16:
            tq, tp = I.f32_to_bf16_bits(zq), I.f32_to_bf16_bits(zp)     # small integers: exact in bf16
        else:
            tq, tp = zq, zp
        res = O.verify(tq, tp, tok, 0.0, 0, seed=int(rng.integers(1 << 62)))
        for b in range(B):
            miss = np.nonzero(tok[b] != a[b, :gamma])[0]
            n = int(miss[0]) if miss.size else gamma
            assert res.n_accepted[b] == n, (V, b)
            want = np.full(gamma + 1, -1, np.int32)
            want[:n] = tok[b, :n]
            want[n] = a[b, n]
            assert np.array_equal(res.out_tokens[b], want), (V, b, res.out_tokens[b], want)
        # the same outputs with other draft rows, another seed, or top-k = 1 at T = 1
        other = O.verify(tq, tq[:, :gamma].copy(), tok, 0.0, 3, seed=99)
        k1 = O.verify(tq, tp, tok, 1.0, 1, seed=7)
        for r in (other, k1):
            assert np.array_equal(r.out_tokens, res.out_tokens) and np.array_equal(r.n_accepted, res.n_accepted)
    # T -> 0 limit of the general rule: with distinct logits at least 1 apart,
    # softmax(z / 1e-3) is exactly one-hot in fp64 and gives the same result
    V, gamma, B = 40, 4, 200
    zq = np.stack([np.stack([rng.permutation(V) for _ in range(gamma + 1)]) for _ in range(B)]).astype(np.float32)
    zp = np.stack([np.stack([rng.permutation(V) for _ in range(gamma)]) for _ in range(B)]).astype(np.float32)
    a = np.argmax(zq, axis=2)
    tok = np.where(rng.random((B, gamma)) < 0.7, a[:, :gamma], np.argmax(zp, axis=2)).astype(np.int32)
    g0 = O.verify(zq, zp, tok, 0.0, 0, seed=5)
    gs = O.verify(zq, zp, tok, 1e-3, 0, seed=5)
    assert np.array_equal(g0.out_tokens, gs.out_tokens) and np.array_equal(g0.n_accepted, gs.n_accepted)


# ---------------------------------------------------------------------------
# Draft sampler (the draft's own step before verification, DRAFT stream)
# ---------------------------------------------------------------------------
def check_draft_sampler(n: int = 200_000, seed: int = 41):
    """Tokens follow the draft row's adjusted distribution (chi-square, with T
    and top-k; never outside the kept set); T = 0 gives the first largest
    logit; the DRAFT stream is not the SAMPLE stream; seq_offset shifts the
    streams like the sequence index."""
    rng = np.random.default_rng(seed)
    V = 64
    z = rng.normal(0, 2, V).astype(np.float32)
    for T, K, P in ((1.0, 0, 1.0), (0.7, 5, 1.0), (1.3, 40, 1.0), (1.0, 30, 0.8)):
        rows = np.broadcast_to(z, (n, 1, V)).copy()
        tok, gap = O.draft_sample(rows, T, K, seed=seed + 1, top_p=P)
        p = O.row_probs(z, T, K, P)
        counts = np.bincount(tok[:, 0], minlength=V)
        assert np.all(counts[p == 0] == 0), (T, K)
        pv = chi2_pvalue(counts, p)
        assert pv > 1e-6, f"draft sampler T={T} K={K}: chi2 p = {pv}"
        assert np.all(gap > 0)
    # T = 0: the first largest logit, whatever the seed
    zi = rng.integers(-3, 4, (50, 3, 30)).astype(np.float32)
    tok0, _ = O.draft_sample(zi, 0.0, 0, seed=5)
    assert np.array_equal(tok0, np.argmax(zi, axis=2))
    # the DRAFT stream differs from the SAMPLE stream at the same (seq, pos):
    # on a uniform row each stream's draw is its own arg-max of -ln E
    flat = np.zeros((2000, 1, V), np.float32)
    dtok, _ = O.draft_sample(flat, 1.0, 0, seed=9)
    stok = O.gumbel_sample_many(np.full(V, 1.0), seed=9, seq0=0, n=2000, pos=0)
    assert np.mean(dtok[:, 0] == stok) < 0.05
    # seq_offset: sequence b at offset o is sequence b + o at offset 0
    rows = rng.normal(0, 1, (12, 2, V)).astype(np.float32)
    full, _ = O.draft_sample(rows, 1.0, 0, seed=3)
    part, _ = O.draft_sample(rows[5:], 1.0, 0, seed=3, seq_offset=5)
    assert np.array_equal(full[5:], part)


# ---------------------------------------------------------------------------
# Nucleus (top-p), reading R10 of the oracle
# ---------------------------------------------------------------------------
def _nucleus_numpy(z: np.ndarray, T: float, K: int, P: float):
    """Written out with numpy: softmax of top-k(z)/T, then the shortest prefix
    of the stable descending order with mass >= P, renormalised.  Returns the
    probabilities and the distance of the cut from flipping."""
    z64 = z.astype(np.float64)
    V = z.shape[0]
    order = np.argsort(-z64, kind="stable")
    kept = order[:K] if 0 < K < V else order
    x = z64[kept] / float(np.float32(T))
    e = np.exp(x - x.max())
    pk = e / e.sum()
    probs = np.zeros(V)
    margin = np.inf
    P = float(np.float32(P))  # top_p crosses the C ABI as a float
    if 0 < P < 1:
        cum = np.cumsum(pk)
        m = int(np.searchsorted(cum, P, side="left"))
        m = min(m, len(pk) - 1)
        margin = min(cum[m] - P, P - cum[m - 1]) if m > 0 else cum[0] - P
        pk = pk[: m + 1] / cum[m]
        kept = kept[: m + 1]
    probs[kept] = pk
    return probs, margin


def check_nucleus(seed: int = 51):
    """Top-p kept sets and probabilities equal a numpy statement of R10 (rows
    with many tied logits included); P >= 1 or <= 0 changes nothing; a tiny P
    keeps only the first largest logit; the verified first token follows q
    under top-p (chi-square)."""
    rng = np.random.default_rng(seed)
    checked = 0
    for trial in range(300):
        V = int(rng.choice([5, 50, 700]))
        z = (rng.integers(-4, 5, V) if trial % 2 else rng.normal(0, 2, V)).astype(np.float32)
        T = float(rng.choice([1.0, 0.7, 1.6]))
        K = int(rng.choice([0, 3, 20, V]))
        P = float(rng.choice([0.3, 0.75, 0.9, 0.999]))
        want, margin = _nucleus_numpy(z, T, K, P)
        if margin < 1e-12:
            continue  # a cut that rounding can move; not a test of the rule
        got = O.row_probs(z, T, K, P)
        assert np.array_equal(got > 0, want > 0), (V, T, K, P)
        np.testing.assert_allclose(got, want, rtol=1e-12, atol=0)
        assert abs(O.nucleus_margin(z, T, K, P) - margin) < 1e-9
        checked += 1
    assert checked > 250
    z = rng.normal(0, 2, 64).astype(np.float32)
    for P in (1.0, 1.5, 0.0, -1.0):
        np.testing.assert_array_equal(O.row_probs(z, 0.8, 10, P), O.row_probs(z, 0.8, 10))
    tiny = O.row_probs(z, 0.8, 0, 1e-9)
    assert np.count_nonzero(tiny) == 1 and tiny[np.argmax(z)] == 1.0
    check_output_is_q(temperature=0.9, top_k=0, top_p=0.8)
    check_output_is_q(temperature=1.1, top_k=6, top_p=0.7)
