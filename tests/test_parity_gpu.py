"""Parity of the HIP path (through the C ABI) with the oracle, on the GPU.

Small-size cases compare every sequence and every per-position probability;
full-size workloads run in the launch configuration the benchmark times and
compare against the oracle on every sequence (the oracle is fast enough with
all host threads).  The bar is documented in tests/parity.py."""
import sys
import warnings

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


SMALL = [("c0", None, [3000, 3001, 3002, 3003]),
         ("c1", None, [3001, 3101, 3201]),
         ("c2", 6, [3002, 3102]),
         ("c3", 3, [3003, 3103]),
         ("c4a", 48, [3004]),
         ("c4b", 48, [3004, 3104]),
         ("c4c", 48, [3004])]


@pytest.mark.parametrize("name,B,seeds", SMALL, ids=[s[0] for s in SMALL])
def test_parity_small(name, B, seeds):
    w = I.make(name, B=B)
    _say(f"case {name} B={w.B} gamma={w.gamma} V={w.V} dtype={w.spec.dtype} T={w.temperature} K={w.top_k}")
    tensors = PT.to_device(w)
    for seed in seeds:
        g = PT.run_gpu(w, seed, tensors=tensors)
        _check(PT.compare(w, seed, g), f"{name} seed {seed}")


FULL = ["c2", "c3", "c4a", "c4b", "c4c"]


@pytest.mark.parametrize("sigma", [0.5, 2.0])
def test_parity_one_position_per_launch(sigma):
    """Inputs large enough (537 MB of rows) that the library judges one
    position per launch, with gamma = 8 so sequences finish at every launch."""
    w = I.make("c4b", B=64, gamma=8, V=131072, draft_sigma=sigma, data_seed=1077, draft_seed=2077)
    _say(f"case window-1 B={w.B} gamma={w.gamma} V={w.V} sigma={sigma}")
    import rejection_sampling_verify_17_amd as S
    assert S.launch_names(w.B, w.gamma, w.V, S.SV_F32, 0) == ["k_rows", "k_judge"] + ["k_rows"] * 8
    tensors = PT.to_device(w)
    for seed in (3100, 3101):
        g = PT.run_gpu(w, seed, tensors=tensors)
        _check(PT.compare(w, seed, g), f"window-1 sigma {sigma} seed {seed}")
        _say(f"n histogram {np.bincount(g.n_accepted, minlength=w.gamma + 1).tolist()}")


@pytest.mark.parametrize("name", FULL)
def test_parity_full_size(name):
    """Full workload, benchmark launch geometry, every sequence against the oracle."""
    w = I.make(name)
    _say(f"case {name} full B={w.B} gamma={w.gamma} V={w.V}")
    tensors = PT.to_device(w)
    seed = 3000 + int(name[1])
    g = PT.run_gpu(w, seed, tensors=tensors)
    rep = PT.compare(w, seed, g)
    _check(rep, f"{name} full")
    n = g.n_accepted
    _say(f"{name}: mean accepted {n.mean():.3f}, all-kept {np.mean(n == w.gamma):.3f}")


def test_60k_total_variation_on_gpu():
    """The page's 60,000-draw TV test (blog post 46, §4) on GPU outputs: at the
    most divergent position of c0, TV(empirical, q) <= the direct-sampling p99,
    and the 60,000 outputs equal the oracle's."""
    import oracle_checks as C
    w = I.make("c0")
    tvs = [C.tv(O.row_probs(w.draft[0, j], 1.0), O.row_probs(w.target[0, j], 1.0)) for j in range(w.gamma)]
    jstar = int(np.argmax(tvs))
    rep_w = I.replicate_position(w, 0, jstar, 60_000, seed=3001)
    _say(f"case c0-60k j*={jstar} TV(p,q)={tvs[jstar]:.4f}")
    g = PT.run_gpu(rep_w, 3000, debug=False)
    q = O.row_probs(w.target[0, jstar], 1.0)
    counts = np.bincount(g.out_tokens[:, 0], minlength=w.V)
    got = C.tv(counts / 60_000, q)
    thr = C.direct_tv_threshold(q)
    _say(f"TV(gpu samples, q) = {got:.5f}; direct-sampling p99 = {thr:.5f}")
    assert got <= thr
    rep = PT.compare(rep_w, 3000, g, check_probs=False)
    _POOL["c0-60k"] = rep
    _check(rep, "c0-60k")


# Pooled mismatch rate: every workload at its full size under 20 verify
# seeds each, pooled with the 60,000-sequence run above.  Exemptions (knife
# edges, tests/parity.py) are counted and printed per workload and pooled.
_POOL = {}
POOLED = ["c0", "c1", "c2", "c2p", "c3", "c3p", "c4a", "c4b", "c4c"]
POOL_SEEDS = 20


@pytest.mark.parametrize("name", POOLED)
def test_pooled_seeds(name):
    w = I.make(name)
    _say(f"case pooled {name} B={w.B} gamma={w.gamma} V={w.V} K={w.top_k} top_p={w.top_p}, {POOL_SEEDS} seeds")
    tensors = PT.to_device(w)
    rep = PT.Report()
    for k in range(POOL_SEEDS):
        seed = 5000 + 100 * k + POOLED.index(name)
        g = PT.run_gpu(w, seed, tensors=tensors, debug=False)
        rep.merge(PT.compare(w, seed, g, check_probs=False))
    _POOL[name] = rep
    _check(rep, f"pooled {name}")


def test_pooled_total():
    missing = [n for n in POOLED + ["c0-60k"] if n not in _POOL]
    if missing:
        pytest.skip(f"pooled parts not run in this session: {missing}")
    tot = PT.Report()
    lines = []
    keys = ("sequences", "mismatches", "exempt_accept", "exempt_token", "exempt_nucleus", "exempt_equal")
    for n in POOLED + ["c0-60k"]:
        tot.merge(_POOL[n])
        sm = _POOL[n].summary()
        lines.append(f"  {n}: " + ", ".join(f"{k} {sm[k]}" for k in keys))
    sm = tot.summary()
    lines.append("  pooled: " + ", ".join(f"{k} {sm[k]}" for k in keys) + f", mismatch_rate {sm['mismatch_rate']:.2e}")
    _say("pooled over all workloads x 20 seeds and the 60k run:", sm)
    # shown in the warnings summary of a quiet run, so the counts reach its log
    warnings.warn(ParityReport("pooled parity, every workload x 20 verify seeds + the 60k run:\n" + "\n".join(lines)))
    assert tot.sequences >= 128_000
    assert tot.mismatches == 0 and tot.ok()


class ParityReport(UserWarning):
    """Counts of a parity run, reported through the warnings summary."""


def test_deterministic_and_geometry_independent():
    """Same call twice is bit-identical; a sub-batch with seq_offset reproduces
    the full batch's rows although its launch geometry differs."""
    w = I.make("c2", B=24)
    t = PT.to_device(w)
    a = PT.run_gpu(w, 77, tensors=t, debug=False)
    b = PT.run_gpu(w, 77, tensors=t, debug=False)
    assert np.array_equal(a.out_tokens, b.out_tokens) and np.array_equal(a.n_accepted, b.n_accepted)
    sub = I.from_arrays(w.target[5:9], w.draft[5:9], w.tokens[5:9], w.temperature, w.top_k)
    c = PT.run_gpu(sub, 77, seq_offset=5, debug=False)
    assert np.array_equal(c.out_tokens, a.out_tokens[5:9])


def test_large_batch_invalid_tokens_and_sub_batches():
    """Large inputs (one position per launch): drafted tokens outside [0, V)
    flag their sequence; a sub-batch with the matching seq_offset draws the
    same random numbers, so it matches the oracle on the same sequences; every
    sequence equals the oracle."""
    import rejection_sampling_verify_17_amd as S
    w = I.make("c4b", B=512)
    assert S.launch_names(w.B, w.gamma, w.V, S.SV_F32, 0)[:2] == ["k_rows", "k_judge"]
    tok = w.tokens.copy()
    tok[3, 0] = w.V
    tok[100, 3] = -2
    w2 = I.from_arrays(w.target, w.draft, tok, w.temperature, w.top_k)
    _say(f"case large batch B={w2.B} gamma={w2.gamma} V={w2.V}, two invalid sequences")
    g = PT.run_gpu(w2, 3004)
    assert g.n_accepted[3] == -1 and np.all(g.out_tokens[3] == -1)
    assert g.n_accepted[100] == -1 and np.all(g.out_tokens[100] == -1)
    _check(PT.compare(w2, 3004, g), "large batch")
    sub = I.from_arrays(w2.target[160:480], w2.draft[160:480], tok[160:480], w2.temperature, w2.top_k)
    gs = PT.run_gpu(sub, 3004, seq_offset=160)
    _check(PT.compare(sub, 3004, gs, seq_offset=160), "large sub-batch")
    same = np.mean(np.all(gs.out_tokens == g.out_tokens[160:480], axis=1))
    _say(f"sub-batch rows equal to the full batch's: {same:.4f}")


def test_invalid_tokens_flagged():
    w = I.make("c1")
    tok = w.tokens.copy()
    tok[2, 1] = w.V
    tok[5, 0] = -7
    w2 = I.from_arrays(w.target, w.draft, tok, w.temperature, w.top_k)
    g = PT.run_gpu(w2, 5)
    assert g.n_accepted[2] == -1 and np.all(g.out_tokens[2] == -1)
    assert g.n_accepted[5] == -1 and np.all(g.out_tokens[5] == -1)
    _check(PT.compare(w2, 5, g, check_probs=False), "invalid tokens")


def _edge_workloads():
    rng = np.random.default_rng(123)
    out = []
    # V = 2, gamma = 1
    t = rng.normal(0, 1, (16, 2, 2)).astype(np.float32)
    d = rng.normal(0, 1, (16, 1, 2)).astype(np.float32)
    out.append(("V2", I.from_arrays(t, d, rng.integers(0, 2, (16, 1)).astype(np.int32))))
    # gamma = 64 (the maximum), small V
    t = rng.normal(0, 1, (3, 65, 100)).astype(np.float32)
    d = (t[:, :64] + rng.normal(0, 0.05, (3, 64, 100))).astype(np.float32)
    w = I.from_arrays(t, d, np.zeros((3, 64), np.int32))
    w.tokens[:] = I.sample_rows(d.reshape(-1, 100), 1.0, 0, rng).reshape(3, 64)
    out.append(("gamma64", w))
    # -inf logits (masked vocabulary) in both inputs
    t = rng.normal(0, 2, (8, 4, 300)).astype(np.float32)
    d = rng.normal(0, 2, (8, 3, 300)).astype(np.float32)
    t[:, :, 50:120] = -np.inf
    d[:, :, 100:200] = -np.inf
    w = I.from_arrays(t, d, np.zeros((8, 3), np.int32))
    w.tokens[:] = I.sample_rows(d.reshape(-1, 300), 1.0, 0, rng).reshape(8, 3)
    out.append(("neg-inf", w))
    # constant rows: uniform distributions
    t = np.full((4, 3, 257), 0.5, np.float32)
    out.append(("constant", I.from_arrays(t, t[:, :2].copy(), rng.integers(0, 257, (4, 2)).astype(np.int32))))
    # bf16 with odd V: rows start on 2-byte boundaries every other row
    t = rng.normal(0, 3, (5, 3, 4099)).astype(np.float32)
    d = (t[:, :2] + rng.normal(0, 1, (5, 2, 4099))).astype(np.float32)
    tb, db = I.f32_to_bf16_bits(t), I.f32_to_bf16_bits(d)
    w = I.from_arrays(tb, db, np.zeros((5, 2), np.int32), temperature=0.9)
    w.tokens[:] = I.sample_rows(I.bf16_bits_to_f32(db).reshape(-1, 4099), 0.9, 0, rng).reshape(5, 2)
    out.append(("bf16-oddV", w))
    # the same rows with top-k: every shift of a row inside its 16-byte block
    out.append(("bf16-oddV-topk", I.from_arrays(tb, db, w.tokens.copy(), temperature=0.9, top_k=20)))
    w2 = out[-1][1]
    w2.tokens[:] = I.sample_rows(I.bf16_bits_to_f32(db).reshape(-1, 4099), 0.9, 20, rng).reshape(5, 2)
    # top-k with heavy ties (integer logits), K = 1, 7, V - 1, both dtypes
    for K in (1, 7, 499):
        t = rng.integers(-4, 5, (6, 3, 500)).astype(np.float32)
        d = rng.integers(-4, 5, (6, 2, 500)).astype(np.float32)
        w = I.from_arrays(t, d, np.zeros((6, 2), np.int32), top_k=K)
        w.tokens[:] = I.sample_rows(d.reshape(-1, 500), 1.0, K, rng).reshape(6, 2)
        out.append((f"ties-topk{K}", w))
        tb, db = I.f32_to_bf16_bits(t), I.f32_to_bf16_bits(d)
        out.append((f"ties-topk{K}-bf16", I.from_arrays(tb, db, w.tokens.copy(), top_k=K)))
    # top-k larger than the lists the library keeps (1024): scans rows instead
    t = rng.normal(0, 2, (2, 3, 6000)).astype(np.float32)
    d = (t[:, :2] + rng.normal(0, 1, (2, 2, 6000))).astype(np.float32)
    w = I.from_arrays(t, d, np.zeros((2, 2), np.int32), top_k=3000)
    w.tokens[:] = I.sample_rows(d.reshape(-1, 6000), 1.0, 3000, rng).reshape(2, 2)
    out.append(("topk-large", w))
    # top-k where more than the LDS candidate capacity tie at the threshold
    t = np.zeros((2, 3, 20000), np.float32)
    t[:, :, ::7] = 1.0
    d = t[:, :2].copy()
    d[:, :, ::11] = 2.0
    w = I.from_arrays(t, d, np.zeros((2, 2), np.int32), top_k=40)
    w.tokens[:] = I.sample_rows(d.reshape(-1, 20000), 1.0, 40, rng).reshape(2, 2)
    out.append(("topk-overflow", w))
    # constant rows with top-k: every entry ties, chunks overflow the LDS
    # candidate buffer, the smallest indices are kept
    t = np.full((3, 3, 20000), 0.25, np.float32)
    d = t[:, :2].copy()
    d[:, :, 5000:5100] = 1.0
    w = I.from_arrays(t, d, np.zeros((3, 2), np.int32), top_k=10)
    w.tokens[:] = I.sample_rows(d.reshape(-1, 20000), 1.0, 10, rng).reshape(3, 2)
    out.append(("topk-constant-rows", w))
    # p == q with top-k: every draft kept, bonus row selected in chunks
    t = rng.normal(0, 2, (16, 4, 40000)).astype(np.float32)
    w = I.from_arrays(t, t[:, :3].copy(), np.zeros((16, 3), np.int32), top_k=20)
    w.tokens[:] = I.sample_rows(t[:, :3].reshape(-1, 40000), 1.0, 20, rng).reshape(16, 3)
    out.append(("topk-p-equals-q", w))
    # p == q: everything kept, bonus from row gamma
    t = rng.normal(0, 2, (32, 4, 1000)).astype(np.float32)
    w = I.from_arrays(t, t[:, :3].copy(), np.zeros((32, 3), np.int32))
    w.tokens[:] = I.sample_rows(t[:, :3].reshape(-1, 1000), 1.0, 0, rng).reshape(32, 3)
    out.append(("p-equals-q", w))
    return out


EDGES = _edge_workloads()


@pytest.mark.parametrize("name,w", EDGES, ids=[e[0] for e in EDGES])
def test_edge_cases(name, w):
    _say(f"case edge {name} B={w.B} gamma={w.gamma} V={w.V} K={w.top_k} dtype={w.target.dtype}")
    for seed in (11, 12):
        g = PT.run_gpu(w, seed)
        _check(PT.compare(w, seed, g), f"edge {name} seed {seed}")
    if name in ("p-equals-q", "topk-p-equals-q"):
        assert np.all(g.n_accepted == w.gamma)


def test_workspace_reuse_across_shapes():
    """One workspace, calls of different shapes and paths back to back (dense
    and top-k layouts overlap): each call clears what it counts in."""
    import torch
    import rejection_sampling_verify_17_amd as S
    ws = torch.full((S.workspace_bytes(256, 8, 152064, 50, S.SV_BF16) + (1 << 20),), 0x5A, dtype=torch.uint8,
                    device="cuda")
    for name, B, seed in (("c1", 8, 1), ("c3", 8, 2), ("c2", 4, 3), ("c3", 2, 6), ("c1", 8, 4), ("c4b", 64, 5)):
        w = I.make(name, B=B)
        tgt, drf, tok = PT.to_device(w)
        out, n = S.verify(tgt, drf, tok, w.temperature, w.top_k, seed=seed, workspace=ws)
        torch.cuda.synchronize()
        g = PT.GpuResult(out.cpu().numpy(), n.cpu().numpy())
        _check(PT.compare(w, seed, g, check_probs=False), f"reuse {name}")


def test_non_default_stream():
    import torch
    import rejection_sampling_verify_17_amd as S
    w = I.make("c1")
    tgt, drf, tok = PT.to_device(w)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        out, n = S.verify(tgt, drf, tok, w.temperature, seed=9)
    s.synchronize()
    g = PT.GpuResult(out.cpu().numpy(), n.cpu().numpy())
    _check(PT.compare(w, 9, g, check_probs=False), "stream")


# ---------------------------------------------------------------------------
# Arg-max mode (temperature 0): exact, no knife-edges
# ---------------------------------------------------------------------------
GREEDY = [("g2", 8), ("g4b", 96), ("g2", None), ("g4b", None)]


@pytest.mark.parametrize("name,B", GREEDY, ids=[f"{n}-B{b or 'full'}" for n, b in GREEDY])
def test_greedy_parity(name, B):
    """Every sequence equals the oracle bit for bit (full size: the benchmark's
    launch geometry); the seed changes nothing; the debug outputs are NaN."""
    w = I.make(name, B=B)
    _say(f"case greedy {name} B={w.B} gamma={w.gamma} V={w.V} dtype={w.spec.dtype}")
    tensors = PT.to_device(w)
    g = PT.run_gpu(w, 5, tensors=tensors)
    _check(PT.compare(w, 5, g), f"greedy {name}")
    g2 = PT.run_gpu(w, 6, tensors=tensors, debug=False)
    assert np.array_equal(g.out_tokens, g2.out_tokens) and np.array_equal(g.n_accepted, g2.n_accepted)
    n = g.n_accepted
    _say(f"{name}: mean accepted {n.mean():.3f}, all-kept {np.mean(n == w.gamma):.3f}")


def _greedy_edges():
    rng = np.random.default_rng(321)
    out = []

    def argmax_tokens(t, frac):
        a = np.argmax(I.logits_f32(t)[:, :-1], axis=2)
        r = rng.integers(0, t.shape[2], a.shape)
        return np.where(rng.random(a.shape) < frac, a, r).astype(np.int32)

    # heavy ties (integer logits), both dtypes, drafts mostly the target's choice
    t = rng.integers(-3, 4, (24, 5, 700)).astype(np.float32)
    d = rng.integers(-3, 4, (24, 4, 700)).astype(np.float32)
    tok = argmax_tokens(t, 0.85)
    out.append(("ties", I.from_arrays(t, d, tok, temperature=0.0)))
    out.append(("ties-bf16", I.from_arrays(I.f32_to_bf16_bits(t), I.f32_to_bf16_bits(d), tok, temperature=0.0)))
    # signed zeros: -0 and +0 are equal, the first of them wins
    t = np.zeros((6, 3, 300), np.float32)
    t[:, :, ::3] = -0.0
    t[3:, :, 0] = -1.0
    tok = np.array([[0, 0], [0, 1], [1, 0], [1, 1], [1, 2], [2, 1]], np.int32)
    out.append(("signed-zero", I.from_arrays(t, t[:, :2].copy(), tok, temperature=0.0)))
    # -inf entries (masked vocabulary) and a single finite entry
    t = rng.normal(0, 2, (8, 4, 333)).astype(np.float32)
    t[:, :, 10:300] = -np.inf
    t[:4, 1, :] = -np.inf
    t[:4, 1, 200] = 5.0
    out.append(("neg-inf", I.from_arrays(t, t[:, :3].copy(), argmax_tokens(t, 0.9), temperature=0.0)))
    # gamma = 64 (eight windows) with long accepted prefixes
    t = rng.normal(0, 1, (5, 65, 100)).astype(np.float32)
    out.append(("gamma64", I.from_arrays(t, t[:, :64].copy(), argmax_tokens(t, 0.97), temperature=0.0)))
    # V = 2, gamma = 1
    t = rng.normal(0, 1, (40, 2, 2)).astype(np.float32)
    out.append(("V2", I.from_arrays(t, t[:, :1].copy(), argmax_tokens(t, 0.5), temperature=0.0)))
    # bf16 with odd V: rows start at every 2-byte offset of a 16-byte block
    t = rng.normal(0, 3, (9, 4, 4099)).astype(np.float32)
    tb = I.f32_to_bf16_bits(t)
    out.append(("bf16-oddV", I.from_arrays(tb, tb[:, :3].copy(), argmax_tokens(tb, 0.7), temperature=0.0)))
    # the maximum at the first and at the last entry of a row
    t = rng.normal(0, 1, (4, 3, 5003)).astype(np.float32)
    t[:2, :, 0] = 9.0
    t[2:, :, -1] = 9.0
    out.append(("ends", I.from_arrays(t, t[:, :2].copy(), argmax_tokens(t, 0.8), temperature=0.0)))
    # top-k given: changes nothing in the arg-max mode
    t = rng.normal(0, 2, (16, 4, 2000)).astype(np.float32)
    out.append(("topk-ignored", I.from_arrays(t, t[:, :3].copy(), argmax_tokens(t, 0.8), temperature=0.0,
                                              top_k=5)))
    return out


GREEDY_EDGES = _greedy_edges()


@pytest.mark.parametrize("name,w", GREEDY_EDGES, ids=[e[0] for e in GREEDY_EDGES])
def test_greedy_edge_cases(name, w):
    _say(f"case greedy edge {name} B={w.B} gamma={w.gamma} V={w.V} dtype={w.target.dtype}")
    g = PT.run_gpu(w, 11)
    _check(PT.compare(w, 11, g), f"greedy edge {name}")


def test_greedy_invalid_tokens_and_workspace_reuse():
    """Invalid drafts flag their sequence; one dirty workspace serves greedy,
    sampling and top-k calls in turn."""
    import torch
    import rejection_sampling_verify_17_amd as S
    ws = torch.full((S.workspace_bytes(256, 8, 152064, 50, S.SV_BF16) + (1 << 20),), 0x5A, dtype=torch.uint8,
                    device="cuda")
    w = I.make("g4b", B=64)
    tok = w.tokens.copy()
    tok[3, 2] = w.V
    tok[7, 0] = -1
    wi = I.from_arrays(w.target, w.draft, tok, temperature=0.0)
    for name, wk in (("g4b-invalid", wi), ("c3", I.make("c3", B=4)), ("g2", I.make("g2", B=6)),
                     ("c1", I.make("c1")), ("g4b-invalid", wi)):
        tgt, drf, tk = PT.to_device(wk)
        out, n = S.verify(tgt, drf, tk, wk.temperature, wk.top_k, seed=2, workspace=ws)
        torch.cuda.synchronize()
        g = PT.GpuResult(out.cpu().numpy(), n.cpu().numpy())
        _check(PT.compare(wk, 2, g, check_probs=False), f"reuse {name}")
    assert g.n_accepted[3] == -1 and g.n_accepted[7] == -1 and np.all(g.out_tokens[3] == -1)


# ---------------------------------------------------------------------------
# Nucleus (top-p after top-k)
# ---------------------------------------------------------------------------
NUCLEUS = [("c3p", 8), ("c3p", None), ("c2p", 8), ("c2p", None)]


@pytest.mark.parametrize("name,B", NUCLEUS, ids=[f"{n}-B{b or 'full'}" for n, b in NUCLEUS])
def test_nucleus_parity(name, B):
    w = I.make(name, B=B)
    _say(f"case nucleus {name} B={w.B} gamma={w.gamma} V={w.V} T={w.temperature} K={w.top_k} P={w.top_p}")
    tensors = PT.to_device(w)
    for seed in ((3301, 3302) if B else (3303,)):
        g = PT.run_gpu(w, seed, tensors=tensors)
        _check(PT.compare(w, seed, g), f"{name} seed {seed}")


def _nucleus_edges():
    rng = np.random.default_rng(909)
    out = []

    def drafted(d, T, K, P):
        return I.sample_rows(I.logits_f32(d).reshape(-1, d.shape[2]), T, K, rng, top_p=P).reshape(d.shape[:2])

    for K, P in ((7, 0.6), (50, 1e-6), (20, 0.999)):
        t = rng.integers(-4, 5, (6, 3, 500)).astype(np.float32)          # ties at and around the cut
        d = rng.integers(-4, 5, (6, 2, 500)).astype(np.float32)
        tok = drafted(d, 1.0, K, P)
        out.append((f"ties-K{K}-P{P}", I.from_arrays(t, d, tok, top_k=K, top_p=P)))
        out.append((f"ties-K{K}-P{P}-bf16", I.from_arrays(I.f32_to_bf16_bits(t), I.f32_to_bf16_bits(d), tok,
                                                          top_k=K, top_p=P)))
    t = rng.normal(0, 1, (3, 3, 6000)).astype(np.float32)                 # K at the maximum, flat rows
    d = (t[:, :2] + rng.normal(0, 0.5, (3, 2, 6000))).astype(np.float32)
    out.append(("K1024-P0.5", I.from_arrays(t, d, drafted(d, 1.0, 1024, 0.5), top_k=1024, top_p=0.5)))
    tb = I.f32_to_bf16_bits(rng.normal(0, 3, (5, 3, 4099)).astype(np.float32))  # every 2-byte row offset
    db = I.f32_to_bf16_bits((I.bf16_bits_to_f32(tb[:, :2]) + rng.normal(0, 1, (5, 2, 4099))).astype(np.float32))
    out.append(("bf16-oddV", I.from_arrays(tb, db, drafted(db, 0.9, 40, 0.8), temperature=0.9, top_k=40,
                                           top_p=0.8)))
    t = rng.normal(0, 2, (16, 4, 3000)).astype(np.float32)               # p == q: all kept, bonus under top-p
    out.append(("p-equals-q", I.from_arrays(t, t[:, :3].copy(), drafted(t[:, :3], 1.0, 30, 0.7), top_k=30,
                                            top_p=0.7)))
    # no top-k: the cut by mass over the whole row (and K above the 1024 the
    # lists hold), ties at the cut, tiny and large P, both dtypes
    for P in (0.6, 1e-6, 0.999):
        t = rng.integers(-4, 5, (6, 3, 700)).astype(np.float32)
        d = rng.integers(-4, 5, (6, 2, 700)).astype(np.float32)
        tok = drafted(d, 1.0, 0, P)
        out.append((f"noK-ties-P{P}", I.from_arrays(t, d, tok, top_p=P)))
        out.append((f"noK-ties-P{P}-bf16", I.from_arrays(I.f32_to_bf16_bits(t), I.f32_to_bf16_bits(d), tok,
                                                          top_p=P)))
    t = rng.normal(0, 1, (4, 3, 9000)).astype(np.float32)                 # flat rows: thousands kept
    d = (t[:, :2] + rng.normal(0, 0.3, (4, 2, 9000))).astype(np.float32)
    out.append(("noK-flat-P0.9", I.from_arrays(t, d, drafted(d, 1.0, 0, 0.9), top_p=0.9)))
    out.append(("K2000-P0.8", I.from_arrays(t, d, drafted(d, 1.0, 2000, 0.8), top_k=2000, top_p=0.8)))
    tb = I.f32_to_bf16_bits(rng.normal(0, 3, (5, 3, 4099)).astype(np.float32))  # every 2-byte row offset
    db = I.f32_to_bf16_bits((I.bf16_bits_to_f32(tb[:, :2]) + rng.normal(0, 1, (5, 2, 4099))).astype(np.float32))
    out.append(("noK-bf16-oddV", I.from_arrays(tb, db, drafted(db, 0.9, 0, 0.8), temperature=0.9, top_p=0.8)))
    t = rng.normal(0, 2, (16, 4, 3000)).astype(np.float32)               # p == q without top-k
    out.append(("noK-p-equals-q", I.from_arrays(t, t[:, :3].copy(), drafted(t[:, :3], 1.0, 0, 0.7), top_p=0.7)))
    t = rng.normal(0, 2, (8, 4, 2000)).astype(np.float32)                # -inf entries inside the row
    t[:, :, 100:900] = -np.inf
    d = (t[:, :3] + rng.normal(0, 0.5, (8, 3, 2000))).astype(np.float32)
    out.append(("noK-neg-inf", I.from_arrays(t, d, drafted(d, 1.0, 0, 0.95), top_p=0.95)))
    tb, db = I.f32_to_bf16_bits(t), I.f32_to_bf16_bits(d)
    out.append(("noK-neg-inf-bf16", I.from_arrays(tb, db, drafted(db, 1.0, 0, 0.95), top_p=0.95)))
    # every logit negative, ties at the cut: the cut's key lies below the
    # sign flip (bf16: its low key bits are all ones)
    for P in (0.6, 0.97):
        t = rng.integers(-14, -5, (6, 3, 700)).astype(np.float32)
        d = (t[:, :2] + rng.integers(-1, 2, (6, 2, 700))).astype(np.float32)
        tok = drafted(d, 1.0, 0, P)
        out.append((f"noK-negative-P{P}", I.from_arrays(t, d, tok, top_p=P)))
        out.append((f"noK-negative-P{P}-bf16", I.from_arrays(I.f32_to_bf16_bits(t), I.f32_to_bf16_bits(d), tok,
                                                              top_p=P)))
    return out


NUCLEUS_EDGES = _nucleus_edges()


@pytest.mark.parametrize("name,w", NUCLEUS_EDGES, ids=[e[0] for e in NUCLEUS_EDGES])
def test_nucleus_edge_cases(name, w):
    _say(f"case nucleus edge {name} B={w.B} gamma={w.gamma} V={w.V} K={w.top_k} P={w.top_p}")
    for seed in (13, 14):
        g = PT.run_gpu(w, seed)
        _check(PT.compare(w, seed, g), f"nucleus edge {name} seed {seed}")
    if name in ("p-equals-q", "noK-p-equals-q"):
        assert np.all(g.n_accepted == w.gamma)


# ---------------------------------------------------------------------------
# Extreme shapes and temperatures, every path
# ---------------------------------------------------------------------------
def _extreme_workloads():
    rng = np.random.default_rng(4242)
    out = []
    # many sequences, tiny vocabulary (grids far larger than the chip)
    t = rng.normal(0, 2, (65536, 3, 16)).astype(np.float32)
    d = (t[:, :2] + rng.normal(0, 1, (65536, 2, 16))).astype(np.float32)
    tok = I.sample_rows(d.reshape(-1, 16), 1.0, 0, rng).reshape(65536, 2)
    out.append(("B65536-V16", I.from_arrays(t, d, tok)))
    out.append(("B65536-V16-topk3", I.from_arrays(t, d, I.sample_rows(d.reshape(-1, 16), 1.0, 3, rng).reshape(65536, 2),
                                                  top_k=3)))
    out.append(("B65536-V16-argmax", I.from_arrays(t, d, np.argmax(d, axis=2).astype(np.int32), temperature=0.0)))
    # a million-entry vocabulary (4 MB rows; every thread walks many vectors)
    V = 1 << 20
    t = rng.normal(0, 3, (2, 3, V)).astype(np.float32)
    d = (t[:, :2] + rng.normal(0, 1, (2, 2, V))).astype(np.float32)
    out.append(("V1M", I.from_arrays(t, d, I.sample_rows(d.reshape(-1, V), 1.0, 0, rng).reshape(2, 2))))
    tb, db = I.f32_to_bf16_bits(t), I.f32_to_bf16_bits(d)
    out.append(("V1M-bf16-topk40", I.from_arrays(tb, db, I.sample_rows(I.bf16_bits_to_f32(db).reshape(-1, V), 1.0, 40,
                                                                        rng).reshape(2, 2), top_k=40)))
    out.append(("V1M-argmax", I.from_arrays(t, d, np.argmax(d, axis=2).astype(np.int32), temperature=0.0)))
    # temperatures far from 1
    t = rng.normal(0, 2, (16, 4, 3000)).astype(np.float32)
    d = (t[:, :3] + rng.normal(0, 0.5, (16, 3, 3000))).astype(np.float32)
    for T in (0.02, 50.0):
        out.append((f"T{T}", I.from_arrays(t, d, I.sample_rows(d.reshape(-1, 3000), T, 0, rng).reshape(16, 3),
                                           temperature=T)))
    return out


EXTREME = _extreme_workloads()


@pytest.mark.parametrize("name,w", EXTREME, ids=[e[0] for e in EXTREME])
def test_extreme_shapes(name, w):
    _say(f"case extreme {name} B={w.B} gamma={w.gamma} V={w.V} T={w.temperature} K={w.top_k}")
    g = PT.run_gpu(w, 21, debug=w.B <= 4096)
    _check(PT.compare(w, 21, g, check_probs=w.B <= 4096), f"extreme {name}")
