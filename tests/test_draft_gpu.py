"""Draft-token sampling and acceptance counts on the GPU, against the oracle.

Tokens must equal the oracle's draws on the same DRAFT stream bit for bit,
except a draw whose two best keys (natural log) are within 1e-5 in the
oracle (a knife-edge arg-max, decided by rounding); at temperature 0 without
exception.  The acceptance histogram must equal a count of n_accepted."""
import sys

import numpy as np
import pytest

import parity as PT
from oracle import oracle as O
from workloads import synth as I

pytestmark = pytest.mark.gpu

KNIFE = 1e-5


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _draft_tensor(w):
    import torch
    if w.draft.dtype == np.uint16:
        return torch.from_numpy(w.draft.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(w.draft).cuda()


def _compare_draft(w, seed, got, seq_offset=0):
    want, gap, margin = O.draft_sample(w.draft, w.temperature, w.top_k, seed=seed, seq_offset=seq_offset,
                                       top_p=w.top_p, with_margin=True)
    diff = got != want
    # knife-edges: near-tied best keys, or (top-p) a nucleus cut within rounding
    exempt = diff & ((gap < KNIFE) | (margin < KNIFE)) if w.temperature != 0.0 else np.zeros_like(diff)
    bad = diff & ~exempt
    _say(f"rows {got.size}, differing {int(diff.sum())}, knife-edge {int(exempt.sum())}")
    assert not bad.any(), f"{int(bad.sum())} draws differ: first at {np.argwhere(bad)[:5].tolist()}"
    if w.top_k > 0 and w.temperature != 0.0:   # every draw lies in the kept set
        for b, j in zip(*np.nonzero(np.ones_like(got, dtype=bool))):
            if (b * w.gamma + j) % 97 == 0 and margin[b, j] >= KNIFE:
                assert O.row_probs(w.draft[b, j], w.temperature, w.top_k, w.top_p)[got[b, j]] > 0
    return want


CASES = [("c4b", 64), ("c4b", None), ("c2", 4), ("c3", 8), ("c3p", 8), ("c2p", 8), ("g4b", 32), ("c1", None)]


@pytest.mark.parametrize("name,B", CASES, ids=[f"{n}-B{b or 'full'}" for n, b in CASES])
def test_draft_sample_parity(name, B):
    import torch
    import rejection_sampling_verify_17_amd as S
    w = I.make(name, B=B)
    _say(f"case draft {name} B={w.B} gamma={w.gamma} V={w.V} T={w.temperature} K={w.top_k}")
    d = _draft_tensor(w)
    for seed in (7, 8):
        got = S.draft_sample(d, w.temperature, w.top_k, seed=seed, top_p=w.top_p)
        torch.cuda.synchronize()
        _compare_draft(w, seed, got.cpu().numpy())


def _edge_drafts():
    rng = np.random.default_rng(77)
    out = []
    z = rng.integers(-3, 4, (6, 3, 500)).astype(np.float32)           # heavy ties
    for T, K in ((1.0, 0), (1.0, 7), (0.0, 0), (0.6, 1)):
        out.append((f"ties-T{T}-K{K}", I.from_arrays(np.zeros((6, 4, 500), np.float32), z,
                                                     np.zeros((6, 3), np.int32), temperature=T, top_k=K)))
    zb = I.f32_to_bf16_bits(rng.normal(0, 3, (5, 2, 4099)).astype(np.float32))  # every 2-byte row offset
    out.append(("bf16-oddV", I.from_arrays(np.zeros((5, 3, 4099), np.uint16), zb, np.zeros((5, 2), np.int32),
                                           temperature=0.9)))
    out.append(("bf16-oddV-topk", I.from_arrays(np.zeros((5, 3, 4099), np.uint16), zb,
                                                np.zeros((5, 2), np.int32), temperature=0.9, top_k=30)))
    z2 = rng.normal(0, 1, (40, 1, 2)).astype(np.float32)
    out.append(("V2", I.from_arrays(np.zeros((40, 2, 2), np.float32), z2, np.zeros((40, 1), np.int32))))
    zt = rng.integers(-3, 4, (6, 3, 500)).astype(np.float32)
    out.append(("ties-K20-P0.6", I.from_arrays(np.zeros((6, 4, 500), np.float32), zt, np.zeros((6, 3), np.int32),
                                               top_k=20, top_p=0.6)))
    out.append(("ties-noK-P0.6", I.from_arrays(np.zeros((6, 4, 500), np.float32), zt, np.zeros((6, 3), np.int32),
                                               top_p=0.6)))
    zf = rng.normal(0, 1, (3, 2, 9000)).astype(np.float32)
    out.append(("flat-K2000-P0.8", I.from_arrays(np.zeros((3, 3, 9000), np.float32), zf, np.zeros((3, 2), np.int32),
                                                 top_k=2000, top_p=0.8)))
    zi = rng.normal(0, 2, (4, 2, 3000)).astype(np.float32)
    zi[:, :, 100:2900] = -np.inf
    out.append(("neg-inf", I.from_arrays(np.zeros((4, 3, 3000), np.float32), zi, np.zeros((4, 2), np.int32))))
    return out


EDGE = _edge_drafts()


@pytest.mark.parametrize("name,w", EDGE, ids=[e[0] for e in EDGE])
def test_draft_sample_edges(name, w):
    import torch
    import rejection_sampling_verify_17_amd as S
    _say(f"case draft edge {name} B={w.B} gamma={w.gamma} V={w.V} T={w.temperature} K={w.top_k}")
    got = S.draft_sample(_draft_tensor(w), w.temperature, w.top_k, seed=3, seq_offset=11, top_p=w.top_p)
    torch.cuda.synchronize()
    _compare_draft(w, 3, got.cpu().numpy(), seq_offset=11)


def test_draft_then_verify_then_count():
    """A whole step on the GPU: draw the drafts, verify them, count the
    acceptances; every stage equals the oracle (or a plain count)."""
    import torch
    import rejection_sampling_verify_17_amd as S
    w = I.make("c4b", B=256)
    tgt, drf, _ = PT.to_device(w)
    tok = S.draft_sample(drf, w.temperature, w.top_k, seed=21)
    torch.cuda.synchronize()
    tok_np = tok.cpu().numpy()
    _compare_draft(w, 21, tok_np)
    w2 = I.from_arrays(w.target, w.draft, tok_np, w.temperature, w.top_k)
    out, n = S.verify(tgt, drf, tok, w.temperature, w.top_k, seed=22)
    torch.cuda.synchronize()
    g = PT.GpuResult(out.cpu().numpy(), n.cpu().numpy())
    rep = PT.compare(w2, 22, g, check_probs=False)
    _say("verify of GPU drafts", rep.summary())
    assert rep.ok() and rep.mismatches == 0
    h = S.accept_histogram(n, w.gamma)
    torch.cuda.synchronize()
    want = np.bincount(g.n_accepted + 1, minlength=w.gamma + 2)
    assert np.array_equal(h.cpu().numpy(), want)
    _say(f"acceptance histogram (invalid, n=0..{w.gamma}): {h.cpu().numpy().tolist()}")


def test_accept_histogram_counts():
    import torch
    import rejection_sampling_verify_17_amd as S
    rng = np.random.default_rng(5)
    for B, gamma in ((1, 1), (1000, 4), (70000, 64)):
        n = rng.integers(-1, gamma + 1, B).astype(np.int32)
        n[:: 7] = gamma + 3      # never written by sv_verify: counted as invalid
        h = S.accept_histogram(torch.from_numpy(n).cuda(), gamma)
        torch.cuda.synchronize()
        want = np.bincount(np.where((n < 0) | (n > gamma), 0, n + 1), minlength=gamma + 2)
        assert np.array_equal(h.cpu().numpy(), want), (B, gamma)
