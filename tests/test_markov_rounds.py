"""Speculative decoding over a Markov model pair: the committed sequences
follow the target chain (oracle on the CPU; the GPU path on the GPU, with its
trajectories equal to the oracle's)."""
import numpy as np
import pytest

import markov_rounds as M
from workloads import synth as I


def _tv_and_noise(counts: np.ndarray, probs: np.ndarray, seed: int = 3, runs: int = 100):
    n = int(counts.sum())
    got = 0.5 * np.abs(counts / n - probs).sum()
    rng = np.random.default_rng(seed)
    flat = probs.ravel()
    noise = [0.5 * np.abs(rng.multinomial(n, flat) / n - flat).sum() for _ in range(runs)]
    return got, float(np.quantile(noise, 0.99))


def test_oracle_rounds_follow_the_target_chain():
    """Two-token prefixes of the committed sequences are distributed as the
    target chain's, within the noise of sampling the chain directly (TV at
    most the 99th percentile of direct samples of the same size)."""
    pair = I.markov_pair(V=16, seed=11)
    B = 120_000
    x0 = np.full(B, 3, np.int32)
    tr = M.run_oracle(pair, x0, gamma=3, rounds=2)
    assert all(len(s) >= 2 for s in tr.tokens)
    got, thr = _tv_and_noise(M.first_two_counts(tr, pair.V), M.exact_first_two(pair, 3))
    print(f"TV {got:.5f}, direct-sampling p99 {thr:.5f}, mean accepted {np.mean(tr.n_per_round[0]):.3f}")
    assert got <= thr
    # the drafts are really the draft's: a worse draft is accepted less
    far = I.markov_pair(V=16, seed=11, draft_sigma=4.0)
    tr_far = M.run_oracle(far, x0[:20_000], gamma=3, rounds=1)
    assert np.mean(tr_far.n_per_round[0]) < np.mean(tr.n_per_round[0]) - 0.3


@pytest.mark.gpu
def test_gpu_rounds_equal_oracle_rounds():
    """Three rounds of 3,000 sequences: drafts, n and committed tokens equal
    the oracle's bit for bit (any knife-edge decision would be reported by a
    mismatch here; V = 64 makes one unlikely)."""
    pair = I.markov_pair(V=64, seed=21)
    x0 = (np.arange(3000) % 64).astype(np.int32)
    g = M.run_gpu(pair, x0, gamma=4, rounds=3)
    o = M.run_oracle(pair, x0, gamma=4, rounds=3)
    for r in range(3):
        assert np.array_equal(g.drafts[r], o.drafts[r]), f"round {r}: drafts differ"
        assert np.array_equal(g.n_per_round[r], o.n_per_round[r]), f"round {r}: n differs"
    assert g.tokens == o.tokens


@pytest.mark.gpu
def test_gpu_rounds_follow_the_target_chain():
    pair = I.markov_pair(V=32, seed=31)
    B = 400_000
    x0 = np.full(B, 5, np.int32)
    tr = M.run_gpu(pair, x0, gamma=4, rounds=2)
    assert all(len(s) >= 2 for s in tr.tokens)
    got, thr = _tv_and_noise(M.first_two_counts(tr, pair.V), M.exact_first_two(pair, 5))
    print(f"TV {got:.5f}, direct-sampling p99 {thr:.5f}")
    assert got <= thr


def test_oracle_acceptance_by_draft_length():
    """The oracle's rounds against the chain's exact all-accepted rates
    (a pin of the acceptance rule through a closed form), and E_g = sum A_i."""
    pair = I.markov_pair(V=32, seed=41)
    x0 = np.full(30_000, 7, np.int32)
    M.check_acceptance_by_draft_length(M.run_oracle, B=30_000)


@pytest.mark.gpu
def test_gpu_acceptance_by_draft_length():
    """The same table from the GPU path (draft sampler and verification),
    equal to the oracle's sequence by sequence."""
    pair = I.markov_pair(V=64, seed=43)
    x0 = np.full(60_000, 9, np.int32)
    gs = range(1, 9)
    n = M.acceptance_by_draft_length(M.run_gpu, pair, x0, gs)
    M.draft_length_table(n, M.exact_all_accepted(pair, 9, 8), "gpu")
    o = M.acceptance_by_draft_length(M.run_oracle, pair, x0, gs)
    for g in gs:
        assert np.array_equal(n[g], o[g]), f"gamma {g}: GPU and oracle differ"
