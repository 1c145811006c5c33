"""The oracle against what the pages and the mathematics fix (CPU only).

Each test names the passage it pins; the checks themselves live in
oracle_checks.py so the mutant tests can rerun them on broken copies."""
import numpy as np
import pytest

import oracle_checks as C
from oracle import oracle as O
from workloads import synth as I


def test_philox_matches_rocrand_engine():
    """Philox4x32-10 (Salmon et al., SC'11) equals rocRAND's engine, run from its
    public source header on the CPU, on 4096 counters and keys."""
    import rocrand_ref  # CPU-only helper, built from rocRAND's source header
    rr = rocrand_ref.load()
    if rr is None:
        pytest.skip("hipcc not available to build the rocRAND helper")
    C.check_philox_vs_rocrand(rr)


def test_word_layout():
    C.check_word_layout()


def test_variates():
    C.check_variates()


def test_golden_worked_examples():
    """Hand-derived values of the acceptance rule and residual (tests/golden)."""
    C.check_golden_examples()


def test_golden_adjusted_distributions():
    """Hand-worked top-k, nucleus and arg-max rows (tests/golden)."""
    C.check_golden_adjusted()


def test_golden_token_probs():
    """Hand-worked p_j(t_j), q_j(t_j) per position (tests/golden)."""
    C.check_golden_token_probs()


def test_enumeration_v4_output_equals_q():
    """P1 + P2: exact enumeration over all 2^24 acceptance uniforms."""
    C.check_enumeration_v4()


def test_accept_rate_and_n_distribution():
    """P2 + P3: Monte-Carlo acceptance rate and distribution of n vs closed forms."""
    C.check_accept_rate_and_n_distribution()


@pytest.mark.parametrize("temperature,top_k", [(1.0, 0), (0.6, 0), (1.0, 5)])
def test_output_distribution_is_q(temperature, top_k):
    C.check_output_is_q(temperature=temperature, top_k=top_k)


def test_60k_total_variation_at_most_divergent_position():
    """P4: the page's 60,000-draw TV test, on workload c0."""
    w = I.make("c0")
    info = C.check_60k_tv(w)
    print(info)


def test_special_cases():
    C.check_special_cases()


def test_nucleus():
    """Top-p (ai-trend.me, section "how it works": nucleus sampling is sampling
    from an adjusted distribution)."""
    C.check_nucleus()


def test_greedy_mode():
    """T = 0 (arg-max mode of the ai-trend.me page, section "how it works")."""
    C.check_greedy()


def test_draft_sampler():
    """Draft tokens for a step ([SDE] "how it works": the draft proposes first)."""
    C.check_draft_sampler()


def test_gumbel_sampler_is_multinomial():
    C.check_gumbel_sampler()


def test_row_probs_vs_torch_softmax():
    C.check_row_probs_vs_torch()


def test_topk_vs_stable_sort():
    C.check_topk_vs_stable_sort()


@pytest.mark.parametrize("name,B", [("c0", 1), ("c1", 8), ("c2", 4), ("c3", 3), ("c4b", 16)])
def test_output_structure_on_workloads(name, B):
    w = I.make(name, B=B)
    res = O.verify(w.target, w.draft, w.tokens, w.temperature, w.top_k, seed=3000)
    C.check_output_structure(w, res)
    # u and ratio are recorded exactly for the judged prefix
    for b in range(B):
        n = res.n_accepted[b]
        judged = min(n + 1, w.gamma)
        assert np.all(np.isfinite(res.u[b, :judged]))
        assert np.all(np.isnan(res.u[b, judged:]))


def test_invalid_draft_token_marks_sequence():
    w = I.make("c0")
    tok = w.tokens.copy()
    tgt = np.concatenate([w.target] * 3)
    drf = np.concatenate([w.draft] * 3)
    tok = np.concatenate([tok] * 3)
    tok[1, 2] = w.V          # out of range
    tok[2, 0] = -1
    res = O.verify(tgt, drf, tok, 1.0, 0, seed=1)
    assert res.n_accepted[0] >= 0
    assert res.n_accepted[1] == -1 and np.all(res.out_tokens[1] == -1)
    assert res.n_accepted[2] == -1 and np.all(res.out_tokens[2] == -1)


def test_oracle_is_deterministic_and_thread_independent():
    w = I.make("c1")
    a = O.verify(w.target, w.draft, w.tokens, w.temperature, 0, seed=5, nthreads=1)
    b = O.verify(w.target, w.draft, w.tokens, w.temperature, 0, seed=5, nthreads=4)
    assert np.array_equal(a.out_tokens, b.out_tokens)
    assert np.array_equal(a.n_accepted, b.n_accepted)
    # seq_offset shifts the streams: sequence b at offset o == sequence b+o at offset 0
    w2 = I.make("c1", B=4)
    full = O.verify(w.target, w.draft, w.tokens, w.temperature, 0, seed=5, seq_offset=0)
    part = O.verify(w.target[4:], w.draft[4:], w.tokens[4:], w.temperature, 0, seed=5, seq_offset=4)
    assert np.array_equal(full.out_tokens[4:], part.out_tokens)
    assert w2.target.shape[0] == 4 and np.array_equal(w2.target, w.target[:4])
