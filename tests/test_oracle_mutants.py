"""Plant plausible mistakes in a copy of the oracle (on the CPU) and show that
at least one pin catches each of them.  The oracle itself is never modified."""
import os
import shutil
import tempfile

import pytest

import oracle_checks as C
from oracle import oracle as O
from workloads import synth as I

# (name, text in sv_oracle.c, replacement, checks expected to catch it)
MUTANTS = [
    ("residual sign flipped", "double d = q[v] - p[v];", "double d = p[v] - q[v];",
     ["enumeration", "output_is_q"]),
    ("ratio inverted", "return u < q_t / p_t;", "return u < p_t / q_t;",
     ["enumeration", "golden", "draft_length"]),
    ("bonus from row gamma-1",
     "((size_t)b * (gamma + 1) + gamma) * V * esz", "((size_t)b * (gamma + 1) + gamma - 1) * V * esz",
     ["special"]),
    ("one uniform for every position",
     "svo_word(seed, seq, (uint32_t)j, 0u, SVO_ACCEPT)", "svo_word(seed, seq, 0u, 0u, SVO_ACCEPT)",
     ["n_distribution"]),
    ("Gumbel noise sign flipped", "key = log(w[v]) - log(svo_exponential", "key = log(w[v]) + log(svo_exponential",
     ["gumbel"]),
    ("temperature multiplies", "exp(svo_logit(row, dtype, v) / T - m)", "exp(svo_logit(row, dtype, v) * T - m)",
     ["torch"]),
    ("top-k ties keep the larger index", "return (x->v < y->v) ? -1 : (x->v > y->v);",
     "return (x->v > y->v) ? -1 : (x->v < y->v);", ["topk"]),
    ("token the target never emits is accepted",
     "if (!(q_t > 0.0)) return 0;", "if (!(q_t > 0.0)) return 1;", ["enumeration", "special"]),
    ("Philox key bump skipped", "k0 += PHX_W0;", "k0 += 0;", ["philox"]),
    ("draft tokens drawn on the SAMPLE stream",
     "svo_gumbel_draw(p, V, seed, seq_offset + (uint64_t)b, (uint32_t)j, SVO_DRAFT, &g)",
     "svo_gumbel_draw(p, V, seed, seq_offset + (uint64_t)b, (uint32_t)j, SVO_SAMPLE, &g)", ["draft"]),
    ("draft row without temperature",
     "svo_row_probs_p(prow, dtype, V, temperature, top_k, top_p, p, keep, &mg);\n                if (margin) margin[(size_t)b",
     "svo_row_probs_p(prow, dtype, V, 1.0f, top_k, top_p, p, keep, &mg);\n                if (margin) margin[(size_t)b", ["draft"]),
    ("token probabilities of p and q swapped",
     "svo_row_probs_p(qrow, dtype, V, temperature, top_k, top_p, row, keep, NULL);",
     "svo_row_probs_p(prow, dtype, V, temperature, top_k, top_p, row, keep, NULL);", ["token_probs"]),
    ("token probabilities without top-k",
     "svo_row_probs_p(prow, dtype, V, temperature, top_k, top_p, row, keep, NULL);",
     "svo_row_probs_p(prow, dtype, V, temperature, 0, top_p, row, keep, NULL);", ["token_probs"]),
    ("nucleus drops the entry that reaches P", "if (cum >= P) { m = i; break; }",
     "if (cum >= P) { m = i - 1; cum = before; break; }", ["nucleus", "golden_adjusted"]),
    ("arg-max ties keep the larger index",
     "if (svo_logit(row, dtype, v) > svo_logit(row, dtype, best)) best = v;",
     "if (svo_logit(row, dtype, v) >= svo_logit(row, dtype, best)) best = v;", ["greedy"]),
]


def _run(check):
    if check == "enumeration":
        C.check_enumeration_v4()
    elif check == "golden":
        C.check_golden_examples()
    elif check == "output_is_q":
        C.check_output_is_q(B=100_000)
    elif check == "special":
        C.check_special_cases()
    elif check == "n_distribution":
        C.check_accept_rate_and_n_distribution(B=100_000)
    elif check == "gumbel":
        C.check_gumbel_sampler(n=100_000)
    elif check == "torch":
        C.check_row_probs_vs_torch()
    elif check == "topk":
        C.check_topk_vs_stable_sort()
    elif check == "draft":
        C.check_draft_sampler(n=100_000)
    elif check == "golden_adjusted":
        C.check_golden_adjusted()
    elif check == "nucleus":
        C.check_nucleus()
    elif check == "token_probs":
        C.check_golden_token_probs()
    elif check == "greedy":
        C.check_greedy()
    elif check == "draft_length":
        import markov_rounds as M
        M.check_acceptance_by_draft_length(M.run_oracle, B=20_000)
    elif check == "philox":
        import rocrand_ref
        rr = rocrand_ref.load()
        if rr is None:
            pytest.skip("no hipcc for the rocRAND helper")
        C.check_philox_vs_rocrand(rr, n=256)
    else:
        raise KeyError(check)


@pytest.mark.parametrize("name,old,new,checks", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(name, old, new, checks):
    src = open(O.SRC).read()
    assert src.count(old) == 1, f"mutation site not unique: {old!r}"
    tmp = tempfile.mkdtemp(prefix="svo_mutant_")
    try:
        msrc = os.path.join(tmp, "sv_oracle.c")
        with open(msrc, "w") as f:
            f.write(src.replace(old, new))
        lib = O.load(O.build(force=True, src=msrc, out=os.path.join(tmp, "libmut.so")))
        prev = O.use(lib)
        try:
            caught = []
            for check in checks:
                try:
                    _run(check)
                except AssertionError:
                    caught.append(check)
            assert caught, f"mutant '{name}' passed every check in {checks}"
        finally:
            O.use(prev)
    finally:
        shutil.rmtree(tmp)
