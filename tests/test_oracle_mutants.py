"""Each planted mistake in a copy of the oracle must be caught by a pin.

The mistakes are the plausible ones: a wrong rounding, a flipped sort or
comparison, a dropped term of the chunk size, a wrong index, a missing
state update. Each mutant is compiled from the oracle's C source with one
substitution and run through the same checks as the oracle itself."""
import os

import numpy as np
import pytest

import oracle
import pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "ue_oracle.c")

MUTANTS = {
    "quota floors": ("(total + R - 1) / R", "total / R"),
    "candidates lightest first": ("counts[prev] > counts[e] ||",
                                  "counts[prev] < counts[e] ||"),
    "candidate ties id desc": ("counts[prev] == counts[e] && prev < e",
                               "counts[prev] == counts[e] && prev > e"),
    "destination most loaded": ("if (d < 0 || load[x] < load[d])",
                                "if (d < 0 || load[x] > load[d])"),
    "destination ties highest id": ("if (d < 0 || load[x] < load[d])",
                                    "if (d < 0 || load[x] <= load[d])"),
    "destination may sit at quota": ("nfree[x] <= 0 || load[x] >= Q",
                                     "nfree[x] <= 0 || load[x] > Q"),
    "destination needs no free slot": ("nfree[x] <= 0 || load[x] >= Q",
                                       "load[x] >= Q"),
    "chunk ignores headroom": ("if (Q - load[d] < m)", "if (0)"),
    "chunk ignores remainder": ("if (rem[e] < m)", "if (0)"),
    "chunk ignores source excess": ("int64_t m = load[r] - Q;",
                                    "int64_t m = rem[e];"),
    "highest spare slot first": ("N + (S - nfree[d])", "N + (nfree[d] - 1)"),
    "source load not reduced": ("load[r] -= m;", ";"),
    "free slot not consumed": ("nfree[d] -= 1;", ";"),
    "master keeps full count": ("rep_cap[n] = (int32_t)rem[e];",
                                "rep_cap[n] = counts[e];"),
    "native rank round robin": ("load[e / N] += counts[e];",
                                "load[e % R] += counts[e];"),
    "native slot index": ("rep_slot[n] = (e / N) * NS + (e % N);",
                          "rep_slot[n] = (e / N) * NS;"),
    "inclusive slot offsets": ("slot_off[p + 1] = slot_off[p] + slot_cap[p];",
                               "slot_off[p + 1] = slot_off[p] + slot_cap[p]"
                               " + (p == 0 ? slot_cap[0] : 0);"),
    "prefix boundary inclusive": ("if (j < prefix + rep_cap[i])",
                                  "if (j <= prefix + rep_cap[i])"),
    "position ignores prefix": ("slot_off[p] + (j - prefix)",
                                "slot_off[p] + j"),
    "rank of slot": ("rank_counts[p / NS] += 1;", "rank_counts[p % R] += 1;"),
    "upper id bound": ("if (e < 0 || e >= n_experts) {\n            ++invalid;",
                       "if (e < 0 || e > n_experts) {\n            ++invalid;"),
    "residual is max excess": ("residual += load[r] - Q;",
                               "residual = load[r] - Q;"),
    "quota counts experts": ("(total + R - 1) / R", "(total + E - 1) / E"),
    "no exhausted flag": ("exhausted = 1;\n                break;",
                          "break;"),
    "best fit takes the most headroom": ("load[x] > load[b])",
                                         "load[x] < load[b])"),
    "best fit ties highest id": ("load[x] > load[b])", "load[x] >= load[b])"),
    "best fit ignores the fit": ("Q - load[x] >= m &&", ""),
    "search keeps the last quota that works": ("Q = M;\n                break;",
                                               "Q = M;"),
    "search step rounds down": ("(Q0 + 255) / 256", "Q0 / 256"),
    "search skips the plain quota": ("for (int32_t j = 0; j < 64; ++j)",
                                     "for (int32_t j = 1; j < 64; ++j)"),
    "plan made at the plain quota": (
        "const int exhausted = greedy_at(counts, E, R, S, policy, Q, load,",
        "const int exhausted = greedy_at(counts, E, R, S, policy, Q0, load,"),
    "replica before master": ("rep_slot[n] = (e / N) * NS + (e % N);\n"
                              "        rep_cap[n] = (int32_t)rem[e];\n"
                              "        ++n;\n",
                              ""),
}


def run_all_pins():
    for case in pins.golden_cases():
        pins.check_golden(case)
    rng = np.random.default_rng(11)
    for _ in range(300):
        pins.check_instance(*pins.random_instance(rng))
    for _ in range(300):
        pins.check_instance(*pins.random_instance(rng), policy=1)
    for _ in range(150):
        pins.check_instance(*pins.random_instance(rng), quota_mode=1)
    for _ in range(150):
        pins.check_instance(*pins.random_instance(rng), policy=1,
                            quota_mode=1)
    pins.check_no_spares(np.random.default_rng(1))
    pins.check_one_rank(np.random.default_rng(2))
    pins.check_balanced()
    pins.check_single_hot(max_ranks=6)
    pins.check_invalid_ids()


def test_unmutated_oracle_passes():
    run_all_pins()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site for '{name}' not unique"
    mutated = tmp_path / "mutant.c"
    mutated.write_text(src.replace(old, new))
    lib = oracle.build(out=str(tmp_path / "libmutant.so"), src=str(mutated),
                       strict=False)
    with oracle.library(lib):
        with pytest.raises((AssertionError, IndexError, ValueError)):
            run_all_pins()
