"""Each planted mistake in a copy of the oracle must be caught by a pin.

The mistakes are the plausible ones: a wrong rounding, a flipped sort or
comparison, a dropped term of the chunk size, a wrong index, a missing
state update. Each mutant is compiled from the oracle's C source with one
substitution and run through the same checks as the oracle itself."""
import os
import subprocess
import sys

import numpy as np
import pytest

# the module also runs as a child process (see caught()), outside pytest
_ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if _ROOT not in sys.path:
    sys.path.insert(0, _ROOT)

import oracle  # noqa: E402
import pins  # noqa: E402

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
                          "break;", 2),
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
        "const int exhausted = pass_at(policy, counts, E, R, S, Q0, Q, load,",
        "const int exhausted = pass_at(policy, counts, E, R, S, Q0, Q0, load,"),
    "search grain 128": ("(Q0 + 255) / 256", "(Q0 + 127) / 128"),
    "search 32 steps": ("for (int32_t j = 0; j < 64; ++j)",
                        "for (int32_t j = 0; j < 32; ++j)"),
    "search without a working step keeps the last one tried": (
        "        for (int32_t j = 0; j < 64; ++j) {\n"
        "            const int64_t M = Q0 + j * step;\n",
        "        for (int32_t j = 0; j < 64; ++j) {\n"
        "            const int64_t M = Q0 + j * step;\n"
        "            Q = M;\n"),
    "fault counted in rank counts": (
        "        const int32_t p = rep_slot[hit];\n",
        "        const int32_t p = rep_slot[hit];\n"
        "        rank_counts[p / NS] += 1;\n"),
    "faulted assignment keeps a position": ("        inv_perm[a] = -1;\n",
                                            "        inv_perm[a] = 0;\n"),
    "ids out of range not counted as faults": (
        "        if (e < 0 || e >= E) {\n            ++faults;",
        "        if (e < 0 || e >= E) {\n            ;"),
    "capacity overflow goes to the last replica": (
        "        if (hit < 0) {\n            ++faults;\n            continue;\n        }",
        "        if (hit < 0) {\n            hit = rep_off[e + 1] - 1;\n"
        "            prefix -= rep_cap[hit];\n        }"),
    "cover: small amounts largest first": (
        "before = ge ? amt0[p] > amt0[e] : amt0[p] < amt0[e];",
        "before = amt0[p] > amt0[e];"),
    "cover: large amounts smallest first": (
        "before = ge ? amt0[p] > amt0[e] : amt0[p] < amt0[e];",
        "before = amt0[p] < amt0[e];"),
    "cover: amount equal to H0 counted as large": (
        "const int gp = amt0[p] > H0, ge = amt0[e] > H0;",
        "const int gp = amt0[p] >= H0, ge = amt0[e] >= H0;"),
    "cover: large amounts first": ("before = gp < ge;", "before = gp > ge;"),
    "cover: H0 at the pass's quota": (
        "if (S > 0 && load[r] < Q0 && Q0 - load[r] > H0)\n            H0 = Q0 - load[r];",
        "if (S > 0 && load[r] < Q && Q - load[r] > H0)\n            H0 = Q - load[r];"),
    "cover: order from the pass's amounts": (
        "amounts_at(counts, E, R, load, Q0, amt0);",
        "amounts_at(counts, E, R, load, Q, amt0);"),
    "cover: amounts from the lightest expert": (
        "                if (best < 0 || counts[e] > counts[best])\n                    best = e;\n            }\n            prev = best;",
        "                if (best < 0 || counts[e] < counts[best])\n                    best = e;\n            }\n            prev = best;"),
    "ascending: amounts largest first": (
        "before = amt0[p] != amt0[e] ? amt0[e] > amt0[p] : p < e;",
        "before = amt0[p] != amt0[e] ? amt0[e] < amt0[p] : p < e;"),
    "ascending: ties to the higher id": (
        "before = amt0[p] != amt0[e] ? amt0[e] > amt0[p] : p < e;",
        "before = amt0[p] != amt0[e] ? amt0[e] > amt0[p] : p > e;"),
    "ascending: covering order instead": ("if (ascending)\n", "if (0)\n"),
    "cover: least loaded instead of best fit": (
        "pick_destination(load, nfree, R, Q, need, 1)",
        "pick_destination(load, nfree, R, Q, need, 0)"),
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
    for _ in range(300):
        pins.check_instance(*pins.random_instance(rng), policy=2)
    for _ in range(150):
        pins.check_instance(*pins.random_instance(rng), policy=2,
                            quota_mode=1)
    for _ in range(300):
        pins.check_instance(*pins.random_instance(rng), policy=3)
    for _ in range(150):
        pins.check_instance(*pins.random_instance(rng), policy=3,
                            quota_mode=1)
    pins.check_no_spares(np.random.default_rng(1))
    pins.check_one_rank(np.random.default_rng(2))
    pins.check_balanced()
    pins.check_single_hot(max_ranks=6)
    pins.check_invalid_ids()


# exit status of the child when a pin caught the mistake
CAUGHT = 3


def build_mutant(name, tmp_path):
    old, new, *times = MUTANTS[name]
    times = times[0] if times else 1     # sites the mistake is planted at
    src = open(SRC).read()
    assert src.count(old) == times, \
        f"mutation site for '{name}' found {src.count(old)} times"
    mutated = tmp_path / "mutant.c"
    mutated.write_text(src.replace(old, new))
    return oracle.build(out=str(tmp_path / "libmutant.so"), src=str(mutated),
                        strict=False)


def caught(lib, replays):
    """Runs every pin against the mutant library in a child process. A pin
    failing, or the mutant crashing (a planted mistake can overrun the
    oracle's own buffers), both count as caught; the child passing every
    pin does not, and any other failure of the child is an error."""
    proc = subprocess.run(
        [sys.executable, os.path.abspath(__file__), lib, str(int(replays))],
        capture_output=True, text=True, timeout=600)
    if proc.returncode == 0:
        return False
    if proc.returncode == CAUGHT or proc.returncode < 0:
        return True
    raise RuntimeError(f"mutant run failed (rc {proc.returncode}):\n"
                       f"{proc.stderr[-2000:]}")


def test_unmutated_oracle_passes():
    run_all_pins()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    assert caught(build_mutant(name, tmp_path), replays=True)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught_without_replays(name, tmp_path):
    """The same, with the Python replays of the rule (quota steps, chunk
    destinations) switched off: the hand-worked cases, closed forms,
    library routines, invariants and brute force must catch every
    mistake on their own."""
    assert caught(build_mutant(name, tmp_path), replays=False)


if __name__ == "__main__":
    # child process of caught(): argv = library path, replays (0 or 1)
    pins.REPLAYS = bool(int(sys.argv[2]))
    with oracle.library(sys.argv[1]):
        try:
            run_all_pins()
        except (AssertionError, IndexError, ValueError):
            sys.exit(CAUGHT)
    sys.exit(0)
