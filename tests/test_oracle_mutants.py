"""The rounding pins catch plausible mistakes in the oracle (CPU only).

Each case plants one mistake in a copy of oracle/tsenor_oracle.c -- a
different reading of the local search or the fill than the one the design
takes from the TSENOR review ("What carries the argument") -- builds the copy
into a temporary library and runs the hand-derived golden cases against it.
Every mutant must fail at least one of them; the unmodified source must pass
all of them through the same harness.
"""
import ctypes
import json
import os
import subprocess

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "tsenor_oracle.c")
GOLDEN = os.path.join(ROOT, "tests", "golden")

R2_HEAD = """        for (int i = 0; i < M; ++i) {
            if (r[i] >= N) continue;
            for (int j = 0; j < M; ++j) {
                if (c[j] >= N) continue;
                for (int ip = 0; ip < M; ++ip)"""

MUTANTS = {
    # the local search looks only at the first deficient pair (like the fill)
    "r2_first_pair_only": (R2_HEAD, """        int fi = 0, fj = 0;
        while (r[fi] >= N) ++fi;
        while (c[fj] >= N) ++fj;
        for (int i = fi; i <= fi; ++i) {
            if (r[i] >= N) continue;
            for (int j = fj; j <= fj; ++j) {
                if (c[j] >= N) continue;
                for (int ip = 0; ip < M; ++ip)"""),
    # ties broken with the deficient column before the deficient row
    "r2_ties_column_first": (R2_HEAD, """        for (int j = 0; j < M; ++j) {
            if (c[j] >= N) continue;
            for (int i = 0; i < M; ++i) {
                if (r[i] >= N) continue;
                for (int ip = 0; ip < M; ++ip)"""),
    # ties to the lexicographically largest move
    "r2_ties_largest": ("""                        float s = sum - A[ip * M + jp];
                        if (!found || s > best) {
                            found = 1;
                            best = s;
                            bi = i; bj = j; bip = ip; bjp = jp;""",
                        """                        float s = sum - A[ip * M + jp];
                        if (!found || s >= best) {
                            found = 1;
                            best = s;
                            bi = i; bj = j; bip = ip; bjp = jp;"""),
    # the fill starts from the last deficient row
    "r3_last_row": ("""        int i = 0, j = 0;
        while (r[i] >= N) ++i;""", """        int i = M - 1, j = 0;
        while (r[i] >= N) --i;"""),
}


def _build(tmp_path, name, patch):
    src = open(SRC).read()
    if patch is not None:
        old, new = patch
        assert src.count(old) == 1, name
        src = src.replace(old, new)
    c = tmp_path / f"{name}.c"
    so = tmp_path / f"lib{name}.so"
    c.write_text(src)
    subprocess.check_call(["gcc", "-O1", "-fPIC", "-shared", "-ffp-contract=off", "-o", str(so),
                           str(c), "-lm"])
    lib = ctypes.CDLL(str(so))
    P, I = ctypes.c_void_p, ctypes.c_int
    lib.oracle_round_block.argtypes = [P, P, I, I, I, P, P, P, P, P]
    return lib


def _golden_failures(lib):
    """Number of golden cases whose mask, counts or applied moves differ."""
    bad = 0
    for fname in ("rounding_cases.json", "rounding_cases_d2.json"):
        with open(os.path.join(GOLDEN, fname)) as f:
            g = json.load(f)
        S = np.ascontiguousarray(np.array(g["S"], np.float32))
        M = S.shape[0]
        for case in g["cases"]:
            A = np.ascontiguousarray(np.array(case["A"], np.float32))
            Z = np.zeros((M, M), np.uint8)
            Zg = np.zeros((M, M), np.uint8)
            info = np.zeros(3, np.int32)
            sc = np.zeros(M * M, np.float32)
            mv = np.zeros((M * M, 4), np.int32)
            p = lambda a: a.ctypes.data_as(ctypes.c_void_p)
            st = lib.oracle_round_block(p(S), p(A), g["N"], M, case["L"], p(Z), p(info), p(Zg),
                                        p(sc), p(mv))
            n = int(info[1] + info[2])
            same = (st == 0 and np.array_equal(Z, np.array(case["mask"]))
                    and list(info) == case["info"]
                    and np.array_equal(sc[:n], np.array(case["scores"], np.float32))
                    and ("moves" not in case or mv[:n].tolist() == case["moves"]))
            bad += not same
    return bad


def test_unmodified_oracle_passes_the_harness(tmp_path):
    assert _golden_failures(_build(tmp_path, "original", None)) == 0


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_fails_a_golden_case(tmp_path, name):
    assert _golden_failures(_build(tmp_path, name, MUTANTS[name])) > 0, name
