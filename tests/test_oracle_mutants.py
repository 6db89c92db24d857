"""Planted mistakes in the oracle, on the CPU: each mutant of ``oracle/oracle.c``
(a dropped term, a wrong sign, a transposed operand, a wrong index, a wrong
rounding, a wrong grouping order) is compiled with the oracle's own flags,
loaded in place of the real library, and run through the oracle's pins.  At
least one pin must reject every mutant: the pins pin the oracle, they do not
merely agree with it.  Every mutant keeps its memory accesses inside the
arrays the real code touches, so a mutant can only give wrong numbers."""
import os
import subprocess

import pytest

import oracle
import test_oracle_pins as P
from oracle import build as obuild

# (name, text in oracle.c, replacement)
MUTANTS = [
    ("drop the scale alpha/r", "y = yb + s * acc;", "y = yb + acc;"),
    ("subtract the update", "y = yb + s * acc;", "y = yb - s * acc;"),
    ("scale r/alpha", "alpha[a] / (float)r", "(float)r / alpha[a]"),
    ("B page read rank-rows (transposed)",
     "(int64_t)((k % 16) / 8) * 8 * tb->pw + (int64_t)(j % tb->pw) * 8 +\n                (k % 8)",
     "(int64_t)(k % 16) * tb->pw + (j % tb->pw)"),
    ("B page read as 16 contiguous ranks per column",
     "(int64_t)((k % 16) / 8) * 8 * tb->pw + (int64_t)(j % tb->pw) * 8 +\n                (k % 8)",
     "(int64_t)(j % tb->pw) * 16 + (k % 16)"),
    ("A page read column-major (transposed)", "(int64_t)(k % 16) * tb->pw + (i % tb->pw)",
     "(int64_t)(i % 16) * tb->pw + (k % tb->pw)"),
    ("B column page ignored", "(k / 16) * ncol + j / tb->pw;", "(k / 16) * ncol;"),
    ("expand drops the last rank", "for (int32_t k = 0; k < r; ++k) {\n          float w = 0.0f;",
     "for (int32_t k = 0; k < r - 1; ++k) {\n          float w = 0.0f;"),
    ("shrink reads X reversed", "load_elem(X, dtype, (int64_t)t * ldx + i)",
     "load_elem(X, dtype, (int64_t)t * ldx + (tb->d_in - 1 - i))"),
    ("bf16 by truncation", "if (rest > 0x8000u || (rest == 0x8000u && (keep & 1u))) keep += 1u;", ""),
    ("bf16 ties away from zero", "(rest == 0x8000u && (keep & 1u))", "(rest == 0x8000u)"),
    ("segments in descending adapter id", "for (int32_t a = 0; a < N; ++a) {\n    int32_t cnt = 0;",
     "for (int32_t a = N - 1; a >= 0; --a) {\n    int32_t cnt = 0;"),
    # V_total (which sizes v) stays right, the segment offsets come out low,
    # so every write lands at or below its true position
    ("v offsets short by the token count", "v_indptr[S + 1] = (int32_t)v;", "v_indptr[S + 1] = (int32_t)(v - cnt);"),
    ("base-only tokens counted invalid", "if (ids[t] != -1) ++n_invalid;", "++n_invalid;"),
]


def _pins():
    return [
        ("segments vs stable sort", lambda: [P.test_segments_match_stable_sort(s) for s in range(3)]),
        ("page gather round trip", lambda: P.test_page_gather_round_trip(2, {})),
        ("bf16 rounding vs library cast", P.test_bf16_rounding_matches_library_cast),
        ("merge identity (float64)", P.test_merge_identity_float64),
        ("per-adapter brute force (float64)", lambda: P.test_brute_force_per_adapter(2, {"dtype": "f32"}, 1e-5)),
        ("shrink vs float64", P.test_shrink_matches_float64),
        ("one-hot closed form", P.test_one_hot_closed_form_exact),
        ("alpha = r unscaled form", P.test_alpha_equals_rank_is_unscaled_form),
        ("base-only and invalid tokens", P.test_base_only_and_invalid_tokens_keep_base),
    ]


@pytest.fixture(scope="module")
def source():
    with open(obuild.SRC) as f:
        return f.read()


def _compile(src_text, out_dir, name):
    src = os.path.join(out_dir, f"{name}.c")
    lib = os.path.join(out_dir, f"{name}.so")
    with open(src, "w") as f:
        f.write(src_text)
    subprocess.run(["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC",
                    "-shared", "-o", lib, src], check=True, capture_output=True)
    return lib


@pytest.mark.parametrize("i", range(len(MUTANTS)), ids=[m[0] for m in MUTANTS])
def test_pins_reject_planted_mistake(i, source, tmp_path, monkeypatch):
    name, old, new = MUTANTS[i]
    assert source.count(old) == 1, f"mutation site not unique: {name}"
    lib = _compile(source.replace(old, new), str(tmp_path), f"mutant{i}")
    monkeypatch.setattr(oracle, "LIB_PATH", lib)
    monkeypatch.setattr(oracle, "_lib", None)
    caught = []
    for pin, fn in _pins():
        try:
            fn()
        except (AssertionError, ValueError):
            caught.append(pin)
    monkeypatch.setattr(oracle, "_lib", None)
    print(f"{name}: rejected by {caught}")
    assert caught, f"no pin rejects the mutant '{name}'"


def test_unmutated_copy_passes_every_pin(source, tmp_path, monkeypatch):
    """The harness itself: the same compile of the unchanged source passes."""
    lib = _compile(source, str(tmp_path), "same")
    monkeypatch.setattr(oracle, "LIB_PATH", lib)
    monkeypatch.setattr(oracle, "_lib", None)
    for _, fn in _pins():
        fn()
    monkeypatch.setattr(oracle, "_lib", None)
