"""Mutation testing of the oracle's pins (CPU only).

Each mutant is a copy of the oracle with one plausible mistake planted in it
(a dropped term, a wrong sign or index, a transposed operand, or one of the
pitfalls the pages list).  The pin suite tests/test_oracle_pins.py is rerun
against the copy in a subprocess and must fail.  A mutant whose text no
longer matches the oracle source fails this test too, so the list follows
edits of the oracle.
"""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
C_SRC = os.path.join(ROOT, "oracle", "ref_attn.c")
PY_SRC = os.path.join(ROOT, "oracle", "online.py")
PINS = os.path.join(ROOT, "tests", "test_oracle_pins.py")

C_MUTANTS = {
    "no_max_subtraction": [("l += exp(s[j] - m);", "l += exp(s[j]);"),
                           ("double a = exp(s[j] - m) / l;", "double a = exp(s[j]) / l;"),
                           ("*lse = m + log(l);", "*lse = log(l);")],
    "wrong_sign_in_weight": [("double a = exp(s[j] - m) / l;", "double a = exp(m - s[j]) / l;")],
    "dropped_scale": [("s[j] = scale * dot;", "s[j] = dot;")],
    "transposed_k": [("dot += (double)qi[c] * (double)kj[c];",
                      "dot += (double)qi[c] * (double)kb[c * Nk + j];")],
    "causal_off_by_one": [("(!causal || j <= i)", "(!causal || j < i)")],
    "lse_without_max": [("*lse = m + log(l);", "*lse = log(l);")],
    "mask_ignored": [("(!mask || mask[b * Nk + j])", "(1)")],
    "masked_row_lse_zero": [("*lse = -INFINITY;", "*lse = 0.0;")],
    "value_row_reversed": [("const float *vj = v + j * ldv;",
                            "const float *vj = v + (n - 1 - j) * ldv;")],
    "max_skips_last_key": [("        if (s[j] > m) m = s[j];",
                            "        if (s[j] > m && j + 1 < n) m = s[j];")],
    "no_normalisation": [("double a = exp(s[j] - m) / l;", "double a = exp(s[j] - m);")],
}

PY_MUTANTS = {
    "rescale_only_l": [("o_t = alpha * o_t + p @ v[lo:hi]", "o_t = o_t + p @ v[lo:hi]")],
    "finite_m_init": [("    m = -math.inf\n    l = 0.0", "    m = 0.0\n    l = 0.0")],
    "local_block_max": [("p = np.array([_exp(x - m_new) for x in s_blk])",
                         "p = np.array([_exp(x - m_blk) for x in s_blk])")],
    "normalise_per_block": [("o_t = alpha * o_t + p @ v[lo:hi]",
                             "o_t = (alpha * o_t + p @ v[lo:hi]) / l")],
    "mask_after_block_max": [("        s[~vis] = -math.inf\n", "")],
    "alpha_sign": [("alpha = _exp(m - m_new)", "alpha = _exp(m_new - m)")],
    "merge_l_not_rescaled": [('l += alpha * st["l"]', 'l += st["l"]')],
    "merge_o_not_rescaled": [('o_t = o_t + alpha * np.asarray(st["o_tilde"], dtype=np.float64)',
                              'o_t = o_t + np.asarray(st["o_tilde"], dtype=np.float64)')],
    "merge_base_is_min": [('big_m = max(st["m"] for st in states)',
                           'big_m = min(st["m"] for st in states)')],
    "merge_alpha_sign": [('alpha = _exp(st["m"] - big_m)', 'alpha = _exp(big_m - st["m"])')],
    "partial_state_unshifted": [("np.exp(np.where(vis, s - m, 0.0))", "np.exp(np.where(vis, s, 0.0))")],
}


def _mutate(src, edits):
    for old, new in edits:
        assert src.count(old) == 1, "mutation text not found once: %r" % old
        src = src.replace(old, new)
    return src


def _run_pins(env_extra):
    env = dict(os.environ)
    env.update(env_extra)
    r = subprocess.run([sys.executable, "-m", "pytest", PINS, "-x", "-q", "-p", "no:cacheprovider"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    return r.returncode, r.stdout[-2000:]


@pytest.mark.parametrize("name", sorted(C_MUTANTS))
def test_c_oracle_mutant_is_caught(name, tmp_path):
    src = _mutate(open(C_SRC).read(), C_MUTANTS[name])
    path = tmp_path / "mutant.c"
    path.write_text(src)
    lib = tmp_path / "libmutant.so"
    subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-o", str(lib), str(path), "-lm"],
                   check=True)
    rc, out = _run_pins({"FA_TEST_MUTANT_ORACLE_LIB": str(lib)})
    assert rc != 0, "pins did not catch C mutant %s:\n%s" % (name, out)


@pytest.mark.parametrize("name", sorted(PY_MUTANTS))
def test_online_mutant_is_caught(name, tmp_path):
    src = _mutate(open(PY_SRC).read(), PY_MUTANTS[name])
    if name == "mask_after_block_max":
        # mask applied to the weights after the maximum was taken
        src = _mutate(src, [("            p = np.array([_exp(x - m_new) for x in s_blk])\n",
                             "            p = np.array([_exp(x - m_new) for x in s_blk])\n"
                             "            if visible is not None:\n"
                             "                p = p * vis[lo:hi]\n")])
    path = tmp_path / "online_mutant.py"
    path.write_text(src)
    rc, out = _run_pins({"FA_TEST_MUTANT_ONLINE_SRC": str(path)})
    assert rc != 0, "pins did not catch online mutant %s:\n%s" % (name, out)


def test_unmutated_copies_pass(tmp_path):
    """The harness itself: unmodified copies of both files pass the pins."""
    lib = tmp_path / "libcopy.so"
    subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-o", str(lib), C_SRC, "-lm"],
                   check=True)
    path = tmp_path / "online_copy.py"
    path.write_text(open(PY_SRC).read())
    rc, out = _run_pins({"FA_TEST_MUTANT_ORACLE_LIB": str(lib),
                         "FA_TEST_MUTANT_ONLINE_SRC": str(path)})
    assert rc == 0, out
