"""Mutation harness for the oracle's pins (CPU only).

Each case plants one plausible mistake in a scratch copy of ``oracle/`` (a
dropped term, a flipped sign, an off-by-one mask, a wrong head or position
index, a transposed operand) and runs the pin tests against that copy in a
child process.  The pins must fail on every mutant; an unmutated copy must
pass, so a failure here cannot come from the harness itself.

The mutants run four at a time from one session fixture; each case then
reports the outcome of its own mutant.
"""
import concurrent.futures
import os
import shutil
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

PIN_FILES = ["test_oracle_rope.py", "test_oracle_ntk.py", "test_oracle_attention.py",
             "test_oracle_cache_window.py", "test_oracle_mask.py", "test_oracle_fused.py"]

# (name, file under oracle/, text to find, replacement, which occurrence (1-based)).
# Left out as equivalent (no input tells them apart): the dynamic NTK test
# ``seq_len < max_position`` (alpha is exactly 1 at seq_len == max_position) and
# dropping the upper clamp of kv_len (a numpy slice past the end stops there).
MUTANTS = [
    # rope: frequencies, angles, pairing, position scaling
    ("inv_freq_sign", "rope.py", "-2.0 * i / np.float64(head_dim)", "2.0 * i / np.float64(head_dim)", 1),
    ("inv_freq_no_two", "rope.py", "-2.0 * i / np.float64(head_dim)", "-1.0 * i / np.float64(head_dim)", 1),
    ("inv_freq_base_d_minus_2", "rope.py", "-2.0 * i / np.float64(head_dim)", "-2.0 * i / np.float64(head_dim - 2)", 1),
    ("linear_factor_multiplies", "rope.py", "/ np.float64(linear_factor)", "* np.float64(linear_factor)", 1),
    ("half_first_sign", "rope.py", "x1 * c - x2 * s", "x1 * c + x2 * s", 1),
    ("half_second_sign", "rope.py", "x2 * c + x1 * s", "x2 * c - x1 * s", 1),
    ("half_sin_cos_swapped", "rope.py", "x2 * c + x1 * s", "x2 * s + x1 * c", 1),
    ("interleaved_sign", "rope.py", "x1 * c - x2 * s", "x1 * c + x2 * s", 2),
    ("interleaved_pairs_swapped", "rope.py", "x[..., 0::2], x[..., 1::2]", "x[..., 1::2], x[..., 0::2]", 1),
    ("half_split_off_by_one", "rope.py", "x[..., : D // 2], x[..., D // 2:]", "x[..., : D // 2], np.roll(x[..., D // 2:], 1, axis=-1)", 1),
    ("k_not_rotated", "rope.py", "rotate(k, pos, theta, linear_factor, style))", "k)", 1),
    ("default_positions_from_one", "rope.py", "np.arange(S)", "np.arange(1, S + 1)", 1),
    # ntk
    ("ntk_exponent_inverted", "ntk.py", "np.float64(D) / np.float64(D - 2)", "np.float64(D - 2) / np.float64(D)", 1),
    ("ntk_dynamic_offset", "ntk.py", "- (np.float64(factor) - 1.0)", "- np.float64(factor)", 1),
    ("ntk_dynamic_alpha_is_factor", "ntk.py", "alpha = np.float64(factor) * np.float64(seq_len) / np.float64(max_position) - (np.float64(factor) - 1.0)",
     "alpha = np.float64(factor)", 1),
    # attention: scale, masks, softmax, head map, caches
    ("scale_dropped", "attention.py", "np.float64(scale) * (qh @ kh.T)", "(qh @ kh.T)", 1),
    ("scale_squared", "attention.py", "np.float64(scale) * (qh @ kh.T)", "np.float64(scale) ** 2 * (qh @ kh.T)", 1),
    ("scores_transposed", "attention.py", "np.float64(scale) * (qh @ kh.T)", "np.float64(scale) * (kh @ qh.T)", 1),
    ("causal_excludes_diagonal", "attention.py", "j > pos, -np.inf", "j >= pos, -np.inf", 1),
    ("causal_top_left", "attention.py", "np.arange(Sq)[:, None] + (Sk - Sq)", "np.arange(Sq)[:, None]", 1),
    ("window_off_by_one", "attention.py", "j <= pos - window", "j < pos - window", 1),
    ("softmax_not_normalised", "attention.py", "return p / tot", "return p", 1),
    ("softmax_dead_rows_nan", "attention.py", "tot = np.where(dead, 1.0, tot)", "tot = np.where(dead, 0.0, tot)", 1),
    ("gqa_modulo_map", "attention.py", "kh = h // G\n        s = _scores", "kh = h % Hkv\n        s = _scores", 1),
    ("mask_ignored", "attention.py", "s = s + mask[b, h if mask.shape[1] > 1 else 0]", "s = s", 1),
    ("mask_head_zero", "attention.py", "mask[b, h if mask.shape[1] > 1 else 0]", "mask[b, 0]", 1),
    ("mask_transposed", "attention.py", "mask[b, h if mask.shape[1] > 1 else 0]", "mask[b, h if mask.shape[1] > 1 else 0].T", 1),
    ("cache_len_ignored", "attention.py", "kk = np.asarray(k_cache[b, kh, :L, :]", "kk = np.asarray(k_cache[b, kh, :, :]", 1),
    ("cache_v_from_k", "attention.py", "vv = np.asarray(v_cache[b, kh, :L, :]", "vv = np.asarray(k_cache[b, kh, :L, :]", 1),
    ("cache_empty_rows_nan", "attention.py", "out[b, :, h, :] = 0.0", "out[b, :, h, :] = np.nan", 1),
    ("decode_len_off_by_one", "attention.py", "kk = np.asarray(k_cache[b, kh, :L, :]", "kk = np.asarray(k_cache[b, kh, :max(L - 1, 1), :]", 2),
    ("decode_group_slice", "attention.py", "qg = q[b, kh * G:(kh + 1) * G, :]", "qg = q[b, kh::Hkv, :]", 1),
    ("decode_negative_len", "attention.py", "L = int(min(max(int(kv_lens[b]), 0), max_kv))\n        if L == 0:\n            continue",
     "L = int(min(int(kv_lens[b]), max_kv))\n        if L == 0:\n            continue", 1),
    ("cache_negative_len", "attention.py", "L = int(min(max(int(kv_lens[b]), 0), max_kv))\n        kh",
     "L = int(min(int(kv_lens[b]), max_kv))\n        kh", 1),
    ("append_v_gets_k", "attention.py", "vc[b, :, s, :] = v_new[b]", "vc[b, :, s, :] = k_new[b]", 1),
    ("append_out_of_range_wraps", "attention.py", "if 0 <= s < kc.shape[2]:", "if s < kc.shape[2]:", 1),
    # fused
    ("fused_k_unrotated", "fused.py", "attention(q_rot, k_rot,", "attention(q_rot, np.asarray(k, dtype=np.float64),", 1),
    ("fused_decode_position_is_len", "fused.py", "pos = slots if", "pos = kv_lens if", 1),
    ("fused_decode_k_unrotated", "fused.py", "kv_append(k_cache, v_cache, k_rot,", "kv_append(k_cache, v_cache, np.asarray(k_new, dtype=np.float64),", 1),
]


def _plant(tree, fname, old, new, nth):
    path = os.path.join(tree, "oracle", fname)
    with open(path, encoding="utf-8") as f:
        src = f.read()
    at = -1
    for _ in range(nth):
        at = src.find(old, at + 1)
        if at < 0:
            raise AssertionError(f"mutation site {old!r} (occurrence {nth}) no longer in oracle/{fname}")
    with open(path, "w", encoding="utf-8") as f:
        f.write(src[:at] + new + src[at + len(old):])


def _run(case, base):
    """Copy the oracle and its pins to a scratch tree, plant the mistake and
    run the pins there; returns (case name, pytest exit code, output tail)."""
    name, fname, old, new, nth = case
    tree = os.path.join(base, name)
    shutil.copytree(os.path.join(ROOT, "oracle"), os.path.join(tree, "oracle"),
                    ignore=shutil.ignore_patterns("__pycache__"))
    os.makedirs(os.path.join(tree, "tests"))
    shutil.copytree(os.path.join(ROOT, "tests", "golden"), os.path.join(tree, "tests", "golden"))
    for f in ["conftest.py"] + PIN_FILES:
        shutil.copy(os.path.join(ROOT, "tests", f), os.path.join(tree, "tests", f))
    with open(os.path.join(tree, "pytest.ini"), "w") as f:
        f.write("[pytest]\ntestpaths = tests\n")
    if fname is not None:
        _plant(tree, fname, old, new, nth)
    env = dict(os.environ, PYTHONDONTWRITEBYTECODE="1", OMP_NUM_THREADS="1")
    env.pop("PYTHONPATH", None)
    p = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", "tests"],
                       cwd=tree, env=env, capture_output=True, text=True, timeout=300)
    return name, p.returncode, (p.stdout + p.stderr)[-1500:]


@pytest.fixture(scope="module")
def outcomes():
    cases = [("unmutated", None, None, None, 0)] + MUTANTS
    with tempfile.TemporaryDirectory(prefix="oracle_mutants_") as base:
        with concurrent.futures.ThreadPoolExecutor(max_workers=4) as ex:
            results = list(ex.map(lambda c: _run(c, base), cases))
    return {name: (rc, tail) for name, rc, tail in results}


def test_unmutated_copy_passes(outcomes):
    rc, tail = outcomes["unmutated"]
    assert rc == 0, tail


@pytest.mark.parametrize("name", [m[0] for m in MUTANTS])
def test_pins_catch_mutant(outcomes, name):
    rc, tail = outcomes[name]
    # exit code 1: tests ran and at least one failed (not a collection or usage error)
    assert rc == 1, f"mutant {name} not caught (pytest exit {rc}):\n{tail}"


def test_mutant_names_unique():
    names = [m[0] for m in MUTANTS]
    assert len(names) == len(set(names))
