"""Mutation check of the oracle's pins (CPU only).

Each case plants one plausible mistake in a temporary copy of the oracle (a
dropped or flipped term, a wrong index, a transposed operand, the wrong
comparison, the wrong array) and runs the oracle's pin tests against that
copy; every mistake must make at least one pin fail.  The repository's own
oracle is never modified: the copy, with the pin tests, their fixtures and
the input generators, lives in a temporary directory.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

PIN_TESTS = ["test_oracle_her.py", "test_oracle_iql.py", "test_oracle_aw_budget.py", "test_oracle_philox_bf16.py",
             "test_oracle_per.py", "test_oracle_sentinel.py", "test_oracle_conditioning.py"]

# (file, original text, mistake)
MUTATIONS = [
    ("iql.py", "dz1 = R(dh1 * (z1 > 0.0))", "dz1 = R(dh1 * (z1 >= -1e-3))"),                  # relu' of the wrong side
    ("iql.py", "dv = -2.0 * w * diff / B", "dv = 2.0 * w * diff / B"),                          # sign of dL/dV
    ("iql.py", "w = np.where(diff >= 0.0, tau, 1.0 - tau)", "w = np.where(diff >= 0.0, 1.0 - tau, tau)"),
    ("iql.py", 'g["w1"] = dz1.T @ X', 'g["w1"] = dz1.T @ np.abs(X)'),
    ("iql.py", 'dh1 = dz2 @ R(p["w2"])', 'dh1 = dz2 @ R(p["w2"]).T[:dz2.shape[1], :]'),       # transposed W2
    ("iql.py", "m_hat = m_new / (1.0 - hp.beta1 ** t)", "m_hat = m_new"),                     # no bias correction
    ("iql.py", 'g["b2"] = dz2.sum(axis=0)', 'g["b2"] = dz2.mean(axis=0)'),
    ("iql.py", "w2 = flat[o:o + H2 * H1].reshape(H2, H1)", "w2 = flat[o:o + H2 * H1].reshape(H1, H2).T"),
    ("iql.py", "return r + gamma * (1.0 - d) * np.asarray(v_next, dtype=np.float64)",
     "return r + gamma * np.asarray(v_next, dtype=np.float64)"),                               # terminal rows
    ("iql.py", "return (1.0 - tau) * np.asarray(target, dtype=np.float64) + tau * np.asarray(online, dtype=np.float64)",
     "return tau * np.asarray(target, dtype=np.float64) + (1.0 - tau) * np.asarray(online, dtype=np.float64)"),
    ("her.py", "goal = np.asarray(next_states[don, :G], dtype=np.float32)",
     "goal = np.asarray(states[don, :G], dtype=np.float32)"),                                  # s instead of s'
    ("her.py", "out_ns[:, :G] = goal", "pass"),
    ("her.py", "return end - 1", "return end"),
    ("her.py", "hit = dist < np.float32(threshold)", "hit = dist <= np.float32(threshold)"),
    ("her.py", "dist = np.sqrt(acc).astype(np.float32)", "dist = acc"),                       # squared distance
    ("her.py", "return np.where(span > 0, pick, src)", "return np.where(span > 0, pick, src + 1)"),
    ("her.py", "return np.concatenate([w, np.ones(int(n_her), dtype=np.float32)])",
     "return np.concatenate([np.ones(int(n_her), dtype=np.float32), w])"),                   # HER rows first
    ("aw.py", "x = beta * np.clip(Q - V[:, None], -CLAMP, CLAMP)",
     "x = np.clip(beta * (Q - V[:, None]), -CLAMP, CLAMP)"),                                  # clamp after beta
    ("budget.py", "if norm > budget and norm > 0.0:", "if norm > 1.0 and norm > 0.0:"),
    ("philox.py", "c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0",
     "c0, c1, c2, c3 = hi0 ^ c1 ^ k0, lo1, hi1 ^ c3 ^ k1, lo0"),                              # swapped words
    ("bf16.py", "lsb = (bits >> np.uint64(16)) & np.uint64(1)", "lsb = np.uint64(0)"),        # truncation-ish rounding
    ("per.py", 'return np.searchsorted(prefix, u, side="right")', 'return np.searchsorted(prefix, u, side="left")'),
    ("per.py", "w = (pi.min() / pi) ** beta", "w = (pi / pi.max()) ** beta"),
    ("sentinel.py", "return (b & np.uint32(0x7F800000)) == np.uint32(0x7F800000)",
     "return (b & np.uint32(0x7FFFFFFF)) > np.uint32(0x7F800000)"),                           # NaN only
]


def _copy_tree(dst):
    shutil.copytree(os.path.join(ROOT, "oracle"), os.path.join(dst, "oracle"),
                    ignore=shutil.ignore_patterns("__pycache__"))
    shutil.copytree(os.path.join(ROOT, "synth"), os.path.join(dst, "synth"),
                    ignore=shutil.ignore_patterns("__pycache__"))
    os.makedirs(os.path.join(dst, "tests"))
    for f in PIN_TESTS + ["conftest.py"]:
        shutil.copy(os.path.join(ROOT, "tests", f), os.path.join(dst, "tests", f))
    shutil.copytree(os.path.join(ROOT, "tests", "golden"), os.path.join(dst, "tests", "golden"))
    with open(os.path.join(dst, "pytest.ini"), "w") as fh:
        fh.write("[pytest]\ntestpaths = tests\naddopts = -p no:cacheprovider\n")


def _pins_fail(tree):
    env = dict(os.environ, PYTHONDONTWRITEBYTECODE="1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-m", "not gpu", *["tests/" + f for f in PIN_TESTS]],
                       cwd=tree, capture_output=True, text=True, env=env, timeout=600)
    return r.returncode != 0, r.stdout[-2000:]


@pytest.fixture(scope="module")
def tree(tmp_path_factory):
    d = str(tmp_path_factory.mktemp("oracle_copy"))
    _copy_tree(d)
    failed, out = _pins_fail(d)
    assert not failed, "the unmodified copy must pass its pins:\n" + out
    return d


@pytest.mark.parametrize("fname,orig,mistake", MUTATIONS, ids=[f"{m[0]}:{i}" for i, m in enumerate(MUTATIONS)])
def test_every_planted_mistake_fails_a_pin(tree, fname, orig, mistake):
    path = os.path.join(tree, "oracle", fname)
    with open(path) as fh:
        src = fh.read()
    assert src.count(orig) == 1, f"anchor not found once in {fname}: {orig}"
    with open(path, "w") as fh:
        fh.write(src.replace(orig, mistake))
    try:
        failed, out = _pins_fail(tree)
    finally:
        with open(path, "w") as fh:
            fh.write(src)
    assert failed, f"no pin caught {fname}: {mistake}\n{out}"
