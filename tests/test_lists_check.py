"""The host-side work-list validator (backlite_check_lists) on the CPU: lists
the oracle derives from masks pass; each kind of malformed list is rejected
with its reason; and the validator's source, built on its own with the address
and undefined-behaviour sanitizers, runs the same cases clean."""
import os
import shutil
import subprocess

import numpy as np
import pytest

from oracle import backlite_oracle as orc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "block_sparse_attention_fa_amd", "csrc", "lists_check.cpp")
DRIVER = os.path.join(ROOT, "tests", "native", "lists_check_driver.cpp")


@pytest.fixture(scope="module")
def lib():
    from block_sparse_attention_fa_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("libbacklite.so is not built (run __graft_entry__.build())")
    return _lib


def _lists(n, causal, window, seed, H=3, negl=0.3):
    """A mask the oracle selects on random inputs, and its lists."""
    g = np.random.default_rng(seed)
    q, k, v = (g.standard_normal((1, n, H, 16)) * 2 for _ in range(3))
    f = orc.forward(q, k, v, causal=causal, window=window)
    keep = orc.mask_from_stats(f["tile_lse"], f["lse"], n, causal, negl, window=window)
    return [np.ascontiguousarray(a) for a in orc.lists_from_keep(keep)]


CASES = [(1000, False, 0), (777, True, 0), (900, True, 300)]


@pytest.mark.parametrize("n,causal,window", CASES)
def test_valid_lists_pass(lib, n, causal, window):
    qc, qi, kc, ki = _lists(n, causal, window, 1)
    lib.check_lists(qc, qi, kc, ki, 1, 3, n, causal, window)


def _mutations(qc, qi, kc, ki, T, causal):
    """(name, lists) pairs, each with one defect of a kind the validator names."""
    out = []
    h = 1
    qt = int(np.argmax(qc[0, h]))
    a = [x.copy() for x in (qc, qi, kc, ki)]
    a[0][0, h, qt] = T + 1
    out.append(("count", a))
    a = [x.copy() for x in (qc, qi, kc, ki)]
    a[0][0, h, qt] = -1
    out.append(("count", a))
    a = [x.copy() for x in (qc, qi, kc, ki)]
    a[1][0, h, qt, 0] = T
    out.append(("not a key tile", a))
    if qc[0, h, qt] >= 2:
        a = [x.copy() for x in (qc, qi, kc, ki)]
        a[1][0, h, qt, 1] = a[1][0, h, qt, 0]
        out.append(("ascending", a))
    kt = int(np.argmax(kc[0, h]))
    a = [x.copy() for x in (qc, qi, kc, ki)]
    a[3][0, h, kt, 0] = T + 3
    out.append(("not a query tile", a))
    a = [x.copy() for x in (qc, qi, kc, ki)]
    a[2][0, h, kt] -= 1            # one pair fewer on the k side
    out.append(("pairs", a))
    if causal:
        # a key tile above the diagonal appended to query tile 0's list
        a = [x.copy() for x in (qc, qi, kc, ki)]
        c = a[0][0, h, 0]
        a[1][0, h, 0, c] = T - 1
        a[0][0, h, 0] = c + 1
        out.append(("causal", a))
    return out


@pytest.mark.parametrize("n,causal,window", CASES)
def test_malformed_lists_rejected(lib, n, causal, window):
    qc, qi, kc, ki = _lists(n, causal, window, 2)
    T = orc.ntiles(n)
    reason = {"count": "outside", "causal": "causal diagonal"}
    for what, (a, b, c, d) in _mutations(qc, qi, kc, ki, T, causal):
        with pytest.raises(lib.BackliteError, match=reason.get(what, what)):
            lib.check_lists(a, b, c, d, 1, 3, n, causal, window)


def test_window_violation_rejected(lib):
    n, w = 900, 300
    qc, qi, kc, ki = _lists(n, True, w, 3)
    # query tile 6 (rows 768-899) may not reach key tile 0 (keys 0-127) under a 300-key window
    qt = 6
    assert 0 not in qi[0, 0, qt, :qc[0, 0, qt]]
    qi2, qc2 = qi.copy(), qc.copy()
    row = sorted([0] + list(qi[0, 0, qt, :qc[0, 0, qt]]))
    qi2[0, 0, qt, :len(row)] = row
    qc2[0, 0, qt] = len(row)
    with pytest.raises(lib.BackliteError, match="window"):
        lib.check_lists(qc2, qi2, kc, ki, 1, 3, n, True, w)


def _write_case_files(tmp, cases):
    """Binary case files for the sanitizer driver: header + the four arrays."""
    paths = []
    for i, (B, H, n, causal, window, expect_ok, (qc, qi, kc, ki)) in enumerate(cases):
        p = os.path.join(tmp, f"case{i}.bin")
        with open(p, "wb") as fh:
            np.array([B, H, n, int(causal), window, int(expect_ok)], np.int32).tofile(fh)
            qc.astype(np.int32).tofile(fh)
            qi.view(np.uint16).tofile(fh)
            kc.astype(np.int32).tofile(fh)
            ki.view(np.uint16).tofile(fh)
        paths.append(p)
    return paths


def test_validator_under_address_and_ub_sanitizers(tmp_path):
    """Build lists_check.cpp with a small driver under -fsanitize=address,
    undefined (host code only, plain g++) and run valid and malformed cases:
    the verdicts must match and the sanitizers must stay silent."""
    cxx = shutil.which("g++")
    if cxx is None:
        pytest.skip("no g++")
    exe = str(tmp_path / "lists_check_asan")
    cmd = [cxx, "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", f"-I{os.path.join(ROOT, 'include')}", SRC, DRIVER, "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0 and "sanitize" in r.stderr and "cannot find" in r.stderr:
        pytest.skip("sanitizer runtime not installed")
    assert r.returncode == 0, r.stderr
    cases = []
    for n, causal, window in CASES:
        qc, qi, kc, ki = _lists(n, causal, window, 4)
        cases.append((1, 3, n, causal, window, True, (qc, qi, kc, ki)))
        for _, arrs in _mutations(qc, qi, kc, ki, orc.ntiles(n), causal):
            cases.append((1, 3, n, causal, window, False, tuple(arrs)))
    paths = _write_case_files(str(tmp_path), cases)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe, *paths], capture_output=True, text=True, env=env)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "ERROR" not in r.stderr and "runtime error" not in r.stderr, r.stderr
    assert r.stdout.count("ok") == len(paths), r.stdout
