"""The library's host logic under AddressSanitizer and UBSan (CPU only).

tests/c/host_sanitized.cpp is compiled with g++ together with the library's
own host sources (layout.cpp, common.cpp) and -fsanitize=address,undefined
-fno-sanitize-recover=all, so any out-of-bounds access or signed overflow
aborts the run.  It is driven over seeded random layouts (every mode, N up
to 12, empty and ragged tensors, invalid arguments), layouts at sizes where
int64 arithmetic would wrap, and world sizes up to 2^31 - 1; every result is
compared with the oracle's exact integers, and every refusal with the
condition that calls for it.  The alias sweep that guards every written
buffer is compared with a pairwise brute force on random byte ranges, and so
is the index of a plan's buffers that the plan calls check their further
buffers against.
"""

import os
import random
import shutil
import subprocess

import pytest

from oracle import layout as OL

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "rank_step_amd", "csrc")
I64_MAX = (1 << 63) - 1
MODES = {0: OL.FLAT, 1: OL.SHARD0, 2: OL.OWNER}
DT = {0: "f32", 1: "bf16"}
OK, E_ARG, E_DTYPE = 0, -1, -2
VIEW_FIELDS = ("shard_numel", "valid", "global_offset", "view_offset", "view_numel",
               "tensor_offset", "owner")
SUMMARY_FIELDS = ("logical_numel", "physical_numel", "shard_numel", "pad_numel", "bytes_param",
                  "bytes_grad", "bytes_optim", "bytes_master", "bytes_grad_unsharded")

pytestmark = pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")


@pytest.fixture(scope="module")
def exe(tmp_path_factory):
    out = tmp_path_factory.mktemp("san") / "host_sanitized"
    # host-only build with g++ (no device code involved)
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(ROOT, "tests", "c", "host_sanitized.cpp"),
           os.path.join(CSRC, "layout.cpp"), os.path.join(CSRC, "common.cpp"), "-o", str(out)]
    subprocess.run(cmd, check=True, timeout=300)
    return str(out)


def _env():
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "detect_leaks=1:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    return env


def _run_layout(exe, cases):
    text = "\n".join(" ".join(str(x) for x in (m, N, r, hm, len(sh), *[v for s in sh for v in s]))
                     for m, N, r, hm, sh in cases) + "\n"
    p = subprocess.run([exe, "layout"], input=text, capture_output=True, text=True, timeout=600,
                       env=_env())
    assert p.returncode == 0, p.stderr[-4000:]
    lines = p.stdout.splitlines()
    assert len(lines) == len(cases)
    return lines


def _violations(mode, N, rank, shapes):
    """Error codes the documented argument checks call for (empty: valid)."""
    codes = set()
    if mode not in MODES or N < 1 or not 0 <= rank < N:
        codes.add(E_ARG)
    for numel, dim0, dt in shapes:
        if dt not in DT:
            codes.add(E_DTYPE)
        if numel < 0 or dim0 < 0 or (numel > 0 and (dim0 < 1 or numel % dim0)):
            codes.add(E_ARG)
    if mode == 0 and len({dt for _, _, dt in shapes}) > 1:
        codes.add(E_DTYPE)
    if sum(n for n, _, _ in shapes) > I64_MAX:
        codes.add(E_ARG)
    return codes


def _expected(mode, N, rank, has_master, shapes):
    views, summ = OL.layout(MODES[mode], N, rank, [(n, d, DT[t]) for n, d, t in shapes],
                            bool(has_master))
    vals = [getattr(v, f) for v in views for f in VIEW_FIELDS]
    vals += [getattr(summ, f) for f in SUMMARY_FIELDS]
    return vals


def _check(cases, lines, oracle_n=None):
    for case, line in zip(cases, lines):
        mode, N, rank, hm, shapes = case
        got = line.split()
        rc = int(got[0])
        assert "nomessage" not in got, case
        bad = _violations(mode, N, rank, shapes)
        if bad:
            assert rc in bad, (case, rc, bad)
            continue
        n_eff = oracle_n(case) if oracle_n else N
        exp = _expected(mode, n_eff, rank, hm, shapes)
        if max(abs(v) for v in exp) > I64_MAX:
            assert rc == E_ARG, (case, rc)
            continue
        assert rc == OK, (case, rc)
        assert [int(x) for x in got[1:]] == exp, case


def _shape(rnd):
    k = rnd.random()
    if k < 0.1:
        return (0, rnd.choice([0, 1, 5]), 0)
    if k < 0.2:
        return (1, 1, 0)
    dim0 = rnd.randint(1, 40)
    return (dim0 * rnd.randint(0, 300), dim0, 0)


def test_random_layouts(exe):
    rnd = random.Random(7)
    cases = []
    for _ in range(3000):
        mode = rnd.choice([0, 1, 2, 2, 1, 0, 3, -1]) if rnd.random() < 0.05 else rnd.randint(0, 2)
        N = rnd.randint(1, 12) if rnd.random() > 0.03 else rnd.choice([0, -3])
        rank = rnd.randrange(max(N, 1)) if rnd.random() > 0.05 else rnd.choice([-1, N])
        dt = rnd.randint(0, 1)
        shapes = []
        for _ in range(rnd.randint(0, 9)):
            n, d, _ = _shape(rnd)
            t = dt if mode == 0 and rnd.random() > 0.05 else rnd.randint(0, 1)
            if rnd.random() < 0.03:
                n, d = rnd.choice([(-5, 1), (7, 3), (6, 0), (4, -1)])
            if rnd.random() < 0.01:
                t = 7
            shapes.append((n, d, t))
        cases.append((mode, N, rank, rnd.randint(0, 1), shapes))
    _check(cases, _run_layout(exe, cases))


def test_layouts_where_int64_would_wrap(exe):
    big = [1 << 40, (1 << 40) + 1, 1 << 60, (1 << 61) + 3, 1 << 62, I64_MAX // 3, I64_MAX - 7, I64_MAX]
    rnd = random.Random(11)
    cases = []
    for _ in range(600):
        mode = rnd.randint(0, 2)
        # the oracle's OWNER placement scans every rank per parameter: keep N small there
        N = rnd.choice([1, 2, 3, 7, 8, 1000] + ([] if mode == 2 else [1 << 20, (1 << 31) - 1]))
        rank = rnd.choice([0, N - 1, N // 2])
        dt = rnd.randint(0, 1)
        shapes = []
        for _ in range(rnd.randint(1, 4)):
            n = rnd.choice(big)
            d = rnd.choice([1, n]) if n > 0 else 1
            shapes.append((n, d, dt if mode == 0 else rnd.randint(0, 1)))
        cases.append((mode, N, rank, rnd.randint(0, 1), shapes))
    _check(cases, _run_layout(exe, cases))


def test_owner_layout_at_huge_world_sizes(exe):
    """OWNER mode with up to 2^31 - 1 ranks and a handful of parameters.
    With at least as many ranks as parameters, greedy largest-first placement
    only ever uses the first n_tensors ranks (every unused rank has load 0,
    and ties go to the lowest rank), so the oracle runs at min(N, n + 1)
    ranks and ranks past that own nothing."""
    rnd = random.Random(5)
    cases = []
    for _ in range(200):
        N = rnd.choice([(1 << 31) - 1, 1 << 30, 123456789, 1 << 20])
        shapes = [(rnd.choice([0, 1, 4096, 1 << 20]) * rnd.randint(0, 3), 1, rnd.randint(0, 1))
                  for _ in range(rnd.randint(0, 8))]
        shapes = [(n, max(d, 1) if n else d, t) for n, d, t in shapes]
        rank = rnd.choice([0, 1, 2, 5, N - 1])
        cases.append((2, N, rank, rnd.randint(0, 1), shapes))
    lines = _run_layout(exe, cases)

    def small_n(case):
        return min(case[1], len(case[4]) + 1)

    near = [(c, ln) for c, ln in zip(cases, lines) if c[2] < small_n(c)]
    far = [(c, ln) for c, ln in zip(cases, lines) if c[2] >= small_n(c)]
    _check([c for c, _ in near], [ln for _, ln in near], oracle_n=small_n)
    for (mode, N, rank, hm, shapes), line in far:
        vals = [int(x) for x in line.split()]
        assert vals[0] == OK
        views = [vals[1 + 7 * i:8 + 7 * i] for i in range(len(shapes))]
        assert all(v[0] == 0 and v[1] == 0 and v[4] == 0 for v in views)
        assert all(0 <= v[6] < len(shapes) for v in views)


def test_alias_sweep_matches_brute_force(exe):
    p = subprocess.run([exe, "alias", "12345", "200000"], capture_output=True, text=True,
                       timeout=600, env=_env())
    assert p.returncode == 0, p.stderr[-4000:]
    cases, mismatches = (int(x) for x in p.stdout.split())
    assert cases == 200000 and mismatches == 0


def test_plan_footprint_matches_brute_force(exe):
    p = subprocess.run([exe, "footprint", "777", "50000"], capture_output=True, text=True,
                       timeout=600, env=_env())
    assert p.returncode == 0, p.stderr[-4000:]
    cases, queries, mismatches = (int(x) for x in p.stdout.split())
    assert cases == 50000 and queries == 32 * 50000 and mismatches == 0
