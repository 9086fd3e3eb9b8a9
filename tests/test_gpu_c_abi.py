"""The whole path from plain C on the GPU: tests/c/step_from_c (built by
__graft_entry__.build()) allocates with the HIP runtime, runs one fused
multi-tensor step through the C ABI and writes its inputs and outputs.  No
PyTorch is involved in the step.  The outputs must match the oracle to the
parity bar and the kernel's stated fp32 sequence bit for bit, with +0 in the
padding whatever the inputs hold there.  tests/c/graph_from_c captures
fsdp_mt_step_capturable in a HIP graph from C and checks every replay
against fixed-count eager steps bit for bit (it reports the result itself)."""

import os
import subprocess

import numpy as np
import pytest

from oracle import step as O
from rank_step_amd.workloads import HPARAMS
from tests import parity as PR

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
EXE = os.path.join(ROOT, "tests", "c", "step_from_c")
NS = 8


def test_step_from_plain_c(gpu, tmp_path):
    assert os.path.exists(EXE), "tests/c/step_from_c is missing: run __graft_entry__.build() first"
    out = tmp_path / "step.bin"
    subprocess.run([EXE, str(out)], check=True, timeout=120)
    raw = out.read_bytes()
    pos = 0

    def take(dtype, n):
        nonlocal pos
        a = np.frombuffer(raw, dtype=dtype, count=n, offset=pos)
        pos += a.nbytes
        return a

    hp = dict(HPARAMS)
    for i in range(3):
        S, va = (int(x) for x in take(np.int64, 2))
        sl_bits = take(np.uint16, NS * S).reshape(NS, S)
        p0, m0, v0 = (take(np.float32, S) for _ in range(3))
        p1, m1, v1 = (take(np.float32, S) for _ in range(3))
        b1 = take(np.uint16, S)
        sl = O.widen_bf16_bits(sl_bits)
        ref = O.rank_step(p0.astype(np.float64), m0.astype(np.float64), v0.astype(np.float64), sl, va, 1, hp)
        fl = PR.floors(p0[:va].astype(np.float64), m0[:va].astype(np.float64), v0[:va].astype(np.float64),
                       sl[:, :va], {k: r[:va] for k, r in ref.items()}, hp, 1)
        for nm, got in (("p", p1), ("m", m1), ("v", v1)):
            PR.assert_close(f"C shard {i} {nm}", got[:va], ref[nm][:va], fl[nm])
            PR.check_pad_zero(f"C shard {i} {nm}", got, va)
        PR.check_bf16(f"C shard {i} bf16", b1[:va], p1[:va], ref["p"][:va], fl["p"])
        PR.check_pad_zero(f"C shard {i} bf16", b1, va)
        rp, rm, rv = PR.fp32_replica_step(p0, m0, v0, sl, va, 1, hp)
        for nm, got, want in (("p", p1, rp), ("m", m1, rm), ("v", v1, rv)):
            assert np.array_equal(got[:va].view(np.uint32), want.view(np.uint32)), f"C shard {i} {nm}"
    assert pos == len(raw)


def test_graph_from_plain_c(gpu):
    exe = os.path.join(ROOT, "tests", "c", "graph_from_c")
    assert os.path.exists(exe), "tests/c/graph_from_c is missing: run __graft_entry__.build() first"
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    assert "graph_from_c: ok" in r.stdout
