"""The C ABI from plain C (CPU only): tests/c/layout_from_c.c includes
include/fsdp_step.h as C99, links librank_step.so and calls the host-only
layout entry point; its output must equal the oracle's layout, and a bad
rank must come back as FSDP_E_ARG with a message."""

import json
import os
import shutil
import subprocess

import pytest

from oracle import layout as OL
from rank_step_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SHAPES = [(256 * 256, 256, "f32"), (256, 256, "f32"), (1024 * 256, 1024, "f32"), (256 * 1024, 256, "f32")]


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs a C compiler")
def test_layout_from_plain_c(tmp_path):
    lib = B.lib_path()
    assert os.path.exists(lib), "build librank_step.so first"
    exe = tmp_path / "layout_from_c"
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"),
                    os.path.join(ROOT, "tests", "c", "layout_from_c.c"), "-o", str(exe),
                    lib, "-Wl,-rpath," + os.path.dirname(lib)], check=True, timeout=120)
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60, check=True).stdout
    rows = [json.loads(line) for line in out.splitlines()]
    fields = ("shard_numel", "valid", "global_offset", "view_offset", "view_numel", "tensor_offset", "owner")
    summ = ("logical_numel", "physical_numel", "shard_numel", "pad_numel", "bytes_param", "bytes_grad",
            "bytes_optim", "bytes_master", "bytes_grad_unsharded")
    for row in rows[:-1]:
        ref_v, ref_s = OL.layout(row["mode"], 4, row["rank"], SHAPES, False)
        assert row["views"] == [[getattr(v, f) for f in fields] for v in ref_v], row
        assert row["summary"] == [getattr(ref_s, f) for f in summ], row
    assert len(rows) == 3 * 4 + 1
    assert rows[-1] == {"bad_rank": -1, "message": 1}
