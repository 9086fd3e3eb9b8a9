"""Plain, slow, double-precision CPU oracle for one FSDP FULL_SHARD rank step.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute anything in this package: only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, no
constants and no helpers with the HIP library in ``rank_step_amd/``, and it
imports nothing from there.

What it computes (one data-parallel rank's share of the step between the
backward reduce-scatter and the next forward all-gather):

* ``oracle.layout``  -- the shard layout (FlatParameter with tail padding, or
  per-parameter Shard(0)) and the per-rank byte summary.  Exact integers.
* ``oracle.step``    -- the fp32 mean of the N incoming gradient slices, the
  decoupled-weight-decay AdamW update on the shard only, and the
  round-to-nearest-even bf16 cast of the updated shard.  float64 throughout.
* ``oracle.clip``    -- global gradient-norm clipping across the ranks'
  shards (squared norms summed over ranks, one coefficient for all).
* ``oracle.fp8``     -- the fp8 (OCP E4M3) all-gather copy with per-tensor
  dynamic scales.
* ``oracle.accum``   -- gradient accumulation over micro-batches, with a
  reduce-scatter every micro-batch or once at the end (no_sync).

Sources (the pages this follows; cited by page title and section):

* "PyTorch 训练框架内核深度解析 -- 第18章 FSDP：ZeRO 风格的参数分片"
  (yangyitao.com book, chapter 18), below "FSDP chapter".
* "NCCL ZeRO / FSDP state sharding" (blog.cptz.space), below "ZeRO state
  sharding post".
* "PyTorch FSDP2 后端特性介绍" (MindSpeed-LLM docs), below "FSDP2 features doc".
* The torchtitan FSDP2/HSDP/meta-init article (gsyq.cn), below "torchtitan
  FSDP2 article".

Pins: every function here is checked by ``tests/test_oracle_*.py`` against
values the pages print, closed forms of the update rule, invariants and brute
force; none is "parity unpinned" except where the function's docstring says
so.
"""

from . import accum, clip, fp8, layout, step  # noqa: F401
