"""HIP graph capture of the step entry points: replays equal eager calls bit for bit.

A caller may capture a whole optimizer step in a HIP graph (torch's
CUDAGraph on ROCm) once its plan exists.  The plan calls only launch
kernels on the caller's stream: no allocation, no host synchronisation and no
memset.  The sequences captured:
  * the fused step (one launch);
  * the clipped step: reduce + sum of squares, clip coefficient, scaled update;
  * the fp8 step: step with amax, per-tensor amax, fp8 codes;
  * the fused and clipped steps of a plan whose shards name their slices
    through tables of pointers (its own kernel variants).
Each graph is replayed several times, with eager work (fresh gradients) and
synchronisations between the replays.  After every replay, the state and
outputs must equal a twin state driven by the same calls made eagerly.  The
eager calls are themselves checked against the oracle in the other GPU tests.

The step count and learning rate reach the kernels by value, so a captured
step keeps the ones it was captured with: every replay equals an eager step
at the captured count, and differs from one at the advancing count (the
limitation the header states at fsdp_adamw_hparams).
"""

import pytest
import torch

from rank_step_amd import binding as B
from rank_step_amd.state import RankState
from rank_step_amd.workloads import WORKLOADS

pytestmark = pytest.mark.gpu

REPLAYS = 4


def _bits(t):
    if t is None:
        return None
    return t.view(torch.int16) if t.element_size() == 2 else (
        t.view(torch.uint8) if t.element_size() == 1 else t.view(torch.int32))


def _same(a, b, what):
    for name in ("master", "exp_avg", "exp_avg_sq", "grad_out", "ag_slot", "fp8"):
        x, y = getattr(a, name), getattr(b, name)
        if x is None:
            continue
        assert torch.equal(_bits(x), _bits(y)), f"{what}: {name} differs"


def _pair(w, gpu, **kw):
    a = RankState(w, 0, gpu, **kw)
    b = RankState(w, 0, gpu, **kw)
    return a, b


def _run(w, a, b, gpu, calls, extra=(), init=None):
    """calls(state, bufs) enqueues one step on the current stream; bufs holds
    that state's own scalars (zero, or the value ``init`` gives the name).
    Captures calls(b) once, then replays."""
    init = init or {}
    bufs_a = {k: torch.full((n,), init.get(k, 0.0), dtype=dt, device=gpu) for k, (n, dt) in extra}
    bufs_b = {k: torch.full((n,), init.get(k, 0.0), dtype=dt, device=gpu) for k, (n, dt) in extra}
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        calls(b, bufs_b)
    torch.cuda.synchronize()
    # capture recorded the launches without running them
    for rep in range(REPLAYS):
        a.load_grads(rep + 1)
        b.load_grads(rep + 1)
        calls(a, bufs_a)
        g.replay()
        torch.cuda.synchronize()
        _same(a, b, f"{w.name} replay {rep}")
        for k in bufs_a:
            assert torch.equal(bufs_a[k], bufs_b[k]) or (
                torch.isnan(bufs_a[k]).all() and torch.isnan(bufs_b[k]).all()), f"{k} replay {rep}"
    del g


def test_fused_step_graph(gpu):
    w = WORKLOADS[3]
    a, b = _pair(w, gpu, bf16_out=True)
    a.make_plan(with_grad_out=False)
    b.make_plan(with_grad_out=False)
    _run(w, a, b, gpu, lambda st, _: st.plan.step(w.hparams, 3))
    a.close()
    b.close()


def test_clipped_step_graph(gpu):
    w = WORKLOADS[3]
    a, b = _pair(w, gpu, bf16_out=True, grad_out=True)
    a.make_plan()
    b.make_plan()

    def calls(st, bufs):
        st.plan.reduce_sqnorm(bufs["sq"])
        B.fsdp_clip_coef(bufs["coef"], bufs["norm"], bufs["sq"], 1, 0.05)
        st.plan.step_clipped(w.hparams, 2, bufs["coef"])

    _run(w, a, b, gpu, calls, extra=(("sq", (1, torch.float64)), ("coef", (1, torch.float32)),
                                     ("norm", (1, torch.float64))))
    a.close()
    b.close()


def test_fp8_step_graph(gpu):
    w = WORKLOADS[3]
    a, b = _pair(w, gpu, bf16_out=False, fp8_out=True)
    a.make_plan(with_grad_out=False, with_bf16=False)
    b.make_plan(with_grad_out=False, with_bf16=False)
    n = len(a.segments)

    def calls(st, bufs):
        st.plan.step_amax(w.hparams, 4, bufs["amax"])
        st.plan.cast_fp8(bufs["amax"], 1, bufs["scale"])

    _run(w, a, b, gpu, calls, extra=(("amax", (n, torch.float32)), ("scale", (n, torch.float32))))
    a.close()
    b.close()



def test_delayed_fp8_step_graph(gpu):
    """The one-pass fp8 step with scales fixed before the step: captured once,
    replayed with the same scale buffer; codes, amax and state equal eager."""
    w = WORKLOADS[3]
    a, b = _pair(w, gpu, bf16_out=True, fp8_out=True)
    a.make_plan(with_grad_out=False)
    b.make_plan(with_grad_out=False)
    n = len(a.segments)

    def calls(st, bufs):
        st.plan.step_fp8(w.hparams, 5, bufs["scale"], bufs["amax"])

    _run(w, a, b, gpu, calls, extra=(("scale", (n, torch.float32)), ("amax", (n, torch.float32))),
         init={"scale": 448.0 / 0.05})
    a.close()
    b.close()


def _table_plan(st):
    """A plan over st whose shards name their slices through tables of
    pointers (the rows of st's slice buffer)."""
    es = st.slices.element_size()
    base = st.slices.data_ptr()
    recs = []
    for d, (off, length, held, _) in zip(st.mt_tensors(with_grad_out=True, with_fp8=False),
                                         st.segments):
        d = dict(d)
        d.pop("grad_slices")
        d.pop("slice_stride")
        d["grad_slice_ptrs"] = [base + es * (q * st.slice_stride + off) for q in range(st.w.n_slices)]
        recs.append(d)
    st.plan = B.MtPlan(recs, st.w.n_slices, st.w.slice_dtype)


def test_slice_table_steps_graph(gpu):
    """A plan with tables of slice pointers runs its own kernel variants:
    the fused step and the clipped step captured and replayed."""
    w = WORKLOADS[3]
    a, b = _pair(w, gpu, bf16_out=True, grad_out=True)
    _table_plan(a)
    _table_plan(b)

    def calls(st, bufs):
        st.plan.step(w.hparams, 3)
        st.plan.reduce_sqnorm(bufs["sq"])
        B.fsdp_clip_coef(bufs["coef"], None, bufs["sq"], 1, 0.05)
        st.plan.step_clipped(w.hparams, 4, bufs["coef"])

    _run(w, a, b, gpu, calls, extra=(("sq", (1, torch.float64)), ("coef", (1, torch.float32))))


def test_general_plan_graph(gpu):
    """A plan whose shards need the any-alignment forms (odd sizes: split
    shards, slices at an odd stride, the bf16 copy in an all-gather slot off
    a vector boundary) runs the general kernel variants: the fused, clipped
    and one-pass fp8 steps captured and replayed."""
    from tests.test_gpu_workloads import ODD
    w = ODD["shard0"]
    kw = dict(bf16_out=True, grad_out=True, ag_full=True, fp8_out=True)
    a, b = RankState(w, 1, gpu, **kw), RankState(w, 1, gpu, **kw)
    assert (a.total * 1) % 4 != 0, "rank 1's all-gather slot should start off a vector boundary"
    a.make_plan()
    b.make_plan()
    n = len(a.segments)

    def calls(st, bufs):
        st.plan.step(w.hparams, 3)
        st.plan.reduce_sqnorm(bufs["sq"])
        B.fsdp_clip_coef(bufs["coef"], None, bufs["sq"], 1, 0.05)
        st.plan.step_clipped(w.hparams, 4, bufs["coef"])
        st.plan.step_fp8(w.hparams, 5, bufs["scale"], bufs["amax"])

    _run(w, a, b, gpu, calls,
         extra=(("sq", (1, torch.float64)), ("coef", (1, torch.float32)),
                ("scale", (n, torch.float32)), ("amax", (n, torch.float32))),
         init={"scale": 448.0 / 0.05})
    a.close()
    b.close()


def test_graph_replays_keep_the_captured_step_count(gpu):
    """Captured at t=3 and replayed four times: each replay equals an eager
    step at t=3, not one at t = 3, 4, 5, 6 -- the bias corrections and the
    learning rate are fixed at capture."""
    w = WORKLOADS[3]
    kw = dict(bf16_out=True)
    fixed, graphed, advancing = (RankState(w, 0, gpu, **kw) for _ in range(3))
    for st in (fixed, graphed, advancing):
        st.make_plan(with_grad_out=False)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        graphed.plan.step(w.hparams, 3)
    torch.cuda.synchronize()
    for rep in range(REPLAYS):
        for st in (fixed, graphed, advancing):
            st.load_grads(rep + 1)
        fixed.plan.step(w.hparams, 3)
        advancing.plan.step(w.hparams, 3 + rep)
        g.replay()
        torch.cuda.synchronize()
        _same(fixed, graphed, f"replay {rep} against eager t=3")
        if rep > 0:
            assert not torch.equal(_bits(advancing.master), _bits(graphed.master)), \
                f"replay {rep} should not equal an eager step at t={3 + rep}"
    del g
    for st in (fixed, graphed, advancing):
        st.close()
