"""GPU: the capturable step calls, whose step count lives in device memory.

fsdp_mt_step_capturable and fsdp_mt_step_clipped_capturable advance a device
int64 count and step at the new count, deriving the count's scalars on the
device with the host's operations; given a device learning rate they derive
the rate's scalars from it the same way.  So:
  * eager calls equal fsdp_mt_step / fsdp_mt_step_clipped at t = 1, 2, ...
    bit for bit (one-range and chunk-table plans, both store policies);
  * the fp8 forms (fsdp_mt_step_amax_capturable, fsdp_mt_step_fp8_capturable)
    replayed from captured graphs equal the fixed-count fp8 calls, codes,
    maxima and scales included;
  * one captured HIP graph, replayed with eager work and synchronisations
    between replays, steps through t = 1, 2, ... and equals the eager
    fixed-count calls at each t bit for bit, the count ending at the number
    of replays;
  * with the learning rate in device memory, written before each replay, the
    replays follow a schedule (warmup, then decay) and equal the eager calls
    at each step's rate bit for bit: the fused step on one-range and
    chunk-table plans, the clipped step and both fp8 forms;
  * counts far out (t up to 10^6, where the bias corrections are 1) still
    agree with the host's scalars;
  * an empty plan advances the count only; bad arguments are refused before
    any work is queued.
The fixed-count calls are checked against the oracle in the other GPU tests.
"""

import pytest
import torch

from rank_step_amd import binding as B
from rank_step_amd.state import RankState
from rank_step_amd.workloads import WORKLOADS

pytestmark = pytest.mark.gpu

STEPS = 4


def _bits(t):
    return t.view(torch.int16) if t.element_size() == 2 else t.view(torch.int32)


def _same(a, b, what):
    for name in ("master", "exp_avg", "exp_avg_sq", "grad_out", "ag_slot"):
        x, y = getattr(a, name), getattr(b, name)
        if x is None:
            continue
        assert torch.equal(_bits(x), _bits(y)), f"{what}: {name} differs"


def _pair(cfg, gpu, **kw):
    w = WORKLOADS[cfg]
    return w, RankState(w, 0, gpu, **kw), RankState(w, 0, gpu, **kw)


@pytest.mark.parametrize("cfg", [3, 2])
def test_eager_capturable_equals_fixed_count(cfg, gpu):
    """Config 3 (bf16 slices, one range) and config 2 (fp32 slices, one flat
    shard); the table path is covered by the graph test below."""
    w, a, b = _pair(cfg, gpu, bf16_out=w_bf16(cfg))
    a.make_plan(with_grad_out=False)
    b.make_plan(with_grad_out=False)
    count = torch.zeros(1, dtype=torch.int64, device=gpu)
    for t in range(1, STEPS + 1):
        a.load_grads(t)
        b.load_grads(t)
        a.plan.step(w.hparams, t)
        b.plan.step_capturable(w.hparams, count)
        torch.cuda.synchronize()
        _same(a, b, f"{w.name} t={t}")
        assert int(count.item()) == t
    a.close()
    b.close()


def w_bf16(cfg):
    return WORKLOADS[cfg].bf16_out


def _table_order_plan(st, **kw):
    """A plan over the rank's shards listed in reverse: not back to back in
    list order, so its step goes through the chunk table."""
    recs = st.mt_tensors(**kw)[::-1]
    st.plan = B.MtPlan(recs, st.w.n_slices, st.w.slice_dtype)
    assert st.plan.info()["step_one_range"] == 0
    return st.plan


@pytest.mark.parametrize("table", [False, True])
def test_graph_replays_advance_the_count(table, gpu):
    w, a, b = _pair(3, gpu, bf16_out=True)
    if table:
        _table_order_plan(a, with_grad_out=False, with_fp8=False)
        _table_order_plan(b, with_grad_out=False, with_fp8=False)
    else:
        a.make_plan(with_grad_out=False)
        b.make_plan(with_grad_out=False)
    count = torch.zeros(1, dtype=torch.int64, device=gpu)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        b.plan.step_capturable(w.hparams, count)
    torch.cuda.synchronize()
    assert int(count.item()) == 0, "capture ran the launches"
    for t in range(1, STEPS + 1):
        a.load_grads(t)
        b.load_grads(t)
        a.plan.step(w.hparams, t)
        g.replay()
        torch.cuda.synchronize()
        _same(a, b, f"replay {t}")
        assert int(count.item()) == t
    del g
    a.close()
    b.close()


# a learning-rate schedule: linear warmup over two steps, then decay, and a
# last step at rate 0 (the fused-step test only), where the parameters must
# not move at all while the moments still do
SCHEDULE = [5e-4, 1e-3, 8e-4, 6.4e-4, 5.12e-4, 0.0]


def _lr(t):
    return SCHEDULE[t - 1]


@pytest.mark.parametrize("table", [False, True])
def test_graph_replays_follow_a_device_learning_rate(table, gpu):
    w, a, b = _pair(3, gpu, bf16_out=True)
    if table:
        _table_order_plan(a, with_grad_out=False, with_fp8=False)
        _table_order_plan(b, with_grad_out=False, with_fp8=False)
    else:
        a.make_plan(with_grad_out=False)
        b.make_plan(with_grad_out=False)
    count = torch.zeros(1, dtype=torch.int64, device=gpu)
    lr = torch.zeros(1, dtype=torch.float64, device=gpu)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        b.plan.step_capturable(w.hparams, count, lr_dev=lr)
    torch.cuda.synchronize()
    for t in range(1, len(SCHEDULE) + 1):
        a.load_grads(t)
        b.load_grads(t)
        before = (b.master.clone(), b.exp_avg.clone())
        a.plan.step(dict(w.hparams, lr=_lr(t)), t)
        lr.fill_(_lr(t))
        g.replay()
        torch.cuda.synchronize()
        _same(a, b, f"lr replay {t}")
        assert int(count.item()) == t
        if _lr(t) == 0.0:
            assert torch.equal(_bits(b.master), _bits(before[0])), "rate 0 moved the parameters"
            assert not torch.equal(_bits(b.exp_avg), _bits(before[1]))
    # the same rate from the device and from the host: the eager forms agree too
    a.load_grads(9)
    b.load_grads(9)
    lr.fill_(3e-4)
    a.plan.step(dict(w.hparams, lr=3e-4), len(SCHEDULE) + 1)
    b.plan.step_capturable(w.hparams, count, lr_dev=lr)
    torch.cuda.synchronize()
    _same(a, b, "eager, device rate")
    del g
    a.close()
    b.close()


def test_clipped_graph_replays_advance_the_count(gpu):
    """With the learning rate in device memory as well."""
    w, a, b = _pair(3, gpu, bf16_out=True, grad_out=True)
    a.make_plan()
    b.make_plan()
    mk = lambda n, dt: torch.zeros(n, dtype=dt, device=gpu)
    sq_a, coef_a, norm_a = mk(1, torch.float64), mk(1, torch.float32), mk(1, torch.float64)
    sq_b, coef_b, norm_b = mk(1, torch.float64), mk(1, torch.float32), mk(1, torch.float64)
    count = torch.zeros(1, dtype=torch.int64, device=gpu)
    lr = mk(1, torch.float64)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        b.plan.reduce_sqnorm(sq_b)
        B.fsdp_clip_coef(coef_b, norm_b, sq_b, 1, 0.05)
        b.plan.step_clipped_capturable(w.hparams, count, coef_b, lr_dev=lr)
    torch.cuda.synchronize()
    for t in range(1, STEPS + 1):
        a.load_grads(t)
        b.load_grads(t)
        a.plan.reduce_sqnorm(sq_a)
        B.fsdp_clip_coef(coef_a, norm_a, sq_a, 1, 0.05)
        a.plan.step_clipped(dict(w.hparams, lr=_lr(t)), t, coef_a)
        lr.fill_(_lr(t))
        g.replay()
        torch.cuda.synchronize()
        _same(a, b, f"clipped replay {t}")
        assert torch.equal(coef_a, coef_b)
        assert int(count.item()) == t
    del g
    a.close()
    b.close()


def _same_fp8(a, b, what):
    _same(a, b, what)
    assert torch.equal(a.fp8, b.fp8), f"{what}: fp8 codes differ"


def test_fp8_graph_replays_advance_the_count(gpu):
    """Dynamic scaling (step with amax, then the codes) and delayed scaling
    (one pass with the previous step's scales), each captured once; the
    learning rate in device memory."""
    w, a, b = _pair(3, gpu, bf16_out=False, fp8_out=True)
    a.make_plan(with_grad_out=False, with_bf16=False)
    b.make_plan(with_grad_out=False, with_bf16=False)
    n = len(a.segments)
    mk = lambda: torch.zeros(n, dtype=torch.float32, device=gpu)
    amax_a, scale_a, amax_b, scale_b = mk(), mk(), mk(), mk()
    count = torch.zeros(1, dtype=torch.int64, device=gpu)
    lr = torch.zeros(1, dtype=torch.float64, device=gpu)
    torch.cuda.synchronize()
    g_dyn = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_dyn):
        b.plan.step_amax_capturable(w.hparams, count, amax_b, lr_dev=lr)
        b.plan.cast_fp8(amax_b, 1, scale_b)
    g_del = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_del):
        b.plan.step_fp8_capturable(w.hparams, count, scale_b, amax_b, lr_dev=lr)
    torch.cuda.synchronize()
    assert int(count.item()) == 0
    for t in range(1, STEPS + 1):
        a.load_grads(t)
        b.load_grads(t)
        hp_t = dict(w.hparams, lr=_lr(t))
        lr.fill_(_lr(t))
        if t % 2:
            a.plan.step_amax(hp_t, t, amax_a)
            a.plan.cast_fp8(amax_a, 1, scale_a)
            g_dyn.replay()
        else:
            a.plan.step_fp8(hp_t, t, scale_a, amax_a)
            g_del.replay()
        torch.cuda.synchronize()
        _same_fp8(a, b, f"fp8 replay {t}")
        assert torch.equal(amax_a, amax_b) and torch.equal(scale_a, scale_b)
        assert int(count.item()) == t
    del g_dyn, g_del
    a.close()
    b.close()


def test_far_counts_agree_with_the_host(gpu):
    """Counts where beta2^t is far from 1 and where it has vanished: the
    device-derived scalars step exactly as the host's."""
    w, a, b = _pair(3, gpu, bf16_out=True)
    a.make_plan(with_grad_out=False)
    b.make_plan(with_grad_out=False)
    count = torch.zeros(1, dtype=torch.int64, device=gpu)
    a.load_grads(1)
    b.load_grads(1)
    for t in (2, 3, 17, 999, 1000, 4097, 65536, 10 ** 6):
        count.fill_(t - 1)
        a.plan.step(w.hparams, t)
        b.plan.step_capturable(w.hparams, count)
        torch.cuda.synchronize()
        _same(a, b, f"t={t}")
        assert int(count.item()) == t
    a.close()
    b.close()


def test_empty_plan_and_refusals(gpu):
    w = WORKLOADS[3]
    count = torch.zeros(1, dtype=torch.int64, device=gpu)
    empty = B.MtPlan([], 8, "bf16")
    empty.step_capturable(w.hparams, count)
    torch.cuda.synchronize()
    assert int(count.item()) == 1
    empty.close()

    st = RankState(w, 0, gpu, bf16_out=True, grad_out=True)
    st.make_plan()
    before = [x.clone() for x in (st.master, st.exp_avg, st.exp_avg_sq)]
    coef = torch.ones(1, dtype=torch.float32, device=gpu)
    with pytest.raises(B.FsdpError, match="FSDP_E_ARG"):
        st.plan.step_capturable(w.hparams, None)
    with pytest.raises(B.FsdpError, match="FSDP_E_ARG"):
        st.plan.step_clipped_capturable(w.hparams, None, coef)
    wide = torch.zeros(3, dtype=torch.int64, device=gpu)
    with pytest.raises(B.FsdpError, match="FSDP_E_ALIGN"):
        B.fsdp_mt_step_capturable(st.plan.handle, w.hparams, wide.view(torch.int32)[1:].data_ptr())
    with pytest.raises(B.FsdpError, match="FSDP_E_ALIAS"):
        B.fsdp_mt_step_capturable(st.plan.handle, w.hparams, st.exp_avg.data_ptr())
    with pytest.raises(B.FsdpError, match="FSDP_E_ALIAS"):
        B.fsdp_mt_step_clipped_capturable(st.plan.handle, w.hparams, coef.data_ptr(), coef.data_ptr())
    # the device learning rate: 8-byte aligned, no written buffer of the plan,
    # not on the count
    lr_buf = torch.zeros(4, dtype=torch.float64, device=gpu)
    with pytest.raises(B.FsdpError, match="FSDP_E_ALIGN"):
        st.plan.step_capturable(w.hparams, count, lr_dev=lr_buf.view(torch.int32)[1:].data_ptr())
    with pytest.raises(B.FsdpError, match="FSDP_E_ALIAS"):
        st.plan.step_capturable(w.hparams, count, lr_dev=st.exp_avg.data_ptr())
    with pytest.raises(B.FsdpError, match="FSDP_E_ALIAS"):
        st.plan.step_capturable(w.hparams, count, lr_dev=st.ag_slot.data_ptr())
    with pytest.raises(B.FsdpError, match="FSDP_E_ALIAS"):
        st.plan.step_capturable(w.hparams, count, lr_dev=count.data_ptr())
    with pytest.raises(B.FsdpError, match="FSDP_E_ALIAS"):
        st.plan.step_clipped_capturable(w.hparams, count, coef, lr_dev=st.grad_out.data_ptr())
    amax = torch.zeros(len(st.segments), dtype=torch.float32, device=gpu)
    with pytest.raises(B.FsdpError, match="FSDP_E_ARG"):
        st.plan.step_amax_capturable(w.hparams, None, amax)   # (the plan has no fp8 copy either)
    bad = dict(w.hparams, lr=-1.0)
    with pytest.raises(B.FsdpError, match="FSDP_E_ARG"):
        st.plan.step_capturable(bad, count)
    torch.cuda.synchronize()
    assert int(count.item()) == 1, "a refused call advanced the count"
    for x, y in zip(before, (st.master, st.exp_avg, st.exp_avg_sq)):
        assert torch.equal(_bits(x), _bits(y)), "a refused call changed the state"
    st.close()
