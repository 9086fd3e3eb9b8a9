"""One rank's optimizer state of a workload, resident in HBM, and its plan.

Sizes come from the library's own ``fsdp_shard_layout`` and the placement of
the buffers from its ``fsdp_rank_buffer_layout``; torch only allocates the
memory.  Layout of the buffers: one device allocation per rank, carved into
regions that each start on a 2 MiB boundary (the order below):

* ``master``, ``exp_avg``, ``exp_avg_sq``: fp32 ``[S_total]``, the rank's
  local shards of every parameter packed in registration order (FLAT: the one
  flat shard), each shard at its ``view_offset``;
* ``slices``: ``[N, S_total]`` in the slice dtype, rows ``slice_stride`` =
  S_total rounded up to 64, plus 256, elements apart (S_total when N is 1) --
  slice q is the q-th incoming gradient
  buffer of this rank's shard, i.e. the rank's chunk of rank q's full
  gradient -- so the slice stride of every shard is ``slice_stride``;
* ``ag``: bf16 all-gather input.  With ``ag_full`` it is the packed
  ``[N * S_total]`` buffer of the next all-gather and this rank writes the
  slot at ``rank * S_total``; otherwise only this rank's slot is allocated;
* ``grad_out`` (fp32 ``[S_total]``) and ``fp8`` (bytes ``[S_total]``) when
  asked for.

Why one allocation and a padded stride: the fused step streams a dozen
arrays in lockstep, element k of each at once, so how those arrays fall on
HBM channels and banks relative to each other sets its speed.  Separate
allocations leave that to where the driver puts each one: the 7B shard's step
took 5.34-5.93 ms over such placements.  Carved from one allocation, the
arrays keep their relative offsets; with the slice rows 256 elements past
S_total apart it took 5.34-5.45 ms in every placement measured, and with
rows exactly S_total apart up to 5.57.
"""

import torch

from . import binding
from .workloads import grad_slices, init_master, init_seed, shapes_of

_DT = {"f32": torch.float32, "bf16": torch.bfloat16}


class RankState:
    def __init__(self, w, rank, device, bf16_out=True, grad_out=False, ag_full=False,
                 garbage_pad=False, fp8_out=False):
        self.w = w
        self.rank = rank
        self.device = device
        views, summ = binding.fsdp_shard_layout(w.mode, w.world_size, rank, shapes_of(w),
                                                w.has_master)
        self.views = views
        self.summary = summ
        total = summ["shard_numel"]
        self.total = total
        if w.mode == "flat":
            # one flat shard; is_norm does not apply to a flat unit
            segs = [(0, total, views[0]["valid"] if views else 0, False)] if total else []
        else:
            segs = [(v["view_offset"], v["shard_numel"], v["valid"], p.is_norm)
                    for v, p in zip(views, w.params) if v["shard_numel"] > 0]
        self.segments = segs
        sdt = _DT[w.slice_dtype]
        slots = (w.world_size if ag_full else 1) if bf16_out else 0
        lay = binding.fsdp_rank_buffer_layout(total, w.n_slices, w.slice_dtype, slots, grad_out, fp8_out)
        self.buffer_layout = lay
        self.slice_stride = lay["slice_stride"]
        n_ag = total * slots
        offs = {"master": lay["param_offset"], "exp_avg": lay["exp_avg_offset"],
                "exp_avg_sq": lay["exp_avg_sq_offset"], "slices": lay["slices_offset"],
                "ag": lay["bf16_offset"], "grad_out": lay["grad_out_offset"], "fp8": lay["fp8_offset"]}
        ra = lay["region_align"]
        size = max(1, (lay["total_bytes"] + ra - 1) // ra * ra)   # a whole number of regions
        self._mem = torch.empty(size, dtype=torch.uint8, device=device)

        def region(name, dt, n):
            es = torch.empty(0, dtype=dt).element_size()
            assert offs[name] >= 0, name
            return self._mem[offs[name]:offs[name] + n * es].view(dt)

        self.master = region("master", torch.float32, total)
        self.master.copy_(init_master(total, segs, init_seed(w.cfg, rank), device,
                                      garbage_pad=garbage_pad))
        self.exp_avg = region("exp_avg", torch.float32, total).zero_()
        self.exp_avg_sq = region("exp_avg_sq", torch.float32, total).zero_()
        if garbage_pad:
            for off, length, held, _ in segs:
                self.exp_avg[off + held:off + length] = float("nan")
                self.exp_avg_sq[off + held:off + length] = float("inf")
        rows = region("slices", sdt, w.n_slices * self.slice_stride).view(w.n_slices, self.slice_stride)
        rows.fill_(float("nan") if sdt != torch.uint8 else 0)   # the padding is never read
        self.slices = rows[:, :total]
        self.ag = None
        self.ag_slot = None
        if bf16_out:
            self.ag = region("ag", torch.bfloat16, n_ag).zero_()
            self.ag_slot = self.ag[rank * total:(rank + 1) * total] if ag_full else self.ag
        self.grad_out = region("grad_out", torch.float32, total) if grad_out else None
        # fp8 all-gather copy (this rank's slot), codes as bytes
        self.fp8 = region("fp8", torch.uint8, total).zero_() if fp8_out else None
        self.plan = None

    def load_grads(self, step):
        """Fill the slice buffer with step ``step``'s seeded gradients."""
        grad_slices(self.w, self.total, step, self.rank, self.device, out=self.slices)

    def mt_tensors(self, with_grad_out=True, with_bf16=True, with_fp8=True):
        es = self.slices.element_size()
        base = {
            "param": self.master.data_ptr(), "m": self.exp_avg.data_ptr(),
            "v": self.exp_avg_sq.data_ptr(), "s": self.slices.data_ptr(),
            "ag": self.ag_slot.data_ptr() if (self.ag_slot is not None and with_bf16) else None,
            "f8": self.fp8.data_ptr() if (self.fp8 is not None and with_fp8) else None,
            "g": self.grad_out.data_ptr() if (self.grad_out is not None and with_grad_out) else None,
        }
        out = []
        for off, length, held, _ in self.segments:
            out.append({
                "param_fp32": base["param"] + 4 * off,
                "exp_avg": base["m"] + 4 * off,
                "exp_avg_sq": base["v"] + 4 * off,
                "grad_slices": base["s"] + es * off,
                "slice_stride": self.slice_stride,
                "unshard_bf16_out": None if base["ag"] is None else base["ag"] + 2 * off,
                "grad_shard_out": None if base["g"] is None else base["g"] + 4 * off,
                "unshard_fp8_out": None if base["f8"] is None else base["f8"] + off,
                "shard_numel": length,
                "valid": held,
            })
        return out

    def make_plan(self, stream=None, with_grad_out=True, with_bf16=True, with_fp8=True):
        self.plan = binding.MtPlan(self.mt_tensors(with_grad_out, with_bf16, with_fp8),
                                   self.w.n_slices, self.w.slice_dtype, stream)
        return self.plan

    def step(self, t, stream=None):
        self.plan.step(self.w.hparams, t, stream)

    def close(self):
        if self.plan is not None:
            self.plan.close()
            self.plan = None
