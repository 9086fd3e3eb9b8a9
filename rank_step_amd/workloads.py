"""Synthetic workloads: parameter shapes and seeded input generators.

This module holds no arithmetic of the rank step itself -- no layout, no
reduction, no update, no cast.  It lists the parameter shapes of each
workload and draws seeded random inputs (initial weights, incoming gradient
slices) for buffers whose sizes the caller passes in.  Both the HIP parity
tests and the CPU oracle tests draw their inputs here; random values go in as
plain inputs to both sides.

Workloads (all synthetic; the pages use no dataset):

1. tiny_mlp_flat_n4   FLAT, N=4, fp32.  W1[256,256], b1[256], W2[1024,256],
                      W3[256,1024] flattened to 590,080 elements.
2. mlp128m_flat_n4    FLAT, N=4, fp32, no master copy: 24 x [1024,1365] plus a
                      [8192] remainder = 2**25 elements (128 MiB), the size of
                      the fp32 MLP measured in the ZeRO state sharding post.
3. llama7b_block_n8   Shard(0), N=8: one Llama-7B-style block (hidden 4096,
                      FFN 11008), bf16 params with fp32 master/m/v.
4. llama7b_full_n8    Shard(0), N=8: 32 such blocks + embedding and lm_head
                      [32000,4096] + final norm = 291 local shards.
5. llama70b_full_n32  Shard(0), N=32: 80 blocks of hidden 8192, FFN 28672,
                      8 KV heads of 128, vocab 128256 = 723 local shards.
6. mlp128m_zero1_n4   ZeRO-1 owners, N=4: the ZeRO state sharding post's MLP
                      as 8 equal fp32 Linear weights [2048,2048] (128 MiB),
                      two whole weights updated per rank.

Value recipe: weights ~ N(0, 0.02) fp32, norm weights 1.0, moments 0.  Slice
q of rank r at step t is drawn with seed 1000*cfg + 100*t + 10*r + q (mask /
outlier draws: that seed + 50), as N(0, sigma) fp32, then masked or scaled,
then rounded to the slice dtype by torch's own conversion.
"""

from dataclasses import dataclass, field

import torch

HPARAMS = {"lr": 1e-3, "beta1": 0.9, "beta2": 0.999, "eps": 1e-8, "weight_decay": 0.01}


@dataclass(frozen=True)
class Param:
    name: str
    dims: tuple
    dtype: str          # parameter dtype: "f32" or "bf16"
    is_norm: bool = False

    @property
    def numel(self):
        n = 1
        for d in self.dims:
            n *= d
        return n

    @property
    def dim0(self):
        return self.dims[0] if self.dims else 1


@dataclass(frozen=True)
class Workload:
    cfg: int
    name: str
    mode: str                 # "flat" or "shard0"
    world_size: int
    params: tuple
    slice_dtype: str          # "f32" or "bf16"
    n_slices: int             # slices per element reaching the rank step
    has_master: bool
    bf16_out: bool            # whether the timed step writes the bf16 copy
    steps: int
    grad_sigma: float
    zero_frac: float = 0.0    # Bernoulli fraction of slice elements set to +0
    outlier_frac: float = 0.0  # Bernoulli fraction scaled by outlier_scale
    outlier_scale: float = 1.0
    hparams: dict = field(default_factory=lambda: dict(HPARAMS))


def _llama_block(prefix, hidden, ffn, kv_dim, dtype):
    return [
        Param(f"{prefix}.wq", (hidden, hidden), dtype),
        Param(f"{prefix}.wk", (kv_dim, hidden), dtype),
        Param(f"{prefix}.wv", (kv_dim, hidden), dtype),
        Param(f"{prefix}.wo", (hidden, hidden), dtype),
        Param(f"{prefix}.w_gate", (ffn, hidden), dtype),
        Param(f"{prefix}.w_up", (ffn, hidden), dtype),
        Param(f"{prefix}.w_down", (hidden, ffn), dtype),
        Param(f"{prefix}.attn_norm", (hidden,), dtype, True),
        Param(f"{prefix}.ffn_norm", (hidden,), dtype, True),
    ]


def _llama(n_layers, hidden, ffn, kv_dim, vocab, dtype):
    ps = [Param("embed", (vocab, hidden), dtype)]
    for i in range(n_layers):
        ps += _llama_block(f"layers.{i}", hidden, ffn, kv_dim, dtype)
    ps.append(Param("final_norm", (hidden,), dtype, True))
    ps.append(Param("lm_head", (vocab, hidden), dtype))
    return tuple(ps)


def _workloads():
    tiny = (Param("W1", (256, 256), "f32"), Param("b1", (256,), "f32"),
            Param("W2", (1024, 256), "f32"), Param("W3", (256, 1024), "f32"))
    mlp = tuple(Param(f"fc{i}", (1024, 1365), "f32") for i in range(24)) + (
        Param("remainder", (8192,), "f32"),)
    return {
        1: Workload(1, "tiny_mlp_flat_n4", "flat", 4, tiny, "f32", 4, False, False, 3, 1e-2),
        2: Workload(2, "mlp128m_flat_n4", "flat", 4, mlp, "f32", 4, False, False, 10, 1e-3,
                    zero_frac=0.1),
        3: Workload(3, "llama7b_block_n8", "shard0", 8,
                    tuple(_llama_block("layers.0", 4096, 11008, 4096, "bf16")),
                    "bf16", 8, True, True, 5, 1e-3),
        4: Workload(4, "llama7b_full_n8", "shard0", 8,
                    _llama(32, 4096, 11008, 4096, 32000, "bf16"),
                    "bf16", 8, True, True, 5, 1e-3, outlier_frac=0.01, outlier_scale=100.0),
        5: Workload(5, "llama70b_full_n32", "shard0", 32,
                    _llama(80, 8192, 28672, 1024, 128256, "bf16"),
                    "f32", 1, True, True, 3, 1e-4),
        6: Workload(6, "mlp128m_zero1_n4", "owner", 4,
                    tuple(Param(f"linear{i}", (2048, 2048), "f32") for i in range(8)),
                    "f32", 4, False, False, 3, 1e-3),
    }


WORKLOADS = _workloads()


def shapes_of(w):
    """(numel, dim0, dtype) triples in registration order."""
    return [(p.numel, p.dim0, p.dtype) for p in w.params]


# ---------------------------------------------------------------------------
# seeded generators


def init_seed(cfg, rank):
    return 1000 * cfg + rank


def slice_seed(cfg, step, rank, q):
    return 1000 * cfg + 100 * step + 10 * rank + q


def _gen(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def init_master(total, segments, seed, device, garbage_pad=False):
    """fp32 initial weights for a local buffer of ``total`` elements.

    ``segments`` lists (offset, length, held, is_norm): a stretch of the
    buffer, how many of its leading elements are real data, and whether it is
    a norm weight (initialised to 1.0).  The trailing ``length - held``
    elements of each segment are filled with +0, or with large garbage when
    ``garbage_pad`` is set (the step must overwrite them with +0).
    """
    g = _gen(device, seed)
    x = torch.randn(total, generator=g, device=device, dtype=torch.float32) * 0.02
    for off, length, held, is_norm in segments:
        if is_norm and held > 0:
            x[off:off + held] = 1.0
        if length > held:
            x[off + held:off + length] = 1.0e30 if garbage_pad else 0.0
    return x


def grad_slices(w, total, step, rank, device, n_slices=None, stride=None, out=None):
    """Gradient slices of one rank: a ``[n_slices, stride]`` tensor in the
    workload's slice dtype, of which the first ``total`` columns are drawn.

    ``out`` (optional) is filled in place instead of allocating.  Columns
    beyond ``total`` (a wider stride) hold NaN garbage that the step must
    never read; pad positions inside ``total`` hold random values that the
    step must ignore as well.
    """
    n = w.n_slices if n_slices is None else n_slices
    stride = total if stride is None else stride
    dt = torch.float32 if w.slice_dtype == "f32" else torch.bfloat16
    if out is None:
        out = torch.full((n, stride), float("nan"), dtype=dt, device=device)
    else:
        assert out.shape[0] == n and out.shape[1] >= total and out.dtype == dt
    for q in range(n):
        s = slice_seed(w.cfg, step, rank, q)
        x = torch.randn(total, generator=_gen(device, s), device=device,
                        dtype=torch.float32)
        x.mul_(w.grad_sigma)
        if w.zero_frac > 0.0 or w.outlier_frac > 0.0:
            u = torch.rand(total, generator=_gen(device, s + 50), device=device)
            if w.zero_frac > 0.0:
                x.masked_fill_(u < w.zero_frac, 0.0)
            if w.outlier_frac > 0.0:
                x = torch.where(u < w.outlier_frac, x * w.outlier_scale, x)
            del u
        out[q, :total].copy_(x)
        del x
    return out
