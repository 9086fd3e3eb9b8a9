"""Oracle: shard layout of one rank (exact integer arithmetic, pure Python).

Test infrastructure only (see ``oracle/__init__``).

Two modes, both written from the pages' statement of the problem:

FLAT (FSDP-1 FlatParameter)
    FSDP chapter §18.12 "FlatParameter": the parameters of one wrap unit are
    flattened and concatenated, in registration order, into one 1-D vector
    (its example: 589824 + 768 + 768 = 591360 elements) and that vector is
    sharded once; all parameters of a unit share one dtype.
    ZeRO state sharding post, section "FlatParameter 与 Padding": when the
    element count does not divide by N the vector is padded at its end to
    P_physical = N * ceil(P_logical / N), the all-gather output holds exactly
    N times the shard, and a rank's view of an original parameter is a 1-D
    piece that may be empty (size 0).  Rank r therefore owns the padded flat
    range [r*S, r*S + S) with S = ceil(P / N).

SHARD0 (FSDP-2 per-parameter Shard(0))
    FSDP2 features doc, section "DTensor": each parameter is sharded on its own
    along dim 0 ([4096, 4096] -> a [512, 4096] local tensor per rank at 8
    ranks); torchtitan FSDP2 article §2.3: (C_out, C_in) -> (C_out/N, C_in).
    FSDP chapter §18.14: an [8, 8] weight gives a [4, 8] local shard at 2
    ranks.  Where N does not divide dim 0 the pages are silent; the reading
    taken is ceil(d0/N) rows per rank with trailing ranks padded with zero
    rows (possibly all padding).

OWNER (ZeRO-1, ZeroRedundancyOptimizer)
    ZeRO state sharding post, "ZeRO-1：Optimizer State Sharding" and
    "Optimizer Step 的所有权": whole parameters are handed to owner ranks; only
    the owner keeps their optimizer state and updates them, then broadcasts
    them; parameters and gradients stay replicated (its measured table: 128 /
    128 / 64 MiB per rank for 128 MiB of fp32 at N = 4, factors 4 / 4 / 2).
    Owners should be balanced by bytes, not by parameter count (the post lists
    count-balancing among its mistakes).  The assignment rule is not printed;
    the reading taken is the greedy largest-first one: parameters in
    decreasing byte size (ties: lower index first) each go to the rank with
    the fewest bytes so far (ties: lower rank).

Byte summary
    FSDP chapter §18.39: while micro-batches accumulate under no_sync the
    gradient stays unsharded, N times the size of the sharded one.
    ZeRO state sharding post, tables "Canonical ZeRO 状态公式" and "实测状态因子":
    at stage 3 every rank holds P/N parameters, P/N gradients and 2P/N
    optimizer state (fp32 AdamW: 4P/N bytes-worth in total), e.g. 32 / 32 /
    64 MiB per rank for 128 MiB of fp32 parameters at N = 4.  torchtitan FSDP2
    article §2.3: with bf16 parameters plus an fp32 master copy and both fp32
    moments the optimizer side costs 12 bytes per parameter.

Record fields per (tensor i, rank r), identical in both modes:

    shard_numel    length of the local buffer tensor i's data lives in
                   (FLAT: the whole flat shard S; SHARD0: ceil(d0/N)*row)
    valid          leading elements of that buffer that are real data; the
                   rest, [valid, shard_numel), is zero padding
    global_offset  element offset of tensor i in the unpadded concatenation
                   of all tensors in the order given
    view_offset    where tensor i's local piece starts, in the rank's local
                   storage (FLAT: inside the flat shard; SHARD0: inside the
                   packed concatenation of this rank's shards in order)
    view_numel     elements of tensor i that rank r holds (may be 0)
    tensor_offset  index, in tensor i flattened, of the first element held

For an empty FLAT view the offsets are the clipped positions where the piece
would start: view_offset = min(lo - r*S, S), tensor_offset = min(lo - o_i, n_i)
with lo = max(o_i, r*S).
"""

from dataclasses import dataclass

FLAT = 0
SHARD0 = 1
OWNER = 2

DTYPE_SIZE = {"f32": 4, "bf16": 2}


@dataclass(frozen=True)
class View:
    shard_numel: int
    valid: int
    global_offset: int
    view_offset: int
    view_numel: int
    tensor_offset: int
    owner: int = -1


@dataclass(frozen=True)
class Summary:
    logical_numel: int   # sum of numel over the tensors
    physical_numel: int  # padded element count across all N ranks
    shard_numel: int     # this rank's local element count (pad included)
    pad_numel: int       # this rank's padding elements
    bytes_param: int     # local parameter bytes in the parameter dtype(s)
    bytes_grad: int      # local fp32 gradient shard bytes (reduce dtype fp32)
    bytes_optim: int     # local exp_avg + exp_avg_sq bytes (fp32 each)
    bytes_master: int    # local fp32 master bytes (0 without a master copy)
    bytes_grad_unsharded: int  # fp32 gradient held while accumulating without reducing


def _ceil_div(a, b):
    return -(-a // b)


def _clamp(x, lo, hi):
    return max(lo, min(x, hi))


def flat_layout(numels, world_size, rank):
    """FLAT views of every tensor for ``rank``; returns (views, S, P, valid_r).

    FSDP chapter §18.12 and ZeRO state sharding post "FlatParameter 与 Padding".
    """
    assert world_size >= 1 and 0 <= rank < world_size
    P = sum(numels)
    S = _ceil_div(P, world_size)
    lo_r = rank * S
    hi_r = lo_r + S
    valid_r = _clamp(P - lo_r, 0, S)
    views = []
    o = 0
    for n in numels:
        lo = max(o, lo_r)
        hi = min(o + n, hi_r)
        if hi > lo:
            vo, vn, to = lo - lo_r, hi - lo, lo - o
        else:
            vo, vn, to = min(lo - lo_r, S), 0, min(lo - o, n)
        views.append(View(S, valid_r, o, vo, vn, to))
        o += n
    return views, S, P, valid_r


def shard0_view(numel, dim0, world_size, rank):
    """Shard(0) piece of one tensor: (shard_numel, valid, tensor_offset).

    FSDP2 features doc "DTensor"; torchtitan FSDP2 article §2.3.
    """
    if numel == 0:
        return 0, 0, 0
    row = numel // dim0
    c = _ceil_div(dim0, world_size)
    rows_held = _clamp(dim0 - rank * c, 0, c)
    first_row = min(rank * c, dim0)
    return c * row, rows_held * row, first_row * row


def owner_assignment(sizes, world_size):
    """ZeRO-1 owners of whole parameters, balanced by bytes: (numel, dtype)
    pairs in, one rank per parameter out (greedy, largest first)."""
    nbytes = [n * DTYPE_SIZE[d] for n, d in sizes]
    order = sorted(range(len(sizes)), key=lambda i: (-nbytes[i], i))
    load = [0] * world_size
    owners = [0] * len(sizes)
    for i in order:
        q = min(range(world_size), key=lambda r: (load[r], r))
        owners[i] = q
        load[q] += nbytes[i]
    return owners


def layout(mode, world_size, rank, shapes, has_master):
    """Views and byte summary for ``rank``.

    ``shapes`` is a list of (numel, dim0, dtype) with dtype in {"f32", "bf16"};
    a 0-d tensor is (1, 1, dtype).  FLAT requires a single dtype (FSDP chapter
    §18.12: FlatParameter rejects mixed dtypes); raises ValueError otherwise.
    """
    if mode == FLAT:
        dts = {d for _, _, d in shapes}
        if len(dts) > 1:
            raise ValueError("FLAT layout needs one dtype per unit")
        views, S, P, valid_r = flat_layout([n for n, _, _ in shapes], world_size, rank)
        esize = DTYPE_SIZE[dts.pop()] if dts else 4
        local = S
        pad = S - valid_r
        physical = world_size * S
        bytes_param = S * esize
    elif mode == SHARD0:
        views = []
        o = 0
        packed = 0
        physical = 0
        bytes_param = 0
        pad = 0
        for numel, dim0, dt in shapes:
            sn, valid, toff = shard0_view(numel, dim0, world_size, rank)
            views.append(View(sn, valid, o, packed, valid, toff))
            o += numel
            packed += sn
            physical += world_size * sn
            bytes_param += sn * DTYPE_SIZE[dt]
            pad += sn - valid
        P = o
        local = packed
    elif mode == OWNER:
        owners = owner_assignment([(n, d) for n, _, d in shapes], world_size)
        views = []
        o = 0
        packed = 0
        for (numel, _, _), own in zip(shapes, owners):
            mine = own == rank
            views.append(View(numel if mine else 0, numel if mine else 0, o, packed,
                              numel if mine else 0, 0, own))
            o += numel
            if mine:
                packed += numel
        P = o
        local = packed
        physical = P
        pad = 0
        bytes_param = sum(n * DTYPE_SIZE[d] for n, _, d in shapes)
    else:
        raise ValueError("unknown layout mode")
    summary = Summary(
        logical_numel=P,
        physical_numel=physical,
        shard_numel=local,
        pad_numel=pad,
        bytes_param=bytes_param,
        bytes_grad=4 * (P if mode == OWNER else local),   # ZeRO-1: gradients replicated
        bytes_optim=8 * local,
        bytes_master=4 * local if has_master else 0,
        # FSDP chapter §18.26 / §18.39: with no_sync the gradient stays
        # unsharded -- the padded flat vector, or the full parameters
        bytes_grad_unsharded=4 * (physical if mode == FLAT else P),
    )
    return views, summary
