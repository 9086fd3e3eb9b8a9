"""Pins of the oracle's layout against the pages' printed values, the padding
formula and brute-force ownership invariants (CPU only)."""

import json
import os

import pytest

from oracle import layout as L
from rank_step_amd.workloads import WORKLOADS, shapes_of

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "layout_examples.json")))


def test_flat_concat_example():
    g = GOLD["flat_concat"]
    shapes = [(n, d0, "f32") for n, d0 in zip(g["numels"], [s[0] for s in g["shapes"]])]
    views, summ = L.layout(L.FLAT, 1, 0, shapes, False)
    assert summ.logical_numel == g["flat_numel"]
    assert [v.global_offset for v in views] == [0, 589824, 589824 + 768]
    assert all(v.view_numel == n for v, n in zip(views, g["numels"]))


@pytest.mark.parametrize("P,N,phys", GOLD["padding_formula"]["cases"])
def test_padding_formula(P, N, phys):
    _, summ = L.layout(L.FLAT, N, 0, [(P, max(P, 1), "f32")], False)
    assert summ.physical_numel == phys
    assert summ.physical_numel % N == 0
    assert summ.physical_numel == summ.shard_numel * N


@pytest.mark.parametrize("case", GOLD["shard0_examples"]["cases"])
def test_shard0_examples(case):
    dims, N, ld = case["dims"], case["world_size"], case["local_dims"]
    numel = dims[0] * dims[1]
    for r in range(N):
        views, _ = L.layout(L.SHARD0, N, r, [(numel, dims[0], "bf16")], True)
        v = views[0]
        assert v.shard_numel == ld[0] * ld[1]
        assert v.valid == ld[0] * ld[1]
        assert v.tensor_offset == r * ld[0] * ld[1]


def test_stage3_bytes_example():
    g = GOLD["stage3_bytes"]
    w = WORKLOADS[2]
    assert sum(p.numel for p in w.params) * 4 == g["logical_param_bytes"]
    MiB = 1 << 20
    for r in range(w.world_size):
        _, s = L.layout(L.FLAT, w.world_size, r, shapes_of(w), False)
        assert s.bytes_param == g["per_rank_param_mib"] * MiB
        assert s.bytes_grad == g["per_rank_grad_mib"] * MiB
        assert s.bytes_optim == g["per_rank_optim_mib"] * MiB
        assert s.bytes_master == 0


def test_mixed_precision_bytes_7b():
    g = GOLD["mixed_precision_bytes"]
    w = WORKLOADS[4]
    views, s = L.layout(L.SHARD0, 8, 0, shapes_of(w), True)
    assert len(views) == 291
    assert s.shard_numel == 842_301_952
    assert s.bytes_master + s.bytes_optim == g["optim_plus_master_bytes_per_param"] * 842_301_952
    assert s.bytes_param == g["bf16_bytes_per_param"] * 842_301_952 == 1_684_603_904


def _flat_brute(numels, N):
    P = sum(numels)
    owner = {}
    concat = []
    tensor_of = []
    for i, n in enumerate(numels):
        tensor_of += [(i, j) for j in range(n)]
    valid_sum = 0
    S = None
    for r in range(N):
        views, S, P_, valid_r = L.flat_layout(numels, N, r)
        assert P_ == P
        valid_sum += valid_r
        # padded flat vector seen through the rank's shard
        for k in range(S):
            gidx = r * S + k
            concat.append(gidx if gidx < P else None)
            if k < valid_r:
                assert gidx < P
                owner.setdefault(gidx, []).append((r, k))
            else:
                assert gidx >= P
        o = 0
        for i, v in enumerate(views):
            for j in range(v.view_numel):
                # element j of the view is tensor i's element tensor_offset + j
                k = v.view_offset + j
                assert k < valid_r
                assert tensor_of[r * S + k] == (i, v.tensor_offset + j)
            assert v.global_offset == o
            if v.view_numel == 0:
                # an empty view sits where the tensor meets the shard: a tensor
                # that ends at or before the shard's start is seen at offset 0,
                # past its last element; one that starts at or after the
                # shard's end, at offset S, before its first element
                n = numels[i]
                if o + n <= r * S:
                    assert (v.view_offset, v.tensor_offset) == (0, n)
                elif o >= r * S + S:
                    assert (v.view_offset, v.tensor_offset) == (S, 0)
                else:
                    assert (v.view_offset, v.tensor_offset) == (o - r * S, 0)
            o += numels[i]
    assert valid_sum == P
    assert sorted(owner) == list(range(P))
    assert all(len(o) == 1 for o in owner.values())
    assert concat[:P] == list(range(P)) and all(c is None for c in concat[P:])
    assert len(concat) == N * S


def test_flat_bruteforce_small():
    import itertools
    import random
    rnd = random.Random(7)
    for N in range(1, 10):
        for P in range(0, 65):
            # split P into 1..4 tensors (zero-size tensors included)
            k = rnd.randint(1, 4)
            cuts = sorted(rnd.randint(0, P) for _ in range(k - 1))
            numels = [b - a for a, b in zip([0] + cuts, cuts + [P])]
            _flat_brute(numels, N)
    for numels in itertools.product([0, 1, 3, 8], repeat=3):
        for N in (1, 2, 3, 5, 8):
            _flat_brute(list(numels), N)


def test_shard0_bruteforce_small():
    for N in range(1, 10):
        for d0 in range(0, 21):
            for row in (1, 2, 3):
                numel = d0 * row
                seen = []
                valid_sum = 0
                sizes = set()
                for r in range(N):
                    views, s = L.layout(L.SHARD0, N, r, [(numel, max(d0, 1), "f32")], False)
                    v = views[0]
                    sizes.add(v.shard_numel)
                    assert v.shard_numel % max(row, 1) == 0
                    assert 0 <= v.valid <= v.shard_numel
                    # the rank's first row, or the tensor's end for an all-padding rank
                    assert 0 <= v.tensor_offset <= numel
                    if v.valid == 0:
                        assert v.tensor_offset == numel
                    seen += list(range(v.tensor_offset, v.tensor_offset + v.valid))
                    valid_sum += v.valid
                    assert s.pad_numel == v.shard_numel - v.valid
                assert len(sizes) == 1          # every rank holds the same local size
                assert valid_sum == numel
                assert seen == list(range(numel))   # rank order concatenation is the tensor


def test_tiny_mlp_rank_views():
    w = WORKLOADS[1]
    S = 147_520
    got = []
    for r in range(4):
        views, s = L.layout(L.FLAT, 4, r, shapes_of(w), False)
        assert s.shard_numel == S and s.pad_numel == 0 and s.physical_numel == 590_080
        got.append([(v.view_offset, v.view_numel, v.tensor_offset) for v in views])
    # rank 0 = W1 + b1 + the first 81,728 elements of W2
    assert got[0] == [(0, 65536, 0), (65536, 256, 0), (65792, 81728, 0), (S, 0, 0)]
    # rank 1 lies inside W2
    assert got[1][2] == (0, S, 81728) and got[1][3][1] == 0 and got[1][0][1] == 0
    # rank 2 = the tail of W2 + the head of W3
    assert got[2][2] == (0, 262144 - 81728 - S, 81728 + S)
    assert got[2][3] == (262144 - 81728 - S, S - (262144 - 81728 - S), 0)
    # rank 3 lies inside W3 and ends at its end
    v3 = got[3][3]
    assert v3[0] == 0 and v3[1] == S and v3[2] + v3[1] == 262144


def test_mlp128m_rank0():
    w = WORKLOADS[2]
    views, s = L.layout(L.FLAT, 4, 0, shapes_of(w), False)
    assert s.logical_numel == 1 << 25 and s.shard_numel == 8_388_608 and s.pad_numel == 0
    full = [i for i, v in enumerate(views) if v.view_numel == 1_397_760]
    assert full == [0, 1, 2, 3, 4, 5]
    assert views[6].view_numel == 2048 and views[6].tensor_offset == 0
    assert all(v.view_numel == 0 for v in views[7:])


@pytest.mark.parametrize("cfg,n_tensors,local", [(3, 9, 25_297_920), (4, 291, 842_301_952),
                                                 (5, 723, 2_204_803_328)])
def test_shard0_workload_counts(cfg, n_tensors, local):
    w = WORKLOADS[cfg]
    views, s = L.layout(L.SHARD0, w.world_size, 0, shapes_of(w), True)
    assert len(views) == n_tensors
    assert s.shard_numel == local and s.pad_numel == 0
    assert s.physical_numel == s.logical_numel == local * w.world_size
    # packed offsets are the running sum of local sizes
    off = 0
    for v in views:
        assert v.view_offset == off
        off += v.shard_numel


def test_flat_rejects_mixed_dtypes():
    with pytest.raises(ValueError):
        L.layout(L.FLAT, 2, 0, [(4, 4, "f32"), (4, 4, "bf16")], False)


def test_stage3_formula_random_shapes():
    import random
    rnd = random.Random(3)
    for _ in range(200):
        N = rnd.randint(1, 16)
        shapes = [(rnd.randint(0, 5000), 1, "f32") for _ in range(rnd.randint(1, 6))]
        shapes = [(n, max(n, 1), d) for n, _, d in shapes]
        P = sum(n for n, _, _ in shapes)
        phys = N * (-(-P // N))
        for r in range(N):
            _, s = L.layout(L.FLAT, N, r, shapes, False)
            total = s.bytes_param + s.bytes_grad + s.bytes_optim
            assert total * N == 4 * 4 * phys      # 4 fp32 words per physical element


def test_no_sync_gradient_is_n_times_the_shard():
    # FSDP chapter §18.39: the unsharded gradient kept under no_sync is N times
    # the sharded gradient (not multiplied by the number of micro-batches)
    w = WORKLOADS[2]
    for r in range(4):
        _, s = L.layout(L.FLAT, 4, r, shapes_of(w), False)
        assert s.bytes_grad_unsharded == 4 * s.bytes_grad == 4 * (1 << 25)
    _, s = L.layout(L.FLAT, 3, 0, [(10, 10, "f32")], False)
    assert s.bytes_grad_unsharded == 4 * 12 == 3 * s.bytes_grad
    w = WORKLOADS[4]
    _, s = L.layout(L.SHARD0, 8, 0, shapes_of(w), True)
    assert s.bytes_grad_unsharded == 8 * s.bytes_grad == 4 * 6_738_415_616


def test_zero1_page_table():
    g = GOLD["zero1_bytes"]
    n = g["param_dims"][0] * g["param_dims"][1]
    shapes = [(n, g["param_dims"][0], "f32")] * g["n_params"]
    N = g["world_size"]
    MiB = 1 << 20
    P_bytes = 4 * n * g["n_params"]
    tot = [0, 0, 0]
    for r in range(N):
        views, s = L.layout(L.OWNER, N, r, shapes, False)
        assert s.bytes_param == g["per_rank_param_mib"] * MiB
        assert s.bytes_grad == g["per_rank_grad_mib"] * MiB
        assert s.bytes_optim == g["per_rank_optim_mib"] * MiB
        assert sum(v.owner == r for v in views) == 2
        tot = [tot[0] + s.bytes_param, tot[1] + s.bytes_grad, tot[2] + s.bytes_optim]
    assert [t / P_bytes for t in tot] == g["factors"]


def test_owner_balances_bytes_not_counts():
    # one large and three small parameters at N=2: byte balance gives the large
    # one a rank of its own (count balance would pair it with a small one)
    views, _ = L.layout(L.OWNER, 2, 0, [(1000, 1, "f32"), (10, 1, "f32"), (10, 1, "f32"),
                                        (10, 1, "f32")], False)
    assert [v.owner for v in views] == [0, 1, 1, 1]
    # bf16 parameters weigh half as much per element: by bytes the order is
    # 400 B, 360 B, 240 B -> owners 1, 0, 1 (by element count it would be 0, 1, 1)
    views, _ = L.layout(L.OWNER, 2, 0, [(120, 1, "bf16"), (100, 1, "f32"), (90, 1, "f32")], False)
    assert [v.owner for v in views] == [1, 0, 1]


def test_owner_bruteforce_invariants():
    import random
    rnd = random.Random(11)
    for _ in range(300):
        N = rnd.randint(1, 9)
        shapes = [(rnd.randint(0, 5000), 1, rnd.choice(["f32", "bf16"])) for _ in range(rnd.randint(0, 12))]
        shapes = [(n, max(n, 1), d) for n, _, d in shapes]
        owners = None
        loads = []
        for r in range(N):
            views, s = L.layout(L.OWNER, N, r, shapes, True)
            if owners is None:
                owners = [v.owner for v in views]
            assert [v.owner for v in views] == owners          # one assignment seen by all ranks
            off = 0
            for (n, _, d), v in zip(shapes, views):
                mine = v.owner == r
                assert v.view_offset == off and v.view_numel == (n if mine else 0)
                assert v.shard_numel == v.valid == v.view_numel and v.tensor_offset == 0
                off += v.view_numel
            assert s.shard_numel == off and s.pad_numel == 0
            assert s.bytes_optim == 8 * off and s.bytes_master == 4 * off
            loads.append(sum(n * L.DTYPE_SIZE[d] for (n, _, d), o in zip(shapes, owners) if o == r))
        assert all(0 <= o < N for o in owners)
        biggest = max([n * L.DTYPE_SIZE[d] for n, _, d in shapes], default=0)
        assert max(loads) - min(loads) <= biggest                # greedy balance bound
