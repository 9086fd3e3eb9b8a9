"""The layout oracle's pins must catch plausible mistakes: each mutant below
plants one in a copy of a layout helper (on the CPU) and at least one pin of
tests/test_oracle_layout.py has to fail against it.  The unmutated copies pass
every pin, so each failure is the planted mistake's."""

import pytest

from oracle import layout as L
import tests.test_oracle_layout as pins


def _expand(fn):
    """A pin as zero-argument calls, one per parametrized case."""
    marks = [m for m in getattr(fn, "pytestmark", []) if m.name == "parametrize"]
    if not marks:
        return [fn]
    names = [n.strip() for n in marks[0].args[0].split(",")]
    calls = []
    for case in marks[0].args[1]:
        vals = tuple(case) if len(names) > 1 else (case,)
        calls.append(lambda vals=vals: fn(**dict(zip(names, vals))))
    return calls


PINS = [c for name in sorted(dir(pins)) if name.startswith("test_")
        for c in _expand(getattr(pins, name))]


def _flat(kind):
    def flat_layout(numels, world_size, rank):
        P = sum(numels)
        S = P // world_size if kind == "shard_size_floor" else -(-P // world_size)
        lo_r = rank * S
        hi_r = lo_r + S
        if kind == "valid_not_clamped_at_zero":
            valid_r = min(P - lo_r, S)
        elif kind == "valid_not_clamped_at_shard":
            valid_r = max(P - lo_r, 0)
        else:
            valid_r = max(0, min(P - lo_r, S))
        views = []
        o = 0
        for n in numels:
            lo = max(o, lo_r)
            hi = min(o + n, hi_r)
            if hi > lo:
                vo = lo if kind == "view_offset_global" else lo - lo_r
                to = lo - lo_r if kind == "tensor_offset_from_shard" else lo - o
                vn = hi - lo
            else:
                vo = lo - lo_r if kind == "empty_view_offset_unclamped" else min(lo - lo_r, S)
                to = lo - o if kind == "empty_tensor_offset_unclamped" else min(lo - o, n)
                vn = 0
            views.append(L.View(S, valid_r, o, vo, vn, to))
            o += n
        return views, S, P, valid_r
    return flat_layout


def _shard0(kind):
    def shard0_view(numel, dim0, world_size, rank):
        if numel == 0:
            return 0, 0, 0
        row = numel // dim0
        c = dim0 // world_size if kind == "rows_floor" else -(-dim0 // world_size)
        if kind == "rows_not_clamped_at_zero":
            held = min(dim0 - rank * c, c)
        else:
            held = max(0, min(dim0 - rank * c, c))
        first = rank * c if kind == "first_row_unclamped" else min(rank * c, dim0)
        return c * row, held * row, first * row
    return shard0_view


def _owner(kind):
    def owner_assignment(sizes, world_size):
        nbytes = [n if kind == "balance_by_count_of_elements" else n * L.DTYPE_SIZE[d]
                  for n, d in sizes]
        order = sorted(range(len(sizes)), key=lambda i: (-nbytes[i], i))
        if kind == "smallest_first":
            order = order[::-1]
        load = [0] * world_size
        held = [0] * world_size
        owners = [0] * len(sizes)
        for j, i in enumerate(order):
            if kind == "ties_to_higher_rank":
                q = min(range(world_size), key=lambda r: (load[r], -r))
            elif kind == "fewest_parameters":
                q = min(range(world_size), key=lambda r: (held[r], r))
            elif kind == "round_robin":
                q = j % world_size
            else:
                q = min(range(world_size), key=lambda r: (load[r], r))
            owners[i] = q
            load[q] += nbytes[i]
            held[q] += 1
        return owners
    return owner_assignment


FLAT_MUTANTS = ["shard_size_floor", "valid_not_clamped_at_zero", "valid_not_clamped_at_shard",
                "view_offset_global", "tensor_offset_from_shard", "empty_view_offset_unclamped",
                "empty_tensor_offset_unclamped"]
SHARD0_MUTANTS = ["rows_floor", "rows_not_clamped_at_zero", "first_row_unclamped"]
OWNER_MUTANTS = ["balance_by_count_of_elements", "smallest_first", "ties_to_higher_rank",
                 "fewest_parameters", "round_robin"]


def _patch(monkeypatch, flat="none", shard0="none", owner="none"):
    monkeypatch.setattr(L, "flat_layout", _flat(flat))
    monkeypatch.setattr(L, "shard0_view", _shard0(shard0))
    monkeypatch.setattr(L, "owner_assignment", _owner(owner))


def _caught():
    n = 0
    for pin in PINS:
        try:
            pin()
        except AssertionError:
            n += 1
    return n


def test_unmutated_copies_pass_every_pin(monkeypatch):
    assert len(PINS) >= 20
    _patch(monkeypatch)
    for pin in PINS:
        pin()


@pytest.mark.parametrize("kind", FLAT_MUTANTS)
def test_flat_mutant_is_caught(kind, monkeypatch):
    _patch(monkeypatch, flat=kind)
    assert _caught() >= 1, kind


@pytest.mark.parametrize("kind", SHARD0_MUTANTS)
def test_shard0_mutant_is_caught(kind, monkeypatch):
    _patch(monkeypatch, shard0=kind)
    assert _caught() >= 1, kind


@pytest.mark.parametrize("kind", OWNER_MUTANTS)
def test_owner_mutant_is_caught(kind, monkeypatch):
    _patch(monkeypatch, owner=kind)
    assert _caught() >= 1, kind
