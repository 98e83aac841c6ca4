"""The kernels' workgroup order (tile_map in csrc/attn_device.h), evaluated on the host through
attn_tile_order_probe: every launch must give each (unit, tile) pair to exactly one workgroup, or an
output tile would go unwritten (or be written twice). Also checks the locality properties the order is
built for: with a unit count that is a multiple of 8 a unit's tiles stay on one XCD (workgroup i runs on
XCD i % 8), the query-tile passes and the dense dK/dV passes keep at most four of an XCD's units in flight
at a time, and a unit's tiles rotate through the XCD's four shader engines (workgroup i on engine
(i / 8) % 4). No GPU needed."""
import itertools

import pytest

import scaled_dot_product_02_amd as sd

SHAPES = [(1, 1), (2, 1), (3, 7), (8, 1), (8, 4), (8, 5), (16, 64), (24, 5), (32, 64), (40, 3), (40, 33),
          (48, 7), (56, 32), (64, 30), (72, 9), (128, 64), (136, 17), (256, 32), (512, 30), (2048, 2), (12, 64)]


@pytest.mark.parametrize("units,tiles", SHAPES)
@pytest.mark.parametrize("reverse,order", list(itertools.product([False, True], ["tile_major", "query", "grouped"])))
def test_order_is_a_bijection(units, tiles, reverse, order):
    u, t = sd.attn_tile_order_probe(units, tiles, reverse=reverse, order=order)
    pairs = set(zip(u, t))
    assert len(u) == units * tiles
    assert all(0 <= x < units for x in u) and all(0 <= x < tiles for x in t)
    assert len(pairs) == units * tiles


@pytest.mark.parametrize("units,tiles", [(s, t) for s, t in SHAPES if s % 8 == 0])
@pytest.mark.parametrize("order", ["tile_major", "query", "grouped"])
def test_unit_keeps_one_xcd(units, tiles, order):
    u, _ = sd.attn_tile_order_probe(units, tiles, reverse=True, order=order)
    xcd = {}
    for i, x in enumerate(u):
        assert xcd.setdefault(x, i % 8) == i % 8


@pytest.mark.parametrize("units,tiles", [(40, 33), (56, 32), (64, 30), (72, 9), (136, 17), (256, 32), (512, 30)])
@pytest.mark.parametrize("order", ["query", "grouped"])
def test_four_units_in_flight(units, tiles, order):
    """Above four units per XCD, each XCD's sequence takes its units four at a time (the last group may be
    smaller): in every stretch of 4 * tiles consecutive workgroups of one XCD, starting at a group boundary,
    only that group's units occur, each with all its tiles, longest (highest, reverse order) first."""
    u, t = sd.attn_tile_order_probe(units, tiles, reverse=True, order=order)
    per_xcd = units // 8
    for x in range(8):
        seq = [(u[i], t[i]) for i in range(x, units * tiles, 8)]
        for g0 in range(0, per_xcd, 4):
            n = min(4, per_xcd - g0)
            chunk = seq[g0 * tiles:(g0 + n) * tiles]
            assert len({a for a, _ in chunk}) == n
            assert sorted(chunk) == sorted((a, b) for a in {a for a, _ in chunk} for b in range(tiles))
            tiles_in_order = [b for _, b in chunk]
            assert tiles_in_order == sorted(tiles_in_order, reverse=True)


@pytest.mark.parametrize("units,tiles", [(64, 32), (256, 32), (32, 64), (128, 64)])
@pytest.mark.parametrize("order", ["tile_major", "query", "grouped"])
def test_tiles_rotate_through_shader_engines(units, tiles, order):
    """Each unit's tiles are spread evenly over the four shader engines of its XCD."""
    u, _ = sd.attn_tile_order_probe(units, tiles, reverse=True, order=order)
    counts = {}
    for i, x in enumerate(u):
        counts.setdefault(x, [0, 0, 0, 0])[(i // 8) % 4] += 1
    for c in counts.values():
        assert max(c) - min(c) <= 1, c


def test_few_tiles_are_unit_major():
    """With at most four tiles per unit, consecutive workgroups of one XCD take one unit's tiles in the
    query-tile passes; the dK/dV passes keep their rounds there (tile-major, grouped four units at a time)."""
    u, t = sd.attn_tile_order_probe(2048, 2, reverse=True, order="query")
    for x in range(8):
        seq = [u[i] for i in range(x, len(u), 8)]
        assert all(seq[2 * k] == seq[2 * k + 1] for k in range(len(seq) // 2))
    u, t = sd.attn_tile_order_probe(2048, 2, order="grouped")
    for x in range(8):
        seq = [(u[i], t[i]) for i in range(x, len(u), 8)]
        assert [b for _, b in seq[:8]] == [0, 0, 0, 0, 1, 1, 1, 1]


def test_tile_major_rounds():
    """The packed dK/dV passes keep plain tile-major rounds: workgroup i runs tile i // units."""
    for units, tiles in ((128, 64), (40, 7), (12, 5)):
        _, t = sd.attn_tile_order_probe(units, tiles, order="tile_major")
        assert t == [i // units for i in range(units * tiles)]


def test_probe_declines_bad_arguments():
    from scaled_dot_product_02_amd import _binding
    with pytest.raises(RuntimeError):
        _binding.attn_tile_order_probe(0, 4)
    with pytest.raises(RuntimeError):
        _binding.attn_tile_order_probe(4, 1 << 23)
    L = _binding.lib()
    u = (_binding.ctypes.c_int32 * 4)()
    assert L.attn_tile_order_probe(2, 2, 0, 3, u, u, 4) != 0  # unknown order
    assert L.attn_tile_order_probe(2, 2, 2, 1, u, u, 4) != 0  # reverse not 0/1
    assert L.attn_tile_order_probe(2, 2, 0, 1, u, u, 3) != 0  # n != units * tiles
