"""The decode split plan never holds more chunks than the plan buffer and the
decode grid are sized for (CPU only).

The chunk-size rule is restated here from its description in the library
(units of even length: one round of 512 chunks, none shorter than 2048 slots;
ragged lengths, the longest above twice the mean: up to three rounds; at least
one chunk per unit), and
the capacity is read from the library itself: dms_plan_words(shape) =
16 + (units + 1) + max_chunks + 2 * units.  Ragged length mixes between 513
and 1535 units are the case the capacity once missed."""

import numpy as np
import pytest

from decode_attention_learned_amd import lib

TARGET, ROUNDS, PAGE = 512, 3, 64


def plan_chunks(n):
    """Chunks of a plan for per-unit slot counts n (the rule stated above)."""
    n = np.asarray(n, dtype=np.int64)
    units, total, mx = n.size, int(n.sum()), int(n.max())
    ragged = mx * units > 2 * total
    budget = (ROUNDS if ragged else 1) * TARGET
    if units >= budget:
        per = -(-mx // PAGE)
    else:
        room = PAGE * (budget - units)
        per = -(-total // room)
    C = max(PAGE if ragged else 2048, PAGE * max(1, per))
    return int(np.where(n > 0, -(-n // C), 1).sum())


def capacity(units):
    s = lib.DmsShape(units, 1, 4, 128, 64, 16, 8, 64, lib.DMS_KV_BF16)
    return lib.plan_words(s) - 16 - (units + 1) - 2 * units


@pytest.mark.parametrize("units", [1, 7, 511, 512, 513, 600, 800, 1024, 1535, 1536, 1537, 4096])
def test_plan_fits_its_buffer(units):
    lib.load()
    cap = capacity(units)
    rng = np.random.Generator(np.random.PCG64(units))
    cases = [
        np.full(units, 4110),                                         # even
        np.where(np.arange(units) % 4 == 0, 3001, 17),                # a quarter keep everything
        np.where(np.arange(units) == 0, 32768, 16),                   # one long unit
        (rng.beta(7, 1, units) < 0.5) * 30000 + 20,                   # two length classes
        np.maximum(1, (32768 * (1 - rng.beta(7, 1, units))).astype(np.int64)),  # Beta(7,1) rates
        np.where(np.arange(units) % 2 == 0, 0, 5000),                 # empty units mixed in
    ]
    for n in cases:
        assert plan_chunks(n) <= cap, (units, plan_chunks(n), cap)


def test_the_ragged_800_unit_case():
    """100 sequences x 8 KV heads, a quarter of the units long: 1200 chunks, which
    must fit (a capacity of one chunk per unit would hold 800)."""
    lib.load()
    n = np.where(np.arange(800) % 4 == 0, 3001, 17)
    assert plan_chunks(n) > 800
    assert plan_chunks(n) <= capacity(800)
