"""The CPU oracle against its pins (no GPU). See ``pins.py`` for what each
pin compares with."""

import pytest

import oracle
import pins


@pytest.fixture(scope="module")
def o():
    return oracle.load()


@pytest.mark.parametrize("pin", pins.ALL, ids=lambda p: p.__name__)
def test_pin(o, pin):
    pin(o)


def test_golden_fixtures_present():
    names = {p.name for p in pins.golden_cases()}
    assert {"q4_0_single_block.txt", "q4_0_two_rows_two_blocks.txt",
            "q8_0_two_rows.txt", "q4_k_single_superblock.txt"} <= names


def test_sampled_matches_full(o):
    import numpy as np
    import synth

    x = synth.activations(3, 512, seed=2)
    for fmt, w in (("q4_0", synth.q4_0_weights(40, 512, seed=2)),
                   ("q8_0", synth.q8_0_weights(40, 512, seed=2)),
                   ("q4_k", synth.q4_k_weights(40, 512, seed=2))):
        y, s = o.matmul(fmt, x, w, 40, 512)
        ms = np.array([0, 2, 1, 2]); ns = np.array([0, 39, 17, 5])
        ya, sa = o.matmul_at(fmt, x, w, 40, 512, ms, ns)
        assert np.array_equal(ya, y[ms, ns]) and np.array_equal(sa, s[ms, ns])


def test_empty_shapes(o):
    import numpy as np
    import synth

    y, s = o.matmul("q4_0", np.zeros((0, 64), np.float32), synth.q4_0_weights(3, 64), 3, 64)
    assert y.shape == (0, 3)
    y, s = o.matmul("q8_0", np.zeros((2, 64), np.float32), np.zeros(0, np.uint8), 0, 64)
    assert y.shape == (2, 0)
