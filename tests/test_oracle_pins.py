"""The oracle against its pins (CPU only)."""
import os

import numpy as np
import pytest

import oracle
import pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin(oracle.get())


def test_page_shape_sizes():
    """Printed sizes fix D = 16, the 15 zonal rows and C = 32 at E = 647170."""
    fx = pins._golden("shape_sizes.txt")
    E = int(fx["edges"])
    surface = E * 15 * 32 * 4
    assert round(surface / 1e9, 1) == float(fx["message_surface_gb"])
    drop_mb = int(fx["peak_alloc_off_mb"]) - int(fx["peak_alloc_on_mb"])
    assert abs(drop_mb - surface / 1e6) < 1.0          # 1242 MB vs 1242.6 MB
    assert round(E * 16 * 16 * 4 / 1e6) == int(fx["dense_wigner_mb"])
    assert round(E * (3 * 16 - 2) * 4 / 1e6) == int(fx["band_mb"])


def test_row_ladder_sizes():
    """Degree blocks of the lmax = 3 ladder have 3/5/7 rows (row groups)."""
    assert [int(np.sum(pins.DEG == l)) for l in (1, 2, 3)] == [3, 5, 7]
    assert pins.DEG[0] == 0


def test_layout_example_arithmetic():
    fx = pins._golden("layout_worked_example.txt")
    E, C = int(fx["edges"]), int(fx["channels"])
    assert E * 3 * C == int(fx["radial_floats"])
    assert ((E - 1) * 3 + 2) * C == int(fx["last_edge_slot2_start"])
    assert ((E - 1) * 3 + 2) * C + int(fx["padded_lanes"]) - 1 == int(fx["last_padded_float"])
