"""The fp64 oracle against its pins (CPU only)."""
import numpy as np
import pytest

import oracle
from tests.oracle_pins import PINS, random_case


@pytest.fixture(scope="module")
def orc():
    oracle.build(force=False)
    return oracle.Oracle()


@pytest.mark.parametrize("pin", PINS, ids=[p.__name__ for p in PINS])
def test_pin(orc, pin):
    pin(orc)


def test_threads_do_not_change_results(orc):
    args, h0 = random_case(81, batch=3, dim=7, L=33, N=16)
    o1, l1 = orc.scan(**args, softplus=True, h0=h0, nthreads=1)
    o4, l4 = orc.scan(**args, softplus=True, h0=h0, nthreads=4)
    assert np.array_equal(o1, o4) and np.array_equal(l1, l4)


def test_rejects_unsupported_dstate(orc):
    args, _ = random_case(82, N=257, L=4)   # beyond the oracle's 256-state rows
    with pytest.raises(ValueError):
        orc.scan(**args)


def test_scan_row_matches_scan(orc):
    args, h0 = random_case(83)
    out, last = orc.scan(**args, softplus=True, h0=h0)
    b, d = 1, 2
    o, l = orc.scan_row(args["u"][b, d], args["delta"][b, d], args["A"][d],
                        args["B"][b], args["C"][b], D_d=args["D"][d],
                        z=args["z"][b, d], bias_d=args["delta_bias"][d],
                        softplus=True, h0=h0[b, d])
    assert np.array_equal(o, out[b, d]) and np.array_equal(l, last[b, d])
