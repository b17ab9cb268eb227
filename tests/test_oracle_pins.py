"""The CPU oracle against its pins (hand-worked fixtures, closed forms, exact arithmetic,
library special cases and invariants); see oracle_pins.py."""
import pytest

import oracle
import oracle_pins


@pytest.fixture(scope="module")
def orc():
    return oracle.default()


@pytest.mark.parametrize("pin", oracle_pins.PINS, ids=lambda p: p.__name__)
def test_pin(orc, pin):
    pin(orc)


def test_argument_errors(orc):
    import numpy as np
    x = np.zeros((2, 8), np.uint16)
    with pytest.raises(ValueError):
        orc.fused([x], x, np.zeros(9, np.uint16), 1e-6)
    with pytest.raises(TypeError):
        orc.reduce([x.astype(np.int32)])


@pytest.mark.parametrize("threads", [1, 2, 3, 7, 16, 64])
def test_row_slices_on_host_threads_give_the_oracle_result(orc, threads):
    """oracle.fused_threads (rows cut into contiguous slices, each computed by the same
    single-threaded function on its own host thread) is what the GPU tests compare the largest
    problems with: it must give the single-threaded oracle's bits, for any slicing, including more
    threads than rows and slices of unequal length."""
    import numpy as np
    from all_reduce_residual_way_amd import synth
    for m, dist in ((37, "normal"), (5, "stress")):
        p = synth.make_problem(3, m, 520, seed=40 + m + threads, dist=dist)
        ro1, out1 = orc.fused(p.inputs, p.residual, p.weight, p.eps)
        ro2, out2 = orc.fused_threads(p.inputs, p.residual, p.weight, p.eps, threads)
        assert np.array_equal(ro1, ro2) and np.array_equal(out1, out2), (m, dist, threads)
