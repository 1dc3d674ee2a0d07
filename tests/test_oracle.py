"""The fp64 oracle against its pins (CPU only)."""
import numpy as np
import pytest

import oracle
from tests import oracle_pins as P


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin(oracle.bra_oracle)


@pytest.mark.parametrize("bad", [
    dict(N=1, H=7, W=8, C=4, heads=2, S=2, topk=1),
    dict(N=1, H=8, W=8, C=5, heads=2, S=2, topk=1),
    dict(N=1, H=8, W=8, C=4, heads=2, S=2, topk=0),
    dict(N=1, H=8, W=8, C=4, heads=2, S=2, topk=5),
    dict(N=0, H=8, W=8, C=4, heads=2, S=2, topk=1),
])
def test_preconditions_raise(bad):
    with pytest.raises(ValueError):
        oracle.check_shapes(**bad)


def test_route_override_out_of_range():
    q = np.zeros((1, 4, 4, 2))
    with pytest.raises(ValueError):
        oracle.bra_forward(q, q, q, np.zeros((2, 5, 5)), None, 1, 2, 1,
                           route_override=np.full((1, 4, 1), 4))
