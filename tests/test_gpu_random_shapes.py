"""GPU parity on seeded random shapes: bucket counts from 1 to 64, experts per
bucket from 1 to 32 (up to 1024 experts), top-k up to 16, batches from 0 to
5000 tokens (tile and group boundaries drawn often), 1 to 64 channels, bf16
rows of 8 to 2048 values or FP8 rows of 1 to 16 blocks, empty slots, exact and
capacity mode, with and without get_dispatch_layout's outputs passed to the
first dispatch.  Every case runs the layout, the first dispatch and the
combine against the oracle (tests.test_gpu_edge.run_case)."""

import numpy as np
import pytest

from tests.test_gpu_edge import _rand, run_case

pytestmark = pytest.mark.gpu

CASES = 32


def shape(case: int):
    rng = np.random.default_rng(9400 + case)
    R = int(rng.choice([1, 2, 3, 4, 6, 8, 12, 16, 24, 32, 64]))
    P = int(rng.choice([1, 2, 4, 8, 16, 32]))
    while R * P > 1024:
        P //= 2
    E = R * P
    K = int(rng.integers(1, min(16, E) + 1))
    if rng.random() < 0.3:
        T = int(rng.choice([0, 1, 63, 64, 65, 255, 256, 257, 4096]))
    else:
        T = int(rng.integers(2, 5001))
    C = int(rng.integers(1, 65))
    fp8 = bool(rng.random() < 0.25)
    H = int(128 * rng.integers(1, 17)) if fp8 else int(8 * rng.integers(1, 257))
    return dict(T=T, E=E, K=K, R=R, C=C, H=H, fp8=fp8, capacity=bool(rng.random() < 0.6),
                from_layout=bool(rng.random() < 0.5),
                p_empty=float(rng.choice([0.0, 0.0, 0.05, 0.3])))


def test_shapes_cover_the_paths():
    """The draw reaches the one-launch first pack, the borrowing first pack,
    the general layout, FP8 and the largest bucket count."""
    s = [shape(c) for c in range(CASES)]
    one_launch = [x for x in s if x["capacity"] and 0 < x["T"] <= 4096 and x["R"] % 4 == 0
                  and x["R"] <= 16 and not x["fp8"]]
    assert one_launch and any(x["from_layout"] for x in one_launch)
    assert any(x["T"] > 4096 or x["R"] % 4 for x in s)
    assert any(x["fp8"] for x in s) and any(x["R"] == 64 for x in s)
    assert any(x["T"] == 0 for x in s) or any(x["T"] == 1 for x in s)


@pytest.mark.parametrize("case", range(CASES))
def test_random_shape(oracle, case):
    s = shape(case)
    idx = _rand(s["T"], s["E"], s["K"], p_empty=s["p_empty"], seed=case)
    run_case(oracle, idx, s["H"], s["E"], s["R"], s["C"], seed=case, capacity=s["capacity"],
             fp8=s["fp8"], from_layout=s["from_layout"])
