"""The prefill kernel variants (SEGKV_TUNE_PREFILL_KERNEL 2: four waves of
64 rows; 3: two wave groups one phase apart over host-balanced item lists;
4: the default's work software pipelined across tiles; 5: two workgroups
of 4 waves x 32 rows per CU over 128-row items) against the fp64
oracle, to the same bar as the default kernel: bf16 outputs within max-abs
2e-2 and LSE within 1e-3; bitwise repeatable."""

import numpy as np
import pytest

from long_context_serving_amd import segkv as S
from long_context_serving_amd import workloads as wl

from gpu_helpers import compare, gpu_run

pytestmark = pytest.mark.gpu

VARIANTS = [2, 3, 4, 5]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    S.load_library()


@pytest.mark.parametrize("kernel", VARIANTS)
@pytest.mark.parametrize("case", [
    # kv_lens, q_lens, hq, hkv, d, page, windows
    ((333,), (333,), 8, 2, 128, 64, (0, 100)),
    ((200,), (200,), 4, 4, 64, 16, (0, 1, 7, 64)),
    ((640,), (640,), 12, 4, 128, 16, (13, 0, 200, 640)),        # G = 3 does not divide the row tile
    ((600,), (600,), 16, 1, 128, 64, (0,)),                     # G = 16
    ((900, 17, 64, 500), (900, 5, 64, 1), 16, 4, 128, 64, (0, 64, 128, 33)),  # varlen batch with a cache fill
    ((2000,), (333,), 8, 8, 128, 32, (0, 1000, 10, 77, 0, 0, 3, 2000)),
])
def test_variant_matches_oracle(kernel, case):
    kv, q, hq, hkv, d, p, windows = case
    w = wl.small_workload("variant", kv, q, hq, hkv, d, p, windows, seed=sum(kv) + hq + d)
    x = wl.make_inputs(w)
    o, lse = gpu_run(w, x, prefill_kernel=kernel)
    compare(w, x, o, lse)


@pytest.mark.parametrize("kernel", VARIANTS)
def test_variant_split_and_relocated(kernel):
    w = wl.small_workload("variant_split", (1500, 700), (1500, 300), 16, 2, 128, 64, (0, 256), seed=77)
    x = wl.make_inputs(w)
    o, lse = gpu_run(w, x, split_tiles=3, prefill_kernel=kernel)
    compare(w, x, o, lse)
    rope = dict(deltas=[[4000, -20], [0, 123456]])
    o, lse = gpu_run(w, x, rope=rope, prefill_kernel=kernel)
    compare(w, x, o, lse, rope=rope)


@pytest.mark.parametrize("kernel", VARIANTS)
def test_variant_many_short_items_and_repeatable(kernel):
    """More items than workgroups, most of one or two tiles, run twice:
    bitwise equal."""
    kv = tuple(64 * (1 + i % 3) + 7 * i for i in range(40))
    w = wl.small_workload("variant_short", kv, kv, 8, 2, 128, 64, (0, 16), seed=3)
    x = wl.make_inputs(w)
    (o1, l1), (o2, l2) = gpu_run(w, x, repeat=2, prefill_kernel=kernel)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    compare(w, x, o1, l1)
