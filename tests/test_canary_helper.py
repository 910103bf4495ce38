"""The canary check of the GPU tests (GuardedPools), on CPU tensors: it
flags writes to the guard pages and to pages no segment held, and accepts
writes to held pages."""

import pytest

from gpu_helpers import GuardedPools


class _Ctx:
    """Stands in for a context: one layer, one sequence, one KV head holding `pages`."""

    num_layers, max_seqs, num_kv_heads = 1, 1, 1

    def __init__(self, pages):
        self.pages = pages

    def page_table(self, layer, seq, g):
        return 0, 0, self.pages


def test_untouched_pools_pass():
    gp = GuardedPools(10, 16, 64, device="cpu")
    gp.note(_Ctx([3, 4]))
    assert gp.check()


def test_writes_to_held_pages_pass():
    gp = GuardedPools(10, 16, 64, device="cpu")
    gp.note(_Ctx([3, 4]))
    gp.k[3].fill_(1.0)
    gp.v[4, 0, 0] = 2.0
    assert gp.check()


@pytest.mark.parametrize("where", ["k_before", "k_after", "v_before", "v_after", "k_never", "v_never"])
def test_stray_writes_are_flagged(where):
    gp = GuardedPools(10, 16, 64, device="cpu")
    gp.note(_Ctx([3, 4]))
    t = gp.k_all if where.startswith("k") else gp.v_all
    page = {"before": 0, "after": gp.g + gp.n, "never": gp.g + 7}[where.split("_")[1]]
    t[page, 1, 1] = 0.0
    with pytest.raises(AssertionError):
        gp.check()
