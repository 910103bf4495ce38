"""segkv_decode_noalloc (the decode variant for callers that cannot
allocate: its tables and partials live in the library's fixed device
scratch) against segkv_decode on the same state: two calls in a row, the
second on a smaller batch, each bit for bit equal to the workspace path and
within the oracle's tolerance; device memory is unchanged by the calls."""

import numpy as np
import pytest

from gpu_helpers import compare, say
from long_context_serving_amd import runner as R
from long_context_serving_amd import segkv as S
from long_context_serving_amd import workloads as wl

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    S.load_library()


def _decode_pair(w, x, seq_subset=None):
    """Workspace decode and no-alloc decode of the same context state."""
    import torch
    dev = R.to_device(w, x)
    run = R.WorkloadRun(w, dev).load()
    try:
        ids = run.seq_ids if seq_subset is None else [run.seq_ids[i] for i in seq_subset]
        q = dev.q if seq_subset is None else dev.q[seq_subset].contiguous()
        o_ref, l_ref = run.ctx.decode(0, ids, q)
        o = torch.full_like(q, 3.0)
        lse = torch.full(q.shape[:2], 5.0, dtype=torch.float32, device=q.device)
        torch.cuda.synchronize()
        free0 = torch.cuda.mem_get_info()[0]
        run.ctx.decode(0, ids, q, o, lse, no_alloc=True)
        torch.cuda.synchronize()
        assert torch.cuda.mem_get_info()[0] == free0
        assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16)), "outputs differ from segkv_decode"
        assert torch.equal(lse, l_ref), "lse differs from segkv_decode"
        return S.bf16_bits(o), lse.cpu().numpy().astype(np.float64)
    finally:
        run.close()


def test_noalloc_decode_matches_decode_twice_second_smaller():
    # first call: 12 sequences of mixed lengths (split segments, combine)
    w1 = wl.Workload("noalloc_big", tuple(int(v) for v in np.linspace(3000, 20000, 12)), (1,) * 12, 32, 8, 128, 64,
                     (0, 512, 1024, 0, 2048, 300, 4096, 64), seed=61, decode=True)
    x1 = wl.make_inputs(w1)
    say("no-alloc decode, 12 sequences")
    o1, l1 = _decode_pair(w1, x1)
    compare(w1, x1, o1, l1)
    # second call: fewer, shorter sequences; the scratch still holds the first call's bytes
    w2 = wl.Workload("noalloc_small", (700, 1500, 90), (1, 1, 1), 32, 8, 128, 64,
                     (0, 512, 1024, 0, 2048, 300, 4096, 64), seed=62, decode=True)
    x2 = wl.make_inputs(w2)
    say("no-alloc decode, 3 sequences")
    o2, l2 = _decode_pair(w2, x2)
    compare(w2, x2, o2, l2)


def test_noalloc_decode_full_size_32k():
    w = wl.DECODE_32K
    x = wl.make_inputs(w)
    say("no-alloc decode, 32K x 31")
    o, lse = _decode_pair(w, x)
    compare(w, x, o, lse)


def test_noalloc_decode_needs_outputs_and_device_context():
    import torch
    kv = S.SegKV(1, 4, 2, 64, 16, 2, 64, [0, 8], planning=True)
    with pytest.raises(S.SegKVError) as e:
        kv._check(kv._lib.segkv_decode_noalloc(kv._h, 0, 0, None, None, None, None))
    assert e.value.code == S.SEGKV_E_STATE
    kv.close()
    w = wl.Workload("noalloc_args", (100,), (1,), 4, 2, 64, 16, (0, 8), seed=63, decode=True)
    dev = R.to_device(w, wl.make_inputs(w))
    run = R.WorkloadRun(w, dev).load()
    with pytest.raises(ValueError):
        run.ctx.decode(0, run.seq_ids, dev.q, no_alloc=True)
    o = torch.empty_like(dev.q)
    lse = torch.empty(dev.q.shape[:2], dtype=torch.float32, device="cuda")
    with pytest.raises(S.SegKVError) as e:
        run.ctx.decode(0, [5], dev.q, o, lse, no_alloc=True)
    assert e.value.code == S.SEGKV_E_RANGE
    run.close()
