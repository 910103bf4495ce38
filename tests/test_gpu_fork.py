"""GPU parity of copy-on-write forks: sequences forked from a parent share
its pages, append their own tokens (copying a shared partial tail page
first), and attend over parent tokens + their own, against the fp64 oracle
on each sequence's token history.  The parent's output must not change
(bit for bit) when its forks append."""

import numpy as np
import pytest

from long_context_serving_amd import segkv as S
from long_context_serving_amd import workloads as wl
from oracle import attention as A

from gpu_helpers import LSE_TOL, O_TOL, GuardedPools, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    S.load_library()


class Scenario:
    """Token rows drawn once; each sequence's history is a list of row ids."""

    def __init__(self, hq, hkv, d, p, windows, n_tokens, seqs, seed, pages=None):
        import torch
        self.w = wl.small_workload("fork", (n_tokens,), (n_tokens,), hq, hkv, d, p, windows, seed)
        self.x = wl.make_inputs(self.w)
        self.q = S.bf16_tensor(self.x.q)
        self.k = S.bf16_tensor(self.x.k)
        self.v = S.bf16_tensor(self.x.v)
        self.windows = tuple(windows)
        n_pages = pages or (seqs * (n_tokens // p + 2) * hkv)
        self.canary = GuardedPools(n_pages, p, d)
        self.kv = S.SegKV(1, hq, hkv, d, p, seqs, n_pages, list(windows), softmax_scale=self.w.scale,
                          page_order_seed=seed + 1, k_pool=self.canary.k, v_pool=self.canary.v)
        self.hist = {}
        self.next_row = 0
        self.torch = torch

    def take(self, n):
        r = np.arange(self.next_row, self.next_row + n)
        self.next_row += n
        return r

    def append(self, seqs, counts, n_query):
        rows = [self.take(n) for n in counts]
        for s, r in zip(seqs, rows):
            self.hist.setdefault(s, []).extend(r.tolist())
        idx = self.torch.from_numpy(np.concatenate(rows + [np.zeros(0, np.int64)])).cuda()
        self.kv.append_pages(0, seqs, counts, n_query, self.k.index_select(0, idx).contiguous(),
                             self.v.index_select(0, idx).contiguous())
        self.canary.note(self.kv)

    def fork(self, src, dst):
        self.kv.fork(src, dst)
        self.hist[dst] = list(self.hist[src])

    def prefill(self, seqs, q_lens):
        rows = np.concatenate([np.asarray(self.hist[s][len(self.hist[s]) - n:], np.int64)
                               for s, n in zip(seqs, q_lens)] + [np.zeros(0, np.int64)])
        q = self.q.index_select(0, self.torch.from_numpy(rows).cuda()).contiguous()
        o, lse = self.kv.prefill(0, seqs, q_lens, q)
        self.torch.cuda.synchronize()
        return S.bf16_bits(o), lse.cpu().numpy().astype(np.float64)

    def decode(self, seqs):
        rows = np.array([self.hist[s][-1] for s in seqs], np.int64)
        q = self.q.index_select(0, self.torch.from_numpy(rows).cuda()).contiguous()
        o, lse = self.kv.decode(0, seqs, q)
        self.torch.cuda.synchronize()
        return S.bf16_bits(o), lse.cpu().numpy().astype(np.float64)

    def check(self, seqs, q_lens, o_bits, lse):
        at = 0
        worst = (0.0, 0.0)
        for s, n in zip(seqs, q_lens):
            h = np.asarray(self.hist[s], np.int64)
            ref_o, ref_l = A.attend_sequence(A.bf16_bits_to_f64(self.x.q[h[len(h) - n:]]),
                                             A.bf16_bits_to_f64(self.x.k[h]), A.bf16_bits_to_f64(self.x.v[h]),
                                             self.windows, self.w.scale)
            do = np.abs(A.bf16_bits_to_f64(o_bits[at:at + n]) - ref_o).max()
            dl = np.abs(lse[at:at + n] - ref_l).max()
            worst = (max(worst[0], do), max(worst[1], dl))
            at += n
        say(f"  max|do|={worst[0]:.3e} max|dlse|={worst[1]:.3e}")
        assert worst[0] <= O_TOL and worst[1] <= LSE_TOL

    def close(self):
        self.canary.check()
        self.kv.close()


@pytest.mark.parametrize("case", [
    # hq, hkv, d, page, windows, parent_len, children (n_new, n_query)
    (16, 4, 128, 64, (0, 100, 300, 64), 1000, [(200, 200), (1, 1), (77, 3), (64, 64)]),
    (8, 2, 64, 16, (0, 20), 333, [(50, 50), (5, 5), (16, 1)]),
    (32, 8, 128, 32, (0, 512, 512, 512, 512, 512, 512, 512), 2048, [(300, 300), (300, 300)]),
])
def test_forks_append_and_attend_over_parent_plus_own_tokens(case):
    hq, hkv, d, p, windows, parent_len, children = case
    say(f"fork hq={hq} hkv={hkv} d={d} p={p} W={windows} parent={parent_len} children={children}")
    n_tok = parent_len + sum(n for n, _ in children) + 8
    sc = Scenario(hq, hkv, d, p, windows, n_tok, 1 + len(children), seed=parent_len + d)
    sc.append([0], [parent_len], [1])
    pre = sc.decode([0])
    sc.check([0], [1], *pre)
    for i in range(len(children)):
        sc.fork(0, 1 + i)
    ids = list(range(1, 1 + len(children)))
    sc.append(ids, [n for n, _ in children], [q for _, q in children])
    o, lse = sc.prefill(ids, [q for _, q in children])
    sc.check(ids, [q for _, q in children], o, lse)
    post = sc.decode([0])
    assert np.array_equal(pre[0], post[0]) and np.array_equal(pre[1], post[1])
    od, ld = sc.decode(ids)
    sc.check(ids, [1] * len(ids), od, ld)
    sc.close()


def test_fork_of_a_fork_and_parent_appends_after_forks():
    sc = Scenario(8, 2, 128, 16, (0, 40), 1200, 4, seed=3)
    sc.append([0], [250], [0])
    sc.fork(0, 1)
    sc.append([1], [30], [30])      # child copies the shared tail (250 % 16 = 10 tokens)
    sc.fork(1, 2)                   # grandchild shares the child's private tail
    sc.append([0], [20], [20])      # parent writes its own copy of the tail
    sc.append([2], [7], [7])
    sc.append([1], [3], [3])
    o, lse = sc.prefill([0, 1, 2], [20, 3, 7])
    sc.check([0, 1, 2], [20, 3, 7], o, lse)
    sc.kv.release(1)                # the grandchild keeps the pages it shares with the released child
    sc.append([2], [1], [1])
    o, lse = sc.prefill([2], [1])
    sc.check([2], [1], o, lse)
    sc.close()


def test_many_forks_share_the_parent_pages():
    sc = Scenario(16, 4, 128, 64, (0, 256, 256, 256), 4096 + 40, 9, seed=11)
    sc.append([0], [4096], [0])
    used0 = sc.kv.num_pages - sc.kv.free_pages()
    for i in range(1, 9):
        sc.fork(0, i)
    assert sc.kv.num_pages - sc.kv.free_pages() == used0
    sc.append(list(range(1, 9)), [5] * 8, [5] * 8)
    used = sc.kv.num_pages - sc.kv.free_pages()
    # 4096 is page-aligned: each fork adds one new page per KV head, nothing is copied
    assert used == used0 + 8 * 4
    o, lse = sc.prefill(list(range(1, 9)), [5] * 8)
    sc.check(list(range(1, 9)), [5] * 8, o, lse)
    sc.close()
