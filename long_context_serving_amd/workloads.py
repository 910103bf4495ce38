"""Seeded synthetic workloads for segmented paged attention.

This module only describes shapes and draws random inputs.  It holds none of
the attention arithmetic, so both the HIP path (through the binding) and the
CPU oracle can take their inputs from it without sharing any of the method.

Recipe (the same for every workload):

* ``rng = numpy.random.default_rng(seed)``;
* draw ``standard_normal`` float32 arrays in the order Q, K, V, shaped
  ``[tokens][heads][head_dim]`` (Q over the query tokens of all sequences,
  K and V over all cached tokens of all sequences, sequences concatenated);
* round each float32 to bfloat16 with round-to-nearest-even and keep the raw
  16-bit patterns (``uint16``).

The shapes follow the layer shapes the pages name for their head statistics
(Mistral-7B, Llama-3.3-70B: "Xiaohongshu Open-Sources RedKnot" page, section
"What Happened", item 1).  Every workload has one global KV head (window 0)
and the rest local, matching the minority-global head split given there.
No dataset or weight is involved.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import Sequence, Tuple

import numpy as np


@dataclass(frozen=True)
class Workload:
    """One synthetic attention layer workload.

    ``kv_lens[b]`` is the cache length of sequence b after its query tokens
    have been appended; its last ``q_lens[b]`` tokens are the queries.  Tokens
    before those (``kv_lens[b] - q_lens[b]``) are a cache fill appended with no
    pending queries.  ``windows[g]`` is the window of KV head g: 0 = global,
    W >= 1 = local with the W most recent tokens.
    """

    name: str
    kv_lens: Tuple[int, ...]
    q_lens: Tuple[int, ...]
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    page_size: int
    windows: Tuple[int, ...]
    seed: int
    decode: bool = False
    description: str = ""

    @property
    def n_seqs(self) -> int:
        return len(self.kv_lens)

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.head_dim))

    @property
    def page_order_seed(self) -> int:
        return self.seed + 100

    def fill_lens(self) -> Tuple[int, ...]:
        return tuple(k - q for k, q in zip(self.kv_lens, self.q_lens))

    def all_global(self) -> "Workload":
        """The comparison arm: same shapes and inputs, every head global."""
        return Workload(self.name + "_all_global", self.kv_lens, self.q_lens,
                        self.num_q_heads, self.num_kv_heads, self.head_dim,
                        self.page_size, tuple(0 for _ in self.windows),
                        self.seed, self.decode, self.description)

    def with_windows(self, windows: Sequence[int]) -> "Workload":
        return Workload(self.name, self.kv_lens, self.q_lens, self.num_q_heads,
                        self.num_kv_heads, self.head_dim, self.page_size,
                        tuple(int(w) for w in windows), self.seed, self.decode,
                        self.description)


def _varlen_lengths() -> Tuple[int, ...]:
    rng = np.random.default_rng(2026)
    return tuple(int(x) for x in rng.integers(8192, 32768, endpoint=True, size=4))


def _local(n: int, w: int) -> Tuple[int, ...]:
    return (0,) + (w,) * (n - 1)


TINY_MHA = Workload(
    "tiny_mha_L512", (512,), (512,), 4, 4, 64, 16, _local(4, 64), seed=1,
    description="1 seq, L=512, 4 heads (1 global, 3 local W=64), D=64, page 16")

MISTRAL7B_PREFILL = Workload(
    "mistral7b_prefill_L8192", (8192,), (8192,), 32, 8, 128, 64,
    _local(8, 1024), seed=2,
    description="1 seq, L=8192, Hq 32 / Hkv 8, D=128, 1 global + 7 local W=1024, page 64")

_VL = _varlen_lengths()
LLAMA70B_VARLEN_PREFILL = Workload(
    "llama70b_varlen_prefill", _VL, _VL, 64, 8, 128, 64, _local(8, 2048), seed=3,
    description="4 seqs, L uniform in [8K,32K] (seed 2026), Hq 64 / Hkv 8, D=128, "
                "1 global + 7 local W=2048, page 64")

DECODE_32K = Workload(
    "decode_32k_x31", (32768,) * 31, (1,) * 31, 64, 8, 128, 64, _local(8, 4096),
    seed=4, decode=True,
    description="31 seqs, 1 query over 32768 cached tokens, Hq 64 / Hkv 8, D=128, "
                "1 global + 7 local W=4096, page 64, split-KV")

CHUNKED_PREFILL_128K = Workload(
    "chunked_prefill_128k", (131072,), (8192,), 32, 8, 128, 64, _local(8, 4096),
    seed=5,
    description="1 seq, 122880 cached + 8192-token query chunk, Hq 32 / Hkv 8, D=128, "
                "1 global + 7 local W=4096, page 64")

WORKLOADS = {w.name: w for w in (TINY_MHA, MISTRAL7B_PREFILL, LLAMA70B_VARLEN_PREFILL,
                                 DECODE_32K, CHUNKED_PREFILL_128K)}


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even.

    Inputs here are finite normals, so no NaN handling is needed; an
    infinity or NaN input raises.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    if not np.all(np.isfinite(x)):
        raise ValueError("bf16 packing expects finite inputs")
    u = x.view(np.uint32)
    rounded = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return rounded.astype(np.uint16)


@dataclass
class Inputs:
    """Raw bf16 bit patterns of one workload (host memory)."""

    q: np.ndarray      # uint16 [sum q_lens][Hq][D]
    k: np.ndarray      # uint16 [sum kv_lens][Hkv][D]
    v: np.ndarray      # uint16 [sum kv_lens][Hkv][D]
    cu_q: np.ndarray   # int64 [n_seqs + 1]
    cu_kv: np.ndarray  # int64 [n_seqs + 1]
    extra: dict = field(default_factory=dict)


def make_inputs(w: Workload, seed: int | None = None, q_scale: float = 1.0) -> Inputs:
    """Draw Q, K, V for workload ``w`` following the module recipe.

    ``q_scale`` multiplies the float32 Q draw before bf16 rounding (a peaky
    softmax stress input); 1.0 is the plain recipe.
    """
    rng = np.random.default_rng(w.seed if seed is None else seed)
    nq = int(sum(w.q_lens))
    nkv = int(sum(w.kv_lens))
    q = rng.standard_normal((nq, w.num_q_heads, w.head_dim), dtype=np.float32)
    if q_scale != 1.0:
        q *= np.float32(q_scale)
    qb = to_bf16_bits(q)
    del q
    k = rng.standard_normal((nkv, w.num_kv_heads, w.head_dim), dtype=np.float32)
    kb = to_bf16_bits(k)
    del k
    v = rng.standard_normal((nkv, w.num_kv_heads, w.head_dim), dtype=np.float32)
    vb = to_bf16_bits(v)
    del v
    cu_q = np.concatenate([[0], np.cumsum(w.q_lens)]).astype(np.int64)
    cu_kv = np.concatenate([[0], np.cumsum(w.kv_lens)]).astype(np.int64)
    return Inputs(qb, kb, vb, cu_q, cu_kv)


def small_workload(name: str, kv_lens, q_lens, hq: int, hkv: int, d: int, p: int,
                   windows, seed: int) -> Workload:
    """A free-form workload for parity sweeps (same recipe, any shape)."""
    return Workload(name, tuple(int(x) for x in kv_lens), tuple(int(x) for x in q_lens),
                    hq, hkv, d, p, tuple(int(x) for x in windows), seed)


# ------------------------------------------------------------ head merge

TAKE_A, TAKE_B, MERGE = 0, 1, 2  # mode bytes of the head-decomposition merge


@dataclass(frozen=True)
class MergeWorkload:
    """Inputs of the head-decomposition merge for one reused document.

    ``rows`` document rows x ``num_q_heads`` heads.  Query heads of the
    KV groups in ``global_kv_heads`` are recomputed online (take B).
    Local heads take the offline partial A except on:

    * protected rows, recomputed online (take B): every row at a
      ``boundary_every``-token boundary, the last ``tail`` rows, the last
      ``query_rows`` rows (query and new tokens) and a seeded
      ``dirty_frac`` fraction (dirty rows and the indexer's top rows).
      This is the protected-row set RedKnot-MLA lists ("RedKnot-MLA:
      Multi-Head Offline-Online Reuse for DeepSeek-V4 Long-Context Serving"
      review, "Strengths");
    * the first ``window - 1`` rows, which in the live request also see
      keys before the document.  Their offline partial is merged (MERGE)
      with an online partial over those keys.

    Partials: o ~ N(0, 0.5^2) rounded to bf16; lse ~ N(ln(keys), 2^2), with
    a seeded ``empty_frac`` of each side set to -inf (a part without keys).
    """

    name: str
    rows: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    window: int
    tail: int
    query_rows: int
    boundary_every: int
    dirty_frac: float
    seed: int
    global_kv_heads: Tuple[int, ...] = (0,)
    empty_frac: float = 0.0

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads


@dataclass
class MergeInputs:
    o_a: np.ndarray    # uint16 bf16 bits [rows][Hq][D]
    lse_a: np.ndarray  # float32 [rows][Hq]
    o_b: np.ndarray
    lse_b: np.ndarray
    mode: np.ndarray   # uint8 [rows][Hq]


def merge_modes(mw: MergeWorkload) -> np.ndarray:
    """Mode byte of every (row, head) following the class docstring."""
    rng = np.random.default_rng(mw.seed + 1)
    protected = np.zeros(mw.rows, bool)
    protected[:: mw.boundary_every] = True
    protected[max(0, mw.rows - mw.tail):] = True
    protected[max(0, mw.rows - mw.query_rows):] = True
    protected |= rng.random(mw.rows) < mw.dirty_frac
    local = np.array([(h // mw.group) not in mw.global_kv_heads for h in range(mw.num_q_heads)])
    mode = np.full((mw.rows, mw.num_q_heads), TAKE_A, np.uint8)
    mode[: max(0, mw.window - 1), :] = MERGE
    mode[protected, :] = TAKE_B
    mode[:, ~local] = TAKE_B
    return mode


def make_merge_inputs(mw: MergeWorkload) -> MergeInputs:
    rng = np.random.default_rng(mw.seed)
    shape = (mw.rows, mw.num_q_heads)
    keys = np.log(np.minimum(np.arange(1, mw.rows + 1), mw.window or mw.rows))[:, None]
    o_a = to_bf16_bits(rng.standard_normal(shape + (mw.head_dim,), dtype=np.float32) * np.float32(0.5))
    o_b = to_bf16_bits(rng.standard_normal(shape + (mw.head_dim,), dtype=np.float32) * np.float32(0.5))
    lse_a = (keys + 2.0 * rng.standard_normal(shape)).astype(np.float32)
    lse_b = (keys + 2.0 * rng.standard_normal(shape)).astype(np.float32)
    if mw.empty_frac > 0:
        lse_a[rng.random(shape) < mw.empty_frac] = -np.inf
        lse_b[rng.random(shape) < mw.empty_frac] = -np.inf
    return MergeInputs(o_a, lse_a, o_b, lse_b, merge_modes(mw))


MERGE_128K = MergeWorkload(
    "merge_128k_doc", rows=131072, num_q_heads=32, num_kv_heads=8, head_dim=128, window=4096,
    tail=32768, query_rows=512, boundary_every=128, dirty_frac=0.02, seed=6)
