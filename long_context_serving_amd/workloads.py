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
