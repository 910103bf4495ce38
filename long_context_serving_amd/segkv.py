"""Thin ctypes binding of libsegkv (include/segkv.h).

Argument marshalling only: every step of the attention path runs in the HIP
library.  PyTorch supplies device memory (tensors) and the stream.  The
binding never computes attention itself, and raises if the library has not
been built.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np

from .build import LIB_PATH

SEGKV_OK = 0
SEGKV_E_INVAL = -1
SEGKV_E_NOMEM = -2
SEGKV_E_RANGE = -3
SEGKV_E_DEVICE = -4
SEGKV_E_STATE = -5

KERNEL_SCATTER = 0
KERNEL_PREFILL = 1
KERNEL_DECODE_SPLIT = 2
KERNEL_COMBINE = 3
KERNEL_MERGE = 4
KERNEL_SCORE = 5
KERNEL_SCORE_REDUCE = 6
KERNEL_TOPK = 7
KERNEL_UPLOAD = 8
KERNEL_COUNT = 9

TUNE_DECODE_MIN_PAGES = 0
TUNE_PREFILL_SPLIT_TILES = 1
TUNE_PREFILL_ORDER = 2
TUNE_PREFILL_KERNEL = 3

# Every entry point include/segkv.h declares.
EXPORTED = (
    "segkv_create", "segkv_destroy", "segkv_append_pages", "segkv_prefill", "segkv_decode",
    "segkv_release", "segkv_page_table", "segkv_free_pages", "segkv_set_timing",
    "segkv_read_timing", "segkv_set_tuning", "segkv_last_error", "segkv_set_relocation", "segkv_merge",
    "segkv_fork", "segkv_token_scores", "segkv_topk", "segkv_workspace_bytes", "segkv_decode_noalloc",
)

MERGE_TAKE_A = 0
MERGE_TAKE_B = 1
MERGE_LSE = 2

ROPE_ROTATE_HALF = 0
ROPE_INTERLEAVED = 1


class SegKVError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"segkv error {code}: {msg}")
        self.code = code


class _Config(ctypes.Structure):
    _fields_ = [
        ("num_layers", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("max_seqs", ctypes.c_int32),
        ("num_pages", ctypes.c_int64),
        ("head_window", ctypes.POINTER(ctypes.c_int32)),
        ("softmax_scale", ctypes.c_float),
        ("page_order_seed", ctypes.c_uint64),
        ("k_pool", ctypes.c_void_p),
        ("v_pool", ctypes.c_void_p),
        ("stream", ctypes.c_void_p),
        ("rope_theta", ctypes.c_float),
        ("rope_style", ctypes.c_int32),
        ("rope_dims", ctypes.c_int32),
        ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_uint64),
        ("max_batch_q_tokens", ctypes.c_int32),
        ("pad0", ctypes.c_int32),
    ]


_lib = None


def load_library(path: Optional[str] = None):
    """Load libsegkv.so (built in-tree by long_context_serving_amd.build; the
    environment variable SEGKV_LIBRARY may name another build of it)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or os.environ.get("SEGKV_LIBRARY") or LIB_PATH
    if not os.path.exists(p):
        raise ImportError(f"{p} is missing: build it with `python -m long_context_serving_amd.build` "
                          "(there is no fallback path)")
    lib = ctypes.CDLL(p)
    i32, i64, vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p
    pi32 = ctypes.POINTER(ctypes.c_int32)
    lib.segkv_workspace_bytes.argtypes = [ctypes.POINTER(_Config), i32]
    lib.segkv_workspace_bytes.restype = ctypes.c_size_t
    lib.segkv_create.argtypes = [ctypes.POINTER(_Config), ctypes.POINTER(vp)]
    lib.segkv_create.restype = ctypes.c_int
    lib.segkv_destroy.argtypes = [vp]
    lib.segkv_destroy.restype = None
    lib.segkv_append_pages.argtypes = [vp, i32, i32, pi32, pi32, pi32, vp, vp]
    lib.segkv_append_pages.restype = ctypes.c_int
    lib.segkv_prefill.argtypes = [vp, i32, i32, pi32, pi32, vp, vp, vp]
    lib.segkv_prefill.restype = ctypes.c_int
    lib.segkv_decode.argtypes = [vp, i32, i32, pi32, vp, vp, vp]
    lib.segkv_decode.restype = ctypes.c_int
    lib.segkv_decode_noalloc.argtypes = [vp, i32, i32, pi32, vp, vp, vp]
    lib.segkv_decode_noalloc.restype = ctypes.c_int
    lib.segkv_release.argtypes = [vp, i32]
    lib.segkv_release.restype = ctypes.c_int
    lib.segkv_page_table.argtypes = [vp, i32, i32, i32, pi32, pi32, pi32, pi32, i32]
    lib.segkv_page_table.restype = ctypes.c_int
    lib.segkv_free_pages.argtypes = [vp]
    lib.segkv_free_pages.restype = i64
    lib.segkv_set_timing.argtypes = [vp, i32]
    lib.segkv_set_timing.restype = ctypes.c_int
    lib.segkv_read_timing.argtypes = [vp, i32, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(i64)]
    lib.segkv_read_timing.restype = ctypes.c_int
    lib.segkv_set_tuning.argtypes = [vp, i32, i64]
    lib.segkv_set_tuning.restype = ctypes.c_int
    lib.segkv_token_scores.argtypes = [vp, i32, i32, pi32, pi32, vp, vp, vp]
    lib.segkv_token_scores.restype = ctypes.c_int
    lib.segkv_topk.argtypes = [vp, i32, pi32, vp, pi32, vp]
    lib.segkv_topk.restype = ctypes.c_int
    lib.segkv_fork.argtypes = [vp, i32, i32]
    lib.segkv_fork.restype = ctypes.c_int
    lib.segkv_merge.argtypes = [vp, i64, vp, vp, vp, vp, vp, vp, vp]
    lib.segkv_merge.restype = ctypes.c_int
    lib.segkv_set_relocation.argtypes = [vp, i32, pi32]
    lib.segkv_set_relocation.restype = ctypes.c_int
    lib.segkv_last_error.argtypes = [vp]
    lib.segkv_last_error.restype = ctypes.c_char_p
    if path is None:
        _lib = lib
    return lib


def _i32(xs) -> "ctypes.Array":
    arr = np.ascontiguousarray(np.asarray(xs, dtype=np.int32))
    return arr, arr.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


def bf16_tensor(bits: np.ndarray, device="cuda"):
    """uint16 bf16 bit patterns -> torch.bfloat16 tensor on ``device``."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)
    return t.to(device) if device is not None else t


def bf16_bits(t) -> np.ndarray:
    """torch.bfloat16 tensor -> uint16 bit patterns on the host."""
    import torch
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def _check_dev(t, name, dtype=None):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")


class SegKV:
    """One libsegkv context.

    ``planning=True`` builds a host-only context (allocator and page tables,
    no device pools, no HIP call).  Otherwise K/V pools are allocated with
    torch on the current device unless given: K and V of num_pages * page *
    D bf16 each (pages of K rows and of transposed V rows, in the library's
    own in-page order).  The device workspace is a
    torch uint8 tensor, ``workspace`` if given, else one of
    ``workspace_bytes`` or segkv_workspace_bytes(config, max_batch_q_tokens)
    bytes; the library allocates no device memory of its own.
    """

    def __init__(self, num_layers: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                 page_size: int, max_seqs: int, num_pages: int, head_window: Sequence[int],
                 softmax_scale: float = 0.0, page_order_seed: int = 0, planning: bool = False,
                 k_pool=None, v_pool=None, stream=None, rope_theta: float = 0.0, rope_style: int = 0,
                 rope_dims: int = 0, workspace=None, workspace_bytes: Optional[int] = None,
                 max_batch_q_tokens: int = 16384):
        self._lib = load_library()
        self.num_layers, self.num_q_heads, self.num_kv_heads = num_layers, num_q_heads, num_kv_heads
        self.head_dim, self.page_size, self.max_seqs, self.num_pages = head_dim, page_size, max_seqs, num_pages
        self._win, win_p = _i32(np.asarray(head_window, dtype=np.int32).reshape(-1))
        if num_layers > 0 and num_kv_heads > 0 and self._win.size != num_layers * num_kv_heads:
            raise ValueError(f"head_window must hold num_layers * num_kv_heads = {num_layers * num_kv_heads} entries")
        self.k_pool = self.v_pool = None
        self.stream = None
        cfg = _Config()
        cfg.num_layers, cfg.num_q_heads, cfg.num_kv_heads = num_layers, num_q_heads, num_kv_heads
        cfg.head_dim, cfg.page_size, cfg.max_seqs, cfg.num_pages = head_dim, page_size, max_seqs, num_pages
        cfg.head_window = win_p
        cfg.softmax_scale = softmax_scale
        cfg.page_order_seed = page_order_seed
        cfg.rope_theta, cfg.rope_style, cfg.rope_dims = rope_theta, rope_style, rope_dims
        cfg.max_batch_q_tokens = max_batch_q_tokens
        self.workspace = None
        if not planning:
            import torch
            if k_pool is None:
                k_pool = torch.empty((num_pages, page_size, head_dim), dtype=torch.bfloat16, device="cuda")
            if v_pool is None:
                v_pool = torch.empty((num_pages, head_dim, page_size), dtype=torch.bfloat16, device="cuda")
            _check_dev(k_pool, "k_pool", torch.bfloat16)
            _check_dev(v_pool, "v_pool", torch.bfloat16)
            if k_pool.numel() != num_pages * page_size * head_dim or v_pool.numel() != k_pool.numel():
                raise ValueError("pool sizes do not match num_pages * page_size * head_dim")
            self.k_pool, self.v_pool = k_pool, v_pool
            self.stream = stream if stream is not None else torch.cuda.current_stream()
            cfg.k_pool = k_pool.data_ptr()
            cfg.v_pool = v_pool.data_ptr()
            cfg.stream = self.stream.cuda_stream
            if workspace is None:
                n = workspace_bytes or self._lib.segkv_workspace_bytes(ctypes.byref(cfg), max_batch_q_tokens)
                if n == 0:
                    raise ValueError("invalid configuration (segkv_workspace_bytes returned 0)")
                workspace = torch.empty(int(n), dtype=torch.uint8, device=k_pool.device)
            _check_dev(workspace, "workspace", torch.uint8)
            self.workspace = workspace
            cfg.workspace = workspace.data_ptr()
            cfg.workspace_bytes = workspace.numel()
        self._cfg = cfg
        h = ctypes.c_void_p()
        rc = self._lib.segkv_create(ctypes.byref(cfg), ctypes.byref(h))
        if rc != SEGKV_OK:
            raise SegKVError(rc, self._lib.segkv_last_error(None).decode())
        self._h = h

    # -- plumbing ----------------------------------------------------------
    def _check(self, rc: int):
        if rc != SEGKV_OK:
            raise SegKVError(rc, self.last_error())
        return rc

    @staticmethod
    def workspace_bytes_for(num_layers, num_q_heads, num_kv_heads, head_dim, page_size, max_seqs, num_pages,
                            head_window, max_batch_q_tokens) -> int:
        """segkv_workspace_bytes of a configuration (0 if it is invalid)."""
        lib = load_library()
        win, win_p = _i32(np.asarray(head_window, dtype=np.int32).reshape(-1))
        cfg = _Config()
        cfg.num_layers, cfg.num_q_heads, cfg.num_kv_heads = num_layers, num_q_heads, num_kv_heads
        cfg.head_dim, cfg.page_size, cfg.max_seqs, cfg.num_pages = head_dim, page_size, max_seqs, num_pages
        cfg.head_window = win_p
        return int(lib.segkv_workspace_bytes(ctypes.byref(cfg), max_batch_q_tokens))

    def last_error(self) -> str:
        return self._lib.segkv_last_error(self._h).decode()

    def close(self):
        if getattr(self, "_h", None):
            self._lib.segkv_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    # -- C ABI mirrors -----------------------------------------------------
    def append_pages(self, layer: int, seq_ids, new_lens, n_query, k_new=None, v_new=None) -> int:
        """Append new_lens[b] K/V rows to seq_ids[b]; the last n_query[b]
        become pending queries.  k_new/v_new: bf16 [sum new][Hkv][D] (None in
        a planning-only context)."""
        ids, ids_p = _i32(seq_ids)
        cu, cu_p = _i32(np.concatenate([[0], np.cumsum(np.asarray(new_lens, dtype=np.int64))]))
        nq, nq_p = _i32(n_query)
        if len(nq) != len(ids) or len(cu) != len(ids) + 1:
            raise ValueError("seq_ids, new_lens and n_query must have the same length")
        kp = vp = None
        if k_new is not None or v_new is not None:
            import torch
            for t, name in ((k_new, "k_new"), (v_new, "v_new")):
                _check_dev(t, name, torch.bfloat16)
                if tuple(t.shape) != (int(cu[-1]), self.num_kv_heads, self.head_dim):
                    raise ValueError(f"{name} must be [{int(cu[-1])}, {self.num_kv_heads}, {self.head_dim}]")
            kp, vp = k_new.data_ptr(), v_new.data_ptr()
        return self._check(self._lib.segkv_append_pages(self._h, layer, len(ids), ids_p, cu_p, nq_p, kp, vp))

    def prefill(self, layer: int, seq_ids, q_lens, q, o=None, lse=None, want_lse: bool = True):
        """Varlen prefill; q bf16 [sum q_lens][Hq][D].  Returns (o, lse)."""
        import torch
        ids, ids_p = _i32(seq_ids)
        cu, cu_p = _i32(np.concatenate([[0], np.cumsum(np.asarray(q_lens, dtype=np.int64))]))
        if len(cu) != len(ids) + 1:
            raise ValueError("seq_ids and q_lens must have the same length")
        nq = int(cu[-1])
        _check_dev(q, "q", torch.bfloat16)
        if tuple(q.shape) != (nq, self.num_q_heads, self.head_dim):
            raise ValueError(f"q must be [{nq}, {self.num_q_heads}, {self.head_dim}]")
        if o is None:
            o = torch.empty_like(q)
        _check_dev(o, "o", torch.bfloat16)
        if o.shape != q.shape:
            raise ValueError("o must have q's shape")
        if lse is None and want_lse:
            lse = torch.empty((nq, self.num_q_heads), dtype=torch.float32, device=q.device)
        if lse is not None:
            _check_dev(lse, "lse", torch.float32)
            if tuple(lse.shape) != (nq, self.num_q_heads):
                raise ValueError("lse must be [sum q_lens, Hq]")
        self._check(self._lib.segkv_prefill(self._h, layer, len(ids), ids_p, cu_p, q.data_ptr(), o.data_ptr(),
                                            lse.data_ptr() if lse is not None else None))
        return o, lse

    def token_scores(self, layer: int, seq_ids, q_lens, q, lse, scores=None):
        """Attention mass each query-chunk token receives (fp32 [sum q_lens]);
        q and lse as given to / returned by prefill."""
        import torch
        ids, ids_p = _i32(seq_ids)
        cu, cu_p = _i32(np.concatenate([[0], np.cumsum(np.asarray(q_lens, dtype=np.int64))]))
        if len(cu) != len(ids) + 1:
            raise ValueError("seq_ids and q_lens must have the same length")
        nq = int(cu[-1])
        _check_dev(q, "q", torch.bfloat16)
        _check_dev(lse, "lse", torch.float32)
        if tuple(q.shape) != (nq, self.num_q_heads, self.head_dim) or tuple(lse.shape) != (nq, self.num_q_heads):
            raise ValueError("q must be [sum q_lens, Hq, D] and lse [sum q_lens, Hq]")
        if scores is None:
            scores = torch.empty(nq, dtype=torch.float32, device=q.device)
        _check_dev(scores, "scores", torch.float32)
        if tuple(scores.shape) != (nq,):
            raise ValueError("scores must be [sum q_lens]")
        self._check(self._lib.segkv_token_scores(self._h, layer, len(ids), ids_p, cu_p, q.data_ptr(), lse.data_ptr(),
                                                 scores.data_ptr()))
        return scores

    def topk(self, counts, scores, k, out=None):
        """Top-k indices (ascending, local to each sequence) of each
        sequence's slice of scores; returns int32 [sum k]."""
        import torch
        cu, cu_p = _i32(np.concatenate([[0], np.cumsum(np.asarray(counts, dtype=np.int64))]))
        kk, k_p = _i32(k)
        if len(kk) != len(cu) - 1:
            raise ValueError("counts and k must have the same length")
        _check_dev(scores, "scores", torch.float32)
        if tuple(scores.shape) != (int(cu[-1]),):
            raise ValueError("scores must be [sum counts]")
        total = int(kk.sum())
        if out is None:
            out = torch.empty(total, dtype=torch.int32, device=scores.device)
        _check_dev(out, "out", torch.int32)
        if tuple(out.shape) != (total,):
            raise ValueError("out must be [sum k]")
        self._check(self._lib.segkv_topk(self._h, len(kk), cu_p, scores.data_ptr(), k_p, out.data_ptr()))
        return out

    def decode(self, layer: int, seq_ids, q, o=None, lse=None, want_lse: bool = True, no_alloc: bool = False):
        """One-token decode; q bf16 [n_seqs][Hq][D].  Returns (o, lse).
        ``no_alloc`` calls segkv_decode_noalloc (fixed device scratch); o and
        lse must then be given when wanted, since the binding allocates
        nothing either."""
        import torch
        if no_alloc and (o is None or (lse is None and want_lse)):
            raise ValueError("no_alloc decode needs o (and lse) preallocated")
        ids, ids_p = _i32(seq_ids)
        _check_dev(q, "q", torch.bfloat16)
        if tuple(q.shape) != (len(ids), self.num_q_heads, self.head_dim):
            raise ValueError(f"q must be [{len(ids)}, {self.num_q_heads}, {self.head_dim}]")
        if o is None:
            o = torch.empty_like(q)
        _check_dev(o, "o", torch.bfloat16)
        if lse is None and want_lse:
            lse = torch.empty((len(ids), self.num_q_heads), dtype=torch.float32, device=q.device)
        if lse is not None:
            _check_dev(lse, "lse", torch.float32)
        fn = self._lib.segkv_decode_noalloc if no_alloc else self._lib.segkv_decode
        self._check(fn(self._h, layer, len(ids), ids_p, q.data_ptr(), o.data_ptr(),
                       lse.data_ptr() if lse is not None else None))
        return o, lse

    def merge(self, o_a, lse_a, o_b, lse_b, mode, o=None, lse=None, want_lse: bool = True):
        """Head-decomposition merge: per (row, head) take A, take B or
        log-sum-exp merge (mode uint8 [rows][Hq] of MERGE_*).  o_*: bf16
        [rows][Hq][D], lse_*: fp32 [rows][Hq].  Returns (o, lse)."""
        import torch
        _check_dev(o_a, "o_a", torch.bfloat16)
        rows = o_a.shape[0] if o_a.dim() == 3 else -1
        want = (rows, self.num_q_heads, self.head_dim)
        for t, name, dt, shape in ((o_a, "o_a", torch.bfloat16, want), (o_b, "o_b", torch.bfloat16, want),
                                   (lse_a, "lse_a", torch.float32, want[:2]), (lse_b, "lse_b", torch.float32, want[:2]),
                                   (mode, "mode", torch.uint8, want[:2])):
            _check_dev(t, name, dt)
            if tuple(t.shape) != shape:
                raise ValueError(f"{name} must be {list(shape)}")
        if o is None:
            o = torch.empty_like(o_a)
        _check_dev(o, "o", torch.bfloat16)
        if tuple(o.shape) != want:
            raise ValueError(f"o must be {list(want)}")
        if lse is None and want_lse:
            lse = torch.empty(want[:2], dtype=torch.float32, device=o_a.device)
        if lse is not None:
            _check_dev(lse, "lse", torch.float32)
            if tuple(lse.shape) != want[:2]:
                raise ValueError(f"lse must be {list(want[:2])}")
        self._check(self._lib.segkv_merge(self._h, rows, o_a.data_ptr(), lse_a.data_ptr(), o_b.data_ptr(),
                                          lse_b.data_ptr(), mode.data_ptr(), o.data_ptr(),
                                          lse.data_ptr() if lse is not None else None))
        return o, lse

    def release(self, seq_id: int):
        return self._check(self._lib.segkv_release(self._h, seq_id))

    def fork(self, src_seq: int, dst_seq: int):
        """dst_seq (empty) shares src_seq's tokens and pages (copy-on-write)."""
        return self._check(self._lib.segkv_fork(self._h, src_seq, dst_seq))

    def set_relocation(self, seq_id: int, deltas=None):
        """Query-side RoPE relocation offsets of one sequence: int32
        [num_layers][num_kv_heads] (None = all zero)."""
        if deltas is None:
            return self._check(self._lib.segkv_set_relocation(self._h, seq_id, None))
        d = np.asarray(deltas, dtype=np.int64).reshape(-1)
        if d.size != self.num_layers * self.num_kv_heads:
            raise ValueError(f"deltas must hold num_layers * num_kv_heads = {self.num_layers * self.num_kv_heads}")
        if np.any(np.abs(d) >= 2 ** 31):
            raise ValueError("deltas must fit int32")
        arr, p = _i32(d)
        return self._check(self._lib.segkv_set_relocation(self._h, seq_id, p))

    def page_table(self, layer: int, seq_id: int, kv_head: int):
        """(first_token, kv_len, page ids as int32 numpy array)."""
        ft, kl, n = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
        self._check(self._lib.segkv_page_table(self._h, layer, seq_id, kv_head, ctypes.byref(ft),
                                               ctypes.byref(kl), ctypes.byref(n), None, 0))
        ids = np.zeros(n.value, dtype=np.int32)
        self._check(self._lib.segkv_page_table(self._h, layer, seq_id, kv_head, None, None, None,
                                               ids.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)), n.value))
        return ft.value, kl.value, ids

    def free_pages(self) -> int:
        v = self._lib.segkv_free_pages(self._h)
        if v < 0:
            raise SegKVError(int(v), self.last_error())
        return int(v)

    def set_timing(self, enable, kernels=None):
        """Record HIP events around launches of ``kernels`` (ids KERNEL_*;
        None = all) while ``enable`` is true."""
        if not enable:
            mask = 0
        elif kernels is None:
            mask = (1 << KERNEL_COUNT) - 1
        else:
            mask = 0
            for k in kernels:
                mask |= 1 << int(k)
        return self._check(self._lib.segkv_set_timing(self._h, mask))

    def read_timing(self, kernel: int):
        """(total milliseconds, launches) of one kernel since timing was enabled."""
        ms, n = ctypes.c_double(), ctypes.c_int64()
        self._check(self._lib.segkv_read_timing(self._h, kernel, ctypes.byref(ms), ctypes.byref(n)))
        return ms.value, n.value

    def set_tuning(self, knob: int, value: int):
        return self._check(self._lib.segkv_set_tuning(self._h, knob, int(value)))
