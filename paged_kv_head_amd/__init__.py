"""Paged MLA decode for AMD Instinct MI355X (gfx950).

Thin ctypes binding over ``libmla_decode.so`` (C ABI in
``include/mla_decode.h``).  Function names match the C entry points; the
wrappers only marshal arguments (torch tensors -> device pointers, the
current HIP stream) and turn nonzero statuses into exceptions.  Every step of
the computation runs in the library's HIP kernels; there is no fallback.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

__all__ = [
    "MLA_KV_BF16", "MLA_KV_FP8_656", "MLA_FLAG_NATURAL_BASE", "MlaError", "Problem",
    "library_path", "mla_decode_num_units", "mla_decode_num_parts", "mla_decode_metadata_size",
    "mla_decode_workspace_bytes", "mla_decode_get_metadata", "mla_decode_paged",
    "mla_decode_paged_fp8", "mla_decode_sparse_fp8", "mla_decode_combine", "mla_last_error",
    "mla_decode_with_kvcache", "mla_kv_quantize_fp8", "mla_sparse_prefill_workspace_bytes",
    "mla_sparse_prefill", "mla_sparse_prefill_num_parts", "mla_decode_check_inputs",
    "mla_decode_kernel_name", "mla_clock_probe", "shader_clock_mhz", "problem_for",
    "workload_tensors", "mla_decode_paged_noalloc", "NOALLOC_SCRATCH_BYTES", "IndexProblem",
    "mla_fp8_index_workspace_bytes", "mla_fp8_index_top_k", "index_problem_for", "index_tensors",
    "mla_fp8_index_scores", "mla_fp8_index_select",
]

MLA_KV_BF16 = 0
MLA_KV_FP8_656 = 1
MLA_FLAG_NATURAL_BASE = 1

MLA_OK = 0
MLA_ERR_INVALID_ARGUMENT = 1
MLA_ERR_UNSUPPORTED = 2
MLA_ERR_WORKSPACE_TOO_SMALL = 3
MLA_ERR_HIP = 4

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libmla_decode.so")


class MlaError(RuntimeError):
    """A nonzero status from the library; ``status`` holds the code."""

    def __init__(self, status: int, message: str):
        super().__init__(f"[mla status {status}] {message}")
        self.status = status


class Problem(ctypes.Structure):
    """Mirror of ``mla_problem``."""

    _fields_ = [
        ("batch", ctypes.c_int32), ("s_q", ctypes.c_int32), ("h_q", ctypes.c_int32),
        ("h_kv", ctypes.c_int32), ("d_qk", ctypes.c_int32), ("d_v", ctypes.c_int32),
        ("page_size", ctypes.c_int32), ("num_pages", ctypes.c_int32),
        ("max_pages_per_seq", ctypes.c_int32), ("topk", ctypes.c_int32),
        ("kv_format", ctypes.c_int32), ("is_causal", ctypes.c_int32), ("flags", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float),
    ]

    @classmethod
    def make(cls, *, batch, s_q, h_q, num_pages, max_pages_per_seq, softmax_scale, topk=0,
             kv_format=MLA_KV_BF16, is_causal=0, flags=0, h_kv=1, d_qk=576, d_v=512,
             page_size=64) -> "Problem":
        return cls(batch, s_q, h_q, h_kv, d_qk, d_v, page_size, num_pages, max_pages_per_seq,
                   topk, kv_format, is_causal, flags, float(softmax_scale))


class IndexProblem(ctypes.Structure):
    """Mirror of ``mla_index_problem`` (FP8 top-k indexer)."""

    _fields_ = [(n, ctypes.c_int32) for n in ("batch", "s_q", "h", "d", "page_size", "num_pages",
                                              "max_pages_per_seq", "topk", "kpool", "is_causal")]

    @classmethod
    def make(cls, *, batch, s_q, h, num_pages, max_pages_per_seq, topk, kpool=1, is_causal=0,
             d=512, page_size=64) -> "IndexProblem":
        return cls(batch, s_q, h, d, page_size, num_pages, max_pages_per_seq, topk, kpool, is_causal)


_lib = None


def library_path() -> str:
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise ImportError(
            f"libmla_decode.so is not built ({_LIB_PATH}); run paged_kv_head_amd/build.py")
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    PP = ctypes.POINTER(Problem)
    I32 = ctypes.c_int32
    SZ = ctypes.c_size_t
    lib.mla_decode_num_units.argtypes = [PP]
    lib.mla_decode_num_units.restype = I32
    lib.mla_decode_num_parts.argtypes = [PP, ctypes.c_int, ctypes.POINTER(I32)]
    lib.mla_decode_metadata_size.argtypes = [PP, I32, ctypes.POINTER(SZ), ctypes.POINTER(SZ)]
    lib.mla_decode_workspace_bytes.argtypes = [PP, I32, ctypes.POINTER(SZ)]
    lib.mla_decode_get_metadata.argtypes = [PP, P, I32, P, P, P]
    lib.mla_decode_paged.argtypes = [PP, P, P, P, P, P, P, I32, P, P, SZ, P, P, P]
    lib.mla_decode_paged_fp8.argtypes = [PP, P, P, P, P, P, I32, P, P, SZ, P, P, P]
    lib.mla_decode_sparse_fp8.argtypes = [PP, P, P, P, P, P, P, I32, P, P, SZ, P, P, P]
    lib.mla_decode_combine.argtypes = [PP, I32, P, P, SZ, P, P, P]
    lib.mla_decode_paged_noalloc.argtypes = [PP, P, P, P, P, P, P, I32, P, P, P, P]
    IP = ctypes.POINTER(IndexProblem)
    lib.mla_fp8_index_workspace_bytes.argtypes = [IP, ctypes.POINTER(SZ)]
    lib.mla_fp8_index_top_k.argtypes = [IP, P, P, P, P, P, P, SZ, P, P, P]
    lib.mla_fp8_index_scores.argtypes = [IP, P, P, P, P, P, P, SZ, P]
    lib.mla_fp8_index_select.argtypes = [IP, P, P, SZ, P, P, P]
    lib.mla_kv_quantize_fp8.argtypes = [I32, I32, I32, I32, I32, P, P, P, P, P]
    lib.mla_decode_check_inputs.argtypes = [PP, P, P, P, P]
    lib.mla_sparse_prefill_workspace_bytes.argtypes = [I32, I32, I32, I32, I32, I32, ctypes.POINTER(SZ)]
    lib.mla_sparse_prefill.argtypes = [I32, I32, I32, I32, I32, I32, ctypes.c_float, P, P, P, I32, P,
                                       SZ, P, P, P]
    for fn in ("mla_decode_num_parts", "mla_decode_metadata_size", "mla_decode_workspace_bytes",
               "mla_decode_get_metadata", "mla_decode_paged", "mla_decode_paged_fp8",
               "mla_decode_sparse_fp8", "mla_decode_combine", "mla_kv_quantize_fp8",
               "mla_sparse_prefill_workspace_bytes", "mla_sparse_prefill",
               "mla_decode_check_inputs", "mla_decode_paged_noalloc",
               "mla_fp8_index_workspace_bytes", "mla_fp8_index_top_k", "mla_fp8_index_scores",
               "mla_fp8_index_select"):
        getattr(lib, fn).restype = ctypes.c_int
    lib.mla_last_error.argtypes = []
    lib.mla_last_error.restype = ctypes.c_char_p
    lib.mla_decode_kernel_name.argtypes = [PP]
    lib.mla_decode_kernel_name.restype = ctypes.c_char_p
    lib.mla_clock_probe.argtypes = [P, I32, I32, P]
    lib.mla_clock_probe.restype = ctypes.c_int
    _lib = lib
    return lib


def mla_last_error() -> str:
    return _load().mla_last_error().decode()


def _check(status: int) -> None:
    """Invalid arguments raise ValueError (the message names the argument);
    every other failure raises MlaError."""
    if status == MLA_OK:
        return
    msg = mla_last_error()
    if status == MLA_ERR_INVALID_ARGUMENT:
        raise ValueError(msg)
    raise MlaError(status, msg)


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch.Tensor")
    if t.numel() > 0 and not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return ctypes.c_void_p(t.data_ptr()) if t.data_ptr() else None


def _expect(name, t, dtype, numel, at_least=False):
    if t is None:
        raise ValueError(f"{name}: missing tensor")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name}: dtype {t.dtype}, expected {dtype}")
    n = t.numel() * t.element_size() if dtype is None else t.numel()
    if (n < numel) if at_least else (n != numel):
        raise ValueError(f"{name}: {n} {'bytes' if dtype is None else 'elements'}, expected "
                         f"{'at least ' if at_least else ''}{numel}")
    if t.device.type != "cuda":
        raise ValueError(f"{name}: must be a device tensor")


def _check_decode_tensors(p: Problem, q, kv_pool, block_table, cache_seqlens, indices, out, lse):
    """Buffer sizes are not visible to the C ABI; check them here so that no
    kernel can be handed a buffer smaller than the problem says."""
    rows = p.batch * p.s_q * p.h_q
    _expect("q", q, torch.bfloat16, rows * 576)
    row_bytes = 1152 if p.kv_format == MLA_KV_BF16 else 656
    _expect("kv_pool", kv_pool, None, p.num_pages * p.page_size * row_bytes)
    _expect("block_table", block_table, torch.int32, p.batch * p.max_pages_per_seq)
    _expect("cache_seqlens", cache_seqlens, torch.int32, p.batch)
    if p.topk > 0:
        _expect("indices", indices, torch.int32, p.batch * p.s_q * p.topk)
    _expect("out", out, torch.bfloat16, rows * 512)
    _expect("lse", lse, torch.float32, rows)


def _check_meta_tensors(p: Problem, num_parts, sched, num_splits):
    n_sched, n_splits = mla_decode_metadata_size(p, num_parts)
    _expect("sched", sched, torch.int32, n_sched, at_least=True)
    _expect("num_splits", num_splits, torch.int32, n_splits, at_least=True)


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def problem_for(w, *, natural: bool = False, softmax_scale=None) -> Problem:
    """``Problem`` of a workload object (attributes batch, s_q, h_q,
    num_pages, max_pages_per_seq, softmax_scale, topk, kv_format, is_causal),
    optionally with another scale or the natural base."""
    return Problem.make(
        batch=w.batch, s_q=w.s_q, h_q=w.h_q, num_pages=w.num_pages,
        max_pages_per_seq=w.max_pages_per_seq,
        softmax_scale=w.softmax_scale if softmax_scale is None else softmax_scale,
        topk=w.topk, kv_format=w.kv_format, is_causal=w.is_causal,
        flags=MLA_FLAG_NATURAL_BASE if natural else 0)


def workload_tensors(w, device="cuda"):
    """Device tensors of a workload's host arrays: (q bf16, kv_pool uint8,
    block_table int32, cache_seqlens int32, indices int32 or None)."""
    import numpy as np

    dev = torch.device(device)
    q = torch.from_numpy(np.ascontiguousarray(w.q).view(np.int16)).to(dev).view(torch.bfloat16)
    kv = torch.from_numpy(np.ascontiguousarray(w.kv)).to(dev)
    bt = torch.from_numpy(np.ascontiguousarray(w.block_table)).to(dev)
    sl = torch.from_numpy(np.ascontiguousarray(w.cache_seqlens)).to(dev)
    idx = None if w.indices is None else torch.from_numpy(np.ascontiguousarray(w.indices)).to(dev)
    return q, kv, bt, sl, idx


def index_problem_for(w) -> IndexProblem:
    """``IndexProblem`` of an indexer workload (attributes batch, s_q, h,
    num_pages, max_pages_per_seq, topk, kpool, is_causal)."""
    return IndexProblem.make(batch=w.batch, s_q=w.s_q, h=w.h, num_pages=w.num_pages,
                             max_pages_per_seq=w.max_pages_per_seq, topk=w.topk, kpool=w.kpool,
                             is_causal=w.is_causal)


def index_tensors(w, device="cuda"):
    """Device tensors of an indexer workload: (q codes uint8, q scales
    float32, kv_pool uint8, block_table int32, cache_seqlens int32)."""
    import numpy as np

    dev = torch.device(device)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    return t(w.q_codes), t(w.q_scales), t(w.kv), t(w.block_table), t(w.cache_seqlens)


def mla_fp8_index_workspace_bytes(p: IndexProblem) -> int:
    n = ctypes.c_size_t(0)
    _check(_load().mla_fp8_index_workspace_bytes(ctypes.byref(p), ctypes.byref(n)))
    return int(n.value)


def mla_fp8_index_top_k(p: IndexProblem, q_fp8, q_scale, kv_pool, block_table, cache_seqlens,
                        workspace, indices, scores=None, stream=None):
    """FP8 top-k indexer: per query token the top-k visible cache rows by the
    head-summed FP8 score, in ascending row order, -1 fill (see mla_index.h)."""
    tokens = p.batch * p.s_q
    _expect("q_fp8", q_fp8, torch.uint8, tokens * p.h * 512)
    _expect("q_scale", q_scale, torch.float32, tokens * p.h * 4)
    _expect("kv_pool", kv_pool, None, p.num_pages * p.page_size * 656)
    _expect("block_table", block_table, torch.int32, p.batch * p.max_pages_per_seq)
    _expect("cache_seqlens", cache_seqlens, torch.int32, p.batch)
    _expect("indices", indices, torch.int32, tokens * p.topk)
    if scores is not None:
        _expect("scores", scores, torch.float32, tokens * p.topk)
    _expect("workspace", workspace, None, mla_fp8_index_workspace_bytes(p), at_least=True)
    _check(_load().mla_fp8_index_top_k(
        ctypes.byref(p), _ptr(q_fp8), _ptr(q_scale), _ptr(kv_pool), _ptr(block_table),
        _ptr(cache_seqlens), _ptr(workspace), workspace.numel() * workspace.element_size(),
        _ptr(indices), _ptr(scores), _stream(stream)))


def mla_fp8_index_scores(p: IndexProblem, q_fp8, q_scale, kv_pool, block_table, cache_seqlens,
                         workspace, stream=None):
    """Score phase of the indexer: fp32 scores [B, s_q, 64 * max_pages_per_seq]
    into ``workspace`` (rows that are not visible: unspecified)."""
    tokens = p.batch * p.s_q
    _expect("q_fp8", q_fp8, torch.uint8, tokens * p.h * 512)
    _expect("q_scale", q_scale, torch.float32, tokens * p.h * 4)
    _expect("kv_pool", kv_pool, None, p.num_pages * p.page_size * 656)
    _expect("block_table", block_table, torch.int32, p.batch * p.max_pages_per_seq)
    _expect("cache_seqlens", cache_seqlens, torch.int32, p.batch)
    _expect("workspace", workspace, None, mla_fp8_index_workspace_bytes(p), at_least=True)
    _check(_load().mla_fp8_index_scores(
        ctypes.byref(p), _ptr(q_fp8), _ptr(q_scale), _ptr(kv_pool), _ptr(block_table),
        _ptr(cache_seqlens), _ptr(workspace), workspace.numel() * workspace.element_size(),
        _stream(stream)))


def mla_fp8_index_select(p: IndexProblem, cache_seqlens, workspace, indices, scores=None, stream=None):
    """Selection phase of the indexer, from a workspace the score phase filled."""
    tokens = p.batch * p.s_q
    _expect("cache_seqlens", cache_seqlens, torch.int32, p.batch)
    _expect("indices", indices, torch.int32, tokens * p.topk)
    if scores is not None:
        _expect("scores", scores, torch.float32, tokens * p.topk)
    _expect("workspace", workspace, None, mla_fp8_index_workspace_bytes(p), at_least=True)
    _check(_load().mla_fp8_index_select(
        ctypes.byref(p), _ptr(cache_seqlens), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _ptr(indices), _ptr(scores), _stream(stream)))


def mla_decode_kernel_name(p: Problem) -> str:
    """Name of the kernel mla_decode_paged launches for this problem."""
    name = _load().mla_decode_kernel_name(ctypes.byref(p))
    if name is None:
        _check(MLA_ERR_INVALID_ARGUMENT)
    return name.decode()


def mla_clock_probe(out, workgroups: int, spins: int, stream=None):
    """Enqueue the shader-clock probe; ``out`` is a device int64 tensor of
    2 * workgroups elements (cycles, 100 MHz ticks per workgroup)."""
    _expect("out", out, torch.int64, 2 * workgroups, at_least=True)
    _check(_load().mla_clock_probe(_ptr(out), int(workgroups), int(spins), _stream(stream)))


def shader_clock_mhz(device="cuda", workgroups: int = 256, spins: int = 20000) -> float:
    """Median shader clock (MHz) of the workgroups of one probe launch with
    the matrix cores busy; synchronises the device."""
    out = torch.zeros(2 * workgroups, dtype=torch.int64, device=device)
    mla_clock_probe(out, workgroups, spins)
    torch.cuda.synchronize()
    v = out.view(workgroups, 2).cpu().double()
    ratio = (v[:, 0] / v[:, 1].clamp(min=1)).median().item()
    return 100.0 * ratio


def mla_decode_num_units(p: Problem) -> int:
    return int(_load().mla_decode_num_units(ctypes.byref(p)))


def mla_decode_num_parts(p: Problem, device: int = 0) -> int:
    n = ctypes.c_int32(0)
    _check(_load().mla_decode_num_parts(ctypes.byref(p), int(device), ctypes.byref(n)))
    return int(n.value)


def mla_decode_metadata_size(p: Problem, num_parts: int) -> Tuple[int, int]:
    a, b = ctypes.c_size_t(0), ctypes.c_size_t(0)
    _check(_load().mla_decode_metadata_size(ctypes.byref(p), int(num_parts), ctypes.byref(a), ctypes.byref(b)))
    return int(a.value), int(b.value)


def mla_decode_workspace_bytes(p: Problem, num_parts: int) -> int:
    n = ctypes.c_size_t(0)
    _check(_load().mla_decode_workspace_bytes(ctypes.byref(p), int(num_parts), ctypes.byref(n)))
    return int(n.value)


def mla_decode_get_metadata(p: Problem, cache_seqlens, num_parts, sched, num_splits, stream=None):
    _expect("cache_seqlens", cache_seqlens, torch.int32, p.batch)
    _check_meta_tensors(p, num_parts, sched, num_splits)
    _check(_load().mla_decode_get_metadata(ctypes.byref(p), _ptr(cache_seqlens), int(num_parts),
                                           _ptr(sched), _ptr(num_splits), _stream(stream)))


def mla_decode_paged(p: Problem, q, kv_pool, block_table, cache_seqlens, indices, sched, num_parts,
                     num_splits, workspace, out, lse, stream=None):
    _check_decode_tensors(p, q, kv_pool, block_table, cache_seqlens, indices, out, lse)
    _check_meta_tensors(p, num_parts, sched, num_splits)
    _check(_load().mla_decode_paged(
        ctypes.byref(p), _ptr(q), _ptr(kv_pool), _ptr(block_table), _ptr(cache_seqlens),
        _ptr(indices), _ptr(sched), int(num_parts), _ptr(num_splits), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _ptr(out), _ptr(lse), _stream(stream)))


def mla_decode_paged_fp8(p: Problem, q, kv_pool, block_table, cache_seqlens, sched, num_parts,
                         num_splits, workspace, out, lse, stream=None):
    _check_decode_tensors(p, q, kv_pool, block_table, cache_seqlens, None, out, lse)
    _check_meta_tensors(p, num_parts, sched, num_splits)
    _check(_load().mla_decode_paged_fp8(
        ctypes.byref(p), _ptr(q), _ptr(kv_pool), _ptr(block_table), _ptr(cache_seqlens),
        _ptr(sched), int(num_parts), _ptr(num_splits), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _ptr(out), _ptr(lse), _stream(stream)))


def mla_decode_sparse_fp8(p: Problem, q, kv_pool, block_table, cache_seqlens, indices, sched,
                          num_parts, num_splits, workspace, out, lse, stream=None):
    _check_decode_tensors(p, q, kv_pool, block_table, cache_seqlens, indices, out, lse)
    _check_meta_tensors(p, num_parts, sched, num_splits)
    _check(_load().mla_decode_sparse_fp8(
        ctypes.byref(p), _ptr(q), _ptr(kv_pool), _ptr(block_table), _ptr(cache_seqlens),
        _ptr(indices), _ptr(sched), int(num_parts), _ptr(num_splits), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _ptr(out), _ptr(lse), _stream(stream)))


# Bytes of the library's static scratch behind mla_decode_paged_noalloc.
NOALLOC_SCRATCH_BYTES = 96 << 20


def mla_decode_paged_noalloc(p: Problem, q, kv_pool, block_table, cache_seqlens, indices, sched,
                             num_parts, num_splits, out, lse, stream=None):
    """Decode and combine in one call with no workspace: the split partials
    live in the library's static per-GPU scratch (calls that overlap on one
    GPU race)."""
    _check_decode_tensors(p, q, kv_pool, block_table, cache_seqlens, indices, out, lse)
    _check_meta_tensors(p, num_parts, sched, num_splits)
    _check(_load().mla_decode_paged_noalloc(
        ctypes.byref(p), _ptr(q), _ptr(kv_pool), _ptr(block_table), _ptr(cache_seqlens),
        _ptr(indices), _ptr(sched), int(num_parts), _ptr(num_splits), _ptr(out), _ptr(lse),
        _stream(stream)))


def mla_decode_combine(p: Problem, num_parts, num_splits, workspace, out, lse, stream=None):
    rows = p.batch * p.s_q * p.h_q
    _expect("out", out, torch.bfloat16, rows * 512)
    _expect("lse", lse, torch.float32, rows)
    _expect("num_splits", num_splits, torch.int32, mla_decode_metadata_size(p, num_parts)[1], at_least=True)
    _check(_load().mla_decode_combine(
        ctypes.byref(p), int(num_parts), _ptr(num_splits), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _ptr(out), _ptr(lse), _stream(stream)))


def mla_decode_check_inputs(p: Problem, block_table, cache_seqlens, stream=None) -> Tuple[int, int]:
    """Checks cache lengths and the reachable block-table entries on the
    device; returns (number of bad sequences, first bad sequence or -1).
    Synchronises the stream to read the answer."""
    _expect("block_table", block_table, torch.int32, p.batch * p.max_pages_per_seq)
    _expect("cache_seqlens", cache_seqlens, torch.int32, p.batch)
    res = torch.empty(2, dtype=torch.int32, device=cache_seqlens.device)
    _check(_load().mla_decode_check_inputs(ctypes.byref(p), _ptr(block_table), _ptr(cache_seqlens),
                                           _ptr(res), _stream(stream)))
    r = res.cpu()
    return int(r[0]), int(r[1])


def mla_kv_quantize_fp8(kv_new, start_pos, block_table, kv_pool, page_size: int = 64,
                        stream=None):
    """Quantise kv_new (bf16 [B, n_new, 576]) into the 656-byte FP8 rows of
    kv_pool (uint8 [num_pages, page_size, 656], written in place) at logical
    positions start_pos[b] + j through block_table (int32 [B, max_pages])."""
    if kv_new.dim() != 3 or kv_new.shape[2] != 576:
        raise ValueError(f"kv_new: shape {tuple(kv_new.shape)}, expected [B, n_new, 576]")
    B, n_new, _ = kv_new.shape
    if block_table.dim() != 2 or block_table.shape[0] != B:
        raise ValueError(f"block_table: shape {tuple(block_table.shape)}, expected [{B}, max_pages]")
    if kv_pool.dim() != 3 or kv_pool.shape[1] != page_size or kv_pool.shape[2] != 656:
        raise ValueError(f"kv_pool: shape {tuple(kv_pool.shape)}, expected [num_pages, {page_size}, 656]")
    _expect("kv_new", kv_new, torch.bfloat16, B * n_new * 576)
    _expect("start_pos", start_pos, torch.int32, B)
    _expect("block_table", block_table, torch.int32, block_table.numel())
    _expect("kv_pool", kv_pool, torch.uint8, kv_pool.numel())
    _check(_load().mla_kv_quantize_fp8(
        int(B), int(n_new), int(page_size), int(kv_pool.shape[0]), int(block_table.shape[1]),
        _ptr(kv_new), _ptr(start_pos), _ptr(block_table), _ptr(kv_pool), _stream(stream)))


def mla_sparse_prefill_num_parts(h_q: int, topk: int, kv_format: int = MLA_KV_BF16,
                                 device: int = 0) -> int:
    """Parts that fill the GPU for a sparse prefill with h_q heads."""
    p = Problem.make(batch=1, s_q=1, h_q=h_q, num_pages=1, max_pages_per_seq=1, softmax_scale=1.0,
                     topk=topk, kv_format=kv_format)
    return mla_decode_num_parts(p, device)


def mla_sparse_prefill_workspace_bytes(s_q, h_q, s_kv, topk, kv_format, num_parts) -> int:
    n = ctypes.c_size_t(0)
    _check(_load().mla_sparse_prefill_workspace_bytes(int(s_q), int(h_q), int(s_kv), int(topk),
                                                      int(kv_format), int(num_parts), ctypes.byref(n)))
    return int(n.value)


def mla_sparse_prefill(q, kv, indices, softmax_scale, *, kv_format=MLA_KV_BF16, natural_base=False,
                       num_parts=None, workspace=None, out=None, lse=None, stream=None):
    """Sparse prefill over a flat latent cache.  q bf16 [s_q, h_q, 576];
    kv [s_kv, 576] bf16 or [s_kv, 656] uint8 (MLA_KV_FP8_656); indices int32
    [s_q, topk].  Returns (out bf16 [s_q, h_q, 512], lse float32 [s_q, h_q])."""
    if q.dim() != 3 or q.shape[2] != 576:
        raise ValueError(f"q: shape {tuple(q.shape)}, expected [s_q, h_q, 576]")
    s_q, h_q = int(q.shape[0]), int(q.shape[1])
    if indices.dim() != 2 or indices.shape[0] != s_q:
        raise ValueError(f"indices: shape {tuple(indices.shape)}, expected [{s_q}, topk]")
    topk = int(indices.shape[1])
    row_bytes = 1152 if kv_format == MLA_KV_BF16 else 656
    kv_bytes = kv.numel() * kv.element_size()
    if kv.dim() < 1 or kv_bytes % row_bytes or kv.shape[0] * row_bytes != kv_bytes:
        raise ValueError(f"kv: shape {tuple(kv.shape)} is not [s_kv, {row_bytes} bytes]")
    s_kv = int(kv.shape[0])
    _expect("q", q, torch.bfloat16, s_q * h_q * 576)
    _expect("kv", kv, None, s_kv * row_bytes)
    _expect("indices", indices, torch.int32, s_q * topk)
    if num_parts is None:
        num_parts = mla_sparse_prefill_num_parts(h_q, topk, kv_format, q.device.index or 0)
    need = mla_sparse_prefill_workspace_bytes(s_q, h_q, s_kv, topk, kv_format, num_parts)
    if workspace is None:
        workspace = torch.empty(max(256, need), dtype=torch.uint8, device=q.device)
    if workspace.numel() and workspace.data_ptr() % 256:
        raise ValueError("workspace: must be 256-byte aligned")
    _expect("workspace", workspace, torch.uint8, need, at_least=True)
    if out is None:
        out = torch.empty((s_q, h_q, 512), dtype=torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty((s_q, h_q), dtype=torch.float32, device=q.device)
    _expect("out", out, torch.bfloat16, s_q * h_q * 512)
    _expect("lse", lse, torch.float32, s_q * h_q)
    _check(_load().mla_sparse_prefill(
        s_q, h_q, s_kv, topk, int(kv_format), MLA_FLAG_NATURAL_BASE if natural_base else 0,
        float(softmax_scale), _ptr(q), _ptr(kv), _ptr(indices), int(num_parts), _ptr(workspace),
        workspace.numel(), _ptr(out), _ptr(lse), _stream(stream)))
    return out, lse


class DecodePlan:
    """Device buffers for one problem shape: metadata and workspace.

    Allocated once (torch caching allocator) and reused across layers and
    steps: ``metadata`` enqueues the scheduler once per decode step,
    ``decode`` enqueues decode and combine (per layer) on the stream.
    """

    def __init__(self, p: Problem, device="cuda", num_parts: Optional[int] = None):
        self.p = p
        dev = torch.device(device)
        self.num_parts = num_parts if num_parts is not None else mla_decode_num_parts(p, dev.index or 0)
        n_sched, n_splits = mla_decode_metadata_size(p, self.num_parts)
        self.sched = torch.empty(n_sched, dtype=torch.int32, device=dev)
        self.num_splits = torch.empty(n_splits, dtype=torch.int32, device=dev)
        ws = mla_decode_workspace_bytes(p, self.num_parts)
        self.workspace = torch.empty(max(16, ws), dtype=torch.uint8, device=dev)

    def metadata(self, cache_seqlens, stream=None):
        mla_decode_get_metadata(self.p, cache_seqlens, self.num_parts, self.sched, self.num_splits, stream)

    def decode(self, q, kv_pool, block_table, cache_seqlens, indices, out, lse, stream=None):
        mla_decode_paged(self.p, q, kv_pool, block_table, cache_seqlens, indices, self.sched,
                         self.num_parts, self.num_splits, self.workspace, out, lse, stream)
        mla_decode_combine(self.p, self.num_parts, self.num_splits, self.workspace, out, lse, stream)


def mla_decode_with_kvcache(q, kv_pool, block_table, cache_seqlens, softmax_scale, *,
                            is_causal=False, kv_format=MLA_KV_BF16, indices=None,
                            natural_base=False, num_parts=None, out=None, lse=None):
    """One-call decode: metadata, decode and combine on the current stream.

    q bf16 [B, s_q, h_q, 576]; kv_pool uint8/bf16 [num_pages, 64, row]
    (row = 576 bf16, or 656 bytes for MLA_KV_FP8_656); block_table int32
    [B, max_pages]; cache_seqlens int32 [B]; indices int32 [B, s_q, topk] or
    None.  Returns (out bf16 [B, s_q, h_q, 512], lse float32 [B, s_q, h_q]).
    """
    B, s_q, h_q, _ = q.shape
    topk = 0 if indices is None else int(indices.shape[-1])
    p = Problem.make(batch=B, s_q=s_q, h_q=h_q, num_pages=int(kv_pool.shape[0]),
                     max_pages_per_seq=int(block_table.shape[1]), softmax_scale=softmax_scale,
                     topk=topk, kv_format=kv_format, is_causal=int(bool(is_causal)),
                     flags=MLA_FLAG_NATURAL_BASE if natural_base else 0)
    plan = DecodePlan(p, q.device, num_parts)
    if out is None:
        out = torch.empty((B, s_q, h_q, 512), dtype=torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty((B, s_q, h_q), dtype=torch.float32, device=q.device)
    plan.metadata(cache_seqlens)
    plan.decode(q, kv_pool, block_table, cache_seqlens, indices, out, lse)
    return out, lse
