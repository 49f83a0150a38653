"""C-ABI library checks that need no GPU: it loads, exports every symbol the
header declares, and rejects malformed arguments on the host (no device is
touched: the checks run before any HIP call)."""

import ctypes
import os
import re

import pytest

import torch

import paged_kv_head_amd as mla

# These calls pass fake device addresses and rely on the host-side checks
# rejecting them before any launch: run them only where no GPU exists.
pytestmark = pytest.mark.skipif(torch.cuda.is_available(),
                                reason="host-only checks with fake device addresses")

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include",
                      "mla_decode.h")
FAKE = 0x10000  # an aligned non-null address; never dereferenced by these calls


def declared_functions():
    inc = os.path.dirname(HEADER)
    text = "".join(open(os.path.join(inc, f)).read() for f in sorted(os.listdir(inc)) if f.endswith(".h"))
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mla_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for want in ("mla_decode_get_metadata", "mla_decode_paged", "mla_decode_combine",
                 "mla_decode_paged_fp8", "mla_decode_sparse_fp8", "mla_kv_quantize_fp8",
                 "mla_last_error"):
        assert want in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(mla.library_path())
    for name in declared_functions():
        assert hasattr(lib, name), name


def good(**kw):
    d = dict(batch=2, s_q=1, h_q=16, num_pages=7, max_pages_per_seq=5, softmax_scale=1 / 24)
    d.update(kw)
    return mla.Problem.make(**d)


def call_paged(p, **ptrs):
    lib = mla._load()
    a = dict(q=FAKE, kv=FAKE, bt=FAKE, sl=FAKE, idx=None, sched=FAKE, parts=4, splits=FAKE,
             ws=FAKE, ws_bytes=1 << 40, out=FAKE, lse=FAKE)
    a.update(ptrs)
    v = lambda x: None if x is None else ctypes.c_void_p(x)
    return lib.mla_decode_paged(ctypes.byref(p), v(a["q"]), v(a["kv"]), v(a["bt"]), v(a["sl"]),
                                v(a["idx"]), v(a["sched"]), a["parts"], v(a["splits"]), v(a["ws"]),
                                a["ws_bytes"], v(a["out"]), v(a["lse"]), None)


@pytest.mark.parametrize("field,value,status,needle", [
    ("h_kv", 2, mla.MLA_ERR_UNSUPPORTED, "h_kv"),
    ("d_qk", 512, mla.MLA_ERR_UNSUPPORTED, "d_qk"),
    ("d_v", 576, mla.MLA_ERR_UNSUPPORTED, "d_v"),
    ("page_size", 16, mla.MLA_ERR_UNSUPPORTED, "page_size"),
    ("s_q", 0, mla.MLA_ERR_INVALID_ARGUMENT, "s_q"),
    ("h_q", 0, mla.MLA_ERR_INVALID_ARGUMENT, "h_q"),
    ("batch", -1, mla.MLA_ERR_INVALID_ARGUMENT, "batch"),
    ("num_pages", 0, mla.MLA_ERR_INVALID_ARGUMENT, "num_pages"),
    ("max_pages_per_seq", 0, mla.MLA_ERR_INVALID_ARGUMENT, "max_pages_per_seq"),
    ("kv_format", 7, mla.MLA_ERR_INVALID_ARGUMENT, "kv_format"),
    ("is_causal", 2, mla.MLA_ERR_INVALID_ARGUMENT, "is_causal"),
    ("flags", 8, mla.MLA_ERR_INVALID_ARGUMENT, "flags"),
    ("softmax_scale", float("nan"), mla.MLA_ERR_INVALID_ARGUMENT, "softmax_scale"),
    ("softmax_scale", float("inf"), mla.MLA_ERR_INVALID_ARGUMENT, "softmax_scale"),
    ("topk", -3, mla.MLA_ERR_INVALID_ARGUMENT, "topk"),
])
def test_problem_fields_rejected(field, value, status, needle):
    p = good(**{field: value}) if field in ("softmax_scale",) else good()
    if field != "softmax_scale":
        setattr(p, field, value)
    assert call_paged(p) == status
    assert needle in mla.mla_last_error()


def test_sparse_causal_rejected():
    p = good(topk=8, is_causal=1)
    assert call_paged(p, idx=FAKE) == mla.MLA_ERR_INVALID_ARGUMENT
    assert "is_causal" in mla.mla_last_error()


@pytest.mark.parametrize("name", ["q", "kv", "bt", "sl", "sched", "splits", "ws", "out", "lse"])
def test_null_pointer_named(name):
    assert call_paged(good(), **{name: None}) == mla.MLA_ERR_INVALID_ARGUMENT
    err = mla.mla_last_error()
    assert "NULL" in err


@pytest.mark.parametrize("name,label", [("q", "q"), ("kv", "kv_pool"), ("out", "out"), ("ws", "workspace")])
def test_misaligned_pointer_named(name, label):
    assert call_paged(good(), **{name: FAKE + 4}) == mla.MLA_ERR_INVALID_ARGUMENT
    assert mla.mla_last_error().startswith(label)


def test_indices_must_match_topk():
    assert call_paged(good(), idx=FAKE) == mla.MLA_ERR_INVALID_ARGUMENT
    assert "indices" in mla.mla_last_error()
    assert call_paged(good(topk=4), idx=None) == mla.MLA_ERR_INVALID_ARGUMENT
    assert "indices" in mla.mla_last_error()


def test_workspace_too_small():
    p = good()
    need = mla.mla_decode_workspace_bytes(p, 4)
    assert call_paged(p, ws_bytes=need - 1) == mla.MLA_ERR_WORKSPACE_TOO_SMALL
    assert "workspace_bytes" in mla.mla_last_error()


@pytest.mark.parametrize("parts", [0, -1, 65537])
def test_num_parts_range(parts):
    assert call_paged(good(), parts=parts) == mla.MLA_ERR_INVALID_ARGUMENT
    assert "num_parts" in mla.mla_last_error()


def test_named_entry_points_check_format():
    lib = mla._load()
    p = good()  # bf16, dense
    v = ctypes.c_void_p(FAKE)
    st = lib.mla_decode_paged_fp8(ctypes.byref(p), v, v, v, v, v, 4, v, v, 1 << 40, v, v, None)
    assert st == mla.MLA_ERR_INVALID_ARGUMENT and "kv_format" in mla.mla_last_error()
    p = good(kv_format=mla.MLA_KV_FP8_656)
    st = lib.mla_decode_sparse_fp8(ctypes.byref(p), v, v, v, v, v, v, 4, v, v, 1 << 40, v, v, None)
    assert st == mla.MLA_ERR_INVALID_ARGUMENT and "topk" in mla.mla_last_error()


def test_sizes_and_units():
    p = good(batch=3, s_q=2, h_q=128)
    assert mla.mla_decode_num_units(p) == 3
    assert mla.mla_decode_metadata_size(p, 10) == (80, 4)
    p.topk = 64
    assert mla.mla_decode_num_units(p) == 6
    assert mla.mla_decode_metadata_size(p, 10) == (80, 7)
    assert mla.mla_decode_workspace_bytes(p, 10) > 0


def test_python_wrapper_raises_value_error():
    p = good(h_kv=3)
    with pytest.raises(mla.MlaError):
        mla.mla_decode_workspace_bytes(p, 4)
    p = good(s_q=0)
    with pytest.raises(ValueError, match="s_q"):
        mla.mla_decode_workspace_bytes(p, 4)


def test_combine_checks():
    lib = mla._load()
    p = good()
    v = ctypes.c_void_p(FAKE)
    assert lib.mla_decode_combine(ctypes.byref(p), 4, None, v, 1 << 40, v, v, None) == mla.MLA_ERR_INVALID_ARGUMENT
    assert "num_splits" in mla.mla_last_error()
    assert lib.mla_decode_combine(ctypes.byref(p), 4, v, v, 16, v, v, None) == mla.MLA_ERR_WORKSPACE_TOO_SMALL


def call_writer(batch=2, n_new=3, page_size=64, num_pages=7, max_pages=5, kv_new=FAKE,
                start_pos=FAKE, bt=FAKE, pool=FAKE):
    lib = mla._load()
    v = lambda x: None if x is None else ctypes.c_void_p(x)
    return lib.mla_kv_quantize_fp8(batch, n_new, page_size, num_pages, max_pages, v(kv_new),
                                   v(start_pos), v(bt), v(pool), None)


@pytest.mark.parametrize("kw, status, word", [
    (dict(batch=-1), mla.MLA_ERR_INVALID_ARGUMENT, "batch"),
    (dict(n_new=-2), mla.MLA_ERR_INVALID_ARGUMENT, "n_new"),
    (dict(page_size=16), mla.MLA_ERR_UNSUPPORTED, "page_size"),
    (dict(num_pages=0), mla.MLA_ERR_INVALID_ARGUMENT, "num_pages"),
    (dict(max_pages=0), mla.MLA_ERR_INVALID_ARGUMENT, "max_pages_per_seq"),
    (dict(batch=1 << 16, n_new=1 << 16), mla.MLA_ERR_UNSUPPORTED, "n_new"),
    (dict(kv_new=None), mla.MLA_ERR_INVALID_ARGUMENT, "kv_new"),
    (dict(kv_new=FAKE + 8), mla.MLA_ERR_INVALID_ARGUMENT, "kv_new"),
    (dict(start_pos=None), mla.MLA_ERR_INVALID_ARGUMENT, "start_pos"),
    (dict(bt=None), mla.MLA_ERR_INVALID_ARGUMENT, "block_table"),
    (dict(pool=None), mla.MLA_ERR_INVALID_ARGUMENT, "kv_pool"),
    (dict(pool=FAKE + 4), mla.MLA_ERR_INVALID_ARGUMENT, "kv_pool"),
])
def test_writer_rejects_bad_arguments(kw, status, word):
    assert call_writer(**kw) == status
    assert mla.mla_last_error().startswith(word)


def test_writer_with_no_tokens_launches_nothing():
    # zero tokens is a valid no-op: it must succeed without touching the GPU
    assert call_writer(batch=0) == mla.MLA_OK
    assert call_writer(n_new=0) == mla.MLA_OK


def call_prefill(s_q=4, h_q=16, s_kv=100, topk=8, fmt=0, flags=0, scale=0.5, q=FAKE, kv=FAKE,
                 idx=FAKE, parts=4, ws=FAKE, ws_bytes=1 << 40, out=FAKE, lse=FAKE):
    lib = mla._load()
    v = lambda x: None if x is None else ctypes.c_void_p(x)
    return lib.mla_sparse_prefill(s_q, h_q, s_kv, topk, fmt, flags, scale, v(q), v(kv), v(idx),
                                  parts, v(ws), ws_bytes, v(out), v(lse), None)


@pytest.mark.parametrize("kw, status, word", [
    (dict(s_q=-1), mla.MLA_ERR_INVALID_ARGUMENT, "s_q"),
    (dict(h_q=0), mla.MLA_ERR_INVALID_ARGUMENT, "h_q"),
    (dict(s_kv=0), mla.MLA_ERR_INVALID_ARGUMENT, "s_kv"),
    (dict(topk=0), mla.MLA_ERR_INVALID_ARGUMENT, "topk"),
    (dict(fmt=7), mla.MLA_ERR_INVALID_ARGUMENT, "kv_format"),
    (dict(flags=4), mla.MLA_ERR_INVALID_ARGUMENT, "flags"),
    (dict(scale=float("nan")), mla.MLA_ERR_INVALID_ARGUMENT, "softmax_scale"),
    (dict(parts=0), mla.MLA_ERR_INVALID_ARGUMENT, "num_parts"),
    (dict(q=None), mla.MLA_ERR_INVALID_ARGUMENT, "q"),
    (dict(kv=FAKE + 8), mla.MLA_ERR_INVALID_ARGUMENT, "kv"),
    (dict(idx=None), mla.MLA_ERR_INVALID_ARGUMENT, "indices"),
    (dict(ws=FAKE + 16), mla.MLA_ERR_INVALID_ARGUMENT, "workspace"),
    (dict(out=None), mla.MLA_ERR_INVALID_ARGUMENT, "out"),
    (dict(lse=None), mla.MLA_ERR_INVALID_ARGUMENT, "lse"),
    (dict(ws_bytes=1024), mla.MLA_ERR_WORKSPACE_TOO_SMALL, "workspace_bytes"),
])
def test_prefill_rejects_bad_arguments(kw, status, word):
    assert call_prefill(**kw) == status
    assert mla.mla_last_error().startswith(word)


def test_prefill_workspace_grows_with_chunk_not_beyond():
    a = mla.mla_sparse_prefill_workspace_bytes(100, 128, 5000, 64, 0, 256)
    b = mla.mla_sparse_prefill_workspace_bytes(2048, 128, 5000, 64, 0, 256)
    c = mla.mla_sparse_prefill_workspace_bytes(100000, 128, 5000, 64, 0, 256)
    assert a < b == c
    assert call_prefill(s_q=0, ws_bytes=mla.mla_sparse_prefill_workspace_bytes(0, 16, 100, 8, 0, 4)) == mla.MLA_OK


def test_check_inputs_rejects_bad_arguments():
    lib = mla._load()
    p = good()
    assert lib.mla_decode_check_inputs(None, ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE),
                                       ctypes.c_void_p(FAKE), None) == mla.MLA_ERR_INVALID_ARGUMENT
    assert lib.mla_decode_check_inputs(ctypes.byref(p), ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE),
                                       None, None) == mla.MLA_ERR_INVALID_ARGUMENT
    assert mla.mla_last_error().startswith("result")
    assert lib.mla_decode_check_inputs(ctypes.byref(p), None, ctypes.c_void_p(FAKE),
                                       ctypes.c_void_p(FAKE), None) == mla.MLA_ERR_INVALID_ARGUMENT
    assert mla.mla_last_error().startswith("block_table")


def test_decode_kernel_name():
    """The kernel the library picks for a problem, read on the host: dense
    units of at most 32 rows (either format) go to the small-head kernel."""
    assert mla.mla_decode_kernel_name(good(h_q=16)) == "decode_small_kernel"
    assert mla.mla_decode_kernel_name(good(h_q=16, s_q=2)) == "decode_small_kernel"
    assert mla.mla_decode_kernel_name(good(h_q=32, kv_format=mla.MLA_KV_FP8_656)) == "decode_small_kernel"
    assert mla.mla_decode_kernel_name(good(h_q=33)) == "decode_kernel"
    assert mla.mla_decode_kernel_name(good(h_q=128, s_q=2)) == "decode_kernel"
    assert mla.mla_decode_kernel_name(good(h_q=16, topk=64)) == "decode_kernel"
    with pytest.raises(ValueError, match="s_q"):
        mla.mla_decode_kernel_name(good(s_q=0))


def test_clock_probe_rejects_bad_arguments():
    lib = mla._load()
    assert lib.mla_clock_probe(None, 256, 10, None) == mla.MLA_ERR_INVALID_ARGUMENT
    assert "out" in mla.mla_last_error()
    assert lib.mla_clock_probe(ctypes.c_void_p(FAKE), 0, 10, None) == mla.MLA_ERR_INVALID_ARGUMENT
    assert "workgroups" in mla.mla_last_error()
    assert lib.mla_clock_probe(ctypes.c_void_p(FAKE), 4, 0, None) == mla.MLA_ERR_INVALID_ARGUMENT
    assert "spins" in mla.mla_last_error()


def call_noalloc(p, parts=4, idx=None):
    lib = mla._load()
    v = ctypes.c_void_p
    return lib.mla_decode_paged_noalloc(ctypes.byref(p), v(FAKE), v(FAKE), v(FAKE), v(FAKE),
                                        None if idx is None else v(idx), v(FAKE), parts, v(FAKE),
                                        v(FAKE), v(FAKE), None)


def test_noalloc_size_limit_checked_on_the_host():
    """The allocation-free call rejects a problem whose split partials exceed
    its static scratch, before any HIP call, naming the limit."""
    assert mla.NOALLOC_SCRATCH_BYTES == 96 << 20
    text = open(HEADER).read()
    assert re.search(r"#define MLA_NOALLOC_SCRATCH_BYTES \(\(size_t\)96 << 20\)", text)
    p = good(batch=128, s_q=2, h_q=128)
    fits = max(n for n in range(1, 2049) if mla.mla_decode_workspace_bytes(p, n) <= mla.NOALLOC_SCRATCH_BYTES)
    assert mla.mla_decode_workspace_bytes(p, 128) <= mla.NOALLOC_SCRATCH_BYTES  # 64.3 MiB
    assert call_noalloc(p, parts=fits + 1) == mla.MLA_ERR_WORKSPACE_TOO_SMALL
    assert "static scratch" in mla.mla_last_error()
    assert call_noalloc(good(), idx=FAKE) == mla.MLA_ERR_INVALID_ARGUMENT
    assert "indices" in mla.mla_last_error()


def index_good(**kw):
    d = dict(batch=2, s_q=2, h=64, num_pages=9, max_pages_per_seq=4, topk=16)
    d.update(kw)
    return mla.IndexProblem.make(**d)


def call_index(p, ws_bytes=1 << 40, **ptrs):
    lib = mla._load()
    a = dict(q=FAKE, qs=FAKE, kv=FAKE, bt=FAKE, sl=FAKE, ws=FAKE, idx=FAKE, sc=None)
    a.update(ptrs)
    v = lambda x: None if x is None else ctypes.c_void_p(x)
    return lib.mla_fp8_index_top_k(ctypes.byref(p), v(a["q"]), v(a["qs"]), v(a["kv"]), v(a["bt"]),
                                   v(a["sl"]), v(a["ws"]), ws_bytes, v(a["idx"]), v(a["sc"]), None)


@pytest.mark.parametrize("field,value,status", [
    ("h", 0, mla.MLA_ERR_INVALID_ARGUMENT), ("h", 4097, mla.MLA_ERR_UNSUPPORTED),
    ("d", 576, mla.MLA_ERR_UNSUPPORTED), ("page_size", 32, mla.MLA_ERR_UNSUPPORTED),
    ("max_pages_per_seq", 1025, mla.MLA_ERR_UNSUPPORTED), ("topk", 0, mla.MLA_ERR_INVALID_ARGUMENT),
    ("topk", 257, mla.MLA_ERR_INVALID_ARGUMENT), ("kpool", 0, mla.MLA_ERR_INVALID_ARGUMENT),
    ("is_causal", 2, mla.MLA_ERR_INVALID_ARGUMENT), ("s_q", 0, mla.MLA_ERR_INVALID_ARGUMENT),
    ("batch", -1, mla.MLA_ERR_INVALID_ARGUMENT), ("num_pages", 0, mla.MLA_ERR_INVALID_ARGUMENT),
])
def test_index_problem_fields_rejected(field, value, status):
    p = index_good()
    setattr(p, field, value)
    assert call_index(p) == status
    assert field in mla.mla_last_error()


def test_index_pointers_and_workspace_checked():
    p = index_good()
    for name, arg in [("q_fp8", "q"), ("q_scale", "qs"), ("kv_pool", "kv"), ("block_table", "bt"),
                      ("cache_seqlens", "sl"), ("workspace", "ws"), ("indices", "idx")]:
        assert call_index(p, **{arg: None}) == mla.MLA_ERR_INVALID_ARGUMENT
        assert name in mla.mla_last_error()
    assert call_index(p, q=FAKE + 4) == mla.MLA_ERR_INVALID_ARGUMENT  # alignment
    need = mla.mla_fp8_index_workspace_bytes(p)
    assert need == 2 * 2 * 4 * 64 * 4 + 2 * 2 * 512 * 4  # fp32 scores [B, s_q, 64 * max_pages], Qsum [B, s_q, 512]
    assert call_index(p, ws_bytes=need - 1) == mla.MLA_ERR_WORKSPACE_TOO_SMALL
