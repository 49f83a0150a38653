"""HIP graph capture of the library's calls.

The calls only enqueue kernels on the given stream (no allocation, copy,
memset or synchronisation), so a caller may capture them in a graph.  Each
case runs the calls eagerly, captures the same calls, then replays the graph
several times with eager work of the program (refilling the outputs, a
synchronisation) between the replays, and checks every replay bit for bit
against the eager result: the calls are deterministic for a fixed input."""

import numpy as np
import pytest
import torch

import paged_kv_head_amd as mla
import synth
from tests.harness import to_device

pytestmark = pytest.mark.gpu

REPLAYS = 3


def bits(t: torch.Tensor) -> np.ndarray:
    """The raw bytes of a tensor (NaN-safe exact comparison)."""
    return t.contiguous().view(torch.uint8).cpu().numpy()


def capture_and_replay(enqueue, outputs, refill):
    """Eager run, capture, REPLAYS replays; every replay must reproduce the
    eager bytes of `outputs`."""
    refill()
    enqueue()
    torch.cuda.synchronize()
    want = [bits(t) for t in outputs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        enqueue()
    torch.cuda.synchronize()
    for rep in range(REPLAYS):
        refill()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, (t, w) in enumerate(zip(outputs, want)):
            assert np.array_equal(bits(t), w), f"replay {rep}: output {k} differs from the eager run"
    return want


@pytest.mark.parametrize("make", [
    pytest.param(lambda: synth.config_workload(2, batch=6), id="dense_bf16_split_units"),
    pytest.param(lambda: synth.config_workload(3, batch=3), id="dense_bf16_causal_two_tokens"),
    pytest.param(lambda: synth.config_workload(4, batch=2), id="dense_fp8"),
    pytest.param(lambda: synth.config_workload(5, batch=2), id="sparse_fp8"),
    pytest.param(lambda: synth.make_workload("g16", batch=5, h_q=16, s_q=1,
                                             seqlens=[3000, 1, 700, 0, 5000], seed=71), id="small_heads"),
])
def test_decode_step_in_a_graph(make):
    """Metadata, decode and combine of one step, captured together."""
    w = make()
    print(f"{w.name}: batch {w.batch}, h_q {w.h_q}, s_q {w.s_q}", flush=True)
    q, kv, bt, sl, idx = to_device(w)
    p = mla.problem_for(w)
    plan = mla.DecodePlan(p, q.device)
    out = torch.empty((w.batch, w.s_q, w.h_q, 512), dtype=torch.bfloat16, device=q.device)
    lse = torch.empty((w.batch, w.s_q, w.h_q), dtype=torch.float32, device=q.device)

    def refill():
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        plan.sched.fill_(-1)
        plan.num_splits.fill_(-1)

    def enqueue():
        plan.metadata(sl)
        plan.decode(q, kv, bt, sl, idx, out, lse)

    capture_and_replay(enqueue, [out, lse], refill)


def test_noalloc_decode_in_a_graph():
    """The entry point without a workspace, captured after one eager call
    has taken the scratch address."""
    w = synth.config_workload(2, batch=4)
    q, kv, bt, sl, idx = to_device(w)
    p = mla.problem_for(w)
    plan = mla.DecodePlan(p, q.device)
    out = torch.empty((w.batch, w.s_q, w.h_q, 512), dtype=torch.bfloat16, device=q.device)
    lse = torch.empty((w.batch, w.s_q, w.h_q), dtype=torch.float32, device=q.device)
    plan.metadata(sl)

    def refill():
        out.fill_(float("nan"))
        lse.fill_(float("nan"))

    def enqueue():
        mla.mla_decode_paged_noalloc(p, q, kv, bt, sl, idx, plan.sched, plan.num_parts,
                                     plan.num_splits, out, lse)

    capture_and_replay(enqueue, [out, lse], refill)


def test_indexer_in_a_graph():
    w = synth.make_index_workload("g_index", batch=3, s_q=2, h=32, seqlens=[2000, 64, 777], seed=72,
                                  topk=100, is_causal=1)
    p = mla.index_problem_for(w)
    qc, qs, kv, bt, sl = mla.index_tensors(w)
    ws = torch.empty(mla.mla_fp8_index_workspace_bytes(p), dtype=torch.uint8, device="cuda")
    idx = torch.empty((w.batch, w.s_q, w.topk), dtype=torch.int32, device="cuda")
    sc = torch.empty((w.batch, w.s_q, w.topk), dtype=torch.float32, device="cuda")

    def refill():
        idx.fill_(-7)
        sc.fill_(float("nan"))

    capture_and_replay(lambda: mla.mla_fp8_index_top_k(p, qc, qs, kv, bt, sl, ws, idx, sc),
                       [idx, sc], refill)


def test_writer_in_a_graph():
    w = synth.make_append("g_append", batch=3, n_new=100, start_pos=[0, 37, 250], seed=73)
    dev = torch.device("cuda")
    kv_new = torch.from_numpy(w.kv_new.view(np.int16)).to(dev).view(torch.bfloat16)
    sp = torch.from_numpy(w.start_pos).to(dev)
    bt = torch.from_numpy(w.block_table).to(dev)
    pool0 = torch.from_numpy(w.pool).to(dev)
    pool = pool0.clone()

    def refill():
        pool.copy_(pool0)

    capture_and_replay(lambda: mla.mla_kv_quantize_fp8(kv_new, sp, bt, pool), [pool], refill)


def test_sparse_prefill_in_a_graph():
    """More query tokens than one prefill chunk: several decode launches."""
    w = synth.make_sparse_prefill("g_prefill", s_q=2100, h_q=16, s_kv=3000, topk=128, seed=74,
                                  kv_format=1, invalid_frac=0.05)
    dev = torch.device("cuda")
    q = torch.from_numpy(w.q.view(np.int16)).to(dev).view(torch.bfloat16)
    kv = torch.from_numpy(w.kv).to(dev)
    ix = torch.from_numpy(w.indices).to(dev)
    parts = mla.mla_sparse_prefill_num_parts(w.h_q, w.topk, w.kv_format)
    need = mla.mla_sparse_prefill_workspace_bytes(w.s_q, w.h_q, w.kv.shape[0], w.topk, w.kv_format, parts)
    ws = torch.empty(max(256, need), dtype=torch.uint8, device=dev)
    out = torch.empty((w.s_q, w.h_q, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((w.s_q, w.h_q), dtype=torch.float32, device=dev)

    def refill():
        out.fill_(float("nan"))
        lse.fill_(float("nan"))

    capture_and_replay(lambda: mla.mla_sparse_prefill(q, kv, ix, w.softmax_scale, kv_format=w.kv_format,
                                                      num_parts=parts, workspace=ws, out=out, lse=lse),
                       [out, lse], refill)
