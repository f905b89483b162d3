"""Every call is stream-ordered with no host synchronization and no memset,
so a chain of calls can be captured into a HIP graph (the header's promise).
The MTP decode step (scores, then top-16) and a ragged causal prefill batch
are captured once, replayed several times with eager work and
synchronizations between the replays, and every replay must reproduce the
eager results bit for bit."""

import numpy as np
import pytest
import torch

import workloads
from gpu_util import announce, dev

pytestmark = pytest.mark.gpu


def _replay_check(capture, outputs, reps=4):
    """Run `capture` eagerly, then capture it into a graph and replay it
    `reps` times, zeroing the outputs in between; compare every replay."""
    capture()
    torch.cuda.synchronize()
    want = [o.clone() for o in outputs]
    stream = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            capture()
    torch.cuda.synchronize()
    for r in range(reps):
        for o in outputs:
            o.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, w in zip(outputs, want):
            assert torch.equal(o, w), f"replay {r} differs from the eager result"


def test_decode_step_in_a_graph():
    import page_scoring_top_amd as ps
    d = workloads.mtp_decode()
    R, W = d.num_reqs, d.width
    kv, bt, seq = dev(d.kv_cache), dev(d.block_table), dev(d.seq_lens)
    q, qs = dev(d.q), dev(d.q_scale)
    scores = torch.zeros((R, 32, W), dtype=torch.float32, device="cuda")
    own = torch.zeros((R, 32), dtype=torch.int32, device="cuda")
    out = torch.zeros((R * 32, 16), dtype=torch.int32, device="cuda")

    def step():
        ps.indexer_score_decode(kv, bt, seq, q, qs, d.qlen, W, scores, own, num_reqs=R)
        ps.topk16_select(scores.view(R * 32, W), W, out, valid_len=own.view(-1),
                         append_page=own.view(-1))

    announce("graph: mtp decode step")
    _replay_check(step, [scores, own, out])


def test_ragged_prefill_and_mxfp8_in_a_graph():
    import page_scoring_top_amd as ps
    r = workloads.ragged_prefill_inputs("graph-ragged", 9, [40, 200, 7], [300, 900, 7], 4)
    T = r.p.q.shape[0]
    q, qs, k, ks = dev(r.p.q), dev(r.p.q_scale), dev(r.p.k), dev(r.p.k_scale)
    q_start, k_start, k_len = dev(r.q_start), dev(r.k_start), dev(r.k_len)
    scores = torch.zeros((T, r.width), dtype=torch.float32, device="cuda")
    row_len = torch.zeros(T, dtype=torch.int32, device="cuda")
    out = torch.zeros((T, 16), dtype=torch.int32, device="cuda")
    xa = workloads.mx_activations(3, 64, 2048)
    x = dev(xa.view(np.int16)).view(torch.bfloat16)
    xq = torch.zeros((64, 2048), dtype=torch.uint8, device="cuda")
    xs = torch.zeros((64, 64), dtype=torch.uint8, device="cuda")

    def chain():
        ps.indexer_score_prefill_ragged(q, qs, k, ks, q_start, k_start, k_len, 200, r.width,
                                        scores, row_len)
        ps.topk16_select(scores, r.width, out, valid_len=row_len)
        ps.mxfp8_e4m3_quantize(x, xq, xs)

    announce("graph: ragged prefill, top-16, mxfp8")
    _replay_check(chain, [scores, row_len, out, xq, xs])


def test_prepared_calls_eager_and_in_a_graph():
    """PreparedCall launches exactly what the direct call launches, and
    again() re-marshals it on the stream current at that time, so it can be
    captured into a graph on a side stream."""
    import page_scoring_top_amd as ps
    d = workloads.tiny_decode()
    W = d.width
    kv, bt, seq = dev(d.kv_cache), dev(d.block_table), dev(d.seq_lens)
    q, qs = dev(d.q), dev(d.q_scale)
    direct = torch.zeros((1, 32, W), device="cuda")
    own_d = torch.zeros((1, 32), dtype=torch.int32, device="cuda")
    ps.indexer_score_decode(kv, bt, seq, q, qs, d.qlen, W, direct, own_d)
    torch.cuda.synchronize()

    scores = torch.zeros((1, 32, W), device="cuda")
    own = torch.zeros((1, 32), dtype=torch.int32, device="cuda")
    call = ps.prepare(ps.indexer_score_decode, kv, bt, seq, q, qs, d.qlen, W, scores, own)
    announce("prepared call: tiny decode, eager")
    call()
    torch.cuda.synchronize()
    assert torch.equal(scores, direct) and torch.equal(own, own_d)

    announce("prepared call: tiny decode, again() captured on a side stream")
    scores.zero_()
    own.zero_()
    _replay_check(lambda: call.again()(), [scores, own])
    assert torch.equal(scores, direct) and torch.equal(own, own_d)


def test_fused_prefill_topk_in_a_graph():
    """indexer_prefill_topk16 (two kernels over a workspace) replayed from a
    graph gives the eager rows every time."""
    import page_scoring_top_amd as ps
    T, H, N = 300, 4, 20000
    p = workloads.prefill_inputs("graph-ptk", 81, T, H, N)
    q, qs, k, ks = dev(p.q), dev(p.q_scale), dev(p.k), dev(p.k_scale)
    out = torch.zeros((T, 16), dtype=torch.int32, device="cuda")
    ws = ps.prefill_topk16_workspace(T, N, "cuda")

    def step():
        ps.indexer_prefill_topk16(q, qs, k, ks, out, ws)

    announce("graph: fused prefill top-16")
    _replay_check(step, [out])
