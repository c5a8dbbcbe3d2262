"""The C-ABI's stream contract on the GPU.

Every entry point enqueues on the stream it is given and never synchronises (include/fa.h).
These tests run the entry points on a non-default stream, with inputs made on that
stream, and compare the results bit for bit with the same calls on the default stream;
and they capture the forward and the allocation-free backward in a HIP graph, then
replay it several times with new inputs copied in between, comparing every replay with
eager calls on the same inputs (the library launches kernels only: no memsets, copies or
synchronisations that a graph could not hold)."""
import pytest
import torch

import synthetic
from tests import gpu_checks as G

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _inputs(B, H, N, d, seed, dtype="bf16"):
    return [x.to(DEV) for x in synthetic.draw_qkv(B, H, N, d, seed=seed, dtype=dtype)]


def _equal(a, b):
    return all(torch.equal(x, y) for x, y in zip(a, b))


def test_side_stream_matches_default_stream(fa):
    B, H, N, d = 2, 3, 300, 128
    q, k, v = _inputs(B, H, N, d, seed=701)
    qf, kf, vf = _inputs(1, 2, 200, 64, seed=702, dtype="f32")
    do = _inputs(B, H, N, d, seed=703)[0]
    signs = torch.from_numpy(synthetic.draw_signs(d, 704)).to(DEV)

    def run_all(stream):
        out = {}
        out["bf16"] = fa.fa_fwd(q, k, v, causal=True, stream=stream)
        out["f32"] = fa.fa_fwd(qf, kf, vf, causal=False, stream=stream)
        o, lse = out["bf16"]
        out["bwd"] = fa.fa_bwd(q, k, v, o, do, lse, causal=True, stream=stream)
        out["fp8"] = fa.fp8_attention(q, k, v, signs, causal=True, stream=stream)[:2]
        o_parts, lse_parts = fa.fa_fwd_split(q, k, v, 3, 0, 0, N, True, None, stream=stream)
        out["split"] = fa.fa_merge(o_parts, lse_parts, q.dtype, stream=stream)
        return out

    G.log("case streams: default stream")
    ref = run_all(None)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()  # default priority
    G.log("case streams: side stream")
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        got = run_all(side)
    side.synchronize()
    for name in ref:
        assert _equal(ref[name], got[name]), name


def test_graph_capture_replays(fa):
    """fa_fwd and fa_bwd_noalloc captured in one graph; three replays on fresh inputs."""
    B, H, N, d = 1, 2, 333, 128
    q, k, v = _inputs(B, H, N, d, seed=711)
    do = _inputs(B, H, N, d, seed=712)[0]
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=DEV)
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))

    def step():
        fa.fa_fwd(q, k, v, causal=True, o=o, lse=lse)
        fa.fa_bwd_noalloc(q, k, v, o, do, lse, causal=True, dq=dq, dk=dk, dv=dv)

    # warm-up outside the capture (the no-alloc entry point looks up its workspace on its
    # first call on a device)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()

    for rep in range(3):
        G.log(f"case graph replay {rep}")
        nq, nk, nv = _inputs(B, H, N, d, seed=720 + rep)
        ndo = _inputs(B, H, N, d, seed=730 + rep)[0]
        # eager work between replays: new inputs copied into the captured buffers
        q.copy_(nq)
        k.copy_(nk)
        v.copy_(nv)
        do.copy_(ndo)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = (o.clone(), lse.clone(), dq.clone(), dk.clone(), dv.clone())
        eo, el = fa.fa_fwd(nq, nk, nv, causal=True)
        edq, edk, edv = fa.fa_bwd(nq, nk, nv, eo, ndo, el, causal=True)
        torch.cuda.synchronize()
        assert _equal(got, (eo, el, edq, edk, edv)), rep


def test_concurrent_calls_on_two_streams(fa):
    """Different problems in flight at once on two streams (the library keeps no mutable
    state between calls apart from the no-alloc workspace, which is not used here): each
    result bit-identical to the same call run alone."""
    a = _inputs(1, 4, 1500, 128, seed=741)
    b = _inputs(2, 2, 900, 64, seed=742)
    do_a = _inputs(1, 4, 1500, 128, seed=743)[0]
    alone_a = fa.fa_fwd(*a, causal=True)
    alone_ga = fa.fa_bwd(*a, alone_a[0], do_a, alone_a[1], causal=True)
    alone_b = fa.fa_fwd(*b, causal=False)
    torch.cuda.synchronize()
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    sa.wait_stream(torch.cuda.current_stream())
    sb.wait_stream(torch.cuda.current_stream())
    G.log("case concurrent calls on two streams")
    for _ in range(3):
        with torch.cuda.stream(sa):
            got_a = fa.fa_fwd(*a, causal=True, stream=sa)
            got_ga = fa.fa_bwd(*a, got_a[0], do_a, got_a[1], causal=True, stream=sa)
        with torch.cuda.stream(sb):
            got_b = fa.fa_fwd(*b, causal=False, stream=sb)
        torch.cuda.synchronize()
        assert _equal(alone_a, got_a) and _equal(alone_ga, got_ga) and _equal(alone_b, got_b)
