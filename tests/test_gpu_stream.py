"""Streams and graphs at the boundary.

* The rotary table of a theta is built on the device, on the stream of the
  first call that uses it (the block builds `freqs` once, at construction:
  Wan2.2 source reading (blog.leeguoo.com), ch. 4, "1つの block の完全な
  forward"), so that no call blocks and a first use can be captured into a
  HIP graph.  A captured self-attention call with a theta the library has
  never seen is replayed several times, with eager work in between, and
  every replay is checked against the oracle and against an eager call.
* The binding allocates a call's workspace and outputs on the stream the
  call is enqueued on: a call on a side stream without a workspace must give
  the same bits as one on the current stream, even when the current stream
  reuses freed memory right after the call returns.
"""
import numpy as np
import pytest
import torch

import oracle
from parity_util import assert_parity, from_dev, to_dev, widen
from video_diffusion_transformer_wanattn_amd import seeded
from video_diffusion_transformer_wanattn_amd import wanattn as wa

pytestmark = pytest.mark.gpu


def inputs(B, N, heads, seed):
    return [seeded.normal_bf16((B, N, heads, 128), seed, s, 0.5) for s in (1, 2, 3)]


def test_graph_capture_of_a_first_theta_use():
    grid = (7, 9, 11)
    N, heads = 693, 3
    q, k, v = inputs(1, N, heads, 1100)
    dq, dk, dv = to_dev(q), to_dev(k), to_dev(v)
    # eager work first: the device is set up, theta 10000 is built
    warm = wa.self_attention(dq, dk, dv, grid, theta=10000.0)
    torch.cuda.synchronize()
    theta = 7777.0          # used nowhere else in the test process
    ws = torch.empty(wa.self_workspace_bytes(1, N, heads), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(dq)
    ws_n = torch.empty_like(dq)
    out_n = torch.empty_like(dq)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            wa.self_attention(dq, dk, dv, grid, theta=theta, workspace=ws, out=out)
            wa.self_attention(dq, dk, dv, grid, theta=theta, block_causal=True, chunk_frames=2, out=out_n,
                              workspace=ws_n)
    torch.cuda.current_stream().wait_stream(s)
    ref = oracle.self_rows(q, k, v, grid, theta=theta)
    ref_c = oracle.self_rows(q, k, v, grid, theta=theta, block_causal=True, chunk_frames=2)
    first = None
    for rep in range(4):
        out.fill_(float("nan"))
        out_n.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        got, got_c = from_dev(out), from_dev(out_n)
        e = assert_parity(got, ref, what=f"replay {rep}")
        assert_parity(got_c, ref_c, what=f"replay {rep} block-causal")
        print(f"replay {rep}: {e}", flush=True)
        if first is None:
            first = (got, got_c)
        np.testing.assert_array_equal(got, first[0])
        np.testing.assert_array_equal(got_c, first[1])
        # eager work between replays, on other thetas and on the captured one
        # (thetas other tests use too: the library keeps 8 per device)
        th = 10000.0 if rep % 2 == 0 else 777.0
        other = wa.self_attention(dq, dk, dv, grid, theta=th)
        torch.cuda.synchronize()
        assert_parity(from_dev(other), oracle.self_rows(q, k, v, grid, theta=th), what=f"eager theta {th}")
    eager = wa.self_attention(dq, dk, dv, grid, theta=theta)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(from_dev(eager), first[0])
    del warm


def test_side_stream_without_workspace():
    grid = (5, 24, 36)
    N, heads = 4320, 16
    q, k, v = inputs(1, N, heads, 1200)
    dq, dk, dv = to_dev(q), to_dev(k), to_dev(v)
    base = wa.self_attention(dq, dk, dv, grid)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    got = wa.self_attention(dq, dk, dv, grid, stream=s)
    # the current stream takes memory as soon as the call returns; had the
    # workspace come from its pool, these writes could land in it mid-kernel
    junk = [torch.full((wa.self_workspace_bytes(1, N, heads) // 2,), 7.0, dtype=torch.bfloat16, device="cuda")
            for _ in range(3)]
    torch.cuda.synchronize()
    np.testing.assert_array_equal(from_dev(got), from_dev(base))
    del junk
    # the prologue's workspace (y and the GEMM library's) likewise
    p = seeded.prologue_tensors(1, 300, 512, seed=3)
    pd = {n: (torch.from_numpy(a).cuda() if n in ("e0", "e1") else to_dev(a)) for n, a in p.items()}
    args = [pd[n] for n in ("x", "e0", "e1", "wq", "bq", "wk", "bk", "wv", "bv", "gq", "gk")]
    ref = wa.prologue(*args)
    torch.cuda.synchronize()
    s.wait_stream(torch.cuda.current_stream())
    side = wa.prologue(*args, stream=s)
    junk = [torch.full((wa.prologue_workspace_bytes(1, 300, 512) // 2,), 3.0, dtype=torch.bfloat16, device="cuda")
            for _ in range(2)]
    torch.cuda.synchronize()
    for a, b in zip(side, ref):
        np.testing.assert_array_equal(from_dev(a), from_dev(b))
    del junk


def test_prepare_then_calls_on_two_streams():
    # a theta first used on one stream, then at once on another: the second
    # waits for the first's table build through the library's event
    grid = (5, 8, 8)
    q, k, v = inputs(1, 320, 4, 1300)
    dq, dk, dv = to_dev(q), to_dev(k), to_dev(v)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    s1.wait_stream(torch.cuda.current_stream())
    s2.wait_stream(torch.cuda.current_stream())
    a = wa.self_attention(dq, dk, dv, grid, theta=4321.0, stream=s1)
    b = wa.self_attention(dq, dk, dv, grid, theta=4321.0, stream=s2)
    torch.cuda.synchronize()
    ref = oracle.self_rows(q, k, v, grid, theta=4321.0)
    assert_parity(from_dev(a), ref, what="stream 1")
    np.testing.assert_array_equal(from_dev(a), from_dev(b))
    wa.prepare(9876.0)
    c = wa.rope3d(dk, grid, theta=9876.0)
    torch.cuda.synchronize()
    assert np.max(np.abs(widen(from_dev(c)) - oracle.rope3d(k, grid, 9876.0))) < 2e-2
