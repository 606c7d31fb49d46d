"""wanattn_self_noalloc: wanattn_self for callers that cannot allocate, its
scratch (rotated keys, key-split partials, queue counters) in the library's
static per-device array instead of a caller workspace.

Checked through the C ABI against wanattn_self with a full workspace (the
same kernels and launch configuration: bitwise equal) and against the fp64
oracle, on calls in a row with shrinking inputs (the scratch keeps the last
call's contents), and the size limit is checked on the host before anything
is launched.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from parity_util import assert_parity, from_dev, to_dev
from video_diffusion_transformer_wanattn_amd import seeded
from video_diffusion_transformer_wanattn_amd import wanattn as wa

THETA = 10000.0
GiB = 1 << 30


def test_noalloc_rejects_beyond_scratch_before_launch():
    lib = wa.load_library()
    # 75,600 tokens x 40 heads: 774 MB of rotated keys, more than the scratch
    g = ctypes.byref(wa.Grid3D(21, 45, 80, 0, 0, 0))
    q, k, v, o = (ctypes.c_void_p(i * 4 * GiB) for i in (1, 2, 3, 4))
    st = lib.wanattn_self_noalloc(q, k, v, o, 1, 75600, 40, 128, g, THETA, 0.088, 0, 3, None, None)
    assert st == wa.E_UNSUPPORTED
    assert b"scratch" in lib.wanattn_last_error()
    assert 75600 * 40 * 256 + 256 > wa.NOALLOC_SCRATCH_BYTES >= 32760 * 40 * 256 + 256
    # argument errors come first, as in wanattn_self (nothing touches a GPU)
    assert lib.wanattn_self_noalloc(None, k, v, o, 1, 75600, 40, 128, g, THETA, 0.088, 0, 3, None,
                                    None) == wa.E_INVALID
    g2 = ctypes.byref(wa.Grid3D(2, 3, 4, 0, 0, 0))
    assert lib.wanattn_self_noalloc(q, k, v, q, 1, 24, 2, 128, g2, THETA, 0.088, 0, 3, None,
                                    None) == wa.E_INVALID          # o aliases q
    assert lib.wanattn_self_noalloc(q, k, v, o, 1, 24, 2, 64, g2, THETA, 0.088, 0, 3, None,
                                    None) == wa.E_UNSUPPORTED      # head_dim


# three calls in a row, each smaller than the one before: the 1.3B model's
# 480p layer (32,760 x 12), a launch whose last query tiles run as key-split
# items on a 256-CU chip (4,320 tokens x 16 heads: 16 tiles past the first
# wave), then a block-causal call of two batches with kv_lens
CASES = [
    dict(grid=(21, 30, 52), heads=12, B=1, kw={}, rows=40),
    dict(grid=(5, 24, 36), heads=16, B=1, kw={}, rows=40),
    dict(grid=(6, 6, 8), heads=2, B=2, kw=dict(block_causal=True, chunk_frames=2, kv_lens=[100, 288]), rows=None),
]


@pytest.mark.gpu
def test_noalloc_matches_workspace_call_on_calls_in_a_row():
    for i, c in enumerate(CASES):
        grid, heads, B, kw = c["grid"], c["heads"], c["B"], c["kw"]
        N = int(np.prod(grid))
        print(f"noalloc case {i}: B={B} grid={grid} heads={heads} {kw}", flush=True)
        q, k, v = (seeded.normal_bf16((B, N, heads, 128), 900 + i, s, 0.5) for s in (1, 2, 3))
        dq, dk, dv = to_dev(q), to_dev(k), to_dev(v)
        out_n = torch.empty_like(dq)
        wa.self_attention_noalloc(dq, dk, dv, grid, theta=THETA, out=out_n, **kw)
        ws = torch.empty(wa.self_workspace_bytes(B, N, heads), dtype=torch.uint8, device="cuda")
        out_w = wa.self_attention(dq, dk, dv, grid, theta=THETA, workspace=ws, **kw)
        torch.cuda.synchronize()
        got_n, got_w = from_dev(out_n), from_dev(out_w)
        np.testing.assert_array_equal(got_n, got_w)
        rows = None if c["rows"] is None else seeded.sample_rows(N, c["rows"], seed=i, must=(N - 1, N - 257))
        ref = oracle.self_rows(q, k, v, grid, rows=rows, theta=THETA, **kw)
        sel = got_n if rows is None else got_n[:, rows]
        e = assert_parity(sel, ref, what=f"noalloc case {i}")
        print(f"noalloc case {i}: {e}", flush=True)
        del dq, dk, dv, out_n, out_w, ws
