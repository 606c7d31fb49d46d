"""GPU parity of the KV-cache streaming call (Self Forcing, one chunk against
the cache of the chunks before it and itself; long-video survey (atlascloud.ai),
"ルート3 · Self Forcing") against the fp64 oracle.  The cache keys are rotated
on the GPU with wanattn_rope3d, as a caller would when appending a chunk; the
oracle rotates the raw keys itself.
"""
import numpy as np
import pytest
import torch

import oracle
from parity_util import assert_parity, from_dev, to_dev
from video_diffusion_transformer_wanattn_amd import seeded
from video_diffusion_transformer_wanattn_amd import wanattn as wa

pytestmark = pytest.mark.gpu
THETA = 10000.0


def gen(shape, seed, stream, sigma):
    return seeded.normal_bf16(shape, seed, stream, sigma)


def gpu_kv(q, k, v, cache_grid, cache_offsets, grid_q, q_offsets, kv_lens=None):
    kc = wa.rope3d(to_dev(k), cache_grid, theta=THETA, offsets=cache_offsets)
    o = wa.self_attention_kv(to_dev(q), kc, to_dev(v), grid_q, theta=THETA, kv_lens=kv_lens,
                             offsets=q_offsets)
    torch.cuda.synchronize()
    return from_dev(o)


@pytest.mark.parametrize("sigma", [0.5, 1.5])
def test_stream_chunk_by_chunk(sigma):
    # a 6-frame clip of 9 x 10 tokens per frame (90 tokens: ragged against the
    # 64-key tiles and the 256-row query tiles), chunks of 2 frames
    F, H, W, C, B, heads = 6, 9, 10, 2, 2, 2
    HW = H * W
    q, k = (gen((B, F * HW, heads, 128), 40, s, sigma) for s in (1, 2))
    v = gen((B, F * HW, heads, 128), 40, 3, 0.5)
    for c in range(F // C):
        rows = slice(c * C * HW, (c + 1) * C * HW)
        n = (c + 1) * C * HW
        qc = np.ascontiguousarray(q[:, rows])
        got = gpu_kv(qc, np.ascontiguousarray(k[:, :n]), np.ascontiguousarray(v[:, :n]),
                     ((c + 1) * C, H, W), (0, 0, 0), (C, H, W), (c * C, 0, 0))
        ref = oracle.kv_rows(qc, k[:, :n], v[:, :n], (C, H, W, c * C, 0, 0), kv_frame0=0, theta=THETA)
        assert_parity(got, ref, what=f"kv chunk {c} sigma {sigma}")


def test_rolling_window_offsets_and_lengths():
    # the cache keeps frames 2..6 (a rolling window); the chunk is frame 7 and 8;
    # height/width offsets on both, different visible prefixes per batch
    H, W, heads, B = 7, 11, 3, 2
    HW = H * W
    q = gen((B, 2 * HW, heads, 128), 41, 1, 1.0)
    k = gen((B, 5 * HW, heads, 128), 41, 2, 1.0)
    v = gen((B, 5 * HW, heads, 128), 41, 3, 0.5)
    lens = [5 * HW - 7, 3 * HW]
    got = gpu_kv(q, k, v, (5, H, W), (2, 1, 3), (2, H, W), (7, 1, 3), kv_lens=lens)
    ref = oracle.kv_rows(q, k, v, (2, H, W, 7, 1, 3), kv_frame0=2, theta=THETA, kv_lens=lens)
    assert_parity(got, ref, what="rolling window")


def test_full_size_last_chunk_of_165_frames():
    # the last chunk (frames 39..41, 4,680 tokens) of the 165-frame, 40-head
    # Self Forcing workload against the full 42-frame cache (65,520 tokens)
    wl = seeded.WORKLOADS["wan14b_480p_165f_causal"]
    t = seeded.workload_tensors(wl, seed=0, cross=False)
    HW = wl.H * wl.W
    c0 = wl.F - wl.chunk_frames
    qc = np.ascontiguousarray(t["q"][:, c0 * HW:])
    rows = seeded.sample_rows(qc.shape[1], 40, seed=5, must=(0, qc.shape[1] - 1))
    kc = wa.rope3d(to_dev(t["k"]), (wl.F, wl.H, wl.W), theta=THETA)
    o = wa.self_attention_kv(to_dev(qc), kc, to_dev(t["v"]), (wl.chunk_frames, wl.H, wl.W),
                             theta=THETA, offsets=(c0, 0, 0))
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o.float()).all())
    got = from_dev(o[:, torch.from_numpy(rows.astype(np.int64)).cuda()])
    del kc, o
    ref = oracle.kv_rows(qc, t["k"], t["v"], (wl.chunk_frames, wl.H, wl.W, c0, 0, 0), kv_frame0=0,
                         rows=rows, theta=THETA)
    assert_parity(got, ref, what="165f last chunk")
    # the same rows of block-causal self attention over the whole clip
    ref_bc = oracle.self_rows(t["q"], t["k"], t["v"], (wl.F, wl.H, wl.W), rows=rows + c0 * HW,
                              theta=THETA, block_causal=True, chunk_frames=wl.chunk_frames)
    np.testing.assert_allclose(ref, ref_bc, rtol=0, atol=1e-12)


def test_kv_errors_raise_without_launch():
    q = to_dev(gen((1, 24, 1, 128), 42, 1, 0.5))
    kc = to_dev(gen((1, 36, 1, 128), 42, 2, 0.5))
    with pytest.raises(wa.WanattnError):
        wa.self_attention_kv(q, kc[:, :30].contiguous(), kc[:, :30].contiguous(), (2, 3, 4))   # not whole frames
    with pytest.raises(wa.WanattnError):
        wa.self_attention_kv(q, kc, kc.clone(), (2, 3, 4), kv_lens=[37])
