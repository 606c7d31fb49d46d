"""GPU parity at the edges of the ABI's ranges, against the fp64 oracle:
more batches than one launch takes with length arrays (the library splits
them into launches of 256), positions on the last row of the RoPE tables
(1023 on every axis), and very many heads (wide token rows, so the kernels'
32-bit row offsets are exercised far from zero).
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


def test_many_batches_with_lengths_span_launches():
    # 260 batches of a 2 x 2 x 5 grid (20 tokens): the self call with kv_lens
    # and the cross call with ctx_lens run as a launch of 256 batches and one
    # of 4; every batch has its own visible prefix
    B, grid, N, heads, M = 260, (2, 2, 5), 20, 2, 9
    q, k = (gen((B, N, heads, 128), 900, s, 1.0) for s in (1, 2))
    v = gen((B, N, heads, 128), 900, 3, 0.5)
    kc, vc = (gen((B, M, heads, 128), 900, s, 0.5) for s in (4, 5))
    lens = [1 + (7 * b) % N for b in range(B)]
    clens = [1 + (5 * b) % M for b in range(B)]
    got = from_dev(wa.self_attention(to_dev(q), to_dev(k), to_dev(v), grid, theta=THETA, kv_lens=lens))
    gotc = from_dev(wa.cross_attention(to_dev(q), to_dev(kc), to_dev(vc), ctx_lens=clens))
    torch.cuda.synchronize()
    assert_parity(got, oracle.self_rows(q, k, v, grid, theta=THETA, kv_lens=lens), what="260 batches self")
    assert_parity(gotc, oracle.cross_rows(q, kc, vc, ctx_lens=clens), what="260 batches cross")


def test_positions_on_the_last_table_row():
    # offsets put the last frame, row and column at position 1023 on their axes
    grid, heads = (3, 4, 6), 2
    off = (1021, 1020, 1018)
    N = 72
    q, k = (gen((1, N, heads, 128), 901, s, 1.5) for s in (1, 2))
    v = gen((1, N, heads, 128), 901, 3, 0.5)
    got = from_dev(wa.self_attention(to_dev(q), to_dev(k), to_dev(v), grid, theta=THETA, offsets=off))
    torch.cuda.synchronize()
    assert_parity(got, oracle.self_rows(q, k, v, grid, theta=THETA, offsets=off), what="positions up to 1023")
    with pytest.raises(wa.WanattnError):
        wa.self_attention(to_dev(q), to_dev(k), to_dev(v), grid, theta=THETA, offsets=(1022, 0, 0))


def test_many_heads_wide_rows():
    # 4096 heads: one token row is 1 MiB, a 64-key tile spans 64 MiB of rows;
    # 70 tokens give a full and a partial key tile
    grid, heads = (2, 5, 7), 4096
    N = 70
    q, k = (gen((1, N, heads, 128), 902, s, 1.0) for s in (1, 2))
    v = gen((1, N, heads, 128), 902, 3, 0.5)
    got = from_dev(wa.self_attention(to_dev(q), to_dev(k), to_dev(v), grid, theta=THETA))
    torch.cuda.synchronize()
    hs = np.array([0, 1, 2047, 4094, 4095])
    ref = oracle.self_rows(q[:, :, hs], k[:, :, hs], v[:, :, hs], grid, theta=THETA)
    assert_parity(got[:, :, hs], ref, what="4096 heads")
    kc, vc = (gen((1, 33, heads, 128), 902, s, 0.5) for s in (4, 5))
    gotc = from_dev(wa.cross_attention(to_dev(q), to_dev(kc), to_dev(vc)))
    torch.cuda.synchronize()
    assert_parity(gotc[:, :, hs], oracle.cross_rows(q[:, :, hs], kc[:, :, hs], vc[:, :, hs]),
                  what="4096 heads cross")
