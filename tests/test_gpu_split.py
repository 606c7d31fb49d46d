"""GPU parity of the key-split tail of bidirectional self attention, against
the fp64 oracle.

A launch whose workgroups fill the chip whole times over plus a remainder of
at most half the chip runs the remainder's query tiles as several workgroups
each, over ranges of the keys (without remainder, from 12 waves on, the last
wave's tiles in two), and combines their partial softmax results (each
against its own running reference) in a second kernel.  The shapes here
are chosen from the device's compute-unit count so that the split happens,
with 4 ranges and with 3 (per-batch key lengths shorten the ranges), and the
last whole wave of a launch without remainder in 2; the rows of the split
tiles are compared.  With scores spread wide enough that the
ranges' references differ by several powers of two, the split's error is
held to that of the same kernel run unsplit.  A workspace without room
for the partials turns the split off.
"""
import numpy as np
import pytest
import torch

import oracle
from parity_util import assert_parity, errors, from_dev, split_heads, to_dev
from video_diffusion_transformer_wanattn_amd import seeded
from video_diffusion_transformer_wanattn_amd import wanattn as wa

pytestmark = pytest.mark.gpu
THETA = 10000.0


def gen(shape, seed, stream, sigma):
    return seeded.normal_bf16(shape, seed, stream, sigma)


def ncu():
    return torch.cuda.get_device_properties(0).multi_processor_count


def tail_case(seed, sigma):
    # 2000 tokens (8 query tiles, 32 key tiles); heads so that the launch is
    # 1.25 chips of workgroups: the last quarter chip runs as 4 key ranges
    grid, N = (5, 20, 20), 2000
    n_cu = ncu()
    heads = max(1, (n_cu + n_cu // 4) // 8)
    q, k = (gen((1, N, heads, 128), seed, s, sigma) for s in (1, 2))
    v = gen((1, N, heads, 128), seed, 3, 0.5)
    hs = np.array(sorted({h for _, h in split_heads(1, N, heads, n_cu)} | {0}))
    return grid, N, heads, q, k, v, hs


@pytest.mark.parametrize("sigma", [0.5, 1.5])
def test_split_tail_four_ranges(sigma):
    grid, N, heads, q, k, v, hs = tail_case(910, sigma)
    got = from_dev(wa.self_attention(to_dev(q), to_dev(k), to_dev(v), grid, theta=THETA))
    torch.cuda.synchronize()
    ref = oracle.self_rows(q[:, :, hs], k[:, :, hs], v[:, :, hs], grid, theta=THETA)
    assert_parity(got[:, :, hs], ref, what=f"split tail, 4 ranges, sigma {sigma}")


def test_split_tail_wide_scores_no_worse_than_unsplit():
    # sigma 2: score std ~4, each range's reference far from the others'.  The
    # bf16 rounding of the scaled queries alone puts the kernel near the max
    # gate here, split or not; the split must add nothing material to it
    grid, N, heads, q, k, v, hs = tail_case(913, 2.0)
    dq, dk, dv = to_dev(q), to_dev(k), to_dev(v)
    ws = torch.empty(N * heads * 128 * 2, dtype=torch.uint8, device="cuda")
    split = from_dev(wa.self_attention(dq, dk, dv, grid, theta=THETA))
    whole = from_dev(wa.self_attention(dq, dk, dv, grid, theta=THETA, workspace=ws))
    torch.cuda.synchronize()
    ref = oracle.self_rows(q[:, :, hs], k[:, :, hs], v[:, :, hs], grid, theta=THETA)
    es, ew = errors(split[:, :, hs], ref), errors(whole[:, :, hs], ref)
    print(f"split {es}\nunsplit {ew}")
    assert es["finite"] and es["rel_rms"] <= 1e-2
    assert es["max_abs"] <= ew["max_abs"] + 2.0 ** -8
    assert es["mean_abs"] <= 1.05 * ew["mean_abs"] + 1e-5


def test_split_tail_with_kv_lens():
    # two batches; the remainder lies in batch 1, whose 1500 visible keys
    # (24 key tiles) allow 3 ranges of 8 key tiles
    grid, N, B = (5, 20, 20), 2000, 2
    n_cu = ncu()
    heads = max(1, (n_cu + n_cu // 4) // 16)
    lens = [N, 1500]
    q, k = (gen((B, N, heads, 128), 911, s, 1.0) for s in (1, 2))
    v = gen((B, N, heads, 128), 911, 3, 0.5)
    got = from_dev(wa.self_attention(to_dev(q), to_dev(k), to_dev(v), grid, theta=THETA, kv_lens=lens))
    torch.cuda.synchronize()
    pairs = split_heads(B, N, heads, n_cu)
    hs = np.array(sorted({h for _, h in pairs} | {0}))
    ref = oracle.self_rows(q[:, :, hs], k[:, :, hs], v[:, :, hs], grid, theta=THETA, kv_lens=lens)
    assert_parity(got[:, :, hs], ref, what="split tail with kv_lens")


def test_split_last_whole_wave_in_two():
    # 12 whole waves of tiles and no remainder: the last wave runs as 2 key
    # ranges per tile; sampled rows of every tile, all split heads
    grid, N = (5, 20, 20), 2000
    n_cu = ncu()
    heads = max(1, 12 * n_cu // 8)
    q, k = (gen((1, N, heads, 128), 914, s, 1.0) for s in (1, 2))
    v = gen((1, N, heads, 128), 914, 3, 0.5)
    got = from_dev(wa.self_attention(to_dev(q), to_dev(k), to_dev(v), grid, theta=THETA))
    torch.cuda.synchronize()
    hs = np.array(sorted({h for _, h in split_heads(1, N, heads, n_cu)} | {0}))
    rows = seeded.sample_rows(N, 48, seed=914, must=tuple(256 * t + x for t in range(8) for x in (0, 255)))
    ref = oracle.self_rows(q[:, :, hs], k[:, :, hs], v[:, :, hs], grid, rows=rows, theta=THETA)
    assert_parity(got[:, rows][:, :, hs], ref, what="last whole wave split in two")


def test_workspace_without_room_turns_the_split_off():
    grid, N = (5, 20, 20), 2000
    n_cu = ncu()
    heads = max(1, (n_cu + n_cu // 4) // 8)
    q, k = (gen((1, N, heads, 128), 912, s, 1.0) for s in (1, 2))
    v = gen((1, N, heads, 128), 912, 3, 0.5)
    dq, dk, dv = to_dev(q), to_dev(k), to_dev(v)
    full = wa.self_workspace_bytes(1, N, heads)
    kbytes = N * heads * 128 * 2
    assert full > kbytes  # the reported size includes room for the partials
    ws = torch.empty(kbytes, dtype=torch.uint8, device="cuda")
    got_small = from_dev(wa.self_attention(dq, dk, dv, grid, theta=THETA, workspace=ws))
    got_full = from_dev(wa.self_attention(dq, dk, dv, grid, theta=THETA))
    torch.cuda.synchronize()
    hs = np.array(sorted({h for _, h in split_heads(1, N, heads, n_cu)}))
    ref = oracle.self_rows(q[:, :, hs], k[:, :, hs], v[:, :, hs], grid, theta=THETA)
    assert_parity(got_small[:, :, hs], ref, what="no room for partials")
    assert_parity(got_full[:, :, hs], ref, what="with room for partials")
    # outside the split tiles both calls run the same workgroups: identical bits
    other = np.setdiff1d(np.arange(heads), hs)
    assert np.array_equal(got_small[:, :, other], got_full[:, :, other])


@pytest.mark.parametrize("name", ["wan14b_720p_81f", "wan14b_480p_81f", "wan14b_480p_165f_causal"])
def test_every_tile_written_at_full_size(name):
    # the persistent launch hands out every query tile exactly once through
    # its work queues: an output filled with NaN beforehand has none left
    wl = seeded.WORKLOADS[name]
    t = seeded.workload_tensors(wl, seed=0, cross=False)
    q, k, v = to_dev(t["q"]), to_dev(t["k"]), to_dev(t["v"])
    o = torch.full_like(q, float("nan"))
    wa.self_attention(q, k, v, (wl.F, wl.H, wl.W), theta=THETA, block_causal=wl.block_causal,
                      chunk_frames=wl.chunk_frames, out=o)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o).all())


def test_full_size_two_batches_with_kv_lens():
    # 32,760 tokens x 40 heads, two batches with 32,760 and 20,000 visible keys:
    # 10,240 tiles = 40 whole waves on 256 CUs, so the last wave (batch 1's
    # last heads) runs as key ranges taken from the shorter batch's length;
    # sampled rows of both batches, every head
    wl = seeded.WORKLOADS["wan14b_480p_81f"]
    grid = (wl.F, wl.H, wl.W)
    B, lens = 2, [wl.N, 20000]
    q, k = (gen((B, wl.N, wl.heads, 128), 915, s, 1.0) for s in (1, 2))
    v = gen((B, wl.N, wl.heads, 128), 915, 3, 0.5)
    o = wa.self_attention(to_dev(q), to_dev(k), to_dev(v), grid, theta=THETA, kv_lens=lens)
    torch.cuda.synchronize()
    rows = seeded.sample_rows(wl.N, 24, seed=915, must=(wl.N - 1, wl.N - 257, 19999, 20000))
    got = from_dev(o[:, torch.from_numpy(rows.astype(np.int64)).cuda()])
    assert bool(torch.isfinite(o.float()).all())
    del o
    ref = oracle.self_rows(q, k, v, grid, rows=rows, theta=THETA, kv_lens=lens)
    assert_parity(got, ref, what="two batches with kv_lens at full size")


def test_split_tail_eight_ranges():
    # 4,320 tokens (17 query tiles, 68 key tiles) x heads so that the launch is
    # one chip of tiles plus a sixteenth: that remainder runs as 8 key ranges
    # (the most the library makes) of 8 or 9 key tiles each
    grid, N = (4, 30, 36), 4320
    n_cu = ncu()
    heads = max(1, (n_cu + n_cu // 16) // 17)
    q, k = (gen((1, N, heads, 128), 916, s, 1.0) for s in (1, 2))
    v = gen((1, N, heads, 128), 916, 3, 0.5)
    got = from_dev(wa.self_attention(to_dev(q), to_dev(k), to_dev(v), grid, theta=THETA))
    torch.cuda.synchronize()
    hs = np.array(sorted({h for _, h in split_heads(1, N, heads, n_cu)} | {0}))
    rows = seeded.sample_rows(N, 96, seed=916, must=tuple(256 * t for t in range(17)) + (N - 1,))
    ref = oracle.self_rows(q[:, :, hs], k[:, :, hs], v[:, :, hs], grid, rows=rows, theta=THETA)
    assert_parity(got[:, rows][:, :, hs], ref, what="split tail, 8 ranges")
