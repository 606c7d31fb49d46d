"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle on the
same seeded bf16 inputs, element by element.

Small shapes are compared on every row and span several 256-row query tiles
and 64-key tiles with ragged tails; the five workload shapes run at full size
in the launch configuration the benchmark times, compared on sampled rows.
"""

import numpy as np
import pytest
import torch

import oracle
from parity_util import assert_parity, from_dev, plant_needles, to_dev, widen
from video_diffusion_transformer_wanattn_amd import seeded
from video_diffusion_transformer_wanattn_amd import wanattn as wa

pytestmark = pytest.mark.gpu
THETA = 10000.0


def gen(shape, seed, stream, sigma=0.5):
    return seeded.normal_bf16(shape, seed, stream, sigma)


def qkv(B, N, heads, seed, sigma=0.5):
    """q and k ~ N(0,1)*sigma; v stays at the workloads' 0.5 (the output scale)."""
    return [gen((B, N, heads, 128), seed, s, sg) for s, sg in ((1, sigma), (2, sigma), (3, 0.5))]


def gpu_self(q, k, v, grid, **kw):
    out = wa.self_attention(to_dev(q), to_dev(k), to_dev(v), grid, theta=THETA, **kw)
    torch.cuda.synchronize()
    return from_dev(out)


def gpu_cross(q, kc, vc, **kw):
    out = wa.cross_attention(to_dev(q), to_dev(kc), to_dev(vc), **kw)
    torch.cuda.synchronize()
    return from_dev(out)


def rope_mat(x_bits, pos):
    return oracle.rope_vec(widen(x_bits), pos, THETA)


# ---------------------------------------------------------------------------
# tiny workload, every row
# ---------------------------------------------------------------------------

def test_tiny_workload_self_and_cross():
    wl = seeded.WORKLOADS["tiny"]
    t = seeded.workload_tensors(wl, seed=0)
    grid = (wl.F, wl.H, wl.W)
    got = gpu_self(t["q"], t["k"], t["v"], grid)
    ref = oracle.self_rows(t["q"], t["k"], t["v"], grid, theta=THETA)
    assert_parity(got, ref, what="tiny self")
    got = gpu_cross(t["q"], t["text_k"], t["text_v"])
    ref = oracle.cross_rows(t["q"], t["text_k"], t["text_v"])
    assert_parity(got, ref, what="tiny cross")


@pytest.mark.parametrize("grid,heads,B", [((1, 1, 1), 1, 1), ((3, 5, 7), 3, 2), ((7, 9, 11), 2, 1),
                                          ((2, 16, 16), 2, 2), ((5, 13, 11), 1, 1)])
def test_self_ragged_shapes(grid, heads, B):
    N = int(np.prod(grid))
    q, k, v = qkv(B, N, heads, seed=100 + N)
    assert_parity(gpu_self(q, k, v, grid), oracle.self_rows(q, k, v, grid, theta=THETA),
                  what=f"self {grid}")


def test_self_kv_lens():
    grid = (5, 8, 13)
    q, k, v = qkv(3, 520, 2, seed=7)
    lens = [1, 77, 520]
    got = gpu_self(q, k, v, grid, kv_lens=lens)
    ref = oracle.self_rows(q, k, v, grid, theta=THETA, kv_lens=lens)
    assert_parity(got, ref, what="kv_lens")
    # a single visible key returns its value exactly
    np.testing.assert_array_equal(got[0], np.broadcast_to(v[0, :1], got[0].shape))


@pytest.mark.parametrize("grid,chunk", [((9, 6, 10), 3), ((6, 5, 7), 2), ((5, 8, 8), 1), ((4, 6, 9), 9),
                                        ((14, 4, 5), 3)])
def test_self_block_causal(grid, chunk):
    N = int(np.prod(grid))
    q, k, v = qkv(1, N, 2, seed=200 + N + chunk)
    got = gpu_self(q, k, v, grid, block_causal=True, chunk_frames=chunk)
    ref = oracle.self_rows(q, k, v, grid, theta=THETA, block_causal=True, chunk_frames=chunk)
    assert_parity(got, ref, what=f"block-causal {grid} chunk {chunk}")


def test_block_causal_with_kv_lens():
    grid = (6, 6, 8)
    q, k, v = qkv(2, 288, 2, seed=31)
    lens = [100, 288]
    got = gpu_self(q, k, v, grid, block_causal=True, chunk_frames=2, kv_lens=lens)
    ref = oracle.self_rows(q, k, v, grid, theta=THETA, block_causal=True, chunk_frames=2, kv_lens=lens)
    assert_parity(got, ref, what="block-causal + kv_lens")


@pytest.mark.parametrize("M", [1, 7, 32, 100, 512])
def test_cross_ragged(M):
    q = gen((2, 300, 3, 128), 40 + M, 1)
    kc, vc = gen((2, M, 3, 128), 40 + M, 2), gen((2, M, 3, 128), 40 + M, 3)
    assert_parity(gpu_cross(q, kc, vc), oracle.cross_rows(q, kc, vc), what=f"cross M={M}")
    lens = [max(1, M // 3), M]
    assert_parity(gpu_cross(q, kc, vc, ctx_lens=lens), oracle.cross_rows(q, kc, vc, ctx_lens=lens),
                  what=f"cross M={M} ctx_lens")


# ---------------------------------------------------------------------------
# discriminating inputs
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("grid", [(5, 8, 8), (21, 6, 8)])
def test_peaked_scores(grid):
    # sigma 1.5: score std ~2.25, the running max moves often
    N = int(np.prod(grid))
    q, k, v = qkv(1, N, 2, seed=300 + N, sigma=1.5)
    assert_parity(gpu_self(q, k, v, grid), oracle.self_rows(q, k, v, grid, theta=THETA),
                  what=f"peaked {grid}")
    kc, vc = gen((1, 77, 2, 128), 301, 4, 1.5), gen((1, 77, 2, 128), 301, 5)
    assert_parity(gpu_cross(q, kc, vc), oracle.cross_rows(q, kc, vc), what="peaked cross")


def test_planted_needles_check_rope_positions():
    grid = (5, 8, 8)
    N = 320
    q, k, v = qkv(1, N, 2, seed=400)
    rng = np.random.default_rng(1)
    js = rng.permutation(N)[:64]
    is_ = rng.permutation(N)[:64]
    k = plant_needles(q, k, grid, list(zip(is_, js)))
    got = gpu_self(q, k, v, grid)
    ref = oracle.self_rows(q, k, v, grid, theta=THETA)
    assert_parity(got, ref, what="needles")
    for i, j in zip(is_, js):
        np.testing.assert_allclose(widen(got[0, i]), widen(v[0, j]), atol=3e-2)


def test_mask_needles_in_later_chunks_have_no_effect():
    grid = (6, 4, 5)   # 20 tokens per frame, chunks of 2 frames = 40 tokens
    N = 120
    q, k, v = qkv(1, N, 2, seed=500)
    pairs = [(3, 45), (39, 40), (41, 119), (60, 85)]   # key j always in a later chunk than row i
    kn = plant_needles(q, k, grid, pairs)
    got = gpu_self(q, kn, v, grid, block_causal=True, chunk_frames=2)
    ref = oracle.self_rows(q, kn, v, grid, theta=THETA, block_causal=True, chunk_frames=2)
    assert_parity(got, ref, what="mask needles")
    bidir = gpu_self(q, kn, v, grid)
    for i, j in pairs:
        # visible (bidirectional) the needle takes the row; masked it has no pull
        np.testing.assert_allclose(widen(bidir[0, i]), widen(v[0, j]), atol=3e-2)
        assert np.max(np.abs(widen(got[0, i]) - widen(v[0, j]))) > 0.1


# ---------------------------------------------------------------------------
# invariants on the GPU
# ---------------------------------------------------------------------------

def test_gpu_invariants():
    grid = (5, 8, 8)
    N = 320
    q, k, v = qkv(1, N, 3, seed=600, sigma=1.5)
    ones = np.full((1, N, 3, 128), 0x3F80, np.uint16)
    got = widen(gpu_self(q, k, ones, grid))
    assert np.max(np.abs(got - 1.0)) <= 2 ** -7
    row = v[:, :1]
    const = np.ascontiguousarray(np.broadcast_to(row, v.shape))
    got = widen(gpu_self(q, k, const, grid))
    np.testing.assert_allclose(got, np.broadcast_to(widen(row), got.shape), rtol=2 ** -7, atol=1e-6)
    got = gpu_self(q, k, v, grid, kv_lens=[1])
    np.testing.assert_array_equal(got, np.broadcast_to(v[:, :1], got.shape))
    # a common shift of every position leaves the output unchanged (bf16 noise)
    a = gpu_self(q, k, v, grid)
    b = gpu_self(q, k, v, grid, offsets=(3, 100, 900))
    ref = oracle.self_rows(q, k, v, grid, theta=THETA)
    assert_parity(a, ref, what="offset 0")
    assert_parity(b, ref, what="offset shifted")
    assert_parity(b, widen(a), what="shifted vs unshifted")


def test_deterministic():
    grid = (7, 9, 11)
    q, k, v = qkv(1, 693, 2, seed=700)
    a = gpu_self(q, k, v, grid)
    b = gpu_self(q, k, v, grid)
    np.testing.assert_array_equal(a, b)


@pytest.mark.parametrize("heads", [3, 1, 5, 9])
def test_rope3d_matches_oracle(heads):
    # one wave per token row, lane group hq taking heads hq, hq + 4, ...:
    # head counts below 4 and not a multiple of 4 leave groups idle or uneven
    grid = (5, 7, 9)
    x = gen((2, 315, heads, 128), 800 + heads, 1, 1.0)
    ref = oracle.rope3d(x, grid, THETA, offsets=(4, 2, 1))
    xd = to_dev(x)
    y = from_dev(wa.rope3d(xd, grid, THETA, offsets=(4, 2, 1)))
    err = np.abs(widen(y) - ref)
    # bf16 rounding (half an ulp: 2^-9 relative) plus the fp32 rotation error
    assert np.all(err <= 2 ** -8 * np.abs(ref) + 1e-5), float(np.max(err))
    wa.rope3d(xd, grid, THETA, offsets=(4, 2, 1), out=xd)       # in place
    torch.cuda.synchronize()
    np.testing.assert_array_equal(from_dev(xd), y)


def test_errors_raise_without_launch():
    q = torch.zeros(1, 24, 2, 128, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(wa.WanattnError):
        wa.self_attention(q, q.clone(), q.clone(), (2, 3, 3))
    with pytest.raises(wa.WanattnError):
        wa.self_attention(q, q.clone(), q.clone(), (2, 3, 4), block_causal=True, chunk_frames=0)
    with pytest.raises(wa.WanattnError):
        wa.self_attention(q, q.clone(), q.clone(), (2, 3, 4), out=q)


# ---------------------------------------------------------------------------
# the five workload shapes at full size, sampled rows
# ---------------------------------------------------------------------------

FULL = ["wan13b_480p_81f", "wan14b_480p_81f", "wan14b_720p_81f", "wan14b_480p_165f_causal"]


@pytest.mark.parametrize("name", FULL)
def test_full_size_workload_sampled_rows(name):
    wl = seeded.WORKLOADS[name]
    grid = (wl.F, wl.H, wl.W)
    t = seeded.workload_tensors(wl, seed=0)
    # the last query tiles of the last heads run as key-split workgroups when
    # the launch ends in a partial wave: rows from the last tiles of every head
    must = (wl.N - 1, wl.N - 257, wl.N - 3000)
    if wl.block_causal:
        ct = wl.chunk_frames * wl.H * wl.W
        must += tuple(x for c in range(wl.N // ct) for x in (c * ct, (c + 1) * ct - 1))
    rows = seeded.sample_rows(wl.N, 40, seed=wl.wid, must=must)
    q, k, v = to_dev(t["q"]), to_dev(t["k"]), to_dev(t["v"])
    o = wa.self_attention(q, k, v, grid, theta=THETA, block_causal=wl.block_causal,
                          chunk_frames=wl.chunk_frames)
    oc = wa.cross_attention(q, to_dev(t["text_k"]), to_dev(t["text_v"]))
    torch.cuda.synchronize()
    o_rows = from_dev(o[:, torch.from_numpy(rows.astype(np.int64)).cuda()])
    oc_rows = from_dev(oc[:, torch.from_numpy(rows.astype(np.int64)).cuda()])
    assert bool(torch.isfinite(o.float()).all()) and bool(torch.isfinite(oc.float()).all())
    del q, k, v, o, oc
    ref = oracle.self_rows(t["q"], t["k"], t["v"], grid, rows=rows, theta=THETA,
                           block_causal=wl.block_causal, chunk_frames=wl.chunk_frames)
    assert_parity(o_rows, ref, what=f"{name} self")
    refc = oracle.cross_rows(t["q"], t["text_k"], t["text_v"], rows=rows)
    assert_parity(oc_rows, refc, what=f"{name} cross")
