"""GPU parity of cross attention's persistent launch (Wan paper explainer
(0h-n0.github.io), text-encoder section: softmax(Q K_text^T / sqrt(d_k))
V_text; Wan2.2 source reading (blog.leeguoo.com), ch. 4: cross_attn(x,
context, context_lens)).

A launch of at least one workgroup per compute unit takes its query tiles in
a fixed order and loads each next tile's queries and first key tiles during
the current tile's epilogue; tiles whose text has fewer than 4 key tiles
(ctx_len <= 192) are not prefetched.  Every row is compared with the fp64
oracle on a shape with both kinds of tiles, and at full size every output
row must be written (NaN-filled beforehand).
"""
import numpy as np
import pytest
import torch

import oracle
from parity_util import assert_parity, from_dev, to_dev
from video_diffusion_transformer_wanattn_amd import seeded
from video_diffusion_transformer_wanattn_amd import wanattn as wa

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("M,lens,N", [(512, [512, 100], 4096), (512, None, 4096), (77, [77, 1], 4096),
                                       (300, [300, 193], 4096), (512, [512, 300], 3996),
                                       (640, [640, 256], 4096), (512, [320, 448], 4096)])
def test_cross_persistent_every_row(M, lens, N):
    # 2 x 16 x 16 = 512 query tiles: the persistent launch on a 256-CU chip;
    # N = 3996 leaves the last tile of every head with 156 rows, so its last
    # two waves' rows all lie past the last token (their query loads repeat it).
    # Text lengths that are whole 64-key tiles (256, 320, 448, 512, 640) run
    # their last tiles unmasked: 4 tiles (256) only there, 10 tiles (640) and
    # 5 or 7 tiles (320, 448) with a masked remainder after them
    B, heads = 2, 16
    q = seeded.normal_bf16((B, N, heads, 128), 1400 + M + N, 1, 0.5)
    kc = seeded.normal_bf16((B, M, heads, 128), 1400 + M, 2, 0.5)
    vc = seeded.normal_bf16((B, M, heads, 128), 1400 + M, 3, 0.5)
    out = torch.full((B, N, heads, 128), float("nan"), dtype=torch.bfloat16, device="cuda")
    wa.cross_attention(to_dev(q), to_dev(kc), to_dev(vc), ctx_lens=lens, out=out)
    torch.cuda.synchronize()
    got = from_dev(out)
    ref = oracle.cross_rows(q, kc, vc, ctx_lens=lens)
    e = assert_parity(got, ref, what=f"cross persistent M={M} lens={lens} N={N}")
    print(f"cross persistent M={M} lens={lens} N={N}: {e}", flush=True)
    again = wa.cross_attention(to_dev(q), to_dev(kc), to_dev(vc), ctx_lens=lens)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(from_dev(again), got)


def test_cross_every_row_written_at_full_size():
    wl = seeded.WORKLOADS["wan14b_720p_81f"]
    t = seeded.workload_tensors(wl, seed=0, self_attn=False)
    q = to_dev(t["q"])
    o = torch.full_like(q, float("nan"))
    wa.cross_attention(q, to_dev(t["text_k"]), to_dev(t["text_v"]), out=o)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o).all())


def test_cross_repeated_calls_identical_at_full_size():
    # 75,600 x 40 queries against 512 text keys, 40 calls on the same inputs:
    # every output equal to the first, bit for bit.  (A wait at a work item's
    # start that counted the previous item's output stores as the last
    # operations outstanding let some waves read their prefetched queries
    # before the loads landed: a few groups of 4 rows of one head came out
    # wrong in about 1 call in 10.)
    wl = seeded.WORKLOADS["wan14b_720p_81f"]
    t = seeded.workload_tensors(wl, seed=1, self_attn=False)
    q, kc, vc = to_dev(t["q"]), to_dev(t["text_k"]), to_dev(t["text_v"])
    first = wa.cross_attention(q, kc, vc)
    o = torch.empty_like(first)
    differ = []
    for i in range(40):
        wa.cross_attention(q, kc, vc, out=o)
        torch.cuda.synchronize()
        n = int((o.view(torch.int16) != first.view(torch.int16)).sum())
        if n:
            differ.append((i, n))
    assert not differ, differ
