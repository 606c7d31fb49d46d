"""Classifier-free guidance batching (Wan2.2 source reading (blog.leeguoo.com):
the sampler evaluates the conditional and the unconditional prediction, and the
context lengths come from each trimmed prompt): one launch with B = 2 for the
same latent tokens and two different text contexts of different lengths.
"""
import numpy as np
import pytest
import torch

import oracle
from parity_util import assert_parity, from_dev, split_heads, to_dev
from video_diffusion_transformer_wanattn_amd import seeded
from video_diffusion_transformer_wanattn_amd import wanattn as wa

pytestmark = pytest.mark.gpu
THETA = 10000.0


def test_cfg_pair_in_one_launch_32760_tokens():
    wl = seeded.WORKLOADS["wan14b_480p_81f"]
    grid = (wl.F, wl.H, wl.W)
    t = seeded.workload_tensors(wl, seed=0)
    # the same latent for both samples; the unconditional context is another prompt
    tu = seeded.normal_bf16((1, wl.text_len, wl.heads, 128), 3, 16 * wl.wid + 9, wl.sigma)
    tv = seeded.normal_bf16((1, wl.text_len, wl.heads, 128), 3, 16 * wl.wid + 10, wl.sigma)
    q2, k2, v2 = (np.concatenate([t[n], t[n]]) for n in ("q", "k", "v"))
    kc2 = np.concatenate([t["text_k"], tu])
    vc2 = np.concatenate([t["text_v"], tv])
    lens = [77, 23]
    q, k, v = to_dev(q2), to_dev(k2), to_dev(v2)
    o = wa.self_attention(q, k, v, grid, theta=THETA)
    oc = wa.cross_attention(q, to_dev(kc2), to_dev(vc2), ctx_lens=lens)
    torch.cuda.synchronize()
    # identical inputs give identical self-attention outputs in both samples,
    # bit for bit on the tiles both run whole; the launch's last wave (the
    # last heads of sample 1) runs as two key ranges combined in another
    # order: there the two differ by rounding only (at most 2 bf16 steps of
    # the largest output), and both samples are held to the oracle below
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    split = sorted({h for _, h in split_heads(2, wl.N, wl.heads, n_cu)})
    whole = [h for h in range(wl.heads) if h not in split]
    assert torch.equal(o[0][:, whole], o[1][:, whole])
    if split:
        a, b = o[0][:, split].float(), o[1][:, split].float()
        assert float((a - b).abs().max()) <= 2.0 ** -6 * float(a.abs().max())
    rows = seeded.sample_rows(wl.N, 32, seed=11, must=(wl.N - 1, wl.N - 300, wl.N - 3000))
    idx = torch.from_numpy(rows.astype(np.int64)).cuda()
    got_s = from_dev(o[:, idx])
    got_c = from_dev(oc[:, idx])
    del q, k, v, o, oc
    ref_s = oracle.self_rows(t["q"], t["k"], t["v"], grid, rows=rows, theta=THETA)
    assert_parity(got_s[:1], ref_s, what="cfg self, sample 0")
    assert_parity(got_s[1:], ref_s, what="cfg self, sample 1")
    ref_c = oracle.cross_rows(q2, kc2, vc2, rows=rows, ctx_lens=lens)
    assert_parity(got_c, ref_c, what="cfg cross")
    # the two contexts really differ in the result
    assert np.abs(ref_c[0] - ref_c[1]).max() > 1e-3
