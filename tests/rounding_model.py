"""A numpy model of the roundings the HIP self-attention path makes, for
explaining its error against the fp64 oracle (test code: it shares nothing
with the oracle or the kernels and models only where values are rounded).

The kernel, per (batch, head):
  k' = bf16( rotate_fp32(k) )                     the key rotation pass
  q' = bf16( rotate_fp32(q) * fp32(scale log2 e) ) the attention kernel's Q load
  s  = q' . k'  accumulated in fp32                (bf16 MFMA)
  p  = exp2(s - m)  in fp32                       (m: the row reference)
  l  = sum p  (fp32, unrounded p)
  O  = sum bf16(p) v  (fp32)                      (bf16 MFMA)
  o  = bf16( O * (1 / l) )
where rotate_fp32 multiplies each (re, im) pair by (cos, sin) values computed
in fp64 and rounded to fp32.  Where the kernel keeps a lazy reference (m moves
only when p would exceed 2^12), p carries the same relative rounding at any
reference, so the model uses the row maximum.
"""
import numpy as np

from video_diffusion_transformer_wanattn_amd import seeded

WIDTHS = (44, 42, 42)   # time, height, width segments of a 128-wide head
LOG2E = 1.4426950408889634


def bf16(x):
    """float32 values rounded to bf16 (nearest even), as float32."""
    return seeded.bf16_bits_to_f32(seeded.f32_to_bf16_bits_array(np.asarray(x, np.float32)))


def pair_tables(theta, positions):
    """fp32 (cos, sin) for each of the 64 pairs at integer positions
    [n, 3] -> two float32 arrays [n, 64]."""
    ang = []
    for a, D in enumerate(WIDTHS):
        k = np.arange(D // 2, dtype=np.float64)
        w = np.power(float(theta), -2.0 * k / D)
        ang.append(positions[:, a:a + 1].astype(np.float64) * w[None, :])
    ang = np.concatenate(ang, axis=1)
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


def rotate_fp32(x_bits, positions, theta):
    """[n, 128] bf16 bits rotated in fp32 -> float32 [n, 128]."""
    x = seeded.bf16_bits_to_f32(x_bits).astype(np.float32)
    c, s = pair_tables(theta, positions)
    re, im = x[:, 0::2], x[:, 1::2]
    out = np.empty_like(x)
    out[:, 0::2] = re * c - im * s
    out[:, 1::2] = re * s + im * c
    return out


def grid_positions(grid, offsets=(0, 0, 0)):
    F, H, W = grid
    n = np.arange(F * H * W)
    return np.stack([n // (H * W) + offsets[0], (n // W) % H + offsets[1], n % W + offsets[2]], axis=1)


def self_attention(q_bits, k_bits, v_bits, grid, theta=10000.0, scale=None, rows=None):
    """Bidirectional self attention of one batch, every head: [N, heads, 128]
    bf16 bits -> float32 [len(rows), heads, 128] (bf16 values)."""
    N, heads, d = q_bits.shape
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    rows = np.arange(N) if rows is None else np.asarray(rows)
    pos = grid_positions(grid)
    qscale = np.float32(np.float32(scale) * np.float32(LOG2E))
    out = np.empty((len(rows), heads, d), np.float32)
    for h in range(heads):
        kp = bf16(rotate_fp32(k_bits[:, h], pos, theta))
        qp = bf16(rotate_fp32(q_bits[rows, h], pos[rows], theta) * qscale)
        v = seeded.bf16_bits_to_f32(v_bits[:, h]).astype(np.float32)
        s = qp @ kp.T                                  # fp32 accumulation
        p = np.exp2(s - s.max(axis=1, keepdims=True)).astype(np.float32)
        l = p.sum(axis=1, dtype=np.float32)
        o = bf16(p) @ v
        out[:, h] = bf16(o * (np.float32(1.0) / l)[:, None])
    return out


def with_roundings(q, k, v, grid, round_qk, round_p, round_o, theta=10000.0):
    """fp64 attention of batch 0 ([1, N, heads, 128] bf16 bits) with only the
    chosen roundings of the path applied: the bf16 q' and k' operands, the
    bf16 probabilities, the bf16 output.  float64 [N, heads, 128]."""
    N, heads = q.shape[1], q.shape[2]
    pos = grid_positions(grid)
    out = np.empty((N, heads, 128))
    for h in range(heads):
        kp = rotate_fp32(k[0][:, h], pos, theta).astype(np.float64)
        qp = rotate_fp32(q[0][:, h], pos, theta).astype(np.float64) * (LOG2E / np.sqrt(128))
        if round_qk:
            kp, qp = bf16(kp).astype(np.float64), bf16(qp).astype(np.float64)
        vv = seeded.bf16_bits_to_f32(v[0][:, h]).astype(np.float64)
        s = qp @ kp.T
        p = np.exp2(s - s.max(axis=1, keepdims=True))
        l = p.sum(axis=1)
        o = ((bf16(p).astype(np.float64) if round_p else p) @ vv) / l[:, None]
        out[:, h] = bf16(o) if round_o else o
    return out
