"""Seeded synthetic inputs shared by the oracle side and the HIP side.

Nothing here computes attention or rotary embeddings.  The module turns a
(seed, stream) pair into bf16 bit patterns of N(0,1)*sigma samples with the
counter-based generator defined in ``seeded.c`` (SplitMix64 output function +
Box-Muller), and records the workload shapes that the pages describe:

* Wan2.2 source reading (blog.leeguoo.com), ch. 4 "DiT: 75600 token attention":
  patch size (1, 2, 2), 3,600 tokens per latent frame and 75,600 tokens for an
  81-frame 720p clip; head dim 5120 / 40 = 128.
* Long-video survey (atlascloud.ai), "Why long video is hard": about 32.7k
  tokens at 81 frames and 65.5k at 165 frames (480p).
* Same survey, "Route 3: Self Forcing": bidirectional attention replaced by
  causal attention over chunks, with earlier chunks kept as a KV cache.

The values are synthetic: the pages' workload is activations of trained
models, which are not available, so seeded Gaussians of the same shapes stand
in for them.
"""
from __future__ import annotations

import ctypes
import hashlib
import os
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libseeded.so")
# tests/test_sanitizers.py points this at a build with the address and
# undefined-behaviour sanitizers
_OVERRIDE = os.environ.get("WANATTN_SEEDED_LIB")

# Tensor ids inside a workload; stream = workload_id * 16 + tensor id.
Q, K, V, TEXT_K, TEXT_V = 0, 1, 2, 3, 4


@dataclass(frozen=True)
class Workload:
    name: str
    wid: int          # workload id, part of the stream number
    F: int            # latent frames
    H: int            # token rows per frame
    W: int            # token columns per frame
    heads: int
    head_dim: int
    text_len: int     # cross-attention keys (text tokens)
    block_causal: bool
    chunk_frames: int  # latent frames per causal chunk (used iff block_causal)
    sigma: float = 0.5
    batch: int = 1

    @property
    def N(self) -> int:
        return self.F * self.H * self.W

    @property
    def tensor_bytes(self) -> int:
        return self.batch * self.N * self.heads * self.head_dim * 2


WORKLOADS = {
    "tiny": Workload("tiny", 1, 5, 8, 8, 4, 128, 32, False, 3),
    "wan13b_480p_81f": Workload("wan13b_480p_81f", 2, 21, 30, 52, 12, 128, 512, False, 3),
    "wan14b_480p_81f": Workload("wan14b_480p_81f", 3, 21, 30, 52, 40, 128, 512, False, 3),
    "wan14b_720p_81f": Workload("wan14b_720p_81f", 4, 21, 45, 80, 40, 128, 512, False, 3),
    "wan14b_480p_165f_causal": Workload("wan14b_480p_165f_causal", 5, 42, 30, 52, 40, 128, 512, True, 3),
}


_lib = None


def _load():
    global _lib
    if _lib is None:
        path = _OVERRIDE or LIB_PATH
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: run __graft_entry__.build() first")
        lib = ctypes.CDLL(path)
        lib.seeded_normal_bf16.restype = ctypes.c_int
        lib.seeded_normal_bf16.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint64,
                                           ctypes.c_uint64, ctypes.c_uint64, ctypes.c_double,
                                           ctypes.c_int]
        lib.seeded_word.restype = ctypes.c_uint64
        lib.seeded_word.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint64]
        lib.seeded_f32_to_bf16.restype = ctypes.c_uint16
        lib.seeded_f32_to_bf16.argtypes = [ctypes.c_float]
        _lib = lib
    return _lib


def default_threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def normal_bf16(shape, seed: int, stream: int, sigma: float, threads: int | None = None,
                with_f32: bool = False):
    """bf16 bit patterns (uint16 array of ``shape``) of N(0,1)*sigma samples."""
    lib = _load()
    n = int(np.prod(shape)) if len(shape) else 1
    out = np.empty(shape, dtype=np.uint16)
    f32 = np.empty(shape, dtype=np.float32) if with_f32 else None
    rc = lib.seeded_normal_bf16(out.ctypes.data, f32.ctypes.data if with_f32 else None,
                                n, seed, stream, sigma, threads or default_threads())
    if rc != 0:
        raise RuntimeError("seeded_normal_bf16 failed")
    return (out, f32) if with_f32 else out


def word(seed: int, stream: int, k: int) -> int:
    return int(_load().seeded_word(seed, stream, k))


def f32_to_bf16_bits(x: float) -> int:
    return int(_load().seeded_f32_to_bf16(x))


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def f32_to_bf16_bits_array(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 bit patterns (nearest even), vectorised."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    nan = np.isnan(np.asarray(x, dtype=np.float32))
    if nan.any():
        r[nan] = 0x7FC0
    return r


def workload_tensors(wl: Workload, seed: int = 0, threads: int | None = None,
                     self_attn: bool = True, cross: bool = True):
    """Q, K, V ([B, N, heads, d]) and text K, V ([B, M, heads, d]) as bf16 bits."""
    base = wl.wid * 16
    shp = (wl.batch, wl.N, wl.heads, wl.head_dim)
    tshp = (wl.batch, wl.text_len, wl.heads, wl.head_dim)
    out = {"q": normal_bf16(shp, seed, base + Q, wl.sigma, threads)}
    if self_attn:
        out["k"] = normal_bf16(shp, seed, base + K, wl.sigma, threads)
        out["v"] = normal_bf16(shp, seed, base + V, wl.sigma, threads)
    if cross:
        out["text_k"] = normal_bf16(tshp, seed, base + TEXT_K, wl.sigma, threads)
        out["text_v"] = normal_bf16(tshp, seed, base + TEXT_V, wl.sigma, threads)
    return out


PROLOGUE_STREAM = 1 << 20   # stream numbers of the prologue tensors start here


def prologue_tensors(B: int, N: int, dim: int, seed: int = 0, x_sigma: float = 1.0,
                     x_shift: float = 0.0, mod_sigma: float = 0.5, threads: int | None = None):
    """Inputs of the self-attention prologue as bf16 bits (e0/e1 as float32):
    x [B, N, dim] ~ N(x_shift, x_sigma^2); Wq, Wk, Wv [dim, dim] ~ N(0, 1/dim)
    (nn.Linear layout); biases ~ N(0, 0.1^2); RMSNorm gammas 1 + N(0, 0.1^2);
    the modulation shift e0 and scale e1 [B, dim] ~ N(0, mod_sigma^2)."""
    st = PROLOGUE_STREAM
    g = lambda shape, i, sig: normal_bf16(shape, seed, st + i, sig, threads)
    x = g((B, N, dim), 0, x_sigma)
    if x_shift:
        x = f32_to_bf16_bits_array(bf16_bits_to_f32(x) + np.float32(x_shift))
    w = [g((dim, dim), 1 + i, 1.0 / np.sqrt(dim)) for i in range(3)]
    b = [g((dim,), 4 + i, 0.1) for i in range(3)]
    gam = [f32_to_bf16_bits_array(np.float32(1.0) + bf16_bits_to_f32(g((dim,), 7 + i, 0.1))) for i in range(2)]
    e0 = bf16_bits_to_f32(g((B, dim), 9, mod_sigma)).copy()
    e1 = bf16_bits_to_f32(g((B, dim), 10, mod_sigma)).copy()
    return {"x": x, "e0": e0, "e1": e1, "wq": w[0], "wk": w[1], "wv": w[2], "bq": b[0], "bk": b[1],
            "bv": b[2], "gq": gam[0], "gk": gam[1]}


JITTER_STREAM = (1 << 20) + 64   # stream of the per-head RoPE base draws


def jitter_thetas(heads: int, seed: int = 0, theta: float = 10000.0, sigma: float = 0.1) -> np.ndarray:
    """Per-head RoPE bases theta * (1 + eps_h), eps_h ~ N(0, sigma^2) rounded to
    bf16 (the random draws of multi-head RoPE jitter, passed to both sides)."""
    eps = bf16_bits_to_f32(normal_bf16((heads,), seed, JITTER_STREAM, sigma)).astype(np.float64)
    return theta * (1.0 + eps)


def sha256(a: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


def sample_rows(N: int, R: int, seed: int, must: tuple = ()) -> np.ndarray:
    """Sorted distinct query rows: row 0, row N-1, the last partial 256-row
    tile, any ``must`` rows, and seeded-uniform rows up to R in total."""
    rows = {0, N - 1}
    tail0 = (N // 256) * 256
    for r in (tail0, tail0 + 1, (tail0 + N - 1) // 2):
        if 0 <= r < N:
            rows.add(r)
    for r in must:
        if 0 <= r < N:
            rows.add(int(r))
    rng = np.random.Generator(np.random.Philox(seed))
    while len(rows) < min(R, N):
        rows.add(int(rng.integers(0, N)))
    return np.array(sorted(rows), dtype=np.int32)
