"""ORACLE -- test infrastructure only.

A plain fp64 CPU statement of the Wan 3D-RoPE self/cross attention (see the
header of ``wanattn_oracle.c`` for the pages and sections each function
follows).  Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s
``cpu_baseline`` leg may import this package; the HIP library never does and
shares no code with it.

Inputs are bf16 bit patterns (uint16 numpy arrays); outputs are float64.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(_HERE, "wanattn_oracle.c")
LIB_PATH = os.path.join(_HERE, "liboracle.so")
# tests/test_oracle_mutants.py points this at deliberately broken builds of the
# oracle to show that the pins catch them
_OVERRIDE = os.environ.get("WANATTN_ORACLE_LIB")

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with the host C compiler (no GPU code involved)."""
    if force or not os.path.exists(LIB_PATH):
        tmp = LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread",
                               "-o", tmp, SRC, "-lm"])
        os.replace(tmp, LIB_PATH)
    return LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if _OVERRIDE:
            lib = ctypes.CDLL(_OVERRIDE)
        else:
            if not os.path.exists(LIB_PATH):
                build(force=False)
            lib = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        i32 = ctypes.c_int
        f64 = ctypes.c_double
        lib.orc_axis_dims.argtypes = [i32, P]
        lib.orc_axis_dims.restype = None
        lib.orc_omega.argtypes = [f64, i32, i32]
        lib.orc_omega.restype = f64
        lib.orc_decode.argtypes = [i32, i32, i32, P]
        lib.orc_decode.restype = None
        lib.orc_rope_vec.argtypes = [P, P, i32, i32, i32, i32, f64]
        lib.orc_rope_vec.restype = None
        lib.orc_rope3d.argtypes = [P, P, i32, i32, i32, i32, i32, i32, i32, i32, i32, i32, f64]
        lib.orc_rope3d.restype = None
        lib.orc_self_rows.argtypes = [P, P, P, i32, i32, i32, i32, i32, i32, i32, i32, i32, i32,
                                      f64, f64, i32, i32, P, i32, P, P, i32]
        lib.orc_self_rows.restype = i32
        lib.orc_self_rows_heads.argtypes = [P, P, P, i32, i32, i32, i32, i32, i32, i32, i32, i32, i32,
                                            P, f64, i32, i32, P, i32, P, P, i32]
        lib.orc_self_rows_heads.restype = i32
        lib.orc_cross_rows.argtypes = [P, P, P, i32, i32, i32, i32, i32, f64, P, i32, P, P, i32]
        lib.orc_kv_rows.argtypes = [P, P, P, i32, i32, i32, i32, i32, i32, i32, i32, i32, i32, i32, i32,
                                    f64, f64, P, i32, P, P, i32]
        lib.orc_kv_rows.restype = i32
        lib.orc_kv_rows_heads.argtypes = [P, P, P, i32, i32, i32, i32, i32, i32, i32, i32, i32, i32, i32,
                                          i32, P, f64, P, i32, P, P, i32]
        lib.orc_kv_rows_heads.restype = i32
        lib.orc_prologue_rows.argtypes = [P] * 11 + [i32, i32, i32, f64, f64, i32, P, P, P, P, i32]
        lib.orc_prologue_rows.restype = i32
        lib.orc_cross_rows.restype = i32
        lib.orc_token_grid.argtypes = [i32, i32, i32, P]
        lib.orc_token_grid.restype = None
        _lib = lib
    return _lib


def _threads(n):
    return int(n) if n else max(1, min(16, os.cpu_count() or 1))


def _u16(a):
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint16:
        raise TypeError("oracle inputs are bf16 bit patterns (uint16)")
    return a


def axis_dims(head_dim: int):
    out = np.zeros(3, dtype=np.int32)
    _load().orc_axis_dims(head_dim, out.ctypes.data)
    return tuple(int(x) for x in out)


def omega(theta: float, D: int, k: int) -> float:
    return float(_load().orc_omega(theta, D, k))


def decode(n: int, H: int, W: int):
    out = np.zeros(3, dtype=np.int32)
    _load().orc_decode(n, H, W, out.ctypes.data)
    return tuple(int(x) for x in out)


def token_grid(frames: int, height: int, width: int):
    out = np.zeros(3, dtype=np.int32)
    _load().orc_token_grid(frames, height, width, out.ctypes.data)
    return tuple(int(x) for x in out)


def rope_vec(x, pos, theta: float = 10000.0):
    """Rotate one fp64 head vector at RoPE positions pos = (pf, ph, pw)."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    y = np.empty_like(x)
    _load().orc_rope_vec(x.ctypes.data, y.ctypes.data, x.shape[0], int(pos[0]), int(pos[1]),
                         int(pos[2]), theta)
    return y


def rope3d(x, grid, theta: float = 10000.0, offsets=(0, 0, 0)):
    """fp64 RoPE of a bf16 tensor [B, N, heads, d] on grid (F, H, W)."""
    x = _u16(x)
    B, N, heads, d = x.shape
    F, H, W = grid
    assert N == F * H * W
    y = np.empty(x.shape, dtype=np.float64)
    _load().orc_rope3d(x.ctypes.data, y.ctypes.data, B, N, heads, d, F, H, W, *offsets, theta)
    return y


def self_rows(q, k, v, grid, rows=None, theta: float = 10000.0, scale: float | None = None,
              block_causal: bool = False, chunk_frames: int = 1, kv_lens=None,
              offsets=(0, 0, 0), threads: int | None = None, theta_per_head=None):
    """Self attention with 3D RoPE for query ``rows`` (all rows if None).
    ``theta_per_head`` ([heads], optional): multi-head RoPE jitter, head h
    rotating with its own base (``theta`` is then unused).

    Returns fp64 [B, len(rows), heads, d]."""
    q, k, v = _u16(q), _u16(k), _u16(v)
    B, N, heads, d = q.shape
    assert k.shape == q.shape and v.shape == q.shape
    F, H, W = grid
    if rows is None:
        rows = np.arange(N, dtype=np.int32)
    rows = np.ascontiguousarray(rows, dtype=np.int32)
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    kvl = None if kv_lens is None else np.ascontiguousarray(kv_lens, dtype=np.int32)
    out = np.empty((B, rows.shape[0], heads, d), dtype=np.float64)
    if theta_per_head is not None:
        th = np.ascontiguousarray(theta_per_head, dtype=np.float64)
        if th.shape != (heads,):
            raise ValueError("theta_per_head needs one value per head")
        rc = _load().orc_self_rows_heads(q.ctypes.data, k.ctypes.data, v.ctypes.data, B, N, heads, d, F, H,
                                         W, int(offsets[0]), int(offsets[1]), int(offsets[2]), th.ctypes.data,
                                         scale, 1 if block_causal else 0, int(chunk_frames),
                                         None if kvl is None else kvl.ctypes.data, rows.shape[0],
                                         rows.ctypes.data, out.ctypes.data, _threads(threads))
        if rc != 0:
            raise ValueError("orc_self_rows_heads rejected its arguments")
        return out
    rc = _load().orc_self_rows(q.ctypes.data, k.ctypes.data, v.ctypes.data, B, N, heads, d, F, H, W,
                               int(offsets[0]), int(offsets[1]), int(offsets[2]), theta, scale,
                               1 if block_causal else 0, int(chunk_frames),
                               None if kvl is None else kvl.ctypes.data, rows.shape[0],
                               rows.ctypes.data, out.ctypes.data, _threads(threads))
    if rc != 0:
        raise ValueError("orc_self_rows rejected its arguments")
    return out


def kv_rows(q, k, v, grid_q, kv_frame0: int = 0, rows=None, theta: float = 10000.0,
            scale: float | None = None, kv_lens=None, threads: int | None = None, theta_per_head=None):
    """A chunk of queries against a key/value cache (Self Forcing streaming).

    q: [B, Nq, heads, d] on the grid ``grid_q`` = (Fq, H, W, f0, h0, w0) (the
    chunk's first frame is f0); k, v: [B, Nkv, heads, d], Nkv / (H W) whole
    frames whose first frame is ``kv_frame0``, raw (the oracle rotates them).
    Every key j < kv_lens[b] is visible.  ``theta_per_head`` ([heads],
    optional): multi-head RoPE jitter (``theta`` is then unused).
    Returns fp64 [B, len(rows), heads, d]."""
    q, k, v = _u16(q), _u16(k), _u16(v)
    B, Nq, heads, d = q.shape
    Nkv = k.shape[1]
    assert k.shape == (B, Nkv, heads, d) and v.shape == k.shape
    Fq, H, W, f0, h0, w0 = grid_q
    if rows is None:
        rows = np.arange(Nq, dtype=np.int32)
    rows = np.ascontiguousarray(rows, dtype=np.int32)
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    kvl = None if kv_lens is None else np.ascontiguousarray(kv_lens, dtype=np.int32)
    out = np.empty((B, rows.shape[0], heads, d), dtype=np.float64)
    if theta_per_head is not None:
        th = np.ascontiguousarray(theta_per_head, dtype=np.float64)
        if th.shape != (heads,):
            raise ValueError("theta_per_head needs one value per head")
        rc = _load().orc_kv_rows_heads(q.ctypes.data, k.ctypes.data, v.ctypes.data, B, Nq, Nkv, heads, d, Fq,
                                       H, W, int(f0), int(kv_frame0), int(h0), int(w0), th.ctypes.data, scale,
                                       None if kvl is None else kvl.ctypes.data, rows.shape[0],
                                       rows.ctypes.data, out.ctypes.data, _threads(threads))
        if rc != 0:
            raise ValueError("orc_kv_rows_heads rejected its arguments")
        return out
    rc = _load().orc_kv_rows(q.ctypes.data, k.ctypes.data, v.ctypes.data, B, Nq, Nkv, heads, d, Fq, H, W,
                             int(f0), int(kv_frame0), int(h0), int(w0), theta, scale,
                             None if kvl is None else kvl.ctypes.data, rows.shape[0], rows.ctypes.data,
                             out.ctypes.data, _threads(threads))
    if rc != 0:
        raise ValueError("orc_kv_rows rejected its arguments")
    return out


def prologue_rows(x, e0, e1, wq, bq, wk, bk, wv, bv, gq, gk, rows=None, eps_ln: float = 1e-6,
                  eps_rms: float = 1e-6, threads: int | None = None):
    """Self-attention prologue of one block: norm1(x) * (1 + e1) + e0, the q, k,
    v projections, RMSNorm of q and k.  x bf16 bits [B, N, dim]; e0, e1 float32
    [B, dim]; weights bf16 bits [dim, dim]; biases and gammas bf16 bits [dim].
    Returns fp64 (q, k, v), each [B, len(rows), dim]."""
    x = _u16(x)
    B, N, dim = x.shape
    ws = [_u16(w) for w in (wq, wk, wv)]
    vs = [_u16(a) for a in (bq, bk, bv, gq, gk)]
    assert all(w.shape == (dim, dim) for w in ws) and all(a.shape == (dim,) for a in vs)
    e0 = np.ascontiguousarray(e0, dtype=np.float32).reshape(B, dim)
    e1 = np.ascontiguousarray(e1, dtype=np.float32).reshape(B, dim)
    if rows is None:
        rows = np.arange(N, dtype=np.int32)
    rows = np.ascontiguousarray(rows, dtype=np.int32)
    outs = [np.empty((B, rows.shape[0], dim), dtype=np.float64) for _ in range(3)]
    rc = _load().orc_prologue_rows(x.ctypes.data, e0.ctypes.data, e1.ctypes.data, ws[0].ctypes.data,
                                   vs[0].ctypes.data, ws[1].ctypes.data, vs[1].ctypes.data,
                                   ws[2].ctypes.data, vs[2].ctypes.data, vs[3].ctypes.data,
                                   vs[4].ctypes.data, B, N, dim, float(eps_ln), float(eps_rms),
                                   rows.shape[0], rows.ctypes.data, outs[0].ctypes.data,
                                   outs[1].ctypes.data, outs[2].ctypes.data, _threads(threads))
    if rc != 0:
        raise ValueError("orc_prologue_rows rejected its arguments")
    return tuple(outs)


def cross_rows(q, k_ctx, v_ctx, rows=None, scale: float | None = None, ctx_lens=None,
               threads: int | None = None):
    """Cross attention (no RoPE) for query ``rows``; fp64 [B, len(rows), heads, d]."""
    q, k_ctx, v_ctx = _u16(q), _u16(k_ctx), _u16(v_ctx)
    B, N, heads, d = q.shape
    M = k_ctx.shape[1]
    assert k_ctx.shape == (B, M, heads, d) and v_ctx.shape == k_ctx.shape
    if rows is None:
        rows = np.arange(N, dtype=np.int32)
    rows = np.ascontiguousarray(rows, dtype=np.int32)
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    cl = None if ctx_lens is None else np.ascontiguousarray(ctx_lens, dtype=np.int32)
    out = np.empty((B, rows.shape[0], heads, d), dtype=np.float64)
    rc = _load().orc_cross_rows(q.ctypes.data, k_ctx.ctypes.data, v_ctx.ctypes.data, B, N, M, heads,
                                d, scale, None if cl is None else cl.ctypes.data, rows.shape[0],
                                rows.ctypes.data, out.ctypes.data, _threads(threads))
    if rc != 0:
        raise ValueError("orc_cross_rows rejected its arguments")
    return out
