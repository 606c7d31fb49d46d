"""Python binding of libwanattn (ctypes).  Argument marshalling only: every
step of the computation runs in the HIP kernels behind the C ABI declared in
include/wanattn.h.  Tensors are torch bf16 tensors on the GPU, contiguous,
[B, tokens, heads, 128]; work is enqueued on torch's current stream.

There is no fallback: if the library is missing or the GPU is absent the
calls raise.
"""
from __future__ import annotations

import ctypes
import math
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libwanattn.so")

OK, E_INVALID, E_UNSUPPORTED, E_HIP = 0, 1, 2, 3
MASK_NONE, MASK_BLOCK_CAUSAL = 0, 1
HEAD_DIM = 128
MAX_POS = 1024
MAX_LEN_BATCH = 256
MAX_JITTER_HEADS = 256

EXPORTS = ("wanattn_rope3d", "wanattn_self", "wanattn_self_workspace_bytes", "wanattn_self_jitter",
           "wanattn_self_jitter_workspace_bytes", "wanattn_self_kv", "wanattn_rope_tables_bytes",
           "wanattn_rope_tables", "wanattn_rope3d_tables", "wanattn_self_kv_tables",
           "wanattn_cross", "wanattn_prologue", "wanattn_prologue_workspace_bytes", "wanattn_prepare",
           "wanattn_status_string", "wanattn_last_error", "wanattn_version", "wanattn_self_noalloc",
           "wanattn_prologue_rms", "wanattn_self_qknorm")

NOALLOC_SCRATCH_BYTES = 512 << 20


class WanattnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"wanattn status {status}: {message}")
        self.status = status


class Grid3D(ctypes.Structure):
    _fields_ = [("F", ctypes.c_int32), ("H", ctypes.c_int32), ("W", ctypes.c_int32),
                ("f0", ctypes.c_int32), ("h0", ctypes.c_int32), ("w0", ctypes.c_int32)]


_lib = None


def load_library(path: str = LIB_PATH):
    """Load libwanattn and declare its signatures (no GPU needed for this)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing; build it with "
                           "`python -m video_diffusion_transformer_wanattn_amd.build`")
    lib = ctypes.CDLL(path)
    P, i32, f64, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_double, ctypes.c_float
    G = ctypes.POINTER(Grid3D)
    lib.wanattn_rope3d.argtypes = [P, P, i32, i32, i32, i32, G, f64, P]
    lib.wanattn_rope3d.restype = ctypes.c_int
    lib.wanattn_self.argtypes = [P, P, P, P, i32, i32, i32, i32, G, f64, f32, ctypes.c_int, i32, P,
                                 P, ctypes.c_size_t, P]
    lib.wanattn_self.restype = ctypes.c_int
    lib.wanattn_self_noalloc.argtypes = [P, P, P, P, i32, i32, i32, i32, G, f64, f32, ctypes.c_int, i32, P, P]
    lib.wanattn_self_noalloc.restype = ctypes.c_int
    lib.wanattn_self_workspace_bytes.argtypes = [i32, i32, i32, i32]
    lib.wanattn_self_workspace_bytes.restype = ctypes.c_size_t
    lib.wanattn_self_jitter.argtypes = [P, P, P, P, i32, i32, i32, i32, G, P, f32, ctypes.c_int, i32, P,
                                        P, ctypes.c_size_t, P]
    lib.wanattn_self_jitter.restype = ctypes.c_int
    lib.wanattn_self_jitter_workspace_bytes.argtypes = [i32, i32, i32, i32]
    lib.wanattn_self_jitter_workspace_bytes.restype = ctypes.c_size_t
    lib.wanattn_self_kv.argtypes = [P, P, P, P, i32, i32, i32, i32, i32, G, f64, f32, P, P]
    lib.wanattn_self_kv.restype = ctypes.c_int
    lib.wanattn_rope_tables_bytes.argtypes = [i32]
    lib.wanattn_rope_tables_bytes.restype = ctypes.c_size_t
    lib.wanattn_rope_tables.argtypes = [P, i32, P, ctypes.c_size_t, P]
    lib.wanattn_rope_tables.restype = ctypes.c_int
    lib.wanattn_rope3d_tables.argtypes = [P, P, i32, i32, i32, i32, G, P, ctypes.c_size_t, P]
    lib.wanattn_rope3d_tables.restype = ctypes.c_int
    lib.wanattn_self_kv_tables.argtypes = [P, P, P, P, i32, i32, i32, i32, i32, G, P, ctypes.c_size_t, f32, P,
                                           P]
    lib.wanattn_self_kv_tables.restype = ctypes.c_int
    lib.wanattn_cross.argtypes = [P, P, P, P, i32, i32, i32, i32, i32, f32, P, P]
    lib.wanattn_cross.restype = ctypes.c_int
    lib.wanattn_prologue.argtypes = [P] * 14 + [i32, i32, i32, f32, f32, P, ctypes.c_size_t, P]
    lib.wanattn_prologue.restype = ctypes.c_int
    lib.wanattn_prologue_rms.argtypes = [P] * 13 + [i32, i32, i32, f32, f32, P, ctypes.c_size_t, P]
    lib.wanattn_prologue_rms.restype = ctypes.c_int
    lib.wanattn_self_qknorm.argtypes = [P, P, P, P, i32, i32, i32, i32, G, f64, f32, ctypes.c_int, i32, P,
                                        P, P, P, P, ctypes.c_size_t, P]
    lib.wanattn_self_qknorm.restype = ctypes.c_int
    lib.wanattn_prologue_workspace_bytes.argtypes = [i32, i32, i32]
    lib.wanattn_prologue_workspace_bytes.restype = ctypes.c_size_t
    lib.wanattn_prepare.argtypes = [f64]
    lib.wanattn_prepare.restype = ctypes.c_int
    lib.wanattn_status_string.argtypes = [ctypes.c_int]
    lib.wanattn_status_string.restype = ctypes.c_char_p
    lib.wanattn_last_error.argtypes = []
    lib.wanattn_last_error.restype = ctypes.c_char_p
    lib.wanattn_version.argtypes = []
    lib.wanattn_version.restype = i32
    _lib = lib
    return lib


def _raise_on(status: int):
    if status != OK:
        lib = load_library()
        raise WanattnError(status, lib.wanattn_last_error().decode(errors="replace"))


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _on(stream):
    """Context in which torch allocates the tensors a call on ``stream`` uses
    (outputs, workspaces): their memory then belongs to that stream's pool and
    is only handed out again after the work enqueued there."""
    import contextlib
    import torch
    return torch.cuda.stream(stream) if stream is not None else contextlib.nullcontext()


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _lens(lens, B):
    if lens is None:
        return None
    arr = (ctypes.c_int32 * B)(*[int(x) for x in lens])
    return arr


def _grid(grid, offsets):
    F, H, W = (int(x) for x in grid)
    f0, h0, w0 = (int(x) for x in offsets)
    return Grid3D(F, H, W, f0, h0, w0)


def _dims(t, *others):
    import torch
    for x in (t, *others):
        if x is None:
            continue
        if not x.is_cuda:
            raise ValueError("tensors must live on the GPU")
        if x.dtype != torch.bfloat16:
            raise ValueError("tensors must be bfloat16")
        if not x.is_contiguous():
            raise ValueError("tensors must be contiguous")
        if x.dim() != 4:
            raise ValueError("expected [B, tokens, heads, head_dim] tensors")
    return tuple(int(x) for x in t.shape)


def _tables(tables):
    if not tables.is_cuda or not tables.is_contiguous():
        raise ValueError("tables must be a contiguous GPU tensor (see rope_tables)")
    return _ptr(tables), tables.numel() * tables.element_size()


def rope_tables(theta_per_head, out=None, stream=None):
    """Per-head rotary tables (head h with RoPE base theta_per_head[h]) for
    the streamed jitter calls; a uint8 GPU tensor unless ``out`` is given."""
    import torch
    lib = load_library()
    th = [float(x) for x in theta_per_head]
    heads = len(th)
    need = int(lib.wanattn_rope_tables_bytes(heads))
    if out is None:
        with _on(stream):
            out = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")
    ptr, nbytes = _tables(out)
    _raise_on(lib.wanattn_rope_tables((ctypes.c_double * max(heads, 1))(*th), heads, ptr, nbytes,
                                      _stream(stream)))
    return out


def rope3d(x, grid, theta: float = 10000.0, offsets=(0, 0, 0), out=None, stream=None, tables=None):
    """3D RoPE of x ([B, N, heads, 128] bf16); out may be x (in place).
    ``tables`` (from rope_tables): rotate head h with its own table instead."""
    import torch
    lib = load_library()
    if out is None:
        with _on(stream):
            out = torch.empty_like(x)
    B, N, heads, d = _dims(x, out)
    if tuple(out.shape) != tuple(x.shape):
        raise ValueError("out must have the shape of x")
    g = _grid(grid, offsets)
    if tables is not None:
        tp, tb = _tables(tables)
        _raise_on(lib.wanattn_rope3d_tables(_ptr(x), _ptr(out), B, N, heads, d, ctypes.byref(g), tp, tb,
                                            _stream(stream)))
        return out
    _raise_on(lib.wanattn_rope3d(_ptr(x), _ptr(out), B, N, heads, d, ctypes.byref(g), float(theta),
                                 _stream(stream)))
    return out


def self_workspace_bytes(B: int, N: int, heads: int, head_dim: int = HEAD_DIM) -> int:
    return int(load_library().wanattn_self_workspace_bytes(B, N, heads, head_dim))


def self_jitter_workspace_bytes(B: int, N: int, heads: int, head_dim: int = HEAD_DIM) -> int:
    return int(load_library().wanattn_self_jitter_workspace_bytes(B, N, heads, head_dim))


def self_attention(q, k, v, grid, theta: float = 10000.0, scale: float | None = None,
                   block_causal: bool = False, chunk_frames: int = 3, kv_lens=None,
                   offsets=(0, 0, 0), out=None, workspace=None, stream=None, theta_per_head=None):
    """softmax(RoPE(q) RoPE(k)^T * scale) v, bidirectional or latent-frame block-causal.

    theta_per_head: optional [heads] RoPE bases (multi-head RoPE jitter; theta
    is then unused).  workspace: optional GPU tensor of at least
    self_workspace_bytes(...) bytes (self_jitter_workspace_bytes(...) with
    theta_per_head); the rotated keys (and per-head tables) go there, and the
    partial results of the key-split tail where it has room for them (a
    workspace of just the rotated keys' size runs without that split);
    allocated per call when not given."""
    import torch
    lib = load_library()
    if out is None:
        with _on(stream):
            out = torch.empty_like(q)
    B, N, heads, d = _dims(q, k, v, out)
    if not (tuple(k.shape) == tuple(v.shape) == tuple(out.shape) == tuple(q.shape)):
        raise ValueError("q, k, v and out must have the same shape")
    if kv_lens is not None and len(kv_lens) != B:
        raise ValueError("kv_lens needs one entry per batch")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    g = _grid(grid, offsets)
    mask = MASK_BLOCK_CAUSAL if block_causal else MASK_NONE
    lens = _lens(kv_lens, B)
    jitter = theta_per_head is not None
    if jitter:
        th = [float(x) for x in theta_per_head]
        if len(th) != heads:
            raise ValueError("theta_per_head needs one value per head")
        th_arr = (ctypes.c_double * heads)(*th)
        need = int(lib.wanattn_self_jitter_workspace_bytes(B, N, heads, d))
    else:
        need = int(lib.wanattn_self_workspace_bytes(B, N, heads, d))
    if workspace is None:
        # on the launch stream's pool: the kernels still read it after this returns
        with _on(stream):
            workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    if not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous GPU tensor")
    ws_bytes = workspace.numel() * workspace.element_size()
    if jitter:
        _raise_on(lib.wanattn_self_jitter(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, N, heads, d,
                                          ctypes.byref(g), th_arr, float(scale), mask, int(chunk_frames),
                                          lens, _ptr(workspace), ws_bytes, _stream(stream)))
        return out
    _raise_on(lib.wanattn_self(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, N, heads, d, ctypes.byref(g),
                               float(theta), float(scale), mask, int(chunk_frames), lens,
                               _ptr(workspace), ws_bytes, _stream(stream)))
    return out


def self_attention_noalloc(q, k, v, grid, theta: float = 10000.0, scale: float | None = None,
                           block_causal: bool = False, chunk_frames: int = 3, kv_lens=None,
                           offsets=(0, 0, 0), out=None, stream=None):
    """self_attention through wanattn_self_noalloc: no workspace, the library's
    static per-device scratch instead (B * N * heads * 256 + 256 bytes must fit
    NOALLOC_SCRATCH_BYTES).  Calls that overlap on one device race.  With
    ``out`` given, nothing is allocated."""
    import torch
    lib = load_library()
    if out is None:
        with _on(stream):
            out = torch.empty_like(q)
    B, N, heads, d = _dims(q, k, v, out)
    if not (tuple(k.shape) == tuple(v.shape) == tuple(out.shape) == tuple(q.shape)):
        raise ValueError("q, k, v and out must have the same shape")
    if kv_lens is not None and len(kv_lens) != B:
        raise ValueError("kv_lens needs one entry per batch")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    g = _grid(grid, offsets)
    mask = MASK_BLOCK_CAUSAL if block_causal else MASK_NONE
    _raise_on(lib.wanattn_self_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, N, heads, d, ctypes.byref(g),
                                       float(theta), float(scale), mask, int(chunk_frames), _lens(kv_lens, B),
                                       _stream(stream)))
    return out


def self_attention_kv(q, k_cache, v_cache, grid_q, theta: float = 10000.0, scale: float | None = None,
                      kv_lens=None, offsets=(0, 0, 0), out=None, stream=None, tables=None):
    """One chunk of queries (grid_q frames at RoPE offsets ``offsets``) against a
    key/value cache of whole frames; k_cache holds keys already rotated by
    their own positions (see rope3d).  Every key j < kv_lens[b] is visible.
    ``tables`` (from rope_tables): per-head RoPE tables (multi-head jitter;
    the cache must have been rotated with the same tables)."""
    import torch
    lib = load_library()
    if out is None:
        with _on(stream):
            out = torch.empty_like(q)
    B, Nq, heads, d = _dims(q, k_cache, v_cache, out)
    Nkv = int(k_cache.shape[1])
    if tuple(k_cache.shape) != (B, Nkv, heads, d) or tuple(v_cache.shape) != (B, Nkv, heads, d):
        raise ValueError("k_cache and v_cache must be [B, Nkv, heads, head_dim] like q")
    if tuple(out.shape) != tuple(q.shape):
        raise ValueError("out must have the shape of q")
    if kv_lens is not None and len(kv_lens) != B:
        raise ValueError("kv_lens needs one entry per batch")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    g = _grid(grid_q, offsets)
    if tables is not None:
        tp, tb = _tables(tables)
        _raise_on(lib.wanattn_self_kv_tables(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(out), B, Nq, Nkv, heads,
                                             d, ctypes.byref(g), tp, tb, float(scale), _lens(kv_lens, B),
                                             _stream(stream)))
        return out
    _raise_on(lib.wanattn_self_kv(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(out), B, Nq, Nkv, heads, d,
                                  ctypes.byref(g), float(theta), float(scale), _lens(kv_lens, B),
                                  _stream(stream)))
    return out


def cross_attention(q, k_ctx, v_ctx, scale: float | None = None, ctx_lens=None, out=None,
                    stream=None):
    """softmax(q k_ctx^T * scale) v_ctx over M text tokens, no RoPE."""
    import torch
    lib = load_library()
    if out is None:
        with _on(stream):
            out = torch.empty_like(q)
    B, N, heads, d = _dims(q, k_ctx, v_ctx, out)
    M = int(k_ctx.shape[1])
    if tuple(k_ctx.shape) != (B, M, heads, d) or tuple(v_ctx.shape) != (B, M, heads, d):
        raise ValueError("k_ctx and v_ctx must be [B, M, heads, head_dim] like q")
    if tuple(out.shape) != tuple(q.shape):
        raise ValueError("out must have the shape of q")
    if ctx_lens is not None and len(ctx_lens) != B:
        raise ValueError("ctx_lens needs one entry per batch")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    lens = _lens(ctx_lens, B)
    _raise_on(lib.wanattn_cross(_ptr(q), _ptr(k_ctx), _ptr(v_ctx), _ptr(out), B, N, M, heads, d,
                                float(scale), lens, _stream(stream)))
    return out


def prologue_workspace_bytes(B: int, N: int, dim: int) -> int:
    return int(load_library().wanattn_prologue_workspace_bytes(B, N, dim))


def prologue(x, e0, e1, wq, bq, wk, bk, wv, bv, gq, gk, eps_ln: float = 1e-6, eps_rms: float = 1e-6,
             out=None, workspace=None, stream=None):
    """The block's self-attention inputs from its hidden state: LayerNorm(x)
    modulated by (e0, e1), the q/k/v projections, RMSNorm of q and k.

    x: [B, N, dim] bf16; e0, e1: [B, dim] float32; weights [dim, dim] bf16
    (nn.Linear layout); biases and gammas [dim] bf16.  Returns (q, k, v), each
    [B, N, dim] bf16 (view them as [B, N, dim // 128, 128] for the attention
    calls).  out: optional (q, k, v) tensors; workspace: optional GPU tensor of
    at least prologue_workspace_bytes(B, N, dim) bytes, 256-byte aligned."""
    import torch
    lib = load_library()
    if x.dim() != 3:
        raise ValueError("x must be [B, N, dim]")
    B, N, dim = (int(a) for a in x.shape)
    if out is None:
        with _on(stream):
            out = tuple(torch.empty_like(x) for _ in range(3))
    mats, vecs = (wq, wk, wv), (bq, bk, bv, gq, gk)
    for t in (x, *out, *mats, *vecs):
        if not t.is_cuda or t.dtype != torch.bfloat16 or not t.is_contiguous():
            raise ValueError("x, weights, biases, gammas and outputs must be contiguous bf16 GPU tensors")
    for t in (e0, e1):
        if not t.is_cuda or t.dtype != torch.float32 or not t.is_contiguous():
            raise ValueError("e0 and e1 must be contiguous float32 GPU tensors")
        if tuple(t.shape) != (B, dim):
            raise ValueError("e0 and e1 must be [B, dim]")
    if any(tuple(t.shape) != (B, N, dim) for t in out):
        raise ValueError("outputs must be [B, N, dim]")
    if any(tuple(t.shape) != (dim, dim) for t in mats) or any(tuple(t.shape) != (dim,) for t in vecs):
        raise ValueError("weights must be [dim, dim] and biases/gammas [dim]")
    need = int(lib.wanattn_prologue_workspace_bytes(B, N, dim))
    if workspace is None:
        with _on(stream):
            workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=x.device)
    if not workspace.is_cuda or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous GPU tensor")
    ws_bytes = workspace.numel() * workspace.element_size()
    _raise_on(lib.wanattn_prologue(_ptr(x), _ptr(e0), _ptr(e1), _ptr(wq), _ptr(bq), _ptr(wk), _ptr(bk),
                                   _ptr(wv), _ptr(bv), _ptr(gq), _ptr(gk), _ptr(out[0]), _ptr(out[1]),
                                   _ptr(out[2]), B, N, dim, float(eps_ln), float(eps_rms),
                                   _ptr(workspace), ws_bytes, _stream(stream)))
    return tuple(out)


def prologue_rms(x, e0, e1, wq, bq, wk, bk, wv, bv, eps_ln: float = 1e-6, eps_rms: float = 1e-6,
                 out=None, rms=None, workspace=None, stream=None):
    """prologue() with the QK-Norm left to self_attention_qknorm: returns (q, k,
    v, rms) with q and k before the RMSNorm and rms a float32 [2, B * N] tensor
    of the RMSNorm factors (q's row, then k's)."""
    import torch
    lib = load_library()
    if x.dim() != 3:
        raise ValueError("x must be [B, N, dim]")
    B, N, dim = (int(a) for a in x.shape)
    with _on(stream):
        if out is None:
            out = tuple(torch.empty_like(x) for _ in range(3))
        if rms is None:
            rms = torch.empty(2, B * N, dtype=torch.float32, device=x.device)
    for t in (x, *out, wq, wk, wv, bq, bk, bv):
        if not t.is_cuda or t.dtype != torch.bfloat16 or not t.is_contiguous():
            raise ValueError("x, weights, biases and outputs must be contiguous bf16 GPU tensors")
    for t in (e0, e1):
        if not t.is_cuda or t.dtype != torch.float32 or not t.is_contiguous() or tuple(t.shape) != (B, dim):
            raise ValueError("e0 and e1 must be contiguous float32 GPU tensors [B, dim]")
    if not rms.is_cuda or rms.dtype != torch.float32 or not rms.is_contiguous() or rms.numel() != 2 * B * N:
        raise ValueError("rms must be a contiguous float32 GPU tensor of 2 * B * N values")
    if any(tuple(t.shape) != (B, N, dim) for t in out):
        raise ValueError("outputs must be [B, N, dim]")
    if any(tuple(t.shape) != (dim, dim) for t in (wq, wk, wv)) or any(tuple(t.shape) != (dim,) for t in (bq, bk, bv)):
        raise ValueError("weights must be [dim, dim] and biases [dim]")
    need = int(lib.wanattn_prologue_workspace_bytes(B, N, dim))
    if workspace is None:
        with _on(stream):
            workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=x.device)
    ws_bytes = workspace.numel() * workspace.element_size()
    _raise_on(lib.wanattn_prologue_rms(_ptr(x), _ptr(e0), _ptr(e1), _ptr(wq), _ptr(bq), _ptr(wk), _ptr(bk),
                                       _ptr(wv), _ptr(bv), _ptr(out[0]), _ptr(out[1]), _ptr(out[2]), _ptr(rms),
                                       B, N, dim, float(eps_ln), float(eps_rms), _ptr(workspace), ws_bytes,
                                       _stream(stream)))
    return (*out, rms)


def self_attention_qknorm(q, k, v, rms, gq, gk, grid, theta: float = 10000.0, scale: float | None = None,
                          block_causal: bool = False, chunk_frames: int = 3, kv_lens=None, offsets=(0, 0, 0),
                          out=None, workspace=None, stream=None):
    """self_attention on prologue_rms's outputs: q and k before the QK-Norm
    ([B, N, heads, 128] bf16), rms its factors, gq and gk its weights
    ([heads * 128] bf16); the norm is applied as q is loaded and k rotated."""
    import torch
    lib = load_library()
    if out is None:
        with _on(stream):
            out = torch.empty_like(q)
    B, N, heads, d = _dims(q, k, v, out)
    if not (tuple(k.shape) == tuple(v.shape) == tuple(out.shape) == tuple(q.shape)):
        raise ValueError("q, k, v and out must have the same shape")
    if not rms.is_cuda or rms.dtype != torch.float32 or not rms.is_contiguous() or rms.numel() != 2 * B * N:
        raise ValueError("rms must be a contiguous float32 GPU tensor of 2 * B * N values")
    for g in (gq, gk):
        if not g.is_cuda or g.dtype != torch.bfloat16 or not g.is_contiguous() or g.numel() != heads * d:
            raise ValueError("gq and gk must be contiguous bf16 GPU tensors of heads * head_dim values")
    if kv_lens is not None and len(kv_lens) != B:
        raise ValueError("kv_lens needs one entry per batch")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    need = int(lib.wanattn_self_workspace_bytes(B, N, heads, d))
    if workspace is None:
        with _on(stream):
            workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    ws_bytes = workspace.numel() * workspace.element_size()
    mask = MASK_BLOCK_CAUSAL if block_causal else MASK_NONE
    _raise_on(lib.wanattn_self_qknorm(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, N, heads, d,
                                      ctypes.byref(_grid(grid, offsets)), float(theta), float(scale), mask,
                                      int(chunk_frames), _lens(kv_lens, B), _ptr(rms), _ptr(gq), _ptr(gk),
                                      _ptr(workspace), ws_bytes, _stream(stream)))
    return out


def prepare(theta: float = 10000.0):
    _raise_on(load_library().wanattn_prepare(float(theta)))
