"""The C-ABI library loads without a GPU, exports every symbol that
include/wanattn.h declares, and rejects bad arguments before it launches
anything (no compute is called here)."""
import ctypes
import os
import re

import pytest

from video_diffusion_transformer_wanattn_amd import wanattn as wa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "wanattn.h")

A = ctypes.c_void_p(1 << 20)      # 16-byte aligned dummy addresses, never dereferenced
B_ = ctypes.c_void_p(2 << 30)
C = ctypes.c_void_p(3 << 30)
O = ctypes.c_void_p(4 << 30)
WS = ctypes.c_void_p(5 << 30)


@pytest.fixture(scope="module")
def lib():
    return wa.load_library()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(wanattn_\w+)\s*\(", text, re.M)))


def test_header_declarations_are_exported(lib):
    names = declared_functions()
    assert set(names) == set(wa.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_status_strings(lib):
    assert lib.wanattn_version() == 1
    assert lib.wanattn_status_string(0) == b"ok"
    assert lib.wanattn_status_string(1) == b"invalid argument"
    assert lib.wanattn_status_string(2) == b"unsupported"
    assert lib.wanattn_status_string(3) == b"HIP error"


def g(F, H, W, f0=0, h0=0, w0=0):
    return ctypes.byref(wa.Grid3D(F, H, W, f0, h0, w0))


def call_self(lib, q=A, k=B_, v=C, o=O, B=1, N=24, heads=2, d=128, grid=None, theta=1e4, scale=0.088,
              mask=0, chunk=3, lens=None, ws=WS, ws_bytes=1 << 20):
    grid = grid if grid is not None else g(2, 3, 4)
    return lib.wanattn_self(q, k, v, o, B, N, heads, d, grid, theta, scale, mask, chunk, lens, ws,
                            ws_bytes, None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), wa.E_INVALID),
    (dict(o=ctypes.c_void_p((4 << 30) + 8)), wa.E_INVALID),        # misaligned
    (dict(B=0), wa.E_INVALID),
    (dict(N=0), wa.E_INVALID),
    (dict(heads=0), wa.E_INVALID),
    (dict(d=64), wa.E_UNSUPPORTED),
    (dict(heads=65537, N=24), wa.E_UNSUPPORTED),                  # above WANATTN_MAX_HEADS
    (dict(N=25), wa.E_INVALID),                                   # N != F*H*W
    (dict(grid=None, N=24), wa.E_INVALID),
    (dict(theta=0.0), wa.E_INVALID),
    (dict(theta=float("nan")), wa.E_INVALID),
    (dict(scale=0.0), wa.E_INVALID),
    (dict(mask=7), wa.E_INVALID),
    (dict(mask=1, chunk=0), wa.E_INVALID),
    (dict(o=A), wa.E_INVALID),                                    # o aliases q
    (dict(o=ctypes.c_void_p((1 << 20) + 4096)), wa.E_INVALID),     # o overlaps q
    (dict(ws=None), wa.E_INVALID),
    (dict(ws=ctypes.c_void_p((5 << 30) + 4)), wa.E_INVALID),      # misaligned workspace
    (dict(ws_bytes=24 * 2 * 128 * 2 - 16), wa.E_INVALID),          # workspace too small
    (dict(ws=ctypes.c_void_p((2 << 30) + 256)), wa.E_INVALID),     # workspace overlaps k
])
def test_self_rejects(lib, kw, status):
    if "grid" in kw and kw["grid"] is None:
        kw = dict(kw)
        kw["grid"] = ctypes.cast(None, ctypes.POINTER(wa.Grid3D))
    assert call_self(lib, **kw) == status
    assert lib.wanattn_last_error()


# room for the fp32 partials of one key-split workgroup: 256 rows x 128 O
# values and (l, bias) per row; then 256 bytes of work-queue counters
SPLIT_ITEM = 256 * 128 * 4 + 256 * 8
QUEUE = 256


def test_workspace_size(lib):
    # rotated keys, plus partials for as many split workgroups as the launch
    # has workgroups (at most 512), plus the queue counters
    assert lib.wanattn_self_workspace_bytes(2, 24, 3, 128) == 2 * 24 * 3 * 128 * 2 + 6 * SPLIT_ITEM + QUEUE
    assert lib.wanattn_self_workspace_bytes(1, 75600, 40, 128) == 75600 * 40 * 128 * 2 + 512 * SPLIT_ITEM + QUEUE
    assert lib.wanattn_self_workspace_bytes(2, 24, 3, 64) == 0
    assert lib.wanattn_self_workspace_bytes(0, 24, 3, 128) == 0


def test_workspace_room_for_partials_is_checked_for_overlap(lib):
    # the rotated keys' part of the workspace ends before k, the partials'
    # room does not: rejected when the caller offers that room
    kbytes = 24 * 2 * 128 * 2
    full = lib.wanattn_self_workspace_bytes(1, 24, 2, 128)
    ws = ctypes.c_void_p((2 << 30) - kbytes - 256)
    assert call_self(lib, ws=ws, ws_bytes=full) == wa.E_INVALID
    assert "overlaps" in lib.wanattn_last_error().decode()


def test_launch_size_limit(lib):
    # 256 batches x 65536 heads x 1 query tile = 2^24 workgroups of 256 threads:
    # one more thread than a launch takes; rejected before anything is launched
    g16 = g(1, 16, 16)
    big = 1 << 44
    assert lib.wanattn_self(A, B_, C, O, 256, 256, 65536, 128, g16, 1e4, 0.088, 0, 1, None, ctypes.c_void_p(big),
                            big, None) == wa.E_UNSUPPORTED
    assert "exceed one launch" in lib.wanattn_last_error().decode()
    assert lib.wanattn_cross(A, B_, C, O, 256, 256, 8, 65536, 128, 0.088, None, None) == wa.E_UNSUPPORTED
    assert lib.wanattn_self_kv(A, B_, C, O, 256, 256, 256, 65536, 128, g16, 1e4, 0.088, None, None) == wa.E_UNSUPPORTED


def test_self_rejects_positions_beyond_table(lib):
    assert call_self(lib, N=24, grid=g(2, 3, 4, 1023, 0, 0)) == wa.E_INVALID
    assert call_self(lib, N=24, grid=g(2, 3, 4, 0, 1022, 0)) == wa.E_INVALID
    assert call_self(lib, N=24, grid=g(2, 3, 4, 0, 0, -1)) == wa.E_INVALID


def test_self_rejects_bad_lengths(lib):
    lens = (ctypes.c_int32 * 2)(24, 25)
    assert call_self(lib, B=2, lens=lens) == wa.E_INVALID
    lens = (ctypes.c_int32 * 2)(0, 5)
    assert call_self(lib, B=2, lens=lens) == wa.E_INVALID
    # more batches than one launch takes: every entry is still checked (one
    # bad length past the first launch's 256 is rejected before any launch)
    big = (ctypes.c_int32 * 300)(*([24] * 299 + [25]))
    assert call_self(lib, B=300, lens=big, ws_bytes=1 << 28) == wa.E_INVALID


def test_self_kv_rejects(lib):
    # queries: 2 frames of 3x4 = 24 tokens; cache: 5 frames = 60 tokens
    def call(q=A, k=B_, v=C, o=O, B=1, Nq=24, Nkv=60, heads=2, d=128, grid=None, theta=1e4,
             scale=0.088, lens=None):
        grid = grid if grid is not None else g(2, 3, 4, 3, 0, 0)
        return lib.wanattn_self_kv(q, k, v, o, B, Nq, Nkv, heads, d, grid, theta, scale, lens, None)
    assert call(k=None) == wa.E_INVALID
    assert call(o=ctypes.c_void_p((4 << 30) + 8)) == wa.E_INVALID          # misaligned
    assert call(Nq=25) == wa.E_INVALID                                      # Nq != F*H*W
    assert call(Nkv=58) == wa.E_INVALID                                     # not whole frames
    assert call(Nkv=0) == wa.E_INVALID
    assert call(d=64) == wa.E_UNSUPPORTED
    assert call(heads=65537) == wa.E_UNSUPPORTED
    assert call(grid=g(2, 3, 4, 1023, 0, 0)) == wa.E_INVALID               # chunk positions past the table
    assert call(theta=0.0) == wa.E_INVALID
    assert call(scale=-1.0) == wa.E_INVALID
    assert call(o=B_) == wa.E_INVALID                                       # o aliases the cache
    assert call(lens=(ctypes.c_int32 * 1)(61)) == wa.E_INVALID
    assert call(lens=(ctypes.c_int32 * 1)(0)) == wa.E_INVALID
    assert lib.wanattn_last_error()


def test_cross_rejects(lib):
    def call(q=A, k=B_, v=C, o=O, B=1, N=24, M=8, heads=2, d=128, scale=0.088, lens=None):
        return lib.wanattn_cross(q, k, v, o, B, N, M, heads, d, scale, lens, None)
    assert call(v=None) == wa.E_INVALID
    assert call(M=0) == wa.E_INVALID
    assert call(d=96) == wa.E_UNSUPPORTED
    assert call(heads=65537) == wa.E_UNSUPPORTED
    assert call(o=B_) == wa.E_INVALID
    assert call(lens=(ctypes.c_int32 * 1)(9)) == wa.E_INVALID
    assert call(lens=(ctypes.c_int32 * 1)(0)) == wa.E_INVALID
    assert call(scale=float("inf")) == wa.E_INVALID


def test_rope3d_rejects(lib):
    def call(x=A, y=O, B=1, N=24, heads=2, d=128, grid=None, theta=1e4):
        return lib.wanattn_rope3d(x, y, B, N, heads, d, grid if grid is not None else g(2, 3, 4), theta, None)
    assert call(x=None) == wa.E_INVALID
    assert call(y=ctypes.c_void_p((1 << 20) + 16)) == wa.E_INVALID   # partial overlap
    assert call(N=23) == wa.E_INVALID
    assert call(d=256) == wa.E_UNSUPPORTED
    assert call(theta=-1.0) == wa.E_INVALID
    assert call(grid=g(2, 3, 4, 0, 0, 1021)) == wa.E_INVALID


def test_self_jitter_workspace_and_rejects(lib):
    tab = 3 * 1024 * 32 * 8                       # one head's rotary table
    assert lib.wanattn_self_jitter_workspace_bytes(2, 24, 3, 128) == (3 * tab + 2 * 24 * 3 * 128 * 2 + 6 * SPLIT_ITEM
                                                                      + QUEUE)
    assert lib.wanattn_self_jitter_workspace_bytes(1, 24, 257, 128) == 0
    assert lib.wanattn_self_jitter_workspace_bytes(1, 24, 3, 64) == 0
    th3 = (ctypes.c_double * 3)(1e4, 5e2, 2e5)
    need = 3 * tab + 24 * 3 * 128 * 2

    def call(q=A, k=B_, v=C, o=O, B=1, N=24, heads=3, d=128, grid=None, th=th3, scale=0.088, mask=0,
             chunk=1, lens=None, ws=WS, ws_bytes=need):
        return lib.wanattn_self_jitter(q, k, v, o, B, N, heads, d, grid if grid is not None else g(2, 3, 4),
                                       th, scale, mask, chunk, lens, ws, ws_bytes, None)
    assert call(th=None) == wa.E_INVALID
    assert call(th=(ctypes.c_double * 3)(1e4, 0.0, 1e4)) == wa.E_INVALID
    assert call(th=(ctypes.c_double * 3)(1e4, float("nan"), 1e4)) == wa.E_INVALID
    assert call(th=(ctypes.c_double * 3)(1e4, 1e4, -1.0)) == wa.E_INVALID
    assert call(heads=257, th=(ctypes.c_double * 257)(*([1e4] * 257))) == wa.E_UNSUPPORTED
    assert call(d=64) == wa.E_UNSUPPORTED
    assert call(N=23) == wa.E_INVALID
    assert call(ws_bytes=need - 1) == wa.E_INVALID          # the tables count too
    assert call(ws=None) == wa.E_INVALID
    assert call(ws=ctypes.c_void_p((4 << 30) - 16)) == wa.E_INVALID  # workspace runs into o
    assert call(o=B_) == wa.E_INVALID
    assert call(mask=1, chunk=0) == wa.E_INVALID
    assert call(scale=0.0) == wa.E_INVALID
    assert call(lens=(ctypes.c_int32 * 1)(25)) == wa.E_INVALID
    assert lib.wanattn_last_error()


def test_rope_tables_calls_reject():
    tab = 3 * 1024 * 32 * 8
    assert lib_bytes(3) == 3 * tab and lib_bytes(0) == 0 and lib_bytes(257) == 0
    lib = wa.load_library()
    th = (ctypes.c_double * 3)(1e4, 5e2, 2e5)
    T = ctypes.c_void_p(6 << 30)
    # building
    assert lib.wanattn_rope_tables(None, 3, T, 3 * tab, None) == wa.E_INVALID
    assert lib.wanattn_rope_tables((ctypes.c_double * 3)(1e4, -1.0, 1e4), 3, T, 3 * tab, None) == wa.E_INVALID
    assert lib.wanattn_rope_tables((ctypes.c_double * 257)(*([1e4] * 257)), 257, T, 257 * tab, None) == wa.E_UNSUPPORTED
    assert lib.wanattn_rope_tables(th, 0, T, 3 * tab, None) == wa.E_INVALID
    assert lib.wanattn_rope_tables(th, 3, None, 3 * tab, None) == wa.E_INVALID
    assert lib.wanattn_rope_tables(th, 3, ctypes.c_void_p((6 << 30) + 8), 3 * tab, None) == wa.E_INVALID
    assert lib.wanattn_rope_tables(th, 3, T, 3 * tab - 1, None) == wa.E_INVALID

    # rotating with them
    def rope(x=A, y=O, B=1, N=24, heads=3, d=128, grid=None, t=T, tb=3 * tab):
        return lib.wanattn_rope3d_tables(x, y, B, N, heads, d, grid if grid is not None else g(2, 3, 4), t, tb, None)
    assert rope(x=None) == wa.E_INVALID
    assert rope(t=None) == wa.E_INVALID
    assert rope(tb=2 * tab) == wa.E_INVALID                     # tables for fewer heads
    assert rope(y=ctypes.c_void_p((6 << 30) + 4096)) == wa.E_INVALID  # y inside the tables
    assert rope(N=23) == wa.E_INVALID
    assert rope(d=64) == wa.E_UNSUPPORTED
    assert rope(heads=300, tb=300 * tab) == wa.E_UNSUPPORTED

    # attending with them
    def kv(q=A, k=B_, v=C, o=O, B=1, Nq=24, Nkv=60, heads=3, d=128, grid=None, t=T, tb=3 * tab, scale=0.088,
           lens=None):
        return lib.wanattn_self_kv_tables(q, k, v, o, B, Nq, Nkv, heads, d,
                                          grid if grid is not None else g(2, 3, 4, 3, 0, 0), t, tb, scale, lens,
                                          None)
    assert kv(t=None) == wa.E_INVALID
    assert kv(tb=tab) == wa.E_INVALID
    assert kv(o=ctypes.c_void_p(6 << 30)) == wa.E_INVALID       # o on the tables
    assert kv(Nkv=58) == wa.E_INVALID
    assert kv(q=None) == wa.E_INVALID
    assert kv(lens=(ctypes.c_int32 * 1)(61)) == wa.E_INVALID
    assert kv(heads=300, tb=300 * tab) == wa.E_UNSUPPORTED
    assert lib.wanattn_last_error()


def lib_bytes(heads):
    return wa.load_library().wanattn_rope_tables_bytes(heads)


GEMM_WS = 128 << 20  # hipBLASLt's share of the prologue workspace


def test_prologue_workspace_size(lib):
    assert lib.wanattn_prologue_workspace_bytes(1, 24, 256) == 24 * 256 * 2 + GEMM_WS
    assert lib.wanattn_prologue_workspace_bytes(2, 5, 8) == 256 + GEMM_WS      # y rounded up to 256 bytes
    assert lib.wanattn_prologue_workspace_bytes(1, 24, 12) == 0
    assert lib.wanattn_prologue_workspace_bytes(1, 24, 8200) == 0
    assert lib.wanattn_prologue_workspace_bytes(0, 24, 256) == 0
    assert lib.wanattn_prologue_workspace_bytes(1 << 12, 1 << 13, 128) == 0   # more than 2^24 tokens


def test_prologue_rejects(lib):
    # 14 tensors at distinct, far-apart, 256-byte aligned dummy addresses
    base = [ctypes.c_void_p((i + 1) << 32) for i in range(14)]
    ws = ctypes.c_void_p(15 << 32)

    def call(ptrs=None, B=1, N=24, dim=256, eps_ln=1e-6, eps_rms=1e-6, ws=ws, ws_bytes=None):
        ptrs = list(base) if ptrs is None else ptrs
        if ws_bytes is None:
            ws_bytes = 24 * 256 * 2 + GEMM_WS
        return lib.wanattn_prologue(*ptrs, B, N, dim, eps_ln, eps_rms, ws, ws_bytes, None)

    for i in range(14):                          # every pointer checked for NULL and alignment
        ptrs = list(base)
        ptrs[i] = None
        assert call(ptrs) == wa.E_INVALID, i
        ptrs[i] = ctypes.c_void_p(((i + 1) << 32) + 8)
        assert call(ptrs) == wa.E_INVALID, i
    assert call(B=0) == wa.E_INVALID
    assert call(N=0) == wa.E_INVALID
    assert call(dim=12) == wa.E_INVALID
    assert call(dim=0) == wa.E_INVALID
    assert call(dim=8200) == wa.E_UNSUPPORTED
    assert call(B=1 << 12, N=1 << 13, dim=128, ws_bytes=1 << 40) == wa.E_UNSUPPORTED
    assert call(eps_ln=-1e-6) == wa.E_INVALID
    assert call(eps_rms=float("nan")) == wa.E_INVALID
    assert call(eps_ln=float("inf")) == wa.E_INVALID
    ptrs = list(base)
    ptrs[11] = base[0]                           # q aliases x
    assert call(ptrs) == wa.E_INVALID
    ptrs = list(base)
    ptrs[13] = ctypes.c_void_p((12 << 32) + 4096)  # v overlaps k
    assert call(ptrs) == wa.E_INVALID
    ptrs = list(base)
    ptrs[12] = ctypes.c_void_p((4 << 32) + 16)   # k inside the bytes of wq (256 x 256 bf16)
    assert call(ptrs) == wa.E_INVALID
    assert call(ws=None) == wa.E_INVALID
    assert call(ws=ctypes.c_void_p((15 << 32) + 16)) == wa.E_INVALID        # workspace not 256-aligned
    assert call(ws_bytes=24 * 256 * 2 + GEMM_WS - 1) == wa.E_INVALID
    assert call(ws=ctypes.c_void_p((14 << 32) - (1 << 20))) == wa.E_INVALID  # workspace runs into v
    assert lib.wanattn_last_error()


def test_prologue_rms_rejects(lib):
    # the prologue that leaves the QK-Norm to the attention call: 13 tensors
    # (no gammas) and the factors' buffer, checked like the prologue's
    base = [ctypes.c_void_p((i + 1) << 32) for i in range(12)]
    rms = ctypes.c_void_p(13 << 32)
    ws = ctypes.c_void_p(15 << 32)

    def call(ptrs=None, rms=rms, B=1, N=24, dim=256, ws=ws, ws_bytes=24 * 256 * 2 + GEMM_WS):
        ptrs = list(base) if ptrs is None else ptrs
        return lib.wanattn_prologue_rms(*ptrs, rms, B, N, dim, 1e-6, 1e-6, ws, ws_bytes, None)

    assert call(rms=None) == wa.E_INVALID
    assert "rms" in lib.wanattn_last_error().decode()
    assert call(rms=ctypes.c_void_p((13 << 32) + 4)) == wa.E_INVALID             # not 16-byte aligned
    for i in range(12):
        ptrs = list(base)
        ptrs[i] = None
        assert call(ptrs) == wa.E_INVALID, i
    assert call(rms=ctypes.c_void_p((12 << 32) + 256)) == wa.E_INVALID           # rms inside v
    assert "rms overlaps" in lib.wanattn_last_error().decode()
    assert call(rms=ctypes.c_void_p((15 << 32) + 4096)) == wa.E_INVALID          # rms inside the workspace
    assert call(dim=12) == wa.E_INVALID
    assert call(ws_bytes=24 * 256 * 2 + GEMM_WS - 1) == wa.E_INVALID


def test_self_qknorm_rejects(lib):
    # self attention with the QK-Norm applied in the call: the self checks,
    # then the factors and the gammas
    R = ctypes.c_void_p(6 << 30)
    GQ = ctypes.c_void_p(7 << 30)
    GK = ctypes.c_void_p(8 << 30)

    def call(rms=R, gq=GQ, gk=GK, o=O, N=24, ws=WS, ws_bytes=1 << 20, theta=1e4):
        return lib.wanattn_self_qknorm(A, B_, C, o, 1, N, 2, 128, g(2, 3, 4), theta, 0.088, 0, 3, None,
                                       rms, gq, gk, ws, ws_bytes, None)

    for kw in (dict(rms=None), dict(gq=None), dict(gk=None)):
        assert call(**kw) == wa.E_INVALID, kw
        assert "gq" in lib.wanattn_last_error().decode()
    assert call(rms=ctypes.c_void_p((6 << 30) + 2)) == wa.E_INVALID               # rms not 4-byte aligned
    assert call(gq=ctypes.c_void_p((7 << 30) + 8)) == wa.E_INVALID                # gamma not 16-byte aligned
    assert call(rms=ctypes.c_void_p((4 << 30) + 64)) == wa.E_INVALID              # rms inside o
    assert "o overlaps" in lib.wanattn_last_error().decode()
    assert call(gk=ctypes.c_void_p((5 << 30) + 64)) == wa.E_INVALID               # gamma inside the workspace
    assert "workspace overlaps" in lib.wanattn_last_error().decode()
    assert call(N=25) == wa.E_INVALID                                             # N != F*H*W
    assert call(theta=0.0) == wa.E_INVALID
    assert call(ws_bytes=16) == wa.E_INVALID                                      # workspace too small


def test_binding_refuses_host_tensors():
    import torch
    x = torch.zeros(1, 24, 2, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        wa.rope3d(x, (2, 3, 4), out=x)
    with pytest.raises(ValueError):
        wa.self_attention(x, x, x, (2, 3, 4), out=x)
    y = torch.zeros(1, 24, 256, dtype=torch.bfloat16)
    w = torch.zeros(256, 256, dtype=torch.bfloat16)
    b = torch.zeros(256, dtype=torch.bfloat16)
    e = torch.zeros(1, 256)
    with pytest.raises(ValueError):
        wa.prologue(y, e, e, w, b, w, b, w, b, b, b, out=(y, y, y))


def test_bench_refuses_more_than_one_gpu():
    # the benchmark measures one device; asked for more it exits before any GPU work
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=root)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""
