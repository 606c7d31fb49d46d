"""Benchmark of the Wan 3D-RoPE attention hot path on one MI355X.

One step = one DiT-block attention pass over one batch of synthetic input:
wanattn_self (3D RoPE fused, bidirectional or block-causal per workload)
followed by wanattn_cross (text tokens), both through the C ABI on torch's
current stream.  Inputs are resident in HBM before the timed region.

Prints ONE JSON line (rank 0).  `value` is the step's algorithmic attention
TFLOP/s (self + cross FLOPs / step time); the self-attention kernel's own
rate and its fraction of the bf16 MFMA peak are in `roofline`.

FLOP counts (Wan2.2 source reading (blog.leeguoo.com), ch. 8: 2 x 2 x L^2 x dim
for the Q K^T and A V products):
  self  = 4 * d * heads * (visible query-key pairs)   (N^2 when bidirectional)
  cross = 4 * d * heads * N * M
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X published dense bf16 MFMA peak
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "attn_fwd_wan14b_720p_81f_hbm_traffic.txt")


def kernel_sources_digest():
    """sha256 over the kernel sources, the public header and the build script
    (the flags the library is compiled with live there)."""
    import glob
    import hashlib
    pkg = os.path.join(ROOT, "video_diffusion_transformer_wanattn_amd")
    files = sorted(glob.glob(os.path.join(pkg, "csrc", "*")))
    files += [os.path.join(ROOT, "include", "wanattn.h"), os.path.join(pkg, "build.py")]
    h = hashlib.sha256()
    for f in files:
        h.update(os.path.relpath(f, ROOT).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(workload):
    """HBM bytes per self-attention launch from the committed counter summary,
    or None when it was taken on other kernel sources or another workload."""
    try:
        fields = dict(line.split(":", 1) for line in open(TRAFFIC_SUMMARY) if ":" in line)
    except OSError:
        return None
    fields = {k.strip(): v.strip() for k, v in fields.items()}
    if fields.get("source_sha256") != kernel_sources_digest() or fields.get("workload") != workload:
        return None
    try:
        return int(fields["attn_fetch_bytes_per_launch"]) + int(fields["attn_write_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def visible_pairs(wl, kv_len=None):
    """Query-key pairs the mask allows (block-causal: own and earlier chunks)."""
    N = wl.N
    L = N if kv_len is None else kv_len
    if not wl.block_causal:
        return N * L
    ct = wl.chunk_frames * wl.H * wl.W
    total = 0
    for c0 in range(0, N, ct):
        rows = min(ct, N - c0)
        total += rows * min(L, c0 + ct)
    return total


def flops(wl):
    d, h = wl.head_dim, wl.heads
    return 4 * d * h * visible_pairs(wl) * wl.batch, 4 * d * h * wl.N * wl.text_len * wl.batch


def host_cpus():
    """The host CPUs this process may use: os.cpu_count(), the affinity set,
    the cgroup CPU quota (if any) and the CPU model."""
    info = {"os_cpu_count": os.cpu_count()}
    try:
        info["affinity"] = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        info["affinity"] = os.cpu_count()
    try:
        quota, period = open("/sys/fs/cgroup/cpu.max").read().split()[:2]
        info["cgroup_quota_cpus"] = None if quota == "max" else round(int(quota) / int(period), 2)
    except (OSError, ValueError):
        info["cgroup_quota_cpus"] = None
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    info["model"] = model
    usable = info["affinity"] or 1
    if info["cgroup_quota_cpus"]:
        usable = min(usable, max(1, int(info["cgroup_quota_cpus"] + 0.5)))
    info["usable"] = usable
    return info


def cpu_baseline(wl, t, threads):
    """Time the fp64 oracle on sampled query rows (all heads) and extrapolate.

    t(R) = a + b R for R rows of every head (a: rotating every key of every
    head, b: one row of every head); full self = a + b N.  Cross needs no
    rotation: full = b_c N.  The oracle is used as it stands."""
    import numpy as np
    import oracle
    from video_diffusion_transformer_wanattn_amd import seeded

    grid = (wl.F, wl.H, wl.W)
    R1, R2 = 64, 448
    rows1 = seeded.sample_rows(wl.N, R1, seed=1)
    rows2 = seeded.sample_rows(wl.N, R2, seed=2)
    kw = dict(theta=10000.0, block_causal=wl.block_causal, chunk_frames=wl.chunk_frames,
              threads=threads)

    def timed(fn):
        t0 = time.perf_counter()
        fn()
        return time.perf_counter() - t0

    t1 = timed(lambda: oracle.self_rows(t["q"], t["k"], t["v"], grid, rows=rows1, **kw))
    log(f"cpu oracle: {len(rows1)} rows x {wl.heads} heads in {t1:.2f}s")
    t2 = timed(lambda: oracle.self_rows(t["q"], t["k"], t["v"], grid, rows=rows2, **kw))
    log(f"cpu oracle: {len(rows2)} rows x {wl.heads} heads in {t2:.2f}s")
    b = max((t2 - t1) / (len(rows2) - len(rows1)), 1e-12)
    a = max(t1 - b * len(rows1), 0.0)
    if wl.block_causal:
        # rows cost in proportion to their visible keys: scale by the mean
        # visible fraction relative to the sampled rows' mean
        ct = wl.chunk_frames * wl.H * wl.W
        vis = lambda r: min(wl.N, (r // ct + 1) * ct)
        mean_all = visible_pairs(wl) / wl.N
        mean_s = float(np.mean([vis(r) for r in np.concatenate([rows1, rows2])]))
        b *= mean_all / mean_s
    rc = seeded.sample_rows(wl.N, 64, seed=3)
    tc = timed(lambda: oracle.cross_rows(t["q"], t["text_k"], t["text_v"], rows=rc, threads=threads))
    log(f"cpu oracle: cross {len(rc)} rows in {tc:.2f}s")
    t_self = a + b * wl.N
    t_cross = tc / len(rc) * wl.N
    f_self, f_cross = flops(wl)
    # the same on one core, on fewer rows (the key rotation dominates there)
    s1, s2 = seeded.sample_rows(wl.N, 4, seed=4), seeded.sample_rows(wl.N, 12, seed=5)
    kw1 = dict(kw, threads=1)
    u1 = timed(lambda: oracle.self_rows(t["q"], t["k"], t["v"], grid, rows=s1, **kw1))
    u2 = timed(lambda: oracle.self_rows(t["q"], t["k"], t["v"], grid, rows=s2, **kw1))
    log(f"cpu oracle, one core: {len(s1)} and {len(s2)} rows x {wl.heads} heads in {u1:.2f}s and {u2:.2f}s")
    b1 = max((u2 - u1) / (len(s2) - len(s1)), 1e-12)
    a1 = max(u1 - b1 * len(s1), 0.0)
    if wl.block_causal:
        b1 *= b / max((t2 - t1) / (len(rows2) - len(rows1)), 1e-12)   # the same visible-key weighting
    t_self1 = a1 + b1 * wl.N
    cpus = host_cpus()
    return {
        "value": (f_self + f_cross) / (t_self + t_cross) / 1e12,
        "unit": "TFLOP/s",
        "cores": threads,
        "host": {"cpu_model": cpus["model"], "os_cpu_count": cpus["os_cpu_count"], "affinity_cpus": cpus["affinity"],
                 "cgroup_quota_cpus": cpus["cgroup_quota_cpus"]},
        "kind": "oracle",
        "sample": (f"fp64 oracle on {len(rows1)} and {len(rows2)} sampled query rows x {wl.heads} heads "
                   f"(self, incl. rotating all keys) and {len(rc)} rows (cross); extrapolated as "
                   f"t = a + b*rows to all {wl.N} rows: self {t_self:.1f} s, cross {t_cross:.1f} s "
                   f"per step"),
        "cpu_s_measured": t1 + t2 + tc + u1 + u2,
        "one_core": {"value": f_self / t_self1 / 1e12, "unit": "TFLOP/s", "cores": 1,
                     "sample": (f"self attention only: {len(s1)} and {len(s2)} rows x {wl.heads} heads on one "
                                f"thread, extrapolated to {t_self1:.0f} s per step")},
    }


def cfg_leg(torch, wa, wl, q, k, v, kc, vc, steps, warmup):
    """One classifier-free-guidance step: the conditional and unconditional
    samples (the same latent tokens, two text contexts trimmed to 77 and 23
    tokens) through self and cross attention in one launch each (B = 2)."""
    grid = (wl.F, wl.H, wl.W)
    q2, k2, v2 = (torch.cat([x, x]) for x in (q, k, v))
    kc2 = torch.cat([kc, kc.flip(1)])
    vc2 = torch.cat([vc, vc.flip(1)])
    lens = [77, 23]
    o2, oc2 = torch.empty_like(q2), torch.empty_like(q2)
    stream = torch.cuda.current_stream()
    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        wa.self_attention(q2, k2, v2, grid, out=o2)
        if ev is not None:
            ev[1].record(stream)
        wa.cross_attention(q2, kc2, vc2, ctx_lens=lens, out=oc2)
        if ev is not None:
            ev[2].record(stream)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for e in evs:
        step(e)
    torch.cuda.synchronize()
    s_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / steps
    c_ms = sum(e[1].elapsed_time(e[2]) for e in evs) / steps
    f_self = 2 * 4 * wl.head_dim * wl.heads * wl.N * wl.N
    f_cross = 4 * wl.head_dim * wl.heads * wl.N * sum(lens)
    log(f"cfg pair: self {s_ms:.3f} ms, cross {c_ms:.3f} ms")
    return {"batch": 2, "ctx_lens": lens, "self_ms": round(s_ms, 3), "cross_ms": round(c_ms, 4),
            "self_tflops": round(f_self / (s_ms * 1e-3) / 1e12, 2),
            "self_frac": round(f_self / (s_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "cross_tflops_visible": round(f_cross / (c_ms * 1e-3) / 1e12, 2)}


def kv_stream_leg(torch, seeded, wa, steps, warmup, jitter=False):
    """One streaming step of Self Forcing: rotate the new chunk's keys into the
    cache (wanattn_rope3d) and attend the chunk's queries to the whole cache
    (wanattn_self_kv).  Times both with HIP events on the launch stream.
    jitter: with multi-head RoPE jitter (per-head tables built once)."""
    import numpy as np
    wl = seeded.WORKLOADS["wan14b_480p_165f_causal"]
    t = seeded.workload_tensors(wl, seed=0, cross=False)
    hw = wl.H * wl.W
    c0 = wl.F - wl.chunk_frames
    dev = lambda bits: torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()
    q = dev(t["q"][:, c0 * hw:])
    k_raw, v = dev(t["k"]), dev(t["v"])
    tables = wa.rope_tables(seeded.jitter_thetas(wl.heads, seed=0)) if jitter else None
    kc = wa.rope3d(k_raw, (wl.F, wl.H, wl.W), tables=tables)   # cache of the earlier chunks, rotated once
    new_k = k_raw[:, c0 * hw:]
    o = torch.empty_like(q)
    stream = torch.cuda.current_stream()
    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        wa.rope3d(new_k, (wl.chunk_frames, wl.H, wl.W), offsets=(c0, 0, 0), out=kc[:, c0 * hw:], tables=tables)
        if ev is not None:
            ev[1].record(stream)
        wa.self_attention_kv(q, kc, v, (wl.chunk_frames, wl.H, wl.W), offsets=(c0, 0, 0), out=o, tables=tables)
        if ev is not None:
            ev[2].record(stream)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for e in evs:
        step(e)
    torch.cuda.synchronize()
    rope_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / steps
    attn_ms = sum(e[1].elapsed_time(e[2]) for e in evs) / steps
    nq, nkv = q.shape[1], k_raw.shape[1]
    f = 4 * wl.head_dim * wl.heads * nq * nkv
    log(f"kv stream{' (jitter)' if jitter else ''}: chunk {nq} x cache {nkv} x {wl.heads} heads: attention {attn_ms:.3f} ms, "
        f"cache append {rope_ms:.3f} ms")
    return {"workload": "wan14b_480p_165f_causal, last chunk (frames 39-41) against the 42-frame cache",
            "q_tokens": nq, "kv_tokens": nkv, "heads": wl.heads, "flops": f,
            "attn_ms": round(attn_ms, 4), "attn_tflops": round(f / (attn_ms * 1e-3) / 1e12, 2),
            "attn_frac": round(f / (attn_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "append_rope_ms": round(rope_ms, 4)}


def jitter_leg(torch, seeded, wa, wl, q, k, v, steps, warmup):
    """Self attention with multi-head RoPE jitter (each head its own RoPE base,
    seeded theta (1 + eps_h)): per-head tables built on the device, the keys
    rotated with them, the attention kernel reading its head's table."""
    thetas = seeded.jitter_thetas(wl.heads, seed=0)
    grid = (wl.F, wl.H, wl.W)
    o = torch.empty_like(q)
    ws = torch.empty(wa.self_jitter_workspace_bytes(wl.batch, wl.N, wl.heads), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        wa.self_attention(q, k, v, grid, block_causal=wl.block_causal, chunk_frames=wl.chunk_frames,
                          theta_per_head=thetas, out=o, workspace=ws)
        if ev is not None:
            ev[1].record(stream)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    for e in evs:
        step(e)
    torch.cuda.synchronize()
    ms = sum(e[0].elapsed_time(e[1]) for e in evs) / steps
    f_self, _ = flops(wl)
    log(f"jitter: self attention with per-head RoPE bases {ms:.3f} ms")
    return {"ms": round(ms, 3), "tflops": round(f_self / (ms * 1e-3) / 1e12, 2),
            "frac": round(f_self / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "thetas": "10000 (1 + eps_h), eps_h ~ N(0, 0.1^2) seeded"}


def prologue_leg(torch, seeded, wa, wl, steps, warmup):
    """The block's self-attention prologue at the workload's token count and
    dim = heads * 128 (5120 for the 14B model): modulated LayerNorm, the three
    q/k/v projections with bias, RMSNorm of q and k, in one wanattn_prologue
    call timed with HIP events on the launch stream."""
    import numpy as np
    dim = wl.heads * wl.head_dim
    t = seeded.prologue_tensors(wl.batch, wl.N, dim, seed=1)
    dev = lambda bits: torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()
    d = {k: dev(v) for k, v in t.items() if k not in ("e0", "e1")}
    e0, e1 = (torch.from_numpy(t[k]).cuda() for k in ("e0", "e1"))
    out = tuple(torch.empty_like(d["x"]) for _ in range(3))
    ws = torch.empty(wa.prologue_workspace_bytes(wl.batch, wl.N, dim), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        wa.prologue(d["x"], e0, e1, d["wq"], d["bq"], d["wk"], d["bk"], d["wv"], d["bv"], d["gq"], d["gk"],
                    out=out, workspace=ws)
        if ev is not None:
            ev[1].record(stream)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    for e in evs:
        step(e)
    torch.cuda.synchronize()
    ms = sum(e[0].elapsed_time(e[1]) for e in evs) / steps
    rows = wl.batch * wl.N
    gemm_flops = 3 * 2 * rows * dim * dim
    row_bytes = 2 * rows * dim * 2 + 4 * rows * dim * 2     # LayerNorm x -> y, RMSNorm q, k in place
    floor_ms = gemm_flops / (PEAK_BF16_TFLOPS * 1e12) * 1e3 + row_bytes / (PEAK_HBM_GBS * 1e9) * 1e3
    log(f"prologue: {rows} tokens x dim {dim}: {ms:.3f} ms (floor {floor_ms:.3f} ms)")
    res = {"workload": f"{wl.name} prologue: {rows} tokens x dim {dim}", "ms": round(ms, 3),
           "gemm_flops": gemm_flops, "row_pass_bytes": row_bytes,
           "tflops_over_gemm_flops": round(gemm_flops / (ms * 1e-3) / 1e12, 2),
           "floor_ms": round(floor_ms, 3), "frac_of_floor": round(floor_ms / ms, 4)}

    # the block up to the attention output, two ways: the prologue with the
    # RMSNorm in place then wanattn_self, or the prologue that leaves the
    # RMSNorm to wanattn_self_qknorm (one pass over q and k fewer)
    shp = (wl.batch, wl.N, wl.heads, wl.head_dim)
    grid = (wl.F, wl.H, wl.W)
    o = torch.empty(shp, dtype=torch.bfloat16, device="cuda")
    rms = torch.empty(2, rows, dtype=torch.float32, device="cuda")
    sws = torch.empty(wa.self_workspace_bytes(*shp), dtype=torch.uint8, device="cuda")
    kw = dict(block_causal=wl.block_causal, chunk_frames=wl.chunk_frames, out=o, workspace=sws)
    qv, kv, vv = (t.view(shp) for t in out)

    def block_in_place():
        wa.prologue(d["x"], e0, e1, d["wq"], d["bq"], d["wk"], d["bk"], d["wv"], d["bv"], d["gq"], d["gk"],
                    out=out, workspace=ws)
        wa.self_attention(qv, kv, vv, grid, **kw)

    def block_deferred():
        wa.prologue_rms(d["x"], e0, e1, d["wq"], d["bq"], d["wk"], d["bk"], d["wv"], d["bv"], out=out, rms=rms,
                        workspace=ws)
        wa.self_attention_qknorm(qv, kv, vv, rms, d["gq"], d["gk"], grid, **kw)

    bsteps = max(2, min(steps, 5))
    for name, fn in (("block_norm_in_place_ms", block_in_place), ("block_norm_deferred_ms", block_deferred)):
        for _ in range(max(1, min(warmup, 2))):
            fn()
        torch.cuda.synchronize()
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(bsteps)]
        for e in evs:
            e[0].record(stream)
            fn()
            e[1].record(stream)
        torch.cuda.synchronize()
        res[name] = round(sum(e[0].elapsed_time(e[1]) for e in evs) / bsteps, 3)
        log(f"block ({name}): {res[name]:.3f} ms")
    return res


METRIC_WORKLOADS = ("wan14b_480p_81f", "wan13b_480p_81f", "wan14b_720p_81f")


def metric_points(torch, seeded, wa, wl_main, main_tflops, main_ms, steps, warmup):
    """Self attention (wanattn_self, the benchmark's launch configuration) at
    every size the metric names: 32,760 tokens (40 and 12 heads) and 75,600
    tokens (40 heads, the step's own figures).  HIP events on the launch stream."""
    import numpy as np
    points = []
    for name in METRIC_WORKLOADS:
        wl = seeded.WORKLOADS[name]
        f_self, _ = flops(wl)
        if name == wl_main.name:
            ms, tf = main_ms, main_tflops
        else:
            t = seeded.workload_tensors(wl, seed=0, cross=False)
            dev = lambda b: torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).view(torch.bfloat16).cuda()
            q, k, v = dev(t["q"]), dev(t["k"]), dev(t["v"])
            o = torch.empty_like(q)
            ws = torch.empty(wa.self_workspace_bytes(wl.batch, wl.N, wl.heads), dtype=torch.uint8, device="cuda")
            grid = (wl.F, wl.H, wl.W)
            stream = torch.cuda.current_stream()
            call = lambda: wa.self_attention(q, k, v, grid, block_causal=wl.block_causal,
                                             chunk_frames=wl.chunk_frames, out=o, workspace=ws)
            for _ in range(warmup):
                call()
            torch.cuda.synchronize()
            evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
            for e0, e1 in evs:
                e0.record(stream)
                call()
                e1.record(stream)
            torch.cuda.synchronize()
            ms = sum(e0.elapsed_time(e1) for e0, e1 in evs) / steps
            tf = f_self / (ms * 1e-3) / 1e12
            del q, k, v, o, ws
            torch.cuda.empty_cache()
        log(f"metric point {name}: {wl.N} tokens x {wl.heads} heads: self {ms:.3f} ms, {tf:.1f} TFLOP/s")
        points.append({"workload": name, "tokens": wl.N, "heads": wl.heads, "self_ms": round(ms, 3),
                       "tflops": round(tf, 2), "frac": round(tf / PEAK_BF16_TFLOPS, 4)})
    return points


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="wan14b_720p_81f")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-metric-points", action="store_true",
                    help="skip timing self attention at the metric's other sizes (32,760 tokens x 40 and 12 heads)")
    ap.add_argument("--cpu-threads", type=int, default=0)
    ap.add_argument("--kv-stream", action="store_true",
                    help="also time one Self Forcing streaming step: the last 3-frame chunk of the "
                         "165-frame, 40-head workload against its full 42-frame key/value cache")
    ap.add_argument("--cfg", action="store_true",
                    help="also time one classifier-free-guidance step of the workload: both "
                         "samples (same latent, text contexts of 77 and 23 tokens) in one launch")
    ap.add_argument("--jitter", action="store_true",
                    help="also time self attention with multi-head RoPE jitter (per-head RoPE bases)")
    ap.add_argument("--prologue", action="store_true",
                    help="also time the block's self-attention prologue (modulated LayerNorm, q/k/v "
                         "projections, QK RMSNorm) at the workload's tokens and dim = heads * 128")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="BYTES",
                    help="also run one plain device copy of BYTES bytes after the timed "
                         "region (a known-size kernel for calibrating memory counters)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the attention kernels run on one device; "
              "sharding heads over several GPUs is not implemented; run with --gpus 1",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from video_diffusion_transformer_wanattn_amd import seeded
    from video_diffusion_transformer_wanattn_amd import wanattn as wa

    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    torch.cuda.set_device(0)
    wl = seeded.WORKLOADS[args.workload]
    grid = (wl.F, wl.H, wl.W)
    log(f"workload {wl.name}: grid {grid} = {wl.N} tokens x {wl.heads} heads x {wl.head_dim}, "
        f"text {wl.text_len}, block_causal={wl.block_causal}")
    t = seeded.workload_tensors(wl, seed=args.seed)
    log("inputs generated")

    def dev(bits):
        import numpy as np
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()

    q, k, v = dev(t["q"]), dev(t["k"]), dev(t["v"])
    kc, vc = dev(t["text_k"]), dev(t["text_v"])
    o_self = torch.empty_like(q)
    o_cross = torch.empty_like(q)
    wa.prepare(10000.0)
    torch.cuda.synchronize()
    log("inputs resident on the GPU")

    stream = torch.cuda.current_stream()
    ev = lambda: torch.cuda.Event(enable_timing=True)
    # rotated keys and the key-split partials, allocated once
    ws = torch.empty(wa.self_workspace_bytes(wl.batch, wl.N, wl.heads), dtype=torch.uint8, device="cuda")

    def step(events=None):
        if events is not None:
            events[0].record(stream)
        wa.self_attention(q, k, v, grid, block_causal=wl.block_causal, chunk_frames=wl.chunk_frames,
                          out=o_self, workspace=ws)
        if events is not None:
            events[1].record(stream)
        wa.cross_attention(q, kc, vc, out=o_cross)
        if events is not None:
            events[2].record(stream)

    for i in range(args.warmup):
        step()
        torch.cuda.synchronize()
        log(f"warmup {i + 1}/{args.warmup}")
    per = [[ev(), ev(), ev()] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(per[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    if args.copy_probe > 0:
        # an elementwise kernel that reads BYTES and writes BYTES (a same-device
        # copy_ may go to a DMA engine, which the shader counters do not see)
        src = torch.ones(args.copy_probe // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        log(f"copy probe: {args.copy_probe} bytes")
        del src, dst
    self_ms = [e[0].elapsed_time(e[1]) for e in per]
    cross_ms = [e[1].elapsed_time(e[2]) for e in per]
    step_ms = wall * 1e3 / args.steps
    log(f"timed {args.steps} steps: {step_ms:.3f} ms/step (self {sum(self_ms) / len(self_ms):.3f} ms, "
        f"cross {sum(cross_ms) / len(cross_ms):.3f} ms)")

    f_self, f_cross = flops(wl)
    self_avg = sum(self_ms) / len(self_ms)
    cross_avg = sum(cross_ms) / len(cross_ms)
    achieved = f_self / (self_avg * 1e-3) / 1e12
    cross_bytes = (2 * wl.N + 2 * wl.text_len) * wl.heads * wl.head_dim * 2 * wl.batch

    result = {
        "metric": "self-attn TFLOP/s + % bf16 MFMA peak at 32,760 and 75,600 tokens (1 GPU)",
        "value": round((f_self + f_cross) / (step_ms * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "batch": wl.batch, "tokens": wl.N, "grid": list(grid),
                   "heads": wl.heads, "head_dim": wl.head_dim, "text_tokens": wl.text_len,
                   "mask": "block_causal" if wl.block_causal else "bidirectional",
                   "chunk_frames": wl.chunk_frames if wl.block_causal else None,
                   "rope_theta": 10000.0, "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": measured_traffic(wl.name), "kernel": "attn_fwd_kernel (wanattn_self)",
                     "flops_per_launch": f_self},
        "self_ms": round(self_avg, 3),
        "self_ms_median": round(statistics.median(self_ms), 3),
        "self_ms_min": round(min(self_ms), 3),
        "self_tflops": round(achieved, 2),
        "cross_ms": round(cross_avg, 4),
        "cross_ms_median": round(statistics.median(cross_ms), 4),
        "cross_ms_min": round(min(cross_ms), 4),
        "cross_tflops": round(f_cross / (cross_avg * 1e-3) / 1e12, 2),
        "cross_gbs": round(cross_bytes / (cross_avg * 1e-3) / 1e9, 1),
        "cross_frac_hbm": round(cross_bytes / (cross_avg * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
        "cross_frac_mfma": round(f_cross / (cross_avg * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        # the binding roof is the larger of the two times at peak
        "cross_bound": "mfma" if f_cross / PEAK_BF16_TFLOPS / 1e12 >= cross_bytes / PEAK_HBM_GBS / 1e9 else "hbm",
    }
    if args.kv_stream:
        result["kv_stream"] = kv_stream_leg(torch, seeded, wa, args.steps, args.warmup)
        if args.jitter:
            result["kv_stream_jitter"] = kv_stream_leg(torch, seeded, wa, args.steps, args.warmup, jitter=True)
    if args.cfg:
        del o_self, o_cross
        result["cfg_batch"] = cfg_leg(torch, wa, wl, q, k, v, kc, vc, args.steps, args.warmup)
    if args.jitter:
        result["jitter"] = jitter_leg(torch, seeded, wa, wl, q, k, v, args.steps, args.warmup)
    if args.prologue:
        result["prologue"] = prologue_leg(torch, seeded, wa, wl, args.steps, args.warmup)
    if not args.no_metric_points:
        result["metric_points"] = metric_points(torch, seeded, wa, wl, achieved, self_avg, args.steps, args.warmup)
    if not args.no_cpu_baseline:
        # every CPU this process may run on (the affinity set, within any cgroup quota)
        threads = args.cpu_threads or host_cpus()["usable"]
        result["cpu_baseline"] = cpu_baseline(wl, t, threads)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
