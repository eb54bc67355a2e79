"""Benchmark of the chunkwise gated delta rule (Muir) on one MI355X.

Prints ONE JSON line. A step is one pass of the chunk forward over one layer call of
the long-context workload (B=1, H=16, d=128, T=32768, chunk 256, bf16 q/k/v, fp32
gates and state): the parallel phase (decay products, pivoted operands, Gram blocks)
then the sequential phase (block-Neumann solve, readout, state carry). ``value`` is
tokens/s per layer over the timed steps, with inputs already resident in HBM.

Also measured in the same run and reported as secondary fields: the 1.34B-class
shape at T=4096 (B=8, chunk 128 and 256), the output-gate epilogue, the shared-erase
variant, the forward with its gates made from the low-rank gate projection, and the
decode step (B=256 x H=16 x 128x128 fp32 states, one layer call) in GB/s. Each kernel's average duration comes from HIP
events recorded around it on the stream it runs on. ``cpu_baseline`` is the CPU
oracle's fp32 token recurrence on the same long-context workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--only main]
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK = 8.0e12          # bytes/s, MI355X HBM3E
BF16_PEAK = 2.5166e15      # flop/s, dense bf16 MFMA (256 CU x 4096 flop/clk x 2.4 GHz)
NAMES = "q k v a g e w r".split()


def algorithmic(d, chunk, qkv_bytes=2):
    """Per token-head algorithmic bytes and MFMA flops of each phase.

    prepare: reads q, k (qkv dtype) and a, g (fp32); Gram M and P: 2*C*d flops.
    scan:    reads v (qkv dtype), e, w (fp32), writes o (qkv dtype);
             H, (Qh*gamma) S0, (K*beta)^T U: 6*d*d flops; solve and P U: 2*C*d flops.
    """
    return {
        "prepare": {"bytes": 2 * d * qkv_bytes + 2 * d * 4, "flops": 2 * chunk * d},
        "scan": {"bytes": 2 * d * qkv_bytes + 2 * d * 4, "flops": 6 * d * d + 2 * chunk * d},
    }


def flop_tally(C, d, leaf=16):
    """Flops per token-head of the chunk forward as these kernels organise it, split into the
    matrix-core products and the vector work around them (algorithmic counts: the useful
    multiply-adds, 2 flops each, of a chunk of C tokens with 16-token leaves, divided by C).

    Matrix cores: the Gram blocks between leaves and inside them (M strictly lower, P
    inclusive), the three state products (K*gamma) S0, (Qh*gamma) S0, (K*beta)^T U, the solve's
    terms between leaves and the readout P U. Vector: decay running products (prefix and
    suffix), operand scalings, the scaling of every off-diagonal Gram block by the decay of the
    blocks between, the scalings of the diagonal blocks' four recursion levels, the leaf
    substitution (a coefficient and an FMA per strictly-lower entry and value column), the
    right-hand side w*v - e*acc, and the state's pair decay (one multiply per state entry per
    32-token leaf pair). The pages put 98% of the chunkwise flops on the matrix units (liuch.name
    summary, third bullet)."""
    nb = C // leaf
    lower = leaf * (leaf - 1) // 2            # strictly-lower entries of a leaf
    pairs = nb * (nb - 1) // 2                # leaf pairs (later, earlier) in a chunk
    mfma = {
        "gram_between_leaves": pairs * 2 * leaf * leaf * 2 * d / C,
        "gram_inside_leaves": nb * (lower + lower + leaf) * 2 * d / C,
        "state_products": 3 * 2 * d * d,
        "solve_between_leaves": pairs * leaf * leaf * 2 * d / C,
        "readout_PU": (C * (C + 1) // 2) * 2 * d / C,
    }
    valu = {
        "decay_products": 2 * d,
        "operand_scaling": 8 * d,
        "gram_block_scaling": pairs * leaf * d / C,
        "diag_level_scaling": 4 * 2 * d,
        "leaf_substitution": nb * lower * 3 * d / C,
        "rhs": 3 * d,
        "state_pair_decay": d * d / 32,
    }
    m, v = sum(mfma.values()), sum(valu.values())
    return {"mfma": mfma, "valu": valu, "mfma_flops": m, "valu_flops": v,
            "mfma_share": m / (m + v)}


CSRC = os.path.join(ROOT, "gated_delta_rule_06_amd", "csrc")
# The sources of the channel-wise chunk kernels: the kernel file and the headers it includes.
CHUNK_SOURCES = [os.path.join(CSRC, f) for f in
                 ("chunk_fwd.hip", "chunk_scan_split.hip", "scan_leaf.hpp", "chunk_layout.hpp",
                  "layout.hpp", "mfma.hpp", "common.hpp")]


def code_sha(*paths):
    """sha256 prefix of C/HIP sources with their comments and whitespace removed, so that
    it changes with the code but not with its comments."""
    import hashlib
    import re
    h = hashlib.sha256()
    for path in paths:
        text = open(path).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        text = re.sub(r"\s+", "", text)
        h.update(text.encode())
    return h.hexdigest()[:16]


def measured_traffic(kernel):
    """HBM bytes per call of `kernel` ('prepare', or 'scan': the split scan and its readout kernel)
    on the long-context workload,
    from the rocprofv3 FETCH_SIZE / WRITE_SIZE summary under profiles/ (scaled by the copy
    calibration recorded there). None when the summary is missing or was taken on
    different code (its code_sha differs from the current source's)."""
    import re
    path = os.path.join(ROOT, "profiles", "chunk_fwd_long_context_hbm_counters.md")
    try:
        text = open(path).read()
        sha = code_sha(*CHUNK_SOURCES)
    except OSError:
        return None
    m = re.search(r"traffic sha=(\w+) prepare_bytes=(\d+) scan_bytes=(\d+)", text)
    if not m or m.group(1) != sha:
        return None
    return float(m.group(2) if kernel == "prepare" else m.group(3))


def measured_mfma():
    """Matrix-core busy shares of the long-context prepare and scan and the executed-flop share on
    the matrix cores, from the rocprofv3 counter summary under profiles/, or None when it was
    taken on different code."""
    import re
    path = os.path.join(ROOT, "profiles", "chunk_fwd_mfma_counters.md")
    try:
        text = open(path).read()
        sha = code_sha(*CHUNK_SOURCES)
    except OSError:
        return None
    m = re.search(r"mfma sha=(\w+) prepare_busy=([\d.]+) scan_busy=([\d.]+) mfma_share_executed=([\d.]+)",
                  text)
    if not m or m.group(1) != sha:
        return None
    return {"prepare_mfma_busy": float(m.group(2)), "scan_mfma_busy": float(m.group(3)),
            "mfma_share_of_executed_flops": float(m.group(4))}


def to_dev(inp, dev):
    import numpy as np
    import torch
    qdt = torch.bfloat16 if inp["qkv"] == "bf16" else torch.float32
    return {n: torch.from_numpy(np.ascontiguousarray(inp[n])).to(
        dev, qdt if n in ("q", "k", "v") else torch.float32) for n in NAMES}


def time_chunk(inp, chunk, dev, steps, warmup, og=None):
    """Time `steps` chunk forwards; returns dict of per-step and per-kernel times (ms).
    With `og` (a numpy [B,T,H,dv] array) the scan runs the output-gate epilogue."""
    import numpy as np
    import torch
    import gated_delta_rule_06_amd as muir
    t = to_dev(inp, dev)
    og_t = None if og is None else torch.from_numpy(np.ascontiguousarray(og)).to(dev)
    B, T, H, d = inp["B"], inp["T"], inp["H"], inp["d"]
    code = muir.MUIR_BF16 if inp["qkv"] == "bf16" else muir.MUIR_F32
    ws = torch.empty(muir.chunk_fwd_workspace_size(B, T, H, d, d, chunk, code),
                     dtype=torch.uint8, device=dev)
    o = torch.empty_like(t["v"])
    s_out = torch.empty(B, H, d, d, dtype=torch.float32, device=dev)

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        muir.chunk_fwd_prepare(t["q"], t["k"], t["a"], t["g"], t["r"], chunk=chunk, workspace=ws)
        if ev is not None:
            ev[1].record()
        muir.chunk_fwd_scan(t["v"], t["e"], t["w"], None, chunk=chunk, workspace=ws, o=o,
                            s_out=s_out, og=og_t)
        if ev is not None:
            ev[2].record()

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3
    prep = [e[0].elapsed_time(e[1]) for e in evs]
    scan = [e[1].elapsed_time(e[2]) for e in evs]
    total = evs[0][0].elapsed_time(evs[-1][2])
    assert torch.isfinite(o.float()).all() and torch.isfinite(s_out).all()
    return {"ms_per_step": total / steps, "wall_ms_per_step": wall / steps,
            "prepare_ms": sum(prep) / steps, "scan_ms": sum(scan) / steps,
            "o": o, "s_out": s_out}


def nonfinite_heads(o, s_out):
    """Heads (b, h) with any non-finite value in their output or final state."""
    import torch
    bad_o = ~torch.isfinite(o.float()).all(dim=3).all(dim=1)     # [B, H]
    bad_s = ~torch.isfinite(s_out).all(dim=3).all(dim=2)         # [B, H]
    return int((bad_o | bad_s).sum().item())


def time_scalar_erase(inp, es, chunk, dev, steps, warmup):
    """Time `steps` shared-erase forwards (e one value per token and head): the prepare, the
    chunk-parallel solve (inverse and per-chunk products) and the scan (state recurrence and
    readout), each between HIP events on the stream."""
    import numpy as np
    import torch
    import gated_delta_rule_06_amd as muir
    t = to_dev(inp, dev)
    e_t = torch.from_numpy(np.ascontiguousarray(es)).to(dev)
    B, T, H, d = inp["B"], inp["T"], inp["H"], inp["d"]
    ws = torch.empty(muir.chunk_fwd_scalar_erase_workspace_size(B, T, H, d, d, chunk),
                     dtype=torch.uint8, device=dev)
    o = torch.empty_like(t["v"])
    s_out = torch.empty(B, H, d, d, dtype=torch.float32, device=dev)

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        muir.chunk_fwd_prepare(t["q"], t["k"], t["a"], t["g"], t["r"], chunk=chunk, workspace=ws)
        if ev is not None:
            ev[1].record()
        muir.chunk_fwd_scalar_erase_solve(t["v"], e_t, t["w"], chunk=chunk, workspace=ws)
        if ev is not None:
            ev[2].record()
        muir.chunk_fwd_scalar_erase_scan(B=B, T=T, H=H, d=d, chunk=chunk, workspace=ws, o=o,
                                         s_out=s_out)
        if ev is not None:
            ev[3].record()

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    for i in range(steps):
        step(evs[i])
    torch.cuda.synchronize()
    phase = lambda a, b: sum(e[a].elapsed_time(e[b]) for e in evs) / steps
    total = evs[0][0].elapsed_time(evs[-1][3]) / steps
    assert torch.isfinite(o.float()).all() and torch.isfinite(s_out).all()
    tok_heads = B * T * H
    # Algorithmic bytes per token-head: q, k (bf16), a, g (fp32) | e (one fp32) | v (bf16),
    # e, w (fp32), o (bf16).
    nbytes = (2 * d * 2 + 2 * d * 4) + 4 + (d * 2 + 4 + d * 4 + d * 2)
    sec = total * 1e-3
    return {"tokens_per_s_per_layer": B * T / sec, "ms_per_call": total,
            "prepare_ms": phase(0, 1), "solve_ms": phase(1, 2), "scan_ms": phase(2, 3),
            "hbm_frac": nbytes * tok_heads / sec / HBM_PEAK}


def time_lowrank(inp, lr, chunk, dev, steps, warmup):
    """The forward with its gates from the low-rank gate projection: the fused call
    (muir_chunk_fwd_lowrank) and, for comparison, the gate kernel writing all four gates
    followed by the plain forward; each timed with HIP events over `steps` calls."""
    import torch
    import gated_delta_rule_06_amd as muir
    t = to_dev(inp, dev)
    B, T, H, d = inp["B"], inp["T"], inp["H"], inp["d"]
    z = torch.from_numpy(lr["z"]).to(dev, torch.bfloat16)
    names = ("decay", "erase", "write", "read")
    U = {n: torch.from_numpy(lr["U_" + n]).to(dev, torch.bfloat16) for n in names}
    c = {n: torch.from_numpy(lr["c_" + n]).to(dev) for n in names}
    o = torch.empty_like(t["v"])
    s_out = torch.empty(B, H, d, d, dtype=torch.float32, device=dev)
    ws = torch.empty(int(muir.lib().muir_chunk_fwd_lowrank_workspace_size(B, T, H, d, d, chunk)),
                     dtype=torch.uint8, device=dev)
    gates = {k: torch.empty((B, T, H, d), dtype=torch.float32, device=dev) for k in "aewg"}

    def fused():
        muir.chunk_fwd_lowrank(t["q"], t["k"], t["v"], z, U, c, t["r"], chunk=chunk, o=o,
                               s_out=s_out, workspace=ws)

    def unfused():
        muir.lowrank_gates(z, U, c, H=H, d=d, out=gates)
        muir.chunk_fwd(t["q"], t["k"], t["v"], gates["a"], gates["g"], gates["e"], gates["w"],
                       t["r"], chunk=chunk, o=o, s_out=s_out, workspace=ws)

    def timed(fn):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    tf, tu = timed(fused), timed(unfused)
    assert torch.isfinite(o.float()).all() and torch.isfinite(s_out).all()
    return {"tokens_per_s_per_layer": B * T / (tf * 1e-3), "ms_per_call": tf,
            "unfused_ms_per_call": tu}


def chunk_report(name, inp, chunk, r):
    d, tok_heads = inp["d"], inp["B"] * inp["T"] * inp["H"]
    alg = algorithmic(d, chunk)
    out = {"workload": name, "chunk": chunk,
           "tokens_per_s_per_layer": inp["B"] * inp["T"] / (r["ms_per_step"] * 1e-3),
           "ms_per_call": r["ms_per_step"], "prepare_ms": r["prepare_ms"], "scan_ms": r["scan_ms"]}
    call_bytes = sum(p["bytes"] for p in alg.values()) * tok_heads
    call_flops = sum(p["flops"] for p in alg.values()) * tok_heads
    sec = r["ms_per_step"] * 1e-3
    out["hbm_frac"] = call_bytes / sec / HBM_PEAK
    out["mfma_frac"] = call_flops / sec / BF16_PEAK
    return out


def bwd_bytes(d, qkv_bytes=2):
    """Algorithmic bytes of the backward pass per token-head: q, k, v, dO read once (qkv dtype),
    a, g, e, w read once (fp32), dq, dk, dv, a*dL/da, dg, de, dw written once (fp32)."""
    return 4 * d * qkv_bytes + 4 * d * 4 + 7 * d * 4


def time_backward(inp, dev, steps, warmup, name):
    """Time `steps` backward calls (forward rerun inside, chunks of 64) with HIP events on the
    stream the library is called on."""
    import numpy as np
    import torch
    import gated_delta_rule_06_amd as muir
    t = to_dev(inp, dev)
    B, T, H, d = inp["B"], inp["T"], inp["H"], inp["d"]
    code = muir.MUIR_BF16 if inp["qkv"] == "bf16" else muir.MUIR_F32
    rng = np.random.default_rng(7)
    do = torch.from_numpy(rng.standard_normal((B, T, H, d), dtype=np.float32)).to(dev, t["v"].dtype)
    ws = torch.empty(muir.chunk_bwd_workspace_size(B, T, H, d, d, 64, code), dtype=torch.uint8,
                     device=dev)
    args = [t[n] for n in NAMES]
    out = muir.chunk_bwd(*args, do=do, workspace=ws)
    for _ in range(warmup):
        muir.chunk_bwd(*args, do=do, workspace=ws, out=out)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        muir.chunk_bwd(*args, do=do, workspace=ws, out=out)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    assert all(torch.isfinite(x).all() for x in out.values())
    ach = bwd_bytes(d) * B * T * H / (ms * 1e-3)
    return {"workload": name, "chunk": 64, "ms_per_call": ms,
            "tokens_per_s_per_layer": B * T / (ms * 1e-3),
            "workspace_GB": ws.numel() / 1e9,
            "call_roofline": {"bound": "hbm", "achieved_GBps": ach / 1e9,
                              "peak_GBps": HBM_PEAK / 1e9, "frac": ach / HBM_PEAK,
                              "bytes_per_token_head": bwd_bytes(d)}}


def time_decode(dev, steps, warmup):
    import numpy as np
    import torch
    import gated_delta_rule_06_amd as muir
    import workloads
    cfg = workloads.DECODE_CONFIG
    B, H, d = cfg.B, cfg.H, cfg.d
    u, r = workloads.decode_base(cfg, L=1)
    u_t = torch.from_numpy(u.astype(np.float32)).to(dev)
    x = workloads.decode_step_inputs_torch(0, u_t, dev, B=B, cfg=cfg)
    args = [x[n][0] for n in ("q", "k", "v", "a", "g", "e", "w")]
    r_t = torch.from_numpy(r[0]).to(dev)
    state = torch.randn(B, H, d, d, device=dev) * 0.1
    o = torch.empty(B, H, d, dtype=torch.bfloat16, device=dev)
    for _ in range(warmup):
        muir.decode_step(*args, r_t, state, o=o)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        muir.decode_step(*args, r_t, state, o=o)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    per_head = 2 * d * d * 4 + 3 * d * 2 + 4 * d * 4 + d * 2   # 134,144 B at d = 128
    gbs = per_head * B * H / (ms * 1e-3) / 1e9
    assert torch.isfinite(state).all()
    return {"workload": "decode B256 H16 d128, one layer call repeated on the same 268 MB of "
                        "state (much of it stays in the 256 MB last-level cache; the 24-layer "
                        "workload below is the HBM figure)", "ms_per_call": ms,
            "GB_per_s": gbs, "hbm_frac": gbs * 1e9 / HBM_PEAK, "bytes_per_head_step": per_head}


def time_decode_workload(dev, steps, warmup):
    """The decode workload: every step runs the 24 layer calls (B=256 sequences x 16 heads,
    128x128 fp32 states, 6.4 GB of state in all) on that step's freshly drawn inputs. The
    24 calls of each step are timed between HIP events on the launch stream; drawing the
    next step's inputs happens outside them."""
    import numpy as np
    import torch
    import gated_delta_rule_06_amd as muir
    import workloads
    cfg = workloads.DECODE_CONFIG
    B, L, H, d = cfg.B, cfg.L, cfg.H, cfg.d
    u, r = workloads.decode_base(cfg)
    u_t = torch.from_numpy(u.astype(np.float32)).to(dev)
    r_t = torch.from_numpy(r).to(dev)
    states = torch.zeros(L, B, H, d, d, device=dev)
    o = torch.empty(L, B, H, d, dtype=torch.bfloat16, device=dev)
    ms = []
    for step in range(warmup + steps):
        x = workloads.decode_step_inputs_torch(step, u_t, dev, B=B, cfg=cfg)
        args = [x[n] for n in ("q", "k", "v", "a", "g", "e", "w")]
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for layer in range(L):
            muir.decode_step(*[t[layer] for t in args], r_t[layer], states[layer], o=o[layer])
        e1.record()
        if step >= warmup:
            ms.append((e0, e1))
        del x, args
    torch.cuda.synchronize()
    step_ms = sum(a.elapsed_time(b) for a, b in ms) / steps
    per_head = 2 * d * d * 4 + 3 * d * 2 + 4 * d * 4 + d * 2
    gbs = per_head * B * H * L / (step_ms * 1e-3) / 1e9
    assert torch.isfinite(states).all() and torch.isfinite(o.float()).all()
    return {"workload": f"decode B{B} x {L} layers x H{H} d{d}, fp32 states ({B * L * H * d * d * 4 / 1e9:.2f} GB)",
            "steps_timed": steps, "ms_per_step_24_layers": step_ms,
            "tokens_per_s": B / (step_ms * 1e-3), "GB_per_s": gbs, "hbm_frac": gbs * 1e9 / HBM_PEAK,
            "s_for_1024_steps": step_ms * 1024 / 1e3}


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_decode_baseline(dev, steps=48):
    """The CPU oracle's fp32 token recurrence on a bounded sample of the decode workload: one
    layer's 256 x 16 states from a random state, `steps` tokens each (the oracle's loop over
    tokens is the decode step repeated), extrapolated linearly to 24 layers x 1024 steps."""
    import numpy as np
    import torch
    import oracle
    import workloads
    cfg = workloads.DECODE_CONFIG
    B, H, d = cfg.B, cfg.H, cfg.d
    u, r = workloads.decode_base(cfg, L=1)
    u_t = torch.from_numpy(u.astype(np.float32)).to(dev)
    xs = [workloads.decode_step_inputs_torch(i, u_t, dev, B=B, cfg=cfg) for i in range(steps)]
    host = {n: np.stack([x[n][0].float().cpu().numpy() for x in xs], axis=1) for n in xs[0]}
    del xs
    s0 = (np.random.default_rng(4).standard_normal((B, H, d, d)) * 0.1).astype(np.float32)
    threads = oracle.max_threads()
    t0 = time.perf_counter()
    oracle.recurrent(host["q"], host["k"], host["v"], host["a"], host["g"], host["e"], host["w"],
                     r[0], s0=s0, precision="f32", threads=threads)
    sec = time.perf_counter() - t0
    full = sec / steps * cfg.L * 1024
    per_head = 2 * d * d * 4 + 3 * d * 2 + 4 * d * 4 + d * 2
    return {"value": cfg.L * 1024 / full, "unit": "decode steps/s (24 layers, 256 sequences)",
            "cores": threads, "kind": "oracle", "extrapolated": True,
            "state_GB_per_s": per_head * B * H * steps / sec / 1e9,
            "s_for_1024_steps": full,
            "sample": f"fp32 token recurrence in C (OpenMP) over one layer's {B}x{H} states for "
                      f"{steps} tokens ({sec:.1f} s), extrapolated linearly to {cfg.L} layers x 1024 steps"}


def cpu_baseline(inp, budget_s=20.0):
    """The CPU oracle (fp32 token recurrence, as it stands) on a bounded sample of the
    long-context workload: all 16 heads, the first T_s tokens, T_s sized from a short
    probe so the measured run takes at most ~budget_s."""
    import oracle
    threads = oracle.max_threads()
    T = inp["T"]
    sl = lambda n, T_s: inp[n][:, :T_s] if n != "r" else inp[n]
    probe = min(T, 1024)
    t0 = time.perf_counter()
    oracle.recurrent(*[sl(n, probe) for n in NAMES], precision="f32", threads=threads)
    per_tok = (time.perf_counter() - t0) / probe
    T_s = int(min(T, max(probe, budget_s / max(per_tok, 1e-9))))
    t0 = time.perf_counter()
    oracle.recurrent(*[sl(n, T_s) for n in NAMES], precision="f32", threads=threads)
    sec = time.perf_counter() - t0
    return {"value": inp["B"] * T_s / sec, "unit": "tokens/s/layer", "cores": threads,
            "kind": "oracle", "cpu_model": cpu_model(),
            "sample": f"fp32 token recurrence in C (OpenMP) on the first {T_s} of {T} tokens, "
                      f"all {inp['H']} heads, B={inp['B']}, d={inp['d']}; {sec:.1f} s"}


def sampled_head_errors(inp, o, s_out, heads):
    """Per-head max relative error (max |x - ref| / max |ref| over the head) of the timed
    call's output and final state on the given heads, against the oracle's fp64 recurrence
    over the whole sequence (run beside the CPU baseline, outside any timed region)."""
    import numpy as np
    import oracle
    sl = {n: np.ascontiguousarray(inp[n][:, :, heads]) if n != "r" else inp[n][heads] for n in NAMES}
    o_ref, s_ref = oracle.recurrent(*[sl[n] for n in NAMES])
    o_g = o[:, :, heads].float().cpu().numpy()
    s_g = s_out[:, heads].cpu().numpy()
    eo = np.abs(o_g - o_ref).max(axis=(0, 1, 3)) / np.abs(o_ref).max(axis=(0, 1, 3))
    es = np.abs(s_g - s_ref).max(axis=(0, 2, 3)) / np.abs(s_ref).max(axis=(0, 2, 3))
    return {"heads": list(heads), "o_max_rel_err": [float(x) for x in eo],
            "state_max_rel_err": [float(x) for x in es],
            "stress_heads": [h for h in heads if h in inp["stress_heads"]]}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--only", choices=["all", "main", "t4k", "decode", "scalar", "lowrank", "bwd",
                                       "copy"],
                    default="all",
                    help="'copy' times a plain 1 GiB device copy: the known-size kernel that "
                         "calibrates the FETCH_SIZE / WRITE_SIZE counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the chunk forward shards over (batch, head) with no "
              f"communication and no multi-GPU path is built; --gpus {args.gpus} is not run.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import workloads
    dev = torch.device("cuda", 0)
    torch.cuda.init()
    if args.only == "copy":
        n = 1 << 30
        src = torch.ones(n // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        dst.copy_(src)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(args.steps):
            dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / args.steps
        print(json.dumps({"metric": "device copy GB/s", "value": 2 * n / (ms * 1e-3) / 1e9,
                          "unit": "GB/s", "bytes_read_per_launch": n, "bytes_written_per_launch": n,
                          "ms_per_launch": ms, "n_gpus": 1, "steps": args.steps}), flush=True)
        return

    result = {"metric": "chunk-fwd tokens/s/layer @H16 d128 T4K/32K; %MFMA peak; "
                        "decode-step HBM GB/s",
              "unit": "tokens/s/layer", "n_gpus": 1, "steps": args.steps,
              "warmup": args.warmup, "higher_is_better": True, "scaling": "weak",
              "vs_baseline": None, "dtype": "bf16", "data": "synthetic"}
    secondary = {}
    main_inp = main_out = None
    if args.only in ("all", "main"):
        main_inp = workloads.chunk_inputs(3)
        name = "chunk_fwd long-context B1 H16 d128 T32768 C256 bf16"
        print(f"bench: {name}", file=sys.stderr, flush=True)
        r = time_chunk(main_inp, 256, dev, args.steps, args.warmup)
        rep = chunk_report(name, main_inp, 256, r)
        result["value"] = rep["tokens_per_s_per_layer"]
        result["ms_per_step"] = r["ms_per_step"]
        result["config"] = {"workload": name, "B": 1, "T": 32768, "H": 16, "d": 128,
                            "chunk": 256, "qkv": "bf16", "gates": "fp32", "state": "fp32"}
        alg = algorithmic(128, 256)
        tok_heads = main_inp["B"] * main_inp["T"] * main_inp["H"]
        dom = "scan" if r["scan_ms"] >= r["prepare_ms"] else "prepare"
        dom_ms = r[f"{dom}_ms"]
        ach = alg[dom]["bytes"] * tok_heads / (dom_ms * 1e-3) / 1e9
        # The sequential phase is two launches: the split scan and the readout kernel it hands
        # S0 and U to; its HIP-event time and its counter traffic cover both.
        kname = ("chunk_scan (chunk_scan_split_kernel + chunk_readout_kernel)" if dom == "scan"
                 else "chunk_prepare")
        result["roofline"] = {"bound": "hbm", "kernel": kname, "achieved": ach,
                              "peak": HBM_PEAK / 1e9, "unit": "GB/s",
                              "frac": ach * 1e9 / HBM_PEAK, "traffic": measured_traffic(dom),
                              "avg_ms": dom_ms}
        result["phases_ms"] = {"prepare": r["prepare_ms"], "scan": r["scan_ms"]}
        result["nan_heads"] = nonfinite_heads(r["o"], r["s_out"])
        main_out = (r["o"], r["s_out"])
        result["call_roofline"] = {"hbm_frac": rep["hbm_frac"], "mfma_frac_bf16": rep["mfma_frac"],
                                   "counters": measured_mfma()}
        tally = flop_tally(256, 128)
        result["flop_share"] = {"mfma_share_algorithmic": tally["mfma_share"],
                                "mfma_flops_per_token_head": tally["mfma_flops"],
                                "valu_flops_per_token_head": tally["valu_flops"]}
        # The same call with the output-gate epilogue fused into the readout.
        og = workloads.output_gate(1, 32768, 16, 128, seed=3)
        rg = time_chunk(main_inp, 256, dev, args.steps, args.warmup, og=og)
        del og
        secondary["long_context_output_gate"] = {
            "workload": name + " + output-gate epilogue (og fp32)",
            "tokens_per_s_per_layer": 32768 / (rg["ms_per_step"] * 1e-3),
            "ms_per_call": rg["ms_per_step"], "prepare_ms": rg["prepare_ms"],
            "scan_ms": rg["scan_ms"]}
    if args.only in ("all", "t4k"):
        inp = workloads.chunk_inputs(2)
        for chunk in (128, 256):
            name = f"chunk_fwd 1.34B-class B8 H16 d128 T4096 C{chunk} bf16"
            print(f"bench: {name}", file=sys.stderr, flush=True)
            r = time_chunk(inp, chunk, dev, args.steps, args.warmup)
            secondary[f"t4k_c{chunk}"] = chunk_report(name, inp, chunk, r)
        del inp
        if "value" not in result:
            best = secondary["t4k_c256"]
            result["value"] = best["tokens_per_s_per_layer"]
            result["ms_per_step"] = best["ms_per_call"]
            result["config"] = {"workload": best["workload"]}
    if args.only in ("all", "scalar"):
        # The shared-erase variant (one erase strength per token and head), same inputs.
        for cfg, chunk, key in ((3, 256, "long_context_scalar_erase"),
                                (2, 128, "t4k_c128_scalar_erase")):
            inp = main_inp if (cfg == 3 and main_inp is not None) else workloads.chunk_inputs(cfg)
            es = workloads.scalar_erase(inp["B"], inp["T"], inp["H"], seed=cfg)
            name = (f"chunk_fwd_scalar_erase B{inp['B']} H{inp['H']} d{inp['d']} T{inp['T']} "
                    f"C{chunk} bf16, e [B,T,H]")
            print(f"bench: {name}", file=sys.stderr, flush=True)
            secondary[key] = {"workload": name, "chunk": chunk,
                              **time_scalar_erase(inp, es, chunk, dev, args.steps, args.warmup)}
            del inp, es
        if "value" not in result:
            first = secondary["long_context_scalar_erase"]
            result["value"] = first["tokens_per_s_per_layer"]
            result["ms_per_step"] = first["ms_per_call"]
            result["config"] = {"workload": first["workload"]}
    if args.only in ("all", "lowrank"):
        # Gates from the low-rank gate projection, made inside the call.
        for cfg, chunk, key in ((3, 256, "long_context_lowrank_gates"),
                                (2, 128, "t4k_c128_lowrank_gates")):
            inp = main_inp if (cfg == 3 and main_inp is not None) else workloads.chunk_inputs(cfg)
            lr = workloads.lowrank_gate_inputs(cfg)
            name = (f"chunk_fwd_lowrank B{inp['B']} H{inp['H']} d{inp['d']} T{inp['T']} C{chunk} "
                    f"bf16, gates from z [B,T,512] and rank 64/64/128/128 up-projections")
            print(f"bench: {name}", file=sys.stderr, flush=True)
            secondary[key] = {"workload": name, "chunk": chunk,
                              **time_lowrank(inp, lr, chunk, dev, args.steps, args.warmup)}
            del inp, lr
        if "value" not in result:
            first = secondary["long_context_lowrank_gates"]
            result["value"] = first["tokens_per_s_per_layer"]
            result["ms_per_step"] = first["ms_per_call"]
            result["config"] = {"workload": first["workload"]}
    if args.only in ("all", "bwd"):
        # The backward pass (gradients of every input), chunks of 64.
        for cfg, key in ((2, "t4k_backward"), (3, "long_context_backward")):
            inp = main_inp if (cfg == 3 and main_inp is not None) else workloads.chunk_inputs(cfg)
            name = (f"chunk_bwd B{inp['B']} H{inp['H']} d{inp['d']} T{inp['T']} C64 bf16, "
                    f"every input's gradient")
            print(f"bench: {name}", file=sys.stderr, flush=True)
            secondary[key] = time_backward(inp, dev, max(3, args.steps // 2), args.warmup, name)
            del inp
        if "value" not in result:
            first = secondary["t4k_backward"]
            result["value"] = first["tokens_per_s_per_layer"]
            result["ms_per_step"] = first["ms_per_call"]
            result["config"] = {"workload": first["workload"]}
    if args.only in ("all", "decode"):
        print("bench: decode step B256 H16 d128", file=sys.stderr, flush=True)
        secondary["decode"] = time_decode(dev, max(50, args.steps * 10), args.warmup * 5)
        print("bench: decode workload, 24 layers", file=sys.stderr, flush=True)
        secondary["decode_workload"] = time_decode_workload(dev, max(16, args.steps * 2), 2)
        if not args.no_cpu:
            print("bench: CPU oracle decode baseline", file=sys.stderr, flush=True)
            secondary["decode_workload"]["cpu_baseline"] = cpu_decode_baseline(dev)
        if "value" not in result:
            result["value"] = secondary["decode"]["GB_per_s"]
            result["unit"] = "GB/s"
            result["ms_per_step"] = secondary["decode"]["ms_per_call"]
            result["config"] = {"workload": secondary["decode"]["workload"]}
    result["secondary"] = secondary
    if main_inp is not None and not args.no_cpu:
        print("bench: CPU oracle baseline", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(main_inp)
        print("bench: sampled heads of the timed output against the oracle", file=sys.stderr,
              flush=True)
        result["parity"] = sampled_head_errors(main_inp, *main_out, heads=[0, 1, 15])
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
