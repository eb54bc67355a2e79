"""GPU parity of the low-rank gate projection (muir_lowrank_gates) against the oracle's
definition (oracle/gates.py, fp64), and of the chunk forward driven by those gates against
the fp64 token recurrence.

Bars: the gates themselves are fp32 arithmetic on bf16-exact inputs, so they must match the
fp64 definition to 2e-6 absolute for the sigmoid gates and 1e-4 relative (plus 1e-7
absolute) for the decay, whose exp(-exp(y)) amplifies an error in y by exp(y). The forward
keeps the 2e-2 per-head bar of the bf16 chunk forward."""
import numpy as np
import pytest
import torch

import gated_delta_rule_06_amd as muir
import oracle
import workloads
from parity import NAMES, o_err, s_err, to_device, to_numpy

pytestmark = pytest.mark.gpu

GATE_NAMES = {"a": "decay", "e": "erase", "w": "write", "g": "read"}


def dev_weights(lr, device):
    U = {n: torch.from_numpy(lr["U_" + n]).to(device=device, dtype=torch.bfloat16)
         for n in ("decay", "erase", "write", "read")}
    c = {n: torch.from_numpy(lr["c_" + n]).to(device) for n in ("decay", "erase", "write", "read")}
    return U, c


def ref_gates(lr):
    return dict(zip("aewg", oracle.lowrank_gates(
        lr["z"], lr["U_decay"], lr["U_erase"], lr["U_write"], lr["U_read"],
        lr["c_decay"], lr["c_erase"], lr["c_write"], lr["c_read"])))


def gpu_gates(lr, H, d, device, which=("a", "e", "w", "g")):
    z = torch.from_numpy(lr["z"]).to(device=device, dtype=torch.bfloat16)
    U, c = dev_weights(lr, device)
    out = muir.lowrank_gates(z, U, c, H=H, d=d, which=which)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in out.items()}


def check_gates(got, ref, what):
    for k, x in got.items():
        r = ref[k]
        assert np.isfinite(x).all(), f"{what}: non-finite {k}"
        if k == "a":
            bad = np.abs(x - r) > 1e-4 * np.abs(r) + 1e-7
        else:
            bad = np.abs(x - r) > 2e-6
        print(f"{what} {k}: max abs err {np.abs(x - r).max():.2e}", flush=True)
        assert not bad.any(), f"{what}: gate {k} off at {np.argwhere(bad)[:5].tolist()}"


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("T", [1, 37, 300])
def test_gates_small(device, d, T):
    lr = workloads.lowrank_gate_inputs(0, B=2, T=T, H=3, d=d, seed=500 + T)
    check_gates(gpu_gates(lr, 3, d, device), ref_gates(lr), f"gates T={T} d={d}")


def test_gates_long_context_shape_sampled(device):
    """The long-context shape (stress heads included): every gate of the GPU call, checked
    on the first 1024 tokens and 1024 tokens drawn across the sequence."""
    lr = workloads.lowrank_gate_inputs(3)
    got = gpu_gates(lr, 16, 128, device)
    rng = np.random.default_rng(7)
    toks = np.unique(np.concatenate([np.arange(1024), rng.integers(0, 32768, 1024)]))
    sub = dict(lr)
    sub["z"] = lr["z"][:, toks]
    check_gates({k: v[:, toks] for k, v in got.items()}, ref_gates(sub), "gates long context")


def test_only_requested_gates_are_written(device):
    lr = workloads.lowrank_gate_inputs(0, B=1, T=50, H=2, d=64, seed=9)
    z = torch.from_numpy(lr["z"]).to(device=device, dtype=torch.bfloat16)
    U, c = dev_weights(lr, device)
    sentinel = {k: torch.full((1, 50, 2, 64), 7.0, device=device) for k in "aewg"}
    muir.lowrank_gates(z, U, c, H=2, d=64, which=("e",), out=sentinel)
    torch.cuda.synchronize()
    for k in "awg":
        assert bool((sentinel[k] == 7.0).all())
    check_gates({"e": sentinel["e"].cpu().numpy()}, ref_gates(lr), "only e")


@pytest.mark.parametrize("d,chunk", [(64, 64), (128, 256)])
def test_forward_driven_by_lowrank_gates(device, d, chunk):
    """The chunk forward on the GPU-made gates against the fp64 recurrence on the oracle's
    gates: the whole low-rank-gated layer."""
    B, T, H = 2, 300, 2
    inp = workloads.chunk_inputs(0, B=B, T=T, H=H, d=d, qkv="bf16", seed=600 + d)
    lr = workloads.lowrank_gate_inputs(0, B=B, T=T, H=H, d=d, seed=600 + d)
    ref = ref_gates(lr)
    full = dict(inp)
    for k in "aewg":
        full[k] = ref[k]
    o_ref, s_ref = oracle.recurrent(*[full[n] for n in NAMES])
    gates = gpu_gates(lr, H, d, device)
    t = to_device(inp, device, "bf16")
    for k in "aewg":
        t[k] = torch.from_numpy(gates[k]).to(device)
    o, s = muir.chunk_fwd(*[t[n] for n in NAMES], chunk=chunk)
    torch.cuda.synchronize()
    eo, es = o_err(to_numpy(o), o_ref), s_err(to_numpy(s), s_ref)
    print(f"low-rank forward d={d} C={chunk}: o={eo.max():.3e} state={es.max():.3e}", flush=True)
    assert max(eo.max(), es.max()) <= 2e-2


def lowrank_fwd(inp, lr, device, chunk, s0=None):
    t = to_device(inp, device, "bf16")
    z = torch.from_numpy(lr["z"]).to(device=device, dtype=torch.bfloat16)
    U, c = dev_weights(lr, device)
    s0t = None if s0 is None else torch.from_numpy(np.asarray(s0, np.float32)).to(device)
    o, s = muir.chunk_fwd_lowrank(t["q"], t["k"], t["v"], z, U, c, t["r"], s0t, chunk=chunk)
    torch.cuda.synchronize()
    return to_numpy(o), to_numpy(s)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("chunk", [64, 128, 256])
@pytest.mark.parametrize("T", [15, 300])
def test_fused_lowrank_forward_parity(device, d, chunk, T):
    """Gates made inside the call: against the fp64 recurrence on the oracle's gates."""
    B, H = 2, 2
    inp = workloads.chunk_inputs(0, B=B, T=T, H=H, d=d, qkv="bf16", seed=700 + T)
    lr = workloads.lowrank_gate_inputs(0, B=B, T=T, H=H, d=d, seed=700 + T)
    ref = ref_gates(lr)
    full = dict(inp)
    for k in "aewg":
        full[k] = ref[k]
    o_ref, s_ref = oracle.recurrent(*[full[n] for n in NAMES])
    o, s = lowrank_fwd(inp, lr, device, chunk)
    eo, es = o_err(o, o_ref), s_err(s, s_ref)
    print(f"fused low-rank T={T} d={d} C={chunk}: o={eo.max():.3e} state={es.max():.3e}", flush=True)
    assert np.isfinite(o).all() and np.isfinite(s).all()
    assert max(eo.max(), es.max()) <= 2e-2


@pytest.mark.parametrize("d,B,chunk", [(128, 2, 128), (64, 4, 64)])
def test_gates_made_inside_the_scan_parity(device, d, B, chunk):
    """B*H*d/8 = 512 runs 16-column tiles, where e and w are made inside the scan (chunk <=
    128): against the fp64 recurrence on the oracle's gates, with a ragged tail and a
    non-zero initial state."""
    H, T = 16, 300
    inp = workloads.chunk_inputs(0, B=B, T=T, H=H, d=d, qkv="bf16", seed=760 + d)
    lr = workloads.lowrank_gate_inputs(0, B=B, T=T, H=H, d=d, seed=760 + d)
    s0 = (np.random.default_rng(760 + d).standard_normal((B, H, d, d)) * 0.3).astype(np.float32)
    ref = ref_gates(lr)
    full = dict(inp)
    for k in "aewg":
        full[k] = ref[k]
    o_ref, s_ref = oracle.recurrent(*[full[n] for n in NAMES], s0=s0)
    o, s = lowrank_fwd(inp, lr, device, chunk, s0)
    eo, es = o_err(o, o_ref), s_err(s, s_ref)
    print(f"gates in the scan d={d} C={chunk}: o={eo.max():.3e} state={es.max():.3e}", flush=True)
    assert np.isfinite(o).all() and np.isfinite(s).all()
    assert max(eo.max(), es.max()) <= 2e-2


@pytest.mark.parametrize("cfg,chunk", [(2, 128), (2, 256), (3, 256)])
def test_fused_equals_gate_kernel_then_forward(device, cfg, chunk):
    """At the 1.34B-class and long-context shapes: the fused call is bit for bit the gate
    kernel's four gates fed to the plain forward (same products, same order). The cases
    cover e and w made inside the scan (16-column tiles, C=128) and made by the gate kernel
    first (16-column tiles at C=256, 8-column tiles on the long-context shape)."""
    inp = workloads.chunk_inputs(cfg)
    lr = workloads.lowrank_gate_inputs(cfg)
    B, T, H, d = inp["B"], inp["T"], inp["H"], inp["d"]
    o1, s1 = lowrank_fwd(inp, lr, device, chunk)
    gates = gpu_gates(lr, H, d, device)
    t = to_device(inp, device, "bf16")
    for k in "aewg":
        t[k] = torch.from_numpy(gates[k]).to(device)
    o2, s2 = muir.chunk_fwd(*[t[n] for n in NAMES], chunk=chunk)
    torch.cuda.synchronize()
    assert np.array_equal(o1, to_numpy(o2)) and np.array_equal(s1, to_numpy(s2))


@pytest.mark.parametrize("B,T,H,d,chunk", [(1, 300, 2, 128, 256), (2, 77, 3, 64, 64), (1, 15, 4, 128, 128)])
def test_fused_packed_gates_ragged_tail(device, B, T, H, d, chunk):
    """Few heads (one 8-column scan workgroup per compute unit at most), so the gate kernel
    stores e and w tile-packed and the split scan reads them so; with a ragged tail (rows past
    T read zero) and a non-zero initial state the fused call is still bit for bit the gate
    kernel's four gates, stored as [B, T, H, d], fed to the plain forward."""
    inp = workloads.chunk_inputs(1, B=B, T=T, H=H, d=d, qkv="bf16", seed=800 + T)
    lr = workloads.lowrank_gate_inputs(1, B=B, T=T, H=H, d=d, seed=800 + T)
    s0 = (np.random.default_rng(T).standard_normal((B, H, d, d)) * 0.3).astype(np.float32)
    print(f"packed gates B{B} T{T} H{H} d{d} C{chunk}", flush=True)
    o1, s1 = lowrank_fwd(inp, lr, device, chunk, s0)
    gates = gpu_gates(lr, H, d, device)
    t = to_device(inp, device, "bf16")
    for k in "aewg":
        t[k] = torch.from_numpy(gates[k]).to(device)
    o2, s2 = muir.chunk_fwd(*[t[n] for n in NAMES], s0=torch.from_numpy(s0).to(device), chunk=chunk)
    torch.cuda.synchronize()
    assert np.array_equal(o1, to_numpy(o2)) and np.array_equal(s1, to_numpy(s2))


# ---- The output gate from z's output slice (rank 128, z[..., 128:256]) ----

def gpu_output_gate(lr, device):
    z = torch.from_numpy(lr["z"]).to(device=device, dtype=torch.bfloat16)
    Uo = torch.from_numpy(lr["U_output"]).to(device=device, dtype=torch.bfloat16)
    co = torch.from_numpy(lr["c_output"]).to(device)
    og = muir.lowrank_output_gate(z, Uo, co)
    torch.cuda.synchronize()
    return og.cpu().numpy()


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("T", [1, 37, 300])
def test_output_gate_small(device, d, T):
    """og = sigmoid(z[..., 128:256] U_o^T + c_o) against the oracle, to the sigmoid gates'
    2e-6 absolute bar."""
    lr = workloads.lowrank_gate_inputs(0, B=2, T=T, H=3, d=d, seed=800 + T)
    got = gpu_output_gate(lr, device)
    ref = oracle.output_gate(lr["z"], lr["U_output"], lr["c_output"])
    check_gates({"og": got}, {"og": ref}, f"output gate T={T} d={d}")


def test_output_gate_long_context_shape_sampled(device):
    """The long-context shape (B1 T32768 H16 d128): sampled token rows against the oracle."""
    lr = workloads.lowrank_gate_inputs(3)
    got = gpu_output_gate(lr, device)
    rows = np.array([0, 1, 15, 16, 255, 256, 4095, 16384, 32766, 32767])
    ref = oracle.output_gate(lr["z"][:, rows], lr["U_output"], lr["c_output"])
    check_gates({"og": got[:, rows]}, {"og": ref}, "output gate long context")
    assert np.isfinite(got).all() and ((got > 0) & (got < 1)).all()


def dev_weights5(lr, device):
    U, c = dev_weights(lr, device)
    U["output"] = torch.from_numpy(lr["U_output"]).to(device=device, dtype=torch.bfloat16)
    c["output"] = torch.from_numpy(lr["c_output"]).to(device)
    return U, c


def lowrank_gated_fwd(inp, lr, device, chunk, s0=None):
    t = to_device(inp, device, "bf16")
    z = torch.from_numpy(lr["z"]).to(device=device, dtype=torch.bfloat16)
    U, c = dev_weights5(lr, device)
    s0t = None if s0 is None else torch.from_numpy(np.asarray(s0, np.float32)).to(device)
    o, s = muir.chunk_fwd_lowrank_gated(t["q"], t["k"], t["v"], z, U, c, t["r"], s0t, chunk=chunk)
    torch.cuda.synchronize()
    return to_numpy(o), to_numpy(s)


def ref_gated(inp, lr, s0=None):
    ref = ref_gates(lr)
    full = dict(inp)
    for k in "aewg":
        full[k] = ref[k]
    o_ref, s_ref = oracle.recurrent(*[full[n] for n in NAMES], s0=s0)
    return o_ref * oracle.output_gate(lr["z"], lr["U_output"], lr["c_output"]), s_ref


@pytest.mark.parametrize("d,B,H,chunk", [(64, 2, 2, 64), (128, 2, 2, 256), (128, 2, 16, 128),
                                         (64, 4, 16, 64)])
@pytest.mark.parametrize("T", [15, 300])
def test_fused_lowrank_gated_parity(device, d, B, H, chunk, T):
    """All five gates made inside the call: the stored output against the fp64 recurrence on
    the oracle's four gates times the oracle's output gate, with a non-zero initial state.
    The 16-head cases (B*H*d/8 = 512, chunk <= 128) form og in the scan's gate wavefront;
    the others take it from the gate kernel."""
    inp = workloads.chunk_inputs(0, B=B, T=T, H=H, d=d, qkv="bf16", seed=900 + T + d)
    lr = workloads.lowrank_gate_inputs(0, B=B, T=T, H=H, d=d, seed=900 + T + d)
    s0 = (np.random.default_rng(900 + T).standard_normal((B, H, d, d)) * 0.3).astype(np.float32)
    o, s = lowrank_gated_fwd(inp, lr, device, chunk, s0)
    o_ref, s_ref = ref_gated(inp, lr, s0)
    eo, es = o_err(o, o_ref), s_err(s, s_ref)
    print(f"fused gated T={T} d={d} H={H} C={chunk}: o={eo.max():.3e} state={es.max():.3e}", flush=True)
    assert np.isfinite(o).all() and np.isfinite(s).all()
    assert max(eo.max(), es.max()) <= 2e-2


@pytest.mark.parametrize("cfg,chunk", [(2, 128), (2, 256), (3, 256)])
def test_fused_gated_equals_gate_kernels_then_gated_forward(device, cfg, chunk):
    """The fused gated call is bit for bit the gate kernel's gates and output gate fed to
    the output-gated forward: og made in the scan's gate wavefront (C=128), by the gate
    kernel with 16-column tiles (C=256), and on the long-context shape's split scan."""
    inp = workloads.chunk_inputs(cfg)
    lr = workloads.lowrank_gate_inputs(cfg)
    B, T, H, d = inp["B"], inp["T"], inp["H"], inp["d"]
    o1, s1 = lowrank_gated_fwd(inp, lr, device, chunk)
    gates = gpu_gates(lr, H, d, device)
    og = torch.from_numpy(gpu_output_gate(lr, device)).to(device)
    t = to_device(inp, device, "bf16")
    for k in "aewg":
        t[k] = torch.from_numpy(gates[k]).to(device)
    o2, s2 = muir.chunk_fwd(*[t[n] for n in NAMES], chunk=chunk, og=og)
    torch.cuda.synchronize()
    assert np.array_equal(o1, to_numpy(o2)) and np.array_equal(s1, to_numpy(s2))
