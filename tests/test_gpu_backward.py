"""GPU parity of muir_chunk_bwd against the fp64 backward oracle (token adjoint recurrence,
itself pinned against autograd, finite differences and closed forms on the CPU).

Bar: per-head max relative error (max |x - ref| / max |ref| over the head's slice) of every
gradient <= 1e-5 for fp32 q/k/v and <= 2e-2 for bf16, with every value finite. Why these
bounds: the backward's own arithmetic is fp32 throughout (about 1e-6 measured), but it starts
from the forward's u, which the bf16 path forms with bf16 matrix-core operands (relative
error about 2^-8 per operand; the forward's own bar is 2e-2). The gradients are sums of
products of u with fp32 terms and inherit that error; measured, at most 5.3e-3 (the
log-decay gradient, a cumulative sum).
Calls go through the C ABI via the Python binding.
"""
import numpy as np
import pytest
import torch

import gated_delta_rule_06_amd as muir
import workloads
from oracle import backward as obw
from parity import NAMES, o_err, s_err, to_device, to_numpy

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "bf16": 2e-2}
TOKEN_GRADS = ("q", "k", "v", "la", "g", "e", "w")


def _cotangents(rng, B, T, H, d, qkv, with_ds):
    do = rng.standard_normal((B, T, H, d)).astype(np.float32)
    if qkv == "bf16":
        do = workloads.round_bf16(do)
    dS = (rng.standard_normal((B, H, d, d)) * 0.3).astype(np.float32) if with_ds else None
    return do, dS


def gpu_bwd(inp, device, s0, do, dS, qkv):
    t = to_device(inp, device, qkv)
    qdt = torch.bfloat16 if qkv == "bf16" else torch.float32
    s0t = None if s0 is None else torch.from_numpy(s0).to(device)
    dst = None if dS is None else torch.from_numpy(dS).to(device)
    dot = torch.from_numpy(do).to(device=device, dtype=qdt)
    out = muir.chunk_bwd(*[t[n] for n in NAMES], s0=s0t, do=dot, ds_out=dst, chunk=64)
    torch.cuda.synchronize()
    return {n: to_numpy(x) for n, x in out.items()}


def ref_bwd(inp, s0, do, dS, heads=None):
    """fp64 oracle gradients (optionally of a subset of heads, which is exact: heads are
    independent and dr is per head)."""
    sl = (lambda x: x) if heads is None else (lambda x: x[:, :, heads])
    args = [sl(np.asarray(inp[n], np.float64)) for n in ("q", "k", "v", "a", "g", "e", "w")]
    r = np.asarray(inp["r"], np.float64)
    r = r if heads is None else r[heads]
    B, T, H, d = args[0].shape
    s0_ = None if s0 is None else (s0 if heads is None else s0[:, heads])
    dS_ = np.zeros((B, H, d, d)) if dS is None else (dS if heads is None else dS[:, heads])
    return obw.grads_adjoint(*args, r, s0_, sl(do), dS_)


def assert_grad_parity(got, ref, tol, what, heads=None):
    sl = (lambda x: x) if heads is None else (lambda x: x[:, :, heads])
    errs = {}
    for n in TOKEN_GRADS:
        errs[n] = o_err(sl(got[n]), ref[n]).max()
    g_r = got["r"] if heads is None else got["r"][heads]
    errs["r"] = float((np.abs(g_r - ref["r"]).max(axis=1) / np.maximum(np.abs(ref["r"]).max(axis=1), 1e-300)).max())
    g_s = got["s0"] if heads is None else got["s0"][:, heads]
    errs["s0"] = s_err(g_s, ref["s0"]).max()
    print(f"{what}: " + " ".join(f"d{n}={e:.2e}" for n, e in errs.items()), flush=True)
    for n, x in got.items():
        assert np.isfinite(x).all(), f"{what}: non-finite d{n}"
    bad = {n: e for n, e in errs.items() if not e <= tol}
    assert not bad, f"{what}: over {tol}: {bad}"


@pytest.mark.parametrize("qkv", ["f32", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("T", [1, 15, 64, 65, 200])
def test_small_shapes(device, qkv, d, T):
    """One token, a partial block, an exact chunk, one token past it, several chunks with a
    ragged tail; with and without an initial state and a final-state cotangent."""
    B, H = 2, 2
    inp = workloads.chunk_inputs(0, B=B, T=T, H=H, d=d, qkv=qkv, seed=2000 + T)
    rng = np.random.default_rng(T + d)
    s0 = (rng.standard_normal((B, H, d, d)) * 0.3).astype(np.float32) if T % 2 else None
    do, dS = _cotangents(rng, B, T, H, d, qkv, with_ds=(T % 3 != 0))
    got = gpu_bwd(inp, device, s0, do, dS, qkv)
    ref = ref_bwd(inp, s0, do, dS)
    assert_grad_parity(got, ref, TOL[qkv], f"T={T} d={d} {qkv}")


@pytest.mark.parametrize("qkv", ["f32", "bf16"])
@pytest.mark.parametrize("B,d", [(2, 128), (4, 64)])
def test_wide_scan_tiles(device, qkv, B, d):
    """Enough heads (B * H * d / 16 >= 256) for the reverse scan's 16-column tiles; the other
    cases here run its 8-column tiles."""
    T, H = 130, 16
    inp = workloads.chunk_inputs(0, B=B, T=T, H=H, d=d, qkv=qkv, seed=3000 + d)
    rng = np.random.default_rng(d)
    s0 = (rng.standard_normal((B, H, d, d)) * 0.3).astype(np.float32)
    do, dS = _cotangents(rng, B, T, H, d, qkv, with_ds=True)
    got = gpu_bwd(inp, device, s0, do, dS, qkv)
    ref = ref_bwd(inp, s0, do, dS)
    assert_grad_parity(got, ref, TOL[qkv], f"B={B} H={H} T={T} d={d} {qkv} (16-column scan tiles)")


def test_zero_length(device):
    """T = 0: the initial state's gradient is the final state's cotangent; dr is zero."""
    B, H, d = 2, 3, 64
    inp = workloads.chunk_inputs(0, B=B, T=1, H=H, d=d, qkv="f32", seed=7)
    t = to_device(inp, device, "f32")
    empty = {n: x[:, :0].contiguous() for n, x in t.items() if n != "r"}
    dS = torch.randn(B, H, d, d, device=device)
    out = muir.chunk_bwd(*[empty[n] if n != "r" else t["r"] for n in NAMES], s0=None,
                         do=empty["v"], ds_out=dS, chunk=64)
    torch.cuda.synchronize()
    assert torch.equal(out["s0"], dS)
    assert torch.count_nonzero(out["r"]).item() == 0


def test_errors(device):
    inp = workloads.chunk_inputs(0, B=1, T=8, H=1, d=64, qkv="f32", seed=8)
    t = to_device(inp, device, "f32")
    do = torch.zeros_like(t["v"])
    with pytest.raises(muir.MuirError, match="UNSUPPORTED"):
        muir.chunk_bwd(*[t[n] for n in NAMES], do=do, chunk=128)
    with pytest.raises(muir.MuirError, match="ALIAS"):
        muir.chunk_bwd(*[t[n] for n in NAMES], do=do, out={"q": t["a"]})


def test_long_context_sampled_heads(device):
    """The long-context shape (B=1, T=4096, H=16, d=128, bf16), run whole on the GPU; the
    first and last heads against the oracle."""
    B, T, H, d = 1, 4096, 16, 128
    inp = workloads.chunk_inputs(0, B=B, T=T, H=H, d=d, qkv="bf16", seed=4242)
    rng = np.random.default_rng(4242)
    s0 = (rng.standard_normal((B, H, d, d)) * 0.3).astype(np.float32)
    do, dS = _cotangents(rng, B, T, H, d, "bf16", with_ds=True)
    got = gpu_bwd(inp, device, s0, do, dS, "bf16")
    heads = [0, H - 1]
    ref = ref_bwd(inp, s0, do, dS, heads=heads)
    assert_grad_parity(got, ref, TOL["bf16"], "T=4096 H=16 d=128 bf16 heads 0,15", heads=heads)
