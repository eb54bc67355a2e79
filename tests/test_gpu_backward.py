"""GPU parity of muir_chunk_bwd against the fp64 backward oracle (token adjoint recurrence,
itself pinned against autograd, finite differences and closed forms on the CPU).

Bar: per-head max relative error (max |x - ref| / max |ref| over the head's slice) of every
gradient <= 1e-5 for fp32 q/k/v and <= 2e-2 for bf16, with every value finite. Why these
bounds: on the fp32 path the backward's arithmetic is fp32 throughout (about 1e-6 measured).
The bf16 path starts from the forward's u, formed with bf16 matrix-core operands (relative
error about 2^-8 per operand; the forward's own bar is 2e-2), and its reverse scan multiplies
K*beta, P, Q_hat*gamma and K*gamma as bf16 operands (the adjoint and dP as exact hi + lo
pairs). Measured, the largest error is 1.4e-2, the log-decay gradient of the long-context
shape (a cumulative sum over the sequence); it is the same with fp32 scan operands, so it
comes from u. The scan's bf16 operands bring dv, dw, de and ds0 from about 1e-6 to at most
5e-3.
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
    """fp64 oracle gradients, from the C token adjoint (pinned against autograd and finite
    differences on the CPU); optionally of a subset of heads, which is exact: heads are
    independent and dr is summed per head."""
    sl = (lambda x: x) if heads is None else (lambda x: x[:, :, heads])
    args = [sl(np.asarray(inp[n], np.float64)) for n in ("q", "k", "v", "a", "g", "e", "w")]
    r = np.asarray(inp["r"], np.float64)
    r = r if heads is None else r[heads]
    B, T, H, d = args[0].shape
    s0_ = None if s0 is None else (s0 if heads is None else s0[:, heads])
    dS_ = np.zeros((B, H, d, d)) if dS is None else (dS if heads is None else dS[:, heads])
    return obw.grads_c(*args, r, s0_, sl(do), dS_)


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
    """Enough heads (B * H * d / 8 > 256) that the forward scan the backward reruns (the saving
    instance) is the two-wavefront scan with 16-column value tiles on the bf16 path; the smaller
    bf16 cases here rerun it on the split scan (8-column tiles, four wavefronts). The reverse scan
    itself runs 16-column tiles in every case; what this case adds to it is H = 16 heads per
    batch row, two full groups of eight."""
    T, H = 130, 16
    inp = workloads.chunk_inputs(0, B=B, T=T, H=H, d=d, qkv=qkv, seed=3000 + d)
    rng = np.random.default_rng(d)
    s0 = (rng.standard_normal((B, H, d, d)) * 0.3).astype(np.float32)
    do, dS = _cotangents(rng, B, T, H, d, qkv, with_ds=True)
    got = gpu_bwd(inp, device, s0, do, dS, qkv)
    ref = ref_bwd(inp, s0, do, dS)
    assert_grad_parity(got, ref, TOL[qkv], f"B={B} H={H} T={T} d={d} {qkv} (16-column forward tiles)")


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


def test_one_row_t4096_sampled_heads(device):
    """One batch row of the 1.34B-class shape (B=1, T=4096, H=16, d=128, bf16) with an initial
    state, run whole on the GPU; the first and last heads against the oracle."""
    B, T, H, d = 1, 4096, 16, 128
    inp = workloads.chunk_inputs(0, B=B, T=T, H=H, d=d, qkv="bf16", seed=4242)
    rng = np.random.default_rng(4242)
    s0 = (rng.standard_normal((B, H, d, d)) * 0.3).astype(np.float32)
    do, dS = _cotangents(rng, B, T, H, d, "bf16", with_ds=True)
    got = gpu_bwd(inp, device, s0, do, dS, "bf16")
    heads = [0, H - 1]
    ref = ref_bwd(inp, s0, do, dS, heads=heads)
    assert_grad_parity(got, ref, TOL["bf16"], "T=4096 H=16 d=128 bf16 heads 0,15", heads=heads)


def _extreme_decays(a, seed):
    """Decays of exactly 0, 1e-30 and 1 mixed into the given ones, plus a run of 40 tokens at
    a = 1 on head 1 (the same mix as the forward's extreme-decay test)."""
    rng = np.random.default_rng(seed)
    pick = rng.uniform(size=a.shape)
    a = a.copy()
    a[pick < 0.05] = 0.0
    a[(pick >= 0.05) & (pick < 0.1)] = 1e-30
    a[(pick >= 0.1) & (pick < 0.2)] = 1.0
    a[:, 100:140, 1, :] = 1.0
    return a


@pytest.mark.parametrize("qkv", ["f32", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
def test_stress_and_extreme_decays(device, qkv, d):
    """Long-context stress inputs (heads 0 mod 4 with a ~ U(1e-3, 0.05) per token and row, the
    others with half-lives up to 1e5 tokens) with exact zeros, 1e-30 and ones mixed in. Every
    pivot of the backward (16-token blocks, 4-token sub-blocks, their halves) and the reverse
    cumulative sum of the log-decay gradient meet products that underflow or vanish; every
    gradient, la included, must stay finite and on the oracle."""
    B, T, H = 1, 300, 4
    inp = workloads.chunk_inputs(3, B=B, T=T, H=H, d=d, qkv=qkv, seed=5100 + d)
    inp["a"] = _extreme_decays(inp["a"], 5200 + d)
    rng = np.random.default_rng(5300 + d)
    s0 = (rng.standard_normal((B, H, d, d)) * 0.3).astype(np.float32)
    do, dS = _cotangents(rng, B, T, H, d, qkv, with_ds=True)
    got = gpu_bwd(inp, device, s0, do, dS, qkv)
    ref = ref_bwd(inp, s0, do, dS)
    assert_grad_parity(got, ref, TOL[qkv], f"stress + extreme decays T={T} d={d} {qkv}")


def test_heads_that_forget_everything(device):
    """Every decay of head 2 exactly zero (each token sees only its own write) and of head 3
    at 1e-30, next to a stress head and an ordinary one, on the fp32 path (bar 1e-5). On heads
    2 and 3 the log-decay gradient a * dL/da is zero or about 1e-30 times the others, so a
    per-head relative error is undefined there: la is held to the bar relative to its largest
    value over the whole call instead; every other gradient per head as usual."""
    B, T, H, d = 1, 200, 4, 64
    inp = workloads.chunk_inputs(3, B=B, T=T, H=H, d=d, qkv="f32", seed=5400)
    inp["a"][:, :, 2] = 0.0
    inp["a"][:, :, 3] = 1e-30
    rng = np.random.default_rng(5401)
    do, dS = _cotangents(rng, B, T, H, d, "f32", with_ds=True)
    got = gpu_bwd(inp, device, None, do, dS, "f32")
    ref = ref_bwd(inp, None, do, dS)
    for n, x in got.items():
        assert np.isfinite(x).all(), f"non-finite d{n}"
    la_err = np.abs(got["la"] - ref["la"]).max() / np.abs(ref["la"]).max()
    print(f"la error relative to the call's largest la: {la_err:.2e}; "
          f"largest |la| on the a = 0 head {np.abs(got['la'][:, :, 2]).max():.2e}", flush=True)
    assert la_err <= TOL["f32"]
    got_rest = dict(got, la=ref["la"])
    assert_grad_parity(got_rest, ref, TOL["f32"], "a = 0 and 1e-30 heads fp32 (la above)")


def test_long_context_shape_sampled_heads(device):
    """The long-context backward shape, B=1 H=16 d=128 T=32768 bf16 with the stress heads
    (0 mod 4), run whole on the GPU: heads 0 (stress), 1 and 15 against the oracle over the
    whole sequence, every gradient finite on every head."""
    B, T, H, d = 1, 32768, 16, 128
    inp = workloads.chunk_inputs(3, B=B, T=T, H=H, d=d, qkv="bf16", seed=3)
    rng = np.random.default_rng(5500)
    do, dS = _cotangents(rng, B, T, H, d, "bf16", with_ds=True)
    got = gpu_bwd(inp, device, None, do, dS, "bf16")
    heads = [0, 1, 15]
    ref = ref_bwd(inp, None, do, dS, heads=heads)
    assert_grad_parity(got, ref, TOL["bf16"], "T=32768 H=16 d=128 bf16 heads 0,1,15", heads=heads)


def test_batch8_shape_sampled_heads(device):
    """The 1.34B-class backward shape, B=8 H=16 d=128 T=4096 bf16 (the one the bench times),
    run whole on the GPU: heads 0 and 15 of every batch row against the oracle (dr of those
    heads summed over all eight rows), every gradient finite everywhere."""
    B, T, H, d = 8, 4096, 16, 128
    inp = workloads.chunk_inputs(2, B=B, T=T, H=H, d=d, qkv="bf16", seed=2)
    rng = np.random.default_rng(5600)
    s0 = (rng.standard_normal((B, H, d, d)) * 0.3).astype(np.float32)
    do, dS = _cotangents(rng, B, T, H, d, "bf16", with_ds=True)
    got = gpu_bwd(inp, device, s0, do, dS, "bf16")
    heads = [0, 15]
    ref = ref_bwd(inp, s0, do, dS, heads=heads)
    assert_grad_parity(got, ref, TOL["bf16"], "B=8 T=4096 H=16 d=128 bf16 heads 0,15", heads=heads)


def test_deterministic(device):
    """Two identical backward calls give the same bits (no atomics in any reduction)."""
    B, T, H, d = 2, 333, 4, 128
    inp = workloads.chunk_inputs(3, B=B, T=T, H=H, d=d, qkv="bf16", seed=5700)
    rng = np.random.default_rng(5701)
    s0 = (rng.standard_normal((B, H, d, d)) * 0.3).astype(np.float32)
    do, dS = _cotangents(rng, B, T, H, d, "bf16", with_ds=True)
    g1 = gpu_bwd(inp, device, s0, do, dS, "bf16")
    g2 = gpu_bwd(inp, device, s0, do, dS, "bf16")
    for n in g1:
        assert np.array_equal(g1[n], g2[n]), f"d{n} differs between runs"
