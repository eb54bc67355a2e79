"""GPU parity of the shared-erase forward (muir_chunk_fwd_scalar_erase): one erase strength
per token and head, e [B,T,H]. Its result is the token recurrence's with e broadcast over
the value channels, so the fp64 oracle is called with exactly that broadcast. Same bar as
the channel-wise forward: per-head max relative error of o and of the final state <= 2e-2
(bf16 q/k/v), every value finite. Calls go through the C ABI via the Python binding."""
import numpy as np
import pytest
import torch

import gated_delta_rule_06_amd as muir
import oracle
import workloads
from parity import NAMES, o_err, s_err, to_device, to_numpy

pytestmark = pytest.mark.gpu

TOL = 2e-2


def with_scalar_erase(inp, es):
    """The inputs with the per-channel e replaced by es broadcast over the value channels."""
    out = dict(inp)
    out["e"] = np.ascontiguousarray(np.broadcast_to(es[..., None], inp["e"].shape), np.float32)
    return out


def gpu_fwd(inp, es, device, chunk, s0=None, workspace=None):
    t = to_device(inp, device, "bf16")
    t["e"] = torch.from_numpy(np.ascontiguousarray(es, np.float32)).to(device)
    s0t = None if s0 is None else torch.from_numpy(np.asarray(s0, np.float32)).to(device)
    o, s = muir.chunk_fwd_scalar_erase(*[t[n] for n in NAMES], s0=s0t, chunk=chunk,
                                       workspace=workspace)
    torch.cuda.synchronize()
    return to_numpy(o), to_numpy(s)


def ref_fwd(inp, es, s0=None):
    full = with_scalar_erase(inp, es)
    return oracle.recurrent(*[full[n] for n in NAMES], s0=s0)


def assert_parity(o, s, o_ref, s_ref, what, tol=TOL):
    eo, es = o_err(o, o_ref), s_err(s, s_ref)
    print(f"{what}: max head err o={eo.max():.3e} state={es.max():.3e}", flush=True)
    assert np.isfinite(o).all() and np.isfinite(s).all(), f"{what}: non-finite output"
    where = ""
    if eo.max() > tol:
        b, h = np.unravel_index(np.argmax(eo), eo.shape)
        diff = np.abs(o[b, :, h].astype(np.float64) - o_ref[b, :, h]).max(axis=-1)
        bad = np.nonzero(diff > tol * np.abs(o_ref[b, :, h]).max())[0]
        where = f" worst head (b={b}, h={h}): tokens {bad.min()}..{bad.max()} ({bad.size} rows)"
    assert max(eo.max(), es.max()) <= tol, (f"{what}: o err per head {np.round(eo, 6).tolist()}, "
                                            f"state err per head {np.round(es, 6).tolist()}{where}")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("chunk", [64, 128, 256])
@pytest.mark.parametrize("T", [1, 15, 64, 65, 300])
def test_small_shapes(device, d, chunk, T):
    """Several tiles and a ragged last chunk, with a non-zero initial state."""
    inp = workloads.chunk_inputs(0, B=2, T=T, H=2, d=d, qkv="bf16", seed=3000 + T)
    es = workloads.scalar_erase(2, T, 2, seed=3000 + T)
    s0 = (np.random.default_rng(T).standard_normal((2, 2, d, d)) * 0.3).astype(np.float32)
    o, s = gpu_fwd(inp, es, device, chunk, s0)
    assert_parity(o, s, *ref_fwd(inp, es, s0), f"scalar erase T={T} d={d} C={chunk}")


def test_config1_166m_shape(device):
    inp = workloads.chunk_inputs(1)
    es = workloads.scalar_erase(inp["B"], inp["T"], inp["H"], seed=1)
    o, s = gpu_fwd(inp, es, device, 64)
    assert_parity(o, s, *ref_fwd(inp, es), "scalar erase config1 C=64")


@pytest.fixture(scope="module")
def config2():
    inp = workloads.chunk_inputs(2)
    es = workloads.scalar_erase(inp["B"], inp["T"], inp["H"], seed=2)
    return inp, es, ref_fwd(inp, es)


@pytest.mark.parametrize("chunk", [128, 256])
def test_config2_134b_shape(device, config2, chunk):
    inp, es, (o_ref, s_ref) = config2
    o, s = gpu_fwd(inp, es, device, chunk)
    assert_parity(o, s, o_ref, s_ref, f"scalar erase config2 C={chunk}")


def test_config3_long_context_stress(device):
    """The long-context workload (T = 32768, C = 256, four fast-decay stress heads)."""
    inp = workloads.chunk_inputs(3)
    es = workloads.scalar_erase(inp["B"], inp["T"], inp["H"], seed=3)
    o, s = gpu_fwd(inp, es, device, 256)
    assert_parity(o, s, *ref_fwd(inp, es), "scalar erase config3 C=256")


def test_agrees_with_the_channel_wise_forward(device, config2):
    """The per-channel path fed the broadcast gate solves the same recurrence: both within
    the bar of each other too (a cross-check of two independent kernels, not a parity
    claim)."""
    inp, es, _ = config2
    o1, s1 = gpu_fwd(inp, es, device, 256)
    full = with_scalar_erase(inp, es)
    t = to_device(full, device, "bf16")
    o2, s2 = muir.chunk_fwd(*[t[n] for n in NAMES], chunk=256)
    torch.cuda.synchronize()
    assert_parity(o1, s1, to_numpy(o2), to_numpy(s2), "scalar vs channel-wise path")


@pytest.mark.parametrize("value", [0.0, 1.0])
def test_no_erase_and_full_erase(device, value):
    """Degenerate gates: e = 0 (gated linear attention, the system is the identity) and
    e = 1 (the whole prediction erased, the largest off-diagonal inverse entries)."""
    inp = workloads.chunk_inputs(0, B=2, T=300, H=2, d=128, qkv="bf16", seed=41)
    es = np.full((2, 300, 2), value, np.float32)
    o, s = gpu_fwd(inp, es, device, 256)
    assert_parity(o, s, *ref_fwd(inp, es), f"scalar erase e={value}")


@pytest.mark.parametrize("chunk", [64, 256])
def test_extreme_decays(device, chunk):
    """Decays of exactly 0, 1e-30 and 1 mixed into U(1e-3, 0.05) stress rows, and a run of
    a = 1 on one head: no product is ever divided, so every value stays finite."""
    inp = workloads.chunk_inputs(3, B=1, T=600, H=4, seed=43)
    a = inp["a"]
    pick = np.random.default_rng(44).uniform(size=a.shape)
    a[pick < 0.05] = 0.0
    a[(pick >= 0.05) & (pick < 0.1)] = 1e-30
    a[(pick >= 0.1) & (pick < 0.2)] = 1.0
    a[:, 100:140, 1, :] = 1.0
    es = workloads.scalar_erase(1, 600, 4, seed=43)
    o, s = gpu_fwd(inp, es, device, chunk)
    assert_parity(o, s, *ref_fwd(inp, es), f"scalar erase extreme decays C={chunk}")


def test_scan_entry_reuses_the_solved_workspace(device):
    """The scan alone, rerun on the workspace a full call left, reproduces it bit for bit
    (it writes only the chunk start states, the same ones each time)."""
    B, T, H, d, C = 2, 700, 3, 128, 256
    inp = workloads.chunk_inputs(0, B=B, T=T, H=H, d=d, qkv="bf16", seed=44)
    es = workloads.scalar_erase(B, T, H, seed=44)
    need = muir.chunk_fwd_scalar_erase_workspace_size(B, T, H, d, d, C)
    ws = torch.empty(need, dtype=torch.uint8, device=device)
    o1, s1 = gpu_fwd(inp, es, device, C, workspace=ws)
    o2 = torch.empty((B, T, H, d), dtype=torch.bfloat16, device=device)
    s2 = torch.empty((B, H, d, d), dtype=torch.float32, device=device)
    for _ in range(2):
        muir.chunk_fwd_scalar_erase_scan(B=B, T=T, H=H, d=d, chunk=C, workspace=ws, o=o2, s_out=s2)
    torch.cuda.synchronize()
    assert np.array_equal(to_numpy(o2), o1) and np.array_equal(to_numpy(s2), s1)


def test_three_phase_calls_equal_the_full_call(device):
    """prepare, solve and scan as separate calls give exactly the full call's result."""
    B, T, H, d, C = 1, 520, 2, 128, 128
    inp = workloads.chunk_inputs(0, B=B, T=T, H=H, d=d, qkv="bf16", seed=47)
    es = workloads.scalar_erase(B, T, H, seed=47)
    o1, s1 = gpu_fwd(inp, es, device, C)
    t = to_device(inp, device, "bf16")
    et = torch.from_numpy(es).to(device)
    ws = torch.empty(muir.chunk_fwd_scalar_erase_workspace_size(B, T, H, d, d, C),
                     dtype=torch.uint8, device=device)
    o2 = torch.empty_like(t["v"])
    s2 = torch.empty((B, H, d, d), dtype=torch.float32, device=device)
    muir.chunk_fwd_prepare(t["q"], t["k"], t["a"], t["g"], t["r"], chunk=C, workspace=ws)
    muir.chunk_fwd_scalar_erase_solve(t["v"], et, t["w"], chunk=C, workspace=ws)
    muir.chunk_fwd_scalar_erase_scan(B=B, T=T, H=H, d=d, chunk=C, workspace=ws, o=o2, s_out=s2)
    torch.cuda.synchronize()
    assert np.array_equal(to_numpy(o2), o1) and np.array_equal(to_numpy(s2), s1)


def test_split_sequence_and_empty_sequence(device):
    """Two calls carrying the state through s0 / s_out equal one call over the whole
    sequence to the bar; T = 0 copies s0 into s_out."""
    B, T, H, d = 1, 600, 2, 64
    inp = workloads.chunk_inputs(0, B=B, T=T, H=H, d=d, qkv="bf16", seed=45)
    es = workloads.scalar_erase(B, T, H, seed=45)
    o_ref, s_ref = ref_fwd(inp, es)
    cut = 250
    first = {n: (inp[n][:, :cut] if n != "r" else inp[n]) for n in NAMES}
    second = {n: (inp[n][:, cut:] if n != "r" else inp[n]) for n in NAMES}
    o1, s1 = gpu_fwd(first, es[:, :cut], device, 128)
    o2, s2 = gpu_fwd(second, es[:, cut:], device, 128, s0=s1)
    assert_parity(np.concatenate([o1, o2], axis=1), s2, o_ref, s_ref, "scalar erase split")

    empty = {n: (inp[n][:, :0] if n != "r" else inp[n]) for n in NAMES}
    s0 = (np.random.default_rng(5).standard_normal((B, H, d, d))).astype(np.float32)
    o0, s0_out = gpu_fwd(empty, np.zeros((B, 0, H), np.float32), device, 64, s0=s0)
    assert o0.shape == (B, 0, H, d) and np.array_equal(s0_out, s0)
