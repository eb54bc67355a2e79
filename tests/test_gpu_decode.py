"""GPU parity of muir_decode_step against the fp64 CPU oracle (token recurrence with the
state carried across calls), including the 24-layer x 1024-step decode workload on a
seeded sample of (sequence, layer, head) slots."""
import numpy as np
import pytest
import torch

import gated_delta_rule_06_amd as muir
import oracle
import workloads
from parity import NAMES, o_err, s_err, to_device, to_numpy

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}


@pytest.mark.parametrize("qkv", ["f32", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
def test_steps_carry_state(device, qkv, d):
    B, H, T = 3, 2, 20
    inp = workloads.chunk_inputs(0, B=B, T=T, H=H, d=d, qkv=qkv, seed=20 + d)
    s0 = (np.random.default_rng(d).standard_normal((B, H, d, d)) * 0.3).astype(np.float32)
    t = to_device(inp, device, qkv)
    state = torch.from_numpy(s0).to(device)
    outs = []
    for step in range(T):
        args = [t[n][:, step].contiguous() if n != "r" else t[n] for n in NAMES]
        outs.append(muir.decode_step(*args, state))
    torch.cuda.synchronize()
    o = np.stack([to_numpy(x) for x in outs], axis=1)
    o_ref, s_ref = oracle.recurrent(*[inp[n] for n in NAMES], s0=s0)
    eo, es = o_err(o, o_ref), s_err(to_numpy(state), s_ref)
    print(f"decode d={d} {qkv}: o={eo.max():.2e} state={es.max():.2e}", flush=True)
    assert eo.max() <= TOL[qkv] and es.max() <= TOL[qkv]


def test_decode_matches_chunk_forward(device):
    inp = workloads.chunk_inputs(2, B=2, T=90, H=2, seed=21)
    t = to_device(inp, device, "bf16")
    o_chunk, s_chunk = muir.chunk_fwd(*[t[n] for n in NAMES], chunk=64)
    state = torch.zeros_like(s_chunk)
    outs = [muir.decode_step(*[t[n][:, i].contiguous() if n != "r" else t[n] for n in NAMES],
                             state) for i in range(90)]
    torch.cuda.synchronize()
    o_dec = torch.stack(outs, dim=1)
    eo = o_err(to_numpy(o_dec), to_numpy(o_chunk))
    es = s_err(to_numpy(state), to_numpy(s_chunk))
    assert eo.max() <= 2e-2 and es.max() <= 2e-2


def test_decode_workload_sampled_slots(device):
    """24 layers x 16 heads x 256 sequences, 1024 steps: final state and last output on
    a seeded sample of 1024 (sequence, layer, head) slots against the fp64 oracle."""
    cfg = workloads.DECODE_CONFIG
    B, L, H, d, steps = cfg.B, cfg.L, cfg.H, cfg.d, cfg.steps
    u, r = workloads.decode_base(cfg)
    u_t = torch.from_numpy(u.astype(np.float32)).to(device)
    r_t = torch.from_numpy(r).to(device)
    states = [torch.zeros(B, H, d, d, device=device) for _ in range(L)]
    rng = np.random.default_rng(cfg.seed)
    nslot = 1024
    flat = rng.choice(B * L * H, size=nslot, replace=False)
    sb, sl, sh = flat // (L * H), (flat // H) % L, flat % H
    idx_b = torch.from_numpy(sb).to(device)
    idx_l = torch.from_numpy(sl).to(device)
    idx_h = torch.from_numpy(sh).to(device)
    hist = {n: np.empty((1, steps, nslot, d), np.float32) for n in NAMES if n != "r"}
    last_o = None
    for step in range(steps):
        x = workloads.decode_step_inputs_torch(step, u_t, device, B=B, cfg=cfg)
        outs = []
        for layer in range(L):
            args = [x[n][layer] for n in NAMES if n != "r"]
            outs.append(muir.decode_step(*args[:7], r_t[layer], states[layer]))
        for n in hist:
            hist[n][0, step] = x[n][idx_l, idx_b, idx_h].float().cpu().numpy()
        if step == steps - 1:
            last_o = torch.stack(outs)[idx_l, idx_b, idx_h].float().cpu().numpy()
        if step % 256 == 0:
            print(f"decode workload step {step}", flush=True)
    torch.cuda.synchronize()
    final = torch.stack(states)[idx_l, idx_b, idx_h].cpu().numpy()        # [nslot, d, d]
    assert np.isfinite(final).all() and np.isfinite(last_o).all()
    r_slots = r[sl, sh]                                                     # [nslot, d]
    o_ref, s_ref = oracle.recurrent(hist["q"], hist["k"], hist["v"], hist["a"], hist["g"],
                                    hist["e"], hist["w"], r_slots)
    es = s_err(final[None], s_ref)
    eo = o_err(last_o[None, None], o_ref[:, -1:])
    print(f"decode workload: state err max {es.max():.2e}, last o err max {eo.max():.2e}",
          flush=True)
    assert es.max() <= cfg.tol and eo.max() <= cfg.tol


def test_decode_is_deterministic(device):
    """The same steps from the same state give the same bits (no atomics in the reductions)."""
    B, H, d, T = 8, 16, 128, 6
    inp = workloads.chunk_inputs(2, B=B, T=T, H=H, d=d, qkv="bf16", seed=31)
    s0 = (np.random.default_rng(31).standard_normal((B, H, d, d)) * 0.3).astype(np.float32)
    t = to_device(inp, device, "bf16")
    runs = []
    for _ in range(2):
        state = torch.from_numpy(s0).to(device)
        outs = [muir.decode_step(*[t[n][:, i].contiguous() if n != "r" else t[n] for n in NAMES],
                                 state) for i in range(T)]
        torch.cuda.synchronize()
        runs.append((torch.stack(outs, 1).cpu(), state.cpu()))
    assert torch.equal(runs[0][0], runs[1][0]) and torch.equal(runs[0][1], runs[1][1])


def test_static_readout(device):
    """The static-readout setting (query gate g = 1 everywhere, so the read is r * q alone),
    the form the pages run at million-token passkey lengths: chunk forward at C = 256 and the
    decode step against the oracle."""
    inp = workloads.chunk_inputs(3, B=1, T=700, H=4, qkv="bf16", seed=32)
    inp["g"] = np.ones_like(inp["g"])
    t = to_device(inp, device, "bf16")
    o, s = muir.chunk_fwd(*[t[n] for n in NAMES], chunk=256)
    state = torch.zeros_like(s)
    outs = [muir.decode_step(*[t[n][:, i].contiguous() if n != "r" else t[n] for n in NAMES],
                             state) for i in range(64)]
    torch.cuda.synchronize()
    o_ref, s_ref = oracle.recurrent(*[inp[n] for n in NAMES])
    eo, es = o_err(to_numpy(o), o_ref), s_err(to_numpy(s), s_ref)
    print(f"static readout chunk: o={eo.max():.2e} state={es.max():.2e}", flush=True)
    assert eo.max() <= TOL["bf16"] and es.max() <= TOL["bf16"]
    o64, _ = oracle.recurrent(*[inp[n][:, :64] if n != "r" else inp[n] for n in NAMES])
    ed = o_err(np.stack([to_numpy(x) for x in outs], 1), o64)
    assert ed.max() <= TOL["bf16"]
