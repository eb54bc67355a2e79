"""GPU parity of the output-gate epilogue (muir_chunk_fwd_gated): the stored output is
o * og elementwise, o being the readout of the token recurrence, and the state is the
ungated one. Compared with the fp64 oracle's o times og, to the same per-head bar as the
ungated forward; og = 1 must reproduce the ungated call bit for bit and og = 0 must give
exact zeros."""
import numpy as np
import pytest
import torch

import gated_delta_rule_06_amd as muir
import oracle
import workloads
from parity import NAMES, o_err, s_err, to_device, to_numpy

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}


def run(inp, device, chunk, og=None, s0=None):
    t = to_device(inp, device, inp["qkv"])
    ogt = None if og is None else torch.from_numpy(np.asarray(og, np.float32)).to(device)
    s0t = None if s0 is None else torch.from_numpy(np.asarray(s0, np.float32)).to(device)
    o, s = muir.chunk_fwd(*[t[n] for n in NAMES], s0=s0t, chunk=chunk, og=ogt)
    torch.cuda.synchronize()
    return to_numpy(o), to_numpy(s)


@pytest.mark.parametrize("qkv", ["f32", "bf16"])
@pytest.mark.parametrize("d,chunk", [(64, 64), (128, 128), (128, 256)])
@pytest.mark.parametrize("T", [37, 300])
def test_output_gate_parity(device, qkv, d, chunk, T):
    inp = workloads.chunk_inputs(0, B=2, T=T, H=2, d=d, qkv=qkv, seed=2000 + T)
    og = workloads.output_gate(2, T, 2, d, seed=2000 + T)
    s0 = (np.random.default_rng(T).standard_normal((2, 2, d, d)) * 0.3).astype(np.float32)
    o, s = run(inp, device, chunk, og, s0)
    o_ref, s_ref = oracle.recurrent(*[inp[n] for n in NAMES], s0=s0)
    eo, es = o_err(o, o_ref * og), s_err(s, s_ref)
    print(f"gated T={T} d={d} C={chunk} {qkv}: o={eo.max():.3e} state={es.max():.3e}", flush=True)
    assert np.isfinite(o).all() and np.isfinite(s).all()
    assert max(eo.max(), es.max()) <= TOL[qkv]


@pytest.mark.parametrize("qkv", ["f32", "bf16"])
def test_output_gate_one_is_the_ungated_forward(device, qkv):
    inp = workloads.chunk_inputs(0, B=1, T=200, H=3, d=128, qkv=qkv, seed=31)
    o1, s1 = run(inp, device, 128)
    og, sg = run(inp, device, 128, og=np.ones((1, 200, 3, 128), np.float32))
    assert np.array_equal(o1, og) and np.array_equal(s1, sg)


def test_output_gate_zero_gives_zero_output_and_the_same_state(device):
    inp = workloads.chunk_inputs(0, B=1, T=130, H=2, d=64, qkv="bf16", seed=32)
    _, s1 = run(inp, device, 64)
    o0, s0 = run(inp, device, 64, og=np.zeros((1, 130, 2, 64), np.float32))
    assert not o0.any() and np.array_equal(s1, s0)
