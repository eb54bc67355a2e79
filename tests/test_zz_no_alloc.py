"""muir_chunk_fwd_noalloc (the chunk forward whose workspace is the library's static device
scratch) against muir_chunk_fwd with a caller-given workspace: the same kernels on the same
inputs, so the same bits. Two calls in a row, the second smaller than the first, so the second
runs on scratch that still holds the first call's data. Called through the C ABI."""
import ctypes

import numpy as np
import pytest
import torch

import gated_delta_rule_06_amd as muir
import workloads
from parity import NAMES, to_device

pytestmark = pytest.mark.gpu


def _noalloc(t, s0, B, T, H, d, chunk):
    o = torch.empty_like(t["v"])
    s_out = torch.empty(B, H, d, d, dtype=torch.float32, device=t["v"].device)
    p = lambda x: ctypes.c_void_p(x.data_ptr()) if x is not None else None
    st = muir.lib().muir_chunk_fwd_noalloc(
        *[p(t[n]) for n in NAMES], p(s0), p(o), p(s_out), B, T, H, d, d, chunk, muir.MUIR_BF16,
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, muir.last_error()
    return o, s_out


def test_noalloc_matches_the_workspace_call_twice(device):
    cases = [
        # 16 heads x 16 chunks of 256 tokens at d = 128: 113 MiB of the 128 MiB scratch.
        dict(cfg=2, B=1, T=4096, H=16, d=128, chunk=256, seed=71, s0=False),
        # Smaller, ragged, with an initial state: runs on the first call's leftovers.
        dict(cfg=1, B=2, T=300, H=3, d=64, chunk=64, seed=72, s0=True),
    ]
    limit = muir.lib().muir_chunk_fwd_noalloc_max_workspace()
    for c in cases:
        B, T, H, d, chunk = c["B"], c["T"], c["H"], c["d"], c["chunk"]
        assert muir.chunk_fwd_workspace_size(B, T, H, d, d, chunk, muir.MUIR_BF16) <= limit
        inp = workloads.chunk_inputs(c["cfg"], B=B, T=T, H=H, d=d, qkv="bf16", seed=c["seed"])
        t = to_device(inp, device, "bf16")
        s0 = None
        if c["s0"]:
            s0 = torch.from_numpy((np.random.default_rng(c["seed"]).standard_normal(
                (B, H, d, d)) * 0.3).astype(np.float32)).to(device)
        print(f"noalloc B{B} T{T} H{H} d{d} C{chunk}", flush=True)
        o1, s1 = _noalloc(t, s0, B, T, H, d, chunk)
        o2, s2 = muir.chunk_fwd(*[t[n] for n in NAMES], s0=s0, chunk=chunk)
        torch.cuda.synchronize()
        assert torch.isfinite(o1.float()).all() and torch.isfinite(s1).all()
        assert torch.equal(o1, o2), f"o differs (B{B} T{T} H{H} d{d} C{chunk})"
        assert torch.equal(s1, s2), f"state differs (B{B} T{T} H{H} d{d} C{chunk})"


def test_noalloc_refuses_sizes_beyond_the_scratch(device):
    """The long-context shape needs 904 MiB of workspace: refused before any launch."""
    B, T, H, d = 1, 32768, 16, 128
    v = torch.zeros(1, dtype=torch.bfloat16, device=device)
    p = ctypes.c_void_p(v.data_ptr())
    st = muir.lib().muir_chunk_fwd_noalloc(p, p, p, p, p, p, p, p, None, p, None, B, T, H, d, d,
                                           256, muir.MUIR_BF16, None)
    assert st == 4 and "static scratch" in muir.last_error()
