"""Seeded synthetic inputs for the chunkwise gated delta rule and its decode step.

This module holds input recipes only: shapes, distributions, draw order and the
bf16 rounding of q/k/v. It contains no part of the recurrence itself, and both the
CPU oracle and the GPU path take their inputs from here.

The recipes follow the workloads of the Muir pages ("Muir: Linear Attention with
Sensitivity-Allocated Gating and Matched-Filter Readout", arXiv 2611.08376): a
166M-class layer (H=12, d=64), a 1.34B-class layer (H=16, d=128, 24 layers), the
4K training length and the 16K/32K long-context points, multi-timescale per-row
decay with slow rows carrying ~100x the energy of fast rows, and a decode step
against the fixed 25 MB fp32 state.

Readings of points the pages leave open (this recipe takes the plainest one for each):
  * decay a = exp(-exp(u + eps)), eps ~ N(0, 0.1) per token and row; u is the
    log of the decay rate, so a stays in (0, 1];
  * half-life workloads: h = 10**U(0, log10 Hmax), u = ln(ln 2 / h), i.e. the
    base decay is 2**(-1/h);
  * the base u is per (head, row), shared over the batch (per (layer, head, row)
    for the decode workload);
  * r_i = sqrt(1 - a_base_i), divided by its mean over the rows of the head;
  * stress heads (h % 4 == 0 in the long-context workload): a ~ U(1e-3, 0.05)
    iid per token and row, r = 1;
  * q, k = L2-normalise(SiLU(N(0,1))) with a 1e-12 guard, then q, k, v rounded
    to bf16 (round-to-nearest-even); the oracle consumes the rounded values.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

__all__ = [
    "ChunkConfig", "DecodeConfig", "CHUNK_CONFIGS", "DECODE_CONFIG",
    "round_bf16", "chunk_inputs", "decode_base", "decode_step_inputs_torch",
    "decode_seed", "output_gate", "scalar_erase", "lowrank_gate_inputs", "GATE_RANKS",
]


@dataclass(frozen=True)
class ChunkConfig:
    """One chunk-forward workload (a single layer call)."""
    name: str
    B: int
    H: int
    d: int
    T: int
    chunks: tuple
    qkv: str            # "f32" or "bf16"
    decay: str          # "uniform_u" (u ~ U(-6, 0)) or "halflife"
    hmax: float = 0.0   # largest half-life for "halflife"
    stress: bool = False
    seed: int = 0
    tol: float = 2e-2   # max relative error per head (o and final state)


CHUNK_CONFIGS = {
    0: ChunkConfig("tiny-fp32 B1 H2 d64 T256", 1, 2, 64, 256, (64,), "f32",
                   "uniform_u", seed=0, tol=1e-4),
    1: ChunkConfig("166M-class B8 H12 d64 T4096", 8, 12, 64, 4096, (64,), "bf16",
                   "halflife", hmax=1e4, seed=1),
    2: ChunkConfig("1.34B-class B8 H16 d128 T4096", 8, 16, 128, 4096, (128, 256),
                   "bf16", "halflife", hmax=1e5, seed=2),
    3: ChunkConfig("long-context B1 H16 d128 T32768", 1, 16, 128, 32768, (256,),
                   "bf16", "halflife", hmax=1e5, stress=True, seed=3),
}


@dataclass(frozen=True)
class DecodeConfig:
    """The recurrent decode workload: B sequences x L layers x H heads, one token per step."""
    B: int = 256
    L: int = 24
    H: int = 16
    d: int = 128
    steps: int = 1024
    seed: int = 4
    tol: float = 2e-2
    name: str = field(default="decode B256 L24 H16 d128 x1024 steps")


DECODE_CONFIG = DecodeConfig()


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returns float32.

    Non-finite inputs are not expected here (the generators never produce them).
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32)
    lsb = (bits >> np.uint32(16)) & np.uint32(1)
    rounded = (bits + np.uint32(0x7FFF) + lsb) & np.uint32(0xFFFF0000)
    return rounded.view(np.float32)


def _silu_normalise(x: np.ndarray) -> np.ndarray:
    """SiLU then L2-normalise over the last axis (1e-12 guard), float32, in place."""
    x = np.asarray(x, dtype=np.float32)
    den = np.exp(-x)
    den += np.float32(1.0)
    x /= den
    del den
    n = np.sqrt(np.einsum("...i,...i->...", x, x, dtype=np.float64))[..., None]
    x /= np.maximum(n, 1e-12).astype(np.float32)
    return x


def _sigmoid(x: np.ndarray) -> np.ndarray:
    """Logistic function, float32, in place."""
    x = np.asarray(x, dtype=np.float32)
    np.negative(x, out=x)
    np.exp(x, out=x)
    x += np.float32(1.0)
    np.reciprocal(x, out=x)
    return x


_BLOCK = 1 << 22   # elements per independent random stream


def _normal(seq: np.random.SeedSequence, shape) -> np.ndarray:
    """float32 N(0,1) array filled from fixed-size blocks, each with its own stream
    spawned from ``seq``; the result does not depend on the number of threads."""
    from concurrent.futures import ThreadPoolExecutor
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32)
    nblk = (n + _BLOCK - 1) // _BLOCK
    kids = seq.spawn(nblk)

    def fill(i):
        gen = np.random.Generator(np.random.PCG64(kids[i]))
        gen.standard_normal(out=out[i * _BLOCK:(i + 1) * _BLOCK], dtype=np.float32)

    if nblk == 1:
        fill(0)
    else:
        with ThreadPoolExecutor(max_workers=min(16, nblk)) as ex:
            list(ex.map(fill, range(nblk)))
    return out.reshape(shape)


def _base_u(rng: np.random.Generator, decay: str, hmax: float, shape) -> np.ndarray:
    """Log decay rate u per row (float64). a_base = exp(-exp(u))."""
    if decay == "uniform_u":
        return rng.uniform(-6.0, 0.0, size=shape)
    if decay == "halflife":
        log_h = rng.uniform(0.0, math.log10(hmax), size=shape)
        return np.log(math.log(2.0) / (10.0 ** log_h))
    raise ValueError(f"unknown decay recipe {decay!r}")


def _row_scale(u: np.ndarray) -> np.ndarray:
    """Static readout row scale from the base decay: sqrt(1 - a_base), mean 1 per head."""
    a_base = np.exp(-np.exp(u))
    r = np.sqrt(1.0 - a_base)
    return r / np.mean(r, axis=-1, keepdims=True)


def chunk_inputs(cfg: ChunkConfig | int, *, B=None, T=None, H=None, d=None,
                 seed=None, qkv=None) -> dict:
    """Draw the inputs of one chunk-forward workload.

    Sizes may be overridden (same distributions, smaller shapes) for tests.
    Streams: ``SeedSequence(seed).spawn(9)`` gives one stream each, in this order, for
    the base u [H,d], eps, q, k, v, e, w, g (each [B,T,H,d], drawn in blocks of 2**22
    elements with their own spawned streams) and the stress-head decays.

    Returns float32 numpy arrays q, k, v, a, g, e, w ([B,T,H,d]) and r ([H,d]);
    q, k, v already hold bf16-representable values when ``qkv == "bf16"``.
    """
    if isinstance(cfg, int):
        cfg = CHUNK_CONFIGS[cfg]
    B = cfg.B if B is None else B
    T = cfg.T if T is None else T
    H = cfg.H if H is None else H
    d = cfg.d if d is None else d
    seed = cfg.seed if seed is None else seed
    qkv = cfg.qkv if qkv is None else qkv
    seqs = np.random.SeedSequence(seed).spawn(9)
    shape = (B, T, H, d)

    u = _base_u(np.random.Generator(np.random.PCG64(seqs[0])), cfg.decay, cfg.hmax, (H, d))
    a = _normal(seqs[1], shape)                           # eps / 0.1
    a *= np.float32(0.1)
    a += u.astype(np.float32)[None, None]
    np.exp(a, out=a)
    np.negative(a, out=a)
    np.exp(a, out=a)                                       # a = exp(-exp(u + eps))
    q = _silu_normalise(_normal(seqs[2], shape))
    k = _silu_normalise(_normal(seqs[3], shape))
    v = _normal(seqs[4], shape)
    e = _sigmoid(_normal(seqs[5], shape))
    w = _sigmoid(_normal(seqs[6], shape))
    g = _sigmoid(_normal(seqs[7], shape))
    r = _row_scale(u)

    stress_heads = [h for h in range(H) if h % 4 == 0] if cfg.stress else []
    if stress_heads:
        rng_s = np.random.Generator(np.random.PCG64(seqs[8]))
        a_s = rng_s.uniform(1e-3, 0.05, size=(B, T, len(stress_heads), d)).astype(np.float32)
        for i, h in enumerate(stress_heads):
            a[:, :, h, :] = a_s[:, :, i, :]
            r[h, :] = 1.0

    if qkv == "bf16":
        q, k, v = round_bf16(q), round_bf16(k), round_bf16(v)
    elif qkv != "f32":
        raise ValueError(f"unknown qkv dtype {qkv!r}")
    return dict(q=q, k=k, v=v, a=a, g=g, e=e, w=w, r=r.astype(np.float32),
                stress_heads=stress_heads, config=cfg, B=B, T=T, H=H, d=d, qkv=qkv)


# ----------------------------------------------------------------------------
# Decode workload: base decay per (layer, head, row) from numpy; per-step draws
# on the device with a torch generator seeded from (4, step).
# ----------------------------------------------------------------------------

def output_gate(B: int, T: int, H: int, d: int, seed: int) -> np.ndarray:
    """Output-gate values og = sigmoid(N(0,1)) [B,T,H,d] float32, like e, w and g, from a
    stream of their own (``SeedSequence((seed, 10))``), so the other inputs of the same
    seed are unchanged."""
    return _sigmoid(_normal(np.random.SeedSequence((seed, 10)), (B, T, H, d)))


def scalar_erase(B: int, T: int, H: int, seed: int) -> np.ndarray:
    """One erase strength per token and head, e = sigmoid(N(0,1)) [B,T,H] float32, like the
    per-channel e, from a stream of its own (``SeedSequence((seed, 11))``)."""
    return _sigmoid(_normal(np.random.SeedSequence((seed, 11)), (B, T, H)))


# Rank slices of the fused gate projection's output z, in the gate table's order: decay 64,
# erase 64, output 128, write 128, read 128.
GATE_RANKS = (("decay", 64), ("erase", 64), ("output", 128), ("write", 128), ("read", 128))


def lowrank_gate_inputs(cfg: ChunkConfig | int, *, B=None, T=None, H=None, d=None,
                        seed=None) -> dict:
    """Inputs of the low-rank gate projection for a chunk workload: z [B,T,512] (the shared
    down-projection's output) and, per gate n in (decay, erase, write, read, output), an
    up-projection U_n [H,d,r_n] and an offset c_n [H,d].

    Recipe (one stream each, from ``SeedSequence((seed, 12)).spawn(5)``: z, then U for
    decay, erase, write, read): z ~ N(0,1); U_decay ~ N(0, 0.1^2/64), so that the decay's
    log-rate jitter z U has std 0.1 as in the decay recipe, with c_decay = the base log
    rate u of the configuration; U_erase, U_write, U_read ~ N(0, 1/r), so their
    pre-activations are N(0,1) as for sigmoid(N(0,1)), with zero offsets. On stress heads
    (h % 4 == 0 where the configuration has them) c_decay = ln(-ln 0.0255) and U_decay ~
    N(0, 1/64): decays spread over roughly 1e-4 .. 0.25. z and every U are rounded to bf16.
    """
    if isinstance(cfg, int):
        cfg = CHUNK_CONFIGS[cfg]
    B = cfg.B if B is None else B
    T = cfg.T if T is None else T
    H = cfg.H if H is None else H
    d = cfg.d if d is None else d
    seed = cfg.seed if seed is None else seed
    seqs = np.random.SeedSequence((seed, 12)).spawn(5)
    u = _base_u(np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed).spawn(9)[0])),
                cfg.decay, cfg.hmax, (H, d))
    z = round_bf16(_normal(seqs[0], (B, T, 512)))
    out = {"z": z}
    ranks = dict(GATE_RANKS)
    stress = [h for h in range(H) if h % 4 == 0] if cfg.stress else []
    for i, n in enumerate(("decay", "erase", "write", "read")):
        r = ranks[n]
        U = _normal(seqs[1 + i], (H, d, r))
        if n == "decay":
            U *= np.float32(0.1 / math.sqrt(r))
            c = u.astype(np.float32)
            for h in stress:
                U[h] *= np.float32(10.0)
                c[h] = np.float32(math.log(-math.log(0.0255)))
        else:
            U *= np.float32(1.0 / math.sqrt(r))
            c = np.zeros((H, d), np.float32)
        out["U_" + n] = round_bf16(U)
        out["c_" + n] = c
    # The output gate (rank 128), from a stream of its own (``SeedSequence((seed, 13))``) so
    # that the other inputs of the same seed are unchanged: U_output ~ N(0, 1/128), zero
    # offsets, like the erase, write and read gates.
    Uo = _normal(np.random.SeedSequence((seed, 13)), (H, d, ranks["output"]))
    Uo *= np.float32(1.0 / math.sqrt(ranks["output"]))
    out["U_output"] = round_bf16(Uo)
    out["c_output"] = np.zeros((H, d), np.float32)
    return out


def decode_base(cfg: DecodeConfig = DECODE_CONFIG, *, L=None, H=None, d=None):
    """Base log-rate u [L,H,d] (float64) and row scale r [L,H,d] (float32)."""
    L = cfg.L if L is None else L
    H = cfg.H if H is None else H
    d = cfg.d if d is None else d
    rng = np.random.default_rng(cfg.seed)
    u = rng.uniform(-6.0, 0.0, size=(L, H, d))
    return u, _row_scale(u).astype(np.float32)


def decode_seed(step: int, cfg: DecodeConfig = DECODE_CONFIG) -> int:
    """Seed of the per-step generator: the pair (4, step) packed into one integer."""
    return (cfg.seed << 32) | int(step)


def decode_step_inputs_torch(step: int, u_lhd, device, *, B: int,
                             cfg: DecodeConfig = DECODE_CONFIG, qkv_dtype=None):
    """Draw one decode step's inputs for every (layer, sequence, head) on ``device``.

    ``u_lhd`` is the base log-rate as a float32 torch tensor [L,H,d] on ``device``.
    Returns a dict of tensors shaped [L,B,H,d]: q, k, v (bf16 unless ``qkv_dtype``
    says otherwise) and a, g, e, w (float32). Draw order: eps, q, k, v, e, w, g.
    """
    import torch
    qkv_dtype = torch.bfloat16 if qkv_dtype is None else qkv_dtype
    L, H, d = u_lhd.shape
    gen = torch.Generator(device=device)
    gen.manual_seed(decode_seed(step, cfg))
    shape = (L, B, H, d)

    def normal():
        return torch.randn(shape, generator=gen, device=device, dtype=torch.float32)

    eps = normal() * 0.1
    a = torch.exp(-torch.exp(u_lhd[:, None] + eps))
    q = torch.nn.functional.silu(normal())
    q = q / q.norm(dim=-1, keepdim=True).clamp_min(1e-12)
    k = torch.nn.functional.silu(normal())
    k = k / k.norm(dim=-1, keepdim=True).clamp_min(1e-12)
    v = normal()
    e = torch.sigmoid(normal())
    w = torch.sigmoid(normal())
    g = torch.sigmoid(normal())
    return dict(q=q.to(qkv_dtype), k=k.to(qkv_dtype), v=v.to(qkv_dtype),
                a=a, g=g, e=e, w=w)
