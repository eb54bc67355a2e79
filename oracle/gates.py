"""Low-rank gate generation, the plain definition (fp64, numpy). TEST INFRASTRUCTURE, like
the rest of this package.

The pages fuse the five gates into one projection of total rank 512: one shared
down-projection, then a separate up-projection per gate with its own rank, decay 64,
erase 64, output 128, write 128 and dynamic read 128 (openai-hub news page, section on
sensitivity-allocated gating, gate table; liuch.name summary, second bullet). The
down-projection's output z [B, T, 512] is the input here, its rank slices in the table's
order. What the pages leave open, and the reading taken:
  * the pre-activation of gate n is y_n = z[..., slice_n] U_n + c_n, with U_n [H, d, r_n]
    per head and channel and a per-channel offset c_n [H, d];
  * the decay is a = exp(-exp(y_a)): y_a is the log decay rate, as in the workloads'
    decay recipe (base rate plus a per-token jitter), so a stays in (0, 1];
  * the erase, write and query (dynamic read) gates are sigmoid(y);
  * the output gate is sigmoid(y_output) as well, per value channel, and multiplies the
    readout o_t elementwise after the read (it feeds none of the recurrence's four gates).
"""
from __future__ import annotations

import numpy as np

# Rank slices of z, in the gate table's order.
RANKS = {"decay": 64, "erase": 64, "output": 128, "write": 128, "read": 128}
SLICES = {}
_o = 0
for _n, _r in RANKS.items():
    SLICES[_n] = slice(_o, _o + _r)
    _o += _r
RANK = _o  # 512

__all__ = ["RANKS", "SLICES", "RANK", "preactivation", "lowrank_gates", "output_gate"]


def preactivation(z, U, c, name):
    """y [B,T,H,d] = z[..., slice(name)] @ U[h]^T + c[h] in fp64 (U [H,d,r], c [H,d])."""
    zs = np.asarray(z, dtype=np.float64)[..., SLICES[name]]          # [B,T,r]
    U = np.asarray(U, dtype=np.float64)                              # [H,d,r]
    y = np.einsum("btr,hdr->bthd", zs, U)
    return y + np.asarray(c, dtype=np.float64)[None, None]


def lowrank_gates(z, Ua, Ue, Uw, Ug, ca, ce, cw, cg):
    """The four gates of the recurrence from the low-rank projection: a (decay), e (erase),
    w (write) and g (query gate), each [B,T,H,d] fp64."""
    a = np.exp(-np.exp(preactivation(z, Ua, ca, "decay")))
    sig = lambda y: 1.0 / (1.0 + np.exp(-y))
    e = sig(preactivation(z, Ue, ce, "erase"))
    w = sig(preactivation(z, Uw, cw, "write"))
    g = sig(preactivation(z, Ug, cg, "read"))
    return a, e, w, g


def output_gate(z, Uo, co):
    """The output gate og [B,T,H,dv] fp64 = sigmoid(z[..., 128:256] Uo^T + co) from the
    rank-128 output slice of the same projection (Uo [H,dv,128], co [H,dv]); the gated
    readout is o_t * og_t."""
    y = preactivation(z, Uo, co, "output")
    return 1.0 / (1.0 + np.exp(-y))
