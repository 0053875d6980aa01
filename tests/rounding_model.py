"""A CPU model of the 16-bit paths' activation rounding (test infrastructure).

Both 16-bit modes (FlashSchNet §4.4: 16-bit MLP arithmetic with fp32
accumulation) round activations as they enter a matrix product; the weights
are rounded once, exactly as the oracle's own quantizers do.

* bf16 filter: four activations per edge are rounded to bfloat16: the radial
  basis b~(d) = RBF(d) C(d), its derivative along d, the shifted-softplus
  output of the filter's first layer and that output's derivative along d
  (the filter's d-derivative is carried forward). The update and readout
  layers keep fp32-grade products.
* W16A16: the same four filter activations are rounded to fp16, and so is
  the input of every atom-wise product: the aggregated messages h and the
  update's softplus output, the readout's input features, and in the
  gradients the update's incoming gradient, its gated hidden gradient and the
  readout's gated output weights.

The filter is evaluated in base-2 units, so its four activations are rounded
after scaling by log2 e (the envelope carries the factor; the first layer's
biases are scaled to match and the filter output is scaled back by ln 2).
The atom-wise layers work in natural units; their per-column power-of-two
weight scales multiply some inputs before rounding, which changes nothing
but the treatment of fp16 subnormals.

This module applies exactly those roundings to an fp64 copy of the oracle's
arithmetic (the oracle keeps every activation exact). With the default
scales it predicts a path's deviation from the oracle: the bf16 filter's to
within fp32 arithmetic, W16A16's in distribution only (it also rounds the
features, so a tie decided differently on the GPU tips later ones). Other
scales give other samples of the same rounding, which is how the 16-bit
parity bars are checked against what the rounding itself does. Only tests
use it.
"""
from __future__ import annotations

import numpy as np

from oracle import schnet as S

LOG2E = 1.4426950408889634074


def round_bf16(a, scale=1.0):
    """bf16(fp32(a * scale)) / scale, round to nearest even at both steps."""
    v = np.asarray(np.asarray(a, dtype=np.float64) * scale, dtype=np.float32)
    return S._bf16_round(v).astype(np.float64) / scale


def round_f16(a, scale=1.0):
    """fp16(fp32(a * scale)) / scale, round to nearest even at both steps."""
    v = np.asarray(np.asarray(a, dtype=np.float64) * scale, dtype=np.float32)
    return v.astype(np.float16).astype(np.float64) / scale


def rounded_energy_forces(desc, flat, pos, types, rowptr, col, n_replicas, periodic=False,
                          box=0.0, scale=LOG2E, atom_scale=1.0, rnd=True):
    """Energies [R], forces [R*N, 3] and per-atom energies of a 16-bit model
    (desc.filter_dtype bf16 filter or W16A16) with its activations rounded as
    above: the filter's at `scale`, W16A16's atom-wise ones at `atom_scale`
    (rnd=False: no rounding, which reproduces the oracle and pins this copy
    of its arithmetic)."""
    if desc.filter_dtype == S.FILTER_BF16:
        Rf = lambda a: round_bf16(a, scale)
        Ra = lambda a: a
    elif desc.filter_dtype == S.W16A16:
        Rf = lambda a: round_f16(a, scale)
        Ra = lambda a: round_f16(a, atom_scale)
    else:
        raise ValueError("a 16-bit model is expected")
    if not rnd:
        Rf = Ra = lambda a: a
    W = S.unpack_weights(desc, flat)
    src, dst = S._edges(rowptr, col)
    n = len(types)
    Sd, Ss = S._incidence(dst, n), S._incidence(src, n)
    u, d = S.edge_vectors(pos, src, dst, periodic, box)
    mask = (d < desc.r_cut).astype(np.float64)
    g, C = S.rbf(d, desc), S.cutoff(d, desc.r_cut)
    bt = Rf(g * C[:, None])
    dbt = Rf(S.rbf_deriv(d, desc) * C[:, None] + g * S.cutoff_deriv(d, desc.r_cut)[:, None])
    x = W["emb"][np.asarray(types)]
    tape = []
    for blk in W["blocks"]:
        a1 = bt @ blk["Wf1"] + blk["cf1"]
        s1 = Rf(S.ssp(a1))
        ds1 = Rf(S.sigmoid(a1) * (dbt @ blk["Wf1"]))
        w = (s1 @ blk["Wf2"] + blk["cf2"]) * mask[:, None]
        dw = (ds1 @ blk["Wf2"]) * mask[:, None]          # d w_e / d d_e
        au = Ra(Sd @ (x[src] * w)) @ blk["Wu1"] + blk["cu1"]
        tape.append((x, w, dw, au))
        x = x + Ra(S.ssp(au)) @ blk["Wu2"] + blk["cu2"]
    ao = Ra(x) @ W["Wo1"] + W["co1"]
    eps = S.ssp(ao) @ W["Wo2"] + W["co2"][0]
    g_x = Ra(S.sigmoid(ao) * W["Wo2"][None, :]) @ W["Wo1"].T
    g_d = np.zeros_like(d)
    for blk, (x, w, dw, au) in zip(reversed(W["blocks"]), reversed(tape)):
        g_m = (Ra((Ra(g_x) @ blk["Wu2"].T) * S.sigmoid(au)) @ blk["Wu1"].T)[dst]
        g_d += np.einsum("ec,ec->e", g_m * x[src], dw)
        g_x = g_x + Ss @ (g_m * w)
    g_u = (g_d / np.where(d > 0, d, 1.0))[:, None] * u
    return eps.reshape(n_replicas, -1).sum(axis=1), -(Sd @ g_u - Ss @ g_u), eps
