"""A CPU model of the bf16 filter path's rounding (test infrastructure).

The bf16 filter path (SchNet's continuous-filter convolution with its filter
network in bfloat16; FlashSchNet §4.4 names 16-bit filter arithmetic) rounds
four activations per edge to bfloat16 before they enter a matrix product:
the radial basis b~(d) = RBF(d) C(d), its derivative along d, the
shifted-softplus output of the filter's first layer, and that output's
derivative along d (the filter's d-derivative is carried forward). It
evaluates the filter in base-2 units, so each of these values is rounded
after scaling by log2 e (the envelope carries the factor; the first layer's
biases are scaled to match and the filter output is scaled back by ln 2).
Everything else is fp32 arithmetic.

This module applies exactly those roundings to an fp64 copy of the oracle's
arithmetic (the oracle itself keeps every activation exact), with the same
bf16-rounded weights. With ``scale=LOG2E`` it predicts the path's deviation
from the oracle; other scales give other samples of the same rounding, which
is how the 16-bit parity bars are checked against what bf16 rounding itself
does. Only tests use it.
"""
from __future__ import annotations

import numpy as np

from oracle import schnet as S

LOG2E = 1.4426950408889634074


def round_bf16(a, scale=1.0):
    """bf16(fp32(a * scale)) / scale, round to nearest even at both steps."""
    v = np.asarray(np.asarray(a, dtype=np.float64) * scale, dtype=np.float32)
    return S._bf16_round(v).astype(np.float64) / scale


def rounded_energy_forces(desc, flat, pos, types, rowptr, col, n_replicas, periodic=False,
                          box=0.0, scale=LOG2E, rnd=True):
    """Energies [R], forces [R*N, 3] and per-atom energies with the four
    filter activations rounded as above (rnd=False: no rounding, which
    reproduces the oracle and pins this copy of its arithmetic)."""
    R = (lambda a: round_bf16(a, scale)) if rnd else (lambda a: a)
    W = S.unpack_weights(desc, flat)
    src, dst = S._edges(rowptr, col)
    n = len(types)
    Sd, Ss = S._incidence(dst, n), S._incidence(src, n)
    u, d = S.edge_vectors(pos, src, dst, periodic, box)
    mask = (d < desc.r_cut).astype(np.float64)
    g, C = S.rbf(d, desc), S.cutoff(d, desc.r_cut)
    bt = R(g * C[:, None])
    dbt = R(S.rbf_deriv(d, desc) * C[:, None] + g * S.cutoff_deriv(d, desc.r_cut)[:, None])
    x = W["emb"][np.asarray(types)]
    tape = []
    for blk in W["blocks"]:
        a1 = bt @ blk["Wf1"] + blk["cf1"]
        s1 = R(S.ssp(a1))
        ds1 = R(S.sigmoid(a1) * (dbt @ blk["Wf1"]))
        w = (s1 @ blk["Wf2"] + blk["cf2"]) * mask[:, None]
        dw = (ds1 @ blk["Wf2"]) * mask[:, None]          # d w_e / d d_e
        au = (Sd @ (x[src] * w)) @ blk["Wu1"] + blk["cu1"]
        tape.append((x, w, dw, au))
        x = x + S.ssp(au) @ blk["Wu2"] + blk["cu2"]
    ao = x @ W["Wo1"] + W["co1"]
    eps = S.ssp(ao) @ W["Wo2"] + W["co2"][0]
    g_x = (S.sigmoid(ao) * W["Wo2"][None, :]) @ W["Wo1"].T
    g_d = np.zeros_like(d)
    for blk, (x, w, dw, au) in zip(reversed(W["blocks"]), reversed(tape)):
        g_m = (((g_x @ blk["Wu2"].T) * S.sigmoid(au)) @ blk["Wu1"].T)[dst]
        g_d += np.einsum("ec,ec->e", g_m * x[src], dw)
        g_x = g_x + Ss @ (g_m * w)
    g_u = (g_d / np.where(d > 0, d, 1.0))[:, None] * u
    return eps.reshape(n_replicas, -1).sum(axis=1), -(Sd @ g_u - Ss @ g_u), eps
