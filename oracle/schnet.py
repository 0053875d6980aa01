"""SchNet energy and forces in fp64: the unfused definition.

Follows FlashSchNet (arXiv 2602.13140) §3.2 "SchNet model": distances and
radial basis, filter network, CFConv message passing and aggregation, energy
readout, forces via the gradient; §4.2 "Fused forward operator" for where the
cosine envelope sits (on the basis, before the filter network); §4.1
"Precision contract" for the fp32 inputs and outputs.

Readings of what the page leaves open (its displayed equations lost their
bodies in extraction):
* RBF: Gaussians exp(-(d - mu_k)^2 / (2 sigma^2)), centres mu_k evenly spaced
  from rbf_min to rbf_max inclusive, sigma equal to the spacing;
* envelope C(d) = (cos(pi d / r_cut) + 1) / 2 for d < r_cut, else 0;
  basis b~ = RBF(d) * C(d);
* filter network Linear(Dr -> D), shifted softplus, Linear(D -> D);
* message m_e = x_src * w_e, no atom-wise layer before the gather;
* update x' = x + Linear(ssp(Linear(h))) with D -> D -> D;
* readout eps_i = Linear(ssp(Linear(x_i))) with D -> H -> 1;
* ssp(x) = ln(1 + e^x) - ln 2;
* an edge with d >= r_cut in the list (a list built with a skin) contributes
  nothing: its message and all of its gradients are zero;
* forces F = -dE/dr, by hand-derived reverse mode through every step.

The aggregation sum over incoming edges (and the backward sums over source
and destination) are written as products with 0/1 incidence matrices, which
is the plain definition of "sum over e with dst[e] = i".
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import scipy.sparse as sp

LN2 = np.log(2.0)
FILTER_F32 = 0
FILTER_BF16 = 1
W16A16 = 2
# fp32 filter whose products the kernels evaluate on fp16 hi/lo pairs: the
# model itself is the fp32 one, so the oracle treats it as FILTER_F32
FILTER_F16X2 = 3


@dataclass(frozen=True)
class ModelDesc:
    n_types: int
    D: int
    Dr: int
    T: int
    rbf_min: float
    rbf_max: float
    r_cut: float
    H: int
    filter_dtype: int = FILTER_F32


def _bf16_round(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even), returned as
    float32. Bit manipulation of the IEEE encoding; NaN is not expected."""
    u = np.asarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    u = (u + 0x7FFF + lsb) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


def f16_channel_quantize(W: np.ndarray) -> np.ndarray:
    """Per-output-channel 16-bit weights (§4.4 "Channel-wise quantization"),
    with power-of-two scales as the reading of the page's per-channel scales.

    Column n of W [fan_in][fan_out] (a vector is one column) gets the scale
    s_n = 2^e where its largest magnitude is m 2^e with m in [0.5, 1) (s_n = 1
    for an all-zero column); the column is divided by s_n (exact), rounded to
    IEEE half precision (nearest, ties to even) and multiplied back. Returns
    float32 of W's shape."""
    W = np.asarray(W, dtype=np.float32)
    col = W.reshape(W.shape[0], -1)
    amax = np.max(np.abs(col), axis=0)
    _, e = np.frexp(amax)
    s = np.where(amax > 0, np.ldexp(np.float32(1.0), e), np.float32(1.0)).astype(np.float32)
    q = (col / s).astype(np.float16).astype(np.float32) * s
    return q.reshape(W.shape)


def unpack_weights(desc: ModelDesc, flat) -> dict:
    """Split the flat fp32 vector into named fp64 arrays.

    Order: Emb[n_types][D]; per block Wf1[Dr][D], cf1[D], Wf2[D][D], cf2[D],
    Wu1[D][D], cu1[D], Wu2[D][D], cu2[D]; then Wo1[D][H], co1[H], Wo2[H],
    co2[1]. With a bf16 filter network the two filter weight matrices of every
    block are first rounded to bfloat16 (their biases stay fp32); with
    W16A16 every MLP weight (Wf1, Wf2, Wu1, Wu2, Wo1, Wo2) goes through
    f16_channel_quantize (biases and the embedding stay fp32). FILTER_F32 and
    FILTER_F16X2 use the weights as given."""
    flat = np.asarray(flat, dtype=np.float32)
    D, Dr, H = desc.D, desc.Dr, desc.H
    off = 0

    def take(*shape):
        nonlocal off
        n = int(np.prod(shape))
        a = flat[off:off + n].reshape(shape)
        off += n
        return a

    W = {"emb": take(desc.n_types, D), "blocks": []}
    for _ in range(desc.T):
        blk = {}
        for name, shape in (("Wf1", (Dr, D)), ("cf1", (D,)), ("Wf2", (D, D)), ("cf2", (D,)),
                            ("Wu1", (D, D)), ("cu1", (D,)), ("Wu2", (D, D)), ("cu2", (D,))):
            blk[name] = take(*shape)
        if desc.filter_dtype == FILTER_BF16:
            for name in ("Wf1", "Wf2"):
                blk[name] = _bf16_round(blk[name])
        elif desc.filter_dtype == W16A16:
            for name in ("Wf1", "Wf2", "Wu1", "Wu2"):
                blk[name] = f16_channel_quantize(blk[name])
        W["blocks"].append(blk)
    W["Wo1"] = take(D, H)
    W["co1"] = take(H)
    W["Wo2"] = take(H)
    W["co2"] = take(1)
    if desc.filter_dtype == W16A16:
        W["Wo1"] = f16_channel_quantize(W["Wo1"])
        W["Wo2"] = f16_channel_quantize(W["Wo2"])
    if off != flat.size:
        raise ValueError(f"weight vector has {flat.size} values, model needs {off}")

    def f64(x):
        if isinstance(x, dict):
            return {k: f64(v) for k, v in x.items()}
        if isinstance(x, list):
            return [f64(v) for v in x]
        return np.asarray(x, dtype=np.float64)

    return f64(W)


# ---------------------------------------------------------------- elementwise pieces
def ssp(x):
    """Shifted softplus ln(1 + e^x) - ln 2, in the overflow-free form
    max(x, 0) + ln(1 + e^-|x|) - ln 2."""
    return np.maximum(x, 0.0) + np.log1p(np.exp(-np.abs(x))) - LN2


def sigmoid(x):
    """Derivative of ssp: 1 / (1 + e^-x)."""
    e = np.exp(-np.abs(x))
    return np.where(x >= 0, 1.0 / (1.0 + e), e / (1.0 + e))


def rbf_centres(desc: ModelDesc):
    mu = desc.rbf_min + np.arange(desc.Dr) * ((desc.rbf_max - desc.rbf_min) / (desc.Dr - 1))
    sigma = (desc.rbf_max - desc.rbf_min) / (desc.Dr - 1)
    return mu, sigma


def rbf(d, desc: ModelDesc):
    """Gaussian basis g_k(d) = exp(-(d - mu_k)^2 / (2 sigma^2)); [E, Dr]."""
    mu, sigma = rbf_centres(desc)
    z = (np.asarray(d)[..., None] - mu) / sigma
    return np.exp(-0.5 * z * z)


def rbf_deriv(d, desc: ModelDesc):
    """d g_k / d d = -(d - mu_k) / sigma^2 * g_k(d)."""
    mu, sigma = rbf_centres(desc)
    diff = np.asarray(d)[..., None] - mu
    return -(diff / (sigma * sigma)) * np.exp(-0.5 * (diff / sigma) ** 2)


def cutoff(d, r_cut):
    """Cosine envelope (cos(pi d / r_cut) + 1) / 2 inside the cutoff, 0 outside."""
    d = np.asarray(d, dtype=np.float64)
    return np.where(d < r_cut, 0.5 * (np.cos(np.pi * d / r_cut) + 1.0), 0.0)


def cutoff_deriv(d, r_cut):
    d = np.asarray(d, dtype=np.float64)
    return np.where(d < r_cut, -0.5 * (np.pi / r_cut) * np.sin(np.pi * d / r_cut), 0.0)


# ---------------------------------------------------------------- graph plumbing
def _edges(rowptr, col):
    rowptr = np.asarray(rowptr, dtype=np.int64)
    src = np.asarray(col, dtype=np.int64)
    dst = np.repeat(np.arange(len(rowptr) - 1), np.diff(rowptr))
    return src, dst


def _incidence(index, n_nodes):
    """0/1 matrix S [n_nodes, E] with S[index[e], e] = 1, so S @ M sums the
    rows of M that belong to each node."""
    E = len(index)
    return sp.csr_matrix((np.ones(E), (index, np.arange(E))), shape=(n_nodes, E))


def edge_vectors(pos, src, dst, periodic, box):
    """u_e = r_dst - r_src (minimum image for a periodic cube), d_e = |u_e|."""
    p = np.asarray(pos, dtype=np.float64)
    u = p[dst] - p[src]
    if periodic:
        L = float(np.float32(box))
        u = u - L * np.round(u / L)
    d = np.sqrt(np.einsum("ij,ij->i", u, u))
    return u, d


# ---------------------------------------------------------------- the model
def _forward(desc, W, pos, types, src, dst, periodic, box):
    """Forward pass; returns per-atom energies and everything the gradient needs."""
    n = len(types)
    S_dst = _incidence(dst, n)
    u, d = edge_vectors(pos, src, dst, periodic, box)
    mask = (d < desc.r_cut).astype(np.float64)
    g = rbf(d, desc)
    C = cutoff(d, desc.r_cut)
    bt = g * C[:, None]                                  # b~_e = RBF(d_e) C(d_e)
    x = W["emb"][np.asarray(types)]                      # x^(0)_i = Emb[Z_i]
    tape = []
    for blk in W["blocks"]:
        a1 = bt @ blk["Wf1"] + blk["cf1"]
        s1 = ssp(a1)
        w = (s1 @ blk["Wf2"] + blk["cf2"]) * mask[:, None]   # w_e = MLP_filter(b~_e)
        m = x[src] * w                                        # m_e = x_src * w_e
        h = S_dst @ m                                         # h_i = sum_{dst[e]=i} m_e
        au = h @ blk["Wu1"] + blk["cu1"]
        x_next = x + ssp(au) @ blk["Wu2"] + blk["cu2"]        # residual update
        tape.append((x, a1, w, h, au))
        x = x_next
    ao = x @ W["Wo1"] + W["co1"]
    eps = ssp(ao) @ W["Wo2"] + W["co2"][0]                    # eps_i = MLP_out(x^(T)_i)
    return eps, dict(u=u, d=d, mask=mask, g=g, C=C, tape=tape, ao=ao, S_dst=S_dst)


def _replica_sums(eps, n_replicas):
    return eps.reshape(n_replicas, -1).sum(axis=1)


def forward_trace(desc: ModelDesc, flat_weights, pos, types, rowptr, col, periodic=False,
                  box=0.0, weights=None):
    """Per-atom energies and the per-block tape (x, a1, w, h, au) of the forward."""
    W = weights if weights is not None else unpack_weights(desc, flat_weights)
    src, dst = _edges(rowptr, col)
    eps, c = _forward(desc, W, pos, types, src, dst, periodic, box)
    return eps, c["tape"]


def energy(desc: ModelDesc, flat_weights, pos, types, rowptr, col, n_replicas=1,
           periodic=False, box=0.0, weights=None):
    """Energy per replica, fp64 [R]."""
    W = weights if weights is not None else unpack_weights(desc, flat_weights)
    src, dst = _edges(rowptr, col)
    eps, _ = _forward(desc, W, pos, types, src, dst, periodic, box)
    return _replica_sums(eps, n_replicas)


def energy_forces(desc: ModelDesc, flat_weights, pos, types, rowptr, col, n_replicas=1,
                  periodic=False, box=0.0, weights=None, return_eps=False):
    """Energy per replica [R] and forces [R*N, 3], both fp64.

    The reverse pass takes the chain backwards step by step; the sums over
    edges that share a destination or a source are incidence products
    (FlashSchNet §3.2 "Forces via autodiff": the gradient through aggregation
    is a sum over source nodes)."""
    W = weights if weights is not None else unpack_weights(desc, flat_weights)
    src, dst = _edges(rowptr, col)
    n = len(types)
    eps, c = _forward(desc, W, pos, types, src, dst, periodic, box)
    S_dst = c["S_dst"]
    S_src = _incidence(src, n)
    u, d, mask, g, C = c["u"], c["d"], c["mask"], c["g"], c["C"]

    # dE/d eps_i = 1 for every atom
    g_ao = sigmoid(c["ao"]) * W["Wo2"][None, :]
    g_x = g_ao @ W["Wo1"].T
    g_d = np.zeros_like(d)
    for blk, (x, a1, w, _h, au) in zip(reversed(W["blocks"]), reversed(c["tape"])):
        g_au = (g_x @ blk["Wu2"].T) * sigmoid(au)
        g_h = g_au @ blk["Wu1"].T
        g_m = g_h[dst]                              # h_i sums m_e over dst[e] = i
        g_x_prev = g_x + S_src @ (g_m * w)          # m_e depends on x_src[e]
        g_w = g_m * x[src] * mask[:, None]
        g_a1 = (g_w @ blk["Wf2"].T) * sigmoid(a1)
        g_bt = g_a1 @ blk["Wf1"].T
        g_d += np.einsum("ek,ek->e", g_bt, rbf_deriv(d, desc) * C[:, None]
                         + g * cutoff_deriv(d, desc.r_cut)[:, None])
        g_x = g_x_prev
    safe_d = np.where(d > 0, d, 1.0)
    g_u = (g_d / safe_d)[:, None] * u               # d d_e / d u_e = u_e / d_e
    g_pos = S_dst @ g_u - S_src @ g_u               # u_e = r_dst - r_src
    E = _replica_sums(eps, n_replicas)
    if return_eps:
        return E, -g_pos, eps
    return E, -g_pos
