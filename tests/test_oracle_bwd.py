"""Pins of the float64 backward oracle against facts fixed outside it.

torch autograd in float64 through torch's own SDPA (a library routine) with a bias built here
by indexing; central finite differences of the oracle's own forward on tiny inputs; and exact
identities of the softmax gradient.  CPU only.
"""

import math

import numpy as np
import pytest
import torch

import oracle


def _rng(seed):
    return np.random.default_rng(seed)


def _case(seed, mode, B=2, S=24, Hq=4, Hkv=2, D=5, R=3, Rb=7):
    rng = _rng(seed)
    q = rng.standard_normal((B, S, Hq, D))
    k = rng.standard_normal((B, S, Hkv, D))
    v = rng.standard_normal((B, S, Hkv, D))
    do = rng.standard_normal((B, S, Hq, D))
    table = rng.standard_normal((Hq, Rb))
    r = rng.standard_normal((B, S, Hq, R))
    E = rng.standard_normal((R, Rb) if mode == "rproj_shared" else (Hq, R, Rb))
    return q, k, v, do, table, r, E


def _autograd(q, k, v, do, table, r, E, *, mode, scale, window, Rb, temp_len):
    """Gradients by torch autograd (float64): SDPA with the queries and the bias scaled by the
    temperature, the bias gathered here from table / r.E by distance."""
    B, S, Hq, D = q.shape
    G = Hq // k.shape[2]
    t = {n: torch.tensor(x, dtype=torch.float64, requires_grad=True)
         for n, x in dict(q=q, k=k, v=v, table=table, r=r, E=E).items()}
    i = torch.arange(S)[:, None]
    j = torch.arange(S)[None, :]
    delta = i - j
    vis = delta >= 0
    if window:
        vis &= delta < window
    inband = (delta >= 0) & (delta < Rb)
    idx = delta.clamp(0, Rb - 1)
    if mode == "table":
        bias = t["table"][:, idx] * inband                          # [Hq, S, S]
        bias = bias[None].expand(B, Hq, S, S)
    elif mode in ("rproj", "rproj_shared"):
        bank = t["E"] if mode == "rproj" else t["E"][None].expand(Hq, -1, -1)   # [Hq, R, Rb]
        curves = torch.einsum("bihf,hfd->bhid", t["r"], bank)        # [B, Hq, S, Rb]
        bias = torch.gather(curves, 3, idx[None, None].expand(B, Hq, S, S)) * inband
    else:
        bias = torch.zeros(B, Hq, S, S, dtype=torch.float64)
    n = vis.sum(dim=1).to(torch.float64)
    tau = torch.ones(S, dtype=torch.float64) if not temp_len else \
        torch.clamp(torch.log(n) / math.log(temp_len), min=1.0)
    qh = t["q"].permute(0, 2, 1, 3) * tau[None, None, :, None]
    kh = t["k"].permute(0, 2, 1, 3).repeat_interleave(G, dim=1)
    vh = t["v"].permute(0, 2, 1, 3).repeat_interleave(G, dim=1)
    mask = torch.where(vis, 0.0, -math.inf).to(torch.float64)
    o = torch.nn.functional.scaled_dot_product_attention(
        qh, kh, vh, attn_mask=mask + bias * tau[None, None, :, None], scale=scale)
    loss = (o.permute(0, 2, 1, 3) * torch.from_numpy(do)).sum()
    loss.backward()
    return {n: (x.grad.numpy() if x.grad is not None else None) for n, x in t.items()}


@pytest.mark.parametrize("mode,window,Rb,temp_len", [
    ("none", 0, 7, 0), ("table", 0, 7, 0), ("table", 9, 30, 0), ("rproj", 0, 7, 0),
    ("rproj", 11, 6, 5), ("rproj_shared", 0, 9, 0), ("table", 0, 5, 4),
    ("rproj_shared", 13, 13, 6)])
def test_backward_matches_autograd_sdpa(mode, window, Rb, temp_len):
    q, k, v, do, table, r, E = _case(7 + Rb + window, mode, Rb=Rb)
    got = oracle.prefill_backward(q, k, v, do, scale=0.6, window=window, bias_range=Rb, mode=mode,
                                  table=table, r=r, E=E, temp_len=temp_len)
    ref = _autograd(q, k, v, do, table, r, E, mode=mode, scale=0.6, window=window, Rb=Rb,
                    temp_len=temp_len)
    for name in ("dq", "dk", "dv"):
        np.testing.assert_allclose(got[name], ref[name[1:]], atol=1e-11, err_msg=name)
    if mode == "table":
        np.testing.assert_allclose(got["dtable"], ref["table"], atol=1e-11)
    if mode in ("rproj", "rproj_shared"):
        np.testing.assert_allclose(got["dr"], ref["r"], atol=1e-11)
        np.testing.assert_allclose(got["dE"], ref["E"], atol=1e-11)


def _fd(f, x, idx, h=1e-6):
    xp = x.copy()
    xm = x.copy()
    xp[idx] += h
    xm[idx] -= h
    return (f(xp) - f(xm)) / (2 * h)


@pytest.mark.parametrize("mode", ["table", "rproj", "rproj_shared"])
def test_backward_matches_finite_differences(mode):
    """Central differences of the oracle's forward (loss = <o, dout>) at sampled entries."""
    q, k, v, do, table, r, E = _case(3, mode, B=1, S=9, Hq=2, Hkv=1, D=3, R=2, Rb=4)
    kw = dict(scale=0.8, window=6, bias_range=4, mode=mode, temp_len=3)
    got = oracle.prefill_backward(q, k, v, do, table=table, r=r, E=E, **kw)

    def loss(q=q, k=k, v=v, table=table, r=r, E=E):
        o, _ = oracle.prefill(q, k, v, table=table, r=r, E=E, **kw)
        return float((o * do).sum())

    rng = _rng(9)
    params = {"dq": ("q", q), "dk": ("k", k), "dv": ("v", v)}
    if mode == "table":
        params["dtable"] = ("table", table)
    else:
        params["dr"] = ("r", r)
        params["dE"] = ("E", E)
    for gname, (pname, x) in params.items():
        for _ in range(6):
            idx = tuple(int(rng.integers(0, n)) for n in x.shape)
            num = _fd(lambda y: loss(**{pname: y}), x, idx)
            assert abs(got[gname][idx] - num) < 1e-6, (gname, idx, got[gname][idx], num)


def test_backward_identities():
    """Exact identities of the softmax gradient:
    * sum_j dv_j = sum over the group's heads of sum_i dout_i (each row of P sums to 1);
    * the bias gradient of a row sums to zero (softmax is shift invariant), so when every
      visible pair is in band the table gradient sums to zero per head;
    * constant values: o is constant, so dq, dk and the bias gradients vanish."""
    q, k, v, do, table, r, E = _case(5, "table", S=20, Rb=20)
    g = oracle.prefill_backward(q, k, v, do, scale=0.5, window=0, bias_range=20, mode="table",
                                table=table)
    G = q.shape[2] // k.shape[2]
    lhs = g["dv"].sum(axis=1)                                   # [B, Hkv, D]
    rhs = do.sum(axis=1).reshape(do.shape[0], k.shape[2], G, -1).sum(axis=2)
    np.testing.assert_allclose(lhs, rhs, atol=1e-12)
    np.testing.assert_allclose(g["dtable"].sum(axis=1), 0.0, atol=1e-12)
    assert np.abs(g["dtable"]).max() > 1e-3
    vc = np.ones_like(v) * 0.7
    g2 = oracle.prefill_backward(q, k, vc, do, scale=0.5, bias_range=20, mode="table",
                                 table=table)
    for name in ("dq", "dk", "dtable"):
        assert np.abs(g2[name]).max() < 1e-12, name
