"""Pins of the float64 oracle against facts fixed outside the oracle itself.

Each test ties one part of the oracle to a textbook routine, a closed form, a
hand-derived fixture or a brute-force loop written independently here, so that
a dropped term, a wrong sign, a wrong index or a transposed operand in the
oracle fails at least one of them.  CPU only.
"""

import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _sdpa_f64(q, k, v, *, scale, window=0, bias=None):
    """torch SDPA in float64 on the CPU (textbook routine), GQA by repeating kv heads.

    q [B,S,Hq,D], k/v [B,S,Hkv,D] numpy; bias [Hq,S,S] or None.
    """
    B, S, Hq, D = q.shape
    G = Hq // k.shape[2]
    qt = torch.from_numpy(q).permute(0, 2, 1, 3)
    kt = torch.from_numpy(k).permute(0, 2, 1, 3).repeat_interleave(G, dim=1)
    vt = torch.from_numpy(v).permute(0, 2, 1, 3).repeat_interleave(G, dim=1)
    if window == 0 and bias is None:
        o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True,
                                                             scale=scale)
    else:
        i = torch.arange(S)[:, None]
        j = torch.arange(S)[None, :]
        vis = (i - j >= 0)
        if window:
            vis &= (i - j < window)
        mask = torch.where(vis, 0.0, -math.inf).to(torch.float64)
        if bias is not None:
            mask = mask[None] + torch.from_numpy(bias)
        o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask,
                                                             scale=scale)
    return o.permute(0, 2, 1, 3).numpy()


# --- P1: no bias reduces to plain causal softmax attention (library routine) ----------

@pytest.mark.parametrize("G", [1, 2, 4])
@pytest.mark.parametrize("window", [0, 300])
def test_plain_causal_matches_sdpa(G, window):
    """Zero bias with a window >= the sequence is plain causal attention (torch SDPA, fp64)."""
    rng = _rng(10 + G)
    B, S, Hkv, D = 2, 37, 2, 16
    Hq = Hkv * G
    q = rng.standard_normal((B, S, Hq, D))
    k = rng.standard_normal((B, S, Hkv, D))
    v = rng.standard_normal((B, S, Hkv, D))
    ref = _sdpa_f64(q, k, v, scale=0.3)
    for mode, kw in (("none", {}),
                     ("table", dict(table=np.zeros((Hq, 8)))),
                     ("rproj", dict(r=rng.standard_normal((B, S, Hq, 3)), E=np.zeros((Hq, 3, 8))))):
        o, _ = oracle.prefill(q, k, v, scale=0.3, window=window, bias_range=8, mode=mode, **kw)
        np.testing.assert_allclose(o, ref, rtol=0, atol=1e-12)


def test_sliding_window_matches_sdpa_mask():
    """Window W keeps keys with 0 <= i-j < W: SDPA with the same boolean band as an additive mask."""
    rng = _rng(3)
    B, S, H, D = 1, 50, 2, 8
    q, k, v = (rng.standard_normal((B, S, H, D)) for _ in range(3))
    for W in (1, 2, 7, 49, 50):
        o, _ = oracle.prefill(q, k, v, scale=0.5, window=W)
        np.testing.assert_allclose(o, _sdpa_f64(q, k, v, scale=0.5, window=W), atol=1e-12)
    # W = 1: every row sees only itself, so o = v of its own kv head
    o, _ = oracle.prefill(q, k, v, scale=0.5, window=1)
    np.testing.assert_allclose(o, v, atol=1e-15)


def test_gqa_head_mapping_is_floor_division():
    """Query head h reads kv head floor(h / G): make kv heads distinct and check directly."""
    B, S, Hkv, G, D = 1, 5, 3, 2, 4
    q = np.zeros((B, S, Hkv * G, D))
    k = np.zeros((B, S, Hkv, D))
    v = np.zeros((B, S, Hkv, D))
    for g in range(Hkv):
        v[0, :, g, :] = 10.0 * (g + 1)
    o, _ = oracle.prefill(q, k, v, scale=1.0)
    for h in range(Hkv * G):
        np.testing.assert_allclose(o[0, :, h, :], 10.0 * (h // G + 1))


# --- P2: the page's code listing -------------------------------------------------------

def test_listing_worked_example():
    """The oracle's r.E bias with a head-shared bank equals the hand-computed listing output."""
    fx = json.load(open(os.path.join(GOLDEN, "listing_bias_4tok.json")))
    rs = np.array(fx["relative_states"], dtype=np.float64)        # (T, H, C)
    proj = np.array(fx["proj"], dtype=np.float64)                  # (C, R_dist)
    expected = np.array(fx["expected_bias"], dtype=np.float64)     # (H, T, T)
    T, H, C = rs.shape
    E = np.broadcast_to(proj, (H,) + proj.shape)                   # shared bank: E[h] = proj
    for key in ("positions", "shifted_positions"):
        pos = np.array(fx[key])
        for h in range(H):
            beta = oracle.bias_matrix("rproj", pos, pos, proj.shape[1], h, r_rows=rs[:, h, :], E=E)
            np.testing.assert_array_equal(beta, expected[h])


def test_listing_worked_example_shared_bank():
    """Mode rproj_shared takes the listing's single bank as it stands ([R, range], no head axis)."""
    fx = json.load(open(os.path.join(GOLDEN, "listing_bias_4tok.json")))
    rs = np.array(fx["relative_states"], dtype=np.float64)        # (T, H, C)
    proj = np.array(fx["proj"], dtype=np.float64)                  # (C, R_dist)
    expected = np.array(fx["expected_bias"], dtype=np.float64)     # (H, T, T)
    pos = np.array(fx["positions"])
    for h in range(rs.shape[1]):
        beta = oracle.bias_matrix("rproj_shared", pos, pos, proj.shape[1], h, r_rows=rs[:, h, :], E=proj)
        np.testing.assert_array_equal(beta, expected[h])


def test_rproj_bias_through_sdpa_mask():
    """r.E bias + causal window, fed to torch SDPA as an additive mask, equals the oracle."""
    rng = _rng(7)
    B, S, Hq, Hkv, D, R, Rb, W = 1, 40, 4, 2, 8, 3, 12, 20
    q = rng.standard_normal((B, S, Hq, D))
    k = rng.standard_normal((B, S, Hkv, D))
    v = rng.standard_normal((B, S, Hkv, D))
    r = rng.standard_normal((B, S, Hq, R))
    E = rng.standard_normal((Hq, R, Rb))
    # bias written out element by element, independent of the oracle's vectorised form
    bias = np.zeros((Hq, S, S))
    for h in range(Hq):
        for i in range(S):
            for j in range(S):
                d = i - j
                if 0 <= d < Rb:
                    bias[h, i, j] = sum(r[0, i, h, f] * E[h, f, d] for f in range(R))
    ref = _sdpa_f64(q, k, v, scale=0.25, window=W, bias=bias)
    o, _ = oracle.prefill(q, k, v, scale=0.25, window=W, bias_range=Rb, mode="rproj", r=r, E=E)
    np.testing.assert_allclose(o, ref, atol=1e-12)


# --- P3: only the distance matters -------------------------------------------------------

@pytest.mark.parametrize("mode", ["table", "rproj"])
def test_translation_invariance(mode):
    rng = _rng(11)
    B, S, Hq, Hkv, D, R, Rb = 1, 30, 2, 1, 8, 4, 9
    q = rng.standard_normal((B, S, Hq, D))
    k = rng.standard_normal((B, S, Hkv, D))
    v = rng.standard_normal((B, S, Hkv, D))
    kw = dict(table=rng.standard_normal((Hq, Rb))) if mode == "table" else \
        dict(r=rng.standard_normal((B, S, Hq, R)), E=rng.standard_normal((Hq, R, Rb)))
    pos = np.arange(S)
    for W in (0, 11):
        o0, l0 = oracle.attention(q, k, v, qpos=pos, kpos=pos, scale=0.4, window=W,
                                  bias_range=Rb, mode=mode, **kw)
        o1, l1 = oracle.attention(q, k, v, qpos=pos + 1000, kpos=pos + 1000, scale=0.4, window=W,
                                  bias_range=Rb, mode=mode, **kw)
        np.testing.assert_allclose(o1, o0, atol=1e-13)
        np.testing.assert_allclose(l1, l0, atol=1e-13)


# --- P4: ALiBi closed form ------------------------------------------------------------------

def _alibi_closed_form(i, m):
    """o_i = sum_j j x^(i-j) / sum_j x^(i-j), x = e^-m, summed in closed form (geometric series)."""
    x = math.exp(-m)
    return i - x * (1 - (i + 1) * x ** i + i * x ** (i + 1)) / ((1 - x) * (1 - x ** (i + 1)))


def test_alibi_closed_form():
    """Table b_delta = -m*delta over the whole causal range, zero content, v_j = j."""
    S, H = 24, 4
    slopes = [2.0 ** (-8.0 * (h + 1) / H) for h in range(H)] + [0.5]
    H = len(slopes)
    q = np.zeros((1, S, H, 1))
    k = np.zeros((1, S, H, 1))
    v = np.arange(S, dtype=np.float64).reshape(1, S, 1, 1).repeat(H, axis=2)
    table = np.array([[-m * d for d in range(S)] for m in slopes])
    o, _ = oracle.prefill(q, k, v, scale=1.0, bias_range=S, mode="table", table=table)
    for h, m in enumerate(slopes):
        for i in range(S):
            # the closed form cancels (1 - x is small for gentle slopes): 1e-9 is its own accuracy
            assert abs(o[0, i, h, 0] - _alibi_closed_form(i, m)) < 1e-9
    # spot values of the closed form at m = 0.5 (rounded to 7 decimals)
    assert round(_alibi_closed_form(1, 0.5), 7) == 0.6224593
    assert round(_alibi_closed_form(3, 0.5), 7) == 2.0845765
    assert round(_alibi_closed_form(10, 0.5), 7) == 8.5036449


# --- P5: NoPE tail: keys beyond the bias range are a set --------------------------------------

@pytest.mark.parametrize("mode", ["table", "rproj"])
def test_nope_tail_permutation(mode):
    """Permuting K/V among keys >= bias_range before every query leaves the output unchanged."""
    rng = _rng(21)
    B, S, Hq, Hkv, D, R, Rb = 1, 64, 2, 1, 8, 3, 10
    q = rng.standard_normal((B, S, Hq, D))
    k = rng.standard_normal((B, S, Hkv, D))
    v = rng.standard_normal((B, S, Hkv, D))
    kw = dict(table=rng.standard_normal((Hq, Rb)) * 3) if mode == "table" else \
        dict(r=rng.standard_normal((B, S, Hq, R)), E=rng.standard_normal((Hq, R, Rb)))
    rows = np.arange(40, S)                      # query set, min position 40
    far = np.arange(0, 40 - Rb + 1)              # keys with i - j >= Rb for every row
    o0, l0 = oracle.prefill(q, k, v, scale=0.3, bias_range=Rb, mode=mode, rows=rows, **kw)
    perm = np.arange(S)
    perm[far] = rng.permutation(far)
    o1, l1 = oracle.prefill(q, k[:, perm], v[:, perm], scale=0.3, bias_range=Rb, mode=mode,
                            rows=rows, **kw)
    np.testing.assert_allclose(o1, o0, atol=1e-12)
    np.testing.assert_allclose(l1, l0, atol=1e-12)
    # negative control: moving keys that lie inside the bias range changes the output
    near = np.arange(40 - Rb + 1, 40)
    perm2 = np.arange(S)
    perm2[near] = near[::-1]
    o2, _ = oracle.prefill(q, k[:, perm2], v[:, perm2], scale=0.3, bias_range=Rb, mode=mode,
                           rows=rows, **kw)
    assert np.abs(o2 - o0).max() > 1e-6


# --- P6: hand-derived 4-token cases -----------------------------------------------------------

def _num(x):
    if isinstance(x, list) and x[0] == "ln":
        return math.log(x[1])
    return float(x)


@pytest.mark.parametrize("case", json.load(open(os.path.join(GOLDEN, "hand_cases_4tok.json")))["cases"],
                         ids=lambda c: c["name"])
def test_hand_cases(case):
    T = 4
    q = np.array([_num(x) for x in case["q"]]).reshape(1, T, 1, 1)
    k = np.array([_num(x) for x in case["k"]]).reshape(1, T, 1, 1)
    v = np.array([1.0, 2.0, 4.0, 8.0]).reshape(1, T, 1, 1)
    kw = {}
    if case["mode"] == "table":
        kw["table"] = np.array([[_num(x) for x in case["table"]]])
    elif case["mode"] == "rproj":
        kw["E"] = np.array([[[_num(x) for x in row] for row in case["E"]]])
        kw["r"] = np.array(case["r"], dtype=np.float64).reshape(1, T, 1, -1)
    o, lse = oracle.prefill(q, k, v, scale=case["scale"], window=case["window"],
                            bias_range=case["bias_range"], mode=case["mode"], **kw)
    want = np.array([a / b for a, b in case["expected"]])
    np.testing.assert_allclose(o[0, :, 0, 0], want, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse[0, 0], np.log(case["expected_weight_sum"]), atol=1e-13)


# --- P7: brute force on tiny inputs ----------------------------------------------------------

def _brute(q, k, v, qpos, kpos, scale, window, Rb, mode, table, r, E):
    """Pure-Python double loop of the definition (independent of the vectorised oracle)."""
    B, Sq, Hq, D = q.shape
    G = Hq // k.shape[2]
    o = np.zeros(q.shape)
    lse = np.zeros((B, Hq, Sq))
    for b in range(B):
        for h in range(Hq):
            g = h // G
            for i in range(Sq):
                scores, vals = [], []
                for j in range(k.shape[1]):
                    d = int(qpos[i]) - int(kpos[j])
                    if d < 0 or (window and d >= window):
                        continue
                    s = scale * sum(q[b, i, h, t] * k[b, j, g, t] for t in range(D))
                    if mode != "none" and d < Rb:
                        if mode == "table":
                            s += table[h, d]
                        elif mode == "rproj_shared":        # one bank E[f, d] for every head
                            s += sum(r[b, i, h, f] * E[f, d] for f in range(E.shape[0]))
                        else:
                            s += sum(r[b, i, h, f] * E[h, f, d] for f in range(E.shape[1]))
                    scores.append(s)
                    vals.append(v[b, j, g, :])
                mx = max(scores)
                w = [math.exp(s - mx) for s in scores]
                tot = sum(w)
                o[b, i, h, :] = sum(wi * vi for wi, vi in zip(w, vals)) / tot
                lse[b, h, i] = mx + math.log(tot)
    return o, lse


@pytest.mark.parametrize("seed,mode,W,Rb,G", [
    (s, m, W, Rb, G) for s, (m, W, Rb, G) in enumerate(itertools.product(
        ["none", "table", "rproj", "rproj_shared"], [0, 1, 5], [1, 4, 40], [1, 3]))])
def test_bruteforce_small(seed, mode, W, Rb, G):
    rng = _rng(100 + seed)
    B, S, Hkv, D, R = 2, 13, 1, 3, 2
    Hq = Hkv * G
    q = rng.standard_normal((B, S, Hq, D))
    k = rng.standard_normal((B, S, Hkv, D))
    v = rng.standard_normal((B, S, Hkv, D))
    table = rng.standard_normal((Hq, Rb))
    r = rng.standard_normal((B, S, Hq, R))
    E = rng.standard_normal((Hq, R, Rb) if mode != "rproj_shared" else (R, Rb))
    pos = np.arange(S) + 5
    o, lse = oracle.attention(q, k, v, qpos=pos, kpos=pos, scale=0.7, window=W, bias_range=Rb,
                              mode=mode, table=table, r=r, E=E)
    ob, lb = _brute(q, k, v, pos, pos, 0.7, W, Rb, mode, table, r, E)
    np.testing.assert_allclose(o, ob, atol=1e-12)
    np.testing.assert_allclose(lse, lb, atol=1e-12)


@pytest.mark.parametrize("mode,W,Rb", [("rproj", 0, 6), ("table", 7, 7), ("none", 4, 1),
                                       ("rproj_shared", 9, 5)])
def test_decode_matches_bruteforce(mode, W, Rb):
    """Decode: one query at position kv_len-1 against cache rows [0, kv_len)."""
    rng = _rng(5)
    B, L, Lmax, Hq, Hkv, D, R = 3, 17, 20, 4, 2, 5, 3
    q = rng.standard_normal((B, Hq, D))
    kc = rng.standard_normal((B, Lmax, Hkv, D))
    vc = rng.standard_normal((B, Lmax, Hkv, D))
    r = rng.standard_normal((B, Hq, R))
    E = rng.standard_normal((Hq, R, Rb) if mode != "rproj_shared" else (R, Rb))
    table = rng.standard_normal((Hq, Rb))
    o, lse = oracle.decode(q, kc, vc, L, scale=0.45, window=W, bias_range=Rb, mode=mode,
                           table=table, r=r, E=E)
    ob, lb = _brute(q[:, None], kc[:, :L], vc[:, :L], [L - 1], np.arange(L), 0.45, W, Rb, mode,
                    table, r[:, None], E)
    np.testing.assert_allclose(o, ob[:, 0], atol=1e-12)
    np.testing.assert_allclose(lse, lb[:, :, 0], atol=1e-12)


def test_bias_zero_at_range_boundary():
    """At delta == bias_range the bias is exactly 0 (hard cut-off), at bias_range - 1 it is not."""
    Rb = 6
    table = np.arange(1, Rb + 1, dtype=np.float64)[None, :]
    pos = np.arange(10)
    beta = oracle.bias_matrix("table", pos, pos, Rb, 0, table=table)
    for i in range(10):
        for j in range(10):
            d = i - j
            assert beta[i, j] == (d + 1 if 0 <= d < Rb else 0.0)


# --- P9: context-length temperature ---------------------------------------------------------
# "Thinking Machines dropped RoPE", section "The temperature scale is dependent on context
# length": global layers multiply the queries and the position bias by a factor of the number
# of keys the query sees, flat up to a threshold and logarithmic beyond (log-n scaling).

def test_temperature_values():
    """tau = 1 up to the threshold T, then log base T of n: tau(T^k) = k, tau(T^(k/2)) = k/2."""
    T = 4
    n = np.array([1, 2, 3, 4, 8, 16, 32, 64, 256])
    np.testing.assert_allclose(oracle.temperature(n, T), [1, 1, 1, 1, 1.5, 2, 2.5, 3, 4],
                               rtol=1e-15)
    np.testing.assert_array_equal(oracle.temperature(n, 0), np.ones(len(n)))
    big = oracle.temperature([131072, 131073, 131072 ** 2], 131072)
    assert big[0] == 1.0 and 1.0 < big[1] < 1.0 + 1e-5
    assert big[2] == pytest.approx(2.0, rel=1e-14)


@pytest.mark.parametrize("window", [0, 16])
def test_temperature_equal_logits_closed_form(window):
    """Equal visible logits L give lse = tau(n) * L + ln n; tau multiplies content and bias."""
    S, T = 64, 4
    q = np.ones((1, S, 1, 1))
    k = np.ones((1, S, 1, 1))
    v = _rng(31).standard_normal((1, S, 1, 1))
    table = np.full((1, S), 0.25)                      # bias 0.25 at every distance
    _, lse = oracle.prefill(q, k, v, scale=0.5, bias_range=S, mode="table", table=table,
                            window=window, temp_len=T)
    L = 0.5 * 1.0 + 0.25
    tau_of = {1: 1.0, 2: 1.0, 4: 1.0, 8: 1.5, 16: 2.0, 32: 2.5, 64: 3.0}
    checked = 0
    for i in range(S):
        n = min(i + 1, window) if window else i + 1
        if n in tau_of:
            assert abs(lse[0, 0, i] - (tau_of[n] * L + math.log(n))) < 1e-12, (i, n)
            checked += 1
    assert checked >= 5
    # content only (no bias): the factor reaches the q.k term alone
    _, lse0 = oracle.prefill(q, k, v, scale=0.5, window=window, temp_len=T)
    i = 63
    n = min(i + 1, window) if window else i + 1
    assert abs(lse0[0, 0, i] - (tau_of[n] * 0.5 + math.log(n))) < 1e-12


@pytest.mark.parametrize("mode,window", [("table", 20), ("rproj", 0), ("rproj_shared", 9)])
def test_temperature_is_query_and_bias_scaling(mode, window):
    """torch SDPA with each query row and its bias row multiplied by tau(n_i) gives the oracle's
    tempered attention (the page's description: queries and position bias scaled by tau)."""
    rng = _rng(41)
    B, S, Hq, Hkv, D, R, Rb, T = 1, 48, 2, 1, 8, 3, 12, 5
    q = rng.standard_normal((B, S, Hq, D))
    k = rng.standard_normal((B, S, Hkv, D))
    v = rng.standard_normal((B, S, Hkv, D))
    table = rng.standard_normal((Hq, Rb))
    r = rng.standard_normal((B, S, Hq, R))
    E = rng.standard_normal((R, Rb) if mode == "rproj_shared" else (Hq, R, Rb))
    o, lse = oracle.prefill(q, k, v, scale=0.4, window=window, bias_range=Rb, mode=mode,
                            table=table, r=r, E=E, temp_len=T)
    # bias built here by direct indexing, independent of the oracle's bias_matrix
    bias = np.zeros((Hq, S, S))
    for h in range(Hq):
        for i in range(S):
            for j in range(max(0, i - Rb + 1), i + 1):
                d = i - j
                if mode == "table":
                    bias[h, i, j] = table[h, d]
                else:
                    bank = E if mode == "rproj_shared" else E[h]
                    bias[h, i, j] = float(r[0, i, h] @ bank[:, d])
    n = np.arange(1, S + 1)
    if window:
        n = np.minimum(n, window)
    tau = np.array([max(1.0, math.log(x) / math.log(T)) for x in n])
    ref = _sdpa_f64(q * tau[None, :, None, None], k, v, scale=0.4, window=window,
                    bias=bias * tau[None, :, None])
    np.testing.assert_allclose(o, ref, atol=1e-12)
    assert np.abs(tau - 1).max() > 0.3          # the case reaches well past the threshold
    # negative control: without the temperature the result differs
    o_flat, _ = oracle.prefill(q, k, v, scale=0.4, window=window, bias_range=Rb, mode=mode,
                               table=table, r=r, E=E)
    assert np.abs(o_flat - o).max() > 1e-3


def test_temperature_flat_below_threshold_and_decode():
    """A threshold at or above every visible count changes nothing; decode tempers like the
    last prefill row (the query sees kv_len keys, or the window)."""
    rng = _rng(43)
    B, S, Hq, Hkv, D, Rb = 2, 30, 4, 2, 6, 9
    q = rng.standard_normal((B, S, Hq, D))
    k = rng.standard_normal((B, S, Hkv, D))
    v = rng.standard_normal((B, S, Hkv, D))
    table = rng.standard_normal((Hq, Rb))
    kw = dict(scale=0.5, bias_range=Rb, mode="table", table=table)
    o0, l0 = oracle.prefill(q, k, v, **kw)
    o1, l1 = oracle.prefill(q, k, v, temp_len=S, **kw)
    np.testing.assert_array_equal(o0, o1)
    np.testing.assert_array_equal(l0, l1)
    for W in (0, 11):
        op, lp = oracle.prefill(q, k, v, window=W, temp_len=3, **kw)
        od, ld = oracle.decode(q[:, -1], k, v, S, window=W, temp_len=3, **kw)
        np.testing.assert_allclose(od, op[:, -1], atol=1e-13)
        np.testing.assert_allclose(ld, lp[:, :, -1], atol=1e-13)
