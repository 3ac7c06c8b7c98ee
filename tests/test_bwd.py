"""GPU parity of the backward pass: the HIP library (through its C ABI) against the float64
oracle's gradients (oracle.prefill_backward), on the same seeded inputs.

The library's forward provides o and lse; the oracle recomputes everything in float64 from
q, k, v, dout and the bias parameters.  Bar per gradient tensor: relative L2 error <= 5e-3 (the
forward's bar) and max |err| <= 2e-2 * max |reference|, with floors (RMS 1e-3, maximum 1e-2)
for references that vanish.  The kernels round P and dZ to bf16 before the MFMAs, and the
stored o enters rowsum(dout * o), each about 2^-9 relative; the bias reaches the recomputed
logits in fp32 (E as a bf16 high and low part).  dr takes 7.5e-3: its product adds two more
bf16 operands (E and the diagonal sums of dZ, each rounded once more), and with a sharp bias
(E at std 1.0) it measures about 5e-3.  The fp32 path (vector-ALU kernels, no bf16 rounding)
takes the forward's fp32 bar: 1e-5 relative L2 and 1e-5 of the largest reference element.
"""

import sys
import zlib

import numpy as np
import pytest
import torch

import oracle
import transformer_attention_learned_amd as rba
from transformer_attention_learned_amd.workloads import WORKLOADS, Workload, make_inputs

pytestmark = pytest.mark.gpu

REL_L2, REL_L2_DR, MAX_REL = 5e-3, 7.5e-3, 2e-2
# fp32 path: the fp32 bar of the forward (1e-5), relative L2 and max |err| / max |ref| alike;
# fp32 products and sums of a few hundred terms sit near 1e-7-1e-6
F32_REL = 1e-5


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    rba.load_library()


def _t2np(t):
    return t.detach().to("cpu", torch.float64).numpy()


def _dout(w, like):
    gen = torch.Generator(device=like.device)
    gen.manual_seed(w.seed + 7919)
    return torch.randn(like.shape, generator=gen, device=like.device,
                       dtype=torch.float32).to(like.dtype)


def run_bwd(w: Workload, inp, dout):
    o, lse = rba.fwd(inp["q"], inp["k"], inp["v"], window=w.window, bias_range=w.bias_range,
                     mode=w.mode, table=inp["table"], r=inp["r"], E=inp["E"], scale=w.scale,
                     temp_len=w.temp_len, return_lse=True)
    g = rba.bwd(inp["q"], inp["k"], inp["v"], o, lse, dout, window=w.window,
                bias_range=w.bias_range, mode=w.mode, table=inp["table"], r=inp["r"], E=inp["E"],
                scale=w.scale, temp_len=w.temp_len)
    torch.cuda.synchronize()
    return g


def compare(name, got, ref, f32=False):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    # floors for references that vanish (dq, dk and the bias gradients when every row sees a
    # single key, where dS is zero up to rounding): an RMS of 1e-3 per element and a maximum of
    # 1e-2 for bf16.  fp32: there dZ = P (dP - rowsum) cancels two fp32 sums of D products of
    # size about 1 taken in different orders, a residue of about 2^-24 D (1-3e-6 at D = 32) per
    # element, times scale * k in dq and dk and times r or E (up to about 3) in dE and dr; the
    # floors (RMS 1e-1, maximum 1) allow 1e-6 RMS and 1e-5 at most against such a vanishing
    # reference at the 1e-5 bar
    floor_rms, floor_max = (1e-1, 1.0) if f32 else (1e-3, 1e-2)
    scale = max(float(np.abs(ref).max()), floor_max)
    max_rel = float(np.abs(got - ref).max()) / scale
    rel = float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), floor_rms * np.sqrt(ref.size)))
    _say(f"    {name}: rel_l2={rel:.3e} max_err/max_ref={max_rel:.3e}")
    if f32:
        assert rel <= F32_REL and max_rel <= F32_REL, (name, rel, max_rel)
    else:
        bar = REL_L2_DR if name.startswith("dr") else REL_L2
        assert rel <= bar and max_rel <= MAX_REL, (name, rel, max_rel)


def check_bwd(w: Workload, heads=None):
    """heads: optional list of kv heads whose slice the oracle evaluates (all when None)."""
    _say(f"  bwd case {w.name}: B={w.B} S={w.S} Hq={w.Hq} Hkv={w.Hkv} D={w.D} W={w.window} "
         f"Rb={w.bias_range} mode={w.mode} R={w.R} temp_len={w.temp_len} seed={w.seed}")
    inp = make_inputs(w, device="cuda")
    dout = _dout(w, inp["q"])
    g = run_bwd(w, inp, dout)
    G = w.Hq // w.Hkv
    kvs = list(range(w.Hkv)) if heads is None else heads
    shared = w.mode == "rproj_shared"
    dE_ref = None
    for hk in kvs:
        hs = slice(hk * G, (hk + 1) * G)
        sub = lambda t: None if t is None else t[:, :, hs].contiguous()
        ref = oracle.prefill_backward(
            sub(inp["q"]), inp["k"][:, :, hk:hk + 1].contiguous(),
            inp["v"][:, :, hk:hk + 1].contiguous(), sub(dout), scale=w.scale, window=w.window,
            bias_range=w.bias_range, mode=w.mode,
            table=None if inp["table"] is None else inp["table"][hs],
            r=sub(inp["r"]),
            E=None if inp["E"] is None else (inp["E"] if shared else inp["E"][hs]),
            temp_len=w.temp_len)
        f32 = w.dtype == "f32"
        compare(f"dq[kv {hk}]", _t2np(g["dq"][:, :, hs]), ref["dq"], f32)
        compare(f"dk[kv {hk}]", _t2np(g["dk"][:, :, hk:hk + 1]), ref["dk"], f32)
        compare(f"dv[kv {hk}]", _t2np(g["dv"][:, :, hk:hk + 1]), ref["dv"], f32)
        if w.mode == "table":
            compare(f"dtable[kv {hk}]", _t2np(g["dtable"][hs]), ref["dtable"], f32)
        if w.mode in ("rproj", "rproj_shared"):
            compare(f"dr[kv {hk}]", _t2np(g["dr"][:, :, hs]), ref["dr"], f32)
            if shared:
                dE_ref = ref["dE"] if dE_ref is None else dE_ref + ref["dE"]
            else:
                compare(f"dE[kv {hk}]", _t2np(g["dE"][hs]), ref["dE"], f32)
    if shared and heads is None:
        compare("dE (shared bank)", _t2np(g["dE"]), dE_ref, w.dtype == "f32")


def small(**kw):
    base = dict(kind="prefill", dtype="bf16", B=1, Hq=4, Hkv=1, D=128, S=200, window=0,
                bias_range=64, mode="rproj", R=8, seed=0, rmsnorm_qk=True)
    base.update(kw)
    name = "bwd_" + "_".join(f"{k}{v}" for k, v in kw.items())
    return Workload(name=name, **base)


SWEEP = [
    dict(S=1), dict(S=63), dict(S=64), dict(S=65), dict(S=200), dict(S=700),
    dict(S=300, mode="none"), dict(S=333, mode="table", bias_range=100),
    dict(S=333, mode="table", window=130, bias_range=77), dict(S=300, window=64, bias_range=64),
    dict(S=700, window=512, bias_range=512, Hq=8, Hkv=2), dict(S=1100, bias_range=1024),
    dict(S=257, Hq=8, Hkv=2), dict(S=150, B=2, Hq=4, Hkv=2), dict(S=129, Hq=3, Hkv=3),
    dict(S=260, D=64), dict(S=260, D=64, mode="table", window=100),
    dict(S=129, R=3), dict(S=129, R=16), dict(S=300, window=1), dict(S=300, bias_range=1),
    dict(S=700, mode="rproj_shared", R=16, window=512, bias_range=512, Hq=8, Hkv=2,
         logit_scale="inv_d"),
    dict(S=400, mode="rproj_shared", R=5, bias_range=77, D=64),
    dict(S=1000, temp_len=100), dict(S=333, mode="table", bias_range=100, temp_len=2),
    dict(S=600, window=300, temp_len=64, mode="rproj_shared", R=8),
    # table mode with GQA groups of several heads (the dk/dv kernel stages each head's row as
    # its walk reaches it), with a window and a temperature, and with 4,200 distances
    dict(S=333, mode="table", bias_range=100, Hq=8, Hkv=2),
    dict(S=500, mode="table", window=200, bias_range=150, Hq=4, Hkv=1, temp_len=64),
    dict(S=300, mode="table", bias_range=4200, Hq=8, Hkv=1, D=64),
    # the tile rings at their smallest: one 32-row tile per head (the dk/dv kernel's head, and
    # with it the staged table row, changes every step), two tiles, a window narrower than a tile
    dict(S=20, mode="table", bias_range=30, Hq=4, Hkv=1),
    dict(S=40, mode="table", window=8, bias_range=16, Hq=8, Hkv=2),
    dict(S=33, mode="rproj", window=5, bias_range=40, Hq=4, Hkv=1),
    dict(S=96, mode="none", window=40, Hq=3, Hkv=1, D=64),
    dict(S=70, mode="rproj", R=16, D=64, Hq=4, Hkv=2, temp_len=16),
]


# Sharp input-dependent biases (E drawn with std 0.5 and 1.0: a bias RMS of about 1.4 and 2.8 at
# R = 8), the per-token sharp locality the input-dependent form is for ("Thinking Machines
# dropped RoPE", the paragraph after the code listing); a table drawn with std 3 as the control.
SHARP = [
    dict(S=1100, Hq=8, Hkv=2, window=512, bias_range=512, e_std=0.5),
    dict(S=1100, Hq=8, Hkv=2, window=512, bias_range=512, e_std=1.0),
    dict(S=1300, bias_range=1024, e_std=1.0),
    dict(S=700, mode="rproj_shared", R=16, window=512, bias_range=512, e_std=1.0, Hq=8, Hkv=2,
         logit_scale="inv_d"),
    dict(S=600, window=300, bias_range=200, e_std=1.0, R=11, Hq=6, Hkv=2),
    dict(S=600, mode="table", bias_range=300, table_std=3.0),
]


@pytest.mark.parametrize("kw", SHARP, ids=lambda kw: "-".join(f"{k}{v}" for k, v in kw.items()))
def test_bwd_sharp_bias(kw):
    check_bwd(small(seed=zlib.crc32(repr(sorted(kw.items())).encode()) % 10007, **kw))


@pytest.mark.parametrize("kw", SWEEP, ids=lambda kw: "-".join(f"{k}{v}" for k, v in kw.items()))
def test_bwd_small(kw):
    check_bwd(small(seed=zlib.crc32(repr(sorted(kw.items())).encode()) % 10007, **kw))


def test_bwd_local_layer_slice():
    """The local-layer shape (window 512, r.E bias over 512 distances, GQA 4) at full length;
    the oracle evaluates one kv-head group (its 4 query heads)."""
    w = WORKLOADS["local_prefill"].with_(B=1, name="bwd_local_slice")
    check_bwd(w, heads=[3])


def test_bwd_global_layer_shape():
    """A global-layer shape: full causal, r.E bias over 1024 distances then content only."""
    w = WORKLOADS["global_prefill"].with_(S=4096, name="bwd_global_4k", temp_len=0)
    check_bwd(w, heads=[0, 5])


def test_bwd_deterministic_dq_dk_dv():
    w = small(S=700, window=300, bias_range=200, Hq=8, Hkv=2)
    inp = make_inputs(w, device="cuda")
    dout = _dout(w, inp["q"])
    g1 = run_bwd(w, inp, dout)
    g2 = run_bwd(w, inp, dout)
    for n in ("dq", "dk", "dv", "dr"):
        assert torch.equal(g1[n], g2[n]), n


@pytest.mark.parametrize("R,D", [(8, 128), (16, 64)])
def test_bwd_r_load_paths(R, D):
    """With R = 8 or 16 and r 16-byte aligned, a lane reads its row's 8 features of r in one
    16-byte load; an r two bytes past such a boundary takes the 2-byte loads.  The features,
    hence the gradients, are the same either way (dE up to the order of its atomics)."""
    w = small(S=300, R=R, D=D, window=128, bias_range=160, Hq=4, Hkv=2)
    inp = make_inputs(w, device="cuda")
    dout = _dout(w, inp["q"])
    r = inp["r"]
    assert r.data_ptr() % 16 == 0
    buf = torch.empty(r.numel() + 8, dtype=r.dtype, device=r.device)
    r_off = buf[1:1 + r.numel()].view(r.shape)
    r_off.copy_(r)
    assert r_off.data_ptr() % 16 == 2
    g0 = run_bwd(w, inp, dout)
    g1 = run_bwd(w, dict(inp, r=r_off), dout)
    for n in ("dq", "dk", "dv", "dr"):
        assert torch.equal(g0[n], g1[n]), n
    torch.testing.assert_close(g0["dE"], g1["dE"], rtol=1e-5, atol=1e-6)


# fp32 backward: the vector-ALU kernels against the same oracle at the fp32 bar
F32_SWEEP = [
    dict(S=1), dict(S=33), dict(S=200), dict(S=200, mode="none"),
    dict(S=200, mode="table", bias_range=50), dict(S=300, mode="table", window=70, bias_range=40),
    dict(S=200, D=64, Hq=4, Hkv=2), dict(S=130, D=128, R=16, Hq=2, Hkv=1),
    dict(S=250, mode="rproj_shared", R=5, bias_range=77, window=100, Hq=4, Hkv=2,
         logit_scale="inv_d"),
    dict(S=300, temp_len=64, window=150, bias_range=100), dict(S=200, e_std=1.0),
    dict(S=120, bias_range=1),
    # the block's staged distances straddle the end of the range (33) with 16 E rows, and a
    # table longer than the sequence
    dict(S=161, R=16, bias_range=33, window=90, e_std=1.0),
    dict(S=100, mode="table", bias_range=300),
]


@pytest.mark.parametrize("kw", F32_SWEEP, ids=lambda kw: "-".join(f"{k}{v}" for k, v in kw.items()))
def test_bwd_f32(kw):
    base = dict(dtype="f32", D=32, Hq=2, Hkv=1)
    base.update(kw)
    check_bwd(small(seed=zlib.crc32(repr(sorted(base.items())).encode()) % 10007, **base))


def test_bwd_f32_tiny_layer():
    """The tiny fp32 local layer (window 64, table bias) end to end."""
    check_bwd(WORKLOADS["tiny_local_f32"].with_(name="bwd_tiny_f32"))


def test_bwd_f32_single_key_rows():
    """Window 1: every row sees only its own key, so P = 1, o = v and dZ = P (dP - rowsum) is zero;
    what the fp32 kernels return for dq, dk, dr and dE is the rounding of two fp32 dot products of
    length D, at most 2 gamma_D sum_d |dout v| per row (gamma_D = D 2^-24, the classical bound of
    a recursive fp32 sum), carried through each gradient's formula; dv is the group's summed dout."""
    w = small(dtype="f32", D=32, Hq=3, Hkv=1, B=2, S=97, window=1, seed=6545)
    inp = make_inputs(w, device="cuda")
    dout = _dout(w, inp["q"])
    g = run_bwd(w, inp, dout)
    q, k, v, do, r, E = (_t2np(t) for t in (inp["q"], inp["k"], inp["v"], dout, inp["r"], inp["E"]))
    G = w.Hq // w.Hkv
    vh = np.repeat(v, G, axis=2)                                   # [B, S, Hq, D]
    res = 2 * w.D * 2.0 ** -24 * np.abs(do * vh).sum(-1)           # |dZ| bound per (b, i, h)
    bound = {
        "dq": w.scale * res[..., None] * np.abs(np.repeat(k, G, axis=2)),
        "dk": w.scale * (res[..., None] * np.abs(q)).reshape(w.B, w.S, w.Hkv, G, w.D).sum(3),
        "dr": res[..., None] * np.abs(E[:, :, 0])[None, None],
    }
    dE_bound = np.zeros_like(E)
    dE_bound[:, :, 0] = np.einsum("bih,bihf->hf", res, np.abs(r))
    for name in ("dq", "dk", "dr"):
        got = np.abs(_t2np(g[name]))
        _say(f"    {name}: max |got| = {got.max():.3e}, max bound = {bound[name].max():.3e}")
        assert np.all(got <= 1.01 * bound[name] + 1e-30), name
    gE = np.abs(_t2np(g["dE"]))
    _say(f"    dE: max |got| = {gE.max():.3e}, max bound = {dE_bound.max():.3e}")
    assert np.all(gE <= 1.01 * dE_bound + 1e-30)
    compare("dv", _t2np(g["dv"]), do.reshape(w.B, w.S, w.Hkv, G, w.D).sum(3), f32=True)
