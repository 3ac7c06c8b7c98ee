"""GPU parity of the backward pass: the HIP library (through its C ABI) against the float64
oracle's gradients (oracle.prefill_backward), on the same seeded inputs.

The library's forward provides o and lse; the oracle recomputes everything in float64 from
q, k, v, dout and the bias parameters.  Bar for every gradient tensor: relative L2 error
<= 1e-2 and max |err| <= 2e-2 * max |reference| (bf16 rounding of P and dZ before the MFMAs,
and of the stored o in rowsum(dout * o), each about 2^-9 relative), with floors (RMS 1e-3,
maximum 1e-2) for references that vanish.
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

REL_L2, MAX_REL = 1e-2, 2e-2


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


def compare(name, got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    # floors for references that vanish (dq, dk and the bias gradients when every row sees a
    # single key, where dS is zero up to fp32 rounding): an RMS of 1e-3 per element, a
    # maximum of 1e-2
    scale = max(float(np.abs(ref).max()), 1e-2)
    max_rel = float(np.abs(got - ref).max()) / scale
    rel = float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-3 * np.sqrt(ref.size)))
    _say(f"    {name}: rel_l2={rel:.3e} max_err/max_ref={max_rel:.3e}")
    assert rel <= REL_L2 and max_rel <= MAX_REL, (name, rel, max_rel)


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
        compare(f"dq[kv {hk}]", _t2np(g["dq"][:, :, hs]), ref["dq"])
        compare(f"dk[kv {hk}]", _t2np(g["dk"][:, :, hk:hk + 1]), ref["dk"])
        compare(f"dv[kv {hk}]", _t2np(g["dv"][:, :, hk:hk + 1]), ref["dv"])
        if w.mode == "table":
            compare(f"dtable[kv {hk}]", _t2np(g["dtable"][hs]), ref["dtable"])
        if w.mode in ("rproj", "rproj_shared"):
            compare(f"dr[kv {hk}]", _t2np(g["dr"][:, :, hs]), ref["dr"])
            if shared:
                dE_ref = ref["dE"] if dE_ref is None else dE_ref + ref["dE"]
            else:
                compare(f"dE[kv {hk}]", _t2np(g["dE"][hs]), ref["dE"])
    if shared and heads is None:
        compare("dE (shared bank)", _t2np(g["dE"]), dE_ref)


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
]


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
