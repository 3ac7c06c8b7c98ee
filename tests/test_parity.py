"""GPU parity: the HIP library (through its C ABI) against the float64 oracle.

Every case draws seeded inputs on the GPU, runs the library, copies exactly
those inputs to the host and evaluates the oracle on them (all rows for small
cases; a deterministic row sample at the full workload sizes).

Bars: bf16 max |err| <= 2e-2 and relative L2 <= 5e-3; fp32 <= 1e-5 (both).
"""

import os
import sys
import zlib

import numpy as np
import pytest
import torch

import oracle
import transformer_attention_learned_amd as rba
from transformer_attention_learned_amd.workloads import WORKLOADS, Workload, make_inputs

pytestmark = pytest.mark.gpu

BF16_MAX_ABS, BF16_REL_L2 = 2e-2, 5e-3
# bf16 log-sum-exp: the row sum adds the bf16-rounded probabilities (each within the bf16 unit
# roundoff 2^-8 = 3.9e-3 relative), so ln l is off by at most 3.9e-3 when one term dominates;
# fp32 rounding and the bias's residual add under 1e-4
BF16_LSE_MAX_ABS = 5e-3
F32_TOL = 1e-5


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    rba.load_library()
    return torch.device("cuda:0")


def _errs(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape
    assert np.all(np.isfinite(got)), "non-finite output"
    max_abs = float(np.abs(got - ref).max()) if got.size else 0.0
    rel = float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30)) if got.size else 0.0
    return max_abs, rel


def assert_parity(got, ref, dtype, what=""):
    max_abs, rel = _errs(got, ref)
    _say(f"    parity {what}: max_abs={max_abs:.3e} rel_l2={rel:.3e}")
    if dtype == "f32":
        assert max_abs <= F32_TOL and rel <= F32_TOL, (what, max_abs, rel)
    else:
        assert max_abs <= BF16_MAX_ABS and rel <= BF16_REL_L2, (what, max_abs, rel)


def assert_lse(got, ref, dtype, what=""):
    """The log-sum-exp, in natural log units, to an absolute bar (its values are about 6, so a
    relative L2 bar would say little).

    On the bf16 path the row sum adds the bf16-rounded probabilities (the same ones the P.V
    product uses), each within 2^-8 relative, so lse is off by at most about 3.9e-3; the bar is
    BF16_LSE_MAX_ABS = 5e-3.  fp32: F32_TOL.
    """
    max_abs, rel = _errs(got, ref)
    _say(f"    lse {what}: max_abs={max_abs:.3e} rel_l2={rel:.3e}")
    if dtype == "f32":
        assert max_abs <= F32_TOL, (what, max_abs)
    else:
        assert max_abs <= BF16_LSE_MAX_ABS, (what, max_abs)


def _t2np(t):
    return t.detach().to("cpu", torch.float64).numpy()


def run_prefill(w: Workload, inp):
    return rba.fwd(inp["q"], inp["k"], inp["v"], window=w.window, bias_range=w.bias_range,
                   mode=w.mode, table=inp["table"], r=inp["r"], E=inp["E"], scale=w.scale,
                   temp_len=w.temp_len, return_lse=True)


def check_prefill(w: Workload, rows=None, dev="cuda:0"):
    _say(f"  case {w.name}: B={w.B} S={w.S} Hq={w.Hq} Hkv={w.Hkv} D={w.D} W={w.window} "
         f"Rb={w.bias_range} mode={w.mode} dtype={w.dtype} seed={w.seed}")
    inp = make_inputs(w, device=dev)
    o, lse = run_prefill(w, inp)
    torch.cuda.synchronize()
    ref_o, ref_lse = oracle.prefill(inp["q"], inp["k"], inp["v"], scale=w.scale,
                                    temp_len=w.temp_len, window=w.window,
                                    bias_range=w.bias_range, mode=w.mode, table=inp["table"],
                                    r=inp["r"], E=inp["E"], rows=rows)
    if rows is None:
        got_o, got_lse = _t2np(o), _t2np(lse)
    else:
        idx = torch.as_tensor(rows, device=o.device)
        got_o, got_lse = _t2np(o[:, idx]), _t2np(lse[:, :, idx])
    assert_parity(got_o, ref_o, w.dtype, w.name)
    assert_lse(got_lse, ref_lse, w.dtype, w.name)
    return o


def small(**kw):
    base = dict(kind="prefill", dtype="bf16", B=1, Hq=4, Hkv=1, D=128, S=200, window=0,
                bias_range=64, mode="rproj", R=8, seed=0, rmsnorm_qk=True)
    base.update(kw)
    name = "small_" + "_".join(f"{k}{v}" for k, v in kw.items())
    return Workload(name=name, **base)


# --- small prefill sweep: tile edges, ragged tails, window / range boundaries -------------

SWEEP = [
    dict(S=1), dict(S=4), dict(S=63), dict(S=64), dict(S=65), dict(S=127), dict(S=1000),
    dict(S=300, window=1), dict(S=300, window=2), dict(S=300, window=63), dict(S=300, window=64),
    dict(S=300, window=65), dict(S=700, window=512, bias_range=512),
    dict(S=300, bias_range=1), dict(S=300, bias_range=64), dict(S=1200, bias_range=1024),
    dict(S=200, mode="none"), dict(S=333, mode="table", bias_range=100),
    dict(S=333, mode="table", window=130, bias_range=77),
    dict(S=257, Hq=8, Hkv=2), dict(S=257, Hq=2, Hkv=1), dict(S=257, Hq=3, Hkv=3),
    dict(S=190, Hq=8, Hkv=1, window=37, bias_range=20), dict(S=150, B=2, Hq=4, Hkv=2),
    dict(S=260, D=64), dict(S=260, D=64, mode="table", window=100),
    dict(S=129, R=3), dict(S=129, R=16), dict(S=129, R=11, window=50),
    dict(S=500, mode="rproj", window=96, bias_range=40, Hq=4, Hkv=4),
    # one bank shared by every head, the essay's form: R = 16 curves, logits scaled by 1/d
    dict(S=700, mode="rproj_shared", R=16, window=512, bias_range=512, Hq=8, Hkv=2,
         logit_scale="inv_d"),
    dict(S=1100, mode="rproj_shared", R=16, bias_range=1024, logit_scale="inv_d"),
    dict(S=333, mode="rproj_shared", R=5, window=130, bias_range=77, D=64),
    # context-length temperature past a small threshold: rows that see more than temp_len
    # keys have their logits (content and bias) sharpened by ln n / ln temp_len
    dict(S=1000, temp_len=100), dict(S=700, window=512, bias_range=512, temp_len=64),
    dict(S=333, mode="table", bias_range=100, temp_len=2),
    dict(S=1100, mode="rproj_shared", R=16, bias_range=1024, logit_scale="inv_d", temp_len=256),
    dict(S=260, D=64, temp_len=50), dict(S=190, Hq=6, Hkv=2, temp_len=20, mode="table"),
    # windows and ranges off the 32-key step grid, larger than the sequence, or equal (every
    # visible key in band: the branch-free r.E path with its first steps cut by the window)
    dict(S=300, window=1000, bias_range=2000), dict(S=333, window=100, bias_range=100),
    dict(S=333, window=33, bias_range=40, mode="table"), dict(S=290, window=95, bias_range=95, R=16),
    dict(S=450, window=200, bias_range=31), dict(S=450, window=200, bias_range=33, mode="none"),
    # table ranges too long for the split kernel's LDS take the generic kernel (table rows read
    # from global memory)
    dict(S=2200, mode="table", bias_range=2048, Hq=8, Hkv=2),
    dict(S=2200, mode="table", window=600, bias_range=2048, Hq=8, Hkv=2),
    # the generic kernel without bias: head_dim 128 with a GQA ratio of 2, head_dim 64
    dict(S=200, mode="none", Hq=2, Hkv=1), dict(S=260, D=64, mode="none", window=90),
    # windows inside the bias range with more work items (batch x head group x 64-row tile)
    # than CUs: the kernel walks runs of items per workgroup, runs cross head groups and batch
    # entries, tails are ragged
    dict(S=1000, B=3, Hq=32, Hkv=8, window=300, bias_range=512),
    dict(S=700, B=4, Hq=32, Hkv=8, R=16, window=512, bias_range=512, temp_len=300),
]


@pytest.mark.parametrize("kw", SWEEP, ids=lambda kw: "-".join(f"{k}{v}" for k, v in kw.items()))
def test_prefill_small(kw):
    check_prefill(small(seed=zlib.crc32(repr(sorted(kw.items())).encode()) % 10007, **kw))


# Sharp input-dependent biases: E drawn at std 0.5 and 1.0 (a bias RMS of about 1.4 and 2.8 at
# R = 8), the per-token sharp locality the input-dependent form is for ("Thinking Machines
# dropped RoPE", the paragraph after the code listing: one token can demand sharp locality while
# the next reaches back through the whole window).  The kernels carry E as a bf16 high and low
# part and keep the formed curve in fp32, so these stay inside the bf16 bar; a table at std 3 is
# the control (the table path always reads fp32).
SHARP = [
    dict(S=1100, Hq=8, Hkv=2, window=512, bias_range=512, e_std=0.5),
    dict(S=1100, Hq=8, Hkv=2, window=512, bias_range=512, e_std=1.0),
    dict(S=1100, Hq=8, Hkv=2, window=512, bias_range=512, e_std=1.0, R=16),
    dict(S=1500, Hq=8, Hkv=2, bias_range=1024, e_std=0.5),
    dict(S=1500, Hq=8, Hkv=2, bias_range=1024, e_std=1.0),
    dict(S=1500, Hq=8, Hkv=2, bias_range=1024, e_std=1.0, R=16),
    dict(S=1300, mode="rproj_shared", R=16, bias_range=1024, e_std=1.0, logit_scale="inv_d"),
    dict(S=900, window=512, bias_range=512, e_std=1.0, D=64),
    dict(S=700, window=300, bias_range=200, e_std=1.0, R=11, Hq=6, Hkv=2),
    dict(S=1100, Hq=8, Hkv=2, mode="table", bias_range=1024, table_std=3.0),
]


@pytest.mark.parametrize("kw", SHARP, ids=lambda kw: "-".join(f"{k}{v}" for k, v in kw.items()))
def test_prefill_sharp_bias(kw):
    check_prefill(small(seed=zlib.crc32(repr(sorted(kw.items())).encode()) % 10007, **kw))


@pytest.mark.parametrize("kw", [dict(S=200, mode="table", bias_range=40, window=50),
                                dict(S=130, mode="rproj", R=5, bias_range=30),
                                dict(S=70, mode="none", Hq=4, Hkv=2, D=64),
                                dict(S=3, mode="table", bias_range=2, D=128),
                                dict(S=90, mode="rproj_shared", R=16, bias_range=33, window=60,
                                     logit_scale="inv_d"),
                                dict(S=150, mode="table", bias_range=40, window=70, temp_len=9)],
                         ids=["table", "rproj", "none_gqa", "tiny", "rproj_shared", "temp"])
def test_prefill_f32_small(kw):
    check_prefill(small(dtype="f32", rmsnorm_qk=False, **kw))


def test_prefill_f32_tiny_local_workload():
    check_prefill(WORKLOADS["tiny_local_f32"])


def test_prefill_empty():
    q = torch.empty((2, 0, 4, 128), dtype=torch.bfloat16, device="cuda")
    o = rba.fwd(q, q[:, :, :1].contiguous(), q[:, :, :1].contiguous())
    assert o.shape == q.shape


def test_prefill_deterministic():
    w = small(S=700, window=300, bias_range=200, Hq=8, Hkv=2)
    inp = make_inputs(w, device="cuda")
    o1, l1 = run_prefill(w, inp)
    o2, l2 = run_prefill(w, inp)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


# --- full workload sizes (row samples) ------------------------------------------------------

def _sample_rows(S, Rb, seed, n_edge=64, n_rand=64):
    rng = np.random.default_rng(seed)
    rows = set(range(min(S, n_edge)))
    rows |= set(range(max(0, Rb - 40), min(S, Rb + 40)))
    rows |= set(range(max(0, S - n_edge), S))
    rows |= set(rng.choice(S, size=min(S, n_rand), replace=False).tolist())
    return np.array(sorted(rows))


def test_local_prefill_workload():
    """Every output element of the local-layer workload against the full oracle."""
    check_prefill(WORKLOADS["local_prefill"])


def test_local_prefill_workload_sharp_bias():
    """The local-layer workload with E at std 1.0 (bias RMS about 2.8), row sample."""
    w = WORKLOADS["local_prefill"].with_(name="local_prefill_e1", e_std=1.0)
    check_prefill(w, rows=_sample_rows(w.S, w.bias_range, 2, n_edge=128, n_rand=256))


def test_global_prefill_workload_sharp_bias():
    """The global-layer workload with E at std 1.0, row sample."""
    w = WORKLOADS["global_prefill"].with_(name="global_prefill_e1", e_std=1.0)
    check_prefill(w, rows=_sample_rows(w.S, w.bias_range, 3, n_edge=32, n_rand=32))


def test_global_prefill_workload():
    w = WORKLOADS["global_prefill"]
    check_prefill(w, rows=_sample_rows(w.S, w.bias_range, 3, n_edge=48, n_rand=48))


def test_long_global_prefill_workload():
    w = WORKLOADS["long_global_prefill"]
    check_prefill(w, rows=_sample_rows(w.S, w.bias_range, 4, n_edge=32, n_rand=32))


# --- decode ----------------------------------------------------------------------------------

def run_decode(w: Workload, inp, kv_len):
    return rba.decode(inp["q"], inp["k"], inp["v"], kv_len, window=w.window,
                      bias_range=w.bias_range, mode=w.mode, table=inp["table"], r=inp["r"],
                      E=inp["E"], scale=w.scale, temp_len=w.temp_len, return_lse=True)


def check_decode(w: Workload, kv_len, batches=None, key_margin=None):
    _say(f"  case {w.name}: B={w.B} L_max={w.S} kv_len={kv_len} Hq={w.Hq} Hkv={w.Hkv} D={w.D} "
         f"W={w.window} Rb={w.bias_range} mode={w.mode} dtype={w.dtype} seed={w.seed}")
    inp = make_inputs(w, device="cuda")
    o, lse = run_decode(w, inp, kv_len)
    torch.cuda.synchronize()
    batches = list(range(w.B)) if batches is None else batches
    # keys before the window can not contribute; the oracle still sees `key_margin`
    # invisible rows before it so that the window edge is exercised
    k0 = 0
    if key_margin is not None and w.window:
        k0 = max(0, kv_len - w.window - key_margin)
    kpos = np.arange(k0, kv_len)
    for b in batches:
        qb = inp["q"][b:b + 1][:, None]
        kb = inp["k"][b:b + 1, k0:kv_len]
        vb = inp["v"][b:b + 1, k0:kv_len]
        rb = None if inp["r"] is None else inp["r"][b:b + 1][:, None]
        ro, rl = oracle.attention(qb, kb, vb, qpos=[kv_len - 1], kpos=kpos, scale=w.scale,
                                  temp_len=w.temp_len,
                                  window=w.window, bias_range=w.bias_range, mode=w.mode,
                                  table=inp["table"], r=rb, E=inp["E"])
        assert_parity(_t2np(o[b]), ro[0, 0], w.dtype, f"{w.name} b={b}")
        assert_lse(_t2np(lse[b]), rl[0, :, 0], w.dtype, f"{w.name} b={b}")


DEC_SWEEP = [
    dict(S=100, kv_len=1), dict(S=100, kv_len=5), dict(S=100, kv_len=63), dict(S=100, kv_len=64),
    dict(S=100, kv_len=65), dict(S=2000, kv_len=1000), dict(S=6000, kv_len=5000),
    dict(S=6000, kv_len=5000, window=100), dict(S=3000, kv_len=2999, window=1),
    dict(S=6000, kv_len=4100, bias_range=1024), dict(S=600, kv_len=600, mode="table", bias_range=70),
    dict(S=9000, kv_len=8191, mode="none", Hq=8, Hkv=8), dict(S=300, kv_len=260, Hq=16, Hkv=2, D=64),
    dict(S=3000, kv_len=2500, R=13, Hq=4, Hkv=4, window=700, bias_range=300),
    dict(S=3000, kv_len=2600, mode="rproj_shared", R=16, window=512, bias_range=512,
         logit_scale="inv_d"),
    dict(S=5000, kv_len=4500, mode="rproj_shared", R=8, bias_range=1024, Hq=32, Hkv=8),
    # groups of more than 16 query heads take the 32x32-MFMA kernel
    dict(S=3000, kv_len=2900, Hq=32, Hkv=1, window=700, bias_range=512),
    dict(S=2000, kv_len=1999, Hq=24, Hkv=1, mode="table", bias_range=300),
    dict(S=700, kv_len=650, Hq=32, Hkv=1, D=64, mode="none"),
    # context-length temperature (the query sees kv_len keys, or the window)
    dict(S=6000, kv_len=5000, temp_len=1024), dict(S=3000, kv_len=2900, window=700, temp_len=100),
    dict(S=3000, kv_len=2900, Hq=32, Hkv=1, bias_range=512, temp_len=300),
    dict(S=2000, kv_len=900, mode="table", bias_range=300, temp_len=1000),
    # sharp input-dependent biases (E at std 1.0)
    dict(S=3000, kv_len=2900, window=512, bias_range=512, e_std=1.0),
    dict(S=3000, kv_len=2900, bias_range=1024, e_std=1.0),
    dict(S=3000, kv_len=2900, Hq=32, Hkv=1, bias_range=1024, e_std=1.0, R=16),
]


@pytest.mark.parametrize("kw", DEC_SWEEP, ids=lambda kw: "-".join(f"{k}{v}" for k, v in kw.items()))
def test_decode_small(kw):
    kv_len = kw.pop("kv_len")
    base = dict(kind="decode", dtype="bf16", B=3, Hq=8, Hkv=2, D=128, S=100, window=0,
                bias_range=64, mode="rproj", R=8, seed=11)
    base.update(kw)
    w = Workload(name="dec_" + "_".join(f"{k}{v}" for k, v in kw.items()), **base)
    check_decode(w, kv_len)


# Waves of five 32-row tiles (32 sequences x 8 kv heads make the split give each wave 160 rows)
# with the bias range covering the last seven waves: on contiguous caches the curves of a wave's
# first four tiles are formed up front and those of later in-band tiles one tile ahead, and a
# wave's last tile is ragged.  Checked on a few sequences.
@pytest.mark.parametrize("mode", ["rproj", "table"])
def test_decode_late_curves(mode):
    w = Workload(name=f"dec_late_{mode}", kind="decode", dtype="bf16", B=32, Hq=16, Hkv=8, D=128,
                 S=4200, window=0, bias_range=1024, mode=mode, R=8, seed=21)
    check_decode(w, 4100, batches=[0, 17, 31])


@pytest.mark.parametrize("kw", [dict(mode="rproj", window=0), dict(mode="table", window=20),
                                dict(mode="rproj_shared", window=40, logit_scale="inv_d"),
                                dict(mode="rproj", window=0, temp_len=16)],
                         ids=["rproj", "table_window", "rproj_shared", "temp"])
def test_decode_f32_small(kw):
    w = Workload(name="dec_f32", kind="decode", dtype="f32", B=2, Hq=4, Hkv=2, D=64, S=300,
                 bias_range=50, R=4, seed=3, **kw)
    check_decode(w, 250)


# the fp32 kernel splits each key tile over four waves: caches shorter than the split, one key,
# a window of one, ragged tiles, head_dim 128 and 32
@pytest.mark.parametrize("kv_len,kw", [(1, dict()), (3, dict(window=2)), (65, dict(window=1)),
                                       (130, dict(D=128, mode="table")), (70, dict(D=32, window=64))],
                         ids=["one_key", "three_keys", "window_1", "d128_table", "d32_window"])
def test_decode_f32_short(kv_len, kw):
    base = dict(B=2, Hq=4, Hkv=2, D=64, S=200, window=0, bias_range=50, R=4, seed=5, mode="rproj")
    base.update(kw)
    w = Workload(name="dec_f32_short", kind="decode", dtype="f32", **base)
    check_decode(w, kv_len)


def test_decode_global_workload():
    w = WORKLOADS["decode_global"]
    check_decode(w, w.S, batches=[0, 9, 31, 63])


def test_decode_local_workload():
    w = WORKLOADS["decode_local"]
    check_decode(w, w.S, key_margin=64)
