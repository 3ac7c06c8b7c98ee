"""GPU checks of the MXFP4 KV cache: the quantiser against the oracle's encoding bit for bit,
and decode over MXFP4 caches (contiguous, and paged with a length per sequence) against the
float64 oracle on the dequantised caches.

In the decode cases the oracle encodes the evaluated sequences itself (oracle/mxfp4.py), the
GPU's bytes must equal its bytes, and the expected outputs come from the oracle's own
dequantised caches.  Decode bar: the bf16 bar of the other decode tests (max |err| <= 2e-2,
relative L2 <= 5e-3) on o and lse.
"""

import sys
import zlib

import numpy as np
import pytest
import torch

import oracle
from oracle import mxfp4
import transformer_attention_learned_amd as rba
from transformer_attention_learned_amd.workloads import WORKLOADS, Workload, make_inputs
from paged_pool import logical_rows, paginate

pytestmark = pytest.mark.gpu

BF16_MAX_ABS, BF16_REL_L2 = 2e-2, 5e-3
BF16_LSE_MAX_ABS = 5e-3   # lse: the row sum of bf16-rounded probabilities, within 2^-8 of ln l


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    rba.load_library()


def _host_quant(x):
    """Oracle MXFP4 encoding of a bf16 tensor [..., D] -> (packed codes, scales) as uint8 tensors."""
    codes, sb = mxfp4.quantize(x)
    return torch.from_numpy(mxfp4.pack(codes)), torch.from_numpy(sb)


@pytest.mark.parametrize("D", [64, 128])
def test_quantize_bit_exact(D):
    gen = torch.Generator(device="cuda")
    gen.manual_seed(5)
    rows = 3000
    x = torch.randn((rows, D), generator=gen, device="cuda", dtype=torch.float32)
    # block magnitudes over a wide exponent range, exact midpoints, zero and tiny blocks
    k = torch.randint(-30, 30, (rows, D // 32), generator=gen, device="cuda").to(torch.float32)
    x = x * torch.exp2(k).repeat_interleave(32, dim=1)
    mids = torch.tensor([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 4.0], device="cuda")
    x[0, :8] = mids
    x[0, 8:16] = -mids
    x[1, :32] = 0.0
    x[2, :32] = 1e-30
    x[3, 32:64] = -0.0
    xb = x.to(torch.bfloat16).contiguous()
    codes, scales = rba.kv_quantize_fp4(xb)
    torch.cuda.synchronize()
    ref_codes, ref_sb = mxfp4.quantize(xb)
    np.testing.assert_array_equal(scales.cpu().numpy(), ref_sb)
    np.testing.assert_array_equal(codes.cpu().numpy(), mxfp4.pack(ref_codes))
    # the midpoints row: the scale is 2^0 and each midpoint went to its even neighbour
    deq = mxfp4.dequantize(mxfp4.unpack(codes[0].cpu().numpy()), scales[0].cpu().numpy())
    np.testing.assert_array_equal(deq[:8], [0, 1, 1, 2, 2, 4, 4, 4])


def _check_decode(w: Workload, kv_len, batches=None):
    """Quantise the caches on the GPU, decode, and compare with the oracle: the oracle encodes the
    evaluated sequences itself (its bytes must equal the GPU's) and decodes the dequantised rows."""
    _say(f"  fp4 decode case {w.name}: B={w.B} L={w.S} kv_len={kv_len} Hq={w.Hq} Hkv={w.Hkv} "
         f"W={w.window} Rb={w.bias_range} mode={w.mode} temp_len={w.temp_len} seed={w.seed}")
    inp = make_inputs(w, device="cuda")
    batches = list(range(w.B)) if batches is None else batches
    kc, ks = rba.kv_quantize_fp4(inp["k"])
    vc, vs = rba.kv_quantize_fp4(inp["v"])
    o, lse = rba.decode_fp4(inp["q"], kc, ks, vc, vs, kv_len, window=w.window,
                            bias_range=w.bias_range, mode=w.mode, table=inp["table"], r=inp["r"],
                            E=inp["E"], scale=w.scale, temp_len=w.temp_len, return_lse=True)
    torch.cuda.synchronize()
    idx = torch.tensor(batches)
    hk, hks = _host_quant(inp["k"][idx, :kv_len].cpu())
    hv, hvs = _host_quant(inp["v"][idx, :kv_len].cpu())
    assert torch.equal(kc[idx, :kv_len].cpu(), hk) and torch.equal(ks[idx, :kv_len].cpu(), hks)
    assert torch.equal(vc[idx, :kv_len].cpu(), hv) and torch.equal(vs[idx, :kv_len].cpu(), hvs)
    kd = mxfp4.dequantize(mxfp4.unpack(hk.numpy()), hks.numpy())
    vd = mxfp4.dequantize(mxfp4.unpack(hv.numpy()), hvs.numpy())
    sub = lambda t: None if t is None else t[idx.to(t.device)]
    ro, rl = oracle.decode(sub(inp["q"]), kd, vd, kv_len, scale=w.scale, window=w.window,
                           bias_range=w.bias_range, mode=w.mode, table=inp["table"],
                           r=sub(inp["r"]), E=inp["E"], temp_len=w.temp_len)
    got_o = o[idx.cuda()].to("cpu", torch.float64).numpy()
    got_l = lse[idx.cuda()].to("cpu", torch.float64).numpy()
    for name, g, r in (("o", got_o, ro), ("lse", got_l, rl)):
        assert np.all(np.isfinite(g))
        max_abs = float(np.abs(g - r).max())
        rel = float(np.linalg.norm(g - r) / np.linalg.norm(r))
        _say(f"    parity fp4 {name}: max_abs={max_abs:.3e} rel_l2={rel:.3e}")
        if name.endswith("lse"):
            assert max_abs <= BF16_LSE_MAX_ABS, (name, max_abs)
        else:
            assert max_abs <= BF16_MAX_ABS and rel <= BF16_REL_L2, (name, max_abs, rel)


CASES = [
    dict(S=100, kv_len=1), dict(S=100, kv_len=65), dict(S=3000, kv_len=2999),
    dict(S=6000, kv_len=5000, bias_range=1024), dict(S=6000, kv_len=5000, window=512, bias_range=512),
    dict(S=2000, kv_len=1999, mode="table", bias_range=300), dict(S=1500, kv_len=1400, mode="none"),
    dict(S=3000, kv_len=2600, mode="rproj_shared", R=16, window=512, bias_range=512,
         logit_scale="inv_d"),
    dict(S=3000, kv_len=2900, Hq=16, Hkv=1, window=700), dict(S=4000, kv_len=3000, temp_len=1024),
    # head_dim 64: a lane's K fragment is 8 code bytes of one 32-element block
    dict(S=3000, kv_len=2999, D=64), dict(S=2000, kv_len=1500, D=64, mode="table", bias_range=300,
                                           window=700),
    dict(S=1000, kv_len=999, D=64, Hq=16, Hkv=1, mode="rproj_shared", R=16, logit_scale="inv_d"),
    dict(S=100, kv_len=1, D=64),
    # groups of 17..32 query heads: the 32x32 MFMA kernel with its MXFP4 path
    dict(S=2000, kv_len=1999, Hq=32, Hkv=1), dict(S=100, kv_len=1, Hq=32, Hkv=1),
    dict(S=3000, kv_len=2500, Hq=24, Hkv=1, window=700, mode="table", bias_range=300),
    dict(S=1500, kv_len=1400, Hq=20, Hkv=1, D=64, mode="rproj_shared", R=16, logit_scale="inv_d"),
    dict(S=2500, kv_len=2400, Hq=32, Hkv=1, R=16, temp_len=512),
]


@pytest.mark.parametrize("kw", CASES, ids=lambda kw: "-".join(f"{k}{v}" for k, v in kw.items()))
def test_decode_fp4_matches_oracle(kw):
    kv_len = kw.pop("kv_len")
    base = dict(kind="decode", dtype="bf16", B=3, Hq=8, Hkv=2, D=128, S=100, window=0,
                bias_range=64, mode="rproj", R=8, seed=zlib.crc32(repr(sorted(kw.items())).encode()) % 1000)
    base.update(kw)
    w = Workload(name="fp4_" + "_".join(f"{k}{v}" for k, v in kw.items()), **base)
    _check_decode(w, kv_len)


def test_decode_fp4_local_layer_workload():
    """The local-layer decode shape (B64, window 512, 2048-row caches), three sequences checked."""
    w = WORKLOADS["decode_local"].with_(S=2048, name="fp4_decode_local")
    _check_decode(w, 2048, batches=[0, 17, 63])


def test_quantize_then_decode_equals_host_quantised_decode():
    """Caches quantised on the GPU give the same bytes, hence the same decode, as the oracle's."""
    w = Workload(name="fp4_ident", kind="decode", dtype="bf16", B=2, Hq=8, Hkv=2, D=128, S=1024,
                 window=0, bias_range=256, mode="rproj", R=8, seed=77)
    inp = make_inputs(w, device="cuda")
    kc, ks = rba.kv_quantize_fp4(inp["k"])
    vc, vs = rba.kv_quantize_fp4(inp["v"])
    hkc, hks = _host_quant(inp["k"].cpu())
    torch.cuda.synchronize()
    assert torch.equal(kc.cpu(), hkc) and torch.equal(ks.cpu(), hks)
    o1 = rba.decode_fp4(inp["q"], kc, ks, vc, vs, 1000, bias_range=256, mode="rproj", r=inp["r"],
                        E=inp["E"])
    hvc, hvs = _host_quant(inp["v"].cpu())
    o2 = rba.decode_fp4(inp["q"], hkc.cuda(), hks.cuda(), hvc.cuda(), hvs.cuda(), 1000,
                        bias_range=256, mode="rproj", r=inp["r"], E=inp["E"])
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)


# ---- paged MXFP4 pools ---------------------------------------------------------------------------

def _check_paged(w: Workload, lens, page_size):
    """Scatter the seeded caches into shuffled pools, quantise the pools on the GPU (their bytes
    must equal the oracle's encoding), decode through the block table with a length per
    sequence, and compare each sequence with the oracle on its own dequantised logical rows."""
    _say(f"  fp4 paged case {w.name}: B={w.B} L={w.S} Hq={w.Hq} Hkv={w.Hkv} W={w.window} "
         f"Rb={w.bias_range} mode={w.mode} R={w.R} page={page_size} lens={lens} seed={w.seed}")
    inp = make_inputs(w, device="cuda")
    gen = torch.Generator(device="cpu")
    gen.manual_seed(w.seed + 29)
    kp, bt = paginate(inp["k"], page_size, 3, gen)
    gen.manual_seed(w.seed + 29)
    vp, bt2 = paginate(inp["v"], page_size, 3, gen)
    assert torch.equal(bt, bt2)
    kc, ks = rba.kv_quantize_fp4(kp)
    vc, vs = rba.kv_quantize_fp4(vp)
    kv_lens = torch.tensor(lens, dtype=torch.int32, device="cuda")
    o, lse = rba.decode_fp4_paged(inp["q"], kc, ks, vc, vs, bt, kv_lens, max(lens),
                                  window=w.window, bias_range=w.bias_range, mode=w.mode,
                                  table=inp["table"], r=inp["r"], E=inp["E"], scale=w.scale,
                                  temp_len=w.temp_len, return_lse=True)
    torch.cuda.synchronize()
    hk, hks = _host_quant(kp.cpu())
    hv, hvs = _host_quant(vp.cpu())
    assert torch.equal(kc.cpu(), hk) and torch.equal(ks.cpu(), hks)
    assert torch.equal(vc.cpu(), hv) and torch.equal(vs.cpu(), hvs)
    got_o = o.to("cpu", torch.float64).numpy()
    got_l = lse.to("cpu", torch.float64).numpy()
    assert np.all(np.isfinite(got_o)) and np.all(np.isfinite(got_l))
    ref_o, ref_l = np.zeros_like(got_o), np.zeros_like(got_l)
    btc = bt.cpu()
    for b, L in enumerate(lens):
        deq = lambda c, sc: mxfp4.dequantize(mxfp4.unpack(logical_rows(c, btc[b], L).numpy()),
                                             logical_rows(sc, btc[b], L).numpy())[None]
        ro, rl = oracle.decode(inp["q"][b:b + 1], deq(hk, hks), deq(hv, hvs), L, scale=w.scale,
                               window=w.window, bias_range=w.bias_range, mode=w.mode,
                               table=inp["table"], r=None if inp["r"] is None else inp["r"][b:b + 1],
                               E=inp["E"], temp_len=w.temp_len)
        ref_o[b], ref_l[b] = ro[0], rl[0]
    for name, g, r in (("o", got_o, ref_o), ("lse", got_l, ref_l)):
        max_abs = float(np.abs(g - r).max())
        rel = float(np.linalg.norm(g - r) / np.linalg.norm(r))
        _say(f"    parity fp4 paged {name}: max_abs={max_abs:.3e} rel_l2={rel:.3e}")
        if name.endswith("lse"):
            assert max_abs <= BF16_LSE_MAX_ABS, (name, max_abs)
        else:
            assert max_abs <= BF16_MAX_ABS and rel <= BF16_REL_L2, (name, max_abs, rel)


PAGED_CASES = [
    (dict(), [700, 1, 33, 640], 16),
    (dict(window=96), [700, 97, 96, 95], 64),
    (dict(mode="table", bias_range=100, window=300), [699, 250, 301, 1], 256),
    (dict(mode="none", Hq=4, Hkv=4), [512, 511, 513, 2], 32),
    (dict(mode="rproj_shared", R=16, window=512, bias_range=512, logit_scale="inv_d", S=1300),
     [1300, 1000, 513, 17], 64),
    (dict(B=3, S=5000, bias_range=1024, Hq=32, Hkv=2), [5000, 4097, 1025], 128),
    (dict(S=3000, temp_len=256), [3000, 2000, 257, 100], 64),
    (dict(D=64), [700, 1, 33, 640], 16),
    (dict(D=64, window=96, mode="table", bias_range=50, Hq=8, Hkv=1), [700, 97, 96, 2], 64),
    (dict(Hq=32, Hkv=1), [700, 1, 33, 640], 32),
]


@pytest.mark.parametrize("kw,lens,page", PAGED_CASES,
                         ids=lambda x: "-".join(f"{k}{v}" for k, v in x.items()) if isinstance(x, dict) else str(x))
def test_decode_fp4_paged_matches_oracle(kw, lens, page):
    base = dict(kind="decode", dtype="bf16", B=4, Hq=8, Hkv=2, D=128, S=700, window=0,
                bias_range=64, mode="rproj", R=8,
                seed=zlib.crc32(repr((sorted(kw.items()), lens, page)).encode()) % 10007)
    base.update(kw)
    _check_paged(Workload(name="fp4_paged", **base), lens, page)


@pytest.mark.parametrize("window,page", [(0, 32), (512, 16)])
def test_fp4_paged_identity_equals_contiguous(window, page):
    """Identity block table, equal lengths: bitwise the contiguous MXFP4 decode."""
    w = Workload(name="fp4_ident_paged", kind="decode", dtype="bf16", B=3, Hq=8, Hkv=2, D=128,
                 S=4096, window=window, bias_range=512, mode="rproj", R=8, seed=41)
    inp = make_inputs(w, device="cuda")
    kc, ks = rba.kv_quantize_fp4(inp["k"])
    vc, vs = rba.kv_quantize_fp4(inp["v"])
    kv_len = 4000
    o1, l1 = rba.decode_fp4(inp["q"], kc, ks, vc, vs, kv_len, window=window, bias_range=512,
                            mode="rproj", r=inp["r"], E=inp["E"], return_lse=True)
    B, mp = w.B, w.S // page
    pages = lambda t: t.reshape((B * mp, page) + tuple(t.shape[2:]))
    bt = torch.arange(B * mp, dtype=torch.int32, device="cuda").view(B, mp)
    lens = torch.full((B,), kv_len, dtype=torch.int32, device="cuda")
    o2, l2 = rba.decode_fp4_paged(inp["q"], pages(kc), pages(ks), pages(vc), pages(vs), bt, lens,
                                  kv_len, window=window, bias_range=512, mode="rproj", r=inp["r"],
                                  E=inp["E"], return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
