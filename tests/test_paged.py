"""GPU parity of decode over a paged cache with a cache length per sequence.

The seeded contiguous caches of a decode workload are scattered into a shuffled page pool;
the library reads them through the block table, and the float64 oracle evaluates each
sequence on its contiguous cache at its own length.  An identity block table with equal
lengths must reproduce the contiguous decode bit for bit (same kernel, same split).
"""

import sys
import zlib

import numpy as np
import pytest
import torch

import oracle
import transformer_attention_learned_amd as rba
from transformer_attention_learned_amd.workloads import Workload, make_inputs
from paged_pool import paginate

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


def _t2np(t):
    return t.detach().to("cpu", torch.float64).numpy()


def _check(w, lens, page_size, n_extra=3):
    _say(f"  paged case: B={w.B} L={w.S} Hq={w.Hq} Hkv={w.Hkv} D={w.D} W={w.window} "
         f"Rb={w.bias_range} mode={w.mode} R={w.R} page={page_size} lens={lens}")
    inp = make_inputs(w, device="cuda")
    gen = torch.Generator(device="cpu")
    gen.manual_seed(w.seed + 17)
    kp, bt = paginate(inp["k"], page_size, n_extra, gen)
    gen.manual_seed(w.seed + 17)
    vp, bt2 = paginate(inp["v"], page_size, n_extra, gen)
    assert torch.equal(bt, bt2)
    kv_lens = torch.tensor(lens, dtype=torch.int32, device="cuda")
    o, lse = rba.decode_paged(inp["q"], kp, vp, bt, kv_lens, max(lens), window=w.window,
                              bias_range=w.bias_range, mode=w.mode, table=inp["table"],
                              r=inp["r"], E=inp["E"], scale=w.scale, temp_len=w.temp_len,
                              return_lse=True)
    torch.cuda.synchronize()
    got_o, got_l = _t2np(o), _t2np(lse)
    assert np.all(np.isfinite(got_o)) and np.all(np.isfinite(got_l))
    ref_o = np.zeros_like(got_o)
    ref_l = np.zeros_like(got_l)
    for b, L in enumerate(lens):
        ro, rl = oracle.decode(inp["q"], inp["k"], inp["v"], L, scale=w.scale,
                               temp_len=w.temp_len, window=w.window,
                               bias_range=w.bias_range, mode=w.mode, table=inp["table"],
                               r=inp["r"], E=inp["E"], batch=[b])
        ref_o[b], ref_l[b] = ro[0], rl[0]
    for name, g, r in (("o", got_o, ref_o), ("lse", got_l, ref_l)):
        max_abs = float(np.abs(g - r).max())
        rel = float(np.linalg.norm(g - r) / np.linalg.norm(r))
        _say(f"    parity paged {name}: max_abs={max_abs:.3e} rel_l2={rel:.3e}")
        if name.endswith("lse"):
            assert max_abs <= BF16_LSE_MAX_ABS, (name, max_abs)
        else:
            assert max_abs <= BF16_MAX_ABS and rel <= BF16_REL_L2, (name, max_abs, rel)


def _w(**kw):
    base = dict(name="paged", kind="decode", dtype="bf16", B=4, Hq=8, Hkv=2, D=128, S=700,
                window=0, bias_range=64, mode="rproj", R=8, seed=23)
    base.update(kw)
    return Workload(**base)


CASES = [
    (dict(), [700, 1, 33, 640], 16),
    (dict(), [700, 500, 64, 65], 32),
    (dict(window=96), [700, 97, 96, 95], 64),
    (dict(mode="table", bias_range=100, window=300), [699, 250, 301, 1], 256),
    (dict(mode="none", Hq=4, Hkv=4), [512, 511, 513, 2], 32),
    (dict(mode="rproj_shared", R=16, window=512, bias_range=512, logit_scale="inv_d", S=1300),
     [1300, 1000, 513, 17], 64),
    (dict(D=64, Hq=16, Hkv=2, S=300), [300, 299, 150, 48], 16),
    (dict(B=3, S=5000, bias_range=1024, Hq=32, Hkv=8), [5000, 4097, 1025], 128),
    # context-length temperature follows each sequence's own length
    (dict(S=3000, temp_len=256), [3000, 2000, 257, 100], 64),
    # waves of five 32-row tiles (32 sequences x 8 kv heads) with the bias range covering the
    # last waves: curves of in-band tiles past a wave's fourth are formed one tile ahead, page
    # entries are read a tile ahead, lengths end inside a tile
    (dict(B=32, Hq=16, Hkv=8, S=4200, bias_range=1024),
     [4100, 4099, 4064, 3000, 1025, 1024, 700, 33] * 4, 64),
    (dict(B=32, Hq=16, Hkv=8, S=4200, bias_range=1024, mode="table"),
     [4100, 3333, 2048, 4031] * 8, 16),
]


@pytest.mark.parametrize("kw,lens,page", CASES,
                         ids=lambda x: "-".join(f"{k}{v}" for k, v in x.items()) if isinstance(x, dict) else str(x))
def test_decode_paged_matches_oracle(kw, lens, page):
    seed = zlib.crc32(repr((sorted(kw.items()), lens, page)).encode()) % 10007
    _check(_w(seed=seed, **kw), lens, page)


@pytest.mark.parametrize("window,page", [(0, 32), (512, 16)])
def test_paged_identity_equals_contiguous(window, page):
    """Identity block table, equal lengths: bitwise the contiguous decode."""
    w = Workload(name="ident", kind="decode", dtype="bf16", B=3, Hq=8, Hkv=2, D=128, S=4096,
                 window=window, bias_range=512, mode="rproj", R=8, seed=31)
    inp = make_inputs(w, device="cuda")
    kv_len = 4000
    o1, l1 = rba.decode(inp["q"], inp["k"], inp["v"], kv_len, window=window, bias_range=512,
                        mode="rproj", r=inp["r"], E=inp["E"], return_lse=True)
    B, L = w.B, w.S
    mp = L // page
    kp = inp["k"].reshape(B * mp, page, w.Hkv, w.D)
    vp = inp["v"].reshape(B * mp, page, w.Hkv, w.D)
    bt = torch.arange(B * mp, dtype=torch.int32, device="cuda").view(B, mp)
    lens = torch.full((B,), kv_len, dtype=torch.int32, device="cuda")
    o2, l2 = rba.decode_paged(inp["q"], kp, vp, bt, lens, kv_len, window=window, bias_range=512,
                              mode="rproj", r=inp["r"], E=inp["E"], return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
