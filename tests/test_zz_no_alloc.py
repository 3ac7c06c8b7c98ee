"""GPU check of relbias_attn_decode_noalloc (the decode entry point that allocates nothing and
keeps its split partials in the library's fixed per-GPU scratch) against relbias_attn_decode
with a caller workspace: same kernels, so the outputs must agree exactly (and in particular
within the bf16 bar), on two calls in a row, the second with a smaller input."""

import sys

import pytest
import torch

import transformer_attention_learned_amd as rba
from transformer_attention_learned_amd.workloads import Workload, make_inputs

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    rba.load_library()


def _case(w, kv_len):
    inp = make_inputs(w, device="cuda")
    kw = dict(window=w.window, bias_range=w.bias_range, mode=w.mode, table=inp["table"], r=inp["r"],
              E=inp["E"], scale=w.scale, temp_len=w.temp_len, return_lse=True)
    need = rba.decode_workspace_size(w.B, w.Hq, w.Hkv, w.D, kv_len, w.window)
    _say(f"  noalloc case {w.name}: B={w.B} kv_len={kv_len} Hq={w.Hq} Hkv={w.Hkv} W={w.window} "
         f"Rb={w.bias_range} mode={w.mode}: split scratch {need} bytes")
    assert need <= rba.DECODE_NOALLOC_SCRATCH_BYTES
    ref_o, ref_l = rba.decode(inp["q"], inp["k"], inp["v"], kv_len, **kw)
    got_o, got_l = rba.decode_noalloc(inp["q"], inp["k"], inp["v"], kv_len, **kw)
    torch.cuda.synchronize()
    d = (got_o.float() - ref_o.float()).abs().max().item()
    rel = ((got_o.float() - ref_o.float()).norm() / ref_o.float().norm()).item()
    _say(f"    max_abs={d:.3e} rel_l2={rel:.3e} identical={torch.equal(got_o, ref_o)}")
    assert d <= 2e-2 and rel <= 5e-3
    assert torch.equal(got_o, ref_o) and torch.equal(got_l, ref_l)
    return need


def test_noalloc_matches_decode_two_calls():
    """A global-layer decode step (64 sequences, 65,536 cached rows: several splits, the largest
    use of the scratch), then a smaller one (5 sequences, 5,000 rows, table bias): the second
    call reuses the scratch the first one left behind."""
    big = Workload("noalloc_global", "decode", "bf16", B=64, Hq=32, Hkv=8, D=128, S=65536, window=0,
                   bias_range=1024, mode="rproj", seed=21)
    small = Workload("noalloc_small", "decode", "bf16", B=5, Hq=16, Hkv=4, D=128, S=6000,
                     window=0, bias_range=300, mode="table", seed=22)
    n1 = _case(big, big.S)
    n2 = _case(small, 5000)
    assert n1 > n2 > 0


def test_noalloc_rejects_oversized_scratch():
    """A shape whose split partials exceed the fixed scratch is refused before any launch (the
    buffers are real and sized for the shape all the same)."""
    B, Hq, Hkv, D, L = 8, 32, 1, 128, 65536
    need = rba.decode_workspace_size(B, Hq, Hkv, D, L, 0)
    assert need > rba.DECODE_NOALLOC_SCRATCH_BYTES, need
    q = torch.zeros((B, Hq, D), dtype=torch.bfloat16, device="cuda")
    kc = torch.zeros((B, L, Hkv, D), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(rba.LibraryError, match="scratch") as ei:
        rba.decode_noalloc(q, kc, kc, L)
    assert ei.value.status == rba.RBA_ENOTSUP
    # the same shape runs through the workspace entry point
    o = rba.decode(q, kc, kc, L)
    torch.cuda.synchronize()
    assert torch.all(o == 0)
