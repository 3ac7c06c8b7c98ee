"""Decode steps captured in HIP graphs (torch.cuda.CUDAGraph), as a serving loop may run them:
every replay must give the eager call's result, with the program's own eager work (other library
calls on other inputs, overwrites of the output) and synchronizations between the replays.  The
library records no memory-set nodes: scratch comes from the caller's workspace and is written
by the kernels themselves."""
import pytest
import torch

import transformer_attention_learned_amd as rba
from transformer_attention_learned_amd.workloads import Workload, make_inputs, paged_view

pytestmark = pytest.mark.gpu


def _case(**kw):
    base = dict(name="graph", kind="decode", dtype="bf16", B=3, Hq=8, Hkv=2, D=128, S=2000,
                window=0, bias_range=256, mode="rproj", R=8, seed=11)
    base.update(kw)
    return Workload(**base)


CASES = [
    dict(),                                     # several splits and the combine kernel
    dict(window=512, bias_range=512, S=1500),   # one split
    dict(mode="table", S=700, Hq=12, Hkv=2),   # G = 6, the 16-column kernel
    dict(Hq=48, Hkv=2, S=900),                 # G = 24, the 32-column kernel
]


def _replays(call, out, eager_ref, other):
    dev = out.device
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()
    for rep in range(4):
        out.fill_(float("nan"))
        other()                          # eager work between the replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager_ref), f"replay {rep} differs from the eager call"
    del g


@pytest.mark.parametrize("kw", CASES, ids=lambda kw: "-".join(f"{k}{v}" for k, v in kw.items()) or "default")
def test_decode_graph_replay(kw):
    dev = torch.device("cuda:0")
    w = _case(**kw)
    inp = make_inputs(w, device=dev)
    o_w = _case(**dict(kw, seed=12))
    inp2 = make_inputs(o_w, device=dev)
    args = dict(window=w.window, bias_range=w.bias_range, mode=w.mode, table=inp["table"], r=inp["r"],
                E=inp["E"], scale=w.scale)
    ref = rba.decode(inp["q"], inp["k"], inp["v"], w.S, **args)
    need = rba.decode_workspace_size(w.B, w.Hq, w.Hkv, w.D, w.S, w.window)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    out = torch.empty_like(inp["q"])

    def call():
        rba.decode(inp["q"], inp["k"], inp["v"], w.S, out=out, workspace=ws, **args)

    def other():
        rba.decode(inp2["q"], inp2["k"], inp2["v"], w.S - 5, window=w.window, bias_range=w.bias_range,
                   mode=w.mode, table=inp2["table"], r=inp2["r"], E=inp2["E"], scale=w.scale, workspace=ws)

    torch.cuda.synchronize()
    _replays(call, out, ref, other)


def test_decode_fp4_paged_graph_replay():
    dev = torch.device("cuda:0")
    w = _case(S=1280, window=0, bias_range=300, extra={"page_size": 64})
    inp = make_inputs(w, device=dev)
    kc, ks = rba.kv_quantize_fp4(inp["k"])
    vc, vs = rba.kv_quantize_fp4(inp["v"])
    kcp, vcp, bt = paged_view(w, kc, vc)
    ksp, vsp, _ = paged_view(w, ks, vs)
    lens = torch.full((w.B,), w.S, dtype=torch.int32, device=dev)
    args = dict(window=w.window, bias_range=w.bias_range, mode=w.mode, table=inp["table"], r=inp["r"],
                E=inp["E"], scale=w.scale)
    ref = rba.decode_fp4_paged(inp["q"], kcp, ksp, vcp, vsp, bt, lens, w.S, **args)
    out = torch.empty_like(inp["q"])
    need = rba.decode_workspace_size(w.B, w.Hq, w.Hkv, w.D, w.S, w.window)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)

    def call():
        rba.decode_fp4_paged(inp["q"], kcp, ksp, vcp, vsp, bt, lens, w.S, out=out, workspace=ws, **args)

    def other():
        rba.decode(inp["q"], inp["k"], inp["v"], w.S - 7, workspace=ws, **args)

    torch.cuda.synchronize()
    _replays(call, out, ref, other)
