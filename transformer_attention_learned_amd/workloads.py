"""Seeded synthetic inputs for relative-position-bias attention.

This module only draws tensors (shapes, distributions, seeds); it holds none
of the attention arithmetic.  Tests feed the same draws to the HIP library
and to the float64 oracle; the benchmark uses them for timing.

Workloads (the shapes of the local / global layers described for Inkling:
"Learned Relative-Position Bias", section "Hybrid Attention Interaction",
512-token local window, 1,024-token global bias range):

  tiny_local_f32       B1 H1/1 S256 D32, window 64, table bias (fp32)
  local_prefill        B2 S4096 H32/8 D128, window 512, r.E bias R=8, range 512
  global_prefill       B1 S32768 H32/8 D128, full causal, r.E bias R=8, range 1024
  long_global_prefill  B1 S131072 H16/4 D128, full causal, table bias, range 1024
  decode_global        B64 H32/8 D128 cache 65536, full causal, r.E bias, range 1024
  decode_local         same cache, window 512, r.E bias, range 512

Distributions: N(mean, std) with the second parameter the standard deviation.
q and k of the prefill workloads are RMS-normalised per (token, head) with
unit gain (x / sqrt(mean(x^2) + 1e-6), computed in fp32, then cast).
Draw order per workload: q, k, v, bias parameter (table or E), r.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

MODE_IDS = {"none": 0, "table": 1, "rproj": 2, "rproj_shared": 3}


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str                 # "prefill" | "decode" | "backward" (gradients of a prefill)
    dtype: str                # "f32" | "bf16"
    B: int
    Hq: int
    Hkv: int
    D: int
    S: int                    # prefill sequence length, or decode cache length (kv_len)
    window: int               # 0 = full causal
    bias_range: int
    mode: str                 # "none" | "table" | "rproj" | "rproj_shared"
    R: int = 8
    seed: int = 0
    rmsnorm_qk: bool = False
    table_std: float = 0.5
    table_trend: float = 0.0  # added to table[h, delta]: trend * delta
    e_std: float = 0.1
    logit_scale: str = "rsqrt_d"   # "rsqrt_d": 1/sqrt(D); "inv_d": 1/D (the essay's Inkling form)
    temp_len: int = 0         # context-length temperature threshold (0: none)
    extra: dict = field(default_factory=dict)

    @property
    def scale(self) -> float:
        return 1.0 / self.D if self.logit_scale == "inv_d" else 1.0 / math.sqrt(self.D)

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    def with_(self, **kw) -> "Workload":
        d = dict(self.__dict__)
        d.update(kw)
        return Workload(**d)


# Global layers carry the context-length temperature, flat up to 128k visible keys (at these
# lengths it is exactly 1, but the kernels take the tempered path).
GLOBAL_TEMP_LEN = 131072

WORKLOADS = {
    "tiny_local_f32": Workload("tiny_local_f32", "prefill", "f32", B=1, Hq=1, Hkv=1, D=32, S=256,
                               window=64, bias_range=64, mode="table", seed=1, table_std=0.5),
    "local_prefill": Workload("local_prefill", "prefill", "bf16", B=2, Hq=32, Hkv=8, D=128,
                              S=4096, window=512, bias_range=512, mode="rproj", seed=2,
                              rmsnorm_qk=True),
    "global_prefill": Workload("global_prefill", "prefill", "bf16", B=1, Hq=32, Hkv=8, D=128,
                               S=32768, window=0, bias_range=1024, mode="rproj", seed=3,
                               rmsnorm_qk=True, temp_len=GLOBAL_TEMP_LEN),
    "long_global_prefill": Workload("long_global_prefill", "prefill", "bf16", B=1, Hq=16, Hkv=4,
                                    D=128, S=131072, window=0, bias_range=1024, mode="table",
                                    seed=4, rmsnorm_qk=True, table_std=0.5, table_trend=-0.01,
                                    temp_len=GLOBAL_TEMP_LEN),
    "decode_global": Workload("decode_global", "decode", "bf16", B=64, Hq=32, Hkv=8, D=128,
                              S=65536, window=0, bias_range=1024, mode="rproj", seed=5,
                              temp_len=GLOBAL_TEMP_LEN),
    "decode_local": Workload("decode_local", "decode", "bf16", B=64, Hq=32, Hkv=8, D=128,
                             S=65536, window=512, bias_range=512, mode="rproj", seed=5),
    # the same decode steps over a paged cache: 64-row pages in a pool, each sequence's pages
    # scattered by a seeded permutation (the page-table layout of a serving engine)
    "decode_global_paged": Workload("decode_global_paged", "decode", "bf16", B=64, Hq=32, Hkv=8,
                                    D=128, S=65536, window=0, bias_range=1024, mode="rproj", seed=5,
                                    temp_len=GLOBAL_TEMP_LEN, extra={"page_size": 64}),
    "decode_local_paged": Workload("decode_local_paged", "decode", "bf16", B=64, Hq=32, Hkv=8,
                                   D=128, S=65536, window=512, bias_range=512, mode="rproj", seed=5,
                                   extra={"page_size": 64}),
}


# The decode steps over MXFP4 caches (the caches quantised once before timing).
for _name in ("decode_global", "decode_local"):
    WORKLOADS[_name + "_fp4"] = WORKLOADS[_name].with_(name=_name + "_fp4", extra={"kv": "fp4"})
    # and over MXFP4 page pools (the paged layout above)
    WORKLOADS[_name + "_paged_fp4"] = WORKLOADS[_name].with_(
        name=_name + "_paged_fp4", extra={"kv": "fp4", "page_size": 64})

# Backward passes of the three prefill layers (same inputs, plus the output gradient).
for _name in ("local_prefill", "global_prefill", "long_global_prefill"):
    WORKLOADS[_name + "_bwd"] = WORKLOADS[_name].with_(name=_name + "_bwd", kind="backward")


def paged_view(w: Workload, k, v, seed=None):
    """Page pools and block table over the contiguous caches of a decode workload.

    The caches [B, L, Hkv, D] are viewed as B * L / page_size pages (no copy); sequence b's
    logical page p is pool page perm[b * max_pages + p] for a seeded permutation, so the
    table scatters every sequence over the pool.  Returns (k_pages, v_pages, block_table).
    """
    ps = w.extra["page_size"]
    B, L, Hkv, D = k.shape
    mp = L // ps
    gen = torch.Generator(device="cpu")
    gen.manual_seed((w.seed if seed is None else seed) + 1000)
    perm = torch.randperm(B * mp, generator=gen).to(torch.int32).to(k.device)
    return (k.view(B * mp, ps, Hkv, D), v.view(B * mp, ps, Hkv, D), perm.view(B, mp))


def _randn(shape, gen, device, dtype, chunk_elems=1 << 28):
    """N(0, 1) draw in `dtype`, generated chunk by chunk along dim 0 to bound fp32 temporaries."""
    out = torch.empty(shape, dtype=dtype, device=device)
    n0 = shape[0]
    per = max(1, int(math.prod(shape[1:])))
    rows = max(1, chunk_elems // per)
    for s in range(0, n0, rows):
        e = min(n0, s + rows)
        out[s:e] = torch.randn((e - s,) + tuple(shape[1:]), generator=gen, device=device,
                               dtype=torch.float32).to(dtype)
    return out


def _rmsnorm_randn(shape, gen, device, dtype, chunk_elems=1 << 28):
    out = torch.empty(shape, dtype=dtype, device=device)
    n0 = shape[0]
    per = max(1, int(math.prod(shape[1:])))
    rows = max(1, chunk_elems // per)
    for s in range(0, n0, rows):
        e = min(n0, s + rows)
        x = torch.randn((e - s,) + tuple(shape[1:]), generator=gen, device=device,
                        dtype=torch.float32)
        x = x * torch.rsqrt(x.pow(2).mean(dim=-1, keepdim=True) + 1e-6)
        out[s:e] = x.to(dtype)
    return out


def make_inputs(w: Workload, device="cpu", seed=None):
    """Draw every input of workload `w` on `device` (seeded, deterministic per device).

    Prefill returns q [B,S,Hq,D], k/v [B,S,Hkv,D], r [B,S,Hq,R] (rproj); backward the same
    plus dout [B,S,Hq,D] (N(0,1), drawn after every other input);
    decode returns q [B,Hq,D], k/v caches [B,S,Hkv,D], r [B,Hq,R].
    table [Hq, bias_range] fp32 (table mode), E [Hq, R, bias_range] fp32 (rproj) or
    [R, bias_range] (rproj_shared: one bank for every head).
    """
    gen = torch.Generator(device=device)
    gen.manual_seed(w.seed if seed is None else seed)
    dt = w.torch_dtype
    if w.kind in ("prefill", "backward"):
        B, S = w.B, w.S
        qshape, kshape = (B, S, w.Hq, w.D), (B, S, w.Hkv, w.D)
        rshape = (B, S, w.Hq, w.R)
        # the RMS norm runs over the head dim, so draw as [B*S, H, D] and normalise dim -1
        if w.rmsnorm_qk:
            q = _rmsnorm_randn((B * S, w.Hq, w.D), gen, device, dt).view(qshape)
            k = _rmsnorm_randn((B * S, w.Hkv, w.D), gen, device, dt).view(kshape)
        else:
            q = _randn((B * S, w.Hq, w.D), gen, device, dt).view(qshape)
            k = _randn((B * S, w.Hkv, w.D), gen, device, dt).view(kshape)
        v = _randn((B * S, w.Hkv, w.D), gen, device, dt).view(kshape)
    else:
        B, L = w.B, w.S
        q = _randn((B, w.Hq, w.D), gen, device, dt)
        k = _randn((B * L, w.Hkv, w.D), gen, device, dt).view(B, L, w.Hkv, w.D)
        v = _randn((B * L, w.Hkv, w.D), gen, device, dt).view(B, L, w.Hkv, w.D)
        rshape = (B, w.Hq, w.R)
    table = E = r = None
    if w.mode == "table":
        t = torch.randn((w.Hq, w.bias_range), generator=gen, device=device,
                        dtype=torch.float32) * w.table_std
        if w.table_trend:
            t = t + w.table_trend * torch.arange(w.bias_range, device=device,
                                                 dtype=torch.float32)[None, :]
        table = t.contiguous()
    elif w.mode in ("rproj", "rproj_shared"):
        eshape = (w.Hq, w.R, w.bias_range) if w.mode == "rproj" else (w.R, w.bias_range)
        E = (torch.randn(eshape, generator=gen, device=device, dtype=torch.float32) * w.e_std).contiguous()
        r = torch.randn(rshape, generator=gen, device=device, dtype=torch.float32).to(dt)
    dout = None
    if w.kind == "backward":   # gradient on the output, drawn last
        dout = _randn((w.B * w.S, w.Hq, w.D), gen, device, dt).view(q.shape)
    return dict(q=q, k=k, v=v, table=table, E=E, r=r, dout=dout)


def small_case(dtype="bf16", B=1, S=200, Hq=4, Hkv=2, D=128, window=0, bias_range=64,
               mode="rproj", R=8, seed=0, kind="prefill", rmsnorm_qk=True):
    """A reduced workload for parity tests (same distributions, smaller shapes)."""
    return Workload(f"small_{kind}_{mode}", kind, dtype, B=B, Hq=Hq, Hkv=Hkv, D=D, S=S,
                    window=window, bias_range=bias_range, mode=mode, R=R, seed=seed,
                    rmsnorm_qk=rmsnorm_qk)
