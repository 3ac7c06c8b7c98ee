"""C ABI checks that need no GPU: the library loads, exports every declared
symbol, and rejects invalid arguments in host code before any HIP call."""

import ctypes
import os
import re

import pytest

import transformer_attention_learned_amd as rba

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "relbias_attn.h")

EINVAL, ENOTSUP = rba.RBA_EINVAL, rba.RBA_ENOTSUP
BF16, F32 = 1, 0
P = 4096  # a 16-byte aligned dummy address; never dereferenced (validation fails first)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(rba.library_path()):
        from transformer_attention_learned_amd.build import build_library
        build_library()
    return rba.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(relbias_attn_\w+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) == {"relbias_attn_fwd", "relbias_attn_fwd_workspace_size", "relbias_attn_decode",
                          "relbias_attn_decode_workspace_size", "relbias_attn_decode_paged",
                          "relbias_attn_decode_paged_workspace_size", "relbias_attn_last_error",
                          "relbias_attn_version", "relbias_attn_bwd",
                          "relbias_attn_bwd_workspace_size", "relbias_attn_kv_quantize_fp4",
                          "relbias_attn_decode_fp4", "relbias_attn_decode_noalloc",
                          "relbias_attn_decode_fp4_paged"}
    for n in names:
        assert hasattr(lib, n), n
    assert "gfx950" in rba.version()


def _fwd(lib, **kw):
    a = dict(dtype=BF16, q=P, k=P, v=P, o=P, lse=None, B=1, S=16, Hq=4, Hkv=2, D=128, window=0,
             bias_range=8, mode=0, table=None, r=None, E=None, R=0, scale=0.1, temp_len=0,
             ws=None, wsb=0, stream=None)
    a.update(kw)
    return lib.relbias_attn_fwd(a["dtype"], a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"],
                                a["S"], a["Hq"], a["Hkv"], a["D"], a["window"], a["bias_range"],
                                a["mode"], a["table"], a["r"], a["E"], a["R"], a["scale"],
                                a["temp_len"], a["ws"], a["wsb"], a["stream"])


def _dec(lib, **kw):
    a = dict(dtype=BF16, q=P, k=P, v=P, o=P, lse=None, B=2, L=100, kv_len=50, Hq=8, Hkv=2, D=128,
             window=0, bias_range=8, mode=0, table=None, r=None, E=None, R=0, scale=0.1,
             temp_len=0, ws=None, wsb=0, stream=None)
    a.update(kw)
    return lib.relbias_attn_decode(a["dtype"], a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"],
                                   a["L"], a["kv_len"], a["Hq"], a["Hkv"], a["D"], a["window"],
                                   a["bias_range"], a["mode"], a["table"], a["r"], a["E"], a["R"],
                                   a["scale"], a["temp_len"], a["ws"], a["wsb"], a["stream"])


def test_mode_constants_match_header():
    """The binding's mode numbers are the header's enum values."""
    text = open(HEADER).read()
    for name, value in (("RBA_BIAS_NONE", 0), ("RBA_BIAS_TABLE", 1), ("RBA_BIAS_RPROJ", 2),
                        ("RBA_BIAS_RPROJ_SHARED", 3)):
        assert re.search(rf"\b{name}\s*=\s*{value}\b", text), name
    assert rba.MODES == {"none": 0, "table": 1, "rproj": 2, "rproj_shared": 3}


@pytest.mark.parametrize("kw,code,needle", [
    (dict(dtype=7), EINVAL, "dtype"),
    (dict(Hq=6, Hkv=4), EINVAL, "multiple"),
    (dict(Hkv=0), EINVAL, "Hkv"),
    (dict(window=-1), EINVAL, "window"),
    (dict(mode=5), EINVAL, "mode"),
    (dict(D=96), ENOTSUP, "head_dim"),
    (dict(dtype=F32, D=48), ENOTSUP, "head_dim"),
    (dict(mode=1, table=None), EINVAL, "table"),
    (dict(mode=1, table=P, bias_range=0), EINVAL, "bias_range"),
    (dict(mode=2, r=P, E=P, R=17), ENOTSUP, "R="),
    (dict(mode=2, r=P, E=P, R=0), ENOTSUP, "R="),
    (dict(mode=2, r=None, E=P, R=8), EINVAL, "r and E"),
    (dict(mode=2, r=P, E=P + 2, R=8), EINVAL, "E is not"),
    (dict(mode=3, r=P, E=P, R=17), ENOTSUP, "R="),
    (dict(mode=3, r=P, E=None, R=8), EINVAL, "r and E"),
    (dict(mode=4), EINVAL, "mode"),
    (dict(q=None), EINVAL, "non-NULL"),
    (dict(o=P + 8), EINVAL, "aligned"),
    (dict(B=-1), EINVAL, "B="),
    (dict(scale=float("nan")), EINVAL, "scale"),
    (dict(mode=1, table=P, bias_range=(1 << 20) + 1), ENOTSUP, "bias_range"),
    (dict(temp_len=1), EINVAL, "temp_len"),
    (dict(temp_len=-5), EINVAL, "temp_len"),
])
def test_fwd_rejects(lib, kw, code, needle):
    assert _fwd(lib, **kw) == code
    assert needle in rba.last_error()


def test_fwd_workspace_policy(lib):
    # the input-dependent bias takes a converted copy of E, a bf16 high and low part per feature:
    # heads x (bias_range + 2 * 64 + 1) rows x 16 (R <= 8) or 32 (R <= 16) entries x 2 bytes,
    # 256-aligned
    ws = lib.relbias_attn_fwd_workspace_size
    assert ws(BF16, 2, 4096, 32, 8, 128, 512, 512, 2, 8, 0.088) == 32 * 641 * 16 * 2
    assert ws(BF16, 2, 4096, 32, 8, 128, 512, 512, 3, 16, 0.088) == (641 * 32 * 2 + 255) // 256 * 256
    assert ws(BF16, 1, 300, 4, 1, 128, 64, 100, 2, 11, 0.088) == (4 * 229 * 32 * 2 + 255) // 256 * 256
    assert ws(BF16, 1, 32768, 32, 8, 128, 0, 1024, 2, 8, 0.088) == 32 * 1153 * 16 * 2
    # no converted copy: other bias modes, fp32, shapes outside the kernel
    assert ws(BF16, 2, 4096, 32, 8, 128, 512, 512, 0, 0, 0.088) == 0
    assert ws(BF16, 2, 4096, 32, 8, 128, 512, 512, 1, 0, 0.088) == 0
    assert ws(F32, 2, 4096, 32, 8, 128, 512, 512, 2, 8, 0.088) == 0
    assert ws(BF16, 2, 4096, 32, 8, 64, 512, 512, 2, 8, 0.088) == 0
    assert ws(BF16, 2, 4096, 6, 2, 128, 512, 512, 2, 8, 0.088) == 0
    assert ws(BF16, 2, 4096, 32, 8, 128, 512, 77, 2, 8, 0.088) == 0
    # arguments the forward would reject
    assert ws(BF16, 2, 4096, 32, 8, 128, 512, 512, 2, 17, 0.088) == 0
    assert ws(BF16, 2, 4096, 32, 7, 128, 512, 512, 2, 8, 0.088) == 0


@pytest.mark.parametrize("kw,needle", [
    (dict(ws=None, wsb=0), "required"),
    (dict(ws=P, wsb=1024), "too small"),
    (dict(ws=P + 8, wsb=1 << 20), "16-byte"),
])
def test_fwd_workspace_rejects(lib, kw, needle):
    local = dict(mode=2, r=P, E=P, R=8, window=64, bias_range=64, Hq=4, Hkv=1, S=100)
    assert _fwd(lib, **local, **kw) == EINVAL
    assert needle in rba.last_error()


def test_fwd_empty_is_a_noop(lib):
    assert _fwd(lib, B=0) == 0
    assert _fwd(lib, S=0, q=None, k=None, v=None, o=None) == 0
    assert rba.last_error() == ""


@pytest.mark.parametrize("kw,code,needle", [
    (dict(kv_len=0), EINVAL, "kv_len"),
    (dict(kv_len=101), EINVAL, "kv_len"),
    (dict(Hq=66, Hkv=1), ENOTSUP, "Hq/Hkv"),
    (dict(k=None), EINVAL, "non-NULL"),
    (dict(v=P + 4), EINVAL, "aligned"),
    (dict(D=32), ENOTSUP, "head_dim"),
    (dict(mode=2, r=P, E=P, R=0), ENOTSUP, "R="),
    (dict(temp_len=1), EINVAL, "temp_len"),
])
def test_decode_rejects(lib, kw, code, needle):
    assert _dec(lib, **kw) == code
    assert needle in rba.last_error()


def test_decode_workspace_policy(lib):
    # long caches are split and need a workspace; short (or windowed) ones do not
    n = rba.decode_workspace_size(64, 32, 8, 128, 65536, 0)
    assert n > 0 and n % (32 * 64 * (128 + 2) * 4) == 0
    assert rba.decode_workspace_size(64, 32, 8, 128, 65536, 512) == 0
    assert rba.decode_workspace_size(1, 1, 1, 64, 10, 0) == 0
    # a split decode without (enough) workspace is rejected before any launch
    st = _dec(lib, B=64, Hq=32, Hkv=8, L=65536, kv_len=65536)
    assert st == EINVAL and "workspace" in rba.last_error()
    st = _dec(lib, B=64, Hq=32, Hkv=8, L=65536, kv_len=65536, ws=P, wsb=n - 4)
    assert st == EINVAL and "too small" in rba.last_error()


def test_binding_refuses_without_library(monkeypatch, tmp_path):
    """The binding never falls back to another implementation when the library is absent."""
    monkeypatch.setattr(rba, "_LIB", None)
    monkeypatch.setattr(rba, "library_path", lambda: str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="not built"):
        rba.load_library()


def _paged(lib, **kw):
    a = dict(dtype=BF16, q=P, kp=P, vp=P, bt=P, lens=P, o=P, lse=None, B=2, num_pages=8,
             page_size=32, max_pages=4, max_kv_len=100, Hq=8, Hkv=2, D=128, window=0,
             bias_range=8, mode=0, table=None, r=None, E=None, R=0, scale=0.1, temp_len=0, ws=None,
             wsb=0, stream=None)
    a.update(kw)
    return lib.relbias_attn_decode_paged(
        a["dtype"], a["q"], a["kp"], a["vp"], a["bt"], a["lens"], a["o"], a["lse"], a["B"],
        a["num_pages"], a["page_size"], a["max_pages"], a["max_kv_len"], a["Hq"], a["Hkv"], a["D"],
        a["window"], a["bias_range"], a["mode"], a["table"], a["r"], a["E"], a["R"], a["scale"],
        a["temp_len"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,code,needle", [
    (dict(dtype=F32, D=64), ENOTSUP, "bf16 only"),
    (dict(page_size=24), ENOTSUP, "page_size"),
    (dict(page_size=0), ENOTSUP, "page_size"),
    (dict(max_kv_len=129), EINVAL, "max_kv_len"),
    (dict(max_kv_len=0), EINVAL, "max_kv_len"),
    (dict(num_pages=0), EINVAL, "num_pages"),
    (dict(bt=None), EINVAL, "non-NULL"),
    (dict(lens=None), EINVAL, "non-NULL"),
    (dict(bt=P + 2), EINVAL, "4-byte"),
    (dict(kp=P + 8), EINVAL, "aligned"),
    (dict(Hq=66, Hkv=1), ENOTSUP, "Hq/Hkv"),
    (dict(mode=2, r=P, E=P, R=0), ENOTSUP, "R="),
    (dict(B=-1), EINVAL, "B="),
    (dict(temp_len=-1), EINVAL, "temp_len"),
])
def test_decode_paged_rejects(lib, kw, code, needle):
    assert _paged(lib, **kw) == code
    assert needle in rba.last_error()


def test_decode_paged_empty_and_workspace(lib):
    assert _paged(lib, B=0) == 0
    # the paged launch is sized for max_kv_len: same scratch as a contiguous cache of that length
    for args in [(64, 32, 8, 128, 65536, 0), (64, 32, 8, 128, 65536, 512), (1, 4, 1, 64, 100, 0)]:
        assert (lib.relbias_attn_decode_paged_workspace_size(*args)
                == lib.relbias_attn_decode_workspace_size(*args))


def _bwd(lib, **kw):
    a = dict(dtype=BF16, q=P, k=P, v=P, o=P, lse=P, do=P, dq=P, dk=P, dv=P, dtable=None, dr=None,
             dE=None, B=1, S=16, Hq=4, Hkv=2, D=128, window=0, bias_range=8, mode=0, table=None,
             r=None, E=None, R=0, scale=0.1, temp_len=0, ws=P, wsb=1 << 20, stream=None)
    a.update(kw)
    return lib.relbias_attn_bwd(
        a["dtype"], a["q"], a["k"], a["v"], a["o"], a["lse"], a["do"], a["dq"], a["dk"], a["dv"],
        a["dtable"], a["dr"], a["dE"], a["B"], a["S"], a["Hq"], a["Hkv"], a["D"], a["window"],
        a["bias_range"], a["mode"], a["table"], a["r"], a["E"], a["R"], a["scale"],
        a["temp_len"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,code,needle", [
    (dict(dtype=F32, D=96), ENOTSUP, "head_dim"),
    (dict(dtype=F32, mode=2, r=P, E=P, R=8, dr=P + 2, dE=P), EINVAL, "dr and dE"),
    (dict(dtype=7), EINVAL, "dtype"),
    (dict(Hq=6, Hkv=4), EINVAL, "multiple"),
    (dict(D=96), ENOTSUP, "head_dim"),
    (dict(lse=None), EINVAL, "non-NULL"),
    (dict(do=None), EINVAL, "non-NULL"),
    (dict(dk=P + 8), EINVAL, "aligned"),
    (dict(mode=1, table=P, dtable=None), EINVAL, "dtable"),
    (dict(mode=2, r=P, E=P, R=8, dr=P, dE=None), EINVAL, "dr and dE"),
    (dict(mode=3, r=P, E=P, R=8, dr=None, dE=P), EINVAL, "dr and dE"),
    (dict(ws=None), EINVAL, "workspace"),
    (dict(wsb=4), EINVAL, "too small"),
    (dict(ws=P + 4), EINVAL, "16-byte"),
    (dict(temp_len=1), EINVAL, "temp_len"),
    (dict(B=-1), EINVAL, "B="),
    # bias parameters staged in LDS: one distance past what the bf16 kernels hold
    (dict(mode=1, table=P, dtable=P, bias_range=14017), ENOTSUP, "LDS"),
    (dict(mode=1, table=P, dtable=P, bias_range=17089, D=64), ENOTSUP, "LDS"),
    (dict(mode=2, r=P, E=P, R=16, dr=P, dE=P, bias_range=1665), ENOTSUP, "LDS"),
    (dict(mode=2, r=P, E=P, R=8, dr=P, dE=P, bias_range=3457), ENOTSUP, "LDS"),
])
def test_bwd_rejects(lib, kw, code, needle):
    assert _bwd(lib, **kw) == code
    assert needle in rba.last_error()


def test_bwd_empty_and_workspace(lib):
    assert _bwd(lib, B=0) == 0
    assert _bwd(lib, S=0, q=None) == 0
    assert lib.relbias_attn_bwd_workspace_size(2, 100, 8, 0, 64) == 6400       # rowsum only
    assert lib.relbias_attn_bwd_workspace_size(2, 100, 8, 1, 64) == 6400
    # r.E: plus E as bf16 high and low parts, heads x (bias_range + 129) rows x 32 entries x 2
    # bytes: independent of the sequence length (one bank for the shared form)
    assert lib.relbias_attn_bwd_workspace_size(2, 100, 8, 2, 512) == 6400 + 8 * 641 * 32 * 2
    assert lib.relbias_attn_bwd_workspace_size(2, 100, 8, 3, 77) == 6400 + 1 * 206 * 32 * 2
    assert (lib.relbias_attn_bwd_workspace_size(1, 1 << 20, 32, 2, 1024) ==
            (1 << 20) * 32 * 4 + 32 * 1153 * 32 * 2)
    assert lib.relbias_attn_bwd_workspace_size(0, 100, 8, 2, 64) == 0


def test_fp4_rejects(lib):
    q = lib.relbias_attn_kv_quantize_fp4
    assert q(P, P, P, 10, 48, None) == EINVAL and "multiple of 32" in rba.last_error()
    assert q(P, P, P, -1, 64, None) == EINVAL
    assert q(None, P, P, 4, 64, None) == EINVAL and "non-NULL" in rba.last_error()
    assert q(P + 8, P, P, 4, 64, None) == EINVAL and "aligned" in rba.last_error()
    assert q(P, P, P, 0, 64, None) == 0

    def dec(**kw):
        a = dict(q=P, kc=P, ks=P, vc=P, vs=P, o=P, lse=None, B=2, L=100, kv_len=50, Hq=8, Hkv=2,
                 D=128, window=0, bias_range=8, mode=0, table=None, r=None, E=None, R=0,
                 scale=0.1, temp_len=0, ws=None, wsb=0)
        a.update(kw)
        return lib.relbias_attn_decode_fp4(
            a["q"], a["kc"], a["ks"], a["vc"], a["vs"], a["o"], a["lse"], a["B"], a["L"],
            a["kv_len"], a["Hq"], a["Hkv"], a["D"], a["window"], a["bias_range"], a["mode"],
            a["table"], a["r"], a["E"], a["R"], a["scale"], a["temp_len"], a["ws"], a["wsb"], None)
    assert dec(D=96) == ENOTSUP and "head_dim" in rba.last_error()
    assert dec(Hq=64, Hkv=1) == ENOTSUP and "<= 32" in rba.last_error()
    assert dec(kv_len=0) == EINVAL and "kv_len" in rba.last_error()
    assert dec(ks=None) == EINVAL and "non-NULL" in rba.last_error()
    assert dec(vc=P + 4) == EINVAL and "aligned" in rba.last_error()
    assert dec(temp_len=1) == EINVAL and "temp_len" in rba.last_error()
    assert dec(B=0) == 0


def _fp4_paged(lib, **kw):
    a = dict(q=P, kc=P, ks=P, vc=P, vs=P, bt=P, lens=P, o=P, lse=None, B=2, num_pages=8,
             page_size=32, max_pages=4, max_kv_len=100, Hq=8, Hkv=2, D=128, window=0,
             bias_range=8, mode=0, table=None, r=None, E=None, R=0, scale=0.1, temp_len=0, ws=None,
             wsb=0)
    a.update(kw)
    return lib.relbias_attn_decode_fp4_paged(
        a["q"], a["kc"], a["ks"], a["vc"], a["vs"], a["bt"], a["lens"], a["o"], a["lse"], a["B"],
        a["num_pages"], a["page_size"], a["max_pages"], a["max_kv_len"], a["Hq"], a["Hkv"], a["D"],
        a["window"], a["bias_range"], a["mode"], a["table"], a["r"], a["E"], a["R"], a["scale"],
        a["temp_len"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,code,needle", [
    (dict(D=96), ENOTSUP, "head_dim"),
    (dict(Hq=64, Hkv=1), ENOTSUP, "<= 32"),
    (dict(page_size=24), ENOTSUP, "page_size"),
    (dict(max_kv_len=129), EINVAL, "max_kv_len"),
    (dict(max_kv_len=0), EINVAL, "max_kv_len"),
    (dict(num_pages=0), EINVAL, "num_pages"),
    (dict(bt=None), EINVAL, "non-NULL"),
    (dict(lens=P + 2), EINVAL, "4-byte"),
    (dict(ks=None), EINVAL, "non-NULL"),
    (dict(vc=P + 4), EINVAL, "aligned"),
    (dict(mode=1, table=None), EINVAL, "table"),
    (dict(temp_len=1), EINVAL, "temp_len"),
    (dict(B=-1), EINVAL, "B="),
    (dict(max_kv_len=5000, num_pages=200, max_pages=200, ws=None), EINVAL, "workspace"),
    (dict(max_kv_len=5000, num_pages=200, max_pages=200, ws=P, wsb=4), EINVAL, "too small"),
])
def test_decode_fp4_paged_rejects(lib, kw, code, needle):
    assert _fp4_paged(lib, **kw) == code
    assert needle in rba.last_error()


def test_decode_fp4_paged_empty(lib):
    assert _fp4_paged(lib, B=0) == 0
    assert _fp4_paged(lib, B=0, q=None, bt=None) == 0


# --- the binding checks the exact shapes of the bias parameters before any library call -----

def _cpu_inputs(S=16, Hq=4, Hkv=2, D=128, B=1):
    import torch
    q = torch.zeros((B, S, Hq, D), dtype=torch.bfloat16)
    k = torch.zeros((B, S, Hkv, D), dtype=torch.bfloat16)
    return q, k, k.clone()


@pytest.mark.parametrize("mode,shapes,needle", [
    ("table", dict(table=(4, 7)), "table must be"),         # shorter than bias_range
    ("table", dict(table=(2, 8)), "table must be"),         # fewer heads than Hq
    ("rproj", dict(E=(4, 8, 7), r=(1, 16, 4, 8)), "E must be"),
    ("rproj", dict(E=(3, 8, 8), r=(1, 16, 4, 8)), "E must be"),
    ("rproj_shared", dict(E=(8, 5), r=(1, 16, 4, 8)), "E must be"),
    ("rproj", dict(E=(4, 8, 8), r=(1, 16, 4, 6)), "r must end in"),
])
def test_binding_checks_bias_shapes(lib, mode, shapes, needle):
    import torch
    q, k, v = _cpu_inputs()
    kw = {n: torch.zeros(s, dtype=torch.float32 if n != "r" else torch.bfloat16) for n, s in shapes.items()}
    with pytest.raises(ValueError, match=needle):
        rba.fwd(q, k, v, bias_range=8, mode=mode, **kw)
    with pytest.raises(ValueError, match=needle):
        rba.bwd(q, k, v, q, torch.zeros((1, 4, 16)), q, bias_range=8, mode=mode, **kw)
    qd = torch.zeros((1, 4, 128), dtype=torch.bfloat16)
    kc = torch.zeros((1, 32, 2, 128), dtype=torch.bfloat16)
    kwd = dict(kw)
    if "r" in kwd:
        kwd["r"] = torch.zeros((1,) + tuple(shapes["r"][2:]), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match=needle):
        rba.decode(qd, kc, kc, 20, bias_range=8, mode=mode, **kwd)


def test_binding_rejects_unknown_mode(lib):
    q, k, v = _cpu_inputs()
    with pytest.raises(ValueError, match="unknown bias mode"):
        rba.fwd(q, k, v, bias_range=8, mode=7)


def test_decode_noalloc_rejects(lib):
    """The allocation-free decode: bf16 only; sizes whose split partials exceed the fixed scratch
    are refused in host code before anything is launched; the usual argument checks apply."""
    assert "RBA_DECODE_NOALLOC_SCRATCH_BYTES (16 * 1024 * 1024)" in open(HEADER).read()

    def dec(**kw):
        a = dict(dtype=BF16, q=P, k=P, v=P, o=P, lse=None, B=2, L=100, kv_len=50, Hq=8, Hkv=2,
                 D=128, window=0, bias_range=8, mode=0, table=None, r=None, E=None, R=0, scale=0.1,
                 temp_len=0, stream=None)
        a.update(kw)
        return lib.relbias_attn_decode_noalloc(
            a["dtype"], a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["L"], a["kv_len"],
            a["Hq"], a["Hkv"], a["D"], a["window"], a["bias_range"], a["mode"], a["table"], a["r"],
            a["E"], a["R"], a["scale"], a["temp_len"], a["stream"])
    assert dec(dtype=F32, D=64) == ENOTSUP and "bf16 only" in rba.last_error()
    big = dict(B=8, Hq=32, Hkv=1, L=65536, kv_len=65536)
    assert lib.relbias_attn_decode_workspace_size(8, 32, 1, 128, 65536, 0) > rba.DECODE_NOALLOC_SCRATCH_BYTES
    assert dec(**big) == ENOTSUP and "scratch" in rba.last_error()
    assert dec(kv_len=0) == EINVAL and "kv_len" in rba.last_error()
    assert dec(q=None) == EINVAL and "non-NULL" in rba.last_error()
    assert dec(temp_len=1) == EINVAL
    assert dec(B=0) == 0
