"""MXFP4 encoding of a KV cache (test infrastructure only, like the rest of this package).

The pages list an FP4 KV cache among Inkling's KV-cache compression methods and name MXFP4
among the FP4 formats of its training ("models/inkling" (archdiff), the component diagram:
the KV-cache compression and the FP8-to-FP4 training components).  The pages do not define the
format; this module takes the OCP Microscaling (MX) definition of MXFP4, read plainly:
  * blocks of 32 consecutive elements along the head dimension share one scale 2^s stored as
    an E8M0 byte (s + 127);
  * each element is an FP4 E2M1 code: sign bit (bit 3) and a magnitude code 0..7 for
    0, 0.5, 1, 1.5, 2, 3, 4, 6;
  * quantisation: s = floor(log2(max |x|)) - 2 (2 = the largest E2M1 exponent), then each
    x / 2^s is rounded to the nearest E2M1 magnitude, ties to the even code, saturating at 6.
Readings where the definition leaves room (each pinned in tests/test_mxfp4.py):
  * s is clamped to [-126, 127] (E8M0 byte 1..254); an all-zero block gets byte 0 and codes 0;
  * the sign bit is set iff x < 0 (a negative value that rounds to magnitude 0 gives code 8);
  * packing: element 2j of a row in the low nibble of byte j, element 2j + 1 in the high nibble.
"""

from __future__ import annotations

import numpy as np

E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
BLOCK = 32


def _f64(x):
    if hasattr(x, "detach"):
        import torch
        return x.detach().to(device="cpu", dtype=torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def e2m1_code(v):
    """Magnitude code (0..7) of the E2M1 value nearest to |v|, ties to the even code, values
    beyond 6 saturating at code 7.  Written as a nearest-neighbour search over the 8 values."""
    a = np.abs(np.asarray(v, dtype=np.float64))
    dist = np.abs(a[..., None] - E2M1)                       # [..., 8]
    best = dist.min(axis=-1, keepdims=True)
    cand = dist == best                                      # one or two nearest codes
    codes = np.arange(8)
    # among the nearest codes prefer an even one (the two candidates of a tie are neighbours)
    pref = np.where(cand, np.where(codes % 2 == 0, 0, 1), 2)
    return pref.argmin(axis=-1)


def quantize(x):
    """x [..., D] (D a multiple of 32) -> (codes uint8 [..., D] with the sign in bit 3, scale
    bytes uint8 [..., D / 32])."""
    x = _f64(x)
    D = x.shape[-1]
    if D % BLOCK:
        raise ValueError("the last dimension must be a multiple of 32")
    xb = x.reshape(x.shape[:-1] + (D // BLOCK, BLOCK))
    amax = np.abs(xb).max(axis=-1)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(amax > 0, amax, 1.0)))
    s = np.clip(e - 2, -126, 127)
    sbyte = np.where(amax > 0, s + 127, 0).astype(np.uint8)
    v = xb / np.exp2(s)[..., None]
    mag = e2m1_code(v)
    codes = (mag + np.where(xb < 0, 8, 0)).astype(np.uint8)
    return codes.reshape(x.shape), sbyte


def dequantize(codes, sbytes):
    """Values of codes [..., D] and scale bytes [..., D / 32] (float64).  Byte 0 reads as 0."""
    codes = np.asarray(codes).astype(np.int64)
    sb = np.asarray(sbytes).astype(np.int64)
    D = codes.shape[-1]
    mag = E2M1[codes & 7] * np.where(codes & 8, -1.0, 1.0)
    scale = np.where(sb > 0, np.exp2(sb - 127.0), 0.0)
    return (mag.reshape(codes.shape[:-1] + (D // BLOCK, BLOCK)) * scale[..., None]).reshape(codes.shape)


def pack(codes):
    """codes [..., D] -> bytes [..., D / 2]: element 2j low nibble, 2j + 1 high nibble."""
    c = np.asarray(codes).astype(np.uint8)
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def unpack(packed):
    p = np.asarray(packed).astype(np.uint8)
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.uint8)
    out[..., 0::2] = p & 15
    out[..., 1::2] = p >> 4
    return out
