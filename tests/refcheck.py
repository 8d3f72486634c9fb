"""Independent second formulations used to pin the oracle (tests only).

None of these call the oracle: they rebuild each rule a different way
(brute-force nearest-neighbour search over torch's float8 decode table,
torch's own casts, numpy float32 arithmetic) so that a mistake in the
oracle's formulation shows up as a disagreement.
"""
from __future__ import annotations

import numpy as np
import torch

E4M3, E5M2 = 0, 1
TORCH_DT = {E4M3: torch.float8_e4m3fn, E5M2: torch.float8_e5m2}
FMAX = {E4M3: 448.0, E5M2: 57344.0}


def torch_decode_table(fmt: int) -> np.ndarray:
    codes = torch.arange(256, dtype=torch.uint8)
    return codes.view(TORCH_DT[fmt]).to(torch.float64).numpy()


def nearest_code(x: np.ndarray, fmt: int) -> np.ndarray:
    """Saturating round-to-nearest, ties-to-even-code, by exhaustive search.

    x is clamped to [-max, max] (saturation), then for every element the code
    whose value is nearest is chosen; among equally near codes the one with
    an even code (last bit 0) wins.  NaN -> 0x7F | sign.
    """
    with np.errstate(invalid="ignore"):    # signalling NaN payloads raise the flag when widened
        x = np.asarray(x, dtype=np.float32).astype(np.float64).reshape(-1)
    table = torch_decode_table(fmt)
    pos_codes = np.array([c for c in range(128) if np.isfinite(table[c])], dtype=np.int64)
    pos_vals = table[pos_codes]
    out = np.empty(x.size, dtype=np.uint8)
    sign = np.signbit(x)
    nan = np.isnan(x)
    ax = np.minimum(np.abs(np.where(nan, 0.0, x)), FMAX[fmt])
    # distances to every non-negative finite value: [n, ncodes]
    best = np.empty(x.size, dtype=np.int64)
    step = 1 << 16
    for i in range(0, x.size, step):
        d = np.abs(ax[i:i + step, None] - pos_vals[None, :])
        dmin = d.min(axis=1, keepdims=True)
        cand = d == dmin
        # prefer even codes among ties
        even = (pos_codes[None, :] & 1) == 0
        pick_even = cand & even
        has_even = pick_even.any(axis=1)
        idx = np.where(has_even, pick_even.argmax(axis=1), cand.argmax(axis=1))
        best[i:i + step] = pos_codes[idx]
    out[:] = best.astype(np.uint8) | np.where(sign, 0x80, 0x00).astype(np.uint8)
    out[nan] = (0x7F | np.where(sign[nan], 0x80, 0)).astype(np.uint8)
    return out


def torch_cast_codes(x: np.ndarray, fmt: int) -> np.ndarray:
    """torch's (non-saturating, RNE) float32 -> float8 cast, as codes."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(TORCH_DT[fmt]).view(torch.uint8).numpy()


def torch_overflows(x: np.ndarray, fmt: int) -> np.ndarray:
    """True where torch's non-saturating cast of a non-NaN value gives NaN/Inf."""
    x = np.asarray(x, dtype=np.float32)
    t = torch.from_numpy(np.ascontiguousarray(x)).to(TORCH_DT[fmt]).to(torch.float32).numpy()
    return ~np.isnan(x) & ~np.isfinite(t)


def torch_bf16(x: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def f32_from_bf16(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def np_scale(amax: np.ndarray, margin: float, fmt: int) -> np.ndarray:
    """numpy float32 evaluation of max / (amax * margin) with the fallback to 1."""
    amax = np.asarray(amax, dtype=np.float32)
    with np.errstate(all="ignore"):
        d = (amax * np.float32(margin)).astype(np.float32)
        s = (np.float32(FMAX[fmt]) / d).astype(np.float32)
    bad = ~(d > 0) | ~np.isfinite(d) | ~np.isfinite(s)
    return np.where(bad, np.float32(1.0), s).astype(np.float32)


def brute_quantize(h: np.ndarray, relu2: bool, fmt: int, scale=None, group: bool = False):
    """Brute-force composition of the quantizer from torch/numpy primitives.

    Returns (bf16 copy bits, codes, amax bits, saturation count, group scale_inv).
    """
    h = np.asarray(h, dtype=np.uint16)
    x = f32_from_bf16(h)
    if relu2:
        with np.errstate(all="ignore"):
            a = np.where(x > 0, (x * x).astype(np.float32), np.float32(0.0)).astype(np.float32)
        b = torch_bf16(a)
    else:
        b = h.copy()
    bf = f32_from_bf16(b)
    mag = (b & 0x7FFF).astype(np.uint32) << 16
    amax_bits = int(mag.max()) if mag.size else 0
    gsi = None
    if group:
        rows, cols = h.shape
        g = mag.reshape(rows, cols // 128, 128).max(axis=2).view(np.float32)
        sg = np_scale(g, 1.0, fmt)
        with np.errstate(all="ignore"):
            gsi = (np.float32(1.0) / sg).astype(np.float32)
        s = np.repeat(sg, 128, axis=1).reshape(rows, cols)
    else:
        s = np.float32(scale)
    with np.errstate(all="ignore"):
        v = (bf * s).astype(np.float32)
    codes = nearest_code(v, fmt).reshape(h.shape)
    sat = int(torch_overflows(v, fmt).sum())
    return b, codes, amax_bits, sat, gsi


def boundary_values(fmt: int) -> np.ndarray:
    """float32 values at and around every rounding boundary of the format."""
    table = torch_decode_table(fmt)
    vals = np.unique(table[np.isfinite(table) & (table >= 0)])
    pts = [vals, (vals[:-1] + vals[1:]) / 2.0]
    # past the top: the midpoint to the next (non-finite) step and beyond
    top = vals[-1]
    gap = vals[-1] - vals[-2]
    pts.append(np.array([top + gap / 2, top + gap, top * 2, 1e30, 2.0 ** -10, 2.0 ** -17,
                         2.0 ** -149, 0.0]))
    base = np.concatenate(pts).astype(np.float32)
    up = np.nextafter(base, np.float32(np.inf))
    dn = np.nextafter(base, np.float32(-np.inf))
    allv = np.concatenate([base, up, dn, np.array([np.inf, np.nan], dtype=np.float32)])
    allv = np.concatenate([allv, -allv])
    return allv.astype(np.float32)
