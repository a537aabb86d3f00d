"""Helpers for the GPU parity tests: host <-> device copies and the
comparison rules for the fused compressor's outputs."""
from __future__ import annotations

import hashlib

import numpy as np
import torch

import oracle
from tests import spec


def dev(a: np.ndarray) -> torch.Tensor:
    """numpy -> device tensor with the same bits (uint16 as int16)."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).cuda()


def host(t: torch.Tensor, dtype=None) -> np.ndarray:
    a = t.detach().cpu().numpy()
    if dtype is not None:
        a = a.view(dtype)
    return a


def sha(a: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


def row_parts(cache: np.ndarray, layout: str, page_size: int, slot: int):
    db, sb, _, _ = oracle.layout_bytes(layout)
    p, r = divmod(int(slot), page_size)
    d = cache[p, r * db:(r + 1) * db]
    s = cache[p, page_size * db + r * sb: page_size * db + (r + 1) * sb]
    return d, s


def written_mask(cache_shape, layout: str, page_size: int, slots) -> np.ndarray:
    db, sb, _, _ = oracle.layout_bytes(layout)
    m = np.zeros(cache_shape, bool)
    for slot in slots:
        p, r = divmod(int(slot), page_size)
        m[p, r * db:(r + 1) * db] = True
        m[p, page_size * db + r * sb: page_size * db + (r + 1) * sb] = True
    return m


# --------------------------------------------------------------- tolerances
REL = 2e-2


def assert_latent_close(g: np.ndarray, o: np.ndarray, what="latent"):
    """|g - o| <= 2e-2 |o| + 2e-2 * 2^-6 * rms(o_row), elementwise (bf16 rows)."""
    gv, ov = spec.bf16_value(g), spec.bf16_value(o)
    rms = np.sqrt(np.mean(ov * ov, axis=-1, keepdims=True))
    tol = REL * np.abs(ov) + REL * 2.0 ** -6 * rms
    bad = np.abs(gv - ov) > tol
    assert not bad.any(), (what, np.argwhere(bad)[:5], gv[bad][:5], ov[bad][:5])


def _ordinal_fp8(c):
    c = c.astype(np.int64)
    mag = c & 0x7F
    return np.where(c & 0x80, -mag, mag)


def _ordinal_fp4(n):
    n = n.astype(np.int64)
    mag = n & 7
    return np.where(n & 8, -mag, mag)


def assert_rows_close(layout: str, gd, gs, od, os_, ref_vals):
    """Fused-path cache rows: where the scale bytes agree every code is
    within one step of the oracle's; where a scale differs the dequantized
    values agree within the latent tolerance plus one quantization step.
    gd/gs/od/os_: [n, data], [n, scale] byte arrays; ref_vals: the oracle's
    fp64 values of the rows (bf16 of z) for the tolerance."""
    n = gd.shape[0]
    gq = oracle.dequant_row(layout, gd, gs)
    oq = oracle.dequant_row(layout, od, os_)
    gv, ov = spec.bf16_value(gq), spec.bf16_value(oq)
    t8 = spec.e4m3_table()
    if layout == "V41_FP4":
        nib = lambda d: np.stack([d & 0xF, d >> 4], -1).reshape(n, 512)
        gc, oc = _ordinal_fp4(nib(gd)), _ordinal_fp4(nib(od))
        same = np.repeat(gs == os_, 16, axis=1)
        step = np.repeat(np.abs(t8[np.maximum(gs, os_)]), 16, axis=1) * 2.0
        nq = 512
    else:
        nq = 512 if layout == "V41" else 448
        g = 32 if layout == "V41" else 64
        gc, oc = _ordinal_fp8(gd[:, :nq]), _ordinal_fp8(od[:, :nq])
        same = np.repeat(gs[:, : nq // g] == os_[:, : nq // g], g, axis=1)
        E = np.maximum(gs[:, : nq // g], os_[:, : nq // g]).astype(np.float64)
        step = np.repeat(2.0 ** (E - 127) * 32.0, g, axis=1)     # one step near 448 s
    dc = np.abs(gc - oc)
    assert np.all(dc[same[:, :nq]] <= 1), ("code step", np.argwhere((dc > 1) & same[:, :nq])[:5])
    rv = np.abs(ref_vals[:, :nq])
    rms = np.sqrt(np.mean(ref_vals * ref_vals, axis=-1, keepdims=True))
    tol = REL * rv + REL * 2.0 ** -6 * rms + step
    diff = np.abs(gv[:, :nq] - ov[:, :nq])
    bad = (~same[:, :nq]) & (diff > tol)
    assert not bad.any(), ("scale-differs rows", np.argwhere(bad)[:5])
    if layout == "V4":
        assert_latent_close(gq[:, 448:], oq[:, 448:], "v4 rope part")
