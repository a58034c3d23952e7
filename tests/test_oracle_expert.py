"""Pins of weight decoding and the fp64 expert (CPU only): bf16 over all
65,536 codes, E2M1 and E8M0 against the OCP MX table, nibble and scale order
against the generator's source values, and the SwiGLU expert against
explicit loops and scipy's logistic function."""
import json
import math
import os

import numpy as np
import pytest
from scipy.special import expit

import workload as W
from oracle import expert as X


def bf16_formula(code):
    s = (code >> 15) & 1
    e = (code >> 7) & 0xFF
    m = code & 0x7F
    sign = -1.0 if s else 1.0
    if e == 0xFF:
        return sign * math.inf if m == 0 else math.nan
    if e == 0:
        return sign * m * 2.0 ** (-133)          # 2^-126 * m / 128
    return sign * (1.0 + m / 128.0) * 2.0 ** (e - 127)


def test_bf16_all_codes():
    codes = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = X.bf16_to_f64(codes)
    ref = np.array([bf16_formula(int(c)) for c in codes])
    nan = np.isnan(ref)
    assert (np.isnan(got) == nan).all()
    assert (got[~nan] == ref[~nan]).all()
    # signed zero kept
    assert math.copysign(1.0, got[0x8000]) == -1.0


def test_e2m1_and_e8m0_vs_ocp_table(golden_dir):
    with open(os.path.join(golden_dir, "ocp_mx_e2m1.json")) as f:
        g = json.load(f)
    for code, val in g["e2m1_positive"].items():
        c = int(code)
        assert X.e2m1_value(c) == val
        assert X.e2m1_value(c | 8) == -val
    assert X.e8m0_value(127) == 1.0 and X.e8m0_value(128) == 2.0
    assert X.e8m0_value(0) == math.ldexp(1.0, -127)
    assert X.e8m0_value(254) == math.ldexp(1.0, 127)
    assert math.isnan(X.e8m0_value(255))
    for b in range(255):
        assert X.e8m0_value(b) == math.ldexp(1.0, b - 127)


def test_mxfp4_nibble_and_scale_order():
    """Hand-built 1 x 64 matrix: element i is code (i % 16), block 0 scale 2,
    block 1 scale 1/4."""
    codes = np.zeros(32, np.uint8)
    for j in range(32):
        lo, hi = (2 * j) % 16, (2 * j + 1) % 16
        codes[j] = lo | (hi << 4)
    scales = np.array([128, 125], np.uint8)
    got = X.mxfp4_matrix(codes, scales, 1, 64)[0]
    for i in range(64):
        sc = 2.0 if i < 32 else 0.25
        assert got[i] == X.e2m1_value(i % 16) * sc


def test_mxfp4_bank_decodes_close_to_source_normals():
    """The generator quantises known normals; the oracle's decode of the bank
    must land within half a grid step of each source value (a swapped nibble,
    a transposed scale or a wrong matrix offset would not)."""
    wl = W.Workload(name="t", L=1, E=2, k=1, H=64, I=96, w_dtype="mxfp4", act_dtype="bf16",
                    n_slots=1, bw_pcie_mbps=1, bw_host_mbps=2, steps=1, T=1, seed=77)
    raw = W.bank(wl, 1)
    wg, wu, wd = X.expert_weights(raw, "mxfp4", wl.H, wl.I)
    srcs = [(wg, 0, wl.I, wl.H), (wu, 1, wl.I, wl.H), (wd, 2, wl.H, wl.I)]
    for dec, mat, rows, cols in srcs:
        v = W.normal_f32(wl.seed, W.TAG_WEIGHT, 1, mat, rows * cols, wl.w_sigma).astype(np.float64)
        v = v.reshape(rows, cols)
        blk = v.reshape(rows, cols // 32, 32)
        amax = np.abs(blk).max(-1)
        scale = 2.0 ** (np.floor(np.log2(amax)) - 2)
        err = np.abs(dec.reshape(rows, cols // 32, 32) - blk)
        # grid steps are 0.5, 1, 2 scale units below 2, 4, 6; above 6 the
        # quantiser saturates (amax / scale lies in [4, 8))
        a = np.abs(blk) / scale[..., None]
        step = np.where(a < 2, 0.5, np.where(a < 4, 1.0, 2.0))
        bound = np.where(a <= 6, 0.5 * step, a - 6.0) * scale[..., None]
        assert (err <= bound * (1 + 1e-6) + 1e-12).all()
        assert (a < 8).all() and (a.max(-1) >= 4).all()


def test_bf16_bank_equals_rounded_source():
    wl = W.Workload(name="t", L=1, E=1, k=1, H=32, I=16, w_dtype="bf16", act_dtype="bf16",
                    n_slots=1, bw_pcie_mbps=1, bw_host_mbps=2, steps=1, T=1, seed=5)
    raw = W.bank(wl, 0)
    wg, wu, wd = X.expert_weights(raw, "bf16", wl.H, wl.I)
    for dec, mat in ((wg, 0), (wu, 1), (wd, 2)):
        v = W.normal_f32(wl.seed, W.TAG_WEIGHT, 0, mat, wl.H * wl.I, wl.w_sigma)
        assert np.abs(dec.ravel() - v) .max() <= np.abs(v).max() * 2.0 ** -8


def test_ffn_against_loops_and_expit():
    rng = np.random.default_rng(0)
    H, I, T = 5, 3, 4
    wg, wu = rng.normal(size=(I, H)), rng.normal(size=(I, H))
    wd = rng.normal(size=(H, I))
    x = rng.normal(size=(T, H))
    got = X.ffn(x, (wg, wu, wd))
    for t in range(T):
        h = []
        for i in range(I):
            g = sum(wg[i, c] * x[t, c] for c in range(H))
            u = sum(wu[i, c] * x[t, c] for c in range(H))
            h.append(g * expit(g) * u)
        for r in range(H):
            ref = sum(wd[r, i] * h[i] for i in range(I))
            assert got[t, r] == pytest.approx(ref, rel=1e-12, abs=1e-14)


def test_silu_extremes():
    z = np.array([-1e4, -50.0, 0.0, 50.0, 1e4])
    s = X.silu(z)
    assert np.all(np.isfinite(s))
    assert s[0] == 0.0 and s[2] == 0.0 and s[4] == 1e4
    assert np.allclose(s, z * expit(z), rtol=1e-15, atol=0)
