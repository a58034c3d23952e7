"""The seeded generator (CPU only): Philox4x32-10 known-answer vectors,
determinism, stream independence and the stated workload statistics."""
import numpy as np
import pytest

import workload as W


def test_philox_known_answers():
    """Known-answer vectors of Philox4x32-10 published with the Random123
    library (Salmon et al., SC'11)."""
    kat = [
        ([0, 0, 0, 0], [0, 0], [0x6627e8d5, 0xe169c58d, 0xbc57ac4c, 0x9b00dbd8]),
        ([0xffffffff] * 4, [0xffffffff] * 2, [0x408f276d, 0x41c83b0e, 0xa20bc7c6, 0x6d5451fd]),
        ([0x243f6a88, 0x85a308d3, 0x13198a2e, 0x03707344], [0xa4093822, 0x299f31d0],
         [0xd16cfe09, 0x94fdcceb, 0x5001e420, 0x24126ea1]),
    ]
    for ctr, key, out in kat:
        assert W.philox_block(ctr, key).tolist() == out


def test_streams_deterministic_and_distinct():
    a = W.normal_f32(1, 2, 3, 4, 1001)
    b = W.normal_f32(1, 2, 3, 4, 1001)
    c = W.normal_f32(1, 2, 3, 5, 1001)
    assert np.array_equal(a, b) and not np.array_equal(a, c)
    # a prefix of a longer stream is the shorter stream
    assert np.array_equal(W.normal_f32(1, 2, 3, 4, 37), a[:37])
    z = W.normal_f32(9, 9, 9, 9, 400_000)
    assert abs(z.mean()) < 0.01 and abs(z.std() - 1) < 0.01


def test_bank_is_regenerable_alone():
    wl = W.TINY
    many = np.empty(W.slot_stride(wl) * wl.n_ids, np.uint8)
    W.fill_banks(wl, many, 0, wl.n_ids)
    for u in (0, 7, 15):
        s = W.slot_stride(wl)
        assert np.array_equal(many[u * s:(u + 1) * s], W.bank(wl, u))


def test_slot_sizes():
    assert W.expert_bytes(W.TINY) == 98_304
    assert W.expert_bytes(W.QWEN_BF16) == 9_437_184
    assert W.expert_bytes(W.DSV4_MXFP4) == 13_369_344
    for wl in W.WORKLOADS:
        assert W.slot_stride(wl) % 256 == 0
    assert W.QWEN_BF16.n_slots == int(0.37 * W.QWEN_BF16.n_ids)
    assert W.DSV4_MXFP4.n_slots == int(0.11 * W.DSV4_MXFP4.n_ids)
    assert W.QWEN_ELASTIC.resize == {128: int(0.15 * 6144), 256: int(0.30 * 6144), 384: 1843}
    assert W.DSV4_PREFILL.n_slots == 2 * W.DSV4_PREFILL.E


def test_zipf_popularity():
    wl = W.DSV4_MXFP4
    lp = W.log_popularity(wl, 3)
    p = np.exp(lp)
    assert p.sum() == pytest.approx(1.0)
    r = np.sort(p)[::-1]
    assert r[0] / r[9] == pytest.approx(10 ** wl.zipf_s, rel=1e-9)
    assert sorted(W.popularity_order(wl, 3).tolist()) == list(range(wl.E))


def test_reuse_calibration():
    """The stickiness bonus gives mean step-to-step reuse 0.60 +- 0.01 on the
    Qwen-shaped decode workload (measured on its own first 128 steps)."""
    lg = W.decode_logits(W.QWEN_BF16, steps=128)
    assert abs(W.reuse_fraction(lg, W.QWEN_BF16.k) - 0.60) <= 0.01


def test_uniforms_strictly_inside_unit_interval_and_logits_finite():
    u = W.uniform(1005, W.TAG_NOISE, 0, 0, 1 << 20)
    assert u.min() > 0.0 and u.max() < 1.0
    # the largest possible draw stays below 1 and gives a finite Gumbel
    top = ((2 ** 24 - 1) + 0.5) / 2 ** 24
    assert top < 1.0 and np.isfinite(-np.log(-np.log(top)))
    lg = W.decode_logits(W.QWEN_ELASTIC, steps=160)
    assert np.isfinite(lg).all()
