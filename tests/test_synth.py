"""The input generator: storage formats and determinism (no GPU)."""
import os

import numpy as np
import pytest

import moe_synth as S

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def bits(f):
    return int(np.array([f], dtype=np.float32).view(np.uint32)[0])


def f32(b):
    return np.array([b], dtype=np.uint32).view(np.float32)


@pytest.mark.parametrize("in_bits,out_bits", [
    (0x3F800000, 0x3F80),  # 1.0
    (0x3F808000, 0x3F80),  # halfway, even stays
    (0x3F818000, 0x3F82),  # halfway, odd rounds up to even
    (0x3F807FFF, 0x3F80),
    (0x3F808001, 0x3F81),
    (0xBF808001, 0xBF81),  # sign is kept
    (0x80000000, 0x8000),  # -0.0
    (0x7F800000, 0x7F80),  # +inf
    (0x7F7FFFFF, 0x7F80),  # largest float rounds to inf
    (0x00000001, 0x0000),  # smallest subnormal rounds to +0
])
def test_bf16_round_to_nearest_even(in_bits, out_bits):
    assert int(S.bf16_bits(f32(in_bits))[0]) == out_bits


def test_bf16_nan_stays_nan_and_widening_is_exact():
    r = S.bf16_bits(np.array([np.nan], dtype=np.float32))
    assert np.isnan(S.bf16_bits_to_f32(r))[0]
    b = np.arange(0, 0x7F80, 97, dtype=np.uint16)
    assert np.array_equal(S.bf16_bits(S.bf16_bits_to_f32(b)), b)


def test_quantiser_invariants():
    g = np.random.default_rng(0)
    w = S.bf16_bits_to_f32(S.bf16_bits(g.standard_normal((3, 40, 64)).astype(np.float32) * 0.02))
    w[1, 5] = 0.0  # an all-zero channel
    q, s = S.quantize_int8_rows(w)
    assert q.dtype == np.int8 and s.dtype == np.float32 and s.shape == (3, 40)
    assert np.all(np.abs(q.astype(int)) <= 127)
    nz = s > 0
    assert np.all(np.max(np.abs(q.astype(int)), axis=-1)[nz] == 127)
    assert s[1, 5] == 0 and np.all(q[1, 5] == 0)
    err = np.abs(w.astype(np.float64) - q.astype(np.float64) * s[..., None].astype(np.float64))
    # half a step, plus the fp32 rounding of w / scale (|w / scale| <= 127.5)
    assert np.all(err <= s[..., None].astype(np.float64) * (0.5 + 128 * 2.0 ** -24))


def test_quantiser_rounds_half_to_even():
    w = np.array([[127.0, 0.5, 1.5, 2.5, -0.5, -2.5]], dtype=np.float32)  # scale = 1
    q, s = S.quantize_int8_rows(w)
    assert s[0] == 1.0
    assert q[0].tolist() == [127, 0, 2, 2, 0, -2]


def read_golden(name):
    vals = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                k, v = line.split()
                vals[k] = float(v)
    return vals


def test_int8_format_reproduces_the_pages_memory_reduction():
    g = read_golden("int8_memory_reduction.txt")
    d, I = int(g["d_model"]), int(g["d_ff"])
    w = np.zeros((I, d), dtype=np.float32)
    w[:, 0] = 1.0
    qg, sg = S.quantize_int8_rows(w)
    qd, sd = S.quantize_int8_rows(np.zeros((d, I), dtype=np.float32) + 1.0)
    int8_bytes = 2 * (qg.nbytes + sg.nbytes) + qd.nbytes + sd.nbytes
    bf16_bytes = 2 * (3 * d * I)
    reduction = 100.0 * (1.0 - int8_bytes / bf16_bytes)
    assert round(reduction, 2) == g["reduction_percent"]


def test_generator_is_deterministic_and_stream_separated():
    wl = S.TINY_F32
    a = S.make_layer(wl, 0, seed=0)
    b = S.make_layer(wl, 0, seed=0, threads=1)
    c = S.make_layer(wl, 0, seed=1)
    for f in ("w_router", "w_gate", "w_up", "w_down"):
        assert np.array_equal(getattr(a, f), getattr(b, f))
        assert not np.array_equal(getattr(a, f), getattr(c, f))
    assert not np.array_equal(a.w_gate, a.w_up)
    assert a.w_gate.shape == (8, 512, 256) and a.w_down.shape == (8, 256, 512)
    assert a.w_router.shape == (8, 256) and a.w_gate.dtype == np.float32
    x = S.make_tokens(wl, 16)
    assert x.shape == (16, 256) and abs(float(x.std()) - 1.0) < 0.05
    assert abs(float(a.w_gate.std()) - 0.02) < 0.001


def test_generator_bf16_int8_and_zipf_layouts():
    import dataclasses
    wl = dataclasses.replace(S.DEEPSEEK_I8, d=64, I=32)
    L = S.make_layer(wl)
    assert L.w_gate.dtype == np.int8 and L.w_gate.shape == (66, 32, 64)
    assert L.s_gate.shape == (66, 32) and L.s_down.shape == (66, 64)
    assert L.w_router.dtype == np.uint16 and L.w_router.shape == (64, 64)
    b = L.bias
    assert b.shape == (64,) and b.max() == 0.0
    assert np.isclose(b.min(), -1.2 * np.log(64), rtol=1e-6)
    assert len(np.unique(b)) == 64
