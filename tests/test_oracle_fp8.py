"""Pins of the oracle's FP8 functions (E4M3 codes, UE8M0 block scales, FP8 expert FFN).

The element format is pinned to the format's fixed points and to torch's float8_e4m3fn
conversion (an independent implementation of the same format); the scale rule to the
exact 2^-8 value the LightLLM PR #1687 page's quantisation test expects and to its
defining inequality; the FP8 FFN to numpy fp64 matrix products on exactly representable
inputs.
"""
import numpy as np
import pytest
import torch

import oracle

QB = oracle.QBLOCK


def torch_encode(v: np.ndarray) -> np.ndarray:
    """torch's conversion of fp32 values to float8_e4m3fn codes."""
    t = torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_e4m3_fixed_points():
    v = oracle.e4m3_value(np.arange(256))
    assert v[0x7E] == 448.0 and v[0xFE] == -448.0          # largest finite
    assert v[0x08] == 2.0 ** -6                             # smallest normal
    assert v[0x01] == 2.0 ** -9                             # smallest subnormal
    assert v[0x38] == 1.0
    assert v[0x00] == 0.0 and np.signbit(v[0x80]) and v[0x80] == 0.0
    assert sorted(np.nonzero(np.isnan(v))[0].tolist()) == [0x7F, 0xFF]
    pos = v[:0x7F]
    assert np.all(np.diff(pos) > 0)                         # codes 0..126 increase
    assert np.array_equal(v[0x80:0xFF], -pos)               # sign bit


def test_e4m3_decode_matches_torch():
    c = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(c.copy()).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = oracle.e4m3_value(c)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])


def test_e4m3_encode_matches_torch_at_midpoints_and_random():
    pos = oracle.e4m3_value(np.arange(0x7F))
    mids = (pos[:-1] + pos[1:]) / 2                       # exact in fp32
    f = np.concatenate([pos, mids])
    f = np.concatenate([f, -f]).astype(np.float32)
    up = np.nextafter(f, np.float32(np.inf))
    dn = np.nextafter(f, np.float32(-np.inf))
    rng = np.random.default_rng(7)
    rnd = np.concatenate([rng.uniform(-448, 448, 200_000),
                          rng.uniform(-2.0 ** -5, 2.0 ** -5, 100_000)]).astype(np.float32)
    v = np.concatenate([f, up, dn, rnd])
    v = v[np.abs(v) <= 448]
    got = oracle.e4m3_encode(v.astype(np.float64))
    assert np.array_equal(got, torch_encode(v))
    # round trip of every finite code
    c = np.array([i for i in range(256) if i not in (0x7F, 0xFF)], np.uint8)
    assert np.array_equal(oracle.e4m3_encode(oracle.e4m3_value(c)), c)


def test_ue8m0_page_value_and_definition():
    # the PR's quantisation test expects a scale of exactly 2^-8 (rtol = atol = 0)
    exp_of = lambda a: int(oracle.ue8m0([a])[0]) - 127
    for amax in (1.75, 1.0, 0.9, 1.5, 0.8750001):
        assert exp_of(amax) == -8, amax
        assert np.ldexp(1.0, exp_of(amax)) == 2.0 ** -8
    assert exp_of(0.875) == -9                             # 0.875 = 448 * 2^-9 exactly
    assert oracle.ue8m0([448.0])[0] == 127 and oracle.ue8m0([449.0])[0] == 128
    assert oracle.ue8m0([0.0])[0] == 127
    rng = np.random.default_rng(3)
    amax = np.exp(rng.uniform(-60, 60, 50_000))
    e = oracle.ue8m0(amax).astype(np.int64) - 127
    assert np.all(amax <= 448.0 * np.ldexp(1.0, e))
    assert np.all(amax > 448.0 * np.ldexp(1.0, e - 1))


def test_quant_rows_block_rule_and_error_bound():
    rng = np.random.default_rng(5)
    x = (rng.standard_normal((40, 256)) * np.exp(rng.uniform(-8, 8, (40, 1)))).astype(np.float32)
    x[3, 32:64] = 0.0                                     # an all-zero block
    codes, scales = oracle.quant_rows(x)
    assert codes.shape == (40, 256) and scales.shape == (40, 8)
    blocks = x.reshape(40, 8, QB).astype(np.float64)
    e = scales.astype(np.int64) - 127
    assert np.array_equal(scales, oracle.ue8m0(np.abs(blocks).max(axis=2)).reshape(40, 8))
    assert scales[3, 1] == 127 and np.all(codes[3, 32:64] == 0)
    # codes are the format's rounding of x * 2^-e (torch's conversion), blockwise
    scaled = (blocks * np.ldexp(1.0, -e)[:, :, None]).astype(np.float32).reshape(40, 256)
    assert np.array_equal(codes, torch_encode(scaled))
    # rounding to nearest: error <= half a step (2^-4 relative for normals, 2^-10 * 2^e below)
    deq = oracle.dequant(codes, scales, axis=1)
    sc = np.ldexp(1.0, np.repeat(e, QB, axis=1))
    bound = np.maximum(np.abs(x) * 2.0 ** -4, sc * 2.0 ** -10)
    assert np.all(np.abs(deq - x) <= bound)


def test_quant_weights_blocks_run_along_the_reduction_dimension():
    rng = np.random.default_rng(9)
    w = rng.standard_normal((3, 64, 40)).astype(np.float32)
    codes, scales = oracle.quant_weights(w)
    assert codes.shape == (3, 64, 40) and scales.shape == (3, 2, 40)
    for e in range(3):
        c2, s2 = oracle.quant_rows(np.ascontiguousarray(w[e].T))
        assert np.array_equal(codes[e], c2.T) and np.array_equal(scales[e], s2.T)


def exact_fp8(rng, shape_rows, n):
    """Rows of n values exactly representable as E4M3 with block scales that the scale rule
    reproduces: random codes, one element per block forced into (224, 448]."""
    codes = rng.integers(0, 0x7F, (shape_rows, n), dtype=np.int64).astype(np.uint8)
    codes |= (rng.integers(0, 2, codes.shape) << 7).astype(np.uint8)
    top = rng.integers(0x77, 0x7F, (shape_rows, n // QB))
    pos = rng.integers(0, QB, (shape_rows, n // QB))
    for r in range(shape_rows):
        for b in range(n // QB):
            codes[r, b * QB + pos[r, b]] = top[r, b] | (codes[r, b * QB + pos[r, b]] & 0x80)
    scales = rng.integers(120, 124, (shape_rows, n // QB)).astype(np.uint8)
    return codes, scales


@pytest.mark.parametrize("E,H,I,n", [(1, 64, 64, 7), (3, 96, 64, 25)])
def test_ffn_rows_fp8_against_numpy(E, H, I, n):
    rng = np.random.default_rng(E * 1000 + H)
    xq, xs = exact_fp8(rng, n, H)
    x = oracle.dequant(xq, xs, axis=1)
    # re-quantising the exactly representable rows reproduces codes and scales
    c2, s2 = oracle.quant_rows(x)
    assert np.array_equal(s2, xs)
    assert np.array_equal(oracle.dequant(c2, s2, axis=1), x)
    ws = {}
    for name, (K, N) in (("g", (H, I)), ("u", (H, I)), ("d", (I, H))):
        c, s = exact_fp8(rng, E * N, K)
        c = np.ascontiguousarray(np.transpose(c.reshape(E, N, K), (0, 2, 1)))
        s = np.ascontiguousarray(np.transpose(s.reshape(E, N, K // QB), (0, 2, 1)))
        ws[name] = (c, s)
    deq = {k: oracle.dequant(c, s, axis=1) for k, (c, s) in ws.items()}
    row_expert = rng.integers(0, E, n).astype(np.int32)
    yp, a, ac, asc = oracle.ffn_rows_fp8(xq, xs, row_expert, ws["g"], ws["u"], ws["d"], want_a=True)
    for r in range(n):
        e = row_expert[r]
        g = x[r] @ deq["g"][e]
        u = x[r] @ deq["u"][e]
        with np.errstate(over="ignore"):  # exp(-g) = inf for very negative g: silu -> -0
            a_ref = g / (1.0 + np.exp(-g)) * u
        assert np.allclose(a[r], a_ref, rtol=1e-12, atol=1e-12 * np.abs(a_ref).max())
        # a is quantised with the row rule before the down projection
        qc, qs = oracle.quant_rows(a[r][None, :])
        assert np.array_equal(ac[r], qc[0]) and np.array_equal(asc[r], qs[0])
        y_ref = oracle.dequant(qc, qs, axis=1)[0] @ deq["d"][e]
        assert np.allclose(yp[r], y_ref, rtol=1e-12, atol=1e-12 * np.abs(y_ref).max())
