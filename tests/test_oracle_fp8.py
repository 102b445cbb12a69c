"""Pins for the FP8 (E4M3) quantisation oracle: the format's closed forms, a
hand-worked fixture, torch's own float8_e4m3fn conversion (a library special
case), error bounds, group invariants and exactness on representable data
(no GPU)."""
import json
import os

import numpy as np
import pytest
import torch

from oracle import fp8


def _golden(golden_dir):
    with open(os.path.join(golden_dir, "e4m3_quant_example.json")) as f:
        return json.load(f)


def _bits(x):
    return hex(int(np.float32(x).view(np.uint32)))


# ------------------------------------------------------------ the format ---

def test_e4m3_closed_form_codes():
    # Sign, exponent (bias 7) and mantissa fields of a few codes, by hand.
    table = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x38: 1.0, 0x39: 1.125,
             0x40: 2.0, 0x70: 128.0, 0x71: 144.0, 0x77: 240.0, 0x78: 256.0, 0x7E: 448.0,
             0x80: -0.0, 0xB8: -1.0, 0xFE: -448.0}
    for code, value in table.items():
        got = fp8.e4m3_value(np.uint8(code))
        assert got == value and np.signbit(got) == np.signbit(value), hex(code)
    assert np.isnan(fp8.e4m3_value(np.uint8(0x7F))) and np.isnan(fp8.e4m3_value(np.uint8(0xFF)))
    finite = fp8.e4m3_value(np.arange(256, dtype=np.uint8))
    finite = finite[np.isfinite(finite)]
    assert finite.size == 254 and finite.max() == 448.0 and finite.min() == -448.0


def test_e4m3_decode_matches_torch_for_every_code():
    codes = np.arange(256, dtype=np.uint8)
    ours = fp8.e4m3_value(codes)
    lib = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    np.testing.assert_array_equal(ours, lib)


def _e4m3_grid():
    v = fp8.e4m3_value(np.arange(256, dtype=np.uint8))
    return np.unique(v[np.isfinite(v)])


def test_e4m3_encode_matches_torch_rounding():
    # torch's float32 -> float8_e4m3fn cast rounds to nearest even and keeps
    # the sign bit: an independent implementation of the same encoding.
    rng = np.random.default_rng(0)
    grid = _e4m3_grid()
    mids = (grid[:-1] + grid[1:]) / 2                      # every tie
    x = np.concatenate([rng.uniform(-448, 448, 200_000), rng.uniform(-0.02, 0.02, 200_000),
                        rng.standard_normal(100_000) * 8, grid, mids, np.nextafter(mids, 0), np.nextafter(mids, 1e9),
                        [-0.0, 0.0]]).astype(np.float32)
    x = x[np.abs(x) <= 448]
    ours = fp8.e4m3_encode(x.astype(np.float64))
    lib = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(ours, lib)


def test_e4m3_round_trip_and_monotone():
    codes = np.arange(256, dtype=np.uint8)
    v = fp8.e4m3_value(codes)
    ok = np.isfinite(v)
    np.testing.assert_array_equal(fp8.e4m3_encode(v[ok]), codes[ok])
    x = np.linspace(0, 448, 100_001)
    y = fp8.e4m3_value(fp8.e4m3_encode(x))
    assert np.all(np.diff(y) >= 0)
    # Nearest: no grid point is closer than the chosen one.
    grid = _e4m3_grid()
    dist = np.abs(grid[None, :] - x[:2001, None]).min(axis=1)
    np.testing.assert_array_equal(np.abs(y[:2001] - x[:2001]), dist)


def test_e4m3_encode_rejects_out_of_range():
    with pytest.raises(ValueError):
        fp8.e4m3_encode(np.array([449.0]))
    with pytest.raises(ValueError):
        fp8.e4m3_encode(np.array([np.nan]))


# ------------------------------------------------------- quantisation ---

def test_quantize_hand_example(golden_dir):
    g = _golden(golden_dir)
    for r in g["rows"]:
        codes, scale = fp8.quantize_q(np.array(r["x"], dtype=np.float64)[None, None, None, :])
        assert codes.ravel().tolist() == r["codes"], r["name"]
        assert _bits(scale.ravel()[0]) == r["scale_bits"], r["name"]
    kt = g["k_tiles"]
    codes, scale = fp8.quantize_k(np.array(kt["k"], dtype=np.float64)[None, None], kt["tile"])
    assert codes[0, 0].tolist() == kt["codes"]
    assert [_bits(s) for s in scale.ravel()] == kt["scale_bits"]


def _bf16_values(shape, rng, gain=1.0):
    x = torch.from_numpy(rng.standard_normal(shape) * gain).to(torch.bfloat16)
    return x.double().numpy()


def test_quantize_error_bound_and_amax_code():
    rng = np.random.default_rng(1)
    q = _bf16_values((2, 3, 70, 16), rng, 3.0)
    q[0, 0, 5] = 0.0                                         # a zero token
    q[1, 2, 9, :8] *= 1e-4                                   # values far below the group maximum
    codes, scale = fp8.quantize_q(q)
    deq = fp8.dequantize(codes, scale[..., None])
    s = scale.astype(np.float64)[..., None]
    # Half a quantum: 2^-4 relative in the normal range, 2^-10 * scale below
    # it; 2^-21 covers the fp32 roundings of inv and y.
    bound = (2.0 ** -4 + 2.0 ** -21) * np.abs(q) + 2.0 ** -10 * s
    assert np.all(np.abs(deq - q) <= bound)
    # The element holding the group maximum maps to +-448.
    amax_pos = np.abs(q).argmax(axis=-1)
    top = np.take_along_axis(codes, amax_pos[..., None], axis=-1)[..., 0]
    nonzero = np.abs(q).max(axis=-1) > 0
    assert np.all(np.isin(top[nonzero], [0x7E, 0xFE]))
    assert np.all(codes[0, 0, 5] == 0) and scale[0, 0, 5] == 0


def test_quantize_group_scaling_and_locality():
    # Scaling one group by 2 doubles its scale and keeps every code; other
    # groups do not change.  Catches a wrong grouping (per token vs per tile,
    # wrong tile boundaries) of the K quantiser.
    rng = np.random.default_rng(2)
    N, tile = 150, 64                                        # tiles of 64, 64 and 22 tokens
    k = _bf16_values((1, 2, N, 8), rng)
    codes, scale = fp8.quantize_k(k, tile)
    assert scale.shape == (1, 2, 3)
    for t in range(3):
        k2 = k.copy()
        k2[:, 0, t * tile:(t + 1) * tile] *= 2.0
        c2, s2 = fp8.quantize_k(k2, tile)
        np.testing.assert_array_equal(c2, codes)
        np.testing.assert_array_equal(s2[:, 0, t], 2 * scale[:, 0, t])
        others = [u for u in range(3) if u != t]
        np.testing.assert_array_equal(s2[:, 0, others], scale[:, 0, others])
        np.testing.assert_array_equal(s2[:, 1], scale[:, 1])
    # One large value in a tile moves only that tile.
    k3 = k.copy()
    k3[0, 1, 70, 3] = 100.0
    c3, s3 = fp8.quantize_k(k3, tile)
    changed = np.any(c3 != codes, axis=-1)[0, 1]
    assert set(np.nonzero(changed)[0] // tile) == {1}
    assert s3[0, 1, 1] > scale[0, 1, 1] and s3[0, 1, 0] == scale[0, 1, 0] and s3[0, 1, 2] == scale[0, 1, 2]
    # Per token for Q: scaling one token changes only that token's scale.
    qc, qs = fp8.quantize_q(k)
    k4 = k.copy()
    k4[0, 0, 3] *= 4.0
    qc4, qs4 = fp8.quantize_q(k4)
    np.testing.assert_array_equal(qc4, qc)
    assert qs4[0, 0, 3] == 4 * qs[0, 0, 3]
    mask = np.ones(qs.shape, bool)
    mask[0, 0, 3] = False
    np.testing.assert_array_equal(qs4[mask], qs[mask])


def test_dequantisation_is_exact_on_representable_data():
    # Q rows and K tiles built from E4M3 values times a power of two, each
    # group holding +-448 * 2^e: inv and scale are exact powers of two and the
    # dequantised operands equal the inputs (fp8 attention is then exactly
    # the attention of the inputs).
    rng = np.random.default_rng(3)
    grid = _e4m3_grid()
    B, H, N, d = 1, 2, 100, 16
    q = rng.choice(grid, size=(B, H, N, d)) * 2.0 ** -6
    q[..., 0] = 448 * 2.0 ** -6
    k = rng.choice(grid, size=(B, H, N, d)) * 2.0 ** -7
    k[:, :, ::7, 1] = -448 * 2.0 ** -7                      # every 64-token tile holds one
    qk = fp8.quantize_qk(q, k)
    np.testing.assert_array_equal(qk.q_deq, q)
    np.testing.assert_array_equal(qk.k_deq, k)
    assert np.all(np.isin(qk.q_scale, [2.0 ** -6])) and np.all(np.isin(qk.k_scale, [2.0 ** -7]))


def test_quantize_qk_shapes_and_dequantised_values():
    rng = np.random.default_rng(4)
    q = _bf16_values((2, 1, 130, 8), rng)
    k = _bf16_values((2, 1, 130, 8), rng)
    qk = fp8.quantize_qk(q, k)
    assert qk.q_codes.shape == q.shape and qk.q_scale.shape == (2, 1, 130)
    assert qk.k_codes.shape == k.shape and qk.k_scale.shape == (2, 1, 3)
    tiles = np.arange(130) // 64
    np.testing.assert_array_equal(qk.k_deq, fp8.e4m3_value(qk.k_codes) * qk.k_scale[:, :, tiles, None])
    np.testing.assert_array_equal(qk.q_deq, fp8.e4m3_value(qk.q_codes) * qk.q_scale[..., None])
