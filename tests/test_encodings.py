"""Pins of the oracle's storage encoders against torch's own conversions (a library routine)
and against the formats' definitions (no GPU)."""
import numpy as np
import torch

from oracle import (bf16_decode, bf16_encode, e4m3_decode, e4m3_encode, fp16_decode, fp16_encode,
                    quantize_rows_e4m3)


def _e4m3_torch(x32):
    return torch.from_numpy(np.asarray(x32, dtype=np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_e4m3_decode_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ours = e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])
    assert ours[0x7E] == 448.0 and ours[0x01] == 2.0 ** -9 and ours[0x08] == 2.0 ** -6
    assert np.isnan(ours[0x7F]) and np.isnan(ours[0xFF])


def test_e4m3_encode_round_trip_and_ties():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    vals = e4m3_decode(codes).astype(np.float32)
    back = e4m3_encode(vals)
    # +0 and -0 keep their sign; every other finite code round-trips
    assert np.array_equal(back, codes)
    # exact midpoints between neighbours round to the even mantissa
    pos = np.sort(np.unique(e4m3_decode(np.arange(0, 0x7F, dtype=np.uint8))))
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)
    assert np.all(mids.astype(np.float64) == (pos[:-1] + pos[1:]) / 2)   # midpoints exact in f32
    got = e4m3_decode(e4m3_encode(mids))
    lo_code = e4m3_encode(pos[:-1].astype(np.float32))
    hi_code = e4m3_encode(pos[1:].astype(np.float32))
    even = np.where(lo_code % 2 == 0, pos[:-1], pos[1:])
    assert np.array_equal(got, even)
    assert np.array_equal(e4m3_encode(mids), _e4m3_torch(mids))
    del hi_code


def test_e4m3_encode_matches_torch_in_range():
    rng = np.random.default_rng(0)
    x = (rng.standard_normal(400000) * np.exp(rng.uniform(-14, 6.2, 400000))).astype(np.float32)
    x = x[np.abs(x) <= 448.0]
    assert np.array_equal(e4m3_encode(x), _e4m3_torch(x))


def test_e4m3_saturates_and_nan():
    big = np.array([448.0, 449.0, 463.99, 464.0, 500.0, 1e30, -1e30, np.inf, -np.inf], dtype=np.float32)
    c = e4m3_encode(big)
    assert list(c) == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0x7E, 0xFE]
    assert np.all(e4m3_decode(c) == np.sign(big) * 448.0)
    assert e4m3_encode(np.array([np.nan], dtype=np.float32))[0] == 0x7F


def test_quantize_rows_scale_and_error_bound():
    rng = np.random.default_rng(1)
    rows = (rng.standard_normal((64, 576)) * 0.4).astype(np.float32)
    rows[3] = 0.0
    codes, scales = quantize_rows_e4m3(rows)
    assert scales.dtype == np.float32 and scales[3] == 1.0 and np.all(codes[3] == 0)
    amax = np.abs(rows).max(1)
    nz = amax > 0
    assert np.array_equal(scales[nz], (amax[nz] / np.float32(448)).astype(np.float32))
    deq = e4m3_decode(codes) * scales[:, None].astype(np.float64)
    # error at most half a spacing: spacing <= 2^-3 relative for normals, 2^-9 * scale absolute
    err = np.abs(deq - rows)
    bound = np.maximum(np.abs(rows) * 2.0 ** -4, 2.0 ** -10 * scales[:, None]) * (1 + 1e-6)
    assert np.all(err <= bound)
    # the largest element of each row lands on (or next to) the top code 448
    top = np.abs(e4m3_decode(codes)).max(1)
    assert np.all(top[nz] == 448.0)


def test_bf16_matches_torch():
    rng = np.random.default_rng(2)
    u = rng.integers(0, 2 ** 32, 300000, dtype=np.uint64).astype(np.uint32)
    x = u.view(np.float32)
    x = x[np.isfinite(x)]
    # add exact ties (low 16 bits = 0x8000) for both parities
    ties = (rng.integers(0, 2 ** 16, 5000, dtype=np.uint32) << 16 | 0x8000).view(np.float32)
    x = np.concatenate([x, ties[np.isfinite(ties)]])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bf16_encode(x), ref)
    assert np.array_equal(bf16_decode(ref), torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16).double().numpy())


def test_fp16_matches_torch():
    rng = np.random.default_rng(3)
    x = (rng.standard_normal(200000) * np.exp(rng.uniform(-20, 11, 200000))).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(fp16_encode(x), ref)
    assert np.array_equal(fp16_decode(ref), torch.from_numpy(ref.view(np.int16)).view(torch.float16).double().numpy())


# ---------------------------------------------------------------- fp6 e2m3 (no torch type: the
# format's definition and brute force are the references)
def _e2m3_table():
    """Every code's value written out from the definition: sign, exponent e (bias 1), mantissa m:
    e = 0 -> m/8 (subnormal), else (1 + m/8) * 2^(e-1)."""
    vals = {}
    for c in range(64):
        s, e, m = c >> 5, (c >> 3) & 3, c & 7
        mag = m / 8.0 if e == 0 else (1.0 + m / 8.0) * 2.0 ** (e - 1)
        vals[c] = -mag if s else mag
    return vals


def test_e2m3_decode_all_codes():
    from oracle import e2m3_decode
    tab = _e2m3_table()
    codes = np.arange(64, dtype=np.uint8)
    assert np.array_equal(e2m3_decode(codes), np.array([tab[c] for c in range(64)]))
    mags = sorted({abs(v) for v in tab.values()})
    assert len(mags) == 32 and mags[1] == 0.125 and mags[8] == 1.0 and mags[-1] == 7.5
    assert np.signbit(e2m3_decode(np.array([0x20], dtype=np.uint8)))[0]    # -0 keeps its sign
    # codes are monotonic in magnitude: neighbouring codes are neighbouring values
    assert np.all(np.diff(e2m3_decode(np.arange(32, dtype=np.uint8))) > 0)


def test_e2m3_encode_round_trip():
    from oracle import e2m3_decode, e2m3_encode
    codes = np.arange(64, dtype=np.uint8)
    assert np.array_equal(e2m3_encode(e2m3_decode(codes).astype(np.float32)), codes)


def _e2m3_brute(x):
    """Nearest e2m3 value by exhaustive search over the 32 magnitudes, ties to the even code,
    saturating at 7.5 (the reference the arithmetic encoder is pinned to)."""
    mags = np.array([abs(v) for c, v in sorted(_e2m3_table().items()) if c < 32])
    out = np.empty(len(x), dtype=np.uint8)
    for i, v in enumerate(np.asarray(x, dtype=np.float64)):
        a = min(abs(v), 7.5)
        d = np.abs(mags - a)
        best = np.flatnonzero(d == d.min())
        c = int(best[0]) if len(best) == 1 else int(best[best % 2 == 0][0])
        out[i] = c | (0x20 if np.signbit(v) else 0)
    return out


def test_e2m3_encode_matches_brute_force():
    from oracle import e2m3_encode
    rng = np.random.default_rng(11)
    x = np.concatenate([
        (rng.standard_normal(60000) * np.exp(rng.uniform(-6, 2.5, 60000))).astype(np.float32),
        rng.uniform(-9, 9, 20000).astype(np.float32),
    ])
    assert np.array_equal(e2m3_encode(x), _e2m3_brute(x))


def test_e2m3_ties_and_saturation():
    from oracle import e2m3_decode, e2m3_encode
    pos = e2m3_decode(np.arange(32, dtype=np.uint8))
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)
    assert np.all(mids.astype(np.float64) == (pos[:-1] + pos[1:]) / 2)     # exact in float32
    got = e2m3_encode(mids).astype(np.int64)
    lo = np.arange(31)
    assert np.array_equal(got, np.where(lo % 2 == 0, lo, lo + 1))           # the even neighbour
    big = np.array([7.5, 7.74, 7.75, 8.0, 1e30, -7.76, -1e30, np.inf, -np.inf], dtype=np.float32)
    assert list(e2m3_encode(big)) == [0x1F, 0x1F, 0x1F, 0x1F, 0x1F, 0x3F, 0x3F, 0x1F, 0x3F]
    assert e2m3_encode(np.array([np.nan], dtype=np.float32))[0] == 0


def test_e2m3_packing_bit_positions():
    from oracle import pack_e2m3, unpack_e2m3
    # code j sits at bits 6j .. 6j + 5 of a little-endian stream
    for j in range(8):
        c = np.zeros(8, dtype=np.uint8)
        c[j] = 0x3F
        p = pack_e2m3(c).astype(np.int64)
        stream = sum(int(b) << (8 * i) for i, b in enumerate(p))
        assert stream == 0x3F << (6 * j), j
    rng = np.random.default_rng(12)
    codes = rng.integers(0, 64, (7, 576), dtype=np.uint8)
    p = pack_e2m3(codes)
    assert p.shape == (7, 432)
    assert np.array_equal(unpack_e2m3(p, 576), codes)


def test_quantize_rows_e2m3_scale_and_error_bound():
    from oracle import e2m3_decode, quantize_rows_e2m3
    rng = np.random.default_rng(13)
    rows = (rng.standard_normal((64, 576)) * 0.4).astype(np.float32)
    rows[5] = 0.0
    codes, scales = quantize_rows_e2m3(rows)
    assert scales[5] == 1.0 and np.all(codes[5] == 0)
    amax = np.abs(rows).max(1)
    nz = amax > 0
    assert np.array_equal(scales[nz], (amax[nz] / np.float32(7.5)).astype(np.float32))
    deq = e2m3_decode(codes) * scales[:, None].astype(np.float64)
    # at most half a spacing: 2^-4 relative for normals, 2^-4 * scale absolute below 1 * scale
    bound = np.maximum(np.abs(rows) * 2.0 ** -4, 2.0 ** -4 * scales[:, None]) * (1 + 1e-6)
    assert np.all(np.abs(deq - rows) <= bound)
    assert np.all(np.abs(e2m3_decode(codes)).max(1)[nz] == 7.5)
