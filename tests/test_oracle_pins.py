"""Pins of the CPU oracle against what the pages and mathematics fix.

Nothing here compares the oracle with itself: each check uses an independent
formulation (closed-form threshold tables, numpy/torch library rounding,
exact rational arithmetic, brute force on tiny inputs) or a number printed on
the pages (tests/golden/*.json, each with its citation).
"""
import json
import os
from fractions import Fraction as F

import numpy as np
import pytest
import torch

import oracle
from oracle import exact

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def bf16_bits(values):
    t = torch.tensor(values, dtype=torch.float32).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def bits_to_f32(b):
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# ------------------------------------------------------------------ E2M1 grid
def test_e2m1_value_set_matches_pages():
    gd = gold("e2m1_grid.json")
    vals = [oracle.e2m1_value(c) for c in range(16)]
    mags = sorted({abs(v) for v in vals})
    assert mags == gd["magnitudes"]
    assert sorted(v for v in vals if v > 0) == [m for m in gd["magnitudes"] if m > 0]
    assert sorted(-v for v in vals if v < 0) == [m for m in gd["magnitudes"] if m > 0]
    # 16 codes, +0 and -0 coincide as values: 15 distinct values
    assert len(set(vals)) == gd["distinct_values"]
    assert max(abs(v) for v in vals) == gd["max_magnitude"]
    # S1E2M1 layout: sign is bit 3; code 8 is -0
    assert np.signbit(oracle.e2m1_value(8)) and oracle.e2m1_value(8) == 0.0
    for c in range(8):
        e, m = c >> 1, c & 1
        expect = m * 0.5 if e == 0 else (1 + m / 2) * 2.0 ** (e - 1)   # bias 1, 1 mantissa bit
        assert oracle.e2m1_value(c) == expect


def _e2m1_by_thresholds(y: np.ndarray) -> np.ndarray:
    """RNE onto {0,.5,1,1.5,2,3,4,6} written as a threshold table: a midpoint
    between two grid values goes to the neighbour whose code is even."""
    k = np.zeros(y.shape, dtype=np.int8)
    k += y > 0.25      # 0.25: midpoint of 0 (code 0) and 0.5 (code 1) -> 0
    k += y >= 0.75     # 0.75: 0.5 (1) | 1 (2) -> 2
    k += y > 1.25      # 1.25: 1 (2) | 1.5 (3) -> 2
    k += y >= 1.75     # 1.75: 1.5 (3) | 2 (4) -> 4
    k += y > 2.5       # 2.5: 2 (4) | 3 (5) -> 4
    k += y >= 3.5      # 3.5: 3 (5) | 4 (6) -> 6
    k += y > 5.0       # 5: 4 (6) | 6 (7) -> 6; above 6 saturates at 7
    return k


def test_e2m1_encode_exhaustive_up_to_8():
    """Every non-negative float32 in [0, 8], then a sample of larger ones."""
    hi = np.uint32(0x41000000)  # 8.0
    step = 1 << 24
    for start in range(0, int(hi) + 1, step):
        bits = np.arange(start, min(start + step, int(hi) + 1), dtype=np.uint32)
        y = bits.view(np.float32)
        got = oracle.e2m1_encode_array(y)
        want = _e2m1_by_thresholds(y)
        bad = np.nonzero(got != want)[0]
        assert bad.size == 0, f"first mismatch at y={y[bad[0]]!r}: {got[bad[0]]} vs {want[bad[0]]}"
    rng = np.random.default_rng(1)
    big = rng.integers(0x41000001, 0x7F800000, size=1 << 20, dtype=np.uint32).view(np.float32)
    assert np.all(oracle.e2m1_encode_array(big) == 7)


# ------------------------------------------------------------------ E4M3
def _e4m3_closed_form(v: np.ndarray) -> np.ndarray:
    """OCP E4M3FN (bias 7, max 448), RNE via np.rint on exactly scaled values."""
    v = v.astype(np.float64)
    out = np.zeros(v.shape, dtype=np.int16)
    sub = v < 2.0 ** -6
    out[sub] = np.rint(v[sub] * 512.0).astype(np.int16)       # m * 2^-9, m = 0..8 (8 == 2^-6 == 0x08)
    nrm = ~sub
    fr, e = np.frexp(v[nrm])                                  # v = fr * 2^e, fr in [0.5, 1)
    m = np.rint(fr * 16.0).astype(np.int64)                   # 8..16
    e = e.astype(np.int64) - 1 + (m == 16)
    m = np.where(m == 16, 8, m)
    code = ((e + 7) << 3) | (m - 8)
    out[nrm] = np.minimum(code, 0x7E).astype(np.int16)        # saturate at 448
    return out


def test_e4m3_value_table():
    vals = [oracle.e4m3_value(b) for b in range(0x7F)]
    assert vals[0x7E] == 448.0 and vals[1] == 2.0 ** -9 and vals[8] == 2.0 ** -6
    assert all(a < b for a, b in zip(vals, vals[1:]))          # strictly increasing, no NaN used


def test_e4m3_encode_dense():
    rng = np.random.default_rng(2)
    # strided sweep over all floats in [0, 1024] plus dense windows around every
    # grid value and every midpoint between neighbours
    sweep = np.arange(0, 0x44800000, 97, dtype=np.uint32).view(np.float32)
    grid = np.array([oracle.e4m3_value(b) for b in range(0x7F)], dtype=np.float64)
    mids = (grid[:-1] + grid[1:]) / 2
    pts = np.concatenate([grid, mids, [448.0, 464.0, 480.0, 2.0 ** -10]]).astype(np.float32)
    win = (pts.view(np.uint32)[:, None].astype(np.int64) + np.arange(-300, 301)[None, :]).clip(0, 0x7F7FFFFF)
    dense = win.astype(np.uint32).ravel().view(np.float32)
    rnd = rng.uniform(0, 600, size=1 << 20).astype(np.float32)
    for v in (sweep, dense, rnd):
        got = oracle.e4m3_encode_array(v)
        want = _e4m3_closed_form(v)
        bad = np.nonzero(got != want)[0]
        assert bad.size == 0, f"v={v[bad[0]]!r}: {got[bad[0]]:#x} vs {want[bad[0]]:#x}"


def test_e4m3_documented_examples():
    assert oracle.e4m3_encode(1.0625) == 0x38      # tie 1 | 1.125 -> even mantissa 1.0
    assert oracle.e4m3_encode(1.1875) == 0x3A      # tie 1.125 | 1.25 -> 1.25
    assert oracle.e4m3_encode(464.0) == 0x7E       # saturates at 448
    assert oracle.e4m3_encode(2.0 ** -10) == 0     # tie 0 | 2^-9 -> 0
    assert oracle.e4m3_encode(1.5 * 2.0 ** -10) == 1


# ------------------------------------------------------------------ bf16 RNE
def test_f32_to_bf16_matches_torch():
    hi = np.arange(0, 0x10000, 131, dtype=np.uint32)
    hi = hi[(hi & 0x7F80) != 0x7F80]
    hi = np.unique(np.concatenate([hi, [0x3F80, 0x0000, 0x8000, 0x0001, 0x7F7F, 0xFF7F & 0xFFFF]]))
    bits = (hi[:, None] << 16 | np.arange(0x10000, dtype=np.uint32)[None, :]).ravel()
    f = bits.view(np.float32)
    got = oracle.f32_to_bf16_array(f)
    want = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, f"f={f[bad[0]]!r}: {got[bad[0]]:#x} vs {want[bad[0]]:#x}"


# ------------------------------------------------------------------ storage
def test_storage_is_0p5625_bytes_per_value():
    gs = gold("storage.json")
    x = bf16_bits(np.random.default_rng(3).standard_normal((8, 64)))
    q, sf, g = oracle.quantize(x)
    n = x.size
    assert q.nbytes + sf.nbytes == gs["bytes_per_value"] * n
    assert 8 * (q.nbytes + sf.nbytes) / n == gs["bits_per_value"]
    assert 16 / gs["bits_per_value"] == pytest.approx(gs["ratio_vs_fp16_about"], abs=0.1)
    assert 8 / gs["bits_per_value"] == pytest.approx(gs["ratio_vs_fp8_about"], abs=0.05)
    assert g.nbytes == 4          # one FP32 scale per tensor


def test_kv_size_worked_example():
    gk = gold("kv_size_example.json")
    L, H, D, T = gk["layers"], gk["kv_heads"], gk["head_dim"], gk["context_tokens"]
    assert 2 * L * H * D == gk["values_per_token"]
    # encode one token of K and one of V through the oracle and count bytes
    rng = np.random.default_rng(4)
    k = bf16_bits(rng.standard_normal((L, 1, H, D)))
    v = bf16_bits(rng.standard_normal((L, 1, H, D)))
    gl = np.full((L, H), 0.01, dtype=np.float32)
    kq, ksf = oracle.kv_encode(k, gl)
    vq, vsf = oracle.kv_encode(v, gl)
    per_token = kq.nbytes + ksf.nbytes + vq.nbytes + vsf.nbytes
    assert per_token == gk["rows"]["nvfp4"]["per_token_KiB"] * 1024
    assert per_token * T == gk["rows"]["nvfp4"]["per_context_GiB"] * 2 ** 30
    for fmt in ("bf16", "fp8"):
        row = gk["rows"][fmt]
        assert gk["values_per_token"] * row["bytes_per_value"] == row["per_token_KiB"] * 1024
        assert gk["values_per_token"] * row["bytes_per_value"] * T == row["per_context_GiB"] * 2 ** 30


# ------------------------------------------------------------------ crafted tensors
def _tensor_with_g1(blocks):
    """Row of 16-value blocks; the last block holds 2688 so amax = 6*448 -> g = 1."""
    row = [v for b in blocks for v in b] + [2688.0] + [0.0] * 15
    return bf16_bits([row])


@pytest.mark.parametrize("j", [-9, -3, 0, 2, 6])
def test_e2m1_ties_go_to_even_code(j):
    grid = gold("e2m1_grid.json")["magnitudes"]
    mids = [(a + b) / 2 for a, b in zip(grid, grid[1:])]          # 0.25 .. 5
    blk = [6.0 * 2 ** j] + [m * 2 ** j for m in mids] + [-m * 2 ** j for m in mids] + [-0.0]
    assert len(blk) == 16
    x = _tensor_with_g1([blk])
    q, sf, g = oracle.quantize(x)
    assert g[0] == 1.0
    assert sf[0, 0] == oracle.e4m3_encode(2.0 ** j) and oracle.e4m3_value(sf[0, 0]) == 2.0 ** j
    codes = np.stack([q[0] & 15, q[0] >> 4], axis=1).ravel()[:16]
    even = [k if k % 2 == 0 else k + 1 for k in range(7)]        # midpoint k|k+1 -> even code
    assert codes[0] == 7
    assert list(codes[1:8]) == even
    assert list(codes[8:15]) == [8 | c for c in even]
    assert codes[15] == 8                                        # -0 keeps its sign
    assert sf[0, 1] == 0x7E                                      # amax block: s = 448


def test_e4m3_tie_in_block_scale():
    x = _tensor_with_g1([[6.375] + [0.0] * 15])                  # 6.375 / 6 = 1.0625: tie -> 1.0
    q, sf, g = oracle.quantize(x)
    assert g[0] == 1.0 and sf[0, 0] == 0x38
    assert (q[0, 0] & 15) == 7                                   # 6.375 / 1 saturates to 6


def test_nibble_order_low_first():
    x = _tensor_with_g1([[6.0, 0.5, 1.0, -1.5] + [0.0] * 12])
    q, sf, g = oracle.quantize(x)
    assert sf[0, 0] == 0x38                                      # s = 1
    assert q[0, 0] == (7 | (1 << 4)) and q[0, 1] == (2 | (11 << 4))


def test_all_zero_and_signed_zero():
    x = bf16_bits([[0.0, -0.0] * 16])
    q, sf, g = oracle.quantize(x)
    assert g[0] == 0.0 and np.all(sf == 0)
    assert np.all(q == 0x80)
    y = oracle.dequantize(q, sf, g)
    assert np.all(y == np.array([0x0000, 0x8000] * 16, dtype=np.uint16))


def test_global_amax_element():
    rng = np.random.default_rng(5)
    for scale in (1e-3, 1.0, 37.0, 3e4):
        x = bf16_bits(rng.standard_normal((16, 64)) * scale)
        q, sf, g = oracle.quantize(x)
        xf = bits_to_f32(x)
        amax = np.abs(xf).max()
        r, c = np.unravel_index(np.abs(xf).argmax(), xf.shape)
        assert sf[r, c // 16] == 0x7E
        code = (q[r, c // 2] >> (4 * (c % 2))) & 15
        assert code & 7 == 7
        back = oracle.f32_to_bf16_array(np.array([np.float32(2688.0) * g[0]], dtype=np.float32))
        assert bits_to_f32(back)[0] == amax


def test_block_amax_keeps_fp8_precision():
    """The block max is carried by an E4M3 scale: in every normal-scale block the
    largest element gets the top E2M1 code and 6*s*g is within 2^-4 of bamax
    (axbrief.com, 'E2M1 format and two-level scaling': the block amax is kept at
    FP8 precision; one of the 16 values)."""
    rng = np.random.default_rng(6)
    checked = 0
    for dist in ("normal", "t3", "outlier"):
        z = rng.standard_normal((64, 256))
        if dist == "t3":
            z = z / np.sqrt(rng.chisquare(3, z.shape) / 3)
        if dist == "outlier":
            z = z * 0.02 * np.where(rng.random(z.shape) < 0.01, 50, 1)
        x = bf16_bits(z)
        q, sf, g = oracle.quantize(x)
        xf = np.abs(bits_to_f32(x)).reshape(64, -1, 16)
        codes = np.stack([q & 15, q >> 4], axis=-1).reshape(64, -1, 16) & 7
        for r in range(64):
            for b in range(xf.shape[1]):
                if sf[r, b] >= 0x08:                       # normal E4M3 scale
                    assert codes[r, b].max() == 7
                    deq_max = 6 * oracle.e4m3_value(sf[r, b]) * float(g[0])
                    assert abs(deq_max - xf[r, b].max()) <= 2 ** -4 * xf[r, b].max() * 1.0001
                    checked += 1
    assert checked > 3000


def test_idempotence_on_normal_scale_blocks():
    rng = np.random.default_rng(7)
    for scale in (1e-30, 1e-4, 1.0, 1e3, 1e30):
        x = bf16_bits(rng.standard_normal((32, 128)) * scale)
        q, sf, g = oracle.quantize(x)
        y = oracle.dequantize(q, sf, g)
        q2, sf2, g2 = oracle.quantize(y)
        assert g2[0] == g[0]
        ok = sf >= 0x08
        assert ok.mean() > 0.99
        assert np.array_equal(sf2[ok], sf[ok])
        qb = np.repeat(ok, 8, axis=1)
        assert np.array_equal(q2[qb], q[qb])


def test_subnormal_scale_exception_is_real():
    """Known exception to idempotence: a block whose E4M3 scale is subnormal and
    whose largest code is below 6 re-quantizes to a different scale."""
    bamax = 6 * 1.6 * 2.0 ** -9
    x = _tensor_with_g1([[bamax] + [0.0] * 15])
    q, sf, g = oracle.quantize(x)
    # bamax/6 = 1.6*2^-9 rounds on the subnormal E4M3 grid to 2*2^-9 (byte 2);
    # the element then sits at 6*1.6/2 = 4.8 -> code 6 (value 4), not the top code
    assert sf[0, 0] == 2 and (q[0, 0] & 7) == 6
    y = oracle.dequantize(q, sf, g)
    q2, sf2, _ = oracle.quantize(y)
    assert sf2[0, 0] != sf[0, 0]


# ------------------------------------------------------------------ exact rationals
def _rand_tensor(rng, rows, cols):
    mode = rng.integers(0, 5)
    if mode == 0:
        z = rng.standard_normal((rows, cols))
    elif mode == 1:
        z = rng.standard_normal((rows, cols)) * 10.0 ** rng.uniform(-40, 38)
    elif mode == 2:
        z = rng.standard_normal((rows, cols)) * np.where(rng.random((rows, cols)) < 0.1, 1e4, 1)
    elif mode == 3:                                          # bf16 subnormals mixed in
        z = rng.standard_normal((rows, cols)) * 2.0 ** -128
    else:                                                    # wide dynamic range per block
        z = rng.standard_normal((rows, cols)) * 2.0 ** rng.integers(-20, 20, (rows, cols))
    return bf16_bits(np.clip(z, -3e38, 3e38))


def test_quantize_matches_exact_rationals():
    rng = np.random.default_rng(8)
    for trial in range(40):
        x = _rand_tensor(rng, 3, 32)
        q, sf, g = oracle.quantize(x)
        codes, scales, ge = exact.quantize_rows(x.tolist())
        assert F(float(g[0])) == ge
        assert sf.tolist() == scales
        qc = np.stack([q & 15, q >> 4], axis=-1).reshape(3, 32)
        assert qc.tolist() == codes, f"trial {trial}"


def test_quantize_with_scale_matches_exact_rationals():
    rng = np.random.default_rng(9)
    for trial in range(30):
        x = _rand_tensor(rng, 2, 32)
        gval = np.float32(abs(rng.standard_normal()) * 10.0 ** rng.uniform(-8, 3))
        q, sf = oracle.quantize_with_scale(x[None], np.array([gval]))
        codes, scales, _ = exact.quantize_rows(x.tolist(), g=F(float(gval)))
        assert sf[0].tolist() == scales
        assert np.stack([q[0] & 15, q[0] >> 4], -1).reshape(2, 32).tolist() == codes


def _division_sensitive_cases(rng, n=2000):
    """(x, d) pairs where RN32(x/d) and RN32(x * RN32(1/d)) land in different E2M1
    cells -- an oracle that used a reciprocal instead of a division would fail."""
    out = []
    while len(out) < 8:
        d = rng.uniform(0.5, 1.0, n).astype(np.float32)
        for b in (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0):
            x = (np.float32(b) * d).astype(np.float32)
            xb = bf16_bits(x)
            xf = bits_to_f32(xb)
            y_div = (xf / d).astype(np.float32)
            y_rcp = (xf * (np.float32(1) / d).astype(np.float32)).astype(np.float32)
            diff = _e2m1_by_thresholds(y_div) != _e2m1_by_thresholds(y_rcp)
            for i in np.nonzero(diff)[0][:2]:
                out.append((xb[i], float(d[i])))
    return out


def test_element_division_sensitive_cases():
    rng = np.random.default_rng(10)
    cases = _division_sensitive_cases(rng)
    checked = 0
    for xb, d in cases:
        # quantize_with_scale with g = d and a block scale of exactly 1 (bamax = 6 d)
        sixd = bf16_bits([6.0 * d])[0]
        row = np.array([[sixd] + [xb] + [0] * 14], dtype=np.uint16)
        gval = np.float32(d)
        if oracle.block_scale(bits_to_f32([sixd])[0], gval) != 0x38:
            continue
        q, sf = oracle.quantize_with_scale(row[None], np.array([gval]))
        codes, scales, _ = exact.quantize_rows(row.tolist(), g=F(float(gval)))
        assert (q[0, 0, 0] >> 4) == codes[0][1]
        checked += 1
    assert checked >= 4


def test_dequant_matches_fp64_product_and_exact():
    rng = np.random.default_rng(11)
    codes = rng.integers(0, 16, size=4096)
    sbytes = rng.integers(0, 0x7F, size=4096)
    gs = (np.abs(rng.standard_normal(4096)) * 10.0 ** rng.uniform(-30, 30, 4096)).astype(np.float32)
    lut = np.array([oracle.e2m1_value(c) for c in range(16)])
    sv = np.array([oracle.e4m3_value(b) for b in range(0x7F)])
    exact64 = lut[codes] * sv[sbytes] * gs.astype(np.float64)       # exact: <= 30 significant bits
    f32 = exact64.astype(np.float32)                                # one RNE rounding
    for i in range(4096):
        got = oracle.decode_element(int(codes[i]), int(sbytes[i]), float(gs[i]))
        assert np.float32(got) == f32[i] or (got == 0 and f32[i] == 0)
        if i < 300:
            assert F(got) == exact.dequant_value(int(codes[i]), int(sbytes[i]), F(float(gs[i])))
    # full tensor path: bf16 output equals torch's RNE of the same fp32 values
    x = bf16_bits(rng.standard_normal((64, 128)) * 3)
    q, sf, g = oracle.quantize(x)
    y = oracle.dequantize(q, sf, g)
    d64 = oracle.dequantize_f64_unscaled(q, sf) * float(g[0])
    want = torch.from_numpy(d64.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(y, want)


# ------------------------------------------------------------------ contractions
def _exact_deq(q, sf, r, k):
    code = (int(q[r, k // 2]) >> (4 * (k % 2))) & 15
    return exact.E2M1[code & 7] * (-1 if code & 8 else 1) * exact.E4M3[int(sf[r, k // 16])]


def test_gemm_f64_against_exact_triple_loop():
    rng = np.random.default_rng(12)
    M, N, K = 3, 4, 48
    a = bf16_bits(rng.standard_normal((M, K)))
    b = bf16_bits(rng.standard_normal((N, K)) * 5)
    aq, asf, ag = oracle.quantize(a)
    bq, bsf, bg = oracle.quantize(b)
    C = oracle.gemm_f64(aq, asf, ag[0], bq, bsf, bg[0])
    for m in range(M):
        for n in range(N):
            s = sum(_exact_deq(aq, asf, m, k) * _exact_deq(bq, bsf, n, k) for k in range(K))
            want = F(float(ag[0])) * F(float(bg[0])) * s
            assert abs(F(C[m, n]) - want) <= abs(want) * F(1, 2 ** 48) + F(1, 2 ** 1000)
    # not symmetric in its operands: swapping A and B transposes C
    Ct = oracle.gemm_f64(bq, bsf, bg[0], aq, asf, ag[0])
    assert np.allclose(Ct, C.T, rtol=1e-15)


def test_grouped_gemm_f64_against_exact_sums():
    """Each routed row uses its own expert's weight and scale; an empty expert
    and rows of different experts are checked with exact rational sums."""
    rng = np.random.default_rng(21)
    E, N, K = 3, 2, 32
    offsets = np.array([0, 2, 2, 5], dtype=np.int32)      # expert 1 receives no rows
    a = bf16_bits(rng.standard_normal((5, K)))
    aq, asf, ag = oracle.quantize(a)
    w = [bf16_bits(rng.standard_normal((N, K)) * (e + 1) * 3) for e in range(E)]
    enc = [oracle.quantize(x) for x in w]
    bq = np.stack([t[0] for t in enc])
    bsf = np.stack([t[1] for t in enc])
    bg = np.array([t[2][0] for t in enc], dtype=np.float32)
    C = oracle.grouped_gemm_f64(aq, asf, ag[0], bq, bsf, bg, offsets)
    expert_of_row = [0, 0, 2, 2, 2]
    for m in range(5):
        e = expert_of_row[m]
        for n in range(N):
            s = sum(_exact_deq(aq, asf, m, k) * _exact_deq(bq[e], bsf[e], n, k) for k in range(K))
            want = F(float(ag[0])) * F(float(bg[e])) * s
            assert abs(F(C[m, n]) - want) <= abs(want) * F(1, 2 ** 48) + F(1, 2 ** 1000)
    # routing a row to another expert changes its output (the expert index is used)
    C2 = oracle.grouped_gemm_f64(aq, asf, ag[0], bq, bsf, bg, np.array([0, 3, 3, 5], np.int32))
    assert not np.allclose(C2[2], C[2])


def test_decode_attention_closed_forms():
    """n = 1 gives the token's V exactly; q = 0 gives uniform weights (the mean
    of the V rows); permuting tokens (K and V together) changes nothing; a
    token whose logit dominates by far takes all the weight."""
    rng = np.random.default_rng(31)
    L, H, Hq, n, D = 2, 2, 4, 6, 32
    k = bf16_bits(rng.standard_normal((L, n, H, D)))
    v = bf16_bits(rng.standard_normal((L, n, H, D)))
    kg = np.full((L, H), 0.002, np.float32)
    vg = np.full((L, H), 0.0015, np.float32)
    kq, ksf = oracle.kv_encode(k, kg)
    vq, vsf = oracle.kv_encode(v, vg)
    qv = bf16_bits(rng.standard_normal((L, Hq, D)))
    vhat = np.stack([[oracle.dequantize_f64_unscaled(vq[l, h], vsf[l, h]) * float(vg[l, h])
                      for h in range(H)] for l in range(L)])                  # [L][H][n][D]
    one = oracle.decode_attention_f64(qv, kq[:, :, :1], ksf[:, :, :1], kg, vq[:, :, :1], vsf[:, :, :1], vg, 0.3)
    for hq in range(Hq):
        assert np.array_equal(one[:, hq], vhat[:, hq // 2, 0])
    zero = oracle.decode_attention_f64(np.zeros_like(qv), kq, ksf, kg, vq, vsf, vg, 0.3)
    for hq in range(Hq):
        assert np.allclose(zero[:, hq], vhat[:, hq // 2].mean(axis=1), rtol=1e-14, atol=1e-15)
    perm = rng.permutation(n)
    a = oracle.decode_attention_f64(qv, kq, ksf, kg, vq, vsf, vg, 0.3)
    b = oracle.decode_attention_f64(qv, kq[:, :, perm], ksf[:, :, perm], kg, vq[:, :, perm], vsf[:, :, perm], vg, 0.3)
    assert np.allclose(a, b, rtol=1e-13, atol=1e-15)
    big = oracle.decode_attention_f64(qv, kq, ksf, kg, vq, vsf, vg, 1e6)   # the arg-max token wins
    logits = oracle.decode_qk_f64(qv, kq, ksf, kg)
    for l in range(L):
        for hq in range(Hq):
            t = int(np.argmax(logits[l, hq]))
            assert np.allclose(big[l, hq], vhat[l, hq // 2, t], rtol=1e-12, atol=1e-15)


def test_decode_qk_against_exact_sums():
    rng = np.random.default_rng(13)
    L, H, Hq, n, D = 2, 2, 8, 3, 32
    k = bf16_bits(rng.standard_normal((L, n, H, D)))
    qv = bf16_bits(rng.standard_normal((L, Hq, D)))
    kg = np.array([[0.002, 0.0017], [0.0021, 0.001]], dtype=np.float32)
    kq, ksf = oracle.kv_encode(k, kg)
    logits = oracle.decode_qk_f64(qv, kq, ksf, kg)
    for l in range(L):
        for hq in range(Hq):
            h = hq // (Hq // H)                                   # GQA: Hq/H query heads per KV head
            for t in range(n):
                s = F(0)
                for d in range(D):
                    s += exact.bf16_to_fraction(int(qv[l, hq, d])) * _exact_deq(kq[l, h], ksf[l, h], t, d)
                want = s * F(float(kg[l, h]))
                assert abs(F(logits[l, hq, t]) - want) <= abs(want) * F(1, 2 ** 45) + F(1, 2 ** 1000)


def test_decode_qk_single_block_closed_form():
    """head_dim 16: one block, logit = g * s * sum_d E2M1(code_d) * q_d."""
    rng = np.random.default_rng(14)
    k = bf16_bits(rng.standard_normal((1, 5, 1, 16)))
    qv = bf16_bits(rng.standard_normal((1, 4, 16)))
    kg = np.array([[0.0013]], dtype=np.float32)
    kq, ksf = oracle.kv_encode(k, kg)
    logits = oracle.decode_qk_f64(qv, kq, ksf, kg)
    qf = bits_to_f32(qv).astype(np.float64)
    for hq in range(4):
        for t in range(5):
            codes = [(int(kq[0, 0, t, j // 2]) >> (4 * (j % 2))) & 15 for j in range(16)]
            dot = sum(oracle.e2m1_value(c) * qf[0, hq, j] for j, c in enumerate(codes))
            want = float(kg[0, 0]) * oracle.e4m3_value(int(ksf[0, 0, t, 0])) * dot
            assert logits[0, hq, t] == pytest.approx(want, rel=1e-14, abs=1e-300)


def test_kv_encode_places_each_token_row():
    rng = np.random.default_rng(15)
    L, n, H, D = 3, 5, 2, 32
    k = bf16_bits(rng.standard_normal((L, n, H, D)) * rng.uniform(0.1, 10, (L, n, H, 1)))
    kg = (np.abs(rng.standard_normal((L, H))) * 0.01 + 1e-3).astype(np.float32)
    kq, ksf = oracle.kv_encode(k, kg)
    for l in range(L):
        for h in range(H):
            for t in range(n):
                q1, s1 = oracle.quantize_with_scale(k[l, t, h][None, None], kg[l, h:h + 1])
                assert np.array_equal(kq[l, h, t], q1[0, 0]) and np.array_equal(ksf[l, h, t], s1[0, 0])
    back = oracle.kv_read(kq, ksf, kg)
    assert back.shape == (L, H, n, D)
    for l in range(L):
        for h in range(H):
            want = oracle.dequantize(kq[l, h][None], ksf[l, h][None], kg[l, h:h + 1])[0]
            assert np.array_equal(back[l, h], want)


def test_nonfinite_input_is_rejected():
    x = bf16_bits([[1.0] * 15 + [float("inf")]])
    with pytest.raises(ValueError):
        oracle.quantize(x)


def test_caller_scale_overflow_saturates():
    """With a caller-supplied tensor scale the quotients can overflow binary32:
    +inf saturates at the format maxima (448 for E4M3, 6 for E2M1); an infinite
    d6 or d gives zero scales / signed-zero codes."""
    x = bf16_bits([[3e38, -1.0] + [0.0] * 14])
    q, sf = oracle.quantize_with_scale(x[None], np.array([1e-38], dtype=np.float32))
    assert sf[0, 0, 0] == 0x7E
    assert (q[0, 0, 0] & 15) == 7 and (q[0, 0, 0] >> 4) == 15
    codes, scales, _ = exact.quantize_rows(x.tolist(), g=F(float(np.float32(1e-38))))
    assert scales[0] == [0x7E] and codes[0][:2] == [7, 15]
    q, sf = oracle.quantize_with_scale(x[None], np.array([3e38], dtype=np.float32))
    assert sf[0, 0, 0] == 0 and q[0, 0, 0] == 0x80
    codes, scales, _ = exact.quantize_rows(x.tolist(), g=F(float(np.float32(3e38))))
    assert scales[0] == [0] and codes[0][:2] == [0, 8]


def test_thread_count_does_not_change_results():
    x = bf16_bits(np.random.default_rng(16).standard_normal((3, 64, 256)))
    a = oracle.quantize(x, nthreads=1)
    b = oracle.quantize(x, nthreads=0)
    for u, v in zip(a, b):
        assert np.array_equal(u, v)


# ------------------------------------------------------------------ MXFP4
def _mx_rand(rng, rows, cols):
    kind = rng.integers(0, 3)
    if kind == 0:
        z = rng.standard_normal((rows, cols))
    elif kind == 1:                                          # per-block magnitudes over a wide range
        z = rng.standard_normal((rows, cols)) * 2.0 ** rng.integers(-60, 60, (rows, cols // 32)).repeat(32, axis=1)
    else:                                                    # tiny blocks: the clamped exponent
        z = rng.standard_normal((rows, cols)) * 2.0 ** -128
    return bf16_bits(np.clip(z, -3e38, 3e38))


def test_mx_storage_is_4p25_bits_per_value():
    gs = gold("storage.json")
    x = bf16_bits(np.random.default_rng(31).standard_normal((8, 128)))
    q, sf = oracle.mx_quantize(x)
    assert 8 * (q.nbytes + sf.nbytes) / x.size == gs["mxfp4_bits_per_value"]
    assert sf.shape == (8, 128 // 32)            # one scale per 32 values


def test_mx_scales_are_powers_of_two():
    """UE8M0: every finite scale is 2^k (mantissa 0.5 under frexp), byte b is
    2^(b-127), byte 255 is NaN."""
    import math
    for b in range(255):
        v = oracle.e8m0_value(b)
        m, e = math.frexp(v)
        assert m == 0.5 and e - 1 == b - 127
    assert math.isnan(oracle.e8m0_value(255))
    x = _mx_rand(np.random.default_rng(32), 16, 256)
    _, sf = oracle.mx_quantize(x)
    for b in np.unique(sf):
        assert math.frexp(oracle.e8m0_value(int(b)))[0] == 0.5


def test_mx_block_scale_against_frexp():
    """X = floor(log2 amax) - 2, clamped; floor(log2) taken from frexp."""
    import math
    rng = np.random.default_rng(33)
    vals = np.concatenate([
        (rng.random(4000) * 2.0 ** rng.integers(-149, 128, 4000)).astype(np.float32),
        np.float32(2.0) ** np.arange(-149, 128).astype(np.float32),
        np.nextafter(np.float32(2.0) ** np.arange(-148, 128).astype(np.float32), np.float32(0)),
    ])
    for v in vals:
        v = float(v)
        if v == 0 or math.isinf(v):
            continue
        e = math.frexp(v)[1] - 1                  # v = m 2^(e+1), m in [0.5, 1)
        want = min(127, max(-127, e - 2)) + 127
        assert oracle.mx_block_scale(v) == want, v
    assert oracle.mx_block_scale(0.0) == 0
    assert oracle.mx_block_scale(6.0) == 127 and oracle.mx_block_scale(8.0) == 128
    assert oracle.mx_block_scale(float("inf")) == -1 and oracle.mx_block_scale(-1.0) == -1


def test_mx_roundtrip_is_exact_on_the_scaled_grid():
    """A block whose values are E2M1 values times 2^k is stored exactly."""
    rng = np.random.default_rng(34)
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
    for _ in range(50):
        rows, cols = 4, 128
        mags = grid[rng.integers(0, 8, (rows, cols))]
        mags[:, ::32] = grid[rng.integers(1, 8, (rows, cols // 32))]     # no all-zero block
        k = rng.integers(-120, 120, (rows, cols // 32)).repeat(32, axis=1)
        x = bf16_bits(mags * np.where(rng.random((rows, cols)) < 0.5, -1, 1) * 2.0 ** k)
        q, sf = oracle.mx_quantize(x)
        y = oracle.mx_dequantize(q, sf)
        assert np.array_equal(bits_to_f32(y), bits_to_f32(x))


def test_mx_saturation_and_ties():
    """With X fixed by the block max: values in (6, 8) 2^X saturate to 6 2^X;
    5 2^X (midway between 4 and 6) goes to 4 (even code 6); 0.25 2^X to 0."""
    row = [7.5, 7.0, 5.0, 0.25, 0.75, 2.5, -3.5, -5.0] + [0.0] * 24
    for k in (-20, 0, 13):
        x = bf16_bits(np.array([row]) * 2.0 ** k)
        q, sf = oracle.mx_quantize(x)
        assert sf[0, 0] == k + 127                  # floor(log2 7.5) - 2 = 0
        y = bits_to_f32(oracle.mx_dequantize(q, sf))[0, :8] / 2.0 ** k
        assert y.tolist() == [6.0, 6.0, 4.0, 0.0, 1.0, 2.0, -4.0, -4.0]


def test_mx_quantize_matches_exact_rationals():
    rng = np.random.default_rng(35)
    for trial in range(30):
        x = _mx_rand(rng, 3, 64)
        q, sf = oracle.mx_quantize(x)
        codes, scales = exact.mx_quantize_rows(x.tolist())
        assert sf.tolist() == scales, f"trial {trial}"
        qc = np.stack([q & 15, q >> 4], axis=-1).reshape(3, 64)
        assert qc.tolist() == codes, f"trial {trial}"


def test_mx_dequant_against_library_rounding():
    """bf16 of E2M1 * 2^(b-127) via ldexp and torch's RNE conversion, for every
    code and every scale byte; byte 255 gives NaN."""
    codes = np.arange(16, dtype=np.uint8)
    for b in range(256):
        q = np.tile((codes[0::2] | (codes[1::2] << 4)).reshape(1, 8), (1, 2))   # 32 values
        sf = np.full((1, 1), b, dtype=np.uint8)
        y = bits_to_f32(oracle.mx_dequantize(q, sf))[0]
        mags = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
        vals = np.tile(np.concatenate([mags, -mags]), 2)
        if b == 255:
            assert np.isnan(y).all()
            continue
        want = torch.tensor(np.ldexp(vals, b - 127), dtype=torch.float64).to(torch.float32).to(torch.bfloat16)
        assert np.array_equal(y, want.float().numpy()), b
    # exact fp64 values
    q = np.array([[0x71] * 16], dtype=np.uint8)           # codes 1 (0.5) and 7 (6)
    assert oracle.mx_dequantize_f64(q, np.array([[130]], dtype=np.uint8))[0, :2].tolist() == [4.0, 48.0]


def test_mx_gemm_f64_against_exact_sums():
    rng = np.random.default_rng(36)
    M, N, K = 3, 4, 96
    aq, asf = oracle.mx_quantize(bf16_bits(rng.standard_normal((M, K))))
    bq, bsf = oracle.mx_quantize(bf16_bits(rng.standard_normal((N, K)) * 40))

    def deq(q, sf, r, k):
        code = (int(q[r, k // 2]) >> (4 * (k % 2))) & 15
        return exact.E2M1[code & 7] * (-1 if code & 8 else 1) * F(2) ** (int(sf[r, k // 32]) - 127)

    C = oracle.mx_gemm_f64(aq, asf, bq, bsf)
    for m in range(M):
        for n in range(N):
            want = sum(deq(aq, asf, m, k) * deq(bq, bsf, n, k) for k in range(K))
            assert abs(F(C[m, n]) - want) <= abs(want) * F(1, 2 ** 48) + F(1, 2 ** 1000)


def test_mx_nonfinite_and_shape_rejected():
    x = bf16_bits(np.ones((2, 32)))
    x[1, 5] = 0x7F80
    with pytest.raises(ValueError):
        oracle.mx_quantize(x)
    with pytest.raises(ValueError):
        oracle.mx_quantize(bf16_bits(np.ones((2, 48))))


# ------------------------------------------------------------------ training variants
def test_philox_known_answers():
    """Philox4x32-10 against the known-answer vectors published with the
    generator (Salmon et al., SC 2011, Random123 test vectors)."""
    cases = [
        ([0, 0, 0, 0], [0, 0], [0x6627e8d5, 0xe169c58d, 0xbc57ac4c, 0x9b00dbd8]),
        ([0xffffffff] * 4, [0xffffffff] * 2, [0x408f276d, 0x41c83b0e, 0xa20bc7c6, 0x6d5451fd]),
        ([0x243f6a88, 0x85a308d3, 0x13198a2e, 0x03707344], [0xa4093822, 0x299f31d0],
         [0xd16cfe09, 0x94fdcceb, 0x5001e420, 0x24126ea1]),
    ]
    for ctr, key, want in cases:
        assert oracle.philox4x32_10(ctr, key).tolist() == want


def _hadamard16():
    from scipy.linalg import hadamard
    return hadamard(16).astype(np.float64)


def test_rht_matches_the_hadamard_matrix():
    """The fp32 butterfly equals H16 diag(s) x / 4 with scipy's Sylvester
    Hadamard matrix: exactly on small integers, within 4 fp32 roundings
    otherwise; H H^T = 16 I."""
    H = _hadamard16()
    assert np.array_equal(H @ H.T, 16 * np.eye(16))
    rng = np.random.default_rng(41)
    for _ in range(200):
        signs = int(rng.integers(0, 1 << 16))
        s = np.array([-1.0 if (signs >> j) & 1 else 1.0 for j in range(16)])
        xi = rng.integers(-64, 64, 16).astype(np.float32)
        assert np.array_equal(oracle.rht16(xi, signs).astype(np.float64), H @ (s * xi) / 4)
        xf = (rng.standard_normal(16) * 2.0 ** rng.integers(-30, 30)).astype(np.float32)
        got = oracle.rht16(xf, signs).astype(np.float64)
        want = H @ (s * xf.astype(np.float64)) / 4
        assert np.all(np.abs(got - want) <= 4 * 2.0 ** -24 * np.abs(xf).sum())


def test_rht_is_orthogonal():
    """Applying the transform twice with no signs returns s .* x, and dot
    products survive the transform (the Wgrad contraction is unchanged)."""
    rng = np.random.default_rng(42)
    for _ in range(100):
        signs = int(rng.integers(0, 1 << 16))
        s = np.array([-1.0 if (signs >> j) & 1 else 1.0 for j in range(16)], dtype=np.float32)
        a = rng.integers(-50, 50, 16).astype(np.float32)
        b = rng.integers(-50, 50, 16).astype(np.float32)
        ta, tb = oracle.rht16(a, signs), oracle.rht16(b, signs)
        assert np.array_equal(oracle.rht16(ta, 0), s * a)
        assert float(np.dot(ta.astype(np.float64), tb)) == float(np.dot(a.astype(np.float64), b))


def test_sr_example_of_the_pages():
    """A value 0.7 of the way between two neighbours rounds up with
    probability 0.7 (to 2^-16): over all 65536 draws, on every E2M1 gap."""
    grid = [0, 0.5, 1, 1.5, 2, 3, 4, 6]
    for k in range(7):
        y = np.float32(grid[k] + 0.7 * (grid[k + 1] - grid[k]))
        p = (float(y) - grid[k]) / (grid[k + 1] - grid[k])
        ups = sum(oracle.e2m1_encode_sr(float(y), u) == k + 1 for u in range(0, 65536, 1))
        assert abs(ups / 65536 - 0.7) < 2 ** -15
        assert ups == int(np.ceil(p * 65536))
        assert all(oracle.e2m1_encode_sr(float(y), u) in (k, k + 1) for u in (0, 12345, 65535))


def test_sr_is_unbiased_over_the_draws():
    """The mean over all 65536 draws of the rounded value is y within one
    part in 2^16 of the gap; grid values never move; 6 and above stay 6."""
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
    rng = np.random.default_rng(43)
    for y in np.concatenate([rng.random(20) * 6, grid]).astype(np.float32):
        codes = np.array([oracle.e2m1_encode_sr(float(y), u) for u in range(0, 65536, 16)])
        mean = grid[codes].mean()
        gap = 2.0 if y >= 4 else 1.0 if y >= 2 else 0.5
        assert abs(mean - float(y)) <= gap * 16 / 65536 + 1e-12
        if float(y) in grid:
            assert np.all(grid[codes] == float(y))
    assert oracle.e2m1_encode_sr(7.5, 0) == 7 and oracle.e2m1_encode_sr(6.0, 65535) == 7


def test_variant_zero_is_the_plain_recipe():
    x = _rand_tensor(np.random.default_rng(44), 32, 64)
    q0, s0, g0 = oracle.quantize(x)
    q1, s1, g1 = oracle.quantize_ex(x, 0)
    assert np.array_equal(q0, q1) and np.array_equal(s0, s1) and np.array_equal(g0, g1)


def _nibbles(q):
    return np.stack([q & 15, q >> 4], axis=-1).reshape(q.shape[:-1] + (2 * q.shape[-1],))


def test_2d_scaling_is_transpose_invariant():
    """The pages' reason for 16x16 weight blocks: quantizing W^T gives the
    transpose of quantizing W (codes and tile scales)."""
    rng = np.random.default_rng(45)
    for _ in range(10):
        x = _rand_tensor(rng, 48, 80)
        xt = np.ascontiguousarray(x.T)
        q, sf, g = oracle.quantize_ex(x, oracle.TWO_D)
        qt, sft, gt = oracle.quantize_ex(xt, oracle.TWO_D)
        assert g[0] == gt[0]
        assert np.array_equal(_nibbles(qt), _nibbles(q).T)
        assert np.array_equal(sft[::16], sf[::16].T)          # one byte per tile, stored per row
        assert np.all(sf.reshape(3, 16, 5)[:, :, :] == sf.reshape(3, 16, 5)[:, :1, :])
        # COLWISE describes x^T
        qc, sfc, gc = oracle.quantize_ex(x, oracle.TWO_D | oracle.COLWISE)
        assert np.array_equal(qc, qt) and np.array_equal(sfc, sft)
    # row-wise 1x16 blocks are not transpose invariant in general
    x = _rand_tensor(np.random.default_rng(46), 32, 32)
    q, _, _ = oracle.quantize_ex(x, 0)
    qt, _, _ = oracle.quantize_ex(np.ascontiguousarray(x.T), 0)
    assert not np.array_equal(_nibbles(qt), _nibbles(q).T)


def test_colwise_quantizes_the_transpose():
    rng = np.random.default_rng(47)
    x = _rand_tensor(rng, 64, 48)
    for v in (0, oracle.SR, oracle.RHT, oracle.RHT | oracle.SR):
        a = oracle.quantize_ex(x, v | oracle.COLWISE, signs=0xA5C3, seed=9, offset=3)
        b = oracle.quantize_ex(np.ascontiguousarray(x.T), v, signs=0xA5C3, seed=9, offset=3)
        for u, w in zip(a, b):
            assert np.array_equal(u, w)


def test_variants_match_exact_rationals():
    """2D tiles, RHT and stochastic rounding re-derived with exact rationals
    (the RHT values from the pinned butterfly, the draws from the pinned
    Philox stream)."""
    rng = np.random.default_rng(48)
    for trial in range(6):
        x = _rand_tensor(rng, 16, 32)
        xs = [[exact.bf16_to_fraction(int(b)) for b in row] for row in x.tolist()]
        # 2D
        q, sf, g = oracle.quantize_ex(x, oracle.TWO_D)
        codes, scales, ge = exact.quantize_values(xs, tiles=True)
        assert F(float(g[0])) == ge and sf.tolist() == scales
        # the sign bit comes from the input bits (a bf16 -0 has no rational sign)
        want = [[(c & 7) | (8 if (b & 0x8000) else 0) for c, b in zip(cr, br)] for cr, br in zip(codes, x.tolist())]
        assert _nibbles(q).tolist() == want, f"2D trial {trial}"
        # RHT (+ SR)
        signs, seed, off = int(rng.integers(0, 1 << 16)), int(rng.integers(0, 1 << 40)), int(rng.integers(0, 99))
        v = np.stack([np.concatenate([oracle.rht16(bits_to_f32(row[c:c + 16]), signs) for c in range(0, 32, 16)])
                      for row in x])
        vf = [[F(float(a)) for a in row] for row in v]
        for variant in (oracle.RHT, oracle.RHT | oracle.SR, oracle.SR):
            vals = vf if variant & oracle.RHT else [[F(float(a)) for a in bits_to_f32(row)] for row in x]
            draws = None
            if variant & oracle.SR:
                draws = []
                for r in range(16):
                    dr = []
                    for c in range(32):
                        i = r * 32 + c
                        n = i // 8 + off
                        w = oracle.philox4x32_10([n & 0xffffffff, n >> 32, 0, 0], [seed & 0xffffffff, seed >> 32])
                        dr.append(int(w[(i & 7) >> 1] >> (16 * (i & 1))) & 0xffff)
                    draws.append(dr)
            q, sf, g = oracle.quantize_ex(x, variant, signs=signs, seed=seed, offset=off)
            codes, scales, ge = exact.quantize_values(vals, draws=draws)
            src = v if variant & oracle.RHT else bits_to_f32(x)
            neg = np.signbit(src)
            want = [[(c & 7) | (8 if n else 0) for c, n in zip(cr, nr)] for cr, nr in zip(codes, neg.tolist())]
            assert F(float(g[0])) == ge and sf.tolist() == scales, f"variant {variant} trial {trial}"
            assert _nibbles(q).tolist() == want, f"variant {variant} trial {trial}"


def test_variant_shape_rules():
    x = _rand_tensor(np.random.default_rng(49), 24, 32)
    with pytest.raises(ValueError):
        oracle.quantize_ex(x, oracle.TWO_D)                  # rows % 16
    with pytest.raises(ValueError):
        oracle.quantize_ex(x, oracle.COLWISE)
    with pytest.raises(ValueError):
        oracle.quantize_ex(_rand_tensor(np.random.default_rng(50), 32, 32), oracle.TWO_D | oracle.RHT)
    oracle.quantize_ex(x, oracle.RHT | oracle.SR)            # row-wise variants take any row count
