"""Pins for the CPU oracle: what the pages and the mathematics fix, checked
against the oracle without re-typing its formulas.

Each test names what pins it: a value the pages print, the OCP E4M3 table, a
closed form, an invariant, a brute-force search, or a library routine the
special case reduces to.
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle
from fp8_kv_cache_row_amd import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
D = 128


def _read_kv(name):
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            k, v = line.split()
            out[k] = v
    return out


# --------------------------------------------------------------- E4M3 table --

def test_decode_spot_values_match_ocp_table():
    """OCP OFP8 E4M3 special values (golden fixture)."""
    for code_hex, val in _read_kv("e4m3_spot_values.txt").items():
        got = oracle.e4m3_decode(int(code_hex, 16))
        if val == "nan":
            assert math.isnan(got), code_hex
        elif val == "-0":
            assert got == 0.0 and math.copysign(1.0, got) < 0, code_hex
        else:
            assert got == float(val), (code_hex, got, val)
            assert math.copysign(1.0, got) == math.copysign(1.0, float(val))


def test_decode_table_structure():
    """254 finite codes, 2 NaNs, sign symmetry, strictly increasing magnitudes."""
    t = oracle.e4m3_decode_table()
    assert np.isnan(t).sum() == 2 and np.isnan(t[0x7F]) and np.isnan(t[0xFF])
    pos = t[:0x7F]
    assert np.all(np.diff(pos) > 0), "codes 0x00..0x7E must increase"
    assert pos.size == 127 and pos[-1] == 448.0
    for c in range(0x7F):
        assert t[c | 0x80] == -t[c]
    # within a normal binade the grid step is constant: 8 codes per binade
    for e in range(1, 16):
        codes = [(e << 3) | m for m in range(8) if ((e << 3) | m) < 0x7F]
        vals = t[codes]
        steps = np.diff(vals)
        assert np.allclose(steps, steps[0]) if steps.size else True
        assert vals[0] == 2.0 ** (e - 7)


def test_every_finite_value_exact_in_bf16():
    """Library routine: torch's float64 -> bfloat16 cast leaves every finite E4M3 value unchanged."""
    t = oracle.e4m3_decode_table()
    fin = t[np.isfinite(t)]
    back = torch.tensor(fin, dtype=torch.float64).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(back, fin)


# ------------------------------------------------------------------ encode --

def _brute_force_encode(y: np.ndarray) -> np.ndarray:
    """Nearest finite E4M3 magnitude by exhaustive search, ties to the even code.

    Independent of the oracle's encoder: it only uses the (pinned) decode table.
    """
    t = oracle.e4m3_decode_table()
    mags = t[:0x7F]  # codes 0..126, increasing
    y = np.asarray(y, np.float32).astype(np.float64)
    a = np.abs(y)
    dist = np.abs(a[:, None] - mags[None, :])
    best = dist.min(axis=1, keepdims=True)
    cand = dist == best
    idx = np.arange(mags.size)[None, :]
    even_choice = np.where(cand & (idx % 2 == 0), idx, 10_000).min(axis=1)
    any_choice = np.where(cand, idx, 10_000).min(axis=1)
    code = np.where(cand.sum(axis=1) > 1, even_choice, any_choice).astype(np.uint8)
    sign = np.signbit(y).astype(np.uint8) << 7
    return code | sign


def test_encode_round_trip_all_finite_codes():
    """encode(decode(c)) == c for all 254 finite codes, both zeros included."""
    for c in range(256):
        v = oracle.e4m3_decode(c)
        if math.isnan(v):
            continue
        assert oracle.e4m3_encode(v) == c, hex(c)


def test_encode_matches_brute_force_on_all_bf16_patterns():
    """Every bf16 value of magnitude <= 448 (ties and near-ties included)."""
    pats = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    f = wl.bf16_bits_to_f32(pats)
    f = f[np.isfinite(f) & (np.abs(f) <= 448.0)]
    got = oracle.e4m3_encode_array(f)
    for chunk in range(0, f.size, 8192):
        sl = slice(chunk, chunk + 8192)
        assert np.array_equal(got[sl], _brute_force_encode(f[sl]))


def test_encode_matches_brute_force_at_midpoints_and_neighbours():
    """fp32 midpoints between adjacent E4M3 values, and one fp32 ulp either side."""
    t = oracle.e4m3_decode_table()[:0x7F]
    mids = ((t[:-1] + t[1:]) / 2).astype(np.float32)
    pts = np.concatenate([mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(1e9)),
                          t.astype(np.float32), np.float32(2.0 ** -10) * np.arange(0, 20, dtype=np.float32)])
    pts = np.concatenate([pts, -pts])
    assert np.array_equal(oracle.e4m3_encode_array(pts), _brute_force_encode(pts))


def test_encode_matches_brute_force_random_fp32():
    rng = np.random.default_rng(1234)
    y = (rng.standard_normal(40000) * np.exp(rng.uniform(-12, 6, 40000))).astype(np.float32)
    y = y[np.abs(y) <= 448]
    assert np.array_equal(oracle.e4m3_encode_array(y), _brute_force_encode(y))


def test_encode_saturates_and_keeps_signed_zero():
    assert oracle.e4m3_encode(448.0) == 0x7E
    assert oracle.e4m3_encode(460.0) == 0x7E
    assert oracle.e4m3_encode(470.0) == 0x7E  # past the 448/480 midpoint: never the NaN code
    assert oracle.e4m3_encode(-479.0) == 0xFE
    assert oracle.e4m3_encode(1e30) == 0x7E
    assert oracle.e4m3_encode(-1000.0) == 0xFE
    assert oracle.e4m3_encode(-0.0) == 0x80
    assert oracle.e4m3_encode(-1e-6) == 0x80  # rounds to zero, keeps the sign
    assert oracle.e4m3_encode(2.0 ** -10) == 0x00  # exact tie between 0 and 2^-9 -> even (0)
    assert oracle.e4m3_encode(3 * 2.0 ** -10) == 0x02  # tie between codes 1 and 2 -> 2


# ---------------------------------------------------------------- quantize --

def _ulp_e4m3(a):
    a = np.abs(np.asarray(a, np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -30)))
    return np.maximum(2.0 ** -9, 2.0 ** (e - 3))


def test_quantize_error_bound_half_ulp_times_scale():
    """|x - decode(c)*s| <= (half an E4M3 ulp of x/s + fp32 division slop) * s."""
    case = wl.layer_decode(seed=3, ctx=64, pool_rows=512, with_new_token=False)
    rows = case.k_rows.reshape(-1, D)
    codes, scales = oracle.quantize_rows(rows)
    x = wl.bf16_bits_to_f32(rows).astype(np.float64)
    xhat = oracle.dequantize(codes, scales)
    s = scales.astype(np.float64)[:, None]
    y = x / s
    bound = (0.5 * _ulp_e4m3(y) + np.abs(y) * 2.0 ** -23) * s
    assert np.all(np.abs(x - xhat) <= bound)
    # the scale is amax/448 to within one fp32 rounding
    amax = np.abs(x).max(axis=1)
    assert np.all(np.abs(scales.astype(np.float64) * 448.0 - amax) <= amax * 2.0 ** -23)
    # the largest element of every row lands on the top code
    top = np.take_along_axis(codes, np.abs(x).argmax(axis=1)[:, None], axis=1)[:, 0]
    assert np.all((top & 0x7F) == 0x7E)


def test_quantize_power_of_two_scales_closed_form():
    """amax = 448 * 2^k gives s = 2^k exactly and codes = nearest-even encode(x * 2^-k)."""
    rng = np.random.default_rng(7)
    for k in (-20, -3, 0, 1, 5):
        x = rng.standard_normal((16, D)).astype(np.float32) * np.float32(2.0 ** k) * 60
        x = np.clip(x, -448 * 2.0 ** k, 448 * 2.0 ** k).astype(np.float32)
        xb = wl.bf16_bits(x)
        xb[:, 5] = wl.bf16_bits(np.array([448 * 2.0 ** k], np.float32))[0]
        codes, scales = oracle.quantize_rows(xb)
        assert np.all(scales == np.float32(2.0 ** k))
        y = wl.bf16_bits_to_f32(xb) * np.float32(2.0 ** -k)  # exact
        assert np.array_equal(codes, _brute_force_encode(y.ravel()).reshape(codes.shape))


def test_quantize_all_bf16_patterns_at_unit_scale():
    rows = wl.all_bf16_patterns_row_batches()
    codes, scales = oracle.quantize_rows(rows)
    assert np.all(scales == 1.0)
    ref = _brute_force_encode(wl.bf16_bits_to_f32(rows).ravel()).reshape(codes.shape)
    assert np.array_equal(codes, ref)


def test_quantize_zero_row_and_signed_zeros():
    row = np.zeros((2, D), np.uint16)
    row[0, ::2] = 0x8000  # -0.0 in bf16
    codes, scales = oracle.quantize_rows(row)
    assert scales[0] == 0.0 and scales[1] == 0.0
    assert np.all(codes[0, ::2] == 0x80) and np.all(codes[0, 1::2] == 0x00)
    assert np.all(codes[1] == 0x00)


def test_quantize_tiny_row_subnormal_scale():
    """amax below 448 * 2^-126 gives a subnormal fp32 scale; the error bound still holds."""
    x = np.zeros((1, D), np.float32)
    x[0, :8] = np.float32(2.0 ** -130) * np.arange(1, 9, dtype=np.float32)
    xb = wl.bf16_bits(x)
    codes, scales = oracle.quantize_rows(xb)
    assert 0 < scales[0] < np.finfo(np.float32).tiny
    xhat = oracle.dequantize(codes, scales)[0]
    xf = wl.bf16_bits_to_f32(xb)[0].astype(np.float64)
    # s is subnormal, so x/s may exceed 448 slightly and saturate; allow one E4M3 step at the top
    assert np.all(np.abs(xhat - xf) <= 32.0 * scales[0] + 1e-300)


# -------------------------------------------------------------- bf16 / ws --

def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(5)
    f = (rng.standard_normal(20000) * np.exp(rng.uniform(-80, 80, 20000))).astype(np.float32)
    # exact ties: low 16 bits == 0x8000
    ties = (rng.integers(0, 1 << 15, 2000).astype(np.uint32) << 16 | 0x8000).view(np.float32)
    f = np.concatenate([f, ties, -ties, np.array([0.0, -0.0, 1e-40, -1e-41], np.float32)])
    f = f[np.isfinite(f)]
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([oracle.f32_to_bf16(v) for v in f], np.uint16)
    assert np.array_equal(got, ref)


def test_reconstruct_power_of_two_scale_is_exact():
    rng = np.random.default_rng(9)
    codes = rng.integers(0, 256, (32, 2, D)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x12
    scales = np.full((32, 2), np.float32(2.0 ** -5), np.float32)
    ws = oracle.reconstruct(codes, scales, np.arange(32, dtype=np.int32)[::-1].copy(), 2)
    exact = oracle.e4m3_decode_table()[codes[::-1]] * 2.0 ** -5
    assert np.array_equal(wl.bf16_bits_to_f32(ws).astype(np.float64), exact)


def test_reconstruct_matches_torch_float_ops():
    """Library routine: torch float32 product then torch's bf16 cast."""
    rng = np.random.default_rng(11)
    codes = rng.integers(0, 256, (40, 4, D)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x33
    scales = (rng.uniform(0.001, 0.1, (40, 4))).astype(np.float32)
    scales[0, 0] = np.float32(1e-42)  # subnormal scale: products become fp32 subnormals
    rows = rng.permutation(40).astype(np.int32)[:25]
    ws = oracle.reconstruct(codes, scales, rows, 4)
    dec = torch.tensor(oracle.e4m3_decode_table()[codes[rows]], dtype=torch.float32)
    ref = (dec * torch.from_numpy(scales[rows])[..., None]).to(torch.bfloat16)
    assert np.array_equal(ws, ref.view(torch.int16).numpy().view(np.uint16))


# --------------------------------------------------------------- accounting --

def test_pool_bytes_match_pages():
    g = _read_kv("pool_bytes.txt")
    L, H, Dh = int(g["n_layers"]), int(g["n_kv_heads"]), int(g["head_dim"])
    fp8 = oracle.fp8_bytes_per_token(L, H, Dh)
    bf16 = oracle.bf16_bytes_per_token(L, H, Dh)
    assert fp8 == int(g["fp8_bytes_per_token"])
    assert bf16 == int(g["bf16_bytes_per_token"])
    R = int(g["pool_rows"])
    assert fp8 * R == int(g["fp8_pool_bytes"])
    assert bf16 * R == int(g["bf16_pool_bytes"])
    ws = oracle.bf16_workspace_bytes(R, H, Dh)
    assert ws == int(g["bf16_workspace_bytes"])
    saving = 100.0 * (1 - (fp8 * R + ws) / (bf16 * R))
    assert round(saving, 2) == float(g["fp8_plus_workspace_saving_percent"])
    assert round(100.0 * (1 - fp8 / bf16), 1) == float(g["fp8_per_token_reduction_percent"])


# ------------------------------------------------------------ decode attn --

def _pool_from_values(k_codes, v_codes, k_scales, v_scales):
    return (np.ascontiguousarray(k_codes, np.uint8), np.ascontiguousarray(v_codes, np.uint8),
            np.ascontiguousarray(k_scales, np.float32), np.ascontiguousarray(v_scales, np.float32))


def _q_bits(q):
    return wl.bf16_bits(np.asarray(q, np.float32))


def test_decode_identical_keys_give_mean_of_v():
    rng = np.random.default_rng(0)
    R, Hkv, Hq, L = 40, 1, 8, 33
    krow = wl.bf16_bits(rng.standard_normal((1, Hkv, D)).astype(np.float32))
    kc, ks = oracle.quantize_rows(np.repeat(krow, R, axis=0))
    vc, vs = oracle.quantize_rows(wl.bf16_bits(rng.standard_normal((R, Hkv, D)).astype(np.float32)))
    table = rng.permutation(R)[:L].astype(np.int32)[None]
    q = _q_bits(rng.standard_normal((1, Hq, D)))
    out = oracle.decode_attention(q, kc, vc, ks, vs, table, np.array([L], np.int32), 0.0883883, Hkv)
    vhat = oracle.dequantize(vc, vs)[table[0], 0]
    np.testing.assert_allclose(out[0], np.broadcast_to(vhat.mean(axis=0), (Hq, D)), rtol=1e-12, atol=1e-14)


def test_decode_single_row_returns_that_v():
    rng = np.random.default_rng(1)
    vc, vs = oracle.quantize_rows(wl.bf16_bits(rng.standard_normal((4, 2, D)).astype(np.float32)))
    kc, ks = oracle.quantize_rows(wl.bf16_bits(rng.standard_normal((4, 2, D)).astype(np.float32)))
    q = _q_bits(rng.standard_normal((1, 4, D)))
    out = oracle.decode_attention(q, kc, vc, ks, vs, np.array([[2]], np.int32), np.array([1], np.int32), 0.09, 2)
    vhat = oracle.dequantize(vc, vs)[2]
    for h in range(4):
        np.testing.assert_array_equal(out[0, h], vhat[h // 2])


def test_decode_hand_computed_softmax_weights():
    """Scores 0, 1, 2 (exact codes, unit scales, sm_scale 1) -> weights e^z / sum e^z."""
    R, Hkv = 3, 1
    kc = np.zeros((R, Hkv, D), np.uint8)
    kc[:, 0, 0] = [0x00, 0x38, 0x40]  # 0.0, 1.0, 2.0
    vc = np.zeros((R, Hkv, D), np.uint8)
    for r in range(R):
        vc[r, 0, r] = 0x38  # one-hot rows of value 1.0
    ks = np.ones((R, Hkv), np.float32)
    vs = np.full((R, Hkv), 0.5, np.float32)
    q = np.zeros((1, 1, D), np.float32)
    q[0, 0, 0] = 1.0
    out = oracle.decode_attention(_q_bits(q), kc, vc, ks, vs, np.array([[0, 1, 2]], np.int32),
                                  np.array([3], np.int32), 1.0, Hkv)
    den = 1 + math.e + math.e ** 2
    expect = [0.5 * 1 / den, 0.5 * math.e / den, 0.5 * math.e ** 2 / den]
    np.testing.assert_allclose(out[0, 0, :3], expect, rtol=1e-14)
    assert np.all(out[0, 0, 3:] == 0)


def test_decode_softmax_scale_and_key_scale_enter_scores():
    """Two keys with dots 0 and 1 * k_scale; weight ratio must be exp(sm_scale * k_scale)."""
    kc = np.zeros((2, 1, D), np.uint8)
    kc[1, 0, 0] = 0x38
    vc = np.zeros((2, 1, D), np.uint8)
    vc[0, 0, 0] = 0x38
    vc[1, 0, 1] = 0x38
    ks = np.array([[1.0], [3.0]], np.float32)
    vs = np.ones((2, 1), np.float32)
    q = np.zeros((1, 1, D), np.float32)
    q[0, 0, 0] = 2.0
    out = oracle.decode_attention(_q_bits(q), kc, vc, ks, vs, np.array([[0, 1]], np.int32),
                                  np.array([2], np.int32), 0.25, 1)
    ratio = out[0, 0, 1] / out[0, 0, 0]
    np.testing.assert_allclose(ratio, math.exp(0.25 * 2.0 * 3.0), rtol=1e-13)


def test_decode_gqa_head_mapping_consecutive_groups():
    """Hq=8, Hkv=2: heads 0-3 read KV head 0, heads 4-7 read KV head 1."""
    R = 5
    kc = np.zeros((R, 2, D), np.uint8)
    vc = np.zeros((R, 2, D), np.uint8)
    vc[:, 0, :] = 0x38  # 1.0
    vc[:, 1, :] = 0x40  # 2.0
    ks = np.ones((R, 2), np.float32)
    vs = np.ones((R, 2), np.float32)
    rng = np.random.default_rng(2)
    q = _q_bits(rng.standard_normal((1, 8, D)))
    out = oracle.decode_attention(q, kc, vc, ks, vs, np.arange(R, dtype=np.int32)[None],
                                  np.array([R], np.int32), 0.1, 2)
    assert np.all(out[0, :4] == 1.0) and np.all(out[0, 4:] == 2.0)


def test_decode_zero_query_is_uniform_average():
    case = wl.layer_decode(seed=4, ctx=100, pool_rows=150, n_q_heads=8, n_kv_heads=2, with_new_token=False)
    kc, ks = oracle.quantize_rows(case.k_rows)
    vc, vs = oracle.quantize_rows(case.v_rows)
    q = np.zeros_like(case.q)
    out = oracle.decode_attention(q, kc, vc, ks, vs, case.table, case.seq_lens, case.sm_scale, 2)
    vhat = oracle.dequantize(vc, vs)[case.table[0]]  # [L][Hkv][D]
    for h in range(8):
        np.testing.assert_allclose(out[0, h], vhat[:, h // 4].mean(axis=0), rtol=1e-12, atol=1e-15)


def test_decode_dominant_key():
    rng = np.random.default_rng(3)
    R = 20
    kc = np.zeros((R, 1, D), np.uint8)
    kc[7, 0, :] = 0x7E  # 448 in every channel
    ks = np.ones((R, 1), np.float32)
    vc, vs = oracle.quantize_rows(wl.bf16_bits(rng.standard_normal((R, 1, D)).astype(np.float32)))
    q = np.full((1, 1, D), 1.0, np.float32)
    out = oracle.decode_attention(_q_bits(q), kc, vc, ks, vs, np.arange(R, dtype=np.int32)[None],
                                  np.array([R], np.int32), 0.1, 1)
    np.testing.assert_allclose(out[0, 0], oracle.dequantize(vc, vs)[7, 0], rtol=0, atol=1e-12)


def test_decode_row_permutation_invariance_and_unreferenced_rows():
    case = wl.layer_decode(seed=5, ctx=300, pool_rows=400, n_q_heads=8, n_kv_heads=1, with_new_token=False)
    kc, ks = oracle.quantize_rows(case.k_rows)
    vc, vs = oracle.quantize_rows(case.v_rows)
    base = oracle.decode_attention(case.q, kc, vc, ks, vs, case.table, case.seq_lens, case.sm_scale, 1)
    rng = np.random.default_rng(6)
    perm = rng.permutation(400)  # new row p holds old row perm[p]
    inv = np.argsort(perm)
    t2 = inv[case.table].astype(np.int32)
    out = oracle.decode_attention(case.q, kc[perm], vc[perm], ks[perm], vs[perm], t2, case.seq_lens,
                                  case.sm_scale, 1)
    np.testing.assert_allclose(out, base, rtol=1e-12, atol=1e-14)
    # rows outside the table do not matter
    unused = np.setdiff1d(np.arange(400), case.table[0])
    kc2, vc2 = kc.copy(), vc.copy()
    kc2[unused] = 0x55
    vc2[unused] = 0x66
    out2 = oracle.decode_attention(case.q, kc2, vc2, ks, vs, case.table, case.seq_lens, case.sm_scale, 1)
    np.testing.assert_array_equal(out2, base)


def test_decode_empty_sequence_gives_zeros():
    kc = np.zeros((2, 1, D), np.uint8)
    out = oracle.decode_attention(_q_bits(np.ones((2, 2, D))), kc, kc, np.ones((2, 1), np.float32),
                                  np.ones((2, 1), np.float32), np.array([[0, 1], [1, 0]], np.int32),
                                  np.array([0, 2], np.int32), 0.1, 1)
    assert np.all(out[0] == 0)
    assert np.all(np.isfinite(out[1]))


def test_decode_brute_force_tiny_against_float128_free_sum():
    """17 keys (a page size the pages test): compare with a direct fp64 log-sum-exp
    evaluation written from the softmax definition using math.fsum."""
    rng = np.random.default_rng(17)
    R, Hkv, Hq, L = 17, 1, 4, 17
    kc, ks = oracle.quantize_rows(wl.bf16_bits(rng.standard_normal((R, Hkv, D)).astype(np.float32)))
    vc, vs = oracle.quantize_rows(wl.bf16_bits(rng.standard_normal((R, Hkv, D)).astype(np.float32)))
    q = _q_bits(rng.standard_normal((1, Hq, D)))
    table = rng.permutation(R).astype(np.int32)[None]
    sm = 0.0883883461356163
    out = oracle.decode_attention(q, kc, vc, ks, vs, table, np.array([L], np.int32), sm, Hkv)
    kh = oracle.dequantize(kc, vs * 0 + ks)[:, 0]
    vh = oracle.dequantize(vc, vs)[:, 0]
    qf = wl.bf16_bits_to_f32(q)[0].astype(np.float64)
    for h in range(Hq):
        z = [math.fsum(qf[h] * kh[r]) * np.float64(np.float32(sm)) for r in table[0]]
        w = [math.exp(zz - max(z)) for zz in z]
        tot = math.fsum(w)
        ref = [math.fsum(w[i] * vh[table[0, i], d] for i in range(L)) / tot for d in range(D)]
        np.testing.assert_allclose(out[0, h], ref, rtol=1e-10, atol=1e-13)


# ----------------------------------------------------------- prefill attn --

def test_prefill_first_query_without_prefix_returns_first_value():
    rng = np.random.default_rng(8)
    T, Hq, Hkv = 5, 4, 2
    q = _q_bits(rng.standard_normal((T, Hq, D)))
    k = _q_bits(rng.standard_normal((T, Hkv, D)))
    v = _q_bits(rng.standard_normal((T, Hkv, D)))
    out = oracle.prefill_attention(q, None, None, k, v, 0.1, q_idx=[0])
    for h in range(Hq):
        np.testing.assert_array_equal(out[0, h], wl.bf16_bits_to_f32(v[0, h // 2]))


def test_prefill_identical_keys_causal_running_mean():
    """All keys equal -> query i averages prefix values and chunk values 0..i."""
    rng = np.random.default_rng(9)
    P, T, Hq, Hkv = 6, 7, 2, 1
    krow = _q_bits(rng.standard_normal((1, Hkv, D)))
    wsk = np.repeat(krow, P, 0)
    kcur = np.repeat(krow, T, 0)
    wsv = _q_bits(rng.standard_normal((P, Hkv, D)))
    vcur = _q_bits(rng.standard_normal((T, Hkv, D)))
    q = _q_bits(rng.standard_normal((T, Hq, D)))
    out = oracle.prefill_attention(q, wsk, wsv, kcur, vcur, 0.1)
    allv = np.concatenate([wl.bf16_bits_to_f32(wsv), wl.bf16_bits_to_f32(vcur)], 0)[:, 0].astype(np.float64)
    for i in range(T):
        np.testing.assert_allclose(out[i, 0], allv[:P + i + 1].mean(0), rtol=1e-12, atol=1e-14)


def test_prefill_causality_and_prefix_visibility():
    rng = np.random.default_rng(10)
    P, T, Hq, Hkv = 4, 6, 4, 2
    mk = lambda s: _q_bits(rng.standard_normal(s))
    q, kc, vc = mk((T, Hq, D)), mk((T, Hkv, D)), mk((T, Hkv, D))
    wk, wv = mk((P, Hkv, D)), mk((P, Hkv, D))
    base = oracle.prefill_attention(q, wk, wv, kc, vc, 0.09)
    kc2, vc2 = kc.copy(), vc.copy()
    kc2[4:] = mk((2, Hkv, D))
    vc2[4:] = mk((2, Hkv, D))
    out = oracle.prefill_attention(q, wk, wv, kc2, vc2, 0.09)
    np.testing.assert_array_equal(out[:4], base[:4])  # queries 0..3 cannot see rows 4, 5
    assert not np.allclose(out[4:], base[4:])
    wv2 = wv.copy()
    wv2[0] = mk((Hkv, D))
    out3 = oracle.prefill_attention(q, wk, wv2, kc, vc, 0.09, q_idx=[0])
    assert not np.allclose(out3[0], base[0])  # every query sees the prefix


def test_prefill_gqa_head_mapping():
    P, T, Hq, Hkv = 3, 2, 4, 2
    z = np.zeros
    wsk = z((P, Hkv, D), np.uint16)
    kcur = z((T, Hkv, D), np.uint16)
    wsv = z((P, Hkv, D), np.float32)
    vcur = z((T, Hkv, D), np.float32)
    wsv[:, 1] = 3.0
    vcur[:, 1] = 3.0
    wsv[:, 0] = -1.0
    vcur[:, 0] = -1.0
    q = _q_bits(np.random.default_rng(0).standard_normal((T, Hq, D)))
    out = oracle.prefill_attention(q, wsk, _q_bits(wsv), kcur, _q_bits(vcur), 0.1)
    assert np.all(out[:, :2] == -1.0) and np.all(out[:, 2:] == 3.0)
