"""GPU parity: quantize-on-write and prefill reconstruction, bit-exact against the oracle."""
import numpy as np
import pytest
import torch

import oracle
import fp8_kv_cache_row_amd as fk
from fp8_kv_cache_row_amd import workloads as wl

from gpu_common import (DEV, assert_bits_equal, build_pool, oracle_pool, pool_arrays, say, to_dev,
                        to_dev_bf16)

pytestmark = pytest.mark.gpu
D = 128


def _quantize_rows_gpu(rows_bits: np.ndarray, layout="separate"):
    """rows [N][128] bf16 bits -> (codes, scales) via the HIP path (1 KV head, slot r = r)."""
    n = rows_bits.shape[0]
    pool = fk.Fp8KvPool(n, 1, layout=layout, device=DEV)
    x = to_dev_bf16(rows_bits.reshape(n, 1, D))
    fk.fp8kv_quantize_rows(pool, x, x, torch.arange(n, dtype=torch.int32, device=DEV))
    kc, vc, ks, vs = pool_arrays(pool)
    assert_bits_equal(kc, vc, "K and V paths of the same rows")
    return kc[:, 0], ks[:, 0]


@pytest.mark.parametrize("layout", ["separate", "interleaved"])
def test_tiny_case_codes_and_scales_bit_exact(layout):
    say(f"quantize tiny 256 K + 256 V rows, layout={layout}")
    case = wl.tiny_decode(0)
    pool = build_pool(case, layout)
    kc, vc, ks, vs = pool_arrays(pool)
    okc, ovc, oks, ovs = oracle_pool(case)
    assert_bits_equal(kc, okc, "K codes")
    assert_bits_equal(vc, ovc, "V codes")
    assert_bits_equal(ks, oks, "K scales")
    assert_bits_equal(vs, ovs, "V scales")


def test_every_bf16_pattern_at_unit_scale():
    say("quantize all bf16 patterns with |x| <= 448 (scale 1)")
    rows = wl.all_bf16_patterns_row_batches()
    codes, scales = _quantize_rows_gpu(rows)
    oc, os_ = oracle.quantize_rows(rows)
    assert_bits_equal(codes, oc, "codes")
    assert_bits_equal(scales, os_, "scales")


def test_edge_rows():
    say("quantize edge rows: zero, signed zeros, subnormal scale, powers of two, huge, ties")
    rng = np.random.default_rng(42)
    rows = []
    rows.append(np.zeros(D, np.float32))
    z = np.zeros(D, np.float32)
    z[::3] = -0.0
    rows.append(z)
    t = np.zeros(D, np.float32)
    t[:8] = np.float32(2.0 ** -130) * np.arange(1, 9)
    rows.append(t)
    t2 = np.zeros(D, np.float32)
    t2[5] = -np.float32(2.0 ** -133)  # the smallest bf16 subnormal
    rows.append(t2)
    for k in (-40, -10, -1, 0, 3, 20, 100):
        r = (rng.standard_normal(D) * 50).astype(np.float32)
        r = np.clip(r, -448, 448) * np.float32(2.0 ** k)
        r[7] = np.float32(448.0 * 2.0 ** k)
        rows.append(r.astype(np.float32))
    big = (rng.standard_normal(D) * 1e30).astype(np.float32)
    rows.append(big)
    one = np.full(D, 1.0, np.float32)
    one[0] = 448.0
    rows.append(one)
    mix = (rng.standard_normal(D) * np.exp(rng.uniform(-20, 20, D))).astype(np.float32)
    rows.append(mix)
    bits = wl.bf16_bits(np.stack(rows))
    codes, scales = _quantize_rows_gpu(bits)
    oc, os_ = oracle.quantize_rows(bits)
    assert_bits_equal(codes, oc, "codes")
    assert_bits_equal(scales, os_, "scales")


def test_random_rows_many_scales():
    say("quantize 40,000 random rows spanning 60 binades of scale")
    rng = np.random.default_rng(7)
    n = 40000
    x = rng.standard_normal((n, D)).astype(np.float32)
    x *= np.exp2(rng.integers(-30, 30, (n, 1))).astype(np.float32)
    x[:, :4] *= 8
    bits = wl.bf16_bits(x)
    codes, scales = _quantize_rows_gpu(bits)
    oc, os_ = oracle.quantize_rows(bits)
    assert_bits_equal(codes, oc, "codes")
    assert_bits_equal(scales, os_, "scales")


def test_scatter_into_slots_leaves_other_rows_untouched():
    say("quantize 8,192 chunk tokens x 4 heads into scattered slots; canary rows")
    case = wl.chunked_prefill(0)
    R, H = case.pool_rows, case.n_kv_heads
    pool = fk.Fp8KvPool(R, H, device=DEV)
    pool.k_codes.fill_(0xA5)
    pool.v_codes.fill_(0x5A)
    pool.k_scales.fill_(-7.0)
    pool.v_scales.fill_(-9.0)
    slots = case.chunk_slots
    fk.fp8kv_quantize_rows(pool, to_dev_bf16(case.k_cur), to_dev_bf16(case.v_cur), to_dev(slots))
    torch.cuda.synchronize()
    kc, vc, ks, vs = pool_arrays(pool)
    okc, oks = oracle.quantize_rows(case.k_cur)
    ovc, ovs = oracle.quantize_rows(case.v_cur)
    assert_bits_equal(kc[slots], okc, "K codes at slots")
    assert_bits_equal(vc[slots], ovc, "V codes at slots")
    assert_bits_equal(ks[slots], oks, "K scales at slots")
    assert_bits_equal(vs[slots], ovs, "V scales at slots")
    other = np.setdiff1d(np.arange(R), slots)
    assert np.all(kc[other] == 0xA5) and np.all(vc[other] == 0x5A)
    assert np.all(ks[other] == -7.0) and np.all(vs[other] == -9.0)


def test_strided_source_tokens():
    """Source rows with a token stride larger than Hkv*128 (e.g. a fused QKV buffer)."""
    say("quantize from a strided [T][stride] source")
    rng = np.random.default_rng(3)
    T, H = 37, 2
    stride = 3 * H * D + 8
    buf = wl.bf16_bits(rng.standard_normal((T, stride)).astype(np.float32))
    dev = to_dev_bf16(buf)
    k = dev[:, :H * D].view(T, H, D)
    v = dev[:, 2 * H * D:3 * H * D].view(T, H, D)
    pool = fk.Fp8KvPool(64, H, device=DEV)
    slots = rng.permutation(64)[:T].astype(np.int32)
    fk.fp8kv_quantize_rows(pool, k, v, to_dev(slots))
    kc, vc, ks, vs = pool_arrays(pool)
    okc, oks = oracle.quantize_rows(buf[:, :H * D].reshape(T, H, D))
    ovc, ovs = oracle.quantize_rows(buf[:, 2 * H * D:3 * H * D].reshape(T, H, D))
    assert_bits_equal(kc[slots], okc, "K codes")
    assert_bits_equal(vc[slots], ovc, "V codes")
    assert_bits_equal(ks[slots], oks, "K scales")
    assert_bits_equal(vs[slots], ovs, "V scales")


@pytest.mark.parametrize("layout", ["separate", "interleaved"])
def test_reconstruct_every_code_both_orientations(layout):
    """All 256 codes (NaN codes replaced) through K and V reconstruction, with
    unit, power-of-two, general and subnormal scales: bit-exact, signed zero kept."""
    say(f"reconstruct all codes, layout={layout}")
    R, H = 64, 2
    pool = fk.Fp8KvPool(R, H, layout=layout, device=DEV)
    codes = np.tile(np.arange(256, dtype=np.uint8).reshape(2, 128), (R // 2, 1)).reshape(R, 1, D)
    codes = np.repeat(codes, H, axis=1)
    codes[(codes & 0x7F) == 0x7F] = 0x00
    vcodes = codes[::-1].copy()
    rng = np.random.default_rng(1)
    ks = rng.uniform(1e-3, 1.0, (R, H)).astype(np.float32)
    ks[0] = 1.0
    ks[1] = 2.0 ** -7
    ks[2] = np.float32(1e-40)  # subnormal scale
    vs = rng.uniform(1e-3, 1.0, (R, H)).astype(np.float32)
    vs[3] = 1.0
    pool.k_codes.copy_(to_dev(codes))
    pool.v_codes.copy_(to_dev(vcodes))
    if layout == "separate":
        pool.k_scales.copy_(to_dev(ks))
        pool.v_scales.copy_(to_dev(vs))
    else:
        off = 2 * H * D
        pool.record[:, off:off + 4 * H].copy_(to_dev(ks.view(np.uint8).reshape(R, 4 * H)))
        pool.record[:, off + 4 * H:off + 8 * H].copy_(to_dev(vs.view(np.uint8).reshape(R, 4 * H)))
    rows = np.random.default_rng(2).permutation(R).astype(np.int32)[:48]
    P = rows.size
    q = torch.zeros((1, 2 * H, D), dtype=torch.bfloat16, device=DEV)
    kcur = torch.zeros((1, H, D), dtype=torch.bfloat16, device=DEV)
    ws_k = torch.full((P + 3, H, D), 7.0, dtype=torch.bfloat16, device=DEV)
    ws_v = torch.full((P + 3, H, D), 7.0, dtype=torch.bfloat16, device=DEV)
    fk.fp8kv_prefill_attn(pool, q, kcur, kcur, to_dev(rows), ws_k, ws_v, 0.1)
    torch.cuda.synchronize()
    gk = ws_k.view(torch.int16).cpu().numpy().view(np.uint16)
    gv = ws_v.view(torch.int16).cpu().numpy().view(np.uint16)
    assert_bits_equal(gk[:P], oracle.reconstruct(codes, ks, rows, H), "ws_k")
    assert_bits_equal(gv[:P], oracle.reconstruct(vcodes, vs, rows, H), "ws_v")
    assert np.all(gk[P:] == 0x40E0) and np.all(gv[P:] == 0x40E0)  # rows past P untouched (7.0)
