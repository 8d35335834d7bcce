"""GPU parity of the INT8 per-row KV format (the pages list INT8 KV beside FP8:
FreeToken PR #897 description and "Regression and CUDA isolation"; read here
as the symmetric counterpart of the FP8 format, s = amax/127, codes rounded
half to even in [-127, 127]).

Codes, scales and reconstructed rows must match the oracle bit for bit;
attention within rel-L2 5e-3 / max-abs 2e-2 of the fp64 oracle over the same
INT8 pool bytes.
"""
import numpy as np
import pytest
import torch

import oracle
import fp8_kv_cache_row_amd as fk
from fp8_kv_cache_row_amd import workloads as wl

from gpu_common import (DEV, assert_bits_equal, assert_close, bf16_to_f64, build_pool, oracle_pool, pool_arrays, say,
                        to_dev, to_dev_bf16)

pytestmark = pytest.mark.gpu
I8 = "int8"


def _oracle(case, ref_pool, seq_lens=None, window=0):
    kc, vc, ks, vs = ref_pool
    lens = case.seq_lens if seq_lens is None else seq_lens
    return oracle.decode_attention(case.q, kc, vc, ks, vs, case.table, lens, case.sm_scale, case.n_kv_heads,
                                   window=window, fmt=I8)


def _check_pool(pool, ref_pool, what):
    for name, a, b in zip(("K codes", "V codes", "K scales", "V scales"), pool_arrays(pool), ref_pool):
        assert_bits_equal(a, b, f"{what}: {name}")


@pytest.mark.parametrize("D", [128, 256])
@pytest.mark.parametrize("layout", ["separate", "interleaved", "interleaved128"])
def test_int8_32k_layer(D, layout):
    say(f"INT8 decode 32K, D={D}, layout={layout}")
    case = wl.layer_decode(90, head_dim=D, with_new_token=False)
    pool = build_pool(case, layout, I8)
    ref_pool = oracle_pool(case, I8)
    _check_pool(pool, ref_pool, f"INT8 D={D}")
    out = fk.fp8kv_decode_attn(pool, to_dev_bf16(case.q), to_dev(case.table), to_dev(case.seq_lens),
                               case.max_seq_len, case.sm_scale)
    torch.cuda.synchronize()
    assert_close(bf16_to_f64(out), _oracle(case, ref_pool), f"INT8 D={D} 32K")


@pytest.mark.parametrize("D", [128, 256])
def test_int8_quantize_every_bf16_pattern_at_unit_scale(D):
    """Rows holding 127 have s = 1 exactly; every bf16 value up to 127 in magnitude."""
    say(f"INT8 quantize of every bf16 pattern <= 127, D={D}")
    pats = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    f = wl.bf16_bits_to_f32(pats)
    pats = pats[np.isfinite(f) & (np.abs(f) <= 127.0)]
    per = D - 1
    n = -(-pats.size // per)
    rows = np.zeros((n, 1, D), np.uint16)
    rows[:, 0, 0] = wl.bf16_bits(np.array([-127.0], np.float32))[0]
    rows[:, 0, 1:] = np.concatenate([pats, np.zeros(n * per - pats.size, np.uint16)]).reshape(n, per)
    codes, scales = oracle.quantize_rows(rows, I8)
    pool = fk.Fp8KvPool(n, 1, device=DEV, head_dim=D, code_format=I8)
    fk.fp8kv_quantize_rows(pool, to_dev_bf16(rows), to_dev_bf16(rows), torch.arange(n, dtype=torch.int32, device=DEV))
    torch.cuda.synchronize()
    kc, vc, ks, vs = pool_arrays(pool)
    assert_bits_equal(kc, codes, "codes")
    assert_bits_equal(vc, codes, "codes (V)")
    assert_bits_equal(ks, scales, "scales")


def test_int8_zero_and_tiny_rows():
    say("INT8 quantize: all-zero rows, signed zeros, subnormal scales")
    rows = np.zeros((4, 2, 128), np.float32)
    rows[1, :, ::3] = -0.0
    rows[2, 0, :8] = np.float32(2.0 ** -130) * np.arange(1, 9)
    rows[3, 1, 5] = 1e-38
    bits = wl.bf16_bits(rows)
    bits[1, :, ::3] = 0x8000
    codes, scales = oracle.quantize_rows(bits, I8)
    pool = fk.Fp8KvPool(4, 2, device=DEV, code_format=I8)
    fk.fp8kv_quantize_rows(pool, to_dev_bf16(bits), to_dev_bf16(bits), torch.arange(4, dtype=torch.int32, device=DEV))
    torch.cuda.synchronize()
    kc, _, ks, _ = pool_arrays(pool)
    assert_bits_equal(kc, codes, "codes")
    assert_bits_equal(ks, scales, "scales")


@pytest.mark.parametrize("L", [1, 17, 513, 8192])
@pytest.mark.parametrize("G", [4, 8])
def test_int8_lengths_and_gqa(L, G):
    say(f"INT8 decode L={L} GQA {G}")
    case = wl.layer_decode(91, ctx=L, pool_rows=L + 40, n_q_heads=4 * G, n_kv_heads=4, with_new_token=False)
    pool = build_pool(case, fmt=I8)
    out = fk.fp8kv_decode_attn(pool, to_dev_bf16(case.q), to_dev(case.table), to_dev(case.seq_lens), L,
                               case.sm_scale)
    torch.cuda.synchronize()
    assert_close(bf16_to_f64(out), _oracle(case, oracle_pool(case, I8)), f"INT8 L={L} G={G}")


@pytest.mark.parametrize("cap", [1, 8, 64])
def test_int8_batched_split_caps(cap):
    say(f"INT8 decode 16 requests, max_splits={cap}")
    case = wl.batched_decode(92, n_req=16, lo=1, hi=12000)
    pool = build_pool(case, fmt=I8)
    out = fk.fp8kv_decode_attn(pool, to_dev_bf16(case.q), to_dev(case.table), to_dev(case.seq_lens),
                               case.max_seq_len, case.sm_scale, max_splits=cap)
    torch.cuda.synchronize()
    got, ref = bf16_to_f64(out), _oracle(case, oracle_pool(case, I8))
    assert_close(got, ref, f"INT8 batched cap={cap}")
    for b in range(case.batch):
        assert_close(got[b], ref[b], f"  request {b} (L={case.seq_lens[b]})")


@pytest.mark.parametrize("D", [128, 256])
@pytest.mark.parametrize("L", [1, 2, 1000, 32768])
def test_int8_append(D, L):
    say(f"INT8 decode+append D={D} L={L}")
    case = wl.layer_decode(93, ctx=L, pool_rows=L + 291, head_dim=D)
    pool = build_pool(case, fmt=I8)
    kc, vc, ks, vs = oracle_pool(case, I8)
    nkc, nks = oracle.quantize_rows(case.new_k, I8)
    nvc, nvs = oracle.quantize_rows(case.new_v, I8)
    row = int(case.table[0, L - 1])
    kc[row], vc[row], ks[row], vs[row] = nkc[0], nvc[0], nks[0], nvs[0]
    lens = np.array([L], np.int32)
    out = fk.fp8kv_decode_attn_append(pool, to_dev_bf16(case.q), to_dev_bf16(case.new_k), to_dev_bf16(case.new_v),
                                      to_dev(np.array([row], np.int32)), to_dev(case.table), to_dev(lens), L,
                                      case.sm_scale)
    torch.cuda.synchronize()
    _check_pool(pool, (kc, vc, ks, vs), f"INT8 append D={D}")
    ref = oracle.decode_attention(case.q, kc, vc, ks, vs, case.table, lens, case.sm_scale, case.n_kv_heads, fmt=I8)
    assert_close(bf16_to_f64(out), ref, f"INT8 append D={D} L={L}")


@pytest.mark.parametrize("D,G,nq,W", [(128, 8, 8, 0), (256, 8, 3, 0), (128, 4, 3, 4095), (256, 8, 1, 17),
                                      (128, 16, 8, 1023)])
def test_int8_rows_and_window(D, G, nq, W):
    say(f"INT8 rows/window: D={D} GQA {G} n_qrows={nq} window={W}")
    Hkv = 2 if G == 16 else 4
    case = wl.layer_decode(94, ctx=20000, pool_rows=20100, n_q_heads=G * Hkv, n_kv_heads=Hkv, head_dim=D,
                           with_new_token=False, n_qrows=nq)
    pool = build_pool(case, fmt=I8)
    q = case.q if case.q.ndim == 4 else case.q[:, None]
    out = fk.fp8kv_decode_attn_rows(pool, to_dev_bf16(q), to_dev(case.table), to_dev(case.seq_lens),
                                    case.max_seq_len, case.sm_scale, window=W)
    torch.cuda.synchronize()
    ref = _oracle(case, oracle_pool(case, I8), window=W)
    assert_close(bf16_to_f64(out), ref if ref.ndim == 4 else ref[:, None], f"INT8 D={D} rows={nq} W={W}")


def test_int8_extreme_codes_through_decode():
    """Rows whose codes hit -127 and 127 in every channel: the widening to
    bf16 is exact at the ends of the range (one key dominates, L = 1 keeps the
    value row)."""
    say("INT8 decode over +-127 codes")
    R, L = 40, 33
    k = np.where(np.arange(128) % 2 == 0, 1.0, -1.0).astype(np.float32)[None, None].repeat(R, 0)
    v = np.random.default_rng(95).standard_normal((R, 1, 128)).astype(np.float32)
    v[:, 0, 0] = 127.0
    v[:, 0, 1] = -127.0
    case = wl.DecodeCase("int8_extreme", 8, 1, R, wl.bf16_bits(k), wl.bf16_bits(v),
                         wl.bf16_bits(np.random.default_rng(96).standard_normal((1, 8, 128)).astype(np.float32)),
                         np.arange(L, dtype=np.int32)[None], np.array([L], np.int32), wl.softmax_scale())
    pool = build_pool(case, fmt=I8)
    ref_pool = oracle_pool(case, I8)
    _check_pool(pool, ref_pool, "extreme")
    assert set(np.unique(ref_pool[0].view(np.int8))) == {-127, 127}
    out = fk.fp8kv_decode_attn(pool, to_dev_bf16(case.q), to_dev(case.table), to_dev(case.seq_lens), L, case.sm_scale)
    torch.cuda.synchronize()
    assert_close(bf16_to_f64(out), _oracle(case, ref_pool), "extreme codes")
