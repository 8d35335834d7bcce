"""GPU parity of the VALU-only decode stage 1 (fp8kv_decode_stage1_valu, merged
by fp8kv_decode_merge) against the fp64 oracle, and against the MFMA stage 1
on the same inputs: the tiny case, the 32K-context layer, every GQA ratio with
one-round and several-round split choices, ragged lengths, a batch with an
empty request, and the rejected shapes."""
import numpy as np
import pytest
import torch

import oracle
import fp8_kv_cache_row_amd as fk
from fp8_kv_cache_row_amd import binding as B
from fp8_kv_cache_row_amd import workloads as wl

from gpu_common import DEV, assert_close, bf16_to_f64, build_pool, oracle_pool, say, to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu


def _valu(pool, case, max_splits=0, seq_lens=None, max_seq_len=None):
    q = to_dev_bf16(case.q)
    t = to_dev(case.table)
    sl = to_dev((case.seq_lens if seq_lens is None else seq_lens).astype(np.int32))
    msl = case.max_seq_len if max_seq_len is None else max_seq_len
    ws = fk.binding.fp8kv_decode_stage1_valu(pool, q, t, sl, msl, case.sm_scale, max_splits=max_splits)
    out = fk.fp8kv_decode_merge(ws, q.shape[0], q.shape[1], max_splits=max_splits)
    torch.cuda.synchronize()
    return bf16_to_f64(out)


def _mfma(pool, case, max_splits=0, seq_lens=None, max_seq_len=None):
    sl = to_dev((case.seq_lens if seq_lens is None else seq_lens).astype(np.int32))
    msl = case.max_seq_len if max_seq_len is None else max_seq_len
    out = fk.fp8kv_decode_attn(pool, to_dev_bf16(case.q), to_dev(case.table), sl, msl, case.sm_scale,
                               max_splits=max_splits)
    torch.cuda.synchronize()
    return bf16_to_f64(out)


def _oracle(case, seq_lens=None):
    kc, vc, ks, vs = oracle_pool(case)
    return oracle.decode_attention(case.q, kc, vc, ks, vs, case.table,
                                   case.seq_lens if seq_lens is None else seq_lens, case.sm_scale, case.n_kv_heads)


def test_valu_tiny():
    say("VALU stage 1: tiny GQA-8, 256 rows")
    case = wl.tiny_decode(0)
    pool = build_pool(case)
    assert_close(_valu(pool, case), _oracle(case), "valu tiny")


def test_valu_layer_32k_matches_oracle_and_mfma():
    say("VALU stage 1: 32K context, 32 q / 4 KV heads")
    case = wl.layer_decode(0, with_new_token=False)
    pool = build_pool(case, "interleaved")
    ref = _oracle(case)
    got = _valu(pool, case)
    assert_close(got, ref, "valu 32K")
    assert_close(_mfma(pool, case), ref, "mfma 32K")
    assert np.abs(got - _mfma(pool, case)).max() <= 2e-2


@pytest.mark.parametrize("G,Hkv", [(1, 8), (2, 4), (4, 4), (8, 4), (16, 2)])
def test_valu_gqa_ratios(G, Hkv):
    say(f"VALU stage 1: GQA {G}, {Hkv} KV heads, 3,001 keys, split caps auto and 2")
    case = wl.layer_decode(4, ctx=3001, pool_rows=4000, n_q_heads=G * Hkv, n_kv_heads=Hkv, with_new_token=False)
    pool = build_pool(case)
    ref = _oracle(case)
    assert_close(_valu(pool, case), ref, f"valu G={G}")
    assert_close(_valu(pool, case, max_splits=2), ref, f"valu G={G} cap 2")


@pytest.mark.parametrize("L", [1, 63, 64, 65, 513, 4097])
def test_valu_ragged_lengths(L):
    say(f"VALU stage 1: L={L}")
    case = wl.layer_decode(2, ctx=max(L, 1), pool_rows=5000, with_new_token=False)
    pool = build_pool(case)
    lens = np.array([L], np.int32)
    assert_close(_valu(pool, case, seq_lens=lens, max_seq_len=L), _oracle(case, seq_lens=lens), f"valu L={L}")


def test_valu_batch_with_an_empty_request():
    say("VALU stage 1: 8 requests of 50..3000 keys, request 2 empty")
    case = wl.batched_decode(6, n_req=8, lo=50, hi=3000)
    lens = case.seq_lens.copy()
    lens[2] = 0
    pool = build_pool(case)
    got = _valu(pool, case, seq_lens=lens)
    assert np.all(got[2] == 0.0)
    keep = np.arange(8) != 2
    assert_close(got[keep], _oracle(case, seq_lens=lens)[keep], "valu batch")


def test_valu_rejects_other_formats_and_head_dims():
    case = wl.layer_decode(3, ctx=64, pool_rows=100, with_new_token=False)
    q, t, sl = to_dev_bf16(case.q), to_dev(case.table), to_dev(case.seq_lens)
    for kw in ({"code_format": "int8"},):
        pool = fk.Fp8KvPool(100, 4, device=DEV, **kw)
        with pytest.raises(B.Fp8KvError) as e:
            fk.binding.fp8kv_decode_stage1_valu(pool, q, t, sl, 64, case.sm_scale)
        assert e.value.status == 2
    c256 = wl.layer_decode(3, ctx=64, pool_rows=100, with_new_token=False, head_dim=256)
    pool = fk.Fp8KvPool(100, 4, device=DEV, head_dim=256)
    with pytest.raises(B.Fp8KvError) as e:
        fk.binding.fp8kv_decode_stage1_valu(pool, to_dev_bf16(c256.q), t, sl, 64, c256.sm_scale)
    assert e.value.status == 2
