"""GPU parity: several new tokens per request written and attended in one call
(fp8kv_decode_attn_rows_append).

Request b's last n_qrows positions are new tokens: the call must leave the pool
exactly as fp8kv_quantize_rows of those tokens would (codes and scales bit for
bit, every other row untouched), and query row j must attend causally, and
within the window, over positions up to its own -- within the attention
tolerance of the fp64 oracle run on the oracle-quantized pool.
"""
import numpy as np
import pytest
import torch

import oracle
import fp8_kv_cache_row_amd as fk
from fp8_kv_cache_row_amd import workloads as wl

from gpu_common import (assert_bits_equal, assert_close, bf16_to_f64, build_pool, oracle_pool, pool_arrays, say,
                        to_dev, to_dev_bf16)

pytestmark = pytest.mark.gpu


def _new_tokens(case, nq, seed):
    """Fresh bf16 K/V for each request's last nq positions, and their rows."""
    rng = np.random.default_rng(seed)
    B, H, D = case.batch, case.n_kv_heads, case.head_dim
    k = wl.bf16_bits(wl.draw_normal(rng, (B, nq, H, D)))
    v = wl.bf16_bits(wl.draw_normal(rng, (B, nq, H, D), 0.5))
    slots = np.array([[case.table[b, case.seq_lens[b] - nq + j] for j in range(nq)] for b in range(B)], np.int32)
    return k, v, slots


def _oracle(case, k, v, slots, window, fmt="e4m3"):
    kc, vc, ks, vs = oracle_pool(case, fmt)
    nkc, nks = oracle.quantize_rows(k.reshape(-1, case.n_kv_heads, case.head_dim), fmt)
    nvc, nvs = oracle.quantize_rows(v.reshape(-1, case.n_kv_heads, case.head_dim), fmt)
    rows = slots.reshape(-1)
    kc[rows], vc[rows], ks[rows], vs[rows] = nkc, nvc, nks, nvs
    out = oracle.decode_attention(case.q, kc, vc, ks, vs, case.table, case.seq_lens, case.sm_scale,
                                  case.n_kv_heads, window=window, fmt=fmt)
    return (kc, vc, ks, vs), out


def _run(pool, case, k, v, slots, window, max_splits=0):
    out = fk.fp8kv_decode_attn_rows_append(pool, to_dev_bf16(case.q), to_dev_bf16(k), to_dev_bf16(v), to_dev(slots),
                                           to_dev(case.table), to_dev(case.seq_lens), case.max_seq_len,
                                           case.sm_scale, window=window, max_splits=max_splits)
    torch.cuda.synchronize()
    return bf16_to_f64(out)


def _check(pool, ref_pools, what):
    for name, a, b in zip(("K codes", "V codes", "K scales", "V scales"), pool_arrays(pool), ref_pools):
        assert_bits_equal(a, b, f"{what}: {name}")


@pytest.mark.parametrize("nq,D,Hq,Hkv,W,L", [
    (3, 128, 32, 4, 0, 5000), (8, 128, 32, 4, 0, 32768), (8, 128, 32, 4, 5, 2000), (3, 256, 32, 4, 0, 3000),
    (8, 256, 16, 4, 17, 4000), (2, 128, 32, 2, 17, 700), (8, 128, 8, 8, 0, 1000), (3, 128, 32, 4, 0, 3),
    (8, 128, 32, 4, 1, 900)])
def test_rows_append(nq, D, Hq, Hkv, W, L):
    say(f"rows+append: {nq} new tokens, D={D}, {Hq} q / {Hkv} KV heads, window {W}, {L} keys")
    case = wl.layer_decode(90 + nq + W, ctx=L, pool_rows=L + 41, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=D,
                           with_new_token=False, n_qrows=nq)
    k, v, slots = _new_tokens(case, nq, 7 + L)
    pool = build_pool(case)
    ref_pools, ref = _oracle(case, k, v, slots, W)
    got = _run(pool, case, k, v, slots, W)
    _check(pool, ref_pools, f"nq={nq} W={W}")
    assert_close(got, ref, f"nq={nq} D={D} W={W} L={L}")


@pytest.mark.parametrize("cap,W", [(0, 0), (3, 0), (8, 100), (0, 100)])
def test_rows_append_batched(cap, W):
    say(f"rows+append: 16 requests, 3 new tokens each, window {W}, max_splits={cap}")
    case = wl.batched_decode(91, n_req=16, lo=3, hi=6000, n_qrows=3)
    k, v, slots = _new_tokens(case, 3, 91)
    pool = build_pool(case)
    ref_pools, ref = _oracle(case, k, v, slots, W)
    got = _run(pool, case, k, v, slots, W, max_splits=cap)
    _check(pool, ref_pools, f"batched cap={cap} W={W}")
    assert_close(got, ref, f"batched cap={cap} W={W}")


@pytest.mark.parametrize("nq,D,W", [(8, 128, 0), (3, 256, 17), (8, 128, 5)])
def test_rows_append_int8_pool(nq, D, W):
    say(f"rows+append over an INT8 pool: {nq} new tokens, D={D}, window {W}, 9,000 keys")
    case = wl.layer_decode(93 + W, ctx=9000, pool_rows=9100, with_new_token=False, n_qrows=nq, head_dim=D)
    k, v, slots = _new_tokens(case, nq, 93 + W)
    pool = build_pool(case, fmt="int8")
    ref_pools, ref = _oracle(case, k, v, slots, W, fmt="int8")
    got = _run(pool, case, k, v, slots, W)
    _check(pool, ref_pools, f"int8 nq={nq} W={W}")
    assert_close(got, ref, f"int8 rows+append nq={nq} D={D} W={W}")


def test_rows_append_one_row_is_the_fused_step():
    """n_qrows = 1 is fp8kv_decode_attn_append bit for bit (same kernels)."""
    say("rows+append with one row == fp8kv_decode_attn_append (bit-exact)")
    case = wl.layer_decode(94, ctx=4000, pool_rows=4100)
    slot = np.array([case.table[0, case.seq_lens[0] - 1]], np.int32)
    pool_a, pool_b = build_pool(case), build_pool(case)
    a = fk.fp8kv_decode_attn_append(pool_a, to_dev_bf16(case.q), to_dev_bf16(case.new_k), to_dev_bf16(case.new_v),
                                    to_dev(slot), to_dev(case.table), to_dev(case.seq_lens), case.max_seq_len,
                                    case.sm_scale)
    b = fk.fp8kv_decode_attn_rows_append(pool_b, to_dev_bf16(case.q[:, None]), to_dev_bf16(case.new_k[:, None]),
                                         to_dev_bf16(case.new_v[:, None]), to_dev(slot.reshape(1, 1)),
                                         to_dev(case.table), to_dev(case.seq_lens), case.max_seq_len, case.sm_scale)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b[:, 0].view(torch.int16))
    for x, y in zip(pool_arrays(pool_a), pool_arrays(pool_b)):
        assert_bits_equal(x, y, "pool")


def test_rows_append_graph_replay():
    """Captured in a HIP graph and replayed three times, with eager work and
    synchronizations between the replays: every replay's output and pool are
    bit-identical to the eager call's (rewriting the same new tokens)."""
    say("rows+append captured in a graph, 3 replays vs eager")
    case = wl.layer_decode(95, ctx=6000, pool_rows=6100, with_new_token=False, n_qrows=3)
    k, v, slots = _new_tokens(case, 3, 95)
    pool = build_pool(case)
    dev = {"q": to_dev_bf16(case.q), "k": to_dev_bf16(k), "v": to_dev_bf16(v), "s": to_dev(slots),
           "t": to_dev(case.table), "l": to_dev(case.seq_lens)}
    ws = fk.decode_workspace(3, case.n_q_heads)
    out = torch.empty_like(dev["q"])
    stream = torch.cuda.Stream()

    def call():
        fk.fp8kv_decode_attn_rows_append(pool, dev["q"], dev["k"], dev["v"], dev["s"], dev["t"], dev["l"],
                                         case.max_seq_len, case.sm_scale, window=17, workspace=ws, out=out,
                                         stream=stream)

    with torch.cuda.stream(stream):
        call()
    stream.synchronize()
    ref_out = out.clone()
    ref_pool = pool_arrays(pool)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        call()
    for rep in range(3):
        out.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16)), f"replay {rep}"
        for a, b in zip(pool_arrays(pool), ref_pool):
            assert_bits_equal(a, b, f"replay {rep}: pool")
