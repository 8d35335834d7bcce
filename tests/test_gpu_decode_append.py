"""GPU parity: the decode step with the new token's quantize-on-write folded in
(fp8kv_decode_attn_append).

The call must leave the pool exactly as fp8kv_quantize_rows of the new tokens
would (codes and scales bit for bit, every other row untouched) and return
attention over all positions including the new token, within the attention
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


def _oracle_step(case, seq_lens=None):
    """Oracle pool with each request's new token quantized into its row, and
    the fp64 attention over it."""
    lens = case.seq_lens if seq_lens is None else seq_lens
    kc, vc, ks, vs = oracle_pool(case)
    nkc, nks = oracle.quantize_rows(case.new_k)
    nvc, nvs = oracle.quantize_rows(case.new_v)
    for b in range(case.batch):
        row = int(case.table[b, lens[b] - 1])
        kc[row], vc[row], ks[row], vs[row] = nkc[b], nvc[b], nks[b], nvs[b]
    out = oracle.decode_attention(case.q, kc, vc, ks, vs, case.table, lens, case.sm_scale, case.n_kv_heads)
    return (kc, vc, ks, vs), out


def _run_append(pool, case, seq_lens=None, max_seq_len=None, max_splits=0):
    lens = case.seq_lens if seq_lens is None else seq_lens
    msl = int(lens.max()) if max_seq_len is None else max_seq_len
    slots = np.array([case.table[b, lens[b] - 1] for b in range(case.batch)], np.int32)
    out = fk.fp8kv_decode_attn_append(pool, to_dev_bf16(case.q), to_dev_bf16(case.new_k), to_dev_bf16(case.new_v),
                                      to_dev(slots), to_dev(case.table), to_dev(np.asarray(lens, np.int32)), msl,
                                      case.sm_scale, max_splits=max_splits)
    torch.cuda.synchronize()
    return out


def _check_pool(pool, ref_pools, what):
    got = pool_arrays(pool)
    for name, a, b in zip(("K codes", "V codes", "K scales", "V scales"), got, ref_pools):
        assert_bits_equal(a, b, f"{what}: {name}")


@pytest.mark.parametrize("layout", ["separate", "interleaved", "interleaved128"])
def test_append_32k_layer(layout):
    say(f"decode+append 32K, 32 q / 4 KV heads, layout={layout}")
    case = wl.layer_decode(0)
    pool = build_pool(case, layout)
    ref_pools, ref = _oracle_step(case)
    out = bf16_to_f64(_run_append(pool, case))
    _check_pool(pool, ref_pools, "32K")
    assert_close(out, ref, "32K append")


def test_append_agrees_with_quantize_then_decode():
    say("decode+append == quantize_rows then decode_attn (pool bit-exact, outputs within rounding)")
    case = wl.layer_decode(3, ctx=6000, pool_rows=7000)
    pool_a = build_pool(case)
    pool_b = build_pool(case)
    out_a = bf16_to_f64(_run_append(pool_a, case))
    slot = to_dev(case.table[:, -1].copy())
    fk.fp8kv_quantize_rows(pool_b, to_dev_bf16(case.new_k), to_dev_bf16(case.new_v), slot)
    out_b = bf16_to_f64(fk.fp8kv_decode_attn(pool_b, to_dev_bf16(case.q), to_dev(case.table), to_dev(case.seq_lens),
                                             case.max_seq_len, case.sm_scale))
    torch.cuda.synchronize()
    for a, b, name in zip(pool_arrays(pool_a), pool_arrays(pool_b), ("kc", "vc", "ks", "vs")):
        assert_bits_equal(a, b, name)
    # Both are within the oracle tolerance; they differ only in fp32 summation
    # order of the new token's score.
    assert np.abs(out_a - out_b).max() <= 2e-2
    _, ref = _oracle_step(case)
    assert_close(out_a, ref, "append")
    assert_close(out_b, ref, "two calls")


@pytest.mark.parametrize("cap", [1, 3, 8, 64, 256])
def test_append_split_caps(cap):
    say(f"decode+append 20,000 context, max_splits={cap}")
    case = wl.layer_decode(9, ctx=20000, pool_rows=21000)
    pool = build_pool(case)
    ref_pools, ref = _oracle_step(case)
    out = bf16_to_f64(_run_append(pool, case, max_splits=cap))
    _check_pool(pool, ref_pools, f"cap={cap}")
    assert_close(out, ref, f"cap={cap}")


@pytest.mark.parametrize("L", [1, 2, 31, 32, 33, 64, 65, 129, 1000])
def test_append_lengths(L):
    say(f"decode+append L={L}")
    case = wl.layer_decode(4, ctx=max(L, 1), pool_rows=2000)
    pool = build_pool(case)
    lens = np.array([L], np.int32)
    ref_pools, ref = _oracle_step(case, lens)
    out = _run_append(pool, case, seq_lens=lens, max_seq_len=L)
    _check_pool(pool, ref_pools, f"L={L}")
    got = bf16_to_f64(out)
    assert_close(got, ref, f"L={L}")
    if L == 1:
        # A single key: every query head of group g returns that key's V row,
        # dequantized as the prefill reconstruction does it (bf16 of fl32(c*s)).
        row = int(case.table[0, 0])
        v_ws = oracle.reconstruct(ref_pools[1], ref_pools[3], np.array([row], np.int32), case.n_kv_heads)[0]
        G = case.n_q_heads // case.n_kv_heads
        want = np.repeat(v_ws, G, axis=0)
        assert_bits_equal(out.view(torch.int16).cpu().numpy()[0].view(np.uint16), want, "L=1 output")


@pytest.mark.parametrize("G,Hkv", [(1, 4), (2, 4), (4, 2), (8, 1), (16, 2)])
def test_append_gqa_ratios(G, Hkv):
    say(f"decode+append GQA {G}, {Hkv} KV heads")
    case = wl.layer_decode(5, ctx=3000, pool_rows=3500, n_q_heads=G * Hkv, n_kv_heads=Hkv)
    pool = build_pool(case)
    ref_pools, ref = _oracle_step(case)
    out = bf16_to_f64(_run_append(pool, case))
    _check_pool(pool, ref_pools, f"G={G}")
    assert_close(out, ref, f"G={G} Hkv={Hkv}")


def test_append_batched_16_requests():
    say("decode+append 16 requests, lengths 1,024..32,768, GQA 4")
    case = wl.batched_decode(0, with_new_token=True)
    pool = build_pool(case)
    ref_pools, ref = _oracle_step(case)
    for cap in (0, 8, 13):
        if cap:
            pool = build_pool(case)
        out = bf16_to_f64(_run_append(pool, case, max_splits=cap))
        _check_pool(pool, ref_pools, f"batched cap={cap}")
        assert_close(out, ref, f"batched cap={cap}")
        for b in range(case.batch):
            assert_close(out[b], ref[b], f"  request {b} (L={case.seq_lens[b]})")


def test_append_graph_replay():
    say("decode+append captured in a HIP graph, replayed 4 times")
    case = wl.layer_decode(6, ctx=8192, pool_rows=9000)
    pool = build_pool(case)
    q, nk, nv = to_dev_bf16(case.q), to_dev_bf16(case.new_k), to_dev_bf16(case.new_v)
    t, sl = to_dev(case.table), to_dev(case.seq_lens)
    ws = fk.decode_workspace(1, case.n_q_heads)
    out = torch.empty_like(q)
    slot = to_dev(case.table[:, -1].copy())

    def step():
        fk.fp8kv_decode_attn_append(pool, q, nk, nv, slot, t, sl, case.max_seq_len, case.sm_scale, workspace=ws,
                                    out=out)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    eager = out.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for i in range(4):
        out.fill_(0)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), f"replay {i} differs"
        _ = (q.float() * 2).sum().item()  # unrelated eager work between replays
    ref_pools, ref = _oracle_step(case)
    _check_pool(pool, ref_pools, "graph")
    assert_close(bf16_to_f64(eager), ref, "graph")


def _run_append_window(pool, case, window, max_splits=0):
    lens = case.seq_lens
    slots = np.array([case.table[b, lens[b] - 1] for b in range(case.batch)], np.int32)
    out = fk.fp8kv_decode_attn_append(pool, to_dev_bf16(case.q), to_dev_bf16(case.new_k), to_dev_bf16(case.new_v),
                                      to_dev(slots), to_dev(case.table), to_dev(np.asarray(lens, np.int32)),
                                      int(lens.max()), case.sm_scale, max_splits=max_splits, window=window)
    torch.cuda.synchronize()
    return out


def _oracle_step_window(case, window, fmt="e4m3"):
    kc, vc, ks, vs = oracle_pool(case, fmt)
    nkc, nks = oracle.quantize_rows(case.new_k, fmt)
    nvc, nvs = oracle.quantize_rows(case.new_v, fmt)
    for b in range(case.batch):
        row = int(case.table[b, case.seq_lens[b] - 1])
        kc[row], vc[row], ks[row], vs[row] = nkc[b], nvc[b], nks[b], nvs[b]
    out = oracle.decode_attention(case.q, kc, vc, ks, vs, case.table, case.seq_lens, case.sm_scale,
                                  case.n_kv_heads, window=window, fmt=fmt)
    return (kc, vc, ks, vs), out


@pytest.mark.parametrize("W,L,D", [(1, 100, 128), (17, 1, 128), (17, 5000, 128), (4095, 32768, 128),
                                   (4095, 3000, 128), (255, 20000, 256)])
def test_append_window(W, L, D):
    """The fused step with a sliding window: the pool ends up exactly as with
    fp8kv_quantize_rows of the new token, and the new token (position L - 1)
    attends to positions L - W .. L - 1 (W = 1: only itself)."""
    say(f"decode+append with window {W}, {L} keys, D={D}")
    case = wl.layer_decode(80 + W % 7, ctx=L, pool_rows=L + 59, head_dim=D)
    pool = build_pool(case)
    ref_pools, ref = _oracle_step_window(case, W)
    out = bf16_to_f64(_run_append_window(pool, case, W))
    _check_pool(pool, ref_pools, f"window {W}")
    assert_close(out, ref, f"window {W} L={L}")


@pytest.mark.parametrize("cap", [0, 3, 8])
def test_append_window_batched(cap):
    say(f"decode+append with window 1,023, 16 requests, max_splits={cap}")
    case = wl.batched_decode(81, n_req=16, lo=1, hi=6000, with_new_token=True)
    pool = build_pool(case)
    ref_pools, ref = _oracle_step_window(case, 1023)
    out = bf16_to_f64(_run_append_window(pool, case, 1023, max_splits=cap))
    _check_pool(pool, ref_pools, f"window batched cap={cap}")
    assert_close(out, ref, f"window batched cap={cap}")


def test_append_window_covering_everything_is_the_plain_append():
    """A window of at least the request length masks nothing: the windowed
    stage 1 and merge give the plain fused step's output bit for bit."""
    say("decode+append: a window covering every position == no window (bit-exact)")
    case = wl.layer_decode(82, ctx=3000, pool_rows=3100)
    pool_a = build_pool(case)
    pool_b = build_pool(case)
    a = _run_append(pool_a, case)
    b = _run_append_window(pool_b, case, 3001)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    for x, y in zip(pool_arrays(pool_a), pool_arrays(pool_b)):
        assert_bits_equal(x, y, "pool")


@pytest.mark.parametrize("D", [128, 256])
def test_append_window_int8_pool(D):
    say(f"decode+append with window 255 over an INT8 pool, D={D}")
    case = wl.layer_decode(83, ctx=12000, pool_rows=12100, head_dim=D)
    pool = build_pool(case, fmt="int8")
    ref_pools, ref = _oracle_step_window(case, 255, fmt="int8")
    out = bf16_to_f64(_run_append_window(pool, case, 255))
    _check_pool(pool, ref_pools, f"int8 window D={D}")
    assert_close(out, ref, f"int8 window D={D}")


@pytest.mark.parametrize("kind,new_k0,cached_k0", [
    ("layer", 1024.0, None), ("layer", -1024.0, None), ("layer", 1024.0, 1024.0),
    ("batch6", 1024.0, None), ("batch6", -1024.0, None), ("batch6", 1024.0, 1024.0),
    ("batch16", 1024.0, 1024.0)])
def test_append_with_keys_far_apart(kind, new_k0, cached_k0):
    """Every query has q[0] = 4; the new token's K has k[0] = new_k0 in every KV
    head (~520 log2 units above, or below, every cached key), and with
    cached_k0 the cached keys at positions 40 and 2,600 have k[0] = cached_k0
    (far above their wave's first keys: those waves sum their keys again with
    a running maximum).  The one-request layer and the 6-request batch run in
    one workgroup round, where stage 1 takes the new token and folds it into
    split 0's partial; the 16-request batch runs the streaming shape, where
    the merge takes it.  Pool bit-exact and output against the fp64 oracle,
    every request."""
    say(f"decode+append, keys far apart ({kind}, new k[0] = {new_k0}, cached k[0] = {cached_k0})")
    if kind == "layer":
        case = wl.layer_decode(4, ctx=6000, pool_rows=6100)
    elif kind == "batch6":
        case = wl.batched_decode(5, n_req=6, lo=1024, hi=6000, with_new_token=True)
    else:
        case = wl.batched_decode(6, with_new_token=True)
    case.q[..., 0] = wl.bf16_bits(np.float32([4.0]))[0]
    case.new_k[:, :, 0] = wl.bf16_bits(np.float32([new_k0]))[0]
    if cached_k0 is not None:
        big = wl.bf16_bits(np.float32([cached_k0]))[0]
        for b in range(case.batch):
            for pos in (40, 2600):
                if pos < case.seq_lens[b] - 1:
                    case.k_rows[case.table[b, pos], :, 0] = big
    pool = build_pool(case)
    ref_pools, ref = _oracle_step(case)
    out = bf16_to_f64(_run_append(pool, case))
    assert np.isfinite(out).all()
    _check_pool(pool, ref_pools, kind)
    for b in range(case.batch):
        assert_close(out[b], ref[b], f"{kind} request {b} (L={case.seq_lens[b]})")
