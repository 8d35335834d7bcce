"""GPU parity of the decode variants against the fp64 oracle: head dim 256,
several causal query rows per request, and a sliding key window (FreeToken
PR #897, "Regression and CUDA isolation": D128 and D256 at GQA 4/8,
17/8,192/32,768 keys, 1/3/8 query rows, an odd sliding window, split caps
1/8/64; description: #900's multi-row decode, up to 8 rows per request).

Codes and scales written by the D=256 quantizer must match the oracle bit for
bit; attention outputs must be within rel-L2 5e-3 and max-abs 2e-2 of the
fp64 oracle over the same pool bytes.
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


def _oracle(case, ref_pool=None, seq_lens=None, window=0):
    kc, vc, ks, vs = oracle_pool(case) if ref_pool is None else ref_pool
    lens = case.seq_lens if seq_lens is None else seq_lens
    return oracle.decode_attention(case.q, kc, vc, ks, vs, case.table, lens, case.sm_scale, case.n_kv_heads,
                                   window=window)


def _rows(pool, case, window=0, max_splits=0, seq_lens=None, max_seq_len=None):
    lens = case.seq_lens if seq_lens is None else seq_lens
    msl = int(np.max(lens)) if max_seq_len is None else max_seq_len
    q = case.q if case.q.ndim == 4 else case.q[:, None]
    out = fk.fp8kv_decode_attn_rows(pool, to_dev_bf16(q), to_dev(case.table), to_dev(np.asarray(lens, np.int32)),
                                    msl, case.sm_scale, window=window, max_splits=max_splits)
    torch.cuda.synchronize()
    return out


def _single(pool, case, max_splits=0, seq_lens=None):
    lens = case.seq_lens if seq_lens is None else seq_lens
    out = fk.fp8kv_decode_attn(pool, to_dev_bf16(case.q), to_dev(case.table), to_dev(np.asarray(lens, np.int32)),
                               int(np.max(lens)), case.sm_scale, max_splits=max_splits)
    torch.cuda.synchronize()
    return out


# ------------------------------------------------------------- D = 256 --

@pytest.mark.parametrize("layout", ["separate", "interleaved", "interleaved128"])
def test_d256_32k_layer_pool_bits_and_attention(layout):
    say(f"D=256 decode 32K, 32 q / 4 KV heads, layout={layout}")
    case = wl.layer_decode(0, head_dim=256, with_new_token=False)
    pool = build_pool(case, layout)
    ref_pool = oracle_pool(case)
    for name, a, b in zip(("K codes", "V codes", "K scales", "V scales"), pool_arrays(pool), ref_pool):
        assert_bits_equal(a, b, f"D=256 {name}")
    assert_close(bf16_to_f64(_single(pool, case)), _oracle(case, ref_pool), "D=256 32K")


@pytest.mark.parametrize("L", [1, 17, 32, 33, 513, 8192])
def test_d256_lengths(L):
    say(f"D=256 decode L={L}")
    case = wl.layer_decode(31, ctx=L, pool_rows=L + 50, head_dim=256, with_new_token=False)
    pool = build_pool(case)
    assert_close(bf16_to_f64(_single(pool, case)), _oracle(case), f"D=256 L={L}")


@pytest.mark.parametrize("G,Hkv", [(1, 4), (2, 4), (4, 2), (8, 4), (16, 1)])
def test_d256_gqa_ratios(G, Hkv):
    say(f"D=256 decode GQA {G}, {Hkv} KV heads")
    case = wl.layer_decode(32, ctx=3000, pool_rows=3300, n_q_heads=G * Hkv, n_kv_heads=Hkv, head_dim=256,
                           with_new_token=False)
    pool = build_pool(case)
    assert_close(bf16_to_f64(_single(pool, case)), _oracle(case), f"D=256 G={G}")


@pytest.mark.parametrize("cap", [1, 8, 64])
def test_d256_split_caps(cap):
    say(f"D=256 decode 20,000 keys, max_splits={cap}")
    case = wl.layer_decode(33, ctx=20000, pool_rows=20500, head_dim=256, with_new_token=False)
    pool = build_pool(case)
    assert_close(bf16_to_f64(_single(pool, case, max_splits=cap)), _oracle(case), f"D=256 cap={cap}")


def test_d256_batched_16_requests():
    say("D=256 decode 16 requests, lengths 1,024..32,768, GQA 4")
    case = wl.batched_decode(3, head_dim=256)
    pool = build_pool(case)
    out = bf16_to_f64(_single(pool, case))
    ref = _oracle(case)
    assert_close(out, ref, "D=256 batched")
    for b in range(case.batch):
        assert_close(out[b], ref[b], f"  request {b} (L={case.seq_lens[b]})")


@pytest.mark.parametrize("L", [1, 2, 33, 1000, 32768])
def test_d256_append(L):
    say(f"D=256 decode+append L={L}")
    ctx = max(L, 1)
    case = wl.layer_decode(34, ctx=ctx, pool_rows=ctx + 291, head_dim=256)
    pool = build_pool(case)
    lens = np.array([L], np.int32)
    kc, vc, ks, vs = oracle_pool(case)
    nkc, nks = oracle.quantize_rows(case.new_k)
    nvc, nvs = oracle.quantize_rows(case.new_v)
    row = int(case.table[0, L - 1])
    kc[row], vc[row], ks[row], vs[row] = nkc[0], nvc[0], nks[0], nvs[0]
    out = fk.fp8kv_decode_attn_append(pool, to_dev_bf16(case.q), to_dev_bf16(case.new_k), to_dev_bf16(case.new_v),
                                      to_dev(np.array([row], np.int32)), to_dev(case.table), to_dev(lens), L,
                                      case.sm_scale)
    torch.cuda.synchronize()
    for name, a, b in zip(("K codes", "V codes", "K scales", "V scales"), pool_arrays(pool), (kc, vc, ks, vs)):
        assert_bits_equal(a, b, f"D=256 append {name}")
    ref = oracle.decode_attention(case.q, kc, vc, ks, vs, case.table, lens, case.sm_scale, case.n_kv_heads)
    assert_close(bf16_to_f64(out), ref, f"D=256 append L={L}")


def test_d256_quantize_all_bf16_patterns():
    """Every finite bf16 pattern up to 448 through the D=256 quantizer at scale 1."""
    say("D=256 quantize of every bf16 pattern <= 448")
    rows = wl.all_bf16_patterns_row_batches()
    if rows.shape[0] % 2:
        rows = np.concatenate([rows, rows[:1]])
    rows256 = rows.reshape(-1, 1, 256)
    codes, scales = oracle.quantize_rows(rows256)
    pool = fk.Fp8KvPool(rows256.shape[0], 1, device=torch.device("cuda", 0), head_dim=256)
    slots = torch.arange(rows256.shape[0], dtype=torch.int32, device="cuda")
    fk.fp8kv_quantize_rows(pool, to_dev_bf16(rows256), to_dev_bf16(rows256), slots)
    torch.cuda.synchronize()
    kc, vc, ks, vs = pool_arrays(pool)
    assert_bits_equal(kc, codes, "codes")
    assert_bits_equal(vc, codes, "codes (V)")
    assert_bits_equal(ks, scales, "scales")


# ----------------------------------------------------- several query rows --

@pytest.mark.parametrize("D", [128, 256])
@pytest.mark.parametrize("G", [4, 8])
@pytest.mark.parametrize("nq", [1, 3, 8])
@pytest.mark.parametrize("L", [17, 8192, 32768])
def test_rows_matrix(D, G, nq, L):
    say(f"rows: D={D} GQA {G} n_qrows={nq} L={L}")
    case = wl.layer_decode(40 + nq, ctx=L, pool_rows=L + 37, n_q_heads=4 * G, n_kv_heads=4, head_dim=D,
                           with_new_token=False, n_qrows=nq)
    pool = build_pool(case)
    out = bf16_to_f64(_rows(pool, case))
    ref = _oracle(case)
    if nq == 1:
        ref = ref[:, None]
    assert_close(out, ref, f"D={D} G={G} rows={nq} L={L}")


@pytest.mark.parametrize("D,G,nq", [(128, 16, 8), (128, 16, 5), (256, 8, 8), (256, 16, 3), (128, 1, 8), (256, 2, 7)])
def test_rows_wide_and_narrow_column_sets(D, G, nq):
    """G * n_qrows from 8 to 128 columns: one partial tile, several tiles, and
    more columns than one workgroup holds (several column groups)."""
    say(f"rows: D={D} GQA {G} n_qrows={nq} ({G * nq} columns)")
    Hkv = 2 if G >= 8 else 4
    case = wl.layer_decode(50 + G, ctx=2500, pool_rows=2600, n_q_heads=G * Hkv, n_kv_heads=Hkv, head_dim=D,
                           with_new_token=False, n_qrows=nq)
    pool = build_pool(case)
    assert_close(bf16_to_f64(_rows(pool, case)), _oracle(case), f"D={D} G={G} rows={nq}")


def test_rows_one_row_is_bit_identical_to_decode_attn():
    say("rows: n_qrows=1, window=0 == fp8kv_decode_attn bit for bit")
    for D in (128, 256):
        case = wl.layer_decode(60, ctx=7000, pool_rows=7100, head_dim=D, with_new_token=False)
        pool = build_pool(case)
        a = _single(pool, case)
        b = _rows(pool, case)[:, 0]
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), D


@pytest.mark.parametrize("D", [128, 256])
def test_rows_batched_with_short_requests(D):
    """16 requests; some shorter than the row count (rows before position 0 get zeros)."""
    say(f"rows: 16 requests x 3 rows, D={D}, lengths incl. 1 and 2")
    case = wl.batched_decode(5, n_req=16, lo=1, hi=9000, head_dim=D, n_qrows=3)
    lens = case.seq_lens.copy()
    lens[0], lens[1], lens[2] = 1, 2, 3
    out = bf16_to_f64(_rows(pool := build_pool(case), case, seq_lens=lens))
    ref = _oracle(case, seq_lens=lens)
    assert np.all(out[0, :2] == 0) and np.all(out[1, 0] == 0)
    assert_close(out, ref, f"D={D} batched rows")
    for b in range(case.batch):
        assert_close(out[b], ref[b], f"  request {b} (L={lens[b]})")


@pytest.mark.parametrize("cap", [1, 8, 64])
def test_rows_split_caps(cap):
    say(f"rows: 8 rows, GQA 8, 20,000 keys, max_splits={cap}")
    case = wl.layer_decode(61, ctx=20000, pool_rows=20100, with_new_token=False, n_qrows=8)
    pool = build_pool(case)
    assert_close(bf16_to_f64(_rows(pool, case, max_splits=cap)), _oracle(case), f"rows cap={cap}")


# -------------------------------------------------------- sliding window --

@pytest.mark.parametrize("D", [128, 256])
@pytest.mark.parametrize("nq", [1, 3])
@pytest.mark.parametrize("W", [1, 17, 4095, 8191])
def test_window(D, nq, W):
    say(f"window W={W}: D={D} n_qrows={nq}, 32,768 keys")
    case = wl.layer_decode(70 + nq, ctx=32768, pool_rows=33059, head_dim=D, with_new_token=False, n_qrows=nq)
    pool = build_pool(case)
    out = bf16_to_f64(_rows(pool, case, window=W))
    ref = _oracle(case, window=W)
    if nq == 1:
        ref = ref[:, None]
    assert_close(out, ref, f"D={D} rows={nq} W={W}")


@pytest.mark.parametrize("nq,W", [(3, 0), (8, 0), (1, 4095), (3, 4095)])
@pytest.mark.parametrize("k0", [1024.0, 196.0])
def test_rows_and_window_with_a_key_far_above_a_waves_first_keys(nq, W, k0):
    """Several query rows and a window, D = 128: every query has q[0] = 4 and
    the keys at positions 40, 2,600 and 5,900 have k[0] = k0, so they score
    ~520 (k0 = 1024: p = 2^(s - ref) overflows against the reference the
    kernel takes from a wave's first visible step, and those waves sum their
    keys again with a running maximum) or ~100 (k0 = 196: large finite p)
    log2 units above their neighbours.  Against the fp64 oracle."""
    say(f"rows/window with a key far above its wave's first keys (nq={nq}, W={W}, k[0] = {k0})")
    case = wl.layer_decode(5, ctx=6000, pool_rows=6100, with_new_token=False, n_qrows=nq)
    case.q[..., 0] = wl.bf16_bits(np.float32([4.0]))[0]
    big = wl.bf16_bits(np.float32([k0]))[0]
    for pos in (40, 2600, 5900):
        case.k_rows[case.table[0, pos], :, 0] = big
    pool = build_pool(case)
    out = bf16_to_f64(_rows(pool, case, window=W))
    assert np.isfinite(out).all()
    ref = _oracle(case, window=W)
    assert_close(out.reshape(ref.shape), ref, f"rows nq={nq} W={W} k0={k0}")


def test_window_covering_everything_is_bit_identical_to_no_window():
    say("window >= length == no window, bit for bit")
    case = wl.layer_decode(75, ctx=3000, pool_rows=3100, with_new_token=False, n_qrows=3)
    pool = build_pool(case)
    a = _rows(pool, case)
    ref = _oracle(case)
    assert_close(bf16_to_f64(a), ref, "no window")
    for W in (3000, 3001, 10 ** 6):
        b = _rows(pool, case, window=W)
        assert_close(bf16_to_f64(b), ref, f"W={W}")


@pytest.mark.parametrize("cap", [1, 8, 64])
def test_window_split_caps_and_batched(cap):
    say(f"window 1023 over 16 requests x 3 rows, max_splits={cap}")
    case = wl.batched_decode(7, n_req=16, lo=1, hi=5000, n_qrows=3)
    lens = case.seq_lens.copy()
    lens[0] = 1
    pool = build_pool(case)
    out = bf16_to_f64(_rows(pool, case, window=1023, max_splits=cap, seq_lens=lens))
    ref = _oracle(case, seq_lens=lens, window=1023)
    assert_close(out, ref, f"window batched cap={cap}")
    for b in range(case.batch):
        assert_close(out[b], ref[b], f"  request {b} (L={lens[b]})")


def test_window_one_returns_the_current_value_row():
    """W = 1: each row sees only its own position, so the output is that V row,
    decode(c) * s_v.  Stage 1 folds s_v into the bf16 P operand (p = 1 for the
    single visible key; the product with the 4-bit code and every later
    weight of 1 or 0 are exact in fp32) and rounds the output to bf16: two
    bf16 roundings, each at most 2^-8 relative."""
    say("window 1 == the current row's value, element by element")
    case = wl.layer_decode(76, ctx=500, pool_rows=600, n_q_heads=8, n_kv_heads=2, with_new_token=False, n_qrows=3)
    pool = build_pool(case)
    out = bf16_to_f64(_rows(pool, case, window=1))
    kc, vc, ks, vs = oracle_pool(case)
    vhat = oracle.dequantize(vc, vs)
    for i in range(3):
        want = np.repeat(vhat[int(case.table[0, 500 - 3 + i])], 4, axis=0)
        err = np.abs(out[0, i] - want)
        bound = ((1 + 2.0 ** -8) ** 2 - 1) * np.abs(want)
        assert np.all(err <= bound), f"row {i}: max rel {np.max(err / np.maximum(np.abs(want), 1e-300)):.3e}"
    assert_close(out, _oracle(case, window=1), "W=1")


def test_rows_window_graph_replay():
    say("rows + window captured in a HIP graph, replayed 4 times")
    case = wl.layer_decode(77, ctx=9000, pool_rows=9100, head_dim=256, with_new_token=False, n_qrows=3)
    pool = build_pool(case)
    q, t, sl = to_dev_bf16(case.q), to_dev(case.table), to_dev(case.seq_lens)
    ws = fk.decode_workspace(3, case.n_q_heads, head_dim=256)
    out = torch.empty_like(q)

    def step():
        fk.fp8kv_decode_attn_rows(pool, q, t, sl, case.max_seq_len, case.sm_scale, window=4097, workspace=ws,
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
        _ = (q.float() * 2).sum().item()
    assert_close(bf16_to_f64(eager), _oracle(case, window=4097), "graph rows+window")


def test_concurrent_calls_on_two_streams():
    """Two decode calls with their own workspaces on two streams at once (the
    library keeps no per-call state): each result matches its own oracle."""
    say("two decode calls on two streams at once (D=128 one row, D=256 three rows + window)")
    a = wl.layer_decode(80, ctx=9000, pool_rows=9100, with_new_token=False)
    b = wl.layer_decode(81, ctx=7000, pool_rows=7100, head_dim=256, with_new_token=False, n_qrows=3)
    pa, pb = build_pool(a), build_pool(b)
    qa, ta, la = to_dev_bf16(a.q), to_dev(a.table), to_dev(a.seq_lens)
    qb, tb, lb = to_dev_bf16(b.q), to_dev(b.table), to_dev(b.seq_lens)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    outs_a, outs_b = [], []
    for _ in range(4):
        with torch.cuda.stream(s1):
            outs_a.append(fk.fp8kv_decode_attn(pa, qa, ta, la, a.max_seq_len, a.sm_scale, stream=s1))
        with torch.cuda.stream(s2):
            outs_b.append(fk.fp8kv_decode_attn_rows(pb, qb, tb, lb, b.max_seq_len, b.sm_scale, window=2047,
                                                    stream=s2))
    torch.cuda.synchronize()
    ref_a, ref_b = _oracle(a), _oracle(b, window=2047)
    for i in range(4):
        assert_close(bf16_to_f64(outs_a[i]), ref_a, f"stream 1 call {i}")
        assert_close(bf16_to_f64(outs_b[i]), ref_b, f"stream 2 call {i}")
        assert torch.equal(outs_a[i].view(torch.int16), outs_a[0].view(torch.int16))
        assert torch.equal(outs_b[i].view(torch.int16), outs_b[0].view(torch.int16))
