"""GPU parity: split-K FP8 decode attention against the fp64 oracle.

Covers the tiny case, the 32K-context single layer, the 48-layer 40K step
(quantize-on-write per layer), the 16-request batch, ragged and degenerate
lengths, every supported GQA ratio, split caps 1/8/64/auto, row-permutation
invariance, the exact V path for every finite code, both pool layouts and
HIP-graph replay.
"""
import numpy as np
import pytest
import torch

import oracle
import fp8_kv_cache_row_amd as fk
from fp8_kv_cache_row_amd import workloads as wl

from gpu_common import (DEV, assert_bits_equal, assert_close, bf16_to_f64, build_pool, oracle_pool,
                        pool_arrays, run_decode, say, to_dev, to_dev_bf16)

pytestmark = pytest.mark.gpu
D = 128


def _oracle_decode(case, pools=None, q=None, table=None, seq_lens=None):
    kc, vc, ks, vs = pools if pools is not None else oracle_pool(case)
    return oracle.decode_attention(case.q if q is None else q, kc, vc, ks, vs,
                                   case.table if table is None else table,
                                   case.seq_lens if seq_lens is None else seq_lens,
                                   case.sm_scale, case.n_kv_heads)


@pytest.mark.parametrize("layout", ["separate", "interleaved", "interleaved128"])
def test_tiny_gqa8(layout):
    say(f"decode tiny GQA-8 256 rows, layout={layout}")
    case = wl.tiny_decode(0)
    pool = build_pool(case, layout)
    out = run_decode(pool, case)
    assert_close(bf16_to_f64(out), _oracle_decode(case), "tiny")


def test_layer_32k_all_split_caps():
    say("decode 32K context, 32 q / 4 KV heads, pool 33,059 rows")
    case = wl.layer_decode(0, with_new_token=False)
    pool = build_pool(case)
    ref_pools = oracle_pool(case)
    kc, vc, ks, vs = pool_arrays(pool)
    assert_bits_equal(kc, ref_pools[0], "K codes")
    assert_bits_equal(vc, ref_pools[1], "V codes")
    assert_bits_equal(ks, ref_pools[2], "K scales")
    assert_bits_equal(vs, ref_pools[3], "V scales")
    ref = _oracle_decode(case, ref_pools)
    outs = {}
    for cap in (0, 1, 8, 64):
        say(f"  max_splits={cap}")
        outs[cap] = bf16_to_f64(run_decode(pool, case, max_splits=cap))
        assert_close(outs[cap], ref, f"32K cap={cap}")
    for cap in (1, 8, 64):
        assert np.abs(outs[cap] - outs[0]).max() <= 2e-2


def test_layer_32k_interleaved_pool_matches_separate():
    say("decode 32K, interleaved pool layout")
    case = wl.layer_decode(1, with_new_token=False)
    pool = build_pool(case, "interleaved")
    assert_close(bf16_to_f64(run_decode(pool, case)), _oracle_decode(case), "32K interleaved")


def test_streaming_and_plain_code_loads_agree_bit_for_bit():
    """Pools whose KV heads' code rows fill whole 128-byte lines (separate
    arrays, records padded to 128 bytes) are read with non-temporal loads, the
    1,056-byte records with plain ones; the arithmetic is the same, so the
    outputs are identical, and both match the oracle."""
    say("decode 32K: separate / interleaved128 (non-temporal loads) vs interleaved (plain loads)")
    case = wl.layer_decode(3, with_new_token=False)
    outs = {}
    for layout in ("separate", "interleaved128", "interleaved"):
        pool = build_pool(case, layout)
        outs[layout] = run_decode(pool, case).cpu()
        del pool
        torch.cuda.empty_cache()
    assert torch.equal(outs["separate"].view(torch.int16), outs["interleaved"].view(torch.int16))
    assert torch.equal(outs["interleaved128"].view(torch.int16), outs["interleaved"].view(torch.int16))
    assert_close(bf16_to_f64(outs["interleaved128"]), _oracle_decode(case), "32K interleaved128")


@pytest.mark.parametrize("L", [0, 1, 2, 17, 31, 32, 33, 127, 129, 513, 1000, 4097])
def test_ragged_lengths(L):
    say(f"decode L={L}")
    case = wl.layer_decode(2, ctx=max(L, 1), pool_rows=5000, n_q_heads=32, n_kv_heads=4, with_new_token=False)
    pool = build_pool(case)
    lens = np.array([L], np.int32)
    out = bf16_to_f64(run_decode(pool, case, seq_lens=lens, max_seq_len=L))
    if L == 0:
        assert np.all(out == 0.0)
        return
    ref = _oracle_decode(case, seq_lens=lens)
    assert_close(out, ref, f"L={L}")


def test_single_row_returns_that_row():
    say("decode L=1 returns the dequantized V row")
    case = wl.layer_decode(3, ctx=1, pool_rows=100, with_new_token=False)
    pool = build_pool(case)
    out = bf16_to_f64(run_decode(pool, case))
    kc, vc, ks, vs = oracle_pool(case)
    row = case.table[0, 0]
    vhat = oracle.dequantize(vc, vs)[row]  # [Hkv][D]
    expect = np.repeat(vhat, 8, axis=0)[None]
    # the only roundings are p * v_scale to bf16 (p = 1) and the bf16 output
    assert np.all(np.abs(out - expect) <= np.abs(expect) * 2.0 ** -7 + 1e-30)
    assert_close(out, expect, "L=1")


def test_every_finite_code_through_the_v_path():
    """One row, unit V scale: the output is decode(code) exactly (rounded to bf16, which is exact)."""
    say("decode: all 254 finite codes through the V path")
    R, H = 4, 2
    pool = fk.Fp8KvPool(R, H, device=DEV)
    codes = np.arange(256, dtype=np.uint8).reshape(2, 128)
    codes[(codes & 0x7F) == 0x7F] = 0x00
    vc = np.zeros((R, H, D), np.uint8)
    vc[1, 0] = codes[0]
    vc[1, 1] = codes[1]
    pool.v_codes.copy_(to_dev(vc))
    pool.k_codes.fill_(0x38)
    pool.k_scales.fill_(0.5)
    pool.v_scales.fill_(1.0)
    q = wl.bf16_bits(np.random.default_rng(0).standard_normal((1, 4, D)).astype(np.float32))
    out = fk.fp8kv_decode_attn(pool, to_dev_bf16(q), to_dev(np.array([[1]], np.int32)),
                               to_dev(np.array([1], np.int32)), 1, 0.0883883)
    torch.cuda.synchronize()
    got = bf16_to_f64(out)[0]
    dec = oracle.e4m3_decode_table()[codes]
    assert np.array_equal(got[0], dec[0]) and np.array_equal(got[1], dec[0])
    assert np.array_equal(got[2], dec[1]) and np.array_equal(got[3], dec[1])


@pytest.mark.parametrize("G,Hkv", [(1, 8), (2, 4), (4, 4), (8, 4), (16, 2)])
def test_gqa_ratios(G, Hkv):
    say(f"decode GQA ratio {G} with {Hkv} KV heads")
    case = wl.layer_decode(4, ctx=3001, pool_rows=4000, n_q_heads=G * Hkv, n_kv_heads=Hkv, with_new_token=False)
    pool = build_pool(case)
    ref = _oracle_decode(case)
    assert_close(bf16_to_f64(run_decode(pool, case)), ref, f"G={G}")
    # a cap of 2 splits gives 1,504-key splits: the streaming stage-1 shape
    assert_close(bf16_to_f64(run_decode(pool, case, max_splits=2)), ref, f"G={G} streaming")


def test_long_context_at_the_split_cap():
    """131,072 keys of one request: 256 splits of 512 keys (FP8KV_MAX_SPLITS),
    the streaming stage-1 shape, and a merge folding 256 partials per head in
    four load batches."""
    say("decode 131,072 keys, 32 q / 4 KV heads: 256 splits, streaming stage 1")
    case = wl.layer_decode(12, ctx=131072, pool_rows=131072 + 300)
    pool = build_pool(case)
    ref_pools = oracle_pool(case)
    lens = case.seq_lens - 1  # 131,071 keys: the last split is one key short
    ref = _oracle_decode(case, ref_pools, seq_lens=lens)
    out = run_decode(pool, case, seq_lens=lens)
    assert_close(bf16_to_f64(out), ref, "131,071 keys")
    ws = fk.fp8kv_decode_stage1(pool, to_dev_bf16(case.q), to_dev(case.table), to_dev(case.seq_lens),
                                case.max_seq_len, case.sm_scale)
    torch.cuda.synchronize()
    assert int(ws[:4].view(torch.int32).item()) == 256, "split count"


def test_row_permutation_invariance():
    say("decode: permuting the physical rows (and the table) leaves the output unchanged")
    case = wl.layer_decode(5, ctx=2000, pool_rows=2500, with_new_token=False)
    pool = build_pool(case)
    base = bf16_to_f64(run_decode(pool, case))
    perm = np.random.default_rng(9).permutation(case.pool_rows)
    inv = np.argsort(perm)
    case2 = wl.DecodeCase(case.name, case.n_q_heads, case.n_kv_heads, case.pool_rows, case.k_rows[perm],
                          case.v_rows[perm], case.q, inv[case.table].astype(np.int32), case.seq_lens,
                          case.sm_scale)
    pool2 = build_pool(case2)
    out2 = bf16_to_f64(run_decode(pool2, case2))
    assert np.abs(out2 - base).max() <= 1e-2
    assert_close(out2, _oracle_decode(case), "permuted")


def test_batched_16_requests_gqa4():
    say("decode 16 requests, lengths 1,024..32,768, GQA 4")
    case = wl.batched_decode(0)
    assert int(case.seq_lens.sum()) == 272568
    pool = build_pool(case)
    ref = _oracle_decode(case)
    # caps 3 and 13 leave a partial row of 8 splits in the grid (the extra
    # workgroups redo the last split and store nothing)
    for cap in (0, 8, 3, 13):
        out = bf16_to_f64(run_decode(pool, case, max_splits=cap))
        assert_close(out, ref, f"batched cap={cap}")
        for b in range(case.batch):
            assert_close(out[b], ref[b], f"  request {b} (L={case.seq_lens[b]})")


def test_batched_16_requests_every_pool_layout():
    """The batch runs the streaming stage-1 shape, which reads whole 128-byte
    key lines and trades halves between lanes: with non-temporal loads where
    every KV head's rows fill whole lines (the 1,152-byte records, the split
    code record, the separate arrays) and plain loads otherwise (the unpadded
    1,056-byte and the 1,088-byte records).  Every layout against the oracle."""
    case = wl.batched_decode(0)
    ref = _oracle_decode(case)
    for layout in ("interleaved128", "interleaved", "interleaved64", "split"):
        say(f"decode 16 requests, GQA 4, layout={layout}")
        pool = build_pool(case, layout)
        out = bf16_to_f64(run_decode(pool, case))
        assert_close(out, ref, f"batched layout={layout}")
        for b in range(case.batch):
            assert_close(out[b], ref[b], f"  {layout} request {b} (L={case.seq_lens[b]})")
        del pool


@pytest.mark.parametrize("kind", ["layer", "batch", "layer_one_split"])
@pytest.mark.parametrize("k0", [1024.0, 196.0])
@pytest.mark.parametrize("fmt", ["e4m3", "int8"])
def test_key_far_above_a_waves_first_keys(kind, k0, fmt):
    """Every query has q[0] = 4 and a few keys have k[0] = k0, each placed in
    the second 32-key step of a wave (positions 40 and 2,600 of every request
    long enough), so it scores ~4 k0 / sqrt(128) log2 e above the keys of the
    wave's first step, the kernel's softmax reference: ~520 log2 units for
    k0 = 1024, where p = 2^(s - ref) overflows and those waves must sum their
    keys again with a running maximum; ~100 for k0 = 196, a large but finite
    p on the fixed reference.  The one-layer case runs the 8-wave shape (with
    one split, a wave covers a dozen groups and its second pass re-reads every
    group's rows), the batch the streaming one; against the fp64 oracle,
    every request."""
    say(f"decode with a key far above its wave's first keys ({kind}, k[0] = {k0}, {fmt})")
    if kind.startswith("layer"):
        case = wl.layer_decode(4, ctx=6000, pool_rows=6100, with_new_token=False)
    else:
        case = wl.batched_decode(4, n_req=6, lo=1024, hi=6000)
    case.q[..., 0] = wl.bf16_bits(np.float32([4.0]))[0]
    big = wl.bf16_bits(np.float32([k0]))[0]
    for b in range(case.batch):
        for pos in (40, 2600):
            if pos < case.seq_lens[b]:
                case.k_rows[case.table[b, pos], :, 0] = big
    pool = build_pool(case, fmt=fmt)
    kc, vc, ks, vs = oracle_pool(case, fmt)
    ref = oracle.decode_attention(case.q, kc, vc, ks, vs, case.table, case.seq_lens, case.sm_scale,
                                  case.n_kv_heads, fmt=fmt)
    out = bf16_to_f64(run_decode(pool, case, max_splits=1 if kind == "layer_one_split" else 0))
    assert np.isfinite(out).all()
    for b in range(case.batch):
        assert_close(out[b], ref[b], f"{kind} request {b} (L={case.seq_lens[b]})")


def test_model_step_48_layers_40k():
    """48 layers x (quantize the new token's K/V into slot table[39999], then
    decode over 40,000 rows); the pool holds 40,290 rows per layer."""
    say("decode 48-layer step at 40,000 context (2.04 GB pool)")
    table = wl.model_step_table(0)
    t_dev = to_dev(table)
    lens = to_dev(np.array([table.shape[1]], np.int32))
    new_slot = to_dev(table[:, -1].copy())
    check_layers = {0, 23, 47}
    outs = {}
    for layer in range(48):
        case = wl.model_step_layer(layer, table)
        pool = build_pool(case)
        fk.fp8kv_quantize_rows(pool, to_dev_bf16(case.new_k), to_dev_bf16(case.new_v), new_slot)
        out = fk.fp8kv_decode_attn(pool, to_dev_bf16(case.q), t_dev, lens, table.shape[1], case.sm_scale)
        torch.cuda.synchronize()
        kc, vc, ks, vs = pool_arrays(pool)
        nkc, nks = oracle.quantize_rows(case.new_k)
        nvc, nvs = oracle.quantize_rows(case.new_v)
        row = int(table[0, -1])
        assert_bits_equal(kc[row], nkc[0], f"layer {layer} new K codes")
        assert_bits_equal(vc[row], nvc[0], f"layer {layer} new V codes")
        assert_bits_equal(ks[row], nks[0], f"layer {layer} new K scales")
        assert_bits_equal(vs[row], nvs[0], f"layer {layer} new V scales")
        if layer in check_layers:
            okc, ovc, oks, ovs = oracle_pool(case)
            okc[row], ovc[row], oks[row], ovs[row] = nkc[0], nvc[0], nks[0], nvs[0]
            assert_bits_equal(kc, okc, f"layer {layer} K codes")
            assert_bits_equal(vs, ovs, f"layer {layer} V scales")
            outs[layer] = (bf16_to_f64(out), _oracle_decode(case, (okc, ovc, oks, ovs)))
        del pool
    for layer, (got, ref) in outs.items():
        assert_close(got, ref, f"layer {layer}")


def test_graph_replay_matches_eager():
    say("decode + quantize captured in a HIP graph, replayed 5 times")
    case = wl.layer_decode(6, ctx=8192, pool_rows=9000)
    pool = build_pool(case)
    q = to_dev_bf16(case.q)
    t = to_dev(case.table)
    sl = to_dev(case.seq_lens)
    nk, nv = to_dev_bf16(case.new_k), to_dev_bf16(case.new_v)
    slot = to_dev(case.table[:, -1].copy())
    ws = fk.decode_workspace(1, case.n_q_heads)
    out = torch.empty_like(q)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fk.fp8kv_quantize_rows(pool, nk, nv, slot)
        fk.fp8kv_decode_attn(pool, q, t, sl, case.max_seq_len, case.sm_scale, workspace=ws, out=out)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    eager = out.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fk.fp8kv_quantize_rows(pool, nk, nv, slot)
        fk.fp8kv_decode_attn(pool, q, t, sl, case.max_seq_len, case.sm_scale, workspace=ws, out=out)
    for i in range(5):
        out.fill_(0)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), f"replay {i} differs"
        _ = (q.float() * 2).sum().item()  # unrelated eager work between replays
    ref = oracle_pool(case)
    kc, vc, ks, vs = ref
    row = int(case.table[0, -1])
    nkc, nks = oracle.quantize_rows(case.new_k)
    nvc, nvs = oracle.quantize_rows(case.new_v)
    kc[row], vc[row], ks[row], vs[row] = nkc[0], nvc[0], nks[0], nvs[0]
    assert_close(bf16_to_f64(eager), _oracle_decode(case, (kc, vc, ks, vs)), "graph")


def test_output_guard_bands_untouched():
    say("decode writes only its output rows")
    case = wl.layer_decode(7, ctx=777, pool_rows=1000, with_new_token=False)
    pool = build_pool(case)
    n = case.q.size
    buf = torch.full((n + 2 * 64,), -3.0, dtype=torch.bfloat16, device=DEV)
    out = buf[64:64 + n].view(case.q.shape)
    fk.fp8kv_decode_attn(pool, to_dev_bf16(case.q), to_dev(case.table), to_dev(case.seq_lens), case.max_seq_len,
                         case.sm_scale, out=out)
    torch.cuda.synchronize()
    assert torch.all(buf[:64] == -3.0) and torch.all(buf[64 + n:] == -3.0)
    assert_close(bf16_to_f64(out), _oracle_decode(case), "guarded")


def test_stage1_then_merge_equals_full_call():
    say("decode: stage 1 + merge as separate calls == fp8kv_decode_attn (bit-exact)")
    case = wl.layer_decode(8, ctx=5000, pool_rows=6000, with_new_token=False)
    pool = build_pool(case)
    q, t, sl = to_dev_bf16(case.q), to_dev(case.table), to_dev(case.seq_lens)
    for cap in (0, 3, 64):
        full = fk.fp8kv_decode_attn(pool, q, t, sl, case.max_seq_len, case.sm_scale, max_splits=cap)
        ws = fk.fp8kv_decode_stage1(pool, q, t, sl, case.max_seq_len, case.sm_scale, max_splits=cap)
        two = fk.fp8kv_decode_merge(ws, 1, case.n_q_heads, max_splits=cap)
        torch.cuda.synchronize()
        assert torch.equal(full.view(torch.int16), two.view(torch.int16)), cap


def test_stage1_then_merge_streaming_with_an_empty_first_request():
    """Splits of more than 1,024 keys take the streaming stage-1 shape, where a
    split past its request's length stores an empty partial and leaves early;
    with request 0 empty, split 0 of request 0 is such a split and must still
    write the split count that a separately launched merge reads from the
    workspace (pre-filled with garbage here)."""
    say("decode: streaming stage 1 + merge with request 0 empty, garbage-filled workspace")
    case = wl.batched_decode(11, n_req=6, lo=3000, hi=9000)
    lens = case.seq_lens.copy()
    lens[0] = 0
    pool = build_pool(case)
    ref = _oracle_decode(case, seq_lens=lens)
    q, t, sl = to_dev_bf16(case.q), to_dev(case.table), to_dev(lens)
    for cap in (2, 5):
        ws = fk.decode_workspace(case.batch, case.n_q_heads, max_splits=cap)
        ws.fill_(0x7F)
        fk.fp8kv_decode_stage1(pool, q, t, sl, case.max_seq_len, case.sm_scale, max_splits=cap, workspace=ws)
        two = fk.fp8kv_decode_merge(ws, case.batch, case.n_q_heads, max_splits=cap)
        full = fk.fp8kv_decode_attn(pool, q, t, sl, case.max_seq_len, case.sm_scale, max_splits=cap)
        torch.cuda.synchronize()
        assert int(ws[:4].view(torch.int32).item()) == cap, "split count in the workspace header"
        assert torch.equal(full.view(torch.int16), two.view(torch.int16)), cap
        got = bf16_to_f64(two)
        assert np.all(got[0] == 0.0), "an empty request gets zeros"
        assert_close(got[1:], ref[1:], f"streaming cap={cap}")


def test_out_of_range_padding_entries_are_clamped():
    """Padding entries (positions >= seq_lens[b]) holding -1, INT32_MAX or rows
    past the pool are clamped by the kernels to a real row and masked: the
    output is bit-identical to the same call with row-0 padding."""
    say("decode 16 requests with garbage padding entries")
    case = wl.batched_decode(1, n_req=6, lo=100, hi=3000)
    pool = build_pool(case)
    want = run_decode(pool, case)
    bad = case.table.copy()
    for b in range(case.batch):
        L = int(case.seq_lens[b])
        pad = bad[b, L:]
        pad[0::3] = -1
        pad[1::3] = np.iinfo(np.int32).max
        pad[2::3] = case.pool_rows + 7
    got = run_decode(pool, case, table=bad)
    assert torch.equal(got.view(torch.int16), want.view(torch.int16))
    assert_close(bf16_to_f64(got), _oracle_decode(case), "garbage padding")


@pytest.mark.parametrize("D_,fmt", [(128, "e4m3"), (256, "e4m3"), (128, "int8")])
def test_every_code_at_every_channel_through_the_k_path(D_, fmt):
    """Every finite code at every channel of a key, read through the decode K
    orientation (FreeToken PR #897, "Regression and CUDA isolation": every
    finite value must survive both the K and the V orientation).

    Request b tests one (code c, channel d) pair: its 32 keys are an all-zero
    row (score 0, value 0) except key t_b = (code index + d) % 32, whose K row
    holds c at channel d and zeros elsewhere, with a K scale chosen so that
    q . khat * sm_scale = +3 (q = +-1 at channel d, following the code's sign),
    and whose V row is 1.0 everywhere.  Every output element is then
    e^3 / (e^3 + 31) = 0.393 for a nonzero code and 1/32 for a zero code; a
    code decoded as any other value moves the score by at least 1/16 of 3 and
    the output by at least 0.04.  Compared with the oracle at 1 % relative."""
    say(f"decode: every finite code at every channel through the K path, D={D_}, {fmt}")
    Hq, Hkv, L = 8, 1, 32
    table_v = oracle.code_values(fmt)
    codes = np.array([c for c in range(256) if np.isfinite(table_v[c])], np.uint8)
    B = codes.size * D_
    assert B <= 65535
    ci, d = np.divmod(np.arange(B), D_)
    c = codes[ci]
    val = table_v[c]
    sm = np.float32(wl.softmax_scale(D_))
    # K scale: |decode(c)| * s * sm ~= 3 (s = 1 for a zero code)
    mag = np.where(val != 0, np.abs(val), 1.0).astype(np.float32)
    s = np.where(val != 0, np.float32(3.0) / (mag * sm), np.float32(1.0)).astype(np.float32)
    R = B + 1  # row 0 is the all-zero row; request b's key is row b + 1
    kc = np.zeros((R, Hkv, D_), np.uint8)
    kc[np.arange(B) + 1, 0, d] = c
    vc = np.zeros((R, Hkv, D_), np.uint8)
    one = 0x38 if fmt == "e4m3" else 1
    vc[1:] = one
    ks = np.ones((R, Hkv), np.float32)
    ks[1:, 0] = s
    vs = np.ones((R, Hkv), np.float32)
    t = (ci + d) % L
    table = np.zeros((B, L), np.int32)
    table[np.arange(B), t] = np.arange(B) + 1
    lens = np.full(B, L, np.int32)
    qf = np.zeros((B, Hq, D_), np.float32)
    qf[np.arange(B), :, d] = np.where(val < 0, -1.0, 1.0)[:, None]
    q = wl.bf16_bits(qf)

    pool = fk.Fp8KvPool(R, Hkv, device=DEV, head_dim=D_, code_format=fmt)
    pool.k_codes.copy_(to_dev(kc))
    pool.v_codes.copy_(to_dev(vc))
    pool.k_scales.copy_(to_dev(ks))
    pool.v_scales.copy_(to_dev(vs))
    out = fk.fp8kv_decode_attn(pool, to_dev_bf16(q), to_dev(table), to_dev(lens), L, float(sm), max_splits=1)
    torch.cuda.synchronize()
    got = bf16_to_f64(out)
    ref = oracle.decode_attention(q, kc, vc, ks, vs, table, lens, sm, Hkv, fmt=fmt)
    assert np.all(np.isfinite(got))
    rel = np.abs(got - ref) / np.abs(ref)
    worst = np.unravel_index(np.argmax(rel), rel.shape)
    say(f"  worst relative error {rel.max():.3e} at code 0x{codes[worst[0] // D_]:02x}, channel {worst[0] % D_}")
    assert rel.max() <= 1e-2
    expect = np.where(val != 0, np.exp(3.0) / (np.exp(3.0) + 31.0), 1.0 / 32.0)
    assert np.abs(ref[:, 0, 0] - expect).max() <= 1e-5  # the construction itself


def test_merge_of_a_workspace_no_stage1_wrote_gives_zeros():
    """A zero-filled workspace (split count 0 in its header) merges to zeros and
    reads nothing outside the workspace."""
    say("decode merge over a zero-filled workspace")
    for D_ in (128, 256):
        ws = torch.zeros(fk.fp8kv_decode_workspace_bytes(2, 32, D_, 16), dtype=torch.uint8, device=DEV)
        out = torch.full((2, 32, D_), 7.0, dtype=torch.bfloat16, device=DEV)
        fk.fp8kv_decode_merge(ws, 2, 32, max_splits=16, out=out, head_dim=D_)
        torch.cuda.synchronize()
        assert torch.count_nonzero(out.float()).item() == 0
