"""GPU parity: chunked prefill (reconstruct + causal bf16 MFMA attention) against the oracle."""
import numpy as np
import pytest
import torch

import oracle
import fp8_kv_cache_row_amd as fk
from fp8_kv_cache_row_amd import workloads as wl

from gpu_common import DEV, assert_bits_equal, assert_close, bf16_to_f64, say, to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu
D = 128


def _run(case, layout="separate", q_idx=None, check_ws=True, fmt="e4m3"):
    """Quantize the prefix into the pool, run prefill, then quantize the chunk; compare."""
    P, T, H = case.prefix_k.shape[0], case.q.shape[0], case.n_kv_heads
    pool = fk.Fp8KvPool(case.pool_rows, H, layout=layout, device=DEV, code_format=fmt)
    if P:
        fk.fp8kv_quantize_rows(pool, to_dev_bf16(case.prefix_k), to_dev_bf16(case.prefix_v), to_dev(case.prefix_rows))
    ws_k = torch.empty((max(P, 1), H, D), dtype=torch.bfloat16, device=DEV)
    ws_v = torch.empty_like(ws_k)
    out = fk.fp8kv_prefill_attn(pool, to_dev_bf16(case.q), to_dev_bf16(case.k_cur), to_dev_bf16(case.v_cur),
                                to_dev(case.prefix_rows) if P else None, ws_k, ws_v, case.sm_scale)
    fk.fp8kv_quantize_rows(pool, to_dev_bf16(case.k_cur), to_dev_bf16(case.v_cur), to_dev(case.chunk_slots))
    torch.cuda.synchronize()

    # oracle: its own codes, its own reconstruction, fp64 attention
    okc, oks = oracle.quantize_rows(case.prefix_k, fmt)
    ovc, ovs = oracle.quantize_rows(case.prefix_v, fmt)
    R = case.pool_rows
    pk = np.zeros((R, H, D), np.uint8)
    pv = np.zeros((R, H, D), np.uint8)
    sk = np.zeros((R, H), np.float32)
    sv = np.zeros((R, H), np.float32)
    pk[case.prefix_rows], pv[case.prefix_rows], sk[case.prefix_rows], sv[case.prefix_rows] = okc, ovc, oks, ovs
    ows_k = oracle.reconstruct(pk, sk, case.prefix_rows, H, fmt) if P else None
    ows_v = oracle.reconstruct(pv, sv, case.prefix_rows, H, fmt) if P else None
    if P and check_ws:
        assert_bits_equal(ws_k[:P].view(torch.int16).cpu().numpy().view(np.uint16), ows_k, "ws_k")
        assert_bits_equal(ws_v[:P].view(torch.int16).cpu().numpy().view(np.uint16), ows_v, "ws_v")
    # the chunk's own rows landed in the pool bit-exactly
    ck, cs = oracle.quantize_rows(case.k_cur, fmt)
    cv, cvs = oracle.quantize_rows(case.v_cur, fmt)
    kc_dev, vc_dev = pool.codes()
    ks_dev, vs_dev = pool.scales()
    assert_bits_equal(kc_dev.cpu().numpy()[case.chunk_slots], ck, "chunk K codes")
    assert_bits_equal(ks_dev.cpu().numpy()[case.chunk_slots], cs, "chunk K scales")
    assert_bits_equal(vc_dev.cpu().numpy()[case.chunk_slots], cv, "chunk V codes")
    assert_bits_equal(vs_dev.cpu().numpy()[case.chunk_slots], cvs, "chunk V scales")
    idx = np.arange(T, dtype=np.int32) if q_idx is None else np.asarray(q_idx, np.int32)
    ref = oracle.prefill_attention(case.q, ows_k, ows_v, case.k_cur, case.v_cur, case.sm_scale, q_idx=idx)
    got = bf16_to_f64(out)[idx]
    return got, ref


@pytest.mark.parametrize("P,T,Hq,Hkv", [(0, 1, 8, 1), (0, 37, 32, 4), (64, 1, 32, 4), (100, 37, 32, 4),
                                         (257, 130, 16, 4), (1000, 300, 8, 8), (33, 65, 32, 2),
                                         (500, 200, 4, 4), (200, 90, 8, 4), (1500, 777, 32, 4)])
def test_small_prefills(P, T, Hq, Hkv):
    say(f"prefill P={P} T={T} Hq={Hq} Hkv={Hkv}")
    case = wl.chunked_prefill(seed=P + T, n_prefix=P, n_chunk=T, n_q_heads=Hq, n_kv_heads=Hkv)
    got, ref = _run(case)
    assert_close(got, ref, f"P={P} T={T} G={Hq // Hkv}")


def test_small_prefill_interleaved_pool():
    say("prefill P=300 T=100, interleaved pool")
    case = wl.chunked_prefill(seed=11, n_prefix=300, n_chunk=100)
    got, ref = _run(case, layout="interleaved")
    assert_close(got, ref, "interleaved")


def _sampled_tokens(T, stride, offset, bands):
    """Every `stride`-th chunk token from `offset` (a stride co-prime to 32 meets
    every token offset inside the kernel's 32-token workgroups at G = 8, so every
    wave and both of its 16-row blocks), plus whole 32-token workgroup bands and
    the last 8 tokens."""
    parts = [np.arange(offset, T, stride), np.arange(T - 8, T)]
    parts += [np.arange(b, b + 32) for b in bands]
    return np.unique(np.concatenate(parts)).astype(np.int32)


def test_sampled_tokens_cover_every_workgroup_offset():
    idx = _sampled_tokens(8192, 61, 0, (4096,))
    assert set(np.arange(32)) <= set((idx[idx < 4096] % 32).tolist())


def test_chunked_prefill_8k_prefix_8k_chunk():
    """8,192 historical FP8 rows + 8,192 bf16 chunk tokens, 32 q / 4 KV heads:
    workspace and chunk rows bit-exact for all rows, attention checked against
    the fp64 oracle on every 61st query token, two whole 32-token workgroup
    bands and the last 8 tokens."""
    say("prefill 8K prefix + 8K chunk (sampled rows vs oracle)")
    case = wl.chunked_prefill(0)
    T = case.q.shape[0]
    idx = _sampled_tokens(T, 61, 0, (4096, 7904))
    got, ref = _run(case, q_idx=idx)
    assert_close(got, ref, "8K+8K sampled")


@pytest.mark.parametrize("where,k0,fmt", [("chunk", 1024.0, "e4m3"), ("prefix", 1024.0, "e4m3"), ("chunk", 196.0, "e4m3"),
                                          ("prefix", 1024.0, "int8")])
def test_prefill_key_far_above_each_rows_first_keys(where, k0, fmt):
    """Every query has q[0] = 4 and one key has k[0] = k0, so that key's score
    lies ~4 k0 / sqrt(128) log2 e above the scores of a row's first 32 keys
    (the kernel's softmax reference): ~520 log2 units for k0 = 1024, past
    where p = 2^(s - ref) overflows, so every workgroup that sees the key
    (the chunk key: the tokens from it on; a prefix key: all) must fall back
    to a running maximum, while the others keep the fixed reference; ~100
    units for k0 = 196, large but finite p on the fixed reference.  Checked
    on every row against the fp64 oracle."""
    say(f"prefill with one key far above the first keys ({where}, k[0] = {k0})")
    case = wl.chunked_prefill(seed=21, n_prefix=600, n_chunk=300)
    case.q[:, :, 0] = wl.bf16_bits(np.float32([4.0]))[0]
    big = wl.bf16_bits(np.float32([k0]))[0]
    if where == "chunk":
        case.k_cur[200, :, 0] = big
    else:
        case.prefix_k[450, :, 0] = big
    got, ref = _run(case, fmt=fmt)
    assert np.isfinite(got).all()
    assert_close(got, ref, f"one key far above ({where}, {k0}, {fmt})")


@pytest.mark.parametrize("P,T,Hq,Hkv", [(0, 37, 32, 4), (100, 37, 32, 4), (257, 130, 16, 4), (1000, 300, 8, 8)])
def test_small_prefills_int8_pool(P, T, Hq, Hkv):
    say(f"prefill over an INT8 pool P={P} T={T} Hq={Hq} Hkv={Hkv}")
    case = wl.chunked_prefill(seed=P + T + 1, n_prefix=P, n_chunk=T, n_q_heads=Hq, n_kv_heads=Hkv)
    got, ref = _run(case, fmt="int8")
    assert_close(got, ref, f"int8 P={P} T={T}")


def test_chunked_prefill_8k_prefix_8k_chunk_int8_pool():
    say("prefill 8K prefix + 8K chunk over an INT8 pool (sampled rows vs oracle)")
    case = wl.chunked_prefill(2)
    T = case.q.shape[0]
    idx = _sampled_tokens(T, 61, 29, (2048,))
    got, ref = _run(case, q_idx=idx, fmt="int8", layout="interleaved")
    assert_close(got, ref, "int8 8K+8K sampled")


def test_prefill_graph_replay_matches_eager():
    """Reconstruct + attention captured in a HIP graph and replayed three times,
    with eager work and synchronizations between the replays: every replay's
    output and workspace are bit-identical to the eager call's."""
    say("prefill P=700 T=300 captured in a graph, 3 replays vs eager")
    case = wl.chunked_prefill(seed=5, n_prefix=700, n_chunk=300)
    P, H = case.prefix_k.shape[0], case.n_kv_heads
    pool = fk.Fp8KvPool(case.pool_rows, H, device=DEV)
    fk.fp8kv_quantize_rows(pool, to_dev_bf16(case.prefix_k), to_dev_bf16(case.prefix_v), to_dev(case.prefix_rows))
    q, kc, vc, rows = to_dev_bf16(case.q), to_dev_bf16(case.k_cur), to_dev_bf16(case.v_cur), to_dev(case.prefix_rows)
    ws_k = torch.empty((P, H, D), dtype=torch.bfloat16, device=DEV)
    ws_v = torch.empty_like(ws_k)
    out = torch.empty_like(q)
    stream = torch.cuda.Stream(device=DEV)
    with torch.cuda.stream(stream):
        fk.fp8kv_prefill_attn(pool, q, kc, vc, rows, ws_k, ws_v, case.sm_scale, out=out, stream=stream)
    stream.synchronize()
    ref_out, ref_k, ref_v = out.clone(), ws_k.clone(), ws_v.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        fk.fp8kv_prefill_attn(pool, q, kc, vc, rows, ws_k, ws_v, case.sm_scale, out=out, stream=stream)
    for rep in range(3):
        out.fill_(0)
        ws_k.fill_(0)
        ws_v.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref_out.view(torch.int16)), f"replay {rep}: out"
        assert torch.equal(ws_k.view(torch.int16), ref_k.view(torch.int16)), f"replay {rep}: ws_k"
        assert torch.equal(ws_v.view(torch.int16), ref_v.view(torch.int16)), f"replay {rep}: ws_v"


@pytest.mark.parametrize("P,T,Hq,Hkv", [(0, 37, 32, 4), (300, 100, 32, 4), (1000, 300, 8, 8), (777, 513, 16, 2)])
def test_prefill_over_a_bf16_workspace(P, T, Hq, Hkv):
    """fp8kv_prefill_attn_workspace over bf16 prefix rows given directly (a BF16
    KV cache, no reconstruction) against the fp64 oracle on the same rows."""
    say(f"prefill over a bf16 workspace P={P} T={T} Hq={Hq} Hkv={Hkv}")
    case = wl.chunked_prefill(seed=P + 3 * T, n_prefix=P, n_chunk=T, n_q_heads=Hq, n_kv_heads=Hkv)
    ws_k = to_dev_bf16(case.prefix_k) if P else None
    ws_v = to_dev_bf16(case.prefix_v) if P else None
    out = fk.fp8kv_prefill_attn_workspace(to_dev_bf16(case.q), to_dev_bf16(case.k_cur), to_dev_bf16(case.v_cur),
                                          ws_k, ws_v, case.sm_scale)
    torch.cuda.synchronize()
    ref = oracle.prefill_attention(case.q, case.prefix_k if P else None, case.prefix_v if P else None,
                                   case.k_cur, case.v_cur, case.sm_scale)
    assert_close(bf16_to_f64(out), ref, f"bf16 workspace P={P} T={T}")


def test_prefill_workspace_call_is_step_two_of_the_fp8_call():
    """Attention over the workspace that fp8kv_prefill_attn rebuilt is that call's
    output, bit for bit."""
    say("prefill: fp8kv_prefill_attn_workspace over the rebuilt workspace == fp8kv_prefill_attn")
    case = wl.chunked_prefill(seed=9, n_prefix=1200, n_chunk=333)
    P, H = case.prefix_k.shape[0], case.n_kv_heads
    pool = fk.Fp8KvPool(case.pool_rows, H, device=DEV)
    fk.fp8kv_quantize_rows(pool, to_dev_bf16(case.prefix_k), to_dev_bf16(case.prefix_v), to_dev(case.prefix_rows))
    q, kc, vc = to_dev_bf16(case.q), to_dev_bf16(case.k_cur), to_dev_bf16(case.v_cur)
    ws_k = torch.empty((P, H, D), dtype=torch.bfloat16, device=DEV)
    ws_v = torch.empty_like(ws_k)
    a = fk.fp8kv_prefill_attn(pool, q, kc, vc, to_dev(case.prefix_rows), ws_k, ws_v, case.sm_scale)
    b = fk.fp8kv_prefill_attn_workspace(q, kc, vc, ws_k, ws_v, case.sm_scale)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
