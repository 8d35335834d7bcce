"""GPU parity of fp8kv_decode_attn_append_noalloc (the decode step whose split
partials live in the library's fixed per-device array) against
fp8kv_decode_attn_append (the same step over a caller workspace) and the
oracle: two calls in a row, the second smaller, then a call too large for the
array, which must be rejected before anything is written."""
import numpy as np
import pytest
import torch

import oracle
import fp8_kv_cache_row_amd as fk
from fp8_kv_cache_row_amd import binding as B
from fp8_kv_cache_row_amd import workloads as wl

from gpu_common import DEV, assert_bits_equal, assert_close, bf16_to_f64, build_pool, oracle_pool, say, to_dev, \
    to_dev_bf16

pytestmark = pytest.mark.gpu


def _step(case, noalloc):
    """One decode step (quantize the new token + attention) on a fresh pool."""
    pool = build_pool(case, "interleaved")
    q, nk, nv = to_dev_bf16(case.q), to_dev_bf16(case.new_k), to_dev_bf16(case.new_v)
    t, sl = to_dev(case.table), to_dev(case.seq_lens)
    last = case.table[np.arange(case.table.shape[0]), case.seq_lens.astype(np.int64) - 1]
    slot = to_dev(np.ascontiguousarray(last, dtype=np.int32))
    out = torch.full_like(q, 3.0)
    if noalloc:
        fk.binding.fp8kv_decode_attn_append_noalloc(pool, q, nk, nv, slot, t, sl, case.max_seq_len, case.sm_scale,
                                                    out=out)
    else:
        fk.fp8kv_decode_attn_append(pool, q, nk, nv, slot, t, sl, case.max_seq_len, case.sm_scale, out=out)
    torch.cuda.synchronize()
    return pool, out


def _oracle_step(case):
    kc, vc, ks, vs = oracle_pool(case)
    last = case.table[np.arange(case.table.shape[0]), case.seq_lens.astype(np.int64) - 1]
    nkc, nks = oracle.quantize_rows(case.new_k)
    nvc, nvs = oracle.quantize_rows(case.new_v)
    kc[last], ks[last], vc[last], vs[last] = nkc, nks, nvc, nvs
    out = oracle.decode_attention(case.q, kc, vc, ks, vs, case.table, case.seq_lens, case.sm_scale, case.n_kv_heads)
    return out, (kc, vc, ks, vs)


def _compare(case, what):
    p_ref, o_ref = _step(case, noalloc=False)
    p_new, o_new = _step(case, noalloc=True)
    assert torch.equal(o_new.view(torch.int16), o_ref.view(torch.int16)), f"{what}: output differs"
    for a, b, name in zip(p_new._buffers, p_ref._buffers, ("pool",)):
        assert torch.equal(a, b), f"{what}: {name} differs"
    ref, pools = _oracle_step(case)
    assert_close(bf16_to_f64(o_new), ref, what)
    kc, vc = p_new.codes()
    ks, vs = p_new.scales()
    for got, want, name in zip((kc, vc, ks, vs), pools, ("K codes", "V codes", "K scales", "V scales")):
        assert_bits_equal(got.cpu().numpy(), want, f"{what}: {name}")


def test_noalloc_step_matches_the_workspace_step_twice_then_smaller():
    say("noalloc decode step: 32K context, then a 16-request batch of shorter contexts")
    _compare(wl.layer_decode(0), "32K step")
    _compare(wl.batched_decode(3, n_req=16, lo=100, hi=3000, with_new_token=True), "16-request batch")
    _compare(wl.layer_decode(7, ctx=1000, pool_rows=1200, n_q_heads=16, n_kv_heads=2), "1K step")


def test_noalloc_step_rejects_a_call_larger_than_its_array():
    say("noalloc decode step: a batch whose partials exceed the array is rejected")
    # 512 requests x 32 heads x 64 splits (512-key splits of 32,768 keys) x 129 floats > 32 MiB
    Bn, Hq, Hkv, L = 512, 32, 4, 32768
    pool = fk.Fp8KvPool(1024, Hkv, device=DEV)
    q = torch.zeros((Bn, Hq, 128), dtype=torch.bfloat16, device=DEV)
    nk = torch.zeros((Bn, Hkv, 128), dtype=torch.bfloat16, device=DEV)
    table = torch.zeros((Bn, L), dtype=torch.int32, device=DEV)
    lens = torch.full((Bn,), L, dtype=torch.int32, device=DEV)
    slots = torch.arange(Bn, dtype=torch.int32, device=DEV)
    out = torch.full_like(q, 5.0)
    with pytest.raises(B.Fp8KvError) as e:
        fk.binding.fp8kv_decode_attn_append_noalloc(pool, q, nk, nk, slots, table, lens, L, 0.088, max_splits=64,
                                                    out=out)
    assert e.value.status == 4  # FP8KV_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert torch.all(out.float() == 5.0)
    assert torch.count_nonzero(pool.k_codes).item() == 0
