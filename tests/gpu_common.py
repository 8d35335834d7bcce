"""Helpers shared by the GPU parity tests (not a test module).

Inputs come from fp8_kv_cache_row_amd.workloads; expected values come only
from the CPU oracle.  Tolerance for attention outputs: relative L2 <= 5e-3 and
max abs <= 2e-2 against the fp64 oracle on the same dequantized inputs; codes,
scales and reconstructed bf16 rows must match bit for bit.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
import fp8_kv_cache_row_amd as fk
from fp8_kv_cache_row_amd import workloads as wl

REL_L2_TOL = 5e-3
MAX_ABS_TOL = 2e-2
DEV = torch.device("cuda", 0)


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(DEV).view(torch.bfloat16)


def to_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def bf16_to_f64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def assert_close(got: np.ndarray, ref: np.ndarray, what: str):
    err = got - ref
    rel = float(np.linalg.norm(err) / max(np.linalg.norm(ref), 1e-300))
    mab = float(np.abs(err).max()) if err.size else 0.0
    say(f"  {what}: rel_l2={rel:.3e} max_abs={mab:.3e}")
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    assert rel <= REL_L2_TOL and mab <= MAX_ABS_TOL, f"{what}: rel_l2={rel:.3e} max_abs={mab:.3e}"
    return rel, mab


def build_pool(case, layout: str = "separate", fmt: str = "e4m3") -> fk.Fp8KvPool:
    """Quantize every pool row of a DecodeCase through the HIP path (row r -> slot r)."""
    pool = fk.Fp8KvPool(case.pool_rows, case.n_kv_heads, layout=layout, device=DEV, head_dim=case.head_dim,
                        code_format=fmt)
    slots = torch.arange(case.pool_rows, dtype=torch.int32, device=DEV)
    fk.fp8kv_quantize_rows(pool, to_dev_bf16(case.k_rows), to_dev_bf16(case.v_rows), slots)
    return pool


def pool_arrays(pool: fk.Fp8KvPool):
    kc, vc = pool.codes()
    ks, vs = pool.scales()
    return kc.cpu().numpy(), vc.cpu().numpy(), ks.cpu().numpy(), vs.cpu().numpy()


def assert_bits_equal(a: np.ndarray, b: np.ndarray, what: str):
    a = np.ascontiguousarray(a)
    b = np.ascontiguousarray(b)
    assert a.shape == b.shape, (what, a.shape, b.shape)
    if a.dtype == np.float32:
        a, b = a.view(np.uint32), b.view(np.uint32)
    bad = np.count_nonzero(a != b)
    assert bad == 0, f"{what}: {bad} of {a.size} elements differ"


def oracle_pool(case, fmt: str = "e4m3"):
    kc, ks = oracle.quantize_rows(case.k_rows, fmt)
    vc, vs = oracle.quantize_rows(case.v_rows, fmt)
    return kc, vc, ks, vs


def run_decode(pool, case, max_splits: int = 0, q_bits=None, table=None, seq_lens=None, max_seq_len=None):
    q = to_dev_bf16(case.q if q_bits is None else q_bits)
    t = to_dev((case.table if table is None else table).astype(np.int32))
    sl = to_dev((case.seq_lens if seq_lens is None else seq_lens).astype(np.int32))
    msl = case.max_seq_len if max_seq_len is None else max_seq_len
    out = fk.fp8kv_decode_attn(pool, q, t, sl, msl, case.sm_scale, max_splits=max_splits)
    torch.cuda.synchronize()
    return out
