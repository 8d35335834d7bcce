"""Seeded synthetic inputs for the FP8 per-row KV cache path.

This module only draws random numbers and lays them out. It holds none of the
method's arithmetic (no quantization, no attention): both the HIP library and
the CPU oracle consume exactly the bytes produced here.

Shapes follow the workloads described on the pages:
  * FreeToken PR #853, "Hardware and reproducibility" and "Validation":
    a 48-layer model with 4 KV heads of dimension 128, a page-size-1 pool of
    33,059 (or 40,290) physical rows whose slots are randomized.
  * FreeToken PR #897, "Fresh R9700 stage-1 A/B": D=128, 32 query heads,
    GQA 4/8, batch 1, 8K/32K keys, randomized physical slots.
  * FreeToken PR #853, "Paired end-to-end A/B": the 8K historical prefix +
    8K new-token prefill operator.
  * FreeToken PR #897, "Regression and CUDA isolation": head dims 128 and
    256, 1/3/8 query rows per request, 17/8,192/32,768 keys.

Values are drawn as float32 from numpy's PCG64 generator and rounded to bf16
(round to nearest even) by torch's CPU cast; arrays of bf16 are returned as
their uint16 bit patterns.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np
import torch

HEAD_DIM = 128
N_OUTLIER_CHANNELS = 4
OUTLIER_GAIN = 8.0


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 array -> bf16 bit patterns (uint16), rounded by torch's CPU cast."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float32 values (exact widening)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def softmax_scale(head_dim: int = HEAD_DIM) -> float:
    """1/sqrt(head_dim) rounded once to float32 (the value passed to both sides)."""
    return float(np.float32(1.0 / np.sqrt(np.float64(head_dim))))


def outlier_channels(rng: np.random.Generator, n_kv_heads: int, head_dim: int = HEAD_DIM) -> np.ndarray:
    """Per KV head, 4 distinct channels that carry x8 outliers in K."""
    return np.stack([rng.choice(head_dim, N_OUTLIER_CHANNELS, replace=False)
                     for _ in range(n_kv_heads)]).astype(np.int64)


def draw_k(rng: np.random.Generator, n: int, n_kv_heads: int,
           outliers: Optional[np.ndarray], head_dim: int = HEAD_DIM) -> np.ndarray:
    x = rng.standard_normal((n, n_kv_heads, head_dim), dtype=np.float32)
    if outliers is not None:
        for h in range(n_kv_heads):
            x[:, h, outliers[h]] *= np.float32(OUTLIER_GAIN)
    return x


def draw_normal(rng: np.random.Generator, shape, std: float = 1.0) -> np.ndarray:
    x = rng.standard_normal(shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


@dataclass
class DecodeCase:
    """One decode-attention call over a page-size-1 FP8 pool.

    k_rows / v_rows: bf16 bits [pool_rows][n_kv_heads][D]; pool row r holds
    k_rows[r] once quantized.  q: bf16 bits [batch][n_q_heads][D], or
    [batch][n_qrows][n_q_heads][D] for a request's last n_qrows positions.
    table: int32 [batch][table_stride] logical -> physical row map.
    new_k / new_v (optional): bf16 bits [batch][n_kv_heads][D] of the token
    written during the step into slot table[b][seq_lens[b]-1].
    """
    name: str
    n_q_heads: int
    n_kv_heads: int
    pool_rows: int
    k_rows: np.ndarray
    v_rows: np.ndarray
    q: np.ndarray
    table: np.ndarray
    seq_lens: np.ndarray
    sm_scale: float
    new_k: Optional[np.ndarray] = None
    new_v: Optional[np.ndarray] = None

    @property
    def batch(self) -> int:
        return int(self.q.shape[0])

    @property
    def head_dim(self) -> int:
        return int(self.q.shape[-1])

    @property
    def n_qrows(self) -> int:
        return 1 if self.q.ndim == 3 else int(self.q.shape[1])

    @property
    def max_seq_len(self) -> int:
        return int(self.seq_lens.max()) if self.seq_lens.size else 0


@dataclass
class PrefillCase:
    """One chunked-prefill call: P historical FP8 rows + a T-token bf16 chunk.

    prefix_k / prefix_v: bf16 bits [P][n_kv_heads][128] quantized into pool rows
    prefix_rows[j] before the call.  q: [T][n_q_heads][128]; k_cur / v_cur:
    [T][n_kv_heads][128]; chunk_slots: pool rows the chunk is quantized into.
    """
    name: str
    n_q_heads: int
    n_kv_heads: int
    pool_rows: int
    prefix_rows: np.ndarray
    chunk_slots: np.ndarray
    prefix_k: np.ndarray
    prefix_v: np.ndarray
    q: np.ndarray
    k_cur: np.ndarray
    v_cur: np.ndarray
    sm_scale: float


def tiny_decode(seed: int = 0) -> DecodeCase:
    """256 K and 256 V rows of 1 KV head, 8 query heads (GQA 8), identity table."""
    rng = np.random.default_rng(seed)
    n = 256
    k = draw_normal(rng, (n, 1, HEAD_DIM))
    v = draw_normal(rng, (n, 1, HEAD_DIM))
    q = draw_normal(rng, (1, 8, HEAD_DIM))
    return DecodeCase("tiny_gqa8_256", 8, 1, n, bf16_bits(k), bf16_bits(v), bf16_bits(q),
                      np.arange(n, dtype=np.int32).reshape(1, n), np.array([n], np.int32),
                      softmax_scale())


def _draw_q(rng: np.random.Generator, batch: int, n_qrows: int, n_q_heads: int, head_dim: int) -> np.ndarray:
    """Query rows [batch][n_q_heads][D] (one row) or [batch][n_qrows][n_q_heads][D];
    one row draws the same numbers as the multi-row shape would."""
    q = draw_normal(rng, (batch, n_qrows, n_q_heads, head_dim))
    return q[:, 0] if n_qrows == 1 else q


def layer_decode(seed: int = 0, ctx: int = 32768, pool_rows: int = 33059,
                 n_q_heads: int = 32, n_kv_heads: int = 4, with_new_token: bool = True,
                 head_dim: int = HEAD_DIM, n_qrows: int = 1) -> DecodeCase:
    """One layer of batch-1 decode: 32 q / 4 KV heads, 32,768 of 33,059 pool rows.

    K ~ N(0,1) with 4 fixed x8 outlier channels per head; V ~ 0.5*N(0,1);
    q ~ N(0,1); table = a seeded permutation of the pool, first `ctx` entries.
    """
    rng = np.random.default_rng(seed)
    out = outlier_channels(rng, n_kv_heads, head_dim)
    k = draw_k(rng, pool_rows, n_kv_heads, out, head_dim)
    v = draw_normal(rng, (pool_rows, n_kv_heads, head_dim), 0.5)
    q = _draw_q(rng, 1, n_qrows, n_q_heads, head_dim)
    table = rng.permutation(pool_rows)[:ctx].astype(np.int32).reshape(1, ctx)
    nk = nv = None
    if with_new_token:
        nk = bf16_bits(draw_k(rng, 1, n_kv_heads, out, head_dim))
        nv = bf16_bits(draw_normal(rng, (1, n_kv_heads, head_dim), 0.5))
    name = f"layer_decode_{ctx}" + ("" if head_dim == HEAD_DIM else f"_d{head_dim}") + \
        ("" if n_qrows == 1 else f"_{n_qrows}rows")
    return DecodeCase(name, n_q_heads, n_kv_heads, pool_rows,
                      bf16_bits(k), bf16_bits(v), bf16_bits(q), table,
                      np.array([ctx], np.int32), softmax_scale(head_dim), nk, nv)


def model_step_table(seed: int = 0, ctx: int = 40000, pool_rows: int = 40290) -> np.ndarray:
    """Row table shared by all layers of the 48-layer step."""
    rng = np.random.default_rng(seed)
    return rng.permutation(pool_rows)[:ctx].astype(np.int32).reshape(1, ctx)


def model_step_layer(layer: int, table: np.ndarray, seed: int = 0, pool_rows: int = 40290,
                     n_q_heads: int = 32, n_kv_heads: int = 4) -> DecodeCase:
    """Layer `layer` of the 48-layer, 40,000-context decode step (seed (seed, layer))."""
    rng = np.random.default_rng((seed, layer))
    out = outlier_channels(rng, n_kv_heads)
    k = draw_k(rng, pool_rows, n_kv_heads, out)
    v = draw_normal(rng, (pool_rows, n_kv_heads, HEAD_DIM), 0.5)
    q = draw_normal(rng, (1, n_q_heads, HEAD_DIM))
    nk = bf16_bits(draw_k(rng, 1, n_kv_heads, out))
    nv = bf16_bits(draw_normal(rng, (1, n_kv_heads, HEAD_DIM), 0.5))
    ctx = table.shape[1]
    return DecodeCase(f"model_step_layer{layer}", n_q_heads, n_kv_heads, pool_rows,
                      bf16_bits(k), bf16_bits(v), bf16_bits(q), table,
                      np.array([ctx], np.int32), softmax_scale(), nk, nv)


def batched_decode(seed: int = 0, n_req: int = 16, lo: int = 1024, hi: int = 32768,
                   n_q_heads: int = 16, n_kv_heads: int = 4, with_new_token: bool = False,
                   head_dim: int = HEAD_DIM, n_qrows: int = 1) -> DecodeCase:
    """16 requests with seeded lengths in [1024, 32768], GQA 4, shared scattered pool.

    With new tokens, request b's token goes to table[b][lens[b]-1]; they are
    drawn after everything else, so the other arrays do not depend on it.
    """
    rng = np.random.default_rng(seed)
    lens = rng.integers(lo, hi, n_req, endpoint=True).astype(np.int64)
    pool_rows = int(lens.sum())
    perm = rng.permutation(pool_rows).astype(np.int32)
    out = outlier_channels(rng, n_kv_heads, head_dim)
    k = draw_k(rng, pool_rows, n_kv_heads, out, head_dim)
    v = draw_normal(rng, (pool_rows, n_kv_heads, head_dim), 0.5)
    q = _draw_q(rng, n_req, n_qrows, n_q_heads, head_dim)
    max_len = int(lens.max())
    table = np.zeros((n_req, max_len), np.int32)
    starts = np.concatenate([[0], np.cumsum(lens)[:-1]])
    for b in range(n_req):
        table[b, :lens[b]] = perm[starts[b]:starts[b] + lens[b]]
    nk = nv = None
    if with_new_token:
        nk = bf16_bits(draw_k(rng, n_req, n_kv_heads, out, head_dim))
        nv = bf16_bits(draw_normal(rng, (n_req, n_kv_heads, head_dim), 0.5))
    name = "batched_gqa4_16req" + ("" if head_dim == HEAD_DIM else f"_d{head_dim}") + \
        ("" if n_qrows == 1 else f"_{n_qrows}rows")
    return DecodeCase(name, n_q_heads, n_kv_heads, pool_rows,
                      bf16_bits(k), bf16_bits(v), bf16_bits(q), table,
                      lens.astype(np.int32), softmax_scale(head_dim), nk, nv)


def chunked_prefill(seed: int = 0, n_prefix: int = 8192, n_chunk: int = 8192,
                    n_q_heads: int = 32, n_kv_heads: int = 4) -> PrefillCase:
    """8,192 historical FP8 rows + an 8,192-token bf16 chunk, causal, 32 q / 4 KV heads."""
    rng = np.random.default_rng(seed)
    out = outlier_channels(rng, n_kv_heads)
    pool_rows = n_prefix + n_chunk
    perm = rng.permutation(pool_rows).astype(np.int32)
    pk = draw_k(rng, n_prefix, n_kv_heads, out)
    pv = draw_normal(rng, (n_prefix, n_kv_heads, HEAD_DIM))
    q = draw_normal(rng, (n_chunk, n_q_heads, HEAD_DIM))
    kc = draw_k(rng, n_chunk, n_kv_heads, out)
    vc = draw_normal(rng, (n_chunk, n_kv_heads, HEAD_DIM))
    return PrefillCase(f"prefill_{n_prefix}p_{n_chunk}t", n_q_heads, n_kv_heads, pool_rows,
                       perm[:n_prefix].copy(), perm[n_prefix:].copy(),
                       bf16_bits(pk), bf16_bits(pv), bf16_bits(q), bf16_bits(kc), bf16_bits(vc),
                       softmax_scale())


def all_bf16_patterns_row_batches() -> np.ndarray:
    """Rows of 128 bf16 that together contain every bf16 bit pattern of magnitude <= 448.

    Each row holds 448.0 (so the row's amax is exactly 448 and its scale exactly 1)
    followed by 127 patterns; the patterns cover all 65,536 encodings except NaN/Inf
    and finite values above 448 in magnitude.
    """
    pats = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    f = bf16_bits_to_f32(pats)
    keep = np.isfinite(f) & (np.abs(f) <= 448.0)
    pats = pats[keep]
    per = HEAD_DIM - 1
    n_rows = -(-pats.size // per)
    rows = np.zeros((n_rows, HEAD_DIM), np.uint16)
    fill = np.concatenate([pats, np.zeros(n_rows * per - pats.size, np.uint16)])
    rows[:, 0] = bf16_bits(np.array([448.0], np.float32))[0]
    rows[:, 1:] = fill.reshape(n_rows, per)
    return rows
