"""The C ABI without a GPU: the library loads, exports every declared symbol,
and every host-side validation error comes back as its status code before any
HIP call is made."""
import ctypes
import os
import subprocess

import pytest
import torch

from fp8_kv_cache_row_amd import binding as B

OK, INVALID, UNSUPPORTED, ALIGN, WORKSPACE, HIP = range(6)
A = 1 << 20  # a fake, 256-byte-aligned "device address"; never dereferenced


@pytest.fixture(scope="module")
def lib():
    return B.load()


def test_every_declared_symbol_is_exported(lib):
    names = B.declared_symbols()
    assert set(names) >= {"fp8kv_quantize_rows", "fp8kv_decode_attn", "fp8kv_prefill_attn",
                          "fp8kv_decode_attn_append", "fp8kv_decode_attn_rows", "fp8kv_decode_stage1",
                          "fp8kv_decode_merge",
                          "fp8kv_decode_workspace_bytes", "fp8kv_status_string"}
    for n in names:
        assert hasattr(lib, n), n


def test_measurement_libraries_load_and_export_their_entry_points(lib):
    """The benchmark's measurement builds: the read floors, and the per-wave
    timeline build, which is the same sources (every declared entry point)
    plus its two timeline accessors."""
    pkg = os.path.dirname(B.lib_path())
    floor = ctypes.CDLL(os.path.join(pkg, "libfp8kv_floor.so"))
    for n in ("fp8kv_floor_read", "fp8kv_floor_gather"):
        assert hasattr(floor, n), n
    tl = ctypes.CDLL(os.path.join(pkg, "libfp8kv_timeline.so"))
    for n in list(B.declared_symbols()) + ["fp8kv_timeline_read", "fp8kv_timeline_clear"]:
        assert hasattr(tl, n), n
    assert not hasattr(lib, "fp8kv_timeline_read")  # the product library has no timeline


def test_pool_struct_matches_the_header():
    """The ctypes mirror has the C struct's size and field offsets."""
    assert ctypes.sizeof(B.PoolLayer) == 72
    offs = {name: getattr(B.PoolLayer, name).offset for name, _ in B.PoolLayer._fields_}
    assert offs == {"k_codes": 0, "v_codes": 8, "k_scales": 16, "v_scales": 24, "num_rows": 32, "n_kv_heads": 40,
                    "head_dim": 44, "code_row_stride": 48, "scale_row_stride": 56, "code_format": 64,
                    "reserved": 68}


def test_status_strings(lib):
    for s in range(6):
        assert B.status_string(s).startswith("FP8KV_")
    assert "UNKNOWN" in B.status_string(99)


def _pool(**kw):
    p = dict(k_codes=A, v_codes=2 * A, k_scales=3 * A, v_scales=4 * A, num_rows=100, n_kv_heads=4,
             head_dim=128, code_row_stride=512, scale_row_stride=4, code_format=0)
    p.update(kw)
    return B.PoolLayer(p["k_codes"], p["v_codes"], p["k_scales"], p["v_scales"], p["num_rows"],
                       p["n_kv_heads"], p["head_dim"], p["code_row_stride"], p["scale_row_stride"],
                       p["code_format"], 0)


def _quant(lib, pool, k=A, v=A, stride=512, slots=A, n=4):
    return lib.fp8kv_quantize_rows(ctypes.byref(pool), k, v, stride, slots, n, None)


def _decode(lib, pool, q=A, batch=1, hq=32, table=A, tstride=1024, lens=A, maxlen=1000, sm=0.088,
            splits=0, ws=A, wsb=None, out=A):
    if wsb is None:
        wsb = lib.fp8kv_decode_workspace_bytes(batch, hq, pool.head_dim, splits)
    return lib.fp8kv_decode_attn(ctypes.byref(pool), q, batch, hq, table, tstride, lens, maxlen, sm, splits,
                                 ws, wsb, out, None)


def _rows(lib, pool, q=A, batch=1, nq=3, hq=32, table=A, tstride=1024, lens=A, maxlen=1000, window=0, sm=0.088,
          splits=0, ws=A, wsb=None, out=A):
    if wsb is None:
        wsb = lib.fp8kv_decode_workspace_bytes(batch * max(nq, 1), hq, pool.head_dim, splits)
    return lib.fp8kv_decode_attn_rows(ctypes.byref(pool), q, batch, nq, hq, table, tstride, lens, maxlen, window, sm,
                                      splits, ws, wsb, out, None)


def _prefill(lib, pool, q=A, kc=A, vc=A, T=16, hq=32, rows=A, P=8, wsk=A, wsv=A, cap=8, sm=0.088, out=A):
    return lib.fp8kv_prefill_attn(ctypes.byref(pool), q, kc, vc, T, hq, rows, P, wsk, wsv, cap, sm, out, None)


def test_quantize_validation(lib):
    assert lib.fp8kv_quantize_rows(None, A, A, 512, A, 4, None) == INVALID
    assert _quant(lib, _pool(k_codes=0)) == INVALID
    assert _quant(lib, _pool(head_dim=64)) == UNSUPPORTED
    assert _quant(lib, _pool(code_format=2)) == UNSUPPORTED
    assert _quant(lib, _pool(code_format=-1)) == UNSUPPORTED
    assert _quant(lib, _pool(head_dim=192, code_row_stride=768)) == UNSUPPORTED
    assert _quant(lib, _pool(head_dim=256)) == INVALID               # code_row_stride 512 < 4 * 256
    assert _quant(lib, _pool(head_dim=256, code_row_stride=1024)) == INVALID  # token stride 512 < 4 * 256
    assert _quant(lib, _pool(num_rows=0)) == INVALID
    assert _quant(lib, _pool(code_row_stride=256)) == INVALID        # < Hkv * 128
    assert _quant(lib, _pool(scale_row_stride=2)) == INVALID
    assert _quant(lib, _pool(k_codes=A + 4)) == ALIGN                # codes need 16 B
    assert _quant(lib, _pool(code_row_stride=520)) == ALIGN
    assert _quant(lib, _pool(v_scales=4 * A + 2)) == ALIGN
    assert _quant(lib, _pool(), k=0) == INVALID
    assert _quant(lib, _pool(), n=-1) == INVALID
    assert _quant(lib, _pool(), n=0) == OK                           # no-op, nothing launched
    assert _quant(lib, _pool(), stride=256) == INVALID
    assert _quant(lib, _pool(), stride=516) == ALIGN
    assert _quant(lib, _pool(), k=A + 8) == ALIGN


def test_decode_validation(lib):
    p = _pool()
    assert _decode(lib, _pool(v_scales=0)) == INVALID
    assert _decode(lib, p, q=0) == INVALID
    assert _decode(lib, p, batch=0) == INVALID
    assert _decode(lib, p, hq=30) == INVALID                         # not a multiple of Hkv
    assert _decode(lib, p, hq=12) == UNSUPPORTED                     # G = 3
    assert _decode(lib, p, hq=128) == UNSUPPORTED                    # G = 32
    assert _decode(lib, p, tstride=500) == INVALID                   # table row shorter than max_seq_len
    assert _decode(lib, p, maxlen=-1) == INVALID
    assert _decode(lib, p, sm=float("nan")) == INVALID
    for bad in (0.0, -0.0, -0.088, float("inf"), float("-inf")):    # softmax scale finite and > 0
        assert _decode(lib, p, sm=bad) == INVALID, bad
        assert _append(lib, p, sm=bad) == INVALID, bad
        assert _rows(lib, p, nq=3, sm=bad) == INVALID, bad
    assert lib.fp8kv_decode_stage1(ctypes.byref(p), A, 1, 32, A, 1024, A, 1000, 0.0, 0, A, 1 << 30, None) == INVALID
    assert _decode(lib, p, q=A + 2) == ALIGN
    assert _decode(lib, p, out=A + 8) == ALIGN
    assert _decode(lib, p, table=A + 2) == ALIGN
    assert _decode(lib, p, ws=0) == WORKSPACE
    assert _decode(lib, p, wsb=100) == WORKSPACE
    assert _decode(lib, p, ws=A + 16) == ALIGN
    assert _decode(lib, p, batch=65536, wsb=1 << 62) == UNSUPPORTED  # over FP8KV_MAX_DECODE_GROUPS
    assert _decode(lib, _pool(head_dim=256)) == INVALID               # code_row_stride 512 < 4 * 256
    p256 = _pool(head_dim=256, code_row_stride=1024)
    small = lib.fp8kv_decode_workspace_bytes(1, 32, 128, 0)
    assert _decode(lib, p256, wsb=small) == WORKSPACE                 # D = 256 partials need twice the room


def test_decode_rows_validation(lib):
    p = _pool()
    assert _rows(lib, p, nq=0) == INVALID
    assert _rows(lib, p, nq=9) == INVALID                             # more than FP8KV_MAX_QUERY_ROWS
    assert _rows(lib, p, window=-1) == INVALID
    assert _rows(lib, p, hq=12) == UNSUPPORTED
    assert _rows(lib, p, out=0) == INVALID
    assert _rows(lib, p, out=A + 2) == ALIGN
    assert _rows(lib, p, q=A + 2) == ALIGN
    one_row = lib.fp8kv_decode_workspace_bytes(1, 32, 128, 0)
    assert _rows(lib, p, nq=3, wsb=one_row) == WORKSPACE              # partials for 3 rows
    assert _rows(lib, p, batch=0) == INVALID
    # 8 rows of GQA 8 are 64 columns: two column groups of 32 share the launch dimension
    assert _rows(lib, p, nq=8, batch=32768, wsb=1 << 62) == UNSUPPORTED
    assert _rows(lib, p, tstride=999) == INVALID


def test_decode_stage_validation(lib):
    p = _pool()
    wsb = lib.fp8kv_decode_workspace_bytes(1, 32, 128, 0)
    s1 = lambda **kw: lib.fp8kv_decode_stage1(ctypes.byref(p), kw.get("q", A), 1, kw.get("hq", 32), A, 1024, A,
                                              1000, 0.088, 0, kw.get("ws", A), kw.get("wsb", wsb), None)
    assert s1(q=0) == INVALID
    assert s1(hq=12) == UNSUPPORTED
    assert s1(wsb=wsb - 1) == WORKSPACE
    assert s1(ws=A + 64) == ALIGN
    m = lambda **kw: lib.fp8kv_decode_merge(kw.get("b", 1), 32, kw.get("d", 128), kw.get("splits", 0),
                                            kw.get("ws", A), kw.get("wsb", wsb), kw.get("out", A), None)
    assert m(b=0) == INVALID
    assert m(d=64) == UNSUPPORTED
    assert m(d=256) == WORKSPACE                                      # the D = 128 workspace is too small
    assert m(out=0) == INVALID
    assert m(ws=0) == WORKSPACE
    assert m(splits=300, wsb=100) == WORKSPACE
    assert m(out=A + 2) == ALIGN


def _append(lib, p, **kw):
    wsb = lib.fp8kv_decode_workspace_bytes(1, 32, p.head_dim, 0)
    return lib.fp8kv_decode_attn_append(ctypes.byref(p), kw.get("q", A), 1, kw.get("hq", 32), kw.get("kn", A),
                                        kw.get("vn", 2 * A), kw.get("nstride", 512), kw.get("slots", A), A, 1024, A,
                                        kw.get("maxlen", 1000), kw.get("sm", 0.088), 0, A, kw.get("wsb", wsb),
                                        kw.get("out", A), None)


def _append_window(lib, p, window, **kw):
    wsb = lib.fp8kv_decode_workspace_bytes(1, 32, p.head_dim, 0)
    return lib.fp8kv_decode_attn_append_window(ctypes.byref(p), kw.get("q", A), 1, 32, kw.get("kn", A), 2 * A, 512,
                                               A, A, 1024, A, kw.get("maxlen", 1000), window, 0.088, 0, A,
                                               kw.get("wsb", wsb), kw.get("out", A), None)


def test_decode_append_window_validation(lib):
    p = _pool()
    assert _append_window(lib, p, -1) == INVALID                     # negative window
    assert _append_window(lib, p, 17, kn=0) == INVALID
    assert _append_window(lib, p, 17, maxlen=0) == INVALID
    assert _append_window(lib, p, 17, kn=A + 8) == ALIGN
    assert _append_window(lib, p, 17, wsb=10) == WORKSPACE


def _rows_append(lib, p, nq=3, **kw):
    wsb = lib.fp8kv_decode_workspace_bytes(nq, 32, p.head_dim, 0)
    return lib.fp8kv_decode_attn_rows_append(ctypes.byref(p), kw.get("q", A), 1, nq, 32, kw.get("kn", A), 2 * A, 512,
                                             A, A, 1024, A, kw.get("maxlen", 1000), kw.get("window", 0), 0.088, 0,
                                             A, kw.get("wsb", wsb), kw.get("out", A), None)


def test_decode_rows_append_validation(lib):
    p = _pool()
    assert _rows_append(lib, p, nq=0) == INVALID
    assert _rows_append(lib, p, nq=9) == INVALID                     # more than FP8KV_MAX_QUERY_ROWS
    assert _rows_append(lib, p, nq=8, maxlen=7) == INVALID           # every new token needs a position
    assert _rows_append(lib, p, window=-1) == INVALID
    assert _rows_append(lib, p, kn=0) == INVALID
    assert _rows_append(lib, p, out=A + 2) == ALIGN
    one_row = lib.fp8kv_decode_workspace_bytes(1, 32, 128, 0)
    assert _rows_append(lib, p, nq=3, wsb=one_row) == WORKSPACE       # partials for 3 rows


def test_decode_append_validation(lib):
    p = _pool()
    assert _append(lib, p, kn=0) == INVALID
    assert _append(lib, p, vn=0) == INVALID
    assert _append(lib, p, out=0) == INVALID
    assert _append(lib, p, slots=0) == INVALID
    assert _append(lib, p, slots=A + 2) == ALIGN
    assert _append(lib, p, maxlen=0) == INVALID                      # the new token needs a position
    assert _append(lib, p, nstride=256) == INVALID                   # shorter than Hkv * 128
    assert _append(lib, p, nstride=516) == ALIGN
    assert _append(lib, p, kn=A + 8) == ALIGN
    assert _append(lib, p, hq=12) == UNSUPPORTED
    assert _append(lib, p, wsb=10) == WORKSPACE
    p256 = _pool(head_dim=256, code_row_stride=1024)
    assert _append(lib, p256, nstride=512) == INVALID                # shorter than Hkv * 256
    assert _append(lib, p256, nstride=1024, kn=A + 8) == ALIGN


def test_decode_workspace_bytes(lib):
    f = lib.fp8kv_decode_workspace_bytes
    assert f(1, 32, 128, 64) == 256 + 1 * 32 * 64 * 129 * 4
    assert f(2, 16, 128, 0) == 256 + 2 * 16 * 256 * 129 * 4          # 0 = the library's cap
    assert f(1, 8, 128, 10_000) == 256 + 1 * 8 * 256 * 129 * 4
    assert f(3, 32, 256, 64) == 256 + 3 * 32 * 64 * 257 * 4
    assert f(0, 8, 128, 1) == 0 and f(1, 0, 128, 1) == 0 and f(1, 8, 128, -1) == 0
    assert f(1, 8, 64, 1) == 0


def test_prefill_validation(lib):
    p = _pool()
    assert _prefill(lib, _pool(k_scales=0)) == INVALID
    assert _prefill(lib, p, q=0) == INVALID
    assert _prefill(lib, p, T=0) == INVALID
    assert _prefill(lib, p, P=-1) == INVALID
    assert _prefill(lib, p, hq=24) == UNSUPPORTED                    # G = 6
    assert _prefill(lib, p, rows=0) == INVALID
    assert _prefill(lib, p, wsk=0) == WORKSPACE
    assert _prefill(lib, p, cap=7) == WORKSPACE
    assert _prefill(lib, p, wsv=A + 2) == ALIGN
    assert _prefill(lib, p, kc=A + 4) == ALIGN
    assert _prefill(lib, p, sm=float("nan")) == INVALID
    for bad in (0.0, -0.0, -1.0, float("inf"), float("-inf")):
        assert _prefill(lib, p, sm=bad) == INVALID, bad
    assert _prefill(lib, _pool(head_dim=256, code_row_stride=1024)) == UNSUPPORTED  # prefill runs at D = 128


def _prefill_ws(lib, q=A, kc=A, vc=A, T=16, hq=32, hkv=4, wsk=A, wsv=A, P=8, sm=0.088, out=A):
    return lib.fp8kv_prefill_attn_workspace(q, kc, vc, T, hq, hkv, wsk, wsv, P, sm, out, None)


def test_prefill_workspace_validation(lib):
    assert _prefill_ws(lib, q=0) == INVALID
    assert _prefill_ws(lib, out=0) == INVALID
    assert _prefill_ws(lib, T=0) == INVALID
    assert _prefill_ws(lib, P=-1) == INVALID
    assert _prefill_ws(lib, hkv=0) == INVALID
    assert _prefill_ws(lib, hq=30) == INVALID                        # not a multiple of Hkv
    assert _prefill_ws(lib, hq=12) == UNSUPPORTED                    # G = 3
    for bad in (0.0, -1.0, float("inf"), float("nan")):
        assert _prefill_ws(lib, sm=bad) == INVALID, bad
    assert _prefill_ws(lib, wsk=0) == WORKSPACE
    assert _prefill_ws(lib, wsv=A + 2) == ALIGN
    assert _prefill_ws(lib, q=A + 8) == ALIGN
    assert _prefill_ws(lib, P=0, wsk=0, wsv=0, q=A + 8) == ALIGN     # no prefix: ws pointers unused


@pytest.mark.skipif(torch.cuda.device_count() > 0,
                    reason="valid-looking fake pointers must never reach a real GPU")
def test_valid_arguments_reach_the_device_check(lib):
    """With all arguments valid the call gets as far as the device query, which
    fails (no GPU here) with FP8KV_ERR_HIP; only runs where no device is visible."""
    assert _quant(lib, _pool()) == HIP
    assert _decode(lib, _pool()) == HIP
    assert _decode(lib, _pool(code_format=1)) == HIP
    assert _decode(lib, _pool(head_dim=256, code_row_stride=1024)) == HIP
    assert _rows(lib, _pool(), nq=8, window=17) == HIP
    # the largest accepted batches (FP8KV_MAX_DECODE_GROUPS launch groups)
    assert _decode(lib, _pool(), batch=65535, wsb=1 << 62) == HIP
    assert _rows(lib, _pool(), nq=8, batch=32767, wsb=1 << 62) == HIP    # two column groups per request
    assert _rows(lib, _pool(), nq=3, batch=65535, wsb=1 << 62) == HIP    # 24 columns: one group
    assert _prefill(lib, _pool()) == HIP
    wsb = lib.fp8kv_decode_workspace_bytes(1, 32, 128, 0)
    assert lib.fp8kv_decode_stage1(ctypes.byref(_pool()), A, 1, 32, A, 1024, A, 1000, 0.088, 0, A, wsb, None) == HIP
    assert lib.fp8kv_decode_merge(1, 32, 128, 0, A, wsb, A, None) == HIP
    assert _append(lib, _pool()) == HIP
    assert _append_window(lib, _pool(), 17) == HIP
    assert _rows_append(lib, _pool(), nq=8, window=5) == HIP
    assert _prefill_ws(lib) == HIP
    assert _prefill_ws(lib, P=0, wsk=0, wsv=0) == HIP


def test_header_is_plain_c99_and_the_library_links(tmp_path, lib):
    """A C99 program compiled with -Wall -Werror against include/fp8kv.h, linked
    to libfp8kv.so, runs the host-side validation paths (no device work)."""
    here = os.path.dirname(os.path.abspath(__file__))
    pkg = os.path.dirname(B.lib_path())
    exe = tmp_path / "abi_from_c"
    subprocess.run(["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic", "-I",
                    os.path.dirname(B.header_path()), os.path.join(here, "c", "abi_from_c.c"), "-o", str(exe),
                    "-L", pkg, "-lfp8kv", f"-Wl,-rpath,{pkg}"], check=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0 and "abi_from_c: ok" in r.stdout, r.stdout + r.stderr
