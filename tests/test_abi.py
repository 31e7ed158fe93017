"""Host-side checks of the C ABI that need no GPU: the library loads, exports every entry
point declared in include/indexer_fp4.h, and its size queries and argument checks behave as
documented (every error path below returns before any device call)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "indexer_fp4.h")
LIB = os.path.join(ROOT, "sparse_attention_indexer_fp4_amd", "libindexer_fp4.so")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(LIB):  # build without importing the package (it loads the library)
        import importlib.util

        spec = importlib.util.spec_from_file_location(
            "_ifp4_build", os.path.join(ROOT, "sparse_attention_indexer_fp4_amd", "build.py"))
        build = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(build)
        build.build()
    lib = ctypes.CDLL(LIB)
    lib.indexer_fp4_last_error.restype = ctypes.c_char_p
    for name in ("indexer_fp4_decode_sched_bytes", "indexer_fp4_prefill_sched_bytes",
                 "indexer_topk_workspace_bytes"):
        getattr(lib, name).restype = ctypes.c_int64
    lib.indexer_topk_workspace_bytes.argtypes = [ctypes.c_int32, ctypes.c_int64, ctypes.c_int32]
    return lib


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?(?:int|int64_t|char|void)\s*\*?\s*(indexer_\w+)\s*\(",
                                 text, flags=re.M)))


def test_every_declared_symbol_is_exported(L):
    names = declared_functions()
    assert len(names) == 17, names
    for n in names:
        assert hasattr(L, n), n
    import sparse_attention_indexer_fp4_amd as pkg_module  # noqa: F401  (binding loads too)

    assert set(pkg_module.EXPORTS) == set(names)


def test_probe_library_loads_and_rejects_bad_arguments():
    """The instruction-mix probe (bench.py --mfma-valu-probe) is a library of its own: it loads,
    exports its one entry point, and rejects a mode or size out of range before any device call."""
    path = os.path.join(ROOT, "sparse_attention_indexer_fp4_amd", "libindexer_fp4_probe.so")
    if not os.path.exists(path):
        pytest.skip("probe library not built")
    P = ctypes.CDLL(path)
    f = P.indexer_fp4_probe_mfma_valu
    f.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int] + [ctypes.c_void_p] * 4
    f.restype = ctypes.c_int
    buf = ctypes.c_void_p(16)  # never dereferenced: every call below fails its checks first
    assert f(6, 10, 1, buf, buf, buf, None) == -1
    assert f(-1, 10, 1, buf, buf, buf, None) == -1
    assert f(0, 0, 1, buf, buf, buf, None) == -1
    assert f(0, 10, 0, buf, buf, buf, None) == -1
    assert f(0, 10, 1, None, buf, buf, None) == -1


def test_size_queries(L):
    # decode: 8-word header + cum[B+1] + unit_begin[U+1] + unit_seq/unit_page/unit_run[U]
    assert L.indexer_fp4_decode_sched_bytes(8, 1, 512) == 4 * (8 + 9 + 513 + 3 * 512)
    assert L.indexer_fp4_decode_sched_bytes(-1, 1, 512) < 0
    assert L.indexer_fp4_decode_sched_bytes(8, 1, 0) < 0
    # a schedule buffer sized for next_n = n serves next_n = 1 (the pages' unit-count invariant
    # f(n) >= f(1)); here the units are (sequence, page) items, so the size does not depend on
    # next_n at all
    for b, u in [(1, 512), (8, 512), (16, 37), (3, 4096)]:
        sizes = [L.indexer_fp4_decode_sched_bytes(b, n, u) for n in (1, 2, 3, 4)]
        assert min(sizes) == max(sizes) == sizes[0] > 0, (b, u, sizes)
    # prefill: 16-word header + unit records [U] x16 + tiles[max] x8 + cum[max+1] + unit_begin[U+1]
    # + unit_tile[U] + req_tile[R+1] + item pages [max * bt_ld], with max = rows/16 + R tiles
    L.indexer_fp4_prefill_sched_bytes.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int64]
    mt = 2048 // 16 + 4
    assert L.indexer_fp4_prefill_sched_bytes(4, 2048, 256, 68) == \
        4 * (16 + 16 * 256 + 8 * mt + mt + 1 + 257 + 256 + 5 + mt * 68)
    assert L.indexer_fp4_prefill_sched_bytes(0, 2048, 256, 68) < 0
    assert L.indexer_fp4_prefill_sched_bytes(4, 2048, 256, 0) < 0
    assert L.indexer_topk_workspace_bytes(8, 131072, 2048) >= 0
    assert L.indexer_topk_workspace_bytes(8, 131072, 0) < 0


def _err(L):
    msg = L.indexer_fp4_last_error().decode()
    L.indexer_last_error.restype = ctypes.c_char_p
    assert L.indexer_last_error().decode() == msg  # the same message under the shorter name
    return msg


def test_host_argument_errors(L):
    P, I32, I64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    L.indexer_fp4_decode_schedule.argtypes = [P, I32, I32, I32, P, I64, P, P]
    # next_n out of range
    assert L.indexer_fp4_decode_schedule(None, 8, 5, 512, None, 0, None, None) == -1
    assert "next_n=5" in _err(L)
    # schedule buffer too small: never silently truncated
    assert L.indexer_fp4_decode_schedule(None, 8, 1, 512, None, 100, None, None) == -2
    assert "needs" in _err(L) and "100" in _err(L)
    L.indexer_fp4_prefill_schedule.argtypes = [P, P, I32, I32, I32, P, I64, I64, P, I64, P, P]
    assert L.indexer_fp4_prefill_schedule(None, None, 4, 1001, 4096, None, 68, 100, None, 0, None, None) == -1
    assert "multiple of 8" in _err(L)
    assert L.indexer_fp4_prefill_schedule(None, None, 4, 1000, 256, None, 0, 100, None, 0, None, None) == -1
    assert "bt_ld=0" in _err(L)
    assert L.indexer_fp4_prefill_schedule(P(16), P(16), 4, 1000, 256, P(16), 68, 100, P(16), 64, P(16), None) == -2
    assert "needs" in _err(L)
    L.indexer_fp4_score_decode.argtypes = [P, P, P, I32, P, P, I64, P, I64, I32, I32, P, I64, I32, P, P, I64, P, P]
    # head count not a multiple of 16 (the MFMA tile height)
    assert L.indexer_fp4_score_decode(None, None, None, 24, None, None, 0, None, 8, 1, 1, None, 0, 512, None,
                                      None, 512, None, None) == -1
    assert "n_heads=24" in _err(L)
    # logits row too short for the block table
    assert L.indexer_fp4_score_decode(None, None, None, 64, None, None, 0, None, 8, 1, 1, None, 0, 512, None,
                                      None, 500, None, None) == -2
    assert "logits_ld=500" in _err(L)
    # a schedule buffer smaller than a schedule of the call's sizes (the unit table would be
    # read past its end)
    need = L.indexer_fp4_decode_sched_bytes(1, 1, 512)
    assert L.indexer_fp4_score_decode(P(16), P(16), P(16), 64, P(16), P(16), 1, P(16), 8, 1, 1, P(16), need - 4,
                                      512, P(16), P(16), 512, None, None) == -2
    assert "sched_bytes" in _err(L) and str(need) in _err(L)
    # a row histogram that is not 16-byte aligned
    assert L.indexer_fp4_score_decode(None, None, None, 64, None, None, 0, None, 8, 0, 1, P(16), 1 << 20, 512,
                                      P(16), None, 512, P(20), None) == -1
    assert "row_hist" in _err(L)
    L.indexer_fp4_score_prefill.argtypes = [P, P, P, I32, P, P, I64, I64, I32, P, I64, I32, I32, P, I64, P]
    assert L.indexer_fp4_score_prefill(None, None, None, 64, None, None, 0, 8, 0, None, 0, 512, 8, None, 512,
                                       None) == -1
    need = L.indexer_fp4_prefill_sched_bytes(2, 16, 256, 8)
    assert L.indexer_fp4_score_prefill(P(16), P(16), P(16), 64, P(16), P(16), 1, 8, 2, P(16), need - 1, 256, 16,
                                       P(16), 512, None) == -2
    assert "sched_bytes" in _err(L)
    assert L.indexer_fp4_score_prefill(P(16), P(16), P(16), 64, P(16), P(16), 1, 8, 2, P(16), need, 256, 16,
                                       P(16), 500, None) == -2
    assert "logits_ld=500" in _err(L)
    L.indexer_topk.argtypes = [P, I64, I32, P, I64, I32, P, I64, P, I64, P, P]
    assert L.indexer_topk(None, 100, 4, None, 100, 0, None, 16, None, 0, None, None) == -1
    assert "k=0" in _err(L)
    assert L.indexer_topk(None, 100, 4, None, 100, 32, None, 16, None, 0, None, None) == -2
    assert "topk_ld=16" in _err(L)
    assert L.indexer_topk(None, 100, 4, None, 200, 32, None, 32, None, 0, None, None) == -1
    assert L.indexer_topk(None, 100, 0, None, 100, 32, None, 32, None, 0, P(20), None) == -1
    assert "row_hist" in _err(L)
    # the allocation-free top-k refuses sizes whose workspace exceeds its fixed scratch array
    L.indexer_topk_noalloc.argtypes = [P, I64, I32, P, I64, I32, P, I64, P, P]
    assert L.indexer_topk_noalloc(None, 1 << 20, 64, None, 1 << 20, 2048, None, 2048, None, None) == -2
    assert "scratch array" in _err(L) and "n_rows=64" in _err(L)
    assert L.indexer_topk_noalloc(None, 100, 4, None, 100, 0, None, 16, None, None) == -1
    L.indexer_topk_merge.argtypes = [P, P, I64, I32, I32, I32, P, I64, P]
    assert L.indexer_topk_merge(None, None, 16, 2, 16, 0, None, 16, None) == -1
    assert L.indexer_topk_merge(None, None, 16, 2, 16, 8192, None, 8192, None) == -1
    assert L.indexer_topk_merge(None, None, 8, 2, 16, 8, None, 8, None) == -1
    assert "cand_ld=8" in _err(L)
    assert L.indexer_topk_merge(P(16), P(16), 16, 2, 16, 8, P(16), 4, None) == -2
    L.indexer_fp4_quant_and_cache.argtypes = [P, I64, I64, P, P, P, I64, P, I64, I32, P, P, P]
    assert L.indexer_fp4_quant_and_cache(None, 4, 128, None, None, None, 1, None, 0, 0, None, None, None) == -1
    assert L.indexer_fp4_quant_and_cache(P(16), 4, 100, P(16), P(16), P(16), 1, None, 0, 0, None, None, None) == -1
    assert "k_ld=100" in _err(L)
    F32 = ctypes.c_float
    L.indexer_fp4_norm_rope_quant_and_cache.argtypes = [P, I64, I64, P, P, F32, P, P, I64, I32, I32, P, P, P, I64,
                                                        P, I32, P, P, P, F32, P, I32, P, P]
    fused = L.indexer_fp4_norm_rope_quant_and_cache

    def call(rope_dim=0, bias=None, weight=None, eps=1e-6, positions=None, cs=None, max_pos=0, q=None, heads=0,
             n_tok=4, k_ld=128):
        return fused(P(16), n_tok, k_ld, weight, bias, eps, positions, cs, max_pos, rope_dim, 0, P(16), P(16),
                     P(16), 1, q, heads, P(16), P(16), P(16), 1.0, P(16), 0, None, None)
    assert call(rope_dim=24) == -1 and "rope_dim=24" in _err(L)
    assert call(rope_dim=144) == -1
    assert call(bias=P(16)) == -1 and "bias" in _err(L)
    assert call(weight=P(16), eps=-1.0) == -1 and "eps" in _err(L)
    assert call(rope_dim=64) == -1 and "cos/sin" in _err(L)
    assert call(k_ld=120) == -1 and "k_ld=120" in _err(L)
    assert call(q=P(16), heads=0) == -1 and "n_heads=0" in _err(L)
    assert call(n_tok=-1) == -1
    L.indexer_fp4_write_and_score_decode.argtypes = [P, I64, P, P, F32, P, P, I64, I32, I32, P, P, P, F32, I32, I32,
                                                     P, P, I64, P, I64, I32, P, I64, I32, P, P, I64, P, P]
    ws_fn = L.indexer_fp4_write_and_score_decode

    def ws_call(heads=64, rope_dim=0, k_ld=128, bias=None, weight=None, eps=1e-6, k=P(16), bt_ld=4, ld=256,
                sched_bytes=1 << 20, batch=2, positions=None, cs=None, max_pos=0):
        return ws_fn(k, k_ld, weight, bias, eps, positions, cs, max_pos, rope_dim, 0, P(16), P(16), P(16), 1.0, 0,
                     heads, P(16), P(16), 8, P(16), bt_ld, batch, P(16), sched_bytes, 16, P(16), P(16), ld, None, None)
    assert ws_call(heads=144) == -1 and "n_heads=144" in _err(L)
    assert ws_call(heads=24) == -1
    assert ws_call(rope_dim=24) == -1 and "rope_dim=24" in _err(L)
    assert ws_call(rope_dim=64) == -1 and "cos/sin" in _err(L)
    assert ws_call(bias=P(16)) == -1 and "bias" in _err(L)
    assert ws_call(weight=P(16), eps=-1.0) == -1 and "eps" in _err(L)
    assert ws_call(k_ld=120) == -1 and "k_ld=120" in _err(L)
    assert ws_call(k=None) == -1 and "NULL" in _err(L)
    assert ws_call(ld=200) == -2 and "logits_ld=200" in _err(L)
    assert ws_call(sched_bytes=16) == -2 and "sched_bytes=16" in _err(L)
    assert ws_call(k=P(8)) == -1 and "aligned" in _err(L)
