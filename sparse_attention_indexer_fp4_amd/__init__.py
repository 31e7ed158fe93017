"""Python binding of the gfx950 FP4 sparse-indexer library (libindexer_fp4.so).

Argument marshalling only: every function takes torch tensors that live on the GPU, checks
their dtype/device/contiguity, and passes raw pointers, sizes and the current HIP stream to
the C entry point of the same name (see include/indexer_fp4.h for the exact semantics). All
computation happens in the library's HIP kernels; there is no fallback. If the shared
library has not been built, importing this package raises ImportError.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libindexer_fp4.so")

PAGE = 64
HEAD_DIM = 128
ROW_MULTIPLE = 8   # a prefill step's padded row count is a multiple of this
TILE_ROWS = 16     # prefill rows per tile
DEV_BAD_PAGE, DEV_TABLE_SHORT, DEV_BAD_SCHEDULE, DEV_BAD_LENGTH = 1, 2, 4, 8
DEV_BAD_POSITION, DEV_SLOT_OUT_OF_POOL = 16, 32
# persistent-grid sizes the scorers default to (units = workgroups)
DECODE_UNITS = 512
PREFILL_UNITS = 256  # one 16-wave unit per CU

EXPORTS = (
    "indexer_fp4_last_error",
    "indexer_last_error",
    "indexer_fp4_quant_and_cache",
    "indexer_fp4_norm_rope_quant_and_cache",
    "indexer_fp4_decode_sched_bytes",
    "indexer_fp4_decode_schedule",
    "indexer_fp4_prefill_sched_bytes",
    "indexer_fp4_prefill_schedule",
    "indexer_fp4_score_decode",
    "indexer_fp4_write_and_score_decode",
    "indexer_fp4_score_prefill",
    "indexer_fp8_quant_and_cache",
    "indexer_fp8_score_decode",
    "indexer_topk_workspace_bytes",
    "indexer_topk_merge",
    "indexer_topk",
    "indexer_topk_noalloc",
)


class IndexerError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"[{code}] {message}")
        self.code = code


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() (hipcc, gfx950) first")
    L = ctypes.CDLL(LIB_PATH)
    P, I32, I64, F32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
    sig = {
        "indexer_fp4_last_error": ([], ctypes.c_char_p),
        "indexer_fp4_quant_and_cache": ([P, I64, I64, P, P, P, I64, P, I64, I32, P, P, P], ctypes.c_int),
        "indexer_fp4_norm_rope_quant_and_cache": ([P, I64, I64, P, P, F32, P, P, I64, I32, I32, P, P, P, I64, P, I32,
                                                   P, P, P, F32, P, I32, P, P], ctypes.c_int),
        "indexer_fp4_decode_sched_bytes": ([I32, I32, I32], I64),
        "indexer_fp4_decode_schedule": ([P, I32, I32, I32, P, I64, P, P], ctypes.c_int),
        "indexer_fp4_prefill_sched_bytes": ([I32, I32, I32, I64], I64),
        "indexer_fp4_prefill_schedule": ([P, P, I32, I32, I32, P, I64, I64, P, I64, P, P], ctypes.c_int),
        "indexer_fp4_score_decode": ([P, P, P, I32, P, P, I64, P, I64, I32, I32, P, I64, I32, P, P, I64, P, P],
                                     ctypes.c_int),
        "indexer_fp4_write_and_score_decode": ([P, I64, P, P, F32, P, P, I64, I32, I32, P, P, P, F32, I32, I32, P, P,
                                                I64, P, I64, I32, P, I64, I32, P, P, I64, P, P], ctypes.c_int),
        "indexer_fp4_score_prefill": ([P, P, P, I32, P, P, I64, I64, I32, P, I64, I32, I32, P, I64, P],
                                      ctypes.c_int),
        "indexer_fp8_quant_and_cache": ([P, I64, I64, P, P, P, I64, P, I64, I32, P, P, P], ctypes.c_int),
        "indexer_fp8_score_decode": ([P, P, P, I32, P, P, I64, P, I64, I32, I32, P, I64, I32, P, P, I64, P, P],
                                     ctypes.c_int),
        "indexer_topk_workspace_bytes": ([I32, I64, I32], I64),
        "indexer_topk": ([P, I64, I32, P, I64, I32, P, I64, P, I64, P, P], ctypes.c_int),
        "indexer_topk_merge": ([P, P, I64, I32, I32, I32, P, I64, P], ctypes.c_int),
        "indexer_topk_noalloc": ([P, I64, I32, P, I64, I32, P, I64, P, P], ctypes.c_int),
    }
    for name, (args, res) in sig.items():
        fn = getattr(L, name)
        fn.argtypes = args
        fn.restype = res
    return L


lib = _load()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _dev(t: torch.Tensor, name: str, dtype=None, contiguous=True):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a GPU tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _nbytes(t: torch.Tensor) -> int:
    return t.numel() * t.element_size()


def _check(rc: int):
    if rc != 0:
        raise IndexerError(rc, lib.indexer_fp4_last_error().decode())


def indexer_fp4_quant_and_cache(k, slot_mapping, kv_packed, kv_scale, q=None, q_packed=None, q_scale=None):
    """k: bf16 [n_tok, >=128] (row stride k.stride(0)); slot_mapping int64 [n_tok];
    kv_packed uint8 [n_pages, 64, 64]; kv_scale uint8 [n_pages, 4, 64];
    q: bf16 [rows, H, 128] or None -> q_packed uint8 [rows, H, 64], q_scale uint8 [rows, H, 4]."""
    _quant(lib.indexer_fp4_quant_and_cache, 64, k, slot_mapping, kv_packed, kv_scale, q, q_packed, q_scale)


def indexer_fp8_quant_and_cache(k, slot_mapping, kv_packed, kv_scale, q=None, q_packed=None, q_scale=None):
    """MXFP8 comparator writer: as indexer_fp4_quant_and_cache with kv_packed uint8
    [n_pages, 64, 128] and q_packed uint8 [rows, H, 128]."""
    _quant(lib.indexer_fp8_quant_and_cache, 128, k, slot_mapping, kv_packed, kv_scale, q, q_packed, q_scale)


def _quant(fn, vec_bytes, k, slot_mapping, kv_packed, kv_scale, q, q_packed, q_scale):
    if kv_packed.dim() != 3 or kv_packed.shape[1:] != (64, vec_bytes):
        raise ValueError(f"kv_packed must be [n_pages, 64, {vec_bytes}]")
    if q_packed is not None and q_packed.shape[-1] != vec_bytes:
        raise ValueError(f"q_packed rows must hold {vec_bytes} bytes")
    _dev(kv_packed, "kv_packed", torch.uint8)
    _dev(kv_scale, "kv_scale", torch.uint8)
    n_tok = 0 if k is None else k.shape[0]
    if k is not None:
        _dev(k, "k", torch.bfloat16, contiguous=False)
        if k.dim() != 2 or k.stride(1) != 1:
            raise ValueError("k must be 2-D with unit stride along the head dimension")
        _dev(slot_mapping, "slot_mapping", torch.int64)
    rows, heads = 0, 0
    if q is not None:
        _dev(q, "q", torch.bfloat16)
        rows, heads, d = q.shape
        if d != HEAD_DIM:
            raise ValueError("q must be [rows, heads, 128]")
        _dev(q_packed, "q_packed", torch.uint8)
        _dev(q_scale, "q_scale", torch.uint8)
    _check(fn(
        _ptr(k), n_tok, 0 if k is None else k.stride(0), _ptr(slot_mapping), _ptr(kv_packed), _ptr(kv_scale),
        kv_packed.shape[0], _ptr(q), rows, heads, _ptr(q_packed), _ptr(q_scale), _stream(kv_packed)))


def indexer_fp4_norm_rope_quant_and_cache(k, slot_mapping, kv_packed, kv_scale, positions=None, cos_sin=None,
                                          rope_dim=0, interleaved=False, k_norm_weight=None, k_norm_bias=None,
                                          eps=1e-6, q=None, q_packed=None, q_scale=None, weights=None,
                                          weight_scale=1.0, weights_mqa=None, all_q=False, err=None):
    """Fused writer: k [n_tok, >=128] bf16 -> LayerNorm (if k_norm_weight) -> RoPE (first rope_dim
    elements, cos_sin fp32 [max_pos, rope_dim]) -> MXFP4 cache write; q [n_tok, H, 128] bf16 ->
    RoPE -> q_packed/q_scale; weights_mqa = weight_scale * weights (fp32 [n_tok, H]).
    err: optional int32 [1] device word for the INDEXER_FP4_DEV_* flags."""
    _dev(k, "k", torch.bfloat16, contiguous=False)
    if k.dim() != 2 or k.stride(1) != 1:
        raise ValueError("k must be 2-D with unit stride along the head dimension")
    n_tok = k.shape[0]
    _dev(slot_mapping, "slot_mapping", torch.int64)
    _dev(kv_packed, "kv_packed", torch.uint8)
    _dev(kv_scale, "kv_scale", torch.uint8)
    max_pos = 0
    if rope_dim:
        _dev(positions, "positions", torch.int64)
        _dev(cos_sin, "cos_sin", torch.float32)
        if cos_sin.dim() != 2 or cos_sin.shape[1] != rope_dim:
            raise ValueError("cos_sin must be [max_pos, rope_dim]")
        max_pos = cos_sin.shape[0]
    for t, name in ((k_norm_weight, "k_norm_weight"), (k_norm_bias, "k_norm_bias")):
        if t is not None:
            _dev(t, name, torch.float32)
    heads = 0
    if q is not None:
        _dev(q, "q", torch.bfloat16)
        if q.dim() != 3 or q.shape[0] != n_tok or q.shape[2] != HEAD_DIM:
            raise ValueError("q must be [n_tok, heads, 128]")
        heads = q.shape[1]
        _dev(q_packed, "q_packed", torch.uint8)
        _dev(q_scale, "q_scale", torch.uint8)
        _dev(weights, "weights", torch.float32)
        _dev(weights_mqa, "weights_mqa", torch.float32)
    if err is not None:
        _dev(err, "err", torch.int32)
    _check(lib.indexer_fp4_norm_rope_quant_and_cache(
        _ptr(k), n_tok, k.stride(0), _ptr(k_norm_weight), _ptr(k_norm_bias), float(eps), _ptr(positions),
        _ptr(cos_sin), max_pos, int(rope_dim), int(bool(interleaved)), _ptr(slot_mapping), _ptr(kv_packed),
        _ptr(kv_scale), kv_packed.shape[0], _ptr(q), heads, _ptr(q_packed), _ptr(q_scale), _ptr(weights),
        float(weight_scale), _ptr(weights_mqa), int(bool(all_q)), _ptr(err), _stream(kv_packed)))


def indexer_fp4_decode_sched_bytes(batch: int, next_n: int, n_units: int) -> int:
    return int(lib.indexer_fp4_decode_sched_bytes(batch, next_n, n_units))


def indexer_fp4_prefill_sched_bytes(n_req: int, n_rows_padded: int, n_units: int, bt_ld: int) -> int:
    return int(lib.indexer_fp4_prefill_sched_bytes(n_req, n_rows_padded, n_units, bt_ld))


def indexer_fp4_decode_schedule(context_lens, next_n, n_units, sched, row_len):
    """context_lens int32 [B]; sched uint8/int32 buffer; row_len int32 [B*next_n] (outputs)."""
    _dev(context_lens, "context_lens", torch.int32)
    _dev(sched, "sched")
    _dev(row_len, "row_len", torch.int32)
    _check(lib.indexer_fp4_decode_schedule(
        _ptr(context_lens), context_lens.shape[0], next_n, n_units, _ptr(sched),
        sched.numel() * sched.element_size(), _ptr(row_len), _stream(sched)))


def indexer_fp4_prefill_schedule(cu_rows, start_pos, n_rows_padded, n_units, block_table, n_pages, sched, row_len):
    """cu_rows int32 [R+1], start_pos int32 [R], block_table int32 [R, bt_ld] (row i = request i);
    n_pages: pages of the cache planes the scorer reads. Outputs: sched, row_len int32 [n_rows_padded]."""
    _dev(cu_rows, "cu_rows", torch.int32)
    _dev(start_pos, "start_pos", torch.int32)
    _dev(block_table, "block_table", torch.int32)
    _dev(sched, "sched")
    _dev(row_len, "row_len", torch.int32)
    if block_table.dim() != 2 or block_table.shape[0] != start_pos.shape[0]:
        raise ValueError("block_table must be [n_req, bt_ld]")
    _check(lib.indexer_fp4_prefill_schedule(
        _ptr(cu_rows), _ptr(start_pos), start_pos.shape[0], n_rows_padded, n_units, _ptr(block_table),
        block_table.shape[1], int(n_pages), _ptr(sched), _nbytes(sched), _ptr(row_len), _stream(sched)))


def indexer_fp4_score_decode(q_packed, q_scale, weights, kv_packed, kv_scale, block_table, next_n, sched, n_units,
                             row_len, logits, row_hist=None):
    """q_packed [B*next_n, H, 64], q_scale [B*next_n, H, 4], weights fp32 [B*next_n, H],
    block_table int32 [B, W], logits fp32 [B*next_n, LD] (row stride logits.stride(0)).

    row_hist: optional int32 [B*next_n, 4096] (zero-filled before first use; see
    row_histogram) that the scorer fills for indexer_topk."""
    _score_decode(lib.indexer_fp4_score_decode, 64, q_packed, q_scale, weights, kv_packed, kv_scale, block_table,
                  next_n, sched, n_units, row_len, logits, row_hist)


def indexer_fp4_write_and_score_decode(k, slot_mapping, kv_packed, kv_scale, q, weights, block_table, sched, n_units,
                                       row_len, logits, positions=None, cos_sin=None, rope_dim=0, interleaved=False,
                                       k_norm_weight=None, k_norm_bias=None, eps=1e-6, weight_scale=1.0, all_q=False,
                                       row_hist=None):
    """The fused writer and the decode scorer in one launch (next_n = 1): k [B, >=128] bf16 and
    q [B, H, 128] bf16 with weights fp32 [B, H] are normalized, rotated and quantized as
    indexer_fp4_norm_rope_quant_and_cache does (each key to its slot), and the sequences'
    logits written as indexer_fp4_score_decode writes them from the quantized rows."""
    _dev(k, "k", torch.bfloat16, contiguous=False)
    if k.dim() != 2 or k.stride(1) != 1:
        raise ValueError("k must be 2-D with unit stride along the head dimension")
    for t, name, dt in ((slot_mapping, "slot_mapping", torch.int64), (kv_packed, "kv_packed", torch.uint8),
                        (kv_scale, "kv_scale", torch.uint8), (q, "q", torch.bfloat16),
                        (weights, "weights", torch.float32), (block_table, "block_table", torch.int32),
                        (row_len, "row_len", torch.int32)):
        _dev(t, name, dt)
    _dev(sched, "sched")
    _dev(logits, "logits", torch.float32, contiguous=False)
    if logits.stride(1) != 1:
        raise ValueError("logits rows must be contiguous")
    if kv_packed.dim() != 3 or kv_packed.shape[1:] != (64, 64):
        raise ValueError("kv_packed must be [n_pages, 64, 64]")
    batch, bt_ld = block_table.shape
    if q.dim() != 3 or q.shape[0] != batch or q.shape[2] != HEAD_DIM or k.shape[0] != batch:
        raise ValueError("q must be [B, H, 128] and k [B, >=128] for the table's B sequences")
    max_pos = 0
    if rope_dim:
        _dev(positions, "positions", torch.int64)
        _dev(cos_sin, "cos_sin", torch.float32)
        if cos_sin.dim() != 2 or cos_sin.shape[1] != rope_dim:
            raise ValueError("cos_sin must be [max_pos, rope_dim]")
        max_pos = cos_sin.shape[0]
    for t, name in ((k_norm_weight, "k_norm_weight"), (k_norm_bias, "k_norm_bias")):
        if t is not None:
            _dev(t, name, torch.float32)
    _check_hist(row_hist, batch)
    _check(lib.indexer_fp4_write_and_score_decode(
        _ptr(k), k.stride(0), _ptr(k_norm_weight), _ptr(k_norm_bias), float(eps), _ptr(positions), _ptr(cos_sin),
        max_pos, int(rope_dim), int(bool(interleaved)), _ptr(slot_mapping), _ptr(q), _ptr(weights),
        float(weight_scale), int(bool(all_q)), q.shape[1], _ptr(kv_packed), _ptr(kv_scale), kv_packed.shape[0],
        _ptr(block_table), bt_ld, batch, _ptr(sched), _nbytes(sched), n_units, _ptr(row_len), _ptr(logits),
        logits.stride(0), _ptr(row_hist), _stream(logits)))


def indexer_fp8_score_decode(q_packed, q_scale, weights, kv_packed, kv_scale, block_table, next_n, sched, n_units,
                             row_len, logits, row_hist=None):
    """MXFP8 comparator scorer: as indexer_fp4_score_decode over 128-byte vectors."""
    _score_decode(lib.indexer_fp8_score_decode, 128, q_packed, q_scale, weights, kv_packed, kv_scale, block_table,
                  next_n, sched, n_units, row_len, logits, row_hist)


def _score_decode(fn, vec_bytes, q_packed, q_scale, weights, kv_packed, kv_scale, block_table, next_n, sched,
                  n_units, row_len, logits, row_hist):
    if kv_packed.dim() != 3 or kv_packed.shape[1:] != (64, vec_bytes) or q_packed.shape[-1] != vec_bytes:
        raise ValueError(f"planes must hold {vec_bytes}-byte vectors")
    _dev(q_packed, "q_packed", torch.uint8)
    _dev(q_scale, "q_scale", torch.uint8)
    _dev(weights, "weights", torch.float32)
    _dev(kv_packed, "kv_packed", torch.uint8)
    _dev(kv_scale, "kv_scale", torch.uint8)
    _dev(block_table, "block_table", torch.int32)
    _dev(sched, "sched")
    _dev(row_len, "row_len", torch.int32)
    _dev(logits, "logits", torch.float32, contiguous=False)
    if logits.stride(1) != 1:
        raise ValueError("logits rows must be contiguous")
    batch, bt_ld = block_table.shape
    _check_hist(row_hist, batch * next_n)
    _check(fn(
        _ptr(q_packed), _ptr(q_scale), _ptr(weights), q_packed.shape[1], _ptr(kv_packed), _ptr(kv_scale),
        kv_packed.shape[0], _ptr(block_table), bt_ld, batch, next_n, _ptr(sched), _nbytes(sched), n_units,
        _ptr(row_len), _ptr(logits), logits.stride(0), _ptr(row_hist), _stream(logits)))


def indexer_fp4_score_prefill(q_packed, q_scale, weights, kv_packed, kv_scale, n_req, bt_ld, sched, n_units,
                              n_rows_padded, logits):
    """q/weights/logits have n_rows_padded rows; n_req, bt_ld, n_units, n_rows_padded and the cache's
    page count as given to indexer_fp4_prefill_schedule (which resolved the block table)."""
    _dev(q_packed, "q_packed", torch.uint8)
    _dev(q_scale, "q_scale", torch.uint8)
    _dev(weights, "weights", torch.float32)
    _dev(kv_packed, "kv_packed", torch.uint8)
    _dev(kv_scale, "kv_scale", torch.uint8)
    _dev(sched, "sched")
    _dev(logits, "logits", torch.float32, contiguous=False)
    if logits.stride(1) != 1:
        raise ValueError("logits rows must be contiguous")
    _check(lib.indexer_fp4_score_prefill(
        _ptr(q_packed), _ptr(q_scale), _ptr(weights), q_packed.shape[1], _ptr(kv_packed), _ptr(kv_scale),
        kv_packed.shape[0], int(bt_ld), int(n_req), _ptr(sched), _nbytes(sched), n_units, n_rows_padded,
        _ptr(logits), logits.stride(0), _stream(logits)))


HIST_BINS = 4096


def row_histogram(n_rows: int, device="cuda"):
    """A zeroed per-row histogram for indexer_fp4_score_decode / indexer_topk."""
    return torch.zeros(n_rows, HIST_BINS, dtype=torch.int32, device=device)


def _check_hist(row_hist, n_rows):
    if row_hist is None:
        return
    _dev(row_hist, "row_hist", torch.int32)
    if row_hist.numel() < n_rows * HIST_BINS:
        raise ValueError(f"row_hist holds {row_hist.numel()} words, needs {n_rows} x {HIST_BINS}")


def indexer_topk_workspace_bytes(n_rows: int, max_len: int, k: int) -> int:
    return int(lib.indexer_topk_workspace_bytes(n_rows, max_len, k))


def indexer_topk(logits, row_len, max_len, k, topk_idx, workspace=None, row_hist=None):
    """logits fp32 [rows, LD]; row_len int32 [rows]; topk_idx int32 [rows, >=k] (output).

    workspace: uint8 device buffer of indexer_topk_workspace_bytes(...) bytes, any contents
    (a call writes every word it reads first).
    row_hist: the histogram indexer_fp4_score_decode filled for these logits (left zeroed)."""
    _dev(logits, "logits", torch.float32, contiguous=False)
    _dev(row_len, "row_len", torch.int32)
    _dev(topk_idx, "topk_idx", torch.int32, contiguous=False)
    if logits.stride(1) != 1 or topk_idx.stride(1) != 1:
        raise ValueError("logits and topk_idx rows must be contiguous")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check_hist(row_hist, logits.shape[0])
    _check(lib.indexer_topk(
        _ptr(logits), logits.stride(0), logits.shape[0], _ptr(row_len), max_len, k, _ptr(topk_idx),
        topk_idx.stride(0), _ptr(workspace), ws_bytes, _ptr(row_hist), _stream(logits)))


NOALLOC_SCRATCH_BYTES = 32 << 20


def indexer_topk_noalloc(logits, row_len, max_len, k, topk_idx, row_hist=None):
    """indexer_topk with the library's fixed per-GPU scratch array instead of a workspace
    (allocates nothing; calls that overlap on one GPU race)."""
    _dev(logits, "logits", torch.float32, contiguous=False)
    _dev(row_len, "row_len", torch.int32)
    _dev(topk_idx, "topk_idx", torch.int32, contiguous=False)
    if logits.stride(1) != 1 or topk_idx.stride(1) != 1:
        raise ValueError("logits and topk_idx rows must be contiguous")
    _check_hist(row_hist, logits.shape[0])
    _check(lib.indexer_topk_noalloc(
        _ptr(logits), logits.stride(0), logits.shape[0], _ptr(row_len), max_len, k, _ptr(topk_idx),
        topk_idx.stride(0), _ptr(row_hist), _stream(logits)))


def indexer_topk_merge(cand_score, cand_index, k, topk_idx):
    """cand_score fp32 [rows, C], cand_index int32 [rows, C] (< 0: empty slot);
    topk_idx int32 [rows, >=k] (output): the k best candidates' indices, ascending."""
    _dev(cand_score, "cand_score", torch.float32)
    _dev(cand_index, "cand_index", torch.int32)
    _dev(topk_idx, "topk_idx", torch.int32, contiguous=False)
    if cand_score.shape != cand_index.shape:
        raise ValueError("cand_score and cand_index must have the same shape")
    if topk_idx.stride(1) != 1:
        raise ValueError("topk_idx rows must be contiguous")
    rows, n = cand_score.shape
    _check(lib.indexer_topk_merge(_ptr(cand_score), _ptr(cand_index), n, rows, n, k, _ptr(topk_idx),
                                  topk_idx.stride(0), _stream(cand_score)))


# ---- schedule-buffer inspection (host copies; for tests and diagnostics) -----------------

def sched_error(sched) -> int:
    """Device-side error flags of a schedule buffer (synchronizes)."""
    return int(sched.view(torch.int32)[1].item())


def read_decode_schedule(sched, batch: int, n_units: int) -> dict:
    w = sched.view(torch.int32).cpu().numpy()
    cum = 8
    ub = cum + batch + 1
    us = ub + n_units + 1
    up = us + n_units
    ur = up + n_units
    return {"header": w[:8].copy(), "cum_pages": w[cum:cum + batch + 1].copy(),
            "unit_begin": w[ub:ub + n_units + 1].copy(), "unit_seq": w[us:us + n_units].copy(),
            "unit_page": w[up:up + n_units].copy(), "unit_run": w[ur:ur + n_units].copy()}


def read_prefill_schedule(sched, n_req: int, n_rows_padded: int, n_units: int, bt_ld: int) -> dict:
    """Host copy of a prefill schedule: tiles as {first row, rows, request, pages} (the
    oracle's fields) plus the library's own per-tile, per-unit and per-item words."""
    w = sched.view(torch.int32).cpu().numpy()
    max_tiles = n_rows_padded // TILE_ROWS + n_req
    urec = 16
    tiles = urec + 16 * n_units
    cum = tiles + 8 * max_tiles
    ub = cum + max_tiles + 1
    ut = ub + n_units + 1
    rt = ut + n_units
    ip = rt + n_req + 1
    n_tiles, items = int(w[5]), int(w[6])
    t8 = w[tiles:tiles + 8 * n_tiles].reshape(n_tiles, 8).copy()
    return {"header": w[:16].copy(), "tiles": t8[:, [0, 1, 4, 5]].copy(), "tile_words": t8,
            "cum_items": w[cum:cum + n_tiles + 1].copy(), "unit_begin": w[ub:ub + n_units + 1].copy(),
            "unit_tile": w[ut:ut + n_units].copy(), "unit_records": w[urec:tiles].reshape(n_units, 16).copy(),
            "item_phys": w[ip:ip + items].copy()}
