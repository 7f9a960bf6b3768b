"""Python binding of libdsa (MI355X / gfx950 DSA layer).

Argument marshalling only: every step of the layer runs in the HIP kernels of
libdsa.so, which this module loads from the package directory.  There is no
fallback: if the library is missing or a call fails, an exception is raised.
PyTorch supplies device memory and the stream.

Entry points (same names as include/dsa.h):
    dsa_indexer_scores, dsa_topk, dsa_translate_pages,
    sparse_mla_decode, sparse_mla_prefill, dsa_workspace_size,
    dsa_quantize_q, dsa_cache_insert (the step's front end)
plus `decode_step`, which chains them for one layer step.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdsa.so")
# the debug build (DSA_DEBUG=1): same entry points, plus device notes of the
# metadata the kernels clamped or skipped (check_debug_flag)
DEBUG_LIB_PATH = os.path.join(_HERE, "libdsa_debug.so")
DEBUG_VIS_CLAMPED, DEBUG_ABSENT_PAGE, DEBUG_ROW_OUTSIDE, DEBUG_REQ_OUTSIDE = 1, 2, 4, 8

DSA_OK, DSA_ERR_INVALID_ARG, DSA_ERR_UNSUPPORTED, DSA_ERR_WORKSPACE, DSA_ERR_HIP = range(5)
KEY_FP8, KEY_MXFP4, KEY_NVFP4 = 1, 2, 3
LAT_BF16, LAT_FP8, LAT_NVFP4 = 1, 2, 3
Q_BF16, Q_FP8, Q_MXFP4 = 1, 2, 3
OP_INDEXER, OP_TOPK, OP_MLA_DECODE, OP_MLA_PREFILL, OP_TOPK_SHARDED, OP_MSA_DECODE = 1, 2, 3, 4, 5, 6
OP_INDEXER_PREFIX = 7

KEY_FMT = {"fp8": KEY_FP8, "mxfp4": KEY_MXFP4, "nvfp4": KEY_NVFP4}
LAT_FMT = {"bf16": LAT_BF16, "fp8": LAT_FP8, "nvfp4": LAT_NVFP4}
Q_FMT = {"bf16": Q_BF16, "fp8": Q_FP8, "mxfp4": Q_MXFP4}
KEY_TOKEN_BYTES = {KEY_FP8: 132, KEY_MXFP4: 68, KEY_NVFP4: 72}
LAT_TOKEN_BYTES = {LAT_BF16: 1152, LAT_FP8: 580, LAT_NVFP4: 352}   # data bytes per token
LAT_ROW_BYTES = {LAT_BF16: 1152, LAT_FP8: 640, LAT_NVFP4: 384}     # bytes per latent row in a page

EXPORTS = ("dsa_indexer_scores", "dsa_topk", "dsa_translate_pages", "sparse_mla_decode",
           "sparse_mla_prefill", "dsa_workspace_size", "dsa_status_str", "dsa_last_error",
           "dsa_abi_version", "dsa_quantize_q", "dsa_cache_insert", "dsa_topk_sharded",
           "dsa_msa_decode", "dsa_indexer_scores_prefix", "sparse_mla_decode_noalloc",
           "dsa_check_debug_flag")


class DsaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{message} (status {status})")
        self.status = status


class Cache(ctypes.Structure):
    _fields_ = [("base", ctypes.c_void_p), ("page_bytes", ctypes.c_int64),
                ("page_size_log2", ctypes.c_int32), ("num_pages", ctypes.c_int32),
                ("fmt", ctypes.c_int32)]


class Batch(ctypes.Structure):
    _fields_ = [("num_requests", ctypes.c_int32), ("num_rows", ctypes.c_int32),
                ("req_row_start", ctypes.c_void_p), ("tok_req", ctypes.c_void_p),
                ("tok_vis", ctypes.c_void_p), ("block_table", ctypes.c_void_p),
                ("bt_stride", ctypes.c_int32), ("max_vis", ctypes.c_int32),
                ("max_rows_per_req", ctypes.c_int32)]


class IndexerArgs(ctypes.Structure):
    _fields_ = [("batch", Batch), ("keys", Cache), ("q", ctypes.c_void_p),
                ("q_fmt", ctypes.c_int32), ("q_scale", ctypes.c_void_p),
                ("w", ctypes.c_void_p), ("scores", ctypes.c_void_p), ("ld", ctypes.c_int64)]


class IndexerPrefixArgs(ctypes.Structure):
    _fields_ = [("base", IndexerArgs), ("num_groups", ctypes.c_int32), ("group_row_start", ctypes.c_void_p),
                ("group_first_req", ctypes.c_void_p), ("prefix_len", ctypes.c_int32),
                ("max_rows_per_group", ctypes.c_int32), ("workspace", ctypes.c_void_p),
                ("workspace_bytes", ctypes.c_size_t)]


class TopkArgs(ctypes.Structure):
    _fields_ = [("batch", Batch), ("scores", ctypes.c_void_p), ("ld", ctypes.c_int64),
                ("k", ctypes.c_int32), ("idx", ctypes.c_void_p), ("rows", ctypes.c_void_p),
                ("page_size_log2", ctypes.c_int32), ("num_pages", ctypes.c_int32), ("count", ctypes.c_void_p),
                ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t)]


class TopkShardedArgs(ctypes.Structure):
    _fields_ = [("num_rows", ctypes.c_int32), ("num_shards", ctypes.c_int32), ("scores", ctypes.c_void_p),
                ("ld", ctypes.c_int64), ("tok_vis", ctypes.c_void_p), ("max_vis", ctypes.c_int32),
                ("k", ctypes.c_int32), ("cand", ctypes.c_int32), ("idx", ctypes.c_void_p),
                ("count", ctypes.c_void_p), ("resend", ctypes.c_void_p), ("workspace", ctypes.c_void_p),
                ("workspace_bytes", ctypes.c_size_t)]


class MsaArgs(ctypes.Structure):
    _fields_ = [("batch", Batch), ("index_keys", ctypes.c_void_p), ("kv", ctypes.c_void_p),
                ("num_blocks", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
                ("top_blocks", ctypes.c_int32), ("q_idx", ctypes.c_void_p), ("q", ctypes.c_void_p),
                ("k_scale", ctypes.c_float), ("v_scale", ctypes.c_float), ("sm_scale", ctypes.c_float),
                ("sel_blocks", ctypes.c_void_p), ("out", ctypes.c_void_p), ("lse", ctypes.c_void_p),
                ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t)]


class MlaArgs(ctypes.Structure):
    _fields_ = [("num_rows", ctypes.c_int32), ("num_heads", ctypes.c_int32),
                ("q", ctypes.c_void_p), ("latents", Cache), ("rows", ctypes.c_void_p),
                ("k", ctypes.c_int32), ("sm_scale", ctypes.c_float),
                ("num_splits", ctypes.c_int32), ("out", ctypes.c_void_p),
                ("lse", ctypes.c_void_p), ("workspace", ctypes.c_void_p),
                ("workspace_bytes", ctypes.c_size_t)]


class QuantQArgs(ctypes.Structure):
    _fields_ = [("num_rows", ctypes.c_int32), ("q", ctypes.c_void_p), ("w", ctypes.c_void_p),
                ("fmt", ctypes.c_int32), ("q_out", ctypes.c_void_p), ("q_scale", ctypes.c_void_p),
                ("w_folded", ctypes.c_void_p)]


class InsertArgs(ctypes.Structure):
    _fields_ = [("num_tokens", ctypes.c_int32), ("num_requests", ctypes.c_int32),
                ("tok_req", ctypes.c_void_p), ("tok_pos", ctypes.c_void_p),
                ("block_table", ctypes.c_void_p), ("bt_stride", ctypes.c_int32),
                ("key_vals", ctypes.c_void_p), ("keys", Cache),
                ("lat_vals", ctypes.c_void_p), ("latents", Cache)]


_lib = None


def load(path: str | None = None) -> ctypes.CDLL:
    """Load libdsa.so (raises if it has not been built).  The environment
    variable DSA_DEBUG_LIB=1 selects libdsa_debug.so instead, and DSA_LIB=path
    any other build of the library; one process holds one library."""
    global _lib
    if _lib is not None:
        return _lib
    if path is None:
        path = os.environ.get("DSA_LIB") or (DEBUG_LIB_PATH if os.environ.get("DSA_DEBUG_LIB") == "1" else LIB_PATH)
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m sparse_attention_03_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i32 = ctypes.c_void_p, ctypes.c_int32
    for name, argt in (("dsa_indexer_scores", [ctypes.POINTER(IndexerArgs), vp]),
                       ("dsa_topk", [ctypes.POINTER(TopkArgs), vp]),
                       ("sparse_mla_decode", [ctypes.POINTER(MlaArgs), vp]),
                       ("sparse_mla_prefill", [ctypes.POINTER(MlaArgs), vp]),
                       ("sparse_mla_decode_noalloc", [ctypes.POINTER(MlaArgs), vp]),
                       ("dsa_translate_pages", [vp, i32, ctypes.POINTER(Batch), i32, i32, vp, vp]),
                       ("dsa_quantize_q", [ctypes.POINTER(QuantQArgs), vp]),
                       ("dsa_cache_insert", [ctypes.POINTER(InsertArgs), vp]),
                       ("dsa_topk_sharded", [ctypes.POINTER(TopkShardedArgs), vp]),
                       ("dsa_msa_decode", [ctypes.POINTER(MsaArgs), vp]),
                       ("dsa_indexer_scores_prefix", [ctypes.POINTER(IndexerPrefixArgs), vp])):
        f = getattr(lib, name)
        f.argtypes = argt
        f.restype = ctypes.c_int
    lib.dsa_workspace_size.argtypes = [i32, vp]
    lib.dsa_workspace_size.restype = ctypes.c_size_t
    lib.dsa_status_str.argtypes = [ctypes.c_int]
    lib.dsa_status_str.restype = ctypes.c_char_p
    lib.dsa_last_error.argtypes = []
    lib.dsa_last_error.restype = ctypes.c_char_p
    lib.dsa_abi_version.argtypes = []
    lib.dsa_abi_version.restype = ctypes.c_int32
    lib.dsa_check_debug_flag.argtypes = []
    lib.dsa_check_debug_flag.restype = ctypes.c_int32
    _lib = lib
    return lib


def _check(status: int, what: str):
    if status != DSA_OK:
        lib = load()
        raise DsaError(status, f"{what}: {lib.dsa_status_str(status).decode()}: {lib.dsa_last_error().decode()}")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


# ------------------------------------------------------------ views
def cache_view(pool: torch.Tensor, page_size: int, fmt: int, page_bytes: Optional[int] = None) -> Cache:
    """A paged pool stored as a uint8 tensor [num_pages, page_bytes]."""
    assert pool.dtype == torch.uint8 and pool.dim() == 2 and pool.is_contiguous()
    assert page_size & (page_size - 1) == 0
    return Cache(pool.data_ptr(), int(page_bytes or pool.shape[1]), page_size.bit_length() - 1,
                 int(pool.shape[0]), int(fmt))


def batch_view(req_row_start: torch.Tensor, tok_req: torch.Tensor, tok_vis: torch.Tensor,
               block_table: Optional[torch.Tensor], max_vis: int, max_rows_per_req: int) -> Batch:
    for t in (req_row_start, tok_req, tok_vis):
        assert t.dtype == torch.int32 and t.is_contiguous()
    bt_stride = 0
    if block_table is not None:
        assert block_table.dtype == torch.int32 and block_table.is_contiguous()
        bt_stride = int(block_table.shape[1])
    return Batch(int(req_row_start.numel() - 1), int(tok_vis.numel()), req_row_start.data_ptr(),
                 tok_req.data_ptr(), tok_vis.data_ptr(), _ptr(block_table), bt_stride,
                 int(max_vis), int(max_rows_per_req))


# ------------------------------------------------------------ entry points
def dsa_indexer_scores(args: IndexerArgs, stream=None):
    _check(load().dsa_indexer_scores(ctypes.byref(args), _stream(stream)), "dsa_indexer_scores")


def dsa_indexer_scores_prefix(args: IndexerPrefixArgs, stream=None):
    _check(load().dsa_indexer_scores_prefix(ctypes.byref(args), _stream(stream)), "dsa_indexer_scores_prefix")


def indexer_prefix_args(base: IndexerArgs, group_row_start: torch.Tensor, group_first_req: torch.Tensor,
                        prefix_len: int, max_rows_per_group: int, device) -> tuple:
    """(IndexerPrefixArgs, workspace tensor) for dsa_indexer_scores_prefix."""
    for t in (group_row_start, group_first_req):
        assert t.dtype == torch.int32 and t.is_contiguous()
    a = IndexerPrefixArgs(base, int(group_first_req.numel()), group_row_start.data_ptr(),
                          group_first_req.data_ptr(), int(prefix_len), int(max_rows_per_group), None, 0)
    ws = workspace(dsa_workspace_size(OP_INDEXER_PREFIX, a), device)
    a.workspace = _ptr(ws)
    a.workspace_bytes = 0 if ws is None else ws.numel()
    return a, ws


def dsa_topk(args: TopkArgs, stream=None):
    _check(load().dsa_topk(ctypes.byref(args), _stream(stream)), "dsa_topk")


def dsa_translate_pages(idx: torch.Tensor, k: int, batch: Batch, page_size_log2: int, num_pages: int,
                        rows: torch.Tensor, stream=None):
    _check(load().dsa_translate_pages(idx.data_ptr(), int(k), ctypes.byref(batch), int(page_size_log2),
                                      int(num_pages), rows.data_ptr(), _stream(stream)), "dsa_translate_pages")


def dsa_check_debug_flag() -> int:
    """Bits (DEBUG_*) the debug library's kernels noted since the last call,
    cleared; waits for the device.  -1 from the release library."""
    return int(load().dsa_check_debug_flag())


def sparse_mla_decode(args: MlaArgs, stream=None):
    _check(load().sparse_mla_decode(ctypes.byref(args), _stream(stream)), "sparse_mla_decode")


def sparse_mla_prefill(args: MlaArgs, stream=None):
    _check(load().sparse_mla_prefill(ctypes.byref(args), _stream(stream)), "sparse_mla_prefill")


def sparse_mla_decode_noalloc(args: MlaArgs, stream=None):
    """sparse_mla_decode with the split partials in the library's own device
    scratch (args.workspace is ignored); nothing is allocated."""
    _check(load().sparse_mla_decode_noalloc(ctypes.byref(args), _stream(stream)), "sparse_mla_decode_noalloc")


def dsa_quantize_q(args: QuantQArgs, stream=None):
    _check(load().dsa_quantize_q(ctypes.byref(args), _stream(stream)), "dsa_quantize_q")


def dsa_cache_insert(args: InsertArgs, stream=None):
    _check(load().dsa_cache_insert(ctypes.byref(args), _stream(stream)), "dsa_cache_insert")


def dsa_topk_sharded(args: TopkShardedArgs, stream=None):
    _check(load().dsa_topk_sharded(ctypes.byref(args), _stream(stream)), "dsa_topk_sharded")


def dsa_msa_decode(args: MsaArgs, stream=None):
    _check(load().dsa_msa_decode(ctypes.byref(args), _stream(stream)), "dsa_msa_decode")


def dsa_workspace_size(op: int, args) -> int:
    return int(load().dsa_workspace_size(int(op), ctypes.cast(ctypes.byref(args), ctypes.c_void_p)))


# ------------------------------------------------------------ convenience
def workspace(nbytes: int, device) -> Optional[torch.Tensor]:
    """Caller-owned workspace (256-byte aligned by the torch allocator)."""
    if nbytes == 0:
        return None
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def indexer_args(batch: Batch, keys: Cache, q: torch.Tensor, w: torch.Tensor, scores: torch.Tensor,
                 q_scale: Optional[torch.Tensor] = None) -> IndexerArgs:
    """q: bf16 [T,32,128]; E4M3 codes uint8 [T,32,128] with fp32 q_scale [T,32];
    or E2M1 pairs uint8 [T,32,64] with E8M0 q_scale uint8 [T,32,4]."""
    if q.dtype == torch.bfloat16:
        q_fmt = Q_BF16
    else:
        assert q.dtype == torch.uint8 and q_scale is not None
        q_fmt = Q_FP8 if q.shape[-1] == 128 else Q_MXFP4
    return IndexerArgs(batch, keys, q.data_ptr(), q_fmt, _ptr(q_scale), w.data_ptr(),
                       scores.data_ptr(), int(scores.stride(0)))


def topk_args(batch: Batch, scores: torch.Tensor, k: int, idx: torch.Tensor,
              rows: Optional[torch.Tensor] = None, page_size_log2: int = 0, num_pages: int = 0,
              count: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None) -> TopkArgs:
    return TopkArgs(batch, scores.data_ptr(), int(scores.stride(0)), int(k), idx.data_ptr(), _ptr(rows),
                    int(page_size_log2), int(num_pages), _ptr(count), _ptr(ws), 0 if ws is None else ws.numel())


def mla_args(q: torch.Tensor, latents: Cache, rows: torch.Tensor, out: torch.Tensor,
             lse: Optional[torch.Tensor], sm_scale: float, num_splits: int = 0,
             ws: Optional[torch.Tensor] = None) -> MlaArgs:
    T, H, _ = q.shape
    return MlaArgs(int(T), int(H), q.data_ptr(), latents, rows.data_ptr(), int(rows.shape[1]),
                   float(sm_scale), int(num_splits), out.data_ptr(), _ptr(lse), _ptr(ws),
                   0 if ws is None else ws.numel())


def quantize_q(q: torch.Tensor, w: Optional[torch.Tensor] = None, fmt: str = "fp8", fold: bool = False,
               stream=None):
    """Index-query quantisation (dsa_quantize_q) into new tensors.  FP8:
    returns (codes uint8 [T,32,128], scale fp32 [T,32], w_folded fp32 [T,32]
    or None); MXFP4: (codes uint8 [T,32,64], E8M0 uint8 [T,32,4], None)."""
    assert q.dtype == torch.bfloat16 and q.is_contiguous() and q.shape[1:] == (32, 128)
    T, dev = int(q.shape[0]), q.device
    if fmt == "fp8":
        out = torch.empty(T, 32, 128, dtype=torch.uint8, device=dev)
        scale = torch.empty(T, 32, dtype=torch.float32, device=dev)
    else:
        out = torch.empty(T, 32, 64, dtype=torch.uint8, device=dev)
        scale = torch.empty(T, 32, 4, dtype=torch.uint8, device=dev)
    wf = torch.empty(T, 32, dtype=torch.float32, device=dev) if fold else None
    dsa_quantize_q(QuantQArgs(T, q.data_ptr(), _ptr(w), Q_FMT[fmt], out.data_ptr(), scale.data_ptr(), _ptr(wf)),
                   stream)
    return out, scale, wf


def cache_insert(tok_req: torch.Tensor, tok_pos: torch.Tensor, num_requests: int,
                 block_table: Optional[torch.Tensor], page_size: int,
                 key_vals: Optional[torch.Tensor] = None, key_pool: Optional[torch.Tensor] = None,
                 key_fmt: str = "fp8", lat_vals: Optional[torch.Tensor] = None,
                 lat_pool: Optional[torch.Tensor] = None, lat_fmt: str = "fp8", stream=None):
    """Write new tokens' keys / latents (bf16) into the pools (dsa_cache_insert)."""
    for t in (tok_req, tok_pos):
        assert t.dtype == torch.int32 and t.is_contiguous()
    bt_stride = 0
    if block_table is not None:
        assert block_table.dtype == torch.int32 and block_table.is_contiguous()
        bt_stride = int(block_table.shape[1])
    keys = cache_view(key_pool, page_size, KEY_FMT[key_fmt]) if key_pool is not None else Cache()
    lats = cache_view(lat_pool, page_size, LAT_FMT[lat_fmt]) if lat_pool is not None else Cache()
    for v, d in ((key_vals, 128), (lat_vals, 576)):
        assert v is None or (v.dtype == torch.bfloat16 and v.is_contiguous() and v.shape[-1] == d)
    dsa_cache_insert(InsertArgs(int(tok_req.numel()), int(num_requests), tok_req.data_ptr(), tok_pos.data_ptr(),
                                _ptr(block_table), bt_stride, _ptr(key_vals), keys, _ptr(lat_vals), lats), stream)


class ShardedTopk:
    """The sharded top-k merge (dsa_topk_sharded) over fixed buffers: local
    scores [W, T, ld] fp32 in the interleaved shard layout."""

    def __init__(self, scores: torch.Tensor, tok_vis: torch.Tensor, max_vis: int, k: int, cand: int = 0):
        assert scores.dtype == torch.float32 and scores.dim() == 3 and scores.is_contiguous()
        assert tok_vis.dtype == torch.int32 and tok_vis.is_contiguous()
        W, T, ld = (int(x) for x in scores.shape)
        dev = scores.device
        self.idx = torch.empty(T, k, dtype=torch.int32, device=dev)
        self.count = torch.empty(T, dtype=torch.int32, device=dev)
        self.resend = torch.empty(T, W, dtype=torch.int32, device=dev)
        self.args = TopkShardedArgs(T, W, scores.data_ptr(), ld, tok_vis.data_ptr(), int(max_vis), int(k),
                                    int(cand), self.idx.data_ptr(), self.count.data_ptr(),
                                    self.resend.data_ptr(), None, 0)
        self.ws = workspace(dsa_workspace_size(OP_TOPK_SHARDED, self.args), dev)
        self.args.workspace = _ptr(self.ws)
        self.args.workspace_bytes = 0 if self.ws is None else self.ws.numel()

    def __call__(self, stream=None):
        dsa_topk_sharded(self.args, stream)
        return self.idx, self.count, self.resend


def topk_sharded(scores: torch.Tensor, tok_vis: torch.Tensor, max_vis: int, k: int, cand: int = 0,
                 stream=None):
    """One call of dsa_topk_sharded into new tensors: (idx [T,k], count [T],
    resend flags [T,W])."""
    return ShardedTopk(scores, tok_vis, max_vis, k, cand)(stream)


class MsaDecode:
    """The MSA block-sparse decode step (dsa_msa_decode) over fixed buffers.
    idx_pool uint8 [blocks, 128*128]; kv_pool uint8 [blocks, 128*2*Hkv*128];
    block_table int32 [R, nblk]; q_idx bf16 [T, Hkv, 128]; q bf16 [T, Hq, 128]."""

    def __init__(self, *, req_row_start, tok_req, tok_vis, block_table, idx_pool, kv_pool, q_idx, q,
                 max_vis: int, max_rows_per_req: int, top_blocks: int = 16, k_scale: float = 1.0,
                 v_scale: float = 1.0, sm_scale: Optional[float] = None):
        dev = q.device
        T, hq, _ = q.shape
        hkv = int(q_idx.shape[1])
        for t in (idx_pool, kv_pool, q_idx, q):
            assert t.is_contiguous()
        self.batch = batch_view(req_row_start, tok_req, tok_vis, block_table, max_vis, max_rows_per_req)
        self.sel = torch.empty(T, hkv, top_blocks, dtype=torch.int32, device=dev)
        self.out = torch.empty(T, hq, 128, dtype=torch.float32, device=dev)
        self.lse = torch.empty(T, hq, dtype=torch.float32, device=dev)
        sm = 1.0 / 128 ** 0.5 if sm_scale is None else sm_scale
        self.args = MsaArgs(self.batch, idx_pool.data_ptr(), kv_pool.data_ptr(), int(idx_pool.shape[0]), hkv,
                            int(hq), int(top_blocks), q_idx.data_ptr(), q.data_ptr(), float(k_scale),
                            float(v_scale), float(sm), self.sel.data_ptr(), self.out.data_ptr(),
                            self.lse.data_ptr(), None, 0)
        self.ws = workspace(dsa_workspace_size(OP_MSA_DECODE, self.args), dev)
        self.args.workspace = _ptr(self.ws)
        self.args.workspace_bytes = 0 if self.ws is None else self.ws.numel()
        self._keep = (req_row_start, tok_req, tok_vis, block_table, idx_pool, kv_pool, q_idx, q)

    def __call__(self, stream=None):
        dsa_msa_decode(self.args, stream)
        return self.sel, self.out, self.lse


class DecodeStep:
    """One DSA layer step (indexer -> top-k with fused translation -> sparse
    MLA) over fixed buffers; every stage is one libdsa call on one stream."""

    def __init__(self, *, batch: Batch, keys: Cache, latents: Cache, q_idx: torch.Tensor,
                 w: torch.Tensor, q_mla: torch.Tensor, k: int, sm_scale: float,
                 q_idx_scale: Optional[torch.Tensor] = None, prefill: bool = False,
                 num_splits: int = 0):
        dev = q_mla.device
        T, H, _ = q_mla.shape
        self.T, self.H, self.k, self.prefill = T, H, k, prefill
        ld = (batch.max_vis + 3) // 4 * 4
        self.scores = torch.empty(T, ld, dtype=torch.float32, device=dev)
        self.idx = torch.empty(T, k, dtype=torch.int32, device=dev)
        self.rows = torch.empty(T, k, dtype=torch.int32, device=dev)
        self.count = torch.empty(T, dtype=torch.int32, device=dev)
        self.out = torch.empty(T, H, 512, dtype=torch.float32, device=dev)
        self.lse = torch.empty(T, H, dtype=torch.float32, device=dev)
        self.iargs = indexer_args(batch, keys, q_idx, w, self.scores, q_idx_scale)
        self.targs = topk_args(batch, self.scores, k, self.idx, self.rows, latents.page_size_log2,
                               latents.num_pages, self.count)
        self.tws = workspace(dsa_workspace_size(OP_TOPK, self.targs), dev)
        self.targs = topk_args(batch, self.scores, k, self.idx, self.rows, latents.page_size_log2,
                               latents.num_pages, self.count, self.tws)
        self.margs = mla_args(q_mla, latents, self.rows, self.out, self.lse, sm_scale, num_splits)
        op = OP_MLA_PREFILL if prefill else OP_MLA_DECODE
        self.mws = workspace(dsa_workspace_size(op, self.margs), dev)
        self.margs = mla_args(q_mla, latents, self.rows, self.out, self.lse, sm_scale, num_splits, self.mws)
        self._keep = (q_idx, w, q_mla, q_idx_scale)

    def indexer(self, stream=None):
        dsa_indexer_scores(self.iargs, stream)

    def topk(self, stream=None):
        dsa_topk(self.targs, stream)

    def mla(self, stream=None):
        (sparse_mla_prefill if self.prefill else sparse_mla_decode)(self.margs, stream)

    def __call__(self, stream=None):
        self.indexer(stream)
        self.topk(stream)
        self.mla(stream)
        return self.out, self.lse


def make_step(*, key_pool: torch.Tensor, lat_pool: torch.Tensor, page_size: int, key_fmt: str,
              lat_fmt: str, req_row_start: torch.Tensor, tok_req: torch.Tensor, tok_vis: torch.Tensor,
              block_table: Optional[torch.Tensor], q_idx: torch.Tensor, w: torch.Tensor,
              q_mla: torch.Tensor, k: int, sm_scale: float, q_idx_scale: Optional[torch.Tensor] = None,
              prefill: bool = False, num_splits: int = 0, max_vis: Optional[int] = None,
              max_rows_per_req: Optional[int] = None) -> DecodeStep:
    """Build a DecodeStep from paged pools (uint8 [pages, page_bytes]) and
    per-row metadata tensors, all on the GPU."""
    if max_vis is None:
        max_vis = int(tok_vis.max())
    if max_rows_per_req is None:
        max_rows_per_req = int((req_row_start[1:] - req_row_start[:-1]).max())
    batch = batch_view(req_row_start, tok_req, tok_vis, block_table, max_vis, max_rows_per_req)
    keys = cache_view(key_pool, page_size, KEY_FMT[key_fmt])
    lats = cache_view(lat_pool, page_size, LAT_FMT[lat_fmt])
    return DecodeStep(batch=batch, keys=keys, latents=lats, q_idx=q_idx, w=w, q_mla=q_mla, k=k,
                      sm_scale=sm_scale, q_idx_scale=q_idx_scale, prefill=prefill, num_splits=num_splits)
