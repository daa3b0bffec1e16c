"""NVFP4-compressed sparse MLA decode for MI355X (gfx950).

Thin Python binding over the C ABI in include/mla_nvfp4.h: it checks
tensor shapes and dtypes and passes device pointers and the current HIP
stream.  Every step of the computation runs in the library's HIP kernels;
PyTorch only provides device memory and streams.

    quantize_append(latent, rope, slots, cache)        352-byte NVFP4 rows
    quantize_append_2level(..., global_scale)          two-level NVFP4 rows
    fp8_quantize_append(latent, rope, slots, cache)    576-byte FP8 rows
    sparse_decode(q, cache, indices, sm_scale, ...)    -> (out, lse)
    sparse_decode_noalloc(q, cache, indices, ...)      the same without a workspace
    gather_dequant_fp8(cache, indices, ...)            staged comparator step
    indexer_topk(q_idx, keys, ctx_len, topk, ...)      the sparse indexer's lists
    Pool(budget, layers, ...)                          paged pool: capacity, blocks, tables
    kv_pack_blocks / kv_unpack_blocks                  a request's blocks <-> staging buffer
"""

from __future__ import annotations

import torch

from ._lib import MlaError, check, load  # noqa: F401

LATENT_DIM = 512
ROPE_DIM = 64
QK_DIM = 576
NVFP4_ROW_BYTES = 352
FP8_ROW_BYTES = 576
MAX_TOPK = 2048

F16, BF16 = 0, 1
FMT_NVFP4, FMT_FP8 = 0, 1
_FMT = {"nvfp4": FMT_NVFP4, "fp8": FMT_FP8}


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float16:
        return F16
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"expected float16 or bfloat16, got {t.dtype}")


def _stream(t: torch.Tensor):
    return torch.cuda.current_stream(t.device).cuda_stream


def _ptr(t):
    return None if t is None else t.data_ptr()


def _rows2d(x: torch.Tensor, width: int, name: str) -> torch.Tensor:
    if x.dim() != 2 or x.shape[1] != width or x.stride(1) != 1:
        raise ValueError(f"{name} must be [n, {width}] with unit column stride")
    return x


def _device_of(t: torch.Tensor, name: str) -> torch.device:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a tensor in GPU memory")
    return t.device


def _same_device(dev: torch.device, **tensors) -> None:
    """Every given tensor (None = absent) lives on the GPU `dev`."""
    for name, t in tensors.items():
        if t is not None and (not isinstance(t, torch.Tensor) or t.device != dev):
            raise ValueError(f"{name} must be on {dev} like the other arguments")


def _exact(t: torch.Tensor, name: str, shape, dtype) -> None:
    """A contiguous tensor of exactly this shape and dtype (the library writes
    it densely and takes no strides for it)."""
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {dtype} tensor of shape {tuple(shape)}, "
                         f"got {t.dtype} {tuple(t.shape)}")


def _cache_tensor(cache: torch.Tensor, row_bytes: int) -> None:
    if cache.dtype != torch.uint8 or cache.dim() != 2 or cache.shape[1] != row_bytes or not cache.is_contiguous():
        raise ValueError(f"cache must be contiguous uint8 [rows, {row_bytes}]")


def _block_table_args(block_table, token_seq, T: int, dev):
    """Pointers and sizes of an optional block table and its token -> sequence map."""
    if block_table is None:
        return None, None, 0, 0, 0, None
    _same_device(dev, block_table=block_table, token_seq=token_seq)
    if block_table.dtype != torch.int32 or block_table.dim() != 2 or block_table.stride(1) != 1:
        raise ValueError("block_table must be int32 [seqs, blocks] with unit last stride")
    if token_seq is None or token_seq.dtype != torch.int32 or tuple(token_seq.shape) != (T,):
        raise ValueError("token_seq must be int32 [T] when a block table is given")
    token_seq = token_seq.contiguous()
    return (block_table.data_ptr(), token_seq.data_ptr(), block_table.stride(0),
            block_table.shape[0], block_table.shape[1], token_seq)


def _append(fn_name, latent, rope, slots, cache, row_bytes, extra=()):
    lib = load()
    _rows2d(latent, LATENT_DIM, "latent")
    _rows2d(rope, ROPE_DIM, "rope")
    if latent.dtype != rope.dtype:
        raise TypeError("latent and rope must share a dtype")
    if slots.dtype != torch.int64 or slots.dim() != 1 or slots.shape[0] != latent.shape[0]:
        raise ValueError("slots must be int64 [n]")
    if rope.shape[0] != latent.shape[0]:
        raise ValueError("latent and rope must have the same number of rows")
    _cache_tensor(cache, row_bytes)
    _same_device(_device_of(cache, "cache"), latent=latent, rope=rope, slots=slots)
    slots = slots.contiguous()
    st = getattr(lib, fn_name)(_ptr(latent), latent.stride(0), _ptr(rope), rope.stride(0),
                               _dtype_code(latent), latent.shape[0], _ptr(slots), _ptr(cache),
                               cache.shape[0], *extra, _stream(cache))
    check(st, fn_name)


def quantize_append(latent: torch.Tensor, rope: torch.Tensor, slots: torch.Tensor,
                    cache: torch.Tensor) -> None:
    """Encode rows to 352-byte NVFP4 and write them at ``slots`` (negative = skip)."""
    _append("mla_nvfp4_quantize_append", latent, rope, slots, cache, NVFP4_ROW_BYTES)


def quantize_append_2level(latent: torch.Tensor, rope: torch.Tensor, slots: torch.Tensor,
                           cache: torch.Tensor, global_scale: float) -> None:
    """Two-level NVFP4 rows: group scales and codes of latent / global_scale
    (decode with ``sparse_decode(..., kv_scale=global_scale)``)."""
    _append("mla_nvfp4_quantize_append_2level", latent, rope, slots, cache, NVFP4_ROW_BYTES,
            (float(global_scale),))


def fp8_quantize_append(latent, rope, slots, cache, kv_scale: float = 1.0) -> None:
    """Encode rows to 576-byte FP8 (E4M3 of value / kv_scale) at ``slots``."""
    _append("mla_fp8_quantize_append", latent, rope, slots, cache, FP8_ROW_BYTES, (float(kv_scale),))


def num_splits(tokens: int, heads: int, topk: int) -> int:
    return int(load().mla_sparse_decode_num_splits(tokens, heads, topk))


def set_merge_polls(polls: int) -> int:
    """How many times a split polls for the others before leaving its slice of
    the merge to the last arrival (0 = the last arrival merges everything).
    Process-wide; returns the previous value."""
    prev = int(load().mla_sparse_decode_set_merge_polls(int(polls)))
    if prev < 0:
        raise ValueError("polls must be >= 0")
    return prev


def workspace_size(tokens: int, heads: int, topk: int, splits: int = 0) -> int:
    n = int(load().mla_sparse_decode_workspace_size(tokens, heads, topk, splits))
    if n == 0:
        raise MlaError("workspace size query rejected its arguments")
    return n


def make_workspace(tokens: int, heads: int, topk: int, device, splits: int = 0) -> torch.Tensor:
    """A zero-filled workspace for ``sparse_decode`` (reusable across calls)."""
    return torch.zeros(workspace_size(tokens, heads, topk, splits), dtype=torch.uint8, device=device)


def _decode_args(q, cache, indices, fmt, block_table, token_seq, out, lse, workspace):
    """Checked tensors and the C arguments shared by both decode entry points."""
    dev = _device_of(q, "q")
    if q.dim() != 3 or q.shape[2] != QK_DIM or q.stride(2) != 1:
        raise ValueError("q must be [T, H, 576] with unit last stride")
    _dtype_code(q)
    T, H = q.shape[0], q.shape[1]
    if fmt not in _FMT:
        raise ValueError(f"fmt must be one of {sorted(_FMT)}")
    fmt_code = _FMT[fmt]
    _cache_tensor(cache, NVFP4_ROW_BYTES if fmt_code == FMT_NVFP4 else FP8_ROW_BYTES)
    _same_device(dev, cache=cache, indices=indices, workspace=workspace, out=out, lse=lse)
    if indices.dtype != torch.int32 or indices.dim() != 2 or indices.shape[0] != T or indices.stride(1) != 1:
        raise ValueError("indices must be int32 [T, topk] with unit last stride")
    bt_ptr, ts_ptr, bt_stride, bt_rows, bt_cols, token_seq = _block_table_args(block_table, token_seq, T, dev)
    if out is None:
        out = torch.empty((T, H, LATENT_DIM), dtype=q.dtype, device=dev)
    _exact(out, "out", (T, H, LATENT_DIM), q.dtype)
    if lse is None:
        lse = torch.empty((T, H), dtype=torch.float32, device=dev)
    _exact(lse, "lse", (T, H), torch.float32)
    return dev, fmt_code, (bt_ptr, ts_ptr, bt_stride, bt_rows, bt_cols, token_seq), out, lse


def sparse_decode(q: torch.Tensor, cache: torch.Tensor, indices: torch.Tensor, sm_scale: float, *,
                  fmt: str = "nvfp4", kv_scale: float = 1.0, block_table=None, token_seq=None,
                  block_size: int = 64, workspace=None, num_splits: int = 0, out=None, lse=None):
    """Sparse MLA decode; returns (out [T, H, 512] in q's dtype, lse [T, H] float32).

    kv_scale is the cache's per-tensor scale: FP8 rows' power-of-two scale,
    or two-level NVFP4 rows' latent scale (1 for one-level rows)."""
    lib = load()
    dev, fmt_code, bt, out, lse = _decode_args(q, cache, indices, fmt, block_table, token_seq, out, lse,
                                               workspace)
    bt_ptr, ts_ptr, bt_stride, bt_rows, bt_cols, _keep = bt
    T, H, topk = q.shape[0], q.shape[1], indices.shape[1]
    if workspace is None:
        workspace = make_workspace(T, H, topk, dev, num_splits)
    if workspace.dtype != torch.uint8 or workspace.dim() != 1 or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous uint8 vector (see make_workspace)")
    st = lib.mla_sparse_decode(
        q.data_ptr(), _dtype_code(q), T, H, q.stride(0), q.stride(1),
        cache.data_ptr(), fmt_code, cache.shape[0], float(kv_scale),
        indices.data_ptr(), topk, indices.stride(0),
        bt_ptr, int(block_size), bt_stride, bt_rows, bt_cols, ts_ptr,
        float(sm_scale), out.data_ptr(), lse.data_ptr(),
        workspace.data_ptr(), workspace.numel(), int(num_splits), _stream(q))
    check(st, "mla_sparse_decode")
    return out, lse


def sparse_decode_noalloc(q: torch.Tensor, cache: torch.Tensor, indices: torch.Tensor, sm_scale: float,
                          out: torch.Tensor, lse: torch.Tensor, *, fmt: str = "nvfp4", kv_scale: float = 1.0,
                          block_table=None, token_seq=None, block_size: int = 64, num_splits: int = 0):
    """``sparse_decode`` without a workspace, for callers that cannot allocate:
    the library's own per-GPU scratch array serves as workspace.  The caller
    passes out and lse; calls that overlap in time on one GPU race."""
    lib = load()
    _, fmt_code, bt, out, lse = _decode_args(q, cache, indices, fmt, block_table, token_seq, out, lse, None)
    bt_ptr, ts_ptr, bt_stride, bt_rows, bt_cols, _keep = bt
    T, H, topk = q.shape[0], q.shape[1], indices.shape[1]
    st = lib.mla_sparse_decode_noalloc(
        q.data_ptr(), _dtype_code(q), T, H, q.stride(0), q.stride(1),
        cache.data_ptr(), fmt_code, cache.shape[0], float(kv_scale),
        indices.data_ptr(), topk, indices.stride(0),
        bt_ptr, int(block_size), bt_stride, bt_rows, bt_cols, ts_ptr,
        float(sm_scale), out.data_ptr(), lse.data_ptr(), int(num_splits), _stream(q))
    check(st, "mla_sparse_decode_noalloc")
    return out, lse


def gather_dequant_fp8(cache: torch.Tensor, indices: torch.Tensor, fp8_scale: float = 1.0, *,
                       block_table=None, token_seq=None, block_size: int = 64,
                       rows=None, staged_indices=None):
    """Staged comparator step 1: selected NVFP4 rows -> FP8 rows [T*topk, 576] in HBM."""
    lib = load()
    dev = _device_of(cache, "cache")
    _cache_tensor(cache, NVFP4_ROW_BYTES)
    _same_device(dev, indices=indices, rows=rows, staged_indices=staged_indices)
    if indices.dtype != torch.int32 or indices.dim() != 2 or indices.stride(1) != 1:
        raise ValueError("indices must be int32 [T, topk] with unit last stride")
    T, topk = indices.shape
    if rows is None:
        rows = torch.empty((T * topk, FP8_ROW_BYTES), dtype=torch.uint8, device=dev)
    _exact(rows, "rows", (T * topk, FP8_ROW_BYTES), torch.uint8)
    if staged_indices is None:
        staged_indices = torch.empty((T, topk), dtype=torch.int32, device=dev)
    _exact(staged_indices, "staged_indices", (T, topk), torch.int32)
    bt_ptr, ts_ptr, bt_stride, bt_rows, bt_cols, token_seq = _block_table_args(block_table, token_seq, T, dev)
    st = lib.mla_nvfp4_gather_dequant_fp8(
        cache.data_ptr(), cache.shape[0], indices.data_ptr(), T, topk, indices.stride(0),
        bt_ptr, int(block_size), bt_stride, bt_rows, bt_cols, ts_ptr, float(fp8_scale),
        rows.data_ptr(), staged_indices.data_ptr(), _stream(cache))
    check(st, "mla_nvfp4_gather_dequant_fp8")
    return rows, staged_indices


INDEXER_DIM = 128


def indexer_workspace(tokens: int, max_ctx: int, device) -> torch.Tensor:
    """A zero-filled workspace for ``indexer_topk`` (reusable across calls)."""
    n = int(load().mla_indexer_workspace_size(tokens, max_ctx))
    return torch.zeros(max(n, 16), dtype=torch.uint8, device=device)


def indexer_topk(q_idx: torch.Tensor, keys: torch.Tensor, ctx_len: torch.Tensor, topk: int, max_ctx: int, *,
                 key_base=None, block_table=None, token_seq=None, block_size: int = 64,
                 out=None, workspace=None) -> torch.Tensor:
    """The sparse indexer's lists: int32 [T, topk] of each token's best positions
    (physical rows key_base[t] + p without a block table, logical positions with
    one), ascending, padded with -1."""
    lib = load()
    dev = _device_of(keys, "keys")
    if keys.dtype != torch.uint8 or keys.dim() != 2 or keys.shape[1] != INDEXER_DIM or not keys.is_contiguous():
        raise ValueError("keys must be contiguous uint8 [rows, 128] (E4M3 bytes)")
    if q_idx.dtype != torch.uint8 or q_idx.dim() != 2 or q_idx.shape[1] != INDEXER_DIM or q_idx.stride(1) != 1:
        raise ValueError("q_idx must be uint8 [T, 128] (E4M3 bytes) with unit last stride")
    T = q_idx.shape[0]
    _same_device(dev, q_idx=q_idx, ctx_len=ctx_len, key_base=key_base, out=out, workspace=workspace)
    if ctx_len.dtype != torch.int32 or tuple(ctx_len.shape) != (T,):
        raise ValueError("ctx_len must be int32 [T]")
    ctx_len = ctx_len.contiguous()
    bt_ptr, ts_ptr, bt_stride, bt_rows, bt_cols, _keep = _block_table_args(block_table, token_seq, T, dev)
    base_ptr = None
    if block_table is None:
        if key_base is None or key_base.dtype != torch.int64 or tuple(key_base.shape) != (T,):
            raise ValueError("key_base must be int64 [T] without a block table")
        key_base = key_base.contiguous()
        base_ptr = key_base.data_ptr()
    if out is None:
        out = torch.empty((T, topk), dtype=torch.int32, device=dev)
    if out.dtype != torch.int32 or out.dim() != 2 or out.shape != (T, topk) or out.stride(1) != 1:
        raise ValueError(f"out must be int32 [T, {topk}] with unit last stride")
    if workspace is None:
        workspace = indexer_workspace(T, max_ctx, dev)
    if workspace.dtype != torch.uint8 or workspace.dim() != 1 or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous uint8 vector (see indexer_workspace)")
    st = lib.mla_indexer_topk(q_idx.data_ptr(), q_idx.stride(0), keys.data_ptr(), keys.shape[0], T,
                              ctx_len.data_ptr(), int(max_ctx), base_ptr, bt_ptr, int(block_size), bt_stride,
                              bt_rows, bt_cols, ts_ptr, int(topk), out.data_ptr(), out.stride(0),
                              workspace.data_ptr(), workspace.numel(), _stream(keys))
    check(st, "mla_indexer_topk")
    return out


LAYOUTS = {"layer": 0, "block": 1}


class Pool:
    """The library's paged cache pool (host side): capacity in 64-row (or
    block_rows) blocks for `layers` layers of rows plus other per-token state,
    a lowest-free-first block allocator and per-sequence block tables."""

    def __init__(self, budget_bytes: int, layers: int, row_bytes: int = NVFP4_ROW_BYTES,
                 other_bytes: int = 0, block_rows: int = 64, max_seqs: int = 1,
                 max_blocks_per_seq: int = 1):
        import ctypes

        self._lib = load()
        h = ctypes.c_void_p()
        check(self._lib.mla_pool_create(budget_bytes, layers, row_bytes, other_bytes, block_rows, max_seqs,
                                        max_blocks_per_seq, ctypes.byref(h)), "mla_pool_create")
        self._h = h
        self.layers, self.row_bytes, self.block_rows = layers, row_bytes, block_rows
        self.max_seqs, self.max_blocks = max_seqs, max_blocks_per_seq

    def close(self):
        if self._h:
            self._lib.mla_pool_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @property
    def num_blocks(self) -> int:
        return int(self._lib.mla_pool_num_blocks(self._h))

    @property
    def free_blocks(self) -> int:
        return int(self._lib.mla_pool_free_blocks(self._h))

    def reserve(self, seq: int, tokens: int) -> bool:
        """Grow `seq` to hold `tokens` positions; False (nothing taken) if it cannot."""
        st = self._lib.mla_pool_reserve(self._h, seq, tokens)
        if st == 5:
            return False
        check(st, "mla_pool_reserve")
        return True

    def release(self, seq: int) -> None:
        check(self._lib.mla_pool_release(self._h, seq), "mla_pool_release")

    def block_table(self) -> torch.Tensor:
        """Host int32 [max_seqs, max_blocks_per_seq], -1 = no block."""
        t = torch.empty((self.max_seqs, self.max_blocks), dtype=torch.int32)
        check(self._lib.mla_pool_block_table(self._h, t.data_ptr(), self.max_blocks), "mla_pool_block_table")
        return t

    def slots(self, seq: int, first_pos: int, n: int) -> torch.Tensor:
        """Host int64 physical rows of positions first_pos .. first_pos + n - 1."""
        t = torch.empty(n, dtype=torch.int64)
        check(self._lib.mla_pool_slots(self._h, seq, first_pos, n, t.data_ptr() if n else None), "mla_pool_slots")
        return t

    def descriptors(self, seq: int, layout: str):
        """(copy descriptors, bytes) of `seq`'s regions under a layer- or block-major pool."""
        import ctypes

        d, b = ctypes.c_int64(), ctypes.c_int64()
        check(self._lib.mla_pool_descriptors(self._h, seq, LAYOUTS[layout], ctypes.byref(d), ctypes.byref(b)),
              "mla_pool_descriptors")
        return int(d.value), int(b.value)


def pool_capacity_blocks(budget_bytes: int, layers: int, row_bytes: int, other_bytes: int,
                         block_rows: int = 64) -> int:
    return int(load().mla_pool_capacity_blocks(budget_bytes, layers, row_bytes, other_bytes, block_rows))


def _region_args(pool_t, layout, pool_blocks, layers, block_rows, row_bytes, block_ids, staging):
    dev = _device_of(pool_t, "pool")
    _same_device(dev, block_ids=block_ids, staging=staging)
    if pool_t.dtype != torch.uint8 or not pool_t.is_contiguous():
        raise ValueError("pool must be a contiguous uint8 tensor")
    region = block_rows * row_bytes
    if pool_t.numel() < pool_blocks * layers * region:
        raise ValueError("pool is smaller than pool_blocks * layers * block_rows * row_bytes bytes")
    if block_ids.dtype != torch.int32 or block_ids.dim() != 1 or not block_ids.is_contiguous():
        raise ValueError("block_ids must be a contiguous int32 vector")
    n = block_ids.shape[0]
    if staging.dtype != torch.uint8 or not staging.is_contiguous() or staging.numel() < n * layers * region:
        raise ValueError("staging must be a contiguous uint8 tensor of n * layers * block_rows * row_bytes bytes")
    if layout not in LAYOUTS:
        raise ValueError(f"layout must be one of {sorted(LAYOUTS)}")
    return n


def kv_pack_blocks(pool_t, layout: str, pool_blocks: int, layers: int, block_ids, staging,
                   block_rows: int = 64, row_bytes: int = NVFP4_ROW_BYTES) -> None:
    """Gather a request's blocks (all layers) from a pool into a contiguous
    block-major staging buffer [n][layers][block_rows * row_bytes]."""
    n = _region_args(pool_t, layout, pool_blocks, layers, block_rows, row_bytes, block_ids, staging)
    check(load().mla_kv_pack_blocks(pool_t.data_ptr(), LAYOUTS[layout], pool_blocks, layers, block_rows,
                                    row_bytes, block_ids.data_ptr(), n, staging.data_ptr(), _stream(pool_t)),
          "mla_kv_pack_blocks")


def kv_unpack_blocks(staging, block_ids, pool_t, layout: str, pool_blocks: int, layers: int,
                     block_rows: int = 64, row_bytes: int = NVFP4_ROW_BYTES) -> None:
    """Scatter a block-major staging buffer into a pool at block_ids."""
    n = _region_args(pool_t, layout, pool_blocks, layers, block_rows, row_bytes, block_ids, staging)
    check(load().mla_kv_unpack_blocks(staging.data_ptr(), n, block_ids.data_ptr(), pool_t.data_ptr(),
                                      LAYOUTS[layout], pool_blocks, layers, block_rows, row_bytes,
                                      _stream(pool_t)),
          "mla_kv_unpack_blocks")


def gather_probe(cache: torch.Tensor, rows: torch.Tensor, sink: torch.Tensor = None) -> torch.Tensor:
    """Read the given physical rows of a cache and nothing else (a measurement
    aid: the HBM ceiling of a kernel that gathers those rows).  cache is
    contiguous uint8 [rows, row_bytes]; rows is contiguous int32 [n].
    Returns the one-word sink tensor (its contents carry no meaning)."""
    dev = _device_of(cache, "cache")
    if cache.dtype != torch.uint8 or cache.dim() != 2 or not cache.is_contiguous():
        raise ValueError("cache must be contiguous uint8 [rows, row_bytes]")
    if rows.dtype != torch.int32 or rows.dim() != 1 or not rows.is_contiguous():
        raise ValueError("rows must be a contiguous int32 vector")
    if sink is None:
        sink = torch.zeros(1, dtype=torch.int32, device=dev)
    _same_device(dev, rows=rows, sink=sink)
    _exact(sink, "sink", (1,), torch.int32)
    check(load().mla_gather_probe(cache.data_ptr(), cache.shape[0], cache.shape[1], rows.data_ptr(),
                                  rows.numel(), sink.data_ptr(), _stream(cache)),
          "mla_gather_probe")
    return sink


def kernel_timing(enable: bool) -> None:
    """Benchmark instrumentation: time every later library kernel with HIP events."""
    check(load().mla_kernel_timing(1 if enable else 0), "mla_kernel_timing")


def last_kernel_ms() -> float:
    """Kernel duration (ms) of the last timed library launch; waits for it to finish."""
    import ctypes

    ms = ctypes.c_float(0.0)
    check(load().mla_last_kernel_ms(ctypes.byref(ms)), "mla_last_kernel_ms")
    return float(ms.value)
