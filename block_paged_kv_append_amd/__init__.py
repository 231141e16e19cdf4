"""block_paged_kv_append_amd -- attention over a block-paged KV cache on MI355X.

A thin ctypes binding over ``libpkv.so`` (HIP, gfx950), whose C ABI is declared
in ``include/pkv.h``.  The functions below carry the C entry points' names and
only marshal arguments: shapes and dtypes are read from torch tensors, device
pointers and the current HIP stream are passed through, and every step of the
computation runs in the library's kernels.  There is no fallback: if the
library is missing, calls raise.

Pool layout (vLLM/PagedAttention), X = 16 bytes / element size:
    k_pool [num_blocks, num_kv_heads, head_dim // X, 16, X]
    v_pool [num_blocks, num_kv_heads, head_dim, 16]
"""
from __future__ import annotations

import ctypes
import os
import threading
from typing import Optional

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
# PKV_LIBRARY selects another build of the library (e.g. libpkv_timeline.so)
LIB_PATH = os.environ.get("PKV_LIBRARY") or os.path.join(PKG_DIR, "libpkv.so")

PKV_F32 = 0
PKV_BF16 = 1
BLOCK_SIZE = 16

_STATUS = {0: "PKV_OK", -1: "PKV_EINVAL", -2: "PKV_EUNSUPPORTED", -3: "PKV_EWORKSPACE",
           -4: "PKV_EHIP", -5: "PKV_ENOMEM"}

# (name, restype, argtypes) of every entry point in include/pkv.h
_P, _I, _F, _Z = ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
SIGNATURES = {
    "paged_kv_append": (ctypes.c_int, [_P, _P, _P, _I, _P, _P, _I, _I, _I, _I, _I, _P]),
    "paged_kv_copy_blocks": (ctypes.c_int, [_P, _P, _I, _I, _I, _I, _P, _P, _I, _I, _P]),
    "pkv_allocator_create": (ctypes.c_int, [ctypes.POINTER(_P), _I]),
    "pkv_allocator_destroy": (None, [_P]),
    "pkv_allocator_alloc": (ctypes.c_int, [_P, _I, _P]),
    "pkv_allocator_share": (ctypes.c_int, [_P, _P, _I]),
    "pkv_allocator_release": (ctypes.c_int, [_P, _P, _I]),
    "pkv_allocator_prepare_write": (ctypes.c_int, [_P, _P, _I, _I, _P, _P, _P]),
    "pkv_allocator_num_free": (_I, [_P]),
    "pkv_allocator_refcount": (_I, [_P, _I]),
    "paged_attn_decode_workspace_size": (_Z, [_I, _I, _I, _I, _I, _I]),
    "paged_attn_decode": (ctypes.c_int, [_P, _P, _P, _P, _P, _I, _P, _I, _P, _I, _I, _I, _I, _I,
                                         _I, _F, _F, _I, _P, _Z, _I, _P]),
    "paged_attn_decode_splitk": (ctypes.c_int, [_P, _P, _P, _P, _P, _I, _P, _I, _P, _I, _I, _I,
                                                _I, _I, _I, _F, _F, _I, _I, _P, _Z, _I, _P]),
    "paged_attn_decode_no_alloc": (ctypes.c_int, [_P, _P, _P, _P, _P, _I, _P, _I, _P, _I, _I, _I,
                                                  _I, _I, _I, _F, _F, _I, _I, _I, _P]),
    "paged_attn_decode_append": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _I, _P, _I, _P, _I,
                                                _I, _I, _I, _I, _I, _F, _F, _I, _I, _P, _Z, _I,
                                                _P]),
    "paged_attn_decode_sink_h2o": (ctypes.c_int, [_P, _P, _P, _P, _P, _I, _P, _I, _P, _I, _I, _I,
                                                  _I, _I, _I, _F, _F, _I, _I, _P, _P, _I, _P, _Z,
                                                  _I, _P]),
    "paged_attn_prefill": (ctypes.c_int, [_P, _P, _P, _P, _I, _I, _P, _P, _I, _P, _I, _P, _I, _I,
                                          _I, _I, _I, _I, _F, _F, _I, _I, _P]),
    "pkv_decode_graph_create": (ctypes.c_int, [ctypes.POINTER(_P), _P, _P, _P, _P, _P, _P, _P,
                                               _I, _P, _I, _P, _I, _I, _I, _I, _I, _I, _F, _F,
                                               _I, _I, _I]),
    "pkv_decode_graph_launch": (ctypes.c_int, [_P, _P]),
    "pkv_decode_graph_destroy": (None, [_P]),
    "paged_attn_mixed": (ctypes.c_int, [_P, _P, _P, _P, _I, _I, _I, _P, _P, _I, _P, _I, _P, _I, _I,
                                        _I, _I, _I, _I, _F, _F, _I, _P, _Z, _I, _P]),
    "pkv_check_paged_metadata": (ctypes.c_int, [_P, _P, _I, _I, _I, _P, _I, _P, _P]),
    "pkv_hbm_read_probe": (ctypes.c_int, [_P, _Z, _P, _I, _P]),
    "pkv_hbm_gather_probe": (ctypes.c_int, [_P, _P, _Z, _I, _P, _I, _P, _I, _P]),
    "pkv_mfma_rate_probe": (ctypes.c_int, [_P, _I, _I, _P]),
    "pkv_last_error": (ctypes.c_char_p, []),
}

# flag bits of pkv_check_paged_metadata
CHECK_BAD_CONTEXT_LEN = 1
CHECK_BAD_BLOCK_ID = 2
CHECK_BAD_SLOT = 4
CHECK_DUPLICATE_SLOT = 8


class PkvError(RuntimeError):
    def __init__(self, fn: str, code: int, message: str):
        super().__init__(f"{fn} failed with {_STATUS.get(code, code)}: {message}")
        self.code = code


_lib = None
_lib_lock = threading.Lock()


def load_library(path: Optional[str] = None) -> ctypes.CDLL:
    """Load libpkv.so (after torch, so that both share torch's HIP runtime)."""
    global _lib
    with _lib_lock:
        if _lib is not None and path is None:
            return _lib
        import torch  # noqa: F401  -- torch's libamdhip64 must be the one in use

        p = path or LIB_PATH
        if not os.path.exists(p):
            raise RuntimeError(f"{p} is missing: build it with `python -m block_paged_kv_append_amd.build`")
        lib = ctypes.CDLL(p)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        if path is None:
            _lib = lib
        return lib


def pkv_last_error() -> str:
    return load_library().pkv_last_error().decode()


def _check(fn: str, rc: int) -> None:
    if rc != 0:
        raise PkvError(fn, rc, pkv_last_error())


# ---------------------------------------------------------------------------
# tensor marshalling
# ---------------------------------------------------------------------------
def _dtype_code(t) -> int:
    import torch

    if t.dtype == torch.bfloat16:
        return PKV_BF16
    if t.dtype == torch.float32:
        return PKV_F32
    raise TypeError(f"unsupported dtype {t.dtype} (bfloat16 or float32)")


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr()


def _i32(t, name):
    import torch

    if t.dtype != torch.int32:
        raise TypeError(f"{name} must be int32, got {t.dtype}")
    return _ptr(t)


def _stream(stream) -> Optional[int]:
    import torch

    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream or None


def _pool_dims(k_pool, v_pool):
    nb, hkv, d, bs = v_pool.shape
    if bs != BLOCK_SIZE:
        raise ValueError(f"v_pool's last dim must be {BLOCK_SIZE}")
    x = 16 // v_pool.element_size()
    if tuple(k_pool.shape) != (nb, hkv, d // x, BLOCK_SIZE, x):
        raise ValueError(f"k_pool shape {tuple(k_pool.shape)} does not match v_pool {tuple(v_pool.shape)}")
    if k_pool.dtype != v_pool.dtype:
        raise TypeError("k_pool and v_pool dtypes differ")
    return nb, hkv, d


# ---------------------------------------------------------------------------
# entry points
# ---------------------------------------------------------------------------
def paged_kv_append(k_new, v_new, slot_mapping, k_pool, v_pool, stream=None) -> None:
    """Write rows ``k_new/v_new [T, Hkv, D]`` to slots ``slot_mapping [T]``."""
    nb, hkv, d = _pool_dims(k_pool, v_pool)
    T = k_new.shape[0]
    if tuple(k_new.shape) != (T, hkv, d) or tuple(v_new.shape) != (T, hkv, d):
        raise ValueError("k_new/v_new must be [T, num_kv_heads, head_dim]")
    if k_new.dtype != k_pool.dtype or v_new.dtype != k_pool.dtype:
        raise TypeError("k_new/v_new dtype must match the pools")
    if slot_mapping.numel() != T:
        raise ValueError("slot_mapping must have T entries")
    lib = load_library()
    rc = lib.paged_kv_append(_ptr(k_new), _ptr(v_new), _i32(slot_mapping, "slot_mapping"), T,
                             _ptr(k_pool), _ptr(v_pool), nb, hkv, d, BLOCK_SIZE,
                             _dtype_code(k_pool), _stream(stream))
    _check("paged_kv_append", rc)


def paged_kv_copy_blocks(src_ids, dst_ids, k_pool, v_pool, stream=None) -> None:
    """Copy whole blocks ``src_ids[i] -> dst_ids[i]`` (int32 device tensors) in
    both pools (copy-on-write of shared blocks)."""
    nb, hkv, d = _pool_dims(k_pool, v_pool)
    n = src_ids.numel()
    if dst_ids.numel() != n:
        raise ValueError("src_ids and dst_ids must have the same length")
    lib = load_library()
    rc = lib.paged_kv_copy_blocks(_ptr(k_pool), _ptr(v_pool), nb, hkv, d, BLOCK_SIZE,
                                  _i32(src_ids, "src_ids"), _i32(dst_ids, "dst_ids"), n,
                                  _dtype_code(k_pool), _stream(stream))
    _check("paged_kv_copy_blocks", rc)


def check_paged_metadata(num_blocks, block_tables=None, context_lens=None, slot_mapping=None,
                         stream=None) -> int:
    """Check block tables / context lengths ([B, MB] / [B] int32 device tensors)
    and an append's slot mapping ([T] int32) against a pool of ``num_blocks``
    blocks on the device; returns the OR of the CHECK_* flags (0: all valid).
    Waits for the stream to reach the check."""
    import torch

    B = 0 if block_tables is None else block_tables.shape[0]
    MB = 1 if block_tables is None else block_tables.shape[1]
    if B and (context_lens is None or context_lens.numel() != B):
        raise ValueError("context_lens must have one entry per block-table row")
    T = 0 if slot_mapping is None else slot_mapping.numel()
    src = block_tables if block_tables is not None else slot_mapping
    dev = src.device if src is not None else torch.device("cuda")
    flags = torch.empty(1, dtype=torch.int32, device=dev)
    lib = load_library()
    rc = lib.pkv_check_paged_metadata(
        _i32(block_tables, "block_tables") if B else None,
        _i32(context_lens, "context_lens") if B else None, B, MB, int(num_blocks),
        _i32(slot_mapping, "slot_mapping") if T else None, T, _ptr(flags), _stream(stream))
    _check("pkv_check_paged_metadata", rc)
    if stream is None:
        torch.cuda.current_stream(dev).synchronize()
    else:
        stream.synchronize()
    return int(flags.item()) & 0xFFFFFFFF


class BlockAllocator:
    """Host-side refcounted block ids with copy-on-write (``pkv_block_allocator``
    in include/pkv.h).  Ids and table rows are numpy int32 arrays."""

    def __init__(self, num_blocks: int):
        self._lib = load_library()
        h = ctypes.c_void_p()
        _check("pkv_allocator_create", self._lib.pkv_allocator_create(ctypes.byref(h),
                                                                      int(num_blocks)))
        self._h = h

    @staticmethod
    def _arr(ids):
        import numpy as np

        a = np.ascontiguousarray(ids, dtype=np.int32)
        return a, a.ctypes.data_as(ctypes.c_void_p)

    def alloc(self, n: int):
        import numpy as np

        out = np.empty(int(n), dtype=np.int32)
        _check("pkv_allocator_alloc", self._lib.pkv_allocator_alloc(
            self._h, int(n), out.ctypes.data_as(ctypes.c_void_p)))
        return out

    def share(self, ids) -> None:
        a, p = self._arr(ids)
        _check("pkv_allocator_share", self._lib.pkv_allocator_share(self._h, p, a.size))

    def release(self, ids) -> None:
        a, p = self._arr(ids)
        _check("pkv_allocator_release", self._lib.pkv_allocator_release(self._h, p, a.size))

    def prepare_write(self, table_row, first: int, last: int):
        """Copy-on-write for logical blocks ``[first, last]`` of ``table_row``
        (an int32 numpy array, updated in place); returns the (src, dst) pairs
        to copy."""
        import numpy as np

        if table_row.dtype != np.int32 or not table_row.flags.c_contiguous:
            raise TypeError("table_row must be a contiguous int32 numpy array")
        n = max(int(last) - int(first) + 1, 0)
        src, dst = np.empty(n, dtype=np.int32), np.empty(n, dtype=np.int32)
        cnt = ctypes.c_int32(0)
        _check("pkv_allocator_prepare_write", self._lib.pkv_allocator_prepare_write(
            self._h, table_row.ctypes.data_as(ctypes.c_void_p), int(first), int(last),
            src.ctypes.data_as(ctypes.c_void_p), dst.ctypes.data_as(ctypes.c_void_p),
            ctypes.byref(cnt)))
        return src[:cnt.value].copy(), dst[:cnt.value].copy()

    def num_free(self) -> int:
        return int(self._lib.pkv_allocator_num_free(self._h))

    def refcount(self, block: int) -> int:
        return int(self._lib.pkv_allocator_refcount(self._h, int(block)))

    def close(self) -> None:
        if getattr(self, "_h", None) is not None:
            self._lib.pkv_allocator_destroy(self._h)
            self._h = None

    def __del__(self):
        self.close()


def paged_attn_decode_workspace_size(num_seqs, num_kv_heads, gqa_group, head_dim,
                                     max_context_len, partition_size=0) -> int:
    return int(load_library().paged_attn_decode_workspace_size(
        num_seqs, num_kv_heads, gqa_group, head_dim, max_context_len, partition_size))


_ws_cache = {}
_ws_lock = threading.Lock()


def decode_workspace(nbytes: int, device, stream=None):
    """A zero-filled workspace of at least ``nbytes``, cached per device and
    stream (calls on one stream run in order, so they can share it; each call
    leaves its counters at zero again)."""
    import torch

    key = (str(device), _stream(stream))
    with _ws_lock:
        ws = _ws_cache.get(key)
        if ws is None or ws.numel() < nbytes:
            ws = torch.zeros(max(int(nbytes), 256), dtype=torch.uint8, device=device)
            _ws_cache[key] = ws
        return ws


def _decode_dims(out, q, k_pool, v_pool, block_tables, context_lens):
    nb, hkv, d = _pool_dims(k_pool, v_pool)
    B, hq, dq = q.shape
    if dq != d or hq % hkv:
        raise ValueError(f"q shape {tuple(q.shape)} does not fit pools with {hkv} kv heads of {d}")
    if tuple(out.shape) != tuple(q.shape) or out.dtype != q.dtype or q.dtype != k_pool.dtype:
        raise ValueError("out must match q, and q's dtype the pools'")
    if block_tables.dim() != 2 or block_tables.shape[0] != B or context_lens.numel() != B:
        raise ValueError("block_tables [B, MB] and context_lens [B] must match q's batch")
    return nb, hkv, d, B, hq // hkv, block_tables.shape[1]


def paged_attn_decode(out, q, k_pool, v_pool, block_tables, context_lens, max_context_len,
                      scale, softcap=0.0, window=0, lse=None, workspace=None, stream=None) -> None:
    """One-token decode for every sequence; writes ``out [B, Hq, D]`` (and ``lse``)."""
    nb, hkv, d, B, G, MB = _decode_dims(out, q, k_pool, v_pool, block_tables, context_lens)
    need = paged_attn_decode_workspace_size(B, hkv, G, d, max_context_len, 0)
    ws = workspace if workspace is not None else decode_workspace(need, q.device, stream)
    lib = load_library()
    rc = lib.paged_attn_decode(_ptr(out), _ptr(lse), _ptr(q), _ptr(k_pool), _ptr(v_pool), nb,
                               _i32(block_tables, "block_tables"), MB,
                               _i32(context_lens, "context_lens"), int(max_context_len), B, hkv,
                               G, d, BLOCK_SIZE, float(scale), float(softcap), int(window),
                               _ptr(ws), ws.numel() * ws.element_size(), _dtype_code(q),
                               _stream(stream))
    _check("paged_attn_decode", rc)


def paged_attn_decode_splitk(out, q, k_pool, v_pool, block_tables, context_lens,
                             max_context_len, scale, softcap=0.0, window=0, partition_size=512,
                             lse=None, workspace=None, stream=None) -> None:
    """Split-K decode with fixed ``partition_size``-token partitions merged by log-sum-exp."""
    nb, hkv, d, B, G, MB = _decode_dims(out, q, k_pool, v_pool, block_tables, context_lens)
    need = paged_attn_decode_workspace_size(B, hkv, G, d, max_context_len, partition_size)
    ws = workspace if workspace is not None else decode_workspace(need, q.device, stream)
    lib = load_library()
    rc = lib.paged_attn_decode_splitk(_ptr(out), _ptr(lse), _ptr(q), _ptr(k_pool), _ptr(v_pool),
                                      nb, _i32(block_tables, "block_tables"), MB,
                                      _i32(context_lens, "context_lens"), int(max_context_len), B,
                                      hkv, G, d, BLOCK_SIZE, float(scale), float(softcap),
                                      int(window), int(partition_size), _ptr(ws),
                                      ws.numel() * ws.element_size(), _dtype_code(q),
                                      _stream(stream))
    _check("paged_attn_decode_splitk", rc)


def paged_attn_decode_no_alloc(out, q, k_pool, v_pool, block_tables, context_lens,
                               max_context_len, scale, softcap=0.0, window=0, partition_size=0,
                               lse=None, stream=None) -> None:
    """paged_attn_decode (partition_size 0) or paged_attn_decode_splitk
    without a workspace: the library's static per-GPU scratch serves instead,
    and nothing is allocated.  Calls that overlap on one GPU race."""
    nb, hkv, d, B, G, MB = _decode_dims(out, q, k_pool, v_pool, block_tables, context_lens)
    lib = load_library()
    rc = lib.paged_attn_decode_no_alloc(_ptr(out), _ptr(lse), _ptr(q), _ptr(k_pool), _ptr(v_pool),
                                        nb, _i32(block_tables, "block_tables"), MB,
                                        _i32(context_lens, "context_lens"), int(max_context_len),
                                        B, hkv, G, d, BLOCK_SIZE, float(scale), float(softcap),
                                        int(window), int(partition_size), _dtype_code(q),
                                        _stream(stream))
    _check("paged_attn_decode_no_alloc", rc)


def paged_attn_decode_append(out, q, k_new, v_new, k_pool, v_pool, block_tables, context_lens,
                             max_context_len, scale, softcap=0.0, window=0, partition_size=0,
                             lse=None, workspace=None, stream=None) -> None:
    """One decode tick in one launch: rows ``k_new/v_new [B, Hkv, D]`` go to
    position ``L_b - 1`` of each sequence (through its block table) and the
    decode attends to them; ``partition_size > 0`` selects the split-K form."""
    nb, hkv, d, B, G, MB = _decode_dims(out, q, k_pool, v_pool, block_tables, context_lens)
    if tuple(k_new.shape) != (B, hkv, d) or tuple(v_new.shape) != (B, hkv, d):
        raise ValueError("k_new/v_new must be [num_seqs, num_kv_heads, head_dim]")
    if k_new.dtype != k_pool.dtype or v_new.dtype != k_pool.dtype:
        raise TypeError("k_new/v_new dtype must match the pools")
    need = paged_attn_decode_workspace_size(B, hkv, G, d, max_context_len, partition_size)
    ws = workspace if workspace is not None else decode_workspace(need, q.device, stream)
    lib = load_library()
    rc = lib.paged_attn_decode_append(_ptr(out), _ptr(lse), _ptr(q), _ptr(k_new), _ptr(v_new),
                                      _ptr(k_pool), _ptr(v_pool), nb,
                                      _i32(block_tables, "block_tables"), MB,
                                      _i32(context_lens, "context_lens"), int(max_context_len), B,
                                      hkv, G, d, BLOCK_SIZE, float(scale), float(softcap),
                                      int(window), int(partition_size), _ptr(ws),
                                      ws.numel() * ws.element_size(), _dtype_code(q),
                                      _stream(stream))
    _check("paged_attn_decode_append", rc)


def paged_attn_decode_sink_h2o(out, q, k_pool, v_pool, block_tables, context_lens,
                               max_context_len, scale, softcap=0.0, window=0, sink_tokens=0,
                               scores=None, column_mass=None, lse=None, workspace=None,
                               stream=None) -> None:
    """Balanced decode with AttentionSink tokens beside the window and, when
    ``column_mass [B, Hkv, S]`` is given (with ``scores [B, Hq, S]`` and
    ``lse``), the H2O per-token attention mass of the step."""
    nb, hkv, d, B, G, MB = _decode_dims(out, q, k_pool, v_pool, block_tables, context_lens)
    stride = 0
    if column_mass is not None:
        if scores is None or lse is None:
            raise ValueError("column_mass needs scores and lse")
        stride = column_mass.shape[-1]
        if tuple(column_mass.shape) != (B, hkv, stride) or \
                tuple(scores.shape) != (B, hkv * G, stride):
            raise ValueError("column_mass [B, Hkv, S] and scores [B, Hq, S] must agree")
    need = paged_attn_decode_workspace_size(B, hkv, G, d, max_context_len, 0)
    ws = workspace if workspace is not None else decode_workspace(need, q.device, stream)
    lib = load_library()
    rc = lib.paged_attn_decode_sink_h2o(_ptr(out), _ptr(lse), _ptr(q), _ptr(k_pool), _ptr(v_pool),
                                        nb, _i32(block_tables, "block_tables"), MB,
                                        _i32(context_lens, "context_lens"), int(max_context_len),
                                        B, hkv, G, d, BLOCK_SIZE, float(scale), float(softcap),
                                        int(window), int(sink_tokens), _ptr(scores),
                                        _ptr(column_mass), int(stride), _ptr(ws),
                                        ws.numel() * ws.element_size(), _dtype_code(q),
                                        _stream(stream))
    _check("paged_attn_decode_sink_h2o", rc)


def decode_bucket(num_seqs: int) -> int:
    """The batch-size bucket a tick of ``num_seqs`` sequences replays: the
    next power of two."""
    n = 1
    while n < num_seqs:
        n *= 2
    return n


class DecodeGraph:
    """A decode tick (``paged_attn_decode_append``) captured once for a bucket
    of ``q.shape[0]`` rows (``pkv_decode_graph`` in include/pkv.h).  The
    tensors passed here are bound into the graph: write each tick's q, new
    rows, tables and lengths into them (unused rows: length 0), then call
    :meth:`launch`.  The graph owns its workspace."""

    def __init__(self, out, q, k_new, v_new, k_pool, v_pool, block_tables, context_lens,
                 max_context_len, scale, softcap=0.0, window=0, partition_size=0, lse=None):
        nb, hkv, d, B, G, MB = _decode_dims(out, q, k_pool, v_pool, block_tables, context_lens)
        if tuple(k_new.shape) != (B, hkv, d) or tuple(v_new.shape) != (B, hkv, d):
            raise ValueError("k_new/v_new must be [num_seqs, num_kv_heads, head_dim]")
        if k_new.dtype != k_pool.dtype or v_new.dtype != k_pool.dtype:
            raise TypeError("k_new/v_new dtype must match the pools")
        self._lib = load_library()
        self._bound = (out, q, k_new, v_new, k_pool, v_pool, block_tables, context_lens, lse)
        h = ctypes.c_void_p()
        rc = self._lib.pkv_decode_graph_create(
            ctypes.byref(h), _ptr(out), _ptr(lse), _ptr(q), _ptr(k_new), _ptr(v_new),
            _ptr(k_pool), _ptr(v_pool), nb, _i32(block_tables, "block_tables"), MB,
            _i32(context_lens, "context_lens"), int(max_context_len), B, hkv, G, d, BLOCK_SIZE,
            float(scale), float(softcap), int(window), int(partition_size), _dtype_code(q))
        _check("pkv_decode_graph_create", rc)
        self._h = h

    def launch(self, stream=None) -> None:
        if self._h is None:
            raise RuntimeError("DecodeGraph is closed")
        _check("pkv_decode_graph_launch", self._lib.pkv_decode_graph_launch(self._h,
                                                                           _stream(stream)))

    def close(self) -> None:
        if getattr(self, "_h", None) is not None:
            self._lib.pkv_decode_graph_destroy(self._h)
            self._h = None

    def __del__(self):
        self.close()


def paged_attn_prefill(out, q, cu_q_lens, max_q_len, k_pool, v_pool, block_tables, context_lens,
                       max_context_len, scale, softcap=0.0, window=0, lse=None,
                       stream=None) -> None:
    """Causal attention of the chunk rows ``q [Tq, Hq, D]`` over prefix + chunk."""
    nb, hkv, d = _pool_dims(k_pool, v_pool)
    Tq, hq, dq = q.shape
    if dq != d or hq % hkv:
        raise ValueError(f"q shape {tuple(q.shape)} does not fit the pools")
    if tuple(out.shape) != tuple(q.shape) or out.dtype != q.dtype or q.dtype != k_pool.dtype:
        raise ValueError("out must match q, and q's dtype the pools'")
    B = context_lens.numel()
    if cu_q_lens.numel() != B + 1 or block_tables.shape[0] != B:
        raise ValueError("cu_q_lens [B+1], block_tables [B, MB], context_lens [B] disagree")
    lib = load_library()
    rc = lib.paged_attn_prefill(_ptr(out), _ptr(lse), _ptr(q), _i32(cu_q_lens, "cu_q_lens"), Tq,
                                int(max_q_len), _ptr(k_pool), _ptr(v_pool), nb,
                                _i32(block_tables, "block_tables"), block_tables.shape[1],
                                _i32(context_lens, "context_lens"), int(max_context_len), B, hkv,
                                hq // hkv, d, BLOCK_SIZE, float(scale), float(softcap),
                                int(window), _dtype_code(q), _stream(stream))
    _check("paged_attn_prefill", rc)


# ---------------------------------------------------------------------------
# numpy bit arrays <-> device tensors
# ---------------------------------------------------------------------------
def hbm_read_probe(buf, out, num_wgs=None, stream=None) -> None:
    """A plain read of the whole of ``buf`` (a device tensor, its byte size a
    multiple of 16) by ``num_wgs`` workgroups (default: 8 per compute unit),
    each writing one word of ``out`` (int32/uint32, >= num_wgs entries): the
    HBM read rate of a kernel that does nothing else."""
    import torch

    n = num_wgs or 8 * torch.cuda.get_device_properties(buf.device).multi_processor_count
    if out.numel() < n or out.element_size() != 4:
        raise ValueError("out needs num_wgs 32-bit entries")
    lib = load_library()
    _check("pkv_hbm_read_probe", lib.pkv_hbm_read_probe(_ptr(buf), buf.numel() * buf.element_size(),
                                                        _ptr(out), int(n), _stream(stream)))


def hbm_gather_probe(k, v, order, out, num_wgs=None, stream=None) -> None:
    """A read of whole blocks ``order`` (int32 device tensor of block ids) of
    ``k`` and ``v`` (device tensors whose first dimension is the block, each
    block a multiple of 4 KiB): the decode's access pattern over a shuffled
    pool.  ``num_wgs`` workgroups (default: one per compute unit) each write
    one word of ``out``."""
    import torch

    n = num_wgs or torch.cuda.get_device_properties(k.device).multi_processor_count
    if out.numel() < n or out.element_size() != 4:
        raise ValueError("out needs num_wgs 32-bit entries")
    if k.shape[0] != v.shape[0] or k.numel() != v.numel() or k.dtype != v.dtype:
        raise ValueError("k and v must have the same blocks, sizes and dtype")
    nb = k.shape[0]
    block_bytes = k.numel() * k.element_size() // nb
    lib = load_library()
    _check("pkv_hbm_gather_probe",
           lib.pkv_hbm_gather_probe(_ptr(k), _ptr(v), block_bytes, nb, _i32(order, "order"),
                                    order.numel(), _ptr(out), int(n), _stream(stream)))


def mfma_rate_probe(stamps, iters, num_wgs=None, stream=None) -> None:
    """Back-to-back bf16 32x32x16 matrix-core products, ``iters`` x 8 per wave,
    in ``num_wgs`` workgroups of four waves (default: one per compute unit);
    ``stamps`` (int64 device tensor, at least 4 num_wgs entries) receives per
    workgroup the shader-clock counter before and after the loop, then the
    100 MHz counter before and after."""
    import torch

    n = num_wgs or torch.cuda.get_device_properties(stamps.device).multi_processor_count
    if stamps.numel() < 4 * n or stamps.element_size() != 8:
        raise ValueError("stamps needs 4 num_wgs 64-bit entries")
    lib = load_library()
    _check("pkv_mfma_rate_probe",
           lib.pkv_mfma_rate_probe(_ptr(stamps), int(iters), int(n), _stream(stream)))


def from_bits(bits, dtype: str, device="cuda"):
    """uint16 (bf16) / uint32 (fp32) storage bits -> a device tensor."""
    import numpy as np
    import torch

    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)
    elif dtype == "f32":
        t = torch.from_numpy(np.ascontiguousarray(bits).view(np.float32))
    else:
        raise ValueError(dtype)
    return t.to(device)


def to_bits(t):
    """device tensor -> numpy storage bits (uint16 for bf16, uint32 for fp32)."""
    import numpy as np
    import torch

    c = t.detach().contiguous().cpu()
    if c.dtype == torch.bfloat16:
        return c.view(torch.int16).numpy().view(np.uint16)
    if c.dtype == torch.float32:
        return c.numpy().view(np.uint32)
    raise TypeError(c.dtype)


__all__ = [
    "PKV_F32", "PKV_BF16", "BLOCK_SIZE", "PkvError", "SIGNATURES", "load_library",
    "pkv_last_error", "paged_kv_append", "paged_attn_decode_workspace_size",
    "paged_attn_decode", "paged_attn_decode_splitk", "paged_attn_prefill", "decode_workspace",
    "from_bits", "to_bits",
]


def paged_attn_mixed(out, q, cu_q_lens, num_prefill_tokens, max_q_len, k_pool, v_pool,
                     block_tables, context_lens, max_context_len, scale, softcap=0.0, window=0,
                     lse=None, workspace=None, stream=None) -> None:
    """A mixed batch: the ``len(cu_q_lens) - 1`` first sequences are prefill
    chunks (rows ``0 .. num_prefill_tokens - 1``), the others decode rows (one
    row each, after the chunks' rows)."""
    nb, hkv, d = _pool_dims(k_pool, v_pool)
    T, hq, dq = q.shape
    B = context_lens.numel()
    P = cu_q_lens.numel() - 1
    if dq != d or hq % hkv or not 0 <= P <= B or T != num_prefill_tokens + B - P:
        raise ValueError("q rows must be the chunks' rows followed by one row per decode sequence")
    if tuple(out.shape) != tuple(q.shape) or out.dtype != q.dtype or q.dtype != k_pool.dtype:
        raise ValueError("out must match q, and q's dtype the pools'")
    if block_tables.dim() != 2 or block_tables.shape[0] != B:
        raise ValueError("block_tables [B, MB] and context_lens [B] disagree")
    G = hq // hkv
    ws = workspace
    if ws is None and B > P:
        ws = decode_workspace(paged_attn_decode_workspace_size(B - P, hkv, G, d, max_context_len, 0),
                              q.device, stream)
    lib = load_library()
    rc = lib.paged_attn_mixed(_ptr(out), _ptr(lse), _ptr(q),
                              _i32(cu_q_lens, "cu_q_lens") if P > 0 else None, P,
                              int(num_prefill_tokens), int(max_q_len), _ptr(k_pool), _ptr(v_pool),
                              nb, _i32(block_tables, "block_tables"), block_tables.shape[1],
                              _i32(context_lens, "context_lens"), int(max_context_len), B, hkv, G,
                              d, BLOCK_SIZE, float(scale), float(softcap), int(window), _ptr(ws),
                              0 if ws is None else ws.numel() * ws.element_size(), _dtype_code(q),
                              _stream(stream))
    _check("paged_attn_mixed", rc)
