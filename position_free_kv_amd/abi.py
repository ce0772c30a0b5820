"""ctypes binding of libkamera.so (include/kamera.h): same names, argument marshalling only.

Every computation runs in the library's HIP kernels. If the library has not
been built this module raises on first use; there is no other implementation.
"""
from __future__ import annotations

import ctypes
import os
from typing import Iterable, List, Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# KAMERA_LIBRARY names another build of the same library to load instead (the host-code
# sanitizer test loads an AddressSanitizer build of the host part this way)
LIB_PATH = os.environ.get("KAMERA_LIBRARY") or os.path.join(_HERE, "libkamera.so")

GQA, MLA = 0, 1
F32, BF16 = 0, 1
NEOX, GPTJ = 0, 1
PATCH_UNIT_AUTO, PATCH_UNIT_MFMA, PATCH_UNIT_VALU = 0, 1, 2
PATCH, IN_PLACE, POSITIONS = 1, 2, 4
MAX_FACTORS = 4
MAX_RANK = 256
BUILD_MAX_RANK = 64
BUILD_MAX_SUBSPACE = 80
BUILD_MAX_ORBIT = 32
NOALLOC_SCRATCH_BYTES = 4 << 20
PROBE_COPY, PROBE_READ, PROBE_WRITE = 0, 1, 2

STATUS = ["KAMERA_OK", "KAMERA_E_NULL", "KAMERA_E_SHAPE", "KAMERA_E_DTYPE", "KAMERA_E_RANK",
          "KAMERA_E_DELTA", "KAMERA_E_PAGE", "KAMERA_E_OVERLAP", "KAMERA_E_ALIGN",
          "KAMERA_E_WORKSPACE", "KAMERA_E_UNSUPPORTED", "KAMERA_E_HIP"]
EXPORTED = ["kamera_workspace_bytes", "kamera_batch_workspace_bytes", "kamera_relocate", "kamera_rehydrate",
            "kamera_rehydrate_batched", "kamera_rehydrate_batched_noalloc",
            "kamera_plan_upload", "kamera_plan_launch", "kamera_status_string", "kamera_last_error",
            "kamera_version", "kamera_build_workspace_bytes", "kamera_build_patch", "kamera_build_orbit_patch",
            "kamera_stream_probe"]


class Layout(ctypes.Structure):
    _fields_ = [("family", ctypes.c_int32), ("dtype", ctypes.c_int32), ("num_layers", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("latent_dim", ctypes.c_int32), ("rope_dim", ctypes.c_int32), ("pairing", ctypes.c_int32),
                ("page_size", ctypes.c_int32), ("patch_unit", ctypes.c_int32), ("rope_base", ctypes.c_double),
                ("mrope_section", ctypes.c_int32 * 3), ("reserved2", ctypes.c_int32)]


class Factor(ctypes.Structure):
    _fields_ = [("u", ctypes.c_void_p), ("v", ctypes.c_void_p), ("tensor", ctypes.c_int32),
                ("col0", ctypes.c_int32), ("width", ctypes.c_int32), ("rank", ctypes.c_int32),
                ("layer0", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class Chunk(ctypes.Structure):
    _fields_ = [("num_tokens", ctypes.c_int32), ("flags", ctypes.c_uint32), ("delta", ctypes.c_int64),
                ("k_src", ctypes.c_void_p), ("v_src", ctypes.c_void_p), ("src_layer_stride", ctypes.c_int64),
                ("k_dst", ctypes.c_void_p), ("v_dst", ctypes.c_void_p), ("dst_layer_stride", ctypes.c_int64),
                ("block_table", ctypes.POINTER(ctypes.c_int32)), ("positions", ctypes.c_void_p),
                ("slot0", ctypes.c_int32),
                ("num_factors", ctypes.c_int32), ("factors", Factor * MAX_FACTORS)]


class Pool(ctypes.Structure):
    _fields_ = [("k_pool", ctypes.c_void_p), ("v_pool", ctypes.c_void_p), ("num_pages", ctypes.c_int32),
                ("reserved", ctypes.c_int32), ("layer_stride", ctypes.c_int64)]


class Plan(ctypes.Structure):
    _fields_ = [("workspace", ctypes.c_void_p), ("num_tasks", ctypes.c_int64), ("kernel", ctypes.c_int32),
                ("variant", ctypes.c_int32), ("num_chunks", ctypes.c_int32), ("reserved", ctypes.c_int32 * 9)]


class KameraError(RuntimeError):
    def __init__(self, status: int, detail: str):
        self.status = status
        self.name = STATUS[status] if 0 <= status < len(STATUS) else f"status {status}"
        super().__init__(f"{self.name}: {detail}")


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built (no fallback exists)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m position_free_kv_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        L.kamera_workspace_bytes.argtypes = [i32, i64]
        L.kamera_workspace_bytes.restype = sz
        L.kamera_batch_workspace_bytes.argtypes = [ctypes.POINTER(Layout), ctypes.POINTER(Chunk), i32]
        L.kamera_batch_workspace_bytes.restype = sz
        L.kamera_relocate.argtypes = [ctypes.POINTER(Layout), ctypes.POINTER(Pool), ctypes.POINTER(ctypes.c_int32),
                                      i32, i32, i64, vp, sz, vp]
        L.kamera_rehydrate.argtypes = [ctypes.POINTER(Layout), ctypes.POINTER(Chunk), ctypes.POINTER(Pool), vp, sz, vp]
        L.kamera_rehydrate_batched.argtypes = [ctypes.POINTER(Layout), ctypes.POINTER(Chunk), i32,
                                               ctypes.POINTER(Pool), vp, sz, vp]
        L.kamera_rehydrate_batched_noalloc.argtypes = [ctypes.POINTER(Layout), ctypes.POINTER(Chunk), i32,
                                                       ctypes.POINTER(Pool), vp]
        L.kamera_plan_upload.argtypes = [ctypes.POINTER(Layout), ctypes.POINTER(Chunk), i32, ctypes.POINTER(Pool),
                                         vp, sz, vp, ctypes.POINTER(Plan)]
        L.kamera_plan_launch.argtypes = [ctypes.POINTER(Plan), vp]
        L.kamera_build_workspace_bytes.argtypes = [i64, i32, i32]
        L.kamera_build_workspace_bytes.restype = sz
        L.kamera_build_patch.argtypes = [ctypes.POINTER(Layout), i32, vp, vp, i64, i64, i32, i32, i32, i32,
                                         vp, vp, vp, vp, sz, vp]
        L.kamera_build_orbit_patch.argtypes = [ctypes.POINTER(Layout), i32, i32, ctypes.POINTER(vp),
                                               ctypes.POINTER(i64), vp, i64, i32, i32, i32, i32, vp, vp, vp, vp,
                                               sz, vp]
        L.kamera_stream_probe.argtypes = [i32, vp, vp, sz, ctypes.c_uint32, vp]
        for fn in ("kamera_stream_probe", "kamera_relocate", "kamera_rehydrate", "kamera_rehydrate_batched",
                   "kamera_rehydrate_batched_noalloc", "kamera_plan_upload",
                   "kamera_plan_launch", "kamera_build_patch", "kamera_build_orbit_patch"):
            getattr(L, fn).restype = ctypes.c_int
        L.kamera_status_string.argtypes = [ctypes.c_int]
        L.kamera_status_string.restype = ctypes.c_char_p
        L.kamera_last_error.argtypes = []
        L.kamera_last_error.restype = ctypes.c_char_p
        L.kamera_version.argtypes = []
        L.kamera_version.restype = ctypes.c_char_p
        _lib = L
    return _lib


def _check(status: int) -> None:
    if status != 0:
        raise KameraError(status, lib().kamera_last_error().decode())


# --------------------------------------------------------------------------- marshalling
def _ptr(x) -> Optional[int]:
    """Device address of a torch tensor, an int address, or None."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return int(x.data_ptr())


def _stream(stream) -> Optional[int]:
    if stream is None:
        try:
            import torch
            if torch.cuda.is_available():
                return int(torch.cuda.current_stream().cuda_stream)
        except Exception:  # noqa: BLE001
            pass
        return None
    if isinstance(stream, int):
        return stream
    return int(stream.cuda_stream)


def make_layout(family: int, dtype: int, num_layers: int, *, num_kv_heads: int = 0, head_dim: int = 0,
                latent_dim: int = 0, rope_dim: int = 0, pairing: int = NEOX, rope_base: float = 10000.0,
                page_size: int = 16, mrope_section: Sequence[int] = (0, 0, 0),
                patch_unit: int = PATCH_UNIT_AUTO) -> Layout:
    return Layout(family, dtype, num_layers, num_kv_heads, head_dim, latent_dim, rope_dim, pairing, page_size,
                  int(patch_unit), float(rope_base), (ctypes.c_int32 * 3)(*[int(v) for v in mrope_section]), 0)


class ChunkDesc:
    """A kamera_chunk plus the host objects it points into (kept alive with it)."""

    def __init__(self, *, num_tokens: int, delta: int, flags: int, k_src=None, v_src=None, src_layer_stride: int = 0,
                 k_dst=None, v_dst=None, dst_layer_stride: int = 0, block_table=None, slot0: int = 0,
                 factors: Sequence[dict] = (), positions=None):
        c = Chunk()
        c.num_tokens, c.flags, c.delta = int(num_tokens), int(flags), int(delta)
        c.k_src, c.v_src, c.src_layer_stride = _ptr(k_src), _ptr(v_src), int(src_layer_stride)
        c.k_dst, c.v_dst, c.dst_layer_stride = _ptr(k_dst), _ptr(v_dst), int(dst_layer_stride)
        self._table = None
        if block_table is not None:
            self._table = np.ascontiguousarray(block_table, dtype=np.int32)
            c.block_table = self._table.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
        c.positions = _ptr(positions)  # device [T][3] int32 offsets (with the POSITIONS flag)
        c.slot0 = int(slot0)
        if len(factors) > MAX_FACTORS:
            raise ValueError(f"at most {MAX_FACTORS} factors per chunk")
        c.num_factors = len(factors)
        for i, f in enumerate(factors):
            c.factors[i] = Factor(_ptr(f["u"]), _ptr(f["v"]), int(f.get("tensor", 0)), int(f.get("col0", 0)),
                                  int(f["width"]), int(f["rank"]), int(f.get("layer0", 0)), 0)
        self.c = c


def make_pool(k_pool, v_pool=None, num_pages: int = 0, layer_stride: int = 0) -> Pool:
    return Pool(_ptr(k_pool), _ptr(v_pool), int(num_pages), 0, int(layer_stride))


def _chunk_array(chunks: Iterable) -> ctypes.Array:
    cs = [c.c if isinstance(c, ChunkDesc) else c for c in chunks]
    arr = (Chunk * max(len(cs), 1))()
    for i, c in enumerate(cs):
        arr[i] = c
    return arr, len(cs)


def workspace_bytes(num_chunks: int, total_block_table_entries: int = 0) -> int:
    return int(lib().kamera_workspace_bytes(int(num_chunks), int(total_block_table_entries)))


def batch_workspace_bytes(layout: Layout, chunks: Sequence) -> int:
    """Workspace needed by exactly this batch (block tables and per-token cos/sin tables included)."""
    arr, n = _chunk_array(chunks)
    return int(lib().kamera_batch_workspace_bytes(ctypes.byref(layout), arr, n))


def _ws(workspace):
    if workspace is None:
        return None, 0
    if isinstance(workspace, tuple):
        return int(workspace[0]), int(workspace[1])
    return int(workspace.data_ptr()), int(workspace.numel() * workspace.element_size())


def build_workspace_bytes(num_tokens: int, width: int, rank: int) -> int:
    return int(lib().kamera_build_workspace_bytes(int(num_tokens), int(width), int(rank)))


def build_patch(layout: Layout, tensor: int, x_cond, x_canon, num_tokens: int, delta: int, col0: int, width: int,
                rank: int, iterations: int, u_out, v_out, sigma_out, workspace, stream=None) -> None:
    """Top-`rank` factors of x_cond - R(delta) x_canon on columns [col0, col0 + width)."""
    wp, wb = _ws(workspace)
    _check(lib().kamera_build_patch(ctypes.byref(layout), int(tensor), _ptr(x_cond), _ptr(x_canon),
                                    int(num_tokens), int(delta), int(col0), int(width), int(rank),
                                    int(iterations), _ptr(u_out), _ptr(v_out), _ptr(sigma_out), wp, wb,
                                    _stream(stream)))


def build_orbit_patch(layout: Layout, tensor: int, x_conds: Sequence, deltas: Sequence[int], x_canon,
                      num_tokens: int, col0: int, width: int, rank: int, iterations: int, u_out, v_out, sigma_out,
                      workspace, stream=None) -> None:
    """Top-`rank` factors of the mean deficit over the orderings (x_conds[k], deltas[k])."""
    k = len(x_conds)
    conds = (ctypes.c_void_p * max(k, 1))(*[_ptr(x) for x in x_conds])
    ds = (ctypes.c_int64 * max(len(deltas), 1))(*[int(d) for d in deltas])
    wp, wb = _ws(workspace)
    _check(lib().kamera_build_orbit_patch(ctypes.byref(layout), int(tensor), k, conds, ds, _ptr(x_canon),
                                          int(num_tokens), int(col0), int(width), int(rank), int(iterations),
                                          _ptr(u_out), _ptr(v_out), _ptr(sigma_out), wp, wb, _stream(stream)))


def relocate(layout: Layout, pool: Pool, block_table, slot0: int, num_tokens: int, delta: int, workspace,
             stream=None) -> None:
    table = None if block_table is None else np.ascontiguousarray(block_table, dtype=np.int32)
    tp = None if table is None else table.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))
    wp, wb = _ws(workspace)
    _check(lib().kamera_relocate(ctypes.byref(layout), ctypes.byref(pool), tp, int(slot0), int(num_tokens),
                                 int(delta), wp, wb, _stream(stream)))


def rehydrate(layout: Layout, chunk, pool: Optional[Pool], workspace, stream=None) -> None:
    c = chunk.c if isinstance(chunk, ChunkDesc) else chunk
    wp, wb = _ws(workspace)
    _check(lib().kamera_rehydrate(ctypes.byref(layout), ctypes.byref(c), ctypes.byref(pool) if pool else None,
                                  wp, wb, _stream(stream)))


def rehydrate_batched(layout: Layout, chunks: Sequence, pool: Optional[Pool], workspace, stream=None) -> None:
    arr, n = _chunk_array(chunks)
    wp, wb = _ws(workspace)
    _check(lib().kamera_rehydrate_batched(ctypes.byref(layout), arr, n, ctypes.byref(pool) if pool else None,
                                          wp, wb, _stream(stream)))


def rehydrate_batched_noalloc(layout: Layout, chunks: Sequence, pool: Optional[Pool], stream=None) -> None:
    """kamera_rehydrate_batched without a workspace: the library's per-device scratch array serves."""
    arr, n = _chunk_array(chunks)
    _check(lib().kamera_rehydrate_batched_noalloc(ctypes.byref(layout), arr, n, ctypes.byref(pool) if pool else None,
                                                  _stream(stream)))


class PreparedBatch:
    """The marshalled arguments of one kamera_rehydrate_batched call, built once.

    `call()` re-issues the same batch (validation, upload and launch all happen
    again in the library) with no per-call Python marshalling.
    """

    def __init__(self, layout: Layout, chunks: Sequence, pool: Optional[Pool], workspace, stream=None):
        self._chunks = list(chunks)          # keeps block tables alive
        self._layout = layout
        self._pool = pool
        self._arr, self._n = _chunk_array(self._chunks)
        self._wp, self._wb = _ws(workspace)
        self._stream = _stream(stream)
        self._args = (ctypes.byref(layout), self._arr, self._n, ctypes.byref(pool) if pool else None,
                      self._wp, self._wb, self._stream)
        self._fn = lib().kamera_rehydrate_batched

    def call(self) -> None:
        st = self._fn(*self._args)
        if st:
            _check(st)


def plan_upload(layout: Layout, chunks: Sequence, pool: Optional[Pool], workspace, stream=None) -> Plan:
    arr, n = _chunk_array(chunks)
    wp, wb = _ws(workspace)
    plan = Plan()
    _check(lib().kamera_plan_upload(ctypes.byref(layout), arr, n, ctypes.byref(pool) if pool else None, wp, wb,
                                    _stream(stream), ctypes.byref(plan)))
    return plan


def plan_launch(plan: Plan, stream=None) -> None:
    _check(lib().kamera_plan_launch(ctypes.byref(plan), _stream(stream)))


def stream_probe(kind: int, src, dst, nbytes: int, value: int = 0, stream=None) -> None:
    """Streaming probe (measurement only): copy src -> dst, read src (dst a 4 KB sink), or write dst."""
    _check(lib().kamera_stream_probe(int(kind), _ptr(src), _ptr(dst), int(nbytes), int(value) & 0xffffffff,
                                     _stream(stream)))


def version() -> str:
    return lib().kamera_version().decode()
