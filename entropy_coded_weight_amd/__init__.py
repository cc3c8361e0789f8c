"""Entropy-coded weight decoding on AMD MI355X (gfx950).

A thin ctypes binding of ``libentq.so`` (built from ``csrc/`` by
``build.build()``): argument marshalling only. Every step of the decode runs
in the library's HIP kernels; the host encoder is the library's multi-threaded
C++. PyTorch supplies device memory and streams. There is no fallback: if
the library is missing, importing the decode entry points fails loudly.

Entry points (the C ABI in include/entq.h, same names):
  plan(...)               -> Plan     validate a batch, build device tables
  decode(...)                         rANS decode to codes or bf16 (fused
                                      per-row fp32 scale, RNE)
  decode_bf16_split(...)              exponent stream + raw sign/mantissa
                                      bytes -> bit-exact bf16
  count_symbols, build_freq, encode_tensor, bf16_split   host encoder
  encode_batch(...)       -> Batch    convenience: a list of tensors -> blob,
                                      tables, chunk index
  count_symbols_device, encode_device, pack_device, region_bytes
                                      on-device encoder (same regions)
  encode_batch_device(...) -> DeviceBatch  the device path of encode_batch
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import numpy as np

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libentq.so")

KIND_INT8, KIND_E4M3, KIND_BF16EXP = 0, 1, 2
LAYOUT_TILES = 0x100  # or'ed into a tensor's kind: its symbols are in tile order
OUT_CODES, OUT_BF16 = 0, 1
CHUNK_OK, CHUNK_BAD_STATE, CHUNK_BAD_WORDS = 0, 1, 2
PROB_SCALE = 4096

TENSOR_DESC = np.dtype([("kind", "<u4"), ("rows", "<u4"), ("cols", "<u4"),
                        ("chunk_symbols", "<u4"), ("n_symbols", "<u8"),
                        ("out_elem_offset", "<u8"), ("scale_row_offset", "<u8")])
CHUNK_DESC = np.dtype([("tensor", "<u4"), ("n_symbols", "<u4"), ("n_words", "<u4"),
                       ("reserved", "<u4"), ("byte_offset", "<u8"), ("elem_offset", "<u8")])
assert TENSOR_DESC.itemsize == 40 and CHUNK_DESC.itemsize == 32
# entq_gemm_io (include/entq.h): device pointers as integers
GEMM_IO = np.dtype([("x", "<u8"), ("ldx", "<u8"), ("y", "<u8"), ("ldy", "<u8")])
# entq_count_job / entq_pack_job (include/entq.h): device pointers as integers
COUNT_JOB = np.dtype([("symbols", "<u8"), ("n_symbols", "<u8"), ("counts", "<u8")])
PACK_JOB = np.dtype([("scratch", "<u8"), ("n_symbols", "<u8"), ("chunk_symbols", "<u4"),
                     ("reserved", "<u4"), ("n_words", "<u8"), ("offsets", "<u8")])
# entq_encode_job (include/entq.h): device pointers as integers
CHUNK_COUNT_JOB = np.dtype([("symbols", "<u8"), ("n_symbols", "<u8"), ("chunk_symbols", "<u4"),
                            ("reserved", "<u4"), ("counts", "<u8")])
PACK_ADAPTIVE_JOB = np.dtype([("scratch", "<u8"), ("n_symbols", "<u8"), ("chunk_symbols", "<u4"),
                              ("reserved", "<u4"), ("n_words", "<u8"), ("offsets", "<u8"),
                              ("freq", "<u8")])
ENCODE_JOB = np.dtype([("symbols", "<u8"), ("n_symbols", "<u8"), ("chunk_symbols", "<u4"),
                       ("reserved", "<u4"), ("freq", "<u8"), ("scratch", "<u8"),
                       ("scratch_bytes", "<u8"), ("n_words", "<u8")])


class EntqError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {_str(status)} ({status})")


_lib = None


def lib():
    """The loaded libentq.so. Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "entropy_coded_weight_amd.build.build() (no CPU fallback exists)")
        L = ctypes.CDLL(LIB_PATH)
        c = ctypes
        vp, u64, i64 = c.c_void_p, c.c_uint64, c.c_int64
        sigs = {
            "entq_plan_workspace_bytes": (c.c_size_t, [c.c_int, i64]),
            "entq_plan": (c.c_int, [vp, c.c_int, vp, vp, i64, u64, vp, c.c_size_t, vp,
                                    c.POINTER(vp)]),
            "entq_decode": (c.c_int, [vp, vp, vp, c.c_int, vp, vp, vp]),
            "entq_decode_bf16_split": (c.c_int, [vp, vp, vp, vp, vp, vp]),
            "entq_plan_destroy": (None, [vp]),
            "entq_status_str": (c.c_char_p, [c.c_int]),
            "entq_plan_info": (c.c_int, [vp, vp, vp, vp, vp, vp]),
            "entq_count_symbols": (c.c_int, [vp, u64, vp, c.c_int]),
            "entq_build_freq": (c.c_int, [vp, vp]),
            "entq_encode_bound": (u64, [u64, c.c_uint32]),
            "entq_encode_tensor": (c.c_int, [vp, u64, c.c_uint32, vp, c.c_uint32, u64, vp, u64,
                                             vp, vp, c.c_int]),
            "entq_bf16_split": (c.c_int, [vp, u64, vp, vp, c.c_int]),
            "entq_count_symbols_device": (c.c_int, [vp, u64, vp, vp]),
            "entq_encode_device_scratch_bytes": (u64, [u64, c.c_uint32]),
            "entq_region_bytes": (u64, [c.c_uint32]),
            "entq_encode_device": (c.c_int, [vp, u64, c.c_uint32, vp, vp, u64, vp, vp]),
            "entq_pack_device": (c.c_int, [vp, u64, c.c_uint32, vp, vp, vp, vp]),
            "entq_region_offsets_device": (c.c_int, [vp, u64, u64, vp, vp, vp]),
            "entq_encode_device_batch": (c.c_int, [vp, c.c_int, vp]),
            "entq_decode_gemm": (c.c_int, [vp, vp, vp, vp, c.c_int, vp, u64, vp, vp]),
            "entq_decode_gemm_workspace_bytes": (u64, [vp, c.c_int]),
            "entq_plan_adaptive": (c.c_int, [vp, c.c_int, vp, i64, u64, vp, c.c_size_t, vp,
                                             c.POINTER(vp)]),
            "entq_encode_tensor_adaptive": (c.c_int, [vp, u64, c.c_uint32, c.c_uint32, u64, vp,
                                                      u64, vp, vp, c.c_int]),
            "entq_encode_bound_adaptive": (u64, [u64, c.c_uint32]),
            "entq_count_symbols_device_batch": (c.c_int, [vp, c.c_int, vp]),
            "entq_pack_device_batch": (c.c_int, [vp, c.c_int, vp, vp]),
            "entq_decode_gemm_bf16_split": (c.c_int, [vp, vp, vp, vp, c.c_int, vp, u64, vp,
                                                      vp]),
            "entq_count_chunks_device_batch": (c.c_int, [vp, c.c_int, vp]),
            "entq_build_freq_chunks": (c.c_int, [vp, u64, vp, c.c_int]),
            "entq_encode_device_adaptive_batch": (c.c_int, [vp, c.c_int, vp]),
            "entq_region_offsets_device_adaptive": (c.c_int, [vp, u64, u64, vp, vp, vp]),
            "entq_pack_device_adaptive_batch": (c.c_int, [vp, c.c_int, vp, vp]),
            "entq_build_freq_device": (c.c_int, [vp, c.c_uint32, u64, vp, vp]),
            "entq_decode_gemm_static": (c.c_int, [vp, vp, vp, vp, c.c_int, vp, vp]),
            "entq_tile_order": (c.c_int, [vp, c.c_uint32, c.c_uint32, c.c_uint32, vp, c.c_int]),
            "entq_tile_order_device": (c.c_int, [vp, c.c_uint32, c.c_uint32, c.c_uint32, vp, vp]),
            "entq_decode_gemm_tiles_workspace_bytes": (u64, [vp, c.c_int]),
            "entq_decode_gemm_tiles": (c.c_int, [vp, vp, vp, vp, c.c_int, vp, u64, vp, vp]),
            "entq_decode_gemm_tiles_bf16_split": (c.c_int, [vp, vp, vp, vp, c.c_int, vp, u64, vp,
                                                            vp]),
        }
        for name, (res, args) in sigs.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


EXPORTED = ["entq_plan_workspace_bytes", "entq_plan", "entq_decode", "entq_decode_bf16_split",
            "entq_plan_destroy", "entq_status_str", "entq_plan_info", "entq_count_symbols",
            "entq_build_freq", "entq_encode_bound", "entq_encode_tensor", "entq_bf16_split",
            "entq_count_symbols_device", "entq_encode_device_scratch_bytes", "entq_region_bytes",
            "entq_encode_device", "entq_pack_device", "entq_region_offsets_device",
            "entq_encode_device_batch", "entq_decode_gemm", "entq_plan_adaptive",
            "entq_encode_tensor_adaptive", "entq_encode_bound_adaptive",
            "entq_count_symbols_device_batch", "entq_pack_device_batch",
            "entq_decode_gemm_bf16_split", "entq_count_chunks_device_batch",
            "entq_build_freq_chunks", "entq_encode_device_adaptive_batch",
            "entq_region_offsets_device_adaptive", "entq_pack_device_adaptive_batch",
            "entq_build_freq_device", "entq_decode_gemm_workspace_bytes",
            "entq_decode_gemm_static", "entq_tile_order", "entq_decode_gemm_tiles_workspace_bytes",
            "entq_decode_gemm_tiles", "entq_decode_gemm_tiles_bf16_split",
            "entq_tile_order_device"]


def _str(status: int) -> str:
    try:
        return lib().entq_status_str(status).decode()
    except Exception:  # noqa: BLE001 - message only
        return "unknown"


def _check(status: int, what: str):
    if status != 0:
        raise EntqError(status, what)


def _ptr(a) -> int:
    """Address of a numpy array or a torch tensor (host or device)."""
    if a is None:
        return 0
    if isinstance(a, np.ndarray):
        assert a.flags["C_CONTIGUOUS"]
        return a.ctypes.data
    assert a.is_contiguous()
    return a.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def default_threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


# --------------------------------------------------------------------------
# plan and decode
# --------------------------------------------------------------------------

class Plan:
    """A validated batch with its device workspace (a torch uint8 tensor that
    this object keeps alive). The workspace is uploaded on ``stream`` (the
    current stream by default): work on another stream must be ordered after
    it, and the Plan must outlive every decode that uses it."""

    def __init__(self, tensors: np.ndarray, freq_tables, chunk_index: np.ndarray,
                 blob_bytes: int, device="cuda", stream=None):
        """freq_tables None: the chunks carry their own tables
        (entq_plan_adaptive)."""
        import torch
        tensors = np.ascontiguousarray(tensors, dtype=TENSOR_DESC)
        chunk_index = np.ascontiguousarray(chunk_index, dtype=CHUNK_DESC)
        adaptive = freq_tables is None
        if not adaptive:
            freq_tables = np.ascontiguousarray(freq_tables, dtype=np.uint16).reshape(-1, 256)
            assert freq_tables.shape[0] == tensors.shape[0]
        n_t, n_c = int(tensors.shape[0]), int(chunk_index.shape[0])
        ws_bytes = int(lib().entq_plan_workspace_bytes(n_t, n_c))
        raw = torch.empty(ws_bytes + 256, dtype=torch.uint8, device=device)
        shift = (-raw.data_ptr()) % 256
        self.workspace = raw[shift:shift + ws_bytes]
        self._raw = raw
        h = ctypes.c_void_p()
        if adaptive:
            st = lib().entq_plan_adaptive(_ptr(tensors) if n_t else None, n_t,
                                          _ptr(chunk_index) if n_c else None, n_c,
                                          int(blob_bytes), self.workspace.data_ptr(), ws_bytes,
                                          _stream(stream), ctypes.byref(h))
        else:
            st = lib().entq_plan(_ptr(tensors) if n_t else None, n_t,
                                 _ptr(freq_tables) if n_t else None,
                                 _ptr(chunk_index) if n_c else None, n_c, int(blob_bytes),
                                 self.workspace.data_ptr(), ws_bytes, _stream(stream),
                                 ctypes.byref(h))
        _check(st, "entq_plan_adaptive" if adaptive else "entq_plan")
        self.adaptive = adaptive
        self._h = h
        self.n_tensors, self.n_chunks = n_t, n_c
        self.tensors = tensors
        self.blob_bytes = int(blob_bytes)
        oe, sr, nc, nt_, bb = (ctypes.c_uint64(), ctypes.c_uint64(), ctypes.c_int64(),
                               ctypes.c_int(), ctypes.c_uint64())
        _check(lib().entq_plan_info(h, ctypes.byref(oe), ctypes.byref(sr), ctypes.byref(nc),
                                    ctypes.byref(nt_), ctypes.byref(bb)), "entq_plan_info")
        self.out_elems, self.scale_rows = int(oe.value), int(sr.value)

    @property
    def device(self):
        return self.workspace.device

    @property
    def handle(self):
        return self._h

    def close(self):
        if getattr(self, "_h", None) is not None and self._h.value:
            lib().entq_plan_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:  # noqa: BLE001 - interpreter shutdown
            pass


def plan(tensors, freq_tables, chunk_index, blob_bytes, device="cuda", stream=None) -> Plan:
    return Plan(tensors, freq_tables, chunk_index, blob_bytes, device, stream)


EINVAL, EWORKSPACE, ETOOLARGE = -1, -5, -9
# bytes of the static device scratch behind decode_gemm_static (include/entq.h)
GEMM_STATIC_SCRATCH_BYTES = 16 << 20


def _device_buffer(p: Plan, name: str, t, min_elems: int, elem_size: int | None = None,
                   dtypes=None):
    """Checks one device buffer argument against the plan before a launch:
    the kernels dereference raw pointers, so a buffer that is too small, of
    the wrong element size or on another device must be refused here."""
    import torch
    if not isinstance(t, torch.Tensor):
        raise EntqError(EINVAL, f"{name}: a torch tensor on {p.device} is required")
    if t.device != p.device:
        raise EntqError(EINVAL, f"{name} is on {t.device}, the plan on {p.device}")
    if not t.is_contiguous():
        raise EntqError(EINVAL, f"{name} is not contiguous")
    if dtypes is not None and t.dtype not in dtypes:
        raise EntqError(EINVAL, f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if elem_size is not None and t.element_size() != elem_size:
        raise EntqError(EINVAL, f"{name} has {t.element_size()}-byte elements, expected "
                                f"{elem_size}")
    if t.numel() < min_elems:
        raise EntqError(EINVAL, f"{name} holds {t.numel()} elements, the plan needs {min_elems}")


def _dev(name: str, t, min_elems: int = 0, dtypes=None, device=None):
    """Checks a device buffer of a call that has no plan (the device
    encoder, the device tile order): a contiguous torch tensor on a GPU (on
    ``device`` when given), of one of ``dtypes``, with at least
    ``min_elems`` elements -- the kernels dereference its raw pointer, so a
    host tensor or a short buffer must be refused before the launch."""
    import torch
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise EntqError(EINVAL, f"{name}: a torch tensor on a GPU is required")
    if device is not None and t.device != device:
        raise EntqError(EINVAL, f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise EntqError(EINVAL, f"{name} is not contiguous")
    if dtypes is not None and t.dtype not in dtypes:
        raise EntqError(EINVAL, f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if t.numel() < min_elems:
        raise EntqError(EINVAL, f"{name} holds {t.numel()} elements, {min_elems} needed")


def _bytes_dtypes():
    import torch
    return (torch.uint8, torch.int8)


def _freq_dtypes():
    import torch
    return tuple(d for d in (torch.int16, getattr(torch, "uint16", None)) if d is not None)


def _n_chunks(n: int, chunk_symbols: int) -> int:
    if chunk_symbols <= 0:
        raise EntqError(EINVAL, f"chunk_symbols {chunk_symbols}")
    return -(-int(n) // int(chunk_symbols))


def _check_symbols(name: str, sym):
    _dev(name, sym, dtypes=_bytes_dtypes())
    return sym.device


def _status_buffer(p: Plan, chunk_status):
    import torch
    if chunk_status is not None:
        _device_buffer(p, "chunk_status", chunk_status, p.n_chunks, dtypes=(torch.int32,))


def _blob_buffer(p: Plan, name: str, t):
    import torch
    if not isinstance(t, torch.Tensor):
        raise EntqError(EINVAL, f"{name}: a torch tensor on {p.device} is required")
    _device_buffer(p, name, t, -(-p.blob_bytes // t.element_size()))


def decode(p: Plan, compressed, out, out_kind: int, scales=None, chunk_status=None,
           stream=None):
    """Enqueue the decode of every chunk of ``p`` on ``stream``. All buffers
    are device tensors on the plan's device: compressed (the blob, at least
    blob_bytes), out (1-byte elements for OUT_CODES, 2-byte bf16/int16/uint16
    for OUT_BF16, at least out_elems), scales (float32, at least scale_rows;
    OUT_BF16 only), chunk_status (int32 [n_chunks]) or None."""
    import torch
    if out_kind not in (OUT_CODES, OUT_BF16):
        raise EntqError(EINVAL, f"out_kind {out_kind}")
    _blob_buffer(p, "compressed", compressed)
    _device_buffer(p, "out", out, p.out_elems, elem_size=1 if out_kind == OUT_CODES else 2)
    if out_kind == OUT_BF16:
        if scales is None:
            raise EntqError(EINVAL, "scales are required for OUT_BF16")
        _device_buffer(p, "scales", scales, p.scale_rows, dtypes=(torch.float32,))
    else:
        scales = None
    _status_buffer(p, chunk_status)
    st = lib().entq_decode(p.handle, _ptr(compressed), _ptr(out), int(out_kind),
                           _ptr(scales) or None, _ptr(chunk_status) or None, _stream(stream))
    _check(st, "entq_decode")


def _gemm_io(p: Plan, xs, ys):
    """io[] of the fused calls; every activation and result matrix is checked
    against its tensor's shape (x: bf16 [m, >= cols], y: float32 [m, >=
    rows], rows unit-stride, on the plan's device)."""
    import torch
    if not (len(xs) == len(ys) == p.n_tensors):
        raise EntqError(EINVAL, f"{len(xs)} activation and {len(ys)} result matrices for "
                                f"{p.n_tensors} tensors")
    m = xs[0].shape[0] if xs else 0
    io = np.zeros(len(xs), GEMM_IO)
    for t, (x, y) in enumerate(zip(xs, ys)):
        rows, cols = int(p.tensors[t]["rows"]), int(p.tensors[t]["cols"])
        for name, a, dt, width in (("x", x, torch.bfloat16, cols), ("y", y, torch.float32, rows)):
            if not isinstance(a, torch.Tensor) or a.device != p.device:
                raise EntqError(EINVAL, f"{name}[{t}] must be a tensor on {p.device}")
            if a.dtype != dt or a.dim() != 2 or a.shape[0] != m or a.stride(1) != 1:
                raise EntqError(EINVAL, f"{name}[{t}]: {a.dtype} {tuple(a.shape)} stride "
                                        f"{tuple(a.stride())}; expected {dt} [{m}, >= {width}] "
                                        "with unit-stride rows")
            if a.shape[1] < width:
                raise EntqError(EINVAL, f"{name}[{t}] has {a.shape[1]} columns, tensor {t} "
                                        f"needs {width}")
        io[t] = (_ptr(x), x.stride(0), _ptr(y), y.stride(0))
    return io, m


def _gemm_workspace(p: Plan, m: int, workspace):
    """The packed-activation workspace for m rows: None when m <= 16 (no
    gain there) unless given; "none" forces the unpacked reads."""
    import torch
    if isinstance(workspace, str) and workspace == "none":
        return None, 0
    if workspace is None:
        if m <= 16:
            return None, 0
        n = int(lib().entq_decode_gemm_workspace_bytes(p.handle, int(m)))
        raw = torch.empty(n + 256, dtype=torch.uint8, device=p.workspace.device)
        shift = (-raw.data_ptr()) % 256
        workspace = raw[shift:shift + n]
        return workspace, n
    need = int(lib().entq_decode_gemm_workspace_bytes(p.handle, int(m))) if p.handle.value else 0
    _device_buffer(p, "workspace", workspace, need, elem_size=1)
    return workspace, workspace.numel()


def decode_gemm(p: Plan, compressed, scales, xs, ys, chunk_status=None, stream=None,
                workspace=None):
    """Y_t = X_t . W_t^T for every tensor t of the plan, W_t the bf16 weights
    the bf16 decode would write, without writing them: xs[t] is a device
    bfloat16 tensor [m, ldx >= cols] (m <= 64, the same m for all), ys[t] a
    device float32 tensor [m, ldy >= rows]. workspace: a device uint8 tensor
    (256-byte aligned, entq_decode_gemm_workspace_bytes long) for the packed
    activations, None to allocate one when m > 16, or "none"."""
    import torch
    io, m = _gemm_io(p, xs, ys)
    _blob_buffer(p, "compressed", compressed)
    _device_buffer(p, "scales", scales, p.scale_rows, dtypes=(torch.float32,))
    _status_buffer(p, chunk_status)
    ws, wsb = _gemm_workspace(p, m, workspace)
    if ws is not None and workspace is None and stream is not None:
        ws.record_stream(stream)  # allocated here, used on another stream
    st = lib().entq_decode_gemm(p.handle, _ptr(compressed), _ptr(scales) or None,
                                _ptr(io) if len(xs) else None, int(m),
                                _ptr(ws) if ws is not None else None, int(wsb),
                                _ptr(chunk_status) or None, _stream(stream))
    _check(st, "entq_decode_gemm")


def decode_gemm_static(p: Plan, compressed, scales, xs, ys, chunk_status=None, stream=None):
    """decode_gemm with the packed activations in the library's static
    device scratch (entq_decode_gemm_static): no workspace, no allocation,
    results bit for bit those of decode_gemm. Raises EntqError(ETOOLARGE)
    when the packed activations would exceed GEMM_STATIC_SCRATCH_BYTES.
    Calls on one GPU share the scratch: overlapping calls race."""
    import torch
    io, m = _gemm_io(p, xs, ys)
    _blob_buffer(p, "compressed", compressed)
    _device_buffer(p, "scales", scales, p.scale_rows, dtypes=(torch.float32,))
    _status_buffer(p, chunk_status)
    st = lib().entq_decode_gemm_static(p.handle, _ptr(compressed), _ptr(scales) or None,
                                       _ptr(io) if len(xs) else None, int(m),
                                       _ptr(chunk_status) or None, _stream(stream))
    _check(st, "entq_decode_gemm_static")


def decode_gemm_bf16_split(p: Plan, exp_stream, signmant, xs, ys, chunk_status=None,
                           stream=None, workspace=None):
    """decode_gemm for BF16 weights given as a coded exponent stream plus raw
    sign+mantissa bytes (as decode_bf16_split takes them)."""
    io, m = _gemm_io(p, xs, ys)
    _blob_buffer(p, "exp_stream", exp_stream)
    _device_buffer(p, "signmant", signmant, p.out_elems, elem_size=1)
    _status_buffer(p, chunk_status)
    ws, wsb = _gemm_workspace(p, m, workspace)
    if ws is not None and workspace is None and stream is not None:
        ws.record_stream(stream)
    st = lib().entq_decode_gemm_bf16_split(p.handle, _ptr(exp_stream), _ptr(signmant),
                                           _ptr(io) if len(xs) else None, int(m),
                                           _ptr(ws) if ws is not None else None, int(wsb),
                                           _ptr(chunk_status) or None, _stream(stream))
    _check(st, "entq_decode_gemm_bf16_split")


def tile_order(codes: np.ndarray, rows: int, cols: int, chunk_cols: int,
               n_threads: int | None = None) -> np.ndarray:
    """The symbols of a row-major [rows, cols] tensor in tile order for chunks
    of 16 rows x chunk_cols columns (entq_tile_order); encode them with
    chunk_symbols = 16 * chunk_cols for decode_gemm_tiles."""
    codes = np.ascontiguousarray(codes).view(np.uint8).ravel()
    if codes.size != rows * cols:
        raise EntqError(EINVAL, f"{codes.size} codes for a {rows} x {cols} tensor")
    out = np.empty(codes.size, np.uint8)
    _check(lib().entq_tile_order(_ptr(codes) if codes.size else None, rows, cols, chunk_cols,
                                 _ptr(out) if out.size else None, n_threads or default_threads()),
           "entq_tile_order")
    return out


def _tiles_workspace(p: Plan, m: int, workspace, stream):
    """The workspace of the tiled product (packed activations, partial sums):
    the given one after its checks, or one allocated here."""
    import torch
    need = int(lib().entq_decode_gemm_tiles_workspace_bytes(p.handle, int(m))) if p.handle.value \
        else 0
    if workspace is None:
        if need:
            raw = torch.empty(need + 256, dtype=torch.uint8, device=p.workspace.device)
            shift = (-raw.data_ptr()) % 256
            workspace = raw[shift:shift + need]
            if stream is not None:
                workspace.record_stream(stream)  # allocated here, used on another stream
    else:
        _device_buffer(p, "workspace", workspace, need, elem_size=1)
    return workspace, (workspace.numel() if workspace is not None else 0)


def tile_order_device(codes, rows: int, cols: int, chunk_cols: int, out=None, stream=None):
    """tile_order on the device: codes a device tensor of rows x cols bytes
    (row-major, 4-byte aligned); returns (or fills) a device uint8 tensor."""
    import torch
    _dev("codes", codes)
    if codes.numel() * codes.element_size() != rows * cols:
        raise EntqError(EINVAL, f"codes must be {rows} x {cols} contiguous bytes")
    if out is None:
        out = torch.empty(rows * cols, dtype=torch.uint8, device=codes.device)
    else:
        _dev("out", out, 0, None, codes.device)
        if out.numel() * out.element_size() < rows * cols:
            raise EntqError(EINVAL, "out must hold rows x cols bytes on the codes' device")
    _check(lib().entq_tile_order_device(_ptr(codes) or None, rows, cols, chunk_cols,
                                        _ptr(out) or None, _stream(stream)),
           "entq_tile_order_device")
    return out


def decode_gemm_tiles(p: Plan, compressed, scales, xs, ys, chunk_status=None, stream=None,
                      workspace=None):
    """decode_gemm for a plan of tile-ordered tensors (entq_decode_gemm_tiles):
    xs, ys as for decode_gemm (m <= 64). workspace: a device uint8 tensor
    (256-byte aligned, entq_decode_gemm_tiles_workspace_bytes long) for the
    packed activations and the column chunks' partial sums, or None to
    allocate one."""
    import torch
    io, m = _gemm_io(p, xs, ys)
    _blob_buffer(p, "compressed", compressed)
    _device_buffer(p, "scales", scales, p.scale_rows, dtypes=(torch.float32,))
    _status_buffer(p, chunk_status)
    ws, wsb = _tiles_workspace(p, m, workspace, stream)
    st = lib().entq_decode_gemm_tiles(p.handle, _ptr(compressed), _ptr(scales) or None,
                                      _ptr(io) if len(xs) else None, int(m),
                                      _ptr(ws) if ws is not None else None, int(wsb),
                                      _ptr(chunk_status) or None, _stream(stream))
    _check(st, "entq_decode_gemm_tiles")


def decode_gemm_tiles_bf16_split(p: Plan, exp_stream, signmant, xs, ys, chunk_status=None,
                                 stream=None, workspace=None):
    """decode_gemm_tiles for tile-ordered BF16 exponent streams: signmant (1-byte
    elements, at least out_elems) holds the sign+mantissa bytes in the same
    tile order as the exponents."""
    io, m = _gemm_io(p, xs, ys)
    _blob_buffer(p, "exp_stream", exp_stream)
    _device_buffer(p, "signmant", signmant, p.out_elems, elem_size=1)
    _status_buffer(p, chunk_status)
    ws, wsb = _tiles_workspace(p, m, workspace, stream)
    st = lib().entq_decode_gemm_tiles_bf16_split(p.handle, _ptr(exp_stream), _ptr(signmant),
                                                 _ptr(io) if len(xs) else None, int(m),
                                                 _ptr(ws) if ws is not None else None, int(wsb),
                                                 _ptr(chunk_status) or None, _stream(stream))
    _check(st, "entq_decode_gemm_tiles_bf16_split")


def decode_bf16_split(p: Plan, exp_stream, signmant, out, chunk_status=None, stream=None):
    """Exponent stream (the blob) + raw sign/mantissa bytes (1-byte elements,
    at least out_elems) -> bf16 words in out (2-byte elements, at least
    out_elems); all on the plan's device."""
    _blob_buffer(p, "exp_stream", exp_stream)
    _device_buffer(p, "signmant", signmant, p.out_elems, elem_size=1)
    _device_buffer(p, "out", out, p.out_elems, elem_size=2)
    _status_buffer(p, chunk_status)
    st = lib().entq_decode_bf16_split(p.handle, _ptr(exp_stream), _ptr(signmant), _ptr(out),
                                      _ptr(chunk_status) or None, _stream(stream))
    _check(st, "entq_decode_bf16_split")


# --------------------------------------------------------------------------
# host encoder
# --------------------------------------------------------------------------

def count_symbols(symbols: np.ndarray, n_threads: int | None = None) -> np.ndarray:
    symbols = np.ascontiguousarray(symbols).view(np.uint8).ravel()
    counts = np.zeros(256, np.uint64)
    _check(lib().entq_count_symbols(_ptr(symbols) if symbols.size else None, symbols.size,
                                    _ptr(counts), n_threads or default_threads()),
           "entq_count_symbols")
    return counts


def build_freq(counts: np.ndarray) -> np.ndarray:
    counts = np.ascontiguousarray(counts, dtype=np.uint64)
    freq = np.zeros(256, np.uint16)
    _check(lib().entq_build_freq(_ptr(counts), _ptr(freq)), "entq_build_freq")
    return freq


def encode_tensor(symbols: np.ndarray, chunk_symbols: int, freq: np.ndarray, tensor_id: int = 0,
                  base_offset: int = 0, n_threads: int | None = None):
    """Returns (region bytes uint8, chunk descriptors CHUNK_DESC)."""
    symbols = np.ascontiguousarray(symbols).view(np.uint8).ravel()
    freq = np.ascontiguousarray(freq, dtype=np.uint16)
    n = symbols.size
    cap = int(lib().entq_encode_bound(n, chunk_symbols))
    out = np.empty(max(cap, 16), np.uint8)
    k = -(-n // chunk_symbols)
    chunks = np.zeros(max(k, 1), CHUNK_DESC)
    written = ctypes.c_uint64()
    _check(lib().entq_encode_tensor(_ptr(symbols) if n else None, n, chunk_symbols, _ptr(freq),
                                    tensor_id, base_offset, _ptr(out), out.size, _ptr(chunks),
                                    ctypes.byref(written), n_threads or default_threads()),
           "entq_encode_tensor")
    return out[:written.value], chunks[:k]


def encode_tensor_adaptive(symbols: np.ndarray, chunk_symbols: int, tensor_id: int = 0,
                           base_offset: int = 0, n_threads: int | None = None):
    """encode_tensor with per-chunk tables (each region starts with its own
    u16 freq[256]). Returns (region bytes uint8, chunk descriptors)."""
    symbols = np.ascontiguousarray(symbols).view(np.uint8).ravel()
    n = symbols.size
    cap = int(lib().entq_encode_bound_adaptive(n, chunk_symbols))
    out = np.empty(max(cap, 16), np.uint8)
    k = -(-n // chunk_symbols)
    chunks = np.zeros(max(k, 1), CHUNK_DESC)
    written = ctypes.c_uint64()
    _check(lib().entq_encode_tensor_adaptive(_ptr(symbols) if n else None, n, chunk_symbols,
                                             tensor_id, base_offset, _ptr(out), out.size,
                                             _ptr(chunks), ctypes.byref(written),
                                             n_threads or default_threads()),
           "entq_encode_tensor_adaptive")
    return out[:written.value], chunks[:k]


def bf16_split(words: np.ndarray, n_threads: int | None = None):
    words = np.ascontiguousarray(words).view(np.uint16).ravel()
    e = np.empty(words.size, np.uint8)
    sm = np.empty(words.size, np.uint8)
    _check(lib().entq_bf16_split(_ptr(words) if words.size else None, words.size,
                                 _ptr(e) if words.size else None,
                                 _ptr(sm) if words.size else None,
                                 n_threads or default_threads()), "entq_bf16_split")
    return e, sm


@dataclass
class Batch:
    """A batch of tensors in compressed form, as entq_plan consumes it."""
    blob: np.ndarray            # uint8, all chunk regions
    tensors: np.ndarray         # TENSOR_DESC
    freq: np.ndarray            # uint16 [n_tensors, 256]
    chunks: np.ndarray          # CHUNK_DESC

    @property
    def out_elems(self) -> int:
        t = self.tensors
        return int((t["out_elem_offset"] + t["n_symbols"]).max()) if t.size else 0

    @property
    def scale_rows(self) -> int:
        t = self.tensors
        return int((t["scale_row_offset"] + t["rows"]).max()) if t.size else 0


def encode_batch(specs, n_threads: int | None = None) -> Batch:
    """specs: list of dicts {kind, rows, cols, chunk_symbols, symbols (uint8
    codes or exponent bytes, rows*cols)}. Tensors are laid out one after the
    other in the output and in the scale array; each gets its own table."""
    regions, descs = [], []
    tens = np.zeros(len(specs), TENSOR_DESC)
    freqs = np.zeros((len(specs), 256), np.uint16)
    off = out_off = scale_off = 0
    for t, sp in enumerate(specs):
        sym = np.ascontiguousarray(sp["symbols"]).view(np.uint8).ravel()
        rows, cols, C = int(sp["rows"]), int(sp["cols"]), int(sp["chunk_symbols"])
        assert sym.size == rows * cols
        f = build_freq(count_symbols(sym, n_threads))
        if sym.size == 0:
            f[0] = PROB_SCALE
        r, ch = encode_tensor(sym, C, f, t, off, n_threads)
        regions.append(r)
        descs.append(ch)
        off += r.size
        tens[t] = (int(sp["kind"]), rows, cols, C, sym.size, out_off, scale_off)
        freqs[t] = f
        out_off += sym.size
        scale_off += rows
    blob = np.concatenate(regions) if regions else np.zeros(0, np.uint8)
    chunks = np.concatenate(descs) if descs else np.zeros(0, CHUNK_DESC)
    return Batch(blob, tens, freqs, chunks)


def encode_batch_adaptive(specs, n_threads: int | None = None) -> Batch:
    """encode_batch with per-chunk tables; the Batch's freq is None (pass it
    to plan() as such)."""
    regions, descs = [], []
    tens = np.zeros(len(specs), TENSOR_DESC)
    off = out_off = scale_off = 0
    for t, sp in enumerate(specs):
        sym = np.ascontiguousarray(sp["symbols"]).view(np.uint8).ravel()
        rows, cols, C = int(sp["rows"]), int(sp["cols"]), int(sp["chunk_symbols"])
        assert sym.size == rows * cols
        r, ch = encode_tensor_adaptive(sym, C, t, off, n_threads)
        regions.append(r)
        descs.append(ch)
        off += r.size
        tens[t] = (int(sp["kind"]), rows, cols, C, sym.size, out_off, scale_off)
        out_off += sym.size
        scale_off += rows
    blob = np.concatenate(regions) if regions else np.zeros(0, np.uint8)
    chunks = np.concatenate(descs) if descs else np.zeros(0, CHUNK_DESC)
    return Batch(blob, tens, None, chunks)


# --------------------------------------------------------------------------
# on-device encoder
# --------------------------------------------------------------------------

def _check_pack_job(scratch, n, C, nw, offs, blob, what=""):
    import torch
    _dev(what + "blob", blob, 0, _bytes_dtypes())
    k = _n_chunks(n, C)
    _dev(what + "scratch", scratch, 0, _bytes_dtypes(), blob.device)
    _dev(what + "n_words", nw, k, (torch.int32,), blob.device)
    _dev(what + "offsets", offs, k, (torch.int64,), blob.device)


def _check_encode_job(sym, C, freq, scratch, nw, freq_entries, what=""):
    import torch
    dev = _check_symbols(what + "symbols", sym)
    k = _n_chunks(sym.numel(), C)
    _dev(what + "freq", freq, freq_entries, _freq_dtypes(), dev)
    _dev(what + "scratch", scratch, 0, _bytes_dtypes(), dev)
    _dev(what + "n_words", nw, k, (torch.int32,), dev)


def _check_offsets_args(n_words, offsets, end):
    import torch
    _dev("n_words", n_words, 0, (torch.int32,))
    _dev("offsets", offsets, n_words.numel(), (torch.int64,), n_words.device)
    _dev("end", end, 1, (torch.int64,), n_words.device)


def count_symbols_device(symbols, counts=None, stream=None):
    """Byte counts of a device uint8 tensor (16-byte aligned) into a device
    uint64 tensor [256] (zeroed here unless given)."""
    import torch
    dev = _check_symbols("symbols", symbols)
    if counts is None:
        counts = torch.zeros(256, dtype=torch.int64, device=symbols.device)
    _dev("counts", counts, 256, (torch.int64,), dev)
    _check(lib().entq_count_symbols_device(_ptr(symbols) or None, symbols.numel(), _ptr(counts),
                                           _stream(stream)), "entq_count_symbols_device")
    return counts


def region_bytes(n_words: int) -> int:
    return int(lib().entq_region_bytes(int(n_words)))


def encode_device(symbols, chunk_symbols: int, freq: np.ndarray, scratch, n_words, stream=None):
    """Encode one tensor's device symbols into ``scratch`` (device uint8,
    entq_encode_device_scratch_bytes long); word counts to ``n_words``
    (device int32 [n_chunks], 0xFFFFFFFF marks a chunk with a frequency-0
    symbol)."""
    import torch
    dev = _check_symbols("symbols", symbols)
    k = _n_chunks(symbols.numel(), chunk_symbols)
    _dev("scratch", scratch, 0, _bytes_dtypes(), dev)
    _dev("n_words", n_words, k, (torch.int32,), dev)
    freq = np.ascontiguousarray(freq, dtype=np.uint16)
    if freq.size < 256:
        raise EntqError(EINVAL, f"freq holds {freq.size} entries, 256 needed")
    _check(lib().entq_encode_device(_ptr(symbols) or None, symbols.numel(), int(chunk_symbols),
                                    _ptr(freq), _ptr(scratch) or None,
                                    scratch.numel() if scratch is not None else 0,
                                    _ptr(n_words) or None, _stream(stream)), "entq_encode_device")


def pack_device(scratch, n: int, chunk_symbols: int, n_words, offsets, blob, stream=None):
    """Copies each chunk's states and words from ``scratch`` into its region
    of ``blob`` at ``offsets`` (device int64 [k], from region_offsets_device);
    blob must hold the regions up to the end that call reported."""
    _check_pack_job(scratch, n, chunk_symbols, n_words, offsets, blob)
    _check(lib().entq_pack_device(_ptr(scratch) or None, int(n), int(chunk_symbols),
                                  _ptr(n_words) or None, _ptr(offsets) or None,
                                  _ptr(blob) or None, _stream(stream)), "entq_pack_device")


def count_symbols_device_batch(jobs, stream=None):
    """jobs: list of (symbols, counts) device tensors (counts int64 [256],
    zeroed by the caller); one launch per 16 arrays."""
    import torch
    arr = np.zeros(len(jobs), COUNT_JOB)
    for i, (sym, counts) in enumerate(jobs):
        dev = _check_symbols(f"jobs[{i}] symbols", sym)
        _dev(f"jobs[{i}] counts", counts, 256, (torch.int64,), dev)
        arr[i] = (_ptr(sym), sym.numel(), _ptr(counts))
    _check(lib().entq_count_symbols_device_batch(_ptr(arr) if len(jobs) else None, len(jobs),
                                                 _stream(stream)),
           "entq_count_symbols_device_batch")


def pack_device_batch(jobs, blob, stream=None):
    """jobs: list of (scratch, n, chunk_symbols, n_words, offsets) as for
    pack_device; all write into blob; one launch per 16 tensors."""
    arr = np.zeros(len(jobs), PACK_JOB)
    for i, (scratch, n, C, nw, offs) in enumerate(jobs):
        _check_pack_job(scratch, n, C, nw, offs, blob, f"jobs[{i}] ")
        arr[i] = (_ptr(scratch), int(n), int(C), 0, _ptr(nw), _ptr(offs))
    _check(lib().entq_pack_device_batch(_ptr(arr) if len(jobs) else None, len(jobs),
                                        _ptr(blob), _stream(stream)), "entq_pack_device_batch")


def encode_device_batch(jobs, stream=None):
    """jobs: list of (symbols, chunk_symbols, freq, scratch, n_words) with
    device tensors (freq: device uint16/int16 [256]); one launch per 16
    tensors. A chunk of a tensor whose table is invalid or holds a
    frequency-0 symbol gets word count 0xFFFFFFFF."""
    arr = np.zeros(len(jobs), ENCODE_JOB)
    for i, (sym, C, freq, scratch, nw) in enumerate(jobs):
        _check_encode_job(sym, C, freq, scratch, nw, 256, f"jobs[{i}] ")
        arr[i] = (_ptr(sym), sym.numel(), int(C), 0, _ptr(freq), _ptr(scratch),
                  scratch.numel(), _ptr(nw))
    _check(lib().entq_encode_device_batch(_ptr(arr) if len(jobs) else None, len(jobs),
                                          _stream(stream)), "entq_encode_device_batch")


def region_offsets_device(n_words, offsets, end, base_offset: int = 0, stream=None):
    """Region byte offsets of consecutive chunks from their device word
    counts (int32 [k]) into ``offsets`` (device int64 [k]); ``end`` (device
    int64 [1]) gets base_offset + all their bytes."""
    _check_offsets_args(n_words, offsets, end)
    _check(lib().entq_region_offsets_device(_ptr(n_words) or None, n_words.numel(),
                                            int(base_offset), _ptr(offsets) or None, _ptr(end),
                                            _stream(stream)), "entq_region_offsets_device")


def count_chunks_device_batch(jobs, stream=None):
    """jobs: list of (symbols, chunk_symbols, counts) with device tensors;
    counts int32 [ceil(n / chunk_symbols), 256] receives each chunk's byte
    counts. One launch per 16 arrays."""
    import torch
    arr = np.zeros(len(jobs), CHUNK_COUNT_JOB)
    for i, (sym, C, counts) in enumerate(jobs):
        dev = _check_symbols(f"jobs[{i}] symbols", sym)
        _dev(f"jobs[{i}] counts", counts, 256 * _n_chunks(sym.numel(), C), (torch.int32,), dev)
        arr[i] = (_ptr(sym), sym.numel(), int(C), 0, _ptr(counts))
    _check(lib().entq_count_chunks_device_batch(_ptr(arr) if len(jobs) else None, len(jobs),
                                                _stream(stream)),
           "entq_count_chunks_device_batch")


def build_freq_chunks(counts: np.ndarray, n_threads: int | None = None) -> np.ndarray:
    """Host: the table of each row of 256 counts (uint32 [k, 256])."""
    counts = np.ascontiguousarray(counts, dtype=np.uint32).reshape(-1, 256)
    freq = np.zeros(counts.shape, np.uint16)
    _check(lib().entq_build_freq_chunks(_ptr(counts) if counts.size else None, counts.shape[0],
                                        _ptr(freq) if counts.size else None,
                                        n_threads or default_threads()),
           "entq_build_freq_chunks")
    return freq


def build_freq_device(counts, freq, stream=None):
    """Tables from counts on the device: counts int32 or int64 [k, 256]
    (device), freq int16/uint16 [k, 256] (device)."""
    import torch
    _dev("counts", counts, 0, (torch.int32, torch.int64))
    k = counts.numel() // 256
    _dev("freq", freq, k * 256, _freq_dtypes(), counts.device)
    _check(lib().entq_build_freq_device(_ptr(counts) or None, counts.element_size(), k,
                                        _ptr(freq) or None, _stream(stream)),
           "entq_build_freq_device")


def encode_device_adaptive_batch(jobs, stream=None):
    """encode_device_batch with per-chunk tables: jobs are (symbols,
    chunk_symbols, freq, scratch, n_words) with freq a device uint16/int16
    [n_chunks, 256]."""
    arr = np.zeros(len(jobs), ENCODE_JOB)
    for i, (sym, C, freq, scratch, nw) in enumerate(jobs):
        _check_encode_job(sym, C, freq, scratch, nw, 256 * _n_chunks(sym.numel(), C),
                          f"jobs[{i}] ")
        arr[i] = (_ptr(sym), sym.numel(), int(C), 0, _ptr(freq), _ptr(scratch),
                  scratch.numel(), _ptr(nw))
    _check(lib().entq_encode_device_adaptive_batch(_ptr(arr) if len(jobs) else None, len(jobs),
                                                   _stream(stream)),
           "entq_encode_device_adaptive_batch")


def region_offsets_device_adaptive(n_words, offsets, end, base_offset: int = 0, stream=None):
    """region_offsets_device for regions headed by their table."""
    _check_offsets_args(n_words, offsets, end)
    _check(lib().entq_region_offsets_device_adaptive(_ptr(n_words) or None, n_words.numel(),
                                                     int(base_offset), _ptr(offsets) or None,
                                                     _ptr(end), _stream(stream)),
           "entq_region_offsets_device_adaptive")


def pack_device_adaptive_batch(jobs, blob, stream=None):
    """pack_device_batch for regions headed by their table: jobs are
    (scratch, n, chunk_symbols, n_words, offsets, freq)."""
    import torch
    arr = np.zeros(len(jobs), PACK_ADAPTIVE_JOB)
    for i, (scratch, n, C, nw, offs, freq) in enumerate(jobs):
        _check_pack_job(scratch, n, C, nw, offs, blob, f"jobs[{i}] ")
        _dev(f"jobs[{i}] freq", freq, 256 * _n_chunks(n, C), _freq_dtypes(), blob.device)
        arr[i] = (_ptr(scratch), int(n), int(C), 0, _ptr(nw), _ptr(offs), _ptr(freq))
    _check(lib().entq_pack_device_adaptive_batch(_ptr(arr) if len(jobs) else None, len(jobs),
                                                 _ptr(blob), _stream(stream)),
           "entq_pack_device_adaptive_batch")


@dataclass
class DeviceBatch:
    """Like Batch, with the blob left in device memory (a torch uint8 view)."""
    blob: object                # torch uint8 on the device
    tensors: np.ndarray
    freq: np.ndarray
    chunks: np.ndarray

    @property
    def out_elems(self) -> int:
        t = self.tensors
        return int((t["out_elem_offset"] + t["n_symbols"]).max()) if t.size else 0


def _encode_meta(dev, k_all: int, n_freq: int):
    """One zeroed device buffer holding the encoder's per-chunk word counts
    (int32), region offsets (int64), the blob's end (int64) and n_freq
    frequency tables (int16 x 256), so that the host reads them back in one
    copy. Returns (buffer, nw, offs, end, freq, layout)."""
    import torch
    k = max(k_all, 1)

    def up(v):  # every part starts 256-byte aligned, like an allocation of its own
        return -(-v // 256) * 256
    o_offs = up(4 * k)
    o_end = up(o_offs + 8 * k)
    o_freq = up(o_end + 8)
    total = o_freq + 512 * max(n_freq, 1)
    meta = torch.zeros(total, dtype=torch.uint8, device=dev)
    nw = meta[:4 * k].view(torch.int32)
    offs = meta[o_offs:o_offs + 8 * k].view(torch.int64)
    end = meta[o_end:o_end + 8].view(torch.int64)
    freq = meta[o_freq:].view(torch.int16).view(max(n_freq, 1), 256)
    return meta, nw, offs, end, freq, (k, o_offs, o_end, o_freq)


def _read_meta(meta, layout, k_all: int, n_freq: int):
    """The host copy of an _encode_meta buffer: (nw u32, offs u64, end, freq u16)."""
    k, o_offs, o_end, o_freq = layout
    h = meta.cpu().numpy()
    nw = h[:4 * k].view(np.uint32)[:k_all]
    offs = h[o_offs:o_offs + 8 * k].view(np.uint64)[:k_all]
    end = int(h[o_end:o_end + 8].view(np.int64)[0])
    freq = h[o_freq:].view(np.uint16).reshape(max(n_freq, 1), 256)[:n_freq].copy()
    return nw, offs, end, freq


def encode_batch_device(specs, stream=None, events=None) -> DeviceBatch:
    """The device path of encode_batch: specs' ``symbols`` are device uint8
    tensors (contiguous, 16-byte aligned). Counts, frequency tables,
    encoding, the region layout and packing run on the GPU, each step over
    all tensors; the host reads the word counts, offsets and tables once at
    the end (for the chunk index). With
    ``events`` (a list), each kernel launch appends (name, start, end) HIP
    events recorded on the stream around it."""
    import torch
    dev = specs[0]["symbols"].device if specs else torch.device("cuda")
    s = torch.cuda.current_stream(dev) if stream is None else stream
    T = len(specs)
    shapes = []
    for sp in specs:
        sym = sp["symbols"]
        rows, cols, C = int(sp["rows"]), int(sp["cols"]), int(sp["chunk_symbols"])
        n = sym.numel()
        assert n == rows * cols and sym.dtype == torch.uint8 and sym.is_contiguous()
        shapes.append((rows, cols, C, n, -(-n // C)))
    k_all = sum(sh[4] for sh in shapes)
    bound = sum(int(lib().entq_encode_bound(sh[3], sh[2])) for sh in shapes)
    scr = [int(lib().entq_encode_device_scratch_bytes(sh[3], sh[2])) for sh in shapes]
    scr_off = np.concatenate([[0], np.cumsum(scr)]).astype(np.int64)
    blob = torch.empty(max(bound, 16), dtype=torch.uint8, device=dev)
    scratch = torch.empty(max(int(scr_off[-1]), 16), dtype=torch.uint8, device=dev)
    counts = torch.zeros((max(T, 1), 256), dtype=torch.int64, device=dev)
    meta, nw_d, offs_d, end_d, freq_d, layout = _encode_meta(dev, k_all, T)

    def timed(name, fn):
        if events is None:
            return fn()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(s)
        fn()
        b.record(s)
        events.append((name, a, b))

    with torch.cuda.stream(s):
        cjobs = [(sp["symbols"], counts[t]) for t, sp in enumerate(specs) if shapes[t][3]]
        if cjobs:
            timed("count", lambda: count_symbols_device_batch(cjobs, s))
        if T:
            timed("tables", lambda: build_freq_device(counts, freq_d, s))
        jobs, k0 = [], 0
        for t, sp in enumerate(specs):
            rows, cols, C, n, k = shapes[t]
            if k:
                jobs.append((sp["symbols"], C, freq_d[t], scratch[scr_off[t]:scr_off[t + 1]],
                             nw_d[k0:k0 + k]))
            k0 += k
        if jobs:
            timed("encode", lambda: encode_device_batch(jobs, s))
        if k_all:
            timed("offsets", lambda: region_offsets_device(nw_d[:k_all], offs_d[:k_all], end_d,
                                                           0, s))
        pjobs, k0 = [], 0
        for t, sp in enumerate(specs):
            rows, cols, C, n, k = shapes[t]
            if k:
                pjobs.append((scratch[scr_off[t]:scr_off[t + 1]], n, C, nw_d[k0:k0 + k],
                              offs_d[k0:k0 + k]))
            k0 += k
        if pjobs:
            timed("pack", lambda: pack_device_batch(pjobs, blob, s))
        s.synchronize()
        nw, offs, end, freqs = _read_meta(meta, layout, k_all, T)
    for t in range(T):
        if shapes[t][3] == 0:
            freqs[t, 0] = PROB_SCALE  # an empty tensor: any valid table
    if (nw == 0xFFFFFFFF).any():
        raise EntqError(-2, "entq_encode_device: a symbol has frequency 0")
    tens = np.zeros(T, TENSOR_DESC)
    chunks = np.zeros(k_all, CHUNK_DESC)
    k0 = out_off = scale_off = 0
    for t, sp in enumerate(specs):
        rows, cols, C, n, k = shapes[t]
        ch = chunks[k0:k0 + k]
        ch["tensor"] = t
        ch["n_symbols"] = np.minimum(C, n - np.arange(k, dtype=np.int64) * C)
        ch["n_words"] = nw[k0:k0 + k]
        ch["byte_offset"] = offs[k0:k0 + k]
        ch["elem_offset"] = np.arange(k, dtype=np.uint64) * C
        tens[t] = (int(sp["kind"]), rows, cols, C, n, out_off, scale_off)
        out_off += n
        scale_off += rows
        k0 += k
    return DeviceBatch(blob[:end], tens, freqs, chunks)


def encode_batch_device_adaptive(specs, stream=None, events=None) -> DeviceBatch:
    """encode_batch_device with per-chunk tables (the container of
    encode_batch_adaptive, built on the GPU): per-chunk byte counts, their
    tables (entq_build_freq_device), encoding, the region layout and packing,
    each step over all tensors, with no host round trip before the final
    read of the chunk index. The DeviceBatch's freq is None (pass it to
    plan() as such)."""
    import torch
    dev = specs[0]["symbols"].device if specs else torch.device("cuda")
    s = torch.cuda.current_stream(dev) if stream is None else stream
    T = len(specs)
    shapes = []
    for sp in specs:
        sym = sp["symbols"]
        rows, cols, C = int(sp["rows"]), int(sp["cols"]), int(sp["chunk_symbols"])
        n = sym.numel()
        assert n == rows * cols and sym.dtype == torch.uint8 and sym.is_contiguous()
        shapes.append((rows, cols, C, n, -(-n // C)))
    k_all = sum(sh[4] for sh in shapes)
    k0s = np.concatenate([[0], np.cumsum([sh[4] for sh in shapes])]).astype(np.int64)
    bound = sum(int(lib().entq_encode_bound_adaptive(sh[3], sh[2])) for sh in shapes)
    scr = [int(lib().entq_encode_device_scratch_bytes(sh[3], sh[2])) for sh in shapes]
    scr_off = np.concatenate([[0], np.cumsum(scr)]).astype(np.int64)
    blob = torch.empty(max(bound, 16), dtype=torch.uint8, device=dev)
    scratch = torch.empty(max(int(scr_off[-1]), 16), dtype=torch.uint8, device=dev)
    counts = torch.zeros((max(k_all, 1), 256), dtype=torch.int32, device=dev)
    meta, nw_d, offs_d, end_d, _, layout = _encode_meta(dev, k_all, 0)

    def timed(name, fn):
        if events is None:
            return fn()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(s)
        fn()
        b.record(s)
        events.append((name, a, b))

    live = [t for t in range(T) if shapes[t][4]]
    with torch.cuda.stream(s):
        cjobs = [(specs[t]["symbols"], shapes[t][2], counts[k0s[t]:k0s[t + 1]]) for t in live]
        if cjobs:
            timed("count", lambda: count_chunks_device_batch(cjobs, s))
        freq_d = torch.zeros((max(k_all, 1), 256), dtype=torch.int16, device=dev)
        if k_all:
            timed("tables", lambda: build_freq_device(counts[:k_all], freq_d, s))
        jobs = [(specs[t]["symbols"], shapes[t][2], freq_d[k0s[t]:k0s[t + 1]],
                 scratch[scr_off[t]:scr_off[t + 1]], nw_d[k0s[t]:k0s[t + 1]]) for t in live]
        if jobs:
            timed("encode", lambda: encode_device_adaptive_batch(jobs, s))
        if k_all:
            timed("offsets", lambda: region_offsets_device_adaptive(
                nw_d[:k_all], offs_d[:k_all], end_d, 0, s))
        pjobs = [(scratch[scr_off[t]:scr_off[t + 1]], shapes[t][3], shapes[t][2],
                  nw_d[k0s[t]:k0s[t + 1]], offs_d[k0s[t]:k0s[t + 1]], freq_d[k0s[t]:k0s[t + 1]])
                 for t in live]
        if pjobs:
            timed("pack", lambda: pack_device_adaptive_batch(pjobs, blob, s))
        s.synchronize()
        nw, offs, end, _ = _read_meta(meta, layout, k_all, 0)
    if (nw == 0xFFFFFFFF).any():
        raise EntqError(-2, "entq_encode_device_adaptive_batch: a chunk could not be coded")
    tens = np.zeros(T, TENSOR_DESC)
    chunks = np.zeros(k_all, CHUNK_DESC)
    out_off = scale_off = 0
    for t, sp in enumerate(specs):
        rows, cols, C, n, k = shapes[t]
        ch = chunks[k0s[t]:k0s[t + 1]]
        ch["tensor"] = t
        ch["n_symbols"] = np.minimum(C, n - np.arange(k, dtype=np.int64) * C)
        ch["n_words"] = nw[k0s[t]:k0s[t + 1]]
        ch["byte_offset"] = offs[k0s[t]:k0s[t + 1]]
        ch["elem_offset"] = np.arange(k, dtype=np.uint64) * C
        tens[t] = (int(sp["kind"]), rows, cols, C, n, out_off, scale_off)
        out_off += n
        scale_off += rows
    return DeviceBatch(blob[:end], tens, None, chunks)
