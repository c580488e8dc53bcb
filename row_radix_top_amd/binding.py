"""ctypes binding of ``libtopk_ragged.so``: the same entry points as
``include/topk_ragged.h``, with torch tensors used only as device memory and
streams.  Argument marshalling only; every step of the op runs in the HIP
kernels.  If the library is missing the calls raise -- there is no fallback.
"""

from __future__ import annotations

import ctypes
import os
import threading

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "lib", "libtopk_ragged.so")

TOPK_OK = 0
STATUS_NAMES = {0: "TOPK_OK", -1: "TOPK_EINVAL", -2: "TOPK_EUNSUPPORTED_K", -3: "TOPK_EWORKSPACE",
                -4: "TOPK_EDEVICE", -5: "TOPK_ELAUNCH"}
PATH_NONE, PATH_SINGLE, PATH_MULTI = 0, 1, 2
MAX_K = 4096
RADIX_THRESHOLD = 32768

# Every symbol include/topk_ragged.h declares.
EXPORTED = (
    "topk_ragged", "topk_ragged_workspace_size", "topk_ragged_workspace_init",
    "topk_ragged_last_error", "topk_ragged_plan", "topk_ragged_query_plan",
    "topk_ragged_workspace_size_ex", "topk_ragged_ex", "topk_ragged_workspace_status",
    "topk_ragged_debug_keys", "topk_ragged_version", "topk_ragged_read_reference",
    "topk_ragged_offsets", "topk_ragged_offsets_ex", "topk_ragged_values", "topk_ragged_values_ex",
    "topk_ragged_strided", "topk_ragged_strided_workspace_size", "topk_ragged_bf16", "topk_ragged_bf16_ex",
    "topk_ragged_noalloc",
)
NOALLOC_SCRATCH_BYTES = 8 << 20


class DeviceProps(ctypes.Structure):
    _fields_ = [("num_cus", ctypes.c_int32), ("occupancy_single", ctypes.c_int32),
                ("occupancy_multi", ctypes.c_int32), ("max_lds_per_block", ctypes.c_int32),
                ("occupancy_single16", ctypes.c_int32), ("occupancy_multi16", ctypes.c_int32),
                ("occupancy_w512", ctypes.c_int32 * 4), ("occupancy_w1024", ctypes.c_int32 * 4)]


class Plan(ctypes.Structure):
    _fields_ = [("path", ctypes.c_int32), ("kmax", ctypes.c_int32), ("vec", ctypes.c_int32),
                ("block", ctypes.c_int32), ("grid", ctypes.c_int32), ("wg_per_row", ctypes.c_int32),
                ("chunk", ctypes.c_int64), ("resident_cap", ctypes.c_int32),
                ("headroom", ctypes.c_int32), ("lds_bytes", ctypes.c_int32),
                ("fell_back", ctypes.c_int32), ("idx16", ctypes.c_int32),
                ("workspace_bytes", ctypes.c_uint64)]

    def as_dict(self) -> dict:
        return {name: getattr(self, name) for name, _ in self._fields_}


class Overrides(ctypes.Structure):
    _fields_ = [("force_path", ctypes.c_int32), ("force_wg_per_row", ctypes.c_int32),
                ("max_grid", ctypes.c_int32), ("force_vec", ctypes.c_int32),
                ("force_chunk", ctypes.c_int64), ("spin_limit", ctypes.c_uint32),
                ("min_chunk", ctypes.c_int32), ("max_occupancy", ctypes.c_int32),
                ("force_idx32", ctypes.c_int32), ("force_block", ctypes.c_int32),
                ("force_wait_timeout", ctypes.c_int32)]

    @classmethod
    def make(cls, **kw) -> "Overrides | None":
        if not kw:
            return None
        o = cls()
        for k, v in kw.items():
            if v is None:
                continue
            if not hasattr(o, k):
                raise TypeError(f"unknown override {k!r}")
            setattr(o, k, int(v))
        return o


class TopKError(RuntimeError):
    def __init__(self, code: int, where: str, detail: str):
        self.code = code
        super().__init__(f"{where}: {STATUS_NAMES.get(code, code)}: {detail}")


_lib = None
_lock = threading.Lock()


def load() -> ctypes.CDLL:
    """Load the built HIP library; raise if it has not been built."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"HIP library not built: {LIB_PATH} is missing. Build it with "
                "`python -m row_radix_top_amd.build` (or __graft_entry__.build()).")
        lib = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        lib.topk_ragged.argtypes = [vp, i64, vp, i32, i32, i32, vp, vp, vp]
        lib.topk_ragged_ex.argtypes = [vp, i64, vp, i32, i32, i32, vp, vp, vp, ctypes.POINTER(Overrides)]
        lib.topk_ragged_noalloc.argtypes = [vp, i64, vp, i32, i32, i32, vp, vp]
        lib.topk_ragged_workspace_size.argtypes = [i32, i64, i32, vp, ctypes.POINTER(sz)]
        lib.topk_ragged_workspace_size_ex.argtypes = [vp, i32, i64, i32, ctypes.POINTER(Overrides), vp,
                                                      ctypes.POINTER(sz)]
        lib.topk_ragged_workspace_init.argtypes = [vp, sz, vp]
        lib.topk_ragged_last_error.restype = ctypes.c_char_p
        lib.topk_ragged_last_error.argtypes = []
        lib.topk_ragged_plan.argtypes = [ctypes.POINTER(DeviceProps), i32, i64, i32, i32,
                                         ctypes.POINTER(Overrides), ctypes.POINTER(Plan)]
        lib.topk_ragged_query_plan.argtypes = [vp, i32, i64, i32, ctypes.POINTER(Overrides), vp,
                                               ctypes.POINTER(Plan)]
        lib.topk_ragged_workspace_status.argtypes = [vp, vp, ctypes.POINTER(ctypes.c_uint32)]
        lib.topk_ragged_debug_keys.argtypes = [vp, vp, i64, vp]
        lib.topk_ragged_version.argtypes = []
        lib.topk_ragged_read_reference.argtypes = [vp, i64, vp, i32, vp, vp]
        lib.topk_ragged_offsets.argtypes = [vp, i64, vp, vp, i32, i32, i32, vp, vp, vp]
        lib.topk_ragged_offsets_ex.argtypes = [vp, i64, vp, vp, i32, i32, i32, vp, vp, vp,
                                               ctypes.POINTER(Overrides)]
        lib.topk_ragged_values.argtypes = [vp, i64, vp, vp, i32, i32, i32, vp, vp, vp, vp]
        lib.topk_ragged_strided.argtypes = [vp, i64, i64, i64, vp, vp, i32, i32, i32, vp, vp, vp, vp]
        lib.topk_ragged_bf16.argtypes = [vp, i64, vp, vp, i32, i32, i32, vp, vp, vp, vp]
        lib.topk_ragged_bf16_ex.argtypes = [vp, i64, vp, vp, i32, i32, i32, vp, vp, vp, vp,
                                            ctypes.POINTER(Overrides)]
        lib.topk_ragged_strided_workspace_size.argtypes = [i32, i64, i32, vp, ctypes.POINTER(sz)]
        lib.topk_ragged_values_ex.argtypes = [vp, i64, vp, vp, i32, i32, i32, vp, vp, vp, vp,
                                              ctypes.POINTER(Overrides)]
        for name in EXPORTED:
            getattr(lib, name).restype = ctypes.c_int if name != "topk_ragged_last_error" else ctypes.c_char_p
        _lib = lib
        return lib


def last_error() -> str:
    return load().topk_ragged_last_error().decode()


def _check(rc: int, where: str) -> None:
    if rc != TOPK_OK:
        raise TopKError(rc, where, last_error())


def _ov_ptr(ov: Overrides | None):
    return ctypes.byref(ov) if ov is not None else None


# ---------------------------------------------------------------------------
# Host-only planning (no GPU needed)
# ---------------------------------------------------------------------------

def plan_for_props(num_cus: int, occupancy_single: int, occupancy_multi: int, num_rows: int,
                   row_stride: int, K: int, vec_allowed: int = 4, max_lds_per_block: int = 163840,
                   occupancy_single16: int | None = None, occupancy_multi16: int | None = None,
                   occupancy_w512=(0, 0, 0, 0), occupancy_w1024=(0, 0, 0, 0), **overrides) -> dict:
    """The pure planner on made-up device facts.  occupancy_w512 and
    occupancy_w1024 are (single, multi, single16, multi16) of the wider
    instances; zeros mean there are none."""
    props = DeviceProps(num_cus, occupancy_single, occupancy_multi, max_lds_per_block,
                        occupancy_single if occupancy_single16 is None else occupancy_single16,
                        occupancy_multi if occupancy_multi16 is None else occupancy_multi16,
                        (ctypes.c_int32 * 4)(*occupancy_w512), (ctypes.c_int32 * 4)(*occupancy_w1024))
    plan = Plan()
    ov = Overrides.make(**overrides)
    rc = load().topk_ragged_plan(ctypes.byref(props), num_rows, row_stride, K, vec_allowed,
                                 _ov_ptr(ov), ctypes.byref(plan))
    _check(rc, "topk_ragged_plan")
    return plan.as_dict()


# ---------------------------------------------------------------------------
# Device calls (torch tensors as memory, torch streams as streams)
# ---------------------------------------------------------------------------

def _stream_ptr(stream, device=None) -> int:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return int(stream.cuda_stream)


def query_plan(scores, K: int, stream=None, **overrides) -> dict:
    plan = Plan()
    ov = Overrides.make(**overrides)
    rc = load().topk_ragged_query_plan(scores.data_ptr(), scores.shape[0], scores.stride(0), K,
                                       _ov_ptr(ov), _stream_ptr(stream, scores.device),
                                       ctypes.byref(plan))
    _check(rc, "topk_ragged_query_plan")
    return plan.as_dict()


def workspace_size(num_rows: int, row_stride: int, K: int, stream=None, scores=None, device=None,
                   **overrides) -> int:
    out = ctypes.c_size_t(0)
    lib = load()
    sp = _stream_ptr(stream, device if scores is None else scores.device)
    if overrides or scores is not None:
        ptr = scores.data_ptr() if scores is not None else 256
        ov = Overrides.make(**overrides)
        rc = lib.topk_ragged_workspace_size_ex(ptr, num_rows, row_stride, K, _ov_ptr(ov), sp,
                                               ctypes.byref(out))
    else:
        rc = lib.topk_ragged_workspace_size(num_rows, row_stride, K, sp, ctypes.byref(out))
    _check(rc, "topk_ragged_workspace_size")
    return int(out.value)


def workspace_init(ws, stream=None) -> None:
    if ws is None or ws.numel() == 0:
        return
    rc = load().topk_ragged_workspace_init(ws.data_ptr(), ws.numel() * ws.element_size(),
                                           _stream_ptr(stream, ws.device))
    _check(rc, "topk_ragged_workspace_init")


def new_workspace(nbytes: int, device, stream=None):
    """Allocate (torch) and zero (library kernel) a workspace of nbytes."""
    import torch
    if nbytes == 0:
        return None
    ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
    workspace_init(ws, stream)
    return ws


def workspace_status(ws, stream=None) -> int:
    flags = ctypes.c_uint32(0)
    ptr = ws.data_ptr() if ws is not None else None
    dev = ws.device if ws is not None else None
    rc = load().topk_ragged_workspace_status(ptr, _stream_ptr(stream, dev), ctypes.byref(flags))
    _check(rc, "topk_ragged_workspace_status")
    return int(flags.value)


def _validate(scores, lengths, out, K):
    import torch
    if not scores.is_cuda or scores.dtype != torch.float32 or scores.dim() != 2:
        raise TypeError("scores must be a 2-D float32 CUDA tensor")
    if scores.stride(1) != 1:
        raise ValueError("scores must have unit column stride")
    if not lengths.is_cuda or lengths.dtype != torch.int32 or not lengths.is_contiguous():
        raise TypeError("lengths must be a contiguous int32 CUDA tensor")
    if lengths.numel() != scores.shape[0]:
        raise ValueError("lengths must hold one entry per row")
    if out is not None:
        if (not out.is_cuda or out.dtype != torch.int32 or not out.is_contiguous()
                or tuple(out.shape) != (scores.shape[0], K)):
            raise ValueError("out must be a contiguous int32 CUDA tensor of shape [num_rows, K]")


def strided_workspace_size(num_rows: int, num_cols: int, K: int, device=None) -> int:
    """Workspace bytes for topk_ragged_strided on (num_rows, num_cols, K)."""
    n = ctypes.c_size_t(0)
    rc = load().topk_ragged_strided_workspace_size(num_rows, num_cols, K, _stream_ptr(None, device),
                                                   ctypes.byref(n))
    _check(rc, "topk_ragged_strided_workspace_size")
    return int(n.value)


def topk_ragged_strided(scores, lengths, K: int, *, workspace, out=None, out_values=None, row_offsets=None,
                        next_n: int | None = None, stream=None):
    """topk_ragged for a float32 CUDA view with any strides ([num_rows,
    num_cols], e.g. a transpose): each row's valid prefix is packed into the
    workspace first.  Returns the indices, or (indices, values) when
    out_values is given (a float32 [num_rows, K] tensor)."""
    import torch
    if scores.dtype != torch.float32 or not scores.is_cuda or scores.dim() != 2:
        raise ValueError("scores must be a 2-D float32 CUDA tensor")
    if lengths.dtype != torch.int32 or not lengths.is_cuda or not lengths.is_contiguous():
        raise ValueError("lengths must be a contiguous int32 CUDA tensor")
    if next_n is None:
        next_n = int(lengths.shape[1]) if lengths.dim() == 2 else 1
    num_rows, num_cols = scores.shape
    if lengths.numel() != num_rows:
        raise ValueError("one length per row")
    if out is None:
        out = torch.empty((num_rows, K), dtype=torch.int32, device=scores.device)
    ro = None if row_offsets is None else row_offsets.data_ptr()
    vp_ = None if out_values is None else out_values.data_ptr()
    rc = load().topk_ragged_strided(scores.data_ptr(), scores.stride(0), scores.stride(1), num_cols,
                                    lengths.data_ptr(), ro, num_rows, next_n, K, out.data_ptr(), vp_,
                                    workspace.data_ptr() if workspace is not None else None,
                                    _stream_ptr(stream, scores.device))
    _check(rc, "topk_ragged_strided")
    return out if out_values is None else (out, out_values)


def topk_ragged_bf16(scores, lengths, K: int, *, out=None, out_values=None, workspace=None,
                     next_n: int | None = None, stream=None, row_offsets=None, **overrides):
    """topk_ragged over bf16 scores (a torch.bfloat16 CUDA tensor with unit
    column stride).  Returns the indices, or (indices, values) when
    out_values (float32 [num_rows, K]) is given."""
    import torch
    if scores.dtype != torch.bfloat16 or not scores.is_cuda or scores.dim() != 2 or scores.stride(1) != 1:
        raise ValueError("scores must be a 2-D bfloat16 CUDA tensor with unit column stride")
    if lengths.dtype != torch.int32 or not lengths.is_cuda or not lengths.is_contiguous():
        raise ValueError("lengths must be a contiguous int32 CUDA tensor")
    if next_n is None:
        next_n = int(lengths.shape[1]) if lengths.dim() == 2 else 1
    num_rows = scores.shape[0]
    if out is None:
        out = torch.empty((num_rows, K), dtype=torch.int32, device=scores.device)
    ro = None if row_offsets is None else row_offsets.data_ptr()
    vp_ = None if out_values is None else out_values.data_ptr()
    ov = Overrides.make(**overrides)
    args = (scores.data_ptr(), scores.stride(0), lengths.data_ptr(), ro, num_rows, next_n, K, out.data_ptr(), vp_,
            workspace.data_ptr() if workspace is not None else None, _stream_ptr(stream, scores.device))
    lib = load()
    rc = lib.topk_ragged_bf16(*args) if ov is None else lib.topk_ragged_bf16_ex(*args, ctypes.byref(ov))
    _check(rc, "topk_ragged_bf16")
    return out if out_values is None else (out, out_values)


def topk_ragged_values(scores, lengths, K: int, *, out=None, out_values=None, workspace=None,
                       next_n: int | None = None, stream=None, row_offsets=None, **overrides):
    """topk_ragged plus the chosen scores: returns (indices, values), values
    float32 [num_rows, K] with the exact score bits and -inf in the padding."""
    import torch
    if next_n is None:
        next_n = int(lengths.shape[1]) if lengths.dim() == 2 else 1
    _validate(scores, lengths, out, K)
    num_rows = scores.shape[0]
    if out is None:
        out = torch.empty((num_rows, K), dtype=torch.int32, device=scores.device)
    if out_values is None:
        out_values = torch.empty((num_rows, K), dtype=torch.float32, device=scores.device)
    if (out_values.dtype != torch.float32 or not out_values.is_cuda or not out_values.is_contiguous()
            or tuple(out_values.shape) != (num_rows, K)):
        raise ValueError("out_values must be a contiguous float32 CUDA tensor of shape [num_rows, K]")
    ro = None
    if row_offsets is not None:
        if (row_offsets.dtype != torch.int32 or not row_offsets.is_cuda or row_offsets.numel() != num_rows
                or not row_offsets.is_contiguous()):
            raise ValueError("row_offsets must be a contiguous int32 CUDA tensor with one entry per row")
        ro = row_offsets.data_ptr()
    ov = Overrides.make(**overrides)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    lib = load()
    args = (scores.data_ptr(), scores.stride(0), lengths.data_ptr(), ro, num_rows, next_n, K, out.data_ptr(),
            out_values.data_ptr(), ws_ptr, _stream_ptr(stream, scores.device))
    if ov is None:
        rc = lib.topk_ragged_values(*args)
    else:
        rc = lib.topk_ragged_values_ex(*args, ctypes.byref(ov))
    _check(rc, "topk_ragged_values")
    return out, out_values


def topk_ragged(scores, lengths, K: int, *, out=None, workspace=None, next_n: int | None = None,
                stream=None, row_offsets=None, **overrides):
    """Indices of the K largest of the first lengths[r] scores of each row.

    scores: float32 CUDA [num_rows, row_stride-or-wider view] with unit column
    stride; lengths: int32 CUDA [num_rows] or [batch, next_n] (next_n is then
    taken from its second dimension); returns int32 [num_rows, K], ascending
    per row, -1 padded.  workspace: a tensor from new_workspace() sized by
    workspace_size(), needed only when that size is nonzero.  row_offsets:
    int32 CUDA [num_rows]; if given, row r's chosen indices are reported as
    row_offsets[r] + index (topk_ragged_offsets).
    """
    import torch
    if next_n is None:
        next_n = int(lengths.shape[1]) if lengths.dim() == 2 else 1
    _validate(scores, lengths, out, K)
    num_rows = scores.shape[0]
    if out is None:
        out = torch.empty((num_rows, K), dtype=torch.int32, device=scores.device)
    ov = Overrides.make(**overrides)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    lib = load()
    sp = _stream_ptr(stream, scores.device)
    if row_offsets is not None:
        if (row_offsets.dtype != torch.int32 or not row_offsets.is_cuda or row_offsets.numel() != num_rows
                or not row_offsets.is_contiguous()):
            raise ValueError("row_offsets must be a contiguous int32 CUDA tensor with one entry per row")
        args = (scores.data_ptr(), scores.stride(0), lengths.data_ptr(), row_offsets.data_ptr(), num_rows,
                next_n, K, out.data_ptr(), ws_ptr, sp)
        if ov is None:
            rc = lib.topk_ragged_offsets(*args)
        else:
            rc = lib.topk_ragged_offsets_ex(*args, ctypes.byref(ov))
        _check(rc, "topk_ragged_offsets")
        return out
    if ov is None:
        rc = lib.topk_ragged(scores.data_ptr(), scores.stride(0), lengths.data_ptr(), num_rows, next_n,
                             K, out.data_ptr(), ws_ptr, sp)
    else:
        rc = lib.topk_ragged_ex(scores.data_ptr(), scores.stride(0), lengths.data_ptr(), num_rows,
                                next_n, K, out.data_ptr(), ws_ptr, sp, ctypes.byref(ov))
    _check(rc, "topk_ragged")
    return out


def topk_ragged_noalloc(scores, lengths, K: int, *, out=None, next_n: int | None = None, stream=None):
    """topk_ragged without a workspace argument: a launch that needs one
    uses the library's static per-device scratch array (at most
    NOALLOC_SCRATCH_BYTES).  Calls on one GPU share that array, so calls
    that may overlap must be serialised by the caller."""
    import torch
    if next_n is None:
        next_n = int(lengths.shape[1]) if lengths.dim() == 2 else 1
    _validate(scores, lengths, out, K)
    num_rows = scores.shape[0]
    if out is None:
        out = torch.empty((num_rows, K), dtype=torch.int32, device=scores.device)
    rc = load().topk_ragged_noalloc(scores.data_ptr(), scores.stride(0), lengths.data_ptr(), num_rows, next_n, K,
                                    out.data_ptr(), _stream_ptr(stream, scores.device))
    _check(rc, "topk_ragged_noalloc")
    return out


def debug_keys(bits):
    """Device key transform of an int32/uint32-valued CUDA tensor of fp32 bit patterns."""
    import torch
    bits = bits.contiguous()
    keys = torch.empty_like(bits)
    rc = load().topk_ragged_debug_keys(bits.data_ptr(), keys.data_ptr(), bits.numel(),
                                       _stream_ptr(None, bits.device))
    _check(rc, "topk_ragged_debug_keys")
    return keys


def read_reference(scores, lengths, *, out=None, stream=None):
    """Streaming-read reference: the device key of each row's largest valid
    score, read exactly as topk_ragged reads the row (measurement only)."""
    import torch
    _validate(scores, lengths, None, 1)
    num_rows = scores.shape[0]
    if out is None:
        out = torch.empty(num_rows, dtype=torch.int32, device=scores.device)
    rc = load().topk_ragged_read_reference(scores.data_ptr(), scores.stride(0), lengths.data_ptr(), num_rows,
                                           out.data_ptr(), _stream_ptr(stream, scores.device))
    _check(rc, "topk_ragged_read_reference")
    return out


def version() -> int:
    return int(load().topk_ragged_version())
