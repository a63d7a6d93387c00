"""ctypes binding of the topkf C ABI (include/topkf.h).

Argument marshalling only: every step of the selection runs in the HIP
library `libtopkf.so` built from `csrc/topkf.hip`.  torch supplies device
memory and streams.  Importing this module raises if the library has not been
built (see `exact_row_wise_sampled_amd.build`); there is no fallback.

API after the HPC-Ops pull request "feat(topk): add sample-verified exact
Top-K", section "API":

    counter_bytes, workspace_bytes = topk_filtered_workspace_size(num_rows, max_kv_len)
    counters = torch.zeros(counter_bytes, dtype=torch.uint8, device="cuda")
    workspace = torch.empty(workspace_bytes, dtype=torch.uint8, device="cuda")
    topk_filtered(logits, ke, output, num_valid_rows, top_k, counters, workspace)
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtopkf.so")

if not os.path.exists(LIB_PATH):
    raise ImportError("topkf HIP library not built: %s is missing "
                      "(run exact_row_wise_sampled_amd.build.build())" % LIB_PATH)

# torch first: the library then binds to the HIP runtime torch has loaded, so
# both share one runtime instance whatever the caller imported first.
import torch  # noqa: E402,F401

_lib = ctypes.CDLL(LIB_PATH)

K_MAX = 2048
NOALLOC_SCRATCH_BYTES = 256 << 20  # the device array of topk_filtered_noalloc

FAMILY_AUTO = 0
FAMILY_PERSISTENT = 1
FAMILY_KVSPLIT = 2

ROUTE_NAMES = ["sentinel", "primary", "band", "exact_underfill", "exact_direct", "spill",
               "hinted", "reserved7"]
ROUTE_COUNT = 8

STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported shape",
          3: "counter or workspace buffer too small", 4: "HIP runtime error"}


class Plan(ctypes.Structure):
    _fields_ = [("family", ctypes.c_int32), ("stride", ctypes.c_int32), ("dual", ctypes.c_int32),
                ("splits", ctypes.c_int32), ("workers", ctypes.c_int32),
                ("min_segment", ctypes.c_int32), ("band_quarters", ctypes.c_int32),
                ("primary_quarters", ctypes.c_int32)]

    def as_dict(self):
        return {f: getattr(self, f) for f, _ in self._fields_}

    def __repr__(self):
        return "Plan(%s)" % ", ".join("%s=%d" % kv for kv in self.as_dict().items())


_c = ctypes
_i64, _i32, _vp, _sz = _c.c_int64, _c.c_int32, _c.c_void_p, _c.c_size_t

_lib.topk_filtered_workspace_size.restype = _i32
_lib.topk_filtered_workspace_size.argtypes = [_i64, _i64, _c.POINTER(_sz), _c.POINTER(_sz)]
_lib.topk_filtered.restype = _i32
_lib.topk_filtered.argtypes = [_vp, _i64, _i64, _i64, _vp, _vp, _vp, _i32, _vp, _sz, _vp, _sz, _vp]
_lib.topk_filtered_debug.restype = _i32
_lib.topk_filtered_debug.argtypes = [_vp, _i64, _i64, _i64, _vp, _vp, _vp, _i32, _vp, _sz, _vp,
                                     _sz, _c.POINTER(Plan), _vp, _vp]
_lib.topk_filtered_hinted.restype = _i32
_lib.topk_filtered_hinted.argtypes = [_vp, _i64, _i64, _i64, _vp, _vp, _vp, _i32, _vp, _vp, _sz,
                                      _vp, _sz, _vp]
_lib.topk_filtered_hinted_debug.restype = _i32
_lib.topk_filtered_hinted_debug.argtypes = [_vp, _i64, _i64, _i64, _vp, _vp, _vp, _i32, _vp, _vp,
                                            _sz, _vp, _sz, _c.POINTER(Plan), _vp, _vp]
_lib.topk_filtered_noalloc.restype = _i32
_lib.topk_filtered_noalloc.argtypes = [_vp, _i64, _i64, _i64, _vp, _vp, _vp, _i32, _vp]
_lib.topkf_status_string.restype = _c.c_char_p
_lib.topkf_status_string.argtypes = [_i32]
_lib.topkf_plan_for.restype = _i32
_lib.topkf_plan_for.argtypes = [_i64, _i64, _i32, _c.POINTER(Plan)]
_lib.topkf_plan_workspace_size.restype = _i32
_lib.topkf_plan_workspace_size.argtypes = [_c.POINTER(Plan), _i64, _i64, _c.POINTER(_sz),
                                           _c.POINTER(_sz)]
_lib.topkf_coarse_keys.restype = _i32
_lib.topkf_coarse_keys.argtypes = [_vp, _i64, _vp, _vp]
_lib.topkf_coarse_cutoffs.restype = _i32
_lib.topkf_coarse_cutoffs.argtypes = [_vp, _vp, _vp]
_lib.topkf_read_probe.restype = _i32
_lib.topkf_read_probe.argtypes = [_vp, _i64, _vp, _vp]


class TopkfError(RuntimeError):
    def __init__(self, code: int, where: str):
        super().__init__("%s failed: %s (status %d)" % (where, status_string(code), code))
        self.code = code


def status_string(code: int) -> str:
    return _lib.topkf_status_string(int(code)).decode()


def _check(code: int, where: str) -> None:
    if code != 0:
        raise TopkfError(code, where)


def topk_filtered_workspace_size(num_rows: int, max_kv_len: int) -> tuple[int, int]:
    cb, wb = _sz(0), _sz(0)
    _check(_lib.topk_filtered_workspace_size(int(num_rows), int(max_kv_len), _c.byref(cb),
                                             _c.byref(wb)), "topk_filtered_workspace_size")
    return cb.value, wb.value


def plan_for(num_rows: int, max_kv_len: int, cu_count: int) -> Plan:
    p = Plan()
    _check(_lib.topkf_plan_for(int(num_rows), int(max_kv_len), int(cu_count), _c.byref(p)),
           "topkf_plan_for")
    return p


def make_plan(family: int, stride: int, dual: int = 1, splits: int = 1, workers: int = 1,
              min_segment: int = 8192, band_quarters: int = 7,
              primary_quarters: int = 6) -> Plan:
    return Plan(family, stride, dual, splits, workers, min_segment, band_quarters, primary_quarters)


def plan_workspace_size(plan: Plan, num_rows: int, max_kv_len: int) -> tuple[int, int]:
    cb, wb = _sz(0), _sz(0)
    _check(_lib.topkf_plan_workspace_size(_c.byref(plan), int(num_rows), int(max_kv_len),
                                          _c.byref(cb), _c.byref(wb)), "topkf_plan_workspace_size")
    return cb.value, wb.value


def _stream_handle(stream, device):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return stream.cuda_stream


def _check_tensors(logits, ke, output, num_valid_rows, top_k):
    import torch
    if logits.dtype != torch.float32 or logits.dim() != 2:
        raise TypeError("logits must be a 2-D float32 tensor")
    if logits.shape[1] > 0 and logits.stride(1) != 1:
        raise ValueError("logits rows must be contiguous (stride(1) == 1)")
    if ke.dtype != torch.int32 or ke.dim() != 1 or ke.shape[0] != logits.shape[0]:
        raise TypeError("ke must be an int32 tensor with one entry per row")
    if not ke.is_contiguous():
        raise ValueError("ke must be contiguous")
    if output.dtype != torch.int32 or tuple(output.shape) != (logits.shape[0], top_k):
        raise TypeError("output must be an int32 tensor of shape [num_rows, top_k]")
    if not output.is_contiguous():
        raise ValueError("output must be contiguous")
    if num_valid_rows.dtype != torch.int32 or num_valid_rows.numel() != 1:
        raise TypeError("num_valid_rows must be a one-element int32 tensor")
    dev = logits.device
    for t in (ke, output, num_valid_rows):
        if t.device != dev:
            raise ValueError("all tensors must live on the device of logits")
    if dev.type != "cuda":
        raise ValueError("tensors must be on a GPU device")


def topk_filtered(logits, ke, output, num_valid_rows, top_k: int, counters, workspace,
                  stream=None, plan: Plan | None = None, route_stats=None, hint=None) -> None:
    """Exact row-wise Top-K of logits[r, :ke[r]] into output[r] for r < num_valid_rows.

    `plan` and `route_stats` (a uint32/int32 tensor of ROUTE_COUNT entries) select
    the diagnostic entry points; `hint` (float32, one proposed cutoff per row,
    NaN for none) selects topk_filtered_hinted.
    """
    _check_tensors(logits, ke, output, num_valid_rows, top_k)
    for name, t in (("counters", counters), ("workspace", workspace),
                    ("route_stats", route_stats)):
        if t is None:
            continue
        if t.device != logits.device or not t.is_contiguous():
            raise ValueError("%s must be a contiguous tensor on the device of logits" % name)
    if route_stats is not None and (route_stats.element_size() != 4 or
                                    route_stats.numel() < ROUTE_COUNT):
        raise TypeError("route_stats must hold at least %d 32-bit counters" % ROUTE_COUNT)
    m, n = logits.shape
    row_stride = logits.stride(0) if m > 0 else n
    st = _stream_handle(stream, logits.device)
    head = (logits.data_ptr(), m, n, row_stride, ke.data_ptr(), output.data_ptr(),
            num_valid_rows.data_ptr(), int(top_k))
    bufs = (counters.data_ptr(), counters.numel() * counters.element_size(), workspace.data_ptr(),
            workspace.numel() * workspace.element_size())
    debug = plan is not None or route_stats is not None
    pp = _c.byref(plan) if plan is not None else None
    rs = route_stats.data_ptr() if route_stats is not None else None
    if hint is not None:
        if hint.dtype != torch.float32 or hint.dim() != 1 or hint.shape[0] != m:
            raise TypeError("hint must be a float32 tensor with one entry per row")
        if not hint.is_contiguous() or hint.device != logits.device:
            raise ValueError("hint must be contiguous and on the device of logits")
        if debug:
            _check(_lib.topk_filtered_hinted_debug(*head, hint.data_ptr(), *bufs, pp, rs, st),
                   "topk_filtered_hinted_debug")
        else:
            _check(_lib.topk_filtered_hinted(*head, hint.data_ptr(), *bufs, st),
                   "topk_filtered_hinted")
    elif debug:
        _check(_lib.topk_filtered_debug(*head, *bufs, pp, rs, st), "topk_filtered_debug")
    else:
        _check(_lib.topk_filtered(*head, *bufs, st), "topk_filtered")


def topk_filtered_noalloc(logits, ke, output, num_valid_rows, top_k: int, stream=None) -> None:
    """topk_filtered without counter and workspace arguments: the library takes
    both from its own device array (see topk_filtered_noalloc in
    include/topkf.h; calls that overlap on one GPU race)."""
    _check_tensors(logits, ke, output, num_valid_rows, top_k)
    m, n = logits.shape
    row_stride = logits.stride(0) if m > 0 else n
    st = _stream_handle(stream, logits.device)
    _check(_lib.topk_filtered_noalloc(logits.data_ptr(), m, n, row_stride, ke.data_ptr(),
                                      output.data_ptr(), num_valid_rows.data_ptr(), int(top_k),
                                      st), "topk_filtered_noalloc")


def coarse_keys(x, out, stream=None) -> None:
    """out[i] = 11-bit coarse key of x[i] (float32 -> uint16/int16 tensor of equal size)."""
    if x.numel() != out.numel():
        raise ValueError("size mismatch")
    st = _stream_handle(stream, x.device)
    _check(_lib.topkf_coarse_keys(x.data_ptr(), x.numel(), out.data_ptr(), st), "topkf_coarse_keys")


def coarse_cutoffs(table, search, stream=None) -> None:
    """table, search: 2048-element int32/uint32 device tensors; see
    topkf_coarse_cutoffs in include/topkf.h."""
    if table.numel() < 2048 or search.numel() < 2048:
        raise ValueError("need 2048 entries")
    st = _stream_handle(stream, table.device)
    _check(_lib.topkf_coarse_cutoffs(table.data_ptr(), search.data_ptr(), st), "topkf_coarse_cutoffs")


def read_probe(x, sink, stream=None) -> None:
    """Plain 128-bit streaming read of the whole tensor x (the bandwidth
    reference); sink is a one-element int32/uint32 device tensor."""
    st = _stream_handle(stream, x.device)
    _check(_lib.topkf_read_probe(x.data_ptr(), x.numel() * x.element_size(), sink.data_ptr(), st),
           "topkf_read_probe")


class Selector:
    """Owns the counter and workspace buffers of one (num_rows, max_kv_len) shape."""

    def __init__(self, num_rows: int, max_kv_len: int, device="cuda", plan: Plan | None = None):
        import torch
        if plan is None:
            cb, wb = topk_filtered_workspace_size(num_rows, max_kv_len)
        else:
            cb, wb = plan_workspace_size(plan, num_rows, max_kv_len)
        self.plan = plan
        self.counters = torch.zeros(max(cb, 1), dtype=torch.uint8, device=device)
        self.workspace = torch.empty(max(wb, 1), dtype=torch.uint8, device=device)

    def __call__(self, logits, ke, output, num_valid_rows, top_k, stream=None, route_stats=None,
                 hint=None):
        topk_filtered(logits, ke, output, num_valid_rows, top_k, self.counters, self.workspace,
                      stream=stream, plan=self.plan, route_stats=route_stats, hint=hint)
