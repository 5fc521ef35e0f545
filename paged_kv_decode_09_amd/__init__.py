"""Paged-KV batch decode attention for AMD MI355X (gfx950).

A thin ctypes binding over the C-ABI library ``libpkd.so`` (include/pkd.h).
This module only marshals arguments: torch provides device memory and the
current stream, and every step of the computation runs in the library's HIP
kernels. If the library is missing the calls raise; there is no fallback.

Names follow flashinfer.decode.BatchDecodeWithPagedKVCacheWrapper on the
"FlashInfer attention kernels" page (plan() / run() parameters).
"""
import ctypes
import math
import os
from typing import Optional, Sequence, Tuple, Union

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpkd.so")
ABI_VERSION = 4            # PKD_ABI_VERSION of include/pkd.h

PKD_OK, PKD_EINVAL, PKD_EUNSUPPORTED, PKD_EHIP, PKD_ENOMEM, PKD_EWORKSPACE = (
    0, -1, -2, -3, -4, -5)
PKD_F16, PKD_BF16, PKD_E4M3, PKD_F32 = 0, 1, 2, 3
PKD_NHD, PKD_HND = 0, 1

_STATUS = {PKD_EINVAL: "EINVAL", PKD_EUNSUPPORTED: "EUNSUPPORTED",
           PKD_EHIP: "EHIP", PKD_ENOMEM: "ENOMEM", PKD_EWORKSPACE: "EWORKSPACE"}


class PkdError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"pkd {_STATUS.get(status, status)}: {msg}")
        self.status = status


class pkd_plan_params(ctypes.Structure):
    _fields_ = [("batch_size", ctypes.c_int32), ("num_qo_heads", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("page_size", ctypes.c_int32), ("layout", ctypes.c_int32),
                ("q_dtype", ctypes.c_int32), ("kv_dtype", ctypes.c_int32),
                ("o_dtype", ctypes.c_int32), ("sm_scale", ctypes.c_float),
                ("logits_soft_cap", ctypes.c_float),
                ("window_left", ctypes.c_int32),
                ("fixed_split_size", ctypes.c_int32),
                ("disable_split_kv", ctypes.c_int32),
                ("q_len_per_req", ctypes.c_int32),
                ("pos_encoding_mode", ctypes.c_int32),
                ("rope_scale", ctypes.c_float), ("rope_theta", ctypes.c_float)]


class pkd_work_item(ctypes.Structure):
    _fields_ = [("request", ctypes.c_int32), ("kv_head", ctypes.c_int32),
                ("token_begin", ctypes.c_int32), ("token_end", ctypes.c_int32),
                ("page_base", ctypes.c_int32), ("partial", ctypes.c_int32),
                ("chunk", ctypes.c_int32), ("num_chunks", ctypes.c_int32),
                ("query_pos", ctypes.c_int32)]


class pkd_plan_info(ctypes.Structure):
    _fields_ = [("num_items", ctypes.c_int32),
                ("num_workgroups", ctypes.c_int32),
                ("num_split_requests", ctypes.c_int32),
                ("num_partials", ctypes.c_int32),
                ("split_pages", ctypes.c_int32),
                ("workgroups_per_cu", ctypes.c_int32),
                ("attended_tokens", ctypes.c_int64),
                ("workspace_bytes", ctypes.c_size_t)]


_P = ctypes.c_void_p
_SIGS = {
    "pkd_abi_version": (ctypes.c_int32, []),
    "pkd_last_error": (ctypes.c_char_p, []),
    "pkd_plan_create": (ctypes.c_int, [ctypes.POINTER(pkd_plan_params), _P, _P,
                                       _P, _P, ctypes.POINTER(_P)]),
    "pkd_plan_query": (ctypes.c_int, [ctypes.POINTER(pkd_plan_params), _P, _P,
                                      ctypes.c_int32,
                                      ctypes.POINTER(pkd_plan_info), _P,
                                      ctypes.c_int32]),
    "pkd_plan_create_block_table": (ctypes.c_int, [ctypes.POINTER(pkd_plan_params),
                                                   _P, _P, ctypes.c_int32, _P,
                                                   ctypes.POINTER(_P)]),
    "pkd_plan_query_block_table": (ctypes.c_int, [ctypes.POINTER(pkd_plan_params), _P,
                                                  ctypes.c_int32, ctypes.c_int32,
                                                  ctypes.POINTER(pkd_plan_info), _P,
                                                  ctypes.c_int32]),
    "pkd_plan_create_graph": (ctypes.c_int, [ctypes.POINTER(pkd_plan_params),
                                             ctypes.c_int32, _P, _P, _P, _P,
                                             ctypes.POINTER(_P)]),
    "pkd_plan_update": (ctypes.c_int, [_P, _P, _P, _P]),
    "pkd_plan_get_info": (ctypes.c_int, [_P, ctypes.POINTER(pkd_plan_info)]),
    "pkd_plan_workspace_bytes": (ctypes.c_int, [_P, ctypes.POINTER(ctypes.c_size_t)]),
    "pkd_plan_destroy": (None, [_P]),
    "pkd_run": (ctypes.c_int, [_P, _P, _P, _P, ctypes.c_int64, ctypes.c_float,
                               ctypes.c_float, ctypes.c_float, _P, _P, _P, _P,
                               ctypes.c_size_t, _P]),
    "pkd_run_static_workspace": (ctypes.c_int, [_P, _P, _P, _P, ctypes.c_int64,
                                                ctypes.c_float, ctypes.c_float,
                                                ctypes.c_float, _P, _P, _P, _P]),
    "pkd_merge_states": (ctypes.c_int, [_P, _P, ctypes.c_int32, ctypes.c_int32,
                                        ctypes.c_int32, _P, ctypes.c_int32, _P,
                                        _P]),
}

_lib_handle = None


def lib() -> ctypes.CDLL:
    """The loaded C-ABI library; raises if it was not built."""
    global _lib_handle
    if _lib_handle is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m paged_kv_decode_09_amd.build` (no fallback exists)")
        h = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(h, name)
            f.restype = res
            f.argtypes = args
        if h.pkd_abi_version() != ABI_VERSION:
            raise ImportError("libpkd.so ABI version mismatch")
        _lib_handle = h
    return _lib_handle


def _check(status: int) -> None:
    if status != PKD_OK:
        raise PkdError(status, lib().pkd_last_error().decode())


def _dtype_code(dt) -> int:
    if isinstance(dt, str):
        dt = {"float16": torch.float16, "half": torch.float16,
              "bfloat16": torch.bfloat16, "float8_e4m3fn": torch.float8_e4m3fn,
              "f16": torch.float16, "bf16": torch.bfloat16,
              "e4m3": torch.float8_e4m3fn}[dt]
    if dt == torch.float16:
        return PKD_F16
    if dt == torch.bfloat16:
        return PKD_BF16
    if dt in (torch.float8_e4m3fn, torch.uint8):
        return PKD_E4M3
    if dt == torch.float32:
        return PKD_F32
    raise PkdError(PKD_EUNSUPPORTED, f"dtype {dt} is not supported")


_POS_MODES = {"NONE": 0, "ROPE_LLAMA": 1, "ALIBI": 2}

_TORCH_OF = {PKD_F16: torch.float16, PKD_BF16: torch.bfloat16,
             PKD_F32: torch.float32}


def _host_i32(x) -> np.ndarray:
    if isinstance(x, torch.Tensor):
        x = x.detach().cpu().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.int32))


def _stream_ptr(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _foreign_stream(stream):
    """The torch stream `stream` names when it is not torch's current stream,
    else None. Tensors the binding allocates on the current stream for a run
    on such a stream are marked as in use on it (record_stream), so that the
    caching allocator hands their memory to no other tensor before that
    run's kernel has finished with it."""
    if stream is None:
        return None
    cur = torch.cuda.current_stream()
    if isinstance(stream, torch.cuda.Stream):
        return None if stream.cuda_stream == cur.cuda_stream else stream
    ptr = int(stream)
    return None if ptr == cur.cuda_stream else torch.cuda.ExternalStream(ptr)


def make_params(batch_size, num_qo_heads, num_kv_heads, head_dim, page_size,
                kv_layout="NHD", window_left=-1, logits_soft_cap=None,
                q_data_type=torch.float16, kv_data_type=None,
                o_data_type=None, sm_scale=None, fixed_split_size=None,
                disable_split_kv=False, q_len_per_req=1, pos_encoding_mode="NONE",
                rope_scale=None, rope_theta=None) -> pkd_plan_params:
    q_code = _dtype_code(q_data_type)
    kv_code = q_code if kv_data_type is None else _dtype_code(kv_data_type)
    o_code = q_code if o_data_type is None else _dtype_code(o_data_type)
    if kv_layout not in ("NHD", "HND"):
        raise PkdError(PKD_EINVAL, f"kv_layout {kv_layout!r} not NHD/HND")
    return pkd_plan_params(
        batch_size=int(batch_size), num_qo_heads=int(num_qo_heads),
        num_kv_heads=int(num_kv_heads), head_dim=int(head_dim),
        page_size=int(page_size),
        layout=PKD_NHD if kv_layout == "NHD" else PKD_HND,
        q_dtype=q_code, kv_dtype=kv_code, o_dtype=o_code,
        sm_scale=(1.0 / math.sqrt(head_dim)) if sm_scale is None else sm_scale,
        logits_soft_cap=0.0 if not logits_soft_cap else logits_soft_cap,
        window_left=int(window_left),
        fixed_split_size=0 if not fixed_split_size else int(fixed_split_size),
        disable_split_kv=int(bool(disable_split_kv)),
        q_len_per_req=1 if q_len_per_req is None else int(q_len_per_req),
        pos_encoding_mode=_POS_MODES.get(pos_encoding_mode, -1)
        if isinstance(pos_encoding_mode, str) else int(pos_encoding_mode),
        rope_scale=1.0 if rope_scale is None else float(rope_scale),
        rope_theta=1e4 if rope_theta is None else float(rope_theta))


def plan_query(indptr, last_page_len, num_cus: int = 256, **kw):
    """Host-only planning (no GPU): (pkd_plan_info, list of work items)."""
    ip, lp = _host_i32(indptr), _host_i32(last_page_len)
    params = make_params(len(lp), **kw)
    info = pkd_plan_info()
    _check(lib().pkd_plan_query(ctypes.byref(params), ip.ctypes.data,
                                lp.ctypes.data, num_cus, ctypes.byref(info),
                                None, 0))
    items = (pkd_work_item * max(info.num_items, 1))()
    _check(lib().pkd_plan_query(ctypes.byref(params), ip.ctypes.data,
                                lp.ctypes.data, num_cus, ctypes.byref(info),
                                ctypes.cast(items, _P), info.num_items))
    return info, list(items)[:info.num_items]


def plan_query_block_table(seq_lens, max_blocks_per_seq: int,
                           num_cus: int = 256, **kw):
    """Host-only planning of a block-table batch: (pkd_plan_info, items)."""
    sl = _host_i32(seq_lens)
    params = make_params(len(sl), **kw)
    info = pkd_plan_info()
    _check(lib().pkd_plan_query_block_table(ctypes.byref(params), sl.ctypes.data,
                                            int(max_blocks_per_seq), num_cus,
                                            ctypes.byref(info), None, 0))
    items = (pkd_work_item * max(info.num_items, 1))()
    _check(lib().pkd_plan_query_block_table(ctypes.byref(params), sl.ctypes.data,
                                            int(max_blocks_per_seq), num_cus,
                                            ctypes.byref(info),
                                            ctypes.cast(items, _P), info.num_items))
    return info, list(items)[:info.num_items]


def _split_cache(paged_kv_cache, layout: int, page_size: int,
                 num_kv_heads: int, head_dim: int):
    """(k pointer, v pointer, page stride in elements, dtype) of a cache."""
    page = (page_size, num_kv_heads, head_dim) if layout == PKD_NHD else (
        num_kv_heads, page_size, head_dim)
    inner = (num_kv_heads * head_dim, head_dim, 1) if layout == PKD_NHD else (
        page_size * head_dim, head_dim, 1)
    if isinstance(paged_kv_cache, (tuple, list)):
        k, v = paged_kv_cache
        for t in (k, v):
            if t.dim() != 4 or tuple(t.shape[1:]) != page or \
                    tuple(t.stride()[1:]) != inner:
                raise PkdError(PKD_EINVAL, f"cache tensor {tuple(t.shape)} is "
                               f"not [pages, {', '.join(map(str, page))}] "
                               "with contiguous pages")
        if k.stride(0) != v.stride(0) or k.dtype != v.dtype:
            raise PkdError(PKD_EINVAL, "k_cache and v_cache must share the "
                           "page stride and dtype")
        return k.data_ptr(), v.data_ptr(), k.stride(0), k.dtype
    c = paged_kv_cache
    if c.dim() != 5 or c.shape[1] != 2 or tuple(c.shape[2:]) != page or \
            tuple(c.stride()[2:]) != inner or \
            c.stride(1) != page_size * num_kv_heads * head_dim:
        raise PkdError(PKD_EINVAL, f"cache {tuple(c.shape)} is not "
                       f"[pages, 2, {', '.join(map(str, page))}] with "
                       "contiguous pages")
    kp = c.data_ptr()
    return kp, kp + c.stride(1) * c.element_size(), c.stride(0), c.dtype


class PagedDecodePlan:
    """One plan (pkd_plan_create): a batch's page table, reused across runs.

    The page table is either CSR (indptr, indices, last_page_len) or, with
    ``block_tables`` (int32 device [B, max_blocks]) and ``seq_lens`` (host or
    device int32 [B]), a block table (pkd_plan_create_block_table); then
    indptr / indices / last_page_len are None.
    """

    def __init__(self, indptr, indices: Optional[torch.Tensor], last_page_len,
                 num_qo_heads: int, num_kv_heads: int, head_dim: int,
                 page_size: int, kv_layout: str = "NHD", window_left: int = -1,
                 logits_soft_cap: Optional[float] = None,
                 q_data_type=torch.float16, kv_data_type=None,
                 o_data_type=None, sm_scale: Optional[float] = None,
                 fixed_split_size: Optional[int] = None,
                 disable_split_kv: bool = False, stream=None,
                 q_len_per_req: int = 1, seq_lens=None,
                 block_tables: Optional[torch.Tensor] = None,
                 graph_max_pages: Optional[int] = None,
                 pos_encoding_mode: str = "NONE", rope_scale=None,
                 rope_theta=None):
        """``graph_max_pages``: make a graph plan (pkd_plan_create_graph) whose
        device memory, launch size and workspace layout hold for any later
        page table of the same batch size with at most that many pages
        (``update``); ``indices`` is then the fixed page index buffer."""
        self._handle = None
        table = block_tables if block_tables is not None else indices
        if table is None or table.dtype != torch.int32 or not table.is_cuda:
            raise PkdError(PKD_EINVAL, "indices / block_tables must be an int32 "
                           "device tensor")
        if block_tables is not None:
            if indptr is not None or indices is not None or \
                    last_page_len is not None or seq_lens is None:
                raise PkdError(PKD_EINVAL, "give either indptr/indices/"
                               "last_page_len or block_tables/seq_lens")
            if block_tables.dim() != 2:
                raise PkdError(PKD_EINVAL, "block_tables must be [batch, "
                               "max_blocks]")
            sl = _host_i32(seq_lens)
            batch = len(sl)
            if block_tables.shape[0] != batch:
                raise PkdError(PKD_EINVAL, "block_tables and seq_lens differ "
                               "in batch size")
        else:
            ip, lp = _host_i32(indptr), _host_i32(last_page_len)
            batch = len(lp)
        self.params = make_params(batch, num_qo_heads, num_kv_heads, head_dim,
                                  page_size, kv_layout, window_left,
                                  logits_soft_cap, q_data_type, kv_data_type,
                                  o_data_type, sm_scale, fixed_split_size,
                                  disable_split_kv, q_len_per_req,
                                  pos_encoding_mode, rope_scale, rope_theta)
        self.indices = table.contiguous()   # borrowed by the plan: keep alive
        h = _P()
        if graph_max_pages is not None:
            if block_tables is not None:
                raise PkdError(PKD_EINVAL, "a graph plan takes a CSR page table")
            _check(lib().pkd_plan_create_graph(
                ctypes.byref(self.params), int(graph_max_pages), ip.ctypes.data,
                lp.ctypes.data, self.indices.data_ptr(), _stream_ptr(stream),
                ctypes.byref(h)))
        elif block_tables is not None:
            _check(lib().pkd_plan_create_block_table(
                ctypes.byref(self.params), sl.ctypes.data,
                self.indices.data_ptr(), int(self.indices.shape[1]),
                _stream_ptr(stream), ctypes.byref(h)))
        else:
            _check(lib().pkd_plan_create(ctypes.byref(self.params),
                                         ip.ctypes.data, lp.ctypes.data,
                                         self.indices.data_ptr(),
                                         _stream_ptr(stream), ctypes.byref(h)))
        self._handle = h
        self.info = pkd_plan_info()
        _check(lib().pkd_plan_get_info(self._handle, ctypes.byref(self.info)))

    def __del__(self):
        if getattr(self, "_handle", None) is not None and _lib_handle is not None:
            _lib_handle.pkd_plan_destroy(self._handle)
            self._handle = None

    @property
    def workspace_bytes(self) -> int:
        n = ctypes.c_size_t()
        _check(lib().pkd_plan_workspace_bytes(self._handle, ctypes.byref(n)))
        return int(n.value)

    def update(self, indptr, last_page_len, stream=None) -> None:
        """A graph plan's new page table (pkd_plan_update): same batch size,
        pages already in the plan's index buffer. Not capturable."""
        ip, lp = _host_i32(indptr), _host_i32(last_page_len)
        if len(lp) != self.params.batch_size or len(ip) != len(lp) + 1:
            raise PkdError(PKD_EINVAL, "a graph plan keeps its batch size "
                           f"({self.params.batch_size})")
        _check(lib().pkd_plan_update(self._handle, ip.ctypes.data,
                                     lp.ctypes.data, _stream_ptr(stream)))
        _check(lib().pkd_plan_get_info(self._handle, ctypes.byref(self.info)))

    def _args(self, q, paged_kv_cache, q_scale, k_scale, v_scale, out, lse,
              return_lse, workspace, allocate_workspace=True):
        p = self.params
        # q, o and lse hold q_len_per_req rows per request
        B = p.batch_size * max(1, p.q_len_per_req)
        nq, hd = p.num_qo_heads, p.head_dim
        if tuple(q.shape) != (B, nq, hd) or not q.is_contiguous():
            raise PkdError(PKD_EINVAL, f"q must be contiguous [{B}, {nq}, {hd}]")
        if _dtype_code(q.dtype) != p.q_dtype:
            raise PkdError(PKD_EINVAL, f"q dtype {q.dtype} differs from the plan")
        kp, vp, stride, kv_dtype = _split_cache(paged_kv_cache, p.layout,
                                                p.page_size, p.num_kv_heads, hd)
        if _dtype_code(kv_dtype) != p.kv_dtype:
            raise PkdError(PKD_EINVAL, f"cache dtype {kv_dtype} differs from "
                           "the plan")
        temps = []        # tensors allocated here for this run
        if out is None:
            out = torch.empty((B, nq, hd), dtype=_TORCH_OF[p.o_dtype],
                              device=q.device)
            temps.append(out)
        elif tuple(out.shape) != (B, nq, hd) or not out.is_contiguous() or \
                _dtype_code(out.dtype) != p.o_dtype:
            raise PkdError(PKD_EINVAL, "out has the wrong shape or dtype")
        if return_lse and lse is None:
            lse = torch.empty((B, nq), dtype=torch.float32, device=q.device)
            temps.append(lse)
        elif lse is not None and (tuple(lse.shape) != (B, nq) or
                                  lse.dtype != torch.float32 or
                                  not lse.is_contiguous()):
            raise PkdError(PKD_EINVAL, f"lse must be contiguous fp32 [{B}, {nq}]")
        ws_bytes = self.workspace_bytes
        if workspace is None and ws_bytes > 0 and allocate_workspace:
            workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
            temps.append(workspace)
        ws_ptr = workspace.data_ptr() if workspace is not None else None
        ws_len = workspace.numel() * workspace.element_size() if \
            workspace is not None else 0
        sc = [1.0 if s is None else float(s) for s in (q_scale, k_scale, v_scale)]
        return (q, kp, vp, stride, sc, out, lse, ws_ptr, ws_len, temps)

    def run(self, q: torch.Tensor, paged_kv_cache, q_scale=None, k_scale=None,
            v_scale=None, out=None, lse=None, return_lse: bool = False,
            workspace: Optional[torch.Tensor] = None, stream=None,
            sinks: Optional[torch.Tensor] = None):
        """o [B * q_len_per_req, num_qo_heads, head_dim], or (o, lse) when
        return_lse. ``sinks``: fp32 device tensor of num_qo_heads values
        ([num_kv_heads, G] or flat), one sink logit per q head."""
        (q, kp, vp, stride, sc, out, lse, ws_ptr, ws_len,
         temps) = self._args(q, paged_kv_cache, q_scale, k_scale, v_scale, out,
                             lse, return_lse or lse is not None, workspace)
        sink_ptr = self._sink_ptr(sinks)
        _check(lib().pkd_run(self._handle, q.data_ptr(), kp, vp, stride,
                             sc[0], sc[1], sc[2], sink_ptr, out.data_ptr(),
                             lse.data_ptr() if lse is not None else None,
                             ws_ptr, ws_len, _stream_ptr(stream)))
        _keep_for_stream(temps, stream)
        return (out, lse) if return_lse else out

    def run_static_workspace(self, q: torch.Tensor, paged_kv_cache, q_scale=None,
                             k_scale=None, v_scale=None, out=None, lse=None,
                             return_lse: bool = False, stream=None,
                             sinks: Optional[torch.Tensor] = None):
        """run() through pkd_run_static_workspace: the split-KV partial states
        go to the library's static workspace on the GPU instead of a caller's
        workspace, so the call allocates nothing when ``out`` (and ``lse``,
        if wanted) are given. Such calls on different streams are ordered
        on the GPU by the library; calls recorded into graphs are not."""
        (q, kp, vp, stride, sc, out, lse, _ws_ptr, _ws_len,
         temps) = self._args(q, paged_kv_cache, q_scale, k_scale, v_scale, out,
                             lse, return_lse or lse is not None, None,
                             allocate_workspace=False)
        _check(lib().pkd_run_static_workspace(
            self._handle, q.data_ptr(), kp, vp, stride, sc[0], sc[1], sc[2],
            self._sink_ptr(sinks), out.data_ptr(),
            lse.data_ptr() if lse is not None else None, _stream_ptr(stream)))
        _keep_for_stream(temps, stream)
        return (out, lse) if return_lse else out

    def _sink_ptr(self, sinks):
        if sinks is None:
            return None
        if sinks.dtype != torch.float32 or not sinks.is_cuda or \
                not sinks.is_contiguous() or \
                sinks.numel() != self.params.num_qo_heads:
            raise PkdError(PKD_EINVAL, "sinks must be a contiguous fp32 "
                           f"device tensor of {self.params.num_qo_heads} "
                           "values")
        return sinks.data_ptr()


def _keep_for_stream(temps, stream) -> None:
    """record_stream on the run's stream for each tensor allocated for the
    run, when that stream is not torch's current stream."""
    fs = _foreign_stream(stream) if temps else None
    if fs is not None:
        for t in temps:
            t.record_stream(fs)


class BatchDecodeWithPagedKVCacheWrapper:
    """plan()/run() in the shape of the wrapper on the FlashInfer page.

    ``float_workspace_buffer`` is a uint8 device tensor used for split-KV
    partial states; it is grown (reallocated) if a plan needs more.

    The constructor takes the page's arguments. With ``use_cuda_graph`` the
    page table lives in the three ``paged_kv_*_buffer`` tensors (all
    required) and the wrapper behaves as
    CUDAGraphBatchDecodeWithPagedKVCacheWrapper: a run captured in a HIP
    graph follows every later plan() of the same batch size and parameters,
    and the workspace is not grown. ``use_tensor_cores`` changes nothing
    (q.K and P.V run on MFMA at every group size); ``backend`` takes "auto"
    only (one gfx950 implementation) and ``jit_args`` None (the kernels are
    built ahead of time).
    """

    def __init__(self, float_workspace_buffer: torch.Tensor,
                 kv_layout: str = "NHD", use_cuda_graph: bool = False,
                 use_tensor_cores: bool = False,
                 paged_kv_indptr_buffer: Optional[torch.Tensor] = None,
                 paged_kv_indices_buffer: Optional[torch.Tensor] = None,
                 paged_kv_last_page_len_buffer: Optional[torch.Tensor] = None,
                 backend: str = "auto", jit_args=None):
        if backend != "auto":
            raise PkdError(PKD_EUNSUPPORTED, f"backend {backend!r}: only 'auto' "
                           "(the gfx950 kernels of this library)")
        if jit_args is not None:
            raise PkdError(PKD_EUNSUPPORTED, "jit_args: the kernels are built "
                           "ahead of time")
        self._ws = float_workspace_buffer
        self._layout = kv_layout
        self._plan: Optional[PagedDecodePlan] = None
        self._graph: Optional[CUDAGraphBatchDecodeWithPagedKVCacheWrapper] = None
        if use_cuda_graph:
            for name, t in (("paged_kv_indptr_buffer", paged_kv_indptr_buffer),
                            ("paged_kv_indices_buffer", paged_kv_indices_buffer),
                            ("paged_kv_last_page_len_buffer",
                             paged_kv_last_page_len_buffer)):
                if t is None:
                    raise PkdError(PKD_EINVAL, f"use_cuda_graph needs {name}")
            self._graph = CUDAGraphBatchDecodeWithPagedKVCacheWrapper(
                float_workspace_buffer, paged_kv_indptr_buffer,
                paged_kv_indices_buffer, paged_kv_last_page_len_buffer,
                kv_layout, use_tensor_cores)

    def reset_workspace_buffer(self, float_workspace_buffer: torch.Tensor,
                               int_workspace_buffer=None) -> None:
        self._ws = float_workspace_buffer

    def plan(self, indptr, indices, last_page_len, num_qo_heads, num_kv_heads,
             head_dim, page_size, pos_encoding_mode="NONE", window_left=-1,
             logits_soft_cap=None, q_data_type=torch.float16,
             kv_data_type=None, o_data_type=None, data_type=None,
             sm_scale=None, rope_scale=None, rope_theta=None,
             non_blocking=True, fixed_split_size=None,
             disable_split_kv=False, q_len_per_req=1, seq_lens=None,
             block_tables=None) -> None:
        """plan() of the page. With ``block_tables`` [B, max_blocks] and
        ``seq_lens`` [B] the page table is a block table; indptr, indices and
        last_page_len are then None."""
        if self._graph is not None:
            if block_tables is not None or seq_lens is not None:
                raise PkdError(PKD_EINVAL, "use_cuda_graph keeps a CSR page "
                               "table in its buffers; block_tables is not "
                               "taken there")
            self._graph.plan(indptr, indices, last_page_len, num_qo_heads,
                             num_kv_heads, head_dim, page_size, pos_encoding_mode,
                             window_left, logits_soft_cap, q_data_type,
                             kv_data_type, o_data_type, data_type, sm_scale,
                             rope_scale, rope_theta, non_blocking,
                             fixed_split_size, disable_split_kv, q_len_per_req)
            self._plan = self._graph._plan
            return
        if data_type is not None:
            q_data_type = data_type
            kv_data_type = kv_data_type or data_type
        self._plan = PagedDecodePlan(
            indptr, None if indices is None else indices.to(torch.int32),
            last_page_len, num_qo_heads,
            num_kv_heads, head_dim, page_size, self._layout, window_left,
            logits_soft_cap, q_data_type, kv_data_type, o_data_type, sm_scale,
            fixed_split_size, disable_split_kv, q_len_per_req=q_len_per_req,
            pos_encoding_mode=pos_encoding_mode, rope_scale=rope_scale,
            rope_theta=rope_theta, seq_lens=seq_lens,
            block_tables=None if block_tables is None else
            block_tables.to(torch.int32))
        need = self._plan.workspace_bytes
        if self._ws.numel() * self._ws.element_size() < need:
            self._ws = torch.empty(need, dtype=torch.uint8,
                                   device=self._ws.device)

    def run(self, q, paged_kv_cache, q_scale=None, k_scale=None, v_scale=None,
            out=None, lse=None, return_lse=False, q_len_per_req=None,
            sinks=None, enable_pdl=None):
        """run() of the page (``enable_pdl``, a launch feature of other
        GPUs, changes nothing here)."""
        if self._plan is None:
            raise PkdError(PKD_EINVAL, "run() before plan()")
        planned = max(1, self._plan.params.q_len_per_req)
        if q_len_per_req is not None and int(q_len_per_req) != planned:
            raise PkdError(PKD_EINVAL, f"q_len_per_req {q_len_per_req} differs "
                           f"from the plan's {planned}")
        if self._graph is not None:
            return self._graph.run(q, paged_kv_cache, q_scale, k_scale, v_scale,
                                   out, lse, return_lse, sinks=sinks)
        ws = self._ws if self._plan.workspace_bytes > 0 else None
        return self._plan.run(q, paged_kv_cache, q_scale, k_scale, v_scale,
                              out, lse, return_lse, ws, sinks=sinks)


class CUDAGraphBatchDecodeWithPagedKVCacheWrapper:
    """The graph-capturable decode wrapper of the page: the page table lives
    in fixed device buffers, plan() (not capturable) rewrites them and the
    plan's work list in place, and a run() captured once in a HIP graph
    serves every later plan() of the same batch size and parameters.

    ``indices_buffer`` bounds the pages of any batch (max_num_pages);
    ``indptr_buffer`` / ``last_page_len_buffer`` hold [batch + 1] / [batch].
    The workspace must hold the plan's capacity-based workspace_bytes.
    """

    def __init__(self, workspace_buffer: torch.Tensor, indptr_buffer: torch.Tensor,
                 indices_buffer: torch.Tensor, last_page_len_buffer: torch.Tensor,
                 kv_layout: str = "NHD", use_tensor_cores: bool = False):
        for name, t in (("indptr_buffer", indptr_buffer),
                        ("indices_buffer", indices_buffer),
                        ("last_page_len_buffer", last_page_len_buffer)):
            if t.dtype != torch.int32 or not t.is_cuda or not t.is_contiguous():
                raise PkdError(PKD_EINVAL, f"{name} must be a contiguous int32 "
                               "device tensor")
        self._ws = workspace_buffer
        self._indptr_buf = indptr_buffer
        self._indices_buf = indices_buffer
        self._last_buf = last_page_len_buffer
        self._layout = kv_layout
        self._plan: Optional[PagedDecodePlan] = None
        self._key = None

    def plan(self, indptr, indices, last_page_len, num_qo_heads, num_kv_heads,
             head_dim, page_size, pos_encoding_mode="NONE", window_left=-1,
             logits_soft_cap=None, q_data_type=torch.float16,
             kv_data_type=None, o_data_type=None, data_type=None,
             sm_scale=None, rope_scale=None, rope_theta=None,
             non_blocking=True, fixed_split_size=None,
             disable_split_kv=False, q_len_per_req=1) -> None:
        if data_type is not None:
            q_data_type = data_type
            kv_data_type = kv_data_type or data_type
        ip, lp = _host_i32(indptr), _host_i32(last_page_len)
        B, n = len(lp), int(ip[-1]) if len(ip) else 0
        if B + 1 > self._indptr_buf.numel() or B > self._last_buf.numel():
            raise PkdError(PKD_EINVAL, f"batch {B} exceeds the indptr / "
                           "last_page_len buffers")
        if n > self._indices_buf.numel():
            raise PkdError(PKD_EINVAL, f"{n} pages exceed the indices buffer "
                           f"({self._indices_buf.numel()})")
        params = make_params(B, num_qo_heads, num_kv_heads, head_dim, page_size,
                             self._layout, window_left, logits_soft_cap,
                             q_data_type, kv_data_type, o_data_type, sm_scale,
                             fixed_split_size, disable_split_kv, q_len_per_req,
                             pos_encoding_mode, rope_scale, rope_theta)
        key = bytes(params)
        src = indices if isinstance(indices, torch.Tensor) else \
            torch.from_numpy(_host_i32(indices))
        if src.numel() < n:
            raise PkdError(PKD_EINVAL, f"indices holds {src.numel()} entries, "
                           f"indptr needs {n}")
        # plan first (it validates), then the page table into the fixed
        # buffers; both are ordered before later runs on the current stream
        if self._plan is None:
            self._plan = PagedDecodePlan(
                ip, self._indices_buf, lp, num_qo_heads, num_kv_heads, head_dim,
                page_size, self._layout, window_left, logits_soft_cap,
                q_data_type, kv_data_type, o_data_type, sm_scale,
                fixed_split_size, disable_split_kv, q_len_per_req=q_len_per_req,
                graph_max_pages=self._indices_buf.numel(),
                pos_encoding_mode=pos_encoding_mode, rope_scale=rope_scale,
                rope_theta=rope_theta)
            self._key = key
        else:
            if key != self._key:
                raise PkdError(PKD_EINVAL, "a graph wrapper keeps its batch size "
                               "and parameters; create a new wrapper")
            self._plan.update(ip, lp)
        self._indptr_buf[:B + 1].copy_(torch.from_numpy(ip), non_blocking=True)
        self._last_buf[:B].copy_(torch.from_numpy(lp), non_blocking=True)
        self._indices_buf[:n].copy_(src[:n].to(torch.int32), non_blocking=True)
        need = self._plan.workspace_bytes
        if self._ws.numel() * self._ws.element_size() < need:
            raise PkdError(PKD_EWORKSPACE, f"workspace of "
                           f"{self._ws.numel() * self._ws.element_size()} bytes "
                           f"< {need} needed by the graph plan's capacity")

    def run(self, q, paged_kv_cache, q_scale=None, k_scale=None, v_scale=None,
            out=None, lse=None, return_lse=False, sinks=None, enable_pdl=None,
            q_len_per_req=None):
        if self._plan is None:
            raise PkdError(PKD_EINVAL, "run() before plan()")
        planned = max(1, self._plan.params.q_len_per_req)
        if q_len_per_req is not None and int(q_len_per_req) != planned:
            raise PkdError(PKD_EINVAL, f"q_len_per_req {q_len_per_req} differs "
                           f"from the plan's {planned}")
        ws = self._ws if self._plan.workspace_bytes > 0 else None
        return self._plan.run(q, paged_kv_cache, q_scale, k_scale, v_scale,
                              out, lse, return_lse, ws, sinks=sinks)


def merge_states(v: torch.Tensor, s: torch.Tensor, out_dtype=None,
                 stream=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Merge attention states (pkd_merge_states).

    v: fp32 [rows, num_states, head_dim]; s: fp32 [rows, num_states]
    natural-log LSE. Returns (v_merged [rows, head_dim], s_merged [rows]).
    """
    if v.dtype != torch.float32 or s.dtype != torch.float32 or \
            v.dim() != 3 or s.shape != v.shape[:2]:
        raise PkdError(PKD_EINVAL, "v must be fp32 [rows, n, hd] and s fp32 "
                       "[rows, n]")
    v, s = v.contiguous(), s.contiguous()
    rows, n, hd = v.shape
    od = torch.float32 if out_dtype is None else out_dtype
    v_out = torch.empty((rows, hd), dtype=od, device=v.device)
    s_out = torch.empty((rows,), dtype=torch.float32, device=v.device)
    _check(lib().pkd_merge_states(v.data_ptr(), s.data_ptr(), rows, n, hd,
                                  v_out.data_ptr(), _dtype_code(od),
                                  s_out.data_ptr(), _stream_ptr(stream)))
    _keep_for_stream([v_out, s_out], stream)
    return v_out, s_out


__all__ = ["lib", "PkdError", "PagedDecodePlan",
           "BatchDecodeWithPagedKVCacheWrapper",
           "CUDAGraphBatchDecodeWithPagedKVCacheWrapper", "merge_states",
           "plan_query",
           "plan_query_block_table",
           "make_params", "pkd_plan_params", "pkd_plan_info", "pkd_work_item"]
