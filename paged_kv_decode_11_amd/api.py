"""Python binding of libpkd (same names as the C ABI, marshalling only).

torch is used for device memory, pinned host memory and streams; every step
of the decode path runs in the library's HIP kernels or its host scheduler.
"""

from __future__ import annotations

import ctypes

import numpy as np

from . import _lib
from ._lib import PkdError, check, pkd_plan_opts  # noqa: F401

_DTYPES = None


class PlanMismatchError(PkdError, ValueError):
    """A run's tensors do not have the shape the current plan was made for
    (raised by the binding before anything is launched; status
    PKD_ERR_STALE_PLAN)."""

    def __init__(self, message: str):
        super().__init__(_lib.PKD_ERR_STALE_PLAN, message)


PLAN_SHAPE_FIELDS = ("batch", "num_qo_heads", "num_kv_heads", "head_dim", "page_size", "q_dtype",
                     "kv_dtype", "kind")


def check_run_args(plan_shape: dict, q, kv_cache, out=None, lse=None) -> None:
    """Refuse a run whose tensors do not fit the plan (PlanMismatchError).

    Uses only .shape / .dtype, so it runs on CPU or meta tensors too.  The
    batch (rows of q) is compared with the plan by pkd_run itself; here q
    must be [rows, num_qo_heads, head_dim], the cache [pages, 2, page_size,
    num_kv_heads, head_dim], and a given out [rows, num_qo_heads, head_dim]
    bf16 and lse [rows, num_qo_heads] fp32 (pkd_run writes exactly those
    extents; any other shape would be read or written past its end)."""
    import torch

    Hq, Hkv, D, P = (plan_shape[k] for k in ("num_qo_heads", "num_kv_heads", "head_dim",
                                            "page_size"))
    if len(q.shape) != 3 or tuple(q.shape[1:]) != (Hq, D):
        raise PlanMismatchError(f"q has shape {tuple(q.shape)}; the plan needs [batch, {Hq}, {D}]")
    if len(kv_cache.shape) != 5 or tuple(kv_cache.shape[1:]) != (2, P, Hkv, D):
        raise PlanMismatchError(f"kv_cache has shape {tuple(kv_cache.shape)}; the plan needs "
                                f"[num_pages, 2, {P}, {Hkv}, {D}]")
    if kv_cache.shape[0] < 1:
        raise PlanMismatchError("kv_cache has no pages")
    rows = q.shape[0]
    if out is not None and (tuple(out.shape) != (rows, Hq, D) or out.dtype != torch.bfloat16):
        raise PlanMismatchError(f"out is {out.dtype} {tuple(out.shape)}; the run writes bf16 "
                                f"[{rows}, {Hq}, {D}]")
    if lse is not None and (tuple(lse.shape) != (rows, Hq) or lse.dtype != torch.float32):
        raise PlanMismatchError(f"lse is {lse.dtype} {tuple(lse.shape)}; the run writes float32 "
                                f"[{rows}, {Hq}]")


def check_append_args(k_new, v_new, batch_indices, positions, kv_cache, kv_indices,
                      kv_indptr) -> None:
    """Refuse an append whose tensors do not fit together (ValueError); only
    .shape / .dtype / .numel() are read.  The kernel writes token t's rows
    of num_kv_heads x head_dim values into a cache of that row size, reads
    batch_indices[t] and positions[t] for t < nnz and kv_indptr[b],
    kv_indptr[b + 1] for b < batch = len(kv_indptr) - 1."""
    import torch

    if len(k_new.shape) != 3:
        raise ValueError(f"k_new must be [nnz, num_kv_heads, head_dim], got {tuple(k_new.shape)}")
    nnz, Hkv, D = k_new.shape
    if tuple(v_new.shape) != tuple(k_new.shape):
        raise ValueError(f"v_new has shape {tuple(v_new.shape)}, k_new {tuple(k_new.shape)}")
    if k_new.dtype != torch.bfloat16 or v_new.dtype != torch.bfloat16:
        raise ValueError("k_new and v_new must be bf16")
    if len(kv_cache.shape) != 5 or kv_cache.shape[1] != 2 or tuple(kv_cache.shape[3:]) != (Hkv, D):
        raise ValueError(f"kv_cache has shape {tuple(kv_cache.shape)}; rows of [{Hkv}, {D}] need "
                         f"[num_pages, 2, page_size, {Hkv}, {D}]")
    if kv_cache.shape[0] < 1 or kv_cache.shape[2] < 1:
        raise ValueError("kv_cache has no pages")
    for name, t in (("batch_indices", batch_indices), ("positions", positions)):
        if len(t.shape) != 1 or t.shape[0] < nnz:
            raise ValueError(f"{name} must be 1-D with at least nnz = {nnz} entries, got "
                             f"{tuple(t.shape)}")
    if len(kv_indptr.shape) != 1 or kv_indptr.shape[0] < 2:
        raise ValueError("kv_indptr must be 1-D with batch + 1 >= 2 entries")
    if len(kv_indices.shape) != 1:
        raise ValueError("kv_indices must be 1-D")


def _dtype_code(dtype) -> int:
    import torch

    global _DTYPES
    if _DTYPES is None:
        _DTYPES = {torch.bfloat16: _lib.PKD_DTYPE_BF16, torch.float16: _lib.PKD_DTYPE_FP16}
        fp8 = getattr(torch, "float8_e4m3fn", None)
        if fp8 is not None:
            _DTYPES[fp8] = _lib.PKD_DTYPE_FP8_E4M3
    if dtype not in _DTYPES:
        raise ValueError(f"unsupported dtype {dtype}")
    return _DTYPES[dtype]


def _opts(fixed_chunk_pages=0, min_chunk_tokens=0, alpha=-1, beta=0, variant="auto",
          all_partials=False):
    v = _lib.VARIANTS[variant] if isinstance(variant, str) else int(variant)
    flags = _lib.PKD_PLAN_ALL_PARTIALS if all_partials else 0
    return pkd_plan_opts(int(fixed_chunk_pages), int(min_chunk_tokens), int(alpha), int(beta), v,
                         flags)


def _host_i32(x) -> np.ndarray:
    if hasattr(x, "detach"):
        x = x.detach().cpu().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.int32))


def _stream_ptr(stream) -> int:
    import torch

    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream)


def plan_host(kv_indptr, kv_last_page_len, num_qo_heads, num_kv_heads, head_dim, page_size,
              num_slots, **opts) -> dict:
    """The schedule pkd_plan would upload, computed on the host (pkd_plan_host),
    decoded into numpy arrays."""
    L = _lib.load()
    indptr = _host_i32(kv_indptr)
    last = _host_i32(kv_last_page_len)
    batch = last.shape[0]
    cap = 64 + num_slots + 1 + 8 * num_slots + 8 * (indptr[-1] + num_slots + 2 * batch) + 4 * batch + 64
    out = np.zeros(int(cap), dtype=np.int32)
    n = ctypes.c_int64(0)
    o = _opts(**opts)
    check(L.pkd_plan_host(indptr.ctypes.data, last.ctypes.data, batch, num_qo_heads, num_kv_heads,
                          head_dim, page_size, num_slots, ctypes.byref(o), out.ctypes.data,
                          out.nbytes, ctypes.byref(n)))
    img = out[: n.value]
    hdr = img[_lib.HEADER_BASE: _lib.HEADER_BASE + len(_lib.H_FIELDS)]
    f = {name: int(hdr[i]) for name, i in _lib.H.items()}
    S, I, ns = f["SLOTS"], f["ITEMS"], f["SPLIT"]
    items8 = img[f["OFF_ITEMS"]: f["OFF_ITEMS"] + 8 * I].reshape(I, 8)
    merges4 = img[f["OFF_MERGE"]: f["OFF_MERGE"] + 4 * ns].reshape(ns, 4)
    return dict(header=f, image=img,
                slot_indptr=img[f["OFF_SLOTS"]: f["OFF_SLOTS"] + S + 1].copy(),
                first_items=img[f["OFF_FIRST"]: f["OFF_FIRST"] + 8 * S].reshape(S, 8).copy(),
                items=items8[:, :5].copy(), item_lengths=items8[:, 5].copy(),
                item_pad=items8[:, 6:].copy(), merges=merges4[:, :3].copy(),
                chunk_pages=f["CHUNK_PAGES"], num_items=I, n_partials=f["PARTIALS"],
                n_split=ns)


def int_workspace_bytes(max_batch, max_nnz, num_slots) -> int:
    return int(_lib.load().pkd_int_workspace_bytes(max_batch, max_nnz, num_slots))


def float_workspace_bytes(max_batch, num_slots, num_qo_heads, head_dim) -> int:
    return int(_lib.load().pkd_float_workspace_bytes(max_batch, num_slots, num_qo_heads, head_dim))


def host_workspace_bytes(max_batch, num_slots) -> int:
    return int(_lib.load().pkd_host_workspace_bytes(max_batch, num_slots))


class DecodePlanRun:
    """One plan slot: a pkd handle plus its three workspaces.

    ``plan`` once per step (host page table, device kv_indices), ``run`` once
    per layer.  Workspaces are sized at construction for ``max_batch``,
    ``max_nnz`` and ``max_qo_heads`` and keep their addresses for the
    object's life, so a run captured in a graph replays correctly after
    later plans."""

    def __init__(self, max_batch: int, max_nnz: int, max_qo_heads: int = 64, head_dim: int = 128,
                 num_slots: int = 0, device=None):
        self._create(device, num_slots)
        S = self.num_slots
        self.max_batch, self.max_nnz = int(max_batch), int(max_nnz)
        self._allocate(int_workspace_bytes(max_batch, max_nnz, S),
                       float_workspace_bytes(max_batch, S, max_qo_heads, head_dim),
                       host_workspace_bytes(max_batch, S))

    def _create(self, device, num_slots):
        import torch

        self._L = _lib.load()
        dev = torch.device("cuda", torch.cuda.current_device() if device is None else device) \
            if not isinstance(device, torch.device) else device
        self.device = dev
        h = ctypes.c_void_p()
        check(self._L.pkd_create(ctypes.byref(h), dev.index or 0, int(num_slots)))
        self._h = h

    def _allocate(self, ib, fb, hb):
        import torch

        dev = self.device
        self.int_workspace = torch.empty(ib, dtype=torch.uint8, device=dev)
        self.float_workspace = torch.empty(fb, dtype=torch.uint8, device=dev)
        self._host_raw = torch.empty(hb + 256, dtype=torch.uint8, pin_memory=True)
        off = (-self._host_raw.data_ptr()) % 256
        self.host_workspace = self._host_raw[off: off + hb]

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value:
            self._L.pkd_destroy(h)
            self._h = None

    @property
    def num_slots(self) -> int:
        return int(self._L.pkd_num_slots(self._h))

    @property
    def plan_id(self) -> int:
        return int(self._L.pkd_plan_id(self._h))

    @property
    def planned_variant(self) -> str:
        """The decode kernel runs of the current plan launch ('dot2', 'mfma',
        'mfma_pv'; '' before any plan)."""
        v = int(self._L.pkd_planned_variant(self._h))
        return {code: name for name, code in _lib.VARIANTS.items() if name != "auto"}.get(v, "")

    @property
    def plan_shape(self):
        """The shape of the current plan (pkd_plan_shape) as a dict of
        PLAN_SHAPE_FIELDS, or None before any plan."""
        v = (ctypes.c_int32 * 8)()
        rc = self._L.pkd_plan_shape(self._h, v)
        if rc == _lib.PKD_ERR_STALE_PLAN:
            return None
        check(rc)
        return dict(zip(PLAN_SHAPE_FIELDS, (int(x) for x in v)))

    def plan(self, kv_indptr, kv_indices, kv_last_page_len, num_qo_heads: int, num_kv_heads: int,
             head_dim: int, page_size: int, q_data_type=None, kv_data_type=None,
             kv_layout: str = "NHD", stream=None, **opts):
        import torch

        q_data_type = torch.bfloat16 if q_data_type is None else q_data_type
        kv_data_type = torch.bfloat16 if kv_data_type is None else kv_data_type
        indptr = _host_i32(kv_indptr)
        last = _host_i32(kv_last_page_len)
        if not (isinstance(kv_indices, torch.Tensor) and kv_indices.is_cuda
                and kv_indices.dtype == torch.int32 and kv_indices.is_contiguous()):
            raise ValueError("kv_indices must be a contiguous int32 tensor on the GPU")
        layout = {"NHD": _lib.PKD_LAYOUT_NHD, "HND": _lib.PKD_LAYOUT_HND}[kv_layout]
        o = _opts(**opts)
        check(self._L.pkd_plan(
            self._h, indptr.ctypes.data, kv_indices.data_ptr(), last.ctypes.data, last.shape[0],
            num_qo_heads, num_kv_heads, head_dim, page_size, _dtype_code(q_data_type),
            _dtype_code(kv_data_type), layout,
            self.int_workspace.data_ptr(), self.int_workspace.numel(),
            self.float_workspace.data_ptr(), self.float_workspace.numel(),
            self.host_workspace.data_ptr(), self.host_workspace.numel(), ctypes.byref(o),
            _stream_ptr(stream)))
        self._keep = kv_indices  # the copy is queued on the stream; keep the source alive

    def run(self, q, kv_cache, out=None, lse=None, return_lse: bool = False, sm_scale=None,
            stream=None, k_scale=None, v_scale=None):
        """Decode for the planned batch; a float8_e4m3fn cache takes per-tensor
        k_scale / v_scale (pkd_run_scaled when a scale is given).  Tensors
        whose shape does not fit the plan raise PlanMismatchError before any
        launch."""
        import torch

        shape = self.plan_shape
        if shape is None:
            raise PkdError(_lib.PKD_ERR_STALE_PLAN, "run before any plan on this handle")
        check_run_args(shape, q, kv_cache, out, lse)
        for name, t in (("q", q), ("kv_cache", kv_cache), ("out", out), ("lse", lse)):
            if t is not None and not (t.is_cuda and t.is_contiguous() and t.device == q.device):
                raise ValueError(f"{name} must be a contiguous tensor on {q.device}")
        if out is None:
            out = torch.empty(tuple(q.shape), dtype=torch.bfloat16, device=q.device)
        if return_lse and lse is None:
            lse = torch.empty(tuple(q.shape[:2]), dtype=torch.float32, device=q.device)
        args = (self._h, q.data_ptr(), q.shape[0], kv_cache.data_ptr(), kv_cache.shape[0],
                _dtype_code(q.dtype), _dtype_code(kv_cache.dtype), out.data_ptr(),
                lse.data_ptr() if lse is not None else None,
                float(sm_scale) if sm_scale is not None else 0.0)
        if k_scale is None and v_scale is None:
            check(self._L.pkd_run(*args, _stream_ptr(stream)))
        else:
            check(self._L.pkd_run_scaled(*args, float(1.0 if k_scale is None else k_scale),
                                         float(1.0 if v_scale is None else v_scale),
                                         _stream_ptr(stream)))
        return (out, lse) if (return_lse or lse is not None) else out

    def read_device_error(self, stream=None) -> int:
        v = ctypes.c_int32(0)
        check(self._L.pkd_read_device_error(self._h, ctypes.byref(v), _stream_ptr(stream)))
        return int(v.value)

    def profile_enable(self, on: bool = True) -> None:
        check(self._L.pkd_profile_enable(self._h, 1 if on else 0))

    def profile_read(self):
        d, m, n = ctypes.c_double(), ctypes.c_double(), ctypes.c_int64()
        check(self._L.pkd_profile_read(self._h, ctypes.byref(d), ctypes.byref(m), ctypes.byref(n)))
        return d.value, m.value, n.value


def merge_state(o_a, lse_a, o_b, lse_b, out=None, lse_out=None, stream=None):
    """Row-wise merge of two states (bf16 o [n, H, 128], fp32 lse [n, H])."""
    import torch

    n, Hh, D = o_a.shape
    if out is None:
        out = torch.empty_like(o_a)
    if lse_out is None:
        lse_out = torch.empty_like(lse_a)
    for t in (o_a, lse_a, o_b, lse_b, out, lse_out):
        if not (t.is_cuda and t.is_contiguous()):
            raise ValueError("merge_state needs contiguous GPU tensors")
    check(_lib.load().pkd_merge_state(o_a.data_ptr(), lse_a.data_ptr(), o_b.data_ptr(),
                                      lse_b.data_ptr(), n, Hh, D, out.data_ptr(),
                                      lse_out.data_ptr(), _stream_ptr(stream)))
    return out, lse_out


def merge_states(o, lse, out=None, lse_out=None, stream=None):
    """Merge k states per row: bf16 o [n, k, H, 128], fp32 lse [n, k, H]."""
    import torch

    n, k, Hh, D = o.shape
    if out is None:
        out = torch.empty((n, Hh, D), dtype=o.dtype, device=o.device)
    if lse_out is None:
        lse_out = torch.empty((n, Hh), dtype=torch.float32, device=o.device)
    for t in (o, lse, out, lse_out):
        if not (t.is_cuda and t.is_contiguous()):
            raise ValueError("merge_states needs contiguous GPU tensors")
    check(_lib.load().pkd_merge_states(o.data_ptr(), lse.data_ptr(), n, k, Hh, D, out.data_ptr(),
                                       lse_out.data_ptr(), _stream_ptr(stream)))
    return out, lse_out


def read_stream(buf, grid: int = 1024, sink=None, stream=None):
    """Read-ceiling kernel: read every byte of the contiguous GPU tensor `buf`
    once (16-byte nontemporal loads).  Returns the uint32 sink whose XOR is
    the XOR of every 32-bit word of `buf` (a measurement aid, not part of the
    decode path)."""
    import torch

    L = _lib.load()
    if not (buf.is_cuda and buf.is_contiguous()):
        raise ValueError("buf must be a contiguous GPU tensor")
    if sink is None:
        sink = torch.empty(int(L.pkd_read_sink_words(grid)), dtype=torch.int32, device=buf.device)
    check(L.pkd_read_stream(buf.data_ptr(), buf.numel() * buf.element_size(), sink.data_ptr(),
                            grid, _stream_ptr(stream)))
    return sink


def read_pages(base, num_pages: int, page_bytes: int, page_ids, grid: int = 1024, sink=None,
               stream=None):
    """Read-ceiling kernel: read the whole page of `page_bytes` at
    base + id * page_bytes for each id of the int32 GPU tensor `page_ids`, in
    order (ids outside [0, num_pages) skipped).  Returns the uint32 sink whose
    XOR is the XOR of every 32-bit word read."""
    import torch

    L = _lib.load()
    if not (base.is_cuda and base.is_contiguous() and page_ids.is_cuda
            and page_ids.is_contiguous() and page_ids.dtype == torch.int32):
        raise ValueError("base and page_ids (int32) must be contiguous GPU tensors")
    if num_pages * page_bytes > base.numel() * base.element_size():
        raise ValueError("num_pages * page_bytes exceeds the buffer")
    if sink is None:
        sink = torch.empty(int(L.pkd_read_sink_words(grid)), dtype=torch.int32, device=base.device)
    check(L.pkd_read_pages(base.data_ptr(), int(num_pages), int(page_bytes), page_ids.data_ptr(),
                           page_ids.numel(), sink.data_ptr(), grid, _stream_ptr(stream)))
    return sink


class StaticPlanRun(DecodePlanRun):
    """A plan slot that needs no workspaces (pkd_plan_static): the plan and
    the partial states live in the library's own device array, so neither
    construction nor planning allocates device memory.  Every StaticPlanRun
    on one GPU shares that array: their plans and runs must not overlap in
    time, and a run after another object's static plan raises
    PKD_ERR_STALE_PLAN."""

    def __init__(self, num_slots: int = 0, device=None):
        self._create(device, num_slots)
        self.max_batch = self.max_nnz = None

    def plan(self, kv_indptr, kv_indices, kv_last_page_len, num_qo_heads: int, num_kv_heads: int,
             head_dim: int, page_size: int, q_data_type=None, kv_data_type=None,
             kv_layout: str = "NHD", stream=None, **opts):
        import torch

        q_data_type = torch.bfloat16 if q_data_type is None else q_data_type
        kv_data_type = torch.bfloat16 if kv_data_type is None else kv_data_type
        indptr = _host_i32(kv_indptr)
        last = _host_i32(kv_last_page_len)
        if not (isinstance(kv_indices, torch.Tensor) and kv_indices.is_cuda
                and kv_indices.dtype == torch.int32 and kv_indices.is_contiguous()):
            raise ValueError("kv_indices must be a contiguous int32 tensor on the GPU")
        layout = {"NHD": _lib.PKD_LAYOUT_NHD, "HND": _lib.PKD_LAYOUT_HND}[kv_layout]
        o = _opts(**opts)
        check(self._L.pkd_plan_static(
            self._h, indptr.ctypes.data, kv_indices.data_ptr(), last.ctypes.data, last.shape[0],
            num_qo_heads, num_kv_heads, head_dim, page_size, _dtype_code(q_data_type),
            _dtype_code(kv_data_type), layout, ctypes.byref(o), _stream_ptr(stream)))
        self._keep = kv_indices


def run_composable(prefix, suffix, q, kv_cache, out=None, lse=None, return_lse: bool = False,
                   sm_scale=None, stream=None, k_scale=None, v_scale=None):
    """The composable format in one call (pkd_run_composable): ``prefix`` a
    SharedPlanRun and ``suffix`` a DecodePlanRun, both planned with
    ``all_partials=True`` for the same requests; returns o (and lse) of every
    request over its group's prefix and its own pages.  A float8_e4m3fn
    cache takes per-tensor k_scale / v_scale (pkd_run_composable_scaled
    when a scale is given)."""
    import torch

    shapes = []
    for r in (prefix, suffix):
        shape = r.plan_shape
        if shape is None:
            raise PkdError(_lib.PKD_ERR_STALE_PLAN, "run_composable before both plans")
        check_run_args(shape, q, kv_cache, out, lse)
        shapes.append(shape)
    for name, t in (("q", q), ("kv_cache", kv_cache), ("out", out), ("lse", lse)):
        if t is not None and not (t.is_cuda and t.is_contiguous() and t.device == q.device):
            raise ValueError(f"{name} must be a contiguous tensor on {q.device}")
    if out is None:
        out = torch.empty(tuple(q.shape), dtype=torch.bfloat16, device=q.device)
    if return_lse and lse is None:
        lse = torch.empty(tuple(q.shape[:2]), dtype=torch.float32, device=q.device)
    args = (prefix._h, suffix._h, q.data_ptr(), q.shape[0], kv_cache.data_ptr(), kv_cache.shape[0],
            _dtype_code(q.dtype), _dtype_code(kv_cache.dtype), out.data_ptr(),
            lse.data_ptr() if lse is not None else None,
            float(sm_scale) if sm_scale is not None else 0.0)
    if k_scale is None and v_scale is None:
        check(_lib.load().pkd_run_composable(*args, _stream_ptr(stream)))
    else:
        check(_lib.load().pkd_run_composable_scaled(
            *args, float(1.0 if k_scale is None else k_scale),
            float(1.0 if v_scale is None else v_scale), _stream_ptr(stream)))
    return (out, lse) if (return_lse or lse is not None) else out


def plan_shared_host(qo_indptr, kv_indptr, kv_last_page_len, num_qo_heads, num_kv_heads, head_dim,
                     page_size, num_slots, **opts) -> dict:
    """The schedule pkd_plan_shared would upload (pkd_plan_shared_host),
    decoded into numpy arrays."""
    L = _lib.load()
    qo = _host_i32(qo_indptr)
    indptr = _host_i32(kv_indptr)
    last = _host_i32(kv_last_page_len)
    G = last.shape[0]
    ib, fb, hb = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    check(L.pkd_shared_workspace_bytes(G, int(qo[-1]), int(indptr[-1]), num_slots, num_qo_heads,
                                       num_kv_heads, head_dim, ctypes.byref(ib), ctypes.byref(fb),
                                       ctypes.byref(hb)))
    extra = 8 * int(indptr[-1]) * num_kv_heads * (-(-int(qo[-1]) * (num_qo_heads // num_kv_heads)
                                                   // 128))  # room for forced chunk sizes
    out = np.zeros(hb.value // 4 + extra + 64, dtype=np.int32)
    n = ctypes.c_int64(0)
    o = _opts(**opts)
    check(L.pkd_plan_shared_host(qo.ctypes.data, indptr.ctypes.data, last.ctypes.data, G,
                                 num_qo_heads, num_kv_heads, head_dim, page_size, num_slots,
                                 ctypes.byref(o), out.ctypes.data, out.nbytes, ctypes.byref(n)))
    img = out[: n.value]
    hdr = img[_lib.HEADER_BASE: _lib.HEADER_BASE + len(_lib.H_FIELDS)]
    f = {name: int(hdr[i]) for name, i in _lib.H.items()}
    S, I, ns, ng = f["SLOTS"], f["ITEMS"], f["SPLIT"], f["NUM_GROUPS"]
    return dict(header=f, image=img,
                slot_indptr=img[f["OFF_SLOTS"]: f["OFF_SLOTS"] + S + 1].copy(),
                first_items=img[f["OFF_FIRST"]: f["OFF_FIRST"] + 8 * S].reshape(S, 8).copy(),
                items=img[f["OFF_ITEMS"]: f["OFF_ITEMS"] + 8 * I].reshape(I, 8).copy(),
                merges=img[f["OFF_MERGE"]: f["OFF_MERGE"] + 4 * ns].reshape(ns, 4)[:, :3].copy(),
                groups=img[f["OFF_GROUPS"]: f["OFF_GROUPS"] + 4 * ng].reshape(ng, 4).copy(),
                chunk_pages=f["CHUNK_PAGES"], num_items=I, n_partials=f["PARTIALS"], n_split=ns)


class SharedPlanRun(DecodePlanRun):
    """A plan slot for shared-prefix (composable) plans: ``plan`` takes a
    group table ``qo_indptr`` (requests of each group) and the page table
    over groups; ``run`` then gives every request's attention state over its
    group's tokens (combine it with the request's own suffix state with
    ``merge_state``).  Workspaces are sized for ``max_groups`` groups over
    ``max_batch`` requests."""

    def __init__(self, max_groups: int, max_batch: int, max_nnz: int, num_qo_heads: int,
                 num_kv_heads: int, head_dim: int = 128, num_slots: int = 0, device=None):
        self._create(device, num_slots)
        S = self.num_slots
        self.max_batch, self.max_nnz = int(max_batch), int(max_nnz)
        ib, fb, hb = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
        check(self._L.pkd_shared_workspace_bytes(max_groups, max_batch, max_nnz, S, num_qo_heads,
                                                 num_kv_heads, head_dim, ctypes.byref(ib),
                                                 ctypes.byref(fb), ctypes.byref(hb)))
        self._allocate(ib.value, fb.value, hb.value)

    def plan(self, qo_indptr, kv_indptr, kv_indices, kv_last_page_len, num_qo_heads: int,
             num_kv_heads: int, head_dim: int, page_size: int, q_data_type=None,
             kv_data_type=None, kv_layout: str = "NHD", stream=None, **opts):
        import torch

        q_data_type = torch.bfloat16 if q_data_type is None else q_data_type
        kv_data_type = torch.bfloat16 if kv_data_type is None else kv_data_type
        qo = _host_i32(qo_indptr)
        indptr = _host_i32(kv_indptr)
        last = _host_i32(kv_last_page_len)
        if not (isinstance(kv_indices, torch.Tensor) and kv_indices.is_cuda
                and kv_indices.dtype == torch.int32 and kv_indices.is_contiguous()):
            raise ValueError("kv_indices must be a contiguous int32 tensor on the GPU")
        layout = {"NHD": _lib.PKD_LAYOUT_NHD, "HND": _lib.PKD_LAYOUT_HND}[kv_layout]
        o = _opts(**opts)
        check(self._L.pkd_plan_shared(
            self._h, qo.ctypes.data, indptr.ctypes.data, kv_indices.data_ptr(), last.ctypes.data,
            last.shape[0], num_qo_heads, num_kv_heads, head_dim, page_size,
            _dtype_code(q_data_type), _dtype_code(kv_data_type), layout,
            self.int_workspace.data_ptr(), self.int_workspace.numel(),
            self.float_workspace.data_ptr(), self.float_workspace.numel(),
            self.host_workspace.data_ptr(), self.host_workspace.numel(), ctypes.byref(o),
            _stream_ptr(stream)))
        self._keep = kv_indices


def append_positions(append_indptr, kv_indptr, kv_last_page_len, page_size, stream=None):
    """Request and sequence position of every new token (device int32
    tensors in, device int32 tensors out); see pkd_append_positions."""
    import torch

    for t in (append_indptr, kv_indptr, kv_last_page_len):
        if not (t.is_cuda and t.dtype == torch.int32 and t.is_contiguous()):
            raise ValueError("append_positions needs contiguous int32 GPU tensors")
    batch = kv_last_page_len.shape[0]
    nnz = int(append_indptr[-1].item())
    b = torch.empty(nnz, dtype=torch.int32, device=append_indptr.device)
    p = torch.empty(nnz, dtype=torch.int32, device=append_indptr.device)
    if nnz:
        check(_lib.load().pkd_append_positions(append_indptr.data_ptr(), kv_indptr.data_ptr(),
                                               kv_last_page_len.data_ptr(), batch, page_size,
                                               b.data_ptr(), p.data_ptr(), _stream_ptr(stream)))
    return b, p


def append_paged_kv_cache(k_new, v_new, batch_indices, positions, kv_cache, kv_indices, kv_indptr,
                          device_error=None, stream=None, k_scale=None, v_scale=None):
    """Write new tokens' K and V rows ([nnz, Hkv, 128] bf16 each) into the
    paged cache [pages, 2, P, Hkv, 128] in place; see pkd_append_paged_kv.
    A float8_e4m3fn cache takes the rows quantised with per-tensor scales
    (pkd_append_paged_kv_scaled when a scale is given)."""
    import torch

    check_append_args(k_new, v_new, batch_indices, positions, kv_cache, kv_indices, kv_indptr)
    nnz, Hkv, D = k_new.shape
    for t in (k_new, v_new, kv_cache):
        if not (t.is_cuda and t.is_contiguous()):
            raise ValueError("k_new, v_new and kv_cache must be contiguous GPU tensors")
    for t in (batch_indices, positions, kv_indices, kv_indptr):
        if not (t.is_cuda and t.dtype == torch.int32 and t.is_contiguous()):
            raise ValueError("index arrays must be contiguous int32 GPU tensors")
    args = (k_new.data_ptr(), v_new.data_ptr(), batch_indices.data_ptr(), positions.data_ptr(), nnz,
            kv_indptr.data_ptr(), kv_indices.data_ptr(), kv_indptr.shape[0] - 1, Hkv, D,
            kv_cache.shape[2], _dtype_code(kv_cache.dtype), _lib.PKD_LAYOUT_NHD,
            kv_cache.data_ptr(), kv_cache.shape[0])
    err = device_error.data_ptr() if device_error is not None else None
    L = _lib.load()
    if k_scale is None and v_scale is None:
        check(L.pkd_append_paged_kv(*args, err, _stream_ptr(stream)))
    else:
        check(L.pkd_append_paged_kv_scaled(
            *args, float(1.0 if k_scale is None else k_scale),
            float(1.0 if v_scale is None else v_scale), err, _stream_ptr(stream)))

