"""Python binding of libetg: the static embedding / tied lm_head service on MI355X.

Argument marshalling only.  Every step of the path runs in the HIP kernels of
``libetg.so`` (built in-tree by ``embedding_table_gather_amd/build.py``);
PyTorch supplies device memory and the current stream.  There is no CPU
fallback: if the library is missing, every call raises.

    t = Table(rows, BF16, vocab, hidden)          # rows: device tensor, borrowed
    x = t.embed_gather(ids)                       # ADR-0008 "POST /v1/embed"
    ids, scores = t.logits_topk(residual, k=10)   # ADR-0008 "POST /v1/logits"
    ids, scores, probs = t.logits_topk_probs(residual, k=10, temperature=1.0)
    logits = t.logits_raw(residual)               # raw logits mode, [B, vocab]
    rows = t.embed_gather_wire(ids, WIRE_I8)      # ADR-0009 wire rows (f16 or i8)
    ids, scores = t.logits_topk_wire(rows, WIRE_I8, k=10)
"""
from __future__ import annotations

import ctypes
import os

import torch

F32, BF16, Q8_0, F16 = 0, 1, 2, 3
WIRE_F32, WIRE_F16, WIRE_I8 = 0, 1, 2
PATH_AUTO, PATH_VALU, PATH_STREAM, PATH_GEMM, PATH_WIDE, PATH_Q8, PATH_ROW, PATH_RANK = 0, 1, 2, 3, 4, 5, 6, 7

# ETG_LIBRARY names another build of the same library (e.g. one whose host code
# carries sanitizers); by default the in-tree libetg.so
LIB_PATH = os.environ.get("ETG_LIBRARY") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libetg.so")

_STATUS = {
    0: "ETG_OK", -1: "ETG_EINVAL", -2: "ETG_EDTYPE", -3: "ETG_ESHAPE", -4: "ETG_EALIGN",
    -5: "ETG_ERANGE", -6: "ETG_EWORKSPACE", -8: "ETG_EHIP",
}

# Functions declared in include/etg.h, with their ctypes signatures.
_I32, _I64, _VP, _F = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p, ctypes.c_float
SIGNATURES = {
    "etg_version": (_I32, []),
    "etg_row_bytes": (_I64, [_I32, _I64]),
    "etg_sqrt_d": (_F, [_I64]),
    "etg_table_create": (_I32, [_VP, _I32, _I64, _I64, ctypes.POINTER(_VP)]),
    "etg_table_destroy": (_I32, [_VP]),
    "etg_embed_gather": (_I32, [_VP, _VP, _I64, _F, _VP, _VP, _VP]),
    "etg_logits_topk_workspace": (_I64, [_VP, _I64, _I32]),
    "etg_logits_topk_workspace_ex": (_I64, [_VP, _I64, _I32, _I32]),
    "etg_logits_topk": (_I32, [_VP, _VP, _I64, _I32, _VP, _VP, _VP, ctypes.c_size_t, _VP]),
    "etg_logits_topk_ex": (_I32, [_VP, _VP, _I64, _I32, _VP, _VP, _VP, ctypes.c_size_t, _I32, _VP]),
    "etg_logits_topk_profiled": (_I32, [_VP, _VP, _I64, _I32, _VP, _VP, _VP, ctypes.c_size_t, _I32, _VP, _VP,
                                        _VP]),
    "etg_logits_topk_probs": (_I32, [_VP, _VP, _I64, _I32, _F, _VP, _VP, _VP, _VP, ctypes.c_size_t, _I32, _VP]),
    "etg_logits_raw_workspace": (_I64, [_VP, _I64, _I32]),
    "etg_logits_raw": (_I32, [_VP, _VP, _I64, _VP, _VP, ctypes.c_size_t, _I32, _VP]),
    "etg_wire_row_bytes": (_I64, [_I32, _I64]),
    "etg_embed_gather_wire": (_I32, [_VP, _VP, _I64, _F, _I32, _VP, _VP, _VP]),
    "etg_logits_topk_wire": (_I32, [_VP, _VP, _I32, _I64, _I32, _VP, _VP, _VP, ctypes.c_size_t, _I32, _VP]),
    "etg_logits_topk_to_host": (_I32, [_VP, _VP, _I64, _I32, _VP, _VP, _VP, ctypes.c_size_t, _I32, _VP, _VP, _VP,
                                       _VP]),
    "etg_hbm_read_probe": (_I32, [_VP, _I64, _VP, _VP]),
    "etg_hbm_write_probe": (_I32, [_VP, _I64, ctypes.c_uint32, _VP]),
    "etg_logits_topk_noalloc": (_I32, [_VP, _VP, _I64, _I32, _VP, _VP, _VP]),
    "etg_step_cache_ids_capacity": (_I64, [_I64]),
    "etg_step_cache_workspace": (_I64, [_VP, _I64, _I32]),
    "etg_step_cache_create": (_I32, [_VP, _I64, _I64, _I32, _I32, _VP, _VP, _VP, _VP, _VP, _VP, ctypes.c_size_t, _VP,
                                     _VP, _VP, ctypes.POINTER(_VP)]),
    "etg_step_cache_destroy": (_I32, [_VP]),
    "etg_step_cache_stats": (_I32, [_VP, ctypes.POINTER(_I64), ctypes.POINTER(_I64)]),
    "etg_step_gather": (_I32, [_VP, _VP, _I64, _F, _VP]),
    "etg_step_logits": (_I32, [_VP, _I64, _VP, _VP]),
    "etg_last_error": (ctypes.c_char_p, []),
}

_lib = None


class EtgError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_STATUS.get(status, status)}: {message}")
        self.status = status


def lib() -> ctypes.CDLL:
    """Load libetg.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with embedding_table_gather_amd/build.py "
                               "(there is no fallback path)")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _check(status: int) -> None:
    if status != 0:
        raise EtgError(status, lib().etg_last_error().decode())


def row_bytes(dtype: int, hidden: int) -> int:
    return int(lib().etg_row_bytes(int(dtype), int(hidden)))


def sqrt_d(hidden: int) -> float:
    return float(lib().etg_sqrt_d(int(hidden)))


def _stream_ptr(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _ptr(t: torch.Tensor):
    return ctypes.c_void_p(t.data_ptr())


def _event_handle(ev, device: torch.device) -> int:
    """The hipEvent_t behind a torch event (created on first record), or a raw
    hipEvent_t handle passed as an int."""
    if isinstance(ev, int):
        return ev
    if ev.cuda_event == 0:
        ev.record(torch.cuda.current_stream(device))
    return ev.cuda_event


class Table:
    """A V x hidden table already in device memory (f32, bf16, f16 or Q8_0 rows).

    ``rows`` is any contiguous CUDA tensor holding exactly vocab * row_bytes bytes
    (e.g. uint16 [V, d] bf16 or f16 bits, float32 [V, d], uint8 [V, 34 d / 32]).  It is
    borrowed: the handle keeps a reference but never copies it.
    """

    def __init__(self, rows: torch.Tensor, dtype: int, vocab: int, hidden: int):
        if not rows.is_cuda:
            raise ValueError("table rows must be a device tensor")
        if not rows.is_contiguous():
            raise ValueError("table rows must be contiguous")
        rb = row_bytes(dtype, hidden)
        if rb < 0:
            raise ValueError(f"hidden {hidden} cannot be stored as dtype {dtype}")
        nbytes = rows.numel() * rows.element_size()
        if nbytes != vocab * rb:
            raise ValueError(f"rows hold {nbytes} bytes, expected {vocab} * {rb}")
        self.rows, self.dtype, self.vocab, self.hidden, self.row_bytes = rows, int(dtype), int(vocab), int(hidden), rb
        self.device = rows.device
        h = ctypes.c_void_p()
        _check(lib().etg_table_create(_ptr(rows), self.dtype, self.vocab, self.hidden, ctypes.byref(h)))
        self._h = h
        self._ws = {}

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and _lib is not None:
            _lib.etg_table_destroy(h)
            self._h = None

    @property
    def handle(self):
        return self._h

    # ------------------------------------------------------------------ gather
    def embed_gather(self, ids: torch.Tensor, scale=None, out: torch.Tensor | None = None,
                     bad_count: torch.Tensor | None = None, check: bool = True) -> torch.Tensor:
        """f32 [n, hidden] rows for int32 ids (ADR-0008 "POST /v1/embed").

        scale: None (no scale), "sqrt_d" (the f32 nearest sqrt(hidden)), or a number.
        check: count bad ids on the device, synchronize, and raise ValueError if
        any; with check=False nothing waits (bad rows are still zero-filled, and
        counted into ``bad_count`` if one is given).
        """
        if ids.dtype != torch.int32 or ids.device != self.device:
            raise ValueError("ids must be an int32 tensor on the table's device")
        ids = ids.contiguous().view(-1)
        n = ids.numel()
        sc = 1.0 if scale is None else (sqrt_d(self.hidden) if scale == "sqrt_d" else float(scale))
        if out is None:
            out = torch.empty((n, self.hidden), dtype=torch.float32, device=self.device)
        elif out.dtype != torch.float32 or not out.is_contiguous() or out.numel() != n * self.hidden:
            raise ValueError("out must be a contiguous float32 tensor of n * hidden values")
        if check and bad_count is None:
            bad_count = torch.zeros(1, dtype=torch.int32, device=self.device)
        bad_ptr = _ptr(bad_count) if bad_count is not None else None
        with torch.cuda.device(self.device):
            _check(lib().etg_embed_gather(self._h, _ptr(ids), n, sc, _ptr(out), bad_ptr,
                                          _stream_ptr(self.device)))
            if check:
                nbad = int(bad_count.item())
                if nbad:
                    raise ValueError(f"bad token id: {nbad} of {n} ids are not in [0, {self.vocab})")
        return out

    def embed_gather_wire(self, ids: torch.Tensor, wire: int, scale=None, out: torch.Tensor | None = None,
                          bad_count: torch.Tensor | None = None) -> torch.Tensor:
        """Rows encoded in a residual wire format: uint8 [n, wire_row_bytes(wire, hidden)]
        (ADR-0009: f16, or per-position [scale][zero point][int8 x hidden]).  No check
        of bad ids beyond counting them into ``bad_count`` if one is given."""
        if ids.dtype != torch.int32 or ids.device != self.device:
            raise ValueError("ids must be an int32 tensor on the table's device")
        ids = ids.contiguous().view(-1)
        n = ids.numel()
        rb = wire_row_bytes(wire, self.hidden)
        sc = 1.0 if scale is None else (sqrt_d(self.hidden) if scale == "sqrt_d" else float(scale))
        if out is None:
            out = torch.empty((n, rb), dtype=torch.uint8, device=self.device)
        elif out.numel() * out.element_size() != n * rb or not out.is_contiguous():
            raise ValueError("out must be a contiguous buffer of n * wire_row_bytes bytes")
        bad_ptr = _ptr(bad_count) if bad_count is not None else None
        with torch.cuda.device(self.device):
            _check(lib().etg_embed_gather_wire(self._h, _ptr(ids), n, sc, int(wire), _ptr(out), bad_ptr,
                                               _stream_ptr(self.device)))
        return out

    # ------------------------------------------------------------------ logits
    def workspace_bytes(self, batch: int, k: int, path: int = PATH_AUTO) -> int:
        n = int(lib().etg_logits_topk_workspace_ex(self._h, int(batch), int(k), int(path)))
        if n < 0:
            _check(n)
        return n

    def workspace(self, batch: int, k: int, path: int = PATH_AUTO) -> torch.Tensor:
        """A device workspace for this shape, cached per (shape, path, current stream).

        Calls on one stream run in order, so they can share a workspace; calls on
        different streams get different ones.  Threads that enqueue on the same
        stream concurrently must pass their own ``workspace``."""
        key = (int(batch), int(k), int(path), torch.cuda.current_stream(self.device).cuda_stream)
        ws = self._ws.get(key)
        if ws is None:
            ws = torch.empty(max(self.workspace_bytes(batch, k, path), 256), dtype=torch.uint8, device=self.device)
            self._ws[key] = ws
        return ws

    def logits_topk(self, residual: torch.Tensor, k: int, path: int = PATH_AUTO,
                    workspace: torch.Tensor | None = None, out_ids: torch.Tensor | None = None,
                    out_scores: torch.Tensor | None = None, events=None):
        """Top-k (ids int32 [B, k], logits f32 [B, k]) of residual @ table.T per row.

        events: optional (before, after) torch.cuda.Event pair, recorded around the
        kernel that streams the table (for timing that kernel alone).
        """
        if residual.dtype != torch.float32 or residual.device != self.device:
            raise ValueError("residual must be a float32 tensor on the table's device")
        R = residual.contiguous().view(-1, self.hidden)
        B = R.shape[0]
        if workspace is None:
            workspace = self.workspace(B, k, path)
        if out_ids is None:
            out_ids = torch.empty((B, k), dtype=torch.int32, device=self.device)
        if out_scores is None:
            out_scores = torch.empty((B, k), dtype=torch.float32, device=self.device)
        ev0 = ev1 = None
        if events is not None:
            ev0, ev1 = (ctypes.c_void_p(_event_handle(e, self.device)) for e in events)
        with torch.cuda.device(self.device):
            _check(lib().etg_logits_topk_profiled(self._h, _ptr(R), B, int(k), _ptr(out_ids), _ptr(out_scores),
                                                  _ptr(workspace), workspace.numel(), int(path), ev0, ev1,
                                                  _stream_ptr(self.device)))
        return out_ids, out_scores

    def logits_topk_noalloc(self, residual: torch.Tensor, k: int, out_ids: torch.Tensor,
                            out_scores: torch.Tensor):
        """logits_topk with the library's own device scratch as the workspace (for
        callers that cannot allocate): writes into the given int32 / float32 [B, k]
        device tensors and allocates nothing.  Calls that overlap on one GPU race."""
        R = self._residual(residual)
        B = R.shape[0]
        for o, dt in ((out_ids, torch.int32), (out_scores, torch.float32)):
            if o.dtype != dt or o.device != self.device or not o.is_contiguous() or o.numel() != B * k:
                raise ValueError("out_ids / out_scores must be contiguous int32 / float32 [B, k] device tensors")
        with torch.cuda.device(self.device):
            _check(lib().etg_logits_topk_noalloc(self._h, _ptr(R), B, int(k), _ptr(out_ids), _ptr(out_scores),
                                                 _stream_ptr(self.device)))
        return out_ids, out_scores

    def logits_topk_to_host(self, residual: torch.Tensor, k: int, path: int = PATH_AUTO,
                            workspace: torch.Tensor | None = None, host_out=None):
        """logits_topk whose answer is also copied, without a synchronisation, into
        page-locked host tensors (host_out: a reusable (int32, float32) pair of
        [B, k] pinned CPU tensors, else new ones).  Returns (host ids, host scores,
        event): the host tensors hold the answer once event.synchronize() (or a true
        event.query())."""
        R = self._residual(residual)
        B = R.shape[0]
        if workspace is None:
            workspace = self.workspace(B, k, path)
        ids = torch.empty((B, k), dtype=torch.int32, device=self.device)
        sc = torch.empty((B, k), dtype=torch.float32, device=self.device)
        if host_out is None:
            host_out = (torch.empty((B, k), dtype=torch.int32, pin_memory=True),
                        torch.empty((B, k), dtype=torch.float32, pin_memory=True))
        h_ids, h_sc = host_out
        if (h_ids.dtype != torch.int32 or h_sc.dtype != torch.float32 or h_ids.device.type != "cpu"
                or h_sc.device.type != "cpu" or h_ids.numel() < B * k or h_sc.numel() < B * k
                or not h_ids.is_contiguous() or not h_sc.is_contiguous()):
            raise ValueError("host_out must be contiguous CPU int32 / float32 tensors of at least B * k entries")
        ev = torch.cuda.Event()
        with torch.cuda.device(self.device):
            evh = ctypes.c_void_p(_event_handle(ev, self.device))
            _check(lib().etg_logits_topk_to_host(self._h, _ptr(R), B, int(k), _ptr(ids), _ptr(sc), _ptr(workspace),
                                                 workspace.numel(), int(path), _ptr(h_ids), _ptr(h_sc), evh,
                                                 _stream_ptr(self.device)))
        return h_ids, h_sc, ev

    def _residual(self, residual: torch.Tensor) -> torch.Tensor:
        if residual.dtype != torch.float32 or residual.device != self.device:
            raise ValueError("residual must be a float32 tensor on the table's device")
        return residual.contiguous().view(-1, self.hidden)

    def logits_topk_probs(self, residual: torch.Tensor, k: int, temperature: float = 1.0,
                          path: int = PATH_AUTO, workspace: torch.Tensor | None = None):
        """Top-k (ids int32 [B, k], logits f32 [B, k], probabilities f32 [B, k]); the
        probabilities are the softmax of logits / temperature over the whole vocabulary."""
        R = self._residual(residual)
        B = R.shape[0]
        if workspace is None:
            workspace = self.workspace(B, k, path)
        ids = torch.empty((B, k), dtype=torch.int32, device=self.device)
        scores = torch.empty((B, k), dtype=torch.float32, device=self.device)
        probs = torch.empty((B, k), dtype=torch.float32, device=self.device)
        with torch.cuda.device(self.device):
            _check(lib().etg_logits_topk_probs(self._h, _ptr(R), B, int(k), float(temperature), _ptr(ids),
                                               _ptr(scores), _ptr(probs), _ptr(workspace), workspace.numel(),
                                               int(path), _stream_ptr(self.device)))
        return ids, scores, probs

    def logits_topk_wire(self, residual: torch.Tensor, wire: int, k: int, path: int = PATH_AUTO,
                         workspace: torch.Tensor | None = None):
        """Top-k (ids, logits) of residual rows given in a wire format: a contiguous
        device buffer of batch * wire_row_bytes(wire, hidden) bytes."""
        rb = wire_row_bytes(wire, self.hidden)
        nbytes = residual.numel() * residual.element_size()
        if residual.device != self.device or not residual.is_contiguous() or nbytes % rb:
            raise ValueError("residual must be a contiguous device buffer of whole wire rows")
        B = nbytes // rb
        if workspace is None:
            workspace = self.workspace(B, k, path)
        ids = torch.empty((B, k), dtype=torch.int32, device=self.device)
        scores = torch.empty((B, k), dtype=torch.float32, device=self.device)
        with torch.cuda.device(self.device):
            _check(lib().etg_logits_topk_wire(self._h, _ptr(residual), int(wire), B, int(k), _ptr(ids), _ptr(scores),
                                              _ptr(workspace), workspace.numel(), int(path),
                                              _stream_ptr(self.device)))
        return ids, scores

    def logits_raw(self, residual: torch.Tensor, path: int = PATH_AUTO, out: torch.Tensor | None = None,
                   workspace: torch.Tensor | None = None) -> torch.Tensor:
        """Raw logits mode: f32 [B, vocab] = residual @ table.T."""
        R = self._residual(residual)
        B = R.shape[0]
        if workspace is None:
            n = int(lib().etg_logits_raw_workspace(self._h, B, int(path)))
            if n < 0:
                _check(n)
            workspace = torch.empty(max(n, 256), dtype=torch.uint8, device=self.device)
        if out is None:
            out = torch.empty((B, self.vocab), dtype=torch.float32, device=self.device)
        elif out.dtype != torch.float32 or out.device != self.device or out.shape != (B, self.vocab) \
                or not out.is_contiguous():
            raise ValueError("out must be a contiguous float32 [batch, vocab] tensor on the table's device")
        with torch.cuda.device(self.device):
            _check(lib().etg_logits_raw(self._h, _ptr(R), B, _ptr(out), _ptr(workspace), workspace.numel(),
                                        int(path), _stream_ptr(self.device)))
        return out


class StepCache:
    """Embed and logits calls for small repeated shapes from host ids to a host
    answer: the kernels read the ids from, and write the top-k answer to, mapped
    page-locked memory (no copy operations), the answer tracked by an event.  With
    use_graphs=True each configuration (token counts bucketed to multiples of 64 or
    256) is captured into a HIP graph on its second hit and replayed after; on this
    platform a graph launch measured slower than the two to four kernel launches it
    replaces, so calls run eagerly by default.

    Owns its buffers as tensors and lends them to the library:
      rows      device f32 [ids capacity, hidden]: the gathered rows
      residual  device f32 [max_batch, hidden]: write the residual rows here
      ids, scores  page-locked CPU [max_batch, k]: the answer after event.synchronize()
    """

    STEP_ID_SLOTS = 4  # ETG_STEP_ID_SLOTS

    def __init__(self, table: Table, max_ids: int, max_batch: int, k: int, use_graphs: bool = False):
        L = lib()
        self.table, self.k, self.max_ids, self.max_batch = table, int(k), int(max_ids), int(max_batch)
        dev = table.device
        cap = int(L.etg_step_cache_ids_capacity(int(max_ids)))
        if cap < 0:
            raise ValueError(f"max_ids {max_ids} out of range")
        ws = int(L.etg_step_cache_workspace(table.handle, int(max_batch), int(k)))
        if ws < 0:
            _check(ws)
        self.d_ids = torch.zeros(cap, dtype=torch.int32, device=dev)
        self.rows = torch.empty((cap, table.hidden), dtype=torch.float32, device=dev)
        self.residual = torch.zeros((int(max_batch), table.hidden), dtype=torch.float32, device=dev)
        self.d_topk_ids = torch.empty((int(max_batch), int(k)), dtype=torch.int32, device=dev)
        self.d_topk_scores = torch.empty((int(max_batch), int(k)), dtype=torch.float32, device=dev)
        self.workspace = torch.empty(max(ws, 256), dtype=torch.uint8, device=dev)
        self.h_ids = torch.zeros((self.STEP_ID_SLOTS, cap), dtype=torch.int32, pin_memory=True)
        self.ids = torch.zeros((int(max_batch), int(k)), dtype=torch.int32, pin_memory=True)
        self.scores = torch.zeros((int(max_batch), int(k)), dtype=torch.float32, pin_memory=True)
        h = ctypes.c_void_p()
        _check(L.etg_step_cache_create(table.handle, int(max_ids), int(max_batch), int(k), int(bool(use_graphs)),
                                       _ptr(self.d_ids),
                                       _ptr(self.rows), _ptr(self.residual), _ptr(self.d_topk_ids),
                                       _ptr(self.d_topk_scores), _ptr(self.workspace), self.workspace.numel(),
                                       _ptr(self.h_ids), _ptr(self.ids), _ptr(self.scores), ctypes.byref(h)))
        self._h = h

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and _lib is not None:
            _lib.etg_step_cache_destroy(h)
            self._h = None

    def gather(self, ids, scale=None) -> torch.Tensor:
        """Rows for host int32 ids (a CPU tensor or array of n ids): a view of the
        first n rows of ``rows``, filled in stream order."""
        import numpy as np
        a = np.ascontiguousarray(ids.numpy() if isinstance(ids, torch.Tensor) else ids, dtype=np.int32).reshape(-1)
        sc = 1.0 if scale is None else (sqrt_d(self.table.hidden) if scale == "sqrt_d" else float(scale))
        with torch.cuda.device(self.table.device):
            _check(lib().etg_step_gather(self._h, a.ctypes.data_as(ctypes.c_void_p), a.size, sc,
                                         _stream_ptr(self.table.device)))
        return self.rows[:a.size]

    def logits(self, batch: int, event=None):
        """Top-k of residual rows [0, batch) into the page-locked ``ids`` / ``scores``;
        returns the event recorded after the copy (wait on it before reading)."""
        ev = event if event is not None else torch.cuda.Event()
        with torch.cuda.device(self.table.device):
            evh = ctypes.c_void_p(_event_handle(ev, self.table.device))
            _check(lib().etg_step_logits(self._h, int(batch), evh, _stream_ptr(self.table.device)))
        return ev

    def stats(self):
        g, r = ctypes.c_int64(), ctypes.c_int64()
        _check(lib().etg_step_cache_stats(self._h, ctypes.byref(g), ctypes.byref(r)))
        return g.value, r.value


def hbm_read_probe(t: torch.Tensor, sink: torch.Tensor | None = None) -> None:
    """Enqueue a plain read stream of the bytes of a contiguous device tensor (a
    multiple of 16 bytes) on the current stream: the measured HBM read reference."""
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError("a contiguous device tensor is required")
    if sink is None:
        sink = torch.empty(1, dtype=torch.int32, device=t.device)
    _check(lib().etg_hbm_read_probe(t.data_ptr(), t.numel() * t.element_size(), sink.data_ptr(),
                                    torch.cuda.current_stream(t.device).cuda_stream))


def hbm_write_probe(t: torch.Tensor, value: int = 0) -> None:
    """Enqueue a plain write stream over the bytes of a contiguous device tensor (a
    multiple of 16 bytes), every 32-bit word set to `value`, on the current stream:
    the measured HBM write reference."""
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError("a contiguous device tensor is required")
    _check(lib().etg_hbm_write_probe(t.data_ptr(), t.numel() * t.element_size(), int(value) & 0xFFFFFFFF,
                                     torch.cuda.current_stream(t.device).cuda_stream))


def wire_row_bytes(wire: int, hidden: int) -> int:
    n = int(lib().etg_wire_row_bytes(int(wire), int(hidden)))
    if n < 0:
        raise ValueError(f"unknown wire format {wire} or hidden {hidden}")
    return n


def embed_gather(table: Table, ids: torch.Tensor, scale=None, **kw) -> torch.Tensor:
    return table.embed_gather(ids, scale=scale, **kw)


def logits_topk(table: Table, residual: torch.Tensor, k: int, **kw):
    return table.logits_topk(residual, k, **kw)
