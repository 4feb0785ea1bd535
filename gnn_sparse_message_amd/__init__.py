"""gnn_sparse_message_amd -- weighted sparse message passing on AMD MI355X (gfx950).

A thin ctypes binding over ``libmp.so`` (declared in ``include/mp.h``).  Every
step of the computation runs in the library's HIP kernels; this module only
marshals arguments: it allocates outputs and graph arrays with torch (torch is
the device allocator and stream provider), passes raw pointers and sizes, and
turns status codes into exceptions.

    g  = mp_graph_build(src, dst, num_nodes)      # stable COO -> CSR + transpose, on device
    Y  = mp_spmm_fwd(g, w, X)                      # Y  = A_w X      (A_w[dst, src] += w)
    dX = mp_spmm_dx(g, w, dY)                      # dX = A_w^T dY
    dw = mp_edge_grad_dw(g, X, dY)                 # dw_e = <X[src_e], dY[dst_e]>, COO order
    dX, dw = mp_spmm_dx_edge_grad(g, w, X, dY)     # both gradients in one pass
    a, m, z = mp_edge_softmax(g, s)                # softmax of edge scores per destination
    ds, t = mp_edge_softmax_backward(g, a, da)     # its backward
    wn = mp_edge_normalize(g, MP_NORM_SYM, w)      # w / sqrt(deg_out(src) deg_in(dst))

(tinymesh "Weighted aggregation experiment": "Decision", "Edge order is
explicit".)  The library must be built (``python gnn_sparse_message_amd/_build.py``
or ``__graft_entry__.build()``); importing this package fails loudly otherwise.
"""
from __future__ import annotations

import ctypes
import os

import torch  # noqa: F401  -- loaded first so libmp.so binds to torch's HIP runtime

__all__ = [
    "Graph", "MpError", "mp_graph_build", "mp_graph_build_async", "mp_graph_finish",
    "mp_graph_build_noalloc", "STATIC_WORKSPACE_BYTES", "mp_graph_build_overlap",
    "mp_graph_build_overlap_workspace_size",
    "mp_graph_build_workspace_size", "mp_spmm_fwd",
    "mp_spmm_dx", "mp_edge_grad_dw", "mp_spmm_dx_edge_grad", "mp_spmm_fwd_heads",
    "mp_spmm_dx_heads", "mp_edge_grad_dw_heads", "mp_spmm_dx_edge_grad_heads", "mp_edge_softmax",
    "mp_edge_softmax_backward", "mp_edge_softmax_heads", "mp_edge_softmax_backward_heads",
    "mp_attention_backward", "mp_attention_backward_scores", "mp_spmm_fwd_softmax", "mp_spmm_fwd_norm", "mp_spmm_dx_norm", "mp_spmm_dx_edge_grad_norm",
    "mp_spmm_dx_edge_grad_pair", "mp_spmm_fwd_pair", "mp_spmm_split_workspace_size",
    "mp_spmm_fwd_split", "mp_spmm_dx_split", "mp_spmm_dx_edge_grad_split",
    "mp_edge_normalize", "MP_NORM_MEAN", "MP_NORM_SYM",
    "mp_status_string", "mp_version", "library_path", "mp_set_owner_overrides",
    "owner_overrides",
    "NUM_CLASSES",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libmp.so")

MP_OK = 0
MP_ERR_NULL, MP_ERR_SHAPE, MP_ERR_DTYPE, MP_ERR_DEVICE, MP_ERR_INDEX = -1, -2, -3, -4, -5
MP_ERR_ALIAS, MP_ERR_ALIGN, MP_ERR_WORKSPACE, MP_ERR_GRAPH, MP_ERR_HIP = -6, -7, -8, -9, -10
MP_ERR_INTERNAL = -11
MP_I32, MP_I64, MP_F32, MP_BF16 = 1, 2, 3, 4
MP_NORM_MEAN, MP_NORM_SYM = 1, 2
GRAPH_INFO_WORDS = 576
GRAPH_BUILT, GRAPH_ON_DEVICE = 0x6d705f6772617068, 0x6d705f6465766963
NUM_CLASSES = 33
STATIC_WORKSPACE_BYTES = 64 << 20   # MP_STATIC_WORKSPACE_BYTES

_DTYPE = {torch.int32: MP_I32, torch.int64: MP_I64, torch.float32: MP_F32,
          torch.bfloat16: MP_BF16}


class MpError(RuntimeError):
    """A non-OK status from libmp.so; ``.status`` holds the code."""

    def __init__(self, status: int, message: str):
        super().__init__(message)
        self.status = status


class MpValueError(MpError, ValueError):
    pass


class MpTypeError(MpError, TypeError):
    pass


class MpIndexError(MpError, IndexError):
    pass


_EXC = {MP_ERR_DTYPE: MpTypeError, MP_ERR_INDEX: MpIndexError, MP_ERR_NULL: MpValueError,
        MP_ERR_SHAPE: MpValueError, MP_ERR_DEVICE: MpValueError, MP_ERR_ALIAS: MpValueError,
        MP_ERR_ALIGN: MpValueError, MP_ERR_WORKSPACE: MpValueError, MP_ERR_GRAPH: MpValueError}


class _MpGraph(ctypes.Structure):
    _fields_ = [
        ("num_nodes", ctypes.c_int64), ("num_edges", ctypes.c_int64),
        ("src", ctypes.c_void_p), ("dst", ctypes.c_void_p),
        ("rowptr", ctypes.c_void_p), ("col", ctypes.c_void_p), ("edge_order", ctypes.c_void_p),
        ("rowptr_t", ctypes.c_void_p), ("col_t", ctypes.c_void_p),
        ("transpose_order", ctypes.c_void_p),
        ("row_plan", ctypes.c_void_p), ("row_plan_t", ctypes.c_void_p),
        ("info", ctypes.c_void_p),
        ("class_count", ctypes.c_int64 * NUM_CLASSES),
        ("class_count_t", ctypes.c_int64 * NUM_CLASSES),
        ("built", ctypes.c_uint64),
    ]


def _load():
    if not os.path.exists(_LIB_PATH):
        raise ImportError(
            f"{_LIB_PATH} is missing: the HIP library has not been built "
            "(run `python __graft_entry__.py` or `python gnn_sparse_message_amd/_build.py`). "
            "There is no fallback.")
    lib = ctypes.CDLL(_LIB_PATH)
    i64, i32, vp, sz = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t
    gp = ctypes.POINTER(_MpGraph)
    sigs = {
        "mp_graph_build_workspace_size": (i32, [i64, i64, ctypes.POINTER(sz)]),
        "mp_graph_build": (i32, [vp, vp, i32, i64, i64, gp, vp, sz, vp]),
        "mp_graph_build_async": (i32, [vp, vp, i32, i64, i64, gp, vp, sz, vp]),
        "mp_graph_build_overlap_workspace_size": (i32, [i64, i64, ctypes.POINTER(sz)]),
        "mp_graph_build_overlap": (i32, [vp, vp, i32, i64, i64, gp, vp, sz, vp, vp, vp]),
        "mp_graph_finish": (i32, [gp, vp]),
        "mp_graph_build_noalloc": (i32, [vp, vp, i32, i64, i64, gp, vp]),
        "mp_spmm_fwd": (i32, [gp, vp, vp, i32, i64, vp, vp]),
        "mp_spmm_dx": (i32, [gp, vp, vp, i32, i64, vp, vp]),
        "mp_edge_grad_dw": (i32, [gp, vp, vp, i32, i64, vp, vp]),
        "mp_spmm_dx_edge_grad": (i32, [gp, vp, vp, vp, i32, i64, vp, vp, vp]),
        "mp_spmm_fwd_heads": (i32, [gp, vp, i64, vp, i32, i64, vp, vp]),
        "mp_spmm_dx_heads": (i32, [gp, vp, i64, vp, i32, i64, vp, vp]),
        "mp_edge_grad_dw_heads": (i32, [gp, vp, vp, i32, i64, i64, vp, vp]),
        "mp_spmm_dx_edge_grad_heads": (i32, [gp, vp, i64, vp, vp, i32, i64, vp, vp, vp]),
        "mp_edge_softmax": (i32, [gp, vp, vp, vp, vp]),
        "mp_edge_softmax_backward": (i32, [gp, vp, vp, vp, vp, vp]),
        "mp_edge_softmax_heads": (i32, [gp, vp, i64, vp, vp, vp]),
        "mp_edge_softmax_backward_heads": (i32, [gp, vp, vp, i64, vp, vp, vp]),
        "mp_attention_backward": (i32, [gp, vp, i64, vp, vp, vp, i32, i64, vp, vp, vp, vp]),
        "mp_attention_backward_scores": (i32, [gp, vp, vp, vp, vp, vp, i32, i64, vp, vp, vp, vp]),
        "mp_spmm_fwd_norm": (i32, [gp, i32, vp, vp, i32, i64, vp, vp]),
        "mp_spmm_fwd_softmax": (i32, [gp, vp, vp, i32, i64, vp, vp, vp]),
        "mp_spmm_dx_norm": (i32, [gp, i32, vp, vp, i32, i64, vp, vp]),
        "mp_spmm_dx_edge_grad_norm": (i32, [gp, i32, vp, vp, vp, i32, i64, vp, vp, vp]),
        "mp_spmm_dx_edge_grad_pair": (i32, [gp, vp, vp, vp, i32, i64, vp, vp]),
        "mp_spmm_fwd_pair": (i32, [gp, vp, vp, i32, i64, vp, vp]),
        "mp_spmm_split_workspace_size": (i32, [gp, i64, ctypes.POINTER(sz)]),
        "mp_spmm_fwd_split": (i32, [gp, vp, vp, i32, i64, vp, vp, sz, vp]),
        "mp_spmm_dx_split": (i32, [gp, vp, vp, i32, i64, vp, vp, sz, vp]),
        "mp_spmm_dx_edge_grad_split": (i32, [gp, vp, vp, vp, i32, i64, vp, vp, vp, sz, vp]),
        "mp_edge_normalize": (i32, [gp, i32, vp, vp, vp]),
        "mp_status_string": (ctypes.c_char_p, [i32]),
        "mp_last_error_detail": (ctypes.c_char_p, []),
        "mp_version": (i32, []),
        "mp_set_owner_overrides": (i32, [i32, i32, i32]),
    }
    for name, (res, args) in sigs.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = _load()


def library_path() -> str:
    return _LIB_PATH


def mp_version() -> int:
    return int(_lib.mp_version())


def mp_status_string(status: int) -> str:
    return _lib.mp_status_string(status).decode()


def mp_set_owner_overrides(hub_min_len: int = -1, hub_apart: int = -1,
                           wave_min_len: int = -1) -> None:
    """Replace the aggregation kernels' owner sizes for every later call in this
    process (tests and tuning only; -1 restores the rule): rows of at least
    hub_min_len edges get a workgroup, of 16 waves in a launch of their own when
    hub_apart is 1 or of four waves in the main launch when 0, and rows of at
    least wave_min_len edges get one wave.  Other owners change the summation
    order, so the bits (not the tolerance) of the results."""
    _check(_lib.mp_set_owner_overrides(int(hub_min_len), int(hub_apart), int(wave_min_len)),
           "mp_set_owner_overrides")


class owner_overrides:
    """Context manager: mp_set_owner_overrides(...) inside the block, the rule
    again after it."""

    def __init__(self, hub_min_len: int = -1, hub_apart: int = -1, wave_min_len: int = -1):
        self.args = (hub_min_len, hub_apart, wave_min_len)

    def __enter__(self):
        mp_set_owner_overrides(*self.args)
        return self

    def __exit__(self, *exc):
        mp_set_owner_overrides(-1, -1, -1)
        return False


def _check(status: int, call: str):
    if status == MP_OK:
        return
    detail = _lib.mp_last_error_detail().decode()
    exc = _EXC.get(status, MpError)
    raise exc(status, f"{call}: {mp_status_string(status)} -- {detail}")


def _ptr(t) -> int:
    return 0 if t is None else int(t.data_ptr())


def _code(t) -> int:
    return _DTYPE.get(t.dtype, 0)   # 0 -> rejected by the library as MP_ERR_DTYPE


def _stream(t) -> int:
    """The current torch stream of t's GPU (0 for host tensors, which the library rejects)."""
    return int(torch.cuda.current_stream(t.device).cuda_stream) if t.is_cuda else 0


def _need_tensor(name, t):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor, got {type(t).__name__}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


class Graph:
    """The lowered topology: torch int32 device tensors plus the C descriptor.

    Arrays (names of ``include/mp.h``): src, dst, rowptr, col, edge_order,
    rowptr_t, col_t, transpose_order, row_plan, row_plan_t; class_count and
    class_count_t are host lists.  Read-only after the build.
    """

    _ARRAYS = ("src", "dst", "rowptr", "col", "edge_order", "rowptr_t", "col_t",
               "transpose_order", "row_plan", "row_plan_t")

    def __init__(self, num_nodes: int, num_edges: int, device):
        n, e = int(num_nodes), int(num_edges)
        self.num_nodes, self.num_edges, self.device = n, e, torch.device(device)
        sizes = {"src": e, "dst": e, "rowptr": n + 1, "col": e, "edge_order": e,
                 "rowptr_t": n + 1, "col_t": e, "transpose_order": e, "row_plan": n,
                 "row_plan_t": n}
        self.arrays = {k: torch.empty(max(v, 0), dtype=torch.int32, device=self.device)
                       for k, v in sizes.items()}
        # the build's device record (index check, rows per class of both plans)
        self.info = torch.empty(GRAPH_INFO_WORDS, dtype=torch.int32, device=self.device)
        d = _MpGraph()
        d.num_nodes, d.num_edges = n, e
        for k in self._ARRAYS:
            setattr(d, k, _ptr(self.arrays[k]) if self.arrays[k].numel() else None)
        d.info = _ptr(self.info)
        self._desc = d

    def __getattr__(self, name):
        arrays = self.__dict__.get("arrays")
        if arrays is not None and name in arrays:
            return arrays[name]
        raise AttributeError(name)

    @property
    def class_count(self):
        return list(self._desc.class_count)

    @property
    def class_count_t(self):
        return list(self._desc.class_count_t)

    @property
    def built(self) -> bool:
        return self._desc.built != 0

    @property
    def on_device(self) -> bool:
        """True after mp_graph_build_async until mp_graph_finish: the class counts
        exist on the device only (the compute calls read them there)."""
        return self._desc.built == GRAPH_ON_DEVICE

    def record_stream(self, stream) -> None:
        """Tell torch's allocator that `stream` uses the graph's arrays (needed
        before the Graph is dropped while work on another stream may still read it)."""
        for t in list(self.arrays.values()) + [self.info]:
            if t.numel():
                t.record_stream(stream)

    @classmethod
    def from_edge_index(cls, edge_index, num_nodes: int) -> "Graph":
        """Build from a [2, E] edge_index (row 0 = source, row 1 = target)."""
        _need_tensor("edge_index", edge_index)
        if edge_index.dim() != 2 or edge_index.shape[0] != 2:
            raise ValueError("edge_index must have shape [2, E]")
        return mp_graph_build(edge_index[0], edge_index[1], num_nodes)


def mp_graph_build_workspace_size(num_nodes: int, num_edges: int) -> int:
    out = ctypes.c_size_t(0)
    _check(_lib.mp_graph_build_workspace_size(int(num_nodes), int(num_edges), ctypes.byref(out)),
           "mp_graph_build_workspace_size")
    return int(out.value)


def _build_graph(fn, name, src, dst, num_nodes, workspace):
    _need_tensor("src", src)
    _need_tensor("dst", dst)
    if src.dim() != 1 or dst.dim() != 1 or src.shape[0] != dst.shape[0]:
        raise ValueError("src and dst must be 1-D with the same length")
    e = int(src.shape[0])
    g = Graph(num_nodes, e, src.device)
    ws_bytes = mp_graph_build_workspace_size(num_nodes, e)
    if workspace is None:
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device=src.device)
    else:
        _need_tensor("workspace", workspace)
        if workspace.dtype != torch.uint8 or workspace.numel() < ws_bytes:
            raise ValueError(f"workspace must be a uint8 tensor of at least {ws_bytes} bytes")
        ws = workspace
    status = fn(_ptr(src) if e else None, _ptr(dst) if e else None, _code(src), int(num_nodes),
                e, ctypes.byref(g._desc), _ptr(ws), ws.numel(), _stream(src))
    _check(status, name)
    return g


def mp_graph_build(src, dst, num_nodes: int, workspace=None) -> Graph:
    """Lower COO edges (src[e] -> dst[e], int32 or int64 device tensors) on device,
    on the current stream; returns once the build has run (one synchronisation)."""
    return _build_graph(_lib.mp_graph_build, "mp_graph_build", src, dst, num_nodes, workspace)


def mp_graph_build_async(src, dst, num_nodes: int, workspace=None) -> Graph:
    """The same lowering, only enqueued on the current stream (no synchronisation):
    the graph's class counts stay on the device and the compute calls read them
    there.  The index check is reported by mp_graph_finish.  Concurrent builds on
    several streams need their own workspaces (mp_graph_build_workspace_size)."""
    return _build_graph(_lib.mp_graph_build_async, "mp_graph_build_async", src, dst, num_nodes,
                  workspace)


def mp_graph_build_overlap_workspace_size(num_nodes: int, num_edges: int) -> int:
    out = ctypes.c_size_t(0)
    _check(_lib.mp_graph_build_overlap_workspace_size(int(num_nodes), int(num_edges),
                                                      ctypes.byref(out)),
           "mp_graph_build_overlap_workspace_size")
    return int(out.value)


def mp_graph_build_overlap(src, dst, num_nodes: int, side_stream, workspace=None):
    """The asynchronous lowering with the transpose direction on `side_stream`:
    the intake, the forward CSR and its plan are enqueued on the current stream,
    the transpose CSR and its plan on `side_stream` (after the intake).  Returns
    (graph, transpose_done): the forward calls may run on the current stream at
    once; calls that read the transpose CSR (mp_spmm_dx and its forms, the fused
    backward and attention backward calls) and mp_graph_finish must run after
    ``torch.cuda.current_stream().wait_event(transpose_done)``."""
    _need_tensor("src", src)
    _need_tensor("dst", dst)
    if src.dim() != 1 or dst.dim() != 1 or src.shape[0] != dst.shape[0]:
        raise ValueError("src and dst must be 1-D with the same length")
    if not isinstance(side_stream, torch.cuda.Stream):
        raise TypeError("side_stream must be a torch.cuda.Stream")
    e = int(src.shape[0])
    g = Graph(num_nodes, e, src.device)
    ws_bytes = mp_graph_build_overlap_workspace_size(num_nodes, e)
    if workspace is None:
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device=src.device)
    else:
        _need_tensor("workspace", workspace)
        if workspace.dtype != torch.uint8 or workspace.numel() < ws_bytes:
            raise ValueError(f"workspace must be a uint8 tensor of at least {ws_bytes} bytes")
        ws = workspace
    done = torch.cuda.Event()
    done.record(side_stream)          # creates the event; the call records it again
    status = _lib.mp_graph_build_overlap(_ptr(src) if e else None, _ptr(dst) if e else None,
                                         _code(src), int(num_nodes), e, ctypes.byref(g._desc),
                                         _ptr(ws), ws.numel(), _stream(src),
                                         side_stream.cuda_stream, done.cuda_event)
    _check(status, "mp_graph_build_overlap")
    # The side stream uses the inputs, the graph's arrays and the workspace.
    for t in [src, dst, ws, g.info] + [a for a in g.arrays.values() if a.numel()]:
        t.record_stream(side_stream)
    g._overlap_ws = ws
    return g, done


def mp_graph_build_noalloc(src, dst, num_nodes: int) -> Graph:
    """mp_graph_build_async with the library's static per-GPU workspace
    (MP_STATIC_WORKSPACE_BYTES) instead of a workspace argument: the C call
    allocates nothing.  This wrapper allocates only the graph's own arrays (the
    call's outputs), before the call.  Builds whose work overlaps on one GPU
    (other streams, other threads) race on that workspace."""
    _need_tensor("src", src)
    _need_tensor("dst", dst)
    if src.dim() != 1 or dst.dim() != 1 or src.shape[0] != dst.shape[0]:
        raise ValueError("src and dst must be 1-D with the same length")
    e = int(src.shape[0])
    g = Graph(num_nodes, e, src.device)
    _check(_lib.mp_graph_build_noalloc(_ptr(src) if e else None, _ptr(dst) if e else None,
                                       _code(src), int(num_nodes), e, ctypes.byref(g._desc),
                                       _stream(src)), "mp_graph_build_noalloc")
    return g


def mp_graph_finish(g: Graph, stream=None) -> Graph:
    """Wait for an asynchronous build (on `stream`, default the current one), copy
    its class counts to the host and raise IndexError if an endpoint was outside
    [0, N).  No-op for a finished graph."""
    st = torch.cuda.current_stream(g.device) if stream is None else stream
    _check(_lib.mp_graph_finish(ctypes.byref(g._desc), st.cuda_stream), "mp_graph_finish")
    return g


def _features(name, t, g: Graph):
    _need_tensor(name, t)
    if t.dim() != 2 or t.shape[0] != g.num_nodes:
        raise ValueError(f"{name} must have shape [{g.num_nodes}, H], got {tuple(t.shape)}")
    return int(t.shape[1])


def _weights(t, g: Graph):
    # The C interface takes w as float32 memory; its dtype cannot be checked there.
    _need_tensor("w", t)
    if t.dtype != torch.float32:
        raise TypeError(f"w must be float32, got {t.dtype}")
    if t.dim() != 1 or t.shape[0] != g.num_edges:
        raise ValueError(f"w must have shape [{g.num_edges}], got {tuple(t.shape)}")


def _out(out, shape, like):
    if out is None:
        return torch.empty(shape, dtype=torch.float32, device=like.device)
    _need_tensor("out", out)
    if out.dtype != torch.float32:
        raise TypeError(f"out must be float32, got {out.dtype}")
    if tuple(out.shape) != tuple(shape):
        raise ValueError(f"out must have shape {tuple(shape)}, got {tuple(out.shape)}")
    return out


def mp_spmm_fwd(g: Graph, w, x, out=None):
    """Y = A_w X, float32 [N, H]."""
    _weights(w, g)
    h = _features("x", x, g)
    y = _out(out, (g.num_nodes, h), x)
    _check(_lib.mp_spmm_fwd(ctypes.byref(g._desc), _ptr(w) if g.num_edges else None, _ptr(x),
                            _code(x), h, _ptr(y), _stream(x)), "mp_spmm_fwd")
    return y


def mp_spmm_dx(g: Graph, w, dy, out=None):
    """dX = A_w^T dY, float32 [N, H]."""
    _weights(w, g)
    h = _features("dy", dy, g)
    dx = _out(out, (g.num_nodes, h), dy)
    _check(_lib.mp_spmm_dx(ctypes.byref(g._desc), _ptr(w) if g.num_edges else None, _ptr(dy),
                           _code(dy), h, _ptr(dx), _stream(dy)), "mp_spmm_dx")
    return dx


def mp_spmm_fwd_norm(g: Graph, mode: int, w, x, out=None):
    """Y = A_{norm(w)} X with the degree normalisation (MP_NORM_MEAN or
    MP_NORM_SYM) applied as each weight is fetched; bitwise
    mp_spmm_fwd(g, mp_edge_normalize(g, mode, w), x)."""
    _weights(w, g)
    h = _features("x", x, g)
    y = _out(out, (g.num_nodes, h), x)
    _check(_lib.mp_spmm_fwd_norm(ctypes.byref(g._desc), int(mode),
                                 _ptr(w) if g.num_edges else None, _ptr(x), _code(x), h,
                                 _ptr(y), _stream(x)), "mp_spmm_fwd_norm")
    return y


def mp_spmm_dx_norm(g: Graph, mode: int, w, dy, out=None):
    """dX = A_{norm(w)}^T dY, normalised at the fetch."""
    _weights(w, g)
    h = _features("dy", dy, g)
    dx = _out(out, (g.num_nodes, h), dy)
    _check(_lib.mp_spmm_dx_norm(ctypes.byref(g._desc), int(mode),
                                _ptr(w) if g.num_edges else None, _ptr(dy), _code(dy), h,
                                _ptr(dx), _stream(dy)), "mp_spmm_dx_norm")
    return dx


def mp_spmm_dx_edge_grad_norm(g: Graph, mode: int, w, x, dy, out_dx=None, out_dw=None):
    """(dX, dw) for Y = A_{norm(w)} X: dX through the normalised weights and dw
    the gradient with respect to the raw weights, c_e <X[src_e], dY[dst_e]>."""
    _weights(w, g)
    h = _features("x", x, g)
    if _features("dy", dy, g) != h:
        raise ValueError("x and dy must have the same feature width")
    code = _code(dy) if x.dtype == dy.dtype else 0
    dx = _out(out_dx, (g.num_nodes, h), dy)
    dw = _out(out_dw, (g.num_edges,), dy)
    _check(_lib.mp_spmm_dx_edge_grad_norm(ctypes.byref(g._desc), int(mode),
                                          _ptr(w) if g.num_edges else None, _ptr(x), _ptr(dy),
                                          code, h, _ptr(dx), _ptr(dw) if g.num_edges else None,
                                          _stream(dy)), "mp_spmm_dx_edge_grad_norm")
    return dx, dw


def _pair(wg, g: Graph):
    _need_tensor("wg", wg)
    if wg.dtype != torch.float32:
        raise TypeError(f"wg must be float32, got {wg.dtype}")
    if wg.dim() != 2 or tuple(wg.shape) != (g.num_edges, 2):
        raise ValueError(f"wg must have shape [{g.num_edges}, 2], got {tuple(wg.shape)}")


def mp_spmm_fwd_pair(g: Graph, wg, x, out=None):
    """Y = A_w X with the weights in column 0 of the interleaved float32 [E, 2]
    array wg (column 1 is not read); bitwise mp_spmm_fwd(g, wg[:, 0], x)."""
    _pair(wg, g)
    h = _features("x", x, g)
    y = _out(out, (g.num_nodes, h), x)
    _check(_lib.mp_spmm_fwd_pair(ctypes.byref(g._desc), _ptr(wg) if g.num_edges else None,
                                 _ptr(x), _code(x), h, _ptr(y), _stream(x)), "mp_spmm_fwd_pair")
    return y


def mp_spmm_dx_edge_grad_pair(g: Graph, wg, x, dy, out_dx=None):
    """Fused backward with weights and gradients interleaved: wg is float32
    [E, 2], wg[:, 0] the weights (read) and wg[:, 1] receiving dw (written in
    place).  Returns dX; dw is the view wg[:, 1]."""
    _pair(wg, g)
    h = _features("x", x, g)
    if _features("dy", dy, g) != h:
        raise ValueError("x and dy must have the same feature width")
    code = _code(dy) if x.dtype == dy.dtype else 0
    dx = _out(out_dx, (g.num_nodes, h), dy)
    _check(_lib.mp_spmm_dx_edge_grad_pair(ctypes.byref(g._desc),
                                          _ptr(wg) if g.num_edges else None, _ptr(x), _ptr(dy),
                                          code, h, _ptr(dx), _stream(dy)),
           "mp_spmm_dx_edge_grad_pair")
    return dx


def mp_edge_grad_dw(g: Graph, x, dy, out=None):
    """dw_e = <X[src_e], dY[dst_e]>, float32 [E] in COO order."""
    h = _features("x", x, g)
    if _features("dy", dy, g) != h:
        raise ValueError("x and dy must have the same feature width")
    code = _code(x) if x.dtype == dy.dtype else 0
    dw = _out(out, (g.num_edges,), x)
    _check(_lib.mp_edge_grad_dw(ctypes.byref(g._desc), _ptr(x), _ptr(dy), code, h,
                                _ptr(dw) if g.num_edges else None, _stream(x)),
           "mp_edge_grad_dw")
    return dw


def mp_spmm_dx_edge_grad(g: Graph, w, x, dy, out_dx=None, out_dw=None):
    """(dX, dw) in one pass over the transpose CSR; equal to mp_spmm_dx and
    mp_edge_grad_dw."""
    _weights(w, g)
    h = _features("x", x, g)
    if _features("dy", dy, g) != h:
        raise ValueError("x and dy must have the same feature width")
    code = _code(dy) if x.dtype == dy.dtype else 0
    dx = _out(out_dx, (g.num_nodes, h), dy)
    dw = _out(out_dw, (g.num_edges,), dy)
    _check(_lib.mp_spmm_dx_edge_grad(ctypes.byref(g._desc), _ptr(w) if g.num_edges else None,
                                     _ptr(x), _ptr(dy), code, h, _ptr(dx),
                                     _ptr(dw) if g.num_edges else None, _stream(dy)),
           "mp_spmm_dx_edge_grad")
    return dx, dw


def mp_spmm_split_workspace_size(g: Graph, h: int) -> int:
    """Bytes of workspace the split calls need for this finished graph and
    feature width (0: no row is long enough to split)."""
    out = ctypes.c_size_t(0)
    _check(_lib.mp_spmm_split_workspace_size(ctypes.byref(g._desc), int(h), ctypes.byref(out)),
           "mp_spmm_split_workspace_size")
    return int(out.value)


def _split_workspace(g: Graph, h: int, workspace, like):
    need = mp_spmm_split_workspace_size(g, h)
    if workspace is None:
        return torch.empty(max(need, 1), dtype=torch.uint8, device=like.device) if need else None
    _need_tensor("workspace", workspace)
    if workspace.dtype != torch.uint8 or workspace.numel() < need:
        raise ValueError(f"workspace must be a uint8 tensor of at least {need} bytes")
    return workspace


def mp_spmm_fwd_split(g: Graph, w, x, out=None, workspace=None):
    """Y = A_w X with the longest rows split across workgroups (partial sums in
    `workspace`, a uint8 device tensor of mp_spmm_split_workspace_size bytes,
    allocated here when None)."""
    _weights(w, g)
    h = _features("x", x, g)
    y = _out(out, (g.num_nodes, h), x)
    ws = _split_workspace(g, h, workspace, x)
    _check(_lib.mp_spmm_fwd_split(ctypes.byref(g._desc), _ptr(w) if g.num_edges else None,
                                  _ptr(x), _code(x), h, _ptr(y), _ptr(ws),
                                  0 if ws is None else ws.numel(), _stream(x)),
           "mp_spmm_fwd_split")
    return y


def mp_spmm_dx_split(g: Graph, w, dy, out=None, workspace=None):
    """dX = A_w^T dY with the longest rows split (as mp_spmm_fwd_split)."""
    _weights(w, g)
    h = _features("dy", dy, g)
    dx = _out(out, (g.num_nodes, h), dy)
    ws = _split_workspace(g, h, workspace, dy)
    _check(_lib.mp_spmm_dx_split(ctypes.byref(g._desc), _ptr(w) if g.num_edges else None,
                                 _ptr(dy), _code(dy), h, _ptr(dx), _ptr(ws),
                                 0 if ws is None else ws.numel(), _stream(dy)),
           "mp_spmm_dx_split")
    return dx


def mp_spmm_dx_edge_grad_split(g: Graph, w, x, dy, out_dx=None, out_dw=None, workspace=None):
    """(dX, dw) in one pass with the longest rows split; dX bitwise
    mp_spmm_dx_split, dw bitwise mp_edge_grad_dw."""
    _weights(w, g)
    h = _features("x", x, g)
    if _features("dy", dy, g) != h:
        raise ValueError("x and dy must have the same feature width")
    code = _code(dy) if x.dtype == dy.dtype else 0
    dx = _out(out_dx, (g.num_nodes, h), dy)
    dw = _out(out_dw, (g.num_edges,), dy)
    ws = _split_workspace(g, h, workspace, dy)
    _check(_lib.mp_spmm_dx_edge_grad_split(ctypes.byref(g._desc),
                                           _ptr(w) if g.num_edges else None, _ptr(x), _ptr(dy),
                                           code, h, _ptr(dx), _ptr(dw) if g.num_edges else None,
                                           _ptr(ws), 0 if ws is None else ws.numel(),
                                           _stream(dy)),
           "mp_spmm_dx_edge_grad_split")
    return dx, dw


def _head_weights(t, g: Graph, h: int) -> int:
    """Check w as [E, K] float32 (K heads dividing the feature width h); returns K."""
    _need_tensor("w", t)
    if t.dtype != torch.float32:
        raise TypeError(f"w must be float32, got {t.dtype}")
    if t.dim() != 2 or t.shape[0] != g.num_edges:
        raise ValueError(f"w must have shape [{g.num_edges}, K], got {tuple(t.shape)}")
    k = int(t.shape[1])
    if k < 1 or h % k != 0:
        raise ValueError(f"{k} heads do not divide the feature width {h}")
    return k


def mp_spmm_fwd_heads(g: Graph, w, x, out=None):
    """Multi-head Y: w is [E, K]; head q of Y (columns q*H/K .. (q+1)*H/K - 1)
    aggregates head q of X with weights w[:, q].  float32 [N, H]."""
    h = _features("x", x, g)
    k = _head_weights(w, g, h)
    y = _out(out, (g.num_nodes, h), x)
    _check(_lib.mp_spmm_fwd_heads(ctypes.byref(g._desc), _ptr(w) if g.num_edges else None, k,
                                  _ptr(x), _code(x), h, _ptr(y), _stream(x)),
           "mp_spmm_fwd_heads")
    return y


def mp_spmm_dx_heads(g: Graph, w, dy, out=None):
    """Multi-head dX = per-head A_w^T dY, float32 [N, H]."""
    h = _features("dy", dy, g)
    k = _head_weights(w, g, h)
    dx = _out(out, (g.num_nodes, h), dy)
    _check(_lib.mp_spmm_dx_heads(ctypes.byref(g._desc), _ptr(w) if g.num_edges else None, k,
                                 _ptr(dy), _code(dy), h, _ptr(dx), _stream(dy)),
           "mp_spmm_dx_heads")
    return dx


def mp_edge_grad_dw_heads(g: Graph, x, dy, heads: int, out=None):
    """dw[e, q] = <X[src_e], dY[dst_e]> over head q's columns, float32 [E, K]."""
    h = _features("x", x, g)
    if _features("dy", dy, g) != h:
        raise ValueError("x and dy must have the same feature width")
    code = _code(x) if x.dtype == dy.dtype else 0
    dw = _out(out, (g.num_edges, int(heads)), x)
    _check(_lib.mp_edge_grad_dw_heads(ctypes.byref(g._desc), _ptr(x), _ptr(dy), code, h,
                                      int(heads), _ptr(dw) if g.num_edges else None,
                                      _stream(x)), "mp_edge_grad_dw_heads")
    return dw


def mp_spmm_dx_edge_grad_heads(g: Graph, w, x, dy, out_dx=None, out_dw=None):
    """Multi-head (dX, dw[E, K]) in one pass; equal to mp_spmm_dx_heads and
    mp_edge_grad_dw_heads."""
    h = _features("x", x, g)
    if _features("dy", dy, g) != h:
        raise ValueError("x and dy must have the same feature width")
    k = _head_weights(w, g, h)
    code = _code(dy) if x.dtype == dy.dtype else 0
    dx = _out(out_dx, (g.num_nodes, h), dy)
    dw = _out(out_dw, (g.num_edges, k), dy)
    _check(_lib.mp_spmm_dx_edge_grad_heads(ctypes.byref(g._desc),
                                           _ptr(w) if g.num_edges else None, k, _ptr(x),
                                           _ptr(dy), code, h, _ptr(dx),
                                           _ptr(dw) if g.num_edges else None, _stream(dy)),
           "mp_spmm_dx_edge_grad_heads")
    return dx, dw


def _edge_f32(name, t, g: Graph):
    _need_tensor(name, t)
    if t.dtype != torch.float32:
        raise TypeError(f"{name} must be float32, got {t.dtype}")
    if t.dim() != 1 or t.shape[0] != g.num_edges:
        raise ValueError(f"{name} must have shape [{g.num_edges}], got {tuple(t.shape)}")


def mp_edge_softmax(g: Graph, scores, out_alpha=None, out_row_stats=None):
    """Softmax of the edge scores over the incoming edges of each destination:
    returns (alpha [E] in COO order, row_stats [N, 2] holding each row's maximum
    and sum of exp(score - maximum)), all float32."""
    _edge_f32("scores", scores, g)
    alpha = _out(out_alpha, (g.num_edges,), scores)
    stats = _out(out_row_stats, (g.num_nodes, 2), scores)
    _check(_lib.mp_edge_softmax(ctypes.byref(g._desc), _ptr(scores) if g.num_edges else None,
                                _ptr(alpha) if g.num_edges else None, _ptr(stats),
                                _stream(scores)), "mp_edge_softmax")
    return alpha, stats


def mp_spmm_fwd_softmax(g: Graph, scores, x, out=None, out_row_stats=None):
    """Y = A_alpha X with alpha = softmax(scores) over each destination, alpha
    formed at the fetch and never written: returns (Y [N, H], row_stats [N, 2]),
    bitwise mp_edge_softmax followed by mp_spmm_fwd on its alpha."""
    _edge_f32("scores", scores, g)
    h = _features("x", x, g)
    y = _out(out, (g.num_nodes, h), x)
    stats = _out(out_row_stats, (g.num_nodes, 2), x)
    _check(_lib.mp_spmm_fwd_softmax(ctypes.byref(g._desc),
                                    _ptr(scores) if g.num_edges else None, _ptr(x), _code(x), h,
                                    _ptr(y), _ptr(stats), _stream(x)), "mp_spmm_fwd_softmax")
    return y, stats


def mp_edge_softmax_backward(g: Graph, alpha, dalpha, out_dscores=None, out_row_dot=None):
    """Backward of mp_edge_softmax: returns (dscores [E] COO order, row_dot [N])."""
    _edge_f32("alpha", alpha, g)
    _edge_f32("dalpha", dalpha, g)
    ds = _out(out_dscores, (g.num_edges,), alpha)
    rdot = _out(out_row_dot, (g.num_nodes,), alpha)
    _check(_lib.mp_edge_softmax_backward(ctypes.byref(g._desc),
                                         _ptr(alpha) if g.num_edges else None,
                                         _ptr(dalpha) if g.num_edges else None,
                                         _ptr(ds) if g.num_edges else None, _ptr(rdot),
                                         _stream(alpha)), "mp_edge_softmax_backward")
    return ds, rdot


def _edge_heads_f32(name, t, g: Graph) -> int:
    """Check t as [E, K] float32 (multi-head edge values); returns K."""
    _need_tensor(name, t)
    if t.dtype != torch.float32:
        raise TypeError(f"{name} must be float32, got {t.dtype}")
    if t.dim() != 2 or t.shape[0] != g.num_edges or t.shape[1] < 1:
        raise ValueError(f"{name} must have shape [{g.num_edges}, K], got {tuple(t.shape)}")
    return int(t.shape[1])


def mp_edge_softmax_heads(g: Graph, scores, out_alpha=None, out_row_stats=None):
    """Per-head softmax of scores [E, K] over each destination's edges: returns
    (alpha [E, K], row_stats [N, K, 2] = (maximum, sum)), float32."""
    k = _edge_heads_f32("scores", scores, g)
    alpha = _out(out_alpha, (g.num_edges, k), scores)
    stats = _out(out_row_stats, (g.num_nodes, k, 2), scores)
    _check(_lib.mp_edge_softmax_heads(ctypes.byref(g._desc),
                                      _ptr(scores) if g.num_edges else None, k,
                                      _ptr(alpha) if g.num_edges else None, _ptr(stats),
                                      _stream(scores)), "mp_edge_softmax_heads")
    return alpha, stats


def mp_edge_softmax_backward_heads(g: Graph, alpha, dalpha, out_dscores=None, out_row_dot=None):
    """Per-head backward: returns (dscores [E, K], row_dot [N, K])."""
    k = _edge_heads_f32("alpha", alpha, g)
    if _edge_heads_f32("dalpha", dalpha, g) != k:
        raise ValueError("alpha and dalpha must have the same number of heads")
    ds = _out(out_dscores, (g.num_edges, k), alpha)
    rdot = _out(out_row_dot, (g.num_nodes, k), alpha)
    _check(_lib.mp_edge_softmax_backward_heads(ctypes.byref(g._desc),
                                               _ptr(alpha) if g.num_edges else None,
                                               _ptr(dalpha) if g.num_edges else None, k,
                                               _ptr(ds) if g.num_edges else None, _ptr(rdot),
                                               _stream(alpha)), "mp_edge_softmax_backward_heads")
    return ds, rdot


def mp_attention_backward(g: Graph, alpha, x, dy, y, out_dx=None, out_dscores=None,
                          out_row_dot=None):
    """Backward of the attention layer Y = A_alpha X, alpha = softmax(scores):
    returns (dX [N, H], dscores shaped like alpha, row_dot [N] or [N, K]) with
    row_dot = <Y, dY> per row (and head).  alpha is [E] (one head) or [E, K];
    y is the float32 forward output for these alpha and x."""
    h = _features("x", x, g)
    if _features("dy", dy, g) != h or _features("y", y, g) != h:
        raise ValueError("x, dy and y must have the same feature width")
    if y.dtype != torch.float32:
        raise TypeError(f"y must be float32, got {y.dtype}")
    _need_tensor("alpha", alpha)
    if alpha.dim() == 1:
        _weights(alpha, g)
        k = 1
    else:
        k = _head_weights(alpha, g, h)
    code = _code(dy) if x.dtype == dy.dtype else 0
    dx = _out(out_dx, (g.num_nodes, h), dy)
    ds = _out(out_dscores, tuple(alpha.shape), dy)
    rdot = _out(out_row_dot, (g.num_nodes,) if alpha.dim() == 1 else (g.num_nodes, k), dy)
    _check(_lib.mp_attention_backward(ctypes.byref(g._desc),
                                      _ptr(alpha) if g.num_edges else None, k, _ptr(x),
                                      _ptr(dy), _ptr(y), code, h, _ptr(dx),
                                      _ptr(ds) if g.num_edges else None, _ptr(rdot),
                                      _stream(dy)), "mp_attention_backward")
    return dx, ds, rdot


def mp_attention_backward_scores(g: Graph, scores, row_stats, x, dy, y, out_dx=None,
                                 out_dscores=None, out_row_dot=None):
    """mp_attention_backward for one head with alpha formed in the walk from the
    scores [E] and the softmax row statistics [N, 2] (of mp_spmm_fwd_softmax or
    mp_edge_softmax): returns (dX, dscores [E], row_dot [N]), bitwise those of
    mp_attention_backward given alpha; out_dscores may be scores itself."""
    h = _features("x", x, g)
    if _features("dy", dy, g) != h or _features("y", y, g) != h:
        raise ValueError("x, dy and y must have the same feature width")
    if y.dtype != torch.float32:
        raise TypeError(f"y must be float32, got {y.dtype}")
    _edge_f32("scores", scores, g)
    _need_tensor("row_stats", row_stats)
    if row_stats.dtype != torch.float32 or tuple(row_stats.shape) != (g.num_nodes, 2):
        raise ValueError(f"row_stats must be float32 [{g.num_nodes}, 2]")
    code = _code(dy) if x.dtype == dy.dtype else 0
    dx = _out(out_dx, (g.num_nodes, h), dy)
    ds = _out(out_dscores, (g.num_edges,), dy)
    rdot = _out(out_row_dot, (g.num_nodes,), dy)
    _check(_lib.mp_attention_backward_scores(ctypes.byref(g._desc),
                                             _ptr(scores) if g.num_edges else None,
                                             _ptr(row_stats), _ptr(x), _ptr(dy), _ptr(y), code, h,
                                             _ptr(dx), _ptr(ds) if g.num_edges else None,
                                             _ptr(rdot), _stream(dy)),
           "mp_attention_backward_scores")
    return dx, ds, rdot


def mp_edge_normalize(g: Graph, mode: int, values, out=None):
    """values / deg_in(dst) (MP_NORM_MEAN) or / sqrt(deg_out(src) deg_in(dst))
    (MP_NORM_SYM), float32 [E] in COO order; `out` may be `values` itself."""
    _edge_f32("values", values, g)
    res = _out(out, (g.num_edges,), values)
    _check(_lib.mp_edge_normalize(ctypes.byref(g._desc), int(mode),
                                  _ptr(values) if g.num_edges else None,
                                  _ptr(res) if g.num_edges else None, _stream(values)),
           "mp_edge_normalize")
    return res
