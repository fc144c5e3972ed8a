"""ctypes binding of libcgtp (include/cgtp.h): argument marshalling only.

Every computation runs in the HIP kernels of libcgtp.so; this module checks
tensor shapes/dtypes/devices, allocates outputs with torch when the caller
does not pass them, and forwards raw device pointers and the current HIP
stream. Importing it fails loudly when the library has not been built.
"""

import ctypes
import os

import numpy as np

_LIB_PATH = os.environ.get("CGTP_LIBRARY") or os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                                           "libcgtp.so")
if not os.path.exists(_LIB_PATH):
    raise ImportError("libcgtp.so is not built: run `python -m clebsch_gordan_tensor_amd.build` "
                      "(or __graft_entry__.build())")
_lib = ctypes.CDLL(_LIB_PATH)

F32, F64, BF16 = 0, 1, 2
W_SHARED, W_PER_ROW = 0, 1
OP_TP_BACKWARD, OP_CONV_BACKWARD, OP_TP_DOUBLE_BACKWARD, OP_CONV_DOUBLE_BACKWARD, OP_CONV_FORWARD = 1, 2, 3, 4, 5
LMAX = 4

_c_i64 = ctypes.c_int64
_c_i32p = ctypes.POINTER(ctypes.c_int32)
_c_i64p = ctypes.POINTER(ctypes.c_int64)
_vp = ctypes.c_void_p

# name -> argument types (restype is cgtp_status = int unless stated)
_SIGS = {
    "cgtp_status_string": ([ctypes.c_int], ctypes.c_char_p),
    "cgtp_last_error": ([], ctypes.c_char_p),
    "cgtp_plan_create": ([ctypes.c_char_p, ctypes.c_char_p, ctypes.c_char_p, ctypes.c_char_p,
                          ctypes.c_int, ctypes.c_int, ctypes.POINTER(_vp)], ctypes.c_int),
    "cgtp_plan_destroy": ([_vp], ctypes.c_int),
    "cgtp_plan_query": ([_vp, _c_i64p, _c_i64p, _c_i64p, _c_i64p, _c_i64p], ctypes.c_int),
    "cgtp_plan_paths": ([_vp, _c_i32p], ctypes.c_int),
    "cgtp_plan_create_ex": ([ctypes.c_char_p, ctypes.c_char_p, ctypes.c_char_p, ctypes.c_char_p,
                             ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.POINTER(_vp)], ctypes.c_int),
    "cgtp_plan_outputs": ([_vp, ctypes.POINTER(ctypes.c_int64), _c_i32p], ctypes.c_int),
    "cgtp_plan_cg": ([_vp, ctypes.c_int32, ctypes.POINTER(ctypes.c_double)], ctypes.c_int),
    "cgtp_tp_forward": ([_vp, _c_i64, _vp, _vp, _vp, _vp, _vp], ctypes.c_int),
    "cgtp_tp_backward": ([_vp, _c_i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp],
                         ctypes.c_int),
    "cgtp_tp_backward_noalloc": ([_vp, _c_i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp], ctypes.c_int),
    "cgtp_csr_from_coo": ([_c_i64, _c_i64, _vp, _vp, _vp, _vp, _vp, _vp], ctypes.c_int),
    "cgtp_graph_create": ([_c_i64, _c_i64, _vp, _vp, _vp, ctypes.POINTER(_vp)], ctypes.c_int),
    "cgtp_graph_destroy": ([_vp], ctypes.c_int),
    "cgtp_graph_transpose": ([_vp, _vp, _vp, _vp], ctypes.c_int),
    "cgtp_conv_forward": ([_vp, _vp, _vp, _vp, _vp, ctypes.c_double, _vp, _vp], ctypes.c_int),
    "cgtp_conv_forward_ws": ([_vp, _vp, _vp, _vp, _vp, ctypes.c_double, _vp, _vp, ctypes.c_size_t, _vp],
                             ctypes.c_int),
    "cgtp_tp_double_backward": ([_vp, _c_i64] + [_vp] * 12 + [ctypes.c_size_t, _vp], ctypes.c_int),
    "cgtp_conv_double_backward": ([_vp, _vp, _vp, _vp, _vp, ctypes.c_double] + [_vp] * 9 + [ctypes.c_size_t, _vp],
                                  ctypes.c_int),
    "cgtp_graph_create_ex": ([_c_i64, _c_i64, _vp, _vp, ctypes.c_int32, _vp, ctypes.POINTER(_vp)], ctypes.c_int),
    "cgtp_conv_backward": ([_vp, _vp, _vp, _vp, _vp, ctypes.c_double, _vp, _vp, _vp, _vp, _vp,
                            ctypes.c_size_t, _vp], ctypes.c_int),
    "cgtp_conv_forward_radial": ([_vp, _vp, _vp, _vp, _vp, _c_i64, _vp, ctypes.c_double, _vp, _vp], ctypes.c_int),
    "cgtp_conv_backward_radial": ([_vp, _vp, _vp, _vp, _vp, _c_i64, _vp, ctypes.c_double, _vp, _vp, _vp, _vp, _vp,
                                   _vp, ctypes.c_size_t, _vp], ctypes.c_int),
    "cgtp_conv_radial_workspace_size": ([_vp, _vp, _c_i64, ctypes.POINTER(ctypes.c_size_t)], ctypes.c_int),
    "cgtp_workspace_size": ([_vp, _vp, _c_i64, ctypes.c_int, ctypes.POINTER(ctypes.c_size_t)], ctypes.c_int),
    "cgtp_sh_forward": ([ctypes.c_int, ctypes.c_int, _c_i64, _vp, _vp, _vp], ctypes.c_int),
    "cgtp_sh_backward": ([ctypes.c_int, ctypes.c_int, _c_i64, _vp, _vp, _vp, _vp], ctypes.c_int),
    "cgtp_linear_create": ([ctypes.c_char_p, ctypes.c_char_p, ctypes.c_int, ctypes.POINTER(_vp)], ctypes.c_int),
    "cgtp_linear_destroy": ([_vp], ctypes.c_int),
    "cgtp_linear_query": ([_vp, _c_i64p, _c_i64p, _c_i64p, _c_i64p], ctypes.c_int),
    "cgtp_linear_paths": ([_vp, _c_i32p], ctypes.c_int),
    "cgtp_linear_forward": ([_vp, _c_i64, _vp, _vp, _vp, _vp], ctypes.c_int),
    "cgtp_linear_backward": ([_vp, _c_i64, _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp], ctypes.c_int),
    "cgtp_linear_workspace_size": ([_vp, _c_i64, ctypes.POINTER(ctypes.c_size_t)], ctypes.c_int),
}
for _name, (_args, _res) in _SIGS.items():
    _f = getattr(_lib, _name)
    _f.argtypes = _args
    _f.restype = _res

EXPORTED = tuple(_SIGS)


class CgtpError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        msg = _lib.cgtp_last_error().decode()
        super().__init__("%s: %s (%s)" % (where, _lib.cgtp_status_string(status).decode(), msg))


def _check(status, where):
    if status != 0:
        raise CgtpError(status, where)


_DT = {"f32": F32, "f64": F64, "bf16": BF16}
_WK = {"shared": W_SHARED, "per_row": W_PER_ROW}


def _torch():
    import torch
    return torch


def _torch_dtype(code):
    t = _torch()
    return {F32: t.float32, F64: t.float64, BF16: t.bfloat16}[code]


def _stream(t):
    torch = _torch()
    return _vp(torch.cuda.current_stream(t.device).cuda_stream)


def _ptr(t):
    return _vp(t.data_ptr()) if t is not None else _vp(0)


def _need(t, shape, dtype, name):
    if t is None:
        raise ValueError("%s is required" % name)
    if not t.is_cuda:
        raise ValueError("%s must be a device tensor" % name)
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))
    if t.dtype != dtype:
        raise ValueError("%s has dtype %s, expected %s" % (name, t.dtype, dtype))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return t


def _ws_bytes(ws):
    """Size in bytes of a caller-provided workspace (any dtype), which must be
    a contiguous device tensor."""
    if not ws.is_cuda:
        raise ValueError("workspace must be a device tensor")
    if not ws.is_contiguous():
        raise ValueError("workspace must be contiguous")
    return ws.numel() * ws.element_size()


_SEL = {"all": 0, "symmetric": 1, "skew": 2}


class Plan:
    """A tensor-product plan in the "uvu" (channel-wise) or "uvw" (fully
    connected) mode (cgtp_plan_create, or cgtp_plan_create_ex for a path
    selection "symmetric" / "skew" or collapsed outputs)."""

    def __init__(self, irreps_x, irreps_y, irreps_out, mode="uvu", dtype="f32", wkind="per_row",
                 select="all", collapse=False):
        self.irreps_x, self.irreps_y, self.irreps_out = irreps_x, irreps_y, irreps_out
        self.mode = mode
        self._ymul = max([int(t.split("x")[0]) if "x" in t else 1 for t in irreps_y.replace(" ", "").split("+") if t]
                         or [1])
        self.dtype_code = _DT[dtype]
        self.wkind = _WK[wkind]
        self.select, self.collapse = select, bool(collapse)
        h = _vp()
        if select == "all" and not collapse:
            _check(_lib.cgtp_plan_create(irreps_x.encode(), irreps_y.encode(), irreps_out.encode(),
                                         mode.encode(), self.dtype_code, self.wkind, ctypes.byref(h)),
                   "cgtp_plan_create")
        else:
            _check(_lib.cgtp_plan_create_ex(irreps_x.encode(), irreps_y.encode(), irreps_out.encode(),
                                            mode.encode(), self.dtype_code, self.wkind, _SEL[select],
                                            int(bool(collapse)), ctypes.byref(h)), "cgtp_plan_create_ex")
        self._h = h
        v = [ctypes.c_int64() for _ in range(5)]
        _check(_lib.cgtp_plan_query(h, *[ctypes.byref(a) for a in v]), "cgtp_plan_query")
        self.dim_x, self.dim_y, self.dim_out, self.num_paths, self.w_numel = (a.value for a in v)

    def __del__(self):
        h = getattr(self, "_h", None)
        if h and _lib is not None:
            _lib.cgtp_plan_destroy(h)
            self._h = None

    @property
    def torch_dtype(self):
        return _torch_dtype(self.dtype_code)

    def paths(self):
        t = np.zeros((self.num_paths, 6), np.int32)
        _check(_lib.cgtp_plan_paths(self._h, t.ctypes.data_as(_c_i32p)), "cgtp_plan_paths")
        return t

    def outputs(self):
        """Output blocks as rows (l3, p3, mul, offset)."""
        n = ctypes.c_int64()
        _check(_lib.cgtp_plan_outputs(self._h, ctypes.byref(n), None), "cgtp_plan_outputs")
        t = np.zeros((n.value, 4), np.int32)
        _check(_lib.cgtp_plan_outputs(self._h, None, t.ctypes.data_as(_c_i32p)), "cgtp_plan_outputs")
        return t

    def cg(self, path):
        _, _, l1, l2, l3, _ = self.paths()[path]
        out = np.zeros((2 * l1 + 1, 2 * l2 + 1, 2 * l3 + 1))
        _check(_lib.cgtp_plan_cg(self._h, int(path), out.ctypes.data_as(ctypes.POINTER(ctypes.c_double))),
               "cgtp_plan_cg")
        return out

    def workspace_size(self, op, B=0, graph=None):
        n = ctypes.c_size_t()
        _check(_lib.cgtp_workspace_size(self._h, graph._h if graph is not None else None, B, op,
                                        ctypes.byref(n)), "cgtp_workspace_size")
        return n.value

    def _w_shape(self, rows):
        return (self.w_numel,) if self.wkind == W_SHARED else (rows, self.w_numel)

    # ------------------------------------------------------------ tensor product
    def tp_forward(self, x, y, w, out=None):
        torch = _torch()
        B = x.shape[0]
        dt = self.torch_dtype
        _need(x, (B, self.dim_x), dt, "x")
        _need(y, (B, self.dim_y), dt, "y")
        _need(w, self._w_shape(B), dt, "w")
        if out is None:
            out = torch.empty((B, self.dim_out), dtype=dt, device=x.device)
        _need(out, (B, self.dim_out), dt, "out")
        _check(_lib.cgtp_tp_forward(self._h, B, _ptr(x), _ptr(y), _ptr(w), _ptr(out), _stream(x)),
               "cgtp_tp_forward")
        return out

    def tp_backward(self, x, y, w, grad_out, need=(True, True, True), out=(None, None, None), ws=None):
        torch = _torch()
        B = x.shape[0]
        dt = self.torch_dtype
        _need(x, (B, self.dim_x), dt, "x")
        _need(y, (B, self.dim_y), dt, "y")
        _need(w, self._w_shape(B), dt, "w")
        _need(grad_out, (B, self.dim_out), dt, "grad_out")
        shapes = [(B, self.dim_x), (B, self.dim_y), self._w_shape(B)]
        res = []
        for k in range(3):
            if not need[k]:
                res.append(None)
                continue
            t = out[k] if out[k] is not None else torch.empty(shapes[k], dtype=dt, device=x.device)
            res.append(_need(t, shapes[k], dt, "grad"))
        # uvw plans and y multiplicities > 1 use the workspace for every gradient
        nws = self.workspace_size(OP_TP_BACKWARD, B) if (need[2] or self.mode != "uvu" or self._ymul > 1) else 0
        if nws and ws is None:
            ws = torch.empty(nws, dtype=torch.uint8, device=x.device)
        _check(_lib.cgtp_tp_backward(self._h, B, _ptr(x), _ptr(y), _ptr(w), _ptr(grad_out),
                                     _ptr(res[0]), _ptr(res[1]), _ptr(res[2]),
                                     _ptr(ws) if nws else _vp(0), _ws_bytes(ws) if nws else 0, _stream(x)),
               "cgtp_tp_backward")
        return tuple(res)

    def tp_backward_noalloc(self, x, y, w, grad_out, need=(True, True, True), out=(None, None, None)):
        """cgtp_tp_backward_noalloc: the backward with shared-weight partials in the
        library's device scratch (no workspace; outputs may be passed in)."""
        torch = _torch()
        B = x.shape[0]
        dt = self.torch_dtype
        _need(x, (B, self.dim_x), dt, "x")
        _need(y, (B, self.dim_y), dt, "y")
        _need(w, self._w_shape(B), dt, "w")
        _need(grad_out, (B, self.dim_out), dt, "grad_out")
        shapes = [(B, self.dim_x), (B, self.dim_y), self._w_shape(B)]
        res = []
        for k in range(3):
            if not need[k]:
                res.append(None)
                continue
            t = out[k] if out[k] is not None else torch.empty(shapes[k], dtype=dt, device=x.device)
            res.append(_need(t, shapes[k], dt, "grad"))
        _check(_lib.cgtp_tp_backward_noalloc(self._h, B, _ptr(x), _ptr(y), _ptr(w), _ptr(grad_out),
                                             _ptr(res[0]), _ptr(res[1]), _ptr(res[2]), _stream(x)),
               "cgtp_tp_backward_noalloc")
        return tuple(res)

    # -------------------------------------------------------------- convolution
    def conv_forward(self, graph, x, sh, w, scale, out=None, ws=None, fp32_running_sum=True):
        """cgtp_conv_forward_ws; for collapsed bf16 plans a workspace for the fp32
        running sum over x blocks is allocated unless ``fp32_running_sum`` is False
        (then the sum is rounded to bf16 after every x block, as cgtp_conv_forward)."""
        torch = _torch()
        dt = self.torch_dtype
        _need(x, (graph.N, self.dim_x), dt, "x")
        _need(sh, (graph.E, self.dim_y), dt, "sh")
        _need(w, (graph.E, self.w_numel), dt, "w")
        if out is None:
            out = torch.empty((graph.N, self.dim_out), dtype=dt, device=x.device)
        _need(out, (graph.N, self.dim_out), dt, "out")
        if ws is None and fp32_running_sum:
            nws = self.workspace_size(OP_CONV_FORWARD, graph=graph)
            if nws:
                ws = torch.empty(nws, dtype=torch.uint8, device=x.device)
        _check(_lib.cgtp_conv_forward_ws(self._h, graph._h, _ptr(x), _ptr(sh), _ptr(w), float(scale), _ptr(out),
                                         _ptr(ws) if ws is not None else _vp(0),
                                         _ws_bytes(ws) if ws is not None else 0, _stream(x)), "cgtp_conv_forward_ws")
        return out

    def _double_outputs(self, shapes, need, out, dt, device):
        torch = _torch()
        res = []
        for k in range(4):
            if not need[k]:
                res.append(None)
                continue
            t = out[k] if out[k] is not None else torch.empty(shapes[k], dtype=dt, device=device)
            res.append(_need(t, shapes[k], dt, "double-backward output"))
        return res

    def tp_double_backward(self, x, y, w, grad_out, gg=(None, None, None), need=(True, True, True, True),
                           out=(None, None, None, None), ws=None):
        """Cotangents of (x, y, w, grad_out) for cotangents gg of the backward's
        (grad_x, grad_y, grad_w) (cgtp_tp_double_backward); None counts as zero."""
        torch = _torch()
        B = x.shape[0]
        dt = self.torch_dtype
        shapes = [(B, self.dim_x), (B, self.dim_y), self._w_shape(B), (B, self.dim_out)]
        for t, shp, nm in zip((x, y, w, grad_out), shapes, ("x", "y", "w", "grad_out")):
            _need(t, shp, dt, nm)
        for t, shp in zip(gg, shapes[:3]):
            if t is not None:
                _need(t, shp, dt, "cotangent")
        res = self._double_outputs(shapes, need, out, dt, x.device)
        nws = self.workspace_size(OP_TP_DOUBLE_BACKWARD, B)
        if ws is None:
            ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=x.device)
        _check(_lib.cgtp_tp_double_backward(self._h, B, _ptr(x), _ptr(y), _ptr(w), _ptr(grad_out),
                                            *[_ptr(t) for t in gg], *[_ptr(t) for t in res], _ptr(ws), _ws_bytes(ws),
                                            _stream(x)), "cgtp_tp_double_backward")
        return tuple(res)

    def conv_double_backward(self, graph, x, sh, w, scale, grad_out, gg=(None, None, None),
                             need=(True, True, True, True), out=(None, None, None, None), ws=None):
        """Cotangents of (x, sh, w, grad_out) for cotangents gg of the
        convolution backward's (grad_x, grad_sh, grad_w) (cgtp_conv_double_backward)."""
        torch = _torch()
        dt = self.torch_dtype
        shapes = [(graph.N, self.dim_x), (graph.E, self.dim_y), (graph.E, self.w_numel), (graph.N, self.dim_out)]
        for t, shp, nm in zip((x, sh, w, grad_out), shapes, ("x", "sh", "w", "grad_out")):
            _need(t, shp, dt, nm)
        for t, shp in zip(gg, shapes[:3]):
            if t is not None:
                _need(t, shp, dt, "cotangent")
        res = self._double_outputs(shapes, need, out, dt, x.device)
        nws = self.workspace_size(OP_CONV_DOUBLE_BACKWARD, graph=graph)
        if ws is None:
            ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=x.device)
        _check(_lib.cgtp_conv_double_backward(self._h, graph._h, _ptr(x), _ptr(sh), _ptr(w), float(scale),
                                              _ptr(grad_out), *[_ptr(t) for t in gg], *[_ptr(t) for t in res],
                                              _ptr(ws), _ws_bytes(ws), _stream(x)), "cgtp_conv_double_backward")
        return tuple(res)

    def conv_backward(self, graph, x, sh, w, scale, grad_out, need=(True, True, True),
                      out=(None, None, None), ws=None):
        torch = _torch()
        dt = self.torch_dtype
        _need(x, (graph.N, self.dim_x), dt, "x")
        _need(sh, (graph.E, self.dim_y), dt, "sh")
        _need(w, (graph.E, self.w_numel), dt, "w")
        _need(grad_out, (graph.N, self.dim_out), dt, "grad_out")
        shapes = [(graph.N, self.dim_x), (graph.E, self.dim_y), (graph.E, self.w_numel)]
        res = []
        for k in range(3):
            if not need[k]:
                res.append(None)
                continue
            t = out[k] if out[k] is not None else torch.empty(shapes[k], dtype=dt, device=x.device)
            res.append(_need(t, shapes[k], dt, "grad"))
        nws = self.workspace_size(OP_CONV_BACKWARD, graph=graph) if (need[0] or need[1]) else 0
        if ws is not None:
            nws = _ws_bytes(ws)
        elif nws:
            ws = torch.empty(nws, dtype=torch.uint8, device=x.device)
        _check(_lib.cgtp_conv_backward(self._h, graph._h, _ptr(x), _ptr(sh), _ptr(w), float(scale),
                                       _ptr(grad_out), _ptr(res[0]), _ptr(res[1]), _ptr(res[2]),
                                       _ptr(ws) if nws else _vp(0), _ws_bytes(ws) if nws else 0,
                                       _stream(x)), "cgtp_conv_backward")
        return tuple(res)


    # -------------------------------------- convolution with the radial last layer
    def radial_workspace_size(self, graph, hidden):
        n = ctypes.c_size_t()
        _check(_lib.cgtp_conv_radial_workspace_size(self._h, graph._h, int(hidden), ctypes.byref(n)),
               "cgtp_conv_radial_workspace_size")
        return n.value

    def conv_forward_radial(self, graph, x, sh, h, W2, scale, out=None):
        """Convolution with w = h W2 formed inside the kernel (cgtp_conv_forward_radial)."""
        torch = _torch()
        dt = self.torch_dtype
        H = W2.shape[0]
        _need(x, (graph.N, self.dim_x), dt, "x")
        _need(sh, (graph.E, self.dim_y), dt, "sh")
        _need(h, (graph.E, H), dt, "h")
        _need(W2, (H, self.w_numel), dt, "W2")
        if out is None:
            out = torch.empty((graph.N, self.dim_out), dtype=dt, device=x.device)
        _need(out, (graph.N, self.dim_out), dt, "out")
        _check(_lib.cgtp_conv_forward_radial(self._h, graph._h, _ptr(x), _ptr(sh), _ptr(h), H, _ptr(W2), float(scale),
                                             _ptr(out), _stream(x)), "cgtp_conv_forward_radial")
        return out

    def conv_backward_radial(self, graph, x, sh, h, W2, scale, grad_out, need=(True, True, True, True),
                             out=(None, None, None, None), ws=None):
        """(grad_x, grad_sh, grad_h, grad_W2) of the radial convolution (cgtp_conv_backward_radial)."""
        torch = _torch()
        dt = self.torch_dtype
        H = W2.shape[0]
        _need(x, (graph.N, self.dim_x), dt, "x")
        _need(sh, (graph.E, self.dim_y), dt, "sh")
        _need(h, (graph.E, H), dt, "h")
        _need(W2, (H, self.w_numel), dt, "W2")
        _need(grad_out, (graph.N, self.dim_out), dt, "grad_out")
        shapes = [(graph.N, self.dim_x), (graph.E, self.dim_y), (graph.E, H), (H, self.w_numel)]
        res = []
        for k in range(4):
            if not need[k]:
                res.append(None)
                continue
            t = out[k] if out[k] is not None else torch.empty(shapes[k], dtype=dt, device=x.device)
            res.append(_need(t, shapes[k], dt, "grad"))
        if ws is None:
            ws = torch.empty(max(self.radial_workspace_size(graph, H), 1), dtype=torch.uint8, device=x.device)
        _check(_lib.cgtp_conv_backward_radial(self._h, graph._h, _ptr(x), _ptr(sh), _ptr(h), H, _ptr(W2), float(scale),
                                              _ptr(grad_out), *[_ptr(t) for t in res], _ptr(ws), _ws_bytes(ws),
                                              _stream(x)), "cgtp_conv_backward_radial")
        return tuple(res)


class Linear:
    """An equivariant linear map irreps_in -> irreps_out (cgtp_linear_create)."""

    def __init__(self, irreps_in, irreps_out, dtype="f32"):
        self.irreps_in, self.irreps_out = irreps_in, irreps_out
        self.dtype_code = _DT[dtype]
        h = _vp()
        _check(_lib.cgtp_linear_create(irreps_in.encode(), irreps_out.encode(), self.dtype_code, ctypes.byref(h)),
               "cgtp_linear_create")
        self._h = h
        v = [ctypes.c_int64() for _ in range(4)]
        _check(_lib.cgtp_linear_query(h, *[ctypes.byref(a) for a in v]), "cgtp_linear_query")
        self.dim_in, self.dim_out, self.num_paths, self.w_numel = (a.value for a in v)

    def __del__(self):
        h = getattr(self, "_h", None)
        if h and _lib is not None:
            _lib.cgtp_linear_destroy(h)
            self._h = None

    @property
    def torch_dtype(self):
        return _torch_dtype(self.dtype_code)

    def paths(self):
        t = np.zeros((self.num_paths, 5), np.int32)
        _check(_lib.cgtp_linear_paths(self._h, t.ctypes.data_as(_c_i32p)), "cgtp_linear_paths")
        return t

    def workspace_size(self, B):
        n = ctypes.c_size_t()
        _check(_lib.cgtp_linear_workspace_size(self._h, B, ctypes.byref(n)), "cgtp_linear_workspace_size")
        return n.value

    def forward(self, x, w, out=None):
        torch = _torch()
        B = x.shape[0]
        dt = self.torch_dtype
        _need(x, (B, self.dim_in), dt, "x")
        _need(w, (self.w_numel,), dt, "w")
        if out is None:
            out = torch.empty((B, self.dim_out), dtype=dt, device=x.device)
        _need(out, (B, self.dim_out), dt, "out")
        _check(_lib.cgtp_linear_forward(self._h, B, _ptr(x), _ptr(w), _ptr(out), _stream(x)), "cgtp_linear_forward")
        return out

    def backward(self, x, w, grad_out, need=(True, True), out=(None, None), ws=None):
        torch = _torch()
        B = x.shape[0]
        dt = self.torch_dtype
        _need(x, (B, self.dim_in), dt, "x")
        _need(w, (self.w_numel,), dt, "w")
        _need(grad_out, (B, self.dim_out), dt, "grad_out")
        shapes = [(B, self.dim_in), (self.w_numel,)]
        res = []
        for k in range(2):
            if not need[k]:
                res.append(None)
                continue
            t = out[k] if out[k] is not None else torch.empty(shapes[k], dtype=dt, device=x.device)
            res.append(_need(t, shapes[k], dt, "grad"))
        nws = self.workspace_size(B) if need[1] else 0
        if nws and ws is None:
            ws = torch.empty(nws, dtype=torch.uint8, device=x.device)
        _check(_lib.cgtp_linear_backward(self._h, B, _ptr(x), _ptr(w), _ptr(grad_out), _ptr(res[0]), _ptr(res[1]),
                                         _ptr(ws) if nws else _vp(0), _ws_bytes(ws) if nws else 0, _stream(x)),
               "cgtp_linear_backward")
        return tuple(res)


class Graph:
    """A CSR-by-destination graph handle (cgtp_graph_create). Keeps the CSR
    tensors alive for as long as the handle exists."""

    def __init__(self, N, row_ptr, src, pad_node=None):
        torch = _torch()
        _need(row_ptr, (N + 1,), torch.int32, "row_ptr")
        E = src.shape[0]
        _need(src, (E,), torch.int32, "src")
        self.N, self.E = int(N), int(E)
        self.row_ptr, self.src = row_ptr, src
        self.pad_node = pad_node
        h = _vp()
        if pad_node is None:
            _check(_lib.cgtp_graph_create(self.N, self.E, _ptr(row_ptr), _ptr(src), _stream(row_ptr),
                                          ctypes.byref(h)), "cgtp_graph_create")
        else:
            _check(_lib.cgtp_graph_create_ex(self.N, self.E, _ptr(row_ptr), _ptr(src), int(pad_node),
                                             _stream(row_ptr), ctypes.byref(h)), "cgtp_graph_create_ex")
        self._h = h

    def __del__(self):
        h = getattr(self, "_h", None)
        if h and _lib is not None:
            _lib.cgtp_graph_destroy(h)
            self._h = None

    def transpose(self):
        torch = _torch()
        col_ptr = torch.empty(self.N + 1, dtype=torch.int32, device=self.row_ptr.device)
        eid = torch.empty(max(self.E, 1), dtype=torch.int32, device=self.row_ptr.device)
        _check(_lib.cgtp_graph_transpose(self._h, _ptr(col_ptr), _ptr(eid), _stream(col_ptr)),
               "cgtp_graph_transpose")
        return col_ptr, eid[:int(col_ptr[-1].item()) if self.N > 0 else 0]


def csr_from_coo(N, src, dst):
    """Device COO (int32) -> (row_ptr, src_sorted, perm), CSR by destination."""
    torch = _torch()
    E = src.shape[0]
    _need(src, (E,), torch.int32, "src")
    _need(dst, (E,), torch.int32, "dst")
    row_ptr = torch.empty(N + 1, dtype=torch.int32, device=src.device)
    src_sorted = torch.empty(E, dtype=torch.int32, device=src.device)
    perm = torch.empty(E, dtype=torch.int32, device=src.device)
    _check(_lib.cgtp_csr_from_coo(N, E, _ptr(src), _ptr(dst), _ptr(row_ptr), _ptr(src_sorted), _ptr(perm),
                                  _stream(src)), "cgtp_csr_from_coo")
    return row_ptr, src_sorted, perm


def _sh_code(t):
    torch = _torch()
    return {torch.float32: F32, torch.float64: F64, torch.bfloat16: BF16}[t.dtype]


def sh_forward(lmax, vec, out=None):
    torch = _torch()
    n = vec.shape[0]
    _need(vec, (n, 3), vec.dtype, "vec")
    if out is None:
        out = torch.empty((n, (lmax + 1) ** 2), dtype=vec.dtype, device=vec.device)
    _need(out, (n, (lmax + 1) ** 2), vec.dtype, "sh")
    _check(_lib.cgtp_sh_forward(lmax, _sh_code(vec), n, _ptr(vec), _ptr(out), _stream(vec)), "cgtp_sh_forward")
    return out


def sh_backward(lmax, vec, grad_sh, out=None):
    torch = _torch()
    n = vec.shape[0]
    _need(vec, (n, 3), vec.dtype, "vec")
    _need(grad_sh, (n, (lmax + 1) ** 2), vec.dtype, "grad_sh")
    if out is None:
        out = torch.empty((n, 3), dtype=vec.dtype, device=vec.device)
    _check(_lib.cgtp_sh_backward(lmax, _sh_code(vec), n, _ptr(vec), _ptr(grad_sh), _ptr(out), _stream(vec)),
           "cgtp_sh_backward")
    return out
