"""ctypes binding of libmoe_int4.so (the C ABI in include/moe_int4.h).

Argument marshalling only: every step of the layer runs in the HIP kernels of
the library. PyTorch supplies device memory and the current HIP stream. The
module raises when the library is missing; there is no fallback path.

Tensor formats:
  bf16 values       torch.bfloat16 tensors (passed as uint16 bit patterns)
  packed int4 codes torch.int32 tensors holding the uint32 words
  logits, y         torch.float32
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_int4.so")

MOE_OK, MOE_EINVAL, MOE_EUNSUPPORTED, MOE_EWORKSPACE, MOE_EHIP = 0, -1, -2, -3, -4

_P = ctypes.c_void_p
_I32 = ctypes.c_int32


class MoeLayerT(ctypes.Structure):
    _fields_ = [("d", _I32), ("f", _I32), ("E", _I32), ("k", _I32), ("f_sh", _I32),
                ("gu_q", _P), ("gu_s", _P), ("gu_b", _P),
                ("dn_q", _P), ("dn_s", _P), ("dn_b", _P),
                ("sh_gu_q", _P), ("sh_gu_s", _P), ("sh_gu_b", _P),
                ("sh_dn_q", _P), ("sh_dn_s", _P), ("sh_dn_b", _P),
                ("prep", _P)]


class MoeRoutingT(ctypes.Structure):
    _fields_ = [("topk_ids", _P), ("topk_w", _P), ("counts", _P), ("offsets", _P),
                ("sorted_pair", _P), ("sorted_token", _P), ("pair_pos", _P),
                ("block_map", _P), ("num_blocks", _P)]


class MoeWorkspaceLayoutT(ctypes.Structure):
    _fields_ = [("decode_form", _I32), ("x16", ctypes.c_int64), ("h", ctypes.c_int64),
                ("h_sh", ctypes.c_int64), ("o", ctypes.c_int64), ("o_sh", ctypes.c_int64),
                ("dec_h", ctypes.c_int64)]


_lib = None


def load() -> ctypes.CDLL:
    """Load the HIP library (once). Raises FileNotFoundError when it is not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise FileNotFoundError(
                f"{LIB_PATH} is missing: build it with grouped_int4_dequant_amd/build.py")
        lib = ctypes.CDLL(LIB_PATH)
        lib.moe_max_blocks.argtypes = [_I32, _I32, _I32]
        lib.moe_max_blocks.restype = _I32
        lib.moe_workspace_bytes.argtypes = [_I32, ctypes.POINTER(MoeLayerT)]
        lib.moe_workspace_bytes.restype = ctypes.c_size_t
        lib.moe_workspace_layout.argtypes = [_I32, ctypes.POINTER(MoeLayerT), ctypes.POINTER(MoeWorkspaceLayoutT)]
        lib.moe_workspace_layout.restype = ctypes.c_int
        lib.moe_route_workspace_bytes.argtypes = [_I32, _I32]
        lib.moe_route_workspace_bytes.restype = ctypes.c_size_t
        lib.moe_route.argtypes = [_P, _I32, _I32, _I32, ctypes.POINTER(MoeRoutingT), _P,
                                  ctypes.c_size_t, _P]
        lib.moe_route.restype = ctypes.c_int
        lib.moe_grouped_gemm_int4.argtypes = [_P, _I32, _P, _I32, _I32, _P, _P, _P, _P, _P, _I32,
                                              _P, _I32, _P]
        lib.moe_grouped_gemm_int4.restype = ctypes.c_int
        lib.moe_layer_forward.argtypes = [ctypes.POINTER(MoeLayerT), _P, _P, _I32, _P,
                                          ctypes.POINTER(MoeRoutingT), _P, ctypes.c_size_t, _P]
        lib.moe_layer_forward.restype = ctypes.c_int
        lib.moe_prefill_chunked.argtypes = [ctypes.POINTER(MoeLayerT), _P, _P, _I32, _I32, _P, _P,
                                            ctypes.c_size_t, _P]
        lib.moe_layer_forward_ablation.argtypes = [ctypes.POINTER(MoeLayerT), _P, _P, _I32, _P,
                                                   ctypes.POINTER(MoeRoutingT), _P, ctypes.c_size_t, _P,
                                                   _I32]
        lib.moe_layer_forward_ablation.restype = ctypes.c_int
        lib.moe_layer_forward_noalloc.argtypes = [ctypes.POINTER(MoeLayerT), _P, _P, _I32, _P,
                                                  ctypes.POINTER(MoeRoutingT), _P]
        lib.moe_layer_forward_noalloc.restype = ctypes.c_int
        lib.moe_layer_forward_checked.argtypes = [ctypes.POINTER(MoeLayerT), _P, _P, _I32, _P,
                                                  ctypes.POINTER(MoeRoutingT), _P, ctypes.c_size_t, _P, _P]
        lib.moe_layer_forward_checked.restype = ctypes.c_int
        lib.moe_router_topk.argtypes = [_P, _I32, _I32, _P, _I32, _I32, _P, _P, _P, _P]
        lib.moe_router_topk.restype = ctypes.c_int
        lib.moe_layer_forward_router.argtypes = [ctypes.POINTER(MoeLayerT), _P, _P, _I32, _P,
                                                 ctypes.POINTER(MoeRoutingT), _P, ctypes.c_size_t, _P]
        lib.moe_layer_forward_router.restype = ctypes.c_int
        lib.moe_layer_graph_create.argtypes = [ctypes.POINTER(MoeLayerT), _P, _P, _I32, _P, _P, ctypes.c_size_t,
                                               _I32, _I32, _P, ctypes.POINTER(_P)]
        lib.moe_layer_graph_create.restype = ctypes.c_int
        lib.moe_layer_graph_launch.argtypes = [_P, _P]
        lib.moe_layer_graph_launch.restype = ctypes.c_int
        lib.moe_layer_graph_destroy.argtypes = [_P]
        lib.moe_layer_graph_destroy.restype = ctypes.c_int
        lib.moe_router_logits.argtypes = [_P, _I32, _I32, _P, _I32, _P, _P]
        lib.moe_router_logits.restype = ctypes.c_int
        lib.moe_ablation_workspace_bytes.argtypes = [_I32, ctypes.POINTER(MoeLayerT), _I32]
        lib.moe_ablation_workspace_bytes.restype = ctypes.c_size_t
        lib.moe_prefill_chunked.restype = ctypes.c_int
        lib.moe_prepared_bytes.argtypes = [ctypes.POINTER(MoeLayerT)]
        lib.moe_prepared_bytes.restype = ctypes.c_size_t
        lib.moe_prepare_weights.argtypes = [ctypes.POINTER(MoeLayerT), _P, ctypes.c_size_t, _P]
        lib.moe_prepare_weights.restype = ctypes.c_int
        lib.moe_status_string.argtypes = [ctypes.c_int]
        lib.moe_status_string.restype = ctypes.c_char_p
        _lib = lib
    return _lib


def status_string(status: int) -> str:
    return load().moe_status_string(int(status)).decode()


def _check(status: int, what: str):
    if status != MOE_OK:
        raise ValueError(f"{what}: {status_string(status)} (status {status})")


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> int:
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _need(t: torch.Tensor, name: str, dtype: torch.dtype, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


class Layer:
    """Device weights of one MoE layer plus the moe_layer_t that points at them."""

    KEYS = ("gu_q", "gu_s", "gu_b", "dn_q", "dn_s", "dn_b",
            "sh_gu_q", "sh_gu_s", "sh_gu_b", "sh_dn_q", "sh_dn_s", "sh_dn_b")

    def __init__(self, d: int, f: int, E: int, k: int, f_sh: int, tensors: Dict[str, torch.Tensor],
                 prepare: bool = True):
        self.d, self.f, self.E, self.k, self.f_sh = d, f, E, k, f_sh
        self.tensors = dict(tensors)
        shapes = {"gu_q": (E, 2 * f, d // 8), "gu_s": (E, 2 * f, d // 64), "gu_b": (E, 2 * f, d // 64),
                  "dn_q": (E, d, f // 8), "dn_s": (E, d, f // 64), "dn_b": (E, d, f // 64),
                  "sh_gu_q": (2 * f_sh, d // 8), "sh_gu_s": (2 * f_sh, d // 64),
                  "sh_gu_b": (2 * f_sh, d // 64), "sh_dn_q": (d, f_sh // 8),
                  "sh_dn_s": (d, f_sh // 64), "sh_dn_b": (d, f_sh // 64)}
        ptrs = {}
        for key in self.KEYS:
            if key.startswith("sh_") and f_sh == 0:
                ptrs[key] = None
                continue
            t = self.tensors[key]
            _need(t, key, torch.int32 if key.endswith("_q") else torch.bfloat16, shapes[key])
            ptrs[key] = t.data_ptr()
        self.c = MoeLayerT(d, f, E, k, f_sh, *[ptrs[k_] for k_ in self.KEYS], None)
        self.prep = None
        if prepare:
            self.prepare()

    def prepare(self, stream=None) -> bool:
        """moe_prepare_weights into a new device buffer, then point c.prep at
        it. Returns False (and leaves c.prep null) when the layer's shape has
        no prepared form (d, f or f_sh not a multiple of 128)."""
        lib = load()
        n = int(lib.moe_prepared_bytes(ctypes.byref(self.c)))
        if n == 0:
            return False
        dev = self.tensors["gu_q"].device
        buf = torch.empty(n + 256, dtype=torch.uint8, device=dev)
        ptr = (buf.data_ptr() + 255) // 256 * 256
        _check(lib.moe_prepare_weights(ctypes.byref(self.c), ptr, n, _stream(stream)), "moe_prepare_weights")
        self.prep, self.c.prep = buf, ptr
        return True

    @classmethod
    def from_numpy(cls, d, f, E, k, f_sh, arrays, device="cuda", prepare: bool = True):
        """Upload generator arrays (uint32 codes, uint16 bf16 bits) to the GPU
        (and, with prepare, build the prepared copy the prefill GEMMs read)."""
        import numpy as np
        ts = {}
        for key, a in arrays.items():
            if key.endswith("_q"):
                ts[key] = torch.from_numpy(np.ascontiguousarray(a).view(np.int32)).to(device)
            else:
                ts[key] = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)
        return cls(d, f, E, k, f_sh, ts, prepare=prepare)


def max_blocks(T: int, E: int, k: int) -> int:
    return int(load().moe_max_blocks(T, E, k))


def prepared_bytes(layer: Layer) -> int:
    return int(load().moe_prepared_bytes(ctypes.byref(layer.c)))


def workspace_bytes(T: int, layer: Layer) -> int:
    return int(load().moe_workspace_bytes(T, ctypes.byref(layer.c)))


def workspace_layout(T: int, layer: Layer) -> Dict[str, int]:
    """moe_workspace_layout: byte offsets of the fp16 intermediates a
    moe_layer_forward call of T tokens keeps in its workspace (-1: absent)."""
    out = MoeWorkspaceLayoutT()
    _check(load().moe_workspace_layout(T, ctypes.byref(layer.c), ctypes.byref(out)), "moe_workspace_layout")
    return {name: int(getattr(out, name)) for name, _ in MoeWorkspaceLayoutT._fields_}


def route_workspace_bytes(T: int, E: int) -> int:
    return int(load().moe_route_workspace_bytes(T, E))


def alloc_routing(T: int, E: int, k: int, device="cuda") -> Dict[str, torch.Tensor]:
    mb = max_blocks(T, E, k)
    i32 = dict(dtype=torch.int32, device=device)
    return dict(topk_ids=torch.empty((T, k), **i32),
                topk_w=torch.empty((T, k), dtype=torch.float32, device=device),
                counts=torch.empty(E, **i32), offsets=torch.empty(E + 1, **i32),
                sorted_pair=torch.empty(T * k, **i32), sorted_token=torch.empty(T * k, **i32),
                pair_pos=torch.empty(T * k, **i32), block_map=torch.empty((mb, 3), **i32),
                num_blocks=torch.empty(1, **i32))


def _routing_struct(r: Dict[str, torch.Tensor]) -> MoeRoutingT:
    for key, t in r.items():
        _need(t, key, torch.float32 if key == "topk_w" else torch.int32)
    return MoeRoutingT(*[r[k].data_ptr() for k in ("topk_ids", "topk_w", "counts", "offsets",
                                                   "sorted_pair", "sorted_token", "pair_pos",
                                                   "block_map", "num_blocks")])


def alloc_workspace(nbytes: int, device="cuda") -> torch.Tensor:
    """Workspace buffer (torch's caching allocator returns 256-byte aligned storage)."""
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)


def route(logits: torch.Tensor, k: int, out: Optional[Dict[str, torch.Tensor]] = None,
          ws: Optional[torch.Tensor] = None, stream=None) -> Dict[str, torch.Tensor]:
    """moe_route: GPU top-k, gates, histogram, scan, stable scatter and block map."""
    T, E = logits.shape
    _need(logits, "logits", torch.float32)
    out = alloc_routing(T, E, k, logits.device) if out is None else out
    need = route_workspace_bytes(T, E)
    ws = alloc_workspace(need, logits.device) if ws is None else ws
    rs = _routing_struct(out)
    _check(load().moe_route(logits.data_ptr(), T, E, k, ctypes.byref(rs), ws.data_ptr(),
                            ws.numel(), _stream(stream)), "moe_route")
    return out


def grouped_gemm_int4(A: torch.Tensor, a_row: Optional[torch.Tensor], N: int, K: int,
                      Wq: torch.Tensor, Ws: torch.Tensor, Wb: torch.Tensor,
                      block_map: torch.Tensor, num_blocks: torch.Tensor, C: torch.Tensor,
                      stream=None) -> torch.Tensor:
    """moe_grouped_gemm_int4: C[p] = A[row(p)] @ W_e(p)^T for the rows of every block."""
    _need(A, "A", torch.bfloat16)
    _need(Wq, "Wq", torch.int32)
    _need(Ws, "Ws", torch.bfloat16)
    _need(Wb, "Wb", torch.bfloat16)
    _need(block_map, "block_map", torch.int32)
    _need(num_blocks, "num_blocks", torch.int32)
    _need(C, "C", torch.float32)
    if a_row is not None:
        _need(a_row, "a_row", torch.int32)
    _check(load().moe_grouped_gemm_int4(A.data_ptr(), A.shape[-1], _ptr(a_row), N, K,
                                        Wq.data_ptr(), Ws.data_ptr(), Wb.data_ptr(),
                                        block_map.data_ptr(), num_blocks.data_ptr(),
                                        block_map.shape[0], C.data_ptr(), C.shape[-1],
                                        _stream(stream)), "moe_grouped_gemm_int4")
    return C


def layer_forward(layer: Layer, x: torch.Tensor, logits: torch.Tensor,
                  y: Optional[torch.Tensor] = None,
                  routing: Optional[Dict[str, torch.Tensor]] = None,
                  ws: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """moe_layer_forward: the whole layer for T tokens into fp32 y."""
    T = x.shape[0]
    _need(x, "x", torch.bfloat16, (T, layer.d))
    _need(logits, "logits", torch.float32, (T, layer.E))
    y = torch.empty((T, layer.d), dtype=torch.float32, device=x.device) if y is None else y
    _need(y, "y", torch.float32, (T, layer.d))
    ws = alloc_workspace(workspace_bytes(T, layer), x.device) if ws is None else ws
    rs = _routing_struct(routing) if routing is not None else None
    _check(load().moe_layer_forward(ctypes.byref(layer.c), x.data_ptr(), logits.data_ptr(), T,
                                    y.data_ptr(), ctypes.byref(rs) if rs is not None else None,
                                    ws.data_ptr(), ws.numel(), _stream(stream)),
           "moe_layer_forward")
    return y


OVERFLOW_X, OVERFLOW_H, OVERFLOW_O = 1, 2, 4


def layer_forward_checked(layer: Layer, x: torch.Tensor, logits: torch.Tensor, overflow: torch.Tensor,
                          y: Optional[torch.Tensor] = None,
                          routing: Optional[Dict[str, torch.Tensor]] = None,
                          ws: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """moe_layer_forward_checked: the layer, ORing OVERFLOW_* bits into the
    int32 device tensor `overflow` (one element, set by the caller) when a
    value kept in fp16 leaves fp16's finite range."""
    T = x.shape[0]
    _need(x, "x", torch.bfloat16, (T, layer.d))
    _need(logits, "logits", torch.float32, (T, layer.E))
    _need(overflow, "overflow", torch.int32, (1,))
    y = torch.empty((T, layer.d), dtype=torch.float32, device=x.device) if y is None else y
    _need(y, "y", torch.float32, (T, layer.d))
    ws = alloc_workspace(workspace_bytes(T, layer), x.device) if ws is None else ws
    rs = _routing_struct(routing) if routing is not None else None
    _check(load().moe_layer_forward_checked(ctypes.byref(layer.c), x.data_ptr(), logits.data_ptr(), T,
                                            y.data_ptr(), ctypes.byref(rs) if rs is not None else None,
                                            ws.data_ptr(), ws.numel(), _stream(stream), overflow.data_ptr()),
           "moe_layer_forward_checked")
    return y


def layer_forward_noalloc(layer: Layer, x: torch.Tensor, logits: torch.Tensor,
                          y: Optional[torch.Tensor] = None,
                          routing: Optional[Dict[str, torch.Tensor]] = None, stream=None) -> torch.Tensor:
    """moe_layer_forward_noalloc: the layer with the library's static per-GPU
    scratch array as its workspace (no device allocation in the call)."""
    T = x.shape[0]
    _need(x, "x", torch.bfloat16, (T, layer.d))
    _need(logits, "logits", torch.float32, (T, layer.E))
    y = torch.empty((T, layer.d), dtype=torch.float32, device=x.device) if y is None else y
    _need(y, "y", torch.float32, (T, layer.d))
    rs = _routing_struct(routing) if routing is not None else None
    _check(load().moe_layer_forward_noalloc(ctypes.byref(layer.c), x.data_ptr(), logits.data_ptr(), T,
                                            y.data_ptr(), ctypes.byref(rs) if rs is not None else None,
                                            _stream(stream)), "moe_layer_forward_noalloc")
    return y


def router_logits(x: torch.Tensor, w_r: torch.Tensor, logits: Optional[torch.Tensor] = None,
                  stream=None) -> torch.Tensor:
    """moe_router_logits: logits fp32 [T][E] = x W_r^T from bf16 x [T][d] and
    bf16 W_r [E][d]."""
    T, d = x.shape
    E = w_r.shape[0]
    _need(x, "x", torch.bfloat16, (T, d))
    _need(w_r, "w_r", torch.bfloat16, (E, d))
    logits = torch.empty((T, E), dtype=torch.float32, device=x.device) if logits is None else logits
    _need(logits, "logits", torch.float32, (T, E))
    _check(load().moe_router_logits(x.data_ptr(), T, d, w_r.data_ptr(), E, logits.data_ptr(), _stream(stream)),
           "moe_router_logits")
    return logits


def router_topk(x: torch.Tensor, w_r: torch.Tensor, k: int, logits: Optional[torch.Tensor] = None,
                stream=None):
    """moe_router_topk: (topk_ids int32 [T][k], topk_w fp32 [T][k]) from bf16
    x [T][d] and bf16 W_r [E][d]; the fp32 logits [T][E] go to `logits`
    (allocated when not given)."""
    T, d = x.shape
    E = w_r.shape[0]
    _need(x, "x", torch.bfloat16, (T, d))
    _need(w_r, "w_r", torch.bfloat16, (E, d))
    logits = torch.empty((T, E), dtype=torch.float32, device=x.device) if logits is None else logits
    _need(logits, "logits", torch.float32, (T, E))
    ids = torch.empty((T, k), dtype=torch.int32, device=x.device)
    w = torch.empty((T, k), dtype=torch.float32, device=x.device)
    _check(load().moe_router_topk(x.data_ptr(), T, d, w_r.data_ptr(), E, k, _ptr(logits), ids.data_ptr(),
                                  w.data_ptr(), _stream(stream)), "moe_router_topk")
    return ids, w


def layer_forward_router(layer: Layer, x: torch.Tensor, w_r: torch.Tensor,
                         y: Optional[torch.Tensor] = None,
                         routing: Optional[Dict[str, torch.Tensor]] = None,
                         ws: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """moe_layer_forward_router: the whole layer from bf16 router weights
    W_r [E][d] instead of logits."""
    T = x.shape[0]
    _need(x, "x", torch.bfloat16, (T, layer.d))
    _need(w_r, "w_r", torch.bfloat16, (layer.E, layer.d))
    y = torch.empty((T, layer.d), dtype=torch.float32, device=x.device) if y is None else y
    _need(y, "y", torch.float32, (T, layer.d))
    ws = alloc_workspace(workspace_bytes(T, layer), x.device) if ws is None else ws
    rs = _routing_struct(routing) if routing is not None else None
    _check(load().moe_layer_forward_router(ctypes.byref(layer.c), x.data_ptr(), w_r.data_ptr(), T, y.data_ptr(),
                                           ctypes.byref(rs) if rs is not None else None, ws.data_ptr(),
                                           ws.numel(), _stream(stream)), "moe_layer_forward_router")
    return y


GRAPH_CONCURRENT = 1


class LayerGraph:
    """moe_layer_graph_create/_launch/_destroy: the layer captured once into a
    HIP graph bound to x, logits, y and a workspace; launch() recomputes y
    from their current contents. concurrent=True runs the shared expert on a
    branch beside the routing (shared_unit_rows rows per item; 0: 96)."""

    def __init__(self, layer: Layer, x: torch.Tensor, logits: torch.Tensor, y: torch.Tensor,
                 ws: Optional[torch.Tensor] = None, concurrent: bool = True, shared_unit_rows: int = 0):
        T = x.shape[0]
        _need(x, "x", torch.bfloat16, (T, layer.d))
        _need(logits, "logits", torch.float32, (T, layer.E))
        _need(y, "y", torch.float32, (T, layer.d))
        ws = alloc_workspace(workspace_bytes(T, layer), x.device) if ws is None else ws
        self._keep = (layer, x, logits, y, ws)  # the graph holds their addresses
        cap = torch.cuda.Stream(device=x.device)
        cap.wait_stream(torch.cuda.current_stream(x.device))
        h = ctypes.c_void_p()
        _check(load().moe_layer_graph_create(ctypes.byref(layer.c), x.data_ptr(), logits.data_ptr(), T,
                                             y.data_ptr(), ws.data_ptr(), ws.numel(),
                                             GRAPH_CONCURRENT if concurrent else 0, shared_unit_rows,
                                             cap.cuda_stream, ctypes.byref(h)), "moe_layer_graph_create")
        self._h = h.value

    def launch(self, stream=None):
        _check(load().moe_layer_graph_launch(self._h, _stream(stream)), "moe_layer_graph_launch")

    def close(self):
        if self._h:
            _check(load().moe_layer_graph_destroy(self._h), "moe_layer_graph_destroy")
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


ABLATIONS = {"none": 0, "tile16": 1, "host_routing": 2, "unfused": 3}


def ablation_workspace_bytes(T: int, layer: Layer, variant: str) -> int:
    n = load().moe_ablation_workspace_bytes(T, ctypes.byref(layer.c), ABLATIONS[variant])
    if n == 0:
        raise ValueError("invalid layer, token count or ablation")
    return n


def layer_forward_ablation(layer: Layer, x: torch.Tensor, logits: torch.Tensor, variant: str,
                           y: Optional[torch.Tensor] = None,
                           routing: Optional[Dict[str, torch.Tensor]] = None,
                           ws: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """moe_layer_forward_ablation: the prefill sequence with one of the pages'
    ablations ("none", "tile16", "host_routing", "unfused"); measurement only."""
    T = x.shape[0]
    _need(x, "x", torch.bfloat16, (T, layer.d))
    _need(logits, "logits", torch.float32, (T, layer.E))
    y = torch.empty((T, layer.d), dtype=torch.float32, device=x.device) if y is None else y
    _need(y, "y", torch.float32, (T, layer.d))
    ws = alloc_workspace(ablation_workspace_bytes(T, layer, variant), x.device) if ws is None else ws
    rs = _routing_struct(routing) if routing is not None else None
    _check(load().moe_layer_forward_ablation(ctypes.byref(layer.c), x.data_ptr(), logits.data_ptr(), T,
                                             y.data_ptr(), ctypes.byref(rs) if rs is not None else None,
                                             ws.data_ptr(), ws.numel(), _stream(stream), ABLATIONS[variant]),
           "moe_layer_forward_ablation")
    return y


def prefill_chunked(layer: Layer, x: torch.Tensor, logits: torch.Tensor, chunk: int = 2048,
                    y: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None,
                    stream=None) -> torch.Tensor:
    """moe_prefill_chunked: the layer over bounded chunks with one reused workspace."""
    T = x.shape[0]
    _need(x, "x", torch.bfloat16, (T, layer.d))
    _need(logits, "logits", torch.float32, (T, layer.E))
    y = torch.empty((T, layer.d), dtype=torch.float32, device=x.device) if y is None else y
    _need(y, "y", torch.float32, (T, layer.d))
    ws = alloc_workspace(workspace_bytes(min(chunk, max(T, 1)), layer), x.device) if ws is None else ws
    _check(load().moe_prefill_chunked(ctypes.byref(layer.c), x.data_ptr(), logits.data_ptr(), T,
                                      chunk, y.data_ptr(), ws.data_ptr(), ws.numel(),
                                      _stream(stream)), "moe_prefill_chunked")
    return y
