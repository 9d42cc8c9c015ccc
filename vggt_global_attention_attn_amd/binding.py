"""ctypes binding over libvggt_attn.so (the C ABI in include/vggt_attn.h).

Argument marshalling only: every step of the computation runs in the library's HIP kernels.
torch supplies device memory and the stream; nothing here computes attention.  If the shared
library is missing, every call raises -- there is no fallback path."""
from __future__ import annotations

import ctypes
import os

import numpy as np

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libvggt_attn.so")

BF16, FP32 = 0, 1
G2F, REF_DENSE, DIAG, MEAN, MEAN_COUNT, PRESCALE_Q = 1, 2, 4, 8, 16, 32
PHASE_SHIFT, MEAN_GLOBAL, G2M, LOG_SIZE = 64, 128, 256, 512

STATUS = {0: "OK", -1: "EINVAL", -2: "EUNSUPPORTED", -3: "ENOSPC", -4: "EALIGN", -5: "EALIAS", -6: "EHIP"}

EXPORTS = ("vggt_attn_plan", "vggt_attn_plan_destroy", "vggt_attn_workspace_bytes", "vggt_attn_counts",
           "vggt_attn_layout", "vggt_attn_forward", "vggt_attn_pack", "vggt_attn_attend",
           "vggt_attn_forward_sized", "vggt_attn_pack_sized", "vggt_attn_forward_noalloc", "vggt_attn_copy_index_set",
           "vggt_attn_layer_schedule", "vggt_attn_last_error")
MODELS = {"vggt": 0, "pi3": 1}
GLOBAL_LAYERS = 24


class VggtAttnError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"{STATUS.get(code, code)}: {message}")
        self.code = code
        self.status = STATUS.get(code, str(code))


class Layout(ctypes.Structure):
    _fields_ = [(name, ctypes.c_int64) for name in (
        "segments", "segment_rows", "keys_per_segment", "off_index", "off_dcount", "off_means",
        "off_partial", "off_kbias", "off_logsize", "off_part", "split_pieces", "off_kmax", "off_kpack", "off_vpack",
        "total_bytes")]

    def as_dict(self) -> dict:
        return {name: int(getattr(self, name)) for name, _ in self._fields_}


_lib = None


def lib() -> ctypes.CDLL:
    """Load the shared library (once); raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m vggt_global_attention_attn_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    vp, i64p = ctypes.c_void_p, ctypes.POINTER(ctypes.c_int64)
    L.vggt_attn_plan.argtypes = [ctypes.POINTER(vp)] + [ctypes.c_int] * 7 + [ctypes.c_uint, ctypes.c_int, ctypes.c_int]
    L.vggt_attn_plan.restype = ctypes.c_int
    L.vggt_attn_plan_destroy.argtypes = [vp]
    L.vggt_attn_plan_destroy.restype = None
    L.vggt_attn_workspace_bytes.argtypes = [vp]
    L.vggt_attn_workspace_bytes.restype = ctypes.c_size_t
    L.vggt_attn_counts.argtypes = [vp, i64p, i64p, i64p, ctypes.POINTER(ctypes.c_double)]
    L.vggt_attn_counts.restype = ctypes.c_int
    L.vggt_attn_layout.argtypes = [vp, ctypes.POINTER(Layout)]
    L.vggt_attn_layout.restype = ctypes.c_int
    L.vggt_attn_forward.argtypes = [vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    L.vggt_attn_forward.restype = ctypes.c_int
    L.vggt_attn_pack.argtypes = [vp, vp, vp, vp, ctypes.c_size_t, vp]
    L.vggt_attn_pack.restype = ctypes.c_int
    L.vggt_attn_attend.argtypes = [vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    L.vggt_attn_attend.restype = ctypes.c_int
    L.vggt_attn_forward_sized.argtypes = [vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    L.vggt_attn_forward_sized.restype = ctypes.c_int
    L.vggt_attn_pack_sized.argtypes = [vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    L.vggt_attn_pack_sized.restype = ctypes.c_int
    L.vggt_attn_forward_noalloc.argtypes = [vp, vp, vp, vp, vp, vp]
    L.vggt_attn_forward_noalloc.restype = ctypes.c_int
    L.vggt_attn_layer_schedule.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.POINTER(ctypes.c_int),
                                           ctypes.POINTER(ctypes.c_uint)]
    L.vggt_attn_layer_schedule.restype = ctypes.c_int
    L.vggt_attn_copy_index_set.argtypes = [vp, vp, ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int32), vp]
    L.vggt_attn_copy_index_set.restype = ctypes.c_int
    L.vggt_attn_last_error.argtypes = []
    L.vggt_attn_last_error.restype = ctypes.c_char_p
    _lib = L
    return L


def _check(rc: int) -> None:
    if rc != 0:
        raise VggtAttnError(rc, lib().vggt_attn_last_error().decode())


def _dtype_code(name: str) -> int:
    if name in ("bf16", "bfloat16"):
        return BF16
    if name in ("fp32", "float32"):
        return FP32
    raise ValueError(f"dtype must be 'bf16' or 'fp32', got {name!r}")


def _stream_handle(stream, device=None):
    if stream is None:
        import torch
        return torch.cuda.current_stream(device).cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _ptr(t) -> int:
    return 0 if t is None else int(t.data_ptr())


class Plan:
    """An immutable description of one global-attention call (see include/vggt_attn.h)."""

    def __init__(self, frames: int, grid_h: int, grid_w: int, heads: int, head_dim: int = 64,
                 n_special: int = 5, sigma: int = 1, ref_dense: bool = True, diag: bool = False,
                 mean: bool = False, mean_count: bool = False, g2f: bool = False,
                 in_dtype: str = "bf16", out_dtype: str = "fp32", prescale_q: bool = False,
                 phase_shift: bool = False, mean_global: bool = False, g2m: bool = False,
                 log_size: bool = False, flags: int | None = None):
        if flags is None:
            flags = ((G2F if g2f else 0) | (REF_DENSE if ref_dense else 0) | (DIAG if diag else 0) |
                     (MEAN if mean else 0) | (MEAN_COUNT if mean_count else 0) |
                     (PRESCALE_Q if prescale_q else 0) | (PHASE_SHIFT if phase_shift else 0) |
                     (MEAN_GLOBAL if mean_global else 0) | (G2M if g2m else 0) | (LOG_SIZE if log_size else 0))
        self._h = ctypes.c_void_p()
        self.frames, self.grid_h, self.grid_w, self.heads, self.head_dim = frames, grid_h, grid_w, heads, head_dim
        self.n_special, self.sigma, self.flags = n_special, sigma, flags
        self.in_dtype, self.out_dtype = in_dtype, out_dtype
        _check(lib().vggt_attn_plan(ctypes.byref(self._h), frames, grid_h, grid_w, n_special, heads, head_dim,
                                    sigma, flags, _dtype_code(in_dtype), _dtype_code(out_dtype)))
        self.L = n_special + grid_h * grid_w
        self.T = frames * self.L

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value and _lib is not None:
            _lib.vggt_attn_plan_destroy(h)
            self._h = None

    @property
    def handle(self) -> ctypes.c_void_p:
        return self._h

    @property
    def workspace_bytes(self) -> int:
        return int(lib().vggt_attn_workspace_bytes(self._h))

    def counts(self) -> dict:
        n_kv, n_mean, n_diag = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
        flops = ctypes.c_double()
        _check(lib().vggt_attn_counts(self._h, ctypes.byref(n_kv), ctypes.byref(n_mean), ctypes.byref(n_diag),
                                      ctypes.byref(flops)))
        return {"n_kv": n_kv.value, "n_mean": n_mean.value, "n_diag": n_diag.value, "flops": flops.value}

    def layout(self) -> dict:
        lay = Layout()
        _check(lib().vggt_attn_layout(self._h, ctypes.byref(lay)))
        return lay.as_dict()

    # -- device calls (torch tensors for memory, a torch stream or raw handle for ordering) --

    def _check_tensor(self, t, name: str, dtype_name: str) -> None:
        import torch
        want = torch.bfloat16 if dtype_name == "bf16" else torch.float32
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
        if t.dtype != want:
            raise ValueError(f"{name} must be {want}, got {t.dtype}")
        if tuple(t.shape) != (self.heads, self.T, self.head_dim) or not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous [{self.heads}, {self.T}, {self.head_dim}], got {tuple(t.shape)}")

    def _check_ws(self, ws) -> None:
        if not ws.is_cuda or not ws.is_contiguous():
            raise ValueError("workspace must be a contiguous GPU tensor")

    def new_workspace(self, device="cuda"):
        import torch
        return torch.empty(max(1, self.workspace_bytes), dtype=torch.uint8, device=device)

    def new_output(self, device="cuda"):
        import torch
        dt = torch.bfloat16 if self.out_dtype == "bf16" else torch.float32
        return torch.empty((self.heads, self.T, self.head_dim), dtype=dt, device=device)

    def forward(self, q, k, v, out, workspace, stream=None) -> None:
        for t, n in ((q, "q"), (k, "k"), (v, "v")):
            self._check_tensor(t, n, self.in_dtype)
        self._check_tensor(out, "out", self.out_dtype)
        self._check_ws(workspace)
        _check(lib().vggt_attn_forward(self._h, _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(workspace),
                                       workspace.numel() * workspace.element_size(),
                                       _stream_handle(stream, q.device)))

    def forward_noalloc(self, q, k, v, out, stream=None) -> None:
        """vggt_attn_forward on the library's static per-GPU workspace (no workspace argument)."""
        for t, n in ((q, "q"), (k, "k"), (v, "v")):
            self._check_tensor(t, n, self.in_dtype)
        self._check_tensor(out, "out", self.out_dtype)
        _check(lib().vggt_attn_forward_noalloc(self._h, _ptr(q), _ptr(k), _ptr(v), _ptr(out),
                                               _stream_handle(stream, q.device)))

    def _check_log_g(self, log_g) -> None:
        import torch
        if log_g is None:
            raise ValueError("this plan has LOG_SIZE: pass log_g")
        if not log_g.is_cuda or log_g.dtype != torch.float32 or tuple(log_g.shape) != (self.T,) \
                or not log_g.is_contiguous():
            raise ValueError(f"log_g must be a contiguous float32 GPU tensor of shape [{self.T}]")

    def forward_sized(self, q, k, v, log_g, out, workspace, stream=None) -> None:
        for t, n in ((q, "q"), (k, "k"), (v, "v")):
            self._check_tensor(t, n, self.in_dtype)
        self._check_tensor(out, "out", self.out_dtype)
        self._check_ws(workspace)
        self._check_log_g(log_g)
        _check(lib().vggt_attn_forward_sized(self._h, _ptr(q), _ptr(k), _ptr(v), _ptr(log_g), _ptr(out),
                                             _ptr(workspace), workspace.numel() * workspace.element_size(),
                                             _stream_handle(stream, q.device)))

    def pack_sized(self, k, v, log_g, workspace, stream=None) -> None:
        for t, n in ((k, "k"), (v, "v")):
            self._check_tensor(t, n, self.in_dtype)
        self._check_ws(workspace)
        self._check_log_g(log_g)
        _check(lib().vggt_attn_pack_sized(self._h, _ptr(k), _ptr(v), _ptr(log_g), _ptr(workspace),
                                          workspace.numel() * workspace.element_size(), _stream_handle(stream, k.device)))

    def pack(self, k, v, workspace, stream=None) -> None:
        for t, n in ((k, "k"), (v, "v")):
            self._check_tensor(t, n, self.in_dtype)
        self._check_ws(workspace)
        _check(lib().vggt_attn_pack(self._h, _ptr(k), _ptr(v), _ptr(workspace),
                                    workspace.numel() * workspace.element_size(), _stream_handle(stream, k.device)))

    def attend(self, q, k, v, out, workspace, stream=None) -> None:
        for t, n in ((q, "q"), (k, "k"), (v, "v")):
            self._check_tensor(t, n, self.in_dtype)
        self._check_tensor(out, "out", self.out_dtype)
        self._check_ws(workspace)
        _check(lib().vggt_attn_attend(self._h, _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(workspace),
                                      workspace.numel() * workspace.element_size(),
                                      _stream_handle(stream, q.device)))

    def index_set(self, workspace, stream=None):
        """(S as int32 token ids, |D_f| per frame) copied from a packed workspace."""
        c = self.counts()
        g2f = bool(self.flags & G2F)
        idx = np.zeros(0 if g2f else c["n_kv"], dtype=np.int32)  # n_kv is 0 under G2M
        dcount = np.zeros(self.frames, dtype=np.int32)
        i32p = ctypes.POINTER(ctypes.c_int32)
        _check(lib().vggt_attn_copy_index_set(
            self._h, _ptr(workspace), idx.ctypes.data_as(i32p) if idx.size else None,
            dcount.ctypes.data_as(i32p), _stream_handle(stream, workspace.device)))
        return idx, dcount


def layer_schedule(model: str = "vggt", sigma: int = 9) -> list:
    """The plan keyword arguments (sigma and form flags) of each of the 24 global layers under
    AVGGT's schedule, as vggt_attn_layer_schedule gives them; combine each with the geometry
    (frames, grid_h, grid_w, heads) to build that layer's Plan."""
    L = lib()
    out = []
    for layer in range(GLOBAL_LAYERS):
        s, f = ctypes.c_int(), ctypes.c_uint()
        _check(L.vggt_attn_layer_schedule(MODELS[model], layer, sigma, ctypes.byref(s), ctypes.byref(f)))
        fl = f.value
        out.append(dict(sigma=s.value, g2f=bool(fl & G2F), ref_dense=bool(fl & REF_DENSE), diag=bool(fl & DIAG),
                        mean=bool(fl & MEAN)))
    return out


class ScheduledLayers:
    """The global layers of one model run under AVGGT's schedule on one geometry: the distinct
    plans (G2F, SGA sigma with the diagonal and mean terms, dense) built once and shared by the
    layers that use them, with a workspace each.  forward(layer, ...) runs that layer's form."""

    def __init__(self, frames: int, grid_h: int, grid_w: int, heads: int, model: str = "vggt", sigma: int = 9,
                 n_special: int = 5, in_dtype: str = "bf16", out_dtype: str = "fp32", device="cuda"):
        self.kinds = layer_schedule(model, sigma)
        self.plans, self.workspaces, self.index = [], [], []
        seen = {}
        for kw in self.kinds:
            key = tuple(sorted(kw.items()))
            if key not in seen:
                seen[key] = len(self.plans)
                self.plans.append(Plan(frames, grid_h, grid_w, heads, n_special=n_special, in_dtype=in_dtype,
                                       out_dtype=out_dtype, **kw))
                self.workspaces.append(None)
            self.index.append(seen[key])
        self.device = device

    def plan(self, layer: int) -> Plan:
        return self.plans[self.index[layer]]

    def forward(self, layer: int, q, k, v, out, stream=None) -> None:
        i = self.index[layer]
        if self.workspaces[i] is None:
            self.workspaces[i] = self.plans[i].new_workspace(self.device)
        self.plans[i].forward(q, k, v, out, self.workspaces[i], stream)

    def flops(self) -> float:
        """Algorithmic FLOPs of one pass over the 24 layers."""
        return sum(self.plan(layer).counts()["flops"] for layer in range(GLOBAL_LAYERS))


def attention(q, k, v, plan: Plan, stream=None, log_g=None):
    """Allocate out and a workspace with torch, run one forward, return out."""
    out = plan.new_output(q.device)
    ws = plan.new_workspace(q.device)
    if plan.flags & LOG_SIZE:
        plan.forward_sized(q, k, v, log_g, out, ws, stream)
    else:
        plan.forward(q, k, v, out, ws, stream)
    return out
