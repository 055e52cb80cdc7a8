"""Python binding of libw4a4 (W4A4 linear layer with fused LoRA, gfx950).

Argument marshalling only: every step of the layer runs in the HIP kernels of
``libw4a4.so``.  PyTorch supplies device memory and the current stream.
There is no fallback: if the library is missing, importing the binding's
entry points raises.

Names follow the C ABI in ``include/w4a4.h``::

    w4a4_weight_layout(N, K, R)          -> (total_bytes, offsets[6])
    w4a4_act_layout(M, K, R)             -> (total_bytes, offsets[3][, lora splits])
    w4a4_pack_weights(N, K, R, wblob, w_fp16=..., or qweight=..., w_scales=...,
                      lora_down=..., lora_up=..., col_scale=..., bias=...)
    w4a4_quantize_act(M, K, R, x, wblob, act)
    w4a4_linear(M, N, K, R, act, wblob, y)
    w4a4_query_variant(M, N, K, R)
    w4a4_debug_group_psums(M, N, K, R, act, wblob, m0, mc, n0, nc, out)
    w4a4_debug_group_psums_glu(M, N, K, R, act, wblob, m0, mc, n0, nc, out)

plus helpers that allocate the blobs as uint8 CUDA tensors.
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "W4A4Error", "lib_path", "load_library", "w4a4_status_string",
    "w4a4_weight_layout", "w4a4_act_layout", "w4a4_pack_weights",
    "w4a4_quantize_act", "w4a4_quantize_act_rmsnorm", "w4a4_linear", "w4a4_linear_glu",
    "w4a4_linear_glu_quant", "w4a4_glu_quant_workspace", "w4a4_linear_glu_quant_noalloc",
    "w4a4_query_variant", "GatedMLPUp", "GatedMLP",
    "w4a4_debug_group_psums", "w4a4_debug_group_psums_glu", "alloc_weight_blob", "alloc_act_blob",
    "PackedLinear", "LayerGraphs", "EXPORTED_SYMBOLS", "PEAKS_SYMBOLS", "load_peaks_library",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
EXPORTED_SYMBOLS = (
    "w4a4_status_string", "w4a4_weight_layout", "w4a4_act_layout",
    "w4a4_pack_weights", "w4a4_quantize_act", "w4a4_quantize_act_rmsnorm", "w4a4_linear",
    "w4a4_linear_glu", "w4a4_linear_glu_quant", "w4a4_glu_quant_workspace", "w4a4_linear_glu_quant_noalloc",
    "w4a4_query_variant",
    "w4a4_debug_group_psums",
    "w4a4_debug_group_psums_glu", "w4a4_graph_begin", "w4a4_graph_end", "w4a4_layer_graph_create", "w4a4_graph_launch",
    "w4a4_graph_destroy",
)


class W4A4Error(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {w4a4_status_string(status)} (status {status})")
        self.status = status


def lib_path() -> str:
    return os.path.join(_HERE, "libw4a4.so")


# The measurement library (include/w4a4_peaks.h): microbenchmarks of the
# attainable int8 MFMA and HBM read peaks, used by the benchmark only.
PEAKS_SYMBOLS = ("w4a4_peak_i8_mfma", "w4a4_peak_i8_mfma_ops", "w4a4_peak_i8_mfma_out_ints",
                 "w4a4_peak_hbm_read", "w4a4_peak_hbm_read_out_ints", "w4a4_peak_roles", "w4a4_peak_roles_ops",
                 "w4a4_peak_roles_out_ints")
_PEAKS = None


def load_peaks_library() -> ctypes.CDLL:
    """libw4a4_peaks.so from the package directory (after torch, like
    load_library); raises if it is not built."""
    global _PEAKS
    if _PEAKS is not None:
        return _PEAKS
    path = os.path.join(_HERE, "libw4a4_peaks.so")
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built; run `python -m w4a4_gemm_lora_amd.build`")
    import torch  # noqa: F401
    lib = ctypes.CDLL(path)
    lib.w4a4_peak_i8_mfma.argtypes = [ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
    lib.w4a4_peak_i8_mfma.restype = ctypes.c_int
    lib.w4a4_peak_i8_mfma_ops.argtypes = [ctypes.c_int32]
    lib.w4a4_peak_i8_mfma_ops.restype = ctypes.c_int64
    lib.w4a4_peak_i8_mfma_out_ints.argtypes = []
    lib.w4a4_peak_i8_mfma_out_ints.restype = ctypes.c_int64
    lib.w4a4_peak_hbm_read.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_void_p]
    lib.w4a4_peak_hbm_read.restype = ctypes.c_int
    lib.w4a4_peak_hbm_read_out_ints.argtypes = []
    lib.w4a4_peak_hbm_read_out_ints.restype = ctypes.c_int64
    lib.w4a4_peak_roles.argtypes = [ctypes.c_int32] * 4 + [ctypes.c_void_p, ctypes.c_void_p]
    lib.w4a4_peak_roles.restype = ctypes.c_int
    lib.w4a4_peak_roles_ops.argtypes = [ctypes.c_int32, ctypes.c_int32]
    lib.w4a4_peak_roles_ops.restype = ctypes.c_int64
    lib.w4a4_peak_roles_out_ints.argtypes = []
    lib.w4a4_peak_roles_out_ints.restype = ctypes.c_int64
    _PEAKS = lib
    return lib


_LIB = None

_i64, _i32, _vp, _sz = ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_size_t


def load_library() -> ctypes.CDLL:
    """Load libw4a4.so from the package directory (raises if it is not built).

    torch is imported first: its bundled HIP runtime then satisfies the
    library's libamdhip64 dependency, so the process holds one HIP runtime
    and the library sees torch's devices, memory and streams.  Loaded before
    torch, the library would pull in the system runtime as a second copy,
    which finds no device once torch's copy has opened the GPU."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = lib_path()
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built; run `python -m w4a4_gemm_lora_amd.build`")
    import torch  # noqa: F401  (binds the library to torch's HIP runtime)
    lib = ctypes.CDLL(path)
    lib.w4a4_status_string.restype = ctypes.c_char_p
    lib.w4a4_status_string.argtypes = [ctypes.c_int]
    lib.w4a4_weight_layout.argtypes = [_i64, _i64, _i32, ctypes.POINTER(_sz), ctypes.POINTER(_sz)]
    lib.w4a4_act_layout.argtypes = [_i64, _i64, _i32, ctypes.POINTER(_sz), ctypes.POINTER(_sz),
                                    ctypes.POINTER(ctypes.c_int32)]
    lib.w4a4_pack_weights.argtypes = [_i64, _i64, _i32] + [_vp] * 9
    lib.w4a4_quantize_act.argtypes = [_i64, _i64, _i32, _vp, _i64, _vp, _vp, _vp]
    lib.w4a4_quantize_act_rmsnorm.argtypes = [_i64, _i64, _i32, _vp, _i64, _vp, ctypes.c_double,
                                              _vp, _vp, _vp]
    lib.w4a4_linear.argtypes = [_i64, _i64, _i64, _i32, _vp, _vp, _vp, _i64, _vp]
    lib.w4a4_linear_glu.argtypes = [_i64, _i64, _i64, _i32, _i32, _vp, _vp, _vp, _i64, _vp]
    lib.w4a4_linear_glu_quant.argtypes = [_i64, _i64, _i64, _i32, _i32, _vp, _vp, _i32, _vp, _vp, _vp, _vp]
    lib.w4a4_glu_quant_workspace.argtypes = [_i64, _i64, _i32, ctypes.POINTER(_sz)]
    lib.w4a4_linear_glu_quant_noalloc.argtypes = [_i64, _i64, _i64, _i32, _i32, _vp, _vp, _i32, _vp, _vp, _vp]
    lib.w4a4_query_variant.argtypes = [_i64, _i64, _i64, _i32]
    lib.w4a4_layer_graph_create.argtypes = [_i64, _i64, _i64, _i32, _vp, _i64, _vp, ctypes.c_double,
                                            _vp, _vp, _vp, _i64, ctypes.POINTER(_vp)]
    lib.w4a4_graph_begin.argtypes = [_vp]
    lib.w4a4_graph_end.argtypes = [_vp, ctypes.POINTER(_vp)]
    lib.w4a4_graph_launch.argtypes = [_vp, _vp]
    lib.w4a4_graph_destroy.argtypes = [_vp]
    lib.w4a4_debug_group_psums.argtypes = [_i64, _i64, _i64, _i32, _vp, _vp, _i64, _i64, _i64, _i64, _vp, _vp]
    lib.w4a4_debug_group_psums_glu.argtypes = lib.w4a4_debug_group_psums.argtypes
    for name in EXPORTED_SYMBOLS:
        if name != "w4a4_status_string":
            getattr(lib, name).restype = ctypes.c_int
    _LIB = lib
    return lib


def w4a4_status_string(status: int) -> str:
    return load_library().w4a4_status_string(int(status)).decode()


def _check(status: int, what: str):
    if status != 0:
        raise W4A4Error(status, what)


def _ptr(t):
    """Device pointer of a tensor (or None)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_cuda:
        raise ValueError("device tensors are required")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return t.data_ptr()


def _stream(stream):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


# ---- host-only queries -------------------------------------------------------
def w4a4_weight_layout(N: int, K: int, R: int):
    lib = load_library()
    tot = _sz()
    offs = (_sz * 6)()
    _check(lib.w4a4_weight_layout(N, K, R, ctypes.byref(tot), offs), "w4a4_weight_layout")
    return tot.value, list(offs)


def w4a4_act_layout(M: int, K: int, R: int, with_splits: bool = False):
    """(total_bytes, offsets[3]) or, with_splits=True, (total, offsets, S)
    where S is the number of LoRA-down partial sums in section [2]."""
    lib = load_library()
    tot = _sz()
    offs = (_sz * 3)()
    ks = ctypes.c_int32()
    _check(lib.w4a4_act_layout(M, K, R, ctypes.byref(tot), offs, ctypes.byref(ks)), "w4a4_act_layout")
    if with_splits:
        return tot.value, list(offs), ks.value
    return tot.value, list(offs)


def w4a4_query_variant(M: int, N: int, K: int, R: int) -> int:
    v = load_library().w4a4_query_variant(M, N, K, R)
    if v < 0:
        raise W4A4Error(-v, "w4a4_query_variant")
    return v


# ---- device calls -------------------------------------------------------------
def w4a4_pack_weights(N, K, R, wblob, w_fp16=None, qweight=None, w_scales=None,
                      lora_down=None, lora_up=None, col_scale=None, bias=None, stream=None):
    st = load_library().w4a4_pack_weights(
        N, K, R, _ptr(w_fp16), _ptr(qweight), _ptr(w_scales), _ptr(lora_down),
        _ptr(lora_up), _ptr(col_scale), _ptr(bias), _ptr(wblob), _stream(stream))
    _check(st, "w4a4_pack_weights")


def w4a4_quantize_act(M, K, R, x, wblob, act, ldx=None, stream=None):
    ldx = K if ldx is None else ldx
    st = load_library().w4a4_quantize_act(M, K, R, _ptr(x), ldx, _ptr(wblob), _ptr(act), _stream(stream))
    _check(st, "w4a4_quantize_act")


def w4a4_quantize_act_rmsnorm(M, K, R, x, gamma, eps, wblob, act, ldx=None, stream=None):
    ldx = K if ldx is None else ldx
    st = load_library().w4a4_quantize_act_rmsnorm(M, K, R, _ptr(x), ldx, _ptr(gamma), float(eps),
                                                  _ptr(wblob), _ptr(act), _stream(stream))
    _check(st, "w4a4_quantize_act_rmsnorm")


def w4a4_linear(M, N, K, R, act, wblob, y, ldy=None, stream=None):
    ldy = N if ldy is None else ldy
    st = load_library().w4a4_linear(M, N, K, R, _ptr(act), _ptr(wblob), _ptr(y), ldy, _stream(stream))
    _check(st, "w4a4_linear")


def w4a4_linear_glu(M, N, K, R, r_gate, act, wblob, y, ldy=None, stream=None):
    ldy = N // 2 if ldy is None else ldy
    st = load_library().w4a4_linear_glu(M, N, K, R, r_gate, _ptr(act), _ptr(wblob), _ptr(y), ldy,
                                        _stream(stream))
    _check(st, "w4a4_linear_glu")


def w4a4_glu_quant_workspace(M, N, R_down):
    """Bytes of workspace w4a4_linear_glu_quant needs (host-only)."""
    n = _sz()
    _check(load_library().w4a4_glu_quant_workspace(M, N, R_down, ctypes.byref(n)), "w4a4_glu_quant_workspace")
    return n.value


def w4a4_linear_glu_quant(M, N, K, R, r_gate, act, wblob, R_down, down_wblob, act_out, workspace,
                          stream=None):
    st = load_library().w4a4_linear_glu_quant(M, N, K, R, r_gate, _ptr(act), _ptr(wblob), R_down,
                                              _ptr(down_wblob), _ptr(act_out), _ptr(workspace),
                                              _stream(stream))
    _check(st, "w4a4_linear_glu_quant")


# Bytes of the library-owned array w4a4_linear_glu_quant_noalloc uses per GPU
NOALLOC_SCRATCH_BYTES = 32 << 20


def w4a4_linear_glu_quant_noalloc(M, N, K, R, r_gate, act, wblob, R_down, down_wblob, act_out, stream=None):
    st = load_library().w4a4_linear_glu_quant_noalloc(M, N, K, R, r_gate, _ptr(act), _ptr(wblob), R_down,
                                                      _ptr(down_wblob), _ptr(act_out), _stream(stream))
    _check(st, "w4a4_linear_glu_quant_noalloc")


def w4a4_debug_group_psums(M, N, K, R, act, wblob, m0, mc, n0, nc, out, stream=None):
    st = load_library().w4a4_debug_group_psums(M, N, K, R, _ptr(act), _ptr(wblob), m0, mc, n0, nc,
                                               _ptr(out), _stream(stream))
    _check(st, "w4a4_debug_group_psums")


def w4a4_debug_group_psums_glu(M, N, K, R, act, wblob, m0, mc, n0, nc, out, stream=None):
    st = load_library().w4a4_debug_group_psums_glu(M, N, K, R, _ptr(act), _ptr(wblob), m0, mc, n0, nc,
                                                   _ptr(out), _stream(stream))
    _check(st, "w4a4_debug_group_psums_glu")


# ---- allocation helpers (torch owns the memory) ------------------------------
def alloc_weight_blob(N, K, R, device="cuda"):
    import torch
    total, _ = w4a4_weight_layout(N, K, R)
    return torch.empty(total, dtype=torch.uint8, device=device)


def alloc_act_blob(M, K, R, device="cuda"):
    import torch
    total, _ = w4a4_act_layout(M, K, R)
    return torch.empty(total, dtype=torch.uint8, device=device)


class PackedLinear:
    """One packed layer: holds the weight blob and runs the two forward calls
    (quantize_act, then linear) on the current stream."""

    def __init__(self, N, K, R, w_fp16=None, qweight=None, w_scales=None,
                 lora_down=None, lora_up=None, col_scale=None, bias=None):
        self.N, self.K, self.R = int(N), int(K), int(R)
        self.wblob = alloc_weight_blob(self.N, self.K, self.R, device=(
            w_fp16 if w_fp16 is not None else qweight).device)
        w4a4_pack_weights(self.N, self.K, self.R, self.wblob, w_fp16=w_fp16, qweight=qweight,
                          w_scales=w_scales, lora_down=lora_down, lora_up=lora_up,
                          col_scale=col_scale, bias=bias)

    def forward(self, x, act=None, y=None):
        import torch
        M = x.shape[0]
        if act is None:
            act = alloc_act_blob(M, self.K, self.R, device=x.device)
        if y is None:
            y = torch.empty((M, self.N), dtype=torch.float16, device=x.device)
        w4a4_quantize_act(M, self.K, self.R, x, self.wblob, act)
        w4a4_linear(M, self.N, self.K, self.R, act, self.wblob, y)
        return y


def interleave_gate_up(gate, up, tile=16):
    """Rows of two [N, ...] tensors interleaved by 16-row tiles: rows
    [32j, 32j+16) from gate, [32j+16, 32j+32) from up (the layout
    w4a4_linear_glu pairs)."""
    import torch
    n = gate.shape[0]
    g = gate.reshape(n // tile, tile, *gate.shape[1:])
    u = up.reshape(n // tile, tile, *up.shape[1:])
    return torch.stack([g, u], dim=1).reshape(2 * n, *gate.shape[1:]).contiguous()


class GatedMLPUp:
    """The gate and up projections of a gated MLP packed as one layer, with
    the gated activation SiLU(gate) * up applied in the GEMM epilogue
    (w4a4_linear_glu).  One activation pass (w4a4_quantize_act, with the two
    layers' L_down side by side) serves both projections.  forward(x)
    returns h = fp16(SiLU(g) * u), [M, N]."""

    def __init__(self, N, K, w_gate, w_up, lora_down_gate=None, lora_up_gate=None,
                 lora_down_up=None, lora_up_up=None, a_gate=None, b_gate=None, a_up=None, b_up=None):
        import torch
        self.N, self.K = int(N), int(K)
        if self.N % 16 or self.N <= 0:
            raise ValueError("each projection needs a positive multiple of 16 columns")
        if (lora_down_gate is None) != (lora_up_gate is None) or (lora_down_up is None) != (lora_up_up is None):
            raise ValueError("give both LoRA factors of a projection, or neither")
        dev = w_gate.device
        rg = 0 if lora_down_gate is None else lora_down_gate.shape[1]
        ru = 0 if lora_down_up is None else lora_down_up.shape[1]
        self.R = rg + ru
        self.r_gate = rg
        ld = lu = None
        if self.R:
            parts = [t for t in (lora_down_gate, lora_down_up) if t is not None]
            ld = torch.cat(parts, dim=1).contiguous()
            lug = torch.zeros((self.N, self.R), dtype=torch.float16, device=dev)
            luu = torch.zeros((self.N, self.R), dtype=torch.float16, device=dev)
            if rg:
                lug[:, :rg] = lora_up_gate
            if ru:
                luu[:, rg:] = lora_up_up
            lu = interleave_gate_up(lug, luu)
        ones = torch.ones(self.N, dtype=torch.float32, device=dev)
        zeros = torch.zeros(self.N, dtype=torch.float32, device=dev)
        a = interleave_gate_up(ones if a_gate is None else a_gate, ones if a_up is None else a_up)
        b = interleave_gate_up(zeros if b_gate is None else b_gate, zeros if b_up is None else b_up)
        w = interleave_gate_up(w_gate, w_up)
        self.wblob = alloc_weight_blob(2 * self.N, self.K, self.R, device=dev)
        w4a4_pack_weights(2 * self.N, self.K, self.R, self.wblob, w_fp16=w, lora_down=ld, lora_up=lu,
                          col_scale=a, bias=b)

    def forward(self, x, act=None, h=None, stream=None):
        import torch
        M = x.shape[0]
        if act is None:
            act = alloc_act_blob(M, self.K, self.R, device=x.device)
        if h is None:
            h = torch.empty((M, self.N), dtype=torch.float16, device=x.device)
        w4a4_quantize_act(M, self.K, self.R, x, self.wblob, act, stream=stream)
        w4a4_linear_glu(M, 2 * self.N, self.K, self.R, self.r_gate, act, self.wblob, h, stream=stream)
        return h


class GatedMLP:
    """A whole gated MLP: gate and up projections packed as one layer
    (GatedMLPUp) and the down projection (PackedLinear with K = the up
    layer's N).  forward(x) runs the activation pass of x, then the gated
    GEMM with its output quantized straight into the down layer's
    activation blob (w4a4_linear_glu_quant: h never goes to memory in fp16
    for M > 16), then the down GEMM; returns y [M, down.N]."""

    def __init__(self, up: "GatedMLPUp", down: PackedLinear):
        if down.K != up.N or up.N % 128:
            raise ValueError("the down projection's K must be the up layer's N, a multiple of 128")
        self.up, self.down = up, down

    def buffers(self, M, device="cuda"):
        """(act, act_h, workspace, y) for M rows."""
        import torch
        ws = w4a4_glu_quant_workspace(M, 2 * self.up.N, self.down.R)
        return (alloc_act_blob(M, self.up.K, self.up.R, device=device),
                alloc_act_blob(M, self.up.N, self.down.R, device=device),
                torch.empty(max(ws, 256), dtype=torch.uint8, device=device),
                torch.empty((M, self.down.N), dtype=torch.float16, device=device))

    def forward(self, x, bufs=None, stream=None):
        M = x.shape[0]
        act, act_h, ws, y = self.buffers(M, device=x.device) if bufs is None else bufs
        u, d = self.up, self.down
        w4a4_quantize_act(M, u.K, u.R, x, u.wblob, act, stream=stream)
        w4a4_linear_glu_quant(M, 2 * u.N, u.K, u.R, u.r_gate, act, u.wblob, d.R, d.wblob if d.R else None,
                              act_h, ws, stream=stream)
        w4a4_linear(M, d.N, d.K, d.R, act_h, d.wblob, y, stream=stream)
        return y


class LayerGraphs:
    """Bucketed replay of a chain of packed layers from native HIP graphs
    ("W4A4 CUDA Kernel for Voice Clone", section 4.3: pre-capture one graph
    per bucket, pad each request to the nearest bucket, copy the data in,
    replay).

    layers: one PackedLinear or a list whose shapes chain (layer i's N is
    layer i+1's K; layer i+1 reads layer i's output).  For every bucket size
    B the whole chain -- each layer's activation pass and GEMM -- is captured
    into one graph (w4a4_graph_begin / w4a4_graph_end on a side stream) over
    buffers sized for B rows.  run(x) copies the request's M rows into the
    smallest bucket with B >= M (rows past M are zeros), replays that graph
    on the current stream and returns a view of the last layer's first M
    output rows (valid until the next run on the same bucket).  gamma/eps:
    the first layer's activation pass is the fused RMSNorm variant.

    One graph per chain rather than per layer: a graph launch costs more
    than the two kernel launches it would replace (measured), so graphs pay
    when they hold many layers."""

    def __init__(self, layers, buckets, gamma=None, eps=1e-6, device="cuda"):
        import torch
        self.layers = list(layers) if isinstance(layers, (list, tuple)) else [layers]
        for a_, b_ in zip(self.layers, self.layers[1:]):
            if a_.N != b_.K:
                raise ValueError("layer shapes do not chain")
        self.buckets = sorted(int(b) for b in buckets)
        self.gamma, self.eps = gamma, float(eps)
        self._g = {}
        self._bufs = {}
        lib = load_library()
        side = torch.cuda.Stream(device=device)
        try:
            for B in self.buckets:
                x = torch.zeros((B, self.layers[0].K), dtype=torch.float16, device=device)
                acts = [alloc_act_blob(B, L.K, L.R, device=device) for L in self.layers]
                ys = [torch.empty((B, L.N), dtype=torch.float16, device=device) for L in self.layers]
                ss = side.cuda_stream
                torch.cuda.synchronize()
                _check(lib.w4a4_graph_begin(ss), "w4a4_graph_begin")
                try:
                    inp = x
                    for j, (L, act, y) in enumerate(zip(self.layers, acts, ys)):
                        if j == 0 and gamma is not None:
                            w4a4_quantize_act_rmsnorm(B, L.K, L.R, inp, gamma, self.eps, L.wblob, act, stream=ss)
                        else:
                            w4a4_quantize_act(B, L.K, L.R, inp, L.wblob, act, stream=ss)
                        w4a4_linear(B, L.N, L.K, L.R, act, L.wblob, y, stream=ss)
                        inp = y
                finally:
                    h = ctypes.c_void_p()
                    st = lib.w4a4_graph_end(ss, ctypes.byref(h))
                _check(st, "w4a4_graph_end")
                self._g[B] = h
                self._bufs[B] = (x, acts, ys)
        except Exception:
            self.close()
            raise

    def bucket_for(self, M):
        for B in self.buckets:
            if B >= M:
                return B
        raise ValueError(f"{M} rows exceed the largest bucket {self.buckets[-1]}")

    def run(self, x, stream=None):
        """Replay the bucket's graph for x on `stream` (default: the current
        stream).  The copy into the bucket buffer and the zeroing of its
        padding rows are enqueued on that same stream, ahead of the replay."""
        import torch
        M = x.shape[0]
        B = self.bucket_for(M)
        xb, _, ys = self._bufs[B]
        st = torch.cuda.current_stream() if stream is None else (
            stream if isinstance(stream, torch.cuda.Stream) else torch.cuda.ExternalStream(stream))
        if st != torch.cuda.current_stream():
            st.wait_stream(torch.cuda.current_stream())   # x was produced on the current stream
        with torch.cuda.stream(st):
            xb[:M].copy_(x)
            if M < B:
                xb[M:].zero_()
        _check(load_library().w4a4_graph_launch(self._g[B], st.cuda_stream), "w4a4_graph_launch")
        return ys[-1][:M]

    def close(self):
        lib = load_library()
        for h in self._g.values():
            lib.w4a4_graph_destroy(h)
        self._g = {}

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
