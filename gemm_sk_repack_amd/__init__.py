"""Python binding of libsk_repack.so: the skinny W4A8 / W6A8 linear for MI355X.

Argument marshalling only.  Every step of the computation runs in the HIP
kernels behind the C ABI declared in include/sk_repack.h; PyTorch is used for
device memory and streams.  If the shared library is missing the import of
this module fails: there is no CPU path.

Function names follow the C ABI: ``sk_repack_w4a8``, ``sk_unrepack_w4a8``,
``sk_gemm_w4a8``, ``sk_gemm_w6a8``, ``sk_gemm_fused_rmsnorm``,
``sk_gemm_fused_swiglu``, ``sk_debug_gemm`` (include/sk_repack.h),
``sk_kv_append``, ``sk_decode_attention``, ``sk_kv_pack_host``
(include/sk_attention.h) and the tree-MTP planner ``MtpPlanner`` over the
``sk_mtp_*`` calls (include/sk_mtp.h, host code).
"""

from __future__ import annotations

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libsk_repack.so")

SK_OK, SK_ERR_NULL, SK_ERR_SHAPE, SK_ERR_ALIGN, SK_ERR_FORMAT, SK_ERR_LAYOUT, SK_ERR_HIP, \
    SK_ERR_UNSUPPORTED, SK_ERR_WORKSPACE = range(9)
SK_F32, SK_BF16 = 0, 1
SK_W4_SYM, SK_W4_CODEBOOK, SK_W6_SYM = 0, 1, 2
SK_LAYOUT_CANONICAL, SK_LAYOUT_STREAM = 0, 1
PRO_NONE, PRO_RMSNORM, PRO_SWIGLU = 0, 1, 2
BITS = {SK_W4_SYM: 4, SK_W4_CODEBOOK: 4, SK_W6_SYM: 6}

# Every symbol include/sk_repack.h and include/sk_repack_test.h declare.
EXPORTS = ["sk_status_string", "sk_repack_w4a8", "sk_unrepack_w4a8", "sk_gemm_workspace_size",
           "sk_gemm_w4a8", "sk_gemm_w4a8_noalloc",
           "sk_gemm_w6a8", "sk_gemm_fused_rmsnorm", "sk_gemm_fused_swiglu",
           "sk_gemm_experts", "sk_quantize_rows", "sk_prologue_rmsnorm", "sk_prologue_swiglu",
           "sk_gemm_w4a8_canonical",
           "sk_gemm_w4a8_canonical_q",
           "sk_debug_gemm",
           "sk_test_repack_on_host", "sk_test_gemm_plan", "sk_test_set_split",
           "sk_test_set_spin_limit", "sk_test_stream_read",
           "sk_kv_append", "sk_decode_attention", "sk_attention_workspace_size", "sk_kv_pack_host",
           "sk_test_attention_plan", "sk_test_set_attention_split",
           "sk_mtp_create", "sk_mtp_destroy", "sk_mtp_observe", "sk_mtp_layout", "sk_mtp_layout_of",
           "sk_mtp_accept", "sk_mtp_expected_tokens", "sk_mtp_state"]


class SkWeightStruct(ctypes.Structure):
    _fields_ = [("n", ctypes.c_int32), ("k", ctypes.c_int32), ("group", ctypes.c_int32),
                ("format", ctypes.c_int32), ("layout", ctypes.c_int32),
                ("reserved", ctypes.c_int32), ("data", ctypes.c_void_p),
                ("bytes", ctypes.c_size_t), ("codebook", ctypes.c_void_p)]


class SkError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: status {status} ({status_string(status)})")


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with gemm_sk_repack_amd/build.py "
                          "(there is no fallback path)")
    lib = ctypes.CDLL(LIB_PATH)
    P, I, I64, F = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float
    W = ctypes.POINTER(SkWeightStruct)
    Z = ctypes.c_size_t
    ZP = ctypes.POINTER(ctypes.c_size_t)
    sig = {
        "sk_status_string": ([I], ctypes.c_char_p),
        "sk_repack_w4a8": ([W, P], I),
        "sk_unrepack_w4a8": ([W, P], I),
        "sk_gemm_workspace_size": ([I, I, I, I, I, I, ZP], I),
        "sk_gemm_w4a8": ([W, P, I, I, P, P, Z, P], I),
        "sk_gemm_w4a8_noalloc": ([W, P, I, I, P, P], I),
        "sk_gemm_w6a8": ([W, P, I, I, P, P, Z, P], I),
        "sk_gemm_fused_rmsnorm": ([W, P, I, P, F, I, P, P, Z, P], I),
        "sk_gemm_fused_swiglu": ([W, P, P, I64, I, I, P, P, Z, P], I),
        "sk_gemm_experts": ([W, I, P, I, P, I, I, P, P, Z, P], I),
        "sk_quantize_rows": ([P, I, I, I, P, P, P], I),
        "sk_prologue_rmsnorm": ([P, I, P, F, I, I, P, P], I),
        "sk_prologue_swiglu": ([P, P, I64, I, I, I, P, P], I),
        "sk_gemm_w4a8_canonical": ([W, P, I, I, P, P, Z, P], I),
        "sk_gemm_w4a8_canonical_q": ([W, P, P, I, P, P, Z, P], I),
        "sk_debug_gemm": ([W, I, P, P, I64, I, P, F, I, P, P, P, P, P, Z, P], I),
        "sk_test_repack_on_host": ([W, P, I], I),
        "sk_test_gemm_plan": ([I, I, I, I, I, I, I, ctypes.POINTER(ctypes.c_int64)], I),
        "sk_test_set_split": ([I], I),
        "sk_test_set_spin_limit": ([I], I),
        "sk_test_stream_read": ([P, I64, I, I, P, P], I),
        "sk_kv_append": ([P, I, I, I, I, P, P, P], I),
        "sk_decode_attention": ([P, I, I, I, P, I, I, F, P, P, Z, P], I),
        "sk_attention_workspace_size": ([I, I, I, I, ZP], I),
        "sk_kv_pack_host": ([P, P, I, I, I, P], I),
        "sk_test_attention_plan": ([I, I, I, I, I, ctypes.POINTER(I), ctypes.POINTER(I)], I),
        "sk_test_set_attention_split": ([I], I),
        "sk_mtp_create": ([ctypes.c_double, I, ctypes.c_double, ctypes.POINTER(P)], I),
        "sk_mtp_destroy": ([P], None),
        "sk_mtp_observe": ([P, P, I, ctypes.c_double, ctypes.c_double, P, P], I),
        "sk_mtp_layout": ([P, P, P, P], I),
        "sk_mtp_layout_of": ([I, P, P], I),
        "sk_mtp_accept": ([P, I, P, P, P], I),
        "sk_mtp_expected_tokens": ([P, P, I, P], I),
        "sk_mtp_state": ([P, P, P, P, P], I),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    return lib


LIB = _load()


def status_string(status: int) -> str:
    return LIB.sk_status_string(status).decode()


def _check(status: int, where: str) -> None:
    if status != SK_OK:
        raise SkError(status, where)


def _ptr(t) -> int | None:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("device tensors only: the library has no CPU path")
    return t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _xt(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return SK_F32
    if t.dtype == torch.bfloat16:
        return SK_BF16
    raise ValueError(f"activations must be float32 or bfloat16, got {t.dtype}")


class QuantWeight:
    """A quantised weight in device memory plus its C descriptor.

    ``data`` is a uint8 CUDA tensor of ``weight_bytes(fmt, n, k, g)`` bytes in
    the canonical layout (packed codes then FP32 scales); after
    ``sk_repack_w4a8`` the same tensor holds the stream layout.
    """

    def __init__(self, data: torch.Tensor, n: int, k: int, group: int, fmt: int,
                 codebook: torch.Tensor | None = None):
        self.data = data
        self.codebook = codebook
        self.desc = SkWeightStruct(n, k, group, fmt, SK_LAYOUT_CANONICAL, 0,
                                   data.data_ptr(), data.numel(),
                                   codebook.data_ptr() if codebook is not None else None)

    n = property(lambda self: self.desc.n)
    k = property(lambda self: self.desc.k)
    group = property(lambda self: self.desc.group)
    fmt = property(lambda self: self.desc.format)
    layout = property(lambda self: self.desc.layout)


def weight_bytes(fmt: int, n: int, k: int, g: int) -> int:
    return n * k * BITS[fmt] // 8 + n * (k // g) * 4


def sk_repack_w4a8(w: QuantWeight, stream=None) -> None:
    _check(LIB.sk_repack_w4a8(ctypes.byref(w.desc), _stream(stream)), "sk_repack_w4a8")


def sk_unrepack_w4a8(w: QuantWeight, stream=None) -> None:
    _check(LIB.sk_unrepack_w4a8(ctypes.byref(w.desc), _stream(stream)), "sk_unrepack_w4a8")


# ----------------------------------------------------------------------------
# workspaces (caller-owned device memory for launches that split their work)
# ----------------------------------------------------------------------------

class Workspace:
    """Zero-filled device memory for the library's split launches (see the
    workspace rules in include/sk_repack.h).  Calls that share one Workspace
    must be ordered on one stream (or by events); give concurrent streams
    their own."""

    def __init__(self, nbytes: int, device=None):
        dev = torch.device("cuda") if device is None else torch.device(device)
        self.nbytes = max(256, (int(nbytes) + 255) // 256 * 256)
        self.tensor = torch.zeros(self.nbytes, dtype=torch.uint8, device=dev)
        if self.tensor.data_ptr() % 256:
            raise RuntimeError("workspace allocation is not 256-byte aligned")

    @property
    def ptr(self) -> int:
        return self.tensor.data_ptr()


_DEFAULT_WS_BYTES = 8 << 20
_default_ws = {}          # device index -> Workspace
_retired_ws = []          # replaced default workspaces: kept alive, a captured graph may use them


def default_workspace(nbytes: int, device=None) -> Workspace:
    """The per-device workspace the wrappers use when none is given.  It grows
    (to at least 8 MiB) only outside stream capture; a replaced one is never
    freed, because a captured graph may still point at it."""
    dev = torch.cuda.current_device() if device is None else torch.device(device).index
    ws = _default_ws.get(dev)
    if ws is None or ws.nbytes < nbytes:
        if torch.cuda.is_current_stream_capturing():
            raise RuntimeError(f"the default workspace must grow to {nbytes} bytes, which it cannot "
                               "do during stream capture: make one call of this shape before "
                               "capturing, or pass workspace=Workspace(...)")
        if ws is not None:
            _retired_ws.append(ws)
        ws = Workspace(max(nbytes, _DEFAULT_WS_BYTES), device=torch.device("cuda", dev))
        _default_ws[dev] = ws
    return ws


_ws_sizes = {}


def gemm_workspace_size(n: int, k: int, group: int, fmt: int, m: int, prologue: int = 0) -> int:
    """Bytes of workspace a GEMM call with these sizes needs on the current device."""
    key = (torch.cuda.current_device() if torch.cuda.is_available() else -1, n, k, group, fmt, m,
           prologue)
    v = _ws_sizes.get(key)
    if v is None:
        out = ctypes.c_size_t()
        _check(LIB.sk_gemm_workspace_size(n, k, group, fmt, m, prologue, ctypes.byref(out)),
               "sk_gemm_workspace_size")
        v = _ws_sizes[key] = out.value
    return v


def _ws_args(need: int, workspace):
    if workspace is not None:
        return workspace.ptr, workspace.nbytes
    if need == 0:
        return None, 0
    ws = default_workspace(need)
    return ws.ptr, ws.nbytes


def _gemm_ws(w: QuantWeight, m: int, prologue: int, workspace, n: int | None = None):
    if workspace is not None:
        return workspace.ptr, workspace.nbytes
    return _ws_args(gemm_workspace_size(w.n if n is None else n, w.k, w.group, w.fmt, m, prologue),
                    None)


def _out(w: QuantWeight, m: int, y):
    if y is None:
        y = torch.empty((m, w.n), dtype=torch.float32, device="cuda")
    return y


def sk_gemm_w4a8(w: QuantWeight, x: torch.Tensor, y=None, stream=None, workspace=None) -> torch.Tensor:
    m = x.shape[0]
    y = _out(w, m, y)
    wp, wb = _gemm_ws(w, m, PRO_NONE, workspace)
    _check(LIB.sk_gemm_w4a8(ctypes.byref(w.desc), _ptr(x), _xt(x), m, _ptr(y), wp, wb,
                            _stream(stream)), "sk_gemm_w4a8")
    return y


def sk_gemm_w4a8_noalloc(w: QuantWeight, x: torch.Tensor, y=None, stream=None) -> torch.Tensor:
    """sk_gemm_w4a8 with the library's fixed device scratch instead of a workspace."""
    m = x.shape[0]
    y = _out(w, m, y)
    _check(LIB.sk_gemm_w4a8_noalloc(ctypes.byref(w.desc), _ptr(x), _xt(x), m, _ptr(y), _stream(stream)),
           "sk_gemm_w4a8_noalloc")
    return y


def sk_gemm_w6a8(w: QuantWeight, x: torch.Tensor, y=None, stream=None, workspace=None) -> torch.Tensor:
    m = x.shape[0]
    y = _out(w, m, y)
    wp, wb = _gemm_ws(w, m, PRO_NONE, workspace)
    _check(LIB.sk_gemm_w6a8(ctypes.byref(w.desc), _ptr(x), _xt(x), m, _ptr(y), wp, wb,
                            _stream(stream)), "sk_gemm_w6a8")
    return y


def sk_gemm_experts(bank: QuantWeight, rows_per_expert: int, experts: torch.Tensor, x: torch.Tensor,
                    y=None, stream=None, workspace=None) -> torch.Tensor:
    """Listed experts of a repacked expert bank (E * rows_per_expert rows) times x, in one
    launch; `experts` is a device int32 tensor of ids, read when the kernel runs.
    Returns y [M, len(experts) * rows_per_expert]."""
    if experts.dtype != torch.int32 or not experts.is_cuda or experts.dim() != 1:
        raise ValueError("experts must be a 1-D int32 device tensor")
    nl = experts.shape[0]
    m = x.shape[0]
    if y is None:
        y = torch.empty((m, nl * rows_per_expert), dtype=torch.float32, device="cuda")
    wp, wb = _gemm_ws(bank, m, PRO_NONE, workspace, n=nl * rows_per_expert)
    _check(LIB.sk_gemm_experts(ctypes.byref(bank.desc), rows_per_expert, _ptr(experts), nl,
                               _ptr(x), _xt(x), m, _ptr(y), wp, wb, _stream(stream)), "sk_gemm_experts")
    return y


def sk_quantize_rows(x: torch.Tensor, q=None, sx=None, stream=None):
    """Per-row int8 quantisation as its own launch (the split path); returns (q, sx)."""
    m, k = x.shape
    if q is None:
        q = torch.empty((m, k), dtype=torch.int8, device="cuda")
    if sx is None:
        sx = torch.empty((m,), dtype=torch.float32, device="cuda")
    _check(LIB.sk_quantize_rows(_ptr(x), _xt(x), m, k, _ptr(q), _ptr(sx), _stream(stream)),
           "sk_quantize_rows")
    return q, sx


def sk_prologue_rmsnorm(x: torch.Tensor, gamma: torch.Tensor, eps: float, h=None, stream=None) -> torch.Tensor:
    """h = RMSNorm(x) written to memory as float32 (the split path's prologue launch)."""
    m, k = x.shape
    if h is None:
        h = torch.empty((m, k), dtype=torch.float32, device=x.device)
    _check(LIB.sk_prologue_rmsnorm(_ptr(x), _xt(x), _ptr(gamma), eps, m, k, _ptr(h), _stream(stream)),
           "sk_prologue_rmsnorm")
    return h


def sk_prologue_swiglu(gate: torch.Tensor, up: torch.Tensor, h=None, stream=None) -> torch.Tensor:
    """h = SwiGLU(gate, up) written to memory as float32; gate and up are [M, K]
    views sharing a row stride (the split path's prologue launch)."""
    m, k = gate.shape
    if up.shape != gate.shape or gate.stride() != up.stride() or gate.stride(1) != 1:
        raise ValueError("gate and up must be row-major [M, K] views with the same row stride")
    if h is None:
        h = torch.empty((m, k), dtype=torch.float32, device=gate.device)
    _check(LIB.sk_prologue_swiglu(_ptr(gate), _ptr(up), gate.stride(0), _xt(gate), m, k, _ptr(h),
                                  _stream(stream)), "sk_prologue_swiglu")
    return h


def sk_gemm_w4a8_canonical(w: QuantWeight, x: torch.Tensor, y=None, stream=None,
                           workspace=None) -> torch.Tensor:
    """W4A8 GEMM on a weight left in the canonical layout (no repack)."""
    m = x.shape[0]
    y = _out(w, m, y)
    wp, wb = _gemm_ws(w, m, PRO_NONE, workspace)
    _check(LIB.sk_gemm_w4a8_canonical(ctypes.byref(w.desc), _ptr(x), _xt(x), m, _ptr(y), wp, wb,
                                      _stream(stream)), "sk_gemm_w4a8_canonical")
    return y


def sk_gemm_w4a8_canonical_q(w: QuantWeight, q: torch.Tensor, sx: torch.Tensor, y=None,
                             stream=None, workspace=None) -> torch.Tensor:
    """The same GEMM on activations already quantised by sk_quantize_rows."""
    m = q.shape[0]
    y = _out(w, m, y)
    wp, wb = _gemm_ws(w, m, PRO_NONE, workspace)
    _check(LIB.sk_gemm_w4a8_canonical_q(ctypes.byref(w.desc), _ptr(q), _ptr(sx), m, _ptr(y), wp, wb,
                                        _stream(stream)), "sk_gemm_w4a8_canonical_q")
    return y


def sk_gemm_fused_rmsnorm(w: QuantWeight, x: torch.Tensor, gamma: torch.Tensor, eps: float,
                          y=None, stream=None, workspace=None) -> torch.Tensor:
    m = x.shape[0]
    y = _out(w, m, y)
    wp, wb = _gemm_ws(w, m, PRO_RMSNORM, workspace)
    _check(LIB.sk_gemm_fused_rmsnorm(ctypes.byref(w.desc), _ptr(x), _xt(x), _ptr(gamma),
                                     ctypes.c_float(eps), m, _ptr(y), wp, wb, _stream(stream)),
           "sk_gemm_fused_rmsnorm")
    return y


def sk_gemm_fused_swiglu(w: QuantWeight, gate: torch.Tensor, up: torch.Tensor, y=None,
                         stream=None, workspace=None) -> torch.Tensor:
    """gate and up are [M, K] views sharing one row stride (e.g. halves of [M, 2K])."""
    m = gate.shape[0]
    if gate.stride() != up.stride() or gate.stride(1) != 1:
        raise ValueError("gate and up must be row-major with the same row stride")
    y = _out(w, m, y)
    wp, wb = _gemm_ws(w, m, PRO_SWIGLU, workspace)
    _check(LIB.sk_gemm_fused_swiglu(ctypes.byref(w.desc), _ptr(gate), _ptr(up), gate.stride(0),
                                    _xt(gate), m, _ptr(y), wp, wb, _stream(stream)),
           "sk_gemm_fused_swiglu")
    return y


def sk_debug_gemm(w: QuantWeight, prologue: int, x: torch.Tensor, x2=None, gamma=None,
                  eps: float = 0.0, want_partials: bool = True, stream=None, workspace=None,
                  y=None, q=None, sx=None, p=None):
    """Runs the GEMM with the export flag; returns (y, q, sx, P or None).  The
    outputs may be given (contiguous device tensors of the right sizes)."""
    m, k = x.shape[0], w.k
    ld = x.stride(0) if prologue == PRO_SWIGLU else k
    if y is None:
        y = torch.empty((m, w.n), dtype=torch.float32, device="cuda")
    if q is None:
        q = torch.empty((m, k), dtype=torch.int8, device="cuda")
    if sx is None:
        sx = torch.empty((m,), dtype=torch.float32, device="cuda")
    if p is None and want_partials:
        p = torch.empty((m, w.n, k // w.group), dtype=torch.int32, device="cuda")
    wp, wb = _gemm_ws(w, m, prologue, workspace)
    _check(LIB.sk_debug_gemm(ctypes.byref(w.desc), prologue, _ptr(x), _ptr(x2), ld, _xt(x),
                             _ptr(gamma), ctypes.c_float(eps), m, _ptr(y), _ptr(q), _ptr(sx),
                             _ptr(p), wp, wb, _stream(stream)), "sk_debug_gemm")
    return y, q, sx, p


PLAN_FIELDS = ["S", "R", "P", "TW", "KW", "spw", "KBs", "KS", "WPR", "lds", "part_floats", "ept",
               "wide", "pipe", "srem"]


def gemm_plan(n: int, k: int, group: int, fmt: int, m: int, cus: int = 256,
              prologue: int = PRO_NONE) -> dict:
    """The launch plan of a GEMM call (test hook; host arithmetic only)."""
    f = (ctypes.c_int64 * len(PLAN_FIELDS))()
    st = LIB.sk_test_gemm_plan(n, k, group, fmt, m, prologue, cus, f)
    out = dict(zip(PLAN_FIELDS, list(f)))
    out["status"] = st
    return out


def set_split(s: int) -> None:
    """Test hook: force the number of K-slices (0 = automatic)."""
    _check(LIB.sk_test_set_split(s), "sk_test_set_split")
    _ws_sizes.clear()              # the plans, hence the workspace sizes, change


def stream_read(buf: torch.Tensor, grid: int, threads: int, out: torch.Tensor, stream=None) -> None:
    """Test hook: the streaming-read probe over the bytes of `buf` (see sk_repack_test.h)."""
    _check(LIB.sk_test_stream_read(_ptr(buf), buf.numel() * buf.element_size(), grid, threads,
                                   _ptr(out), _stream(stream)), "sk_test_stream_read")


def set_spin_limit(polls: int) -> None:
    """Test hook: exchange polls before the local fallback (0 = default)."""
    _check(LIB.sk_test_set_spin_limit(polls), "sk_test_set_spin_limit")


# ----------------------------------------------------------------------------
# grouped-query decode attention over the tiled KV cache (include/sk_attention.h)
# ----------------------------------------------------------------------------

HEAD_DIM = 128
KV_BLOCK = 32                 # cache entries per block
KV_BLOCK_BYTES = 16384        # K tile + V tile of one block


def kv_cache_bytes(hkv: int, cap: int) -> int:
    """Size of a cache buffer for ``hkv`` KV heads and ``cap`` entries (cap % 32 == 0)."""
    return hkv * (cap // KV_BLOCK) * KV_BLOCK_BYTES


def _bf16_bits(t: torch.Tensor) -> torch.Tensor:
    if t.dtype == torch.bfloat16:
        return t
    if t.dtype in (torch.uint16, torch.int16):
        return t
    raise ValueError(f"bfloat16 tensors (or their uint16 bits) expected, got {t.dtype}")


def sk_kv_append(kv: torch.Tensor, hkv: int, cap: int, pos: int, k_new: torch.Tensor,
                 v_new: torch.Tensor, stream=None) -> None:
    """Write entries pos .. pos+T-1 of every KV head; k_new, v_new are [T, Hkv, 128] bf16."""
    k_new, v_new = _bf16_bits(k_new), _bf16_bits(v_new)
    if not (k_new.is_contiguous() and v_new.is_contiguous()) or k_new.shape != v_new.shape:
        raise ValueError("k_new and v_new must be contiguous [T, Hkv, 128] tensors of one shape")
    t = k_new.shape[0] if k_new.dim() == 3 else -1
    _check(LIB.sk_kv_append(_ptr(kv), hkv, cap, pos, t, _ptr(k_new), _ptr(v_new), _stream(stream)),
           "sk_kv_append")


def sk_decode_attention(q: torch.Tensor, hkv: int, kv: torch.Tensor, cap: int, length: int,
                        scale: float | None = None, out=None, stream=None, workspace=None) -> torch.Tensor:
    """O [M, Hq, 128] float32 for query rows q [M, Hq, 128] bf16 over the first ``length`` entries."""
    q = _bf16_bits(q)
    if q.dim() != 3 or not q.is_contiguous():
        raise ValueError("q must be a contiguous [M, Hq, 128] tensor")
    m, hq = q.shape[0], q.shape[1]
    if q.shape[2] != HEAD_DIM:
        raise ValueError("head dimension must be 128")
    if scale is None:
        scale = HEAD_DIM ** -0.5
    if out is None:
        out = torch.empty((m, hq, HEAD_DIM), dtype=torch.float32, device=q.device)
    if workspace is not None:
        wp, wb = workspace.ptr, workspace.nbytes
    else:
        wp, wb = _ws_args(attention_workspace_size(m, hq, hkv, length), None)
    _check(LIB.sk_decode_attention(_ptr(q), m, hq, hkv, _ptr(kv), cap, length, ctypes.c_float(scale),
                                   _ptr(out), wp, wb, _stream(stream)), "sk_decode_attention")
    return out


def attention_workspace_size(m: int, hq: int, hkv: int, length: int) -> int:
    """Bytes of workspace sk_decode_attention needs for these sizes on the current device."""
    out = ctypes.c_size_t()
    _check(LIB.sk_attention_workspace_size(m, hq, hkv, length, ctypes.byref(out)),
           "sk_attention_workspace_size")
    return out.value


def sk_kv_pack_host(k, v, hkv: int, length: int, cap: int):
    """Host packing of k, v ([Hkv, L, 128] uint16 bf16 bits, numpy) into the cache layout (numpy uint8)."""
    import numpy as np
    k = np.ascontiguousarray(k, dtype=np.uint16)
    v = np.ascontiguousarray(v, dtype=np.uint16)
    out = np.empty(kv_cache_bytes(hkv, cap), dtype=np.uint8)
    _check(LIB.sk_kv_pack_host(k.ctypes.data, v.ctypes.data, hkv, length, cap, out.ctypes.data),
           "sk_kv_pack_host")
    return out


def attention_plan(m: int, hq: int, hkv: int, length: int, cus: int = 256):
    """(splits, blocks_per_split) the next sk_decode_attention with these sizes uses."""
    sp, bps = ctypes.c_int(), ctypes.c_int()
    _check(LIB.sk_test_attention_plan(m, hq, hkv, length, cus, ctypes.byref(sp), ctypes.byref(bps)),
           "sk_test_attention_plan")
    return sp.value, bps.value


def set_attention_split(blocks_per_split: int) -> None:
    """Test hook: force the blocks per prefix range (0 = planner)."""
    _check(LIB.sk_test_set_attention_split(blocks_per_split), "sk_test_set_attention_split")


# ----------------------------------------------------------------------------
# adaptive tree-MTP layout planner (include/sk_mtp.h; host code)
# ----------------------------------------------------------------------------

def _i32(values):
    arr = (ctypes.c_int32 * max(1, len(values)))(*values)
    return arr


def mtp_layout_of(index: int) -> list:
    w = (ctypes.c_int32 * 7)()
    d = ctypes.c_int32()
    _check(LIB.sk_mtp_layout_of(index, w, ctypes.byref(d)), "sk_mtp_layout_of")
    return list(w[:d.value])


def mtp_accept(widths, ranks):
    """(accepted drafts, levels revealed) of one verified step."""
    a, o = ctypes.c_int32(), ctypes.c_int32()
    _check(LIB.sk_mtp_accept(_i32(widths), len(widths), _i32(ranks), ctypes.byref(a), ctypes.byref(o)),
           "sk_mtp_accept")
    return a.value, o.value


def mtp_expected_tokens(p, widths) -> float:
    """Expected tokens per step; p is [depth][8] rank probabilities (rank 0 = none)."""
    flat = [float(x) for row in p[:len(widths)] for x in row]
    arr = (ctypes.c_double * len(flat))(*flat)
    out = ctypes.c_double()
    _check(LIB.sk_mtp_expected_tokens(arr, _i32(widths), len(widths), ctypes.byref(out)),
           "sk_mtp_expected_tokens")
    return out.value


class MtpPlanner:
    """Owns one sk_mtp_planner."""

    def __init__(self, decay: float = 0.95, interval: int = 32, gain: float = 1.03):
        h = ctypes.c_void_p()
        _check(LIB.sk_mtp_create(ctypes.c_double(decay), interval, ctypes.c_double(gain), ctypes.byref(h)),
               "sk_mtp_create")
        self._h = h
        self._destroy = LIB.sk_mtp_destroy    # kept: the module global may be gone at exit

    def __del__(self):
        if getattr(self, "_h", None):
            self._destroy(self._h)
            self._h = None

    def observe(self, ranks, verify_ms: float, draft_ms: float) -> list:
        w = (ctypes.c_int32 * 7)()
        d = ctypes.c_int32()
        _check(LIB.sk_mtp_observe(self._h, _i32(ranks), len(ranks), ctypes.c_double(verify_ms),
                                  ctypes.c_double(draft_ms), w, ctypes.byref(d)), "sk_mtp_observe")
        return list(w[:d.value])

    @property
    def index(self) -> int:
        i = ctypes.c_int32()
        _check(LIB.sk_mtp_layout(self._h, ctypes.byref(i), None, None), "sk_mtp_layout")
        return i.value

    def state(self):
        c = (ctypes.c_double * 56)()
        v, dr = ctypes.c_double(), ctypes.c_double()
        st = ctypes.c_int64()
        _check(LIB.sk_mtp_state(self._h, c, ctypes.byref(v), ctypes.byref(dr), ctypes.byref(st)), "sk_mtp_state")
        return [list(c[8 * i:8 * i + 8]) for i in range(7)], v.value, dr.value, st.value
