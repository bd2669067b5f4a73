"""MI355X-native W4A16 group-wise quantized linear layer (AWQ's WQLinear hot path).

A thin binding of the C ABI in ``include/awq.h`` (``libawq_mi355x.so``, built
by ``python -m bit_weight_only_awq_amd.build``).  PyTorch supplies device
memory and the current stream only; every step of the layer runs in the
library's HIP kernels.  There is no fallback: if the library is missing or
the tensors are not on the GPU, the calls raise.

Entry points (same names and arguments as the C ABI):

* ``awq_pack(w, group_size, zero_point)`` -> ``(qweight, scales, qzeros)``
* ``awq_dequant(qweight, scales, qzeros, N, K, group_size, zero_point)``
* ``awq_gemv(x, qweight, scales, qzeros, N, K, group_size, zero_point)``
* ``awq_gemm(x, qweight, scales, qzeros, N, K, group_size, zero_point)``
* ``awq_gemm_workspace_bytes(M, N, K, group_size)``, ``awq_strerror(status)``

plus ``pack(W, q_group_size, zero_point)`` / ``linear(x, packed)`` which pick
GEMV up to 8 tokens and GEMM otherwise, following ``quant_config``'s
``version`` ("Optimization Awq", section "Quantizar seu próprio modelo").
"""
from __future__ import annotations

import ctypes
import os
from typing import NamedTuple, Optional

import torch  # noqa: F401  (loaded first: the library then shares torch's HIP runtime)

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libawq_mi355x.so")

AWQ_OK = 0
AWQ_ERR_NULL = -1
AWQ_ERR_SHAPE = -2
AWQ_ERR_GROUP = -3
AWQ_ERR_ALIGN = -4
AWQ_ERR_UNSUPPORTED = -5
AWQ_ERR_WORKSPACE = -6
AWQ_ERR_HIP = -7
AWQ_ERR_SCRATCH = -8

EXPORTED = ("awq_pack", "awq_dequant", "awq_gemv", "awq_gemm", "awq_gemm_workspace_bytes", "awq_strerror",
            "awq_scale_candidates", "awq_scale_candidates_workspace_bytes", "awq_scale_loss",
            "awq_scale_loss_workspace_bytes", "awq_scale_columns", "awq_clip_search",
            "awq_clip_search_workspace_bytes", "awq_scale_search", "awq_scale_search_workspace_bytes",
            "awq_gemm_noalloc", "awq_gemm_noalloc_max_workspace_bytes")

_lib: Optional[ctypes.CDLL] = None


class AwqError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {awq_strerror(status)} (status {status})")
        self.status = status


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the C ABI library once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with `python -m bit_weight_only_awq_amd.build` (hipcc, gfx950)")
    lib = ctypes.CDLL(path)
    P, I32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    lib.awq_pack.argtypes = [P, I32, I32, I32, I32, P, P, P, P]
    lib.awq_pack.restype = ctypes.c_int
    lib.awq_dequant.argtypes = [P, P, P, P, I32, I32, I32, I32, P]
    lib.awq_dequant.restype = ctypes.c_int
    lib.awq_gemv.argtypes = [P, P, P, P, P, I32, I32, I32, I32, I32, P]
    lib.awq_gemv.restype = ctypes.c_int
    lib.awq_gemm.argtypes = [P, P, P, P, P, I32, I32, I32, I32, I32, P, SZ, P]
    lib.awq_gemm.restype = ctypes.c_int
    lib.awq_gemm_workspace_bytes.argtypes = [I32, I32, I32, I32]
    lib.awq_gemm_workspace_bytes.restype = SZ
    lib.awq_strerror.argtypes = [ctypes.c_int]
    lib.awq_strerror.restype = ctypes.c_char_p
    lib.awq_scale_candidates.argtypes = [P, I32, I32, P, I32, I32, P, I32, P, P, SZ, P]
    lib.awq_scale_candidates.restype = ctypes.c_int
    lib.awq_scale_candidates_workspace_bytes.argtypes = [I32, I32, I32]
    lib.awq_scale_candidates_workspace_bytes.restype = SZ
    lib.awq_scale_search.argtypes = [P, P, I32, I32, I32, I32, I32, P, I32, I32, P, P, P, P, SZ, P]
    lib.awq_scale_search.restype = ctypes.c_int
    lib.awq_scale_search_workspace_bytes.argtypes = [I32, I32, I32, I32]
    lib.awq_scale_search_workspace_bytes.restype = SZ
    lib.awq_gemm_noalloc.argtypes = [P, P, P, P, P, I32, I32, I32, I32, I32, P]
    lib.awq_gemm_noalloc.restype = ctypes.c_int
    lib.awq_gemm_noalloc_max_workspace_bytes.argtypes = []
    lib.awq_gemm_noalloc_max_workspace_bytes.restype = SZ
    lib.awq_scale_loss.argtypes = [P, P, P, I32, I32, I32, I32, I32, I32, P, SZ, P, P]
    lib.awq_scale_loss.restype = ctypes.c_int
    lib.awq_scale_loss_workspace_bytes.argtypes = [I32, I32, I32, I32]
    lib.awq_scale_loss_workspace_bytes.restype = SZ
    lib.awq_scale_columns.argtypes = [P, I32, I32, P, I32, P, P]
    lib.awq_scale_columns.restype = ctypes.c_int
    lib.awq_clip_search.argtypes = [P, P, I32, I32, I32, I32, I32, P, I32, P, P, P, SZ, P]
    lib.awq_clip_search.restype = ctypes.c_int
    lib.awq_clip_search_workspace_bytes.argtypes = [I32, I32, I32, I32, I32]
    lib.awq_clip_search_workspace_bytes.restype = SZ
    _lib = lib
    return lib


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors passed to the AWQ kernels must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors passed to the AWQ kernels must be contiguous")
    return t.data_ptr()


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _check(status: int, where: str) -> None:
    if status != AWQ_OK:
        raise AwqError(status, where)


def awq_strerror(status: int) -> str:
    return load_library().awq_strerror(int(status)).decode()


def awq_gemm_workspace_bytes(M: int, N: int, K: int, group_size: int) -> int:
    return int(load_library().awq_gemm_workspace_bytes(M, N, K, group_size))


def awq_pack(w: torch.Tensor, group_size: int = 128, zero_point: bool = True,
             qweight: Optional[torch.Tensor] = None, scales: Optional[torch.Tensor] = None,
             qzeros: Optional[torch.Tensor] = None):
    """Quantize fp16 ``w`` [N, K] and return ``(qweight int32 [N, K/8], scales fp16 [N/8, K/g, 8],
    qzeros int32 [N/8, K/g] or None)``; the int32 tensors hold the ABI's uint32 words."""
    lib = load_library()
    if w.dtype != torch.float16 or w.dim() != 2:
        raise ValueError("w must be a 2-D float16 tensor [N, K]")
    N, K = w.shape
    G = K // group_size if group_size > 0 else 0
    dev = w.device
    if qweight is None:
        qweight = torch.empty((N, K // 8), dtype=torch.int32, device=dev)
    if scales is None:
        scales = torch.empty((N // 8, G, 8), dtype=torch.float16, device=dev)
    if zero_point and qzeros is None:
        qzeros = torch.empty((N // 8, G), dtype=torch.int32, device=dev)
    st = lib.awq_pack(_ptr(w), N, K, group_size, int(bool(zero_point)), _ptr(qweight), _ptr(scales),
                      _ptr(qzeros) if zero_point else None, _stream(w))
    _check(st, "awq_pack")
    return qweight, scales, (qzeros if zero_point else None)


def awq_dequant(qweight: torch.Tensor, scales: torch.Tensor, qzeros: Optional[torch.Tensor], N: int, K: int,
                group_size: int = 128, zero_point: bool = True, w_out: Optional[torch.Tensor] = None):
    """Decode a packed weight to fp16 [N, K] (test and inspection aid)."""
    lib = load_library()
    if w_out is None:
        w_out = torch.empty((N, K), dtype=torch.float16, device=qweight.device)
    st = lib.awq_dequant(_ptr(qweight), _ptr(scales), _ptr(qzeros) if zero_point else None, _ptr(w_out), N, K,
                         group_size, int(bool(zero_point)), _stream(qweight))
    _check(st, "awq_dequant")
    return w_out


def _xy(x: torch.Tensor, N: int, y: Optional[torch.Tensor]):
    if x.dtype != torch.float16 or x.dim() != 2:
        raise ValueError("x must be a 2-D float16 tensor [M, K]")
    if y is None:
        y = torch.empty((x.shape[0], N), dtype=torch.float16, device=x.device)
    return y


def awq_gemv(x: torch.Tensor, qweight: torch.Tensor, scales: torch.Tensor, qzeros: Optional[torch.Tensor], N: int,
             K: int, group_size: int = 128, zero_point: bool = True, y: Optional[torch.Tensor] = None):
    """Single- and few-token layer Y = X . W'^T for X fp16 [M, K], 1 <= M <= 8; returns fp16 [M, N]."""
    lib = load_library()
    y = _xy(x, N, y)
    st = lib.awq_gemv(_ptr(x), _ptr(qweight), _ptr(scales), _ptr(qzeros) if zero_point else None, _ptr(y),
                      x.shape[0], N, K, group_size, int(bool(zero_point)), _stream(x))
    _check(st, "awq_gemv")
    return y


_WORKSPACES = {}          # (device index, stream handle) -> zero-initialised uint8 tensor
_RETIRED_WORKSPACES = []  # replaced buffers, kept alive for graphs that captured their address


def gemm_workspace(nbytes: int, device=None, stream=None) -> torch.Tensor:
    """The zero-initialised awq_gemm workspace of (``device``, ``stream``), at
    least ``nbytes`` long, kept for later calls on that stream.  awq_gemm
    returns the workspace's counters to zero, so calls in one stream's order
    share it, including calls captured into a HIP graph on that stream.
    Calls on different streams get different buffers, since overlapping
    calls on one buffer would break its per-tile counters.

    Under graph capture the buffer is not created or grown (its zero fill
    would only be recorded into the graph): call once eagerly on the
    capture stream first, or pass ``workspace=`` explicitly."""
    device = torch.device(device) if device is not None else torch.device("cuda", torch.cuda.current_device())
    idx = device.index if device.index is not None else torch.cuda.current_device()
    if stream is None:
        stream = torch.cuda.current_stream(idx)
    key = (idx, stream.cuda_stream)
    ws = _WORKSPACES.get(key)
    if ws is None or ws.numel() < nbytes:
        if torch.cuda.is_current_stream_capturing():
            raise RuntimeError(
                f"awq_gemm needs a {nbytes}-byte split-K workspace on stream {stream.cuda_stream:#x} of cuda:{idx}, "
                "and none of that size exists; a workspace cannot be created during graph capture. Make one "
                "eager call of the largest shape on the capture stream before capturing, or pass workspace= "
                "(a zero-filled uint8 tensor of awq_gemm_workspace_bytes(...) bytes)")
        if ws is not None:
            _RETIRED_WORKSPACES.append(ws)
        with torch.cuda.stream(stream):  # zero fill ordered before this stream's next call
            ws = torch.zeros(max(nbytes, 1 << 20), dtype=torch.uint8, device=torch.device("cuda", idx))
        _WORKSPACES[key] = ws
    return ws


def awq_gemm(x: torch.Tensor, qweight: torch.Tensor, scales: torch.Tensor, qzeros: Optional[torch.Tensor], N: int,
             K: int, group_size: int = 128, zero_point: bool = True, y: Optional[torch.Tensor] = None,
             workspace: Optional[torch.Tensor] = None):
    """Batched layer Y = X . W'^T for X fp16 [M, K]; returns fp16 [M, N]."""
    lib = load_library()
    y = _xy(x, N, y)
    M = x.shape[0]
    need = awq_gemm_workspace_bytes(M, N, K, group_size)
    if need and workspace is None:
        workspace = gemm_workspace(need, x.device)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = lib.awq_gemm(_ptr(x), _ptr(qweight), _ptr(scales), _ptr(qzeros) if zero_point else None, _ptr(y), M, N, K,
                      group_size, int(bool(zero_point)), _ptr(workspace), ws_bytes, _stream(x))
    _check(st, "awq_gemm")
    return y


def awq_gemm_noalloc(x: torch.Tensor, qweight: torch.Tensor, scales: torch.Tensor, qzeros: Optional[torch.Tensor],
                     N: int, K: int, group_size: int = 128, zero_point: bool = True,
                     y: torch.Tensor = None) -> torch.Tensor:
    """awq_gemm with the library's fixed device scratch as the split-K
    workspace: the C call allocates nothing (``y`` must be passed, so that
    this wrapper allocates nothing either).  Calls that may overlap on one
    GPU share the scratch and race."""
    lib = load_library()
    if y is None:
        raise ValueError("awq_gemm_noalloc takes a preallocated output y")
    if x.dtype != torch.float16 or x.dim() != 2:
        raise ValueError("x must be a 2-D float16 tensor [M, K]")
    st = lib.awq_gemm_noalloc(_ptr(x), _ptr(qweight), _ptr(scales), _ptr(qzeros) if zero_point else None, _ptr(y),
                              x.shape[0], N, K, group_size, int(bool(zero_point)), _stream(x))
    _check(st, "awq_gemm_noalloc")
    return y


class PackedWeight(NamedTuple):
    qweight: torch.Tensor
    scales: torch.Tensor
    qzeros: Optional[torch.Tensor]
    N: int
    K: int
    group_size: int
    zero_point: bool


def pack(W: torch.Tensor, q_group_size: int = 128, zero_point: bool = True) -> PackedWeight:
    """Quantize an ``nn.Linear`` weight [out, in] on the GPU (``quant_config``: w_bit 4)."""
    qw, sc, qz = awq_pack(W, q_group_size, zero_point)
    return PackedWeight(qw, sc, qz, W.shape[0], W.shape[1], q_group_size, bool(zero_point))


def pack_fused(weights, q_group_size: int = 128, zero_point: bool = True) -> PackedWeight:
    """Pack several weights that read the same input (e.g. the q, k and v
    projections, or gate and up) as one weight of N = sum of their N, so one
    launch computes all of them ("AI-Research-SKILLs AWQ 高级使用指南", section
    层融合: Q, K, V merged into one GEMM, gate and up fused).

    Each part is quantized by its own ``awq_pack`` call straight into its
    slice of the fused buffers: rows are independent and the scales/zero
    points are stored per octet of rows, so a part with N a multiple of 8 is a
    contiguous slice of every array and the result is bit-identical to packing
    the concatenated weight.  The output of ``linear`` is the concatenation of
    the parts' outputs, in order."""
    weights = list(weights)
    if not weights:
        raise ValueError("pack_fused needs at least one weight")
    K = weights[0].shape[1]
    if any(w.dim() != 2 or w.shape[1] != K for w in weights):
        raise ValueError("fused weights must all be [N_i, K] with the same K")
    N = sum(w.shape[0] for w in weights)
    G = K // q_group_size if q_group_size > 0 else 0
    dev = weights[0].device
    qweight = torch.empty((N, K // 8), dtype=torch.int32, device=dev)
    scales = torch.empty((N // 8, G, 8), dtype=torch.float16, device=dev)
    qzeros = torch.empty((N // 8, G), dtype=torch.int32, device=dev) if zero_point else None
    n0 = 0
    for w in weights:
        n = w.shape[0]
        if n % 8:
            raise ValueError("every fused part needs N % 8 == 0")
        awq_pack(w, q_group_size, zero_point, qweight=qweight[n0:n0 + n], scales=scales[n0 // 8:(n0 + n) // 8],
                 qzeros=qzeros[n0 // 8:(n0 + n) // 8] if zero_point else None)
        n0 += n
    return PackedWeight(qweight, scales, qzeros, N, K, q_group_size, bool(zero_point))


def linear(x: torch.Tensor, pw: PackedWeight, version: str = "auto") -> torch.Tensor:
    """Y = X . W'^T.  ``version`` "GEMV" (up to 8 tokens), "GEMM" (any batch) or "auto"."""
    x2 = x.reshape(-1, pw.K)
    v = version.upper()
    if v == "AUTO":
        v = "GEMV" if x2.shape[0] <= 8 else "GEMM"
    fn = awq_gemv if v == "GEMV" else awq_gemm
    y = fn(x2, pw.qweight, pw.scales, pw.qzeros, pw.N, pw.K, pw.group_size, pw.zero_point)
    return y.reshape(*x.shape[:-1], pw.N)


def awq_scale_candidates(x: torch.Tensor, alphas, w: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Candidate per-channel scales s[c] = max(mean |x|, 1e-4) ** alphas[c] for fp16
    calibration activations ``x`` [M, K]; with ``w`` [N, K] (duo scaling) also
    divided by max(mean |w|, 1e-4) ** (1 - alphas[c]).  Returns fp32
    [len(alphas), K] on x's device."""
    lib = load_library()
    alphas = [float(a) for a in alphas]
    M, K = x.shape
    N = w.shape[0] if w is not None else 0
    s = torch.empty((len(alphas), K), dtype=torch.float32, device=x.device)
    ws = torch.empty(max(1, int(lib.awq_scale_candidates_workspace_bytes(M, N, K))), dtype=torch.uint8,
                     device=x.device)
    arr = (ctypes.c_float * len(alphas))(*alphas)
    st = lib.awq_scale_candidates(_ptr(x), M, K, _ptr(w), N, int(w is not None), ctypes.cast(arr, ctypes.c_void_p),
                                  len(alphas), _ptr(s), _ptr(ws), ws.numel(), _stream(x))
    _check(st, "awq_scale_candidates")
    return s


def awq_scale_loss(x: torch.Tensor, w: torch.Tensor, s: torch.Tensor, group_size: int = 128,
                   zero_point: bool = True) -> torch.Tensor:
    """L(s_c) = ||Q(W s_c)(s_c^-1 X) - W X||_F for every row s_c of the fp32 ``s``
    [count, K]; ``x`` fp16 [M, K], ``w`` fp16 [N, K].  Returns fp64 [count] on the GPU."""
    lib = load_library()
    M, K = x.shape
    N = w.shape[0]
    s2 = s.reshape(-1, K)
    count = s2.shape[0]
    loss = torch.empty(count, dtype=torch.float64, device=x.device)
    ws = torch.empty(max(1, int(lib.awq_scale_loss_workspace_bytes(count, M, N, K))), dtype=torch.uint8,
                     device=x.device)
    st = lib.awq_scale_loss(_ptr(x), _ptr(w), _ptr(s2), count, M, N, K, group_size, int(bool(zero_point)), _ptr(ws),
                            ws.numel(), _ptr(loss), _stream(x))
    _check(st, "awq_scale_loss")
    return loss


DEFAULT_ALPHAS = tuple(i / 20 for i in range(20))


class ScaleSearch(NamedTuple):
    best: torch.Tensor    # int32 [1] on the device: index of the chosen candidate
    scale: torch.Tensor   # fp32 [K] on the device: the chosen s
    losses: torch.Tensor  # fp64 [count] on the device: L(s) of every candidate, in the order of alphas
    alphas: tuple

    @property
    def alpha(self) -> float:
        """The chosen exponent (reads the index back from the device)."""
        return self.alphas[int(self.best.item())]


def awq_scale_search(x: torch.Tensor, w: torch.Tensor, group_size: int = 128, zero_point: bool = True,
                     alphas=DEFAULT_ALPHAS, duo: bool = False) -> ScaleSearch:
    """Activation-aware scale search on the device: L(s) for s = a ** alpha
    (duo: a ** alpha / b ** (1 - alpha)) over ``alphas`` and the first
    candidate with the smallest loss.  ``x`` fp16 [M, K] calibration
    activations, ``w`` fp16 [N, K].  Nothing is read back to the host."""
    lib = load_library()
    alphas = tuple(float(a) for a in alphas)
    M, K = x.shape
    N = w.shape[0]
    dev = x.device
    s_best = torch.empty(K, dtype=torch.float32, device=dev)
    best = torch.empty(1, dtype=torch.int32, device=dev)
    losses = torch.empty(len(alphas), dtype=torch.float64, device=dev)
    ws = torch.empty(max(1, int(lib.awq_scale_search_workspace_bytes(len(alphas), M, N, K))), dtype=torch.uint8,
                     device=dev)
    arr = (ctypes.c_float * len(alphas))(*alphas)
    st = lib.awq_scale_search(_ptr(x), _ptr(w), M, N, K, group_size, int(bool(zero_point)),
                              ctypes.cast(arr, ctypes.c_void_p), len(alphas), int(bool(duo)), _ptr(s_best),
                              _ptr(best), _ptr(losses), _ptr(ws), ws.numel(), _stream(x))
    _check(st, "awq_scale_search")
    return ScaleSearch(best, s_best, losses, alphas)


def search_scale(x: torch.Tensor, w: torch.Tensor, group_size: int = 128, zero_point: bool = True,
                 alphas=None, duo: bool = False) -> ScaleSearch:
    """Activation-aware scale search (default grid 0, 1/20, ..., 19/20).  The
    chosen s is applied as W * s before packing and s^-1 on the activations."""
    return awq_scale_search(x, w, group_size, zero_point, DEFAULT_ALPHAS if alphas is None else alphas, duo)


def awq_scale_columns(src: torch.Tensor, s: torch.Tensor, divide: bool = False,
                      out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """fp16(src * s) per input channel (or fp16(src / s) with ``divide``)."""
    lib = load_library()
    rows, K = src.shape
    if out is None:
        out = torch.empty_like(src)
    st = lib.awq_scale_columns(_ptr(src), rows, K, _ptr(s), int(bool(divide)), _ptr(out), _stream(src))
    _check(st, "awq_scale_columns")
    return out


DEFAULT_CLIP_RATIOS = tuple(1.0 - 0.025 * i for i in range(20))


def awq_clip_search(x: torch.Tensor, w: torch.Tensor, group_size: int = 128, zero_point: bool = True,
                    ratios=DEFAULT_CLIP_RATIOS):
    """Weight clipping: per group, the ratio in ``ratios`` with the smallest
    output error over ``x``.  Returns (clipped fp16 weights [N, K], chosen
    ratio index int32 [N, K / group_size])."""
    lib = load_library()
    M, K = x.shape
    N = w.shape[0]
    ratios = [float(r) for r in ratios]
    out = torch.empty_like(w)
    choice = torch.empty((N, K // group_size), dtype=torch.int32, device=w.device)
    ws = torch.empty(max(1, int(lib.awq_clip_search_workspace_bytes(len(ratios), M, N, K, group_size))),
                     dtype=torch.uint8, device=w.device)
    arr = (ctypes.c_float * len(ratios))(*ratios)
    st = lib.awq_clip_search(_ptr(x), _ptr(w), M, N, K, group_size, int(bool(zero_point)),
                             ctypes.cast(arr, ctypes.c_void_p), len(ratios), _ptr(out), _ptr(choice), _ptr(ws),
                             ws.numel(), _stream(x))
    _check(st, "awq_clip_search")
    return out, choice


class QuantizedLinear(NamedTuple):
    packed: PackedWeight
    input_scale: torch.Tensor  # fp32 [K]: the layer computes on fp16(x / input_scale)
    search: ScaleSearch        # the scale search (chosen index and losses stay on the device)


def quantize_awq(w: torch.Tensor, x: torch.Tensor, q_group_size: int = 128, zero_point: bool = True,
                 alphas=None, clip_ratios=DEFAULT_CLIP_RATIOS, apply_clip: bool = True,
                 duo_scaling: bool = False) -> QuantizedLinear:
    """The activation-aware quantization of one linear layer from calibration
    activations ``x`` [M, K]: scale search (the candidate s with the smallest
    L(s)), weights scaled by s, optional clipping search on the scaled layer,
    then packing; every step on the device, with no host synchronization.
    The packed layer expects activations divided by ``input_scale``
    (``awq_scale_columns(x, s, divide=True)``, or folded into the producer of x)."""
    res = search_scale(x, w, q_group_size, zero_point, alphas, duo_scaling)
    ws = awq_scale_columns(w, res.scale)
    if apply_clip:
        xs = awq_scale_columns(x, res.scale, divide=True)
        ws, _ = awq_clip_search(xs, ws, q_group_size, zero_point, clip_ratios)
    return QuantizedLinear(pack(ws, q_group_size, zero_point), res.scale, res)
