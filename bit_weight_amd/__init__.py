"""Sherry 3:4-sparse ternary matmul for AMD MI355X (gfx950).

Thin ctypes binding over the C ABI of ``libsherry.so`` (declared in
``include/sherry.h``).  The functions here only check tensors, allocate
outputs with PyTorch and pass raw device pointers and the current HIP stream;
every step of the computation runs in the library's HIP kernels.  There is no
CPU fallback: if the library is missing, every call raises.

Method: the page "Sherry框架：三元量化与3:4稀疏优化LLM推理" (pnsm.cn) --
ternary weights with exactly three nonzeros per block of four (§1.1), 5-bit
codes (§2.1), per-segment lookup tables with one float rescale (§2.2), top-3
ternarization (§3.1).
"""

from __future__ import annotations

import ctypes
import os
import threading

import torch

__all__ = [
    "SherryError", "lib", "packed_bytes", "workspace_bytes", "plan", "plan_override",
    "quantize_pack", "quantize_act", "gemm", "gemm_i32", "linear", "linear_scratch_bytes", "concat_packed", "quantize_pack2", "gemm2",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
# SHERRY_LIB names another build of the same library (the host-only
# sanitizer build that the CPU tests make); by default the in-tree one
LIB_PATH = os.environ.get("SHERRY_LIB") or os.path.join(_HERE, "libsherry.so")

STATUS = {
    0: "SHERRY_OK", -1: "SHERRY_ERR_NULL", -2: "SHERRY_ERR_SHAPE",
    -3: "SHERRY_ERR_ALIGN", -4: "SHERRY_ERR_WORKSPACE", -5: "SHERRY_ERR_HIP",
    -6: "SHERRY_ERR_DEVICE", -7: "SHERRY_ERR_PARTIAL",
}


class SherryError(RuntimeError):
    """A non-zero status from libsherry."""

    def __init__(self, status: int, what: str):
        self.status = status
        msg = lib().sherry_status_string(status).decode()
        super().__init__(f"{what}: {msg} ({status})")


_lib = None
_lock = threading.Lock()


def lib() -> ctypes.CDLL:
    """The loaded libsherry.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(
                    f"{LIB_PATH} is missing: build it with "
                    "`python -m bit_weight_amd.build` (or __graft_entry__.build())")
            L = ctypes.CDLL(LIB_PATH)
            vp, i64, sz, ci = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t, ctypes.c_int
            ip = ctypes.POINTER(ctypes.c_int)
            sigs = {
                "sherry_status_string": ([ci], ctypes.c_char_p),
                "sherry_packed_bytes": ([i64, i64], sz),
                "sherry_workspace_bytes": ([i64, i64, i64], sz),
                "sherry_gemm_plan": ([i64, i64, i64, ip, ip, ip, ip, ip], ci),
                "sherry_gemm_plan_override": ([ci, ci, ci, ci], ci),
                "sherry_linear_plan": ([i64, i64, i64, ip, ip, ip, ip, ip, ip], ci),
                "sherry_quantize_pack": ([vp, i64, i64, vp, vp, vp], ci),
                "sherry_quantize_act": ([vp, i64, i64, vp, vp, vp], ci),
                "sherry_gemm": ([vp, vp, vp, vp, vp, i64, i64, i64, vp, sz, vp], ci),
                "sherry_gemm_i32": ([vp, vp, vp, i64, i64, i64, vp, sz, vp], ci),
                "sherry_linear_scratch_bytes": ([i64, i64, i64], sz),
                "sherry_packed2_bytes": ([i64, i64], sz),
                "sherry_quantize_pack2": ([vp, i64, i64, vp, vp, vp], ci),
                "sherry_gemm2_workspace_bytes": ([i64, i64, i64], sz),
                "sherry_gemm2": ([vp, vp, vp, vp, vp, i64, i64, i64, vp, sz, vp], ci),
                "sherry_linear": ([vp, vp, vp, vp, i64, i64, i64, vp, sz, vp, sz, vp], ci),
                "sherry_gemm_noalloc": ([vp, vp, vp, vp, vp, i64, i64, i64, vp], ci),
                "sherry_probe_read": ([vp, sz, vp, ci, ci, ci, vp], ci),
                "sherry_probe_empty": ([vp], ci),
                "sherry_probe_decode": ([ci, vp, ci, ci, vp], ci),
                "sherry_probe_decode_codes": ([ci, ci, ci], i64),
            }
            for name, (args, res) in sigs.items():
                fn = getattr(L, name)
                fn.argtypes = args
                fn.restype = res
            _lib = L
    return _lib


def _check(status: int, what: str) -> None:
    if status != 0:
        raise SherryError(status, what)


def _dev_tensor(t: torch.Tensor, name: str, dtype: torch.dtype) -> int:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise RuntimeError(f"{name} must be on a GPU device, got {t.device}")
    if t.dtype != dtype:
        raise RuntimeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise RuntimeError(f"{name} must be contiguous")
    return t.data_ptr()


def _stream(device: torch.device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def packed_bytes(N: int, K: int) -> int:
    """Bytes of the packed format for an [N,K] weight matrix (N*K*5/32)."""
    return int(lib().sherry_packed_bytes(N, K))


def workspace_bytes(M: int, N: int, K: int) -> int:
    """Scratch bytes sherry_gemm needs for this shape."""
    return int(lib().sherry_workspace_bytes(M, N, K))


def plan(M: int, N: int, K: int) -> dict:
    """Launch plan of the product for a shape (path, grid, block, splits, LDS)."""
    vals = [ctypes.c_int() for _ in range(5)]
    _check(lib().sherry_gemm_plan(M, N, K, *[ctypes.byref(v) for v in vals]), "sherry_gemm_plan")
    path, grid, block, splits, lds = (v.value for v in vals)
    return {"path": PATHS.get(path, str(path)), "grid": grid,
            "block": block, "splits": splits, "lds_bytes": lds}


def linear_plan(M: int, N: int, K: int) -> dict:
    """Launch plan of sherry_linear's product for a shape, and whether the
    quantization is fused into it (one launch)."""
    vals = [ctypes.c_int() for _ in range(6)]
    _check(lib().sherry_linear_plan(M, N, K, *[ctypes.byref(v) for v in vals]), "sherry_linear_plan")
    path, grid, block, splits, lds, fused = (v.value for v in vals)
    return {"path": PATHS.get(path, str(path)), "grid": grid, "block": block,
            "splits": splits, "lds_bytes": lds, "fused": bool(fused)}


PATHS = {0: "lut_gemv", 1: "decode_mfma", 2: "decode_mfma_gemv"}
PATH_IDS = {v: k for k, v in PATHS.items()}


def plan_override(path=None, rw: int = 0, ch: int = 0, splits: int = 0) -> None:
    """Tuning knob for M <= 128: force a path ("lut_gemv", "decode_mfma",
    "decode_mfma_gemv" or None = built-in) and its launch plan (0 = built-in).
    Above M = 16, "decode_mfma" gives the prefill GEMM and the others the
    GEMV.  With "decode_mfma" (any M), rw = 1 or 2 picks tiles of 64 or 128
    tokens."""
    pid = -1 if path is None else PATH_IDS[path]
    _check(lib().sherry_gemm_plan_override(pid, rw, ch, splits), "sherry_gemm_plan_override")


def quantize_pack(W: torch.Tensor):
    """Offline compression of fp32 weights [N,K] -> (packed uint8, alpha fp32 [N])."""
    pW = _dev_tensor(W, "W", torch.float32)
    if W.dim() != 2:
        raise RuntimeError("W must be 2-D [N,K]")
    N, K = W.shape
    nb = packed_bytes(N, K)
    if nb == 0:
        raise SherryError(-2, "sherry_quantize_pack")
    packed = torch.empty(nb, dtype=torch.uint8, device=W.device)
    alpha = torch.empty(N, dtype=torch.float32, device=W.device)
    _check(lib().sherry_quantize_pack(pW, N, K, packed.data_ptr(), alpha.data_ptr(),
                                      _stream(W.device)), "sherry_quantize_pack")
    return packed, alpha


def quantize_act(x: torch.Tensor):
    """Per-token int8 quantization of fp32 activations [M,K] -> (q int8, s_x fp32 [M])."""
    px = _dev_tensor(x, "x", torch.float32)
    if x.dim() != 2:
        raise RuntimeError("x must be 2-D [M,K]")
    M, K = x.shape
    q = torch.empty((M, K), dtype=torch.int8, device=x.device)
    s = torch.empty(M, dtype=torch.float32, device=x.device)
    _check(lib().sherry_quantize_act(px, M, K, q.data_ptr(), s.data_ptr(), _stream(x.device)),
           "sherry_quantize_act")
    return q, s


class _Workspaces:
    """Zero-filled scratch per (device, stream), grown on demand.

    The library leaves a workspace zero-ready after every call, so one buffer
    serves every call issued on its stream."""

    def __init__(self):
        self._bufs = {}

    def get(self, device: torch.device, nbytes: int):
        if nbytes == 0:
            return None
        key = (device.index, torch.cuda.current_stream(device).cuda_stream)
        buf = self._bufs.get(key)
        if buf is None or buf.numel() < nbytes:
            buf = torch.zeros(max(nbytes, 1 << 20), dtype=torch.uint8, device=device)
            self._bufs[key] = buf
        return buf


_workspaces = _Workspaces()


def _gemm_args(x, packed, N, K):
    px = _dev_tensor(x, "x", torch.int8)
    _dev_tensor(packed, "packed", torch.uint8)
    if x.dim() != 2 or x.shape[1] != K:
        raise RuntimeError(f"x must be [M,{K}]")
    if packed.numel() != packed_bytes(N, K):
        raise RuntimeError("packed has the wrong size for [N,K]")
    M = x.shape[0]
    ws = _workspaces.get(x.device, workspace_bytes(M, N, K))
    return px, M, ws


def gemm(x: torch.Tensor, s_x: torch.Tensor, packed: torch.Tensor, alpha: torch.Tensor,
         N: int, K: int, out: torch.Tensor | None = None,
         workspace: torch.Tensor | None = None) -> torch.Tensor:
    """y[M,N] = ((float)(x_int8 @ T^T) * s_x[:,None]) * alpha[None,:]."""
    px, M, ws = _gemm_args(x, packed, N, K)
    _dev_tensor(s_x, "s_x", torch.float32)
    _dev_tensor(alpha, "alpha", torch.float32)
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=x.device)
    py = _dev_tensor(out, "out", torch.float32)
    if workspace is not None:
        ws = workspace
    wp = ws.data_ptr() if ws is not None else None
    wn = ws.numel() if ws is not None else 0
    _check(lib().sherry_gemm(px, s_x.data_ptr(), packed.data_ptr(), alpha.data_ptr(), py, M, N, K,
                             wp, wn, _stream(x.device)), "sherry_gemm")
    return out


def gemm_i32(x: torch.Tensor, packed: torch.Tensor, N: int, K: int,
             out: torch.Tensor | None = None,
             workspace: torch.Tensor | None = None) -> torch.Tensor:
    """acc[M,N] = x_int8 @ T^T in int32 (exact)."""
    px, M, ws = _gemm_args(x, packed, N, K)
    if out is None:
        out = torch.empty((M, N), dtype=torch.int32, device=x.device)
    pa = _dev_tensor(out, "out", torch.int32)
    if workspace is not None:
        ws = workspace
    wp = ws.data_ptr() if ws is not None else None
    wn = ws.numel() if ws is not None else 0
    _check(lib().sherry_gemm_i32(px, packed.data_ptr(), pa, M, N, K, wp, wn, _stream(x.device)),
           "sherry_gemm_i32")
    return out


NOALLOC_SCRATCH_BYTES = 8 << 20   # the static split-K scratch of sherry_gemm_noalloc, per GPU


def gemm_noalloc(x: torch.Tensor, s_x: torch.Tensor, packed: torch.Tensor, alpha: torch.Tensor,
                 N: int, K: int, out: torch.Tensor | None = None) -> torch.Tensor:
    """sherry_gemm without a workspace (sherry_gemm_noalloc): the split-K
    cells live in the library's static per-GPU array; shapes needing more
    than 8 MiB of them are rejected.  Calls that overlap on one GPU race."""
    px = _dev_tensor(x, "x", torch.int8)
    _dev_tensor(packed, "packed", torch.uint8)
    _dev_tensor(s_x, "s_x", torch.float32)
    _dev_tensor(alpha, "alpha", torch.float32)
    if x.dim() != 2 or x.shape[1] != K:
        raise RuntimeError(f"x must be [M,{K}]")
    if packed.numel() != packed_bytes(N, K):
        raise RuntimeError("packed has the wrong size for [N,K]")
    M = x.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=x.device)
    py = _dev_tensor(out, "out", torch.float32)
    _check(lib().sherry_gemm_noalloc(px, s_x.data_ptr(), packed.data_ptr(), alpha.data_ptr(), py, M, N, K,
                                     _stream(x.device)), "sherry_gemm_noalloc")
    return out


def probe_read(buf: torch.Tensor, sink: torch.Tensor, grid: int, block: int, unroll: int) -> None:
    """Diagnostic: stream-read all of `buf` (a contiguous device tensor whose
    byte size is a multiple of 16); `sink` is a device int32 tensor."""
    if not buf.is_contiguous() or buf.device.type != "cuda":
        raise RuntimeError("buf must be a contiguous device tensor")
    nbytes = buf.numel() * buf.element_size()
    _check(lib().sherry_probe_read(buf.data_ptr(), nbytes, sink.data_ptr(), grid, block, unroll,
                                   _stream(buf.device)), "sherry_probe_read")


def probe_empty(device=None) -> None:
    """Diagnostic: one empty kernel launch on the current stream."""
    dev = torch.device("cuda", torch.cuda.current_device()) if device is None else device
    _check(lib().sherry_probe_empty(_stream(dev)), "sherry_probe_empty")


def probe_decode(sink: torch.Tensor, iters: int, grid: int, block: int) -> int:
    """Diagnostic: one launch of the decode step alone (code-pair lookups in
    an LDS table, nothing else); returns the number of codes it decodes.
    `sink` is a device int32 tensor."""
    _check(lib().sherry_probe_decode(iters, sink.data_ptr(), grid, block, _stream(sink.device)),
           "sherry_probe_decode")
    return int(lib().sherry_probe_decode_codes(iters, grid, block))


def linear_scratch_bytes(M: int, N: int, K: int) -> int:
    """Scratch bytes (q and s_x, any content) sherry_linear needs beyond the
    workspace; 0 when the quantization is fused into the product."""
    return int(lib().sherry_linear_scratch_bytes(M, N, K))


_scratch = {}


def linear(x: torch.Tensor, packed: torch.Tensor, alpha: torch.Tensor, N: int, K: int,
           out: torch.Tensor | None = None, workspace: torch.Tensor | None = None,
           scratch: torch.Tensor | None = None) -> torch.Tensor:
    """fp32 activations [M,K] -> y [M,N]: per-token int8 quantization and the
    product in one call (sherry_linear; fused into one kernel for small M)."""
    px = _dev_tensor(x, "x", torch.float32)
    _dev_tensor(packed, "packed", torch.uint8)
    _dev_tensor(alpha, "alpha", torch.float32)
    if x.dim() != 2 or x.shape[1] != K:
        raise RuntimeError(f"x must be [M,{K}]")
    if packed.numel() != packed_bytes(N, K):
        raise RuntimeError("packed has the wrong size for [N,K]")
    M = x.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=x.device)
    py = _dev_tensor(out, "out", torch.float32)
    ws = workspace if workspace is not None else _workspaces.get(x.device, workspace_bytes(M, N, K))
    nsc = linear_scratch_bytes(M, N, K)
    if scratch is None and nsc > 0:
        key = (x.device.index, torch.cuda.current_stream(x.device).cuda_stream)
        scratch = _scratch.get(key)
        if scratch is None or scratch.numel() < nsc:
            scratch = torch.empty(max(nsc, 1 << 20), dtype=torch.uint8, device=x.device)
            _scratch[key] = scratch
    wp = ws.data_ptr() if ws is not None else None
    wn = ws.numel() if ws is not None else 0
    sp = scratch.data_ptr() if scratch is not None else None
    sn = scratch.numel() if scratch is not None else 0
    _check(lib().sherry_linear(px, packed.data_ptr(), alpha.data_ptr(), py, M, N, K, wp, wn, sp, sn,
                               _stream(x.device)), "sherry_linear")
    return out


def concat_packed(parts, Ns, K: int):
    """Group several [N_i, K] packed matrices (e.g. q/k/v or gate/up; every
    N_i but the last a multiple of 64) into one [sum N_i, K] packed matrix.
    The format keeps each 64-row tile of every k-tile contiguous and orders
    tiles row group first, so stacking weights along N stacks their packed
    bytes: the group is plain concatenation, and one sherry_linear call on
    it computes every member's output, sharing one activation quantization
    and one launch.  (A part padded to whole row tiles would leave padding
    rows inside the group, hence the rule.)  `parts` are (packed, alpha)
    pairs; returns (packed, alpha)."""
    packs, alphas = [], []
    if any(n % 64 for n in list(Ns)[:-1]):
        raise RuntimeError("every part but the last needs N_i % 64 == 0 to stack")
    for (pk, al), n in zip(parts, Ns):
        if pk.numel() != packed_bytes(n, K) or al.numel() != n:
            raise RuntimeError("a part has the wrong size for its [N_i, K]")
        packs.append(pk)
        alphas.append(al)
    return torch.cat(packs), torch.cat(alphas)


def quantize_pack2(W: torch.Tensor):
    """The same ternarization as quantize_pack, in the 2-bit baseline format
    -> (packed uint8 [N*K/4], alpha fp32 [N])."""
    pW = _dev_tensor(W, "W", torch.float32)
    if W.dim() != 2:
        raise RuntimeError("W must be 2-D [N,K]")
    N, K = W.shape
    nb = int(lib().sherry_packed2_bytes(N, K))
    if nb == 0:
        raise SherryError(-2, "sherry_quantize_pack2")
    packed = torch.empty(nb, dtype=torch.uint8, device=W.device)
    alpha = torch.empty(N, dtype=torch.float32, device=W.device)
    _check(lib().sherry_quantize_pack2(pW, N, K, packed.data_ptr(), alpha.data_ptr(),
                                       _stream(W.device)), "sherry_quantize_pack2")
    return packed, alpha


def gemm2(x: torch.Tensor, s_x: torch.Tensor, packed: torch.Tensor, alpha: torch.Tensor,
          N: int, K: int, out: torch.Tensor | None = None,
          workspace: torch.Tensor | None = None) -> torch.Tensor:
    """The product on the 2-bit baseline format (M <= 16)."""
    px = _dev_tensor(x, "x", torch.int8)
    _dev_tensor(packed, "packed", torch.uint8)
    _dev_tensor(s_x, "s_x", torch.float32)
    _dev_tensor(alpha, "alpha", torch.float32)
    if x.dim() != 2 or x.shape[1] != K:
        raise RuntimeError(f"x must be [M,{K}]")
    if packed.numel() != int(lib().sherry_packed2_bytes(N, K)):
        raise RuntimeError("packed has the wrong size for [N,K]")
    M = x.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=x.device)
    py = _dev_tensor(out, "out", torch.float32)
    ws = workspace if workspace is not None else _workspaces.get(
        x.device, int(lib().sherry_gemm2_workspace_bytes(M, N, K)))
    wp = ws.data_ptr() if ws is not None else None
    wn = ws.numel() if ws is not None else 0
    _check(lib().sherry_gemm2(px, s_x.data_ptr(), packed.data_ptr(), alpha.data_ptr(), py, M, N, K,
                              wp, wn, _stream(x.device)), "sherry_gemm2")
    return out
