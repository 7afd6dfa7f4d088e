"""GPTQ layer-wise second-order weight quantization on AMD MI355X (gfx950).

Thin ctypes binding over ``libgptq_mi355x.so`` (C ABI in include/gptq.h).
The functions below only marshal arguments: every stage runs in the
library's HIP kernels.  PyTorch supplies device memory (outputs and
workspaces) and the current HIP stream.  If the shared library is missing the
import of the binding raises; there is no fallback path.

Stages (same names as the C ABI):
    hessian_accumulate(H, X)                    H += 2 X^T X   (X token-major)
    prepare_hinv(H, damp)                       -> U, lambda, info
    quantize_layer(W, U, bits, group, block)    -> packed codes, scales, zeros
and the runtime use of the packed layer:
    dequant_matmul(X, qcodes, scales, zeros, bits, group, n)  -> Y = X What^T
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgptq_mi355x.so")

GPTQ_OK, GPTQ_ERR_INVALID_ARG, GPTQ_ERR_UNSUPPORTED, GPTQ_ERR_WORKSPACE, GPTQ_ERR_HIP, GPTQ_ERR_SCRATCH_LIMIT = range(6)
F16, BF16, F32 = 0, 1, 2
_DT = {torch.float16: F16, torch.bfloat16: BF16, torch.float32: F32}

_lib = None


class GPTQError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {status_string(status)} ({status})")
        self.status = status


def _load() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run post_weight_quantization_10_amd.build.build() "
                          "(hipcc, --offload-arch=gfx950)")
    L = ctypes.CDLL(LIB_PATH)
    i64, i32, sz, vp = ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t, ctypes.c_void_p
    f32 = ctypes.c_float
    L.gptq_status_string.argtypes = [i32]
    L.gptq_status_string.restype = ctypes.c_char_p
    L.gptq_version.argtypes = []
    L.gptq_version.restype = i32
    L.gptq_hessian_workspace_bytes.argtypes = [i64, i64]
    L.gptq_hessian_workspace_bytes.restype = sz
    L.gptq_hessian_accumulate.argtypes = [vp, i64, vp, i32, i64, i64, vp, sz, vp]
    L.gptq_hessian_accumulate.restype = i32
    L.gptq_prepare_workspace_bytes.argtypes = [i64]
    L.gptq_prepare_workspace_bytes.restype = sz
    L.gptq_prepare_hinv.argtypes = [vp, i64, f32, vp, vp, vp, vp, sz, vp]
    L.gptq_prepare_hinv.restype = i32
    L.gptq_quantize_workspace_bytes.argtypes = [i64, i64, i64]
    L.gptq_quantize_workspace_bytes.restype = sz
    L.gptq_quantize_layer.argtypes = [vp, i32, i64, i64, i64, vp, i32, i64, i64, vp, vp, vp, vp, i32, vp, sz, vp]
    L.gptq_quantize_layer.restype = i32
    L.gptq_dequant_matmul_workspace_bytes.argtypes = [i64, i64, i64]
    L.gptq_dequant_matmul_workspace_bytes.restype = sz
    L.gptq_dequant_matmul.argtypes = [vp, i32, i64, i64, vp, vp, vp, i64, i64, i32, i64, vp, i64, vp, sz, vp]
    L.gptq_dequant_matmul.restype = i32
    L.gptq_static_scratch_bytes.argtypes = []
    L.gptq_static_scratch_bytes.restype = sz
    L.gptq_dequant_matmul_static.argtypes = [vp, i32, i64, i64, vp, vp, vp, i64, i64, i32, i64, vp, i64, vp]
    L.gptq_dequant_matmul_static.restype = i32
    L.gptq_rotate_hadamard.argtypes = [vp, i32, i64, i64, i64, i64, vp]
    L.gptq_rotate_hadamard.restype = i32
    L.gptq_swiglu.argtypes = [vp, vp, vp, i32, i64, i64, i64, vp]
    L.gptq_swiglu.restype = i32
    L.gptq_residual_add.argtypes = [vp, vp, i32, i64, i64, i64, vp]
    L.gptq_residual_add.restype = i32
    L.gptq_attention.argtypes = [vp, vp, vp, vp, i32, i64, i64, i64, i64, i64, vp]
    L.gptq_attention.restype = i32
    L.gptq_quantize_greedy_workspace_bytes.argtypes = [i64, i64]
    L.gptq_quantize_greedy_workspace_bytes.restype = sz
    L.gptq_quantize_greedy.argtypes = [vp, i32, i64, i64, i64, vp, i32, i64, vp, vp, vp, vp, vp, vp, sz, vp]
    L.gptq_quantize_greedy.restype = i32
    _lib = L
    return L


def lib() -> ctypes.CDLL:
    return _load()


def status_string(status: int) -> str:
    return _load().gptq_status_string(int(status)).decode()


def version() -> int:
    return int(_load().gptq_version())


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(dev: torch.device) -> int:
    return torch.cuda.current_stream(dev).cuda_stream


def _check(fn: str, st: int) -> None:
    if st != GPTQ_OK:
        raise GPTQError(fn, st)


def _require(cond: bool, msg: str) -> None:
    if not cond:
        raise ValueError(msg)


def _workspace(nbytes: int, dev: torch.device) -> torch.Tensor:
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=dev)


# ----------------------------------------------------------------------------- workspace sizes

def hessian_workspace_bytes(n: int, tokens: int) -> int:
    return int(_load().gptq_hessian_workspace_bytes(int(n), int(tokens)))


def prepare_workspace_bytes(n: int) -> int:
    return int(_load().gptq_prepare_workspace_bytes(int(n)))


def quantize_workspace_bytes(m: int, n: int, block_size: int = 128) -> int:
    return int(_load().gptq_quantize_workspace_bytes(int(m), int(n), int(block_size)))


def dequant_matmul_workspace_bytes(tokens: int, m: int, n: int) -> int:
    return int(_load().gptq_dequant_matmul_workspace_bytes(int(tokens), int(m), int(n)))


# ----------------------------------------------------------------------------- the three stages

def hessian_accumulate(H: torch.Tensor, X: torch.Tensor, workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """H += 2 * X^T X for token-major activations X [tokens x n] (fp16, bf16 or
    fp32, rows may be strided).  H is [n x n] float32 contiguous; returns H."""
    _require(H.is_cuda and X.is_cuda and H.device == X.device, "H and X must be on the same GPU")
    _require(H.dtype == torch.float32 and H.dim() == 2 and H.shape[0] == H.shape[1] and H.is_contiguous(),
             "H must be a contiguous float32 [n, n] tensor")
    _require(X.dim() == 2 and X.shape[1] == H.shape[0] and X.stride(1) == 1, "X must be [tokens, n] with unit column stride")
    _require(X.dtype in _DT, f"unsupported activation dtype {X.dtype}")
    n, T = H.shape[0], X.shape[0]
    need = hessian_workspace_bytes(n, T)
    ws = workspace if workspace is not None else _workspace(need, H.device)
    st = _load().gptq_hessian_accumulate(H.data_ptr(), n, X.data_ptr() if T else None, _DT[X.dtype], T,
                                         max(X.stride(0), n), ws.data_ptr(), ws.numel(), _stream(H.device))
    _check("gptq_hessian_accumulate", st)
    return H


def prepare_hinv(H: torch.Tensor, damp: float = 0.01, U: Optional[torch.Tensor] = None,
                 workspace: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """U upper with (H + lambda I)^-1 = U^T U, lambda = damp * mean(diag H).
    Returns (U, lambda [1] float32, info [1] int32) as device tensors; read
    info after a synchronize (0 = success)."""
    _require(H.is_cuda and H.dtype == torch.float32 and H.dim() == 2 and H.shape[0] == H.shape[1]
             and H.is_contiguous(), "H must be a contiguous float32 [n, n] CUDA tensor")
    n = H.shape[0]
    if U is None:
        U = torch.empty_like(H)
    _require(U.shape == H.shape and U.dtype == torch.float32 and U.is_contiguous() and U.device == H.device,
             "U must match H")
    lam = torch.empty(1, dtype=torch.float32, device=H.device)
    info = torch.empty(1, dtype=torch.int32, device=H.device)
    ws = workspace if workspace is not None else _workspace(prepare_workspace_bytes(n), H.device)
    st = _load().gptq_prepare_hinv(H.data_ptr(), n, float(damp), U.data_ptr(), info.data_ptr(), lam.data_ptr(),
                                   ws.data_ptr(), ws.numel(), _stream(H.device))
    _check("gptq_prepare_hinv", st)
    return U, lam, info


def n_groups(n: int, group_size: int) -> int:
    return 1 if group_size <= 0 else (n + group_size - 1) // group_size


def packed_words(n: int, bits: int) -> int:
    return (n * bits + 31) // 32


def quantize_layer(W: torch.Tensor, U: torch.Tensor, bits: int, group_size: int, block_size: int = 128,
                   write_dequant: bool = True, err_sq: bool = True,
                   workspace: Optional[torch.Tensor] = None,
                   out: Optional[Dict[str, torch.Tensor]] = None) -> Dict[str, torch.Tensor]:
    """Blocked GPTQ sweep of W [m x n] (fp16 / bf16 / fp32, row stride >= n)
    against the factor U.  Returns {'qcodes' [m x words] int32 (uint32 bit
    patterns), 'scales' [m x G] float32, 'zeros' [m x G] int32, 'err_sq' [m]}.
    With write_dequant, W is overwritten in place by s (q - z)."""
    _require(W.is_cuda and U.is_cuda and W.device == U.device, "W and U must be on the same GPU")
    _require(W.dim() == 2 and W.stride(1) == 1 and W.dtype in _DT, "W must be [m, n] fp16/bf16/fp32, unit column stride")
    m, n = W.shape
    _require(U.shape == (n, n) and U.dtype == torch.float32 and U.is_contiguous(), "U must be contiguous float32 [n, n]")
    G = n_groups(n, group_size)
    dev = W.device
    o = dict(out or {})
    if "qcodes" not in o:
        o["qcodes"] = torch.empty((m, packed_words(n, bits)), dtype=torch.int32, device=dev)
    if "scales" not in o:
        o["scales"] = torch.empty((m, G), dtype=torch.float32, device=dev)
    if "zeros" not in o:
        o["zeros"] = torch.empty((m, G), dtype=torch.int32, device=dev)
    if err_sq and "err_sq" not in o:
        o["err_sq"] = torch.empty((m,), dtype=torch.float32, device=dev)
    ws = workspace if workspace is not None else _workspace(quantize_workspace_bytes(m, n, block_size), dev)
    st = _load().gptq_quantize_layer(W.data_ptr(), _DT[W.dtype], m, n, max(W.stride(0), n), U.data_ptr(), int(bits),
                                     int(group_size), int(block_size), o["qcodes"].data_ptr(), o["scales"].data_ptr(),
                                     o["zeros"].data_ptr(), _ptr(o.get("err_sq")) if err_sq else None,
                                     1 if write_dequant else 0, ws.data_ptr(), ws.numel(), _stream(dev))
    _check("gptq_quantize_layer", st)
    return o


def greedy_workspace_bytes(m: int, n: int) -> int:
    return int(_load().gptq_quantize_greedy_workspace_bytes(m, n))


def quantize_greedy(W: torch.Tensor, U: torch.Tensor, bits: int, group_size: int, order: bool = True,
                    loss: bool = True, workspace: Optional[torch.Tensor] = None,
                    out: Optional[Dict[str, torch.Tensor]] = None) -> Dict[str, torch.Tensor]:
    """OBQ's greedy-order quantization of W [m x n] (read only) against the
    factor U.  Returns {'qcodes', 'scales', 'zeros'} in quantize_layer's
    layout, plus 'order' [m x n] int32 (column quantized at each step) and
    'loss' [m] float32 (sum of the chosen loss increases) when asked for."""
    _require(W.is_cuda and U.is_cuda and W.device == U.device, "W and U must be on the same GPU")
    _require(W.dim() == 2 and W.stride(1) == 1 and W.dtype in _DT, "W must be [m, n] fp16/bf16/fp32, unit column stride")
    m, n = W.shape
    _require(U.shape == (n, n) and U.dtype == torch.float32 and U.is_contiguous(), "U must be contiguous float32 [n, n]")
    G = n_groups(n, group_size)
    dev = W.device
    o = dict(out or {})
    if "qcodes" not in o:
        o["qcodes"] = torch.empty((m, packed_words(n, bits)), dtype=torch.int32, device=dev)
    if "scales" not in o:
        o["scales"] = torch.empty((m, G), dtype=torch.float32, device=dev)
    if "zeros" not in o:
        o["zeros"] = torch.empty((m, G), dtype=torch.int32, device=dev)
    if order and "order" not in o:
        o["order"] = torch.empty((m, n), dtype=torch.int32, device=dev)
    if loss and "loss" not in o:
        o["loss"] = torch.empty((m,), dtype=torch.float32, device=dev)
    ws = workspace if workspace is not None else _workspace(greedy_workspace_bytes(m, n), dev)
    st = _load().gptq_quantize_greedy(W.data_ptr(), _DT[W.dtype], m, n, max(W.stride(0), n), U.data_ptr(), int(bits),
                                      int(group_size), o["qcodes"].data_ptr(), o["scales"].data_ptr(),
                                      o["zeros"].data_ptr(), _ptr(o.get("order")) if order else None,
                                      _ptr(o.get("loss")) if loss else None, ws.data_ptr(), ws.numel(), _stream(dev))
    _check("gptq_quantize_greedy", st)
    return o


def gptq_layer(W: torch.Tensor, X: torch.Tensor, bits: int, group_size: int, block_size: int = 128,
               damp: float = 0.01, write_dequant: bool = True) -> Dict[str, torch.Tensor]:
    """All three stages for one layer: H from X, the damped inverse factor,
    then the sweep.  Raises if the damped Hessian is not positive definite."""
    n = W.shape[1]
    H = torch.zeros((n, n), dtype=torch.float32, device=W.device)
    hessian_accumulate(H, X)
    U, lam, info = prepare_hinv(H, damp)
    res = quantize_layer(W, U, bits, group_size, block_size, write_dequant=write_dequant)
    if int(info.item()) != 0:
        raise GPTQError("gptq_prepare_hinv (damped Hessian not positive definite)", GPTQ_ERR_INVALID_ARG)
    res.update({"H": H, "U": U, "lambda": lam, "info": info})
    return res


# ----------------------------------------------------------------------------- runtime use of the packed layer

def dequant_matmul(X: torch.Tensor, qcodes: torch.Tensor, scales: torch.Tensor, zeros: torch.Tensor, bits: int,
                   group_size: int, Y: Optional[torch.Tensor] = None,
                   workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Y = X What^T [tokens x m] in X's dtype (fp16 or bf16), with What = s (q - z)
    unpacked from the packed layer (qcodes [m x words], scales / zeros [m x G]).
    X is [tokens x n], unit column stride."""
    _require(X.is_cuda and X.dim() == 2 and X.stride(1) == 1 and X.dtype in (torch.float16, torch.bfloat16),
             "X must be a [tokens, n] fp16/bf16 CUDA tensor with unit column stride")
    m = qcodes.shape[0]
    T, n = X.shape
    dev = X.device
    _require(qcodes.device == dev and qcodes.dtype == torch.int32 and qcodes.is_contiguous()
             and qcodes.shape == (m, packed_words(n, bits)), "qcodes must be contiguous int32 [m, words]")
    G = n_groups(n, group_size)
    _require(scales.shape == (m, G) and scales.dtype == torch.float32 and scales.is_contiguous()
             and scales.device == dev, "scales must be contiguous float32 [m, G]")
    _require(zeros.shape == (m, G) and zeros.dtype == torch.int32 and zeros.is_contiguous() and zeros.device == dev,
             "zeros must be contiguous int32 [m, G]")
    if Y is None:
        Y = torch.empty((T, m), dtype=X.dtype, device=dev)
    _require(Y.dtype == X.dtype and Y.dim() == 2 and Y.shape == (T, m) and Y.stride(1) == 1 and Y.device == dev,
             "Y must be [tokens, m] in X's dtype with unit column stride")
    need = dequant_matmul_workspace_bytes(T, m, n)
    ws = workspace if workspace is not None else (_workspace(need, dev) if need > 0 else None)
    st = _load().gptq_dequant_matmul(X.data_ptr(), _DT[X.dtype], T, max(X.stride(0), n), qcodes.data_ptr(),
                                     scales.data_ptr(), zeros.data_ptr(), m, n, int(bits), int(group_size),
                                     Y.data_ptr(), max(Y.stride(0), m), _ptr(ws), 0 if ws is None else ws.numel(),
                                     _stream(dev))
    _check("gptq_dequant_matmul", st)
    return Y


def static_scratch_bytes() -> int:
    return int(_load().gptq_static_scratch_bytes())


def dequant_matmul_static(X: torch.Tensor, qcodes: torch.Tensor, scales: torch.Tensor, zeros: torch.Tensor,
                          bits: int, group_size: int, Y: torch.Tensor) -> torch.Tensor:
    """dequant_matmul without a workspace: the partial sums go to the
    library's fixed per-GPU buffer, so the call allocates nothing (Y must be
    given).  Calls that overlap in time on one GPU race on that buffer."""
    _require(X.is_cuda and X.dim() == 2 and X.stride(1) == 1 and X.dtype in (torch.float16, torch.bfloat16),
             "X must be a [tokens, n] fp16/bf16 CUDA tensor with unit column stride")
    m = qcodes.shape[0]
    T, n = X.shape
    dev = X.device
    _require(qcodes.device == dev and qcodes.dtype == torch.int32 and qcodes.is_contiguous()
             and qcodes.shape == (m, packed_words(n, bits)), "qcodes must be contiguous int32 [m, words]")
    G = n_groups(n, group_size)
    _require(scales.shape == (m, G) and scales.dtype == torch.float32 and scales.is_contiguous()
             and scales.device == dev, "scales must be contiguous float32 [m, G]")
    _require(zeros.shape == (m, G) and zeros.dtype == torch.int32 and zeros.is_contiguous() and zeros.device == dev,
             "zeros must be contiguous int32 [m, G]")
    _require(Y.dtype == X.dtype and Y.dim() == 2 and Y.shape == (T, m) and Y.stride(1) == 1 and Y.device == dev,
             "Y must be [tokens, m] in X's dtype with unit column stride")
    st = _load().gptq_dequant_matmul_static(X.data_ptr(), _DT[X.dtype], T, max(X.stride(0), n), qcodes.data_ptr(),
                                            scales.data_ptr(), zeros.data_ptr(), m, n, int(bits), int(group_size),
                                            Y.data_ptr(), max(Y.stride(0), m), _stream(dev))
    _check("gptq_dequant_matmul_static", st)
    return Y


def rotate_hadamard(M: torch.Tensor, block: int = 0) -> torch.Tensor:
    """M <- M R in place (R block-diagonal Hadamard of order `block`, scaled
    to be orthogonal; 0 = the largest power of two dividing the row length,
    at most 4096).  M is [rows, n] fp16/bf16/fp32 with unit column stride.
    Returns M."""
    _require(M.is_cuda and M.dim() == 2 and M.stride(1) == 1 and M.dtype in _DT,
             "M must be a [rows, n] fp16/bf16/fp32 CUDA tensor with unit column stride")
    rows, n = M.shape
    st = _load().gptq_rotate_hadamard(M.data_ptr() if rows else None, _DT[M.dtype], rows, n, max(M.stride(0), n),
                                      int(block), _stream(M.device))
    _check("gptq_rotate_hadamard", st)
    return M


def _rows16(t: torch.Tensor, name: str):
    _require(t.is_cuda and t.dim() == 2 and t.stride(1) == 1 and t.dtype in (torch.float16, torch.bfloat16),
             f"{name} must be a [tokens, width] fp16/bf16 CUDA tensor with unit column stride")


def swiglu(G: torch.Tensor, Uo: torch.Tensor, A: Optional[torch.Tensor] = None) -> torch.Tensor:
    """A = silu(G) * Uo (the hidden activations of an MLP block)."""
    _rows16(G, "G")
    _require(Uo.shape == G.shape and Uo.dtype == G.dtype and Uo.stride() == G.stride() and Uo.device == G.device,
             "Uo must match G")
    if A is None:
        A = torch.empty_strided(G.shape, G.stride(), dtype=G.dtype, device=G.device)
    _require(A.shape == G.shape and A.dtype == G.dtype and A.stride() == G.stride(), "A must match G")
    T, f = G.shape
    st = _load().gptq_swiglu(G.data_ptr(), Uo.data_ptr(), A.data_ptr(), _DT[G.dtype], T, f, max(G.stride(0), f),
                             _stream(G.device))
    _check("gptq_swiglu", st)
    return A


def residual_add(X: torch.Tensor, Y: torch.Tensor) -> torch.Tensor:
    """X <- X + Y in place; returns X."""
    _rows16(X, "X")
    _require(Y.shape == X.shape and Y.dtype == X.dtype and Y.stride() == X.stride() and Y.device == X.device,
             "Y must match X")
    T, d = X.shape
    st = _load().gptq_residual_add(X.data_ptr(), Y.data_ptr(), _DT[X.dtype], T, d, max(X.stride(0), d),
                                   _stream(X.device))
    _check("gptq_residual_add", st)
    return X


def attention(Q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, seq_len: int, heads: int,
              O: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Causal multi-head softmax attention over sequences of seq_len
    consecutive tokens; Q, K, V [tokens, heads * head_dim] fp16/bf16 with a
    common row stride.  Returns O in the same layout."""
    _rows16(Q, "Q")
    for t, nm in ((K, "K"), (V, "V")):
        _require(t.shape == Q.shape and t.dtype == Q.dtype and t.stride() == Q.stride() and t.device == Q.device,
                 f"{nm} must match Q")
    T, dm = Q.shape
    _require(heads >= 1 and dm % heads == 0, "the row width must be heads * head_dim")
    if O is None:
        O = torch.empty_strided(Q.shape, Q.stride(), dtype=Q.dtype, device=Q.device)
    _require(O.shape == Q.shape and O.dtype == Q.dtype and O.stride() == Q.stride(), "O must match Q")
    st = _load().gptq_attention(Q.data_ptr(), K.data_ptr(), V.data_ptr(), O.data_ptr(), _DT[Q.dtype], T,
                                int(seq_len), int(heads), dm // heads, max(Q.stride(0), dm), _stream(Q.device))
    _check("gptq_attention", st)
    return O


def quantize_transformer_stack(blocks, X0: torch.Tensor, seq_len: int, heads: int, bits: int = 4,
                               group_size: int = 128, block_size: int = 128, damp: float = 0.01,
                               keep_inputs: bool = False):
    """The network-level loop over transformer blocks (no normalization):
        x <- x + W_o attn(W_q x, W_k x, W_v x);  x <- x + W_down (silu(W_gate x) * (W_up x))
    one layer at a time, each layer's calibration inputs computed by the
    network as quantized so far.  blocks: list of (W_q, W_k, W_v, W_o, W_gate,
    W_up, W_down) CUDA tensors (fp16/bf16, not modified; q/k/v and o are
    [d, d], gate/up [f, d], down [d, f]).  X0: [tokens, d] activations in the
    same dtype, tokens grouped in sequences of seq_len.  Per block: H of x
    (shared by q, k, v: their rows are swept together), Q/K/V through
    gptq_dequant_matmul, A = attention, H of A and the o sweep, x += A W_o^T;
    then H of x (shared by gate and up), G and Uo, A2 = swiglu, H of A2 and the
    down sweep, x += A2 W_down^T.  Returns (per-block dicts with the four
    quantize_layer results and factors, plus every activation when
    keep_inputs, final x)."""
    X = X0.clone()
    out = []

    def factor(Xa):
        n = Xa.shape[1]
        H = torch.zeros((n, n), dtype=torch.float32, device=Xa.device)
        hessian_accumulate(H, Xa)
        U, _, info = prepare_hinv(H, damp)
        return U, info

    def product(Xa, r):
        return dequant_matmul(Xa, r["qcodes"], r["scales"], r["zeros"], bits, group_size)

    for Wq, Wk, Wv, Wo, Wg, Wu, Wd in blocks:
        d = X.shape[1]
        rec = {}
        X_in = X.clone() if keep_inputs else None
        U1, i1 = factor(X)
        rqkv = quantize_layer(torch.cat([Wq, Wk, Wv], dim=0), U1, bits, group_size, block_size, write_dequant=False)
        qkv = product(X, rqkv)                               # [tokens, 3d]: Q | K | V
        Q, K, V = qkv[:, :d], qkv[:, d:2 * d], qkv[:, 2 * d:]
        A = attention(Q, K, V, seq_len, heads)
        U2, i2 = factor(A)
        ro = quantize_layer(Wo.clone(), U2, bits, group_size, block_size, write_dequant=False)
        Yo = product(A, ro)
        X = residual_add(X, Yo)
        X_mid = X.clone() if keep_inputs else None
        U3, i3 = factor(X)
        rgu = quantize_layer(torch.cat([Wg, Wu], dim=0), U3, bits, group_size, block_size, write_dequant=False)
        GU = product(X, rgu)                                 # [tokens, 2f]: G | Uo
        f = Wg.shape[0]
        A2 = swiglu(GU[:, :f], GU[:, f:])
        U4, i4 = factor(A2)
        rd = quantize_layer(Wd.clone(), U4, bits, group_size, block_size, write_dequant=False)
        Yd = product(A2, rd)
        X = residual_add(X, Yd)
        if any(int(t.item()) != 0 for t in (i1, i2, i3, i4)):
            raise GPTQError("gptq_prepare_hinv (a block's Hessian is not positive definite)", GPTQ_ERR_INVALID_ARG)
        rec.update({"qkv": rqkv, "o": ro, "gate_up": rgu, "down": rd, "U": (U1, U2, U3, U4)})
        if keep_inputs:
            rec.update({"X": X_in, "QKV": qkv, "A": A, "Yo": Yo, "X_mid": X_mid, "GU": GU, "A2": A2, "Yd": Yd})
        out.append(rec)
    return out, X


def quantize_mlp_stack(blocks, X0: torch.Tensor, bits: int = 4, group_size: int = 128, block_size: int = 128,
                       damp: float = 0.01, keep_inputs: bool = False):
    """The network-level loop over MLP blocks x <- x + W_down (silu(W_gate x) *
    (W_up x)): one layer at a time, each layer's calibration inputs computed by
    the network as quantized so far.  blocks: list of (W_gate [f, d], W_up
    [f, d], W_down [d, f]) CUDA tensors (fp16/bf16; not modified).  X0:
    [tokens, d] calibration activations in the same dtype.  Per block: H from
    X (shared by gate and up), both swept with its factor; G and Uo through
    gptq_dequant_matmul from the packed codes; A = swiglu(G, Uo); H from A,
    down swept; X <- X + A What_down^T.  Returns (list of per-block dicts with
    the three quantize_layer results, plus X, A, G, Uo and Y when keep_inputs),
    final X)."""
    X = X0.clone()
    out = []
    for Wg, Wu, Wd in blocks:
        d = X.shape[1]
        H = torch.zeros((d, d), dtype=torch.float32, device=X.device)
        hessian_accumulate(H, X)
        U, _, info = prepare_hinv(H, damp)
        rg = quantize_layer(Wg.clone(), U, bits, group_size, block_size, write_dequant=False)
        ru = quantize_layer(Wu.clone(), U, bits, group_size, block_size, write_dequant=False)
        G = dequant_matmul(X, rg["qcodes"], rg["scales"], rg["zeros"], bits, group_size)
        Uo = dequant_matmul(X, ru["qcodes"], ru["scales"], ru["zeros"], bits, group_size)
        A = swiglu(G, Uo)
        f = A.shape[1]
        H2 = torch.zeros((f, f), dtype=torch.float32, device=X.device)
        hessian_accumulate(H2, A)
        U2, _, info2 = prepare_hinv(H2, damp)
        rd = quantize_layer(Wd.clone(), U2, bits, group_size, block_size, write_dequant=False)
        Y = dequant_matmul(A, rd["qcodes"], rd["scales"], rd["zeros"], bits, group_size)
        if int(info.item()) != 0 or int(info2.item()) != 0:
            raise GPTQError("gptq_prepare_hinv (a block's Hessian is not positive definite)", GPTQ_ERR_INVALID_ARG)
        rec = {"gate": rg, "up": ru, "down": rd, "U": U, "U2": U2}
        if keep_inputs:
            rec.update({"X": X.clone(), "G": G, "Uo": Uo, "A": A, "Y": Y})
        X = residual_add(X, Y)
        out.append(rec)
    return out, X
