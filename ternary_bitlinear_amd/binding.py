"""ctypes binding of libbitlinear.so (argument marshalling only).

Torch supplies device memory and streams; every step of the projection runs
in the library's HIP kernels.  There is no CPU fallback: if the library is
missing or fails to load, every call raises.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libbitlinear.so")

STATUS = {
    0: "BITLINEAR_OK", 1: "BITLINEAR_ERR_NULL", 2: "BITLINEAR_ERR_SHAPE", 3: "BITLINEAR_ERR_ALIGN",
    4: "BITLINEAR_ERR_DTYPE", 5: "BITLINEAR_ERR_NO_DEVICE", 6: "BITLINEAR_ERR_ARCH",
    7: "BITLINEAR_ERR_WORKSPACE", 8: "BITLINEAR_ERR_HIP",
}
DTYPES = {"f32": 0, "bf16": 1, "i32": 2}

# Every symbol the header declares, with its ctypes signature.
_c_i64, _c_size, _vp = ctypes.c_int64, ctypes.c_size_t, ctypes.c_void_p
SIGNATURES = {
    "bitlinear_abi_version": (ctypes.c_int, []),
    "bitlinear_packed_bytes": (_c_size, [_c_i64, _c_i64]),
    "bitlinear_pack_workspace_bytes": (_c_size, [_c_i64, _c_i64]),
    "bitlinear_pack_weights": (ctypes.c_int, [_vp, _c_i64, _c_i64, _vp, _vp, _vp, _c_size, _vp]),
    "bitlinear_quant_acts": (ctypes.c_int, [_vp, _c_i64, _c_i64, _vp, _vp, _vp, _vp]),
    "bitlinear_quant_acts_bits": (ctypes.c_int, [_vp, _c_i64, _c_i64, ctypes.c_int, _vp, _vp, _vp,
                                                 _vp]),
    "bitlinear_forward_workspace_bytes": (_c_size, [_c_i64, _c_i64, _c_i64]),
    "bitlinear_forward": (ctypes.c_int, [_vp, _vp, _c_i64, _c_i64, _vp, _vp, _vp, _c_i64, _vp,
                                         ctypes.c_int, _vp, _c_size, _vp]),
    "bitlinear_forward_f32_workspace_bytes": (_c_size, [_c_i64, _c_i64, _c_i64]),
    "bitlinear_forward_f32": (ctypes.c_int, [_vp, _vp, _c_i64, _c_i64, _vp, _c_i64, _vp, ctypes.c_int,
                                             _vp, _vp, _vp, _vp, _c_size, _vp]),
    "bitlinear_forward_grouped_workspace_bytes": (_c_size, [_c_i64, ctypes.c_int, _vp, _c_i64]),
    "bitlinear_forward_grouped": (ctypes.c_int, [ctypes.c_int, _vp, _vp, _vp, _c_i64, _vp, _vp, _vp,
                                                 _c_i64, _vp, ctypes.c_int, _vp, _c_size, _vp]),
    "bitlinear_forward_f32_grouped_workspace_bytes": (_c_size, [_c_i64, ctypes.c_int, _vp, _c_i64]),
    "bitlinear_forward_f32_grouped": (ctypes.c_int, [ctypes.c_int, _vp, _vp, _vp, _c_i64, _vp, _c_i64,
                                                     _vp, ctypes.c_int, _vp, _vp, _vp, _vp, _c_size,
                                                     _vp]),
    "bitlinear_rmsnorm_quant": (ctypes.c_int, [_vp, _vp, _c_i64, _c_i64, _vp, _vp, _vp, _vp]),
    "bitlinear_forward_rmsnorm_workspace_bytes": (_c_size, [_c_i64, _c_i64, _c_i64]),
    "bitlinear_forward_rmsnorm": (ctypes.c_int, [_vp, _vp, _c_i64, _c_i64, _vp, _vp, _c_i64, _vp,
                                                 ctypes.c_int, _vp, _vp, _vp, _vp, _c_size, _vp]),
    "bitlinear_forward_rmsnorm_grouped_workspace_bytes": (_c_size, [_c_i64, ctypes.c_int, _vp,
                                                                    _c_i64]),
    "bitlinear_forward_rmsnorm_grouped": (ctypes.c_int, [ctypes.c_int, _vp, _vp, _vp, _c_i64, _vp,
                                                         _vp, _c_i64, _vp, ctypes.c_int, _vp, _vp,
                                                         _vp, _vp, _c_size, _vp]),
    "bitlinear_forward_kernel": (ctypes.c_int, [ctypes.c_int, _c_i64, ctypes.c_int, _vp, _c_i64]),
    "bitlinear_packed3_bytes": (_c_size, [_c_i64, _c_i64]),
    "bitlinear_pack_weights_base3": (ctypes.c_int, [_vp, _c_i64, _c_i64, _vp, _vp, _vp, _c_size,
                                                    _vp]),
    "bitlinear_forward_base3": (ctypes.c_int, [_vp, _vp, _c_i64, _c_i64, _vp, _vp, _vp, _c_i64,
                                               _vp, ctypes.c_int, _vp]),
    "bitlinear_base3_to_blt2": (ctypes.c_int, [_vp, _c_i64, _c_i64, _vp, _vp]),
    "bitlinear_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "bitlinear_last_error": (ctypes.c_char_p, []),
}

_lib = None


class BitLinearError(RuntimeError):
    def __init__(self, status: int, detail: str):
        self.status = status
        super().__init__(f"{STATUS.get(status, status)}: {detail}")


def load(path: str | None = None) -> ctypes.CDLL:
    """Load the library once.  torch is imported first so that the library binds
    to the HIP runtime torch already loaded (same soname), which makes torch's
    stream handles valid inside the library."""
    global _lib
    if _lib is not None:
        return _lib
    import torch  # noqa: F401  (HIP runtime first)
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is missing: build it with ternary_bitlinear_amd.build.build()")
    lib = ctypes.CDLL(p)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _check(status: int) -> None:
    if status != 0:
        raise BitLinearError(status, _lib.bitlinear_last_error().decode())


def _stream(stream) -> int:
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream if hasattr(s, "cuda_stream") else int(s)


def _dev(t, dtype, name):
    import torch
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def packed_bytes(N: int, K: int) -> int:
    return load().bitlinear_packed_bytes(N, K)


def pack_workspace_bytes(N: int, K: int) -> int:
    return load().bitlinear_pack_workspace_bytes(N, K)


def forward_workspace_bytes(M: int, N: int, K: int) -> int:
    return load().bitlinear_forward_workspace_bytes(M, N, K)


def bitlinear_pack_weights(W, W_packed=None, gamma=None, workspace=None, stream=None):
    """W [N][K] fp32 -> (W_packed uint8 [N][K/4], gamma fp32 [1]) on W's device."""
    import torch
    lib = load()
    _dev(W, torch.float32, "W")
    N, K = W.shape
    if W_packed is None:
        W_packed = torch.empty((N, K // 4), dtype=torch.uint8, device=W.device)
    if gamma is None:
        gamma = torch.empty(1, dtype=torch.float32, device=W.device)
    need = lib.bitlinear_pack_workspace_bytes(N, K)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=W.device)
    _dev(W_packed, torch.uint8, "W_packed")
    _dev(gamma, torch.float32, "gamma")
    _check(lib.bitlinear_pack_weights(W.data_ptr(), N, K, W_packed.data_ptr(), gamma.data_ptr(),
                                      workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                      _stream(stream)))
    return W_packed, gamma


def packed3_bytes(N: int, K: int) -> int:
    return load().bitlinear_packed3_bytes(N, K)


def bitlinear_pack_weights_base3(W, W_packed3=None, gamma=None, workspace=None, stream=None):
    """W [N][K] fp32 -> (W_packed3 uint8 [N][16 ceil(K/80)] in format BLT3-v1, gamma fp32 [1])."""
    import torch
    lib = load()
    _dev(W, torch.float32, "W")
    N, K = W.shape
    if W_packed3 is None:
        W_packed3 = torch.empty((N, 16 * -(-K // 80)), dtype=torch.uint8, device=W.device)
    if gamma is None:
        gamma = torch.empty(1, dtype=torch.float32, device=W.device)
    need = lib.bitlinear_pack_workspace_bytes(N, K)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=W.device)
    _dev(W_packed3, torch.uint8, "W_packed3")
    _dev(gamma, torch.float32, "gamma")
    _check(lib.bitlinear_pack_weights_base3(W.data_ptr(), N, K, W_packed3.data_ptr(),
                                            gamma.data_ptr(), workspace.data_ptr(),
                                            workspace.numel() * workspace.element_size(),
                                            _stream(stream)))
    return W_packed3, gamma


def bitlinear_forward_base3(W_packed3, gamma, X_q, x_scale, x_sum, N=None, K=None,
                            y_dtype="bf16", Y=None, stream=None):
    """BLT3-v1 weights and quantised X (1 <= M <= 16) -> Y [M][N]."""
    import torch
    lib = load()
    _dev(W_packed3, torch.uint8, "W_packed3")
    _dev(X_q, torch.int8, "X_q")
    M, Kx = X_q.shape
    K = Kx if K is None else K
    N = W_packed3.shape[0] if N is None else N
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "i32": torch.int32}[y_dtype]
    if Y is None:
        Y = torch.empty((M, N), dtype=tdt, device=X_q.device)
    _dev(Y, tdt, "Y")
    _check(lib.bitlinear_forward_base3(W_packed3.data_ptr(), gamma.data_ptr(), N, K,
                                       X_q.data_ptr(), x_scale.data_ptr(), x_sum.data_ptr(), M,
                                       Y.data_ptr(), DTYPES[y_dtype], _stream(stream)))
    return Y


def bitlinear_base3_to_blt2(W_packed3, K, W_packed=None, stream=None):
    """BLT3-v1 rows [N][16 ceil(K/80)] -> BLT2-v1 rows [N][K/4] (the same codes)."""
    import torch
    lib = load()
    _dev(W_packed3, torch.uint8, "W_packed3")
    N = W_packed3.shape[0]
    if W_packed is None:
        W_packed = torch.empty((N, K // 4), dtype=torch.uint8, device=W_packed3.device)
    _dev(W_packed, torch.uint8, "W_packed")
    _check(lib.bitlinear_base3_to_blt2(W_packed3.data_ptr(), N, K, W_packed.data_ptr(),
                                       _stream(stream)))
    return W_packed


def bitlinear_quant_acts(X, X_q=None, x_scale=None, x_sum=None, stream=None, bits=8):
    """X [M][K] fp32 -> (X_q int8 [M][K], x_scale fp32 [M], x_sum int32 [M]); bits = 8,
    or 4 for activations in [-7, 7] (still one per int8 element)."""
    import torch
    lib = load()
    _dev(X, torch.float32, "X")
    M, K = X.shape
    if X_q is None:
        X_q = torch.empty((M, K), dtype=torch.int8, device=X.device)
    if x_scale is None:
        x_scale = torch.empty(M, dtype=torch.float32, device=X.device)
    if x_sum is None:
        x_sum = torch.empty(M, dtype=torch.int32, device=X.device)
    _dev(X_q, torch.int8, "X_q")
    _dev(x_scale, torch.float32, "x_scale")
    _dev(x_sum, torch.int32, "x_sum")
    _check(lib.bitlinear_quant_acts_bits(X.data_ptr(), M, K, bits, X_q.data_ptr(),
                                         x_scale.data_ptr(), x_sum.data_ptr(), _stream(stream)))
    return X_q, x_scale, x_sum


def bitlinear_forward(W_packed, gamma, X_q, x_scale, x_sum, N=None, K=None, y_dtype="bf16",
                      Y=None, workspace=None, stream=None):
    """Packed W~ and quantised X -> Y [M][N] (fp32, bf16 or raw int32 accumulators)."""
    import torch
    lib = load()
    _dev(W_packed, torch.uint8, "W_packed")
    _dev(X_q, torch.int8, "X_q")
    M, Kx = X_q.shape
    K = Kx if K is None else K
    N = W_packed.shape[0] if N is None else N
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "i32": torch.int32}[y_dtype]
    if Y is None:
        Y = torch.empty((M, N), dtype=tdt, device=X_q.device)
    _dev(Y, tdt, "Y")
    ws_need = lib.bitlinear_forward_workspace_bytes(M, N, K)
    if workspace is None and ws_need:
        workspace = torch.empty(ws_need, dtype=torch.uint8, device=X_q.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib.bitlinear_forward(W_packed.data_ptr(), gamma.data_ptr(), N, K, X_q.data_ptr(),
                                 x_scale.data_ptr(), x_sum.data_ptr(), M, Y.data_ptr(),
                                 DTYPES[y_dtype], ws_ptr, ws_bytes, _stream(stream)))
    return Y


def forward_f32_workspace_bytes(M: int, N: int, K: int) -> int:
    return load().bitlinear_forward_f32_workspace_bytes(M, N, K)


def bitlinear_forward_f32(W_packed, gamma, X, N=None, y_dtype="bf16", Y=None, X_q_out=None,
                          x_scale_out=None, x_sum_out=None, workspace=None, stream=None):
    """Quantise fp32 X [M][K] and project in one call -> Y [M][N]."""
    return _forward_f32(W_packed, gamma, X, None, N, y_dtype, Y, X_q_out, x_scale_out,
                        x_sum_out, workspace, stream)


def bitlinear_forward_rmsnorm(W_packed, gamma, X, norm_g, N=None, y_dtype="bf16", Y=None,
                              X_q_out=None, x_scale_out=None, x_sum_out=None, workspace=None,
                              stream=None):
    """RMS-normalise fp32 X [M][K] with gain norm_g [K], quantise and project -> Y [M][N]."""
    return _forward_f32(W_packed, gamma, X, norm_g, N, y_dtype, Y, X_q_out, x_scale_out,
                        x_sum_out, workspace, stream)


def _forward_f32(W_packed, gamma, X, norm_g, N, y_dtype, Y, X_q_out, x_scale_out, x_sum_out,
                 workspace, stream):
    import torch
    lib = load()
    _dev(W_packed, torch.uint8, "W_packed")
    _dev(X, torch.float32, "X")
    if norm_g is not None:
        _dev(norm_g, torch.float32, "norm_g")
    M, K = X.shape
    N = W_packed.shape[0] if N is None else N
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "i32": torch.int32}[y_dtype]
    if Y is None:
        Y = torch.empty((M, N), dtype=tdt, device=X.device)
    _dev(Y, tdt, "Y")
    outs = (X_q_out, x_scale_out, x_sum_out)
    if X_q_out is not None:
        _dev(X_q_out, torch.int8, "X_q_out")
        _dev(x_scale_out, torch.float32, "x_scale_out")
        _dev(x_sum_out, torch.int32, "x_sum_out")
    need = (lib.bitlinear_forward_f32_workspace_bytes(M, N, K) if norm_g is None
            else lib.bitlinear_forward_rmsnorm_workspace_bytes(M, N, K))
    if X_q_out is not None and (M <= 16 or lib.bitlinear_forward_workspace_bytes(M, N, K) == 0):
        need = 0   # outputs given and the projection needs no workspace of its own
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=X.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    ptr = [o.data_ptr() if o is not None else None for o in outs]
    if norm_g is None:
        _check(lib.bitlinear_forward_f32(W_packed.data_ptr(), gamma.data_ptr(), N, K,
                                         X.data_ptr(), M, Y.data_ptr(), DTYPES[y_dtype], ptr[0],
                                         ptr[1], ptr[2], ws_ptr, ws_bytes, _stream(stream)))
    else:
        _check(lib.bitlinear_forward_rmsnorm(W_packed.data_ptr(), gamma.data_ptr(), N, K,
                                             X.data_ptr(), norm_g.data_ptr(), M, Y.data_ptr(),
                                             DTYPES[y_dtype], ptr[0], ptr[1], ptr[2], ws_ptr,
                                             ws_bytes, _stream(stream)))
    return Y


def forward_rmsnorm_workspace_bytes(M: int, N: int, K: int) -> int:
    return load().bitlinear_forward_rmsnorm_workspace_bytes(M, N, K)


def bitlinear_rmsnorm_quant(X, norm_g, X_q=None, x_scale=None, x_sum=None, stream=None):
    """RMS-normalise fp32 X [M][K] with gain norm_g [K], then quantise:
    -> (X_q int8 [M][K], x_scale fp32 [M], x_sum int32 [M])."""
    import torch
    lib = load()
    _dev(X, torch.float32, "X")
    _dev(norm_g, torch.float32, "norm_g")
    M, K = X.shape
    if X_q is None:
        X_q = torch.empty((M, K), dtype=torch.int8, device=X.device)
    if x_scale is None:
        x_scale = torch.empty(M, dtype=torch.float32, device=X.device)
    if x_sum is None:
        x_sum = torch.empty(M, dtype=torch.int32, device=X.device)
    _check(lib.bitlinear_rmsnorm_quant(X.data_ptr(), norm_g.data_ptr(), M, K, X_q.data_ptr(),
                                       x_scale.data_ptr(), x_sum.data_ptr(), _stream(stream)))
    return X_q, x_scale, x_sum


MAX_GROUP = 4


def _ptr_array(ts):
    return (ctypes.c_void_p * len(ts))(*[t.data_ptr() for t in ts])


def _i64_array(vals):
    return (ctypes.c_int64 * len(vals))(*vals)


def forward_grouped_workspace_bytes(M: int, Ns, K: int) -> int:
    return load().bitlinear_forward_grouped_workspace_bytes(M, len(Ns), _i64_array(Ns), K)


def forward_f32_grouped_workspace_bytes(M: int, Ns, K: int) -> int:
    return load().bitlinear_forward_f32_grouped_workspace_bytes(M, len(Ns), _i64_array(Ns), K)


def _outputs(Ns, M, y_dtype, device, Y):
    import torch
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "i32": torch.int32}[y_dtype]
    if Y is None:
        Y = [torch.empty((M, n), dtype=tdt, device=device) for n in Ns]
    if len(Y) != len(Ns):
        raise ValueError("one output per projection")
    for y in Y:
        _dev(y, tdt, "Y")
    return Y


def bitlinear_forward_grouped(W_packed, gamma, X_q, x_scale, x_sum, Ns=None, K=None,
                              y_dtype="bf16", Y=None, workspace=None, stream=None):
    """Several packed projections of one quantised X~ -> list of Y [M][N_g]."""
    import torch
    lib = load()
    G = len(W_packed)
    if len(gamma) != G:
        raise ValueError("one gamma per projection")
    for w in W_packed:
        _dev(w, torch.uint8, "W_packed")
    _dev(X_q, torch.int8, "X_q")
    M, Kx = X_q.shape
    K = Kx if K is None else K
    Ns = [w.shape[0] for w in W_packed] if Ns is None else list(Ns)
    Y = _outputs(Ns, M, y_dtype, X_q.device, Y)
    need = lib.bitlinear_forward_grouped_workspace_bytes(M, G, _i64_array(Ns), K)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=X_q.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib.bitlinear_forward_grouped(G, _ptr_array(W_packed), _ptr_array(gamma), _i64_array(Ns),
                                         K, X_q.data_ptr(), x_scale.data_ptr(), x_sum.data_ptr(), M,
                                         _ptr_array(Y), DTYPES[y_dtype], ws_ptr, ws_bytes,
                                         _stream(stream)))
    return Y


def bitlinear_forward_f32_grouped(W_packed, gamma, X, Ns=None, y_dtype="bf16", Y=None,
                                  X_q_out=None, x_scale_out=None, x_sum_out=None, workspace=None,
                                  stream=None):
    """Quantise fp32 X [M][K] once and run every packed projection -> list of Y."""
    return _forward_f32_grouped(W_packed, gamma, X, None, Ns, y_dtype, Y, X_q_out, x_scale_out,
                                x_sum_out, workspace, stream)


def bitlinear_forward_rmsnorm_grouped(W_packed, gamma, X, norm_g, Ns=None, y_dtype="bf16",
                                      Y=None, X_q_out=None, x_scale_out=None, x_sum_out=None,
                                      workspace=None, stream=None):
    """RMS-normalise fp32 X [M][K] with gain norm_g [K], quantise once and run every packed
    projection -> list of Y."""
    return _forward_f32_grouped(W_packed, gamma, X, norm_g, Ns, y_dtype, Y, X_q_out,
                                x_scale_out, x_sum_out, workspace, stream)


def forward_rmsnorm_grouped_workspace_bytes(M: int, Ns, K: int) -> int:
    return load().bitlinear_forward_rmsnorm_grouped_workspace_bytes(M, len(Ns), _i64_array(Ns), K)


KERNELS = {1: "k_decode_dot", 2: "k_decode", 3: "k_skinny", 4: "k_gemm"}
ENTRIES = {"forward": 0, "f32": 1, "rmsnorm": 2}


def forward_kernel(entry: str, M: int, Ns, K: int):
    """(kernel name, quantiser fused) that the forward entry point ("forward",
    "f32" or "rmsnorm", single or grouped over Ns) launches for these sizes."""
    r = load().bitlinear_forward_kernel(ENTRIES[entry], M, len(Ns), _i64_array(Ns), K)
    if r < 0:
        raise BitLinearError(-r, f"forward_kernel: invalid sizes M={M} Ns={list(Ns)} K={K}")
    return KERNELS[r & 15], bool(r & 16)


def _forward_f32_grouped(W_packed, gamma, X, norm_g, Ns, y_dtype, Y, X_q_out, x_scale_out,
                         x_sum_out, workspace, stream):
    import torch
    lib = load()
    if norm_g is not None:
        _dev(norm_g, torch.float32, "norm_g")
    G = len(W_packed)
    if len(gamma) != G:
        raise ValueError("one gamma per projection")
    for w in W_packed:
        _dev(w, torch.uint8, "W_packed")
    _dev(X, torch.float32, "X")
    M, K = X.shape
    Ns = [w.shape[0] for w in W_packed] if Ns is None else list(Ns)
    Y = _outputs(Ns, M, y_dtype, X.device, Y)
    outs = (X_q_out, x_scale_out, x_sum_out)
    if X_q_out is not None:
        _dev(X_q_out, torch.int8, "X_q_out")
        _dev(x_scale_out, torch.float32, "x_scale_out")
        _dev(x_sum_out, torch.int32, "x_sum_out")
    n_arr = _i64_array(Ns)
    need = (lib.bitlinear_forward_f32_grouped_workspace_bytes(M, G, n_arr, K) if norm_g is None
            else lib.bitlinear_forward_rmsnorm_grouped_workspace_bytes(M, G, n_arr, K))
    if X_q_out is not None and (M <= 16 or lib.bitlinear_forward_grouped_workspace_bytes(
            M, G, n_arr, K) == 0):
        need = 0   # outputs given and the projections need no workspace of their own
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=X.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    ptr = [o.data_ptr() if o is not None else None for o in outs]
    if norm_g is None:
        _check(lib.bitlinear_forward_f32_grouped(G, _ptr_array(W_packed), _ptr_array(gamma), n_arr,
                                                 K, X.data_ptr(), M, _ptr_array(Y),
                                                 DTYPES[y_dtype], ptr[0], ptr[1], ptr[2], ws_ptr,
                                                 ws_bytes, _stream(stream)))
    else:
        _check(lib.bitlinear_forward_rmsnorm_grouped(G, _ptr_array(W_packed), _ptr_array(gamma),
                                                     n_arr, K, X.data_ptr(), norm_g.data_ptr(), M,
                                                     _ptr_array(Y), DTYPES[y_dtype], ptr[0],
                                                     ptr[1], ptr[2], ws_ptr, ws_bytes,
                                                     _stream(stream)))
    return Y
