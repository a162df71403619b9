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
    "bitlinear_forward_f32_noalloc": (ctypes.c_int, [_vp, _vp, _c_i64, _c_i64, _vp, _c_i64, _vp,
                                                     ctypes.c_int, _vp, _vp, _vp, _vp]),
    "bitlinear_forward_f32_multi_workspace_bytes": (_c_size, [_c_i64, ctypes.c_int, _vp, _vp]),
    "bitlinear_forward_f32_multi_kernel": (ctypes.c_int, [_c_i64, ctypes.c_int, _vp, _vp]),
    "bitlinear_forward_f32_multi": (ctypes.c_int, [ctypes.c_int, _vp, _vp, _vp, _vp, _vp, _c_i64,
                                                   _vp, ctypes.c_int, _vp, _c_size, _vp]),
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


def _t(t, dtype, name, shape=None, numel=None, min_bytes=None):
    """One tensor argument: a contiguous torch tensor of `dtype` with exactly
    `shape` (or `numel` elements, or at least `min_bytes` bytes).  The C ABI
    sees only a pointer, so this is the only place a wrong size can be caught:
    it raises before any library call."""
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor, got {type(t).__name__}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} must hold {numel} elements, got {t.numel()}")
    if min_bytes is not None and t.numel() * t.element_size() < min_bytes:
        raise ValueError(f"{name} must hold at least {min_bytes} bytes, got "
                         f"{t.numel() * t.element_size()}")
    return t


def _on_device(*named):
    """Every given tensor ((name, tensor) pairs; None skipped) is device memory of
    one GPU."""
    devs = set()
    for name, t in named:
        if t is None:
            continue
        if not t.is_cuda:
            raise TypeError(f"{name} must be a CUDA (HIP) tensor")
        devs.add(t.device)
    if len(devs) > 1:
        raise ValueError(f"all tensors must be on one device, got {sorted(map(str, devs))}")


def _ws(lib_need, workspace, device):
    """The caller's workspace (uint8, at least the size query's bytes) or a new one."""
    import torch
    if workspace is None:
        if not lib_need:
            return None
        return torch.empty(lib_need, dtype=torch.uint8, device=device)
    return _t(workspace, torch.uint8, "workspace", min_bytes=lib_need)


def _ws_args(workspace):
    if workspace is None:
        return None, 0
    return workspace.data_ptr(), workspace.numel() * workspace.element_size()


def _ydt(y_dtype):
    import torch
    if y_dtype not in DTYPES:
        raise ValueError(f"y_dtype must be one of {sorted(DTYPES)}, got {y_dtype!r}")
    return {"f32": torch.float32, "bf16": torch.bfloat16, "i32": torch.int32}[y_dtype]


def _quant_outs(M, K, X_q_out, x_scale_out, x_sum_out):
    """The optional quantiser outputs of the fp32 entry points: all three or none."""
    import torch
    outs = (X_q_out, x_scale_out, x_sum_out)
    given = sum(o is not None for o in outs)
    if given not in (0, 3):
        raise ValueError("X_q_out, x_scale_out and x_sum_out go together")
    if given:
        _t(X_q_out, torch.int8, "X_q_out", shape=(M, K))
        _t(x_scale_out, torch.float32, "x_scale_out", shape=(M,))
        _t(x_sum_out, torch.int32, "x_sum_out", shape=(M,))
    return outs


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
    _t(W, torch.float32, "W")
    if W.dim() != 2:
        raise ValueError(f"W must be 2-D [N][K], got shape {tuple(W.shape)}")
    N, K = W.shape
    if W_packed is None:
        W_packed = torch.empty((N, K // 4), dtype=torch.uint8, device=W.device)
    if gamma is None:
        gamma = torch.empty(1, dtype=torch.float32, device=W.device)
    _t(W_packed, torch.uint8, "W_packed", numel=N * (K // 4))
    _t(gamma, torch.float32, "gamma", numel=1)
    need = lib.bitlinear_pack_workspace_bytes(N, K)
    workspace = _ws(max(need, 16), workspace, W.device)
    _on_device(("W", W), ("W_packed", W_packed), ("gamma", gamma), ("workspace", workspace))
    _check(lib.bitlinear_pack_weights(W.data_ptr(), N, K, W_packed.data_ptr(), gamma.data_ptr(),
                                      *_ws_args(workspace), _stream(stream)))
    return W_packed, gamma


def packed3_bytes(N: int, K: int) -> int:
    return load().bitlinear_packed3_bytes(N, K)


def _packed3_row(K):
    return 16 * -(-K // 80)


def bitlinear_pack_weights_base3(W, W_packed3=None, gamma=None, workspace=None, stream=None):
    """W [N][K] fp32 -> (W_packed3 uint8 [N][16 ceil(K/80)] in format BLT3-v1, gamma fp32 [1])."""
    import torch
    lib = load()
    _t(W, torch.float32, "W")
    if W.dim() != 2:
        raise ValueError(f"W must be 2-D [N][K], got shape {tuple(W.shape)}")
    N, K = W.shape
    if W_packed3 is None:
        W_packed3 = torch.empty((N, _packed3_row(K)), dtype=torch.uint8, device=W.device)
    if gamma is None:
        gamma = torch.empty(1, dtype=torch.float32, device=W.device)
    _t(W_packed3, torch.uint8, "W_packed3", numel=N * _packed3_row(K))
    _t(gamma, torch.float32, "gamma", numel=1)
    need = lib.bitlinear_pack_workspace_bytes(N, K)
    workspace = _ws(max(need, 16), workspace, W.device)
    _on_device(("W", W), ("W_packed3", W_packed3), ("gamma", gamma), ("workspace", workspace))
    _check(lib.bitlinear_pack_weights_base3(W.data_ptr(), N, K, W_packed3.data_ptr(),
                                            gamma.data_ptr(), *_ws_args(workspace),
                                            _stream(stream)))
    return W_packed3, gamma


def _acts_q(X_q, x_scale, x_sum, K=None):
    """Quantised activations: X_q int8 [M][K], x_scale fp32 [M], x_sum int32 [M]."""
    import torch
    _t(X_q, torch.int8, "X_q")
    if X_q.dim() != 2:
        raise ValueError(f"X_q must be 2-D [M][K], got shape {tuple(X_q.shape)}")
    M, Kx = X_q.shape
    if K is not None and K != Kx:
        raise ValueError(f"X_q has {Kx} columns, K = {K}")
    _t(x_scale, torch.float32, "x_scale", shape=(M,))
    _t(x_sum, torch.int32, "x_sum", shape=(M,))
    return M, Kx


def bitlinear_forward_base3(W_packed3, gamma, X_q, x_scale, x_sum, N=None, K=None,
                            y_dtype="bf16", Y=None, stream=None):
    """BLT3-v1 weights and quantised X (1 <= M <= 16) -> Y [M][N]."""
    import torch
    lib = load()
    M, K = _acts_q(X_q, x_scale, x_sum, K)
    _t(W_packed3, torch.uint8, "W_packed3")
    N = W_packed3.shape[0] if N is None else N
    _t(W_packed3, torch.uint8, "W_packed3", numel=N * _packed3_row(K))
    _t(gamma, torch.float32, "gamma", numel=1)
    tdt = _ydt(y_dtype)
    if Y is None:
        Y = torch.empty((M, N), dtype=tdt, device=X_q.device)
    _t(Y, tdt, "Y", shape=(M, N))
    _on_device(("W_packed3", W_packed3), ("gamma", gamma), ("X_q", X_q), ("x_scale", x_scale),
               ("x_sum", x_sum), ("Y", Y))
    _check(lib.bitlinear_forward_base3(W_packed3.data_ptr(), gamma.data_ptr(), N, K,
                                       X_q.data_ptr(), x_scale.data_ptr(), x_sum.data_ptr(), M,
                                       Y.data_ptr(), DTYPES[y_dtype], _stream(stream)))
    return Y


def bitlinear_base3_to_blt2(W_packed3, K, W_packed=None, stream=None):
    """BLT3-v1 rows [N][16 ceil(K/80)] -> BLT2-v1 rows [N][K/4] (the same codes)."""
    import torch
    lib = load()
    _t(W_packed3, torch.uint8, "W_packed3")
    N = W_packed3.shape[0]
    _t(W_packed3, torch.uint8, "W_packed3", numel=N * _packed3_row(K))
    if W_packed is None:
        W_packed = torch.empty((N, K // 4), dtype=torch.uint8, device=W_packed3.device)
    _t(W_packed, torch.uint8, "W_packed", numel=N * (K // 4))
    _on_device(("W_packed3", W_packed3), ("W_packed", W_packed))
    _check(lib.bitlinear_base3_to_blt2(W_packed3.data_ptr(), N, K, W_packed.data_ptr(),
                                       _stream(stream)))
    return W_packed


def bitlinear_quant_acts(X, X_q=None, x_scale=None, x_sum=None, stream=None, bits=8):
    """X [M][K] fp32 -> (X_q int8 [M][K], x_scale fp32 [M], x_sum int32 [M]); bits = 8,
    or 4 for activations in [-7, 7] (still one per int8 element)."""
    import torch
    lib = load()
    _t(X, torch.float32, "X")
    if X.dim() != 2:
        raise ValueError(f"X must be 2-D [M][K], got shape {tuple(X.shape)}")
    M, K = X.shape
    if X_q is None:
        X_q = torch.empty((M, K), dtype=torch.int8, device=X.device)
    if x_scale is None:
        x_scale = torch.empty(M, dtype=torch.float32, device=X.device)
    if x_sum is None:
        x_sum = torch.empty(M, dtype=torch.int32, device=X.device)
    _acts_q(X_q, x_scale, x_sum, K)
    if X_q.shape[0] != M:
        raise ValueError(f"X_q must have shape {(M, K)}, got {tuple(X_q.shape)}")
    _on_device(("X", X), ("X_q", X_q), ("x_scale", x_scale), ("x_sum", x_sum))
    _check(lib.bitlinear_quant_acts_bits(X.data_ptr(), M, K, bits, X_q.data_ptr(),
                                         x_scale.data_ptr(), x_sum.data_ptr(), _stream(stream)))
    return X_q, x_scale, x_sum


def _weights(W_packed, gamma, N, K):
    import torch
    _t(W_packed, torch.uint8, "W_packed")
    N = W_packed.shape[0] if N is None else N
    _t(W_packed, torch.uint8, "W_packed", numel=N * (K // 4))
    _t(gamma, torch.float32, "gamma", numel=1)
    return N


def bitlinear_forward(W_packed, gamma, X_q, x_scale, x_sum, N=None, K=None, y_dtype="bf16",
                      Y=None, workspace=None, stream=None):
    """Packed W~ and quantised X -> Y [M][N] (fp32, bf16 or raw int32 accumulators)."""
    import torch
    lib = load()
    M, K = _acts_q(X_q, x_scale, x_sum, K)
    N = _weights(W_packed, gamma, N, K)
    tdt = _ydt(y_dtype)
    if Y is None:
        Y = torch.empty((M, N), dtype=tdt, device=X_q.device)
    _t(Y, tdt, "Y", shape=(M, N))
    workspace = _ws(lib.bitlinear_forward_workspace_bytes(M, N, K), workspace, X_q.device)
    _on_device(("W_packed", W_packed), ("gamma", gamma), ("X_q", X_q), ("x_scale", x_scale),
               ("x_sum", x_sum), ("Y", Y), ("workspace", workspace))
    _check(lib.bitlinear_forward(W_packed.data_ptr(), gamma.data_ptr(), N, K, X_q.data_ptr(),
                                 x_scale.data_ptr(), x_sum.data_ptr(), M, Y.data_ptr(),
                                 DTYPES[y_dtype], *_ws_args(workspace), _stream(stream)))
    return Y


def forward_f32_workspace_bytes(M: int, N: int, K: int) -> int:
    return load().bitlinear_forward_f32_workspace_bytes(M, N, K)


def bitlinear_forward_f32(W_packed, gamma, X, N=None, y_dtype="bf16", Y=None, X_q_out=None,
                          x_scale_out=None, x_sum_out=None, workspace=None, stream=None):
    """Quantise fp32 X [M][K] and project in one call -> Y [M][N]."""
    return _forward_f32(W_packed, gamma, X, None, N, y_dtype, Y, X_q_out, x_scale_out,
                        x_sum_out, workspace, stream)


NOALLOC_SCRATCH_BYTES = 32 << 20   # BITLINEAR_NOALLOC_SCRATCH_BYTES


def bitlinear_forward_f32_noalloc(W_packed, gamma, X, N=None, y_dtype="bf16", Y=None,
                                  X_q_out=None, x_scale_out=None, x_sum_out=None, stream=None):
    """bitlinear_forward_f32 with the library's own scratch array as workspace (no
    allocation inside the library; calls overlapping on one GPU race on it).
    Y is allocated here when not given."""
    import torch
    lib = load()
    M, K = _acts_f32(X)
    N = _weights(W_packed, gamma, N, K)
    tdt = _ydt(y_dtype)
    if Y is None:
        Y = torch.empty((M, N), dtype=tdt, device=X.device)
    _t(Y, tdt, "Y", shape=(M, N))
    outs = _quant_outs(M, K, X_q_out, x_scale_out, x_sum_out)
    _on_device(("W_packed", W_packed), ("gamma", gamma), ("X", X), ("Y", Y),
               ("X_q_out", X_q_out), ("x_scale_out", x_scale_out), ("x_sum_out", x_sum_out))
    ptr = [o.data_ptr() if o is not None else None for o in outs]
    _check(lib.bitlinear_forward_f32_noalloc(W_packed.data_ptr(), gamma.data_ptr(), N, K,
                                             X.data_ptr(), M, Y.data_ptr(), DTYPES[y_dtype],
                                             ptr[0], ptr[1], ptr[2], _stream(stream)))
    return Y


def bitlinear_forward_rmsnorm(W_packed, gamma, X, norm_g, N=None, y_dtype="bf16", Y=None,
                              X_q_out=None, x_scale_out=None, x_sum_out=None, workspace=None,
                              stream=None):
    """RMS-normalise fp32 X [M][K] with gain norm_g [K], quantise and project -> Y [M][N]."""
    return _forward_f32(W_packed, gamma, X, norm_g, N, y_dtype, Y, X_q_out, x_scale_out,
                        x_sum_out, workspace, stream)


def _acts_f32(X):
    import torch
    _t(X, torch.float32, "X")
    if X.dim() != 2:
        raise ValueError(f"X must be 2-D [M][K], got shape {tuple(X.shape)}")
    return X.shape


def _forward_f32(W_packed, gamma, X, norm_g, N, y_dtype, Y, X_q_out, x_scale_out, x_sum_out,
                 workspace, stream):
    import torch
    lib = load()
    M, K = _acts_f32(X)
    N = _weights(W_packed, gamma, N, K)
    if norm_g is not None:
        _t(norm_g, torch.float32, "norm_g", numel=K)
    tdt = _ydt(y_dtype)
    if Y is None:
        Y = torch.empty((M, N), dtype=tdt, device=X.device)
    _t(Y, tdt, "Y", shape=(M, N))
    outs = _quant_outs(M, K, X_q_out, x_scale_out, x_sum_out)
    need = (lib.bitlinear_forward_f32_workspace_bytes(M, N, K) if norm_g is None
            else lib.bitlinear_forward_rmsnorm_workspace_bytes(M, N, K))
    if X_q_out is not None and (M <= 16 or lib.bitlinear_forward_workspace_bytes(M, N, K) == 0):
        need = 0   # outputs given and the projection needs no workspace of its own
    workspace = _ws(need, workspace, X.device)
    _on_device(("W_packed", W_packed), ("gamma", gamma), ("X", X), ("norm_g", norm_g),
               ("Y", Y), ("X_q_out", X_q_out), ("x_scale_out", x_scale_out),
               ("x_sum_out", x_sum_out), ("workspace", workspace))
    ws_ptr, ws_bytes = _ws_args(workspace)
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
    M, K = _acts_f32(X)
    _t(norm_g, torch.float32, "norm_g", numel=K)
    if X_q is None:
        X_q = torch.empty((M, K), dtype=torch.int8, device=X.device)
    if x_scale is None:
        x_scale = torch.empty(M, dtype=torch.float32, device=X.device)
    if x_sum is None:
        x_sum = torch.empty(M, dtype=torch.int32, device=X.device)
    _t(X_q, torch.int8, "X_q", shape=(M, K))
    _t(x_scale, torch.float32, "x_scale", shape=(M,))
    _t(x_sum, torch.int32, "x_sum", shape=(M,))
    _on_device(("X", X), ("norm_g", norm_g), ("X_q", X_q), ("x_scale", x_scale), ("x_sum", x_sum))
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
    tdt = _ydt(y_dtype)
    if Y is None:
        Y = [torch.empty((M, n), dtype=tdt, device=device) for n in Ns]
    if len(Y) != len(Ns):
        raise ValueError("one output per projection")
    for i, (y, n) in enumerate(zip(Y, Ns)):
        _t(y, tdt, f"Y[{i}]", shape=(M, n))
    return Y


def _group_weights(W_packed, gamma, Ns, K):
    import torch
    G = len(W_packed)
    if not 1 <= G <= MAX_GROUP:
        raise ValueError(f"1 to {MAX_GROUP} projections per call, got {G}")
    if len(gamma) != G:
        raise ValueError("one gamma per projection")
    for i, w in enumerate(W_packed):
        _t(w, torch.uint8, f"W_packed[{i}]")
    Ns = [w.shape[0] for w in W_packed] if Ns is None else list(Ns)
    if len(Ns) != G:
        raise ValueError("one N per projection")
    for i, (w, g, n) in enumerate(zip(W_packed, gamma, Ns)):
        _t(w, torch.uint8, f"W_packed[{i}]", numel=n * (K // 4))
        _t(g, torch.float32, f"gamma[{i}]", numel=1)
    return G, Ns


def _group_named(W_packed, gamma, Y):
    return ([(f"W_packed[{i}]", w) for i, w in enumerate(W_packed)]
            + [(f"gamma[{i}]", g) for i, g in enumerate(gamma)]
            + [(f"Y[{i}]", y) for i, y in enumerate(Y)])


def bitlinear_forward_grouped(W_packed, gamma, X_q, x_scale, x_sum, Ns=None, K=None,
                              y_dtype="bf16", Y=None, workspace=None, stream=None):
    """Several packed projections of one quantised X~ -> list of Y [M][N_g]."""
    lib = load()
    M, K = _acts_q(X_q, x_scale, x_sum, K)
    G, Ns = _group_weights(W_packed, gamma, Ns, K)
    Y = _outputs(Ns, M, y_dtype, X_q.device, Y)
    need = lib.bitlinear_forward_grouped_workspace_bytes(M, G, _i64_array(Ns), K)
    workspace = _ws(need, workspace, X_q.device)
    _on_device(("X_q", X_q), ("x_scale", x_scale), ("x_sum", x_sum), ("workspace", workspace),
               *_group_named(W_packed, gamma, Y))
    _check(lib.bitlinear_forward_grouped(G, _ptr_array(W_packed), _ptr_array(gamma), _i64_array(Ns),
                                         K, X_q.data_ptr(), x_scale.data_ptr(), x_sum.data_ptr(), M,
                                         _ptr_array(Y), DTYPES[y_dtype], *_ws_args(workspace),
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


KERNELS = {1: "k_decode_dot", 2: "k_decode", 3: "k_skinny", 4: "k_gemm", 5: "k_stream"}
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
    M, K = _acts_f32(X)
    if norm_g is not None:
        _t(norm_g, torch.float32, "norm_g", numel=K)
    G, Ns = _group_weights(W_packed, gamma, Ns, K)
    Y = _outputs(Ns, M, y_dtype, X.device, Y)
    outs = _quant_outs(M, K, X_q_out, x_scale_out, x_sum_out)
    n_arr = _i64_array(Ns)
    need = (lib.bitlinear_forward_f32_grouped_workspace_bytes(M, G, n_arr, K) if norm_g is None
            else lib.bitlinear_forward_rmsnorm_grouped_workspace_bytes(M, G, n_arr, K))
    if X_q_out is not None and (M <= 16 or lib.bitlinear_forward_grouped_workspace_bytes(
            M, G, n_arr, K) == 0):
        need = 0   # outputs given and the projections need no workspace of their own
    workspace = _ws(need, workspace, X.device)
    _on_device(("X", X), ("norm_g", norm_g), ("X_q_out", X_q_out),
               ("x_scale_out", x_scale_out), ("x_sum_out", x_sum_out), ("workspace", workspace),
               *_group_named(W_packed, gamma, Y))
    ws_ptr, ws_bytes = _ws_args(workspace)
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


def forward_f32_multi_workspace_bytes(M: int, Ns, Ks) -> int:
    return load().bitlinear_forward_f32_multi_workspace_bytes(M, len(Ns), _i64_array(Ns),
                                                             _i64_array(Ks))


def bitlinear_forward_f32_multi(W_packed, gamma, X, Ns=None, y_dtype="bf16", Y=None,
                                workspace=None, stream=None):
    """Several projections, each with its own fp32 activations X[g] [M][K_g] and
    packed weights W_packed[g] [N_g][K_g/4]: quantise and project every one ->
    list of Y [M][N_g] (one launch for a single token)."""
    import torch
    lib = load()
    G = len(W_packed)
    if not 1 <= G <= MAX_GROUP:
        raise ValueError(f"1 to {MAX_GROUP} projections per call, got {G}")
    if len(gamma) != G or len(X) != G:
        raise ValueError("one gamma and one X per projection")
    shapes = [_acts_f32(x) for x in X]
    Ms = {m for m, _ in shapes}
    if len(Ms) != 1:
        raise ValueError(f"every X must have the same number of tokens, got {sorted(Ms)}")
    M = shapes[0][0]
    Ks = [k for _, k in shapes]
    for i, w in enumerate(W_packed):
        _t(w, torch.uint8, f"W_packed[{i}]")
    Ns = [w.shape[0] for w in W_packed] if Ns is None else list(Ns)
    if len(Ns) != G:
        raise ValueError("one N per projection")
    for i, (w, g, n, k) in enumerate(zip(W_packed, gamma, Ns, Ks)):
        _t(w, torch.uint8, f"W_packed[{i}]", numel=n * (k // 4))
        _t(g, torch.float32, f"gamma[{i}]", numel=1)
    Y = _outputs(Ns, M, y_dtype, X[0].device, Y)
    n_arr, k_arr = _i64_array(Ns), _i64_array(Ks)
    need = lib.bitlinear_forward_f32_multi_workspace_bytes(M, G, n_arr, k_arr)
    workspace = _ws(need, workspace, X[0].device)
    _on_device(("workspace", workspace), *[(f"X[{i}]", x) for i, x in enumerate(X)],
               *_group_named(W_packed, gamma, Y))
    _check(lib.bitlinear_forward_f32_multi(G, _ptr_array(W_packed), _ptr_array(gamma), n_arr,
                                           k_arr, _ptr_array(X), M, _ptr_array(Y),
                                           DTYPES[y_dtype], *_ws_args(workspace),
                                           _stream(stream)))
    return Y


def forward_f32_multi_kernel(M: int, Ns, Ks):
    """("k_stream", True) when bitlinear_forward_f32_multi runs these sizes as
    one launch, None when it runs one bitlinear_forward_f32 per projection."""
    r = load().bitlinear_forward_f32_multi_kernel(M, len(Ns), _i64_array(Ns), _i64_array(Ks))
    if r < 0:
        raise BitLinearError(-r, f"forward_f32_multi_kernel: invalid sizes M={M} Ns={list(Ns)} "
                                 f"Ks={list(Ks)}")
    return (KERNELS[r & 15], bool(r & 16)) if r else None
