"""The Python binding checks every tensor it hands to the C ABI (type, dtype,
contiguity, size, device) and raises before any library call: the ABI sees
only pointers, so a wrong size would otherwise become an out-of-bounds device
access.  Runs on the host: CPU tensors of the wrong size raise ValueError,
CPU tensors of the right size raise TypeError (not device memory)."""
import pytest

torch = pytest.importorskip("torch")

import ternary_bitlinear_amd as tb  # noqa: E402

M, N, K = 3, 48, 64


def f32(*shape):
    return torch.zeros(shape, dtype=torch.float32)


def i8(*shape):
    return torch.zeros(shape, dtype=torch.int8)


def i32(*shape):
    return torch.zeros(shape, dtype=torch.int32)


def u8(*shape):
    return torch.zeros(shape, dtype=torch.uint8)


def acts():
    return i8(M, K), f32(M), i32(M)


@pytest.fixture(scope="module", autouse=True)
def lib():
    from ternary_bitlinear_amd.build import LIB, build
    import os
    if not os.path.exists(LIB):
        build()
    tb.load()


@pytest.mark.parametrize("call", [
    # swapped or truncated weights
    lambda: tb.bitlinear_forward(u8(N, K // 4 - 4), f32(1), *acts(), N=N),
    lambda: tb.bitlinear_forward(u8(N // 2, K // 4), f32(1), *acts(), N=N),
    # gamma, x_scale, x_sum of the wrong length or type
    lambda: tb.bitlinear_forward(u8(N, K // 4), f32(2), *acts()),
    lambda: tb.bitlinear_forward(u8(N, K // 4), f32(1), i8(M, K), f32(M + 1), i32(M)),
    lambda: tb.bitlinear_forward(u8(N, K // 4), f32(1), i8(M, K), f32(M), i32(M - 1)),
    lambda: tb.bitlinear_forward(u8(N, K // 4), f32(1), i8(M, K), f32(M), f32(M)),
    # X_q with K columns other than the weights'
    lambda: tb.bitlinear_forward(u8(N, K // 4), f32(1), i8(M, K), f32(M), i32(M), K=K + 16),
    # a caller-supplied Y of the wrong shape or type
    lambda: tb.bitlinear_forward(u8(N, K // 4), f32(1), *acts(), Y=torch.zeros((M, N + 1),
                                 dtype=torch.bfloat16)),
    lambda: tb.bitlinear_forward(u8(N, K // 4), f32(1), *acts(), y_dtype="f32",
                                 Y=torch.zeros((M, N), dtype=torch.bfloat16)),
    lambda: tb.bitlinear_forward(u8(N, K // 4), f32(1), *acts(), y_dtype="f16"),
    # workspace too small
    lambda: tb.bitlinear_forward(u8(N, 12288 // 4), f32(1), i8(64, 12288), f32(64), i32(64),
                                 workspace=u8(16)),
    # fp32 entry points: outputs of the wrong shape, or only some of them
    lambda: tb.bitlinear_forward_f32(u8(N, K // 4), f32(1), f32(M, K), X_q_out=i8(M, K + 16),
                                     x_scale_out=f32(M), x_sum_out=i32(M)),
    lambda: tb.bitlinear_forward_f32(u8(N, K // 4), f32(1), f32(M, K), X_q_out=i8(M, K)),
    lambda: tb.bitlinear_forward_f32(u8(N, K // 4), f32(1), f32(M, K), Y=f32(M + 1, N),
                                     y_dtype="f32"),
    lambda: tb.bitlinear_forward_f32_noalloc(u8(N, K // 4 + 1), f32(1), f32(M, K)),
    lambda: tb.bitlinear_forward_rmsnorm(u8(N, K // 4), f32(1), f32(M, K), f32(K + 4)),
    lambda: tb.bitlinear_rmsnorm_quant(f32(M, K), f32(K - 4)),
    # quantiser and packer outputs
    lambda: tb.bitlinear_quant_acts(f32(M, K), X_q=i8(M, K - 16)),
    lambda: tb.bitlinear_quant_acts(f32(M, K), x_scale=f32(M + 1)),
    lambda: tb.bitlinear_pack_weights(f32(N, K), W_packed=u8(N, K // 8)),
    lambda: tb.bitlinear_pack_weights(f32(N, K), gamma=f32(2)),
    lambda: tb.bitlinear_pack_weights(f32(N, K), workspace=u8(8)),
    lambda: tb.bitlinear_pack_weights_base3(f32(N, K), W_packed3=u8(N, 4)),
    lambda: tb.bitlinear_forward_base3(u8(N, 8), f32(1), *acts(), N=N),
    lambda: tb.bitlinear_base3_to_blt2(u8(N, 16), K, W_packed=u8(N, K // 8)),
    # grouped: one weight of another K, a missing gamma, an output of the wrong shape
    lambda: tb.bitlinear_forward_grouped([u8(N, K // 4), u8(N, K // 8)], [f32(1), f32(1)], *acts()),
    lambda: tb.bitlinear_forward_grouped([u8(N, K // 4), u8(N, K // 4)], [f32(1)], *acts()),
    lambda: tb.bitlinear_forward_grouped([u8(N, K // 4)], [f32(1)], *acts(),
                                         Y=[torch.zeros((M, N - 1), dtype=torch.bfloat16)]),
    lambda: tb.bitlinear_forward_f32_grouped([u8(N, K // 4)] * 5, [f32(1)] * 5, f32(M, K)),
])
def test_wrong_sizes_raise_before_the_library(call):
    # a size, type or count error, found before the device check (these are
    # host tensors, which the device check would refuse too)
    with pytest.raises((ValueError, TypeError)) as e:
        call()
    assert "CUDA" not in str(e.value)


@pytest.mark.parametrize("call", [
    lambda: tb.bitlinear_forward(u8(N, K // 4), f32(1), *acts()),
    lambda: tb.bitlinear_forward_f32(u8(N, K // 4), f32(1), f32(M, K)),
    lambda: tb.bitlinear_forward_f32_noalloc(u8(N, K // 4), f32(1), f32(M, K)),
    lambda: tb.bitlinear_quant_acts(f32(M, K)),
    lambda: tb.bitlinear_pack_weights(f32(N, K)),
    lambda: tb.bitlinear_rmsnorm_quant(f32(M, K), f32(K)),
    lambda: tb.bitlinear_forward_grouped([u8(N, K // 4)] * 2, [f32(1)] * 2, *acts()),
])
def test_host_memory_is_refused(call):
    # right sizes, but host tensors: the library would read them as device
    # pointers
    with pytest.raises(TypeError, match="CUDA"):
        call()


def test_wrong_dtype_and_layout():
    with pytest.raises(TypeError):
        tb.bitlinear_forward(u8(N, K // 4), torch.zeros(1, dtype=torch.float64), *acts())
    with pytest.raises(TypeError):
        tb.bitlinear_quant_acts(torch.zeros((M, K), dtype=torch.float16))
    with pytest.raises(ValueError, match="contiguous"):
        tb.bitlinear_quant_acts(f32(K, M).t())
    with pytest.raises(TypeError):
        tb.bitlinear_forward(u8(N, K // 4).tolist(), f32(1), *acts())
