"""The masked-field dot product of the single-token kernels, emulated on the host.

`dot_word_fields` (ternary_bitlinear_amd/csrc/common.hpp) multiplies one
packed 16-code word with its 16 activations without expanding the codes to
bytes.  Field f of the word's bytes (bits 2f and 2f + 1: the code of
k = 4f + b in byte b) is masked in place, which gives bytes c 4^f for
f = 0, 1, 2; field 3 is shifted down one bit first, which gives c 32.  Each
field is multiplied byte by byte, as signed bytes (v_dot4_i32_i8), with the
activations of the same k into an accumulator of its own, and
`fields_total` divides each accumulator back by its scale.

These tests replay those integer steps on words the oracle packs.  They
check three things:
  - every field sum is an exact multiple of its scale;
  - the total equals the oracle's exact sum_k c_k x~_k;
  - no accumulator leaves int32 for K below 2^18 with the largest operands.
"""
import numpy as np
import pytest

from oracle import bitlinear_oracle as O


def _sdot4_fields(P, Xq):
    """P: packed rows [N][K/4] (BLT2-v1 bytes); Xq: int8 activations [K].
    Returns the four per-field accumulators [N][4] as the kernels form them
    (int64 here, so that an overflow of int32 can be checked)."""
    N = P.shape[0]
    K = Xq.shape[0]
    w = np.ascontiguousarray(P).view("<u4").reshape(N, K // 16).astype(np.uint64)
    x = Xq.astype(np.int64).reshape(K // 16, 4, 4)   # word, dword d (k = 4d + b), byte b
    masks = [(w & (0x03030303 << (2 * f))) for f in range(3)]
    masks.append((w >> 1) & 0x60606060)
    acc = np.zeros((N, 4), dtype=np.int64)
    for f in range(4):
        b = masks[f].astype("<u4").view(np.uint8).reshape(N, K // 16, 4).astype(np.int64)
        b = np.where(b > 127, b - 256, b)              # the instruction's signed bytes
        assert (b >= 0).all() and (b <= 64).all()      # every masked byte is a valid int8
        acc[:, f] = (b * x[None, :, f, :]).sum(axis=(1, 2))
    return acc


def _fields_total(acc):
    scale = np.array([1, 4, 16, 32], dtype=np.int64)
    assert (acc % scale == 0).all(), "a field sum is not a multiple of its scale"
    return acc[:, 0] + (acc[:, 1] >> 2) + (acc[:, 2] >> 4) + (acc[:, 3] >> 5)


@pytest.mark.parametrize("seed,K", [(0, 64), (1, 4096), (2, 8192 + 64), (3, 28672)])
def test_field_dot_equals_exact_product(seed, K):
    rng = np.random.default_rng(seed)
    N = 6
    Wt = rng.integers(-1, 2, size=(N, K)).astype(np.int8)
    Xq = rng.integers(-127, 128, size=K).astype(np.int8)
    P = O.pack_codes(Wt)
    got = _fields_total(_sdot4_fields(P, Xq))
    # codes are c = W~ + 1: sum_k c_k x_k = sum_k W~_k x_k + sum_k x_k
    want = O.integer_matmul(Wt, Xq[None, :])[0] + int(Xq.astype(np.int64).sum())
    assert np.array_equal(got, want)


def test_field_dot_sees_every_field_and_position():
    # One nonzero code at a time: each (k, code) pair must come back with its
    # own activation, so a wrong mask, shift or activation dword fails here.
    K = 16
    Xq = (np.arange(K, dtype=np.int64) * 7 - 50).astype(np.int8)
    for k in range(K):
        for wv in (0, 1):   # codes 1 and 2
            Wt = -np.ones((1, K), dtype=np.int8)   # code 0 everywhere
            Wt[0, k] = wv
            got = _fields_total(_sdot4_fields(O.pack_codes(Wt), Xq))[0]
            assert got == (wv + 1) * int(Xq[k]), (k, wv)


def test_field_accumulators_stay_in_int32_below_two_to_the_18():
    K = (1 << 18) - 16
    for xv in (127, -127):
        Wt = np.ones((1, K), dtype=np.int8)        # code 2 on every weight
        Xq = np.full(K, xv, dtype=np.int8)
        acc = _sdot4_fields(O.pack_codes(Wt), Xq)
        assert np.abs(acc).max() < 2 ** 31
        assert _fields_total(acc)[0] == 2 * xv * K
