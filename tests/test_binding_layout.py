"""CPU tests of the binding's layout rules for views into wider rows: which token (prefill)
or batch (decode) stride a view has, and which views are refused before anything reaches
the library.  A stand-in with the tensor attributes the rules read replaces GPU tensors."""
from __future__ import annotations

import pytest

from mamba_ssd_scan_amd import ssd


class View:
    """shape / stride of a strided view, in elements (what torch reports for one)."""

    def __init__(self, shape, stride, is_cuda=True):
        self.shape, self._stride, self.is_cuda = tuple(shape), tuple(stride), is_cuda

    def stride(self):
        return self._stride

    def dim(self):
        return len(self.shape)

    def numel(self):
        n = 1
        for v in self.shape:
            n *= v
        return n


def dense(shape):
    st, acc = [], 1
    for v in reversed(shape):
        st.append(acc)
        acc *= v
    return View(shape, tuple(reversed(st)))


def test_dense_inputs_have_dense_token_strides():
    assert ssd._token_stride(dense((2, 300, 4, 64)), "x") == 256
    assert ssd._token_stride(dense((2, 300, 4)), "dt") == 4
    assert ssd._token_stride(None, "z") == 0


def test_views_into_layer_rows():
    W, L = 1800, 300
    # x = rows[..., :256] of [2, 300, W] rows: token stride W, batches L * W apart
    assert ssd._token_stride(View((2, L, 4, 64), (L * W, W, 64, 1)), "x") == W
    # dt at the end of the rows
    assert ssd._token_stride(View((2, L, 4), (L * W, W, 1)), "dt") == W
    # one sequence: the batch stride does not matter
    assert ssd._token_stride(View((1, L, 4, 64), (12345, W, 64, 1)), "x") == W
    # one token per sequence: the token stride is the batch stride
    assert ssd._token_stride(View((3, 1, 4, 64), (W, 999, 64, 1)), "x") == W
    # an empty input is read as dense whatever torch reports for it
    assert ssd._token_stride(View((2, 0, 4, 64), (0, 0, 0, 0)), "x") == 256


def test_views_the_kernels_cannot_read():
    W, L = 1800, 300
    with pytest.raises(ValueError, match="contiguous"):   # channels of one token not adjacent
        ssd._token_stride(View((2, L, 64, 4), (L * W, W, 1, 64)), "x")
    with pytest.raises(ValueError, match="batches"):      # the first 150 tokens of 300-token rows
        ssd._token_stride(View((2, 150, 4, 64), (L * W, W, 64, 1)), "x")
    with pytest.raises(ValueError, match="GPU"):
        ssd._token_stride(View((2, L, 4, 64), (L * 256, 256, 64, 1), is_cuda=False), "x")


def test_b_and_c_must_share_a_stride():
    W, L = 1800, 300
    x = View((2, L, 4, 64), (L * W, W, 64, 1))
    dt = dense((2, L, 4))
    Bv = View((2, L, 1, 128), (L * W, W, 128, 1))
    with pytest.raises(ValueError, match="same token stride"):
        ssd._seq_strides(x, dt, Bv, dense((2, L, 1, 128)), None)
    strides, is_dense = ssd._seq_strides(x, dt, Bv, View((2, L, 1, 128), (L * W, W, 128, 1)), None)
    assert strides == (W, W, 4, 0) and not is_dense
    strides, is_dense = ssd._seq_strides(dense((2, L, 4, 64)), dt, dense((2, L, 1, 128)), dense((2, L, 1, 128)),
                                         dense((2, L, 4, 64)))
    assert is_dense and strides == (256, 128, 4, 256)


def test_decode_batch_strides():
    W = 3352
    x = View((64, 80, 64), (W, 64, 1))
    assert ssd._batch_stride(x, "x") == W
    assert ssd._batch_stride(dense((64, 80)), "dt") == 80
    assert ssd._batch_stride(View((1, 80, 64), (7, 64, 1)), "x") == 80 * 64  # one entry: dense
    with pytest.raises(ValueError, match="contiguous"):
        ssd._batch_stride(View((64, 64, 80), (W, 1, 64)), "x")
    strides, is_dense = ssd._step_strides(x, View((64, 80), (W, 1)), View((64, 1, 128), (W, 128, 1)),
                                          View((64, 1, 128), (W, 128, 1)), None)
    assert strides == (W, W, W, 0) and not is_dense
