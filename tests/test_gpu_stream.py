"""GPU checks of the measurement yardstick (libyardstick, beside the product):
the copy and the fill touch exactly the requested bytes, the read leaves its
scratch alone, and bad arguments are refused on the host."""

import ctypes

import pytest
import torch

import yardstick as Y
from gpu_common import DEV

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [0, 16, 4096 + 48, (1 << 20) + 16 * 1023])
def test_copy_fill_read_touch_exactly_the_bytes(nbytes):
    g = torch.Generator(device="cpu").manual_seed(nbytes)
    src = torch.randint(0, 256, (nbytes + 64,), generator=g, dtype=torch.uint8).to(DEV)
    dst = torch.full((nbytes + 64,), 7, dtype=torch.uint8, device=DEV)
    Y.stream(Y.COPY, src, dst, nbytes)
    torch.cuda.synchronize()
    assert torch.equal(dst[:nbytes], src[:nbytes]) and bool((dst[nbytes:] == 7).all())
    Y.stream(Y.FILL, None, dst, nbytes)
    torch.cuda.synchronize()
    assert not dst[:nbytes].any() and bool((dst[nbytes:] == 7).all())
    scratch = torch.full((16,), 5, dtype=torch.uint8, device=DEV)
    Y.stream(Y.READ, src, scratch, nbytes)
    torch.cuda.synchronize()
    assert bool((scratch == 5).all())


def test_bad_arguments_are_refused():
    a = torch.zeros(256, dtype=torch.uint8, device=DEV)
    b = torch.zeros(256, dtype=torch.uint8, device=DEV)
    L = Y.lib()
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    p = lambda t, off=0: ctypes.c_void_p(t.data_ptr() + off)  # noqa: E731
    assert L.ys_stream(s, Y.COPY, p(a), p(b), 24) == -1          # not a multiple of 16
    assert L.ys_stream(s, Y.COPY, p(a, 8), p(b), 32) == -1       # misaligned source
    assert L.ys_stream(s, Y.FILL, None, p(b, 4), 32) == -1       # misaligned destination
    assert L.ys_stream(s, 7, p(a), p(b), 32) == -1                      # unknown mode
    assert L.ys_stream(s, Y.READ, None, p(b), 32) == -1          # read without a source
    assert L.ys_stream(s, Y.COPY, p(a), p(b), -16) == -1
    with pytest.raises(ValueError):
        Y.stream(Y.COPY, a, b, 512)                              # beyond the tensors
