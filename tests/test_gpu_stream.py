"""GPU checks of the measurement yardstick (grpo_stream_probe): the copy and
the fill touch exactly the requested bytes, the read leaves its scratch
alone, and bad arguments are refused on the host."""

import pytest
import torch

from gpu_common import DEV
from grpo_token_level_amd import _capi as C
from grpo_token_level_amd import ops

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [0, 16, 4096 + 48, (1 << 20) + 16 * 1023])
def test_copy_fill_read_touch_exactly_the_bytes(nbytes):
    g = torch.Generator(device="cpu").manual_seed(nbytes)
    src = torch.randint(0, 256, (nbytes + 64,), generator=g, dtype=torch.uint8).to(DEV)
    dst = torch.full((nbytes + 64,), 7, dtype=torch.uint8, device=DEV)
    ops.stream_probe(C.STREAM_COPY, src, dst, nbytes)
    torch.cuda.synchronize()
    assert torch.equal(dst[:nbytes], src[:nbytes]) and bool((dst[nbytes:] == 7).all())
    ops.stream_probe(C.STREAM_FILL, None, dst, nbytes)
    torch.cuda.synchronize()
    assert not dst[:nbytes].any() and bool((dst[nbytes:] == 7).all())
    scratch = torch.full((16,), 5, dtype=torch.uint8, device=DEV)
    ops.stream_probe(C.STREAM_READ, src, scratch, nbytes)
    torch.cuda.synchronize()
    assert bool((scratch == 5).all())


def test_bad_arguments_are_refused():
    a = torch.zeros(256, dtype=torch.uint8, device=DEV)
    b = torch.zeros(256, dtype=torch.uint8, device=DEV)
    L = C.lib()
    s = ops._stream()
    p = lambda t, off=0: C.ctypes.c_void_p(t.data_ptr() + off)  # noqa: E731
    assert L.grpo_stream_probe(s, C.STREAM_COPY, p(a), p(b), 24) == -1          # not a multiple of 16
    assert L.grpo_stream_probe(s, C.STREAM_COPY, p(a, 8), p(b), 32) == -1       # misaligned source
    assert L.grpo_stream_probe(s, C.STREAM_FILL, None, p(b, 4), 32) == -1       # misaligned destination
    assert L.grpo_stream_probe(s, 7, p(a), p(b), 32) == -1                      # unknown mode
    assert L.grpo_stream_probe(s, C.STREAM_READ, None, p(b), 32) == -1          # read without a source
    assert L.grpo_stream_probe(s, C.STREAM_COPY, p(a), p(b), -16) == -1
    with pytest.raises(ValueError):
        ops.stream_probe(C.STREAM_COPY, a, b, 512)                              # beyond the tensors
