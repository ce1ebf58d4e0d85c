"""The streaming probes (lmx_stream_probe) move the bytes they claim: the copy
and row patterns reproduce their source exactly, out of place and in place,
and the write pattern fills the whole buffer (needs an MI355X)."""
import pytest
import torch

from lm_head_cross_pass_amd import _lib

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _probe(a, b, nbytes, row_bytes, mode):
    st = _lib.lmx_stream_probe(a.data_ptr(), b.data_ptr(), nbytes, row_bytes, mode,
                               torch.cuda.current_stream(DEV).cuda_stream)
    _lib.check("lmx_stream_probe", st)
    torch.cuda.synchronize()


@pytest.mark.parametrize("mode", (_lib.LMX_PROBE_COPY, _lib.LMX_PROBE_COPY_BATCHED,
                                  _lib.LMX_PROBE_ROWS_INTERLEAVED, _lib.LMX_PROBE_ROWS_PHASED))
def test_copies_are_exact(mode):
    # 300 rows of 100 KiB: several rows per workgroup, a ragged last step
    row_bytes = 102400
    nbytes = 300 * row_bytes
    g = torch.Generator(device="cpu").manual_seed(5)
    src = torch.randint(-2**31, 2**31 - 1, (nbytes // 4,), dtype=torch.int32, generator=g).to(DEV)
    dst = torch.zeros_like(src)
    _probe(src, dst, nbytes, row_bytes, mode)
    assert torch.equal(dst, src)
    same = src.clone()
    _probe(same, same, nbytes, row_bytes, mode)
    assert torch.equal(same, src)


def test_write_and_read():
    nbytes = 3 * (1 << 20) + 4096
    dst = torch.zeros(nbytes // 4, dtype=torch.int32, device=DEV)
    _probe(dst, dst, nbytes, 0, _lib.LMX_PROBE_WRITE)
    words = dst.view(-1, 4)
    assert bool((words[:, 2] == 0x3c3c3c3c).all()) and bool((words[:, 3] == 0x3c3c3c3c).all())
    sink = torch.zeros(4096, dtype=torch.int32, device=DEV)
    _probe(dst, sink, nbytes, 0, _lib.LMX_PROBE_READ)
    assert bool((sink == 0).all())
