"""ce_fwd_bwd_noalloc (the workspace in the library's fixed scratch array)
against ce_fwd_bwd with a caller workspace, through the C ABI (needs an
MI355X).

Two calls in a row on one GPU, the second with fewer rows, so the second
reads the scratch after the first has left its contents there; each result
must equal the workspace entry point's bit for bit (the same kernels run on
the same inputs), which is tighter than the tolerances against the oracle.

Because the entry point allocates nothing, a caller can capture it in a HIP
graph: captured once on static buffers, the graph is replayed on new logits
and targets written into those buffers, with eager work and synchronizations
between the replays, and every replay must equal ce_fwd_bwd on the same
inputs bit for bit.
"""
import pytest
import torch

import workloads
from lm_head_cross_pass_amd import _lib

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _outs():
    return (torch.empty((), dtype=torch.float32, device=DEV),
            torch.empty((), dtype=torch.int64, device=DEV),
            torch.empty((), dtype=torch.int32, device=DEV))


@pytest.mark.parametrize("dtype", (torch.bfloat16, torch.float32))
def test_noalloc_matches_the_workspace_entry_point(dtype):
    code = {torch.bfloat16: _lib.LMX_BF16, torch.float32: _lib.LMX_F32}[dtype]
    stream = torch.cuda.current_stream(DEV).cuda_stream
    # (rows, vocabulary, reduction, z, in place): the second call is smaller
    for B, V, red, z, in_place in ((4096, 50257, _lib.LMX_MEAN, 1e-4, False),
                                   (1000, 32000, _lib.LMX_SUM, 0.0, True)):
        logits, target = workloads.small_ce(B, V, dtype=dtype, sigma=3.0, n_ignored=B // 20,
                                            seed=B + V, boost=8.0)
        t = target.to(DEV)
        x_ref = logits.to(DEV)
        g_ref = x_ref if in_place else torch.empty_like(x_ref)
        o_ref = _outs()
        ws = torch.empty(_lib.ce_workspace_bytes(B, V, code), dtype=torch.uint8, device=DEV)
        _lib.check("ce_fwd_bwd", _lib.ce_fwd_bwd(
            x_ref.data_ptr(), g_ref.data_ptr(), t.data_ptr(), B, V, code, -100, red, z,
            o_ref[0].data_ptr(), o_ref[1].data_ptr(), o_ref[2].data_ptr(), ws.data_ptr(),
            ws.numel(), stream))
        x = logits.to(DEV)
        g = x if in_place else torch.empty_like(x)
        o = _outs()
        _lib.check("ce_fwd_bwd_noalloc", _lib.ce_fwd_bwd_noalloc(
            x.data_ptr(), g.data_ptr(), t.data_ptr(), B, V, code, -100, red, z,
            o[0].data_ptr(), o[1].data_ptr(), o[2].data_ptr(), stream))
        torch.cuda.synchronize()
        assert torch.equal(g, g_ref)
        assert torch.equal(o[0], o_ref[0]) and int(o[1]) == int(o_ref[1]) == B - B // 20
        assert int(o[2]) == int(o_ref[2]) == 0


def test_noalloc_rejects_more_rows_than_its_scratch():
    stream = torch.cuda.current_stream(DEV).cuda_stream
    B, V = (1 << 20) + 1, 8
    x = torch.zeros((B, V), dtype=torch.bfloat16, device=DEV)
    t = torch.zeros(B, dtype=torch.int64, device=DEV)
    o = _outs()
    o[0].fill_(7.0)
    st = _lib.ce_fwd_bwd_noalloc(x.data_ptr(), x.data_ptr(), t.data_ptr(), B, V, _lib.LMX_BF16,
                                 -100, _lib.LMX_SUM, 0.0, o[0].data_ptr(), o[1].data_ptr(),
                                 o[2].data_ptr(), stream)
    torch.cuda.synchronize()
    assert st == _lib.LMX_ERR_SCRATCH
    assert float(o[0]) == 7.0 and bool((x == 0).all())     # nothing was enqueued
    # exactly the maximum is accepted
    B = 1 << 20
    st = _lib.ce_fwd_bwd_noalloc(x.data_ptr(), x.data_ptr(), t.data_ptr(), B, V, _lib.LMX_BF16,
                                 -100, _lib.LMX_SUM, 0.0, o[0].data_ptr(), o[1].data_ptr(),
                                 o[2].data_ptr(), stream)
    torch.cuda.synchronize()
    assert st == _lib.LMX_OK and int(o[1]) == B


@pytest.mark.parametrize("in_place", (False, True))
def test_noalloc_replayed_from_a_graph(in_place):
    B, V, code, red, z = 1000, 50257, _lib.LMX_BF16, _lib.LMX_MEAN, 1e-4
    x = torch.empty((B, V), dtype=torch.bfloat16, device=DEV)
    t = torch.empty(B, dtype=torch.int64, device=DEV)
    g = x if in_place else torch.empty_like(x)
    o = _outs()

    def call(stream):
        return _lib.ce_fwd_bwd_noalloc(x.data_ptr(), g.data_ptr(), t.data_ptr(), B, V, code, -100,
                                       red, z, o[0].data_ptr(), o[1].data_ptr(),
                                       o[2].data_ptr(), stream)

    inputs = [workloads.small_ce(B, V, dtype=torch.bfloat16, sigma=3.0, n_ignored=40 + 10 * i,
                                 seed=100 + i, boost=8.0) for i in range(3)]
    # an eager call first: the library looks up its scratch array's address on
    # the device's first call, outside the capture
    x.copy_(inputs[0][0].to(DEV))
    t.copy_(inputs[0][1].to(DEV))
    side = torch.cuda.Stream(DEV)
    side.wait_stream(torch.cuda.current_stream(DEV))
    with torch.cuda.stream(side):
        _lib.check("ce_fwd_bwd_noalloc", call(side.cuda_stream))
    torch.cuda.current_stream(DEV).wait_stream(side)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        _lib.check("ce_fwd_bwd_noalloc", call(torch.cuda.current_stream(DEV).cuda_stream))
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream(DEV).cuda_stream
    for logits, target in inputs + inputs[:1]:
        # eager work of the program between replays: new inputs into the
        # captured buffers, the reference call on copies of them
        x.copy_(logits.to(DEV))
        t.copy_(target.to(DEV))
        x_ref = x.clone()
        g_ref = x_ref if in_place else torch.empty_like(x_ref)
        o_ref = _outs()
        ws = torch.empty(_lib.ce_workspace_bytes(B, V, code), dtype=torch.uint8, device=DEV)
        _lib.check("ce_fwd_bwd", _lib.ce_fwd_bwd(
            x_ref.data_ptr(), g_ref.data_ptr(), t.data_ptr(), B, V, code, -100, red, z,
            o_ref[0].data_ptr(), o_ref[1].data_ptr(), o_ref[2].data_ptr(), ws.data_ptr(),
            ws.numel(), stream))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(g, g_ref)
        assert torch.equal(o[0], o_ref[0])
        assert int(o[1]) == int(o_ref[1]) == int((target != -100).sum())
        assert int(o[2]) == int(o_ref[2]) == 0
