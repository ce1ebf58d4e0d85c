"""The C ABI on the host (no GPU): the library loads, exports every function
``include/lmx.h`` declares, sizes workspaces, and rejects bad arguments with
the documented status before touching the device.

The argument-check calls pass made-up addresses: the library only does
arithmetic on them on the host and returns an error status before any HIP
call, so nothing is ever dereferenced.
"""
import os

import pytest

from lm_head_cross_pass_amd import _lib

F32, BF16 = _lib.LMX_F32, _lib.LMX_BF16
MEAN, SUM = _lib.LMX_MEAN, _lib.LMX_SUM
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
A = 1 << 40          # a fake, 256-byte aligned device address
WS = 1 << 20


@pytest.fixture(scope="module", autouse=True)
def built_library():
    if not os.path.exists(_lib.LIB_PATH):
        from lm_head_cross_pass_amd import build
        build.build()
    _lib.load()


def test_every_declared_function_is_exported():
    names = _lib.header_functions()
    assert set(names) == {"ce_fwd_bwd", "ce_workspace_bytes", "ce_fwd_bwd_noalloc", "linear_ce",
                          "linear_ce_workspace_bytes", "linear_ce_chunk_rows",
                          "lmx_status_string", "lmx_copy", "lmx_stream_probe", "lmx_scale",
                          "selective_log_softmax",
                          "ce_loss_rows", "ce_loss_rows_vjp", "linear_loss_logits",
                          "linear_loss_grads", "linear_loss_workspace_bytes",
                          "linear_loss_logits_workspace_bytes"}
    lib = _lib.load()
    for n in names:
        assert hasattr(lib, n), n


def test_library_binds_every_symbol_eagerly():
    # every kernel's host stub must be defined: a lazily bound library would
    # only fail at the first launch of a kernel whose stub is missing
    import subprocess
    import sys
    code = ("import ctypes, os, sys; ctypes.CDLL(sys.argv[1], mode=os.RTLD_NOW); print('ok')")
    r = subprocess.run([sys.executable, "-c", code, _lib.LIB_PATH], capture_output=True,
                       text=True)
    assert r.returncode == 0 and "ok" in r.stdout, r.stderr


def test_only_the_abi_is_exported():
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True,
                         text=True)
    if out.returncode != 0:
        pytest.skip("nm not available")
    exported = {ln.split()[-1] for ln in out.stdout.splitlines() if " T " in ln}
    assert exported == set(_lib.header_functions())


def test_status_strings():
    for code in _lib.STATUS:
        assert _lib.status_string(code)
    assert _lib.status_string(12345) == "unknown status"


def test_workspace_sizes():
    assert _lib.ce_workspace_bytes(16384, 128256, BF16) >= 16384 * 4
    assert _lib.ce_workspace_bytes(0, 10, F32) > 0
    assert _lib.ce_workspace_bytes(-1, 10, F32) == 0
    assert _lib.ce_workspace_bytes(4, 0, F32) == 0
    assert _lib.ce_workspace_bytes(4, 10, 7) == 0
    assert _lib.ce_workspace_bytes(4, 1 << 30, BF16) == 0
    assert _lib.ce_workspace_bytes(4, (1 << 29) - 8, F32) == 0
    assert _lib.ce_workspace_bytes(4, (1 << 29) - 8, BF16) > 0
    assert _lib.linear_ce_workspace_bytes(8192, 768, 50257, BF16, 1024, 0, 0) > 0
    assert _lib.linear_ce_workspace_bytes(8192, 768, 50257, F32, 1024, 0, 0) == 0
    assert _lib.linear_ce_workspace_bytes(8192, 768, 50257, BF16, -1, 0, 0) == 0
    assert _lib.linear_ce_workspace_bytes(8192, 768, 50257, BF16, 1024, 5, 0) == 0
    assert _lib.linear_ce_workspace_bytes(8192, 768, 50257, BF16, 1024, 0, -1) == 0
    assert _lib.linear_ce_workspace_bytes(8192, 768, 4194048 + 1, BF16, 1024, 0, 0) == 0
    assert _lib.linear_ce_workspace_bytes(8192, 2097088 + 8, 1000, BF16, 1024, 0, 0) == 0


def test_grad_weight_group_budget_bounds_the_workspace():
    # inputs [BT, 4096] x weight [128256, 4096], chunks of 2048: G^T of one
    # chunk is 128256 x 2048 bf16 (525 MB; 128256 is a multiple of 256)
    D, V, C = 4096, 128256, 2048
    gt_chunk = 128256 * 2048 * 2
    acc32 = V * D * 4

    def ws(BT, accum, budget):
        return _lib.linear_ce_workspace_bytes(BT, D, V, BF16, C, accum, budget)
    # the default budget (2 GiB: four chunks per product) does not grow with BT
    # beyond the per-row loss terms
    base = ws(16384, 0, 0)
    assert ws(65536, 0, 0) - base <= (65536 - 16384) * 4 + 256
    # the default is the 2 GiB budget given explicitly
    assert ws(16384, 0, 1 << 31) == base
    # a chunk's packed X^T columns, and its packed X_c (the group's chunks are
    # packed together, one copy per chunk of the group)
    xt_chunk = D * 2048 * 2
    # fp32 mode: one product over all 8 chunks keeps no fp32 accumulator but
    # holds 4 more chunks of G^T, X^T and packed X_c
    one = ws(16384, 0, 8 * gt_chunk)
    assert 4 * gt_chunk - acc32 < one - base <= 4 * (gt_chunk + 2 * xt_chunk) - acc32 + 4096
    # a budget of one chunk: 3 chunks less of G^T, X^T and packed X_c than the default
    small = ws(16384, 0, gt_chunk)
    assert 3 * gt_chunk <= base - small <= 3 * (gt_chunk + 2 * xt_chunk) + (64 << 20)
    # weight-dtype mode keeps no fp32 accumulator
    assert ws(16384, 1, 0) <= base - acc32


def test_chunk_rows():
    assert _lib.linear_ce_chunk_rows(8192, 50257, 1024) == 1024
    assert _lib.linear_ce_chunk_rows(100, 50257, 1024) == 100
    c = _lib.linear_ce_chunk_rows(16384, 128256, 0)
    assert 1 <= c <= 16384


def _ce(**kw):
    args = dict(logits=A, grad=A + (1 << 34), target=A + (2 << 34), B=8, V=1000, dtype=F32,
                ignore=-100, red=MEAN, z=0.0, loss=A + (3 << 34), n=None, bad=None,
                ws=A + (4 << 34), wsb=WS, stream=None)
    args.update(kw)
    return _lib.ce_fwd_bwd(args["logits"], args["grad"], args["target"], args["B"], args["V"],
                           args["dtype"], args["ignore"], args["red"], args["z"], args["loss"],
                           args["n"], args["bad"], args["ws"], args["wsb"], args["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(loss=None), _lib.LMX_ERR_NULL),
    (dict(ws=None), _lib.LMX_ERR_NULL),
    (dict(logits=None), _lib.LMX_ERR_NULL),
    (dict(target=None), _lib.LMX_ERR_NULL),
    (dict(B=-1), _lib.LMX_ERR_SIZE),
    (dict(V=0), _lib.LMX_ERR_SIZE),
    (dict(V=1 << 30), _lib.LMX_ERR_SIZE),
    (dict(V=(1 << 29) - 8), _lib.LMX_ERR_SIZE),          # fp32 row past 2^31 - 64 bytes
    (dict(B=1 << 62), _lib.LMX_ERR_SIZE),
    (dict(dtype=3), _lib.LMX_ERR_ENUM),
    (dict(red=2), _lib.LMX_ERR_ENUM),
    (dict(logits=A + 2), _lib.LMX_ERR_ALIGN),           # fp32 needs 4-byte alignment
    (dict(target=A + 4), _lib.LMX_ERR_ALIGN),
    (dict(grad=A + (1 << 34) + 4), _lib.LMX_ERR_ALIGN), # differs from logits modulo 16
    (dict(ws=A + 64), _lib.LMX_ERR_WORKSPACE),
    (dict(wsb=16), _lib.LMX_ERR_WORKSPACE),
    (dict(grad=A + 4000 * 4 + 16 * 0), _lib.LMX_ERR_ALIAS),  # overlaps logits, not equal
])
def test_ce_argument_errors(kw, status):
    assert _ce(**kw) == status


def _lin(**kw):
    args = dict(x=A, w=A + (1 << 34), t=A + (2 << 34), BT=64, D=64, V=1000, dtype=BF16,
                ignore=-100, red=MEAN, z=0.0, chunk=16, acc=0, gb=0, loss=A + (3 << 34),
                gx=A + (5 << 34), gw=A + (6 << 34), n=None, bad=None, ws=A + (4 << 34),
                wsb=1 << 40, stream=None)
    args.update(kw)
    return _lib.linear_ce(args["x"], args["w"], args["t"], args["BT"], args["D"], args["V"],
                          args["dtype"], args["ignore"], args["red"], args["z"], args["chunk"],
                          args["acc"], args["gb"], args["loss"], args["gx"], args["gw"], args["n"],
                          args["bad"], args["ws"], args["wsb"], args["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(w=None), _lib.LMX_ERR_NULL),
    (dict(gw=None), _lib.LMX_ERR_NULL),
    (dict(x=None), _lib.LMX_ERR_NULL),
    (dict(BT=-1), _lib.LMX_ERR_SIZE),
    (dict(D=0), _lib.LMX_ERR_SIZE),
    (dict(V=0), _lib.LMX_ERR_SIZE),
    (dict(V=4194048 + 1), _lib.LMX_ERR_SIZE),           # 32-bit offsets of 256-row panels
    (dict(D=2097088 + 8), _lib.LMX_ERR_SIZE),
    (dict(BT=5 << 20, chunk=4194240 + 64), _lib.LMX_ERR_SIZE),  # chunk > 4194240 rows
    (dict(chunk=-1), _lib.LMX_ERR_CHUNK),
    (dict(gb=-1), _lib.LMX_ERR_SIZE),
    (dict(dtype=F32), _lib.LMX_ERR_UNSUPPORTED),
    (dict(dtype=3), _lib.LMX_ERR_ENUM),
    (dict(red=5), _lib.LMX_ERR_ENUM),
    (dict(acc=2), _lib.LMX_ERR_ENUM),
    (dict(D=60), _lib.LMX_ERR_ALIGN),
    (dict(x=A + 8), _lib.LMX_ERR_ALIGN),
    (dict(gw=A + (6 << 34) + 2), _lib.LMX_ERR_ALIGN),
    (dict(ws=A + 128), _lib.LMX_ERR_WORKSPACE),
    (dict(wsb=256), _lib.LMX_ERR_WORKSPACE),
    (dict(gx=A + 64), _lib.LMX_ERR_ALIAS),               # overlaps inputs
    (dict(gw=A + (1 << 34) + 1024), _lib.LMX_ERR_ALIAS), # overlaps weight
])
def test_linear_ce_argument_errors(kw, status):
    assert _lin(**kw) == status


def test_scale_argument_errors():
    S = A + (5 << 34)
    assert _lib.lmx_scale(A, A, 8, 3, S, None) == _lib.LMX_ERR_ENUM
    assert _lib.lmx_scale(A, A, -1, F32, S, None) == _lib.LMX_ERR_SIZE
    assert _lib.lmx_scale(A, A, 0, F32, None, None) == _lib.LMX_OK      # nothing to do
    assert _lib.lmx_scale(None, A, 8, F32, S, None) == _lib.LMX_ERR_NULL
    assert _lib.lmx_scale(A, A, 8, F32, None, None) == _lib.LMX_ERR_NULL
    assert _lib.lmx_scale(A + 2, A + (1 << 34), 8, F32, S, None) == _lib.LMX_ERR_ALIGN
    assert _lib.lmx_scale(A + 1, A + (1 << 34), 8, _lib.LMX_BF16, S, None) == _lib.LMX_ERR_ALIGN
    assert _lib.lmx_scale(A, A, 8, F32, S + 2, None) == _lib.LMX_ERR_ALIGN
    assert _lib.lmx_scale(A, A + 16, 8, F32, S, None) == _lib.LMX_ERR_ALIAS   # partial overlap
    assert _lib.lmx_scale(A, A + (1 << 34), 8, F32, A + (1 << 34) + 4, None) == _lib.LMX_ERR_ALIAS


def test_copy_argument_errors():
    assert _lib.lmx_copy(None, A, 16, None) == _lib.LMX_ERR_NULL
    assert _lib.lmx_copy(A + 8, A + (1 << 34), 16, None) == _lib.LMX_ERR_ALIGN
    assert _lib.lmx_copy(A, A + 16, 64, None) == _lib.LMX_ERR_ALIAS
    assert _lib.lmx_copy(A, A, 0, None) == _lib.LMX_OK
    probe = _lib.lmx_stream_probe
    assert probe(A, A + (1 << 34), 1 << 20, 0, 9, None) == _lib.LMX_ERR_ENUM
    assert probe(None, A, 1 << 20, 0, _lib.LMX_PROBE_COPY, None) == _lib.LMX_ERR_NULL
    assert probe(A, A + (1 << 34), (1 << 20) + 8, 0, _lib.LMX_PROBE_COPY, None) == _lib.LMX_ERR_SIZE
    assert probe(A + 8, A + (1 << 34), 1 << 20, 0, _lib.LMX_PROBE_COPY, None) == _lib.LMX_ERR_ALIGN
    assert probe(A, A + 64, 1 << 20, 0, _lib.LMX_PROBE_COPY, None) == _lib.LMX_ERR_ALIAS
    assert probe(A, A + 64, 1 << 20, 0, _lib.LMX_PROBE_READ, None) == _lib.LMX_ERR_ALIAS
    assert probe(A, A, 1 << 20, 1000, _lib.LMX_PROBE_ROWS_PHASED, None) == _lib.LMX_ERR_SIZE
    assert probe(A, A, 1 << 20, 1 << 19, _lib.LMX_PROBE_ROWS_PHASED, None) == _lib.LMX_ERR_SIZE
    assert probe(A, A, 0, 0, _lib.LMX_PROBE_COPY, None) == _lib.LMX_OK


def _rows(fn, **kw):
    args = dict(logits=A, index=A + (2 << 34), B=8, V=1000, dtype=F32, ignore=-100,
                out=A + (3 << 34), n=None, bad=None, ws=A + (4 << 34), wsb=WS, stream=None)
    args.update(kw)
    if fn == "selective_log_softmax":
        return _lib.selective_log_softmax(args["logits"], args["index"], args["B"], args["V"],
                                          args["dtype"], args["out"], args["bad"], args["ws"],
                                          args["wsb"], args["stream"])
    return _lib.ce_loss_rows(args["logits"], args["index"], args["B"], args["V"], args["dtype"],
                             args["ignore"], args["out"], args["n"], args["bad"], args["ws"],
                             args["wsb"], args["stream"])


@pytest.mark.parametrize("fn", ("selective_log_softmax", "ce_loss_rows"))
@pytest.mark.parametrize("kw,status", [
    (dict(ws=None), _lib.LMX_ERR_NULL),
    (dict(out=None), _lib.LMX_ERR_NULL),
    (dict(logits=None), _lib.LMX_ERR_NULL),
    (dict(B=-1), _lib.LMX_ERR_SIZE),
    (dict(V=0), _lib.LMX_ERR_SIZE),
    (dict(V=1 << 30), _lib.LMX_ERR_SIZE),
    (dict(dtype=3), _lib.LMX_ERR_ENUM),
    (dict(logits=A + 2), _lib.LMX_ERR_ALIGN),
    (dict(index=A + (2 << 34) + 4), _lib.LMX_ERR_ALIGN),
    (dict(out=A + (3 << 34) + 2), _lib.LMX_ERR_ALIGN),
    (dict(ws=A + 64), _lib.LMX_ERR_WORKSPACE),
    (dict(wsb=16), _lib.LMX_ERR_WORKSPACE),
    (dict(out=A + 64), _lib.LMX_ERR_ALIAS),                 # inside the logits
    (dict(B=0, logits=None, index=None, out=None), _lib.LMX_OK),
])
def test_row_forward_argument_errors(fn, kw, status):
    assert _rows(fn, **kw) == status


def _vjp(**kw):
    args = dict(logits=A, target=A + (2 << 34), loss=A + (3 << 34), g=A + (5 << 34),
                grad=A + (1 << 34), B=8, V=1000, dtype=F32, ignore=-100, stream=None)
    args.update(kw)
    return _lib.ce_loss_rows_vjp(args["logits"], args["target"], args["loss"], args["g"],
                                 args["grad"], args["B"], args["V"], args["dtype"],
                                 args["ignore"], args["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(g=None), _lib.LMX_ERR_NULL),
    (dict(loss=None), _lib.LMX_ERR_NULL),
    (dict(grad=None), _lib.LMX_ERR_NULL),
    (dict(B=-1), _lib.LMX_ERR_SIZE),
    (dict(V=0), _lib.LMX_ERR_SIZE),
    (dict(dtype=5), _lib.LMX_ERR_ENUM),
    (dict(loss=A + (3 << 34) + 2), _lib.LMX_ERR_ALIGN),
    (dict(grad=A + (1 << 34) + 4), _lib.LMX_ERR_ALIGN),     # differs from logits modulo 16
    (dict(grad=A + 4000 * 4), _lib.LMX_ERR_ALIAS),          # overlaps logits, not equal
    (dict(g=A + (1 << 34) + 64), _lib.LMX_ERR_ALIAS),       # g inside the gradient
    (dict(B=0, logits=None, target=None, loss=None, g=None, grad=None), _lib.LMX_OK),
])
def test_vjp_argument_errors(kw, status):
    assert _vjp(**kw) == status


def _grads(**kw):
    args = dict(x=A, w=A + (1 << 34), g=A + (2 << 34), ldg=1000, rows=16, BT=64, D=64, V=1000,
                dtype=BF16, chunk=16, acc=0, idx=0, gx=A + (5 << 34), gw=A + (6 << 34),
                ws=A + (4 << 34), wsb=1 << 40, stream=None)
    args.update(kw)
    return _lib.linear_loss_grads(args["x"], args["w"], args["g"], args["ldg"], args["rows"],
                                  args["BT"], args["D"], args["V"], args["dtype"], args["chunk"],
                                  args["acc"], args["idx"], args["gx"], args["gw"], args["ws"],
                                  args["wsb"], args["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(gw=None), _lib.LMX_ERR_NULL),
    (dict(g=None), _lib.LMX_ERR_NULL),
    (dict(BT=0), _lib.LMX_ERR_SIZE),
    (dict(ldg=999), _lib.LMX_ERR_SIZE),
    (dict(ldg=4194048 + 8), _lib.LMX_ERR_SIZE),           # stride beyond the 32-bit panel offsets
    (dict(rows=15), _lib.LMX_ERR_SIZE),                   # not the chunk's size
    (dict(idx=4), _lib.LMX_ERR_CHUNK),                    # 64 / 16 = 4 chunks
    (dict(idx=-1), _lib.LMX_ERR_CHUNK),
    (dict(chunk=-2), _lib.LMX_ERR_CHUNK),
    (dict(dtype=F32), _lib.LMX_ERR_UNSUPPORTED),
    (dict(acc=3), _lib.LMX_ERR_ENUM),
    (dict(V=1001, ldg=1001), _lib.LMX_ERR_ALIGN),         # gradient rows must be 16-byte rows
    (dict(g=A + (2 << 34) + 8), _lib.LMX_ERR_ALIGN),
    (dict(ws=A + (4 << 34) + 128), _lib.LMX_ERR_WORKSPACE),
    (dict(wsb=1024), _lib.LMX_ERR_WORKSPACE),
    (dict(gx=A + (2 << 34) + 64), _lib.LMX_ERR_ALIAS),   # inside the logits gradient
])
def test_linear_loss_grads_argument_errors(kw, status):
    assert _grads(**kw) == status


def test_noalloc_argument_errors():
    # host checks return before any HIP call: more rows than the fixed scratch
    # holds, and the argument errors of ce_fwd_bwd
    f = _lib.ce_fwd_bwd_noalloc
    loss, n, bad = A + (3 << 34), A + (3 << 34) + 64, A + (3 << 34) + 128
    big = (1 << 20) + 1
    assert f(A, A, A + (2 << 34), big, 1000, BF16, -100, 0, 0.0, loss, n, bad,
             None) == _lib.LMX_ERR_SCRATCH
    assert f(A, A, A + (2 << 34), 16, 1000, BF16, -100, 0, 0.0, None, n, bad,
             None) == _lib.LMX_ERR_NULL
    assert f(A, A, A + (2 << 34), 16, 1000, 9, -100, 0, 0.0, loss, n, bad,
             None) == _lib.LMX_ERR_ENUM
    assert f(A, A + 64, A + (2 << 34), 16, 1000, BF16, -100, 0, 0.0, loss, n, bad,
             None) == _lib.LMX_ERR_ALIAS
    assert _lib.status_string(_lib.LMX_ERR_SCRATCH).startswith("more rows")


def test_linear_loss_logits_argument_errors():
    f = _lib.linear_loss_logits
    O = A + (3 << 34)   # logits
    assert f(A, None, 16, 64, 1000, BF16, O, 1000, None, 0, None) == _lib.LMX_ERR_NULL
    assert f(A, A + (1 << 34), 16, 64, 1000, BF16, O, 999, None, 0, None) == _lib.LMX_ERR_SIZE
    # an output stride beyond what 32-bit offsets over 256 rows reach
    assert f(A, A + (1 << 34), 16, 64, 1000, BF16, O, 4194048 + 8, None, 0,
             None) == _lib.LMX_ERR_SIZE
    assert f(A, A + (1 << 34), 16, 64, 1000, 7, O, 1000, None, 0, None) == _lib.LMX_ERR_ENUM
    assert f(A, A + (1 << 34), 16, 60, 1000, BF16, O, 1000, None, 0, None) == _lib.LMX_ERR_ALIGN
    assert f(A, A + (1 << 34), 16, 64, 1000, BF16, A + 64, 1000, None, 0,
             None) == _lib.LMX_ERR_ALIAS
    assert f(None, A, 0, 64, 1000, BF16, None, 1000, None, 0, None) == _lib.LMX_OK
    # the workspace holds the packed chunk inputs: required, aligned, big enough
    need = _lib.linear_loss_logits_workspace_bytes(16, 64, BF16)
    ws = A + (5 << 34)
    assert f(A, A + (1 << 34), 16, 64, 1000, BF16, O, 1000, None, need,
             None) == _lib.LMX_ERR_NULL
    assert f(A, A + (1 << 34), 16, 64, 1000, BF16, O, 1000, ws + 64, need,
             None) == _lib.LMX_ERR_WORKSPACE
    assert f(A, A + (1 << 34), 16, 64, 1000, BF16, O, 1000, ws, need - 1,
             None) == _lib.LMX_ERR_WORKSPACE
    assert _lib.linear_loss_workspace_bytes(64, 64, 1000, BF16, 16, 0) > 0
    assert _lib.linear_loss_workspace_bytes(64, 64, 1000, F32, 16, 0) == 0


def test_linear_loss_logits_workspace_bytes():
    # 32-row blocks of 64-wide K steps, 4 KiB each (the packed chunk inputs)
    assert _lib.linear_loss_logits_workspace_bytes(2048, 4096, BF16) == 64 * 64 * 4096
    assert _lib.linear_loss_logits_workspace_bytes(100, 72, _lib.LMX_F16) == 4 * 2 * 4096
    assert _lib.linear_loss_logits_workspace_bytes(0, 64, BF16) > 0
    assert _lib.linear_loss_logits_workspace_bytes(16, 64, F32) == 0
    assert _lib.linear_loss_logits_workspace_bytes(-1, 64, BF16) == 0
    assert _lib.linear_loss_logits_workspace_bytes(16, 0, BF16) == 0


def test_header_is_plain_c_and_links(tmp_path):
    """include/lmx.h compiles as C99 and C++ and a C program links against
    liblmx.so and calls the host-only entry points (no GPU needed)."""
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not found")
    inc = os.path.join(ROOT, "include")
    src = tmp_path / "t.c"
    src.write_text(
        '#include "lmx.h"\n#include <stdio.h>\n#include <string.h>\n'
        "int main(void) {\n"
        "  if (strcmp(lmx_status_string(LMX_OK), \"ok\") != 0) return 1;\n"
        "  if (lmx_scale(0, 0, -1, LMX_BF16, 0, 0) != LMX_ERR_SIZE) return 2;\n"
        "  if (ce_workspace_bytes(16, 1000, LMX_F16) == 0) return 3;\n"
        "  if (linear_ce_chunk_rows(16384, 128256, 2048) != 2048) return 4;\n"
        "  printf(\"ok\\n\");\n  return 0;\n}\n")
    exe = tmp_path / "t"
    libdir = os.path.dirname(_lib.LIB_PATH)
    r = subprocess.run([gcc, "-std=c99", "-Wall", "-Werror", "-I", inc, str(src), "-o", str(exe),
                        "-L", libdir, "-llmx", "-Wl,-rpath," + libdir],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True)
    assert r.returncode == 0 and r.stdout.strip() == "ok", (r.returncode, r.stdout, r.stderr)
    gxx = shutil.which("g++")
    if gxx is not None:
        r = subprocess.run([gxx, "-std=c++17", "-fsyntax-only", "-Wall", "-Werror", "-x", "c++",
                            "-I", inc, str(src)], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    # with no built library the binding raises (there is no CPU fallback), and
    # the torch-facing functions refuse host tensors instead of computing on them
    import torch
    from lm_head_cross_pass_amd import functional as F
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "liblmx.so"))
    monkeypatch.setattr(_lib, "_lib", None)
    with pytest.raises(RuntimeError, match="no CPU fallback"):
        _lib.load()
    with pytest.raises(ValueError, match="no CPU path"):
        F.cross_entropy(torch.zeros(2, 8), torch.zeros(2, dtype=torch.int64))
    with pytest.raises(ValueError, match="no CPU path"):
        F.linear_cross_entropy(torch.zeros(2, 8, dtype=torch.bfloat16),
                               torch.zeros(4, 8, dtype=torch.bfloat16),
                               torch.zeros(2, dtype=torch.int64))
