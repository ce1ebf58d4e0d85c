"""GPU parity of linear_ce against the fp64 oracle (needs an MI355X).

Tolerances (bf16 inputs): loss within 2e-3 relative; grad_inputs and
grad_weight within 1e-2 relative Frobenius norm of the oracle's exact values;
N exact. 'weight' accumulation is compared with the oracle's chunk-by-chunk
bf16 emulation at the same tolerance. The GPU path rounds the logits and the
logits gradient to bf16 between its matmuls (the matmuls run in bf16); the
oracle models no intermediate rounding, and the tolerance covers it.

fp16 inputs (the same path with fp16 matmuls): loss within 5e-4 relative and
gradients within 2e-3 relative Frobenius (fp16 keeps 3 more significand bits
than bf16; the emulated error of the two roundings is about 2e-4 on these
workloads). The mean's 1/N is applied to the fp32 products, never to the fp16
logits gradient, so probabilities p/N below fp16's smallest subnormal do not
vanish: ``test_fp16_mean_over_a_large_batch`` is the case where they would.
The fp16 outputs themselves are gradients of a mean over thousands of tokens,
often below 2^-14, where fp16 holds only subnormals with a fixed spacing of
2^-24; the output's own rounding (the oracle's value rounded to fp16) is
therefore added to the fp16 gradient bar:
||got - ref|| <= tol ||ref|| + ||fp16(ref) - ref||.
"""
import math

import pytest
import torch

import oracle
import workloads
from oracle import linear_ce as olce
from lm_head_cross_pass_amd import functional as F

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _rel(a, b):
    b = b.double()
    n = float(b.norm())
    d = float((a.double().cpu() - b).norm())
    return d / n if n > 0 else d


TOL = {torch.bfloat16: (2e-3, 1e-2), torch.float16: (5e-4, 2e-3)}   # loss rel, grad rel


def _grad_ok(got, ref, dtype):
    """The gradient bar: relative Frobenius error, plus for fp16 outputs the
    error of rounding the exact value to fp16 itself."""
    ref = ref.double()
    d = float((got.double().cpu() - ref).norm())
    allow = TOL[dtype][1] * float(ref.norm())
    if dtype == torch.float16:
        allow += float((oracle.round_to_fp16(ref) - ref).norm())
    return d <= allow


def _run(X, W, t, red, z, chunk, accum="fp32"):
    out = F.linear_ce(X.to(DEV), W.to(DEV), t.to(DEV), -100, red, z, chunk, accum)
    torch.cuda.synchronize()
    return out


CASES = [
    # BT, D, V, chunk
    (96, 64, 1000, 32),
    (100, 72, 333, 37),        # ragged last chunk, V not a tile multiple
    (64, 136, 129, 64),        # one chunk; D not a multiple of 64
    (257, 128, 4099, 100),
    (300, 256, 8192, 0),       # default chunk size
    (1024, 64, 257, 1024),     # one chunk of 1024 rows; ksplit > 1 path
    (256, 64, 1000, 64),       # four chunks, one grad_weight product over all of them
    (250, 80, 777, 50),        # five chunks, the last one ragged
]


@pytest.mark.parametrize("BT,D,V,chunk", CASES)
def test_shapes_against_oracle(BT, D, V, chunk):
    X, W, t = workloads.small_linear_ce(BT, D, V, n_ignored=max(1, BT // 20), seed=BT + V)
    for red, z in (("mean", 1e-4), ("sum", 0.0), ("mean", 0.5)):
        ref = oracle.linear_cross_entropy(X, W, t, -100, red, z)
        loss, gx, gw, n, bad = _run(X, W, t, red, z, chunk)
        assert int(n) == ref["n_valid"] and int(bad) == 0
        assert float(loss) == pytest.approx(ref["loss"], rel=2e-3)
        assert _rel(gx, ref["grad_inputs"]) <= 1e-2
        assert _rel(gw, ref["grad_weight"]) <= 1e-2
        # ignored rows get exactly zero grad_inputs
        ign = (t == -100).nonzero().flatten()
        assert bool((gx[ign.to(DEV)] == 0).all())


def test_chunk_size_does_not_change_fp32_results():
    X, W, t = workloads.small_linear_ce(192, 64, 700, n_ignored=9, seed=4)
    ref = oracle.linear_cross_entropy(X, W, t, -100, "mean", 1e-4)
    outs = [_run(X, W, t, "mean", 1e-4, c) for c in (1, 7, 64, 192)]
    for loss, gx, gw, n, _ in outs:
        assert float(loss) == pytest.approx(ref["loss"], rel=2e-3)
        assert _rel(gx, ref["grad_inputs"]) <= 1e-2
        assert _rel(gw, ref["grad_weight"]) <= 1e-2
    # grad_inputs rows do not depend on the chunking beyond the rounding of G
    for o in outs[1:]:
        assert _rel(o[1], outs[0][1].cpu()) <= 1e-2


def test_weight_accumulation_follows_the_chunked_rounding():
    X, W, t = workloads.small_linear_ce(512, 64, 300, n_ignored=10, seed=6)
    chunk = 16
    emu = oracle.linear_cross_entropy(X, W, t, -100, "sum", 0.0, "weight", chunk_size=chunk)
    exact = oracle.linear_cross_entropy(X, W, t, -100, "sum", 0.0)
    loss, gx, gw, n, _ = _run(X, W, t, "sum", 0.0, chunk, "weight")
    assert float(loss) == pytest.approx(exact["loss"], rel=2e-3)
    assert _rel(gw, emu["grad_weight"]) <= 1e-2
    assert _rel(gx, exact["grad_inputs"]) <= 1e-2
    _, _, gw32, _, _ = _run(X, W, t, "sum", 0.0, chunk, "fp32")
    assert _rel(gw32, exact["grad_weight"]) <= 1e-2
    # rounding after each of 32 chunks moves the result toward the emulation
    d_emu = float((gw.double().cpu() - emu["grad_weight"]).norm())
    d_exact = float((gw.double().cpu() - exact["grad_weight"]).norm())
    assert d_emu < d_exact


def test_empty_and_all_ignored():
    X, W, t = workloads.small_linear_ce(40, 64, 100, seed=2)
    Xd, Wd = X.to(DEV), W.to(DEV)
    loss, gx, gw, n, _ = F.linear_ce(Xd[:0], Wd, t[:0].to(DEV), -100, "mean", 0.0, 16)
    assert math.isnan(float(loss)) and int(n) == 0 and bool((gw == 0).all())
    tt = torch.full((40,), -100)
    loss, gx, gw, n, _ = F.linear_ce(Xd, Wd, tt.to(DEV), -100, "mean", 0.0, 16)
    assert math.isnan(float(loss)) and bool((gx == 0).all()) and bool((gw == 0).all())
    loss, gx, gw, n, _ = F.linear_ce(Xd, Wd, tt.to(DEV), -100, "sum", 0.0, 16)
    assert float(loss) == 0.0


def test_out_of_range_targets_are_flagged():
    X, W, t = workloads.small_linear_ce(64, 64, 100, seed=3)
    t = t.clone()
    t[5] = 100
    t[9] = -7
    loss, gx, gw, n, bad = _run(X, W, t, "sum", 0.0, 32)
    assert int(bad) == 1 and int(n) == 62
    assert bool((gx[5] == 0).all()) and bool((gx[9] == 0).all())
    t2 = t.clone()
    t2[5] = -100
    t2[9] = -100
    ref = oracle.linear_cross_entropy(X, W, t2, -100, "sum", 0.0)
    assert float(loss) == pytest.approx(ref["loss"], rel=2e-3)


def test_autograd_wrapper():
    from lm_head_cross_pass_amd import linear_cross_entropy
    X, W, t = workloads.small_linear_ce(64, 64, 500, n_ignored=3, seed=7)
    Xd = X.to(DEV).requires_grad_(True)
    Wd = W.to(DEV).requires_grad_(True)
    loss = linear_cross_entropy(Xd, Wd, t.to(DEV), -100, "mean", 1e-4, chunk_size=16)
    (3.0 * loss).backward()
    ref = oracle.linear_cross_entropy(X, W, t, -100, "mean", 1e-4)
    assert float(loss.detach()) == pytest.approx(ref["loss"], rel=2e-3)
    assert _rel(Xd.grad, 3.0 * ref["grad_inputs"]) <= 1e-2
    assert _rel(Wd.grad, 3.0 * ref["grad_weight"]) <= 1e-2


def test_repeatable_bitwise():
    X, W, t = workloads.small_linear_ce(256, 128, 3000, n_ignored=5, seed=9)
    a = _run(X, W, t, "mean", 1e-4, 64)
    b = _run(X, W, t, "mean", 1e-4, 64)
    assert float(a[0]) == float(b[0])
    assert torch.equal(a[1], b[1]) and torch.equal(a[2], b[2])


@pytest.mark.parametrize("BT,D,V,chunk,accum", [
    (256, 128, 3000, 64, "fp32"),     # full chunks: G^T from the grad_inputs GEMM
    (250, 72, 777, 64, "fp32"),       # ragged last chunk, padded vocabulary and K
    (250, 72, 777, 64, "weight"),
    (8448, 64, 2048, 8448, "fp32"),   # split-tail launches along rows
])
def test_workspace_contents_do_not_matter(BT, D, V, chunk, accum):
    # every padding row and column the GEMMs read is written by the same call:
    # a workspace full of NaN bit patterns gives the same bits as a zeroed one
    X, W, t = workloads.small_linear_ce(BT, D, V, n_ignored=7, seed=17)
    Xd, Wd, td = X.to(DEV), W.to(DEV), t.to(DEV)
    from lm_head_cross_pass_amd import _lib
    nbytes = _lib.linear_ce_workspace_bytes(BT, D, V, _lib.LMX_BF16, chunk,
                                            0 if accum == "fp32" else 1, 0)
    outs = []
    for fill in (0x00, 0xFF):
        ws = torch.full((nbytes,), fill, dtype=torch.uint8, device=DEV)
        outs.append(F.linear_ce(Xd, Wd, td, -100, "mean", 1e-4, chunk, accum, workspace=ws))
    torch.cuda.synchronize()
    a, b = outs
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1]) and torch.equal(a[2], b[2])
    assert not bool(torch.isnan(a[2].float()).any())


def test_workload_bt8192_d768_v50257_full():
    w = workloads.LCE_BT8192_D768_V50257
    X, W, t = workloads.linear_ce_inputs(w)
    loss, gx, gw, n, bad = _run(X, W, t, w.reduction, w.z_loss, w.chunk_size, "fp32")
    assert int(n) == w.BT - w.n_ignored == 7782
    ref = oracle.linear_cross_entropy(X, W, t, -100, w.reduction, w.z_loss, block_rows=1024)
    assert float(loss) == pytest.approx(ref["loss"], rel=2e-3)
    assert _rel(gx, ref["grad_inputs"]) <= 1e-2
    assert _rel(gw, ref["grad_weight"]) <= 1e-2


def test_weight_accumulation_with_split_tail_launches():
    # D = 768, V = 50257, two chunks of 1024 in 'weight' mode: one grad_weight
    # product over both chunks (K = 2048) rounds to bf16 after the first chunk
    # inside its K loop; its large tiles leave a last wave under a third full,
    # so the last rows go to a second launch on small tiles
    BT, D, V, C = 2048, 768, 50257, 1024
    X, W, t = workloads.small_linear_ce(BT, D, V, n_ignored=20, seed=47)
    emu = oracle.linear_cross_entropy(X, W, t, -100, "mean", 1e-4, "weight", chunk_size=C,
                                      block_rows=512)
    loss, gx, gw, n, bad = _run(X, W, t, "mean", 1e-4, C, "weight")
    assert int(n) == BT - 20 and int(bad) == 0
    assert float(loss) == pytest.approx(emu["loss"], rel=2e-3)
    assert _rel(gx, emu["grad_inputs"]) <= 1e-2
    assert _rel(gw, emu["grad_weight"]) <= 1e-2


def test_grouped_products_with_k_split_tail_sampled():
    """V = 86016 at D = 64 gives grad_weight 336 large tiles: the last 80 row
    tiles run with K split in three, and their partials are reduced into the
    fp32 accumulator (store, then add) or, in the last group, added and rounded
    to bf16. Thirteen chunks of 2048 make groups of 6, 6 and 1; checked on
    sampled rows, the split rows among them."""
    BT, D, V, C = 13 * 2048, 64, 86016, 2048
    X, W, t = workloads.small_linear_ce(BT, D, V, n_ignored=100, seed=53)
    loss, gx, gw, n, bad = _run(X, W, t, "mean", 1e-4, C, "fp32")
    g = torch.Generator().manual_seed(4)
    rows = torch.randperm(BT, generator=g)[:16].tolist()
    vrows = (torch.randperm(V, generator=g)[:12].tolist() + [65535, 65536, 70000, V - 1]
             + [int(t[rows[0]])])
    ref = olce.linear_cross_entropy_sampled(X, W, t, rows, vrows, -100, "mean", 1e-4,
                                            block_rows=1024)
    assert int(n) == BT - 100 and int(bad) == 0
    assert float(loss) == pytest.approx(ref["loss"], rel=2e-3)
    assert _rel(gx.cpu()[rows], ref["grad_inputs_rows"]) <= 1e-2
    assert _rel(gw.cpu()[vrows], ref["grad_weight_rows"]) <= 1e-2


def test_split_tail_along_rows():
    # one chunk of 8448 rows at V = 2048: its logits product (taken as
    # W X_c^T) has 8 x 33 large tiles, so the last 256 token rows go to a
    # second launch on small tiles (the split along the dimension with more
    # tiles); the first launch alone writes the packed W^T for grad_inputs
    BT, D, V = 8448, 64, 2048
    X, W, t = workloads.small_linear_ce(BT, D, V, n_ignored=40, seed=43)
    loss, gx, gw, n, bad = _run(X, W, t, "mean", 1e-4, BT, "fp32")
    ref = oracle.linear_cross_entropy(X, W, t, -100, "mean", 1e-4, block_rows=1024)
    assert int(n) == BT - 40 and int(bad) == 0
    assert float(loss) == pytest.approx(ref["loss"], rel=2e-3)
    assert _rel(gx, ref["grad_inputs"]) <= 1e-2
    assert _rel(gw, ref["grad_weight"]) <= 1e-2


@pytest.mark.parametrize("accum", ("fp32", "weight"))
def test_logits_split_tail_along_vocabulary_rows(accum):
    # V = 76800 (300 tile rows of W) and chunks of 256 rows (one tile column):
    # chunk 0's logits product runs its first 256 tile rows as one launch and
    # the last 11264 vocabulary rows on small tiles, and both launches write
    # their part of the packed W^T; D = 200 is no multiple of 32 (the packed
    # operands' last block and K step are part zeros) and the third chunk is
    # ragged (88 rows)
    BT, D, V, C = 600, 200, 76800, 256
    X, W, t = workloads.small_linear_ce(BT, D, V, n_ignored=30, seed=61)
    ref = oracle.linear_cross_entropy(X, W, t, -100, "mean", 1e-4, accum, chunk_size=C,
                                      block_rows=200)
    loss, gx, gw, n, bad = _run(X, W, t, "mean", 1e-4, C, accum)
    assert int(n) == BT - 30 and int(bad) == 0
    assert float(loss) == pytest.approx(ref["loss"], rel=2e-3)
    assert _rel(gx, ref["grad_inputs"]) <= 1e-2
    assert _rel(gw, ref["grad_weight"]) <= 1e-2


def test_grouped_grad_weight_products_sampled():
    """Nine chunks of 2048 rows at V = 128256: fp32 accumulation groups four
    chunks per grad_weight product (G^T of 2 GiB; all nine do not fit that plus
    the accumulator), so the products are a first group (fp32 store), a middle
    group (read-modify-write) and the last chunk alone (read-modify-write and
    bf16 cast); checked on sampled rows."""
    BT, D, V, C = 9 * 2048, 64, 128256, 2048
    X, W, t = workloads.small_linear_ce(BT, D, V, n_ignored=200, seed=12)
    loss, gx, gw, n, bad = _run(X, W, t, "mean", 1e-4, C, "fp32")
    g = torch.Generator().manual_seed(3)
    rows = torch.randperm(BT, generator=g)[:16].tolist()
    vrows = torch.randperm(V, generator=g)[:16].tolist() + [int(t[rows[0]]), V - 1]
    ref = olce.linear_cross_entropy_sampled(X, W, t, rows, vrows, -100, "mean", 1e-4,
                                            block_rows=1024)
    assert int(n) == BT - 200 and int(bad) == 0
    assert float(loss) == pytest.approx(ref["loss"], rel=2e-3)
    assert _rel(gx.cpu()[rows], ref["grad_inputs_rows"]) <= 1e-2
    assert _rel(gw.cpu()[vrows], ref["grad_weight_rows"]) <= 1e-2


@pytest.mark.slow
@pytest.mark.parametrize("accum,dtype", (("fp32", torch.bfloat16), ("weight", torch.bfloat16),
                                         ("fp32", torch.float16)))
def test_workload_bt16384_d4096_v128256_sampled(accum, dtype):
    # fp16: the same seeded values converted (every bf16 value of these
    # magnitudes is an fp16 value or rounds to the nearest fp16 subnormal);
    # mean over N = 16056 is where scaling G itself would underflow in fp16
    w = workloads.LCE_BT16384_D4096_V128256
    X, W, t = workloads.linear_ce_inputs(w)
    X, W = X.to(dtype), W.to(dtype)
    lt, gt = TOL[dtype]
    loss, gx, gw, n, bad = _run(X, W, t, w.reduction, w.z_loss, w.chunk_size, accum)
    assert int(n) == 16056 and int(bad) == 0
    g = torch.Generator().manual_seed(2)
    rows = torch.randperm(w.BT, generator=g)[:24].tolist()
    vrows = torch.randperm(w.V, generator=g)[:24].tolist() + [int(t[rows[0]])]
    ref = olce.linear_cross_entropy_sampled(X, W, t, rows, vrows, -100, w.reduction, w.z_loss,
                                            block_rows=1024)
    assert float(loss) == pytest.approx(ref["loss"], rel=lt)
    assert _grad_ok(gx.cpu()[rows], ref["grad_inputs_rows"], dtype)
    assert _grad_ok(gw.cpu()[vrows], ref["grad_weight_rows"], dtype)


@pytest.mark.parametrize("BT,D,V,chunk", CASES)
def test_fp16_shapes_against_oracle(BT, D, V, chunk):
    X, W, t = workloads.small_linear_ce(BT, D, V, dtype=torch.float16,
                                        n_ignored=max(1, BT // 20), seed=BT + V)
    lt, gt = TOL[torch.float16]
    for red, z in (("mean", 1e-4), ("sum", 0.0), ("mean", 0.5)):
        ref = oracle.linear_cross_entropy(X, W, t, -100, red, z)
        loss, gx, gw, n, bad = _run(X, W, t, red, z, chunk)
        assert gx.dtype == torch.float16 and gw.dtype == torch.float16
        assert int(n) == ref["n_valid"] and int(bad) == 0
        assert float(loss) == pytest.approx(ref["loss"], rel=lt)
        assert _grad_ok(gx, ref["grad_inputs"], torch.float16)
        assert _grad_ok(gw, ref["grad_weight"], torch.float16)
        ign = (t == -100).nonzero().flatten()
        assert bool((gx[ign.to(DEV)] == 0).all())


def test_fp16_weight_accumulation_follows_the_chunked_rounding():
    X, W, t = workloads.small_linear_ce(512, 64, 300, dtype=torch.float16, n_ignored=10, seed=6)
    chunk = 16
    lt, gt = TOL[torch.float16]
    emu = oracle.linear_cross_entropy(X, W, t, -100, "sum", 0.0, "weight", chunk_size=chunk)
    exact = oracle.linear_cross_entropy(X, W, t, -100, "sum", 0.0)
    loss, gx, gw, n, _ = _run(X, W, t, "sum", 0.0, chunk, "weight")
    assert float(loss) == pytest.approx(exact["loss"], rel=lt)
    assert _grad_ok(gw, emu["grad_weight"], torch.float16)
    assert _grad_ok(gx, exact["grad_inputs"], torch.float16)
    d_emu = float((gw.double().cpu() - emu["grad_weight"]).norm())
    d_exact = float((gw.double().cpu() - exact["grad_weight"]).norm())
    assert d_emu < d_exact


@pytest.mark.parametrize("z", (1e-4, 0.5))
def test_fp16_mean_over_a_large_batch(z):
    # N = 1946 valid rows over V = 32000: the mean's p/N is about 1.6e-8, under
    # fp16's smallest subnormal 2^-24; scaling G itself would lose the softmax
    # part of every gradient row (an error of 2e-2 to 1e-1 here)
    BT, D, V = 2048, 64, 32000
    X, W, t = workloads.small_linear_ce(BT, D, V, dtype=torch.float16, n_ignored=102, seed=21)
    lt, gt = TOL[torch.float16]
    ref = oracle.linear_cross_entropy(X, W, t, -100, "mean", z, block_rows=512)
    for accum in ("fp32", "weight"):
        loss, gx, gw, n, bad = _run(X, W, t, "mean", z, 512, accum)
        assert int(n) == BT - 102 == ref["n_valid"]
        assert float(loss) == pytest.approx(ref["loss"], rel=lt)
        assert _grad_ok(gx, ref["grad_inputs"], torch.float16)
        assert _grad_ok(gw, ref["grad_weight"], torch.float16)


def test_fp16_autograd_wrapper_and_dtype_checks():
    from lm_head_cross_pass_amd import linear_cross_entropy
    X, W, t = workloads.small_linear_ce(64, 64, 500, dtype=torch.float16, n_ignored=3, seed=7)
    Xd = X.to(DEV).requires_grad_(True)
    Wd = W.to(DEV).requires_grad_(True)
    loss = linear_cross_entropy(Xd, Wd, t.to(DEV), -100, "mean", 1e-4, chunk_size=16)
    (3.0 * loss).backward()
    lt, gt = TOL[torch.float16]
    ref = oracle.linear_cross_entropy(X, W, t, -100, "mean", 1e-4)
    assert float(loss.detach()) == pytest.approx(ref["loss"], rel=lt)
    assert _grad_ok(Xd.grad, 3.0 * ref["grad_inputs"], torch.float16)
    assert _grad_ok(Wd.grad, 3.0 * ref["grad_weight"], torch.float16)
    with pytest.raises(ValueError):   # inputs and weight in different formats
        F.linear_ce(X.to(DEV), W.to(DEV).bfloat16(), t.to(DEV), -100, "mean", 0.0, 16)


def test_page_signature_chunked_linear_cross_entropy():
    from lm_head_cross_pass_amd import chunked_linear_cross_entropy, linear_cross_entropy
    X, W, t = workloads.small_linear_ce(96, 64, 700, n_ignored=4, seed=23)
    grads = []
    for fn in (lambda x, w: chunked_linear_cross_entropy(x, w, t.to(DEV), -100, "mean", 1e-4,
                                                         "fp32", chunk_size=32),
               lambda x, w: linear_cross_entropy(x, w, t.to(DEV), -100, "mean", 1e-4, 32, "fp32")):
        Xd = X.to(DEV).requires_grad_(True)
        Wd = W.to(DEV).requires_grad_(True)
        loss = fn(Xd, Wd)
        loss.backward()
        grads.append((loss.detach(), Xd.grad, Wd.grad))
    torch.cuda.synchronize()
    for a, b in zip(grads[0], grads[1]):
        assert torch.equal(a, b)
    ref = oracle.linear_cross_entropy(X, W, t, -100, "mean", 1e-4)
    assert float(grads[0][0]) == pytest.approx(ref["loss"], rel=2e-3)
    # the default chunk size of the page's signature
    loss = chunked_linear_cross_entropy(X.to(DEV), W.to(DEV), t.to(DEV))
    assert float(loss) == pytest.approx(oracle.linear_cross_entropy(X, W, t, -100, "mean", 0.0)["loss"],
                                        rel=2e-3)


@pytest.mark.parametrize("BT,D,V,chunk", [(1, 8, 5, 0), (3, 16, 7, 1), (513, 8, 31, 256),
                                          (40, 24, 2, 16)])
@pytest.mark.parametrize("dtype", (torch.bfloat16, torch.float16))
def test_tiny_edges(BT, D, V, chunk, dtype):
    # one row, the smallest D the operand alignment allows, two classes, a
    # chunk of one row, a ragged last chunk of one row
    X, W, t = workloads.small_linear_ce(BT, D, V, dtype=dtype, n_ignored=BT // 8, seed=BT * D + V)
    lt, gt = TOL[dtype]
    for red, z in (("mean", 1e-4), ("sum", 0.5)):
        ref = oracle.linear_cross_entropy(X, W, t, -100, red, z)
        for accum in ("fp32", "weight"):
            loss, gx, gw, n, bad = _run(X, W, t, red, z, chunk, accum)
            assert int(n) == ref["n_valid"] and int(bad) == 0
            assert float(loss) == pytest.approx(ref["loss"], rel=lt)
            if accum == "weight":
                emu = oracle.linear_cross_entropy(X, W, t, -100, red, z, "weight",
                                                  chunk_size=olce_chunk(BT, V, chunk))
                assert _grad_ok(gw, emu["grad_weight"], dtype)
            else:
                assert _grad_ok(gw, ref["grad_weight"], dtype)
            assert _grad_ok(gx, ref["grad_inputs"], dtype)


def olce_chunk(BT, V, chunk):
    from lm_head_cross_pass_amd import _lib
    return int(_lib.linear_ce_chunk_rows(BT, V, chunk))


@pytest.mark.parametrize("dtype", (torch.bfloat16, torch.float16))
def test_grad_weight_groups_of_any_size(dtype):
    """32 chunks of 16 rows, grad_weight taken over groups of 1, 3 (the last
    group ragged) or all 32 chunks (the budget in bytes of G^T, 512 x 64 x 2 a
    chunk). 'weight' mode rounds after every chunk inside a group's product and
    carries the running bf16 gradient from group to group, so every grouping
    gives the same bits, close to the chunk-by-chunk emulation; 'fp32' mode
    stays within the bar of the exact value for every grouping; grad_inputs
    does not depend on the grouping."""
    BT, D, V, C = 512, 64, 300, 16
    X, W, t = workloads.small_linear_ce(BT, D, V, dtype=dtype, n_ignored=10, seed=31)
    Xd, Wd, td = X.to(DEV), W.to(DEV), t.to(DEV)
    per_chunk = 512 * 64 * 2
    budgets = (per_chunk, 3 * per_chunk, 0)
    emu = oracle.linear_cross_entropy(X, W, t, -100, "mean", 1e-4, "weight", chunk_size=C)
    exact = oracle.linear_cross_entropy(X, W, t, -100, "mean", 1e-4)
    outs = {acc: [F.linear_ce(Xd, Wd, td, -100, "mean", 1e-4, C, acc, group_bytes=b)
                  for b in budgets] for acc in ("fp32", "weight")}
    torch.cuda.synchronize()
    w = outs["weight"]
    for o in w[1:]:
        assert torch.equal(o[2], w[0][2]) and torch.equal(o[1], w[0][1])
        assert float(o[0]) == float(w[0][0])
    assert _grad_ok(w[0][2], emu["grad_weight"], dtype)
    d_emu = float((w[0][2].double().cpu() - emu["grad_weight"]).norm())
    d_exact = float((w[0][2].double().cpu() - exact["grad_weight"]).norm())
    assert d_emu < d_exact
    for o in outs["fp32"]:
        assert _grad_ok(o[2], exact["grad_weight"], dtype)
        assert torch.equal(o[1], w[0][1])
        assert float(o[0]) == pytest.approx(exact["loss"], rel=TOL[dtype][0])


@pytest.mark.parametrize("accum", ("fp32", "weight"))
def test_grad_weight_short_k_small_tile_tail(accum):
    """D = 768, V = 50257, chunks of 512 with a budget of one chunk: every
    grad_weight product has K = 512, too short to split its last wave of rows
    along K, so those rows go to a second launch on small tiles (fp32 mode:
    store, read-modify-write, the last rounding to bf16; 'weight' mode: the
    running bf16 gradient loaded by each later product)."""
    BT, D, V, C = 1024, 768, 50257, 512
    X, W, t = workloads.small_linear_ce(BT, D, V, n_ignored=20, seed=59)
    per_chunk = 50432 * 512 * 2
    loss, gx, gw, n, bad = F.linear_ce(X.to(DEV), W.to(DEV), t.to(DEV), -100, "mean", 1e-4, C,
                                       accum, group_bytes=per_chunk)
    torch.cuda.synchronize()
    ref = oracle.linear_cross_entropy(X, W, t, -100, "mean", 1e-4, accum, chunk_size=C,
                                      block_rows=512)
    assert int(n) == BT - 20 and int(bad) == 0
    assert float(loss) == pytest.approx(ref["loss"], rel=2e-3)
    assert _rel(gx, ref["grad_inputs"]) <= 1e-2
    assert _rel(gw, ref["grad_weight"]) <= 1e-2


@pytest.mark.parametrize("accum", (0, 1))
def test_linear_ce_replayed_from_a_graph(accum):
    """linear_ce with a caller workspace allocates and synchronizes nothing, so
    a HIP graph can capture a whole call (every chunk's launches): captured once
    on static buffers, replayed on new inputs, weight and targets written into
    them, with eager work and synchronizations between the replays; each
    replay equals an eager call on the same inputs bit for bit (both
    accumulation modes, several grad_weight groups, a ragged last chunk)."""
    from lm_head_cross_pass_amd import _lib
    BT, D, V, C = 1000, 128, 3000, 96
    group = 3 * (3072 * 128 * 2)   # G^T of three chunks (ldv 3072, ldc 128)
    X = torch.empty((BT, D), dtype=torch.bfloat16, device=DEV)
    W = torch.empty((V, D), dtype=torch.bfloat16, device=DEV)
    t = torch.empty(BT, dtype=torch.int64, device=DEV)
    code = _lib.LMX_BF16
    wsb = _lib.linear_ce_workspace_bytes(BT, D, V, code, C, accum, group)

    def call(stream, gx, gw, out, ws):
        _lib.check("linear_ce", _lib.linear_ce(
            X.data_ptr(), W.data_ptr(), t.data_ptr(), BT, D, V, code, -100, _lib.LMX_MEAN, 1e-4,
            C, accum, group, out[0:1].data_ptr(), gx.data_ptr(), gw.data_ptr(),
            out[1:2].data_ptr(), out[2:3].data_ptr(), ws.data_ptr(), wsb, stream))

    def buffers():
        # the loss (fp32) and the flag (int32) fill half of their int64 slots:
        # zeroed, so that the slots compare whole
        return (torch.empty_like(X), torch.empty_like(W),
                torch.zeros(4, dtype=torch.int64, device=DEV),
                torch.empty(wsb, dtype=torch.uint8, device=DEV))

    inputs = [workloads.small_linear_ce(BT, D, V, n_ignored=30 + 7 * i, seed=300 + i)
              for i in range(3)]
    gx, gw, out, ws = buffers()
    X.copy_(inputs[0][0].to(DEV))
    W.copy_(inputs[0][1].to(DEV))
    t.copy_(inputs[0][2].to(DEV))
    side = torch.cuda.Stream(DEV)
    side.wait_stream(torch.cuda.current_stream(DEV))
    with torch.cuda.stream(side):
        call(side.cuda_stream, gx, gw, out, ws)
    torch.cuda.current_stream(DEV).wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call(torch.cuda.current_stream(DEV).cuda_stream, gx, gw, out, ws)
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream(DEV).cuda_stream
    for Xh, Wh, th in inputs + inputs[:1]:
        X.copy_(Xh.to(DEV))
        W.copy_(Wh.to(DEV))
        t.copy_(th.to(DEV))
        rgx, rgw, rout, rws = buffers()
        call(stream, rgx, rgw, rout, rws)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(gx, rgx) and torch.equal(gw, rgw)
        assert torch.equal(out[:3], rout[:3])
        assert int(out[1]) == int((th != -100).sum())
