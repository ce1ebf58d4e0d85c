"""Pins of the fp64 oracle against things other than itself (CPU only).

Each check is chosen so that a plausible slip in the oracle (a dropped term, a
wrong sign or index, a transposed operand, the wrong reduction scale) fails at
least one of them; ``test_planted_mistakes_are_caught`` plants such slips in a
copy of the oracle's row function and shows that the pins catch each one.

Sources of truth used here:

* autograd-free central finite differences of the oracle's own loss;
* closed forms derived by hand: uniform logits, one dominant logit, V = 2;
* invariants of the definition (gradient row sums, ignored rows, shift
  invariance, mean times N equals sum);
* reductions to library routines: ``torch.nn.functional.cross_entropy``,
  ``log_softmax`` + ``gather`` (the greyhound page's ``selective_log_softmax``
  equivalence) and torch autograd, all in fp64;
* the bfloat16 format definition and torch's own fp32 -> bf16 cast.
"""
import math

import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle import ce as oce
from oracle import linear_ce as olce
from oracle.bf16 import round_to_bf16
from oracle.fp16 import round_to_fp16
import workloads

torch.set_default_dtype(torch.float64)

ZS = (0.0, 1e-4, 0.5)
REDS = ("mean", "sum")


def _tiny_logits(B=4, V=7, seed=1, ignored=(2,)):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(B, V, generator=g, dtype=torch.float64) * 1.5
    t = torch.randint(0, V, (B,), generator=g)
    for r in ignored:
        t[r] = -100
    return x, t


def _loss(x, t, red, z):
    return oracle.cross_entropy(x, t, -100, red, z, want_grad=False)["loss"]


# ---------------------------------------------------------------- finite differences
def _fd_ce_error(z, red):
    """Max |central difference - oracle gradient| and the tolerance for it."""
    x, t = _tiny_logits()
    out = oracle.cross_entropy(x, t, -100, red, z)
    h = 1e-6
    fd = torch.empty_like(x)
    for i in range(x.shape[0]):
        for j in range(x.shape[1]):
            xp = x.clone(); xp[i, j] += h
            xm = x.clone(); xm[i, j] -= h
            fd[i, j] = (_loss(xp, t, red, z) - _loss(xm, t, red, z)) / (2 * h)
    err = float((fd - out["grad"]).abs().max())
    return err, 1e-8 + 1e-7 * float(fd.abs().max())


@pytest.mark.parametrize("z", ZS)
@pytest.mark.parametrize("red", REDS)
def test_ce_gradient_matches_central_differences(z, red):
    err, tol = _fd_ce_error(z, red)
    assert err <= tol


def _fd_linear_error(z, red, BT=4, D=3, V=5, seed=3):
    g = torch.Generator().manual_seed(seed)
    X = torch.randn(BT, D, generator=g)
    W = torch.randn(V, D, generator=g) * 0.7
    t = torch.randint(0, V, (BT,), generator=g)
    t[1] = -100
    out = olce.linear_cross_entropy(X, W, t, -100, red, z)

    def L(Xv, Wv):
        return olce.linear_cross_entropy(Xv, Wv, t, -100, red, z)["loss"]

    h = 1e-6
    worst = 0.0
    for M, grad, is_x in ((X, out["grad_inputs"], True), (W, out["grad_weight"], False)):
        fd = torch.empty_like(M)
        for i in range(M.shape[0]):
            for j in range(M.shape[1]):
                Mp = M.clone(); Mp[i, j] += h
                Mm = M.clone(); Mm[i, j] -= h
                lp = L(Mp, W) if is_x else L(X, Mp)
                lm = L(Mm, W) if is_x else L(X, Mm)
                fd[i, j] = (lp - lm) / (2 * h)
        worst = max(worst, float((fd - grad).abs().max()) / (1e-8 + 1e-7 * float(fd.abs().max())))
    return worst


@pytest.mark.parametrize("z", (0.0, 0.5))
@pytest.mark.parametrize("red", REDS)
def test_linear_ce_gradients_match_central_differences(z, red):
    assert _fd_linear_error(z, red) <= 1.0


# ---------------------------------------------------------------- closed forms
@pytest.mark.parametrize("V", (1000, 50257, 128256))
@pytest.mark.parametrize("z", (0.0, 1e-4))
@pytest.mark.parametrize("red", REDS)
def test_uniform_logits_closed_form(V, z, red):
    # all V logits equal c: lse = c + log V, loss = log V + z (c + log V)^2,
    # gradient = scale * ((1 + 2 z lse) / V - onehot)
    c = 0.75
    x = torch.full((3, V), c)
    t = torch.tensor([5, -100, V - 1])
    out = oracle.cross_entropy(x, t, -100, red, z)
    lse = c + math.log(V)
    per_row = math.log(V) + z * lse * lse
    n = 2
    expect = per_row * n / (n if red == "mean" else 1)
    assert out["loss"] == pytest.approx(expect, rel=1e-13)
    scale = 1.0 / n if red == "mean" else 1.0
    g = out["grad"]
    assert float(g[0, 0]) == pytest.approx(scale * (1 + 2 * z * lse) / V, rel=1e-12)
    assert float(g[0, 5]) == pytest.approx(scale * ((1 + 2 * z * lse) / V - 1), rel=1e-12)
    assert bool((g[1] == 0).all())


def test_uniform_logits_known_values():
    # natural logs of the vocabulary sizes of the workloads (z = 0 uniform loss)
    for V, val in ((1000, 6.907755278982137), (50257, 10.82490511970208),
                   (128256, 11.761783545564427)):
        assert val == math.log(V)
        out = oracle.cross_entropy(torch.zeros(1, V), torch.tensor([0]), -100, "mean", 0.0)
        assert out["loss"] == pytest.approx(val, abs=1e-12)


@pytest.mark.parametrize("M", (0.5, 4.0, 12.0))
def test_one_dominant_logit_closed_form(M):
    # x_t = M, every other logit 0: loss = log(1 + (V-1) e^-M), p_t = 1/(1+(V-1)e^-M)
    V = 50257
    x = torch.zeros(1, V)
    x[0, 17] = M
    out = oracle.cross_entropy(x, torch.tensor([17]), -100, "sum", 0.0)
    assert out["loss"] == pytest.approx(math.log1p((V - 1) * math.exp(-M)), rel=1e-12)
    p_t = 1.0 / (1.0 + (V - 1) * math.exp(-M))
    p_o = 1.0 / (math.exp(M) + V - 1)
    assert float(out["grad"][0, 17]) == pytest.approx(p_t - 1.0, rel=1e-12)
    assert float(out["grad"][0, 3]) == pytest.approx(p_o, rel=1e-12)


def test_two_classes_is_softplus():
    g = torch.Generator().manual_seed(5)
    x = torch.randn(16, 2, generator=g) * 4
    t = torch.randint(0, 2, (16,), generator=g)
    out = oracle.cross_entropy(x, t, -100, "sum", 0.0)
    other = x.gather(1, (1 - t).unsqueeze(1)).squeeze(1)
    tgt = x.gather(1, t.unsqueeze(1)).squeeze(1)
    d = other - tgt
    sp = torch.where(d > 0, d + torch.log1p(torch.exp(-d)), torch.log1p(torch.exp(d)))
    assert out["row_loss"].tolist() == pytest.approx(sp.tolist(), rel=1e-13)


# ---------------------------------------------------------------- invariants
@pytest.mark.parametrize("z", ZS)
def test_gradient_row_sums_and_ignored_rows(z):
    x, t = _tiny_logits(B=6, V=11, seed=2, ignored=(0, 4))
    for red in REDS:
        out = oracle.cross_entropy(x, t, -100, red, z)
        n = out["n_valid"]
        scale = 1.0 / n if red == "mean" else 1.0
        rs = out["grad"].sum(dim=1)
        for i in range(6):
            if int(t[i]) == -100:
                assert bool((out["grad"][i] == 0).all())
                assert float(out["row_loss"][i]) == 0.0
            else:
                expect = scale * 2 * z * float(out["lse"][i])
                assert float(rs[i]) == pytest.approx(expect, abs=1e-14)


def test_mean_times_n_equals_sum_and_ignored_rows_do_not_matter():
    x, t = _tiny_logits(B=5, V=9, seed=4, ignored=(1, 3))
    m = oracle.cross_entropy(x, t, -100, "mean", 1e-4)
    s = oracle.cross_entropy(x, t, -100, "sum", 1e-4)
    assert m["loss"] * m["n_valid"] == pytest.approx(s["loss"], rel=1e-14)
    x2 = x.clone()
    x2[1] = 1e3 * torch.randn(9)          # change only ignored rows
    s2 = oracle.cross_entropy(x2, t, -100, "sum", 1e-4)
    assert s2["loss"] == s["loss"]


def test_shift_invariance_at_zero_z():
    x, t = _tiny_logits(B=4, V=13, seed=6, ignored=())
    a = oracle.cross_entropy(x, t, -100, "mean", 0.0)
    b = oracle.cross_entropy(x + torch.tensor([[3.0], [-40.0], [0.25], [90.0]]), t, -100,
                             "mean", 0.0)
    assert b["loss"] == pytest.approx(a["loss"], rel=1e-13)
    assert float((a["grad"] - b["grad"]).abs().max()) < 1e-14


def test_large_logits_are_stable():
    x = torch.tensor([[1000.0, 999.0, -1000.0], [-5e4, -5e4 + 1, -5e4 + 2]])
    out = oracle.cross_entropy(x, torch.tensor([0, 2]), -100, "sum", 0.0)
    assert math.isfinite(out["loss"])
    assert out["row_loss"][0] == pytest.approx(math.log1p(math.exp(-1) + math.exp(-2000)),
                                               rel=1e-12)


def test_ignore_index_inside_range_takes_precedence():
    x, _ = _tiny_logits(B=3, V=5, seed=8, ignored=())
    t = torch.tensor([2, 4, 2])
    out = oracle.cross_entropy(x, t, 2, "mean", 0.0)
    assert out["n_valid"] == 1
    assert bool((out["grad"][0] == 0).all()) and bool((out["grad"][2] == 0).all())


def test_out_of_range_target_raises_and_empty_mean_is_nan():
    x, _ = _tiny_logits(B=2, V=5, ignored=())
    with pytest.raises(ValueError):
        oracle.cross_entropy(x, torch.tensor([0, 5]), -100, "mean", 0.0)
    with pytest.raises(ValueError):
        oracle.cross_entropy(x, torch.tensor([-3, 1]), -100, "mean", 0.0)
    out = oracle.cross_entropy(x, torch.tensor([-100, -100]), -100, "mean", 0.0)
    assert math.isnan(out["loss"]) and out["n_valid"] == 0
    assert bool((out["grad"] == 0).all())
    out = oracle.cross_entropy(x, torch.tensor([-100, -100]), -100, "sum", 0.0)
    assert out["loss"] == 0.0


# ---------------------------------------------------------------- library routines
@pytest.mark.parametrize("red", REDS)
def test_matches_torch_cross_entropy_and_autograd(red):
    x, t = _tiny_logits(B=9, V=31, seed=9, ignored=(0, 5, 7))
    for z in ZS:
        out = oracle.cross_entropy(x, t, -100, red, z)
        xr = x.clone().requires_grad_(True)
        ce = F.cross_entropy(xr, t, ignore_index=-100, reduction="sum")
        valid = (t != -100)
        zl = z * (torch.logsumexp(xr, dim=1)[valid] ** 2).sum()
        tot = ce + zl
        if red == "mean":
            tot = tot / valid.sum()
        tot.backward()
        assert out["loss"] == pytest.approx(float(tot.detach()), rel=1e-13)
        assert float((xr.grad - out["grad"]).abs().max()) < 1e-14
        if z == 0.0:
            lib = F.cross_entropy(x, t, ignore_index=-100, reduction=red)
            assert out["loss"] == pytest.approx(float(lib), rel=1e-13)


def test_negated_row_loss_is_selected_log_softmax():
    x, t = _tiny_logits(B=7, V=40, seed=10, ignored=())
    out = oracle.cross_entropy(x, t, -100, "sum", 0.0)
    sel = torch.gather(x.log_softmax(dim=-1), -1, t.unsqueeze(-1)).squeeze(-1)
    assert float((out["row_loss"] + sel).abs().max()) < 1e-13


def test_linear_ce_with_identity_weight_reduces_to_ce():
    g = torch.Generator().manual_seed(11)
    BT, D = 6, 8
    X = torch.randn(BT, D, generator=g)
    t = torch.randint(0, D, (BT,), generator=g)
    t[2] = -100
    lin = oracle.linear_cross_entropy(X, torch.eye(D), t, -100, "mean", 1e-4)
    ce = oracle.cross_entropy(X, t, -100, "mean", 1e-4)
    assert lin["loss"] == pytest.approx(ce["loss"], rel=1e-14)
    assert float((lin["grad_inputs"] - ce["grad"]).abs().max()) < 1e-15
    assert float((lin["grad_weight"] - ce["grad"].T @ X).abs().max()) < 1e-14


def test_linear_ce_matches_torch_autograd():
    g = torch.Generator().manual_seed(12)
    BT, D, V = 10, 6, 17
    X = torch.randn(BT, D, generator=g)
    W = torch.randn(V, D, generator=g) * 0.3
    t = torch.randint(0, V, (BT,), generator=g)
    t[[1, 8]] = -100
    for z in (0.0, 1e-4, 0.5):
        for red in REDS:
            out = oracle.linear_cross_entropy(X, W, t, -100, red, z)
            Xr = X.clone().requires_grad_(True)
            Wr = W.clone().requires_grad_(True)
            logits = Xr @ Wr.T
            valid = t != -100
            tot = F.cross_entropy(logits, t, ignore_index=-100, reduction="sum") + \
                z * (torch.logsumexp(logits, dim=1)[valid] ** 2).sum()
            if red == "mean":
                tot = tot / valid.sum()
            tot.backward()
            assert out["loss"] == pytest.approx(float(tot.detach()), rel=1e-13)
            assert float((Xr.grad - out["grad_inputs"]).abs().max()) < 1e-13
            assert float((Wr.grad - out["grad_weight"]).abs().max()) < 1e-13


def test_linear_ce_blocking_does_not_change_results():
    g = torch.Generator().manual_seed(13)
    X = torch.randn(9, 5, generator=g)
    W = torch.randn(7, 5, generator=g)
    t = torch.randint(0, 7, (9,), generator=g)
    t[4] = -100
    ref = oracle.linear_cross_entropy(X, W, t, -100, "mean", 1e-4, block_rows=9)
    for br in (1, 3, 4):
        o = oracle.linear_cross_entropy(X, W, t, -100, "mean", 1e-4, block_rows=br)
        assert o["loss"] == pytest.approx(ref["loss"], rel=1e-14)
        assert float((o["grad_inputs"] - ref["grad_inputs"]).abs().max()) < 1e-14
        assert float((o["grad_weight"] - ref["grad_weight"]).abs().max()) < 1e-14


def test_sampled_linear_oracle_equals_full_oracle():
    X, W, t = workloads.small_linear_ce(40, 16, 23, dtype=torch.bfloat16, n_ignored=3, seed=2)
    full = oracle.linear_cross_entropy(X, W, t, -100, "mean", 1e-4)
    rows, cols = [0, 7, 39], [0, 5, 22]
    s = olce.linear_cross_entropy_sampled(X, W, t, rows, cols, -100, "mean", 1e-4,
                                          block_rows=16)
    assert s["loss"] == pytest.approx(full["loss"], rel=1e-14)
    assert float((s["grad_inputs_rows"] - full["grad_inputs"][rows]).abs().max()) < 1e-15
    assert float((s["grad_weight_rows"] - full["grad_weight"][cols]).abs().max()) < 1e-15


# ---------------------------------------------------------------- bf16 and weight mode
def test_round_to_bf16_matches_format_and_torch_cast():
    one = 1.0
    cases = {
        one + 2 ** -8: one,                     # exact tie -> even (1.0)
        one + 3 * 2 ** -8: one + 2 ** -6,       # tie -> even (mantissa 2)
        one + 2 ** -8 + 2 ** -20: one + 2 ** -7,
        -(one + 2 ** -7): -(one + 2 ** -7),     # representable
        2.0 ** -133: 2.0 ** -133,               # smallest subnormal
        2.0 ** -135: 0.0,                       # rounds to zero
        3.3895313892515355e38: 3.3895313892515355e38,   # largest finite
        3.40e38: math.inf,                      # rounds past the largest finite
    }
    for v, want in cases.items():
        assert float(round_to_bf16(torch.tensor([v]))[0]) == want
    g = torch.Generator().manual_seed(14)
    vals = torch.cat([torch.randn(20000, generator=g, dtype=torch.float32) *
                      torch.exp2(torch.randint(-140, 120, (20000,), generator=g).float()),
                      torch.tensor([0.0, -0.0, float("inf"), -float("inf")])])
    ours = round_to_bf16(vals.double())
    theirs = vals.to(torch.bfloat16).double()
    assert torch.equal(ours, theirs)


def test_round_to_fp16_matches_format_and_torch_cast():
    one = 1.0
    cases = {
        one + 2 ** -11: one,                    # exact tie -> even (1.0)
        one + 3 * 2 ** -11: one + 2 ** -9,      # tie -> even (mantissa 2)
        one + 2 ** -11 + 2 ** -20: one + 2 ** -10,
        2.0 ** -24: 2.0 ** -24,                 # smallest subnormal
        2.0 ** -26: 0.0,                        # rounds to zero
        3 * 2.0 ** -26: 2.0 ** -24,             # 0.75 quantum rounds up
        65504.0: 65504.0,                       # largest finite
        65519.0: 65504.0,                       # below the overflow midpoint
        65520.0: math.inf,                      # tie at the midpoint -> even -> overflow
    }
    for v, want in cases.items():
        assert float(round_to_fp16(torch.tensor([v]))[0]) == want, v
    g = torch.Generator().manual_seed(15)
    vals = torch.cat([torch.randn(20000, generator=g, dtype=torch.float32) *
                      torch.exp2(torch.randint(-30, 18, (20000,), generator=g).float()),
                      torch.tensor([0.0, -0.0, float("inf"), -float("inf")])])
    ours = round_to_fp16(vals.double())
    theirs = vals.to(torch.float16).double()
    assert torch.equal(ours, theirs)


def test_weight_mode_emulation():
    X, W, t = workloads.small_linear_ce(48, 8, 13, dtype=torch.bfloat16, n_ignored=4, seed=3)
    exact = oracle.linear_cross_entropy(X, W, t, -100, "mean", 0.0)
    one = oracle.linear_cross_entropy(X, W, t, -100, "mean", 0.0, "weight", chunk_size=48)
    # one chunk: a single rounding of the exact result
    assert torch.equal(one["grad_weight"], round_to_bf16(exact["grad_weight"]))
    many = oracle.linear_cross_entropy(X, W, t, -100, "mean", 0.0, "weight", chunk_size=8)
    # each of the 6 roundings moves a value by at most half a bf16 ulp of the
    # running value, which is never larger than the sum of the partial magnitudes
    bound = 6 * 2.0 ** -8 * exact["grad_weight"].abs().max()
    assert float((many["grad_weight"] - exact["grad_weight"]).abs().max()) <= float(bound)
    assert not torch.equal(many["grad_weight"], one["grad_weight"])
    assert torch.equal(many["grad_inputs"], exact["grad_inputs"])
    assert many["loss"] == exact["loss"]


def test_weight_mode_emulation_follows_the_weight_dtype():
    X, W, t = workloads.small_linear_ce(48, 8, 13, dtype=torch.float16, n_ignored=4, seed=3)
    exact = oracle.linear_cross_entropy(X, W, t, -100, "mean", 0.0)
    one = oracle.linear_cross_entropy(X, W, t, -100, "mean", 0.0, "weight", chunk_size=48)
    assert torch.equal(one["grad_weight"], round_to_fp16(exact["grad_weight"]))
    many = oracle.linear_cross_entropy(X, W, t, -100, "mean", 0.0, "weight", chunk_size=8)
    bound = 6 * 2.0 ** -11 * exact["grad_weight"].abs().max()
    assert float((many["grad_weight"] - exact["grad_weight"]).abs().max()) <= float(bound)


# Hand-worked three-chunk cases of the weight-dtype accumulation (greyhound
# functional API page, chunked_linear_cross_entropy, grad_weight_accum_dtype:
# the running gradient is kept in the weight's dtype and rounds between
# chunks). With a zero weight and V = 2 every logit is 0, so every softmax is
# exactly (1/2, 1/2); with all targets 1 and the sum reduction each row's
# logits gradient is (+1/2, -1/2), and the product of chunk c for weight row 0
# is P_c = (x_2c + x_2c+1) / 2 (D = 1, chunks of two rows). Row 1 is the
# negation of row 0 (rounding to nearest even is symmetric).
#
# bf16 (8 significant bits; spacing 2^-8 in [0.5, 1), 2^-7 in [1, 2), 2^-6 in
# [2, 4)). In units of 2^-10: x = 1024, 1032, 1040, 1048, 1032, 4, so
# P = 1028, 1044, 518 and the exact sum is 2590 (2.529296875).
#   per chunk:      rnd(1028) = 1024 (tie between 1024 and 1032; 1024 even),
#                   rnd(1024 + 1044 = 2068) = 2064 (2064 or 2080; 4 away),
#                   rnd(2064 + 518 = 2582) = 2576 (2576 or 2592; 6 away)
#                   -> 2576 / 1024 = 161/64;
#   exact, rounded once:          rnd(2590) = 2592 (2 away) -> 81/32;
#   P_c rounded too:              rnd(1044) = 1040 (tie, even), rnd(518) = 520
#                                 (tie, even): 1024 + 1040 = 2064,
#                                 rnd(2064 + 520 = 2584) = 2592 (tie, even);
#   first rounding skipped:       rnd(1028 + 1044 = 2072) = 2080 (tie, even),
#                                 rnd(2080 + 518 = 2598) = 2592;
#   last two chunks together:     rnd(1044 + 518 = 1562) = 1560,
#                                 rnd(1024 + 1560 = 2584) = 2592 (tie, even).
# fp16 (11 significant bits) is the same case three bits finer: in units of
# 2^-13, x = 8192, 8200, 8208, 8216, 8200, 4, P = 8196, 8212, 4102, and the
# per-chunk result is 20496 / 8192 = 1281/512 where every slip above gives
# 641/256 (the exact sum is 20510 / 8192).
_HAND_WORKED = {
    torch.bfloat16: ([1.0, 1 + 2.0 ** -7, 1 + 2.0 ** -6, 1 + 3 * 2.0 ** -7, 1 + 2.0 ** -7, 2.0 ** -8],
                     161 / 64, 81 / 32, 2590 / 1024),
    torch.float16: ([1.0, 1 + 2.0 ** -10, 1 + 2.0 ** -9, 1 + 3 * 2.0 ** -10, 1 + 2.0 ** -10,
                     2.0 ** -11], 1281 / 512, 641 / 256, 20510 / 8192),
}


@pytest.mark.parametrize("dtype", (torch.bfloat16, torch.float16))
def test_weight_mode_emulation_hand_worked(dtype):
    xs, per_chunk, slip, exact_sum = _HAND_WORKED[dtype]
    X = torch.tensor(xs, dtype=torch.float64).to(dtype).reshape(6, 1)
    assert X.double().flatten().tolist() == xs                  # exact in the format
    W = torch.zeros(2, 1, dtype=dtype)
    t = torch.ones(6, dtype=torch.int64)
    emu = oracle.linear_cross_entropy(X, W, t, -100, "sum", 0.0, "weight", chunk_size=2)
    assert emu["grad_weight"].flatten().tolist() == [per_chunk, -per_chunk]
    assert per_chunk != slip
    exact = oracle.linear_cross_entropy(X, W, t, -100, "sum", 0.0)
    assert exact["grad_weight"].flatten().tolist() == [exact_sum, -exact_sum]
    rnd = round_to_bf16 if dtype == torch.bfloat16 else round_to_fp16
    assert float(rnd(torch.tensor([exact_sum]))[0]) == slip
    # grad_inputs rows: G_r W = 0 for a zero weight
    assert bool((emu["grad_inputs"] == 0).all())
    # one chunk of all six rows is the exact sum rounded once
    one = oracle.linear_cross_entropy(X, W, t, -100, "sum", 0.0, "weight", chunk_size=6)
    assert one["grad_weight"].flatten().tolist() == [slip, -slip]


# ---------------------------------------------------------------- golden fixture
def test_golden_small_workload_is_reproduced():
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "ce_b8_v1000_f32.txt")
    rows = [ln.split() for ln in open(path) if ln.strip() and not ln.startswith("#")]
    logits, target = workloads.ce_inputs(workloads.CE_B8_V1000_F32)
    for z, red, n, loss in rows:
        out = oracle.cross_entropy(logits, target, -100, red, float(z))
        assert out["n_valid"] == int(n)
        assert out["loss"] == float.fromhex(loss)


# ---------------------------------------------------------------- sensitivity
_REAL_ROWS = oce.cross_entropy_rows


def _mutant_rows(kind):
    def rows(x, target, valid, scale, z, want_grad=True):
        lse, rl, g = _REAL_ROWS(x, target, valid, scale, z, want_grad)
        if g is None:
            return lse, rl, g
        x64 = x.to(torch.float64)
        p = torch.exp(x64 - lse.unsqueeze(1))
        if kind == "drop_z_grad":
            g = g - scale * (2 * z * lse).unsqueeze(1) * p * valid.unsqueeze(1)
        elif kind == "sign":
            g = -g
        elif kind == "no_scale":
            g = g / scale if scale not in (0.0, math.inf) else g
        elif kind == "onehot_index":
            t = target.clamp(0, x.shape[1] - 1)
            g = g.clone()
            r = torch.arange(len(t))
            g[r, t] += scale * valid
            g[r, (t + 1) % x.shape[1]] -= scale * valid
        return lse, rl, g
    return rows


@pytest.mark.parametrize("kind", ("drop_z_grad", "sign", "no_scale", "onehot_index"))
def test_planted_mistakes_are_caught(kind, monkeypatch):
    monkeypatch.setattr(oce, "cross_entropy_rows", _mutant_rows(kind))
    caught = any(_fd_ce_error(z, red)[0] > _fd_ce_error(z, red)[1]
                 for red in REDS for z in ZS)
    assert caught, kind


def test_planted_linear_mistakes_are_caught(monkeypatch):
    real = olce.linear_cross_entropy

    def transposed_dw(*a, **k):             # grad_weight = (G^T X)^T, square V = D
        out = real(*a, **k)
        out = dict(out)
        out["grad_weight"] = out["grad_weight"].T.contiguous()
        return out

    def dropped_z(*a, **k):                 # z-loss gradient left out of G
        out = dict(real(*a, **k))
        args = list(a)
        args[5] = 0.0
        out["grad_inputs"] = real(*args, **k)["grad_inputs"]
        return out

    monkeypatch.setattr(olce, "linear_cross_entropy", transposed_dw)
    assert _fd_linear_error(0.0, "mean", BT=4, D=4, V=4) > 1.0
    monkeypatch.setattr(olce, "linear_cross_entropy", dropped_z)
    assert _fd_linear_error(0.5, "sum") > 1.0


@pytest.mark.parametrize("skip", ({1}, {1, 2}, {2}))
def test_planted_weight_mode_mistakes_are_caught(skip, monkeypatch):
    # the emulation rounds once per chunk; skipping the rounding after chunk 1
    # (first rounding missed), after chunks 1 and 2 (exact sum rounded once) or
    # after chunk 2 alone must fail the hand-worked pin
    real = olce.round_to_bf16
    calls = []

    def mutant(v):
        calls.append(1)
        return v.clone() if len(calls) in skip else real(v)

    monkeypatch.setattr(olce, "round_to_bf16", mutant)
    xs, per_chunk, _, _ = _HAND_WORKED[torch.bfloat16]
    X = torch.tensor(xs, dtype=torch.float64).to(torch.bfloat16).reshape(6, 1)
    W = torch.zeros(2, 1, dtype=torch.bfloat16)
    t = torch.ones(6, dtype=torch.int64)
    emu = olce.linear_cross_entropy(X, W, t, -100, "sum", 0.0, "weight", chunk_size=2)
    assert len(calls) == 3
    assert emu["grad_weight"].flatten().tolist() != [per_chunk, -per_chunk]


def test_weight_dtype_accumulation_is_blocking_independent():
    # the element-wise rounding applied to row blocks on several threads gives
    # the same values as one call over the whole matrix
    g = torch.Generator().manual_seed(21)
    dW = round_to_bf16(torch.randn(103, 17, generator=g) * 1e-3)
    P = torch.randn(103, 17, generator=g) * 1e-3
    one = olce.accumulate_weight_dtype(dW, P, torch.bfloat16, 1)
    assert torch.equal(one, round_to_bf16(dW + P))
    assert torch.equal(olce.accumulate_weight_dtype(dW, P, torch.bfloat16, 4), one)
    assert torch.equal(olce.accumulate_weight_dtype(dW, P, torch.float16, 3),
                       round_to_fp16(dW + P))
