"""Throughput of the cross-entropy hot path on one MI355X.

One step is one pass of the whole path over one batch of seeded synthetic
input, inputs already resident in HBM (the K steps' CE passes are timed back to
back, then their linear-CE calls, each part after its own warmup;
``ms_per_step`` is the sum of the two parts' wall time per step):

* CE fwd+bwd over logits [16384, 128256] bf16 ~ N(0, 3), 2% ignored rows,
  z = 0, sum reduction, gradient written in place over the logits (each timed
  step gets its own pre-generated copy of the logits, so every step reads
  fresh logits);
* chunked linear-CE with inputs [16384, 4096] bf16 ~ N(0, 1), weight
  [128256, 4096] bf16 ~ N(0, 0.02), 2% ignored, chunk 2048, mean, z = 0,
  fp32 grad_weight accumulation, the library's default grad_weight grouping
  (2 GiB of transposed logits gradient per product: four chunks).

The JSON line reports the CE leg as ``value`` (GB/s of algorithmic traffic:
one read of the logits, one write of the gradient, the int64 targets) with its
roofline against the 8 TB/s HBM peak, and the linear-CE leg under
``linear_ce`` (TFLOP/s of the three matmuls, 6 BT V D, against the 2.5 PFLOP/s
dense bf16 MFMA peak) with its workspace bytes, plus, each timed on its own,
'weight' accumulation and both modes with one grad_weight product over every
chunk (``one_group``: the G^T budget that holds all eight chunks).
``next_rows`` times the per-row entry points on the CE leg's logits (forward-only
reduced CE, selective_log_softmax, the unreduced per-row CE and its VJP), each
in GB/s of its own algorithmic bytes; ``linear_ce.generic_chunked_loss`` times the
generic chunked linear loss with the library's cross-entropy as the caller's loss
on the linear-CE inputs; ``fp16`` times the CE and the fused linear-CE on the
same values converted to IEEE binary16. ``cpu_baseline`` is the fp64 oracle timed
on the host on a bounded sample of the same CE workload. ``traffic`` (HBM bytes)
and the linear leg's ``mfma_busy`` (each GEMM's matrix-core busy share and the
clock under that load) come from the committed rocprofv3 counter summaries in
``profiles/`` and are null when those were taken on other kernel code.

    python bench.py [--gpus 1] [--steps 10] [--warmup 3]
                    [--legs ce,linear,rows,generic,fp16,small] [--no-cpu]

``small_workloads`` times the two GPT-2-shaped workloads, CE [4096, 50257] and
linear-CE 8192 x 768 x 50257, each with its roofline fraction and, where a
counter summary of the same code is committed, its HBM traffic. Every timed
figure is the mean over back-to-back calls (``ms_median`` beside it).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
PROFILES = os.path.join(ROOT, "profiles")


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def source_digest(*names: str) -> str:
    """Digest of the code of these kernel sources (comments and blank lines
    removed), which ties a stored counter summary to the code it measured."""
    import re
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "lm_head_cross_pass_amd", "csrc", n)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        code = "\n".join(ln.rstrip() for ln in text.splitlines() if ln.strip())
        h.update(code.encode())
    return h.hexdigest()[:16]


def stored_values(counter_file: str, digest: str):
    """The `key = value` lines of a committed counter summary, if it matches the
    current source (else None)."""
    path = os.path.join(PROFILES, counter_file)
    if not os.path.exists(path):
        return None
    vals = {}
    for ln in open(path):
        if "=" in ln and not ln.lstrip().startswith("#"):
            k, v = ln.split("=", 1)
            vals[k.strip()] = v.strip()
    return vals if vals.get("source_digest") == digest else None


def stored_traffic(counter_file: str, digest: str, key: str = "hbm_bytes_per_launch"):
    """HBM bytes per launch (or per call) from a committed counter summary, if it
    matches the current source."""
    vals = stored_values(counter_file, digest)
    if vals is None or key not in vals:
        return None
    return float(vals[key])


def per_call_ms(fn, n: int, warm: int, stream):
    """Times n calls of fn back to back on `stream` with HIP events between
    them (after `warm` untimed calls); returns the per-call times in ms."""
    import torch
    for _ in range(warm):
        fn()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
    torch.cuda.synchronize()
    ev[0].record(stream)
    for i in range(n):
        fn()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    return [ev[i].elapsed_time(ev[i + 1]) for i in range(n)]


def mean_median(ts):
    import statistics
    return sum(ts) / len(ts), statistics.median(ts)


def gt_group_bytes_all(BT: int, V: int, chunk: int) -> int:
    """A grad_weight group budget that covers every chunk of the call: the
    transposed logits gradient of all chunks (vocabulary padded to 256, chunk
    rows to 64, 2 bytes)."""
    ldv = (V + 255) // 256 * 256
    ldc = (chunk + 63) // 64 * 64
    return (BT + chunk - 1) // chunk * ldv * ldc * 2


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--legs", default="ce,linear,rows,generic,fp16,small",
                    help="ce, linear, rows (per-row entry points; needs ce), generic (the "
                         "generic chunked linear loss; needs linear), fp16 (the ce and linear "
                         "legs' workloads in fp16), small (the two GPT-2-shaped workloads)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle cpu_baseline leg")
    ap.add_argument("--weight-steps", type=int, default=3)
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        return 2
    legs = set(args.legs.split(","))

    import torch
    import workloads
    from lm_head_cross_pass_amd import _lib

    if not os.path.exists(_lib.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    K, W = args.steps, args.warmup

    # ------------------------------------------------------------ inputs
    ce_w = workloads.CE_B16384_V128256_BF16
    lin_w = workloads.LCE_BT16384_D4096_V128256
    if "ce" in legs:
        log(f"generating {ce_w.name}")
        logits_h, target_h = workloads.ce_inputs(ce_w)
        target = target_h.to(dev)
        first = logits_h.to(dev)
        ncopies = K + 1
        log(f"placing {ncopies} copies of the logits in HBM "
            f"({ncopies * first.numel() * 2 / 2**30:.1f} GiB)")
        copies = [first] + [first.clone() for _ in range(ncopies - 1)]
        ce_ws = torch.empty(_lib.ce_workspace_bytes(ce_w.B, ce_w.V, _lib.LMX_BF16),
                            dtype=torch.uint8, device=dev)
        ce_out = [torch.empty((), dtype=torch.float32, device=dev),
                  torch.empty((), dtype=torch.int64, device=dev),
                  torch.empty((), dtype=torch.int32, device=dev)]

        def ce_call(x):
            st = _lib.ce_fwd_bwd(x.data_ptr(), x.data_ptr(), target.data_ptr(), ce_w.B, ce_w.V,
                                 _lib.LMX_BF16, -100, _lib.LMX_SUM, ce_w.z_loss[0],
                                 ce_out[0].data_ptr(), ce_out[1].data_ptr(), ce_out[2].data_ptr(),
                                 ce_ws.data_ptr(), ce_ws.numel(), stream.cuda_stream)
            _lib.check("ce_fwd_bwd", st)
    if "linear" in legs:
        log(f"generating {lin_w.name}")
        X_h, W_h, t_h = workloads.linear_ce_inputs(lin_w)
        X, Wt, tl = X_h.to(dev), W_h.to(dev), t_h.to(dev)
        del X_h, W_h
        gx, gw = torch.empty_like(X), torch.empty_like(Wt)
        lin_out = [torch.empty((), dtype=torch.float32, device=dev),
                   torch.empty((), dtype=torch.int64, device=dev),
                   torch.empty((), dtype=torch.int32, device=dev)]
        one_group = gt_group_bytes_all(lin_w.BT, lin_w.V, lin_w.chunk_size)

        def lin_ws_bytes(accum, group_bytes=0):
            return _lib.linear_ce_workspace_bytes(lin_w.BT, lin_w.D, lin_w.V, _lib.LMX_BF16,
                                                  lin_w.chunk_size, accum, group_bytes)
        ws_bytes = max(lin_ws_bytes(_lib.LMX_ACC_F32), lin_ws_bytes(_lib.LMX_ACC_WEIGHT),
                       lin_ws_bytes(_lib.LMX_ACC_F32, one_group))
        lin_ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)

        def lin_call(accum, group_bytes=0):
            st = _lib.linear_ce(X.data_ptr(), Wt.data_ptr(), tl.data_ptr(), lin_w.BT, lin_w.D,
                                lin_w.V, _lib.LMX_BF16, -100, _lib.LMX_MEAN, lin_w.z_loss,
                                lin_w.chunk_size, accum, group_bytes, lin_out[0].data_ptr(),
                                gx.data_ptr(), gw.data_ptr(), lin_out[1].data_ptr(),
                                lin_out[2].data_ptr(), lin_ws.data_ptr(), lin_ws.numel(),
                                stream.cuda_stream)
            _lib.check("linear_ce", st)

    # ------------------------------------------------------------ timed steps
    # A step is one CE pass and one linear-CE call. The K CE passes are timed
    # back to back, then the K linear-CE calls, each part after its own W warmup
    # calls, so that neither is timed in the transition from the other (a CE
    # pass issued right after a GEMM-heavy call measured about 1% slower).
    # copies[0] stays pristine; the CE warmup works in place on copies[1], which
    # is then restored, and timed CE pass i consumes copies[i + 1].
    log(f"warmup {W} and timing {K} steps")
    ce_ms = lin_ms = 0.0
    wall_ms = 0.0
    if "ce" in legs:
        for _ in range(W):
            ce_call(copies[1])
        copies[1].copy_(copies[0])
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(K + 1)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        ev[0].record(stream)
        for i in range(K):
            ce_call(copies[i + 1])
            ev[i + 1].record(stream)
        torch.cuda.synchronize()
        wall_ms += (time.perf_counter() - t0) * 1e3 / K
        ce_ms, ce_med = mean_median([ev[i].elapsed_time(ev[i + 1]) for i in range(K)])
    if "linear" in legs:
        for _ in range(W):
            lin_call(_lib.LMX_ACC_F32)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(K + 1)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        ev[0].record(stream)
        for i in range(K):
            lin_call(_lib.LMX_ACC_F32)
            ev[i + 1].record(stream)
        torch.cuda.synchronize()
        wall_ms += (time.perf_counter() - t0) * 1e3 / K
        lin_ms, lin_med = mean_median([ev[i].elapsed_time(ev[i + 1]) for i in range(K)])
    log(f"step {wall_ms:.3f} ms (ce {ce_ms:.3f} ms, linear {lin_ms:.3f} ms)")

    line = {
        "metric": "CE fwd+bwd GB/s (% HBM peak) @V=128256; linear-CE TFLOP/s (% MFMA peak)",
        "value": None, "unit": "GB/s", "n_gpus": 1, "steps": K, "warmup": W,
        "ms_per_step": round(wall_ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded, shapes and distributions of the workloads)",
        "config": {"workload": "", "parallelism": "none (one GPU)"},
    }
    workload_names = []
    if "ce" in legs:
        ce_bytes = 2 * ce_w.B * ce_w.V * 2 + 8 * ce_w.B
        gbps = ce_bytes / (ce_ms * 1e-3) / 1e9
        digest = source_digest("ce.hip", "common.h")
        traffic = stored_traffic("ce_rows_b16384_v128256_bf16.counters.txt", digest)
        line["value"] = round(gbps, 1)
        line["roofline"] = {"bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS,
                            "unit": "GB/s", "frac": round(gbps / HBM_PEAK_GBPS, 4),
                            "traffic": traffic,
                            "algorithmic_bytes_per_launch": ce_bytes,
                            "ms_per_launch": round(ce_ms, 4), "ms_median": round(ce_med, 4),
                            "kernel": "ce_rows_reg_kernel<bf16,1024,16> (+ count, finish)"}
        workload_names.append(ce_w.name)
        line["config"].update({"ce_B": ce_w.B, "ce_V": ce_w.V, "ce_reduction": "sum",
                               "ce_in_place": True})
    if "linear" in legs:
        flops = 6.0 * lin_w.BT * lin_w.V * lin_w.D
        tf = flops / (lin_ms * 1e-3) / 1e12
        lin_digest = source_digest("gemm.h", "linear_ce.hip", "ce.hip", "common.h")
        lin_traffic = stored_traffic("linear_ce_bt16384_d4096_v128256_c2048.counters.txt",
                                     lin_digest, "hbm_bytes_per_call")
        # matrix-core busy share of each GEMM's cycles and the clock under that
        # load, from the committed counter summary of the same code
        mv = stored_values("linear_ce_bt16384_d4096_v128256_c2048.mfma.txt", lin_digest)
        mfma_busy = None
        if mv is not None:
            mfma_busy = {k[len("mfma_busy_"):]: float(v) for k, v in mv.items()
                         if k.startswith("mfma_busy_")}
            if "clock_ghz_under_load" in mv:
                mfma_busy["clock_ghz"] = float(mv["clock_ghz_under_load"])
        lin = {"value": round(tf, 1), "unit": "TFLOP/s", "ms_per_call": round(lin_ms, 3),
               "ms_median": round(lin_med, 3),
               "workspace_bytes": lin_ws_bytes(_lib.LMX_ACC_F32),
               "roofline": {"bound": "mfma", "achieved": round(tf, 1),
                            "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                            "frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": lin_traffic,
                            "algorithmic_flops_per_call": flops,
                            "mfma_busy": mfma_busy,
                            "kernel": "whole linear_ce call (gemm_nt_bdir_kernel x3 per chunk + CE)"}}
        # 'weight' accumulation, and both modes with one grad_weight product over
        # every chunk (a G^T budget that holds them all: more workspace, no
        # fp32 accumulator), each timed on its own
        if args.weight_steps > 0:
            for key, accum, gb in (("weight_accum", _lib.LMX_ACC_WEIGHT, 0),
                                   ("one_group", _lib.LMX_ACC_F32, one_group),
                                   ("weight_accum_one_group", _lib.LMX_ACC_WEIGHT, one_group)):
                wms, wmed = mean_median(per_call_ms(lambda: lin_call(accum, gb),
                                                    args.weight_steps, 1, stream))
                lin[key] = {"value": round(flops / (wms * 1e-3) / 1e12, 1), "unit": "TFLOP/s",
                            "ms_per_call": round(wms, 3), "ms_median": round(wmed, 3),
                            "group_bytes": gb, "workspace_bytes": lin_ws_bytes(accum, gb)}
                log(f"linear-CE {key}: {wms:.3f} ms")
        # the generic chunked loss with the library's cross-entropy as the caller's
        # loss (sum reduction, fp32 accumulation), on the same inputs
        if "generic" in legs:
            from lm_head_cross_pass_amd import functional as LF
            gen_ws = torch.empty(_lib.linear_loss_workspace_bytes(
                lin_w.BT, lin_w.D, lin_w.V, _lib.LMX_BF16, lin_w.chunk_size, _lib.LMX_ACC_F32),
                dtype=torch.uint8, device=dev)

            def gen_call():
                return LF.chunked_linear_loss_fwd(X, Wt, LF.cross_entropy_loss_and_grad, (tl,),
                                                  chunk_size=lin_w.chunk_size, workspace=gen_ws)
            gen_call()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record(stream)
            for _ in range(3):
                gen_call()
            e1.record(stream)
            torch.cuda.synchronize()
            gms = e0.elapsed_time(e1) / 3
            lin["generic_chunked_loss"] = {"value": round(flops / (gms * 1e-3) / 1e12, 1),
                                           "unit": "TFLOP/s", "ms_per_call": round(gms, 3),
                                           "loss": "library cross-entropy, sum"}
            log(f"generic chunked loss: {gms:.3f} ms")
        line["linear_ce"] = lin
        workload_names.append(lin_w.name)
        line["config"].update({"lin_BT": lin_w.BT, "lin_D": lin_w.D, "lin_V": lin_w.V,
                               "lin_chunk": lin_w.chunk_size, "lin_accum": "fp32"})
        if line["value"] is None:
            line["value"], line["unit"] = lin["value"], "TFLOP/s"
    line["config"]["workload"] = " + ".join(workload_names)

    # ------------------------------------------------------------ HBM ceilings (context)
    # streaming patterns of known size over the CE leg's 4.2 GB buffers: read
    # only, write only, two copy shapes and the two row patterns of the widest
    # CE row kernel (in place, rows of the CE workload's width); bytes moved
    # count a read and a write separately
    if "ce" in legs:
        nb = ce_w.B * ce_w.V * 2
        src, dst = copies[0], copies[1]
        sink = torch.empty(16384, dtype=torch.uint8, device=dev)
        row_bytes = ce_w.V * 2
        probes = (("read", _lib.LMX_PROBE_READ, src, sink, nb),
                  ("write", _lib.LMX_PROBE_WRITE, src, dst, nb),
                  ("copy", _lib.LMX_PROBE_COPY, src, dst, 2 * nb),
                  ("copy_batched", _lib.LMX_PROBE_COPY_BATCHED, src, dst, 2 * nb),
                  ("copy_batched_in_place", _lib.LMX_PROBE_COPY_BATCHED, dst, dst, 2 * nb),
                  ("rows_interleaved_in_place", _lib.LMX_PROBE_ROWS_INTERLEAVED, dst, dst, 2 * nb),
                  ("rows_phased_in_place", _lib.LMX_PROBE_ROWS_PHASED, dst, dst, 2 * nb))
        ceil = {"unit": "GB/s", "buffer_bytes": nb, "row_bytes": row_bytes}
        for name, mode, a, b, moved in probes:
            def probe_call(a=a, b=b, mode=mode):
                _lib.check("lmx_stream_probe", _lib.lmx_stream_probe(
                    a.data_ptr(), b.data_ptr(), nb, row_bytes, mode, stream.cuda_stream))
            ms, med = mean_median(per_call_ms(probe_call, 5, 1, stream))
            ceil[name] = round(moved / (med * 1e-3) / 1e9, 1)
        log(f"hbm ceilings (GB/s): {ceil}")
        line["hbm_ceiling"] = ceil

    # ------------------------------------------------------------ per-row entry points
    # forward-only reduced CE, selective_log_softmax, the unreduced per-row CE and
    # its VJP, on the same [16384, 128256] bf16 logits (resident in HBM)
    if "ce" in legs and "rows" in legs:
        B, V = ce_w.B, ce_w.V
        src, dst = copies[0], copies[1]
        index = torch.clamp(target, min=0)
        rl = torch.empty(B, dtype=torch.float32, device=dev)
        lp = torch.empty(B, dtype=torch.float32, device=dev)
        g = workloads.row_upstream(B).to(dev)
        sp = stream.cuda_stream

        def fwd_only():
            _lib.check("ce_fwd_bwd", _lib.ce_fwd_bwd(
                src.data_ptr(), None, target.data_ptr(), B, V, _lib.LMX_BF16, -100, _lib.LMX_SUM,
                0.0, ce_out[0].data_ptr(), ce_out[1].data_ptr(), ce_out[2].data_ptr(),
                ce_ws.data_ptr(), ce_ws.numel(), sp))

        def sel():
            _lib.check("selective_log_softmax", _lib.selective_log_softmax(
                src.data_ptr(), index.data_ptr(), B, V, _lib.LMX_BF16, lp.data_ptr(),
                ce_out[2].data_ptr(), ce_ws.data_ptr(), ce_ws.numel(), sp))

        def rows_fwd():
            _lib.check("ce_loss_rows", _lib.ce_loss_rows(
                src.data_ptr(), target.data_ptr(), B, V, _lib.LMX_BF16, -100, rl.data_ptr(),
                ce_out[1].data_ptr(), ce_out[2].data_ptr(), ce_ws.data_ptr(), ce_ws.numel(), sp))

        def vjp():
            _lib.check("ce_loss_rows_vjp", _lib.ce_loss_rows_vjp(
                src.data_ptr(), target.data_ptr(), rl.data_ptr(), g.data_ptr(), dst.data_ptr(),
                B, V, _lib.LMX_BF16, -100, sp))

        read_bytes = B * V * 2 + 8 * B
        legs_rows = (("ce_forward_only", fwd_only, read_bytes),
                     ("selective_log_softmax", sel, read_bytes + 4 * B),
                     ("ce_loss_rows", rows_fwd, read_bytes + 4 * B),
                     ("ce_loss_rows_vjp", vjp, 2 * B * V * 2 + 16 * B))
        rows_line = {"workload": ce_w.name, "unit": "GB/s", "peak": HBM_PEAK_GBPS}
        rows_fwd()
        # every entry point runs a few times before any is timed, so that the
        # first one timed does not pay for the switch from the GEMM-heavy legs
        for _ in range(3):
            for _, fn, _ in legs_rows:
                fn()
        for name, fn, nbytes in legs_rows:
            for _ in range(3):
                fn()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record(stream)
            for _ in range(10):
                fn()
            e1.record(stream)
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / 10
            gbps = nbytes / (ms * 1e-3) / 1e9
            rows_line[name] = {"value": round(gbps, 1), "ms_per_call": round(ms, 4),
                               "algorithmic_bytes": nbytes, "frac": round(gbps / HBM_PEAK_GBPS, 4)}
            log(f"{name}: {ms:.3f} ms, {gbps:.0f} GB/s")
        line["next_rows"] = rows_line

    # ------------------------------------------------------------ fp16 inputs
    # the same workloads with the values converted to IEEE binary16: the CE row
    # kernel (out of place) and the fused linear-CE with fp16 matmuls
    if "fp16" in legs:
        f16 = {}
        if "ce" in legs:
            B, V = ce_w.B, ce_w.V
            x16 = copies[0].to(torch.float16)
            g16 = torch.empty_like(x16)

            def ce16():
                _lib.check("ce_fwd_bwd", _lib.ce_fwd_bwd(
                    x16.data_ptr(), g16.data_ptr(), target.data_ptr(), B, V, _lib.LMX_F16, -100,
                    _lib.LMX_SUM, 0.0, ce_out[0].data_ptr(), ce_out[1].data_ptr(),
                    ce_out[2].data_ptr(), ce_ws.data_ptr(), ce_ws.numel(), stream.cuda_stream))
            for _ in range(3):
                ce16()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record(stream)
            for _ in range(10):
                ce16()
            e1.record(stream)
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / 10
            nbytes = 2 * B * V * 2 + 8 * B
            gbps = nbytes / (ms * 1e-3) / 1e9
            f16["ce_fwd_bwd"] = {"value": round(gbps, 1), "unit": "GB/s", "ms_per_call": round(ms, 4),
                                 "frac": round(gbps / HBM_PEAK_GBPS, 4),
                                 "workload": ce_w.name + " as fp16, out of place"}
            log(f"fp16 CE: {ms:.3f} ms, {gbps:.0f} GB/s")
            del x16, g16
        if "linear" in legs:
            X16, W16 = X.to(torch.float16), Wt.to(torch.float16)
            gx16, gw16 = torch.empty_like(X16), torch.empty_like(W16)

            def lin16():
                _lib.check("linear_ce", _lib.linear_ce(
                    X16.data_ptr(), W16.data_ptr(), tl.data_ptr(), lin_w.BT, lin_w.D, lin_w.V,
                    _lib.LMX_F16, -100, _lib.LMX_MEAN, lin_w.z_loss, lin_w.chunk_size,
                    _lib.LMX_ACC_F32, 0, lin_out[0].data_ptr(), gx16.data_ptr(), gw16.data_ptr(),
                    lin_out[1].data_ptr(), lin_out[2].data_ptr(), lin_ws.data_ptr(),
                    lin_ws.numel(), stream.cuda_stream))
            lin16()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record(stream)
            for _ in range(3):
                lin16()
            e1.record(stream)
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / 3
            flops = 6.0 * lin_w.BT * lin_w.V * lin_w.D
            tf = flops / (ms * 1e-3) / 1e12
            f16["linear_ce"] = {"value": round(tf, 1), "unit": "TFLOP/s", "ms_per_call": round(ms, 3),
                                "frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4),
                                "workload": lin_w.name + " as fp16, fp32 accumulation"}
            log(f"fp16 linear-CE: {ms:.3f} ms, {tf:.0f} TFLOP/s")
            del X16, W16, gx16, gw16
        line["fp16"] = f16

    # ------------------------------------------------------------ GPT-2-shaped workloads
    # the two smaller workloads, shaped after GPT-2's tied 50257 x 768 head:
    # CE [4096, 50257] bf16, mean, z 1e-4, out of place (four copies of the
    # logits in rotation, so that a call does not find its input in the 256 MB
    # MALL from the call before), and linear-CE [8192, 768] x [50257, 768],
    # chunk 1024, fp32 accumulation
    if "small" in legs:
        sm = {}
        cw = workloads.CE_B4096_V50257_BF16
        xh, th = workloads.ce_inputs(cw)
        t2 = th.to(dev)
        xs = [xh.to(dev) for _ in range(4)]
        g2 = torch.empty_like(xs[0])
        ws2 = torch.empty(_lib.ce_workspace_bytes(cw.B, cw.V, _lib.LMX_BF16), dtype=torch.uint8,
                          device=dev)
        o2 = [torch.empty((), dtype=torch.float32, device=dev),
              torch.empty((), dtype=torch.int64, device=dev),
              torch.empty((), dtype=torch.int32, device=dev)]
        rot = [0]

        def ce2():
            x2 = xs[rot[0] % len(xs)]
            rot[0] += 1
            _lib.check("ce_fwd_bwd", _lib.ce_fwd_bwd(
                x2.data_ptr(), g2.data_ptr(), t2.data_ptr(), cw.B, cw.V, _lib.LMX_BF16, -100,
                _lib.LMX_MEAN, cw.z_loss[0], o2[0].data_ptr(), o2[1].data_ptr(), o2[2].data_ptr(),
                ws2.data_ptr(), ws2.numel(), stream.cuda_stream))
        lw = workloads.LCE_BT8192_D768_V50257
        Xh, Wh, tlh = workloads.linear_ce_inputs(lw)
        X4, W4, t4 = Xh.to(dev), Wh.to(dev), tlh.to(dev)
        gx4, gw4 = torch.empty_like(X4), torch.empty_like(W4)
        ws4_bytes = _lib.linear_ce_workspace_bytes(lw.BT, lw.D, lw.V, _lib.LMX_BF16,
                                                   lw.chunk_size, _lib.LMX_ACC_F32, 0)
        ws4 = torch.empty(ws4_bytes, dtype=torch.uint8, device=dev)

        def lin4():
            _lib.check("linear_ce", _lib.linear_ce(
                X4.data_ptr(), W4.data_ptr(), t4.data_ptr(), lw.BT, lw.D, lw.V, _lib.LMX_BF16,
                -100, _lib.LMX_MEAN, lw.z_loss, lw.chunk_size, _lib.LMX_ACC_F32, 0,
                o2[0].data_ptr(), gx4.data_ptr(), gw4.data_ptr(), o2[1].data_ptr(),
                o2[2].data_ptr(), ws4.data_ptr(), ws4.numel(), stream.cuda_stream))

        ms, med = mean_median(per_call_ms(ce2, 20, 4, stream))
        nbytes = 2 * cw.B * cw.V * 2 + 8 * cw.B
        gbps = nbytes / (ms * 1e-3) / 1e9
        sm[cw.name] = {"value": round(gbps, 1), "unit": "GB/s", "ms_per_call": round(ms, 4),
                       "ms_median": round(med, 4), "frac": round(gbps / HBM_PEAK_GBPS, 4),
                       "algorithmic_bytes": nbytes,
                       "traffic": stored_traffic("ce_rows_b4096_v50257_bf16.counters.txt",
                                                 source_digest("ce.hip", "common.h")),
                       "kernel": "ce_rows_reg_kernel<bf16,512,13> (+ count, finish)"}
        log(f"{cw.name}: {ms * 1e3:.1f} us, {gbps:.0f} GB/s")
        ms, med = mean_median(per_call_ms(lin4, 20, 3, stream))
        flops = 6.0 * lw.BT * lw.V * lw.D
        tf = flops / (ms * 1e-3) / 1e12
        sm[lw.name] = {"value": round(tf, 1), "unit": "TFLOP/s", "ms_per_call": round(ms, 4),
                       "ms_median": round(med, 4), "frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4),
                       "algorithmic_flops": flops, "workspace_bytes": ws4_bytes,
                       "traffic": stored_traffic(
                           "linear_ce_bt8192_d768_v50257_c1024.counters.txt",
                           source_digest("gemm.h", "linear_ce.hip", "ce.hip", "common.h"),
                           "hbm_bytes_per_call"),
                       "kernel": "whole linear_ce call"}
        log(f"{lw.name}: {ms:.3f} ms, {tf:.0f} TFLOP/s")
        line["small_workloads"] = sm
        del xs, g2, X4, W4, gx4, gw4

    # ------------------------------------------------------------ oracle on the host
    if not args.no_cpu and "ce" in legs:
        import oracle
        del copies
        # blocks of 2048 rows, in order, until about 20 s of host work or all rows
        blk, rows, dt = 2048, 0, 0.0
        log(f"cpu_baseline: fp64 oracle on row blocks of {ce_w.name}")
        while rows < ce_w.B and dt < 20.0:
            sel = slice(rows, min(rows + blk, ce_w.B))
            t0 = time.perf_counter()
            oracle.cross_entropy(logits_h[sel], target_h[sel], -100, "sum", 0.0)
            dt += time.perf_counter() - t0
            rows = sel.stop
        sb = 2 * rows * ce_w.V * 2 + 8 * rows
        line["cpu_baseline"] = {"value": round(sb / dt / 1e9, 3), "unit": "GB/s",
                                "cores": torch.get_num_threads(), "kind": "oracle",
                                "sample": f"first {rows} of {ce_w.B} rows of the CE workload "
                                          f"in blocks of {blk} (loss and gradient, fp64), "
                                          f"{dt:.1f} s"}
    if not args.no_cpu and "linear" in legs:
        import oracle
        # the linear-CE oracle on the first rows of the linear workload: logits,
        # loss, grad_inputs rows and the full grad_weight of those rows, in fp64
        R = 1536
        log(f"cpu_baseline: fp64 linear-CE oracle on {R} rows of {lin_w.name}")
        Xs, Ws, ts = X[:R].cpu(), Wt.cpu(), tl[:R].cpu()
        t0 = time.perf_counter()
        oracle.linear_cross_entropy(Xs, Ws, ts, -100, lin_w.reduction, lin_w.z_loss)
        ldt = time.perf_counter() - t0
        lfl = 6.0 * R * lin_w.V * lin_w.D
        line.setdefault("linear_ce", {})["cpu_baseline"] = {
            "value": round(lfl / ldt / 1e12, 4), "unit": "TFLOP/s",
            "cores": torch.get_num_threads(), "kind": "oracle",
            "sample": f"first {R} of {lin_w.BT} rows of the linear-CE workload (loss, grad_inputs "
                      f"rows, grad_weight, fp64), {ldt:.1f} s"}
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
