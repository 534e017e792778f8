#!/usr/bin/env python3
"""Benchmark of the Sliding Tile Attention hot path on one MI355X.

One step = the whole forward path on one batch of the HunyuanVideo-shaped
workload: raster-order Q, K, V in, raster-order O and LSE out, in one launch of
sta_forward_raster, whose loads do the tile reorder (raster -> tile-major) and
whose stores the unreorder, on latent (30, 48, 80), tile (6, 8, 8), 24 heads,
head_dim 128, bf16, window (3, 3, 3) tiles for every head.  Inputs are seeded
synthetic N(0, 1) tensors already resident in HBM when the timed region starts.

value = counted forward FLOPs per step / step time, where counted FLOPs are
4 * L^2 * D per computed (query tile, key tile) pair (Q K^T and P V only; no
skipped pair, no softmax).  The JSON line also carries:
  roofline      the step's forward kernel, timed with events on its stream;
  cpu_baseline  the fp64 CPU oracle timed on a bounded sample of the workload;
  legs          the same step with separate reorder kernels; dense attention
                from the same library (speedup denominator); reorder bandwidth;
                the mixed-window, Wan-shaped, 2D and padded forwards; the
                backward at the fine-tuning shape, with mixed windows at
                (30,48,80) and on the padded latent; the window mass of five
                candidate windows; and a matrix-core calibration loop.
Everything runs on one GPU; --gpus above 1 is refused.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA: 256 CU x 2.4 GHz x 4096 FLOP/clk
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
FWD_SOURCES = [os.path.join(ROOT, "sparse_sliding_tile_amd", "csrc", f)
               for f in ("fwd_bf16.hip", "mfma_common.h", "sta_common.h", "kernels.h")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "sta_forward_hunyuan_30x48x80_traffic.txt")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-legs", action="store_true", help="time only the main forward step")
    p.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU oracle sample time")
    return p.parse_args()


def kh(window, n):
    out = 1
    for a, b in zip(window, n):
        out *= min(a, b)
    return out


def fwd_flops(latent, tile, windows, batch, head_dim):
    n = [-(-a // b) for a, b in zip(latent, tile)]   # tile grid (padded latents: ceil)
    L = tile[0] * tile[1] * tile[2]
    nt = n[0] * n[1] * n[2]
    return sum(batch * nt * kh(w, n) * 4 * L * L * head_dim for w in windows)


def real_token_flops(latent, tile, windows, batch, head_dim):
    """Counted forward FLOP over real tokens only: for every computed (query
    tile, key tile) pair, 4 * D * (real queries of the one) * (real keys of the
    other).  Equal to fwd_flops for a latent of whole tiles."""
    n = [-(-a // b) for a, b in zip(latent, tile)]
    ext = [[min(t_, a - i * t_) for i in range(m)] for a, t_, m in zip(latent, tile, n)]

    def start(q, w, m):
        wp = min(w, m)
        return min(max(q - wp // 2, 0), m - wp), wp
    total = 0
    for w in windows:
        # per dimension: sum over query tiles of real(q) * sum of real(k) in its window
        per_dim = []
        for d in range(3):
            acc = 0
            for qi in range(n[d]):
                s0, wp = start(qi, w[d], n[d])
                acc += ext[d][qi] * sum(ext[d][s0:s0 + wp])
            per_dim.append(acc)
        total += batch * 4 * head_dim * per_dim[0] * per_dim[1] * per_dim[2]
    return total


class Timer:
    """Events on the current stream (the stream libsta launches on)."""

    def __init__(self, torch):
        self.torch = torch
        self.pairs = []

    def __enter__(self):
        self.e0 = self.torch.cuda.Event(enable_timing=True)
        self.e1 = self.torch.cuda.Event(enable_timing=True)
        self.e0.record()
        return self

    def __exit__(self, *a):
        self.e1.record()
        self.pairs.append((self.e0, self.e1))

    def total_ms(self):
        return sum(a.elapsed_time(b) for a, b in self.pairs)

    def each_ms(self):
        return sorted(a.elapsed_time(b) for a, b in self.pairs)


def source_hash(paths=None):
    """Hash of the forward kernel's code: its source and the headers it uses,
    with comments and blank lines dropped (a comment edit is no kernel change),
    and the compiler flags of the build (without include paths, which differ
    from machine to machine)."""
    from sparse_sliding_tile_amd import build as libbuild
    h = hashlib.sha256()
    for path in paths or FWD_SOURCES:
        with open(path) as f:
            for line in f:
                code = line.split("//", 1)[0].rstrip()
                if code:
                    h.update(code.encode() + b"\n")
    fl = libbuild.FLAGS
    h.update(" ".join(f for i, f in enumerate(fl) if f != "-I" and (i == 0 or fl[i - 1] != "-I")).encode())
    return h.hexdigest()[:16]


def read_traffic():
    """HBM bytes per sta_forward launch from the committed rocprofv3 counter
    summary, and where that figure comes from; the bytes are None when the
    file is missing or the kernel's code changed since it was measured."""
    rel = os.path.relpath(TRAFFIC_FILE, ROOT)
    try:
        vals = {}
        with open(TRAFFIC_FILE) as f:
            for line in f:
                if ":" in line and not line.startswith("#"):
                    k, v = line.split(":", 1)
                    vals[k.strip()] = v.strip()
        measured, current = vals.get("source_sha256_16"), source_hash()
        if measured != current:
            return None, (f"null: {rel} was measured on kernel code {measured}, the code now hashes to "
                          f"{current}")
        return float(vals["hbm_bytes_per_launch"]), (
            f"{rel} (rocprofv3 --pmc FETCH_SIZE and WRITE_SIZE runs of this bench, scaled by a copy of known "
            f"size; kernel code hash {measured}, the code this run executes)")
    except (OSError, KeyError, ValueError):
        return None, f"null: {rel} missing or unreadable"


def cpu_baseline(x, latent, tile, window, head_dim, target_s):
    """The fp64 oracle, as it stands, on consecutive query tiles of head 0."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # threadpoolctl missing: report the machine's cores
        threads = os.cpu_count()
    n = [a // b for a, b in zip(latent, tile)]
    L = tile[0] * tile[1] * tile[2]
    q, k, v = (oracle.reorder(x[nm][:, :1].float().numpy().astype(np.float64), latent, tile)
               for nm in ("q", "k", "v"))
    done, t0 = 0, time.perf_counter()
    while True:
        rows = np.arange(done * L, (done + 1) * L)
        oracle.forward(q, k, v, latent, tile, [window], head_dim ** -0.5, rows=rows)
        done += 1
        el = time.perf_counter() - t0
        if el >= target_s or done >= n[0] * n[1] * n[2]:
            break
    flops = done * kh(window, n) * 4 * L * L * head_dim
    nt, heads = n[0] * n[1] * n[2], x["q"].shape[1]
    return {"value": round(flops / el / 1e12, 6), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "blas_threads": threads, "os_cpu_count": os.cpu_count(), "cpu_model": cpu_model(),
            "s_per_query_tile": round(el / done, 4),
            "extrapolated_s_per_launch": round(el / done * nt * heads, 1),  # x tiles x heads, extrapolated
            "sample": f"{done} query tiles ({done * L} rows) of head 0 of 24, all {L * n[0] * n[1] * n[2]} keys "
                      f"masked, fp64 numpy; {el:.1f} s; value counts the same 4*L^2*D per computed tile "
                      f"pair as the GPU figure; host CPU: {cpu_model()}"}


def cpu_model():
    """The host CPU's model string (lscpu, else /proc/cpuinfo)."""
    try:
        import subprocess
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            if line.startswith("Model name:"):
                return line.split(":", 1)[1].strip()
    except (OSError, ValueError, subprocess.SubprocessError):
        pass
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on exactly one GPU (asked for --gpus {args.gpus}, WORLD_SIZE {world}): "
              "the library has no multi-GPU path (heads are independent, so more GPUs would each take "
              "a share of the heads).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import sparse_sliding_tile_amd as sta
    from sparse_sliding_tile_amd import inputs as I

    sta.lib()
    dev = torch.device("cuda:0")
    name = "hunyuan_30x48x80_w333"
    w = I.WORKLOADS[name]
    latent, tile, wins, D, B, Hh = w["latent"], w["tile"], w["windows"], w["head_dim"], w["batch"], w["heads"]
    S = latent[0] * latent[1] * latent[2]
    log(f"[bench] generating {name} inputs")
    x = I.workload_inputs(name)
    q, k, v = (x[nm].to(dev) for nm in ("q", "k", "v"))
    qt, kt, vt, ot = (torch.empty_like(q) for _ in range(4))
    o = torch.empty_like(q)
    lse = torch.empty((B, Hh, S), dtype=torch.float32, device=dev)
    flops = fwd_flops(latent, tile, wins, B, D)
    fwd_timer = Timer(torch)

    # One step is the whole forward path on raster-order tensors in one launch:
    # the tile reorder of q, k, v and the unreorder of o happen in the kernel's
    # own loads and stores (sta_forward_raster).  The same path with separate
    # reorder kernels is timed as a leg.
    def step(timed):
        if timed:
            with fwd_timer:
                sta.forward_raster(q, k, v, latent, tile, wins, out=o, lse=lse)
        else:
            sta.forward_raster(q, k, v, latent, tile, wins, out=o, lse=lse)

    # A plain copy of known size (691,200 KiB read and written) in every run:
    # the reference the FETCH_SIZE / WRITE_SIZE counters are scaled by.
    sta.tile_reorder(q, latent, tile, out=qt)

    log(f"[bench] warmup {args.warmup}")
    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    log(f"[bench] timing {args.steps} steps")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for _ in range(args.steps):
        step(True)
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = e0.elapsed_time(e1) / args.steps
    fwd_ms = fwd_timer.total_ms() / args.steps
    log(f"[bench] step {ms_step:.3f} ms (wall {wall * 1e3 / args.steps:.3f} ms), forward kernel {fwd_ms:.3f} ms")
    achieved = flops / (fwd_ms * 1e-3) / 1e12
    each = fwd_timer.each_ms()   # per-step times of the same timed steps
    traffic, traffic_source = read_traffic()
    result = {
        "metric": "effective TFLOP/s and % bf16 MFMA peak, STA fwd at (30,48,80) latent",
        "value": round(flops / (ms_step * 1e-3) / 1e12, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": name, "latent": list(latent), "tile": list(tile), "heads": Hh,
                   "head_dim": D, "batch": B, "window": list(wins[0]),
                   "step": "sta_forward_raster: tile reorder of q,k,v and unreorder of o inside the "
                           "forward kernel's loads and stores (one launch)",
                   "pct_of_peak_step": round(100 * flops / (ms_step * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2),
                   "step_ms_median": round(each[len(each) // 2], 4), "step_ms_min": round(each[0], 4)},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 3), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic, "traffic_source": traffic_source,
                     "kernel": "sta_forward_raster (fwd_bf16_kernel, raster instance)",
                     "kernel_ms": round(fwd_ms, 4), "flops_per_launch": flops},
    }

    if not args.no_legs:
        legs = {}
        # the same step with separate reorder kernels (and the tile-major
        # tensors the dense leg uses)
        def reorder_step(t_step, t_fwd):
            with t_step:
                sta.tile_reorder(q, latent, tile, out=qt)
                sta.tile_reorder(k, latent, tile, out=kt)
                sta.tile_reorder(v, latent, tile, out=vt)
                with t_fwd:
                    sta.forward(qt, kt, vt, latent, tile, wins, out=ot, lse=lse)
                sta.tile_unreorder(ot, latent, tile, out=o)
        reorder_step(Timer(torch), Timer(torch))
        rt_step, rt_fwd = Timer(torch), Timer(torch)
        for _ in range(5):
            reorder_step(rt_step, rt_fwd)
        torch.cuda.synchronize()
        legs["step_with_reorder_kernels"] = {
            "ms": round(rt_step.total_ms() / 5, 3), "tflops": round(flops / (rt_step.total_ms() / 5) / 1e9, 1),
            "sta_forward_ms": round(rt_fwd.total_ms() / 5, 3),
            "sta_forward_tflops": round(flops / (rt_fwd.total_ms() / 5) / 1e9, 1),
            "note": "reorder q,k,v + sta_forward (tile-major) + unreorder o, five launches"}
        # dense denominator on the same tensors
        dense_t = Timer(torch)
        sta.dense_forward(qt, kt, vt, out=o, want_lse=False)
        for _ in range(2):
            with dense_t:
                sta.dense_forward(qt, kt, vt, out=o, want_lse=False)
        torch.cuda.synchronize()
        dense_ms = dense_t.total_ms() / 2
        dense_flops = B * Hh * 4 * S * S * D
        legs["dense_forward"] = {"ms": round(dense_ms, 3), "tflops": round(dense_flops / dense_ms / 1e9, 1),
                                 "speedup_sta_over_dense": round(dense_ms / fwd_ms, 2),
                                 "ideal_speedup": round(dense_flops / flops, 2)}
        # reorder bandwidth (one tensor: read + write)
        rt = Timer(torch)
        for _ in range(5):
            with rt:
                sta.tile_reorder(q, latent, tile, out=qt)
        torch.cuda.synchronize()
        r_ms = rt.total_ms() / 5
        nbytes = 2 * q.numel() * q.element_size()
        legs["tile_reorder"] = {"ms": round(r_ms, 4), "GB/s": round(nbytes / r_ms / 1e6, 1),
                                "frac_of_hbm_peak": round(nbytes / r_ms / 1e6 / PEAK_HBM_GBS, 3),
                                "tensor": list(q.shape)}
        ut = Timer(torch)
        for _ in range(5):
            with ut:
                sta.tile_unreorder(ot, latent, tile, out=o)
        torch.cuda.synchronize()
        u_ms = ut.total_ms() / 5
        legs["tile_unreorder"] = {"ms": round(u_ms, 4), "GB/s": round(nbytes / u_ms / 1e6, 1),
                                  "frac_of_hbm_peak": round(nbytes / u_ms / 1e6 / PEAK_HBM_GBS, 3),
                                  "tensor": list(q.shape)}
        # what a plain contiguous device copy of the same bytes reaches here
        # (torch's copy_): the practical ceiling for the two copies above
        ct = Timer(torch)
        for _ in range(5):
            with ct:
                qt.copy_(q)
        torch.cuda.synchronize()
        c_ms = ct.total_ms() / 5
        legs["plain_copy_reference"] = {
            "ms": round(c_ms, 4), "GB/s": round(nbytes / c_ms / 1e6, 1),
            "frac_of_hbm_peak": round(nbytes / c_ms / 1e6 / PEAK_HBM_GBS, 3),
            "reorder_over_copy_rate": round(c_ms / r_ms, 3), "unreorder_over_copy_rate": round(c_ms / u_ms, 3),
            "note": "torch's contiguous copy_ of the same tensor, same bytes read and written"}
        # (q, k, v, o, lse stay: the padded raster leg alternates with the bench step)
        del qt, kt, vt, ot
        torch.cuda.empty_cache()
        g = torch.Generator(device=dev).manual_seed(1)

        def rand(shape):
            return torch.randn(shape, generator=g, device=dev, dtype=torch.float32).to(torch.bfloat16)

        # reorder / unreorder round trip at the Wan shape (24,48,80), 40 heads:
        # each an HBM-bound copy (read + write of one tensor)
        ww = I.WORKLOADS["wan_24x48x80_w335"]
        wshape = (ww["batch"], ww["heads"], sta.raster_len(ww["latent"]), ww["head_dim"])
        xr = rand(wshape)
        xt, xb = torch.empty_like(xr), torch.empty_like(xr)
        sta.tile_reorder(xr, ww["latent"], ww["tile"], out=xt)
        sta.tile_unreorder(xt, ww["latent"], ww["tile"], out=xb)
        tr, tu, trt = Timer(torch), Timer(torch), Timer(torch)
        for _ in range(5):
            with trt:
                with tr:
                    sta.tile_reorder(xr, ww["latent"], ww["tile"], out=xt)
                with tu:
                    sta.tile_unreorder(xt, ww["latent"], ww["tile"], out=xb)
        torch.cuda.synchronize()
        wbytes = 2 * xr.numel() * xr.element_size()
        rt_ok = bool(torch.equal(xb.view(torch.int16), xr.view(torch.int16)))
        legs["wan_reorder_round_trip"] = {
            "tensor": list(wshape), "bytes_per_copy": wbytes,
            "reorder_ms": round(tr.total_ms() / 5, 4), "reorder_GB/s": round(wbytes / (tr.total_ms() / 5) / 1e6, 1),
            "unreorder_ms": round(tu.total_ms() / 5, 4),
            "unreorder_GB/s": round(wbytes / (tu.total_ms() / 5) / 1e6, 1),
            "round_trip_ms": round(trt.total_ms() / 5, 4),
            "round_trip_GB/s": round(2 * wbytes / (trt.total_ms() / 5) / 1e6, 1),
            "frac_of_hbm_peak": round(2 * wbytes / (trt.total_ms() / 5) / 1e6 / PEAK_HBM_GBS, 3),
            "round_trip_bit_exact": rt_ok}
        del xr, xt, xb

        for lname in ("hunyuan_30x48x80_mixed", "wan_24x48x80_w335", "image_2d_1x128x128_w155",
                      "hunyuan_29x45x76_w333_padded"):
            lw = I.WORKLOADS[lname]
            lS = sta.tile_major_len(lw["latent"], lw["tile"])
            shape = (lw["batch"], lw["heads"], lS, lw["head_dim"])
            a, b_, c = rand(shape), rand(shape), rand(shape)
            out = torch.empty_like(a)
            ll = torch.empty(shape[:3], dtype=torch.float32, device=dev)
            t = Timer(torch)
            sta.forward(a, b_, c, lw["latent"], lw["tile"], lw["windows"], out=out, lse=ll)
            for _ in range(5):
                with t:
                    sta.forward(a, b_, c, lw["latent"], lw["tile"], lw["windows"], out=out, lse=ll)
            torch.cuda.synchronize()
            lms = t.total_ms() / 5
            lf = fwd_flops(lw["latent"], lw["tile"], lw["windows"], lw["batch"], lw["head_dim"])
            legs[lname] = {"ms": round(lms, 3), "tflops": round(lf / lms / 1e9, 1),
                           "pct_of_peak": round(100 * lf / lms / 1e9 / PEAK_BF16_TFLOPS, 2)}
            if lname.endswith("padded"):
                rf = real_token_flops(lw["latent"], lw["tile"], lw["windows"], lw["batch"], lw["head_dim"])
                legs[lname].update({"counted": "tflops over the padded tile grid", "real_token_tflops":
                                    round(rf / lms / 1e9, 1), "real_token_pct_of_peak":
                                    round(100 * rf / lms / 1e9 / PEAK_BF16_TFLOPS, 2),
                                    "real_token_share_of_counted": round(rf / lf, 4)})
                # the padded step in one launch on raster tensors of the real
                # tokens (no reorder kernels), against the whole-tile step
                rshape = (lw["batch"], lw["heads"], sta.raster_len(lw["latent"]), lw["head_dim"])
                ra, rb, rc = rand(rshape), rand(rshape), rand(rshape)
                rout = torch.empty_like(ra)
                rl = torch.empty(rshape[:3], dtype=torch.float32, device=dev)
                sta.forward_raster(ra, rb, rc, lw["latent"], lw["tile"], lw["windows"], out=rout, lse=rl)
                # alternated with the whole-tile bench step, so that both see
                # the same clocks (a later leg can run at a lower clock than
                # the timed steps at the start)
                rtm, wtm = Timer(torch), Timer(torch)
                for _ in range(10):
                    with rtm:
                        sta.forward_raster(ra, rb, rc, lw["latent"], lw["tile"], lw["windows"], out=rout, lse=rl)
                    with wtm:
                        sta.forward_raster(q, k, v, latent, tile, wins, out=o, lse=lse)
                torch.cuda.synchronize()
                # medians of the per-call times: one slow stretch of the run
                # does not move them
                rms, wms = rtm.each_ms()[5], wtm.each_ms()[5]
                legs[lname + "_raster_step"] = {
                    "ms": round(rms, 3), "tflops": round(lf / rms / 1e9, 1),
                    "pct_of_peak": round(100 * lf / rms / 1e9 / PEAK_BF16_TFLOPS, 2),
                    "real_token_pct_of_peak": round(100 * rf / rms / 1e9 / PEAK_BF16_TFLOPS, 2),
                    "whole_tile_step_ms_alternated": round(wms, 3),
                    "over_whole_tile_step": round(rms / wms, 4),
                    "over_timed_bench_step": round(rms / ms_step, 4),
                    "ms_mean": round(rtm.total_ms() / 10, 3),
                    "note": "sta_forward_raster, one launch, raster tensors of the real tokens; median of "
                            "10 calls; over_whole_tile_step = this time / the (30,48,80) bench step timed "
                            "in alternation with it (median of 10)"}
                del ra, rb, rc, rout, rl
            if lname.endswith("mixed"):
                legs[lname]["windows"] = [list(x_) for x_ in lw["windows"]]
            del a, b_, c, out, ll
        # backward at the fine-tuning shape, at the HunyuanVideo shape with the
        # mixed per-head windows, and on the padded latent (29,45,76)
        for bname, iters in (("finetune_24x64x64_w355", 3), ("hunyuan_30x48x80_mixed", 2),
                             ("hunyuan_29x45x76_w333_padded", 2)):
            fw = I.WORKLOADS[bname]
            fS = sta.tile_major_len(fw["latent"], fw["tile"])
            shape = (fw["batch"], fw["heads"], fS, fw["head_dim"])
            a, b_, c, do = rand(shape), rand(shape), rand(shape), rand(shape)
            out, ll = sta.forward(a, b_, c, fw["latent"], fw["tile"], fw["windows"])
            ws = torch.empty(sta.backward_workspace_bytes(shape[0], shape[1], shape[3], fw["latent"], fw["tile"]),
                             dtype=torch.uint8, device=dev)
            t = Timer(torch)
            sta.backward(a, b_, c, out, do, ll, fw["latent"], fw["tile"], fw["windows"], workspace=ws)
            for _ in range(iters):
                with t:
                    sta.backward(a, b_, c, out, do, ll, fw["latent"], fw["tile"], fw["windows"], workspace=ws)
            torch.cuda.synchronize()
            bms = t.total_ms() / iters
            bflops = fwd_flops(fw["latent"], fw["tile"], fw["windows"], fw["batch"], fw["head_dim"]) * 10 // 4
            legs[bname + "_backward"] = {
                "ms": round(bms, 3), "tflops": round(bflops / bms / 1e9, 1),
                "pct_of_peak": round(100 * bflops / bms / 1e9 / PEAK_BF16_TFLOPS, 2),
                "real_token_pct_of_peak": round(
                    100 * real_token_flops(fw["latent"], fw["tile"], fw["windows"], fw["batch"], fw["head_dim"])
                    * 10 // 4 / bms / 1e9 / PEAK_BF16_TFLOPS, 2),
                "counted": "10*L^2*D per tile pair (5 GEMMs, padded grid for a padded latent); the kernels run 8 (dQ, dV and dK passes)"}
            del a, b_, c, do, out, ll, ws
        # window search, measurement side: attention mass of the five
        # candidate windows of the mixed-window workload, all 24 heads
        sw = I.WORKLOADS["hunyuan_30x48x80_w333"]
        sS = sta.tile_major_len(sw["latent"], sw["tile"])
        shape = (sw["batch"], sw["heads"], sS, sw["head_dim"])
        a, b_ = rand(shape), rand(shape)
        cands = [(5, 6, 10), (3, 3, 3), (3, 3, 5), (5, 3, 3), (1, 6, 10)]
        ws = torch.empty(sta.window_mass_workspace_bytes(shape[0], shape[1], sw["latent"], sw["tile"], len(cands)),
                         dtype=torch.uint8, device=dev)
        mass = sta.window_mass(a, b_, sw["latent"], sw["tile"], cands, workspace=ws)
        t = Timer(torch)
        for _ in range(2):
            with t:
                sta.window_mass(a, b_, sw["latent"], sw["tile"], cands, workspace=ws, out=mass)
        torch.cuda.synchronize()
        sms = t.total_ms() / 2
        # counted: Q K^T (2*L^2*D per tile pair) over the full window, the one
        # pass every candidate's share is read from
        sflops = fwd_flops(sw["latent"], sw["tile"], [(5, 6, 10)] * shape[1], shape[0], shape[3]) // 2
        legs["window_mass_5_candidates"] = {
            "ms": round(sms, 3), "tflops": round(sflops / sms / 1e9, 1),
            "pct_of_peak": round(100 * sflops / sms / 1e9 / PEAK_BF16_TFLOPS, 2),
            "mean_mass": [round(float(x_), 4) for x_ in mass.mean(dim=(1, 2)).tolist()],
            "counted": "2*L^2*D per tile pair (Q K^T) over the full window (one pass for all candidates)"}
        del a, b_, ws, mass
        # the matrix cores alone on N(0, 1) bf16 operands and on zeros: the rate
        # the power limit leaves on data like the inputs, next to the nominal peak
        from sparse_sliding_tile_amd import calib
        ceil = {}
        for kind in ("randn", "zeros"):
            ops = rand((1 << 19,)) if kind == "randn" else torch.zeros(1 << 19, dtype=torch.bfloat16, device=dev)
            cout, cfl = calib.calib_mfma_bf16(ops, 20000, 512)
            for _ in range(60):
                calib.calib_mfma_bf16(ops, 20000, 512, out=cout)
            t = Timer(torch)
            for _ in range(40):
                with t:
                    calib.calib_mfma_bf16(ops, 20000, 512, out=cout)
            torch.cuda.synchronize()
            ceil[kind] = cfl / (t.total_ms() / 40) / 1e9
            del ops, cout
        legs["mfma_calibration"] = {
            "tflops_randn_operands": round(ceil["randn"], 1), "tflops_zero_operands": round(ceil["zeros"], 1),
            "sta_forward_frac_of_randn_rate": round(achieved / ceil["randn"], 3),
            "note": "bf16 32x32x16 MFMA loop, 2 waves per SIMD, no memory traffic"}
        result["legs"] = legs

    # The CPU oracle runs last: its many host threads would otherwise still be
    # busy while the legs submit their GPU work.
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline")
        result["cpu_baseline"] = cpu_baseline(x, latent, tile, wins[0], D, args.cpu_seconds)
    else:
        result["cpu_baseline"] = None

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
