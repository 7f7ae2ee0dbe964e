"""Benchmark: effective HBM bandwidth of the swizzled LDS transpose on one GPU.

Headline workload: fp32 4096x4096 row-major -> column-major transpose through
32x32 LDS tiles with the chosen Swizzle<B,M,S>.  One step = one call of
swz_transpose on that matrix.  Inputs are resident in HBM before timing; the
calls rotate over enough source/destination pairs (>= 512 MiB) that the
256 MB Infinity Cache cannot hold the working set, so traffic reaches HBM.

Prints ONE JSON line.  Extra fields: the other workloads and layouts
(swizzle / pad / plain), a device-to-device copy of the same bytes as the
practical ceiling, and the CPU oracle as a reported baseline.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--quick]
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "effective HBM GB/s (% of 8 TB/s) for swizzled LDS transpose; LDS conflict cycles"
HBM_PEAK_GBS = 8000.0
CACHE_DEFEAT_BYTES = 512 * 2**20  # 2x the 256 MB Infinity Cache


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def n_pairs(bytes_per_pair):
    return max(2, -(-CACHE_DEFEAT_BYTES // bytes_per_pair))


def time_steps(step, steps, warmup):
    """Run warmup steps, then time exactly `steps` steps with HIP events on
    the current stream (the stream the kernels are launched on)."""
    import torch

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record()
    for i in range(steps):
        step(warmup + i)
    end.record()
    end.synchronize()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return start.elapsed_time(end), wall


def median_rate(step, bytes_per_step, steps=50, warmup=10, batches=3):
    rates, mss = [], []
    for _ in range(batches):
        ms, _ = time_steps(step, steps, warmup)
        mss.append(ms / steps)
        rates.append(bytes_per_step * steps / (ms * 1e-3) / 1e9)
    order = sorted(range(batches), key=lambda i: rates[i])
    mid = order[batches // 2]
    return rates[mid], mss[mid]


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--quick", action="store_true", help="headline only, no other workloads")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="budget of the CPU oracle leg")
    args = ap.parse_args(argv)
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported (the path has no "
              "multi-GPU part: each GPU would run the same kernel on its own shard).", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import tiled_movement_amd as T
    import workloads as W

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    def dev_copy(a, k):
        base = torch.from_numpy(np.ascontiguousarray(a).view(np.int32 if a.itemsize == 4 else np.int16)).to(dev)
        return [base] + [base.clone() for _ in range(k - 1)]

    # ---------------------------------------------------------------- headline
    rows = cols = 4096
    a = W.fp32_matrix(rows, cols, seed=0)
    nbytes = a.nbytes
    k = n_pairs(2 * nbytes)
    srcs = dev_copy(a, k)
    dsts = [torch.empty((cols, rows), dtype=torch.int32, device=dev) for _ in range(k)]
    plan = T.swz_plan(0, rows, cols, 4, "swizzle", T.READ_AUTO)
    log(f"headline plan: {plan}, {k} buffer pairs")

    # Timed loops call the C ABI with pointers and stream resolved up front, so
    # host-side marshalling stays far below the kernel time.
    lib = T.lib
    stream = torch.cuda.current_stream(dev).cuda_stream
    sp, dp = [s.data_ptr() for s in srcs], [d.data_ptr() for d in dsts]

    def check(rc, what):
        if rc != 0:
            raise RuntimeError(f"{what}: {T.strerror(rc)}")

    def step(i):
        j = i % k
        rc = lib.swz_transpose(sp[j], dp[j], rows, cols, 4, T.LAYOUT_SWIZZLE, T.READ_AUTO, None, stream)
        if rc:
            check(rc, "swz_transpose")

    ms, wall = time_steps(step, args.steps, args.warmup)
    bytes_per_step = 2 * nbytes
    ms_per_step = ms / args.steps
    value = bytes_per_step * args.steps / (ms * 1e-3) / 1e9
    log(f"headline: {value:.1f} GB/s, {ms_per_step * 1e3:.2f} us/step, wall {wall:.3f} s")

    extra = {}
    if not args.quick:
        # Practical ceiling: device-to-device copy of the same bytes.
        def copy_step(i):
            j = i % k
            dsts[j].view(-1).copy_(srcs[j].view(-1))

        rate, msc = median_rate(copy_step, 2 * nbytes)
        extra["d2d_copy_64MiB"] = {"GBps": round(rate, 1), "us": round(msc * 1e3, 2)}
        log(f"d2d copy: {rate:.1f} GB/s")

        configs = []
        for layout in ("swizzle", "pad", "plain"):
            configs.append(("fp32_4096x4096_transpose", layout, (rows, cols), 4, T.READ_SCALAR_COL, 1))
        for layout in ("swizzle", "pad", "plain"):
            configs.append(("fp16_8192x8192_transpose", layout, (8192, 8192), 2, T.READ_B64_4X4, 1))
        for layout in ("swizzle", "pad", "plain"):
            configs.append(("bf16_64x4096x128_convert", layout, (4096, 128), 2, T.READ_B128_8X8, 64))
        inputs = {}
        for name, layout, (r, c), esz, kind, batch in configs:
            if name not in inputs:
                if name.startswith("fp32"):
                    arr = a
                elif name.startswith("fp16"):
                    arr = W.fp16_matrix(r, c, seed=0)
                else:
                    arr = W.bf16_tensor((batch, r, c), seed=0)
                kk = n_pairs(2 * arr.nbytes)
                s_ = dev_copy(arr, kk)
                d_ = [torch.empty_like(s_[0]) for _ in range(kk)]
                inputs[name] = (s_, d_, arr.nbytes)
            s_, d_, nb = inputs[name]
            kk = len(s_)

            lay = T.LAYOUTS[layout]
            sps, dps = [t.data_ptr() for t in s_], [t.data_ptr() for t in d_]

            def cstep(i, sps=sps, dps=dps, r=r, c=c, esz=esz, kind=kind, batch=batch, lay=lay, kk=kk):
                j = i % kk
                rc = lib.swz_convert_layout(sps[j], dps[j], batch, r, c, esz, lay, kind, None, stream)
                if rc:
                    check(rc, "swz_convert_layout")

            rate, msc = median_rate(cstep, 2 * nb)
            pl = T.swz_plan(0, r, c, esz, layout, kind)
            wc, rc = T.swz_predict_conflicts(kind, layout)
            extra[f"{name}/{layout}"] = {
                "GBps": round(rate, 1), "frac": round(rate / HBM_PEAK_GBS, 4), "us": round(msc * 1e3, 2),
                "params": pl["params"], "pad": pl["pad_elems"], "lds_bytes": pl["lds_bytes"],
                "predicted_conflict_cycles_per_tile": {"write": wc, "read": rc},
            }
            log(f"{name}/{layout}: {rate:.1f} GB/s")
        del inputs

        # operand staging: A then B^T, one call each per step
        ao, bo = W.bf16_operands(8192, 8192, 4096, seed=0)
        for layout in ("swizzle", "pad", "plain"):
            kk = n_pairs(2 * ao.nbytes)
            sa, sb = dev_copy(ao, kk), dev_copy(bo, kk)
            fa = [torch.empty_like(sa[0]) for _ in range(kk)]
            fb = [torch.empty_like(sb[0]) for _ in range(kk)]

            lay = T.LAYOUTS[layout]
            pa, pb = [t.data_ptr() for t in sa], [t.data_ptr() for t in sb]
            pfa, pfb = [t.data_ptr() for t in fa], [t.data_ptr() for t in fb]

            def sstep(i, lay=lay, pa=pa, pb=pb, pfa=pfa, pfb=pfb, kk=kk):
                j = i % kk
                rc = lib.swz_stage_operand(pa[j], pfa[j], 8192, 4096, 2, T.FRAG_MFMA_F32_16X16X32_BF16, lay, None,
                                           stream)
                rc |= lib.swz_stage_operand(pb[j], pfb[j], 8192, 4096, 2, T.FRAG_MFMA_F32_16X16X32_BF16, lay, None,
                                            stream)
                if rc:
                    check(rc, "swz_stage_operand")

            rate, msc = median_rate(sstep, 2 * (ao.nbytes + bo.nbytes))
            pl = T.swz_plan(1, 8192, 4096, 2, layout)
            extra[f"bf16_operand_staging_A8192x4096_B4096x8192/{layout}"] = {
                "GBps": round(rate, 1), "frac": round(rate / HBM_PEAK_GBS, 4), "us_per_A_plus_B": round(msc * 1e3, 2),
                "params": pl["params"], "pad": pl["pad_elems"],
            }
            log(f"staging/{layout}: {rate:.1f} GB/s")
            del sa, sb, fa, fb

        # swizzle map: 125 calls of 65536 offsets (launch-bound)
        x = torch.arange(65536, dtype=torch.int32, device=dev)
        y = torch.empty_like(x)
        triples = W.map_triples()

        cparams = [T.Params(*t) for t in triples]
        xp, yp = x.data_ptr(), y.data_ptr()

        def mstep(i):
            rc = lib.swz_map(xp, yp, 65536, cparams[i % len(cparams)], stream)
            if rc:
                check(rc, "swz_map")

        rate, msm = median_rate(mstep, 2 * 65536 * 4, steps=250, warmup=25)
        extra["map_65536_x125"] = {"us_per_call": round(msm * 1e3, 3), "GBps": round(rate, 1)}
        log(f"map: {msm * 1e3:.2f} us/call")

    # -------------------------------------------------------------- CPU oracle
    cpu = None
    try:
        import oracle

        got = dsts[0].cpu().numpy().view(np.uint32)
        reps, t_cpu = 0, 0.0
        ref = None
        while t_cpu < args.cpu_seconds or reps == 0:
            t1 = time.perf_counter()
            ref = oracle.transpose(a)
            t_cpu += time.perf_counter() - t1
            reps += 1
        cpu = {
            "value": round(2 * nbytes * reps / t_cpu / 1e9, 3),
            "unit": "GB/s",
            "cores": 1,
            "kind": "oracle",
            "sample": f"{reps} full 4096x4096 fp32 transposes by the oracle (NumPy strided copy, one thread), "
                      f"{t_cpu:.1f} s",
            "matches_gpu": bool(np.array_equal(ref, got)),
        }
        log(f"cpu oracle: {cpu['value']} GB/s over {reps} reps; GPU output matches: {cpu['matches_gpu']}")
    except Exception as e:  # the oracle leg is a reported baseline only
        log(f"cpu baseline skipped: {e!r}")

    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": "fp32 4096x4096 row-major -> column-major transpose, 32x32 LDS tiles, scalar column reads",
            "rows": rows, "cols": cols, "elem_bytes": 4, "layout": "swizzle",
            "swizzle_BMS": list(plan["params"]), "buffer_pairs": k,
        },
        "roofline": {
            "bound": "hbm", "achieved": round(value, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(value / HBM_PEAK_GBS, 4), "traffic": None,
        },
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
