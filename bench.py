"""Benchmark: effective HBM bandwidth of the swizzled LDS transpose on one GPU.

Headline workload: fp32 4096x4096 row-major -> column-major transpose through
32x32 LDS tiles with the chosen Swizzle<B,M,S>.  One step = one call of
swz_transpose on that matrix (one kernel launch).  Inputs are resident in HBM
before timing; the calls rotate over enough source/destination pairs
(>= 512 MiB) that the 256 MB Infinity Cache cannot hold the working set, so
traffic reaches HBM.

Prints ONE JSON line.  Extra fields: the other workloads and layouts
(swizzle / pad / plain / direct), the library's reference copy of the same
bytes (the practical read-once / write-once ceiling; it copies the
workloads' own random bytes, since an all-zero buffer copies about 4%
faster), the runtime's own device copy, the LDS bank-conflict counters of
the kernels (from a record taken with rocprofv3 on the current kernel
sources), and the CPU oracle timed on every workload as a reported
baseline, each checked bit for bit against the GPU result.

Usage:
  python bench.py [--gpus 1] [--steps K] [--warmup W] [--quick]
  python bench.py --workload NAME --layout swizzle|pad|plain|direct [--steps K] [--pairs P]
      time one workload only (used for profiler runs), optionally rotating over
      exactly P buffer pairs; NAME is one of
      fp32_transpose, fp16_transpose, fp16_transpose_tr, u8_transpose, bf16_convert,
      bf16_stage, fp32_narrow8, fp16_narrow8, u8_narrow16, fp32_transpose_long, map, map_batch, copy,
      copy_128, copy_zero, memcpy_d2d,
      bf16_gemm, bf16_gemm_fused, bf16_gemm_fused_bf16c, torch_mm_bf16
  python bench.py --tile-orders [--elem-bytes 4 2] [--mib 64]
      time every tile order of the transposes on matrices of one size and
      several shapes, and what swz_tune_tile_order picks for each (a table on
      stdout instead of the JSON line)
  python bench.py --order-shapes [--elem-bytes 4 2]
      every tile order and the shape's default order on matrices of 32 to
      512 MiB with sides from 39 values between 1,024 and 16,384, as shares
      of a copy (a table)

Timing: warm-up steps, then a short spin kernel on the launch stream before
the start event, so the host has queued the first launches by the time the
timed region starts (without it the first steps of a short run wait for the
host); the region between the two HIP events holds exactly the timed steps.
"""

from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "effective HBM GB/s (% of 8 TB/s) for swizzled LDS transpose; LDS conflict cycles"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 matrix peak
CACHE_DEFEAT_BYTES = 512 * 2**20  # 2x the 256 MB Infinity Cache

WORKLOADS = {
    "fp32_transpose": "fp32 4096x4096 row-major -> column-major transpose, 32x32 LDS tiles, 4-byte column reads",
    "fp32_transpose_long": "fp32 8192x2048 -> 2048x8192 transpose (64 MiB, 32 KiB output rows), default tile order",
    "fp16_transpose": "fp16 8192x8192 row-major -> column-major transpose, 64x64 LDS tiles, 8-byte reads of 4x4 blocks",
    "fp16_transpose_tr": "fp16 8192x8192 row-major -> column-major transpose, 64x64 LDS tiles, gfx950 8-byte transpose reads",
    "bf16_convert": "bf16 [64,4096,128] -> [64,128,4096] layout conversion, 64x128 LDS tiles, 16-byte reads of 8x8 blocks",
    "u8_transpose": "1-byte (int8 / fp8 bits) 8192x8192 row-major -> column-major transpose, 128x128 LDS tiles, gfx950 8-bit transpose reads",
    "fp32_narrow8": "fp32 [2097152][8] -> [8][2097152] transpose (64 MiB), whole-row 128x8 LDS tiles, the swizzle spanning rows",
    "fp16_narrow8": "fp16 [4194304][8] -> [8][4194304] transpose (64 MiB), whole-row 256x8 LDS tiles, 2-byte column reads",
    "u8_narrow16": "1-byte [4194304][16] -> [16][4194304] transpose (64 MiB), whole-row 1024x16 LDS tiles, 4-byte reads of 16x4 blocks",
    "fp32_rows3": "fp32 [5592405][3] -> [3][5592405] transpose (64 MiB, output rows off the 64-byte lines), flat whole-row tiles of 1344 rows",
    "u8_rows48": "1-byte [1398101][48] -> [48][1398101] transpose (64 MiB, output rows off the 64-byte lines), flat whole-row tiles of 256 rows, word swizzle, runs shifted onto the output lines",
    "bf16_stage": "bf16 operand staging A[8192x4096] row-major + B[4096x8192] column-major into 16x16x32 fragments, both in one launch",
    "map": "Swizzle<B,M,S> of int32 offsets 0..65535, one call per (B,M,S), 125 triples",
    "map_batch": "Swizzle<B,M,S> of int32 offsets 0..65535 under all 125 triples in one call (8,192,000 outputs)",
    "bf16_gemm": "C[8192x8192] fp32 = A * B^T from the staged fragments of A[8192x4096] and B[4096x8192] (16x16x32 bf16 MFMA)",
    "bf16_gemm_fused": "C[8192x8192] fp32 = A * B^T, A[8192x4096] row-major and B[4096x8192] column-major staged through swizzled 256x64 LDS tiles inside the GEMM (16x16x32 bf16 MFMA)",
    "bf16_gemm_fused_bf16c": "the same fused GEMM with C written as bf16 (rounded to nearest even), like the runtime library GEMM below",
    "torch_mm_bf16": "runtime library GEMM (torch.mm, bf16 in and out) of the same 8192x8192x4096 product, for context",
    "copy": "reference 16-byte vector copy of 64 MiB (read once, write once) of the fp32 workload's random input",
    "copy_128": "reference 16-byte vector copy of 128 MiB (the byte count of the 256 MiB workloads) of the fp16 workload's random input",
    "copy_zero": "the same copy of 64 MiB of zeros (for context: zeros copy faster)",
    "memcpy_d2d": "runtime device-to-device copy (hipMemcpyAsync through torch) of 64 MiB, for context",
}


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")
CONFLICT_FILE = os.path.join(ROOT, "profiles", "lds_conflicts.json")
KERNEL_SOURCES = ("kernels_tile.hip", "kernels_copy.hip", "swz_common.h", "kernels_rows.hip")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def code_text(src):
    """C++ source without its comments, trailing blanks and empty lines: what
    the compiler sees, up to layout.  (The kernel sources hold no string
    literal with a comment marker in it.)"""
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    src = re.sub(r"//[^\n]*", "", src)
    return "\n".join(ln.rstrip() for ln in src.splitlines() if ln.strip())


def kernel_sources_digest():
    """sha256 of the code of the kernel sources (comments aside) that the
    counter records (TRAFFIC_FILE, CONFLICT_FILE) were taken on."""
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "tiled_movement_amd", "csrc", name), encoding="utf-8") as f:
            h.update(code_text(f.read()).encode())
    return h.hexdigest()


def measured_traffic(name):
    """HBM bytes per launch from rocprofv3 FETCH_SIZE / WRITE_SIZE runs, each
    scaled by the same counter's reading for the reference copy; None when
    no such record exists or the kernels changed since it was taken."""
    data = _current_record(TRAFFIC_FILE)
    if data is None:
        return None
    rec = data.get("workloads", {}).get(name)
    return None if rec is None else rec.get("bytes_per_launch")


def _current_record(path):
    """The record in `path` if it was taken on the kernel sources as they are
    now (same digest), else None."""
    try:
        with open(path) as f:
            data = json.load(f)
    except (OSError, ValueError):
        return None
    return data if data.get("kernel_sources_sha256") == kernel_sources_digest() else None


def measured_conflicts(name):
    """LDS bank-conflict counters per layout of one workload, from rocprofv3
    runs (SQ_LDS_BANK_CONFLICT, SQ_LDS_IDX_ACTIVE, SQ_INSTS_LDS per dispatch),
    as conflict cycles per tile and per LDS instruction; None when no record
    exists for the workload or the kernels changed since it was taken."""
    data = _current_record(CONFLICT_FILE)
    rec = None if data is None else data.get("workloads", {}).get(name)
    if not rec:
        return None
    out = {}
    for layout, r in rec.items():
        out[layout] = {"conflict_cycles_per_tile": r["conflict_cycles_per_tile"],
                       "conflict_cycles_per_lds_instr": r["conflict_cycles_per_lds_instr"],
                       "SQ_LDS_BANK_CONFLICT": r["SQ_LDS_BANK_CONFLICT"],
                       "SQ_LDS_IDX_ACTIVE": r["SQ_LDS_IDX_ACTIVE"], "SQ_INSTS_LDS": r["SQ_INSTS_LDS"]}
    return out


PAIRS_OVERRIDE = None  # --pairs: rotate over exactly this many buffer pairs


def n_pairs(bytes_per_pair):
    if PAIRS_OVERRIDE:
        return PAIRS_OVERRIDE
    return max(2, -(-CACHE_DEFEAT_BYTES // bytes_per_pair))


PREFILL_CYCLES = 1_000_000  # spin before the start event: about 0.5 ms at the shader clock


def time_steps(step, steps, warmup):
    """Run warmup steps, then time exactly `steps` steps with HIP events on
    the current stream (the stream the kernels are launched on).  A spin
    kernel ahead of the start event keeps the GPU busy while the host queues
    the first steps, so the timed region is the steps' own run time."""
    import torch

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    torch.cuda._sleep(PREFILL_CYCLES)
    start.record()
    for i in range(steps):
        step(warmup + i)
    end.record()
    end.synchronize()
    torch.cuda.synchronize()
    return start.elapsed_time(end), time.perf_counter() - t0


def median_rate(step, bytes_per_step, steps=50, warmup=10, batches=5):
    rates, mss = [], []
    for _ in range(batches):
        ms, _ = time_steps(step, steps, warmup)
        mss.append(ms / steps)
        rates.append(bytes_per_step * steps / (ms * 1e-3) / 1e9)
    mid = sorted(range(batches), key=lambda i: rates[i])[batches // 2]
    return rates[mid], mss[mid]


class Ctx:
    """Device, stream and helpers shared by the workload builders."""

    def __init__(self):
        import numpy as np
        import torch

        import tiled_movement_amd as T

        self.np, self.torch, self.T = np, torch, T
        self.dev = torch.device("cuda:0")
        torch.cuda.set_device(self.dev)
        self.lib = T.lib
        self.stream = torch.cuda.current_stream(self.dev).cuda_stream

    def copies(self, a, k):
        np, torch = self.np, self.torch
        base = torch.from_numpy(np.ascontiguousarray(a).view({4: np.int32, 2: np.int16, 1: np.uint8}[a.itemsize])).to(self.dev)
        return [base] + [base.clone() for _ in range(k - 1)]

    def check(self, rc, what):
        if rc != 0:
            raise RuntimeError(f"{what}: {self.T.strerror(rc)}")


def build(ctx, name, layout):
    """Return (step, bytes_per_step, info) for one workload.  Timed steps call
    the C ABI with pointers and stream resolved up front, so host-side
    marshalling stays far below the kernel time."""
    import workloads as W

    T, lib, stream = ctx.T, ctx.lib, ctx.stream
    lay = T.LAYOUTS[layout]
    info = {"workload": WORKLOADS[name], "layout": layout}

    if name in ("fp32_transpose", "fp16_transpose", "fp16_transpose_tr", "bf16_convert", "u8_transpose", "fp32_narrow8",
                "fp16_narrow8", "u8_narrow16", "fp32_transpose_long", "fp32_rows3", "u8_rows48"):
        if name == "fp32_rows3":
            r = (64 << 20) // 12
            a, esz, kind, (batch, r, c) = W.fp32_matrix(r, 3, seed=0), 4, T.READ_ROWS, (1, r, 3)
        elif name == "u8_rows48":
            r = (64 << 20) // 48
            a, esz, kind, (batch, r, c) = W.u8_matrix(r, 48, seed=0), 1, T.READ_ROWS, (1, r, 48)
        elif name == "fp32_narrow8":
            a, esz, kind, (batch, r, c) = W.fp32_matrix(1 << 21, 8, seed=0), 4, T.READ_NARROW8, (1, 1 << 21, 8)
        elif name == "fp16_narrow8":
            a, esz, kind, (batch, r, c) = W.fp16_matrix(1 << 22, 8, seed=0), 2, T.READ_HNARROW8, (1, 1 << 22, 8)
        elif name == "u8_narrow16":
            a, esz, kind, (batch, r, c) = W.u8_matrix(1 << 22, 16, seed=0), 1, T.READ_BNARROW16, (1, 1 << 22, 16)
        elif name == "fp32_transpose":
            a, esz, kind, (batch, r, c) = W.fp32_matrix(4096, 4096, seed=0), 4, T.READ_SCALAR_COL, (1, 4096, 4096)
        elif name == "fp32_transpose_long":
            a, esz, kind, (batch, r, c) = W.fp32_matrix(8192, 2048, seed=0), 4, T.READ_SCALAR_COL, (1, 8192, 2048)
        elif name == "fp16_transpose":
            a, esz, kind, (batch, r, c) = W.fp16_matrix(8192, 8192, seed=0), 2, T.READ_B64_4X4, (1, 8192, 8192)
        elif name == "fp16_transpose_tr":
            a, esz, kind, (batch, r, c) = W.fp16_matrix(8192, 8192, seed=0), 2, T.READ_B64_TR16, (1, 8192, 8192)
        elif name == "u8_transpose":
            a, esz, kind, (batch, r, c) = W.u8_matrix(8192, 8192, seed=0), 1, T.READ_B64_TR8, (1, 8192, 8192)
        else:
            a, esz, kind, (batch, r, c) = W.bf16_tensor((64, 4096, 128), seed=0), 2, T.READ_B128_8X8, (64, 4096, 128)
        k = n_pairs(2 * a.nbytes)
        srcs = ctx.copies(a, k)
        dsts = [ctx.torch.empty_like(srcs[0]) for _ in range(k)]
        sp, dp = [t.data_ptr() for t in srcs], [t.data_ptr() for t in dsts]

        def step(i):
            j = i % k
            rc = lib.swz_convert_layout(sp[j], dp[j], batch, r, c, esz, lay, kind, None, stream)
            if rc:
                ctx.check(rc, "swz_convert_layout")

        pl = T.swz_plan(0, r, c, esz, layout, kind)
        info.update({"shape": [batch, r, c], "elem_bytes": esz, "params": list(pl["params"]),
                     "pad_elems": pl["pad_elems"], "lds_bytes": pl["lds_bytes"], "threads": pl["threads"],
                     "buffer_pairs": k})
        if kind != T.READ_ROWS:  # the flat-row kind's reads depend on the width, not on the kind alone
            wc, rc_ = T.swz_predict_conflicts(kind, layout)
            info["predicted_conflict_cycles_per_tile"] = {"write": wc, "read": rc_}
        info["_io"] = (a, srcs, dsts, step)
        return step, 2 * a.nbytes, info

    if name == "bf16_stage":
        ao, bo = W.bf16_operands(8192, 8192, 4096, seed=0)
        k = n_pairs(2 * (ao.nbytes + bo.nbytes))
        sa, sb = ctx.copies(ao, k), ctx.copies(bo, k)
        fa = [ctx.torch.empty_like(sa[0]) for _ in range(k)]
        fb = [ctx.torch.empty_like(sb[0]) for _ in range(k)]
        pa, pb = [t.data_ptr() for t in sa], [t.data_ptr() for t in sb]
        pfa, pfb = [t.data_ptr() for t in fa], [t.data_ptr() for t in fb]
        frag = T.FRAG_MFMA_F32_16X16X32_BF16

        def step(i):  # both operands in one launch
            j = i % k
            rc = lib.swz_stage_operands(pa[j], pfa[j], 8192, pb[j], pfb[j], 8192, 4096, 2, frag, lay, None, stream)
            if rc:
                ctx.check(rc, "swz_stage_operands")

        pl = T.swz_plan(1, 8192, 4096, 2, layout)
        wc, rc_ = T.swz_predict_conflicts(T.READ_MFMA_16X16X32, layout)
        info.update({"params": list(pl["params"]), "pad_elems": pl["pad_elems"], "lds_bytes": pl["lds_bytes"],
                     "threads": pl["threads"], "buffer_pairs": k, "launches_per_step": 1,
                     "predicted_conflict_cycles_per_tile": {"write": wc, "read": rc_}})
        info["_keep"] = (sa, sb, fa, fb)
        info["_io"] = (ao, bo, fa[0], fb[0], step)
        return step, 2 * (ao.nbytes + bo.nbytes), info

    if name == "bf16_gemm":
        m = n = 8192
        k = 4096
        ao, bo = W.bf16_operands(m, n, k, seed=0)
        fa = ctx.torch.empty(ao.size, dtype=ctx.torch.int16, device=ctx.dev)
        fb = ctx.torch.empty(bo.size, dtype=ctx.torch.int16, device=ctx.dev)
        T.swz_stage_operand(ctx.copies(ao, 1)[0], fa, m, k)
        T.swz_stage_operand(ctx.copies(bo, 1)[0], fb, n, k)
        c = ctx.torch.empty((m, n), dtype=ctx.torch.float32, device=ctx.dev)
        pfa, pfb, pc = fa.data_ptr(), fb.data_ptr(), c.data_ptr()
        frag = T.FRAG_MFMA_F32_16X16X32_BF16

        def step(i):
            rc = lib.swz_gemm_frag(pfa, pfb, pc, m, n, k, frag, stream)
            if rc:
                ctx.check(rc, "swz_gemm_frag")

        info.update({"m": m, "n": n, "k": k, "flops_per_step": 2 * m * n * k, "unit_of_value": "TFLOP/s"})
        info["_keep"] = (fa, fb, c)
        return step, 2 * m * n * k, info

    if name in ("bf16_gemm_fused", "bf16_gemm_fused_bf16c"):
        m = n = 8192
        k = 4096
        ao, bo = W.bf16_operands(m, n, k, seed=0)
        a, bt = ctx.copies(ao, 1)[0], ctx.copies(bo, 1)[0]
        bf16c = name == "bf16_gemm_fused_bf16c"
        c = ctx.torch.empty((m, n), dtype=ctx.torch.int16 if bf16c else ctx.torch.float32, device=ctx.dev)
        pa, pb, pc = a.data_ptr(), bt.data_ptr(), c.data_ptr()
        ctype = T.C_BF16 if bf16c else T.C_F32

        def step(i):
            rc = lib.swz_gemm_ex(pa, pb, pc, m, n, k, lay, None, ctype, stream)
            if rc:
                ctx.check(rc, "swz_gemm_ex")

        pl = T.swz_plan(1, m, k, 2, "direct" if layout == "swizzle" else layout)
        info.update({"m": m, "n": n, "k": k, "flops_per_step": 2 * m * n * k, "unit_of_value": "TFLOP/s",
                     "params": list(pl["params"])})
        info["_keep"] = (a, bt, c)
        return step, 2 * m * n * k, info

    if name == "torch_mm_bf16":
        m = n = 8192
        k = 4096
        ao, bo = W.bf16_operands(m, n, k, seed=0)
        a = ctx.copies(ao, 1)[0].view(ctx.torch.bfloat16)
        b = ctx.copies(bo, 1)[0].view(ctx.torch.bfloat16).t().contiguous()  # B [k][n]
        out = ctx.torch.empty((m, n), dtype=ctx.torch.bfloat16, device=ctx.dev)

        def step(i):
            ctx.torch.mm(a, b, out=out)

        info.update({"m": m, "n": n, "k": k})
        info["_keep"] = (a, b, out)
        return step, 2 * m * n * k, info

    if name == "map":
        x = ctx.torch.arange(65536, dtype=ctx.torch.int32, device=ctx.dev)
        y = ctx.torch.empty_like(x)
        cparams = [T.Params(*t) for t in W.map_triples()]
        xp, yp = x.data_ptr(), y.data_ptr()

        def step(i):
            rc = lib.swz_map(xp, yp, 65536, cparams[i % len(cparams)], stream)
            if rc:
                ctx.check(rc, "swz_map")

        info["_keep"] = (x, y)
        return step, 2 * 65536 * 4, info

    if name == "map_batch":
        triples = W.map_triples()
        x = ctx.torch.arange(65536, dtype=ctx.torch.int32, device=ctx.dev)
        k = n_pairs(4 * 65536 * len(triples))
        ys = [ctx.torch.empty((len(triples), 65536), dtype=ctx.torch.int32, device=ctx.dev) for _ in range(k)]
        arr = (T.Params * len(triples))(*[T.Params(*t) for t in triples])
        xp, yps = x.data_ptr(), [y.data_ptr() for y in ys]

        def step(i):
            rc = lib.swz_map_batch(xp, yps[i % k], 65536, ctypes.addressof(arr), len(triples), stream)
            if rc:
                ctx.check(rc, "swz_map_batch")

        info["_keep"] = (x, ys, arr)
        info["_io"] = (W.map_offsets(65536), triples, ys[0], step)
        info["buffer_pairs"] = k
        # bytes: one read of the offsets per triple (from cache) is not HBM
        # traffic; the algorithmic bytes are the input once and every output
        return step, 4 * 65536 * (1 + len(triples)), info

    if name in ("copy", "copy_128", "copy_zero", "memcpy_d2d"):
        # the workloads' own input bytes (64 MiB: the fp32 matrix, 128 MiB:
        # the fp16 one); copy_zero copies zeros
        nbytes = (128 if name == "copy_128" else 64) * 2**20
        k = n_pairs(2 * nbytes)
        if name == "copy_zero":
            srcs = [ctx.torch.zeros(nbytes // 4, dtype=ctx.torch.int32, device=ctx.dev) for _ in range(k)]
        else:
            a = W.fp16_matrix(8192, 8192, seed=0) if name == "copy_128" else W.fp32_matrix(4096, 4096, seed=0)
            srcs = [t.view(-1) for t in ctx.copies(a, k)]
        dsts = [ctx.torch.empty_like(s) for s in srcs]
        sp, dp = [t.data_ptr() for t in srcs], [t.data_ptr() for t in dsts]

        def step(i):
            j = i % k
            if name == "memcpy_d2d":
                dsts[j].copy_(srcs[j])
                return
            rc = lib.swz_copy(sp[j], dp[j], nbytes, stream)
            if rc:
                ctx.check(rc, "swz_copy")

        info["_keep"] = (srcs, dsts)
        info["buffer_pairs"] = k
        return step, 2 * nbytes, info

    raise ValueError(name)


def host_cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def _oracle_legs(name, info):
    """For one workload: the plain C oracle (threads -> result), the NumPy
    oracle (-> result), the GPU's result of step 0 on the host, the
    algorithmic bytes of one oracle pass, and what one pass is."""
    import numpy as np
    import torch

    import oracle
    from oracle import c_ref

    if name == "map_batch":
        x, triples, y_dev, step = info["_io"]
        step(0)
        torch.cuda.synchronize()
        got = y_dev.cpu().numpy()

        def c_leg(threads):
            from concurrent.futures import ThreadPoolExecutor  # ctypes calls release the GIL
            with ThreadPoolExecutor(threads) as pool:
                return np.stack(list(pool.map(lambda p: c_ref.swizzle_map(x, *p), triples)))

        def np_leg():
            return np.stack([oracle.swizzle_map(x, *p) for p in triples])

        return c_leg, np_leg, got, 4 * x.size * (1 + len(triples)), f"the {len(triples)} triples over {x.size} offsets"
    if name == "bf16_stage":
        ao, bo, fa, fb, step = info["_io"]
        step(0)
        torch.cuda.synchronize()
        got = np.concatenate([fa.cpu().numpy().view(np.uint16).ravel(), fb.cpu().numpy().view(np.uint16).ravel()])

        def c_leg(threads):
            return np.concatenate([c_ref.stage_operand(ao, threads).ravel(), c_ref.stage_operand(bo, threads).ravel()])

        def np_leg():
            return np.concatenate([oracle.stage_operand(ao).ravel(), oracle.stage_operand(bo).ravel()])

        return c_leg, np_leg, got, 2 * (ao.nbytes + bo.nbytes), "A and B staged into fragments"
    a, srcs, dsts, step = info["_io"]
    step(0)  # buffer pair 0 holds the result again
    torch.cuda.synchronize()
    got = dsts[0].cpu().numpy().view(a.dtype).reshape(-1)
    return (lambda threads: c_ref.convert_layout(a, threads).reshape(-1),
            lambda: (oracle.transpose(a) if a.ndim == 2 else oracle.convert_layout(a)).reshape(-1),
            got, 2 * a.nbytes, "x".join(str(d) for d in a.shape) + " transposed")


def cpu_baseline(name, info, seconds):
    """The oracle on the host cores, bounded to about `seconds` in all: the
    plain C oracle with one thread per host core (at most 16, the machine's CPU
    share), then with one thread, then the NumPy oracle; rates in GB/s of the
    same algorithmic bytes as the GPU figure; the GPU's result checked bit
    for bit against both oracles."""
    import numpy as np

    from oracle import c_ref

    c_leg, np_leg, got, nbytes, what = _oracle_legs(name, info)
    threads = max(1, min(16, os.cpu_count() or 1))

    def rate(fn, budget):
        reps, t, out = 0, 0.0, None
        while t < budget or reps == 0:
            t1 = time.perf_counter()
            out = fn()
            t += time.perf_counter() - t1
            reps += 1
        return nbytes * reps / t / 1e9, reps, t, out

    c_ref.lib()  # compile outside the timed loop
    v_n, reps_n, t_n, ref = rate(lambda: c_leg(threads), 0.5 * seconds)
    v_1, _, _, _ = rate(lambda: c_leg(1), 0.25 * seconds)
    v_np, _, _, ref_np = rate(np_leg, 0.25 * seconds)
    same = lambda r: r.shape == got.shape and bool(np.array_equal(r.view(got.dtype), got))
    return {
        "value": round(v_n, 3),
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"{reps_n} full passes ({what}) by the plain C oracle (scalar loops, gcc -O2, "
                  f"{threads} threads), {t_n:.1f} s",
        "single_thread_GBps": round(v_1, 3),
        "numpy_oracle_GBps": round(v_np, 3),
        "cpu_model": host_cpu_model(),
        "matches_gpu": same(ref) and same(ref_np),
    }


def tile_order_sweep(elem_bytes, mib):
    """Every tile order of the transposes on matrices of `mib` MiB and shapes
    from 256 rows up to 256 columns: each order pinned (swz_set_tile_order),
    rotating over four buffer pairs of random bytes, best of three batches of
    100 calls timed with HIP events; then what swz_tune_tile_order picks on
    one pair.
    Pins are removed afterwards.  Returns the lines of a table."""
    import torch

    import tiled_movement_amd as T

    orders = {T.ORDER_DIAGONAL: "diagonal", T.ORDER_HALF_DIAGONAL: "half", T.ORDER_COLUMNS: "columns",
              T.ORDER_STEEP_DIAGONAL: "steep", T.ORDER_SLOPE_8: "1/8", T.ORDER_SLOPE_16: "1/16",
              T.ORDER_SLOPE_32: "1/32"}
    pairs, nbytes = 4, mib << 20
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(0)
    srcs = [torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device=dev, generator=gen) for _ in range(pairs)]
    dsts = [torch.empty((nbytes,), dtype=torch.uint8, device=dev) for _ in range(pairs)]
    sp, dp = [t.data_ptr() for t in srcs], [t.data_ptr() for t in dsts]

    def rate(rows, cols, esz):
        def launch(i):
            rc = T.lib.swz_transpose(sp[i % pairs], dp[i % pairs], rows, cols, esz, T.LAYOUT_SWIZZLE, T.READ_AUTO,
                                     None, stream.cuda_stream)
            if rc:
                raise T.SwzError(rc, "swz_transpose")

        best = 0.0
        for _ in range(3):
            ms, _ = time_steps(launch, 100, 10)
            best = max(best, 2.0 * nbytes * 100 / (ms * 1e-3) / 1e9)
        return best

    lines = ["| elem bytes | rows x cols | output pitch | " + " | ".join(orders.values()) + " | tuned |",
             "|---|---|---|" + "---|" * len(orders) + "---|"]
    for esz in elem_bytes:
        elems, rows = nbytes // esz, 256
        while rows <= elems // 256:
            cols = elems // rows
            rates = {}
            for order, oname in orders.items():
                T.swz_set_tile_order(1, rows, cols, esz, T.READ_AUTO, order)
                rates[oname] = rate(rows, cols, esz)
            chosen = T.swz_tune_tile_order(srcs[0], dsts[0], 1, rows, cols, esz, "swizzle", reps=20, stream=stream)
            T.swz_set_tile_order(1, rows, cols, esz, T.READ_AUTO, -1)
            lines.append(f"| {esz} | {rows} x {cols} | {rows * esz} B | "
                         + " | ".join(f"{rates[n]:,.0f}" for n in orders.values()) + f" | {orders[chosen]} |")
            log(lines[-1])
            rows *= 2
    return lines


ORDER_SHAPE_DIMS = (1024, 1280, 1536, 1792, 2048, 2304, 2560, 2816, 2944, 3072, 3328, 3584, 3840, 3968, 4096, 4160,
                    4352, 4608, 4864, 5120, 5376, 5760, 6144, 6400, 6656, 6912, 7168, 7424, 8128, 8192, 8704, 9216,
                    9728, 10240, 11264, 12288, 13312, 14336, 16384)


def order_shape_sweep(elem_bytes, dims=ORDER_SHAPE_DIMS, lo_mib=32, hi_mib=512):
    """Every tile order, and the shape's default order, on every rows x cols
    matrix with sides from `dims` and 32 to 512 MiB, as a share of the
    reference copy of the same bytes: buffers carved from one 1 GiB source
    and one 1 GiB destination, rotating over as many as fit (at most 512 MiB
    of them), median of three batches of 20 calls.  Returns the lines of a
    table, closed by the mean over the shapes of each column."""
    import torch

    import tiled_movement_amd as T

    names = ["diagonal", "half", "columns", "steep", "1/8", "1/16", "1/32"]
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev).cuda_stream
    gen = torch.Generator(device=dev)
    gen.manual_seed(0)
    src = torch.randint(0, 256, (1 << 30,), dtype=torch.uint8, device=dev, generator=gen)
    dst = torch.empty_like(src)

    def rate(fn, pairs, nbytes):
        rates = []
        for _ in range(3):
            ms, _ = time_steps(lambda i: fn(i % pairs), 20, 3)
            rates.append(2.0 * nbytes * 20 / (ms * 1e-3) / 1e9)
        return sorted(rates)[1]

    lines = ["| elem bytes | rows x cols | copy GB/s | " + " | ".join(names) + " | default | best |",
             "|---|---|---|" + "---|" * len(names) + "---|---|"]
    sums = [0.0] * (len(names) + 2)
    count = 0
    for esz in elem_bytes:
        for rows in dims:
            for cols in dims:
                nbytes = rows * cols * esz
                if not lo_mib << 20 <= nbytes <= hi_mib << 20:
                    continue
                per = -(-nbytes // 4096) * 4096
                pairs = max(1, min((512 << 20) // per, (1 << 30) // per))
                sp = [src.data_ptr() + i * per for i in range(pairs)]
                dp = [dst.data_ptr() + i * per for i in range(pairs)]
                cb = nbytes // 16 * 16
                copy = rate(lambda j: T.lib.swz_copy(sp[j], dp[j], cb, stream), pairs, cb)

                def conv(j):
                    rc = T.lib.swz_transpose(sp[j], dp[j], rows, cols, esz, T.LAYOUT_SWIZZLE, T.READ_AUTO, None,
                                             stream)
                    if rc:
                        raise T.SwzError(rc, "swz_transpose")

                dflt = T.swz_get_tile_order(1, rows, cols, esz)
                shares = []
                for order in T.ORDERS:
                    T.swz_set_tile_order(1, rows, cols, esz, T.READ_AUTO, order)
                    shares.append(rate(conv, pairs, nbytes) / copy)
                T.swz_set_tile_order(1, rows, cols, esz, T.READ_AUTO, -1)
                row = shares + [shares[dflt], max(shares)]
                sums = [a + b for a, b in zip(sums, row)]
                count += 1
                lines.append(f"| {esz} | {rows} x {cols} | {copy:,.0f} | " + " | ".join(f"{v:.3f}" for v in shares)
                             + f" | {names[dflt]} {shares[dflt]:.3f} | {max(shares):.3f} |")
                log(lines[-1])
    lines.append(f"| mean of {count} | | | " + " | ".join(f"{v / max(count, 1):.3f}" for v in sums) + " |")
    return lines


def random_shape_sweep(n, seed=7, lo_mib=16, hi_mib=96):
    """AUTO transposes of `n` seeded random shapes (element size 1, 2 or 4;
    columns log-uniform in 1 .. 16384; rows filling lo_mib .. hi_mib MiB, so
    the pitches and row counts are mostly not multiples of 16 bytes or 64
    bytes), each as a share of the reference copy of the same bytes: buffers
    carved from one 2 GiB source and one 2 GiB destination, rotating over up
    to 16 pairs, median of three batches of 10 calls.  Returns the lines of
    a table, closed by the median share per element size."""
    import random
    import statistics

    import torch

    import tiled_movement_amd as T

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev).cuda_stream
    gen = torch.Generator(device=dev)
    gen.manual_seed(0)
    src = torch.randint(0, 256, (2 << 30,), dtype=torch.uint8, device=dev, generator=gen)
    dst = torch.empty_like(src)
    rng = random.Random(seed)

    def rate(fn, pairs, nbytes):
        rates = []
        for _ in range(3):
            ms, _ = time_steps(lambda i: fn(i % pairs), 10, 2)
            rates.append(2.0 * nbytes * 10 / (ms * 1e-3) / 1e9)
        return sorted(rates)[1]

    lines = ["| elem bytes | rows x cols | pitch % 16 | output row % 64 | kind | order | copy GB/s | GB/s | share |",
             "|---|---|---|---|---|---|---|---|---|"]
    shares = {1: [], 2: [], 4: []}
    for _ in range(n):
        esz = rng.choice((1, 2, 4))
        mib = rng.uniform(lo_mib, hi_mib)
        cols = max(1, int(round(2 ** rng.uniform(0, 14))))
        rows = max(1, int(mib * 2**20 / (cols * esz)))
        nbytes = rows * cols * esz
        per = -(-nbytes // 4096) * 4096
        pairs = max(1, min((2 << 30) // per, 16))
        sp = [src.data_ptr() + i * per for i in range(pairs)]
        dp = [dst.data_ptr() + i * per for i in range(pairs)]
        cb = nbytes // 16 * 16
        copy = rate(lambda j: T.lib.swz_copy(sp[j], dp[j], cb, stream), pairs, cb)

        def conv(j):
            rc = T.lib.swz_transpose(sp[j], dp[j], rows, cols, esz, T.LAYOUT_SWIZZLE, T.READ_AUTO, None, stream)
            if rc:
                raise T.SwzError(rc, "swz_transpose")

        got = rate(conv, pairs, nbytes)
        kind = T.swz_plan(0, rows, cols, esz, "swizzle", T.READ_AUTO)["read_kind"]
        shares[esz].append(got / copy)
        lines.append(f"| {esz} | {rows} x {cols} | {cols * esz % 16} | {rows * esz % 64} | {kind} | "
                     f"{T.swz_get_tile_order(1, rows, cols, esz)} | {copy:,.0f} | {got:,.0f} | {got / copy:.3f} |")
        log(lines[-1])
    for esz, v in shares.items():
        if v:
            lines.append(f"| median of {len(v)}, {esz}-byte | | | | | | | | {statistics.median(v):.3f} |")
    return lines


# The reference copy whose launch moves the same bytes as one launch of the
# workload (staging: both operands, 128 MiB, in one launch).
COPY_OF = {"fp32_transpose": "copy", "fp16_transpose": "copy_128", "fp16_transpose_tr": "copy_128",
           "u8_transpose": "copy", "bf16_convert": "copy", "bf16_stage": "copy_128", "fp32_narrow8": "copy",
           "fp16_narrow8": "copy", "u8_narrow16": "copy", "fp32_rows3": "copy", "u8_rows48": "copy"}
# Workloads whose oracle is timed beside them in the full run (the headline's
# own is the line's cpu_baseline).
ORACLE_TIMED = ("fp16_transpose", "bf16_convert", "bf16_stage", "map_batch")


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--quick", action="store_true", help="headline only, no other workloads")
    ap.add_argument("--workload", choices=sorted(WORKLOADS), default=None)
    ap.add_argument("--layout", choices=["swizzle", "pad", "plain", "direct"], default="swizzle")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="budget of the headline's CPU oracle leg (each other workload's gets a quarter)")
    ap.add_argument("--pairs", type=int, default=None,
                    help="rotate over this many source/destination pairs (default: enough for 512 MiB)")
    ap.add_argument("--tile-orders", action="store_true", help="sweep the transposes' tile orders instead")
    ap.add_argument("--elem-bytes", type=int, nargs="+", default=[4, 2], help="--tile-orders: element sizes")
    ap.add_argument("--mib", type=int, default=64, help="--tile-orders: matrix size in MiB (a power of two)")
    ap.add_argument("--order-shapes", action="store_true",
                    help="every tile order and the default order on many shapes, as shares of a copy")
    ap.add_argument("--random-shapes", type=int, default=0,
                    help="AUTO transposes of this many seeded random shapes, as shares of a copy")
    args = ap.parse_args(argv)
    global PAIRS_OVERRIDE
    PAIRS_OVERRIDE = args.pairs
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported (the path has no "
              "multi-GPU part: each GPU would run the same kernel on its own shard).", file=sys.stderr)
        return 2

    ctx = Ctx()
    if args.tile_orders:
        print("\n".join(tile_order_sweep(args.elem_bytes, args.mib)), flush=True)
        return 0
    if args.order_shapes:
        print("\n".join(order_shape_sweep(args.elem_bytes)), flush=True)
        return 0
    if args.random_shapes:
        print("\n".join(random_shape_sweep(args.random_shapes)), flush=True)
        return 0
    name = args.workload or "fp32_transpose"
    layout = args.layout if args.workload else "swizzle"
    step, nbytes, info = build(ctx, name, layout)
    log(f"{name}/{layout}: {({k: v for k, v in info.items() if not k.startswith('_')})}")
    ms, wall = time_steps(step, args.steps, args.warmup)
    launches = info.get("launches_per_step", 1)
    ms_per_step = ms / args.steps
    value = nbytes * args.steps / (ms * 1e-3) / 1e9
    log(f"{name}/{layout}: {value:.1f} GB/s, {ms_per_step * 1e3:.2f} us/step, wall {wall:.3f} s")

    extra, oracle_timed = {}, {}
    if not args.quick and args.workload is None:
        for wname in ("copy", "copy_128", "copy_zero", "memcpy_d2d", "fp32_transpose", "fp16_transpose",
                      "fp16_transpose_tr", "u8_transpose", "bf16_convert", "bf16_stage", "fp32_narrow8",
                      "fp16_narrow8", "u8_narrow16", "fp32_rows3", "u8_rows48", "map", "bf16_gemm", "bf16_gemm_fused",
                      "bf16_gemm_fused_bf16c", "torch_mm_bf16"):
            for lay in (("swizzle",) if wname in ("copy", "copy_128", "copy_zero", "memcpy_d2d", "map", "bf16_gemm",
                                                  "torch_mm_bf16", "bf16_gemm_fused_bf16c")
                        else ("swizzle", "plain") if wname in ("bf16_gemm_fused", "fp32_rows3", "u8_rows48")
                        else ("swizzle", "pad", "plain", "direct")):
                s2, nb2, inf2 = build(ctx, wname, lay)
                if wname == "map":
                    rate, ms2 = median_rate(s2, nb2, steps=250, warmup=25)
                    extra["map/swizzle"] = {"us_per_call": round(ms2 * 1e3, 3)}
                    log(f"map: {ms2 * 1e3:.2f} us/call")
                    s3, nb3, inf3 = build(ctx, "map_batch", "swizzle")
                    rate3, ms3 = median_rate(s3, nb3, steps=100, warmup=10)
                    extra["map/swizzle"].update({"batch_us_per_125_triples": round(ms3 * 1e3, 2),
                                                 "batch_GBps": round(rate3, 1)})
                    log(f"map batch: {ms3 * 1e3:.2f} us per 125 triples, {rate3:.1f} GB/s")
                    oracle_timed["map_batch"] = cpu_baseline("map_batch", inf3, args.cpu_seconds / 4)
                    log(f"cpu oracle, map: {oracle_timed['map_batch']['value']} GB/s")
                    del s3, inf3
                    continue
                if wname in ("bf16_gemm", "bf16_gemm_fused", "bf16_gemm_fused_bf16c", "torch_mm_bf16"):
                    rate, ms2 = median_rate(s2, nb2, steps=20, warmup=5)
                    tflops = rate / 1e3  # nb2 counts flops, so rate is GFLOP/s
                    key = f"{wname}/{lay}" if wname == "bf16_gemm_fused" else wname
                    extra[key] = {"TFLOPs": round(tflops, 1), "frac_of_mfma_bf16_peak": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                                    "us_per_step": round(ms2 * 1e3, 1), "m": 8192, "n": 8192, "k": 4096}
                    log(f"{key}: {tflops:.1f} TFLOP/s")
                    del s2, inf2
                    ctx.torch.cuda.empty_cache()
                    continue
                rate, ms2 = median_rate(s2, nb2)
                rec = {k: v for k, v in inf2.items() if not k.startswith("_") and k != "workload"}
                rec.update({"GBps": round(rate, 1), "frac": round(rate / HBM_PEAK_GBS, 4),
                            "us_per_step": round(ms2 * 1e3, 2)})
                ref = extra.get(f"{COPY_OF.get(wname)}/swizzle")
                if ref:  # share of the reference copy of the same bytes per launch
                    rec["frac_of_copy"] = round(rate / ref["GBps"], 4)
                mc = measured_conflicts(wname)
                if mc and lay in mc:
                    rec["measured_conflict_cycles_per_tile"] = mc[lay]["conflict_cycles_per_tile"]
                    rec["measured_conflict_cycles_per_lds_instr"] = mc[lay]["conflict_cycles_per_lds_instr"]
                extra[f"{wname}/{lay}"] = rec
                log(f"{wname}/{lay}: {rate:.1f} GB/s")
                if lay == "swizzle" and wname in ORACLE_TIMED:
                    oracle_timed[wname] = cpu_baseline(wname, inf2, args.cpu_seconds / 4)
                    log(f"cpu oracle, {wname}: {oracle_timed[wname]['value']} GB/s, "
                        f"GPU output matches: {oracle_timed[wname]['matches_gpu']}")
                del s2, inf2
                ctx.torch.cuda.empty_cache()
        # Long output rows: the default tile order, then the one
        # swz_tune_tile_order pins for the shape (the pin is removed after).
        s2, nb2, inf2 = build(ctx, "fp32_transpose_long", "swizzle")
        rate_d, ms_d = median_rate(s2, nb2)
        _, srcs2, dsts2, _ = inf2["_io"]
        T = ctx.T
        chosen = T.swz_tune_tile_order(srcs2[0], dsts2[0], 1, 8192, 2048, 4, "swizzle", T.READ_SCALAR_COL, reps=10)
        rate_t, ms_t = median_rate(s2, nb2)
        T.swz_set_tile_order(1, 8192, 2048, 4, T.READ_SCALAR_COL, -1)
        extra["fp32_transpose_long/swizzle"] = {"shape": [1, 8192, 2048], "GBps_default_order": round(rate_d, 1),
                                                "GBps_tuned_order": round(rate_t, 1), "tuned_order": chosen,
                                                "us_per_step_tuned": round(ms_t * 1e3, 2)}
        log(f"fp32 8192x2048: {rate_d:.1f} GB/s default order, {rate_t:.1f} GB/s with order {chosen}")
        del s2, inf2, srcs2, dsts2
        ctx.torch.cuda.empty_cache()
        # The headline and its copy ceiling again with 16 buffer pairs (2 GiB
        # rotating): no reuse of the Infinity Cache or of address
        # translations between calls of one pair.
        saved, PAIRS_OVERRIDE = PAIRS_OVERRIDE, 16
        for wname in ("fp32_transpose", "copy"):
            s2, nb2, inf2 = build(ctx, wname, "swizzle")
            rate, ms2 = median_rate(s2, nb2)
            extra[f"{wname}/swizzle@16pairs"] = {"GBps": round(rate, 1), "frac": round(rate / HBM_PEAK_GBS, 4),
                                                 "us_per_step": round(ms2 * 1e3, 2), "buffer_pairs": 16}
            log(f"{wname}/swizzle, 16 buffer pairs: {rate:.1f} GB/s")
            del s2, inf2
            ctx.torch.cuda.empty_cache()
        PAIRS_OVERRIDE = saved
        extra["cpu_baseline"] = oracle_timed

    cpu = None
    if name == "fp32_transpose" and "_io" in info:
        try:
            cpu = cpu_baseline(name, info, args.cpu_seconds)
            log(f"cpu oracle: {cpu['value']} GB/s; GPU output matches: {cpu['matches_gpu']}")
        except Exception as e:  # a reported baseline only
            log(f"cpu baseline skipped: {e!r}")

    config = {k: v for k, v in info.items() if not k.startswith("_")}
    if name in COPY_OF or name in ("map", "map_batch"):
        config["measured_lds_conflicts"] = measured_conflicts(name)
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
        "dtype": {"fp32_transpose": "f32", "fp32_narrow8": "f32", "fp32_rows3": "f32", "u8_rows48": "u8", "fp32_transpose_long": "f32", "fp16_narrow8": "f16", "u8_narrow16": "u8", "fp16_transpose": "f16", "fp16_transpose_tr": "f16", "u8_transpose": "u8", "map": "int32", "map_batch": "int32", "copy": "u8", "copy_128": "u8", "copy_zero": "u8", "memcpy_d2d": "u8"}.get(name, "bf16"),
        "data": "synthetic",
        "config": config,
        "roofline": {
            "bound": "hbm",
            "achieved": round(value, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(value / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic(name),
            "algorithmic_bytes_per_launch": nbytes // launches,
            "launches_per_step": launches,
        },
        "cpu_baseline": cpu,
        "extra": extra,
    }
    if name in ("bf16_gemm", "bf16_gemm_fused", "bf16_gemm_fused_bf16c", "torch_mm_bf16"):  # a contraction: flops, against the bf16 matrix peak
        tflops = value / 1e3
        line.update({"metric": "bf16 GEMM, TFLOP/s", "value": round(tflops, 1),
                     "unit": "TFLOP/s", "dtype": "bf16"})
        line["roofline"] = {"bound": "mfma", "achieved": round(tflops, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                            "unit": "TFLOP/s", "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": None,
                            "algorithmic_flops_per_launch": nbytes}
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
