"""Time every tile order of the transposes on matrices of one size (64 MiB
unless --mib says otherwise) and several shapes, and what
swz_tune_tile_order picks for each.

Each shape is transposed with each order pinned (swz_set_tile_order),
rotating over four buffer pairs (512 MiB at 64 MiB, twice the Infinity Cache), best
of three batches of 100 calls timed with HIP events; then the tuner runs on
one pair and its choice is recorded.  Pins are removed afterwards.

Usage:
  python -m tiled_movement_amd.tile_order_sweep [--elem-bytes 4 2] [--mib 64] [--out sweep.md]
"""

from __future__ import annotations

import argparse
import sys

import torch

import tiled_movement_amd as T

ORDERS = {T.ORDER_DIAGONAL: "diagonal", T.ORDER_HALF_DIAGONAL: "half", T.ORDER_COLUMNS: "columns",
          T.ORDER_STEEP_DIAGONAL: "steep"}
BYTES = 64 << 20
PAIRS = 4


def time_order(srcs, dsts, rows, cols, esz, stream, nbytes=BYTES):
    sp, dp, sh = [s.data_ptr() for s in srcs], [d.data_ptr() for d in dsts], stream.cuda_stream

    def launch(i):  # the C call itself: host overhead far below the kernel time
        rc = T.lib.swz_transpose(sp[i % PAIRS], dp[i % PAIRS], rows, cols, esz, T.LAYOUT_SWIZZLE, T.READ_AUTO, None, sh)
        if rc:
            raise T.SwzError(rc, "swz_transpose")

    best = 0.0
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for _ in range(3):
        for i in range(10):
            launch(i)
        torch.cuda.synchronize()
        e0.record()
        for i in range(100):
            launch(i)
        e1.record()
        e1.synchronize()
        best = max(best, 2.0 * nbytes * 100 / (e0.elapsed_time(e1) * 1e-3) / 1e9)
    return best


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--elem-bytes", type=int, nargs="+", default=[4, 2])
    ap.add_argument("--mib", type=int, default=BYTES >> 20, help="matrix size in MiB (a power of two)")
    ap.add_argument("--out", default=None)
    args = ap.parse_args(argv)
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    lines = ["| elem bytes | rows x cols | output pitch | " + " | ".join(ORDERS.values()) + " | tuned |",
             "|---|---|---|" + "---|" * len(ORDERS) + "---|"]
    nbytes = args.mib << 20
    srcs = [torch.full((nbytes,), p + 1, dtype=torch.uint8, device=dev) for p in range(PAIRS)]
    dsts = [torch.empty((nbytes,), dtype=torch.uint8, device=dev) for _ in range(PAIRS)]
    for esz in args.elem_bytes:
        elems = nbytes // esz
        rows = 256
        while rows <= elems // 256:
            cols = elems // rows
            rates = {}
            for order, name in ORDERS.items():
                T.swz_set_tile_order(1, rows, cols, esz, T.READ_AUTO, order)
                rates[name] = time_order(srcs, dsts, rows, cols, esz, stream, nbytes)
            chosen = T.swz_tune_tile_order(srcs[0], dsts[0], 1, rows, cols, esz, "swizzle", reps=20, stream=stream)
            T.swz_set_tile_order(1, rows, cols, esz, T.READ_AUTO, -1)
            lines.append(f"| {esz} | {rows} x {cols} | {rows * esz} B | "
                         + " | ".join(f"{rates[n]:,.0f}" for n in ORDERS.values()) + f" | {ORDERS[chosen]} |")
            print(lines[-1], flush=True)
            rows *= 2
    text = "\n".join(lines) + "\n"
    if args.out:
        with open(args.out, "w") as f:
            f.write(text)
    return 0


if __name__ == "__main__":
    sys.exit(main())
