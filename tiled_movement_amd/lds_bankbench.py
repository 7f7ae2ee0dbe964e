"""Measure the gfx950 LDS bank model with programmed lane patterns.

Runs swz_lds_probe (one workgroup of 16 waves per pattern, 96 KiB of LDS so
one pattern owns a CU) and records the shader-clock cycles each access costs.

Pattern families:
  base    all lanes on consecutive addresses (no conflict under any model)
  pair    only lanes i and j active, asking one bank for two different words
          (bytes 0 and 1024); extra cycles mean i and j share an LDS phase
  pairc   the same lanes on neighbouring words (control)
  bank    lanes 0 and j, lane j at byte 128 / 256 / 512: which distances
          are bank-equal tells the bank count
  stride  all lanes, lane l at byte width*s*l
  kernel  every LDS access of one tile of each kernel, in each layout
  subword 1- and 2-byte accesses (ds_read_u8/u16, ds_write_b8/b16): the
          same base, phase (lane 0 with lane j), bank-distance and stride
          tests, plus lanes 0 and j on two bytes of one 4-byte word (a
          shared word: no conflict if words, not bytes, are what conflict)

Usage:
  python -m tiled_movement_amd.lds_bankbench --out lds_bank.json
  python -m tiled_movement_amd.lds_bankbench --per-dispatch --families kernel,bank ...
      (one dispatch per pattern, for rocprofv3 --pmc counter runs)
"""

from __future__ import annotations

import argparse
import json
import sys
import time

import numpy as np
import torch

import tiled_movement_amd as T

WIDTHS = (4, 8, 16)


def pat(name, width, write, addrs, active=None):
    if active is None:
        active = [a is not None and a >= 0 for a in addrs]
    a = [int(x) if (x is not None and x >= 0) else 0 for x in addrs]
    mask = 0
    for l, on in enumerate(active):
        if on:
            mask |= 1 << l
    return {"name": name, "width": width, "write": int(write), "addrs": a, "mask": mask}


def patterns(families):
    out = []
    for w in WIDTHS:
        for wr in (0, 1):
            tag = f"{'w' if wr else 'r'}{8 * w}"
            if "base" in families:
                out.append(pat(f"base/{tag}/contig", w, wr, [l * w for l in range(64)]))
                out.append(pat(f"base/{tag}/one_lane", w, wr, [0] + [-1] * 63))
                if not wr:
                    out.append(pat(f"base/{tag}/broadcast", w, wr, [0] * 64))
            if "pair" in families:
                for i in range(64):
                    for j in range(i + 1, 64):
                        addrs = [-1] * 64
                        addrs[i], addrs[j] = 0, 1024
                        out.append(pat(f"pair/{tag}/{i}/{j}", w, wr, addrs))
            if "pairc" in families:
                for j in range(1, 64):
                    addrs = [-1] * 64
                    addrs[0], addrs[j] = 0, w
                    out.append(pat(f"pairc/{tag}/0/{j}", w, wr, addrs))
            if "bank" in families:
                for dist in (64, 128, 256, 512):
                    for j in (1, 2, 3, 4, 8, 15, 16, 31, 32, 63):
                        addrs = [-1] * 64
                        addrs[0], addrs[j] = 0, dist
                        out.append(pat(f"bank/{tag}/{dist}/{j}", w, wr, addrs))
    if "stride" in families:
        for w in WIDTHS:
            for wr in (0, 1):
                for s in (1, 2, 3, 4, 5, 8, 9, 16, 17, 32, 33, 64, 65):
                    out.append(pat(f"stride/{'w' if wr else 'r'}{8 * w}/{s}", w, wr, [w * s * l for l in range(64)]))
    if "subword" in families:
        for w in (1, 2):
            for wr in (0, 1):
                tag = f"{'w' if wr else 'r'}{8 * w}"
                out.append(pat(f"subword/{tag}/contig", w, wr, [l * w for l in range(64)]))
                out.append(pat(f"subword/{tag}/one_lane", w, wr, [0] + [-1] * 63))
                if not wr:
                    out.append(pat(f"subword/{tag}/broadcast", w, wr, [0] * 64))
                for j in range(1, 64):
                    addrs = [-1] * 64
                    addrs[0], addrs[j] = 0, 1024  # one bank, two words
                    out.append(pat(f"subword/{tag}/pair/0/{j}", w, wr, addrs))
                    addrs = [-1] * 64
                    addrs[0], addrs[j] = 0, 4  # neighbouring words (control)
                    out.append(pat(f"subword/{tag}/pairc/0/{j}", w, wr, addrs))
                    addrs = [-1] * 64
                    addrs[0], addrs[j] = 0, 4 - w  # two parts of one word
                    out.append(pat(f"subword/{tag}/sameword/0/{j}", w, wr, addrs))
                for dist in (64, 128, 256, 512):
                    addrs = [-1] * 64
                    addrs[0], addrs[1] = 0, dist
                    out.append(pat(f"subword/{tag}/bank/{dist}/1", w, wr, addrs))
                for s_ in (1, 2, 4, 8, 16, 32, 64, 65, 128, 129):
                    out.append(pat(f"subword/{tag}/stride/{s_}", w, wr, [w * s_ * l for l in range(64)]))
    if "kernel" in families:
        for kind, kname in [(T.READ_SCALAR_COL, "scalar_col"), (T.READ_B64_4X4, "b64_4x4"),
                            (T.READ_B128_8X8, "b128_8x8"), (T.READ_MFMA_16X16X32, "mfma"),
                            (T.READ_HNARROW8, "hnarrow8"), (T.READ_BNARROW16, "bnarrow16")]:
            for layout in ("swizzle", "pad", "plain"):
                for wr in (1, 0):
                    for idx, (addrs, width) in enumerate(T.swz_kernel_accesses(kind, layout, None, wr)):
                        out.append(pat(f"kernel/{kname}/{layout}/{'w' if wr else 'r'}/{idx}", width, wr, addrs))
    return out


def run(pats, iters, waves, per_dispatch, dev):
    """Cycles per access (median over waves) for every pattern."""
    results = {}
    groups = {}
    for p in pats:
        groups.setdefault((p["width"], p["write"]), []).append(p)
    for (w, wr), ps in groups.items():
        addrs = torch.tensor(np.array([p["addrs"] for p in ps], dtype=np.uint32).view(np.int32), device=dev)
        masks = torch.tensor(np.array([p["mask"] for p in ps], dtype=np.uint64).view(np.int64), device=dev)
        cyc = torch.zeros(len(ps) * waves, dtype=torch.int64, device=dev)
        if per_dispatch:
            for g in range(len(ps)):
                T.swz_lds_probe(addrs[g:], masks[g:], 1, w, wr, iters, waves, cyc[g * waves:])
        else:
            T.swz_lds_probe(addrs, masks, len(ps), w, wr, iters, waves, cyc)
        torch.cuda.synchronize()
        c = cyc.cpu().numpy().reshape(len(ps), waves).astype(np.float64)
        per_access = np.median(c, axis=1) / (iters * 8)
        for p, v, row in zip(ps, per_access, c):
            results[p["name"]] = {"cycles_per_access": float(v), "wave_min": float(row.min() / (iters * 8)),
                                  "wave_max": float(row.max() / (iters * 8)), "width": w, "write": wr,
                                  "mask": p["mask"]}
        print(f"group width={w} write={wr}: {len(ps)} patterns", flush=True)
    return results


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--out", required=True)
    ap.add_argument("--families", default="base,pair,pairc,bank,stride,kernel")
    ap.add_argument("--iters", type=int, default=64)
    ap.add_argument("--waves", type=int, default=16)
    ap.add_argument("--per-dispatch", action="store_true")
    args = ap.parse_args(argv)
    dev = torch.device("cuda:0")
    fams = set(args.families.split(","))
    pats = patterns(fams)
    print(f"{len(pats)} patterns, families {sorted(fams)}", flush=True)
    t0 = time.time()
    # warm-up launch (code object load, clocks)
    run(pats[:8], args.iters, args.waves, False, dev)
    res = run(pats, args.iters, args.waves, args.per_dispatch, dev)
    meta = {
        "device": torch.cuda.get_device_name(0),
        "iters": args.iters,
        "waves": args.waves,
        "per_dispatch": args.per_dispatch,
        "order": [p["name"] for p in pats],
        "seconds": time.time() - t0,
    }
    with open(args.out, "w") as f:
        json.dump({"meta": meta, "results": res}, f)
    print(f"wrote {args.out} ({len(res)} patterns, {time.time() - t0:.1f} s)", flush=True)


if __name__ == "__main__":
    sys.exit(main())
