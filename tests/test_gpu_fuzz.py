"""Seeded random transposes through AUTO (needs a GPU): shapes from one
element to a few MiB with any pitch, batches, the swizzled, plain and
padded layouts and pointers at random offsets from a 256-byte boundary, so
that every routing rule of the read-kind and grid choice is met (whole-row
and flat-row kinds, the XCD-grouped grids for output rows or pointers off
the 64-byte lines, the element path).  Each output is compared whole with
the oracle."""

import numpy as np
import pytest

import oracle as O
import workloads as W

import torch  # noqa: E402  (hard imports: a GPU run without them fails, never skips)

import tiled_movement_amd as T  # noqa: E402

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
GEN = {4: W.fp32_matrix, 2: W.fp16_matrix, 1: W.u8_matrix}
SIGNED = {np.dtype(np.uint32): np.int32, np.dtype(np.uint16): np.int16, np.dtype(np.uint8): np.int8}


def test_seeded_random_auto_transposes():
    rng = np.random.default_rng(2031)
    done = unsupported = 0
    for case in range(120):
        esz = int(rng.choice([1, 2, 4]))
        cols = max(1, int(2 ** rng.uniform(0, 11.6)))
        rows = max(1, int(2 ** rng.uniform(0, 13)))
        rows = min(rows, max(1, (4 << 20) // (cols * esz)))
        batch = 1 if rng.random() < 0.8 else int(rng.integers(2, 4))
        layout = str(rng.choice(["swizzle", "plain", "pad"]))
        so, do = (int(rng.choice([0, esz, 4 if esz <= 4 else 0, 16, 64])) // esz * esz for _ in range(2))
        a = GEN[esz](batch * rows, cols, seed=case).reshape(batch, rows, cols)
        print("case:", case, esz, (batch, rows, cols), layout, so, do, flush=True)
        lead_s, lead_d = so // esz, do // esz
        src = torch.from_numpy(np.concatenate([np.zeros(lead_s, a.dtype), a.reshape(-1)]).view(SIGNED[a.dtype])).to(DEV)
        dst = torch.zeros(lead_d + a.size, dtype=src.dtype, device=DEV)
        try:
            T.swz_convert_layout(src[lead_s:], dst[lead_d:], batch, rows, cols, esz, layout)
        except T.SwzError as e:  # rows under one 4-byte LDS store have no padded layout
            assert layout == "pad" and e.status == T.SWZ_EUNSUPPORTED and cols * esz < 4, (case, e)
            unsupported += 1
            continue
        torch.cuda.synchronize()
        got = dst.cpu().numpy().view(a.dtype)
        assert np.array_equal(got[lead_d:].reshape(batch, cols, rows), O.convert_layout(a)), case
        assert not got[:lead_d].any(), case
        done += 1
    assert done >= 100 and done + unsupported == 120
