"""Plain CPU oracle: swizzle map, tile address maps, the data-movement results,
a brute-force per-wavefront bank-conflict counter and the parameter chooser.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Slow and obvious on
purpose: NumPy and Python loops, no blocking, no fusion.

Pages cited (title, then section):
  [CuTe-DSL]  "NVIDIA CuTe Swizzle"
  [Handbook]  "CuTe Swizzle 学习手册"
  [Intro]     "cutlass 入门"
  [HowItWorks] "CUDA 013 - Swizzle 的工作原理"

Readings taken where the pages are silent or disagree (listed again in the
design notes):
  * M is counted in elements, not bytes ([CuTe-DSL] derivation of MBase and
    [HowItWorks] §计算公式 both count elements; [Handbook] §Swizzle<B,M,S>
    三个参数的含义 speaks of bytes, which is the same map with M raised by
    log2(element size) and the offset scaled to bytes).
  * Offsets are unsigned 32-bit bit patterns; shifts are logical.
  * A bank "word" is bank_bytes wide; lanes touching the same word of a bank
    are served together (broadcast), lanes touching different words of one
    bank within one phase are serialised ([Handbook] §什么情况下产生冲突;
    [HowItWorks] §什么是 Bank Conflict; [CuTe-DSL] on two f16 in one word).
  * The minimum number of phases a wide access needs is not a conflict
    ([CuTe-DSL], remark on ldmatrix.x4); conflict cycles are counted per
    phase as (worst per-bank word count - 1).
"""

from __future__ import annotations

from collections import defaultdict
from dataclasses import dataclass, field
from typing import Dict, Iterable, List, Optional, Sequence, Tuple

import numpy as np

__all__ = [
    "swizzle",
    "swizzle_clear_set",
    "swizzle_signed",
    "swizzle_map",
    "fold_collision",
    "fold_strides",
    "tile_offset",
    "transpose",
    "convert_layout",
    "stage_operand",
    "stage_operand_loops",
    "bf16_to_f64",
    "f32_to_bf16_bits",
    "gemm_bf16",
    "gemm_error_bound",
    "BankModel",
    "LdsModel",
    "nvidia_model",
    "conflict_report",
    "access_addresses",
    "pattern_cycles",
    "choose",
    "rule_bits",
]

# --------------------------------------------------------------------------
# 1. The swizzle map
# --------------------------------------------------------------------------


def swizzle(x, B: int, M: int, S: int):
    """Swizzle<B,M,S> of an element offset.

    [Handbook] §Swizzle 数学公式: take the B-bit field that starts at bit M+S,
    shift it down by S and XOR it into the B-bit field that starts at bit M;
    every other bit passes through unchanged.

    ``x`` may be a Python int (returns int) or a NumPy integer array (returns
    uint32, the input taken as 32-bit unsigned bit patterns).
    """
    if B < 0 or M < 0 or S < 0:
        raise ValueError("swizzle parameters must be non-negative")
    mask = (1 << B) - 1
    if isinstance(x, (int, np.integer)):
        x = int(x) & 0xFFFFFFFF
        return x ^ (((x >> (M + S)) & mask) << M)
    u = np.asarray(x).astype(np.int64) & 0xFFFFFFFF
    out = u ^ (((u >> (M + S)) & mask) << M)
    return (out & 0xFFFFFFFF).astype(np.uint32)


def swizzle_clear_set(offset, base: int, bits: int, shift: int):
    """The same map in the form [HowItWorks] §计算公式 gives it.

    Note the argument order of that page: (base, bits, shift) = (M, B, S).
    Extract ZZ (``bits`` bits from ``base``) and YY (``bits`` bits from
    ``base + shift``), clear the ZZ field, then write ZZ xor YY into it.
    Scalar Python ints only; written independently of ``swizzle``.
    """
    offset = int(offset) & 0xFFFFFFFF
    field_mask = (1 << bits) - 1
    zz = (offset >> base) & field_mask
    yy = (offset >> (base + shift)) & field_mask
    cleared = offset & ~(field_mask << base) & 0xFFFFFFFF
    return cleared | ((zz ^ yy) << base)


def swizzle_signed(x, B: int, M: int, S: int):
    """Swizzle<B,M,S> for a shift of either sign.

    [CuTe-DSL] (the SShift comment of its bit diagram): the shift says how
    far the YYY mask sits from the ZZZ mask that keeps MBase low bits
    constant; a positive shift puts YYY above ZZZ (the XOR moves YYY right,
    onto ZZZ), a negative shift puts it below (the XOR moves YYY left).  So
    for S >= 0 the source field is bits [M+S, M+S+B) and the target [M, M+B);
    for S < 0 the source is [M, M+B) and the target [M+|S|, M+|S|+B).  The
    target becomes target XOR source; all other bits pass through.  Scalar
    ints or NumPy integer arrays (taken as uint32).
    """
    if B < 0 or M < 0:
        raise ValueError("B and M must be non-negative")
    src_lo = M + max(S, 0)
    dst_lo = M + max(-S, 0)
    mask = (1 << B) - 1
    if isinstance(x, (int, np.integer)):
        x = int(x) & 0xFFFFFFFF
        return (x ^ (((x >> src_lo) & mask) << dst_lo)) & 0xFFFFFFFF
    u = np.asarray(x).astype(np.int64) & 0xFFFFFFFF
    return ((u ^ (((u >> src_lo) & mask) << dst_lo)) & 0xFFFFFFFF).astype(np.uint32)


def swizzle_map(offsets: np.ndarray, B: int, M: int, S: int) -> np.ndarray:
    """Elementwise swizzle of int32 offsets, output int32 (same bit pattern);
    S may be negative (``swizzle_signed``)."""
    a = np.asarray(offsets)
    if a.dtype != np.int32:
        raise TypeError("swizzle_map takes int32 offsets")
    if S < 0:
        return swizzle_signed(a.view(np.uint32), B, M, S).view(np.int32)
    return swizzle(a.view(np.uint32), B, M, S).view(np.int32)


def fold_collision(active: int, B: int, M: int, S: int) -> int:
    """[Intro] §swizzle 融入 layout 优化: with A the OR of every offset a
    slice can reach (its active bits), collision = A & ~sw(A) has a one at
    each target bit whose source bit is also active; the slice folds into a
    plain layout exactly when it is zero."""
    a = int(active) & 0xFFFFFFFF
    return a & ~swizzle_signed(a, B, M, S) & 0xFFFFFFFF


def fold_strides(base: int, active: int, B: int, M: int, S: int):
    """The folded layout of a collision-free slice: (sw(base), {bit: stride})
    with sw(base | x) = sw(base) + sum of the strides of x's bits.  Each
    stride is the signed change of sw(base) when that one active bit is set
    (computed directly from the map, one bit at a time)."""
    sb = swizzle_signed(base, B, M, S)
    out = {}
    for b in range(32):
        if (active >> b) & 1:
            out[b] = int(swizzle_signed(base | (1 << b), B, M, S)) - int(sb)
    return int(sb), out


# --------------------------------------------------------------------------
# 2. Where a logical tile element lives in the on-chip scratch tile
# --------------------------------------------------------------------------


def tile_offset(r, c, width: int, layout: str, params=None, pad: int = 0):
    """Physical element offset of logical element (r, c) of a row-major tile.

    * ``swizzle``: the row-major offset r*width+c pushed through Swizzle<B,M,S>
      ([Handbook] ① composition of a swizzle with a row-major layout;
      [HowItWorks] §更通用的映射规则: the swizzle acts on the flat offset).
    * ``pad``: rows of width+pad elements ([HowItWorks] §如何避免 Bank Conflict,
      the 32x33 array).
    * ``plain``: rows of width elements, no remapping.
    """
    lin_r = np.asarray(r, dtype=np.int64)
    lin_c = np.asarray(c, dtype=np.int64)
    if layout == "swizzle":
        B, M, S = params
        out = swizzle(lin_r * width + lin_c, B, M, S)
        return out.astype(np.int64) if isinstance(out, np.ndarray) else out
    if layout == "pad":
        return lin_r * (width + pad) + lin_c
    if layout == "plain":
        return lin_r * width + lin_c
    raise ValueError(f"unknown layout {layout!r}")


# --------------------------------------------------------------------------
# 3. What the data-movement calls compute (plain definitions)
# --------------------------------------------------------------------------


def transpose(src: np.ndarray) -> np.ndarray:
    """Row-major [rows][cols] -> its transpose stored row-major [cols][rows].

    The tile engine of [Handbook] §冲突的典型场景 and [HowItWorks]
    §如何避免 Bank Conflict exists to read a row-major tile by columns; the
    whole-matrix result is dst[c][r] = src[r][c], a plain bit copy.
    """
    if src.ndim != 2:
        raise ValueError("transpose takes a 2-D array")
    rows, cols = src.shape
    dst = np.empty((cols, rows), dtype=src.dtype)
    dst[...] = src.T
    return dst


def convert_layout(src: np.ndarray) -> np.ndarray:
    """Batched [batch][rows][cols] -> [batch][cols][rows]: a transpose per batch entry."""
    if src.ndim != 3:
        raise ValueError("convert_layout takes a 3-D array")
    batch, rows, cols = src.shape
    dst = np.empty((batch, cols, rows), dtype=src.dtype)
    for b in range(batch):
        dst[b] = transpose(src[b])
    return dst


FRAG_ROWS = 16  # rows (M or N) of one 16x16x32 operand fragment
FRAG_K = 32  # k extent of one fragment
FRAG_LANES = 64
FRAG_ELEMS = 8  # 16-bit elements each lane holds


def stage_operand(x: np.ndarray) -> np.ndarray:
    """Operand fragments of a K-contiguous 16-bit matrix x[mn][k].

    Output frag[i][j][l][e] = x[16*i + l % 16][32*j + 8*(l // 16) + e] for
    i < mn/16, j < k/32, lane l < 64, e < 8: each lane of a 64-wide wave holds
    eight consecutive k values of one row, the four 16-lane groups covering
    the 32-wide k step.  This is the operand register layout of the CDNA
    16x16x32 16-bit matrix instruction.  The pages' own version of this step
    is the ldmatrix / WGMMA read of a swizzled tile ([CuTe-DSL] ldmatrix
    rationale; [Handbook] ⑤); they do not fix a lane order for AMD hardware.
    Written as an index gather from the formula.
    """
    if x.ndim != 2:
        raise ValueError("stage_operand takes a 2-D array")
    mn, k = x.shape
    if mn % FRAG_ROWS or k % FRAG_K:
        raise ValueError("mn must be a multiple of 16 and k of 32")
    i = np.arange(mn // FRAG_ROWS).reshape(-1, 1, 1, 1)
    j = np.arange(k // FRAG_K).reshape(1, -1, 1, 1)
    lane = np.arange(FRAG_LANES).reshape(1, 1, -1, 1)
    e = np.arange(FRAG_ELEMS).reshape(1, 1, 1, -1)
    row = FRAG_ROWS * i + lane % 16
    col = FRAG_K * j + 8 * (lane // 16) + e
    return x[row, col]


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bf16 bit patterns: the upper half of an fp32 word."""
    b = np.asarray(bits).astype(np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """bf16 bit patterns of fp32 values rounded to nearest, ties to the even
    pattern, by the definition: of the two bf16 values around x (its bit
    pattern cut to the upper half, and the next one away from zero), take the
    nearer one; NaN becomes a quiet NaN.  Written out per element in fp64
    (every fp32 and bf16 value is exact there); the next value past the
    largest finite bf16 is 2^128, which rounds to infinity."""
    x = np.asarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lo = (u >> 16) << 16
    hi = lo + (1 << 16)
    xv = x.astype(np.float64)
    # NaN inputs (and the patterns past infinity) are sorted out at the end
    with np.errstate(over="ignore", invalid="ignore"):
        lov = lo.astype(np.uint32).view(np.float32).astype(np.float64)
        hiv = hi.astype(np.uint32).view(np.float32).astype(np.float64)
        hiv = np.where(np.isinf(hiv) & ~np.isinf(lov), np.sign(xv) * 2.0 ** 128, hiv)
        d_lo, d_hi = np.abs(xv - lov), np.abs(hiv - xv)
    even_lo = ((lo >> 16) & 1) == 0
    take_hi = (d_hi < d_lo) | ((d_hi == d_lo) & ~even_lo)
    out = np.where(take_hi, hi >> 16, lo >> 16)
    out = np.where(np.isnan(xv), (u >> 16) | 0x40, out)
    return out.astype(np.uint16)


def gemm_bf16(a_bits: np.ndarray, bt_bits: np.ndarray) -> np.ndarray:
    """C = A * B^T of bf16 operands (A [m][k], B^T [n][k], as bit patterns),
    in fp64 -- the product the staged fragments feed to the matrix unit
    ([CuTe-DSL] ldmatrix / WGMMA as the consumer of the staged tile;
    [Handbook] ⑤).  The step is a library matmul over exact fp64 values."""
    return bf16_to_f64(a_bits) @ bf16_to_f64(bt_bits).T


def gemm_error_bound(a_bits: np.ndarray, bt_bits: np.ndarray, chunk: int = 32) -> np.ndarray:
    """Per-element bound on |fp32 result - exact| for a sum of k products
    taken `chunk` at a time and accumulated in fp32: each of the k/chunk
    accumulations and each chunk's own summation round at most once per
    step, so |error| <= (k/chunk + chunk) * 2^-24 * sum_k |a| |b| (a
    first-order bound; tests use it with a factor of 2 of margin)."""
    k = np.asarray(a_bits).shape[1]
    steps = k // chunk + chunk
    return steps * 2.0 ** -24 * (np.abs(bf16_to_f64(a_bits)) @ np.abs(bf16_to_f64(bt_bits)).T)


def stage_operand_loops(x: np.ndarray) -> np.ndarray:
    """Pure-Python loop version of ``stage_operand`` for tiny inputs."""
    mn, k = x.shape
    out = np.empty((mn // 16, k // 32, 64, 8), dtype=x.dtype)
    for i in range(mn // 16):
        for j in range(k // 32):
            for lane in range(64):
                for e in range(8):
                    out[i, j, lane, e] = x[16 * i + lane % 16, 32 * j + 8 * (lane // 16) + e]
    return out


# --------------------------------------------------------------------------
# 4. Bank model and the brute-force per-wavefront conflict counter
# --------------------------------------------------------------------------


@dataclass
class BankModel:
    """Banks of the on-chip scratch and how a wave's lanes are split into phases.

    ``n_banks`` banks of ``bank_bytes`` each; byte address a lies in bank
    (a // bank_bytes) % n_banks ([Handbook] §Shared Memory 的 Bank 结构 gives
    this with 32 banks of 4 bytes; [HowItWorks] §什么是 memory bank).
    ``phases[width]`` lists the lane groups served together by an access of
    ``width`` bytes per lane; by default consecutive groups of
    n_banks*bank_bytes // width lanes (one bank row per phase).
    """

    n_banks: int
    bank_bytes: int
    n_lanes: int = 64
    phases: Dict[int, List[List[int]]] = field(default_factory=dict)

    def phase_groups(self, width: int) -> List[List[int]]:
        if width in self.phases:
            return self.phases[width]
        per = max(1, min(self.n_lanes, (self.n_banks * self.bank_bytes) // max(width, 1)))
        return [list(range(s, min(s + per, self.n_lanes))) for s in range(0, self.n_lanes, per)]


@dataclass
class LdsModel:
    """A bank model per access direction and width.

    The pages give one geometry for every access ([Handbook] §Shared Memory 的
    Bank 结构).  Reading taken for hardware where the geometry depends on the
    access: each (direction, bytes per lane) has its own BankModel."""

    read: Dict[int, BankModel]
    write: Dict[int, BankModel]

    def for_access(self, width: int, write: bool) -> BankModel:
        return (self.write if write else self.read)[width]


def nvidia_model() -> BankModel:
    """32 banks x 4 bytes, 32-thread warps: the model every page assumes."""
    return BankModel(n_banks=32, bank_bytes=4, n_lanes=32)


def conflict_report(addrs: Sequence[Optional[int]], width: int, model: BankModel):
    """Conflicts of one access instruction.

    ``addrs[l]`` is lane l's byte address (None = lane inactive), each lane
    touching ``width`` bytes.  Returns (cycles, worst_degree, degrees), where
    a phase's degree is the largest number of distinct words any one bank is
    asked for, and cycles = sum over phases of (degree - 1).
    """
    cycles = 0
    worst = 0
    degrees = []
    for lanes in model.phase_groups(width):
        words_of_bank: Dict[int, set] = defaultdict(set)
        for lane in lanes:
            if lane >= len(addrs) or addrs[lane] is None:
                continue
            a = int(addrs[lane])
            first = a // model.bank_bytes
            last = (a + width - 1) // model.bank_bytes
            for w in range(first, last + 1):
                words_of_bank[w % model.n_banks].add(w)
        degree = max((len(s) for s in words_of_bank.values()), default=0)
        degrees.append(degree)
        if degree:
            cycles += degree - 1
            worst = max(worst, degree)
    return cycles, worst, degrees


def access_addresses(coords, width_elems: int, tile_cols: int, esz: int, layout: str,
                     params=None, pad: int = 0):
    """Byte addresses of one tile access: ``coords[l]`` = (row, col) of the
    first element lane l touches (None = inactive)."""
    out = []
    for rc in coords:
        if rc is None:
            out.append(None)
            continue
        r, c = rc
        out.append(int(tile_offset(r, c, tile_cols, layout, params, pad)) * esz)
    return out


def pattern_cycles(instrs, tile_cols: int, esz: int, layout: str, model,
                   params=None, pad: int = 0, write: bool = False):
    """Total conflict cycles and worst degree over a list of instructions,
    each given as (coords, width_bytes).  ``model`` is a BankModel, or an
    LdsModel from which the (direction, width) geometry is taken."""
    total = 0
    worst = 0
    for coords, width in instrs:
        addrs = access_addresses(coords, width // esz, tile_cols, esz, layout, params, pad)
        m = model.for_access(width, write) if isinstance(model, LdsModel) else model
        c, w, _ = conflict_report(addrs, width, m)
        total += c
        worst = max(worst, w)
    return total, worst


# --------------------------------------------------------------------------
# 5. Choosing Swizzle<B,M,S>
# --------------------------------------------------------------------------


def _log2_exact(v: int) -> int:
    if v <= 0 or v & (v - 1):
        raise ValueError(f"{v} is not a power of two")
    return v.bit_length() - 1


def rule_bits(esz: int, vec_bytes: int, model: BankModel) -> int:
    """B as the pages derive it: log2 of how many vectors fill one bank row.

    [CuTe-DSL]: with 32 banks of 4 bytes one bank row holds 64 f16; 16-byte
    vectors leave 3 bits.  [HowItWorks] §CuTe 通用 swizzle 映射规则解析 item 2:
    4-byte elements give 5 bits, 8-byte elements 4 bits.
    """
    row_bytes = model.n_banks * model.bank_bytes
    return max(0, _log2_exact(row_bytes // max(vec_bytes, 1)) if row_bytes >= vec_bytes else 0)


def choose(esz: int, vec_bytes: int, tile_rows: int, tile_cols: int, write_instrs, read_instrs,
           model):
    """(B, M, S) for a tile staged by ``write_instrs`` and read by ``read_instrs``.

    The pages' derivation ([CuTe-DSL]; [HowItWorks] §CuTe 通用 swizzle 映射规则解析
    and §使用示例):
      * M = log2(elements per vector), so a vector stays contiguous;
      * B = log2(vectors per bank row), limited so that the XOR source field
        also lies inside the tile (M + 2B <= log2(tile elements));
      * S places the source field on the row bits; here it is the smallest
        S >= B whose predicted conflict cycles (write + read) are least,
        which reproduces log2(row vectors) for the pages' column reads and
        groups rows when a row is narrower than a bank row (their int[32][8]
        example).
    If no S reaches zero cycles at that B, every B in 1..Bmax is tried and
    the least-cycles triple wins, ties to the B nearest the rule, then the
    smaller S.  Returns ((B, M, S), cycles).

    ``model`` is one BankModel for every access, or an LdsModel; then the bank
    row that sets B is the one the reads see (the layout exists for them).
    """
    M = _log2_exact(max(vec_bytes // esz, 1))
    log_tile = _log2_exact(tile_rows * tile_cols)
    b_max = (log_tile - M) // 2
    row_model = model.for_access(read_instrs[0][1], False) if isinstance(model, LdsModel) else model
    b_rule = min(rule_bits(esz, vec_bytes, row_model), b_max)

    def cost(B, S):
        cw, _ = pattern_cycles(write_instrs, tile_cols, esz, "swizzle", model, (B, M, S), write=True)
        cr, _ = pattern_cycles(read_instrs, tile_cols, esz, "swizzle", model, (B, M, S), write=False)
        return cw + cr

    best = None
    for S in range(b_rule, log_tile - M - b_rule + 1):
        cyc = cost(b_rule, S)
        if best is None or cyc < best[1]:
            best = ((b_rule, M, S), cyc)
        if cyc == 0:
            return (b_rule, M, S), 0
    for B in range(1, b_max + 1):
        for S in range(B, log_tile - M - B + 1):
            cyc = cost(B, S)
            key = (cyc, abs(B - b_rule), S)
            bkey = (best[1], abs(best[0][0] - b_rule), best[0][2])
            if key < bkey:
                best = ((B, M, S), cyc)
    return best
