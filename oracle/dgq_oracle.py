"""CPU oracle for dynamic-group INT8 KV-cache compression (DGQ) and paged decode attention.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check in ``__graft_entry__`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  The library (HIP kernels, C ABI,
Python binding) never imports, links or calls it, and this module imports nothing from the
library: the two share no code.  Only the seeded input generator (``dgq_data``) feeds both.

It is written to be read against the pages, not to be fast: plain NumPy, one step per function,
in the order the method describes, each function naming the passage it follows.

Pages cited (titles as they appear on the pages; addresses for the reader):

* "DGQ article" -- DeepSeek KV-cache dynamic group quantization write-up,
  http://www.pptc.cn/news/101026.  Section 2.2 (the DGQ idea: variance curve along the sequence,
  16-token sliding window, 3~5 segments, per-segment min/max, INT8 codes, 1-bit identifier);
  section 3.2 (segment identifier storage variants, length-aware group count); section 3.3 (the
  memory formula: 1 byte per element plus 1 bit per token per head).
* "PagedAttention article" -- DeepSeek-V4 high-concurrency KV-cache article,
  https://deepseek.csdn.net/6a0bbfa610ee7a33f27399ed.html.  "PagedAttention implementation"
  (logical blocks mapped to physical blocks through a block table) and the paged forward pass.
* "Quantization article" -- http://cnnetsun.cn/a/2561798, section 2.1: the asymmetric quantization
  template clamp(round(x / scale) + zero_point, lo, hi).

Readings of points the pages leave open (each is a choice, listed with its reason in the design
notes; "parity unpinned" below marks the ones nothing on the pages can confirm):

R1  Inputs are float16; each value is taken as float32 and -0 becomes +0 (x + 0.0).
R2  Variance statistics use an exact fixed-point image n = rint(clamp(x, -32, 32) * 512)
    (ties to even), so every moment is an integer and the change points do not depend on the
    order of a floating-point sum.  (parity unpinned: grid and clamp are ours)
R3  Window statistic of the 16-token window starting at s (all head_dim channels of those
    tokens): Q(s) = N * sum(n^2) - (sum n)^2 with N = 16 * head_dim, i.e. N^2 times the window's
    population variance.  The sliding window moves one token at a time.
R4  Candidate cut t in [16, L-16]: score(t) = (max(Q(t-16), Q(t)) + 1) / (min(Q(t-16), Q(t)) + 1),
    one IEEE float64 division.
R5  Selection: up to max_segments-1 cuts; each round takes the highest remaining score (smallest
    t on ties); the first cut is always taken, later ones only if score >= tau (tau = 2.0);
    a taken cut removes every candidate within 15 tokens of it.  L < 32 gives one segment.
    (parity unpinned: tau and the forced first cut are ours; they give the pages' 2..5 segments)
R6  Segments are contiguous token ranges; K decides the cuts and V shares them; K and V each
    have their own per-segment min/max (one scalar per segment, all channels).
R7  Boundary bit per token and head: 1 exactly at the first token of every segment but the first.
R8  scale = fp32(fp32(max - min) / 255); code = clamp(rint(fp32(fp32(x - min) * inv)), 0, 255) - 128
    with inv = fp32(255 / fp32(max - min)) (0 when max == min); every step rounds to nearest even.
R9  Dequantized value = (code + 128) * scale + min.
R10 Decode: softmax(q . k_hat / sqrt(head_dim)) . v_hat over all cached tokens, query head g uses
    kv head g // (hq / hkv); no mask, no rotary step (the synthetic keys stand for post-rotary keys).
R11 Append: see ``AppendState``.  (parity unpinned: the rule is ours)
R12 Segment-count policies, both off by default.  Length-aware cap (DGQ article 3.2): a sequence
    of L tokens gets at most 2 segments below 2048 tokens, 3 below 16384, else
    floor(log2(L / 1024)) + 2 but never more than 5; the cap lowers max_segments, never raises it.
    Variance floor MIN_VAR (DGQ article 5.3, "tokens whose variance is below the threshold go into
    one group"): a candidate cut is dropped when both of its windows have a population variance
    (over the window's 16 x head_dim values, on the fixed-point grid) below min_var, i.e. when
    max(Q_left, Q_right) < min_var * N^2 * 512^2; the append window test obeys the same floor.
    (parity unpinned: "both windows below" is our reading of the floor)
R13 Marker format (DGQ article 3.2, the variant that keeps the segment identifier inside the
    INT8 data instead of a separate bit tensor by leaving the two end byte values unused).  Data
    codes take 254 levels: c = clamp(rint(fp32(fp32(x - min) * inv)), 0, 253) - 127 in
    [-127, 126], inv = fp32(253 / fp32(max - min)) (0 when max == min), scale =
    fp32(fp32(max - min) / 253), value (c + 127) * scale + min.  The byte values -128 and 127
    carry no data: the key byte of channel 0 of the first token of every segment but the first
    holds a marker, 127 when that element's own code is >= 0 and -128 otherwise, and every byte,
    marker or not, is dequantized with the same formula (a marker stands for min - scale or
    max + scale).  The identifier of token t is "its channel-0 key byte is -128 or 127"; segment
    starts are unchanged, and the segment table still records them.  (parity unpinned: the
    marker's place, its choice between the two values and its dequantized value are ours)
"""

from __future__ import annotations

import dataclasses
import math
from typing import List, Optional

import numpy as np

WIN = 16            # sliding-window length, DGQ article section 2.2 (win_size=16)
FP_SCALE = 512.0    # R2: fixed-point grid 2^-9
FP_CLAMP = 32.0     # R2: statistics clamp
TAU = 2.0           # R5
MAX_SEGMENTS = 5    # DGQ article section 2.2: 3~5 segments; 2..5 with the forced first cut
SEG_CAPACITY = 16   # segment-table entries per (sequence, kv head) for appends
CODE_LEVELS = 255   # INT8: 256 codes, 255 steps between min and max
MARKER_LEVELS = 253  # R13: 254 data codes, 253 steps; -128 and 127 are markers
MARK_LOW, MARK_HIGH = -128, 127
FORMATS = ("bitmap", "marker")


def format_levels(fmt: str):
    """(steps between min and max, code of the minimum) of a storage format (R8 / R13)."""
    if fmt == "bitmap":
        return CODE_LEVELS, -128
    if fmt == "marker":
        return MARKER_LEVELS, -127
    raise ValueError(f"unknown format {fmt!r}")


# ----------------------------------------------------------------------------------------------
# Compression of one (sequence, kv head): DGQ article section 2.2
# ----------------------------------------------------------------------------------------------

def canonical_f32(x16: np.ndarray) -> np.ndarray:
    """R1: float16 -> float32, with -0 turned into +0."""
    return np.asarray(x16, dtype=np.float16).astype(np.float32) + np.float32(0.0)


def fixed_point(x16: np.ndarray) -> np.ndarray:
    """R2: integer image of each value used only for the variance statistics."""
    x = canonical_f32(x16).astype(np.float64)
    return np.rint(np.clip(x, -FP_CLAMP, FP_CLAMP) * FP_SCALE).astype(np.int64)


def token_moments(k16: np.ndarray):
    """Per-token first and second moments of the fixed-point keys: a_t = sum_d n, b_t = sum_d n^2."""
    n = fixed_point(k16)
    return n.sum(axis=1), (n * n).sum(axis=1)


def window_q(a: np.ndarray, b: np.ndarray, head_dim: int) -> np.ndarray:
    """R3: the variance curve.  Q[s] for every window [s, s+16), s = 0 .. L-16 (int64)."""
    length = len(a)
    if length < WIN:
        return np.zeros(0, dtype=np.int64)
    ca = np.concatenate([[0], np.cumsum(a, dtype=np.int64)])
    cb = np.concatenate([[0], np.cumsum(b, dtype=np.int64)])
    sum_a = ca[WIN:] - ca[:-WIN]
    sum_b = cb[WIN:] - cb[:-WIN]
    n_elems = WIN * head_dim
    return n_elems * sum_b - sum_a * sum_a


def variance_floor_q(min_var: float, head_dim: int) -> float:
    """R12: the variance floor on the Q scale, N^2 * 512^2 * min_var (an exact power-of-two scaling
    of min_var for head_dim 64 and 128)."""
    n_elems = WIN * head_dim
    return float(np.float64(min_var) * np.float64(n_elems * n_elems) * np.float64(FP_SCALE * FP_SCALE))


def change_scores(q: np.ndarray, length: int, floor_q: float = 0.0) -> np.ndarray:
    """R4: score of every candidate t = 16 .. L-16 (index i <-> t = 16 + i), float64; with a
    variance floor (R12) a candidate whose two windows are both below it scores -inf."""
    if length < 2 * WIN:
        return np.zeros(0, dtype=np.float64)
    left = q[0:length - 2 * WIN + 1]          # window [t-16, t)
    right = q[WIN:length - WIN + 1]           # window [t, t+16)
    hi = np.maximum(left, right).astype(np.float64) + 1.0
    lo = np.minimum(left, right).astype(np.float64) + 1.0
    score = hi / lo
    if floor_q > 0.0:
        score = np.where(np.maximum(left, right).astype(np.float64) < floor_q, -np.inf, score)
    return score


def select_cuts(scores: np.ndarray, max_segments: int = MAX_SEGMENTS, tau: float = TAU) -> List[int]:
    """R5: greedy change-point selection; returns the sorted cut positions t.  Candidates scoring
    -inf (below the variance floor) are never taken."""
    alive = np.isfinite(scores)
    cuts: List[int] = []
    for _ in range(max(0, max_segments - 1)):
        if not alive.any():
            break
        masked = np.where(alive, scores, -np.inf)
        i = int(np.argmax(masked))            # first occurrence = smallest t among ties
        if cuts and not masked[i] >= tau:
            break
        cuts.append(WIN + i)
        alive[max(0, i - (WIN - 1)):i + WIN] = False
    return sorted(cuts)


def length_aware_cap(length: int) -> int:
    """R12, DGQ article 3.2: the most segments a sequence of `length` tokens may get."""
    if length < 2048:
        return 2
    if length < 16384:
        return 3
    return min(5, int(math.floor(math.log2(length / 1024))) + 2)


def segment_starts(k16: np.ndarray, max_segments: int = MAX_SEGMENTS, tau: float = TAU,
                   min_var: float = 0.0, length_aware: bool = False) -> List[int]:
    """Segment start positions of one head's keys ([] for an empty sequence)."""
    length, head_dim = k16.shape
    if length == 0:
        return []
    if length_aware:
        max_segments = min(max_segments, length_aware_cap(length))
    if length < 2 * WIN or max_segments <= 1:
        return [0]
    a, b = token_moments(k16)
    scores = change_scores(window_q(a, b, head_dim), length, variance_floor_q(min_var, head_dim))
    return [0] + select_cuts(scores, max_segments, tau)


@dataclasses.dataclass
class SegParams:
    start: int
    kmin: np.float32
    kmax: np.float32
    vmin: np.float32
    vmax: np.float32
    levels: int = CODE_LEVELS

    @property
    def kscale(self) -> np.float32:
        return quant_scale(self.kmin, self.kmax, self.levels)

    @property
    def vscale(self) -> np.float32:
        return quant_scale(self.vmin, self.vmax, self.levels)


def quant_scale(mn, mx, levels: int = CODE_LEVELS) -> np.float32:
    """R8 (R13): step between adjacent codes, fp32((max - min) / levels)."""
    diff = np.float32(np.float32(mx) - np.float32(mn))
    return np.float32(diff / np.float32(levels))


def quant_inv(mn, mx, levels: int = CODE_LEVELS) -> np.float32:
    """R8 (R13): fp32(levels / (max - min)), or 0 for a constant range."""
    diff = np.float32(np.float32(mx) - np.float32(mn))
    if not diff > 0:
        return np.float32(0.0)
    return np.float32(np.float32(levels) / diff)


def range_of(x16: np.ndarray):
    """Min and max of a block of values (canonical float32)."""
    x = canonical_f32(x16)
    return np.float32(x.min()), np.float32(x.max())


def segment_params(k16: np.ndarray, v16: np.ndarray, starts: List[int],
                   levels: int = CODE_LEVELS) -> List[SegParams]:
    """R6: each segment's own key and value min/max (DGQ article section 2.2)."""
    length = k16.shape[0]
    bounds = list(starts) + [length]
    out = []
    for j, s in enumerate(starts):
        e = bounds[j + 1]
        kmin, kmax = range_of(k16[s:e])
        vmin, vmax = range_of(v16[s:e])
        out.append(SegParams(s, kmin, kmax, vmin, vmax, levels))
    return out


def encode(x16: np.ndarray, mn, mx, fmt: str = "bitmap") -> np.ndarray:
    """R8 (R13): asymmetric INT8 codes of ``x16`` for the range [mn, mx] (Quantization article
    2.1): 255 steps from -128 in the bitmap format, 253 steps from -127 in the marker format."""
    levels, low = format_levels(fmt)
    x = canonical_f32(x16)
    inv = quant_inv(mn, mx, levels)
    d = (x - np.float32(mn)).astype(np.float32)
    u = (d * inv).astype(np.float32)
    c = np.clip(np.rint(u), 0, levels).astype(np.int16) + low
    return c.astype(np.int8)


def dequant(codes: np.ndarray, mn, scale, fmt: str = "bitmap") -> np.ndarray:
    """R9 (R13): float64 reconstruction (code - low) * scale + min, low = the code of the minimum
    (-128 bitmap, -127 marker)."""
    _, low = format_levels(fmt)
    return (codes.astype(np.float64) - float(low)) * np.float64(scale) + np.float64(mn)


def place_marker(code) -> np.int8:
    """R13: the marker that replaces a segment's first key byte (channel 0): 127 for a code in the
    upper half of the range, -128 for one in the lower half."""
    return np.int8(MARK_HIGH if int(code) >= 0 else MARK_LOW)


def marker_bits(kcodes: np.ndarray) -> np.ndarray:
    """R13: the identifier read back from the data: token t starts a segment iff its channel-0 key
    byte is one of the two marker values."""
    first = np.asarray(kcodes, np.int8).reshape(len(kcodes), -1)[:, 0]
    return (first == MARK_LOW) | (first == MARK_HIGH)


def boundary_bits(starts: List[int], length: int) -> np.ndarray:
    """R7: the 1-bit segment identifier per token (DGQ article section 2.2; separate tensor as in
    the original scheme of section 3.2)."""
    bits = np.zeros(length, dtype=bool)
    for s in starts[1:]:
        bits[s] = True
    return bits


@dataclasses.dataclass
class HeadCompressed:
    length: int
    segs: List[SegParams]
    kcodes: np.ndarray      # int8 [L][D]
    vcodes: np.ndarray      # int8 [L][D]
    bits: np.ndarray        # bool [L]: the identifier (a bit tensor in the bitmap format; read
                            # from the marker bytes of kcodes in the marker format)
    fmt: str = "bitmap"

    @property
    def starts(self) -> List[int]:
        return [s.start for s in self.segs]

    def seg_of(self) -> np.ndarray:
        """Segment index of every token."""
        idx = np.zeros(self.length, dtype=np.int64)
        for j, s in enumerate(self.segs):
            idx[s.start:] = j
        return idx

    def khat(self) -> np.ndarray:
        return _dequant_by_segment(self.kcodes, self.segs, "k", self.fmt)

    def vhat(self) -> np.ndarray:
        return _dequant_by_segment(self.vcodes, self.segs, "v", self.fmt)


def _dequant_by_segment(codes, segs, which, fmt="bitmap"):
    out = np.empty(codes.shape, dtype=np.float64)
    bounds = [s.start for s in segs] + [codes.shape[0]]
    for j, s in enumerate(segs):
        mn = s.kmin if which == "k" else s.vmin
        sc = s.kscale if which == "k" else s.vscale
        out[bounds[j]:bounds[j + 1]] = dequant(codes[bounds[j]:bounds[j + 1]], mn, sc, fmt)
    return out


def encode_by_segment(x16: np.ndarray, segs: List[SegParams], which: str, fmt: str = "bitmap") -> np.ndarray:
    """Codes of a whole head, each token with its own segment's range; in the marker format the
    first key byte of every segment but the first is its marker (R13)."""
    out = np.empty(x16.shape, dtype=np.int8)
    bounds = [s.start for s in segs] + [x16.shape[0]]
    for j, s in enumerate(segs):
        mn, mx = (s.kmin, s.kmax) if which == "k" else (s.vmin, s.vmax)
        out[bounds[j]:bounds[j + 1]] = encode(x16[bounds[j]:bounds[j + 1]], mn, mx, fmt)
    if fmt == "marker" and which == "k":
        for s in segs[1:]:
            if s.start < x16.shape[0]:
                out[s.start, 0] = place_marker(out[s.start, 0])
    return out


def compress_head(k16: np.ndarray, v16: np.ndarray, max_segments: int = MAX_SEGMENTS,
                  tau: float = TAU, min_var: float = 0.0, length_aware: bool = False,
                  fmt: str = "bitmap") -> HeadCompressed:
    """The whole DGQ compression of one (sequence, kv head): cuts, params, codes, identifier."""
    k16 = np.asarray(k16, dtype=np.float16)
    v16 = np.asarray(v16, dtype=np.float16)
    if not (np.isfinite(k16).all() and np.isfinite(v16).all()):
        raise ValueError("DGQ compression needs finite inputs")
    length = k16.shape[0]
    levels, _ = format_levels(fmt)
    starts = segment_starts(k16, max_segments, tau, min_var, length_aware)
    segs = segment_params(k16, v16, starts, levels)
    return HeadCompressed(length, segs, encode_by_segment(k16, segs, "k", fmt),
                          encode_by_segment(v16, segs, "v", fmt), boundary_bits(starts, length), fmt)


# ----------------------------------------------------------------------------------------------
# Streaming append: re-decide only the tail block (R11)
# ----------------------------------------------------------------------------------------------

def pair_score(q_left: int, q_right: int) -> float:
    """R4 applied to two windows."""
    return float(np.float64(max(q_left, q_right) + 1) / np.float64(min(q_left, q_right) + 1))


def window_q_of(a_list, b_list, head_dim: int) -> int:
    """R3 for one 16-token window given its tokens' moments."""
    sa = int(sum(int(x) for x in a_list))
    sb = int(sum(int(x) for x in b_list))
    return WIN * head_dim * sb - sa * sa


class AppendState:
    """One (sequence, kv head) after ``compress_head``, advanced one token at a time.

    The open span is [r0, L): the tokens appended into the current tail block since it was last
    sealed (r0 = the compressed length at first).  Tokens before r0 are frozen.  On every append:

    1. the token joins the open span;
    2. S = the segment holding token r0 - 1 (the base segment);
    3. the span needs its own segment if it already has one, or if the table is empty, or if any
       span key lies outside [S.kmin, S.kmax] or any span value outside [S.vmin, S.vmax], or if the
       span has 16 tokens, the ring holds the 16 tokens before r0, the score of (ring window,
       first 16 span tokens) is >= tau and (R12) not both windows are below the variance floor;
    4. if so, the span is a segment starting at r0 whose min/max cover the span (bit r0 set when
       r0 > 0); with a full table it joins S instead, codes saturate, and the clamp counter goes
       up by one for this append;
    5. every span token is re-encoded with the chosen segment's range;
    6. when L reaches a multiple of the block size the span is sealed: r0 = L, the ring keeps the
       moments of the last 16 tokens.

    The decision can only move from "join" to "own segment" (range violations stay in the span,
    the window test is fixed once the span has 16 tokens), so frozen codes never change.
    """

    def __init__(self, comp: HeadCompressed, k16_prefix: np.ndarray, block_size: int,
                 seg_capacity: int = SEG_CAPACITY, tau: float = TAU, min_var: float = 0.0):
        self.fmt = comp.fmt
        self.levels, _ = format_levels(comp.fmt)
        self.head_dim = comp.kcodes.shape[1]
        self.floor_q = variance_floor_q(min_var, self.head_dim)
        self.block_size = block_size
        self.capacity = seg_capacity
        self.tau = tau
        self.length = comp.length
        self.segs: List[SegParams] = [dataclasses.replace(s) for s in comp.segs]
        self.kcodes = [row for row in comp.kcodes]
        self.vcodes = [row for row in comp.vcodes]
        self.bits = list(comp.bits)
        self.r0 = comp.length
        a, b = token_moments(np.asarray(k16_prefix, dtype=np.float16).reshape(-1, self.head_dim))
        keep = min(WIN, comp.length)
        self.ring_a = [int(x) for x in a[comp.length - keep:]]
        self.ring_b = [int(x) for x in b[comp.length - keep:]]
        self.stage_k: List[np.ndarray] = []
        self.stage_v: List[np.ndarray] = []
        self.span_own = False
        self.clamped = 0

    def _base(self) -> Optional[SegParams]:
        """The segment before the open span, or None when the span starts the sequence."""
        before = self.segs[:-1] if self.span_own else self.segs
        return before[-1] if before else None

    def append(self, k_row: np.ndarray, v_row: np.ndarray) -> None:
        k_row = np.asarray(k_row, dtype=np.float16).reshape(self.head_dim)
        v_row = np.asarray(v_row, dtype=np.float16).reshape(self.head_dim)
        if not (np.isfinite(k_row).all() and np.isfinite(v_row).all()):
            raise ValueError("DGQ append needs finite inputs")
        self.stage_k.append(k_row)
        self.stage_v.append(v_row)
        self.length += 1
        self.kcodes.append(np.zeros(self.head_dim, dtype=np.int8))
        self.vcodes.append(np.zeros(self.head_dim, dtype=np.int8))
        self.bits.append(False)
        span_k = np.stack(self.stage_k)
        span_v = np.stack(self.stage_v)

        base = self._base()
        if self.span_own or base is None:
            want_own = True
        else:
            kmn, kmx = range_of(span_k)
            vmn, vmx = range_of(span_v)
            want_own = bool(kmn < base.kmin or kmx > base.kmax or vmn < base.vmin or vmx > base.vmax)
            if not want_own and len(self.stage_k) >= WIN and len(self.ring_a) == WIN:
                a, b = token_moments(span_k[:WIN])
                q_left = window_q_of(self.ring_a, self.ring_b, self.head_dim)
                q_right = window_q_of(a, b, self.head_dim)
                above_floor = not (float(np.float64(max(q_left, q_right))) < self.floor_q)
                want_own = above_floor and pair_score(q_left, q_right) >= self.tau

        if want_own and not self.span_own:
            if len(self.segs) >= self.capacity:
                self.clamped += 1
                want_own = False
            else:
                kmn, kmx = range_of(span_k)
                vmn, vmx = range_of(span_v)
                self.segs.append(SegParams(self.r0, kmn, kmx, vmn, vmx, self.levels))
                self.span_own = True
                if self.r0 > 0:
                    self.bits[self.r0] = True
        elif want_own and self.span_own:
            kmn, kmx = range_of(span_k)
            vmn, vmx = range_of(span_v)
            self.segs[-1] = SegParams(self.r0, kmn, kmx, vmn, vmx, self.levels)

        seg = self.segs[-1] if self.span_own else base
        kc = encode(span_k, seg.kmin, seg.kmax, self.fmt)
        vc = encode(span_v, seg.vmin, seg.vmax, self.fmt)
        if self.fmt == "marker" and self.span_own and self.r0 > 0:
            kc[0, 0] = place_marker(kc[0, 0])          # R13: the span's segment starts at r0
        for i in range(len(self.stage_k)):
            self.kcodes[self.r0 + i] = kc[i]
            self.vcodes[self.r0 + i] = vc[i]

        if self.length % self.block_size == 0:
            a, b = token_moments(span_k)
            self.ring_a = (self.ring_a + [int(x) for x in a])[-WIN:]
            self.ring_b = (self.ring_b + [int(x) for x in b])[-WIN:]
            self.r0 = self.length
            self.stage_k, self.stage_v = [], []
            self.span_own = False

    def snapshot(self) -> HeadCompressed:
        return HeadCompressed(self.length, [dataclasses.replace(s) for s in self.segs],
                              np.stack(self.kcodes) if self.kcodes else np.zeros((0, self.head_dim), np.int8),
                              np.stack(self.vcodes) if self.vcodes else np.zeros((0, self.head_dim), np.int8),
                              np.asarray(self.bits, dtype=bool), self.fmt)


# ----------------------------------------------------------------------------------------------
# Fixed 64-channel group INT8 baseline: DGQ article section 2.2 (the LLM.int8()-style scheme it
# compares against: every 64-dim chunk of a token has its own min/max)
# ----------------------------------------------------------------------------------------------

GROUP = 64


def group64_compress(x16: np.ndarray):
    """Codes int8 [L][D] and per-(token, group) min/max float16 [L][D/64] of one head: R8 applied
    to every 64-channel group of every token with that group's own range."""
    x16 = np.asarray(x16, dtype=np.float16)
    length, head_dim = x16.shape
    ng = head_dim // GROUP
    x = canonical_f32(x16).reshape(length, ng, GROUP)
    mn = x.min(axis=2)
    mx = x.max(axis=2)
    diff = (mx - mn).astype(np.float32)
    with np.errstate(divide="ignore"):
        inv = np.where(diff > 0, np.float32(CODE_LEVELS) / diff, np.float32(0.0)).astype(np.float32)
    d = (x - mn[:, :, None]).astype(np.float32)
    u = (d * inv[:, :, None]).astype(np.float32)
    codes = (np.clip(np.rint(u), 0, CODE_LEVELS).astype(np.int16) - 128).astype(np.int8)
    return codes.reshape(length, head_dim), mn.astype(np.float16), mx.astype(np.float16)


def group64_dequant(codes: np.ndarray, gmin: np.ndarray, gmax: np.ndarray) -> np.ndarray:
    """R9 per (token, group)."""
    length, head_dim = codes.shape
    ng = head_dim // GROUP
    mn = np.asarray(gmin, np.float16).astype(np.float32)
    mx = np.asarray(gmax, np.float16).astype(np.float32)
    scale = ((mx - mn).astype(np.float32) / np.float32(CODE_LEVELS)).astype(np.float32)
    c = codes.reshape(length, ng, GROUP).astype(np.float64)
    out = (c + 128.0) * scale.astype(np.float64)[:, :, None] + mn.astype(np.float64)[:, :, None]
    return out.reshape(length, head_dim)


# ----------------------------------------------------------------------------------------------
# Decode attention over the cache (PagedAttention article, paged forward pass; R10)
# ----------------------------------------------------------------------------------------------

def decode_attention(q16: np.ndarray, khat: np.ndarray, vhat: np.ndarray,
                     softmax_scale: Optional[float] = None) -> np.ndarray:
    """One decode query per query head against one kv head's cache, float64.

    q16 [G][D] (the query heads that share this kv head), khat/vhat [L][D] -> out [G][D].
    An empty cache gives zeros.
    """
    q = np.asarray(q16, dtype=np.float16).astype(np.float64)
    length, head_dim = khat.shape
    if length == 0:
        return np.zeros((q.shape[0], head_dim))
    scale = 1.0 / math.sqrt(head_dim) if softmax_scale is None else float(softmax_scale)
    s = scale * (khat @ q.T)                       # [L][G]
    p = np.exp(s - s.max(axis=0, keepdims=True))
    return (p.T @ vhat) / p.sum(axis=0)[:, None]


def rel_err(out: np.ndarray, ref: np.ndarray) -> float:
    """max over query heads of ||out - ref||_inf / ||ref||_inf (the acceptance metric)."""
    out = np.asarray(out, dtype=np.float64).reshape(-1, ref.shape[-1])
    ref = np.asarray(ref, dtype=np.float64).reshape(-1, ref.shape[-1])
    num = np.abs(out - ref).max(axis=1)
    den = np.maximum(np.abs(ref).max(axis=1), 1e-30)
    return float((num / den).max())


# ----------------------------------------------------------------------------------------------
# Byte accounting: DGQ article section 3.3 memory formula
# ----------------------------------------------------------------------------------------------

def page_formula_bytes(num_layers: int, num_heads: int, head_dim: int, seq_len: int):
    """(fp16 bytes, DGQ bytes) exactly as the formula states: K and V at 2 bytes each, versus
    1 byte per element plus 0.125 byte (1 bit) per token per head per layer."""
    fp16 = 2 * num_layers * num_heads * head_dim * seq_len * 2
    dgq = 2 * num_layers * num_heads * head_dim * seq_len * 1 + num_layers * num_heads * seq_len * 0.125
    return fp16, dgq


def compressed_bytes(lengths, num_kv_heads: int, head_dim: int, seg_counts=None, entry_bytes: int = 32,
                     fmt: str = "bitmap"):
    """Bytes the compressed cache of one layer uses: codes, bits (none in the marker format, R13),
    and (if given) the segment tables, which the page's formula leaves out."""
    format_levels(fmt)
    total_tokens = int(np.sum(lengths))
    codes = 2 * total_tokens * num_kv_heads * head_dim
    bits = total_tokens * num_kv_heads / 8.0 if fmt == "bitmap" else 0.0
    params = 0 if seg_counts is None else int(np.sum(seg_counts)) * entry_bytes
    return {"codes": codes, "bits": bits, "params": params}
