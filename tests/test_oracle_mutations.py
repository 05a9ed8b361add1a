"""Plant plausible mistakes in the CPU oracle (on the CPU, via monkeypatch) and check that the
pins catch every one: a dropped term, an off-by-one window, a wrong tie rule, a transposed
operand, a wrong rounding, swapped K/V, a missing scale."""

import math

import numpy as np
import pytest

import oracle_pins as P
from oracle import dgq_oracle as O


def _window_q_short(a, b, head_dim):
    length = len(a)
    if length < O.WIN:
        return np.zeros(0, dtype=np.int64)
    w = O.WIN - 1
    ca = np.concatenate([[0], np.cumsum(a)])
    cb = np.concatenate([[0], np.cumsum(b)])
    sa = ca[w:] - ca[:-w]
    sb = cb[w:] - cb[:-w]
    return (O.WIN * head_dim * sb - sa * sa)[:length - O.WIN + 1]


def _window_q_no_square(a, b, head_dim):
    ca = np.concatenate([[0], np.cumsum(a)])
    cb = np.concatenate([[0], np.cumsum(b)])
    return O.WIN * head_dim * (cb[O.WIN:] - cb[:-O.WIN]) - (ca[O.WIN:] - ca[:-O.WIN])


def _scores_shifted(q, length, floor_q=0.0):
    if length < 2 * O.WIN:
        return np.zeros(0)
    left = q[1:length - 2 * O.WIN + 2]
    right = q[O.WIN:length - O.WIN + 1]
    n = min(len(left), len(right))
    left, right = left[:n], right[:n]
    return (np.maximum(left, right) + 1.0) / (np.minimum(left, right) + 1.0)


def _scores_no_plus_one(q, length, floor_q=0.0):
    if length < 2 * O.WIN:
        return np.zeros(0)
    left = q[0:length - 2 * O.WIN + 1].astype(np.float64)
    right = q[O.WIN:length - O.WIN + 1].astype(np.float64)
    with np.errstate(divide="ignore", invalid="ignore"):
        return np.maximum(left, right) / np.minimum(left, right)


def _select_largest_t(scores, max_segments=5, tau=2.0):
    alive = np.ones(len(scores), dtype=bool)
    cuts = []
    for _ in range(max(0, max_segments - 1)):
        if not alive.any():
            break
        masked = np.where(alive, scores, -np.inf)
        i = len(masked) - 1 - int(np.argmax(masked[::-1]))
        if cuts and not masked[i] >= tau:
            break
        cuts.append(O.WIN + i)
        alive[max(0, i - (O.WIN - 1)):i + O.WIN] = False
    return sorted(cuts)


def _select_wide_suppression(scores, max_segments=5, tau=2.0):
    alive = np.ones(len(scores), dtype=bool)
    cuts = []
    for _ in range(max(0, max_segments - 1)):
        if not alive.any():
            break
        masked = np.where(alive, scores, -np.inf)
        i = int(np.argmax(masked))
        if cuts and not masked[i] >= tau:
            break
        cuts.append(O.WIN + i)
        alive[max(0, i - O.WIN):i + O.WIN + 1] = False
    return sorted(cuts)


def _select_strict_tau(scores, max_segments=5, tau=2.0):
    alive = np.ones(len(scores), dtype=bool)
    cuts = []
    for _ in range(max(0, max_segments - 1)):
        if not alive.any():
            break
        masked = np.where(alive, scores, -np.inf)
        i = int(np.argmax(masked))
        if cuts and not masked[i] > tau:
            break
        cuts.append(O.WIN + i)
        alive[max(0, i - (O.WIN - 1)):i + O.WIN] = False
    return sorted(cuts)


def _scale_256(mn, mx, levels=O.CODE_LEVELS):
    return np.float32(np.float32(np.float32(mx) - np.float32(mn)) / np.float32(256))


def _inv_256(mn, mx, levels=O.CODE_LEVELS):
    diff = np.float32(np.float32(mx) - np.float32(mn))
    return np.float32(0) if not diff > 0 else np.float32(np.float32(256) / diff)


def _encode_floor(x16, mn, mx, fmt="bitmap"):
    levels, low = O.format_levels(fmt)
    x = O.canonical_f32(x16)
    inv = O.quant_inv(mn, mx, levels)
    u = ((x - np.float32(mn)) * inv).astype(np.float32)
    return (np.clip(np.floor(u), 0, levels).astype(np.int16) + low).astype(np.int8)


def _dequant_no_offset(codes, mn, scale, fmt="bitmap"):
    return codes.astype(np.float64) * np.float64(scale) + np.float64(mn)


def _params_swapped(k16, v16, starts, levels=O.CODE_LEVELS):
    return O.__dict__["_orig_segment_params"](v16, k16, starts, levels)


def _levels_marker_255(fmt):
    return (O.CODE_LEVELS, -128)


def _encode_by_segment_marker_on_v(x16, segs, which, fmt="bitmap"):
    """Mistake: the markers go into the value bytes instead of the key bytes."""
    out = O.__dict__["_orig_encode_by_segment"](x16, segs, which, fmt)
    if fmt != "marker":
        return out
    for s in segs[1:]:
        if which == "k":
            out[s.start, 0] = O.encode(x16[s.start:s.start + 1, :1], s.kmin, s.kmax, fmt)[0, 0]
        else:
            out[s.start, 0] = O.place_marker(out[s.start, 0])
    return out


def _dequant_marker_offset_128(codes, mn, scale, fmt="bitmap"):
    return (codes.astype(np.float64) + 128.0) * np.float64(scale) + np.float64(mn)


def _place_marker_inverted(code):
    return np.int8(O.MARK_LOW if int(code) >= 0 else O.MARK_HIGH)


class _AppendNoMarker(O.AppendState):
    """Mistake: the span's own segment gets no marker in the marker format."""

    def append(self, k_row, v_row):
        r0 = self.r0
        super().append(k_row, v_row)
        if self.fmt == "marker" and r0 > 0 and self.r0 == r0 and self.span_own:
            seg = self.segs[-1]
            self.kcodes[r0] = O.encode(np.asarray(self.stage_k[0]).reshape(1, -1), seg.kmin, seg.kmax, self.fmt)[0]


def _attention_no_scale(q16, khat, vhat, softmax_scale=None):
    return O.__dict__["_orig_decode_attention"](q16, khat, vhat, softmax_scale=1.0)


def _attention_values_are_keys(q16, khat, vhat, softmax_scale=None):
    return O.__dict__["_orig_decode_attention"](q16, khat, khat, softmax_scale)


def _attention_no_max_shift(q16, khat, vhat, softmax_scale=None):
    q = np.asarray(q16, np.float64)
    scale = 1.0 / math.sqrt(khat.shape[1])
    s = scale * (khat @ q.T)
    p = np.exp(s)
    return (p.T @ vhat) / p.sum(axis=0)[:, None] * 1.0000001


def _bits_with_first(starts, length):
    bits = np.zeros(length, dtype=bool)
    for s in starts:
        bits[s] = True
    return bits


def _fixed_point_clamp16(x16):
    x = O.canonical_f32(x16).astype(np.float64)
    return np.rint(np.clip(x, -16, 16) * O.FP_SCALE).astype(np.int64)


def _fixed_point_trunc(x16):
    x = O.canonical_f32(x16).astype(np.float64)
    return np.trunc(np.clip(x, -O.FP_CLAMP, O.FP_CLAMP) * O.FP_SCALE).astype(np.int64)


class _AppendNoReencode(O.AppendState):
    """Mistake: only the newest token is encoded, even when the span's range changes."""

    def append(self, k_row, v_row):
        keep_k = [c.copy() for c in self.kcodes]
        keep_v = [c.copy() for c in self.vcodes]
        super().append(k_row, v_row)
        n = len(keep_k)
        for i in range(n):
            self.kcodes[i] = keep_k[i]
            self.vcodes[i] = keep_v[i]


def _scores_floor_on_min(q, length, floor_q=0.0):
    if length < 2 * O.WIN:
        return np.zeros(0)
    left = q[0:length - 2 * O.WIN + 1]
    right = q[O.WIN:length - O.WIN + 1]
    sc = (np.maximum(left, right) + 1.0) / (np.minimum(left, right) + 1.0)
    return np.where(np.minimum(left, right) < floor_q, -np.inf, sc) if floor_q > 0 else sc


def _cap_inclusive(length):
    if length <= 2048:
        return 2
    if length <= 16384:
        return 3
    return min(5, int(math.floor(math.log2(length / 1024))) + 2)



def _g64_dequant_offset_127(codes, gmin, gmax):
    length, head_dim = codes.shape
    ng = head_dim // O.GROUP
    mn = np.asarray(gmin, np.float16).astype(np.float32)
    mx = np.asarray(gmax, np.float16).astype(np.float32)
    scale = ((mx - mn) / np.float32(O.CODE_LEVELS)).astype(np.float32)
    c = codes.reshape(length, ng, O.GROUP).astype(np.float64)
    return ((c + 127.0) * scale[:, :, None] + mn[:, :, None]).reshape(length, head_dim)


def _g64_dequant_levels_256(codes, gmin, gmax):
    length, head_dim = codes.shape
    ng = head_dim // O.GROUP
    mn = np.asarray(gmin, np.float16).astype(np.float32)
    mx = np.asarray(gmax, np.float16).astype(np.float32)
    scale = ((mx - mn) / np.float32(256)).astype(np.float32)
    c = codes.reshape(length, ng, O.GROUP).astype(np.float64)
    return ((c + 128.0) * scale[:, :, None] + mn[:, :, None]).reshape(length, head_dim)


def _canonical_keeps_negative_zero(x16):
    return np.asarray(x16, dtype=np.float16).astype(np.float32)


MUTATIONS = {
    "variance_floor_on_min_window": ("change_scores", _scores_floor_on_min, [P.check_min_var_floor]),
    "length_cap_inclusive_edges": ("length_aware_cap", _cap_inclusive, [P.check_length_cap]),
    "window_15_tokens": ("window_q", _window_q_short, [P.check_window_q_against_variance]),
    "window_drops_square": ("window_q", _window_q_no_square, [P.check_window_q_against_variance]),
    "score_left_window_shift": ("change_scores", _scores_shifted, [P.check_scores_closed_form, P.check_step_change_cut]),
    "score_without_plus_one": ("change_scores", _scores_no_plus_one, [P.check_scores_closed_form]),
    "ties_to_largest_t": ("select_cuts", _select_largest_t, [P.check_selection_twin]),
    "suppression_radius_16": ("select_cuts", _select_wide_suppression, [P.check_selection_twin]),
    "tau_strict": ("select_cuts", _select_strict_tau, [P.check_selection_twin]),
    "scale_over_256": ("quant_scale", _scale_256, [P.check_codes, P.check_dequant_closed_form]),
    "inv_256": ("quant_inv", _inv_256, [P.check_codes]),
    "encode_floor": ("encode", _encode_floor, [P.check_codes]),
    "dequant_without_offset": ("dequant", _dequant_no_offset, [P.check_codes, P.check_dequant_closed_form]),
    "k_v_swapped": ("segment_params", _params_swapped, [P.check_minmax_library]),
    "attention_no_scale": ("decode_attention", _attention_no_scale, [P.check_attention]),
    "attention_values_are_keys": ("decode_attention", _attention_values_are_keys, [P.check_attention]),
    "attention_no_max_shift": ("decode_attention", _attention_no_max_shift, [P.check_attention]),
    "bit_on_first_token": ("boundary_bits", _bits_with_first, [P.check_bits]),
    "fixed_point_clamp_16": ("fixed_point", _fixed_point_clamp16, [P.check_fixed_point]),
    "fixed_point_truncates": ("fixed_point", _fixed_point_trunc, [P.check_fixed_point]),
    "append_keeps_stale_codes": ("AppendState", _AppendNoReencode, [P.check_append_cut]),
    "marker_format_255_levels": ("format_levels", _levels_marker_255, [P.check_marker_format]),
    "marker_on_value_bytes": ("encode_by_segment", _encode_by_segment_marker_on_v, [P.check_marker_format]),
    "marker_dequant_offset_128": ("dequant", _dequant_marker_offset_128, [P.check_marker_format]),
    "marker_choice_inverted": ("place_marker", _place_marker_inverted, [P.check_marker_format]),
    "append_without_marker": ("AppendState", _AppendNoMarker, [P.check_marker_append]),
    "g64_dequant_offset_127": ("group64_dequant", _g64_dequant_offset_127, [P.check_group64]),
    "g64_dequant_levels_256": ("group64_dequant", _g64_dequant_levels_256, [P.check_group64]),
    "no_negzero_canonicalization": ("canonical_f32", _canonical_keeps_negative_zero, [P.check_negative_zero]),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_mutation(name, monkeypatch):
    attr, fake, checks = MUTATIONS[name]
    monkeypatch.setitem(O.__dict__, "_orig_segment_params", O.segment_params)
    monkeypatch.setitem(O.__dict__, "_orig_decode_attention", O.decode_attention)
    monkeypatch.setitem(O.__dict__, "_orig_encode_by_segment", O.encode_by_segment)
    monkeypatch.setattr(O, attr, fake)
    caught = []
    for check in checks:
        try:
            check()
        except Exception as exc:  # AssertionError, or the mutated code breaking outright
            caught.append((check.__name__, type(exc).__name__))
    assert caught, f"no pin caught mutation {name}"
