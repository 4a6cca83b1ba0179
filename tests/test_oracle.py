"""The float64 oracle against its pins, and planted mistakes against the pins.

CPU only.  A planted mistake is patched into the oracle module for the length
of one test (pytest's monkeypatch), never into the library.
"""
import numpy as np
import pytest

import oracle.paged_attention as O
from tests import oracle_pins as pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_oracle_pin(pin):
    pin(O)


# --- planted mistakes: each must make at least one pin fail ---------------------

_attend = O.attend
_gather_blocks = O._gather_sequence_blocks
_merge = O.merge_partials
_ranges = O.partition_ranges
_token_location = O.token_location
_append = O.kv_append
_fp8 = O.fp8_e4m3_value
_fp8_encode = O.fp8_e4m3_encode
_append_fp8 = O.kv_append_fp8


def _encode_ties_away(x):
    """Round half away from zero instead of to the even code."""
    x = np.asarray(x, dtype=np.float64)
    c = _fp8_encode(x)
    pos = O.fp8_e4m3_decode(np.arange(0x7F))
    a = np.abs(x)
    i = np.clip(np.searchsorted(pos, a), 1, 0x7E)
    tie = (pos[i] - a == a - pos[i - 1]) & (a < 448)
    return np.where(tie, (i | (c & 0x80)).astype(np.uint8), c)


def _attend_lse_without_max(q_rows, K, V, scale):
    o, lse = _attend(q_rows, K, V, scale)
    if K.shape[0] == 0:
        return o, lse
    s = float(np.float32(scale)) * (np.asarray(q_rows, dtype=np.float64) @ K.T)
    return o, lse - s.max(axis=1)


def _merge_wrong_sign(o_parts, lse_parts):
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    L = np.max(lse_parts, axis=0)
    w = np.exp(np.where(np.isneginf(lse_parts), -np.inf, L[None] - lse_parts))
    o = (w[..., None] * np.asarray(o_parts)).sum(0) / w.sum(0)[..., None]
    return o, L + np.log(w.sum(0))


def _merge_unnormalised(o_parts, lse_parts):
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    L = lse_parts.max(axis=0)
    w = np.exp(lse_parts - L[None])
    o = (w[..., None] * np.asarray(o_parts)).sum(0)          # the division by sum(w) is missing
    return o, L + np.log(w.sum(0))


MUTANTS = {
    "slot_off_by_one": ("token_location", lambda row, t, bs=16: (int(row[t // bs]), (t + 1) % bs)),
    "frame_ignores_table": ("_gather_sequence_blocks",
                            lambda pool, row, n, g, bs: _gather_blocks(
                                pool, np.arange(len(row)), n, g, bs)),
    "gqa_modulo": ("kv_head_of", lambda h, nq, nkv: h % nkv),
    "scale_dropped": ("attend", lambda q, K, V, scale: _attend(q, K, V, 1.0)),
    "lse_without_max": ("attend", _attend_lse_without_max),
    "last_token_dropped": ("attend", lambda q, K, V, scale: _attend(q, K[:-1], V[:-1], scale)
                           if K.shape[0] > 1 else _attend(q, K, V, scale)),
    "merge_wrong_sign": ("merge_partials", _merge_wrong_sign),
    "merge_unnormalised": ("merge_partials", _merge_unnormalised),
    "append_one_slot_late": ("kv_append",
                             lambda k, v, kn, vn, bt, lens, bs=16: _append(
                                 k, v, kn, vn, bt, [n + 1 if 0 < n and n % bs else n for n in lens],
                                 bs)),
    "fp8_bias_8": ("fp8_e4m3_value",
                   lambda code: _fp8(code) / 2.0 if (int(code) >> 3) & 0xF else _fp8(code)),
    "fp8_encode_ties_away": ("fp8_e4m3_encode", _encode_ties_away),
    "append_fp8_times_scale": ("kv_append_fp8",
                               lambda k, v, kn, vn, bt, lens, ks, vs, bs=16: _append_fp8(
                                   k, v, kn, vn, bt, lens, 1.0 / ks, 1.0 / vs, bs)),
    "partition_end_short": ("partition_ranges",
                            lambda n, P: [(lo, max(lo, hi - 1)) if hi - lo > 1 else (lo, hi)
                                          for lo, hi in _ranges(n, P)]),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(O, attr, fn)
    failed = []
    for pin in pins.ALL_PINS:
        try:
            pin(O)
        except (AssertionError, FloatingPointError, ValueError, IndexError):
            failed.append(pin.__name__)
    assert failed, f"planted mistake {name!r} passed every pin"
