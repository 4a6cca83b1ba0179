"""The multi-query and cascade oracle against its pins, and planted mistakes against them.

CPU only.  A planted mistake is patched into the oracle module for the length
of one test (pytest's monkeypatch), never into the library.
"""
import numpy as np
import pytest

import oracle.multi_query as MQ
import oracle.paged_attention as O
from tests import oracle_pins_mq as pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_oracle_pin(pin):
    pin(MQ, O)


_visible = MQ.visible_tokens
_cascade = MQ.cascade_attention
_reads = MQ.cascade_read_tokens
_mq = MQ.multi_query_attention


def _cascade_prefix_short(q, k, v, pt, pl, gs, st, sl, scale, bs=16):
    return _cascade(q, k, v, pt, [max(0, int(n) - 1) for n in pl], gs, st, sl, scale, bs)


def _mq_rows_shifted(q, k, v, table, lens, qs, scale, causal=True, bs=16):
    """Each sequence's queries read from the next row (wraps inside the sequence)."""
    q2 = np.array(q, copy=True)
    for s in range(len(lens)):
        a, b = int(qs[s]), int(qs[s + 1])
        if b - a > 1:
            q2[a:b] = np.roll(q[a:b], -1, axis=0)
    return _mq(q2, k, v, table, lens, qs, scale, causal, bs)


MUTANTS = {
    "causal_without_own_token": ("visible_tokens",
                                 lambda n, nq, i, causal: _visible(n, nq, i, causal) - 1
                                 if causal and _visible(n, nq, i, causal) > 0 else
                                 _visible(n, nq, i, causal)),
    "causal_from_chunk_start": ("visible_tokens",
                                lambda n, nq, i, causal: min(int(n), int(i) + 1) if causal
                                else int(n)),
    "mask_always_on": ("visible_tokens", lambda n, nq, i, causal: _visible(n, nq, i, True)),
    "gqa_modulo": ("kv_head_of", lambda h, nq, nkv: h % nkv),
    "cascade_prefix_short": ("cascade_attention", _cascade_prefix_short),
    "cascade_reads_without_suffix": ("cascade_read_tokens",
                                     lambda P, s: (len(s) * int(P), int(P))),
    "query_rows_shifted": ("multi_query_attention", _mq_rows_shifted),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(MQ, attr, fn)
    failed = []
    for pin in pins.ALL_PINS:
        try:
            pin(MQ, O)
        except (AssertionError, FloatingPointError, ValueError, IndexError):
            failed.append(pin.__name__)
    assert failed, f"planted mistake {name!r} passed every pin"
