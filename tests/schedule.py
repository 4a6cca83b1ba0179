"""Where the decode library stores its split-K partials: a reader of the
workspace contract that ``pda_workspace_layout`` documents in the C header.

This is not part of the method and not part of the oracle.  The pages fix only
that a sequence's KV may be cut into contiguous token ranges whose partials are
merged afterwards (KernelFlume paper §3.1, §3.2); how the library deals those
ranges to its work-groups is its own schedule, stated in the header: each
sequence's tokens are cut into units of P tokens (the last one shorter), the
units of all sequences in order form one stream of U units, and run w covers
units [w*k, (w+1)*k) with k = ceil(U / n_runs).  Tests use this to find each
stored partial, which the oracle then recomputes from the definition over the
same token range.
"""
from __future__ import annotations


def workspace_segments(context_lens, unit_tokens, n_runs):
    """One (w, b, tok_lo, tok_hi) per sequence b that run w touches, in stream order."""
    P = int(unit_tokens)
    nu = [-(-int(n) // P) for n in context_lens]
    U = sum(nu)
    if U == 0:
        return []
    k = -(-U // int(n_runs))
    before = [sum(nu[:b]) for b in range(len(nu))]
    out = []
    for w in range(int(n_runs)):
        u_lo, u_hi = w * k, min((w + 1) * k, U)
        for b, n in enumerate(context_lens):
            lo = max(u_lo, before[b]) - before[b]
            hi = min(u_hi, before[b] + nu[b]) - before[b]
            if hi > lo:
                out.append((w, b, lo * P, min(hi * P, int(n))))
    return out
