"""Token-range ("segment") masks for decode (test infrastructure only).

Sources:
  * Declarative Attention post, "Declarative attention protocol": three modes
    -- global sees the whole context, focus sees only one named region, local
    sees only the model's own recent output; the kept token ranges are rounded
    outward to KV-block boundaries so whole blocks are read, costing at most a
    few dozen extra tokens per boundary; regions are ~2048-token chunks.
  * Million-token-context post, "Three modes, three reasoning states": the
    same three modes as KV-visibility sets.
  * LoZA post, "2. ZigZag architecture": streaming sparse attention over a
    fixed window (1024 tokens).
  * Million-token-context post, "Not a free lunch": among the safeguards, a
    minimum neighbourhood around the focused region.
Readings taken: "own recent output" = the last local_len cached tokens; focus
adds that local tail to the chunk; streaming keeps n_sink leading tokens plus
the last local_len tokens exactly (token level, no rounding); ranges are
sorted and overlapping or touching ranges are merged.
"""

SEG_GLOBAL, SEG_FOCUS, SEG_LOCAL, SEG_STREAMING = 0, 1, 2, 3


def _merge(ranges):
    out = []
    for a, b in sorted((a, b) for a, b in ranges if b > a):
        if out and a <= out[-1][1]:
            out[-1] = (out[-1][0], max(out[-1][1], b))
        else:
            out.append((a, b))
    return out


def _round_out(a, b, n, page):
    """[a, b) widened to page boundaries, clipped to [0, n)."""
    lo = (max(0, a) // page) * page
    hi = min(n, -(-b // page) * page)
    return lo, hi


def build_segments(mode, n, chunk_start=0, chunk_len=2048, local_len=1024, n_sink=4, page=16,
                   min_nb=0):
    """Sorted, merged [start, end) token ranges that `mode` admits for a
    sequence of n cached tokens.  min_nb: the focus chunk is first widened by
    min_nb tokens on each side (million-token-context post, "Not a free
    lunch": a minimum neighbourhood around the focused region as a
    safeguard; the post gives no size)."""
    if mode == SEG_GLOBAL:
        return [(0, n)]
    if mode == SEG_LOCAL:
        return _merge([_round_out(n - local_len, n, n, page)])
    if mode == SEG_FOCUS:
        return _merge([_round_out(chunk_start - min_nb, chunk_start + chunk_len + min_nb, n, page),
                       _round_out(n - local_len, n, n, page)])
    if mode == SEG_STREAMING:
        return _merge([(0, min(n_sink, n)), (max(0, n - local_len), n)])
    raise ValueError("unknown segment mode")
