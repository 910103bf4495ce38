"""Oracle of which tokens a head's segment must store.

TEST INFRASTRUCTURE (see the package docstring of ``oracle``).

SegPagedAttention keeps KV pages per (layer, head) and per segment, and for
a head stores only the tokens that head needs ("Xiaohongshu Open-Sources
RedKnot" page, section "What Happened", item 3; "RedKnot: Head-Aware KV Reuse
and SegPagedAttention" page, section "The Three Core Mechanisms in Detail",
third mechanism).  The pages do not say when a token stops being needed; the
reading taken here:

* a global head needs every token;
* a local head with window W needs token j while some query that can still
  come may see it.  The earliest such query is the first of the ``n_query``
  tokens just appended (``kv_len - n_query``), or the next token to come when
  ``n_query`` is 0.  Queries at positions >= p_q see keys >= p_q - W + 1, so
  the head needs keys >= max(0, p_q - W + 1);
* storage is in whole pages of ``page_size`` tokens aligned to the logical
  token index, so the segment starts at that bound rounded down to a page.
"""

from __future__ import annotations


def earliest_pending_query(kv_len: int, n_query: int) -> int:
    if not 0 <= n_query <= kv_len:
        raise ValueError("need 0 <= n_query <= kv_len")
    return kv_len - n_query


def first_needed_token(kv_len: int, n_query: int, window: int) -> int:
    """Smallest key index any pending or future query can still see."""
    if window < 0:
        raise ValueError("window must be >= 0")
    if window == 0:
        return 0
    return max(0, earliest_pending_query(kv_len, n_query) - window + 1)


def segment_first_token(kv_len: int, n_query: int, window: int, page_size: int) -> int:
    """Logical index of the first token held by the segment's first page."""
    return page_size * (first_needed_token(kv_len, n_query, window) // page_size)


def segment_pages(kv_len: int, first_token: int, page_size: int) -> int:
    """Pages the segment holds for tokens [first_token, kv_len)."""
    if kv_len <= first_token:
        return 0
    return -(-(kv_len - first_token) // page_size)


def segment_after_appends(appends, window: int, page_size: int):
    """Follow a sequence of appends [(n_new, n_query), ...] of one head.

    The segment start never moves back: a token dropped earlier is gone.
    Returns (kv_len, first_token, n_pages) after the last append.
    """
    kv_len = 0
    first = 0
    for n_new, n_query in appends:
        if n_new < 0 or not 0 <= n_query <= n_new:
            raise ValueError("need n_new >= 0 and 0 <= n_query <= n_new")
        kv_len += n_new
        first = max(first, segment_first_token(kv_len, n_query, window, page_size))
    return kv_len, first, segment_pages(kv_len, first, page_size)
