"""Token-level oracle of copy-on-write forks of per-head segments.

TEST INFRASTRUCTURE (see the package docstring of ``oracle``).

RedKnot's experimental multi-request shared KV manager lets requests fork
one another's per-head KV and applies copy-on-write when a request appends
or repairs ("RedKnot: Head-Aware KV Reuse and SegPagedAttention" page,
sections "Getting Started: Repository Layout and Entry Points" and
"Experimental Features and Current Limitations").  This model is the plain
definition of that behaviour for the segments of one layer:

* a page is a Python object whose slots hold the labels of the tokens
  stored in it.  Two segments share a page iff they hold the same object;
* ``fork(src, dst)``: dst gets src's token history and references to the
  very same page objects of every KV head;
* ``append``: every KV head stores the new tokens its segment keeps (the
  storage rule of ``oracle.segments``: a local head drops the pages wholly
  below its window start).  Before a token is written into an existing page
  that another segment also holds, the writer replaces its reference with a
  private copy of that page (copy-on-write);
* ``release(seq)``: drops the sequence's references.

A page is in use while some segment holds it; ``pages_in_use`` counts the
distinct objects.  The readings: sharing is per page of one (layer, KV
head) segment, and a copy is made only for a page that will be written.
"""

from __future__ import annotations

from . import segments as SG


class Page:
    __slots__ = ("slots",)

    def __init__(self, page_size: int):
        self.slots = [None] * page_size

    def copy(self) -> "Page":
        p = Page(len(self.slots))
        p.slots = list(self.slots)
        return p


class ForkModel:
    def __init__(self, windows, page_size: int):
        self.windows = tuple(windows)
        self.P = page_size
        self.history = {}   # seq -> list of token labels
        self.pending = {}   # seq -> earliest pending query position
        self.segs = {}      # (seq, g) -> [first_token, [Page, ...]]

    # -- helpers -----------------------------------------------------------
    def _refs(self, page: Page) -> int:
        return sum(1 for _, pages in self.segs.values() for p in pages if p is page)

    def kv_len(self, seq) -> int:
        return len(self.history.get(seq, ()))

    # -- operations --------------------------------------------------------
    def append(self, seq, labels, n_query: int):
        hist = self.history.setdefault(seq, [])
        old = len(hist)
        hist.extend(labels)
        new = len(hist)
        for g, w in enumerate(self.windows):
            first, pages = self.segs.setdefault((seq, g), [0, []])
            if w > 0:
                start = max(first, SG.segment_first_token(new, n_query, w, self.P))
                drop = min(len(pages), (start - first) // self.P)
                del pages[:drop]
                first = start
            self.segs[(seq, g)][0] = first
            for j in range(max(old, first), new):
                idx = (j - first) // self.P
                if idx == len(pages):
                    pages.append(Page(self.P))
                elif self._refs(pages[idx]) > 1:
                    pages[idx] = pages[idx].copy()
                pages[idx].slots[(j - first) % self.P] = hist[j]
        self.pending[seq] = new - n_query

    def fork(self, src, dst):
        if self.kv_len(dst):
            raise ValueError("fork target must be empty")
        self.history[dst] = list(self.history.get(src, []))
        self.pending[dst] = self.pending.get(src, 0)
        for g in range(len(self.windows)):
            first, pages = self.segs.get((src, g), [0, []])
            self.segs[(dst, g)] = [first, list(pages)]

    def release(self, seq):
        self.history.pop(seq, None)
        self.pending.pop(seq, None)
        for g in range(len(self.windows)):
            self.segs.pop((seq, g), None)

    # -- queries -----------------------------------------------------------
    def pages_in_use(self) -> int:
        return len({id(p) for _, pages in self.segs.values() for p in pages})

    def segment(self, seq, g):
        """(first_token, kv_len, [Page, ...]) of one segment."""
        first, pages = self.segs.get((seq, g), [0, []])
        return first, self.kv_len(seq), list(pages)

    def stored_labels(self, seq, g):
        """The labels the segment's pages hold for tokens first .. kv_len-1."""
        first, n, pages = self.segment(seq, g)
        return [pages[(j - first) // self.P].slots[(j - first) % self.P] for j in range(first, n)]
