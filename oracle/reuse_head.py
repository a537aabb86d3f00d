"""Oracle model of the sparse-prefill dequant reuse ("head").

TEST INFRASTRUCTURE ONLY, like the rest of ``oracle/``: only the tests may
use it.

Written from sglang PR #45909 (summary): the layers that read one kv source
reuse its dequant.  The buffer's head remembers which source its rows hold,
keyed by (source cache, gather ids, row count); ``get_with_head`` returns the
rows and whether the head already held that source; a plain ``get``, a
reallocation of the buffer, or the start of a new forward forgets the head.
The skipped dequants would have written the same rows (the page's premise:
no later layer of the forward writes that cache), so a hit returns what a
fresh dequant of the same rows returns.

Reading: a miss runs the dequant and makes its key the head; a plain get
runs the dequant and leaves no head.  Keys are compared as given: the caller
names the source cache and the id list by identity tokens (for the C ABI,
its pointers and sizes).
"""
from __future__ import annotations

from typing import Callable, Hashable

import numpy as np


class SparsePrefillKVBuffer:
    """``dequant(source, ids, n)`` computes the rows (the oracle's gather);
    the buffer holds the last rows it produced."""

    def __init__(self, dequant: Callable[[Hashable, Hashable, int], np.ndarray]):
        self._dequant = dequant
        self.head = None
        self.rows = None

    def get_with_head(self, source: Hashable, ids: Hashable, n: int):
        """-> (rows, hit)"""
        key = (source, ids, n)
        if self.head == key:
            return self.rows, True
        self.rows = self._dequant(source, ids, n)
        self.head = key
        return self.rows, False

    def get(self, source: Hashable, ids: Hashable, n: int) -> np.ndarray:
        """a plain get: the dequant runs and the head is forgotten"""
        self.rows = self._dequant(source, ids, n)
        self.head = None
        return self.rows

    def reallocate(self) -> None:
        self.head = None
        self.rows = None

    def begin_forward(self) -> None:
        self.head = None
