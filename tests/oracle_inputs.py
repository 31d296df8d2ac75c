"""Oracle inputs from the seeded generators (test side), and an independent dict trie."""
from __future__ import annotations

import numpy as np

from oracle.inputs import model_for, prefixes_for, request_for  # noqa: F401


def dict_trie(items: np.ndarray):
    """Dict-of-sets trie: prefix tuple -> set of next codes (independent of PrefixSet)."""
    t = {}
    for it in items.tolist():
        for s in range(len(it)):
            t.setdefault(tuple(it[:s]), set()).add(it[s])
    return t
