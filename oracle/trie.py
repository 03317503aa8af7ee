"""Append-only record arena addressed by parent indices (oracle).

Follows:
* Engineering Exploration of Generative Recall, §4.4 Tree-Based Attention:
  beam candidates live in a trie, a shared prefix is stored once, and a token
  sees only the ancestors on its own branch.
* OneLA (Abstract): every beam is the shared prompt plus compact, append-only
  records of its own divergent transitions; a light ancestry index says which
  records make up a beam's history, and beams advance without moving or copying
  records that already exist.

Representation (one request r): records k[r][n], v[r][n] ([H][d] each) and
parent[r][n] in [-1, n): -1 means "child of the prompt".  A chain is the list
of nodes from the root-most record down to a beam's own record.
"""
from __future__ import annotations

import numpy as np


class TrieError(ValueError):
    """Invalid trie data: a parent outside [-1, own id), a node outside the
    arena, a parent-beam index outside the previous level, or a chain longer
    than the allowed depth."""


def new_arena(R: int, capacity: int, H: int, d: int):
    """Empty arena: k, v zero [R][capacity][H][d] float32, parent -1."""
    k = np.zeros((R, capacity, H, d), np.float32)
    v = np.zeros((R, capacity, H, d), np.float32)
    parent = np.full((R, capacity), -1, np.int32)
    return k, v, parent


def trie_append(arena_k, arena_v, parent, base, k_new, v_new,
                parent_beam=None, prev_nodes=None):
    """Append one record per new beam j at node base + j (OneLA Abstract:
    append-only records; existing records are neither moved nor copied).

    k_new, v_new: [R][n_new][H][d].  parent_beam: [R][n_new] index into
    prev_nodes (which beam of the previous step the new beam extends), or None
    for a first level whose records hang off the prompt.  prev_nodes:
    [R][n_prev] arena node of each previous beam.  Returns (arena_k, arena_v,
    parent, node_out) as new arrays; node_out[r][j] = base + j.
    """
    arena_k = arena_k.copy()
    arena_v = arena_v.copy()
    parent = parent.copy()
    R, n_new = k_new.shape[0], k_new.shape[1]
    cap = parent.shape[1]
    if base < 0 or base + n_new > cap:
        raise TrieError("append past arena capacity")
    node_out = np.zeros((R, n_new), np.int32)
    for r in range(R):
        for j in range(n_new):
            n = base + j
            arena_k[r, n] = k_new[r, j]
            arena_v[r, n] = v_new[r, j]
            if parent_beam is None:
                p = -1
            else:
                pb = int(parent_beam[r, j])
                if not 0 <= pb < prev_nodes.shape[1]:
                    raise TrieError("parent beam outside the previous level")
                p = int(prev_nodes[r, pb])
                if not -1 <= p < n:
                    raise TrieError("parent id must lie in [-1, own id)")
            parent[r, n] = p
            node_out[r, j] = n
    return arena_k, arena_v, parent, node_out


def chain(parent_row: np.ndarray, node: int, max_depth: int):
    """Nodes on the branch of `node`, root-most first, ending with `node`
    itself (§4.4: a token attends to the ancestors of its own branch only).
    Raises TrieError on an out-of-range id, a parent that is not older than
    its child, or more than `max_depth` records."""
    cap = parent_row.shape[0]
    nodes = []
    n = int(node)
    while n != -1:
        if not 0 <= n < cap:
            raise TrieError("node id outside the arena")
        nodes.append(n)
        if len(nodes) > max_depth:
            raise TrieError("chain longer than max_depth")
        p = int(parent_row[n])
        if not -1 <= p < n:
            raise TrieError("parent id must lie in [-1, own id)")
        n = p
    return nodes[::-1]
