"""Static sparse-tree buffers (the oracle of the host tree builder).

Follows "大模型推理 memory bandwidth bound (5) - Medusa", section 二.2
``generate_medusa_buffers()``: the tree is given as ``medusa_choices``, one rank
path per non-root node (e.g. ``(0, 1, 0)`` = rank-0 child of the root, then its
rank-1 child, then that node's rank-0 child).  From it the page derives, with a
printed 64-node example:

* the sorted choices (by depth, then lexicographically); node index = 1 +
  position in that order, the root is node 0;
* ``medusa_attn_mask`` -- node i may attend to node j iff j is an ancestor of i
  or i itself; the root column is all ones (section 一.2, and the 2-head figure:
  the query "is" on the path ["I", "is"] sees only its parent and itself);
* ``tree_indices`` -- where each node's token sits in the flat candidate list
  ``[root, head1 top-K, ..., headH top-K]``: ``1 + K*(depth-1) + last rank``;
* ``medusa_position_ids`` -- the depth of each node;
* ``retrieve_indices`` -- one row per root-to-leaf path, padded with -1.

Reading taken where the page is silent: the row order of ``retrieve_indices``
is by decreasing leaf node index (this reproduces the printed example exactly),
and the stride K is the top-K width, by default one more than the largest rank
used anywhere in the tree (10 for the printed tree).

Test infrastructure only (see ``oracle/__init__``).
"""
import numpy as np


def sort_choices(choices):
    """Sort rank paths by (depth, lexicographic ranks)."""
    return sorted((tuple(int(r) for r in c) for c in choices), key=lambda c: (len(c), c))


def validate_choices(choices, max_nodes=None):
    """Raise ValueError unless the choices form a prefix-closed tree without duplicates."""
    cs = [tuple(c) for c in choices]
    if len(set(cs)) != len(cs):
        raise ValueError("duplicate choice")
    s = set(cs)
    for c in cs:
        if len(c) == 0:
            raise ValueError("empty choice (the root is implicit)")
        if any(r < 0 for r in c):
            raise ValueError("negative rank")
        if len(c) > 1 and c[:-1] not in s:
            raise ValueError("choice %r has no parent in the tree" % (c,))
    if max_nodes is not None and len(cs) + 1 > max_nodes:
        raise ValueError("tree has more than %d nodes" % max_nodes)


def is_prefix(a, b):
    """True when rank path ``a`` is a prefix of (or equal to) rank path ``b``."""
    return len(a) <= len(b) and tuple(b[: len(a)]) == tuple(a)


def tree_buffers(choices, K=None):
    """Build every static tree buffer from a list of rank-path choices.

    Returns a dict with
      T, D, P, K            node count (with root), depth, leaf-path count, top-K stride
      sorted                sorted choices (list of tuples)
      depth      [T]        int64, depth of each node (root 0)
      parent     [T]        int64, parent node (root -1)
      tree_indices [T]      int64, index into the flat candidate list
      anc        [T, T]     bool, anc[i, j] = node j is an ancestor of i or j == i
      retrieve   [P, D+1]   int64, node indices root..leaf, padded with -1
      path_len   [P]        int64, number of real (non-pad) entries in each row
    """
    validate_choices(choices)
    srt = sort_choices(choices)
    T = len(srt) + 1
    paths = [()] + srt  # rank path of each node, root first
    if K is None:
        K = 1 + max(max(c) for c in srt) if srt else 1
    if any(max(c) >= K for c in srt):
        raise ValueError("rank >= K")
    node_of = {p: i for i, p in enumerate(paths)}

    depth = np.array([len(p) for p in paths], dtype=np.int64)
    D = int(depth.max())
    parent = np.array([-1] + [node_of[p[:-1]] for p in paths[1:]], dtype=np.int64)
    tree_indices = np.array([0] + [1 + K * (len(p) - 1) + p[-1] for p in paths[1:]], dtype=np.int64)

    # Brute force over all pairs: j is visible to i iff path_j is a prefix of path_i.
    anc = np.zeros((T, T), dtype=bool)
    for i in range(T):
        for j in range(T):
            anc[i, j] = is_prefix(paths[j], paths[i])

    # A leaf is a node that is not a proper prefix of any other node.
    leaves = [i for i in range(T)
              if not any(len(paths[j]) > len(paths[i]) and is_prefix(paths[i], paths[j])
                         for j in range(T))]
    leaves.sort(reverse=True)
    P = len(leaves)
    retrieve = -np.ones((P, D + 1), dtype=np.int64)
    path_len = np.zeros(P, dtype=np.int64)
    for r, leaf in enumerate(leaves):
        p = paths[leaf]
        row = [node_of[p[:k]] for k in range(len(p) + 1)]
        retrieve[r, : len(row)] = row
        path_len[r] = len(row)
    return dict(T=T, D=D, P=P, K=K, sorted=srt, depth=depth, parent=parent,
                tree_indices=tree_indices, anc=anc, retrieve=retrieve, path_len=path_len)


def anc_bits(anc):
    """Pack a boolean [T, T] ancestor mask into one 64-bit word per row (bit j = column j)."""
    anc = np.asarray(anc, dtype=bool)
    T = anc.shape[0]
    if T > 64:
        raise ValueError("bit rows hold at most 64 nodes")
    out = np.zeros(T, dtype=np.uint64)
    for i in range(T):
        v = 0
        for j in range(T):
            if anc[i, j]:
                v |= 1 << j
        out[i] = np.uint64(v)
    return out


def chain_choices(n):
    """Rank paths of a chain: one rank-0 node per depth 1..n (mask = causal)."""
    return [tuple([0] * k) for k in range(1, n + 1)]


def dense_choices(topks):
    """Cartesian (dense) tree of the per-head top-k widths, e.g. (2, 3) -> 2 + 6 nodes."""
    out = []
    frontier = [()]
    for k in topks:
        nxt = [p + (r,) for p in frontier for r in range(k)]
        out.extend(nxt)
        frontier = nxt
    return out
