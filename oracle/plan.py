"""Independent re-derivation of the split-KV work plan (oracle; test infrastructure only).

The pages keep the split schedule of the persistent decode opaque
(``rocm_aiter_mla``, ``AiterMLAMetadataBuilder``: work / reduce maps filled by
a library call with kv_granularity 16).  The library fixes its own rule, and
this module restates it from its definition so that the library's plan can be
compared element by element.  Parity of the plan is pinned by invariants (each
key range covered exactly once, in order; partial slots contiguous; part count
within the CU budget), not by the pages.

Rule (integers only):
  g = 64 keys per granule; c0 = 3 granules of cost per segment; MINC = 4.
  rows per request R = Sq*N; head groups HG = ceil(R / 128).
  part budget P = max(1, floor(C / HG)) for C compute units.
  G_b = ceil(L_b / g); W = sum_b (G_b + c0).
  For target = max(ceil(W / P), c0 + MINC), target + 1, ...: fill parts
  greedily in request order (below) and stop at the first target that gives
  at most P parts.
  Fill: walk requests b in order with a cursor s (granules done).  With
  rem = G_b - s and room = target - load - c0, close the current part when it
  is non-empty and room < min(rem, MINC); otherwise append the segment
  (b, s, s + min(rem, room)) and add c0 + that many granules to the load.
  An empty request (G_b = 0) still gets one segment of zero keys.
  A segment covers keys [s*g, min(e*g, L_b)).  Requests with more than one
  segment get partial slots base_b .. base_b + n_b - 1, bases assigned in
  increasing b; other segments write the output directly (slot -1).
"""
from __future__ import annotations

GRANULE = 64
SEG_COST = 3
MIN_CHUNK = 4
GROUP_ROWS = 128


def head_groups(Sq: int, N: int) -> int:
    return -(-(Sq * N) // GROUP_ROWS)


def _fill(G, target):
    parts, cur, load = [], [], 0
    for b, Gb in enumerate(G):
        s = 0
        while True:
            rem = Gb - s
            room = target - load - SEG_COST
            if cur and room < min(rem, MIN_CHUNK):
                parts.append(cur)
                cur, load = [], 0
                continue
            take = min(rem, room)
            cur.append((b, s, s + take))
            load += SEG_COST + take
            s += take
            if s == Gb:
                break
    if cur:
        parts.append(cur)
    return parts


def split_plan(seq_lens, Sq: int, N: int, num_cus: int):
    """Returns dict(items=[(part, b, kv_start, kv_end, partial)], reduce=[(b, base, n)],
    num_parts, num_partials, head_groups)."""
    L = [int(x) for x in seq_lens]
    G = [-(-x // GRANULE) for x in L]
    hg = head_groups(Sq, N)
    P = max(1, num_cus // hg)
    W = sum(g + SEG_COST for g in G)
    target = max(-(-W // P), SEG_COST + MIN_CHUNK)
    while True:
        parts = _fill(G, target)
        if len(parts) <= P:
            break
        target += 1
    nseg = [0] * len(L)
    for part in parts:
        for (b, _, _) in part:
            nseg[b] += 1
    base = [-1] * len(L)
    reduce, nxt = [], 0
    for b in range(len(L)):
        if nseg[b] > 1:
            base[b] = nxt
            reduce.append((b, nxt, nseg[b]))
            nxt += nseg[b]
    seen = [0] * len(L)
    items = []
    for p, part in enumerate(parts):
        for (b, s, e) in part:
            ks = s * GRANULE
            ke = min(e * GRANULE, L[b])
            if nseg[b] > 1:
                pidx = base[b] + seen[b]
                seen[b] += 1
            else:
                pidx = -1
            items.append((p, b, ks, ke, pidx))
    return dict(items=items, reduce=reduce, num_parts=len(parts), num_partials=nxt,
                head_groups=hg, target=target)


def workspace_bytes(num_partials: int, Sq: int, N: int, Lkv: int = 512) -> int:
    """fp16 partial outputs [partials, Sq*N rounded up to whole 32-row blocks, Lkv], then
    fp32 partial LSE [partials, Sq*N] and fp32 partial row sums [partials, Sq*N]."""
    rows = (Sq * N + 31) // 32 * 32
    return num_partials * (rows * Lkv * 2 + Sq * N * 8)


def gather_rows_all(block_table, seq_lens, page_size: int):
    """Physical row of every key, request-major: entry e covering page_size tokens
    expands to rows e*page_size .. e*page_size + page_size - 1 (``rocm_aiter_mla``,
    ``AiterMLAMetadataBuilder._build_decode``)."""
    out = []
    for b, L in enumerate(seq_lens):
        for j in range(int(L)):
            out.append(int(block_table[b][j // page_size]) * page_size + j % page_size)
    return out
