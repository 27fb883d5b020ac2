"""A model, in Python integers, of the records the ragged prep kernel writes
(attn_plan.hip, ragged_prep_kernel): the candidate cuts, the estimate that
picks one, the class order and the numbering of nodes, units, slots and merged
blocks.  Scheduling only: no attention arithmetic here.  The CPU tests check
its invariants (every (request, row block, key) covered once, slots and merged
blocks within the launch bounds); a GPU test checks the device's records
against it word for word."""

TILE = 32
# per-kernel planning costs (setup tiles, shortest piece in tiles, pieces the
# merge pass combines per tile-step): the bf16 matrix-core and the VALU
# kernels, and the fp32 matrix-core kernel
COST_DEFAULT = (10, 8, 16)
COST_F32 = (1, 1, 80)
MAX_TAIL = 16
N_BODY, N_TAIL = 4, 5
N_CANDS = 1 + N_BODY * N_TAIL
SORT_MAX = 4096
DEAL = 8
FIELDS = ("q_start", "q_len", "prefix", "n_blk", "b_split", "b_chunk", "t_split", "t_chunk", "slot0", "merge0")


def launch_bounds(B, H, max_q, rpb, target):
    """(units, slots, merged blocks) the host sizes the launch for."""
    n_rb = -(-(max_q * H) // rpb)
    slots = max(2 * target, min(MAX_TAIL * B, 4 * target))
    blocks = B * n_rb
    return blocks + slots, slots, min(blocks, slots // 2)


NO_CUT = 1 << 30


def caps(T0, c, min_piece):
    if c == 0:
        return NO_CUT, NO_CUT
    i, j = divmod(c - 1, N_TAIL)
    num, den = (2, 3) if i == 0 else (1, 1 << (i - 1))
    body = min(T0, NO_CUT) * num // den
    tail = body >> j
    return min(max(body, min_piece), NO_CUT), max(tail, min_piece)


def cut(tiles, cap_b, cap_t):
    n = -(-tiles // cap_b)
    cb = -(-tiles // n)
    nb = -(-tiles // cb)
    n = min(-(-tiles // cap_t), MAX_TAIL)
    n = max(n, nb)
    ct = -(-tiles // n)
    nt = -(-tiles // ct)
    return nb, cb, nt, ct


def bucket(t):
    e = t.bit_length() - 1
    return min(63, 4 * e + (((t << 2) >> e) & 3))


def bucket_lo(k):
    return ((4 + (k & 3)) << (k >> 2)) >> 2


def estimate(work, units, d_min, d_max, pieces, per_step, hist, M):
    e = float(work) / M + 0.5 * d_min
    e = max(e, float(d_max))
    if units > M:
        cum = 0
        for k in range(63, -1, -1):
            cum += hist[k]
            if cum >= M + 1:
                e = max(e, float(d_max + bucket_lo(k)))
                break
    return e + float(pieces) / per_step


def clamp_lengths(prefix, q_len, max_q, kv_stride, n_nodes=None):
    """Per request (q, P): q_len into [0, max_q]; then the packed nodes into
    the caller's n_nodes rows (the request that crosses n_nodes keeps its nodes
    below it, later requests none); prefix into [0, kv_stride - q]."""
    out, start = [], 0
    for b in range(len(q_len)):
        q = min(max(q_len[b], 0), max_q)
        qc = q if n_nodes is None else min(q, max(0, n_nodes - start))
        start += q
        out.append((qc, min(max(prefix[b], 0), kv_stride - qc)))
    return out


def plan(prefix, q_len, H, max_q, kv_stride, rpb, target, cost=COST_DEFAULT, n_nodes=None):
    """The records: {"req": [dict per request], "cls_u0", "cls_id", "units",
    "merges", "choice"}.  n_nodes: the caller's packed node rows (None: no
    bound)."""
    SETUP, min_piece, per_step = cost
    B = len(q_len)
    _, max_slots, _ = launch_bounds(B, H, max_q, rpb, target)
    rl = [(q, P, -(-(q * H) // rpb), -(-(P + q) // TILE))
          for q, P in clamp_lengths(prefix, q_len, max_q, kv_stride, n_nodes)]
    W0 = sum(nblk * (tiles + SETUP) for _, _, nblk, tiles in rl)
    Wt = sum(nblk * tiles for _, _, nblk, tiles in rl)
    T0 = max(1, W0 // target)
    est = []
    for c in range(N_CANDS):
        cb_, ct_ = caps(T0, c, min_piece)
        units = pieces = 0
        d_min, d_max = 1 << 31, 0
        hist = [0] * 64
        for q, P, nblk, tiles in rl:
            if nblk == 0:
                continue
            nbd, cb, nt, ct = cut(tiles, cb_, ct_)
            last_b, last_t = tiles - (nbd - 1) * cb, tiles - (nt - 1) * ct
            n_before = nblk - 1
            units += n_before * nbd + nt
            pieces += (n_before * nbd if nbd > 1 else 0) + (nt if nt > 1 else 0)
            d_min = min(d_min, min(last_b if n_before else 1 << 31, last_t) + SETUP)
            d_max = max(d_max, max(cb if n_before else 0, ct) + SETUP)
            if n_before:
                if nbd > 1:
                    hist[bucket(cb + SETUP)] += n_before * (nbd - 1)
                hist[bucket(last_b + SETUP)] += n_before
            if nt > 1:
                hist[bucket(ct + SETUP)] += nt - 1
            hist[bucket(last_t + SETUP)] += 1
        if pieces > max_slots or units == 0:
            est.append(0.0 if c == 0 else -1.0)
        else:
            est.append(estimate(Wt + SETUP * units, units, d_min, d_max, pieces, per_step, hist, target))
    best = 0
    for c in range(1, N_CANDS):
        if est[c] >= 0.0 and est[c] < est[best]:
            best = c
    cap_b, cap_t = caps(T0, best, min_piece)
    reqs = []
    o_q = o_slot = o_merge = 0
    for q, P, nblk, tiles in rl:
        nbd, cb, nt, ct = cut(tiles, cap_b, cap_t) if nblk else (1, tiles, 1, tiles)
        reqs.append(dict(q_start=o_q, q_len=q, prefix=P, n_blk=nblk, b_split=nbd, b_chunk=cb * TILE, t_split=nt,
                         t_chunk=ct * TILE, slot0=o_slot, merge0=o_merge))
        if nblk:
            o_q += q
            o_slot += ((nblk - 1) * nbd if nbd > 1 else 0) + (nt if nt > 1 else 0)
            o_merge += (nblk - 1 if nbd > 1 else 0) + (1 if nt > 1 else 0)

    def cls(i):
        r = reqs[i >> 1]
        if r["n_blk"] == 0:
            return 0, 0
        if i & 1:
            return r["t_split"], r["t_chunk"] // TILE
        if r["n_blk"] > 1:
            return (r["n_blk"] - 1) * r["b_split"], r["b_chunk"] // TILE
        return 0, 0

    ids = list(range(2 * B))
    if 2 * B <= SORT_MAX:
        ids.sort(key=lambda i: ((0xffffffff - (cls(i)[1] if cls(i)[0] else 0)), i))
    u0, u = [], 0
    for i in ids:
        u0.append(u)
        u += cls(i)[0]
    return dict(req=reqs, cls_u0=u0, cls_id=ids, units=u, merges=o_merge, choice=best, max_slots=max_slots, H=H,
                rpb=rpb)


def merge_table(rec):
    """Per merged row block, in merged-block order: (first slot, pieces, first
    output row, rows that exist)."""
    H, rpb = rec["H"], rec["rpb"]
    tab = []
    for r in rec["req"]:
        if r["n_blk"] == 0:
            continue
        body = r["n_blk"] - 1 if r["b_split"] > 1 else 0
        for m in range(body):
            tab.append((r["slot0"] + m * r["b_split"], r["b_split"], r["q_start"] * H + m * rpb, rpb))
        if r["t_split"] > 1:
            rb = r["n_blk"] - 1
            tab.append((r["slot0"] + body * r["b_split"], r["t_split"], r["q_start"] * H + rb * rpb,
                        r["q_len"] * H - rb * rpb))
    assert len(tab) == rec["merges"]
    return tab


def decode(rec, x, H):
    """Block x -> (request, row block, piece, k_begin, k_end, slot) or None,
    as decode_unit_ragged does."""
    if x >= rec["units"]:
        return None
    whole = rec["units"] // (8 * DEAL) * (8 * DEAL)
    if x < whole:  # runs of DEAL consecutive units per XCD (block x runs on XCD x % 8)
        x = (x // 8 // DEAL) * (8 * DEAL) + (x % 8) * DEAL + (x // 8) % DEAL
    u0 = rec["cls_u0"]
    lo, hi = 0, len(u0) - 1
    while lo < hi:
        mid = (lo + hi + 1) >> 1
        if u0[mid] <= x:
            lo = mid
        else:
            hi = mid - 1
    cid, local = rec["cls_id"][lo], x - u0[lo]
    b = cid >> 1
    r = rec["req"][b]
    n_before, bs = r["n_blk"] - 1, r["b_split"]
    if cid & 1 == 0:
        rb, piece, chunk = local % n_before, local // n_before, r["b_chunk"]
        slot = r["slot0"] + rb * bs + piece if bs > 1 else -1
    else:
        rb, piece, chunk = n_before, local, r["t_chunk"]
        slot = r["slot0"] + (n_before * bs if bs > 1 else 0) + piece if r["t_split"] > 1 else -1
    kv = r["prefix"] + r["q_len"]
    k0 = piece * chunk
    return b, rb, piece, k0, min(kv, k0 + chunk), slot


def records_words(rec):
    """The records and the merge table as the device lays them out (int32
    words; the table starts at the next multiple of four words, the gap
    unwritten and read as zero from a zeroed workspace)."""
    words = []
    for r in rec["req"]:
        words += [r[f] for f in FIELDS]
    words += rec["cls_u0"] + rec["cls_id"] + [rec["units"], rec["merges"], rec["choice"]]
    words += [0] * (-len(words) % 4)
    for e in merge_table(rec):
        words += list(e)
    return words
