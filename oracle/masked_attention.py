"""Plain float64 oracle: the teacher-forcing mask and masked attention + JVP.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Notation (Causal-rCM, arXiv 2606.25473): a side holds ``N_h = T_f * F``
tokens (``T_f`` tokens per latent frame, ``F`` frames); a chunk holds
``c`` frames, i.e. ``T = T_f * c`` tokens.  ``tf_layout = 0`` is the plain
block-causal (DF) sequence of ``N = N_h`` tokens; ``tf_layout = 1`` is the
teacher-forcing packed sequence [clean | noisy] of ``N = 2 N_h`` tokens
(section 3.1.1, eq. 8).

Readings of the pages taken here (the display formulas survive only as
their numbers, so each is the plain reading of the surrounding text):

* clean tokens see every clean token of the same or an earlier chunk
  (block-causal, bidirectional inside a chunk) and never a noisy token;
* a noisy token of chunk c sees the clean tokens of chunks strictly before
  c and every noisy token of its own chunk c, nothing else (section 3.1.1:
  each noisy chunk attends to its allowed clean history and its own noisy
  tokens);
* scores are scaled by 1/sqrt(d) unless a scale is given; the same scale
  multiplies the score tangent (Appendix B, eqs. 42-43);
* masked pairs carry probability exactly zero and no tangent: the tangent
  is taken through the masked map with the mask held fixed (Appendix B,
  text after eq. 43);
* the log-sum-exp output is natural-log based (Algorithm 1 returns it
  beside O and its tangent).
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class MaskDesc:
    tokens_per_frame: int
    n_frames: int
    frames_per_chunk: int
    tf_layout: int

    @property
    def side_len(self) -> int:
        return self.tokens_per_frame * self.n_frames

    @property
    def seq_len(self) -> int:
        return self.side_len * (2 if self.tf_layout else 1)

    @property
    def chunk_len(self) -> int:
        return self.tokens_per_frame * self.frames_per_chunk

    @property
    def n_chunks(self) -> int:
        return self.n_frames // self.frames_per_chunk


@dataclass(frozen=True)
class ChunkListDesc:
    """Teacher-forcing / block-causal mask whose chunks have arbitrary sizes
    (section 4: a cA-B pattern is an initial chunk of A latent frames, then
    chunks of B frames).  ``chunk_lens`` are the chunk lengths in tokens of
    one side, in order; the rule is that of ``MaskDesc`` with chunk index
    taken from these boundaries."""
    chunk_lens: tuple
    tf_layout: int

    @property
    def side_len(self) -> int:
        return int(sum(self.chunk_lens))

    @property
    def seq_len(self) -> int:
        return self.side_len * (2 if self.tf_layout else 1)


@dataclass(frozen=True)
class RangeMask:
    """Query groups x key intervals (Appendix B, sparse custom mask
    representation): each group is a contiguous query interval with a list
    of allowed key intervals; query i may see key j iff i lies in a group one
    of whose intervals holds j.  Rows in no group see no key.
    ``groups`` = ((row_lo, row_hi, ((key_lo, key_hi), ...)), ...), half-open."""
    seq_len: int
    groups: tuple


def _as_desc(desc):
    if isinstance(desc, (MaskDesc, ChunkListDesc, RangeMask)):
        return desc
    return MaskDesc(*desc)


# ----------------------------------------------------------------------------
# Mask (section 2.3; section 3.1.1; section 4 chunking; Table 2 legend)
# ----------------------------------------------------------------------------

def _side_and_chunk(desc: MaskDesc, idx):
    """Token index -> (is_noisy, chunk index); works on ints and int arrays."""
    idx = np.asarray(idx, dtype=np.int64)
    noisy = (idx >= desc.side_len) if desc.tf_layout else np.zeros(idx.shape, dtype=bool)
    pos = idx % desc.side_len
    return noisy, pos // desc.chunk_len


def _chunklist_side_and_chunk(desc: ChunkListDesc, idx):
    idx = np.asarray(idx, dtype=np.int64)
    noisy = (idx >= desc.side_len) if desc.tf_layout else np.zeros(idx.shape, dtype=bool)
    pos = idx % desc.side_len
    starts = np.cumsum((0,) + tuple(desc.chunk_lens))[:-1]
    return noisy, np.searchsorted(starts, pos, side="right") - 1


def _range_group(desc: RangeMask, idx):
    """Group index of each query row (-1: in no group)."""
    idx = np.asarray(idx, dtype=np.int64)
    out = np.full(idx.shape, -1, dtype=np.int64)
    for g, (lo, hi, _) in enumerate(desc.groups):
        out[(idx >= lo) & (idx < hi)] = g
    return out


def allowed(desc, i, j):
    """allowed(i, j): may query token i attend to key token j?  (broadcasts)"""
    desc = _as_desc(desc)
    if isinstance(desc, RangeMask):
        i, j = np.broadcast_arrays(np.asarray(i, dtype=np.int64), np.asarray(j, dtype=np.int64))
        g = _range_group(desc, i)
        out = np.zeros(i.shape, dtype=bool)
        for gi, (_, _, ivs) in enumerate(desc.groups):
            sel = g == gi
            for lo, hi in ivs:
                out |= sel & (j >= lo) & (j < hi)
        return out
    if isinstance(desc, ChunkListDesc):
        qi_noisy, qi_chunk = _chunklist_side_and_chunk(desc, i)
        kj_noisy, kj_chunk = _chunklist_side_and_chunk(desc, j)
    else:
        qi_noisy, qi_chunk = _side_and_chunk(desc, i)
        kj_noisy, kj_chunk = _side_and_chunk(desc, j)
    clean_row = (~qi_noisy) & (~kj_noisy) & (kj_chunk <= qi_chunk)
    noisy_row = qi_noisy & (((~kj_noisy) & (kj_chunk < qi_chunk)) | (kj_noisy & (kj_chunk == qi_chunk)))
    return clean_row | noisy_row


def mask_dense(desc) -> np.ndarray:
    """The [N, N] boolean mask, straight from ``allowed``.  Small N only."""
    desc = _as_desc(desc)
    n = desc.seq_len
    return allowed(desc, np.arange(n)[:, None], np.arange(n)[None, :])


def allowed_row(desc, i: int) -> np.ndarray:
    """Boolean [N] vector of the keys query i may see, straight from ``allowed``."""
    desc = _as_desc(desc)
    return allowed(desc, np.int64(i), np.arange(desc.seq_len))


def row_groups(desc):
    """Rows that share one key set, as (first row, stop row), covering all
    rows: one (side, chunk) pair of a chunked mask; one query group of a
    range mask, and the runs of rows in no group.

    ``allowed(i, j)`` depends on i only through its side and chunk (or its
    group), so the rows of one group share one key set; grouping them is
    vectorisation of the definition, not a different algorithm.
    """
    desc = _as_desc(desc)
    if isinstance(desc, RangeMask):
        out, at = [], 0
        for lo, hi, _ in sorted(desc.groups):
            if lo > at:
                out.append((at, lo))
            out.append((lo, hi))
            at = hi
        if at < desc.seq_len:
            out.append((at, desc.seq_len))
        return out
    sides = 2 if desc.tf_layout else 1
    lens = desc.chunk_lens if isinstance(desc, ChunkListDesc) else (desc.chunk_len,) * desc.n_chunks
    out = []
    for s in range(sides):
        lo = s * desc.side_len
        for t in lens:
            out.append((lo, lo + t))
            lo += t
    return out


def _row_key(desc, rows):
    """A hashable label per row; rows with one label share one key set."""
    if isinstance(desc, RangeMask):
        return [(int(g),) for g in np.atleast_1d(_range_group(desc, rows))]
    if isinstance(desc, ChunkListDesc):
        noisy, chunk = _chunklist_side_and_chunk(desc, rows)
    else:
        noisy, chunk = _side_and_chunk(desc, rows)
    return list(zip(np.atleast_1d(noisy).tolist(), np.atleast_1d(chunk).tolist()))


def pair_count(desc) -> int:
    """Number of allowed (query, key) pairs per (b, h), by summing the mask."""
    desc = _as_desc(desc)
    total = 0
    for lo, hi in row_groups(desc):
        total += int(allowed_row(desc, lo).sum()) * (hi - lo)
    return total


# ----------------------------------------------------------------------------
# Tile geometry and classification (Appendix B, "sparse custom mask
# representation": tasks are query blocks; whole key/value blocks outside
# every allowed range are skipped)
# ----------------------------------------------------------------------------

def query_blocks(desc, block_q: int):
    """Query blocks as (start, stop): each side is cut from its own start; a
    range mask is cut from row 0 over the whole sequence."""
    desc = _as_desc(desc)
    if isinstance(desc, RangeMask):
        n = desc.seq_len
        return [(lo, min(lo + block_q, n)) for lo in range(0, n, block_q)]
    sides = 2 if desc.tf_layout else 1
    out = []
    for s in range(sides):
        base = s * desc.side_len
        for lo in range(0, desc.side_len, block_q):
            out.append((base + lo, base + min(lo + block_q, desc.side_len)))
    return out


def key_tiles(desc, block_k: int):
    """Key tiles as (start, stop), cut from key 0 over the whole sequence."""
    desc = _as_desc(desc)
    n = desc.seq_len
    return [(lo, min(lo + block_k, n)) for lo in range(0, n, block_k)]


def tile_classes(desc, block_q: int, block_k: int) -> np.ndarray:
    """uint8 [n_query_blocks, n_key_tiles]: 0 no allowed pair, 1 every pair
    allowed, 2 otherwise -- counted from ``allowed`` row by row."""
    desc = _as_desc(desc)
    qb = query_blocks(desc, block_q)
    kt = key_tiles(desc, block_k)
    n = desc.seq_len
    edges = np.array([lo for lo, _ in kt] + [n])
    widths = np.diff(edges)
    out = np.zeros((len(qb), len(kt)), dtype=np.uint8)
    cache = {}
    for bi, (lo, hi) in enumerate(qb):
        counts = np.zeros(len(kt), dtype=np.int64)
        for i in range(lo, hi):
            key = _row_key(desc, np.int64(i))[0]
            if key not in cache:
                row = allowed_row(desc, i).astype(np.int64)
                cache[key] = np.add.reduceat(row, edges[:-1])
            counts += cache[key]
        rows = hi - lo
        cls = np.where(counts == 0, 0, np.where(counts == rows * widths, 1, 2))
        out[bi] = cls.astype(np.uint8)
    return out


# ----------------------------------------------------------------------------
# Masked attention and its JVP (Appendix B, eqs. 42-44)
# ----------------------------------------------------------------------------

def _scale(d: int, scale):
    return 1.0 / math.sqrt(d) if scale is None or scale <= 0 else float(scale)


def _rows_forward(q, k, v, tq, tk, tv, keys, scale):
    """Rows sharing one key set: two-pass softmax, then the analytic tangent.

    s_ij   = scale * q_i . k_j                       (eq. 42)
    ts_ij  = scale * (tq_i . k_j + q_i . tk_j)       (eq. 43)
    p_ij   = exp(s_ij - m_i) / l_i over allowed j, 0 elsewhere
    o_i    = sum_j p_ij v_j,      lse_i = m_i + ln l_i
    tp_ij  = p_ij (ts_ij - sum_k p_ik ts_ik)         (softmax tangent)
    to_i   = sum_j tp_ij v_j + sum_j p_ij tv_j       (eq. 44)
    """
    kk, vv, tkk, tvv = k[keys], v[keys], tk[keys], tv[keys]
    s = scale * (q @ kk.T)
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    l = e.sum(axis=1, keepdims=True)
    p = e / l
    o = p @ vv
    lse = (m + np.log(l))[:, 0]
    ts = scale * (tq @ kk.T + q @ tkk.T)
    rbar = (p * ts).sum(axis=1, keepdims=True)
    tp = p * (ts - rbar)
    to = tp @ vv + p @ tvv
    return o, to, lse


def masked_attention_jvp_slice(q, k, v, tq, tk, tv, desc, scale=None, rows=None):
    """One (b, h) slice.  q, k, tq, tk are [N, d]; v, tv are [N, dv] (any float
    type, widened to float64).

    Returns float64 (o [R, dv], to [R, dv], lse [R]) for ``rows`` (default: all).
    """
    desc = _as_desc(desc)
    arrs = [np.asarray(x, dtype=np.float64) for x in (q, k, v, tq, tk, tv)]
    q, k, v, tq, tk, tv = arrs
    n, d = q.shape
    dv = v.shape[1]
    if n != desc.seq_len:
        raise ValueError(f"sequence length {n} does not match the mask ({desc.seq_len})")
    sc = _scale(d, scale)
    rows = np.arange(n) if rows is None else np.asarray(rows, dtype=np.int64)
    o = np.zeros((len(rows), dv))
    to = np.zeros((len(rows), dv))
    lse = np.full(len(rows), -np.inf)
    groups = {}
    for pos, key in enumerate(_row_key(desc, rows)):
        groups.setdefault(key, []).append(pos)
    for _, positions in groups.items():
        positions = np.asarray(positions)
        sel = rows[positions]
        keys = np.nonzero(allowed_row(desc, int(sel[0])))[0]
        if keys.size == 0:  # rows that see no key (e.g. in no group): zero output, lse = -inf
            continue
        o_g, to_g, lse_g = _rows_forward(q[sel], k, v, tq[sel], tk, tv, keys, sc)
        o[positions], to[positions], lse[positions] = o_g, to_g, lse_g
    return o, to, lse


def masked_attention_jvp(q, k, v, tq, tk, tv, desc, scale=None):
    """Full [B, H, N, d] tensors -> float64 (o, to, lse [B, H, N])."""
    q = np.asarray(q)
    b_, h_, n, d = q.shape
    o = np.empty((b_, h_, n, d))
    to = np.empty((b_, h_, n, d))
    lse = np.empty((b_, h_, n))
    for b in range(b_):
        for h in range(h_):
            o[b, h], to[b, h], lse[b, h] = masked_attention_jvp_slice(
                q[b, h], k[b, h], v[b, h], tq[b, h], tk[b, h], tv[b, h], desc, scale)
    return o, to, lse


def masked_attention_jvp_rows(slices, desc, rows, scale=None):
    """Selected rows of one (b, h) slice; ``slices`` = (q, k, v, tq, tk, tv)."""
    return masked_attention_jvp_slice(*slices, desc, scale=scale, rows=rows)


def masked_attention_jvp_scalar(q, k, v, tq, tk, tv, desc, scale=None):
    """Pure-Python scalar loops over one (b, h) slice; for N <= ~96 only.

    Same definition as ``masked_attention_jvp_slice``, written without NumPy
    so that the vectorised code is checked by an independent route.
    """
    desc = _as_desc(desc)
    q, k, v, tq, tk, tv = [[[float(x) for x in row] for row in np.asarray(a)] for a in (q, k, v, tq, tk, tv)]
    n, d = len(q), len(q[0])
    sc = _scale(d, scale)

    def dot(a, b):
        return math.fsum(x * y for x, y in zip(a, b))

    o = [[0.0] * d for _ in range(n)]
    to = [[0.0] * d for _ in range(n)]
    lse = [-math.inf] * n
    for i in range(n):
        keys = [j for j in range(n) if bool(allowed(desc, i, j))]
        if not keys:
            continue
        s = {j: sc * dot(q[i], k[j]) for j in keys}
        ts = {j: sc * (dot(tq[i], k[j]) + dot(q[i], tk[j])) for j in keys}
        m = max(s.values())
        l = math.fsum(math.exp(s[j] - m) for j in keys)
        p = {j: math.exp(s[j] - m) / l for j in keys}
        rbar = math.fsum(p[j] * ts[j] for j in keys)
        for c in range(d):
            o[i][c] = math.fsum(p[j] * v[j][c] for j in keys)
            to[i][c] = math.fsum(p[j] * (ts[j] - rbar) * v[j][c] + p[j] * tv[j][c] for j in keys)
        lse[i] = m + math.log(l)
    return np.array(o), np.array(to), np.array(lse)


# ----------------------------------------------------------------------------
# Clean tangent zero (section 3.1.2, teacher-forcing sCM, the text after
# eq. 17: the JVP runs through the same packed forward under the same
# teacher-forcing mask; the clean context has zero tangent and only the noisy
# tokens move)
# ----------------------------------------------------------------------------

def zero_clean_tangents(tq, tk, tv, desc):
    """Float64 copies of the tangents with every clean token's row set to 0
    (whatever the clean rows held before, NaN included)."""
    desc = _as_desc(desc)
    if not desc.tf_layout:
        raise ValueError("the clean / noisy split needs tf_layout = 1")
    out = []
    for t in (tq, tk, tv):
        t = np.array(t, dtype=np.float64, copy=True)
        t[..., : desc.side_len, :] = 0.0
        out.append(t)
    return out


def masked_attention_jvp_slice_ctz(q, k, v, tq, tk, tv, desc, scale=None, rows=None):
    """One (b, h) slice with the clean tokens' tangents taken as zero."""
    tq, tk, tv = zero_clean_tangents(tq, tk, tv, desc)
    return masked_attention_jvp_slice(q, k, v, tq, tk, tv, desc, scale=scale, rows=rows)


def pair_counts_by_class(desc):
    """Allowed (query, key) pairs per (b, h), split as (clean rows, noisy rows
    against clean keys, noisy rows against noisy keys), by summing the mask.
    With tf_layout = 0 every pair is a clean-row pair."""
    desc = _as_desc(desc)
    cc = nc = nn = 0
    for lo, hi in row_groups(desc):
        keys = allowed_row(desc, lo)
        clean_keys = int(keys[: desc.side_len].sum())
        noisy_keys = int(keys[desc.side_len:].sum())
        if desc.tf_layout and lo >= desc.side_len:
            nc += clean_keys * (hi - lo)
            nn += noisy_keys * (hi - lo)
        else:
            cc += (clean_keys + noisy_keys) * (hi - lo)
    return cc, nc, nn


def useful_flops(desc, head_dim, clean_tangent_zero=False):
    """Useful FLOPs per (b, h): 2 per multiply-add of the products the result
    needs over allowed pairs.  General: q.k, tq.k, q.tk, p.v, p.tv, (p ts).v,
    i.e. 12 d per pair.  Clean tangent zero: clean rows need q.k and p.v
    (4 d); noisy rows against clean keys need q.k, tq.k, p.v, (p ts).v (8 d);
    noisy rows against noisy keys need all six (12 d)."""
    cc, nc, nn = pair_counts_by_class(desc)
    if clean_tangent_zero:
        return head_dim * (4 * cc + 8 * nc + 12 * nn)
    return head_dim * 12 * (cc + nc + nn)


# ----------------------------------------------------------------------------
# Backward of the masked attention (section 3.2.1: the FlashAttention-2 based
# kernel with custom masks; training the student needs the gradients of the
# same masked attention).  The plain gradient of o = softmax(s) v with
# s = scale q k^T under the mask, for an output cotangent do:
#   dv_j = sum_i p_ij do_i
#   dp_ij = do_i . v_j,   delta_i = sum_j p_ij dp_ij (= do_i . o_i)
#   ds_ij = p_ij (dp_ij - delta_i)            (0 where masked)
#   dq_i = scale sum_j ds_ij k_j,   dk_j = scale sum_i ds_ij q_i
# ----------------------------------------------------------------------------

def masked_attention_bwd_slice(q, k, v, do, desc, scale=None):
    """One (b, h) slice: float64 (dq [N, d], dk [N, d], dv [N, dv], delta [N])."""
    desc = _as_desc(desc)
    q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
    n, d = q.shape
    if n != desc.seq_len:
        raise ValueError(f"sequence length {n} does not match the mask ({desc.seq_len})")
    sc = _scale(d, scale)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    delta = np.zeros(n)
    for lo, hi in row_groups(desc):
        keys = np.nonzero(allowed_row(desc, lo))[0]
        if keys.size == 0:
            continue
        kk, vv = k[keys], v[keys]
        s = sc * (q[lo:hi] @ kk.T)
        e = np.exp(s - s.max(axis=1, keepdims=True))
        p = e / e.sum(axis=1, keepdims=True)
        dp = do[lo:hi] @ vv.T
        dl = (p * dp).sum(axis=1)
        ds = p * (dp - dl[:, None])
        dq[lo:hi] = sc * (ds @ kk)
        dk[keys] += sc * (ds.T @ q[lo:hi])
        dv[keys] += p.T @ do[lo:hi]
        delta[lo:hi] = dl
    return dq, dk, dv, delta


def masked_attention_bwd(q, k, v, do, desc, scale=None):
    """Full [B, H, N, d] tensors -> float64 (dq, dk, dv, delta [B, H, N])."""
    q = np.asarray(q)
    b_, h_, n, d = q.shape
    out = [np.empty((b_, h_, n, d)) for _ in range(3)] + [np.empty((b_, h_, n))]
    for b in range(b_):
        for h in range(h_):
            r = masked_attention_bwd_slice(q[b, h], k[b, h], v[b, h], do[b, h], desc, scale)
            for o_, x in zip(out, r):
                o_[b, h] = x
    return tuple(out)


def masked_attention_bwd_rows(q, k, v, do, desc, rows, scale=None, batch_rows=256):
    """The same backward restricted to the query rows ``rows`` of one (b, h)
    slice: float64 (dq [len(rows), d], dk_part [N, d], dv_part [N, dv],
    delta [len(rows)]), where dk_part and dv_part hold the contributions of
    these rows only (sum over i in rows of the per-pair terms).  For a key
    whose attending rows all lie in ``rows`` they are that key's full dk and
    dv; dq and delta of a row need only that row.  Consecutive rows (in
    sorted order) with the same allowed keys are taken together, at most
    ``batch_rows`` at a time."""
    desc = _as_desc(desc)
    q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
    n, d = q.shape
    sc = _scale(d, scale)
    rows = np.asarray(rows, dtype=np.int64)
    dq = np.zeros((rows.size, d))
    delta = np.zeros(rows.size)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    order = np.argsort(rows, kind="stable")
    i = 0
    while i < order.size:
        mask = allowed_row(desc, int(rows[order[i]]))
        j = i + 1
        while j < order.size and j - i < batch_rows and np.array_equal(allowed_row(desc, int(rows[order[j]])), mask):
            j += 1
        sel = order[i:j]
        rr = rows[sel]
        keys = np.nonzero(mask)[0]
        i = j
        if keys.size == 0:  # a row that sees no key (range lists): P = 0, every term is 0
            continue
        kk, vv = k[keys], v[keys]
        s = sc * (q[rr] @ kk.T)
        e = np.exp(s - s.max(axis=1, keepdims=True))
        p = e / e.sum(axis=1, keepdims=True)
        dp = do[rr] @ vv.T
        dl = (p * dp).sum(axis=1)
        ds = p * (dp - dl[:, None])
        dq[sel] = sc * (ds @ kk)
        dk[keys] += sc * (ds.T @ q[rr])
        dv[keys] += p.T @ do[rr]
        delta[sel] = dl
    return dq, dk, dv, delta


def backward_useful_flops(desc, head_dim):
    """2 per multiply-add of the five products over allowed pairs (s, dp, dv,
    dk, dq): 10 d per pair, per (b, h)."""
    return 10 * head_dim * pair_count(desc)
