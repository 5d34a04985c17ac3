"""Host half of the decode step: batch sanitising, ubatch splitting, KV cells.

Oracle - test infrastructure only.  Defines, independently of the C++
runtime, which cell every token lands in and which code ``decode`` returns.

Pages:
  * engine page ("llama.cpp AI LLM Engine - how it works"), Step 10: the
    ``llama_batch`` fields and the allocator's autofill (missing seq ids ->
    sequence 0, missing positions -> seq_pos_max(s)+1 onward, missing output
    flags -> last token only) and its id checks.
  * engine page, Steps 11-12: ``init_batch`` splits the whole batch up front
    (simple split with one stream, equal split with several), then finds KV
    slots for all ubatches before committing any; failure -> return code 1.
    Return codes 0 / 1 / 2 / -1 / -2 / -3.
  * decode-loop page ("Decode loop: batching, KV cache, memory management"),
    "KV cache details": cells hold pos (-1 = empty) and the set of
    sequences using them (a cell can be shared); defrag moves cells to
    close the gaps (the section's before / after figure), and a failed
    slot search is retried once after it; "Error recovery and state
    rollback": ``apply`` is the only mutation, a failed ubatch is undone
    with seq_rm(s, pos_min[s], -1).
  * engine page, Step 10: a token may belong to several sequences
    (n_seq_id > 1); positions are counted per sequence.

Readings where the pages are silent:
  * positions given by the caller must be consecutive per sequence in
    batch order and continue from seq_pos_max(s)+1 when the sequence
    already holds cells (an empty sequence may start at any p >= 0),
    else -1; a token of several sequences must continue each of them,
    and autofilled positions follow its first sequence;
  * a token of several sequences is stored once, in one cell holding all
    of them, which needs a unified cache (one stream), else -1; its
    query attends to the cells of its first sequence;
  * slot search: in ubatch token order each token takes the lowest-index
    empty cell of its stream;
  * seq_rm(s, ...) takes s out of the matching cells and frees a cell once
    no sequence holds it; seq_cp(src, dst, p0, p1) adds dst to src's cells
    with p0 <= pos < p1 in a unified cache, and between streams copies the
    whole of src's stream (only for the full range: p0 < 0, p1 < 0)
    replacing dst's; seq_keep(s) drops every other sequence;
  * defrag packs each stream's occupied cells into its lowest indices,
    ordered by (lowest sequence of the cell, position, old index), as in
    the figure;
  * equal split: the sequences that still have tokens, in order of first
    appearance (at most n_ubatch of them), each give
    k = min(min remaining, n_ubatch // n_seqs) tokens; the ubatch lists
    them sequence by sequence;
  * output rows are the flagged tokens in batch order.
"""
from dataclasses import dataclass, field
from typing import List, Optional, Sequence

import numpy as np

LLAMA_MAX_SEQ = 256      # upper bound on n_seq_max (engine page, Step 7)

RC_OK, RC_NO_SLOT, RC_ABORTED = 0, 1, 2
RC_INVALID, RC_ALLOC, RC_COMPUTE = -1, -2, -3


@dataclass
class Batch:
    """Mirror of ``llama_batch`` (engine page, Step 10).  ``seq_id`` holds one
    sequence id per token (or a list of lists with ``n_seq_id``)."""
    token: Sequence[int]
    pos: Optional[Sequence[int]] = None
    seq_id: Optional[Sequence] = None
    n_seq_id: Optional[Sequence[int]] = None
    logits: Optional[Sequence[int]] = None
    embd: Optional[object] = None


@dataclass
class UBatch:
    """Mirror of ``llama_ubatch`` (decode-loop page, "Batch pipeline")."""
    idx: np.ndarray          # batch index of each token, in ubatch order
    token: np.ndarray
    pos: np.ndarray
    seq: np.ndarray          # first sequence of each token
    output: np.ndarray       # bool
    n_seq_tokens: int
    n_seqs: int
    seqs: List[tuple] = field(default_factory=list)   # all sequences of each token

    @property
    def n_tokens(self) -> int:
        return int(self.idx.size)


@dataclass
class SanitizedBatch:
    token: np.ndarray
    pos: np.ndarray
    seq: np.ndarray
    output: np.ndarray
    seq_order: List[int] = field(default_factory=list)  # first appearance
    seqs: List[tuple] = field(default_factory=list)


class KVMemory:
    """Cell bookkeeping of a plain KV cache with one or several streams.

    One stream when the cache is unified, else one stream per sequence with
    n_ctx / n_seq_max cells each (engine page, Step 7; architecture page,
    Example 10).  Each cell holds a position (-1 = empty) and the set of
    sequences using it, ``has[stream, cell, seq]``.
    """

    def __init__(self, n_stream: int, n_cells: int, unified: bool,
                 n_seq_max: Optional[int] = None):
        self.n_stream = n_stream
        self.n_cells = n_cells
        self.unified = unified
        if n_seq_max is None:
            n_seq_max = LLAMA_MAX_SEQ if unified or n_stream == 1 else n_stream
        self.n_seq_max = n_seq_max
        self.pos = np.full((n_stream, n_cells), -1, np.int64)
        self.has = np.zeros((n_stream, n_cells, n_seq_max), bool)

    def stream_of(self, s: int) -> int:
        return 0 if self.unified else int(s)

    def occupy(self, st: int, cells, positions, seqs) -> None:
        """Set cells of stream st to (position, sequence set); seqs holds
        one sequence id or a tuple of them for all cells."""
        cells = np.atleast_1d(cells)
        self.pos[st, cells] = positions
        self.has[st, cells] = False
        self.has[st, cells[:, None], np.atleast_1d(seqs)[None, :]] = True

    def _cells_of(self, s: int):
        st = self.stream_of(s)
        return st, np.flatnonzero(self.has[st, :, s])

    def seq_pos_max(self, s: int) -> int:
        st, c = self._cells_of(s)
        return int(self.pos[st, c].max()) if c.size else -1

    def seq_pos_min(self, s: int) -> int:
        st, c = self._cells_of(s)
        return int(self.pos[st, c].min()) if c.size else -1

    def _free_unused(self, st: int) -> None:
        self.pos[st, ~self.has[st].any(axis=1)] = -1

    @staticmethod
    def _range(p0: int, p1: int):
        return (0 if p0 < 0 else p0), (np.iinfo(np.int64).max if p1 < 0 else p1)

    def seq_rm(self, s: int, p0: int, p1: int) -> bool:
        """Take sequence s (every sequence if s < 0) out of the cells with
        p0 <= pos < p1; p0 < 0 means 0, p1 < 0 means no upper bound.  A cell
        no sequence holds any more is empty."""
        if s >= self.n_seq_max:
            return False
        lo, hi = self._range(p0, p1)
        for st in range(self.n_stream):
            inr = (self.pos[st] >= lo) & (self.pos[st] < hi)
            if s >= 0:
                self.has[st, inr, s] = False
            else:
                self.has[st, inr, :] = False
            self._free_unused(st)
        return True

    def seq_cp(self, src: int, dst: int, p0: int, p1: int) -> bool:
        """Give dst the cells of src with p0 <= pos < p1.  Between streams
        only the whole sequence can be copied: dst's stream becomes a copy
        of src's (the caller copies the K/V rows of the stream too)."""
        if not (0 <= src < self.n_seq_max and 0 <= dst < self.n_seq_max):
            return False
        if src == dst:
            return True
        ss, sd = self.stream_of(src), self.stream_of(dst)
        if ss == sd:
            lo, hi = self._range(p0, p1)
            sel = self.has[ss, :, src] & (self.pos[ss] >= lo) & (self.pos[ss] < hi)
            self.has[ss, sel, dst] = True
            return True
        if p0 >= 0 or p1 >= 0:
            return False
        self.has[sd] = False
        self.pos[sd] = -1
        sel = self.has[ss, :, src]
        self.pos[sd, sel] = self.pos[ss, sel]
        self.has[sd, sel, dst] = True
        return True

    def seq_keep(self, s: int) -> bool:
        """Drop every sequence but s from every cell."""
        if not 0 <= s < self.n_seq_max:
            return False
        for st in range(self.n_stream):
            keep = self.has[st, :, s].copy()
            self.has[st] = False
            self.has[st, keep, s] = True
            self._free_unused(st)
        return True

    def defrag(self) -> List[np.ndarray]:
        """Pack each stream's occupied cells into its lowest indices, in
        order of (lowest sequence, position, old index).  Returns per stream
        ``src``: new cell j holds what was in cell src[j]."""
        out = []
        for st in range(self.n_stream):
            used = np.flatnonzero(self.pos[st] >= 0)
            first = np.argmax(self.has[st, used], axis=1)
            src = used[np.lexsort((used, self.pos[st, used], first))]
            pos, has = self.pos[st, src].copy(), self.has[st, src].copy()
            self.pos[st] = -1
            self.has[st] = False
            self.pos[st, :src.size] = pos
            self.has[st, :src.size] = has
            out.append(src)
        return out

    def n_kv(self, stream: int) -> int:
        """Cells an attention pass must scan: highest used index + 1."""
        used = np.flatnonzero(self.pos[stream] >= 0)
        return int(used[-1]) + 1 if used.size else 0

    def find_slots(self, ubatches: List[UBatch]) -> Optional[List[np.ndarray]]:
        """Cells for every token of every ubatch, found before any is
        committed; None if some token finds no empty cell."""
        free = [list(np.flatnonzero(self.pos[st] < 0)) for st in range(self.n_stream)]
        heads = [0] * self.n_stream
        out = []
        for ub in ubatches:
            cells = np.empty(ub.n_tokens, np.int64)
            for t in range(ub.n_tokens):
                st = self.stream_of(int(ub.seq[t]))
                if heads[st] >= len(free[st]):
                    return None
                cells[t] = free[st][heads[st]]
                heads[st] += 1
            out.append(cells)
        return out

    def apply(self, ub: UBatch, cells: np.ndarray) -> None:
        for t in range(ub.n_tokens):
            st = self.stream_of(int(ub.seq[t]))
            seqs = ub.seqs[t] if ub.seqs else (int(ub.seq[t]),)
            self.occupy(st, int(cells[t]), int(ub.pos[t]), list(seqs))

    def fill_sequence(self, s: int, n_pos: int) -> Optional[np.ndarray]:
        """Occupy the n_pos lowest empty cells of s's stream with positions
        0..n_pos-1 of sequence s (used to pre-fill a long context).  The
        sequence must be empty.  Returns the cells or None."""
        st = self.stream_of(s)
        if self.seq_pos_max(s) >= 0:
            return None
        free = np.flatnonzero(self.pos[st] < 0)
        if free.size < n_pos:
            return None
        cells = free[:n_pos]
        self.occupy(st, cells, np.arange(n_pos), s)
        return cells


def sanitize(batch: Batch, n_vocab: int, n_seq_max: int, n_batch: int,
             mem: KVMemory):
    """Validate and autofill a batch.  Returns (rc, SanitizedBatch|None)."""
    if batch.embd is not None:
        return RC_INVALID, None
    token = np.asarray(batch.token, dtype=np.int64).reshape(-1)
    n = token.size
    if n <= 0 or n > n_batch:
        return RC_INVALID, None
    if np.any(token < 0) or np.any(token >= n_vocab):
        return RC_INVALID, None
    if batch.seq_id is None:
        seqs = [(0,)] * n
    else:
        if len(batch.seq_id) != n:
            return RC_INVALID, None
        seqs = []
        for i, v in enumerate(batch.seq_id):
            row = [int(x) for x in np.atleast_1d(v)]
            if batch.n_seq_id is not None:
                k = int(batch.n_seq_id[i])
                if k < 1 or k > len(row):
                    return RC_INVALID, None
                row = row[:k]
            if not row or len(set(row)) != len(row):
                return RC_INVALID, None
            seqs.append(tuple(row))
    if any(s < 0 or s >= n_seq_max for row in seqs for s in row):
        return RC_INVALID, None
    if any(len(row) > 1 for row in seqs) and mem.n_stream != 1:
        return RC_INVALID, None            # shared cells need a unified cache
    seq = np.asarray([row[0] for row in seqs], np.int64)
    order: List[int] = []
    for s in seq.tolist():
        if s not in order:
            order.append(s)
    nxt = {s: mem.seq_pos_max(s) + 1 for row in seqs for s in row}
    if batch.pos is None:
        pos = np.empty(n, np.int64)
        fill = dict(nxt)
        for i in range(n):
            pos[i] = fill[seqs[i][0]]
            for s in seqs[i]:
                fill[s] = pos[i] + 1
    else:
        pos = np.asarray(batch.pos, dtype=np.int64).reshape(-1)
        if pos.size != n:
            return RC_INVALID, None
    started = set()
    for i in range(n):
        for s in seqs[i]:
            if s not in started and nxt[s] == 0:
                # an empty sequence may start at any position >= 0
                if pos[i] < 0:
                    return RC_INVALID, None
                nxt[s] = int(pos[i])
            started.add(s)
            if pos[i] != nxt[s]:
                return RC_INVALID, None
            nxt[s] += 1
    if batch.logits is None:
        out = np.zeros(n, bool)
        out[-1] = True
    else:
        out = np.asarray(batch.logits).reshape(-1) != 0
        if out.size != n:
            return RC_INVALID, None
    return RC_OK, SanitizedBatch(token, pos, seq, out, order, seqs)


def _make_ubatch(sb: SanitizedBatch, idx: List[int], n_seq_tokens: int,
                 n_seqs: int) -> UBatch:
    ix = np.asarray(idx, dtype=np.int64)
    return UBatch(ix, sb.token[ix], sb.pos[ix], sb.seq[ix], sb.output[ix],
                  n_seq_tokens, n_seqs, [sb.seqs[i] for i in idx])


def split_simple(sb: SanitizedBatch, n_ubatch: int) -> List[UBatch]:
    """Consecutive chunks of at most n_ubatch tokens in batch order."""
    n = sb.token.size
    return [_make_ubatch(sb, list(range(i, min(n, i + n_ubatch))),
                         min(n, i + n_ubatch) - i, 1)
            for i in range(0, n, n_ubatch)]


def split_equal(sb: SanitizedBatch, n_ubatch: int) -> List[UBatch]:
    """Equal-length per-sequence chunks (reading in the module docstring)."""
    queues = {s: [i for i in range(sb.token.size) if sb.seq[i] == s]
              for s in sb.seq_order}
    heads = {s: 0 for s in sb.seq_order}
    out = []
    while True:
        live = [s for s in sb.seq_order if heads[s] < len(queues[s])][:n_ubatch]
        if not live:
            return out
        k = min(min(len(queues[s]) - heads[s] for s in live),
                n_ubatch // len(live))
        idx = []
        for s in live:
            idx.extend(queues[s][heads[s]:heads[s] + k])
            heads[s] += k
        out.append(_make_ubatch(sb, idx, k, len(live)))


@dataclass
class Plan:
    rc: int
    ubatches: List[UBatch] = field(default_factory=list)
    cells: List[np.ndarray] = field(default_factory=list)
    out_row: Optional[np.ndarray] = None     # per batch index, -1 if none
    n_outputs: int = 0


def plan_batch(batch: Batch, mem: KVMemory, n_vocab: int, n_seq_max: int,
               n_batch: int, n_ubatch: int) -> Plan:
    """Sanitise, split and find slots; ``mem`` is not changed.

    The decode-loop page ("KV cache details") compacts a fragmented cache
    and searches again when no slot is found.  The slot search here takes
    any free cell of the stream, and compaction keeps the number of free
    cells, so a second search cannot succeed: a failed search returns
    RC_NO_SLOT with the cache as it was (compaction stays available as
    KVMemory.defrag)."""
    rc, sb = sanitize(batch, n_vocab, n_seq_max, n_batch, mem)
    if rc != RC_OK:
        return Plan(rc)
    ubs = split_simple(sb, n_ubatch) if mem.n_stream == 1 else split_equal(sb, n_ubatch)
    assert sum(u.n_tokens for u in ubs) == sb.token.size
    cells = mem.find_slots(ubs)
    if cells is None:
        return Plan(RC_NO_SLOT)
    out_row = np.full(sb.token.size, -1, np.int64)
    flagged = np.flatnonzero(sb.output)
    out_row[flagged] = np.arange(flagged.size)
    return Plan(RC_OK, ubs, cells, out_row, int(flagged.size))


def rollback_ubatch(mem: KVMemory, ub: UBatch) -> None:
    """Undo a committed ubatch: seq_rm(s, pos_min[s], -1) for its sequences."""
    pos_min = {}
    for t in range(ub.n_tokens):
        for s in (ub.seqs[t] if ub.seqs else (int(ub.seq[t]),)):
            pos_min[s] = min(pos_min.get(s, int(ub.pos[t])), int(ub.pos[t]))
    for s, p in pos_min.items():
        mem.seq_rm(s, p, -1)


def context_geometry(n_ctx: int, n_seq_max: int, kv_unified: bool):
    """n_ctx padded up to a multiple of 256, then split into streams
    (engine page, Step 7; architecture page, Example 10).
    Returns (n_ctx_padded, n_stream, cells_per_stream)."""
    n_ctx = (n_ctx + 255) // 256 * 256
    n_stream = 1 if kv_unified else n_seq_max
    return n_ctx, n_stream, n_ctx // n_stream
