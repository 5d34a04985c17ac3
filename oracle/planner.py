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
    "KV cache details": cells hold pos (-1 = empty) and their sequence;
    "Error recovery and state rollback": ``apply`` is the only mutation, a
    failed ubatch is undone with seq_rm(s, pos_min[s], -1).

Readings where the pages are silent (also listed in the design doc):
  * positions given by the caller must be consecutive per sequence in
    batch order and continue from seq_pos_max(s)+1 when the sequence
    already holds cells (an empty sequence may start at any p >= 0),
    else -1;
  * one sequence per token (n_seq_id == 1), else -1;
  * slot search: in ubatch token order each token takes the lowest-index
    empty cell of its stream;
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
    seq: np.ndarray
    output: np.ndarray       # bool
    n_seq_tokens: int
    n_seqs: int

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


class KVMemory:
    """Cell bookkeeping of a plain KV cache with one or several streams.

    One stream when the cache is unified, else one stream per sequence with
    n_ctx / n_seq_max cells each (engine page, Step 7; architecture page,
    Example 10).  Each cell holds (pos, seq), -1 = empty.
    """

    def __init__(self, n_stream: int, n_cells: int, unified: bool):
        self.n_stream = n_stream
        self.n_cells = n_cells
        self.unified = unified
        self.pos = np.full((n_stream, n_cells), -1, np.int64)
        self.seq = np.full((n_stream, n_cells), -1, np.int64)

    def stream_of(self, s: int) -> int:
        return 0 if self.unified else int(s)

    def _cells_of(self, s: int):
        st = self.stream_of(s)
        return st, np.flatnonzero(self.seq[st] == s)

    def seq_pos_max(self, s: int) -> int:
        st, c = self._cells_of(s)
        return int(self.pos[st, c].max()) if c.size else -1

    def seq_pos_min(self, s: int) -> int:
        st, c = self._cells_of(s)
        return int(self.pos[st, c].min()) if c.size else -1

    def seq_rm(self, s: int, p0: int, p1: int) -> bool:
        """Empty the cells of sequence s (all sequences if s < 0) with
        p0 <= pos < p1; p0 < 0 means 0, p1 < 0 means no upper bound."""
        lo = 0 if p0 < 0 else p0
        hi = np.iinfo(np.int64).max if p1 < 0 else p1
        for st in range(self.n_stream):
            sel = (self.pos[st] >= lo) & (self.pos[st] < hi) & (self.seq[st] >= 0)
            if s >= 0:
                sel &= self.seq[st] == s
            self.pos[st, sel] = -1
            self.seq[st, sel] = -1
        return True

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
            self.pos[st, cells[t]] = int(ub.pos[t])
            self.seq[st, cells[t]] = int(ub.seq[t])

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
        self.pos[st, cells] = np.arange(n_pos)
        self.seq[st, cells] = s
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
        seq = np.zeros(n, np.int64)
    else:
        if batch.n_seq_id is not None and any(int(v) != 1 for v in batch.n_seq_id):
            return RC_INVALID, None
        seq = np.asarray([v[0] if isinstance(v, (list, tuple, np.ndarray)) else v
                          for v in batch.seq_id], dtype=np.int64)
        if seq.size != n:
            return RC_INVALID, None
    if np.any(seq < 0) or np.any(seq >= n_seq_max):
        return RC_INVALID, None
    order: List[int] = []
    for s in seq.tolist():
        if s not in order:
            order.append(s)
    nxt = {s: mem.seq_pos_max(s) + 1 for s in order}
    if batch.pos is None:
        pos = np.empty(n, np.int64)
        for i in range(n):
            s = int(seq[i])
            pos[i] = nxt[s]
            nxt[s] += 1
    else:
        pos = np.asarray(batch.pos, dtype=np.int64).reshape(-1)
        if pos.size != n:
            return RC_INVALID, None
        started = set()
        for i in range(n):
            s = int(seq[i])
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
    return RC_OK, SanitizedBatch(token, pos, seq, out, order)


def _make_ubatch(sb: SanitizedBatch, idx: List[int], n_seq_tokens: int,
                 n_seqs: int) -> UBatch:
    ix = np.asarray(idx, dtype=np.int64)
    return UBatch(ix, sb.token[ix], sb.pos[ix], sb.seq[ix], sb.output[ix],
                  n_seq_tokens, n_seqs)


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
    """Sanitise, split and find slots (no mutation of ``mem``)."""
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
        s = int(ub.seq[t])
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
