"""Oracle byte-level BPE (the E stage of F = E* o G) and the full encoder.

TokTier summary page, Appendix A.1: every pre-token is encoded on its own, with
no state crossing pre-tokens, and the token sequence of the text is the
concatenation.  §4.2 of the same page says the GPU runs exactly this BPE per
piece.  The merge rule itself is not printed on the pages; this is the classic
byte-level BPE encode:

  * ids 0..255 are raw byte values; merge number r (its rank) makes the token
    with id 256 + r out of the adjacent pair (x, y);
  * repeat: among adjacent pairs that have a merge, take the one of lowest rank
    (the leftmost one if the same pair occurs several times), replace it by its
    token; stop when no adjacent pair has a merge.

Three implementations with the same semantics live here:
  bpe_classic -- the textbook O(L^2) loop above, used for everything small;
  bpe_heap    -- a heap over (rank, position) with a doubly linked list,
                 O(L log L), needed for the 1,000,000-byte single piece;
  bpe_naive   -- brute force of a different shape: for r = 0, 1, 2, ... replace
                 every left-to-right non-overlapping occurrence of merge r.  On
                 a consistent table (both operands of merge r have ids below
                 256 + r) it must agree with bpe_classic.

The whole-word rule of the Llama family (same page, §4.2: with ignore_merges
the whole pre-token is matched against the vocabulary first, and a match
skips the merges) is the ``ignore_merges`` option of the encoders.  Reading:
a piece whose bytes equal a vocabulary token becomes that one token; if
several ids share those bytes, the smallest (the first to enter the
vocabulary); any other piece goes through BPE as above.
"""
import heapq

from .pretok import split_bytes


class Vocab:
    """A merge table in rank order: merges[r] = (x, y) makes id 256 + r."""

    def __init__(self, merges):
        self.merges = [(int(x), int(y)) for x, y in merges]
        self.rank = {}
        for r, (x, y) in enumerate(self.merges):
            if (x, y) in self.rank:
                raise ValueError("duplicate merge pair %r" % ((x, y),))
            if not (0 <= x < 256 + r and 0 <= y < 256 + r):
                raise ValueError("merge %d uses an id that does not exist yet" % r)
            self.rank[(x, y)] = r
        self.tok_bytes = [bytes([b]) for b in range(256)]
        for x, y in self.merges:
            self.tok_bytes.append(self.tok_bytes[x] + self.tok_bytes[y])
        self._token_id = None

    @property
    def token_id(self):
        """bytes -> the smallest id whose bytes they are (the vocabulary)."""
        if self._token_id is None:
            d = {}
            for i, b in enumerate(self.tok_bytes):
                d.setdefault(b, i)
            self._token_id = d
        return self._token_id

    @property
    def size(self):
        return 256 + len(self.merges)


def bpe_classic(ids, rank):
    """Textbook lowest-rank-first merge loop (leftmost on equal pairs)."""
    ids = list(ids)
    while True:
        best_r, best_i = None, None
        for i in range(len(ids) - 1):
            r = rank.get((ids[i], ids[i + 1]))
            if r is not None and (best_r is None or r < best_r):
                best_r, best_i = r, i
        if best_r is None:
            return ids
        ids[best_i:best_i + 2] = [256 + best_r]


def bpe_heap(ids, rank):
    """Same result as bpe_classic, via a min-heap of (rank, left position).

    Positions are the original indices, kept in text order by a doubly linked
    list, so among equal ranks the heap pops the leftmost pair first.  A heap
    entry is used only if the pair it names is still adjacent and unchanged.
    """
    n = len(ids)
    if n < 2:
        return list(ids)
    tok = list(ids)
    nxt = list(range(1, n)) + [-1]
    prv = [-1] + list(range(0, n - 1))
    heap = []
    for i in range(n - 1):
        r = rank.get((tok[i], tok[i + 1]))
        if r is not None:
            heap.append((r, i, i + 1, tok[i], tok[i + 1]))
    heapq.heapify(heap)
    alive = [True] * n
    while heap:
        r, i, j, x, y = heapq.heappop(heap)
        if not (alive[i] and alive[j] and nxt[i] == j and tok[i] == x and tok[j] == y):
            continue
        tok[i] = 256 + r
        alive[j] = False
        k = nxt[j]
        nxt[i] = k
        if k != -1:
            prv[k] = i
            rk = rank.get((tok[i], tok[k]))
            if rk is not None:
                heapq.heappush(heap, (rk, i, k, tok[i], tok[k]))
        p = prv[i]
        if p != -1:
            rp = rank.get((tok[p], tok[i]))
            if rp is not None:
                heapq.heappush(heap, (rp, p, i, tok[p], tok[i]))
    out, i = [], 0
    while i != -1:
        out.append(tok[i])
        i = nxt[i]
    return out


def bpe_naive(ids, merges):
    """Brute force: for each merge in rank order, replace all of its
    left-to-right non-overlapping occurrences."""
    ids = list(ids)
    for r, (x, y) in enumerate(merges):
        out, i = [], 0
        while i < len(ids):
            if i + 1 < len(ids) and ids[i] == x and ids[i + 1] == y:
                out.append(256 + r)
                i += 2
            else:
                out.append(ids[i])
                i += 1
        ids = out
    return ids


def bpe(piece, vocab, ignore_merges=False):
    """BPE of one pre-token (bytes).  Long pieces take the heap form.  With
    ignore_merges, a piece that is a vocabulary token is that token."""
    if ignore_merges:
        t = vocab.token_id.get(bytes(piece))
        if t is not None:
            return [t]
    if len(piece) > 64:
        return bpe_heap(piece, vocab.rank)
    return bpe_classic(piece, vocab.rank)


def encode(data, vocab, pattern_id, memo=None, ignore_merges=False):
    """Token ids of UTF-8 ``data``: concatenation of the BPE of every piece.

    ``memo`` (optional dict) caches piece -> ids; BPE is a pure function of the
    piece, so the memo never changes the result (the two modes use different
    keys, so one memo may serve both).
    """
    pieces, _ = split_bytes(data, pattern_id)
    out = []
    for p in pieces:
        if memo is not None:
            key = (1, p) if ignore_merges else p
            r = memo.get(key)
            if r is None:
                r = bpe(p, vocab, ignore_merges)
                memo[key] = r
            out.extend(r)
        else:
            out.extend(bpe(p, vocab, ignore_merges))
    return out


def encode_batch(data, offsets, vocab, pattern_id, memo=None, ignore_merges=False):
    """Per-sequence encode of a concatenated batch; returns (ids, out_offsets)."""
    ids, out_off = [], [0]
    for s in range(len(offsets) - 1):
        ids.extend(encode(data[offsets[s]:offsets[s + 1]], vocab, pattern_id, memo, ignore_merges))
        out_off.append(len(ids))
    return ids, out_off


def decode(ids, vocab):
    """Bytes of a token sequence, UTF-8 decoded (strict)."""
    return b"".join(vocab.tok_bytes[i] for i in ids).decode("utf-8")


def token_starts(ids, vocab, base=0):
    """Byte offset where each token begins, plus the end: T + 1 values.

    The device-side byte-offset export (TokTier summary page, §8 Path C and
    Appendix E path C; §4.4 and §7 note that the pages' GPU path emits ids
    only).  Token i covers bytes [starts[i], starts[i+1]) of the input: the
    offsets are the running sum of the tokens' byte lengths, from ``base``.
    """
    starts = [base]
    for i in ids:
        starts.append(starts[-1] + len(vocab.tok_bytes[i]))
    return starts


def encode_offsets(data, offsets, vocab, pattern_id, memo=None, ignore_merges=False):
    """Ids and token starts of a text (offsets None) or a concatenated batch.

    Returns (ids, starts, counts).  Starts are offsets into the whole buffer
    ``data`` (a batch text s begins at offsets[s]); starts[T] = len(data).
    counts is [T] for one text, else the per-text id offsets [B + 1].
    """
    if offsets is None:
        ids = encode(data, vocab, pattern_id, memo, ignore_merges)
        return ids, token_starts(ids, vocab), [len(ids)]
    ids, counts = encode_batch(data, offsets, vocab, pattern_id, memo, ignore_merges)
    starts = []
    for s in range(len(offsets) - 1):
        starts.extend(token_starts(ids[counts[s]:counts[s + 1]], vocab, offsets[s])[:-1])
    starts.append(len(data))
    return ids, starts, counts
