"""Oracle BPE trainer: learns the merge tables the workloads use.

The pages fix no vocabulary, so each workload's merge table is learned here
from a seeded synthetic corpus, which makes this oracle the reference tokenizer
of the project (TokTier summary page, §1.3: the output must equal the reference
tokenizer's).  Byte-level BPE training, read plainly:

  1. split the corpus into pre-tokens with the workload's rule set and count
     each distinct piece;
  2. write every piece as its UTF-8 byte ids, weighted by its count;
  3. repeat up to M times: count every adjacent position pair (x, y) over all
     pieces, weighted; take the pair with the highest count, ties broken by the
     smallest (x, y); stop early when that count is below 2; record it as the
     next merge r (new id 256 + r) and replace its left-to-right
     non-overlapping occurrences in every piece.

The counts are kept incrementally (a piece touched by a merge has all of its
pair contributions removed and re-added) with a lazy max-heap; a test checks
this against recounting from scratch on small corpora.
"""
import heapq
from collections import Counter, defaultdict

from .pretok import split


def piece_counts(text, pattern_id):
    """Distinct pre-tokens of a corpus (str) with their multiplicities."""
    return Counter(split(text, pattern_id))


def train_from_counts(counts, n_merges):
    """Learn up to ``n_merges`` merges from {piece str or bytes: count}.

    Returns (merges, chosen_counts): merges[r] = (x, y) makes id 256 + r.
    """
    words, freq = [], []
    for p, c in counts.items():
        b = p.encode("utf-8") if isinstance(p, str) else bytes(p)
        if len(b) >= 2:
            words.append(list(b))
            freq.append(int(c))

    pair_count = defaultdict(int)
    pair_where = defaultdict(set)
    for wi, w in enumerate(words):
        f = freq[wi]
        for x, y in zip(w, w[1:]):
            pair_count[(x, y)] += f
            pair_where[(x, y)].add(wi)
    heap = [(-c, x, y) for (x, y), c in pair_count.items()]
    heapq.heapify(heap)

    merges, chosen = [], []
    while len(merges) < n_merges and heap:
        negc, a, b = heapq.heappop(heap)
        c = pair_count.get((a, b), 0)
        if c == 0 or -negc != c:
            continue  # stale heap entry
        if c < 2:
            break
        new = 256 + len(merges)
        merges.append((a, b))
        chosen.append(c)
        changed = set()
        for wi in pair_where.pop((a, b)):
            w = words[wi]
            f = freq[wi]
            for x, y in zip(w, w[1:]):
                pair_count[(x, y)] -= f
                changed.add((x, y))
            nw, i = [], 0
            while i < len(w):
                if i + 1 < len(w) and w[i] == a and w[i + 1] == b:
                    nw.append(new)
                    i += 2
                else:
                    nw.append(w[i])
                    i += 1
            words[wi] = nw
            for x, y in zip(nw, nw[1:]):
                pair_count[(x, y)] += f
                pair_where[(x, y)].add(wi)
                changed.add((x, y))
        for p in changed:
            cp = pair_count[p]
            if cp > 0:
                heapq.heappush(heap, (-cp, p[0], p[1]))
            else:
                del pair_count[p]
                pair_where.pop(p, None)
    return merges, chosen


def train_bpe(text, pattern_id, n_merges):
    """Merges learned from a corpus string with rule set ``pattern_id``."""
    return train_from_counts(piece_counts(text, pattern_id), n_merges)
