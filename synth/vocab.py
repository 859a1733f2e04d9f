"""Seeded merge tables derived from a trained one, for the whole-word rule.

A table learned by BPE training has no token that its own BPE fails to reach,
so the whole-word rule (ignore_merges) would change nothing on it.  Tables of
real models do have such tokens.  ``extend_merges`` appends merges of random
pairs of letter tokens at the end of a trained table (each operand already
exists, so the table stays consistent), which gives the rule something to do,
and ``word_text`` draws text in which the new tokens appear as words.  Only
the byte strings of tokens are computed here, no encoding.
"""
import random


def _token_bytes(merges):
    tb = [bytes([b]) for b in range(256)]
    for x, y in merges:
        tb.append(tb[int(x)] + tb[int(y)])
    return tb


def extend_merges(merges, extra, seed, long_words=False):
    """merges (a sequence of (x, y) pairs) plus ``extra`` new merges of letter
    tokens (the left one may start with a space).  With long_words, only
    pairs whose joined bytes are 17..48 long."""
    merges = [(int(x), int(y)) for x, y in merges]
    tb = _token_bytes(merges)
    letters = [i for i in range(256, len(tb)) if tb[i].lstrip(b" ").isalpha()]
    rng = random.Random(seed)
    have = set(merges)
    target = len(merges) + extra
    while len(merges) < target:
        x, y = rng.choice(letters), rng.choice(letters)
        if (x, y) in have or tb[y].startswith(b" "):
            continue
        if long_words and not 17 <= len(tb[x]) + len(tb[y]) <= 48:
            continue
        have.add((x, y))
        merges.append((x, y))
        tb.append(tb[x] + tb[y])
    return merges


def word_text(merges, first_new, n_parts, seed, filler):
    """Text of n_parts items: half are the byte strings of tokens first_new ..
    (the appended ones), half are drawn by ``filler(k, seed)``, each followed
    by a separator."""
    tb = _token_bytes(merges)
    words = tb[256 + first_new:]
    rng = random.Random(seed)
    parts = []
    for _ in range(n_parts):
        parts.append(rng.choice(words) if rng.random() < 0.5 else filler(rng.randint(5, 60), rng.randint(0, 99)))
        parts.append(rng.choice([b" ", b"\n", b".", b"("]))
    return b"".join(parts)
