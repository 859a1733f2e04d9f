"""Pins for the oracle BPE trainer (oracle.train).

What pins it, besides itself:
  * a from-scratch trainer written here (recount every pair of every piece at
    every step, no incremental state, no heap) must learn the same table;
  * invariants: the chosen counts never increase; every merge uses ids that
    already exist (a consistent table); the learned vocabulary round-trips;
  * determinism: the stored tables carry a SHA-256, and re-learning the small
    table from its seeded corpus reproduces the stored file.
"""
import hashlib
import io
import json
import os
from collections import Counter

import numpy as np
import pytest

from oracle.bpe import Vocab, decode, encode
from oracle.pretok import CL100K, GPT2, split
from oracle.train import train_bpe, train_from_counts

DATA = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "data")


def recount_trainer(text, pattern_id, n_merges):
    words = Counter(tuple(p.encode()) for p in split(text, pattern_id))
    merges, chosen = [], []
    while len(merges) < n_merges:
        counts = Counter()
        for w, f in words.items():
            for i in range(len(w) - 1):
                counts[(w[i], w[i + 1])] += f
        if not counts:
            break
        best = min(counts, key=lambda p: (-counts[p], p))
        if counts[best] < 2:
            break
        new = 256 + len(merges)
        merges.append(best)
        chosen.append(counts[best])
        nw = Counter()
        for w, f in words.items():
            out, i = [], 0
            while i < len(w):
                if i + 1 < len(w) and (w[i], w[i + 1]) == best:
                    out.append(new)
                    i += 2
                else:
                    out.append(w[i])
                    i += 1
            nw[tuple(out)] += f
        words = nw
    return merges, chosen


@pytest.mark.parametrize("pattern_id,seed", [(GPT2, 1), (CL100K, 2), (CL100K, 3)])
def test_incremental_equals_recount(pattern_id, seed):
    from synth import mix_text
    text = mix_text(6_000, seed, multibyte=(seed == 3)).decode()
    got = train_bpe(text, pattern_id, 250)
    want = recount_trainer(text, pattern_id, 250)
    assert got == want


def test_early_stop_when_no_pair_repeats():
    merges, chosen = train_from_counts({"ab": 1, "cd": 1}, 10)
    assert merges == [] and chosen == []
    merges, chosen = train_from_counts({"abab": 1}, 10)
    # (a,b) occurs twice -> merged; then (ab,ab) occurs once -> stop
    assert merges == [(97, 98)] and chosen == [2]


def test_tie_break_smallest_pair():
    merges, _ = train_from_counts({"ba": 3, "ab": 3}, 1)
    assert merges == [(97, 98)]


def test_stored_tables_invariants_and_digests():
    with open(os.path.join(DATA, "manifest.json")) as f:
        manifest = json.load(f)
    for name, rec in manifest.items():
        path = os.path.join(DATA, "vocab_%s.npy" % name)
        with open(path, "rb") as f:
            raw = f.read()
        assert hashlib.sha256(raw).hexdigest() == rec["sha256"]
        arr = np.load(io.BytesIO(raw))
        assert arr.dtype == np.int32 and arr.shape == (rec["merges"], 2)
        Vocab(arr)  # raises unless consistent and duplicate-free


def test_chosen_counts_non_increasing_and_round_trip():
    from synth import code_text
    text = code_text(200_000, 17).decode()
    merges, chosen = train_bpe(text, GPT2, 1500)
    assert all(a >= b for a, b in zip(chosen, chosen[1:]))
    v = Vocab(merges)
    probe = code_text(5_000, 18)
    assert decode(encode(probe, v, GPT2), v).encode() == probe


@pytest.mark.slow
def test_small_table_reproduces_from_seed():
    from synth.text import CORPORA, corpus
    _, _, _, pat, m = CORPORA["c1"]
    merges, _ = train_bpe(corpus("c1").decode(), pat, m)
    stored = np.load(os.path.join(DATA, "vocab_c1.npy"))
    assert np.array_equal(np.asarray(merges, dtype=np.int32), stored)
