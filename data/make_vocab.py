"""Learn and store the merge tables of the three vocabularies.

Calls only the seeded corpus generators (``synth``) and the oracle trainer
(``oracle.train``).  Writes ``data/vocab_<name>.npy`` (int32 [M, 2], merges in
rank order: row r makes token id 256 + r) and records the corpus recipe, the
merge count reached and the file's SHA-256 in ``data/manifest.json``.

    python data/make_vocab.py c1 c2 c3
"""
import hashlib
import json
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(HERE))

from oracle.train import piece_counts, train_from_counts  # noqa: E402
from synth.text import CORPORA, corpus  # noqa: E402


def build(name):
    kind, size, seed, pattern_id, m = CORPORA[name]
    t0 = time.time()
    text = corpus(name).decode("utf-8")
    counts = piece_counts(text, pattern_id)
    t1 = time.time()
    merges, chosen = train_from_counts(counts, m)
    t2 = time.time()
    arr = np.asarray(merges, dtype=np.int32).reshape(-1, 2)
    path = os.path.join(HERE, "vocab_%s.npy" % name)
    np.save(path, arr)
    with open(path, "rb") as f:
        sha = hashlib.sha256(f.read()).hexdigest()
    rec = {
        "corpus": kind, "corpus_chars": size, "corpus_seed": seed,
        "pattern_id": pattern_id, "merges_requested": m, "merges": len(merges),
        "distinct_pieces": len(counts), "last_count": chosen[-1] if chosen else None,
        "sha256": sha, "split_s": round(t1 - t0, 1), "train_s": round(t2 - t1, 1),
    }
    print(name, rec, flush=True)
    return rec


def main(names):
    mpath = os.path.join(HERE, "manifest.json")
    for name in names:
        rec = build(name)
        manifest = {}
        if os.path.exists(mpath):
            with open(mpath) as f:
                manifest = json.load(f)
        manifest[name] = rec
        with open(mpath, "w") as f:
            json.dump(manifest, f, indent=1, sort_keys=True)


if __name__ == "__main__":
    main(sys.argv[1:] or ["c1", "c2", "c3"])
