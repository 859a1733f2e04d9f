"""Write tests/golden/expected.json: oracle results of the full-size workloads.

Calls only the seeded generators (``synth``) and the oracle (``oracle``).  For
every workload it stores the byte and char counts, the number of pre-tokens P
and a SHA-256 of their int32 byte offsets, the number of tokens T and a SHA-256
of the int32 token ids (little endian), a SHA-256 of the int32 byte offset
of every token followed by the byte count, and for the batch workload the
per-sequence token offsets.  The GPU tests compare against these digests.

    python tests/golden/make_golden.py [name ...]
"""
import hashlib
import json
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

from oracle.bpe import Vocab, encode, encode_batch, token_starts  # noqa: E402
from oracle.pretok import piece_starts_batch, split_bytes  # noqa: E402
from synth.text import WORKLOADS, workload  # noqa: E402


def sha(arr):
    return hashlib.sha256(np.ascontiguousarray(arr, dtype="<i4").tobytes()).hexdigest()


def golden(name):
    data, offs, pat, voc = workload(name)
    vocab = Vocab(np.load(os.path.join(ROOT, "data", "vocab_%s.npy" % voc)))
    t0 = time.time()
    memo = {}
    if offs is None:
        _, starts = split_bytes(data, pat)
        ids = encode(data, vocab, pat, memo)
        out_off = None
        tstarts = token_starts(ids, vocab)
    else:
        starts = piece_starts_batch(data, offs.tolist(), pat)
        ids, out_off = encode_batch(data, offs.tolist(), vocab, pat, memo)
        # a batch's texts are contiguous, so the running byte sum over all ids
        # gives offsets into the whole buffer
        tstarts = token_starts(ids, vocab)
    rec = {
        "bytes": len(data),
        "chars": len(data.decode("utf-8")),
        "pattern_id": pat,
        "vocab": voc,
        "pieces": len(starts),
        "pieces_sha256": sha(starts),
        "tokens": len(ids),
        "ids_sha256": sha(ids),
        "token_starts_sha256": sha(tstarts),
        "oracle_s": round(time.time() - t0, 1),
    }
    if out_off is not None:
        rec["seqs"] = len(offs) - 1
        rec["out_offsets"] = [int(x) for x in out_off]
    print(name, {k: v for k, v in rec.items() if k != "out_offsets"}, flush=True)
    return rec


def main(names):
    path = os.path.join(HERE, "expected.json")
    for name in names:
        rec = golden(name)
        cur = {}
        if os.path.exists(path):
            with open(path) as f:
                cur = json.load(f)
        cur[name] = rec
        with open(path, "w") as f:
            json.dump(cur, f, indent=1, sort_keys=True)


if __name__ == "__main__":
    main(sys.argv[1:] or list(WORKLOADS))
