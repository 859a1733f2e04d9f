"""The five workloads at full size on the GPU, against stored oracle digests.

tests/golden/expected.json holds, per workload, the oracle's pre-token offsets,
token ids and token byte offsets as SHA-256 digests (written by tests/golden/make_golden.py,
which calls only the oracle and the seeded generators).  The GPU output must
match them bit for bit, in the same launch configuration bench.py times (one
tt_encode per text, one tt_encode_batch for the 64-text batch).  On a
mismatch the oracle is run in-process to name the first differing token.
"""
import hashlib
import json
import os

import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import exact_byte_level_amd as tt  # noqa: E402
from synth.text import workload  # noqa: E402

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
with open(os.path.join(ROOT, "tests", "golden", "expected.json")) as f:
    EXPECTED = json.load(f)


def sha(a):
    return hashlib.sha256(np.ascontiguousarray(a, dtype="<i4").tobytes()).hexdigest()


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)


def _first_diff(got, data, offs, pat, voc):
    from oracle.bpe import Vocab, encode, encode_batch
    v = Vocab(np.load(os.path.join(ROOT, "data", "vocab_%s.npy" % voc)))
    want = encode(data, v, pat, {}) if offs is None else encode_batch(data, offs.tolist(), v, pat, {})[0]
    want = np.asarray(want, dtype=np.int32)
    k = min(len(got), len(want))
    d = np.nonzero(got[:k] != want[:k])[0]
    return "GPU %d tokens, oracle %d; first difference at %s" % (len(got), len(want), d[0] if len(d) else k)


@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c4", "c5a", "c5b", "c5c", "c5d", "w100k", "o2", "ds"])
def test_workload_bit_exact(name):
    exp = EXPECTED[name]
    data, offs, pat, voc = workload(name)
    print("workload %s: %d bytes, pattern %d, vocab %s" % (name, len(data), pat, voc), flush=True)
    assert len(data) == exp["bytes"]
    tt.load(np.load(os.path.join(ROOT, "data", "vocab_%s.npy" % voc)), pattern_id=pat)
    x = torch.frombuffer(bytearray(data), dtype=torch.uint8).cuda()
    off = None if offs is None else torch.tensor(offs, dtype=torch.int64, device="cuda")
    starts = tt.pretokenize(x, off).cpu().numpy()
    assert len(starts) == exp["pieces"] and sha(starts) == exp["pieces_sha256"]
    if off is None:
        ids = tt.encode(x).cpu().numpy()
    else:
        ids, out_off = tt.encode_batch(x, off)
        ids = ids.cpu().numpy()
        assert out_off.tolist() == exp["out_offsets"]
    if len(ids) != exp["tokens"] or sha(ids) != exp["ids_sha256"]:
        raise AssertionError(_first_diff(ids, data, offs, pat, voc))
    # a second run on the same buffers is identical (no state leaks between calls)
    again = tt.encode(x).cpu().numpy() if off is None else tt.encode_batch(x, off)[0].cpu().numpy()
    assert np.array_equal(again, ids)


@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c4", "c5a", "c5b", "c5c", "c5d", "w100k", "o2", "ds"])
def test_workload_offsets_bit_exact(name):
    """tt_encode_offsets: the same ids, and every token's byte offset equal to
    the oracle's running byte length (digest), at full size."""
    exp = EXPECTED[name]
    data, offs, pat, voc = workload(name)
    print("offsets workload %s: %d bytes, pattern %d, vocab %s" % (name, len(data), pat, voc), flush=True)
    tt.load(np.load(os.path.join(ROOT, "data", "vocab_%s.npy" % voc)), pattern_id=pat)
    x = torch.frombuffer(bytearray(data), dtype=torch.uint8).cuda()
    if offs is None:
        ids, starts = tt.encode_offsets(x)
    else:
        ids, starts, cnt = tt.encode_offsets(x, torch.tensor(offs, dtype=torch.int64, device="cuda"))
        assert cnt.tolist() == exp["out_offsets"]
    ids, starts = ids.cpu().numpy(), starts.cpu().numpy()
    assert len(ids) == exp["tokens"] and sha(ids) == exp["ids_sha256"]
    assert len(starts) == exp["tokens"] + 1 and starts[-1] == len(data)
    assert sha(starts) == exp["token_starts_sha256"]
