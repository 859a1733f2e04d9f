"""Vocabularies wider than 2^16 ids on the GPU, against the oracle.

The pair-rank table stores a 32-bit key per slot: with ids below 2^v it keeps
x << (32 - v) | y >> (2v - 32) and spreads the buckets over 2^(2v - 32)
partitions by (x ^ y), which give back the dropped bits of y.  The trained
tables here have v = 16 (50K merges: no partition) and v = 17 (100K: 4
partitions); these cases extend the 50K table with merges of random letter
tokens (synth.extend_merges, a consistent table) to 150,000 merges (v = 18,
16 partitions) and 530,000 merges (v = 20, 256 partitions, ids up to
530,255) and encode text whose words are the new tokens' byte strings, so
that merges into ids above 2^17 and 2^19 happen.  Ids and byte offsets must
equal the oracle's.
"""
import os

import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import exact_byte_level_amd as tt  # noqa: E402
from oracle.bpe import Vocab, encode as oracle_encode, encode_offsets as oracle_offsets  # noqa: E402
from oracle.pretok import GPT2  # noqa: E402
from synth import extend_merges, mix_text, word_text  # noqa: E402

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)
    yield
    torch.cuda.synchronize()


@pytest.mark.parametrize("n_merges,v_bits", [(150_000, 18), (530_000, 20)])
def test_wide_vocabulary_against_oracle(n_merges, v_bits):
    base = np.load(os.path.join(ROOT, "data", "vocab_c2.npy"))
    merges = np.asarray(extend_merges(base, n_merges - len(base), seed=n_merges), dtype=np.int32)
    assert (1 << (v_bits - 1)) < 256 + len(merges) <= (1 << v_bits)
    text = word_text(merges, len(base), 3000, 7, lambda k, s: mix_text(k, s))
    print("wide vocabulary: %d merges, %d bytes" % (len(merges), len(text)), flush=True)
    tt.load(merges, pattern_id=GPT2)
    v = Vocab(merges)
    want = np.asarray(oracle_encode(text, v, GPT2), dtype=np.int32)
    assert int(want.max()) >= 1 << 17  # merges into the wide ids do happen
    x = torch.frombuffer(bytearray(text), dtype=torch.uint8).cuda()
    got = tt.encode(x).cpu().numpy()
    assert len(got) == len(want)
    d = np.nonzero(got != want)[0]
    assert len(d) == 0, int(d[0])
    ids, starts = tt.encode_offsets(x)
    wi, ws, _ = oracle_offsets(text, None, v, GPT2, {})
    assert np.array_equal(ids.cpu().numpy(), np.asarray(wi, dtype=np.int32))
    assert np.array_equal(starts.cpu().numpy(), np.asarray(ws, dtype=np.int32))
