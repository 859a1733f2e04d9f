"""The whole-word rule (ignore_merges) on the GPU against the oracle.

TokTier summary page, §4.2: for the Llama family the whole pre-token is first
matched against the vocabulary and a match skips the merges (tt_load_bpe_ex
with TT_LOAD_IGNORE_MERGES).  A table learned by BPE training has no token
that its own BPE fails to reach, so the cases append merges of random letter
tokens to a trained table (synth.extend_merges) and draw text with the new
tokens as words (synth.word_text): short words (the whole-pre-token cache)
and words of 17-48 bytes (the hashed whole-word table).  Every case compares
ids (and byte offsets where exported) with oracle.bpe in the same mode,
element by element, and checks that the two modes really differ on it.
"""
import os

import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import exact_byte_level_amd as tt  # noqa: E402
from oracle.bpe import Vocab, encode as oracle_encode, encode_offsets as oracle_offsets  # noqa: E402
from oracle.pretok import CL100K, GPT2  # noqa: E402
from synth import code_text, extend_merges, mix_text, word_text  # noqa: E402

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)
    yield
    torch.cuda.synchronize()


def say(*a):
    print(*a, flush=True)


def dev(data):
    return torch.frombuffer(bytearray(data), dtype=torch.uint8).cuda()


def _mb(n, seed):
    return mix_text(n, seed, multibyte=True)


def _case(name, long_words, seed):
    base = np.load(os.path.join(ROOT, "data", "vocab_%s.npy" % name))
    merges = extend_merges(base, 300, seed, long_words=long_words)
    return len(base), merges, Vocab(merges)


@pytest.mark.parametrize("name,pattern,filler", [("c2", GPT2, code_text), ("c3", CL100K, _mb)])
@pytest.mark.parametrize("long_words", [False, True])
def test_words_against_oracle(name, pattern, filler, long_words):
    first, merges, v = _case(name, long_words, 31 + long_words)
    data = word_text(merges, first, 20_000, 32, filler)
    want_whole = oracle_encode(data, v, pattern, {}, ignore_merges=True)
    want_plain = oracle_encode(data, v, pattern, {})
    assert want_whole != want_plain
    say("whole-word rule: %s pattern %d long_words %s, %d bytes" % (name, pattern, long_words, len(data)))
    tt.load(merges, pattern_id=pattern, ignore_merges=True)
    assert tt.encode(dev(data)).cpu().numpy().tolist() == want_whole
    tt.load(merges, pattern_id=pattern)
    assert tt.encode(dev(data)).cpu().numpy().tolist() == want_plain


def test_batch_and_offsets():
    first, merges, v = _case("c3", True, 33)
    texts = [word_text(merges, first, 300, 40 + k, code_text) for k in range(8)] + [b"", b"x"]
    data = b"".join(texts)
    offs = np.cumsum([0] + [len(t) for t in texts]).astype(np.int64)
    say("whole-word rule: batch of %d texts with offsets, %d bytes" % (len(texts), len(data)))
    tt.load(merges, pattern_id=CL100K, ignore_merges=True)
    ids, starts, cnt = tt.encode_offsets(dev(data), torch.tensor(offs, device="cuda"))
    wi, ws, wc = oracle_offsets(data, offs.tolist(), v, CL100K, {}, ignore_merges=True)
    assert cnt.tolist() == wc
    assert np.array_equal(ids.cpu().numpy(), np.asarray(wi, dtype=np.int32))
    assert np.array_equal(starts.cpu().numpy(), np.asarray(ws, dtype=np.int32))


def test_session_appends():
    first, merges, v = _case("c2", True, 34)
    src = word_text(merges, first, 4_000, 35, code_text)
    tt.load(merges, pattern_id=GPT2, ignore_merges=True)
    s = tt.Session(400_000, 256)
    text = src[:5_000]
    s.reset(dev(text))
    pos = len(text)
    say("whole-word rule: session of %d bytes in appends" % len(src))
    for k in range(30):
        d = src[pos:pos + 37 * (k + 1)]
        pos += len(d)
        s.append(dev(d))
        text += d
        ids = s.ids().cpu().numpy().tolist()
        assert ids == oracle_encode(text, v, GPT2, {}, ignore_merges=True), k
    s.close()


def test_trained_table_unchanged():
    merges = np.load(os.path.join(ROOT, "data", "vocab_c1.npy"))
    data = code_text(100_000, 36)
    say("whole-word rule on a trained table, %d bytes" % len(data))
    tt.load(merges, pattern_id=GPT2, ignore_merges=True)
    whole = tt.encode(dev(data)).cpu().numpy()
    tt.load(merges, pattern_id=GPT2)
    assert np.array_equal(whole, tt.encode(dev(data)).cpu().numpy())
