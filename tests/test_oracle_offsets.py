"""Pins for the oracle's token byte offsets (oracle.bpe.token_starts).

The device-side byte-offset export is Path C of the TokTier summary page (§8
and Appendix E); §4.4 and §7 there note that the pages' own GPU path emits ids
only.  The oracle gives token i the byte span [starts[i], starts[i+1]).

What pins it, besides itself:
  * a hand-worked example (below), offsets counted by hand;
  * closed form: with no merges every token is one byte, so starts = 0..n;
  * invariants from an independent stage: every pre-token start of the split
    (oracle.pretok, which knows nothing of BPE) is a token start, the offsets
    rise strictly and end at n, and the bytes of each span are the bytes the
    decoder gives for that token;
  * a third-party implementation: HF ``tokenizers`` built from the same merges
    reports the same (start, end) spans on ASCII text, where its char offsets
    are byte offsets;
  * batch: the spans of every text are its own spans shifted by the text's
    start in the buffer.
"""
import os

import numpy as np
import pytest

from oracle.bpe import Vocab, decode, encode, encode_offsets, token_starts
from oracle.pretok import CL100K, GPT2, split_bytes

DATA = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "data")


def _vocab(name):
    return Vocab(np.load(os.path.join(DATA, "vocab_%s.npy" % name)))


def test_hand_worked_example():
    # merges: r0 = (l, l) -> 256 "ll", r1 = (h, e) -> 257 "he",
    # r2 = (257, 256) -> 258 "hell", r3 = (258, o) -> 259 "hello".
    # GPT-2-style split of "hello  hello": "hello" | " " | " hello" (a run of
    # two spaces before a letter gives up its last space to the word).
    # "hello" -> [259]; " " -> [32]; " hello" -> [32, 259].
    # Spans: [0,5) "hello", [5,6) " ", [6,7) " ", [7,12) "hello".
    v = Vocab([(108, 108), (104, 101), (257, 256), (258, 111)])
    data = b"hello  hello"
    ids, starts, counts = encode_offsets(data, None, v, GPT2)
    assert ids == [259, 32, 32, 259]
    assert starts == [0, 5, 6, 7, 12]
    assert counts == [4]


@pytest.mark.parametrize("pat", [GPT2, CL100K])
def test_no_merges_gives_every_byte(pat):
    from synth import mix_text
    v = Vocab([])
    data = mix_text(3_000, 5, multibyte=True)
    ids, starts, _ = encode_offsets(data, None, v, pat)
    assert ids == list(data)
    assert starts == list(range(len(data) + 1))


@pytest.mark.parametrize("pat", [GPT2, CL100K])
def test_spans_tile_the_text_and_hold_piece_starts(pat):
    from synth import code_text, mix_text
    v = _vocab("c1")
    for data in (code_text(20_000, 3), mix_text(8_000, 4, multibyte=True), b"", b"a", b"a" * 5000):
        ids, starts, counts = encode_offsets(data, None, v, pat)
        assert counts == [len(ids)] and len(starts) == len(ids) + 1
        assert starts[0] == 0 and starts[-1] == len(data)
        assert all(a < b for a, b in zip(starts, starts[1:]))
        _, pstarts = split_bytes(data, pat)
        assert set(pstarts) <= set(starts)
        for i, t in enumerate(ids):
            assert data[starts[i]:starts[i + 1]] == v.tok_bytes[t]
        assert decode(ids, v).encode() == data


def test_batch_spans_are_shifted_text_spans():
    from synth import code_text, mix_text
    v = _vocab("c1")
    texts = [code_text(3_000, 11), b"", mix_text(2_000, 12, multibyte=True), b" ", code_text(500, 13)]
    data = b"".join(texts)
    offs = [0]
    for t in texts:
        offs.append(offs[-1] + len(t))
    ids, starts, counts = encode_offsets(data, offs, v, CL100K)
    assert len(starts) == len(ids) + 1 and starts[-1] == len(data)
    for s, t in enumerate(texts):
        own = token_starts(encode(t, v, CL100K), v)
        assert starts[counts[s]:counts[s + 1]] == [offs[s] + x for x in own[:-1]]


def _bytes_to_unicode():
    # GPT-2's printable remapping of the 256 byte values, as HF ByteLevel uses it.
    bs = list(range(ord("!"), ord("~") + 1)) + list(range(0xA1, 0xAD)) + list(range(0xAE, 0x100))
    cs = bs[:]
    k = 0
    for b in range(256):
        if b not in bs:
            bs.append(b)
            cs.append(256 + k)
            k += 1
    return {b: chr(c) for b, c in zip(bs, cs)}


def test_matches_hf_tokenizers_offsets():
    tk = pytest.importorskip("tokenizers")
    from synth import code_text
    v = _vocab("c1")
    m = _bytes_to_unicode()
    strs = ["".join(m[b] for b in t) for t in v.tok_bytes]
    if len(set(strs)) != len(strs):
        pytest.skip("vocab has two tokens with the same bytes")
    model = tk.models.BPE(vocab={s: i for i, s in enumerate(strs)},
                          merges=[(strs[x], strs[y]) for x, y in v.merges])
    tok = tk.Tokenizer(model)
    tok.pre_tokenizer = tk.pre_tokenizers.ByteLevel(add_prefix_space=False, use_regex=True)
    text = code_text(30_000, 78)
    enc = tok.encode(text.decode())
    ids = encode(text, v, GPT2)
    assert enc.ids == ids
    starts = token_starts(ids, v)
    assert [a for a, _ in enc.offsets] == starts[:-1]
    assert [b for _, b in enc.offsets] == starts[1:]
