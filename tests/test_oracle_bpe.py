"""Pins for the oracle BPE and encoder (oracle.bpe).

What pins it, besides itself:
  * brute force: on every word of length <= 6 over {a, b, c, space} and many
    random consistent merge tables, the classic loop, the heap form and the
    naive "merge rank r everywhere, r = 0, 1, ..." must agree;
  * the non-concatenativity example of TokTier summary page §1.2 / §3.2: with
    a vocabulary where "pipe" and "pipeline" are single tokens,
    tok("pipe") + tok("line") differs from tok("pipeline");
  * closed forms: no merges gives the UTF-8 bytes; a doubling chain vocabulary
    turns a run of L letters into the binary expansion of L;
  * a hand-worked example where merging local minima in parallel goes wrong
    and the classic loop does not;
  * round trip decode(encode(x)) == x, and the factorisation
    encode(text) == concat(BPE(piece)) of Appendix A.1;
  * a third-party implementation: HF ``tokenizers`` BPE built from the same
    merges must give the same ids on a whole GPT-2-style text.
"""
import itertools
import os
import random

import numpy as np
import pytest

from oracle.bpe import Vocab, bpe, bpe_classic, bpe_heap, bpe_naive, decode, encode
from oracle.pretok import CL100K, GPT2, split_bytes

DATA = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "data")


def random_consistent_table(rng, alphabet, n_merges):
    """Random merge table whose operands always exist before the merge."""
    ids = list(alphabet)
    merges, seen = [], set()
    tries = 0
    while len(merges) < n_merges and tries < 50 * n_merges:
        tries += 1
        x, y = rng.choice(ids), rng.choice(ids)
        if (x, y) in seen:
            continue
        seen.add((x, y))
        merges.append((x, y))
        ids.append(256 + len(merges) - 1)
    return merges


def test_brute_force_classic_heap_naive_agree():
    alpha = [ord(c) for c in "abc "]
    words = [list(t) for n in range(7) for t in itertools.product(alpha, repeat=n)]
    assert len(words) == 5461
    rng = random.Random(3)
    for _ in range(25):
        merges = random_consistent_table(rng, alpha, rng.randint(1, 14))
        v = Vocab(merges)
        for w in words:
            c = bpe_classic(w, v.rank)
            assert bpe_naive(w, merges) == c
            assert bpe_heap(w, v.rank) == c


def test_random_long_words_heap_matches_classic():
    rng = random.Random(4)
    for _ in range(200):
        merges = random_consistent_table(rng, [97, 98, 99], rng.randint(1, 40))
        v = Vocab(merges)
        w = [rng.choice([97, 98, 99]) for _ in range(rng.randint(0, 300))]
        assert bpe_heap(w, v.rank) == bpe_classic(w, v.rank) == bpe_naive(w, merges)


def _tiny_pipe_vocab():
    # ids: p=112 i=105 e=101 l=108 n=110
    merges = [(112, 105), (256, 112), (257, 101),    # pi, pip, pipe(258)
              (108, 105), (259, 110), (260, 101),    # li, lin, line(261)
              (258, 261)]                            # pipeline(262)
    return Vocab(merges)


def test_pipe_line_not_concatenative():
    v = _tiny_pipe_vocab()
    a, b, ab = (encode(s, v, GPT2) for s in (b"pipe", b"line", b"pipeline"))
    assert a == [258] and b == [261] and ab == [262]
    assert a + b != ab
    assert v.tok_bytes[262] == b"pipeline"


def test_zero_merges_gives_utf8_bytes():
    v = Vocab([])
    text = "héllo 世界 😀 12\n".encode()
    assert encode(text, v, CL100K) == list(text)


@pytest.mark.parametrize("length", list(range(0, 40)) + [1000, 100_003])
def test_doubling_chain_closed_form(length):
    # a+a -> a2 (256), a2+a2 -> a4 (257), a4+a4 -> a8 (258)
    v = Vocab([(97, 97), (256, 256), (257, 257)])
    got = bpe(b"a" * length, v)
    want = [258] * (length // 8)
    rem = length % 8
    for bit, tok in ((4, 257), (2, 256), (1, 97)):
        if rem & bit:
            want.append(tok)
    assert got == want


def test_local_minimum_counterexample():
    # r0 = (a,b), r1 = (ab,b), r2 = (b,a).  "abba": classic merges (a,b) first,
    # then (ab,b) beats (b,a): [abb, a].  Merging the local minima (a,b) and
    # (b,a) in one step would give [ab, ba] instead.
    v = Vocab([(97, 98), (256, 98), (98, 97)])
    assert bpe_classic(b"abba", v.rank) == [257, 97]
    assert bpe_naive(b"abba", v.merges) == [257, 97]


def test_equal_pair_runs_merge_leftmost_first():
    v = Vocab([(97, 97)])
    assert bpe_classic(b"aaa", v.rank) == [256, 97]
    assert bpe_classic(b"aaaaa", v.rank) == [256, 256, 97]


def test_vocab_rejects_inconsistent_tables():
    with pytest.raises(ValueError):
        Vocab([(97, 256)])
    with pytest.raises(ValueError):
        Vocab([(97, 98), (97, 98)])


def _vocab(name):
    return Vocab(np.load(os.path.join(DATA, "vocab_%s.npy" % name)))


def test_round_trip_and_factorisation_on_code_text():
    from synth import code_text, mix_text
    v = _vocab("c1")
    for text in (code_text(20_000, 9), mix_text(5_000, 9, multibyte=True)):
        for pat in (GPT2, CL100K):
            ids = encode(text, v, pat)
            assert decode(ids, v).encode() == text
            pieces, _ = split_bytes(text, pat)
            assert ids == [t for p in pieces for t in bpe_classic(p, v.rank)]
            assert len(pieces) <= len(ids) <= len(text)


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


def test_matches_hf_tokenizers_bpe():
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
    text = code_text(30_000, 77)
    assert tok.encode(text.decode()).ids == encode(text, v, GPT2)
