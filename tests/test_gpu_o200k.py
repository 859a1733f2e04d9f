"""o200k-style rules on the GPU (tt_pretokenize and tt_encode through the C ABI)
against the CPU oracle, bit for bit.

Brute force over every string of length <= 5 of a class-covering alphabet
(both cases, an Lo letter, a combining mark, '/', contraction letters), random
multibyte strings, runs that cross tiles for each fact carried between tiles
(digit groups, whitespace before CR/LF, CR/LF after "other" chars, CR/LF/'/'
tails, upper-case runs to the end of a word, Lm/Lo runs after a lower-case
letter), contraction chains (back-to-back suffixes, whose attachment
alternates from the chain's first suffix) inside a tile, across tile starts
and over whole tiles, Lm/Lo/mark runs into a tile right after a contraction,
and a 1M-char encode.
"""
import itertools
import os
import random
import re

import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import exact_byte_level_amd as tt  # noqa: E402
from oracle.bpe import Vocab, encode as oracle_encode, encode_batch as oracle_encode_batch, token_starts  # noqa: E402
from oracle.pretok import O200K, piece_starts_batch, split_bytes  # noqa: E402
from synth import mix_text  # noqa: E402

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
# an apostrophe with a contraction shape after it, right after another one
_SHAPE = "(?:[sStTmMdD]|[rRvV][eE]|[lL][lL])"
CHAIN = re.compile("'" + _SHAPE + "'" + _SHAPE)


def say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)
    yield
    torch.cuda.synchronize()


def dev(data):
    return torch.frombuffer(bytearray(data), dtype=torch.uint8).cuda() if len(data) else torch.empty(
        0, dtype=torch.uint8, device="cuda")


def load(name="c3"):
    merges = np.load(os.path.join(ROOT, "data", "vocab_%s.npy" % name))
    tt.load(merges, pattern_id=O200K)
    return Vocab(merges)


def batch(strings):
    data, offs = b"", [0]
    for s in strings:
        data += s.encode()
        offs.append(len(data))
    return data, offs


def gpu_starts(data, offsets=None):
    off = None if offsets is None else torch.tensor(offsets, dtype=torch.int64, device="cuda")
    return tt.pretokenize(dev(data), off).cpu().numpy().tolist()


def check_batch(strings):
    """GPU starts of the batch equal the oracle's; on a difference, name the
    first string where they part."""
    data, offs = batch(strings)
    got, want = gpu_starts(data, offs), piece_starts_batch(data, offs, O200K)
    if got == want:
        return
    k = next((i for i, (a, b) in enumerate(zip(got, want)) if a != b), min(len(got), len(want)))
    pos = min(got[k] if k < len(got) else len(data), want[k] if k < len(want) else len(data))
    s = int(np.searchsorted(np.asarray(offs), pos, side="right")) - 1
    raise AssertionError("first difference in string %d %r: gpu %s oracle %s" % (
        s, strings[s], [x - offs[s] for x in got if offs[s] <= x < offs[s + 1]],
        [x - offs[s] for x in want if offs[s] <= x < offs[s + 1]]))


ALPHA = ["a", "A", "s", "S", "r", "e", "ª", "́", "1", ".", "/", "'", " ", "\n"]


def test_every_short_string():
    load()
    strings = ["".join(t) for n in range(6) for t in itertools.product(ALPHA, repeat=n)]
    assert sum(1 for s in strings if CHAIN.search(s)) == 120
    say("o200k brute force: %d strings" % len(strings))
    check_batch(strings)


ALPHA2 = ALPHA + list("lLvVmMdDtTEéÉ中\U0001f600") + [
    "　", "\xa0", "2", "²", "_", "(", "\t", "\r", "ǅ", "ʰ", "कि", "İ", "ß"]


def test_random_multibyte_strings():
    load()
    rng = random.Random(91)
    strings = []
    while len(strings) < 40_000:
        s = "".join(rng.choice(ALPHA2) for _ in range(rng.randint(0, 40)))
        strings.append(s)
    say("o200k random batch: %d strings" % len(strings))
    check_batch(strings)


LONG_RUNS = [
    "a" + "1" * 20_000 + "x" + "2" * 4_097,                 # digit groups
    ".\n" + "\n" * 9_000 + " " * 9_000 + "z",             # CR/LF after "other", whitespace
    "x" + " " * 8_191 + "\n" + " " * 8_193,               # whitespace run ending in CR/LF
    "*/\n" + "/" * 5_000 + "x",                           # a tail of '/' across tiles
    "a.\n" + "/\n" * 3_000 + ".b",                        # interleaved tail
    "q" + "/" * 4_000 + "\n" + "y",                       # '/' in the "other" run, then a tail
    "x" + "A" * 5_000 + "b" + "C" * 3_000 + ".",          # upper-case runs: to the word end or not
    "x" + "中" * 3_000 + "A" + "中" * 2_000 + "Bc",  # Lo runs after a lower-case letter
    "X" + "ª" * 3_000 + "AB",                        # Lo run after upper case, upper tail
    "́" * 4_000 + "AB" + "ª" * 2_000 + "C",     # marks run
    "it's" + "b" * 6_000 + "'re" + "c" * 3,                # contractions around a long word
]


def test_runs_crossing_tiles():
    load()
    for text in LONG_RUNS:
        data = text.encode()
        say("o200k long runs: %d bytes" % len(data))
        _, want = split_bytes(data, O200K)
        assert gpu_starts(data) == want
    check_batch(LONG_RUNS)


def _tile_edge_text(seed, tile=1024, ntiles=48):
    rng = random.Random(seed)
    runs = [" ", "7", "x", "X", ".", "\n", "\t", "'", "\r\n", "/", "ª", "́", "\n/"]
    out = bytearray()
    for t in range(1, ntiles):
        edge = t * tile
        ch = rng.choice(runs)
        k = rng.choice([1, 2, 3, 15, 16, 17, 31, 32, 33, 60, 64, 70, 130])
        left = rng.randint(0, k)
        while len(out) < edge - left * len(ch.encode()):
            word = rng.choice(["ab", "don't", "we're", "x1", "Il", "HTMLParser", "9", "..", " ", "\n", "a/b",
                               "Été", "CamelCase"])
            out += word.encode()
        out += (ch * k).encode()
        out += rng.choice([b"'s", b"'LL", b"q", b"Q", b"1", b"!", b" ", b"/", b"\n"])
    return bytes(out)


def test_runs_across_tile_edges():
    data = _tile_edge_text(77)
    assert not CHAIN.search(data.decode())
    v = load("c1")
    say("o200k tile edges: %d bytes" % len(data))
    _, want = split_bytes(data, O200K)
    assert gpu_starts(data) == want
    got = tt.encode(dev(data)).cpu().numpy()
    assert np.array_equal(got, np.asarray(oracle_encode(data, v, O200K, {}), dtype=np.int32))


def test_encode_mix_1m():
    v = load("c3")
    data = mix_text(1_000_000, 203, multibyte=True)
    say("o200k encode: %d bytes" % len(data))
    got = tt.encode(dev(data)).cpu().numpy()
    want = np.asarray(oracle_encode(data, v, O200K, {}), dtype=np.int32)
    assert np.array_equal(got, want)


CHAIN_TEXTS = ["a's's", "it's'll go", "x" * 3000 + "'d've", "'s's's", " 's's", "a'S'Re'll'd", "A'LL'M'T'D'S'VE",
               "Don't'cha", "rock'n'roll's'", "3's's", "x's'sa's", "'rE's'm", "y" * 100 + "'s" * 300 + " z"]


def _chain_edge_text(seed, units=(1, 4), tile=1024, ntiles=40):
    """At each tile start, a chain of shapes (their count drawn from units)
    whose first shape lies before it, after a letter or a space, so that the
    tile start falls anywhere in the chain."""
    rng = random.Random(seed)
    shapes = ["'s", "'S", "'t", "'m", "'d", "'re", "'Re", "'rE", "'ve", "'ll", "'LL"]
    out = bytearray()
    for t in range(1, ntiles):
        chain = "".join(rng.choice(shapes) for _ in range(rng.randint(*units))).encode()
        head = t * tile - rng.randint(0, len(chain) - 1)
        if head - 1 <= len(out):
            continue
        while len(out) < head - 1:
            out += rng.choice([b"ab ", b"it ", b"x1 ", b"Q ", b". ", b"\n"])
        del out[head - 1:]
        out += rng.choice([b"a", b" ", b"Z", b"."])
        out += chain + rng.choice([b" ", b"x", b"'", b"!", b"\n"])
    return bytes(out)


def _check_text(text, v):
    data = text.encode()
    say("o200k chain: %d bytes %r" % (len(data), text[-12:]))
    _, want = split_bytes(data, O200K)
    assert gpu_starts(data) == want
    got = tt.encode(dev(data)).cpu().numpy()
    assert np.array_equal(got, np.asarray(oracle_encode(data, v, O200K, {}), dtype=np.int32))


def test_contraction_chains():
    v = load()
    texts = CHAIN_TEXTS + [_chain_edge_text(s).decode() for s in (5, 6, 7)]
    for text in texts:
        _check_text(text, v)
    check_batch(texts)
    # a lone contraction and a quote after one
    for text in ["it's", "'it's'", "rock'n'roll"]:
        got = tt.encode(dev(text.encode())).cpu().numpy()
        assert np.array_equal(got, np.asarray(oracle_encode(text.encode(), v, O200K, {}), dtype=np.int32))


def test_long_chains_across_tiles():
    """Chains whose first shape lies tiles before the tile start: the chain
    state is carried between tiles."""
    v = load()
    texts = ["x" + "'s" * 2000, " " * 1000 + "'re" * 10 + " a", "Q" + "'d're'LL" * 700 + "x",
             "'" + "s'" * 3000, " " * 1020 + "'s" * 20 + "A", "y" * 1015 + "'rE" * 5 + "'m" * 900 + "ª" * 9 + "Ab"]
    texts += [_chain_edge_text(s, units=(5, 40)).decode() for s in (8, 9)]
    texts += [_chain_edge_text(s, units=(200, 900), ntiles=24).decode() for s in (10,)]
    for text in texts:
        _check_text(text, v)
    # the same texts as one batch: chains cut by sequence starts
    check_batch(texts + ["'s's", "x's'" + "d's" * 700, "'ll" * 400])


def test_mark_runs_after_contractions_across_tiles():
    """An Lm/Lo/mark run that reaches a tile start right after a contraction:
    whether the contraction attached (then the run restarts the word) decides
    the split of an upper-case letter after the run.  The run's start, the
    contraction or its chain's head may lie before the tile's view."""
    v = load()
    texts = []
    for lead in ["it's", "a's's", "its", "x'S", "x're're", "It'd", "I'm'", "x'LL'd"]:
        for run in ["中" * 600, "ª" * 700, "́" * 530, "ª" * 7, "ʰ" * 3]:
            for pad in (0, 1, 5, 1000):
                texts.append("y " * pad + lead + run + "Ab")
    # a chain that ends just before a tile's halo, its head out of view, then
    # an Lo run up to the tile start: both parities of the chain
    for units in (19, 20):
        t = "y " * 484 + "yx" + "'s" * 20 + "ª" * 7 + "Ab"
        texts.append(t if units == 20 else t.replace("yx'", "yx''", 1))
    for text in texts:
        _check_text(text, v)
    check_batch(texts)


def test_random_chain_and_mark_text():
    """A long random text of contraction shapes, apostrophes, Lm/Lo/marks,
    case runs and separators: every tile start falls somewhere random in it."""
    v = load()
    toks = ["'s", "'re", "'ll", "'d", "'S", "'LL", "'Ve", "'", "a", "A", "s", "e", "l", "中", "ª", "́", "ʰ",
            " ", "x", "\n", "1", "AB", "Ab", ".", "y's"]
    for seed in (1, 2):
        rng = random.Random(seed)
        text = "".join(rng.choice(toks) for _ in range(90_000))
        _check_text(text, v)


def test_chain_batch_encode_and_offsets():
    """tt_encode_batch and tt_encode_offsets on a batch of chain and mark-run
    texts (sequence starts inside chains and runs): ids, per-sequence token
    offsets and every token's byte start against the oracle."""
    v = load()
    texts = CHAIN_TEXTS + ["x" + "'s" * 700, "'ll" * 400, "it's" + "中" * 600 + "Ab", "a's's" + "ª" * 700 + "Ab",
                           _chain_edge_text(11, units=(5, 40), ntiles=12).decode(), "", "'", "s", "ª" * 5 + "A"]
    data, offs = batch(texts)
    want_ids, want_off = oracle_encode_batch(data, offs, v, O200K, {})
    off_t = torch.tensor(offs, dtype=torch.int64, device="cuda")
    say("o200k chain batch: %d texts, %d bytes" % (len(texts), len(data)))
    ids, out_off = tt.encode_batch(dev(data), off_t)
    assert out_off.tolist() == want_off
    assert np.array_equal(ids.cpu().numpy(), np.asarray(want_ids, dtype=np.int32))
    ids2, starts, cnt = tt.encode_offsets(dev(data), off_t)
    assert cnt.tolist() == want_off
    assert np.array_equal(ids2.cpu().numpy(), np.asarray(want_ids, dtype=np.int32))
    want_st = []
    for q in range(len(texts)):
        want_st += token_starts(want_ids[want_off[q]:want_off[q + 1]], v, offs[q])[:-1]
    assert starts.cpu().numpy().tolist() == want_st + [len(data)]


def test_sessions_are_refused():
    load()
    s = tt.Session(1024) if hasattr(tt, "Session") else None
    if s is None:
        pytest.skip("no session binding")
    with pytest.raises(tt.TTError) as ei:
        s.reset(dev(b"hello world"))
    assert ei.value.code == tt.TT_EINVAL
