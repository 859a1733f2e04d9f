"""Pieces longer than 2 KiB on the GPU: chunked encodes stitched at compatible
token pairs, with exact global-minimum rounds as the fallback -- all against
the oracle.

A long piece is cut into 32-byte chunks counted from its first byte; each
chunk is encoded alone and neighbouring chunks join where their edge tokens
are compatible, else a re-encoded window replaces the tokens around the
junction.  A junction that no window within the limits repairs sends the
whole piece to the rounds.  The cases below are built so that both paths
run, and that they meet in one tile:
  * random words (2 to 26 letters) at many lengths and offsets: stitched, with
    repair windows at a good share of the junctions;
  * runs of one byte: every full chunk comes from the run table;
  * a run of spaces of length 32 k + 1 under the cl100k-style table: the last
    chunk is one space, and 16 spaces + 1 space is itself a token, so the last
    junction cannot be repaired (fallback);
  * the doubling-chain table (a, aa, ..., a^4096): a 32-byte chunk is one
    token and two of them merge, so every junction fails (fallback);
  * a fallback piece and a stitched piece ending and starting in one tile,
    with ordinary text before and after;
  * batches with long pieces at text edges, and byte offsets of both kinds.
"""
import os
import random

import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import exact_byte_level_amd as tt  # noqa: E402
from oracle.bpe import Vocab, encode as oracle_encode, encode_batch as oracle_batch  # noqa: E402
from oracle.bpe import encode_offsets as oracle_offsets  # noqa: E402
from oracle.pretok import CL100K, GPT2  # noqa: E402
from synth import mix_text, random_word  # noqa: E402

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
K_CHAIN = 12
CHAIN = np.asarray([(97, 97)] + [(256 + i, 256 + i) for i in range(K_CHAIN - 1)], dtype=np.int32)


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)
    yield
    torch.cuda.synchronize()


def say(*a):
    print(*a, flush=True)


def load(name, pattern):
    merges = np.load(os.path.join(ROOT, "data", "vocab_%s.npy" % name))
    tt.load(merges, pattern_id=pattern)
    return Vocab(merges)


def gpu(data):
    return tt.encode(torch.frombuffer(bytearray(data), dtype=torch.uint8).cuda()).cpu().numpy()


def check(data, v, pattern, what):
    say("%s: %d bytes, pattern %d" % (what, len(data), pattern))
    want = np.asarray(oracle_encode(data, v, pattern, {}), dtype=np.int32)
    got = gpu(data)
    assert len(got) == len(want), (what, len(got), len(want))
    d = np.nonzero(got != want)[0]
    assert len(d) == 0, (what, int(d[0]))


@pytest.mark.parametrize("pattern,voc", [(GPT2, "c2"), (CL100K, "c3")])
def test_random_words_at_many_lengths_and_offsets(pattern, voc):
    v = load(voc, pattern)
    rng = random.Random(71 + pattern)
    alphabets = ["ab", "acgt", "etaoinshrdlu", "abcdefghijklmnopqrstuvwxyz"]
    parts = []
    for k, length in enumerate((2049, 2050, 2079, 2080, 2081, 3072, 4095, 4096, 4097, 9000, 33_000)):
        parts.append(mix_text(rng.randint(1, 2500), 300 + k))
        parts.append(b" ")
        parts.append(random_word(length, 500 + k, alphabets[k % 4]))
    parts.append(b".")
    check(b"".join(parts), v, pattern, "random words")


def test_one_byte_runs_take_the_run_table():
    for voc, pattern in (("c2", GPT2), ("c3", CL100K)):
        v = load(voc, pattern)
        parts = []
        for k, ch in enumerate(b" \tz9_\n"):
            parts.append(code_like(700 + k))
            parts.append(bytes([ch]) * (2048 + 32 * k + 7 * k * k))
        check(b"".join(parts) + b"end", v, pattern, "one-byte runs")


def code_like(seed):
    return mix_text(random.Random(seed).randint(10, 1500), seed) + b"x"


def test_space_run_whose_last_junction_fails():
    v = load("c3", CL100K)
    for k in (65, 66, 97, 200):
        # the spaces before the final letter: 32 k + 1 of them end the run piece
        data = b"ab " + b" " * (32 * k + 1) + b"y" + mix_text(500, 77)
        check(data, v, CL100K, "space run of %d" % (32 * k + 2))


def test_chain_table_falls_back_to_rounds():
    tt.load(CHAIN, pattern_id=CL100K)
    for length in (2049, 2080, 5000, 40_000, 100_003):
        data = b"a" * length
        got = gpu(data).tolist()
        want = [256 + K_CHAIN - 1] * (length >> K_CHAIN)
        rem = length & ((1 << K_CHAIN) - 1)
        want += [97 if b == 0 else 256 + b - 1 for b in range(K_CHAIN - 1, -1, -1) if rem & (1 << b)]
        say("chain table, %d letters" % length)
        assert got == want


def test_fallback_and_stitched_pieces_in_one_tile():
    # pieces: [letters (stitched)] [spaces, 32 k + 1 of them (fallback)]
    # [' y'] ...; and the other way round; with text on both sides.  Tiles
    # hold the end of one long piece and the start of the next.
    v = load("c3", CL100K)
    rng = random.Random(5)
    for pre in (0, 1, 700, 1023, 1024, 1500):
        for first_fails in (False, True):
            word = random_word(3000 + rng.randint(0, 64), 900 + pre, "etaoinshrdlu")
            # a run of 32 k + 2 spaces before a letter: the run piece is 32 k + 1 spaces
            spaces = b" " * (32 * 70 + 2)
            head = (mix_text(pre, 910 + pre) + b"x") if pre else b""
            if first_fails:
                body = spaces + b"y" + word + b"." + random_word(2500, 7, "ab")
            else:
                body = word + spaces + b"y" + spaces + b"z"
            check(head + body + b"\n" + mix_text(300, 3), v, CL100K, "mixed long pieces, pre %d" % pre)


def test_batch_with_long_pieces_at_text_edges():
    v = load("c3", CL100K)
    texts = [random_word(5000, 1, "abc"), b" " * (32 * 80 + 1), b"", mix_text(3000, 9) + b" " * 2600,
             random_word(2049, 2), b"q" + b" " * (32 * 64 + 1) + b"r", random_word(70_000, 3, "etaoinshrdlu")]
    data = b"".join(texts)
    offs = np.cumsum([0] + [len(t) for t in texts]).astype(np.int64)
    say("batch with long pieces: %d texts, %d bytes" % (len(texts), len(data)))
    ids, out_off = tt.encode_batch(torch.frombuffer(bytearray(data), dtype=torch.uint8).cuda(),
                                   torch.tensor(offs, dtype=torch.int64, device="cuda"))
    want, want_off = oracle_batch(data, offs.tolist(), v, CL100K, {})
    assert out_off.tolist() == want_off
    assert np.array_equal(ids.cpu().numpy(), np.asarray(want, dtype=np.int32))


def test_byte_offsets_of_stitched_and_fallback_pieces():
    v = load("c3", CL100K)
    data = (mix_text(1000, 4) + b" " + random_word(12_345, 4, "etaoinshrdlu") + b" " * (32 * 90 + 1) + b"w"
            + random_word(3000, 5, "ab") + b"\n")
    say("offsets of long pieces: %d bytes" % len(data))
    ids, starts = tt.encode_offsets(torch.frombuffer(bytearray(data), dtype=torch.uint8).cuda())
    wi, ws, _ = oracle_offsets(data, None, v, CL100K, {})
    assert np.array_equal(ids.cpu().numpy(), np.asarray(wi, dtype=np.int32))
    assert np.array_equal(starts.cpu().numpy(), np.asarray(ws, dtype=np.int32))
