"""GPU path (libtt through the C ABI) against the CPU oracle, bit for bit.

Piece level (tt_pretokenize) and end to end (tt_encode, tt_encode_batch), the
two check levels of the correctness campaign on TokTier's summary page (§5.2),
on seeded synthetic text, brute-force batches of every short string over a
class-covering alphabet, long runs that cross tiles, and the edge cases
(empty input, empty sequences, invalid UTF-8, bad offsets, no merges).
"""
import itertools
import os
import random

import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import exact_byte_level_amd as tt  # noqa: E402
from oracle.bpe import Vocab, encode as oracle_encode, encode_batch as oracle_encode_batch  # noqa: E402
from oracle.pretok import CL100K, GPT2, piece_starts_batch, split_bytes  # noqa: E402
from synth import code_text, mix_text  # noqa: E402

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
_VOCABS = {}


def vocab(name):
    if name not in _VOCABS:
        _VOCABS[name] = np.load(os.path.join(ROOT, "data", "vocab_%s.npy" % name))
    return _VOCABS[name]


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


def load(name_or_merges, pattern):
    merges = vocab(name_or_merges) if isinstance(name_or_merges, str) else name_or_merges
    tt.load(merges, pattern_id=pattern)
    return Vocab(merges)


def gpu_starts(data, pattern, offsets=None):
    load("c1", pattern)
    off = None if offsets is None else torch.tensor(offsets, dtype=torch.int64, device="cuda")
    return tt.pretokenize(dev(data), off).cpu().numpy().tolist()


# ------------------------------------------------------------- piece level

@pytest.mark.parametrize("pattern", [GPT2, CL100K])
def test_pretokenize_code_text(pattern):
    data = code_text(65_536, 101)
    say("pretokenize code_text 64KiB seed 101 pattern", pattern)
    _, want = split_bytes(data, pattern)
    assert gpu_starts(data, pattern) == want


@pytest.mark.parametrize("pattern", [GPT2, CL100K])
def test_pretokenize_multibyte_mix(pattern):
    data = mix_text(300_000, 7, multibyte=True)
    say("pretokenize mix 300K chars multibyte seed 7 pattern", pattern)
    _, want = split_bytes(data, pattern)
    assert gpu_starts(data, pattern) == want


ALPHA = ["a", "s", "r", "e", "S", "1", ".", "'", " ", "\n", "\t", "\r"]


def _batch(strings):
    parts = [s.encode() for s in strings]
    offs = [0]
    for p in parts:
        offs.append(offs[-1] + len(p))
    return b"".join(parts), offs


@pytest.mark.parametrize("pattern", [GPT2, CL100K])
def test_pretokenize_every_short_string(pattern):
    strings = ["".join(t) for n in range(6) for t in itertools.product(ALPHA, repeat=n)]
    data, offs = _batch(strings)
    say("pretokenize brute force: %d strings, %d bytes, pattern %d" % (len(strings), len(data), pattern))
    assert gpu_starts(data, pattern, offs) == piece_starts_batch(data, offs, pattern)


ALPHA2 = ALPHA + list("lLvVmdDtTEé中😀") + ["　", "\xa0", "2", "²", "_", "(", "\x0b", "٣", "\x85", "ſ"]


@pytest.mark.parametrize("pattern", [GPT2, CL100K])
def test_pretokenize_random_multibyte_strings(pattern):
    rng = random.Random(21 + pattern)
    strings = ["".join(rng.choice(ALPHA2) for _ in range(rng.randint(0, 40))) for _ in range(40_000)]
    data, offs = _batch(strings)
    say("pretokenize random batch: %d strings, %d bytes, pattern %d" % (len(strings), len(data), pattern))
    assert gpu_starts(data, pattern, offs) == piece_starts_batch(data, offs, pattern)


LONG_RUNS = [
    "a" + "1" * 20_000 + "x" + "2" * 4_097,
    ".\n" + "\n" * 9_000 + " " * 9_000 + "z",
    ";" + "\n" * 5_000 + "\t" * 3 + "\n" + " " * 12_000 + "q",
    " " * 50_000 + "7",
    "x" + " " * 8_191 + "\n" + " " * 8_193,
    "٣" * 5_000 + "1" * 7,
    "b" * 70_000 + "'s" + "c" * 5,
    "é" * 9_000 + " " + "中" * 3_000,
]


@pytest.mark.parametrize("pattern", [GPT2, CL100K])
def test_pretokenize_runs_crossing_tiles(pattern):
    for text in LONG_RUNS:
        data = text.encode()
        say("pretokenize long runs: %d bytes, pattern %d" % (len(data), pattern))
        _, want = split_bytes(data, pattern)
        assert gpu_starts(data, pattern) == want
    data, offs = _batch(LONG_RUNS)
    assert gpu_starts(data, pattern, offs) == piece_starts_batch(data, offs, pattern)


def _tile_edge_text(seed, tile=1024, ntiles=48):
    # runs of 1..130 chars of each class placed across every tile boundary,
    # contractions split by a boundary, and every other tile holding one
    # 2-byte char (so that ASCII-only and mixed tiles alternate)
    rng = random.Random(seed)
    runs = [" ", "7", "x", ".", "\n", "\t", "'", "\r\n"]
    out = bytearray()
    for t in range(1, ntiles):
        edge = t * tile
        ch = rng.choice(runs)
        k = rng.choice([1, 2, 3, 60, 63, 64, 65, 66, 70, 100, 130])
        left = rng.randint(0, k)
        while len(out) < edge - left * len(ch.encode()):
            word = rng.choice(["ab", "don't", "we're", "x1", "Il", "9", "..", " ", "\n"])
            out += word.encode()
            if t % 2 and rng.random() < 0.02:
                out += "é".encode()
        out += (ch * k).encode()
        out += rng.choice([b"'s", b"'LL", b"q", b"1", b"!", b" "])
    return bytes(out)


@pytest.mark.parametrize("pattern", [GPT2, CL100K])
def test_runs_across_tile_edges(pattern):
    data = _tile_edge_text(60 + pattern)
    say("tile edges: %d bytes, pattern %d" % (len(data), pattern))
    _, want = split_bytes(data, pattern)
    assert gpu_starts(data, pattern) == want
    v = load("c1", pattern)
    got = gpu_encode(data)
    assert np.array_equal(got, np.asarray(oracle_encode(data, v, pattern, {}), dtype=np.int32))


# ------------------------------------------------------------- end to end

def gpu_encode(data):
    return tt.encode(dev(data)).cpu().numpy()


def check_encode(data, name, pattern, memo=None):
    v = load(name, pattern)
    say("encode %d bytes vocab %s pattern %d" % (len(data), name, pattern))
    got = gpu_encode(data)
    want = np.asarray(oracle_encode(data, v, pattern, memo), dtype=np.int32)
    if not np.array_equal(got, want):
        k = int(np.argmax(got[:min(len(got), len(want))] != want[:min(len(got), len(want))]))
        raise AssertionError("mismatch: %d vs %d tokens, first difference at %d" % (len(got), len(want), k))


def test_encode_code_text_gpt2():
    check_encode(code_text(65_536, 101), "c1", GPT2)


def test_encode_mix_gpt2_large_vocab():
    check_encode(mix_text(200_000, 31), "c2", GPT2, {})


def test_encode_multibyte_cl100k():
    check_encode(mix_text(200_000, 32, multibyte=True), "c1", CL100K, {})


def test_encode_full_mix_1m_gpt2():
    check_encode(mix_text(1_000_000, 102), "c2", GPT2, {})


def test_encode_batch_with_empty_sequences():
    rng = random.Random(9)
    texts = []
    for i in range(60):
        k = rng.choice([0, 0, 1, 5, 100, 3000, 20_000])
        texts.append(mix_text(k, 500 + i, multibyte=True) if k else b"")
    data = b"".join(texts)
    offs = np.cumsum([0] + [len(t) for t in texts]).astype(np.int64)
    for name, pattern in (("c1", CL100K), ("c2", GPT2)):
        v = load(name, pattern)
        say("encode_batch %d texts %d bytes pattern %d" % (len(texts), len(data), pattern))
        ids, out_off = tt.encode_batch(dev(data), torch.tensor(offs, device="cuda"))
        want, want_off = oracle_encode_batch(data, offs.tolist(), v, pattern, {})
        assert out_off.numpy().tolist() == want_off
        assert np.array_equal(ids.cpu().numpy(), np.asarray(want, dtype=np.int32))


def test_long_pieces_chain_closed_form():
    # a+a, aa+aa, ... up to a^(2^K): a run of L letters encodes to the binary
    # expansion of L (closed form), through the per-lane and the long-piece paths
    K = 12
    merges = [(97, 97)] + [(256 + i, 256 + i) for i in range(K - 1)]
    load(np.asarray(merges, dtype=np.int32), CL100K)
    for length in (1, 2, 3, 31, 32, 33, 64, 65, 100, 1000, 4095, 4096, 4097, 8191, 70_001, 300_000):
        say("chain vocab, 'a' x", length)
        got = gpu_encode(b"a" * length).tolist()
        want = [256 + K - 1] * (length >> K)
        rem = length & ((1 << K) - 1)
        for bit in range(K - 1, -1, -1):
            if rem & (1 << bit):
                want.append(97 if bit == 0 else 256 + bit - 1)
        assert got == want


def test_long_pieces_against_oracle():
    v = load("c2", GPT2)
    rng = random.Random(3)
    for length in (33, 40, 64, 65, 200, 1000, 5000):
        word = "".join(rng.choice("abcdefghijklmnopqrstuvwxyz") for _ in range(length)).encode()
        for text in (word, b" " + word, b"x" * length, b" " * length + b"y"):
            say("long piece", len(text))
            got = gpu_encode(text).tolist()
            assert got == oracle_encode(text, v, GPT2)


def test_pieces_over_two_kib_mixed_with_text():
    # pieces longer than 2 KiB are merged by a whole workgroup (exact rounds
    # with alternating merges inside runs of equal pairs); mix them with
    # ordinary text so that every path runs in one call
    rng = random.Random(44)
    for name, pattern in (("c2", GPT2), ("c3", CL100K)):
        v = load(name, pattern)
        parts = []
        for i in range(12):
            parts.append(mix_text(3000, 900 + i))
            kind = i % 4
            k = rng.randint(2049, 12000)
            if kind == 0:
                parts.append(b" " * k + b"x")
            elif kind == 1:
                parts.append(b"9" * k if pattern == GPT2 else b"z" * k)
            elif kind == 2:
                parts.append(b" " + "".join(rng.choice("ab") for _ in range(k)).encode())
            else:
                parts.append(b"\n" + b"\t " * (k // 2) + b"q")
        data = b"".join(parts)
        say("pieces over 2 KiB: %d bytes pattern %d" % (len(data), pattern))
        got = gpu_encode(data)
        want = np.asarray(oracle_encode(data, v, pattern, {}), dtype=np.int32)
        assert np.array_equal(got, want)


# A piece longer than 2 KiB is set up by every group of 9 tiles (9 KiB) it
# covers, each writing its share of the starting ids and pair ranks; the last
# group to finish merges the piece.  These cases put long pieces' starts and
# ends on and around tile and group edges, place long pieces next to each
# other (so that one tile holds the end of one and the start of the next),
# and run many merge rounds on one piece.
GROUP = 9 * 1024


def test_long_pieces_across_share_groups():
    v = load("c3", CL100K)
    cases = []
    for pre in (0, 1, 1023, 1024, 1025, GROUP - 1, GROUP, GROUP + 1, 2 * GROUP - 2500):
        for length in (2049, GROUP - 1, GROUP, GROUP + 1, 3 * GROUP + 5, 40_000):
            head = (b"x" * (pre - 1) + b" ") if pre else b""
            cases.append(head + b" " * length + b"y" + b"a" * (length // 3) + b"\n")
    rng = random.Random(46)
    parts = []
    for i in range(10):
        parts.append(rng.choice([b" ", b"a", b"-", b"7"]) * rng.randint(2049, 30_000))
        if i % 3:
            parts.append(code_text(rng.randint(1, 2000), 600 + i))
    cases.append(b"".join(parts))
    for k, data in enumerate(cases):
        say("long pieces across share groups: case %d, %d bytes" % (k, len(data)))
        got = gpu_encode(data)
        want = np.asarray(oracle_encode(data, v, CL100K, {}), dtype=np.int32)
        assert np.array_equal(got, want), k


def test_long_random_piece_many_rounds():
    # one 60,000-letter word: thousands of distinct merges, one round each
    v = load("c2", GPT2)
    rng = random.Random(47)
    word = "".join(rng.choice("etaoinshrdlu") for _ in range(60_000)).encode()
    for data in (word, b" " + word + b" " + word[:20_000]):
        say("long random piece, %d bytes" % len(data))
        assert gpu_encode(data).tolist() == oracle_encode(data, v, GPT2)


@pytest.mark.parametrize("letters", [100_000, 300_000])
def test_long_random_words_timed_sizes(letters):
    # the random-letter words whose encode times are reported (seed 5, the
    # 12-letter alphabet, 50K merges), bit-exact at full length, and one in a
    # cl100k-style text between other words
    v = load("c2", GPT2)
    rng = random.Random(5)
    word = "".join(rng.choice("etaoinshrdlu") for _ in range(letters)).encode()
    say("random word of %d letters" % letters)
    got = gpu_encode(word)
    want = np.asarray(oracle_encode(word, v, GPT2), dtype=np.int32)
    assert np.array_equal(got, want)
    v3 = load("c3", CL100K)
    data = b"begin " + word[: letters // 3] + b" end\n" + mix_text(20_000, 49)
    say("random word of %d letters in a cl100k-style text" % (letters // 3))
    assert np.array_equal(gpu_encode(data), np.asarray(oracle_encode(data, v3, CL100K, {}), dtype=np.int32))


def test_long_pieces_in_a_batch():
    v = load("c3", CL100K)
    texts = [b"a" * 2500, b"b" * 30_000, b"", b" " * 20_000 + b"x", code_text(3000, 48), b"c" * 2049,
             b"d" * GROUP, b" " * (2 * GROUP) + b"\n"]
    data = b"".join(texts)
    offs = np.cumsum([0] + [len(t) for t in texts]).astype(np.int64)
    say("batch of %d texts with long pieces, %d bytes" % (len(texts), len(data)))
    ids, out_off = tt.encode_batch(dev(data), torch.tensor(offs, device="cuda"))
    want, want_off = oracle_encode_batch(data, offs.tolist(), v, CL100K, {})
    assert out_off.numpy().tolist() == want_off
    assert np.array_equal(ids.cpu().numpy(), np.asarray(want, dtype=np.int32))


def test_pipe_line_vocab_on_gpu():
    merges = np.asarray([(112, 105), (256, 112), (257, 101), (108, 105), (259, 110), (260, 101), (258, 261)],
                        dtype=np.int32)
    load(merges, GPT2)
    assert gpu_encode(b"pipe").tolist() == [258]
    assert gpu_encode(b"line").tolist() == [261]
    assert gpu_encode(b"pipeline").tolist() == [262]
    assert gpu_encode(b"pipe line").tolist() == [258, 32, 261]


def test_zero_merges_gives_bytes():
    load(np.zeros((0, 2), dtype=np.int32), CL100K)
    data = mix_text(50_000, 3, multibyte=True)
    assert gpu_encode(data).tolist() == list(data)


def test_empty_and_tiny_inputs():
    load("c1", GPT2)
    assert gpu_encode(b"").tolist() == []
    assert gpu_encode(b"x").tolist() == [ord("x")]
    ids, off = tt.encode_batch(dev(b""), torch.zeros(4, dtype=torch.int64, device="cuda"))
    assert ids.numel() == 0 and off.tolist() == [0, 0, 0, 0]
    assert tt.pretokenize(dev(b"")).numel() == 0


BAD_UTF8 = [b"\xff", b"abc\x80", b"\xc3", b"ok \xed\xa0\x80", b"\xc0\xaf", b"\xf4\x90\x80\x80", b"\xe2\x82",
            b"a" * 5000 + b"\xe2\x28\xa1" + b"b" * 5000, b"\xf0\x9f\x98"]


def test_invalid_utf8_reports_error():
    load("c1", CL100K)
    for bad in BAD_UTF8:
        with pytest.raises(tt.TTError) as e:
            gpu_encode(bad)
        assert e.value.code == tt.TT_EUTF8
    # a char split across two batch sequences is invalid in both
    data = "é".encode()
    with pytest.raises(tt.TTError) as e:
        tt.encode_batch(dev(data), torch.tensor([0, 1, 2], dtype=torch.int64, device="cuda"))
    assert e.value.code == tt.TT_EUTF8
    # valid input right after still works
    assert gpu_encode(b"fine") .size > 0


def test_bad_offsets_report_error():
    load("c1", GPT2)
    for offs in ([0, 5, 3, 10], [1, 5, 10], [0, 5, 11], [0, 12, 10]):
        with pytest.raises(tt.TTError) as e:
            tt.encode_batch(dev(b"0123456789"), torch.tensor(offs, dtype=torch.int64, device="cuda"))
        assert e.value.code == tt.TT_EOFFSETS


def test_unaligned_input_pointer():
    # the tile loader takes 16-byte loads only from a 16-byte aligned text
    v = load("c2", GPT2)
    data = mix_text(100_000, 78)
    buf = dev(b"#" * 7 + data)
    x = buf[7:]  # data_ptr is 7 bytes past an aligned allocation
    assert x.data_ptr() % 16 != 0
    assert np.array_equal(tt.encode(x).cpu().numpy(), np.asarray(oracle_encode(data, v, GPT2, {}), dtype=np.int32))
    _, want = split_bytes(data, GPT2)
    assert tt.pretokenize(x).cpu().numpy().tolist() == want


def test_repeat_runs_are_identical():
    load("c2", GPT2)
    data = dev(mix_text(500_000, 77))
    a = tt.encode(data).cpu().numpy()
    b = tt.encode(data).cpu().numpy()
    assert np.array_equal(a, b)
