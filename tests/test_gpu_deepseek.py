"""DeepSeek-style rules on the GPU (tt_pretokenize and tt_encode through the
C ABI) against the CPU oracle, bit for bit.

Brute force over every string of length <= 5 of a class-covering alphabet
(ASCII and other letters, a mark, digits, CJK and kana chars with the kana
middle dot, ASCII and other punctuation/symbols, whitespace, a control char),
random multibyte strings, runs that cross tiles (digit groups, whitespace
before CR/LF, CR/LF after punctuation, CJK runs, ASCII-letter runs after
punctuation), tile edges and a 1M-char encode.
"""
import itertools
import os
import random

import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import exact_byte_level_amd as tt  # noqa: E402
from oracle.bpe import Vocab, encode as oracle_encode  # noqa: E402
from oracle.pretok import DEEPSEEK, piece_starts_batch, split_bytes  # noqa: E402
from synth import mix_text  # noqa: E402

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


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
    tt.load(merges, pattern_id=DEEPSEEK)
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
    data, offs = batch(strings)
    got, want = gpu_starts(data, offs), piece_starts_batch(data, offs, DEEPSEEK)
    if got == want:
        return
    k = next((i for i, (a, b) in enumerate(zip(got, want)) if a != b), min(len(got), len(want)))
    pos = min(got[k] if k < len(got) else len(data), want[k] if k < len(want) else len(data))
    s = int(np.searchsorted(np.asarray(offs), pos, side="right")) - 1
    raise AssertionError("first difference in string %d %r: gpu %s oracle %s" % (
        s, strings[s], [x - offs[s] for x in got if offs[s] <= x < offs[s + 1]],
        [x - offs[s] for x in want if offs[s] <= x < offs[s + 1]]))


ALPHA = ["a", "é", "́", "1", "中", "あ", "・", ".", "_", "€", " ", "\t", "\n", "\x00"]


def test_every_short_string():
    load()
    strings = ["".join(t) for n in range(6) for t in itertools.product(ALPHA, repeat=n)]
    say("deepseek brute force: %d strings" % len(strings))
    check_batch(strings)


ALPHA2 = ALPHA + list("sSzZ09$'(") + ["文", "゛", "ー", "ア", "゠", "²", "٣", "\r", "\xa0", "​", "",
                                    "\U0001f600", "ǅ"]


def test_random_multibyte_strings():
    load()
    rng = random.Random(93)
    strings = ["".join(rng.choice(ALPHA2) for _ in range(rng.randint(0, 40))) for _ in range(40_000)]
    say("deepseek random batch: %d strings" % len(strings))
    check_batch(strings)


LONG_RUNS = [
    "a" + "1" * 20_000 + "x" + "2" * 4_097,
    ".\n" + "\n" * 9_000 + " " * 9_000 + "z",
    "x" + " " * 8_191 + "\n" + " " * 8_193,
    "x" + "中" * 3_000 + "a" + "あ・い" * 700 + "b",
    "_" + "a" * 5_000 + ".b" + "c" * 2_000,
    "\t" * 3_000 + "." + "\x00" * 2_000 + "a",
    " " * 4_000 + "1",
]


def test_runs_crossing_tiles():
    load()
    for text in LONG_RUNS:
        data = text.encode()
        say("deepseek long runs: %d bytes" % len(data))
        _, want = split_bytes(data, DEEPSEEK)
        assert gpu_starts(data) == want
    check_batch(LONG_RUNS)


def _tile_edge_text(seed, tile=1024, ntiles=48):
    rng = random.Random(seed)
    runs = [" ", "7", "x", "X", ".", "\n", "\t", "'", "\r\n", "_", "中", "é", "\x00", "・"]
    out = bytearray()
    for t in range(1, ntiles):
        edge = t * tile
        ch = rng.choice(runs)
        k = rng.choice([1, 2, 3, 15, 16, 17, 31, 32, 33, 60, 64, 70, 130])
        left = rng.randint(0, k)
        while len(out) < edge - left * len(ch.encode()):
            word = rng.choice(["ab", "don't", "we're", "x1", "_init", "HTMLParser", "9", "..", " ", "\n", "a/b",
                               "Été", "中文", "$x", "€5"])
            out += word.encode()
        out += (ch * k).encode()
        out += rng.choice([b"'s", b"q", b"Q", b"1", b"!", b" ", b"/", b"\n"])
    return bytes(out)


def test_runs_across_tile_edges():
    data = _tile_edge_text(79)
    v = load("c1")
    say("deepseek tile edges: %d bytes" % len(data))
    _, want = split_bytes(data, DEEPSEEK)
    assert gpu_starts(data) == want
    got = tt.encode(dev(data)).cpu().numpy()
    assert np.array_equal(got, np.asarray(oracle_encode(data, v, DEEPSEEK, {}), dtype=np.int32))


def test_encode_mix_1m():
    v = load("c3")
    data = mix_text(1_000_000, 203, multibyte=True)
    say("deepseek encode: %d bytes" % len(data))
    got = tt.encode(dev(data)).cpu().numpy()
    assert np.array_equal(got, np.asarray(oracle_encode(data, v, DEEPSEEK, {}), dtype=np.int32))


def test_letter_run_after_punctuation_across_a_tile_start():
    # an ASCII-letter run after '_' / '.' that covers a whole tile's left
    # context, then a non-ASCII letter: the punctuation char's piece is
    # decided from the summary pass, before or after a space
    v = load()
    for pre in ("x" * 1000 + ".", "x" * 1000 + " .", "x" * 999 + "._", "\u4e2d" * 300 + "_"):
        for k in (20, 100, 1500):
            text = pre + "a" * k + "\u00e9b"
            got = tt.encode(dev(text.encode())).cpu().numpy()
            want = np.asarray(oracle_encode(text.encode(), v, DEEPSEEK, {}), dtype=np.int32)
            assert np.array_equal(got, want), (pre[-3:], k)
