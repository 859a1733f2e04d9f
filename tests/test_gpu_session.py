"""Sessions (incremental repair, tt_session_*) against the oracle's full encode.

TokTier summary page, §3.3: after every append the session's ids and token
byte starts must equal a fresh encode of the whole text (oracle.bpe
encode_offsets), whichever way the library took: a splice at the first window,
after window doublings, or a full encode.  Cases: streams of appends of the
pages' sizes (a few chars to a few thousand) on code-like and multi-byte text,
tiny windows that put the splice next to the window edges, tails that defeat
every window (long digit, space, newline and letter runs), invalid or split
UTF-8 in an append (rejected, session unchanged), empty appends, a 1M-char
context, capacity and tokenizer-reload errors.
"""
import os
import random

import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import exact_byte_level_amd as tt  # noqa: E402
from oracle.bpe import Vocab, encode_offsets as oracle_offsets  # noqa: E402
from oracle.pretok import CL100K, GPT2  # noqa: E402
from synth import code_text, mix_text  # noqa: E402

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
    return torch.frombuffer(bytearray(data), dtype=torch.uint8).cuda() if len(data) else torch.empty(
        0, dtype=torch.uint8, device="cuda")


def load(name, pattern):
    merges = np.load(os.path.join(ROOT, "data", "vocab_%s.npy" % name))
    tt.load(merges, pattern_id=pattern)
    return Vocab(merges)


def check(s, text, v, pattern, memo):
    assert bytes(s.text().cpu().numpy().tobytes()) == text
    ids, starts, _ = oracle_offsets(text, None, v, pattern, memo)
    assert np.array_equal(s.ids().cpu().numpy(), np.asarray(ids, dtype=np.int32))
    assert np.array_equal(s.starts().cpu().numpy(), np.asarray(starts, dtype=np.int32))
    assert s.sizes() == (len(text), len(ids))


def _whole_chars(src, pos, k):
    end = min(len(src), pos + k)
    while end < len(src) and (src[end] & 0xC0) == 0x80:
        end += 1
    return src[pos:end]


@pytest.mark.parametrize("pattern,vocab_name", [(GPT2, "c1"), (CL100K, "c3")])
@pytest.mark.parametrize("tail", [64, 256, 0])
def test_append_stream(pattern, vocab_name, tail):
    v = load(vocab_name, pattern)
    memo = {}
    rng = random.Random(77 + pattern + tail)
    s = tt.Session(300_000, tail)
    text = mix_text(4_000, 70 + pattern, multibyte=True)
    say("session stream pattern", pattern, "tail", tail)
    s.reset(dev(text))
    check(s, text, v, pattern, memo)
    src = code_text(60_000, 71 + pattern) + mix_text(30_000, 72, multibyte=True)
    pos, ways = 0, {}
    for _ in range(60):
        d = _whole_chars(src, pos, rng.choice([1, 2, 3, 9, 40, 300, 1400, 3800]))
        pos += len(d)
        info = s.append(dev(d))
        text += d
        ways[info["doublings"]] = ways.get(info["doublings"], 0) + 1
        assert info["tokens"] == s.sizes()[1]
        check(s, text, v, pattern, memo)
    say("  ways", ways)
    assert ways.get(0, 0) > 30
    s.close()


@pytest.mark.parametrize("pattern,vocab_name", [(GPT2, "c1"), (CL100K, "c3")])
def test_tails_that_defeat_windows(pattern, vocab_name):
    v = load(vocab_name, pattern)
    memo = {}
    s = tt.Session(200_000, 64)
    text = code_text(5_000, 80)
    s.reset(dev(text))
    say("session long tails pattern", pattern)
    seen = set()
    for filler in (b"7" * 9000, b" " * 9000, b"\n" * 700 + b"x", b"q" * 9000, b"\xe4\xb8\xad" * 3000, b" \t" * 2000):
        for d in (filler, b"12 ab", b" cd"):
            info = s.append(dev(d))
            text += d
            seen.add(info["doublings"])
            check(s, text, v, pattern, memo)
    assert -1 in seen and 0 in seen


def test_invalid_appends_leave_the_session_unchanged():
    v = load("c3", CL100K)
    memo = {}
    s = tt.Session(100_000)
    text = code_text(10_000, 81)
    s.reset(dev(text))
    say("session invalid appends")
    for bad in (b"ok \xff", b"\xe4\xb8", b"\x80abc", b"a\xed\xa0\x80"):
        with pytest.raises(tt.TTError) as e:
            s.append(dev(bad))
        assert e.value.code == tt.TT_EUTF8
        check(s, text, v, CL100K, memo)
    info = s.append(dev(b""))
    assert info["doublings"] == 0 and info["tokens"] == s.sizes()[1]
    s.append(dev(" fine 中".encode()))
    text += " fine 中".encode()
    check(s, text, v, CL100K, memo)


def test_capacity_reset_and_reload():
    v = load("c1", GPT2)
    memo = {}
    s = tt.Session(1_000, 128)
    say("session capacity / reset / reload")
    s.reset(dev(b""))
    check(s, b"", v, GPT2, memo)
    s.append(dev(b"hello world"))
    check(s, b"hello world", v, GPT2, memo)
    with pytest.raises(tt.TTError) as e:
        s.append(dev(b"x" * 990))
    assert e.value.code == tt.TT_ETOOBIG
    check(s, b"hello world", v, GPT2, memo)
    with pytest.raises(tt.TTError) as e:
        s.reset(dev(b"y" * 1001))
    assert e.value.code == tt.TT_ETOOBIG
    s.reset(dev(b"abc def"))
    load("c1", GPT2)  # a reload makes the session stale
    with pytest.raises(tt.TTError) as e:
        s.append(dev(b" ghi"))
    assert e.value.code == tt.TT_ESTALE
    s.reset(dev(b"abc def"))
    s.append(dev(b" ghi"))
    check(s, b"abc def ghi", v, GPT2, memo)


@pytest.mark.parametrize("pattern,vocab_name", [(GPT2, "c1"), (CL100K, "c3")])
def test_large_appends(pattern, vocab_name):
    """Appends whose window is over 64 KiB (spliced by the grid-wide copy) and
    small ones after them (spliced by the search's own workgroup)."""
    v = load(vocab_name, pattern)
    memo = {}
    s = tt.Session(400_000, 256)
    text = mix_text(6_000, 90 + pattern, multibyte=True)
    s.reset(dev(text))
    say("session large appends pattern", pattern)
    src = mix_text(200_000, 91 + pattern, multibyte=True)
    pos = 0
    for k in (80_000, 300, 70_000, 1400):
        d = _whole_chars(src, pos, k)
        pos += len(d)
        info = s.append(dev(d))
        text += d
        assert info["tokens"] == s.sizes()[1]
        check(s, text, v, pattern, memo)
    s.close()


def test_million_char_context():
    v = load("c2", GPT2)
    from synth.text import workload
    data, _, pat, voc = workload("c2")
    assert pat == GPT2 and voc == "c2"
    memo = {}
    s = tt.Session(len(data) + 100_000)
    s.reset(dev(data))
    text = data
    say("session 1M-char context, 4 appends")
    rng = random.Random(83)
    src = mix_text(40_000, 84)
    pos = 0
    for k in (1400, 3800, 50, 12_000):
        d = _whole_chars(src, pos, k)
        pos += len(d)
        info = s.append(dev(d))
        text += d
        assert info["doublings"] == 0 and info["window_bytes"] < 2048 + len(d) + 4
        check(s, text, v, GPT2, memo)
