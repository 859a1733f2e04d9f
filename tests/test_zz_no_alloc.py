"""tt_encode_noalloc (the entry point that allocates nothing) against tt_encode.

The no-alloc variant runs the same kernels on a fixed per-device scratch array
instead of the library's workspace.  Two calls in a row on each rule set, the
second with a smaller input (so it reuses the array with the first call's
contents still in it), must give exactly tt_encode's ids; the smaller one is
also checked against the oracle.  The texts hold pieces longer than 2 KiB, so
the long-piece stitching slots kept in the array are exercised too.
"""
import os
import random

import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import exact_byte_level_amd as tt  # noqa: E402
from oracle.bpe import Vocab, encode as oracle_encode  # noqa: E402
from oracle.pretok import CL100K, GPT2  # noqa: E402
from synth import mix_text  # noqa: E402

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def say(*a):
    print(*a, flush=True)


def text_of(n_chars, seed, multibyte):
    """The code/log mix with a 3,000-space run and a 3,000-letter random word."""
    rng = random.Random(seed)
    base = mix_text(n_chars, seed, multibyte=multibyte).decode()
    word = "".join(rng.choice("etaoinshrdlu") for _ in range(3000))
    cut = len(base) // 3  # in chars, so no multibyte char is split
    return (base[:cut] + " " * 3000 + "x" + base[cut:2 * cut] + " " + word + base[2 * cut:]).encode()


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)
    yield
    torch.cuda.synchronize()


@pytest.mark.parametrize("pattern,voc", [(GPT2, "c2"), (CL100K, "c3")])
def test_noalloc_equals_encode_on_two_calls(pattern, voc):
    merges = np.load(os.path.join(ROOT, "data", "vocab_%s.npy" % voc))
    tt.load(merges, pattern_id=pattern)
    v = Vocab(merges)
    big = text_of(1_700_000, 61 + pattern, pattern == CL100K)
    small = text_of(90_001, 62 + pattern, pattern == CL100K)
    assert len(big) <= tt.NOALLOC_MAX_BYTES and len(small) < len(big)
    for k, t in enumerate((big, small)):
        say("noalloc: pattern %d, call %d, %d bytes" % (pattern, k, len(t)))
        x = torch.frombuffer(bytearray(t), dtype=torch.uint8).cuda()
        want = tt.encode(x).cpu().numpy()
        out = torch.full((len(t),), -7, dtype=torch.int32, device="cuda")
        out_n = torch.full((1,), -99, dtype=torch.int64, device="cuda")
        tt.encode_noalloc_into(x, out, out_n)
        torch.cuda.synchronize()
        T = int(out_n.item())
        assert T == len(want), (k, T, len(want))
        assert np.array_equal(out[:T].cpu().numpy(), want), k
        if t is small:
            assert np.array_equal(want, np.asarray(oracle_encode(t, v, pattern), dtype=np.int32))


def test_noalloc_at_the_size_limit():
    # an input of exactly the maximum size fits the scratch array
    merges = np.load(os.path.join(ROOT, "data", "vocab_c2.npy"))
    tt.load(merges, pattern_id=GPT2)
    t = text_of(2_200_000, 64, False)[: tt.NOALLOC_MAX_BYTES]
    assert len(t) == tt.NOALLOC_MAX_BYTES
    say("noalloc: %d bytes (the limit)" % len(t))
    x = torch.frombuffer(bytearray(t), dtype=torch.uint8).cuda()
    want = tt.encode(x).cpu().numpy()
    out = torch.full((len(t),), -7, dtype=torch.int32, device="cuda")
    out_n = torch.full((1,), -99, dtype=torch.int64, device="cuda")
    tt.encode_noalloc_into(x, out, out_n)
    torch.cuda.synchronize()
    T = int(out_n.item())
    assert T == len(want)
    assert np.array_equal(out[:T].cpu().numpy(), want)


def test_noalloc_limits_and_empty_input():
    merges = np.load(os.path.join(ROOT, "data", "vocab_c1.npy"))
    tt.load(merges, pattern_id=GPT2)
    out_n = torch.full((1,), -99, dtype=torch.int64, device="cuda")
    empty = torch.empty(0, dtype=torch.uint8, device="cuda")
    tt.encode_noalloc_into(empty, torch.empty(1, dtype=torch.int32, device="cuda"), out_n)
    torch.cuda.synchronize()
    assert int(out_n.item()) == 0
    # one byte over the limit is refused on the host, before any device work
    over = torch.zeros(tt.NOALLOC_MAX_BYTES + 1, dtype=torch.uint8, device="cuda")
    with pytest.raises(tt.TTError) as ei:
        tt.encode_noalloc_into(over, torch.empty(over.numel(), dtype=torch.int32, device="cuda"), out_n)
    assert ei.value.code == tt.TT_ETOOBIG
    # invalid UTF-8 is reported in the count, as by tt_encode
    bad = torch.tensor([97, 0xFF, 98], dtype=torch.uint8, device="cuda")
    tt.encode_noalloc_into(bad, torch.empty(3, dtype=torch.int32, device="cuda"), out_n)
    torch.cuda.synchronize()
    assert int(out_n.item()) == tt.TT_EUTF8
