"""Inputs at the library's size limit (TT_MAX_BYTES - 1 bytes, 1 GiB) on the GPU,
and a 64 MiB single pre-token.

The text is K copies of a 1 MB mix whose end and start meet at a pre-token
boundary (checked with the oracle: the encode of two copies is the encode of
one, twice).  Every pre-token is encoded on its own (TokTier summary page,
Appendix A.1), so the expected ids of the whole text are the oracle's ids of
one copy, K times.  The test compares all ~250M ids of the GPU output with
them, and checks that TT_MAX_BYTES bytes are refused before any work.
"""
import os

import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import exact_byte_level_amd as tt  # noqa: E402
from oracle.bpe import Vocab, encode as oracle_encode  # noqa: E402
from oracle.pretok import CL100K, GPT2  # noqa: E402
from synth import mix_text  # noqa: E402

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIMIT = 1 << 30  # TT_MAX_BYTES


def say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)
    yield
    torch.cuda.synchronize()


def test_largest_input_bit_exact():
    merges = np.load(os.path.join(ROOT, "data", "vocab_c2.npy"))
    v = Vocab(merges)
    copy = b"start " + mix_text(1_000_000, 61) + b" end."
    one = oracle_encode(copy, v, GPT2, {})
    assert oracle_encode(copy + copy, v, GPT2, {}) == one + one  # the copies meet at a piece boundary
    k = (LIMIT - 1) // len(copy)
    data = copy * k
    say("largest input: %d copies of %d bytes = %d bytes (limit %d)" % (k, len(copy), len(data), LIMIT))
    tt.load(merges, pattern_id=GPT2)
    x = torch.frombuffer(bytearray(data), dtype=torch.uint8).cuda()
    del data
    ids = tt.encode(x)
    torch.cuda.synchronize()
    say("  %d tokens" % ids.numel())
    assert ids.numel() == k * len(one)
    got = ids.view(k, len(one))
    want = torch.tensor(one, dtype=torch.int32, device="cuda")
    assert bool((got == want).all())
    del ids, got, x
    torch.cuda.empty_cache()


def test_giant_piece_in_a_large_input():
    # one pre-token of 64 MiB + a ragged tail of letters: its first round is
    # shared over thousands of tile groups, the searches for its ends cross
    # dozens of runs of 2,048 tiles, and its merges run on one workgroup.
    # Closed forms: with a+a, aa+aa, ... up to a^(2^K) the ids are the binary
    # expansion of the length; with a trained table that has no aa merge, the
    # bytes themselves.
    length = (64 << 20) + 12_345
    x = torch.full((length,), 97, dtype=torch.uint8, device="cuda")
    K = 12
    merges = np.asarray([(97, 97)] + [(256 + i, 256 + i) for i in range(K - 1)], dtype=np.int32)
    tt.load(merges, pattern_id=CL100K)
    say("giant piece: %d letters, doubling-chain table" % length)
    ids = tt.encode(x)
    torch.cuda.synchronize()
    rem = length & ((1 << K) - 1)
    tail = [97 if bit == 0 else 256 + bit - 1 for bit in range(K - 1, -1, -1) if rem & (1 << bit)]
    head = length >> K
    assert ids.numel() == head + len(tail)
    assert bool((ids[:head] == 256 + K - 1).all())
    assert ids[head:].cpu().tolist() == tail
    tt.load(np.load(os.path.join(ROOT, "data", "vocab_c3.npy")), pattern_id=CL100K)
    say("giant piece: %d letters, trained table without aa" % length)
    ids = tt.encode(x)
    torch.cuda.synchronize()
    assert ids.numel() == length and bool((ids == 97).all())
    del ids, x
    torch.cuda.empty_cache()


def test_limit_is_refused():
    tt.load(np.load(os.path.join(ROOT, "data", "vocab_c1.npy")), pattern_id=GPT2)
    x = torch.zeros(1, dtype=torch.uint8, device="cuda")
    out = torch.empty(1, dtype=torch.int32, device="cuda")
    out_n = torch.empty(1, dtype=torch.int64, device="cuda")
    # the size is checked before any pointer is used
    rc = tt.lib().tt_encode(x.data_ptr(), LIMIT, out.data_ptr(), out_n.data_ptr(),
                            __import__("ctypes").c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == tt.TT_ETOOBIG
