"""Encodes captured into a HIP graph after tt_reserve, replayed on new inputs.

The C ABI promises that an encode allocates nothing once the workspace is
reserved and enqueues only on the caller's stream, so it can be captured.  A
graph fixes the sizes it was captured with (n, the number of texts) but not
the device data: each replay here gets new text (and, for a batch, new text
boundaries) copied into the captured buffers, with eager encodes of other
sizes and host synchronisations between the replays, and every replay is
compared with the oracle element by element.  The texts hold pieces longer
than 2 KiB, so the per-call counters of the long-piece hand-over are reset
inside the graph as well.
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
from synth import mix_text  # noqa: E402

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
N = 48_000


@pytest.fixture(scope="module", autouse=True)
def _device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)
    yield
    torch.cuda.synchronize()


def say(*a):
    print(*a, flush=True)


def setup(name, pattern):
    merges = np.load(os.path.join(ROOT, "data", "vocab_%s.npy" % name))
    tt.load(merges, pattern_id=pattern)
    tt.reserve(4 * N, 16)
    return Vocab(merges)


def text_of(seed, n=N):
    """n ASCII bytes: the code/log mix with a 3,000-space run and a
    3,000-letter random word (pieces past 2 KiB) at seeded places."""
    rng = random.Random(seed)
    base = mix_text(n, seed)
    word = "".join(rng.choice("etaoinshrdlu") for _ in range(3000)).encode()
    a = rng.randrange(1000, n // 2 - 7000)
    b = rng.randrange(n // 2, n - 4000)
    t = base[:a] + b" " * 3000 + b"x" + base[a + 3001:b] + b" " + word + base[b + 3001:]
    assert len(t) == n
    return t


def capture(fn):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()  # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def eager_noise(k):
    """Eager work between replays: an encode of another size, torch ops, a sync."""
    y = torch.frombuffer(bytearray(mix_text(5_000 + 977 * k, 900 + k)), dtype=torch.uint8).cuda()
    tt.encode(y)
    (torch.arange(100_000, device="cuda") * 3).sum().item()


@pytest.mark.parametrize("pattern", [GPT2, CL100K])
def test_graph_replays_of_encode(pattern):
    v = setup("c1" if pattern == GPT2 else "c3", pattern)
    say("graph: tt_encode of %d bytes, pattern %d, 4 replays" % (N, pattern))
    x = torch.empty(N, dtype=torch.uint8, device="cuda")
    out = torch.empty(N, dtype=torch.int32, device="cuda")
    out_n = torch.empty(1, dtype=torch.int64, device="cuda")
    x.copy_(torch.frombuffer(bytearray(text_of(1)), dtype=torch.uint8))
    g = capture(lambda: tt.encode_into(x, out, out_n))
    memo = {}
    for k in range(4):
        t = text_of(10 + k)
        x.copy_(torch.frombuffer(bytearray(t), dtype=torch.uint8))
        out.fill_(-7)
        g.replay()
        torch.cuda.synchronize()
        T = int(out_n.item())
        want = oracle_encode(t, v, pattern, memo)
        assert T == len(want), (k, T, len(want))
        assert np.array_equal(out[:T].cpu().numpy(), np.asarray(want, dtype=np.int32)), k
        eager_noise(k)


def test_graph_replays_of_batch_with_new_boundaries():
    v = setup("c3", CL100K)
    B = 6
    say("graph: tt_encode_batch of %d bytes in %d texts, boundaries changed per replay" % (N, B))
    x = torch.empty(N, dtype=torch.uint8, device="cuda")
    off = torch.empty(B + 1, dtype=torch.int64, device="cuda")
    out = torch.empty(N, dtype=torch.int32, device="cuda")
    out_off = torch.empty(B + 1, dtype=torch.int64, device="cuda")

    def bounds(seed):
        rng = random.Random(seed)
        cuts = sorted(rng.sample(range(1, N), B - 2))
        return [0, 0] + cuts + [N]  # the first text is empty

    x.copy_(torch.frombuffer(bytearray(text_of(2)), dtype=torch.uint8))
    off.copy_(torch.tensor(bounds(2), dtype=torch.int64))
    g = capture(lambda: tt.encode_batch_into(x, off, out, out_off))
    memo = {}
    for k in range(3):
        t, o = text_of(20 + k), bounds(20 + k)
        x.copy_(torch.frombuffer(bytearray(t), dtype=torch.uint8))
        off.copy_(torch.tensor(o, dtype=torch.int64))
        g.replay()
        torch.cuda.synchronize()
        wi, wo = oracle_batch(t, o, v, CL100K, memo)
        assert out_off.cpu().tolist() == wo, k
        assert np.array_equal(out[:wo[-1]].cpu().numpy(), np.asarray(wi, dtype=np.int32)), k
        eager_noise(k)


def test_graph_replays_of_offsets():
    v = setup("c1", GPT2)
    say("graph: tt_encode_offsets of %d bytes, 3 replays" % N)
    x = torch.empty(N, dtype=torch.uint8, device="cuda")
    out = torch.empty(N, dtype=torch.int32, device="cuda")
    starts = torch.empty(N + 1, dtype=torch.int32, device="cuda")
    cnt = torch.empty(1, dtype=torch.int64, device="cuda")
    x.copy_(torch.frombuffer(bytearray(text_of(3)), dtype=torch.uint8))
    g = capture(lambda: tt.encode_offsets_into(x, None, out, starts, cnt))
    memo = {}
    for k in range(3):
        t = text_of(30 + k)
        x.copy_(torch.frombuffer(bytearray(t), dtype=torch.uint8))
        g.replay()
        torch.cuda.synchronize()
        wi, ws, _ = oracle_offsets(t, None, v, GPT2, memo)
        T = int(cnt.item())
        assert T == len(wi), k
        assert np.array_equal(out[:T].cpu().numpy(), np.asarray(wi, dtype=np.int32)), k
        assert np.array_equal(starts[:T + 1].cpu().numpy(), np.asarray(ws, dtype=np.int32)), k
        eager_noise(k)


def test_reserved_workspace_is_never_reallocated():
    """After tt_reserve the workspace stays where a captured graph points: a
    larger encode or session is refused (TT_ETOOBIG) rather than served by a
    new allocation, and the graph still replays correctly afterwards.  The
    reservation ends at the next tt_reserve or tt_load_bpe."""
    v = setup("c1", GPT2)
    say("reserve: graph captured under a %d-byte reservation, larger calls refused" % (4 * N))
    x = torch.empty(N, dtype=torch.uint8, device="cuda")
    out = torch.empty(N, dtype=torch.int32, device="cuda")
    out_n = torch.empty(1, dtype=torch.int64, device="cuda")
    x.copy_(torch.frombuffer(bytearray(text_of(4)), dtype=torch.uint8))
    g = capture(lambda: tt.encode_into(x, out, out_n))
    big_text = mix_text(6 * N, 77)
    big = torch.frombuffer(bytearray(big_text), dtype=torch.uint8).cuda()
    with pytest.raises(tt.TTError) as ei:
        tt.encode(big)
    assert ei.value.code == tt.TT_ETOOBIG
    with pytest.raises(tt.TTError) as ei:
        tt.Session(6 * N)
    assert ei.value.code == tt.TT_ETOOBIG
    t = text_of(40)
    x.copy_(torch.frombuffer(bytearray(t), dtype=torch.uint8))
    g.replay()
    torch.cuda.synchronize()
    want = oracle_encode(t, v, GPT2)
    T = int(out_n.item())
    assert T == len(want)
    assert np.array_equal(out[:T].cpu().numpy(), np.asarray(want, dtype=np.int32))
    # a new reservation may resize; a new load ends the reservation
    tt.reserve(8 * N, 1)
    want_big = np.asarray(oracle_encode(big_text, v, GPT2), dtype=np.int32)
    assert np.array_equal(tt.encode(big).cpu().numpy(), want_big)
    v = setup("c1", GPT2)  # reserves 4 * N again
    with pytest.raises(tt.TTError):
        tt.encode(big)
    tt.load(np.load(os.path.join(ROOT, "data", "vocab_c1.npy")), pattern_id=GPT2)
    assert np.array_equal(tt.encode(big).cpu().numpy(), want_big)
