"""Shadow verification: sampled background re-checks of encodes.

TokTier summary page, §3 (the shadow branch of the serving architecture) and
§4.3 (runtime): a random fraction of calls (5 % online, every call offline) is
re-encoded in a background thread by a standard tokenizer; a call whose ids
differ is quarantined, that is, kept with its input for offline reproduction.
§5.8 measures it with injected token errors (substitutions, deletions,
shifted splits).

The standard tokenizer is the caller's: any callable that maps the bytes of
one text to its ids.  This module never tokenizes anything itself, and a check
changes no output: the ids returned are always the GPU's.

The hot-path cost of a sampled call is two device-to-device copies on the
caller's stream (the input bytes and the ids, so that the caller may reuse its
buffers at once) and an event; an unsampled call costs one draw from a seeded
generator.  The background thread waits on the event, copies the snapshot to
the host and runs the standard tokenizer there.  When more than ``max_pending``
checks wait, a sampled call is dropped (counted) rather than blocking.

    sv = ShadowVerifier(reference=my_cpu_tokenizer, rate=0.05)
    ids = sv.encode(u8_cuda_tensor)          # the GPU's ids, as tt.encode
    ...
    sv.drain(); print(sv.stats(), sv.quarantine)
"""
import json
import os
import queue
import random
import threading
from dataclasses import dataclass, field

import numpy as np


@dataclass
class Sample:
    """One quarantined text: its bytes, the ids under test, the standard
    tokenizer's ids and the first index where they differ."""
    call: int          # index of the call among all calls seen by the verifier
    text_index: int    # index of the text inside a batch (0 for a single text)
    data: bytes
    ids: list
    ref_ids: list
    first_diff: int
    error: str = ""    # set when the standard tokenizer raised instead
    extra: dict = field(default_factory=dict)


def first_difference(a, b):
    """Smallest index where two id sequences differ (len of the shorter one
    when one is a prefix of the other), or -1 when they are equal."""
    a = np.asarray(a, dtype=np.int64)
    b = np.asarray(b, dtype=np.int64)
    k = min(len(a), len(b))
    d = np.flatnonzero(a[:k] != b[:k])
    if len(d):
        return int(d[0])
    return -1 if len(a) == len(b) else k


class ShadowVerifier:
    """Re-checks a seeded random fraction ``rate`` of encodes against
    ``reference`` (bytes -> sequence of ids) in a background thread.

    ``encoder`` and ``batch_encoder`` default to the library's ``encode`` and
    ``encode_batch``; they may be any functions with the same contract (a test
    substitutes faulty ones).  ``quarantine_dir``, when given, receives each
    quarantined sample as ``sample_<k>.bin`` (the text) and ``sample_<k>.json``
    (ids, standard ids, first difference).  At most ``max_quarantine`` samples
    are kept; later mismatches are still counted.
    """

    def __init__(self, reference, rate=0.05, seed=0, encoder=None, batch_encoder=None,
                 max_pending=64, quarantine_dir=None, max_quarantine=1000, on_mismatch=None):
        if not callable(reference):
            raise TypeError("reference must be callable: bytes -> ids")
        if not 0.0 <= rate <= 1.0:
            raise ValueError("rate must lie in [0, 1]")
        self.reference = reference
        self.rate = float(rate)
        self._rng = random.Random(seed)
        self._encoder = encoder
        self._batch_encoder = batch_encoder
        self.quarantine_dir = quarantine_dir
        self.max_quarantine = int(max_quarantine)
        self.on_mismatch = on_mismatch
        self.quarantine = []
        self._lock = threading.Lock()
        self._calls = 0
        self._sampled = 0
        self._dropped = 0
        self._checked = 0
        self._texts = 0
        self._mismatches = 0
        self._errors = 0
        self.last_error = ""
        self._q = queue.Queue(maxsize=max(1, int(max_pending)))
        self._closed = False
        self._worker = threading.Thread(target=self._run, name="tt-shadow", daemon=True)
        self._worker.start()

    # -- calls under test ------------------------------------------------------------

    def encode(self, data, stream=None):
        """Ids of one text (as ``encode``), sampled for a background check."""
        enc = self._encoder
        if enc is None:
            from . import encode as enc
        ids = enc(data, stream) if stream is not None else enc(data)
        self.observe(data, ids, stream=stream)
        return ids

    def encode_batch(self, data, offsets, stream=None):
        """(ids, out_offsets) of a batch (as ``encode_batch``), sampled for a
        background check of every text in it."""
        enc = self._batch_encoder
        if enc is None:
            from . import encode_batch as enc
        ids, out_off = enc(data, offsets, stream) if stream is not None else enc(data, offsets)
        self.observe(data, ids, offsets=offsets, out_offsets=out_off, stream=stream)
        return ids, out_off

    def observe(self, data, ids, offsets=None, out_offsets=None, n_ids=None, stream=None):
        """Count one call whose ids the caller already has and sample it.

        ``data`` is the uint8 input and ``ids`` the ids of the whole call; for
        a batch, ``offsets`` and ``out_offsets`` are the input and output
        offsets [B + 1].  After an asynchronous ``encode_into`` on ``stream``,
        pass the id buffer as ``ids`` and the device count ``out_n`` as
        ``n_ids``: the check reads the count when the call has finished (a
        negative count, a data error, agrees with a standard tokenizer that
        raises).  Returns True when the call was queued for a check."""
        with self._lock:
            call = self._calls
            self._calls += 1
            if self._closed:
                raise RuntimeError("ShadowVerifier is closed")
        if self.rate <= 0.0 or self._rng.random() >= self.rate:
            return False
        with self._lock:
            self._sampled += 1
        snap = self._snapshot(data, ids, offsets, out_offsets, n_ids, stream)
        try:
            self._q.put_nowait((call, snap))
        except queue.Full:
            with self._lock:
                self._dropped += 1
            return False
        return True

    @staticmethod
    def _snapshot(data, ids, offsets, out_offsets, n_ids, stream):
        """Copies of the call's tensors, taken in stream order, plus an event
        that marks when they are complete (device tensors only)."""
        parts = [data, ids, offsets, out_offsets, n_ids]
        if getattr(data, "is_cuda", False):
            import torch
            s = stream if stream is not None else torch.cuda.current_stream()
            with torch.cuda.stream(s):
                copies = [None if p is None else (p.clone() if torch.is_tensor(p) else p) for p in parts]
                ev = torch.cuda.Event()
                ev.record(s)
            return copies, ev
        copies = [None if p is None else _host_copy(p) for p in parts]
        return copies, None

    # -- background side ---------------------------------------------------------------

    def _run(self):
        while True:
            item = self._q.get()
            try:
                if item is None:
                    return
                call, (parts, ev) = item
                if ev is not None:
                    ev.synchronize()
                self._check(call, *[None if p is None else _to_numpy(p) for p in parts])
            except Exception as e:  # noqa: BLE001 - the thread must outlive a failing hook or write
                with self._lock:
                    self._errors += 1
                    self.last_error = "%s: %s" % (type(e).__name__, e)
            finally:
                self._q.task_done()

    def _check(self, call, data, ids, offsets, out_offsets, n_ids):
        raw = data.astype(np.uint8).tobytes()
        code = 0
        if n_ids is not None:
            n = int(np.asarray(n_ids).reshape(-1)[-1])
            ids, code = (ids[:n], 0) if n >= 0 else (ids[:0], n)
        if offsets is None:
            texts = [(0, raw, ids)]
        else:
            offsets = offsets.astype(np.int64)
            out_offsets = out_offsets.astype(np.int64)
            texts = [(b, raw[offsets[b]:offsets[b + 1]], ids[out_offsets[b]:out_offsets[b + 1]])
                     for b in range(len(offsets) - 1)]
        bad = []
        for b, text, got in texts:
            err = ""
            try:
                r = self.reference(text)
                ref = np.asarray(r if hasattr(r, "__len__") else list(r), dtype=np.int64).reshape(-1)
            except Exception as e:  # noqa: BLE001 - a failure of the standard tokenizer is a finding too
                ref, err = np.zeros(0, dtype=np.int64), "%s: %s" % (type(e).__name__, e)
            if code:
                # the encoder reported a data error: right only if the standard one fails too
                d = -1 if err else 0
                err = err or "encoder reported error %d; the standard tokenizer did not" % code
            else:
                d = first_difference(got, ref) if not err else 0
            if d >= 0:
                # lists only for the (rare) quarantined samples: the comparison
                # itself stays in numpy, so the thread holds the interpreter lock
                # for little time on a clean check
                bad.append(Sample(call, b, text, got.tolist(), ref.tolist(), d, err))
        with self._lock:
            self._checked += 1
            self._texts += len(texts)
            self._mismatches += len(bad)
            keep = bad[:max(0, self.max_quarantine - len(self.quarantine))]
            self.quarantine.extend(keep)
            first_k = len(self.quarantine) - len(keep)
        for k, s in enumerate(keep):
            if self.quarantine_dir:
                _write_sample(self.quarantine_dir, first_k + k, s)
        for s in bad:
            if self.on_mismatch is not None:
                self.on_mismatch(s)

    # -- control -----------------------------------------------------------------------

    def drain(self):
        """Wait until every queued check has run."""
        self._q.join()

    def stats(self):
        """Counts so far: calls seen, calls sampled, sampled calls dropped
        (queue full), calls checked, texts checked, texts that mismatched, and
        checks that failed in the verifier itself (a raising ``on_mismatch``
        hook, an unwritable ``quarantine_dir``; the last one is kept in
        ``last_error``)."""
        with self._lock:
            return {"calls": self._calls, "sampled": self._sampled, "dropped": self._dropped,
                    "checked": self._checked, "texts": self._texts, "mismatches": self._mismatches,
                    "errors": self._errors}

    def close(self):
        """Run the queued checks, then stop the background thread."""
        with self._lock:
            if self._closed:
                return
            self._closed = True
        self._q.put(None)
        self._worker.join()

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()


def _to_numpy(x):
    if hasattr(x, "detach"):
        return x.detach().cpu().numpy()
    return np.asarray(x)


def _host_copy(x):
    if hasattr(x, "detach"):
        return x.detach().clone()
    if isinstance(x, (bytes, bytearray)):
        return np.frombuffer(bytes(x), dtype=np.uint8).copy()
    return np.array(x, copy=True)


def _write_sample(root, k, s):
    os.makedirs(root, exist_ok=True)
    base = os.path.join(root, "sample_%d" % k)
    with open(base + ".bin", "wb") as f:
        f.write(s.data)
    with open(base + ".json", "w") as f:
        json.dump({"call": s.call, "text_index": s.text_index, "first_diff": s.first_diff, "error": s.error,
                   "ids": s.ids, "ref_ids": s.ref_ids}, f)


def load_sample(path_base):
    """(bytes, record) of a quarantined sample written under ``quarantine_dir``
    (``path_base`` without the .bin / .json suffix), for offline reproduction."""
    with open(path_base + ".bin", "rb") as f:
        data = f.read()
    with open(path_base + ".json") as f:
        rec = json.load(f)
    return data, rec
