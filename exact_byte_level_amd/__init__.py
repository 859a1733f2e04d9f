"""exact_byte_level_amd -- exact byte-level BPE tokenization on one MI355X.

Thin ctypes binding over libtt.so (C ABI in include/tt.h).  Every step of the
tokenization runs in the library's HIP kernels; this module only marshals
arguments: PyTorch provides device memory (``data_ptr()``) and the current HIP
stream.  If libtt.so is missing the binding raises; there is no CPU fallback.

    import exact_byte_level_amd as tt
    tt.load(merges, pattern_id=tt.PATTERN_CL100K)   # merges: int32 [M, 2], rank order
    ids = tt.encode(torch.frombuffer(text, dtype=torch.uint8).cuda())
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtt.so")

PATTERN_GPT2 = 0
PATTERN_CL100K = 1

TT_OK = 0
TT_EINVAL = -1
TT_ETABLE = -2
TT_ENOMEM = -3
TT_EHIP = -4
TT_EUTF8 = -5
TT_ENOTLOADED = -6
TT_EOFFSETS = -7
TT_ETOOBIG = -8
TT_ESTALE = -9
TT_EUNSUPPORTED = -10

_lib = None


class TTError(RuntimeError):
    def __init__(self, code, where):
        self.code = code
        super().__init__("%s: %s (%d)" % (where, strerror(code) if _lib else "error", code))


def lib():
    """The loaded libtt.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libtt.so not built (%s); run exact_byte_level_amd.build.build()" % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
        L.tt_load_bpe.argtypes = [vp, vp, i64, i32]
        L.tt_load_bpe_ex.argtypes = [vp, vp, i64, i32, ctypes.c_uint32]
        L.tt_reserve.argtypes = [i64, i32]
        L.tt_encode.argtypes = [vp, i64, vp, vp, vp]
        L.tt_encode_noalloc.argtypes = [vp, i64, vp, vp, vp]
        L.tt_encode_batch.argtypes = [vp, i64, vp, i32, vp, vp, vp]
        L.tt_pretokenize.argtypes = [vp, i64, vp, i32, vp, vp, vp]
        L.tt_encode_offsets.argtypes = [vp, i64, vp, i32, vp, vp, vp, vp]
        L.tt_session_create.argtypes = [i64, i64, vp]
        L.tt_session_destroy.argtypes = [vp]
        L.tt_session_reset.argtypes = [vp, vp, i64, vp]
        L.tt_session_append.argtypes = [vp, vp, i64, vp, vp]
        L.tt_session_view.argtypes = [vp, vp, vp, vp, vp, vp]
        L.tt_session_read.argtypes = [vp, vp, vp, vp, vp]
        L.tt_char_class.argtypes = [ctypes.c_uint32]
        L.tt_profile.argtypes = [ctypes.c_int]
        L.tt_profile_read.argtypes = [ctypes.POINTER(ctypes.c_char_p), ctypes.POINTER(ctypes.c_float), ctypes.c_int]
        L.tt_free.argtypes = []
        L.tt_free.restype = None
        L.tt_strerror.argtypes = [ctypes.c_int]
        L.tt_strerror.restype = ctypes.c_char_p
        for f in ("tt_load_bpe", "tt_load_bpe_ex", "tt_reserve", "tt_encode", "tt_encode_noalloc", "tt_encode_batch", "tt_pretokenize", "tt_encode_offsets",
                  "tt_session_create", "tt_session_destroy", "tt_session_reset", "tt_session_append",
                  "tt_session_view", "tt_session_read", "tt_char_class", "tt_profile", "tt_profile_read"):
            getattr(L, f).restype = ctypes.c_int
        _lib = L
    return _lib


def strerror(code):
    return lib().tt_strerror(int(code)).decode()


def _check(rc, where):
    if rc != TT_OK:
        raise TTError(rc, where)


_RAW_STREAM = None


def _stream(stream, dev=None):
    """The HIP stream to enqueue on: the given torch stream, else the current
    stream of device dev (the data's device).  The current stream is read as
    a raw handle: building a torch Stream object for it costs a few
    microseconds, which a single request would wait for on the GPU."""
    global _RAW_STREAM
    if stream is not None:
        return ctypes.c_void_p(stream.cuda_stream)
    import torch
    if _RAW_STREAM is None:
        _RAW_STREAM = getattr(torch._C, "_cuda_getCurrentRawStream", False)
    if dev is None:
        dev = torch.cuda.current_device()
    if _RAW_STREAM:
        return ctypes.c_void_p(_RAW_STREAM(dev))
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


LOAD_IGNORE_MERGES = 1


def load(merges, ranks=None, pattern_id=PATTERN_GPT2, ignore_merges=False):
    """Load a merge table: merges int32 [M, 2]; merge k makes id 256 + ranks[k]
    (ranks defaults to 0..M-1, i.e. rows in rank order).  ignore_merges turns
    on the whole-word rule: a piece that is a vocabulary token becomes it."""
    m = np.ascontiguousarray(np.asarray(merges, dtype=np.int32).reshape(-1, 2))
    r = None if ranks is None else np.ascontiguousarray(np.asarray(ranks, dtype=np.int32).reshape(-1))
    if r is not None and len(r) != len(m):
        raise ValueError("ranks must have one entry per merge")
    rc = lib().tt_load_bpe_ex(m.ctypes.data if len(m) else None, None if r is None else r.ctypes.data,
                              len(m), int(pattern_id), LOAD_IGNORE_MERGES if ignore_merges else 0)
    _check(rc, "tt_load_bpe_ex")


def reserve(max_bytes, max_seqs=1):
    _check(lib().tt_reserve(int(max_bytes), int(max_seqs)), "tt_reserve")


def encode_into(data, out_ids, out_n, stream=None):
    """Enqueue an encode of a uint8 CUDA tensor into caller buffers (no sync)."""
    n = data.numel()
    rc = lib().tt_encode(data.data_ptr() if n else None, n, out_ids.data_ptr(), out_n.data_ptr(),
                         _stream(stream, data.device.index))
    _check(rc, "tt_encode")


def encode(data, stream=None):
    """Token ids (int32 CUDA tensor) of one UTF-8 text held in a uint8 CUDA tensor."""
    import torch
    assert data.dtype == torch.uint8 and data.is_cuda and data.is_contiguous()
    out = torch.empty(max(data.numel(), 1), dtype=torch.int32, device=data.device)
    out_n = torch.empty(1, dtype=torch.int64, device=data.device)
    encode_into(data, out, out_n, stream)
    t = int(out_n.item())
    if t < 0:
        raise TTError(t, "tt_encode")
    return out[:t]


NOALLOC_MAX_BYTES = 1 << 21


def encode_noalloc_into(data, out_ids, out_n, stream=None):
    """tt_encode_noalloc: as encode_into, but the library allocates nothing
    (a fixed per-device scratch array; inputs up to NOALLOC_MAX_BYTES)."""
    n = data.numel()
    rc = lib().tt_encode_noalloc(data.data_ptr() if n else None, n, out_ids.data_ptr(), out_n.data_ptr(),
                                 _stream(stream, data.device.index))
    _check(rc, "tt_encode_noalloc")


def encode_batch_into(data, offsets, out_ids, out_offsets, stream=None):
    n = data.numel()
    rc = lib().tt_encode_batch(data.data_ptr() if n else None, n, offsets.data_ptr(), offsets.numel() - 1,
                               out_ids.data_ptr(), out_offsets.data_ptr(), _stream(stream, data.device.index))
    _check(rc, "tt_encode_batch")


def encode_batch(data, offsets, stream=None):
    """(ids, out_offsets) for concatenated texts with int64 CUDA offsets [B+1]."""
    import torch
    assert offsets.dtype == torch.int64 and offsets.is_cuda
    out = torch.empty(max(data.numel(), 1), dtype=torch.int32, device=data.device)
    out_off = torch.empty(offsets.numel(), dtype=torch.int64, device=data.device)
    encode_batch_into(data, offsets, out, out_off, stream)
    off = out_off.cpu()
    t = int(off[-1])
    if t < 0:
        raise TTError(t, "tt_encode_batch")
    return out[:t], off


def pretokenize(data, offsets=None, stream=None):
    """Byte offsets (int32 CUDA tensor) of every pre-token start (no sentinel)."""
    import torch
    n = data.numel()
    starts = torch.empty(n + 1, dtype=torch.int32, device=data.device)
    out_np = torch.empty(1, dtype=torch.int64, device=data.device)
    rc = lib().tt_pretokenize(data.data_ptr() if n else None, n,
                              None if offsets is None else offsets.data_ptr(),
                              1 if offsets is None else offsets.numel() - 1,
                              starts.data_ptr(), out_np.data_ptr(), _stream(stream, data.device.index))
    _check(rc, "tt_pretokenize")
    p = int(out_np.item())
    if p < 0:
        raise TTError(p, "tt_pretokenize")
    return starts[:p]


def encode_offsets_into(data, offsets, out_ids, out_starts, out_counts, stream=None):
    """Enqueue an encode with byte offsets into caller buffers (no sync)."""
    n = data.numel()
    rc = lib().tt_encode_offsets(data.data_ptr() if n else None, n,
                                 None if offsets is None else offsets.data_ptr(),
                                 1 if offsets is None else offsets.numel() - 1,
                                 out_ids.data_ptr(), out_starts.data_ptr(), out_counts.data_ptr(),
                                 _stream(stream, data.device.index))
    _check(rc, "tt_encode_offsets")


def encode_offsets(data, offsets=None, stream=None):
    """Token ids and byte starts of one text, or of a batch with int64 CUDA offsets.

    Returns (ids, starts) for one text and (ids, starts, out_offsets) for a
    batch: token i covers bytes [starts[i], starts[i+1]) of ``data`` (offsets
    into the whole buffer) and starts[T] = n.
    """
    import torch
    assert data.dtype == torch.uint8 and data.is_cuda and data.is_contiguous()
    n = data.numel()
    out = torch.empty(max(n, 1), dtype=torch.int32, device=data.device)
    starts = torch.empty(n + 1, dtype=torch.int32, device=data.device)
    cnt = torch.empty(1 if offsets is None else offsets.numel(), dtype=torch.int64, device=data.device)
    encode_offsets_into(data, offsets, out, starts, cnt, stream)
    c = cnt.cpu()
    t = int(c[-1])
    if t < 0:
        raise TTError(t, "tt_encode_offsets")
    if offsets is None:
        return out[:t], starts[:t + 1]
    return out[:t], starts[:t + 1], c


class Session:
    """A growing text kept on the device with its ids and token byte starts;
    appends are repaired from a tail window (tt_session_* in include/tt.h).

        s = tt.Session(capacity=4 << 20)
        s.reset(u8_cuda_tensor)
        info = s.append(u8_cuda_delta)   # {'doublings': 0..5 or -1, ...}
        ids, starts = s.ids(), s.starts()
    """

    def __init__(self, capacity, tail_bytes=0):
        h = ctypes.c_void_p()
        _check(lib().tt_session_create(int(capacity), int(tail_bytes), ctypes.byref(h)), "tt_session_create")
        self._h = h

    def close(self):
        if self._h:
            lib().tt_session_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def reset(self, data, stream=None):
        n = data.numel()
        _check(lib().tt_session_reset(self._h, data.data_ptr() if n else None, n, _stream(stream)),
               "tt_session_reset")

    def append(self, delta, stream=None):
        """Append a uint8 CUDA tensor; returns how the tokens were repaired."""
        info = (ctypes.c_int64 * 4)()
        n = delta.numel()
        _check(lib().tt_session_append(self._h, delta.data_ptr() if n else None, n, info, _stream(stream)),
               "tt_session_append")
        return {"doublings": int(info[0]), "window_bytes": int(info[1]), "splice": int(info[2]),
                "tokens": int(info[3])}

    def sizes(self):
        n, t = ctypes.c_int64(), ctypes.c_int64()
        _check(lib().tt_session_view(self._h, None, ctypes.byref(n), None, None, ctypes.byref(t)), "tt_session_view")
        return n.value, t.value

    def _read(self, which, stream=None):
        import torch
        n, t = self.sizes()
        size, dtype = {"text": (n, torch.uint8), "ids": (t, torch.int32), "starts": (t + 1, torch.int32)}[which]
        out = torch.empty(max(size, 1), dtype=dtype, device="cuda")
        ptrs = [None, None, None]
        ptrs[["text", "ids", "starts"].index(which)] = out.data_ptr()
        _check(lib().tt_session_read(self._h, *ptrs, _stream(stream)), "tt_session_read")
        return out[:size]

    def text(self, stream=None):
        return self._read("text", stream)

    def ids(self, stream=None):
        return self._read("ids", stream)

    def starts(self, stream=None):
        return self._read("starts", stream)


def char_class(cp):
    """Class of a code point in the compiled table: 0 other, 1 L, 2 N, 3 White_Space."""
    return lib().tt_char_class(int(cp))


def profile(enable):
    """Switch per-kernel event timing of later calls on or off."""
    _check(lib().tt_profile(1 if enable else 0), "tt_profile")


def profile_read(cap=64):
    """[(kernel name, ms)] of the last call (waits for it)."""
    names = (ctypes.c_char_p * cap)()
    ms = (ctypes.c_float * cap)()
    k = lib().tt_profile_read(names, ms, cap)
    if k < 0:
        raise TTError(k, "tt_profile_read")
    return [(names[i].decode(), float(ms[i])) for i in range(k)]


def free():
    lib().tt_free()
