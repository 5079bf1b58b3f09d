"""Tensor-level calls of the SplitZip codec: marshalling of torch tensors
(device memory and streams only) into the C ABI.  No codec arithmetic is done
here; calibrate, encode and decode run entirely in the HIP kernels."""
from __future__ import annotations

import ctypes

import torch

from . import _abi
from ._abi import CHUNK, Codebook, Item, Meta, SlotItem, SplitZipError

CODEBOOK_BYTES = ctypes.sizeof(Codebook)
META_BYTES = ctypes.sizeof(Meta)


def _stream(stream, device) -> int:
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return int(stream.cuda_stream)


def _bits(x: torch.Tensor) -> torch.Tensor:
    if x.dtype is not torch.bfloat16:
        # page 2: only BF16 is encoded (other formats, e.g. FP8, would expand)
        raise ValueError("SplitZip expects a bfloat16 tensor, got %s" % x.dtype)
    if not x.is_cuda:
        raise ValueError("SplitZip runs on the GPU: move the tensor to a HIP device")
    if not x.is_contiguous():
        raise ValueError("SplitZip expects a contiguous tensor")
    return x.reshape(-1).view(torch.int16)


def payload_size(n: int, n_esc: int) -> int:
    return _abi.splitzip_payload_size(n, n_esc)


class Workspace:
    """Device scratch for calibrate / encode, sized for tensors of up to n_max
    elements (or, with ``batch_ns``, for batched calls on tensors of those
    sizes).  One workspace per stream that runs codec calls concurrently."""

    def __init__(self, n_max: int = 0, device=None, stream=None, batch_ns=None):
        device = torch.device(device if device is not None else "cuda")
        self.n_max = n_max
        self.nbytes = _abi.splitzip_workspace_size(n_max)
        if batch_ns is not None:
            self.nbytes = max(self.nbytes, _abi.splitzip_workspace_size_batch(list(batch_ns)))
        self.buf = torch.empty(self.nbytes, dtype=torch.uint8, device=device)
        _abi._check("splitzip_workspace_init",
                    _abi.splitzip_workspace_init(self.buf.data_ptr(), self.nbytes,
                                                 _stream(stream, device)))

    def ptr(self) -> int:
        return self.buf.data_ptr()


def new_codebook(device) -> torch.Tensor:
    return torch.empty(CODEBOOK_BYTES, dtype=torch.uint8, device=device)


def new_meta(device) -> torch.Tensor:
    return torch.empty(META_BYTES, dtype=torch.uint8, device=device)


def calibrate(x: torch.Tensor, ws: Workspace, cb: torch.Tensor | None = None,
              stream=None) -> torch.Tensor:
    """Per-tensor top-16 exponent codebook (device bytes of splitzip_codebook)."""
    xb = _bits(x)
    if cb is None:
        cb = new_codebook(x.device)
    _buf(cb, CODEBOOK_BYTES, "codebook")
    _same_gpu(x.device, ws.buf)
    _abi._check("splitzip_calibrate",
                _abi.splitzip_calibrate(xb.data_ptr(), xb.numel(), cb.data_ptr(), ws.ptr(),
                                        ws.nbytes, _stream(stream, x.device)))
    return cb


def payload_for(cb: torch.Tensor, n: int) -> torch.Tensor:
    """A payload buffer for an n-element tensor encoded with ``cb``: exactly
    its payload's length when ``cb`` was calibrated on that tensor (n_esc =
    total - covered), else the all-escape bound.  Reads the codebook back,
    so it synchronises with the device."""
    c = read_codebook(cb)
    e = c.total - c.covered if c.total == n and c.covered <= n else n
    return torch.empty(max(payload_size(n, e), 16), dtype=torch.uint8, device=cb.device)


def encode(x: torch.Tensor, cb: torch.Tensor, ws: Workspace, payload: torch.Tensor | None = None,
           meta: torch.Tensor | None = None, stream=None, chunk_size: int = CHUNK):
    """Encode into ``payload`` (allocated for the all-escape bound, 8.5 bytes
    per element, when None; ``payload_for`` gives one of the payload's own
    length).  Returns (payload, meta) as uint8 tensors; the payload occupies
    the first meta.comp_bytes bytes.  ``payload`` may be pinned host memory:
    the kernels then write it over the host link (an offload without a
    separate copy)."""
    xb = _bits(x)
    n = xb.numel()
    if payload is None:
        payload = torch.empty(max(payload_size(n, n), 16), dtype=torch.uint8, device=x.device)
    capacity = _buf(payload, 0, "payload")
    if meta is None:
        meta = new_meta(x.device)
    _buf(cb, CODEBOOK_BYTES, "codebook")
    _buf(meta, META_BYTES, "metadata")
    _same_gpu(x.device, ws.buf, payload, cb, meta)
    _abi._check("splitzip_encode_chunked",
                _abi.splitzip_encode_chunked(xb.data_ptr(), n, cb.data_ptr(), chunk_size,
                                             payload.data_ptr(), capacity,
                                             meta.data_ptr(), ws.ptr(), ws.nbytes,
                                             _stream(stream, x.device)))
    return payload, meta


def decode(payload: torch.Tensor, meta: torch.Tensor, cb_or_dec_lut: torch.Tensor, n: int,
           out: torch.Tensor | None = None, status: torch.Tensor | None = None,
           stream=None) -> torch.Tensor:
    """Decode to a flat bfloat16 tensor of n elements (``out`` when given).
    ``cb_or_dec_lut`` is a device codebook or a 16-byte dec_lut tensor.  The
    payload may also sit in pinned host memory: the kernel then reads it over
    the host link while it decodes (no separate copy)."""
    dev = _gpu_of(out, meta, cb_or_dec_lut, payload)
    payload_bytes = _buf(payload, 0, "payload")
    if out is None:
        out = torch.empty(n, dtype=torch.bfloat16, device=dev)
    if out.dtype is not torch.bfloat16 or not out.is_contiguous() or out.numel() != n:
        raise ValueError("out must be a contiguous bfloat16 tensor of n elements")
    _device_or_pinned(out, "output")
    _buf(meta, META_BYTES, "metadata")
    st_ptr = _status_ptr(status)
    _same_gpu(dev, payload, meta, cb_or_dec_lut, out, status)
    lut_ptr = _lut_ptr(cb_or_dec_lut)
    _abi._check("splitzip_decode",
                _abi.splitzip_decode(payload.data_ptr(), payload_bytes, meta.data_ptr(),
                                     lut_ptr, out.data_ptr(), n, st_ptr, _stream(stream, dev)))
    return out


def _device_or_pinned(t: torch.Tensor, what: str) -> None:
    # a kernel may only touch pageable host memory by faulting
    if t.device.type != "cuda" and not t.is_pinned():
        raise ValueError("the %s must be on the GPU or in pinned host memory" % what)


def _buf(t: torch.Tensor, nbytes: int, what: str) -> int:
    """Checks a raw buffer handed to the kernels (device or pinned host,
    contiguous, at least ``nbytes`` bytes) and returns its size in bytes."""
    _device_or_pinned(t, what)
    if not t.is_contiguous():
        raise ValueError("the %s must be a contiguous tensor" % what)
    size = t.numel() * t.element_size()
    if size < nbytes:
        raise ValueError("the %s needs at least %d bytes, got %d" % (what, nbytes, size))
    return size


def _status_ptr(status: torch.Tensor | None) -> int:
    if status is None:
        return 0
    if status.dtype is not torch.int32:
        raise ValueError("the status word must be an int32 tensor")
    _buf(status, 4, "status word")
    return status.data_ptr()


def _same_gpu(dev: torch.device, *tensors) -> None:
    # every device buffer of one call lives on the GPU the call runs on
    for t in tensors:
        if t is not None and t.device.type == "cuda" and t.device != dev:
            raise ValueError("all device buffers of a call must be on %s, got %s" % (dev, t.device))


def _gpu_of(*tensors) -> torch.device:
    for t in tensors:
        if t is not None and t.device.type == "cuda":
            return t.device
    raise ValueError("decode needs its output, metadata or codebook on the GPU")


def _lut_ptr(cb_or_dec_lut: torch.Tensor) -> int:
    size = _buf(cb_or_dec_lut, 0, "codebook")
    if size == CODEBOOK_BYTES:
        return cb_or_dec_lut.data_ptr() + _abi.DEC_LUT_OFFSET
    if size != 16:
        raise ValueError("expected a codebook (%d bytes) or a 16-byte dec_lut, got %d bytes"
                         % (CODEBOOK_BYTES, size))
    return cb_or_dec_lut.data_ptr()


def decode_slot(slot: torch.Tensor, meta: torch.Tensor, cb_or_dec_lut: torch.Tensor, n: int,
                stash: torch.Tensor, status: torch.Tensor | None = None,
                stream=None, resident: bool = False) -> torch.Tensor:
    """Decode in place: ``slot`` (contiguous device tensor of any dtype, at
    least max(2n, payload_size(n, 0)) bytes) holds the payload at its head;
    afterwards its first 2n bytes hold the n bfloat16 values, returned as a
    flat bfloat16 view.  ``stash`` is device scratch of at least comp_bytes
    bytes that does not overlap the slot.  ``resident`` takes the form that
    needs the whole grid resident at once (faster on a GPU the decode has to
    itself, see ``decode_slots``)."""
    if resident:
        return decode_slots([slot], [meta], [cb_or_dec_lut], [n], [stash], status=status,
                            stream=stream, resident=True)[0]
    if not slot.is_contiguous():
        # page 1, decode_slot_into: the slot must be contiguous
        raise ValueError("the slot tensor must be contiguous")
    raw = slot.reshape(-1).view(torch.uint8)
    _device_or_pinned(raw, "slot")
    stash_bytes = _buf(stash, 0, "stash")
    _buf(meta, META_BYTES, "metadata")
    st_ptr = _status_ptr(status)
    _same_gpu(slot.device, stash, meta, cb_or_dec_lut, status)
    _abi._check("splitzip_decode_slot",
                _abi.splitzip_decode_slot(raw.data_ptr(), raw.numel(), meta.data_ptr(),
                                          _lut_ptr(cb_or_dec_lut), n, stash.data_ptr(),
                                          stash_bytes, st_ptr, _stream(stream, slot.device)))
    return raw[: 2 * n].view(torch.bfloat16)


def decode_slots(slots, metas, cbs_or_luts, ns, stashes, status: torch.Tensor | None = None,
                 stream=None, resident: bool = False):
    """In-place decode of a group of slots (see ``decode_slot``), up to 32
    per launch.  Returns the flat bfloat16 views of the slots.  With
    ``resident`` the library's resident form runs (one grid barrier per
    slot, overlapping tiles held in registers; it gives up and finishes the
    slots later when concurrent work keeps its grid from being placed), else
    the multi-pass form, which shares the GPU with concurrent work."""
    count = len(slots)
    if not (len(metas) == len(cbs_or_luts) == len(ns) == len(stashes) == count):
        raise ValueError("one meta, codebook, size and stash per slot")
    items = (SlotItem * max(count, 1))()
    raws = []
    for k in range(count):
        if not slots[k].is_contiguous():
            raise ValueError("the slot tensors must be contiguous")
        raw = slots[k].reshape(-1).view(torch.uint8)
        _device_or_pinned(raw, "slot")
        _buf(metas[k], META_BYTES, "metadata")
        raws.append(raw)
        it = items[k]
        it.slot, it.slot_bytes = raw.data_ptr(), raw.numel()
        it.meta, it.dec_lut, it.n = metas[k].data_ptr(), _lut_ptr(cbs_or_luts[k]), ns[k]
        it.stash = stashes[k].data_ptr()
        it.stash_bytes = _buf(stashes[k], 0, "stash")
    st_ptr = _status_ptr(status)
    dev = _gpu_of(*slots, *metas) if count else torch.device("cuda")
    _same_gpu(dev, *slots, *stashes, *metas, *cbs_or_luts, status)
    fn = "splitzip_decode_slot_batch_resident" if resident else "splitzip_decode_slot_batch"
    _abi._check(fn, getattr(_abi, fn)(items, count, st_ptr, _stream(stream, dev)))
    return [raw[: 2 * n].view(torch.bfloat16) for raw, n in zip(raws, ns)]


def read_codebook(cb: torch.Tensor) -> Codebook:
    host = cb.detach().to("cpu").numpy().tobytes()
    return Codebook.from_buffer_copy(host)


def read_meta(meta: torch.Tensor) -> Meta:
    host = meta.detach().to("cpu").numpy().tobytes()
    return Meta.from_buffer_copy(host)


class Batch:
    """Per-tensor buffers of a batched call: codebook, payload, metadata and
    output for each tensor of ``xs`` (device tensors of bfloat16).  The item
    array is built once, so repeated calls only cross the C ABI."""

    def __init__(self, xs, device=None, capacities=None):
        self.xs = [_bits(x) for x in xs]
        device = self.xs[0].device if self.xs else torch.device(device or "cuda")
        self.ns = [x.numel() for x in self.xs]
        caps = capacities or [max(payload_size(n, n), 16) for n in self.ns]
        self.cbs = [new_codebook(device) for _ in self.xs]
        self.payloads = [torch.empty(c, dtype=torch.uint8, device=device) for c in caps]
        self.metas = [torch.zeros(META_BYTES, dtype=torch.uint8, device=device) for _ in self.xs]
        self.outs = [torch.empty(n, dtype=torch.bfloat16, device=device) for n in self.ns]
        self.items = (Item * max(len(self.xs), 1))()
        for k, x in enumerate(self.xs):
            it = self.items[k]
            it.x, it.n, it.cb = x.data_ptr(), self.ns[k], self.cbs[k].data_ptr()
            it.payload, it.capacity = self.payloads[k].data_ptr(), self.payloads[k].numel()
            it.meta, it.out = self.metas[k].data_ptr(), self.outs[k].data_ptr()
        self.count = len(self.xs)
        self.device = device

    def fit_payloads(self, slack: int = 0):
        """Size every payload buffer for the payload its tensor has under the
        codebook the last calibrate wrote: n_esc = total - covered, exact for
        a codebook calibrated on that tensor (every exponent outside the
        top 16 escapes; page "splitzip_codec.py -- SplitZip codec adapter
        for diffusers-dynamic-offloader", calibrate_codebook), instead of the
        all-escape bound (8.5 bytes per element) the buffers start with.  A
        codebook whose total is not this tensor's length keeps the bound.
        Reads the codebooks back, so it synchronises with the device; an
        encode that would not fit still reports SPLITZIP_ERR_CAPACITY in its
        metadata."""
        for k, cb in enumerate(self.cbs):
            c = read_codebook(cb)
            n = self.ns[k]
            e = c.total - c.covered if c.total == n and c.covered <= n else n
            cap = max(payload_size(n, e) + slack, 16)
            self.payloads[k] = torch.empty(cap, dtype=torch.uint8, device=self.device)
            self.items[k].payload, self.items[k].capacity = self.payloads[k].data_ptr(), cap

    def calibrate(self, ws: Workspace, stream=None):
        _abi._check("splitzip_calibrate_batch",
                    _abi.splitzip_calibrate_batch(self.items, self.count, ws.ptr(), ws.nbytes,
                                                  _stream(stream, self.device)))

    def encode(self, ws: Workspace, stream=None):
        _abi._check("splitzip_encode_batch",
                    _abi.splitzip_encode_batch(self.items, self.count, ws.ptr(), ws.nbytes,
                                               _stream(stream, self.device)))

    def decode(self, status: torch.Tensor | None = None, stream=None):
        st_ptr = _status_ptr(status)
        _abi._check("splitzip_decode_batch",
                    _abi.splitzip_decode_batch(self.items, self.count, st_ptr,
                                               _stream(stream, self.device)))
