"""In-place decode: the payload sits at the head of the buffer that receives
the decoded tensor (page "splitzip_codec.py -- SplitZip codec adapter for
diffusers-dynamic-offloader", GpuSplitZipDecoder.decode_slot_into), checked
element by element against the input and the oracle's payload, and a
host-to-device pipeline that lands payloads in their slots on a copy stream
while another stream expands them."""
import numpy as np
import pytest
import torch

import lossless_bf16_tensor_splitzip_amd as S
from lossless_bf16_tensor_splitzip_amd import _abi
import oracle
import workloads as W
from test_gpu_parity import DEV, _say, host_bits, meta_to_device, workspace

pytestmark = pytest.mark.gpu

TILE = 8192
FILL = 0xA5


def setup_module(module):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    S.lib()


@pytest.fixture(params=["two", "passes2", "passes3", "passes8", "resident", "resident_abort",
                        "coop"])
def form(request, monkeypatch):
    """Form of the in-place decode: the library's multi-pass form (the
    default entry points; its default number of passes, or 2, 3 or 8
    passes), the resident form (the resident entry point; one grid barrier
    per slot, in an ordinary launch), the same with a zero barrier wait, so
    that nearly every barrier gives up and the slot is finished by the
    deferral kernel (the path taken when concurrent work keeps the grid
    from being placed), or the resident form launched cooperatively (forced
    for every call)."""
    monkeypatch.delenv("SPLITZIP_SLOT_WAIT_US", raising=False)
    monkeypatch.delenv("SPLITZIP_SLOT_LAUNCH", raising=False)
    monkeypatch.delenv("SPLITZIP_SLOT_PASSES", raising=False)
    if request.param == "resident_abort":
        monkeypatch.setenv("SPLITZIP_SLOT_WAIT_US", "0")
    elif request.param == "coop":
        monkeypatch.setenv("SPLITZIP_SLOT_LAUNCH", "coop")
    elif request.param.startswith("passes"):
        monkeypatch.setenv("SPLITZIP_SLOT_PASSES", request.param[len("passes"):])
    _RESIDENT[0] = request.param in ("resident", "resident_abort", "coop")
    yield request.param
    _RESIDENT[0] = False


_RESIDENT = [False]


def decode_slot(*args, **kw):
    """S.decode_slot in the form the test's `form` fixture chose."""
    return S.decode_slot(*args, resident=_RESIDENT[0], **kw)


def decode_slots(*args, **kw):
    return S.decode_slots(*args, resident=_RESIDENT[0], **kw)


def slot_for(payload: bytes, n: int, extra: int = 0) -> torch.Tensor:
    size = max(2 * n, S.payload_size(n, 0), len(payload)) + extra
    slot = torch.full((size,), FILL, dtype=torch.uint8)
    if payload:
        slot[: len(payload)] = torch.frombuffer(bytearray(payload), dtype=torch.uint8)
    return slot.to(DEV)


def stash_for(comp: int, extra: int = 0) -> torch.Tensor:
    return torch.full((max(comp, 16) + extra,), 0x5A, dtype=torch.uint8, device=DEV)


def oracle_case(x_cpu):
    xs = host_bits(x_cpu.reshape(-1))
    ocb = oracle.calibrate(xs)
    opay, om = oracle.encode(xs, ocb)
    return xs, ocb, opay, om


def run_slot(opay, om, dec_lut, validate=True, extra=0, stash_extra=0, ascending=False):
    n = om.n
    slot = slot_for(opay, n, extra)
    stash = stash_for(om.comp_bytes, stash_extra)
    lut = torch.tensor(np.asarray(dec_lut, np.uint8)).to(DEV)
    st = torch.zeros(1, dtype=torch.int32, device=DEV) if validate else None
    out = decode_slot(slot, meta_to_device(om, ascending), lut, n, stash, status=st)
    torch.cuda.synchronize()
    return slot, host_bits(out), (int(st.item()) if validate else 0)


def check_slot(x_cpu, name, extra=0, stash_extra=0):
    xs, ocb, opay, om = oracle_case(x_cpu)
    n = om.n
    _say("slot case %s n=%d e=%d comp=%d" % (name, n, om.n_esc, om.comp_bytes))
    # the oracle's escapes are ascending: decoded with and without the flag
    # that says so (per-tile patch, or the order-independent pass)
    for validate, ascending in ((False, True), (False, False), (True, True)):
        slot, out, st = run_slot(opay, om, ocb.dec_lut, validate, extra, stash_extra, ascending=ascending)
        assert st == 0
        assert np.array_equal(out, xs), name
        # bytes past the decoded tensor and past the payload are left alone
        tail = slot[max(2 * n, om.comp_bytes):].cpu().numpy()
        assert (tail == FILL).all(), name
        if om.comp_bytes > 2 * n:   # payload longer than the tensor: its tail stays
            assert slot[2 * n: om.comp_bytes].cpu().numpy().tobytes() == opay[2 * n:]


SIZES = [1, 2, 3, 7, 8, 9, 1023, 1025, 4095, 8191, 8192, 8193, 2 * TILE, 2 * TILE + 1,
         3 * TILE - 1, 4 * TILE, 4 * TILE + 5, 11 * TILE + 3, 100_003, 1_000_003]


@pytest.mark.parametrize("n", SIZES)
def test_slot_gaussian(n, form):
    check_slot(W.gaussian_weight(n, seed=100 + n % 97), "gaussian")


@pytest.mark.parametrize("n", [1, 9, 8193, 3 * TILE + 77, 65_537])
def test_slot_escape_heavy(n, form):
    # most exponents escape: the payload is longer than the tensor's 2n bytes
    check_slot(W.log_uniform_stress(n, seed=200 + n % 89), "escape heavy")


@pytest.mark.parametrize("n,esc_every", [(16 * TILE, 40), (16 * TILE + 3, 7), (40 * TILE, 3)])
def test_slot_split_positions(n, esc_every, form):
    """Escape densities that move the first directly decoded tile."""
    b = host_bits(W.gaussian_weight(n, seed=300 + esc_every)).copy()
    k = np.arange(0, n, esc_every)
    # planted values over 40 large exponents: most of them escape
    b[k] = ((k & 1) << 15) | ((150 + (k // esc_every) % 40) << 7) | (k & 0x7F)
    x = torch.from_numpy(b.view(np.int16)).view(torch.bfloat16)
    check_slot(x, "esc every %d" % esc_every, extra=12345)


@pytest.mark.parametrize("n", [3 * TILE + 77, 40 * TILE, 1_000_003])
def test_slot_buffers_larger_than_the_payload(n, form):
    """Slot and stash much longer than the payload: the last pass of the
    multi-pass form then runs workgroups for tiles past the payload's end
    that find nothing to do (their count is bounded by the buffers, not by
    the payload the kernels read)."""
    check_slot(W.gaussian_weight(n, seed=400 + n % 83), "large buffers",
               extra=7 * 2 * TILE + 5, stash_extra=5 * 2 * TILE + 13)


@pytest.mark.parametrize("seed", range(12))
def test_slot_random_sizes_densities_and_passes(seed, monkeypatch):
    """Seeded random sizes (1 .. 3M elements), escape densities (none to
    about half the elements) and pass counts of the multi-pass form: every
    in-place decode equals the input bit for bit, and the slot's bytes past
    the output are left alone."""
    rnd = np.random.default_rng(5000 + seed)
    n = int(rnd.integers(1, 3_000_000))
    passes = int(rnd.integers(2, 9))
    every = int(rnd.choice([0, 997, 61, 7, 2]))
    monkeypatch.setenv("SPLITZIP_SLOT_PASSES", str(passes))
    monkeypatch.delenv("SPLITZIP_SLOT_LAUNCH", raising=False)
    b = host_bits(W.gaussian_weight(n, seed=600 + seed)).copy()
    if every:
        k = np.arange(0, n, every)
        b[k] = ((k & 1) << 15) | ((150 + (k // every) % 40) << 7) | (k & 0x7F)
    x = torch.from_numpy(b.view(np.int16)).view(torch.bfloat16)
    _say("random slot case seed=%d n=%d passes=%d every=%d" % (seed, n, passes, every))
    check_slot(x, "random", extra=int(rnd.integers(0, 3 * 2 * TILE)),
               stash_extra=int(rnd.integers(0, 3 * 2 * TILE)))


def test_slot_matches_gpu_encode_and_plain_decode(form):
    """GPU encode -> payload copied to the slot head -> in-place decode, equal
    to the out-of-place decode, on one 33,554,432-element KV-cache tensor."""
    x = W.kv_cache_tensor(3, 1, device=DEV).reshape(-1)
    n = x.numel()
    ws = workspace(n)
    cb = S.calibrate(x, ws)
    payload, meta = S.encode(x, cb, ws)
    plain = S.decode(payload, meta, cb, n)
    m = S.read_meta(meta)
    slot = torch.empty(2 * n, dtype=torch.uint8, device=DEV)
    slot[: m.comp_bytes].copy_(payload[: m.comp_bytes])
    stash = torch.empty(m.comp_bytes, dtype=torch.uint8, device=DEV)
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    out = decode_slot(slot, meta, cb, n, stash, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    assert torch.equal(out.view(torch.int16), x.view(torch.int16))
    assert torch.equal(plain.view(torch.int16), x.view(torch.int16))
    # and again without validation, into the same slot
    slot[: m.comp_bytes].copy_(payload[: m.comp_bytes])
    out = decode_slot(slot, meta, cb, n, stash)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), x.view(torch.int16))


@pytest.mark.parametrize("make,n,seed", [(W.gaussian_weight, 40 * 2**20 + 5, 1),
                                         (W.log_uniform_stress, 40 * 2**20 + 3, 2)])
def test_slot_beyond_register_reach(make, n, seed, form):
    """More tiles overlap the payload than the resident form's grid holds in
    registers (3 per workgroup): the rest, and the partial last tile, go
    through the stash; stress data also gives held tiles with more escapes
    than their LDS list takes.  GPU encode, then the in-place decode with the
    stream marked ascending or not, with and without validation."""
    x = make(n, seed=2000 + seed).reshape(-1).to(DEV)
    ws = workspace(n)
    cb = S.calibrate(x, ws)
    payload, meta = S.encode(x, cb, ws)
    m = S.read_meta(meta)
    _say("slot beyond reach n=%d e=%d comp=%d form=%s" % (n, m.n_esc, m.comp_bytes, form))
    unmarked = meta.clone()
    unmarked[_abi.Meta.flags.offset: _abi.Meta.flags.offset + 4] = 0
    slot = torch.empty(max(2 * n, m.comp_bytes), dtype=torch.uint8, device=DEV)
    stash = torch.empty(m.comp_bytes, dtype=torch.uint8, device=DEV)
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    for md, status in ((meta, None), (meta, st), (unmarked, None), (unmarked, st)):
        slot.fill_(FILL)
        slot[: m.comp_bytes].copy_(payload[: m.comp_bytes])
        out = decode_slot(slot, md, cb, n, stash, status=status)
        torch.cuda.synchronize()
        assert int(st.item()) == 0
        assert torch.equal(out.view(torch.int16), x.view(torch.int16))
    del slot, stash, payload


def test_slot_rejects_bad_metadata_and_leaves_slot(form):
    x = W.gaussian_weight(5 * TILE + 11, seed=400)
    xs, ocb, opay, om = oracle_case(x)
    n = om.n
    lut = torch.tensor(np.asarray(ocb.dec_lut, np.uint8)).to(DEV)
    # stash shorter than the payload
    slot = slot_for(opay, n)
    before = slot.cpu().clone()
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    decode_slot(slot, meta_to_device(om), lut, n, stash_for(om.comp_bytes)[: om.comp_bytes - 1],
                  status=st)
    torch.cuda.synchronize()
    assert int(st.item()) & _abi.DEC_BAD_META
    assert torch.equal(slot.cpu(), before)
    # offsets that do not follow the layout
    bad = oracle.Meta(om.n, om.n_pairs, om.chunk_size, om.n_esc, om.comp_bytes,
                      (0, om.offsets[1] + 4) + tuple(om.offsets[2:]))
    st.zero_()
    decode_slot(slot, meta_to_device(bad), lut, n, stash_for(om.comp_bytes), status=st)
    torch.cuda.synchronize()
    assert int(st.item()) & _abi.DEC_BAD_META
    assert torch.equal(slot.cpu(), before)
    # non-contiguous slot and overlapping stash are argument errors
    with pytest.raises(ValueError):
        decode_slot(slot.view(-1, 2)[:, 0], meta_to_device(om), lut, n, stash_for(16))
    with pytest.raises(S.SplitZipError):
        decode_slot(slot, meta_to_device(om), lut, n, slot[-om.comp_bytes:])


def test_slot_unsorted_escape_stream_with_validation(form):
    n = 6 * TILE + 77
    x = torch.full((n,), 1.0, dtype=torch.bfloat16)
    pos = [3, 900, 5000, 8191, 8192, 9000, 17000, 24000, 40000, n - 1]
    x[pos] = torch.tensor([2.0, -4.0, 8.0, 0.5, 16.0, -0.25, 3.0, 64.0, -8.0, -2.0],
                          dtype=torch.bfloat16)
    xs = host_bits(x)
    ocb = oracle.calibrate(np.array([0x3F80], np.uint16))
    opay, om = oracle.encode(xs, ocb)
    e = om.n_esc
    buf = bytearray(opay)
    for sec, width in ((2, 4), (3, 2), (4, 1)):
        at = om.offsets[sec]
        items = [bytes(buf[at + width * r: at + width * (r + 1)]) for r in range(e)]
        for k, r in enumerate(range(e)[::-1]):
            buf[at + width * k: at + width * (k + 1)] = items[r]
    _, out, st = run_slot(bytes(buf), om, ocb.dec_lut)
    assert st & _abi.DEC_NOT_INCREASING
    assert np.array_equal(out, xs)


def test_h2d_pipeline_into_slots(form):
    """Payloads in pinned host memory are copied into the heads of their
    slots on a copy stream; a second stream waits on each copy's event and
    expands the slot in place, while the next copies proceed."""
    sizes = [1_000_003, 4 * TILE, 2_500_001, 77, 3_000_000, 8193]
    xs = [W.gaussian_weight(n, seed=500 + k) if k != 3 else W.log_uniform_stress(n, seed=9)
          for k, n in enumerate(sizes)]
    ws = workspace(max(sizes))
    host, metas, cbs = [], [], []
    for x in xs:
        xd = x.to(DEV)
        cb = S.calibrate(xd, ws)
        payload, meta = S.encode(xd, cb, ws)
        m = S.read_meta(meta)
        h = torch.empty(m.comp_bytes, dtype=torch.uint8, pin_memory=True)
        h.copy_(payload[: m.comp_bytes].cpu())
        host.append(h)
        metas.append(meta)
        cbs.append(cb)
    slots = [torch.empty(max(2 * n, h.numel()), dtype=torch.uint8, device=DEV)
             for n, h in zip(sizes, host)]
    stash = torch.empty(max(h.numel() for h in host), dtype=torch.uint8, device=DEV)
    copy_s, dec_s = torch.cuda.Stream(), torch.cuda.Stream()
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    torch.cuda.synchronize()
    outs = []
    for k, n in enumerate(sizes):
        with torch.cuda.stream(copy_s):
            slots[k][: host[k].numel()].copy_(host[k], non_blocking=True)
            ev = torch.cuda.Event()
            ev.record(copy_s)
        dec_s.wait_event(ev)
        outs.append(decode_slot(slots[k], metas[k], cbs[k], n, stash, status=st, stream=dec_s))
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    for x, out in zip(xs, outs):
        assert np.array_equal(host_bits(out.cpu()), host_bits(x))


def test_slot_batch_matches_inputs_across_launches(form):
    """40 payloads of mixed sizes and escape densities (two launch pairs),
    each at the head of its own slot, decoded in place as one group."""
    g = torch.Generator().manual_seed(11)
    sizes = [int(v) for v in torch.randint(1, 200_000, (40,), generator=g)]
    sizes[3], sizes[17], sizes[33] = 0, 8192, 3 * 8192 + 1
    xs = [W.log_uniform_stress(n, seed=700 + k) if k % 7 == 3 else W.gaussian_weight(n, seed=700 + k)
          for k, n in enumerate(sizes)]
    slots, metas, luts, stashes, want = [], [], [], [], []
    for x in xs:
        xs_h, ocb, opay, om = oracle_case(x)
        slots.append(slot_for(opay, om.n))
        metas.append(meta_to_device(om))
        luts.append(torch.tensor(np.asarray(ocb.dec_lut, np.uint8)).to(DEV))
        stashes.append(stash_for(om.comp_bytes))
        want.append(xs_h)
    _say("slot batch of %d" % len(xs))
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    outs = decode_slots(slots, metas, luts, sizes, stashes, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    for k, (out, w) in enumerate(zip(outs, want)):
        assert np.array_equal(host_bits(out.cpu()), w), k


@pytest.mark.parametrize("make,n", [(W.gaussian_weight, 1_000_003), (W.log_uniform_stress, 77_777),
                                    (W.gaussian_weight, 8 * 32768 * 128)])
def test_decode_straight_from_pinned_host_memory(make, n):
    """The payload stays in pinned host memory and the decode kernel reads it
    over the host link (no copy, no slot): same output as from HBM."""
    x = make(n, seed=1800).reshape(-1)
    xs, ocb, opay, om = oracle_case(x)
    host = torch.empty(len(opay) + 16, dtype=torch.uint8, pin_memory=True)
    host[: len(opay)] = torch.frombuffer(bytearray(opay), dtype=torch.uint8)
    lut = torch.tensor(np.asarray(ocb.dec_lut, np.uint8)).to(DEV)
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    out = S.decode(host[: len(opay)], meta_to_device(om), lut, n, status=st)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    assert np.array_equal(host_bits(out.cpu()), xs)
    with pytest.raises(ValueError):
        S.decode(torch.zeros(len(opay), dtype=torch.uint8), meta_to_device(om), lut, n)


@pytest.mark.parametrize("make,n", [(W.gaussian_weight, 1_000_003), (W.log_uniform_stress, 77_777),
                                    (W.gaussian_weight, 8 * 32768 * 128)])
def test_encode_straight_into_pinned_host_memory(make, n):
    """The kernels write the payload over the host link into pinned host
    memory (an offload without a separate copy): the oracle's bytes."""
    x = make(n, seed=1900).reshape(-1)
    xs, ocb, opay, om = oracle_case(x)
    xd = x.to(DEV)
    ws = workspace(n)
    cb = S.calibrate(xd, ws)
    host = torch.empty(S.payload_size(n, n), dtype=torch.uint8, pin_memory=True)
    payload, meta = S.encode(xd, cb, ws, payload=host)
    torch.cuda.synchronize()
    m = S.read_meta(meta)
    assert m.status == 0 and m.comp_bytes == om.comp_bytes
    assert host[: m.comp_bytes].numpy().tobytes() == opay
    with pytest.raises(ValueError):
        S.encode(xd, cb, ws, payload=torch.empty(16, dtype=torch.uint8))


def test_slot_groups_on_concurrent_streams(form):
    """Two groups of slots decoded at the same time on two streams, with
    plain decodes on a third stream: every output exact.  In the resident
    form each group's grid fills the GPU, so the two contend for it and a
    barrier may give up (the deferral kernel then finishes the slots); in a
    cooperative launch the runtime places each grid whole."""
    g = torch.Generator().manual_seed(13)
    sizes = [int(v) for v in torch.randint(50_000, 3_000_000, (12,), generator=g)]
    cases = []
    for k, n in enumerate(sizes):
        x = W.gaussian_weight(n, seed=900 + k) if k % 4 else W.log_uniform_stress(n, seed=900 + k)
        xs_h, ocb, opay, om = oracle_case(x)
        cases.append((xs_h, ocb, opay, om))
    groups = [cases[0:5], cases[5:10]]
    plain = cases[10:]
    streams = [torch.cuda.Stream() for _ in range(3)]
    st = [torch.zeros(1, dtype=torch.int32, device=DEV) for _ in range(3)]
    results = []
    for rnd in range(3):
        outs = []
        bufs = []
        for gi, grp in enumerate(groups):
            slots = [slot_for(c[2], c[3].n) for c in grp]
            metas = [meta_to_device(c[3], True) for c in grp]
            luts = [torch.tensor(np.asarray(c[1].dec_lut, np.uint8)).to(DEV) for c in grp]
            stashes = [stash_for(c[3].comp_bytes) for c in grp]
            bufs.append((slots, metas, luts, stashes))
        pl = []
        for c in plain:
            pay = torch.frombuffer(bytearray(c[2] + b"\0" * 16), dtype=torch.uint8).to(DEV)
            pl.append((pay, meta_to_device(c[3], True),
                       torch.tensor(np.asarray(c[1].dec_lut, np.uint8)).to(DEV), c[3].n))
        torch.cuda.synchronize()
        _say("concurrent slot groups (%s), round %d" % (form, rnd))
        for gi, (slots, metas, luts, stashes) in enumerate(bufs):
            with torch.cuda.stream(streams[gi]):
                outs.append(decode_slots(slots, metas, luts, [c[3].n for c in groups[gi]], stashes,
                                           status=st[gi], stream=streams[gi]))
        with torch.cuda.stream(streams[2]):
            pouts = [S.decode(p, m, l, n, status=st[2], stream=streams[2]) for p, m, l, n in pl]
        torch.cuda.synchronize()
        assert [int(s.item()) for s in st] == [0, 0, 0]
        for gi, grp in enumerate(groups):
            for out, c in zip(outs[gi], grp):
                assert np.array_equal(host_bits(out.cpu()), c[0])
        for out, c in zip(pouts, plain):
            assert np.array_equal(host_bits(out.cpu()), c[0])


def test_resident_blocks_across_many_streams():
    """The resident form's barrier blocks belong to the streams that used one
    last (64 per device): resident decodes on 70 streams in turn (blocks
    handed from stream to stream), then on 8 streams at once, every slot
    exact."""
    n = 3 * TILE + 4099
    x = W.gaussian_weight(n, seed=950)
    xs_h, ocb, opay, om = oracle_case(x)
    lut = torch.tensor(np.asarray(ocb.dec_lut, np.uint8)).to(DEV)
    meta = meta_to_device(om, True)
    streams = [torch.cuda.Stream() for _ in range(70)]
    _say("resident decodes on 70 streams in turn")
    for k, st in enumerate(streams):
        slot = slot_for(opay, n)
        stash = stash_for(om.comp_bytes)
        torch.cuda.synchronize()
        with torch.cuda.stream(st):
            out = S.decode_slot(slot, meta, lut, n, stash, stream=st, resident=True)
        st.synchronize()
        assert np.array_equal(host_bits(out.cpu()), xs_h), k
    _say("resident decodes on 8 streams at once")
    bufs = [(slot_for(opay, n), stash_for(om.comp_bytes)) for _ in range(8)]
    torch.cuda.synchronize()
    outs = []
    for (slot, stash), st in zip(bufs, streams[:8]):
        with torch.cuda.stream(st):
            outs.append(S.decode_slot(slot, meta, lut, n, stash, stream=st, resident=True))
    torch.cuda.synchronize()
    for k, out in enumerate(outs):
        assert np.array_equal(host_bits(out.cpu()), xs_h), k
