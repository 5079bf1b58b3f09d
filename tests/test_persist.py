"""Codebook / metadata JSON in the pages' key format and the coverage gate
(host-side helpers; no GPU)."""
import base64
import json

import numpy as np

import lossless_bf16_tensor_splitzip_amd as S
from lossless_bf16_tensor_splitzip_amd import persist
import oracle
import workloads as W


def oracle_codebook(x):
    ocb = oracle.calibrate(x)
    cb = S.Codebook()
    for name in ("enc_lut", "enc_lut_marked", "dec_lut", "common_lut"):
        arr = getattr(cb, name)
        for k, v in enumerate(getattr(ocb, name)):
            arr[k] = int(v)
    cb.n_codes, cb.covered, cb.total = ocb.n_codes, ocb.covered, ocb.total
    for k, c in enumerate(ocb.counts):
        cb.counts[k] = int(c)
    return ocb, cb


def test_codebook_json_round_trip_and_page_keys():
    x = W.bits(W.log_uniform_stress(50_000, seed=80)).numpy().view(np.uint16)
    ocb, cb = oracle_codebook(x)
    d = json.loads(json.dumps(persist.codebook_to_json(cb)))
    # the keys of the page's SplitZipCodebook.to_json, tables as base64 bytes
    for name in ("coverage", "enc_lut", "enc_lut_marked", "dec_lut", "common_lut"):
        assert name in d
    assert base64.b64decode(d["dec_lut"]) == ocb.dec_lut.tobytes()
    assert base64.b64decode(d["enc_lut_marked"]) == ocb.enc_lut_marked.tobytes()
    assert abs(d["coverage"] - ocb.covered / ocb.total) < 1e-15
    back = persist.codebook_from_json(d)
    assert bytes(back) == bytes(cb)


def test_codebook_from_page_only_keys():
    x = W.bits(W.gaussian_weight(20_001, seed=81)).numpy().view(np.uint16)
    ocb, cb = oracle_codebook(x)
    d = persist.codebook_to_json(cb)
    page_form = {k: d[k] for k in ("coverage", "enc_lut", "enc_lut_marked", "dec_lut", "common_lut")}
    back = persist.codebook_from_json(page_form)
    assert bytes(back.dec_lut) == ocb.dec_lut.tobytes()
    assert bytes(back.enc_lut_marked) == ocb.enc_lut_marked.tobytes()
    assert back.n_codes == ocb.n_codes


def test_meta_json_round_trip():
    x = W.bits(W.log_uniform_stress(9_999, seed=82)).numpy().view(np.uint16)
    ocb = oracle.calibrate(x)
    _, om = oracle.encode(x, ocb)
    m = S.Meta()
    m.n, m.n_pairs, m.chunk_size, m.n_esc, m.comp_bytes = om.n, om.n_pairs, 1024, om.n_esc, om.comp_bytes
    for k in range(5):
        m.offsets[k] = om.offsets[k]
    m.covered, m.total = ocb.covered, ocb.total
    d = json.loads(json.dumps(persist.meta_to_json(m)))
    for key in ("n", "n_pairs", "chunk_size", "n_esc", "comp_bytes", "offsets", "coverage"):
        assert key in d
    assert d["offsets"] == list(om.offsets)
    assert bytes(persist.meta_from_json(d)) == bytes(m)


def test_coverage_gate():
    cb = S.Codebook()
    cb.total = 1000
    for covered, expect in ((989, False), (990, True), (1000, True)):
        cb.covered = covered
        assert persist.passes_coverage_gate(cb) is expect
    cb.total = cb.covered = 0
    assert persist.coverage(cb) == 1.0 and persist.passes_coverage_gate(cb)
    # weight-like data passes; broad exponent distributions do not
    _, good = oracle_codebook(W.bits(W.gaussian_weight(100_000, seed=83)).numpy().view(np.uint16))
    _, bad = oracle_codebook(W.bits(W.log_uniform_stress(100_000, seed=84)).numpy().view(np.uint16))
    assert persist.passes_coverage_gate(good) and not persist.passes_coverage_gate(bad)


def test_manifest_entry_format():
    x = W.bits(W.gaussian_weight(4097, seed=85)).numpy().view(np.uint16)
    ocb, cb = oracle_codebook(x)
    _, om = oracle.encode(x, ocb)
    m = S.Meta()
    m.n, m.n_pairs, m.chunk_size, m.n_esc, m.comp_bytes = om.n, om.n_pairs, 1024, om.n_esc, om.comp_bytes
    for k in range(5):
        m.offsets[k] = om.offsets[k]
    e = json.loads(json.dumps(persist.manifest_entry("w", (17, 241), cb, m)))
    assert e["raw"] is False and e["shape"] == [17, 241] and e["dtype"] == "bfloat16"
    assert base64.b64decode(e["codebook"]["dec_lut"]) == ocb.dec_lut.tobytes()
    assert e["meta"]["comp_bytes"] == om.comp_bytes
    r = persist.manifest_entry("w", (3,), None, None)
    assert r["raw"] is True and "codebook" not in r


def test_codebook_json_rejects_marked_values_above_16():
    x = W.bits(W.gaussian_weight(5_001, seed=85)).numpy().view(np.uint16)
    _, cb = oracle_codebook(x)
    d = persist.codebook_to_json(cb)
    raw = bytearray(base64.b64decode(d["enc_lut_marked"]))
    raw[7] = 17
    d["enc_lut_marked"] = base64.b64encode(bytes(raw)).decode()
    try:
        persist.codebook_from_json(d)
    except ValueError:
        pass
    else:
        raise AssertionError("a marked table with 17 was accepted")


def test_meta_json_ascending_flag():
    m = S.Meta()
    m.n, m.n_pairs, m.chunk_size = 10, 5, 1024
    m.flags = 1
    d = json.loads(json.dumps(persist.meta_to_json(m)))
    assert d["ascending"] is True
    assert persist.meta_from_json(d).flags == 1
    # the pages' PayloadMeta keys say nothing about the order: flag clear
    page = {k: d[k] for k in ("n", "n_pairs", "chunk_size", "n_esc", "comp_bytes", "offsets",
                              "coverage")}
    assert persist.meta_from_json(page).flags == 0
