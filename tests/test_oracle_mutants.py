"""Mutation check of the oracle's pins: each plausible mistake below is planted
in a private copy of the oracle's C source (on the CPU, in a temporary
directory), and at least one pin must catch it.  The mutants cover a dropped
term, a wrong sign or shift, swapped operands, a reversed order and a broken
alignment rule."""
import os
import subprocess

import pytest

import oracle
import oracle_pins as P

SRC = os.path.join(os.path.dirname(oracle.__file__), "splitzip_oracle.c")

MUTANTS = {
    # nibble order swapped in both directions (round trip still holds)
    "low_nibble_first": [
        ("pk[i / 2] = (uint8_t)(nibble << 4); /* reading R4: even -> high */",
         "pk[i / 2] = (uint8_t)(nibble);"),
        ("pk[i / 2] = (uint8_t)(pk[i / 2] | nibble);",
         "pk[i / 2] = (uint8_t)(pk[i / 2] | (nibble << 4));"),
        ("(i % 2 == 0) ? (unsigned)(pk[i / 2] >> 4) : (unsigned)(pk[i / 2] & 0xFu)",
         "(i % 2 == 0) ? (unsigned)(pk[i / 2] & 0xFu) : (unsigned)(pk[i / 2] >> 4)"),
    ],
    "ties_by_larger_value": [
        ("if (a->value != b->value) return a->value < b->value ? -1 : 1;",
         "if (a->value != b->value) return a->value > b->value ? -1 : 1;"),
    ],
    "least_frequent_first": [
        ("if (a->count != b->count) return a->count > b->count ? -1 : 1;",
         "if (a->count != b->count) return a->count < b->count ? -1 : 1;"),
    ],
    "fifteen_codes": [
        ("int top = distinct < 16 ? distinct : 16;", "int top = distinct < 15 ? distinct : 15;"),
    ],
    "covered_counts_codes": [("cov += bins[code].count;", "cov += 1;")],
    "big_endian_chunk_id": [
        ("p[0] = (uint8_t)(v & 0xFFu);\n    p[1] = (uint8_t)((v >> 8) & 0xFFu);\n"
         "    p[2] = (uint8_t)((v >> 16) & 0xFFu);\n    p[3] = (uint8_t)((v >> 24) & 0xFFu);",
         "p[3] = (uint8_t)(v & 0xFFu);\n    p[2] = (uint8_t)((v >> 8) & 0xFFu);\n"
         "    p[1] = (uint8_t)((v >> 16) & 0xFFu);\n    p[0] = (uint8_t)((v >> 24) & 0xFFu);"),
        ("return (uint32_t)p[0] | ((uint32_t)p[1] << 8) | ((uint32_t)p[2] << 16) |\n"
         "           ((uint32_t)p[3] << 24);",
         "return (uint32_t)p[3] | ((uint32_t)p[2] << 8) | ((uint32_t)p[1] << 16) |\n"
         "           ((uint32_t)p[0] << 24);"),
    ],
    "chunk_and_position_transposed": [
        ("put_le32(buf + off[2] + 4 * r, (uint32_t)(i / chunk));\n"
         "        put_le16(buf + off[3] + 2 * r, (uint32_t)(i % chunk));",
         "put_le32(buf + off[2] + 4 * r, (uint32_t)(i % chunk));\n"
         "        put_le16(buf + off[3] + 2 * r, (uint32_t)(i / chunk));"),
        ("uint64_t idx = (uint64_t)cid * chunk + pos;", "uint64_t idx = (uint64_t)pos * chunk + (uint64_t)cid;"),
    ],
    "escapes_descending": [
        ("uint64_t i = esc_idx[r];", "uint64_t i = esc_idx[n_esc - 1 - r];"),
    ],
    "escape_writes_code_15": [
        ("unsigned nibble = m & 0xFu;", "unsigned nibble = m > 15 ? 15u : m;"),
    ],
    "sign_dropped": [
        ("return (unsigned)(((bits >> 8) & 0x80u) | (bits & 0x7Fu));",
         "return (unsigned)(bits & 0x7Fu);"),
    ],
    "exponent_top_bit_dropped": [
        ("return (unsigned)((bits >> 7) & 0xFFu);", "return (unsigned)((bits >> 7) & 0x7Fu);"),
    ],
    "align_to_8": [
        ("return (v + 3u) & ~(uint64_t)3u;", "return (v + 7u) & ~(uint64_t)7u;"),
    ],
    "esc_val_not_aligned": [
        ("off[4] = round_up4(off[3] + 2 * n_esc);", "off[4] = off[3] + 2 * n_esc;"),
    ],
    "escape_patch_dropped": [
        ("out[idx] = rebuild(sm[idx], ex);", "(void)ex;"),
    ],
    "escape_uses_wrong_sm": [
        ("out[idx] = rebuild(sm[idx], ex);", "out[idx] = rebuild(sm[r], ex);"),
    ],
}


def _build_mutant(tmp_path, name, edits):
    src = open(SRC).read()
    for old, new in edits:
        assert src.count(old) == 1, (name, old)  # the oracle source moved: update the mutant
        src = src.replace(old, new)
    cpath = tmp_path / (name + ".c")
    cpath.write_text(src)
    so = tmp_path / ("lib" + name + ".so")
    subprocess.run(["gcc", "-O1", "-std=c11", "-fPIC", "-shared", str(cpath), "-o", str(so)],
                   check=True, capture_output=True)
    return oracle.OracleLib(str(so))


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(tmp_path, name):
    o = _build_mutant(tmp_path, name, MUTANTS[name])
    caught = []
    for pin in P.ALL_PINS:
        try:
            if pin is P.pin_bruteforce_alphabet:
                pin(o, max_full_n=2, sampled=((4, 200),))
            else:
                pin(o)
        except Exception as exc:  # AssertionError or a rejected payload
            caught.append((pin.__name__, type(exc).__name__))
    assert caught, "mutant %s passed every pin" % name
