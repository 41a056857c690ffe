"""Pins of oracle.policy against the statements of the "Module attn_splitk"
page (items parse, parse_gqa_pack, resolve_policy, resolve_gqa_pack,
DECODE_GQA_PACK_DECLARED, and the module's invariants)."""
import pytest

from oracle import geometry as g
from oracle import policy as pol

L0, A0 = (g.LEGACY, 0), (g.AUTO, 0)


@pytest.mark.parametrize("text,want", [
    # the four forms parse lists: legacy | auto | 0/off/false/no | a count
    ("legacy", L0), ("auto", A0),
    ("0", (g.PINNED, 1)), ("off", (g.PINNED, 1)), ("false", (g.PINNED, 1)), ("no", (g.PINNED, 1)),
    ("1", (g.PINNED, 1)), ("5", (g.PINNED, 5)), ("16", (g.PINNED, 16)),
    # "clamped to 1..=MAX_DECODE_SPLITS"
    ("17", (g.PINNED, 16)), ("264", (g.PINNED, 16)), ("0000", (g.PINNED, 1)),
    # "trimmed and case-insensitive"
    ("  AUTO ", A0), ("\tLegacy\n", L0), (" Off", (g.PINNED, 1)), ("NO", (g.PINNED, 1)),
    (" 12 ", (g.PINNED, 12)),
    # none of the forms
    ("", None), ("   ", None), ("automatic", None), ("-3", None), ("3.5", None),
    ("yes", None), ("on", None), ("1 2", None),
])
def test_parse(text, want):
    assert pol.parse(text) == want


@pytest.mark.parametrize("text,want", [
    ("1", True), ("on", True), ("true", True), ("yes", True),
    ("0", False), ("off", False), ("false", False), ("no", False),
    (" YES\t", True), ("Off ", False),
    ("", None), ("2", None), ("enable", None), ("auto", None),
])
def test_parse_gqa_pack(text, want):
    assert pol.parse_gqa_pack(text) == want


def test_resolve_policy():
    # the declaration, overridden by a parseable environment value
    assert pol.resolve_policy("auto", None) == A0
    assert pol.resolve_policy("auto", "legacy") == L0
    assert pol.resolve_policy("legacy", "4") == (g.PINNED, 4)
    assert pol.resolve_policy("auto", "bogus") == A0        # unparseable env: ignored
    # an unparseable declaration is Legacy
    assert pol.resolve_policy("bogus", None) == L0
    assert pol.resolve_policy("bogus", "bogus") == L0
    assert pol.resolve_policy("bogus", "auto") == A0


def test_resolve_gqa_pack():
    assert pol.DECODE_GQA_PACK_DECLARED is False            # "off, for every target"
    assert pol.resolve_gqa_pack(False, None) is False
    assert pol.resolve_gqa_pack(False, "on") is True
    assert pol.resolve_gqa_pack(True, "0") is False
    assert pol.resolve_gqa_pack(True, "maybe") is True       # unparseable: declared stands


def test_only_legacy_reads_the_batch():
    """Module invariant: under Auto and Pinned the split count depends only on
    (sm_count, num_q_heads) and the pin; only Legacy reads the batch."""
    for text in ("auto", "3", "off"):
        code, pin = pol.parse(text)
        counts = {g.num_splits(code, pin, 256, 32, s, 8) for s in (1, 8, 64, 512)}
        assert len(counts) == 1
    code, pin = pol.parse("legacy")
    counts = {g.num_splits(code, pin, 256, 8, s, 4) for s in (1, 8, 64, 512)}
    assert len(counts) > 1
