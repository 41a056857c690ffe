"""Split-count policy and packed-kernel switch resolution, in plain Python.

Test infrastructure (see ``oracle/__init__.py``).  Written from the
"Module attn_splitk" page, items parse, parse_gqa_pack, resolve_policy,
resolve_gqa_pack, policy_from_env, gqa_pack_enabled and
DECODE_GQA_PACK_DECLARED; nothing here is shared with the HIP library's C++.

A policy is returned as a (code, pin) pair: (LEGACY, 0), (AUTO, 0) or
(PINNED, n).  Readings where the page is silent:
  * "trimmed and case-insensitive" is taken over ASCII: the characters
    space, tab, newline, carriage return, vertical tab and form feed are
    trimmed, and only A-Z fold to a-z;
  * "a decimal count" is one or more ASCII digits, no sign; a count is
    clamped to 1..MAX_DECODE_SPLITS whatever its size;
  * "0/off/false/no" disables split-K, i.e. Pinned 1 (the count 0 clamps to
    the same value).
"""
from __future__ import annotations

from .geometry import AUTO, LEGACY, MAX_DECODE_SPLITS, PINNED

DECODE_GQA_PACK_DECLARED = False        # attn_splitk page: "off, for every target"
SPLITK_ENV = "METRALE_ATTN_DECODE_SPLITK"
GQA_PACK_ENV = "METRALE_ATTN_DECODE_GQA_PACK"

_ASCII_SPACE = " \t\n\r\x0b\x0c"
_OFF_WORDS = ("0", "off", "false", "no")
_ON_WORDS = ("1", "on", "true", "yes")


def _norm(s: str) -> str:
    t = s.strip(_ASCII_SPACE)
    return "".join(chr(ord(c) + 32) if "A" <= c <= "Z" else c for c in t)


def parse(s):
    """legacy | auto | 0/off/false/no | a decimal count (clamped to
    1..=MAX_DECODE_SPLITS); None when the text is none of these."""
    if s is None:
        return None
    t = _norm(s)
    if t == "legacy":
        return (LEGACY, 0)
    if t == "auto":
        return (AUTO, 0)
    if t in _OFF_WORDS:
        return (PINNED, 1)
    if t and all("0" <= c <= "9" for c in t):
        return (PINNED, max(1, min(MAX_DECODE_SPLITS, int(t))))
    return None


def parse_gqa_pack(s):
    """1/on/true/yes -> True, 0/off/false/no -> False, else None."""
    if s is None:
        return None
    t = _norm(s)
    if t in _ON_WORDS:
        return True
    if t in _OFF_WORDS:
        return False
    return None


def resolve_policy(declared, env_value):
    """The declaration, overridden by a parseable environment value; an
    unparseable declaration is Legacy."""
    from_env = parse(env_value)
    if from_env is not None:
        return from_env
    from_decl = parse(declared)
    return from_decl if from_decl is not None else (LEGACY, 0)


def resolve_gqa_pack(declared: bool, env_value) -> bool:
    """The declared state, overridden by a parseable environment value."""
    v = parse_gqa_pack(env_value)
    return bool(declared) if v is None else v
