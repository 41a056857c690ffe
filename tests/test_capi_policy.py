"""The C ABI's policy resolution (pda_parse_splitk_policy, pda_parse_gqa_pack,
pda_resolve_policy, pda_policy_from_env, pda_resolve_gqa_pack,
pda_gqa_pack_enabled) against oracle.policy.  Host only; no GPU."""
import itertools
import os
import subprocess
import sys

import pytest

import paged_decode_attention_splitk_amd as P
from oracle import policy as pol

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _corpus():
    words = ["legacy", "auto", "0", "off", "false", "no", "1", "on", "true", "yes", "3", "16",
             "17", "264", "4294967296", "99999999999999999999999", "", "-1", "+2", "2.0",
             "autox", "legac", "o ff", "0x10"]
    out = set()
    for w in words:
        for case in (str.lower, str.upper, str.title):
            for pad in ("", " ", "\t", "\n ", " \r\x0b\x0c"):
                out.add(pad + case(w) + pad[::-1])
    out.update([" auto", "auto ", "ａｕｔｏ", "1\x00"[:1]])
    return sorted(out)


@pytest.mark.parametrize("text", _corpus())
def test_parse_matches_oracle(text):
    assert P.pda_parse_splitk_policy(text) == pol.parse(text)
    assert P.pda_parse_gqa_pack(text) == pol.parse_gqa_pack(text)


def test_parse_null():
    assert P.pda_parse_splitk_policy(None) is None
    assert P.pda_parse_gqa_pack(None) is None


def test_resolution_matches_oracle():
    vals = [None, "auto", "legacy", "7", "off", "bogus", " ON ", "0"]
    for decl, env in itertools.product(vals, vals):
        assert P.pda_resolve_policy(decl, env) == pol.resolve_policy(decl, env), (decl, env)
    for decl, env in itertools.product([False, True], vals):
        assert P.pda_resolve_gqa_pack(decl, env) == pol.resolve_gqa_pack(decl, env), (decl, env)
    assert P.pda_splitk_declared() == "auto"
    assert P.pda_decode_gqa_pack_declared() is pol.DECODE_GQA_PACK_DECLARED


_CHILD = r"""
import os, sys
sys.path.insert(0, sys.argv[1])
import paged_decode_attention_splitk_amd as P
from oracle import policy as pol
first = P.pda_gqa_pack_enabled()
want = pol.resolve_gqa_pack(pol.DECODE_GQA_PACK_DECLARED, os.environ.get(pol.GQA_PACK_ENV))
assert first == want, (first, want)
# resolved once: later environment changes do not move it
os.environ[pol.GQA_PACK_ENV] = "off" if first else "on"
assert P.pda_gqa_pack_enabled() == first
# the split policy reads the environment on every call
for v in (None, "legacy", "5", "junk", "auto"):
    if v is None:
        os.environ.pop(pol.SPLITK_ENV, None)
    else:
        os.environ[pol.SPLITK_ENV] = v
    got = P.pda_policy_from_env()
    assert got == pol.resolve_policy(P.pda_splitk_declared(), v), (v, got)
print("child ok", first)
"""


@pytest.mark.parametrize("pack_env", [None, "on", " TRUE ", "off", "garbage"])
def test_environment_resolution_in_a_fresh_process(pack_env):
    env = {k: v for k, v in os.environ.items()
           if k not in (pol.GQA_PACK_ENV, pol.SPLITK_ENV)}
    if pack_env is not None:
        env[pol.GQA_PACK_ENV] = pack_env
    r = subprocess.run([sys.executable, "-c", _CHILD, ROOT], env=env, capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    expect = pol.resolve_gqa_pack(False, pack_env)
    assert r.stdout.strip().endswith(str(expect))
