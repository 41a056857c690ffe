"""FP64 CPU oracle for paged-decode attention with split-K.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import or call anything in this package.  The HIP library never routes
through it, and this package imports nothing from the HIP library or its
Python binding: the two share no code.  Inputs reach both from the seeded
generators in ``workloads`` (which hold no attention arithmetic).

Contents
--------
``oracle.attention``  plain softmax attention in FP64 over tokens gathered
                      through the block table (one-shot decode, per-split
                      partials, tiled running state).
``oracle.geometry``   the launch-geometry formulas of the attn_splitk module
                      page, written out in Python integers.
``oracle.prefill``    causal paged prefill (the prefill page's kernel), FP64.
``oracle.fp8``        paged decode over an FP8 (OCP E4M3) cache with per-tensor
                      scales, FP64 (scale semantics: parity unpinned).
``oracle.policy``     that page's policy grammar and resolution rules
                      (parse, parse_gqa_pack, resolve_policy,
                      resolve_gqa_pack).

Pins (what each function is checked against, in ``tests/test_oracle_*.py``):
brute-force pure-Python loops on tiny inputs, torch's FP64
scaled_dot_product_attention on the CPU, closed forms (one token, two
tokens, q = 0, equal keys, empty sequence), invariances (block-table
permutation with a matching pool relayout, merge of per-split partials), and
the worked numbers printed on the attn_splitk module page.

Parity unpinned: the FP8 scale semantics (``oracle.fp8``; the pages name FP8
launches but print no format or scaling), the split partition rule (``geometry.split_chunk``) and the
value of the per-split floor, and the reading of the tiled call's
``last_block_valid_slots``, have no value printed on the pages; they are
checked only for self-consistency (partials merge to the one-pass result;
tiles fold to the whole-sequence state).
"""
