"""Python binding of ``libpda.so``, the MI355X paged-decode attention library.

Every ``pda_*`` function here has the name, argument order and meaning of the
C function declared in ``include/pda.h``; the binding only marshals
arguments (a torch tensor becomes its ``data_ptr()``, a torch stream its
``cuda_stream``; ``None`` as a stream means torch's current stream) and
turns negative return codes into :class:`PdaError`.  All device work runs in
the library's HIP kernels; nothing here computes attention.

``paged_decode`` and :class:`TiledAttention` are small conveniences on top
that take torch tensors and derive the sizes from their shapes.

Importing this module raises ``ImportError`` if ``libpda.so`` has not been
built (``python paged_decode_attention_splitk_amd/_build.py``); there is no
fallback implementation.
"""
from __future__ import annotations

import ctypes
import os

try:
    # torch ships its own copy of the HIP runtime (soname libamdhip64.so.7);
    # loading it first makes libpda.so bind to that same copy, so device
    # pointers and streams from torch are valid in the library's calls.
    import torch  # noqa: F401
except ImportError:  # geometry and validation calls work without torch
    torch = None

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpda.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it with `python paged_decode_attention_splitk_amd/_build.py` "
        "(hipcc, gfx950). There is no CPU fallback.")

_lib = ctypes.CDLL(LIB_PATH)

PDA_OK = 0
PDA_NOT_APPLICABLE = 1
PDA_EINVAL = -22
PDA_ENOMEM = -12
PDA_EHIP_BASE = -1000

PDA_SPLITK_LEGACY = 0
PDA_SPLITK_AUTO = 1
PDA_SPLITK_PINNED = 2

PDA_DECODE_UNPACKED = 0
PDA_DECODE_PACKED = 1
PDA_DECODE_DEFAULT = 2

_u32, _u64, _i32, _i64 = ctypes.c_uint32, ctypes.c_uint64, ctypes.c_int32, ctypes.c_int64
_vp, _f32, _int = ctypes.c_void_p, ctypes.c_float, ctypes.c_int


class pda_splitk_policy(ctypes.Structure):
    _fields_ = [("policy", _i32), ("pin", _u32)]

    def astuple(self):
        return (self.policy, self.pin)


class pda_tiled_dims(ctypes.Structure):
    _fields_ = [("max_seqs", _u32), ("num_q_heads", _u32), ("num_kv_heads", _u32),
                ("head_dim", _u32), ("block_size", _u32), ("tile_capacity", _u32)]


_SIGS = {
    "pda_max_decode_splits": (_u32, []),
    "pda_splitk_target_waves": (_u32, []),
    "pda_gqa_pack_width": (_u32, []),
    "pda_gqa_pack_head_dim": (_u32, []),
    "pda_min_kv_per_split": (_u32, []),
    "pda_max_head_dim": (_u32, []),
    "pda_auto_splits": (_u32, [_u32, _u32]),
    "pda_split_ref_seqs": (_u32, [_u32, _u32]),
    "pda_legacy_splits": (_u32, [_u32, _u32, _u32]),
    "pda_pinned_splits": (_u32, [_u32]),
    "pda_num_splits": (_u32, [_int, _u32, _u32, _u32, _u32, _u32]),
    "pda_workspace_slots": (_u64, [_u64, _u32, _u32, _u32]),
    "pda_gqa_pack_shape_ok": (_int, [_u32, _u32, _u32]),
    "pda_gqa_pack_ctas": (_u64, [_u32, _u32]),
    "pda_split_chunk": (_u32, [_u32, _u32, _u32]),
    "pda_device_cu_count": (_int, [_int, ctypes.POINTER(_u32)]),
    "pda_parse_splitk_policy": (_int, [ctypes.c_char_p, ctypes.POINTER(pda_splitk_policy)]),
    "pda_parse_gqa_pack": (_int, [ctypes.c_char_p, ctypes.POINTER(_int)]),
    "pda_splitk_declared": (ctypes.c_char_p, []),
    "pda_resolve_policy": (None, [ctypes.c_char_p, ctypes.c_char_p,
                                  ctypes.POINTER(pda_splitk_policy)]),
    "pda_policy_from_env": (None, [ctypes.POINTER(pda_splitk_policy)]),
    "pda_decode_gqa_pack_declared": (_int, []),
    "pda_resolve_gqa_pack": (_int, [_int, ctypes.c_char_p]),
    "pda_gqa_pack_enabled": (_int, []),
    "pda_paged_decode": (_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _u64, _u32, _u32, _u32,
                                _u32, _u32, _u32, _u32, _f32, _u32, _u32, _vp]),
    "pda_paged_decode_noalloc": (_int, [_vp, _vp, _vp, _vp, _vp, _vp, _u32, _u32, _u32, _u32,
                                        _u32, _u32, _u32, _f32, _u32, _u32, _vp]),
    "pda_splitk_merge": (_int, [_vp, _u64, _vp, _u32, _u32, _u32, _u32, _vp]),
    "pda_splitk_partials": (_int, [_vp, _vp, _vp, _vp, _vp, _vp, _u64, _u32, _u32, _u32, _u32,
                                   _u32, _u32, _u32, _f32, _u32, _u32, _vp]),
    "pda_paged_decode_fp8": (_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _u64, _u32, _u32, _u32,
                                    _u32, _u32, _u32, _u32, _f32, _f32, _f32, _u32, _u32, _vp]),
    "pda_splitk_partials_fp8": (_int, [_vp, _vp, _vp, _vp, _vp, _vp, _u64, _u32, _u32, _u32,
                                       _u32, _u32, _u32, _u32, _f32, _f32, _f32, _u32, _u32,
                                       _vp]),
    "pda_prefill_applies": (_int, [_u32, _u32, _u32, _int, _u32]),
    "pda_paged_prefill": (_int, [_vp, _vp, _vp, _vp, _vp, _u32, _u32, _u32, _u32, _u32, _u32,
                                 _u32, _u32, _u32, _u32, _f32, _vp]),
    "pda_tiled_validate": (_int, [ctypes.POINTER(pda_tiled_dims)]),
    "pda_tiled_create": (_int, [ctypes.POINTER(pda_tiled_dims), ctypes.POINTER(_vp)]),
    "pda_tiled_destroy": (None, [_vp]),
    "pda_tiled_get_dims": (_int, [_vp, ctypes.POINTER(pda_tiled_dims)]),
    "pda_tiled_state": (_int, [_vp, ctypes.POINTER(_vp), ctypes.POINTER(_vp),
                               ctypes.POINTER(_vp)]),
    "pda_tiled_paged_strides": (None, [ctypes.POINTER(pda_tiled_dims), ctypes.POINTER(_i64)]),
    "pda_tiled_scratch_pool_strides": (None, [ctypes.POINTER(pda_tiled_dims),
                                              ctypes.POINTER(_i64)]),
    "pda_tiled_begin_step": (_int, [_vp, _u32, _vp]),
    "pda_tiled_step_tile": (_int, [_vp, _vp, _vp, _vp, _u64, _vp, _vp, _u32, _i64, _i64, _i64,
                                   _i32, _vp]),
    "pda_tiled_finalize": (_int, [_vp, _vp, _u32, _vp]),
    "pda_last_error": (ctypes.c_char_p, []),
}

for _name, (_res, _args) in _SIGS.items():
    _fn = getattr(_lib, _name)
    _fn.restype = _res
    _fn.argtypes = _args

EXPORTED = tuple(_SIGS)


class PdaError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"pda error {code}: {message}")
        self.code = code


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    dp = getattr(x, "data_ptr", None)
    if dp is not None:
        return dp()
    raise TypeError(f"expected a device pointer (int) or tensor, got {type(x)!r}")


def _stream(s):
    if s is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(s, int):
        return s
    return s.cuda_stream


def _check(rc: int) -> int:
    if rc < 0:
        raise PdaError(rc, pda_last_error())
    return rc


# ---------------------------------------------------------------- constants
def pda_max_decode_splits() -> int: return _lib.pda_max_decode_splits()
def pda_splitk_target_waves() -> int: return _lib.pda_splitk_target_waves()
def pda_gqa_pack_width() -> int: return _lib.pda_gqa_pack_width()
def pda_gqa_pack_head_dim() -> int: return _lib.pda_gqa_pack_head_dim()
def pda_min_kv_per_split() -> int: return _lib.pda_min_kv_per_split()
def pda_max_head_dim() -> int: return _lib.pda_max_head_dim()


# ---------------------------------------------------------------- geometry
def pda_auto_splits(cu_count, num_q_heads): return _lib.pda_auto_splits(cu_count, num_q_heads)
def pda_split_ref_seqs(num_seqs, max_decode_seqs):
    return _lib.pda_split_ref_seqs(num_seqs, max_decode_seqs)
def pda_legacy_splits(cu_count, num_q_heads, ref_seqs):
    return _lib.pda_legacy_splits(cu_count, num_q_heads, ref_seqs)
def pda_pinned_splits(pin): return _lib.pda_pinned_splits(pin)
def pda_num_splits(policy, pin, cu_count, num_q_heads, num_seqs, max_decode_seqs):
    return _lib.pda_num_splits(policy, pin, cu_count, num_q_heads, num_seqs, max_decode_seqs)
def pda_workspace_slots(rows, num_q_heads, num_splits, head_dim):
    return _lib.pda_workspace_slots(rows, num_q_heads, num_splits, head_dim)
def pda_gqa_pack_shape_ok(num_q_heads, num_kv_heads, head_dim):
    return bool(_lib.pda_gqa_pack_shape_ok(num_q_heads, num_kv_heads, head_dim))
def pda_gqa_pack_ctas(num_kv_heads, num_seqs): return _lib.pda_gqa_pack_ctas(num_kv_heads, num_seqs)
def pda_split_chunk(seq_len, num_splits, block_size):
    return _lib.pda_split_chunk(seq_len, num_splits, block_size)


def pda_device_cu_count(device: int = 0) -> int:
    n = _u32(0)
    _check(_lib.pda_device_cu_count(device, ctypes.byref(n)))
    return n.value


# ---------------------------------------------------------------- policy
def _cstr(x):
    if x is None:
        return None
    return x.encode() if isinstance(x, str) else bytes(x)


def pda_parse_splitk_policy(s):
    """(policy, pin) for a parseable string, else None."""
    p = pda_splitk_policy()
    return p.astuple() if _lib.pda_parse_splitk_policy(_cstr(s), ctypes.byref(p)) else None


def pda_parse_gqa_pack(s):
    """True / False for a parseable string, else None."""
    on = _int(0)
    return bool(on.value) if _lib.pda_parse_gqa_pack(_cstr(s), ctypes.byref(on)) else None


def pda_splitk_declared() -> str: return _lib.pda_splitk_declared().decode()


def pda_resolve_policy(declared, env_value):
    p = pda_splitk_policy()
    _lib.pda_resolve_policy(_cstr(declared), _cstr(env_value), ctypes.byref(p))
    return p.astuple()


def pda_policy_from_env():
    p = pda_splitk_policy()
    _lib.pda_policy_from_env(ctypes.byref(p))
    return p.astuple()


def pda_decode_gqa_pack_declared() -> bool: return bool(_lib.pda_decode_gqa_pack_declared())
def pda_resolve_gqa_pack(declared, env_value) -> bool:
    return bool(_lib.pda_resolve_gqa_pack(int(bool(declared)), _cstr(env_value)))
def pda_gqa_pack_enabled() -> bool: return bool(_lib.pda_gqa_pack_enabled())


def pda_last_error() -> str:
    return (_lib.pda_last_error() or b"").decode()


# ---------------------------------------------------------------- one-shot
def pda_paged_decode(q, k_cache, v_cache, block_tables, seq_lens, out, workspace,
                     workspace_floats, num_seqs, num_q_heads, num_kv_heads, head_dim,
                     block_size, max_blocks_per_seq, num_blocks, scale, num_splits,
                     flags=PDA_DECODE_UNPACKED, stream=None) -> int:
    return _check(_lib.pda_paged_decode(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), _ptr(seq_lens), _ptr(out),
        _ptr(workspace), workspace_floats, num_seqs, num_q_heads, num_kv_heads, head_dim,
        block_size, max_blocks_per_seq, num_blocks, scale, num_splits, flags, _stream(stream)))


def pda_paged_decode_noalloc(q, k_cache, v_cache, block_tables, seq_lens, out, num_seqs,
                             num_q_heads, num_kv_heads, head_dim, block_size,
                             max_blocks_per_seq, num_blocks, scale, num_splits,
                             flags=PDA_DECODE_UNPACKED, stream=None) -> int:
    return _check(_lib.pda_paged_decode_noalloc(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), _ptr(seq_lens), _ptr(out),
        num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
        num_blocks, scale, num_splits, flags, _stream(stream)))


def pda_splitk_merge(workspace, workspace_floats, out, num_seqs, num_q_heads, head_dim,
                     num_splits, stream=None) -> int:
    return _check(_lib.pda_splitk_merge(_ptr(workspace), workspace_floats, _ptr(out), num_seqs,
                                        num_q_heads, head_dim, num_splits, _stream(stream)))


def pda_splitk_partials(q, k_cache, v_cache, block_tables, seq_lens, workspace,
                        workspace_floats, num_seqs, num_q_heads, num_kv_heads, head_dim,
                        block_size, max_blocks_per_seq, num_blocks, scale, num_splits,
                        flags=PDA_DECODE_UNPACKED, stream=None) -> int:
    return _check(_lib.pda_splitk_partials(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), _ptr(seq_lens),
        _ptr(workspace), workspace_floats, num_seqs, num_q_heads, num_kv_heads, head_dim,
        block_size, max_blocks_per_seq, num_blocks, scale, num_splits, flags, _stream(stream)))


# ---------------------------------------------------------------- FP8 cache
def pda_paged_decode_fp8(q, k_cache, v_cache, block_tables, seq_lens, out, workspace,
                         workspace_floats, num_seqs, num_q_heads, num_kv_heads, head_dim,
                         block_size, max_blocks_per_seq, num_blocks, scale, k_scale, v_scale,
                         num_splits, flags=PDA_DECODE_UNPACKED, stream=None) -> int:
    return _check(_lib.pda_paged_decode_fp8(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), _ptr(seq_lens), _ptr(out),
        _ptr(workspace), workspace_floats, num_seqs, num_q_heads, num_kv_heads, head_dim,
        block_size, max_blocks_per_seq, num_blocks, scale, k_scale, v_scale, num_splits, flags,
        _stream(stream)))


def pda_splitk_partials_fp8(q, k_cache, v_cache, block_tables, seq_lens, workspace,
                            workspace_floats, num_seqs, num_q_heads, num_kv_heads, head_dim,
                            block_size, max_blocks_per_seq, num_blocks, scale, k_scale, v_scale,
                            num_splits, flags=PDA_DECODE_UNPACKED, stream=None) -> int:
    return _check(_lib.pda_splitk_partials_fp8(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables), _ptr(seq_lens),
        _ptr(workspace), workspace_floats, num_seqs, num_q_heads, num_kv_heads, head_dim,
        block_size, max_blocks_per_seq, num_blocks, scale, k_scale, v_scale, num_splits, flags,
        _stream(stream)))


# ---------------------------------------------------------------- prefill
def pda_prefill_applies(num_q_heads, num_kv_heads, head_dim, causal=True, sliding_window=0):
    return bool(_lib.pda_prefill_applies(num_q_heads, num_kv_heads, head_dim, int(bool(causal)),
                                         sliding_window))


def pda_paged_prefill(q, k_cache, v_cache, out, block_table, q_len, kv_len, q_offset,
                      num_q_heads, num_kv_heads, head_dim, block_size, max_blocks, num_blocks,
                      scale, sliding_window=0, stream=None) -> int:
    return _check(_lib.pda_paged_prefill(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(out), _ptr(block_table), q_len, kv_len,
        q_offset, num_q_heads, num_kv_heads, head_dim, block_size, max_blocks, num_blocks,
        sliding_window, scale, _stream(stream)))


# ---------------------------------------------------------------- tiled
def _dims(d) -> pda_tiled_dims:
    if isinstance(d, pda_tiled_dims):
        return d
    return pda_tiled_dims(*d)


def pda_tiled_validate(dims) -> int:
    return _check(_lib.pda_tiled_validate(ctypes.byref(_dims(dims))))


def pda_tiled_create(dims) -> int:
    h = _vp(0)
    _check(_lib.pda_tiled_create(ctypes.byref(_dims(dims)), ctypes.byref(h)))
    return h.value


def pda_tiled_destroy(handle) -> None:
    _lib.pda_tiled_destroy(handle)


def pda_tiled_get_dims(handle) -> pda_tiled_dims:
    d = pda_tiled_dims()
    _check(_lib.pda_tiled_get_dims(handle, ctypes.byref(d)))
    return d


def pda_tiled_state(handle):
    m, l, o = _vp(0), _vp(0), _vp(0)
    _check(_lib.pda_tiled_state(handle, ctypes.byref(m), ctypes.byref(l), ctypes.byref(o)))
    return m.value, l.value, o.value


def pda_tiled_paged_strides(dims):
    out = (_i64 * 3)()
    _lib.pda_tiled_paged_strides(ctypes.byref(_dims(dims)), out)
    return tuple(out)


def pda_tiled_scratch_pool_strides(dims):
    out = (_i64 * 3)()
    _lib.pda_tiled_scratch_pool_strides(ctypes.byref(_dims(dims)), out)
    return tuple(out)


def pda_tiled_begin_step(handle, num_seqs, stream=None) -> int:
    return _check(_lib.pda_tiled_begin_step(handle, num_seqs, _stream(stream)))


def pda_tiled_step_tile(handle, q, k_pool, v_pool, pool_blocks, tile_blocks, tile_block_counts,
                        num_seqs, blk_stride, tok_stride, kvh_stride, last_block_valid_slots,
                        stream=None) -> int:
    return _check(_lib.pda_tiled_step_tile(
        handle, _ptr(q), _ptr(k_pool), _ptr(v_pool), pool_blocks, _ptr(tile_blocks),
        _ptr(tile_block_counts), num_seqs, blk_stride, tok_stride, kvh_stride,
        last_block_valid_slots, _stream(stream)))


def pda_tiled_finalize(handle, out, num_seqs, stream=None) -> int:
    return _check(_lib.pda_tiled_finalize(handle, _ptr(out), num_seqs, _stream(stream)))


# ---------------------------------------------------------------- conveniences
def paged_decode(q, k_cache, v_cache, block_tables, seq_lens, scale, num_splits,
                 out=None, workspace=None, packed=False, stream=None):
    """One-shot decode on torch tensors (q: bf16 [S, nq, D]; caches: bf16
    [num_blocks, block_size, nkv, D]; block_tables, seq_lens: int32).
    Allocates ``out`` and the workspace with torch if not given."""
    import torch
    S, nq, D = q.shape
    nb, bs, nkv, D2 = k_cache.shape
    assert D2 == D and v_cache.shape == k_cache.shape
    if out is None:
        out = torch.empty((S, nq, D), dtype=torch.bfloat16, device=q.device)
    wsf = pda_workspace_slots(S, nq, num_splits, D) if num_splits > 1 else 0
    if workspace is None and wsf:
        workspace = torch.empty(wsf, dtype=torch.float32, device=q.device)
    rc = pda_paged_decode(q, k_cache, v_cache, block_tables, seq_lens, out, workspace,
                          workspace.numel() if workspace is not None else 0, S, nq, nkv, D, bs,
                          block_tables.shape[1], nb, scale, num_splits,
                          PDA_DECODE_PACKED if packed else PDA_DECODE_UNPACKED, stream)
    if rc == PDA_NOT_APPLICABLE:
        raise PdaError(rc, pda_last_error())
    return out


class TiledAttention:
    """Owning wrapper of a ``pda_tiled`` handle (allocated on torch's current device)."""

    def __init__(self, max_seqs, num_q_heads, num_kv_heads, head_dim, block_size, tile_capacity):
        self.dims = pda_tiled_dims(max_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                                   tile_capacity)
        self.handle = pda_tiled_create(self.dims)

    def close(self):
        if self.handle:
            pda_tiled_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def state(self):
        return pda_tiled_state(self.handle)

    def paged_strides(self):
        return pda_tiled_paged_strides(self.dims)

    def scratch_pool_strides(self):
        return pda_tiled_scratch_pool_strides(self.dims)

    def begin_step(self, num_seqs, stream=None):
        pda_tiled_begin_step(self.handle, num_seqs, stream)

    def step_tile(self, q, k_pool, v_pool, pool_blocks, tile_blocks, tile_block_counts,
                  num_seqs, strides, last_block_valid_slots, stream=None):
        pda_tiled_step_tile(self.handle, q, k_pool, v_pool, pool_blocks, tile_blocks,
                            tile_block_counts, num_seqs, strides[0], strides[1], strides[2],
                            last_block_valid_slots, stream)

    def finalize(self, out, num_seqs, stream=None):
        pda_tiled_finalize(self.handle, out, num_seqs, stream)
