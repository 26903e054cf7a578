"""The C-ABI library loads, exports every declared symbol, and validates on the host.

CPU only: nothing here launches a kernel.  Configuration and argument checks
run before any HIP call, so they are exercised without a GPU.
"""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "memory_bound_transformer_decode_amd", "libdec.so")

pytestmark = pytest.mark.skipif(not os.path.exists(LIB), reason="libdec.so not built")


def declared_functions():
    names = set()
    for f in os.listdir(os.path.join(ROOT, "include")):
        if f.endswith(".h"):
            src = open(os.path.join(ROOT, "include", f)).read()
            src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
            names |= set(re.findall(r"\b(dec_[a-z_0-9]+)\s*\(", src))
    return sorted(names)


def test_every_declared_symbol_is_exported():
    from memory_bound_transformer_decode_amd import dec
    lib = dec.load_library()
    names = declared_functions()
    assert set(dec.EXPORTS) <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def _cfg(**kw):
    from memory_bound_transformer_decode_amd import dec, synth
    base = dict(num_blocks=64, max_batch=8, max_seq_len=128)
    base.update(kw)
    return dec.make_config(synth.TINY, **base)


def test_workspace_bytes_valid_and_invalid():
    from memory_bound_transformer_decode_amd import dec
    lib = dec.load_library()
    c = _cfg()
    n = lib.dec_workspace_bytes(ctypes.byref(c))
    assert n > 0 and n % 256 == 0
    # workspace grows with the batch capacity
    c64 = _cfg(max_batch=64)
    assert lib.dec_workspace_bytes(ctypes.byref(c64)) > n
    bad = _cfg()
    bad.d_head = 96
    assert lib.dec_workspace_bytes(ctypes.byref(bad)) == 0
    assert b"d_head" in lib.dec_last_error()


@pytest.mark.parametrize("field,value,code,needle", [
    ("d_model", 100, -1, b"d_model"),
    ("n_kv_heads", 3, -1, b"n_q_heads"),
    ("block_size", 32, -4, b"block_size"),
    ("max_batch", 13, -1, b"max_batch"),
    ("max_seq_len", 0, -1, b"max_seq_len"),
    ("vocab", 1001, -1, b"vocab"),
    ("weight_dtype", 7, -1, b"dtype"),
    ("flags", 1 << 9, -1, b"flag"),
    ("flags", 32, -1, b"flag"),
    ("kv_dtype", 2, -1, b"dtype"),
    ("max_seq_len", 524289, -4, b"max_seq_len"),
    ("rms_eps", 0.0, -1, b"rms_eps"),
    ("num_blocks", 0, -1, b"num_blocks"),
])
def test_create_rejects_bad_config_before_touching_the_gpu(field, value, code, needle):
    from memory_bound_transformer_decode_amd import dec
    lib = dec.load_library()
    c = _cfg()
    setattr(c, field, value)
    ctx = ctypes.c_void_p()
    rc = lib.dec_create(ctypes.byref(c), None, ctypes.c_void_p(16), ctypes.c_void_p(256), 1 << 30,
                        ctypes.c_void_p(16), ctypes.byref(ctx))
    assert rc == code
    assert needle in lib.dec_last_error()
    assert ctx.value is None


def test_create_rejects_small_or_misaligned_workspace():
    from memory_bound_transformer_decode_amd import dec
    lib = dec.load_library()
    c = _cfg()
    need = lib.dec_workspace_bytes(ctypes.byref(c))
    ctx = ctypes.c_void_p()
    rc = lib.dec_create(ctypes.byref(c), None, ctypes.c_void_p(16), ctypes.c_void_p(256), need - 1,
                        ctypes.c_void_p(16), ctypes.byref(ctx))
    assert rc == dec.DEC_E_INVALID and b"workspace" in lib.dec_last_error()
    rc = lib.dec_create(ctypes.byref(c), None, ctypes.c_void_p(16), ctypes.c_void_p(128), need,
                        ctypes.c_void_p(16), ctypes.byref(ctx))
    assert rc == dec.DEC_E_INVALID and b"256-byte" in lib.dec_last_error()
    rc = lib.dec_create(ctypes.byref(c), None, None, ctypes.c_void_p(256), need,
                        ctypes.c_void_p(16), ctypes.byref(ctx))
    assert rc == dec.DEC_E_INVALID


def test_null_context_calls():
    from memory_bound_transformer_decode_amd import dec
    lib = dec.load_library()
    assert lib.dec_step(None, None) == dec.DEC_E_INVALID
    assert lib.dec_load_weights(None, None) == dec.DEC_E_INVALID
    assert lib.dec_get_info(None, None, None) == dec.DEC_E_INVALID
    assert lib.dec_get_step_info(None, None) == dec.DEC_E_INVALID
    assert lib.dec_verify(None, None) == dec.DEC_E_INVALID
    assert lib.dec_prefill(None, None, None) == dec.DEC_E_INVALID
    assert lib.dec_set_flags(None, 0) == dec.DEC_E_INVALID
    assert lib.dec_sample_greedy(None, None) == dec.DEC_E_INVALID
    assert lib.dec_destroy(None) == dec.DEC_OK
    out = ctypes.c_double()
    assert lib.dec_bw_probe(None, 16, 1, None, ctypes.byref(out)) == dec.DEC_E_INVALID


def test_unknown_flag_bits_rejected():
    from memory_bound_transformer_decode_amd import dec
    lib = dec.load_library()
    c = _cfg(flags=1 << 20)
    ctx = ctypes.c_void_p()
    rc = lib.dec_create(ctypes.byref(c), None, ctypes.c_void_p(16), ctypes.c_void_p(256), 1 << 30,
                        ctypes.c_void_p(16), ctypes.byref(ctx))
    assert rc == dec.DEC_E_INVALID
    assert b"flag" in lib.dec_last_error()


def test_int8_weights_accepted_by_the_workspace_query():
    from memory_bound_transformer_decode_amd import dec
    lib = dec.load_library()
    c = _cfg()
    c.weight_dtype = dec.DEC_INT8
    assert lib.dec_workspace_bytes(ctypes.byref(c)) > 0


def test_unfused_flag_accepted_by_the_workspace_query():
    from memory_bound_transformer_decode_amd import dec
    lib = dec.load_library()
    c = _cfg(flags=dec.FLAG_UNFUSED)
    assert lib.dec_workspace_bytes(ctypes.byref(c)) > 0
