"""dec_attention_noalloc -- the attention call for callers that cannot allocate device
memory -- against dec_attention, the same kernels with the caller's workspace (needs an
MI355X).  Two calls in a row on the static scratch, the second with a smaller input:
outputs bit-identical to dec_attention's on the same inputs.
"""

import ctypes

import numpy as np
import pytest
import torch

from harness import log, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dec():
    return require_gpu()


def inputs(n, Hq, Hkv, dh, kv, lens, max_blocks, seed):
    rng = np.random.default_rng(seed)
    nb = n * max_blocks + 3
    vals = torch.from_numpy(rng.standard_normal((2, 2, nb, Hkv, 16, dh)).astype(np.float32))
    pool = vals.to(torch.bfloat16 if kv == "bf16" else torch.float8_e4m3fn).cuda()
    bt = rng.permutation(nb)[: n * max_blocks].reshape(n, max_blocks).astype(np.int32)
    q = torch.from_numpy((rng.standard_normal((n, Hq, dh)) * 2.0).astype(np.float32)).cuda()
    return q, pool, torch.from_numpy(np.asarray(lens, np.int32)).cuda(), torch.from_numpy(bt).cuda()


def noalloc(dec, q, pool, lens, bt, layer=1):
    lib = dec.load_library()
    desc = dec.attn_desc(q, pool, layer, bt)
    out = torch.empty(q.shape[0], q.shape[1] * q.shape[2], dtype=torch.bfloat16, device="cuda")
    P = ctypes.c_void_p
    rc = lib.dec_attention_noalloc(ctypes.byref(desc), P(q.data_ptr()), P(pool.data_ptr()), P(lens.data_ptr()),
                                   P(bt.data_ptr()), P(out.data_ptr()), P(torch.cuda.current_stream().cuda_stream))
    if rc != dec.DEC_OK:
        raise dec.DecError(rc, lib.dec_last_error().decode())
    return out


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_noalloc_matches_workspace_call_twice(dec, kv):
    # first call: 40 rows, long contexts (several splits per row); second: 3 rows
    big = inputs(40, 32, 8, 128, kv, [int(x) for x in np.random.default_rng(1).integers(-1, 2047, 40)], 128, 11)
    small = inputs(3, 10, 2, 64, kv, [5, 0, 700], 64, 12)
    outs = []
    for q, pool, lens, bt in (big, small):
        a = noalloc(dec, q, pool, lens, bt)
        b = dec.attention(q, pool, 1, lens, bt)
        torch.cuda.synchronize()
        outs.append((a, b))
    for a, b in outs:
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    log(f"no-alloc attention {kv}: two calls bit-identical to the workspace call")


def test_noalloc_rejects_shapes_beyond_the_scratch(dec):
    lib = dec.load_library()
    desc = dec.DecAttnDesc(64, 8, 1, 128, 0, 1, 0, 4096, 32768)  # 64 rows x 64 splits x 8 heads x 128
    assert lib.dec_attention_workspace_bytes(ctypes.byref(desc)) > (8 << 20)
    P = ctypes.c_void_p
    dummy = torch.empty(16, dtype=torch.float32, device="cuda")
    rc = lib.dec_attention_noalloc(ctypes.byref(desc), P(dummy.data_ptr()), P(dummy.data_ptr()), P(dummy.data_ptr()),
                                   P(dummy.data_ptr()), P(dummy.data_ptr()), None)
    assert rc == dec.DEC_E_CAPACITY
    assert b"scratch" in lib.dec_last_error()
