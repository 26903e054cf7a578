"""dec_attention (the attention step as a call of its own) against the oracle's
attention on the same cache bits (needs an MI355X).

Inputs: q ~ N(0, 1) fp32 (scaled so the softmax is neither flat nor one-hot), K/V
~ N(0, 1) in the cache format, block tables a seeded permutation of the pool, a
length mix with empty rows (-1), one position, block edges, and contexts long enough
for several splits.  Bar: the output is bf16 (8 significant bits), so each element may
differ from the fp64 value by its rounding, up to 2^-8 of its magnitude, plus the
kernel's arithmetic (q and the probabilities kept as bf16 high + low parts, about 2^-16;
fp32 exponentials and sums): |o - o_ref| <= 2^-8 |o_ref| + 2^-10 max|o_ref| over the
head vector, and exactly 0 for an empty row.
"""

import numpy as np
import pytest
import torch

from memory_bound_transformer_decode_amd import synth
from oracle import codecs
from oracle import decoder as OD

from harness import log, require_gpu

pytestmark = pytest.mark.gpu
REL, ABS = 2.0 ** -8, 2.0 ** -10


@pytest.fixture(scope="module")
def dec():
    return require_gpu()


def make_inputs(n, Hq, Hkv, dh, kv, lens, max_blocks, seed, L=2, layer=1):
    rng = np.random.default_rng(seed)
    nb = n * max_blocks + 5
    shape = (L, 2, nb, Hkv, 16, dh)
    vals = torch.from_numpy(rng.standard_normal(shape).astype(np.float32))
    pool = vals.to(torch.bfloat16 if kv == "bf16" else torch.float8_e4m3fn).cuda()
    bt = rng.permutation(nb)[: n * max_blocks].reshape(n, max_blocks).astype(np.int32)
    q = (rng.standard_normal((n, Hq, dh)) * 2.0).astype(np.float32)
    return (torch.from_numpy(q).cuda(), pool, torch.from_numpy(np.asarray(lens, np.int32)).cuda(),
            torch.from_numpy(bt).cuda(), bt)


def oracle_attention(q, pool_codes, kvfmt, lens, bt, layer, Hkv):
    n, Hq, dh = q.shape
    g = Hq // Hkv
    cache = OD.PagedKVCache(pool_codes, kvfmt)
    out = np.zeros((n, Hq, dh))
    for r in range(n):
        if lens[r] < 0:
            continue
        for c in range(Hkv):
            K = cache.read(layer, 0, bt[r], lens[r] + 1, c)
            V = cache.read(layer, 1, bt[r], lens[r] + 1, c)
            for j in range(c * g, (c + 1) * g):
                out[r, j] = OD.attend(q[r, j].astype(np.float64), K, V)
    return out


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
@pytest.mark.parametrize("Hq,Hkv,dh", [(8, 8, 64), (10, 2, 64), (32, 8, 128), (64, 8, 128), (8, 1, 128)])
def test_attention_matches_oracle(dec, kv, Hq, Hkv, dh):
    lens = [0, 15, 16, 17, -1, 1000, 333, 2047]
    n = len(lens)
    max_blocks = 128
    q, pool, lens_t, bt_t, bt = make_inputs(n, Hq, Hkv, dh, kv, lens, max_blocks, seed=Hq * 7 + dh + (kv == "fp8"))
    o = dec.attention(q, pool, 1, lens_t, bt_t)
    torch.cuda.synchronize()
    got = o.view(torch.int16).cpu().numpy().view(np.uint16).reshape(n, Hq, dh)
    got = codecs.bf16_decode(got)
    ref = oracle_attention(q.cpu().numpy(), synth.kv_codes_numpy(pool), kv, lens, bt, 1, Hkv)
    worst = 0.0
    for r in range(n):
        if lens[r] < 0:
            assert np.all(got[r] == 0.0)
            continue
        for j in range(Hq):
            scale = np.max(np.abs(ref[r, j]))
            err = np.abs(got[r, j] - ref[r, j])
            worst = max(worst, float(np.max(err / (REL * np.abs(ref[r, j]) + ABS * scale))))
    log(f"attention {kv} Hq={Hq} Hkv={Hkv} dh={dh}: worst error / bar {worst:.3f}")
    assert worst <= 1.0


def test_attention_workspace_and_argument_errors(dec):
    q, pool, lens_t, bt_t, _ = make_inputs(2, 8, 2, 64, "bf16", [5, 9], 4, seed=3)
    desc = dec.attn_desc(q, pool, 0, bt_t)
    lib = dec.load_library()
    import ctypes
    need = lib.dec_attention_workspace_bytes(ctypes.byref(desc))
    assert need > 0 and need % 256 == 0
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    out = torch.empty(2, 8 * 64, dtype=torch.bfloat16, device="cuda")
    P = ctypes.c_void_p
    args = (P(q.data_ptr()), P(pool.data_ptr()), P(lens_t.data_ptr()), P(bt_t.data_ptr()), P(out.data_ptr()))
    assert lib.dec_attention(ctypes.byref(desc), *args, P(ws.data_ptr()), need - 1, None) == dec.DEC_E_INVALID
    bad = dec.DecAttnDesc(*[getattr(desc, f) for f, _ in desc._fields_])
    bad.layer = 2
    assert lib.dec_attention(ctypes.byref(bad), *args, P(ws.data_ptr()), need, None) == dec.DEC_E_INVALID
    bad = dec.DecAttnDesc(*[getattr(desc, f) for f, _ in desc._fields_])
    bad.n_rows = 65
    assert lib.dec_attention_workspace_bytes(ctypes.byref(bad)) == 0
    assert lib.dec_attention(ctypes.byref(desc), *args, P(ws.data_ptr()), need,
                             P(torch.cuda.current_stream().cuda_stream)) == dec.DEC_OK
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all()
