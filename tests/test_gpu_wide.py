"""GPU parity for d = m = 1024 (the vector-search shape) through the C ABI.

Encode: rotate/quantize kernel + matrix-core QJL projection against the fp64
oracle under the rules in tests/parity.py.  Sizes cover ragged 64-key tiles
of the projection and the special keys.
"""

import math

import numpy as np
import pytest

import oracle as O
from kv_cache_vector_rotate_amd import workloads as W
from parity import check_encode

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
K = pytest.importorskip("kv_cache_vector_rotate_amd")

D = 1024


def _dev(a, dtype):
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to("cuda")
    return t.to(dtype) if dtype != torch.float32 else t


def _keys(rng, G, N, unit=True):
    scale = np.exp(rng.normal(0, math.sqrt(0.5), D))
    k = rng.standard_normal((G, N, D)) * scale
    if unit:
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    else:
        k[..., rng.choice(D, 4, replace=False)] *= 20
    return k.astype(np.float32)


def _round_bf16(a):
    return W.bf16_bits_to_f32(W.f32_to_bf16_bits(a))


def _encode_check(bits, keys, dtype, seed=42):
    G, N, d = keys.shape
    cbo = O.make_codebook(d, bits, d, seed)
    cb = K.Codebook(d, bits, d, seed)
    print(f"[case] wide encode G={G} N={N} bits={bits} dtype={dtype}", flush=True)
    packed = K.encode_keys(cb, _dev(keys, dtype))
    torch.cuda.synchronize()
    buf = packed.cpu().numpy()
    codes, signs, nu16, rho16 = O.unpack(cbo, buf, G, N)
    st = check_encode(cbo, keys.reshape(-1, d), codes.reshape(-1, d), signs.reshape(-1, d),
                      nu16.reshape(-1), rho16.reshape(-1))
    return cb, cbo, packed, buf, st


@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_wide_encode(bits, dt):
    rng = np.random.default_rng(31 * bits + (1 if dt == "bf16" else 0))
    keys = _keys(rng, 2, 97, unit=(dt == "f32"))
    dtype = torch.bfloat16 if dt == "bf16" else torch.float32
    if dt == "bf16":
        keys = _round_bf16(keys)
    _encode_check(bits, keys, dtype, seed=7 + bits)


def test_wide_encode_special_keys():
    rng = np.random.default_rng(3)
    keys = _keys(rng, 1, 70)
    keys[0, 0] = 0.0
    keys[0, 1] = 0.0
    keys[0, 1, 5] = 1e-12          # below the zero-norm rule
    keys[0, 2] = 0.0
    keys[0, 2, 700] = 2.0          # one-hot
    keys[0, 3] = 0.25              # constant
    keys[0, 4] = 0.0
    keys[0, 4, :2] = 1.0           # exact zeros after the rotation
    _, cbo, _, buf, _ = _encode_check(4, keys, torch.float32)
    codes, signs, nu16, rho16 = O.unpack(cbo, buf, 1, 70)
    assert not codes[0, :2].any() and not signs[0, :2].any()
    assert float(nu16[0, 0]) == 0.0 and float(nu16[0, 1]) == 0.0


def test_wide_encode_search_workload_sample():
    """The first 4096 vectors of the 1M-vector search workload (b = 4)."""
    wl = W.workload(4)
    keys = W.group_keys(wl, 0, 0, 4096)[None]
    _encode_check(wl.bits, keys, torch.float32)


def test_wide_encode_chunk_boundary():
    """More keys than one workspace chunk (65,536): records past the first
    chunk are encoded exactly like the ones before it."""
    rng = np.random.default_rng(8)
    n = 65536 + 300
    base = _keys(rng, 1, 300)
    keys = np.concatenate([np.zeros((1, 65536, D), np.float32), base], axis=1)
    keys[0, :300] = base[0]
    cb = K.Codebook(D, 4)
    print("[case] wide encode chunk boundary", flush=True)
    packed = K.encode_keys(cb, _dev(keys, torch.float32)).cpu().numpy()
    cbo = O.make_codebook(D, 4, D, 42)
    codes, signs, nu16, rho16 = O.unpack(cbo, packed, 1, n)
    assert np.array_equal(codes[0, :300], codes[0, 65536:])
    assert np.array_equal(signs[0, :300], signs[0, 65536:])
    assert np.array_equal(nu16[0, :300], nu16[0, 65536:])
    assert not codes[0, 300:65536].any() and not nu16[0, 300:65536].any()
