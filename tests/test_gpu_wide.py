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


@pytest.mark.parametrize("G,N,dt", [(37, 5, "f32"), (3, 3001, "bf16"), (1, 1, "f32")])
def test_wide_encode_tiles_across_groups(G, N, dt):
    """32-key tiles that span several groups (N = 5), workgroups that walk
    more than one tile with bf16 keys (9003 keys), and a single key."""
    rng = np.random.default_rng(100 + G + N)
    keys = _keys(rng, G, N, unit=(dt == "f32"))
    dtype = torch.bfloat16 if dt == "bf16" else torch.float32
    if dt == "bf16":
        keys = _round_bf16(keys)
    _encode_check(4, keys, dtype, seed=11)


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


def test_wide_encode_many_tiles_per_workgroup():
    """65,836 keys: every workgroup walks several 32-key tiles (the fragment
    ring and the key prefetch run on from tile to tile), and records late in
    the launch are encoded exactly like the same keys early in it."""
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


def _score_check(cb, cbo, packed, buf, q, keys, dtype):
    from parity import check_logits
    G, Qg, d = q.shape
    N = keys.shape[1]
    print(f"[case] wide score G={G} Qg={Qg} N={N} bits={cb.bits}", flush=True)
    lg = K.score_logits(cb, _dev(q, dtype), packed, N).cpu().numpy()
    ref = O.score(cbo, buf, G, N, q)
    return check_logits(lg, ref, q, np.linalg.norm(keys.astype(np.float64), axis=-1))


@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_wide_score(bits, dt):
    rng = np.random.default_rng(77 * bits + (1 if dt == "bf16" else 0))
    G, N, Qg = 2, 333, 5
    keys = _keys(rng, G, N, unit=(dt == "f32"))
    q = rng.standard_normal((G, Qg, D)).astype(np.float32)
    dtype = torch.bfloat16 if dt == "bf16" else torch.float32
    if dt == "bf16":
        keys, q = _round_bf16(keys), _round_bf16(q)
    cb, cbo, packed, buf, _ = _encode_check(bits, keys, dtype, seed=3 + bits)
    _score_check(cb, cbo, packed, buf, q, keys, dtype)


def _check_topk(idx, sc, ref, q, knorm, k):
    """idx/sc [G, Qg, k] from the GPU; ref [G, Qg, N] oracle estimates."""
    G, Qg, N = ref.shape
    tol = 1e-4 * np.linalg.norm(q.astype(np.float64), axis=-1)[..., None] * knorm.max()
    kk = min(k, N)
    assert np.all(idx[..., kk:] == -1) and np.all(np.isneginf(sc[..., kk:]))
    idx, sc = idx[..., :kk].astype(np.int64), sc[..., :kk].astype(np.float64)
    assert np.all((idx >= 0) & (idx < N))
    o_idx, o_val = O.top_k(ref, min(kk + 1, N))
    for g in range(G):
        for h in range(Qg):
            t = tol[g, h, 0]
            ids = idx[g, h]
            assert len(set(ids.tolist())) == kk, "duplicate indices"
            assert np.all(np.abs(sc[g, h] - ref[g, h, ids]) <= t), "scores differ from the oracle's"
            # order: non-increasing; among equal scores, increasing index
            d = np.diff(sc[g, h])
            assert np.all(d <= 0) and np.all((d < 0) | (np.diff(ids) > 0))
            kth = o_val[g, h, kk - 1]
            assert np.all(ref[g, h, ids] >= kth - 2 * t), "a returned key is not among the best"
            nxt = o_val[g, h, kk] if N > kk else -np.inf
            sure = o_idx[g, h, :kk][o_val[g, h, :kk] > nxt + 2 * t]
            assert set(sure.tolist()) <= set(ids.tolist()), "a clear top-k key is missing"


def test_wide_topk_search_sample():
    """Top-10 of 256 queries over the first 16,384 vectors of the search workload."""
    wl = W.workload(4)
    n = 16384
    keys = W.group_keys(wl, 0, 0, n)[None]
    q = W.group_queries(wl, 0)[None]
    cb = K.Codebook(D, wl.bits)
    cbo = O.make_codebook(D, wl.bits, D, 42)
    print("[case] wide top-10 search sample", flush=True)
    packed = K.encode_keys(cb, _dev(keys, torch.float32))
    idx, sc = K.score_topk(cb, _dev(q, torch.float32), packed, n, 10)
    torch.cuda.synchronize()
    buf = packed.cpu().numpy()
    ref = O.score(cbo, buf, 1, n, q)
    _check_topk(idx.cpu().numpy(), sc.cpu().numpy(), ref, q, np.linalg.norm(keys, axis=-1), 10)


@pytest.mark.parametrize("N,k", [(5, 10), (70, 10), (1000, 16), (3000, 1)])
def test_wide_topk_ragged(N, k):
    rng = np.random.default_rng(N + k)
    G, Qg = 2, 6
    keys = _keys(rng, G, N)
    q = rng.standard_normal((G, Qg, D)).astype(np.float32)
    cb = K.Codebook(D, 4)
    cbo = O.make_codebook(D, 4, D, 42)
    print(f"[case] wide top-{k} N={N}", flush=True)
    packed = K.encode_keys(cb, _dev(keys, torch.float32))
    idx, sc = K.score_topk(cb, _dev(q, torch.float32), packed, N, k)
    torch.cuda.synchronize()
    ref = O.score(cbo, packed.cpu().numpy(), G, N, q)
    _check_topk(idx.cpu().numpy(), sc.cpu().numpy(), ref, q, np.linalg.norm(keys, axis=-1), k)


@pytest.mark.parametrize("bits,N,Qg,k", [(4, 1000, 40, 10), (3, 333, 32, 16), (2, 5000, 70, 5), (4, 129, 256, 1)])
def test_wide_topk_many_queries(bits, N, Qg, k):
    """32 or more queries per group take the matrix-core top-k: ragged vector
    tiles, ragged query blocks, every supported code width."""
    rng = np.random.default_rng(N + Qg + k + bits)
    G = 1 if Qg > 64 else 2
    keys = _keys(rng, G, N)
    q = rng.standard_normal((G, Qg, D)).astype(np.float32) * np.exp(rng.normal(0, 1, (G, Qg, 1)))
    cb = K.Codebook(D, bits)
    cbo = O.make_codebook(D, bits, D, 42)
    print(f"[case] wide matrix-core top-{k} bits={bits} N={N} Qg={Qg}", flush=True)
    packed = K.encode_keys(cb, _dev(keys, torch.float32))
    idx, sc = K.score_topk(cb, _dev(q, torch.float32), packed, N, k)
    torch.cuda.synchronize()
    ref = O.score(cbo, packed.cpu().numpy(), G, N, q)
    _check_topk(idx.cpu().numpy(), sc.cpu().numpy(), ref, q, np.linalg.norm(keys, axis=-1), k)


def test_wide_topk_argument_errors():
    import ctypes
    cb = K.Codebook(D, 4)
    lib = K.library()
    assert lib.tq_score_topk_workspace_bytes(cb.handle, 1, 4, 100, 17) == 0
    q = torch.zeros((1, 4, D), device="cuda")
    packed = torch.zeros(K.packed_nbytes(cb, 1, 100), dtype=torch.uint8, device="cuda")
    idx = torch.empty((1, 4, 10), dtype=torch.int32, device="cuda")
    sc = torch.empty((1, 4, 10), device="cuda")
    args = (cb.handle, ctypes.c_void_p(q.data_ptr()), 0, 1, 4, ctypes.c_void_p(packed.data_ptr()), 100)
    assert lib.tq_score_topk(*args, 17, ctypes.c_void_p(idx.data_ptr()), ctypes.c_void_p(sc.data_ptr()),
                             None, 0, None) == -2
    assert lib.tq_score_topk(*args, 10, ctypes.c_void_p(idx.data_ptr()), ctypes.c_void_p(sc.data_ptr()),
                             None, 0, None) == -5
    cb128 = K.Codebook(128, 3)
    assert lib.tq_score_topk(cb128.handle, ctypes.c_void_p(q.data_ptr()), 0, 1, 4,
                             ctypes.c_void_p(packed.data_ptr()), 100, 10, ctypes.c_void_p(idx.data_ptr()),
                             ctypes.c_void_p(sc.data_ptr()), None, 0, None) == -2
