"""GPU parity with the exact-Beta codebook (TQ_CODEBOOK_BETA): the kernels
read their levels and thresholds from the codebook, so every path must match
the oracle built with the same law."""

import math

import numpy as np
import pytest

import oracle as O
from kv_cache_vector_rotate_amd import workloads as W
from parity import attention_tolerance, check_encode, check_logits, check_values

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
K = pytest.importorskip("kv_cache_vector_rotate_amd")


def _dev(a, dtype):
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to("cuda")
    return t.to(dtype) if dtype != torch.float32 else t


def _rows(rng, G, N, d):
    scale = np.exp(rng.normal(0, math.sqrt(0.5), d))
    scale[rng.choice(d, 4, replace=False)] *= 20
    return (rng.standard_normal((G, N, d)) * scale).astype(np.float32)


@pytest.mark.parametrize("d,bits,dt", [(128, 3, "bf16"), (128, 4, "f32"), (1024, 4, "f32"), (1024, 2, "bf16")])
def test_beta_encode_and_score(d, bits, dt):
    rng = np.random.default_rng(d + bits)
    G, N, Qg = 2, 301, 5
    keys = _rows(rng, G, N, d)
    q = rng.standard_normal((G, Qg, d)).astype(np.float32)
    dtype = torch.bfloat16 if dt == "bf16" else torch.float32
    if dt == "bf16":
        keys = W.bf16_bits_to_f32(W.f32_to_bf16_bits(keys))
        q = W.bf16_bits_to_f32(W.f32_to_bf16_bits(q))
    cb = K.Codebook(d, bits, d, 9, kind="beta")
    cbo = O.make_codebook(d, bits, d, 9, kind="beta")
    print(f"[case] beta d={d} bits={bits} dtype={dt}", flush=True)
    packed = K.encode_keys(cb, _dev(keys, dtype))
    lg = K.score_logits(cb, _dev(q, dtype), packed, N)
    torch.cuda.synchronize()
    buf = packed.cpu().numpy()
    codes, signs, nu16, rho16 = O.unpack(cbo, buf, G, N)
    check_encode(cbo, keys.reshape(-1, d), codes.reshape(-1, d), signs.reshape(-1, d),
                 nu16.reshape(-1), rho16.reshape(-1))
    check_logits(lg.cpu().numpy(), O.score(cbo, buf, G, N, q), q,
                 np.linalg.norm(keys.astype(np.float64), axis=-1))


def test_beta_values_and_attention():
    rng = np.random.default_rng(55)
    G, N, Qg, d = 2, 700, 4, 128
    k = _rows(rng, G, N, d)
    v = _rows(rng, G, N, d)
    q = rng.standard_normal((G, Qg, d)).astype(np.float32)
    cb = K.Codebook(d, 3, kind="beta")
    cbo = O.make_codebook(d, 3, d, 42, kind="beta")
    print("[case] beta values and attention", flush=True)
    kb = K.encode_keys(cb, _dev(k, torch.float32))
    vb = K.encode_values(cb, _dev(v, torch.float32))
    out = K.attention_decode(cb, _dev(q, torch.float32), kb, vb, N)
    lg = K.score_logits(cb, _dev(q, torch.float32), kb, N)
    torch.cuda.synchronize()
    vbuf = vb.cpu().numpy()
    codes, nu16 = O.unpack_values(cbo, vbuf, G, N)
    check_values(cbo, v.reshape(-1, d), codes.reshape(-1, d), nu16.reshape(-1))
    ref = O.attention_from_logits(cbo, lg.cpu().numpy().astype(np.float64), vbuf, G, N)
    vhat = O.decode_values(cbo, vbuf, G, N)
    assert np.all(np.abs(out.cpu().numpy() - ref) <= attention_tolerance(vhat))


def test_beta_many_query_topk():
    rng = np.random.default_rng(66)
    G, N, Qg, d, k = 1, 2000, 48, 1024, 10
    keys = _rows(rng, G, N, d)
    q = rng.standard_normal((G, Qg, d)).astype(np.float32)
    cb = K.Codebook(d, 4, kind="beta")
    cbo = O.make_codebook(d, 4, d, 42, kind="beta")
    print("[case] beta matrix-core top-k", flush=True)
    packed = K.encode_keys(cb, _dev(keys, torch.float32))
    idx, sc = K.score_topk(cb, _dev(q, torch.float32), packed, N, k)
    torch.cuda.synchronize()
    ref = O.score(cbo, packed.cpu().numpy(), G, N, q)
    tol = 1e-4 * np.linalg.norm(q.astype(np.float64), axis=-1)[..., None] * np.linalg.norm(keys, axis=-1).max()
    idx, sc = idx.cpu().numpy().astype(np.int64), sc.cpu().numpy().astype(np.float64)
    o_idx, o_val = O.top_k(ref, k + 1)
    for h in range(Qg):
        t = tol[0, h, 0]
        assert np.all(np.abs(sc[0, h] - ref[0, h, idx[0, h]]) <= t)
        assert np.all(ref[0, h, idx[0, h]] >= o_val[0, h, k - 1] - 2 * t)
