"""GPU tests of zero padding: vectors of d elements, d not a power of two,
run in D = tq_rotation_dim(d) dimensions with the missing coordinates read
as zeros [ICLR 2026 digest, 実装のポイント].

* Records written from rows of d elements are byte-identical to the records
  of the same rows padded with zeros to D under the D codebook (same seed),
  and pass the oracle's parity rules;
* logits, decoded keys, value records and attention outputs equal the D
  codebook's on padded inputs (bit for bit; decoded and attention rows keep
  their first d coordinates) and the oracle's within the parity rules;
* d = 768 (D = 1024): encode, score and top-k the same way.
"""

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


def _bf16(a):
    return W.bf16_bits_to_f32(W.f32_to_bf16_bits(a))


def _rows(rng, G, N, d, outliers=True):
    scale = np.exp(rng.normal(0, math.sqrt(0.5), d))
    if outliers:
        scale[rng.choice(d, 4, replace=False)] *= 20
    return (rng.standard_normal((G, N, d)) * scale).astype(np.float32)


def _pad(a, D):
    return np.pad(a, [(0, 0)] * (a.ndim - 1) + [(0, D - a.shape[-1])])


@pytest.mark.parametrize("din", [80, 96, 112])
@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_padded_encode_score_decode(din, bits, dt):
    rng = np.random.default_rng(3000 + din + 10 * bits + (1 if dt == "bf16" else 0))
    G, N, Qg, D = 2, 77, 5, 128
    k = _rows(rng, G, N, din)
    q = rng.standard_normal((G, Qg, din)).astype(np.float32)
    dtype = torch.bfloat16 if dt == "bf16" else torch.float32
    if dt == "bf16":
        k, q = _bf16(k), _bf16(q)
    k[0, 3] = 0.0                                   # zero-vector rule on a padded row
    cb = K.Codebook(din, bits, seed=23)
    cbD = K.Codebook(D, bits, seed=23)
    cbo = O.make_codebook(din, bits, D, 23)
    assert (cb.D, cb.m) == (D, D)
    print(f"[case] pad din={din} bits={bits} dtype={dt}", flush=True)
    kb = K.encode_keys(cb, _dev(k, dtype))
    kbD = K.encode_keys(cbD, _dev(_pad(k, D), dtype))
    lg = K.score_logits(cb, _dev(q, dtype), kb, N)
    lgD = K.score_logits(cbD, _dev(_pad(q, D), dtype), kb, N)
    dec = K.decode_mse(cb, kb, G, N)
    decD = K.decode_mse(cbD, kb, G, N)
    torch.cuda.synchronize()
    assert torch.equal(kb, kbD)
    assert torch.equal(lg, lgD)
    assert dec.shape == (G, N, din) and torch.equal(dec, decD[..., :din])
    buf = kb.cpu().numpy()
    codes, signs, nu16, rho16 = O.unpack(cbo, buf, G, N)
    check_encode(cbo, k.reshape(-1, din), codes.reshape(-1, D), signs.reshape(-1, D),
                 nu16.reshape(-1), rho16.reshape(-1))
    knorm = np.linalg.norm(k.astype(np.float64), axis=-1)
    check_logits(lg.cpu().numpy(), O.score(cbo, buf, G, N, q), q, knorm)
    ref = O.decode_mse(cbo, buf, G, N)
    assert np.allclose(dec.cpu().numpy(), ref, rtol=0, atol=2e-6 * max(1.0, float(np.abs(ref).max())))


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_padded_append_and_cache(dt):
    rng = np.random.default_rng(77)
    din, D, G, Ncap, Qg = 96, 128, 3, 64, 4
    k = _rows(rng, G, 50, din)
    q = rng.standard_normal((G, Qg, din)).astype(np.float32)
    dtype = torch.bfloat16 if dt == "bf16" else torch.float32
    if dt == "bf16":
        k, q = _bf16(k), _bf16(q)
    cb = K.Codebook(din, 3)
    kd = _dev(k, dtype)
    print(f"[case] pad append dtype={dt}", flush=True)
    ref = K.encode_keys(cb, kd)
    cache = torch.zeros(K.packed_nbytes(cb, G, Ncap), dtype=torch.uint8, device="cuda")
    K.append_keys(cb, kd[:, :30].contiguous(), cache, Ncap, 0)
    for t in range(30, 50):
        K.append_keys(cb, kd[:, t:t + 1].contiguous(), cache, Ncap, t)
    lc = K.score_cache(cb, _dev(q, dtype), cache, Ncap, 50)
    torch.cuda.synchronize()
    # the appends (latency kernel, float32 rotation) against the oracle, and
    # against tq_encode_keys's records but for the few the parity rules leave open
    cbo = O.make_codebook(din, 3, D, 42)
    c1 = [np.ascontiguousarray(np.asarray(a)[:, :50]) for a in O.unpack(cbo, cache.cpu().numpy(), G, Ncap)]
    c2 = O.unpack(cbo, ref.cpu().numpy(), G, 50)
    codes, signs, nu16, rho16 = c1
    check_encode(cbo, k.reshape(-1, din), codes.reshape(-1, D), signs.reshape(-1, D),
                 nu16.reshape(-1), rho16.reshape(-1))
    differ = np.zeros((G, 50), bool)
    for a, b in zip(c1, c2):
        a8, b8 = a.view(np.uint8).reshape(G, 50, -1), np.asarray(b).view(np.uint8).reshape(G, 50, -1)
        differ |= np.any(a8 != b8, axis=-1)
    assert int(differ.sum()) <= 2
    knorm = np.linalg.norm(k.astype(np.float64), axis=-1)
    compact = O.pack(cbo, codes, signs, nu16, rho16)
    check_logits(lc.cpu().numpy(), O.score(cbo, compact, G, 50, q), q, knorm)


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_padded_values_and_attention(bits):
    rng = np.random.default_rng(500 + bits)
    din, D, G, N, Qg = 112, 128, 2, 300, 6
    k = _rows(rng, G, N, din)
    v = _rows(rng, G, N, din, outliers=False)
    q = rng.standard_normal((G, Qg, din)).astype(np.float32)
    cb = K.Codebook(din, bits)
    cbD = K.Codebook(D, bits)
    cbo = O.make_codebook(din, bits, D, 42)
    print(f"[case] pad attention bits={bits}", flush=True)
    kb = K.encode_keys(cb, _dev(k, torch.float32))
    vb = K.encode_values(cb, _dev(v, torch.float32))
    vbD = K.encode_values(cbD, _dev(_pad(v, D), torch.float32))
    out = K.attention_decode(cb, _dev(q, torch.float32), kb, vb, N)
    outD = K.attention_decode(cbD, _dev(_pad(q, D), torch.float32), kb, vb, N, scale=1.0 / math.sqrt(din))
    lg = K.score_logits(cb, _dev(q, torch.float32), kb, N)
    torch.cuda.synchronize()
    assert torch.equal(vb, vbD)
    assert out.shape == (G, Qg, din) and torch.equal(out, outD[..., :din])
    vbuf = vb.cpu().numpy()
    codes, nu16 = O.unpack_values(cbo, vbuf, G, N)
    check_values(cbo, v.reshape(-1, din), codes.reshape(-1, D), nu16.reshape(-1))
    ref = O.attention_from_logits(cbo, lg.cpu().numpy().astype(np.float64), vbuf, G, N)
    vhat = O.decode_values(cbo, vbuf, G, N)
    assert np.all(np.abs(out.cpu().numpy() - ref) <= attention_tolerance(vhat))


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_padded_wide(dt):
    """d = 768 runs in D = 1024 (the vector-search path)."""
    rng = np.random.default_rng(768)
    din, D, G, N, Qg = 768, 1024, 1, 700, 3
    x = rng.standard_normal((G, N, din)) * np.exp(rng.normal(0, math.sqrt(0.5), din))
    x = (x / np.linalg.norm(x, axis=-1, keepdims=True)).astype(np.float32)
    q = rng.standard_normal((G, Qg, din)).astype(np.float32)
    dtype = torch.bfloat16 if dt == "bf16" else torch.float32
    if dt == "bf16":
        x, q = _bf16(x), _bf16(q)
    cb = K.Codebook(din, 4)
    cbD = K.Codebook(D, 4)
    cbo = O.make_codebook(din, 4, D, 42)
    print(f"[case] pad wide dtype={dt}", flush=True)
    kb = K.encode_keys(cb, _dev(x, dtype))
    kbD = K.encode_keys(cbD, _dev(_pad(x, D), dtype))
    lg = K.score_logits(cb, _dev(q, dtype), kb, N)
    lgD = K.score_logits(cbD, _dev(_pad(q, D), dtype), kb, N)
    idx, sc = K.score_topk(cb, _dev(q, dtype), kb, N, 10)
    idxD, scD = K.score_topk(cbD, _dev(_pad(q, D), dtype), kb, N, 10)
    torch.cuda.synchronize()
    assert torch.equal(kb, kbD)
    assert torch.equal(lg, lgD)
    assert torch.equal(idx, idxD) and torch.equal(sc, scD)
    buf = kb.cpu().numpy()
    codes, signs, nu16, rho16 = O.unpack(cbo, buf, G, N)
    check_encode(cbo, x.reshape(-1, din), codes.reshape(-1, D), signs.reshape(-1, D),
                 nu16.reshape(-1), rho16.reshape(-1))
    check_logits(lg.cpu().numpy(), O.score(cbo, buf, G, N, q), q,
                 np.linalg.norm(x.astype(np.float64), axis=-1))
