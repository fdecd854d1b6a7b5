"""GPU parity for rotation dimensions D = 2048 and 4096 through the C ABI.

Vectors longer than 1024 coordinates are zero-padded to the next power of
two (the pages' example: 3072 -> 4096 [ICLR 2026 digest, 実装のポイント]):
d = 1536 runs in D = 2048 and d = 3072 in D = 4096; d = 2048 needs no
padding.  Encode (rules of tests/parity.py), score and decode against the
fp64 oracle, for float32 and bfloat16 inputs; a padded codebook gives the
same records and logits as the D codebook on the zero-padded inputs.
"""

import functools
import math

import numpy as np
import pytest

import oracle as O
from kv_cache_vector_rotate_amd import workloads as W
from parity import check_encode, check_logits

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
K = pytest.importorskip("kv_cache_vector_rotate_amd")


@functools.lru_cache(maxsize=None)
def _oracle_cb(d, bits, D, seed):
    return O.make_codebook(d, bits, D, seed)


def _dev(a, dtype):
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to("cuda")
    return t.to(dtype) if dtype != torch.float32 else t


def _bf16(a):
    return W.bf16_bits_to_f32(W.f32_to_bf16_bits(a))


def _pad(a, D):
    out = np.zeros(a.shape[:-1] + (D,), np.float32)
    out[..., :a.shape[-1]] = a
    return out


def _rows(rng, G, N, d, unit):
    x = rng.standard_normal((G, N, d)) * np.exp(rng.normal(0, math.sqrt(0.5), d))
    if unit:
        x /= np.linalg.norm(x, axis=-1, keepdims=True)
    else:
        x[..., rng.choice(d, 4, replace=False)] *= 20
    return x.astype(np.float32)


@pytest.mark.parametrize("din,bits,dt", [(1536, 3, "f32"), (1536, 4, "bf16"), (2048, 2, "f32"),
                                         (3072, 4, "f32"), (3072, 3, "bf16")])
def test_wider_encode_score_decode(din, bits, dt):
    rng = np.random.default_rng(din + 10 * bits + (1 if dt == "bf16" else 0))
    D = K.rotation_dim(din)
    G, N, Qg = 2, 83, 5
    x = _rows(rng, G, N, din, unit=(dt == "f32"))
    x[0, 0] = 0.0                                        # zero record
    q = rng.standard_normal((G, Qg, din)).astype(np.float32)
    dtype = torch.bfloat16 if dt == "bf16" else torch.float32
    if dt == "bf16":
        x, q = _bf16(x), _bf16(q)
    cb = K.Codebook(din, bits)
    cbo = _oracle_cb(din, bits, D, 42)
    print(f"[case] wider d={din} D={D} bits={bits} dtype={dt}", flush=True)
    kb = K.encode_keys(cb, _dev(x, dtype))
    ws = torch.empty(max(16, K.score_workspace_nbytes(cb, G, Qg)), dtype=torch.uint8, device="cuda")
    lg = K.score_logits(cb, _dev(q, dtype), kb, N, ws=ws)
    dec = K.decode_mse(cb, kb, G, N)
    dec16 = K.decode_mse(cb, kb, G, N, dtype=torch.bfloat16)
    torch.cuda.synchronize()
    buf = kb.cpu().numpy()
    codes, signs, nu16, rho16 = O.unpack(cbo, buf, G, N)
    check_encode(cbo, x.reshape(-1, din), codes.reshape(-1, D), signs.reshape(-1, D),
                 nu16.reshape(-1), rho16.reshape(-1))
    check_logits(lg.cpu().numpy(), O.score(cbo, buf, G, N, q), q,
                 np.linalg.norm(x.astype(np.float64), axis=-1))
    ref = O.decode_mse(cbo, buf, G, N)
    assert dec.shape == (G, N, din)
    nu = nu16.astype(np.float64)[..., None]
    assert np.all(np.abs(dec.cpu().numpy().astype(np.float64) - ref) <= 1e-5 * nu)
    assert torch.equal(dec16.view(torch.int16), dec.to(torch.bfloat16).view(torch.int16))
    if din != D:
        # the padded codebook equals the D codebook on zero-padded rows
        cbD = K.Codebook(D, bits)
        kbD = K.encode_keys(cbD, _dev(_pad(x, D), dtype))
        lgD = K.score_logits(cbD, _dev(_pad(q, D), dtype), kb, N, ws=ws)
        torch.cuda.synchronize()
        assert torch.equal(kb, kbD)
        assert torch.equal(lg, lgD)


def test_wider_ragged_ranges_and_groups():
    """Many keys per group (several key ranges and 64-key tiles with a ragged
    tail) at D = 2048, one query chunk with a ragged query count."""
    rng = np.random.default_rng(2222)
    din, bits, G, N, Qg = 2048, 3, 3, 2500, 6
    x = _rows(rng, G, N, din, unit=False)
    q = rng.standard_normal((G, Qg, din)).astype(np.float32)
    cb = K.Codebook(din, bits)
    cbo = _oracle_cb(din, bits, din, 42)
    print("[case] wider ragged", flush=True)
    kb = K.encode_keys(cb, _dev(x, torch.float32))
    lg = K.score_logits(cb, _dev(q, torch.float32), kb, N)
    torch.cuda.synchronize()
    buf = kb.cpu().numpy()
    codes, signs, nu16, rho16 = O.unpack(cbo, buf, G, N)
    for g in range(G):
        check_encode(cbo, x[g], codes[g], signs[g], nu16[g], rho16[g])
    check_logits(lg.cpu().numpy(), O.score(cbo, buf, G, N, q), q,
                 np.linalg.norm(x.astype(np.float64), axis=-1))


def test_wider_topk_is_unsupported():
    cb = K.Codebook(3072, 4)
    kb = torch.zeros(K.packed_nbytes(cb, 1, 100), dtype=torch.uint8, device="cuda")
    q = torch.zeros((1, 2, 3072), device="cuda")
    with pytest.raises(K.TQError):
        K.score_topk(cb, q, kb, 100, 10)
    torch.cuda.synchronize()
