"""GPU parity of the value path and decode attention through the C ABI.

Value records against the oracle's MSE-only encoder (code and norm rules of
tests/parity.py); decode attention against the oracle's softmax over the same
packed keys and values: tightly when the oracle is given the GPU's logits
(same records, same logits: only fp32 exponentials and sums differ), and
within the bound the logit tolerance implies when the oracle uses its own
fp64 logits.
"""

import math

import numpy as np
import pytest

import oracle as O
from kv_cache_vector_rotate_amd import workloads as W
from parity import attention_tolerance, check_logits, check_values

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
K = pytest.importorskip("kv_cache_vector_rotate_amd")


def _dev(a, dtype):
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to("cuda")
    return t.to(dtype) if dtype != torch.float32 else t


def _bf16(a):
    return W.bf16_bits_to_f32(W.f32_to_bf16_bits(a))


def _rows(rng, G, N, d=128, outliers=True):
    scale = np.exp(rng.normal(0, math.sqrt(0.5), d))
    if outliers:
        scale[rng.choice(d, 4, replace=False)] *= 20
    return (rng.standard_normal((G, N, d)) * scale).astype(np.float32)


def _encode_values_checked(cb, cbo, v, dtype):
    G, N, d = v.shape
    print(f"[case] value encode G={G} N={N} bits={cb.bits} dtype={dtype}", flush=True)
    vb = K.encode_values(cb, _dev(v, dtype))
    torch.cuda.synchronize()
    buf = vb.cpu().numpy()
    codes, nu16 = O.unpack_values(cbo, buf, G, N)
    check_values(cbo, v.reshape(-1, d), codes.reshape(-1, d), nu16.reshape(-1))
    # the layout itself, padding of the last tile included: the buffer is the
    # oracle's packing of the codes and norms it holds, byte for byte
    assert np.array_equal(buf.view(np.uint8), O.pack_values(cbo, codes, nu16))
    return vb, buf


@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("N", [1, 15, 16, 17, 33, 300])   # 16- and 32-key tile edges
def test_value_encode(bits, dt, N):
    rng = np.random.default_rng(900 + 10 * bits + N + (5 if dt == "bf16" else 0))
    v = _rows(rng, 3, N)
    dtype = torch.bfloat16 if dt == "bf16" else torch.float32
    if dt == "bf16":
        v = _bf16(v)
    cb = K.Codebook(128, bits, 128, 17)
    cbo = O.make_codebook(128, bits, 128, 17)
    _encode_values_checked(cb, cbo, v, dtype)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_value_special_rows(dt):
    """Zero rows, a row below the zero-norm rule, one-hot, constant and
    two-hot rows: exact codes (rotated zeros take the non-negative level)."""
    rng = np.random.default_rng(12)
    v = _bf16(_rows(rng, 1, 40))
    v[0, 0] = 0.0
    v[0, 1] = 0.0
    v[0, 1, 7] = 1e-12
    v[0, 2] = 0.0
    v[0, 2, 90] = -4.0
    v[0, 3] = 0.25
    v[0, 4] = 0.0
    v[0, 4, [3, 4]] = 1.0
    dtype = torch.bfloat16 if dt == "bf16" else torch.float32
    if dt == "bf16":
        v[0, 1, 7] = 0.0            # bf16 keeps 1e-12; the f32 case checks the rule
    cb = K.Codebook(128, 3)
    cbo = O.make_codebook(128, 3, 128, 42)
    _, buf = _encode_values_checked(cb, cbo, v, dtype)
    codes, nu16 = O.unpack_values(cbo, buf, 1, 40)
    ref = O.encode_values(cbo, v[0, :5].astype(np.float64))
    assert not codes[0, :2].any() and float(nu16[0, 0]) == 0.0 and float(nu16[0, 1]) == 0.0
    assert np.array_equal(codes[0, 2:5].astype(np.int64), ref.codes[2:5].astype(np.int64))


def _attention_case(bits, G, N, Qg, dt, seed):
    rng = np.random.default_rng(seed)
    k = _rows(rng, G, N)
    v = _rows(rng, G, N, outliers=False)
    q = rng.standard_normal((G, Qg, 128)).astype(np.float32)
    dtype = torch.bfloat16 if dt == "bf16" else torch.float32
    if dt == "bf16":
        k, v, q = _bf16(k), _bf16(v), _bf16(q)
    cb = K.Codebook(128, bits)
    cbo = O.make_codebook(128, bits, 128, 42)
    print(f"[case] attention bits={bits} G={G} N={N} Qg={Qg} dtype={dt}", flush=True)
    kb = K.encode_keys(cb, _dev(k, dtype))
    vb = K.encode_values(cb, _dev(v, dtype))
    qd = _dev(q, dtype)
    out = K.attention_decode(cb, qd, kb, vb, N)
    lg = K.score_logits(cb, qd, kb, N)
    torch.cuda.synchronize()
    kbuf, vbuf = kb.cpu().numpy(), vb.cpu().numpy()
    out, lg = out.cpu().numpy().astype(np.float64), lg.cpu().numpy().astype(np.float64)
    vhat = O.decode_values(cbo, vbuf, G, N)
    # same logits on both sides
    ref = O.attention_from_logits(cbo, lg, vbuf, G, N)
    err = np.abs(out - ref)
    tol = attention_tolerance(vhat)
    assert np.all(err <= tol), f"worst |delta|/tol = {np.max(err / tol):.3g}"
    # the oracle's own logits: the logit rule bounds the softmax weights
    ref_lg = O.score(cbo, kbuf, G, N, q)
    knorm = np.linalg.norm(k.astype(np.float64), axis=-1)
    check_logits(lg, ref_lg, q, knorm)
    dl = (1e-4 / math.sqrt(128)) * np.linalg.norm(q.astype(np.float64), axis=-1) * knorm.max(axis=1)[:, None]
    ref2 = O.attention_from_logits(cbo, ref_lg, vbuf, G, N)
    tol2 = attention_tolerance(vhat, extra=0.0) + (np.expm1(2 * dl) * np.max(np.linalg.norm(vhat, axis=-1), axis=-1)[:, None])[..., None]
    assert np.all(np.abs(out - ref2) <= tol2)
    return out


@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("N,Qg", [(1, 4), (63, 1), (65, 5), (1000, 8)])
def test_attention_ragged(bits, N, Qg):
    _attention_case(bits, 2, N, Qg, "f32", 1000 + 7 * bits + N + Qg)


def test_attention_value_norm_range():
    """Value norms from 2^-20 to 2^14 (rising and falling along the keys,
    all tiny, all large): the weights' power-of-2 scale follows the largest
    norm a wave has seen, and its sums are rescaled when a later tile raises
    it.  260 groups of 1100 keys put two key tiles on some waves of every
    range."""
    rng = np.random.default_rng(77)
    G, N, Qg = 260, 1100, 4
    k = _rows(rng, G, N)
    v = _rows(rng, G, N, outliers=False)
    v /= np.linalg.norm(v, axis=-1, keepdims=True)
    ramp = np.linspace(-20.0, 12.0, N)
    prof = np.empty((G, N))
    prof[0::4] = ramp
    prof[1::4] = ramp[::-1]
    prof[2::4] = -20.0
    prof[3::4] = 14.0
    v = (v * np.exp2(prof)[..., None]).astype(np.float32)
    q = rng.standard_normal((G, Qg, 128)).astype(np.float32)
    cb = K.Codebook(128, 3)
    cbo = O.make_codebook(128, 3, 128, 42)
    print(f"[case] attention value norm range G={G} N={N}", flush=True)
    kb = K.encode_keys(cb, _dev(k, torch.float32))
    vb = K.encode_values(cb, _dev(v, torch.float32))
    qd = _dev(q, torch.float32)
    out = K.attention_decode(cb, qd, kb, vb, N)
    lg = K.score_logits(cb, qd, kb, N)
    torch.cuda.synchronize()
    vbuf = vb.cpu().numpy()
    out, lg = out.cpu().numpy().astype(np.float64), lg.cpu().numpy().astype(np.float64)
    vhat = O.decode_values(cbo, vbuf, G, N)
    ref = O.attention_from_logits(cbo, lg, vbuf, G, N)
    tol = attention_tolerance(vhat)
    err = np.abs(out - ref)
    assert np.all(err <= tol), f"worst |delta|/tol = {np.max(err / tol):.3g}"


def test_attention_bf16_long():
    _attention_case(3, 3, 5000, 4, "bf16", 4242)


def test_attention_workload1_sampled_groups():
    """The Llama-3.1-8B-shaped decode workload (128 groups x 8192 keys, bf16,
    b = 3) in the benchmark's launch configuration; values drawn like the
    keys; two groups checked against the oracle."""
    wl = W.workload(1)
    cb = K.Codebook(128, 3)
    cbo = O.make_codebook(128, 3, 128, 42)
    keys = torch.from_numpy(W.all_keys(wl).view(np.int16)).cuda().view(torch.bfloat16)
    vals = keys.flip(1).contiguous()          # a different row per position
    q = torch.from_numpy(W.all_queries(wl).view(np.int16)).cuda().view(torch.bfloat16)
    print("[case] attention workload 1", flush=True)
    kb = K.encode_keys(cb, keys)
    vb = K.encode_values(cb, vals)
    out = K.attention_decode(cb, q, kb, vb, wl.N)
    lg = K.score_logits(cb, q, kb, wl.N)
    torch.cuda.synchronize()
    G, N = wl.G, wl.N
    kbuf, vbuf = kb.cpu().numpy(), vb.cpu().numpy()
    for g in (5, 101):
        kg = O.pack(cbo, *[a[g:g + 1] for a in O.unpack(cbo, kbuf, G, N)])
        c, n16 = O.unpack_values(cbo, vbuf, G, N)
        vg = O.pack_values(cbo, c[g:g + 1], n16[g:g + 1])
        ref = O.attention_from_logits(cbo, lg[g:g + 1].cpu().numpy(), vg, 1, N)
        vhat = O.decode_values(cbo, vg, 1, N)
        assert np.all(np.abs(out[g:g + 1].cpu().numpy() - ref) <= attention_tolerance(vhat))
        assert kg.size == O.packed_nbytes(cbo, 1, N)


def test_attention_argument_errors():
    import ctypes
    cb = K.Codebook(128, 3)
    lib = K.library()
    G, Qg, N = 1, 4, 64
    q = torch.zeros((G, Qg, 128), device="cuda")
    kb = torch.zeros(K.packed_nbytes(cb, G, N), dtype=torch.uint8, device="cuda")
    vb = torch.zeros(K.value_packed_nbytes(cb, G, N), dtype=torch.uint8, device="cuda")
    out = torch.empty((G, Qg, 128), device="cuda")
    need = K.attention_workspace_nbytes(cb, G, Qg, N)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    base = (cb.handle, p(q), 0, G, Qg, p(kb), p(vb))
    assert lib.tq_attention_decode(*base, N, 0.1, p(out), p(ws), need - 16, None) == -5
    assert lib.tq_attention_decode(*base, N, 0.0, p(out), p(ws), need, None) == -1
    assert lib.tq_attention_decode(*base, 0, 0.1, p(out), p(ws), need, None) == -1
    assert lib.tq_attention_decode(*base, N, 0.1, p(out), p(ws), need, None) == 0
    cbw = K.Codebook(1024, 4)
    assert lib.tq_encode_values(cbw.handle, p(q), 0, 1, 1, p(vb), None) == -2
    assert K.attention_workspace_nbytes(cbw, G, Qg, N) == 0
    torch.cuda.synchronize()
