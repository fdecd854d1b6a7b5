"""GPU tests of the write-time value cache: tq_append_values and tq_attention_cache.

A value cache of Ncap records per group is filled in pieces: whole 16-value
tiles (the tile encoder of tq_encode_values) and ragged pieces and single
tokens (the per-value latency kernel, which sets a value's bits inside a tile
it shares with other values).  Every appended record must pass the oracle's
value rules, records written by the tile encoder must equal tq_encode_values's
byte for byte, and no other record, nor the rest of a shared tile, may change.
Attention over a prefix of a key and a value cache must equal
tq_attention_decode on compact copies of that prefix bit for bit, and the
oracle's softmax over the prefix within the attention tolerance.
"""

import ctypes
import math

import numpy as np
import pytest

import oracle as O
from kv_cache_vector_rotate_amd import workloads as W
from parity import attention_tolerance, check_logits, check_values

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
K = pytest.importorskip("kv_cache_vector_rotate_amd")

FILL = 0xA5   # bytes of records nobody has written yet


def _dev(a, dtype):
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to("cuda")
    return t.to(dtype) if dtype != torch.float32 else t


def _bf16(a):
    return W.bf16_bits_to_f32(W.f32_to_bf16_bits(a))


def _rows(rng, G, N, d=128):
    scale = np.exp(rng.normal(0, math.sqrt(0.5), d))
    return (rng.standard_normal((G, N, d)) * scale).astype(np.float32)


def _value_prefix(cbo, buf, G, Ncap, L):
    """Compact value records of the first L values of each group of a cache."""
    codes, nu16 = O.unpack_values(cbo, buf, G, Ncap)
    return O.pack_values(cbo, np.ascontiguousarray(codes[:, :L]), np.ascontiguousarray(nu16[:, :L]))


def _key_prefix(cbo, buf, G, Ncap, L):
    codes, signs, nu16, rho16 = O.unpack(cbo, buf, G, Ncap)
    c = np.ascontiguousarray
    return O.pack(cbo, c(codes[:, :L]), c(signs[:, :L]), c(nu16[:, :L]), c(rho16[:, :L]))


def _tile_words(cbo, buf, G, Ncap):
    """uint32 code words of a value cache, [G, tiles, 16 * bits * d / 32]."""
    T = (Ncap + 15) // 16
    nw = G * T * 16 * cbo.bits * cbo.d // 32
    return np.asarray(buf).view(np.uint8)[: nw * 4].view(np.uint32).reshape(G, T, -1)


@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_append_values_pieces(bits, dt):
    rng = np.random.default_rng(600 + bits + (50 if dt == "bf16" else 0))
    G, N, Ncap = 3, 77, 100
    v = _rows(rng, G, N)
    dtype = torch.bfloat16 if dt == "bf16" else torch.float32
    if dt == "bf16":
        v = _bf16(v)
    cb = K.Codebook(128, bits, 128, 11)
    cbo = O.make_codebook(128, bits, 128, 11)
    vd = _dev(v, dtype)
    print(f"[case] append values bits={bits} dtype={dt}", flush=True)
    ref = K.encode_values(cb, vd).cpu().numpy()
    cache = torch.full((K.value_packed_nbytes(cb, G, Ncap),), FILL, dtype=torch.uint8, device="cuda")
    # whole tiles, single tokens, a ragged piece inside one tile, a whole
    # tile, a ragged tail that ends inside a tile
    pieces = [(0, 32)] + [(t, 1) for t in range(32, 40)] + [(40, 8), (48, 16), (64, N - 64)]
    for pos, T in pieces:
        K.append_values(cb, vd[:, pos:pos + T].contiguous(), cache, Ncap, pos)
    torch.cuda.synchronize()
    buf = cache.cpu().numpy()
    codes, nu16 = O.unpack_values(cbo, buf, G, Ncap)
    check_values(cbo, v.reshape(-1, 128), codes[:, :N].reshape(-1, 128), nu16[:, :N].reshape(-1))
    # the tile encoder's pieces: the same records as tq_encode_values
    rcodes, rnu16 = O.unpack_values(cbo, ref, G, N)
    for a, b in ((0, 32), (48, 64)):
        assert np.array_equal(codes[:, a:b], rcodes[:, a:b])
        assert np.array_equal(nu16[:, a:b].view(np.uint16), rnu16[:, a:b].view(np.uint16))
    # the latency kernel's records: norms equal unless flagged by the rules
    # (checked above); nothing past N written
    fill = np.full_like(buf, FILL)
    fcodes, fnu16 = O.unpack_values(cbo, fill, G, Ncap)
    assert np.array_equal(codes[:, N:], fcodes[:, N:]), "codes past the appended values changed"
    assert np.all(nu16[:, N:].view(np.uint8) == FILL), "norms past the appended values changed"
    words = _tile_words(cbo, buf, G, Ncap)
    assert np.all(words[:, (N + 15) // 16:].view(np.uint8) == FILL), "tiles past the last value changed"


def test_append_values_single_tokens_share_tiles():
    """Eight groups, 40 single-token appends each in a scattered order: every
    value lands in a tile whose other values were written before or after it."""
    rng = np.random.default_rng(31)
    G, N = 8, 40
    v = _bf16(_rows(rng, G, N))
    cb = K.Codebook(128, 3)
    cbo = O.make_codebook(128, 3, 128, 42)
    vd = _dev(v, torch.bfloat16)
    cache = torch.full((K.value_packed_nbytes(cb, G, N),), FILL, dtype=torch.uint8, device="cuda")
    print("[case] append values scattered single tokens", flush=True)
    for t in rng.permutation(N):
        K.append_values(cb, vd[:, t:t + 1].contiguous(), cache, N, int(t))
    ref = K.encode_values(cb, vd)
    torch.cuda.synchronize()
    buf = cache.cpu().numpy()
    codes, nu16 = O.unpack_values(cbo, buf, G, N)
    check_values(cbo, v.reshape(-1, 128), codes.reshape(-1, 128), nu16.reshape(-1))
    rcodes, _ = O.unpack_values(cbo, ref.cpu().numpy(), G, N)
    # float32 rotation against the tile encoder's: level indices differ only at
    # coordinates the rules flag (a handful at most)
    assert int((codes != rcodes).sum()) <= 8
    # the padding of the last tile (values 40 .. 47) is untouched
    tail = O.unpack_values(cbo, np.concatenate([buf[: _tile_words(cbo, buf, G, N).nbytes],
                                                np.zeros(2 * G * 48, np.uint8)]), G, 48)[0]
    ftail = O.unpack_values(cbo, np.full(O.value_packed_nbytes(cbo, G, 48), FILL, np.uint8), G, 48)[0]
    assert np.array_equal(tail[:, N:], ftail[:, N:])


@pytest.mark.parametrize("bits", [2, 4])
def test_append_values_padded_width(bits):
    """d = 112 values run in D = 128 (zero padding), both append paths."""
    rng = np.random.default_rng(700 + bits)
    din, G, N, Ncap = 112, 2, 50, 64
    v = _rows(rng, G, N, din)
    cb = K.Codebook(din, bits)
    cbo = O.make_codebook(din, bits, 128, 42)
    vd = _dev(v, torch.float32)
    cache = torch.full((K.value_packed_nbytes(cb, G, Ncap),), FILL, dtype=torch.uint8, device="cuda")
    print(f"[case] append values padded bits={bits}", flush=True)
    for pos, T in ((0, 16), (16, 5), (21, 11), (32, 16), (48, 2)):
        K.append_values(cb, vd[:, pos:pos + T].contiguous(), cache, Ncap, pos)
    torch.cuda.synchronize()
    codes, nu16 = O.unpack_values(cbo, cache.cpu().numpy(), G, Ncap)
    check_values(cbo, v.reshape(-1, din), codes[:, :N].reshape(-1, 128), nu16[:, :N].reshape(-1))


def test_decode_loop_attention_cache():
    """One token per group per step into key and value caches of 300 records;
    each step runs attention over the filled prefix."""
    rng = np.random.default_rng(78)
    G, Qg, Ncap, prefill, steps = 8, 4, 300, 250, 20
    k = _bf16(_rows(rng, G, prefill + steps))
    v = _bf16(_rows(rng, G, prefill + steps))
    q = _bf16(rng.standard_normal((steps, G, Qg, 128)).astype(np.float32))
    cb = K.Codebook(128, 3)
    cbo = O.make_codebook(128, 3, 128, 42)
    kd, vd = _dev(k, torch.bfloat16), _dev(v, torch.bfloat16)
    kc = torch.zeros(K.packed_nbytes(cb, G, Ncap), dtype=torch.uint8, device="cuda")
    vc = torch.full((K.value_packed_nbytes(cb, G, Ncap),), FILL, dtype=torch.uint8, device="cuda")
    print("[case] decode loop with attention over the cache", flush=True)
    K.append_keys(cb, kd[:, :prefill].contiguous(), kc, Ncap, 0)
    K.append_values(cb, vd[:, :prefill].contiguous(), vc, Ncap, 0)
    out, lgs = [], []
    for s in range(steps):
        L = prefill + s + 1
        K.append_keys(cb, kd[:, L - 1:L].contiguous(), kc, Ncap, L - 1)
        K.append_values(cb, vd[:, L - 1:L].contiguous(), vc, Ncap, L - 1)
        qd = _dev(q[s], torch.bfloat16)
        out.append(K.attention_cache(cb, qd, kc, vc, Ncap, L))
        lgs.append(K.score_cache(cb, qd, kc, Ncap, L))
    torch.cuda.synchronize()
    kbuf, vbuf = kc.cpu().numpy(), vc.cpu().numpy()
    L = prefill + steps
    codes, nu16 = O.unpack_values(cbo, vbuf, G, Ncap)
    check_values(cbo, v.reshape(-1, 128), codes[:, :L].reshape(-1, 128), nu16[:, :L].reshape(-1))
    knorm = np.linalg.norm(k.astype(np.float64), axis=-1)
    for s in (0, 9, steps - 1):
        L = prefill + s + 1
        vp = _value_prefix(cbo, vbuf, G, Ncap, L)
        lg = lgs[s].cpu().numpy().astype(np.float64)
        check_logits(lg, O.score(cbo, _key_prefix(cbo, kbuf, G, Ncap, L), G, L, q[s]), q[s], knorm[:, :L])
        ref = O.attention_from_logits(cbo, lg, vp, G, L)
        err = np.abs(out[s].cpu().numpy() - ref)
        tol = attention_tolerance(O.decode_values(cbo, vp, G, L))
        assert np.all(err <= tol), f"step {s}: worst |delta|/tol = {np.max(err / tol):.3g}"
    # compact copies of the last prefix through tq_attention_decode: the same bits
    L = prefill + steps
    kcomp = torch.from_numpy(_key_prefix(cbo, kbuf, G, Ncap, L)).cuda()
    vcomp = torch.from_numpy(_value_prefix(cbo, vbuf, G, Ncap, L)).cuda()
    full = K.attention_decode(cb, _dev(q[-1], torch.bfloat16), kcomp, vcomp, L)
    torch.cuda.synchronize()
    assert torch.equal(full, out[-1])


@pytest.mark.parametrize("L", [1, 17, 64, 65, 299])
def test_attention_cache_prefix_lengths(L):
    """Prefixes that end inside a 16-value tile and a 64-key score tile of a
    cache whose unwritten records hold arbitrary bytes."""
    rng = np.random.default_rng(900 + L)
    G, Qg, Ncap = 3, 5, 300
    k = _rows(rng, G, Ncap)
    v = _rows(rng, G, Ncap)
    q = rng.standard_normal((G, Qg, 128)).astype(np.float32)
    cb = K.Codebook(128, 4)
    cbo = O.make_codebook(128, 4, 128, 42)
    kc = torch.full((K.packed_nbytes(cb, G, Ncap),), FILL, dtype=torch.uint8, device="cuda")
    vc = torch.full((K.value_packed_nbytes(cb, G, Ncap),), FILL, dtype=torch.uint8, device="cuda")
    print(f"[case] attention over a cache prefix L={L}", flush=True)
    K.append_keys(cb, _dev(k[:, :L], torch.float32), kc, Ncap, 0)
    K.append_values(cb, _dev(v[:, :L], torch.float32), vc, Ncap, 0)
    qd = _dev(q, torch.float32)
    out = K.attention_cache(cb, qd, kc, vc, Ncap, L)
    lg = K.score_cache(cb, qd, kc, Ncap, L)
    torch.cuda.synchronize()
    vp = _value_prefix(cbo, vc.cpu().numpy(), G, Ncap, L)
    ref = O.attention_from_logits(cbo, lg.cpu().numpy().astype(np.float64), vp, G, L)
    tol = attention_tolerance(O.decode_values(cbo, vp, G, L))
    assert np.all(np.abs(out.cpu().numpy() - ref) <= tol)
    kcomp = torch.from_numpy(_key_prefix(cbo, kc.cpu().numpy(), G, Ncap, L)).cuda()
    full = K.attention_decode(cb, qd, kcomp, torch.from_numpy(vp).cuda(), L)
    torch.cuda.synchronize()
    assert torch.equal(full, out)


def test_value_cache_argument_errors():
    cb = K.Codebook(128, 3)
    lib = K.library()
    G, Ncap, Qg = 2, 64, 4
    kc = torch.zeros(K.packed_nbytes(cb, G, Ncap), dtype=torch.uint8, device="cuda")
    vc = torch.zeros(K.value_packed_nbytes(cb, G, Ncap), dtype=torch.uint8, device="cuda")
    vals = torch.zeros((G, 4, 128), dtype=torch.bfloat16, device="cuda")
    q = torch.zeros((G, Qg, 128), dtype=torch.bfloat16, device="cuda")
    out = torch.empty((G, Qg, 128), device="cuda")
    ws = torch.empty(K.attention_workspace_nbytes(cb, G, Qg, Ncap), dtype=torch.uint8, device="cuda")
    vp, cp = ctypes.c_void_p(vals.data_ptr()), ctypes.c_void_p(vc.data_ptr())
    assert lib.tq_append_values(cb.handle, vp, 1, G, 4, cp, Ncap, 61, None) == -1   # past the end
    assert lib.tq_append_values(cb.handle, vp, 1, G, 4, cp, Ncap, -1, None) == -1
    assert lib.tq_append_values(cb.handle, vp, 7, G, 4, cp, Ncap, 0, None) == -1    # dtype
    assert lib.tq_append_values(cb.handle, vp, 1, G, 0, cp, Ncap, 64, None) == 0    # empty no-op
    assert lib.tq_append_values(cb.handle, vp, 1, G, 4, cp, Ncap, 60, None) == 0
    qp, kp, op = ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(kc.data_ptr()), ctypes.c_void_p(out.data_ptr())
    wp, wn = ctypes.c_void_p(ws.data_ptr()), ws.numel()
    f = ctypes.c_float(1.0)
    assert lib.tq_attention_cache(cb.handle, qp, 1, G, Qg, kp, cp, Ncap, Ncap + 1, f, op, wp, wn, None) == -1
    assert lib.tq_attention_cache(cb.handle, qp, 1, G, Qg, kp, cp, Ncap, 0, f, op, wp, wn, None) == -1
    assert lib.tq_attention_cache(cb.handle, qp, 1, G, Qg, kp, cp, Ncap, 8, ctypes.c_float(0.0), op, wp, wn,
                                  None) == -1
    assert lib.tq_attention_cache(cb.handle, qp, 1, G, Qg, kp, cp, Ncap, Ncap, f, op, wp, 16, None) == -5
    assert lib.tq_attention_cache(cb.handle, qp, 1, G, Qg, kp, cp, Ncap, Ncap, f, op, wp, wn, None) == 0
    cbw = K.Codebook(1024, 4)
    assert lib.tq_append_values(cbw.handle, vp, 1, G, 4, cp, Ncap, 0, None) == -2
    assert lib.tq_attention_cache(cbw.handle, qp, 1, G, Qg, kp, cp, Ncap, 4, f, op, wp, wn, None) == -2
    torch.cuda.synchronize()
