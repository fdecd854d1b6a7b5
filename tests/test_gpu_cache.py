"""GPU tests of the write-time cache calls: tq_append_keys and tq_score_cache.

A cache of Ncap records per group is filled in pieces (a prefill chunk, then
one token per decode step).  Appends of up to 2048 keys take the latency
kernel (float32 rotation and projection): its records must pass the oracle's
parity rules and differ from tq_encode_keys's only where those rules flag a
coordinate.  Larger appends take the tile encoder: its records must be
byte-identical to tq_encode_keys's.  No other record may change.  Scoring a
prefix of the cache must equal the oracle's estimator on that prefix.
"""

import ctypes
import math

import numpy as np
import pytest

import oracle as O
from kv_cache_vector_rotate_amd import workloads as W
from parity import check_encode, check_logits

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
K = pytest.importorskip("kv_cache_vector_rotate_amd")

FILL = 0xA5   # bytes of records nobody has written yet


def _dev(a, dtype):
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to("cuda")
    return t.to(dtype) if dtype != torch.float32 else t


def _keys(rng, G, N, d=128):
    scale = np.exp(rng.normal(0, math.sqrt(0.5), d))
    scale[rng.choice(d, 4, replace=False)] *= 20
    return (rng.standard_normal((G, N, d)) * scale).astype(np.float32)


def _records(cbo, buf, G, Ncap):
    """(plane words [G, P, Ncap, 4], norms [G, Ncap]) views of a packed cache."""
    buf = np.asarray(buf).view(np.uint8)
    npl = G * cbo.bits * Ncap * 4
    planes = buf[: npl * 4].view(np.uint32).reshape(G, cbo.bits, Ncap, 4)
    norms = buf[npl * 4:].view(np.uint32).reshape(G, Ncap)
    return planes, norms


def _prefix_buffer(cbo, buf, G, Ncap, L):
    codes, signs, nu16, rho16 = O.unpack(cbo, buf, G, Ncap)
    return O.pack(cbo, codes[:, :L], signs[:, :L], nu16[:, :L], rho16[:, :L])


@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_append_pieces_match_encode(bits, dt):
    rng = np.random.default_rng(500 + bits + (50 if dt == "bf16" else 0))
    G, N, Ncap = 3, 77, 100
    keys = _keys(rng, G, N)
    dtype = torch.bfloat16 if dt == "bf16" else torch.float32
    if dt == "bf16":
        keys = W.bf16_bits_to_f32(W.f32_to_bf16_bits(keys))
    cb = K.Codebook(128, bits, 128, 11)
    cbo = O.make_codebook(128, bits, 128, 11)
    kd = _dev(keys, dtype)
    print(f"[case] append bits={bits} dtype={dt}", flush=True)
    ref = K.encode_keys(cb, kd).cpu().numpy()
    cache = torch.full((K.packed_nbytes(cb, G, Ncap),), FILL, dtype=torch.uint8, device="cuda")
    # a prefill chunk, single decode tokens, then a ragged chunk
    pieces = [(0, 40)] + [(t, 1) for t in range(40, 45)] + [(45, N - 45)]
    for pos, T in pieces:
        K.append_keys(cb, kd[:, pos:pos + T].contiguous(), cache, Ncap, pos)
    torch.cuda.synchronize()
    buf = cache.cpu().numpy()
    pc, nc = _records(cbo, buf, G, Ncap)
    pr, nr = _records(cbo, ref, G, N)
    assert np.all(pc[:, :, N:].view(np.uint8) == FILL) and np.all(nc[:, N:].view(np.uint8) == FILL)
    codes, signs, nu16, rho16 = O.unpack(cbo, buf, G, Ncap)
    check_encode(cbo, keys.reshape(-1, 128), codes[:, :N].reshape(-1, 128),
                 signs[:, :N].reshape(-1, 128), nu16[:, :N].reshape(-1), rho16[:, :N].reshape(-1))
    # the latency kernel against the tile encoder: the same records but for
    # the few the parity rules leave open
    same = np.all(pc[:, :, :N] == pr, axis=(1, 3)) & (nc[:, :N] == nr)
    assert int((~same).sum()) <= 3, f"{int((~same).sum())} of {G * N} records differ from tq_encode_keys"


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_append_bulk_rows_take_the_tile_encoder(dt):
    """An append of more than 2048 keys (3 groups x 700) goes through the tile
    encoder: byte-identical records to tq_encode_keys, at an offset."""
    rng = np.random.default_rng(510 + (1 if dt == "bf16" else 0))
    G, T, Ncap, pos = 3, 700, 750, 33
    keys = _keys(rng, G, T)
    dtype = torch.bfloat16 if dt == "bf16" else torch.float32
    if dt == "bf16":
        keys = W.bf16_bits_to_f32(W.f32_to_bf16_bits(keys))
    cb = K.Codebook(128, 3)
    cbo = O.make_codebook(128, 3, 128, 42)
    kd = _dev(keys, dtype)
    print(f"[case] append bulk dtype={dt}", flush=True)
    cache = torch.full((K.packed_nbytes(cb, G, Ncap),), FILL, dtype=torch.uint8, device="cuda")
    K.append_keys(cb, kd, cache, Ncap, pos)
    ref = K.encode_keys(cb, kd).cpu().numpy()
    torch.cuda.synchronize()
    pc, nc = _records(cbo, cache.cpu().numpy(), G, Ncap)
    pr, nr = _records(cbo, ref, G, T)
    assert np.array_equal(pc[:, :, pos:pos + T], pr) and np.array_equal(nc[:, pos:pos + T], nr)
    assert np.all(pc[:, :, :pos].view(np.uint8) == FILL) and np.all(pc[:, :, pos + T:].view(np.uint8) == FILL)
    assert np.all(nc[:, :pos].view(np.uint8) == FILL) and np.all(nc[:, pos + T:].view(np.uint8) == FILL)


def test_decode_loop_score_cache():
    """One token per group per step into a cache of 300 records; each step
    scores the filled prefix, checked against the oracle on some steps."""
    rng = np.random.default_rng(77)
    G, Qg, Ncap, prefill, steps = 8, 4, 300, 250, 20
    keys = W.bf16_bits_to_f32(W.f32_to_bf16_bits(_keys(rng, G, prefill + steps)))
    q = W.bf16_bits_to_f32(W.f32_to_bf16_bits(rng.standard_normal((steps, G, Qg, 128)).astype(np.float32)))
    cb = K.Codebook(128, 3)
    cbo = O.make_codebook(128, 3, 128, 42)
    kd = _dev(keys, torch.bfloat16)
    cache = torch.zeros(K.packed_nbytes(cb, G, Ncap), dtype=torch.uint8, device="cuda")
    print("[case] decode loop", flush=True)
    K.append_keys(cb, kd[:, :prefill].contiguous(), cache, Ncap, 0)
    out = []
    for s in range(steps):
        L = prefill + s + 1
        K.append_keys(cb, kd[:, L - 1:L].contiguous(), cache, Ncap, L - 1)
        out.append(K.score_cache(cb, _dev(q[s], torch.bfloat16), cache, Ncap, L))
    torch.cuda.synchronize()
    buf = cache.cpu().numpy()
    knorm = np.linalg.norm(keys.astype(np.float64), axis=-1)
    for s in (0, 7, steps - 1):
        L = prefill + s + 1
        ref = O.score(cbo, _prefix_buffer(cbo, buf, G, Ncap, L), G, L, q[s])
        check_logits(out[s].cpu().numpy(), ref, q[s], knorm[:, :L])
    # the same records scored through tq_score_logits on a compact copy agree bit for bit
    L = prefill + steps
    compact = torch.from_numpy(_prefix_buffer(cbo, buf, G, Ncap, L)).cuda()
    full = K.score_logits(cb, _dev(q[-1], torch.bfloat16), compact, L)
    assert torch.equal(full, out[-1])


def test_cache_argument_errors():
    cb = K.Codebook(128, 3)
    lib = K.library()
    G, Ncap = 2, 64
    cache = torch.zeros(K.packed_nbytes(cb, G, Ncap), dtype=torch.uint8, device="cuda")
    keys = torch.zeros((G, 4, 128), dtype=torch.bfloat16, device="cuda")
    q = torch.zeros((G, 4, 128), dtype=torch.bfloat16, device="cuda")
    lg = torch.empty((G, 4, Ncap), device="cuda")
    kp, cp = ctypes.c_void_p(keys.data_ptr()), ctypes.c_void_p(cache.data_ptr())
    assert lib.tq_append_keys(cb.handle, kp, 1, G, 4, cp, Ncap, 61, None) == -1   # past the end
    assert lib.tq_append_keys(cb.handle, kp, 1, G, 4, cp, Ncap, -1, None) == -1
    assert lib.tq_append_keys(cb.handle, kp, 1, G, 0, cp, Ncap, 64, None) == 0    # empty no-op
    assert lib.tq_append_keys(cb.handle, kp, 1, G, 4, cp, Ncap, 60, None) == 0
    qp, lp = ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(lg.data_ptr())
    assert lib.tq_score_cache(cb.handle, qp, 1, G, 4, cp, Ncap, Ncap + 1, lp, None) == -1
    assert lib.tq_score_cache(cb.handle, qp, 1, G, 4, cp, Ncap, 0, lp, None) == 0
    cbw = K.Codebook(1024, 4)
    assert lib.tq_append_keys(cbw.handle, kp, 1, G, 4, cp, Ncap, 0, None) == -2
    assert lib.tq_score_cache(cbw.handle, qp, 1, G, 4, cp, Ncap, 4, lp, None) == -2
    torch.cuda.synchronize()
