"""GPU parity of the paged value pool and of decode attention over paged caches.

Key and value pools share one shuffled page table.  Keys and values are
appended as a prefill chunk and then one token per group per step; the value
records found through the table must pass the oracle's value rules (values
of one 16-value tile arrive in different calls), and nothing outside the
written positions may change.  Attention over the paged caches, with group
lengths that differ (one group empty), must equal the oracle's softmax over
the gathered records: tightly against the paged scorer's logits, and within
the bound the logit tolerance implies against the oracle's own logits.
Invalid table entries drop their positions from the softmax.
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

D = 128
SENTINEL = 0xA5


def _rows(rng, G, N, outliers=True):
    scale = np.exp(rng.normal(0, math.sqrt(0.5), D))
    if outliers:
        scale[rng.choice(D, 4, replace=False)] *= 20
    return (rng.standard_normal((G, N, D)) * scale).astype(np.float32)


def _dev(a, dtype):
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to("cuda")
    return t.to(dtype) if dtype != torch.float32 else t


def _exact(a, dtype):
    if dtype == torch.bfloat16:
        return W.bf16_bits_to_f32(W.f32_to_bf16_bits(a))
    return a


def _i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to("cuda")


def _key_records(cbo, kbuf, num_pages, ps, table, g, n):
    """Compact key records (one group) of logical positions n of group g."""
    codes, signs, nu16, rho16 = O.unpack(cbo, kbuf, num_pages, ps)
    pg, sl = table[g, n // ps], n % ps
    c = np.ascontiguousarray
    return O.pack(cbo, c(codes[pg, sl][None]), c(signs[pg, sl][None]), c(nu16[pg, sl][None]),
                  c(rho16[pg, sl][None]))


def _value_records(cbo, vbuf, num_pages, ps, table, g, n):
    """(compact value records of one group, codes, nu16) of positions n of group g."""
    codes, nu16 = O.unpack_values(cbo, vbuf, num_pages, ps)
    pg, sl = table[g, n // ps], n % ps
    vc, vn = np.ascontiguousarray(codes[pg, sl][None]), np.ascontiguousarray(nu16[pg, sl][None])
    return O.pack_values(cbo, vc, vn), vc[0], vn[0]


def _check_group(cbo, out_g, lg_g, kbuf, vbuf, num_pages, ps, table, g, n, k, q):
    """Attention of group g over positions n against the oracle."""
    L = n.size
    kc = _key_records(cbo, kbuf, num_pages, ps, table, g, n)
    vc, _, _ = _value_records(cbo, vbuf, num_pages, ps, table, g, n)
    vhat = O.decode_values(cbo, vc, 1, L)
    # the paged scorer's logits (the attention's own arithmetic) at the positions
    ref = O.attention_from_logits(cbo, lg_g[None][..., n].astype(np.float64), vc, 1, L)
    err = np.abs(out_g[None] - ref)
    tol = attention_tolerance(vhat)
    assert np.all(err <= tol), f"group {g}: worst |delta|/tol = {np.max(err / tol):.3g}"
    # the oracle's own logits
    ref_lg = O.score(cbo, kc, 1, L, q[g:g + 1])
    knorm = np.linalg.norm(k[g:g + 1, n].astype(np.float64), axis=-1)
    check_logits(lg_g[None][..., n], ref_lg, q[g:g + 1], knorm)
    dl = (1e-4 / math.sqrt(D)) * np.linalg.norm(q[g:g + 1].astype(np.float64), axis=-1) * knorm.max(axis=1)[:, None]
    ref2 = O.attention_from_logits(cbo, ref_lg, vc, 1, L)
    tol2 = attention_tolerance(vhat) + (np.expm1(2 * dl) * np.max(np.linalg.norm(vhat, axis=-1), axis=-1)[:, None])[..., None]
    assert np.all(np.abs(out_g[None] - ref2) <= tol2)


@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("ps", [64, 128])
def test_paged_values_and_attention(bits, dt, ps):
    rng = np.random.default_rng(1200 + 10 * bits + ps + (5 if dt == "bf16" else 0))
    dtype = torch.bfloat16 if dt == "bf16" else torch.float32
    G, Qg, ppg, pre, steps = 5, 6, 4, 100, 5
    num_pages = G * ppg + 3                                 # three spare pages nobody maps
    perm = rng.permutation(num_pages)
    table = perm[:G * ppg].reshape(G, ppg).astype(np.int32)
    spare = perm[G * ppg:]
    cb = K.Codebook(D, bits)
    cbo = O.make_codebook(D, bits, D, 42)
    total = pre + steps
    k = _exact(_rows(rng, G, total), dtype)
    v = _exact(_rows(rng, G, total, outliers=False), dtype)
    q = _exact(rng.standard_normal((G, Qg, D)).astype(np.float32), dtype)
    kd, vd, tdev = _dev(k, dtype), _dev(v, dtype), _i32(table)
    kpool = torch.full((K.paged_pool_nbytes(cb, num_pages, ps),), SENTINEL, dtype=torch.uint8, device="cuda")
    vpool = torch.full((K.paged_value_pool_nbytes(cb, num_pages, ps),), SENTINEL, dtype=torch.uint8,
                       device="cuda")
    print(f"[case] paged attention bits={bits} dt={dt} ps={ps}", flush=True)
    zero = _i32(np.zeros(G, np.int32))
    K.paged_append_keys(cb, kd[:, :pre].contiguous(), kpool, ps, tdev, zero)
    K.paged_append_values(cb, vd[:, :pre].contiguous(), vpool, ps, tdev, zero)
    for s in range(steps):
        at = _i32(np.full(G, pre + s, np.int32))
        K.paged_append_keys(cb, kd[:, pre + s:pre + s + 1].contiguous(), kpool, ps, tdev, at)
        K.paged_append_values(cb, vd[:, pre + s:pre + s + 1].contiguous(), vpool, ps, tdev, at)
    lens = np.array([0, 1, 64, 103, total], np.int32)
    Lmax = 128
    qd = _dev(q, dtype)
    out = K.paged_attention(cb, qd, kpool, vpool, ps, tdev, _i32(lens), Lmax)
    lg = K.paged_score(cb, qd, kpool, ps, tdev, _i32(lens), Lmax)
    torch.cuda.synchronize()
    kbuf, vbuf = kpool.cpu().numpy(), vpool.cpu().numpy()
    out, lg = out.cpu().numpy().astype(np.float64), lg.cpu().numpy()
    # value records of every written position: the oracle's value rules
    n_all = np.arange(total)
    for g in range(G):
        _, vc, vn = _value_records(cbo, vbuf, num_pages, ps, table, g, n_all)
        check_values(cbo, v[g], vc, vn)
    # spare pages untouched in both pools
    vcodes_words = num_pages * (ps // 16) * 16 * bits * D // 32
    vw = vbuf[: vcodes_words * 4].view(np.uint32).reshape(num_pages, -1)
    assert np.all(vw[spare].view(np.uint8) == SENTINEL)
    vnorms = vbuf[vcodes_words * 4:].view(np.uint16).reshape(num_pages, ps)
    assert np.all(vnorms[spare].view(np.uint8) == SENTINEL)
    assert np.all(vnorms[table[:, -1]].view(np.uint8) == SENTINEL)   # the last page of each group: unwritten
    assert np.all(out[0] == 0.0)                                      # an empty group: zeros
    for g in range(1, G):
        _check_group(cbo, out[g], lg[g], kbuf, vbuf, num_pages, ps, table, g, np.arange(int(lens[g])), k, q)


def test_paged_attention_skips_invalid_pages():
    """A group whose second page entry is -1 and one whose entry lies past the
    pool: their positions are neither written nor weighed."""
    rng = np.random.default_rng(4242)
    bits, ps, G, ppg, Qg, total = 3, 64, 3, 3, 4, 180
    num_pages = G * ppg
    table = rng.permutation(num_pages).reshape(G, ppg).astype(np.int32)
    table[1, 1] = -1
    table[2, 2] = num_pages + 5
    cb = K.Codebook(D, bits)
    cbo = O.make_codebook(D, bits, D, 42)
    k = _rows(rng, G, total)
    v = _rows(rng, G, total, outliers=False)
    q = rng.standard_normal((G, Qg, D)).astype(np.float32)
    tdev = _i32(table)
    kpool = torch.zeros(K.paged_pool_nbytes(cb, num_pages, ps), dtype=torch.uint8, device="cuda")
    vpool = torch.full((K.paged_value_pool_nbytes(cb, num_pages, ps),), SENTINEL, dtype=torch.uint8,
                       device="cuda")
    print("[case] paged attention with invalid entries", flush=True)
    zero = _i32(np.zeros(G, np.int32))
    K.paged_append_keys(cb, _dev(k, torch.float32), kpool, ps, tdev, zero)
    K.paged_append_values(cb, _dev(v, torch.float32), vpool, ps, tdev, zero)
    lens = np.full(G, total, np.int32)
    qd = _dev(q, torch.float32)
    out = K.paged_attention(cb, qd, kpool, vpool, ps, tdev, _i32(lens), total).cpu().numpy().astype(np.float64)
    lg = K.paged_score(cb, qd, kpool, ps, tdev, _i32(lens), total).cpu().numpy()
    torch.cuda.synchronize()
    kbuf, vbuf = kpool.cpu().numpy(), vpool.cpu().numpy()
    n = np.arange(total)
    keep = {0: n, 1: n[(n < ps) | (n >= 2 * ps)], 2: n[n < 2 * ps]}
    for g in range(G):
        tg = np.where((table[g] >= 0) & (table[g] < num_pages), table[g], 0)
        _check_group(cbo, out[g], lg[g], kbuf, vbuf, num_pages, ps, tg[None].repeat(G, 0), g, keep[g], k, q)


def test_paged_attention_argument_errors():
    import ctypes
    cb = K.Codebook(D, 3)
    lib = K.library()
    G, Qg, ps, ppg = 2, 4, 64, 2
    num_pages = G * ppg
    kpool = torch.zeros(K.paged_pool_nbytes(cb, num_pages, ps), dtype=torch.uint8, device="cuda")
    vpool = torch.zeros(K.paged_value_pool_nbytes(cb, num_pages, ps), dtype=torch.uint8, device="cuda")
    table = _i32(np.arange(num_pages).reshape(G, ppg))
    lens = _i32(np.full(G, 10, np.int32))
    q = torch.zeros((G, Qg, D), dtype=torch.bfloat16, device="cuda")
    out = torch.empty((G, Qg, D), device="cuda")
    ws = torch.empty(K.attention_workspace_nbytes(cb, G, Qg, 128), dtype=torch.uint8, device="cuda")
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    f = ctypes.c_float(1.0)
    call = lambda Lmax, scale, wsb, page=ps: lib.tq_paged_attention(
        cb.handle, P(q), 1, G, Qg, P(kpool), P(vpool), num_pages, page, P(table), ppg, P(lens), Lmax, scale,
        P(out), P(ws), wsb, None)
    assert call(0, f, ws.numel()) == -1
    assert call(128, ctypes.c_float(0.0), ws.numel()) == -1
    assert call(128, f, 16) == -5
    assert call(128, f, ws.numel(), page=48) == -2
    assert call(128, f, ws.numel()) == 0
    vals = torch.zeros((G, 1, D), dtype=torch.bfloat16, device="cuda")
    pos = _i32(np.zeros(G, np.int32))
    assert lib.tq_paged_append_values(cb.handle, P(vals), 1, G, 1, P(vpool), num_pages, 48, P(table), ppg, P(pos),
                                      None) == -2
    assert lib.tq_paged_append_values(cb.handle, P(vals), 7, G, 1, P(vpool), num_pages, ps, P(table), ppg, P(pos),
                                      None) == -1
    assert lib.tq_paged_append_values(cb.handle, P(vals), 1, G, 0, P(vpool), num_pages, ps, P(table), ppg, P(pos),
                                      None) == 0
    torch.cuda.synchronize()
    # zero caches, lengths 10: uniform weights over zero values
    assert torch.count_nonzero(out) == 0
