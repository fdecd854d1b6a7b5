"""GPU parity of the paged key cache through the C ABI.

Pool pages are assigned to groups in a shuffled order; keys are appended in a
bulk prefill and then one token per group per step (rows of many groups share
an encoder tile), at group positions that differ; the records found through
the page table must be the oracle's encoding of each key (rules of
tests/parity.py) and paged scores must equal the oracle's estimator on those
records.  A ring (logical pages reusing a group's physical pages) covers
wrap-around: after three turns the pages hold the last window, which is
scored through a rotated view of the table.  Table entries outside the pool
and positions past the table are neither written nor scored.
"""

import math

import numpy as np
import pytest

import oracle as O
from kv_cache_vector_rotate_amd import workloads as W
from parity import check_encode, check_logits

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
K = pytest.importorskip("kv_cache_vector_rotate_amd")

D = 128
SENTINEL = 0xA5


def _rows(rng, G, N):
    scale = np.exp(rng.normal(0, math.sqrt(0.5), D))
    scale[rng.choice(D, 4, replace=False)] *= 20
    k = (rng.standard_normal((G, N, D)) * scale).astype(np.float32)
    return k


def _dev(a, dtype):
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to("cuda")
    return t.to(dtype) if dtype != torch.float32 else t


def _exact(a, dtype):
    """Values the GPU sees for keys of this dtype."""
    if dtype == torch.bfloat16:
        return W.bf16_bits_to_f32(W.f32_to_bf16_bits(a))
    return a


def _i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to("cuda")


def _gather(cbo, pool, num_pages, ps, table, g, n):
    """Records (codes, signs, nu16, rho16) of logical positions n of group g."""
    codes, signs, nu16, rho16 = O.unpack(cbo, pool, num_pages, ps)
    pg = table[g, n // ps]
    sl = n % ps
    return codes[pg, sl], signs[pg, sl], nu16[pg, sl], rho16[pg, sl]


@pytest.mark.parametrize("bits,dt,ps", [(3, "bf16", 64), (2, "f32", 128), (4, "bf16", 128), (4, "f32", 64)])
def test_paged_append_and_score(bits, dt, ps):
    rng = np.random.default_rng(500 + 10 * bits + ps + (1 if dt == "bf16" else 0))
    dtype = torch.bfloat16 if dt == "bf16" else torch.float32
    G, ppg, Qg = 6, 5, 5
    num_pages = G * ppg + 3
    perm = rng.permutation(num_pages)
    table = perm[: G * ppg].reshape(G, ppg).astype(np.int32)
    cap = ppg * ps
    cb = K.Codebook(D, bits)
    cbo = O.make_codebook(D, bits, D, 42)
    pool = torch.full((K.paged_pool_nbytes(cb, num_pages, ps),), SENTINEL, dtype=torch.uint8, device="cuda")
    keys = _exact(_rows(rng, G, cap), dtype)
    start = np.array([0, 7, ps, 2 * ps - 1, 3, 0], dtype=np.int64)[:G]
    pre = 2 * ps + 5                                     # bulk prefill: rows [start, start + pre)
    print(f"[case] paged prefill bits={bits} dt={dt} ps={ps}", flush=True)
    K.paged_append_keys(cb, _dev(np.stack([keys[g, start[g]:start[g] + pre] for g in range(G)]), dtype),
                        pool, ps, _i32(table), _i32(start))
    lens = start + pre
    for step in range(20):                               # one token per group per step
        new = np.stack([keys[g, lens[g]:lens[g] + 1] for g in range(G)])
        K.paged_append_keys(cb, _dev(new, dtype), pool, ps, _i32(table), _i32(lens))
        lens = lens + 1
    torch.cuda.synchronize()
    buf = pool.cpu().numpy()
    for g in range(G):
        n = np.arange(start[g], lens[g])
        c, s, nu, rho = _gather(cbo, buf, num_pages, ps, table, g, n)
        check_encode(cbo, keys[g, start[g]:lens[g]], c, s, nu, rho)
    # pages no group maps, and slots never written, keep their old bytes
    spare = perm[G * ppg:]
    per_page = K.paged_pool_nbytes(cb, 1, ps)
    nplane = num_pages * ps * bits * 16
    planes = buf[:nplane].reshape(num_pages, bits, ps, 16)
    assert np.all(planes[spare] == SENTINEL)
    g0 = 1                                               # group 1 starts at 7: slots 0..6 of its first page
    assert np.all(planes[table[g0, 0], :, :start[g0]] == SENTINEL)
    assert per_page * num_pages == buf.size
    # scores of positions [0, len) where all were written (groups starting at 0)
    q = _exact(rng.standard_normal((G, Qg, D)).astype(np.float32), dtype)
    Lmax = int(lens.max()) + 17
    out = torch.full((G, Qg, Lmax), -7.0, device="cuda")
    slens = np.where(start == 0, lens, 0).astype(np.int32)
    print(f"[case] paged score bits={bits} Lmax={Lmax}", flush=True)
    K.paged_score(cb, _dev(q, dtype), pool, ps, _i32(table), _i32(slens), Lmax, out=out)
    torch.cuda.synchronize()
    lg = out.cpu().numpy()
    for g in range(G):
        L = int(slens[g])
        assert np.all(lg[g, :, L:] == -7.0)
        if L == 0:
            continue
        c, s, nu, rho = _gather(cbo, buf, num_pages, ps, table, g, np.arange(L))
        one = O.pack(cbo, c[None], s[None], nu[None], rho[None])
        ref = O.score(cbo, one, 1, L, q[g:g + 1])
        check_logits(lg[g:g + 1, :, :L], ref, q[g:g + 1],
                     np.linalg.norm(keys[g:g + 1, :L].astype(np.float64), axis=-1))


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_paged_bulk_rows_take_the_tile_encoder(dt):
    """A bulk append of more rows than the latency path takes (2048)
    goes through the tile encoder in its paged form: records equal the
    oracle's and the tile encoder's own records from tq_encode_keys."""
    rng = np.random.default_rng(31 + (1 if dt == "bf16" else 0))
    dtype = torch.bfloat16 if dt == "bf16" else torch.float32
    bits, ps, G, ppg, T = 3, 64, 8, 6, 300
    num_pages = G * ppg
    table = rng.permutation(num_pages).reshape(G, ppg).astype(np.int32)
    cb = K.Codebook(D, bits)
    cbo = O.make_codebook(D, bits, D, 42)
    keys = _exact(_rows(rng, G, T), dtype)
    pool = torch.full((K.paged_pool_nbytes(cb, num_pages, ps),), SENTINEL, dtype=torch.uint8, device="cuda")
    print(f"[case] paged bulk dt={dt}", flush=True)
    K.paged_append_keys(cb, _dev(keys, dtype), pool, ps, _i32(table), _i32(np.full(G, 5, np.int32)))
    flat = K.encode_keys(cb, _dev(keys, dtype))
    torch.cuda.synchronize()
    buf = pool.cpu().numpy()
    fc, fs, fn, fr = O.unpack(cbo, flat.cpu().numpy(), G, T)
    for g in range(G):
        c, s_, nu, rho = _gather(cbo, buf, num_pages, ps, table, g, np.arange(5, 5 + T))
        assert np.array_equal(c, fc[g]) and np.array_equal(s_, fs[g])
        assert np.array_equal(nu.view(np.uint16), fn[g].view(np.uint16))
        assert np.array_equal(rho.view(np.uint16), fr[g].view(np.uint16))
        check_encode(cbo, keys[g], c, s_, nu, rho)


def test_paged_ring_wraps_and_scores_the_window():
    """Each group owns R pages; logical page p lives in physical page
    ring[g][p % R], so positions past R pages overwrite the oldest.  After three
    turns the window of the last R pages is scored through a rotated view of
    the table."""
    rng = np.random.default_rng(77)
    bits, ps, R, G, Qg = 3, 64, 3, 4, 4
    turns = 3
    total = turns * R * ps + 2 * ps                      # ends on a page boundary
    num_pages = G * R
    ring = rng.permutation(num_pages).reshape(G, R).astype(np.int32)
    lp = total // ps
    table = np.stack([ring[g][np.arange(lp) % R] for g in range(G)]).astype(np.int32)
    cb = K.Codebook(D, bits)
    cbo = O.make_codebook(D, bits, D, 42)
    pool = torch.zeros(K.paged_pool_nbytes(cb, num_pages, ps), dtype=torch.uint8, device="cuda")
    keys = _exact(_rows(rng, G, total), torch.bfloat16)
    kd = _dev(keys, torch.bfloat16)
    tdev = _i32(table)
    pos = 0
    print("[case] paged ring", flush=True)
    while pos < total:                                   # chunks of 50 tokens, then single tokens
        T = 50 if pos < total - 100 else 1
        T = min(T, total - pos)
        K.paged_append_keys(cb, kd[:, pos:pos + T].contiguous(), pool, ps, tdev,
                            _i32(np.full(G, pos, np.int32)))
        pos += T
    torch.cuda.synchronize()
    buf = pool.cpu().numpy()
    first = lp - R                                       # the window: logical pages [first, lp)
    view = np.stack([ring[g][np.arange(first, lp) % R] for g in range(G)]).astype(np.int32)
    W0 = first * ps
    for g in range(G):
        n = np.arange(R * ps)
        c, s, nu, rho = _gather(cbo, buf, num_pages, ps, view, g, n)
        check_encode(cbo, keys[g, W0:W0 + R * ps], c, s, nu, rho)
    q = rng.standard_normal((G, Qg, D)).astype(np.float32)
    q = _exact(q, torch.bfloat16)
    lens = np.full(G, R * ps, np.int32)
    lg = K.paged_score(cb, _dev(q, torch.bfloat16), pool, ps, _i32(view), _i32(lens), R * ps).cpu().numpy()
    for g in range(G):
        c, s, nu, rho = _gather(cbo, buf, num_pages, ps, view, g, np.arange(R * ps))
        one = O.pack(cbo, c[None], s[None], nu[None], rho[None])
        ref = O.score(cbo, one, 1, R * ps, q[g:g + 1])
        check_logits(lg[g:g + 1], ref, q[g:g + 1],
                     np.linalg.norm(keys[g:g + 1, W0:W0 + R * ps].astype(np.float64), axis=-1))


def test_paged_invalid_entries_are_skipped():
    rng = np.random.default_rng(9)
    bits, ps, G, ppg = 3, 64, 3, 2
    num_pages = 4
    table = np.array([[0, -1], [1, 99], [2, 3]], np.int32)
    cb = K.Codebook(D, bits)
    pool = torch.full((K.paged_pool_nbytes(cb, num_pages, ps),), SENTINEL, dtype=torch.uint8, device="cuda")
    keys = _rows(rng, G, 2 * ps + 10)                    # rows past the table's two pages too
    print("[case] paged invalid entries", flush=True)
    K.paged_append_keys(cb, _dev(keys, torch.float32), pool, ps, _i32(table), _i32(np.zeros(G)))
    torch.cuda.synchronize()
    buf = pool.cpu().numpy()
    nplane = num_pages * ps * bits * 16
    planes = buf[:nplane].reshape(num_pages, bits, ps, 16)
    assert not np.all(planes[0] == SENTINEL) and not np.all(planes[3] == SENTINEL)
    cbo = O.make_codebook(D, bits, D, 42)
    for g, pg in ((0, 0), (1, 1), (2, 2), (2, 3)):
        lpage = int(np.where(table[g] == pg)[0][0])
        n = np.arange(lpage * ps, (lpage + 1) * ps)
        c, s, nu, rho = _gather(cbo, buf, num_pages, ps, table, g, n)
        check_encode(cbo, keys[g, n], c, s, nu, rho)
    q = rng.standard_normal((G, 4, D)).astype(np.float32)
    out = torch.full((G, 4, 2 * ps), -3.0, device="cuda")
    K.paged_score(cb, _dev(q, torch.float32), pool, ps, _i32(table),
                  _i32(np.full(G, 2 * ps, np.int32)), 2 * ps, out=out)
    lg = out.cpu().numpy()
    assert np.all(lg[0, :, ps:] == -3.0) and np.all(lg[1, :, ps:] == -3.0)
    assert np.all(lg[2] != -3.0) and np.all(lg[0, :, :ps] != -3.0)


@pytest.mark.parametrize("rows,dt", [(1, "bf16"), (700, "f32")])
def test_paged_zero_padded_d(rows, dt):
    """d = 96 runs in D = 128 on the paged path too: three single rows take the
    latency kernel, three groups of 700 rows (2100 > 2048) the tile encoder in
    paged form; records and paged scores against the oracle's padded codebook."""
    rng = np.random.default_rng(900 + rows)
    din, bits, ps, G, Qg = 96, 3, 64, 3, 4
    dtype = torch.bfloat16 if dt == "bf16" else torch.float32
    ppg = -(-(rows + 5) // ps)
    num_pages = G * ppg
    table = rng.permutation(num_pages).reshape(G, ppg).astype(np.int32)
    cb = K.Codebook(din, bits)
    cbo = O.make_codebook(din, bits, D, 42)
    assert cb.D == D
    pool = torch.full((K.paged_pool_nbytes(cb, num_pages, ps),), SENTINEL, dtype=torch.uint8, device="cuda")
    x = rng.standard_normal((G, rows, din)) * np.exp(rng.normal(0, math.sqrt(0.5), din))
    x = _exact(x.astype(np.float32), dtype)
    x[0, 0] = 0.0                                        # zero record
    start = np.array([0, 5, 3], dtype=np.int64)
    print(f"[case] paged d=96 rows={rows} dt={dt}", flush=True)
    K.paged_append_keys(cb, _dev(x, dtype), pool, ps, _i32(table), _i32(start))
    torch.cuda.synchronize()
    buf = pool.cpu().numpy()
    for g in range(G):
        c, s, nu, rho = _gather(cbo, buf, num_pages, ps, table, g, np.arange(start[g], start[g] + rows))
        check_encode(cbo, x[g], c, s, nu, rho)
    q = _exact(rng.standard_normal((G, Qg, din)).astype(np.float32), dtype)
    lens = np.array([rows, 0, 0], dtype=np.int32)       # group 0 starts at 0
    out = torch.full((G, Qg, rows), -5.0, device="cuda")
    K.paged_score(cb, _dev(q, dtype), pool, ps, _i32(table), _i32(lens), rows, out=out)
    torch.cuda.synchronize()
    lg = out.cpu().numpy()
    assert np.all(lg[1:] == -5.0)
    c, s, nu, rho = _gather(cbo, buf, num_pages, ps, table, 0, np.arange(rows))
    one = O.pack(cbo, c[None], s[None], nu[None], rho[None])
    check_logits(lg[:1], O.score(cbo, one, 1, rows, q[:1]), q[:1],
                 np.linalg.norm(x[:1].astype(np.float64), axis=-1))


def test_paged_argument_errors():
    cb = K.Codebook(D, 3)
    lib = K.library()
    import ctypes
    buf = torch.zeros(1 << 16, dtype=torch.uint8, device="cuda")
    p = ctypes.c_void_p(buf.data_ptr())
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    # page size not a multiple of 64, non-positive pages, bad dtype
    assert lib.tq_paged_append_keys(cb.handle, p, 0, 1, 1, p, 4, 48, p, 1, p, st) == -2
    assert lib.tq_paged_append_keys(cb.handle, p, 0, 1, 1, p, 0, 64, p, 1, p, st) == -1
    assert lib.tq_paged_append_keys(cb.handle, p, 7, 1, 1, p, 4, 64, p, 1, p, st) == -1
    assert lib.tq_paged_score(cb.handle, p, 0, 1, 300, p, 4, 64, p, 1, p, 64, p, st) == -2
    cbw = K.Codebook(1024, 4)
    assert lib.tq_paged_score(cbw.handle, p, 0, 1, 4, p, 4, 64, p, 1, p, 64, p, st) == -2
    torch.cuda.synchronize()
