"""GPU coverage of boundary paths beyond the main parity suite, through the C ABI.

* decode_mse: float32 and bfloat16 outputs at d = 128 and d = 1024 (and a
  zero-padded d of D = 1024) against the oracle's MSE reconstruction;
* the scorer is deterministic: the same call twice gives bit-identical logits,
  at a ragged size and on the full Llama-3.1-8B-shaped decode workload;
* value records on the full Llama-3.1-8B-shaped workload, sampled groups
  checked in full against the oracle's value encoder;
* the vector-search encoder on the whole 16,384-vector subset the oracle
  checks, and on all 1,048,576 vectors in one launch (the benchmark's
  configuration): sampled records against the oracle, a rerun bit-identical;
* the binding refuses buffers smaller than the call reads or writes (the C ABI
  cannot see allocation sizes), before anything is launched.
"""

import math

import numpy as np
import pytest

import oracle as O
from kv_cache_vector_rotate_amd import workloads as W
from parity import check_encode, check_values

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
K = pytest.importorskip("kv_cache_vector_rotate_amd")


def _dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to("cuda")
    return t.to(dtype) if dtype not in (None, torch.float32) else t


def _rows(rng, G, N, d, outliers=True):
    scale = np.exp(rng.normal(0, math.sqrt(0.5), d))
    if outliers:
        scale[rng.choice(d, 4, replace=False)] *= 20
    return (rng.standard_normal((G, N, d)) * scale).astype(np.float32)


def _bf16_to_f64(t):
    bits = t.view(torch.int16).cpu().numpy().view(np.uint16)
    return W.bf16_bits_to_f32(bits).astype(np.float64)


@pytest.mark.parametrize("d,bits", [(128, 2), (128, 3), (128, 4), (1024, 2), (1024, 4), (528, 3)])
def test_decode_mse_f32_and_bf16(d, bits):
    """decode_mse against the oracle: float32 within float32 rounding of the
    reconstruction; bfloat16 within half a bfloat16 ulp of the exact value
    plus that float32 error, and equal to the float32 result rounded to
    nearest even."""
    rng = np.random.default_rng(1000 + d + bits)
    G, N = 2, 77
    keys = _rows(rng, G, N, d)
    keys[1, 3] = 0.0                      # zero record decodes to zeros
    cb = K.Codebook(d, bits, None, 5)
    cbo = O.make_codebook(d, bits, cb.D, 5)
    print(f"[case] decode d={d} bits={bits}", flush=True)
    packed = K.encode_keys(cb, _dev(keys))
    f32 = K.decode_mse(cb, packed, G, N)
    b16 = K.decode_mse(cb, packed, G, N, dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert f32.shape == (G, N, d) and b16.shape == (G, N, d)
    ref = O.decode_mse(cbo, packed.cpu().numpy(), G, N)          # [G, N, d] fp64
    _, _, nu16, _ = O.unpack(cbo, packed.cpu().numpy(), G, N)
    nu = nu16.astype(np.float64)[..., None]
    ferr = 1e-5 * nu                       # float32 butterfly of D terms, scaled by nu~
    got = f32.cpu().numpy().astype(np.float64)
    assert np.all(np.abs(got - ref) <= ferr)
    gb = _bf16_to_f64(b16)
    # half a bfloat16 ulp is at most 2^-8 of the value
    assert np.all(np.abs(gb - ref) <= 2.0 ** -8 * np.abs(ref) + 2 * ferr)
    # and the bfloat16 rows are the float32 rows rounded to nearest even
    assert torch.equal(b16.view(torch.int16), f32.to(torch.bfloat16).view(torch.int16))
    assert not gb[1, 3].any() and not got[1, 3].any()


def test_score_is_deterministic_ragged():
    rng = np.random.default_rng(12)
    G, N, Qg = 3, 1234, 6
    keys = _dev(_rows(rng, G, N, 128), torch.bfloat16)
    q = _dev(rng.standard_normal((G, Qg, 128)), torch.bfloat16)
    for bits in (2, 3, 4):
        cb = K.Codebook(128, bits)
        packed = K.encode_keys(cb, keys)
        a = K.score_logits(cb, q, packed, N).clone()
        b = K.score_logits(cb, q, packed, N)
        torch.cuda.synchronize()
        assert torch.equal(a.view(torch.int32), b.view(torch.int32))


def test_workload1_score_bit_identical_rerun_and_value_records():
    """Llama-3.1-8B-shaped decode workload (128 groups x 8192 bf16 keys, b = 3)
    in the launch configuration the benchmark times: scoring the packed cache
    twice gives bit-identical logits; value records of the same rows (values
    drawn like the keys) match the oracle's value encoder on sampled groups."""
    wl = W.workload(1)
    keys_bits = W.all_keys(wl)
    q_bits = W.all_queries(wl)
    keys = torch.from_numpy(keys_bits.view(np.int16)).to("cuda").view(torch.bfloat16)
    q = torch.from_numpy(q_bits.view(np.int16)).to("cuda").view(torch.bfloat16)
    cb = K.Codebook(128, 3)
    cbo = O.make_codebook(128, 3, 128, 42)
    print("[case] workload 1 score rerun", flush=True)
    packed = K.encode_keys(cb, keys)
    a = K.score_logits(cb, q, packed, wl.N).clone()
    b = K.score_logits(cb, q, packed, wl.N)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))
    print("[case] workload 1 value records", flush=True)
    vals = keys.flip(1).contiguous()
    vb = K.encode_values(cb, vals)
    torch.cuda.synchronize()
    buf = vb.cpu().numpy()
    codes, nu16 = O.unpack_values(cbo, buf, wl.G, wl.N)
    for g in (0, 64, 127):
        vg = W.bf16_bits_to_f32(keys_bits[g][::-1].copy())
        check_values(cbo, vg, codes[g], nu16[g])


def test_search_encode_whole_oracle_subset():
    """The vector-search encoder (d = m = 1024, b = 4) on the first 16,384
    vectors of the 1M-vector workload, every record checked."""
    wl = W.workload(4)
    n = 16384
    keys = W.group_keys(wl, 0, 0, n)[None]
    cbo = O.make_codebook(1024, wl.bits, 1024, 42)
    cb = K.Codebook(1024, wl.bits)
    print("[case] search encode 16384", flush=True)
    packed = K.encode_keys(cb, _dev(keys))
    torch.cuda.synchronize()
    buf = packed.cpu().numpy()
    codes, signs, nu16, rho16 = O.unpack(cbo, buf, 1, n)
    for s0 in range(0, n, 4096):
        sl = slice(s0, s0 + 4096)
        check_encode(cbo, keys[0, sl], codes[0, sl], signs[0, sl], nu16[0, sl], rho16[0, sl])


def test_search_encode_full_size_sampled():
    """All 1,048,576 vectors of the search workload encoded in one launch, as
    the benchmark runs it (every workgroup walks ~128 tiles): ~2,000 sampled
    records (the first and last tiles among them) against the oracle, and a
    second launch bit-identical to the first."""
    wl = W.workload(4)
    N, d, step = wl.N, wl.d, 1 << 16
    rng = np.random.default_rng(404)
    sample = np.unique(np.concatenate([rng.choice(N, 2000, replace=False),
                                       [0, 1, 31, 32, 33, N - 33, N - 32, N - 1]]))
    keys = torch.empty((1, N, d), dtype=torch.float32, device="cuda")
    rows = []
    print("[case] search encode full size: generating", flush=True)
    for s0 in range(0, N, step):
        chunk = W.group_keys(wl, 0, s0, min(step, N - s0))
        keys[0, s0:s0 + chunk.shape[0]] = torch.from_numpy(chunk).to("cuda")
        sel = sample[(sample >= s0) & (sample < s0 + chunk.shape[0])]
        rows.append(chunk[sel - s0])
    host = np.concatenate(rows)
    cb = K.Codebook(d, wl.bits)
    cbo = O.make_codebook(d, wl.bits, d, 42)
    print("[case] search encode full size: encoding", flush=True)
    packed = K.encode_keys(cb, keys)
    again = K.encode_keys(cb, keys)
    torch.cuda.synchronize()
    assert torch.equal(packed, again)
    # records of the sampled vectors, gathered into a packed buffer of their own
    P = wl.bits
    words = packed.view(torch.int32)
    planes = words[:P * N * (d // 32)].view(P, N, d // 32)
    norms = words[P * N * (d // 32):P * N * (d // 32) + N]
    idx = torch.from_numpy(sample).to("cuda")
    sub = torch.cat([planes[:, idx, :].reshape(-1), norms[idx]]).cpu().numpy().view(np.uint8)
    codes, signs, nu16, rho16 = O.unpack(cbo, sub, 1, len(sample))
    check_encode(cbo, host, codes[0], signs[0], nu16[0], rho16[0])


def test_binding_refuses_undersized_buffers():
    rng = np.random.default_rng(5)
    G, N, Qg = 2, 100, 4
    cb = K.Codebook(128, 3)
    keys = _dev(_rows(rng, G, N, 128))
    q = _dev(rng.standard_normal((G, Qg, 128)))
    packed = K.encode_keys(cb, keys)
    short = packed[: packed.numel() - 16]
    vpk = K.encode_values(cb, keys)
    with pytest.raises(ValueError):
        K.score_logits(cb, q, short, N)
    with pytest.raises(ValueError):
        K.score_cache(cb, q, packed, N + 1, N)          # Ncap past the buffer
    with pytest.raises(ValueError):
        K.score_cache(cb, q, packed, N, N + 1)          # length past Ncap
    with pytest.raises(ValueError):
        K.decode_mse(cb, short, G, N)
    with pytest.raises(ValueError):
        K.decode_mse(cb, packed, G, N, out=torch.empty((G, N, 127), device="cuda"))
    with pytest.raises(ValueError):
        K.decode_mse(cb, packed, G, N, out=torch.empty((G, N, 128), device="cuda")[:, :, ::2])
    with pytest.raises(TypeError):
        K.decode_mse(cb, packed, G, N, out=torch.empty((G, N, 128), dtype=torch.float16, device="cuda"))
    with pytest.raises(ValueError):
        K.attention_decode(cb, q, short, vpk, N)
    with pytest.raises(ValueError):
        K.attention_decode(cb, q, packed, vpk[: vpk.numel() - 2], N)
    with pytest.raises(ValueError):
        K.dense_logits_bf16(q.to(torch.bfloat16), keys[:1].to(torch.bfloat16))
    cbw = K.Codebook(1024, 4)
    kw = _dev(_rows(rng, 1, 50, 1024, outliers=False))
    pw = K.encode_keys(cbw, kw)
    with pytest.raises(ValueError):
        K.score_topk(cbw, _dev(rng.standard_normal((1, 3, 1024))), pw[:-4], 50, 5)
    torch.cuda.synchronize()
