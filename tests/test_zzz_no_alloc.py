"""tq_attention_decode_noalloc (static device scratch, nothing allocated by the
library) against tq_attention_decode with a caller workspace, through the C
ABI: bit-identical outputs on two calls in a row, the second with a smaller
input, and a clear error for sizes beyond the scratch array."""

import ctypes
import math

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
K = pytest.importorskip("kv_cache_vector_rotate_amd")


def _rows(rng, G, N, d=128):
    scale = np.exp(rng.normal(0, math.sqrt(0.5), d))
    scale[rng.choice(d, 4, replace=False)] *= 20
    return torch.from_numpy((rng.standard_normal((G, N, d)) * scale).astype(np.float32)).to("cuda")


@pytest.mark.parametrize("bits", [3, 4])
def test_noalloc_attention_equals_workspace_call(bits):
    rng = np.random.default_rng(4242 + bits)
    cb = K.Codebook(128, bits)
    # two calls in a row on the shared scratch, the second smaller than the first
    for G, Qg, N, dt in ((96, 4, 5000, torch.bfloat16), (5, 6, 333, torch.float32)):
        print(f"[case] noalloc attention bits={bits} G={G} Qg={Qg} N={N}", flush=True)
        keys = _rows(rng, G, N).to(dt)
        vals = _rows(rng, G, N).to(dt)
        q = torch.from_numpy(rng.standard_normal((G, Qg, 128)).astype(np.float32)).to("cuda").to(dt)
        kp = K.encode_keys(cb, keys)
        vp = K.encode_values(cb, vals)
        assert K.attention_workspace_nbytes(cb, G, Qg, N) <= K.attention_noalloc_max_nbytes()
        ref = K.attention_decode(cb, q, kp, vp, N)
        out = torch.full((G, Qg, 128), float("nan"), device="cuda")
        K.attention_decode_noalloc(cb, q, kp, vp, N, out=out)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int32), ref.view(torch.int32))


def test_noalloc_attention_refuses_sizes_beyond_scratch():
    cb = K.Codebook(128, 3)
    lib = K.library()
    G, Qg, N = 128, 4, 20000            # logits alone need 40 MB
    assert K.attention_workspace_nbytes(cb, G, Qg, N) > K.attention_noalloc_max_nbytes()
    small = torch.zeros(4096, dtype=torch.uint8, device="cuda")
    out = torch.zeros(16, dtype=torch.float32, device="cuda")
    p = ctypes.c_void_p(small.data_ptr())
    rc = lib.tq_attention_decode_noalloc(cb.handle, p, K.TQ_F32, G, Qg, p, p, N, 0.1,
                                         ctypes.c_void_p(out.data_ptr()),
                                         ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == -5          # TQ_ERR_WORKSPACE, nothing launched
    torch.cuda.synchronize()
