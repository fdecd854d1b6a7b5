"""CPU tests of the C-ABI library: it loads, exports every declared entry
point, its host-side tables agree with the oracle's independent ones, and its
argument validation returns the documented status codes (no GPU needed)."""

import ctypes
import os
import re

import numpy as np
import pytest

import oracle as O
import kv_cache_vector_rotate_amd as K

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    txt = open(os.path.join(ROOT, "include", "tq.h")).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(tq_[a-z0-9_]+)\s*\(", txt)))


def test_library_exports_every_declared_symbol():
    lib = K.library()
    declared = _declared()
    assert declared, "no declarations parsed"
    assert sorted(K.EXPORTED_SYMBOLS) == declared
    for name in declared:
        assert hasattr(lib, name), name


@pytest.mark.parametrize("d,bits,seed", [(128, 2, 42), (128, 3, 42), (128, 4, 1), (1024, 4, 42), (32, 3, 5)])
def test_host_tables_match_oracle(d, bits, seed):
    t = K.codebook_tables(d, bits, d, seed)
    cb = O.make_codebook(d, bits, d, seed)
    assert np.max(np.abs(t["levels"] - cb.levels)) < 1e-12 / np.sqrt(d)
    assert np.max(np.abs(t["thresholds"] - cb.thresholds)) < 1e-12 / np.sqrt(d)
    assert np.array_equal(t["delta"], cb.delta)
    assert np.array_equal(t["S_rot"], cb.S_rot)                      # bit-identical draws
    assert np.max(np.abs(t["S"] - cb.S)) < 1e-12
    assert np.max(np.abs(t["S"] @ cb.R.T - cb.S_rot)) < 1e-12


def test_host_tables_reject_unsupported():
    lib = K.library()
    for d, bits, m in ((100, 3, 100), (8192, 3, 8192), (128, 5, 128), (128, 1, 128), (128, 3, 64), (16, 3, 16)):
        assert lib.tq_codebook_tables(d, bits, m, 1, None, None, None, None, None) == -2


def test_argument_validation_without_gpu():
    lib = K.library()
    # null out-pointer
    assert lib.tq_make_codebook(128, 3, 128, 1, None) == -1
    # unsupported parameters are rejected before any device work
    h = ctypes.c_void_p()
    assert lib.tq_make_codebook(256, 3, 256, 1, ctypes.byref(h)) == -2
    assert lib.tq_make_codebook(128, 3, 64, 1, ctypes.byref(h)) == -2
    assert h.value is None
    # null codebook
    assert lib.tq_encode_keys(None, None, 0, 1, 1, None, None) == -1
    assert lib.tq_score_logits(None, None, 0, 1, 1, None, 1, None, None, 0, None) == -1
    assert lib.tq_decode_mse(None, None, 1, 1, None, 0, None) == -1
    assert lib.tq_append_keys(None, None, 0, 1, 1, None, 8, 0, None) == -1
    assert lib.tq_score_cache(None, None, 0, 1, 1, None, 8, 8, None, None) == -1
    assert lib.tq_codebook_export(None, None, None, None, None, None) == -1
    assert lib.tq_codebook_info(None, None, None, None, None) == -1
    assert lib.tq_packed_bytes(None, 1, 1) == 0
    assert lib.tq_score_workspace_bytes(None, 1, 1) == 0
    lib.tq_free_codebook(None)
    # comparator: unsupported shapes, empty no-op, null pointers
    assert lib.tq_dense_logits_bf16(None, None, 1, 4, 1, 64, None, None) == -2
    assert lib.tq_dense_logits_bf16(None, None, 1, 9, 1, 128, None, None) == -2
    assert lib.tq_dense_logits_bf16(None, None, 0, 4, 1, 128, None, None) == 0
    assert lib.tq_dense_logits_bf16(None, None, 1, 4, 1, 128, None, None) == -1
    assert lib.tq_dense_logits_bf16(None, None, -1, 4, 1, 128, None, None) == -1


def test_status_strings():
    lib = K.library()
    for code in (0, -1, -2, -3, -4, -5, -99):
        s = lib.tq_status_string(code)
        assert isinstance(s, bytes) and s
    assert lib.tq_last_hip_error() == 0


def test_packed_bytes_formula():
    """The record holds (bits-1) code planes, one sign plane and two halves."""
    for d, bits in ((128, 2), (128, 3), (128, 4), (1024, 4)):
        kb, _ = O.kv_bytes_per_vector(d, bits)
        assert kb == (bits - 1) * d // 8 + d // 8 + 4
    assert O.kv_bytes_per_vector(128, 3)[0] == 52
    assert O.kv_bytes_per_vector(1024, 4)[0] == 516


def test_rotation_dim_and_padded_tables():
    """Zero padding to the next power of two [ICLR 2026 digest, 実装のポイント]:
    the host rule, and the padded codebook's tables are the D-dimensional
    oracle's (same seed)."""
    lib = K.library()
    for d, D in ((96, 128), (80, 128), (112, 128), (128, 128), (32, 32), (16, 32), (48, 64),
                 (768, 1024), (1008, 1024), (1024, 1024), (100, 0), (1000, 0), (1040, 2048),
                 (1536, 2048), (2048, 2048), (3072, 4096), (4096, 4096), (4100, 0), (8192, 0), (0, 0)):
        assert lib.tq_rotation_dim(d) == D, d
        assert K.rotation_dim(d) == D
    for d in (96, 768, 1536):
        D = lib.tq_rotation_dim(d)
        t = K.codebook_tables(d, 4, D, 42)
        cb = O.make_codebook(d, 4, D, 42)
        assert cb.d == D and cb.din == d
        assert np.max(np.abs(t["levels"] - cb.levels)) < 1e-12 / np.sqrt(D)
        assert np.array_equal(t["delta"], cb.delta)
        assert np.array_equal(t["S_rot"], cb.S_rot)
        assert np.max(np.abs(t["S"] - cb.S)) < 1e-12
    # m must be the padded dimension; 256 and 512 have no device kernels
    assert lib.tq_codebook_tables(96, 3, 96, 1, None, None, None, None, None) == -2
    h = ctypes.c_void_p()
    assert lib.tq_make_codebook(192, 3, 256, 1, ctypes.byref(h)) == -2
    assert lib.tq_make_codebook(48, 3, 64, 1, ctypes.byref(h)) == -2


def test_padded_beta_tables_are_the_power_of_two_tables():
    a = K.codebook_tables(96, 3, 128, 42, kind="beta")
    b = K.codebook_tables(128, 3, 128, 42, kind="beta")
    for f in ("levels", "thresholds", "delta", "S", "S_rot"):
        assert np.array_equal(a[f], b[f]), f
