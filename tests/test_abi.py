"""The C ABI library loads and exports what include/lsh_attn.h declares, and its
argument checks run on the host (no GPU needed: they return before any HIP call)."""
import ctypes
import os
import re

import pytest

import lsh_attention_hash_amd as lat

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lsh_attn.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(lsh_(?:attn|ffn)_\w+)\s*\(", text)))


def test_header_declares_the_expected_entry_points():
    assert _declared_functions() == sorted(lat.EXPORTED_SYMBOLS)


def test_library_exports_every_declared_symbol():
    lib = lat.load_library()
    for name in _declared_functions():
        assert hasattr(lib, name), name
    with open("/proc/self/maps") as f:
        assert lat.library_path() in f.read()


def test_strerror_is_total():
    lib = lat.load_library()
    for code in range(0, 6):
        assert lib.lsh_attn_strerror(code)
    assert lib.lsh_attn_strerror(-7) == b"unknown status"
    assert lib.lsh_attn_strerror(0) == b"ok"


def _create(**kw):
    lib = lat.load_library()
    base = dict(batch=1, heads=2, seq_len=256, head_dim=64, n_buckets=8, n_rounds=2,
                chunk_len=64, causal=0, dtype=lat.BF16, out_dtype=lat.BF16, flags=0)
    base.update(kw)
    cfg = lat.Config(**base)
    h = ctypes.c_void_p(123)
    rc = lib.lsh_attn_create(ctypes.byref(cfg), ctypes.byref(h))
    return rc, h


@pytest.mark.parametrize("kw,code", [
    (dict(seq_len=100), 1),          # not a multiple of chunk_len
    (dict(seq_len=0), 1),
    (dict(batch=0), 1),
    (dict(heads=-1), 1),
    (dict(n_buckets=3), 1),          # odd
    (dict(n_buckets=0), 1),
    (dict(n_buckets=65538), 1),      # above 65536
    (dict(n_rounds=0), 1),
    (dict(chunk_len=0), 1),
    (dict(causal=2), 1),
    (dict(flags=128), 1),            # unknown flag
    (dict(seq_len=1 << 25, chunk_len=64), 1),
    (dict(head_dim=96), 2),          # valid but not implemented
    (dict(head_dim=256), 2),
    (dict(dtype=7), 2),
    (dict(out_dtype=3), 2),
    (dict(chunk_len=512, seq_len=1024), 2),
])
def test_create_rejects_bad_configs_on_the_host(kw, code):
    rc, h = _create(**kw)
    assert rc == code
    assert h.value is None  # handle cleared on error


def test_null_pointers_are_invalid():
    lib = lat.load_library()
    h = ctypes.c_void_p()
    assert lib.lsh_attn_create(None, ctypes.byref(h)) == 1
    cfg = lat.Config(1, 1, 64, 64, 2, 1, 64, 0, 0, 0, 0)
    assert lib.lsh_attn_create(ctypes.byref(cfg), None) == 1
    assert lib.lsh_attn_forward(None, None, None, None, None, None, None, None, None) == 1
    assert lib.lsh_attn_get_stats(None, None) == 1
    assert lib.lsh_attn_workspace_bytes(None, None) == 1
    assert lib.lsh_attn_destroy(None) == 0


def test_binding_refuses_when_library_missing(monkeypatch, tmp_path):
    monkeypatch.setattr(lat, "_LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(lat, "_lib", None)
    with pytest.raises(RuntimeError, match="not built"):
        lat.load_library()


@pytest.mark.parametrize("kw,code", [
    (dict(max_rows=0), 1),
    (dict(d_model=0), 1),
    (dict(d_ff=-8), 1),
    (dict(chunk_rows=-1), 1),
    (dict(dtype=5), 2),
    (dict(d_model=100), 2),           # not a multiple of 8
    (dict(d_ff=1020), 2),
    # off the matrix-core path (fp32) with a chunk above 2^31 elements
    (dict(dtype=0, max_rows=1 << 22, d_ff=1024), 2),
])
def test_ffn_create_rejects_bad_configs_on_the_host(kw, code):
    lib = lat.load_library()
    base = dict(max_rows=1024, chunk_rows=0, d_model=128, d_ff=512, dtype=lat.BF16)
    base.update(kw)
    cfg = lat.FFNConfig(**base)
    h = ctypes.c_void_p(123)
    assert lib.lsh_ffn_create(ctypes.byref(cfg), ctypes.byref(h)) == code
    assert h.value is None


def test_ffn_null_handle_and_pointers_are_invalid():
    lib = lat.load_library()
    assert lib.lsh_ffn_create(None, None) == 1
    assert lib.lsh_ffn_forward(None, 1, None, None, None, None, None, None, None, None) == 1
    assert lib.lsh_ffn_set_timing(None, 1) == 1
    assert lib.lsh_ffn_workspace_bytes(None, None) == 1
    assert lib.lsh_ffn_destroy(None) == 0


def test_static_forward_rejects_on_the_host():
    """lsh_attn_forward_static checks the config and the size of its workspace
    against the static scratch before any HIP call (fake, aligned pointers:
    nothing is launched)."""
    lib = lat.load_library()
    P = ctypes.c_void_p
    fake = P(4096)

    def call(**kw):
        base = dict(batch=1, heads=2, seq_len=256, head_dim=64, n_buckets=8, n_rounds=2,
                    chunk_len=64, causal=0, dtype=lat.BF16, out_dtype=lat.BF16, flags=0)
        base.update(kw)
        cfg = lat.Config(**base)
        return lib.lsh_attn_forward_static(ctypes.byref(cfg), fake, fake, fake, fake, None,
                                           None, None, None)

    assert call(seq_len=100) == 1                    # invalid config
    assert call(head_dim=96) == 2                    # unsupported shape
    assert call(flags=lat.FLAG_BACKWARD) == 2        # no backward without a handle
    # Text-64K needs ~1.6 GB of workspace: beyond the 64 MiB scratch
    assert call(batch=1, heads=8, seq_len=65536, head_dim=128, n_buckets=1024,
                n_rounds=4, causal=1) == 5
    assert lib.lsh_attn_forward_static(None, fake, fake, fake, fake, None, None, None,
                                       None) == 1
    assert b"static scratch" in lib.lsh_attn_strerror(5)
