"""The C-ABI library loads and exports every entry point include/kvz.h declares (no GPU).

No compute call is made here; it only loads the shared object and looks up symbols.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvz.h")
LIB = os.path.join(ROOT, "decode_attention_kvz_amd", "libkvz.so")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(kvz_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_boundary():
    names = _declared()
    for need in ("kvz_encode_pages", "kvz_decode_block", "kvz_decode_attention",
                 "kvz_slot_alloc", "kvz_slot_free", "kvz_bf16_decode_attention"):
        assert need in names


@pytest.mark.skipif(not os.path.exists(LIB), reason="libkvz.so not built")
def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(LIB)
    missing = [n for n in _declared() if not hasattr(lib, n)]
    assert not missing, missing
    assert lib.kvz_version() == 1


@pytest.mark.skipif(not os.path.exists(LIB), reason="libkvz.so not built")
def test_binding_names_match_the_header():
    from decode_attention_kvz_amd import kvz
    assert sorted(kvz.EXPORTED) == _declared()
    for n in kvz.EXPORTED:
        assert callable(getattr(kvz, n))


@pytest.mark.skipif(not os.path.exists(LIB), reason="libkvz.so not built")
def test_host_side_argument_checks_without_a_gpu():
    """Size queries and argument validation run on the host only."""
    from decode_attention_kvz_amd import kvz
    assert kvz.kvz_pool_state_bytes(1 << 20) > 256
    with pytest.raises(kvz.KvzError) as e:
        kvz.kvz_pool_state_bytes(100)
    assert e.value.code == kvz.KVZ_EINVAL
    assert kvz.kvz_attn_workspace_bytes(16, 32, 8, 512, 16) >= 16 * 8 * 16 * 4 * 130 * 4
    with pytest.raises(kvz.KvzError):
        kvz.kvz_attn_workspace_bytes(-1, 32, 8, 512, 0)
    # the streaming-read reference rejects bad arguments before anything reaches the device
    lib = kvz._lib
    assert lib.kvz_stream_read(None, 16, None, 0, None) == kvz.KVZ_EINVAL
    assert lib.kvz_stream_read(ctypes.c_void_p(256), 24, ctypes.c_void_p(256), 0, None) == kvz.KVZ_EINVAL
    assert lib.kvz_stream_read(ctypes.c_void_p(256), 32, ctypes.c_void_p(256), -1, None) == kvz.KVZ_EINVAL
