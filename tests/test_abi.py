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


@pytest.mark.skipif(not os.path.exists(LIB), reason="libkvz.so not built")
def test_pool_capacity_hand_worked():
    """Capacity report from pool counters (host arithmetic), against numbers worked by hand:
    capacity 10000 granules, 3000 used from the frontier, free runs [10, 0, 5, 0, 2], 100 live
    groups holding 40 raw blocks; 2 layers x 4 KV heads -> 16 groups per 16-token page.
      free = 7000 + (10*12 + 5*14 + 2*16) = 7222 granules
      guaranteed groups = 7000 // 16 + min(free runs) = 437 + 0 -> 27 pages, 432 tokens
      expected run = 12 + 4 * 40 / 400 = 12.4 granules -> 7222 / (12.4 * 16) = 36.4 -> 36 pages"""
    from decode_attention_kvz_amd import kvz
    st = {"capacity_granules": 10000, "frontier_granules": 3000, "free_runs": [10, 0, 5, 0, 2],
          "live_runs": 100, "live_granules": 1240, "live_raw_blocks": 40, "enospc": 0,
          "bad_frees": 0}
    c = kvz.kvz_pool_capacity(st, 2, 4)
    assert c["free_granules"] == 7222
    assert c["guaranteed_groups"] == 437 and c["guaranteed_pages"] == 27
    assert c["guaranteed_tokens"] == 432
    assert abs(c["expected_group_granules"] - 12.4) < 1e-12
    assert c["expected_pages"] == 36 and c["expected_tokens"] == 576
    # every bin non-empty: the smallest bin adds to the guarantee
    st["free_runs"] = [10, 3, 5, 7, 2]
    c = kvz.kvz_pool_capacity(st, 2, 4)
    assert c["guaranteed_groups"] == 437 + 2
    # nothing live: assume all-raw runs
    st.update(live_runs=0, live_raw_blocks=0, live_granules=0)
    assert kvz.kvz_pool_capacity(st, 1, 1)["expected_group_granules"] == 16.0
    with pytest.raises(kvz.KvzError):
        kvz.kvz_pool_capacity(st, 0, 4)


@pytest.mark.skipif(not os.path.exists(LIB), reason="libkvz.so not built")
def test_gaac_entry_points_reject_bad_arguments_on_the_host():
    """The second format's calls validate their arguments before anything reaches a device."""
    from decode_attention_kvz_amd import kvz
    lib = kvz._lib
    p = ctypes.c_void_p(256)
    assert lib.kvz_gaac_calibrate(None, 1, p, p, None) == kvz.KVZ_EINVAL          # items null, n > 0
    assert lib.kvz_gaac_calibrate(p, -1, p, p, None) == kvz.KVZ_EINVAL
    assert lib.kvz_gaac_calibrate(p, 1, ctypes.c_void_p(258), p, None) == kvz.KVZ_EINVAL  # hist misaligned
    assert lib.kvz_gaac_encode_pages(None, p, 1, 0, None) == kvz.KVZ_EINVAL       # no pool
    assert lib.kvz_gaac_decompress_pages(p, 4096, p, p, -1, 8, p, None) == kvz.KVZ_EINVAL
    assert lib.kvz_gaac_decompress_pages(p, 4096, p, p, 1, 0, p, None) == kvz.KVZ_EINVAL
    assert lib.kvz_gaac_decompress_pages(p, 4096, ctypes.c_void_p(260), p, 1, 8, p, None) == kvz.KVZ_EINVAL
    assert lib.kvz_gaac_decompress_pages(p, 4096, p, p, 0, 8, p, None) == kvz.KVZ_OK   # nothing to do
    args = kvz.AttnArgs(q=256, out=256, arena=256, arena_bytes=1 << 20, meta=256, n_phys_pages=1,
                        block_table=256, seq_lens=256, n_comp_pages=256, tail=None, batch=1,
                        num_q_heads=8, num_kv_heads=2, head_dim=128, page_size=16, max_pages=1,
                        splits=1, sm_scale=0.1, workspace=256, workspace_bytes=1 << 20)
    assert lib.kvz_gaac_decode_attention(ctypes.byref(args), None, None) == kvz.KVZ_EINVAL   # no bases
    assert lib.kvz_gaac_decode_attention(ctypes.byref(args), ctypes.c_void_p(260), None) == kvz.KVZ_EINVAL
    args.head_dim = 64
    assert lib.kvz_gaac_decode_attention(ctypes.byref(args), p, None) == kvz.KVZ_EUNSUPPORTED


@pytest.mark.skipif(not os.path.exists(LIB), reason="libkvz.so not built")
def test_fp8_entry_points_reject_bad_arguments_on_the_host():
    """The FP8 format's calls validate their arguments before anything reaches a device; an FP8
    pool has twice the granules (128 bytes) of a BF16 pool over the same arena."""
    from decode_attention_kvz_amd import kvz
    lib = kvz._lib
    p = ctypes.c_void_p(256)
    assert kvz.kvz_fp8_pool_state_bytes(1 << 20) >= kvz.kvz_pool_state_bytes(1 << 20)
    with pytest.raises(kvz.KvzError):
        kvz.kvz_fp8_pool_state_bytes(200)                                          # < 2 granules
    assert lib.kvz_fp8_calibrate(p, 1, 7, p, p, None) == kvz.KVZ_EINVAL          # unknown format
    assert lib.kvz_fp8_calibrate(None, 1, 0, p, p, None) == kvz.KVZ_EINVAL       # items null
    assert lib.kvz_fp8_calibrate(p, 1, 1, ctypes.c_void_p(258), p, None) == kvz.KVZ_EINVAL
    assert lib.kvz_fp8_encode_pages(None, p, 1, 0, 0, None) == kvz.KVZ_EINVAL    # no pool
    assert lib.kvz_fp8_decompress_pages(p, 4096, p, p, 1, 8, 2, p, None) == kvz.KVZ_EINVAL
    assert lib.kvz_fp8_decompress_pages(p, 4096, p, p, -1, 8, 0, p, None) == kvz.KVZ_EINVAL
    assert lib.kvz_fp8_decompress_pages(p, 4096, ctypes.c_void_p(260), p, 1, 8, 0, p, None) == kvz.KVZ_EINVAL
    assert lib.kvz_fp8_decompress_pages(p, 4096, p, p, 0, 8, 1, p, None) == kvz.KVZ_OK
    assert lib.kvz_fp8_pack_pages(p, p, -1, 8, None) == kvz.KVZ_EINVAL
    assert lib.kvz_fp8_pack_pages(ctypes.c_void_p(257), p, 1, 8, None) == kvz.KVZ_EINVAL
    assert lib.kvz_fp8_pack_pages(p, p, 0, 8, None) == kvz.KVZ_OK
    args = kvz.Fp8AttnArgs(q=256, out=256, arena=256, arena_bytes=1 << 20, meta=256, bases=None,
                           pages=256, n_phys_pages=1, block_table=256, seq_lens=256,
                           n_comp_pages=256, tail=None, batch=1, num_q_heads=8, num_kv_heads=2,
                           head_dim=128, page_size=16, max_pages=1, splits=1, format=0,
                           sm_scale=0.1, k_scale=1.0, v_scale=1.0, workspace=256,
                           workspace_bytes=1 << 20)
    assert lib.kvz_fp8_decode_attention(None, None) == kvz.KVZ_EINVAL
    assert lib.kvz_fp8_decode_attention(ctypes.byref(args), None) == kvz.KVZ_EINVAL      # no bases
    args.bases = 260
    assert lib.kvz_fp8_decode_attention(ctypes.byref(args), None) == kvz.KVZ_EINVAL      # misaligned
    args.bases, args.arena_bytes = 256, 1024
    assert lib.kvz_fp8_decode_attention(ctypes.byref(args), None) == kvz.KVZ_EINVAL      # arena < 2048
    args.pages = 264
    assert lib.kvz_fp8_raw_decode_attention(ctypes.byref(args), None) == kvz.KVZ_EINVAL  # pages misaligned
    args.format = 3
    assert lib.kvz_fp8_decode_attention(ctypes.byref(args), None) == kvz.KVZ_EINVAL
    assert lib.kvz_fp8_raw_decode_attention(ctypes.byref(args), None) == kvz.KVZ_EINVAL
    args.format, args.head_dim = 1, 64
    assert lib.kvz_fp8_decode_attention(ctypes.byref(args), None) == kvz.KVZ_EUNSUPPORTED


def test_binding_rejects_host_and_misshapen_tensors_before_the_call():
    """The binding checks device-memory arguments (GPU tensor, contiguous, dtype, shape, size)
    before any library call: a host pointer or a short buffer would reach a kernel otherwise."""
    torch = pytest.importorskip("torch")
    from decode_attention_kvz_amd import kvz
    b, hq, hkv = 2, 8, 2
    q = torch.zeros((b, hq, 128), dtype=torch.bfloat16)
    out = torch.zeros((b, hq, 128), dtype=torch.float32)
    meta = torch.zeros((4, hkv, 2, 8), dtype=torch.uint8)
    bt = torch.zeros((b, 4), dtype=torch.int32)
    lens = torch.zeros((b,), dtype=torch.int32)
    ws = torch.zeros((1 << 16,), dtype=torch.uint8)
    with pytest.raises(ValueError, match="GPU tensor"):
        kvz.kvz_decode_attention(q, out, ws, meta, bt, lens, lens, None, 0.1, ws)
    with pytest.raises(ValueError, match="GPU tensor"):
        kvz.kvz_fp8_pack_pages(torch.zeros((1, 2, hkv, 16, 128), dtype=torch.uint8),
                               torch.zeros((1,), dtype=torch.uint8))
    with pytest.raises(ValueError, match="required"):
        kvz.kvz_stream_read(None, None)
    # the argument check itself, on tensors that claim to live on the GPU (no memory is touched)

    class FakeDev:
        def __init__(self, t):
            self.t, self.is_cuda = t, True

        def __getattr__(self, k):
            return getattr(self.t, k)

    dq = FakeDev(q)
    assert kvz._dev("q", dq, dtype=torch.bfloat16, shape=(None, None, 128)) is dq
    with pytest.raises(ValueError, match="must be torch.float32"):
        kvz._dev("out", dq, dtype=torch.float32)
    with pytest.raises(ValueError, match="shape"):
        kvz._dev("out", FakeDev(out[:, :4].contiguous()), shape=(b, hq, 128))
    with pytest.raises(ValueError, match="contiguous"):
        kvz._dev("q", FakeDev(q.transpose(0, 1)))
    with pytest.raises(ValueError, match="at least"):
        kvz._dev("ws", FakeDev(ws), min_bytes=(1 << 16) + 1)
    with pytest.raises(ValueError, match="16 bytes"):
        kvz._check_meta(FakeDev(torch.zeros((4, hkv, 8), dtype=torch.uint8)))


@pytest.mark.skipif(not os.path.exists(LIB), reason="libkvz.so not built")
def test_binding_constants_and_stats_layout_match_the_header():
    """Every KVZ_ constant the binding defines has the header's value, and the binding's pool
    statistics record has the header's fields (all 64-bit: the header's count of uint64_t
    fields, arrays counted by length)."""
    from decode_attention_kvz_amd import kvz
    text = open(HEADER).read()
    defines = {m.group(1): int(m.group(2), 0) for m in
               re.finditer(r"^#define\s+(KVZ_\w+)\s+\(?(-?(?:0x[0-9a-fA-F]+|\d+))u?\)?", text, re.M)}
    checked = 0
    for name, value in defines.items():
        if hasattr(kvz, name):
            assert getattr(kvz, name) == value, name
            checked += 1
    assert checked >= 5
    body = re.search(r"typedef struct \{(.*?)\} kvz_pool_stats_t;", text, re.S).group(1)
    body = re.sub(r"/\*.*?\*/", "", body, flags=re.S)
    n_words = 0
    for m in re.finditer(r"uint64_t\s+(\w+)(?:\[(\d+)\])?;", body):
        n_words += int(m.group(2) or 1)
    assert ctypes.sizeof(kvz.PoolStats) == 8 * n_words
    assert [f[0] for f in kvz.PoolStats._fields_][-1] == "encoder_halted"
