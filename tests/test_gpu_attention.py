"""GPU parity of the fused compressed decode attention and the BF16 baseline against the oracle.

Tolerance (stated for the method): per output row, max_d |o - r| / max_d |r| <= 2e-3, and
non-finite positions equal.  Storage-mode invariance is bitwise.
"""
import numpy as np
import pytest
import torch

from decode_attention_kvz_amd import kvz, paged, synth

from gpu_util import (announce, build_layer, check_rows, oracle_attention_rows, report_effective,
                      run_bf16, run_fused, scaled_queries, sm_scale)

pytestmark = pytest.mark.gpu


def _layer(pages, seq_lens, n_comp, seed, arena_bytes=None, flags=0):
    if arena_bytes is None:
        arena_bytes = int(pages.numel() * 2 * 1.05) + (1 << 20)
    arena = paged.SlotArena(arena_bytes)
    return arena, build_layer(arena, pages, seq_lens, n_comp, seed=seed, flags=flags)


@pytest.mark.parametrize("forced_exp,forced_frac", [(12.0, 0.10), (-16.0, 0.10), (0.0, 0.0)])
def test_tiny_config_matches_oracle(forced_exp, forced_frac):
    """1 sequence, 8 query / 2 KV heads, 256 tokens (16 compressed pages), seed 0."""
    announce(f"tiny attention forced=({forced_exp},{forced_frac})")
    pages = synth.kv_pages(1, 17, 2, seed=0, forced_frac=forced_frac, forced_exp=forced_exp,
                           device="cuda")
    q = synth.queries(1, 8, seed=0, device="cuda")
    arena, layer = _layer(pages, [256], [16], seed=0)
    got = run_fused(layer, arena, q, sm_scale()).cpu().numpy()
    ref = oracle_attention_rows(layer, q, sm_scale(), [0])[0]
    worst = check_rows(got[0], ref, what="fused")
    announce(f"  max row rel err {worst:.2e}")


def test_ragged_tails_and_empty_sequences():
    """Sequences with 0..16 tail tokens, with no compressed pages, and of length 0."""
    announce("ragged tails")
    seq_lens = [16 * 5 + 0, 16 * 3 + 1, 16 * 7 + 15, 5, 0, 16 * 2 + 16, 16 * 9 + 8, 16]
    n_comp = [5, 3, 7, 0, 0, 2, 9, 0]
    pages = synth.kv_pages(len(seq_lens), 10, 2, seed=7, forced_frac=0.1, forced_exp=-16.0,
                           device="cuda")
    q = synth.queries(len(seq_lens), 8, seed=7, device="cuda")
    arena, layer = _layer(pages, seq_lens, n_comp, seed=7)
    got = run_fused(layer, arena, q, sm_scale()).cpu().numpy()
    ref = oracle_attention_rows(layer, q, sm_scale(), range(len(seq_lens)))
    for b in range(len(seq_lens)):
        check_rows(got[b], ref[b], what=f"seq {b}")
    assert not got[4].any(), "a sequence of length 0 gives zeros"
    base = run_bf16(layer, q, sm_scale()).cpu().numpy()
    for b in range(len(seq_lens)):
        check_rows(base[b], ref[b], what=f"baseline seq {b}")


@pytest.mark.parametrize("hq,hkv", [(8, 8), (16, 8), (32, 8), (24, 4), (64, 4), (48, 3)])
def test_query_group_sizes(hq, hkv):
    announce(f"group sizes hq={hq} hkv={hkv}")
    bsz = 3
    pages = synth.kv_pages(bsz, 6, hkv, seed=11, forced_frac=0.05, forced_exp=-16.0,
                           device="cuda")
    q = synth.queries(bsz, hq, seed=11, device="cuda")
    seq_lens, n_comp = [16 * 5 + 3, 16 * 2, 16 * 4 + 11], [5, 2, 4]
    arena, layer = _layer(pages, seq_lens, n_comp, seed=11)
    got = run_fused(layer, arena, q, sm_scale()).cpu().numpy()
    ref = oracle_attention_rows(layer, q, sm_scale(), range(bsz))
    for b in range(bsz):
        check_rows(got[b], ref[b], what=f"seq {b}")


def test_storage_mode_invariance_is_bitwise():
    """The same KV stored compressed or all-raw gives bit-identical outputs (lossless)."""
    announce("storage-mode invariance")
    pages = synth.kv_pages(4, 21, 8, seed=12, forced_frac=0.05, device="cuda")
    q = synth.queries(4, 32, seed=12, device="cuda")
    seq_lens, n_comp = [16 * 20 + 7, 16 * 13, 16 * 20 + 16, 16 * 1 + 2], [20, 13, 20, 1]
    arena_a, la = _layer(pages, seq_lens, n_comp, seed=12)
    arena_b, lb = _layer(pages, seq_lens, n_comp, seed=12, flags=kvz.KVZ_ENC_FORCE_RAW)
    for splits in (0, 3):
        oa = run_fused(la, arena_a, q, sm_scale(), splits)
        ob = run_fused(lb, arena_b, q, sm_scale(), splits)
        assert torch.equal(oa, ob)
    st_a, st_b = arena_a.stats(), arena_b.stats()
    assert st_a["live_raw_blocks"] < st_b["live_raw_blocks"] == st_b["live_runs"] * 4


def test_split_count_changes_output_only_by_rounding():
    announce("split invariance")
    pages = synth.kv_pages(2, 41, 8, seed=13, forced_frac=0.05, forced_exp=-16.0, device="cuda")
    q = synth.queries(2, 32, seed=13, device="cuda")
    seq_lens, n_comp = [16 * 40 + 9, 16 * 33], [40, 33]
    arena, layer = _layer(pages, seq_lens, n_comp, seed=13)
    outs = [run_fused(layer, arena, q, sm_scale(), s).cpu().numpy() for s in (1, 2, 5, 17, 0)]
    for o in outs[1:]:
        for b in range(2):
            check_rows(o[b], outs[0][b], tol=1e-5, what="splits")
    ref = oracle_attention_rows(layer, q, sm_scale(), range(2))
    for b in range(2):
        check_rows(outs[-1][b], ref[b], what=f"seq {b}")


@pytest.mark.parametrize("splits", [2, 3, 4])
def test_in_kernel_split_merge_reads_this_calls_partials(splits):
    """Split counts that merge inside the attention kernel: calls alternate between two query
    sets on one workspace, 40 times; every output equals the first one for its queries bit for
    bit (a merge that read a previous call's partials, or missed this call's, would differ),
    and a ragged batch (one sequence cut into more pieces) matches the oracle."""
    announce(f"in-kernel merge, splits={splits}")
    # forced elements tiny (2^-16 sigma): every piece carries real softmax weight, so a stale or
    # missing partial changes the output
    pages = synth.kv_pages(6, 41, 8, seed=15, forced_frac=0.05, forced_exp=-16.0, device="cuda")
    seq_lens, n_comp = [16 * 40 + 7, 16 * 3, 16 * 40, 16 * 22 + 1, 5, 16 * 37 + 16], [40, 3, 40, 22, 0, 37]
    arena, layer = _layer(pages, seq_lens, n_comp, seed=15)
    qs = [synth.queries(6, 32, seed=150 + k, device="cuda") for k in range(2)]
    ws = paged.workspace(6, 32, 8, layer.block_table.shape[1], splits, device="cuda")

    def call(q):
        out = torch.empty((6, 32, 128), dtype=torch.float32, device="cuda")
        kvz.kvz_decode_attention(q, out, arena.arena, layer.meta, layer.block_table,
                                 layer.seq_lens, layer.n_comp, layer.tail, sm_scale(), ws, splits)
        return out
    first = [call(q).clone() for q in qs]
    outs = [call(qs[i % 2]) for i in range(40)]
    torch.cuda.synchronize()
    for i, o in enumerate(outs):
        assert torch.equal(o, first[i % 2]), i
    for k in range(2):
        eff = {}
        ref = oracle_attention_rows(layer, qs[k], sm_scale(), range(6), eff)
        got = first[k].cpu().numpy()
        for b in range(6):
            check_rows(got[b], ref[b], what=f"q{k} seq {b}")
        report_effective({b: e for b, e in eff.items() if b != 4}, f"q{k}")


def test_non_finite_values_propagate_like_the_oracle():
    """NaN and Inf in K and V (stress values): the positions of non-finite outputs equal the
    oracle's."""
    announce("non-finite propagation")
    pages = synth.kv_pages(4, 9, 2, seed=14, forced_frac=0.0, device="cuda")
    bits = pages.view(torch.int16)
    bits[0, 2, 1, 0, 3, 17] = 0x7FC0          # NaN in V: one output dim of head group 0
    bits[1, 4, 0, 1, 5, 3] = 0x7F80           # +Inf in K: scores of head group 1 go non-finite
    bits[2, 8, 1, 0, 2, 40] = -128            # -Inf (0xFF80) in V on the tail page
    q = synth.queries(4, 8, seed=14, device="cuda")
    seq_lens, n_comp = [16 * 8 + 4, 16 * 8 + 4, 16 * 8 + 4, 16 * 8], [8, 8, 8, 8]
    arena, layer = _layer(pages, seq_lens, n_comp, seed=14)
    got = run_fused(layer, arena, q, sm_scale()).cpu().numpy()
    ref = oracle_attention_rows(layer, q, sm_scale(), range(4))
    for b in range(4):
        check_rows(got[b], ref[b], what=f"seq {b}")
    assert not np.isfinite(got[0]).all() and not np.isfinite(got[2]).all()


def _full_size_sampled(bsz, n_pages_total, n_comp_pages, tail_tokens, hq, hkv, u_max, forced,
                       seed, samples, forced_exp=12.0, q_log2_scale=0, min_effective=None):
    """One layer at full shape with the automatic split count: sampled rows against the oracle,
    and every row of the fused kernel bit for bit against the uncompressed kernel (the same
    split count; the restore is exact).  Reports how many keys the checked softmaxes spread
    over and, with min_effective, requires more than that many for every checked head."""
    pages = synth.kv_pages(bsz, n_pages_total, hkv, seed=seed, u_max=u_max, forced_frac=forced,
                           forced_exp=forced_exp, device="cuda")
    q = scaled_queries(synth.queries(bsz, hq, seed=seed, device="cuda"), q_log2_scale)
    seq_lens = [16 * n_comp_pages + tail_tokens] * bsz
    arena, layer = _layer(pages, seq_lens, [n_comp_pages] * bsz, seed=seed)
    got_t = run_fused(layer, arena, q, sm_scale())
    base_t = run_bf16(layer, q, sm_scale())
    torch.cuda.synchronize()
    assert torch.equal(got_t, base_t)
    got, base = got_t.cpu().numpy(), base_t.cpu().numpy()
    eff = {}
    ref = oracle_attention_rows(layer, q, sm_scale(), samples, eff)
    worst = 0.0
    for b in samples:
        worst = max(worst, check_rows(got[b], ref[b], what=f"fused seq {b}"))
        check_rows(base[b], ref[b], what=f"baseline seq {b}")
    announce(f"  max row rel err {worst:.2e}")
    lo = report_effective(eff, f"forced 2^{forced_exp:g} x{forced}, q x2^{q_log2_scale}")
    if min_effective is not None:
        assert lo > min_effective, f"softmax too concentrated for this check: {lo:.1f} keys"
    return arena


# Forced elements: as the workloads specify (+-sigma 2^12, which makes the softmax one-hot and
# checks that the dominant key is found and its V restored), tiny (2^-16 sigma: the blocks still
# go raw but no key dominates) and none.  The broad variants also scale q down by a power of two
# so that every checked head spreads its softmax over more than 10 keys: accumulation over the
# whole context and the split merge weights are then what the check measures.
LLAMA_SAMPLES = [0, 4, 9, 13, 17, 22, 26, 31]
QWEN_SAMPLES = [0, 2, 5, 7, 9, 11, 13, 15]
DATA_VARIANTS = [
    pytest.param(12.0, 1.0, 0, None, id="forced2^12"),
    pytest.param(-16.0, 1.0, 0, None, id="forced2^-16"),
    pytest.param(0.0, 0.0, 0, None, id="unforced"),
    pytest.param(-16.0, 1.0, -3, 10.0, id="forced2^-16-broad"),
    pytest.param(0.0, 0.0, -3, 10.0, id="unforced-broad"),
]


@pytest.mark.parametrize("forced_exp,forced_scale,q_log2,min_eff", DATA_VARIANTS)
def test_llama_shape_layer_sampled(forced_exp, forced_scale, q_log2, min_eff):
    """Batch 32, 32 query / 8 KV heads, 2048 tokens, all pages compressed, 5% of blocks with a
    forced element: one layer at full shape with the automatic split count, 8 sequences."""
    announce(f"llama-shaped layer forced=2^{forced_exp:g} q x2^{q_log2}")
    _full_size_sampled(32, 128, 128, 0, 32, 8, 3.0, 0.05 * forced_scale, 1, LLAMA_SAMPLES,
                       forced_exp, q_log2, min_eff)


@pytest.mark.parametrize("forced_exp,forced_scale,q_log2,min_eff", DATA_VARIANTS)
def test_qwen_shape_8k_layer_sampled(forced_exp, forced_scale, q_log2, min_eff):
    """Batch 16, 32 query / 8 KV heads, 8192 tokens: 511 compressed pages plus a 16-token
    BF16 tail, u~U[-5,5], 5% forced: one layer at full shape (two pieces per sequence, merged
    inside the attention kernel), 8 sequences."""
    announce(f"qwen-shaped 8k layer forced=2^{forced_exp:g} q x2^{q_log2}")
    _full_size_sampled(16, 512, 511, 16, 32, 8, 5.0, 0.05 * forced_scale, 2, QWEN_SAMPLES,
                       forced_exp, q_log2, min_eff)


@pytest.mark.parametrize("forced_exp,forced_scale,q_log2,min_eff", DATA_VARIANTS)
def test_long_context_layer_sampled(forced_exp, forced_scale, q_log2, min_eff):
    """Batch 1, 32 query / 8 KV heads, 131072 tokens: 32 pieces per KV head across the chip,
    merged by the combine kernel's uniform-map path."""
    announce(f"131k-token layer forced=2^{forced_exp:g} q x2^{q_log2}")
    _full_size_sampled(1, 8192, 8192, 0, 32, 8, 3.0, 0.10 * forced_scale, 4, [0],
                       forced_exp, q_log2, min_eff)


@pytest.mark.parametrize("splits", [5, 8, 32, 33])
def test_equal_length_batch_split_merge_matches_oracle(splits):
    """Equal lengths give the uniform split map: up to 32 pieces per sequence the combine
    kernel merges from its speculative loads, above that by its general path.  Non-degenerate
    data (tiny forced elements, q scaled down), every row against the oracle."""
    announce(f"equal-length batch, splits={splits}")
    bsz, n_comp = 4, 96
    pages = synth.kv_pages(bsz, n_comp + 1, 8, seed=18, forced_frac=0.05, forced_exp=-16.0,
                           device="cuda")
    q = scaled_queries(synth.queries(bsz, 32, seed=18, device="cuda"), -2)
    seq_lens = [16 * n_comp + 11] * bsz
    arena, layer = _layer(pages, seq_lens, [n_comp] * bsz, seed=18)
    got_t = run_fused(layer, arena, q, sm_scale(), splits)
    base_t = run_bf16(layer, q, sm_scale(), splits)
    one_t = run_fused(layer, arena, q, sm_scale(), 1)
    torch.cuda.synchronize()
    assert torch.equal(got_t, base_t)
    got, one = got_t.cpu().numpy(), one_t.cpu().numpy()
    eff = {}
    ref = oracle_attention_rows(layer, q, sm_scale(), range(bsz), eff)
    for b in range(bsz):
        check_rows(got[b], ref[b], what=f"seq {b}")
        check_rows(got[b], one[b], tol=1e-5, what=f"seq {b} vs one piece")
    assert report_effective(eff, f"splits {splits}") > 10.0


@pytest.mark.parametrize("splits", [0, 3, 8])
def test_ragged_batch_balanced_splits(splits):
    """Lengths from one page to 40 pages and an empty sequence: long sequences are cut into more
    splits than short ones.  Every row meets the tolerance against the oracle, and the fused
    kernel equals the uncompressed one bit for bit at the same split count."""
    announce(f"ragged batch splits={splits}")
    n_comp = [40, 1, 0, 17, 33, 5]
    seq_lens = [16 * 40 + 3, 16 * 1 + 16, 0, 16 * 17, 16 * 33 + 9, 16 * 5 + 1]
    pages = synth.kv_pages(6, 41, 2, seed=16, forced_frac=0.05, forced_exp=-16.0, device="cuda")
    q = synth.queries(6, 8, seed=16, device="cuda")
    arena, layer = _layer(pages, seq_lens, n_comp, seed=16)
    fused = run_fused(layer, arena, q, sm_scale(), splits)
    base = run_bf16(layer, q, sm_scale(), splits)
    torch.cuda.synchronize()
    assert torch.equal(fused, base)
    ref = oracle_attention_rows(layer, q, sm_scale(), range(6))
    got = fused.cpu().numpy()
    for b in range(6):
        if seq_lens[b] == 0:
            assert (got[b] == 0).all()
        else:
            check_rows(got[b], ref[b], what=f"ragged seq {b}")


@pytest.mark.parametrize("ragged", [True, False])
def test_large_batch_split_map(ragged):
    """72 sequences (more than one wave's worth): the split map scans the batch in two chunks.
    Ragged lengths (some empty) and equal lengths, two splits per sequence on average."""
    announce(f"72-sequence batch ragged={ragged}")
    bsz = 72
    if ragged:
        n_comp = [(7 * i) % 11 for i in range(bsz)]
        seq_lens = [16 * n + 5 * (i % 3) for i, n in enumerate(n_comp)]
    else:
        n_comp = [3] * bsz
        seq_lens = [16 * 3 + 7] * bsz
    pages = synth.kv_pages(bsz, 12, 2, seed=17, forced_frac=0.05, forced_exp=-16.0, device="cuda")
    q = synth.queries(bsz, 4, seed=17, device="cuda")
    arena, layer = _layer(pages, seq_lens, n_comp, seed=17)
    fused = run_fused(layer, arena, q, sm_scale(), 2)
    base = run_bf16(layer, q, sm_scale(), 2)
    torch.cuda.synchronize()
    assert torch.equal(fused, base)
    rows = [b for b in range(bsz) if seq_lens[b] > 0]
    ref = oracle_attention_rows(layer, q, sm_scale(), rows)
    got = fused.cpu().numpy()
    for b in range(bsz):
        if seq_lens[b] == 0:
            assert (got[b] == 0).all()
    for b in rows:
        check_rows(got[b], ref[b], what=f"seq {b}")


def test_breakdown_variants_run_and_full_part_equals_the_call():
    """The measurement entry points: KVZ_PART_ALL is the attention call itself (bit for bit, fused
    and BF16), the load-only and load+restore variants run on the same arguments, write
    nothing to out and leave the merge counters at zero."""
    announce("breakdown variants")
    bsz, n_comp = 6, 40
    pages = synth.kv_pages(bsz, n_comp + 1, 8, seed=19, forced_frac=0.05, forced_exp=-16.0,
                           device="cuda")
    q = synth.queries(bsz, 32, seed=19, device="cuda")
    seq_lens = [16 * n_comp + 7] * bsz
    arena, layer = _layer(pages, seq_lens, [n_comp] * bsz, seed=19)
    want = run_fused(layer, arena, q, sm_scale(), 2)
    want_bf16 = run_bf16(layer, q, sm_scale(), 2)
    ws = paged.workspace(bsz, 32, 8, n_comp, 2)
    got = torch.full_like(want, float("nan"))
    kvz.kvz_decode_attention_part(q, got, arena.arena, layer.meta, layer.block_table,
                                  layer.seq_lens, layer.n_comp, layer.tail, sm_scale(), ws,
                                  kvz.KVZ_PART_ALL, 2)
    torch.cuda.synchronize()
    assert torch.equal(got, want)
    for part in (kvz.KVZ_PART_LOAD, kvz.KVZ_PART_LOAD_RESTORE):
        untouched = torch.full_like(want, -7.0)
        kvz.kvz_decode_attention_part(q, untouched, arena.arena, layer.meta, layer.block_table,
                                      layer.seq_lens, layer.n_comp, layer.tail, sm_scale(), ws,
                                      part, 2)
        torch.cuda.synchronize()
        assert (untouched == -7.0).all()
    assert kvz.kvz_attn_workspace_status(ws) == 0
    assert int(ws[:256 + 4 * bsz * 8].count_nonzero()) == 0
    # the BF16 kernel's variants over the same pages
    nat = torch.zeros((layer.meta.shape[0], 2, 8, 16, 128), dtype=torch.bfloat16, device="cuda")
    for b in range(bsz):
        phys = torch.as_tensor(layer.phys_of[b, :n_comp], device="cuda", dtype=torch.long)
        nat[phys] = layer.pages[b, :n_comp]
    store = paged.pack_bf16_pages(nat)
    got_b = torch.full_like(want, float("nan"))
    kvz.kvz_bf16_decode_attention_part(q, got_b, store, layer.block_table, layer.seq_lens,
                                       layer.n_comp, layer.tail, sm_scale(), ws, 8,
                                       kvz.KVZ_PART_ALL, 2)
    untouched = torch.full_like(want, -7.0)
    kvz.kvz_bf16_decode_attention_part(q, untouched, store, layer.block_table, layer.seq_lens,
                                       layer.n_comp, layer.tail, sm_scale(), ws, 8,
                                       kvz.KVZ_PART_LOAD, 2)
    torch.cuda.synchronize()
    assert torch.equal(got_b, want_bf16)
    assert (untouched == -7.0).all()
    with pytest.raises(kvz.KvzError):
        kvz.kvz_bf16_decode_attention_part(q, untouched, store, layer.block_table, layer.seq_lens,
                                           layer.n_comp, layer.tail, sm_scale(), ws, 8,
                                           kvz.KVZ_PART_LOAD_RESTORE, 2)
