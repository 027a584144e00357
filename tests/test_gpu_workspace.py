"""The attention workspace across calls: one zero-filled workspace reused for calls of different
batch sizes, KV head counts and split counts (merges inside the attention kernel and in the
combine kernel) gives exactly what a fresh workspace gives, and its status word stays clear; a
counter that no zeroed workspace can hold (set from the host) raises the sticky
KVZ_WS_BAD_COUNTER flag, which a new zero-fill clears.  A ragged batch whose long sequence gets
more than four pieces at an in-kernel split count is checked against the oracle."""
import numpy as np
import pytest
import torch

from decode_attention_kvz_amd import kvz, paged, synth

from gpu_util import (announce, build_layer, check_rows, oracle_attention_rows, run_fused,
                      sm_scale)

pytestmark = pytest.mark.gpu

STATUS_BYTES = 256   # the status area at the front of every workspace


def _case(bsz, hkv, n_pages, seed):
    pages = synth.kv_pages(bsz, n_pages + 1, hkv, seed=seed, forced_frac=0.05, forced_exp=-16.0,
                           device="cuda")
    n_comp = [max(1, n_pages - 2 * b) for b in range(bsz)]
    seq_lens = [16 * n + (5 + 3 * b) % 17 for b, n in enumerate(n_comp)]
    arena = paged.SlotArena(bsz * (n_pages + 1) * hkv * 2 * 4096 + (1 << 20))
    layer = build_layer(arena, pages, seq_lens, n_comp, seed=seed)
    q = synth.queries(bsz, 4 * hkv, seed=seed, device="cuda")
    return arena, layer, q


def _call(arena, layer, q, ws, splits):
    out = torch.full((q.shape[0], q.shape[1], 128), float("nan"), dtype=torch.float32,
                     device="cuda")
    kvz.kvz_decode_attention(q, out, arena.arena, layer.meta, layer.block_table, layer.seq_lens,
                             layer.n_comp, layer.tail, sm_scale(), ws, splits)
    return out


def test_one_workspace_reused_across_sizes():
    announce("one workspace reused across batch / head / split changes")
    # (batch, KV heads, pages, splits): growing and shrinking batch * KV heads, in-kernel merges
    # (2..4 splits) and the combine kernel (8), then the first case again
    plan = [(6, 8, 20, 2), (12, 8, 12, 3), (3, 4, 30, 4), (16, 8, 9, 2), (8, 8, 24, 8),
            (2, 2, 40, 3), (6, 8, 20, 2)]
    cases = {}
    need = 0
    for bsz, hkv, n_pages, splits in plan:
        key = (bsz, hkv, n_pages)
        if key not in cases:
            cases[key] = _case(bsz, hkv, n_pages, seed=40 + bsz + hkv)
        need = max(need, kvz.kvz_attn_workspace_bytes(bsz, 4 * hkv, hkv, n_pages, splits))
    shared = torch.zeros(need, dtype=torch.uint8, device="cuda")
    for bsz, hkv, n_pages, splits in plan:
        arena, layer, q = cases[(bsz, hkv, n_pages)]
        got = _call(arena, layer, q, shared, splits)
        fresh = _call(arena, layer, q, paged.workspace(bsz, 4 * hkv, hkv, n_pages, splits), splits)
        torch.cuda.synchronize()
        assert torch.equal(got, fresh), (bsz, hkv, n_pages, splits)
    assert kvz.kvz_attn_workspace_status(shared) == 0
    # the counters and the status word are zero again after the calls
    assert int(shared[:STATUS_BYTES + 4 * 16 * 8].count_nonzero()) == 0


def test_bad_counter_sets_sticky_flag():
    announce("workspace status: a counter set from the host")
    arena, layer, q = _case(6, 8, 20, seed=47)
    ws = paged.workspace(6, 32, 8, 20, 2)
    want = _call(arena, layer, q, ws, 2)
    assert kvz.kvz_attn_workspace_status(ws) == 0
    # counters of (sequence 0..5, KV head 0) set to a count no zeroed workspace holds: the
    # pieces of those pairs see it, none of them merges, every kernel exits normally
    cnt = ws[STATUS_BYTES:STATUS_BYTES + 4 * 6 * 8].view(torch.int32)
    cnt[:6].fill_(1000)
    _call(arena, layer, q, ws, 2)
    flags = kvz.kvz_attn_workspace_status(ws)
    assert flags & kvz.KVZ_WS_BAD_COUNTER
    _call(arena, layer, q, ws, 2)   # still set: the flag is sticky
    assert kvz.kvz_attn_workspace_status(ws) & kvz.KVZ_WS_BAD_COUNTER
    ws.zero_()
    again = _call(arena, layer, q, ws, 2)
    torch.cuda.synchronize()
    assert kvz.kvz_attn_workspace_status(ws) == 0
    assert torch.equal(again, want)


def test_ragged_long_sequence_merges_more_than_four_pieces():
    """At an in-kernel split count (4) the balanced map gives the long sequence most of the
    batch's pieces; its merge takes them four at a time."""
    announce("ragged batch: one long sequence, many pieces merged in the kernel")
    bsz, hkv = 4, 4
    n_comp = [120, 2, 1, 3]
    seq_lens = [16 * n + t for n, t in zip(n_comp, [7, 16, 0, 9])]
    pages = synth.kv_pages(bsz, 121, hkv, seed=48, forced_frac=0.05, forced_exp=-16.0,
                           device="cuda")
    q = synth.queries(bsz, 4 * hkv, seed=48, device="cuda")
    arena = paged.SlotArena(bsz * 121 * hkv * 2 * 4096 + (1 << 20))
    layer = build_layer(arena, pages, seq_lens, n_comp, seed=48)
    got_t = run_fused(layer, arena, q, sm_scale(), 4)
    one_t = run_fused(layer, arena, q, sm_scale(), 1)
    torch.cuda.synchronize()
    got, one = got_t.cpu().numpy(), one_t.cpu().numpy()
    ref = oracle_attention_rows(layer, q, sm_scale(), range(bsz))
    for b in range(bsz):
        check_rows(got[b], ref[b], what=f"seq {b}")
        check_rows(got[b], one[b], tol=1e-5, what=f"seq {b} vs one piece")
    assert np.isfinite(got).all()
