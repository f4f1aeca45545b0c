"""Host-side checks that need no GPU: the C-ABI library loads and exports every
declared entry point, and the planner builds, balances and validates schedules
(dry runs) or rejects shapes it cannot tile."""

import ctypes
import os
import re

import pytest

from tile_scheduled_persistent_amd import tiles
from tile_scheduled_persistent_amd.configs import LLAMA_1B, QWEN3_06B, QWEN3_4B, TINY, WORKLOADS, scaled

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    names = set()
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            text = open(os.path.join(ROOT, "include", fn)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names.update(re.findall(r"\b(tiles_[a-z_]+)\s*\(", text))
    return sorted(names)


def test_library_exports_every_declared_symbol():
    L = tiles.lib()
    declared = _declared_functions()
    assert "tiles_plan_create" in declared and "tiles_decode" in declared and "tiles_plan_destroy" in declared
    missing = [n for n in declared if not hasattr(L, n)]
    assert not missing, missing


def test_null_arguments_are_rejected_without_a_gpu():
    L = tiles.lib()
    assert L.tiles_decode(None, None, 0, 1, None, None) == tiles.TILES_E_ARG
    assert L.tiles_decode_noalloc(None, None, 0, 1, None, None) == tiles.TILES_E_ARG
    assert L.tiles_decode_sampled(None, None, 0, 1, None, None, None) == tiles.TILES_E_ARG
    assert L.tiles_verify(None, None, None, 1, None, None) == tiles.TILES_E_ARG
    assert "null" in tiles.last_error()
    assert L.tiles_plan_create(None, None) is None
    L.tiles_plan_destroy(None)  # NULL-safe
    assert L.tiles_plan_status(None) == tiles.TILES_E_ARG
    assert L.tiles_plan_debug_spin_limit(None, 1) == tiles.TILES_E_ARG
    assert L.tiles_plan_debug_corrupt(None) == tiles.TILES_E_ARG
    # the stream-read helper checks its arguments before touching the device
    assert L.tiles_stream_read(None, 1 << 20, 1, None, None) == tiles.TILES_E_ARG
    assert L.tiles_stream_read(1, 1 << 20, 0, 1, None) == tiles.TILES_E_ARG      # no workgroups
    assert L.tiles_stream_read(1, 1000, 1, 1, None) == tiles.TILES_E_ARG         # not whole 8 KB per wavefront
    assert "multiple" in tiles.last_error()
    # the edge-latency helper too
    assert L.tiles_edge_latency(None, 1, 10, 100, None, None) == tiles.TILES_E_ARG
    assert L.tiles_edge_latency(1, 0, 10, 100, 1, None) == tiles.TILES_E_ARG       # peer is not workgroup 0
    assert L.tiles_edge_latency(1, 256, 10, 100, 1, None) == tiles.TILES_E_ARG
    assert L.tiles_edge_latency(1, 8, 0, 100, 1, None) == tiles.TILES_E_ARG        # no round trips
    assert L.tiles_edge_latency(1, 8, 10, 0, 1, None) == tiles.TILES_E_ARG         # no polls allowed
    assert "spin_limit" in tiles.last_error()


@pytest.mark.parametrize("key", list(WORKLOADS))
def test_dry_run_every_workload(key):
    wl = WORKLOADS[key]
    m = wl.model
    info = tiles.dry_run(m, wl.capacity, n_workers=256)
    per = 5 if info.combine_mode == 1 else 6
    assert info.waves_per_step == per * m.n_layers + 1
    assert info.n_workers == 256 and info.block_threads == 512
    assert 84 * 1024 <= info.lds_bytes <= 160 * 1024
    assert info.weight_bytes_per_step == m.weight_bytes_per_token()
    # balanced over each GEMV wave's busy workers (the planner's validator enforces "within one row
    # of a perfect split" itself; o_proj tiles may hold ~6 rows each, so one row is up to ~17 %)
    assert info.max_over_mean < 1.2
    assert info.kv_splits >= 1 and info.kv_splits * m.n_kv_heads <= 256


def test_dry_run_is_deterministic():
    a = tiles.dry_run(LLAMA_1B, 1087)
    b = tiles.dry_run(LLAMA_1B, 1087)
    assert a.checksum == b.checksum
    c = tiles.dry_run(LLAMA_1B, 1088)
    assert c.checksum != a.checksum


def test_llama_wave_geometry():
    info = tiles.dry_run(LLAMA_1B, 1087)
    # 12 QKV rows, 8 o_proj rows, 32 gate/up pairs, 8 down rows, 501 vocab rows per worker
    assert info.packed_bytes >= LLAMA_1B.weight_bytes_per_token() - 2 * LLAMA_1B.hidden


@pytest.mark.parametrize("kw", [dict(kv_splits=1, combine_mode=1), dict(kv_splits=8, combine_mode=2),
                                dict(kv_splits=32, combine_mode=2)])
def test_forced_split_and_combine_modes(kw):
    info = tiles.dry_run(QWEN3_4B, 1087, **kw)
    assert info.kv_splits == kw["kv_splits"]
    assert info.combine_mode == kw["combine_mode"]


@pytest.mark.parametrize("bad, code", [
    (dict(head_dim=96), tiles.TILES_E_CONFIG),
    (dict(n_kv_heads=3), tiles.TILES_E_CONFIG),
    (dict(n_heads=40, n_kv_heads=8), tiles.TILES_E_CONFIG),   # 5 query heads per KV head
    (dict(n_layers=0), tiles.TILES_E_CONFIG),
])
def test_untileable_shapes_are_rejected(bad, code):
    m = scaled(TINY, **bad)
    with pytest.raises(tiles.TilesError) as e:
        tiles.dry_run(m, 32)
    assert e.value.code == code


def test_attention_heads_per_tile():
    # planner choice: the group's query heads spread over as many tiles as the workers allow
    assert tiles.dry_run(LLAMA_1B, 1087).attn_heads == 1
    for t in (1, 2, 4):
        info = tiles.dry_run(LLAMA_1B, 1087, attn_heads=t)
        assert info.attn_heads == t
    with pytest.raises(tiles.TilesError) as e:
        tiles.dry_run(LLAMA_1B, 1087, attn_heads=3)  # does not divide the 4 query heads per KV head
    assert e.value.code == tiles.TILES_E_CONFIG
    with pytest.raises(tiles.TilesError) as e:
        tiles.dry_run(LLAMA_1B, 1087, kv_splits=16, attn_heads=1)  # 8 x 4 x 16 tiles > 256 workers
    assert e.value.code == tiles.TILES_E_CONFIG


def test_kv_capacity_limit():
    tiles.dry_run(TINY, 1 << 23)
    with pytest.raises(tiles.TilesError) as e:
        tiles.dry_run(TINY, (1 << 23) + 1)
    assert e.value.code == tiles.TILES_E_CONFIG


def test_too_many_splits_rejected():
    with pytest.raises(tiles.TilesError) as e:
        tiles.dry_run(LLAMA_1B, 1087, kv_splits=33)
    assert e.value.code == tiles.TILES_E_CONFIG


def test_ragged_shape_plans():
    m = scaled(TINY, name="ragged", n_layers=3, hidden=384, n_heads=6, n_kv_heads=2, ffn=1000, vocab=1000)
    info = tiles.dry_run(m, 40)
    assert info.weight_bytes_per_step == m.weight_bytes_per_token()


def test_small_worker_counts_plan():
    for W in [16, 37, 100]:
        info = tiles.dry_run(QWEN3_06B, 200, n_workers=W)
        assert info.n_workers == W


def test_o_proj_placement():
    # planner choice and 1: all workers; 2: exactly the workers without an attention tile
    wl = WORKLOADS["llama1b"]
    for op in (0, 1):
        assert tiles.dry_run(wl.model, wl.capacity, o_placement=op).o_workers == 256
    info = tiles.dry_run(wl.model, wl.capacity, o_placement=2)
    n_attn = wl.model.n_kv_heads * (wl.model.n_heads // wl.model.n_kv_heads // info.attn_heads) * info.kv_splits
    assert info.o_workers == 256 - n_attn == 96
    # a separate combine wave keeps o_proj on all workers
    assert tiles.dry_run(wl.model, wl.capacity, o_placement=2, combine_mode=2).o_workers == 256
    with pytest.raises(tiles.TilesError) as e:
        tiles.dry_run(wl.model, wl.capacity, o_placement=3)
    assert e.value.code == tiles.TILES_E_CONFIG


# ---------------------------------------------------------------------------
# the plan validator rejects each planted mistake with the rule it breaks
# ---------------------------------------------------------------------------

VALIDATOR_MUTATIONS = [
    (1, "GEMV rows not covered exactly once"),
    (2, "GEMV rows not covered exactly once"),
    (3, "attention/combine tile"),
    (4, "attention/combine tiles do not cover every head"),
    (5, "attention tile out of range"),
    (6, "tagged buffers overlap"),
    (7, "tagged buffer misaligned or out of bounds"),
    (8, "worker bytes unbalanced"),
    (9, "waves out of dependency order"),
    (10, "waves out of dependency order"),
    (11, "packed tiles overlap"),
    (12, "is not its source row"),
    (13, "source rows not packed exactly once"),
    (14, "norm gains misplaced"),
    (15, "bad LDS staging area"),
]


def test_validator_accepts_the_unmutated_plans():
    for m, pos in ((LLAMA_1B, 1087), (QWEN3_06B, 1087), (TINY, 64)):
        assert tiles.debug_validate(m, pos, 0) == tiles.TILES_OK, tiles.last_error()


@pytest.mark.parametrize("mutation,message", VALIDATOR_MUTATIONS, ids=[str(m) for m, _ in VALIDATOR_MUTATIONS])
def test_validator_rejects_planted_mistake(mutation, message):
    rc = tiles.debug_validate(LLAMA_1B, 1087, mutation)
    assert rc == tiles.TILES_E_PLAN, (rc, tiles.last_error())
    assert message in tiles.last_error()


def test_validator_mutation_hook_arguments():
    assert tiles.debug_validate(TINY, 64, 99) == tiles.TILES_E_ARG
    assert tiles.lib().tiles_plan_debug_validate(None, 256, 0) == tiles.TILES_E_ARG


# ---------------------------------------------------------------------------
# weight-only INT8: the library's quantizer gives the oracle's codes and scales bit for bit, and
# INT8 plans build, validate and stream the bytes the workload definition counts
# ---------------------------------------------------------------------------

def test_library_int8_quantizer_matches_the_oracle_bit_for_bit():
    import numpy as np
    import torch

    from oracle import quantize_rows_int8 as oracle_quantize
    rng = np.random.default_rng(21)
    rows = [rng.standard_normal((200, 333)) * (10.0 ** rng.integers(-8, 6, 200))[:, None],
            np.zeros((3, 333)),                                       # rows of zeros
            np.full((2, 333), 2.5 * 2 ** -7), ]                      # ties: W / s = 127 and 2.5 (after the max)
    rows[2][:, 0] = 127 / 128
    w32 = np.concatenate(rows).astype(np.float32)
    bits = torch.from_numpy(w32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    bits[5, 7] = 0x0001  # a subnormal BF16
    bits[6, 9] = 0x8000  # -0
    q_lib, s_lib = tiles.quantize_rows_int8(bits)
    q_orc, s_orc = oracle_quantize(bits)
    assert np.array_equal(s_lib.view(np.uint32), s_orc.view(np.uint32))
    assert np.array_equal(q_lib, q_orc)
    assert q_lib[-1, 1] == 2 and q_lib[-1, 0] == 127
    assert tiles.lib().tiles_quantize_rows_int8(None, 1, 1, None, None) == tiles.TILES_E_ARG


@pytest.mark.parametrize("key", ["llama1b_int8", "qwen06b_int8", "qwen4b_int8"])
def test_int8_plans_validate_and_count_the_workload_bytes(key):
    wl = WORKLOADS[key]
    info = tiles.dry_run(wl.model, wl.capacity, weights="int8")
    assert info.weight_format == 1
    assert info.weight_bytes_per_step == wl.model.int8_weight_bytes_per_token()
    assert tiles.debug_validate(wl.model, wl.capacity, 0, weights="int8") == tiles.TILES_OK, tiles.last_error()
    bf = tiles.dry_run(wl.model, wl.capacity)
    assert bf.weight_format == 0 and bf.weight_bytes_per_step == wl.model.weight_bytes_per_token()


def test_int8_plan_of_ragged_and_untied_shapes():
    m = scaled(TINY, name="ragged-untied", n_layers=3, hidden=384, n_heads=6, n_kv_heads=2, ffn=1000, vocab=1000,
               tie_embeddings=False)
    assert tiles.debug_validate(m, 64, 0, weights="int8") == tiles.TILES_OK, tiles.last_error()
    for mutation in (12, 13):  # packed rows exchanged, a packing copy dropped
        assert tiles.debug_validate(m, 64, mutation, weights="int8") == tiles.TILES_E_PLAN


@pytest.mark.parametrize("m,sampling", [(TINY, (0.7, 32, 0.9)), (LLAMA_1B, (0.6, 20, 0.95)), (QWEN3_06B, (1.0, 1, 1.0)),
                                        (QWEN3_4B, (0.6, 32, 0.95))])
def test_sampling_plans_validate(m, sampling):
    """Sampling plans carry top_k and leave room in LDS for every worker's top_k candidates
    (2 words each) in the token gather; the LDS total stays within the CU's 160 KB."""
    info = tiles.dry_run(m, 1100, sampling=sampling)
    assert info.top_k == sampling[1]
    assert info.lds_bytes <= 160 * 1024
    greedy = tiles.dry_run(m, 1100)
    assert greedy.top_k == 0 and greedy.checksum != info.checksum


@pytest.mark.parametrize("sampling", [(1.0, 33, 0.9), (0.0, 8, 0.9), (-1.0, 8, 0.9), (float("inf"), 8, 0.9),
                                      (float("nan"), 8, 0.9), (1.0, 8, 0.0), (1.0, 8, 1.5), (1.0, 8, float("nan")),
                                      (1.0, -1, 0.9)])
def test_bad_sampling_parameters_are_rejected(sampling):
    with pytest.raises(tiles.TilesError) as e:
        tiles.dry_run(TINY, 40, sampling=sampling)
    assert e.value.code == tiles.TILES_E_CONFIG


def test_sampling_limits_top_k_by_vocab_and_workers():
    small_vocab = scaled(TINY, name="v16", vocab=16)
    with pytest.raises(tiles.TilesError):
        tiles.dry_run(small_vocab, 40, sampling=(1.0, 17, 1.0))
    assert tiles.dry_run(small_vocab, 40, sampling=(1.0, 16, 1.0)).top_k == 16
    with pytest.raises(tiles.TilesError) as e:
        tiles.dry_run(TINY, 40, n_workers=300, sampling=(1.0, 8, 1.0))
    assert "256 workers" in tiles.last_error() or e.value.code == tiles.TILES_E_CONFIG



@pytest.mark.parametrize("key", ["qwen4b_32k_kv8", "llama1b_kv8"])
def test_int8_kv_plans_validate(key):
    """INT8 KV plans: at most 4096 positions per split (the split count is raised to fit), LDS for the
    split's scales, the KV format in the plan info; the same shapes with BF16 KV plan differently."""
    wl = WORKLOADS[key]
    info = tiles.dry_run(wl.model, wl.capacity, kv="int8")
    assert info.kv_format == 1
    assert info.lds_bytes <= 160 * 1024
    assert (wl.capacity + info.kv_splits - 1) // info.kv_splits <= 4096
    assert tiles.dry_run(wl.model, wl.capacity).checksum != info.checksum
    assert tiles.lib().tiles_plan_debug_validate(ctypes.byref(tiles.make_config(wl.model, wl.capacity, kv="int8")),
                                                 256, 0) == tiles.TILES_OK


def test_int8_kv_format_and_split_limits_rejected():
    cfg = tiles.make_config(TINY, 40)
    cfg.kv_format = 2
    info = tiles.PlanInfo()
    assert tiles.lib().tiles_plan_dry_run(ctypes.byref(cfg), 256, ctypes.byref(info)) == tiles.TILES_E_CONFIG
    with pytest.raises(tiles.TilesError):  # a forced split count leaving more than 4096 positions per split
        tiles.dry_run(TINY, 9000, kv="int8", kv_splits=2)
    assert "4096 positions per split" in tiles.last_error()
    # the planner raises its own split count to fit; 4096 positions per split are accepted
    assert tiles.dry_run(TINY, 9000, kv="int8").kv_splits >= 3
    assert tiles.dry_run(TINY, 8192, kv="int8", kv_splits=2).kv_splits == 2
    assert tiles.lib().tiles_kv_convert_int8(None, None, None, 1, 0, None) == tiles.TILES_E_ARG


# ---------------------------------------------------------------------------------------------
# verify plans (tokens_per_step > 1)
# ---------------------------------------------------------------------------------------------

@pytest.mark.parametrize("m,pos,mt", [(LLAMA_1B, 1087, 2), (LLAMA_1B, 1087, 3), (QWEN3_06B, 1087, 2), (QWEN3_4B, 1087, 2),
                                      (TINY, 80, 2), (TINY, 80, 3), (TINY, 80, 4)],
                         ids=["llama1b-2", "llama1b-3", "qwen06b-2", "qwen4b-2", "tiny-2", "tiny-3", "tiny-4"])
def test_verify_plans_validate(m, pos, mt):
    """A verify plan holds at most 4 query rows per attention tile, fits the LDS, records its positions
    per step, merges the splits in the o_proj prologue or in a wave of its own (one more per layer),
    and is not the decode plan's schedule."""
    info = tiles.dry_run(m, pos, tokens_per_step=mt)
    dec = tiles.dry_run(m, pos)
    assert info.tokens_per_step == mt and dec.tokens_per_step == 1
    assert info.waves_per_step == m.n_layers * (5 if info.combine_mode == 1 else 6) + 1
    assert info.attn_heads * mt <= 4
    assert info.lds_bytes <= 160 * 1024
    assert info.checksum != dec.checksum
    cfg = tiles.make_config(m, pos, tokens_per_step=mt)
    assert tiles.lib().tiles_plan_debug_validate(ctypes.byref(cfg), 256, 0) == tiles.TILES_OK, tiles.last_error()


def test_verify_plan_split_merge_placement():
    """The o_proj prologue merges the splits of every position where the input and partial areas hold
    mt * (Qpad + n_heads * S * (head_dim + 4)) floats beside the rest and one staging batch (the
    Llama-3.2-1B shape at 2 positions, 5 splits); the Qwen3 shapes merge in a wave of their own.  Forced,
    the prologue merge fits the Qwen3-0.6B shape without staging and not the Qwen3-4B shape; a forced own
    wave is honoured."""
    assert tiles.dry_run(LLAMA_1B, 1087, tokens_per_step=2).combine_mode == 1
    assert tiles.dry_run(LLAMA_1B, 1087, tokens_per_step=2, combine_mode=2).combine_mode == 2
    for m in (QWEN3_06B, QWEN3_4B):
        assert tiles.dry_run(m, 1087, tokens_per_step=2).combine_mode == 2
    assert tiles.dry_run(QWEN3_06B, 1087, tokens_per_step=2, combine_mode=1).combine_mode == 1
    with pytest.raises(tiles.TilesError):
        tiles.dry_run(QWEN3_4B, 1087, tokens_per_step=2, combine_mode=1)


def test_verify_plan_at_32k_positions_takes_fewer_splits():
    """The Qwen3-4B shape at 32K positions: the decode plan puts 4 query heads and one of 32 splits in each
    of 256 attention tiles; a 2-position verify plan holds at most 2 heads per tile, so it takes 16
    splits (a forced 32 is rejected)."""
    wl = WORKLOADS["qwen4b_32k"]
    dec = tiles.dry_run(wl.model, wl.capacity)
    assert (dec.kv_splits, dec.attn_heads) == (32, 4)
    info = tiles.dry_run(wl.model, wl.capacity, tokens_per_step=2)
    assert (info.kv_splits, info.attn_heads) == (16, 2)
    assert info.stage_batches == 0 and dec.stage_batches >= 1  # no LDS room left for a staging batch
    with pytest.raises(tiles.TilesError):
        tiles.dry_run(wl.model, wl.capacity, tokens_per_step=2, kv_splits=32)


def test_verify_plans_bound_the_heads_per_attention_tile():
    """Qwen3-4B has 4 query heads per KV head: with 2 positions per step a tile holds at most 2 heads.
    The planner takes the fewest heads per tile whose tiles fit the workers; where only 4 would fit
    (40 workers, 4 splits), the verify plan is rejected, as is an explicit attn_heads of 4."""
    assert tiles.dry_run(QWEN3_4B, 1087, tokens_per_step=2, attn_heads=2).attn_heads == 2
    assert tiles.dry_run(QWEN3_4B, 1087, tokens_per_step=2, kv_splits=4, n_workers=64).attn_heads == 2
    assert tiles.dry_run(QWEN3_4B, 1087, kv_splits=4, n_workers=40).attn_heads == 4
    for kw in (dict(kv_splits=4, n_workers=40), dict(attn_heads=4)):
        with pytest.raises(tiles.TilesError):
            tiles.dry_run(QWEN3_4B, 1087, tokens_per_step=2, **kw)


@pytest.mark.parametrize("kw", [dict(tokens_per_step=5), dict(tokens_per_step=8), dict(tokens_per_step=-1),
                                dict(tokens_per_step=2, sampling=(1.0, 4, 1.0)), dict(tokens_per_step=2, combine_mode=3)],
                         ids=["five", "eight", "negative", "sampled", "bad-combine-mode"])
def test_verify_plan_options_rejected(kw):
    with pytest.raises(tiles.TilesError) as e:
        tiles.dry_run(TINY, 80, **kw)
    assert e.value.code == tiles.TILES_E_CONFIG


def test_verify_plan_limits():
    """Positions per step are bounded by the LDS, which holds one input vector of the FFN width per
    position: the Llama-3.2-1B shape (ffn 8192) holds 3 (without a staging batch) and not 4, the
    Qwen3-0.6B shape (ffn 3072, head_dim 128) 4, the Qwen3-4B shape (ffn 9728) 2."""
    info = tiles.dry_run(LLAMA_1B, 1087, tokens_per_step=3)
    assert info.stage_batches == 0 and info.combine_mode == 2
    assert tiles.dry_run(QWEN3_06B, 1087, tokens_per_step=4).tokens_per_step == 4
    assert tiles.dry_run(QWEN3_4B, 1087, tokens_per_step=2).tokens_per_step == 2
    for m, mt in ((LLAMA_1B, 4), (QWEN3_4B, 3)):
        with pytest.raises(tiles.TilesError):
            tiles.dry_run(m, 1087, tokens_per_step=mt)
    assert tiles.dry_run(LLAMA_1B, 1087, tokens_per_step=0).tokens_per_step == 1
    assert tiles.dry_run(LLAMA_1B, 1087, tokens_per_step=1).checksum == tiles.dry_run(LLAMA_1B, 1087).checksum


def test_long_gemv_tiles_in_int8_and_sampling_plans_rejected():
    """The kernel's INT8 scales and sampled candidates cover 640 rows of a GEMV block: with a 200,000-word
    vocabulary the LM-head tiles hold 782 rows while the row blocks of these plans may be longer, so
    INT8 and sampling plans are rejected (a greedy BF16 plan is fine)."""
    big = scaled(LLAMA_1B, name="bigvocab", vocab=200000)
    assert tiles.dry_run(big, 1100).lds_bytes > 0
    for kw in (dict(weights="int8"), dict(sampling=(1.0, 8, 1.0))):
        with pytest.raises(tiles.TilesError) as e:
            tiles.dry_run(big, 1100, **kw)
        assert e.value.code == tiles.TILES_E_PLAN and "640 rows" in tiles.last_error()


def test_decode_plans_have_a_staging_batch():
    """A one-position step stages a batch of a compute wavefront's own range in every plan, so every decode
    plan must hold at least one staging batch (else the plan is rejected)."""
    for key in ("llama1b", "qwen06b", "qwen4b", "qwen4b_32k", "llama1b_int8", "llama1b_kv8", "qwen4b_32k_kv8"):
        wl = WORKLOADS[key]
        info = tiles.dry_run(wl.model, wl.capacity, weights=wl.weights, kv=wl.kv)
        assert 1 <= info.stage_batches <= 2, key


def test_int8_kv_verify_plans():
    """Verify plans with the INT8 KV cache: the split's scales area beside the attention tile's rows, the
    KV format in the plan info; on the Qwen3-4B shape at 32K positions the 2-position plan takes 16
    splits of up to 2050 positions (scale areas of 2112), the one-position plan 32 (1088)."""
    for key, mt in (("llama1b_kv8", 2), ("llama1b_kv8", 3)):
        wl = WORKLOADS[key]
        info = tiles.dry_run(wl.model, wl.capacity, kv="int8", tokens_per_step=mt)
        assert info.kv_format == 1 and info.tokens_per_step == mt and info.lds_bytes <= 160 * 1024
    wl = WORKLOADS["qwen4b_32k_kv8"]
    assert tiles.dry_run(wl.model, wl.capacity, kv="int8").kv_splits == 32
    info = tiles.dry_run(wl.model, wl.capacity, kv="int8", tokens_per_step=2)
    assert info.kv_splits == 16 and info.tokens_per_step == 2 and info.attn_heads == 2
    assert info.lds_bytes <= 160 * 1024
    assert tiles.lib().tiles_plan_debug_validate(
        ctypes.byref(tiles.make_config(wl.model, wl.capacity, kv="int8", tokens_per_step=2)), 256, 0) == tiles.TILES_OK
