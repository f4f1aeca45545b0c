"""GPU parity of the persistent tile kernel against the CPU oracle (called through
the C ABI).  Small models are compared at every step; the full-size workloads
are compared on the steps the oracle can reproduce from its own inputs."""

import ctypes

import numpy as np
import pytest
import torch

from tile_scheduled_persistent_amd import synth, tiles
from tile_scheduled_persistent_amd.configs import TINY, WORKLOADS, scaled

from parity_util import (HIDDEN_REL_L2, Setup, check_step, compare_free_running, compare_sampled_teacher_forced,
                         compare_teacher_forced, kv8_rows_close, kv_rows_close, run_gpu, run_gpu_sampled,
                         split_int8_cache, top2_margin, MARGIN)

pytestmark = pytest.mark.gpu

RAGGED = scaled(TINY, name="ragged", n_layers=3, hidden=384, n_heads=6, n_kv_heads=2, ffn=1000, vocab=1000)
QK128 = scaled(TINY, name="tiny-qk128", head_dim=128, n_heads=4, n_kv_heads=1, qk_norm=True, rms_eps=1e-6,
               rope_theta=1e6)
# Llama-3.2-1B widths on two layers: a compute wavefront's share of a gate/up or down tile spans
# more than two batches, so the staged (direct-to-LDS) part of the weight prefetch runs
WIDE = scaled(TINY, name="wide-2layer", n_layers=2, hidden=2048, n_heads=32, n_kv_heads=8, head_dim=64, ffn=8192,
              vocab=4096, rms_eps=1e-5, rope_theta=5e5)


def _oracle_forced(setup: Setup, inputs_prefix, n_steps, plan, pos0=None, tag=""):
    """GPU one step per launch, fed the oracle's tokens (prompt first); every step compared."""
    o = setup.oracle()
    okv = setup.oracle_kv()
    kv = setup.fresh_kv(plan)
    pos = setup.n_cached if pos0 is None else pos0
    tok = inputs_prefix[0]
    margins = []
    for i in range(n_steps):
        g_t, g_l, g_h = run_gpu(plan, kv, tok, 1)
        o_l, o_h = o.step(okv, tok, pos + i)
        o_t = int(np.argmax(o_l))
        margins.append(check_step(f"{tag} step {i}", g_l[0], g_h[0], o_l, o_h, int(g_t[0]), o_t))
        tok = inputs_prefix[i + 1] if i + 1 < len(inputs_prefix) else o_t
    # the KV rows the GPU wrote against the oracle's (same bar as the hidden states)
    if setup.kv == "int8":
        kv8_rows_close(tag, kv, okv, pos, n_steps)
    else:
        kv_rows_close(f"{tag} K", kv.k, okv["k"], pos, n_steps)
        kv_rows_close(f"{tag} V", kv.v, okv["v"], pos, n_steps)
    return margins


def test_tiny_every_step_against_oracle():
    wl = WORKLOADS["tiny"]
    s = Setup(TINY, wl.capacity, 0)
    prompt = synth.make_tokens(TINY, wl.prompt_len)
    with s.plan() as plan:
        _oracle_forced(s, prompt, wl.prompt_len + wl.n_steps, plan, tag="tiny")


def test_tiny_workload_as_specified_free_running():
    """8 prompt steps of one token each, then one 15-step launch; oracle free-running."""
    wl = WORKLOADS["tiny"]
    s = Setup(TINY, wl.capacity, 0)
    prompt = synth.make_tokens(TINY, wl.prompt_len)
    o = s.oracle()
    okv = s.oracle_kv()
    kv = s.fresh_kv()
    with s.plan() as plan:
        for i, t in enumerate(prompt):
            g_t, g_l, g_h = run_gpu(plan, kv, t, 1)
            o_l, o_h = o.step(okv, t, i)
            check_step(f"prompt {i}", g_l[0], g_h[0], o_l, o_h, int(g_t[0]), int(np.argmax(o_l)))
        first = int(g_t[0])
        if first != int(np.argmax(o_l)):
            pytest.skip("first generated token differs at a low-margin step; later steps not comparable")
        g_t, g_l, g_h = run_gpu(plan, kv, first, wl.n_steps)
        o_res = o.decode(okv, first, wl.prompt_len, wl.n_steps)
        n = compare_free_running("tiny gen", g_t, g_l, g_h, o_res, wl.n_steps)
        assert n >= 1


def _full_run(s: Setup, token, n, flags=tiles.TILES_DEBUG_HIDDEN):
    kv = s.fresh_kv()
    with s.plan(flags=flags) as plan:
        g_t, g_l, g_h = run_gpu(plan, kv, token, n, want_hidden=bool(flags & tiles.TILES_DEBUG_HIDDEN))
    return g_t, g_l, g_h, kv


def test_tiny_bitwise_repeatable():
    wl = WORKLOADS["tiny"]
    s = Setup(TINY, wl.capacity, 8)
    tok = synth.make_tokens(TINY, 1)[0]
    a = _full_run(s, tok, 15)
    b = _full_run(s, tok, 15)
    assert np.array_equal(a[0], b[0])
    assert np.array_equal(a[1].view(np.uint32), b[1].view(np.uint32))
    assert np.array_equal(a[2].view(np.uint32), b[2].view(np.uint32))
    assert torch.equal(a[3].k, b[3].k) and torch.equal(a[3].v, b[3].v)


def test_tiny_one_launch_equals_single_step_launches():
    """k launches of 1 step (fed the same tokens) equal 1 launch of k steps, bit for bit."""
    wl = WORKLOADS["tiny"]
    s = Setup(TINY, wl.capacity, 8)
    tok = synth.make_tokens(TINY, 1)[0]
    g_t, g_l, g_h, kv_a = _full_run(s, tok, 15)
    kv = s.fresh_kv()
    with s.plan() as plan:
        t = tok
        for i in range(15):
            t1, l1, h1 = run_gpu(plan, kv, t, 1)
            assert int(t1[0]) == int(g_t[i])
            assert np.array_equal(l1[0].view(np.uint32), g_l[i].view(np.uint32))
            assert np.array_equal(h1[0].view(np.uint32), g_h[i].view(np.uint32))
            t = int(t1[0])
    assert torch.equal(kv.k, kv_a.k) and torch.equal(kv.v, kv_a.v)


def test_poison_mode_changes_nothing():
    s = Setup(TINY, 40, 20)
    tok = 7
    a = _full_run(s, tok, 12)
    b = _full_run(s, tok, 12, flags=tiles.TILES_DEBUG_HIDDEN | tiles.TILES_POISON)
    assert np.array_equal(a[1].view(np.uint32), b[1].view(np.uint32))
    assert np.array_equal(a[0], b[0])


def _bits_equal(a, b):
    assert np.array_equal(a[0], b[0])
    assert np.array_equal(a[1].view(np.uint32), b[1].view(np.uint32))
    assert np.array_equal(a[2].view(np.uint32), b[2].view(np.uint32))
    assert torch.equal(a[3].k.view(torch.int16), b[3].k.view(torch.int16))
    assert torch.equal(a[3].v.view(torch.int16), b[3].v.view(torch.int16))


def test_poison_with_the_cache_filled_to_capacity():
    """length + n_steps == capacity: the NaN-poisoned rows include the last row of every head, the
    one masked attention slots read; masked slots must discard it (regression: they used to weigh
    it by 0, and 0 * NaN poisoned the sums)."""
    s = Setup(TINY, 32, 20)
    a = _full_run(s, 7, 12)
    b = _full_run(s, 7, 12, flags=tiles.TILES_DEBUG_HIDDEN | tiles.TILES_POISON)
    _bits_equal(a, b)


def test_nan_in_the_unused_cache_tail_changes_nothing():
    """A cache whose rows past the launch's last position hold NaN gives bit-identical results."""
    s = Setup(TINY, 48, 20)
    a = _full_run(s, 7, 12)
    kv = s.fresh_kv()
    nan = torch.tensor(float("nan"), dtype=torch.bfloat16, device="cuda")
    kv.k[:, :, 20:] = nan
    kv.v[:, :, 20:] = nan
    with s.plan() as plan:
        g_t, g_l, g_h = run_gpu(plan, kv, 7, 12)
    b = (g_t, g_l, g_h, kv)
    assert np.array_equal(a[0], b[0])
    assert np.array_equal(a[1].view(np.uint32), b[1].view(np.uint32))
    assert np.array_equal(a[2].view(np.uint32), b[2].view(np.uint32))
    assert torch.equal(a[3].k[:, :, :32].view(torch.int16), kv.k[:, :, :32].view(torch.int16))
    assert torch.equal(a[3].v[:, :, :32].view(torch.int16), kv.v[:, :, :32].view(torch.int16))


def test_argmax_tie_takes_the_lowest_index():
    """Embedding rows 100 and 3000 made identical and dominant (tied head): their logits are equal
    bit for bit, and the greedy token is the lower index, on the GPU (the rows sit in the LM-head
    tiles of different workers, so the cross-worker reduction decides) as in the oracle."""
    s = Setup(TINY, 16, 0)
    row = torch.full((TINY.hidden,), 0.5, dtype=torch.bfloat16)
    for r in (100, 3000):
        s.w_dev["embed"][r] = row.cuda()
        s.w_bits["embed"][r] = synth.bits(row)
    with s.plan() as plan:
        g_t, g_l, _ = run_gpu(plan, s.fresh_kv(), 100, 3)
    o = s.oracle().decode(s.oracle_kv(), 100, 0, 3)
    for i in range(3):
        assert g_l[i][100] == g_l[i][3000] == g_l[i].max()
        assert o["logits"][i][100] == o["logits"][i][3000] == o["logits"][i].max()
    assert list(g_t) == [100, 100, 100] and list(o["tokens"]) == [100, 100, 100]


def test_ragged_shapes_group3_padding():
    s = Setup(RAGGED, 64, 37)
    toks = synth.make_tokens(RAGGED, 1)
    with s.plan() as plan:
        _oracle_forced(s, toks, 12, plan, tag="ragged")


@pytest.mark.parametrize("o_placement", [0, 2])
def test_wide_layers_staged_prefetch(o_placement):
    # o_placement 2: o_proj tiles only on the workers without an attention tile (they stage their
    # o_proj share in the attention wave, the attention workers stage gate/up in the o_proj wave)
    s = Setup(WIDE, 96, 70)
    toks = synth.make_tokens(WIDE, 1)
    with s.plan(o_placement=o_placement) as plan:
        info = plan.info()
        assert o_placement == 0 or 0 < info.o_workers < info.n_workers
        _oracle_forced(s, toks, 6, plan, tag=f"wide o_placement={o_placement}")


@pytest.mark.parametrize("heads", [0, 2, 4])
def test_qk_norm_head_dim_128(heads):
    s = Setup(QK128, 64, 29)
    toks = synth.make_tokens(QK128, 1)
    with s.plan(attn_heads=heads) as plan:
        assert heads == 0 or plan.info().attn_heads == heads
        _oracle_forced(s, toks, 10, plan, tag=f"qk128 heads/tile={heads}")


@pytest.mark.parametrize("splits,mode", [(1, 1), (3, 1), (3, 2), (7, 2), (16, 2)])
def test_split_counts_and_combine_placement(splits, mode):
    m = scaled(TINY, name="tiny-long")
    s = Setup(m, 400, 333)
    toks = synth.make_tokens(m, 1)
    with s.plan(kv_splits=splits, combine_mode=mode) as plan:
        info = plan.info()
        assert info.kv_splits == splits and info.combine_mode == mode
        _oracle_forced(s, toks, 5, plan, tag=f"S={splits} mode={mode}")


def test_empty_splits_at_short_length():
    """More splits than positions: empty splits contribute nothing."""
    m = scaled(TINY, name="tiny-short")
    s = Setup(m, 16, 0)
    toks = synth.make_tokens(m, 6)
    with s.plan(kv_splits=8, combine_mode=1) as plan:
        _oracle_forced(s, toks, 6, plan, tag="short")


def test_error_paths():
    s = Setup(TINY, 24, 20)
    with s.plan() as plan:
        kv = s.fresh_kv()
        out = torch.zeros(64, dtype=torch.int32, device="cuda")
        for bad_tok in [-1, TINY.vocab]:
            with pytest.raises(tiles.TilesError) as e:
                plan.decode(kv, bad_tok, 1, out)
            assert e.value.code == tiles.TILES_E_ARG
        for n in [0, 65]:
            with pytest.raises((tiles.TilesError, ValueError)):
                plan.decode(kv, 1, n, out)
        with pytest.raises(tiles.TilesError) as e:
            plan.decode(kv, 1, 5, out)  # 20 + 5 > 24
        assert e.value.code == tiles.TILES_E_ARG
        assert kv.length == 20
        plan.decode(kv, 1, 4, out)     # exactly fills the cache
        assert plan.status() == tiles.TILES_OK and kv.length == 24
        plan.debug_corrupt()
        kv2 = s.fresh_kv()
        with pytest.raises(tiles.TilesError) as e:
            plan.decode(kv2, 1, 1, out)
        assert e.value.code == tiles.TILES_E_PLAN


def test_corrupted_device_schedule_is_detected_in_the_launch():
    """A bit flipped in the device copy of the schedule (the host copy and its checksum intact): the
    worker that loads it finds its hash changed and leaves before using it, the others leave at their
    next wait, and the status reports TILES_E_PLAN; out_tokens stays untouched."""
    s = Setup(TINY, 24, 8)
    with s.plan() as plan:
        run_gpu(plan, s.fresh_kv(), 3, 2)  # the intact plan decodes
        plan.debug_corrupt_device()
        out = torch.full((4,), -7, dtype=torch.int32, device="cuda")
        plan.decode(s.fresh_kv(), 3, 4, out)
        assert plan.status() == tiles.TILES_E_PLAN
        assert "schedule" in tiles.last_error()
        assert plan.status() == tiles.TILES_OK  # the status word was cleared
        assert out.cpu().tolist() == [-7, -7, -7, -7]


# ---------------------------------------------------------------------------
# full-size workloads: the launch bench.py times (one launch of all steps)
# ---------------------------------------------------------------------------

FULL = ["llama1b", "qwen06b", "qwen4b", "qwen4b_32k", "llama1b_int8"]


@pytest.mark.slow
@pytest.mark.timeout(900)
@pytest.mark.parametrize("key", FULL)
def test_full_size_workload_every_step(key):
    """The launch bench.py times, every step: the oracle is teacher-forced on the GPU's own tokens
    (step i of both consumes the same input), so every step is compared, the last one included.
    The timed configuration itself (no debug buffers, no logits) gives the same tokens and the same
    cache bytes as the checked one."""
    wl = WORKLOADS[key]
    m = wl.model
    n = wl.n_steps
    s = Setup(m, wl.capacity, wl.n_cached, key_scale=wl.key_scale, gen_device="cuda", weights=wl.weights)
    tok = synth.make_tokens(m, 1)[0]
    kv_timed = s.fresh_kv()
    with s.plan(flags=0) as plan:
        out_t = torch.zeros(n, dtype=torch.int32, device="cuda")
        plan.decode(kv_timed, tok, n, out_t, None)
        assert plan.status() == tiles.TILES_OK, tiles.last_error()
        timed_tokens = out_t.cpu().numpy().astype(np.int64)
    kv = s.fresh_kv()
    with s.plan() as plan:
        g_t, g_l, g_h = run_gpu(plan, kv, tok, n)
    assert np.array_equal(timed_tokens, g_t), "timed configuration gives other tokens"
    assert torch.equal(kv_timed.k.view(torch.int16), kv.k.view(torch.int16))
    assert torch.equal(kv_timed.v.view(torch.int16), kv.v.view(torch.int16))
    del kv_timed
    print(f"{key}: GPU launch of {n} steps done; teacher-forced oracle for all {n} steps", flush=True)
    okv = s.oracle_kv()
    o_res = s.oracle().decode(okv, tok, wl.n_cached, n, teacher=[int(t) for t in g_t[:-1]], widen_kv_once=True)
    stats = compare_teacher_forced(key, g_t, g_l, g_h, o_res)
    assert stats["steps"] == n
    k_rel, k_frac = kv_rows_close(f"{key} K", kv.k, okv["k"], wl.n_cached, n)
    v_rel, v_frac = kv_rows_close(f"{key} V", kv.v, okv["v"], wl.n_cached, n)
    print(f"{key}: {n} of {n} steps compared; max hidden rel L2 {stats['hidden_rel_l2_max']:.2e}, max logit abs err "
          f"{stats['logit_abs_max']:.2e}, tokens checked at margin > 0.1: {stats['tokens_checked']} "
          f"(smallest oracle margin {stats['min_margin']:.3f}); cached K/V rows rel L2 {k_rel:.2e} / {v_rel:.2e}, "
          f"entries differing {k_frac:.3%} / {v_frac:.3%}", flush=True)


@pytest.mark.slow
def test_llama_full_size_repeatable_and_chunk_invariant():
    wl = WORKLOADS["llama1b"]
    m = wl.model
    s = Setup(m, wl.capacity, wl.n_cached, gen_device="cuda")
    tok = synth.make_tokens(m, 1)[0]
    a = _full_run(s, tok, wl.n_steps, flags=0)
    b = _full_run(s, tok, wl.n_steps, flags=0)
    assert np.array_equal(a[0], b[0])
    assert np.array_equal(a[1].view(np.uint32), b[1].view(np.uint32))
    assert torch.equal(a[3].k, b[3].k) and torch.equal(a[3].v, b[3].v)
    kv = s.fresh_kv()
    with s.plan(flags=0) as plan:
        t = tok
        for i in range(wl.n_steps):
            t1, l1, _ = run_gpu(plan, kv, t, 1, want_hidden=False)
            assert int(t1[0]) == int(a[0][i])
            assert np.array_equal(l1[0].view(np.uint32), a[1][i].view(np.uint32))
            t = int(t1[0])
    assert torch.equal(kv.k, a[3].k) and torch.equal(kv.v, a[3].v)


def test_watchdog_gives_up_and_the_plan_recovers():
    # A one-round watchdog (set from the host) makes ordinary waits give up: the launch ends early
    # with every worker leaving after its next input barrier, the status reports it, and once the
    # default is back the same plan decodes bit-identically to a fresh plan.
    s = Setup(WIDE, 96, 70)
    tok = synth.make_tokens(WIDE, 1)[0]
    n = 8
    with s.plan() as plan:
        plan.debug_spin_limit(1)
        out_t = torch.zeros(n, dtype=torch.int32, device="cuda")
        plan.decode(s.fresh_kv(), tok, n, out_t)
        assert plan.status() == tiles.TILES_E_KERNEL
        assert plan.status() == tiles.TILES_OK  # the fault word was cleared
        plan.debug_spin_limit(0)
        g_t, g_l, g_h = run_gpu(plan, s.fresh_kv(), tok, n)
    with s.plan() as fresh:
        r_t, r_l, r_h = run_gpu(fresh, s.fresh_kv(), tok, n)
    assert np.array_equal(g_t, r_t)
    assert np.array_equal(g_l.view(np.uint32), r_l.view(np.uint32))
    assert np.array_equal(g_h.view(np.uint32), r_h.view(np.uint32))


# ---------------------------------------------------------------------------
# the stream-read ceiling kernel (measurement helper): it reads every byte it is given
# ---------------------------------------------------------------------------

def test_stream_read_reads_every_word():
    g = torch.Generator().manual_seed(5)
    n_groups = 4
    unit = n_groups * 8 * 8 * 1024
    host = torch.randint(-2**31, 2**31 - 1, (3 * unit // 4,), dtype=torch.int64, generator=g).to(torch.int32)
    expect = int(np.bitwise_xor.reduce(host.numpy().view(np.uint32)))
    buf = host.cuda()
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    tiles.stream_read(buf, n_groups, sink)
    torch.cuda.synchronize()
    assert int(sink.cpu().numpy().view(np.uint32)[0]) == expect
    with pytest.raises(tiles.TilesError) as e:
        tiles.stream_read(buf[: unit // 4 - 4], n_groups, sink)  # not a multiple of the per-launch unit
    assert e.value.code == tiles.TILES_E_ARG


# ---------------------------------------------------------------------------
# the edge-latency helper: every round trip completes, at a plausible cost, and a one-poll limit
# ends the exchange early instead of waiting
# ---------------------------------------------------------------------------

def test_edge_latency_round_trips_complete():
    words = torch.zeros(64, dtype=torch.int32, device="cuda")
    out = torch.zeros(3, dtype=torch.int64, device="cuda")
    for peer in (1, 8):
        words.zero_()
        out.zero_()
        tiles.edge_latency(words, peer, 500, out)
        torch.cuda.synchronize()
        ticks, gave_up_peer, gave_up_0 = (int(x) for x in out.cpu())
        assert gave_up_peer == 0 and gave_up_0 == 0
        # both words hold the last count: every one of the 500 round trips happened
        w = words.cpu()
        assert int(w[0]) == 500 and int(w[16]) == 500
        us = ticks * 0.01 / 500
        assert 0.05 < us < 50.0, us
    # a limit of one poll: the first wait that is not answered at once gives up; the launch ends
    words.zero_()
    out.zero_()
    tiles.edge_latency(words, 8, 1000, out, spin_limit=1)
    torch.cuda.synchronize()
    assert int(out[1]) != 0 or int(out[2]) != 0
    with pytest.raises(tiles.TilesError) as e:
        tiles.edge_latency(words[:8], 8, 10, out)
    assert e.value.code == tiles.TILES_E_ARG


# ---------------------------------------------------------------------------
# the in-kernel trace: recording it changes no result, and its stamps are ordered
# ---------------------------------------------------------------------------

def test_trace_is_bit_neutral_and_its_stamps_are_ordered():
    s = Setup(WIDE, 96, 70)
    tok = synth.make_tokens(WIDE, 1)[0]
    n = 6
    a = _full_run(s, tok, n)
    kv = s.fresh_kv()
    with s.plan(flags=tiles.TILES_DEBUG_HIDDEN | tiles.TILES_TRACE) as plan:
        g_t, g_l, g_h = run_gpu(plan, kv, tok, n)
        _, tr = plan.read_debug(hidden=False, trace=True)
        W = plan.info().n_workers
    _bits_equal(a, (g_t, g_l, g_h, kv))
    tr = tr.astype(np.int64)  # [steps, waves, W, 12], 100 MHz wall clock
    assert tr.shape[0] == n and tr.shape[2] == W
    start, staged, done, published, after_a = tr[..., 0], tr[..., 1], tr[..., 2], tr[..., 3], tr[..., 7]
    assert (start > 0).all() and (published > 0).all()
    assert (start <= staged).all() and (staged <= after_a).all() and (after_a <= published).all()
    assert (staged <= done).all() and (done <= published).all()
    # per worker, waves follow one another: a wave starts after the previous one published
    seq_start = start.reshape(-1, W)
    seq_pub = published.reshape(-1, W)
    assert (seq_start[1:] >= seq_pub[:-1]).all()
    # the first compute wavefront's own stamps (when it had a share) sit between the barriers
    first_cw_done = tr[..., 4]
    has = first_cw_done != 0
    assert (first_cw_done[has] >= staged[has]).all() and (first_cw_done[has] <= published[has]).all()


# ---------------------------------------------------------------------------
# weight-only INT8 linear layers: the GPU's INT8 tiles against the oracle's INT8 model
# ---------------------------------------------------------------------------

def test_int8_tiny_every_step_against_oracle():
    wl = WORKLOADS["tiny"]
    s = Setup(TINY, wl.capacity, 0, weights="int8")
    prompt = synth.make_tokens(TINY, wl.prompt_len)
    with s.plan() as plan:
        assert plan.info().weight_format == 1
        _oracle_forced(s, prompt, wl.prompt_len + wl.n_steps, plan, tag="tiny int8")


def test_int8_ragged_untied_padding():
    # hidden 384 and ffn 1000 pad to 1024-column INT8 chunks; an untied head of its own
    m = scaled(RAGGED, name="ragged-untied", tie_embeddings=False)
    s = Setup(m, 64, 37, weights="int8")
    toks = synth.make_tokens(m, 1)
    with s.plan() as plan:
        _oracle_forced(s, toks, 10, plan, tag="ragged int8")


def test_int8_wide_layers_and_qk_norm():
    s = Setup(WIDE, 96, 70, weights="int8")
    with s.plan() as plan:
        _oracle_forced(s, synth.make_tokens(WIDE, 1), 6, plan, tag="wide int8")
    s = Setup(QK128, 64, 29, weights="int8")
    with s.plan(attn_heads=2) as plan:
        _oracle_forced(s, synth.make_tokens(QK128, 1), 8, plan, tag="qk128 int8")


def test_int8_repeatable_and_chunk_invariant():
    s = Setup(WIDE, 96, 70, weights="int8")
    tok = synth.make_tokens(WIDE, 1)[0]
    a = _full_run(s, tok, 10)
    b = _full_run(s, tok, 10)
    _bits_equal(a, b)
    kv = s.fresh_kv()
    with s.plan() as plan:
        t = tok
        for i in range(10):
            t1, l1, h1 = run_gpu(plan, kv, t, 1)
            assert int(t1[0]) == int(a[0][i])
            assert np.array_equal(l1[0].view(np.uint32), a[1][i].view(np.uint32))
            t = int(t1[0])



# ---------------------------------------------------------------------------
# sampled decoding (top-k / top-p inside the launch)
# ---------------------------------------------------------------------------

SAMPLINGS = [(0.7, 20, 0.95), (1.5, 32, 1.0), (0.3, 5, 0.5), (1.0, 1, 1.0)]


@pytest.mark.parametrize("sampling", SAMPLINGS, ids=[f"T{t}-k{k}-p{p}" for t, k, p in SAMPLINGS])
def test_sampled_tiny_every_step_against_oracle(sampling):
    """One sampled launch of 20 steps after 10 cached positions, every step against the oracle
    teacher-forced on the GPU's tokens with the same uniforms: hidden states, logits and the draw
    (exact away from a decision boundary, among the top k + 1 near one); the K/V rows written."""
    n, cached = 20, 10
    s = Setup(TINY, cached + n + 2, cached)
    tok = synth.make_tokens(TINY, 1)[0]
    u = synth.make_uniforms(TINY, n)
    kv = s.fresh_kv()
    with s.plan(sampling=sampling) as plan:
        assert plan.info().top_k == sampling[1]
        g_t, g_l, g_h = run_gpu_sampled(plan, kv, tok, n, u)
    okv = s.oracle_kv()
    o_res = s.oracle().decode(okv, tok, cached, n, teacher=[int(t) for t in g_t[:-1]], sampling=sampling, uniforms=u)
    stats = compare_sampled_teacher_forced(f"tiny sampled {sampling}", g_t, g_l, g_h, o_res, sampling, u)
    print(f"tiny sampled {sampling}: {stats}", flush=True)
    assert stats["steps"] == n and stats["draws_exact"] >= n // 2
    kv_rows_close("tiny sampled K", kv.k, okv["k"], cached, n)
    kv_rows_close("tiny sampled V", kv.v, okv["v"], cached, n)


def test_sampled_top1_equals_greedy_bit_for_bit():
    """top_k = 1 keeps only the argmax (lowest id on ties), whatever T, top_p and u: the sampled
    launch gives the greedy launch's tokens, logits and cache bytes exactly."""
    s = Setup(WIDE, 96, 70)
    tok = synth.make_tokens(WIDE, 1)[0]
    n = 12
    kv_g = s.fresh_kv()
    with s.plan() as plan:
        g = run_gpu(plan, kv_g, tok, n)
    kv_s = s.fresh_kv()
    with s.plan(sampling=(0.8, 1, 0.5)) as plan:
        r = run_gpu_sampled(plan, kv_s, tok, n, synth.make_uniforms(WIDE, n))
    assert np.array_equal(g[0], r[0])
    assert np.array_equal(g[1].view(np.uint32), r[1].view(np.uint32))
    assert torch.equal(kv_g.k, kv_s.k) and torch.equal(kv_g.v, kv_s.v)


def test_sampled_repeatable_and_chunk_invariant():
    """A sampled launch repeats bit for bit, and n one-step launches (each with its step's uniform)
    give the n-step launch's tokens and logits exactly."""
    s = Setup(WIDE, 96, 70)
    sampling = (0.8, 16, 0.9)
    tok = synth.make_tokens(WIDE, 1)[0]
    n = 10
    u = synth.make_uniforms(WIDE, n)
    with s.plan(sampling=sampling) as plan:
        kv_a = s.fresh_kv()
        a = run_gpu_sampled(plan, kv_a, tok, n, u)
        kv_b = s.fresh_kv()
        b = run_gpu_sampled(plan, kv_b, tok, n, u)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1].view(np.uint32), b[1].view(np.uint32))
        assert torch.equal(kv_a.k, kv_b.k) and torch.equal(kv_a.v, kv_b.v)
        kv = s.fresh_kv()
        t = tok
        for i in range(n):
            t1, l1, _ = run_gpu_sampled(plan, kv, t, 1, u[i:i + 1], want_hidden=False)
            assert int(t1[0]) == int(a[0][i])
            assert np.array_equal(l1[0].view(np.uint32), a[1][i].view(np.uint32))
            t = int(t1[0])
        assert torch.equal(kv.k, kv_a.k) and torch.equal(kv.v, kv_a.v)


def test_sampled_equal_logits_draw_in_closed_form():
    """A model whose logits are all exactly equal (zero linear weights, identical embedding rows,
    tied head): the top_k candidates are ids 0 .. k - 1 with weight 1 each, so with top_k = 32 the
    draw at step i is id floor(32 u_i), and with top_p = 1/2 the prefix is 16 long and the draw
    floor(16 u_i) (exact in FP32: the cumulative weights are the integers 1 .. 32)."""
    m = TINY
    w = synth.make_weights(m, device="cuda")
    for d in w["layers"]:
        for name in ("wq", "wk", "wv", "wo", "w_gate", "w_up", "w_down"):
            d[name].zero_()
    w["embed"].fill_(0.25)
    k = torch.zeros((m.n_layers, m.n_kv_heads, 16, m.head_dim), dtype=torch.bfloat16, device="cuda")
    u = np.array([0.0, 0.03, 0.5, 0.249, 0.25, 0.97, 0.999, 0.6, 0.7812, 0.1], np.float32)
    n = len(u)
    for top_p, width in ((1.0, 32), (0.5, 16)):
        kv = tiles.KVCache(k.clone(), k.clone(), 2)
        with tiles.Plan(m, w, 16, sampling=(0.9, 32, top_p)) as plan:
            g_t, g_l, _ = run_gpu_sampled(plan, kv, 7, n, u, want_hidden=False)
        assert np.all(g_l == g_l[:, :1]), "logits not all equal"
        assert list(g_t) == [int(np.floor(width * float(x))) for x in u], (top_p, list(g_t))


def test_sampling_entry_point_errors():
    s = Setup(TINY, 40, 10)
    out = torch.zeros(2, dtype=torch.int32, device="cuda")
    u = torch.full((2,), 0.5, dtype=torch.float32, device="cuda")
    kv = s.fresh_kv()
    with s.plan(sampling=(1.0, 4, 1.0)) as plan:
        with pytest.raises(tiles.TilesError) as e:
            plan.decode(kv, 0, 2, out)  # a sampling plan needs the uniforms
        assert e.value.code == tiles.TILES_E_ARG
        c = tiles.KV(kv.k.data_ptr(), kv.v.data_ptr(), kv.capacity, kv.length)
        assert tiles.lib().tiles_decode(plan._h, ctypes.byref(c), 0, 2, out.data_ptr(), None) == tiles.TILES_E_ARG
        assert "tiles_decode_sampled" in tiles.last_error()
        assert tiles.lib().tiles_decode_noalloc(plan._h, ctypes.byref(c), 0, 2, out.data_ptr(), None) == tiles.TILES_E_ARG
    with s.plan() as greedy:
        with pytest.raises(tiles.TilesError) as e:
            greedy.decode(kv, 0, 2, out, uniforms=u)
        assert e.value.code == tiles.TILES_E_ARG
    assert kv.length == 10


@pytest.mark.slow
@pytest.mark.timeout(900)
def test_full_size_sampled_every_step():
    """The sampled launch bench.py times (Llama-3.2-1B shape, 64 steps, T 0.6, top-k 20, top-p
    0.95), every step against the oracle teacher-forced on the GPU's tokens with the same
    uniforms; the timed configuration (no debug buffers, no logits) gives the same tokens and
    cache bytes."""
    key = "llama1b_sampled"
    wl = WORKLOADS[key]
    m, n = wl.model, wl.n_steps
    s = Setup(m, wl.capacity, wl.n_cached, gen_device="cuda")
    tok = synth.make_tokens(m, 1)[0]
    u = synth.make_uniforms(m, n)
    kv_timed = s.fresh_kv()
    with s.plan(flags=0, sampling=wl.sampling) as plan:
        out_t = torch.zeros(n, dtype=torch.int32, device="cuda")
        plan.decode(kv_timed, tok, n, out_t, None, uniforms=torch.from_numpy(u).cuda())
        assert plan.status() == tiles.TILES_OK, tiles.last_error()
        timed_tokens = out_t.cpu().numpy().astype(np.int64)
    kv = s.fresh_kv()
    with s.plan(sampling=wl.sampling) as plan:
        g_t, g_l, g_h = run_gpu_sampled(plan, kv, tok, n, u)
    assert np.array_equal(timed_tokens, g_t), "timed configuration gives other tokens"
    assert torch.equal(kv_timed.k.view(torch.int16), kv.k.view(torch.int16))
    assert torch.equal(kv_timed.v.view(torch.int16), kv.v.view(torch.int16))
    del kv_timed
    print(f"{key}: GPU launch of {n} steps done; teacher-forced oracle for all {n} steps", flush=True)
    okv = s.oracle_kv()
    o_res = s.oracle().decode(okv, tok, wl.n_cached, n, teacher=[int(t) for t in g_t[:-1]], widen_kv_once=True,
                              sampling=wl.sampling, uniforms=u)
    stats = compare_sampled_teacher_forced(key, g_t, g_l, g_h, o_res, wl.sampling, u)
    assert stats["steps"] == n and stats["draws_exact"] >= n // 2
    print(f"{key}: {n} of {n} steps compared; max hidden rel L2 {stats['hidden_rel_l2_max']:.2e}, max logit abs err "
          f"{stats['logit_abs_max']:.2e}, draws compared exactly {stats['draws_exact']} of {n}; distinct tokens "
          f"{len(set(g_t.tolist()))}", flush=True)



# ---------------------------------------------------------------------------
# INT8 KV cache with smoothed keys
# ---------------------------------------------------------------------------

def test_kv8_conversion_matches_the_oracle_bit_for_bit():
    """The library's conversion of a BF16 cache prefix (smoothing factors, codes, scales) equals the
    oracle's bit for bit (the same FP32 operations, correctly rounded divisions)."""
    from oracle import convert_kv_int8

    for m, cap, cached in ((TINY, 40, 29), (QK128, 64, 37), (TINY, 16, 0)):
        s = Setup(m, cap, cached, key_scale=True)
        with s.plan(kv_format="int8") as plan:
            assert plan.info().kv_format == 1
            kv = tiles.KVCache.convert_int8(plan, s.k0, s.v0, cached)
            torch.cuda.synchronize()
        o = convert_kv_int8(s.kv_bits, cached)
        kq, vq, ks, vs, sg = split_int8_cache(kv)
        assert kv.length == cached
        assert np.array_equal(sg, o["sigma"])
        assert np.array_equal(kq[:, :, :cached], o["kq"][:, :, :cached])
        assert np.array_equal(vq[:, :, :cached], o["vq"][:, :, :cached])
        assert np.array_equal(ks[:, :, :cached], o["ks"][:, :, :cached])
        assert np.array_equal(vs[:, :, :cached], o["vs"][:, :, :cached])


def test_kv8_tiny_every_step_against_oracle():
    wl = WORKLOADS["tiny"]
    s = Setup(TINY, wl.capacity, 0, kv="int8")
    prompt = synth.make_tokens(TINY, wl.prompt_len)
    with s.plan() as plan:
        _oracle_forced(s, prompt, wl.prompt_len + wl.n_steps, plan, tag="tiny kv8")


@pytest.mark.parametrize("heads", [0, 2, 4])
def test_kv8_qk_norm_head_dim_128_with_outlier_keys(heads):
    # cached keys with per-channel scales U(0.5, 4): what the smoothing is for
    s = Setup(QK128, 64, 37, key_scale=True, kv="int8")
    with s.plan(attn_heads=heads) as plan:
        _oracle_forced(s, synth.make_tokens(QK128, 1), 10, plan, tag=f"qk128 kv8 heads {heads}")


@pytest.mark.parametrize("splits,mode", [(1, 1), (3, 2), (7, 2)])
def test_kv8_split_counts_ragged_and_wide(splits, mode):
    s = Setup(RAGGED, 48, 30, kv="int8")
    with s.plan(kv_splits=splits, combine_mode=mode) as plan:
        _oracle_forced(s, synth.make_tokens(RAGGED, 1), 6, plan, tag=f"ragged kv8 S{splits}")
    s = Setup(WIDE, 96, 70, kv="int8")
    with s.plan() as plan:
        _oracle_forced(s, synth.make_tokens(WIDE, 1), 6, plan, tag="wide kv8")


def test_kv8_repeatable_chunk_invariant_and_poison_at_capacity():
    """Bit-identical repeats; one-step launches equal the multi-step launch; with the cache filled to
    capacity, poisoned (NaN) scales of the rows a launch writes change nothing."""
    s = Setup(WIDE, 80, 70, kv="int8")
    tok = synth.make_tokens(WIDE, 1)[0]
    n = 10
    with s.plan() as plan:
        kv_a = s.fresh_kv(plan)
        a = run_gpu(plan, kv_a, tok, n)
        kv_b = s.fresh_kv(plan)
        b = run_gpu(plan, kv_b, tok, n)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1].view(np.uint32), b[1].view(np.uint32))
        assert torch.equal(kv_a.k, kv_b.k) and torch.equal(kv_a.k_scale, kv_b.k_scale)
        kv = s.fresh_kv(plan)
        t = tok
        for i in range(n):
            t1, l1, _ = run_gpu(plan, kv, t, 1, want_hidden=False)
            assert int(t1[0]) == int(a[0][i])
            assert np.array_equal(l1[0].view(np.uint32), a[1][i].view(np.uint32))
            t = int(t1[0])
        assert torch.equal(kv.k, kv_a.k) and torch.equal(kv.v_scale, kv_a.v_scale)
    with s.plan(flags=tiles.TILES_POISON | tiles.TILES_DEBUG_HIDDEN) as plan:
        kv_p = s.fresh_kv(plan)
        p = run_gpu(plan, kv_p, tok, n)
    assert kv_p.length == kv_p.capacity
    assert np.array_equal(a[0], p[0]) and np.array_equal(a[1].view(np.uint32), p[1].view(np.uint32))
    assert torch.equal(kv_p.k, kv_a.k) and torch.equal(kv_p.k_scale, kv_a.k_scale)


def test_kv8_entry_point_errors():
    s = Setup(TINY, 40, 10, kv="int8")
    with s.plan() as plan:
        kv = s.fresh_kv(plan)
        out = torch.zeros(2, dtype=torch.int32, device="cuda")
        bad = tiles.KVCache(kv.k, None, kv.length, kv.k_scale, None, kv.k_smooth)
        c = bad.struct()
        assert tiles.lib().tiles_decode(plan._h, ctypes.byref(c), 0, 2, out.data_ptr(), None) == tiles.TILES_E_ARG
        assert "k_scale" in tiles.last_error()
        with pytest.raises(tiles.TilesError):
            tiles.KVCache.convert_int8(plan, s.k0, s.v0, 41)  # length beyond the capacity
    s16 = Setup(TINY, 40, 10)
    with s16.plan() as plan:  # a BF16 plan converts nothing
        with pytest.raises(tiles.TilesError):
            tiles.KVCache.convert_int8(plan, s16.k0, s16.v0, 10)


FULL_KV8 = ["qwen4b_32k_kv8", "llama1b_kv8"]


@pytest.mark.slow
@pytest.mark.timeout(900)
@pytest.mark.parametrize("key", FULL_KV8)
def test_full_size_kv8_every_step(key):
    """The INT8 KV launch bench.py times, every step against the oracle teacher-forced on the GPU's
    tokens (its own INT8 cache converted from the same BF16 prefix); the timed configuration gives the
    same tokens and cache bytes."""
    wl = WORKLOADS[key]
    m, n = wl.model, wl.n_steps
    s = Setup(m, wl.capacity, wl.n_cached, key_scale=wl.key_scale, gen_device="cuda", kv="int8")
    tok = synth.make_tokens(m, 1)[0]
    with s.plan(flags=0) as plan:
        kv_timed = s.fresh_kv(plan)
        out_t = torch.zeros(n, dtype=torch.int32, device="cuda")
        plan.decode(kv_timed, tok, n, out_t, None)
        assert plan.status() == tiles.TILES_OK, tiles.last_error()
        timed_tokens = out_t.cpu().numpy().astype(np.int64)
    with s.plan() as plan:
        kv = s.fresh_kv(plan)
        g_t, g_l, g_h = run_gpu(plan, kv, tok, n)
    assert np.array_equal(timed_tokens, g_t), "timed configuration gives other tokens"
    assert torch.equal(kv_timed.k, kv.k) and torch.equal(kv_timed.k_scale, kv.k_scale)
    del kv_timed
    print(f"{key}: GPU launch of {n} steps done; teacher-forced oracle for all {n} steps", flush=True)
    okv = s.oracle_kv()
    o_res = s.oracle().decode(okv, tok, wl.n_cached, n, teacher=[int(t) for t in g_t[:-1]], widen_kv_once=True)
    stats = compare_teacher_forced(key, g_t, g_l, g_h, o_res)
    assert stats["steps"] == n
    rows = kv8_rows_close(key, kv, okv, wl.n_cached, n)
    print(f"{key}: {n} of {n} steps compared; max hidden rel L2 {stats['hidden_rel_l2_max']:.2e}, max logit abs err "
          f"{stats['logit_abs_max']:.2e}, tokens checked at margin > 0.1: {stats['tokens_checked']}; written rows "
          f"(dequantized rel L2, codes differing, scale rel) K {rows['K'][0]:.2e} {rows['K'][1]:.3%} {rows['K'][2]:.1e}, "
          f"V {rows['V'][0]:.2e} {rows['V'][1]:.3%} {rows['V'][2]:.1e}", flush=True)


# ---------------------------------------------------------------------------------------------
# greedy verify steps (tiles_verify)
# ---------------------------------------------------------------------------------------------

def _greedy_continuation(s, plan, tok, n):
    """The GPU's own free-running greedy tokens, logits and cache after n steps from a fresh cache."""
    kv = s.fresh_kv(plan)
    g_t, g_l, _ = run_gpu(plan, kv, tok, n, want_hidden=False)
    return kv, [int(t) for t in g_t], g_l


@pytest.mark.parametrize("kvfmt,weights", [("bf16", "bf16"), ("int8", "bf16"), ("bf16", "int8")])
def test_verify_of_the_greedy_continuation_is_the_greedy_launch_bit_for_bit(kvfmt, weights):
    """Drafts equal to the launch's own greedy tokens: every draft accepted, the argmaxes, logits and
    written cache bytes identical to the free-running launch (each position consumes the same token),
    and the verified output is that continuation one token further (BF16 or INT8 cache, BF16 or INT8
    weights)."""
    s = Setup(WIDE, 96, 60, kv=kvfmt, weights=weights)
    tok = synth.make_tokens(WIDE, 1)[0]
    m = 12
    with s.plan() as plan:
        kv_g, g, g_l = _greedy_continuation(s, plan, tok, m)
        kv = s.fresh_kv(plan)
        out_l = torch.zeros((m, WIDE.vocab), dtype=torch.float32, device="cuda")
        a, n, out = plan.verify(kv, [tok] + g[:m - 1], out_logits=out_l)
    assert n == m - 1 and list(a) == g and list(out) == g
    assert np.array_equal(out_l.cpu().numpy(), g_l)
    assert torch.equal(kv.k, kv_g.k) and (kv.v is None or torch.equal(kv.v, kv_g.v))
    if kv.int8:
        assert torch.equal(kv.k_scale, kv_g.k_scale) and torch.equal(kv.v_scale, kv_g.v_scale)
    assert kv.length == 60 + m


def test_verify_wrong_drafts_against_the_oracle():
    """A wrong draft at position j: the GPU accepts j - 1 drafts and yields the greedy token there, as
    the oracle's verify does; every position's logits and hidden states against the oracle
    teacher-forced on the same tokens."""
    s = Setup(WIDE, 96, 60)
    tok = synth.make_tokens(WIDE, 1)[0]
    m = 10
    with s.plan() as plan:
        _, g, _ = _greedy_continuation(s, plan, tok, m)
        for j in (1, 4, 9):
            drafts = list(g[:m - 1])
            drafts[j - 1] = (g[j - 1] + 7) % WIDE.vocab
            tokens = [tok] + drafts
            kv = s.fresh_kv(plan)
            out_l = torch.zeros((m, WIDE.vocab), dtype=torch.float32, device="cuda")
            a, n, out = plan.verify(kv, tokens, out_logits=out_l)
            hid = plan.read_debug(hidden=True)[0]
            o = s.oracle()
            o_dec = o.decode(s.oracle_kv(), tokens[0], 60, m, teacher=tokens[1:])
            compare_teacher_forced(f"verify j={j}", a, out_l.cpu().numpy(), hid, o_dec)
            o_ver = o.verify(s.oracle_kv(), tokens, 60)
            margins = [top2_margin(o_dec["logits"][i]) for i in range(m)]
            if min(margins[:j]) > MARGIN:  # every decision up to the wrong draft is clear
                assert n == o_ver["accepted"] == j - 1, (j, n, o_ver["accepted"])
                assert list(out) == list(o_ver["tokens"]) == g[:j]


@pytest.mark.slow
@pytest.mark.timeout(600)
def test_full_size_verify_sixteen_tokens():
    """A 16-token verify step on the Llama-3.2-1B shape at 1023 cached positions, drafts the GPU's own
    greedy continuation with a wrong token at position 10: nine accepted, and all 16 positions against
    the oracle teacher-forced on the same tokens."""
    wl = WORKLOADS["llama1b"]
    mdl = wl.model
    s = Setup(mdl, wl.capacity, wl.n_cached, gen_device="cuda")
    tok = synth.make_tokens(mdl, 1)[0]
    m = 16
    with s.plan(flags=0) as plan:
        _, g, _ = _greedy_continuation(s, plan, tok, m)
        drafts = list(g[:m - 1])
        drafts[9] = (g[9] + 1) % mdl.vocab
        tokens = [tok] + drafts
        kv = s.fresh_kv(plan)
        out_l = torch.zeros((m, mdl.vocab), dtype=torch.float32, device="cuda")
        a, n, out = plan.verify(kv, tokens, out_logits=out_l)
    assert n == 9 and list(out) == g[:10]
    o_dec = s.oracle().decode(s.oracle_kv(), tokens[0], wl.n_cached, m, teacher=tokens[1:], keep_hidden=True,
                              widen_kv_once=True)
    stats = compare_teacher_forced("llama1b verify", a, out_l.cpu().numpy(), None, o_dec)
    print(f"llama1b verify: {m} positions compared, accepted {n}; max logit abs err {stats['logit_abs_max']:.2e}",
          flush=True)


def test_verify_of_sixty_four_positions_to_capacity():
    """The longest verify step (64 positions) ending exactly at the cache's capacity, without logits:
    with drafts the greedy continuation every draft is accepted and the argmaxes equal the greedy
    launch's; the cache length the binding reports is the one before the call + 64."""
    s = Setup(TINY, 74, 10)
    tok = synth.make_tokens(TINY, 1)[0]
    with s.plan() as plan:
        kv_g, g, _ = _greedy_continuation(s, plan, tok, 64)
        kv = s.fresh_kv(plan)
        a, n, out = plan.verify(kv, [tok] + g[:63])
        assert n == 63 and list(a) == g and list(out) == g
        assert kv.length == 74
        assert torch.equal(kv.k, kv_g.k) and torch.equal(kv.v, kv_g.v)
        kv = s.fresh_kv(plan)
        kv.length = 11  # one position past what 64 more fit
        with pytest.raises(tiles.TilesError):
            plan.verify(kv, [tok] + g[:63])


# ---------------------------------------------------------------------------------------------
# verify plans: tokens_per_step consecutive positions through every tile per step
# ---------------------------------------------------------------------------------------------

# (shape, positions per step, weights, combine_mode: 0 planner choice -- the o_proj prologue where the
# LDS holds it, else a wave of its own --, or 2, the splits merged in a wave of their own)
VERIFY_PLANS = [("tiny", 2, "bf16", 0), ("tiny", 3, "bf16", 0), ("tiny", 4, "bf16", 0), ("wide", 2, "bf16", 0),
                ("wide", 3, "bf16", 0), ("wide", 2, "int8", 0), ("wide", 3, "int8", 0), ("wide", 2, "bf16", 2),
                ("tiny", 4, "bf16", 2)]


def _verify_plan_case(s, plan, tag, tokens, pos, check_hidden=True):
    """One verify call of a verify plan against the oracle: every position's argmax, logits (and hidden
    states) teacher-forced on the same tokens, the K/V rows written for every position, and the
    accepted count and verified tokens against the oracle's verify where its decisions are clear."""
    m = len(tokens)
    mdl = s.m
    kv = s.fresh_kv(plan)
    kv.length = pos
    out_l = torch.zeros((m, mdl.vocab), dtype=torch.float32, device="cuda")
    a, n, out = plan.verify(kv, tokens, out_logits=out_l)
    hid = plan.read_debug(hidden=True)[0] if check_hidden else None
    o = s.oracle()
    okv = s.oracle_kv()
    o_dec = o.decode(okv, tokens[0], pos, m, teacher=tokens[1:], widen_kv_once=True)
    stats = compare_teacher_forced(tag, a, out_l.cpu().numpy(), hid, o_dec)
    if s.kv == "int8":
        kv8_rows_close(tag, kv, okv, pos, m)
    else:
        kv_rows_close(f"{tag} K", kv.k, okv["k"], pos, m)
        kv_rows_close(f"{tag} V", kv.v, okv["v"], pos, m)
    o_acc = 0
    while o_acc < m - 1 and int(o_dec["tokens"][o_acc]) == tokens[o_acc + 1]:
        o_acc += 1
    margins = [top2_margin(o_dec["logits"][i]) for i in range(m)]
    if min(margins[:o_acc + 1]) > MARGIN:  # every decision the acceptance depends on is clear
        assert n == o_acc, (tag, n, o_acc)
        assert list(out) == list(tokens[1:n + 1]) + [int(o_dec["tokens"][n])]
    assert kv.length == pos + n + 1
    return a, n, stats


@pytest.mark.parametrize("shape,mt,weights,combine", VERIFY_PLANS,
                         ids=[f"{a}-{b}-{c}-c{d}" for a, b, c, d in VERIFY_PLANS])
def test_verify_plan_against_the_oracle(shape, mt, weights, combine):
    """A verify plan (mt positions per step through every tile, BF16 or INT8 weights, the splits merged
    in the o_proj prologue or in a wave of their own), drafts the decode plan's greedy continuation,
    whole or with a wrong token at position 3 or 8: every position against the oracle teacher-forced
    on the same tokens, the written K/V rows, and the acceptance against the oracle's."""
    mdl = TINY if shape == "tiny" else WIDE
    s = Setup(mdl, 96, 60, weights=weights)
    tok = synth.make_tokens(mdl, 1)[0]
    m = 12
    with s.plan() as dplan:
        _, g, _ = _greedy_continuation(s, dplan, tok, m)
    with s.plan(tokens_per_step=mt, combine_mode=combine) as plan:
        info = plan.info()
        assert info.tokens_per_step == mt and (info.combine_mode == combine if combine else info.combine_mode in (1, 2))
        for j in (None, 3, 8):
            drafts = list(g[:m - 1])
            if j is not None:
                drafts[j - 1] = (g[j - 1] + 7) % mdl.vocab
            tag = f"{shape} mt={mt} {weights} combine={info.combine_mode} j={j}"
            _, n, stats = _verify_plan_case(s, plan, tag, [tok] + drafts, 60)
            print(f"{tag}: accepted {n}; max hidden rel L2 {stats['hidden_rel_l2_max']:.2e}, max logit abs err "
                  f"{stats['logit_abs_max']:.2e}, tokens checked {stats['tokens_checked']}", flush=True)


@pytest.mark.parametrize("shape,mt,kvfmt", [("tiny", 3, "bf16"), ("wide", 2, "int8"), ("qk128", 4, "bf16")])
def test_verify_plan_repeatable_and_chunk_invariant(shape, mt, kvfmt):
    """A verify plan's results repeat bit for bit (argmax, logits, accepted count, every cache byte),
    and one call of 12 positions equals two calls split at a step boundary (6 + 6, or 8 + 4 at 4
    positions per step), with drafts that are all accepted, bit for bit."""
    mdl = {"tiny": TINY, "wide": WIDE, "qk128": QK128}[shape]
    s = Setup(mdl, 96, 60, kv=kvfmt)
    tok = synth.make_tokens(mdl, 1)[0]
    m = 12
    with s.plan() as dplan:
        _, g, _ = _greedy_continuation(s, dplan, tok, m)
    g = [int(x) for x in g]

    def cache_bytes(kv):
        if kvfmt == "int8":
            return [kv.k.clone(), kv.k_scale.clone(), kv.v_scale.clone()]
        return [kv.k.clone(), kv.v.clone()]

    def run(plan, calls):
        kv = s.fresh_kv(plan)
        kv.length = 60
        argmax, logits, accepted = [], [], []
        for toks in calls:
            out_l = torch.zeros((len(toks), mdl.vocab), dtype=torch.float32, device="cuda")
            a, n, _ = plan.verify(kv, toks, out_logits=out_l)
            argmax += [int(x) for x in a]
            logits.append(out_l.cpu().numpy().view(np.uint32))
            accepted.append(n)
        return argmax, np.concatenate(logits), accepted, cache_bytes(kv), kv.length

    drafts = list(g[:m - 1])
    drafts[6] = (g[6] + 9) % mdl.vocab
    c1 = 8 if mt == 4 else 6
    with s.plan(tokens_per_step=mt) as plan:
        assert plan.info().tokens_per_step == mt
        r1 = run(plan, [[tok] + drafts])
        r2 = run(plan, [[tok] + drafts])
        assert r1[0] == r2[0] and np.array_equal(r1[1], r2[1]) and r1[2] == r2[2] and r1[4] == r2[4]
        assert all(torch.equal(x, y) for x, y in zip(r1[3], r2[3]))
        # drafts the plan accepts in full: the decode plan's continuation, corrected with this plan's own
        # argmax wherever a near-tie decides otherwise
        seq = list(g[:m - 1])
        for _ in range(m):
            whole = run(plan, [[tok] + seq])
            if whole[2][0] == m - 1:
                break
            seq[whole[2][0]] = whole[0][whole[2][0]]
        assert whole[2] == [m - 1], whole[2]
        split = run(plan, [[tok] + seq[:c1 - 1], [seq[c1 - 1]] + seq[c1:m - 1]])
        assert split[2] == [c1 - 1, m - c1 - 1], split[2]
        assert whole[0] == split[0] and np.array_equal(whole[1], split[1]) and whole[4] == split[4]
        assert all(torch.equal(x, y) for x, y in zip(whole[3], split[3]))
    print(f"{shape} mt={mt} {kvfmt}: repeats and a {c1} + {m - c1} split identical; accepted {r1[2][0]} of the "
          f"drafts with a wrong token at position 7", flush=True)


@pytest.mark.parametrize("shape,heads,mt", [("qk128", 1, 2), ("qk128", 2, 2), ("tiny", 2, 2), ("qk128", 1, 3),
                                             ("qk128", 1, 4)])
def test_verify_plan_heads_per_attention_tile(shape, heads, mt):
    """Verify plans with 1 or 2 query heads per attention tile at 2 positions (2 or 4 query rows), and
    with head_dim 128 at 3 and 4 positions (the RoPE rows of 4 x 128 dimensions beside the attention
    tile's areas), q/k norm, against the oracle as above."""
    mdl = QK128 if shape == "qk128" else TINY
    s = Setup(mdl, 64, 29)
    tok = synth.make_tokens(mdl, 1)[0]
    m = 10
    with s.plan() as dplan:
        _, g, _ = _greedy_continuation(s, dplan, tok, m)
    drafts = list(g[:m - 1])
    drafts[5] = (g[5] + 3) % mdl.vocab
    m = m - m % mt
    with s.plan(tokens_per_step=mt, attn_heads=heads) as plan:
        assert plan.info().attn_heads == heads
        _, n, stats = _verify_plan_case(s, plan, f"{shape} mt={mt} heads/tile={heads}", [tok] + drafts[:m - 1], 29)
    print(f"{shape} mt={mt} heads/tile={heads}: accepted {n}; {stats}", flush=True)


# Qwen3-4B widths (head_dim 128, q/k norm, 4 query heads per KV head) on two layers, FFN 12288: a
# 2-position verify plan with 2 heads per attention tile and 16 splits has no LDS room for staging
W128 = scaled(TINY, name="wide128-2layer", n_layers=2, hidden=2560, n_heads=32, n_kv_heads=8, head_dim=128, ffn=12288,
              vocab=4096, qk_norm=True, rms_eps=1e-6, rope_theta=1e6)


def test_verify_plan_without_staging():
    """A verify plan whose LDS holds no staging batch (the case of the Qwen3-4B shape at 32K positions),
    2 query heads per tile, 16 splits merged in their own wave, ~1000 cached positions: against the
    oracle as above."""
    s = Setup(W128, 1100, 1000)
    tok = synth.make_tokens(W128, 1)[0]
    m = 8
    with s.plan() as dplan:
        assert dplan.info().stage_batches >= 1
        _, g, _ = _greedy_continuation(s, dplan, tok, m)
    with s.plan(tokens_per_step=2, attn_heads=2, kv_splits=16, combine_mode=2) as plan:
        info = plan.info()
        assert (info.stage_batches, info.attn_heads, info.kv_splits) == (0, 2, 16)
        _, n, stats = _verify_plan_case(s, plan, "no staging", [tok] + g[:m - 1], 1000)
    print(f"no staging: accepted {n}; {stats}", flush=True)


def test_verify_plan_split_boundary_inside_a_step():
    """7 splits, a 2-position step at positions 41 and 42 with the last split starting at 42: position 42's
    row sees it, position 41's sees none of that split (an empty partial that the merge must drop);
    later steps keep both positions in one split.  Against the oracle as above."""
    mdl = scaled(TINY, name="tiny-long")
    s = Setup(mdl, 120, 41)
    tok = synth.make_tokens(mdl, 1)[0]
    m = 12
    with s.plan() as dplan:
        _, g, _ = _greedy_continuation(s, dplan, tok, m)
    for combine in (1, 2):
        with s.plan(tokens_per_step=2, kv_splits=7, combine_mode=combine) as plan:
            assert plan.info().kv_splits == 7
            _, n, stats = _verify_plan_case(s, plan, f"split boundary combine={combine}", [tok] + g[:m - 1], 41)
        print(f"split boundary combine={combine}: accepted {n}; {stats}", flush=True)


@pytest.mark.parametrize("shape,mt", [("tiny", 2), ("tiny", 3), ("wide", 2), ("qk128", 2), ("qk128", 3)])
def test_verify_plan_int8_kv(shape, mt):
    """Verify plans with the INT8 KV cache (each of the step's rows quantized in the attention prologue,
    its scales beside the split's staged ones): drafts the INT8-cache decode plan's greedy continuation
    with a wrong token at position 6, every position and the written codes and scales against the
    oracle's INT8 cache teacher-forced on the same tokens, and the acceptance against the oracle's."""
    mdl = {"tiny": TINY, "wide": WIDE, "qk128": QK128}[shape]
    s = Setup(mdl, 96, 60, kv="int8")
    tok = synth.make_tokens(mdl, 1)[0]
    m = 12
    with s.plan() as dplan:
        _, g, _ = _greedy_continuation(s, dplan, tok, m)
    drafts = list(g[:m - 1])
    drafts[5] = (g[5] + 5) % mdl.vocab
    m = m - m % mt
    with s.plan(tokens_per_step=mt) as plan:
        assert plan.info().kv_format == 1 and plan.info().tokens_per_step == mt
        _, n, stats = _verify_plan_case(s, plan, f"{shape} int8 kv mt={mt}", [tok] + drafts[:m - 1], 60)
    print(f"{shape} int8 kv mt={mt}: accepted {n}; max hidden rel L2 {stats['hidden_rel_l2_max']:.2e}, max logit abs "
          f"err {stats['logit_abs_max']:.2e}", flush=True)


def test_verify_plan_of_sixty_four_positions_to_capacity():
    """A 4-position verify plan over 64 positions (16 steps) ending exactly at the cache's capacity, the
    drafts the greedy continuation: against the oracle; one position more is rejected."""
    s = Setup(TINY, 74, 10)
    tok = synth.make_tokens(TINY, 1)[0]
    with s.plan() as dplan:
        _, g, _ = _greedy_continuation(s, dplan, tok, 64)
    with s.plan(tokens_per_step=4) as plan:
        _, n, stats = _verify_plan_case(s, plan, "tiny mt=4 to capacity", [tok] + g[:63], 10)
        print(f"tiny mt=4 64 positions: accepted {n}; {stats}", flush=True)
        kv = s.fresh_kv(plan)
        kv.length = 11
        with pytest.raises(tiles.TilesError):
            plan.verify(kv, [tok] + g[:63])


def test_verify_plan_entry_point_errors():
    """A verify plan runs tiles_verify only, with m a multiple of its positions per step; a plan that
    cannot hold the step's input vectors is not created."""
    s = Setup(TINY, 40, 10)
    with s.plan(tokens_per_step=2) as plan:
        kv = s.fresh_kv(plan)
        L = tiles.lib()
        c = kv.struct()
        out = torch.zeros(8, dtype=torch.int32, device="cuda")
        for toks in ([1, 2, 3], [1]):
            buf = (ctypes.c_int32 * len(toks))(*toks)
            assert L.tiles_verify(plan._h, ctypes.byref(c), buf, len(toks), ctypes.c_void_p(out.data_ptr()),
                                  None) == tiles.TILES_E_ARG
            assert "multiple" in tiles.last_error()
        assert L.tiles_decode(plan._h, ctypes.byref(c), 1, 2, ctypes.c_void_p(out.data_ptr()), None) == tiles.TILES_E_ARG
        assert "tiles_verify" in tiles.last_error()
        assert L.tiles_decode_noalloc(plan._h, ctypes.byref(c), 1, 2, ctypes.c_void_p(out.data_ptr()),
                                      None) == tiles.TILES_E_ARG
        assert kv.length == 10
    with pytest.raises(tiles.TilesError):
        Setup(WIDE, 40, 10).plan(tokens_per_step=4)


@pytest.mark.slow
@pytest.mark.timeout(600)
@pytest.mark.parametrize("mt", [2, 3])
def test_full_size_verify_plan_sixteen_tokens(mt):
    """A verify step of 16 positions (2-position plan) or 15 (3-position plan) on the Llama-3.2-1B shape at
    1023 cached positions, drafts the decode plan's greedy continuation with a wrong token at position
    10: every position and the written K/V rows against the oracle teacher-forced on the same tokens,
    and the acceptance against the oracle's."""
    wl = WORKLOADS["llama1b"]
    mdl = wl.model
    s = Setup(mdl, wl.capacity, wl.n_cached, gen_device="cuda")
    tok = synth.make_tokens(mdl, 1)[0]
    m = 16 - 16 % mt
    with s.plan(flags=0) as dplan:
        _, g, _ = _greedy_continuation(s, dplan, tok, m)
    drafts = list(g[:m - 1])
    drafts[9] = (g[9] + 1) % mdl.vocab
    with s.plan(flags=0, tokens_per_step=mt) as plan:
        _, n, stats = _verify_plan_case(s, plan, f"llama1b verify plan mt={mt}", [tok] + drafts, wl.n_cached,
                                        check_hidden=False)
    print(f"llama1b verify plan mt={mt}: {m} positions compared, accepted {n}; max logit abs err "
          f"{stats['logit_abs_max']:.2e}, "
          f"tokens checked {stats['tokens_checked']}", flush=True)


def test_verify_entry_point_errors():
    s = Setup(TINY, 40, 10)
    with s.plan() as plan:
        kv = s.fresh_kv(plan)
        L = tiles.lib()
        c = kv.struct()
        out = torch.zeros(4, dtype=torch.int32, device="cuda")
        for toks, m in (([1, 2], 0), ([1] * 65, 65), ([1, TINY.vocab], 2), ([-1], 1)):
            buf = (ctypes.c_int32 * len(toks))(*toks)
            assert L.tiles_verify(plan._h, ctypes.byref(c), buf, m, ctypes.c_void_p(out.data_ptr()), None) == tiles.TILES_E_ARG
        assert L.tiles_verify(plan._h, ctypes.byref(c), None, 1, ctypes.c_void_p(out.data_ptr()), None) == tiles.TILES_E_ARG
    s = Setup(TINY, 40, 10)
    with s.plan(sampling=(1.0, 4, 1.0)) as plan:
        kv = s.fresh_kv(plan)
        c = kv.struct()
        buf = (ctypes.c_int32 * 1)(1)
        assert tiles.lib().tiles_verify(plan._h, ctypes.byref(c), buf, 1, ctypes.c_void_p(out.data_ptr()), None) == tiles.TILES_E_ARG
        assert "greedy" in tiles.last_error()


def test_kv8_splits_longer_than_2048_positions():
    """INT8 KV splits of up to 3,000 positions (the split's scale areas sized to the plan's longest
    split, 3,008 positions, staged in 6 loads per wavefront): a decode plan and a 2-position verify plan
    with 2 forced splits after 5,900 cached positions, against the oracle's INT8 cache as above."""
    mdl = scaled(TINY, name="tiny-6k")
    s = Setup(mdl, 6000, 5900, key_scale=True, kv="int8")
    tok = synth.make_tokens(mdl, 1)[0]
    with s.plan(kv_splits=2) as plan:
        assert plan.info().kv_splits == 2
        _oracle_forced(s, [tok], 6, plan, tag="kv8 3000-position splits")
    m = 8
    with s.plan(kv_splits=2) as dplan:
        _, g, _ = _greedy_continuation(s, dplan, tok, m)
    drafts = list(g[:m - 1])
    drafts[4] = (g[4] + 5) % mdl.vocab
    with s.plan(kv_splits=2, tokens_per_step=2) as plan:
        assert (plan.info().kv_splits, plan.info().tokens_per_step) == (2, 2)
        _, n, stats = _verify_plan_case(s, plan, "kv8 3000-position splits mt=2", [tok] + drafts, 5900)
    print(f"kv8 3000-position splits mt=2: accepted {n}; {stats}", flush=True)


@pytest.mark.slow
@pytest.mark.timeout(900)
@pytest.mark.parametrize("kv", ["bf16", "int8"])
def test_full_size_verify_plan_at_32k_positions(kv):
    """An 8-position step of a 2-position verify plan on the Qwen3-4B shape after 32767 cached positions
    (16 splits, 2 query heads per attention tile, the splits merged in a wave of their own; INT8 KV:
    splits of up to 2,050 positions), drafts the decode plan's greedy continuation: all 8 positions and
    the written K/V rows (codes and scales) against the oracle teacher-forced on the same tokens, and
    the acceptance against the oracle's."""
    key = "qwen4b_32k" if kv == "bf16" else "qwen4b_32k_kv8"
    wl = WORKLOADS[key]
    mdl = wl.model
    s = Setup(mdl, wl.capacity, wl.n_cached, key_scale=wl.key_scale, gen_device="cuda", kv=kv)
    tok = synth.make_tokens(mdl, 1)[0]
    m = 8
    with s.plan(flags=0) as dplan:
        _, g, _ = _greedy_continuation(s, dplan, tok, m)
    with s.plan(flags=0, tokens_per_step=2) as plan:
        info = plan.info()
        assert (info.kv_splits, info.attn_heads, info.combine_mode) == (16, 2, 2)
        _, n, stats = _verify_plan_case(s, plan, f"{key} verify plan", [tok] + g[:m - 1], wl.n_cached,
                                        check_hidden=False)
    print(f"{key} verify plan: {m} positions compared, accepted {n}; max logit abs err "
          f"{stats['logit_abs_max']:.2e}, tokens checked {stats['tokens_checked']}, smallest oracle margin "
          f"{stats['min_margin']:.3f}", flush=True)
