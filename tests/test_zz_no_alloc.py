"""The allocation-free decode entry point (tiles_decode_noalloc, called through the C ABI) against
tiles_decode: the same tokens, logits, hidden states and cache bytes, bit for bit, on two calls in a
row (the second with a smaller model and fewer steps, so it runs on what the first left in the shared
scratch array), and a clear rejection of a plan whose scratch does not fit the array."""

import numpy as np
import pytest
import torch

from tile_scheduled_persistent_amd import synth, tiles
from tile_scheduled_persistent_amd.configs import TINY, scaled

from parity_util import Setup

pytestmark = pytest.mark.gpu

WIDE = scaled(TINY, name="wide-2layer", n_layers=2, hidden=2048, n_heads=32, n_kv_heads=8, head_dim=64, ffn=8192,
              vocab=4096, rms_eps=1e-5, rope_theta=5e5)


def _launch(s, plan, tok, n, noalloc):
    kv = s.fresh_kv()
    out_t = torch.zeros(n, dtype=torch.int32, device="cuda")
    out_l = torch.zeros((n, s.m.vocab), dtype=torch.float32, device="cuda")
    plan.decode(kv, tok, n, out_t, out_l, noalloc=noalloc)
    assert plan.status() == tiles.TILES_OK, tiles.last_error()
    torch.cuda.synchronize()
    hid = plan.read_debug(hidden=True)[0]
    return out_t.cpu().numpy(), out_l.cpu().numpy(), hid, kv


def _same(a, b):
    assert np.array_equal(a[0], b[0])
    assert np.array_equal(a[1].view(np.uint32), b[1].view(np.uint32))
    assert np.array_equal(a[2].view(np.uint32), b[2].view(np.uint32))
    assert torch.equal(a[3].k.view(torch.int16), b[3].k.view(torch.int16))
    assert torch.equal(a[3].v.view(torch.int16), b[3].v.view(torch.int16))


def test_noalloc_matches_tiles_decode_on_two_calls_in_a_row():
    cases = [(WIDE, 96, 70, 8), (TINY, 24, 10, 3)]  # the second call: a smaller plan, fewer steps
    setups = [Setup(m, cap, cached) for m, cap, cached, _ in cases]
    toks = [synth.make_tokens(m, 1)[0] for m, *_ in cases]
    plans = [s.plan() for s in setups]
    try:
        got = [_launch(s, p, t, c[3], noalloc=True) for s, p, t, c in zip(setups, plans, toks, cases)]
        ref = [_launch(s, p, t, c[3], noalloc=False) for s, p, t, c in zip(setups, plans, toks, cases)]
        for g, r in zip(got, ref):
            _same(g, r)
        # and once more after the plan-owned path ran: the static array is cleared by each launch
        _same(_launch(setups[1], plans[1], toks[1], cases[1][3], noalloc=True), ref[1])
    finally:
        for p in plans:
            p.close()


def test_noalloc_rejects_a_plan_whose_scratch_does_not_fit():
    # 128 layers with 64 KV splits merged in a wave of their own: about 10 MB of tagged buffers
    m = scaled(TINY, name="tiny-128-layers", n_layers=128)
    s = Setup(m, 16, 4)
    with s.plan(kv_splits=64, combine_mode=2) as plan:
        out = torch.zeros(2, dtype=torch.int32, device="cuda")
        kv = s.fresh_kv()
        with pytest.raises(tiles.TilesError) as e:
            plan.decode(kv, 1, 2, out, noalloc=True)
        assert e.value.code == tiles.TILES_E_ARG and "exceeds" in str(e.value)
        assert kv.length == 4
        plan.decode(kv, 1, 2, out)  # the plan-owned path still serves it
        assert plan.status() == tiles.TILES_OK
