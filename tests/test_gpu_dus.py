"""Device planner of the dilated unmasking rounds against the oracle's schedule (GPU, bit-exact)."""
import numpy as np
import pytest
import torch

import synth
from oracle.dus import dus_rounds
from tests.gpu_util import DEV
from token_skipping_denoise_amd import api

pytestmark = pytest.mark.gpu


def _base_force(seed, B, S):
    # 0 normal, 1 must-activate, 2 locked, mixed so that max(force, mark) is exercised
    vals = synth.randint(seed, (B, S), 8).numpy()
    return np.choose(np.minimum(vals, 3), [0, 0, 1, 2]).astype(np.uint8)


def _expected(base, lo, block, a, rounds, r, mark):
    want = base.copy()
    plan = dus_rounds(block, a, rounds=rounds if rounds > 0 else None)
    for o in plan[r]:
        want[:, lo + o] = np.maximum(want[:, lo + o], mark)
    return want


@pytest.mark.parametrize("block,a,rounds", [(1, 2, 0), (2, 2, 0), (3, 2, 0), (5, 3, 0), (16, 2, 0), (17, 2, 0),
                                            (17, 2, 3), (31, 4, 0), (64, 2, 0), (100, 3, 0), (257, 2, 0),
                                            (16, 2, 6)])
def test_dus_mark_matches_schedule(block, a, rounds):
    B, lo = 3, 5
    S = lo + block + 7
    n = len(dus_rounds(block, a, rounds=rounds if rounds > 0 else None))
    for r in range(n):
        for mark in (api.FORCE_ON, api.FORCE_EXCLUDED):
            print(f"dus_mark block={block} a={a} rounds={rounds} round={r} mark={mark}", flush=True)
            base = _base_force(synth.seed_of(block, a, r, mark), B, S)
            force = torch.from_numpy(base).to(DEV)
            api.dus_mark(force, lo, block, r, a=a, rounds=rounds, mark=mark)
            torch.cuda.synchronize()
            got = force.cpu().numpy()
            assert np.array_equal(got, _expected(base, lo, block, a, rounds, r, mark)), f"round {r}"


def test_dus_rounds_cover_block_once():
    """Marking every round of a block on zeros sets each position exactly once (round order recorded)."""
    B, S, lo, block, a = 2, 80, 9, 64, 2
    force = torch.zeros((B, S), dtype=torch.uint8, device=DEV)
    seen = np.zeros((B, S), dtype=np.int64)
    n = len(dus_rounds(block, a))
    for r in range(n):
        force.zero_()
        api.dus_mark(force, lo, block, r, a=a)
        torch.cuda.synchronize()
        seen += force.cpu().numpy().astype(np.int64)
    assert np.all(seen[:, lo:lo + block] == 1)
    assert np.all(seen[:, :lo] == 0) and np.all(seen[:, lo + block:] == 0)


@pytest.mark.parametrize("kw", [dict(lo=0, block=9, round=4), dict(lo=-1, block=4, round=0), dict(lo=8, block=4, round=0),
                                dict(lo=0, block=0, round=0), dict(lo=0, block=4, round=0, a=1),
                                dict(lo=0, block=4, round=0, mark=0), dict(lo=0, block=4, round=-1)])
def test_dus_mark_rejects_bad_arguments(kw):
    force = torch.zeros((2, 10), dtype=torch.uint8, device=DEV)
    args = dict(kw)
    lo, block, r = args.pop("lo"), args.pop("block"), args.pop("round")
    with pytest.raises(api.DllmError):
        api.dus_mark(force, lo, block, r, **args)
    torch.cuda.synchronize()
    assert int(force.sum()) == 0
