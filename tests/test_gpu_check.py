"""The checking build (libdllm_check.so, -DDLLM_CHECK) records violated index and token
preconditions in its device error word while every kernel still stays in bounds and finishes (GPU).

Each case passes a malformed device array that the normal build's kernels already survive (an
out-of-range index marks its row dead, a token id is clamped), so no kernel is made to fault: the
checking build must set the matching bit and otherwise compute exactly what the normal build does.
"""
import ctypes

import pytest
import torch

import synth
from synth import workloads
from token_skipping_denoise_amd import _ffi, api

pytestmark = pytest.mark.gpu
DEV = "cuda"
ACTIVE_COUNT, INDEX_RANGE, INDEX_ORDER, TOKEN_RANGE = 1, 2, 4, 8


def _word(lib):
    w = ctypes.c_uint32()
    assert lib.dllm_check_word(ctypes.byref(w), 1) == 0
    return w.value


def _gather(lib, src, idx, nact, k_max):
    B, S, w = src.shape
    dst = torch.zeros((B * k_max, w), dtype=src.dtype, device=DEV)
    st = lib.dllm_gather_rows(src.data_ptr(), idx.data_ptr(), nact.data_ptr(), B, S, k_max, w, _ffi.DLLM_BF16,
                              dst.data_ptr(), torch.cuda.current_stream().cuda_stream)
    assert st == 0
    torch.cuda.synchronize()
    return dst


def test_gather_preconditions_are_recorded():
    lib = _ffi.load_check()
    _word(lib)
    B, S, w, k_max = 2, 8, 64, 4
    src = synth.normal(synth.seed_of(81), (B, S, w), 1.0, torch.bfloat16).to(DEV)
    cases = [  # (idx rows, n_active, expected bits)
        ([[0, 2, 5, 7], [1, 3, 4, 6]], [4, 3], 0),
        ([[0, 2, 5, 9], [1, 3, 4, 6]], [4, 4], INDEX_RANGE),
        ([[0, 5, 2, 7], [1, 3, 4, 6]], [4, 4], INDEX_ORDER),
        ([[0, 2, 5, 7], [1, 3, 4, 6]], [5, 4], ACTIVE_COUNT),
        ([[0, -3, 5, 7], [6, 3, 4, 6]], [4, 2], INDEX_RANGE | INDEX_ORDER),
    ]
    for rows, na, bits in cases:
        idx = torch.tensor(rows, dtype=torch.int32, device=DEV)
        nact = torch.tensor(na, dtype=torch.int32, device=DEV)
        dst = _gather(lib, src, idx, nact, k_max)
        assert _word(lib) == bits, (rows, na)
        for b in range(B):
            for j in range(min(na[b], k_max)):
                i = rows[b][j]
                if 0 <= i < S:   # every in-range live row is still gathered
                    assert torch.equal(dst[b * k_max + j], src[b, i])


def test_layer_and_step_checks_match_the_normal_build():
    """A layer call with an out-of-range live index and a step with an out-of-range token: the bits
    are set and the outputs are bit-identical to the normal build's on the same inputs."""
    chk, lib = _ffi.load_check(), _ffi.load()
    _word(chk)
    dims = workloads.shrink(workloads.LLADA, n_layers=2, d=256, n_heads=2, n_kv_heads=2, d_ff=512, vocab=1000,
                            B=1, S=64, prompt=32)
    w = workloads.model_weights(dims, device=DEV, std=0.05)
    model = api.Model(w, dims.n_heads, dims.n_kv_heads, dims.mask_id)
    k_max = 8
    x0 = synth.normal(synth.seed_of(82), (k_max, dims.d), 1.0, torch.bfloat16).to(DEV)
    kc0 = synth.normal(synth.seed_of(83), (1, dims.S, 2, 128), 1.0, torch.bfloat16).to(DEV)
    idx = torch.tensor([[1, 4, 9, 20, 33, 40, 63, 70]], dtype=torch.int32, device=DEV)  # 70 >= S
    nact = torch.tensor([8], dtype=torch.int32, device=DEV)
    ws = api.alloc_workspace(model, 1, dims.S, k_max)
    outs = []
    for L in (lib, chk):
        x, kc, vc = x0.clone(), kc0.clone(), kc0.clone()
        mc = model.bind(1, dims.S)
        st = L.dllm_layer_sparse(ctypes.byref(mc), 0, x.data_ptr(), idx.data_ptr(), nact.data_ptr(), k_max,
                                 kc.data_ptr(), vc.data_ptr(), ws.data_ptr(), ws.numel(),
                                 torch.cuda.current_stream().cuda_stream)
        assert st == 0
        torch.cuda.synchronize()
        outs.append((x, kc, vc))
    assert _word(chk) == INDEX_RANGE
    live = [0, 1, 2, 3, 4, 5, 6]
    assert torch.equal(outs[0][0][live], outs[1][0][live])
    assert torch.equal(outs[0][1], outs[1][1]) and torch.equal(outs[0][2], outs[1][2])
    # an out-of-range token id in a full step: clamped alike by both builds, flagged by the check
    tok = workloads.initial_tokens(dims).to(DEV)
    tok[0, 5] = dims.vocab + 7
    finals = []
    for L in (lib, chk):
        st_ = api.State(model, tok.clone(), k_max=k_max)
        ws2 = api.alloc_workspace(model, 1, dims.S, k_max)
        cfg = api.step_cfg(1, True, ws=ws2)
        mc = model.bind(1, dims.S)
        assert L.dllm_skip_step(ctypes.byref(mc), ctypes.byref(st_.c), ctypes.byref(cfg),
                                torch.cuda.current_stream().cuda_stream) == 0
        torch.cuda.synchronize()
        finals.append(st_.h_fin.clone())
    assert _word(chk) == TOKEN_RANGE
    assert torch.equal(finals[0], finals[1])
    assert _word(chk) == 0          # cleared by the previous read
