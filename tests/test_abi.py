"""The C-ABI library loads and exports every entry point of include/dllm.h (CPU only).

Only host-side entry points run here: workspace planning and argument
validation, which return before any kernel launch.
"""
import ctypes
import os
import re

import pytest

from token_skipping_denoise_amd import _ffi

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "dllm.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(dllm_[a-z_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_ffi.LIB_PATH):
        pytest.fail("libdllm.so is not built (run __graft_entry__.build())")
    return _ffi.load()


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert set(names) == set(_ffi.EXPORTED)
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_status_strings(lib):
    assert lib.dllm_version() == 300
    assert lib.dllm_status_string(0) == b"ok"
    assert lib.dllm_status_string(4) == b"workspace missing or too small"


def test_workspace_size_planning(lib):
    d = _ffi.Dims(1, 512, 4096, 32, 32, 128, 12288, 126464, 32)
    n128 = lib.dllm_workspace_size(ctypes.byref(d), _ffi.DLLM_BF16, 128)
    n512 = lib.dllm_workspace_size(ctypes.byref(d), _ffi.DLLM_BF16, 512)
    assert 0 < n128 <= n512
    # logits of every row dominate: at least B*S*V*4 bytes
    assert n512 >= 512 * 126464 * 4
    # invalid: head_dim 64 unsupported by the bf16 attention, k_max > S, bad dtype
    bad = _ffi.Dims(1, 512, 4096, 64, 64, 64, 12288, 126464, 32)
    assert lib.dllm_workspace_size(ctypes.byref(bad), _ffi.DLLM_BF16, 128) == 0
    assert lib.dllm_workspace_size(ctypes.byref(d), _ffi.DLLM_BF16, 513) == 0
    assert lib.dllm_workspace_size(ctypes.byref(d), 7, 128) == 0
    tiny = _ffi.Dims(1, 128, 256, 4, 4, 64, 768, 1024, 2)
    assert lib.dllm_workspace_size(ctypes.byref(tiny), _ffi.DLLM_F32, 32) > 0


def test_bf16_shapes_past_32_bit_offsets_are_rejected(lib):
    """bf16 kernels address with 32-bit byte offsets: the shapes whose SwiGLU weight, GEMM
    tile or per-sequence K/V cache would reach 2 GiB are refused before any launch."""
    ok = _ffi.Dims(1, 4096, 8192, 64, 8, 128, 65536 - 128, 32000, 1)  # (d_ff + 128) d 2 B = 2^30
    assert lib.dllm_workspace_size(ctypes.byref(ok), _ffi.DLLM_BF16, 64) > 0
    wide_ffn = _ffi.Dims(1, 4096, 8192, 64, 8, 128, 131072, 32000, 1)  # SwiGLU span 2^31 B
    long_kv = _ffi.Dims(1, 1 << 20, 4096, 64, 8, 128, 12288, 32000, 1)  # K/V of one sequence 2 GiB
    big_k = _ffi.Dims(1, 512, 4096 * 1024, 32, 32, 128, 12288, 32000, 1)  # 256 rows x 4M x 2 B = 2 GiB
    for bad in (wide_ffn, long_kv, big_k):
        assert lib.dllm_workspace_size(ctypes.byref(bad), _ffi.DLLM_BF16, 64) == 0


def test_argument_validation_returns_before_launch(lib):
    cfg = _ffi.ScoreCfg(0.5, 0, 0, 0, 4, 0.0)
    fake = ctypes.c_void_p(16)   # never dereferenced: validation fails first
    # NULL inputs
    assert lib.dllm_score_select(None, None, None, 1, None, None, None, 1, 8, 8, ctypes.byref(cfg),
                                 None, None, None, 4, None) == 1
    # k > k_max
    cfg_big = _ffi.ScoreCfg(0.5, 0, 0, 0, 9, 0.0)
    assert lib.dllm_score_select(fake, fake, None, 1, fake, None, None, 1, 8, 8, ctypes.byref(cfg_big),
                                 fake, fake, fake, 4, None) == 1
    # width not a multiple of 8 for bf16
    assert lib.dllm_score_select(fake, fake, None, 1, fake, None, None, 1, 8, 12, ctypes.byref(cfg),
                                 fake, fake, fake, 4, None) == 2
    # bad dtype
    assert lib.dllm_gather_rows(fake, fake, fake, 1, 8, 4, 8, 5, fake, None) == 3
    # k_max > S
    assert lib.dllm_gather_rows(fake, fake, fake, 1, 8, 9, 8, 1, fake, None) == 2
    # confidence pass with a bad exclude id
    assert lib.dllm_confidence_kl(fake, None, 0, fake, 4, 10, 10, 0, fake, fake, None, None) == 2
    # confidence pass with an unknown previous-logit precision
    assert lib.dllm_confidence_kl(fake, fake, 7, fake, 4, 10, 3, 0, fake, fake, None, None) == 3
    # dilated round planner: missing force map, block past S, base a < 2, round >= R, mark 0
    assert lib.dllm_dus_mark(None, 1, 10, 0, 4, 2, 0, 0, 1, None) == 1
    assert lib.dllm_dus_mark(fake, 1, 10, 8, 4, 2, 0, 0, 1, None) == 2
    assert lib.dllm_dus_mark(fake, 1, 10, 0, 4, 1, 0, 0, 1, None) == 1
    assert lib.dllm_dus_mark(fake, 1, 10, 0, 4, 2, 0, 2, 1, None) == 1
    assert lib.dllm_dus_mark(fake, 1, 10, 0, 4, 2, 0, 0, 0, None) == 1
    # skip step without a model
    assert lib.dllm_skip_step(None, None, None, None) == 1


def _fake_step_args(n_layers=2):
    """A model / state / step config whose pointers are never dereferenced (validation fails
    first), keeping the host arrays alive on the returned tuple."""
    F = 0x1000                                         # 16-byte aligned, never read
    lw = (_ffi.LayerW * n_layers)(*[_ffi.LayerW(*([F] * 6), None, None) for _ in range(n_layers)])
    m = _ffi.ModelC(_ffi.Dims(1, 8, 128, 1, 1, 128, 128, 16, n_layers), 1, 1e4, 1e-5, 15, F,
                    ctypes.cast(lw, ctypes.POINTER(_ffi.LayerW)), F, F)
    kv = (ctypes.c_void_p * n_layers)(*([F] * n_layers))
    st = _ffi.StateC()
    for f in ("tokens", "h_fin", "conf", "kl", "argmax", "idx", "n_active", "force"):
        setattr(st, f, F)
    st.k_cache = ctypes.cast(kv, ctypes.POINTER(ctypes.c_void_p))
    st.v_cache = ctypes.cast(kv, ctypes.POINTER(ctypes.c_void_p))
    st.h_bnd[0] = st.h_bnd[1] = F
    st.k_max = 4
    st.have_prev = 1
    cfg = _ffi.StepCfg()
    cfg.boundary_layer = 0
    cfg.full_step = 0
    cfg.score = _ffi.ScoreCfg(0.0, 0, 1, 0, 2, 0.0)
    cfg.lock_kl_eps = -1.0
    cfg.layer_cache = 1
    return m, st, cfg, (lw, kv)


def test_layer_cache_validation_returns_before_launch(lib):
    m, st, cfg, keep = _fake_step_args()
    # per-layer caches missing
    assert lib.dllm_skip_step(ctypes.byref(m), ctypes.byref(st), ctypes.byref(cfg), None) == 1
    caches = (ctypes.c_void_p * 2)(0x1000, 0x1000)
    st.x_in_cache = ctypes.cast(caches, ctypes.POINTER(ctypes.c_void_p))
    st.x_out_cache = ctypes.cast(caches, ctypes.POINTER(ctypes.c_void_p))
    # the boundary must leave a cached layer; nested boundaries do not combine with the cache
    cfg.boundary_layer = 2
    assert lib.dllm_skip_step(ctypes.byref(m), ctypes.byref(st), ctypes.byref(cfg), None) == 1
    cfg.boundary_layer = 0
    cfg.n_nested = 1
    cfg.nested_layer[0] = 1
    cfg.nested_k[0] = 1
    st.h_nested[0] = 0x1000
    assert lib.dllm_skip_step(ctypes.byref(m), ctypes.byref(st), ctypes.byref(cfg), None) == 1
    cfg.n_nested = 0
    # a misaligned cache row buffer
    bad = (ctypes.c_void_p * 2)(0x1000, 0x1004)
    st.x_out_cache = ctypes.cast(bad, ctypes.POINTER(ctypes.c_void_p))
    assert lib.dllm_skip_step(ctypes.byref(m), ctypes.byref(st), ctypes.byref(cfg), None) == 1
    # everything valid but no workspace: still no launch
    st.x_out_cache = ctypes.cast(caches, ctypes.POINTER(ctypes.c_void_p))
    assert lib.dllm_skip_step(ctypes.byref(m), ctypes.byref(st), ctypes.byref(cfg), None) == 4


def test_timing_hook_is_per_call_and_validated(lib):
    """The measurement hook travels in the step config of one call (no process-wide state): a
    malformed hook is refused before any launch, and a well-formed one passes validation."""
    m, st, cfg, keep = _fake_step_args()
    cfg.layer_cache = 0
    cfg.boundary_layer = 1
    bad = _ffi.Timing(_ffi.TK_QKV, 0, 4, 0, None, None)       # capacity without event arrays
    cfg.timing = ctypes.pointer(bad)
    assert lib.dllm_skip_step(ctypes.byref(m), ctypes.byref(st), ctypes.byref(cfg), None) == 1
    neg = _ffi.Timing(_ffi.TK_QKV, 0, -1, 0, None, None)
    cfg.timing = ctypes.pointer(neg)
    assert lib.dllm_skip_step(ctypes.byref(m), ctypes.byref(st), ctypes.byref(cfg), None) == 1
    ev = (ctypes.c_void_p * 4)()
    good = _ffi.Timing(_ffi.TK_QKV, 0, 4, 0, ctypes.cast(ev, ctypes.POINTER(ctypes.c_void_p)),
                       ctypes.cast(ev, ctypes.POINTER(ctypes.c_void_p)))
    cfg.timing = ctypes.pointer(good)
    # valid hook, no workspace: refused for the workspace, still before any launch
    assert lib.dllm_skip_step(ctypes.byref(m), ctypes.byref(st), ctypes.byref(cfg), None) == 4
    assert good.count == 0
    assert not hasattr(lib, "dllm_set_timing")


def test_noalloc_layer_rejects_oversize_before_any_launch(lib):
    """The allocation-free layer call refuses shapes whose scratch exceeds the library's array
    (here a dense 512-row LLaDA-8B-shaped layer, about 75 MB) before touching the device, and
    validates its arguments like dllm_layer_sparse."""
    m, st, cfg, keep = _fake_step_args()
    big = _ffi.ModelC(_ffi.Dims(1, 512, 4096, 32, 32, 128, 12288, 126464, 2), 1, 1e4, 1e-5, 126463, 0x1000,
                      m.layers, 0x1000, 0x1000)
    F = ctypes.c_void_p(0x1000)
    assert lib.dllm_layer_sparse_noalloc(ctypes.byref(big), 0, F, F, F, 512, F, F, None) == 4
    assert lib.dllm_layer_sparse_noalloc(ctypes.byref(big), 2, F, F, F, 128, F, F, None) == 1   # layer out of range
    assert lib.dllm_layer_sparse_noalloc(ctypes.byref(big), 0, F, F, F, 513, F, F, None) == 2   # k_max > S
    assert lib.dllm_layer_sparse_noalloc(ctypes.byref(big), 0, None, F, F, 128, F, F, None) == 1
    assert lib.dllm_layer_sparse_noalloc(None, 0, F, F, F, 128, F, F, None) == 1


def test_misaligned_packed_weights_rejected(lib):
    """Packed weight copies are read with 16-byte fragment loads: a model whose packed LM head or
    packed layer weight is not 16-byte aligned fails validation (EINVAL) before the allocation-free
    call reaches its scratch-size check (EWORKSPACE for this 512-row shape)."""
    m, st, cfg, keep = _fake_step_args()
    F = ctypes.c_void_p(0x1000)
    big = _ffi.ModelC(_ffi.Dims(1, 512, 4096, 32, 32, 128, 12288, 126464, 2), 1, 1e4, 1e-5, 126463, 0x1000,
                      m.layers, 0x1000, 0x1000)
    call = lambda mod: lib.dllm_layer_sparse_noalloc(ctypes.byref(mod), 0, F, F, F, 512, F, F, None)
    assert call(big) == 4
    big.lm_head_packed = 0x2000
    assert call(big) == 4
    big.lm_head_packed = 0x2008
    assert call(big) == 1
    big.lm_head_packed = None
    lw = (_ffi.LayerW * 2)(*[_ffi.LayerW(*([0x1000] * 6), None, None, 0x3004) for _ in range(2)])
    big.layers = ctypes.cast(lw, ctypes.POINTER(_ffi.LayerW))
    assert call(big) == 1


def test_checking_build_exports_the_same_entry_points(lib):
    """libdllm_check.so (-DDLLM_CHECK) is the same ABI; the normal build records nothing and says so
    without touching the device."""
    chk = _ffi.load_check()
    for n in declared_functions():
        assert hasattr(chk, n), n
    assert chk.dllm_version() == lib.dllm_version()
    w = ctypes.c_uint32(77)
    assert lib.dllm_check_word(ctypes.byref(w), 1) == 1 and w.value == 0
    assert lib.dllm_check_word(None, 0) == 1


def test_struct_layouts_match_header(tmp_path):
    """Every ctypes struct of the binding has the header's size and field offsets (gcc, CPU only)."""
    import shutil
    import subprocess
    gcc = shutil.which("gcc") or shutil.which("cc")
    if gcc is None:
        pytest.skip("no C compiler")
    structs = {"dllm_dims": _ffi.Dims, "dllm_score_cfg": _ffi.ScoreCfg, "dllm_state": _ffi.StateC,
               "dllm_step_cfg": _ffi.StepCfg, "dllm_timing": _ffi.Timing, "dllm_layer_w": _ffi.LayerW,
               "dllm_model": _ffi.ModelC}
    lines = ["#include <stdio.h>", "#include <stddef.h>", '#include "dllm.h"', "int main(void) {"]
    for cname, py in structs.items():
        lines.append(f'  printf("{cname} size %zu\\n", sizeof({cname}));')
        for fname, _ in py._fields_:
            lines.append(f'  printf("{cname} {fname} %zu\\n", offsetof({cname}, {fname}));')
    lines += ["  return 0;", "}"]
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines) + "\n")
    exe = tmp_path / "layout"
    subprocess.run([gcc, "-std=c99", "-I", os.path.dirname(HEADER), str(src), "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split("\n")
    got = {}
    for line in out:
        if line:
            parts = line.split()
            got[(parts[0], parts[1])] = int(parts[2])
    for cname, py in structs.items():
        assert got[(cname, "size")] == ctypes.sizeof(py), cname
        for fname, _ in py._fields_:
            assert got[(cname, fname)] == getattr(py, fname).offset, f"{cname}.{fname}"


def test_product_path_never_touches_the_oracle():
    """The package (binding and HIP sources) neither imports nor names the CPU oracle: only the
    tests, smoke() and the bench's CPU-baseline leg may use it."""
    pkg = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "token_skipping_denoise_amd")
    offenders = []
    for root, _, files in os.walk(pkg):
        if "_build" in root or "__pycache__" in root:
            continue
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(root, f)).read()
                if re.search(r"^\s*(from|import)\s+oracle\b|\boracle[./]", text, flags=re.M):
                    offenders.append(f)
    assert offenders == []


def test_binding_fails_loudly_without_the_library(tmp_path):
    """No fallback path: loading a missing library raises instead of computing anything else."""
    saved = _ffi._LIB
    _ffi._LIB = None
    try:
        with pytest.raises(RuntimeError, match="missing"):
            _ffi.load(str(tmp_path / "libdllm.so"))
    finally:
        _ffi._LIB = saved


def _plan(lib, M, N, K, swiglu=False):
    nw, sp = ctypes.c_int32(), ctypes.c_int32()
    ok = lib.dllm_packed_plan(M, N, K, int(swiglu), ctypes.byref(nw), ctypes.byref(sp))
    return (nw.value, sp.value) if ok else None


def test_packed_plan_choices(lib):
    """The packed-weight planner (host only): one workgroup per CU, 256 CUs.  At the LLaDA-8B
    shapes over 128 rows it keeps one full round of 256 workgroups per product; the Dream-7B
    shapes (d 3584, F 18944, 28 + 2 x 4 heads of 128) are covered too."""
    # LLaDA-8B: QKV 12288 x 4096, O 4096 x 4096, gate/up 24576 x 4096 (fused), down 4096 x 12288
    assert _plan(lib, 128, 12288, 4096) == (3, 2)
    assert _plan(lib, 128, 4096, 4096) == (4, 8)
    assert _plan(lib, 128, 24576, 4096, swiglu=True) == (3, 1)
    assert _plan(lib, 128, 4096, 12288) == (4, 8)
    # Dream-7B: QKV 4608 x 3584 (48 tiles x 4), O 3584 x 3584 and down 3584 x 18944 (28 tiles x 8)
    assert _plan(lib, 128, 4608, 3584) == (3, 4)
    assert _plan(lib, 128, 3584, 3584) == (4, 8)
    assert _plan(lib, 128, 3584, 18944) == (4, 8)
    assert _plan(lib, 128, 37888, 3584, swiglu=True) is not None
    # outside the path: more than 128 rows, no rows, K not a multiple of 64, too few stages
    assert _plan(lib, 129, 4096, 4096) is None
    assert _plan(lib, 0, 4096, 4096) is None
    assert _plan(lib, 64, 4096, 4000) is None
    assert _plan(lib, 64, 4096, 320) is None  # 5 stages of 64: fewer than any wave count keeps in flight


def test_packed_plan_invariants(lib):
    """Every shape with d and F multiples of 64 (and at least 6 stages) gets a plan, and every plan
    is one the kernel can run: N splits into whole workgroups, every K split holds the stages in
    flight (7 for 3-4 waves, 6 for 2), split counts are ones the epilogues sum (1, 2, 4, 8), the
    fused gate/up product is never split."""
    for N in range(64, 8193, 448):
        for K in range(384, 20000, 1216):
            for swiglu in (False, True):
                p = _plan(lib, 96, N, K, swiglu)
                assert p is not None, (N, K, swiglu)
                nw, sp = p
                assert nw in (2, 3, 4) and N % (32 * nw) == 0 and sp in (1, 2, 4, 8)
                assert (K // 64) // sp >= (6 if nw == 2 else 7)
                assert not (swiglu and sp != 1)
