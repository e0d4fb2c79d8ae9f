"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every function the headers declare, sizes its buffers as documented, and
rejects bad arguments before launching anything."""
import ctypes
import os
import re

import pytest

from block_discrete_diffusion_dg_amd import binding as B
from block_discrete_diffusion_dg_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    names = set()
    for h in ("dg.h", "dg_test.h"):
        text = open(os.path.join(ROOT, "include", h)).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        for m in re.finditer(r"\b(dg_[a-z_0-9]+)\s*\(", text):
            names.add(m.group(1))
    return sorted(names)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        pytest.fail("libdg.so not built: run __graft_entry__.build()")
    return B.load()


def test_every_declared_symbol_is_exported_and_bound(lib):
    names = header_functions()
    assert len(names) >= 15
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(B.SIGNATURES), set(names) ^ set(B.SIGNATURES)


def _cfg(model=synth.FULL, max_ctx=4096, max_requests=2, max_rows=512, **kw):
    c = B.DGConfig()
    for name in ("n_layers", "d_model", "n_q_heads", "n_kv_heads", "head_dim", "n_experts", "top_k",
                 "d_expert", "d_shared", "vocab", "canvas"):
        setattr(c, name, getattr(model, name))
    c.max_ctx, c.max_requests, c.max_rows = max_ctx, max_requests, max_rows
    c.rms_eps, c.rope_theta, c.tau_first, c.tau_last = 1e-6, 1e4, 0.8, 0.4
    for k, v in kw.items():
        setattr(c, k, v)
    return c


def test_buffer_sizes(lib):
    c = _cfg()
    want_kv = 30 * 2 * 8 * 4096 * 128 * 2
    assert lib.dg_kv_cache_bytes(ctypes.byref(c)) == want_kv
    ws = lib.dg_workspace_bytes(ctypes.byref(c))
    lay = B.DGWsLayout()
    assert lib.dg_workspace_layout(ctypes.byref(c), ctypes.byref(lay)) == B.DG_OK
    assert lay.total == ws > 0
    offs = [getattr(lay, n) for n in B.WS_FIELDS[:-1]]
    assert all(o % 256 == 0 for o in offs) and offs == sorted(offs)
    assert ctypes.sizeof(B.DGRowStats) == 40


def test_binding_structs_match_the_c_header(tmp_path):
    """The ctypes mirrors of the public structs have the header's field
    offsets and sizes (a plain C compiler reads dg.h / dg_test.h)."""
    structs = {"dg_config": B.DGConfig, "dg_row_stats": B.DGRowStats, "dg_step_args": B.DGStepArgs,
               "dg_weights": B.DGWeights, "dg_layer_weights": B.DGLayerWeights,
               "dg_ws_layout": B.DGWsLayout}
    lines = ["#include <stdio.h>", "#include <stddef.h>", '#include "dg_test.h"', "int main(void) {"]
    for cname, py in structs.items():
        lines.append(f'  printf("{cname} size %zu\\n", sizeof({cname}));')
        for fname, _ in py._fields_:
            lines.append(f'  printf("{cname} {fname} %zu\\n", offsetof({cname}, {fname}));')
    lines += ["  return 0;", "}"]
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines) + "\n")
    exe = tmp_path / "layout"
    import subprocess
    subprocess.run(["gcc", "-std=c11", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)],
                   check=True)
    got = {}
    for line in subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.splitlines():
        cname, field, val = line.split()
        got[(cname, field)] = int(val)
    for cname, py in structs.items():
        assert got[(cname, "size")] == ctypes.sizeof(py), cname
        for fname, _ in py._fields_:
            assert got[(cname, fname)] == getattr(py, fname).offset, (cname, fname)


@pytest.mark.parametrize("field,value", [("head_dim", 96), ("d_model", 1000), ("n_experts", 136),
                                         ("top_k", 9), ("vocab", 1000), ("canvas", 24),
                                         ("max_rows", 100), ("n_q_heads", 12), ("max_ctx", 300),
                                         ("max_ctx", 4096 + 16)])
def test_unsupported_shapes_rejected(lib, field, value):
    c = _cfg(**{field: value})
    assert lib.dg_workspace_bytes(ctypes.byref(c)) == 0
    w = B.DGWeights(1, 1, None)
    h = ctypes.c_void_p()
    assert lib.dg_create(ctypes.byref(c), ctypes.byref(w), 1, 1, 1 << 40, ctypes.byref(h)) == B.DG_EINVAL


def _fake_ctx(lib, **kw):
    """A context over fake device addresses: only host-side paths may run on it."""
    c = _cfg(model=synth.TINY, max_ctx=256, max_requests=2, max_rows=64, **kw)
    layers = (B.DGLayerWeights * c.n_layers)()
    for i in range(c.n_layers):
        for n in B.LAYER_FIELDS:
            setattr(layers[i], n, 0x1000)
    w = B.DGWeights(0x1000, 0x1000, layers)
    h = ctypes.c_void_p()
    ws = lib.dg_workspace_bytes(ctypes.byref(c))
    assert lib.dg_create(ctypes.byref(c), ctypes.byref(w), 0x1000, 0x1000, ws - 1,
                         ctypes.byref(h)) == B.DG_ECAPACITY
    assert lib.dg_create(ctypes.byref(c), ctypes.byref(w), 0x1000, 0x1000, ws, ctypes.byref(h)) == B.DG_OK
    return h


def test_argument_and_capacity_errors_launch_nothing(lib):
    h = _fake_ctx(lib)
    try:
        assert lib.dg_cache_len(h, 0) == 0 and lib.dg_cache_len(h, 5) == -1
        # bad slot / negative length / null ids
        assert lib.dg_prefill(h, None, 7, 0x2000, 10) == B.DG_EINVAL
        assert lib.dg_prefill(h, None, 0, 0x2000, -1) == B.DG_EINVAL
        assert lib.dg_prefill(h, None, 0, None, 10) == B.DG_EINVAL
        # prompt beyond max_ctx (256): capacity error, length unchanged
        assert lib.dg_prefill(h, None, 0, 0x2000, 257) == B.DG_ECAPACITY
        assert lib.dg_cache_len(h, 0) == 0
        assert b"max_ctx" in lib.dg_last_error(h)
        # set_cache_len bounds
        assert lib.dg_set_cache_len(h, 0, 257) == B.DG_ECAPACITY
        assert lib.dg_set_cache_len(h, 0, 225) == B.DG_OK and lib.dg_cache_len(h, 0) == 225
        # a block of 32 rows no longer fits: capacity error, nothing launched
        req = (ctypes.c_int32 * 1)(0)
        assert lib.dg_commit_block(h, None, 1, req, 0x2000) == B.DG_ECAPACITY
        assert lib.dg_cache_len(h, 0) == 225
        dup = (ctypes.c_int32 * 2)(1, 1)
        assert lib.dg_commit_block(h, None, 2, dup, 0x2000) == B.DG_EINVAL
        # step arguments
        a = B.DGStepArgs()
        reqs = (ctypes.c_int32 * 1)(1)
        seeds = (ctypes.c_uint64 * 1)(0)
        blocks = (ctypes.c_int32 * 1)(0)
        a.n_req, a.req, a.seed, a.block = 1, reqs, seeds, blocks
        a.d_canvas, a.d_committed = 0x3000, 0x4000
        a.step, a.n_steps = 1, 4
        lib.dg_set_cache_len(h, 1, 225)
        assert lib.dg_denoise_step(h, None, ctypes.byref(a)) == B.DG_ECAPACITY
        lib.dg_set_cache_len(h, 1, 0)
        a.step = 0
        assert lib.dg_denoise_step(h, None, ctypes.byref(a)) == B.DG_EINVAL
        a.step = 5
        assert lib.dg_denoise_step(h, None, ctypes.byref(a)) == B.DG_EINVAL
        a.step = 2
        a.confidence = 2  # neither DG_CONF_PROB nor DG_CONF_ENTROPY
        assert lib.dg_denoise_step(h, None, ctypes.byref(a)) == B.DG_EINVAL
        assert b"confidence" in lib.dg_last_error(h)
        a.confidence = B.CONFIDENCE["entropy"]
        a.stop_entropy = float("nan")
        assert lib.dg_denoise_step(h, None, ctypes.byref(a)) == B.DG_EINVAL
        assert b"NaN" in lib.dg_last_error(h)
        a.stop_entropy = 0.0
        a.candidate = 2  # neither DG_CAND_ARGMAX nor DG_CAND_SAMPLE
        assert lib.dg_denoise_step(h, None, ctypes.byref(a)) == B.DG_EINVAL
        assert b"candidate" in lib.dg_last_error(h)
        a.candidate = B.CANDIDATE["sample"]
        blocks[0] = 1 << 15  # beyond the counter's block field
        assert lib.dg_denoise_step(h, None, ctypes.byref(a)) == B.DG_EINVAL
        assert b"block" in lib.dg_last_error(h)
        blocks[0] = 0
        a.candidate = B.CANDIDATE["argmax"]
        a.n_req = 3  # 3 * 32 rows > max_rows 64
        assert lib.dg_denoise_step(h, None, ctypes.byref(a)) == B.DG_ECAPACITY
        # AR step: bad sizes and slots, and a full cache, launch nothing
        one = (ctypes.c_int32 * 1)(0)
        assert lib.dg_ar_step(h, None, 0, one, 0x2000, 0x3000) == B.DG_EINVAL
        assert lib.dg_ar_step(h, None, 1, one, None, 0x3000) == B.DG_EINVAL
        assert lib.dg_ar_step(h, None, 2, dup, 0x2000, 0x3000) == B.DG_EINVAL
        lib.dg_set_cache_len(h, 0, 256)
        assert lib.dg_ar_step(h, None, 1, one, 0x2000, 0x3000) == B.DG_ECAPACITY
        assert lib.dg_cache_len(h, 0) == 256
        assert lib.dg_reset(h, 0) == B.DG_OK and lib.dg_cache_len(h, 0) == 0
        assert lib.dg_reset(h, 9) == B.DG_EINVAL
    finally:
        lib.dg_destroy(h)


def test_pack_weight_rejects_bad_arguments(lib):
    # every check runs on the host before a launch: fake addresses are safe
    ok_src, ok_dst = 0x100000, 0x900000
    assert lib.dg_pack_weight(None, None, ok_dst, 16, 64) == B.DG_EINVAL
    assert lib.dg_pack_weight(None, ok_src, None, 16, 64) == B.DG_EINVAL
    assert lib.dg_pack_weight(None, ok_src, ok_dst, 24, 64) == B.DG_EINVAL   # n % 16
    assert lib.dg_pack_weight(None, ok_src, ok_dst, 16, 96) == B.DG_EINVAL   # k % 64
    assert lib.dg_pack_weight(None, ok_src, ok_dst, 0, 64) == B.DG_EINVAL
    # 16 x 64 bf16 = 2048 bytes: destinations overlapping the source are refused
    assert lib.dg_pack_weight(None, ok_src, ok_src + 2046, 16, 64) == B.DG_EINVAL
    assert lib.dg_pack_weight(None, ok_src + 2046, ok_src, 16, 64) == B.DG_EINVAL


def test_quantize_fp8_rejects_bad_arguments(lib):
    ok_src, ok_dst, ok_sc = 0x100000, 0x900000, 0xA00000
    q = lib.dg_quantize_fp8
    assert q(None, None, ok_dst, ok_sc, 16, 64) == B.DG_EINVAL
    assert q(None, ok_src, None, ok_sc, 16, 64) == B.DG_EINVAL
    assert q(None, ok_src, ok_dst, None, 16, 64) == B.DG_EINVAL
    assert q(None, ok_src, ok_dst, ok_sc, 24, 64) == B.DG_EINVAL  # n % 16
    assert q(None, ok_src, ok_dst, ok_sc, 16, 96) == B.DG_EINVAL  # k % 64
    assert q(None, ok_src, ok_dst, ok_sc, -16, 64) == B.DG_EINVAL
    # 16 x 64: 2048 source bytes, 1024 destination bytes; overlaps are refused
    assert q(None, ok_src, ok_src + 2047, ok_sc, 16, 64) == B.DG_EINVAL
    assert q(None, ok_src + 1023, ok_src, ok_sc, 16, 64) == B.DG_EINVAL


def test_fp8_experts_need_their_scales(lib):
    c = _cfg(model=synth.TINY, max_ctx=256, max_requests=1, max_rows=32)
    c.expert_format = 2
    assert lib.dg_workspace_bytes(ctypes.byref(c)) == 0  # unknown format: unsupported config
    c.expert_format = B.WEIGHT_FORMAT["fp8"]
    layers = (B.DGLayerWeights * c.n_layers)()
    for n in B.LAYER_FIELDS:
        setattr(layers[0], n, 0x1000)
    w = B.DGWeights(0x1000, 0x1000, layers)
    ws = lib.dg_workspace_bytes(ctypes.byref(c))
    h = ctypes.c_void_p()
    assert lib.dg_create(ctypes.byref(c), ctypes.byref(w), 0x1000, 0x1000, ws, ctypes.byref(h)) == B.DG_EINVAL
    for n in B.SCALE_FIELDS:
        setattr(layers[0], n, 0x2000)
    assert lib.dg_create(ctypes.byref(c), ctypes.byref(w), 0x1000, 0x1000, ws, ctypes.byref(h)) == B.DG_OK
    lib.dg_destroy(h)

def test_route_noalloc_rejects_sizes_and_arguments_on_the_host(lib):
    # every check runs before any HIP call: fake addresses are safe here
    p = 0x100000
    rows_max = B.ROUTE_NOALLOC_MAX_ROWS
    assert lib.dg_route_noalloc(None, p, rows_max + 1, 128, 8, p, p, p, p, p, p) == B.DG_ECAPACITY
    assert lib.dg_route_noalloc(None, p, 0, 128, 8, p, p, p, p, p, p) == B.DG_EINVAL
    assert lib.dg_route_noalloc(None, p, 16, 129, 8, p, p, p, p, p, p) == B.DG_EINVAL
    assert lib.dg_route_noalloc(None, p, 16, 124, 8, p, p, p, p, p, p) == B.DG_EINVAL  # not a multiple of 8
    assert lib.dg_route_noalloc(None, p, 16, 8, 9, p, p, p, p, p, p) == B.DG_EINVAL
    assert lib.dg_route_noalloc(None, p, 16, 128, 8, p, p, None, p, p, p) == B.DG_EINVAL
