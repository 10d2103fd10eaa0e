"""Host-side checks of the C ABI: the library loads, exports every function
``include/dg.h`` declares, and rejects bad arguments before touching a GPU."""
import ctypes
import os
import re
import subprocess

import pytest

import canvas_denoising_moe_amd as dg
from canvas_denoising_moe_amd import binding
from synth import C1, C3

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _header_functions():
    txt = open(os.path.join(ROOT, "include", "dg.h")).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(dg_[a-z0-9_]+)\s*\(", txt)))


def test_header_declares_the_boundary():
    names = _header_functions()
    for required in ("dg_init_weights", "dg_load_prompt_kv", "dg_denoise_step", "dg_generate_block"):
        assert required in names


def test_library_exports_every_declared_symbol():
    L = dg.lib()
    missing = [n for n in _header_functions() if not hasattr(L, n)]
    assert not missing, missing
    # the binding declares a signature for every exported function
    assert sorted(binding.exported_symbols()) == _header_functions()


def test_struct_layouts_match_the_c_compiler(tmp_path):
    # compile the header with the host C compiler and compare sizes/offsets
    src = tmp_path / "layout.c"
    fields = [f for f, _ in binding.DGConfig._fields_]
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "dg.h"', "int main(void) {",
             '  printf("%zu %zu\\n", sizeof(dg_config), sizeof(dg_layer_weights));']
    lines += [f'  printf("%zu\\n", offsetof(dg_config, {f}));' for f in fields]
    lines += ["  return 0;", "}"]
    src.write_text("\n".join(lines))
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split()
    assert int(out[0]) == ctypes.sizeof(binding.DGConfig)
    assert int(out[1]) == ctypes.sizeof(binding.DGLayerWeights)
    for f, off in zip(fields, out[2:]):
        assert getattr(binding.DGConfig, f).offset == int(off), f


def _create(cfg):
    h = ctypes.c_void_p()
    st = dg.lib().dg_create(ctypes.byref(cfg), 0, None, ctypes.byref(h))
    return st, h


@pytest.mark.parametrize("field,value,status", [
    ("n_layers", 0, dg.DG_EINVAL),
    ("hidden", 100, dg.DG_EUNSUPPORTED),
    ("n_kv_heads", 3, dg.DG_EINVAL),
    ("top_k", 9, dg.DG_EINVAL),
    ("n_shared", 2, dg.DG_EUNSUPPORTED),
    ("max_batch", 65, dg.DG_EINVAL),
    ("canvas_len", 20, dg.DG_EUNSUPPORTED),
    ("dtype", 7, dg.DG_EINVAL),
    ("expert_format", 2, dg.DG_EINVAL),
])
def test_create_rejects_bad_configs_before_any_device_call(field, value, status):
    cfg = dg.make_config(C3.model, 1, 4096)
    setattr(cfg, field, value)
    st, h = _create(cfg)
    assert st == status
    assert not h.value
    assert dg.lib().dg_last_error(None)  # message for the failed create


def test_batch_capacity_limit():
    cfg = dg.make_config(C3.model, 17, 4096)  # 17 * 256 > 4096 rows
    st, h = _create(cfg)
    assert st == dg.DG_EUNSUPPORTED and not h.value


def test_kernel_entry_points_reject_null_arguments():
    L = dg.lib()
    assert L.dg_k_argmax_conf(None, 4, 16, None, None, None) == dg.DG_EINVAL
    assert L.dg_k_moe_route(None, 4, 16, 2, None, None, None, None, None, None) == dg.DG_EINVAL
    one = (ctypes.c_int32 * 1)(1)
    assert L.dg_k_lock_select(1, 8, None, None, None, None, one, None) == dg.DG_EINVAL
    # oversized routing problem
    fake = ctypes.c_void_p(16)
    assert L.dg_k_moe_route(fake, 5000, 128, 8, fake, fake, None, None, None, None) == dg.DG_EINVAL
    zero = (ctypes.c_int32 * 1)(0)
    assert L.dg_k_lock_select(1, 8, fake, fake, fake, fake, zero, None) == dg.DG_EINVAL


def test_context_calls_reject_null_context():
    L = dg.lib()
    assert L.dg_denoise_step(None, 1, None, None, None, None, None) == dg.DG_EINVAL
    assert L.dg_generate_block(None, 1, 8, None, None) == dg.DG_EINVAL
    assert L.dg_destroy(None) == dg.DG_OK


def test_eb_entry_points_validate_on_the_host():
    L = dg.lib()
    fake = ctypes.c_void_p(16)
    seeds = (ctypes.c_uint32 * 2)(1, 2)
    # missing outputs / seeds, pass outside [0, t_max), rows not a multiple of the canvas
    assert L.dg_k_eb_rows(fake, 64, 128, 32, 0, 48, seeds, 0, None, fake, fake, None) == dg.DG_EINVAL
    assert L.dg_k_eb_rows(fake, 64, 128, 32, 0, 48, None, 0, fake, fake, fake, None) == dg.DG_EINVAL
    assert L.dg_k_eb_rows(fake, 64, 128, 32, 48, 48, seeds, 0, fake, fake, fake, None) == dg.DG_EINVAL
    assert L.dg_k_eb_rows(fake, 65, 128, 32, 0, 48, seeds, 0, fake, fake, fake, None) == dg.DG_EINVAL
    assert L.dg_k_eb_rows(fake, 65 * 32, 128, 32, 0, 48, seeds, 0, fake, fake, fake, None) == dg.DG_EINVAL
    assert L.dg_k_eb_noise(64, 128, 32, 0, seeds, 0, None, None) == dg.DG_EINVAL
    assert L.dg_k_eb_noise(64, 128, 32, -1, seeds, 0, fake, None) == dg.DG_EINVAL
    assert L.dg_k_eb_select(1, 8, fake, fake, fake, fake, fake, None, fake, 0, 48, None) == dg.DG_EINVAL
    assert L.dg_k_eb_select(1, 8, fake, fake, fake, fake, fake, fake, fake, -1, 48, None) == dg.DG_EINVAL
    assert L.dg_k_eb_select(1, 8, fake, fake, fake, fake, fake, fake, fake, 0, 0, None) == dg.DG_EINVAL
    assert L.dg_k_eb_select(65, 8, fake, fake, fake, fake, fake, fake, fake, 0, 48, None) == dg.DG_EINVAL
    # empty work is a no-op with NULL pointers
    assert L.dg_k_eb_rows(None, 0, 128, 32, 0, 48, None, 0, None, None, None, None) == dg.DG_OK
    assert L.dg_k_eb_select(0, 8, None, None, None, None, None, None, None, 0, 48, None) == dg.DG_OK


def test_eb_context_calls_reject_null_context():
    L = dg.lib()
    seeds = (ctypes.c_uint32 * 1)(1)
    passes = (ctypes.c_int32 * 1)()
    assert L.dg_eb_step(None, 1, None, None, 0, 48, seeds, 0, None, None, None, None, None) == dg.DG_EINVAL
    assert L.dg_generate_block_eb(None, 1, None, None, seeds, 0, 48, passes) == dg.DG_EINVAL
    assert L.dg_k_lm_sample(None, 1, None, 0, 48, seeds, 0, None, None, None) == dg.DG_EINVAL


def test_mxfp4_experts_need_a_bf16_context():
    import dataclasses

    from synth import C1
    cfg = dg.make_config(dataclasses.replace(C1.model, expert_format="mxfp4"), 1, 64)  # C1 is fp32
    st, h = _create(cfg)
    assert st == dg.DG_EUNSUPPORTED and not h.value
    with pytest.raises(ValueError):
        dg.make_config(dataclasses.replace(C1.model, expert_format="int3"), 1, 64)
