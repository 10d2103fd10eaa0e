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
