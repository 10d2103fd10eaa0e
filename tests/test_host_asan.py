"""The runtime's host-side validation under AddressSanitizer.

A debug build of the library with the host side instrumented
(``build(asan=True)``: ``-fsanitize=address`` on the host compile only, the
device code unchanged) is loaded into a fresh Python process with the
sanitizer's runtime preloaded.  That process drives every host path that
needs no GPU: configurations rejected field by field (each error message
formatted into the context-free error slot), the batch-capacity limit, a
valid configuration that reaches device discovery and fails there, NULL and
out-of-range arguments of the single-kernel and context entry points, and
the entropy-bounded sampler's argument checks.  Any invalid read or write,
use after free or double free in that code aborts the process with a
sanitizer report; the test asserts a clean exit."""
import glob
import os
import subprocess
import sys
import textwrap

import pytest

from canvas_denoising_moe_amd import build as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

SCRIPT = textwrap.dedent("""
    import ctypes, sys
    sys.path.insert(0, {root!r})
    from canvas_denoising_moe_amd import binding as b
    b.LIB_PATH = {lib!r}
    from synth import C3
    L = b.lib()
    maps = open("/proc/self/maps").read()
    assert "libclang_rt.asan" in maps and {lib!r} in maps  # the instrumented build, under the sanitizer
    assert L.dg_destroy(None) == b.DG_OK

    def create(cfg):
        h = ctypes.c_void_p()
        return L.dg_create(ctypes.byref(cfg), 0, None, ctypes.byref(h)), h

    for field, value, status in [("n_layers", 0, b.DG_EINVAL), ("hidden", 100, b.DG_EUNSUPPORTED),
                                 ("n_kv_heads", 3, b.DG_EINVAL), ("top_k", 9, b.DG_EINVAL),
                                 ("n_shared", 2, b.DG_EUNSUPPORTED), ("max_batch", 65, b.DG_EINVAL),
                                 ("canvas_len", 20, b.DG_EUNSUPPORTED), ("dtype", 7, b.DG_EINVAL),
                                 ("expert_format", 2, b.DG_EINVAL), ("vocab", -16, b.DG_EUNSUPPORTED),
                                 ("window", -1, b.DG_EINVAL)]:
        cfg = b.make_config(C3.model, 1, 4096)
        setattr(cfg, field, value)
        st, h = create(cfg)
        assert st == status and not h.value, (field, st)
        assert L.dg_last_error(None), field
    st, h = create(b.make_config(C3.model, 17, 4096))
    assert st == b.DG_EUNSUPPORTED and not h.value
    # a valid configuration passes the checks and fails at device discovery
    st, h = create(b.make_config(C3.model, 1, 4096))
    assert st == b.DG_EHIP and not h.value, st
    assert b"device" in L.dg_last_error(None)
    assert L.dg_create(None, 0, None, None) == b.DG_EINVAL

    fake = ctypes.c_void_p(16)
    one = (ctypes.c_int32 * 1)(1)
    zero = (ctypes.c_int32 * 1)(0)
    seeds = (ctypes.c_uint32 * 2)(1, 2)
    assert L.dg_k_argmax_conf(None, 4, 16, None, None, None) == b.DG_EINVAL
    assert L.dg_k_moe_route(None, 4, 16, 2, None, None, None, None, None, None) == b.DG_EINVAL
    assert L.dg_k_moe_route(fake, 5000, 128, 8, fake, fake, None, None, None, None) == b.DG_EINVAL
    assert L.dg_k_lock_select(1, 8, None, None, None, None, one, None) == b.DG_EINVAL
    assert L.dg_k_lock_select(1, 8, fake, fake, fake, fake, zero, None) == b.DG_EINVAL
    assert L.dg_denoise_step(None, 1, None, None, None, None, None) == b.DG_EINVAL
    assert L.dg_generate_block(None, 1, 8, None, None) == b.DG_EINVAL
    assert L.dg_k_eb_rows(fake, 64, 128, 32, 0, 48, seeds, 0, None, fake, fake, None) == b.DG_EINVAL
    assert L.dg_k_eb_rows(fake, 64, 128, 32, 48, 48, seeds, 0, fake, fake, fake, None) == b.DG_EINVAL
    assert L.dg_k_eb_rows(fake, 65 * 32, 128, 32, 0, 48, seeds, 0, fake, fake, fake, None) == b.DG_EINVAL
    assert L.dg_k_eb_noise(64, 128, 32, -1, seeds, 0, fake, None) == b.DG_EINVAL
    assert L.dg_k_eb_select(65, 8, fake, fake, fake, fake, fake, fake, fake, 0, 48, None) == b.DG_EINVAL
    assert L.dg_k_eb_rows(None, 0, 128, 32, 0, 48, None, 0, None, None, None, None) == b.DG_OK
    print("host checks done")
""")


def _sanitizer_runtime():
    hits = sorted(glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return hits[-1] if hits else None


def test_host_validation_under_address_sanitizer():
    try:
        B.hipcc()
    except RuntimeError:
        pytest.skip("hipcc is not available to build the sanitizer build")
    rt = _sanitizer_runtime()
    if rt is None:
        pytest.skip("the sanitizer runtime of the ROCm compiler is not installed")
    lib = B.build(asan=True)
    env = dict(os.environ, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:exitcode=86",
               HIP_VISIBLE_DEVICES="")
    r = subprocess.run([sys.executable, "-c", SCRIPT.format(root=ROOT, lib=lib)], env=env,
                       capture_output=True, text=True, timeout=300)
    assert "AddressSanitizer" not in r.stderr, r.stderr[-4000:]
    assert r.returncode == 0, r.stderr[-4000:]
    assert "host checks done" in r.stdout
