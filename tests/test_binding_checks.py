"""Host-side argument checks of the Python binding.

The C ABI takes plain pointers and cannot see a buffer's size, so the
binding checks every tensor's element count before it calls into the
library: a short buffer would send a kernel or a copy out of bounds.  These
tests drive the checks on a context object that never reached the library
(no GPU here): a size mismatch is reported as such, and tensors of the right
sizes get as far as the device check, proving no size check fired."""
import numpy as np
import pytest
import torch

from canvas_denoising_moe_amd import binding
from synth import C1, C3


def _fake_ctx(model, max_batch=1):
    ctx = object.__new__(binding.Context)
    ctx.model = model
    ctx.max_batch = max_batch
    ctx.wdtype = torch.bfloat16 if model.dtype == "bf16" else torch.float32
    ctx._keep = []
    ctx._h = None
    return ctx


def _canvas(B, N, dtype=torch.int32):
    return torch.zeros((B, N), dtype=dtype)


def test_denoise_step_checks_sizes_first():
    m = C1.model
    ctx = _fake_ctx(m, max_batch=2)
    N = m.canvas_len
    with pytest.raises(ValueError, match="positions per canvas"):
        ctx.denoise_step(_canvas(1, N + 1), _canvas(1, N + 1, torch.uint8), [4])
    with pytest.raises(ValueError, match="locked: 31 elements, expected 32"):
        ctx.denoise_step(_canvas(1, N), torch.zeros(N - 1, dtype=torch.uint8), [4])
    with pytest.raises(ValueError, match="conf: 16 elements"):
        ctx.denoise_step(_canvas(1, N), _canvas(1, N, torch.uint8), [4], conf=torch.zeros(16))
    with pytest.raises(ValueError, match="steps_left"):
        ctx.denoise_step(_canvas(2, N), _canvas(2, N, torch.uint8), [4])
    with pytest.raises(ValueError, match=r"batch 3 outside \[1, 2\]"):
        ctx.denoise_step(_canvas(3, N), _canvas(3, N, torch.uint8), [4, 4, 4])
    # right sizes: the next check is the device check (no library call yet)
    with pytest.raises(ValueError, match="must be a device tensor"):
        ctx.denoise_step(_canvas(2, N), _canvas(2, N, torch.uint8), [4, 4], conf=torch.zeros(2 * N),
                         pred=torch.zeros(2 * N, dtype=torch.int32))


def test_trace_must_hold_the_batch():
    m = C1.model
    ctx = _fake_ctx(m, max_batch=2)
    N = m.canvas_len
    ctx._keep = [torch.zeros((m.n_layers, N, m.top_k), dtype=torch.int32)]  # room for one canvas
    with pytest.raises(ValueError, match="route trace"):
        ctx.denoise_step(_canvas(2, N), _canvas(2, N, torch.uint8), [4, 4])
    with pytest.raises(ValueError, match="must be a device tensor"):
        ctx.denoise_step(_canvas(1, N), _canvas(1, N, torch.uint8), [4])


def test_prompt_kv_sizes_per_layer():
    m = C1.model
    ctx = _fake_ctx(m)
    L = m.n_layers
    n = 64 * m.n_kv_heads * m.head_dim
    good = [torch.zeros(n) for _ in range(L)]
    with pytest.raises(ValueError, match="one tensor per layer"):
        ctx.load_prompt_kv(0, 64, good[:1], good)
    short = list(good)
    short[1] = torch.zeros(n - 1)
    with pytest.raises(ValueError, match=r"v\[1\]"):
        ctx.load_prompt_kv(0, 64, good, short)
    with pytest.raises(ValueError, match="must be a device tensor"):
        ctx.load_prompt_kv(0, 64, good, good)


def test_prompt_kv_window_length():
    # a sliding-window layer holds min(prompt_len, window) positions
    m = C3.model
    ctx = _fake_ctx(m)
    L = m.n_layers
    per = m.n_kv_heads * m.head_dim
    ks = [torch.zeros(m.kv_len(l, 4096) * per, dtype=torch.bfloat16) for l in range(L)]
    wrong = list(ks)
    wrong[0] = torch.zeros(4096 * per, dtype=torch.bfloat16)  # layer 0 is local: 1024 positions
    with pytest.raises(ValueError, match=r"k\[0\]: 4194304 elements, expected 1048576"):
        ctx.load_prompt_kv(0, 4096, wrong, ks)


def test_weights_and_hidden_sizes():
    m = C1.model
    ctx = _fake_ctx(m)
    w = {k: torch.zeros(v) for k, v in ctx._layer_sizes().items()}
    w["w_down"] = torch.zeros(5)
    with pytest.raises(ValueError, match="w_down"):
        ctx.set_layer_weights(0, w)
    with pytest.raises(ValueError, match="embed"):
        ctx.set_embedding(torch.zeros(7), torch.zeros(m.hidden))
    x = torch.zeros((m.canvas_len + 1, m.hidden))
    with pytest.raises(ValueError, match="whole number of canvases"):
        ctx.forward_hidden(x, x)
    x = torch.zeros((m.canvas_len, m.hidden))
    with pytest.raises(ValueError, match="x_out"):
        ctx.forward_layers(0, 1, x, torch.zeros(3))


def test_single_kernel_sizes():
    m = C1.model
    ctx = _fake_ctx(m)
    M = m.canvas_len
    with pytest.raises(ValueError, match="logits"):
        ctx.k_lm_head(1, torch.zeros(M * m.hidden), torch.zeros(M * m.vocab - 1))
    with pytest.raises(ValueError, match="idx"):
        ctx.k_moe_ffn(0, 1, torch.zeros(M * m.hidden), torch.zeros(M, dtype=torch.int32),
                      torch.zeros(M * m.top_k), torch.zeros(M * m.hidden))
    with pytest.raises(ValueError, match="conf"):
        binding.k_argmax_conf(torch.zeros((4, 16)), torch.zeros(4, dtype=torch.int32), torch.zeros(3))
    with pytest.raises(ValueError, match="perm"):
        binding.k_moe_route(torch.zeros((4, 16)), 2, torch.zeros(8, dtype=torch.int32), torch.zeros(8),
                            perm=torch.zeros(4, dtype=torch.int32))
    with pytest.raises(ValueError, match="steps_left"):
        binding.k_lock_select(torch.zeros((2, 8)), torch.zeros((2, 8), dtype=torch.int32),
                              torch.zeros((2, 8), dtype=torch.int32), torch.zeros((2, 8), dtype=torch.uint8), [1])


def test_every_entry_reaches_the_device_check_with_right_sizes():
    # right-sized host tensors pass every size check and stop at the device
    # check, before any argument reaches ctypes (a size check that rebinds an
    # argument name would surface here as a ctypes type error)
    m = C1.model
    ctx = _fake_ctx(m, max_batch=2)
    B, N, V, H = 2, m.canvas_len, m.vocab, m.hidden
    M = B * N
    i32 = lambda *s: torch.zeros(s, dtype=torch.int32)
    f32 = lambda *s: torch.zeros(s)
    dev = "must be a device tensor"
    with pytest.raises(ValueError, match=dev):
        binding.k_eb_rows(f32(M, V), N, 3, 48, [1, 2], 0, i32(M), f32(M), i32(M))
    with pytest.raises(ValueError, match=dev):
        binding.k_eb_noise(M, V, N, 3, [1, 2], 0, f32(M * V))
    with pytest.raises(ValueError, match=dev):
        binding.k_eb_select(f32(B, N), i32(B, N), i32(B, N), i32(B, N), torch.zeros((B, N), dtype=torch.uint8),
                            i32(B, N), i32(B), 3, 48)
    with pytest.raises(ValueError, match=dev):
        binding.k_lock_select(f32(B, N), i32(B, N), i32(B, N), torch.zeros((B, N), dtype=torch.uint8), [2, 2])
    with pytest.raises(ValueError, match=dev):
        binding.k_argmax_conf(f32(4, 16), i32(4), f32(4))
    with pytest.raises(ValueError, match=dev):
        binding.k_moe_route(f32(4, 16), 2, i32(8), f32(8), i32(16), i32(18), i32(8))
    with pytest.raises(ValueError, match=dev):
        ctx.k_lm_sample(B, f32(M * H), 3, 48, [1, 2], 0, i32(M), f32(M), i32(M))
    with pytest.raises(ValueError, match=dev):
        ctx.k_lm_argmax(B, f32(M * H), i32(M), f32(M))
    with pytest.raises(ValueError, match=dev):
        ctx.eb_step(i32(B, N), torch.zeros((B, N), dtype=torch.uint8), 3, 48, [1, 2], 0, i32(B, N), i32(B),
                    f32(B, N), i32(B, N), i32(B, N))
    with pytest.raises(ValueError, match=dev):
        ctx.generate_block_eb(i32(B, N), torch.zeros((B, N), dtype=torch.uint8), [1, 2])
    with pytest.raises(ValueError, match=dev):
        ctx.generate_block(i32(B, N), torch.zeros((B, N), dtype=torch.uint8), 4)
    with pytest.raises(ValueError, match=dev):
        ctx.commit_tokens(i32(B, N), 3)
    kv = [f32(m.kv_len(l, 64) * m.n_kv_heads * m.head_dim) for l in range(m.n_layers)]
    with pytest.raises(ValueError, match=dev):
        ctx.load_prompt_kv(0, 64, kv, kv)
    q = f32(M * m.n_heads * m.head_dim)
    kk = f32(M * m.n_kv_heads * m.head_dim)
    with pytest.raises(ValueError, match=dev):
        ctx.k_qkv(0, B, f32(M * H), q, kk, kk)
    with pytest.raises(ValueError, match=dev):
        ctx.k_canvas_attn(0, B, q, kk, kk, q)
