"""Kernel-level parity: each HIP kernel through the C ABI against the oracle
on the same seeded inputs.  Integer decisions are bit-exact; floats meet the
per-tensor max relative error of their storage format (2e-2 bf16, 1e-4 fp32)."""
import numpy as np
import pytest

from gpu_util import TOL, host64, needs_gpu, rel_err, say
from oracle import model as om
from synth import configs, gen, upload

pytestmark = [pytest.mark.gpu, needs_gpu]


@pytest.fixture(scope="module")
def torch():
    import torch as _t
    return _t


@pytest.fixture(scope="module")
def dg():
    import canvas_denoising_moe_amd as _dg
    _dg.lib()
    return _dg


# ------------------------------------------------------------ argmax / conf --

@pytest.mark.parametrize("rows,V", [(48, 262144), (7, 1024), (1, 16), (0, 64)])
def test_argmax_conf_bit_exact(torch, dg, rows, V):
    say("argmax_conf", rows, V)
    logits = gen.activations(7, 1, (rows, V), std=2.0, dtype="f32") if rows else np.zeros((0, V), np.float32)
    if rows > 5:
        logits[3, 100] = logits[3, V - 5] = logits[3].max() + 0.5  # exact tie -> lower id
        logits[5, :] = 0.25  # flat row: id 0, conf 1/V
    lt = torch.from_numpy(np.ascontiguousarray(logits)).cuda()
    pred = torch.full((rows,), -1, dtype=torch.int32, device="cuda")
    conf = torch.zeros(rows, dtype=torch.float32, device="cuda")
    dg.k_argmax_conf(lt, pred, conf)
    torch.cuda.synchronize()
    if rows == 0:
        return
    p_ref, c_ref = om.argmax_conf(logits.astype(np.float64))
    assert np.array_equal(pred.cpu().numpy(), p_ref)
    c = conf.cpu().numpy().astype(np.float64)
    assert np.max(np.abs(c - c_ref) / c_ref) <= 1e-6
    if rows > 5:
        assert int(pred[3]) == 100 and int(pred[5]) == 0
        assert abs(float(conf[5]) * V - 1.0) < 1e-5


# ------------------------------------------------------------- lock select --

# the last case: canvas 0 already fully locked (nothing to lock, nothing may
# change), canvas 1 with nothing locked and every confidence equal (the
# lowest positions win), canvas 2 with one free slot on its last pass
@pytest.mark.parametrize("B,N,steps,edge", [(4, 256, [1, 2, 5, 12], False), (1, 4096, [3], False),
                                            (2, 16, [7, 1], False), (64, 32, [4] * 64, False),
                                            (3, 256, [2, 2, 1], True)])
def test_lock_select_bit_exact(torch, dg, B, N, steps, edge):
    say("lock_select", B, N, "edge" if edge else "")
    rng = np.random.default_rng([41, B, N])
    conf = (rng.integers(0, 40, size=(B, N)) / 40.0).astype(np.float32)  # many exact ties
    locked = (rng.random((B, N)) < 0.3).astype(np.uint8)
    if edge:
        locked[0] = 1
        locked[1] = 0
        conf[1] = 0.5
        locked[2] = 1
        locked[2, 77] = 0
    tokens = rng.integers(0, 1000, size=(B, N)).astype(np.int32)
    pred = rng.integers(1000, 2000, size=(B, N)).astype(np.int32)
    t_ref, l_ref, _ = om.lock_select(conf.astype(np.float64), pred, tokens, locked, steps)
    tt, lt = torch.from_numpy(tokens).cuda(), torch.from_numpy(locked).cuda()
    dg.k_lock_select(torch.from_numpy(conf).cuda(), torch.from_numpy(pred).cuda(), tt, lt, steps)
    torch.cuda.synchronize()
    assert np.array_equal(tt.cpu().numpy(), t_ref)
    assert np.array_equal(lt.cpu().numpy(), l_ref)
    if edge:
        assert np.array_equal(t_ref[0], tokens[0])  # a full canvas is left alone
        assert np.array_equal(np.nonzero(l_ref[1])[0], np.arange(128))  # ceil(256 / 2), lowest first
        assert l_ref[2].all() and t_ref[2, 77] == pred[2, 77]


# ----------------------------------------------------------------- routing --

def _expected_scatter(idx, E):
    rows, k = idx.shape
    counts = np.bincount(idx.reshape(-1), minlength=E)
    offsets = np.concatenate([[0], np.cumsum(counts)])
    perm = [t * k + s for e in range(E) for t in range(rows) for s in range(k) if idx[t, s] == e]
    return counts, offsets, np.array(perm)


# the last three: the largest expert count at the scatter's bitmap bound
# (256 experts x 2048 rows = 16384 words), an expert count that leaves part
# of every lane's last logit group empty with a ragged row count, and k = 1
@pytest.mark.parametrize("rows,E,k,std,integer", [(256, 128, 8, 1.0, False), (1024, 128, 8, 2.0, False),
                                                  (256, 128, 8, 1.0, True), (4096, 128, 8, 1.0, False),
                                                  (32, 16, 2, 1.0, True), (1, 16, 2, 1.0, False),
                                                  (2048, 256, 8, 1.0, True), (77, 100, 3, 1.0, False),
                                                  (64, 200, 1, 2.0, True)])
def test_moe_route_bit_exact(torch, dg, rows, E, k, std, integer):
    say("moe_route", rows, E, k, integer)
    r = gen.router_logits(5 + rows, rows, E, std)
    if integer:  # forced ties
        r = np.round(r * 2).astype(np.float32)
    idx = torch.empty((rows, k), dtype=torch.int32, device="cuda")
    gates = torch.empty((rows, k), dtype=torch.float32, device="cuda")
    counts = torch.empty(E, dtype=torch.int32, device="cuda")
    offsets = torch.empty(E + 2, dtype=torch.int32, device="cuda")
    perm = torch.empty(rows * k, dtype=torch.int32, device="cuda")
    dg.k_moe_route(torch.from_numpy(r).cuda(), k, idx, gates, counts, offsets, perm)
    torch.cuda.synchronize()
    i_ref, g_ref = om.route(r.astype(np.float64), k)
    assert np.array_equal(idx.cpu().numpy(), i_ref)
    assert rel_err(gates.cpu().numpy(), g_ref) <= 1e-6
    c_ref, o_ref, p_ref = _expected_scatter(i_ref, E)
    assert np.array_equal(counts.cpu().numpy(), c_ref)
    off = offsets.cpu().numpy()
    assert np.array_equal(off[:E + 1], o_ref) and off[E + 1] == rows * k + rows
    assert np.array_equal(perm.cpu().numpy(), p_ref)


# -------------------------------------------------- q/k/v, attention ------

ATTN_MODEL = configs.ModelConfig(
    n_layers=2, hidden=2048, n_heads=16, n_kv_heads=8, head_dim=128, n_experts=16, top_k=8,
    expert_ffn=64, vocab=0, canvas_len=256, window=1024, global_layer_mask=0b10,
    has_lm_head=False, dtype="bf16")
ATTN_W = configs.Workload(name="attn-test", model=ATTN_MODEL, batch=2, prompt_len=1024, n_steps=1, seed=11)
MAXP = 33000


@pytest.fixture(scope="module")
def actx(torch, dg):
    ctx = dg.Context(ATTN_MODEL, max_batch=2, max_prompt_len=MAXP)
    for l in range(ATTN_MODEL.n_layers):
        ctx.set_layer_weights(l, upload.layer_to_device(ATTN_W, l))
    torch.cuda.synchronize()
    yield ctx
    ctx.close()


def _load_prompts(torch, ctx, w, lens):
    kv = []
    for b, L in enumerate(lens):
        wb = w.replace(prompt_len=L)
        ks, vs, kvb = [], [], []
        for l in range(w.model.n_layers):
            k, v = gen.prompt_kv(wb, l, b)
            ks.append(upload.to_device(k, "bf16"))
            vs.append(upload.to_device(v, "bf16"))
            kvb.append((om.bf16_bits_to_f64(k), om.bf16_bits_to_f64(v)))
        ctx.load_prompt_kv(b, L, ks, vs)
        kv.append(kvb)
    torch.cuda.synchronize()
    return kv


@pytest.mark.parametrize("B", [1, 2])
def test_qkv_rope_matches_oracle(torch, actx, B):
    # one canvas: 32-row entries; two canvases fill the chip with 64-row entries
    m = ATTN_MODEL
    lens = [1024, 4000][:B]
    _load_prompts(torch, actx, ATTN_W, lens)
    N = m.canvas_len
    a_bits = gen.activations(12, 2, (B * N, m.hidden), std=1.0, dtype="bf16")
    a = upload.to_device(a_bits, "bf16")
    for l in range(m.n_layers):
        say("qkv layer", l)
        q = torch.empty((B, N, m.n_heads, m.head_dim), dtype=torch.bfloat16, device="cuda")
        k = torch.empty((B, N, m.n_kv_heads, m.head_dim), dtype=torch.bfloat16, device="cuda")
        v = torch.empty_like(k)
        actx.k_qkv(l, B, a, q, k, v)
        torch.cuda.synchronize()
        lw = {n: om.bf16_bits_to_f64(x) for n, x in gen.layer_weights(ATTN_W, l).items()}
        qr, kr, vr = om.qkv_rope(om.bf16_bits_to_f64(a_bits), lw, m, l, lens, om.bf16_round)
        for name, g, r in (("q", q, qr), ("k", k, kr), ("v", v, vr)):
            e = rel_err(host64(g), r)
            print(f"layer {l} {name} rel err {e:.3e}")
            assert e <= TOL["bf16"], (l, name, e)


ATTN_CASES = [
    # (layer, prompt lens per canvas, canvas keys)
    (1, [1024, 1024], True),      # global layer, the one-layer workload's prompt
    (0, [4096, 1024], True),      # local layer: last 1024 of a 4096 prompt
    (1, [4096, 77], True),        # global, ragged prompt (not a multiple of 8 or 64)
    (1, [32768, 1000], True),     # long prompt: many key splits
    (1, [0, 5], True),            # no prompt: pure canvas self-attention
    (0, [1000, 3], False),        # prompt keys only
]


@pytest.mark.parametrize("layer,lens,ck", ATTN_CASES)
def test_canvas_attention_matches_oracle(torch, actx, layer, lens, ck):
    m = ATTN_MODEL
    say("attention", layer, lens, ck)
    kv = _load_prompts(torch, actx, ATTN_W, lens)
    B, N = len(lens), m.canvas_len
    qb = gen.activations(13, 3, (B, N, m.n_heads, m.head_dim), std=1.0, dtype="bf16")
    kb = gen.activations(13, 4, (B, N, m.n_kv_heads, m.head_dim), std=1.0, dtype="bf16")
    vb = gen.activations(13, 5, (B, N, m.n_kv_heads, m.head_dim), std=1.0, dtype="bf16")
    o = torch.empty((B, N, m.n_heads * m.head_dim), dtype=torch.bfloat16, device="cuda")
    actx.k_canvas_attn(layer, B, upload.to_device(qb, "bf16"), upload.to_device(kb, "bf16"),
                       upload.to_device(vb, "bf16"), o, canvas_keys=ck)
    torch.cuda.synchronize()
    pkv = [kv[b][layer] for b in range(B)]
    ref = om.canvas_attention(om.bf16_bits_to_f64(qb), om.bf16_bits_to_f64(kb), om.bf16_bits_to_f64(vb),
                              pkv, om.bf16_round, canvas_keys=ck)
    got = host64(o).reshape(B * N, -1)
    e = rel_err(got, ref)
    print(f"attention layer {layer} lens {lens} canvas_keys {ck}: rel err {e:.3e}")
    assert e <= TOL["bf16"]


MHA_MODEL = configs.ModelConfig(
    n_layers=1, hidden=2048, n_heads=64, n_kv_heads=32, head_dim=64, n_experts=16, top_k=8,
    expert_ffn=64, vocab=0, canvas_len=256, window=1024, global_layer_mask=0b1,
    has_lm_head=False, dtype="bf16")
MHA_W = configs.Workload(name="attn-mha-test", model=MHA_MODEL, batch=2, prompt_len=100, n_steps=1, seed=17)


@pytest.mark.parametrize("lens,ck", [
    ([100, 37], True),   # prompt lengths not multiples of 8: the general kernel, whose 32 KV
                         # heads x 8 query tiles fill the chip without key splits
    ([64, 40], False),   # the direct-copy kernel with one 64-key tile per canvas
])
def test_canvas_attention_single_split(torch, dg, lens, ck):
    # one key split per canvas: the attention kernel normalises and stores its
    # output itself (grouped heads, head size 64); no merge runs
    m = MHA_MODEL
    say("attention single split", lens, ck)
    B, N = len(lens), m.canvas_len
    with dg.Context(m, max_batch=B, max_prompt_len=128) as ctx:
        ctx.set_layer_weights(0, upload.layer_to_device(MHA_W, 0))
        kv = _load_prompts(torch, ctx, MHA_W, lens)
        qb = gen.activations(18, 3, (B, N, m.n_heads, m.head_dim), std=1.0, dtype="bf16")
        kb = gen.activations(18, 4, (B, N, m.n_kv_heads, m.head_dim), std=1.0, dtype="bf16")
        vb = gen.activations(18, 5, (B, N, m.n_kv_heads, m.head_dim), std=1.0, dtype="bf16")
        o = torch.empty((B, N, m.n_heads * m.head_dim), dtype=torch.bfloat16, device="cuda")
        ctx.k_canvas_attn(0, B, upload.to_device(qb, "bf16"), upload.to_device(kb, "bf16"),
                          upload.to_device(vb, "bf16"), o, canvas_keys=ck)
        torch.cuda.synchronize()
    ref = om.canvas_attention(om.bf16_bits_to_f64(qb), om.bf16_bits_to_f64(kb), om.bf16_bits_to_f64(vb),
                              [kv[b][0] for b in range(B)], om.bf16_round, canvas_keys=ck)
    e = rel_err(host64(o).reshape(B * N, -1), ref)
    print(f"attention single split {lens} canvas keys {ck}: rel err {e:.3e}")
    assert e <= TOL["bf16"]


def test_single_cached_kv_returns_that_value_bit_exact(torch, actx):
    m = ATTN_MODEL
    say("attention single cached kv")
    kv = _load_prompts(torch, actx, ATTN_W, [1, 1])
    B, N = 2, m.canvas_len
    qb = gen.activations(14, 3, (B, N, m.n_heads, m.head_dim), std=3.0, dtype="bf16")
    zeros = torch.zeros((B, N, m.n_kv_heads, m.head_dim), dtype=torch.bfloat16, device="cuda")
    o = torch.empty((B, N, m.n_heads * m.head_dim), dtype=torch.bfloat16, device="cuda")
    for layer in (0, 1):
        actx.k_canvas_attn(layer, B, upload.to_device(qb, "bf16"), zeros, zeros, o, canvas_keys=False)
        torch.cuda.synchronize()
        got = host64(o).reshape(B, N, m.n_heads, m.head_dim)
        for b in range(B):
            v = kv[b][layer][1][0]  # [Hkv, D]
            want = np.repeat(v, m.n_heads // m.n_kv_heads, axis=0)  # head h reads kv head h // 2
            assert np.array_equal(got[b], np.broadcast_to(want, got[b].shape))


# -------------------------------------------------------------- experts ----

@pytest.fixture(scope="module")
def c2ctx(torch, dg):
    from synth import C2
    ctx = dg.Context(C2.model, max_batch=1, max_prompt_len=C2.prompt_len)
    upload.load_context(ctx, C2)
    yield ctx
    ctx.close()


def _concentrated_routing(M, E, k, pattern):
    """Routing that piles rows onto few experts.  "same8": every token picks
    experts 0..7 in its own order (each gets all M rows, split over several
    work entries; the other experts stay empty).  "hot127": slot 0 of every
    token is expert 127, the other slots distinct random experts.  Gates are
    a softmax over random logits of the k picks."""
    rng = np.random.default_rng([31, M, E, k, len(pattern)])
    idx = np.empty((M, k), dtype=np.int64)
    for t in range(M):
        if pattern == "same8":
            idx[t] = rng.permutation(k)
        else:
            idx[t, 0] = E - 1
            idx[t, 1:] = rng.choice(E - 1, size=k - 1, replace=False)
    z = rng.standard_normal((M, k))
    g = np.exp(z - z.max(axis=1, keepdims=True))
    return idx, g / g.sum(axis=1, keepdims=True)


@pytest.mark.parametrize("pattern", ["router", "same8", "hot127"])
def test_moe_ffn_matches_oracle(torch, c2ctx, pattern):
    from synth import C2
    m = C2.model
    say("moe_ffn C2 layer 0, routing", pattern)
    M = C2.batch * m.canvas_len
    f_bits = gen.activations(15, 6, (M, m.hidden), std=1.0, dtype="bf16")
    if pattern == "router":
        r = gen.router_logits(16, M, m.n_experts, 1.0).astype(np.float64)
        idx, gates = om.route(r, m.top_k)
    else:
        idx, gates = _concentrated_routing(M, m.n_experts, m.top_k, pattern)
    out = torch.empty((M, m.hidden), dtype=torch.float32, device="cuda")
    c2ctx.k_moe_ffn(0, C2.batch, upload.to_device(f_bits, "bf16"),
                    torch.from_numpy(idx.astype(np.int32)).cuda(),
                    torch.from_numpy(gates.astype(np.float32)).cuda(), out)
    torch.cuda.synchronize()
    lw = {n: om.bf16_bits_to_f64(x) for n, x in gen.layer_weights(C2, 0).items()}
    g32 = gates.astype(np.float32).astype(np.float64)
    m_ref, *_ = om.moe_block(om.bf16_bits_to_f64(f_bits), lw, m.top_k, om.bf16_round,
                             route_override=lambda rr, i, g: (idx, g32))
    e = rel_err(host64(out), m_ref)
    print(f"moe_ffn ({pattern} routing) rel err {e:.3e}")
    assert e <= TOL["bf16"]


# ------------------------------------------------------------ LM head ------

LM_MODEL = configs.ModelConfig(
    n_layers=1, hidden=256, n_heads=2, n_kv_heads=1, head_dim=128, n_experts=16, top_k=2,
    expert_ffn=64, vocab=1040, canvas_len=48, window=1024, global_layer_mask=0b1,
    has_lm_head=True, dtype="bf16")
LM_W = configs.Workload(name="lm-test", model=LM_MODEL, batch=2, prompt_len=16, n_steps=1, seed=19)


def test_lm_head_and_fused_argmax(torch, dg):
    # 96 rows (a partial 128-row group) and 65 column blocks (a partial
    # 256-column vocabulary tile); two rows with planted exact ties
    m = LM_MODEL
    B, N, V, H = LM_W.batch, m.canvas_len, m.vocab, m.hidden
    M = B * N
    say("lm head", M, V)
    E_bits = gen.embed(LM_W)
    h_bits = gen.activations(25, 1, (M, H), std=1.0, dtype="bf16")
    h_bits[5] = 0          # every logit 0: argmax id 0, conf 1/V
    E_bits[700] = E_bits[300]  # ids 300 and 700 tie in every row: 300 can win, 700 never
    with dg.Context(m, max_batch=B, max_prompt_len=LM_W.prompt_len) as ctx:
        ctx.set_embedding(upload.to_device(E_bits, "bf16"), upload.to_device(gen.norm_final(LM_W), "bf16"))
        h = upload.to_device(h_bits, "bf16")
        logits = torch.empty((M, V), dtype=torch.float32, device="cuda")
        ctx.k_lm_head(B, h, logits)
        pred = torch.full((M,), -1, dtype=torch.int32, device="cuda")
        conf = torch.zeros(M, dtype=torch.float32, device="cuda")
        ctx.k_lm_argmax(B, h, pred, conf)
        pred2 = torch.full((M,), -1, dtype=torch.int32, device="cuda")
        conf2 = torch.zeros(M, dtype=torch.float32, device="cuda")
        dg.k_argmax_conf(logits, pred2, conf2)
        torch.cuda.synchronize()
    E = om.bf16_bits_to_f64(E_bits)
    ref = om.lm_logits(om.bf16_bits_to_f64(h_bits), E)
    e = rel_err(host64(logits), ref)
    print(f"LM head logits rel err {e:.3e}")
    assert e <= TOL["bf16"]
    # the fused reduction equals the row reduction of the same logits
    p, c = pred.cpu().numpy(), conf.cpu().numpy().astype(np.float64)
    assert np.array_equal(p, pred2.cpu().numpy())
    assert np.max(np.abs(c - conf2.cpu().numpy()) / c) <= 1e-6
    assert p[5] == 0 and abs(c[5] * V - 1.0) < 1e-5
    assert not np.any(p == 700)
    # and the oracle's decision wherever its top-2 gap clears the rounding noise
    p_ref, c_ref = om.argmax_conf(ref)
    srt = np.sort(ref, axis=1)
    clear = (srt[:, -1] - srt[:, -2]) > 1e-4
    assert np.array_equal(p[clear], p_ref[clear])
    assert np.max(np.abs(c - c_ref) / c_ref) <= 1e-3
