// Host runtime behind the C ABI in include/dg.h: owns the packed weights,
// the prompt KV copies and the workspaces, validates every call before it
// enqueues anything, and sequences the kernels of a denoise pass on the
// caller's stream.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "common.h"
#include "dg.h"

// Scratch of dg_k_lm_argmax_noalloc: the fused LM head's (max, sum, argmax)
// partials, one per (vocabulary tile of 256, row), in an array every device
// holds from the library's load to the end of the process.  Host code must
// not use the array's name as a device address: dg_create looks up each
// device's own copy once (hipGetSymbolAddress with that device current) and
// the entry point passes that address.
constexpr long long kNoAllocParts = 1ll << 20;  // (vocabulary tile, row) pairs: 12 MiB
static __device__ __align__(256) float scratch[3 * kNoAllocParts];

namespace {

std::string g_create_error;

// per device: the address of its copy of `scratch` (null until looked up)
std::mutex g_scratch_mu;
void* g_scratch_dev[64] = {nullptr};

// Looks up the current device's copy of `scratch` once; returns it (null on failure).
void* scratch_addr(int dev) {
  if (dev < 0 || dev >= 64) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) {
      (void)hipGetLastError();
      return nullptr;
    }
    g_scratch_dev[dev] = p;
  }
  return g_scratch_dev[dev];
}

struct LayerW {
  void* qkv = nullptr;   // packed [(Hq+2Hkv)D/16][H/32][64][8]
  void* wo = nullptr;    // packed [H/16][HqD/32][64][8]
  void* router = nullptr;    // packed [E/16][H/32][64][8]
  void* gu = nullptr;   // (E+1) experts, packed gate|up interleave [2F/16][H/32][64][8]
  void* down = nullptr;  // (E+1) experts, packed [H/16][F/32][64][8]
  // MXFP4 experts: gu / down hold the codes, these the scales (launch_quant_mxfp4 layout)
  void* gu_s = nullptr;
  void* down_s = nullptr;
  void* norm[4] = {nullptr, nullptr, nullptr, nullptr};  // in, pa, pf, pf2
  bool set = false;
};

struct SlotKV {
  int prompt_len = -1;
  std::vector<void*> k, v;       // per layer: K [Hkv][len][D], V^T [Hkv][D][len]
  std::vector<long long> cap;    // allocated positions per layer
  std::vector<int> len;
  // per layer: the buffers a block commit writes the grown cache into (then
  // swapped with k / v)
  std::vector<void*> k2, v2;
  std::vector<long long> cap2;
};

}  // namespace

struct dg_ctx {
  dg_config c{};
  int dev = 0;
  hipStream_t st = nullptr;
  int bf16 = 0;
  size_t es = 4;
  std::vector<LayerW> L;
  void* embed = nullptr;
  void* norm_final = nullptr;
  bool embed_set = false;
  std::vector<SlotKV> slots;
  float2* rope = nullptr;  // [max_batch][N][D/2]
  // workspaces
  float *x = nullptr, *ao = nullptr, *rl = nullptr, *gates = nullptr, *y = nullptr, *logits = nullptr,
        *conf = nullptr, *part_o = nullptr, *part_m = nullptr, *part_l = nullptr;
  void *a = nullptr, *f = nullptr, *q = nullptr, *kc = nullptr, *vc = nullptr, *o = nullptr, *u = nullptr;
  int32_t *idx = nullptr, *offsets = nullptr, *perm = nullptr, *arows = nullptr, *pred = nullptr;
  // fused LM head + argmax (bf16): per-(vocabulary tile, row) partials
  float *lm_m = nullptr, *lm_s = nullptr;
  int32_t* lm_i = nullptr;
  // sampler mode partials, per-row entropy / sample, and the state of the
  // entropy-bounded loop (greedy tokens of the previous pass, status flags)
  float *lm_u = nullptr, *lm_g = nullptr;
  int32_t* lm_gi = nullptr;
  float* eb_ent = nullptr;
  int32_t *eb_samp = nullptr, *eb_prev = nullptr, *eb_status = nullptr;
  int32_t* eb_status_host = nullptr;  // pinned
  // pinned: an out-of-range token id seen by the embedding, ((row + 1) << 32) | id;
  // the next call on the context reports it
  uint64_t* bad_id = nullptr;
  bool lm_fused = false;
  long long part_cap = 0;
  int32_t* trace = nullptr;
  // expert work list built by the router: entries, and [count, ent_off[E + 2]]
  int4* work = nullptr;
  int32_t* work_count = nullptr;
  std::string err;
  std::vector<void*> owned;
  // kernel timing: classes timed (bit mask) and event pairs per class (pool
  // reused after a reset)
  int prof = 0;
  std::vector<hipEvent_t> ev_pool;
  size_t ev_used = 0;
  std::vector<std::pair<hipEvent_t, hipEvent_t>> prof_rec[DG_PROF_COUNT];
};

namespace {

dg_status fail(dg_ctx* ctx, dg_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  if (ctx) ctx->err = buf; else g_create_error = buf;
  return s;
}

#define HIPX(expr)                                                                       \
  do {                                                                                   \
    hipError_t _e = (expr);                                                              \
    if (_e != hipSuccess) return fail(ctx, DG_EHIP, "%s: %s", #expr, hipGetErrorString(_e)); \
  } while (0)

dg_status dalloc(dg_ctx* ctx, void** p, size_t bytes) {
  *p = nullptr;
  if (bytes == 0) return DG_OK;
  hipError_t e = hipMalloc(p, bytes);
  if (e != hipSuccess) {
    *p = nullptr;
    (void)hipGetLastError();
    return fail(ctx, DG_ENOMEM, "hipMalloc(%zu bytes) failed: %s", bytes, hipGetErrorString(e));
  }
  ctx->owned.push_back(*p);
  return DG_OK;
}

void dfree(dg_ctx* ctx, void* p) {
  if (!p) return;
  for (auto& q : ctx->owned)
    if (q == p) { q = nullptr; break; }
  (void)hipFree(p);
}

#define TRY(expr)                      \
  do {                                 \
    dg_status _s = (expr);             \
    if (_s != DG_OK) return _s;        \
  } while (0)

template <typename P> dg_status dalloc_t(dg_ctx* ctx, P** p, size_t bytes) {
  void* v = nullptr;
  dg_status s = dalloc(ctx, &v, bytes);
  *p = reinterpret_cast<P*>(v);
  return s;
}

// ---- kernel timing (events on the context's stream) ------------------------
hipEvent_t next_event(dg_ctx* ctx) {
  if (ctx->ev_used == ctx->ev_pool.size()) {
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    ctx->ev_pool.push_back(e);
  }
  return ctx->ev_pool[ctx->ev_used++];
}
hipEvent_t prof_start(dg_ctx* ctx, int kind) {
  if (!((ctx->prof >> kind) & 1)) return nullptr;
  hipEvent_t e = next_event(ctx);
  if (e && hipEventRecord(e, ctx->st) != hipSuccess) return nullptr;
  return e;
}
void prof_stop(dg_ctx* ctx, int kind, hipEvent_t s) {
  if (!s) return;
  hipEvent_t e = next_event(ctx);
  if (!e || hipEventRecord(e, ctx->st) != hipSuccess) return;
  ctx->prof_rec[kind].push_back({s, e});
}
// Event pair bound to the dispatches of one launcher call (no marker packets
// between kernels); empty when timing is off.  Every profiled launcher call
// launches at least one kernel, so both events are always recorded.
KTime prof_kernel(dg_ctx* ctx, int kind) {
  KTime t;
  if (!((ctx->prof >> kind) & 1)) return t;
  hipEvent_t a = next_event(ctx), b = next_event(ctx);
  if (!a || !b) return t;
  t.start = a; t.stop = b;
  ctx->prof_rec[kind].push_back({a, b});
  return t;
}

bool is_global(const dg_config& c, int l) { return (c.global_layer_mask >> l) & 1ull; }

// Row tiles of 16 per streaming-GEMM entry for the expert and dense GEMMs
// (the router GEMM, split over K, keeps 16-row entries).
constexpr int kStreamMT = 2;
constexpr int kEntryRows = 16 * kStreamMT;

// Row tiles per entry of a dense projection with NB n-blocks (8 per
// workgroup tile) over M rows: starting from mt, doubled up to 4 while the
// grid keeps at least one workgroup per CU, so that with many rows each
// weight tile is read from L2 by fewer entries (measured on four canvases:
// output projection 26.0 -> 22.6 us and q/k/v projection 51.7 -> 41.3 us with
// 64-row entries; 128-row entries made the q/k/v projection slower, 53.1
// against 51.3 us, as its A rows are then staged in four synchronous chunks).
// The choice does not change any row's result (an MFMA row depends only on its
// own A row, and the k order is the same).
int dense_mt(int NB, int M, int mt) {
  const long long tiles = (NB + 7) / 8;
  while (mt < 4 && tiles * ((M + 32 * mt - 1) / (32 * mt)) >= 256) mt *= 2;
  return mt;
}

// capacity of the expert work list for M tokens in entries of er rows: every
// routed expert adds at most one partial entry beyond M*k/er, the shared
// expert M/er (the workspace is sized for the smallest entries, 32 rows)
int work_cap(const dg_config& c, int M, int er = kEntryRows) {
  return c.n_experts + (M * c.top_k + er - 1) / er + (M + er - 1) / er;
}

// split-K factor of the router GEMM: its weights are small (H x E), so the K
// range is cut into kRouterSplit slices to spread the stream over many
// workgroups; the routing kernel adds the partial logits in slice order
constexpr int kRouterSplit = 8;
// MXFP4 expert storage: per expert, codes (bytes) and scales (bytes) of an
// operand with NB n-blocks and K / 32 k-steps (k-groups of four, padded)
struct QSize { long long codes, scales; };
QSize mxfp4_size(long long NB, long long K) {
  const long long KG = ((K >> 5) + 3) >> 2;
  return QSize{NB * KG * 1024, NB * KG * 64};
}
bool mxfp4(const dg_config& c) { return c.expert_format == DG_EXPERT_MXFP4; }
// Row tiles of 16 per expert work entry: 64-row entries once the experts
// average 48 routed rows or more (several canvases), so fewer entries re-read
// each weight tile from L2; 32-row entries otherwise.  Measured on four
// canvases (1024 rows): gate|up 191 -> 170 us, down 109 -> 104 us; on one
// canvas 64-row entries were slower (96.9 / 57.8 us against 95.6 / 54.5).  The
// choice does not change any row's result: an MFMA row depends only on its own
// A row, and the k order is the same.
int expert_mt(const dg_config& c, int M) {
  return (c.dtype == DG_BF16 && !mxfp4(c) && M * c.top_k >= 48 * c.n_experts) ? 4 : kStreamMT;
}

int router_split(const dg_config& c) { return ((c.hidden / 32) % kRouterSplit) == 0 ? kRouterSplit : 1; }
int kv_len(const dg_config& c, int l, int prompt_len) {
  return is_global(c, l) ? prompt_len : (prompt_len < c.window ? prompt_len : c.window);
}

dg_status check_config(const dg_config* c) {
  dg_ctx* ctx = nullptr;
  if (!c) return fail(ctx, DG_EINVAL, "config is NULL");
  if (c->n_layers < 1 || c->n_layers > 64) return fail(ctx, DG_EINVAL, "n_layers must be in [1, 64]");
  // the norm kernels hold a row of the residual stream in registers: H <= 4096
  const int kmax = 4096;
  if (c->hidden <= 0 || c->hidden % 32 || c->hidden > kmax)
    return fail(ctx, DG_EUNSUPPORTED, "hidden must be a positive multiple of 32 (<= %d)", kmax);
  if (c->expert_ffn > kmax) return fail(ctx, DG_EUNSUPPORTED, "expert_ffn must be <= %d", kmax);
  if (c->n_heads <= 0 || c->n_kv_heads <= 0 || c->n_heads % c->n_kv_heads)
    return fail(ctx, DG_EINVAL, "n_heads must be a positive multiple of n_kv_heads");
  if (c->head_dim <= 0 || c->head_dim % 32 || c->head_dim > 256)
    return fail(ctx, DG_EUNSUPPORTED, "head_dim must be a multiple of 32 in [32, 256]");
  if (c->n_experts <= 0 || c->n_experts % 16 || c->n_experts > 256)
    return fail(ctx, DG_EUNSUPPORTED, "n_experts must be a multiple of 16 in [16, 256]");
  if (c->top_k < 1 || c->top_k > 8 || c->top_k > c->n_experts)
    return fail(ctx, DG_EINVAL, "top_k must be in [1, min(8, n_experts)]");
  if (c->n_shared != 1) return fail(ctx, DG_EUNSUPPORTED, "exactly one shared expert is supported");
  if (c->expert_ffn <= 0 || c->expert_ffn % 32)
    return fail(ctx, DG_EUNSUPPORTED, "expert_ffn must be a positive multiple of 32");
  if (c->has_lm_head && (c->vocab <= 0 || c->vocab % 16))
    return fail(ctx, DG_EUNSUPPORTED, "vocab must be a positive multiple of 16");
  if (c->canvas_len <= 0 || c->canvas_len % 16 || c->canvas_len > 4096)
    return fail(ctx, DG_EUNSUPPORTED, "canvas_len must be a multiple of 16 in [16, 4096]");
  if (c->max_batch < 1 || c->max_batch > DG_MAX_BATCH)
    return fail(ctx, DG_EINVAL, "max_batch must be in [1, 64]");
  const long long M = (long long)c->max_batch * c->canvas_len;
  if (M > 4096) return fail(ctx, DG_EUNSUPPORTED, "max_batch * canvas_len must be <= 4096");
  if ((long long)c->n_experts * ((M + 31) / 32) > 16384)
    return fail(ctx, DG_EUNSUPPORTED, "n_experts * ceil(max_batch*canvas_len/32) must be <= 16384");
  if (c->window < 0 || c->max_prompt_len < 0) return fail(ctx, DG_EINVAL, "window and max_prompt_len must be >= 0");
  if (c->dtype != DG_F32 && c->dtype != DG_BF16) return fail(ctx, DG_EINVAL, "dtype must be DG_F32 or DG_BF16");
  if (c->expert_format != DG_EXPERT_NATIVE && c->expert_format != DG_EXPERT_MXFP4)
    return fail(ctx, DG_EINVAL, "expert_format must be DG_EXPERT_NATIVE or DG_EXPERT_MXFP4");
  if (c->expert_format == DG_EXPERT_MXFP4 && c->dtype != DG_BF16)
    return fail(ctx, DG_EUNSUPPORTED, "MXFP4 experts need a DG_BF16 context");
  if (!(c->rope_theta > 0.f) || !(c->prope_frac >= 0.f && c->prope_frac <= 1.f) || !(c->rms_eps >= 0.f))
    return fail(ctx, DG_EINVAL, "rope_theta > 0, prope_frac in [0, 1] and rms_eps >= 0 required");
  return DG_OK;
}

dg_status enter(dg_ctx* ctx) {
  if (!ctx) return fail(nullptr, DG_EINVAL, "context is NULL");
  ctx->err.clear();
  HIPX(hipSetDevice(ctx->dev));
  // surface asynchronous faults of earlier work without blocking
  HIPX(hipGetLastError());
  // an out-of-range token id recorded by an earlier call's embedding (seen
  // once that work has run): reported once, then cleared
  if (ctx->bad_id) {
    const uint64_t b = __atomic_exchange_n(ctx->bad_id, (uint64_t)0, __ATOMIC_ACQ_REL);
    if (b) {
      const long long row = (long long)(b >> 32) - 1;
      const int32_t id = (int32_t)(uint32_t)b;
      return fail(ctx, DG_EINVAL,
                  "an earlier call was given token id %d at row %lld (canvas %lld, position %lld), outside "
                  "[0, %d); that row was embedded as zeros",
                  id, row, row / ctx->c.canvas_len, row % ctx->c.canvas_len, ctx->c.vocab);
    }
  }
  return DG_OK;
}

dg_status alloc_workspaces(dg_ctx* ctx) {
  const dg_config& c = ctx->c;
  const size_t M = (size_t)c.max_batch * c.canvas_len;
  const size_t H = c.hidden, D = c.head_dim, E = c.n_experts, K = c.top_k, F = c.expert_ffn;
  const size_t es = ctx->es;
  const size_t rows_r = M * K + M;
  TRY(dalloc_t(ctx, &ctx->x, M * H * 4));
  TRY(dalloc_t(ctx, &ctx->ao, M * H * 4));
  TRY(dalloc(ctx, &ctx->a, M * H * es));
  TRY(dalloc(ctx, &ctx->f, M * H * es));
  TRY(dalloc(ctx, &ctx->q, M * c.n_heads * D * es));
  TRY(dalloc(ctx, &ctx->kc, M * c.n_kv_heads * D * es));
  TRY(dalloc(ctx, &ctx->vc, M * c.n_kv_heads * D * es));
  TRY(dalloc(ctx, &ctx->o, M * c.n_heads * D * es));
  TRY(dalloc_t(ctx, &ctx->rl, (size_t)kRouterSplit * M * E * 4));
  TRY(dalloc_t(ctx, &ctx->idx, M * K * 4));
  TRY(dalloc_t(ctx, &ctx->gates, M * K * 4));
  TRY(dalloc_t(ctx, &ctx->offsets, (E + 2) * 4));
  TRY(dalloc_t(ctx, &ctx->perm, rows_r * 4));
  TRY(dalloc_t(ctx, &ctx->arows, rows_r * 4));
  TRY(dalloc(ctx, &ctx->u, rows_r * F * es));
  TRY(dalloc_t(ctx, &ctx->y, rows_r * H * 4));
  ctx->lm_fused = c.has_lm_head && ctx->bf16 && lm_head_supported((int)M, c.hidden, c.vocab);
  if (ctx->lm_fused) {
    const size_t parts = (size_t)((c.vocab / 16 + 15) / 16) * M;
    TRY(dalloc_t(ctx, &ctx->lm_m, parts * 4));
    TRY(dalloc_t(ctx, &ctx->lm_s, parts * 4));
    TRY(dalloc_t(ctx, &ctx->lm_i, parts * 4));
    TRY(dalloc_t(ctx, &ctx->lm_u, parts * 4));
    TRY(dalloc_t(ctx, &ctx->lm_g, parts * 4));
    TRY(dalloc_t(ctx, &ctx->lm_gi, parts * 4));
  } else if (c.has_lm_head) {
    TRY(dalloc_t(ctx, &ctx->logits, M * (size_t)c.vocab * 4));
  }
  TRY(dalloc_t(ctx, &ctx->pred, M * 4));
  TRY(dalloc_t(ctx, &ctx->conf, M * 4));
  if (c.has_lm_head) {
    TRY(dalloc_t(ctx, &ctx->eb_ent, M * 4));
    TRY(dalloc_t(ctx, &ctx->eb_samp, M * 4));
    TRY(dalloc_t(ctx, &ctx->eb_prev, M * 4));
    TRY(dalloc_t(ctx, &ctx->eb_status, (size_t)c.max_batch * 4));
    void* hp = nullptr;
    HIPX(hipHostMalloc(&hp, (size_t)c.max_batch * 4, hipHostMallocDefault));
    ctx->eb_status_host = static_cast<int32_t*>(hp);
    void* bp = nullptr;
    HIPX(hipHostMalloc(&bp, sizeof(uint64_t), hipHostMallocDefault));
    ctx->bad_id = static_cast<uint64_t*>(bp);
    *ctx->bad_id = 0;
  }
  TRY(dalloc_t(ctx, &ctx->rope, (size_t)c.max_batch * c.canvas_len * (D / 2) * sizeof(float2)));
  // attention split partials: up to 64 splits of every query row
  const long long qrows = (long long)M * c.n_heads;
  ctx->part_cap = qrows * 64;
  TRY(dalloc_t(ctx, &ctx->part_o, (size_t)ctx->part_cap * D * 4));
  TRY(dalloc_t(ctx, &ctx->part_m, (size_t)ctx->part_cap * 4));
  TRY(dalloc_t(ctx, &ctx->part_l, (size_t)ctx->part_cap * 4));
  TRY(dalloc_t(ctx, &ctx->work, (size_t)work_cap(c, (int)M) * sizeof(int4)));
  // entry count, then the first entry of every expert, the shared expert and the end
  TRY(dalloc_t(ctx, &ctx->work_count, (size_t)(E + 3) * 4));
  HIPX(hipMemset(ctx->work_count, 0, (size_t)(E + 3) * 4));
  HIPX(hipDeviceSynchronize());
  return DG_OK;
}

bool weights_ready(const dg_ctx* ctx) {
  for (const auto& l : ctx->L)
    if (!l.set) return false;
  return !ctx->c.has_lm_head || ctx->embed_set;
}

dg_status check_slots(dg_ctx* ctx, int batch) {
  for (int b = 0; b < batch; ++b)
    if (ctx->slots[b].prompt_len < 0)
      return fail(ctx, DG_ESTATE, "prompt KV of slot %d is not loaded", b);
  return DG_OK;
}

// ---------------------------------------------------------------------------
// pass building blocks
// ---------------------------------------------------------------------------

dg_status enqueue_qkv(dg_ctx* ctx, int l, int B, const void* a, void* q, void* k, void* v,
                      const long long* qs, const long long* ks, const long long* vs) {
  const dg_config& c = ctx->c;
  const int H = c.hidden, D = c.head_dim;
  const int M = B * c.canvas_len;
  StreamArgs g{};
  g.A = a; g.lda = H; g.B = ctx->L[l].qkv; g.K = H;
  g.NB = (c.n_heads + 2 * c.n_kv_heads) * D / 16;
  // 64-row entries once that still fills the chip (several canvases), bf16 only
  g.mt = ctx->bf16 ? dense_mt(g.NB, M, kStreamMT) : kStreamMT;
  g.n_dense = (M + 16 * g.mt - 1) / (16 * g.mt); g.dense_rows = M;
  EpiArgs e{};
  e.kind = EPI_QKV;
  e.q = q; e.k = k; e.v = v;
  for (int i = 0; i < 4; ++i) { e.qs[i] = qs[i]; e.ks[i] = ks[i]; e.vs[i] = vs[i]; }
  e.rope_cs = ctx->rope;
  e.N = c.canvas_len; e.D = D; e.Hq = c.n_heads; e.Hkv = c.n_kv_heads;
  e.n_rot_local = D / 2;
  e.n_rot_global = (int)(c.prope_frac * (float)(D / 2));
  e.is_global = is_global(c, l);
  HIPX(launch_stream(ctx->bf16, g, e, ctx->st));
  return DG_OK;
}

dg_status enqueue_attention(dg_ctx* ctx, int l, int B, void* o, int canvas_keys, int causal = 0) {
  const dg_config& c = ctx->c;
  AttnArgs aa{};
  aa.q = ctx->q; aa.kc = ctx->kc; aa.vc = ctx->vc;
  aa.B = B; aa.N = c.canvas_len; aa.Hq = c.n_heads; aa.Hkv = c.n_kv_heads; aa.D = c.head_dim;
  aa.canvas_keys = canvas_keys;
  aa.causal = causal;
  aa.o = o;
  aa.part_o = ctx->part_o; aa.part_m = ctx->part_m; aa.part_l = ctx->part_l;
  aa.part_cap_rows = ctx->part_cap;
  for (int b = 0; b < B; ++b) {
    aa.kp[b] = ctx->slots[b].k[l];
    aa.vp[b] = ctx->slots[b].v[l];
    aa.lw[b] = ctx->slots[b].len[l];
  }
  HIPX(launch_attention(ctx->bf16, aa, ctx->st, prof_kernel(ctx, DG_PROF_ATTN)));
  return DG_OK;
}

// Routing of layer l.  ROUTE_LOGITS: router logits of ctx->f (split-K partials in
// ctx->rl), then top-k and the scatter; ROUTE_GIVEN: ctx->idx/gates are given.
dg_status enqueue_route(dg_ctx* ctx, int l, int M, int mode) {
  const dg_config& c = ctx->c;
  const int E = c.n_experts, H = c.hidden;
  RouteArgs r{};
  r.mode = mode; r.rows = M; r.E = E; r.k = c.top_k;
  if (mode == ROUTE_LOGITS) {
    EpiArgs e{};
    e.kind = EPI_STORE_F32; e.out = ctx->rl; e.ldo = E;
    StreamArgs g{};
    g.A = ctx->f; g.lda = H; g.B = ctx->L[l].router; g.K = H; g.NB = E / 16;
    g.mt = 1; g.n_dense = (M + 15) / 16; g.dense_rows = M;
    g.ksplit = router_split(c); g.split_stride = (long long)M * E;
    HIPX(launch_stream(ctx->bf16, g, e, ctx->st));
    r.logits = ctx->rl; r.logit_parts = g.ksplit; r.part_stride = g.split_stride;
  }
  r.idx = ctx->idx; r.gates = ctx->gates;
  r.offsets = ctx->offsets; r.perm = ctx->perm; r.a_rows = ctx->arows;
  r.work = ctx->work; r.work_count = ctx->work_count; r.ent_off = ctx->work_count + 1;
  r.entry_rows = 16 * expert_mt(c, M);
  r.with_shared = 1;
  HIPX(launch_route(r, ctx->st));
  return DG_OK;
}

// routed + shared expert FFNs of layer l on f (routing already in idx/gates/perm/arows/work);
// leaves y [M*k + M, H]: row t*k + s holds gate[t,s] * FFN_e(f_t), row M*k + t the shared FFN
dg_status enqueue_experts(dg_ctx* ctx, int l, int M, const void* f) {
  const dg_config& c = ctx->c;
  const int H = c.hidden, F = c.expert_ffn, K = c.top_k;
  StreamArgs g{};
  g.A = f; g.lda = H; g.a_rows = ctx->arows; g.a_rows_max = M;
  g.B = ctx->L[l].gu; g.b_group_stride = 2LL * F * H;
  g.K = H; g.NB = 2 * F / 16; g.mt = expert_mt(c, M);
  if (mxfp4(c)) {
    const QSize q = mxfp4_size(g.NB, H);
    g.qb = 1;
    g.Bq = reinterpret_cast<const uint4*>(ctx->L[l].gu); g.bq_group_stride = q.codes / 16;
    g.Bs = reinterpret_cast<const uint32_t*>(ctx->L[l].gu_s); g.bs_group_stride = q.scales / 4;
  }
  g.work = ctx->work; g.work_count = ctx->work_count; g.work_cap = work_cap(c, M, 16 * expert_mt(c, M));
  g.ent_off = ctx->work_count + 1; g.n_groups = c.n_experts + 1;
  EpiArgs e{};
  e.kind = EPI_GEGLU; e.out = ctx->u; e.ldo = F;
  HIPX(launch_stream(ctx->bf16, g, e, ctx->st, prof_kernel(ctx, DG_PROF_GATE_UP)));

  StreamArgs d{};
  d.A = ctx->u; d.lda = F; d.a_rows = nullptr;
  d.B = ctx->L[l].down; d.b_group_stride = (long long)F * H;
  d.K = F; d.NB = H / 16; d.mt = expert_mt(c, M);
  if (mxfp4(c)) {
    const QSize q = mxfp4_size(d.NB, F);
    d.qb = 1;
    d.Bq = reinterpret_cast<const uint4*>(ctx->L[l].down); d.bq_group_stride = q.codes / 16;
    d.Bs = reinterpret_cast<const uint32_t*>(ctx->L[l].down_s); d.bs_group_stride = q.scales / 4;
  }
  // down keeps the tile-major order: its A rows (u) are few, and spreading the
  // concurrent weight reads over many experts streams faster here
  d.work = ctx->work; d.work_count = ctx->work_count; d.work_cap = work_cap(c, M, 16 * expert_mt(c, M));
  EpiArgs ed{};
  ed.kind = EPI_DOWN; ed.out = ctx->y; ed.ldo = H;
  ed.slot = ctx->perm; ed.gates = ctx->gates; ed.routed_rows = M * K; ed.out_rows = M * K + M;
  HIPX(launch_stream(ctx->bf16, d, ed, ctx->st, prof_kernel(ctx, DG_PROF_DOWN)));
  return DG_OK;
}

// Dense y = A @ W into fp32.  Small weights (the output projection) stream per
// 32-row entry and re-read W from L2; the LM head's 1 GB embedding is read once
// per 64-row chunk by the chunked kernel instead.
dg_status enqueue_dense(dg_ctx* ctx, const void* A, int lda, const void* Bp, int K, int N, int M, float* out,
                        int ldo, bool streaming = true, KTime t = {}) {
  EpiArgs e{};
  e.kind = EPI_STORE_F32; e.out = out; e.ldo = ldo;
  if (streaming) {
    StreamArgs g{};
    g.A = A; g.lda = lda; g.B = Bp; g.K = K; g.NB = N / 16;
    // 32-row entries unless that leaves fewer workgroups than the chip has CUs
    const long long tiles = (g.NB + 7) / 8;
    g.mt = dense_mt(g.NB, M, tiles * ((M + kEntryRows - 1) / kEntryRows) >= 256 ? kStreamMT : 1);
    g.n_dense = (M + 16 * g.mt - 1) / (16 * g.mt); g.dense_rows = M;
    HIPX(launch_stream(ctx->bf16, g, e, ctx->st, t));
  } else {
    GemmArgs g{};
    g.A = A; g.lda = lda; g.B = Bp; g.K = K; g.NB = N / 16; g.static_rows = M;
    HIPX(launch_gemm(ctx->bf16, g, e, 4, ctx->st, t));
  }
  return DG_OK;
}

// Appends the canvas K/V of layer l (ctx->kc / ctx->vc, canvas b) to slot b's
// cache of that layer: the grown visible range goes into the spare buffers,
// which then become the cache (stream order keeps the layer's attention on
// the old ones).  The slot's prompt_len moves on after the last layer.
dg_status append_block_kv(dg_ctx* ctx, int l, int b, int n) {
  const dg_config& c = ctx->c;
  SlotKV& S = ctx->slots[b];
  const int N = c.canvas_len, Hkv = c.n_kv_heads, D = c.head_dim;
  const int old_len = S.len[l], new_len = kv_len(c, l, S.prompt_len + n);
  if (S.k2.empty()) {
    S.k2.assign(c.n_layers, nullptr);
    S.v2.assign(c.n_layers, nullptr);
    S.cap2.assign(c.n_layers, 0);
  }
  if (S.cap2[l] < new_len) {
    const long long cap = kv_len(c, l, c.max_prompt_len);
    HIPX(hipStreamSynchronize(ctx->st));
    dfree(ctx, S.k2[l]);
    dfree(ctx, S.v2[l]);
    S.k2[l] = S.v2[l] = nullptr;
    S.cap2[l] = 0;
    TRY(dalloc(ctx, &S.k2[l], (size_t)(cap * Hkv * D) * ctx->es));
    TRY(dalloc(ctx, &S.v2[l], (size_t)(cap * Hkv * D) * ctx->es));
    S.cap2[l] = cap;
  }
  const long long blk_first = S.prompt_len, old_first = blk_first - old_len;
  const long long first = blk_first + n - new_len;
  const size_t kb = (size_t)b * Hkv * N * D;  // canvas b in the canvas K / V^T buffers
  HIPX(launch_kv_append(ctx->bf16, S.k[l], S.v[l], old_len, old_first,
                        static_cast<char*>(ctx->kc) + kb * ctx->es, static_cast<char*>(ctx->vc) + kb * ctx->es, N, n,
                        blk_first, new_len, first, Hkv, D, S.k2[l], S.v2[l], ctx->st));
  std::swap(S.k[l], S.k2[l]);
  std::swap(S.v[l], S.v2[l]);
  std::swap(S.cap[l], S.cap2[l]);
  S.len[l] = new_len;
  if (S.cap2[l] < S.cap[l]) {
    // the spare is the buffer the cache was loaded into: give it the full
    // capacity now, so later commits only enqueue work
    HIPX(hipStreamSynchronize(ctx->st));
    dfree(ctx, S.k2[l]);
    dfree(ctx, S.v2[l]);
    S.k2[l] = S.v2[l] = nullptr;
    S.cap2[l] = 0;
    TRY(dalloc(ctx, &S.k2[l], (size_t)(S.cap[l] * Hkv * D) * ctx->es));
    TRY(dalloc(ctx, &S.v2[l], (size_t)(S.cap[l] * Hkv * D) * ctx->es));
    S.cap2[l] = S.cap[l];
  }
  return DG_OK;
}

// Decoder layers on ctx->x, with ctx->a holding the normalised input of the
// first layer.  The last layer leaves RMSNorm(x)(1 + w_last_out) in ctx->a when
// w_last_out is given (the final norm before the LM head).  commit: causal
// canvas attention, each layer's canvas K/V appended to the caches right after
// its attention, and nothing after the last layer's attention.
// commit_n > 0: the causal context-building pass of a block commit; after
// each layer's attention the first commit_n positions' K/V join the caches
dg_status enqueue_layers(dg_ctx* ctx, int B, const void* w_last_out, int l0 = 0, int l1 = -1, int commit_n = 0) {
  const dg_config& c = ctx->c;
  const bool commit = commit_n > 0;
  if (l1 < 0) l1 = c.n_layers;
  const int N = c.canvas_len, M = B * N, H = c.hidden, D = c.head_dim;
  const int Hq = c.n_heads, Hkv = c.n_kv_heads, E = c.n_experts, K = c.top_k;
  const long long qs[4] = {(long long)Hq * N * D, (long long)N * D, D, 1};
  const long long ks[4] = {(long long)Hkv * N * D, (long long)N * D, D, 1};
  const long long vs[4] = {(long long)Hkv * D * N, (long long)D * N, 1, N};
  for (int l = l0; l < l1; ++l) {
    const LayerW& W = ctx->L[l];
    TRY(enqueue_qkv(ctx, l, B, ctx->a, ctx->q, ctx->kc, ctx->vc, qs, ks, vs));
    TRY(enqueue_attention(ctx, l, B, ctx->o, 1, commit ? 1 : 0));
    if (commit) {
      for (int b = 0; b < B; ++b) TRY(append_block_kv(ctx, l, b, commit_n));
      if (l + 1 == l1) break;  // later layers' inputs are not needed
    }
    TRY(enqueue_dense(ctx, ctx->o, Hq * D, W.wo, Hq * D, H, M, ctx->ao, H));
    // x += RMSNorm(o Wo)(1 + w_pa); f = RMSNorm(x)(1 + w_pf)
    NormArgs na{};
    na.mode = 0; na.rows = M; na.H = H; na.k = K; na.eps = c.rms_eps;
    na.x = ctx->x; na.delta = ctx->ao; na.w_delta = W.norm[1]; na.w_out = W.norm[2]; na.out = ctx->f;
    HIPX(launch_residual_norm(ctx->bf16, na, ctx->st));
    TRY(enqueue_route(ctx, l, M, ROUTE_LOGITS));
    if (ctx->trace)
      HIPX(hipMemcpyAsync(ctx->trace + (size_t)l * M * K, ctx->idx, (size_t)M * K * 4,
                          hipMemcpyDeviceToDevice, ctx->st));
    TRY(enqueue_experts(ctx, l, M, ctx->f));
    NormArgs nc{};
    nc.mode = 1; nc.rows = M; nc.H = H; nc.k = K; nc.eps = c.rms_eps;
    nc.x = ctx->x; nc.delta = ctx->y; nc.w_delta = c.post_ffn_norm ? W.norm[3] : nullptr;
    nc.w_out = (l + 1 < l1) ? ctx->L[l + 1].norm[0] : w_last_out;
    nc.out = ctx->a;
    HIPX(launch_residual_norm(ctx->bf16, nc, ctx->st));
  }
  return DG_OK;
}

// Tied LM head over h [M, H] into per-row argmax and confidence: fused on
// matrix cores (bf16), else logits into the workspace and a row reduction.
LmArgs lm_args(dg_ctx* ctx, const void* h, int M) {
  LmArgs la{};
  la.h = h; la.M = M; la.K = ctx->c.hidden; la.V = ctx->c.vocab; la.E = ctx->embed;
  la.part_m = ctx->lm_m; la.part_s = ctx->lm_s; la.part_i = ctx->lm_i;
  return la;
}
dg_status enqueue_head(dg_ctx* ctx, const void* h, int M, int32_t* pred, float* conf, KTime t = {}) {
  const dg_config& c = ctx->c;
  if (ctx->lm_fused) {
    LmArgs la = lm_args(ctx, h, M);
    la.pred = pred; la.conf = conf;
    HIPX(launch_lm_head(la, LM_ARGMAX, ctx->st, t));
    return DG_OK;
  }
  TRY(enqueue_dense(ctx, h, c.hidden, ctx->embed, c.hidden, c.vocab, M, ctx->logits, c.vocab, false, t));
  HIPX(launch_argmax_conf(ctx->logits, M, c.vocab, pred, conf, ctx->st));
  return DG_OK;
}

// Sampler statistics of h [M, H]: greedy id, entropy of softmax(l / tau) and
// the Gumbel-max sample per row (fused on matrix cores for bf16, else logits
// into the workspace and a row kernel).
dg_status enqueue_head_eb(dg_ctx* ctx, const void* h, int M, const EbArg& eb, int32_t* pred, float* ent,
                          int32_t* samp, KTime t = {}) {
  const dg_config& c = ctx->c;
  if (ctx->lm_fused) {
    LmArgs la = lm_args(ctx, h, M);
    la.part_u = ctx->lm_u; la.part_g = ctx->lm_g; la.part_gi = ctx->lm_gi;
    la.pred = pred; la.ent = ent; la.samp = samp; la.eb = eb;
    HIPX(launch_lm_head(la, LM_SAMPLE, ctx->st, t));
    return DG_OK;
  }
  TRY(enqueue_dense(ctx, h, c.hidden, ctx->embed, c.hidden, c.vocab, M, ctx->logits, c.vocab, false, t));
  HIPX(launch_eb_rows(ctx->logits, M, c.vocab, eb, pred, ent, samp, ctx->st));
  return DG_OK;
}

// embed -> decoder stack -> final norm into ctx->a
dg_status enqueue_trunk(dg_ctx* ctx, int B, const int32_t* tokens) {
  const dg_config& c = ctx->c;
  const int M = B * c.canvas_len, H = c.hidden;
  HIPX(launch_embed(ctx->bf16, tokens, M, H, c.vocab, c.canvas_len, c.canvas_len, ctx->embed, ctx->x, ctx->bad_id,
                    ctx->st));
  NormArgs n0{};
  n0.mode = 2; n0.rows = M; n0.H = H; n0.k = c.top_k; n0.eps = c.rms_eps;
  n0.x = ctx->x; n0.w_out = ctx->L[0].norm[0]; n0.out = ctx->a;
  HIPX(launch_residual_norm(ctx->bf16, n0, ctx->st));
  TRY(enqueue_layers(ctx, B, ctx->norm_final));
  return DG_OK;
}

dg_status enqueue_pass(dg_ctx* ctx, int B, int32_t* tokens, uint8_t* locked, const StepsArg& steps) {
  const int N = ctx->c.canvas_len, M = B * N;
  TRY(enqueue_trunk(ctx, B, tokens));
  TRY(enqueue_head(ctx, ctx->a, M, ctx->pred, ctx->conf, prof_kernel(ctx, DG_PROF_LM_HEAD)));
  HIPX(launch_lock_select(B, N, ctx->conf, ctx->pred, tokens, locked, steps, ctx->st));
  return DG_OK;
}

// Temperature of pass t of at most t_max: linear from 0.8 to 0.4
// ([4xFaster] "Recommended Inference Settings").
EbArg eb_arg(const dg_config& c, int t, int t_max, const uint32_t* seeds, int B, uint32_t block) {
  EbArg e{};
  const double tau = t_max > 1 ? 0.8 + (0.4 - 0.8) * t / (t_max - 1) : 0.8;
  e.inv_tau = (float)(1.0 / tau);
  e.t = (uint32_t)t;
  e.block = block;
  e.N = c.canvas_len;
  for (int b = 0; b < B; ++b) e.seed[b] = seeds[b];
  return e;
}

// One entropy-bounded pass: the stack, the sampler statistics and the lock step.
dg_status enqueue_pass_eb(dg_ctx* ctx, int B, int32_t* tokens, uint8_t* locked, int t, int t_max,
                          const EbArg& eb, int32_t* prev_pred, int32_t* status) {
  const int N = ctx->c.canvas_len, M = B * N;
  TRY(enqueue_trunk(ctx, B, tokens));
  TRY(enqueue_head_eb(ctx, ctx->a, M, eb, ctx->pred, ctx->eb_ent, ctx->eb_samp, prof_kernel(ctx, DG_PROF_LM_HEAD)));
  HIPX(launch_eb_select(B, N, ctx->eb_ent, ctx->eb_samp, ctx->pred, tokens, locked, prev_pred, status, t, t_max,
                        ctx->st));
  return DG_OK;
}

size_t bytes_of(const dg_ctx* ctx, long long n) { return (size_t)n * ctx->es; }

}  // namespace

// ============================================================================
// C ABI
// ============================================================================

extern "C" {

dg_status dg_create(const dg_config* cfg, int32_t device, void* hip_stream, dg_ctx** out) {
  g_create_error.clear();
  if (!out) return fail(nullptr, DG_EINVAL, "out is NULL");
  *out = nullptr;
  dg_status s = check_config(cfg);
  if (s != DG_OK) return s;
  int ndev = 0;
  hipError_t he = hipGetDeviceCount(&ndev);
  if (he != hipSuccess || ndev <= 0) return fail(nullptr, DG_EHIP, "no HIP device available");
  if (device < 0 || device >= ndev) return fail(nullptr, DG_EINVAL, "device %d out of range", device);
  he = hipSetDevice(device);
  if (he != hipSuccess) return fail(nullptr, DG_EHIP, "hipSetDevice: %s", hipGetErrorString(he));
  if (!scratch_addr(device)) return fail(nullptr, DG_EHIP, "device %d: address of the static scratch not found", device);
  dg_ctx* ctx = new dg_ctx();
  ctx->c = *cfg;
  ctx->dev = device;
  ctx->st = reinterpret_cast<hipStream_t>(hip_stream);
  ctx->bf16 = cfg->dtype == DG_BF16;
  ctx->es = ctx->bf16 ? 2 : 4;
  ctx->L.resize(cfg->n_layers);
  ctx->slots.resize(cfg->max_batch);
  s = alloc_workspaces(ctx);
  if (s != DG_OK) {
    g_create_error = ctx->err;
    dg_destroy(ctx);
    return s;
  }
  *out = ctx;
  return DG_OK;
}

dg_status dg_destroy(dg_ctx* ctx) {
  if (!ctx) return DG_OK;
  (void)hipSetDevice(ctx->dev);
  (void)hipStreamSynchronize(ctx->st);
  for (hipEvent_t e : ctx->ev_pool) (void)hipEventDestroy(e);
  for (void* p : ctx->owned)
    if (p) (void)hipFree(p);
  if (ctx->eb_status_host) (void)hipHostFree(ctx->eb_status_host);
  if (ctx->bad_id) (void)hipHostFree(ctx->bad_id);
  delete ctx;
  return DG_OK;
}

const char* dg_last_error(const dg_ctx* ctx) { return ctx ? ctx->err.c_str() : g_create_error.c_str(); }

dg_status dg_set_layer_weights(dg_ctx* ctx, int32_t layer, const dg_layer_weights* w) {
  TRY(enter(ctx));
  const dg_config& c = ctx->c;
  if (layer < 0 || layer >= c.n_layers) return fail(ctx, DG_EINVAL, "layer %d out of range", layer);
  if (!w) return fail(ctx, DG_EINVAL, "weights are NULL");
  const void* ptrs[15] = {w->wq, w->wk, w->wv, w->wo, w->router, w->w_gate, w->w_up, w->w_down,
                          w->sh_gate, w->sh_up, w->sh_down, w->norm_in, w->norm_pa, w->norm_pf, w->norm_pf2};
  for (int i = 0; i < 15; ++i)
    if (!ptrs[i]) return fail(ctx, DG_EINVAL, "layer %d: weight pointer %d is NULL", layer, i);
  const long long H = c.hidden, D = c.head_dim, E = c.n_experts, F = c.expert_ffn;
  const long long qd = c.n_heads * D, kvd = c.n_kv_heads * D;
  LayerW& L = ctx->L[layer];
  if (!L.qkv) {
    TRY(dalloc(ctx, &L.qkv, bytes_of(ctx, (qd + 2 * kvd) * H)));
    TRY(dalloc(ctx, &L.wo, bytes_of(ctx, qd * H)));
    TRY(dalloc(ctx, &L.router, bytes_of(ctx, H * E)));
    if (mxfp4(c)) {
      const QSize gq = mxfp4_size(2 * F / 16, H), dq = mxfp4_size(H / 16, F);
      TRY(dalloc(ctx, &L.gu, (size_t)((E + 1) * gq.codes)));
      TRY(dalloc(ctx, &L.gu_s, (size_t)((E + 1) * gq.scales)));
      TRY(dalloc(ctx, &L.down, (size_t)((E + 1) * dq.codes)));
      TRY(dalloc(ctx, &L.down_s, (size_t)((E + 1) * dq.scales)));
    } else {
      TRY(dalloc(ctx, &L.gu, bytes_of(ctx, (E + 1) * 2 * F * H)));
      TRY(dalloc(ctx, &L.down, bytes_of(ctx, (E + 1) * F * H)));
    }
    for (int i = 0; i < 4; ++i) TRY(dalloc(ctx, &L.norm[i], bytes_of(ctx, H)));
  }
  const int KB = (int)(H / 32);
  char* qkv = reinterpret_cast<char*>(L.qkv);
  PackArgs p{};
  // q and k with the rotary pairing, v plain; K = H for all three
  p = PackArgs{w->wq, nullptr, qd, (int)H, (int)qd, 1, 1, (int)D, c.n_heads, qkv};
  HIPX(launch_pack(ctx->bf16, p, ctx->st));
  p = PackArgs{w->wk, nullptr, kvd, (int)H, (int)kvd, 1, 1, (int)D, c.n_kv_heads,
               qkv + bytes_of(ctx, (qd / 16) * KB * 512)};
  HIPX(launch_pack(ctx->bf16, p, ctx->st));
  p = PackArgs{w->wv, nullptr, kvd, (int)H, (int)kvd, 1, 0, (int)D, 0,
               qkv + bytes_of(ctx, ((qd + kvd) / 16) * KB * 512)};
  HIPX(launch_pack(ctx->bf16, p, ctx->st));
  p = PackArgs{w->wo, nullptr, H, (int)qd, (int)H, 1, 0, 0, 0, L.wo};
  HIPX(launch_pack(ctx->bf16, p, ctx->st));
  p = PackArgs{w->router, nullptr, E, (int)H, (int)E, 1, 0, 0, 0, L.router};
  HIPX(launch_pack(ctx->bf16, p, ctx->st));
  // routed experts 0..E-1 then the shared expert at index E; MXFP4 experts are
  // packed as bf16 into a scratch buffer first and quantised from there
  void* tmp = nullptr;
  if (mxfp4(c)) TRY(dalloc(ctx, &tmp, bytes_of(ctx, (E + 1) * 2 * F * H)));
  void* gu_dst = mxfp4(c) ? tmp : L.gu;
  p = PackArgs{w->w_gate, w->w_up, F, (int)H, (int)(2 * F), 1, 2, 0, 0, gu_dst};
  HIPX(launch_pack_batched(ctx->bf16, p, (int)E, H * F, 2 * F * H, ctx->st));
  p = PackArgs{w->sh_gate, w->sh_up, F, (int)H, (int)(2 * F), 1, 2, 0, 0,
               reinterpret_cast<char*>(gu_dst) + bytes_of(ctx, E * 2 * F * H)};
  HIPX(launch_pack(ctx->bf16, p, ctx->st));
  if (mxfp4(c))
    HIPX(launch_quant_mxfp4(tmp, (int)E + 1, 2 * F * H, (int)(2 * F / 16), (int)(H / 32),
                            reinterpret_cast<uint4*>(L.gu), reinterpret_cast<uint8_t*>(L.gu_s), ctx->st));
  void* dn_dst = mxfp4(c) ? tmp : L.down;
  p = PackArgs{w->w_down, nullptr, H, (int)F, (int)H, 1, 0, 0, 0, dn_dst};
  HIPX(launch_pack_batched(ctx->bf16, p, (int)E, F * H, F * H, ctx->st));
  p = PackArgs{w->sh_down, nullptr, H, (int)F, (int)H, 1, 0, 0, 0,
               reinterpret_cast<char*>(dn_dst) + bytes_of(ctx, E * F * H)};
  HIPX(launch_pack(ctx->bf16, p, ctx->st));
  if (mxfp4(c)) {
    HIPX(launch_quant_mxfp4(tmp, (int)E + 1, F * H, (int)(H / 16), (int)(F / 32),
                            reinterpret_cast<uint4*>(L.down), reinterpret_cast<uint8_t*>(L.down_s), ctx->st));
    HIPX(hipStreamSynchronize(ctx->st));  // the scratch is read before it is freed
    dfree(ctx, tmp);
  }
  const void* norms[4] = {w->norm_in, w->norm_pa, w->norm_pf, w->norm_pf2};
  for (int i = 0; i < 4; ++i)
    HIPX(hipMemcpyAsync(L.norm[i], norms[i], bytes_of(ctx, H), hipMemcpyDeviceToDevice, ctx->st));
  L.set = true;
  return DG_OK;
}

dg_status dg_set_embedding(dg_ctx* ctx, const void* embed, const void* norm_final) {
  TRY(enter(ctx));
  const dg_config& c = ctx->c;
  if (!c.has_lm_head) return fail(ctx, DG_ESTATE, "context has no LM head");
  if (!embed || !norm_final) return fail(ctx, DG_EINVAL, "embed and norm_final are required");
  const long long H = c.hidden, V = c.vocab;
  if (!ctx->embed) {
    TRY(dalloc(ctx, &ctx->embed, bytes_of(ctx, V * H)));
    TRY(dalloc(ctx, &ctx->norm_final, bytes_of(ctx, H)));
  }
  // the LM head contracts over H: W(k = h, n = v) = embed[v][h]
  PackArgs p{embed, nullptr, H, (int)H, (int)V, 0, 0, 0, 0, ctx->embed};
  HIPX(launch_pack(ctx->bf16, p, ctx->st));
  HIPX(hipMemcpyAsync(ctx->norm_final, norm_final, bytes_of(ctx, H), hipMemcpyDeviceToDevice, ctx->st));
  ctx->embed_set = true;
  return DG_OK;
}

dg_status dg_init_weights(dg_ctx* ctx, const void* embed, const void* norm_final, const dg_layer_weights* layers) {
  TRY(enter(ctx));
  if (!layers) return fail(ctx, DG_EINVAL, "layers is NULL");
  if (ctx->c.has_lm_head) TRY(dg_set_embedding(ctx, embed, norm_final));
  for (int l = 0; l < ctx->c.n_layers; ++l) TRY(dg_set_layer_weights(ctx, l, &layers[l]));
  return DG_OK;
}

dg_status dg_load_prompt_kv(dg_ctx* ctx, int32_t slot, int32_t prompt_len, const void* const* k,
                            const void* const* v) {
  TRY(enter(ctx));
  const dg_config& c = ctx->c;
  if (slot < 0 || slot >= c.max_batch) return fail(ctx, DG_EINVAL, "slot %d out of range", slot);
  if (prompt_len < 0 || prompt_len > c.max_prompt_len)
    return fail(ctx, DG_EINVAL, "prompt_len %d outside [0, max_prompt_len=%d]", prompt_len, c.max_prompt_len);
  if (!k || !v) return fail(ctx, DG_EINVAL, "k and v arrays are required");
  for (int l = 0; l < c.n_layers; ++l)
    if (kv_len(c, l, prompt_len) > 0 && (!k[l] || !v[l]))
      return fail(ctx, DG_EINVAL, "layer %d: K/V pointer is NULL", l);
  SlotKV& S = ctx->slots[slot];
  if (S.k.empty()) {
    S.k.assign(c.n_layers, nullptr);
    S.v.assign(c.n_layers, nullptr);
    S.cap.assign(c.n_layers, 0);
    S.len.assign(c.n_layers, 0);
  }
  const int Hkv = c.n_kv_heads, D = c.head_dim;
  for (int l = 0; l < c.n_layers; ++l) {
    const int len = kv_len(c, l, prompt_len);
    if (len > S.cap[l]) {
      HIPX(hipStreamSynchronize(ctx->st));
      dfree(ctx, S.k[l]);
      dfree(ctx, S.v[l]);
      S.k[l] = S.v[l] = nullptr;
      S.cap[l] = 0;
      TRY(dalloc(ctx, &S.k[l], bytes_of(ctx, (long long)len * Hkv * D)));
      TRY(dalloc(ctx, &S.v[l], bytes_of(ctx, (long long)len * Hkv * D)));
      S.cap[l] = len;
    }
    S.len[l] = len;
    if (len > 0) {
      HIPX(launch_kv_repack(ctx->bf16, k[l], len, Hkv, D, S.k[l], 0, ctx->st));
      HIPX(launch_kv_repack(ctx->bf16, v[l], len, Hkv, D, S.v[l], 1, ctx->st));
    }
  }
  HIPX(launch_rope_table(ctx->rope + (size_t)slot * c.canvas_len * (D / 2), c.canvas_len, D, prompt_len,
                         (double)c.rope_theta, ctx->st));
  S.prompt_len = prompt_len;
  return DG_OK;
}

dg_status dg_denoise_step(dg_ctx* ctx, int32_t batch, int32_t* tokens, uint8_t* locked,
                          const int32_t* steps_left_host, float* conf_out, int32_t* pred_out) {
  TRY(enter(ctx));
  const dg_config& c = ctx->c;
  if (!c.has_lm_head) return fail(ctx, DG_ESTATE, "context has no LM head");
  if (batch < 1 || batch > c.max_batch) return fail(ctx, DG_EINVAL, "batch %d outside [1, %d]", batch, c.max_batch);
  if (!tokens || !locked || !steps_left_host) return fail(ctx, DG_EINVAL, "tokens, locked and steps_left are required");
  if (!weights_ready(ctx)) return fail(ctx, DG_ESTATE, "weights are not loaded");
  TRY(check_slots(ctx, batch));
  StepsArg steps{};
  for (int b = 0; b < batch; ++b) {
    if (steps_left_host[b] < 1) return fail(ctx, DG_EINVAL, "steps_left[%d] = %d < 1", b, steps_left_host[b]);
    steps.v[b] = steps_left_host[b];
  }
  hipEvent_t evp = prof_start(ctx, DG_PROF_PASS);
  TRY(enqueue_pass(ctx, batch, tokens, locked, steps));
  prof_stop(ctx, DG_PROF_PASS, evp);
  const size_t M = (size_t)batch * c.canvas_len;
  if (conf_out) HIPX(hipMemcpyAsync(conf_out, ctx->conf, M * 4, hipMemcpyDeviceToDevice, ctx->st));
  if (pred_out) HIPX(hipMemcpyAsync(pred_out, ctx->pred, M * 4, hipMemcpyDeviceToDevice, ctx->st));
  return DG_OK;
}

namespace {
// The first n of each canvas's N tokens join the prompt caches.  The block
// runs at full width: by the causal mask the positions past n influence none
// before them, and their K/V are not appended.
dg_status commit_tokens(dg_ctx* ctx, int32_t batch, const int32_t* tokens, int n) {
  const dg_config& c = ctx->c;
  if (!c.has_lm_head || !ctx->embed_set) return fail(ctx, DG_ESTATE, "the embedding is not loaded");
  if (batch < 1 || batch > c.max_batch) return fail(ctx, DG_EINVAL, "batch %d outside [1, %d]", batch, c.max_batch);
  if (!tokens) return fail(ctx, DG_EINVAL, "tokens is required");
  if (n < 1 || n > c.canvas_len) return fail(ctx, DG_EINVAL, "n = %d outside [1, %d]", n, c.canvas_len);
  if (!weights_ready(ctx)) return fail(ctx, DG_ESTATE, "weights are not loaded");
  TRY(check_slots(ctx, batch));
  const int N = c.canvas_len, M = batch * N, H = c.hidden;
  for (int b = 0; b < batch; ++b)
    if (ctx->slots[b].prompt_len + n > c.max_prompt_len)
      return fail(ctx, DG_EINVAL, "slot %d: prompt_len %d + %d exceeds max_prompt_len %d", b,
                  ctx->slots[b].prompt_len, n, c.max_prompt_len);
  // the block at positions prompt_len + i, causal within the block
  HIPX(launch_embed(ctx->bf16, tokens, M, H, c.vocab, N, n, ctx->embed, ctx->x, ctx->bad_id, ctx->st));
  NormArgs n0{};
  n0.mode = 2; n0.rows = M; n0.H = H; n0.k = c.top_k; n0.eps = c.rms_eps;
  n0.x = ctx->x; n0.w_out = ctx->L[0].norm[0]; n0.out = ctx->a;
  HIPX(launch_residual_norm(ctx->bf16, n0, ctx->st));
  TRY(enqueue_layers(ctx, batch, nullptr, 0, c.n_layers, n));
  const int D = c.head_dim;
  for (int b = 0; b < batch; ++b) {
    SlotKV& S = ctx->slots[b];
    S.prompt_len += n;
    HIPX(launch_rope_table(ctx->rope + (size_t)b * N * (D / 2), N, D, S.prompt_len, (double)c.rope_theta, ctx->st));
  }
  return DG_OK;
}
}  // namespace

dg_status dg_commit_block(dg_ctx* ctx, int32_t batch, const int32_t* tokens) {
  TRY(enter(ctx));
  return commit_tokens(ctx, batch, tokens, ctx->c.canvas_len);
}

dg_status dg_commit_tokens(dg_ctx* ctx, int32_t batch, const int32_t* tokens, int32_t n) {
  TRY(enter(ctx));
  return commit_tokens(ctx, batch, tokens, n);
}

dg_status dg_get_expert_weight(dg_ctx* ctx, int32_t layer, int32_t expert, int32_t which, void* values,
                               uint8_t* codes, uint8_t* scales) {
  TRY(enter(ctx));
  const dg_config& c = ctx->c;
  if (layer < 0 || layer >= c.n_layers || !ctx->L[layer].set) return fail(ctx, DG_ESTATE, "layer %d not loaded", layer);
  if (expert < 0 || expert > c.n_experts) return fail(ctx, DG_EINVAL, "expert %d outside [0, %d]", expert, c.n_experts);
  if (which < 0 || which > 2) return fail(ctx, DG_EINVAL, "which must be 0 (gate), 1 (up) or 2 (down)");
  if ((codes || scales) && !mxfp4(c)) return fail(ctx, DG_EINVAL, "codes and scales exist only for MXFP4 experts");
  const long long H = c.hidden, F = c.expert_ffn;
  const LayerW& L = ctx->L[layer];
  const bool down = which == 2;
  const int K = (int)(down ? F : H), N = (int)(down ? H : F);
  const long long NB = down ? H / 16 : 2 * F / 16;
  const void* packed = nullptr;
  const uint4* q = nullptr;
  const uint8_t* sc = nullptr;
  if (mxfp4(c)) {
    const QSize qs = mxfp4_size(NB, K);
    q = reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(down ? L.down : L.gu) + expert * qs.codes);
    sc = reinterpret_cast<const uint8_t*>(down ? L.down_s : L.gu_s) + expert * qs.scales;
  } else {
    packed = reinterpret_cast<const char*>(down ? L.down : L.gu) + bytes_of(ctx, expert * NB * 16 * K);
  }
  HIPX(launch_unpack_weight(ctx->bf16, packed, q, sc, K, N, down ? 0 : 2, which == 1 ? 1 : 0, values, codes, scales,
                            ctx->st));
  return DG_OK;
}

dg_status dg_get_prompt_kv(dg_ctx* ctx, int32_t slot, int32_t layer, void* k, void* v, int32_t* len_out) {
  TRY(enter(ctx));
  const dg_config& c = ctx->c;
  if (slot < 0 || slot >= c.max_batch) return fail(ctx, DG_EINVAL, "slot %d out of range", slot);
  if (layer < 0 || layer >= c.n_layers) return fail(ctx, DG_EINVAL, "layer %d out of range", layer);
  const SlotKV& S = ctx->slots[slot];
  if (S.prompt_len < 0) return fail(ctx, DG_ESTATE, "prompt KV of slot %d is not loaded", slot);
  const int len = S.len[layer], Hkv = c.n_kv_heads, D = c.head_dim;
  if (len_out) *len_out = len;
  if (len == 0 || (!k && !v)) return DG_OK;
  const int n[4] = {Hkv, len, D, 1};
  if (k) {  // K [Hkv][len][D] -> [len][Hkv][D]
    const long long ss[4] = {(long long)len * D, D, 1, 0}, ds[4] = {D, (long long)Hkv * D, 1, 0};
    HIPX(launch_permute4(ctx->bf16, S.k[layer], k, n, ss, ds, ctx->st));
  }
  if (v) {  // V^T [Hkv][D][len] -> [len][Hkv][D]
    const int nv[4] = {Hkv, D, len, 1};
    const long long ss[4] = {(long long)D * len, len, 1, 0}, ds[4] = {D, 1, (long long)Hkv * D, 0};
    HIPX(launch_permute4(ctx->bf16, S.v[layer], v, nv, ss, ds, ctx->st));
  }
  return DG_OK;
}

dg_status dg_generate_block(dg_ctx* ctx, int32_t batch, int32_t n_steps, int32_t* tokens, uint8_t* locked) {
  TRY(enter(ctx));
  const dg_config& c = ctx->c;
  if (!c.has_lm_head) return fail(ctx, DG_ESTATE, "context has no LM head");
  if (batch < 1 || batch > c.max_batch) return fail(ctx, DG_EINVAL, "batch %d outside [1, %d]", batch, c.max_batch);
  if (n_steps < 1) return fail(ctx, DG_EINVAL, "n_steps must be >= 1");
  if (!tokens || !locked) return fail(ctx, DG_EINVAL, "tokens and locked are required");
  if (!weights_ready(ctx)) return fail(ctx, DG_ESTATE, "weights are not loaded");
  TRY(check_slots(ctx, batch));
  for (int t = 0; t < n_steps; ++t) {
    StepsArg steps{};
    for (int b = 0; b < batch; ++b) steps.v[b] = n_steps - t;
    hipEvent_t evp = prof_start(ctx, DG_PROF_PASS);
    TRY(enqueue_pass(ctx, batch, tokens, locked, steps));
    prof_stop(ctx, DG_PROF_PASS, evp);
  }
  return DG_OK;
}

namespace {
dg_status check_eb(dg_ctx* ctx, int32_t batch, int32_t t, int32_t t_max, const uint32_t* seeds) {
  const dg_config& c = ctx->c;
  if (!c.has_lm_head) return fail(ctx, DG_ESTATE, "context has no LM head");
  if (batch < 1 || batch > c.max_batch) return fail(ctx, DG_EINVAL, "batch %d outside [1, %d]", batch, c.max_batch);
  if (t_max < 1 || t_max > (1 << 20)) return fail(ctx, DG_EINVAL, "t_max %d outside [1, 2^20]", t_max);
  if (t < 0 || t >= t_max) return fail(ctx, DG_EINVAL, "pass %d outside [0, t_max = %d)", t, t_max);
  if (!seeds) return fail(ctx, DG_EINVAL, "seeds are required");
  if (!weights_ready(ctx)) return fail(ctx, DG_ESTATE, "weights are not loaded");
  return check_slots(ctx, batch);
}
}  // namespace

dg_status dg_eb_step(dg_ctx* ctx, int32_t batch, int32_t* tokens, uint8_t* locked, int32_t t, int32_t t_max,
                     const uint32_t* seeds_host, uint32_t block, int32_t* prev_pred, int32_t* status,
                     float* entropy_out, int32_t* sample_out, int32_t* pred_out) {
  TRY(enter(ctx));
  TRY(check_eb(ctx, batch, t, t_max, seeds_host));
  if (!tokens || !locked || !prev_pred || !status)
    return fail(ctx, DG_EINVAL, "tokens, locked, prev_pred and status are required");
  const dg_config& c = ctx->c;
  const EbArg eb = eb_arg(c, t, t_max, seeds_host, batch, block);
  hipEvent_t evp = prof_start(ctx, DG_PROF_PASS);
  TRY(enqueue_pass_eb(ctx, batch, tokens, locked, t, t_max, eb, prev_pred, status));
  prof_stop(ctx, DG_PROF_PASS, evp);
  const size_t M = (size_t)batch * c.canvas_len;
  if (entropy_out) HIPX(hipMemcpyAsync(entropy_out, ctx->eb_ent, M * 4, hipMemcpyDeviceToDevice, ctx->st));
  if (sample_out) HIPX(hipMemcpyAsync(sample_out, ctx->eb_samp, M * 4, hipMemcpyDeviceToDevice, ctx->st));
  if (pred_out) HIPX(hipMemcpyAsync(pred_out, ctx->pred, M * 4, hipMemcpyDeviceToDevice, ctx->st));
  return DG_OK;
}

dg_status dg_generate_block_eb(dg_ctx* ctx, int32_t batch, int32_t* tokens, uint8_t* locked,
                               const uint32_t* seeds_host, uint32_t block, int32_t t_max, int32_t* passes_out) {
  TRY(enter(ctx));
  TRY(check_eb(ctx, batch, 0, t_max, seeds_host));
  if (!tokens || !locked) return fail(ctx, DG_EINVAL, "tokens and locked are required");
  const dg_config& c = ctx->c;
  std::vector<int32_t> passes(batch, 0);
  HIPX(hipMemsetAsync(ctx->eb_status, 0, (size_t)batch * 4, ctx->st));
  for (int t = 0; t < t_max; ++t) {
    const EbArg eb = eb_arg(c, t, t_max, seeds_host, batch, block);
    hipEvent_t evp = prof_start(ctx, DG_PROF_PASS);
    TRY(enqueue_pass_eb(ctx, batch, tokens, locked, t, t_max, eb, ctx->eb_prev, ctx->eb_status));
    prof_stop(ctx, DG_PROF_PASS, evp);
    // the stop decision is the device's: read the canvases' status after each pass
    HIPX(hipMemcpyAsync(ctx->eb_status_host, ctx->eb_status, (size_t)batch * 4, hipMemcpyDeviceToHost, ctx->st));
    HIPX(hipStreamSynchronize(ctx->st));
    bool all = true;
    for (int b = 0; b < batch; ++b) {
      if ((ctx->eb_status_host[b] & 1) && passes[b] == 0) passes[b] = t + 1;
      all = all && passes[b] != 0;
    }
    if (all) break;
  }
  if (passes_out)
    for (int b = 0; b < batch; ++b) passes_out[b] = passes[b];
  return DG_OK;
}

dg_status dg_forward_layers(dg_ctx* ctx, int32_t batch, int32_t first, int32_t count, const float* x_in,
                            float* x_out) {
  TRY(enter(ctx));
  const dg_config& c = ctx->c;
  if (batch < 1 || batch > c.max_batch) return fail(ctx, DG_EINVAL, "batch %d outside [1, %d]", batch, c.max_batch);
  if (first < 0 || count < 1 || first > c.n_layers - count)
    return fail(ctx, DG_EINVAL, "layers [%d, %d + %d) outside [0, %d)", first, first, count, c.n_layers);
  if (!x_in || !x_out) return fail(ctx, DG_EINVAL, "x_in and x_out are required");
  for (int l = first; l < first + count; ++l)
    if (!ctx->L[l].set) return fail(ctx, DG_ESTATE, "weights of layer %d are not loaded", l);
  TRY(check_slots(ctx, batch));
  const int M = batch * c.canvas_len, H = c.hidden;
  HIPX(hipMemcpyAsync(ctx->x, x_in, (size_t)M * H * 4, hipMemcpyDeviceToDevice, ctx->st));
  NormArgs n0{};
  n0.mode = 2; n0.rows = M; n0.H = H; n0.k = c.top_k; n0.eps = c.rms_eps;
  n0.x = ctx->x; n0.w_out = ctx->L[first].norm[0]; n0.out = ctx->a;
  HIPX(launch_residual_norm(ctx->bf16, n0, ctx->st));
  TRY(enqueue_layers(ctx, batch, nullptr, first, first + count));
  HIPX(hipMemcpyAsync(x_out, ctx->x, (size_t)M * H * 4, hipMemcpyDeviceToDevice, ctx->st));
  return DG_OK;
}

dg_status dg_forward_hidden(dg_ctx* ctx, int32_t batch, const float* x_in, float* x_out) {
  if (!ctx) return dg_forward_layers(ctx, batch, 0, 1, x_in, x_out);
  return dg_forward_layers(ctx, batch, 0, ctx->c.n_layers, x_in, x_out);
}

dg_status dg_set_trace(dg_ctx* ctx, int32_t* route_idx) {
  TRY(enter(ctx));
  ctx->trace = route_idx;
  return DG_OK;
}

// ---- single kernels --------------------------------------------------------

dg_status dg_k_argmax_conf(const float* logits, int32_t rows, int32_t vocab, int32_t* pred, float* conf,
                           void* stream) {
  dg_ctx* ctx = nullptr;
  if (rows < 0 || vocab <= 0 || vocab % 4) return fail(ctx, DG_EINVAL, "rows >= 0 and vocab a positive multiple of 4 required");
  if (rows == 0) return DG_OK;  // nothing to do; pointers may be NULL
  if (!logits || !pred || !conf) return fail(ctx, DG_EINVAL, "logits, pred and conf are required");
  HIPX(launch_argmax_conf(logits, rows, vocab, pred, conf, reinterpret_cast<hipStream_t>(stream)));
  return DG_OK;
}

dg_status dg_k_lock_select(int32_t batch, int32_t n, const float* conf, const int32_t* pred, int32_t* tokens,
                           uint8_t* locked, const int32_t* steps_left_host, void* stream) {
  dg_ctx* ctx = nullptr;
  if (!conf || !pred || !tokens || !locked || !steps_left_host)
    return fail(ctx, DG_EINVAL, "conf, pred, tokens, locked and steps_left are required");
  if (batch < 0 || batch > DG_MAX_BATCH || n < 1 || n > 4096)
    return fail(ctx, DG_EINVAL, "batch must be in [0, 64] and n in [1, 4096]");
  StepsArg steps{};
  for (int b = 0; b < batch; ++b) {
    if (steps_left_host[b] < 1) return fail(ctx, DG_EINVAL, "steps_left[%d] < 1", b);
    steps.v[b] = steps_left_host[b];
  }
  HIPX(launch_lock_select(batch, n, conf, pred, tokens, locked, steps, reinterpret_cast<hipStream_t>(stream)));
  return DG_OK;
}

dg_status dg_k_eb_rows(const float* logits, int32_t rows, int32_t vocab, int32_t canvas_len, int32_t t,
                       int32_t t_max, const uint32_t* seeds_host, uint32_t block, int32_t* pred, float* entropy,
                       int32_t* sample, void* stream) {
  dg_ctx* ctx = nullptr;
  if (rows < 0 || vocab < 1 || canvas_len < 1) return fail(ctx, DG_EINVAL, "rows >= 0, vocab >= 1, canvas_len >= 1 required");
  if (rows % canvas_len || rows / canvas_len > DG_MAX_BATCH)
    return fail(ctx, DG_EINVAL, "rows must be a multiple of canvas_len, at most 64 canvases");
  if (t_max < 1 || t < 0 || t >= t_max) return fail(ctx, DG_EINVAL, "pass %d outside [0, t_max = %d)", t, t_max);
  if (rows == 0) return DG_OK;
  if (!logits || !pred || !entropy || !sample || !seeds_host)
    return fail(ctx, DG_EINVAL, "logits, pred, entropy, sample and seeds are required");
  dg_config c{};
  c.canvas_len = canvas_len;
  const EbArg eb = eb_arg(c, t, t_max, seeds_host, rows / canvas_len, block);
  HIPX(launch_eb_rows(logits, rows, vocab, eb, pred, entropy, sample, reinterpret_cast<hipStream_t>(stream)));
  return DG_OK;
}

dg_status dg_k_eb_noise(int32_t rows, int32_t vocab, int32_t canvas_len, int32_t t, const uint32_t* seeds_host,
                        uint32_t block, float* noise, void* stream) {
  dg_ctx* ctx = nullptr;
  if (rows < 0 || vocab < 1 || canvas_len < 1) return fail(ctx, DG_EINVAL, "rows >= 0, vocab >= 1, canvas_len >= 1 required");
  if (rows % canvas_len || rows / canvas_len > DG_MAX_BATCH)
    return fail(ctx, DG_EINVAL, "rows must be a multiple of canvas_len, at most 64 canvases");
  if (t < 0) return fail(ctx, DG_EINVAL, "pass %d < 0", t);
  if (rows == 0) return DG_OK;
  if (!noise || !seeds_host) return fail(ctx, DG_EINVAL, "noise and seeds are required");
  dg_config c{};
  c.canvas_len = canvas_len;
  const EbArg eb = eb_arg(c, t, t + 1, seeds_host, rows / canvas_len, block);
  HIPX(launch_eb_noise(rows, vocab, eb, noise, reinterpret_cast<hipStream_t>(stream)));
  return DG_OK;
}

dg_status dg_k_eb_select(int32_t batch, int32_t n, const float* entropy, const int32_t* sample,
                         const int32_t* pred, int32_t* tokens, uint8_t* locked, int32_t* prev_pred,
                         int32_t* status, int32_t t, int32_t t_max, void* stream) {
  dg_ctx* ctx = nullptr;
  if (batch < 0 || batch > DG_MAX_BATCH || n < 1 || n > 4096)
    return fail(ctx, DG_EINVAL, "batch must be in [0, 64] and n in [1, 4096]");
  if (t_max < 1 || t < 0 || t >= t_max) return fail(ctx, DG_EINVAL, "pass %d outside [0, t_max = %d)", t, t_max);
  if (batch == 0) return DG_OK;
  if (!entropy || !sample || !pred || !tokens || !locked || !prev_pred || !status)
    return fail(ctx, DG_EINVAL, "entropy, sample, pred, tokens, locked, prev_pred and status are required");
  HIPX(launch_eb_select(batch, n, entropy, sample, pred, tokens, locked, prev_pred, status, t, t_max,
                        reinterpret_cast<hipStream_t>(stream)));
  return DG_OK;
}

dg_status dg_k_moe_route(const float* logits, int32_t rows, int32_t n_experts, int32_t top_k, int32_t* idx,
                         float* gates, int32_t* counts, int32_t* offsets, int32_t* perm, void* stream) {
  dg_ctx* ctx = nullptr;
  if (!logits || !idx || !gates) return fail(ctx, DG_EINVAL, "logits, idx and gates are required");
  if (rows < 1 || rows > 4096 || n_experts < 1 || n_experts > 256 || top_k < 1 || top_k > 8 ||
      top_k > n_experts)
    return fail(ctx, DG_EINVAL, "rows in [1, 4096], E in [1, 256], k in [1, min(8, E)] required");
  if ((long long)n_experts * ((rows + 31) / 32) > 16384)
    return fail(ctx, DG_EINVAL, "E * ceil(rows / 32) must be <= 16384");
  RouteArgs r{};
  r.mode = ROUTE_LOGITS; r.rows = rows; r.E = n_experts; r.k = top_k;
  r.logits = logits; r.logit_parts = 1;
  r.idx = idx; r.gates = gates;
  r.counts = counts; r.offsets = offsets; r.perm = perm;
  HIPX(launch_route(r, reinterpret_cast<hipStream_t>(stream)));
  return DG_OK;
}

dg_status dg_k_qkv(dg_ctx* ctx, int32_t layer, int32_t batch, const void* a, void* q, void* k, void* v) {
  TRY(enter(ctx));
  const dg_config& c = ctx->c;
  if (layer < 0 || layer >= c.n_layers || !ctx->L[layer].set) return fail(ctx, DG_ESTATE, "layer %d not loaded", layer);
  if (batch < 1 || batch > c.max_batch) return fail(ctx, DG_EINVAL, "batch out of range");
  if (!a || !q || !k || !v) return fail(ctx, DG_EINVAL, "a, q, k, v are required");
  TRY(check_slots(ctx, batch));
  const long long N = c.canvas_len, D = c.head_dim, Hq = c.n_heads, Hkv = c.n_kv_heads;
  const long long qs[4] = {N * Hq * D, D, Hq * D, 1};
  const long long ks[4] = {N * Hkv * D, D, Hkv * D, 1};
  return enqueue_qkv(ctx, layer, batch, a, q, k, v, qs, ks, ks);
}

dg_status dg_k_canvas_attn(dg_ctx* ctx, int32_t layer, int32_t batch, const void* q, const void* k, const void* v,
                           void* o, int32_t canvas_keys) {
  TRY(enter(ctx));
  const dg_config& c = ctx->c;
  if (layer < 0 || layer >= c.n_layers) return fail(ctx, DG_EINVAL, "layer out of range");
  if (batch < 1 || batch > c.max_batch) return fail(ctx, DG_EINVAL, "batch out of range");
  if (!q || !k || !v || !o) return fail(ctx, DG_EINVAL, "q, k, v, o are required");
  TRY(check_slots(ctx, batch));
  const int N = c.canvas_len, D = c.head_dim, Hq = c.n_heads, Hkv = c.n_kv_heads;
  {
    const int n[4] = {batch, Hq, N, D};
    const long long ss[4] = {(long long)N * Hq * D, D, (long long)Hq * D, 1};
    const long long ds[4] = {(long long)Hq * N * D, (long long)N * D, D, 1};
    HIPX(launch_permute4(ctx->bf16, q, ctx->q, n, ss, ds, ctx->st));
  }
  {
    const int n[4] = {batch, Hkv, N, D};
    const long long ss[4] = {(long long)N * Hkv * D, D, (long long)Hkv * D, 1};
    const long long dk[4] = {(long long)Hkv * N * D, (long long)N * D, D, 1};
    const long long dv[4] = {(long long)Hkv * D * N, (long long)D * N, 1, N};
    HIPX(launch_permute4(ctx->bf16, k, ctx->kc, n, ss, dk, ctx->st));
    HIPX(launch_permute4(ctx->bf16, v, ctx->vc, n, ss, dv, ctx->st));
  }
  return enqueue_attention(ctx, layer, batch, o, canvas_keys ? 1 : 0);
}

dg_status dg_k_moe_ffn(dg_ctx* ctx, int32_t layer, int32_t batch, const void* f, const int32_t* idx,
                       const float* gates, float* m) {
  TRY(enter(ctx));
  const dg_config& c = ctx->c;
  if (layer < 0 || layer >= c.n_layers || !ctx->L[layer].set) return fail(ctx, DG_ESTATE, "layer %d not loaded", layer);
  if (batch < 1 || batch > c.max_batch) return fail(ctx, DG_EINVAL, "batch out of range");
  if (!f || !idx || !gates || !m) return fail(ctx, DG_EINVAL, "f, idx, gates, m are required");
  const int M = batch * c.canvas_len, K = c.top_k, H = c.hidden;
  HIPX(hipMemcpyAsync(ctx->idx, idx, (size_t)M * K * 4, hipMemcpyDeviceToDevice, ctx->st));
  HIPX(hipMemcpyAsync(ctx->gates, gates, (size_t)M * K * 4, hipMemcpyDeviceToDevice, ctx->st));
  TRY(enqueue_route(ctx, layer, M, ROUTE_GIVEN));
  TRY(enqueue_experts(ctx, layer, M, f));
  HIPX(hipMemsetAsync(m, 0, (size_t)M * H * 4, ctx->st));
  NormArgs nc{};
  nc.mode = 1; nc.rows = M; nc.H = H; nc.k = K; nc.eps = c.rms_eps;
  nc.x = m; nc.delta = ctx->y; nc.w_delta = nullptr; nc.w_out = nullptr;
  HIPX(launch_residual_norm(ctx->bf16, nc, ctx->st));
  return DG_OK;
}

dg_status dg_k_lm_head(dg_ctx* ctx, int32_t batch, const void* h, float* logits) {
  TRY(enter(ctx));
  const dg_config& c = ctx->c;
  if (!c.has_lm_head || !ctx->embed_set) return fail(ctx, DG_ESTATE, "embedding not loaded");
  if (batch < 1 || batch > c.max_batch) return fail(ctx, DG_EINVAL, "batch out of range");
  if (!h || !logits) return fail(ctx, DG_EINVAL, "h and logits are required");
  const int M = batch * c.canvas_len;
  if (ctx->lm_fused) {
    LmArgs la = lm_args(ctx, h, M);
    la.logits = logits;
    HIPX(launch_lm_head(la, LM_STORE, ctx->st));
    return DG_OK;
  }
  return enqueue_dense(ctx, h, c.hidden, ctx->embed, c.hidden, c.vocab, M, logits, c.vocab, false);
}

dg_status dg_k_lm_argmax(dg_ctx* ctx, int32_t batch, const void* h, int32_t* pred, float* conf) {
  TRY(enter(ctx));
  const dg_config& c = ctx->c;
  if (!c.has_lm_head || !ctx->embed_set) return fail(ctx, DG_ESTATE, "embedding not loaded");
  if (batch < 1 || batch > c.max_batch) return fail(ctx, DG_EINVAL, "batch out of range");
  if (!h || !pred || !conf) return fail(ctx, DG_EINVAL, "h, pred and conf are required");
  return enqueue_head(ctx, h, batch * c.canvas_len, pred, conf);
}

dg_status dg_k_lm_argmax_noalloc(dg_ctx* ctx, int32_t batch, const void* h, int32_t* pred, float* conf) {
  TRY(enter(ctx));
  const dg_config& c = ctx->c;
  if (batch < 1 || batch > c.max_batch) return fail(ctx, DG_EINVAL, "batch out of range");
  if (!c.has_lm_head || !ctx->lm_fused)
    return fail(ctx, DG_EUNSUPPORTED, "the allocation-free LM head needs a bf16 context with the fused LM head");
  const int M = batch * c.canvas_len;
  const long long parts = (long long)((c.vocab / 16 + 15) / 16) * M;
  if (parts > kNoAllocParts)
    return fail(ctx, DG_EINVAL,
                "batch %d: %lld (vocabulary tile, row) partials exceed the static scratch of %lld; at most %lld rows "
                "at this vocabulary",
                batch, parts, kNoAllocParts, kNoAllocParts / ((c.vocab / 16 + 15) / 16));
  if (!ctx->embed_set) return fail(ctx, DG_ESTATE, "embedding not loaded");
  if (!h || !pred || !conf) return fail(ctx, DG_EINVAL, "h, pred and conf are required");
  float* sp = static_cast<float*>(scratch_addr(ctx->dev));
  if (!sp) return fail(ctx, DG_EHIP, "address of the static scratch not found");
  LmArgs la = lm_args(ctx, h, M);
  la.part_m = sp;
  la.part_s = sp + kNoAllocParts;
  la.part_i = reinterpret_cast<int32_t*>(sp + 2 * kNoAllocParts);
  la.pred = pred;
  la.conf = conf;
  HIPX(launch_lm_head(la, LM_ARGMAX, ctx->st));
  return DG_OK;
}

dg_status dg_k_lm_sample(dg_ctx* ctx, int32_t batch, const void* h, int32_t t, int32_t t_max,
                         const uint32_t* seeds_host, uint32_t block, int32_t* pred, float* entropy,
                         int32_t* sample) {
  TRY(enter(ctx));
  const dg_config& c = ctx->c;
  if (!c.has_lm_head || !ctx->embed_set) return fail(ctx, DG_ESTATE, "embedding not loaded");
  if (batch < 1 || batch > c.max_batch) return fail(ctx, DG_EINVAL, "batch out of range");
  if (t_max < 1 || t < 0 || t >= t_max) return fail(ctx, DG_EINVAL, "pass %d outside [0, t_max = %d)", t, t_max);
  if (!h || !pred || !entropy || !sample || !seeds_host)
    return fail(ctx, DG_EINVAL, "h, pred, entropy, sample and seeds are required");
  const EbArg eb = eb_arg(c, t, t_max, seeds_host, batch, block);
  return enqueue_head_eb(ctx, h, batch * c.canvas_len, eb, pred, entropy, sample);
}

dg_status dg_profile(dg_ctx* ctx, int32_t mask) {
  TRY(enter(ctx));
  const bool keep = (mask & DG_PROF_KEEP) != 0;
  mask &= ~DG_PROF_KEEP;
  if (mask & ~DG_PROF_ALL) return fail(ctx, DG_EINVAL, "profile mask 0x%x has unknown bits", mask);
  if (mask && !keep) {
    HIPX(hipStreamSynchronize(ctx->st));  // recorded events are done before reuse
    for (auto& r : ctx->prof_rec) r.clear();
    ctx->ev_used = 0;
    // events for 512 timed launches up front, so timing creates none in a timed loop
    while (ctx->ev_pool.size() < 1024) {
      hipEvent_t e = nullptr;
      HIPX(hipEventCreate(&e));
      ctx->ev_pool.push_back(e);
    }
  }
  ctx->prof = mask;
  return DG_OK;
}

dg_status dg_profile_read(dg_ctx* ctx, int32_t kernel, int32_t* launches, double* total_ms) {
  TRY(enter(ctx));
  if (kernel < 0 || kernel >= DG_PROF_COUNT || !launches || !total_ms)
    return fail(ctx, DG_EINVAL, "bad kernel id or NULL output");
  HIPX(hipStreamSynchronize(ctx->st));
  double tot = 0.0;
  for (const auto& pr : ctx->prof_rec[kernel]) {
    float ms = 0.f;
    HIPX(hipEventElapsedTime(&ms, pr.first, pr.second));
    tot += ms;
  }
  *launches = (int32_t)ctx->prof_rec[kernel].size();
  *total_ms = tot;
  return DG_OK;
}

}  // extern "C"
