// Shared device helpers and launcher declarations of the gfx950 kernels.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>
#include <set>
#include <utility>

typedef uint16_t bf16_t;  // raw bf16 bits
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_v __attribute__((ext_vector_type(8)));

#define DG_DEV __device__ __forceinline__

DG_DEV float bf2f(bf16_t h) { return __uint_as_float(((uint32_t)h) << 16); }

// float -> bf16, round to nearest even (the hardware conversion)
DG_DEV bf16_t f2bf(float f) { return __builtin_bit_cast(bf16_t, (__bf16)f); }
// two floats -> packed bf16 pair (lo in bits 0..15), one conversion instruction
typedef __bf16 bf16x2_v __attribute__((ext_vector_type(2)));
typedef float floatx2_v __attribute__((ext_vector_type(2)));
DG_DEV uint32_t f2bf2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((floatx2_v){lo, hi}, bf16x2_v));
}

template <typename T> DG_DEV float to_f(T v);
template <> DG_DEV float to_f<float>(float v) { return v; }
template <> DG_DEV float to_f<bf16_t>(bf16_t v) { return bf2f(v); }

template <typename T> DG_DEV T from_f(float v);
template <> DG_DEV float from_f<float>(float v) { return v; }
template <> DG_DEV bf16_t from_f<bf16_t>(float v) { return f2bf(v); }

// Separation between the last MFMA of a loop and the first read of its
// accumulators: nothing is scheduled across the barrier and 16 wait states
// follow, more than the result latency of any 16x16 MFMA used here.
DG_DEV void mfma_drain() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_nop 7\n\ts_nop 7" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// wave64 reductions
DG_DEV float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
DG_DEV float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// Block-wide sum in a fixed order (deterministic).  `red` holds >= nwaves floats.
DG_DEV float block_sum(float v, float* red) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = (blockDim.x + 63) >> 6;
  v = wave_sum(v);
  __syncthreads();
  if (lane == 0) red[w] = v;
  __syncthreads();
  float s = 0.f;
  for (int i = 0; i < nw; ++i) s += red[i];
  return s;
}

// ----------------------------------------------------------------------------
// launchers (implemented in the .hip files); all return hipError_t
// ----------------------------------------------------------------------------

// Optional timing of one launcher call: `start` takes the start time of its
// first kernel and `stop` the end time of its last one.  The events are bound
// to the kernel dispatches themselves, so timing adds no packets to the stream.
struct KTime { hipEvent_t start = nullptr, stop = nullptr; };

// Raises a kernel's dynamic LDS limit to `bytes` on the current device, once
// per (kernel, device): the attribute belongs to the kernel's code object on
// each device, so a process driving two GPUs sets it on both.
inline hipError_t ensure_lds_limit(const void* fn, int bytes) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  static std::mutex mu;
  static std::set<std::pair<const void*, int>> done;
  std::lock_guard<std::mutex> lock(mu);
  if (done.count({fn, dev})) return hipSuccess;
  e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess) done.insert({fn, dev});
  return e;
}

template <typename F, typename... Args>
inline hipError_t launch_k(F kernel, dim3 grid, dim3 block, size_t lds, hipStream_t s,
                           hipEvent_t ev0, hipEvent_t ev1, Args... args) {
  if (ev0 || ev1)
    hipExtLaunchKernelGGL(kernel, grid, block, (uint32_t)lds, s, ev0, ev1, 0u, args...);
  else
    hipLaunchKernelGGL(kernel, grid, block, lds, s, args...);
  return hipGetLastError();
}

// Weight repack into matrix-core fragment order:
//   dst[((nb*KB + kb)*64 + lane)*8 + j] = W(k = kb*32 + (lane/16)*8 + j,
//                                           n = colmap(nb)*16 + lane%16)
// W(k, n) = src[k*ld + n] when src_kn, else src[n*ld + k].  colmap: 0 = identity,
// 1 = q/k/v rotary pairing (see gemm.hip), 2 = gate/up interleave with the
// second source in src2.
struct PackArgs {
  const void* src; const void* src2; long long ld; int K, N; int src_kn; int colmap;
  int head_dim, n_rope_heads;  // colmap 1
  void* dst;
};
hipError_t launch_pack(int is_bf16, const PackArgs& a, hipStream_t s);
// nbatch matrices: source i at src (and src2) + i*src_bs, destination at dst + i*dst_bs
hipError_t launch_pack_batched(int is_bf16, const PackArgs& a, int nbatch, long long src_bs,
                               long long dst_bs, hipStream_t s);

// MXFP4 (OCP microscaling, 4-bit E2M1 elements, one E8M0 scale per 32
// consecutive k of a column) from packed bf16 fragments [NB][KB][64][8]
// (batch stride src_bs elements).  With KG = ceil(KB / 4):
//   codes  uint32 [batch][NB][KG][64 lanes][4]: word j of a lane holds the 8
//          codes of k-step 4 kg + j in the lane's fragment order, element e in
//          bits 4e..4e+3 (so one 16-byte load feeds four k-steps);
//   scales uint8  [batch][NB][KG][16 columns][4]: byte j = s + 127 of k-step
//          4 kg + j of that column.
// k-steps past KB hold zero codes and scale 2^0.
hipError_t launch_quant_mxfp4(const void* packed, int nbatch, long long src_bs, int NB, int KB, uint4* codes,
                              uint8_t* scales, hipStream_t s);
// The weights a packed expert operand stands for, back in math layout
// [K, N] (T): packed bf16/fp32 fragments (codes == NULL) or MXFP4 codes and
// scales decoded with the streaming GEMM's own conversion (codes_out [K, N]
// and scales_out [K/32, N] receive the raw codes and scale bytes).  colmap 2:
// the gate|up interleave, half selects up (1) or gate (0) and N is F.  Any
// output may be NULL.
hipError_t launch_unpack_weight(int is_bf16, const void* packed, const uint4* codes, const uint8_t* scales, int K,
                                int N, int colmap, int half, void* out, uint8_t* codes_out, uint8_t* scales_out,
                                hipStream_t s);

// Generic skinny GEMM on matrix cores; see gemm.hip for the arguments.
struct GemmArgs {
  const void* A; long long lda;
  const int32_t* a_rows;         // logical row -> A row, NULL = identity
  int a_rows_max;                // rows of A (gathered indices are clamped into range)
  const void* B; long long b_group_stride;  // elements between groups' packed matrices
  int K, NB;                     // K % 32 == 0; NB = N / 16
  int static_row0, static_rows, static_group;  // rows handled by a fixed m-chunk grid
  const int32_t* group_off; int n_groups;      // data-dependent groups 0..n_groups-1
};
enum EpiKind { EPI_STORE_F32 = 0, EPI_GEGLU = 1, EPI_DOWN = 2, EPI_QKV = 3 };
struct EpiArgs {
  int kind;
  void* out; long long ldo;            // STORE_F32 (float), GEGLU (T)
  const int32_t* slot; const float* gates; int routed_rows; int out_rows;  // DOWN
  // QKV: output tensors with strides (elements) over (b, head, i, d)
  void* q; void* k; void* v;
  long long qs[4], ks[4], vs[4];
  const float2* rope_cs;               // [batch][N][D/2] (cos, sin)
  int N, D, Hq, Hkv, n_rot_local, n_rot_global, is_global;
};
hipError_t launch_gemm(int is_bf16, const GemmArgs& g, const EpiArgs& e, int mt, hipStream_t s,
                       KTime t = {});

// Streaming GEMM over work entries of <= 16*mt rows (see gemm.hip).  Dense
// entries cover rows [dense_row0, dense_row0 + dense_rows) of group dense_group
// in steps of 16*mt (n_dense of them); work entries {group, first row, end row,
// -} come from the router, built for the same entry size.
struct StreamArgs {
  const void* A; long long lda;
  const int32_t* a_rows; int a_rows_max;
  const void* B; long long b_group_stride;
  int K, NB;
  int mt;  // row tiles of 16 per entry: 1 or 2
  int n_dense, dense_row0, dense_rows, dense_group;
  const int4* work; const int32_t* work_count; int work_cap;
  // expert-major order of the work list (router output): group e's entries are
  // [ent_off[e], ent_off[e+1]), e < n_groups; NULL: tile-major (tile, entry)
  const int32_t* ent_off; int n_groups;
  // split-K (fp32-store epilogue only): K/32 % ksplit == 0; split s writes its
  // partial sums at out + s * split_stride
  int ksplit; long long split_stride;
  // qb = 1: B in MXFP4 (bf16 contexts): codes Bq and scales Bs in the layout
  // of launch_quant_mxfp4, group strides in uint4 / uint32 units
  int qb;
  const uint4* Bq; long long bq_group_stride;
  const uint32_t* Bs; long long bs_group_stride;
};
hipError_t launch_stream(int is_bf16, const StreamArgs& g, const EpiArgs& e, hipStream_t s,
                         KTime t = {});

// Attention.
#define DG_MAX_BATCH 64
struct AttnArgs {
  const void* q;          // [B][Hq][N][D]
  const void* kc;         // canvas K [B][Hkv][N][D]
  const void* vc;         // canvas V^T [B][Hkv][D][N]
  int B, N, Hq, Hkv, D, canvas_keys;
  int causal;             // canvas key j is visible to canvas query i only when j <= i
  void* o;                // [B*N][Hq*D]
  float* part_o; float* part_m; float* part_l;  // split partials
  long long part_cap_rows;  // capacity of the partial buffers in (split, row) pairs
  const void* kp[DG_MAX_BATCH];  // per canvas: prompt K [Hkv][Lw][D]
  const void* vp[DG_MAX_BATCH];  // per canvas: prompt V^T [Hkv][D][Lw]
  int lw[DG_MAX_BATCH];          // per canvas: prompt keys visible to the layer
  // key splits, set by launch_attention from each canvas's own key count (so a
  // canvas's result never depends on the other canvases of the batch)
  int ns[DG_MAX_BATCH];          // per canvas: splits
  int cl[DG_MAX_BATCH];          // per canvas: keys per split (multiple of 64)
  int ubase[DG_MAX_BATCH + 1];   // per canvas: first work unit (unit = KV head x split)
};
hipError_t launch_attention(int is_bf16, const AttnArgs& a, hipStream_t s, KTime t = {});

// Routing, combine, norms.
// MoE routing (route.hip).  ROUTE_LOGITS: top-k + gates of the router logits
// (sum of logit_parts split-K partials); ROUTE_GIVEN: idx/gates are inputs.  Both
// then build counts/offsets/perm/a_rows/work.  E * ceil(rows/32) <= 16384.
enum RouteMode { ROUTE_LOGITS = 1, ROUTE_GIVEN = 2 };
constexpr int kRouteMaxLds = 16384 * 8;  // bitmap + prefix counts of the scatter workgroup
struct RouteArgs {
  int mode;
  int rows, E, k;
  const float* logits; int logit_parts; long long part_stride;
  float* r_out;
  int32_t* idx; float* gates;
  int32_t* counts; int32_t* offsets; int32_t* perm; int32_t* a_rows;
  int4* work; int32_t* work_count;
  int32_t* ent_off;  // [E + 2]: first work entry of every expert, the shared expert, the end
  int entry_rows;  // rows per work entry (16 * the expert GEMMs' mt)
  int with_shared;
};
hipError_t launch_route(const RouteArgs& a, hipStream_t s);

// x[t] += delta_norm(sum of terms) ; out[t] = T(RMSNorm(x[t]) * (1 + w_out))
// mode 0: terms = delta[t] (one row); mode 1: terms = y[t*k + s] for s < k, then y[rows*k + t];
// mode 2: no delta (only the output norm); w_delta NULL: plain add.
struct NormArgs {
  int mode; int rows, H, k; float eps;
  float* x; const float* delta; const void* w_delta; const void* w_out; void* out;
};
hipError_t launch_residual_norm(int is_bf16, const NormArgs& a, hipStream_t s);
// Embedding gather; ids outside [0, V) read as zero rows and, at positions
// t % N < valid_n, are recorded in *bad (NULL: not recorded), see moe.hip.
hipError_t launch_embed(int is_bf16, const int32_t* tokens, int rows, int H, int V, int N, int valid_n,
                        const void* packed_embed, float* x, uint64_t* bad, hipStream_t s);
hipError_t launch_rope_table(float2* cs, int N, int D, int prompt_len, double theta, hipStream_t s);

// ----------------------------------------------------------------------------
// Entropy-bounded sampling: counter-based noise and per-row statistics
// ----------------------------------------------------------------------------

// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as easy
// as 1, 2, 3", SC 2011): ten rounds of two 32x32 -> 64-bit products with a
// Weyl sequence of round keys.
DG_DEV uint4 philox4x32_10(uint4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t p0 = (uint64_t)0xD2511F53u * c.x, p1 = (uint64_t)0xCD9E8D57u * c.z;
    const uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
    const uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
    c = make_uint4(hi1 ^ c.y ^ k0, lo1, hi0 ^ c.w ^ k1, lo0);
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return c;
}

// Gumbel noise from a 32-bit word: u = (2n + 1) 2^-24 from the top 23 bits
// (exact, strictly inside (0, 1)), g = -log(-log u), written with the
// hardware base-2 logarithm: -log(-log u) = -ln2 log2(-log2 u) - log(ln 2).
// Both arguments are normal floats (-log2 u lies in [8.6e-8, 24]).
DG_DEV float gumbel_from_bits(uint32_t w) {
  const float u = (float)(((w >> 9) << 1) | 1u) * 0x1p-24f;
  const float e2 = -__builtin_amdgcn_logf(u);
  return fmaf(-0.693147180559945309f, __builtin_amdgcn_logf(e2), 0.366512920581664327f);
}

// Sampling score l * (1/tau) + g with the product and the sum rounded apart,
// so the sampled id is the same wherever the same float logit is scored.
DG_DEV float eb_score(float l, float inv_tau, float g) {
#pragma clang fp contract(off)
  const float z = l * inv_tau;
  return z + g;
}

// Per-pass sampler parameters: canvas b of a row is row / N, its position row
// % N; its noise key is (seed[b], block) and the counter's third word the pass.
struct EbArg {
  float inv_tau;
  uint32_t t, block;
  int32_t N;
  uint32_t seed[64];
};

// Per-row statistics of softmax(l / tau) over a vocabulary range: greedy max m
// and its id, S = sum exp(z - m z_), U = sum exp(z - m_z) (z - m_z) with z =
// l / tau and m_z = m / tau, and the best sampling score with its id.
struct EbPart { float m; int i; float S, U, gs; int gi; };

// Merge of two vocabulary ranges; equal maxima and scores keep the lower id.
DG_DEV EbPart eb_merge(EbPart a, EbPart b, float inv_tau) {
  EbPart r;
  if (a.m > b.m || (a.m == b.m && a.i < b.i)) { r.m = a.m; r.i = a.i; } else { r.m = b.m; r.i = b.i; }
  if (a.gs > b.gs || (a.gs == b.gs && a.gi < b.gi)) { r.gs = a.gs; r.gi = a.gi; } else { r.gs = b.gs; r.gi = b.gi; }
  const float mz = r.m * inv_tau;
  float S = 0.f, U = 0.f;
  if (a.S > 0.f) {
    const float d = a.m * inv_tau - mz, f = expf(d);
    S += a.S * f;
    U += (a.U + d * a.S) * f;
  }
  if (b.S > 0.f) {
    const float d = b.m * inv_tau - mz, f = expf(d);
    S += b.S * f;
    U += (b.U + d * b.S) * f;
  }
  r.S = S;
  r.U = U;
  return r;
}

// Entropy (nats) of the merged statistics, log S - U / S, never below 0.
DG_DEV float eb_entropy(const EbPart& p) { return fmaxf(logf(p.S) - p.U / p.S, 0.f); }

// Tied LM head for bf16 contexts (lmhead.hip): h bf16 [M, K] @ E^T with E packed
// as the B operand ([V/16][K/32][64][8]).  Store mode writes logits fp32 [M, V];
// argmax mode writes pred/conf [M] through per-(vocabulary tile, row) partials
// part_* [(V/256 rounded up) * M]; sampler mode writes pred, the entropy ent
// and the sample samp [M] through the partials part_m/s/i and part_u/g/gi.
// Needs K % 128 == 0, M % 16 == 0 and V % 16 == 0.
enum LmMode { LM_STORE = 0, LM_ARGMAX = 1, LM_SAMPLE = 2 };
struct LmArgs {
  const void* h; int M, K, V;
  const void* E;
  float* logits;
  float* part_m; float* part_s; int32_t* part_i;
  float* part_u; float* part_g; int32_t* part_gi;
  int32_t* pred; float* conf;
  float* ent; int32_t* samp;
  EbArg eb;
};
bool lm_head_supported(int M, int K, int V);
hipError_t launch_lm_head(const LmArgs& a, int mode, hipStream_t s, KTime t = {});

// Sampler statistics of fp32 logits [rows, V] (eb.hip): pred, ent, samp [rows].
hipError_t launch_eb_rows(const float* logits, int rows, int V, const EbArg& eb, int32_t* pred, float* ent,
                          int32_t* samp, hipStream_t s);
// The Gumbel noise of rows [rows, V] as the sampler draws it (eb.hip).
hipError_t launch_eb_noise(int rows, int V, const EbArg& eb, float* out, hipStream_t s);
// The entropy-bounded lock step of B canvases of N positions (eb.hip).
// status[b]: bit 0 done, bit 1 a previous pass's greedy tokens are in
// prev_pred, bit 2 this pass stopped the canvas.
hipError_t launch_eb_select(int B, int N, const float* ent, const int32_t* samp, const int32_t* pred,
                            int32_t* tokens, uint8_t* locked, int32_t* prev_pred, int32_t* status, int t,
                            int t_max, hipStream_t s);

// Head: argmax / confidence and the lock step.
hipError_t launch_argmax_conf(const float* logits, int rows, int V, int32_t* pred, float* conf,
                              hipStream_t s);
struct StepsArg { int32_t v[64]; };
hipError_t launch_lock_select(int B, int N, const float* conf, const int32_t* pred, int32_t* tokens,
                              uint8_t* locked, StepsArg steps, hipStream_t s);

// Layout helpers.
hipError_t launch_kv_repack(int is_bf16, const void* src, int L, int Hkv, int D, void* k_dst,
                            int transpose, hipStream_t s);
// K [Hkv][new_len][D] / V^T [Hkv][D][new_len] of one layer after appending the
// first n of a block's N positions (k [Hkv][N][D], v^T [Hkv][D][N]) to the old
// cache; positions are absolute, the new range a suffix of [old ; block
// positions < n] (layout.hip)
hipError_t launch_kv_append(int is_bf16, const void* kold, const void* vold, int old_len, long long old_first,
                            const void* kblk, const void* vblk, int N, int n, long long blk_first, int new_len,
                            long long first, int Hkv, int D, void* knew, void* vnew, hipStream_t s);
// generic 4-d permute copy: dst[(i0,i1,i2,i3) strides ds] = src[(i0,i1,i2,i3) strides ss]
hipError_t launch_permute4(int is_bf16, const void* src, void* dst, const int* dims,
                           const long long* ss, const long long* ds, hipStream_t s);
