// MoE routing of a decoder layer (two launches):
//
//   k_route_topk: top-k of the router logits per token (logit descending, ties
//     to the lower expert) and gates = softmax over the kept logits
//     ([4xFaster] "DiffusionGemma's Technical Architecture": 8 of 128 experts
//     active); the logits may arrive as split-K partial sums, added here in a
//     fixed order.  One wave per token.
//   k_route_scatter: one workgroup builds the (expert, token) membership bitmap
//     in LDS from the chosen ids, then per-expert counts and offsets, the rows
//     of every expert in ascending token order, and the work list of <= 16-row
//     entries the streaming expert GEMMs consume.
//
// The result never depends on scheduling: bits are set with order-independent
// LDS atomics, and ranks are popcounts of the bitmap.  (Routing every token of
// a canvas inside the one scatter workgroup was tried and is far slower: the
// per-token load latencies then run in sequence.)
#include "common.h"

namespace {


// Order-preserving key of a logit: a larger logit has a larger key.  NaN
// counts as -inf and -0 as +0, so equal keys are exactly equal logits; key 0
// is below every logit's key.
DG_DEV unsigned logit_key(float v) {
  unsigned u = v != v ? __float_as_uint(-INFINITY) : __float_as_uint(v);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
DG_DEV float key_logit(unsigned k) { return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k); }

// Maximum of v over the wave, on every lane: an inclusive max-scan within
// rows of 16 lanes (DPP row shifts), then across rows (row broadcasts of
// lanes 15 and 31); lane 63 ends with the whole wave's maximum.
DG_DEV unsigned wave_max_key(unsigned v) {
  v = max(v, (unsigned)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xf, 0xf, false));  // row_shr:1
  v = max(v, (unsigned)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xf, 0xf, false));  // row_shr:2
  v = max(v, (unsigned)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xf, 0xf, false));  // row_shr:4
  v = max(v, (unsigned)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xf, 0xf, false));  // row_shr:8
  v = max(v, (unsigned)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xa, 0xf, false));  // row_bcast:15
  v = max(v, (unsigned)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xc, 0xf, false));  // row_bcast:31
  return (unsigned)__builtin_amdgcn_readlane((int)v, 63);
}

// Top-k of token t by one wave: lane l holds the logits of experts l, l + 64,
// ... in registers (split-K partials summed in slice order).  Round s takes
// the largest key not yet taken (one wave max) and, among the experts holding
// it, the lowest index (ballots), so the slots are in logit-descending order
// with ties to the lower expert.  Lane s < k returns slot s's expert (and
// writes idx / gates), other lanes return -1.
DG_DEV int topk_token(const RouteArgs& a, int t, int lane) {
  const int E = a.E, K = a.k;
  const int parts = a.logit_parts > 0 ? a.logit_parts : 1;
  unsigned key[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = lane + 64 * j;
    float pv[8];
#pragma unroll
    for (int q = 0; q < 8; ++q)  // all partial loads in flight together
      pv[q] = (e < E && q < parts) ? a.logits[q * a.part_stride + (long long)t * E + e] : 0.f;
    float sum = 0.f;
#pragma unroll
    for (int q = 0; q < 8; ++q)
      if (q < parts) sum += pv[q];  // fixed order
    key[j] = e < E ? logit_key(sum) : 0u;
    if (a.r_out && e < E) a.r_out[(long long)t * E + e] = sum;
  }
  float sel_v[8];
  int sel_e[8];
  unsigned used = 0u;  // bit j: expert lane + 64 j taken
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    if (s >= K) break;
    unsigned cand = 0u;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (lane + 64 * j < E && !(used & (1u << j))) cand = max(cand, key[j]);
    const unsigned m = wave_max_key(cand);
    int pick = 0;
    bool found = false;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const unsigned long long b = __ballot(lane + 64 * j < E && !(used & (1u << j)) && key[j] == m);
      if (!found && b) { pick = 64 * j + __builtin_ctzll(b); found = true; }
    }
    if ((pick & 63) == lane) used |= 1u << (pick >> 6);
    sel_v[s] = key_logit(m);
    sel_e[s] = pick;
  }
  int my_e = -1;
  if (lane < K) {
    float sum = 0.f, mine = 0.f;
#pragma unroll
    for (int q = 0; q < 8; ++q)
      if (q < K) {
        const float x = expf(sel_v[q] - sel_v[0]);
        sum += x;
        if (q == lane) { mine = x; my_e = sel_e[q]; }
      }
    a.idx[(long long)t * K + lane] = my_e;
    a.gates[(long long)t * K + lane] = mine / sum;
  }
  return my_e;
}

__global__ __launch_bounds__(64) void k_route_topk(RouteArgs a) {
  topk_token(a, blockIdx.x, threadIdx.x);
}

// The scatter once the membership bitmap bm [E][W] is complete in LDS: counts,
// offsets and entries per expert, then every routed row's position.  ids(p)
// returns the expert of entry p = t * k + s.
template <typename Ids>
DG_DEV void scatter_rows(const RouteArgs& a, uint32_t* bm, int* pre, int* s_cnt, int* s_off, int* s_ent,
                         int* s_total, Ids ids) {
  const int E = a.E, K = a.k;
  const int tid = threadIdx.x, nt = blockDim.x;
  const int W = (a.rows + 31) >> 5;
  const int RK = a.rows * K;
  for (int e = tid; e < E; e += nt) {
    int c = 0;
    for (int w = 0; w < W; ++w) {
      pre[e * W + w] = c;
      c += __popc(bm[e * W + w]);
    }
    s_cnt[e] = c;
    if (a.counts) a.counts[e] = c;
  }
  __syncthreads();
  const int ER = a.entry_rows > 0 ? a.entry_rows : 16;
  const int n_shared = a.with_shared ? (a.rows + ER - 1) / ER : 0;
  if (tid < 64) {
    // exclusive prefix sums of the row counts and entry counts over experts:
    // lane l owns experts 4l..4l+3, then a wave-wide scan of the lane totals
    int c[4], n[4], cs = 0, ns = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = 4 * tid + i;
      c[i] = e < E ? s_cnt[e] : 0;
      n[i] = (c[i] + ER - 1) / ER;
      cs += c[i];
      ns += n[i];
    }
    int ci = cs, ni = ns;  // inclusive scans
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int cu = __shfl_up(ci, o, 64), nu = __shfl_up(ni, o, 64);
      if (tid >= o) { ci += cu; ni += nu; }
    }
    int off = ci - cs, ne = ni - ns;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = 4 * tid + i;
      if (e < E) {
        s_off[e] = off;
        s_ent[e] = ne;
        if (a.ent_off) a.ent_off[e] = ne;
      }
      off += c[i];
      ne += n[i];
    }
    if (tid == 63) {
      if (a.ent_off) {
        a.ent_off[E] = ne;                 // the shared expert's entries follow
        a.ent_off[E + 1] = ne + n_shared;  // end
      }
      // the shared expert's rows follow the routed ones at rows * k (== off when
      // every row's ids are distinct; repeated ids leave [off, rows * k) unused)
      s_off[E] = RK;
      s_off[E + 1] = RK + a.rows;
      *s_total = ne + n_shared;
      if (a.work_count) *a.work_count = ne + n_shared;
    }
  }
  __syncthreads();
  if (a.offsets)
    for (int e = tid; e < E + 2; e += nt) a.offsets[e] = s_off[e];
  if (a.work) {
    for (int e = tid; e < E; e += nt) {
      const int c = s_cnt[e], base = s_off[e];
      for (int q = 0; q * ER < c; ++q)
        a.work[s_ent[e] + q] = make_int4(e, base + q * ER, base + min(c, q * ER + ER), 0);
    }
    const int ne = *s_total - n_shared;
    for (int q = tid; q < n_shared; q += nt)
      a.work[ne + q] = make_int4(E, RK + q * ER, RK + min(a.rows, q * ER + ER), 0);
  }
  for (int p0 = tid; p0 < RK; p0 += nt * 8) {
    int ev[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {  // expert ids of 8 entries in flight together
      const int p = p0 + u * nt;
      ev[u] = p < RK ? ids(p) : 0;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int p = p0 + u * nt;
      if (p < RK) {
        const int e = ev[u] < 0 ? 0 : (ev[u] >= E ? E - 1 : ev[u]);
        const int tt = p / K, wt = tt >> 5;
        const int rank = pre[e * W + wt] + __popc(bm[e * W + wt] & ((1u << (tt & 31)) - 1u));
        const int pos = s_off[e] + rank;
        if (a.perm) a.perm[pos] = p;
        if (a.a_rows) a.a_rows[pos] = tt;
      }
    }
  }
  if (a.with_shared) {
    for (int tt = tid; tt < a.rows; tt += nt) {
      if (a.perm) a.perm[RK + tt] = RK + tt;
      if (a.a_rows) a.a_rows[RK + tt] = tt;
    }
  }
}

// Scatter of routing already in idx (given ids, or a preceding top-k launch).
__global__ __launch_bounds__(1024) void k_route_scatter(RouteArgs a) {
  extern __shared__ uint32_t dyn[];  // bitmap [E][W] words, then per-word prefix counts [E][W]
  __shared__ int s_cnt[256], s_off[258], s_ent[256];
  __shared__ int s_total;
  const int E = a.E, K = a.k;
  const int tid = threadIdx.x, nt = blockDim.x;
  const int W = (a.rows + 31) >> 5, EW = E * W;
  uint32_t* bm = dyn;
  int* pre = reinterpret_cast<int*>(dyn + EW);
  const int RK = a.rows * K;
  for (int i = tid; i < EW; i += nt) bm[i] = 0u;
  __syncthreads();
  for (int p0 = tid; p0 < RK; p0 += nt * 8) {
    int ev[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int p = p0 + u * nt;
      ev[u] = p < RK ? a.idx[p] : 0;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int p = p0 + u * nt;
      if (p < RK) {
        const int e = ev[u] < 0 ? 0 : (ev[u] >= E ? E - 1 : ev[u]);  // ids stay inside the bitmap
        const int tt = p / K;
        atomicOr(&bm[e * W + (tt >> 5)], 1u << (tt & 31));
      }
    }
  }
  __syncthreads();
  scatter_rows(a, bm, pre, s_cnt, s_off, s_ent, &s_total, [&](int p) { return a.idx[p]; });
}

}  // namespace

hipError_t launch_route(const RouteArgs& a, hipStream_t s) {
  if (a.rows <= 0) return hipSuccess;
  if (a.E > 256 || a.k > 8 || (a.mode != ROUTE_LOGITS && a.mode != ROUTE_GIVEN)) return hipErrorInvalidValue;
  const size_t lds = (size_t)a.E * ((a.rows + 31) / 32) * 8;  // bitmap + prefix counts
  if (lds > kRouteMaxLds) return hipErrorInvalidValue;
  hipError_t err = ensure_lds_limit(reinterpret_cast<const void*>(&k_route_scatter), kRouteMaxLds);
  if (err != hipSuccess) return err;
  if (a.mode == ROUTE_LOGITS) {
    hipLaunchKernelGGL(k_route_topk, dim3(a.rows), dim3(64), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(k_route_scatter, dim3(1), dim3(1024), lds, s, a);
  return hipGetLastError();
}
