// MoE routing of a decoder layer (one launch):
//
//   1. top-k of the router logits per token (logit descending, ties to the
//      lower expert) and gates = softmax over the kept logits
//      ([4xFaster] "DiffusionGemma's Technical Architecture": 8 of 128 experts
//      active); the logits may arrive as split-K partial sums, added here in a
//      fixed order;
//   2. token -> expert scatter: per-expert counts and offsets, the rows of
//      every expert in ascending token order, and the work list of <= 16-row
//      entries the streaming expert GEMMs consume.
//
// Step 1 runs one wave per token, four tokens per workgroup.  Expert
// membership is accumulated as bits (expert, token) with device-scope
// atomicOr, which is order-independent; the last workgroup to finish (a
// device-scope ticket) turns the bitmap into counts, offsets, ranks and the
// work list, then clears the bitmap and the ticket for the next launch, so
// the result never depends on scheduling and no host-side reset is needed.
#include "common.h"

namespace {

constexpr int kRowsPerBlock = 4;

DG_DEV void argmax_pair(float& v, int& e) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float ov = __shfl_xor(v, o, 64);
    const int oe = __shfl_xor(e, o, 64);
    if (ov > v || (ov == v && oe < e)) { v = ov; e = oe; }
  }
}

__global__ __launch_bounds__(256) void k_route(RouteArgs a) {
  __shared__ float rs[kRowsPerBlock * 256];
  __shared__ int s_last;
  const int E = a.E, K = a.k;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int t = blockIdx.x * kRowsPerBlock + wave;
  const bool row_ok = t < a.rows;
  const int W = (a.rows + 31) >> 5;

  if (a.mode == ROUTE_LOGITS) {
    const int parts = a.logit_parts > 0 ? a.logit_parts : 1;
    for (int u = tid; u < kRowsPerBlock * E; u += 256) {
      const int r = u / E, e = u % E;
      const int tt = blockIdx.x * kRowsPerBlock + r;
      float s = 0.f;
      if (tt < a.rows)
        for (int q = 0; q < parts; ++q) s += a.logits[q * a.part_stride + (long long)tt * E + e];
      rs[r * E + e] = s;
      if (a.r_out && tt < a.rows) a.r_out[(long long)tt * E + e] = s;
    }
    __syncthreads();
  }

  // ---- 1. top-k and gates, one wave per token
  if (row_ok) {
    if (a.mode == ROUTE_LOGITS) {
      const float* rr = rs + wave * E;
      float sel_v[8];
      int sel_e[8];
      unsigned used = 0u;  // bit j: expert lane + 64 j taken
      for (int s = 0; s < K; ++s) {
        float v = -INFINITY;
        int be = 0x7fffffff;
        for (int j = 0; j * 64 + lane < E; ++j) {
          if (used & (1u << j)) continue;
          const int e = j * 64 + lane;
          const float x = rr[e];
          if (be == 0x7fffffff || x > v || (x == v && e < be)) { v = x; be = e; }
        }
        argmax_pair(v, be);
        if ((be & 63) == lane) used |= 1u << (be >> 6);
#pragma unroll
        for (int q = 0; q < 8; ++q)
          if (q == s) { sel_v[q] = v; sel_e[q] = be; }
      }
      if (lane == 0) {
        float ex[8], sum = 0.f;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          ex[q] = q < K ? expf(sel_v[q] - sel_v[0]) : 0.f;
          sum += ex[q];
        }
#pragma unroll
        for (int q = 0; q < 8; ++q)
          if (q < K) {
            a.idx[(long long)t * K + q] = sel_e[q];
            a.gates[(long long)t * K + q] = ex[q] / sum;
          }
      }
      // every lane holds sel_e; lanes < K set the membership bits
      if (lane < K) {
        int e = 0;
#pragma unroll
        for (int q = 0; q < 8; ++q)
          if (q == lane) e = sel_e[q];
        atomicOr(&a.bm[e * W + (t >> 5)], 1u << (t & 31));
      }
    } else if (lane < K) {
      int e = a.idx[(long long)t * K + lane];
      e = e < 0 ? 0 : (e >= E ? E - 1 : e);  // out-of-range ids must not leave the bitmap
      atomicOr(&a.bm[e * W + (t >> 5)], 1u << (t & 31));
    }
  }

  // ---- 2. the last workgroup builds the scatter
  __threadfence();
  __syncthreads();
  if (tid == 0) s_last = atomicAdd(a.done, 1) == (int)gridDim.x - 1;
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  __shared__ int s_cnt[256], s_off[258], s_ent[256];
  __shared__ int s_total;
  for (int e = tid; e < E; e += 256) {
    int c = 0;
    for (int w = 0; w < W; ++w) c += __popc(a.bm[e * W + w]);
    s_cnt[e] = c;
    if (a.counts) a.counts[e] = c;
  }
  __syncthreads();
  const int RK = a.rows * K;
  const int n_shared = a.with_shared ? (a.rows + 15) / 16 : 0;
  if (tid == 0) {
    int off = 0, ne = 0;
    for (int e = 0; e < E; ++e) {
      s_off[e] = off;
      s_ent[e] = ne;
      off += s_cnt[e];
      ne += (s_cnt[e] + 15) >> 4;
    }
    s_off[E] = off;               // == rows * k
    s_off[E + 1] = off + a.rows;  // the shared expert's rows follow the routed ones
    s_total = ne + n_shared;
    if (a.work_count) *a.work_count = s_total;
  }
  __syncthreads();
  if (a.offsets)
    for (int e = tid; e < E + 2; e += 256) a.offsets[e] = s_off[e];
  if (a.work) {
    for (int e = tid; e < E; e += 256) {
      const int c = s_cnt[e], base = s_off[e];
      for (int q = 0; q * 16 < c; ++q)
        a.work[s_ent[e] + q] = make_int4(e, base + q * 16, base + min(c, q * 16 + 16), 0);
    }
    const int ne = s_total - n_shared;
    for (int q = tid; q < n_shared; q += 256)
      a.work[ne + q] = make_int4(E, RK + q * 16, RK + min(a.rows, q * 16 + 16), 0);
  }
  for (int p = tid; p < RK; p += 256) {
    const int tt = p / K;
    int e = a.idx[p];
    e = e < 0 ? 0 : (e >= E ? E - 1 : e);
    const uint32_t* row = a.bm + e * W;
    const int wt = tt >> 5;
    int rank = __popc(row[wt] & ((1u << (tt & 31)) - 1u));
    for (int w = 0; w < wt; ++w) rank += __popc(row[w]);
    const int pos = s_off[e] + rank;
    if (a.perm) a.perm[pos] = p;
    if (a.a_rows) a.a_rows[pos] = tt;
  }
  if (a.with_shared) {
    for (int tt = tid; tt < a.rows; tt += 256) {
      if (a.perm) a.perm[RK + tt] = RK + tt;
      if (a.a_rows) a.a_rows[RK + tt] = tt;
    }
  }
  __syncthreads();
  for (int i = tid; i < E * W; i += 256) a.bm[i] = 0u;
  if (tid == 0) *a.done = 0;
}

}  // namespace

hipError_t launch_route(const RouteArgs& a, hipStream_t s) {
  if (a.rows <= 0) return hipSuccess;
  if (a.E > 256 || a.k > 8 || (a.mode != ROUTE_LOGITS && a.mode != ROUTE_GIVEN)) return hipErrorInvalidValue;
  const int blocks = (a.rows + kRowsPerBlock - 1) / kRowsPerBlock;
  hipLaunchKernelGGL(k_route, dim3(blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}
