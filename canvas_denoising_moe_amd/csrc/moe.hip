// Router top-k with the token -> expert scatter, the residual / RMSNorm
// kernels (the norm sandwich of [HandsOn] "Detailed Specs", fused with the
// residual adds and the MoE combine), the embedding gather and the RoPE table.
#include "common.h"

namespace {

// One workgroup routes every token: top-k of E logits per token (logit
// descending, ties to the lower expert index), softmax over the kept logits,
// then a deterministic counting sort of the (token, slot) pairs by expert with
// tokens ascending inside an expert.  Membership bits per (expert, token) are
// set with atomicOr (order-independent), so counts, offsets and ranks do not
// depend on thread timing.
__global__ __launch_bounds__(1024) void k_moe_route(const float* __restrict__ logits, int rows, int E,
                                                    int k, int32_t* idx, float* gates, int32_t* counts,
                                                    int32_t* offsets, int32_t* perm, int32_t* a_rows) {
  extern __shared__ uint32_t sm[];
  const int W = (rows + 31) >> 5;
  uint32_t* bm = sm;                                 // [E][W]
  int* offs = reinterpret_cast<int*>(sm + E * W);    // [E + 2]
  const int tid = threadIdx.x, nt = blockDim.x;
  for (int i = tid; i < E * W; i += nt) bm[i] = 0u;
  __syncthreads();

  for (int t = tid; t < rows; t += nt) {
    if (!logits) {  // routing given: only the scatter
      for (int s = 0; s < k; ++s) {
        int e = idx[(long long)t * k + s];
        e = e < 0 ? 0 : (e >= E ? E - 1 : e);  // out-of-range ids must not leave LDS
        atomicOr(&bm[e * W + (t >> 5)], 1u << (t & 31));
      }
      continue;
    }
    const float* r = logits + (long long)t * E;
    float bv[8];
    int be[8];
#pragma unroll
    for (int s = 0; s < 8; ++s) { bv[s] = -INFINITY; be[s] = -1; }
    for (int e = 0; e < E; ++e) {
      const float v = r[e];
      // first slot that v beats (an empty slot, or a strictly smaller logit);
      // equal logits keep the earlier (lower) expert in front
      int p = k;
#pragma unroll
      for (int s = 7; s >= 0; --s)
        if (s < k && (be[s] < 0 || bv[s] < v)) p = s;
      if (p < k) {
#pragma unroll
        for (int s = 7; s > 0; --s)
          if (s < k && s > p) { bv[s] = bv[s - 1]; be[s] = be[s - 1]; }
#pragma unroll
        for (int s = 0; s < 8; ++s)
          if (s == p) { bv[s] = v; be[s] = e; }
      }
    }
    float ex[8], sum = 0.f;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      ex[s] = s < k ? expf(bv[s] - bv[0]) : 0.f;
      sum += ex[s];
    }
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      if (s < k) {
        idx[(long long)t * k + s] = be[s];
        gates[(long long)t * k + s] = ex[s] / sum;
        atomicOr(&bm[be[s] * W + (t >> 5)], 1u << (t & 31));
      }
    }
  }
  __threadfence_block();
  __syncthreads();
  if (tid < E) {
    int c = 0;
    for (int w = 0; w < W; ++w) c += __popc(bm[tid * W + w]);
    offs[tid] = c;
    if (counts) counts[tid] = c;
  }
  __syncthreads();
  if (tid == 0) {
    int acc = 0;
    for (int e = 0; e < E; ++e) {
      const int c = offs[e];
      offs[e] = acc;
      acc += c;
    }
    offs[E] = acc;  // == rows * k
    offs[E + 1] = acc + rows;
  }
  __syncthreads();
  if (offsets)
    for (int e = tid; e < E + 2; e += nt) offsets[e] = offs[e];
  for (int p = tid; p < rows * k; p += nt) {
    const int t = p / k;
    int e = idx[p];
    e = e < 0 ? 0 : (e >= E ? E - 1 : e);
    const uint32_t* row = bm + e * W;
    const int wt = t >> 5;
    int rank = __popc(row[wt] & ((1u << (t & 31)) - 1u));
    for (int w = 0; w < wt; ++w) rank += __popc(row[w]);
    const int pos = offs[e] + rank;
    if (perm) perm[pos] = p;
    if (a_rows) a_rows[pos] = t;
  }
  if (a_rows && perm) {
    const int base = rows * k;
    for (int t = tid; t < rows; t += nt) {
      perm[base + t] = base + t;
      a_rows[base + t] = t;
    }
  }
}

// x[t] += RMSNorm(delta_t) * (1 + w_delta)   (plain add without w_delta)
// out[t] = T(RMSNorm(x[t]) * (1 + w_out))      (skipped without w_out)
// delta_t: mode 0 one row of `delta`; mode 1 the MoE combine
//   sum_{s<k} y[t*k + s] (slot order) + y[rows*k + t]; mode 2 nothing.
template <typename T>
__global__ __launch_bounds__(256) void k_residual_norm(NormArgs a) {
  extern __shared__ float buf[];  // [H]
  __shared__ float red[8];
  const int t = blockIdx.x, tid = threadIdx.x, H = a.H;
  float* x = a.x + (long long)t * H;
  if (a.mode != 2) {
    float ss = 0.f;
    for (int c = tid; c < H; c += blockDim.x) {
      float d;
      if (a.mode == 0) {
        d = a.delta[(long long)t * H + c];
      } else {
        d = 0.f;
        for (int s = 0; s < a.k; ++s) d += a.delta[((long long)t * a.k + s) * H + c];
        d += a.delta[((long long)a.rows * a.k + t) * H + c];
      }
      buf[c] = d;
      ss += d * d;
    }
    if (a.w_delta) {
      const float tot = block_sum(ss, red);
      const float sc = rsqrtf(tot / H + a.eps);
      const T* w = reinterpret_cast<const T*>(a.w_delta);
      for (int c = tid; c < H; c += blockDim.x) x[c] += buf[c] * sc * (1.0f + to_f<T>(w[c]));
    } else {
      for (int c = tid; c < H; c += blockDim.x) x[c] += buf[c];
    }
    __syncthreads();
  }
  if (a.w_out) {
    float ss = 0.f;
    for (int c = tid; c < H; c += blockDim.x) {
      const float v = x[c];
      ss += v * v;
    }
    const float tot = block_sum(ss, red + 4);
    const float sc = rsqrtf(tot / H + a.eps);
    const T* w = reinterpret_cast<const T*>(a.w_out);
    T* out = reinterpret_cast<T*>(a.out) + (long long)t * H;
    for (int c = tid; c < H; c += blockDim.x) out[c] = from_f<T>(x[c] * sc * (1.0f + to_f<T>(w[c])));
  }
}

// x[t, h] = E[token_t, h] read from the fragment-packed embedding
// ([V/16][H/32][64][8]); ids outside [0, V) read as zero rows.
template <typename T>
__global__ void k_embed(const int32_t* __restrict__ tokens, int rows, int H, int V,
                        const T* __restrict__ pe, float* __restrict__ x) {
  const long long total = (long long)rows * H;
  const int KB = H >> 5;
  for (long long i = blockIdx.x * (long long)blockDim.x + threadIdx.x; i < total;
       i += (long long)gridDim.x * blockDim.x) {
    const int t = (int)(i / H), h = (int)(i - (long long)t * H);
    const int v = tokens[t];
    float val = 0.f;
    if (v >= 0 && v < V) {
      const long long o = (((long long)(v >> 4) * KB + (h >> 5)) * 64 + (v & 15) + 16 * ((h & 31) >> 3)) * 8 + (h & 7);
      val = to_f<T>(pe[o]);
    }
    x[i] = val;
  }
}

// cos / sin of pos * theta^(-2j/D) for canvas position i at pos = prompt_len + i,
// evaluated in double so long prompts keep full angle accuracy.
__global__ void k_rope_table(float2* cs, int N, int D, int prompt_len, double theta) {
  const int half = D >> 1;
  const int total = N * half;
  for (int t = blockIdx.x * blockDim.x + threadIdx.x; t < total; t += gridDim.x * blockDim.x) {
    const int i = t / half, j = t - i * half;
    const double inv = pow(theta, -2.0 * j / (double)D);
    const double ang = (double)(prompt_len + i) * inv;
    cs[t] = make_float2((float)cos(ang), (float)sin(ang));
  }
}

}  // namespace

hipError_t launch_moe_route(const float* logits, int rows, int E, int k, int32_t* idx, float* gates,
                            int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* a_rows,
                            hipStream_t s) {
  const int W = (rows + 31) / 32;
  const size_t lds = (size_t)E * W * 4 + (size_t)(E + 2) * 4;
  hipLaunchKernelGGL(k_moe_route, dim3(1), dim3(1024), lds, s, logits, rows, E, k, idx, gates, counts,
                     offsets, perm, a_rows);
  return hipGetLastError();
}

hipError_t launch_residual_norm(int is_bf16, const NormArgs& a, hipStream_t s) {
  if (a.rows <= 0) return hipSuccess;
  const size_t lds = (size_t)a.H * 4;
  if (is_bf16)
    hipLaunchKernelGGL(k_residual_norm<bf16_t>, dim3(a.rows), dim3(256), lds, s, a);
  else
    hipLaunchKernelGGL(k_residual_norm<float>, dim3(a.rows), dim3(256), lds, s, a);
  return hipGetLastError();
}

hipError_t launch_embed(int is_bf16, const int32_t* tokens, int rows, int H, int V, const void* pe,
                        float* x, hipStream_t s) {
  const long long total = (long long)rows * H;
  if (total <= 0) return hipSuccess;
  const unsigned blocks = (unsigned)((total + 255) / 256 < 65536 ? (total + 255) / 256 : 65536);
  if (is_bf16)
    hipLaunchKernelGGL(k_embed<bf16_t>, dim3(blocks), dim3(256), 0, s, tokens, rows, H, V,
                       reinterpret_cast<const bf16_t*>(pe), x);
  else
    hipLaunchKernelGGL(k_embed<float>, dim3(blocks), dim3(256), 0, s, tokens, rows, H, V,
                       reinterpret_cast<const float*>(pe), x);
  return hipGetLastError();
}

hipError_t launch_rope_table(float2* cs, int N, int D, int prompt_len, double theta, hipStream_t s) {
  const int total = N * (D / 2);
  if (total <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_rope_table, dim3((total + 255) / 256), dim3(256), 0, s, cs, N, D, prompt_len, theta);
  return hipGetLastError();
}
