// Per-position prediction and confidence over the vocabulary, and the
// lock-and-remask step that ends a pass.
//
// Confidence is the softmax probability of the argmax token, 1 / sum_v
// exp(l_v - l_max) ([HandsOn] "Detailed Specs": the probability distribution
// judges whether tokens are final).  Each canvas then locks the
// ceil(remaining / steps_left) most confident unlocked positions (ties to the
// lower position): they take their prediction and stay fixed as context; the
// rest keep their placeholder ([4xFaster] "What is Diffusion...";
// [ParadigmShift] "Analysis of Implications").
#include "common.h"

namespace {

struct MaxState { float m; int i; float s; };

// merge two (max, argmax, sum exp(l - max)) states; equal maxima keep the lower index
DG_DEV MaxState merge(MaxState a, MaxState b) {
  MaxState r;
  if (a.m > b.m || (a.m == b.m && a.i < b.i)) { r.m = a.m; r.i = a.i; } else { r.m = b.m; r.i = b.i; }
  const float sa = a.s > 0.f ? a.s * expf(a.m - r.m) : 0.f;
  const float sb = b.s > 0.f ? b.s * expf(b.m - r.m) : 0.f;
  r.s = sa + sb;
  return r;
}

// One workgroup per row; coalesced float4 reads; each thread keeps an online
// (max, argmax, sum) over its columns (ascending), then a fixed-order tree merge.
__global__ __launch_bounds__(256) void k_argmax_conf(const float* __restrict__ logits, int V,
                                                     int32_t* pred, float* conf) {
  __shared__ MaxState red[4];
  const long long row = blockIdx.x;
  const float4* r4 = reinterpret_cast<const float4*>(logits + row * V);
  const int tid = threadIdx.x;
  MaxState st{-INFINITY, 0x7fffffff, 0.f};
  const int n4 = V >> 2, nt = blockDim.x;
  constexpr int U = 8;  // loads in flight per thread
  for (int base = tid; base < n4; base += nt * U) {
    float4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c4 = base + u * nt;
      v[u] = c4 < n4 ? r4[c4] : make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
    }
    // columns are visited in increasing order, so a later equal maximum never replaces
    // an earlier one
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c4 = base + u * nt;
      if (c4 >= n4) break;
      const float vals[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float x = vals[j];
        if (x > st.m) {
          st.s = (st.s > 0.f ? st.s * expf(st.m - x) : 0.f) + 1.0f;
          st.m = x;
          st.i = c4 * 4 + j;
        } else {
          st.s += expf(x - st.m);
        }
      }
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    MaxState ot;
    ot.m = __shfl_xor(st.m, o, 64);
    ot.i = __shfl_xor(st.i, o, 64);
    ot.s = __shfl_xor(st.s, o, 64);
    st = merge(st, ot);
  }
  if ((tid & 63) == 0) red[tid >> 6] = st;
  __syncthreads();
  if (tid == 0) {
    MaxState r = red[0];
    for (int w = 1; w < (int)(blockDim.x >> 6); ++w) r = merge(r, red[w]);
    pred[row] = r.i;
    conf[row] = 1.0f / r.s;
  }
}

// One workgroup per canvas.  rank_i = #{unlocked j : conf_j > conf_i or
// (conf_j == conf_i and j < i)}; position i is selected iff rank_i < k.
// Locked positions enter the comparison as -inf, which no confidence (in
// (0, 1]) falls below or equals; the LDS row is read four values at a time.
__global__ __launch_bounds__(1024) void k_lock_select(int N, const float* __restrict__ conf,
                                                      const int32_t* __restrict__ pred, int32_t* tokens,
                                                      uint8_t* locked, StepsArg steps) {
  extern __shared__ float cs[];  // [N rounded up to 4] conf, -inf where locked
  __shared__ int rem_s;
  const int b = blockIdx.x, tid = threadIdx.x;
  const long long base = (long long)b * N;
  const int N4 = (N + 3) & ~3;
  if (tid == 0) rem_s = 0;
  __syncthreads();
  int rem = 0;
  for (int i = tid; i < N4; i += blockDim.x) {
    const bool lk = i >= N || locked[base + i];
    cs[i] = lk ? -INFINITY : conf[base + i];
    rem += lk ? 0 : 1;
  }
  atomicAdd(&rem_s, rem);
  __syncthreads();
  const int sl = steps.v[b];
  const int kk = (rem_s + sl - 1) / sl;
  const float4* c4 = reinterpret_cast<const float4*>(cs);
  for (int i = tid; i < N; i += blockDim.x) {
    const float ci = cs[i];
    if (ci == -INFINITY) continue;
    int rank = 0;
#pragma unroll 8
    for (int j4 = 0; j4 < (N4 >> 2); ++j4) {
      const float4 v = c4[j4];
      const int j = j4 * 4;
      rank += (v.x > ci || (v.x == ci && j < i)) ? 1 : 0;
      rank += (v.y > ci || (v.y == ci && j + 1 < i)) ? 1 : 0;
      rank += (v.z > ci || (v.z == ci && j + 2 < i)) ? 1 : 0;
      rank += (v.w > ci || (v.w == ci && j + 3 < i)) ? 1 : 0;
    }
    if (rank < kk) {
      tokens[base + i] = pred[base + i];
      locked[base + i] = 1;
    }
  }
}

}  // namespace

hipError_t launch_argmax_conf(const float* logits, int rows, int V, int32_t* pred, float* conf,
                              hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_argmax_conf, dim3(rows), dim3(256), 0, s, logits, V, pred, conf);
  return hipGetLastError();
}

hipError_t launch_lock_select(int B, int N, const float* conf, const int32_t* pred, int32_t* tokens,
                              uint8_t* locked, StepsArg steps, hipStream_t s) {
  if (B <= 0) return hipSuccess;
  const size_t lds = (size_t)((N + 3) & ~3) * 4;
  const int threads = N >= 1024 ? 1024 : ((N + 63) / 64) * 64;
  hipLaunchKernelGGL(k_lock_select, dim3(B), dim3(threads), lds, s, N, conf, pred, tokens, locked, steps);
  return hipGetLastError();
}
