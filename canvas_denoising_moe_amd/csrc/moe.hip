// The residual / RMSNorm
// kernels (the norm sandwich of [HandsOn] "Detailed Specs", fused with the
// residual adds and the MoE combine), the embedding gather and the RoPE table.
#include "common.h"

namespace {

template <typename T> DG_DEV float4 load4(const T* p);
template <> DG_DEV float4 load4<float>(const float* p) { return *reinterpret_cast<const float4*>(p); }
template <> DG_DEV float4 load4<bf16_t>(const bf16_t* p) {
  const uint2 q = *reinterpret_cast<const uint2*>(p);
  return make_float4(__uint_as_float(q.x << 16), __uint_as_float(q.x & 0xffff0000u),
                     __uint_as_float(q.y << 16), __uint_as_float(q.y & 0xffff0000u));
}
template <typename T> DG_DEV void store4(T* p, float4 v);
template <> DG_DEV void store4<float>(float* p, float4 v) { *reinterpret_cast<float4*>(p) = v; }
template <> DG_DEV void store4<bf16_t>(bf16_t* p, float4 v) {
  *reinterpret_cast<uint2*>(p) = make_uint2((uint32_t)f2bf(v.x) | ((uint32_t)f2bf(v.y) << 16),
                                            (uint32_t)f2bf(v.z) | ((uint32_t)f2bf(v.w) << 16));
}
DG_DEV float4 f4add(float4 a, float4 b) { return make_float4(a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w); }
DG_DEV float f4dot(float4 a) { return a.x * a.x + a.y * a.y + a.z * a.z + a.w * a.w; }

// x[t] += RMSNorm(delta_t) * (1 + w_delta)   (plain add without w_delta)
// out[t] = T(RMSNorm(x[t]) * (1 + w_out))      (skipped without w_out)
// delta_t: mode 0 one row of `delta`; mode 1 the MoE combine
//   sum_{s<k} y[t*k + s] (slot order) + y[rows*k + t]; mode 2 nothing.
// One workgroup of NT threads per token; thread i owns float4 columns i,
// i + NT, ... (NV of them, H <= 4 * NT * NV).  Every term of the row (up to k + 1 MoE outputs) is
// loaded before any arithmetic, so a token's whole working set is in flight at
// once; sums of squares are fixed-order block reductions.
template <typename T, int NV, int NT>
__global__ __launch_bounds__(NT) void k_residual_norm(NormArgs a) {
  __shared__ float red[32];
  const int t = blockIdx.x, tid = threadIdx.x;
  const int H = a.H, n4 = H >> 2;
  float4* x4 = reinterpret_cast<float4*>(a.x + (long long)t * H);
  const float4 z4 = make_float4(0.f, 0.f, 0.f, 0.f);
  float4 xv[NV], gd[NV], go[NV];
  const T* wd = reinterpret_cast<const T*>(a.w_delta);
  const T* wo = reinterpret_cast<const T*>(a.w_out);
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int c4 = tid + NT * i;
    xv[i] = c4 < n4 ? x4[c4] : z4;
    // the norm weights too, so no load waits behind a reduction
    gd[i] = (wd && a.mode != 2 && c4 < n4) ? load4<T>(wd + 4 * c4) : z4;
    go[i] = (wo && c4 < n4) ? load4<T>(wo + 4 * c4) : z4;
  }
  if (a.mode != 2) {
    const float4* d4 = reinterpret_cast<const float4*>(a.delta);
    float4 dv[NV];
    if (a.mode == 0) {
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        const int c4 = tid + NT * i;
        dv[i] = c4 < n4 ? d4[(long long)t * n4 + c4] : z4;
      }
    } else {
      // routed terms y[t*k + s] (slot order), then the shared expert's y[rows*k + t]
      float4 tv[8][NV], sv[NV];
#pragma unroll
      for (int s = 0; s < 8; ++s)
#pragma unroll
        for (int i = 0; i < NV; ++i) {
          const int c4 = tid + NT * i;
          tv[s][i] = (s < a.k && c4 < n4) ? d4[((long long)t * a.k + s) * n4 + c4] : z4;
        }
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        const int c4 = tid + NT * i;
        sv[i] = c4 < n4 ? d4[((long long)a.rows * a.k + t) * n4 + c4] : z4;
      }
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        float4 d = z4;
#pragma unroll
        for (int s = 0; s < 8; ++s)
          if (s < a.k) d = f4add(d, tv[s][i]);
        dv[i] = f4add(d, sv[i]);
      }
    }
    float sc = 1.0f;
    if (wd) {
      float ss = 0.f;
#pragma unroll
      for (int i = 0; i < NV; ++i) ss += f4dot(dv[i]);
      sc = rsqrtf(block_sum(ss, red) / H + a.eps);
    }
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int c4 = tid + NT * i;
      if (c4 < n4) {
        float4 d = dv[i];
        if (wd) {
          const float4 g = gd[i];
          d = make_float4(d.x * sc * (1.f + g.x), d.y * sc * (1.f + g.y), d.z * sc * (1.f + g.z),
                          d.w * sc * (1.f + g.w));
        }
        xv[i] = f4add(xv[i], d);
        x4[c4] = xv[i];
      }
    }
  }
  if (wo) {
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < NV; ++i) ss += f4dot(xv[i]);  // columns past H hold zeros
    const float sc = rsqrtf(block_sum(ss, red + 16) / H + a.eps);
    T* out = reinterpret_cast<T*>(a.out) + (long long)t * H;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int c4 = tid + NT * i;
      if (c4 < n4) {
        const float4 g = go[i];
        const float4 v = xv[i];
        store4<T>(out + 4 * c4, make_float4(v.x * sc * (1.f + g.x), v.y * sc * (1.f + g.y),
                                            v.z * sc * (1.f + g.z), v.w * sc * (1.f + g.w)));
      }
    }
  }
}

template <typename T>
hipError_t run_residual_norm(const NormArgs& a, hipStream_t s) {
  const int n4 = a.H >> 2;
  if (n4 <= 256)
    hipLaunchKernelGGL((k_residual_norm<T, 1, 256>), dim3(a.rows), dim3(256), 0, s, a);
  else if (n4 <= 512)
    hipLaunchKernelGGL((k_residual_norm<T, 1, 512>), dim3(a.rows), dim3(512), 0, s, a);
  else
    hipLaunchKernelGGL((k_residual_norm<T, 2, 512>), dim3(a.rows), dim3(512), 0, s, a);
  return hipGetLastError();
}

// x[t, h] = E[token_t, h] read from the fragment-packed embedding
// ([V/16][H/32][64][8]).  An id outside [0, V) reads as a zero row; when its
// position i = t % N lies below valid_n, the row and the id are recorded in
// *bad as ((t + 1) << 32) | id (one 64-bit store per row, by the thread of
// column 0: any recorded pair is a complete one).
template <typename T>
__global__ void k_embed(const int32_t* __restrict__ tokens, int rows, int H, int V, int N, int valid_n,
                        const T* __restrict__ pe, float* __restrict__ x, uint64_t* bad) {
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
    } else if (h == 0 && bad && (t % N) < valid_n) {
      *bad = ((uint64_t)(uint32_t)(t + 1) << 32) | (uint32_t)v;
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

hipError_t launch_residual_norm(int is_bf16, const NormArgs& a, hipStream_t s) {
  if (a.rows <= 0) return hipSuccess;
  if (a.H > 4096 || (a.H & 3) || a.k > 8) return hipErrorInvalidValue;
  return is_bf16 ? run_residual_norm<bf16_t>(a, s) : run_residual_norm<float>(a, s);
}

hipError_t launch_embed(int is_bf16, const int32_t* tokens, int rows, int H, int V, int N, int valid_n,
                        const void* pe, float* x, uint64_t* bad, hipStream_t s) {
  const long long total = (long long)rows * H;
  if (total <= 0) return hipSuccess;
  if (N <= 0) return hipErrorInvalidValue;
  const unsigned blocks = (unsigned)((total + 255) / 256 < 65536 ? (total + 255) / 256 : 65536);
  if (is_bf16)
    hipLaunchKernelGGL(k_embed<bf16_t>, dim3(blocks), dim3(256), 0, s, tokens, rows, H, V, N, valid_n,
                       reinterpret_cast<const bf16_t*>(pe), x, bad);
  else
    hipLaunchKernelGGL(k_embed<float>, dim3(blocks), dim3(256), 0, s, tokens, rows, H, V, N, valid_n,
                       reinterpret_cast<const float*>(pe), x, bad);
  return hipGetLastError();
}

hipError_t launch_rope_table(float2* cs, int N, int D, int prompt_len, double theta, hipStream_t s) {
  const int total = N * (D / 2);
  if (total <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_rope_table, dim3((total + 255) / 256), dim3(256), 0, s, cs, N, D, prompt_len, theta);
  return hipGetLastError();
}
