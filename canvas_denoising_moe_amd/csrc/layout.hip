// Layout changes: prompt KV into head-major K and transposed V, and a generic
// strided 4-d copy used by the single-kernel entry points.
#include "common.h"

namespace {

// src [L][Hkv][D] -> K [Hkv][L][D] (transpose = 0) or V^T [Hkv][D][L] (transpose = 1)
template <typename T>
__global__ void k_kv_repack(const T* __restrict__ src, int L, int Hkv, int D, T* __restrict__ dst,
                            int transpose) {
  const long long total = (long long)L * Hkv * D;
  for (long long i = blockIdx.x * (long long)blockDim.x + threadIdx.x; i < total;
       i += (long long)gridDim.x * blockDim.x) {
    // i enumerates the destination
    long long l, h, d;
    if (!transpose) {
      d = i % D; l = (i / D) % L; h = i / ((long long)D * L);
    } else {
      l = i % L; d = (i / L) % D; h = i / ((long long)D * L);
    }
    dst[i] = src[(l * Hkv + h) * D + d];
  }
}

template <typename T>
__global__ void k_permute4(const T* __restrict__ src, T* __restrict__ dst, int n0, int n1, int n2, int n3,
                           long long s0, long long s1, long long s2, long long s3, long long d0,
                           long long d1, long long d2, long long d3) {
  const long long total = (long long)n0 * n1 * n2 * n3;
  for (long long i = blockIdx.x * (long long)blockDim.x + threadIdx.x; i < total;
       i += (long long)gridDim.x * blockDim.x) {
    const long long i3 = i % n3, i2 = (i / n3) % n2, i1 = (i / ((long long)n3 * n2)) % n1,
                    i0 = i / ((long long)n3 * n2 * n1);
    dst[i0 * d0 + i1 * d1 + i2 * d2 + i3 * d3] = src[i0 * s0 + i1 * s1 + i2 * s2 + i3 * s3];
  }
}

unsigned grid_for(long long total) {
  const long long b = (total + 255) / 256;
  return (unsigned)(b < 65536 ? (b > 0 ? b : 1) : 65536);
}

}  // namespace

hipError_t launch_kv_repack(int is_bf16, const void* src, int L, int Hkv, int D, void* dst, int transpose,
                            hipStream_t s) {
  const long long total = (long long)L * Hkv * D;
  if (total <= 0) return hipSuccess;
  if (is_bf16)
    hipLaunchKernelGGL(k_kv_repack<bf16_t>, dim3(grid_for(total)), dim3(256), 0, s,
                       reinterpret_cast<const bf16_t*>(src), L, Hkv, D, reinterpret_cast<bf16_t*>(dst),
                       transpose);
  else
    hipLaunchKernelGGL(k_kv_repack<float>, dim3(grid_for(total)), dim3(256), 0, s,
                       reinterpret_cast<const float*>(src), L, Hkv, D, reinterpret_cast<float*>(dst),
                       transpose);
  return hipGetLastError();
}

hipError_t launch_permute4(int is_bf16, const void* src, void* dst, const int* n, const long long* ss,
                           const long long* ds, hipStream_t s) {
  const long long total = (long long)n[0] * n[1] * n[2] * n[3];
  if (total <= 0) return hipSuccess;
  if (is_bf16)
    hipLaunchKernelGGL(k_permute4<bf16_t>, dim3(grid_for(total)), dim3(256), 0, s,
                       reinterpret_cast<const bf16_t*>(src), reinterpret_cast<bf16_t*>(dst), n[0], n[1],
                       n[2], n[3], ss[0], ss[1], ss[2], ss[3], ds[0], ds[1], ds[2], ds[3]);
  else
    hipLaunchKernelGGL(k_permute4<float>, dim3(grid_for(total)), dim3(256), 0, s,
                       reinterpret_cast<const float*>(src), reinterpret_cast<float*>(dst), n[0], n[1],
                       n[2], n[3], ss[0], ss[1], ss[2], ss[3], ds[0], ds[1], ds[2], ds[3]);
  return hipGetLastError();
}
