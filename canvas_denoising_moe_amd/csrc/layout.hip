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

// Cache of one layer after the first n positions of a block are appended: the
// new visible range is the last new_len positions of [old visible ; block
// positions 0..n-1].  K is [Hkv][len][D] and V^T [Hkv][D][len]; the block's k
// is [Hkv][N][D] and its v^T [Hkv][D][N] (one canvas of the canvas buffers).  Destination
// position p holds absolute position first + p with first = total - new_len;
// positions below the block's start come from the old cache, whose first
// visible position is old_first.
template <typename T>
__global__ void k_kv_append(const T* __restrict__ kold, const T* __restrict__ vold, int old_len, int old_first,
                            const T* __restrict__ kblk, const T* __restrict__ vblk, int N, int blk_first,
                            int new_len, int first, int Hkv, int D, T* __restrict__ knew, T* __restrict__ vnew) {
  const int total = new_len * Hkv * D;  // < 2^31 (checked by the launcher)
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < total; i += gridDim.x * blockDim.x) {
    {  // K: i = (h * new_len + p) * D + d
      const int d = i % D, hp = i / D;
      const int p = hp % new_len, h = hp / new_len;
      const int a = first + p;
      knew[i] = a >= blk_first ? kblk[(h * N + (a - blk_first)) * D + d]
                               : kold[(h * old_len + (a - old_first)) * D + d];
    }
    {  // V^T: i = (h * D + d) * new_len + p
      const int p = i % new_len, hd = i / new_len;
      const int a = first + p;
      vnew[i] = a >= blk_first ? vblk[hd * N + (a - blk_first)] : vold[hd * old_len + (a - old_first)];
    }
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

hipError_t launch_kv_append(int is_bf16, const void* kold, const void* vold, int old_len, long long old_first,
                            const void* kblk, const void* vblk, int N, int n, long long blk_first, int new_len,
                            long long first, int Hkv, int D, void* knew, void* vnew, hipStream_t s) {
  const long long total = (long long)new_len * Hkv * D;
  if (total <= 0) return hipSuccess;
  if (n < 1 || n > N || first < old_first || blk_first + n != first + new_len || old_first + old_len != blk_first ||
      total >= (1LL << 31) || blk_first + N >= (1LL << 31))
    return hipErrorInvalidValue;  // the new range must be a suffix of [old ; first n of the block]
  if (is_bf16)
    hipLaunchKernelGGL(k_kv_append<bf16_t>, dim3(grid_for(total)), dim3(256), 0, s,
                       reinterpret_cast<const bf16_t*>(kold), reinterpret_cast<const bf16_t*>(vold), old_len,
                       (int)old_first, reinterpret_cast<const bf16_t*>(kblk), reinterpret_cast<const bf16_t*>(vblk),
                       N, (int)blk_first, new_len, (int)first, Hkv, D, reinterpret_cast<bf16_t*>(knew),
                       reinterpret_cast<bf16_t*>(vnew));
  else
    hipLaunchKernelGGL(k_kv_append<float>, dim3(grid_for(total)), dim3(256), 0, s,
                       reinterpret_cast<const float*>(kold), reinterpret_cast<const float*>(vold), old_len,
                       (int)old_first, reinterpret_cast<const float*>(kblk), reinterpret_cast<const float*>(vblk),
                       N, (int)blk_first, new_len, (int)first, Hkv, D, reinterpret_cast<float*>(knew),
                       reinterpret_cast<float*>(vnew));
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
