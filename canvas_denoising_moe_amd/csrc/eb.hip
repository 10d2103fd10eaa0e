// Entropy-bounded (EB) denoising ([4xFaster] "Recommended Inference Settings":
// EB sampler, at most 48 steps, temperature 0.8 -> 0.4, entropy bound 0.1,
// adaptive stop below a mean entropy of 0.005 once the high-probability tokens
// hold for two consecutive passes; [ParadigmShift] "Serving in Production: The
// Role of vLLM": two consecutive passes in agreement halt the block).
//
// k_eb_rows: the sampler's per-row statistics from stored fp32 logits (the LM
// head of fp32 contexts); bf16 contexts get them from the fused LM head.
// k_eb_select: one workgroup per canvas locks the unlocked positions of lowest
// entropy while their running sum stays within the bound (at least one), each
// with its sample; then applies the stop rule.  The order (entropy, then
// position), the running sum, the mean and both comparisons are float32 in a
// fixed sequence, so equal inputs give equal decisions on any device.
#include "common.h"

namespace {

constexpr float kEntropyBound = 0.1f;
constexpr float kStopEntropy = 0.005f;

// One workgroup per row.  A thread owns whole Philox calls: call c covers ids
// (c >> 4) * 64 + (c & 15) + 16 w, w = 0..3, word w of the output.
__global__ __launch_bounds__(256) void k_eb_rows(const float* __restrict__ logits, int V, EbArg eb,
                                                 int32_t* pred, float* ent, int32_t* samp) {
  __shared__ EbPart red[4];
  const int row = blockIdx.x, tid = threadIdx.x;
  const int cb = row / eb.N, pos = row - cb * eb.N;
  const float* L = logits + (long long)row * V;
  const int ncalls = ((V + 63) >> 6) * 16;
  const float inv = eb.inv_tau;
  // greedy maximum first, so every S and U term is taken against the row's m_z
  float m = -INFINITY;
  int mi = 0x7fffffff;
  for (int c = tid; c < ncalls; c += 256) {
    const int base = (c >> 4) * 64 + (c & 15);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int v = base + 16 * w;
      if (v >= V) break;
      const float l = L[v];
      if (l > m || (l == m && v < mi)) { m = l; mi = v; }
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float om = __shfl_xor(m, o, 64);
    const int oi = __shfl_xor(mi, o, 64);
    if (om > m || (om == m && oi < mi)) { m = om; mi = oi; }
  }
  if ((tid & 63) == 0) red[tid >> 6] = EbPart{m, mi, 0.f, 0.f, 0.f, 0};
  __syncthreads();
  for (int w = 0; w < 4; ++w)
    if (red[w].m > m || (red[w].m == m && red[w].i < mi)) { m = red[w].m; mi = red[w].i; }
  __syncthreads();
  const float mz = m * inv;
  EbPart p{m, mi, 0.f, 0.f, -INFINITY, 0x7fffffff};
  for (int c = tid; c < ncalls; c += 256) {
    const int base = (c >> 4) * 64 + (c & 15);
    const uint4 x = philox4x32_10(make_uint4((uint32_t)c, (uint32_t)pos, eb.t, 0u), eb.seed[cb], eb.block);
    const uint32_t words[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int v = base + 16 * w;
      if (v >= V) break;
      const float l = L[v];
      const float d = l * inv - mz, e = expf(d);
      p.S += e;
      p.U += e * d;
      const float sc = eb_score(l, inv, gumbel_from_bits(words[w]));
      if (sc > p.gs || (sc == p.gs && v < p.gi)) { p.gs = sc; p.gi = v; }
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    EbPart q;
    q.m = p.m; q.i = p.i;  // the same greedy maximum everywhere
    q.S = __shfl_xor(p.S, o, 64);
    q.U = __shfl_xor(p.U, o, 64);
    q.gs = __shfl_xor(p.gs, o, 64);
    q.gi = __shfl_xor(p.gi, o, 64);
    p = eb_merge(p, q, inv);
  }
  if ((tid & 63) == 0) red[tid >> 6] = p;
  __syncthreads();
  if (tid == 0) {
    EbPart r = red[0];
    for (int w = 1; w < 4; ++w) r = eb_merge(r, red[w], inv);
    pred[row] = r.i;
    ent[row] = eb_entropy(r);
    samp[row] = r.gi;
  }
}

// The Gumbel noise itself, [rows, V]: one thread per Philox call.
__global__ __launch_bounds__(256) void k_eb_noise(int V, EbArg eb, float* out) {
  const int row = blockIdx.y, c = blockIdx.x * 256 + threadIdx.x;
  const int ncalls = ((V + 63) >> 6) * 16;
  if (c >= ncalls) return;
  const int cb = row / eb.N, pos = row - cb * eb.N;
  const uint4 x = philox4x32_10(make_uint4((uint32_t)c, (uint32_t)pos, eb.t, 0u), eb.seed[cb], eb.block);
  const uint32_t words[4] = {x.x, x.y, x.z, x.w};
  const int base = (c >> 4) * 64 + (c & 15);
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const int v = base + 16 * w;
    if (v < V) out[(long long)row * V + v] = gumbel_from_bits(words[w]);
  }
}

// One workgroup per canvas.  Canvases marked done are left as they are.
// Locked positions rank as +inf, which no entropy (finite, >= 0) exceeds or
// equals; LDS rows are read four values at a time.  The running sum (thread
// 0) and the mean (a thread of the second wave) are sequential float32 sums
// in the stated orders.
__global__ __launch_bounds__(1024) void k_eb_select(int N, const float* __restrict__ ent,
                                                    const int32_t* __restrict__ samp,
                                                    const int32_t* __restrict__ pred, int32_t* tokens,
                                                    uint8_t* locked, int32_t* prev_pred, int32_t* status,
                                                    int t, int t_max) {
  extern __shared__ float lds[];
  const int N4 = (N + 3) & ~3;
  float* H = lds;              // [N4] entropies by position (0 past N)
  float* Hr = lds + N4;        // [N4] the same, +inf where locked or past N
  float* sorted = lds + 2 * N4;  // [N4] unlocked entropies in lock order
  int* rank = reinterpret_cast<int*>(lds + 3 * N4);  // [N4] lock order, -1 locked
  __shared__ int changed_s, nfree_s, k_s, stop_s;
  const int b = blockIdx.x, tid = threadIdx.x;
  const int st = status[b];
  if (st & 1) {
    if (tid == 0) status[b] = st & ~4;
    return;
  }
  const long long base = (long long)b * N;
  if (tid == 0) { changed_s = 0; nfree_s = 0; }
  __syncthreads();
  int nf = 0, changed = 0;
  for (int i = tid; i < N4; i += blockDim.x) {
    if (i >= N) {
      H[i] = 0.f;
      Hr[i] = INFINITY;
      continue;
    }
    const float h = ent[base + i];
    const bool lk = locked[base + i] != 0;
    H[i] = h;
    Hr[i] = lk ? INFINITY : h;
    nf += lk ? 0 : 1;
    const int pr = pred[base + i];
    changed |= pr != prev_pred[base + i];
    prev_pred[base + i] = pr;
  }
  if (changed) changed_s = 1;
  atomicAdd(&nfree_s, nf);
  __syncthreads();
  // lock order: increasing entropy, then increasing position
  const float4* h4 = reinterpret_cast<const float4*>(Hr);
  for (int i = tid; i < N; i += blockDim.x) {
    const float hi = Hr[i];
    if (hi == INFINITY) { rank[i] = -1; continue; }
    int r = 0;
#pragma unroll 8
    for (int j4 = 0; j4 < (N4 >> 2); ++j4) {
      const float4 v = h4[j4];
      const int j = j4 * 4;
      r += (v.x < hi || (v.x == hi && j < i)) ? 1 : 0;
      r += (v.y < hi || (v.y == hi && j + 1 < i)) ? 1 : 0;
      r += (v.z < hi || (v.z == hi && j + 2 < i)) ? 1 : 0;
      r += (v.w < hi || (v.w == hi && j + 3 < i)) ? 1 : 0;
    }
    rank[i] = r;
    sorted[r] = hi;
  }
  __syncthreads();
  const int mean_tid = blockDim.x > 64 ? 64 : 0;
  if (tid == 0) {
    const int nfree = nfree_s;
    int k = 0;
    if (t >= t_max - 1) {
      k = nfree;
    } else {
      float run = 0.f;
      const float4* s4 = reinterpret_cast<const float4*>(sorted);
      bool done = false;
      for (int r4 = 0; r4 < ((nfree + 3) >> 2) && !done; ++r4) {
        const float4 v = s4[r4];
        const float vals[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int r = r4 * 4 + q;
          if (done || r >= nfree) { done = true; break; }
          run += vals[q];
          if (r > 0 && run > kEntropyBound) { done = true; break; }
          k = r + 1;
        }
      }
    }
    k_s = k;
  }
  if (tid == mean_tid) {
    float sum = 0.f;
    const float4* m4 = reinterpret_cast<const float4*>(H);
    for (int i4 = 0; i4 < (N4 >> 2); ++i4) {  // position order; entries past N are 0
      const float4 v = m4[i4];
      sum += v.x;
      sum += v.y;
      sum += v.z;
      sum += v.w;
    }
    const float mean = sum / (float)N;
    stop_s = ((st & 2) && !changed_s && mean < kStopEntropy) ? 1 : 0;
  }
  __syncthreads();
  const int k = k_s, stop = stop_s;
  for (int i = tid; i < N; i += blockDim.x) {
    const int r = rank[i];
    if (r < 0) continue;
    if (r < k) {
      tokens[base + i] = samp[base + i];
      locked[base + i] = 1;
    } else if (stop) {
      tokens[base + i] = pred[base + i];
      locked[base + i] = 1;
    }
  }
  if (tid == 0) status[b] = 2 | (stop ? 4 : 0) | ((stop || k == nfree_s) ? 1 : 0);
}

}  // namespace

hipError_t launch_eb_rows(const float* logits, int rows, int V, const EbArg& eb, int32_t* pred, float* ent,
                          int32_t* samp, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if (V <= 0 || eb.N <= 0 || rows % eb.N != 0 || rows / eb.N > 64) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_eb_rows, dim3(rows), dim3(256), 0, s, logits, V, eb, pred, ent, samp);
  return hipGetLastError();
}

hipError_t launch_eb_noise(int rows, int V, const EbArg& eb, float* out, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if (V <= 0 || eb.N <= 0 || rows % eb.N != 0 || rows / eb.N > 64) return hipErrorInvalidValue;
  const int ncalls = ((V + 63) >> 6) * 16;
  hipLaunchKernelGGL(k_eb_noise, dim3((ncalls + 255) / 256, rows), dim3(256), 0, s, V, eb, out);
  return hipGetLastError();
}

hipError_t launch_eb_select(int B, int N, const float* ent, const int32_t* samp, const int32_t* pred,
                            int32_t* tokens, uint8_t* locked, int32_t* prev_pred, int32_t* status, int t,
                            int t_max, hipStream_t s) {
  if (B <= 0) return hipSuccess;
  if (N <= 0 || N > 4096) return hipErrorInvalidValue;
  const size_t lds = (size_t)((N + 3) & ~3) * 16;
  hipError_t err = ensure_lds_limit(reinterpret_cast<const void*>(&k_eb_select), 4096 * 16);
  if (err != hipSuccess) return err;
  const int threads = N >= 1024 ? 1024 : ((N + 63) / 64) * 64;
  hipLaunchKernelGGL(k_eb_select, dim3(B), dim3(threads), lds, s, N, ent, samp, pred, tokens, locked, prev_pred,
                     status, t, t_max);
  return hipGetLastError();
}
