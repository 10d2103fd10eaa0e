// canvas_attn: every canvas query attends, in one softmax, to the cached
// prompt keys visible to its layer and to every canvas key -- bidirectional,
// no causal mask ([4xFaster] "DiffusionGemma's Technical Architecture"; GQA
// and the local/global split: [HandsOn] "Detailed Specs").  With `causal`
// set, canvas query i sees canvas keys j <= i only: the causal context
// building of a resolved block before the next one ([HandsOn] "How Is This
// Different from Previous Models?", Figure 3).
//
// bf16 path (k_attn_mfma): flash-style with 16x16x32 bf16 MFMAs.
//   * Work unit = (canvas b, KV head g, key split s) x q-tile of 64 query rows.
//     The query rows of a KV head are its Hq/Hkv query heads x N canvas
//     positions, so one K/V tile read from LDS feeds every query head sharing
//     it.  Long prompts are cut into splits of CL keys (a multiple of 64) so
//     the grid fills the chip; partial (O, m, l) are merged by k_attn_merge in
//     a fixed order.
//   * The q-tiles of one (b, g, s) are mapped to one XCD (blocks go
//     round-robin over the 8 XCDs), so their shared K/V chunk is fetched from
//     HBM once and re-read from that XCD's L2.
//   * Scores are computed transposed, S^T = K Q^T, so each lane ends up holding
//     4+4 keys of one query: exactly the B operand of the P V product
//     (O^T = V^T P^T) once k indices of A and B are matched.  No cross-lane
//     shuffle of P is needed; V is kept transposed (V^T) in HBM and LDS.
//   * Online softmax in base 2 with fp32 state; P is rounded to bf16 for the
//     MFMA and the normaliser sums the rounded values, so a single key gives
//     weight exactly 1.
// fp32 path and odd head sizes (k_attn_simple): one workgroup per query row,
// keys in chunks of 256 with the same online-softmax recurrence.
#include "common.h"

namespace {

constexpr float kLog2e = 1.4426950408889634f;

// Flash attention for bf16 with K/V tiles copied straight from global memory
// into LDS (no register staging), two query sub-tiles per wave.
//
//   * Work unit = (canvas b, KV head g, key split s) x q-tile of 128 query
//     rows; each of the 4 waves holds 32 rows as two 16-row sub-tiles, so
//     every K or V fragment read from LDS feeds two MFMAs.
//   * A 64-key tile of K and of V^T is laid out in LDS in MFMA fragment
//     order (1 KB blocks, lane l's 16 bytes at offset 16 l), written by
//     direct global->LDS copies in which every lane fetches exactly the 16
//     bytes it will later read; reads are conflict-free 16-byte loads.  Two
//     LDS stages: the copy of tile t + 1 runs while tile t is consumed.
//   * Scores are computed transposed (S^T = K Q^T).  The keys of a K fragment
//     are permuted (row m of key block kb holds key 32 (kb/2) + 8 (m/4) +
//     4 (kb%2) + m%4) so that every lane ends up holding 8 consecutive keys
//     of one query per 32-key step: the B operand of O^T = V^T P^T, whose A
//     operand (V^T) is then 16 contiguous bytes per lane, copyable as such.
//   * Online softmax in base 2 with a lazily updated reference maximum: the
//     running state is rescaled only when a tile's maximum exceeds the
//     reference by more than 2^8 (P then stays <= 256, exact scaling is
//     unaffected), which skips almost every rescale.  P is rounded to bf16
//     for the MFMA and the normaliser is the MFMA sum of the same rounded P
//     (an all-ones A operand), so a single key gives weight exactly 1.
// Needs every 8-key group of V^T in one source (key counts multiples of 8).
template <int D>
__global__ __launch_bounds__(256, 2) void k_attn_fa(AttnArgs a, int QT, int xcd_map) {
  constexpr int KT = 64;                 // keys per tile
  constexpr int KS = D / 32, DB = D / 16;
  constexpr int NKB = 4 * KS, NVB = 2 * DB;  // 1 KB fragment blocks of a K tile and of a V^T tile
  static_assert(NKB % 4 == 0 && NVB % 4 == 0, "the four waves copy equal shares of a tile");
  __shared__ __align__(16) bf16_t K0[NKB * 512];
  __shared__ __align__(16) bf16_t K1[NKB * 512];
  __shared__ __align__(16) bf16_t V0[NVB * 512];
  __shared__ __align__(16) bf16_t V1[NVB * 512];

  int bid = blockIdx.x, unit, qt;
  if (xcd_map) {
    const int xcd = bid & 7, slot = bid >> 3;
    unit = (slot / QT) * 8 + xcd;
    qt = slot % QT;
  } else {
    unit = bid / QT;
    qt = bid % QT;
  }
  int b = 0;
  while (b + 1 < a.B && a.ubase[b + 1] <= unit) ++b;
  const int S = a.ns[b], CL = a.cl[b];
  const int s = (unit - a.ubase[b]) % S, g = (unit - a.ubase[b]) / S;
  const int group = a.Hq / a.Hkv;
  const int N = a.N;
  const int Lw = a.lw[b];
  const int total = Lw + (a.canvas_keys ? N : 0);
  const int k0 = s * CL, k1 = min(total, k0 + CL);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lg = lane >> 4, lc = lane & 15;
  const int grows = group * N;
  bool qvalid[2];
  int qh[2], qi[2];
  long long row_g[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int qrow = qt * 128 + wave * 32 + j * 16 + lc;
    qvalid[j] = qrow < grows;
    qh[j] = g * group + (qvalid[j] ? qrow / N : 0);
    qi[j] = qvalid[j] ? qrow % N : 0;
    row_g[j] = ((long long)b * a.Hq + qh[j]) * N + qi[j];
  }

  const bf16_t* kp = reinterpret_cast<const bf16_t*>(a.kp[b]) + (long long)g * Lw * D;
  const bf16_t* vp = reinterpret_cast<const bf16_t*>(a.vp[b]) + (long long)g * D * Lw;
  const bf16_t* kc = reinterpret_cast<const bf16_t*>(a.kc) + ((long long)b * a.Hkv + g) * N * D;
  const bf16_t* vc = reinterpret_cast<const bf16_t*>(a.vc) + ((long long)b * a.Hkv + g) * D * N;

  // Q^T fragments of both sub-tiles (B operand of S^T = K Q^T)
  uint4 qf[2][KS];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const bf16_t* qp = reinterpret_cast<const bf16_t*>(a.q) + row_g[j] * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qf[j][ks] = qvalid[j] ? *reinterpret_cast<const uint4*>(qp + ks * 32 + lg * 8) : make_uint4(0, 0, 0, 0);
  }

  floatx4 oacc[2][DB], lacc[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    lacc[j] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < DB; ++i) oacc[j][i] = floatx4{0.f, 0.f, 0.f, 0.f};
  }
  float m_ref[2] = {-INFINITY, -INFINITY};  // reference maximum of P (scaled log2 units)
  const float sc = kLog2e / sqrtf((float)D);
  const uint4 ones = make_uint4(0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u);  // bf16 1.0 pairs

  // Direct copies of one tile into a stage: wave w copies K blocks w, w + 4,
  // ... and V^T blocks w, w + 4, ...  Keys past the split's end are clamped
  // into it (their scores are masked to -inf, so their P is exactly 0).  The
  // wave index is made wave-uniform so every LDS destination is a scalar.
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const int lane_key = 8 * (lc >> 2) + (lc & 3);  // this lane's key within a K block pair
  auto issue = [&](bf16_t* Kd, bf16_t* Vd, int t0) {
#pragma unroll
    for (int i = 0; i < NKB / 4; ++i) {
      const int q = wv + 4 * i, kb = q / KS, ks = q - kb * KS;
      const int key = min(t0 + 32 * (kb >> 1) + 4 * (kb & 1) + lane_key, k1 - 1);
      const bf16_t* src = key < Lw ? kp + key * D : kc + (key - Lw) * D;
      __builtin_amdgcn_global_load_lds((__attribute__((address_space(1))) const void*)(src + ks * 32 + lg * 8),
                                       (__attribute__((address_space(3))) void*)(Kd + q * 512), 16, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < NVB / 4; ++i) {
      const int q = wv + 4 * i, db = q >> 1, ks2 = q & 1;
      const int c = min(t0 + ks2 * 32 + lg * 8, k1 - 8);
      const int d = db * 16 + lc;
      const bf16_t* src = c < Lw ? vp + d * Lw + c : vc + d * N + (c - Lw);
      __builtin_amdgcn_global_load_lds((__attribute__((address_space(1))) const void*)src,
                                       (__attribute__((address_space(3))) void*)(Vd + q * 512), 16, 0, 0);
    }
  };

  // One 64-key tile from a stage.  `edge`: the tile reaches past the split's
  // end or holds canvas keys under the causal mask.
  auto consume = [&](const bf16_t* Ks, const bf16_t* Vs, int t0, bool edge) {
    floatx4 sacc[2][4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      sacc[0][kb] = floatx4{0.f, 0.f, 0.f, 0.f};
      sacc[1][kb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const uint4 kf = *reinterpret_cast<const uint4*>(Ks + (kb * KS + ks) * 512 + lane * 8);
#pragma unroll
        for (int j = 0; j < 2; ++j)
          sacc[j][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_v, kf),
                                                                 __builtin_bit_cast(bf16x8_v, qf[j][ks]),
                                                                 sacc[j][kb], 0, 0, 0);
      }
      // at most one key block's fragments live at a time (register budget of two waves per SIMD)
      __builtin_amdgcn_sched_barrier(0);
    }
    uint32_t pk[2][2][4];
    float mt[2];
    bool need = false;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      if (edge) {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int key = t0 + 32 * (kb >> 1) + 8 * lg + 4 * (kb & 1) + r;
            const bool vis = key < k1 && !(a.causal && key - Lw > qi[j]);
            if (!vis) sacc[j][kb][r] = -INFINITY;
          }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) mx = fmaxf(mx, sacc[j][kb][r]);
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      mt[j] = mx * sc;
      need = need || mt[j] > m_ref[j] + 8.0f;
    }
    if (__any(need)) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const bool up = mt[j] > m_ref[j] + 8.0f;
        const float alpha = up ? exp2f(m_ref[j] - mt[j]) : 1.0f;  // m_ref = -inf: alpha 0, state is 0
        m_ref[j] = up ? mt[j] : m_ref[j];
        lacc[j] *= alpha;
#pragma unroll
        for (int i = 0; i < DB; ++i) oacc[j][i] *= alpha;
      }
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const float mref = m_ref[j] == -INFINITY ? 0.f : m_ref[j];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int q = 0; q < 2; ++q)
          pk[j][kb >> 1][(kb & 1) * 2 + q] = f2bf2(exp2f(fmaf(sacc[j][kb][2 * q], sc, -mref)),
                                                   exp2f(fmaf(sacc[j][kb][2 * q + 1], sc, -mref)));
    }
#pragma unroll
    for (int ks2 = 0; ks2 < 2; ++ks2) {
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const uint4 vf = *reinterpret_cast<const uint4*>(Vs + (db * 2 + ks2) * 512 + lane * 8);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const uint4 pf = make_uint4(pk[j][ks2][0], pk[j][ks2][1], pk[j][ks2][2], pk[j][ks2][3]);
          oacc[j][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_v, vf),
                                                                 __builtin_bit_cast(bf16x8_v, pf), oacc[j][db], 0, 0, 0);
        }
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const uint4 pf = make_uint4(pk[j][ks2][0], pk[j][ks2][1], pk[j][ks2][2], pk[j][ks2][3]);
        lacc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_v, ones),
                                                           __builtin_bit_cast(bf16x8_v, pf), lacc[j], 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  const int ntiles = k1 > k0 ? (k1 - k0 + KT - 1) / KT : 0;
  // tiles that need the mask: past the split's end, or canvas keys (from key
  // Lw on) under the causal mask
  auto edge = [&](int t0) { return t0 + KT > k1 || (a.causal && t0 + KT > Lw); };
  // The copies into a stage are waited for explicitly before the barrier that
  // publishes it: the compiler's own wait before the barrier is missing on the
  // loop's back edge (the copy issued in the second half of an iteration is
  // read in the first half of the next), so without this a wave could pass
  // the barrier while its part of the tile is still in flight.
  auto copies_done = [] { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); };
  if (ntiles > 0) issue(K0, V0, k0);
  for (int it = 0; it < ntiles; it += 2) {
    copies_done();
    __syncthreads();  // tile it is in stage 0 (every wave's copies done); stage 1 is free
    if (it + 1 < ntiles) issue(K1, V1, k0 + (it + 1) * KT);
    {
      const int t0 = k0 + it * KT;
      consume(K0, V0, t0, edge(t0));
    }
    if (it + 1 >= ntiles) break;
    copies_done();
    __syncthreads();  // tile it + 1 is in stage 1; stage 0 is free
    if (it + 2 < ntiles) issue(K0, V0, k0 + (it + 2) * KT);
    {
      const int t0 = k0 + (it + 1) * KT;
      consume(K1, V1, t0, edge(t0));
    }
  }

  mfma_drain();
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    if (!qvalid[j]) continue;
    const float l = lacc[j][0];
    if (S == 1) {
      // a single split: normalise and store the bf16 output directly (the
      // same quotient the merge forms from one split)
      bf16_t* o = reinterpret_cast<bf16_t*>(a.o) + ((long long)b * N + qi[j]) * a.Hq * D + (long long)qh[j] * D;
      auto nrm = [&](float x) { return f2bf(l > 0.f ? x / l : 0.f); };
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int d = db * 16 + lg * 4;
        *reinterpret_cast<uint2*>(o + d) =
            make_uint2((uint32_t)nrm(oacc[j][db][0]) | ((uint32_t)nrm(oacc[j][db][1]) << 16),
                       (uint32_t)nrm(oacc[j][db][2]) | ((uint32_t)nrm(oacc[j][db][3]) << 16));
      }
    } else {
      const long long rows_all = (long long)a.B * a.Hq * N;
      const long long pr = (long long)s * rows_all + row_g[j];
      float* po = a.part_o + pr * D;
#pragma unroll
      for (int db = 0; db < DB; ++db)
        *reinterpret_cast<float4*>(po + db * 16 + lg * 4) =
            make_float4(oacc[j][db][0], oacc[j][db][1], oacc[j][db][2], oacc[j][db][3]);
      if (lg == 0) {
        a.part_m[pr] = m_ref[j];
        a.part_l[pr] = l;
      }
    }
  }
}

template <int D, bool ALIGNED>
__global__ __launch_bounds__(256) void k_attn_mfma(AttnArgs a, int QT, int xcd_map) {
  constexpr int KT = 64;            // keys per tile
  constexpr int KLD = D + 8;        // padded LDS row of K (elements)
  constexpr int VLD = KT + 8;       // padded LDS row of V^T
  constexpr int KVEC = KT * D / 8 / 256;  // 16-byte vectors per thread for a K tile
  constexpr int VVEC = D * KT / 8 / 256;  // same for V^T
  __shared__ __align__(16) bf16_t Ks[KT * KLD];
  __shared__ __align__(16) bf16_t Vs[D * VLD];

  int bid = blockIdx.x, unit, qt;
  if (xcd_map) {
    const int xcd = bid & 7, slot = bid >> 3;
    unit = (slot / QT) * 8 + xcd;
    qt = slot % QT;
  } else {
    unit = bid / QT;
    qt = bid % QT;
  }
  int b = 0;
  while (b + 1 < a.B && a.ubase[b + 1] <= unit) ++b;
  const int S = a.ns[b], CL = a.cl[b];
  const int s = (unit - a.ubase[b]) % S, g = (unit - a.ubase[b]) / S;
  const int group = a.Hq / a.Hkv;
  const int N = a.N;
  const int Lw = a.lw[b];
  const int total = Lw + (a.canvas_keys ? N : 0);
  const int k0 = s * CL, k1 = min(total, k0 + CL);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lg = lane >> 4, lc = lane & 15;
  const int grows = group * N;
  const int qrow = qt * 64 + wave * 16 + lc;
  const bool qvalid = qrow < grows;
  const int qh = g * group + (qvalid ? qrow / N : 0);
  const int qi = qvalid ? qrow % N : 0;
  const long long row_g = ((long long)b * a.Hq + qh) * N + qi;  // global query row

  const bf16_t* kp = reinterpret_cast<const bf16_t*>(a.kp[b]) + (long long)g * Lw * D;
  const bf16_t* vp = reinterpret_cast<const bf16_t*>(a.vp[b]) + (long long)g * D * Lw;
  const bf16_t* kc = reinterpret_cast<const bf16_t*>(a.kc) + ((long long)b * a.Hkv + g) * N * D;
  const bf16_t* vc = reinterpret_cast<const bf16_t*>(a.vc) + ((long long)b * a.Hkv + g) * D * N;

  // Q^T fragments (B operand of S^T = K Q^T)
  uint4 qf[D / 32];
  {
    const bf16_t* qp = reinterpret_cast<const bf16_t*>(a.q) + row_g * D;
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks)
      qf[ks] = qvalid ? *reinterpret_cast<const uint4*>(qp + ks * 32 + lg * 8) : make_uint4(0, 0, 0, 0);
  }

  floatx4 oacc[D / 16];
#pragma unroll
  for (int i = 0; i < D / 16; ++i) oacc[i] = floatx4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;
  const float sc = kLog2e / sqrtf((float)D);

  // K/V tiles go global -> registers -> LDS, two tiles ahead of the one being
  // consumed.  ALIGNED (every 8-key group of V^T lies in one source and the
  // key count is a multiple of 8): loads are unconditional, with key indices
  // clamped into [k0, k1) -- rows past the split's last key only ever meet a
  // score of -inf, i.e. P = 0 -- so the compiler's load counters stay exact
  // and both tiles in flight stay in flight.  Otherwise partial groups are
  // gathered element by element.
  typedef unsigned int v4u __attribute__((ext_vector_type(4)));
  v4u kreg[2][KVEC], vreg[2][VVEC];
  auto load_tile = [&](v4u* kr, v4u* vr, int t0) {
#pragma unroll
    for (int it = 0; it < KVEC; ++it) {
      const int v = tid + it * 256;
      const int row = v / (D / 8), c8 = v % (D / 8);
      int key = t0 + row;
      if constexpr (ALIGNED) {
        key = min(key, k1 - 1);
        const bf16_t* src = key < Lw ? kp + (long long)key * D : kc + (long long)(key - Lw) * D;
        kr[it] = *reinterpret_cast<const v4u*>(src + c8 * 8);
      } else {
        v4u val = {0u, 0u, 0u, 0u};
        if (key < k1) {
          const bf16_t* src = key < Lw ? kp + (long long)key * D : kc + (long long)(key - Lw) * D;
          val = *reinterpret_cast<const v4u*>(src + c8 * 8);
        }
        kr[it] = val;
      }
    }
#pragma unroll
    for (int it = 0; it < VVEC; ++it) {
      const int v = tid + it * 256;
      const int d = v / (KT / 8), c8 = v % (KT / 8);
      int key = t0 + c8 * 8;
      if constexpr (ALIGNED) {
        key = min(key, k1 - 8);
        const bf16_t* src = key < Lw ? vp + (long long)d * Lw + key : vc + (long long)d * N + (key - Lw);
        vr[it] = *reinterpret_cast<const v4u*>(src);
      } else {
        v4u val = {0u, 0u, 0u, 0u};
        const bool in_p = key + 8 <= Lw && (Lw & 7) == 0;
        const bool in_c = key >= Lw && ((key - Lw) & 7) == 0 && (N & 7) == 0;
        if (key + 8 <= k1 && (in_p || in_c)) {
          const bf16_t* src = in_p ? vp + (long long)d * Lw + key : vc + (long long)d * N + (key - Lw);
          val = *reinterpret_cast<const v4u*>(src);
        } else {
          uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const int kk = key + j;
            uint32_t x = 0;
            if (kk < k1) x = kk < Lw ? vp[(long long)d * Lw + kk] : vc[(long long)d * N + (kk - Lw)];
            w[j >> 1] |= x << ((j & 1) * 16);
          }
          val = v4u{w[0], w[1], w[2], w[3]};
        }
        vr[it] = val;
      }
    }
  };
  auto store_tile = [&](const v4u* kr, const v4u* vr) {
#pragma unroll
    for (int it = 0; it < KVEC; ++it) {
      const int v = tid + it * 256;
      const int row = v / (D / 8), c8 = v % (D / 8);
      *reinterpret_cast<v4u*>(&Ks[row * KLD + c8 * 8]) = kr[it];
    }
#pragma unroll
    for (int it = 0; it < VVEC; ++it) {
      const int v = tid + it * 256;
      const int d = v / (KT / 8), c8 = v % (KT / 8);
      *reinterpret_cast<v4u*>(&Vs[d * VLD + c8 * 8]) = vr[it];
    }
  };
  // one 64-key tile of the online softmax from LDS
  auto consume = [&](int t0) {
    // S^T for 4 blocks of 16 keys: sacc[kb][r] = score(key t0+kb*16+lg*4+r, query lc)
    floatx4 sacc[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      sacc[kb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks) {
        const uint4 kf = *reinterpret_cast<const uint4*>(&Ks[(kb * 16 + lc) * KLD + ks * 32 + lg * 8]);
        sacc[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_v, kf),
                                                            __builtin_bit_cast(bf16x8_v, qf[ks]),
                                                            sacc[kb], 0, 0, 0);
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = t0 + kb * 16 + lg * 4 + r;
        const bool vis = key < k1 && !(a.causal && key - Lw > qi);  // canvas key after the query
        const float sv = vis ? sacc[kb][r] * sc : -INFINITY;
        sacc[kb][r] = sv;
        mx = fmaxf(mx, sv);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m_run, mx);
    const bool none = m_new == -INFINITY;
    const float alpha = none ? 1.f : exp2f(m_run - m_new);
    const float mref = none ? 0.f : m_new;
    // P^T fragments: slot j<4 -> key 32*ks2 + 4*lg + j, slot j>=4 -> key 32*ks2 + 16 + 4*lg + j-4
    uint32_t pk[2][4];
    float ls = 0.f;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int q = 0; q < 2; ++q) {  // slots j = (kb & 1) * 4 + 2q, 2q + 1 share one word
        const uint32_t w = f2bf2(exp2f(sacc[kb][2 * q] - mref), exp2f(sacc[kb][2 * q + 1] - mref));
        ls += __uint_as_float(w << 16);
        ls += __uint_as_float(w & 0xffff0000u);
        pk[kb >> 1][(kb & 1) * 2 + q] = w;
      }
    ls += __shfl_xor(ls, 16, 64);
    ls += __shfl_xor(ls, 32, 64);
    l_run = l_run * alpha + ls;
    m_run = m_new;
#pragma unroll
    for (int i = 0; i < D / 16; ++i) oacc[i] *= alpha;
#pragma unroll
    for (int ks2 = 0; ks2 < 2; ++ks2) {
      const uint4 pf = make_uint4(pk[ks2][0], pk[ks2][1], pk[ks2][2], pk[ks2][3]);
#pragma unroll
      for (int db = 0; db < D / 16; ++db) {
        const bf16_t* vrow = &Vs[(db * 16 + lc) * VLD + ks2 * 32 + lg * 4];
        const uint2 lo = *reinterpret_cast<const uint2*>(vrow);
        const uint2 hi = *reinterpret_cast<const uint2*>(vrow + 16);
        const uint4 vf = make_uint4(lo.x, lo.y, hi.x, hi.y);
        oacc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_v, vf),
                                                            __builtin_bit_cast(bf16x8_v, pf),
                                                            oacc[db], 0, 0, 0);
      }
    }
  };

  const int ntiles = k1 > k0 ? (k1 - k0 + KT - 1) / KT : 0;
  if (ntiles > 0) {
    load_tile(kreg[0], vreg[0], k0);
    load_tile(kreg[1], vreg[1], k0 + KT);  // clamped (ALIGNED) or masked past the split
  }
  for (int it = 0; it < ntiles; it += 2) {
    store_tile(kreg[0], vreg[0]);
    __syncthreads();
    load_tile(kreg[0], vreg[0], k0 + (it + 2) * KT);
    consume(k0 + it * KT);
    __syncthreads();
    if (it + 1 >= ntiles) break;
    store_tile(kreg[1], vreg[1]);
    __syncthreads();
    load_tile(kreg[1], vreg[1], k0 + (it + 3) * KT);
    consume(k0 + (it + 1) * KT);
    __syncthreads();
  }

  mfma_drain();
  if (qvalid && S == 1) {
    // a single split: normalise and store the bf16 output directly (the same
    // quotient the merge forms from one split)
    bf16_t* o = reinterpret_cast<bf16_t*>(a.o) + ((long long)b * N + qi) * a.Hq * D + (long long)qh * D;
    auto nrm = [&](float x) { return f2bf(l_run > 0.f ? x / l_run : 0.f); };
#pragma unroll
    for (int db = 0; db < D / 16; ++db) {
      const int d = db * 16 + lg * 4;
      *reinterpret_cast<uint2*>(o + d) =
          make_uint2((uint32_t)nrm(oacc[db][0]) | ((uint32_t)nrm(oacc[db][1]) << 16),
                     (uint32_t)nrm(oacc[db][2]) | ((uint32_t)nrm(oacc[db][3]) << 16));
    }
  } else if (qvalid) {
    const long long rows_all = (long long)a.B * a.Hq * N;
    const long long pr = (long long)s * rows_all + row_g;
    float* po = a.part_o + pr * D;
#pragma unroll
    for (int db = 0; db < D / 16; ++db)
      *reinterpret_cast<float4*>(po + db * 16 + lg * 4) =
          make_float4(oacc[db][0], oacc[db][1], oacc[db][2], oacc[db][3]);
    if (lg == 0) {
      a.part_m[pr] = m_run;
      a.part_l[pr] = l_run;
    }
  }
}

// o[(b*N + i), h*D + d] = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s, splits in order.
// One wave per query row (4 rows per workgroup): lane s fetches split s's
// (m, l), the wave max gives M, then every lane accumulates its D / 64
// columns over the splits in order, 8 splits' loads in flight at a time.
template <typename T>
__global__ __launch_bounds__(256) void k_attn_merge(AttnArgs a) {
  const long long rows_all = (long long)a.B * a.Hq * a.N;
  const long long row = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows_all) return;
  const int S = a.ns[row / ((long long)a.Hq * a.N)];
  if (S == 1) return;  // one split: stored by the attention kernel
  constexpr int DJ = 4;  // columns per lane (D <= 256)
  const int D = a.D;
  const float m_l = lane < S ? a.part_m[lane * rows_all + row] : -INFINITY;
  const float l_l = lane < S ? a.part_l[lane * rows_all + row] : 0.f;
  float M = m_l;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) M = fmaxf(M, __shfl_xor(M, o, 64));
  float num[DJ] = {0.f, 0.f, 0.f, 0.f}, den = 0.f;
  if (M != -INFINITY) {
    constexpr int U = 8;
    for (int s0 = 0; s0 < S; s0 += U) {
      float ov[U][DJ];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int sp = min(s0 + u, S - 1);
#pragma unroll
        for (int j = 0; j < DJ; ++j) {
          const int d = lane + 64 * j;
          ov[u][j] = d < D ? a.part_o[(sp * rows_all + row) * D + d] : 0.f;
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (s0 + u < S) {  // splits in order
          const float mv = __shfl(m_l, s0 + u, 64), lv = __shfl(l_l, s0 + u, 64);
          const float w = exp2f(mv - M);
#pragma unroll
          for (int j = 0; j < DJ; ++j) num[j] += w * ov[u][j];
          den += w * lv;
        }
      }
    }
  }
  const int i = (int)(row % a.N);
  const long long bh = row / a.N;
  const int h = (int)(bh % a.Hq), b = (int)(bh / a.Hq);
  T* o = reinterpret_cast<T*>(a.o) + ((long long)b * a.N + i) * a.Hq * D + (long long)h * D;
#pragma unroll
  for (int j = 0; j < DJ; ++j) {
    const int d = lane + 64 * j;
    if (d < D) o[d] = from_f<T>(den > 0.f ? num[j] / den : 0.f);
  }
}

// One query row per workgroup; generic in T and D (<= 256).
template <typename T>
__global__ __launch_bounds__(256) void k_attn_simple(AttnArgs a) {
  __shared__ float qs[256];
  __shared__ float ps[256];
  __shared__ float red[8];
  const long long row = blockIdx.x;  // (b*Hq + h)*N + i
  const int N = a.N, D = a.D;
  const int i = (int)(row % N);
  const long long bh = row / N;
  const int h = (int)(bh % a.Hq), b = (int)(bh / a.Hq);
  const int g = h / (a.Hq / a.Hkv);
  const int Lw = a.lw[b];
  const int total = Lw + (a.canvas_keys ? N : 0);
  const int tid = threadIdx.x;
  const T* q = reinterpret_cast<const T*>(a.q) + row * D;
  const T* kp = reinterpret_cast<const T*>(a.kp[b]) + (long long)g * Lw * D;
  const T* vp = reinterpret_cast<const T*>(a.vp[b]) + (long long)g * D * Lw;
  const T* kc = reinterpret_cast<const T*>(a.kc) + ((long long)b * a.Hkv + g) * N * D;
  const T* vc = reinterpret_cast<const T*>(a.vc) + ((long long)b * a.Hkv + g) * D * N;
  if (tid < D) qs[tid] = to_f<T>(q[tid]);
  __syncthreads();
  const float scale = 1.0f / sqrtf((float)D);
  float m = -INFINITY, l = 0.f, o = 0.f;
  for (int c0 = 0; c0 < total; c0 += 256) {
    const int key = c0 + tid;
    float sv = -INFINITY;
    if (key < total && !(a.causal && key - Lw > i)) {  // a canvas key after the query is masked
      const T* kr = key < Lw ? kp + (long long)key * D : kc + (long long)(key - Lw) * D;
      float acc = 0.f;
      for (int d = 0; d < D; ++d) acc += qs[d] * to_f<T>(kr[d]);
      sv = acc * scale;
    }
    // block max
    float mx = wave_max(sv);
    __syncthreads();
    if ((tid & 63) == 0) red[tid >> 6] = mx;
    __syncthreads();
    mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    const float m_new = fmaxf(m, mx);
    const float alpha = m == -INFINITY ? 0.f : expf(m - m_new);
    const float p = key < total ? expf(sv - m_new) : 0.f;
    ps[tid] = p;
    const float psum = block_sum(p, red + 4);
    l = l * alpha + psum;
    m = m_new;
    __syncthreads();
    if (tid < D) {
      float acc = 0.f;
      const int nk = min(256, total - c0);
      for (int j = 0; j < nk; ++j) {
        const int kk = c0 + j;
        const float vv = kk < Lw ? to_f<T>(vp[(long long)tid * Lw + kk]) : to_f<T>(vc[(long long)tid * N + (kk - Lw)]);
        acc += ps[j] * vv;
      }
      o = o * alpha + acc;
    }
    __syncthreads();
  }
  if (tid < D) {
    T* out = reinterpret_cast<T*>(a.o);
    out[((long long)b * N + i) * a.Hq * D + (long long)h * D + tid] = from_f<T>(l > 0.f ? o / l : 0.f);
  }
}

}  // namespace

// Split count and length: enough workgroups to cover the 256 CUs once, and no
// split longer than 4096 keys (long prompts); splits are whole 64-key tiles.
// Key splits of canvas b from its own key count only: enough (KV head x split)
// units per canvas to spread one canvas over the chip, at most 4096 keys per
// split, at least 64, at most 64 splits (the partial buffers hold 64 per row).
static void choose_splits(int total, int Hkv, int QT, int* S_out, int* CL_out) {
  const int base = Hkv * QT;
  int S = max((256 + base - 1) / base, (total + 4095) / 4096);
  S = min(S, max(1, (total + 63) / 64));
  S = min(S, 64);
  int CL = ((total + S - 1) / S + 63) / 64 * 64;
  if (CL < 64) CL = 64;
  S = max(1, (total + CL - 1) / CL);
  *S_out = S;
  *CL_out = CL;
}

// Key splits of canvas b for the direct-copy kernel (two workgroups per CU):
// enough (KV head x split x q-tile) workgroups to fill the chip's slots once,
// splits of at most 8192 keys, and for long prompts a split count that fills
// whole rounds of slots; whole 64-key tiles, at most 64 splits.
static void choose_splits_fa(int total, int base, int* S_out, int* CL_out) {
  const int slots = 2 * 256;
  const int smin = (slots + base - 1) / base;
  int S = max(smin, (total + 8191) / 8192);
  if (S > smin && slots % base == 0) {
    const int r = slots / base;
    S = (S + r - 1) / r * r;
  }
  S = min(S, max(1, (total + 63) / 64));
  S = min(S, 64);
  int CL = ((total + S - 1) / S + 63) / 64 * 64;
  if (CL < 64) CL = 64;
  S = max(1, (total + CL - 1) / CL);
  *S_out = S;
  *CL_out = CL;
}

hipError_t launch_attention(int is_bf16, const AttnArgs& a0, hipStream_t st, KTime t) {
  const long long rows_all = (long long)a0.B * a0.Hq * a0.N;
  if (rows_all == 0) return hipSuccess;
  if (a0.B > DG_MAX_BATCH) return hipErrorInvalidValue;
  // every 8-key group of V^T in one source, and key counts multiples of 8
  bool aligned0 = (a0.N & 7) == 0;
  for (int b = 0; b < a0.B; ++b) aligned0 = aligned0 && (a0.lw[b] & 7) == 0;
  if (is_bf16 && (a0.D == 128 || a0.D == 64) && aligned0) {
    AttnArgs a = a0;
    const int QT = (a.Hq / a.Hkv * a.N + 127) / 128;
    int smax = 1;
    a.ubase[0] = 0;
    for (int b = 0; b < a.B; ++b) {
      choose_splits_fa(a.lw[b] + (a.canvas_keys ? a.N : 0), a.Hkv * QT, &a.ns[b], &a.cl[b]);
      smax = max(smax, a.ns[b]);
      a.ubase[b + 1] = a.ubase[b] + a.Hkv * a.ns[b];
    }
    if ((long long)smax * rows_all > a.part_cap_rows) return hipErrorInvalidValue;
    const long long units = a.ubase[a.B];
    const int xcd_map = (units % 8) == 0;
    const dim3 grid((unsigned)(units * QT));
    hipEvent_t stop1 = smax == 1 ? t.stop : nullptr;
    hipError_t e = a.D == 128 ? launch_k(k_attn_fa<128>, grid, dim3(256), 0, st, t.start, stop1, a, QT, xcd_map)
                              : launch_k(k_attn_fa<64>, grid, dim3(256), 0, st, t.start, stop1, a, QT, xcd_map);
    if (e != hipSuccess || smax == 1) return e;
    return launch_k(k_attn_merge<bf16_t>, dim3((unsigned)((rows_all + 3) / 4)), dim3(256), 0, st, nullptr, t.stop, a);
  }
  if (is_bf16 && (a0.D == 128 || a0.D == 64)) {
    AttnArgs a = a0;
    const int QT = (a.Hq / a.Hkv * a.N + 63) / 64;
    int smax = 1;
    a.ubase[0] = 0;
    for (int b = 0; b < a.B; ++b) {
      choose_splits(a.lw[b] + (a.canvas_keys ? a.N : 0), a.Hkv, QT, &a.ns[b], &a.cl[b]);
      smax = max(smax, a.ns[b]);
      a.ubase[b + 1] = a.ubase[b] + a.Hkv * a.ns[b];
    }
    if ((long long)smax * rows_all > a.part_cap_rows) return hipErrorInvalidValue;
    const long long units = a.ubase[a.B];
    const int xcd_map = (units % 8) == 0;
    const dim3 grid((unsigned)(units * QT));
    // every canvas in one split: the kernel stores the output itself and closes the timing
    hipEvent_t stop1 = smax == 1 ? t.stop : nullptr;
    // every 8-key group of V^T in one source, and key counts multiples of 8
    bool aligned = (a.N & 7) == 0;
    for (int b = 0; b < a.B; ++b) aligned = aligned && (a.lw[b] & 7) == 0;
    hipError_t e;
    if (a.D == 128)
      e = aligned ? launch_k(k_attn_mfma<128, true>, grid, dim3(256), 0, st, t.start, stop1, a, QT, xcd_map)
                  : launch_k(k_attn_mfma<128, false>, grid, dim3(256), 0, st, t.start, stop1, a, QT, xcd_map);
    else
      e = aligned ? launch_k(k_attn_mfma<64, true>, grid, dim3(256), 0, st, t.start, stop1, a, QT, xcd_map)
                  : launch_k(k_attn_mfma<64, false>, grid, dim3(256), 0, st, t.start, stop1, a, QT, xcd_map);
    if (e != hipSuccess || smax == 1) return e;
    return launch_k(k_attn_merge<bf16_t>, dim3((unsigned)((rows_all + 3) / 4)), dim3(256), 0, st, nullptr, t.stop, a);
  }
  if (a0.D > 256) return hipErrorInvalidValue;
  if (is_bf16)
    return launch_k(k_attn_simple<bf16_t>, dim3((unsigned)rows_all), dim3(256), 0, st, t.start, t.stop, a0);
  return launch_k(k_attn_simple<float>, dim3((unsigned)rows_all), dim3(256), 0, st, t.start, t.stop, a0);
}
