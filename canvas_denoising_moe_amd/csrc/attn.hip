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
#include <type_traits>

#include "common.h"

namespace {

constexpr float kLog2e = 1.4426950408889634f;

// Flash attention for bf16 with K/V tiles copied straight from global memory
// into LDS (no register staging), two query sub-tiles per wave.
//
//   * Work unit = (canvas b, KV head g, key split s) x q-tile of 256 query
//     rows; each of the 8 waves holds 32 rows as two 16-row sub-tiles, so
//     every K or V fragment read from LDS feeds two MFMAs, and one K/V tile
//     in LDS feeds all 256 rows.
//   * A 64-key tile of K and of V^T is laid out in LDS in MFMA fragment
//     order (1 KB blocks, lane l's 16 bytes at offset 16 l), written by
//     direct global->LDS copies in which every lane fetches exactly the 16
//     bytes it will later read; reads are conflict-free 16-byte loads.  Four
//     LDS stages (128 KB at D = 128): the copies of tiles t + 1 and t + 2 are
//     in flight while tile t is consumed, and tile t + 3 is issued as soon as
//     every wave is done with tile t - 1.  A tile in one source (prompt or
//     canvas keys) is copied from a uniform base plus fixed per-lane offsets;
//     one that crosses the boundary or the split's end goes through registers.
//   * Scores are computed transposed (S^T = K Q^T).  The keys of a K fragment
//     are permuted (row m of key block kb holds key 32 (kb/2) + 8 (m/4) +
//     4 (kb%2) + m%4) so that every lane ends up holding 8 consecutive keys
//     of one query per 32-key step: the B operand of O^T = V^T P^T, whose A
//     operand (V^T) is then 16 contiguous bytes per lane, copyable as such.
//     K and V^T fragments are read from LDS one block ahead of the MFMAs.
//   * Online softmax in base 2 with a lazily updated reference maximum: the
//     running state is rescaled only when a tile's maximum exceeds the
//     reference by more than 2^8 (P then stays <= 256, exact scaling is
//     unaffected), which skips almost every rescale.  P is rounded to bf16
//     for the MFMA and the normaliser is the MFMA sum of the same rounded P
//     (an all-ones A operand), so a single key gives weight exactly 1.  The
//     exponentials use the hardware base-2 exponential directly: arguments
//     are <= 8, and results below the fp32 normal range only ever meet a
//     bf16 rounding that keeps them negligible next to the maximum's weight.
// Needs every 8-key group of V^T in one source (key counts multiples of 8).
template <int D>
__global__ __launch_bounds__(512, 2) void k_attn_fa(AttnArgs a, int QT, int xcd_map) {
  constexpr int KT = 64;                 // keys per tile
  constexpr int NW = 8;                  // waves per workgroup
  constexpr int KS = D / 32, DB = D / 16;
  constexpr int NKB = 4 * KS, NVB = 2 * DB;  // 1 KB fragment blocks of a K tile and of a V^T tile
  constexpr int CKW = NKB / NW, CVW = NVB / NW, CPW = CKW + CVW;  // copies per wave per tile
  static_assert(NKB % NW == 0 && NVB % NW == 0, "the waves copy equal shares of a tile");
  // four stages (K blocks, then V^T blocks); one array per stage, so that
  // reads of a stage are seen to depend only on the copies into it
  __shared__ __align__(16) bf16_t S0[(NKB + NVB) * 512];
  __shared__ __align__(16) bf16_t S1[(NKB + NVB) * 512];
  __shared__ __align__(16) bf16_t S2[(NKB + NVB) * 512];
  __shared__ __align__(16) bf16_t S3[(NKB + NVB) * 512];

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
    const int qrow = qt * 256 + wave * 32 + j * 16 + lc;
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
  // wait for Q here, in a form the compiler sees: otherwise it keeps the
  // loads pending through the copy pipeline and drains all copies at a use
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)

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
  // Byte offsets of this lane's 16 bytes within a tile that lies in one
  // source: K rows are D elements apart; V^T rows (one per d) are a stride
  // apart that depends on the source, so only the in-row part is kept.
  uint32_t koff[CKW], voff[CVW];
  int vrow[CVW];
#pragma unroll
  for (int i = 0; i < CKW; ++i) {
    const int q = wv + NW * i, kb = q / KS, ks = q - kb * KS;
    koff[i] = 2u * (uint32_t)((32 * (kb >> 1) + 4 * (kb & 1) + lane_key) * D + ks * 32 + lg * 8);
  }
#pragma unroll
  for (int i = 0; i < CVW; ++i) {
    const int q = wv + NW * i, db = q >> 1, ks2 = q & 1;
    vrow[i] = db * 16 + lc;
    voff[i] = 2u * (uint32_t)(ks2 * 32 + lg * 8);
  }
  // One direct copy: every lane moves the 16 bytes at base + voff (byte
  // offset) to LDS at dst + 16 lane.  Written as asm so that the compiler's
  // own memory-counter bookkeeping does not see it: it cannot tell the
  // stages apart and would drain every copy in flight before reading any
  // stage; the waits before the barriers below cover these copies.  M0
  // (the LDS destination) is set by the compiler through the constraint;
  // the s_nop is the one wait state a copy to LDS needs after M0 is written.
  auto copy16 = [](bf16_t* dst, const char* base, uint32_t voff) {
    const uint32_t lds = (uint32_t)(size_t)((__attribute__((address_space(3))) bf16_t*)dst);
    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(base), "{m0}"(lds) : "memory");
  };
  auto issue = [&](bf16_t* Kd, bf16_t* Vd, int t0) {
    const bool in_p = t0 + KT <= min(k1, Lw), in_c = t0 >= Lw && t0 + KT <= k1;
    if (in_p || in_c) {
      // the whole tile in one source: a uniform base plus per-lane offsets
      const char* kb_ = reinterpret_cast<const char*>(in_p ? kp + (long long)t0 * D : kc + (long long)(t0 - Lw) * D);
      const char* vb_ = reinterpret_cast<const char*>(in_p ? vp + t0 : vc + (t0 - Lw));
      const uint32_t vstride = 2u * (uint32_t)(in_p ? Lw : N);
#pragma unroll
      for (int i = 0; i < CKW; ++i) copy16(Kd + (wv + NW * i) * 512, kb_, koff[i]);
#pragma unroll
      for (int i = 0; i < CVW; ++i) copy16(Vd + (wv + NW * i) * 512, vb_, vstride * (uint32_t)vrow[i] + voff[i]);
      return;
    }
    // A tile that crosses from prompt to canvas keys or past the split's end
    // (rare): per-lane sources, staged through registers.  Its loads are
    // waited for before the stores to LDS, and the vector memory counter
    // drains in order, so every copy issued before it has landed as well.
    uint4 kr[CKW], vr[CVW];
#pragma unroll
    for (int i = 0; i < CKW; ++i) {
      const int q = wv + NW * i, kb = q / KS, ks = q - kb * KS;
      const int key = min(t0 + 32 * (kb >> 1) + 4 * (kb & 1) + lane_key, k1 - 1);
      const bf16_t* src = key < Lw ? kp + key * D : kc + (key - Lw) * D;
      kr[i] = *reinterpret_cast<const uint4*>(src + ks * 32 + lg * 8);
    }
#pragma unroll
    for (int i = 0; i < CVW; ++i) {
      const int q = wv + NW * i, db = q >> 1, ks2 = q & 1;
      const int c = min(t0 + ks2 * 32 + lg * 8, k1 - 8);
      const int d = db * 16 + lc;
      const bf16_t* src = c < Lw ? vp + d * Lw + c : vc + d * N + (c - Lw);
      vr[i] = *reinterpret_cast<const uint4*>(src);
    }
#pragma unroll
    for (int i = 0; i < CKW; ++i) *reinterpret_cast<uint4*>(Kd + (wv + NW * i) * 512 + lane * 8) = kr[i];
#pragma unroll
    for (int i = 0; i < CVW; ++i) *reinterpret_cast<uint4*>(Vd + (wv + NW * i) * 512 + lane * 8) = vr[i];
  };

  // keys visible to query sub-tile j: below the split's end and, under the
  // causal mask, canvas keys up to the query's own position
  int klim[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) klim[j] = a.causal ? min(k1, Lw + qi[j] + 1) : k1;
  // maximum over the four lanes lc, lc + 16, lc + 32, lc + 48 (one query's
  // keys): the swaps exchange rows 16 and 32 lanes apart
  auto max_lg = [](float x) {
    const uint32_t u = __float_as_uint(x);
    const auto s32 = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    x = fmaxf(__uint_as_float(s32[0]), __uint_as_float(s32[1]));
    const uint32_t w = __float_as_uint(x);
    const auto s16 = __builtin_amdgcn_permlane16_swap(w, w, false, false);
    return fmaxf(__uint_as_float(s16[0]), __uint_as_float(s16[1]));
  };

  // ---- the pieces of one 64-key tile ----
  typedef floatx4 Sacc[2][4];    // S^T of a tile: [sub-tile j][key block kb]
  typedef uint32_t Pk[2][2][4];  // P^T as bf16 pairs: [j][32-key step][word]
  using yes = std::true_type;
  using no = std::false_type;
  auto mref_of = [&](int j) { return m_ref[j] == -INFINITY ? 0.f : m_ref[j]; };
  // two P values of slot pair q of key block kb, rounded to bf16
  auto p_word = [&](const Sacc& acc, int j, int kb, int q, float mr) {
    return f2bf2(__builtin_amdgcn_exp2f(fmaf(acc[j][kb][2 * q], sc, -mr)),
                 __builtin_amdgcn_exp2f(fmaf(acc[j][kb][2 * q + 1], sc, -mr)));
  };
  // S^T = K Q^T of the tile in stage Ks, K fragments read one key block
  // ahead of their MFMAs.  WithP: the P of the previous tile (scores `prev`)
  // is formed in the same block, its exponentials interleaved with these
  // MFMAs, so the vector and matrix units work at the same time.
  auto s_tile = [&](const bf16_t* Ks, Sacc& acc, auto with_p, const Sacc& prev, Pk& pk) {
    constexpr bool WithP = decltype(with_p)::value;
    float mr[2] = {0.f, 0.f};
    if constexpr (WithP) {
      mr[0] = mref_of(0);
      mr[1] = mref_of(1);
    }
    uint4 kfr[2][KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) kfr[0][ks] = *reinterpret_cast<const uint4*>(Ks + ks * 512 + lane * 8);
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      if (kb + 1 < 4) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          kfr[(kb + 1) & 1][ks] = *reinterpret_cast<const uint4*>(Ks + ((kb + 1) * KS + ks) * 512 + lane * 8);
      }
      acc[0][kb] = floatx4{0.f, 0.f, 0.f, 0.f};
      acc[1][kb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[j][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_v, kfr[kb & 1][ks]),
                                                               __builtin_bit_cast(bf16x8_v, qf[j][ks]), acc[j][kb],
                                                               0, 0, 0);
      if constexpr (WithP) {
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int q = 0; q < 2; ++q) pk[j][kb >> 1][(kb & 1) * 2 + q] = p_word(prev, j, kb, q, mr[j]);
      }
      // schedule: the first block's reads, then per block the next block's
      // reads ahead of this block's MFMAs (with the P arithmetic between them)
      if (kb == 0) __builtin_amdgcn_sched_group_barrier(0x100, KS, 0);  // DS read
      if (kb + 1 < 4) __builtin_amdgcn_sched_group_barrier(0x100, KS, 0);
      if constexpr (WithP) {
#pragma unroll
        for (int m = 0; m < 2 * KS; ++m) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
          __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);  // VALU
        }
      } else {
        __builtin_amdgcn_sched_group_barrier(0x008, 2 * KS, 0);
      }
    }
  };
  // P of a tile's scores on their own (no MFMAs to hide them behind)
  auto p_tile = [&](const Sacc& acc, Pk& pk) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const float mr = mref_of(j);
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int q = 0; q < 2; ++q) pk[j][kb >> 1][(kb & 1) * 2 + q] = p_word(acc, j, kb, q, mr);
    }
  };
  // mask (edge tiles) and per-query maximum of a tile's scores, scaled to log2 units
  auto tile_max = [&](Sacc& acc, int t0, bool edge, float (&mt)[2]) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      if (edge) {
        // key t0 + 8 lg + c is visible iff c < rel (c a constant per slot)
        const int rel = klim[j] - t0 - 8 * lg;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            acc[j][kb][r] = 32 * (kb >> 1) + 4 * (kb & 1) + r < rel ? acc[j][kb][r] : -INFINITY;
      }
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) mx = fmaxf(mx, acc[j][kb][r]);
      mt[j] = max_lg(mx) * sc;
    }
  };
  // raise the reference maximum where a tile's maximum exceeds it by more
  // than 2^8, rescaling the running state (rare)
  auto rescale = [&](const float (&mt)[2]) {
    const bool need = mt[0] > m_ref[0] + 8.0f || mt[1] > m_ref[1] + 8.0f;
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
  };
  // O^T += V^T P^T and the row sums (all-ones A operand), V^T fragments read
  // four at a time one group ahead.  WithMax: the (unmasked) maximum of the
  // next tile's scores `nxt` is taken in the same block.
  auto pv_tile = [&](const bf16_t* Vs, const Pk& pk, auto with_max, Sacc& nxt, float (&mt)[2]) {
    constexpr bool WithMax = decltype(with_max)::value;
    constexpr int NG = 2 * DB / 4;  // groups of 4 fragments: (ks2, 4 d blocks)
    uint4 vfr[2][4];
#pragma unroll
    for (int i = 0; i < 4; ++i) vfr[0][i] = *reinterpret_cast<const uint4*>(Vs + i * 2 * 512 + lane * 8);
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
      const int ks2 = gi / (DB / 4), db0 = (gi % (DB / 4)) * 4;
      if (gi + 1 < NG) {
        const int ks2n = (gi + 1) / (DB / 4), db0n = ((gi + 1) % (DB / 4)) * 4;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          vfr[(gi + 1) & 1][i] = *reinterpret_cast<const uint4*>(Vs + ((db0n + i) * 2 + ks2n) * 512 + lane * 8);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const uint4 pf = make_uint4(pk[j][ks2][0], pk[j][ks2][1], pk[j][ks2][2], pk[j][ks2][3]);
          oacc[j][db0 + i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_v, vfr[gi & 1][i]),
                                                                      __builtin_bit_cast(bf16x8_v, pf),
                                                                      oacc[j][db0 + i], 0, 0, 0);
        }
      if (db0 + 4 == DB) {  // last d group of this key step: the row sums
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const uint4 pf = make_uint4(pk[j][ks2][0], pk[j][ks2][1], pk[j][ks2][2], pk[j][ks2][3]);
          lacc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_v, ones),
                                                             __builtin_bit_cast(bf16x8_v, pf), lacc[j], 0, 0, 0);
        }
      }
      if (gi == 0) __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);  // DS read
      if (gi + 1 < NG) __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
      const int nm = db0 + 4 == DB ? 10 : 8;
      if constexpr (WithMax) {
#pragma unroll
        for (int m = 0; m < 8; ++m) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
          __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);  // VALU
        }
        if (nm == 10) __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      } else {
        if (nm == 10)
          __builtin_amdgcn_sched_group_barrier(0x008, 10, 0);  // MFMA (with the row sums)
        else
          __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
      }
    }
    if constexpr (WithMax) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r) mx = fmaxf(mx, nxt[j][kb][r]);
        mt[j] = max_lg(mx) * sc;
      }
    }
  };

  const int ntiles = k1 > k0 ? (k1 - k0 + KT - 1) / KT : 0;
  // tiles that need the mask: past the split's end, or canvas keys (from key
  // Lw on) under the causal mask; they all come after the ones that do not
  auto edge = [&](int t0) { return t0 + KT > k1 || (a.causal && t0 + KT > Lw); };
  const int klast = a.causal ? min(k1, Lw) : k1;
  const int n_main = klast > k0 ? min(ntiles, (klast - k0) / KT) : 0;  // leading unmasked tiles

  // Tile i lives in stage i % 4.  A step waits for the copies of a tile and
  // then passes a barrier; each wave waits until its own copies of that tile
  // have landed, and as the vector memory counter drains in issue order it is
  // enough to allow the copies of the later tiles issued so far (at most
  // two) to remain outstanding.  A tile staged through registers leaves
  // nothing outstanding and has already drained the copies before it, so the
  // counts never wait too little.  The wait and the barrier sit in one asm
  // statement (a __syncthreads() would add a release fence, which drains
  // every copy); lgkmcnt(0) publishes register-staged stores to LDS.
  auto sync_tile = [&](int i, int issued) {
    const int later = issued - 1 - i;
    if (later >= 2)
      asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(2 * CPW) : "memory");
    else if (later == 1)
      asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(CPW) : "memory");
    else
      asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  };
  constexpr int VB = NKB * 512;  // V^T blocks of a stage
  // a stage chosen at run time (the masked tail only: reads through such a
  // pointer are not known to avoid the copies in flight, so they wait for all)
  auto stage = [&](int i) -> bf16_t* {
    const int r = i & 3;
    return r == 0 ? S0 : r == 1 ? S1 : r == 2 ? S2 : S3;
  };

  // Software pipeline over the unmasked tiles: step t waits for tile t + 1,
  // refills the stage of tile t - 1 with tile t + 3, then computes S(t + 1)
  // while forming P(t), and O += P(t) V(t) while taking the maximum of
  // S(t + 1).
  Sacc cur, nxt;
  Pk pk;
  float mt[2] = {-INFINITY, -INFINITY};
  if (ntiles > 0) issue(S0, S0 + VB, k0);
  if (ntiles > 1) issue(S1, S1 + VB, k0 + KT);
  if (ntiles > 2) issue(S2, S2 + VB, k0 + 2 * KT);
  if (ntiles > 0) sync_tile(0, min(3, ntiles));
  if (n_main > 0) {
    s_tile(S0, cur, no{}, cur, pk);
    tile_max(cur, k0, false, mt);
  }
  auto pipe_step = [&](const bf16_t* Vt, const bf16_t* Kn, bf16_t* Is, int t) {
    sync_tile(t + 1, min(t + 3, ntiles));
    if (t + 3 < ntiles) issue(Is, Is + VB, k0 + (t + 3) * KT);
    rescale(mt);
    s_tile(Kn, nxt, yes{}, cur, pk);
    pv_tile(Vt, pk, yes{}, nxt, mt);
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) cur[j][kb] = nxt[j][kb];
  };
  for (int t = 0; t + 1 < n_main; t += 4) {
    pipe_step(S0 + VB, S1, S3, t);
    if (t + 2 >= n_main) break;
    pipe_step(S1 + VB, S2, S0, t + 1);
    if (t + 3 >= n_main) break;
    pipe_step(S2 + VB, S3, S1, t + 2);
    if (t + 4 >= n_main) break;
    pipe_step(S3 + VB, S0, S2, t + 3);
  }
  if (n_main > 0) {  // the last unmasked tile: its scores are in `cur`
    const int t = n_main - 1;
    sync_tile(t + 1, min(t + 3, ntiles));
    if (t + 3 < ntiles) issue(stage(t + 3), stage(t + 3) + VB, k0 + (t + 3) * KT);
    rescale(mt);
    p_tile(cur, pk);
    pv_tile(stage(t) + VB, pk, no{}, nxt, mt);
  }
  for (int t = n_main; t < ntiles; ++t) {  // masked tiles, one at a time
    sync_tile(t + 1, min(t + 3, ntiles));
    if (t + 3 < ntiles) issue(stage(t + 3), stage(t + 3) + VB, k0 + (t + 3) * KT);
    const int t0 = k0 + t * KT;
    s_tile(stage(t), cur, no{}, cur, pk);
    tile_max(cur, t0, edge(t0), mt);
    rescale(mt);
    p_tile(cur, pk);
    pv_tile(stage(t) + VB, pk, no{}, nxt, mt);
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

// Key splits of canvas b for the direct-copy kernel (one workgroup per CU):
// enough (KV head x split x q-tile) workgroups to fill the chip's slots once,
// whole 64-key tiles, at least 256 keys per split, at most 64 splits.  The
// choice depends on the canvas alone, so a canvas's result does not depend on
// the batch it runs in.  The 256-key floor only moves the 1280-key
// sliding-window layers (10 splits of 128 -> 5 of 256): on one canvas it is
// neutral (attention + merge 26.6 -> 26.3 us per layer), on four it halves
// the fp32 partials the merge reads (112.3 -> 99.5 us per layer; a 512-key
// floor gave 89.4 there but 31.1 on one canvas).
static void choose_splits_fa(int total, int base, int* S_out, int* CL_out) {
  const int slots = 256;
  int S = (slots + base - 1) / base;
  S = min(S, max(1, (total + 63) / 64));
  S = min(S, 64);
  int CL = ((total + S - 1) / S + 63) / 64 * 64;
  if (CL < 256) CL = 256;
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
    const int QT = (a.Hq / a.Hkv * a.N + 255) / 256;
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
    hipError_t e = a.D == 128 ? launch_k(k_attn_fa<128>, grid, dim3(512), 0, st, t.start, stop1, a, QT, xcd_map)
                              : launch_k(k_attn_fa<64>, grid, dim3(512), 0, st, t.start, stop1, a, QT, xcd_map);
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
