// Skinny GEMMs on CDNA4 matrix cores: y = A @ W with A row-major activations
// (optionally row-gathered) and W pre-packed into MFMA B-fragment order.
//
// Every dense contraction of the pass runs here: the q/k/v projection with its
// RoPE epilogue, the output projection, the router, the grouped expert GEMMs
// (gate|up with the GELU-tanh gated product, down with the gate scale) and the
// tied LM head.  The decoder's GEMMs have few rows (256 canvas positions, ~16
// per routed expert) and are bound by streaming W from HBM, so the kernel is
// organised around the weight stream:
//
//   * W is packed as [N/16][K/32][64 lanes][8] so the 16x32 B fragment of one
//     16x16x32 bf16 MFMA is one contiguous 1 KB block: one 16-byte load per
//     lane, fully coalesced.  Each weight element is read exactly once per
//     m-chunk.
//   * A workgroup owns 4 waves x WN n-blocks of output columns and up to MT
//     m-tiles of 16 rows; the rows' A chunk (128 of K) is staged once in LDS and
//     shared by the 4 waves, while every wave streams its own W fragments
//     straight into registers with a one-chunk prefetch.
//   * Grouped mode (experts): workgroup (group, n-tile) loops over the rows the
//     router sent to that group (device-side offsets; empty experts exit at
//     once).  The shared expert's rows, whose count the host knows, are spread
//     over a fixed m-chunk grid instead.
//   * For the fixed grid, blocks that share an n-tile are mapped to the same XCD
//     (blocks are dispatched round-robin over the 8 XCDs) so the re-reads of a
//     W tile by other m-chunks hit that XCD's L2.
//
// fp32 workloads use the same packing and loop with 16x16x4 fp32 MFMAs (8 per
// 32-wide k-step); lanes feed matching k indices to A and B, so the sum is the
// plain dot product.
//
// Expert weights may instead be stored as MXFP4 (OCP microscaling: 4-bit E2M1
// elements sharing one E8M0 scale per 32 consecutive k of a column), the
// gfx950-native analogue of the 4-bit builds the pages list ([Experimental]
// and [ParadigmShift] "Serving in Production": GGUF Q4_K_M, NVFP4).  The
// stream then moves a quarter of the bytes: one 16-byte load per lane carries
// the fragments of four k-steps, and v_cvt_scalef32_pk_bf16_fp4 turns them back
// into exact bf16 fragments (every E2M1 value times a power of two is a bf16)
// for the same bf16 MFMAs, activations staying bf16.
#include "common.h"

namespace {

template <typename T> struct Frag;
template <> struct Frag<bf16_t> { uint4 v; };
template <> struct Frag<float> { float4 a, b; };

template <typename T> DG_DEV Frag<T> ld_frag(const T* p);
template <> DG_DEV Frag<bf16_t> ld_frag<bf16_t>(const bf16_t* p) {
  Frag<bf16_t> f;
  f.v = *reinterpret_cast<const uint4*>(p);
  return f;
}
template <> DG_DEV Frag<float> ld_frag<float>(const float* p) {
  Frag<float> f;
  f.a = reinterpret_cast<const float4*>(p)[0];
  f.b = reinterpret_cast<const float4*>(p)[1];
  return f;
}
template <typename T> DG_DEV void st_frag(T* p, const Frag<T>& f);
template <> DG_DEV void st_frag<bf16_t>(bf16_t* p, const Frag<bf16_t>& f) {
  *reinterpret_cast<uint4*>(p) = f.v;
}
template <> DG_DEV void st_frag<float>(float* p, const Frag<float>& f) {
  reinterpret_cast<float4*>(p)[0] = f.a;
  reinterpret_cast<float4*>(p)[1] = f.b;
}
template <typename T> DG_DEV Frag<T> zero_frag();
template <> DG_DEV Frag<bf16_t> zero_frag<bf16_t>() { Frag<bf16_t> f; f.v = make_uint4(0, 0, 0, 0); return f; }
template <> DG_DEV Frag<float> zero_frag<float>() {
  Frag<float> f; f.a = make_float4(0, 0, 0, 0); f.b = f.a; return f;
}

DG_DEV void mma(floatx4& c, const Frag<bf16_t>& a, const Frag<bf16_t>& b) {
  c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_v, a.v),
                                               __builtin_bit_cast(bf16x8_v, b.v), c, 0, 0, 0);
}
DG_DEV void mma(floatx4& c, const Frag<float>& a, const Frag<float>& b) {
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.a.x, b.a.x, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.a.y, b.a.y, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.a.z, b.a.z, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.a.w, b.a.w, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.b.x, b.b.x, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.b.y, b.b.y, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.b.z, b.b.z, c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.b.w, b.b.w, c, 0, 0, 0);
}

// One k-step's B fragment from MXFP4: the lane's 8 codes (element e in bits
// 4e..4e+3) times 2^(sbyte - 127), converted two at a time.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
DG_DEV Frag<bf16_t> dq_fp4(uint32_t w, uint32_t sbyte) {
  const float sc = __uint_as_float(sbyte << 23);
  Frag<bf16_t> f;
  f.v.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 0));
  f.v.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 1));
  f.v.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 2));
  f.v.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, sc, 3));
  return f;
}
DG_DEV uint32_t u4_at(const uint4& v, int j) { return j == 0 ? v.x : j == 1 ? v.y : j == 2 ? v.z : v.w; }

DG_DEV float gelu_tanh(float z) {
  const float k0 = 0.7978845608028654f;  // sqrt(2/pi)
  return 0.5f * z * (1.0f + tanhf(k0 * (z + 0.044715f * z * z * z)));
}

template <typename T> DG_DEV void st(void* base, long long off, float v) {
  reinterpret_cast<T*>(base)[off] = from_f<T>(v);
}

// Epilogue for one output row and lane column, WN consecutive n-blocks.
template <typename T, int WN, int EPI>
DG_DEV void epilogue(const EpiArgs& e, int row, int nb0, int nb_valid, int c, const float* v,
                     long long split_off = 0, const float2* rope = nullptr, const int* down_row = nullptr,
                     const float* down_gate = nullptr) {
  if constexpr (EPI == EPI_STORE_F32) {
    float* out = reinterpret_cast<float*>(e.out) + split_off;
#pragma unroll
    for (int w = 0; w < WN; ++w)
      if (w < nb_valid) out[(long long)row * e.ldo + (nb0 + w) * 16 + c] = v[w];
  } else if constexpr (EPI == EPI_DOWN) {
    const int orow = down_row ? *down_row : e.slot[row];
    if ((unsigned)orow >= (unsigned)e.out_rows) return;
    // shared-expert rows: weight 1
    const float g = down_gate ? *down_gate : (orow < e.routed_rows ? e.gates[orow] : 1.0f);
    float* out = reinterpret_cast<float*>(e.out);
#pragma unroll
    for (int w = 0; w < WN; ++w)
      if (w < nb_valid) out[(long long)orow * e.ldo + (nb0 + w) * 16 + c] = v[w] * g;
  } else if constexpr (EPI == EPI_GEGLU) {
    // n-block 2p holds gate columns, 2p+1 the up columns of the same outputs
#pragma unroll
    for (int p = 0; p < WN / 2; ++p) {
      if (2 * p + 1 >= nb_valid) break;  // pairs past the last n-block
      const int col = ((nb0 + 2 * p) >> 1) * 16 + c;
      st<T>(e.out, (long long)row * e.ldo + col, gelu_tanh(v[2 * p]) * v[2 * p + 1]);
    }
  } else if constexpr (EPI == EPI_QKV) {
    const int b = row / e.N, i = row - b * e.N;
    const int bph = e.D >> 4;  // 16-column blocks per head
#pragma unroll
    for (int p = 0; p < WN / 2; ++p) {
      if (2 * p + 1 >= nb_valid) break;  // pairs past the last n-block
      const int nb = nb0 + 2 * p;
      const int hs = nb / bph, w0 = nb - hs * bph;
      float x1 = v[2 * p], x2 = v[2 * p + 1];
      if (hs < e.Hq + e.Hkv) {
        // rotary pair (d, d + D/2) sits in the two n-blocks of this wave
        const int d = (w0 >> 1) * 16 + c;
        const int n_rot = e.is_global ? e.n_rot_global : e.n_rot_local;
        if (d < n_rot) {
          const float2 cs = rope ? rope[p] : e.rope_cs[((long long)row) * (e.D >> 1) + d];
          const float y1 = x1 * cs.x - x2 * cs.y;
          const float y2 = x2 * cs.x + x1 * cs.y;
          x1 = y1; x2 = y2;
        }
        if (hs < e.Hq) {
          const long long o = b * e.qs[0] + hs * e.qs[1] + i * e.qs[2];
          st<T>(e.q, o + d * e.qs[3], x1);
          st<T>(e.q, o + (d + (e.D >> 1)) * e.qs[3], x2);
        } else {
          const long long o = b * e.ks[0] + (hs - e.Hq) * e.ks[1] + i * e.ks[2];
          st<T>(e.k, o + d * e.ks[3], x1);
          st<T>(e.k, o + (d + (e.D >> 1)) * e.ks[3], x2);
        }
      } else {
        const int h = hs - e.Hq - e.Hkv;
        const int d = w0 * 16 + c;
        const long long o = b * e.vs[0] + h * e.vs[1] + i * e.vs[2];
        st<T>(e.v, o + d * e.vs[3], x1);
        st<T>(e.v, o + (d + 16) * e.vs[3], x2);
      }
    }
  }
}

template <typename T, int MT, int WN, int EPI>
__global__ __launch_bounds__(256) void k_gemm(GemmArgs g, EpiArgs e) {
  constexpr int KC = 4;                  // k-steps (of 32) per staged chunk
  constexpr int KCH = KC * 32;
  constexpr int ROWS = MT * 16;
  constexpr int VEC = 16 / sizeof(T);    // elements per 16-byte vector
  constexpr int LDS_LD = KCH + VEC;      // padded LDS row
  constexpr int VPR = KCH / VEC;         // vectors per row and chunk
  constexpr int VPT = ROWS * VPR / 256;  // vectors per thread
  static_assert(VPT * 256 == ROWS * VPR, "A chunk must split evenly over 256 threads");
  __shared__ __align__(16) T As[ROWS * LDS_LD];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int tiles = (g.NB + 4 * WN - 1) / (4 * WN);
  const int KB = g.K >> 5;
  const int NKC = (KB + KC - 1) / KC;

  // ---- block -> (group, n-tile, rows)
  int bid = blockIdx.x, group, tile, rs, re;
  bool dynamic_rows;
  const int smc = (g.static_rows + ROWS - 1) / ROWS;
  const int n_static = tiles * smc;
  if (bid < n_static) {
    int mc;
    if ((tiles & 7) == 0 && smc > 1) {
      const int xcd = bid & 7, slot = bid >> 3;
      tile = (slot / smc) * 8 + xcd;
      mc = slot % smc;
    } else {
      tile = bid / smc;
      mc = bid % smc;
    }
    group = g.static_group;
    rs = g.static_row0 + mc * ROWS;
    re = min(g.static_row0 + g.static_rows, rs + ROWS);
    dynamic_rows = false;
  } else {
    bid -= n_static;
    group = bid / tiles;
    tile = bid - group * tiles;
    rs = g.group_off[group];
    re = g.group_off[group + 1];
    dynamic_rows = true;
  }
  if (rs >= re) return;  // block-uniform: no rows for this expert

  const T* __restrict__ A = reinterpret_cast<const T*>(g.A);
  const T* __restrict__ Bg = reinterpret_cast<const T*>(g.B) + (long long)group * g.b_group_stride;
  const int nb0 = tile * 4 * WN + wave * WN;
  const int nb_valid = g.NB - nb0;  // wave-uniform; <= 0 means this wave has no columns
  const int c = lane & 15, rg = (lane >> 4) * 4;

  for (int row0 = rs; row0 < re; row0 += ROWS) {
    const int row_end = min(re, row0 + ROWS);
    const int act_mt = (row_end - row0 + 15) >> 4;
    floatx4 acc[MT][WN];
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int w = 0; w < WN; ++w) acc[m][w] = floatx4{0.f, 0.f, 0.f, 0.f};

    uint4 areg[VPT];
    auto loadA = [&](int kc) {
#pragma unroll
      for (int v = 0; v < VPT; ++v) {
        const int idx = tid + v * 256;
        const int rr = idx / VPR, cv = idx - rr * VPR;
        const int r = row0 + rr, k0 = kc * KCH + cv * VEC;
        uint4 val = make_uint4(0, 0, 0, 0);
        if (r < row_end && k0 < g.K) {
          long long ar = r;
          if (g.a_rows) {
            ar = g.a_rows[r];
            ar = ar < 0 ? 0 : (ar >= g.a_rows_max ? g.a_rows_max - 1 : ar);
          }
          val = *reinterpret_cast<const uint4*>(A + ar * g.lda + k0);
        }
        areg[v] = val;
      }
    };
    auto storeA = [&]() {
#pragma unroll
      for (int v = 0; v < VPT; ++v) {
        const int idx = tid + v * 256;
        const int rr = idx / VPR, cv = idx - rr * VPR;
        *reinterpret_cast<uint4*>(&As[rr * LDS_LD + cv * VEC]) = areg[v];
      }
    };
    Frag<T> bcur[KC][WN], bnext[KC][WN];
    auto loadB = [&](int kc, Frag<T> (&bf)[KC][WN]) {
#pragma unroll
      for (int ks = 0; ks < KC; ++ks) {
        const int kb = kc * KC + ks;
#pragma unroll
        for (int w = 0; w < WN; ++w) {
          if (kb < KB && w < nb_valid)
            bf[ks][w] = ld_frag<T>(Bg + ((long long)(nb0 + w) * KB + kb) * 512 + lane * 8);
          else
            bf[ks][w] = zero_frag<T>();
        }
      }
    };

    loadA(0);
    loadB(0, bcur);
    storeA();
    __syncthreads();
    for (int kc = 0; kc < NKC; ++kc) {
      const bool more = kc + 1 < NKC;
      if (more) {
        loadA(kc + 1);
        loadB(kc + 1, bnext);
      }
      const int nks = min(KC, KB - kc * KC);
      if (nb_valid > 0) {
#pragma unroll
        for (int ks = 0; ks < KC; ++ks) {
          if (ks < nks) {
#pragma unroll
            for (int m = 0; m < MT; ++m) {
              if (m < act_mt) {
                const Frag<T> a = ld_frag<T>(&As[(m * 16 + c) * LDS_LD + ks * 32 + (lane >> 4) * 8]);
#pragma unroll
                for (int w = 0; w < WN; ++w) mma(acc[m][w], a, bcur[ks][w]);
              }
            }
          }
        }
      }
      __syncthreads();
      if (more) {
        storeA();
#pragma unroll
        for (int ks = 0; ks < KC; ++ks)
#pragma unroll
          for (int w = 0; w < WN; ++w) bcur[ks][w] = bnext[ks][w];
      }
      __syncthreads();
    }

    mfma_drain();
    if (nb_valid > 0) {
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        if (m < act_mt) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int row = row0 + m * 16 + rg + r;
            if (row < row_end) {
              float v[WN];
#pragma unroll
              for (int w = 0; w < WN; ++w) v[w] = acc[m][w][r];
              epilogue<T, WN, EPI>(e, row, nb0, nb_valid, c, v);
            }
          }
        }
      }
    }
    if (!dynamic_rows) break;
  }
}

// ----------------------------------------------------------------------------
// Streaming GEMM: one workgroup per (work entry of <= 16*MT rows, n-tile of
// 4*WN n-blocks), 4 waves, each wave MT row tiles x WN n-blocks.
//
// Each wave streams the W fragments of its WN n-blocks through an R-deep
// register ring: the load of k-step kb+R is issued as soon as k-step kb is
// consumed, so every wave keeps R*WN KB of weights in flight for the whole of
// K.  The ring's first loads go out before anything else, so the weight
// stream is under way while A is staged.  The entry's A rows are staged into
// LDS in MFMA A-fragment order, [k-step][row tile][64 lanes][8] (every lane
// reads its own 16 contiguous bytes) within an LDS budget of LK KB, copied
// straight from global memory into LDS (bf16; double-buffered half chunks
// when K needs more than one chunk); the ring runs on across chunk boundaries
// (weights do not depend on A).  Loads in the k loop are unconditional so the
// compiler's wait counts stay exact; k-steps past the end use a zero A
// fragment and clamped refills.
//
// Entries come either from a dense row range or from the router's work list
// (expert, first row, end row), in which heavy experts are split into several
// entries that run in parallel.  Blocks are ordered tile-major over (tile,
// entry) and every XCD (blockIdx & 7) takes a contiguous slice, so the entries
// of one expert run back to back on one XCD and share that expert's W tile
// through its L2.  Wider entries (MT = 2, or 4 with many rows) cut the weight
// reads of dense GEMMs and of experts with more rows than one tile.
// ----------------------------------------------------------------------------
// LDS budget of the A staging, in KB: 32 keeps three 32-row workgroups per CU;
// a grid of at most one workgroup per CU (the dense projections of one canvas)
// takes 128 and stages the whole K range of its rows at once.
constexpr int kStreamLdsKB = 32, kStreamLdsWideKB = 128;

template <typename T, int MT, int R, int LK>
constexpr int stream_kc() { return (LK * 1024 / (16 * MT * 32 * (int)sizeof(T))) / R * R; }  // k-steps per chunk

template <typename T, int MT, int WN, int EPI, int R, int LK, int QB = 0>
__global__ __launch_bounds__(256) void k_stream(StreamArgs g, EpiArgs e) {
  constexpr int ROWS = 16 * MT;
  constexpr int KC = stream_kc<T, MT, R, LK>();
  static_assert(KC % R == 0, "the register ring must tile an A chunk");
  // MXFP4: every ring slot holds four k-steps, so chunks hold whole rounds of the ring
  static_assert(QB == 0 || (sizeof(T) == 2 && KC % (4 * R) == 0), "MXFP4 ring rounds must tile an A chunk");
  static_assert(EPI != EPI_DOWN || sizeof(T) != 2 || 4 * ROWS * 16 * WN * 4 <= LK * 1024,
                "the down output tiles must fit the LDS budget");
  extern __shared__ __align__(16) unsigned char smem_raw[];
  T* As = reinterpret_cast<T*>(smem_raw);  // [KC][MT][64][8]
  __shared__ int s_rows[ROWS];
  __shared__ int s_orow[EPI == EPI_DOWN ? ROWS : 1];  // down: output slot of each entry row
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int tiles = (g.NB + 4 * WN - 1) / (4 * WN);
  const int ksplit = g.ksplit > 1 ? g.ksplit : 1;
  int group, rs, re, tile, ks = 0;
  if (g.ent_off) {
    // router work list, expert-major: (expert, tile, entry of the expert), so
    // the entries of one expert share each weight tile through L2 and one
    // entry's A rows are re-staged for consecutive tiles while still in L2.
    // Items are counted on the device and cut into 8 XCD slices.
    const int nw = min(*g.work_count, g.work_cap);
    const long long P = (long long)tiles * nw;
    const long long Q = (P + 7) >> 3, r = blockIdx.x >> 3;
    const long long p = (long long)(blockIdx.x & 7) * Q + r;
    if (r >= Q || p >= P) return;
    int lo = 0, hi = g.n_groups;  // largest e with tiles * ent_off[e] <= p
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if ((long long)tiles * g.ent_off[mid] <= p) lo = mid; else hi = mid;
    }
    const int base = g.ent_off[lo], ne = g.ent_off[lo + 1] - base;
    const long long u = p - (long long)tiles * base;
    tile = (int)(u / ne);
    const int4 en = g.work[base + (int)(u - (long long)tile * ne)];
    group = en.x; rs = en.y; re = min(en.z, en.y + ROWS);
  } else {
    const int J = g.n_dense + g.work_cap;
    const long long P = (long long)tiles * J * ksplit;
    const long long Q = (P + 7) >> 3;
    const long long p = (long long)(blockIdx.x & 7) * Q + (blockIdx.x >> 3);
    if (p >= P) return;
    ks = (int)(p % ksplit);
    const long long pp = p / ksplit;
    tile = (int)(pp / J);
    const int j = (int)(pp - (long long)tile * J);
    if (j < g.n_dense) {
      group = g.dense_group;
      rs = g.dense_row0 + j * ROWS;
      re = min(g.dense_row0 + g.dense_rows, rs + ROWS);
    } else {
      const int w = j - g.n_dense;
      if (w >= *g.work_count) return;
      const int4 en = g.work[w];
      group = en.x; rs = en.y; re = min(en.z, en.y + ROWS);
    }
  }
  if (rs >= re) return;
  const int KBall = g.K >> 5;
  const int KB = KBall / ksplit;  // k-steps of this split
  const int kbase = ks * KB;

  // ---- A row indices (rows past the entry repeat its last row; those output
  // rows are never stored, and an MFMA row depends only on its own A row).
  // The gather index load goes out ahead of the W ring so that its wait does
  // not also wait for the ring.
  int ar = min(rs + tid, re - 1), a_max = 0x7fffffff;
  if (tid < ROWS && g.a_rows) {
    ar = g.a_rows[ar];
    a_max = g.a_rows_max;
  }
  // down: output slot of each of this lane's rows, fetched early like the
  // gather index (its gate follows once the slot is known)
  constexpr int DM = EPI == EPI_DOWN ? MT : 1;
  int dslot[DM][4];
  int orow_t = 0;
  if constexpr (EPI == EPI_DOWN) {
    if (tid < ROWS) orow_t = e.slot[min(rs + tid, re - 1)];
    const int rg = (lane >> 4) * 4;
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int r = 0; r < 4; ++r) dslot[m][r] = e.slot[min(rs + m * 16 + rg + r, re - 1)];
  }

  // ---- W ring prologue
  const T* __restrict__ Bg = reinterpret_cast<const T*>(g.B) + (long long)group * g.b_group_stride;
  const int nb0 = tile * 4 * WN + wave * WN;
  const int nbv = g.NB - nb0;  // wave-uniform count of valid n-blocks (others computed, not stored)
  const T* bptr[WN];
#pragma unroll
  for (int w = 0; w < WN; ++w) {
    const int nb = min(nb0 + w, g.NB - 1);
    bptr[w] = Bg + ((long long)nb * KBall + kbase) * 512 + lane * 8;
  }
  Frag<T> b[QB ? 1 : R][WN];
  // MXFP4: slot i of the ring holds k-steps 4i..4i+3 of its round (codes, scales)
  constexpr int RQ = QB ? R : 1;
  const int KG = (KBall + 3) >> 2;
  const uint4* qptr[WN];
  const uint32_t* sptr[WN];
  uint4 bq[RQ][WN];
  uint32_t bsc[RQ][WN];
  if constexpr (QB == 0) {
#pragma unroll
    for (int i = 0; i < R; ++i)
#pragma unroll
      for (int w = 0; w < WN; ++w) b[i][w] = ld_frag<T>(bptr[w] + (long long)min(i, KB - 1) * 512);
  } else {
    const uint4* Bq = g.Bq + (long long)group * g.bq_group_stride;
    const uint32_t* Bs = g.Bs + (long long)group * g.bs_group_stride;
#pragma unroll
    for (int w = 0; w < WN; ++w) {
      const int nb = min(nb0 + w, g.NB - 1);
      qptr[w] = Bq + (long long)nb * KG * 64 + lane;
      sptr[w] = Bs + (long long)nb * KG * 16 + (lane & 15);
    }
#pragma unroll
    for (int i = 0; i < RQ; ++i)
#pragma unroll
      for (int w = 0; w < WN; ++w) {
        const int kg = min(i, KG - 1);
        bq[i][w] = qptr[w][(long long)kg * 64];
        bsc[i][w] = sptr[w][(long long)kg * 16];
      }
  }

  if (tid < ROWS) {
    ar = ar < 0 ? 0 : (ar >= a_max ? a_max - 1 : ar);
    s_rows[tid] = ar;
    if constexpr (EPI == EPI_DOWN) s_orow[tid] = orow_t;
  }

  float dgate[DM][4];
  if constexpr (EPI == EPI_DOWN) {
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int orow = dslot[m][r];
        dgate[m][r] = (unsigned)orow < (unsigned)e.routed_rows ? e.gates[orow] : 1.0f;
      }
  }

  // RoPE (cos, sin) of this lane's output rows and rotary columns, fetched now
  // so the epilogue does not wait on a load
  constexpr int NP = EPI == EPI_QKV ? WN / 2 : 1;
  float2 rope[MT][4][NP];
  if constexpr (EPI == EPI_QKV) {
    const int c = lane & 15, rg = (lane >> 4) * 4, bph = e.D >> 4;
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const int nb = min(nb0 + 2 * p, g.NB - 1);
      const int hs = nb / bph, d = ((nb - hs * bph) >> 1) * 16 + c;
      const int dd = min(d, (e.D >> 1) - 1);  // columns past the rotary half are never used
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = min(rs + m * 16 + rg + r, re - 1);
          rope[m][r][p] = e.rope_cs[(long long)row * (e.D >> 1) + dd];
        }
    }
  }

  floatx4 acc[MT][WN];
#pragma unroll
  for (int m = 0; m < MT; ++m)
#pragma unroll
    for (int w = 0; w < WN; ++w) acc[m][w] = floatx4{0.f, 0.f, 0.f, 0.f};

  const T* __restrict__ A = reinterpret_cast<const T*>(g.A) + kbase * 32;
  // bf16: each lane's A source row for every row tile (lane l feeds row l % 16 of
  // the tile at k offset 8 * (l / 16) of each k-step)
  const T* arow[MT];
  if constexpr (sizeof(T) == 2) {
    __syncthreads();  // row indices written
#pragma unroll
    for (int m = 0; m < MT; ++m) arow[m] = A + (long long)s_rows[m * 16 + (lane & 15)] * g.lda + (lane >> 4) * 8;
  }
  // bf16 A: the rows of a chunk are copied straight from global memory into
  // LDS in fragment order, one 1 KB fragment block (k-step, row tile) per wave
  // instruction, all in flight at once and no registers held.  When K needs
  // more than one chunk, the LDS budget holds two chunks of KC / 2 k-steps and
  // chunk c + 1 is copied while chunk c is consumed.  The copies are asm, out
  // of the compiler's sight: its wait bookkeeping cannot tell the buffers
  // apart and put a full drain of the vector memory counter before every
  // chunk, emptying the weight ring.  The explicit wait closing a chunk covers
  // them instead: the counter drains in issue order, and only the chunk's
  // NREF weight refills are issued after its successor's copies.  (The
  // compiler's own waits for the ring count those copies as ops it does not
  // know of, so right after them such a wait is stricter than it needs to be
  // by up to the chunk's copies: a small cost against the drain.)  Measured:
  // one canvas gate|up 95.6 -> 94.9 us, MXFP4 gate|up 44.5 -> 42.6 us; four
  // canvases (64-row entries) gate|up 168.3 -> 163.5 us, the pass 16.20 ->
  // 15.92 ms.
  constexpr bool DBUF = sizeof(T) == 2;
  constexpr int KCH = DBUF ? KC / 2 : KC;  // k-steps per chunk when double-buffered
  static_assert(!DBUF || (QB ? KCH % (4 * R) == 0 : KCH % R == 0), "a half chunk must hold whole rounds of the ring");
  constexpr int NREF_ALL = QB ? (KCH / 4) * WN * 2 : KCH * WN;  // refills of one full chunk
  constexpr int NREF = NREF_ALL < 63 ? NREF_ALL : 63;             // fewer is stricter, never wrong
  const bool dbuf = DBUF && KB > KC;
  const int CK = dbuf ? KCH : KC;  // k-steps per chunk
  // fragment block q = (k-step kl, row tile m) sits at q = kl * MT + m; wave w
  // copies the blocks q = w (mod 4), i.e. row tile w % MT of the k-steps
  // kl = w / MT (mod 4 / MT), so each wave needs one source row pointer
  static_assert(4 % MT == 0, "four waves share a chunk's row tiles evenly");
  const T* crow = nullptr;
  if constexpr (sizeof(T) == 2) {
    crow = arow[0];
#pragma unroll
    for (int mm = 1; mm < MT; ++mm)
      if (wave % MT == mm) crow = arow[mm];
  }
  auto copy_chunk = [=](int buf, int k0, int nk) {
    if constexpr (sizeof(T) == 2) {
      T* dst = As + buf * KCH * MT * 512 + (wave % MT) * 512;
      for (int kl = wave / MT; kl < nk; kl += 4 / MT) {
        const T* src = crow + (k0 + kl) * 32;
        const uint32_t lds = (uint32_t)(size_t)((__attribute__((address_space(3))) T*)(dst + kl * MT * 512));
        // the s_nop is the wait state a copy to LDS needs after M0 is written
        asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "{m0}"(lds) : "memory");
      }
    }
  };
  if constexpr (sizeof(T) == 2) {
    copy_chunk(0, 0, min(CK, KB));
    // the first chunk and the ring's first loads (issued before it) both land here
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  }
  for (int kc0 = 0, c = 0; kc0 < KB; kc0 += CK, ++c) {
    const int nk = min(CK, KB - kc0);  // k-steps in this chunk (< CK only in the last one)
    if constexpr (sizeof(T) == 2) {
      // (one chunk when !dbuf, copied above) its buffer was last read in chunk
      // c - 1, before the barrier that closed it
      if (dbuf && kc0 + CK < KB) copy_chunk((c + 1) & 1, kc0 + CK, min(CK, KB - kc0 - CK));
    } else {
      __syncthreads();  // row indices written / previous chunk consumed
      const int k8s = nk * 4;          // 8-element groups per row within the chunk
      const int groups8 = ROWS * k8s;
      constexpr int U = 4;  // fp32: loads in flight, bounded by the ring's registers
      for (int base = tid; base < groups8; base += 256 * U) {
        Frag<T> v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int q = min(base + u * 256, groups8 - 1);  // a repeated group rewrites the same value
          const int r = q / k8s, k8 = q - r * k8s;          // consecutive threads read along a row
          v[u] = ld_frag<T>(A + (long long)s_rows[r] * g.lda + (kc0 * 4 + k8) * 8);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int q = min(base + u * 256, groups8 - 1);
          const int r = q / k8s, k8 = q - r * k8s;
          st_frag<T>(As + (((k8 >> 2) * MT + (r >> 4)) * 64 + (r & 15) + 16 * (k8 & 3)) * 8, v[u]);
        }
      }
      __syncthreads();
    }
    // One branch-free loop over this chunk in groups of R k-steps.  Keeping the
    // accumulators in one loop with no peeled tail also keeps them in place: a
    // peeled tail made the register allocator copy them out of the accumulator
    // registers right behind the last MFMA, and those reads returned values
    // the MFMA had not yet written.
    const T* Ap = As + (dbuf ? (c & 1) * KCH * MT * 512 : 0) + lane * 8;
    if constexpr (QB == 0) {
      for (int kb0 = kc0; kb0 < kc0 + nk; kb0 += R) {
#pragma unroll
        for (int i = 0; i < R; ++i) {
          const int kb = kb0 + i;
          const int kl = min(kb - kc0, nk - 1);
          Frag<T> a[MT];
#pragma unroll
          for (int m = 0; m < MT; ++m) {
            a[m] = ld_frag<T>(Ap + (kl * MT + m) * 512);
            if (kb >= kc0 + nk) a[m] = zero_frag<T>();
          }
#pragma unroll
          for (int m = 0; m < MT; ++m)
#pragma unroll
            for (int w = 0; w < WN; ++w) mma(acc[m][w], a[m], b[i][w]);
          const int kn = min(kb + R, KB - 1);
#pragma unroll
          for (int w = 0; w < WN; ++w) b[i][w] = ld_frag<T>(bptr[w] + (long long)kn * 512);
        }
      }
    } else {
      // rounds of R slots x 4 k-steps; chunk starts are multiples of 4R, so slot
      // i always holds k-group (kb0 / 4) + i; k-steps past K meet a zero A
      // fragment (and zero codes in the padded k-group)
      for (int kb0 = kc0; kb0 < kc0 + nk; kb0 += 4 * RQ) {
#pragma unroll
        for (int i = 0; i < RQ; ++i) {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int kb = kb0 + 4 * i + j;
            const int kl = min(kb - kc0, nk - 1);
            Frag<T> a[MT];
#pragma unroll
            for (int m = 0; m < MT; ++m) {
              a[m] = ld_frag<T>(Ap + (kl * MT + m) * 512);
              if (kb >= kc0 + nk) a[m] = zero_frag<T>();
            }
#pragma unroll
            for (int w = 0; w < WN; ++w) {
              const Frag<bf16_t> bw = dq_fp4(u4_at(bq[i][w], j), (bsc[i][w] >> (8 * j)) & 0xFFu);
#pragma unroll
              for (int m = 0; m < MT; ++m) mma(acc[m][w], a[m], bw);
            }
          }
          const int kgn = min((kb0 >> 2) + i + RQ, KG - 1);
#pragma unroll
          for (int w = 0; w < WN; ++w) {
            bq[i][w] = qptr[w][(long long)kgn * 64];
            bsc[i][w] = sptr[w][(long long)kgn * 16];
          }
        }
      }
    }
    // bf16, more than one chunk: this chunk's LDS reads done and the next
    // chunk landed, in every wave
    if constexpr (sizeof(T) == 2)
      if (dbuf) asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(NREF) : "memory");
  }
  mfma_drain();
  if constexpr (EPI == EPI_DOWN && sizeof(T) == 2) {
    // down: the gate-scaled tile goes through LDS (each wave its own ROWS x
    // 16*WN fp32 block, 16-column groups XOR-swizzled by row quad against bank
    // conflicts) so that every lane stores 16 contiguous bytes of a row
    constexpr int TC = 16 * WN, Q = TC / 4, RPI = 64 / Q;
    static_assert((WN & (WN - 1)) == 0 && 64 % Q == 0 && ROWS % RPI == 0, "down tile shape");
    float* tl = reinterpret_cast<float*>(smem_raw) + wave * ROWS * TC;
    __syncthreads();  // every wave is done with the A chunk
    {
      const int c = lane & 15, rg = (lane >> 4) * 4;
#pragma unroll
      for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int tr = m * 16 + rg + r;
#pragma unroll
          for (int w = 0; w < WN; ++w) tl[tr * TC + (w ^ ((tr >> 2) & (WN - 1))) * 16 + c] = acc[m][w][r] * dgate[m][r];
        }
    }
    __syncthreads();
    float* out = reinterpret_cast<float*>(e.out);
    const int q = lane % Q;
#pragma unroll
    for (int i = 0; i < ROWS / RPI; ++i) {
      const int tr = i * RPI + lane / Q;
      const int orow = s_orow[tr];
      if (rs + tr < re && (q >> 2) < nbv && (unsigned)orow < (unsigned)e.out_rows) {
        const float4 val = *reinterpret_cast<const float4*>(tl + tr * TC + (((q >> 2) ^ ((tr >> 2) & (WN - 1))) * 16) +
                                                            (q & 3) * 4);
        *reinterpret_cast<float4*>(out + (long long)orow * e.ldo + nb0 * 16 + q * 4) = val;
      }
    }
  } else if (nbv > 0) {
    const int c = lane & 15, rg = (lane >> 4) * 4;
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = rs + m * 16 + rg + r;
        if (row < re) {
          float v[WN];
#pragma unroll
          for (int w = 0; w < WN; ++w) v[w] = acc[m][w][r];
          if constexpr (EPI == EPI_DOWN)
            epilogue<T, WN, EPI>(e, row, nb0, nbv, c, v, 0, nullptr, &dslot[m][r], &dgate[m][r]);
          else
            epilogue<T, WN, EPI>(e, row, nb0, nbv, c, v, ks * g.split_stride, rope[m][r]);
        }
      }
  }
}

// workgroups of the streaming GEMM for g, 4*WN n-blocks per tile
template <int WN>
long long stream_blocks(const StreamArgs& g) {
  const int tiles = (g.NB + 4 * WN - 1) / (4 * WN);
  const int ksplit = g.ksplit > 1 ? g.ksplit : 1;
  const long long P = (long long)tiles * (g.n_dense + g.work_cap) * ksplit;
  return ((P + 7) >> 3) << 3;
}

int device_cus() {
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cus[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cus[dev] = n;
  }
  return cus[dev];
}

template <typename T, int MT, int WN, int EPI, int R, int LK, int QB = 0>
hipError_t run_stream(const StreamArgs& g, const EpiArgs& e, hipStream_t s, KTime t) {
  const int ksplit = g.ksplit > 1 ? g.ksplit : 1;
  if (((g.K >> 5) % ksplit) != 0 || (ksplit > 1 && EPI != EPI_STORE_F32)) return hipErrorInvalidValue;
  if (QB && (ksplit > 1 || !g.Bq || !g.Bs)) return hipErrorInvalidValue;
  if (g.ent_off && (ksplit > 1 || g.n_dense > 0 || g.n_groups < 1)) return hipErrorInvalidValue;
  const long long blocks = stream_blocks<WN>(g);
  if (blocks <= 0) return hipSuccess;
  const int KB = (g.K >> 5) / ksplit;
  size_t lds = (size_t)16 * MT * min(KB, stream_kc<T, MT, R, LK>()) * 32 * sizeof(T);
  // bf16 down: the 4 waves' fp32 output tiles reuse the A chunk's LDS
  if (EPI == EPI_DOWN && sizeof(T) == 2) lds = max(lds, (size_t)4 * 16 * MT * 16 * WN * sizeof(float));
  // the chunk plus the kernel's static LDS
  hipError_t err = ensure_lds_limit(reinterpret_cast<const void*>(&k_stream<T, MT, WN, EPI, R, LK, QB>), LK * 1024);
  if (err != hipSuccess) return err;
  return launch_k(k_stream<T, MT, WN, EPI, R, LK, QB>, dim3((unsigned)blocks), dim3(256), lds, s, t.start, t.stop,
                  g, e);
}

// dense projections (q/k/v, output projection, router): the whole K range in
// one chunk when the grid leaves at most one workgroup per CU
template <typename T, int MT, int EPI>
hipError_t run_stream_dense(const StreamArgs& g, const EpiArgs& e, hipStream_t s, KTime t) {
  if constexpr (sizeof(T) == 2) {
    if (stream_blocks<2>(g) <= device_cus()) return run_stream<T, MT, 2, EPI, 8, kStreamLdsWideKB>(g, e, s, t);
  }
  return run_stream<T, MT, 2, EPI, 8, kStreamLdsKB>(g, e, s, t);
}

template <typename T, int MT>
hipError_t run_stream_mt(const StreamArgs& g, const EpiArgs& e, hipStream_t s, KTime t) {
  if (g.qb) {
    // MXFP4 experts: a ring slot holds four k-steps in a quarter of the bytes.
    // gate|up: 4 n-blocks per wave (half the tiles, so each entry's A rows are
    // re-staged half as often) and 2 slots (8 KB per wave in flight); measured
    // on the 30-layer workload: 43.9 us against 46.3 (2 n-blocks, 4 slots),
    // 52-57 us with deeper rings or 64 KB A chunks.  down: 2 slots of 4 n-blocks.
    if constexpr (sizeof(T) == 2) {
      if (e.kind == EPI_GEGLU) return run_stream<T, MT, 4, EPI_GEGLU, 2, kStreamLdsKB, 1>(g, e, s, t);
      if (e.kind == EPI_DOWN)
        return run_stream<T, MT, (MT == 2 ? 4 : 2), EPI_DOWN, (MT == 2 ? 2 : 4), kStreamLdsKB, 1>(g, e, s, t);
    }
    return hipErrorInvalidValue;
  }
  switch (e.kind) {
    case EPI_STORE_F32: return run_stream_dense<T, MT, EPI_STORE_F32>(g, e, s, t);
    case EPI_GEGLU: return run_stream<T, MT, 2, EPI_GEGLU, 8, kStreamLdsKB>(g, e, s, t);
    // down: K = F is short; 4 n-blocks per wave halve the A re-staging, and a
    // 2-deep ring streams fastest here (a deeper one spends its tail on
    // clamped repeat loads)
    case EPI_DOWN:
      return run_stream<T, MT, (MT == 2 ? 4 : 2), EPI_DOWN, (MT == 2 ? 2 : 8), kStreamLdsKB>(g, e, s, t);
    case EPI_QKV: return run_stream_dense<T, MT, EPI_QKV>(g, e, s, t);
  }
  return hipErrorInvalidValue;
}

// dense fp32-output projections over many rows (several canvases): row
// entries of 64 rows, so fewer entries re-read each weight tile from L2; the
// caller keeps the grid at about one workgroup per CU, each staging its A
// rows in 128 KB chunks
template <typename T, int MT>
hipError_t run_stream_wide_rows(const StreamArgs& g, const EpiArgs& e, hipStream_t s, KTime t) {
  if (g.qb || g.ent_off || g.ksplit > 1 || e.kind != EPI_STORE_F32) return hipErrorInvalidValue;
  return run_stream<T, MT, 2, EPI_STORE_F32, 8, kStreamLdsWideKB>(g, e, s, t);
}

// bf16 GEMMs over 64-row entries with a fused epilogue, each with 64 KB of
// LDS (two workgroups per CU), so that a half chunk holds whole rounds of the
// ring: expert gate|up in the 32-row entries' shape, down (whose fp32 output
// tiles need that much at 64 rows), and the q/k/v projection of several
// canvases
template <typename T>
hipError_t run_stream_wide_epi(const StreamArgs& g, const EpiArgs& e, hipStream_t s, KTime t) {
  if constexpr (sizeof(T) == 2) {
    if (!g.qb && e.kind == EPI_GEGLU) return run_stream<T, 4, 2, EPI_GEGLU, 8, 64>(g, e, s, t);
    if (!g.qb && e.kind == EPI_DOWN) return run_stream<T, 4, 4, EPI_DOWN, 2, 64>(g, e, s, t);
    if (!g.qb && e.kind == EPI_QKV) return run_stream<T, 4, 2, EPI_QKV, 8, 64>(g, e, s, t);
  }
  return hipErrorInvalidValue;
}

template <typename T>
hipError_t run_stream_t(const StreamArgs& g, const EpiArgs& e, hipStream_t s, KTime t) {
  if (g.mt == 1) return run_stream_mt<T, 1>(g, e, s, t);
  if (g.mt == 2) return run_stream_mt<T, 2>(g, e, s, t);
  if (g.mt == 4 && e.kind != EPI_STORE_F32) return run_stream_wide_epi<T>(g, e, s, t);
  if (g.mt == 4) return run_stream_wide_rows<T, 4>(g, e, s, t);
  return hipErrorInvalidValue;
}

// ----------------------------------------------------------------------------
// weight repack
// ----------------------------------------------------------------------------
template <typename T>
__global__ void k_pack(PackArgs a, int nbatch, long long src_bs, long long dst_bs) {
  const int KB = a.K >> 5;
  const long long per = (long long)a.N * a.K;
  const long long total = per * nbatch;
  const T* src = reinterpret_cast<const T*>(a.src);
  const T* src2 = reinterpret_cast<const T*>(a.src2);
  T* dst = reinterpret_cast<T*>(a.dst);
  for (long long idx = blockIdx.x * (long long)blockDim.x + threadIdx.x; idx < total;
       idx += (long long)gridDim.x * blockDim.x) {
    const long long bi = idx / per, o = idx - bi * per;
    const int j = (int)(o & 7), lane = (int)((o >> 3) & 63);
    const long long kbnb = o >> 9;
    const int kb = (int)(kbnb % KB), nb = (int)(kbnb / KB);
    const int k = kb * 32 + (lane >> 4) * 8 + j;
    const T* s = src + bi * src_bs;
    int nblk = nb;
    if (a.colmap == 1) {
      const int bph = a.head_dim >> 4, hs = nb / bph, w = nb - hs * bph;
      nblk = hs * bph + ((w & 1) ? (w >> 1) + (bph >> 1) : (w >> 1));
    } else if (a.colmap == 2) {
      nblk = nb >> 1;
      if (nb & 1) s = src2 + bi * src_bs;
    }
    const long long n = (long long)nblk * 16 + (lane & 15);
    dst[bi * dst_bs + o] = a.src_kn ? s[(long long)k * a.ld + n] : s[n * a.ld + k];
  }
}

// ----------------------------------------------------------------------------
// MXFP4 quantisation of packed bf16 fragments (OCP Microscaling Formats v1.0
// conversion: s = floor(log2 max|x|) - 2, clamped to [-126, 127]; each element
// the E2M1 value nearest to x / 2^s, ties to the even mantissa, saturating at
// 6).  One thread per (batch, n-block, k-group, k-step of the group, column):
// the column's 32 values of that k-step sit in lanes c, c+16, c+32, c+48 of
// the bf16 fragment, 8 each.
// ----------------------------------------------------------------------------
DG_DEV uint32_t e2m1_code(float v, int s) {
  const float a = fabsf(ldexpf(v, -s));  // exact: a power-of-two scaling of a bf16
  const uint32_t idx = a <= 0.25f ? 0u : a < 0.75f ? 1u : a <= 1.25f ? 2u : a < 1.75f ? 3u
                     : a <= 2.5f ? 4u : a < 3.5f ? 5u : a <= 5.0f ? 6u : 7u;
  return idx | ((__float_as_uint(v) >> 31) << 3);
}

__global__ __launch_bounds__(256) void k_quant_mxfp4(const bf16_t* __restrict__ src, int nbatch, long long src_bs,
                                                     int NB, int KB, uint32_t* codes, uint8_t* scales) {
  const int KG = (KB + 3) >> 2;
  const long long per = (long long)NB * KG * 64;  // threads per batch
  const long long total = per * nbatch;
  for (long long idx = blockIdx.x * (long long)blockDim.x + threadIdx.x; idx < total;
       idx += (long long)gridDim.x * blockDim.x) {
    const long long bi = idx / per;
    long long o = idx - bi * per;
    const int c = (int)(o & 15), j = (int)((o >> 4) & 3);
    const long long nbkg = o >> 6;  // nb * KG + kg
    const int kg = (int)(nbkg % KG), nb = (int)(nbkg / KG);
    const int kb = kg * 4 + j;
    uint32_t* cw = codes + (bi * per + nbkg * 64) * 4;  // [64 lanes][4]
    uint8_t* sb = scales + bi * per + nbkg * 64;        // [16 columns][4]
    if (kb >= KB) {
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) cw[(c + 16 * gq) * 4 + j] = 0u;
      sb[c * 4 + j] = 127;
      continue;
    }
    const bf16_t* f = src + bi * src_bs + ((long long)nb * KB + kb) * 512;
    float v[4][8];
    float amax = 0.f;
#pragma unroll
    for (int gq = 0; gq < 4; ++gq)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        v[gq][e] = bf2f(f[(c + 16 * gq) * 8 + e]);
        amax = fmaxf(amax, fabsf(v[gq][e]));
      }
    const int ex = (int)((__float_as_uint(amax) >> 23) & 0xFF) - 127;  // floor(log2 amax) for normal amax
    const int s = amax > 0.f ? min(max(ex - 2, -126), 127) : -126;
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      uint32_t wv = 0;
#pragma unroll
      for (int e = 0; e < 8; ++e) wv |= e2m1_code(v[gq][e], s) << (4 * e);
      cw[(c + 16 * gq) * 4 + j] = wv;
    }
    sb[c * 4 + j] = (uint8_t)(s + 127);
  }
}

// Weight element (k, n) of a packed operand back in math layout.
template <typename T>
__global__ __launch_bounds__(256) void k_unpack_weight(const T* __restrict__ packed, const uint32_t* __restrict__ codes,
                                                       const uint8_t* __restrict__ scales, int K, int N, int colmap,
                                                       int half, T* out, uint8_t* codes_out, uint8_t* scales_out) {
  const long long total = (long long)K * N;
  const int KB = K >> 5, KG = (KB + 3) >> 2;
  for (long long idx = blockIdx.x * (long long)blockDim.x + threadIdx.x; idx < total;
       idx += (long long)gridDim.x * blockDim.x) {
    const int k = (int)(idx / N), n = (int)(idx - (long long)k * N);
    const int nb = colmap == 2 ? 2 * (n >> 4) + half : (n >> 4);
    const int kb = k >> 5, lane = (n & 15) + 16 * ((k & 31) >> 3), e = k & 7;
    float v;
    if (codes) {
      const int kg = kb >> 2, j = kb & 3;
      const uint32_t w = codes[(((long long)nb * KG + kg) * 64 + lane) * 4 + j];
      const uint32_t sbyte = scales[(((long long)nb * KG + kg) * 16 + (n & 15)) * 4 + j];
      const Frag<bf16_t> f = dq_fp4(w, sbyte);
      const uint32_t pair = u4_at(f.v, e >> 1);
      v = bf2f((bf16_t)((e & 1) ? (pair >> 16) : (pair & 0xFFFF)));
      if (codes_out) codes_out[idx] = (uint8_t)((w >> (4 * e)) & 15u);
      if (scales_out && (k & 31) == 0) scales_out[(long long)kb * N + n] = (uint8_t)sbyte;
    } else {
      v = to_f<T>(packed[(((long long)nb * KB + kb) * 64 + lane) * 8 + e]);
    }
    if (out) out[idx] = from_f<T>(v);
  }
}

template <typename T, int MT, int WN, int EPI>
hipError_t run_gemm(const GemmArgs& g, const EpiArgs& e, hipStream_t s, KTime t) {
  constexpr int ROWS = MT * 16;
  const int tiles = (g.NB + 4 * WN - 1) / (4 * WN);
  const int smc = (g.static_rows + ROWS - 1) / ROWS;
  const long long blocks = (long long)tiles * smc + (long long)tiles * g.n_groups;
  if (blocks <= 0) return hipSuccess;
  return launch_k(k_gemm<T, MT, WN, EPI>, dim3((unsigned)blocks), dim3(256), 0, s, t.start, t.stop, g, e);
}

template <typename T, int EPI>
hipError_t run_gemm_mt(const GemmArgs& g, const EpiArgs& e, int mt, hipStream_t s, KTime t) {
  // 128-row chunks only for bf16 (the fp32 chunk would exceed 64 KB of LDS)
  if constexpr (sizeof(T) == 2) {
    if (mt >= 8) return run_gemm<T, 8, 2, EPI>(g, e, s, t);
  }
  return run_gemm<T, 4, 2, EPI>(g, e, s, t);
}

template <typename T>
hipError_t run_gemm_t(const GemmArgs& g, const EpiArgs& e, int mt, hipStream_t s, KTime t) {
  switch (e.kind) {
    case EPI_STORE_F32: return run_gemm_mt<T, EPI_STORE_F32>(g, e, mt, s, t);
    case EPI_GEGLU: return run_gemm_mt<T, EPI_GEGLU>(g, e, mt, s, t);
    case EPI_DOWN: return run_gemm_mt<T, EPI_DOWN>(g, e, mt, s, t);
    case EPI_QKV: return run_gemm_mt<T, EPI_QKV>(g, e, mt, s, t);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_gemm(int is_bf16, const GemmArgs& g, const EpiArgs& e, int mt, hipStream_t s, KTime t) {
  return is_bf16 ? run_gemm_t<bf16_t>(g, e, mt, s, t) : run_gemm_t<float>(g, e, mt, s, t);
}

hipError_t launch_stream(int is_bf16, const StreamArgs& g, const EpiArgs& e, hipStream_t s, KTime t) {
  return is_bf16 ? run_stream_t<bf16_t>(g, e, s, t) : run_stream_t<float>(g, e, s, t);
}

hipError_t launch_quant_mxfp4(const void* packed, int nbatch, long long src_bs, int NB, int KB, uint4* codes,
                              uint8_t* scales, hipStream_t s) {
  const long long total = (long long)NB * ((KB + 3) / 4) * 64 * nbatch;
  if (total <= 0) return hipSuccess;
  const long long want = (total + 255) / 256;
  const unsigned blocks = (unsigned)(want < 65536 ? want : 65536);
  hipLaunchKernelGGL(k_quant_mxfp4, dim3(blocks), dim3(256), 0, s, reinterpret_cast<const bf16_t*>(packed), nbatch,
                     src_bs, NB, KB, reinterpret_cast<uint32_t*>(codes), scales);
  return hipGetLastError();
}

hipError_t launch_unpack_weight(int is_bf16, const void* packed, const uint4* codes, const uint8_t* scales, int K,
                                int N, int colmap, int half, void* out, uint8_t* codes_out, uint8_t* scales_out,
                                hipStream_t s) {
  const long long total = (long long)K * N;
  if (total <= 0) return hipSuccess;
  if (codes && !is_bf16) return hipErrorInvalidValue;
  const long long want = (total + 255) / 256;
  const unsigned blocks = (unsigned)(want < 65536 ? want : 65536);
  const uint32_t* cw = reinterpret_cast<const uint32_t*>(codes);
  if (is_bf16)
    hipLaunchKernelGGL(k_unpack_weight<bf16_t>, dim3(blocks), dim3(256), 0, s, reinterpret_cast<const bf16_t*>(packed),
                       cw, scales, K, N, colmap, half, reinterpret_cast<bf16_t*>(out), codes_out, scales_out);
  else
    hipLaunchKernelGGL(k_unpack_weight<float>, dim3(blocks), dim3(256), 0, s, reinterpret_cast<const float*>(packed),
                       cw, scales, K, N, colmap, half, reinterpret_cast<float*>(out), codes_out, scales_out);
  return hipGetLastError();
}

hipError_t launch_pack(int is_bf16, const PackArgs& a, hipStream_t s) {
  return launch_pack_batched(is_bf16, a, 1, 0, 0, s);
}

hipError_t launch_pack_batched(int is_bf16, const PackArgs& a, int nbatch, long long src_bs,
                               long long dst_bs, hipStream_t s) {
  const long long total = (long long)a.N * a.K * nbatch;
  if (total <= 0) return hipSuccess;
  const long long want = (total + 255) / 256;
  const unsigned blocks = (unsigned)(want < 65536 ? want : 65536);
  if (is_bf16)
    hipLaunchKernelGGL(k_pack<bf16_t>, dim3(blocks), dim3(256), 0, s, a, nbatch, src_bs, dst_bs);
  else
    hipLaunchKernelGGL(k_pack<float>, dim3(blocks), dim3(256), 0, s, a, nbatch, src_bs, dst_bs);
  return hipGetLastError();
}
