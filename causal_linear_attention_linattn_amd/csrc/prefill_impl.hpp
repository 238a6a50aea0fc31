// Chunked causal linear-attention prefill for gfx950.
//
// What is computed ("Simple linear attention language models balance the
// recall-throughput tradeoff", Knowl 3 and Knowl 5): for every position i,
//   y_i = phi(q_i) S_i / phi(q_i) z_i,  S_i = sum_{j<=i} phi(k_j)^T v_j,
//   z_i = sum_{j<=i} phi(k_j)^T.
// Knowl 5 splits each tile's work into a causal within-tile term (masked
// quadratic attention) and a prefix term (a product with the accumulated
// state).  Here a tile is a chunk of C = 64 tokens and, per chunk c,
//   O^T   = S'_{c-1}^T phi(Q_c)^T + V'_c^T A_c^T        (inter + intra)
//   A_c   = (phi(Q_c) phi(K_c)^T) masked to j <= i (diagonal included)
//   S'_c  = S'_{c-1} + phi(K_c)^T V'_c
// where V' = [V | 1] carries a column of ones, so the last column of S' is
// z and the last row of O^T is the denominator ("+1" column of Knowl 7's
// state-size count).  Every product is an MFMA (bf16 x bf16 -> fp32, or the
// fp32 MFMA for float inputs); the state S' stays in fp32 accumulators.
//
// Parallel layout.  A workgroup of 4 waves owns one (batch*head, segment):
// a run of consecutive chunks walked in order.  Waves 0..3 produce the
// outputs of the chunk's 16-token tiles (all value columns); every wave w of
// the NW owns state row tiles w, w+NW, w+2NW, ... (16 features each) across
// all columns.  NW = 4, or 8 for the bf16 Taylor state (kChunkWaves).  A bf16 (or
// fp32) copy of S' in LDS, laid out column-major, feeds the inter term of
// every wave.  K, V tiles are staged through LDS transposed (feature- and
// value-major) so that every MFMA operand is one 16-byte LDS read; the next
// chunk's global loads are issued before the current chunk is computed.
//
// Several segments per head: chunk_kernel<OUT = false> sums each segment's
// state, seg_scan_kernel turns those sums into exclusive prefixes (plus the
// optional initial state), and chunk_kernel<OUT = true> starts each segment
// from its prefix.  With one segment per head only the last kernel runs.
//
// Feature order inside the kernels.  ELU1 uses the natural order.  TAYLOR2
// (d_k = 16) stores the 256 pairwise features first (index 16a + b, value
// k_a k_b without the 1/sqrt2, which is moved to the query side as 1/2),
// then the constant (256) and the 16 linear features (257..272), then 15
// zero pads up to 288 = 9 MFMA K blocks.  The exported states use the
// pages' order [1, x, vec(x x^T)/sqrt2] and are converted at the boundary.
#pragma once

#include "device.hpp"
#include "shapes.hpp"

namespace linattn {

// Waves per chunk workgroup.  The Taylor state (18 row tiles) is spread
// over 8 waves for bf16 inputs without decay, so that each holds fewer
// accumulators and two waves share a SIMD (measured on one MI355X at
// B=8 H=16 N=2048: 111.7 -> 106.6 us per call); with the decay factors or
// float tiles the 8-wave build spills (gated: 130 -> 150 us), so those keep 4.
template <int MAP, typename T, bool GATED>
constexpr int kChunkWaves = MAP != MAP_ELU1 && sizeof(T) == 2 && !GATED ? 8 : 4;

template <int MAP, typename T, int DK, int DV, int NWAVES = 4>
struct PrefillShape : StateShape<MAP, DK, DV> {
  using SS = StateShape<MAP, DK, DV>;
  static constexpr int C = 64;
  static constexpr int NW = NWAVES;  // waves per workgroup
  static constexpr int NT = 64 * NW;
  static constexpr int MAXRT = (SS::NRT + NW - 1) / NW;
  static constexpr int EPU = Elem<T>::kPer16B;
  static constexpr int KS = DK + EPU;       // LDS row strides (elements),
  static constexpr int CS = C + EPU;        // padded by 16 bytes
  static constexpr int PS = SS::DP + EPU;
  static constexpr int KUR = DK / EPU;      // 16-byte units per k row
  static constexpr int VUR = DV / EPU;
  static constexpr int UK = C * DK / EPU;   // 16-byte units per k tile
  static constexpr int UV = C * DV / EPU;
  static constexpr int NUK = (UK + NT - 1) / NT;
  static constexpr int NUV = (UV + NT - 1) / NT;
  static constexpr int PK = C / 2 * KUR;    // row-pair units per k tile
  static constexpr int PV = C / 2 * VUR;
  static constexpr int NPK = (PK + NT - 1) / NT;
  static constexpr int NPV = (PV + NT - 1) / NT;
  static constexpr int NQU = MAP == MAP_ELU1 ? SS::NKB * 8 / EPU : DK / EPU;
  static constexpr int NKBS = (DK + 31) / 32;  // K blocks of the scores
};

// Chunks in the register prefetch ring of the chunk walker (chunks c + 2 ..
// c + P are in flight while c is computed): the light segment-sum pass
// affords a deeper ring than the output pass.  Even, so that one unrolled
// trip covers the ring and the two LDS copies.
template <bool OUT>
constexpr int kRing = OUT ? 2 : 4;

// Internal feature row -> exported row (or -1 for padding) and the factor
// that converts an exported value into the internal one.  Internal rows
// 0..255 hold the ordered pairs (a, b) = (r / 16, r % 16) with key feature
// k_a k_b, row 256 the constant and 257..272 the linear features.
//   ordered export: pair (a, b) at 17 + 16 a + b, value internal / sqrt 2;
//   unordered export (sym): pair {a, b} at 17 + p(min, max) with
//     p(a, b) = a d - a (a - 1) / 2 + (b - a), value internal for a != b and
//     internal / sqrt 2 for a == b.  Both (a, b) and (b, a) import from the
//     same exported row; only a <= b is exported (`owner`).
template <int MAP, int DK>
__device__ __forceinline__ int ext_row(int r, bool sym, float& to_internal,
                                       bool& owner) {
  to_internal = 1.0f;
  owner = true;
  if (MAP == MAP_ELU1) return r < DK ? r : -1;
  if (r < 256) {
    if (!sym) {
      to_internal = kSqrt2;
      return 17 + r;
    }
    const int pa = r >> 4, pb = r & 15;
    const int lo = pa < pb ? pa : pb, hi = pa < pb ? pb : pa;
    owner = pa <= pb;
    if (pa == pb) to_internal = kSqrt2;
    return 17 + lo * DK - lo * (lo - 1) / 2 + (hi - lo);
  }
  return r < 273 ? r - 256 : -1;
}

// Exported feature rows of a head's state.
template <int MAP, int DK, int DV>
__device__ __forceinline__ int ext_rows(bool sym) {
  return MAP == MAP_TAYLOR2 && sym ? kSymD<DK> : StateShape<MAP, DK, DV>::D;
}

// One lane's 4 values of state tile (rt, ct) read from the exported
// layout S [D, DV], z [D] of sequence bh, converted to the internal one.
template <int MAP, int DK, int DV>
__device__ __forceinline__ f32x4_t state_in_tile(const float* S_in,
                                                 const float* z_in, bool sym,
                                                 int bh, int rt, int ct,
                                                 int lane) {
  const int D = ext_rows<MAP, DK, DV>(sym);
  f32x4_t r;
  const int col = 16 * ct + (lane & 15);
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int row = 16 * rt + 4 * (lane >> 4) + t;
    float f;
    bool owner;
    const int e = ext_row<MAP, DK>(row, sym, f, owner);
    float val = 0.0f;
    if (e >= 0) {
      if (col < DV)
        val = S_in[((size_t)bh * D + e) * DV + col];
      else if (col == DV)
        val = z_in[(size_t)bh * D + e];
    }
    r[t] = val * f;
  }
  return r;
}

template <int MAP, int DK, int DV>
__device__ __forceinline__ void state_out_tile(float* S_out, float* z_out,
                                               bool sym, int bh, int rt,
                                               int ct, int lane,
                                               const f32x4_t& v) {
  const int D = ext_rows<MAP, DK, DV>(sym);
  const int col = 16 * ct + (lane & 15);
  if (col > DV) return;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int row = 16 * rt + 4 * (lane >> 4) + t;
    float f;
    bool owner;
    const int e = ext_row<MAP, DK>(row, sym, f, owner);
    if (e < 0 || !owner) continue;
    const float val = v[t] / f;
    if (col < DV)
      S_out[((size_t)bh * D + e) * DV + col] = val;
    else
      z_out[(size_t)bh * D + e] = val;
  }
}

// Row-major bf16 tile of R-element rows in LDS, its 16-byte units permuted
// within each row by a function of the row.  The layout is chosen against
// gfx950's LDS as measured with per-pattern bank-conflict counters: 16-byte
// reads are served to pairs of 8-lane blocks (lanes 8b.. with 8(7-b)..) over
// 64 banks, 8-byte and transposed reads to 32 lanes at a time over 64 banks,
// 16-byte writes to 8 lanes at a time over 32 banks.  Rows of 32 or 64
// elements are then unpadded, with unit u of row r stored at
// u ^ (2 (r & 3) ^ (r >> 2)): the staging stores, the key-row reads of the
// scores and the transposed reads of the token-contracted operands are all
// conflict-free.  Other widths keep a 64-byte pad and u ^ (r ^ (r >> 3)).
template <int R>
struct RowTile {
  static constexpr int UPR = R / 8;  // 16-byte units per row
  static constexpr bool kDense = R == 32 || R == 64;
  static constexpr int STRIDE = kDense ? R : R + 32;
  __device__ static __forceinline__ int swz(int row) {
    if constexpr (kDense)
      return ((2 * (row & 3)) ^ (row >> 2)) & (UPR - 1);
    else
      return (row ^ (row >> 3)) & (UPR - 1);
  }
  __device__ static __forceinline__ int off(int row, int unit) {
    return row * STRIDE + 8 * (unit ^ swz(row));
  }
  __device__ static __forceinline__ int off_el(int row, int col) {
    return off(row, col >> 3) + (col & 7);
  }
};

// ---------------------------------------------------------------------------
// The chunk walker.  OUT = false: sum phi(K)^T V' over the segment and store
// it in workspace slot seg + 1 (segments 0 .. nseg-2).  OUT = true: produce
// y for the segment starting from its prefix state.
//
// Global loads are raw buffer loads whose range is the segment itself, so
// rows past the segment end (or past N) read as zero without a branch, and
// y is written with range-checked buffer stores.  Every LDS tile (and the
// LDS copy of the state) exists twice: chunk c is computed from copy c % 2
// while chunk c + 1 is staged into the other, so one barrier per chunk
// suffices and the staging arithmetic of c + 1 can overlap the matrix work
// of c.  Chunks c + 2 .. c + P are in flight in a register ring meanwhile.
//
// Tokens past the segment end need no masking: they read k = 0 and v = 0,
// so they add nothing to the value columns of the state and exactly phi(0)
// each to its z column, which is subtracted once after the walk; a valid
// query never attends to them (causality), and their own y rows are outside
// the store range.  Only chunks after them see the inflated z, and those
// produce no output.
//
// Operands contracted over tokens (phi(K)^T and V' in the state update, V'^T
// in the within-chunk product) need 8 consecutive tokens per lane.  bf16
// tiles are kept row-major and read with the LDS transpose read; float
// tiles are stored transposed (two tokens per store).
// ---------------------------------------------------------------------------
// Operand reads from the chunk tiles in LDS and the within-chunk product of
// one 16-query tile against one 32-token key block ([SLA] Knowl 5: the
// masked quadratic term of a tile).  Shared by the chunk walker and the
// looped LDS-resident throughput probe of the intra-chunk products.
template <int MAP, typename T, int DK, int DV>
struct ChunkTiles {
  using SH = PrefillShape<MAP, T, DK, DV>;
  using E = Elem<T>;
  using frag = typename E::frag;
  static constexpr bool BF = sizeof(T) == 2;
  static constexpr int NCT = SH::NCT;
  using RTK = RowTile<DK>;
  using RTV = RowTile<DV>;

  // 8 tokens (tb .. tb+7) of column c0 + i16 of a row-major bf16 tile
  template <class RT>
  __device__ static __forceinline__ frag tokfrag_bf(const T* base, int tb, int c0, int lane) {
    if constexpr (BF) {
      const int i16 = lane & 15;
      const int r = tb + (i16 >> 2);
      const int col = c0 + 4 * (i16 & 3);
      const uint2 lo = lds_read_tr4(reinterpret_cast<const uint16_t*>(base) + RT::off_el(r, col));
      const uint2 hi = lds_read_tr4(reinterpret_cast<const uint16_t*>(base) + RT::off_el(r + 4, col));
      return __builtin_bit_cast(frag, make_uint4(lo.x, lo.y, hi.x, hi.y));
    } else {
      return E::zero();
    }
  }

  // V' / V'^T operand: lane (column i16 of tile ct, g) slot t <-> token
  // 32 jb2 + 8 g + t
  __device__ static __forceinline__ frag v_frag(const T* sV, int jb2, int ct, int lane) {
    const int i16 = lane & 15, g = lane >> 4;
    if constexpr (BF)
      return tokfrag_bf<RTV>(sV, 32 * jb2 + 8 * g, 16 * ct, lane);
    else
      return E::load8(sV + (16 * ct + i16) * SH::CS + 32 * jb2 + 8 * g);
  }

  // key rows for the scores: lane (key jt, g) slot t <-> feature 32 kbs + 8 g + t
  __device__ static __forceinline__ frag k_rows(const T* sK, int jt, int kbs, int lane) {
    const int f0 = 32 * kbs + 8 * (lane >> 4);
    if (f0 >= DK) return E::zero();
    if constexpr (BF)
      return E::load8(sK + RTK::off(jt, f0 >> 3));
    else
      return E::load8(sK + jt * SH::KS + f0);
  }

  // O^T += V'^T A^T for key block jb2, where A^T = scores^T of the block's
  // keys against the wave's 16 queries (operands bq), kept where keep[] is
  // set (the causal mask); TAYLOR2 turns the raw q.k into 1 + s + s^2 / 2.
  // GATED: each kept score is multiplied by its decay weight, the product
  // of the coefficients after the key up to the query: 2^(Gq - G[key]) from
  // the chunk's running log2 sums G (gk = G of keys 32 jb2 + 8 g + 0..7),
  // or 0 for a key before the query's last reset Lq.
  template <bool GATED = false>
  __device__ static __forceinline__ void within_chunk(const T* sK, const frag (&vf)[NCT - 1],
                                                      const frag (&bq)[SH::NKBS], const bool (&keep)[8],
                                                      const frag& ones, f32x4_t (&O)[NCT], int jb2,
                                                      int lane, const float* gk = nullptr,
                                                      float Gq = 0.0f, int Lq = -1) {
    const int i16 = lane & 15;
    f32x4_t sc[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      sc[h] = {0.0f, 0.0f, 0.0f, 0.0f};
      const int jt = 32 * jb2 + 8 * (i16 >> 2) + 4 * h + (i16 & 3);
#pragma unroll
      for (int kbs = 0; kbs < SH::NKBS; ++kbs) E::mma(sc[h], k_rows(sK, jt, kbs, lane), bq[kbs]);
    }
    float dec[8];
    if constexpr (GATED) {
      const float4 g0 = *reinterpret_cast<const float4*>(gk);
      const float4 g1 = *reinterpret_cast<const float4*>(gk + 4);
      const float G[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
      const int key0 = 32 * jb2 + 8 * (lane >> 4);
#pragma unroll
      for (int e = 0; e < 8; ++e)
        dec[e] = keep[e] && key0 + e >= Lq ? __builtin_amdgcn_exp2f(Gq - G[e]) : 0.0f;
    }
    float f[8];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const float sv = sc[h][t];
        float val;
        if constexpr (MAP == MAP_ELU1) val = sv; else val = 1.0f + sv + 0.5f * sv * sv;
        if constexpr (GATED) val *= dec[4 * h + t];
        f[4 * h + t] = keep[4 * h + t] ? val : 0.0f;
      }
    const frag bA = E::make(f);
#pragma unroll
    for (int ct = 0; ct < NCT - 1; ++ct) E::mma(O[ct], vf[ct], bA);
    E::mma(O[NCT - 1], ones, bA);
  }
};

template <class SH, bool BF>
struct Stage {
  static constexpr int NK = BF ? SH::NUK : 2 * SH::NPK;
  static constexpr int NV = BF ? SH::NUV : 2 * SH::NPV;
  uint4 k[NK];
  uint4 v[NV];
  uint4 q[SH::NQU];
  float gt;  // gated form: decay coefficient of token (lane) of the chunk
};

template <int I, int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

template <int MAP, typename T, int DK, int DV, bool OUT, bool GATED>
__global__ __launch_bounds__((64 * kChunkWaves<MAP, T, GATED>)) void chunk_kernel(PrefillArgs a) {
  using SH = PrefillShape<MAP, T, DK, DV, kChunkWaves<MAP, T, GATED>>;
  using E = Elem<T>;
  using frag = typename E::frag;
  constexpr bool BF = sizeof(T) == 2;
  constexpr int C = SH::C, NCT = SH::NCT, NRT = SH::NRT, NKB = SH::NKB;
  constexpr int KS = SH::KS, CS = SH::CS, PS = SH::PS, EPU = SH::EPU;
  constexpr int P = kRing<OUT>;
  static_assert(P % 2 == 0, "one unrolled trip covers the ring and both LDS copies");
  constexpr uint32_t ES = sizeof(T);
  constexpr uint32_t kOOB = 0x7ffffff0u;  // an offset no segment reaches
  using RTK = RowTile<DK>;
  using RTV = RowTile<DV>;
  using St = Stage<SH, BF>;

  // sK: rows of phi(K) (ELU1) or k (TAYLOR2); needed by the output kernel
  // for the scores and, for bf16 ELU1, by both kernels as the transposed
  // source of phi(K)^T.  sKT: K transposed (float, and TAYLOR2).  sS: the
  // state S'^T in the MFMA operand precision, column-major; two copies
  // unless that does not fit next to the tiles (float TAYLOR2).
  constexpr bool kNeedK = OUT || (BF && MAP == MAP_ELU1);
  constexpr bool kNeedKT = !(BF && MAP == MAP_ELU1);
  constexpr int K_EL = kNeedK ? (BF ? C * RTK::STRIDE : C * KS) : EPU;
  constexpr int KT_EL = kNeedKT ? DK * CS : EPU;
  constexpr int V_EL = BF ? C * RTV::STRIDE : DV * CS;
  constexpr int S_EL = OUT ? SH::NCOL * PS : EPU;
  constexpr int kTileBytes = 2 * (K_EL + KT_EL + V_EL) * (int)sizeof(T) + (GATED ? 2 * C * 16 : 0);
  constexpr int NSB = kTileBytes + 2 * S_EL * (int)sizeof(T) <= 160 * 1024 ? 2 : 1;
  __shared__ __align__(16) T sK0[K_EL];
  __shared__ __align__(16) T sK1[K_EL];
  __shared__ __align__(16) T sKT0[KT_EL];
  __shared__ __align__(16) T sKT1[KT_EL];
  __shared__ __align__(16) T sV0[V_EL];
  __shared__ __align__(16) T sV1[V_EL];
  __shared__ __align__(16) T sS0[S_EL];
  __shared__ __align__(16) T sS1[NSB == 2 ? S_EL : EPU];
  // Gated form, per LDS copy: sG[b][i] = log2 of the decay accumulated from
  // the chunk's last reset at or before token i (or from the chunk start)
  // through token i; sL[b][i] = the index of that reset, or -1; sF[b][i] =
  // the factor of the state carried into the chunk at token i (0 past a
  // reset); sU[b][i] = the weight of token i at the chunk end (0 across a
  // reset and past the segment end).
  __shared__ __align__(16) float sG[2][GATED ? C : 1];
  __shared__ __align__(16) int sL[2][GATED ? C : 1];
  __shared__ __align__(16) float sF[2][GATED ? C : 1];
  __shared__ __align__(16) float sU[2][GATED ? C : 1];
  auto sK = [&](int b) __attribute__((always_inline)) { return b ? sK1 : sK0; };
  auto sKT = [&](int b) __attribute__((always_inline)) { return b ? sKT1 : sKT0; };
  auto sV = [&](int b) __attribute__((always_inline)) { return b ? sV1 : sV0; };
  auto sS = [&](int b) __attribute__((always_inline)) { return (NSB == 2 && b) ? sS1 : sS0; };

  const int tid = threadIdx.x;
  constexpr int NW = SH::NW;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6) & (NW - 1);  // wave-uniform
  // waves that own one of the chunk's 4 query tiles (all of them when NW = 4)
  const bool qwave = NW == 4 || w < 4;
  const int lane = tid & 63;
  // State row tile m of this wave (a tile index >= NRT means none).  The
  // 8-wave output kernels give the output waves 0-3 two tiles each (w, w+4)
  // and waves 4-7 the rest (8 + (w-4) + 4m), which evens out the per-wave
  // matrix work; otherwise wave w owns tiles w, w + NW, ...
  auto row_tile = [&](int m) __attribute__((always_inline)) -> int {
    if constexpr (OUT && NW == 8) {
      static_assert(SH::NRT <= 8 + 4 * SH::MAXRT, "tiles 8.. fit the waves 4-7");
      return w < 4 ? (m < 2 ? w + 4 * m : SH::NRT + 64) : 8 + (w - 4) + 4 * m;
    } else {
      return w + NW * m;
    }
  };
  const int i16 = lane & 15;
  const int g = lane >> 4;

  // OUT: one workgroup per output segment.  Segment sums: one per part of
  // every segment but the last (sum_split parts per segment).
  const int nseg_here = OUT ? a.nseg : (a.nseg - 1) * a.sum_split;
  const int seg_chunks = OUT ? a.seg_chunks : a.seg_chunks / a.sum_split;
  const int bh = blockIdx.x / nseg_here;
  const int seg = blockIdx.x % nseg_here;
  const int64_t N = a.N;
  const int64_t tok_begin = (int64_t)seg * seg_chunks * C;
  int64_t tok_end = tok_begin + (int64_t)seg_chunks * C;
  if (tok_end > N) tok_end = N;
  const int ntok = (int)(tok_end - tok_begin);   // tokens in this segment
  const int nchunks = (ntok + C - 1) / C;

  const T* qg = reinterpret_cast<const T*>(a.q) + ((size_t)bh * N + tok_begin) * DK;
  const T* kg = reinterpret_cast<const T*>(a.k) + ((size_t)bh * N + tok_begin) * DK;
  const T* vg = reinterpret_cast<const T*>(a.v) + ((size_t)bh * N + tok_begin) * DV;
  const auto rq = make_rsrc(qg, (uint32_t)ntok * DK * ES);
  const auto rk = make_rsrc(kg, (uint32_t)ntok * DK * ES);
  const auto rv = make_rsrc(vg, (uint32_t)ntok * DV * ES);
  T* yg = OUT ? reinterpret_cast<T*>(a.y) + ((size_t)bh * N + tok_begin) * DV : nullptr;
  const auto ry = make_rsrc(yg, OUT ? (uint32_t)ntok * DV * ES : 0u);
  const auto rg = make_rsrc(GATED ? a.gate + (size_t)bh * N + tok_begin : nullptr,
                            GATED ? (uint32_t)ntok * 4u : 0u);

  // ------------------------------------------------------------ state ----
  f32x4_t Sacc[SH::MAXRT][NCT];
#pragma unroll
  for (int m = 0; m < SH::MAXRT; ++m) {
    const int rt = row_tile(m);
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      f32x4_t s = {0.0f, 0.0f, 0.0f, 0.0f};
      if (OUT && rt < NRT) {
        if (a.prefix_mode == 2) {
          // scanned workspace: slot seg * sum_split holds the exclusive
          // prefix of the segment
          const f32x4_t* p = reinterpret_cast<const f32x4_t*>(
              a.ws + ((size_t)bh * a.nslot + seg * a.sum_split) * SH::SLOT);
          s = p[(rt * NCT + ct) * 64 + lane];
        } else if (a.S_in != nullptr) {
          s = state_in_tile<MAP, DK, DV>(a.S_in, a.z_in, a.sym != 0, bh, rt, ct,
                                        lane);
        }
      }
      Sacc[m][ct] = s;
    }
  }
  if (OUT && a.prefix_mode == 1 && seg > 0) {
    // Few segments: add the sums of the preceding segments (slots 1 .. seg)
    // directly.  The loads go through a buffer resource that covers exactly
    // those slots, so the fixed-trip loop below issues every load at once
    // and the slots past `seg` read as zero.  (Rows past NRT, which exist
    // only when NRT is not a multiple of the wave count, take an
    // out-of-range offset; those accumulators are never used.)
    // Gated: the state entering segment j + 1 is the one entering segment j
    // scaled by segment j's total decay, plus segment j's own sum; the
    // log2 decays past `seg` read as 0 (factor 1).
    const int npre = seg * a.sum_split;  // sums of the parts before seg
    const auto rw = make_rsrc(a.ws + ((size_t)bh * a.nslot + 1) * SH::SLOT,
                              (uint32_t)npre * SH::SLOT * 4u);
    const auto rl = make_rsrc(GATED ? a.ws_log + (size_t)bh * a.nslot + 1 : nullptr,
                              GATED ? (uint32_t)npre * 4u : 0u);
#pragma unroll
    for (int j = 0; j < kDirectPrefixMax - 1; ++j) {
      float fj = 1.0f;
      if constexpr (GATED)
        fj = __builtin_amdgcn_exp2f(__uint_as_float(buffer_load4(rl, (uint32_t)j * 4u)));
#pragma unroll
      for (int m = 0; m < SH::MAXRT; ++m) {
        const int rt = row_tile(m);
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
          const uint32_t off = rt < NRT ? ((uint32_t)j * SH::SLOT + ((rt * NCT + ct) * 64 + lane) * 4) * 4u
                                        : kOOB;
          const f32x4_t t = __builtin_bit_cast(f32x4_t, buffer_load16(rw, off));
          if constexpr (GATED)
            Sacc[m][ct] = Sacc[m][ct] * fj + t;
          else
            Sacc[m][ct] += t;
        }
      }
    }
  }

  // ones column of V' (and ones row of V'^T): lane column 0 of the last tile
  float onesv[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) onesv[t] = i16 == 0 ? 1.0f : 0.0f;
  const frag ones = E::make(onesv);
  // ------------------------------------------------- tile operand access --
  using CT = ChunkTiles<MAP, T, DK, DV>;
  auto v_frag = [&](int b, int jb2, int ct) __attribute__((always_inline)) -> frag {
    return CT::v_frag(sV(b), jb2, ct, lane);
  };

  // ---------------------------------------------------------- staging ----
  St st[P];

  auto issue = [&](int c, St& s) __attribute__((always_inline)) {
    const uint32_t cb = (uint32_t)c * C;  // first token of chunk c
    if constexpr (BF) {
#pragma unroll
      for (int u = 0; u < St::NK; ++u) {
        const int p = tid + u * SH::NT;
        const uint32_t off = ((cb + p / RTK::UPR) * DK + (p % RTK::UPR) * 8) * ES;
        s.k[u] = buffer_load16(rk, p < SH::UK ? off : kOOB);
      }
#pragma unroll
      for (int u = 0; u < St::NV; ++u) {
        const int p = tid + u * SH::NT;
        const uint32_t off = ((cb + p / RTV::UPR) * DV + (p % RTV::UPR) * 8) * ES;
        s.v[u] = buffer_load16(rv, p < SH::UV ? off : kOOB);
      }
    } else {
#pragma unroll
      for (int u = 0; u < SH::NPK; ++u) {
        const int pu = tid + u * SH::NT;
        const uint32_t r0 = cb + 2 * (pu / SH::KUR);
        const uint32_t e0 = (pu % SH::KUR) * EPU;
        const uint32_t off = pu < SH::PK ? (r0 * DK + e0) * ES : kOOB;
        s.k[2 * u] = buffer_load16(rk, off);
        s.k[2 * u + 1] = buffer_load16(rk, pu < SH::PK ? off + DK * ES : kOOB);
      }
#pragma unroll
      for (int u = 0; u < SH::NPV; ++u) {
        const int pu = tid + u * SH::NT;
        const uint32_t r0 = cb + 2 * (pu / SH::VUR);
        const uint32_t e0 = (pu % SH::VUR) * EPU;
        const uint32_t off = pu < SH::PV ? (r0 * DV + e0) * ES : kOOB;
        s.v[2 * u] = buffer_load16(rv, off);
        s.v[2 * u + 1] = buffer_load16(rv, pu < SH::PV ? off + DV * ES : kOOB);
      }
    }
    if constexpr (OUT) if (qwave) {
      const uint32_t tq = cb + 16 * w + i16;
      if constexpr (MAP == MAP_ELU1) {
        constexpr int UPB = 8 / EPU;  // 16-byte units per 8-feature block
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int h = 0; h < UPB; ++h) {
            const uint32_t f0 = 32 * kb + 8 * g + h * EPU;
            s.q[kb * UPB + h] = buffer_load16(rq, f0 < DK ? (tq * DK + f0) * ES : kOOB);
          }
      } else {
#pragma unroll
        for (int u = 0; u < SH::NQU; ++u)
          s.q[u] = buffer_load16(rq, (tq * DK + u * EPU) * ES);
      }
    }
    if constexpr (GATED) {
      if (w == 0) s.gt = __uint_as_float(buffer_load4(rg, (cb + lane) * 4u));
    }
  };

  // Gated form: the decay of chunk `chunk` from its ring slot into copy b.
  // Wave 0 takes log2 of each coefficient (tokens past the segment end get
  // 0, i.e. a = 1, and never count as resets) and runs a segmented
  // inclusive scan over the 64 tokens: a reset restarts the sum.
  auto stage_gate = [&](const St& s, int b, int chunk) __attribute__((always_inline)) {
    if constexpr (GATED) {
      if (w != 0) return;
      const bool valid = chunk * C + lane < ntok;
      const float lg = __builtin_amdgcn_logf(s.gt);
      const bool reset = valid && !(lg >= kResetLog2);
      float G = valid && !reset ? lg : 0.0f;
      int L = reset ? lane : -1;
      // Inclusive scan of (G, L) under "a later reset wins, else add": steps
      // of 1, 2, 4, 8 lanes inside each row of 16, then the row totals
      // through lanes 15 and 31.  A lane without a source receives the
      // identity (0, -1).
      auto combine = [&](auto ctrl, auto rows) __attribute__((always_inline)) {
        constexpr int CTRL = decltype(ctrl)::value, ROWS = decltype(rows)::value;
        const float Gp = __int_as_float(dpp_move<CTRL, ROWS>(0, __float_as_int(G)));
        const int Lp = dpp_move<CTRL, ROWS>(-1, L);
        if (L < 0) {
          G += Gp;
          L = Lp;
        }
      };
      combine(std::integral_constant<int, 0x111>{}, std::integral_constant<int, 0xf>{});
      combine(std::integral_constant<int, 0x112>{}, std::integral_constant<int, 0xf>{});
      combine(std::integral_constant<int, 0x114>{}, std::integral_constant<int, 0xf>{});
      combine(std::integral_constant<int, 0x118>{}, std::integral_constant<int, 0xf>{});
      combine(std::integral_constant<int, 0x142>{}, std::integral_constant<int, 0xa>{});
      combine(std::integral_constant<int, 0x143>{}, std::integral_constant<int, 0xc>{});

      const float Gend = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(G), C - 1));
      const int Lend = __builtin_amdgcn_readlane(L, C - 1);
      sG[b][lane] = G;
      sL[b][lane] = L;
      sF[b][lane] = L >= 0 ? 0.0f : __builtin_amdgcn_exp2f(G);
      sU[b][lane] = valid && lane >= Lend ? __builtin_amdgcn_exp2f(Gend - G) : 0.0f;
    }
  };

  // Stage a chunk from its ring slot into LDS copy b.
  auto write_tiles = [&](const St& s, int b) __attribute__((always_inline)) {
    if constexpr (BF) {
#pragma unroll
      for (int u = 0; u < St::NK; ++u) {
        const int p = tid + u * SH::NT;
        if (SH::UK % SH::NT == 0 || p < SH::UK) {  // compile-time when tiles divide evenly
          const int row = p / RTK::UPR, unit = p % RTK::UPR;
          if constexpr (MAP == MAP_ELU1) {
            float f[8];
            unpack16<T>(s.k[u], f);
#pragma unroll
            for (int e = 0; e < 8; ++e) f[e] = phi_elu1(f[e]);
            *reinterpret_cast<uint4*>(sK(b) + RTK::off(row, unit)) = pack16<T>(f);
          } else {
            if constexpr (OUT) *reinterpret_cast<uint4*>(sK(b) + RTK::off(row, unit)) = s.k[u];
            const uint32_t wd[4] = {s.k[u].x, s.k[u].y, s.k[u].z, s.k[u].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              sKT(b)[(unit * 8 + 2 * e) * CS + row] = (bf16_t)(wd[e] & 0xffffu);
              sKT(b)[(unit * 8 + 2 * e + 1) * CS + row] = (bf16_t)(wd[e] >> 16);
            }
          }
        }
      }
#pragma unroll
      for (int u = 0; u < St::NV; ++u) {
        const int p = tid + u * SH::NT;
        if (SH::UV % SH::NT == 0 || p < SH::UV)
          *reinterpret_cast<uint4*>(sV(b) + RTV::off(p / RTV::UPR, p % RTV::UPR)) = s.v[u];
      }
    } else {
#pragma unroll
      for (int u = 0; u < SH::NPK; ++u) {
        const int pu = tid + u * SH::NT;
        if (SH::PK % SH::NT == 0 || pu < SH::PK) {
          const int r0 = 2 * (pu / SH::KUR);
          const int e0 = (pu % SH::KUR) * EPU;
          float f0[EPU], f1[EPU];
          unpack16<T>(s.k[2 * u], f0);
          unpack16<T>(s.k[2 * u + 1], f1);
          if constexpr (MAP == MAP_ELU1) {
#pragma unroll
            for (int e = 0; e < EPU; ++e) {
              f0[e] = phi_elu1(f0[e]);
              f1[e] = phi_elu1(f1[e]);
            }
          }
          if constexpr (OUT) {
            *reinterpret_cast<uint4*>(sK(b) + r0 * KS + e0) = pack16<T>(f0);
            *reinterpret_cast<uint4*>(sK(b) + (r0 + 1) * KS + e0) = pack16<T>(f1);
          }
#pragma unroll
          for (int e = 0; e < EPU; ++e) store_pair(sKT(b) + (e0 + e) * CS + r0, f0[e], f1[e]);
        }
      }
#pragma unroll
      for (int u = 0; u < SH::NPV; ++u) {
        const int pu = tid + u * SH::NT;
        if (SH::PV % SH::NT == 0 || pu < SH::PV) {
          const int r0 = 2 * (pu / SH::VUR);
          const int e0 = (pu % SH::VUR) * EPU;
          float f0[EPU], f1[EPU];
          unpack16<T>(s.v[2 * u], f0);
          unpack16<T>(s.v[2 * u + 1], f1);
#pragma unroll
          for (int e = 0; e < EPU; ++e) store_pair(sV(b) + (e0 + e) * CS + r0, f0[e], f1[e]);
        }
      }
    }
  };

  // Query operands, one set per LDS copy (the set of chunk c + 1 is formed
  // while chunk c is computed).
  //   ELU1:    qf[b][kb] = phi(q) over features 32kb + 8g + (0..7)
  //   TAYLOR2: qs[b][u]  = the raw 16-byte units of q (expanded at use)
  frag qf[2][MAP == MAP_ELU1 && OUT ? NKB : 1];
  uint4 qs[2][MAP == MAP_TAYLOR2 && OUT ? SH::NQU : 1];

  auto take_q = [&](const St& s, int b) __attribute__((always_inline)) {
    if constexpr (!OUT) return;
    if (!qwave) return;
    if constexpr (MAP == MAP_ELU1) {
      constexpr int UPB = 8 / EPU;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        float f[8];
#pragma unroll
        for (int h = 0; h < UPB; ++h) {
          float part[EPU];
          unpack16<T>(s.q[kb * UPB + h], part);
#pragma unroll
          for (int e = 0; e < EPU; ++e) f[h * EPU + e] = part[e];
        }
#pragma unroll
        for (int t = 0; t < 8; ++t)
          f[t] = (32 * kb + 8 * g + t < DK) ? phi_elu1(f[t]) : 0.0f;
        qf[b][kb] = E::make(f);
      }
    } else {
#pragma unroll
      for (int u = 0; u < SH::NQU; ++u) qs[b][u] = s.q[u];
    }
  };

  // TAYLOR2 query of the current chunk (lane: query i16 of the wave's tile,
  // lane group g), prepared once per chunk: qa8[k] = q[2k + (g >> 1)] / 2
  // and qb8[t] = q[8 (g & 1) + t] are the two factors of the pair features
  // of block k < 8; q8f is the operand of block 8 (the constant, the linear
  // features, zero pads).  Vector values, not arrays: an array indexed by a
  // loop counter before unrolling can be placed in LDS by the compiler.
  f32x8_t qa8 = {}, qb8 = {};
  frag q8f = E::zero();

  // phi(K)^T operand for state row tile rt, key block jb2: lane (rho = i16,
  // g) slot t <-> feature 16 rt + rho, token 32 jb2 + 8 g + t.
  // GATED: slot t is scaled by u[t], the decay from its token to the chunk
  // end.
  auto kt_frag = [&](int b, int rt, int jb2, const float (&u)[8]) __attribute__((always_inline)) -> frag {
    const int col = 32 * jb2 + 8 * g;
    if constexpr (MAP == MAP_ELU1) {
      if (16 * rt >= DK) return E::zero();
      frag r;
      if constexpr (BF)
        r = CT::template tokfrag_bf<RTK>(sK(b), col, 16 * rt, lane);
      else
        r = E::load8(sKT(b) + (16 * rt + i16) * CS + col);
      if constexpr (GATED) {
        float f[8];
        if constexpr (BF) {
          unpack16<T>(__builtin_bit_cast(uint4, r), f);
        } else {
#pragma unroll
          for (int t = 0; t < 8; ++t) f[t] = r[t];
        }
#pragma unroll
        for (int t = 0; t < 8; ++t) f[t] *= u[t];
        r = E::make(f);
      }
      return r;
    } else {
      float f[8];
      if (rt < 16) {
        float fa[8], fb[8];
        E::load8f(sKT(b) + rt * CS + col, fa);
        E::load8f(sKT(b) + i16 * CS + col, fb);
#pragma unroll
        for (int t = 0; t < 8; ++t) f[t] = fa[t] * fb[t];
      } else if (rt == 16) {
        float fb[8];
        E::load8f(sKT(b) + (i16 == 0 ? 0 : i16 - 1) * CS + col, fb);
#pragma unroll
        for (int t = 0; t < 8; ++t) f[t] = i16 == 0 ? 1.0f : fb[t];
      } else {
        float fb[8];
        E::load8f(sKT(b) + 15 * CS + col, fb);
#pragma unroll
        for (int t = 0; t < 8; ++t) f[t] = i16 == 0 ? fb[t] : 0.0f;
      }
      if constexpr (GATED) {
#pragma unroll
        for (int t = 0; t < 8; ++t) f[t] *= u[t];
      }
      return E::make(f);
    }
  };

  // phi(Q) operand for feature block kb: lane (query i16, g) slot t <->
  // feature 32 kb + 8 g + t.
  auto q_frag = [&](int b, int kb) __attribute__((always_inline)) -> frag {
    if constexpr (MAP == MAP_ELU1) {
      return qf[b][kb < NKB ? kb : 0];
    } else {
      if (kb >= 8) return q8f;
      const float qa = qa8[kb];
      float f[8];
#pragma unroll
      for (int t = 0; t < 8; ++t) f[t] = qa * qb8[t];
      return E::make(f);
    }
  };

  // Write this wave's state tiles into LDS copy b (column-major S'^T).
  auto publish_state = [&](int b) __attribute__((always_inline)) {
#pragma unroll
    for (int m = 0; m < SH::MAXRT; ++m) {
      const int rt = row_tile(m);
      if (rt >= NRT) continue;
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        T* p = sS(b) + (16 * ct + i16) * PS + 16 * rt + 4 * g;
        const f32x4_t s = Sacc[m][ct];
        if constexpr (BF) {
          *reinterpret_cast<uint2*>(p) =
              make_uint2(pack_bf16x2(s[0], s[1]), pack_bf16x2(s[2], s[3]));
        } else {
          *reinterpret_cast<float4*>(p) = make_float4(s[0], s[1], s[2], s[3]);
        }
      }
    }
  };

  // Causal mask of the within-chunk scores (the same for every chunk): lane
  // (key slot 4h + t of block jb2, query il) keeps the score iff the key
  // 32 jb2 + 8 g + 4 h + t is not after the query.
  const int il = 16 * w + i16;
  bool keep[2][8];
#pragma unroll
  for (int jb2 = 0; jb2 < 2; ++jb2)
#pragma unroll
    for (int e = 0; e < 8; ++e) keep[jb2][e] = 32 * jb2 + 8 * g + e <= il;

  // Gated segment-sum pass: log2 of the segment's total decay (-inf once a
  // reset has been passed).
  float seg_log = 0.0f;

  // One chunk, computed from LDS copy b and query set b: stage chunk c + 1
  // from ring slot `nx` into copy 1 - b, refill the slot with chunk c + P,
  // then the outputs (OUT) and the state update of chunk c.
  auto iteration = [&](int c, St& nx, auto bc) __attribute__((always_inline)) {
    constexpr int b = decltype(bc)::value;
    const int cb = c * C;

    write_tiles(nx, 1 - b);
    take_q(nx, 1 - b);
    stage_gate(nx, 1 - b, c + 1);
    issue(c + 1 + P, nx);

    // Gated form: decays of this chunk.  Query il carries the state from
    // before the chunk with factor fq (0 past a reset); the chunk as a whole
    // scales the carried state by fc.
    float Gq = 0.0f, fq = 1.0f, fc = 1.0f;
    int Lq = -1;
    if constexpr (GATED) {
      // chunk-end values are the same for every lane: keep them scalar
      fc = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(
                                         __builtin_bit_cast(int, sF[b][C - 1])));
      if constexpr (OUT) {
        if (qwave) {
          Gq = sG[b][il];
          Lq = sL[b][il];
          fq = sF[b][il];
        }
      } else {
        const float Ge = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(
                                                       __builtin_bit_cast(int, sG[b][C - 1])));
        const int Le = __builtin_amdgcn_readfirstlane(sL[b][C - 1]);
        seg_log = Le >= 0 ? -__builtin_inff() : seg_log + Ge;
      }
    }

    f32x4_t O[OUT ? NCT : 1];
    frag qraw = E::zero();
    if constexpr (OUT) if (qwave) {
      if constexpr (MAP == MAP_TAYLOR2) {
        f32x16_t qx;
#pragma unroll
        for (int u = 0; u < SH::NQU; ++u) {
          float part[EPU];
          unpack16<T>(qs[b][u], part);
#pragma unroll
          for (int e = 0; e < EPU; ++e) qx[u * EPU + e] = part[e];
        }
        float f[8], f8[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          qb8[t] = (g & 1) ? qx[8 + t] : qx[t];
          qa8[t] = 0.5f * ((g >> 1) ? qx[2 * t + 1] : qx[2 * t]);
          f[t] = g < 2 ? qb8[t] : 0.0f;
          const float g0 = t == 0 ? 1.0f : qx[t > 0 ? t - 1 : 0];
          const float g2 = t == 0 ? qx[15] : 0.0f;
          f8[t] = g == 0 ? g0 : (g == 1 ? qx[7 + t] : (g == 2 ? g2 : 0.0f));
        }
        qraw = E::make(f);
        q8f = E::make(f8);
      }
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) O[ct] = {0.0f, 0.0f, 0.0f, 0.0f};

      // prefix term: O^T += S'^T phi(Q)^T
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const frag bq = q_frag(b, kb);
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
          const frag av = E::load8(sS(b) + (16 * ct + i16) * PS + 32 * kb + 8 * g);
          E::mma(O[ct], av, bq);
        }
      }
      if constexpr (GATED) {
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) O[ct] *= fq;
      }
    }
    if constexpr (GATED) {
#pragma unroll
      for (int m = 0; m < SH::MAXRT; ++m)
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) Sacc[m][ct] *= fc;
    }

    // Scheduling hint: interleave the staging arithmetic of chunk c + 1 (phi
    // of k and q, independent of this chunk's products) with this chunk's
    // first MFMAs, eight VALU instructions after each MFMA, so that the
    // matrix unit is not idle while the wave computes phi.  Measured on the
    // ELU1 shapes only; the TAYLOR2 schedule is left to the compiler.
    if constexpr (MAP == MAP_ELU1) {
      constexpr int kInterleave = OUT ? NKB * NCT : SH::MAXRT * NCT * 2;
#pragma unroll
      for (int i = 0; i < kInterleave; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);  // eight VALU
      }
    }

    // Per 32-token key block: the V' operands serve both the within-chunk
    // product (A-operand, V'^T) and the state update (B-operand, V').
#pragma unroll
    for (int jb2 = 0; jb2 < 2; ++jb2) {
      frag vf[NCT - 1];
#pragma unroll
      for (int ct = 0; ct < NCT - 1; ++ct) vf[ct] = v_frag(b, jb2, ct);

      // Gated form: weight u of key 32 jb2 + 8 g + e at the chunk end (zero
      // across a reset, and past the segment end so that those tokens add
      // nothing to the state).
      float u[8];
      if constexpr (GATED) {
        const float4 u0 = *reinterpret_cast<const float4*>(&sU[b][32 * jb2 + 8 * g]);
        const float4 u1 = *reinterpret_cast<const float4*>(&sU[b][32 * jb2 + 8 * g + 4]);
        u[0] = u0.x; u[1] = u0.y; u[2] = u0.z; u[3] = u0.w;
        u[4] = u1.x; u[5] = u1.y; u[6] = u1.z; u[7] = u1.w;
      }

      if constexpr (OUT) if (qwave) {
        // within-chunk term: scores^T of this key block against the wave's
        // queries (key blocks wholly after them come out fully masked)
        frag bq[SH::NKBS];
#pragma unroll
        for (int kbs = 0; kbs < SH::NKBS; ++kbs) {
          if constexpr (MAP == MAP_ELU1) bq[kbs] = q_frag(b, kbs); else bq[kbs] = qraw;
        }
        CT::template within_chunk<GATED>(sK(b), vf, bq, keep[jb2], ones, O, jb2, lane,
                                         GATED ? &sG[b][32 * jb2 + 8 * g] : nullptr, Gq, Lq);
      }

      // state update: S' += phi(K)^T V' for this wave's row tiles
#pragma unroll
      for (int m = 0; m < SH::MAXRT; ++m) {
        const int rt = row_tile(m);
        if (rt >= NRT) continue;
        const frag ak = kt_frag(b, rt, jb2, u);
#pragma unroll
        for (int ct = 0; ct < NCT - 1; ++ct) E::mma(Sacc[m][ct], ak, vf[ct]);
        E::mma(Sacc[m][NCT - 1], ak, ones);
      }
    }

    if constexpr (OUT) if (qwave) {
      // normalise and write y (query il of this chunk; rows past the
      // segment end fall outside the store range)
      const float den = __shfl(O[NCT - 1][0], i16, 64);
      const float rden = GATED && !a.normalize ? 1.0f : fast_rcp(den);
      const uint32_t yrow = ((uint32_t)(cb + il) * DV + 4 * g) * ES;
#pragma unroll
      for (int ct = 0; ct < NCT - 1; ++ct) {
        const f32x4_t o = O[ct];
        const uint32_t off = yrow + 16 * ct * ES;
        if constexpr (BF) {
          const uint2 d = make_uint2(pack_bf16x2(o[0] * rden, o[1] * rden),
                                     pack_bf16x2(o[2] * rden, o[3] * rden));
          __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2_t, d), ry, off, 0, 0);
        } else {
          const uint4 d = make_uint4(__float_as_uint(o[0] * rden), __float_as_uint(o[1] * rden),
                                     __float_as_uint(o[2] * rden), __float_as_uint(o[3] * rden));
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, d), ry, off, 0, 0);
        }
      }
    }
    if constexpr (OUT) {
      // state through chunk c for the prefix term of chunk c + 1
      if constexpr (NSB == 1) lds_barrier();  // every wave is done with sS
      publish_state(1 - b);
    }
    lds_barrier();
  };

  // ------------------------------------------------------------ prologue --
#pragma unroll
  for (int s = 0; s < P; ++s) issue(s, st[s]);
  if constexpr (OUT) publish_state(0);
  write_tiles(st[0], 0);
  take_q(st[0], 0);
  stage_gate(st[0], 0, 0);
  issue(P, st[0]);
  lds_barrier();

  // Chunk c is staged from ring slot c % P into LDS copy c % 2; one trip of
  // P chunks keeps every ring index and copy index a compile-time constant.
  // The loop runs whole trips with no branch between the copies; chunks
  // past the segment end are inert (their loads are out of range and read
  // zeros, their ones column is masked, and no y row of theirs is in the
  // store range), so at most P - 1 empty chunks are walked at the end.
  for (int c0 = 0; c0 < nchunks; c0 += P) {
    static_for<0, P>([&](auto s) __attribute__((always_inline)) {
      constexpr int S = decltype(s)::value;
      iteration(c0 + S, st[(S + 1) % P], std::integral_constant<int, S % 2>{});
    });
  }

  // Every token walked past the segment end (the tail of the last chunk and
  // the empty chunks of the last trip) read k = 0 and v = 0: it added
  // nothing to the value columns and phi(0) to the z column.  Take that
  // back: phi(0) is 1 in every ELU1 feature, and in the TAYLOR2 constant
  // feature (internal row 256) only.  (The gated form gives those tokens
  // weight 0 instead, so that a strongly decayed z is not left to cancel.)
  if constexpr (!GATED) {
    const float n_pad = (float)(((nchunks + P - 1) / P) * P * C - ntok);
#pragma unroll
    for (int m = 0; m < SH::MAXRT; ++m) {
      const int rt = row_tile(m);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int row = 16 * rt + 4 * g + t;
        const bool unit_feature = MAP == MAP_ELU1 ? row < DK : row == 256;
        if (i16 == 0 && unit_feature) Sacc[m][NCT - 1][t] -= n_pad;
      }
    }
  }

  // ------------------------------------------------------------ epilogue --
  if constexpr (OUT) {
    if (seg == a.nseg - 1 && a.S_out != nullptr) {
#pragma unroll
      for (int m = 0; m < SH::MAXRT; ++m) {
        const int rt = row_tile(m);
        if (rt >= NRT) continue;
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
          state_out_tile<MAP, DK, DV>(a.S_out, a.z_out, a.sym != 0, bh, rt,
                                      ct, lane, Sacc[m][ct]);
      }
    }
  } else {
    f32x4_t* p = reinterpret_cast<f32x4_t*>(
        a.ws + ((size_t)bh * a.nslot + seg + 1) * SH::SLOT);
#pragma unroll
    for (int m = 0; m < SH::MAXRT; ++m) {
      const int rt = row_tile(m);
      if (rt >= NRT) continue;
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) p[(rt * NCT + ct) * 64 + lane] = Sacc[m][ct];
    }
    if constexpr (GATED) {
      if (tid == 0) a.ws_log[(size_t)bh * a.nslot + seg + 1] = seg_log;
    }
  }
}

// Exclusive prefix over the summed parts, in place: slot s <- init +
// sum_{p<s} T_p, where slot p+1 held part p's sum T_p and init is the
// initial state (output segment s then reads slot s * sum_split).  Gated
// form: slot s <- 2^l_s slot(s-1) + T_(s-1), with l_s the log2 decay of part
// s - 1 (ws_log).  Used when there are too many parts per head for each
// output workgroup to add up its predecessors itself.
//
// Two levels, so that the serial chain per element is a quarter of the
// slots: a workgroup takes 64 float4 elements of one head's slots, and its
// 4 waves split the slots 1 .. nscan-1 into 4 contiguous groups.  Each
// thread forms its group's total (and the group's log2 decay), the group
// totals meet in LDS, each thread combines the totals of the groups before
// its own into the prefix entering its group, and then rewrites its group's
// slots as running prefixes.
constexpr int kScanCols = 64;    // float4 elements per workgroup
constexpr int kScanGroups = 4;   // slot groups (one per wave)

template <int MAP, int DK, int DV>
__global__ __launch_bounds__(256) void seg_scan_kernel(PrefillArgs a) {
  using SS = StateShape<MAP, DK, DV>;
  constexpr int Q = SS::SLOT / 4;  // float4 per slot
  static_assert(Q % kScanCols == 0, "a slot is whole 64-element columns");
  constexpr int TILES = Q / kScanCols;
  __shared__ f32x4_t tot[kScanGroups][kScanCols];
  __shared__ float ltot[kScanGroups];
  const int bh = blockIdx.x / TILES;
  const int col = threadIdx.x % kScanCols;
  const int e4 = (blockIdx.x % TILES) * kScanCols + col;
  const int grp = threadIdx.x / kScanCols;  // wave-uniform
  const int nscan = (a.nseg - 1) * a.sum_split + 1;  // slot 0 and every sum
  const int per = (nscan - 1 + kScanGroups - 1) / kScanGroups;
  const int s_lo = 1 + grp * per;
  const int s_hi = s_lo + per < nscan ? s_lo + per : nscan;
  f32x4_t* p = reinterpret_cast<f32x4_t*>(a.ws + (size_t)bh * a.nslot * SS::SLOT) + e4;
  const float* lg = a.ws_log != nullptr ? a.ws_log + (size_t)bh * a.nslot : nullptr;

  // group total and the group's log2 decay
  f32x4_t t = {0.0f, 0.0f, 0.0f, 0.0f};
  float lsum = 0.0f;
#pragma unroll 8
  for (int s = s_lo; s < s_hi; ++s) {
    const f32x4_t v = p[(size_t)s * Q];
    if (lg != nullptr) {
      t *= __builtin_amdgcn_exp2f(lg[s]);
      lsum += lg[s];
    }
    t += v;
  }
  tot[grp][col] = t;
  if (col == 0) ltot[grp] = lsum;
  lds_barrier();

  // the state entering this group: the initial state, then earlier groups
  f32x4_t run = {0.0f, 0.0f, 0.0f, 0.0f};
  if (a.S_in != nullptr) {
    const int rt = e4 / (SS::NCT * 64);
    const int ct = (e4 / 64) % SS::NCT;
    run = state_in_tile<MAP, DK, DV>(a.S_in, a.z_in, a.sym != 0, bh, rt, ct, e4 % 64);
  }
  for (int g = 0; g < grp; ++g) {
    if (lg != nullptr) run *= __builtin_amdgcn_exp2f(ltot[g]);
    run += tot[g][col];
  }
  if (grp == 0) p[0] = run;
#pragma unroll 8
  for (int s = s_lo; s < s_hi; ++s) {
    if (lg != nullptr) run *= __builtin_amdgcn_exp2f(lg[s]);
    run += p[(size_t)s * Q];
    p[(size_t)s * Q] = run;
  }
}

template <int MAP, typename T, int DK, int DV, bool GATED>
hipError_t launch_prefill(const PrefillArgs& a, hipStream_t st) {
  using SS = StateShape<MAP, DK, DV>;
  constexpr int NT = 64 * kChunkWaves<MAP, T, GATED>;
  if (a.nseg > 1) {
    hipLaunchKernelGGL((chunk_kernel<MAP, T, DK, DV, false, GATED>),
                       dim3(a.BH * (a.nseg - 1) * a.sum_split), dim3(NT), 0, st, a);
    if (a.prefix_mode == 2) {
      hipLaunchKernelGGL((seg_scan_kernel<MAP, DK, DV>),
                         dim3((unsigned)(a.BH * (SS::SLOT / 4 / kScanCols))), dim3(256), 0,
                         st, a);
    }
  }
  hipLaunchKernelGGL((chunk_kernel<MAP, T, DK, DV, true, GATED>),
                     dim3(a.BH * a.nseg), dim3(NT), 0, st, a);
  return hipGetLastError();
}

}  // namespace linattn
