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
// Parallel layout.  A workgroup of NW waves owns one (batch*head, segment):
// a run of consecutive chunks walked in order.  Waves 0..3 produce the
// outputs of the chunk's 16-token tiles (all value columns).  With NW = 4
// every wave w also owns state row tiles w, w+4, ... (16 features each)
// across all columns.  The bf16 Taylor kernels have NW = 8 (kChunkWaves);
// in their output kernels waves 4..7 own every state row tile and waves
// 0..3 none (the role split below), and in their segment-sum kernels wave w
// owns tiles w, w+8, ....  The plain bf16 ELU1 segment-sum kernel at
// d_k = 64 also has NW = 8: waves w and w+4 share row tile w & 3, wave w
// owning column tiles 0..2 and wave w+4 the rest (the column split).  A
// bf16 (or fp32) copy of S' in LDS, laid out
// column-major, feeds the inter term of every output wave.  K, V tiles are
// staged through LDS (bf16 row-major, read transposed; fp32 transposed) so
// that every MFMA operand is one or two LDS reads; the next chunks' global
// loads are issued before the current chunk is computed.
//
// Several segments per head: chunk_kernel<OUT = false> sums each segment's
// state, seg_scan_kernel turns those sums into exclusive prefixes (plus the
// optional initial state), and chunk_kernel<OUT = true> starts each segment
// from its prefix.  With one segment per head only the last kernel runs.
// At two segments per head (every map, plain or gated) one kernel runs
// instead (chunk_kernel<..., PRE = true>): the
// workgroup of segment 1 walks segment 0 first, advancing the state
// without outputs.
//
// Feature order inside the kernels.  ELU1 uses the natural order.  TAYLOR2
// (d_k = 16) keeps each unordered pair of key coordinates once: k_a k_b
// multiplies q_b k_b q_a k_a and q_a k_a q_b k_b alike, so the second-order
// term sum_{a,b} q_a q_b k_a k_b / 2 equals sum_a q_a^2 k_a^2 / 2 +
// sum_{a<b} q_a q_b k_a k_b, and the state needs 136 pair rows instead of
// 256 (taylor_row: rows 0..127 hold the pairs (a, a + t mod 16), a = r / 8,
// t = r mod 8, rows 128..135 the pairs (t, t + 8)), then the constant (136),
// the 16 linear features (137..152) and 7 zero pads: 160 = 5 MFMA K blocks.
// The query carries the weights (q_a^2 / 2 for a square, q_a q_b for a
// pair).  The exported states use the pages' order [1, x, vec(x x^T)/sqrt2]
// and are converted at the boundary: only the symmetric part of an ordered
// pair block reaches any output, so an initial state's antisymmetric part
// is carried to the exported state (times the total decay in the gated
// form) without entering the walk.
#pragma once

#include "device.hpp"
#include "shapes.hpp"

namespace linattn {

// Waves per chunk workgroup.  The Taylor state (10 row tiles) is spread
// over 8 waves for bf16 inputs, so that each holds fewer accumulators and
// two waves share a SIMD; in the output kernels waves 0-3 then make the
// outputs and waves 4-7 own the state (the role split below).  Measured on
// one MI355X at B=8 H=16 N=2048, with the earlier 18-tile ordered-pair
// state: 111.7 -> 106.6 us per call with every wave doing both, 79.8 ->
// 70.7 us from the role split, and for the gated form 107.2 -> 83.6 us
// (4 waves -> 8 split; 8 waves without the split spilled).
// Float tiles keep 4 waves.  The plain bf16 ELU1 segment-sum kernel at
// d_k = 64 also runs 8 waves: its 4 state row tiles are each shared by two
// waves that own different column tiles (the column split below), so that
// each SIMD holds two waves of a walk whose per-chunk chain is short.
template <int MAP, typename T, int DK, bool GATED, bool OUT>
constexpr int kChunkWaves =
    (MAP != MAP_ELU1 && sizeof(T) == 2) ||
            (MAP == MAP_ELU1 && sizeof(T) == 2 && DK == 64 && !GATED && !OUT)
        ? 8
        : 4;

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
  // Column stride of the LDS state copy.  The bf16 TAYLOR2 copy is unpadded
  // and swizzled instead (kStateSwizzle below); the others are padded by 16
  // bytes.
  static constexpr bool kStateSwizzle = MAP == MAP_TAYLOR2 && sizeof(T) == 2;
  static constexpr int PS = kStateSwizzle ? SS::DP : SS::DP + EPU;
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

// Internal Taylor rows.  The key features k_a k_b of the pair (a, b) and
// of (b, a) are equal, so the state keeps each unordered pair once (the
// query side carries q_a q_b, or q_a^2 / 2 for a square, so that
// phi(q).phi(k) = 1 + q.k + (q.k)^2 / 2 holds):
//   r < 128:         pair (a, b), a = r / 8, b = (a + r % 8) mod 16: the 8
//                    coordinates that follow a circularly (a itself first),
//                    so every pair at circular distance 0..7 appears once;
//   128 <= r < 136:  pair (r - 128, r - 120), the pairs at distance 8;
//   136:             the constant feature;  137 .. 152: the linear ones;
//   153 .. 159:      zero padding (10 row tiles, 5 MFMA K blocks).
// Returns the kind of row r: 0 pair (a, b set), 1 constant, 2 linear (a
// set to the coordinate), 3 padding.
__device__ __forceinline__ int taylor_row(int r, int& a, int& b) {
  a = 0;
  b = 0;
  if (r < 128) {
    a = r >> 3;
    b = (a + (r & 7)) & 15;
    return 0;
  }
  if (r < 136) {
    a = r - 128;
    b = r - 120;
    return 0;
  }
  if (r == 136) return 1;
  if (r < 153) {
    a = r - 137;
    return 2;
  }
  return 3;
}

// Rows of the transposed key tile (k_0 .. k_15, then a row of ones and a
// row of zeros) whose product is lane i16's key feature in state row tile
// rt: internal row 16 rt + i16 (taylor_row) is sKT[pa] * sKT[pb], so that
// the pairs, the constant (ones x ones), the linear features (k_a x ones)
// and the padding (zeros x ones) all take the same two reads and one
// product.  Tiles past the last (unused accumulators) read zeros.
constexpr int kKtOnes = 16, kKtZeros = 17;
__device__ __forceinline__ void taylor_kt_rows(int rt, int i16, int& pa, int& pb) {
  if (rt < 8) {
    pa = 2 * rt + (i16 >> 3);
    pb = (pa + (i16 & 7)) & 15;
  } else if (rt == 8) {
    pa = i16 < 8 ? i16 : (i16 == 8 ? kKtOnes : i16 - 9);
    pb = i16 < 8 ? i16 + 8 : kKtOnes;
  } else {
    pa = rt == 9 && i16 <= 8 ? i16 + 7 : kKtZeros;
    pb = kKtOnes;
  }
}

// Exported feature rows of a head's state.
template <int MAP, int DK, int DV>
__device__ __forceinline__ int ext_rows(bool sym) {
  return MAP == MAP_TAYLOR2 && sym ? kSymD<DK> : StateShape<MAP, DK, DV>::D;
}

// Exported rows of the Taylor maps: ordered pair (a, b) at 17 + 16 a + b;
// unordered pair {a, b}, a <= b, at 17 + a d - a (a - 1) / 2 + (b - a).
__device__ __forceinline__ int ordered_pair_row(int a, int b) { return 17 + 16 * a + b; }
__device__ __forceinline__ int sym_pair_row(int a, int b) {
  const int lo = a < b ? a : b, hi = a < b ? b : a;
  return 17 + lo * 16 - lo * (lo - 1) / 2 + (hi - lo);
}

// One column (col < DV: S, col == DV: z) of the exported layout of
// sequence bh, as a row accessor.
struct ExtCol {
  const float* S;
  const float* z;
  int D, DV, bh, col;
  __device__ __forceinline__ float at(int e) const {
    return col < DV ? S[((size_t)bh * D + e) * DV + col] : z[(size_t)bh * D + e];
  }
};

// One lane's 4 values of state tile (rt, ct) read from the exported
// layout S [D, DV], z [D] of sequence bh, converted to the internal one.
// Taylor pair rows take the pair's symmetric part: the ordered layout's
// (a, b) and (b, a) rows are added (their antisymmetric part contributes
// nothing to any output: q^T A q = 0 for antisymmetric A; the export
// carries it over, state_out_tile).
template <int MAP, int DK, int DV>
__device__ __forceinline__ f32x4_t state_in_tile(const float* S_in,
                                                 const float* z_in, bool sym,
                                                 int bh, int rt, int ct,
                                                 int lane) {
  const int col = 16 * ct + (lane & 15);
  f32x4_t r;
  if constexpr (MAP == MAP_ELU1) {
    // ELU1 keeps its own form of the gather (and of the export below): the
    // compiled schedule of the whole ELU1 output kernel follows it, and the
    // shared row-accessor form cost that kernel 1.5 us (43.8 -> 45.3 us at
    // B=8 H=8 N=4096 d=64) through a different instruction order in its loop
    const int D = DK;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int row = 16 * rt + 4 * (lane >> 4) + t;
      const float f = 1.0f;
      const int e = row < DK ? row : -1;
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
  const ExtCol in{S_in, z_in, ext_rows<MAP, DK, DV>(sym), DV, bh, col};
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int row = 16 * rt + 4 * (lane >> 4) + t;
    float val = 0.0f;
    if (col <= DV) {
      int a, b;
      const int kind = taylor_row(row, a, b);
      if (kind == 0) {
        if (sym)
          val = in.at(sym_pair_row(a, b)) * (a == b ? kSqrt2 : 1.0f);
        else if (a == b)
          val = in.at(ordered_pair_row(a, a)) * kSqrt2;
        else
          val = (in.at(ordered_pair_row(a, b)) + in.at(ordered_pair_row(b, a))) * kInvSqrt2;
      } else if (kind == 1) {
        val = in.at(0);
      } else if (kind == 2) {
        val = in.at(1 + a);
      }
    }
    r[t] = val;
  }
  return r;
}

// Export of one lane's 4 values of state tile (rt, ct).  An ordered Taylor
// pair (a != b) is written to both (a, b) and (b, a); when the call started
// from an ordered S_in, whose pair rows need not agree, their
// antisymmetric part (S_in(a,b) - S_in(b,a)) / 2 is carried over, scaled by
// anti_scale (1, or the gated form's total decay).  In place (S_out is
// S_in) the lane reads both rows before it writes them.
template <int MAP, int DK, int DV>
__device__ __forceinline__ void state_out_tile(float* S_out, float* z_out,
                                               bool sym, int bh, int rt,
                                               int ct, int lane,
                                               const f32x4_t& v,
                                               const float* S_in = nullptr,
                                               const float* z_in = nullptr,
                                               float anti_scale = 1.0f) {
  const int D = ext_rows<MAP, DK, DV>(sym);
  const int col = 16 * ct + (lane & 15);
  if (col > DV) return;
  if constexpr (MAP == MAP_ELU1) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int row = 16 * rt + 4 * (lane >> 4) + t;
      if (row >= DK) continue;
      const float val = v[t] / 1.0f;
      if (col < DV)
        S_out[((size_t)bh * D + row) * DV + col] = val;
      else
        z_out[(size_t)bh * D + row] = val;
    }
    return;
  }
  float* out = col < DV ? S_out : z_out;
  auto addr = [&](int e) -> size_t {
    return col < DV ? ((size_t)bh * D + e) * DV + col : (size_t)bh * D + e;
  };
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int row = 16 * rt + 4 * (lane >> 4) + t;
    {
      int a, b;
      const int kind = taylor_row(row, a, b);
      if (kind == 0) {
        if (sym) {
          out[addr(sym_pair_row(a, b))] = v[t] * (a == b ? kInvSqrt2 : 1.0f);
        } else if (a == b) {
          out[addr(ordered_pair_row(a, a))] = v[t] * kInvSqrt2;
        } else {
          float anti = 0.0f;
          if (S_in != nullptr) {
            const ExtCol in{S_in, z_in, D, DV, bh, col};
            anti = 0.5f * (in.at(ordered_pair_row(a, b)) - in.at(ordered_pair_row(b, a))) *
                   anti_scale;
          }
          const float base = v[t] * kInvSqrt2;
          out[addr(ordered_pair_row(a, b))] = base + anti;
          out[addr(ordered_pair_row(b, a))] = base - anti;
        }
      } else if (kind == 1) {
        out[addr(0)] = v[t];
      } else if (kind == 2) {
        out[addr(1 + a)] = v[t];
      }
    }
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
    if (32 * kbs >= DK) return E::zero();
    // Lanes whose features lie past DK meet zero query slots (the operand
    // builders zero every padded feature), so they read an in-range block
    // rather than branch around the load: finite times zero adds nothing.
    const int f0 = (32 * kbs + 8 * (lane >> 4)) & (DK - 1);
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

// An empty asm statement that takes each argument as read and written: the
// compiler must assume new values, so nothing derived from them before this
// point is reused after it.  Only when ON.
template <class A>
__device__ __forceinline__ void opaque1(A& a) {
  asm volatile("" : "+v"(a));
}
template <bool ON, class... A>
__device__ __forceinline__ void opaque_if(A&... a) {
  if constexpr (ON) (opaque1(a), ...);
}

template <int I, int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

// PRE: the prefix_mode 3 output kernel, a separate instantiation so that
// the other plans keep their own compiled walk.
template <int MAP, typename T, int DK, int DV, bool OUT, bool GATED, bool PRE = false>
__global__ __launch_bounds__((64 * kChunkWaves<MAP, T, DK, GATED, OUT>)) void chunk_kernel(PrefillArgs a) {
  using SH = PrefillShape<MAP, T, DK, DV, kChunkWaves<MAP, T, DK, GATED, OUT>>;
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
  // source of phi(K)^T.  sKT: K transposed (float, and TAYLOR2, where it is
  // fp32 for every input type so that the key products read it without
  // unpacking, with a row of ones and a row of zeros appended,
  // taylor_kt_rows; row stride KCS).  sS: the
  // state S'^T in the MFMA operand precision, column-major; two copies
  // unless that does not fit next to the tiles (float TAYLOR2).
  constexpr bool kNeedK = OUT || (BF && MAP == MAP_ELU1);
  constexpr bool kNeedKT = !(BF && MAP == MAP_ELU1);
  constexpr int K_EL = kNeedK ? (BF ? C * RTK::STRIDE : C * KS) : EPU;
  using KTT = std::conditional_t<MAP == MAP_TAYLOR2, float, T>;
  constexpr int KCS = C + 16 / (int)sizeof(KTT);  // padded by 16 bytes
  constexpr int KT_EL = kNeedKT ? (MAP == MAP_ELU1 ? DK : DK + 2) * KCS : 4;
  constexpr int V_EL = BF ? C * RTV::STRIDE : DV * CS;
  constexpr int S_EL = OUT ? SH::NCOL * PS : EPU;
  constexpr int kTileBytes = 2 * ((K_EL + V_EL) * (int)sizeof(T) + KT_EL * (int)sizeof(KTT)) +
                             (GATED ? 2 * C * 16 : 0);
  constexpr int NSB = kTileBytes + 2 * S_EL * (int)sizeof(T) <= 160 * 1024 ? 2 : 1;
  __shared__ __align__(16) T sK0[K_EL];
  __shared__ __align__(16) T sK1[K_EL];
  __shared__ __align__(16) KTT sKT0[KT_EL];
  __shared__ __align__(16) KTT sKT1[KT_EL];
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
  const int i16 = lane & 15;
  const int g = lane >> 4;

  // OUT: one workgroup per output segment.  Segment sums: one per part of
  // every segment but the last (sum_split parts per segment).
  const int nseg_here = OUT ? a.nseg : (a.nseg - 1) * a.sum_split;
  const int seg_chunks = OUT ? a.seg_chunks : a.seg_chunks / a.sum_split;
  // The PRE kernel places the two workgroups of a head on one XCD (the
  // hardware deals workgroup x + 8 r to XCD x) when the heads fill whole
  // groups of 8: head x + 8 (r / 2), segment r % 2.  Segment 1's pre-pass
  // reads segment 0's k and v shortly before segment 0's workgroup does, so
  // most of those second reads hit that XCD's L2.
  const bool same_xcd = PRE && (a.BH % 8) == 0;
  const int bh = same_xcd ? (int)(blockIdx.x % 8 + 8 * (blockIdx.x / 16))
                          : (int)(blockIdx.x / nseg_here);
  const int seg = same_xcd ? (int)((blockIdx.x / 8) % 2) : (int)(blockIdx.x % nseg_here);
  const int64_t N = a.N;
  int64_t tok_begin = (int64_t)seg * seg_chunks * C;
  int64_t tok_end = tok_begin + (int64_t)seg_chunks * C;
  // prefix_mode 3 (two segments, no segment-sum pass; the PRE kernel):
  // both workgroups of a head walk from token 0.  Segment 0 covers
  // the first seg_chunks chunks; segment 1 walks those chunks first as a
  // pre-pass that only advances the state (chunks before c_out), then makes
  // the outputs of the rest of the sequence.
  constexpr bool kPrePass = PRE;
  static_assert(!PRE || OUT, "the pre-pass kernels");
  int c_out = 0;
  if constexpr (kPrePass) {
    c_out = seg * seg_chunks;
    tok_begin = 0;
    tok_end = seg == 0 ? (int64_t)seg_chunks * C : N;
  }
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

  // ------------------------------------------------------------ roles ----
  // The 8-wave Taylor output kernels run two specialised walks side by
  // side: waves 0-3 make the chunk's outputs and own no state; waves 4-7 own
  // every state row tile (tiles w-4 and w of the pair features, then tiles
  // 8 and 9, the distance-8 pairs, the constant and the linear features, on
  // waves 4 and 5).  The 8-wave ELU1
  // segment-sum kernel runs two column halves: waves w and w+4 share row
  // tile w & 3, wave w owning its first column tiles and wave w+4 the rest.
  // Each walk is straight-line code with registers of its own, and all pass
  // the same barriers.  Other kernels run one walk in which every wave does
  // both outputs and state.
  auto walk = [&](auto role_c) __attribute__((always_inline)) {
    // 1: outputs, 2: state (Taylor output kernels); 3, 4: the column halves
    // of the ELU1 segment sums
    constexpr int ROLE = decltype(role_c)::value;
    const bool qwave_r = ROLE == 1;
    constexpr int kMT = ROLE == 1 || ROLE >= 3 ? 1 : (SH::NRT + 3) / 4;
    static_assert(ROLE >= 3 || (MAP != MAP_ELU1 && SH::NRT == 10), "the split owns 8 + 2 tiles");
    static_assert(ROLE < 3 || (!OUT && SH::NRT == 4), "the column split pairs waves w, w + 4");
    // state row tile m of this wave (a tile index >= NRT means none)
    auto row_tile = [&](int m) __attribute__((always_inline)) -> int {
      return ROLE == 1 ? SH::NRT + 64 : ROLE == 2 ? (w - 4) + 4 * m : (w & 3);
    };
    // the state column tiles this wave owns
    constexpr int kCT0 = ROLE == 4 ? (NCT + 1) / 2 : 0;
    constexpr int kCT1 = ROLE == 3 ? (NCT + 1) / 2 : NCT;
    const int tid_o = tid, lane_o = lane, i16_o = i16, g_o = g;
    {
      // mutable copies of the lane indices (see opaque_if in the walk)
      int tid = tid_o, lane = lane_o, i16 = i16_o, g = g_o;
#include "chunk_walk.inc"
    }
  };

  if constexpr (OUT && NW == 8) {
    if (w < 4)
      walk(std::integral_constant<int, 1>{});
    else
      walk(std::integral_constant<int, 2>{});
  } else if constexpr (MAP == MAP_ELU1 && NW == 8) {
    if (w < 4)
      walk(std::integral_constant<int, 3>{});
    else
      walk(std::integral_constant<int, 4>{});
  } else {
    constexpr int ROLE = 0;  // every wave: outputs (if any) and state
    const bool qwave_r = qwave;
    constexpr int kMT = SH::MAXRT;
    constexpr int kCT0 = 0, kCT1 = NCT;
    auto row_tile = [&](int m) __attribute__((always_inline)) -> int { return w + NW * m; };
#include "chunk_walk.inc"
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
  constexpr int NT = 64 * kChunkWaves<MAP, T, DK, GATED, true>;
  constexpr int NT_SUM = 64 * kChunkWaves<MAP, T, DK, GATED, false>;
  if (a.nseg > 1 && a.prefix_mode < 3) {
    hipLaunchKernelGGL((chunk_kernel<MAP, T, DK, DV, false, GATED>),
                       dim3(a.BH * (a.nseg - 1) * a.sum_split), dim3(NT_SUM), 0, st, a);
    if (a.prefix_mode == 2) {
      hipLaunchKernelGGL((seg_scan_kernel<MAP, DK, DV>),
                         dim3((unsigned)(a.BH * (SS::SLOT / 4 / kScanCols))), dim3(256), 0,
                         st, a);
    }
  }
  if (a.prefix_mode == 3) {
    hipLaunchKernelGGL((chunk_kernel<MAP, T, DK, DV, true, GATED, true>),
                       dim3(a.BH * a.nseg), dim3(NT), 0, st, a);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((chunk_kernel<MAP, T, DK, DV, true, GATED>),
                     dim3(a.BH * a.nseg), dim3(NT), 0, st, a);
  return hipGetLastError();
}

}  // namespace linattn
