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
// a run of consecutive chunks walked in order.  Wave w produces the outputs
// of the chunk's 16-token tile w (all value columns) and owns state row
// tiles w, w+4, w+8, ... (16 features each) across all columns.  A bf16 (or
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

template <int MAP, typename T, int DK, int DV>
struct PrefillShape : StateShape<MAP, DK, DV> {
  using SS = StateShape<MAP, DK, DV>;
  static constexpr int C = 64;
  static constexpr int NW = 4;
  static constexpr int NT = 64 * NW;
  static constexpr int MAXRT = (SS::NRT + NW - 1) / NW;
  static constexpr int EPU = Elem<T>::kPer16B;
  static constexpr int KS = DK + EPU;       // LDS row strides (elements),
  static constexpr int CS = C + EPU;        // padded by 16 bytes
  static constexpr int PS = SS::DP + EPU;
  static constexpr int UK = C * DK / EPU;   // 16-byte units per k tile
  static constexpr int UV = C * DV / EPU;
  static constexpr int NUK = (UK + NT - 1) / NT;
  static constexpr int NUV = (UV + NT - 1) / NT;
  static constexpr int KUR = DK / EPU;      // units per k row
  static constexpr int VUR = DV / EPU;
  static constexpr int NQU = MAP == MAP_ELU1 ? SS::NKB * 8 / EPU : DK / EPU;
  static constexpr int NKBS = (DK + 31) / 32;  // K blocks of the scores
};

// Internal feature row -> exported row (or -1 for padding) and the factor
// that converts an exported value into the internal one.
template <int MAP, int DK>
__device__ __forceinline__ int ext_row(int r, float& to_internal) {
  to_internal = 1.0f;
  if (MAP == MAP_ELU1) return r < DK ? r : -1;
  if (r < 256) {
    to_internal = kSqrt2;
    return 17 + r;
  }
  return r < 273 ? r - 256 : -1;
}

// One lane's 4 values of state tile (rt, ct) read from the exported
// layout S [D, DV], z [D] of sequence bh, converted to the internal one.
template <int MAP, int DK, int DV>
__device__ __forceinline__ f32x4_t state_in_tile(const float* S_in,
                                                 const float* z_in, int bh,
                                                 int rt, int ct, int lane) {
  using SS = StateShape<MAP, DK, DV>;
  f32x4_t r;
  const int col = 16 * ct + (lane & 15);
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int row = 16 * rt + 4 * (lane >> 4) + t;
    float f;
    const int e = ext_row<MAP, DK>(row, f);
    float val = 0.0f;
    if (e >= 0) {
      if (col < DV)
        val = S_in[((size_t)bh * SS::D + e) * DV + col];
      else if (col == DV)
        val = z_in[(size_t)bh * SS::D + e];
    }
    r[t] = val * f;
  }
  return r;
}

template <int MAP, int DK, int DV>
__device__ __forceinline__ void state_out_tile(float* S_out, float* z_out,
                                               int bh, int rt, int ct,
                                               int lane, const f32x4_t& v) {
  using SS = StateShape<MAP, DK, DV>;
  const int col = 16 * ct + (lane & 15);
  if (col > DV) return;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const int row = 16 * rt + 4 * (lane >> 4) + t;
    float f;
    const int e = ext_row<MAP, DK>(row, f);
    if (e < 0) continue;
    const float val = v[t] / f;
    if (col < DV)
      S_out[((size_t)bh * SS::D + e) * DV + col] = val;
    else
      z_out[(size_t)bh * SS::D + e] = val;
  }
}

// ---------------------------------------------------------------------------
// The chunk walker.  OUT = false: sum phi(K)^T V' over the segment and store
// it in workspace slot seg + 1 (segments 0 .. nseg-2).  OUT = true: produce
// y for the segment starting from its prefix state.
// ---------------------------------------------------------------------------
template <int MAP, typename T, int DK, int DV, bool OUT>
__global__ __launch_bounds__(256) void chunk_kernel(PrefillArgs a) {
  using SH = PrefillShape<MAP, T, DK, DV>;
  using E = Elem<T>;
  using frag = typename E::frag;
  constexpr int C = SH::C, NCT = SH::NCT, NRT = SH::NRT, NKB = SH::NKB;
  constexpr int KS = SH::KS, CS = SH::CS, PS = SH::PS, EPU = SH::EPU;

  __shared__ __align__(16) T sK[OUT ? C * KS : EPU];
  __shared__ __align__(16) T sKT[DK * CS];
  __shared__ __align__(16) T sVT[DV * CS];
  __shared__ __align__(16) T sS[OUT ? SH::NCOL * PS : EPU];

  const int tid = threadIdx.x;
  const int w = tid >> 6;
  const int lane = tid & 63;
  const int i16 = lane & 15;
  const int g = lane >> 4;

  const int nseg_here = OUT ? a.nseg : a.nseg - 1;
  const int bh = blockIdx.x / nseg_here;
  const int seg = blockIdx.x % nseg_here;
  const int64_t N = a.N;
  const int64_t tok_begin = (int64_t)seg * a.seg_chunks * C;
  int64_t tok_end = tok_begin + (int64_t)a.seg_chunks * C;
  if (tok_end > N) tok_end = N;
  const int nchunks = (int)((tok_end - tok_begin + C - 1) / C);

  const T* qg = reinterpret_cast<const T*>(a.q) + (size_t)bh * N * DK;
  const T* kg = reinterpret_cast<const T*>(a.k) + (size_t)bh * N * DK;
  const T* vg = reinterpret_cast<const T*>(a.v) + (size_t)bh * N * DV;

  // ------------------------------------------------------------ state ----
  f32x4_t Sacc[SH::MAXRT][NCT];
#pragma unroll
  for (int m = 0; m < SH::MAXRT; ++m) {
    const int rt = w + 4 * m;
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      f32x4_t s = {0.0f, 0.0f, 0.0f, 0.0f};
      if (OUT && rt < NRT) {
        if (a.nseg > 1) {
          const f32x4_t* p = reinterpret_cast<const f32x4_t*>(
              a.ws + ((size_t)bh * a.nseg + seg) * SH::SLOT);
          s = p[(rt * NCT + ct) * 64 + lane];
        } else if (a.S_in != nullptr) {
          s = state_in_tile<MAP, DK, DV>(a.S_in, a.z_in, bh, rt, ct, lane);
        }
      }
      Sacc[m][ct] = s;
    }
  }

  // ones column of V' (and ones row of V'^T): lane column 0 of the last tile
  float onesv[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) onesv[t] = i16 == 0 ? 1.0f : 0.0f;
  const frag ones = E::make(onesv);

  // ---------------------------------------------------------- staging ----
  uint4 kreg[SH::NUK], vreg[SH::NUV], qreg[OUT ? SH::NQU : 1];
  const uint4 z4 = make_uint4(0u, 0u, 0u, 0u);

  auto issue_loads = [&](int c) {
    const int64_t t0 = tok_begin + (int64_t)c * C;
    const bool chunk_ok = c < nchunks;
#pragma unroll
    for (int u = 0; u < SH::NUK; ++u) {
      const int unit = tid + u * SH::NT;
      const int r = unit / SH::KUR;
      const int e0 = (unit % SH::KUR) * EPU;
      kreg[u] = z4;
      if (unit < SH::UK && chunk_ok && t0 + r < tok_end)
        kreg[u] = *reinterpret_cast<const uint4*>(kg + (t0 + r) * DK + e0);
    }
#pragma unroll
    for (int u = 0; u < SH::NUV; ++u) {
      const int unit = tid + u * SH::NT;
      const int r = unit / SH::VUR;
      const int e0 = (unit % SH::VUR) * EPU;
      vreg[u] = z4;
      if (unit < SH::UV && chunk_ok && t0 + r < tok_end)
        vreg[u] = *reinterpret_cast<const uint4*>(vg + (t0 + r) * DV + e0);
    }
    if constexpr (OUT) {
      const int64_t tq = t0 + 16 * w + i16;
      const bool ok = chunk_ok && tq < tok_end;
      if constexpr (MAP == MAP_ELU1) {
        constexpr int UPB = 8 / EPU;  // 16-byte units per 8-feature block
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int h = 0; h < UPB; ++h) {
            const int f0 = 32 * kb + 8 * g + h * EPU;
            qreg[kb * UPB + h] = z4;
            if (ok && f0 < DK)
              qreg[kb * UPB + h] =
                  *reinterpret_cast<const uint4*>(qg + tq * DK + f0);
          }
      } else {
#pragma unroll
        for (int u = 0; u < SH::NQU; ++u) {
          qreg[u] = z4;
          if (ok)
            qreg[u] = *reinterpret_cast<const uint4*>(qg + tq * DK + u * EPU);
        }
      }
    }
  };

  auto write_tiles = [&](int c) {
    const int64_t t0 = tok_begin + (int64_t)c * C;
#pragma unroll
    for (int u = 0; u < SH::NUK; ++u) {
      const int unit = tid + u * SH::NT;
      if (unit < SH::UK) {
        const int r = unit / SH::KUR;
        const int e0 = (unit % SH::KUR) * EPU;
        const bool ok = t0 + r < tok_end;
        float f[EPU];
        unpack16<T>(kreg[u], f);
        if constexpr (MAP == MAP_ELU1) {
#pragma unroll
          for (int e = 0; e < EPU; ++e) f[e] = ok ? phi_elu1(f[e]) : 0.0f;
        }
        if constexpr (OUT) *reinterpret_cast<uint4*>(sK + r * KS + e0) = pack16<T>(f);
#pragma unroll
        for (int e = 0; e < EPU; ++e) sKT[(e0 + e) * CS + r] = E::from_f32(f[e]);
      }
    }
#pragma unroll
    for (int u = 0; u < SH::NUV; ++u) {
      const int unit = tid + u * SH::NT;
      if (unit < SH::UV) {
        const int r = unit / SH::VUR;
        const int e0 = (unit % SH::VUR) * EPU;
        float f[EPU];
        unpack16<T>(vreg[u], f);
#pragma unroll
        for (int e = 0; e < EPU; ++e) sVT[(e0 + e) * CS + r] = E::from_f32(f[e]);
      }
    }
  };

  // Query operands of the current chunk.
  //   ELU1:    qf[kb]  = phi(q) over features 32kb + 8g + (0..7)
  //   TAYLOR2: qv[16]  = q;  qb8[t] = q[8(g&1) + t]
  frag qf[MAP == MAP_ELU1 && OUT ? NKB : 1];
  float qv[MAP == MAP_TAYLOR2 && OUT ? DK : 1];
  float qb8[MAP == MAP_TAYLOR2 && OUT ? 8 : 1];

  auto take_q = [&]() {
    if constexpr (!OUT) return;
    if constexpr (MAP == MAP_ELU1) {
      constexpr int UPB = 8 / EPU;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        float f[8];
#pragma unroll
        for (int h = 0; h < UPB; ++h) {
          float part[EPU];
          unpack16<T>(qreg[kb * UPB + h], part);
#pragma unroll
          for (int e = 0; e < EPU; ++e) f[h * EPU + e] = part[e];
        }
#pragma unroll
        for (int t = 0; t < 8; ++t)
          f[t] = (32 * kb + 8 * g + t < DK) ? phi_elu1(f[t]) : 0.0f;
        qf[kb] = E::make(f);
      }
    } else {
#pragma unroll
      for (int u = 0; u < SH::NQU; ++u) {
        float part[EPU];
        unpack16<T>(qreg[u], part);
#pragma unroll
        for (int e = 0; e < EPU; ++e) qv[u * EPU + e] = part[e];
      }
#pragma unroll
      for (int t = 0; t < 8; ++t) qb8[t] = (g & 1) ? qv[8 + t] : qv[t];
    }
  };

  // phi(K)^T operand for state row tile rt, key block jb2: lane (rho = i16,
  // g) slot t <-> feature 16 rt + rho, token 32 jb2 + 8 g + t.
  auto kt_frag = [&](int rt, int jb2, int nvalid) -> frag {
    const int col = 32 * jb2 + 8 * g;
    if constexpr (MAP == MAP_ELU1) {
      if (16 * rt >= DK) return E::zero();
      return E::load8(sKT + (16 * rt + i16) * CS + col);
    } else {
      float f[8];
      if (rt < 16) {
        float fa[8], fb[8];
        E::load8f(sKT + rt * CS + col, fa);
        E::load8f(sKT + i16 * CS + col, fb);
#pragma unroll
        for (int t = 0; t < 8; ++t) f[t] = fa[t] * fb[t];
      } else if (rt == 16) {
        float fb[8];
        E::load8f(sKT + (i16 == 0 ? 0 : i16 - 1) * CS + col, fb);
#pragma unroll
        for (int t = 0; t < 8; ++t)
          f[t] = i16 == 0 ? (col + t < nvalid ? 1.0f : 0.0f) : fb[t];
      } else {
        float fb[8];
        E::load8f(sKT + 15 * CS + col, fb);
#pragma unroll
        for (int t = 0; t < 8; ++t) f[t] = i16 == 0 ? fb[t] : 0.0f;
      }
      return E::make(f);
    }
  };

  // phi(Q) operand for feature block kb: lane (query i16, g) slot t <->
  // feature 32 kb + 8 g + t.
  auto q_frag = [&](int kb) -> frag {
    if constexpr (MAP == MAP_ELU1) {
      return qf[kb < NKB ? kb : 0];
    } else {
      float f[8];
      if (kb < 8) {
        const float qa = 0.5f * ((g >> 1) ? qv[2 * kb + 1] : qv[2 * kb]);
#pragma unroll
        for (int t = 0; t < 8; ++t) f[t] = qa * qb8[t];
      } else {
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const float g0 = t == 0 ? 1.0f : qv[t > 0 ? t - 1 : 0];
          const float g1 = qv[7 + t];
          const float g2 = t == 0 ? qv[15] : 0.0f;
          f[t] = g == 0 ? g0 : (g == 1 ? g1 : (g == 2 ? g2 : 0.0f));
        }
      }
      return E::make(f);
    }
  };

  // Write this wave's state tiles into the LDS copy (column-major S'^T).
  auto publish_state = [&]() {
#pragma unroll
    for (int m = 0; m < SH::MAXRT; ++m) {
      const int rt = w + 4 * m;
      if (rt >= NRT) continue;
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        T* p = sS + (16 * ct + i16) * PS + 16 * rt + 4 * g;
        const f32x4_t s = Sacc[m][ct];
        if constexpr (sizeof(T) == 2) {
          *reinterpret_cast<uint2*>(p) =
              make_uint2(pack_bf16x2(s[0], s[1]), pack_bf16x2(s[2], s[3]));
        } else {
          *reinterpret_cast<float4*>(p) = make_float4(s[0], s[1], s[2], s[3]);
        }
      }
    }
  };

  // ------------------------------------------------------------ prologue --
  issue_loads(0);
  if constexpr (OUT) publish_state();
  write_tiles(0);
  take_q();
  issue_loads(1);
  lds_barrier();

  T* yg = OUT ? reinterpret_cast<T*>(a.y) + (size_t)bh * N * DV : nullptr;

  for (int c = 0; c < nchunks; ++c) {
    const int64_t t0 = tok_begin + (int64_t)c * C;
    const int nvalid = (int)((tok_end - t0) < C ? (tok_end - t0) : C);

    // V'^T / V' operands for the two 32-token key blocks.
    frag vf[2][NCT - 1];
#pragma unroll
    for (int jb2 = 0; jb2 < 2; ++jb2)
#pragma unroll
      for (int ct = 0; ct < NCT - 1; ++ct)
        vf[jb2][ct] = E::load8(sVT + (16 * ct + i16) * CS + 32 * jb2 + 8 * g);

    if constexpr (OUT) {
      f32x4_t O[NCT];
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) O[ct] = {0.0f, 0.0f, 0.0f, 0.0f};

      // prefix term: O^T += S'^T phi(Q)^T
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const frag bq = q_frag(kb);
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
          const frag av = E::load8(sS + (16 * ct + i16) * PS + 32 * kb + 8 * g);
          E::mma(O[ct], av, bq);
        }
      }

      // within-chunk term: scores^T for keys <= this wave's queries
      frag qraw = E::zero();
      if constexpr (MAP == MAP_TAYLOR2) {
        float f[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) f[t] = g < 2 ? qb8[t] : 0.0f;
        qraw = E::make(f);
      }
      const int il = 16 * w + i16;
#pragma unroll
      for (int jb2 = 0; jb2 < 2; ++jb2) {
        if (32 * jb2 > 16 * w + 15) continue;
        f32x4_t sc[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          sc[h] = {0.0f, 0.0f, 0.0f, 0.0f};
          const int jt = 32 * jb2 + 8 * (i16 >> 2) + 4 * h + (i16 & 3);
#pragma unroll
          for (int kbs = 0; kbs < SH::NKBS; ++kbs) {
            const int f0 = 32 * kbs + 8 * g;
            const frag ak = E::load8(sK + jt * KS + (f0 < DK ? f0 : 0));
            const frag akz = f0 < DK ? ak : E::zero();
            frag bq;
            if constexpr (MAP == MAP_ELU1) bq = q_frag(kbs); else bq = qraw;
            E::mma(sc[h], akz, bq);
          }
        }
        float f[8];
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const int jl = 32 * jb2 + 8 * g + 4 * h + t;
            const float s = sc[h][t];
            float val;
            if constexpr (MAP == MAP_ELU1) val = s; else val = 1.0f + s + 0.5f * s * s;
            f[4 * h + t] = jl <= il ? val : 0.0f;
          }
        const frag bA = E::make(f);
#pragma unroll
        for (int ct = 0; ct < NCT - 1; ++ct) E::mma(O[ct], vf[jb2][ct], bA);
        E::mma(O[NCT - 1], ones, bA);
      }

      // normalise and write y (query il of this chunk)
      const float den = __shfl(O[NCT - 1][0], i16, 64);
      const float rden = 1.0f / den;
      const int64_t tq = t0 + il;
      if (tq < tok_end) {
        T* yrow = yg + tq * DV;
#pragma unroll
        for (int ct = 0; ct < NCT - 1; ++ct) {
          const f32x4_t o = O[ct];
          T* p = yrow + 16 * ct + 4 * g;
          if constexpr (sizeof(T) == 2) {
            *reinterpret_cast<uint2*>(p) =
                make_uint2(pack_bf16x2(o[0] * rden, o[1] * rden),
                           pack_bf16x2(o[2] * rden, o[3] * rden));
          } else {
            *reinterpret_cast<float4*>(p) =
                make_float4(o[0] * rden, o[1] * rden, o[2] * rden, o[3] * rden);
          }
        }
      }
    }

    // state update: S' += phi(K)^T V' for this wave's row tiles
#pragma unroll
    for (int m = 0; m < SH::MAXRT; ++m) {
      const int rt = w + 4 * m;
      if (rt >= NRT) continue;
#pragma unroll
      for (int jb2 = 0; jb2 < 2; ++jb2) {
        const frag ak = kt_frag(rt, jb2, nvalid);
#pragma unroll
        for (int ct = 0; ct < NCT - 1; ++ct) E::mma(Sacc[m][ct], ak, vf[jb2][ct]);
        E::mma(Sacc[m][NCT - 1], ak, ones);
      }
    }

    lds_barrier();  // every wave is done reading the tiles and sS
    if constexpr (OUT) publish_state();
    if (c + 1 < nchunks) {
      write_tiles(c + 1);
      take_q();
      issue_loads(c + 2);
    }
    lds_barrier();
  }

  // ------------------------------------------------------------ epilogue --
  if constexpr (OUT) {
    if (seg == a.nseg - 1 && a.S_out != nullptr) {
#pragma unroll
      for (int m = 0; m < SH::MAXRT; ++m) {
        const int rt = w + 4 * m;
        if (rt >= NRT) continue;
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
          state_out_tile<MAP, DK, DV>(a.S_out, a.z_out, bh, rt, ct, lane,
                                      Sacc[m][ct]);
      }
    }
  } else {
    f32x4_t* p = reinterpret_cast<f32x4_t*>(
        a.ws + ((size_t)bh * a.nseg + seg + 1) * SH::SLOT);
#pragma unroll
    for (int m = 0; m < SH::MAXRT; ++m) {
      const int rt = w + 4 * m;
      if (rt >= NRT) continue;
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) p[(rt * NCT + ct) * 64 + lane] = Sacc[m][ct];
    }
  }
}

// Exclusive prefix over segments, in place: slot s <- init + sum_{p<s} T_p,
// where slot p+1 held segment p's sum T_p and init is the initial state.
template <int MAP, int DK, int DV>
__global__ __launch_bounds__(256) void seg_scan_kernel(PrefillArgs a) {
  using SS = StateShape<MAP, DK, DV>;
  constexpr int Q = SS::SLOT / 4;  // float4 per slot
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int bh = (int)(idx / Q);
  if (bh >= a.BH) return;
  const int e4 = (int)(idx % Q);
  f32x4_t run = {0.0f, 0.0f, 0.0f, 0.0f};
  if (a.S_in != nullptr) {
    const int rt = e4 / (SS::NCT * 64);
    const int ct = (e4 / 64) % SS::NCT;
    run = state_in_tile<MAP, DK, DV>(a.S_in, a.z_in, bh, rt, ct, e4 % 64);
  }
  f32x4_t* p = reinterpret_cast<f32x4_t*>(a.ws + (size_t)bh * a.nseg * SS::SLOT) + e4;
  p[0] = run;
  for (int s = 1; s < a.nseg; ++s) {
    run += p[(size_t)s * Q];
    p[(size_t)s * Q] = run;
  }
}

template <int MAP, typename T, int DK, int DV>
hipError_t launch_prefill(const PrefillArgs& a, hipStream_t st) {
  using SS = StateShape<MAP, DK, DV>;
  if (a.nseg > 1) {
    hipLaunchKernelGGL((chunk_kernel<MAP, T, DK, DV, false>),
                       dim3(a.BH * (a.nseg - 1)), dim3(256), 0, st, a);
    const int64_t threads = (int64_t)a.BH * (SS::SLOT / 4);
    hipLaunchKernelGGL((seg_scan_kernel<MAP, DK, DV>),
                       dim3((unsigned)((threads + 255) / 256)), dim3(256), 0,
                       st, a);
  }
  hipLaunchKernelGGL((chunk_kernel<MAP, T, DK, DV, true>),
                     dim3(a.BH * a.nseg), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace linattn
