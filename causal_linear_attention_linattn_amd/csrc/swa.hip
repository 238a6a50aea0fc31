// Sliding-window softmax attention for gfx950: prefill, the ring cache the
// prefill leaves for generation, and the generation step.
//
// What is computed ("Simple linear attention language models balance the
// recall-throughput tradeoff", Knowl 4; Knowl 5 for the generation kernel):
// query i attends to keys max(0, i - w + 1) .. i (0-based) with softmax
// weights of scale * q_i . k_j, so y_i = sum_j p_ij v_j.  Generation keeps
// the last w keys and values in a ring of w slots (token t in slot t mod w).
//
// Prefill layout.  One workgroup of 4 waves per (batch*head, 64-query tile);
// wave w owns queries 16 w .. 16 w + 15 of the tile.  The tile's band of
// keys is walked in 64-key blocks (for w = 64: the block before the tile and
// the diagonal block), each staged through LDS in the same layouts as the
// linear-attention chunk kernel (row-major, swizzled, with transposed reads
// for bf16).  Per block, each wave forms scores^T (keys x its queries) on
// MFMA, masks them to the band, and updates an online softmax in the log2
// domain: the running maximum m per query rescales the accumulators when it
// grows, and p = 2^(s - m) feeds O^T += [V | 1]^T P^T on MFMA, whose ones
// column accumulates the denominator.  Nothing but q, k, v and y touches
// HBM; neighbouring tiles re-read a key block from L2, which is why the
// workgroup order keeps neighbouring tiles on one XCD.
#include "prefill_impl.hpp"

namespace linattn {

// Workgroup -> (sequence, tile): the hardware deals workgroups to the 8 XCDs
// round robin; give each XCD a contiguous run of tiles so that tiles that
// share key blocks also share an L2.
__device__ __forceinline__ int xcd_local_order(int id, int nwg) {
  if (nwg % 8 != 0) return id;
  return (id % 8) * (nwg / 8) + id / 8;
}

// Per-tile pieces shared by both prefill kernels.  A "block" is 64 keys
// staged in LDS (K row-major; V row-major for bf16 with transposed operand
// reads, transposed for float).  Each wave owns 16 queries (lane column i16)
// and keeps O^T = [V | 1]^T P^T for them plus the running maximum m (log2
// domain).
template <typename T, int D>
struct SwaTile {
  using SH = PrefillShape<MAP_ELU1, T, D, D>;
  using CT = ChunkTiles<MAP_ELU1, T, D, D>;
  using E = Elem<T>;
  using frag = typename E::frag;
  static constexpr bool BF = sizeof(T) == 2;
  static constexpr int C = SH::C, NCT = SH::NCT, EPU = SH::EPU, KS = SH::KS, CS = SH::CS;
  static constexpr int NKBS = SH::NKBS;
  static constexpr uint32_t ES = sizeof(T);
  static constexpr uint32_t kOOB = 0x7ffffff0u;
  using RT = RowTile<D>;
  static constexpr int K_EL = BF ? C * RT::STRIDE : C * KS;
  static constexpr int V_EL = BF ? C * RT::STRIDE : D * CS;
  static constexpr float kNone = -1e30f;  // "minus infinity" keeping 2^(m - m) = 1
  // block staging: bf16 one 16-byte unit per (row, unit) slot; float a unit
  // of two consecutive rows (V is stored transposed, two tokens per store)
  static constexpr int UR = D / EPU;
  static constexpr int NU = BF ? C * UR : C / 2 * UR;
  static constexpr int NS = (NU + 255) / 256;
  static constexpr int NR = BF ? 1 : 2;
  struct Stage {
    uint4 k[NS][NR], v[NS][NR];
  };

  // query operand: lane (query i16, g) slot t <-> feature 32 kbs + 8 g + t
  __device__ static __forceinline__ void load_q(__amdgpu_buffer_rsrc_t rq, int64_t qi,
                                                int g, frag (&bq)[NKBS]) {
#pragma unroll
    for (int kbs = 0; kbs < NKBS; ++kbs) {
      const int f0 = 32 * kbs + 8 * g;
      const uint32_t off = f0 < D ? (uint32_t)((qi * D + f0) * ES) : kOOB;
      if constexpr (BF) {
        bq[kbs] = __builtin_bit_cast(frag, buffer_load16(rq, off));
      } else {
        const uint4 a = buffer_load16(rq, off);
        const uint4 b = buffer_load16(rq, f0 < D ? off + 16u : kOOB);
        const float f[8] = {__uint_as_float(a.x), __uint_as_float(a.y), __uint_as_float(a.z),
                            __uint_as_float(a.w), __uint_as_float(b.x), __uint_as_float(b.y),
                            __uint_as_float(b.z), __uint_as_float(b.w)};
        bq[kbs] = E::make(f);
      }
    }
  }

  // block kb < 0 (before the sequence) reads zeros
  __device__ static __forceinline__ void issue(__amdgpu_buffer_rsrc_t rk,
                                               __amdgpu_buffer_rsrc_t rv, int64_t kb,
                                               int tid, Stage& st) {
    const bool before = kb < 0;
    const uint32_t rb = (uint32_t)(kb * C);  // first key row of the block
#pragma unroll
    for (int u = 0; u < NS; ++u) {
      const int p = tid + 256 * u;
      const int row = NR * (p / UR), e0 = (p % UR) * EPU;
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        const uint32_t off = !before && (NU % 256 == 0 || p < NU) ? ((rb + row + r) * D + e0) * ES
                                                                  : kOOB;
        st.k[u][r] = buffer_load16(rk, off);
        st.v[u][r] = buffer_load16(rv, off);
      }
    }
  }

  __device__ static __forceinline__ void write(T* sK, T* sV, int tid, const Stage& st) {
#pragma unroll
    for (int u = 0; u < NS; ++u) {
      const int p = tid + 256 * u;
      if (NU % 256 != 0 && p >= NU) continue;
      const int row = NR * (p / UR), unit = p % UR, e0 = unit * EPU;
      if constexpr (BF) {
        *reinterpret_cast<uint4*>(sK + RT::off(row, unit)) = st.k[u][0];
        *reinterpret_cast<uint4*>(sV + RT::off(row, unit)) = st.v[u][0];
      } else {
        *reinterpret_cast<uint4*>(sK + row * KS + e0) = st.k[u][0];
        *reinterpret_cast<uint4*>(sK + (row + 1) * KS + e0) = st.k[u][1];
        float a[4], b[4];
        unpack16<T>(st.v[u][0], a);
        unpack16<T>(st.v[u][1], b);
#pragma unroll
        for (int e = 0; e < 4; ++e) store_pair(sV + (e0 + e) * CS + row, a[e], b[e]);
      }
    }
  }

  // One staged block kb against the wave's queries: scores^T on MFMA, the
  // band mask, the online-softmax update and O^T += [V | 1]^T P^T.
  __device__ static __forceinline__ void block(const T* sK, const T* sV, int64_t kb,
                                               int64_t qi, int64_t window, float c,
                                               const frag (&bq)[NKBS], const frag& ones,
                                               f32x4_t (&O)[NCT], float& m, int lane) {
    const int i16 = lane & 15, g = lane >> 4;
    float s2[2][8];
    float bmax = kNone;
#pragma unroll
    for (int jb2 = 0; jb2 < 2; ++jb2) {
      f32x4_t sc[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        sc[h] = {0.0f, 0.0f, 0.0f, 0.0f};
        const int jt = 32 * jb2 + 8 * (i16 >> 2) + 4 * h + (i16 & 3);
#pragma unroll
        for (int kbs = 0; kbs < NKBS; ++kbs) E::mma(sc[h], CT::k_rows(sK, jt, kbs, lane), bq[kbs]);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int64_t key = kb * C + 32 * jb2 + 8 * g + e;
        const bool valid = key >= 0 && key <= qi && key > qi - window;
        s2[jb2][e] = valid ? sc[e >> 2][e & 3] * c : kNone;
        bmax = fmaxf(bmax, s2[jb2][e]);
      }
    }
    bmax = fmaxf(bmax, __shfl_xor(bmax, 16, 64));
    bmax = fmaxf(bmax, __shfl_xor(bmax, 32, 64));
    const float mn = fmaxf(m, bmax);
    const float alpha = __builtin_amdgcn_exp2f(m - mn);
    m = mn;
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) O[ct] *= alpha;
#pragma unroll
    for (int jb2 = 0; jb2 < 2; ++jb2) {
      float p[8];
#pragma unroll
      for (int e = 0; e < 8; ++e)
        p[e] = s2[jb2][e] > 0.5f * kNone ? __builtin_amdgcn_exp2f(s2[jb2][e] - m) : 0.0f;
      const frag bA = E::make(p);
#pragma unroll
      for (int ct = 0; ct < NCT - 1; ++ct) E::mma(O[ct], CT::v_frag(sV, jb2, ct, lane), bA);
      E::mma(O[NCT - 1], ones, bA);
    }
  }

  // y row qi = O / denominator (rows past N fall outside the store range)
  __device__ static __forceinline__ void store(__amdgpu_buffer_rsrc_t ry, int64_t qi,
                                               const f32x4_t (&O)[NCT], int lane) {
    const int i16 = lane & 15, g = lane >> 4;
    const float den = __shfl(O[NCT - 1][0], i16, 64);
    const float rden = fast_rcp(den);
    const uint32_t yrow = (uint32_t)((qi * D + 4 * g) * ES);
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

  __device__ static __forceinline__ frag ones_frag(int lane) {
    float onesv[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) onesv[t] = (lane & 15) == 0 ? 1.0f : 0.0f;
    return E::make(onesv);
  }
};

// One workgroup per (batch*head, 64-query tile), walking the tile's band of
// key blocks; the next block's loads are issued into registers before the
// current block is computed.  (A variant in which one workgroup walks a run
// of tiles and keeps the band's blocks resident in LDS, loading each block
// once, measured slower on one MI355X -- 38.6 vs 33.4 us at B=8 H=8 N=4096
// d=64 w=64: fewer, serial workgroups hide less latency than many short
// ones, whose repeated block loads hit L2.)
template <typename T, int D>
__global__ __launch_bounds__(256) void swa_prefill_kernel(const T* __restrict__ q,
                                                          const T* __restrict__ k,
                                                          const T* __restrict__ v,
                                                          T* __restrict__ y, int64_t N,
                                                          int ntiles, int64_t window,
                                                          float c) {
  using TT = SwaTile<T, D>;
  constexpr int C = TT::C;
  // bf16: a second copy of the block tiles for the two-block walk below
  constexpr int NBUF = TT::BF ? 2 : 1;
  __shared__ __align__(16) T sK[NBUF][TT::K_EL];
  __shared__ __align__(16) T sV[NBUF][TT::V_EL];

  const int id = xcd_local_order(blockIdx.x, gridDim.x);
  const int bh = id / ntiles;
  const int tile = id % ntiles;
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6) & 3;
  const int lane = tid & 63;
  const int64_t i0 = (int64_t)tile * C;
  const int64_t qi = i0 + 16 * w + (lane & 15);  // this lane's query

  const size_t base = (size_t)bh * N * D;
  const uint32_t bytes = (uint32_t)(N * D * TT::ES);
  const auto rq = make_rsrc(q + base, bytes);
  const auto rk = make_rsrc(k + base, bytes);
  const auto rv = make_rsrc(v + base, bytes);
  const auto ry = make_rsrc(y + base, bytes);

  typename TT::frag bq[TT::NKBS];
  TT::load_q(rq, qi, lane >> 4, bq);
  const typename TT::frag ones = TT::ones_frag(lane);
  f32x4_t O[TT::NCT];
#pragma unroll
  for (int ct = 0; ct < TT::NCT; ++ct) O[ct] = {0.0f, 0.0f, 0.0f, 0.0f};
  float m = TT::kNone;

  typename TT::Stage st;
  if (NBUF == 2 && window <= C) {
    // The band of a window of at most C keys is blocks tile-1 and tile
    // (block -1 reads zeros and is masked): straight-line code, each block
    // in its own LDS copy, two barriers.
    TT::issue(rk, rv, tile - 1, tid, st);
    TT::write(sK[0], sV[0], tid, st);
    TT::issue(rk, rv, tile, tid, st);
    lds_barrier();
    TT::block(sK[0], sV[0], tile - 1, qi, window, c, bq, ones, O, m, lane);
    TT::write(sK[NBUF - 1], sV[NBUF - 1], tid, st);
    lds_barrier();
    TT::block(sK[NBUF - 1], sV[NBUF - 1], tile, qi, window, c, bq, ones, O, m, lane);
  } else {
    const int64_t klo = i0 - window + 1 > 0 ? i0 - window + 1 : 0;
    TT::issue(rk, rv, klo / C, tid, st);
    for (int64_t kb = klo / C; kb <= tile; ++kb) {
      TT::write(sK[0], sV[0], tid, st);
      if (kb < tile) TT::issue(rk, rv, kb + 1, tid, st);
      lds_barrier();
      TT::block(sK[0], sV[0], kb, qi, window, c, bq, ones, O, m, lane);
      lds_barrier();  // every wave is done with the block before it is replaced
    }
  }
  TT::store(ry, qi, O, lane);
}

// The ring cache after a prefill of N tokens: slot s holds the last token t
// < N with t mod w = s if t >= N - w, else zeros.  One thread per 16 bytes.
template <typename T, int D>
__global__ __launch_bounds__(256) void swa_fill_cache_kernel(const T* __restrict__ k,
                                                             const T* __restrict__ v,
                                                             T* __restrict__ kc,
                                                             T* __restrict__ vc, int64_t N,
                                                             int64_t BH, int64_t window) {
  constexpr int EPU = Elem<T>::kPer16B;
  constexpr int UR = D / EPU;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= BH * window * UR) return;
  const int u = (int)(idx % UR);
  const int64_t s = (idx / UR) % window;
  const int64_t bh = idx / (UR * window);
  uint4 kk = make_uint4(0u, 0u, 0u, 0u), vv = kk;
  if (s < N) {
    const int64_t t = s + ((N - 1 - s) / window) * window;  // last t = s (mod w)
    const size_t src = ((size_t)bh * N + t) * D + u * EPU;
    kk = *reinterpret_cast<const uint4*>(k + src);
    vv = *reinterpret_cast<const uint4*>(v + src);
  }
  const size_t dst = ((size_t)bh * window + s) * D + u * EPU;
  *reinterpret_cast<uint4*>(kc + dst) = kk;
  *reinterpret_cast<uint4*>(vc + dst) = vv;
}

template <typename T, int D>
hipError_t launch_swa_prefill(const void* q, const void* k, const void* v, void* y,
                              void* kc, void* vc, int64_t BH, int64_t N,
                              int64_t window, float scale, hipStream_t st) {
  const int ntiles = (int)((N + 63) / 64);
  hipLaunchKernelGGL((swa_prefill_kernel<T, D>), dim3((unsigned)(BH * ntiles)), dim3(256), 0,
                     st, reinterpret_cast<const T*>(q), reinterpret_cast<const T*>(k),
                     reinterpret_cast<const T*>(v), reinterpret_cast<T*>(y), N, ntiles, window,
                     scale * kLog2e);
  if (kc != nullptr) {
    const int64_t threads = BH * window * (D / Elem<T>::kPer16B);
    hipLaunchKernelGGL((swa_fill_cache_kernel<T, D>), dim3((unsigned)((threads + 255) / 256)),
                       dim3(256), 0, st, reinterpret_cast<const T*>(k),
                       reinterpret_cast<const T*>(v), reinterpret_cast<T*>(kc),
                       reinterpret_cast<T*>(vc), N, BH, window);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Generation step.  One workgroup (256 threads) per (batch, head) at 0-based
// position p = pos[b]: the new key and value go to slot p mod w, and the
// query attends to the min(p + 1, w) filled slots (the new token's own slot
// is read from the inputs, not from the cache being written).
//   scores: each key row is split over D / EPU threads (one 16-byte unit
//           each), partial dots reduced with lane shuffles;
//   softmax: wave 0 over the scores in LDS (log2 domain);
//   values: thread t owns 4 value columns and every (256 / (D/4))-th slot,
//           partial sums reduced with shuffles, then across waves in LDS.
// A negative position writes NaN to y and leaves the cache alone.
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(256) void swa_decode_kernel(const T* __restrict__ q,
                                                         const T* __restrict__ k,
                                                         const T* __restrict__ v,
                                                         const int64_t* __restrict__ pos,
                                                         T* __restrict__ kc, T* __restrict__ vc,
                                                         T* __restrict__ y, int H, int window,
                                                         float c) {
  using E = Elem<T>;
  constexpr int EPU = E::kPer16B;
  constexpr int UR = D / EPU;        // 16-byte units per row
  constexpr int RPP = 256 / UR;      // key rows per pass
  constexpr int CPR = D / 4;         // 4-column groups per row
  constexpr int VPP = 256 / CPR;     // value rows per pass
  __shared__ float sq[D];
  __shared__ float sp[kSwaMaxWindow];
  __shared__ float red[4][D];
  __shared__ float ssum;

  const int bh = blockIdx.x;
  const int b = bh / H;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int64_t p = pos[b];
  T* yb = y + (size_t)bh * D;
  if (p < 0) {
    if (tid < D) yb[tid] = E::from_f32(__builtin_nanf(""));
    return;
  }
  const int slot = (int)(p % window);
  const int nvalid = p + 1 < window ? (int)(p + 1) : window;
  const T* kn = k + (size_t)bh * D;
  const T* vn = v + (size_t)bh * D;
  T* kcb = kc + (size_t)bh * window * D;
  T* vcb = vc + (size_t)bh * window * D;

  if (tid < D) sq[tid] = E::to_f32(q[(size_t)bh * D + tid]);
  lds_barrier();

  // scores (log2 domain) of the filled slots
  const int u = tid % UR;
  float qf[EPU];
#pragma unroll
  for (int e = 0; e < EPU; ++e) qf[e] = sq[u * EPU + e];
  for (int j0 = 0; j0 < nvalid; j0 += RPP) {
    const int j = j0 + tid / UR;
    float part = 0.0f;
    if (j < nvalid) {
      const T* row = j == slot ? kn : kcb + (size_t)j * D;
      float kf[EPU];
      unpack16<T>(*reinterpret_cast<const uint4*>(row + u * EPU), kf);
#pragma unroll
      for (int e = 0; e < EPU; ++e) part += qf[e] * kf[e];
    }
#pragma unroll
    for (int off = 1; off < UR; off <<= 1) part += __shfl_xor(part, off, 64);
    if (u == 0 && j < nvalid) sp[j] = part * c;
  }
  lds_barrier();

  // softmax weights (unnormalised) and their sum, by wave 0
  if (wv == 0) {
    float mx = -1e30f;
    for (int j = lane; j < nvalid; j += 64) mx = fmaxf(mx, sp[j]);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
    float sum = 0.0f;
    for (int j = lane; j < nvalid; j += 64) {
      const float e = __builtin_amdgcn_exp2f(sp[j] - mx);
      sp[j] = e;
      sum += e;
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) sum += __shfl_xor(sum, off, 64);
    if (lane == 0) ssum = sum;
  }
  lds_barrier();

  // values
  const int cg = tid % CPR;
  float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int j = tid / CPR; j < nvalid; j += VPP) {
    const T* row = (j == slot ? vn : vcb + (size_t)j * D) + 4 * cg;
    float vf[4];
    if constexpr (sizeof(T) == 2) {
      const uint2 r = *reinterpret_cast<const uint2*>(row);
      vf[0] = __uint_as_float(r.x << 16);
      vf[1] = __uint_as_float(r.x & 0xffff0000u);
      vf[2] = __uint_as_float(r.y << 16);
      vf[3] = __uint_as_float(r.y & 0xffff0000u);
    } else {
      const float4 r = *reinterpret_cast<const float4*>(row);
      vf[0] = r.x; vf[1] = r.y; vf[2] = r.z; vf[3] = r.w;
    }
    const float pj = sp[j];
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] += pj * vf[e];
  }
#pragma unroll
  for (int off = CPR; off < 64; off <<= 1)
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] += __shfl_xor(acc[e], off, 64);
  if (lane < CPR) {
#pragma unroll
    for (int e = 0; e < 4; ++e) red[wv][4 * lane + e] = acc[e];
  }
  // the new token into its slot (no thread reads that slot from the cache)
  if (tid < UR) {
    *reinterpret_cast<uint4*>(kcb + (size_t)slot * D + tid * EPU) =
        *reinterpret_cast<const uint4*>(kn + tid * EPU);
    *reinterpret_cast<uint4*>(vcb + (size_t)slot * D + tid * EPU) =
        *reinterpret_cast<const uint4*>(vn + tid * EPU);
  }
  lds_barrier();
  if (tid < D) {
    const float o = red[0][tid] + red[1][tid] + red[2][tid] + red[3][tid];
    yb[tid] = E::from_f32(o * fast_rcp(ssum));
  }
}

// Generation step for windows of at most WM slots (WM = 64 or 128; the
// pages use 64 and at most 128).  Every cache row is loaded at entry through a
// buffer resource over the head's cache (rows past the window read as
// zero; rows not yet filled are masked by selects, since they may hold
// anything), together with the query and the new token, so the step waits
// on HBM once and has no divergent loads.  Partial dot products are summed
// with DPP row shifts; each wave takes the softmax maximum and sum from the
// scores in LDS with DPP wave reductions, and each thread exponentiates the
// scores of its own value rows.  Value partials are summed through LDS.
constexpr int kSwaSmallWindow = 128;
constexpr int kSwaSmallThreads64 = 256;  // threads per head when the window is <= 64

template <typename T, int D, int NTH, int WM>
__global__ __launch_bounds__(NTH) void swa_decode_small_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const int64_t* __restrict__ pos, T* __restrict__ kc, T* __restrict__ vc,
    T* __restrict__ y, int H, int window, float c) {
  using E = Elem<T>;
  constexpr bool BF = sizeof(T) == 2;
  constexpr uint32_t ES = sizeof(T);
  constexpr int EPU = E::kPer16B;
  constexpr int UR = D / EPU;                       // 16-byte units per key row
  constexpr int NK = WM * UR / NTH;                 // key units per thread
  constexpr int CPR = D / 4;                        // 4-column groups per row
  constexpr int VPP = NTH / CPR;                    // value rows per pass
  constexpr int NV = WM / VPP;                      // value groups per thread
  static_assert((WM == 64 || WM == 128) && WM <= kSwaSmallWindow, "window capacity");
  static_assert(NK >= 1 && NV >= 1 && NTH % UR == 0 && NTH % CPR == 0 && NTH >= D,
                "tiling");
  __shared__ float sp[WM];
  __shared__ __align__(16) float red[VPP][D];

  const int bh = blockIdx.x;
  const int b = bh / H;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int64_t p = pos[b];
  T* yb = y + (size_t)bh * D;
  if (p < 0) {
    if (tid < D) yb[tid] = E::from_f32(__builtin_nanf(""));
    return;
  }
  const int slot = (int)(p % window);
  const int nvalid = p + 1 < window ? (int)(p + 1) : window;
  const T* kn = k + (size_t)bh * D;
  const T* vn = v + (size_t)bh * D;
  T* kcb = kc + (size_t)bh * window * D;
  T* vcb = vc + (size_t)bh * window * D;
  const auto rkc = make_rsrc(kcb, (uint32_t)(window * D * ES));
  const auto rvc = make_rsrc(vcb, (uint32_t)(window * D * ES));
  const int u = tid % UR;    // this thread's unit of every key row
  const int cg = tid % CPR;  // and column group of every value row
  const int ph = tid / CPR;  // and value row phase

  // ------------------------------------------------- every load at once --
  uint4 kr[NK];
#pragma unroll
  for (int i = 0; i < NK; ++i)
    kr[i] = buffer_load16(rkc, (uint32_t)((((tid + NTH * i) / UR) * D + u * EPU) * ES));
  uint2 vr2[BF ? NV : 1];
  uint4 vr4[BF ? 1 : NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const uint32_t off = (uint32_t)(((ph + VPP * i) * D + 4 * cg) * ES);
    if constexpr (BF)
      vr2[i] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rvc, off, 0, 0));
    else
      vr4[i] = buffer_load16(rvc, off);
  }
  const uint4 knu = *reinterpret_cast<const uint4*>(kn + u * EPU);
  float vnf[4];
  if constexpr (BF) {
    const uint2 r = *reinterpret_cast<const uint2*>(vn + 4 * cg);
    vnf[0] = __uint_as_float(r.x << 16);
    vnf[1] = __uint_as_float(r.x & 0xffff0000u);
    vnf[2] = __uint_as_float(r.y << 16);
    vnf[3] = __uint_as_float(r.y & 0xffff0000u);
  } else {
    const float4 r = *reinterpret_cast<const float4*>(vn + 4 * cg);
    vnf[0] = r.x; vnf[1] = r.y; vnf[2] = r.z; vnf[3] = r.w;
  }
  float qf[EPU];
  unpack16<T>(*reinterpret_cast<const uint4*>(q + (size_t)bh * D + u * EPU), qf);

  // ------------------------------------------------------------ scores --
#pragma unroll
  for (int i = 0; i < NK; ++i) {
    const int j = (tid + NTH * i) / UR;
    float kf[EPU];
    unpack16<T>(j == slot ? knu : kr[i], kf);
    float part = 0.0f;
#pragma unroll
    for (int e = 0; e < EPU; ++e) part += qf[e] * kf[e];
    if constexpr (UR <= 16) {
      part = group_sum_to_first<UR>(part);
    } else {
      part = group_sum_to_first<16>(part);
      part += __shfl_down(part, 16, 64);
    }
    if (u == 0) sp[j] = j < nvalid ? part * c : -1e30f;
  }
  lds_barrier();

  // softmax statistics, per wave (every slot index is below WM)
  const float s0 = sp[lane], s1 = WM > 64 ? sp[(lane + 64) & (WM - 1)] : -1e30f;
  const float mx = wave_max(fmaxf(s0, s1));
  const float sum = wave_sum((lane < nvalid ? __builtin_amdgcn_exp2f(s0 - mx) : 0.0f) +
                             (WM > 64 && lane + 64 < nvalid ? __builtin_amdgcn_exp2f(s1 - mx)
                                                            : 0.0f));

  // ------------------------------------------------------------ values --
  float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int j = ph + VPP * i;
    float vf[4];
    if (j == slot) {
#pragma unroll
      for (int e = 0; e < 4; ++e) vf[e] = vnf[e];
    } else if constexpr (BF) {
      vf[0] = __uint_as_float(vr2[i].x << 16);
      vf[1] = __uint_as_float(vr2[i].x & 0xffff0000u);
      vf[2] = __uint_as_float(vr2[i].y << 16);
      vf[3] = __uint_as_float(vr2[i].y & 0xffff0000u);
    } else {
      vf[0] = __uint_as_float(vr4[i].x);
      vf[1] = __uint_as_float(vr4[i].y);
      vf[2] = __uint_as_float(vr4[i].z);
      vf[3] = __uint_as_float(vr4[i].w);
    }
    const float pj = __builtin_amdgcn_exp2f(sp[j] - mx);
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] += j < nvalid ? pj * vf[e] : 0.0f;
  }
  *reinterpret_cast<float4*>(&red[ph][4 * cg]) = make_float4(acc[0], acc[1], acc[2], acc[3]);
  // the new token into its slot (no thread reads that slot from the cache)
  if (tid < UR) {
    *reinterpret_cast<uint4*>(kcb + (size_t)slot * D + tid * EPU) = knu;
    *reinterpret_cast<uint4*>(vcb + (size_t)slot * D + tid * EPU) =
        *reinterpret_cast<const uint4*>(vn + tid * EPU);
  }
  lds_barrier();
  if (tid < D) {
    float o = 0.0f;
#pragma unroll
    for (int r = 0; r < VPP; ++r) o += red[r][tid];
    yb[tid] = E::from_f32(o * fast_rcp(sum));
  }
}

template <typename T, int D>
hipError_t launch_swa_decode(const void* q, const void* k, const void* v,
                             const int64_t* pos, void* kc, void* vc, void* y,
                             int64_t B, int64_t H, int64_t window, float scale,
                             hipStream_t st) {
  if (window <= 64) {
    constexpr int NTH = kSwaSmallThreads64;
    hipLaunchKernelGGL((swa_decode_small_kernel<T, D, NTH, 64>), dim3((unsigned)(B * H)), dim3(NTH),
                       0, st, reinterpret_cast<const T*>(q), reinterpret_cast<const T*>(k),
                       reinterpret_cast<const T*>(v), pos, reinterpret_cast<T*>(kc),
                       reinterpret_cast<T*>(vc), reinterpret_cast<T*>(y), (int)H, (int)window,
                       scale * kLog2e);
    return hipGetLastError();
  }
  if (window <= kSwaSmallWindow) {
    hipLaunchKernelGGL((swa_decode_small_kernel<T, D, 256, 128>), dim3((unsigned)(B * H)), dim3(256),
                       0, st, reinterpret_cast<const T*>(q), reinterpret_cast<const T*>(k),
                       reinterpret_cast<const T*>(v), pos, reinterpret_cast<T*>(kc),
                       reinterpret_cast<T*>(vc), reinterpret_cast<T*>(y), (int)H, (int)window,
                       scale * kLog2e);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((swa_decode_kernel<T, D>), dim3((unsigned)(B * H)), dim3(256), 0, st,
                     reinterpret_cast<const T*>(q), reinterpret_cast<const T*>(k),
                     reinterpret_cast<const T*>(v), pos, reinterpret_cast<T*>(kc),
                     reinterpret_cast<T*>(vc), reinterpret_cast<T*>(y), (int)H, (int)window,
                     scale * kLog2e);
  return hipGetLastError();
}

#define LINATTN_SWA_INST(T, D)                                                          \
  template hipError_t launch_swa_prefill<T, D>(const void*, const void*, const void*,    \
                                               void*, void*, void*, int64_t, int64_t,    \
                                               int64_t, float, hipStream_t);             \
  template hipError_t launch_swa_decode<T, D>(const void*, const void*, const void*,     \
                                              const int64_t*, void*, void*, void*,       \
                                              int64_t, int64_t, int64_t, float,          \
                                              hipStream_t);

LINATTN_SWA_INST(bf16_t, 32)
LINATTN_SWA_INST(bf16_t, 64)
LINATTN_SWA_INST(bf16_t, 128)
LINATTN_SWA_INST(float, 32)
LINATTN_SWA_INST(float, 64)
LINATTN_SWA_INST(float, 128)

}  // namespace linattn
