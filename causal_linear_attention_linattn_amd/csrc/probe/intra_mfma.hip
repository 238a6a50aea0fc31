// Throughput probe of the within-chunk products (scores of a 16-query tile
// against a 32-token key block, causal mask, then V'^T A^T) on bf16 tiles
// resident in LDS, looped.  It runs the prefill's own device code
// (ChunkTiles::v_frag and ChunkTiles::within_chunk) with no global traffic,
// so its MFMA rate shows what the intra-chunk GEMMs reach when nothing else
// in the prefill competes with them.  Measurement only: not part of the
// prefill library.
#include <hip/hip_runtime.h>

#include "../prefill_impl.hpp"

namespace linattn {
namespace probe {

template <int MAP, int DK, int DV>
__global__ __launch_bounds__(256) void intra_kernel(int iters, float* sink) {
  using CT = ChunkTiles<MAP, bf16_t, DK, DV>;
  using SH = typename CT::SH;
  using E = Elem<bf16_t>;
  using frag = E::frag;
  constexpr int C = SH::C, NCT = SH::NCT;
  constexpr int K_EL = C * RowTile<DK>::STRIDE;
  constexpr int V_EL = C * RowTile<DV>::STRIDE;
  // two copies, alternated per iteration, as in the double-buffered kernel
  __shared__ __align__(16) bf16_t sK[2][K_EL];
  __shared__ __align__(16) bf16_t sV[2][V_EL];

  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, i16 = lane & 15, g = lane >> 4;
  for (int i = tid; i < 2 * K_EL; i += 256)
    (&sK[0][0])[i] = f32_to_bf16(0.015625f * (float)((i * 37) % 17 - 8));
  for (int i = tid; i < 2 * V_EL; i += 256)
    (&sV[0][0])[i] = f32_to_bf16(0.03125f * (float)((i * 11) % 13 - 6));
  __syncthreads();

  const int il = 16 * w + i16;
  bool keep[2][8];
#pragma unroll
  for (int jb2 = 0; jb2 < 2; ++jb2)
#pragma unroll
    for (int e = 0; e < 8; ++e) keep[jb2][e] = 32 * jb2 + 8 * g + e <= il;
  float onesv[8], qv[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    onesv[t] = i16 == 0 ? 1.0f : 0.0f;
    qv[t] = 0.125f * (float)(((lane + t) % 7) + 1);
  }
  const frag ones = E::make(onesv);
  frag bq[SH::NKBS];
#pragma unroll
  for (int k = 0; k < SH::NKBS; ++k) bq[k] = E::make(qv);

  f32x4_t O[NCT];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) O[ct] = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int it = 0; it < iters; ++it) {
    const int b = it & 1;
#pragma unroll
    for (int jb2 = 0; jb2 < 2; ++jb2) {
      frag vf[NCT - 1];
#pragma unroll
      for (int ct = 0; ct < NCT - 1; ++ct) vf[ct] = CT::v_frag(sV[b], jb2, ct, lane);
      CT::within_chunk(sK[b], vf, bq, keep[jb2], ones, O, jb2, lane);
    }
    asm volatile("" ::: "memory");  // tiles are re-read every iteration
  }
  float s = 0.0f;
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) s += O[ct][0] + O[ct][1] + O[ct][2] + O[ct][3];
  sink[blockIdx.x * 256 + tid] = s;
}

// Plain MFMA throughput: every wave issues 16x16x32 bf16 products on
// register operands into eight independent accumulators, with no memory
// traffic in the loop.  It measures the matrix rate this device reaches,
// beside the published peak.
__global__ __launch_bounds__(256) void peak_mfma_kernel(int iters, float* sink) {
  using E = Elem<bf16_t>;
  using frag = E::frag;
  const int lane = threadIdx.x & 63;
  float av[8], bv[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    av[t] = 0.001f * (float)((lane + t) % 5);
    bv[t] = 0.002f * (float)((3 * lane + t) % 7);
  }
  const frag a = E::make(av), b = E::make(bv);
  f32x4_t acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j) E::mma(acc[j], a, b);
  }
  float s = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j) s += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
  sink[blockIdx.x * 256 + threadIdx.x] = s;
}

// Plain streams of 16-byte vectors: workgroup b walks its own contiguous
// range of per_wg vectors, U vectors per thread in flight (U * 4 KB per
// workgroup and trip).  MODE 0 copies src to dst; MODE 1 only reads src (one value
// per thread is stored at the end, to dst); MODE 2 reads src and writes
// each vector back to the same place.  The HBM rates this device reaches
// for the three access mixes.
template <int MODE, int U>
__global__ __launch_bounds__(256) void stream_kernel(const uint4* __restrict__ src,
                                                     uint4* __restrict__ dst, size_t n16,
                                                     size_t per_wg) {
  const size_t begin = (size_t)blockIdx.x * per_wg;
  size_t end = begin + per_wg;
  if (end > n16) end = n16;
  uint32_t acc = 0;
  for (size_t base = begin + threadIdx.x; base < end; base += U * 256) {
    uint4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (base + u * 256 < end) v[u] = src[base + u * 256];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (base + u * 256 >= end) continue;
      if constexpr (MODE == 0) dst[base + u * 256] = v[u];
      if constexpr (MODE == 1) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
      if constexpr (MODE == 2) {
        v[u].x += 1u;
        const_cast<uint4*>(src)[base + u * 256] = v[u];
      }
    }
  }
  if constexpr (MODE == 1) dst[(size_t)blockIdx.x * 256 + threadIdx.x] = make_uint4(acc, 0, 0, 0);
}

}  // namespace probe
}  // namespace linattn

// MFMA operations per wave per iteration: two key blocks, each with
// 2 * NKBS score products and NCT output products.
extern "C" int linattn_probe_intra_mfma_per_iter(int map) {
  using namespace linattn;
  if (map == 0) return 2 * (2 * PrefillShape<MAP_ELU1, bf16_t, 64, 64>::NKBS + StateShape<MAP_ELU1, 64, 64>::NCT);
  if (map == 1) return 2 * (2 * PrefillShape<MAP_TAYLOR2, bf16_t, 16, 64>::NKBS + StateShape<MAP_TAYLOR2, 16, 64>::NCT);
  return -1;
}

// Launch `workgroups` workgroups of 4 waves, each looping `iters` times over
// the within-chunk products of the bench shapes: map 0 = ELU1 d_k = d_v = 64,
// map 1 = TAYLOR2 d' = 16, d_v = 64; bf16.  `sink` receives 256 floats per
// workgroup.  Returns 0, or the HIP error code.
extern "C" int linattn_probe_intra_mfma(int map, int iters, int workgroups, float* sink,
                                        void* stream) {
  using namespace linattn;
  if (iters < 1 || workgroups < 1 || sink == nullptr) return 1;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (map == 0)
    hipLaunchKernelGGL((probe::intra_kernel<MAP_ELU1, 64, 64>), dim3(workgroups), dim3(256), 0, st,
                       iters, sink);
  else if (map == 1)
    hipLaunchKernelGGL((probe::intra_kernel<MAP_TAYLOR2, 16, 64>), dim3(workgroups), dim3(256), 0,
                       st, iters, sink);
  else
    return 1;
  return (int)hipGetLastError();
}

// Launch `workgroups` workgroups of 4 waves of the plain MFMA loop, `iters`
// trips of 8 products each.  `sink` receives 256 floats per workgroup.
// Returns 0, or the HIP error code.
extern "C" int linattn_probe_peak_mfma(int iters, int workgroups, float* sink, void* stream) {
  using namespace linattn;
  if (iters < 1 || workgroups < 1 || sink == nullptr) return 1;
  hipLaunchKernelGGL(probe::peak_mfma_kernel, dim3(workgroups), dim3(256), 0,
                     reinterpret_cast<hipStream_t>(stream), iters, sink);
  return (int)hipGetLastError();
}

namespace {
template <int U>
int launch_stream(int mode, const uint4* s4, uint4* d4, size_t n16, size_t per_wg, int workgroups,
                  hipStream_t st) {
  using namespace linattn::probe;
  if (mode == 0)
    hipLaunchKernelGGL((stream_kernel<0, U>), dim3(workgroups), dim3(256), 0, st, s4, d4, n16, per_wg);
  else if (mode == 1)
    hipLaunchKernelGGL((stream_kernel<1, U>), dim3(workgroups), dim3(256), 0, st, s4, d4, n16, per_wg);
  else if (mode == 2)
    hipLaunchKernelGGL((stream_kernel<2, U>), dim3(workgroups), dim3(256), 0, st, s4, d4, n16, per_wg);
  else
    return 1;
  return (int)hipGetLastError();
}
}  // namespace

// Stream `bytes` (a multiple of 16, both pointers 16-byte aligned, dst at
// least workgroups * 4 KB) in `workgroups` contiguous ranges, `depth` (4, 8
// or 16) vectors per thread in flight: mode 0 copies src to dst, 1 reads
// src, 2 updates src in place.  Returns 0, or the HIP
// error code (1 for bad arguments).
extern "C" int linattn_probe_stream(int mode, int depth, void* src, void* dst, size_t bytes,
                                    int workgroups, void* stream) {
  if (src == nullptr || dst == nullptr || bytes % 16 != 0 || workgroups < 1 ||
      ((uintptr_t)src & 15) != 0 || ((uintptr_t)dst & 15) != 0 ||
      (size_t)workgroups * 256 * 16 > bytes)
    return 1;
  const size_t n16 = bytes / 16;
  const size_t per_wg = (n16 + workgroups - 1) / workgroups;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const uint4* s4 = reinterpret_cast<const uint4*>(src);
  uint4* d4 = reinterpret_cast<uint4*>(dst);
  if (depth == 4) return launch_stream<4>(mode, s4, d4, n16, per_wg, workgroups, st);
  if (depth == 8) return launch_stream<8>(mode, s4, d4, n16, per_wg, workgroups, st);
  if (depth == 16) return launch_stream<16>(mode, s4, d4, n16, per_wg, workgroups, st);
  return 1;
}
