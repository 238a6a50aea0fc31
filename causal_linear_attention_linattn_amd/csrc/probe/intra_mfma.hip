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
