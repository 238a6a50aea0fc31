// Recurrent generation step and the feature-map export, for gfx950.
//
// Generation ("Simple linear attention language models balance the
// recall-throughput tradeoff", Knowl 3 recurrent equations; Knowl 5 second
// paragraph): per sequence and head,
//   S += phi(k)^T v,  z += phi(k)^T,  y = phi(q) S / phi(q) z
// with the state updated before it is read.  The gated form (the gated
// recurrence in the Hacker News discussion of "Transformers are RNNs", with a
// scalar forget factor) first scales S and z by the step's coefficient a:
//   S = a S + phi(k)^T v,  z = a z + phi(k)^T,
// and may return the numerator phi(q) S unnormalised.  (a = 1 in the plain
// form, where the scaling by exactly 1 changes no bit.)
// Per step the whole state is
// read once and written once, so the step is bound by HBM bandwidth; the
// arithmetic (2 FMA per state element) is negligible.
//
// Layout: one workgroup (256 threads) per (batch, head).  The state block
// S [D, d_v] of a head is contiguous; thread t owns float4 column group
// t % (d_v/4) of rows t / (d_v/4) + k * (1024 / d_v), so each wave reads
// consecutive 16-byte vectors and the whole block is streamed with every
// load issued before the first one is needed.  phi(q), phi(k) are computed
// once into LDS (fp32); partial numerators are reduced across rows with
// lane shuffles, then across the 4 waves through LDS.
#include "device.hpp"

namespace linattn {

// Quadratic feature p (0-based, after the constant and linear ones) of the
// unordered-pair map: pairs a <= b in row-major upper-triangular order,
// weight 1/sqrt 2 on the squares and 1 on the cross products.
template <typename F>
__device__ __forceinline__ float sym_pair_feature(int p, int d, F&& xat) {
  int a = 0;
  while (p >= d - a) {
    p -= d - a;
    ++a;
  }
  const int b = a + p;
  const float xa = xat(a);
  return a == b ? xa * xa * kInvSqrt2 : xa * xat(b);
}

// Feature r of phi(x) in the exported order: ELU1 elementwise; TAYLOR2
// [1, x, vec(x x^T)/sqrt 2] with pair (a, b) at 1 + d + a d + b;
// TAYLOR2_SYM [1, x, unordered pairs].
template <int MAP, int DK>
__device__ __forceinline__ float feature_ext(const float* x, int r) {
  if constexpr (MAP == MAP_ELU1) {
    return phi_elu1(x[r]);
  } else {
    if (r == 0) return 1.0f;
    if (r <= DK) return x[r - 1];
    const int rr = r - 1 - DK;
    if constexpr (MAP == MAP_TAYLOR2_SYM)
      return sym_pair_feature(rr, DK, [&](int i) { return x[i]; });
    return x[rr / DK] * x[rr % DK] * kInvSqrt2;
  }
}

template <int MAP, typename T, int DK, int DV>
__global__ __launch_bounds__(256) void decode_kernel(const T* __restrict__ q,
                                                     const T* __restrict__ k,
                                                     const T* __restrict__ v,
                                                     const float* __restrict__ gate,
                                                     int normalize,
                                                     float* __restrict__ S,
                                                     float* __restrict__ z,
                                                     T* __restrict__ y) {
  using E = Elem<T>;
  constexpr int D = StateShape<MAP, DK, DV>::D;
  constexpr int CPR = DV / 4;         // float4 per state row
  constexpr int RPP = 256 / CPR;      // rows per pass of the workgroup
  constexpr int NP = (D + RPP - 1) / RPP;
  constexpr int NZ = (D + 255) / 256;

  __shared__ float fq[D];
  __shared__ float fk[D];
  __shared__ float xq[DK];
  __shared__ float xk[DK];
  __shared__ __align__(16) float sv[DV];
  __shared__ float4 red[4][CPR];
  __shared__ float dred[4];

  const int bh = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int c4 = tid % CPR;
  const int r0 = tid / CPR;

  float4* S4 = reinterpret_cast<float4*>(S + (size_t)bh * D * DV);
  float* zb = z + (size_t)bh * D;

  // Issue every state load first; they are consumed after phi is ready.
  float4 s[NP];
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int r = r0 + p * RPP;
    s[p] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (r < D) s[p] = S4[r * CPR + c4];
  }
  float zr[NZ];
#pragma unroll
  for (int p = 0; p < NZ; ++p) {
    const int r = tid + 256 * p;
    zr[p] = r < D ? zb[r] : 0.0f;
  }

  const float ga = gate != nullptr ? gate[bh] : 1.0f;
  if (tid < DK) {
    xq[tid] = E::to_f32(q[(size_t)bh * DK + tid]);
    xk[tid] = E::to_f32(k[(size_t)bh * DK + tid]);
  }
  if (tid < DV) sv[tid] = E::to_f32(v[(size_t)bh * DV + tid]);
  lds_barrier();
  for (int r = tid; r < D; r += 256) {
    fq[r] = feature_ext<MAP, DK>(xq, r);
    fk[r] = feature_ext<MAP, DK>(xk, r);
  }
  lds_barrier();

  const float4 vv = reinterpret_cast<const float4*>(sv)[c4];
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int r = r0 + p * RPP;
    if (r < D) {
      const float a = fk[r];
      const float b = fq[r];
      float4 t = s[p];
      t.x = fmaf(a, vv.x, t.x * ga);
      t.y = fmaf(a, vv.y, t.y * ga);
      t.z = fmaf(a, vv.z, t.z * ga);
      t.w = fmaf(a, vv.w, t.w * ga);
      S4[r * CPR + c4] = t;
      acc.x += b * t.x;
      acc.y += b * t.y;
      acc.z += b * t.z;
      acc.w += b * t.w;
    }
  }
  float dp = 0.0f;
#pragma unroll
  for (int p = 0; p < NZ; ++p) {
    const int r = tid + 256 * p;
    if (r < D) {
      const float zn = fmaf(zr[p], ga, fk[r]);
      zb[r] = zn;
      dp += fq[r] * zn;
    }
  }

  // Sum the row partials: lanes with the same column group differ in the
  // lane bits at and above log2(CPR).
#pragma unroll
  for (int off = CPR; off < 64; off <<= 1) {
    acc.x += __shfl_xor(acc.x, off, 64);
    acc.y += __shfl_xor(acc.y, off, 64);
    acc.z += __shfl_xor(acc.z, off, 64);
    acc.w += __shfl_xor(acc.w, off, 64);
  }
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) dp += __shfl_xor(dp, off, 64);
  if (lane < CPR) red[wv][lane] = acc;
  if (lane == 0) dred[wv] = dp;
  lds_barrier();
  if (tid < CPR) {
    float4 n = red[0][tid];
#pragma unroll
    for (int w = 1; w < 4; ++w) {
      n.x += red[w][tid].x;
      n.y += red[w][tid].y;
      n.z += red[w][tid].z;
      n.w += red[w][tid].w;
    }
    const float den = dred[0] + dred[1] + dred[2] + dred[3];
    const float rd = normalize ? fast_rcp(den) : 1.0f;
    T* yp = y + (size_t)bh * DV + 4 * tid;
    if constexpr (sizeof(T) == 2) {
      *reinterpret_cast<uint2*>(yp) =
          make_uint2(pack_bf16x2(n.x * rd, n.y * rd), pack_bf16x2(n.z * rd, n.w * rd));
    } else {
      *reinterpret_cast<float4*>(yp) = make_float4(n.x * rd, n.y * rd, n.z * rd, n.w * rd);
    }
  }
}

template <int MAP, typename T, int DK, int DV>
hipError_t launch_decode(const void* q, const void* k, const void* v,
                         const float* gate, int normalize, float* S, float* z,
                         void* y, int64_t BH, hipStream_t st) {
  hipLaunchKernelGGL((decode_kernel<MAP, T, DK, DV>), dim3((unsigned)BH),
                     dim3(256), 0, st, reinterpret_cast<const T*>(q),
                     reinterpret_cast<const T*>(k), reinterpret_cast<const T*>(v),
                     gate, normalize, S, z, reinterpret_cast<T*>(y));
  return hipGetLastError();
}

// phi(x) per row, exported layout, fp32 out (test and inspection only).
template <int MAP, typename T>
__global__ __launch_bounds__(256) void feature_map_kernel(const T* __restrict__ x,
                                                          int64_t rows, int dk,
                                                          int64_t D,
                                                          float* __restrict__ phi) {
  using E = Elem<T>;
  const int64_t total = rows * D;
  for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * 256) {
    const int64_t row = idx / D;
    const int r = (int)(idx % D);
    const T* xr = x + row * dk;
    float val;
    if constexpr (MAP == MAP_ELU1) {
      val = phi_elu1(E::to_f32(xr[r]));
    } else {
      if (r == 0) {
        val = 1.0f;
      } else if (r <= dk) {
        val = E::to_f32(xr[r - 1]);
      } else if constexpr (MAP == MAP_TAYLOR2_SYM) {
        val = sym_pair_feature(r - 1 - dk, dk,
                               [&](int i) { return E::to_f32(xr[i]); });
      } else {
        const int rr = r - 1 - dk;
        val = E::to_f32(xr[rr / dk]) * E::to_f32(xr[rr % dk]) * kInvSqrt2;
      }
    }
    phi[idx] = val;
  }
}

template <int MAP, typename T>
hipError_t launch_feature_map(const void* x, int64_t rows, int d_k, float* phi,
                              hipStream_t st) {
  const int64_t D = MAP == MAP_ELU1      ? d_k
                    : MAP == MAP_TAYLOR2 ? 1 + d_k + (int64_t)d_k * d_k
                                         : 1 + d_k + (int64_t)d_k * (d_k + 1) / 2;
  const int64_t total = rows * D;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 16384) blocks = 16384;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL((feature_map_kernel<MAP, T>), dim3((unsigned)blocks),
                     dim3(256), 0, st, reinterpret_cast<const T*>(x), rows, d_k,
                     D, phi);
  return hipGetLastError();
}

#define LINATTN_DECODE_INST(MAP, DK, DV)                                          \
  template hipError_t launch_decode<MAP, float, DK, DV>(                          \
      const void*, const void*, const void*, const float*, int, float*, float*,   \
      void*, int64_t, hipStream_t);                                               \
  template hipError_t launch_decode<MAP, bf16_t, DK, DV>(                         \
      const void*, const void*, const void*, const float*, int, float*, float*,   \
      void*, int64_t, hipStream_t);

LINATTN_DECODE_INST(MAP_ELU1, 16, 16)
LINATTN_DECODE_INST(MAP_ELU1, 32, 32)
LINATTN_DECODE_INST(MAP_ELU1, 64, 64)
LINATTN_DECODE_INST(MAP_TAYLOR2, 16, 16)
LINATTN_DECODE_INST(MAP_TAYLOR2, 16, 32)
LINATTN_DECODE_INST(MAP_TAYLOR2, 16, 64)
LINATTN_DECODE_INST(MAP_TAYLOR2_SYM, 16, 16)
LINATTN_DECODE_INST(MAP_TAYLOR2_SYM, 16, 32)
LINATTN_DECODE_INST(MAP_TAYLOR2_SYM, 16, 64)

template hipError_t launch_feature_map<MAP_ELU1, float>(const void*, int64_t, int, float*, hipStream_t);
template hipError_t launch_feature_map<MAP_ELU1, bf16_t>(const void*, int64_t, int, float*, hipStream_t);
template hipError_t launch_feature_map<MAP_TAYLOR2, float>(const void*, int64_t, int, float*, hipStream_t);
template hipError_t launch_feature_map<MAP_TAYLOR2, bf16_t>(const void*, int64_t, int, float*, hipStream_t);
template hipError_t launch_feature_map<MAP_TAYLOR2_SYM, float>(const void*, int64_t, int, float*, hipStream_t);
template hipError_t launch_feature_map<MAP_TAYLOR2_SYM, bf16_t>(const void*, int64_t, int, float*, hipStream_t);

}  // namespace linattn
