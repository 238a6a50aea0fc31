// Shapes and launch arguments shared by the host API and the prefill
// kernels (no kernel code here).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace linattn {

// MAP_TAYLOR2_SYM has the same kernel as MAP_TAYLOR2 but counts each
// unordered pair of key coordinates once.  The prefill runs it on the
// MAP_TAYLOR2 kernels, which differ only in how a state is imported and
// exported (PrefillArgs::sym).
enum { MAP_ELU1 = 0, MAP_TAYLOR2 = 1, MAP_TAYLOR2_SYM = 2 };

// Exported feature rows of the unordered-pair map: 1 + d + d (d + 1) / 2.
template <int DK>
constexpr int kSymD = 1 + DK + DK * (DK + 1) / 2;

// Output workgroups add the sums of the parts before their segment
// themselves (prefix_mode 1) while there are fewer than kDirectPrefixMax of
// them; beyond that a scan kernel forms the prefixes (prefix_mode 2).
constexpr int kDirectPrefixMax = 8;

struct PrefillArgs {
  const void* q;
  const void* k;
  const void* v;
  void* y;
  const float* S_in;
  const float* z_in;
  float* S_out;
  float* z_out;
  float* ws;
  int64_t N;
  int BH;
  int nseg;        // segments per (batch, head)
  int seg_chunks;  // chunks per segment
  int prefix_mode; // 0: one segment; 1: output workgroups add the preceding
                   // segment sums themselves; 2: a scan kernel runs first;
                   // 3: two segments in one launch, segment 1's workgroup
                   // walks segment 0 (seg_chunks chunks) first without
                   // outputs
  int sum_split;   // the segment-sum pass splits each segment into this many
                   // equal parts (more, shorter workgroups when heads are few)
  int nslot;       // workspace slots per (batch, head): nseg * sum_split
  int sym;         // MAP_TAYLOR2 only: S_in/S_out use the unordered-pair
                   // layout (kSymD rows) instead of the ordered one
  // Gated (scalar-decay) calls only: the decay coefficients a [BH, N], the
  // read (1: decayed-sum ratio, 0: numerator only), and the per-slot log2
  // decay of each segment in the workspace (after the slots).
  const float* gate;
  float* ws_log;
  int normalize;
};

// Per-step decays below 2^kResetLog2 are treated as exact resets by the
// gated prefill (the carried state is dropped rather than scaled by the
// tiny factor): the difference is below 2^-64 relative.
constexpr float kResetLog2 = -64.0f;

template <int MAP, int DK, int DV>
struct StateShape {
  static constexpr int D = MAP == MAP_ELU1      ? DK
                           : MAP == MAP_TAYLOR2 ? 1 + DK + DK * DK
                                                : kSymD<DK>;
  // rows of the state inside the prefill kernels: ELU1 d_k rounded up to a
  // 32-row MFMA K block; the Taylor maps keep each unordered pair of key
  // coordinates once (136 pairs, the constant, 16 linear features, padding:
  // 160 rows; prefill_impl.hpp, taylor_row)
  static constexpr int DP = MAP == MAP_ELU1 ? ((DK + 31) / 32) * 32 : 160;
  static constexpr int NRT = DP / 16;    // 16-row tiles of S'
  static constexpr int NKB = DP / 32;    // 32-wide K blocks over features
  static constexpr int NCT = DV / 16 + 1;  // column tiles of S' incl. z
  static constexpr int NCOL = 16 * NCT;
  static constexpr int SLOT = NRT * NCT * 256;  // floats per workspace slot
  static_assert(MAP == MAP_ELU1 || DK == 16, "TAYLOR2 is built for d_k = 16");
  static_assert(DK % 16 == 0 && DV % 16 == 0, "d_k, d_v multiples of 16");
};

template <int MAP, typename T, int DK, int DV, bool GATED>
hipError_t launch_prefill(const PrefillArgs& a, hipStream_t st);

// gate: NULL for the plain recurrence, else one decay per (batch, head);
// normalize as in PrefillArgs (gated calls only).
template <int MAP, typename T, int DK, int DV>
hipError_t launch_decode(const void* q, const void* k, const void* v,
                         const float* gate, int normalize, float* S, float* z,
                         void* y, int64_t BH, hipStream_t st);

// Sliding-window attention (d_k = d_v = D).  The prefill writes the ring
// cache only if kc is non-null.  The generation step holds one float per
// filled slot in LDS, which bounds its window.
constexpr int kSwaMaxWindow = 4096;

template <typename T, int D>
hipError_t launch_swa_prefill(const void* q, const void* k, const void* v, void* y,
                              void* kc, void* vc, int64_t BH, int64_t N,
                              int64_t window, float scale, hipStream_t st);

template <typename T, int D>
hipError_t launch_swa_decode(const void* q, const void* k, const void* v,
                             const int64_t* pos, void* kc, void* vc, void* y,
                             int64_t B, int64_t H, int64_t window, float scale,
                             hipStream_t st);

template <int MAP, typename T>
hipError_t launch_feature_map(const void* x, int64_t rows, int d_k,
                              float* phi, hipStream_t st);

}  // namespace linattn
