// C ABI of the library: argument validation, segment planning and dispatch
// to the kernel instantiations.  Declared in include/linattn.h.
//
// Everything here runs on the host.  Validation finishes before the first
// HIP call, so an invalid call neither launches nor writes anything and
// makes no HIP runtime call at all.
#include <limits.h>
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "linattn.h"
#include "shapes.hpp"

namespace linattn {
typedef uint16_t bf16_t;
}

namespace {

using namespace linattn;

constexpr int kVersion = 100;  // 0.1.0
constexpr int kChunk = 64;     // tokens per chunk inside the prefill kernels
constexpr int kTargetWorkgroups = 256;  // MI355X compute units
constexpr int64_t kMinSegChunks = 8;    // shortest default segment (chunks)
// A segment's q/k/v bytes must fit one buffer descriptor (31-bit range).
constexpr int64_t kMaxSegBytes = ((int64_t)1 << 31) - 4096;
constexpr int64_t kMaxElems = (int64_t)1 << 46;

// Shapes built as prefill kernels.  The unordered-pair Taylor map runs on
// the ordered-pair prefill kernels (PrefillArgs::sym), so it is listed only
// among the decode shapes.
#define LINATTN_FOR_PREFILL_SHAPES(X)                                         \
  X(MAP_ELU1, 16, 16)                                                         \
  X(MAP_ELU1, 32, 32)                                                         \
  X(MAP_ELU1, 64, 64)                                                         \
  X(MAP_TAYLOR2, 16, 16)                                                      \
  X(MAP_TAYLOR2, 16, 32)                                                      \
  X(MAP_TAYLOR2, 16, 64)

#define LINATTN_FOR_SHAPES(X)                                                 \
  LINATTN_FOR_PREFILL_SHAPES(X)                                               \
  X(MAP_TAYLOR2_SYM, 16, 16)                                                  \
  X(MAP_TAYLOR2_SYM, 16, 32)                                                  \
  X(MAP_TAYLOR2_SYM, 16, 64)

static_assert((int)LINATTN_MAP_ELU1 == MAP_ELU1 &&
                  (int)LINATTN_MAP_TAYLOR2 == MAP_TAYLOR2 &&
                  (int)LINATTN_MAP_TAYLOR2_SYM == MAP_TAYLOR2_SYM,
              "map codes of the ABI and the kernels agree");

bool valid_map(int map) {
  return map == LINATTN_MAP_ELU1 || map == LINATTN_MAP_TAYLOR2 ||
         map == LINATTN_MAP_TAYLOR2_SYM;
}

// The map whose prefill kernels run `map`.
int prefill_map(int map) {
  return map == LINATTN_MAP_TAYLOR2_SYM ? MAP_TAYLOR2 : map;
}

bool valid_dtype(int dtype) {
  return dtype == LINATTN_DTYPE_F32 || dtype == LINATTN_DTYPE_BF16;
}

bool is_supported(int map, int dtype, int64_t dk, int64_t dv) {
  if (!valid_map(map) || !valid_dtype(dtype)) return false;
#define X(M, DK, DV) \
  if (map == M && dk == DK && dv == DV) return true;
  LINATTN_FOR_SHAPES(X)
#undef X
  return false;
}

int64_t feature_dim(int map, int64_t dk) {
  if (dk <= 0 || dk > (1 << 20)) return -1;
  if (map == LINATTN_MAP_ELU1) return dk;
  if (map == LINATTN_MAP_TAYLOR2) return 1 + dk + dk * dk;
  if (map == LINATTN_MAP_TAYLOR2_SYM) return 1 + dk + dk * (dk + 1) / 2;
  return -1;
}

int64_t slot_floats(int map, int64_t dk, int64_t dv) {
  map = prefill_map(map);
#define X(M, DK, DV) \
  if (map == M && dk == DK && dv == DV) return StateShape<M, DK, DV>::SLOT;
  LINATTN_FOR_PREFILL_SHAPES(X)
#undef X
  return -1;
}

size_t elem_size(int dtype) { return dtype == LINATTN_DTYPE_F32 ? 4 : 2; }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool aligned4(const void* p) { return ((uintptr_t)p & 3u) == 0; }

struct Range {
  const char* p;
  size_t n;
};

bool overlap(Range a, Range b) {
  if (a.p == nullptr || b.p == nullptr || a.n == 0 || b.n == 0) return false;
  return a.p < b.p + b.n && b.p < a.p + a.n;
}

Range rng(const void* p, int64_t elems, size_t esz) {
  return Range{reinterpret_cast<const char*>(p), (size_t)elems * esz};
}

// Segments along N: each workgroup walks seg_chunks consecutive chunks.
bool plan_segments(int64_t BH, int64_t N, int64_t seg_len, int64_t row_bytes,
                   int* nseg_out, int* seg_chunks_out) {
  const int64_t nchunks = (N + kChunk - 1) / kChunk;
  const int64_t max_seg_chunks = kMaxSegBytes / (kChunk * row_bytes);
  int64_t seg_chunks;
  if (seg_len == 0) {
    int64_t nseg = (kTargetWorkgroups + BH - 1) / BH;
    int64_t max_nseg = nchunks / kMinSegChunks;
    if (max_nseg < 1) max_nseg = 1;
    if (nseg > max_nseg) nseg = max_nseg;
    if (nseg < 1) nseg = 1;
    seg_chunks = (nchunks + nseg - 1) / nseg;
  } else {
    if (seg_len < 0 || seg_len % kChunk != 0) return false;
    seg_chunks = seg_len / kChunk;
  }
  if (seg_chunks > nchunks) seg_chunks = nchunks;
  if (seg_chunks > max_seg_chunks) {
    if (seg_len != 0) return false;
    seg_chunks = max_seg_chunks;
  }
  const int64_t nseg = (nchunks + seg_chunks - 1) / seg_chunks;
  if (BH * nseg > INT_MAX || seg_chunks > INT_MAX) return false;
  *nseg_out = (int)nseg;
  *seg_chunks_out = (int)seg_chunks;
  return true;
}

// The segment-sum pass of the Taylor maps (10 state row tiles per chunk)
// splits each segment into `sum_split` parts when the heads are too few for
// one workgroup per segment to occupy the GPU twice over, as long as a part
// keeps kMinSumChunks chunks: measured on one MI355X at B=8 H=16 N=2048,
// 117 -> 111 us per call.  For ELU1 the extra prefix slots the output
// workgroups then add cost more than the shorter pass saves (43.5 -> 45.6 us
// at B=8 H=8 N=4096 d=64), so it keeps one part.
constexpr int64_t kMinSumChunks = 4;

int sum_split(int map, int64_t BH, int nseg, int seg_chunks) {
  if (map == LINATTN_MAP_ELU1 || nseg <= 1) return 1;
  if (BH * (nseg - 1) >= 2 * kTargetWorkgroups) return 1;
  if (seg_chunks % 2 != 0 || seg_chunks / 2 < kMinSumChunks) return 1;
  return 2;
}

// Chunks of segment 0 in a prefix_mode 3 plan (two segments), a multiple
// of two (the output walk takes two chunks per trip), at least 2 and leaving
// segment 1 at least one chunk.  The share evens out the two workgroups of a
// head: measured on one MI355X at B=8 H=16 N=2048 d_v=64 (32 chunks), bf16
// 20 / 22 / 24 chunks 37.2 / 36.6 / 38.5 us (gated 46.7 / 45.1 / 47.6 us),
// float 18 / 20 / 22 chunks 222 / 210 / 227 us.
int64_t self_prefix_seg0_chunks(int64_t nchunks, int dtype) {
  const int64_t num = dtype == LINATTN_DTYPE_F32 ? 10 : 11;
  int64_t c0 = (nchunks * num / 16) & ~(int64_t)1;
  if (c0 >= nchunks) c0 = (nchunks - 1) & ~(int64_t)1;
  return c0 < 2 ? 2 : c0;
}

// Workspace: BH * nseg * sum_split slots of partial states, then one float
// per slot (the log2 decay of a part in gated calls), padded to 16 bytes.
size_t slots_bytes(int map, int64_t BH, int64_t dk, int64_t dv, int nslot) {
  return (size_t)BH * (size_t)nslot * (size_t)slot_floats(map, dk, dv) * 4u;
}

// ELU1, default plan of two segments per head (128 to 255 heads): one
// launch in which segment 1's workgroup walks segment 0 first without
// outputs (prefix_mode 3, as for the Taylor maps).  Segment 0 takes
// 1 / (2 - r) of the chunks, rounded to whole two-chunk trips, where r
// stands for the cost of a chunk walked without outputs against one with
// them: measured best at 8/16 for the plain map (B=16 H=8 N=2048..4096,
// 6 to 12/16 tried; such a chunk takes ~0.8 us against ~1.3 us) and for
// the gated map (6 to 12/16 tried at B=16 H=8 N=2048..4096).
constexpr int kPreCost16 = 8;

int64_t elu1_seg0_chunks(int64_t nchunks) {
  const double r = kPreCost16 / 16.0;
  int64_t c0 = 2 * (int64_t)(nchunks / (2.0 - r) / 2.0 + 0.5);
  if (c0 >= nchunks) c0 = (nchunks - 1) & ~(int64_t)1;
  return c0 < 2 ? 2 : c0;
}

size_t workspace_bytes(int map, int64_t BH, int64_t dk, int64_t dv, int nseg,
                       int seg_chunks) {
  if (nseg <= 1) return 0;
  const int nslot = nseg * sum_split(map, BH, nseg, seg_chunks);
  const size_t logs = ((size_t)BH * (size_t)nslot * 4u + 15u) & ~(size_t)15u;
  return slots_bytes(map, BH, dk, dv, nslot) + logs;
}

template <bool GATED>
hipError_t dispatch_prefill(int map, int dtype, int64_t dk, int64_t dv,
                            const PrefillArgs& a, hipStream_t st) {
  map = prefill_map(map);
#define X(M, DK, DV)                                                            \
  if (map == M && dk == DK && dv == DV)                                         \
    return dtype == LINATTN_DTYPE_F32 ? launch_prefill<M, float, DK, DV, GATED>(a, st) \
                                      : launch_prefill<M, bf16_t, DK, DV, GATED>(a, st);
  LINATTN_FOR_PREFILL_SHAPES(X)
#undef X
  return hipErrorInvalidValue;
}

hipError_t dispatch_decode(int map, int dtype, int64_t dk, int64_t dv,
                           const void* q, const void* k, const void* v,
                           const float* gate, int normalize, float* S, float* z,
                           void* y, int64_t BH, hipStream_t st) {
#define X(M, DK, DV)                                                            \
  if (map == M && dk == DK && dv == DV)                                         \
    return dtype == LINATTN_DTYPE_F32                                           \
               ? launch_decode<M, float, DK, DV>(q, k, v, gate, normalize, S, z, y, BH, st) \
               : launch_decode<M, bf16_t, DK, DV>(q, k, v, gate, normalize, S, z, y, BH, st);
  LINATTN_FOR_SHAPES(X)
#undef X
  return hipErrorInvalidValue;
}

// The fixed device array behind linattn_prefill_noalloc: the prefill's
// segment part sums live here instead of in a caller-provided workspace.
// Each device the library runs on holds its own copy, zero at module load
// and kept until the process ends.  Host code never names the array itself
// (on the host its name is a stand-in, not a device address); it uses the
// device address that hipGetSymbolAddress returns, looked up once per
// device with that device current.
constexpr size_t kScratchBytes = LINATTN_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// Device address of `scratch` on the current device.
hipError_t scratch_on_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

linattn_status_t prefill_common(int map, int dtype, int64_t B, int64_t H,
                                int64_t N, int64_t d_k, int64_t d_v,
                                const void* q, const void* k, const void* v,
                                bool gated, const float* gate, int normalize,
                                void* y, const float* S_in, const float* z_in,
                                float* S_out, float* z_out, int64_t seg_len,
                                void* workspace, size_t workspace_bytes_given,
                                void* stream, bool fixed_scratch = false) {
  if (!valid_map(map) || !valid_dtype(dtype) || B <= 0 || H <= 0 || N <= 0 ||
      d_k <= 0 || d_v <= 0)
    return LINATTN_ERR_INVALID_ARGUMENT;
  if (!is_supported(map, dtype, d_k, d_v)) return LINATTN_ERR_UNSUPPORTED;
  if (B > kMaxElems / H || N > kMaxElems / (B * H * (d_k > d_v ? d_k : d_v)))
    return LINATTN_ERR_INVALID_ARGUMENT;
  const int64_t BH = B * H;
  if (BH > INT_MAX) return LINATTN_ERR_INVALID_ARGUMENT;
  if (q == nullptr || k == nullptr || v == nullptr || y == nullptr)
    return LINATTN_ERR_INVALID_ARGUMENT;
  if (gated && (gate == nullptr || !aligned4(gate) || (normalize != 0 && normalize != 1)))
    return LINATTN_ERR_INVALID_ARGUMENT;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(y))
    return LINATTN_ERR_INVALID_ARGUMENT;
  if ((S_in == nullptr) != (z_in == nullptr) || (S_out == nullptr) != (z_out == nullptr))
    return LINATTN_ERR_INVALID_ARGUMENT;
  if ((S_in && (!aligned4(S_in) || !aligned4(z_in))) ||
      (S_out && (!aligned4(S_out) || !aligned4(z_out))))
    return LINATTN_ERR_INVALID_ARGUMENT;
  int nseg, seg_chunks;
  const int64_t row_bytes = (d_k > d_v ? d_k : d_v) * (int64_t)elem_size(dtype);
  if (!plan_segments(BH, N, seg_len, row_bytes, &nseg, &seg_chunks))
    return LINATTN_ERR_INVALID_ARGUMENT;

  const size_t es = elem_size(dtype);
  const int64_t D = feature_dim(map, d_k);
  const Range rq = rng(q, BH * N * d_k, es), rk = rng(k, BH * N * d_k, es);
  const Range rv = rng(v, BH * N * d_v, es), ry = rng(y, BH * N * d_v, es);
  const Range rSi = rng(S_in, BH * D * d_v, 4), rzi = rng(z_in, BH * D, 4);
  const Range rSo = rng(S_out, BH * D * d_v, 4), rzo = rng(z_out, BH * D, 4);
  // outputs must not overlap inputs or each other (S_out == S_in and
  // z_out == z_in exactly are allowed: in-place continuation)
  const Range outs[3] = {ry, rSo, rzo};
  const Range ins[3] = {rq, rk, rv};
  for (int i = 0; i < 3; ++i) {
    for (int j = 0; j < 3; ++j)
      if (overlap(outs[i], ins[j])) return LINATTN_ERR_INVALID_ARGUMENT;
    for (int j = i + 1; j < 3; ++j)
      if (overlap(outs[i], outs[j])) return LINATTN_ERR_INVALID_ARGUMENT;
  }
  if (overlap(ry, rSi) || overlap(ry, rzi)) return LINATTN_ERR_INVALID_ARGUMENT;
  if (overlap(rSo, rSi) && S_out != S_in) return LINATTN_ERR_INVALID_ARGUMENT;
  if (overlap(rzo, rzi) && z_out != z_in) return LINATTN_ERR_INVALID_ARGUMENT;
  if (overlap(rSo, rzi) || overlap(rzo, rSi)) return LINATTN_ERR_INVALID_ARGUMENT;
  const Range rg = rng(gated ? gate : nullptr, BH * N, 4);
  for (int i = 0; i < 3; ++i)
    if (overlap(outs[i], rg)) return LINATTN_ERR_INVALID_ARGUMENT;

  const size_t need = workspace_bytes(map, BH, d_k, d_v, nseg, seg_chunks);
  if (fixed_scratch) {
    if (need > kScratchBytes) return LINATTN_ERR_SCRATCH;
    workspace = nullptr;
    if (need > 0) {
      // the only HIP calls before the launch: the device and, on its first
      // use there, the array's address (no allocation)
      if (scratch_on_current_device(&workspace) != hipSuccess) return LINATTN_ERR_HIP;
    }
  } else if (need > 0) {
    if (workspace == nullptr || !aligned16(workspace) || workspace_bytes_given < need)
      return LINATTN_ERR_WORKSPACE;
    const Range rw{reinterpret_cast<const char*>(workspace), need};
    const Range all[9] = {rq, rk, rv, ry, rSi, rzi, rSo, rzo, rg};
    for (int i = 0; i < 9; ++i)
      if (overlap(rw, all[i])) return LINATTN_ERR_INVALID_ARGUMENT;
  }

  PrefillArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.y = y;
  a.S_in = S_in;
  a.z_in = z_in;
  a.S_out = S_out;
  a.z_out = z_out;
  a.ws = reinterpret_cast<float*>(workspace);
  a.N = N;
  a.BH = (int)BH;
  a.nseg = nseg;
  a.seg_chunks = seg_chunks;
  a.sum_split = sum_split(map, BH, nseg, seg_chunks);
  a.nslot = nseg * a.sum_split;
  // With several segments the output workgroups of one head run on
  // different XCDs in no fixed order, and the last one writes S_out / z_out
  // when it ends.  If those alias S_in / z_in, no output workgroup may read
  // the initial state itself: the scan kernel (prefix_mode 2) folds it into
  // the workspace prefixes in an earlier launch.  With one segment the
  // workgroup that reads the state is the one that writes it, after its
  // first chunk has consumed what it read.
  const bool in_place = (S_out != nullptr && S_out == S_in) ||
                        (z_out != nullptr && z_out == z_in);
  a.prefix_mode = nseg == 1 ? 0
                  : (!in_place && (nseg - 1) * a.sum_split <= kDirectPrefixMax - 1) ? 1
                                                                                   : 2;
  a.sym = map == LINATTN_MAP_TAYLOR2_SYM ? 1 : 0;
  a.gate = gated ? gate : nullptr;
  a.ws_log = gated && nseg > 1
                 ? a.ws + slots_bytes(map, BH, d_k, d_v, a.nslot) / sizeof(float)
                 : nullptr;
  a.normalize = gated ? normalize : 1;
  // Taylor maps at two segments per head (the default plan for 128 to 255
  // heads): no segment-sum pass.  The workgroup of segment 1 walks segment
  // 0 itself first, advancing the state without outputs (prefix_mode 3), so
  // the call is one launch and reads no workspace.  Segment 0 takes the
  // larger share of the chunks, since such a chunk costs less than one with
  // outputs.
  const int64_t nchunks = (N + kChunk - 1) / kChunk;
  if (prefill_map(map) == MAP_TAYLOR2 && seg_len == 0 && nseg == 2 && !in_place &&
      nchunks <= kMaxSegBytes / (kChunk * row_bytes)) {
    a.prefix_mode = 3;
    a.seg_chunks = (int)self_prefix_seg0_chunks(nchunks, dtype);
    a.sum_split = 1;
    a.ws_log = nullptr;
  }
  // ELU1 at two segments per head, not in place (both workgroups of a head
  // read the initial state, and segment 1's writes the final one): one
  // launch as well.  The gated kernel holds one workgroup per compute unit,
  // and past 128 heads its late workgroups, which walk the whole sequence,
  // start only when early ones end: measured on one MI355X at B=20 H=8
  // N=3000 d=64 bf16, 127.3 us with the segment-sum plan against 134.8 us;
  // at B=16 H=8 N=4096, 100.4 against 90.8 us.
  if (prefill_map(map) == MAP_ELU1 && seg_len == 0 && nseg == 2 && !in_place &&
      (!gated || BH * 2 <= kTargetWorkgroups) &&
      nchunks <= kMaxSegBytes / (kChunk * row_bytes)) {
    a.prefix_mode = 3;
    a.seg_chunks = (int)elu1_seg0_chunks(nchunks);
    a.sum_split = 1;
    a.ws_log = nullptr;
  }
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const hipError_t e = gated ? dispatch_prefill<true>(map, dtype, d_k, d_v, a, st)
                             : dispatch_prefill<false>(map, dtype, d_k, d_v, a, st);
  return e == hipSuccess ? LINATTN_OK : LINATTN_ERR_HIP;
}

linattn_status_t decode_common(int map, int dtype, int64_t B, int64_t H,
                               int64_t d_k, int64_t d_v, const void* q,
                               const void* k, const void* v, bool gated,
                               const float* gate, int normalize, float* S,
                               float* z, void* y, void* stream) {
  if (!valid_map(map) || !valid_dtype(dtype) || B <= 0 || H <= 0 || d_k <= 0 ||
      d_v <= 0)
    return LINATTN_ERR_INVALID_ARGUMENT;
  if (!is_supported(map, dtype, d_k, d_v)) return LINATTN_ERR_UNSUPPORTED;
  if (B > kMaxElems / H) return LINATTN_ERR_INVALID_ARGUMENT;
  const int64_t BH = B * H;
  if (BH > INT_MAX) return LINATTN_ERR_INVALID_ARGUMENT;
  if (q == nullptr || k == nullptr || v == nullptr || S == nullptr || z == nullptr ||
      y == nullptr)
    return LINATTN_ERR_INVALID_ARGUMENT;
  if (gated && (gate == nullptr || !aligned4(gate) || (normalize != 0 && normalize != 1)))
    return LINATTN_ERR_INVALID_ARGUMENT;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(S) ||
      !aligned16(z) || !aligned16(y))
    return LINATTN_ERR_INVALID_ARGUMENT;
  const size_t es = elem_size(dtype);
  const int64_t D = feature_dim(map, d_k);
  const Range rq = rng(q, BH * d_k, es), rk = rng(k, BH * d_k, es);
  const Range rv = rng(v, BH * d_v, es), ry = rng(y, BH * d_v, es);
  const Range rS = rng(S, BH * D * d_v, 4), rz = rng(z, BH * D, 4);
  const Range ins[3] = {rq, rk, rv};
  const Range outs[3] = {ry, rS, rz};
  for (int i = 0; i < 3; ++i) {
    for (int j = 0; j < 3; ++j)
      if (overlap(outs[i], ins[j])) return LINATTN_ERR_INVALID_ARGUMENT;
    for (int j = i + 1; j < 3; ++j)
      if (overlap(outs[i], outs[j])) return LINATTN_ERR_INVALID_ARGUMENT;
    if (gated && overlap(outs[i], rng(gate, BH, 4))) return LINATTN_ERR_INVALID_ARGUMENT;
  }
  const hipError_t e = dispatch_decode(map, dtype, d_k, d_v, q, k, v,
                                       gated ? gate : nullptr, gated ? normalize : 1,
                                       S, z, y, BH, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? LINATTN_OK : LINATTN_ERR_HIP;
}

bool swa_dim_ok(int64_t d) { return d == 32 || d == 64 || d == 128; }

// The usual softmax scale, 1/sqrt(d), taken when the caller passes NaN
// (d <= 0 gives NaN, which validation rejects with d).
float default_swa_scale(int64_t d) { return d > 0 ? (float)(1.0 / sqrt((double)d)) : NAN; }

hipError_t dispatch_swa_prefill(int dtype, int64_t d, const void* q, const void* k,
                                const void* v, void* y, void* kc, void* vc, int64_t BH,
                                int64_t N, int64_t window, float scale, hipStream_t st) {
#define X(D)                                                                          \
  if (d == D)                                                                         \
    return dtype == LINATTN_DTYPE_F32                                                 \
               ? launch_swa_prefill<float, D>(q, k, v, y, kc, vc, BH, N, window, scale, st) \
               : launch_swa_prefill<bf16_t, D>(q, k, v, y, kc, vc, BH, N, window, scale, st);
  X(32) X(64) X(128)
#undef X
  return hipErrorInvalidValue;
}

hipError_t dispatch_swa_decode(int dtype, int64_t d, const void* q, const void* k,
                               const void* v, const int64_t* pos, void* kc, void* vc,
                               void* y, int64_t B, int64_t H, int64_t window, float scale,
                               hipStream_t st) {
#define X(D)                                                                              \
  if (d == D)                                                                             \
    return dtype == LINATTN_DTYPE_F32                                                     \
               ? launch_swa_decode<float, D>(q, k, v, pos, kc, vc, y, B, H, window, scale, st) \
               : launch_swa_decode<bf16_t, D>(q, k, v, pos, kc, vc, y, B, H, window, scale, st);
  X(32) X(64) X(128)
#undef X
  return hipErrorInvalidValue;
}

bool finite(float x) { return x == x && x - x == 0.0f; }

}  // namespace

extern "C" {

const char* linattn_status_string(int status) {
  switch (status) {
    case LINATTN_OK:
      return "ok";
    case LINATTN_ERR_INVALID_ARGUMENT:
      return "invalid argument (null pointer, non-positive size, misaligned or overlapping buffer, bad segment length)";
    case LINATTN_ERR_UNSUPPORTED:
      return "unsupported combination of feature map, dtype, d_k and d_v";
    case LINATTN_ERR_WORKSPACE:
      return "workspace missing or smaller than linattn_prefill_workspace_bytes()";
    case LINATTN_ERR_HIP:
      return "the HIP runtime reported an error while launching";
    case LINATTN_ERR_SCRATCH:
      return "linattn_prefill_noalloc: the call needs more scratch than the fixed device array holds (LINATTN_NOALLOC_SCRATCH_BYTES); use linattn_prefill with a workspace";
    default:
      return "unknown status";
  }
}

int linattn_version(void) { return kVersion; }

int64_t linattn_feature_dim(int map, int64_t d_k) { return feature_dim(map, d_k); }

int linattn_supported(int map, int dtype, int64_t d_k, int64_t d_v) {
  return is_supported(map, dtype, d_k, d_v) ? 1 : 0;
}

linattn_status_t linattn_feature_map(int map, int dtype, const void* x,
                                     int64_t rows, int64_t d_k, float* phi,
                                     void* stream) {
  if (!valid_map(map) || !valid_dtype(dtype) || rows < 0 || d_k <= 0)
    return LINATTN_ERR_INVALID_ARGUMENT;
  const bool ok_dk = map == LINATTN_MAP_ELU1 ? (d_k == 16 || d_k == 32 || d_k == 64)
                                             : d_k == 16;
  if (!ok_dk) return LINATTN_ERR_UNSUPPORTED;
  if (rows == 0) return LINATTN_OK;
  const int64_t D = feature_dim(map, d_k);
  if (rows > kMaxElems / D) return LINATTN_ERR_INVALID_ARGUMENT;
  if (x == nullptr || phi == nullptr || !aligned16(x) || !aligned16(phi))
    return LINATTN_ERR_INVALID_ARGUMENT;
  if (overlap(rng(x, rows * d_k, elem_size(dtype)), rng(phi, rows * D, 4)))
    return LINATTN_ERR_INVALID_ARGUMENT;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  hipError_t e;
  if (map == LINATTN_MAP_ELU1)
    e = dtype == LINATTN_DTYPE_F32
            ? launch_feature_map<MAP_ELU1, float>(x, rows, (int)d_k, phi, st)
            : launch_feature_map<MAP_ELU1, bf16_t>(x, rows, (int)d_k, phi, st);
  else if (map == LINATTN_MAP_TAYLOR2)
    e = dtype == LINATTN_DTYPE_F32
            ? launch_feature_map<MAP_TAYLOR2, float>(x, rows, (int)d_k, phi, st)
            : launch_feature_map<MAP_TAYLOR2, bf16_t>(x, rows, (int)d_k, phi, st);
  else
    e = dtype == LINATTN_DTYPE_F32
            ? launch_feature_map<MAP_TAYLOR2_SYM, float>(x, rows, (int)d_k, phi, st)
            : launch_feature_map<MAP_TAYLOR2_SYM, bf16_t>(x, rows, (int)d_k, phi, st);
  return e == hipSuccess ? LINATTN_OK : LINATTN_ERR_HIP;
}

size_t linattn_prefill_workspace_bytes(int map, int dtype, int64_t B, int64_t H,
                                       int64_t N, int64_t d_k, int64_t d_v,
                                       int64_t seg_len) {
  if (!valid_map(map) || !valid_dtype(dtype) || B <= 0 || H <= 0 || N <= 0 ||
      d_k <= 0 || d_v <= 0)
    return (size_t)-1;
  if (!is_supported(map, dtype, d_k, d_v)) return (size_t)-1;
  if (B > kMaxElems / H || N > kMaxElems / (B * H)) return (size_t)-1;
  int nseg, seg_chunks;
  const int64_t row_bytes = (d_k > d_v ? d_k : d_v) * (int64_t)elem_size(dtype);
  if (!plan_segments(B * H, N, seg_len, row_bytes, &nseg, &seg_chunks)) return (size_t)-1;
  return workspace_bytes(map, B * H, d_k, d_v, nseg, seg_chunks);
}

linattn_status_t linattn_prefill(int map, int dtype, int64_t B, int64_t H,
                                 int64_t N, int64_t d_k, int64_t d_v,
                                 const void* q, const void* k, const void* v,
                                 void* y, const float* S_in, const float* z_in,
                                 float* S_out, float* z_out, int64_t seg_len,
                                 void* workspace, size_t workspace_bytes_given,
                                 void* stream) {
  return prefill_common(map, dtype, B, H, N, d_k, d_v, q, k, v, false, nullptr, 1,
                        y, S_in, z_in, S_out, z_out, seg_len, workspace,
                        workspace_bytes_given, stream);
}

linattn_status_t linattn_prefill_gated(int map, int dtype, int64_t B, int64_t H,
                                       int64_t N, int64_t d_k, int64_t d_v,
                                       const void* q, const void* k, const void* v,
                                       const float* gate, int normalize, void* y,
                                       const float* S_in, const float* z_in,
                                       float* S_out, float* z_out, int64_t seg_len,
                                       void* workspace, size_t workspace_bytes_given,
                                       void* stream) {
  return prefill_common(map, dtype, B, H, N, d_k, d_v, q, k, v, true, gate, normalize,
                        y, S_in, z_in, S_out, z_out, seg_len, workspace,
                        workspace_bytes_given, stream);
}

linattn_status_t linattn_prefill_noalloc(int map, int dtype, int64_t B, int64_t H,
                                         int64_t N, int64_t d_k, int64_t d_v,
                                         const void* q, const void* k, const void* v,
                                         void* y, const float* S_in, const float* z_in,
                                         float* S_out, float* z_out, int64_t seg_len,
                                         void* stream) {
  return prefill_common(map, dtype, B, H, N, d_k, d_v, q, k, v, false, nullptr, 1,
                        y, S_in, z_in, S_out, z_out, seg_len, nullptr, 0, stream,
                        /*fixed_scratch=*/true);
}

linattn_status_t linattn_decode_step(int map, int dtype, int64_t B, int64_t H,
                                     int64_t d_k, int64_t d_v, const void* q,
                                     const void* k, const void* v, float* S,
                                     float* z, void* y, void* stream) {
  return decode_common(map, dtype, B, H, d_k, d_v, q, k, v, false, nullptr, 1, S, z,
                       y, stream);
}

linattn_status_t linattn_decode_step_gated(int map, int dtype, int64_t B, int64_t H,
                                           int64_t d_k, int64_t d_v, const void* q,
                                           const void* k, const void* v,
                                           const float* gate, int normalize, float* S,
                                           float* z, void* y, void* stream) {
  return decode_common(map, dtype, B, H, d_k, d_v, q, k, v, true, gate, normalize, S,
                       z, y, stream);
}

linattn_status_t linattn_swa_prefill(int dtype, int64_t B, int64_t H, int64_t N,
                                     int64_t d, int64_t window, float scale,
                                     const void* q, const void* k, const void* v,
                                     void* y, void* k_cache, void* v_cache,
                                     void* stream) {
  if (scale != scale) scale = default_swa_scale(d);
  if (!valid_dtype(dtype) || B <= 0 || H <= 0 || N <= 0 || d <= 0 || window <= 0 ||
      !finite(scale))
    return LINATTN_ERR_INVALID_ARGUMENT;
  if (!swa_dim_ok(d)) return LINATTN_ERR_UNSUPPORTED;
  if (B > kMaxElems / H) return LINATTN_ERR_INVALID_ARGUMENT;
  const int64_t BH = B * H;
  const size_t es = elem_size(dtype);
  // one sequence's rows must fit a buffer descriptor; the grid must fit
  if (N > kMaxSegBytes / (d * (int64_t)es)) return LINATTN_ERR_INVALID_ARGUMENT;
  if (BH > INT_MAX / ((N + 63) / 64)) return LINATTN_ERR_INVALID_ARGUMENT;
  if (q == nullptr || k == nullptr || v == nullptr || y == nullptr)
    return LINATTN_ERR_INVALID_ARGUMENT;
  if ((k_cache == nullptr) != (v_cache == nullptr)) return LINATTN_ERR_INVALID_ARGUMENT;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(y) ||
      (k_cache && (!aligned16(k_cache) || !aligned16(v_cache))))
    return LINATTN_ERR_INVALID_ARGUMENT;
  if (k_cache && BH > kMaxElems / (window * d)) return LINATTN_ERR_INVALID_ARGUMENT;
  const Range rq = rng(q, BH * N * d, es), rk = rng(k, BH * N * d, es);
  const Range rv = rng(v, BH * N * d, es), ry = rng(y, BH * N * d, es);
  const int64_t ncache = k_cache ? BH * window * d : 0;
  const Range rkc = rng(k_cache, ncache, es), rvc = rng(v_cache, ncache, es);
  const Range outs[3] = {ry, rkc, rvc};
  const Range ins[3] = {rq, rk, rv};
  for (int i = 0; i < 3; ++i) {
    for (int j = 0; j < 3; ++j)
      if (overlap(outs[i], ins[j])) return LINATTN_ERR_INVALID_ARGUMENT;
    for (int j = i + 1; j < 3; ++j)
      if (overlap(outs[i], outs[j])) return LINATTN_ERR_INVALID_ARGUMENT;
  }
  const hipError_t e = dispatch_swa_prefill(dtype, d, q, k, v, y, k_cache, v_cache, BH, N,
                                            window, scale,
                                            reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? LINATTN_OK : LINATTN_ERR_HIP;
}

linattn_status_t linattn_swa_decode_step(int dtype, int64_t B, int64_t H, int64_t d,
                                         int64_t window, float scale, const void* q,
                                         const void* k, const void* v, const int64_t* pos,
                                         void* k_cache, void* v_cache, void* y,
                                         void* stream) {
  if (scale != scale) scale = default_swa_scale(d);
  if (!valid_dtype(dtype) || B <= 0 || H <= 0 || d <= 0 || window <= 0 || !finite(scale))
    return LINATTN_ERR_INVALID_ARGUMENT;
  if (!swa_dim_ok(d) || window > kSwaMaxWindow) return LINATTN_ERR_UNSUPPORTED;
  if (B > kMaxElems / H) return LINATTN_ERR_INVALID_ARGUMENT;
  const int64_t BH = B * H;
  if (BH > INT_MAX || BH > kMaxElems / (window * d)) return LINATTN_ERR_INVALID_ARGUMENT;
  if (q == nullptr || k == nullptr || v == nullptr || pos == nullptr || k_cache == nullptr ||
      v_cache == nullptr || y == nullptr)
    return LINATTN_ERR_INVALID_ARGUMENT;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(y) ||
      !aligned16(k_cache) || !aligned16(v_cache) || ((uintptr_t)pos & 7u) != 0)
    return LINATTN_ERR_INVALID_ARGUMENT;
  const size_t es = elem_size(dtype);
  const Range rq = rng(q, BH * d, es), rk = rng(k, BH * d, es), rv = rng(v, BH * d, es);
  const Range rp = rng(pos, B, 8), ry = rng(y, BH * d, es);
  const Range rkc = rng(k_cache, BH * window * d, es), rvc = rng(v_cache, BH * window * d, es);
  const Range outs[3] = {ry, rkc, rvc};
  const Range ins[4] = {rq, rk, rv, rp};
  for (int i = 0; i < 3; ++i) {
    for (int j = 0; j < 4; ++j)
      if (overlap(outs[i], ins[j])) return LINATTN_ERR_INVALID_ARGUMENT;
    for (int j = i + 1; j < 3; ++j)
      if (overlap(outs[i], outs[j])) return LINATTN_ERR_INVALID_ARGUMENT;
  }
  const hipError_t e = dispatch_swa_decode(dtype, d, q, k, v, pos, k_cache, v_cache, y, B, H,
                                           window, scale,
                                           reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? LINATTN_OK : LINATTN_ERR_HIP;
}

}  // extern "C"
