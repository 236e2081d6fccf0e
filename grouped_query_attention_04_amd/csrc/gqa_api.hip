// gqa_api.hip -- host side of libgqa for decode, paged decode and cache append: argument validation,
// split-K planning, workspace layout and kernel dispatch.  The prefill entry points are in
// gqa_prefill_api.hip and the planners in gqa_plan.cpp.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>

#include "gqa.h"
#include "gqa_append.h"
#include "gqa_host.h"
#include "gqa_kernels.h"

namespace {

using gqa_host::aligned;
using gqa_host::known_dtype;
using gqa_host::log2_exact;

constexpr int kWaves = 4;              // waves per workgroup (decode)
constexpr int kDefaultWorkgroups = 256;  // one per compute unit of an MI355X
constexpr int kMaxWorkgroups = 65536;
constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

int elt_bytes(int dt) { return dt == GQA_F32 ? 4 : dt == GQA_BF16 ? 2 : 1; }

// Query-head split of the matrix-core kernels.  A group of more than 16 query heads takes two or
// four 16-row query tiles per workgroup, and with few (batch, KV head) pairs such a launch is bound
// by latency, not bytes: each tile's products, the per-piece epilogue and the merge all grow with
// the group while the cache is small.  There each group is cut into hs sub-groups of at most 16
// heads, and every sub-group is a segment of its own (segment head j reads cache head j / hs): hs
// workgroups read each cache tile, each for G / hs query heads.  The hs segments of a cache head are
// adjacent in the tile space, so with 8 or more workgroups per segment the workgroups that read the
// same tiles run at the same time on the same XCD and its L2 serves the repeated reads (B8 Hq64 Hkv1
// L4096: HBM reads 1.2x the cache bytes, 31.0 -> 16.6 us).  hs is the smallest of 2, 3 and 4 that
// divides G into sub-groups of at most 16 (none for other group sizes), used when the split leaves
// at most 32 segments, or 64 for groups above 32 (whose unsplit kernel carries four query tiles):
// B16 Hq64 Hkv1 L4096 32.0 -> 24.7 us at 64 segments, while B32 Hq32 Hkv1 L4096 (64 segments)
// runs 22.7 us unsplit and 27.8 split.
int plan_split(const gqa_shape_t* s) {
  if (s->kv_dtype == GQA_F32) return 1;
  const int G = s->Hq / s->Hkv;
  if (G <= 16) return 1;
  const long long max_segments = G > 32 ? 64 : 32;
  for (int hs = 2; hs <= 4; ++hs)
    if (G % hs == 0 && G / hs <= 16) return (long long)s->B * s->Hkv * hs <= max_segments ? hs : 1;
  return 1;
}

// The library's workgroup count, for segments of G query heads on Hkv segment heads per batch entry
// (after the split).  Every segment that several workgroups share is merged at the end by the one
// that finishes it last, in rounds of partial-result loads whose size grows with the group; above
// 16 query heads per segment a round takes four pieces.  With few segments, 256 workgroups then cut
// each into 32 or more pieces whose merge outlasts the streaming (measured on B8 Hq32 Hkv1 L4096
// before the split: 28.8 us at 256 workgroups, 19.9 us at 64), so there the count is capped at
// eight pieces per segment on average, and at least 64 workgroups.
int plan_workgroups(const gqa_shape_t* s, int G, int Hkv) {
  if (s->num_workgroups > 0) return s->num_workgroups;
  if (G > 16) {
    const long long cap = 8ll * s->B * Hkv;
    return (int)std::max(64ll, std::min((long long)kDefaultWorkgroups, cap));
  }
  return kDefaultWorkgroups;
}

// Workspace: a 256-byte header (the initialisation tag and an error count), a counter area of
// fixed size (one counter per (batch, KV head), for up to kMaxUnits of them), then two
// published-piece slots per workgroup.  Because the counter area never moves, no shape's partial
// results ever land on another shape's counters, and since every call leaves its counters at zero,
// a workspace initialised once can serve calls of any shape.
constexpr size_t kMaxUnits = size_t(1) << 18;
constexpr size_t kHeaderBytes = gqa::kWorkspaceHeaderWords * sizeof(uint32_t);

struct Layout {
  int split;  // query-head split hs
  int workgroups;
  size_t counters_off, ml_off, o_off, total;
};

Layout plan(const gqa_shape_t* s) {
  Layout lo;
  lo.split = plan_split(s);
  const int G = s->Hq / s->Hkv / lo.split;  // query heads per segment
  lo.workgroups = plan_workgroups(s, G, s->Hkv * lo.split);
  const size_t slots = (size_t)lo.workgroups * 2;  // two per workgroup
  lo.counters_off = kHeaderBytes;
  lo.ml_off = kHeaderBytes + kMaxUnits * sizeof(uint32_t);
  lo.o_off = lo.ml_off + align_up(slots * (size_t)G * 2 * sizeof(float));
  lo.total = lo.o_off + align_up(slots * (size_t)G * (size_t)s->d * sizeof(float));
  return lo;
}

template <typename K>
gqa_status_t launch(K kernel, int grid, const gqa::Params& prm, hipStream_t stream) {
  hipLaunchKernelGGL(kernel, dim3(grid), dim3(kWaves * 64), 0, stream, prm);
  return hipGetLastError() == hipSuccess ? GQA_OK : GQA_ERR_HIP;
}

template <int D, int NT, bool FP8, bool PAGED, bool APPEND>
gqa_status_t dispatch_mfma_out(int out_dtype, int grid, const gqa::Params& prm, hipStream_t st) {
  if (out_dtype == GQA_BF16)
    return launch(gqa::decode_mfma_kernel<D, NT, FP8, uint16_t, kWaves, PAGED, APPEND>, grid, prm, st);
  return launch(gqa::decode_mfma_kernel<D, NT, FP8, float, kWaves, PAGED, APPEND>, grid, prm, st);
}

template <int D, bool FP8, bool PAGED, bool APPEND>
gqa_status_t dispatch_mfma(int G, int out_dtype, int grid, const gqa::Params& prm, hipStream_t st) {
  if (G <= 16) return dispatch_mfma_out<D, 1, FP8, PAGED, APPEND>(out_dtype, grid, prm, st);
  if (G <= 32) return dispatch_mfma_out<D, 2, FP8, PAGED, APPEND>(out_dtype, grid, prm, st);
  return dispatch_mfma_out<D, 4, FP8, PAGED, APPEND>(out_dtype, grid, prm, st);
}

template <bool PAGED, bool APPEND = false>
gqa_status_t dispatch_mfma_dtype(int kv_dtype, int d, int G, int out_dtype, int grid, const gqa::Params& prm,
                                 hipStream_t st) {
  if (kv_dtype == GQA_BF16)
    return d == 64 ? dispatch_mfma<64, false, PAGED, APPEND>(G, out_dtype, grid, prm, st)
                   : dispatch_mfma<128, false, PAGED, APPEND>(G, out_dtype, grid, prm, st);
  return d == 64 ? dispatch_mfma<64, true, PAGED, APPEND>(G, out_dtype, grid, prm, st)
                 : dispatch_mfma<128, true, PAGED, APPEND>(G, out_dtype, grid, prm, st);
}

// The dense shape that a paged shape's kernels and workspace are planned with: L is the longest
// sequence a page-table row can describe.
gqa_shape_t dense_equivalent(const gqa_paged_shape_t* s) {
  gqa_shape_t e;
  e.B = s->B;
  e.Hq = s->Hq;
  e.Hkv = s->Hkv;
  e.L = (int32_t)((long long)s->max_blocks * s->block_size);
  e.d = s->d;
  e.q_dtype = s->q_dtype;
  e.kv_dtype = s->kv_dtype;
  e.out_dtype = s->out_dtype;
  e.k_descale = s->k_descale;
  e.v_descale = s->v_descale;
  e.num_workgroups = s->num_workgroups;
  return e;
}

gqa::Params base_params(const void* q, const void* k, const void* v, const int32_t* seq_lens, float scale,
                        void* out, const gqa_shape_t* s, const Layout& lo, void* workspace) {
  gqa::Params prm;
  prm.q = q;
  prm.k = k;
  prm.v = v;
  prm.seq_lens = seq_lens;
  prm.out = out;
  char* ws = static_cast<char*>(workspace);
  prm.counters = reinterpret_cast<uint32_t*>(ws + lo.counters_off);
  prm.header = reinterpret_cast<uint32_t*>(ws);
  prm.part_ml = reinterpret_cast<float*>(ws + lo.ml_off);
  prm.part_o = reinterpret_cast<float*>(ws + lo.o_off);
  prm.B = s->B;
  prm.Hq = s->Hq;
  prm.Hkv = s->Hkv * lo.split;
  prm.L = s->L;
  prm.G = s->Hq / prm.Hkv;
  prm.hs = lo.split;
  prm.W = lo.workgroups;
  prm.qk_scale = (float)((double)scale * (double)s->k_descale * 1.4426950408889634);
  prm.v_descale = s->v_descale;
  prm.block_table = nullptr;
  prm.block_shift = 0;
  prm.max_blocks = 0;
  prm.num_blocks = 0;
  prm.k_new = nullptr;
  prm.v_new = nullptr;
  prm.skipped = nullptr;
  prm.k_enc_descale = s->k_descale;
  prm.v_enc_descale = s->v_descale;
  return prm;
}

template <int D, typename InT, bool PAGED>
gqa_status_t dispatch_append_kv(int kv_dtype, int B, const gqa::AppendParams& ap, hipStream_t st) {
  if (kv_dtype == GQA_F32)
    hipLaunchKernelGGL((gqa::append_kv_kernel<D, InT, 0, PAGED>), dim3(B), dim3(256), 0, st, ap);
  else if (kv_dtype == GQA_BF16)
    hipLaunchKernelGGL((gqa::append_kv_kernel<D, InT, 1, PAGED>), dim3(B), dim3(256), 0, st, ap);
  else
    hipLaunchKernelGGL((gqa::append_kv_kernel<D, InT, 2, PAGED>), dim3(B), dim3(256), 0, st, ap);
  return hipGetLastError() == hipSuccess ? GQA_OK : GQA_ERR_HIP;
}

template <bool PAGED>
gqa_status_t launch_append(int new_dtype, int kv_dtype, int d, int B, const gqa::AppendParams& ap,
                           hipStream_t st) {
  if (new_dtype == GQA_F32)
    return d == 64 ? dispatch_append_kv<64, float, PAGED>(kv_dtype, B, ap, st)
                   : dispatch_append_kv<128, float, PAGED>(kv_dtype, B, ap, st);
  return d == 64 ? dispatch_append_kv<64, uint16_t, PAGED>(kv_dtype, B, ap, st)
                 : dispatch_append_kv<128, uint16_t, PAGED>(kv_dtype, B, ap, st);
}

template <int D, int GT>
gqa_status_t dispatch_f32_out(int out_dtype, int grid, const gqa::Params& prm, hipStream_t st) {
  if (out_dtype == GQA_BF16) return launch(gqa::decode_f32_kernel<D, GT, uint16_t, kWaves>, grid, prm, st);
  return launch(gqa::decode_f32_kernel<D, GT, float, kWaves>, grid, prm, st);
}

template <int D>
gqa_status_t dispatch_f32(int G, int out_dtype, int grid, const gqa::Params& prm, hipStream_t st) {
  if (G <= 1) return dispatch_f32_out<D, 1>(out_dtype, grid, prm, st);
  if (G <= 2) return dispatch_f32_out<D, 2>(out_dtype, grid, prm, st);
  if (G <= 4) return dispatch_f32_out<D, 4>(out_dtype, grid, prm, st);
  if (G <= 8) return dispatch_f32_out<D, 8>(out_dtype, grid, prm, st);
  if (G <= 16) return dispatch_f32_out<D, 16>(out_dtype, grid, prm, st);
  return dispatch_f32_out<D, 32>(out_dtype, grid, prm, st);
}

// Scratch of gqa_decode_static: a file-scope device array, one copy per GPU, that stands in for the
// caller's workspace.  Host code never passes `scratch` itself to a kernel (on the host it names a
// stand-in, not device memory); it uses the device address hipGetSymbolAddress returns for the
// current device, kept per device in static_scratch_ptr.
static __device__ __align__(256) uint8_t scratch[GQA_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex static_scratch_mu;
void* static_scratch_ptr[kMaxDevices];  // guarded by static_scratch_mu; set once per device

// The device address of this GPU's scratch, set up on the device's first call: the address looked
// up, and the workspace initialised (header tag, counters cleared) by a kernel on `stream`, so the
// decode enqueued after it on the same stream finds it ready.  An initialisation enqueued while
// `stream` is being captured into a graph runs only when the graph does, so the device is marked
// ready only by one enqueued outside a capture (until then every call enqueues it again).  nullptr
// on a HIP error.
void* static_scratch(hipStream_t stream) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(static_scratch_mu);
  if (static_scratch_ptr[dev]) return static_scratch_ptr[dev];
  void* ptr = nullptr;
  if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
  hipStreamCaptureStatus capture = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(stream, &capture) != hipSuccess) return nullptr;
  const int n = (int)((kHeaderBytes + kMaxUnits * sizeof(uint32_t)) / sizeof(uint32_t));
  hipLaunchKernelGGL(gqa::init_workspace_kernel, dim3((n + 255) / 256), dim3(256), 0, stream,
                     static_cast<uint32_t*>(ptr), n);
  if (hipGetLastError() != hipSuccess) return nullptr;
  if (capture == hipStreamCaptureStatusNone) static_scratch_ptr[dev] = ptr;
  return ptr;
}

}  // namespace

extern "C" {

gqa_status_t gqa_shape_check(const gqa_shape_t* s) {
  if (!s) return GQA_ERR_INVALID_ARG;
  if (s->B <= 0 || s->Hq <= 0 || s->Hkv <= 0 || s->L <= 0 || s->d <= 0) return GQA_ERR_INVALID_ARG;
  if (s->Hq % s->Hkv != 0) return GQA_ERR_INVALID_ARG;
  if (!known_dtype(s->q_dtype) || !known_dtype(s->kv_dtype) || !known_dtype(s->out_dtype))
    return GQA_ERR_INVALID_ARG;
  if (!std::isfinite(s->k_descale) || !std::isfinite(s->v_descale)) return GQA_ERR_INVALID_ARG;
  if (s->num_workgroups < 0 || s->num_workgroups > kMaxWorkgroups) return GQA_ERR_INVALID_ARG;
  if (s->d != 64 && s->d != 128) return GQA_ERR_UNSUPPORTED;
  if (s->out_dtype != GQA_F32 && s->out_dtype != GQA_BF16) return GQA_ERR_UNSUPPORTED;
  const bool f32_path = s->q_dtype == GQA_F32 && s->kv_dtype == GQA_F32;
  const bool mfma_path = s->q_dtype == GQA_BF16 && (s->kv_dtype == GQA_BF16 || s->kv_dtype == GQA_FP8_E4M3);
  if (!f32_path && !mfma_path) return GQA_ERR_UNSUPPORTED;
  // group sizes: up to 64 query heads per KV head on the matrix cores (four 16-row query tiles), up
  // to 32 on the f32 vector path
  if (s->Hq / s->Hkv > (mfma_path ? 64 : 32)) return GQA_ERR_UNSUPPORTED;
  // per-(batch, KV head) cache slices are addressed with 32-bit byte offsets
  if ((long long)s->L * s->d * elt_bytes(s->kv_dtype) >= (1ll << 31)) return GQA_ERR_UNSUPPORTED;
  // the tile space (tiles of 16 positions per batch entry and KV head) is counted with 32-bit ints
  if ((long long)s->B * s->Hkv * ((s->L + 15) / 16) >= (1ll << 31)) return GQA_ERR_UNSUPPORTED;
  if ((long long)s->B * s->Hq >= (1ll << 31)) return GQA_ERR_UNSUPPORTED;
  if ((size_t)s->B * s->Hkv > kMaxUnits) return GQA_ERR_UNSUPPORTED;
  return GQA_OK;
}

size_t gqa_decode_workspace_bytes(const gqa_shape_t* s) {
  if (gqa_shape_check(s) != GQA_OK) return 0;
  return plan(s).total;
}

gqa_status_t gqa_workspace_init(void* workspace, size_t workspace_bytes, const gqa_shape_t* s,
                                void* stream) {
  const gqa_status_t st = gqa_shape_check(s);
  if (st != GQA_OK) return st;
  if (!workspace || !aligned(workspace, 16)) return GQA_ERR_INVALID_ARG;
  const Layout lo = plan(s);
  if (workspace_bytes < lo.total) return GQA_ERR_WORKSPACE;
  // the header and the whole counter area, whatever this shape's count of (batch, KV head) units
  const int n = (int)((kHeaderBytes + kMaxUnits * sizeof(uint32_t)) / sizeof(uint32_t));
  hipLaunchKernelGGL(gqa::init_workspace_kernel, dim3((n + 255) / 256), dim3(256), 0, (hipStream_t)stream,
                     static_cast<uint32_t*>(workspace), n);
  return hipGetLastError() == hipSuccess ? GQA_OK : GQA_ERR_HIP;
}

gqa_status_t gqa_decode(const void* q, const void* k_cache, const void* v_cache,
                        const int32_t* seq_lens, float scale, void* out, const gqa_shape_t* s,
                        void* workspace, size_t workspace_bytes, void* stream) {
  if (!q || !k_cache || !v_cache || !seq_lens || !out || !s) return GQA_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(out, 16) ||
      !aligned(seq_lens, 4))
    return GQA_ERR_INVALID_ARG;
  if (!std::isfinite(scale)) return GQA_ERR_INVALID_ARG;
  const gqa_status_t st = gqa_shape_check(s);
  if (st != GQA_OK) return st;
  const Layout lo = plan(s);
  if (!workspace || workspace_bytes < lo.total) return GQA_ERR_WORKSPACE;
  if (!aligned(workspace, 16)) return GQA_ERR_INVALID_ARG;

  const gqa::Params prm = base_params(q, k_cache, v_cache, seq_lens, scale, out, s, lo, workspace);
  const int grid = lo.workgroups;
  hipStream_t hs = (hipStream_t)stream;
  if (s->kv_dtype == GQA_F32) {
    return s->d == 64 ? dispatch_f32<64>(prm.G, s->out_dtype, grid, prm, hs)
                      : dispatch_f32<128>(prm.G, s->out_dtype, grid, prm, hs);
  }
  return dispatch_mfma_dtype<false>(s->kv_dtype, s->d, prm.G, s->out_dtype, grid, prm, hs);
}

gqa_status_t gqa_decode_static(const void* q, const void* k_cache, const void* v_cache,
                               const int32_t* seq_lens, float scale, void* out, const gqa_shape_t* s,
                               void* stream) {
  // every check gqa_decode makes before touching the device, plus the scratch's size limit
  if (!q || !k_cache || !v_cache || !seq_lens || !out || !s) return GQA_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(out, 16) ||
      !aligned(seq_lens, 4))
    return GQA_ERR_INVALID_ARG;
  if (!std::isfinite(scale)) return GQA_ERR_INVALID_ARG;
  const gqa_status_t st = gqa_shape_check(s);
  if (st != GQA_OK) return st;
  if (plan(s).total > (size_t)GQA_STATIC_SCRATCH_BYTES) return GQA_ERR_WORKSPACE;
  void* ws = static_scratch((hipStream_t)stream);
  if (!ws) return GQA_ERR_HIP;
  return gqa_decode(q, k_cache, v_cache, seq_lens, scale, out, s, ws, GQA_STATIC_SCRATCH_BYTES, stream);
}

gqa_status_t gqa_paged_shape_check(const gqa_paged_shape_t* s) {
  if (!s) return GQA_ERR_INVALID_ARG;
  if (s->block_size <= 0 || s->max_blocks <= 0 || s->num_blocks <= 0) return GQA_ERR_INVALID_ARG;
  if ((long long)s->max_blocks * s->block_size >= (1ll << 31)) return GQA_ERR_UNSUPPORTED;
  const gqa_shape_t e = dense_equivalent(s);
  const gqa_status_t st = gqa_shape_check(&e);
  if (st != GQA_OK) return st;
  if (s->kv_dtype == GQA_F32) return GQA_ERR_UNSUPPORTED;  // paged caches: bf16 or fp8 only
  const int shift = log2_exact(s->block_size);
  if (shift < 4 || shift > 12) return GQA_ERR_UNSUPPORTED;  // 16 .. 4096 positions per page
  if ((long long)s->max_blocks * s->B >= (1ll << 31)) return GQA_ERR_UNSUPPORTED;
  return GQA_OK;
}

size_t gqa_decode_paged_workspace_bytes(const gqa_paged_shape_t* s) {
  if (gqa_paged_shape_check(s) != GQA_OK) return 0;
  const gqa_shape_t e = dense_equivalent(s);
  return plan(&e).total;
}

gqa_status_t gqa_paged_workspace_init(void* workspace, size_t workspace_bytes, const gqa_paged_shape_t* s,
                                      void* stream) {
  const gqa_status_t st = gqa_paged_shape_check(s);
  if (st != GQA_OK) return st;
  const gqa_shape_t e = dense_equivalent(s);
  return gqa_workspace_init(workspace, workspace_bytes, &e, stream);
}

gqa_status_t gqa_decode_paged(const void* q, const void* k_pages, const void* v_pages,
                              const int32_t* block_table, const int32_t* seq_lens, float scale, void* out,
                              const gqa_paged_shape_t* s, void* workspace, size_t workspace_bytes,
                              void* stream) {
  if (!q || !k_pages || !v_pages || !block_table || !seq_lens || !out || !s) return GQA_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k_pages, 16) || !aligned(v_pages, 16) || !aligned(out, 16) ||
      !aligned(seq_lens, 4) || !aligned(block_table, 4))
    return GQA_ERR_INVALID_ARG;
  if (!std::isfinite(scale)) return GQA_ERR_INVALID_ARG;
  const gqa_status_t st = gqa_paged_shape_check(s);
  if (st != GQA_OK) return st;
  const gqa_shape_t e = dense_equivalent(s);
  const Layout lo = plan(&e);
  if (!workspace || workspace_bytes < lo.total) return GQA_ERR_WORKSPACE;
  if (!aligned(workspace, 16)) return GQA_ERR_INVALID_ARG;

  gqa::Params prm = base_params(q, k_pages, v_pages, seq_lens, scale, out, &e, lo, workspace);
  prm.block_table = block_table;
  prm.block_shift = log2_exact(s->block_size);
  prm.max_blocks = s->max_blocks;
  prm.num_blocks = s->num_blocks;
  return dispatch_mfma_dtype<true>(s->kv_dtype, s->d, prm.G, s->out_dtype, lo.workgroups, prm,
                                   (hipStream_t)stream);
}

// Checks shared by the fused append-and-decode entry points: bf16 new rows, a bf16 or fp8 cache
// (the matrix-core kernels), a bf16 query.
static gqa_status_t fused_append_check(const void* k_new, const void* v_new, const int32_t* skipped,
                                       int q_dtype, int kv_dtype) {
  if (!k_new || !v_new) return GQA_ERR_INVALID_ARG;
  if (!aligned(k_new, 16) || !aligned(v_new, 16) || (skipped && !aligned(skipped, 4))) return GQA_ERR_INVALID_ARG;
  if (q_dtype != GQA_BF16 || (kv_dtype != GQA_BF16 && kv_dtype != GQA_FP8_E4M3)) return GQA_ERR_UNSUPPORTED;
  return GQA_OK;
}

gqa_status_t gqa_decode_append(const void* q, const void* k_new, const void* v_new, void* k_cache,
                               void* v_cache, const int32_t* seq_lens, float scale, void* out,
                               const gqa_shape_t* s, int32_t* skipped_count, void* workspace,
                               size_t workspace_bytes, void* stream) {
  if (!q || !k_cache || !v_cache || !seq_lens || !out || !s) return GQA_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(out, 16) ||
      !aligned(seq_lens, 4))
    return GQA_ERR_INVALID_ARG;
  if (!std::isfinite(scale)) return GQA_ERR_INVALID_ARG;
  gqa_status_t st = gqa_shape_check(s);
  if (st != GQA_OK) return st;
  st = fused_append_check(k_new, v_new, skipped_count, s->q_dtype, s->kv_dtype);
  if (st != GQA_OK) return st;
  const Layout lo = plan(s);
  if (!workspace || workspace_bytes < lo.total) return GQA_ERR_WORKSPACE;
  if (!aligned(workspace, 16)) return GQA_ERR_INVALID_ARG;

  gqa::Params prm = base_params(q, k_cache, v_cache, seq_lens, scale, out, s, lo, workspace);
  prm.k_new = k_new;
  prm.v_new = v_new;
  prm.skipped = skipped_count;
  return dispatch_mfma_dtype<false, true>(s->kv_dtype, s->d, prm.G, s->out_dtype, lo.workgroups, prm,
                                          (hipStream_t)stream);
}

gqa_status_t gqa_decode_append_paged(const void* q, const void* k_new, const void* v_new, void* k_pages,
                                     void* v_pages, const int32_t* block_table, const int32_t* seq_lens,
                                     float scale, void* out, const gqa_paged_shape_t* s,
                                     int32_t* skipped_count, void* workspace, size_t workspace_bytes,
                                     void* stream) {
  if (!q || !k_pages || !v_pages || !block_table || !seq_lens || !out || !s) return GQA_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k_pages, 16) || !aligned(v_pages, 16) || !aligned(out, 16) ||
      !aligned(seq_lens, 4) || !aligned(block_table, 4))
    return GQA_ERR_INVALID_ARG;
  if (!std::isfinite(scale)) return GQA_ERR_INVALID_ARG;
  gqa_status_t st = gqa_paged_shape_check(s);
  if (st != GQA_OK) return st;
  st = fused_append_check(k_new, v_new, skipped_count, s->q_dtype, s->kv_dtype);
  if (st != GQA_OK) return st;
  const gqa_shape_t e = dense_equivalent(s);
  const Layout lo = plan(&e);
  if (!workspace || workspace_bytes < lo.total) return GQA_ERR_WORKSPACE;
  if (!aligned(workspace, 16)) return GQA_ERR_INVALID_ARG;

  gqa::Params prm = base_params(q, k_pages, v_pages, seq_lens, scale, out, &e, lo, workspace);
  prm.block_table = block_table;
  prm.block_shift = log2_exact(s->block_size);
  prm.max_blocks = s->max_blocks;
  prm.num_blocks = s->num_blocks;
  prm.k_new = k_new;
  prm.v_new = v_new;
  prm.skipped = skipped_count;
  return dispatch_mfma_dtype<true, true>(s->kv_dtype, s->d, prm.G, s->out_dtype, lo.workgroups, prm,
                                         (hipStream_t)stream);
}

gqa_status_t gqa_append_kv(const void* k_new, const void* v_new, int32_t new_dtype, void* k_cache,
                           void* v_cache, const gqa_shape_t* s, const int32_t* positions,
                           int32_t* skipped_count, void* stream) {
  if (!k_new || !v_new || !k_cache || !v_cache || !positions || !s) return GQA_ERR_INVALID_ARG;
  if (new_dtype != GQA_F32 && new_dtype != GQA_BF16) return GQA_ERR_INVALID_ARG;
  if (!aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) ||
      !aligned(positions, 4) || !aligned(skipped_count, 4))
    return GQA_ERR_INVALID_ARG;
  const gqa_status_t st = gqa_shape_check(s);
  if (st != GQA_OK) return st;
  if (!(s->k_descale > 0.f) || !(s->v_descale > 0.f)) return GQA_ERR_INVALID_ARG;
  gqa::AppendParams ap;
  ap.k_new = k_new;
  ap.v_new = v_new;
  ap.k_cache = k_cache;
  ap.v_cache = v_cache;
  ap.positions = positions;
  ap.skipped = skipped_count;
  ap.B = s->B;
  ap.Hkv = s->Hkv;
  ap.L = s->L;
  ap.k_descale = s->k_descale;
  ap.v_descale = s->v_descale;
  ap.block_table = nullptr;
  ap.block_shift = 0;
  ap.max_blocks = 0;
  ap.num_blocks = 0;
  return launch_append<false>(new_dtype, s->kv_dtype, s->d, s->B, ap, (hipStream_t)stream);
}

gqa_status_t gqa_append_kv_paged(const void* k_new, const void* v_new, int32_t new_dtype, void* k_pages,
                                 void* v_pages, const int32_t* block_table, const gqa_paged_shape_t* s,
                                 const int32_t* positions, int32_t* skipped_count, void* stream) {
  if (!k_new || !v_new || !k_pages || !v_pages || !block_table || !positions || !s) return GQA_ERR_INVALID_ARG;
  if (new_dtype != GQA_F32 && new_dtype != GQA_BF16) return GQA_ERR_INVALID_ARG;
  if (!aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(k_pages, 16) || !aligned(v_pages, 16) ||
      !aligned(positions, 4) || !aligned(skipped_count, 4) || !aligned(block_table, 4))
    return GQA_ERR_INVALID_ARG;
  const gqa_status_t st = gqa_paged_shape_check(s);
  if (st != GQA_OK) return st;
  if (!(s->k_descale > 0.f) || !(s->v_descale > 0.f)) return GQA_ERR_INVALID_ARG;
  gqa::AppendParams ap;
  ap.k_new = k_new;
  ap.v_new = v_new;
  ap.k_cache = k_pages;
  ap.v_cache = v_pages;
  ap.positions = positions;
  ap.skipped = skipped_count;
  ap.B = s->B;
  ap.Hkv = s->Hkv;
  ap.L = s->max_blocks * s->block_size;
  ap.k_descale = s->k_descale;
  ap.v_descale = s->v_descale;
  ap.block_table = block_table;
  ap.block_shift = log2_exact(s->block_size);
  ap.max_blocks = s->max_blocks;
  ap.num_blocks = s->num_blocks;
  return launch_append<true>(new_dtype, s->kv_dtype, s->d, s->B, ap, (hipStream_t)stream);
}

uint64_t gqa_kv_bytes_per_token(uint32_t layers, uint32_t kv_heads, uint32_t head_dim,
                                uint32_t dtype_bytes) {
  return (uint64_t)2 * layers * kv_heads * head_dim * dtype_bytes;
}

gqa_status_t gqa_validate_seq_lens(const int32_t* seq_lens, int32_t B, int32_t L,
                                   int32_t* bad_count, void* stream) {
  if (!seq_lens || !bad_count || B <= 0 || L < 0 || !aligned(seq_lens, 4) || !aligned(bad_count, 4))
    return GQA_ERR_INVALID_ARG;
  hipLaunchKernelGGL(gqa::count_bad_seq_lens_kernel, dim3(1), dim3(64), 0, (hipStream_t)stream,
                     seq_lens, B, L, bad_count);
  return hipGetLastError() == hipSuccess ? GQA_OK : GQA_ERR_HIP;
}

size_t gqa_stream_read_sink_words(void) { return 4096; }

gqa_status_t gqa_stream_read(const void* src, size_t bytes, void* sink, void* stream) {
  if (!src || !sink || bytes == 0 || bytes % 16 != 0 || !aligned(src, 16) || !aligned(sink, 4))
    return GQA_ERR_INVALID_ARG;
  const size_t n16 = bytes / 16;
  const int grid = 1024;
  const size_t per_wg = (n16 + grid - 1) / grid;
  hipLaunchKernelGGL(gqa::stream_read_kernel, dim3(grid), dim3(256), 0, (hipStream_t)stream,
                     static_cast<const gqa::u32x4_t*>(src), n16, per_wg, static_cast<uint32_t*>(sink));
  return hipGetLastError() == hipSuccess ? GQA_OK : GQA_ERR_HIP;
}

const char* gqa_status_string(gqa_status_t status) {
  switch (status) {
    case GQA_OK: return "GQA_OK: success";
    case GQA_ERR_INVALID_ARG: return "GQA_ERR_INVALID_ARG: null or misaligned pointer, bad dimension, Hq not a multiple of Hkv, bad workgroup count or size overflow";
    case GQA_ERR_UNSUPPORTED: return "GQA_ERR_UNSUPPORTED: head dim, group size, dtype combination or size outside what the library implements";
    case GQA_ERR_WORKSPACE: return "GQA_ERR_WORKSPACE: workspace missing or smaller than gqa_decode_workspace_bytes()";
    case GQA_ERR_HIP: return "GQA_ERR_HIP: the HIP runtime reported an error while enqueueing";
  }
  return "unknown gqa_status_t";
}

}  // extern "C"
