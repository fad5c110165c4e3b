// das_api.cpp -- C ABI of the split-KV decode attention library: argument
// checks, the split plan and the kernel launches.  Declarations and the
// contract of every entry point are in include/das.h.
//
// Split plan: FlashDecoding++ post (TechKnowGenie), §2 (the sequence axis is a
// third grid axis cut into fixed-size chunks) and §6 "chunk size tuning guide"
// (small chunks inflate the phase-2 traffic, large chunks leave compute units
// idle; several times more blocks than compute units).
#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>

#include <hip/hip_runtime.h>

#include "das.h"
#include "das_internal.h"

namespace {

constexpr int kMaxDevices = 64;
std::atomic<int> g_cu_cache[kMaxDevices];

// Workgroups the automatic plan aims for, per four compute units.  One
// 8-wave phase-1 workgroup is resident per CU.  Measured on MI355X, about
// three streaming workgroups per four CUs already saturate HBM, and the
// fewer, longer splits cut the partial results and the per-workgroup start
// and end latencies (32K-row GQA decode: 16 splits 27.6 us, 24 splits
// 25.3 us, 32 splits 25.7 us).
constexpr int64_t kTargetWgsPer4Cus = 3;
// An INT4 cache moves a quarter of the bytes per row, so its call is bound
// by the per-row work on the CUs rather than by HBM, and the fused call aims
// for one workgroup on every CU (128K-row GQA decode: 24 splits 39 us, 32
// splits 33-37 us; an E4M3 cache measured the same with either plan).
constexpr int64_t kTargetWgsPer4CusInt4 = 4;
constexpr int64_t kMaxChunk = 8192;
// Even when the batch alone fills the chip, a maximal-length sequence is cut
// into at least this many splits, so that with variable lengths the last
// running workgroups hold only a fifth of the longest sequence.
constexpr int64_t kMinSplitsLongest = 5;
// das_decode_attention fuses the merge into phase 1 up to this many split
// workgroups per CU (see das_decode_attention below).
constexpr int64_t kFusedWgsPerCu = 4;
// Phase-1 workgroups are spread one per CU unless the grid holds at least
// this many per CU (see run_phase1).
constexpr int64_t kSpreadWgsPerCu = 8;

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
int64_t round_up(int64_t a, int64_t q) { return ceil_div(a, q) * q; }

// Smallest chunk the automatic plan uses.  Each split writes G*(D+2) floats
// of partial state per D*4 bytes of K+V row, so the partial traffic is about
// 2*G/chunk of the K/V bytes (written once, read once); these floors keep it
// near 3%.
int64_t min_chunk(int G) { return G >= 16 ? 1024 : (G >= 8 ? 512 : 256); }

bool supported_dims(int D, int G) {
  return (D == 64 || D == 128) && (G == 1 || G == 2 || G == 4 || G == 8 || G == 16);
}

int device_cus(int32_t num_cus, int* out) {
  if (num_cus > 0) {
    *out = num_cus;
    return DAS_OK;
  }
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return DAS_ELAUNCH;
  if (dev >= 0 && dev < kMaxDevices) {
    const int cached = g_cu_cache[dev].load(std::memory_order_relaxed);
    if (cached > 0) {
      *out = cached;
      return DAS_OK;
    }
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    return DAS_ELAUNCH;
  if (dev >= 0 && dev < kMaxDevices) g_cu_cache[dev].store(n, std::memory_order_relaxed);
  *out = n;
  return DAS_OK;
}

int64_t wgs_for_format(int format) {
  return format == das::kKvInt4 ? kTargetWgsPer4CusInt4 : kTargetWgsPer4Cus;
}

int plan_impl(int32_t B, int32_t Hkv, int32_t G, int32_t Smax, int32_t D, int32_t num_splits,
              int32_t num_cus, int32_t* ns_out, int32_t* chunk_out,
              int64_t wgs_per_4cus = kTargetWgsPer4Cus) {
  if (B < 1 || B > 65535 || Hkv < 1 || Hkv > 65535 || G < 1 || Smax < 1 || D < 1 ||
      num_splits < 0 || num_cus < 0)
    return DAS_EINVAL;
  if (!supported_dims(D, G)) return DAS_ENOTSUP;
  if (num_splits > DAS_MAX_SPLITS) return DAS_EINVAL;
  int64_t chunk;
  if (num_splits > 0) {
    chunk = round_up(ceil_div(Smax, num_splits), DAS_CHUNK_QUANTUM);
  } else {
    int cus = 0;
    const int rc = device_cus(num_cus, &cus);
    if (rc != DAS_OK) return rc;
    const int64_t units = (int64_t)B * Hkv;
    const int64_t target = std::max<int64_t>(1, wgs_per_4cus * cus / 4);
    int64_t ns_fill = ceil_div(target, units);
    if (ns_fill < kMinSplitsLongest) ns_fill = kMinSplitsLongest;
    chunk = round_up(ceil_div(Smax, ns_fill), DAS_CHUNK_QUANTUM);
    if (chunk < min_chunk(G)) chunk = min_chunk(G);
    if (chunk > kMaxChunk) chunk = kMaxChunk;
    // never more splits than the combine kernel can hold
    const int64_t floor_chunk = round_up(ceil_div(Smax, DAS_MAX_SPLITS), DAS_CHUNK_QUANTUM);
    if (chunk < floor_chunk) chunk = floor_chunk;
  }
  const int64_t ns = ceil_div(Smax, chunk);
  if (ns < 1 || ns > DAS_MAX_SPLITS || chunk > INT32_MAX) return DAS_EINVAL;
  *ns_out = (int32_t)ns;
  *chunk_out = (int32_t)chunk;
  return DAS_OK;
}

// Workspace: arrival counters (fixed area of das::kCounterBytes), then
// ws_o [B][Hq][ns][D] floats, then (256-byte aligned) ws_ml [B][Hq][ns][2].
size_t ws_o_offset() { return das::kCounterBytes; }
size_t ws_ml_offset(int32_t B, int32_t Hq, int32_t ns, int32_t D) {
  const size_t end = ws_o_offset() + (size_t)B * Hq * ns * D * sizeof(float);
  return (end + 255) & ~(size_t)255;
}
size_t ws_total(int32_t B, int32_t Hq, int32_t ns, int32_t D) {
  if (ns <= 1) return 0;
  return ws_ml_offset(B, Hq, ns, D) + (size_t)B * Hq * ns * 2 * sizeof(float);
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

struct Checked {
  int32_t G, ns, chunk;
};

// The K/V cache of one call: bf16 rows, E4M3 codes with fp32 scales per
// kv-head, or INT4 codes with fp32 scales per cached row (FlashDecoding++
// post, §4).
struct KvCache {
  const void* k;
  const void* v;
  const float* k_scale;
  const float* v_scale;
  int format;                // das::kKvBf16, kKvE4m3 or kKvInt4
  // paged cache (FlashDecoding++ post, §6): k and v are page pools
  const int32_t* block_table = nullptr;
  int32_t max_blocks = 0, page_size = 0, num_pages = 0, layout = 0;
  bool paged() const { return block_table != nullptr; }
  // bytes of a row of D elements
  int64_t row_bytes(int32_t D) const {
    return format == das::kKvInt4 ? D / 2 : (format == das::kKvE4m3 ? D : 2 * (int64_t)D);
  }
};

// Checks shared by every decode entry point.  Nothing is launched on failure.

int check_decode(const void* q, const void* k, const void* v, const int32_t* seq_lens, int32_t B,
                 int32_t Hq, int32_t Hkv, int32_t Smax, int32_t D, float scale, const void* out,
                 int32_t out_dtype, int32_t num_splits, const void* workspace,
                 size_t workspace_bytes, bool need_inputs, int64_t row_bytes, Checked* c,
                 int32_t page_size = 0, int64_t wgs_per_4cus = kTargetWgsPer4Cus) {
  if (seq_lens == nullptr || out == nullptr) return DAS_EINVAL;
  if (need_inputs && (q == nullptr || k == nullptr || v == nullptr)) return DAS_EINVAL;
  if (B < 1 || Hq < 1 || Hkv < 1 || Smax < 1 || D < 1) return DAS_EINVAL;
  if (Hq % Hkv != 0) return DAS_EINVAL;
  if (out_dtype != DAS_F32 && out_dtype != DAS_BF16) return DAS_EINVAL;
  if (!std::isfinite(scale)) return DAS_EINVAL;
  const int32_t G = Hq / Hkv;
  if (!supported_dims(D, G)) return DAS_ENOTSUP;
  // a sequence's K (or V) rows, plus one tile of overhang, are addressed
  // with 32-bit byte offsets
  if (page_size == 0 && (int64_t)(Smax + 256) * row_bytes > INT32_MAX) return DAS_ENOTSUP;
  if (need_inputs && (!aligned16(q) || !aligned16(k) || !aligned16(v))) return DAS_EINVAL;
  if (!aligned16(out) || ((uintptr_t)seq_lens & 3u) != 0) return DAS_EINVAL;
  int32_t ns = 0, chunk = 0;
  const int rc = plan_impl(B, Hkv, G, Smax, D, num_splits, 0, &ns, &chunk, wgs_per_4cus);
  if (rc != DAS_OK) return rc;
  if (page_size > 0 && chunk % page_size != 0) {
    // a paged cache's chunks are whole pages: fewer, longer splits, so the
    // workspace the unpaged plan asks for is enough
    chunk = (int32_t)(((int64_t)chunk + page_size - 1) / page_size * page_size);
    ns = (int32_t)(((int64_t)Smax + chunk - 1) / chunk);
  }
  if (ns > 1) {
    if (workspace == nullptr || !aligned16(workspace)) return DAS_EWORKSPACE;
    if (workspace_bytes < ws_total(B, Hq, ns, D)) return DAS_EWORKSPACE;
  }
  c->G = G;
  c->ns = ns;
  c->chunk = chunk;
  return DAS_OK;
}

int run_phase1(const void* q, const KvCache& kv, const int32_t* seq_lens, int32_t B, int32_t Hq,
               int32_t Hkv, int32_t Smax, int32_t D, float scale, void* out, int32_t out_dtype,
               float* lse_out, void* workspace, const Checked& c, bool fused, hipStream_t st) {
  das::SplitArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k = kv.k;
  a.v = kv.v;
  a.k_scale = kv.k_scale;
  a.v_scale = kv.v_scale;
  if (kv.paged()) {
    const int64_t R = kv.row_bytes(D);   // bytes of one row of one kv-head
    int shift = 0;
    while ((1 << shift) < kv.page_size) ++shift;
    a.block_table = kv.block_table;
    a.max_blocks = kv.max_blocks;
    a.page_shift = shift;
    a.num_pages = kv.num_pages;
    a.page_bytes = (int64_t)kv.page_size * Hkv * R;
    a.scale_page_stride = kv.page_size * Hkv;   // INT4 row-scale pools
    if (kv.layout == DAS_PAGED_HND) {
      a.row_stride = (int32_t)R;
      a.head_stride = (int32_t)(kv.page_size * R);
      a.scale_head_stride = kv.page_size;
      a.scale_row_stride = 1;
    } else {
      a.row_stride = (int32_t)(Hkv * R);
      a.head_stride = (int32_t)R;
      a.scale_head_stride = 1;
      a.scale_row_stride = Hkv;
    }
  }
  a.seq_lens = seq_lens;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.Smax = Smax;
  a.chunk = c.chunk;
  a.ns = c.ns;
  a.scale_log2e = scale * 1.44269504088896341f;
  a.direct = c.ns == 1;
  a.fused = fused && !a.direct;
  if (!a.direct) {
    char* ws = static_cast<char*>(workspace);
    a.counters = reinterpret_cast<unsigned int*>(ws);
    a.ws_o = reinterpret_cast<float*>(ws + ws_o_offset());
    a.ws_ml = reinterpret_cast<float*>(ws + ws_ml_offset(B, Hq, c.ns, D));
  }
  a.out = out;
  a.lse = lse_out;
  a.out_bf16 = out_dtype == DAS_BF16;
  // One workgroup per CU: left to itself the dispatcher doubles workgroups up
  // on some CUs while others idle whenever fewer workgroups stream than the
  // chip holds (INT4 cache, one workgroup per CU against doubled up: 32K-row
  // GQA decode 15.3 against 18.6 us, 128K 35 against 46 us).  A grid of
  // many workgroups per CU is left to the dispatcher: kernels whose
  // registers and LDS allow two workgroups on a CU (the INT4 matrix-core
  // path) then hide each other's stalls (INT4 varlen B=64 decode, 2560
  // workgroups: 153 us one per CU, 135 us two).  The bf16 kernels with
  // G >= 4 hold more than half a CU's LDS, so they are spread anyway; the
  // E4M3 kernels measure the same either way.
  int cus = 0;
  if (device_cus(0, &cus) != DAS_OK) return DAS_ELAUNCH;
  const bool one_per_cu =
      DAS_ONE_PER_CU != 0 && (int64_t)B * Hkv * c.ns < kSpreadWgsPerCu * (int64_t)cus;
  return das::launch_split_kv_decode(D, c.G, kv.format, kv.paged(), B, a, one_per_cu, st) ==
                 hipSuccess
             ? DAS_OK
             : DAS_ELAUNCH;
}

int run_phase2(const int32_t* seq_lens, int32_t B, int32_t Hq, int32_t Smax, int32_t D,
               const void* workspace, void* out, int32_t out_dtype, float* lse_out,
               const Checked& c, hipStream_t st) {
  if (c.ns <= 1) return DAS_OK;
  das::CombineArgs a{};
  const char* ws = static_cast<const char*>(workspace);
  a.ws_o = reinterpret_cast<const float*>(ws + ws_o_offset());
  a.ws_ml = reinterpret_cast<const float*>(ws + ws_ml_offset(B, Hq, c.ns, D));
  a.Hq = Hq;
  a.Smax = Smax;
  a.chunk = c.chunk;
  a.ns = c.ns;
  a.out = out;
  a.lse = lse_out;
  a.out_bf16 = out_dtype == DAS_BF16;
  return das::launch_lse_combine(D, B, a, st) == hipSuccess ? DAS_OK : DAS_ELAUNCH;
}

int split_impl(const void* q, const KvCache& kv, const int32_t* seq_lens, int32_t B, int32_t Hq,
               int32_t Hkv, int32_t Smax, int32_t D, float scale, void* out, int32_t out_dtype,
               float* lse_out, int32_t num_splits, void* workspace, size_t workspace_bytes,
               void* stream) {
  Checked c{};
  const int rc = check_decode(q, kv.k, kv.v, seq_lens, B, Hq, Hkv, Smax, D, scale, out, out_dtype,
                              num_splits, workspace, workspace_bytes, true, kv.row_bytes(D), &c);
  if (rc != DAS_OK) return rc;
  return run_phase1(q, kv, seq_lens, B, Hq, Hkv, Smax, D, scale, out, out_dtype, lse_out,
                    workspace, c, false, static_cast<hipStream_t>(stream));
}

int decode_impl(const void* q, const KvCache& kv, const int32_t* seq_lens, int32_t B, int32_t Hq,
                int32_t Hkv, int32_t Smax, int32_t D, float scale, void* out, int32_t out_dtype,
                float* lse_out, int32_t num_splits, void* workspace, size_t workspace_bytes,
                void* stream) {
  Checked c{};
  // the fused call's plan for this cache format (das_plan_kv); the
  // phase-1-only entry points keep das_plan's, which das_lse_combine assumes
  const int rc = check_decode(q, kv.k, kv.v, seq_lens, B, Hq, Hkv, Smax, D, scale, out, out_dtype,
                              num_splits, workspace, workspace_bytes, true, kv.row_bytes(D), &c,
                              kv.page_size, wgs_for_format(kv.format));
  if (rc != DAS_OK) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  // One launch: the last workgroup of each (b, kv-head) merges the splits.
  // Every split workgroup then ends with a store-completion wait and a
  // counter round trip while it holds its CU; with many more workgroups than
  // CUs that costs more than a second, small merge kernel (B=64 varlen
  // decode, 2560 workgroups: 375 us fused, 359 us as two kernels), so the
  // merge is fused only up to kFusedWgsPerCu workgroups per CU.  Shapes with
  // more (b, kv-head) pairs than counter slots always use the second kernel.
  int cus = 0;
  if (device_cus(0, &cus) != DAS_OK) return DAS_ELAUNCH;
  const bool fused = (int64_t)B * Hkv <= das::kCounterSlots &&
                     (int64_t)B * Hkv * c.ns <= kFusedWgsPerCu * cus;
  const int rc1 = run_phase1(q, kv, seq_lens, B, Hq, Hkv, Smax, D, scale, out, out_dtype, lse_out,
                             workspace, c, fused, st);
  if (rc1 != DAS_OK || fused) return rc1;
  return run_phase2(seq_lens, B, Hq, Smax, D, workspace, out, out_dtype, lse_out, c, st);
}

}  // namespace

extern "C" {

int das_plan(int32_t B, int32_t Hkv, int32_t G, int32_t Smax, int32_t D, int32_t num_splits,
             int32_t num_cus, int32_t* ns_out, int32_t* chunk_out) {
  if (ns_out == nullptr || chunk_out == nullptr) return DAS_EINVAL;
  return plan_impl(B, Hkv, G, Smax, D, num_splits, num_cus, ns_out, chunk_out);
}

int das_plan_kv(int32_t kv_dtype, int32_t B, int32_t Hkv, int32_t G, int32_t Smax, int32_t D,
                int32_t num_splits, int32_t num_cus, int32_t* ns_out, int32_t* chunk_out) {
  if (ns_out == nullptr || chunk_out == nullptr) return DAS_EINVAL;
  int format;
  switch (kv_dtype) {
    case DAS_BF16: format = das::kKvBf16; break;
    case DAS_E4M3: format = das::kKvE4m3; break;
    case DAS_INT4: format = das::kKvInt4; break;
    default: return DAS_EINVAL;
  }
  return plan_impl(B, Hkv, G, Smax, D, num_splits, num_cus, ns_out, chunk_out,
                   wgs_for_format(format));
}

size_t das_decode_workspace_bytes(int32_t B, int32_t Hq, int32_t Hkv, int32_t Smax, int32_t D,
                                  int32_t num_splits, int32_t num_cus) {
  if (Hkv < 1 || Hq < 1 || Hq % Hkv != 0) return (size_t)-1;
  // enough for the plan of every cache format (they differ only in the
  // automatic plan's target)
  size_t need = 0;
  for (const int64_t target : {kTargetWgsPer4Cus, kTargetWgsPer4CusInt4}) {
    int32_t ns = 0, chunk = 0;
    if (plan_impl(B, Hkv, Hq / Hkv, Smax, D, num_splits, num_cus, &ns, &chunk, target) != DAS_OK)
      return (size_t)-1;
    need = std::max(need, ws_total(B, Hq, ns, D));
  }
  return need;
}

int das_split_kv_decode(const void* q, const void* k_cache, const void* v_cache,
                        const int32_t* seq_lens, int32_t B, int32_t Hq, int32_t Hkv,
                        int32_t Smax, int32_t D, float scale, void* out, int32_t out_dtype,
                        float* lse_out, int32_t num_splits, void* workspace,
                        size_t workspace_bytes, void* stream) {
  const KvCache kv{k_cache, v_cache, nullptr, nullptr, das::kKvBf16};
  return split_impl(q, kv, seq_lens, B, Hq, Hkv, Smax, D, scale, out, out_dtype, lse_out,
                    num_splits, workspace, workspace_bytes, stream);
}

int das_split_kv_decode_fp8(const void* q, const void* k_cache, const void* v_cache,
                            const float* k_scale, const float* v_scale, const int32_t* seq_lens,
                            int32_t B, int32_t Hq, int32_t Hkv, int32_t Smax, int32_t D,
                            float scale, void* out, int32_t out_dtype, float* lse_out,
                            int32_t num_splits, void* workspace, size_t workspace_bytes,
                            void* stream) {
  if (k_scale == nullptr || v_scale == nullptr) return DAS_EINVAL;
  const KvCache kv{k_cache, v_cache, k_scale, v_scale, das::kKvE4m3};
  return split_impl(q, kv, seq_lens, B, Hq, Hkv, Smax, D, scale, out, out_dtype, lse_out,
                    num_splits, workspace, workspace_bytes, stream);
}

int das_split_kv_decode_int4(const void* q, const void* k_cache, const void* v_cache,
                             const float* k_scale, const float* v_scale, const int32_t* seq_lens,
                             int32_t B, int32_t Hq, int32_t Hkv, int32_t Smax, int32_t D,
                             float scale, void* out, int32_t out_dtype, float* lse_out,
                             int32_t num_splits, void* workspace, size_t workspace_bytes,
                             void* stream) {
  if (k_scale == nullptr || v_scale == nullptr) return DAS_EINVAL;
  if (((uintptr_t)k_scale & 3u) != 0 || ((uintptr_t)v_scale & 3u) != 0) return DAS_EINVAL;
  const KvCache kv{k_cache, v_cache, k_scale, v_scale, das::kKvInt4};
  return split_impl(q, kv, seq_lens, B, Hq, Hkv, Smax, D, scale, out, out_dtype, lse_out,
                    num_splits, workspace, workspace_bytes, stream);
}

int das_lse_combine(const int32_t* seq_lens, int32_t B, int32_t Hq, int32_t Hkv, int32_t Smax,
                    int32_t D, int32_t num_splits, const void* workspace,
                    size_t workspace_bytes, void* out, int32_t out_dtype, float* lse_out,
                    void* stream) {
  Checked c{};
  const int rc = check_decode(nullptr, nullptr, nullptr, seq_lens, B, Hq, Hkv, Smax, D, 1.0f, out,
                              out_dtype, num_splits, workspace, workspace_bytes, false, D, &c);
  if (rc != DAS_OK) return rc;
  return run_phase2(seq_lens, B, Hq, Smax, D, workspace, out, out_dtype, lse_out, c,
                    static_cast<hipStream_t>(stream));
}

int das_decode_attention(const void* q, const void* k_cache, const void* v_cache,
                         const int32_t* seq_lens, int32_t B, int32_t Hq, int32_t Hkv,
                         int32_t Smax, int32_t D, float scale, void* out, int32_t out_dtype,
                         float* lse_out, int32_t num_splits, void* workspace,
                         size_t workspace_bytes, void* stream) {
  const KvCache kv{k_cache, v_cache, nullptr, nullptr, das::kKvBf16};
  return decode_impl(q, kv, seq_lens, B, Hq, Hkv, Smax, D, scale, out, out_dtype, lse_out,
                     num_splits, workspace, workspace_bytes, stream);
}

int das_decode_attention_fp8(const void* q, const void* k_cache, const void* v_cache,
                             const float* k_scale, const float* v_scale, const int32_t* seq_lens,
                             int32_t B, int32_t Hq, int32_t Hkv, int32_t Smax, int32_t D,
                             float scale, void* out, int32_t out_dtype, float* lse_out,
                             int32_t num_splits, void* workspace, size_t workspace_bytes,
                             void* stream) {
  if (k_scale == nullptr || v_scale == nullptr) return DAS_EINVAL;
  const KvCache kv{k_cache, v_cache, k_scale, v_scale, das::kKvE4m3};
  return decode_impl(q, kv, seq_lens, B, Hq, Hkv, Smax, D, scale, out, out_dtype, lse_out,
                     num_splits, workspace, workspace_bytes, stream);
}

int das_decode_attention_int4(const void* q, const void* k_cache, const void* v_cache,
                              const float* k_scale, const float* v_scale, const int32_t* seq_lens,
                              int32_t B, int32_t Hq, int32_t Hkv, int32_t Smax, int32_t D,
                              float scale, void* out, int32_t out_dtype, float* lse_out,
                              int32_t num_splits, void* workspace, size_t workspace_bytes,
                              void* stream) {
  if (k_scale == nullptr || v_scale == nullptr) return DAS_EINVAL;
  if (((uintptr_t)k_scale & 3u) != 0 || ((uintptr_t)v_scale & 3u) != 0) return DAS_EINVAL;
  const KvCache kv{k_cache, v_cache, k_scale, v_scale, das::kKvInt4};
  return decode_impl(q, kv, seq_lens, B, Hq, Hkv, Smax, D, scale, out, out_dtype, lse_out,
                     num_splits, workspace, workspace_bytes, stream);
}

int das_decode_attention_paged(const void* q, const void* k_pool, const void* v_pool,
                               int32_t kv_dtype, const float* k_scale, const float* v_scale,
                               const int32_t* block_table, int32_t max_blocks, int32_t page_size,
                               int32_t num_pages, int32_t layout, const int32_t* seq_lens,
                               int32_t B, int32_t Hq, int32_t Hkv, int32_t D, float scale,
                               void* out, int32_t out_dtype, float* lse_out, int32_t num_splits,
                               void* workspace, size_t workspace_bytes, void* stream) {
  if (kv_dtype != DAS_BF16 && kv_dtype != DAS_E4M3 && kv_dtype != DAS_INT4) return DAS_EINVAL;
  const bool fp8 = kv_dtype == DAS_E4M3, int4 = kv_dtype == DAS_INT4;
  if ((fp8 || int4) && (k_scale == nullptr || v_scale == nullptr)) return DAS_EINVAL;
  if (int4 && (((uintptr_t)k_scale & 3u) != 0 || ((uintptr_t)v_scale & 3u) != 0))
    return DAS_EINVAL;
  if (block_table == nullptr || ((uintptr_t)block_table & 3u) != 0) return DAS_EINVAL;
  if (layout != DAS_PAGED_HND && layout != DAS_PAGED_NHD) return DAS_EINVAL;
  if (max_blocks < 1 || num_pages < 1) return DAS_EINVAL;
  if (page_size < 32 || page_size > 65536 || (page_size & (page_size - 1)) != 0)
    return DAS_ENOTSUP;
  if ((int64_t)max_blocks * page_size > INT32_MAX) return DAS_EINVAL;
  // one page (every kv-head) is addressed with 32-bit byte offsets, and so is
  // an INT4 page's pool of row scales
  const int64_t row_bytes = int4 ? D / 2 : (fp8 ? D : 2 * (int64_t)D);
  if ((int64_t)page_size * Hkv * row_bytes > INT32_MAX) return DAS_ENOTSUP;
  if (int4 && (int64_t)page_size * Hkv * 4 > INT32_MAX) return DAS_ENOTSUP;
  KvCache kv{k_pool, v_pool, (fp8 || int4) ? k_scale : nullptr,
             (fp8 || int4) ? v_scale : nullptr,
             int4 ? das::kKvInt4 : (fp8 ? das::kKvE4m3 : das::kKvBf16)};
  kv.block_table = block_table;
  kv.max_blocks = max_blocks;
  kv.page_size = page_size;
  kv.num_pages = num_pages;
  kv.layout = layout;
  return decode_impl(q, kv, seq_lens, B, Hq, Hkv, max_blocks * page_size, D, scale, out, out_dtype,
                     lse_out, num_splits, workspace, workspace_bytes, stream);
}

int das_merge_attn_states(const void* o_a, const float* lse_a, const void* o_b,
                          const float* lse_b, void* o_out, float* lse_out, int64_t rows,
                          int32_t D, int32_t o_dtype, void* stream) {
  if (rows < 0) return DAS_EINVAL;
  if (o_dtype != DAS_F32 && o_dtype != DAS_BF16) return DAS_EINVAL;
  if (D != 64 && D != 128) return DAS_ENOTSUP;
  if (rows == 0) return DAS_OK;
  if (o_a == nullptr || o_b == nullptr || o_out == nullptr || lse_a == nullptr ||
      lse_b == nullptr || lse_out == nullptr)
    return DAS_EINVAL;
  if (!aligned16(o_a) || !aligned16(o_b) || !aligned16(o_out)) return DAS_EINVAL;
  if (rows > (int64_t)4 * 2147483647LL) return DAS_EINVAL;
  das::MergeArgs a{o_a, lse_a, o_b, lse_b, o_out, lse_out, rows, o_dtype == DAS_BF16};
  return das::launch_merge_attn_states(D, a, static_cast<hipStream_t>(stream)) == hipSuccess
             ? DAS_OK
             : DAS_ELAUNCH;
}

const char* das_strerror(int status) {
  switch (status) {
    case DAS_OK: return "success";
    case DAS_EINVAL: return "invalid argument";
    case DAS_ENOTSUP: return "unsupported shape (head dim or GQA group)";
    case DAS_EWORKSPACE: return "workspace missing or too small";
    case DAS_ELAUNCH: return "HIP launch or device query failed";
    default: return "unknown status";
  }
}

}  // extern "C"
