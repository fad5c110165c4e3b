// das_internal.h -- argument blocks and launchers shared by the host API
// (das_api.cpp) and the gfx950 kernels (das_kernels.hip).  Not installed.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace das {

// Phase-1 shape knobs (compile-time; the defaults are the tuned ones).
#ifndef DAS_WAVES
#define DAS_WAVES 8          // waves per phase-1 workgroup
#endif
#ifndef DAS_KV_CACHE_POLICY
#define DAS_KV_CACHE_POLICY 2  // cache-policy bits of the K/V loads: nt (streamed once)
#endif
#ifndef DAS_ONE_PER_CU
#define DAS_ONE_PER_CU 1     // 1: every phase-1 workgroup takes a CU of its own
#endif
#ifndef DAS_MIN_WAVES_PER_EU
#define DAS_MIN_WAVES_PER_EU 2  // waves per SIMD the register allocator must allow
#endif
// Debug build (libdas_debug.so): 1 fills each wave's LDS tile region with
// 0xFF bytes (NaN as bf16, E4M3 and fp32) before its first use and after
// every tile it has finished reading, and the per-wave statistics slots with
// NaN before the stream.  A read that is not ordered after the write it
// needs (a missing wait for a load into LDS, a missing barrier before the
// cross-wave merge) then returns NaN instead of plausible stale values.
// Results are otherwise bit-for-bit those of the regular build.
#ifndef DAS_DEBUG_LDS_POISON
#define DAS_DEBUG_LDS_POISON 0
#endif

constexpr int kWaves = DAS_WAVES;
constexpr int kThreads = 64 * kWaves;
constexpr int kTile = 32;    // K/V rows a wave handles per loop iteration

// K/V cache element formats (FlashDecoding++ post, §4: quantised caches are
// turned back into wider floats on chip).
constexpr int kKvBf16 = 0;   // bf16 rows of D elements
constexpr int kKvE4m3 = 1;   // E4M3 codes, one fp32 scale per kv-head for K and for V
constexpr int kKvInt4 = 2;   // two's-complement 4-bit codes, two per byte (low nibble
                             // first), one fp32 scale per cached row for K and for V

// Phase 1 (FlashDecoding++ post, §3 phase 1).  One workgroup per
// (split, kv-head, batch row); it holds every query head of that kv-head.
struct SplitArgs {
  const uint16_t* q;         // bf16 [B][Hq][D]
  const void* k;             // [B][Hkv][Smax][D] bf16 or E4M3 codes, [..][D/2] INT4 bytes
  const void* v;
  const float* k_scale;      // E4M3: fp32 [Hkv]; INT4: fp32 [B][Hkv][Smax] (paged: a scale
                             // pool shaped like the code pool); bf16: unused
  const float* v_scale;
  const int32_t* seq_lens;   // int32 [B]
  int32_t Hq, Hkv, Smax;
  int32_t chunk, ns;         // rows per split, splits
  float scale_log2e;         // scale * log2(e): logits are kept in base-2 units
  float* ws_o;               // [B][Hq][ns][D] unnormalised partial outputs
  float* ws_ml;              // [B][Hq][ns][2] (split max in base-2 units, exp2 sum)
  void* out;                 // single-split plans: [B][Hq][D] f32 or bf16
  float* lse;                // single-split plans: [B][Hq] natural log, may be null
  int32_t out_bf16;
  int32_t direct;            // 1: single split, write out/lse instead of partials
  int32_t fused;             // 1: the last workgroup of each (b, kv-head) merges the splits
  unsigned int* counters;    // fused: arrival counters [B][Hkv], zero between calls
  // Paged cache (FlashDecoding++ post, §6): k and v point to page pools and
  // row j of sequence b is row j mod P of page block_table[b][j / P].
  const int32_t* block_table;  // [B][max_blocks]
  int32_t max_blocks;
  int32_t page_shift;        // log2 P, P >= 32 rows
  int32_t num_pages;         // pool size; table entries are clamped to it
  int32_t row_stride;        // bytes between rows of one kv-head within a page
  int32_t head_stride;       // bytes between kv-heads within a page
  int64_t page_bytes;        // bytes per page (every kv-head)
  // Paged INT4 cache: k_scale / v_scale are pools of row scales laid out like
  // the code pools; strides in floats.
  int32_t scale_page_stride; // floats per page (every kv-head)
  int32_t scale_head_stride; // floats between kv-heads within a page
  int32_t scale_row_stride;  // floats between rows of one kv-head
};

// Arrival counters live at the start of the workspace, one per (batch row,
// kv-head), in a fixed area so that their place never depends on the shape.
constexpr int kCounterSlots = 65536;
constexpr size_t kCounterBytes = (size_t)kCounterSlots * 4;
// The slot of pair p = b * Hkv + g (p < kCounterSlots): (p mod 1024) * 64 +
// p / 1024, a permutation of the slots that puts consecutive pairs 256 bytes
// apart.  The device-scope additions to one cache line are carried out one
// after another, so counters packed one per word (all 8 of a B = 1, Hkv = 8
// call in one line) made the 256 split workgroups that finish together queue
// for it: about 2 us, against none with the counters on separate lines
// (measured with 256 workgroups of 512 threads, one addition each).
constexpr int counter_slot(int pair) { return (pair & 1023) * 64 + (pair >> 10); }
static_assert(counter_slot(kCounterSlots - 1) == kCounterSlots - 1, "a permutation of the slots");

// Phase 2 (same post, §3 phase 2).  One workgroup per (query head, batch row).
struct CombineArgs {
  const float* ws_o;         // every slot written by phase 1 (empty splits: max -inf)
  const float* ws_ml;
  int32_t Hq, Smax, chunk, ns;   // chunk: rows per block, as in SplitArgs
  void* out;
  float* lse;                // may be null
  int32_t out_bf16;
};

// Two-state LSE merge (SGLang Diffusion "Parallelism Overview", ring merge).
struct MergeArgs {
  const void* o_a;
  const float* lse_a;
  const void* o_b;
  const float* lse_b;
  void* o_out;
  float* lse_out;
  int64_t rows;
  int32_t bf16;
};

// LDS per workgroup and per CU on gfx950 is 160 KiB.  A phase-1 workgroup
// that asks for kOnePerCuLds in total (static + dynamic) leaves no room for
// a second one on its CU.
constexpr int kMaxLdsPerWorkgroup = 160 * 1024;
constexpr int kOnePerCuLds = 84 * 1024;
hipError_t launch_split_kv_decode(int D, int G, int kv_format, bool paged, int B, const SplitArgs& a,
                                  bool one_per_cu, hipStream_t stream);
hipError_t launch_lse_combine(int D, int B, const CombineArgs& a, hipStream_t stream);
hipError_t launch_merge_attn_states(int D, const MergeArgs& a, hipStream_t stream);

}  // namespace das
