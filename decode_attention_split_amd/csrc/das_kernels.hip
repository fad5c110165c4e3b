// das_kernels.hip -- gfx950 kernels for split-KV decode attention.
//
// Sources (cited by page title and section):
//   [FD++]    "FlashDecoding++: 시퀀스 차원 KV 분할 병렬화와 GPU 언더유틸라이제이션 극복을 통한
//             LLM 서빙 극대화" (TechKnowGenie): §2 sequence axis as a grid axis, §3
//             phase 1 (per-chunk max, exponential sum, unnormalised output) and
//             phase 2 (global max, exp(m_c - M) rescale, sum, divide).
//   [SGL-PAR] "병렬 처리 개요 (Parallelism Overview)", SGLang Diffusion docs:
//             "What happens to the shapes" / "Constraints" -- the LSE merge of
//             partial attention states.
//
// Design notes (MI355X / CDNA4):
//   * Decode attention reads every K/V row once and does about G flops per
//     byte, so it is bound by HBM bandwidth.  Phase 1 streams K and V with
//     16-byte loads in which 16 (D=128) or 8 (D=64) consecutive lanes cover
//     one 256/128-byte row, so each wave-wide load covers whole rows.
//   * For G in {4, 8, 16} both products are real (small) matrix products and
//     run on the matrix cores (v_mfma_f32_16x16x32_bf16).  q.K^T is taken as
//     K.q^T, 16 cached rows by the G query heads (G = 16 fills the 16 columns,
//     G = 4 and 8 pad them), so that each
//     lane ends up holding one head's logits for eight rows -- exactly its
//     slots of the A operand of p.V, with no data movement.  p is split into
//     two bf16 halves (p = hi + lo to about 2^-18 relative), so p.V keeps
//     fp32-level accuracy; V is exact in bf16 (and so are E4M3 and the INT4
//     codes).  K and V go through a per-wave LDS tile with an XOR swizzle,
//     staged from registers one tile ahead (a wave's next tile is in flight
//     while it processes the current one); K is read one row per lane, V
//     column-wise with the gfx950 transposing LDS reads
//     (ds_read_b64_tr_b16 / _tr_b8).
//   * For G in {1, 2} q.K^T is a matrix-vector product on the vector ALUs
//     (v_dot2_f32_bf16: exact bf16 products, fp32 accumulation), and p.V runs
//     on the vector ALUs in fp32 straight from the coalesced V registers; p
//     reaches the lanes that need it through a small per-wave LDS buffer.  K
//     goes from HBM straight into the LDS tile (buffer_load ... lds).
//   * The online softmax keeps, per wave and head, a running max (base-2
//     units: logits are scaled by scale*log2(e) in fp32 after the dot) and
//     rescales the partial sums only when the max grows (on the matrix-core
//     path, only when it grows by more than 2^8).
//   * The waves of a workgroup merge their states through LDS at the end;
//     the workgroup then writes its split's (o, m, l) partial, or, for a
//     sequence with a single split, the final output.  With the fused
//     phase 2 the last workgroup of each (batch row, kv-head) to finish
//     merges that pair's partials in the same launch.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <algorithm>
#include <type_traits>

#include "das_internal.h"

namespace das {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr float kLn2 = 0.693147180559945309f;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 u) {
  bf16x8_t r;
  __builtin_memcpy(&r, &u, sizeof(r));
  return r;
}

__device__ __forceinline__ bf16x2_t as_bf16x2(uint32_t u) {
  bf16x2_t r;
  __builtin_memcpy(&r, &u, sizeof(r));
  return r;
}

__device__ __forceinline__ float lane_value(float x, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), lane));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Maximum that propagates NaN (IEEE 754-2019 maximum; v_maximum3_f32, which
// also takes a third operand).  fmaxf ignores a quiet NaN, so in the
// kernels' IEEE mode the compiler first quiets (canonicalises) each operand
// it cannot prove canonical -- every cross-lane value -- at one extra VALU
// instruction per operand.  The running maxima here only ever see finite
// logits and -inf (masked rows); a NaN input makes the output NaN either way.
__device__ __forceinline__ float fmax_prop(float a, float b) {
  return __builtin_elementwise_maximum(a, b);
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float x) {
  __bf16 h = (__bf16)x;  // v_cvt_pk_bf16_f32: round to nearest even
  uint16_t u;
  __builtin_memcpy(&u, &h, sizeof(u));
  return u;
}

__device__ __forceinline__ int clamp_len(int L, int smax) { return L < 0 ? 0 : (L > smax ? smax : L); }

// DPP row reductions: max or sum over each 16-lane row, result in every lane
// of the row (quad swaps, then half-row and row mirrors pair the halves).
template <bool kMax>
__device__ __forceinline__ float row_reduce16(float x) {
  auto op = [](float u, float v) { return kMax ? fmax_prop(u, v) : u + v; };
  x = op(x, __builtin_amdgcn_update_dpp(x, x, 0xB1, 0xF, 0xF, false));   // quad_perm [1,0,3,2]
  x = op(x, __builtin_amdgcn_update_dpp(x, x, 0x4E, 0xF, 0xF, false));   // quad_perm [2,3,0,1]
  x = op(x, __builtin_amdgcn_update_dpp(x, x, 0x141, 0xF, 0xF, false));  // row_half_mirror
  x = op(x, __builtin_amdgcn_update_dpp(x, x, 0x140, 0xF, 0xF, false));  // row_mirror
  return x;
}

// Sum (or max) of x over the lanes that differ from this one only in lane
// bits kLoBit..5, in every one of them.  Bits 5 and 4 use the gfx950 row-swap
// instructions (with both operands equal, the two results of a swap hold
// x[i] and x[i^32], or x[i^16], between them); bit 3 uses a DPP row rotate
// by 8 (lane i^8 within a 16-lane row).  No LDS traffic.
template <int kLoBit, bool kMax>
__device__ __forceinline__ float reduce_lane_bits(float x) {
  static_assert(kLoBit >= 3 && kLoBit <= 6, "lane bits 3..5");
  auto op = [](float u, float v) { return kMax ? fmax_prop(u, v) : u + v; };
  if constexpr (kLoBit <= 5) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                    false, false);
    x = op(__uint_as_float(r[0]), __uint_as_float(r[1]));
  }
  if constexpr (kLoBit <= 4) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x),
                                                    false, false);
    x = op(__uint_as_float(r[0]), __uint_as_float(r[1]));
  }
  if constexpr (kLoBit <= 3) x = op(x, __builtin_amdgcn_update_dpp(x, x, 0x128, 0xF, 0xF, false));
  return x;
}

constexpr int log2_int(int v) { return v <= 1 ? 0 : 1 + log2_int(v / 2); }

// v from lane K of this lane's 16-lane row (DPP row_newbcast), for K = 0..7
// into st[0..7].
template <int K = 0>
__device__ __forceinline__ void row_broadcast8(float2 v, float2* st) {
  st[K] = make_float2(
      __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v.x), 0x150 + K, 0xF, 0xF, false)),
      __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v.y), 0x150 + K, 0xF, 0xF, false)));
  if constexpr (K + 1 < 8) row_broadcast8<K + 1>(v, st);
}

// Raw buffer descriptor over `bytes` bytes at `base`: loads past the end
// return zeros, so a split's rows past its end need no branch.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}

__device__ __forceinline__ uint4 buffer_load16(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
  const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, DAS_KV_CACHE_POLICY);
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// Byte offset of the 16-byte chunk `c` of row `r` in a wave's K tile of
// kRowBytes-byte rows.  Chunk slots are XOR-swizzled with the row's 256-byte
// LDS bank row, so that the lanes that store one row, and the lanes that read
// one column of 16 rows, hit distinct bank groups.
template <int kRowBytes>
__device__ __forceinline__ int k_tile_offset(int r, int c) {
  constexpr int kChunks = kRowBytes / 16;        // 16-byte chunks per row
  constexpr int kRowsPerBank = 256 / kRowBytes;  // rows per 256-byte LDS bank row
  return r * kRowBytes + ((c ^ ((r / kRowsPerBank) % kChunks)) << 4);
}

// Eight E4M3 codes (OCP 8-bit floating point) as eight bf16 values, times
// the power of two `scale`; the conversion is exact (4 significant bits, a
// subset of bf16's range).
__device__ __forceinline__ uint4 e4m3x8_to_bf16x8(uint2 w, float scale = 1.0f) {
  const auto a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.x, scale, false);
  const auto b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.x, scale, true);
  const auto c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.y, scale, false);
  const auto d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.y, scale, true);
  return make_uint4(__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b),
                    __builtin_bit_cast(uint32_t, c), __builtin_bit_cast(uint32_t, d));
}

// Eight E4M3 codes as fp32, in order.
__device__ __forceinline__ void e4m3x8_to_f32(uint2 w, float* f) {
  const auto a = __builtin_amdgcn_cvt_pk_f32_fp8(w.x, false);
  const auto b = __builtin_amdgcn_cvt_pk_f32_fp8(w.x, true);
  const auto c = __builtin_amdgcn_cvt_pk_f32_fp8(w.y, false);
  const auto d = __builtin_amdgcn_cvt_pk_f32_fp8(w.y, true);
  f[0] = a[0]; f[1] = a[1]; f[2] = b[0]; f[3] = b[1];
  f[4] = c[0]; f[5] = c[1]; f[6] = d[0]; f[7] = d[1];
}

// INT4 codes through the E4M3 converters: a two's-complement nibble n with
// its top bit flipped is u = n + 8 in 0..15, and the byte u read as an E4M3
// code is u * 2^-9 exactly (u < 8: subnormal m = u; u >= 8: exponent 1,
// mantissa u - 8).  So the converters give u exactly, and the fixed offset 8
// is taken off by the caller (by linearity, once per dot product or sum).
// The eight codes of one dword w (elements 0..7, element 2i in the low
// nibble of byte i), as bf16 values u in the order 0, 2, 4, 6, 1, 3, 5, 7.
// The codes u of the low nibbles (even elements) and of the high nibbles
// (odd elements) of a dword, one per byte.  Masking before flipping the top
// bit makes each a single three-input bit operation (after a shift for the
// high nibbles).
__device__ __forceinline__ uint32_t int4_low_offset8(uint32_t w) {
  return (w & 0x0F0F0F0Fu) ^ 0x08080808u;
}
__device__ __forceinline__ uint32_t int4_high_offset8(uint32_t w) {
  return ((w >> 4) & 0x0F0F0F0Fu) ^ 0x08080808u;
}
__device__ __forceinline__ uint4 int4x8_to_bf16x8_offset8(uint32_t w) {
  return e4m3x8_to_bf16x8(make_uint2(int4_low_offset8(w), int4_high_offset8(w)), 512.0f);
}

// The eight codes of one dword as fp32 n * 2^-9, in element order (exact:
// u * 2^-9 from the converter minus 8 * 2^-9).
__device__ __forceinline__ void int4x8_to_f32_scaled(uint32_t w, float* f) {
  const uint32_t lo = int4_low_offset8(w), hi = int4_high_offset8(w);
  const auto a = __builtin_amdgcn_cvt_pk_f32_fp8(lo, false);
  const auto b = __builtin_amdgcn_cvt_pk_f32_fp8(lo, true);
  const auto c = __builtin_amdgcn_cvt_pk_f32_fp8(hi, false);
  const auto d = __builtin_amdgcn_cvt_pk_f32_fp8(hi, true);
  constexpr float kOff = 8.0f / 512.0f;
  f[0] = a[0] - kOff; f[2] = a[1] - kOff; f[4] = b[0] - kOff; f[6] = b[1] - kOff;
  f[1] = c[0] - kOff; f[3] = c[1] - kOff; f[5] = d[0] - kOff; f[7] = d[1] - kOff;
}

// Eight bf16 (a uint4, element 2i in the low half of word i) reordered to
// 0, 2, 4, 6, 1, 3, 5, 7: the order int4x8_to_bf16x8_offset8 gives codes in.
__device__ __forceinline__ uint4 bf16x8_even_odd(uint4 w) {
  return make_uint4((w.x & 0xFFFFu) | (w.y << 16), (w.z & 0xFFFFu) | (w.w << 16),
                    (w.x >> 16) | (w.y & 0xFFFF0000u), (w.z >> 16) | (w.w & 0xFFFF0000u));
}

__device__ __forceinline__ uint32_t buffer_load4(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, DAS_KV_CACHE_POLICY);
}

__device__ __forceinline__ uint2 buffer_load8(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  const u32x2_t v = __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, DAS_KV_CACHE_POLICY);
  return make_uint2(v[0], v[1]);
}

// Stores and loads with the sc1 cache policy: coherent at device scope, so a
// workgroup on another XCD (another L2) sees them without an L2 write-back or
// invalidate.
constexpr int kCoherent = 16;  // sc1

__device__ __forceinline__ void coherent_store16(__amdgpu_buffer_rsrc_t r, int off, float4 v) {
  typedef float f4_t __attribute__((ext_vector_type(4)));
  const f4_t w = {v.x, v.y, v.z, v.w};
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(
      unsigned int __attribute__((ext_vector_type(4))), w), r, off, 0, kCoherent);
}

__device__ __forceinline__ void coherent_store8(__amdgpu_buffer_rsrc_t r, int off, float x, float y) {
  typedef unsigned int u2_t __attribute__((ext_vector_type(2)));
  const u2_t w = {__float_as_uint(x), __float_as_uint(y)};
  __builtin_amdgcn_raw_buffer_store_b64(w, r, off, 0, kCoherent);
}

__device__ __forceinline__ float4 coherent_load16(__amdgpu_buffer_rsrc_t r, int off) {
  typedef unsigned int u4_t __attribute__((ext_vector_type(4)));
  const u4_t w = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kCoherent);
  return make_float4(__uint_as_float(w[0]), __uint_as_float(w[1]), __uint_as_float(w[2]),
                     __uint_as_float(w[3]));
}

__device__ __forceinline__ float2 coherent_load8(__amdgpu_buffer_rsrc_t r, int off) {
  typedef unsigned int u2_t __attribute__((ext_vector_type(2)));
  const u2_t w = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, kCoherent);
  return make_float2(__uint_as_float(w[0]), __uint_as_float(w[1]));
}

// Four consecutive outputs, f32 or bf16 (round to nearest even).
__device__ __forceinline__ void store_out4(const SplitArgs& a, size_t e, float x, float y, float z,
                                           float w) {
  if (a.out_bf16) {
    uint16_t* op = reinterpret_cast<uint16_t*>(a.out) + e;
    const uint32_t lo = f32_to_bf16_rne(x) | ((uint32_t)f32_to_bf16_rne(y) << 16);
    const uint32_t hi = f32_to_bf16_rne(z) | ((uint32_t)f32_to_bf16_rne(w) << 16);
    *reinterpret_cast<uint2*>(op) = make_uint2(lo, hi);
  } else {
    *reinterpret_cast<float4*>(reinterpret_cast<float*>(a.out) + e) = make_float4(x, y, z, w);
  }
}

// s_waitcnt immediate that waits until at most n vector-memory operations
// are outstanding (gfx9 encoding: vmcnt in bits 3:0 and 15:14; expcnt and
// lgkmcnt left at their maxima, i.e. not waited for).
constexpr int vmcnt_imm(int n) {
  return (n & 0xF) | (((n >> 4) & 0x3) << 14) | (0x7 << 4) | (0xF << 8);
}

// s_waitcnt immediate that waits until every LDS (and scalar memory)
// operation of the wave has completed.
constexpr int lgkmcnt0_imm() { return 0xF | (0x3 << 14) | (0x7 << 4); }

// Orders this wave's LDS accesses before the point against those after it
// (each wave owns its tile region, so no workgroup barrier is needed).
__device__ __forceinline__ void wave_lds_fence() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Debug build: fills kBytes (a multiple of 16) of this wave's LDS at p with
// 0xFF bytes, ordered after the wave's earlier LDS reads and completed before
// anything after it (including loads that write LDS directly) can land.
template <int kBytes>
__device__ __forceinline__ void poison_wave_lds(unsigned char* p, int lane) {
  static_assert(kBytes % 16 == 0, "16-byte stores");
  if constexpr (DAS_DEBUG_LDS_POISON) {
    wave_lds_fence();
    for (int off = 16 * lane; off < kBytes; off += 1024)
      *reinterpret_cast<uint4*>(p + off) = make_uint4(~0u, ~0u, ~0u, ~0u);
    __builtin_amdgcn_s_waitcnt(lgkmcnt0_imm());
    wave_lds_fence();
  }
}

// Bytes of one cached row of D elements.
template <int D, int kKv>
constexpr int kv_row_bytes() { return kKv == kKvInt4 ? D / 2 : (kKv == kKvE4m3 ? D : 2 * D); }

// LDS region of one wave of split_kv_decode<D, G, kKv>: a K tile and either
// a V tile (G >= 4: p.V on the matrix cores; an INT4 cache adds the tile's
// row scales) or a p buffer (G <= 2).  At the end of the stream the region
// holds the wave's state (G >= 4: G rows of D floats), so it is never
// smaller than that (INT4 tiles with 16 heads are).
template <int D, int G, int kKv>
constexpr int wave_region_bytes() {
  constexpr int tiles = kTile * kv_row_bytes<D, kKv>() * (G >= 4 ? 2 : 1) +
                        (G >= 4 ? (kKv == kKvInt4 ? 2 * kTile * 4 : 0) : kTile * G * 4);
  constexpr int state = G >= 4 ? G * D * 4 : 0;
  return tiles > state ? tiles : state;
}

// Static LDS of the wave regions of split_kv_decode<D, G, kKv>.
template <int D, int G, int kKv>
constexpr int split_smem_bytes() {
  return kWaves * wave_region_bytes<D, G, kKv>();
}

typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef int i32x2_t __attribute__((ext_vector_type(2)));

// gfx950 transposing LDS reads.  Within each 16-lane group, lane 4q+u (b16)
// receives as its element e the element u of the 8 bytes addressed by lane
// 4e+q; lane 8q+u (b8) receives as its byte e the byte u of the 8 bytes
// addressed by lane 2e+q.  So 16 lanes that address 4 (or 8) rows of a
// row-major tile, 16 columns at a time, get one column each.
__device__ __forceinline__ uint2 lds_read_tr16(const unsigned char* p) {
  const i16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4_t*)(p));
  return __builtin_bit_cast(uint2, v);
}

__device__ __forceinline__ uint2 lds_read_tr8(const unsigned char* p) {
  const i32x2_t v = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
      (__attribute__((address_space(3))) i32x2_t*)(p));
  return __builtin_bit_cast(uint2, v);
}

// p as the bf16 A operand pair (hi, lo) with hi + lo = p to about 2^-18
// relative: hi is p rounded to bf16, lo the exact remainder rounded to bf16.
__device__ __forceinline__ void split_bf16x8(const float* p, bf16x8_t& hi, bf16x8_t& lo) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const __bf16 h = (__bf16)p[i];
    hi[i] = h;
    lo[i] = (__bf16)(p[i] - (float)h);
  }
}

constexpr int pow2_floor(int v) { return v < 2 ? v : 2 * pow2_floor(v / 2); }

// ---------------------------------------------------------------------------
// Phase 1: split_kv_decode.  Grid (ns | 1, Hkv, B), kThreads threads.
// kKv: bf16 rows, E4M3 codes with one fp32 scale per kv-head each, or INT4
// codes with one fp32 scale per cached row each (FlashDecoding++ post, §4:
// dequantised on chip, right after the load).
// kPaged: K and V live in page pools listed by a block table (same post,
// §6); a tile never straddles a page (pages are >= 32 rows, chunks whole
// pages), so every tile finds its page with one table entry.  An INT4 pool
// comes with pools of row scales laid out like it.
// ---------------------------------------------------------------------------
// Waves per SIMD the register allocator must allow.  The INT4 kernels with
// G = 4 fit four (128 registers, no spills) and are bound by their per-row
// work, so two of their workgroups on a CU hide each other's stalls; the
// others keep two (their tiles or registers leave room for one workgroup).
template <int G, int kKv>
constexpr int min_waves_per_eu() {
  return (kKv == kKvInt4 && G == 4) ? 4 : DAS_MIN_WAVES_PER_EU;
}

template <int D, int G, int kKv, bool kPaged>
__global__ __launch_bounds__(kThreads, (min_waves_per_eu<G, kKv>()))
    void split_kv_decode_kernel(SplitArgs a) {
  constexpr bool kFp8 = kKv == kKvE4m3;
  constexpr bool kInt4 = kKv == kKvInt4;
  constexpr int kT = kTile;                     // rows per wave per step
  constexpr int kRowBytes = kv_row_bytes<D, kKv>();
  // G >= 4: p.V on the matrix cores, V staged through LDS like K.
  constexpr bool kMfmaPv = G >= 4;
  static_assert(kT == 32, "the operand layouts assume 32-row tiles");
  // G <= 2, V: every lane loads 8 elements (16 bytes of bf16, 8 of E4M3, 4
  // of INT4) of one row, D/8 consecutive lanes covering the row; the p.V
  // sums use the same layout.
  constexpr int kLanesPerRow = D / 8;
  constexpr int kRowsPerLoad = 64 / kLanesPerRow;
  constexpr int kLoads = kT / kRowsPerLoad;  // V loads per lane per tile
  constexpr int kVLaneBytes = kRowBytes / kLanesPerRow;
  // K (and, G >= 4, V) tiles: 16-byte loads, kKLanesPerRow lanes per row.
  constexpr int kKLanesPerRow = kRowBytes / 16;
  constexpr int kKRowsPerLoad = 64 / kKLanesPerRow;
  constexpr int kKLoads = kT / kKRowsPerLoad;
  constexpr int kKTileBytes = kT * kRowBytes;
  constexpr int kVTileBytes = kMfmaPv ? kKTileBytes : 0;
  // INT4 on the matrix-core path: the tile's K row scales, then its V row
  // scales, one float per row
  constexpr int kScaleBytes = (kMfmaPv && kInt4) ? 2 * kT * 4 : 0;
  constexpr int kPBytes = kMfmaPv ? 0 : kT * G * 4;
  constexpr int kWaveBytes = wave_region_bytes<D, G, kKv>();
  static_assert(kWaveBytes >= kKTileBytes + kVTileBytes + kScaleBytes + kPBytes, "tiles fit");
  constexpr int kSmemBytes = split_smem_bytes<D, G, kKv>();
  constexpr int kKBlocks = D / 32;              // MFMA k-blocks of 32 dims
  constexpr int kNBlocks = D / 16;              // p.V MFMA column blocks of 16 dims
  static_assert(kKTileBytes == kKLoads * 1024, "one 1 KiB LDS slab per K load");
  static_assert(kSmemBytes == kWaves * kWaveBytes, "one tile region per wave");
  // End-of-stream state of a wave.  G <= 2: the p.V sums are kept per row
  // group (lanes with the same row of a load) rather than summed across the
  // wave, as many row groups as fit in the wave's own tile region.  G >= 4:
  // the matrix cores have already summed over the rows (one group).
  constexpr int kRowGroups = kMfmaPv ? 1 : 64 / kLanesPerRow;        // 4 (D=128) or 8 (D=64)
  constexpr int kFitGroups = pow2_floor(kWaveBytes / (G * D * 4));
  constexpr int kMergeGroups = kThreads * 4 / (G * D);   // one merging thread per group and quad
  constexpr int kKeptGroups = kRowGroups < kFitGroups
                                  ? (kRowGroups < kMergeGroups ? kRowGroups : kMergeGroups)
                                  : (kFitGroups < kMergeGroups ? kFitGroups : kMergeGroups);
  static_assert(kKeptGroups >= 1, "one wave state fits in its tile region");

  __shared__ __attribute__((aligned(16))) unsigned char smem[kSmemBytes];

  // Grid (ns rounded up to odd, Hkv, B).  Workgroups are dealt to the eight
  // XCDs in linear-id order; an odd split extent keeps split s of every
  // sequence from always landing on the same XCD (when ns is a multiple of
  // 8, every sequence's first split would share XCD 0).  The padding splits
  // exit at once.
  const int s = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (SGPR)
  // The sequence length, read first and through the constant address space
  // (the lengths are read-only for the whole kernel): a scalar load that
  // goes out with the query loads below, before any branch.  Every K/V load
  // waits for it, so the fewer round trips ahead of it the better.
  const int len_in = ((const __attribute__((address_space(4))) int32_t*)a.seq_lens)[b];

  // ---- the query rows, loaded first: their latency overlaps that of the
  // sequence length and the issue of the first K/V tile ----
  // G >= 4: lane i loads, for k-block kb, the 8 dims of chunk 4*kb + i/16 of
  //         head i%16 (zero when >= G; INT4: chunk (i/16)*kKBlocks + kb, the
  //         lane's K bytes being contiguous).
  // G <= 2: lane i loads the part i / kT of D of every head.
  constexpr int kParts = 64 / kT;
  constexpr int kPartDims = D / kParts;
  constexpr int kQRegs = G >= 4 ? kKBlocks : G * (kPartDims / 8);
  uint4 qraw[kQRegs];
  if constexpr (G >= 4) {
    const int hh = lane & 15;
    const uint16_t* qrow = a.q + ((size_t)b * a.Hq + (size_t)g * G + (hh < G ? hh : 0)) * D;
#pragma unroll
    for (int kb = 0; kb < kKBlocks; ++kb) {
      const int c = kInt4 ? (lane >> 4) * kKBlocks + kb : 4 * kb + (lane >> 4);
      const uint4 w = *reinterpret_cast<const uint4*>(qrow + 8 * c);
      qraw[kb] = hh < G ? w : make_uint4(0, 0, 0, 0);
    }
  } else {
    const int part = lane / kT;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const uint4* qrow = reinterpret_cast<const uint4*>(
          a.q + ((size_t)b * a.Hq + (size_t)g * G + h) * D + part * kPartDims);
#pragma unroll
      for (int i = 0; i < kPartDims / 8; ++i) qraw[h * (kPartDims / 8) + i] = qrow[i];
    }
  }

  // Paged cache: the block-table entries of the pages this wave's tiles lie
  // in, read with one vector load, one entry per lane (page_for, below),
  // issued here so that their latency overlaps the length's.  Tile k of the
  // wave (rows row_lo + wave*kT + k*stride ...) lies in the wave's page
  // k >> tiles_per_entry; entry i is the page of its tile i << tiles_per_entry,
  // i.e. table slot first_slot + i * slot_step.  Entries past the table row
  // read as 0 (bounds-checked load) and are never used.
  constexpr int kStrideShift = log2_int(kWaves * kT);
  int tiles_per_entry = 0, first_slot = 0, slot_step = 0, entry_base = 0, table_lane = 0;
  const __amdgpu_buffer_rsrc_t table_rsrc =
      make_rsrc(kPaged ? a.block_table + (size_t)b * a.max_blocks : nullptr,
                kPaged ? a.max_blocks * 4 : 0);
  if constexpr (kPaged) {
    tiles_per_entry = max(a.page_shift - kStrideShift, 0);
    first_slot = (s * a.chunk + wave * kT) >> a.page_shift;
    slot_step = max((kWaves * kT) >> a.page_shift, 1);
    table_lane = (int)__builtin_amdgcn_raw_buffer_load_b32(
        table_rsrc, (first_slot + lane * slot_step) * 4, 0, 0);
  }
  // The length and the arguments the first K/V loads need are wanted here,
  // after the query loads have gone out: not one round trip at a time
  // further down, where the compiler would otherwise move their loads.
  __asm__ volatile("" : : "s"(len_in), "s"(a.k), "s"(a.v), "s"(a.chunk), "s"(a.ns),
                   "s"(a.Smax), "s"(a.Hkv), "s"(a.direct), "s"(a.fused));
  if (s >= a.ns) return;   // a padding split of the odd grid
  // wave-uniform, so everything derived from it -- the stream bounds, the
  // buffer offsets -- is too
  const int L = clamp_len(len_in, a.Smax);
  // The sequence's rows are cut into chunks of a.chunk rows; split s owns
  // chunk s (chunk * ns >= Smax, so every row has a split).
  const int n_chunks = (L + a.chunk - 1) / a.chunk;   // chunks holding valid rows
  const int nsb = min(a.ns, n_chunks);                // splits this sequence uses
  // An empty split exits at once.  With the fused merge nothing reads its
  // slots (split 0 of an empty sequence stays to write out = 0, lse = -inf);
  // otherwise it marks its slots empty (max -inf, sum 0: the merge's
  // identity), so that the separate phase-2 kernel reads every slot without
  // first reading the sequence's length.
  if (!a.direct && s >= n_chunks && !(a.fused && s == 0)) {
    if (!a.fused && tid < G) {
      const size_t row = ((size_t)b * a.Hq + (size_t)g * G + tid) * a.ns + s;
      *reinterpret_cast<float2*>(a.ws_ml + 2 * row) = make_float2(-INFINITY, 0.f);
    }
    return;
  }

  unsigned char* kt = smem + wave * kWaveBytes;
  float* pt = reinterpret_cast<float*>(kt + kKTileBytes);   // G <= 2
  // Per-wave running max and sum per head at the end of the stream.
  __shared__ float wst_ml[kWaves * 2 * G];

  // The sequence's valid rows of K and V as bounds-checked buffers: loads
  // past row L return zeros, and the rows beyond seq_lens are never read.
  // Contiguous cache: the sequence's valid rows as one bounds-checked
  // buffer.  Paged cache: a buffer per tile over its page's valid rows.
  // Either way loads past the last valid row return zeros and the rows
  // beyond seq_lens are never read.
  const int row_stride = kPaged ? a.row_stride : kRowBytes;  // bytes between rows
  const size_t slab = kPaged ? 0 : ((size_t)b * a.Hkv + g) * (size_t)a.Smax * kRowBytes;
  const __amdgpu_buffer_rsrc_t rk_seq =
      make_rsrc(reinterpret_cast<const unsigned char*>(a.k) + slab, kPaged ? 0 : L * kRowBytes);
  const __amdgpu_buffer_rsrc_t rv_seq =
      make_rsrc(reinterpret_cast<const unsigned char*>(a.v) + slab, kPaged ? 0 : L * kRowBytes);
  // INT4, contiguous cache: the sequence's row scales of K and V, L floats
  // each (rows past the sequence read as 0, checked per row); a paged cache
  // builds them per page
  const size_t scale_slab = kPaged ? 0 : ((size_t)b * a.Hkv + g) * (size_t)a.Smax;
  const int scale_bytes = (kInt4 && !kPaged) ? L * 4 : 0;
  const __amdgpu_buffer_rsrc_t rks = make_rsrc(a.k_scale + (kInt4 ? scale_slab : 0), scale_bytes);
  const __amdgpu_buffer_rsrc_t rvs = make_rsrc(a.v_scale + (kInt4 ? scale_slab : 0), scale_bytes);
  int row_end = 0;                              // end of the chunk being streamed
  const int row_in_load = lane / kLanesPerRow;  // this lane's V row within a load
  const int chunk = lane % kLanesPerRow;        // this lane's 8 elements of a V row
  const int lane_off = row_in_load * row_stride + kVLaneBytes * chunk;
  const int k_row_in_load = lane / kKLanesPerRow;
  const int k_slot = lane % kKLanesPerRow;
  // Logits in base-2 units; an E4M3 cache's K scale multiplies the finished
  // dot product, its V scale the finished p.V sums.  An INT4 cache's row
  // scales multiply each row's dot product and each row's p.
  float c2 = a.scale_log2e;
  float v_scale = 1.f;
  if constexpr (kFp8) {
    // (read-only for the whole kernel: scalar loads, as the length)
    c2 *= ((const __attribute__((address_space(4))) float*)a.k_scale)[g];
    v_scale = ((const __attribute__((address_space(4))) float*)a.v_scale)[g];
  }

  // ---- query operand (filled from qraw once the first tile is issued) ----
  // G >= 4: MFMA B operand (q^T); lane i holds head i%16 and the dims it
  //         loaded.  G <= 2: lane i works on row i % kT and the part i / kT
  //         of D; it holds that part of every head as bf16 pairs.
  // INT4 codes convert in the order 0, 2, 4, 6, 1, 3, 5, 7 within each
  // group of 8 dims, so q's dims are held in that order too, and the sum of
  // q over D is kept to take off the codes' offset: (q.(u - 8)) = q.u - 8 sum(q).
  bf16x8_t qa[kKBlocks];
  uint32_t qv[G <= 2 ? G : 1][G <= 2 ? kPartDims / 2 : 1];
  float q8[G <= 2 ? G : 1];     // INT4: 8 * sum(q) per head (G >= 4: the lane's head)

  // ---- per-wave running state (maxima in base-2 units) ----
  // G <= 2: wave-uniform running max per head, this lane's exponential sums,
  //         and p.V sums for this lane's 8 dims of its row.
  float m_run[G];
  float acc[G][8];
  float l_lane[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m_run[h] = -INFINITY;
    l_lane[h] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
  }
  // G >= 4: lane l keeps the running max and exponential sum of head l%16
  //         (the four lanes with that head agree on the max) and the p.V sums
  //         in the MFMA accumulator layout: oacc[nb][r] is head 4*(l/16) + r,
  //         dim 16*nb + l%16.
  //         INT4: oacc[2*cb + h][r] is dim 32*cb + 16*(l%16 / 8) + 2*(l%8) + h,
  //         and osum[r] the sum of head 4*(l/16) + r's p (times the row
  //         scales) that the offset of the codes multiplies.
  float m_lane = -INFINITY, l_sum = 0.f;
  f32x4_t oacc[kNBlocks];
#pragma unroll
  for (int nb = 0; nb < kNBlocks; ++nb) oacc[nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  f32x4_t osum = {0.f, 0.f, 0.f, 0.f};

  // A K tile in LDS: load m fills the 1 KiB slab [m KiB, (m+1) KiB) of the
  // tile, lane l the 16 bytes at 16*l, i.e. row kKRowsPerLoad*m +
  // k_row_in_load, slot k_slot.  The lane fetches the logical chunk whose
  // swizzled slot that is, so the tile ends up in the k_tile_offset layout.
  // G >= 4: V is laid out the same way in the V tile that follows (both
  // staged from registers by stage_tile); G <= 2: K is loaded straight into
  // LDS (buffer_load ... lds) and V goes to registers.
  using VReg = typename std::conditional<
      kInt4, uint32_t, typename std::conditional<kFp8, uint2, uint4>::type>::type;
  // INT4, G <= 2: the K and V scales of this lane's row (lane % kT) of the tile
  float row_ks = 0.f, row_vs = 0.f;
  // Paged cache: the block-table entry of the page holding the wave's tile
  // k (k = 0, 1, ... in stream order), a lane read of the entries loaded at
  // the start; every 64 entries (a split longer than 64 of the wave's pages)
  // the next 64 are loaded, a round trip the stream waits for once.
  auto page_for = [&](int k) -> int {
    const int e = k >> tiles_per_entry;
    if (e >= entry_base + 64) {   // wave-uniform; k grows by one per call
      entry_base += 64;
      table_lane = (int)__builtin_amdgcn_raw_buffer_load_b32(
          table_rsrc, (first_slot + (entry_base + lane) * slot_step) * 4, 0, 0);
    }
    return __builtin_amdgcn_readlane(table_lane, e - entry_base);
  };

  // G <= 2: K straight into the wave's LDS tile, V (and INT4 row scales)
  // into registers.
  // Paged INT4 cache: the row scales of the page holding rows [p0, p0 +
  // nvalid) of this kv-head, as bounds-checked buffers (rows past the
  // sequence read as 0).
  auto page_scales = [&](int page, int nvalid, __amdgpu_buffer_rsrc_t& sk,
                         __amdgpu_buffer_rsrc_t& sv) {
    const size_t so = (size_t)page * (size_t)a.scale_page_stride +
                      (size_t)g * (size_t)a.scale_head_stride;
    const int sbytes = ((nvalid - 1) * a.scale_row_stride + 1) * 4;
    sk = make_rsrc(a.k_scale + so, sbytes);
    sv = make_rsrc(a.v_scale + so, sbytes);
  };
  // INT4: floats between the scales of consecutive rows
  const int scale_row = kPaged ? a.scale_row_stride : 1;

  auto load_tile = [&](int r0, VReg* vr, unsigned char* kbuf, int page) {
    __amdgpu_buffer_rsrc_t rk = rk_seq, rv = rv_seq, sk = rks, sv = rvs;
    int soff = r0 * kRowBytes;
    int srow = r0;   // INT4: the tile's first row within the scale buffers
    if constexpr (kPaged) {
      // this tile's page; a table entry outside the pool is clamped into it
      // (wrong rows, never an access outside the pool)
      const int slot = r0 >> a.page_shift;
      page = min(max(page, 0), a.num_pages - 1);
      const int p0 = slot << a.page_shift;                  // first row of the page
      const int nvalid = min(L - p0, 1 << a.page_shift);    // >= 1: r0 < L
      const size_t off = (size_t)page * (size_t)a.page_bytes + (size_t)g * (size_t)a.head_stride;
      const int bytes = (nvalid - 1) * row_stride + kRowBytes;
      rk = make_rsrc(reinterpret_cast<const unsigned char*>(a.k) + off, bytes);
      rv = make_rsrc(reinterpret_cast<const unsigned char*>(a.v) + off, bytes);
      soff = (r0 - p0) * row_stride;
      if constexpr (kInt4) {
        page_scales(page, nvalid, sk, sv);
        srow = r0 - p0;
      }
    }
    // The tile offsets are the same for every lane.  Said so explicitly: the
    // compiler otherwise keeps the offset's induction variable in a vector
    // register and wraps every load in a loop over its distinct values.
    soff = __builtin_amdgcn_readfirstlane(soff);
    srow = __builtin_amdgcn_readfirstlane(srow);
    if constexpr (kInt4) {
      row_ks = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
          sk, (lane % kT) * scale_row * 4, srow * scale_row * 4, 0));
      row_vs = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
          sv, (lane % kT) * scale_row * 4, srow * scale_row * 4, 0));
    }
#pragma unroll
    for (int m = 0; m < kKLoads; ++m) {
      const int r = kKRowsPerLoad * m + k_row_in_load;
      const int c = k_slot ^ ((r / (256 / kRowBytes)) % kKLanesPerRow);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rk, (__attribute__((address_space(3))) void*)(kbuf + m * 1024), 16,
          r * row_stride + 16 * c, soff, 0, DAS_KV_CACHE_POLICY);
    }
#pragma unroll
    for (int m = 0; m < kLoads; ++m) {
      if constexpr (kInt4)
        vr[m] = buffer_load4(rv, lane_off + m * kRowsPerLoad * row_stride, soff);
      else if constexpr (kFp8)
        vr[m] = buffer_load8(rv, lane_off + m * kRowsPerLoad * row_stride, soff);
      else
        vr[m] = buffer_load16(rv, lane_off + m * kRowsPerLoad * row_stride, soff);
    }
  };

  // G >= 4: the tiles go through registers, one tile ahead of the one being
  // processed.  fetch_tile loads tile r0 -- the 16-byte chunks that go to
  // [m KiB + 16 lane] of the K and V tiles (the layout load_tile's K loads
  // produce), and the INT4 row scales (lanes 0..kT-1 K, kT..63 V) -- and
  // stage_tile writes it into the wave's LDS tiles once the previous tile
  // has been processed.
  // The next tile's loads are thus in flight while the current one is
  // processed, instead of the wave issuing nothing during that time.
  struct TileRegs {
    uint4 k[kMfmaPv ? kKLoads : 1];
    uint4 v[kMfmaPv ? kKLoads : 1];
    float ksc, vsc;   // INT4: the K and V scales of row lane % kT
  };
  auto fetch_tile = [&](int r0, TileRegs& t, int page) {
    __amdgpu_buffer_rsrc_t rk = rk_seq, rv = rv_seq, sk = rks, sv = rvs;
    int soff = r0 * kRowBytes;
    int srow = r0;   // INT4: the tile's first row within the scale buffers
    if constexpr (kPaged) {
      const int slot = r0 >> a.page_shift;
      page = min(max(page, 0), a.num_pages - 1);
      const int p0 = slot << a.page_shift;
      const int nvalid = min(L - p0, 1 << a.page_shift);
      const size_t off = (size_t)page * (size_t)a.page_bytes + (size_t)g * (size_t)a.head_stride;
      const int bytes = (nvalid - 1) * row_stride + kRowBytes;
      rk = make_rsrc(reinterpret_cast<const unsigned char*>(a.k) + off, bytes);
      rv = make_rsrc(reinterpret_cast<const unsigned char*>(a.v) + off, bytes);
      soff = (r0 - p0) * row_stride;
      if constexpr (kInt4) {
        page_scales(page, nvalid, sk, sv);
        srow = r0 - p0;
      }
    }
    soff = __builtin_amdgcn_readfirstlane(soff);   // the same for every lane
    srow = __builtin_amdgcn_readfirstlane(srow);
    if constexpr (kInt4) {
      // Both scales of row lane % kT, each through a wave-uniform
      // descriptor (stage_tile keeps the K ones in lanes [0, kT), the V ones
      // in the others).  Choosing the descriptor per lane would make it
      // divergent, and the compiler then loops over its distinct values with
      // a wait for every outstanding load -- the tile prefetch included --
      // inside the loop; choosing between the two values here would wait for
      // them at once.
      const int soff_s = srow * scale_row * 4, voff_s = (lane % kT) * scale_row * 4;
      t.ksc = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(sk, voff_s, soff_s, 0));
      t.vsc = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(sv, voff_s, soff_s, 0));
    }
#pragma unroll
    for (int m = 0; m < kKLoads; ++m) {
      const int r = kKRowsPerLoad * m + k_row_in_load;
      const int c = k_slot ^ ((r / (256 / kRowBytes)) % kKLanesPerRow);
      t.k[m] = buffer_load16(rk, r * row_stride + 16 * c, soff);
    }
#pragma unroll
    for (int m = 0; m < kKLoads; ++m) {
      const int r = kKRowsPerLoad * m + k_row_in_load;
      const int c = k_slot ^ ((r / (256 / kRowBytes)) % kKLanesPerRow);
      t.v[m] = buffer_load16(rv, r * row_stride + 16 * c, soff);
    }
  };
  auto stage_tile = [&](const TileRegs& t, unsigned char* kbuf) {
    wave_lds_fence();   // the previous tile's LDS reads come first
#pragma unroll
    for (int m = 0; m < kKLoads; ++m)
      *reinterpret_cast<uint4*>(kbuf + m * 1024 + 16 * lane) = t.k[m];
#pragma unroll
    for (int m = 0; m < kKLoads; ++m)
      *reinterpret_cast<uint4*>(kbuf + kKTileBytes + m * 1024 + 16 * lane) = t.v[m];
    // INT4: the K row scales go in with the logit scale folded in
    if constexpr (kInt4)
      reinterpret_cast<float*>(kbuf + 2 * kKTileBytes)[lane] = lane < kT ? t.ksc * c2 : t.vsc;
    wave_lds_fence();
  };

  // Elements 8*grp8 .. 8*grp8+7 of row r of a K tile, as bf16 (INT4: the
  // offset codes u, in the order 0, 2, 4, 6, 1, 3, 5, 7).
  auto k_group = [&](const unsigned char* ktile, int r, int grp8) -> uint4 {
    if constexpr (kInt4) {
      const uint32_t w = *reinterpret_cast<const uint32_t*>(
          ktile + k_tile_offset<kRowBytes>(r, grp8 >> 2) + 4 * (grp8 & 3));
      return int4x8_to_bf16x8_offset8(w);
    } else if constexpr (kFp8) {
      const uint2 w = *reinterpret_cast<const uint2*>(
          ktile + k_tile_offset<kRowBytes>(r, grp8 >> 1) + 8 * (grp8 & 1));
      return e4m3x8_to_bf16x8(w);
    } else {
      return *reinterpret_cast<const uint4*>(ktile + k_tile_offset<kRowBytes>(r, grp8));
    }
  };

  auto process_tile = [&](int r0, const VReg* vr, const unsigned char* ktile) {
    if constexpr (kMfmaPv) {
      // K and V are in LDS (staged by stage_tile).  Every LDS read of the
      // tile's K and V is issued first, so their latency overlaps the q.K^T
      // products and the softmax instead of stalling each product in turn.
      // The INT4 row scales are read where they are used: they are few, and
      // holding them from the start would take registers those kernels lack.
      const unsigned char* vtile = ktile + kKTileBytes;
      const int n = lane & 15, grp = lane >> 4;
      // INT4: the tile's row scales (K at [0, kT), times the logit scale; V at
      // [kT, 2 kT))
      const float* sct = reinterpret_cast<const float*>(ktile + 2 * kKTileBytes);
      // K: the 8 elements per k-block of rows 16*tg + n this lane feeds to
      // the MFMA (INT4: the lane's kKBlocks * 4 contiguous bytes, one dword
      // of 8 codes per k-block)
      uint4 kraw[2][kKBlocks];
#pragma unroll
      for (int tg = 0; tg < 2; ++tg) {
        if constexpr (kInt4) {
          constexpr int kLaneBytes = kKBlocks * 4;
          const unsigned char* kp = ktile +
                                    k_tile_offset<kRowBytes>(16 * tg + n, (grp * kLaneBytes) >> 4) +
                                    ((grp * kLaneBytes) & 15);
          if constexpr (kKBlocks == 4) {
            const uint4 t = *reinterpret_cast<const uint4*>(kp);
            kraw[tg][0].x = t.x; kraw[tg][1].x = t.y; kraw[tg][2].x = t.z; kraw[tg][3].x = t.w;
          } else {
            const uint2 t = *reinterpret_cast<const uint2*>(kp);
            kraw[tg][0].x = t.x; kraw[tg][1].x = t.y;
          }
        } else if constexpr (kFp8) {
#pragma unroll
          for (int kb = 0; kb < kKBlocks; ++kb) {
            const uint2 w = *reinterpret_cast<const uint2*>(
                ktile + k_tile_offset<kRowBytes>(16 * tg + n, (4 * kb + grp) >> 1) +
                8 * ((4 * kb + grp) & 1));
            kraw[tg][kb].x = w.x;
            kraw[tg][kb].y = w.y;
          }
        } else {
#pragma unroll
          for (int kb = 0; kb < kKBlocks; ++kb)
            kraw[tg][kb] = *reinterpret_cast<const uint4*>(
                ktile + k_tile_offset<kRowBytes>(16 * tg + n, 4 * kb + grp));
        }
      }
      // V, read column-wise with the transposing LDS reads.
      //   bf16: column block nb of 16 dims; lane 4q+u of the group gets
      //     element e from lane 4e+q, which addresses row 4*grp + e (+16 for
      //     slots 4..7), dims 16*nb + 4q .. +3.
      //   E4M3: column block nb of 16 dims; lane 8q+u of the group gets byte e
      //     from lane 2e+q, which addresses row 16*(e/4) + 4*grp + e%4,
      //     bytes 16*nb + 8q .. +7.
      //   INT4: column block cb of 32 dims; lane 8q+u of the group gets byte e
      //     from lane 2e+q, which addresses row 16*(e/4) + 4*grp + e%4, bytes
      //     16*cb + 8q .. +7; so byte e holds row e's dims 32*cb + 16q + 2u
      //     (low nibble) and + 1 (high nibble): one column of each of two
      //     MFMAs.
      constexpr int kVBlocks = kInt4 ? D / 32 : kNBlocks;
      uint4 vraw[kVBlocks];
#pragma unroll
      for (int nb = 0; nb < kVBlocks; ++nb) {
        if constexpr (kInt4 || kFp8) {
          const int e = n >> 1;
          const int row = 16 * (e >> 2) + 4 * grp + (e & 3);
          const uint2 w = lds_read_tr8(vtile + k_tile_offset<kRowBytes>(row, nb) + 8 * (lane & 1));
          vraw[nb] = make_uint4(w.x, w.y, 0u, 0u);
        } else {
          const int row = 4 * grp + (n >> 2);
          const int c = 2 * nb + ((lane & 3) >> 1);
          const uint2 w0 =
              lds_read_tr16(vtile + k_tile_offset<kRowBytes>(row, c) + 8 * (lane & 1));
          const uint2 w1 =
              lds_read_tr16(vtile + k_tile_offset<kRowBytes>(row + 16, c) + 8 * (lane & 1));
          vraw[nb] = make_uint4(w0.x, w0.y, w1.x, w1.y);
        }
      }
      float4 ksc[2], vsc[2];   // INT4 row scales of this lane's rows, read where used

      // S^T = K q^T: lane l gets the logits of head n for rows 16*tg + 4*grp + r
      // (rows at or past row_end are masked, which only a split's last tile
      // can hold)
      const bool full = r0 + kT <= row_end;
      float x[2][4];
#pragma unroll
      for (int tg = 0; tg < 2; ++tg) {
        // INT4: the products start from -8 sum(q), so the sum comes out as
        // q.(u - 8) = q.u - 8 sum(q)
        f32x4_t sacc = kInt4 ? f32x4_t{-q8[0], -q8[0], -q8[0], -q8[0]} : f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < kKBlocks; ++kb) {
          uint4 kw;
          if constexpr (kInt4)
            kw = int4x8_to_bf16x8_offset8(kraw[tg][kb].x);
          else if constexpr (kFp8)
            kw = e4m3x8_to_bf16x8(make_uint2(kraw[tg][kb].x, kraw[tg][kb].y));
          else
            kw = kraw[tg][kb];
          sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kw), qa[kb], sacc, 0, 0, 0);
        }
        if constexpr (kInt4) {
          // q.(u - 8) times the row's K scale (which carries the logit scale)
          ksc[tg] = *reinterpret_cast<const float4*>(sct + 16 * tg + 4 * grp);
          x[tg][0] = sacc[0] * ksc[tg].x;
          x[tg][1] = sacc[1] * ksc[tg].y;
          x[tg][2] = sacc[2] * ksc[tg].z;
          x[tg][3] = sacc[3] * ksc[tg].w;
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r) x[tg][r] = sacc[r] * c2;
        }
      }
      if (!full) {
#pragma unroll
        for (int tg = 0; tg < 2; ++tg)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (r0 + 16 * tg + 4 * grp + r >= row_end) x[tg][r] = -INFINITY;
      }
      // tile max of head n over the four lanes that hold it (row r0 is always
      // valid, so the max is finite)
      float mt = fmax_prop(fmax_prop(fmax_prop(x[0][0], x[0][1]), x[0][2]),
                           fmax_prop(fmax_prop(x[0][3], x[1][0]), x[1][1]));
      mt = fmax_prop(fmax_prop(mt, x[1][2]), x[1][3]);
      mt = reduce_lane_bits<4, true>(mt);
      // Lazy rescaling: the running max moves only when a tile's max exceeds
      // it by more than kLazyLog2 (base-2 units).  Until then p = exp2(x - m)
      // stays below 2^kLazyLog2, which the fp32 sums and the hi/lo bf16 split
      // of p carry without loss, and the accumulators need no rescaling; the
      // final division and the LSE use the same m, so the result changes only
      // by rounding.  The first tile always moves it (m starts at -inf).
      constexpr float kLazyLog2 = 8.f;
      if (__builtin_amdgcn_ballot_w64(mt > m_lane + kLazyLog2) != 0) {
        const float mn = fmax_prop(m_lane, mt);
        const float alpha = fast_exp2(m_lane - mn);   // 0 on the first tile
        l_sum *= alpha;
        // row r of this lane's accumulators is head 4*grp + r, whose factor
        // the lane with n = 4*grp + r holds (G = 4: heads 0..3 in group 0;
        // rows of heads >= G are padding)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float f = lane_value(alpha, r);
          if constexpr (G >= 8) f = grp == 1 ? lane_value(alpha, 4 + r) : f;
          if constexpr (G >= 16) {
            f = grp == 2 ? lane_value(alpha, 8 + r) : f;
            f = grp == 3 ? lane_value(alpha, 12 + r) : f;
          }
#pragma unroll
          for (int nb = 0; nb < kNBlocks; ++nb) oacc[nb][r] *= f;
          if constexpr (kInt4) osum[r] *= f;
        }
        m_lane = mn;
      }
      // p in the A operand's k-slot order: slot i of lane group grp is row
      // 16*(i/4) + 4*grp + i%4 (the V operand below uses the same order)
      float pv[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) pv[i] = fast_exp2(x[i / 4][i % 4] - m_lane);
      float lsum = pv[0];
#pragma unroll
      for (int i = 1; i < 8; ++i) lsum += pv[i];
      l_sum += lsum;
      if constexpr (kInt4) {
        // p times the row's V scale (rows past the sequence have scale 0 and p 0)
#pragma unroll
        for (int tg = 0; tg < 2; ++tg)
          vsc[tg] = *reinterpret_cast<const float4*>(sct + kT + 16 * tg + 4 * grp);
        pv[0] *= vsc[0].x; pv[1] *= vsc[0].y; pv[2] *= vsc[0].z; pv[3] *= vsc[0].w;
        pv[4] *= vsc[1].x; pv[5] *= vsc[1].y; pv[6] *= vsc[1].z; pv[7] *= vsc[1].w;
      }
      bf16x8_t ph, pl;
      split_bf16x8(pv, ph, pl);
      // ---- p.V on the matrix cores ----
      if constexpr (kInt4) {
        // The offset 8 of the codes comes off at the end through osum, the
        // same products against a column of ones.
#pragma unroll
        for (int cb = 0; cb < D / 32; ++cb) {
          const uint32_t x0 = vraw[cb].x, x1 = vraw[cb].y;
          const uint4 vlo =
              e4m3x8_to_bf16x8(make_uint2(int4_low_offset8(x0), int4_low_offset8(x1)), 512.0f);
          const uint4 vhi =
              e4m3x8_to_bf16x8(make_uint2(int4_high_offset8(x0), int4_high_offset8(x1)), 512.0f);
          oacc[2 * cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ph, as_bf16x8(vlo), oacc[2 * cb], 0, 0, 0);
          oacc[2 * cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pl, as_bf16x8(vlo), oacc[2 * cb], 0, 0, 0);
          oacc[2 * cb + 1] =
              __builtin_amdgcn_mfma_f32_16x16x32_bf16(ph, as_bf16x8(vhi), oacc[2 * cb + 1], 0, 0, 0);
          oacc[2 * cb + 1] =
              __builtin_amdgcn_mfma_f32_16x16x32_bf16(pl, as_bf16x8(vhi), oacc[2 * cb + 1], 0, 0, 0);
        }
        const uint4 one4 = make_uint4(0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u);
        osum = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ph, as_bf16x8(one4), osum, 0, 0, 0);
        osum = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pl, as_bf16x8(one4), osum, 0, 0, 0);
        return;
      }
#pragma unroll
      for (int nb = 0; nb < kNBlocks; ++nb) {
        const uint4 vw =
            kFp8 ? e4m3x8_to_bf16x8(make_uint2(vraw[nb].x, vraw[nb].y)) : vraw[nb];
        oacc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ph, as_bf16x8(vw), oacc[nb], 0, 0, 0);
        oacc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pl, as_bf16x8(vw), oacc[nb], 0, 0, 0);
      }
      return;
    } else {
      // the K loads were issued before the V loads: wait for them only
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(kLoads));
      wave_lds_fence();

      float alpha[G];
      bool grow = false;
      // lane i: row i % kT, part i / kT of D; then add the parts
      const int n = lane % kT, part = lane / kT;
      float x[G];
#pragma unroll
      for (int h = 0; h < G; ++h) x[h] = 0.f;
#pragma unroll
      for (int cc = 0; cc < kPartDims / 8; ++cc) {
        const uint4 kw = k_group(ktile, n, part * (kPartDims / 8) + cc);
        const uint32_t kwv[4] = {kw.x, kw.y, kw.z, kw.w};
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            x[h] = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(qv[h][4 * cc + i]), as_bf16x2(kwv[i]),
                                                   x[h], false);
      }
      const bool ok = r0 + n < row_end;
#pragma unroll
      for (int h = 0; h < G; ++h) {
        x[h] = reduce_lane_bits<log2_int(kT), false>(x[h]);  // add the parts of D
        if constexpr (kInt4) x[h] = (x[h] - q8[h]) * row_ks;  // q.(u - 8), the row's K scale
        x[h] = ok ? x[h] * c2 : -INFINITY;
        const float mt = row_reduce16<true>(x[h]);
        float tile_max = lane_value(mt, 0);
        if constexpr (kT == 32) tile_max = fmax_prop(tile_max, lane_value(mt, 16));
        const float mn = fmax_prop(m_run[h], tile_max);
        grow |= mn > m_run[h];
        alpha[h] = fast_exp2(m_run[h] - mn);
        m_run[h] = mn;
        const float p = fast_exp2(x[h] - mn);
        l_lane[h] = fmaf(l_lane[h], alpha[h], part == 0 ? p : 0.f);
        x[h] = p;
      }
      if (part == 0) {
        // INT4: p times the row's V scale and 2^9 (the V codes convert to
        // n * 2^-9; rows past the sequence have scale 0 and p 0)
#pragma unroll
        for (int h = 0; h < G; ++h) pt[n * G + h] = kInt4 ? x[h] * (row_vs * 512.0f) : x[h];
      }
      wave_lds_fence();

      // ---- p.V on the vector ALUs ----
      if (grow) {
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[h][e] *= alpha[h];
      }
#pragma unroll
      for (int m = 0; m < kLoads; ++m) {
        const int r = kRowsPerLoad * m + row_in_load;
        float ph[G];
#pragma unroll
        for (int h = 0; h < G; ++h) ph[h] = pt[r * G + h];
        float vf[8];
        if constexpr (kInt4) {
          int4x8_to_f32_scaled(vr[m], vf);
        } else if constexpr (kFp8) {
          e4m3x8_to_f32(vr[m], vf);
        } else {
          const uint32_t vw[4] = {vr[m].x, vr[m].y, vr[m].z, vr[m].w};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            vf[2 * i] = bf16_lo(vw[i]);
            vf[2 * i + 1] = bf16_hi(vw[i]);
          }
        }
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[h][e] = fmaf(ph[h], vf[e], acc[h][e]);
      }
    }
  };

  // Split s streams rows [s * chunk, min((s + 1) * chunk, L)); wave w takes
  // the tiles starting at w * kT, w * kT + kWaves * kT, ...
  const int stride = kWaves * kT;
  const int row_lo = s * a.chunk;
  row_end = min(row_lo + a.chunk, L);
  int r0 = row_lo + wave * kT;
  VReg vr[kLoads];
  TileRegs tr;
  int tile_k = 0;   // paged cache: index of the wave's tile at r0
  // debug build: the wave's tile region and statistics slots start as NaN
  poison_wave_lds<kWaveBytes>(kt, lane);
  if constexpr (DAS_DEBUG_LDS_POISON) {
    if (lane < 2 * G) wst_ml[wave * 2 * G + lane] = __builtin_nanf("");
  }
  if (r0 < row_end) {
    const int page = kPaged ? page_for(0) : 0;
    if constexpr (kMfmaPv)
      fetch_tile(r0, tr, page);
    else
      load_tile(r0, vr, kt, page);
  }

  // The query operand, from the rows loaded at the start (issued before the
  // tile, so waiting for them leaves the tile in flight).
  auto bf16x8_sum = [](uint4 w) {
    return ((bf16_lo(w.x) + bf16_hi(w.x)) + (bf16_lo(w.y) + bf16_hi(w.y))) +
           ((bf16_lo(w.z) + bf16_hi(w.z)) + (bf16_lo(w.w) + bf16_hi(w.w)));
  };
  if constexpr (G >= 4) {
    float qs = 0.f;
#pragma unroll
    for (int kb = 0; kb < kKBlocks; ++kb) {
      uint4 w = qraw[kb];
      if constexpr (kInt4) {
        qs += bf16x8_sum(w);
        w = bf16x8_even_odd(w);
      }
      qa[kb] = as_bf16x8(w);
    }
    if constexpr (kInt4) q8[0] = 8.f * reduce_lane_bits<4, false>(qs);
  } else {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float qs = 0.f;
#pragma unroll
      for (int i = 0; i < kPartDims / 8; ++i) {
        uint4 w = qraw[h * (kPartDims / 8) + i];
        if constexpr (kInt4) {
          qs += bf16x8_sum(w);
          w = bf16x8_even_odd(w);
        }
        qv[h][4 * i + 0] = w.x;
        qv[h][4 * i + 1] = w.y;
        qv[h][4 * i + 2] = w.z;
        qv[h][4 * i + 3] = w.w;
      }
      if constexpr (kInt4) q8[h] = 8.f * reduce_lane_bits<log2_int(kT), false>(qs);
    }
  }

  // Stream.  G >= 4: stage the fetched tile, fetch the wave's next one,
  // process the staged one.  G <= 2: process the tile in flight, then issue
  // the next one.
  if constexpr (kMfmaPv) {
    for (; r0 < row_end; r0 += stride, ++tile_k) {
      stage_tile(tr, kt);
      const int rn = r0 + stride;
      if (rn < row_end) fetch_tile(rn, tr, kPaged ? page_for(tile_k + 1) : 0);
      process_tile(r0, vr, kt);
      poison_wave_lds<kWaveBytes>(kt, lane);   // debug build: the tile is dead
    }
  } else {
    for (; r0 < row_end; r0 += stride, ++tile_k) {
      process_tile(r0, vr, kt);
      poison_wave_lds<kWaveBytes>(kt, lane);   // debug build: the tile is dead
      const int rn = r0 + stride;
      if (rn < row_end) load_tile(rn, vr, kt, kPaged ? page_for(tile_k + 1) : 0);
    }
  }

  // ---- end of the stream: each wave's state into its own tile region ----
  // The wave's tiles are no longer needed, and no other wave touches them:
  // the state goes there without waiting for the others.  Layout [row
  // group][head][D] floats; max and sum per head in wst_ml.
  float* wst = reinterpret_cast<float*>(kt);
  if constexpr (kMfmaPv) {
    l_sum = reduce_lane_bits<4, false>(l_sum);  // lane n: head n's sum over the wave's rows
    if (lane < 4 * G) {                          // lane groups holding real heads
      if constexpr (kInt4) {
        // p.(u - 8) = p.u - 8 sum(p)
        const int d0 = 16 * ((lane & 15) >> 3) + 2 * (lane & 7);
#pragma unroll
        for (int nb = 0; nb < kNBlocks; ++nb)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            wst[(4 * (lane >> 4) + r) * D + 32 * (nb >> 1) + d0 + (nb & 1)] =
                oacc[nb][r] - 8.f * osum[r];
      } else {
#pragma unroll
        for (int nb = 0; nb < kNBlocks; ++nb)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            wst[(4 * (lane >> 4) + r) * D + 16 * nb + (lane & 15)] = oacc[nb][r];
      }
    }
    if (lane < G) {
      wst_ml[wave * 2 * G + lane] = m_lane;
      wst_ml[wave * 2 * G + G + lane] = l_sum;
    }
  } else {
    // acc: lanes lane and lane ^ 2^k for the row-group bits above kKeptGroups
    // are summed; the lanes whose top bits are zero then hold row group
    // rg = lane / kLanesPerRow.
    constexpr int kKeepBit = log2_int(kKeptGroups * kLanesPerRow);   // lowest lane bit summed
    if constexpr (kKeepBit < 6) {
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] = reduce_lane_bits<kKeepBit, false>(acc[h][e]);
    }
    float l_tot[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float t = row_reduce16<false>(l_lane[h]);
      l_tot[h] = lane_value(t, 0) + (kT == 32 ? lane_value(t, 16) : 0.f);
    }
    if (lane < kKeptGroups * kLanesPerRow) {
      const int rg = lane / kLanesPerRow;
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float* dst = wst + (rg * G + h) * D + 8 * chunk;
        *reinterpret_cast<float4*>(dst) = make_float4(acc[h][0], acc[h][1], acc[h][2], acc[h][3]);
        *reinterpret_cast<float4*>(dst + 4) =
            make_float4(acc[h][4], acc[h][5], acc[h][6], acc[h][7]);
      }
    }
    if (lane == 0) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        wst_ml[wave * 2 * G + h] = m_run[h];
        wst_ml[wave * 2 * G + G + h] = l_tot[h];
      }
    }
  }
  __syncthreads();

  // ---- merge the waves: one thread per (row group, head, float4 quad) ----
  // lane = rg * kPairLanes + x, pair (head, quad) = wave * kPairLanes + x, so
  // the row groups of a pair are lanes of one wave and add up with swaps.
  // A sequence that uses at most one split is finished by split 0's
  // workgroup; so is every sequence of a single-split plan.
  const bool finish_here = a.direct || (a.fused && nsb <= 1);
  constexpr int kQuads = D / 4;                 // float4 quads per output row
  constexpr int kPairs = G * kQuads;
  constexpr int kPairLanes = 64 / kKeptGroups;
  constexpr int kMergeWaves = kPairs / kPairLanes;
  static_assert(kPairs % kPairLanes == 0 && kMergeWaves <= kWaves, "whole waves merge");
  // Partials of this (b, kv-head): rows (head, split) of D floats, and
  // (max, sum) pairs.  Offsets stay far below 4 GiB within one kv-head.
  const size_t qh0 = (size_t)b * a.Hq + (size_t)g * G;   // first query head of the group
  const __amdgpu_buffer_rsrc_t ro =
      make_rsrc(a.ws_o + (a.direct ? 0 : qh0 * a.ns * D), G * a.ns * D * 4);
  const __amdgpu_buffer_rsrc_t rml =
      make_rsrc(a.ws_ml + (a.direct ? 0 : qh0 * a.ns * 2), G * a.ns * 2 * 4);
  if (wave < kMergeWaves) {
    const int rg = lane / kPairLanes, x = lane % kPairLanes;
    const int pair = wave * kPairLanes + x;
    const int h = pair / kQuads, quad = pair % kQuads;
    // every wave's state is read before any of it is used, so the LDS
    // reads overlap instead of taking one round trip per wave
    float mw[kWaves], lw[kWaves];
    float4 uw[kWaves];
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      mw[w] = wst_ml[w * 2 * G + h];
      lw[w] = wst_ml[w * 2 * G + G + h];
      uw[w] = *reinterpret_cast<const float4*>(
          reinterpret_cast<const float*>(smem + w * kWaveBytes) + (rg * G + h) * D + 4 * quad);
    }
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, mw[w]);
    // a wave that saw no row (max -inf) weighs 0; so does every wave when M = -inf
    float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
    float lsum = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float f = (mw[w] == -INFINITY) ? 0.f : fast_exp2(mw[w] - M);
      o.x = fmaf(f, uw[w].x, o.x);
      o.y = fmaf(f, uw[w].y, o.y);
      o.z = fmaf(f, uw[w].z, o.z);
      o.w = fmaf(f, uw[w].w, o.w);
      lsum = fmaf(f, lw[w], lsum);
    }
    // add the row groups (M and lsum are the same in all of them)
    constexpr int kGroupBit = log2_int(kPairLanes);
    if constexpr (kGroupBit < 6) {
      o.x = reduce_lane_bits<kGroupBit, false>(o.x);
      o.y = reduce_lane_bits<kGroupBit, false>(o.y);
      o.z = reduce_lane_bits<kGroupBit, false>(o.z);
      o.w = reduce_lane_bits<kGroupBit, false>(o.w);
    }
    if constexpr (kFp8) {
      o.x *= v_scale; o.y *= v_scale; o.z *= v_scale; o.w *= v_scale;
    }
    if (rg == 0) {
      const size_t qh = qh0 + h;
      if (finish_here) {
        const float inv = (M == -INFINITY) ? 0.f : 1.f / lsum;
        store_out4(a, qh * D + 4 * quad, o.x * inv, o.y * inv, o.z * inv, o.w * inv);
        if (quad == 0 && a.lse != nullptr)
          a.lse[qh] = (M == -INFINITY) ? -INFINITY : (M + __log2f(lsum)) * kLn2;
      } else {
        // device-coherent stores (sc1): the merging workgroup may run on another XCD
        const int row = h * a.ns + s;
        coherent_store16(ro, (row * D + 4 * quad) * 4, o);
        if (quad == 0) coherent_store8(rml, row * 8, M, lsum);
      }
    }
  }
  if (!a.fused || finish_here) return;

  // ---- fused phase 2: the last workgroup of this (b, kv-head) to arrive
  // merges every split's partial (FlashDecoding++ post, §3 phase 2) ----
  __shared__ int s_last;
  // This workgroup's partial stores must be complete before it is counted:
  // a store becomes visible to another XCD only about when its
  // acknowledgement arrives, so waiting for it here costs no more than the
  // merging workgroup would otherwise spend waiting for the data.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (tid == 0) {
    unsigned int* cnt = a.counters + counter_slot(b * a.Hkv + g);
    const unsigned int prev = atomicAdd(cnt, 1u);
    const bool last = prev == (unsigned int)(nsb - 1);
    if (last) atomicExch(cnt, 0u);  // leave the counter at zero for the next call
    // A count of nsb or more is impossible in a workspace whose counters
    // started at zero: the caller broke that precondition.  Fail loudly.
    s_last = last ? 1 : (prev >= (unsigned int)nsb ? 2 : 0);
  }
  __syncthreads();
  if (s_last == 2) {
    // NaN outputs (and LSE) for this (b, kv-head), instead of stale ones
    for (int i = tid; i < G * D / 4; i += kThreads) {
      const float nan = __builtin_nanf("");
      store_out4(a, qh0 * D + 4 * i, nan, nan, nan, nan);
    }
    if (tid < G && a.lse != nullptr) a.lse[qh0 + tid] = __builtin_nanf("");
    return;
  }
  if (!s_last) return;

  // One thread per (split group, head, float4 quad): lane = grp * kGroupLanes
  // + x, pair = wave * kGroupLanes + x.  Group grp takes splits grp,
  // grp + kGroups, ...; the groups of a pair are lanes of one wave, so they
  // combine with swaps, in a fixed order whichever workgroup merges.
  constexpr int kGroups = kThreads / kPairs < 4 ? kThreads / kPairs : 4;
  constexpr int kGroupLanes = 64 / kGroups;
  constexpr int kFinalWaves = kPairs / kGroupLanes;
  static_assert(kGroups >= 1 && kPairs % kGroupLanes == 0 && kFinalWaves <= kWaves,
                "whole waves merge the splits");
  if (wave >= kFinalWaves) return;
  const int grp = lane / kGroupLanes, x = lane % kGroupLanes;
  const int pair = wave * kGroupLanes + x;
  const int h = pair / kQuads, quad = pair % kQuads;
  // This thread's splits, merged online: batches of 8 loaded in one round
  // trip, the running sums rescaled when a batch raises the running max.
  // The loads are bound by the CU's address rate, so each 16-lane row (one
  // head, one split group: kGroupLanes is 16 or 32 and divides kQuads) loads
  // the batch's (max, sum) pairs once, lane x the pair of split x % 8, and
  // hands them round with row broadcasts.  (kGroupLanes and kQuads are
  // multiples of 16, so no row spans two heads or two split groups.)
  static_assert(kGroupLanes % 16 == 0 && kQuads % 16 == 0, "one head per row");
  float mt = -INFINITY;
  float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
  float ls = 0.f;
  constexpr int kBatch = 8;
  for (int c0 = grp; c0 < nsb; c0 += kBatch * kGroups) {
    float2 st[kBatch];
    float4 u[kBatch];
    const int cm = c0 + (lane & 7) * kGroups;
    const float2 mine =
        cm < nsb ? coherent_load8(rml, (h * a.ns + cm) * 8) : make_float2(-INFINITY, 0.f);
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const int c = c0 + k * kGroups;
      u[k] = c < nsb ? coherent_load16(ro, ((h * a.ns + c) * D + 4 * quad) * 4)
                     : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    row_broadcast8(mine, st);
    float bm = st[0].x;
#pragma unroll
    for (int k = 1; k < kBatch; ++k) bm = fmaxf(bm, st[k].x);
    const float mn = fmaxf(mt, bm);  // finite: split c0 < nsb is in the batch
    const float alpha = fast_exp2(mt - mn);
    o.x *= alpha; o.y *= alpha; o.z *= alpha; o.w *= alpha;
    ls *= alpha;
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const float w = fast_exp2(st[k].x - mn);  // 0 for the padding slots
      o.x = fmaf(w, u[k].x, o.x);
      o.y = fmaf(w, u[k].y, o.y);
      o.z = fmaf(w, u[k].z, o.z);
      o.w = fmaf(w, u[k].w, o.w);
      ls = fmaf(w, st[k].y, ls);
    }
    mt = mn;
  }
  // combine the groups: global max, rescale, sum (a group without splits
  // has max -inf and weighs 0)
  constexpr int kGroupBit = log2_int(kGroupLanes);
  float M = mt;
  if constexpr (kGroupBit < 6) M = reduce_lane_bits<kGroupBit, true>(mt);
  const float f = (mt == -INFINITY) ? 0.f : fast_exp2(mt - M);
  o.x *= f; o.y *= f; o.z *= f; o.w *= f;
  ls *= f;
  if constexpr (kGroupBit < 6) {
    o.x = reduce_lane_bits<kGroupBit, false>(o.x);
    o.y = reduce_lane_bits<kGroupBit, false>(o.y);
    o.z = reduce_lane_bits<kGroupBit, false>(o.z);
    o.w = reduce_lane_bits<kGroupBit, false>(o.w);
    ls = reduce_lane_bits<kGroupBit, false>(ls);
  }
  if (grp == 0) {
    const size_t qh = qh0 + h;
    const float inv = 1.f / ls;
    store_out4(a, qh * D + 4 * quad, o.x * inv, o.y * inv, o.z * inv, o.w * inv);
    if (quad == 0 && a.lse != nullptr) a.lse[qh] = (M + __log2f(ls)) * kLn2;
  }
}

// ---------------------------------------------------------------------------
// Phase 2: lse_combine.  One wave per (batch row, query head): 4 waves per
// workgroup, 256 threads.
// ---------------------------------------------------------------------------
constexpr int kCombineThreads = 256;
constexpr int kCombineRows = kCombineThreads / 64;   // (b, h) rows per workgroup

// Each lane owns the float4 quad lane % (D/4) of the output row; the wave's
// 64 / (D/4) lane groups take the splits grp, grp + groups, ... and merge
// them online, loading kCombineBatch splits per round trip (statistics and
// partial rows together).  The groups then combine with row swaps (global
// max, rescale, sum), in a fixed order: no LDS and no barrier.
constexpr int kCombineBatch = 4;

template <int D>
__global__ __launch_bounds__(kCombineThreads) void lse_combine_kernel(CombineArgs a, int rows) {
  constexpr int kQuads = D / 4;
  constexpr int kGroups = 64 / kQuads;                 // 2 (D = 128) or 4 (D = 64)
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * kCombineRows + (threadIdx.x >> 6);   // b * Hq + h
  if (row >= rows) return;
  const int quad = lane % kQuads, grp = lane / kQuads;
  // Every slot of the plan is read: phase 1 wrote each split's partial, and
  // marked the splits its sequence does not reach empty (max -inf, sum 0);
  // their partial rows were never written and are not used.
  const int nsb = a.ns;
  const size_t qh = (size_t)row;
  const float2* ml = reinterpret_cast<const float2*>(a.ws_ml + qh * a.ns * 2);
  const float4* po = reinterpret_cast<const float4*>(a.ws_o + qh * a.ns * D) + quad;

  float mt = -INFINITY, ls = 0.f;
  float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int c0 = grp; c0 < nsb; c0 += kCombineBatch * kGroups) {
    float2 st[kCombineBatch];
    float4 pr[kCombineBatch];
#pragma unroll
    for (int k = 0; k < kCombineBatch; ++k) {
      const int c = c0 + k * kGroups;
      st[k] = c < nsb ? ml[c] : make_float2(-INFINITY, 0.f);
      pr[k] = c < nsb ? po[(size_t)c * kQuads] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    float bm = st[0].x;
#pragma unroll
    for (int k = 1; k < kCombineBatch; ++k) bm = fmaxf(bm, st[k].x);
    if (bm == -INFINITY) continue;   // only empty splits in this batch
    const float mn = fmaxf(mt, bm);
    const float alpha = fast_exp2(mt - mn);   // 0 while nothing has been merged
    o.x *= alpha; o.y *= alpha; o.z *= alpha; o.w *= alpha;
    ls *= alpha;
#pragma unroll
    for (int k = 0; k < kCombineBatch; ++k) {
      if (st[k].x == -INFINITY) continue;   // an empty split: its row was never written
      const float w = fast_exp2(st[k].x - mn);
      o.x = fmaf(w, pr[k].x, o.x);
      o.y = fmaf(w, pr[k].y, o.y);
      o.z = fmaf(w, pr[k].z, o.z);
      o.w = fmaf(w, pr[k].w, o.w);
      ls = fmaf(w, st[k].y, ls);
    }
    mt = mn;
  }
  // combine the groups (a group without splits has max -inf and weighs 0)
  constexpr int kGroupBit = log2_int(kQuads);
  const float M = reduce_lane_bits<kGroupBit, true>(mt);
  const float f = (mt == -INFINITY) ? 0.f : fast_exp2(mt - M);
  o.x = reduce_lane_bits<kGroupBit, false>(o.x * f);
  o.y = reduce_lane_bits<kGroupBit, false>(o.y * f);
  o.z = reduce_lane_bits<kGroupBit, false>(o.z * f);
  o.w = reduce_lane_bits<kGroupBit, false>(o.w * f);
  ls = reduce_lane_bits<kGroupBit, false>(ls * f);
  if (grp == 0) {
    const float inv = (M == -INFINITY) ? 0.f : 1.f / ls;   // an empty sequence: out = 0
    const size_t e = qh * D + 4 * quad;
    if (a.out_bf16) {
      uint16_t* op = reinterpret_cast<uint16_t*>(a.out) + e;
      const uint32_t lo = f32_to_bf16_rne(o.x * inv) | ((uint32_t)f32_to_bf16_rne(o.y * inv) << 16);
      const uint32_t hi = f32_to_bf16_rne(o.z * inv) | ((uint32_t)f32_to_bf16_rne(o.w * inv) << 16);
      *reinterpret_cast<uint2*>(op) = make_uint2(lo, hi);
    } else {
      *reinterpret_cast<float4*>(reinterpret_cast<float*>(a.out) + e) =
          make_float4(o.x * inv, o.y * inv, o.z * inv, o.w * inv);
    }
    if (quad == 0 && a.lse != nullptr)
      a.lse[qh] = (M == -INFINITY) ? -INFINITY : (M + __log2f(ls)) * kLn2;
  }
}

// ---------------------------------------------------------------------------
// merge_attn_states ([SGL-PAR] "Constraints": the LSE merge of two partial
// attention states).  Each lane handles four consecutive elements of a row
// (16-byte f32 or 8-byte bf16 accesses), D/4 lanes per row, so a row lies
// within one wave: every lane of the row has read its two LSE values before
// one lane may overwrite one of them in place, and every element is read
// and written by the same lane.  A grid-stride loop over groups of rows.
// ---------------------------------------------------------------------------
constexpr int kMergeThreads = 256;
#ifndef DAS_MERGE_UNROLL
#define DAS_MERGE_UNROLL 4
#endif
constexpr int kMergeUnroll = DAS_MERGE_UNROLL;

template <int D>
constexpr int merge_rows_per_block() { return kMergeThreads / (D / 4); }

template <int D, bool kBf16>
__global__ __launch_bounds__(kMergeThreads) void merge_attn_states_kernel(MergeArgs a) {
  // No contraction into FMAs: wa*oa and wb*ob must round the same way so that
  // swapping the two states gives bitwise the same result.
#pragma clang fp contract(off)
  constexpr int kLanesPerRow = D / 4;
  constexpr int kRows = merge_rows_per_block<D>();
  // Rows per lane per pass: all their loads are issued before any store (a
  // store may alias a later row's input, so the compiler cannot hoist loads
  // past it), which keeps kUnroll rows of each lane in flight.
  constexpr int kUnroll = kMergeUnroll;
  const int sub = threadIdx.x / kLanesPerRow;        // row within a group of kRows
  const int c = (threadIdx.x % kLanesPerRow) * 4;    // first element of this lane
  const int64_t step = (int64_t)gridDim.x * kRows * kUnroll;
  for (int64_t row0 = (int64_t)blockIdx.x * kRows * kUnroll + sub; row0 < a.rows; row0 += step) {
    float la[kUnroll], lb[kUnroll], oa[kUnroll][4], ob[kUnroll][4];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t row = row0 + (int64_t)u * kRows;
      if (row >= a.rows) break;
      la[u] = a.lse_a[row];
      lb[u] = a.lse_b[row];
      const size_t base = (size_t)row * D + c;
      // non-temporal loads and stores: the states stream through once
      if constexpr (kBf16) {
        const u32x2_t ua = __builtin_nontemporal_load(
            reinterpret_cast<const u32x2_t*>(reinterpret_cast<const uint16_t*>(a.o_a) + base));
        const u32x2_t ub = __builtin_nontemporal_load(
            reinterpret_cast<const u32x2_t*>(reinterpret_cast<const uint16_t*>(a.o_b) + base));
        oa[u][0] = bf16_lo(ua[0]); oa[u][1] = bf16_hi(ua[0]); oa[u][2] = bf16_lo(ua[1]); oa[u][3] = bf16_hi(ua[1]);
        ob[u][0] = bf16_lo(ub[0]); ob[u][1] = bf16_hi(ub[0]); ob[u][2] = bf16_lo(ub[1]); ob[u][3] = bf16_hi(ub[1]);
      } else {
        const f32x4_t fa = __builtin_nontemporal_load(
            reinterpret_cast<const f32x4_t*>(reinterpret_cast<const float*>(a.o_a) + base));
        const f32x4_t fb = __builtin_nontemporal_load(
            reinterpret_cast<const f32x4_t*>(reinterpret_cast<const float*>(a.o_b) + base));
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          oa[u][i] = fa[i];
          ob[u][i] = fb[i];
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t row = row0 + (int64_t)u * kRows;
      if (row >= a.rows) break;
      const float mx = fmaxf(la[u], lb[u]);
      float wa = 0.f, wb = 0.f, lse = -INFINITY;
      if (mx != -INFINITY) {
        lse = mx + logf(expf(la[u] - mx) + expf(lb[u] - mx));
        wa = expf(la[u] - lse);
        wb = expf(lb[u] - lse);
      }
      float v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        // products rounded separately so that swapping a and b is bitwise symmetric
        const float ta = wa * oa[u][i];
        const float tb = wb * ob[u][i];
        v[i] = (mx == -INFINITY) ? 0.f : ta + tb;
      }
      const size_t base = (size_t)row * D + c;
      if constexpr (kBf16) {
        const u32x2_t w = {f32_to_bf16_rne(v[0]) | ((uint32_t)f32_to_bf16_rne(v[1]) << 16),
                           f32_to_bf16_rne(v[2]) | ((uint32_t)f32_to_bf16_rne(v[3]) << 16)};
        __builtin_nontemporal_store(
            w, reinterpret_cast<u32x2_t*>(reinterpret_cast<uint16_t*>(a.o_out) + base));
      } else {
        const f32x4_t w = {v[0], v[1], v[2], v[3]};
        __builtin_nontemporal_store(
            w, reinterpret_cast<f32x4_t*>(reinterpret_cast<float*>(a.o_out) + base));
      }
      if (c == 0) a.lse_out[row] = lse;
    }
  }
}

}  // namespace

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
template <int D, int G, int kKv, bool kPaged>
static hipError_t launch_split(int B, const SplitArgs& a, bool one_per_cu, hipStream_t st) {
  // Dynamic LDS that brings the workgroup's total to kOnePerCuLds, more than
  // half a CU's LDS, so no second workgroup fits on the CU and the streaming
  // workgroups spread over all CUs instead of doubling up on some.  The
  // static part already counts toward the total.
  constexpr int kStatic = split_smem_bytes<D, G, kKv>() + kWaves * 2 * G * 4 + 64;
  static_assert(kStatic + 0 <= kMaxLdsPerWorkgroup, "static LDS over the limit");
  constexpr int kPad = kStatic < kOnePerCuLds ? kOnePerCuLds - kStatic : 0;
  static_assert(kStatic + kPad <= kMaxLdsPerWorkgroup, "padded LDS over the limit");
  // The compiled kernel's own static LDS, read once: the pad is dropped (a
  // pure placement hint) if static + pad would not fit in a workgroup.
  static const int static_lds = [] {
    hipFuncAttributes fa;
    if (hipFuncGetAttributes(&fa, reinterpret_cast<const void*>(
                                      &split_kv_decode_kernel<D, G, kKv, kPaged>)) != hipSuccess)
      return -1;
    return (int)fa.sharedSizeBytes;
  }();
  const bool pad_fits = static_lds >= 0 && static_lds + kPad <= kMaxLdsPerWorkgroup;
  dim3 grid((unsigned)(a.ns | 1), (unsigned)a.Hkv, (unsigned)B);
  hipLaunchKernelGGL((split_kv_decode_kernel<D, G, kKv, kPaged>), grid, dim3(kThreads),
                     (unsigned)(one_per_cu && pad_fits ? kPad : 0), st, a);
  return hipGetLastError();
}

template <int kKv, bool kPaged>
static hipError_t launch_split_typed(int D, int G, int B, const SplitArgs& a, bool one_per_cu,
                                     hipStream_t st) {
  if (D == 128) {
    switch (G) {
      case 1: return launch_split<128, 1, kKv, kPaged>(B, a, one_per_cu, st);
      case 2: return launch_split<128, 2, kKv, kPaged>(B, a, one_per_cu, st);
      case 4: return launch_split<128, 4, kKv, kPaged>(B, a, one_per_cu, st);
      case 8: return launch_split<128, 8, kKv, kPaged>(B, a, one_per_cu, st);
      case 16: return launch_split<128, 16, kKv, kPaged>(B, a, one_per_cu, st);
    }
  } else if (D == 64) {
    switch (G) {
      case 1: return launch_split<64, 1, kKv, kPaged>(B, a, one_per_cu, st);
      case 2: return launch_split<64, 2, kKv, kPaged>(B, a, one_per_cu, st);
      case 4: return launch_split<64, 4, kKv, kPaged>(B, a, one_per_cu, st);
      case 8: return launch_split<64, 8, kKv, kPaged>(B, a, one_per_cu, st);
      case 16: return launch_split<64, 16, kKv, kPaged>(B, a, one_per_cu, st);
    }
  }
  return hipErrorInvalidValue;
}

hipError_t launch_split_kv_decode(int D, int G, int kv_format, bool paged, int B,
                                  const SplitArgs& a, bool one_per_cu, hipStream_t st) {
  switch (kv_format) {
    case kKvBf16:
      return paged ? launch_split_typed<kKvBf16, true>(D, G, B, a, one_per_cu, st)
                   : launch_split_typed<kKvBf16, false>(D, G, B, a, one_per_cu, st);
    case kKvE4m3:
      return paged ? launch_split_typed<kKvE4m3, true>(D, G, B, a, one_per_cu, st)
                   : launch_split_typed<kKvE4m3, false>(D, G, B, a, one_per_cu, st);
    case kKvInt4:
      return paged ? launch_split_typed<kKvInt4, true>(D, G, B, a, one_per_cu, st)
                   : launch_split_typed<kKvInt4, false>(D, G, B, a, one_per_cu, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_lse_combine(int D, int B, const CombineArgs& a, hipStream_t st) {
  const int64_t rows64 = (int64_t)B * a.Hq;
  if (rows64 > INT32_MAX) return hipErrorInvalidValue;
  const int rows = (int)rows64;
  dim3 grid((unsigned)((rows + kCombineRows - 1) / kCombineRows));
  if (D == 128)
    hipLaunchKernelGGL(lse_combine_kernel<128>, grid, dim3(kCombineThreads), 0, st, a, rows);
  else if (D == 64)
    hipLaunchKernelGGL(lse_combine_kernel<64>, grid, dim3(kCombineThreads), 0, st, a, rows);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_merge_attn_states(int D, const MergeArgs& a, hipStream_t st) {
  if (a.rows <= 0) return hipSuccess;
  if (D != 64 && D != 128) return hipErrorInvalidValue;
  // One pass per block up to 65536 blocks (2M rows of D = 128): a block per
  // group of rows measured faster than fewer blocks looping (1M rows: 285 us
  // against 302 us with 2048 blocks); larger calls loop.
  constexpr int64_t kMaxBlocks = 65536;
  const int64_t rows_per_block =
      (D == 128 ? merge_rows_per_block<128>() : merge_rows_per_block<64>()) * kMergeUnroll;
  const dim3 grid((unsigned)std::min<int64_t>((a.rows + rows_per_block - 1) / rows_per_block,
                                              kMaxBlocks));
  const dim3 block(kMergeThreads);
  if (D == 128 && a.bf16)
    hipLaunchKernelGGL((merge_attn_states_kernel<128, true>), grid, block, 0, st, a);
  else if (D == 128)
    hipLaunchKernelGGL((merge_attn_states_kernel<128, false>), grid, block, 0, st, a);
  else if (a.bf16)
    hipLaunchKernelGGL((merge_attn_states_kernel<64, true>), grid, block, 0, st, a);
  else
    hipLaunchKernelGGL((merge_attn_states_kernel<64, false>), grid, block, 0, st, a);
  return hipGetLastError();
}

}  // namespace das
