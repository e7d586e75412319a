// Device-side building blocks shared by the gfx950 kernels of the drafting step.
//
// Storage types: bf16 (bit patterns in uint16_t) or fp32.  GEMM operands are fed
// to the CDNA4 matrix cores as "fragments": 8 consecutive K elements per lane.
// A 64-lane wave therefore covers 4 lane groups x 8 = 32 K elements per
// fragment.  For bf16 one fragment is one v_mfma_f32_16x16x32_bf16; for fp32 it
// is eight v_mfma_f32_16x16x4_f32, fragment element j of lane group g being the
// K slot g of the j-th instruction.  Both A and B operands use the same
// (group, element) -> K mapping, so any consistent assignment of K indices to
// (group, element) gives the same contraction.
//
// Output layout of a 16x16 MFMA tile: lane l holds rows 4*(l/16)+i (i=0..3) of
// column l%16.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cmath>

namespace dflash {

typedef uint16_t bf16_t;
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x8_t __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x16_t __attribute__((ext_vector_type(16)));

// ------------------------------------------------------------------ conversions

__device__ __forceinline__ float bf2f(bf16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// float -> bf16, round to nearest, ties to even, by the gfx950 conversion instruction
// (v_cvt_pk_bf16_f32; NaN stays NaN).  Two values per instruction: pk_bf16 packs a
// (low half) and b (high half).
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pk_bf16(float a, float b) {
  const f32x2_t f = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}
__device__ __forceinline__ bf16_t f2bf(float f) { return __builtin_bit_cast(bf16_t, static_cast<__bf16>(f)); }

// maximum over lanes l, l^16, l^32 and l^48 (the four lane groups of a column of a 16x16
// matrix-core tile), by the gfx950 row-swap instructions instead of LDS permutes
__device__ __forceinline__ float max_lane_groups(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float m = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

template <typename T> __device__ __forceinline__ float to_f(T v);
template <> __device__ __forceinline__ float to_f<float>(float v) { return v; }
template <> __device__ __forceinline__ float to_f<bf16_t>(bf16_t v) { return bf2f(v); }

template <typename T> __device__ __forceinline__ T from_f(float v);
template <> __device__ __forceinline__ float from_f<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16_t from_f<bf16_t>(float v) { return f2bf(v); }

// round-trip through the storage type (identity for fp32)
template <typename T> __device__ __forceinline__ float round_to(float v) { return to_f<T>(from_f<T>(v)); }

// ------------------------------------------------------------------ buffer resources

// Raw buffer descriptor over [p, p + bytes): loads at offsets >= bytes return zero.
// Word 3 = 0x00020000 is the gfx9-family raw (untyped, unswizzled) buffer format.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, static_cast<int>(bytes), 0x00020000);
}

// ------------------------------------------------------------------ direct global -> LDS loads

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) void*)p));
}

// 16 bytes per lane from global address g into LDS at (wave-uniform) byte address lds + 16 * lane.
// Issued as an instruction the compiler does not track: it adds no waits of its own for these
// loads, so the caller waits (vmcnt) before reading what they wrote.
__device__ __forceinline__ void dma16(const void* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "s"(lds) : "memory", "m0");
}

// ------------------------------------------------------------------ fragments

template <typename T> struct Frag;

template <> struct Frag<bf16_t> {
  typedef bf16x8_t type;
  __device__ __forceinline__ static type zero() {
    u32x4_t z = {0u, 0u, 0u, 0u};
    return __builtin_bit_cast(type, z);
  }
  __device__ __forceinline__ static type load(const bf16_t* p) {
    return __builtin_bit_cast(type, *reinterpret_cast<const u32x4_t*>(p));
  }
  // 8 elements at byte offset voff + soff of a buffer
  __device__ __forceinline__ static type load_buf(__amdgpu_buffer_rsrc_t r, uint32_t voff, int soff) {
    return __builtin_bit_cast(type, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
  }
  // load 8 floats and round them to bf16
  __device__ __forceinline__ static type load_f32(const float* p) {
    const f32x4_t a = *reinterpret_cast<const f32x4_t*>(p);
    const f32x4_t b = *reinterpret_cast<const f32x4_t*>(p + 4);
    const u32x4_t r = {pk_bf16(a[0], a[1]), pk_bf16(a[2], a[3]), pk_bf16(b[0], b[1]), pk_bf16(b[2], b[3])};
    return __builtin_bit_cast(type, r);
  }
  __device__ __forceinline__ static type from_floats(const float* v) {
    const u32x4_t r = {pk_bf16(v[0], v[1]), pk_bf16(v[2], v[3]), pk_bf16(v[4], v[5]), pk_bf16(v[6], v[7])};
    return __builtin_bit_cast(type, r);
  }
  __device__ __forceinline__ static f32x4_t mma(f32x4_t acc, type a, type b) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
  }
  // zero element j (0..7) when !keep
  __device__ __forceinline__ static type mask(type v, uint32_t keep_bits) {
    u32x4_t r = __builtin_bit_cast(u32x4_t, v);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t m = ((keep_bits >> (2 * j)) & 1u ? 0x0000ffffu : 0u) | ((keep_bits >> (2 * j + 1)) & 1u ? 0xffff0000u : 0u);
      r[j] &= m;
    }
    return __builtin_bit_cast(type, r);
  }
};

template <> struct Frag<float> {
  typedef f32x8_t type;
  __device__ __forceinline__ static type zero() {
    type z = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    return z;
  }
  __device__ __forceinline__ static type load(const float* p) {
    const f32x4_t a = *reinterpret_cast<const f32x4_t*>(p);
    const f32x4_t b = *reinterpret_cast<const f32x4_t*>(p + 4);
    type r = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    return r;
  }
  __device__ __forceinline__ static type load_buf(__amdgpu_buffer_rsrc_t r, uint32_t voff, int soff) {
    const f32x4_t a = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
    const f32x4_t b = __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, voff + 16, soff, 0));
    type v = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    return v;
  }
  __device__ __forceinline__ static type load_f32(const float* p) { return load(p); }
  __device__ __forceinline__ static type from_floats(const float* v) {
    type r = {v[0], v[1], v[2], v[3], v[4], v[5], v[6], v[7]};
    return r;
  }
  __device__ __forceinline__ static f32x4_t mma(f32x4_t acc, type a, type b) {
#pragma unroll
    for (int j = 0; j < 8; ++j) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[j], b[j], acc, 0, 0, 0);
    return acc;
  }
  __device__ __forceinline__ static type mask(type v, uint32_t keep_bits) {
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = ((keep_bits >> j) & 1u) ? v[j] : 0.f;
    return v;
  }
};

// ------------------------------------------------------------------ rotary encoding

// Inverse rotary frequencies theta^(-2i/hd), i < hd/2, in double: filled once per call on the
// host (rope_freq) and carried by value in the epilogues, so no element evaluates exp.
struct RopeFreq {
  double inv[64];
};

inline RopeFreq rope_freq(double theta, int hd) {
  RopeFreq f{};
  const double lt = std::log(theta);
  for (int i = 0; i < hd / 2 && i < 64; ++i) f.inv[i] = std::exp(-(2.0 * i / hd) * lt);
  return f;
}

// cos/sin of the rotary angle pos * inv.  The angle is formed in revolutions and reduced to
// [-1/2, 1/2] in double precision (context positions reach 10^5 and a float angle would be off
// by ~1e-2 rad there), then evaluated by the hardware sine and cosine of 2 pi x
// (v_sin_f32 / v_cos_f32; against double sin/cos at every position below 2^20 and all 64
// frequencies of a 128-wide head, theta 1e6, the largest error is 1.9e-7).
__device__ __forceinline__ void rope_cs(int pos, double inv, float* c, float* s) {
  const double r = static_cast<double>(pos) * (inv * 0.15915494309189533576888376337251);
  const float f = static_cast<float>(r - rint(r));
  *s = __builtin_amdgcn_sinf(f);
  *c = __builtin_amdgcn_cosf(f);
}

// ------------------------------------------------------------------ wave reductions

// Wave-wide sum and maximum without LDS permutes: two quad permutations, the half-row and
// row mirrors (DPP), then the gfx950 row swaps across 16 and 32 lanes.  Each step combines a
// lane with a partner that holds the same partial over a disjoint set of lanes, so the tree
// is fixed and every lane ends with the same value.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_f<0xB1>(v);    // quad_perm [1, 0, 3, 2]
  v += dpp_f<0x4E>(v);    // quad_perm [2, 3, 0, 1]
  v += dpp_f<0x141>(v);   // row_half_mirror
  v += dpp_f<0x140>(v);   // row_mirror
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_f<0xB1>(v));
  v = fmaxf(v, dpp_f<0x4E>(v));
  v = fmaxf(v, dpp_f<0x141>(v));
  v = fmaxf(v, dpp_f<0x140>(v));
  return max_lane_groups(v);
}

// maximum over each aligned group of N lanes (N <= 16, within a DPP row); every lane of a
// group ends with its group's maximum
template <int N>
__device__ __forceinline__ float group_max(float v) {
  static_assert(N == 1 || N == 2 || N == 4 || N == 8 || N == 16, "groups of 1..16 lanes");
  if constexpr (N >= 2) v = fmaxf(v, dpp_f<0xB1>(v));
  if constexpr (N >= 4) v = fmaxf(v, dpp_f<0x4E>(v));
  if constexpr (N >= 8) v = fmaxf(v, dpp_f<0x141>(v));
  if constexpr (N >= 16) v = fmaxf(v, dpp_f<0x140>(v));
  return v;
}

// deterministic block-wide sum (fixed reduction tree); `red` holds >= nwaves floats
__device__ __forceinline__ float block_sum(float v, float* red) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = (blockDim.x + 63) >> 6;
  v = wave_sum(v);
  __syncthreads();
  if (lane == 0) red[w] = v;
  __syncthreads();
  float t = 0.f;
  for (int i = 0; i < nw; ++i) t += red[i];
  return t;
}

// (value, index) order used by every selection: larger value first, then lower index
__device__ __forceinline__ bool better(float va, int ia, float vb, int ib) {
  return va > vb || (va == vb && ia < ib);
}

// 16 E4M3 codes (bytes in k order) widened to two fragments of 8 bf16 values: exact,
// every E4M3 value being a bf16 value.  Each 32-bit word holds 4 codes; the conversion
// takes them two at a time (low half-word first).
__device__ __forceinline__ void fp8x16_to_bf16(u32x4_t raw, bf16x8_t& lo, bf16x8_t& hi) {
  u32x4_t a, b;
  a[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw[0], 1.0f, false));
  a[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw[0], 1.0f, true));
  a[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw[1], 1.0f, false));
  a[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw[1], 1.0f, true));
  b[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw[2], 1.0f, false));
  b[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw[2], 1.0f, true));
  b[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw[3], 1.0f, false));
  b[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw[3], 1.0f, true));
  lo = __builtin_bit_cast(bf16x8_t, a);
  hi = __builtin_bit_cast(bf16x8_t, b);
}

// Scale of an FP8-storage weight row: the float32 stored right after its cols codes.
template <typename T>
__device__ __forceinline__ float fp8_row_scale(const T* row, int cols) {
  return row ? *reinterpret_cast<const float*>(reinterpret_cast<const char*>(row) + cols) : 0.f;
}

}  // namespace dflash
