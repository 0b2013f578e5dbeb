// Device helpers for gfx950 (CDNA4, wave64): cross-lane reductions with DPP
// and v_permlane{16,32}_swap, bfloat16 unpacking, dot2 and stores.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

constexpr int kWave = 64;

__host__ __device__ constexpr int ilog2(int x) { return x <= 1 ? 0 : 1 + ilog2(x >> 1); }

// ---------------------------------------------------------------------------
// Cross-lane exchange by "level".  Level k pairs every lane with one lane of
// the neighbouring aligned group of 2^k lanes:
//   0: quad_perm [1,0,3,2]   (lane ^ 1)
//   1: quad_perm [2,3,0,1]   (lane ^ 2)
//   2: row_half_mirror        (i <-> 7-i inside each 8 lanes)
//   3: row_mirror             (i <-> 15-i inside each 16-lane row)
//   4: v_permlane16_swap      (rows 0<->1, 2<->3)
//   5: v_permlane32_swap      (lanes 0-31 <-> 32-63)
// Applying levels lo..hi-1 in order to a value that is already uniform
// inside aligned groups of 2^lo lanes combines 2^(hi-lo) such groups, and the
// result is uniform inside groups of 2^hi lanes: an all-reduce.
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}

struct OpSum {
  __device__ __forceinline__ float operator()(float a, float b) const { return a + b; }
};
struct OpMax {
  __device__ __forceinline__ float operator()(float a, float b) const { return fmaxf(a, b); }
};

template <int LEVEL, class Op>
__device__ __forceinline__ float level_step(float x, Op op) {
  if constexpr (LEVEL == 0) {
    return op(x, dpp_mov<0xB1>(x));
  } else if constexpr (LEVEL == 1) {
    return op(x, dpp_mov<0x4E>(x));
  } else if constexpr (LEVEL == 2) {
    return op(x, dpp_mov<0x141>(x));
  } else if constexpr (LEVEL == 3) {
    return op(x, dpp_mov<0x140>(x));
  } else if constexpr (LEVEL == 4) {
    const unsigned u = __builtin_bit_cast(unsigned, x);
    auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    return op(__builtin_bit_cast(float, (unsigned)r[0]), __builtin_bit_cast(float, (unsigned)r[1]));
  } else {
    const unsigned u = __builtin_bit_cast(unsigned, x);
    auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return op(__builtin_bit_cast(float, (unsigned)r[0]), __builtin_bit_cast(float, (unsigned)r[1]));
  }
}

template <int LO, int HI, class Op>
__device__ __forceinline__ float reduce_levels(float x, Op op) {
  if constexpr (LO < HI) {
    x = level_step<LO>(x, op);
    return reduce_levels<LO + 1, HI>(x, op);
  } else {
    return x;
  }
}

// Cross-group reduction that keeps each lane's offset inside its group:
// combines lanes i, i +- 2^LO, ... over the whole wave (levels LO..5) for
// values that differ from lane to lane inside a group (e.g. one lane per
// 16-byte chunk of a row).  Partners are exact: quad xor for levels 0-1, row
// rotations by 4 and 8 for levels 2-3 (applied together they cover the four
// quads of a row), the permlane swaps for levels 4-5.
template <int LEVEL, class Op>
__device__ __forceinline__ float aligned_step(float x, Op op) {
  if constexpr (LEVEL == 2) {
    return op(x, dpp_mov<0x124>(x));  // row_ror:4
  } else if constexpr (LEVEL == 3) {
    return op(x, dpp_mov<0x128>(x));  // row_ror:8
  } else {
    return level_step<LEVEL>(x, op);
  }
}

template <int LO, class Op>
__device__ __forceinline__ float reduce_groups(float x, Op op) {
  if constexpr (LO < 6) {
    x = aligned_step<LO>(x, op);
    return reduce_groups<LO + 1>(x, op);
  } else {
    return x;
  }
}

// ---------------------------------------------------------------------------
// bfloat16 (bit patterns in uint16 / packed pairs in uint32)
// ---------------------------------------------------------------------------
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xFFFF0000u); }

// a.lo*b.lo + a.hi*b.hi + c with fp32 accumulation (v_dot2_f32_bf16).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

// Round to nearest even (hardware conversion on gfx950).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const __bf16 a = (__bf16)lo;
  const __bf16 b = (__bf16)hi;
  return (uint32_t)__builtin_bit_cast(uint16_t, a) |
         ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

// A pointer every lane holds the same value of, made provably wave-uniform
// (scalar registers), so that loads through it with uniform indices become
// scalar loads, counted apart from the vector loads in flight.
template <class T>
__device__ __forceinline__ T* uniform_ptr(T* p) {
  const uint64_t v = (uint64_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (T*)(((uint64_t)hi << 32) | lo);
}

// Buffer resource for `bytes` bytes at `base` (raw, untyped 32-bit data
// format); loads through it are bounds-checked against `bytes` (reads past
// the end return 0).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

// 16-byte load at voff (per lane) + soff (wave-uniform) within a buffer.
__device__ __forceinline__ uint4 buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff,
                                               uint32_t soff) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0);
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// Cache-policy operand of buffer instructions on gfx950: the non-temporal
// (nt) bit.  Streaming data that is read exactly once is loaded with it so
// that it does not displace reusable lines; measured on MI355X, a permuted
// 32 KiB-block read of 1.7 GB rises from 6.2 to 7.0 TB/s with it.
constexpr int kCachePolicyNT = 2;

// The same load, non-temporal.
__device__ __forceinline__ uint4 buffer_load16_nt(__amdgpu_buffer_rsrc_t r, uint32_t voff,
                                                  uint32_t soff) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, kCachePolicyNT);
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// 16-byte non-temporal load through a flat global pointer.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load16_nt(const void* p) {
  const u32x4_t v = __builtin_nontemporal_load((const u32x4_t*)p);
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// ---------------------------------------------------------------------------
// e4m3 (fp8) codes: the hardware's packed conversions on gfx950 use the e4m3
// format with bias 7, maximum 448, NaN 0x7F/0xFF, rounding to nearest even.
// ---------------------------------------------------------------------------
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// The 16 codes of a 16-byte chunk as floats, in memory order.
__device__ __forceinline__ void fp8x16_to_f32(const uint4& w, float (&f)[16]) {
  const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const f32x2_t lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)u[i], false);
    const f32x2_t hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)u[i], true);
    f[4 * i] = lo[0];
    f[4 * i + 1] = lo[1];
    f[4 * i + 2] = hi[0];
    f[4 * i + 3] = hi[1];
  }
}

// The 16 codes of a 16-byte chunk as 8 bfloat16 pairs in memory order (pair
// e = codes 2e, 2e + 1, the first in the low half).  Every e4m3 value is a
// bfloat16 value, so the conversion (scale 1) is exact.
__device__ __forceinline__ void fp8x16_to_bf16x2(const uint4& w, uint32_t (&b)[8]) {
  const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    b[2 * i] = __builtin_bit_cast(uint32_t,
                                  __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)u[i], 1.0f, false));
    b[2 * i + 1] = __builtin_bit_cast(uint32_t,
                                      __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)u[i], 1.0f, true));
  }
}

// Two chunks of 16 codes (rows a and b, the same 16 dims) as 16 bfloat16
// pairs: pair e = (a's code e, b's code e), a in the low half.  Bytes are
// interleaved with v_perm_b32, then converted two at a time (exactly).
__device__ __forceinline__ void fp8x16_pairs_to_bf16x2(const uint4& wa, const uint4& wb,
                                                       uint32_t (&p)[16]) {
  const uint32_t ua[4] = {wa.x, wa.y, wa.z, wa.w};
  const uint32_t ub[4] = {wb.x, wb.y, wb.z, wb.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    // bytes (a0, b0, a1, b1) and (a2, b2, a3, b3) of dword i of each row
    const uint32_t lo = __builtin_amdgcn_perm(ub[i], ua[i], 0x05010400u);
    const uint32_t hi = __builtin_amdgcn_perm(ub[i], ua[i], 0x07030602u);
    p[4 * i] = __builtin_bit_cast(uint32_t,
                                  __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)lo, 1.0f, false));
    p[4 * i + 1] = __builtin_bit_cast(uint32_t,
                                      __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)lo, 1.0f, true));
    p[4 * i + 2] = __builtin_bit_cast(uint32_t,
                                      __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)hi, 1.0f, false));
    p[4 * i + 3] = __builtin_bit_cast(uint32_t,
                                      __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)hi, 1.0f, true));
  }
}

// Two floats to two e4m3 codes (low byte = a), nearest even.
// Index of the scale of (physical block, row of the block, KV head) in an fp8
// scale pool laid out [num_blocks][num_kv_heads][block_size]: the rows of one
// head are contiguous, so the rows of one load instruction share one short
// run of scales.
__device__ __forceinline__ int64_t fp8_scale_index(int64_t phys, int row, int kvh,
                                                   int num_kv_heads, int log2_bs) {
  return ((phys * num_kv_heads + kvh) << log2_bs) + row;
}

__device__ __forceinline__ uint32_t f32x2_to_fp8(float a, float b) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xFFFFu;
}

// Masking selects done on bit patterns.  The library is built with relaxed
// NaN handling (so that fmaxf needs no quieting); a select between integers
// cannot be rewritten by any floating-point assumption, so a masked row's
// NaN-poisoned bytes are replaced before they reach any arithmetic.
__device__ __forceinline__ float select_bits(bool keep, float x, float other) {
  return __uint_as_float(keep ? __float_as_uint(x) : __float_as_uint(other));
}
__device__ __forceinline__ uint4 mask_words(bool keep, uint4 w) {
  return keep ? w : make_uint4(0u, 0u, 0u, 0u);
}

// 2^x on the transcendental unit; exact 0 for x = -inf.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

}  // namespace pa
