// Device helpers shared by the gfx950 kernels: vector types, MFMA wrappers,
// base-2 transcendentals and the XCD-aware workgroup order.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace cpattn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();

// Hardware base-2 exponential and logarithm (v_exp_f32 / v_log_f32).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// D(32x32) += A(32x16) * B(16x32), bf16 inputs, fp32 accumulate.
// Lane l supplies A row (l % 32), k-slots 8*(l/32) .. +7, and B column
// (l % 32) for the same k-slots; it receives D[8*(i/4) + 4*(l/32) + i%4][l % 32]
// in element i of the accumulator.
__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// D(16x16) += A(16x32) * B(32x16).  Lane l supplies A row (l % 16), k-slots
// 8*(l/16) .. +7, B column (l % 16) for the same k-slots, and receives
// D[4*(l/16) + i][l % 16] in element i.
__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4& x) { return __builtin_bit_cast(bf16x8, x); }
__device__ __forceinline__ u32x4 as_u32x4(const bf16x8& x) { return __builtin_bit_cast(u32x4, x); }

// Two floats to packed bf16 (round to nearest even), low half = a.
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  bf16x2 v = __builtin_convertvector((f32x2){a, b}, bf16x2);
  return __builtin_bit_cast(uint32_t, v);
}

// Byte-select of two dwords: v_perm_b32.
__device__ __forceinline__ uint32_t perm_b32(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}
// {lo16(a), lo16(b)} and {hi16(a), hi16(b)}
__device__ __forceinline__ uint32_t pack_lo16(uint32_t a, uint32_t b) { return perm_b32(b, a, 0x05040100u); }
__device__ __forceinline__ uint32_t pack_hi16(uint32_t a, uint32_t b) { return perm_b32(b, a, 0x07060302u); }

__device__ __forceinline__ u32x4 ld_global16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ u32x4 ld_lds16(const uint8_t* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ u32x2 ld_lds8(const uint8_t* p) { return *reinterpret_cast<const u32x2*>(p); }
__device__ __forceinline__ void st_lds16(uint8_t* p, const u32x4& v) { *reinterpret_cast<u32x4*>(p) = v; }
__device__ __forceinline__ void st_lds8(uint8_t* p, const u32x2& v) { *reinterpret_cast<u32x2*>(p) = v; }

// 16 bytes from global memory straight into LDS (global_load_lds_dwordx4):
// lane i of the wave writes LDS bytes [lds_base + 16 i, lds_base + 16 i + 16).
// Issued through inline assembly so the compiler does not drain every
// outstanding load before it (it cannot tell which LDS bytes a pending
// transfer writes); the caller waits with s_waitcnt vmcnt before using the
// data.  lds_base must be wave-uniform.
__device__ __forceinline__ void gload_lds16(const void* gptr, uint32_t lds_base) {
  asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(gptr), "{m0}"(__builtin_amdgcn_readfirstlane(lds_base))
               : "memory");
}
// The same transfer addressed as a wave-uniform base in SGPRs plus a 32-bit
// per-lane byte offset (the saddr form): moving the base costs scalar adds
// only, no vector instructions.
__device__ __forceinline__ void gload_lds16(const void* sbase, uint32_t voff, uint32_t lds_base) {
  asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "{m0}"(__builtin_amdgcn_readfirstlane(lds_base))
               : "memory");
}
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const void*)p));
}

// Value of the lane 32 positions away (lanes 0..31 <-> 32..63).
__device__ __forceinline__ float xor32(float x) { return __shfl_xor(x, 32); }

// max / sum of a value and its copy in the lane 32 positions away, through
// v_permlane32_swap: swapping the upper half of x with the lower half of a
// second copy of x leaves {x[l mod 32], x[l mod 32 + 32]} in the two results.
__device__ __forceinline__ float pair32_max(float x) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float pair32_sum(float x) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}

// How a finished row is written.  The kernel holds an unnormalised
// accumulator relative to the base-2 reference m2 and the row sum l.  A plain
// store writes O = acc / l and LSE = (m2 + log2 l) ln 2 (-inf and O = 0 for a
// row with no visible key).  An accumulating store merges that partial with
// the normalised O and natural-log LSE already at the destination, exactly
// (up to rounding) as the LSE merge does: with M the larger of the two LSEs,
// O = (O_old w_old + O_new w_new) / (w_old + w_new), w = exp(LSE - M), and
// LSE = M + ln(w_old + w_new).  Every output value is acc * s_new + old * s_old.
struct RowOut {
  float s_new, s_old, lse;
};
__device__ __forceinline__ RowOut row_out(float m2, float l, bool accumulate, float lse_old) {
  const float lse2 = (l > 0.f) ? m2 + fast_log2(l) : kNegInf;
  if (!accumulate) return RowOut{(l > 0.f) ? 1.f / l : 0.f, 0.f, (l > 0.f) ? lse2 * kLn2 : kNegInf};
  const float old2 = lse_old * kLog2e;
  const float mx = fmaxf(lse2, old2);
  if (mx == kNegInf) return RowOut{0.f, 0.f, kNegInf};
  const float wn = fast_exp2(lse2 - mx), wo = fast_exp2(old2 - mx);
  const float t = 1.f / (wn + wo);
  return RowOut{(l > 0.f) ? wn * t / l : 0.f, wo * t, (mx + fast_log2(wn + wo)) * kLn2};
}

// The LSE merge of n partials of a row, one piece at a time so that every
// kernel that merges rounds identically: with M the largest partial LSE,
// partial c gets the weight w_c = exp(lse_c - M); den and acc sum w_c and
// w_c O_c in partial order; the row is acc / den and its LSE M + ln(den).
__device__ __forceinline__ float merge_weight(float lse, float M) { return fast_exp2((lse - M) * kLog2e); }
__device__ __forceinline__ void merge_acc(f32x4& acc, float w, const f32x4& v) {
  acc[0] = fmaf(w, v[0], acc[0]);
  acc[1] = fmaf(w, v[1], acc[1]);
  acc[2] = fmaf(w, v[2], acc[2]);
  acc[3] = fmaf(w, v[3], acc[3]);
}
__device__ __forceinline__ float merge_inv(float den) { return (den > 0.f) ? 1.f / den : 0.f; }
__device__ __forceinline__ float merged_lse(float M, float den) {
  return (den > 0.f) ? M + fast_log2(den) * kLn2 : kNegInf;
}

// Four consecutive output values, as fp32 or rounded to bf16.
__device__ __forceinline__ void store_row(void* out, bool out_bf16, int64_t off, const f32x4& r) {
  if (out_bf16) {
    const u32x2 pk = {pack_bf16(r[0], r[1]), pack_bf16(r[2], r[3])};
    *reinterpret_cast<u32x2*>(static_cast<__bf16*>(out) + off) = pk;
  } else {
    *reinterpret_cast<f32x4*>(static_cast<float*>(out) + off) = r;
  }
}

// The K/V chunk of the c-th partial to reach owner i, whose visible K/V
// chunks are [0, n) (n >= i + 1: a Q chunk always sees its own K/V chunk).
// Pass-KV sends K/V down the ring, so at step s owner i holds K/V chunk
// (i - s) mod P: the visible ones arrive as i, i-1, ..., 0, then n-1, n-2,
// ..., i+1.  Pass-Q sends Q, so at step s the rank holding K/V chunk
// (i + s) mod P computes owner i's piece: i, i+1, ..., n-1, then 0, 1, ...,
// i-1.  (Equal Q and K/V lengths under the causal mask give n = i + 1.)
__device__ __forceinline__ int arrival_kv(bool pass_q, int i, int n, int c) {
  if (pass_q) return c < n - i ? i + c : c - (n - i);
  return c <= i ? i - c : n + i - c;
}

// Workgroups are dispatched round-robin over the 8 XCDs (workgroup w runs on
// XCD w % 8).  Give each XCD a contiguous range of logical tiles so tiles that
// share K/V (adjacent heads of one query tile) share that XCD's L2.
__device__ __forceinline__ int xcd_logical_block(int w, int total) {
  const int per = total >> 3;
  const int full = per << 3;
  return (w < full) ? ((w & 7) * per + (w >> 3)) : w;
}

}  // namespace cpattn
