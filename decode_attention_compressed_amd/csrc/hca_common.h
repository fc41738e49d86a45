// Shared device helpers for the hca kernels (gfx950).
//
// Codecs follow the OCP bit-field definitions of E4M3 "FN" and E2M1 and the
// bfloat16 truncation of binary32 (storage formats of the V4 page, sections
// 2.1 and 2.2, and the vLLM-0.7.2 page, section 2.2 "fp8_e4m3").  The encoders
// are written with exact float steps (power-of-two scaling and rintf, which
// rounds half to even) so that the same source gives the same codes on the
// host and on the GPU; they are exported to the host for checking.  The
// kernels encode E4M3 with the hardware conversion instead, which gives the
// same codes for every finite binary32 input (an exhaustive GPU probe).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define HCA_HD __host__ __device__ __forceinline__

namespace hca {

HCA_HD uint32_t f2u(float x) { return __builtin_bit_cast(uint32_t, x); }
HCA_HD float u2f(uint32_t u) { return __builtin_bit_cast(float, u); }

// ------------------------------------------------------------------ bf16
HCA_HD uint16_t bf16_encode(float x) {
  // round half to even on the 16 dropped bits (inputs are finite)
  uint32_t u = f2u(x);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
HCA_HD float bf16_decode(uint16_t h) { return u2f((uint32_t)h << 16); }

// ------------------------------------------------------------------ E4M3 (FN)
// value = (-1)^s * 2^(e-7) * (1 + m/8) for e > 0, (-1)^s * 2^-6 * m/8 for e = 0;
// largest finite 448; S.1111.111 is NaN and is never produced.
HCA_HD uint8_t e4m3_encode(float y) {
  const uint32_t sign = (f2u(y) >> 24) & 0x80u;
  float a = fminf(fabsf(y), 448.0f);  // saturate
  uint32_t code;
  if (a < 0.015625f) {  // below 2^-6: subnormal grid of step 2^-9 (8 -> smallest normal)
    code = (uint32_t)rintf(a * 512.0f);
  } else {
    int E = (int)((f2u(a) >> 23) & 0xFFu) - 127;  // -6 .. 8
    uint32_t r = (uint32_t)rintf(ldexpf(a, 3 - E));  // 8 .. 16, half to even
    if (r == 16u) { r = 8u; E += 1; }
    code = ((uint32_t)(E + 7) << 3) | (r - 8u);
  }
  return (uint8_t)(code | sign);
}
// Two codes by the hardware conversion (v_cvt_pk_fp8_f32: OCP E4M3, round half
// to even), after a saturating clamp to [-448, 448], placed in the low (kHi =
// false) or high half of `old`.  Every finite input gives e4m3_encode's codes
// (checked over all binary32 values by hca_probe_e4m3_sweep).
template <bool kHi>
__device__ __forceinline__ uint32_t e4m3_encode2_hw(float a, float b, uint32_t old) {
  a = __builtin_amdgcn_fmed3f(a, -448.0f, 448.0f);
  b = __builtin_amdgcn_fmed3f(b, -448.0f, 448.0f);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)old, kHi);
}
// The quotient x / s for the E4M3 encoder: the code of fl32(x / s) is the code
// of q = x * rs with rs = rcp(s) (within 1 unit in the last place of 1 / s)
// wherever q is in E4M3's normal range and more than 8 units in the last place
// away from the points where E4M3's rounding changes (the midpoints between
// consecutive E4M3 values: the 20 mantissa bits below E4M3's three equal
// 0x80000).  q is within 4 units of fl32(x / s) (three roundings of 2^-24 and
// the reciprocal's 2^-23 of |x / s|), so both lie on the same side of every such
// point, and saturation clamps both alike; everywhere else (zero, E4M3's
// subnormal range, a non-finite q, near a midpoint) the exact quotient is
// taken.
__device__ __forceinline__ float e4m3_quotient(float x, float s, float rs) {
  float q = x * rs;
  const uint32_t u = f2u(q) & 0x7FFFFFFFu;
  if (!(u >= 0x3C800000u && u < 0x7F800000u && ((u & 0xFFFFFu) - 0x7FFF8u) > 16u)) q = x / s;
  return q;
}
// four codes of fl32(v / s) (an fp8 page's encoding), packed little-endian
__device__ __forceinline__ uint32_t e4m3_encode4_div(float v0, float v1, float v2, float v3, float s) {
  const float rs = __builtin_amdgcn_rcpf(s);
  return e4m3_encode2_hw<true>(e4m3_quotient(v2, s, rs), e4m3_quotient(v3, s, rs),
                               e4m3_encode2_hw<false>(e4m3_quotient(v0, s, rs), e4m3_quotient(v1, s, rs), 0u));
}
HCA_HD float e4m3_decode(uint32_t c) {
  const uint32_t e = (c >> 3) & 0xFu, m = c & 7u;
  const float v = e ? ldexpf(1.0f + 0.125f * (float)m, (int)e - 7) : ldexpf((float)m, -9);
  return (c & 0x80u) ? -v : v;
}

// ------------------------------------------------------------------ E2M1
// magnitudes {0, .5, 1, 1.5, 2, 3, 4, 6}; codes 0..7 in that order, bit 3 = sign.
HCA_HD uint32_t e2m1_encode(float y) {
  const uint32_t sign = (f2u(y) >> 28) & 0x8u;
  const float a = fminf(fabsf(y), 6.0f);
  uint32_t code;
  if (a < 2.0f) code = (uint32_t)rintf(a * 2.0f);              // step 0.5
  else if (a < 4.0f) code = 4u + (uint32_t)rintf(a - 2.0f);    // step 1
  else code = 6u + (uint32_t)rintf((a - 4.0f) * 0.5f);         // step 2
  return code | sign;
}
HCA_HD float e2m1_decode(uint32_t c) {
  const uint32_t mag = c & 7u;
  const float v = mag < 4u ? 0.5f * (float)mag : (mag == 4u ? 2.0f : (mag == 5u ? 3.0f : (mag == 6u ? 4.0f : 6.0f)));
  return (c & 8u) ? -v : v;
}

// ------------------------------------------------------------------ score keys
// Monotone map float -> uint32 (larger float, larger key); -0 is folded to +0.
HCA_HD uint32_t order_key(float s) {
  const uint32_t u = f2u(s + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

}  // namespace hca

// ------------------------------------------------------------------ device only
namespace hca {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// RoPE of pair i (dims 2i, 2i+1) at integer position pos: angle pos * theta^(-2i/d),
// reduced modulo 2*pi in fp64 before the fp32 sine/cosine (positions reach 2^20,
// where an fp32 angle would be off by ~0.06 rad).  theta^(-2i/d) is r^i with
// r = theta^(-2/d) taken once on the host in fp64, raised by binary powering
// (at most 22 fp64 multiplies for i < 2048; relative error about i ulp of r,
// which moves an angle at position 2^20 by well under 1e-6 rad).
__device__ __forceinline__ double rope_inv_freq(int i, double r) {
  double acc = 1.0, p = r;
  for (int k = i; k > 0; k >>= 1) {
    acc *= (k & 1) ? p : 1.0;
    p *= p;
  }
  return acc;
}
// rope_inv_freq(4 j + q, r) for q = 0 .. 3 and 0 <= j < 256, bit for bit: the
// same squares of r, multiplied into each power in the same order (a factor
// of 1.0 where a bit is clear, which is exact), but the squares are taken once
// for the four and the two low bits are known for each q.
__device__ __forceinline__ void rope_inv_freq4(int j, double r, double inv[4]) {
  double p = r * r;  // r^2
  inv[0] = 1.0;
  inv[1] = r;
  inv[2] = p;
  inv[3] = r * p;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    p *= p;  // r^(2^(k + 2))
    const double f = ((j >> k) & 1) ? p : 1.0;
#pragma unroll
    for (int q = 0; q < 4; ++q) inv[q] *= f;
  }
}
// cos and sin of pos * inv_freq: the angle in turns (fp64, so that large
// positions keep their fraction), reduced to [-1/2, 1/2] turn, then the hardware
// sine and cosine, which take turns (v_sin_f32 / v_cos_f32: within 1.3e-7 of
// sin / cos(2 pi t) on that range, measured over 2^20 points).
__device__ __forceinline__ void rope_cs(double pos, double inv_freq, float& c, float& s) {
  const double turns = pos * inv_freq * 0.15915494309189535;  // 1 / (2 pi)
  const float t = (float)(turns - rint(turns));
  s = __builtin_amdgcn_sinf(t);
  c = __builtin_amdgcn_cosf(t);
}

// Wave64 reductions: the xor butterfly with strides 32, 16, 8, 4, 2, 1, every
// lane getting the result, on the VALU (a lane shuffle is an LDS round trip).
// Strides 32 and 16 by v_permlane32_swap / v_permlane16_swap (each lane gets
// its own value and lane l ^ 32, resp. l ^ 16); then rotations by 8, 4, 2, 1
// inside each 16-lane row (DPP row_ror): after the steps before, the lane a
// rotation by k reaches holds the value of lane l ^ k, so every step adds the
// same two values as the butterfly (in either order, which IEEE addition does
// not see), and the sums equal the shuffle butterfly's bit for bit.
#define HCA_ROR(v, n) u2f((uint32_t)__builtin_amdgcn_update_dpp(0, (int)f2u(v), 0x120 + (n), 0xF, 0xF, false))
__device__ __forceinline__ float wave_max(float v) {
  const auto a = __builtin_amdgcn_permlane32_swap(f2u(v), f2u(v), false, false);
  v = fmaxf(u2f(a[0]), u2f(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(f2u(v), f2u(v), false, false);
  v = fmaxf(u2f(b[0]), u2f(b[1]));
  v = fmaxf(v, HCA_ROR(v, 8));
  v = fmaxf(v, HCA_ROR(v, 4));
  v = fmaxf(v, HCA_ROR(v, 2));
  return fmaxf(v, HCA_ROR(v, 1));
}
__device__ __forceinline__ float wave_sum(float v) {
  const auto a = __builtin_amdgcn_permlane32_swap(f2u(v), f2u(v), false, false);
  v = u2f(a[0]) + u2f(a[1]);
  const auto b = __builtin_amdgcn_permlane16_swap(f2u(v), f2u(v), false, false);
  v = u2f(b[0]) + u2f(b[1]);
  v = v + HCA_ROR(v, 8);
  v = v + HCA_ROR(v, 4);
  v = v + HCA_ROR(v, 2);
  return v + HCA_ROR(v, 1);
}
#undef HCA_ROR

// Max / sum over the four 16-lane rows of a wave (lanes l, l^16, l^32, l^48),
// every lane getting the result.  Row swaps on the VALU: with both operands x,
// v_permlane32_swap returns (x, x from the other half) split over its two
// results, so the pair holds x[l] and x[l^32] in every lane; v_permlane16_swap
// does the same for x[l] and x[l^16].  Partners combine the same two values,
// so the sum is identical in all four lanes.
__device__ __forceinline__ float rows_max4(float v) {
  const auto a = __builtin_amdgcn_permlane32_swap(f2u(v), f2u(v), false, false);
  v = fmaxf(u2f(a[0]), u2f(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(f2u(v), f2u(v), false, false);
  return fmaxf(u2f(b[0]), u2f(b[1]));
}
__device__ __forceinline__ float rows_sum4(float v) {
  const auto a = __builtin_amdgcn_permlane32_swap(f2u(v), f2u(v), false, false);
  v = u2f(a[0]) + u2f(a[1]);
  const auto b = __builtin_amdgcn_permlane16_swap(f2u(v), f2u(v), false, false);
  return u2f(b[0]) + u2f(b[1]);
}
// max over the four lanes of each quad (DPP quad permutations: partners l ^ 1,
// then l ^ 2), every lane of the quad getting it
__device__ __forceinline__ float quad_max(float v) {
  v = fmaxf(v, u2f((uint32_t)__builtin_amdgcn_update_dpp(0, (int)f2u(v), 0xB1, 0xF, 0xF, false)));  // [1, 0, 3, 2]
  return fmaxf(v, u2f((uint32_t)__builtin_amdgcn_update_dpp(0, (int)f2u(v), 0x4E, 0xF, 0xF, false)));  // [2, 3, 0, 1]
}
// max over each 16-lane row: the quads, then the half-row mirror (a lane of the
// other quad of its half) and the row mirror (a lane of the other half)
__device__ __forceinline__ float row16_max(float v) {
  v = quad_max(v);
  v = fmaxf(v, u2f((uint32_t)__builtin_amdgcn_update_dpp(0, (int)f2u(v), 0x141, 0xF, 0xF, false)));
  return fmaxf(v, u2f((uint32_t)__builtin_amdgcn_update_dpp(0, (int)f2u(v), 0x140, 0xF, 0xF, false)));
}

__device__ __forceinline__ int clampi(int v, int lo, int hi) { return v < lo ? lo : (v > hi ? hi : v); }

// Debug build (-DHCA_DEBUG): where a kernel meets an index its inputs should not
// hold (a page id outside the pool, a block-table slot past the table's width,
// a selected entry outside its sequence's entries, a row outside its page) the
// release build skips the row or the page; the debug build also records a bit
// in this module's device word, which hca_debug_status reads and clears.  The
// word is written by vector atomics only.  Release builds compile the checks
// away.
constexpr uint32_t kDbgPage = 1u, kDbgTable = 2u, kDbgEntry = 4u, kDbgRow = 8u;
#ifdef HCA_DEBUG
static __device__ uint32_t g_hca_dbg;  // one per module: each source file has its own
#define HCA_DBG_CHECK(ok, bit)                        \
  do {                                                \
    if (!(ok)) atomicOr(&::hca::g_hca_dbg, (bit));     \
  } while (0)
// reads (and clears) this module's word; defined once per module by
// HCA_DBG_ACCESSOR(name)
#define HCA_DBG_ACCESSOR(name)                                                                 \
  uint32_t name(bool clear) {                                                                 \
    uint32_t v = 0;                                                                           \
    if (hipMemcpyFromSymbol(&v, HIP_SYMBOL(::hca::g_hca_dbg), sizeof(v), 0, hipMemcpyDeviceToHost) != hipSuccess) \
      return 0x80000000u;                                                                     \
    if (clear) {                                                                              \
      const uint32_t z = 0;                                                                   \
      if (hipMemcpyToSymbol(HIP_SYMBOL(::hca::g_hca_dbg), &z, sizeof(z), 0, hipMemcpyHostToDevice) != hipSuccess) \
        return 0x80000000u;                                                                   \
    }                                                                                         \
    return v;                                                                                 \
  }
#else
#define HCA_DBG_CHECK(ok, bit) ((void)0)
#endif

// Load through the global address space.  Pointers rebuilt from integers (for
// example row addresses kept in LDS) are generic; a generic (flat) load also
// counts against the LDS counter, so every LDS wait would drain it too.
template <typename T>
__device__ __forceinline__ T gload(const void* p) {
  return *(const __attribute__((address_space(1))) T*)(p);
}

}  // namespace hca
