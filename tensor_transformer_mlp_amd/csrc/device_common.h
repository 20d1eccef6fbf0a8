// Device helpers shared by the gfx950 kernels: vector types, bf16 rounding,
// GeLU and its derivative, SiLU, the XCD-aware tile order, raw buffer descriptors,
// direct-to-LDS loads and the LDS transpose read.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tpmlp {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef short i16x8_t __attribute__((ext_vector_type(8)));

constexpr int kNumXcd = 8;              // MI355X: 8 XCDs of 32 CUs, each XCD with its own L2
constexpr uint32_t kOob = 0x80000000u;  // buffer offset beyond every descriptor's range

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// Round-to-nearest-even float -> bf16 (the hardware conversion on gfx950).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float x) {
  __bf16 h = static_cast<__bf16>(x);
  return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, h));
}

// Four floats to four round-to-nearest-even bf16, packed low to high.
__device__ __forceinline__ u32x2_t pack4_bf16(f32x4_t x) {
  return u32x2_t{f32_to_bf16_bits(x[0]) | (f32_to_bf16_bits(x[1]) << 16),
                 f32_to_bf16_bits(x[2]) | (f32_to_bf16_bits(x[3]) << 16)};
}

// h = Phi(-|x|) = erfc(|x| / sqrt 2) / 2 and e = exp(-x^2 / 2), the two
// pieces of GeLU(x) = x Phi(x) (the erf form of GeLU, not the tanh
// approximation) and of GeLU'(x) = Phi(x) + x phi(x).
//
// erfc(z), z >= 0, follows Abramowitz & Stegun, Handbook of Mathematical
// Functions (1964), formula 7.1.26 (after Hastings):
//   erfc(z) = t (a1 + t (a2 + t (a3 + t (a4 + t a5)))) exp(-z^2) + e(z),
//   t = 1 / (1 + p z),  |e(z)| <= 1.5e-7,
// with p = 0.3275911, a1..a5 = 0.254829592, -0.284496736, 1.421413741,
// -1.453152027, 1.061405429.  Here z = |x| / sqrt 2: p z = (p / sqrt 2) |x|
// and exp(-z^2) = 2^(-x^2 log2(e) / 2), and the factor 1/2 is folded into the
// a_i.  The reciprocal and exp2 run on the hardware transcendental unit; the
// whole evaluation is branch-free (ten VALU operations besides the two
// transcendentals), which matters because it runs once per element of Y_i.
__device__ __forceinline__ void phi_parts(float x, float& h, float& e) {
  const float t = __builtin_amdgcn_rcpf(fmaf(0.3275911f * 0.70710678118654752f, fabsf(x), 1.0f));
  float q = fmaf(t, 0.5f * 1.061405429f, 0.5f * -1.453152027f);
  q = fmaf(t, q, 0.5f * 1.421413741f);
  q = fmaf(t, q, 0.5f * -0.284496736f);
  q = fmaf(t, q, 0.5f * 0.254829592f);
  q *= t;
  e = __builtin_amdgcn_exp2f((x * x) * -0.72134752044448170f);  // exp(-x^2 / 2)
  h = q * e;
}

// GeLU(x) = x Phi(x) = max(x, 0) - |x| Phi(-|x|): for x >= 0 it is
// x (1 - Phi(-x)), for x < 0 it is x Phi(x) with Phi(-|x|) = Phi(x).  Written
// this way the sign case costs one maximum and the last step is one fused
// multiply-add (|x| is an operand modifier).
__device__ __forceinline__ float gelu_f32(float x) {
  float h, e;
  phi_parts(x, h, e);
  return fmaf(-fabsf(x), h, fmaxf(x, 0.0f));
}

// y = GeLU(x) and g = GeLU'(x) = Phi(x) + x phi(x), phi(x) = exp(-x^2/2) / sqrt(2 pi).
__device__ __forceinline__ void gelu_and_grad_f32(float x, float& y, float& g) {
  float h, e;
  phi_parts(x, h, e);
  const float Phi = x < 0.0f ? h : 1.0f - h;
  y = fmaf(-fabsf(x), h, fmaxf(x, 0.0f));  // as gelu_f32, bit for bit
  g = fmaf(x * 0.3989422804014327f, e, Phi);
}

// SiLU(x) = x sigma(x) = x / (1 + exp(-x)), with exp(-x) = 2^(-x log2 e) and
// the reciprocal on the transcendental unit.  For x -> -inf the exponential
// overflows to +inf and the reciprocal to 0, giving the limit (-)0.
__device__ __forceinline__ float silu_f32(float x) {
  const float e = __builtin_amdgcn_exp2f(x * -1.4426950408889634f);
  return x * __builtin_amdgcn_rcpf(1.0f + e);
}

// Workgroups are dispatched round-robin over the 8 XCDs (workgroup id b runs
// on XCD b % 8).  xcd_logical regroups the ids 0 .. nb - 1 so that each XCD
// receives a contiguous range of logical ids: b -> (b % 8) (nb / 8) + b / 8
// for the largest multiple of 8 below nb, the rest unchanged (a bijection).
__device__ __forceinline__ int xcd_logical(int bid, int nb) {
  const int full = nb - nb % kNumXcd;
  return bid < full ? (bid % kNumXcd) * (full / kNumXcd) + bid / kNumXcd : bid;
}

// Logical tile id -> (tile_m, tile_n), walking the tiles in column strips of
// `kGroupM` tile rows, so that consecutive ids share rows of A and columns of
// B.
template <int kGroupM>
__device__ __forceinline__ void strip_coords(int logical, int tiles_m, int tiles_n, int& tm, int& tn) {
  const int group = kGroupM * tiles_n;
  const int g = logical / group;
  const int first_m = g * kGroupM;
  const int gm = min(tiles_m - first_m, kGroupM);
  const int local = logical - g * group;
  tm = first_m + local % gm;
  tn = local / gm;
}

// Map the linear workgroup id bid (of nb, the tiles of one output) to a
// (tile_m, tile_n) pair: each XCD receives a contiguous range of logical
// tiles, walked in strips, so that the tiles resident on one XCD at a time
// share rows of A and columns of B in that XCD's L2.
template <int kGroupM>
__device__ __forceinline__ void tile_coords(int bid, int nb, int tiles_m, int tiles_n, int& tm,
                                            int& tn) {
  strip_coords<kGroupM>(xcd_logical(bid, nb), tiles_m, tiles_n, tm, tn);
}

// gfx9 raw buffer descriptor (stride 0, num_records = bytes) as four SGPRs.
// A load whose offset is at or beyond `bytes` returns zeros (and, for a
// direct-to-LDS load, writes zeros to LDS).
__device__ __forceinline__ i32x4_t buffer_desc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  return i32x4_t{(int)(uint32_t)a, (int)(uint32_t)(a >> 32), (int)bytes, 0x00020000};
}

// 16 bytes per lane from global memory straight into LDS: lane l's data lands
// at LDS byte address `lds_addr + 16 l` (lds_addr is a wave-uniform LDS
// offset); out-of-range lanes write zeros.  Written as inline assembly so that
// the compiler does not track the LDS write itself: its conservative alias
// tracking of in-flight LDS DMA would otherwise insert vmcnt(0) waits before
// fragment reads of other stage buffers.  Completion is waited for explicitly
// (vmcnt) before the barrier that publishes a stage; the "memory" clobber
// keeps LDS accesses in order around it.  M0 is set here for the instruction
// (one wait state between the M0 write and the LDS DMA); no compiler-generated
// code in the kernels that use this relies on M0.
__device__ __forceinline__ void lds_dma16(i32x4_t desc, uint32_t lds_addr, uint32_t voff) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %2, 0 offen lds"
      :
      : "s"(__builtin_amdgcn_readfirstlane(lds_addr)), "v"(voff), "s"(desc)
      : "memory", "m0");
}

// LDS byte offset of a __shared__ object (no null check: the object is known
// to live in LDS).
template <typename T>
__device__ __forceinline__ uint32_t lds_offset(T* shared_obj) {
  return (uint32_t)(uintptr_t)((__attribute__((address_space(3))) char*)(char*)shared_obj);
}

// Two ds_read_b64_tr_b16 transpose reads joined into one 8 x bf16 operand.
// Within each group of 16 lanes, lane t addresses 4 consecutive 16-bit values
// of row r0 + t / 4 (columns c0 + 4 (t % 4) ..) and receives column c0 + t of
// rows r0 .. r0 + 3; p0 and p1 address rows r0 and r0 + 4.
__device__ __forceinline__ bf16x8_t ds_read_tr_pair(const char* p0, const char* p1) {
  const i16x4_t lo =
      __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4_t*)p0);
  const i16x4_t hi =
      __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4_t*)p1);
  const i16x8_t v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8_t, v);
}

}  // namespace tpmlp
