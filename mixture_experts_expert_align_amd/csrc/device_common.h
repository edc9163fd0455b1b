// Device-side helpers shared by the gfx950 kernels: vector types for the
// MFMA builtins, bf16 rounding, wave-level match, and the MXFP8 encoder.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int kWave = 64;

__device__ __forceinline__ bf16x8 as_bf16x8(i32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// float -> bf16 bits, round to nearest even (NaN kept quiet).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// Raw buffer resource over [p, p + bytes) (32-bit data format, no stride),
// range check clamped to 2^31 - 1 bytes.  The size is clamped with integer
// arithmetic: a floating-point min would put the descriptor in vector
// registers, and every load through it would become a per-lane loop.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* p, int64_t bytes) {
  const int n = bytes < (int64_t)0x7fffffff ? (int)bytes : 0x7fffffff;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, n, 0x00020000);
}

// Workgroup barrier that waits only for the calling wave's LDS operations:
// its outstanding global loads stay in flight across it (__syncthreads also
// waits for those).  The wait is the builtin (lgkmcnt 0; vmcnt 63 and expcnt
// 7 leave those counters alone), so the compiler's own wait insertion knows
// about it; the empty asm statements with memory clobbers keep the compiler
// from moving memory accesses across the barrier.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xc07f);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Buffer loads that write LDS themselves (buffer_load_dword{x4} ... lds):
// one instruction writes the 64 lanes' 4 or 16 bytes to consecutive LDS at
// the wave-uniform address dst, lane i at byte 4i or 16i.  A lane whose
// offset is past the buffer writes zeros.  The compiler does not count these
// loads in its own waits: the kernels wait for them with wait_vm.
typedef __attribute__((address_space(3))) void lds_void;
__device__ __forceinline__ void lds_load16(__amdgpu_buffer_rsrc_t r, void* dst, uint32_t vo, int so) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)dst, 16, vo, so, 0, 0);
}
__device__ __forceinline__ void lds_load4(__amdgpu_buffer_rsrc_t r, void* dst, uint32_t vo, int so) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)dst, 4, vo, so, 0, 0);
}

// Keeps every instruction on its side: explicit vmcnt waits count loads in
// program order, so neither the compiler's IR passes (memory clobber) nor
// its scheduler may move a load across one of these.
__device__ __forceinline__ void issue_order() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// s_waitcnt vmcnt(N) leaving the other counters alone (gfx9 encoding: vmcnt
// in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8); the memory clobbers keep
// loads from moving across it.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x70 | 0xf00);
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

__device__ __forceinline__ float silu_f32(float v) { return v / (1.0f + expf(-v)); }

// Rank of this lane among the valid lanes of its wave holding the same key
// (lower lanes first), the size of that group, and whether this lane is the
// group's last.  Keys are below 2^nbits; one ballot per key bit narrows each
// lane's mask to the lanes that agree with it on every bit.
__device__ __forceinline__ void wave_match_rank(int key, bool valid, int nbits, int& rank, int& gsize,
                                                bool& is_last) {
  const int lane = __lane_id();
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  uint64_t eq = __ballot(valid);
  for (int j = 0; j < nbits; ++j) {
    const uint64_t b = __ballot((key >> j) & 1);
    eq &= ((key >> j) & 1) ? b : ~b;
  }
  rank = __popcll(eq & below);
  gsize = __popcll(eq);
  is_last = valid && rank == gsize - 1;
}

// ---------------------------------------------------------------------------
// MXFP8 (E4M3FN elements, UE8M0 block scales)
// ---------------------------------------------------------------------------

// Scale code of a block whose largest magnitude is bm (a float32 >= 0):
// e = smallest integer with 448 * 2^e >= bm, code = clamp(e + 127, 0, 254),
// and 0 for an all-zero block.  With bm = f * 2^q, f in [1, 2):
// 448 * 2^e = 1.75 * 2^(e+8), so e = q - 8 + (f > 1.75).  A subnormal bm
// (< 2^-126) always clamps to 0.
__device__ __forceinline__ uint32_t mx_scale_code(float bm) {
  const uint32_t u = __float_as_uint(bm) & 0x7fffffffu;
  const uint32_t ef = u >> 23;
  if (ef == 0) return 0u;
  const uint32_t mant = u & 0x7fffffu;
  int e = (int)ef - 127 - 8 + (mant > 0x600000u ? 1 : 0);
  int code = e + 127;
  code = code < 0 ? 0 : (code > 254 ? 254 : code);
  return (uint32_t)code;
}

// 2^(127 - code) as a float, i.e. the reciprocal of the decoded scale.  code
// is in [0, 254], so the exponent 127 - code lies in [-127, 127]; 2^-127 is a
// float32 subnormal and is built from its bit pattern.
__device__ __forceinline__ float mx_inv_scale(uint32_t code) {
  const int ex = 127 - (int)code;
  if (ex >= -126) return __uint_as_float((uint32_t)(ex + 127) << 23);
  return __uint_as_float(0x00400000u);  // 2^-127 = 2^22 * 2^-149
}

// Four E4M3FN codes, packed little-endian into one word (a in byte 0): each
// |v| <= 448, rounded to the nearest code with ties to even, subnormal codes
// below 2^-6, the sign kept (so -0.0 -> 0x80).  This is gfx950's float32 ->
// fp8 pack conversion (OCP E4M3FN, round to nearest even), two values per
// instruction.  It was compared with a bit-level encoder of that rounding rule
// on every float32 of magnitude <= 448, both signs (2,277,507,074 values): no
// difference.  The block scale keeps every input in that range.
__device__ __forceinline__ uint32_t e4m3_pack4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}

// W row index of intermediate feature f (gate, or up when up = true).
__device__ __forceinline__ int w1_row(int f, bool up, int I, int order) {
  return order == 0 ? (up ? I + f : f) : (32 * (f >> 4) + (f & 15) + (up ? 16 : 0));
}

}  // namespace moe
