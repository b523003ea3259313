// device_util.h - device helpers shared by the attention kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {
namespace dev {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

__device__ inline unsigned pack_bf16(float a, float b) {
  const f32x2 v = {a, b};
  return __builtin_bit_cast(unsigned, __builtin_convertvector(v, bf16x2));
}

__device__ inline float max_pair32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
// The same row max without the canonicalising v_max of each input that
// fmaxf needs in IEEE mode (the median of a, b and +inf is max(a, b) for any
// a, b that are not NaN).
__device__ inline float max_pair32_nn(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  float inf = __builtin_inff();
  asm("" : "+s"(inf));   // opaque, or the median is folded back into fmaxf
  return __builtin_amdgcn_fmed3f(__uint_as_float(r[0]), __uint_as_float(r[1]), inf);
}
// wave-wide votes over the active lanes, as one compare and a scalar test
__device__ inline bool wave_any(bool c) { return __builtin_amdgcn_ballot_w64(c) != 0; }
__device__ inline bool wave_all(bool c) { return __builtin_amdgcn_ballot_w64(!c) == 0; }
__device__ inline float sum_pair32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

typedef __amdgpu_buffer_rsrc_t rsrc_t;

__device__ inline rsrc_t make_rsrc(const void* base, unsigned bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes),
                                           0x00020000);
}

// The same descriptor as four scalar words, for the copy below: base, stride 0,
// `bytes` records (offsets at or past it read as zero), 32-bit data format.
__device__ inline u32x4 make_desc(const void* base, unsigned bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  u32x4 d;
  d[0] = __builtin_amdgcn_readfirstlane(static_cast<unsigned>(a));
  d[1] = __builtin_amdgcn_readfirstlane(static_cast<unsigned>(a >> 32) & 0xffffu);
  d[2] = __builtin_amdgcn_readfirstlane(bytes);
  d[3] = 0x00020000u;
  return d;
}

// 16 bytes per lane from global offset `voff` straight into LDS at
// lds_base + 16 * lane. Written as one asm block so that the compiler neither
// moves it nor adds waits for it: completion is tracked by the vmcnt waits in
// the kernel, before the barrier that publishes the data.
// M0 is named as clobbered although the compiler reserves it: these kernels
// contain no other instruction that reads M0, so nothing is lost.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ inline void copy_to_lds(u32x4 desc, unsigned voff, unsigned lds_base) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %2, 0 offen lds"
      :
      : "s"(lds_base), "v"(voff), "s"(desc)
      : "memory", "m0");
}
#pragma clang diagnostic pop

// x = (this lane's bit of m) ? x : -inf, in x's own register. A plain select
// would let the masked scores of partial tiles live in other registers than
// the unmasked scores of full tiles, and the compiler then copies all 32
// scores on every stage to merge the two paths. The caller forms m as a
// ballot of each compare (one v_cmp each, ANDed on the scalar unit).
__device__ inline void mask_in_place(float& x, uint64_t m, float ninf) {
  asm("v_cndmask_b32 %0, %1, %0, %2" : "+v"(x) : "v"(ninf), "s"(m));
}

__device__ inline unsigned lds_addr(const void* p) {
  return static_cast<unsigned>(reinterpret_cast<uintptr_t>(
      (const __attribute__((address_space(3))) char*)(p)));
}

// vmcnt(n) with the other counters left free (gfx9 s_waitcnt encoding)
template <int N>
__device__ inline void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

}  // namespace dev
}  // namespace fa
