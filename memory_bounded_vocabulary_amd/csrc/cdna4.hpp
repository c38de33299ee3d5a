// CDNA4 (gfx950) device helpers: bf16 MFMA fragments, direct global->LDS
// loads, wait counters and bf16 rounding. Device code only.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lce {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

#define LCE_LDS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// Finite stand-in for -infinity in the running maximum: (-FLT_MAX) - (-FLT_MAX)
// is 0, never NaN, and exp2 of anything below it underflows to 0.
constexpr float kNegBig = -3.4028234663852886e38f;

__device__ __forceinline__ int lane_id() { return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)); }
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// 16x16x32 bf16 MFMA: D = A * B + C. Lane l supplies A[l%16][8*(l/16) .. +7] and
// B[8*(l/16) .. +7][l%16] (8 bf16 each); D element e of lane l sits at
// row 4*(l/16) + e, column l%16. Per flop it draws less power than the
// 32x32x16 shape, which matters because dense bf16 MFMA work on random data
// runs this chip into its power limit well below the peak clock.
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// 16-byte global -> LDS copy issued by a whole wave (direct load into LDS):
// lane l's 16 bytes, read at base + voff (voff per lane), land at
// lds_wave_base + 16*l. base and lds_wave_base must be wave-uniform.
//
// Issued as inline assembly on purpose: the compiler's wait-count pass
// otherwise decides, depending on register allocation, that later LDS reads
// of the *other* buffer must wait for these loads, which serialises the
// pipeline. The callers order LDS explicitly instead: every stage waits with
// s_waitcnt vmcnt and a barrier before reading what was loaded, and only loads
// into a buffer after a barrier that retired all reads of it. The compiler
// does not count these loads in vmcnt, which only makes its own waits for
// other loads stricter (loads complete in order), never weaker. The asm sets
// M0; every direct-to-LDS load of the library goes through here, and no other
// code of these kernels uses M0.
__device__ __forceinline__ void g2lds16(const void* base, uint32_t voff, LCE_LDS void* lds_wave_base) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_wave_base);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2" ::"s"(m0), "v"(voff), "s"(base));
}

// Transposing LDS read (gfx950): see KMajorReader for the lane layout.
__device__ __forceinline__ bf16x4 ds_read_tr16(const LCE_LDS char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LCE_LDS bf16x4*)p);
}

__device__ __forceinline__ void wait_vm0() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
template <int N>
__device__ __forceinline__ void wait_vm() { asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory"); }
__device__ __forceinline__ void wait_lgkm0() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// fp32 -> bf16, round to nearest even (hardware conversion on gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  __bf16 b = (__bf16)f;
  return __builtin_bit_cast(uint16_t, b);
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
}
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// Online log-sum-exp state in the log2 domain: (m, z) stands for 2^m * z.
__device__ __forceinline__ void lse_merge(float& m, float& z, float m2, float z2) {
  float mn = fmaxf(m, m2);
  z = z * fast_exp2(m - mn) + z2 * fast_exp2(m2 - mn);
  m = mn;
}

}  // namespace lce
