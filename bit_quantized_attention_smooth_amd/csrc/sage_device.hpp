// sage_device.hpp -- gfx950 (CDNA4) device primitives shared by the kernels:
// MFMA wrappers, wave-half exchange, format conversions, launch geometry.
//
// MFMA operand layouts used throughout (wave64, verified on the GPU with a
// lane-layout probe):
//   32x32 output tile (16 regs per lane): lane l, reg r holds row
//     (r/4)*8 + (l/32)*4 + r%4 and column l%32.
//   A operand: lane l supplies row l%32, B operand: lane l supplies column
//     l%32; both take their K-slice from half (l/32), and A and B index that
//     slice identically, so any consistent assignment of the K dimension to
//     (half, byte) gives the correct contraction.
//   Scaled FP4 MFMA: each lane's 32 E2M1 values (16 bytes) share the E8M0
//     scale that lane supplies -- exactly one MX block per lane.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <limits.h>

namespace sage {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kLog2_448 = 8.807354922057604f;   // log2(448): the FP8 P~ scale, folded into exp2
constexpr float kLog2_6 = 2.584962500721156f;     // log2(6): the E2M1 max, folded into exp2


// S^T[32 keys x 32 queries] += K[32 x 32] * Q^T, INT8 in, INT32 accumulate.
__device__ __forceinline__ v16i mfma_i8(v4i a, v4i b, v16i c) {
  return __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c, 0, 0, 0);
}
// O^T[32 x 32] += A[32 x 64] * B[64 x 32], FP8 E4M3 in, FP32 accumulate.
__device__ __forceinline__ v16f mfma_f8(v8i a, v8i b, v16f c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}
// O^T[32 x 32] += A[32 x 16] * B[16 x 32], fp16 in (eight per lane), fp32 accumulate.
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
__device__ __forceinline__ v16f mfma_f16(v4i a, v4i b, v16f c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(v8h, a), __builtin_bit_cast(v8h, b), c, 0, 0, 0);
}
// Two floats -> two fp16 (RNE) in one dword, a in the low half.
__device__ __forceinline__ int pack_f16x2(float a, float b) {
  return (int)((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)a) |
               ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)b) << 16));
}
// Scaled FP8 MFMA with E8M0 block scales on A only (B unscaled: byte 127 = 1.0).  The two
// 32-element K blocks are bytes [0, 16) and [16, 32) of both lane halves; row m's scale for
// block b comes from lane m + 32 b.
__device__ __forceinline__ v16f mfma_f8_sa(v8i a, v8i b, v16f c, int sa) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, sa, 0, 127);
}
// Scaled MFMA, both operands MXFP4 (E2M1 with per-lane E8M0 scale byte).
__device__ __forceinline__ v16f mfma_mxfp4(v8i a, v8i b, v16f c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 4, 4, 0, sa, 0, sb);
}

// Exchange with the other wave half (lane l <-> lane l^32); returns the partner's value.
__device__ __forceinline__ float other_half(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(threadIdx.x & 32 ? r[0] : r[1]);
}
__device__ __forceinline__ float half_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// 16-byte direct global -> LDS load: lane L's bytes land at lds + 16 L (the LDS pointer is
// wave-uniform).  The builtin exists only in the device compilation pass.
__device__ __forceinline__ void load_lds16(const void* g, void* lds) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_global_load_lds(g, lds, 16, 0, 0);
#endif
}

// The same 16-byte direct load, hidden from the compiler's tracking of LDS writes.  The builtin
// form makes the compiler wait for every outstanding vector-memory load (s_waitcnt vmcnt(0))
// before the next LDS read of any address, which in a prefetching loop exposes the full latency
// of the load just issued.  Callers of this form order its LDS writes themselves: each wave waits
// with s_waitcnt vmcnt(0) and the workgroup meets a barrier before any wave reads the bytes, and
// nothing reads a buffer while a load into it is in flight.  The instruction has no register
// result (it writes LDS at M0 + 16 lane); the compiler itself puts the wave-uniform base in M0.
__device__ __forceinline__ void load_lds16_async(const void* g, void* lds) {
#if defined(__HIP_DEVICE_COMPILE__)
  typedef __attribute__((address_space(3))) uint8_t lds_u8;
  const uint32_t base = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_u8*)lds);
  asm volatile("global_load_lds_dwordx4 %0, off" : : "v"(g), "{m0}"(base) : "memory");
#endif
}

// load_lds16_async with the global address split into a wave-uniform 64-bit base (held in
// scalar registers) and a per-lane 32-bit byte offset (the "saddr" form of the instruction), so
// a loop that moves the base keeps each lane's offset in one register and does no 64-bit
// vector address arithmetic per load.
__device__ __forceinline__ void load_lds16_async_so(const void* sbase, uint32_t voff, void* lds) {
#if defined(__HIP_DEVICE_COMPILE__)
  typedef __attribute__((address_space(3))) uint8_t lds_u8;
  const uint32_t base = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_u8*)lds);
  asm volatile("global_load_lds_dwordx4 %0, %1" : : "v"(voff), "s"(sbase), "{m0}"(base) : "memory");
#endif
}

// The 4-byte form of load_lds16_async (lane L's dword lands at lds + 4 L), same contract.
__device__ __forceinline__ void load_lds4_async(const void* g, void* lds) {
#if defined(__HIP_DEVICE_COMPILE__)
  typedef __attribute__((address_space(3))) uint8_t lds_u8;
  const uint32_t base = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_u8*)lds);
  asm volatile("global_load_lds_dword %0, off" : : "v"(g), "{m0}"(base) : "memory");
#endif
}

// 4-byte direct global -> LDS load: lane L's dword lands at lds + 4 L.
__device__ __forceinline__ void load_lds4(const void* g, void* lds) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_global_load_lds(g, lds, 4, 0, 0);
#endif
}

// Four floats -> four E4M3 bytes (RNE; inputs here never exceed 448).  The first conversion
// writes the low half of a's own register (its high half is overwritten by the second), so no
// zeroed register is needed when a is dead afterwards.
__device__ __forceinline__ int pack_fp8x4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, __float_as_int(a), false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
}

// Eight floats -> eight E2M1 nibbles in one dword (element 2i in the low nibble of byte i),
// each value divided by `scale` (a power of two) before RNE + saturation.
__device__ __forceinline__ unsigned pack_fp4x8(const float* x, float scale) {
  unsigned w = 0;
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, x[0], x[1], scale, 0);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, x[2], x[3], scale, 1);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, x[4], x[5], scale, 2);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, x[6], x[7], scale, 3);
  return w;
}

// E8M0 byte of an MX block whose element format has largest exponent EMAX (E2M1: 2, E4M3: 8):
// floor(log2 amax) - EMAX + 127, clamped at 0; amax == 0 gives 0.  From the fp32 exponent
// field, so it is exact.
template <int EMAX>
__device__ __forceinline__ unsigned mx_scale_byte(float amax) {
  int ef = (int)((__float_as_uint(amax) >> 23) & 0xff);
  if (ef == 0xff) return 0xff;
  int b = ef - EMAX;
  return (unsigned)(b < 0 ? 0 : b);
}
__device__ __forceinline__ unsigned mx_fp4_scale_byte(float amax) { return mx_scale_byte<2>(amax); }
__device__ __forceinline__ float e8m0_to_float(unsigned b) {
  return b == 0 ? 5.877471754111438e-39f : __uint_as_float(b << 23);   // 2^(b-127)
}

__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }
__device__ __forceinline__ float f16_to_f32(uint16_t h) { return (float)__builtin_bit_cast(_Float16, h); }

// fp32 -> bf16 with round-to-nearest-even (NaN stays NaN): the hardware conversion.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }
__device__ __forceinline__ uint16_t f32_to_f16(float f) { return __builtin_bit_cast(uint16_t, (_Float16)f); }   // RNE

template <int DT> __device__ __forceinline__ float load_io(const uint16_t* p) {
  return DT == 0 ? bf16_to_f32(*p) : f16_to_f32(*p);
}
template <int DT> __device__ __forceinline__ uint16_t to_io(float f) {
  return DT == 0 ? f32_to_bf16(f) : f32_to_f16(f);
}

// Wave64 reductions (butterfly over all 64 lanes).
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}

// Workgroup -> XCD-aware linear id.  The dispatcher deals workgroups round-robin
// to the 8 XCDs; this remaps so that consecutive ids land on one XCD, keeping
// the tiles of one head in one L2.
__device__ __forceinline__ int xcd_remap(int id, int total) {
  constexpr int X = 8;
  if (total % X) return id;
  return (id % X) * (total / X) + id / X;
}

}  // namespace sage
