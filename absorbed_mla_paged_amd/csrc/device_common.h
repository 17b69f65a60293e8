// Device-side helpers shared by the gfx950 kernels of this library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {
namespace dev {

#define MLA_LDS __attribute__((address_space(3)))

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// 16-bit element traits: MFMA operand vectors and round-to-nearest-even
// conversion from fp32 for fp16 (MLA_F16) and bfloat16 (MLA_BF16).
template <int DT> struct Elem;
typedef short s16x4 __attribute__((ext_vector_type(4)));

template <> struct Elem<0> {
  typedef f16x8 vec8;
  typedef f16x4 vec4;
  typedef _Float16 scalar;
  // D = A(16x32) B(32x16) + C
  static __device__ __forceinline__ f32x4 mfma(vec8 a, vec8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
  // D = A(16x16) B(16x16) + C
  static __device__ __forceinline__ f32x4 mfma16(vec4 a, vec4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ vec4 tr_read(const MLA_LDS void* p) {
    typedef __fp16 fp16x4 __attribute__((__vector_size__(4 * sizeof(__fp16))));
    return __builtin_bit_cast(vec4, __builtin_amdgcn_ds_read_tr16_b64_v4f16((MLA_LDS fp16x4*)p));
  }
};
template <> struct Elem<1> {
  typedef bf16x8 vec8;
  typedef bf16x4 vec4;
  typedef __bf16 scalar;
  static __device__ __forceinline__ f32x4 mfma(vec8 a, vec8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 mfma16(vec4 a, vec4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a),
                                                      __builtin_bit_cast(s16x4, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ vec4 tr_read(const MLA_LDS void* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((MLA_LDS vec4*)p);
  }
};

// Wait until at most N vector-memory operations of this wave are
// outstanding (s_waitcnt vmcnt(N); expcnt and lgkmcnt left alone).
template <int N> __device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt field is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Wait until every LDS / scalar-memory operation of this wave has completed.
__device__ __forceinline__ void wait_lgkmcnt0() {
  __builtin_amdgcn_s_waitcnt((15) | (3 << 14) | (7 << 4) | (0 << 8));
}

// One 16-byte-per-lane copy from global memory straight into LDS: lane i's
// 16 bytes land at lds_base + 16 * i (global_load_lds_dwordx4). Issued from
// inline assembly so that the compiler does not put a full vmcnt(0) wait in
// front of every later LDS read: the kernel waits for each stage itself.
// M0 takes the wave-uniform LDS base; one wait state separates the M0 write
// from the load that reads it.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"  // M0 is set and consumed inside the statement
__device__ __forceinline__ void dma16(const void* gptr, uint32_t lds_base) {
  asm volatile(
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, off"
      :
      : "v"(gptr), "s"(__builtin_amdgcn_readfirstlane(lds_base))
      : "memory", "m0");
}

// Same copy with a wave-uniform 64-bit global base in SGPRs and a 32-bit
// per-lane byte offset (global_load_lds_dwordx4 v_off, s_base): no 64-bit
// per-lane address arithmetic or registers.
__device__ __forceinline__ void dma16s(uint32_t voff, const void* sbase, uint32_t lds_base) {
  asm volatile(
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, %1"
      :
      : "v"(voff), "s"(sbase), "s"(__builtin_amdgcn_readfirstlane(lds_base))
      : "memory", "m0");
}
#pragma clang diagnostic pop

// LDS reads issued from inline assembly, for loops that keep several reads
// in flight ahead of the MFMAs consuming them (the compiler's own schedule
// keeps one or two). The compiler does not count these reads, so every use
// must be preceded by lds_wait<N>(value), N = the number of LDS reads issued
// after this one; a wait makes only the values passed to it safe to use. LDS operations complete in order; any other LDS or scalar
// operation the compiler puts in between only makes such a wait stricter.
template <typename T>
__device__ __forceinline__ T lds_read_b128(uint32_t addr) {
  T v;
  asm volatile("ds_read_b128 %0, %1" : "=v"(v) : "v"(addr) : "memory");
  return v;
}
__device__ __forceinline__ u32x2 lds_read_tr_b16(uint32_t addr) {
  u32x2 v;
  asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(v) : "v"(addr) : "memory");
  return v;
}
__device__ __forceinline__ u32x2 lds_read_b64(uint32_t addr) {
  u32x2 v;
  asm volatile("ds_read_b64 %0, %1" : "=v"(v) : "v"(addr) : "memory");
  return v;
}
// 8-bit transposing read: within each group of 16 lanes, lane j receives as
// byte k (k = 0..7) byte j % 8 of the 8 bytes at the address of lane
// 2 k + j / 8 of its group.
__device__ __forceinline__ u32x2 lds_read_tr_b8(uint32_t addr) {
  u32x2 v;
  asm volatile("ds_read_b64_tr_b8 %0, %1" : "=v"(v) : "v"(addr) : "memory");
  return v;
}
// Wait until at most N LDS operations are outstanding; `v` (the value the
// caller waits for) is routed through the statement so that its uses
// cannot be scheduled above it.
template <int N, typename T>
__device__ __forceinline__ void lds_wait(T& v) {
  static_assert(N >= 0 && N < 16, "lgkmcnt field is 4 bits");
  asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(v) : "n"(N));
}

// The same wait guarding two values (both are ready after it).
template <int N, typename T, typename U>
__device__ __forceinline__ void lds_wait(T& v, U& w) {
  static_assert(N >= 0 && N < 16, "lgkmcnt field is 4 bits");
  asm volatile("s_waitcnt lgkmcnt(%2)" : "+v"(v), "+v"(w) : "n"(N));
}

// lds_wait with a count known only after unrolling (n in 0..15).
template <typename T>
__device__ __forceinline__ void lds_wait_n(int n, T& v) {
  switch (n) {
    case 0: lds_wait<0>(v); break;
    case 1: lds_wait<1>(v); break;
    case 2: lds_wait<2>(v); break;
    case 3: lds_wait<3>(v); break;
    case 4: lds_wait<4>(v); break;
    case 5: lds_wait<5>(v); break;
    case 6: lds_wait<6>(v); break;
    case 7: lds_wait<7>(v); break;
    case 8: lds_wait<8>(v); break;
    case 9: lds_wait<9>(v); break;
    case 10: lds_wait<10>(v); break;
    case 11: lds_wait<11>(v); break;
    case 12: lds_wait<12>(v); break;
    case 13: lds_wait<13>(v); break;
    case 14: lds_wait<14>(v); break;
    default: lds_wait<15>(v); break;
  }
}
template <typename T, typename U>
__device__ __forceinline__ void lds_wait_n(int n, T& v, U& w) {
  switch (n) {
    case 0: lds_wait<0>(v, w); break;
    case 1: lds_wait<1>(v, w); break;
    case 2: lds_wait<2>(v, w); break;
    case 3: lds_wait<3>(v, w); break;
    case 4: lds_wait<4>(v, w); break;
    case 5: lds_wait<5>(v, w); break;
    case 6: lds_wait<6>(v, w); break;
    case 7: lds_wait<7>(v, w); break;
    case 8: lds_wait<8>(v, w); break;
    case 9: lds_wait<9>(v, w); break;
    case 10: lds_wait<10>(v, w); break;
    case 11: lds_wait<11>(v, w); break;
    case 12: lds_wait<12>(v, w); break;
    case 13: lds_wait<13>(v, w); break;
    case 14: lds_wait<14>(v, w); break;
    default: lds_wait<15>(v, w); break;
  }
}

// 16-byte stores into a wave-uniform region, written through the L2 to
// device scope (sc1): the lines are not left dirty in this XCD's L2, so the
// release at the end of the kernel has less to write back, and readers on
// other XCDs find them in memory. A buffer store from the builtin (not
// inline asm) lets the compiler keep the data registers untouched until the
// store has read them. Offsets at or past `bytes` are dropped.
struct WtRegion {
  __amdgpu_buffer_rsrc_t rsrc;
  __device__ WtRegion(void* base, uint32_t bytes)
      : rsrc(__builtin_amdgcn_make_buffer_rsrc(base, 0, (int)bytes, 0x00020000)) {}
  static constexpr int kSc1 = 16;   // cache-policy bit: device-scope write-through
  __device__ void store(uint32_t byte_off, f32x4 v) const {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), rsrc, (int)byte_off, 0,
                                           kSc1);
  }
  __device__ void store(uint32_t byte_off, u32x2 v) const {
    __builtin_amdgcn_raw_buffer_store_b64(v, rsrc, (int)byte_off, 0, kSc1);
  }
  __device__ void store(uint32_t byte_off, float v) const {
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), rsrc, (int)byte_off, 0,
                                          kSc1);
  }
};

// Read-only int32 metadata (block table, plan arrays) through the constant
// address space: uniform loads then become scalar (s_load, counted by
// lgkmcnt), so they never wait behind the in-flight LDS DMA on vmcnt.
#define MLA_CONST __attribute__((address_space(4)))
__device__ __forceinline__ int32_t load_const(const int32_t* p, int64_t i) {
  return ((const MLA_CONST int32_t*)p)[i];
}

__device__ __forceinline__ uint32_t lds_addr(const MLA_LDS void* p) {
  return (uint32_t)(uintptr_t)p;
}

__device__ __forceinline__ float shfl_xor(float v, int mask) {
  return __shfl_xor(v, mask, 64);
}

}  // namespace dev
}  // namespace mla
