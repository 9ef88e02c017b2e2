// Device helpers shared by the bf16 and FP8 decode kernels (gfx950): vector
// types, cross-lane reductions, explicit wait counts, the direct global -> LDS
// copies, loads the compiler does not track, and the write-through store.
// Internal to the library; included inside namespace mla { namespace { ... } }.
#pragma once

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

#define LDS_AS(T, p) ((__attribute__((address_space(3))) T*)(p))

// Max / sum over the four 16-lane groups (lanes l, l^16, l^32, l^48).
// permlaneX_swap(x, x) returns the pair {x[l & ~X], x[l | X]} in some order,
// so combining its two results is symmetric in the pair.
// max of three floats in one instruction (the compiler's fmaxf adds NaN
// canonicalization around every operand; v_max3_f32 treats NaN like fmaxf).
__device__ __forceinline__ float max3(float a, float b, float c) {
  float r;
  asm volatile("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

__device__ __forceinline__ float group_max32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return max3(__uint_as_float(r[0]), __uint_as_float(r[1]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float group_max16(float x) {
  auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return max3(__uint_as_float(s[0]), __uint_as_float(s[1]), __uint_as_float(s[1]));
}

__device__ __forceinline__ float group_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}

// Wait until at most N vector-memory operations of this wave are outstanding
// (N is an immediate).  The query loads and LDS copies are inline asm the
// compiler does not count, so every wait on them is explicit.
template <int N>
__device__ __forceinline__ void wait_vmem() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// 16-byte global -> LDS copies (global_load_lds_dwordx4).  Each lane names its
// own source; the 64 lanes of the wave fill 1 KB of LDS starting at M0.  They
// are issued as inline asm on purpose: the compiler's wait-count pass treats a
// pending LDS copy as aliasing every later LDS read and would insert
// s_waitcnt vmcnt(0) before them, serializing the copy of later tiles with the
// compute on this one.  (s_nop 0: one wait state between the M0 write and the
// copy that reads it.)
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

__device__ __forceinline__ void dma16(const void* src, uint32_t lds_dst) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "{m0}"(lds_dst) : "memory");
}

// Same with a 64-bit per-lane address plus an immediate byte offset.  The
// immediate offset moves the LDS destination too (lane l writes LDS byte
// M0 + OFF + 16 l), so callers pass M0 = destination - OFF.
template <int OFF>
__device__ __forceinline__ void dma16_off(const void* src, uint32_t lds_dst) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off offset:%2" ::"v"(src), "{m0}"(lds_dst), "n"(OFF) : "memory");
}

// Same with a uniform base, a 32-bit per-lane offset and an immediate offset
// (which, as above, is added to the LDS destination as well).
template <int OFF>
__device__ __forceinline__ void dma16_saddr(const void* base, uint32_t off, uint32_t lds_dst) {
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 offset:%3" ::"v"(off), "s"(base), "{m0}"(lds_dst), "n"(OFF)
               : "memory");
}

// 4-byte global load into a VGPR, invisible to the compiler's wait counts
// (waited for explicitly).
__device__ __forceinline__ int load4(const int32_t* src) {
  int v;
  asm volatile("global_load_dword %0, %1, off" : "=v"(v) : "v"(src) : "memory");
  return v;
}

// 16-byte global load into VGPRs, invisible to the compiler's wait counts
// (the explicit wait before the first QK^T covers it).
__device__ __forceinline__ bf16x8 load16(const void* src) {
  bf16x8 v;
  asm volatile("global_load_dwordx4 %0, %1, off" : "=v"(v) : "v"(src) : "memory");
  return v;
}

// Calls f(std::integral_constant<int, I>) for I = 0 .. N-1: loop bodies whose
// register names must be compile-time constants.
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// 16-byte store that writes through this XCD's L2 (system-scope coherence
// bits): the kernel's results are read by the next kernel anyway, and lines
// left dirty in L2 would all be written back at the end of the kernel, after
// the last workgroup, instead of while the other workgroups still run.  A
// store of more than 8 bytes reads its data registers after issue, so no VALU
// instruction may overwrite them in the next wait state; the compiler does not
// see this store, hence the s_nop (checked on the assembly).
template <typename V>
__device__ __forceinline__ void store_wt(void* p, const V& v) {
  static_assert(sizeof(V) == 16, "one 16-byte store");
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  asm volatile("global_store_dwordx4 %0, %1, off sc0 sc1\n\ts_nop 1" ::"v"(p), "v"(__builtin_bit_cast(u32x4, v))
               : "memory");
}
