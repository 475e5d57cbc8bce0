// Shared gfx950 device plumbing: vector types, buffer resource descriptors,
// LDS helpers and MFMA wrappers.  No attention arithmetic lives here; the
// numerical contract is in contract.hpp.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace detattn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __amdgpu_buffer_rsrc_t rsrc_t;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr int kWave = 64;

// Raw (stride 0) buffer resource.  Word 3 selects 32-bit data format, the value
// every gfx9-family raw buffer access uses.  Accesses whose byte offset lies at
// or beyond num_records read 0 and drop stores; that range check is what bounds
// every load and store in this library.
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t num_records) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)num_records,
                                           0x00020000);
}

__device__ __forceinline__ uint32_t uniform(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_readfirstlane((int)x);
}
__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

__device__ __forceinline__ u32x4 buf_load16(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ __forceinline__ u32x2 buf_load8(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
}
// Direct global -> LDS load, 16 bytes per lane: lane i writes lds_seg + 16 i
// (lds_seg is wave-uniform; it becomes M0).  A lane whose offset fails the
// range check writes zeros, like a range-checked load into registers.  The
// data lands asynchronously: wait_vm() before the barrier that publishes it.
__device__ __forceinline__ void buf_load16_lds(rsrc_t r, unsigned char* lds_seg, uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      r, (__attribute__((address_space(3))) void*)lds_seg, 16, off, 0, 0, 0);
}
// The words of make_rsrc(base, num_records), for the assembly form below.
__device__ __forceinline__ u32x4 rsrc_words(const void* base, uint32_t num_records) {
  const uint64_t a = (uint64_t)base;
  return u32x4{(uint32_t)a, (uint32_t)(a >> 32) & 0xFFFFu, num_records, 0x00020000u};
}
// buf_load16_lds issued from inline assembly.  The compiler does not count
// this load among its outstanding vector-memory operations, so it places no
// wait for it before later LDS reads (which may be of other stages, with the
// load meant to stay in flight); the caller waits for it with wait_vm_n or
// wait_vm before the barrier that publishes its data.  lds_seg must be
// wave-uniform; M0 takes it, with the one wait state an LDS-destination load
// needs after M0 is written.
__device__ __forceinline__ void buf_load16_lds_async(u32x4 rw, unsigned char* lds_seg,
                                                     uint32_t off) {
  const uint32_t m = uniform((uint32_t)(uintptr_t)(
      (__attribute__((address_space(3))) unsigned char*)lds_seg));
  const u32x4 w = {uniform(rw[0]), uniform(rw[1]), uniform(rw[2]), uniform(rw[3])};
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               ::"s"(m), "v"(off), "s"(w)
               : "memory", "m0");
}
__device__ __forceinline__ void wait_vm() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
// Workgroup barrier that completes this wave's LDS operations (so its LDS
// writes are visible to every wave after it) but not its vector-memory loads:
// __syncthreads() also waits for every outstanding load (vmcnt(0)), which
// would drain loads meant to stay in flight across the barrier.  Loads whose
// data the next step reads must be waited for explicitly (wait_vm_n) before
// it.  The memory clobber keeps the compiler from moving memory accesses
// across the barrier.
__device__ __forceinline__ void barrier_lds() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}
// Wait until at most N vector-memory operations of this wave are outstanding
// (they complete in issue order for this count, so the oldest are done).
template <int N>
__device__ __forceinline__ void wait_vm_n() {
  static_assert(N >= 0 && N < 64, "vmcnt is a 6-bit count");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

__device__ __forceinline__ void buf_store16(rsrc_t r, uint32_t off, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, 0);
}
__device__ __forceinline__ void buf_store8(rsrc_t r, uint32_t off, u32x2 v) {
  __builtin_amdgcn_raw_buffer_store_b64(v, r, off, 0, 0);
}
__device__ __forceinline__ void buf_store4(rsrc_t r, uint32_t off, uint32_t v) {
  __builtin_amdgcn_raw_buffer_store_b32(v, r, off, 0, 0);
}
__device__ __forceinline__ void buf_store2(rsrc_t r, uint32_t off, uint16_t v) {
  __builtin_amdgcn_raw_buffer_store_b16(v, r, off, 0, 0);
}

// ---- LDS ------------------------------------------------------------------
__device__ __forceinline__ void lds_store16(unsigned char* lds, uint32_t off, u32x4 v) {
  *reinterpret_cast<u32x4*>(lds + off) = v;
}
__device__ __forceinline__ u32x4 lds_load16(const unsigned char* lds, uint32_t off) {
  return *reinterpret_cast<const u32x4*>(lds + off);
}
__device__ __forceinline__ u32x2 lds_load8(const unsigned char* lds, uint32_t off) {
  return *reinterpret_cast<const u32x2*>(lds + off);
}
// gfx950 transposing LDS read: within each 16-lane group, lane i receives
// element (i % 4) of the 8-byte chunks addressed by lanes (i / 4) + 4r,
// r = 0..3, in that order.
__device__ __forceinline__ s16x4 lds_load_tr16(const unsigned char* lds, uint32_t off) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(lds + off));
}

// ---- conversions ----------------------------------------------------------
// Bits of an fp32 value.  Takes the value by copy: applied directly to an
// ext-vector element subscript, __builtin_bit_cast reads element 0 instead.
__device__ __forceinline__ uint32_t f32_bits(float x) { return __builtin_bit_cast(uint32_t, x); }
__device__ __forceinline__ float bits_f32(uint32_t u) { return __builtin_bit_cast(float, u); }
__device__ __forceinline__ uint16_t bf16_bits(float x) {
  return __builtin_bit_cast(uint16_t, (__bf16)x);  // round to nearest even
}
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
// Two floats to a packed bf16 pair (round to nearest even), one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}
// Four OCP E4M3FN codes (one dword) to four bf16 values; exact, since every
// E4M3FN value is representable in bf16.  gfx950's packed conversion with a
// unit scale, two codes per instruction (bit-identical, NaN codes included, to
// widening through fp32 and keeping the upper half, checked on the device for
// all 256 codes).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ u32x2 e4m3x4_to_bf16x4(uint32_t w) {
  const bf16x2_t lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
  const bf16x2_t hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true);
  return u32x2{__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
}

// ---- MFMA -----------------------------------------------------------------
// v_mfma_f32_32x32x16_bf16: A is 32x16, lane l supplies
// A[l % 32][8*(l/32) .. +7]; B is 16x32, lane l supplies B[8*(l/32) .. +7][l % 32];
// D is 32x32, lane l holds D[8*(i/4) + 4*(l/32) + i%4][l % 32] in element i.
__device__ __forceinline__ f32x16 mfma_bf16(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
// 32x32x64 fp8 x fp8 (OCP E4M3 operands, format code 0) with unit block
// scales (E8M0 127 = 2^0): 64-wide K per instruction, twice the bf16 rate.
// Lane l supplies row (A) / column (B) l % 32 and 32 K-values of half l / 32;
// both operands use the same K slots, so the sum covers each K-value once.
typedef int i32x8 __attribute__((ext_vector_type(8)));
__device__ __forceinline__ f32x16 mfma_fp8x64(u32x4 a0, u32x4 a1, u32x4 b0, u32x4 b1,
                                              f32x16 c) {
  const i32x8 a = {(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3],
                   (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
  const i32x8 b = {(int)b0[0], (int)b0[1], (int)b0[2], (int)b0[3],
                   (int)b1[0], (int)b1[1], (int)b1[2], (int)b1[3]};
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0x7f, 0, 0x7f);
}

}  // namespace detattn
