// Device helpers shared by the MFMA kernels (gfx950): buffer resources,
// global -> LDS copies that bypass VGPRs, and LDS transpose reads.
#pragma once

#include "common.h"

namespace mtp {

typedef __attribute__((address_space(3))) void lds_void;
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

// A buffer load whose offset is at or past num_records returns zeros; every
// resource built here has num_records < kOOB.
constexpr uint32_t kOOB = 0x80000000u;
constexpr uint32_t kRsrcWord3 = 0x00020000u;

__device__ __forceinline__ lds_void* to_lds(const void* p) {
  return (lds_void*)const_cast<void*>(p);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes),
                                           static_cast<int>(kRsrcWord3));
}

// 16 bytes from byte offset `off` of the resource to LDS: lane l of the wave
// writes bytes [16 l, 16 l + 16) after the wave-uniform LDS address `dst`.
__device__ __forceinline__ void copy16_to_lds(__amdgpu_buffer_rsrc_t rs, void* dst, uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, to_lds(dst), 16, off, 0, 0, 0);
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// The resource of make_rsrc as four scalar words (base, base bits 32..47
// with stride 0, num_records, word 3), for copies issued by copy16_raw.
__device__ __forceinline__ u32x4 rsrc_words(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  u32x4 r;
  r[0] = static_cast<uint32_t>(a);
  r[1] = static_cast<uint32_t>(a >> 32) & 0xffffu;
  r[2] = bytes;
  r[3] = kRsrcWord3;
  return r;
}

// 32-bit LDS address of a pointer into __shared__ memory.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(to_lds(p)));
}

// The copy of copy16_to_lds (lane l writes 16 bytes at LDS address
// dst + 16 l), issued from inline assembly so that the compiler's wait-count
// insertion does not track it: the caller waits for it with an explicit
// s_waitcnt vmcnt.  One wait state separates the M0 write from the load.
// The statement is volatile but clobbers no memory: it keeps its order
// relative to other volatile statements (the explicit waits and barriers,
// which clobber memory), while LDS reads of other stages may be scheduled
// around it.  The caller must not read a stage between issuing a copy into
// it and the wait + barrier that make the copy visible.
// The destination is wave-uniform; readfirstlane states so (it costs
// nothing where the compiler already knows it), so that the "s" operand is
// never a VGPR.
__device__ __forceinline__ void copy16_raw(const u32x4& rs, uint32_t dst, uint32_t off) {
  const uint32_t d = __builtin_amdgcn_readfirstlane(dst);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :: "s"(d), "v"(off), "s"(rs) : "m0");
}

// ds_read_b64_tr_b16: in each group of 16 lanes, lane i receives element j
// (j = 0..3) from the 8-byte word addressed by lane 4j + i/4, at sub-element
// i % 4.  With lane 4j + q pointing at row r0 + j, columns c0 + 4q .. +3 of
// a row-major bf16 matrix, lane i receives column c0 + i of rows r0..r0+3.
__device__ __forceinline__ v4i16 tr_read(const void* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)const_cast<void*>(p));
}

__device__ __forceinline__ bf16x8 cat_bf16x8(v4i16 lo, v4i16 hi) {
  const v4i16 v[2] = {lo, hi};
  return __builtin_bit_cast(bf16x8, v);
}

}  // namespace mtp
