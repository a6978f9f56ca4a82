// LDS ring helpers of the multi-query passes (gfx950): loads from global
// memory straight into LDS, explicit waits on them, and LDS reads the
// compiler does not order behind those loads.
#pragma once

#include "attn_common.h"

namespace pkv {
namespace {

// Wait until at most N vector-memory operations of the wave are outstanding
// (loads complete in issue order), and keep the compiler from moving memory
// accesses across the wait.  Loads straight into LDS are not tracked by the
// compiler's own wait counts, so the ring below waits for them explicitly.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ void load16_to_lds(const uint8_t *src, u4 *lds_row) {
  __builtin_amdgcn_global_load_lds(
      (const __attribute__((address_space(1))) void *)src,
      (__attribute__((address_space(3))) void *)lds_row, 16, 0, 0);
}

// 16-byte LDS read at byte address `addr` + OFF (an LDS offset).  Issued as
// inline assembly: the compiler would otherwise wait for every load in flight
// into LDS before any LDS read (it cannot tell the ring's slots apart).  The
// caller waits with lds_wait before using the value.
template <int OFF>
__device__ __forceinline__ u4 lds_read16(uint32_t addr) {
  u4 x;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(x) : "v"(addr), "i"(OFF));
  return x;
}
__device__ __forceinline__ void lds_wait() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }
// Wait until at most N LDS reads of the wave are outstanding: LDS reads
// complete in issue order, so every read issued N or more reads before the
// latest has returned (scalar loads in flight only make the wait longer).
template <int N>
__device__ __forceinline__ void lds_wait_n() {
  static_assert(N >= 0 && N < 16, "lgkmcnt");
  asm volatile("s_waitcnt lgkmcnt(%0)" ::"i"(N) : "memory");
}
// Makes later uses of x depend on the preceding lds_wait.
__device__ __forceinline__ void after_wait(u4 &x) { asm volatile("" : "+v"(x)); }

template <int I, int N, int STRIDE>
__device__ __forceinline__ void lds_read_row(uint32_t addr, u4 *out) {
  if constexpr (I < N) {
    out[I] = lds_read16<I * STRIDE>(addr);
    lds_read_row<I + 1, N, STRIDE>(addr, out);
  }
}

}  // namespace
}  // namespace pkv
