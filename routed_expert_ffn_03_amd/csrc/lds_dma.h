// Device helpers shared by the kernels that stage MFMA operands in LDS with
// direct-to-LDS buffer loads (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <utility>

#include "common.h"

namespace moe {

// Raw buffer resource over [base, base + bytes): loads past the end return
// zeros instead of touching memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;

__device__ __forceinline__ uint32_t lds_addr(const void* p) { return (uint32_t)(uintptr_t)p; }

// One direct-to-LDS load: each lane's 16 bytes at voff + soff of the buffer
// land in LDS at lds + 16 * lane.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, void* lds, uint32_t voff, uint32_t soff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)lds, 16, voff, soff, 0, 0);
}

// LDS reads issued as inline asm: operand reads must not wait on the
// direct-to-LDS loads of later stages that are still in flight (the compiler
// would make every LDS read wait for all of them).  The caller waits with an
// s_waitcnt that names the destination registers.
template <int OFF>
__device__ __forceinline__ u32x4 ds_read16(uint32_t addr) {
    u32x4 v;
    asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(v) : "v"(addr), "i"(OFF));
    return v;
}

__device__ __forceinline__ uint32_t ds_read4(uint32_t addr) {
    uint32_t v;
    asm volatile("ds_read_b32 %0, %1" : "=v"(v) : "v"(addr));
    return v;
}

// Wait for all of this wave's LDS reads; then tie each destination register
// to a point after the wait (an empty asm that "modifies" it), so that no use
// of it is scheduled before the wait.
__device__ __forceinline__ void lds_wait_all() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

__device__ __forceinline__ void tie_after_wait(u32x4& v) { asm volatile("" : "+v"(v)); }
__device__ __forceinline__ void tie_after_wait(uint32_t& v) { asm volatile("" : "+v"(v)); }

// Workgroup barrier for data exchanged through LDS only: waits for this
// wave's LDS (and scalar) traffic, not for its vector memory loads, which
// __syncthreads() would also drain when direct-to-LDS loads are in flight.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

template <int N>
__device__ __forceinline__ void vm_wait() {
    asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

template <class F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>{}), ...);
}

template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

}  // namespace moe
