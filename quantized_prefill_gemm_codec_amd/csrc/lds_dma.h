// Hardware DMA from memory straight into LDS (buffer_load ... lds) and the
// wait that goes with it, shared by the GEMM and GEMV kernels (device only).
//
// A DMA load writes lane l's element at LDS byte M0 + l * (element size), so
// one instruction fills a contiguous 64-element run of LDS from 64 arbitrary
// per-lane source offsets.  The loads are issued from inline assembly: the
// compiler does not track them, so every consumer waits explicitly with
// wait_vmcnt (loads complete in issue order) and a workgroup barrier.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "unpack.h"

namespace qg {

#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// M0 carries the LDS destination of a DMA load; no other code in these kernels
// uses M0, so clobbering it is safe.
__device__ __forceinline__ void dma_b128(u32x4 rsrc, uint32_t voff, uint32_t soff, uint32_t lds)
{
    asm volatile("s_mov_b32 m0, %3\n\tbuffer_load_dwordx4 %0, %1, %2 offen lds" ::"v"(voff), "s"(rsrc), "s"(soff),
                 "s"(lds)
                 : "memory", "m0");
}
__device__ __forceinline__ void dma_b32(u32x4 rsrc, uint32_t voff, uint32_t soff, uint32_t lds)
{
    asm volatile("s_mov_b32 m0, %3\n\tbuffer_load_dword %0, %1, %2 offen lds" ::"v"(voff), "s"(rsrc), "s"(soff),
                 "s"(lds)
                 : "memory", "m0");
}
#pragma clang diagnostic pop

// Raw buffer descriptor words (base, num_records, gfx9 raw-buffer flags) for
// the inline-assembly loads; out-of-range vector offsets read zero.
__device__ __forceinline__ u32x4 rsrc_words(const void *p, uint32_t bytes)
{
    const uint64_t a = reinterpret_cast<uint64_t>(p);
    return u32x4{uint32_t(a), uint32_t(a >> 32) & 0xFFFFu, bytes, 0x00020000u};
}

// s_waitcnt vmcnt(N) leaving the LDS and export counters alone (gfx9 encoding).
template <int N> __device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Wait until this wave's outstanding LDS reads have returned.  The DMA loads
// above write LDS from the memory path, which the compiler does not order
// against earlier ds_read instructions; a wave that refills a slot it has
// just read issues this first.  (An asm statement with a memory clobber, so
// that no LDS access is moved across it.)
__device__ __forceinline__ void wait_lds_reads() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

__device__ __forceinline__ uint32_t lds_u32(const void *p)
{
    return uint32_t(reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) void *)(p)));
}

}  // namespace qg
