// Small device helpers shared by the tiled kernels.
#pragma once
#include <hip/hip_runtime.h>

#include <type_traits>

namespace qg {

// XOR swizzle of the 16-byte chunks of an X tile row in LDS: row r's chunk c
// sits at column c ^ swz(r), so the 128-bit fragment reads of 16 consecutive
// rows (one MFMA operand) hit distinct banks.
__device__ __forceinline__ int swz(int r) { return (r ^ (r >> 3)) & 7; }

// f(integral_constant<int, 0>) .. f(integral_constant<int, N - 1>), unrolled.
template <int N, int I = 0, class F> __device__ __forceinline__ void static_for(F &&f)
{
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        static_for<N, I + 1>(f);
    }
}

// Scheduling-group masks of __builtin_amdgcn_sched_group_barrier.
constexpr int SG_VALU = 0x002, SG_MFMA = 0x008, SG_VMEM_RD = 0x020, SG_DS_RD = 0x100, SG_DS_WR = 0x200;

}  // namespace qg
