// mfma_util.h - gfx950 matrix-core and memory helpers shared by the verify kernels.
#pragma once

#include "bole_device.h"

namespace bole {

typedef float f32x4 __attribute__((ext_vector_type(4)));

// fp32 x -> bf16 hi + bf16 lo with x ~= hi + lo (relative error about 2^-17).
__device__ __forceinline__ void split_bf16(float x, __bf16 &hi, __bf16 &lo) {
    hi = static_cast<__bf16>(x);
    lo = static_cast<__bf16>(x - static_cast<float>(hi));
}

__device__ __forceinline__ bf16x8 load16(const __bf16 *p) {
    return *reinterpret_cast<const bf16x8 *>(p);
}

// Streaming forms for data that is read or written exactly once: the non-temporal
// cache policy keeps it from displacing lines that other waves still use.
__device__ __forceinline__ bf16x8 load16_stream(const __bf16 *p) {
    return __builtin_nontemporal_load(reinterpret_cast<const bf16x8 *>(p));
}

// v_mfma_f32_16x16x32_bf16: lane l holds A[l%16][8(l/16)+e], B[8(l/16)+e][l%16], and
// C rows 4(l/16) + r of column l%16.
__device__ __forceinline__ f32x4 mfma16_bf16(const bf16x8 &a, const bf16x8 &b, const f32x4 &c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

}  // namespace bole
