// Group-scale decoding shared by the MFMA kernels that multiply fp16 weights by an fp16
// scale pair.  Not part of the public ABI (include/w4a8.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w4a8 {

// The two E4M3FN codes in bits 0..15 of v (bits 0..7 first), each times a power of two
// `scale`, as an fp16 pair: one v_cvt_scalef32_pk_f16_fp8 (gfx950's conversions take the OCP
// format).  Exact for every finite code and scale 1 or 2^7: an e4m3 value has at most 4
// significant bits and |v| <= 448, so v * 2^7 <= 57344 < 65504 and 2^-9 * 2^0 is an fp16
// subnormal.
__device__ __forceinline__ uint32_t e4m3x2_to_f16x2(uint32_t v, float scale) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(v, scale, false));
}

}  // namespace w4a8
