// Shared device helpers for the gfx950 kernels: bfloat16 rounding, MFMA
// vector types, wavefront reductions and the XCD-aware workgroup remap.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace mlp {

constexpr int kWave = 64;      // CDNA wavefront width
constexpr int kXcds = 8;       // MI355X: 8 accelerator complex dies, 32 CUs each

typedef float float16v __attribute__((ext_vector_type(16)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef short short8v __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8v __attribute__((ext_vector_type(8)));

// bfloat16 storage type: the upper 16 bits of an IEEE float32.
typedef uint16_t bf16_t;

// float32 -> bfloat16, round to nearest, ties to even; NaN stays NaN.
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (bf16_t)((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (bf16_t)(u >> 16);
}

__device__ __forceinline__ float bf16_to_f32(bf16_t h) {
    return __uint_as_float(((uint32_t)h) << 16);
}

// Butterfly (xor) reductions over the 64 lanes of a wavefront.  At every
// stage lane i combines v_i with v_{i^m} and lane i^m combines the same two
// values, so all lanes finish with one bitwise-identical result and the order
// of operations is fixed by the lane pattern alone (deterministic).
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int m = 1; m < kWave; m <<= 1) v += __shfl_xor(v, m, kWave);
    return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int m = 1; m < kWave; m <<= 1) v = fmaxf(v, __shfl_xor(v, m, kWave));
    return v;
}

// Workgroups of a launch are handed to the XCDs round robin (id % 8).  Remap
// the hardware id so that each XCD receives one contiguous run of logical ids:
// neighbouring tiles then share their operand rows/columns in that XCD's L2.
// Bijective for any n.
__device__ __forceinline__ int xcd_remap(int id, int n) {
    int xcd = id % kXcds, slot = id / kXcds;
    int per = n / kXcds, rem = n % kXcds;
    return xcd < rem ? xcd * (per + 1) + slot
                     : rem * (per + 1) + (xcd - rem) * per + slot;
}

// Last-arriving-workgroup pattern used by every cross-workgroup reduction:
// each workgroup stores its partial result, executes __threadfence() (an
// agent-scope release: dirty L2 lines are written back so the other XCDs can
// see them), and takes an unsigned integer ticket with atomicAdd.  The
// workgroup that draws the last ticket executes __threadfence() again (an
// agent-scope acquire: stale L1/L2 lines are invalidated), reads every
// partial with ordinary loads and adds them in a fixed order.  No
// floating-point atomics are used anywhere.

}  // namespace mlp
