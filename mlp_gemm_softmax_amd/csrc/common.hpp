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

typedef float float2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));

// float32 -> bfloat16, round to nearest, ties to even (denormals kept, NaN
// stays a quiet NaN): gfx950's v_cvt_pk_bf16_f32, one instruction per pair.
// It was checked bit for bit against the integer rounding (add 0x7fff plus
// the lowest kept bit, truncate; NaN keeps its sign and top payload bits with
// the quiet bit set) on 2^24 values: every tie pattern, denormals, the
// largest finite values, infinities and random bit patterns.
__device__ __forceinline__ uint32_t pack2_bf16(float lo, float hi) {
    const float2v f = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2v));
}

__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
    return __builtin_bit_cast(bf16_t, (__bf16)f);
}

__device__ __forceinline__ float bf16_to_f32(bf16_t h) {
    return __uint_as_float(((uint32_t)h) << 16);
}

// The ReLU value max(v, 0) with a NaN kept: the definition a = z * [z > 0]
// gives NaN for a NaN pre-activation, so a NaN input reaches the logits and
// the loss instead of vanishing here.  The mask [v > 0] is 0 for it.
__device__ __forceinline__ float relu_value(float v) { return v <= 0.f ? 0.f : v; }

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

// Cross-workgroup reductions (split-K partials, row losses) use the
// last-arriving-workgroup pattern without an L2-writeback fence:
//   writer: store the partial with device-scope stores (sc1: acknowledged only
//           once visible to every XCD), wait for the acknowledgements, then
//           take an unsigned integer ticket with atomicAdd;
//   reader: the workgroup that draws the last ticket reads every partial with
//           device-scope loads (sc1: never served from a stale cache line) and
//           adds them in a fixed order.
// An agent-scope __threadfence() would write back the whole L2 of the XCD on
// every workgroup, which serialises across the chip.  No floating-point
// atomics are used anywhere.
__device__ __forceinline__ void store_coherent(float* p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ float load_coherent(const float* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void store_coherent(uint8_t* p, uint8_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint8_t load_coherent(const uint8_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Mean of n <= 64 row losses, written by lane 0 of the calling wavefront:
// lane b takes row b, then the wavefront butterfly, then the other three
// wavefronts' (zero) sums.  These are the additions, in their order, of the
// softmax-CE kernels' own closing mean over 256 threads for n <= 64, so a
// mean taken here has the same bits.
__device__ __forceinline__ void mean_rows_wave(const float* rowloss, int n, float inv_n, float* out) {
    const int lane = threadIdx.x & (kWave - 1);
    float s = 0.f;
    if (lane < n) s += load_coherent(rowloss + lane);
    s = wave_sum(s);
    if (lane == 0) {
        float tot = 0.f;
        tot += s;
        for (int w = 1; w < 4; ++w) tot += 0.f;
        *out = tot * inv_n;
    }
}

// Wait until this thread's stores are acknowledged (and keep the compiler
// from moving memory operations across the wait).
__device__ __forceinline__ void wait_stores() {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// Wait until this thread's outstanding vector-memory loads have landed (also
// the loads that write LDS directly).
__device__ __forceinline__ void wait_loads() {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// Every thread calls this after its coherent stores; returns true in all
// threads of the workgroup that took the last of `expected` tickets, and
// resets the counter for the next launch.
__device__ __forceinline__ bool last_arrival(unsigned* ticket, unsigned expected, int* s_flag) {
    wait_stores();
    __syncthreads();
    if (threadIdx.x == 0) {
        const unsigned old = atomicAdd(ticket, 1u);
        const int last = old == expected - 1;
        if (last) atomicExch(ticket, 0u);
        *s_flag = last;
    }
    __syncthreads();
    return *s_flag != 0;
}

}  // namespace mlp
