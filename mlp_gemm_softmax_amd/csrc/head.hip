// Fused output layer for narrow class counts (C <= 32): the stand-alone head
// kernel (one workgroup of 16 waves per RB batch rows runs head_block, see
// head_body.hpp: logits, softmax-CE and the dX of the last layer) and the
// stand-alone tail kernel (tail.hpp: dW + SGD of the last layer and the mean
// loss).  Both usually ride along with neighbouring launches instead: the
// head with the last hidden layer's forward, the tail with the first layer's
// dW.  For small batches this replaces the logits GEMM, the CE kernel, the
// dX and dW GEMMs of the last layer and the loss mean, whose run time is
// dominated by launch and memory latency.
#include "kernels.hpp"
#include "head_body.hpp"
#include "tail.hpp"

namespace mlp {
namespace {

__global__ __launch_bounds__(kHeadThreads) void head_kernel(HeadParams p) {
    extern __shared__ float lds[];
    __shared__ float4v s_red[kHeadWaves][kWave];   // K-split partial logits
    head_block<false>(p, blockIdx.x * p.RB, lds, s_red);
}

__global__ __launch_bounds__(kHeadThreads) void tail_kernel(TailParams t) {
    __shared__ float4v red[kHeadWaves * 2 * kWave];
    tail_job<kHeadWaves>(t, blockIdx.x, red);
}

}  // namespace

hipError_t launch_tail(const TailParams& t, hipStream_t s) {
    hipLaunchKernelGGL(tail_kernel, dim3(tail_jobs(t.H)), dim3(kHeadThreads), 0, s, t);
    return hipGetLastError();
}

size_t head_lds_bytes(int H, int C, int RB) {
    const int CP = C | 1, HS = H | 1;
    return sizeof(float) * ((size_t)H * CP + (size_t)RB * HS + 2 * (size_t)RB * C) + (size_t)RB * H;
}

int head_max_lds() { return 96 * 1024; }

hipError_t head_prepare() {
    return hipFuncSetAttribute((const void*)head_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                               head_max_lds());
}

hipError_t launch_head(const HeadParams& p, hipStream_t s) {
    const int grid = (p.B + p.RB - 1) / p.RB;
    hipLaunchKernelGGL(head_kernel, dim3(grid), dim3(kHeadThreads), head_lds_bytes(p.H, p.C, p.RB), s, p);
    return hipGetLastError();
}

}  // namespace mlp
