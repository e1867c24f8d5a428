// distill.hip -- squared Euclidean distance per (batch, head) slab between two float
// outputs of the same shape: the per-layer objective of ReHyAt's attention distillation
// (ReHyAt blog, maplevalley.com.cn, 3.1.1: only phi_q and phi_k are trained, to bring the
// hybrid block's output close in L2 to the frozen softmax teacher's on the same inputs).
//
// The work is two streams of HBM reads and a sum, so it is bandwidth-bound: workgroups
// read 16 KB segments of both tensors as float4 with consecutive lanes on consecutive
// 16-byte chunks, and every sum runs in a fixed order (per-lane sequence, xor butterfly in
// the wave, waves in index order, segments in index order), so the result does not depend
// on scheduling and repeated calls give identical bits.
#include "grad.hpp"

namespace rehyat {

namespace {

constexpr int kBlock = 256;
constexpr int kVecPerThread = 16;                              // float4 per lane per segment
constexpr int64_t kSegFloats = (int64_t)kBlock * kVecPerThread * 4;  // 16384 floats

// sum over the workgroup, fixed order; every thread returns the total
__device__ inline float block_sum(float v, float* red) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
    const int wave = threadIdx.x / 64;
    if (threadIdx.x % 64 == 0) red[wave] = v;
    __syncthreads();
    float t = 0.f;
#pragma unroll
    for (int i = 0; i < kBlock / 64; ++i) t += red[i];
    return t;
}

// partial[bh * nseg + s] = sum of (a - b)^2 over segment s of slab bh (len floats per slab)
__global__ __launch_bounds__(kBlock) void sqdist_partial_kernel(const float* __restrict__ a,
                                                                const float* __restrict__ b, int64_t len,
                                                                int nseg, float* __restrict__ partial) {
    __shared__ float red[kBlock / 64];
    const int64_t blk = blockIdx.x;
    const int bh = (int)(blk / nseg), s = (int)(blk % nseg);
    const float4* pa = reinterpret_cast<const float4*>(a + (int64_t)bh * len + s * kSegFloats);
    const float4* pb = reinterpret_cast<const float4*>(b + (int64_t)bh * len + s * kSegFloats);
    const int64_t nvec = (len - s * kSegFloats) / 4;  // float4 left in the slab (len % 4 == 0)
    float acc = 0.f;
#pragma unroll
    for (int j = 0; j < kVecPerThread; ++j) {
        const int64_t i = (int64_t)j * kBlock + threadIdx.x;
        if (i < nvec) {
            const float4 x = pa[i], y = pb[i];
            const float d0 = x.x - y.x, d1 = x.y - y.y, d2 = x.z - y.z, d3 = x.w - y.w;
            acc += d0 * d0 + d1 * d1 + d2 * d2 + d3 * d3;
        }
    }
    const float t = block_sum(acc, red);
    if (threadIdx.x == 0) partial[blk] = t;
}

// loss[bh] = sum over s of partial[bh * nseg + s]
__global__ __launch_bounds__(kBlock) void sqdist_final_kernel(const float* __restrict__ partial, int nseg,
                                                              float* __restrict__ loss) {
    __shared__ float red[kBlock / 64];
    const int bh = blockIdx.x;
    float acc = 0.f;
    for (int s = threadIdx.x; s < nseg; s += kBlock) acc += partial[(int64_t)bh * nseg + s];
    const float t = block_sum(acc, red);
    if (threadIdx.x == 0) loss[bh] = t;
}

}  // namespace

int sqdist_segments(int64_t len) { return (int)((len + kSegFloats - 1) / kSegFloats); }

hipError_t launch_sqdist(const float* a, const float* b, int64_t len, int BH, float* partial, float* loss,
                         hipStream_t stream) {
    const int nseg = sqdist_segments(len);
    if (nseg > 0) {
        hipLaunchKernelGGL(sqdist_partial_kernel, dim3((unsigned)((int64_t)nseg * BH)), dim3(kBlock), 0, stream, a,
                           b, len, nseg, partial);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(sqdist_final_kernel, dim3((unsigned)BH), dim3(kBlock), 0, stream, partial, nseg, loss);
    return hipGetLastError();
}

}  // namespace rehyat
