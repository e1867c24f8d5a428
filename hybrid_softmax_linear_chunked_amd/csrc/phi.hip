// phi.hip -- the polynomial feature map of ReHyAt as a standalone entry point (blog,
// maplevalley.com.cn, section 2.2.2): u = softplus(W x + b) per head, split into P parts,
// each part raised to the powers 1..P, concatenated.  The attention kernels compute phi
// in registers and never call this; it exists for callers and for testing the map.
//
// One wave = 32 tokens; u^T-free formulation: u = X W^T on MFMA (tokens x Dphi), so each
// lane holds one phi row j and 16 tokens, and writes consecutive features across lanes.
#include "common.hpp"
#include "kernels.hpp"

namespace rehyat {

template <class T, int D>
__global__ __launch_bounds__(256) void phi_kernel(const PhiArgs a) {
    using M = Mfma<T>;
    constexpr int KS = M::KS, EPL = M::EPL, NS = D / KS;
    const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64, col = lane % 32, h = lane / 32;
    const int64_t blocks_per_bh = (a.N + 127) / 128;
    const int bh = (int)(blockIdx.x / blocks_per_bh);
    const int64_t t0 = (blockIdx.x % blocks_per_bh) * 128 + wave * 32;
    const int hh = bh % a.H;
    const int Dphi = a.Dphi, P = a.P, F = Dphi * P;
    const T* x = reinterpret_cast<const T*>(a.x) + (int64_t)bh * a.N * D;
    T* feat = reinterpret_cast<T*>(a.feat) + (int64_t)bh * a.N * F;
    const T* w = reinterpret_cast<const T*>(a.w) + (int64_t)hh * Dphi * D;

    typename M::frag xf[NS];
    const int64_t row = t0 + col;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        if (row < a.N) {
            xf[s] = M::load(x + row * D + s * KS + h * EPL);
        } else {
            float zz[EPL];
#pragma unroll
            for (int e = 0; e < EPL; ++e) zz[e] = 0.f;
            xf[s] = M::pack(zz);
        }
    }
    for (int jb = 0; jb < Dphi / 32; ++jb) {
        const int j = jb * 32 + col;
        f32x16 u = zero16();
#pragma unroll
        for (int s = 0; s < NS; ++s) u = M::mma(xf[s], M::load(w + (int64_t)j * D + s * KS + h * EPL), u);
        const float b = a.bias ? a.bias[(int64_t)hh * Dphi + j] : 0.f;
        float uu[16], ph[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            uu[r] = softplus(u[r] + b);
            ph[r] = uu[r];
        }
        for (int pw = 1; pw <= P; ++pw) {
            if (pw > 1) {
#pragma unroll
                for (int r = 0; r < 16; ++r) ph[r] *= uu[r];
            }
            const int f = feat_index(j, pw, Dphi, P);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t tok = t0 + crow(r, h);
                if (tok < a.N) feat[tok * F + f] = from_float<T>(ph[r]);
            }
        }
    }
}

template <class T>
static hipError_t launch_phi_t(const PhiArgs& a, hipStream_t stream) {
    const int64_t blocks = (int64_t)a.BH * ((a.N + 127) / 128);
    switch (a.D) {
        case 32: hipLaunchKernelGGL((phi_kernel<T, 32>), dim3((unsigned)blocks), dim3(256), 0, stream, a); break;
        case 64: hipLaunchKernelGGL((phi_kernel<T, 64>), dim3((unsigned)blocks), dim3(256), 0, stream, a); break;
        case 128: hipLaunchKernelGGL((phi_kernel<T, 128>), dim3((unsigned)blocks), dim3(256), 0, stream, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_phi(const PhiArgs& a, int in_dtype, hipStream_t stream) {
    if (a.N <= 0) return hipSuccess;
    return in_dtype == 1 ? launch_phi_t<bf16>(a, stream) : launch_phi_t<float>(a, stream);
}

}  // namespace rehyat
