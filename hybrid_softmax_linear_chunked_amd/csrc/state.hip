// state.hip -- linear-attention state of ReHyAt (blog, maplevalley.com.cn, section 2.3:
// S = sum phi_k(K)^T V, Z = sum phi_k(K), updated by the frames that leave the softmax
// window).
//
// state_kernel: one workgroup per (batch-head, frame) computes the frame's partial
//   Delta_f = phi_k(K_f)^T V_f  (F x D)  and  sum_tokens phi_k(K_f)  (F),
//   with phi computed on the fly: u = K W_k^T on MFMA (tokens x Dphi), softplus, powers,
//   then Delta += phi^T V on MFMA with phi taken straight from the u registers (the C
//   tile's rows are the tokens, which is the contraction of the second product).  Two
//   forms: state16_kernel (bf16 inputs: 16x16x32 products, each wave owning 16 phi rows
//   over whole tiles, K/V moved by LDS-DMA) and state_kernel (float32 inputs: 32x32x2
//   products, wave (jb, ts) owning the 32 phi rows of block jb and the 32-token half ts
//   of every 64-token tile, the two halves summed through LDS in a fixed order).
// scan_kernel: running sum over frame partials in frame order, either in place (prefix
//   over the clip, chunk-parallel form) or added to a carried state (streaming form).
//   Both forms add the same partials in the same order, so they agree bit for bit.
// copy_kernel: keeps the last To frames of the window as the streaming overlap.
#include <type_traits>

#include "dma.hpp"
#include "kernels.hpp"
#include "state16.hpp"
#include "tiles.hpp"

namespace rehyat {

// Waves: wave = jb * TS + ts.  With P <= 2 the 64-token tile is split between two waves
// (TS = 2, eight waves for Dphi = 128); with larger P one wave takes the whole tile so the
// P x D/32 accumulator tiles still fit in its registers.
template <int P>
struct StateShape {
    static constexpr int TS = P <= 2 ? 2 : 1;
    static constexpr int NW = 4 * TS;  // Dphi <= 128: at most 4 blocks of 32 phi rows
};

template <class T, int D, int P>
__global__ __launch_bounds__(StateShape<P>::NW * 64) void state_kernel(const StateArgs a) {
    using M = Mfma<T>;
    constexpr int TS = StateShape<P>::TS;
    constexpr int NT = StateShape<P>::NW * 64;
    using Tile = KVTile<T, D, NT>;
    constexpr int KS = M::KS, EPL = M::EPL, NS = D / KS, NDB = D / 32, TPB = 16 / EPL;

    extern __shared__ __align__(16) unsigned char smem[];
    T* Ks0 = reinterpret_cast<T*>(smem);
    T* Vs0 = Ks0 + Tile::K_ELEMS;
    T* Ks1 = Vs0 + Tile::V_ELEMS;
    T* Vs1 = Ks1 + Tile::K_ELEMS;

    const int gi = blockIdx.x % a.G;
    const int bh = blockIdx.x / a.G;
    const int hh = bh % a.H;
    const int g = a.g0 + gi;
    const int n = a.n, Dphi = a.Dphi, F = Dphi * P, NJB = Dphi / 32;

    KeySrc<T> src;
    if (g < a.nf1) {
        src.k1 = reinterpret_cast<const T*>(a.k1) + (int64_t)bh * a.kv1_bh_stride + (int64_t)g * n * D;
        src.v1 = reinterpret_cast<const T*>(a.v1) + (int64_t)bh * a.kv1_bh_stride + (int64_t)g * n * D;
    } else {
        src.k1 = reinterpret_cast<const T*>(a.k2) + (int64_t)bh * a.kv2_bh_stride + (int64_t)(g - a.nf1) * n * D;
        src.v1 = reinterpret_cast<const T*>(a.v2) + (int64_t)bh * a.kv2_bh_stride + (int64_t)(g - a.nf1) * n * D;
    }
    src.k2 = src.k1;
    src.v2 = src.v1;
    src.len1 = n;

    const int tid = threadIdx.x;
    const int wave = tid / 64, lane = tid % 64, col = lane % 32, h = lane / 32;
    const bool active = wave < TS * NJB;
    const int jb = wave / TS, ts = wave % TS;
    const int j = jb * 32 + col;  // this lane's phi row

    // W_k^T operand (B of u = K W^T): column j, contraction over d
    typename M::frag wf[NS];
    float bias = 0.f;
    if (active) {
        const T* wk = reinterpret_cast<const T*>(a.wk) + ((int64_t)hh * Dphi + j) * D;
#pragma unroll
        for (int s = 0; s < NS; ++s) wf[s] = M::load(wk + s * KS + h * EPL);
        if (a.bk) bias = a.bk[(int64_t)hh * Dphi + j];
    }

    f32x16 acc[P][NDB];
    float zacc[P];
#pragma unroll
    for (int pw = 0; pw < P; ++pw) {
        zacc[pw] = 0.f;
#pragma unroll
        for (int db = 0; db < NDB; ++db) acc[pw][db] = zero16();
    }

    const int ntiles = (n + Tile::BK - 1) / Tile::BK;
    Tile tile;
    tile.template load<true, false>(src, 0, n, tid);
    tile.store(Ks0, Vs0, tid);
    __syncthreads();
    for (int it = 0; it < ntiles; ++it) {
        const T* Ks = (it & 1) ? Ks1 : Ks0;
        const T* Vs = (it & 1) ? Vs1 : Vs0;
        const int t0 = it * Tile::BK;
        const bool more = it + 1 < ntiles;
        if (more) tile.template load<true, false>(src, t0 + Tile::BK, n, tid);
        if (active) {
#pragma unroll
            for (int sub = ts; sub < 2; sub += TS) {
                f32x16 u = zero16();
#pragma unroll
                for (int s = 0; s < NS; ++s) u = M::mma(Tile::kfrag(Ks, sub, s, col, h), wf[s], u);
                float uu[16], ph[16];
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const bool valid = t0 + sub * 32 + crow(r, h) < n;
                    uu[r] = valid ? softplus_fast<T>(u[r] + bias) : 0.f;
                    ph[r] = uu[r];
                }
#pragma unroll
                for (int pw = 0; pw < P; ++pw) {
                    if (pw > 0) {
#pragma unroll
                        for (int r = 0; r < 16; ++r) ph[r] *= uu[r];
                    }
#pragma unroll
                    for (int r = 0; r < 16; ++r) zacc[pw] += ph[r];
#pragma unroll
                    for (int t = 0; t < TPB; ++t) {
                        const typename M::frag af = M::pack(ph + t * EPL);
#pragma unroll
                        for (int db = 0; db < NDB; ++db)
                            acc[pw][db] = M::mma(af, Tile::vfrag(Vs, db * 32 + col, sub, t, h), acc[pw][db]);
                    }
                }
            }
        }
        if (more) tile.store((it & 1) ? Ks0 : Ks1, (it & 1) ? Vs0 : Vs1, tid);
        __syncthreads();
    }

    // with TS = 2, the ts = 1 wave hands its tiles to ts = 0 through LDS; then store
    float* red = reinterpret_cast<float*>(smem);  // [NJB][16 regs][64 lanes]
    float* Sp = a.Sp + ((int64_t)bh * a.G + gi) * F * D;
    float* Zp = a.Zp + ((int64_t)bh * a.G + gi) * F;
#pragma unroll
    for (int pw = 0; pw < P; ++pw) {
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
            if (TS == 2) {
                if (active && ts == 1) {
#pragma unroll
                    for (int r = 0; r < 16; ++r) red[(jb * 16 + r) * 64 + lane] = acc[pw][db][r];
                }
                __syncthreads();
            }
            if (active && ts == 0) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float v = acc[pw][db][r] + (TS == 2 ? red[(jb * 16 + r) * 64 + lane] : 0.f);
                    const int f = feat_index(jb * 32 + crow(r, h), pw + 1, Dphi, P);
                    Sp[(int64_t)f * D + db * 32 + col] = v;
                }
            }
            if (TS == 2) __syncthreads();
        }
        const float zt = zacc[pw] + other_half(zacc[pw]);
        if (TS == 2) {
            if (active && ts == 1 && h == 0) red[jb * 32 + col] = zt;
            __syncthreads();
        }
        if (active && ts == 0 && h == 0) Zp[feat_index(j, pw + 1, Dphi, P)] = zt + (TS == 2 ? red[jb * 32 + col] : 0.f);
        if (TS == 2) __syncthreads();
    }
}

template <int D, int P>
__global__ __launch_bounds__(kState16Waves * 64) void state16_kernel(const StateArgs a) {
    extern __shared__ __align__(16) unsigned char smem[];
    state16_body<D, P>(a, blockIdx.x, smem);
}

// One workgroup per (batch-head, power, 32-feature block, 32-d block) of S, plus one per
// batch-head for Z.  Each thread carries four running sums; partials are read along d
// (coalesced) and every emitted image block goes through a 32 x 32 LDS tile so that it is
// written as whole 64-byte (bf16) rows of the image, features in slot order.
__device__ inline void copy_body(const CopyArgs& a, int bx, int nbx, int bh);

template <class T>
__global__ __launch_bounds__(256) void scan_kernel(const ScanArgs a) {
    constexpr int EPL = Mfma<T>::EPL;
    constexpr int EPC = 16 / sizeof(T);      // elements per 16-byte chunk
    constexpr int CPR = 32 * sizeof(T) / 16;  // 16-byte chunks per 32-element image row
    const int Dphi = a.Dphi, P = a.P, D = a.D, F = Dphi * P, NJB = Dphi / 32, NDB = D / 32;
    const int bh = blockIdx.y, tid = threadIdx.x;
    const int nscan = P * NJB * NDB + 1;
    if (a.zero_cnt && blockIdx.x == 0 && bh == 0)
        for (int i = tid; i < a.nzero; i += 256) a.zero_cnt[i] = 0u;
    if ((int)blockIdx.x >= nscan) {
        copy_body(a.copy, blockIdx.x - nscan, a.copy_blocks, bh);
        return;
    }
    T* img = reinterpret_cast<T*>(a.simg) + (int64_t)bh * a.slots * F * D;
    float* zimg = a.zimg + (int64_t)bh * a.slots * F;
    const int nc = (a.T + a.Tc - 1) / a.Tc;
    auto ls_of = [&](int cc) {
        const int f0 = cc * a.Tc, f1 = min(f0 + a.Tc, a.T);
        return a.linear_only ? f1 : max(0, f0 - a.To);
    };

    if ((int)blockIdx.x < P * NJB * NDB) {
        __shared__ __align__(16) T tile[32][32 + EPC];  // [d][feature, slot order]
        const int blk = blockIdx.x;
        const int db = blk % NDB, jb = (blk / NDB) % NJB, pw = blk / (NDB * NJB) + 1;
        const int dl = tid % 32, jr = tid / 32;  // this thread: d = db*32 + dl, j = jb*32 + jr + 8k
        int64_t off[4];
        float acc[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            off[k] = (int64_t)feat_index(jb * 32 + jr + 8 * k, pw, Dphi, P) * D + db * 32 + dl;
            acc[k] = 0.f;
        }
        const float* base = a.Sp + (int64_t)bh * a.G * F * D;
        const int64_t stride = (int64_t)F * D;
        auto emit = [&](int slot) {
            __syncthreads();  // the previous block left the tile
#pragma unroll
            for (int k = 0; k < 4; ++k) tile[dl][slot_pos<EPL>(jr + 8 * k)] = from_float<T>(acc[k]);
            __syncthreads();
            if (tid < 32 * CPR) {
                const int row = tid / CPR, c = tid % CPR;
                T* dst = img + (int64_t)slot * F * D + ((int64_t)(pw - 1) * D + db * 32 + row) * Dphi + jb * 32 + c * EPC;
                *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(&tile[row][c * EPC]);
            }
        };
        if (a.S_state) {  // streaming: carried state + this step's frames, in frame order
            float* st = a.S_state + (int64_t)bh * F * D;
#pragma unroll
            for (int k = 0; k < 4; ++k) acc[k] = st[off[k]];
            for (int g = 0; g < a.G; ++g)
#pragma unroll
                for (int k = 0; k < 4; ++k) acc[k] += base[g * stride + off[k]];
#pragma unroll
            for (int k = 0; k < 4; ++k) st[off[k]] = acc[k];
            emit(0);
            return;
        }
        // chunk-parallel: prefix over frames; chunk c reads the prefix through frame ls(c) - 1
        int c = 0;
        while (c < nc && ls_of(c) == 0) ++c;
        for (int g = 0; g < a.G && c < nc; ++g) {
#pragma unroll
            for (int k = 0; k < 4; ++k) acc[k] += base[g * stride + off[k]];
            while (c < nc && ls_of(c) == g + 1) {
                emit(c);
                ++c;
            }
        }
        return;
    }

    // Z: [F] running sums per batch-head, image [P][Dphi] in plain feature order
    const float* zb = a.Zp + (int64_t)bh * a.G * F;
    for (int f = tid; f < F; f += 256) {
        int j, pw;
        feat_split(f, Dphi, P, j, pw);
        const int zo = (pw - 1) * Dphi + j;
        if (a.Z_state) {
            float* st = a.Z_state + (int64_t)bh * F + f;
            float acc = *st;
            for (int g = 0; g < a.G; ++g) acc += zb[(int64_t)g * F + f];
            *st = acc;
            zimg[zo] = acc;
            continue;
        }
        int c = 0;
        while (c < nc && ls_of(c) == 0) ++c;
        float acc = 0.f;
        for (int g = 0; g < a.G && c < nc; ++g) {
            acc += zb[(int64_t)g * F + f];
            while (c < nc && ls_of(c) == g + 1) {
                zimg[(int64_t)c * F + zo] = acc;
                ++c;
            }
        }
    }
}

// Workgroup bx of nbx along x (and batch-head bh) of a copy of 256 threads.
__device__ inline void copy_body(const CopyArgs& a, int bx, int nbx, int bh) {
    const int64_t frame_bytes = (int64_t)a.n * a.D * a.elem_bytes;
    const int64_t chunks = frame_bytes / 16;  // 16-byte pieces per frame
    const int64_t total = chunks * a.cnt;
    for (int64_t i = (int64_t)bx * 256 + threadIdx.x; i < total; i += (int64_t)nbx * 256) {
        const int fl = (int)(i / chunks);
        const int64_t off = (i % chunks) * 16;
        const int fs = a.f0 + fl;
        const char* sk;
        const char* sv;
        if (fs < a.nf1) {
            sk = reinterpret_cast<const char*>(a.s1k) + (bh * a.s1_bh_stride + (int64_t)fs * a.n * a.D) * a.elem_bytes;
            sv = reinterpret_cast<const char*>(a.s1v) + (bh * a.s1_bh_stride + (int64_t)fs * a.n * a.D) * a.elem_bytes;
        } else {
            sk = reinterpret_cast<const char*>(a.s2k) + (bh * a.s2_bh_stride + (int64_t)(fs - a.nf1) * a.n * a.D) * a.elem_bytes;
            sv = reinterpret_cast<const char*>(a.s2v) + (bh * a.s2_bh_stride + (int64_t)(fs - a.nf1) * a.n * a.D) * a.elem_bytes;
        }
        char* dk = reinterpret_cast<char*>(a.dk) + (bh * a.d_bh_stride + (int64_t)fl * a.n * a.D) * a.elem_bytes;
        char* dv = reinterpret_cast<char*>(a.dv) + (bh * a.d_bh_stride + (int64_t)fl * a.n * a.D) * a.elem_bytes;
        *reinterpret_cast<uint4*>(dk + off) = *reinterpret_cast<const uint4*>(sk + off);
        *reinterpret_cast<uint4*>(dv + off) = *reinterpret_cast<const uint4*>(sv + off);
    }
}

__global__ __launch_bounds__(256) void copy_kernel(const CopyArgs a) {
    copy_body(a, blockIdx.x, gridDim.x, blockIdx.y);
}

template <class T, int D, int P>
static hipError_t launch_state_t(const StateArgs& a, hipStream_t stream) {
    // bf16 takes the 16x16x32 LDS-DMA kernel, float32 the register-staged one
    constexpr bool kBf16 = sizeof(T) == 2;
    size_t lds;
    const void* fn;
    if constexpr (kBf16) {
        lds = state16_lds_bytes<D>();
        fn = reinterpret_cast<const void*>(state16_kernel<D, P>);
    } else {
        using Tile = KVTile<T, D, StateShape<P>::NW * 64>;
        const size_t kv = 2 * (size_t)(Tile::K_ELEMS + Tile::V_ELEMS) * sizeof(T);
        const size_t red = (size_t)(a.Dphi / 32) * 16 * 64 * sizeof(float);
        lds = kv > red ? kv : red;
        fn = reinterpret_cast<const void*>(state_kernel<T, D, P>);
    }
    // raise the dynamic LDS limit of this instantiation once per device (idempotent, so a
    // race between host threads only repeats the call)
    static size_t lds_set[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
    if (lds > lds_set[dev]) {
        hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
        lds_set[dev] = lds;
    }
    if constexpr (kBf16) {
        auto kfn = state16_kernel<D, P>;
        hipLaunchKernelGGL(kfn, dim3(a.BH * a.G), dim3(kState16Waves * 64), lds, stream, a);
    } else {
        auto kfn = state_kernel<T, D, P>;
        hipLaunchKernelGGL(kfn, dim3(a.BH * a.G), dim3(StateShape<P>::NW * 64), lds, stream, a);
    }
    return hipGetLastError();
}

template <class T, int D>
static hipError_t launch_state_p(const StateArgs& a, hipStream_t stream) {
    switch (a.P) {
        case 1: return launch_state_t<T, D, 1>(a, stream);
        case 2: return launch_state_t<T, D, 2>(a, stream);
        case 3: return launch_state_t<T, D, 3>(a, stream);
        case 4: return launch_state_t<T, D, 4>(a, stream);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_state(const StateArgs& a, int in_dtype, hipStream_t stream) {
    if (a.G <= 0) return hipSuccess;
    if (in_dtype == 1) {
        switch (a.D) {
            case 32: return launch_state_p<bf16, 32>(a, stream);
            case 64: return launch_state_p<bf16, 64>(a, stream);
            case 128: return launch_state_p<bf16, 128>(a, stream);
        }
    } else {
        switch (a.D) {
            case 32: return launch_state_p<float, 32>(a, stream);
            case 64: return launch_state_p<float, 64>(a, stream);
            case 128: return launch_state_p<float, 128>(a, stream);
        }
    }
    return hipErrorInvalidValue;
}

hipError_t launch_scan(const ScanArgs& a, int in_dtype, hipStream_t stream) {
    if (a.G <= 0) return hipSuccess;
    const dim3 grid((unsigned)(a.P * (a.Dphi / 32) * (a.D / 32) + 1 + a.copy_blocks), a.BH);
    if (in_dtype == 1) hipLaunchKernelGGL(scan_kernel<bf16>, grid, dim3(256), 0, stream, a);
    else hipLaunchKernelGGL(scan_kernel<float>, grid, dim3(256), 0, stream, a);
    return hipGetLastError();
}

__global__ __launch_bounds__(256) void zero_kernel(float* p, int64_t count) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < count; i += (int64_t)gridDim.x * 256) p[i] = 0.f;
}

// Clearing with a kernel rather than a memset keeps the call safe inside captured graphs.
hipError_t launch_zero(float* p, int64_t count, hipStream_t stream) {
    if (count <= 0) return hipSuccess;
    int64_t blocks = (count + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(zero_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, p, count);
    return hipGetLastError();
}

int copy_blocks(const CopyArgs& a) {
    if (a.cnt <= 0) return 0;
    const int64_t total = (int64_t)a.n * a.D * a.elem_bytes / 16 * a.cnt;
    const int64_t blocks = (total + 255) / 256;
    return blocks > 4096 ? 4096 : (int)blocks;
}

hipError_t launch_copy(const CopyArgs& a, hipStream_t stream) {
    const int blocks = copy_blocks(a);
    if (blocks <= 0) return hipSuccess;
    hipLaunchKernelGGL(copy_kernel, dim3((unsigned)blocks, a.BH), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace rehyat
