// grad.hip -- gradients of the attention-distillation objective with respect to the
// feature-map parameters W_q, W_k, b_q, b_k (ReHyAt blog, maplevalley.com.cn, 3.1.1: only
// phi_q and phi_k are trained, towards the frozen softmax teacher's output).
//
// With g_i = 2 (o_i - t_i) and the hybrid output o_i = num_i / den_i (blog 2.2.1), the
// derivative with respect to a linear weight kappa_ij = phi_q(q_i) . phi_k(k_j) is
// a_i . v_j - h_i, a_i = g_i / den_i, h_i = (g_i . o_i) / den_i.  Through the recurrent
// states of blog 2.3 this gives
//   dphi_q(q_i) = S_c a_i - h_i Z_c                      (state of the query's chunk),
//   dphi_k(k_j) = R v_j - r,  R = sum phi_q a^T, r = sum phi_q h over the queries of
//                 every chunk whose linear region holds k_j (a suffix over chunks),
// and the feature map (blog 2.2.2: u = softplus(W x + b), per-part powers u^p) gives
// dpre = sigmoid(pre) sum_p p u^(p-1) dphi_(j,p), dW = sum dpre x^T, db = sum dpre.
//
// The dense products run on the fp32 matrix core (v_mfma_f32_32x32x2f32) so that fp32
// and bf16 inputs share one exact-product path:
//   nt_kernel: C[i][f] = sum_d X[i][d] Y_m[f][d] for row groups that each read one matrix
//              Y_m (a head's W, a chunk's [S | -Z], a key frame's suffix R);
//   tn_kernel: per token segment, C[m][n] = sum_k X[k][m] Y[k][n] (dW and R partials);
// both stage 64 x 32 slices of their operands through LDS with 16-byte loads along rows,
// and each wave reads its MFMA operands from there (one 32x32 output block per wave);
// and every sum over segments, frames, chunks or batches runs in a fixed order, so the
// gradients are bitwise reproducible.
#include <type_traits>

#include "grad.hpp"
#include "common.hpp"
#include "dma.hpp"

namespace rehyat {

namespace {

template <class T>
__device__ inline float load1(const T* p) {
    return (float)*p;
}

__device__ inline f32x16 mma32(float a, float b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

__device__ inline int ls_of(const GradArgs& a, int c) {
    const int f0 = c * a.Tc, f1 = min(f0 + a.Tc, a.T);
    return a.linear_only ? f1 : max(0, f0 - a.To);
}

__device__ inline bf16 to_bf16(float x) { return (bf16)x; }

// One thread's share of an R x C block of a row-major source (rows [r0, r0 + R), columns
// [c0, c0 + C), zero outside rlim / clim), read as 16-byte chunks into registers and written
// to dst[r * LD + c] as DT (bf16 or float).  Reading and writing are separate steps so that a
// loop can read its next block while it multiplies the current one.
template <class T, int R, int C, int LD, class DT = bf16>
struct Slice {
    static constexpr int EPC = sizeof(T) == 2 ? 8 : 4;  // elements per 16-byte chunk
    static constexpr int CPR = C / EPC, N = R * CPR / 256;
    static_assert(R * CPR % 256 == 0, "block is not a whole number of chunks per thread");
    using V = std::conditional_t<sizeof(T) == 2, bf16x8, float4>;
    V v[N];

    __device__ inline void load(const T* src, int64_t ld, int r0, int rlim, int c0, int clim) {
#pragma unroll
        for (int u = 0; u < N; ++u) {
            const int qd = threadIdx.x + 256 * u, r = qd / CPR, c = (qd % CPR) * EPC;
            if (r0 + r < rlim && c0 + c < clim) {
                v[u] = *reinterpret_cast<const V*>(src + (int64_t)(r0 + r) * ld + c0 + c);
            } else if constexpr (sizeof(T) == 2) {
#pragma unroll
                for (int e = 0; e < 8; ++e) v[u][e] = to_bf16(0.f);
            } else {
                v[u] = make_float4(0.f, 0.f, 0.f, 0.f);
            }
        }
    }

    __device__ inline void store(DT* dst) const {
#pragma unroll
        for (int u = 0; u < N; ++u) {
            const int qd = threadIdx.x + 256 * u, r = qd / CPR, c = (qd % CPR) * EPC;
            DT* d = dst + r * LD + c;
            if constexpr (sizeof(DT) == 2 && sizeof(T) == 2) {
                *reinterpret_cast<bf16x8*>(d) = v[u];
            } else if constexpr (sizeof(DT) == 2) {
                bf16x4 w;
                w[0] = to_bf16(v[u].x);
                w[1] = to_bf16(v[u].y);
                w[2] = to_bf16(v[u].z);
                w[3] = to_bf16(v[u].w);
                *reinterpret_cast<bf16x4*>(d) = w;
            } else if constexpr (sizeof(T) == 2) {
#pragma unroll
                for (int e = 0; e < 8; ++e) d[e] = (float)v[u][e];
            } else if constexpr (LD % 4 == 0) {
                *reinterpret_cast<float4*>(d) = v[u];
            } else {
                d[0] = v[u].x;
                d[1] = v[u].y;
                d[2] = v[u].z;
                d[3] = v[u].w;
            }
        }
    }
};

// Rows [r0, r0 + 64) x columns [c0, c0 + 32) of a row-major source as float, dst[r][c] with
// row stride 33 (conflict-free column reads); rows at or past rlim and columns at or past clim
// (a multiple of 4, or of 8 for bf16) read as zero.
template <class T>
using FRowSlice = Slice<T, 64, 32, 33, float>;

// 64 rows x 64 columns per workgroup, one 32x32 block per wave; X and Y slices of 32
// contraction elements staged through LDS with coalesced 16-byte loads.
template <class TX, class TY>
__global__ __launch_bounds__(256) void nt_kernel(const NtArgs a, const GradArgs s) {
    __shared__ float xs[64 * 33], ys[64 * 33];
    const int bt = blockIdx.z;
    const int grp = blockIdx.y / a.tiles_per_group, t = blockIdx.y % a.tiles_per_group;
    const int row0 = grp * a.group_rows + t * 64;
    const int rend = min((grp + 1) * a.group_rows, a.rows);
    if (row0 >= rend) return;
    const int wave = threadIdx.x / 64, lane = threadIdx.x % 64, col = lane % 32, h = lane / 32;
    const int wr = wave / 2, wc = wave % 2;
    const int c0 = blockIdx.x * 64;

    int m;
    if (a.mode == 0) {
        m = bt % s.H;
    } else if (a.mode == 1) {
        m = bt * a.nmat + grp;
    } else if (a.mode == 3) {
        m = bt;
    } else {
        // earliest chunk whose linear region holds key frame grp
        int c = 0;
        while (c < a.nmat && ls_of(s, c) <= grp) ++c;
        m = c < a.nmat ? bt * a.nmat + c : -1;
    }
    float* cb = a.c + (int64_t)bt * a.c_bt_stride;
    const int f = c0 + wc * 32 + col;
    const bool fv = f < a.ncols;
    if (m < 0) {
        if (a.accumulate) return;
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            const int rr = row0 + wr * 32 + crow(q, h);
            if (rr < rend && fv) cb[(int64_t)rr * a.ldc + f] = 0.f;
        }
        return;
    }
    const TX* xb = reinterpret_cast<const TX*>(a.x) + (int64_t)bt * a.x_bt_stride;
    const TY* yb = reinterpret_cast<const TY*>(a.y) + (int64_t)m * a.y_mat_stride;
    f32x16 acc;
#pragma unroll
    for (int q = 0; q < 16; ++q) acc[q] = 0.f;
    FRowSlice<TX> sx;
    FRowSlice<TY> sy;
    sx.load(xb, a.ldx, row0, rend, 0, a.K);
    sy.load(yb, a.ldy, c0, a.ncols, 0, a.K);
    for (int d0 = 0; d0 < a.K; d0 += 32) {
        __syncthreads();  // the previous slice has been read
        sx.store(xs);
        sy.store(ys);
        if (d0 + 32 < a.K) {  // the next slice is read while this one is multiplied
            sx.load(xb, a.ldx, row0, rend, d0 + 32, a.K);
            sy.load(yb, a.ldy, c0, a.ncols, d0 + 32, a.K);
        }
        __syncthreads();
        const float* xr = xs + (wr * 32 + col) * 33 + h;
        const float* yr = ys + (wc * 32 + col) * 33 + h;
#pragma unroll
        for (int st = 0; st < 16; ++st) acc = mma32(xr[2 * st], yr[2 * st], acc);
    }
    if (!fv) return;
    const TY* yrow = yb + (int64_t)f * a.ldy;
    float add = 0.f;
    if (a.colbias) add += a.colbias[(int64_t)(bt % s.H) * a.colbias_head_stride + f];
    if (a.sub_col >= 0) add -= load1<TY>(yrow + a.sub_col);
#pragma unroll
    for (int q = 0; q < 16; ++q) {
        const int rr = row0 + wr * 32 + crow(q, h);
        if (rr < rend) {
            float* dst = cb + (int64_t)rr * a.ldc + f;
            *dst = a.accumulate ? *dst + (acc[q] + add) : acc[q] + add;
        }
    }
}

// Slice [k0, k0 + 32) x [c0, c0 + 64) of a row-major source as float, dst[k][c] with row
// stride 68; rows at or past klim and columns at or past clim read as zero.
template <class T>
using FColSlice = Slice<T, 32, 64, 68, float>;

// Partial C[m][n] = sum over the rows k of one segment of X[k][m] Y[k][n]: 64 x 64 outputs
// per workgroup (one 32x32 block per wave), rows staged 32 at a time through LDS; empty
// segments store zeros.
template <class TX, class TY>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(8))) void tn_kernel(const TnArgs a) {
    __shared__ __align__(16) float xs[32 * 68], ys[32 * 68];
    const int bt = blockIdx.z;
    const int grp = blockIdx.y / a.nseg, sg = blockIdx.y % a.nseg;
    const int wave = threadIdx.x / 64, lane = threadIdx.x % 64, col = lane % 32, h = lane / 32;
    const int wm = wave / 2, wn = wave % 2;
    const int ntn = (a.ncols + 63) / 64;
    const int m0 = (blockIdx.x / ntn) * 64, n0 = (blockIdx.x % ntn) * 64;
    const int gend = min((grp + 1) * a.group_rows, a.rows);
    const int k0 = grp * a.group_rows + sg * a.seg_rows;
    const int k1 = min(k0 + a.seg_rows, gend);
    const TX* xb = reinterpret_cast<const TX*>(a.x) + (int64_t)bt * a.x_bt_stride;
    const TY* yb = reinterpret_cast<const TY*>(a.y) + (int64_t)bt * a.y_bt_stride;
    f32x16 acc;
#pragma unroll
    for (int q = 0; q < 16; ++q) acc[q] = 0.f;
    FColSlice<TX> sx;
    FColSlice<TY> sy;
    if (k0 < k1) {
        sx.load(xb, a.ldx, k0, k1, m0, a.mrows);
        sy.load(yb, a.ldy, k0, k1, n0, a.ncols);
    }
    for (int k = k0; k < k1; k += 32) {
        __syncthreads();
        sx.store(xs);
        sy.store(ys);
        if (k + 32 < k1) {  // the next slice is read while this one is multiplied
            sx.load(xb, a.ldx, k + 32, k1, m0, a.mrows);
            sy.load(yb, a.ldy, k + 32, k1, n0, a.ncols);
        }
        __syncthreads();
        const float* xr = xs + h * 68 + wm * 32 + col;
        const float* yr = ys + h * 68 + wn * 32 + col;
#pragma unroll
        for (int st = 0; st < 16; ++st) acc = mma32(xr[2 * st * 68], yr[2 * st * 68], acc);
    }
    const int mm = m0 + wm * 32, nn = n0 + wn * 32;
    if (mm >= a.mrows || nn >= a.ncols) return;
    float* out = a.part + (((int64_t)bt * a.ngroups + grp) * a.nseg + sg) * a.mrows * a.ncols;
    if (nn + col >= a.ncols) return;
#pragma unroll
    for (int q = 0; q < 16; ++q) {
        const int r = mm + crow(q, h);
        if (r < a.mrows) out[(int64_t)r * a.ncols + nn + col] = acc[q];
    }
}

// bf16 matrix-core forms of the two products, for the softmax branch of the backward with
// bf16 inputs: operands rounded to bf16 (ties to even) while staged, products accumulated
// in fp32 on v_mfma_f32_32x32x16_bf16.  LDS rows hold 32 contraction elements plus 8 of
// padding; a lane reads its 8 consecutive contraction slots with one 16-byte read (the
// segment product reads transposed slices, below).
constexpr int kLd16 = 40;


// rows [r0, r0 + 64) x contraction [c0, c0 + 32) of a row-major source -> dst[r][c] (bf16)
template <class T>
using RowSlice = Slice<T, 64, 32, kLd16>;

template <class T>
__device__ inline void stage16_rows(const T* src, int64_t ld, int r0, int rlim, int c0, int clim, bf16* dst) {
    RowSlice<T> sl;
    sl.load(src, ld, r0, rlim, c0, clim);
    sl.store(dst);
}

__device__ inline f32x16 mma16(const bf16* a, const bf16* b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8*>(a),
                                                   *reinterpret_cast<const bf16x8*>(b), c, 0, 0, 0);
}

// nt_kernel on bf16 operands (modes 0, 1 and 3; no column bias or subtraction)
template <class TX, class TY>
__global__ __launch_bounds__(256) void nt16_kernel(const NtArgs a, const GradArgs s) {
    __shared__ __align__(16) bf16 xs[64 * kLd16], ys[64 * kLd16];
    const int bt = blockIdx.z;
    const int grp = blockIdx.y / a.tiles_per_group, t = blockIdx.y % a.tiles_per_group;
    const int row0 = grp * a.group_rows + t * 64;
    const int rend = min((grp + 1) * a.group_rows, a.rows);
    if (row0 >= rend) return;
    const int wave = threadIdx.x / 64, lane = threadIdx.x % 64, col = lane % 32, h = lane / 32;
    const int wr = wave / 2, wc = wave % 2;
    const int c0 = blockIdx.x * 64;
    const int m = a.mode == 0 ? bt % s.H : a.mode == 1 ? bt * a.nmat + grp : bt;
    const TX* xb = reinterpret_cast<const TX*>(a.x) + (int64_t)bt * a.x_bt_stride;
    const TY* yb = reinterpret_cast<const TY*>(a.y) + (int64_t)m * a.y_mat_stride;
    f32x16 acc;
#pragma unroll
    for (int q = 0; q < 16; ++q) acc[q] = 0.f;
    RowSlice<TX> sx;
    RowSlice<TY> sy;
    sx.load(xb, a.ldx, row0, rend, 0, a.K);
    sy.load(yb, a.ldy, c0, a.ncols, 0, a.K);
    for (int d0 = 0; d0 < a.K; d0 += 32) {
        __syncthreads();
        sx.store(xs);
        sy.store(ys);
        if (d0 + 32 < a.K) {  // the next slice is read while this one is multiplied
            sx.load(xb, a.ldx, row0, rend, d0 + 32, a.K);
            sy.load(yb, a.ldy, c0, a.ncols, d0 + 32, a.K);
        }
        __syncthreads();
        const bf16* xr = xs + (wr * 32 + col) * kLd16 + h * 8;
        const bf16* yr = ys + (wc * 32 + col) * kLd16 + h * 8;
        acc = mma16(xr, yr, acc);
        acc = mma16(xr + 16, yr + 16, acc);
    }
    const int f = c0 + wc * 32 + col;
    if (f >= a.ncols) return;
    float* cb = a.c + (int64_t)bt * a.c_bt_stride;
#pragma unroll
    for (int q = 0; q < 16; ++q) {
        const int rr = row0 + wr * 32 + crow(q, h);
        if (rr < rend) {
            float* dst = cb + (int64_t)rr * a.ldc + f;
            *dst = a.accumulate ? *dst + acc[q] : acc[q];
        }
    }
}

// The two score-shaped products of a chunk window in one pass (bf16 inputs): per 64 x 64
// tile of (query, key), S = Q K^T and dP = G V^T accumulate side by side over D, then
// P = exp(S / sqrt(D) - log den_i) and dS = P (dP - delta_i) / sqrt(D) are written as bf16
// (columns [Lk, ncols_pad) as zeros).  Q, K, V, G bf16 [rows][D].  The two output tiles go
// back through LDS so that every global store is a 16-byte run of a row.
constexpr int kSdpOutLd = 72;  // bf16 per row of a staged 64 x 64 output tile

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(8))) void sdp16_kernel(const bf16* __restrict__ q, const bf16* __restrict__ k,
                                                    const bf16* __restrict__ g, const bf16* __restrict__ v,
                                                    int64_t bt_stride, int D, int Lq, int Lk, int ncols_pad,
                                                    const float* __restrict__ lden, const float* __restrict__ delta,
                                                    int64_t stat_bt_stride, float scale, bf16* __restrict__ P,
                                                    bf16* __restrict__ dS, int64_t p_bt_stride, int ldp) {
    constexpr int TILE = 64 * kLd16, IN = 4 * TILE, OUT = 2 * 64 * kSdpOutLd;
    __shared__ __align__(16) bf16 lds[IN > OUT ? IN : OUT];
    bf16 *qs = lds, *ks = lds + TILE, *gs = lds + 2 * TILE, *vs = lds + 3 * TILE;
    const int bt = blockIdx.z, row0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
    const int wave = threadIdx.x / 64, lane = threadIdx.x % 64, col = lane % 32, h = lane / 32;
    const int wr = wave / 2, wc = wave % 2;
    const bf16* qb = q + (int64_t)bt * bt_stride;
    const bf16* kb = k + (int64_t)bt * bt_stride;
    const bf16* gb = g + (int64_t)bt * bt_stride;
    const bf16* vb = v + (int64_t)bt * bt_stride;
    f32x16 sa, pa;
#pragma unroll
    for (int r = 0; r < 16; ++r) sa[r] = pa[r] = 0.f;
    for (int d0 = 0; d0 < D; d0 += 32) {
        __syncthreads();
        stage16_rows<bf16>(qb, D, row0, Lq, d0, D, qs);
        stage16_rows<bf16>(kb, D, c0, Lk, d0, D, ks);
        stage16_rows<bf16>(gb, D, row0, Lq, d0, D, gs);
        stage16_rows<bf16>(vb, D, c0, Lk, d0, D, vs);
        __syncthreads();
        const int ao = (wr * 32 + col) * kLd16 + h * 8, bo = (wc * 32 + col) * kLd16 + h * 8;
        sa = mma16(qs + ao, ks + bo, sa);
        sa = mma16(qs + ao + 16, ks + bo + 16, sa);
        pa = mma16(gs + ao, vs + bo, pa);
        pa = mma16(gs + ao + 16, vs + bo + 16, pa);
    }
    __syncthreads();  // every wave is done with the operand tiles: reuse the LDS for the outputs
    bf16 *po = lds, *dso = lds + 64 * kSdpOutLd;
    const int fl = wc * 32 + col, f = c0 + fl;
    const bool fv = f < Lk;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int rl = wr * 32 + crow(r, h), rr = row0 + rl;
        float pr = 0.f, ds = 0.f;
        if (fv && rr < Lq) {
            pr = expf(sa[r] * scale - lden[(int64_t)bt * stat_bt_stride + rr]);
            // dS from the bf16-rounded P, as the products that consume P see it
            const float prb = (float)to_bf16(pr);
            ds = prb * (pa[r] - delta[(int64_t)bt * stat_bt_stride + rr]) * scale;
        }
        po[rl * kSdpOutLd + fl] = to_bf16(pr);
        dso[rl * kSdpOutLd + fl] = to_bf16(ds);
    }
    __syncthreads();
    bf16* pb = P + (int64_t)bt * p_bt_stride;
    bf16* db = dS + (int64_t)bt * p_bt_stride;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int qd = threadIdx.x + 256 * u, rl = qd / 8, cl = (qd % 8) * 8;  // 64 rows x 8 chunks
        // ncols_pad is a multiple of 8, so a chunk is wholly inside or wholly outside
        if (row0 + rl < Lq && c0 + cl < ncols_pad) {
            const int64_t o = (int64_t)(row0 + rl) * ldp + c0 + cl;
            *reinterpret_cast<bf16x8*>(pb + o) = *reinterpret_cast<const bf16x8*>(po + rl * kSdpOutLd + cl);
            *reinterpret_cast<bf16x8*>(db + o) = *reinterpret_cast<const bf16x8*>(dso + rl * kSdpOutLd + cl);
        }
    }
}

// tn_kernel on bf16 operands.  Slices of 32 contraction rows x 64 columns are staged row
// major (rows of kTrLd bf16), and each lane reads its 8 contraction slots of one column with
// gfx950's transposing LDS read, in the layout the forward kernel uses for its V^T operand
// (DmaTiles<64, 4>::vfrag: column db*32 + lane%32, slot order depending only on the lane
// half, identical for both operands, so the products pair the same rows).
using TrTile = DmaTiles<64, 4>;
constexpr int kTrLd = TrTile::VLD;  // 96

// contraction rows [k0, k0 + 32) x columns [c0, c0 + 64), row major (rows of kTrLd bf16)
template <class T>
using TrSlice = Slice<T, 32, 64, kTrLd>;

template <class TX, class TY>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(8))) void tn16_kernel(const TnArgs a) {
    __shared__ __align__(16) bf16 xs[32 * kTrLd], ys[32 * kTrLd];
    const int bt = blockIdx.z;
    const int grp = blockIdx.y / a.nseg, sg = blockIdx.y % a.nseg;
    const int wave = threadIdx.x / 64, lane = threadIdx.x % 64, col = lane % 32, h = lane / 32;
    const int wm = wave / 2, wn = wave % 2;
    const int ntn = (a.ncols + 63) / 64;
    const int m0 = (blockIdx.x / ntn) * 64, n0 = (blockIdx.x % ntn) * 64;
    const int gend = min((grp + 1) * a.group_rows, a.rows);
    const int k0 = grp * a.group_rows + sg * a.seg_rows;
    const int k1 = min(k0 + a.seg_rows, gend);
    const TX* xb = reinterpret_cast<const TX*>(a.x) + (int64_t)bt * a.x_bt_stride;
    const TY* yb = reinterpret_cast<const TY*>(a.y) + (int64_t)bt * a.y_bt_stride;
    const int vl = TrTile::vlane(lane);
    f32x16 acc;
#pragma unroll
    for (int q = 0; q < 16; ++q) acc[q] = 0.f;
    TrSlice<TX> sx;
    TrSlice<TY> sy;
    if (k0 < k1) {
        sx.load(xb, a.ldx, k0, k1, m0, a.mrows);
        sy.load(yb, a.ldy, k0, k1, n0, a.ncols);
    }
    for (int k = k0; k < k1; k += 32) {
        __syncthreads();
        sx.store(xs);
        sy.store(ys);
        if (k + 32 < k1) {  // the next slice is read while this one is multiplied
            sx.load(xb, a.ldx, k + 32, k1, m0, a.mrows);
            sy.load(yb, a.ldy, k + 32, k1, n0, a.ncols);
        }
        __syncthreads();
#pragma unroll
        for (int t = 0; t < 2; ++t)
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(TrTile::vfrag(xs, vl, wm, 0, t),
                                                          TrTile::vfrag(ys, vl, wn, 0, t), acc, 0, 0, 0);
    }
    const int mm = m0 + wm * 32, nn = n0 + wn * 32;
    if (mm >= a.mrows || nn + col >= a.ncols) return;
    float* out = a.part + (((int64_t)bt * a.ngroups + grp) * a.nseg + sg) * a.mrows * a.ncols;
#pragma unroll
    for (int q = 0; q < 16; ++q) {
        const int r = mm + crow(q, h);
        if (r < a.mrows) out[(int64_t)r * a.ncols + nn + col] = acc[q];
    }
}

// out[o * ostride + e] (+)= sum_{b < nb} sum_{s < ns} part[((b * no + o) * ns + s) * E + e],
// summed in that order (and then added to out when accumulating)
__global__ __launch_bounds__(256) void reduce_kernel(const float* __restrict__ part, float* __restrict__ out, int nb,
                                                     int no, int ns, int64_t E, int64_t ostride, int accumulate) {
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int o = blockIdx.y;
    if (e >= E) return;
    float acc = 0.f;
    for (int b = 0; b < nb; ++b)
        for (int s = 0; s < ns; ++s) acc += part[(((int64_t)b * no + o) * ns + s) * E + e];
    float* dst = out + (int64_t)o * ostride + e;
    *dst = accumulate ? *dst + acc : acc;
}

// reduce_kernel four elements per thread (E, ostride and both base addresses multiples of 4
// floats), each element summed in the same order
__global__ __launch_bounds__(256) void reduce4_kernel(const float* __restrict__ part, float* __restrict__ out, int nb,
                                                      int no, int ns, int64_t E, int64_t ostride, int accumulate) {
    const int64_t e = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
    const int o = blockIdx.y;
    if (e >= E) return;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int b = 0; b < nb; ++b)
        for (int s = 0; s < ns; ++s) {
            const float4 x = *reinterpret_cast<const float4*>(part + (((int64_t)b * no + o) * ns + s) * E + e);
            acc.x += x.x;
            acc.y += x.y;
            acc.z += x.z;
            acc.w += x.w;
        }
    float4* dst = reinterpret_cast<float4*>(out + (int64_t)o * ostride + e);
    if (accumulate) {
        const float4 y = *dst;
        acc.x = y.x + acc.x;
        acc.y = y.y + acc.y;
        acc.z = y.z + acc.z;
        acc.w = y.w + acc.w;
    }
    *dst = acc;
}

// R[bt][c] <- sum over c' >= c of R[bt][c'] (from the last chunk), in place
__global__ __launch_bounds__(256) void suffix_kernel(float* __restrict__ R, int nc, int64_t E) {
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (e >= E) return;
    float* base = R + (int64_t)blockIdx.y * nc * E + e;
    float acc = 0.f;
    for (int c = nc - 1; c >= 0; --c) {
        acc += base[(int64_t)c * E];
        base[(int64_t)c * E] = acc;
    }
}

// SZ[bt][c][f][d] = [S_c | -Z_c | 0] with S_c, Z_c the sums of the per-frame partials over
// frames [0, ls(c)) in frame order; chunks without a linear region get zeros.
__global__ __launch_bounds__(256) void state_sz_kernel(const GradArgs s, const float* __restrict__ Sp,
                                                       const float* __restrict__ Zp, float* __restrict__ SZ) {
    const int LD = s.D + 32, F = s.F;
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (e >= (int64_t)F * LD) return;
    const int bt = blockIdx.y, f = (int)(e / LD), d = (int)(e % LD);
    const int nc = s.nc;
    float* out = SZ + (int64_t)bt * nc * F * LD + e;
    const float* src = nullptr;
    int64_t stride = 0;
    float sign = 1.f;
    if (d < s.D) {
        src = Sp + ((int64_t)bt * s.G * F + f) * s.D + d;
        stride = (int64_t)F * s.D;
    } else if (d == s.D) {
        src = Zp + (int64_t)bt * s.G * F + f;
        stride = F;
        sign = -1.f;
    }
    float acc = 0.f;
    int g = 0;
    for (int c = 0; c < nc; ++c) {
        const int l = ls_of(s, c);
        for (; g < l && g < s.G; ++g)
            if (src) acc += src[(int64_t)g * stride];
        out[(int64_t)c * F * LD] = sign * acc;
    }
}

// Per query row (kRowsPerWave rows per wave, their loads issued together): g = dout, or
// 2 (o - t) for the distillation objective; 1/den from lse and z; AH[i] = [g / den |
// (g . o) / den | 0 ...] (D + 32 columns), and when asked, delta_i = g . o and log den_i
constexpr int kRowsPerWave = 4;

__global__ __launch_bounds__(256) void rows_kernel(const GradArgs s, const float* __restrict__ o,
                                                   const float* __restrict__ t, const float* __restrict__ dout,
                                                   const float* __restrict__ lse, const float* __restrict__ z,
                                                   float* __restrict__ AH, float* __restrict__ delta,
                                                   float* __restrict__ lden) {
    const int bt = blockIdx.y, wave = threadIdx.x / 64, lane = threadIdx.x % 64;
    const int64_t i0 = ((int64_t)blockIdx.x * 4 + wave) * kRowsPerWave;
    const int D = s.D, LD = D + 32;
    float ov[kRowsPerWave][2], gv[kRowsPerWave][2];
#pragma unroll
    for (int k = 0; k < kRowsPerWave; ++k) {
        const int64_t row = (int64_t)bt * s.N + i0 + k;
        const bool ok = i0 + k < s.N;
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int d = lane + 64 * u;
            ov[k][u] = 0.f;
            gv[k][u] = 0.f;
            if (ok && d < D) {
                ov[k][u] = o[row * D + d];
                gv[k][u] = dout ? dout[row * D + d] : t[row * D + d];
            }
        }
    }
#pragma unroll
    for (int k = 0; k < kRowsPerWave; ++k) {
        if (i0 + k >= s.N) break;
        const int64_t row = (int64_t)bt * s.N + i0 + k;
        float dot = 0.f;
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            if (!dout) gv[k][u] = 2.f * (ov[k][u] - gv[k][u]);
            dot += gv[k][u] * ov[k][u];
        }
#pragma unroll
        for (int msk = 32; msk >= 1; msk >>= 1) dot += __shfl_xor(dot, msk, 64);
        const float L = lse[row], zz = z[row];
        float inv;
        if (L == -INFINITY) {
            inv = 1.f / zz;
        } else if (zz <= 0.f || L > logf(zz)) {
            const float e = expf(-L);
            inv = e / (1.f + zz * e);
        } else {
            inv = 1.f / (zz + expf(L));
        }
        float* ah = AH + row * LD;
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int d = lane + 64 * u;
            if (d < D) ah[d] = gv[k][u] * inv;
        }
        if (lane < 32) ah[D + lane] = lane == 0 ? dot * inv : 0.f;
        if (lane == 0 && delta) {
            delta[row] = dot;
            // log(exp(L) + z), stable for either term dominating
            const float lz = zz > 0.f ? logf(zz) : -INFINITY;
            const float hi = fmaxf(L, lz), lo = fminf(L, lz);
            lden[row] = lo == -INFINITY ? hi : hi + log1pf(expf(lo - hi));
        }
    }
}

__global__ __launch_bounds__(256) void softmax_bwd_kernel(float* __restrict__ S, float* __restrict__ dP,
                                                          const float* __restrict__ lden,
                                                          const float* __restrict__ delta, int64_t stat_bt_stride,
                                                          int Lq, int Lk, int ldp, int64_t bt_stride, float scale) {
    const int bt = blockIdx.z, i = blockIdx.y;
    const int j = blockIdx.x * 256 + threadIdx.x;
    if (j >= ldp) return;
    const int64_t off = (int64_t)bt * bt_stride + (int64_t)i * ldp + j;
    if (j >= Lk) {
        S[off] = 0.f;
        dP[off] = 0.f;
        return;
    }
    const float L = lden[(int64_t)bt * stat_bt_stride + i], dl = delta[(int64_t)bt * stat_bt_stride + i];
    const float pr = expf(S[off] * scale - L);
    S[off] = pr;
    dP[off] = pr * (dP[off] - dl) * scale;
}

// 32 x 32 tiles through LDS
template <class T>
__global__ __launch_bounds__(256) void transpose_kernel(const T* __restrict__ in, int64_t in_bt_stride, int ldi,
                                                        float* __restrict__ out, int64_t out_bt_stride, int ldo,
                                                        int rows, int cols) {
    __shared__ float tile[32][33];
    const int bt = blockIdx.z, r0 = blockIdx.x * 32, c0 = blockIdx.y * 32;
    const int tx = threadIdx.x % 32, ty = threadIdx.x / 32;  // 8 rows of threads
    for (int k = ty; k < 32; k += 8) {
        const int r = r0 + k, c = c0 + tx;
        tile[k][tx] = (r < rows && c < cols) ? (float)in[(int64_t)bt * in_bt_stride + (int64_t)r * ldi + c] : 0.f;
    }
    __syncthreads();
    for (int k = ty; k < 32; k += 8) {
        const int c = c0 + k, r = r0 + tx;
        if (c < cols && r < ldo) out[(int64_t)bt * out_bt_stride + (int64_t)c * ldo + r] = tile[tx][k];
    }
}

// Elementwise feature-map kernels: thread t of a workgroup owns element j = t % Dphi of
// rows t / Dphi, t / Dphi + per, ... (per = 256 / Dphi rows at a time, threads past
// per * Dphi idle) of the workgroup's kPhiRows rows; feature (j, p) of a row sits at
// feat(j, 1) + (p - 1) * len(part of j).
constexpr int kPhiRows = 32;
constexpr int kPhiBatch = 8;  // rows whose loads a thread issues together

__device__ inline int part_len(int j, int Dphi, int P) {
    const int q = Dphi / P, r = Dphi % P;
    return j < r * (q + 1) ? q + 1 : q;
}

// u = softplus(pre) in place of pre, and phi[i][feat(j, p)] = u^p
__global__ __launch_bounds__(256) void phi_fwd_kernel(const GradArgs s, float* __restrict__ U, float* __restrict__ phi) {
    const int per = 256 / s.Dphi, t = threadIdx.x;
    if (t >= per * s.Dphi) return;
    const int j = t % s.Dphi, r_off = t / s.Dphi;
    const int f1 = feat_index(j, 1, s.Dphi, s.P), step = part_len(j, s.Dphi, s.P);
    const int64_t rows = (int64_t)s.BH * s.N;
    const int64_t r0 = (int64_t)blockIdx.x * kPhiRows;
    // the thread's rows r_off, r_off + per, ... in batches of kPhiBatch: every load of a
    // batch is issued before the first result is needed
    for (int b0 = r_off; b0 < kPhiRows; b0 += kPhiBatch * per) {
        float x[kPhiBatch];
#pragma unroll
        for (int i = 0; i < kPhiBatch; ++i) {
            const int rr = b0 + i * per;
            const int64_t row = r0 + rr;
            x[i] = rr < kPhiRows && row < rows ? U[row * s.Dphi + j] : 0.f;
        }
#pragma unroll
        for (int i = 0; i < kPhiBatch; ++i) {
            const int rr = b0 + i * per;
            const int64_t row = r0 + rr;
            if (rr >= kPhiRows || row >= rows) break;
            const float u = fmaxf(x[i], 0.f) + log1pf(expf(-fabsf(x[i])));
            U[row * s.Dphi + j] = u;
            float pw = u;
            float* out = phi + row * s.F + f1;
            for (int p = 0; p < s.P; ++p) {
                out[p * step] = pw;
                pw *= u;
            }
        }
    }
}

// dpre = sigmoid(pre) sum_p p u^(p-1) dphi[feat(j, p)], with sigmoid(pre) = 1 - exp(-u),
// in place of u
__global__ __launch_bounds__(256) void phi_bwd_kernel(const GradArgs s, float* __restrict__ U,
                                                      const float* __restrict__ dphi) {
    const int per = 256 / s.Dphi, t = threadIdx.x;
    if (t >= per * s.Dphi) return;
    const int j = t % s.Dphi, r_off = t / s.Dphi;
    const int f1 = feat_index(j, 1, s.Dphi, s.P), step = part_len(j, s.Dphi, s.P);
    const int64_t rows = (int64_t)s.BH * s.N;
    const int64_t r0 = (int64_t)blockIdx.x * kPhiRows;
    // batches of kPhiBatch rows as in phi_fwd_kernel; dphi of power p + 1 of every row of
    // the batch is loaded before any is used
    for (int b0 = r_off; b0 < kPhiRows; b0 += kPhiBatch * per) {
        float u[kPhiBatch], du[kPhiBatch], upow[kPhiBatch];
#pragma unroll
        for (int i = 0; i < kPhiBatch; ++i) {
            const int rr = b0 + i * per;
            const int64_t row = r0 + rr;
            u[i] = rr < kPhiRows && row < rows ? U[row * s.Dphi + j] : 0.f;
            du[i] = 0.f;
            upow[i] = 1.f;
        }
        for (int p = 0; p < s.P; ++p) {
            float d[kPhiBatch];
#pragma unroll
            for (int i = 0; i < kPhiBatch; ++i) {
                const int rr = b0 + i * per;
                const int64_t row = r0 + rr;
                d[i] = rr < kPhiRows && row < rows ? dphi[row * s.F + f1 + p * step] : 0.f;
            }
#pragma unroll
            for (int i = 0; i < kPhiBatch; ++i) {
                du[i] += (float)(p + 1) * upow[i] * d[i];
                upow[i] *= u[i];
            }
        }
#pragma unroll
        for (int i = 0; i < kPhiBatch; ++i) {
            const int rr = b0 + i * per;
            const int64_t row = r0 + rr;
            if (rr >= kPhiRows || row >= rows) break;
            U[row * s.Dphi + j] = du[i] * -expm1f(-u[i]);
        }
    }
}

// part[bt][sg][j] = sum over the rows of segment sg of X[row][j]: with per = 256 / cols
// (threads from per * cols on idle), thread t sums column t % cols over rows t / cols,
// t / cols + per, ... in order, and the per partial sums of a column are added in index
// order
__global__ __launch_bounds__(256) void colsum_kernel(const float* __restrict__ X, int64_t rows, int cols, int seg_rows,
                                                     float* __restrict__ part) {
    __shared__ float red[256];
    const int bt = blockIdx.y, sg = blockIdx.x, t = threadIdx.x;
    const int per = 256 / cols, j = t % cols, r_off = t / cols;
    const int64_t r0 = (int64_t)sg * seg_rows, r1 = min(r0 + seg_rows, rows);
    float acc = 0.f;
    if (r_off < per) {
        const float* xb = X + (int64_t)bt * rows * cols + j;
#pragma unroll 8
        for (int64_t r = r0 + r_off; r < r1; r += per) acc += xb[r * cols];
    }
    red[t] = acc;
    __syncthreads();
    if (t < cols) {
        float tot = 0.f;
        for (int i = 0; i < per; ++i) tot += red[i * cols + t];
        part[((int64_t)bt * gridDim.x + sg) * cols + t] = tot;
    }
}

template <class TX, class TY>
hipError_t launch_nt_t(NtArgs a, const GradArgs& s, hipStream_t stream) {
    a.tiles_per_group = (a.group_rows + 63) / 64;
    const dim3 grid((a.ncols + 63) / 64, a.ngroups * a.tiles_per_group, s.BH);
    hipLaunchKernelGGL((nt_kernel<TX, TY>), grid, dim3(256), 0, stream, a, s);
    return hipGetLastError();
}

template <class TX, class TY>
hipError_t launch_tn_t(const TnArgs& a, int BH, hipStream_t stream) {
    const int blocks = ((a.mrows + 63) / 64) * ((a.ncols + 63) / 64);
    const dim3 grid(blocks, a.ngroups * a.nseg, BH);
    hipLaunchKernelGGL((tn_kernel<TX, TY>), grid, dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_nt(const NtArgs& a, const GradArgs& s, bool x_bf16, bool y_bf16, hipStream_t stream) {
    if (x_bf16 && y_bf16) return launch_nt_t<bf16, bf16>(a, s, stream);
    if (x_bf16) return launch_nt_t<bf16, float>(a, s, stream);
    if (y_bf16) return launch_nt_t<float, bf16>(a, s, stream);
    return launch_nt_t<float, float>(a, s, stream);
}

hipError_t launch_nt16(NtArgs a, const GradArgs& s, bool x_bf16, bool y_bf16, hipStream_t stream) {
    a.tiles_per_group = (a.group_rows + 63) / 64;
    const dim3 grid((a.ncols + 63) / 64, a.ngroups * a.tiles_per_group, s.BH);
    if (x_bf16 && y_bf16)
        hipLaunchKernelGGL((nt16_kernel<bf16, bf16>), grid, dim3(256), 0, stream, a, s);
    else if (x_bf16)
        hipLaunchKernelGGL((nt16_kernel<bf16, float>), grid, dim3(256), 0, stream, a, s);
    else if (y_bf16)
        hipLaunchKernelGGL((nt16_kernel<float, bf16>), grid, dim3(256), 0, stream, a, s);
    else
        hipLaunchKernelGGL((nt16_kernel<float, float>), grid, dim3(256), 0, stream, a, s);
    return hipGetLastError();
}

hipError_t launch_tn16(const TnArgs& a, int BH, bool x_bf16, bool y_bf16, hipStream_t stream) {
    const int blocks = ((a.mrows + 63) / 64) * ((a.ncols + 63) / 64);
    const dim3 grid(blocks, a.ngroups * a.nseg, BH);
    if (x_bf16 && y_bf16)
        hipLaunchKernelGGL((tn16_kernel<bf16, bf16>), grid, dim3(256), 0, stream, a);
    else if (x_bf16)
        hipLaunchKernelGGL((tn16_kernel<bf16, float>), grid, dim3(256), 0, stream, a);
    else if (y_bf16)
        hipLaunchKernelGGL((tn16_kernel<float, bf16>), grid, dim3(256), 0, stream, a);
    else
        hipLaunchKernelGGL((tn16_kernel<float, float>), grid, dim3(256), 0, stream, a);
    return hipGetLastError();
}

__global__ __launch_bounds__(256) void to_bf16_kernel(const float* __restrict__ in, bf16* __restrict__ out,
                                                      int64_t n4) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (int64_t)gridDim.x * 256) {
        const float4 x = reinterpret_cast<const float4*>(in)[i];
        bf16x4 v;
        v[0] = to_bf16(x.x);
        v[1] = to_bf16(x.y);
        v[2] = to_bf16(x.z);
        v[3] = to_bf16(x.w);
        reinterpret_cast<bf16x4*>(out)[i] = v;
    }
}

hipError_t launch_to_bf16(const float* in, void* out, int64_t n, hipStream_t stream) {
    const int64_t n4 = n / 4;
    int64_t blocks = (n4 + 255) / 256;
    if (blocks > 8192) blocks = 8192;
    if (blocks < 1) return hipSuccess;
    hipLaunchKernelGGL(to_bf16_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, in, reinterpret_cast<bf16*>(out),
                       n4);
    return hipGetLastError();
}

hipError_t launch_sdp16(const void* q, const void* k, const void* g, const void* v, int64_t bt_stride, int D,
                        int Lq, int Lk, int ncols_pad, const float* lden, const float* delta, int64_t stat_bt_stride,
                        float scale, void* P, void* dS, int64_t p_bt_stride, int ldp, int BH, hipStream_t stream) {
    const dim3 grid((unsigned)((ncols_pad + 63) / 64), (unsigned)((Lq + 63) / 64), BH);
    hipLaunchKernelGGL(sdp16_kernel, grid, dim3(256), 0, stream, reinterpret_cast<const bf16*>(q),
                       reinterpret_cast<const bf16*>(k), reinterpret_cast<const bf16*>(g),
                       reinterpret_cast<const bf16*>(v), bt_stride, D, Lq, Lk, ncols_pad, lden, delta,
                       stat_bt_stride, scale, reinterpret_cast<bf16*>(P), reinterpret_cast<bf16*>(dS), p_bt_stride,
                       ldp);
    return hipGetLastError();
}

hipError_t launch_tn(const TnArgs& a, int BH, bool y_bf16, hipStream_t stream) {
    return y_bf16 ? launch_tn_t<float, bf16>(a, BH, stream) : launch_tn_t<float, float>(a, BH, stream);
}

hipError_t launch_grad_reduce(const float* part, float* out, int nb, int no, int ns, int64_t E, hipStream_t stream,
                              int64_t out_stride, bool accumulate) {
    const int64_t os = out_stride < 0 ? E : out_stride;
    const bool v4 = E % 4 == 0 && os % 4 == 0 && reinterpret_cast<uintptr_t>(part) % 16 == 0 &&
                    reinterpret_cast<uintptr_t>(out) % 16 == 0;
    if (v4)
        hipLaunchKernelGGL(reduce4_kernel, dim3((unsigned)((E / 4 + 255) / 256), no), dim3(256), 0, stream, part, out,
                           nb, no, ns, E, os, accumulate ? 1 : 0);
    else
        hipLaunchKernelGGL(reduce_kernel, dim3((unsigned)((E + 255) / 256), no), dim3(256), 0, stream, part, out, nb,
                           no, ns, E, os, accumulate ? 1 : 0);
    return hipGetLastError();
}

hipError_t launch_softmax_bwd(float* S, float* dP, const float* lden, const float* delta, int64_t stat_bt_stride,
                              int BH, int Lq, int Lk, int ldp, int64_t bt_stride, float scale, hipStream_t stream) {
    hipLaunchKernelGGL(softmax_bwd_kernel, dim3((unsigned)((ldp + 255) / 256), Lq, BH), dim3(256), 0, stream, S, dP,
                       lden, delta, stat_bt_stride, Lq, Lk, ldp, bt_stride, scale);
    return hipGetLastError();
}

hipError_t launch_transpose(const void* in, bool in_bf16, int64_t in_bt_stride, int ldi, float* out,
                            int64_t out_bt_stride, int ldo, int rows, int cols, int nbt, hipStream_t stream) {
    const dim3 grid((unsigned)((ldo + 31) / 32), (unsigned)((cols + 31) / 32), nbt);
    if (in_bf16)
        hipLaunchKernelGGL(transpose_kernel<bf16>, grid, dim3(256), 0, stream, reinterpret_cast<const bf16*>(in),
                           in_bt_stride, ldi, out, out_bt_stride, ldo, rows, cols);
    else
        hipLaunchKernelGGL(transpose_kernel<float>, grid, dim3(256), 0, stream, reinterpret_cast<const float*>(in),
                           in_bt_stride, ldi, out, out_bt_stride, ldo, rows, cols);
    return hipGetLastError();
}

hipError_t launch_grad_suffix(float* R, int BH, int nc, int64_t E, hipStream_t stream) {
    hipLaunchKernelGGL(suffix_kernel, dim3((unsigned)((E + 255) / 256), BH), dim3(256), 0, stream, R, nc, E);
    return hipGetLastError();
}

hipError_t launch_grad_state_sz(const GradArgs& s, const float* Sp, const float* Zp, float* SZ, hipStream_t stream) {
    const int64_t E = (int64_t)s.F * (s.D + 32);
    hipLaunchKernelGGL(state_sz_kernel, dim3((unsigned)((E + 255) / 256), s.BH), dim3(256), 0, stream, s, Sp, Zp, SZ);
    return hipGetLastError();
}

hipError_t launch_grad_rows(const GradArgs& s, const float* o, const float* t, const float* dout, const float* lse,
                            const float* z, float* AH, float* delta, float* lden, hipStream_t stream) {
    const int per_wg = 4 * kRowsPerWave;
    hipLaunchKernelGGL(rows_kernel, dim3((unsigned)((s.N + per_wg - 1) / per_wg), s.BH), dim3(256), 0, stream, s, o, t,
                       dout, lse, z, AH, delta, lden);
    return hipGetLastError();
}

hipError_t launch_grad_phi_fwd(const GradArgs& s, float* U, float* phi, hipStream_t stream) {
    const int64_t rows = (int64_t)s.BH * s.N;
    hipLaunchKernelGGL(phi_fwd_kernel, dim3((unsigned)((rows + kPhiRows - 1) / kPhiRows)), dim3(256), 0, stream, s, U,
                       phi);
    return hipGetLastError();
}

hipError_t launch_grad_phi_bwd(const GradArgs& s, float* U, const float* dphi, hipStream_t stream) {
    const int64_t rows = (int64_t)s.BH * s.N;
    hipLaunchKernelGGL(phi_bwd_kernel, dim3((unsigned)((rows + kPhiRows - 1) / kPhiRows)), dim3(256), 0, stream, s, U,
                       dphi);
    return hipGetLastError();
}

hipError_t launch_grad_colsum(const float* X, int BH, int64_t rows, int cols, int seg_rows, float* part,
                              hipStream_t stream) {
    const int nseg = (int)((rows + seg_rows - 1) / seg_rows);
    hipLaunchKernelGGL(colsum_kernel, dim3((unsigned)nseg, BH), dim3(256), 0, stream, X, rows, cols, seg_rows, part);
    return hipGetLastError();
}

}  // namespace rehyat
