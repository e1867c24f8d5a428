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
// The dense products:
//   nt_kernel: C[i][f] = sum_d X[i][d] Y_m[f][d] for row groups that each read one matrix
//              Y_m (a head's W, a chunk's [S | -Z], a key frame's suffix R);
//   tn_kernel: per token segment, C[m][n] = sum_k X[k][m] Y[k][n] (dW and R partials);
// for fp32 inputs on the fp32 matrix core (v_mfma_f32_32x32x2f32, exact products); for
// bf16 inputs (nt16_kernel, tn16_kernel) on the bf16 matrix core with every float operand
// taken as the sum of two bf16 parts (about 2^-15 relative error per product).  Both stage
// 32-element contraction slices of their operands through LDS with 16-byte loads along rows,
// and each wave reads its MFMA operands from there (one 32x32 output block per wave);
// and every sum over segments, frames, chunks or batches runs in a fixed order, so the
// gradients are bitwise reproducible.  Fusions: the pre-activation product writes u =
// softplus(W x + b) and its powers phi (nt_store), and for bf16 inputs with P = 1, 2, 4 the
// feature gradients write dpre over u (ntf16_kernel), so dphi never reaches memory there.
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

// 1 - exp(-u) for u >= 0 (the logistic sigmoid of the pre-activation, with u its softplus): the
// hardware exp2, and below u = 1/16, where that difference would cancel, the series
// u - u^2/2 + u^3/6 - u^4/24 (truncation below 2^-26 relative there)
__device__ inline float one_minus_exp_neg(float u) {
    const float e = 1.f - __builtin_amdgcn_exp2f(-u * 1.4426950408889634f);
    const float t = u * (1.f - u * (0.5f - u * (1.f / 6.f - u * (1.f / 24.f))));
    return u < 0.0625f ? t : e;
}

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

    // Rows gathered: block row r comes from source row rowof(r).
    template <class RowOf>
    __device__ inline void load_rows(const T* src, int64_t ld, RowOf rowof, int c0, int clim) {
#pragma unroll
        for (int u = 0; u < N; ++u) {
            const int qd = threadIdx.x + 256 * u, r = qd / CPR, c = (qd % CPR) * EPC;
            if (c0 + c < clim) {
                v[u] = *reinterpret_cast<const V*>(src + (int64_t)rowof(r) * ld + c0 + c);
            } else if constexpr (sizeof(T) == 2) {
#pragma unroll
                for (int e = 0; e < 8; ++e) v[u][e] = to_bf16(0.f);
            } else {
                v[u] = make_float4(0.f, 0.f, 0.f, 0.f);
            }
        }
    }

    // As bf16 parts for the bf16 matrix core: a bf16 source as it is (into hi only), a
    // float source as hi = bf16(x) (ties to even) and lo = bf16(x - hi).
    __device__ inline void store_split(bf16* hi, bf16* lo) const {
#pragma unroll
        for (int u = 0; u < N; ++u) {
            const int qd = threadIdx.x + 256 * u, r = qd / CPR, c = (qd % CPR) * EPC;
            if constexpr (sizeof(T) == 2) {
                *reinterpret_cast<bf16x8*>(hi + r * LD + c) = v[u];
            } else {
                const float x[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
                bf16x4 wh, wl;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    wh[e] = to_bf16(x[e]);
                    wl[e] = to_bf16(x[e] - (float)wh[e]);
                }
                *reinterpret_cast<bf16x4*>(hi + r * LD + c) = wh;
                *reinterpret_cast<bf16x4*>(lo + r * LD + c) = wl;
            }
        }
    }
};

__device__ inline int part_len(int j, int Dphi, int P);

// Epilogue of the nt products: lane (col, h) holds column f of rows r0 + crow(q, h).
// FAST (bf16 inputs): the softplus of the bf16 forward (hardware exp2 / log2, softplus_fast)
// and phi stored in bf16, the precision in which the bf16 forward multiplies it; else the
// float32 feature map's log1p form and phi in float.
template <bool FAST = false>
__device__ inline void nt_store(const NtArgs& a, const GradArgs& s, int bt, float* cb, int r0, int rend, int f, int h,
                                const f32x16& acc, float add) {
    if (a.softplus) {
        // u = softplus(pre) (the form the forward of the same input type uses) and its powers
        using PT = std::conditional_t<FAST, bf16, float>;
        const int f1 = feat_index(f, 1, s.Dphi, s.P), step = part_len(f, s.Dphi, s.P);
        PT* const pb = a.phi ? reinterpret_cast<PT*>(a.phi) + (int64_t)bt * a.phi_bt_stride + f1 : nullptr;
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            const int rr = r0 + crow(q, h);
            if (rr < rend) {
                const float x = acc[q] + add;
                const float u = FAST ? softplus_fast<bf16>(x) : fmaxf(x, 0.f) + log1pf(expf(-fabsf(x)));
                cb[(int64_t)rr * a.ldc + f] = u;
                if (pb) {
                    float pw = u;
                    PT* out = pb + (int64_t)rr * s.F;
                    for (int p = 0; p < s.P; ++p) {
                        out[p * step] = (PT)pw;
                        pw *= u;
                    }
                }
            }
        }
        return;
    }
#pragma unroll
    for (int q = 0; q < 16; ++q) {
        const int rr = r0 + crow(q, h);
        if (rr < rend) {
            float* dst = cb + (int64_t)rr * a.ldc + f;
            *dst = a.accumulate ? *dst + (acc[q] + add) : acc[q] + add;
        }
    }
}

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
    nt_store(a, s, bt, cb, row0 + wr * 32, rend, f, h, acc, add);
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

// bf16 matrix-core forms of the two products, for bf16 inputs: a bf16 operand enters
// v_mfma_f32_32x32x16_bf16 as it is (exactly), a float operand as two bf16 parts,
// hi = bf16(x) and lo = bf16(x - hi), with |x - hi - lo| <= 2^-16 |x|.  A product takes
// lo*hi + hi*lo + hi*hi (the dropped lo*lo is below 2^-16 of it), so it carries about
// 2^-15 relative error where one bf16 rounding of a float operand would leave 2^-8;
// accumulation is fp32.  Three matrix-core products (one when both operands are bf16) at
// 16 times the fp32 rate.
constexpr int kLd16 = 40;  // bf16 per LDS row of a 32-element contraction slice (8 of padding)

__device__ inline f32x16 mma16(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Tile (x, y, z) of a gx x gy x gz tiling for workgroup blockIdx.x of a one-dimensional grid
// of 8 * ceil(gx gy gz / 8): workgroup g runs on XCD g % 8, and each XCD takes a contiguous
// run of tiles with x fastest, so the tiles that read the same rows (the x of one y, z)
// share an L2.  False for the padding workgroups.
__device__ inline bool xcd_tile(int gx, int gy, int gz, int& x, int& y, int& z) {
    const int total = gx * gy * gz, per = (total + 7) / 8;
    const int t = (int)(blockIdx.x % 8) * per + (int)(blockIdx.x / 8);
    if (t >= total) return false;
    x = t % gx;
    y = (t / gx) % gy;
    z = t / (gx * gy);
    return true;
}

__host__ inline unsigned xcd_grid(int64_t total) { return (unsigned)(8 * ((total + 7) / 8)); }

// C (+)= X Y^T as nt_kernel (every mode, column bias, subtracted column, accumulation),
// contraction slices of 32 staged as bf16 parts; a lane reads its 8 consecutive contraction
// slots of a row with one 16-byte LDS read.
template <class TX, class TY>
__global__ __launch_bounds__(256) void nt16_kernel(const NtArgs a, const GradArgs s) {
    constexpr bool XS = sizeof(TX) == 4, YS = sizeof(TY) == 4;  // float operands: hi and lo
    constexpr int TILE = 64 * kLd16;
    __shared__ __align__(16) bf16 xs[(XS ? 2 : 1) * TILE], ys[(YS ? 2 : 1) * TILE];
    int bx, by, bt;
    if (!xcd_tile((a.ncols + 63) / 64, a.ngroups * a.tiles_per_group, s.BH, bx, by, bt)) return;
    const int grp = by / a.tiles_per_group, t = by % a.tiles_per_group;
    const int row0 = grp * a.group_rows + t * 64;
    const int rend = min((grp + 1) * a.group_rows, a.rows);
    if (row0 >= rend) return;
    const int wave = threadIdx.x / 64, lane = threadIdx.x % 64, col = lane % 32, h = lane / 32;
    const int wr = wave / 2, wc = wave % 2;
    const int c0 = bx * 64;

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
    Slice<TX, 64, 32, kLd16> sx;
    Slice<TY, 64, 32, kLd16> sy;
    sx.load(xb, a.ldx, row0, rend, 0, a.K);
    sy.load(yb, a.ldy, c0, a.ncols, 0, a.K);
    const int xo = (wr * 32 + col) * kLd16 + h * 8, yo = (wc * 32 + col) * kLd16 + h * 8;
    for (int d0 = 0; d0 < a.K; d0 += 32) {
        __syncthreads();  // the previous slice has been read
        sx.store_split(xs, xs + TILE);
        sy.store_split(ys, ys + TILE);
        if (d0 + 32 < a.K) {  // the next slice is read while this one is multiplied
            sx.load(xb, a.ldx, row0, rend, d0 + 32, a.K);
            sy.load(yb, a.ldy, c0, a.ncols, d0 + 32, a.K);
        }
        __syncthreads();
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const bf16x8 xh = *reinterpret_cast<const bf16x8*>(xs + xo + 16 * u);
            const bf16x8 yh = *reinterpret_cast<const bf16x8*>(ys + yo + 16 * u);
            if constexpr (XS) acc = mma16(*reinterpret_cast<const bf16x8*>(xs + TILE + xo + 16 * u), yh, acc);
            if constexpr (YS) acc = mma16(xh, *reinterpret_cast<const bf16x8*>(ys + TILE + yo + 16 * u), acc);
            acc = mma16(xh, yh, acc);
        }
    }
    if (!fv) return;
    const TY* yrow = yb + (int64_t)f * a.ldy;
    float add = 0.f;
    if (a.colbias) add += a.colbias[(int64_t)(bt % s.H) * a.colbias_head_stride + f];
    if (a.sub_col >= 0) add -= load1<TY>(yrow + a.sub_col);
    nt_store<sizeof(TX) == 2 && sizeof(TY) == 2>(a, s, bt, cb, row0 + wr * 32, rend, f, h, acc, add);
}

// The feature gradients (nt modes 1 and 2) with the feature map's backward fused (blog
// 2.2.2), bf16 matrix core as nt16_kernel.  The 64 output columns of a workgroup are the
// JB = 64 / P features j0 .. j0 + JB - 1 with all P powers (column c: power c / JB + 1 of
// feature j0 + c % JB; the rows of Y are read in that order), so the epilogue holds dphi of
// every power of its features and writes, over u in C (= U [bt][N][Dphi], in place),
//   dpre[i][j] = sigmoid(pre) sum_p p u^(p-1) dphi[i][feat(j, p)],  sigmoid(pre) = 1 - exp(-u),
// with 1 - exp(-u) on the hardware exp2 (one_minus_exp_neg; phi_bwd_kernel takes expm1f);
// dphi itself is never stored.  Each output column's
// sums are those of nt16_kernel (the same dphi).  Requires every part length to
// be a multiple of JB: P = 1, 2 or 4 and Dphi a multiple of 64.
template <class TX, class TY, int P>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(sizeof(TX) == 4 ? 5 : 6))) void ntf16_kernel(const NtArgs a, const GradArgs s) {
    constexpr int JB = 64 / P, CLD = 65;
    constexpr bool XS = sizeof(TX) == 4, YS = sizeof(TY) == 4;
    constexpr int TILE = 64 * kLd16;
    // the operand slices and, once the contraction is done, the dphi tile share one LDS area
    // (fewer bytes per workgroup, more workgroups per CU)
    constexpr int XB = (XS ? 2 : 1) * TILE, YB = (YS ? 2 : 1) * TILE;
    constexpr int STAGE = (XB + YB) * (int)sizeof(bf16), CSB = 64 * CLD * (int)sizeof(float);
    __shared__ __align__(16) unsigned char lds[STAGE > CSB ? STAGE : CSB];
    bf16* const xs = reinterpret_cast<bf16*>(lds);
    bf16* const ys = xs + XB;
    float* const cs = reinterpret_cast<float*>(lds);
    int bx, by, bt;
    if (!xcd_tile(s.Dphi / JB, a.ngroups * a.tiles_per_group, s.BH, bx, by, bt)) return;
    const int grp = by / a.tiles_per_group, t = by % a.tiles_per_group;
    const int row0 = grp * a.group_rows + t * 64;
    const int rend = min((grp + 1) * a.group_rows, a.rows);
    if (row0 >= rend) return;
    const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64, col = lane % 32, h = lane / 32;
    const int wr = wave / 2, wc = wave % 2;
    const int j0 = bx * JB;
    float* const U = a.c + (int64_t)bt * a.c_bt_stride;

    int m;
    if (a.mode == 1) {
        m = bt * a.nmat + grp;
    } else {
        // earliest chunk whose linear region holds key frame grp
        int c = 0;
        while (c < a.nmat && ls_of(s, c) <= grp) ++c;
        m = c < a.nmat ? bt * a.nmat + c : -1;
    }
    if (m < 0) {
        // no chunk's state holds these keys: dphi = 0, so dpre = 0
        for (int e = tid; e < 64 * JB; e += 256) {
            const int r = e / JB, row = row0 + r;
            if (row < rend) U[(int64_t)row * a.ldc + j0 + e % JB] = 0.f;
        }
        return;
    }
    // u of the workgroup's 64 x JB outputs, read before the contraction so that its latency
    // overlaps it (each element belongs to this workgroup alone)
    // (thread tid takes column tid % JB of rows r0 + RS * i)
    constexpr int NE = 64 * JB / 256, RS = 256 / JB;
    const int ur0 = row0 + tid / JB;
    float* const ub = U + (int64_t)ur0 * a.ldc + j0 + tid % JB;
    const int64_t ustep = (int64_t)RS * a.ldc;
    float uv[NE];
#pragma unroll
    for (int i = 0; i < NE; ++i) uv[i] = ur0 + RS * i < rend ? ub[i * ustep] : 0.f;
    auto yrow = [&](int c) { return feat_index(j0 + c % JB, c / JB + 1, s.Dphi, P); };
    const TX* xb = reinterpret_cast<const TX*>(a.x) + (int64_t)bt * a.x_bt_stride;
    const TY* yb = reinterpret_cast<const TY*>(a.y) + (int64_t)m * a.y_mat_stride;
    f32x16 acc;
#pragma unroll
    for (int q = 0; q < 16; ++q) acc[q] = 0.f;
    Slice<TX, 64, 32, kLd16> sx;
    Slice<TY, 64, 32, kLd16> sy;
    sx.load(xb, a.ldx, row0, rend, 0, a.K);
    sy.load_rows(yb, a.ldy, yrow, 0, a.K);
    const int xo = (wr * 32 + col) * kLd16 + h * 8, yo = (wc * 32 + col) * kLd16 + h * 8;
    for (int d0 = 0; d0 < a.K; d0 += 32) {
        __syncthreads();  // the previous slice has been read
        sx.store_split(xs, xs + TILE);
        sy.store_split(ys, ys + TILE);
        if (d0 + 32 < a.K) {  // the next slice is read while this one is multiplied
            sx.load(xb, a.ldx, row0, rend, d0 + 32, a.K);
            sy.load_rows(yb, a.ldy, yrow, d0 + 32, a.K);
        }
        __syncthreads();
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const bf16x8 xh = *reinterpret_cast<const bf16x8*>(xs + xo + 16 * u);
            const bf16x8 yh = *reinterpret_cast<const bf16x8*>(ys + yo + 16 * u);
            if constexpr (XS) acc = mma16(*reinterpret_cast<const bf16x8*>(xs + TILE + xo + 16 * u), yh, acc);
            if constexpr (YS) acc = mma16(xh, *reinterpret_cast<const bf16x8*>(ys + TILE + yo + 16 * u), acc);
            acc = mma16(xh, yh, acc);
        }
    }
    // dphi of the tile into LDS (with the -Y[f][sub_col] term of mode 2), then dpre; the tile
    // overwrites the operand slices, so every wave must be done reading them
    const int c = wc * 32 + col;
    const float add = a.sub_col >= 0 ? -load1<TY>(yb + (int64_t)yrow(c) * a.ldy + a.sub_col) : 0.f;
    __syncthreads();
#pragma unroll
    for (int q = 0; q < 16; ++q) cs[(wr * 32 + crow(q, h)) * CLD + c] = acc[q] + add;
    __syncthreads();
    const int jj = tid % JB;
#pragma unroll
    for (int i = 0; i < NE; ++i) {
        const int r = tid / JB + RS * i;
        if (row0 + r >= rend) continue;
        const float u = uv[i];
        float du = 0.f, upow = 1.f;
#pragma unroll
        for (int p = 0; p < P; ++p) {
            du += (float)(p + 1) * upow * cs[r * CLD + p * JB + jj];
            upow *= u;
        }
        ub[i * ustep] = du * one_minus_exp_neg(u);
    }
}

// tn_kernel's segment partials with bf16 parts.  Slices of 32 contraction rows x 64 columns
// are staged row major (rows of kTrLd bf16), and a lane reads its 8 contraction slots of one
// column with the transposing LDS read, in the layout of DmaTiles<64, 4>::vfrag (column
// db * 32 + lane % 32, slot order depending only on the lane half, the same for both
// operands, so the products pair the same rows).
using TrTile = DmaTiles<64, 4>;
constexpr int kTrLd = TrTile::VLD;  // 96

template <class TX, class TY>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(6))) void tn16_kernel(const TnArgs a) {
    constexpr bool XS = sizeof(TX) == 4, YS = sizeof(TY) == 4;
    constexpr int TILE = 32 * kTrLd;
    __shared__ __align__(16) bf16 xs[(XS ? 2 : 1) * TILE], ys[(YS ? 2 : 1) * TILE];
    const int ntn = (a.ncols + 63) / 64;
    int bx, by, bt;
    if (!xcd_tile(((a.mrows + 63) / 64) * ntn, a.ngroups * a.nseg, a.BH, bx, by, bt)) return;
    const int grp = by / a.nseg, sg = by % a.nseg;
    const int wave = threadIdx.x / 64, lane = threadIdx.x % 64, col = lane % 32, h = lane / 32;
    const int wm = wave / 2, wn = wave % 2;
    const int m0 = (bx / ntn) * 64, n0 = (bx % ntn) * 64;
    const int gend = min((grp + 1) * a.group_rows, a.rows);
    const int k0 = grp * a.group_rows + sg * a.seg_rows;
    const int k1 = min(k0 + a.seg_rows, gend);
    const TX* xb = reinterpret_cast<const TX*>(a.x) + (int64_t)bt * a.x_bt_stride;
    const TY* yb = reinterpret_cast<const TY*>(a.y) + (int64_t)bt * a.y_bt_stride;
    const int vl = TrTile::vlane(lane);
    f32x16 acc;
#pragma unroll
    for (int q = 0; q < 16; ++q) acc[q] = 0.f;
    // two slices in flight: slice i + 2 is read into the registers that slice i leaves
    // (the loop is unrolled by two so that each register set keeps a fixed role)
    Slice<TX, 32, 64, kTrLd> sx0, sx1;
    Slice<TY, 32, 64, kTrLd> sy0, sy1;
    if (k0 < k1) {
        sx0.load(xb, a.ldx, k0, k1, m0, a.mrows);
        sy0.load(yb, a.ldy, k0, k1, n0, a.ncols);
    }
    if (k0 + 32 < k1) {
        sx1.load(xb, a.ldx, k0 + 32, k1, m0, a.mrows);
        sy1.load(yb, a.ldy, k0 + 32, k1, n0, a.ncols);
    }
    auto step = [&](auto& sx, auto& sy, int k) {
        __syncthreads();
        sx.store_split(xs, xs + TILE);
        sy.store_split(ys, ys + TILE);
        if (k + 64 < k1) {
            sx.load(xb, a.ldx, k + 64, k1, m0, a.mrows);
            sy.load(yb, a.ldy, k + 64, k1, n0, a.ncols);
        }
        __syncthreads();
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const bf16x8 xh = TrTile::vfrag(xs, vl, wm, 0, u), yh = TrTile::vfrag(ys, vl, wn, 0, u);
            if constexpr (XS) acc = mma16(TrTile::vfrag(xs + TILE, vl, wm, 0, u), yh, acc);
            if constexpr (YS) acc = mma16(xh, TrTile::vfrag(ys + TILE, vl, wn, 0, u), acc);
            acc = mma16(xh, yh, acc);
        }
    };
    for (int k = k0; k < k1; k += 64) {
        step(sx0, sy0, k);
        if (k + 32 < k1) step(sx1, sy1, k + 32);
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

// reduce4_kernel for short rows over many segments (E / 4 <= 64, E and the addresses
// multiples of 4 floats): one workgroup per output row; thread (g, c) adds float4 column c
// of segments [g ns / NG, (g + 1) ns / NG) of every b in order, then the NG group sums are
// added in group order (a fixed order, so the result is reproducible).
__global__ __launch_bounds__(256) void reduce_short_kernel(const float* __restrict__ part, float* __restrict__ out,
                                                           int nb, int no, int ns, int64_t E, int64_t ostride,
                                                           int accumulate) {
    __shared__ float4 gs[256];
    const int E4 = (int)(E / 4), NG = 256 / E4, t = threadIdx.x, c = t % E4, g = t / E4;
    const int o = blockIdx.x;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    if (g < NG) {
        const int s0 = (int)((int64_t)ns * g / NG), s1 = (int)((int64_t)ns * (g + 1) / NG);
        for (int b = 0; b < nb; ++b)
            for (int sg = s0; sg < s1; ++sg) {
                const float4 x = *reinterpret_cast<const float4*>(part + (((int64_t)b * no + o) * ns + sg) * E + 4 * c);
                acc.x += x.x;
                acc.y += x.y;
                acc.z += x.z;
                acc.w += x.w;
            }
    }
    gs[t] = acc;
    __syncthreads();
    if (t >= E4) return;
    float4 sum = gs[t];
    for (int k = 1; k < NG; ++k) {
        const float4 y = gs[k * E4 + t];
        sum.x += y.x;
        sum.y += y.y;
        sum.z += y.z;
        sum.w += y.w;
    }
    float4* dst = reinterpret_cast<float4*>(out + (int64_t)o * ostride + 4 * t);
    if (accumulate) {
        const float4 y = *dst;
        sum.x = y.x + sum.x;
        sum.y = y.y + sum.y;
        sum.z = y.z + sum.z;
        sum.w = y.w + sum.w;
    }
    *dst = sum;
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
// (g . o) / den | 0 ...] (D + 32 columns), and when asked, delta_i = g . o and log den_i,
// and g16 = dout rounded to bf16 (ties to even)
constexpr int kRowsPerWave = 4;

__global__ __launch_bounds__(256) void rows_kernel(const GradArgs s, const float* __restrict__ o,
                                                   const float* __restrict__ t, const float* __restrict__ dout,
                                                   const float* __restrict__ lse, const float* __restrict__ z,
                                                   float* __restrict__ AH, float* __restrict__ delta,
                                                   float* __restrict__ lden, bf16* __restrict__ g16) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const int bt = blockIdx.y, wave = threadIdx.x / 64, lane = threadIdx.x % 64;
    const int64_t i0 = ((int64_t)blockIdx.x * 4 + wave) * kRowsPerWave;
    // two adjacent columns per lane (D = 32, 64 or 128, rows 16-byte aligned): 8-byte loads
    // and 4-byte bf16 stores
    const int D = s.D, LD = D + 32, d = 2 * lane;
    f32x2 ov[kRowsPerWave], gv[kRowsPerWave];
#pragma unroll
    for (int k = 0; k < kRowsPerWave; ++k) {
        const int64_t row = (int64_t)bt * s.N + i0 + k;
        ov[k] = f32x2{0.f, 0.f};
        gv[k] = f32x2{0.f, 0.f};
        if (i0 + k < s.N && d < D) {
            ov[k] = *reinterpret_cast<const f32x2*>(o + row * D + d);
            gv[k] = *reinterpret_cast<const f32x2*>((dout ? dout : t) + row * D + d);
            if (g16) *reinterpret_cast<bf16x2*>(g16 + row * D + d) = bf16x2{to_bf16(gv[k][0]), to_bf16(gv[k][1])};
        }
    }
#pragma unroll
    for (int k = 0; k < kRowsPerWave; ++k) {
        if (i0 + k >= s.N) break;
        const int64_t row = (int64_t)bt * s.N + i0 + k;
        if (!dout) gv[k] = 2.f * (ov[k] - gv[k]);
        float dot = gv[k][0] * ov[k][0] + gv[k][1] * ov[k][1];
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
        if (d < D) *reinterpret_cast<f32x2*>(ah + d) = gv[k] * inv;
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

// Elementwise feature-map kernel: thread t of a workgroup owns element j = t % Dphi of
// rows t / Dphi, t / Dphi + per, ... (per = 256 / Dphi rows at a time, threads past
// per * Dphi idle) of the workgroup's kPhiRows rows; feature (j, p) of a row sits at
// feat(j, 1) + (p - 1) * len(part of j).
constexpr int kPhiRows = 32;
constexpr int kPhiBatch = 8;  // rows whose loads a thread issues together

__device__ inline int part_len(int j, int Dphi, int P) {
    const int q = Dphi / P, r = Dphi % P;
    return j < r * (q + 1) ? q + 1 : q;
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
    // the thread's rows in batches of kPhiBatch (every load of a batch issued before the
    // first result is needed); dphi of power p + 1 of every row of
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
hipError_t launch_nt16_t(NtArgs a, const GradArgs& s, hipStream_t stream) {
    a.tiles_per_group = (a.group_rows + 63) / 64;
    const int64_t tiles = (int64_t)((a.ncols + 63) / 64) * a.ngroups * a.tiles_per_group * s.BH;
    if (tiles >= ((int64_t)1 << 31) - 8) return hipErrorInvalidValue;
    hipLaunchKernelGGL((nt16_kernel<TX, TY>), dim3(xcd_grid(tiles)), dim3(256), 0, stream, a, s);
    return hipGetLastError();
}

template <class TX, class TY, int P>
hipError_t launch_ntf16_p(NtArgs a, const GradArgs& s, hipStream_t stream) {
    a.tiles_per_group = (a.group_rows + 63) / 64;
    const int64_t tiles = (int64_t)(s.Dphi / (64 / P)) * a.ngroups * a.tiles_per_group * s.BH;
    if (tiles >= ((int64_t)1 << 31) - 8) return hipErrorInvalidValue;
    hipLaunchKernelGGL((ntf16_kernel<TX, TY, P>), dim3(xcd_grid(tiles)), dim3(256), 0, stream, a, s);
    return hipGetLastError();
}

template <class TX, class TY>
hipError_t launch_ntf16_t(const NtArgs& a, const GradArgs& s, hipStream_t stream) {
    switch (s.P) {
        case 1: return launch_ntf16_p<TX, TY, 1>(a, s, stream);
        case 2: return launch_ntf16_p<TX, TY, 2>(a, s, stream);
        case 4: return launch_ntf16_p<TX, TY, 4>(a, s, stream);
        default: return hipErrorInvalidValue;
    }
}

template <class TX, class TY>
hipError_t launch_tn16_t(TnArgs a, int BH, hipStream_t stream) {
    const int blocks = ((a.mrows + 63) / 64) * ((a.ncols + 63) / 64);
    const int64_t tiles = (int64_t)blocks * a.ngroups * a.nseg * BH;
    if (tiles >= ((int64_t)1 << 31) - 8) return hipErrorInvalidValue;
    a.BH = BH;
    hipLaunchKernelGGL((tn16_kernel<TX, TY>), dim3(xcd_grid(tiles)), dim3(256), 0, stream, a);
    return hipGetLastError();
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

hipError_t launch_nt(const NtArgs& a, const GradArgs& s, bool x_bf16, bool y_bf16, hipStream_t stream, bool mc16) {
    if (mc16) {
        if (x_bf16 && y_bf16) return launch_nt16_t<bf16, bf16>(a, s, stream);
        if (x_bf16) return launch_nt16_t<bf16, float>(a, s, stream);
        if (y_bf16) return launch_nt16_t<float, bf16>(a, s, stream);
        return launch_nt16_t<float, float>(a, s, stream);
    }
    if (x_bf16 && y_bf16) return launch_nt_t<bf16, bf16>(a, s, stream);
    if (x_bf16) return launch_nt_t<bf16, float>(a, s, stream);
    if (y_bf16) return launch_nt_t<float, bf16>(a, s, stream);
    return launch_nt_t<float, float>(a, s, stream);
}

bool ntf16_fusable(const GradArgs& s) { return (s.P == 1 || s.P == 2 || s.P == 4) && s.Dphi % 64 == 0; }

hipError_t launch_ntf16(const NtArgs& a, const GradArgs& s, bool x_bf16, hipStream_t stream) {
    if (!ntf16_fusable(s) || (a.mode != 1 && a.mode != 2)) return hipErrorInvalidValue;
    return x_bf16 ? launch_ntf16_t<bf16, float>(a, s, stream) : launch_ntf16_t<float, float>(a, s, stream);
}

hipError_t launch_tn(const TnArgs& a, int BH, bool y_bf16, hipStream_t stream, bool mc16, bool x_bf16) {
    if (mc16 && x_bf16) return y_bf16 ? hipErrorInvalidValue : launch_tn16_t<bf16, float>(a, BH, stream);
    if (x_bf16) return hipErrorInvalidValue;
    if (mc16) return y_bf16 ? launch_tn16_t<float, bf16>(a, BH, stream) : launch_tn16_t<float, float>(a, BH, stream);
    return y_bf16 ? launch_tn_t<float, bf16>(a, BH, stream) : launch_tn_t<float, float>(a, BH, stream);
}

hipError_t launch_grad_reduce(const float* part, float* out, int nb, int no, int ns, int64_t E, hipStream_t stream,
                              int64_t out_stride, bool accumulate) {
    const int64_t os = out_stride < 0 ? E : out_stride;
    const bool v4 = E % 4 == 0 && os % 4 == 0 && reinterpret_cast<uintptr_t>(part) % 16 == 0 &&
                    reinterpret_cast<uintptr_t>(out) % 16 == 0;
    if (v4 && E / 4 <= 64 && ns >= 8)  // short rows, many segments: split the segments too
        hipLaunchKernelGGL(reduce_short_kernel, dim3((unsigned)no), dim3(256), 0, stream, part, out, nb, no, ns, E, os,
                           accumulate ? 1 : 0);
    else if (v4)
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
                            const float* z, float* AH, float* delta, float* lden, void* g16, hipStream_t stream) {
    const int per_wg = 4 * kRowsPerWave;
    if (g16 && !dout) return hipErrorInvalidValue;
    hipLaunchKernelGGL(rows_kernel, dim3((unsigned)((s.N + per_wg - 1) / per_wg), s.BH), dim3(256), 0, stream, s, o, t,
                       dout, lse, z, AH, delta, lden, reinterpret_cast<bf16*>(g16));
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
