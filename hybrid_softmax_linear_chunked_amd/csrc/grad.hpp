// grad.hpp -- argument blocks and launchers of the distillation objective (distill.hip)
// and of the gradient and backward kernels (grad.hip), shared with the host library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rehyat {

// Distillation gradients (grad.hip).  Shapes and the chunk schedule of one call.
struct GradArgs {
    int H, BH, N, n, D, Dphi, P, F, T, Tc, To, linear_only, nc, G;
};

// C[bt][i][f] (+)= sum_{d < K} X[bt][i][d] Y_m[f][d] (+ colbias[h][f]) (- Y_m[f][sub_col])
// over row groups of group_rows rows (row tiles never cross a group); the matrix m of a
// group: mode 0 the head of bt, mode 1 chunk = group, mode 2 the earliest chunk whose linear
// region holds key frame = group (none: the rows get zeros, or are left as they are when
// accumulating), mode 3 the slab bt itself.  accumulate: add to C instead of storing.
// softplus (mode 0, no accumulation): C gets u = softplus(result) (the feature map's
// activation, blog 2.2.2) and, when phi is non-null, phi[bt][i][feat(f, p)] = u^p for the
// powers p = 1..P (row stride F, slab stride phi_bt_stride; bf16 elements in the bf16 matrix-
// core product nt16_kernel<bf16, bf16>, float elsewhere).
struct NtArgs {
    const void* x;
    int64_t x_bt_stride;
    int ldx;
    const void* y;
    int64_t y_mat_stride;
    int ldy;
    int nmat, mode, K, ncols, sub_col;
    const float* colbias;
    int64_t colbias_head_stride;
    float* c;
    int64_t c_bt_stride;
    int ldc;
    int rows, group_rows, ngroups, tiles_per_group;
    int accumulate;
    int softplus;
    float* phi;
    int64_t phi_bt_stride;
};

// part[bt][group][seg][m][n] = sum over the rows k of segment seg of group of X[k][m] Y[k][n]
struct TnArgs {
    const void* x;
    int64_t x_bt_stride;
    int ldx;
    const void* y;
    int64_t y_bt_stride;
    int ldy;
    int mrows, ncols;
    float* part;
    int rows, group_rows, ngroups, seg_rows, nseg;
    int BH;  // slabs (set by the bf16 launcher, which decodes its tiles from a 1-D grid)
};

// Softmax branch of the backward, flash style (bwd.hip), bf16 q, k, v and upstream gradient
// g [BH][N][D]; stats = lden [BH * N + 32] then, stat_stride floats on, delta likewise
// (natural log of each query's denominator, dout . o); dq, dk, dv [BH][N][D] float32, added to.
struct BwdArgs {
    const void* q;  // bf16
    const void* k;
    const void* v;
    const void* g;
    const float* stats;
    int64_t stat_stride;
    float* dq;
    float* dk;
    float* dv;
    int BH, N, n, T, Tc, To, linear_only, nc;
    int qtiles, kblocks;  // set by the launcher
    float scale, scale_log2;
};
hipError_t launch_bwd_softmax(BwdArgs a, int D, hipStream_t stream);

// mc16: on the bf16 matrix core, float operands as hi + lo bf16 parts (for bf16 inputs);
// otherwise on the fp32 matrix core
hipError_t launch_nt(const NtArgs& a, const GradArgs& s, bool x_bf16, bool y_bf16, hipStream_t stream,
                     bool mc16 = false);
hipError_t launch_tn(const TnArgs& a, int BH, bool y_bf16, hipStream_t stream, bool mc16 = false, bool x_bf16 = false);
// The feature gradient (mode 1 or 2, float Y) on the bf16 matrix core with the feature map's
// backward fused: a.c is U [BH][N][Dphi] (ldc = Dphi), which gets dpre in place of u.
// Only where ntf16_fusable (P = 1, 2, 4 and Dphi a multiple of 64).
bool ntf16_fusable(const GradArgs& s);
hipError_t launch_ntf16(const NtArgs& a, const GradArgs& s, bool x_bf16, hipStream_t stream);
hipError_t launch_grad_reduce(const float* part, float* out, int nb, int no, int ns, int64_t E, hipStream_t stream,
                              int64_t out_stride = -1, bool accumulate = false);
hipError_t launch_grad_suffix(float* R, int BH, int nc, int64_t E, hipStream_t stream);
hipError_t launch_grad_state_sz(const GradArgs& s, const float* Sp, const float* Zp, float* SZ, hipStream_t stream);
// g16 (optional, only with dout): receives dout rounded to bf16, [BH][N][D]
hipError_t launch_grad_rows(const GradArgs& s, const float* o, const float* t, const float* dout, const float* lse,
                            const float* z, float* AH, float* delta, float* lden, void* g16, hipStream_t stream);
// Softmax branch of the backward on one chunk window (Lq queries x Lk keys, rows of ldp
// floats, slab stride bt_stride): S (raw q.k) becomes P = exp(S / sqrt(D) - log den_i) and
// dP (G_i . v_j) becomes dS = P (dP - delta_i) / sqrt(D); columns Lk..ldp-1 become zero.
hipError_t launch_softmax_bwd(float* S, float* dP, const float* lden, const float* delta, int64_t stat_bt_stride,
                              int BH, int Lq, int Lk, int ldp, int64_t bt_stride, float scale, hipStream_t stream);
// out[bt][c][r] = in[bt][r][c] as float for r < rows, c < cols; out rows hold ldo floats and
// entries r in [rows, ldo) are set to zero.
hipError_t launch_transpose(const void* in, bool in_bf16, int64_t in_bt_stride, int ldi, float* out,
                            int64_t out_bt_stride, int ldo, int rows, int cols, int nbt, hipStream_t stream);
hipError_t launch_grad_phi_bwd(const GradArgs& s, float* U, const float* dphi, hipStream_t stream);
hipError_t launch_grad_colsum(const float* X, int BH, int64_t rows, int cols, int seg_rows, float* part,
                              hipStream_t stream);

// Squared distance per slab between two float tensors [BH, len] (distill.hip): partial
// holds BH * sqdist_segments(len) floats, loss BH floats; len must be a multiple of 4.
int sqdist_segments(int64_t len);
hipError_t launch_sqdist(const float* a, const float* b, int64_t len, int BH, float* partial, float* loss,
                         hipStream_t stream);

}  // namespace rehyat
