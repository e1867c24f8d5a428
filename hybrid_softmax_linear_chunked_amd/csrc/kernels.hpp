// kernels.hpp -- argument blocks and launchers shared by the host library and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rehyat {

// Windowed softmax + fused linear part (attn.hip).
struct AttnArgs {
    const void* q;          // [BH, tokens_q, D] (slab stride q_bh_stride elements)
    void* out;              // same layout as q, out dtype
    int64_t q_bh_stride;
    const void* k1;         // first key/value segment (whole clip in chunk-parallel mode)
    const void* v1;
    int64_t kv1_bh_stride;
    const void* k2;         // second segment (the current chunk in streaming mode)
    const void* v2;
    int64_t kv2_bh_stride;
    // linear state of each chunk as written by the scan kernel: per slot, the image
    // [P][D][Dphi] (input dtype; phi index in 32-block operand slot order) and Z as
    // float [P][Dphi]; slot = bh * img_slots + chunk (parallel) or bh (streaming)
    const void* simg;
    const float* zimg;
    int img_slots;
    const void* wq;         // [H, Dphi, D]
    const float* bq;        // [H, Dphi] or null
    float* aux_o_soft;
    float* aux_lse;
    float* aux_y;
    float* aux_z;
    int64_t aux_bh_stride;  // tokens per slab of the aux arrays
    int H, BH, D, n, T, Tc, To, linear_only, Dphi, P;
    int stream;             // 0: all chunks of a clip; 1: one streaming chunk
    int s_frames, s_held, s_ls;
    int nchunks, tiles_per_chunk, total_tiles, per_xcd;  // grid bookkeeping (set by the launcher)
    float scale_log2;       // log2(e) / sqrt(D)
    // Tail split (bf16 chunk-parallel kernel only; 0 elsewhere): the last split_per_xcd
    // chunk-0 query tiles of each XCD run as two workgroups, one per half of the window,
    // which exchange partials through split_part ([split][half][wave][value][lane] floats)
    // and count their arrival in split_cnt (one per split, zero before the launch; the
    // second arrival merges and sets it back to zero).
    int split_per_xcd;
    float* split_part;
    unsigned* split_cnt;
    // streaming: rows of the chunk also copied after the held frames in the first segment,
    // so that the segment boundary falls on a 64-token tile boundary (the second segment
    // then starts s_pad rows into the chunk)
    int s_pad;
};

// Per-frame partials of phi_k(K)^T V and sum phi_k(K) (state.hip).
struct StateArgs {
    const void* k1;         // frames [0, nf1) of the source
    const void* v1;
    int64_t kv1_bh_stride;
    int nf1;
    const void* k2;         // frames [nf1, ..) of the source
    const void* v2;
    int64_t kv2_bh_stride;
    int g0, G;              // process source frames [g0, g0 + G)
    const void* wk;
    const float* bk;
    float* Sp;              // [BH, G, F, D]
    float* Zp;              // [BH, G, F]
    int H, BH, D, n, Dphi, P;
};

// Running sum over frame partials in frame order (state.hip).  Parallel form: the sums
// start at zero and the state image of chunk c is written once frame ls(c) - 1 has been
// added.  Streaming form: the sums start from the carried S, Z, which are written back
// together with the image of the new state.
struct ScanArgs {
    const float* Sp;        // [BH, G, F, D]
    const float* Zp;        // [BH, G, F]
    int G;
    float* S_state;         // [BH, F, D] (streaming) or null (parallel)
    float* Z_state;         // [BH, F]
    void* simg;             // images [BH, slots, P, D, Dphi]
    float* zimg;            // [BH, slots, P, Dphi]
    int slots;
    int BH, D, Dphi, P;
    int T, Tc, To, linear_only;  // chunk schedule (parallel form)
    unsigned* zero_cnt;     // counters to set to zero on the way (the attention stage's
    int nzero;              // tail-split arrival counters), or null
};

// Copy of frames [f0, f0 + cnt) of a two-segment source into dst frames [0, cnt).
struct CopyArgs {
    const void* s1k;
    const void* s1v;
    int64_t s1_bh_stride;
    int nf1;
    const void* s2k;
    const void* s2v;
    int64_t s2_bh_stride;
    void* dk;
    void* dv;
    int64_t d_bh_stride;
    int f0, cnt, BH, n, D, elem_bytes;
};

struct PhiArgs {
    const void* x;          // [BH, N, D]
    const void* w;          // [H, Dphi, D]
    const float* bias;      // [H, Dphi] or null
    void* feat;             // [BH, N, F]
    int64_t N;
    int H, BH, D, Dphi, P;
};

hipError_t launch_attn(const AttnArgs& a, int in_dtype, int out_dtype, hipStream_t stream);
hipError_t launch_attn_wide(const AttnArgs& a, int out_dtype, hipStream_t stream);
int wide_split_plan(AttnArgs& a);
size_t wide_split_part_bytes(int D);
hipError_t launch_state(const StateArgs& a, int in_dtype, hipStream_t stream);
hipError_t launch_scan(const ScanArgs& a, int in_dtype, hipStream_t stream);
hipError_t launch_copy(const CopyArgs& a, hipStream_t stream);
hipError_t launch_phi(const PhiArgs& a, int in_dtype, hipStream_t stream);
hipError_t launch_zero(float* p, int64_t count, hipStream_t stream);
// Distillation gradients (grad.hip).  Shapes and the chunk schedule of one call.
struct GradArgs {
    int H, BH, N, n, D, Dphi, P, F, T, Tc, To, linear_only, nc, G;
};

// C[bt][i][f] (+)= sum_{d < K} X[bt][i][d] Y_m[f][d] (+ colbias[h][f]) (- Y_m[f][sub_col])
// over row groups of group_rows rows (row tiles never cross a group); the matrix m of a
// group: mode 0 the head of bt, mode 1 chunk = group, mode 2 the earliest chunk whose linear
// region holds key frame = group (none: the rows get zeros, or are left as they are when
// accumulating), mode 3 the slab bt itself.  accumulate: add to C instead of storing.
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
    // bf16 product only (launch_nt16 with epi != 0): the result goes to c16 (bf16, same
    // strides as c) as epi 1: P = exp(C * scale - stat0[row]), epi 2: dS = P (C - stat1[row])
    // * scale with P read from p16 at the same position; columns [ncols, ncols_pad) get 0.
    int epi, ncols_pad;
    const float* stat0;
    const float* stat1;
    int64_t stat_bt_stride;
    float scale;
    const void* p16;
    void* c16;
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
};

hipError_t launch_nt(const NtArgs& a, const GradArgs& s, bool x_bf16, bool y_bf16, hipStream_t stream);
hipError_t launch_tn(const TnArgs& a, int BH, bool y_bf16, hipStream_t stream);
// The same products with operands rounded to bf16 and the bf16 matrix core (nt: modes 0, 1,
// 3 without colbias / sub_col; tn: float X).
hipError_t launch_nt16(NtArgs a, const GradArgs& s, bool x_bf16, bool y_bf16, hipStream_t stream);
hipError_t launch_tn16(const TnArgs& a, int BH, bool x_bf16, bool y_bf16, hipStream_t stream);
hipError_t launch_grad_reduce(const float* part, float* out, int nb, int no, int ns, int64_t E, hipStream_t stream,
                              int64_t out_stride = -1, bool accumulate = false);
hipError_t launch_grad_suffix(float* R, int BH, int nc, int64_t E, hipStream_t stream);
hipError_t launch_grad_state_sz(const GradArgs& s, const float* Sp, const float* Zp, float* SZ, hipStream_t stream);
hipError_t launch_grad_rows(const GradArgs& s, const float* o, const float* t, const float* dout, const float* lse,
                            const float* z, float* AH, float* delta, float* lden, hipStream_t stream);
// Softmax branch of the backward on one chunk window (Lq queries x Lk keys, rows of ldp
// floats, slab stride bt_stride): S (raw q.k) becomes P = exp(S / sqrt(D) - log den_i) and
// dP (G_i . v_j) becomes dS = P (dP - delta_i) / sqrt(D); columns Lk..ldp-1 become zero.
hipError_t launch_softmax_bwd(float* S, float* dP, const float* lden, const float* delta, int64_t stat_bt_stride,
                              int BH, int Lq, int Lk, int ldp, int64_t bt_stride, float scale, hipStream_t stream);
// out[bt][c][r] = in[bt][r][c] as float for r < rows, c < cols; out rows hold ldo floats and
// entries r in [rows, ldo) are set to zero.
hipError_t launch_transpose(const void* in, bool in_bf16, int64_t in_bt_stride, int ldi, float* out,
                            int64_t out_bt_stride, int ldo, int rows, int cols, int nbt, hipStream_t stream);
hipError_t launch_grad_phi_fwd(const GradArgs& s, float* U, float* phi, hipStream_t stream);
hipError_t launch_grad_phi_bwd(const GradArgs& s, float* U, const float* dphi, hipStream_t stream);
hipError_t launch_grad_colsum(const float* X, int BH, int64_t rows, int cols, int seg_rows, float* part,
                              hipStream_t stream);

// Squared distance per slab between two float tensors [BH, len] (distill.hip): partial
// holds BH * sqdist_segments(len) floats, loss BH floats; len must be a multiple of 4.
int sqdist_segments(int64_t len);
hipError_t launch_sqdist(const float* a, const float* b, int64_t len, int BH, float* partial, float* loss,
                         hipStream_t stream);

}  // namespace rehyat
