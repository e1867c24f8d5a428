// kernels.hpp -- argument blocks and launchers shared by the host library and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rehyat {

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
    // streaming: rows of the chunk also copied after the held frames in the first segment,
    // so that the segment boundary falls on a 64-token tile boundary (the second segment
    // then starts s_pad rows into the chunk)
    int s_pad;
    // streaming, bf16: side_blocks more workgroups after the attention tiles compute the
    // state partials of side (the frames leaving the window after this chunk), on the CUs
    // the attention tiles leave free
    int side_blocks;
    StateArgs side;
    // Tail split (bf16 kernel; 0 elsewhere): the last split_per_xcd chunk-0 query tiles of
    // each XCD run as two workgroups, one per half of the window's sweep positions, which
    // exchange their partials through split_part ([split][half][wave][value][lane] floats)
    // and count their arrival in split_cnt (one per split, zero before the launch; the
    // second arrival merges and sets it back to zero).
    int split_per_xcd;
    float* split_part;
    unsigned* split_cnt;
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
    // streaming: copy_blocks more workgroups (along x, after the scan's) run the overlap
    // copy `copy`, which touches none of the scan's data
    int copy_blocks;
    CopyArgs copy;
    unsigned* zero_cnt;     // counters to set to zero on the way (the attention stage's
    int nzero;              // tail-split arrival counters), or null
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
// Tail split plan of a bf16 attention launch (sets a.split_per_xcd; returns the number of
// split tiles) and the scratch bytes of one split.
int wide_split_plan(AttnArgs& a);
size_t wide_split_part_bytes(int D);
hipError_t launch_state(const StateArgs& a, int in_dtype, hipStream_t stream);
hipError_t launch_scan(const ScanArgs& a, int in_dtype, hipStream_t stream);
hipError_t launch_copy(const CopyArgs& a, hipStream_t stream);
int copy_blocks(const CopyArgs& a);  // workgroups along x of launch_copy (0: nothing to copy)
hipError_t launch_phi(const PhiArgs& a, int in_dtype, hipStream_t stream);
hipError_t launch_zero(float* p, int64_t count, hipStream_t stream);

}  // namespace rehyat
