// attn_wide.hip -- bf16 windowed softmax tile kernel, 32 queries per wave, with the linear
// part and the shared normalisation fused into its epilogue (ReHyAt blog,
// maplevalley.com.cn, sections 2.2.1-2.3).
//
// One workgroup = 8 waves x 32 queries of one chunk of one (batch, head): two waves per
// SIMD, so that while one wave runs the softmax of a sub-step on the vector ALU (and its
// LDS operand reads and tile copies), the other keeps the matrix core busy.  A single wave
// per SIMD issues one instruction at a time, and the softmax, operand reads and copies of a
// 64-query wave do not fit in the shadow of its own products (measured on this part: 0.56
// to 0.71 of the MFMA rate for one wave, 0.9 for two).  The 8 waves share one ring of K/V
// tiles, so the HBM and LDS-write traffic per query is that of the 4-wave layout; each K or
// V operand read from LDS now feeds one product, which the LDS read rate (256 B/clk per CU)
// carries at half load.
//
// The window is swept in 32-token sub-steps.  Sub-step u runs
//   (a) S_{u+1}^T = K_{u+1} Q^T          on the matrix core (scores one sub-step ahead),
//   (b) softmax of S_u^T -> P_u           on the vector ALU, interleaved with (a),
//   (c) O^T += V_u^T P_u^T                on the matrix core.
// K and V reach LDS in 64-token tiles by LDS-DMA, two tiles ahead of their use: K in a ring
// of four slots (the look-ahead of (a) reaches into the next tile), V in three.  The tile
// holding the ragged end of the window is swept first, so the steady-state loop sees full
// tiles only and carries no masking.
//
// Softmax reference: scores are taken in the log2 domain against one fixed reference per
// query, the maximum of its first sub-step, so p = exp2(s*log2(e)/sqrt(D) - m) and O is
// never rescaled.  Any fixed m gives the exact result, because the final normalisation
// uses the same m; the only risk is range.  The row sum bounds every p, so a sum above
// 2^64 (or an infinite one) sends the workgroup through a second pass whose reference is
// the exact row maximum, found by a score-only sweep over the window.  Row sums add the
// fp32 weights with plain adds (the packed bf16 dot product runs on the matrix pipe and
// stalls behind the products); the value product takes the same weights rounded to bf16.
#include <type_traits>

#include "attn_common.hpp"
#include "dma.hpp"
#include "state16.hpp"

namespace rehyat {

static constexpr float kWideSumLimit = 18446744073709551616.0f;  // 2^64

// Workgroup layout of the wide kernel: waves, and 32-query blocks per wave.
static constexpr int kWideWaves = 8, kWideQB = 1;

// The sweep as scheduled assembly (generated, wide_substep.inc).  sa / sb hold the scores of
// the current and of the next sub-step (PAR picks which is current), o the unnormalised O^T
// accumulators, q the Q operands, k the K operands of the next scores (read one sub-step
// ahead), vf the V^T operands, pf the bf16 weights, lsum the row sum, m the reference of the
// exponent (log2 domain), sc the score scale (log2(e)/sqrt(D)).  Sub-steps are pipelined: the
// value products of the second key half of a sub-step run in the next one.
// wide_pipe: one sub-step at the given V^T / K read addresses (FIRST: none deferred from a
// previous one).  wide_flush: the deferred products of the last sub-step.  wide_loop: sweep
// positions i0 .. iend-1 (ring slots counted from position i0 - 1) with the copy of K tile i+3
// and V tile i+2 into the rings at LDS byte addresses kring / vring, lane read offsets klane /
// vlane.  The copies start at tokens kt0 / vt0 of the window (64 more per position, held at the
// last tile's ktl; a streaming window's tiles come from segment 1 below token len1, else from
// segment 2); this wave copies 1 KB chunks to kcr[j] / vcr[j] (ring plus chunk offset) from its
// lane offsets koff[j] / voff[j], the last under kmask / vmask where waves issue unequal counts.
#define WIDE_PIPE_ARGS(D)                                                                           \
    f32x16 &sa, f32x16 &sb, f32x16(&o)[D / 32][1], const bf16x8(&q)[1][D / 16], bf16x8(&k)[D / 16], \
        bf16x8(&vf)[D / 16], bf16x8(&pf)[2], float &lsum, float m, float sc, uint32_t vaddr, uint32_t kaddr
#define WIDE_FLUSH_ARGS(D)                                                                          \
    f32x16 &sa, f32x16 &sb, f32x16(&o)[D / 32][1], bf16x8(&k)[D / 16], bf16x8(&vf)[D / 16], bf16x8(&pf)[2]
#define WIDE_LOOP_ARGS(D)                                                                                        \
    f32x16 &sa, f32x16 &sb, f32x16(&o)[D / 32][1], const bf16x8(&q)[1][D / 16], bf16x8(&k)[D / 16],              \
        bf16x8(&vf)[D / 16], bf16x8(&pf)[2], float &lsum, float m, float sc, int i0, int iend, int kt0, int vt0,   \
        int ktl, int len1, const void *k1, const void *v1, const void *k2, const void *v2, uint32_t kring,           \
        uint32_t vring, uint32_t klane, uint32_t vlane, const uint32_t(&kcr)[3], const uint32_t(&vcr)[3],            \
        const uint32_t(&koff)[3], const uint32_t(&voff)[3], uint64_t kmask, uint64_t vmask
template <int D, int PAR, bool FIRST>
__device__ inline void wide_pipe(WIDE_PIPE_ARGS(D));
template <int D>
__device__ inline void wide_flush(WIDE_FLUSH_ARGS(D));
template <int D, bool STREAM>
__device__ inline void wide_loop(WIDE_LOOP_ARGS(D));
// Wait states between the last product of a sweep and compiler code reading S or O.
template <int D>
__device__ inline void wide_guard(f32x16& sa, f32x16& sb, f32x16 (&o)[D / 32][1]);
#include "wide_substep.inc"

// This wave's part of the copy of a 64-token tile: LDS byte offsets of its 1 KB chunks
// (a missing last one gets a valid address), lane byte offsets, and the exec mask of the last.
template <int NI, int PW, int NW>
__device__ inline void copy_share(int wave, const uint32_t (&off)[PW], uint32_t (&c)[3], uint32_t (&o)[3], uint64_t& mask) {
    static_assert(PW <= 3, "more than three copy instructions per wave");
#pragma unroll
    for (int j = 0; j < 3; ++j) {
        c[j] = __builtin_amdgcn_readfirstlane((uint32_t)min(wave + j * NW, NI - 1) * 1024u);
        o[j] = j < PW ? off[j] * (uint32_t)sizeof(bf16) : 0u;
    }
    const bool on = wave + (PW - 1) * NW < NI;
    mask = __builtin_amdgcn_read_exec() & (0ull - (uint64_t)on);
}

// LDS bytes of the one-shot epilogue staging: W_q [Dphi][D + 8], the P powers of the state
// image [P][D][Dphi + 8] (bf16) and Z [P][Dphi] (fp32).
__host__ __device__ inline size_t wide_epilogue_lds_bytes(int D, int Dphi, int P) {
    return ((size_t)Dphi * (D + 8) + (size_t)P * D * (Dphi + 8)) * 2 + (size_t)P * Dphi * 4;
}

// rows x row_bytes (rows contiguous in HBM, row_bytes a multiple of 16) into LDS at dst,
// followed by 16 bytes of padding per row if pad, by LDS-DMA over the NW waves
template <int NW>
__device__ inline void dma_rows(const void* src, int rows, int row_bytes, bool pad, unsigned char* dst, int wave,
                                int lane) {
    const int dch = row_bytes / 16, cpr = dch + (pad ? 1 : 0), nch = rows * cpr;
    // chunk q = 64 j + lane of this wave's j = wave, wave + NW, ...: (row, c) = divmod(q, cpr),
    // stepped by NW * 64 chunks without further divisions
    int q = wave * 64 + lane, row = q / cpr, c = q % cpr;
    const int step_r = NW * 64 / cpr, step_c = NW * 64 % cpr;
    for (int j = wave; j * 64 < nch; j += NW) {
        if (q < nch) dma16_s(src, (uint32_t)(row * row_bytes + (c < dch ? c : 0) * 16), lds_addr(dst + j * 1024));
        q += NW * 64;
        row += step_r;
        c += step_c;
        if (c >= cpr) {
            c -= cpr;
            ++row;
        }
    }
}

// LDS bytes of the output staging of wide_merge_store: per wave 32 rows of D + 16 bytes.
template <class OT, int D>
constexpr size_t wide_out_stage_bytes() {
    return (size_t)kWideWaves * 32 * (D + 16 / sizeof(OT)) * sizeof(OT);
}

// Merge (ReHyAt blog, maplevalley.com.cn, 2.3: out = (2^m O + y) / (2^m l + z), both
// scaled by 2^-max(m, 0)) and store the 32 query rows from r0 of this wave.  The values of
// a row sit in lane (row % 32, h) of the C layout, 4 consecutive d per 16 bytes of output,
// so they go through LDS (this wave's 32 rows, padded) and leave as whole rows: each store
// instruction writes 1 KB of contiguous output.  Partial row writes from every lane took
// tens of microseconds to drain at the end of a workgroup.  Every wave must be done with
// the LDS contents before the call (the barrier below also covers the sweep's last copies,
// once this wave has waited for them).  Aux outputs keep the per-lane path.
template <class OT, int D>
__device__ inline void wide_merge_store(const AttnArgs& a, const Window<bf16>& w, unsigned char* smem, int r0,
                                        int wave, bool has_soft, bool has_lin, const f32x16 (&oacc)[D / 32][kWideQB],
                                        int qb, const f32x16 (&yacc)[D / 32], float m_run, float l_tot, float zq) {
    constexpr int NDB = D / 32, EV = 16 / sizeof(OT), SROW = D + EV, CPR = D / EV;
    const int lane = threadIdx.x % 64, col = lane % 32, h = lane / 32;
    float ca, cg;
    if (has_soft && has_lin) {
        const float M2 = fmaxf(m_run, 0.f);
        const float ea = __builtin_amdgcn_exp2f(m_run - M2);
        const float eg = __builtin_amdgcn_exp2f(-M2);
        const float inv = 1.f / (ea * l_tot + eg * zq);
        ca = ea * inv;
        cg = eg * inv;
    } else if (has_soft) {
        ca = 1.f / l_tot;
        cg = 0.f;
    } else {
        ca = 0.f;
        cg = 1.f / zq;
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's LDS-DMA copies have landed
    __syncthreads();
    OT* st = reinterpret_cast<OT*>(smem) + wave * 32 * SROW;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int d = db * 32 + g * 8 + h * 4;
            float v[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) v[i] = ca * oacc[db][qb][g * 4 + i] + cg * yacc[db][g * 4 + i];
            if constexpr (sizeof(OT) == 4) {
                *reinterpret_cast<float4*>(st + col * SROW + d) = make_float4(v[0], v[1], v[2], v[3]);
            } else {
                bf16x4 o4;
#pragma unroll
                for (int i = 0; i < 4; ++i) o4[i] = (bf16)v[i];
                *reinterpret_cast<bf16x4*>(st + col * SROW + d) = o4;
            }
        }
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the whole wave's rows are in LDS
    __builtin_amdgcn_wave_barrier();
    OT* outs = reinterpret_cast<OT*>(a.out) + (int64_t)w.bh * a.q_bh_stride + (int64_t)w.q0 * D;
#pragma unroll
    for (int it = 0; it < 32 * CPR / 64; ++it) {
        const int c = it * 64 + lane, r = c / CPR, ch = c % CPR;
        if (r0 + r < w.Lq)
            *reinterpret_cast<uint4*>(outs + (int64_t)(r0 + r) * D + ch * EV) =
                *reinterpret_cast<const uint4*>(st + r * SROW + ch * EV);
    }
    if (a.aux_o_soft || a.aux_y || a.aux_lse || a.aux_z)
        merge_store_block<bf16, OT, D>(a, w, r0 + col, has_soft, has_lin, oacc, qb, yacc, m_run, l_tot, zq, false);
}

// Epilogue of the wide kernel when everything it reads fits in LDS at once (ReHyAt blog,
// maplevalley.com.cn, 2.2.2-2.3): W_q, every power of the chunk's state image and Z are
// staged by one round of LDS-DMA behind a single barrier, then each 32-query block computes
// u = W_q q on MFMA from the Q operand registers, phi = per-part powers of softplus(u + b),
// y = sum over powers of S_c^T phi on MFMA (phi straight from the u registers),
// z = phi . Z_c, and merges with its softmax part.
template <class OT, int D, int NW, int QB>
__device__ inline void wide_linear_and_merge(const AttnArgs& a, const Window<bf16>& w, unsigned char* smem, int qw,
                                             int wave, bool has_soft, bool has_lin,
                                             const bf16x8 (&qf)[QB][D / 16], const f32x16 (&oacc)[D / 32][QB],
                                             const float (&m_ref)[QB], const float (&l_tot)[QB]) {
    using T = bf16;
    using M = Mfma<T>;
    constexpr int KS = M::KS, EPL = M::EPL, NS = D / KS, NDB = D / 32, TPB = 16 / EPL;
    const int lane = threadIdx.x % 64, col = lane % 32, h = lane / 32;
    const int Dphi = a.Dphi, P = a.P, NJB = Dphi / 32;
    constexpr int WLD = D + 8;
    const int SLD = Dphi + 8;
    T* Ws = reinterpret_cast<T*>(smem);
    T* Ss = Ws + Dphi * WLD;
    float* Zs = reinterpret_cast<float*>(Ss + P * D * SLD);
    const float* bq = a.bq ? a.bq + (int64_t)w.hh * Dphi : nullptr;

    if (has_lin) {
        __syncthreads();  // every wave is done with the K/V tiles
        dma_rows<NW>(reinterpret_cast<const T*>(a.wq) + (int64_t)w.hh * Dphi * D, Dphi, D * 2, true,
                     reinterpret_cast<unsigned char*>(Ws), wave, lane);
        dma_rows<NW>(reinterpret_cast<const T*>(a.simg) + (int64_t)w.img_slot * P * D * Dphi, P * D, Dphi * 2, true,
                     reinterpret_cast<unsigned char*>(Ss), wave, lane);
        dma_rows<NW>(a.zimg + (int64_t)w.img_slot * P * Dphi, 1, P * Dphi * 4, false,
                     reinterpret_cast<unsigned char*>(Zs), wave, lane);
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
        __syncthreads();
    }
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        f32x16 yacc[NDB];
#pragma unroll
        for (int db = 0; db < NDB; ++db) yacc[db] = zero16();
        float zq = 0.f;
        if (has_lin) {
            // one 32-feature block at a time, every power of it (all powers are staged), so
            // only that block's u and phi are live
            constexpr int JBMAX = 4;  // Dphi <= 128
#pragma unroll
            for (int jb = 0; jb < JBMAX; ++jb) {
                if (jb >= NJB) break;
                f32x16 u = M::mma(M::load(Ws + (jb * 32 + col) * WLD + h * EPL), qf[qb][0], zero16());
#pragma unroll
                for (int st = 1; st < NS; ++st) u = M::mma(M::load(Ws + (jb * 32 + col) * WLD + st * KS + h * EPL), qf[qb][st], u);
                float bb[16];  // rows crow(4 g + i, h) are 4 consecutive features; biases are only 4-byte aligned
#pragma unroll
                for (int r = 0; r < 16; ++r) bb[r] = 0.f;
                if (bq) {
#pragma unroll
                    for (int r = 0; r < 16; ++r) bb[r] = bq[jb * 32 + crow(r, h)];
                }
                float uu[16], ph[16];
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    uu[r] = softplus_fast<T>(u[r] + bb[r]);
                    ph[r] = uu[r];
                }
                for (int pw = 1; pw <= P; ++pw) {
                    if (pw > 1) {
#pragma unroll
                        for (int r = 0; r < 16; ++r) ph[r] *= uu[r];
                    }
                    const float* zp = Zs + (pw - 1) * Dphi + jb * 32 + h * 4;
#pragma unroll
                    for (int g4 = 0; g4 < 4; ++g4) {
                        const float4 z4 = *reinterpret_cast<const float4*>(zp + g4 * 8);
                        zq += ph[g4 * 4 + 0] * z4.x + ph[g4 * 4 + 1] * z4.y + ph[g4 * 4 + 2] * z4.z + ph[g4 * 4 + 3] * z4.w;
                    }
                    const T* Sp = Ss + (pw - 1) * D * SLD;
#pragma unroll
                    for (int t = 0; t < TPB; ++t) {
                        const typename M::frag bfr = M::pack(ph + t * EPL);
#pragma unroll
                        for (int db = 0; db < NDB; ++db) {
                            const typename M::frag sf = M::load(Sp + (db * 32 + col) * SLD + jb * 32 + t * 2 * EPL + h * EPL);
                            yacc[db] = M::mma(sf, bfr, yacc[db]);
                        }
                    }
                }
            }
            zq += other_half(zq);
        }
        wide_merge_store<OT, D>(a, w, smem, qw + qb * 32, wave, has_soft, has_lin, oacc, qb, yacc, m_ref[qb], l_tot[qb], zq);
    }
}

template <class OT, int D, bool STREAM, bool EPI_ALL>
__global__ __launch_bounds__(kWideWaves * 64, 1) void attn_wide_kernel(const AttnArgs a) {
    using T = bf16;
    using M = Mfma<T>;
    constexpr int QB = kWideQB, NW = kWideWaves, NT = NW * 64, BQ = NW * QB * 32;
    using Tile = DmaTiles<D, NW>;
    constexpr int KS = M::KS, EPL = M::EPL, NS = D / KS, NDB = D / 32;
    constexpr int TPB = 32 / KS;  // value-product steps per 32-token sub-step
    constexpr int BK = Tile::BK;
    constexpr int PWMAX = Tile::PWK > Tile::PWV ? Tile::PWK : Tile::PWV;
    static_assert(PWMAX <= TPB * NDB, "a sub-step has fewer product pairs than copy instructions");

    extern __shared__ __align__(16) unsigned char smem[];
    T* const kring = reinterpret_cast<T*>(smem);
    T* const vring = kring + 4 * Tile::K_ELEMS;

    if constexpr (STREAM) {
        // workgroups after the attention tiles: state partials of the frames that leave the
        // window (placed last, so they take the CUs the tiles leave free)
        const int side = (int)blockIdx.x - 8 * a.per_xcd;
        if (side >= 0) {
            if (side < a.side_blocks) state16_any_p<D>(a.side, side, smem);
            return;
        }
    }
    Window<T> w;
    if (!decode_window<T, D, STREAM>(a, w)) return;
    // the decode divides by run-time values on the vector ALU; state that every field is
    // uniform, so that the fields sit in scalar registers instead of vector registers that
    // the sweep would push out to scratch
    {
        auto u = [](int& x) { x = __builtin_amdgcn_readfirstlane(x); };
        u(w.bh); u(w.hh); u(w.c); u(w.qt); u(w.q0); u(w.Lq); u(w.Lk); u(w.ls); u(w.img_slot);
        u(w.src.len1); u(w.split); u(w.half);
        w.src.k1 = static_cast<const T*>(uniform_ptr(w.src.k1));
        w.src.v1 = static_cast<const T*>(uniform_ptr(w.src.v1));
        w.src.k2 = static_cast<const T*>(uniform_ptr(w.src.k2));
        w.src.v2 = static_cast<const T*>(uniform_ptr(w.src.v2));
    }
    if (w.qt * BQ >= w.Lq) return;
    const int Lk = w.Lk;
    const bool has_lin = w.ls > 0;
    const bool has_soft = Lk > 0;

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid / 64);  // wave-uniform
    __builtin_assume(wave >= 0 && wave < NW);
    const int lane = tid % 64, col = lane % 32, h = lane / 32;
    const int qw = w.qt * BQ + wave * QB * 32;
    const bool wave_live = qw < w.Lq;
    const T* qs = reinterpret_cast<const T*>(a.q) + (int64_t)w.bh * a.q_bh_stride + (int64_t)w.q0 * D;

    typename M::frag qf[QB][NS];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const int row = qw + qb * 32 + col;
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            if (row < w.Lq) {
                qf[qb][s] = M::load(qs + (int64_t)row * D + s * KS + h * EPL);
            } else {
                float zz[EPL];
#pragma unroll
                for (int e = 0; e < EPL; ++e) zz[e] = 0.f;
                qf[qb][s] = M::pack(zz);
            }
        }
    }

    const float sc = a.scale_log2;
    const int nt = (Lk + BK - 1) / BK;    // 64-token tiles
    // sweep positions [p0, p1) of this workgroup: all, or one half of a split tile's window
    int p0 = 0, p1 = nt;
    if (w.split >= 0) {
        const int hp = (nt + 1) / 2;
        if (w.half == 0) p1 = hp;
        else p0 = hp;
    }
    const bool ragged = Lk % BK != 0;
    // Tiles are processed last one first: position i of the sweep holds window tile
    // tile_of(i), so the only ragged tile (and the masking it needs) comes before the
    // steady-state loop, which then sees full tiles only.  The softmax sums over keys, so
    // the order is free.
    auto tile_of = [&](int i) { return i == 0 ? nt - 1 : i - 1; };
    const int last_len = Lk - (nt - 1) * BK;  // valid keys of the last tile, 1..64
    // valid keys of sweep sub-step u (two per tile): 32 except in the last tile
    auto key_limit = [&](int u) {
        if (u >= 2) return 32;
        return u == 0 ? min(32, last_len) : max(0, last_len - 32);
    };
    Tile tile;
    tile.init(wave, lane);
    const int vl = Tile::vlane(lane);

    // ring slots count from the first sweep position p0 of this workgroup (the sweep loop has
    // them at fixed offsets)
    auto kslot = [&](int t) { return kring + ((t - p0) & 3) * Tile::K_ELEMS; };
    auto vslot = [&](int t) { return vring + ((t - p0) & 3) * Tile::V_ELEMS; };
    // start the DMA of the K / V tile at sweep position i into the given slot (completion:
    // vmcnt + barrier)
    auto dma_k = [&](int i, T* dst) {
        const int t = tile_of(i);
        if (ragged && i == 0) tile.template issue_k<true, STREAM>(w.src, t * BK, Lk, dst, wave);
        else tile.template issue_k<false, STREAM>(w.src, t * BK, Lk, dst, wave);
    };
    auto dma_v = [&](int i, T* dst) {
        const int t = tile_of(i);
        if (ragged && i == 0) tile.template issue_v<true, STREAM>(w.src, t * BK, Lk, dst, wave);
        else tile.template issue_v<false, STREAM>(w.src, t * BK, Lk, dst, wave);
    };
    // DMA writes of this wave complete, then every wave's are visible
    auto dma_sync = [&]() {
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
        __syncthreads();
    };
    // End of a sweep position: the DMA batch issued one position earlier is complete in every
    // wave.  Vector memory operations complete in issue order, so a wave waits until no more
    // than the batch it issued in this position (counted for the wave with the fewest DMA
    // instructions) is outstanding.  LDS reads need no wait here: after the barrier of
    // position i, the next batch overwrites the K slot of tile i (read in position i-1, its
    // operands consumed by products up to position i) and the V slot of tile i (read and
    // consumed in position i), and a read is complete once its product has issued; only the
    // look-ahead reads of tile i+1 can still be in flight.  The barrier is a bare s_barrier:
    // a workgroup fence would wait for this position's batch as well.  The memory clobber
    // keeps LDS accesses on their side.
    auto tile_sync = [&](bool k_issued, bool v_issued) {
        constexpr int NKMIN = Tile::NIK / NW, NVMIN = Tile::NIV / NW;
        static_assert(NKMIN + NVMIN <= 15, "vmcnt immediate range");
        if (k_issued && v_issued) __builtin_amdgcn_s_waitcnt(0x0F70 | (NKMIN + NVMIN));  // lgkmcnt: no wait
        else if (v_issued) __builtin_amdgcn_s_waitcnt(0x0F70 | NVMIN);
        else __builtin_amdgcn_s_waitcnt(0x0F70);
        asm volatile("s_barrier" ::: "memory");
    };

    // S^T of sweep sub-step u (both query blocks) from the K tile at Ks.  Keys past the
    // window hold copies of the last key here; the softmax masks them.
    auto qk = [&](const T* Ks, int u, f32x16 (&S)[QB]) {
        const int kb = u & 1;
        typename M::frag ka = Tile::kfrag(Ks, kb, 0, col, h), kn;
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            if (s + 1 < NS) kn = Tile::kfrag(Ks, kb, s + 1, col, h);
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) S[qb] = M::mma(ka, qf[qb][s], s == 0 ? zero16() : S[qb]);
            if (s + 1 < NS) ka = kn;
        }
    };
    // row maxima of sweep sub-step u's scores, keys past the window excluded
    auto rowmax = [&](int u, const f32x16 (&S)[QB], float (&mx)[QB]) {
        const int kl = key_limit(u);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                if (crow(r, h) < kl) mx[qb] = fmaxf(mx[qb], S[qb][r]);
    };

    f32x16 oacc[NDB][QB];
    float m_ref[QB], l_run[QB];
    f32x16 SA[QB], SB[QB];

    // Sub-step u (generated assembly, wide_substep.inc): the score products of u+1 with the
    // softmax of u and the V^T operand reads of u, then the value products of u with the K
    // operand reads of u+2 and this wave's part of a tile copy.  MASK (the last tile, swept
    // first): keys of u from key_limit(u) on get a score of -inf first.  At the end of the
    // sweep the look-ahead scores and K reads use ring slots whose contents are never used;
    // every read stays inside the ring.
    static_assert(QB == 1, "the sub-step assembly holds one 32-query block per wave");
    const uint32_t kring_b = lds_addr(kring), vring_b = lds_addr(vring);
    const uint32_t klane_b = (uint32_t)((col * Tile::KLD + h * 8) * 2), vlane_b = (uint32_t)(vl * 2);
    auto kslot_b = [&](int t) { return kring_b + (uint32_t)(((t - p0) & 3) * Tile::K_ELEMS * 2); };
    auto vslot_b = [&](int t) { return vring_b + (uint32_t)(((t - p0) & 3) * Tile::V_ELEMS * 2); };
    typename M::frag kf[NS], vfr[NS], pfr[2];
    auto substep = [&](int u, auto par_tag, auto first_tag, bool mask) {
        constexpr int PAR = decltype(par_tag)::value;
        constexpr bool FIRST = decltype(first_tag)::value;
        f32x16& Sc = PAR == 0 ? SA[0] : SB[0];
        // keys of the ragged last tile (swept first) past the window: -inf
        const int kl = mask ? key_limit(u) : 32;
        if (kl < 32) {
#pragma unroll
            for (int r = 0; r < 16; ++r)
                if (crow(r, h) >= kl) Sc[r] = -INFINITY;
        }
        const uint32_t vaddr = vlane_b + vslot_b(u >> 1) + (uint32_t)((u & 1) * 32 * Tile::VLD * 2);
        const uint32_t kaddr = klane_b + kslot_b((u + 2) >> 1) + (uint32_t)((u & 1) * 32 * Tile::KLD * 2);
        wide_pipe<D, PAR, FIRST>(SA[0], SB[0], oacc, qf, kf, vfr, pfr, l_run[0], m_ref[0], sc, vaddr, kaddr);
    };
    uint32_t kc[3], vc[3], koff_b[3], voff_b[3];
    uint64_t kmask, vmask;
    copy_share<Tile::NIK, Tile::PWK, NW>(wave, tile.koff, kc, koff_b, kmask);
    copy_share<Tile::NIV, Tile::PWV, NW>(wave, tile.voff, vc, voff_b, vmask);
#pragma unroll
    for (int j = 0; j < 3; ++j) {
        kc[j] += kring_b;
        vc[j] += vring_b;
    }

    // one sweep of the window with the current reference; returns the row sums
    auto run = [&](bool first, float (&l_tot)[QB]) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            l_run[qb] = 0.f;
#pragma unroll
            for (int db = 0; db < NDB; ++db) oacc[db][qb] = zero16();
        }
        // Every register the sweep's assembly pins holds a defined value before its first
        // block, so that the compiler places no other operand of that block there.
        SB[0] = zero16();
#pragma unroll
        for (int i = 0; i < NS; ++i) vfr[i] = bf16x8{};
        pfr[0] = pfr[1] = bf16x8{};
        if (p1 > p0) {
            // prologue: positions p0 and p0+1 (K) and p0 (V) in LDS, K of p0+2 and V of p0+1
            // in flight (the batch of position p0-1); scores of the first sub-step
            dma_k(p0, kslot(p0));
            dma_v(p0, vslot(p0));
            if (p0 + 1 < p1) dma_k(p0 + 1, kslot(p0 + 1));
            dma_sync();
            if (p0 + 2 < p1) dma_k(p0 + 2, kslot(p0 + 2));
            if (p0 + 1 < p1) dma_v(p0 + 1, vslot(p0 + 1));
            if (wave_live) {
                qk(kslot(p0), 2 * p0, SA);
#pragma unroll
                for (int st = 0; st < NS; ++st) kf[st] = Tile::kfrag(kslot(p0), 1, st, col, h);
                wide_guard<D>(SA[0], SB[0], oacc);  // the products above wrote SA
                if (first) {
                    float mx[QB];
#pragma unroll
                    for (int qb = 0; qb < QB; ++qb) mx[qb] = -INFINITY;
                    rowmax(2 * p0, SA, mx);
#pragma unroll
                    for (int qb = 0; qb < QB; ++qb) m_ref[qb] = pair_max(mx[qb]) * sc;
                }
            }
            // Sweep position i holds sub-steps 2i and 2i+1 and issues the batch K of tile i+3
            // and V of tile i+2, into the slots position i-1 used (free once its barrier has
            // passed).  Position p0 (with the ragged tile when p0 = 0) issues it ahead of its
            // products by the general copy (clamped to the window, split between the two
            // segments of a streaming window).  Positions p0+1 .. p1-1 run in wide_loop, whose
            // copies are spread over the value products: those tiles are whole, each in one
            // segment (a streaming window's segment boundary is a multiple of 64 tokens or past
            // the last whole tile).  Near the end, where no tile is left to fetch, wide_loop
            // still copies, the last tile into the slot just freed (nothing reads that slot
            // again in this sweep, and the next barrier waits for it), so its loop has no
            // branches and its wait one count.  Waves without queries only copy: in the
            // chunk-parallel kernel by the general copy, in a streaming window the whole tiles.
            {
                const int i = p0;
                const bool kis = i + 3 < p1, vis = i + 2 < p1;
                if (kis) dma_k(i + 3, kslot(i + 3));
                if (vis) dma_v(i + 2, vslot(i + 2));
                if (wave_live) {
                    substep(2 * i, std::integral_constant<int, 0>{}, std::true_type{}, p0 == 0);
                    substep(2 * i + 1, std::integral_constant<int, 1>{}, std::false_type{}, p0 == 0);
                }
                tile_sync(kis, vis);
            }
            if (p0 + 1 < p1) {
                if (wave_live) {
                    // first tokens of the tiles the first loop position copies (tile_of(x) = x - 1 there)
                    const int last = p1 - 1;
                    wide_loop<D, STREAM>(SA[0], SB[0], oacc, qf, kf, vfr, pfr, l_run[0], m_ref[0], sc, p0 + 1, p1,
                                         (min(p0 + 4, last) - 1) * BK, (min(p0 + 3, last) - 1) * BK, (last - 1) * BK,
                                         STREAM ? w.src.len1 : (1 << 30), uniform_ptr(w.src.k1), uniform_ptr(w.src.v1),
                                         uniform_ptr(w.src.k2), uniform_ptr(w.src.v2), kring_b, vring_b, klane_b,
                                         vlane_b, kc, vc, koff_b, voff_b, kmask, vmask);
                } else {
                    const int last = p1 - 1;
                    for (int i = p0 + 1; i < p1; ++i) {
                        if (!STREAM) {
                            const bool kis = i + 3 < p1, vis = i + 2 < p1;
                            if (kis) dma_k(i + 3, kslot(i + 3));
                            if (vis) dma_v(i + 2, vslot(i + 2));
                            tile_sync(kis, vis);
                        } else {
                            const int tk = tile_of(min(i + 3, last)) * BK, tv = tile_of(min(i + 2, last)) * BK;
#pragma unroll
                            for (int j = 0; j < Tile::PWK; ++j) tile.issue_k_at(j, w.src.krow(tk, D), kslot(i + 3), wave);
#pragma unroll
                            for (int j = 0; j < Tile::PWV; ++j) tile.issue_v_at(j, w.src.vrow(tv, D), vslot(i + 2), wave);
                            tile_sync(true, true);
                        }
                    }
                }
            }
            if (wave_live) wide_flush<D>(SA[0], SB[0], oacc, kf, vfr, pfr);
            wide_guard<D>(SA[0], SB[0], oacc);
        }
        bool over = false;
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            l_tot[qb] = l_run[qb] + other_half(l_run[qb]);
            over = over || (wave_live && l_tot[qb] > kWideSumLimit);
        }
        return __syncthreads_or(over);
    };

    float l_tot[QB];
    if (run(true, l_tot)) {
        // exact row maxima by a score-only sweep, as the reference of a second sweep
        float mx[QB];
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) mx[qb] = -INFINITY;
        for (int i = p0; i < p1; ++i) {
            dma_k(i, kslot(0));
            dma_sync();
            if (wave_live) {
                for (int u = 2 * i; u < 2 * i + 2; ++u) {
                    qk(kslot(0), u, SA);
                    rowmax(u, SA, mx);
                }
            }
            __syncthreads();
        }
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) m_ref[qb] = pair_max(mx[qb]) * sc;
        run(false, l_tot);
    }

    if (w.split >= 0) {
        // Tail split: both halves store their partial (unnormalised O, reference, row sum);
        // the second to arrive merges the other's into its own and goes on to the epilogue,
        // the first is done.  Partials and arrival count are agent-scope atomic accesses
        // (stores written through to the level every CU of the device sees, loads served
        // from it), and every wave waits for its stores to complete before the barrier that
        // precedes the count, so the second arrival reads complete partials.  No device-wide
        // fence: on this part it writes back and invalidates the whole L2 of the XCD.
        constexpr int NR = NDB * QB * 16 + 2 * QB;  // values per lane
        float* const pair = a.split_part + (size_t)64 * NR * NW * 2 * w.split;
        float* const mine = pair + (size_t)64 * NR * (w.half * NW + wave) + lane;
        auto put = [](float* p, float x) { __hip_atomic_store(p, x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); };
        auto get = [](const float* p) {
            return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        };
        int r = 0;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int qb = 0; qb < QB; ++qb)
#pragma unroll
                for (int e = 0; e < 16; ++e) put(mine + 64 * r++, oacc[db][qb][e]);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            put(mine + 64 * r++, m_ref[qb]);
            put(mine + 64 * r++, l_tot[qb]);
        }
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's partial stores are complete
        __syncthreads();
        unsigned prev = 0;
        if (tid == 0) prev = __hip_atomic_fetch_add(a.split_cnt + w.split, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (!__syncthreads_or(tid == 0 && prev != 0)) return;
        // the merge is written in half order (half 0's terms first) whichever half runs it,
        // so the result does not depend on the arrival order
        const float* const other = pair + (size_t)64 * NR * ((1 - w.half) * NW + wave) + lane;
        const bool h0 = w.half == 0;
        float f0q[QB], f1q[QB];
        r = NDB * QB * 16;
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            const float mo = get(other + 64 * r++), lo = get(other + 64 * r++);
            const float m0 = h0 ? m_ref[qb] : mo, m1 = h0 ? mo : m_ref[qb];
            const float l0 = h0 ? l_tot[qb] : lo, l1 = h0 ? lo : l_tot[qb];
            const float mm = fmaxf(m0, m1);
            const float f0 = __builtin_amdgcn_exp2f(m0 - mm), f1 = __builtin_amdgcn_exp2f(m1 - mm);
            l_tot[qb] = __builtin_fmaf(l0, f0, l1 * f1);
            m_ref[qb] = mm;
            f0q[qb] = f0;
            f1q[qb] = f1;
        }
        r = 0;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int qb = 0; qb < QB; ++qb)
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const float xs = oacc[db][qb][e], xo = get(other + 64 * r++);
                    const float x0 = h0 ? xs : xo, x1 = h0 ? xo : xs;
                    oacc[db][qb][e] = __builtin_fmaf(x0, f0q[qb], x1 * f1q[qb]);
                }
        if (tid == 0) __hip_atomic_store(a.split_cnt + w.split, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }


    if constexpr (EPI_ALL) wide_linear_and_merge<OT, D, NW, QB>(a, w, smem, qw, wave, has_soft, has_lin, qf, oacc, m_ref, l_tot);
    else linear_and_merge<T, OT, D, QB, NT>(a, w, smem, qw, has_soft, has_lin, qf, oacc, m_ref, l_tot);
}

template <class OT, int D, bool STREAM>
static hipError_t launch_wide_one(const AttnArgs& a, hipStream_t stream) {
    constexpr int NW = kWideWaves, QB = kWideQB;
    constexpr size_t kLdsMax = 160 * 1024;
    using Tile = DmaTiles<D, NW>;
    const size_t kv = (4 * (size_t)Tile::K_ELEMS + 4 * (size_t)Tile::V_ELEMS) * sizeof(bf16);
    const size_t epi_all = wide_epilogue_lds_bytes(D, a.Dphi, a.P);
    const bool all = epi_all <= kLdsMax;
    const size_t epi = all ? epi_all : epilogue_lds_bytes<bf16, D>(a.Dphi);
    size_t lds = kv > epi ? kv : epi;
    if (all && wide_out_stage_bytes<OT, D>() > lds) lds = wide_out_stage_bytes<OT, D>();
    if (STREAM && a.side_blocks > 0 && state16_lds_bytes<D>() > lds) lds = state16_lds_bytes<D>();
    auto fn = all ? attn_wide_kernel<OT, D, STREAM, true> : attn_wide_kernel<OT, D, STREAM, false>;
    static size_t lds_set[2][64] = {};
    hipError_t e = ensure_lds(reinterpret_cast<const void*>(fn), lds, lds_set[all ? 1 : 0]);
    if (e != hipSuccess) return e;
    AttnArgs b = a;
    attn_grid(b, NW * QB * 32);
    hipLaunchKernelGGL(fn, dim3(8 * b.per_xcd + (STREAM ? b.side_blocks : 0)), dim3(NW * 64), lds, stream, b);
    return hipGetLastError();
}

template <class OT, bool STREAM>
static hipError_t launch_wide_d(const AttnArgs& a, hipStream_t stream) {
    switch (a.D) {
        case 32: return launch_wide_one<OT, 32, STREAM>(a, stream);
        case 64: return launch_wide_one<OT, 64, STREAM>(a, stream);
        case 128: return launch_wide_one<OT, 128, STREAM>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

// Tail split plan of a bf16 launch: per XCD, the last kSplitPerXcd chunk-0 query tiles run
// as two halves, where chunk 0's window spans at least four 64-token tiles (each half then
// sweeps two or more).  The rule and the tiles depend on chunk 0 alone (its min(Tc, T)
// frames), so a streaming launch of the first chunk (which splits when the host asks for
// it) splits exactly the tiles the chunk-parallel grid splits, and a one-chunk clip splits
// the same tiles whatever Tc >= T it is run with: the outputs stay equal bit for bit.
// Sets a.split_per_xcd; returns the number of split tiles.
int wide_split_plan(AttnArgs& a) {
    constexpr int kSplitPerXcd = 8, NW = kWideWaves, QB = kWideQB;
    const int want = a.split_per_xcd;
    a.split_per_xcd = 0;
    if (a.linear_only || (a.stream && want == 0)) return 0;
    const int f = a.stream ? a.s_frames : (a.Tc < a.T ? a.Tc : a.T);
    if ((f * a.n + 63) / 64 < 4) return 0;
    a.split_per_xcd = kSplitPerXcd;
    AttnArgs b = a;
    return attn_grid(b, NW * QB * 32);
}

// Scratch bytes of one split: two halves x waves x 64 lanes x (O + reference + sum).
size_t wide_split_part_bytes(int D) {
    const size_t nr = (size_t)(D / 32) * kWideQB * 16 + 2 * kWideQB;
    return 2 * (size_t)kWideWaves * 64 * nr * sizeof(float);
}

hipError_t launch_attn_wide(const AttnArgs& a, int out_dtype, hipStream_t stream) {
    if (out_dtype == 1) return a.stream ? launch_wide_d<bf16, true>(a, stream) : launch_wide_d<bf16, false>(a, stream);
    return a.stream ? launch_wide_d<float, true>(a, stream) : launch_wide_d<float, false>(a, stream);
}

}  // namespace rehyat
