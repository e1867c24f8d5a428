// attn_wide.hip -- bf16 windowed softmax tile kernel, 64 queries per wave, with the linear
// part and the shared normalisation fused into its epilogue (ReHyAt blog,
// maplevalley.com.cn, sections 2.2.1-2.3).
//
// One workgroup = 4 waves x 64 queries (two 32-query blocks per wave) of one chunk of one
// (batch, head), one wave per SIMD with the whole register file.  Every K or V operand read
// from LDS feeds two MFMAs (one per query block): half the LDS read traffic per product of
// a 32-query wave, which is what bounds that layout on this part.
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
// the exact row maximum, found by a score-only sweep over the window.  Row sums are taken
// from the bf16 P actually fed to the value product (dot2 against ones), so numerator
// and denominator see the same rounded weights.
#include <type_traits>

#include "attn_common.hpp"
#include "dma.hpp"

namespace rehyat {

static constexpr float kWideSumLimit = 18446744073709551616.0f;  // 2^64

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// sum of the 8 bf16 of an operand, accumulated in fp32
__device__ inline float sum8(bf16x8 v, float acc) {
    const bf16x2 one = {(bf16)1.0f, (bf16)1.0f};
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 0, 1), one, acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 2, 3), one, acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 4, 5), one, acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(v, v, 6, 7), one, acc, false);
    return acc;
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

// Epilogue of the wide kernel when everything it reads fits in LDS at once (ReHyAt blog,
// maplevalley.com.cn, 2.2.2-2.3): W_q, every power of the chunk's state image and Z are
// staged by one round of LDS-DMA behind a single barrier, then each 32-query block computes
// u = W_q q on MFMA from the Q operand registers, phi = per-part powers of softplus(u + b),
// y = sum over powers of S_c^T phi on MFMA (phi straight from the u registers),
// z = phi . Z_c, and merges with its softmax part.
template <class OT, int D, int NW>
__device__ inline void wide_linear_and_merge(const AttnArgs& a, const Window<bf16>& w, unsigned char* smem, int qw,
                                             int wave, bool has_soft, bool has_lin,
                                             const bf16x8 (&qf)[2][D / 16], const f32x16 (&oacc)[D / 32][2],
                                             const float (&m_ref)[2], const float (&l_tot)[2]) {
    using T = bf16;
    using M = Mfma<T>;
    constexpr int QB = 2, KS = M::KS, EPL = M::EPL, NS = D / KS, NDB = D / 32, TPB = 16 / EPL;
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
        merge_store_block<T, OT, D>(a, w, qw + qb * 32 + col, has_soft, has_lin, oacc, qb, yacc, m_ref[qb], l_tot[qb], zq);
    }
}

template <class OT, int D, bool STREAM, bool EPI_ALL>
__global__ __launch_bounds__(256, 1) void attn_wide_kernel(const AttnArgs a) {
    using T = bf16;
    using M = Mfma<T>;
    constexpr int QB = 2, NW = 4, NT = NW * 64, BQ = NW * QB * 32;
    using Tile = DmaTiles<D, NW>;
    constexpr int KS = M::KS, EPL = M::EPL, NS = D / KS, NDB = D / 32;
    constexpr int TPB = 32 / KS;  // value-product steps per 32-token sub-step
    constexpr int BK = Tile::BK;
    constexpr int PWMAX = Tile::PWK > Tile::PWV ? Tile::PWK : Tile::PWV;
    static_assert(PWMAX <= TPB * NDB, "a sub-step has fewer product pairs than copy instructions");

    extern __shared__ __align__(16) unsigned char smem[];
    T* const kring = reinterpret_cast<T*>(smem);
    T* const vring = kring + 4 * Tile::K_ELEMS;

    Window<T> w;
    if (!decode_window<T, D, STREAM>(a, w)) return;
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
    // sweep positions of this workgroup: all, or one half of a split tile's window
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

    auto kslot = [&](int t) { return kring + (t & 3) * Tile::K_ELEMS; };
    auto vslot = [&](int t) { return vring + (t % 3) * Tile::V_ELEMS; };
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

    // K operands of the look-ahead scores, read one sub-step before their products so the
    // LDS latency is covered by a whole sub-step of work (one wave per SIMD has no other
    // wave to hide it behind)
    typename M::frag kpre[NS];
    auto read_k = [&](int u) {
        const T* Ks = kslot(u >> 1);
#pragma unroll
        for (int st = 0; st < NS; ++st) kpre[st] = Tile::kfrag(Ks, u & 1, st, col, h);
    };

    // Sub-step u (kpre holds the K operands of u+1), one basic block cut by scheduling
    // fences into
    //   V operand reads of u | scores of u+1 with the softmax of u | value product of u with
    //   the K operand reads of u+2.
    // The scores and the softmax are written as 16 segments [MFMA, 1/16 of the softmax]; the
    // compiler's MFMA/exp interleaving places the vector work between the products.  MASK
    // (the last tile, swept first): keys of u from key_limit(u) on get a score of -inf.  At
    // the end of the sweep the look-ahead and the K reads land in ring slots whose contents
    // are never used; every read stays inside the ring.
    auto sub_full = [&](int u, f32x16 (&Sc)[QB], f32x16 (&Sn)[QB], auto mask_tag, auto&& dma_part) {
        constexpr bool MASK = decltype(mask_tag)::value;
        const int kl = MASK ? key_limit(u) : 32;
        if (MASK && kl < 32) {
#pragma unroll
            for (int r = 0; r < 16; ++r)
                if (crow(r, h) >= kl)
#pragma unroll
                    for (int qb = 0; qb < QB; ++qb) Sc[qb][r] = -INFINITY;
        }
        const T* Vs = vslot(u >> 1);
        constexpr int NV = TPB * NDB;
        typename M::frag vf[NV];
#pragma unroll
        for (int i = 0; i < NV; ++i) vf[i] = Tile::vfrag(Vs, vl, i % NDB, u & 1, i / NDB);
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_iglp_opt(2);
        typename M::frag pf[TPB][QB];
        float lsum[QB];
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) lsum[qb] = l_run[qb];
        float pv[QB * 16];
        constexpr int NSEG = NS * QB;
        constexpr int PER = QB * 16 / NSEG;  // softmax values per segment
#pragma unroll
        for (int i = 0; i < NSEG; ++i) {
            const int st = i / QB, qb = i % QB;
            Sn[qb] = M::mma(kpre[st], qf[qb][st], st == 0 ? zero16() : Sn[qb]);
#pragma unroll
            for (int e = 0; e < PER; ++e) {
                const int idx = i * PER + e, q2 = idx / 16, r = idx % 16;
                pv[idx] = __builtin_amdgcn_exp2f(__builtin_fmaf(Sc[q2][r], sc, -m_ref[q2]));
                if ((idx + 1) % EPL == 0) {
                    const int t = r / EPL;
                    pf[t][q2] = M::pack(pv + idx + 1 - EPL);
                    lsum[q2] = sum8(pf[t][q2], lsum[q2]);
                }
            }
        }
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) l_run[qb] = lsum[qb];
        read_k(u + 2);  // unfenced: the scheduler spreads these reads over the value product
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int db = i % NDB, t = i / NDB;
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) oacc[db][qb] = M::mma(vf[i], pf[t][qb], oacc[db][qb]);
            // one DMA instruction of the tile copy after each pair of products, so that the
            // copies issue in the shadow of the products instead of in a burst ahead of them
            if (i < PWMAX) {
                __builtin_amdgcn_sched_barrier(0);
                dma_part(i);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    };

    f32x16 SA[QB], SB[QB];
    // one sweep of the window with the current reference; returns the row sums
    auto run = [&](bool first, float (&l_tot)[QB]) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            l_run[qb] = 0.f;
#pragma unroll
            for (int db = 0; db < NDB; ++db) oacc[db][qb] = zero16();
        }
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
                read_k(2 * p0 + 1);
                if (first) {
                    float mx[QB] = {-INFINITY, -INFINITY};
                    rowmax(2 * p0, SA, mx);
#pragma unroll
                    for (int qb = 0; qb < QB; ++qb) m_ref[qb] = pair_max(mx[qb]) * sc;
                }
            }
            // sweep position i holds sub-steps 2i and 2i+1; position 0 (the last tile of the
            // window) is the only one that can hold a ragged or an empty sub-step
            auto none = [](int) {};
            // Sweep position i: batch K of i+3 and V of i+2, into the slots position i-1 used
            // (free once its barrier has passed), and sub-steps 2i and 2i+1.
            //   UPFRONT: the batch is issued ahead of the products, by the general copy (clamped
            //   to the window, and split between the two segments of a streaming window).  For
            //   position 0 (with the ragged tile), and in the chunk-parallel kernel for waves
            //   without queries.
            //   Otherwise the copy is spread over the products, K over the first sub-step and V
            //   over the second (waves of a streaming window without queries issue it at once):
            //   tiles past position 0 are whole tiles with a uniform base, in one segment.  Near
            //   the end, where no tile is left to fetch, the copy is still issued, of a whole
            //   tile into the slot just freed (nothing reads that slot again in this sweep, and
            //   the next workgroup barrier waits for it), so the loop has no branches and the
            //   wait one count.
            auto position = [&](int i, auto mask_tag, auto upfront_tag) {
                constexpr bool UPFRONT = decltype(upfront_tag)::value;
                const bool kis = i + 3 < p1, vis = i + 2 < p1;
                if (UPFRONT || (!STREAM && !wave_live)) {
                    if (kis) dma_k(i + 3, kslot(i + 3));
                    if (vis) dma_v(i + 2, vslot(i + 2));
                    if (wave_live) {
                        sub_full(2 * i, SA, SB, mask_tag, none);
                        sub_full(2 * i + 1, SB, SA, mask_tag, none);
                    }
                    tile_sync(kis, vis);
                    return;
                }
                const int last = p1 - 1;  // >= i >= 1: a whole tile
                const int tk = tile_of(min(i + 3, last)) * BK, tv = tile_of(min(i + 2, last)) * BK;
                // a streaming window's segment boundary is a multiple of 64 tokens (or past
                // the last whole tile), so each of these tiles lies in one segment
                const T* const kb = STREAM ? w.src.krow(tk, D) : w.src.k1 + (int64_t)tk * D;
                const T* const vb = STREAM ? w.src.vrow(tv, D) : w.src.v1 + (int64_t)tv * D;
                T* const kd = kslot(i + 3);
                T* const vd = vslot(i + 2);
                auto kpart = [&](int j) {
                    if (j < Tile::PWK) tile.issue_k_at(j, kb, kd, wave);
                };
                auto vpart = [&](int j) {
                    if (j < Tile::PWV) tile.issue_v_at(j, vb, vd, wave);
                };
                if (!STREAM || wave_live) {
                    sub_full(2 * i, SA, SB, mask_tag, kpart);
                    sub_full(2 * i + 1, SB, SA, mask_tag, vpart);
                } else {
#pragma unroll
                    for (int j = 0; j < Tile::PWK; ++j) kpart(j);
#pragma unroll
                    for (int j = 0; j < Tile::PWV; ++j) vpart(j);
                }
                tile_sync(true, true);
            };
            if (p0 == 0) position(0, std::true_type{}, std::true_type{});
            else position(p0, std::false_type{}, std::true_type{});
            for (int i = p0 + 1; i < p1; ++i) position(i, std::false_type{}, std::false_type{});
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
        float mx[QB] = {-INFINITY, -INFINITY};
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

    if (!STREAM && w.split >= 0) {
        // Tail split: both halves store their partial (unnormalised O, reference, row sum);
        // the second to arrive merges the other's into its own and goes on to the epilogue,
        // the first is done.  Device-scope fences order the partials before the count.
        constexpr int NR = NDB * QB * 16 + 2 * QB;  // values per lane
        float* const pair = a.split_part + (size_t)64 * NR * NW * 2 * w.split;
        float* const mine = pair + (size_t)64 * NR * (w.half * NW + wave) + lane;
        int r = 0;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int qb = 0; qb < QB; ++qb)
#pragma unroll
                for (int e = 0; e < 16; ++e) mine[64 * r++] = oacc[db][qb][e];
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            mine[64 * r++] = m_ref[qb];
            mine[64 * r++] = l_tot[qb];
        }
        __threadfence();
        __syncthreads();
        unsigned prev = 0;
        if (tid == 0) prev = atomicAdd(a.split_cnt + w.split, 1u);
        if (!__syncthreads_or(tid == 0 && prev != 0)) return;
        __threadfence();
        // the merge is written in half order (half 0's terms first) whichever half runs it,
        // so the result does not depend on the arrival order
        const float* const other = pair + (size_t)64 * NR * ((1 - w.half) * NW + wave) + lane;
        const bool h0 = w.half == 0;
        float f0q[QB], f1q[QB];
        r = NDB * QB * 16;
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            const float mo = other[64 * r++], lo = other[64 * r++];
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
                    const float xs = oacc[db][qb][e], xo = other[64 * r++];
                    const float x0 = h0 ? xs : xo, x1 = h0 ? xo : xs;
                    oacc[db][qb][e] = __builtin_fmaf(x0, f0q[qb], x1 * f1q[qb]);
                }
        if (tid == 0) a.split_cnt[w.split] = 0u;  // ready for the next launch
    }

    if constexpr (EPI_ALL) wide_linear_and_merge<OT, D, NW>(a, w, smem, qw, wave, has_soft, has_lin, qf, oacc, m_ref, l_tot);
    else linear_and_merge<T, OT, D, QB, NT>(a, w, smem, qw, has_soft, has_lin, qf, oacc, m_ref, l_tot);
}

template <class OT, int D, bool STREAM>
static hipError_t launch_wide_one(const AttnArgs& a, hipStream_t stream) {
    constexpr int NW = 4, QB = 2;
    constexpr size_t kLdsMax = 160 * 1024;
    using Tile = DmaTiles<D, NW>;
    const size_t kv = (4 * (size_t)Tile::K_ELEMS + 3 * (size_t)Tile::V_ELEMS) * sizeof(bf16);
    const size_t epi_all = wide_epilogue_lds_bytes(D, a.Dphi, a.P);
    const bool all = epi_all <= kLdsMax;
    const size_t epi = all ? epi_all : epilogue_lds_bytes<bf16, D>(a.Dphi);
    const size_t lds = kv > epi ? kv : epi;
    auto fn = all ? attn_wide_kernel<OT, D, STREAM, true> : attn_wide_kernel<OT, D, STREAM, false>;
    static size_t lds_set[2][64] = {};
    hipError_t e = ensure_lds(reinterpret_cast<const void*>(fn), lds, lds_set[all ? 1 : 0]);
    if (e != hipSuccess) return e;
    AttnArgs b = a;
    attn_grid(b, NW * QB * 32);
    hipLaunchKernelGGL(fn, dim3(8 * b.per_xcd), dim3(NW * 64), lds, stream, b);
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

// Tail split plan of the bf16 chunk-parallel launch: per XCD, the last kSplitPerXcd
// chunk-0 query tiles run as two halves.  Only where the chunk-0 window spans at least four
// 64-token tiles and a longer class exists (otherwise the grid is a single wave of equal
// tiles and halves do not shorten it).  Sets a.split_per_xcd; returns the split count.
int wide_split_plan(AttnArgs& a) {
    constexpr int kSplitPerXcd = 8, NW = 4, QB = 2;
    a.split_per_xcd = 0;
    if (a.stream || a.linear_only || a.nchunks < 2) return 0;
    const int lk0 = (a.Tc < a.T ? a.Tc : a.T) * a.n;
    if ((lk0 + 63) / 64 < 4) return 0;
    a.split_per_xcd = kSplitPerXcd;
    AttnArgs b = a;
    return attn_grid(b, NW * QB * 32);
}

// Scratch bytes of one split: two halves x 4 waves x 64 lanes x (O + reference + sum).
size_t wide_split_part_bytes(int D) {
    const size_t nr = (size_t)(D / 32) * 2 * 16 + 4;
    return 2 * 4 * 64 * nr * sizeof(float);
}

hipError_t launch_attn_wide(const AttnArgs& a, int out_dtype, hipStream_t stream) {
    if (out_dtype == 1) return a.stream ? launch_wide_d<bf16, true>(a, stream) : launch_wide_d<bf16, false>(a, stream);
    return a.stream ? launch_wide_d<float, true>(a, stream) : launch_wide_d<float, false>(a, stream);
}

}  // namespace rehyat
