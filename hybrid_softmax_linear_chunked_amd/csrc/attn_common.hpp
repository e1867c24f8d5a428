// attn_common.hpp -- pieces shared by the attention kernels: which window a workgroup
// works on, the linear part of the hybrid output (phi_q(q) S_c, phi_q(q) . Z_c) and the
// shared normalisation (ReHyAt blog, maplevalley.com.cn, sections 2.2.1, 2.2.2 and 2.3).
#pragma once

#include "tiles.hpp"
#include "kernels.hpp"

namespace rehyat {

// The chunk a workgroup works on: its queries, its softmax window and its linear state.
template <class T>
struct Window {
    int bh, hh, c, qt;
    int q0, Lq, Lk, ls;
    int img_slot;
    KeySrc<T> src;
    int split, half;  // tail split index (-1: whole tile) and which half of the sweep
};

// Share of XCD x of N items dealt as 8 contiguous runs.
__host__ __device__ inline int xcd_share(int64_t N, int x) { return (int)(N * (x + 1) / 8 - N * x / 8); }
// Number of split tiles of XCD x: the last `per` of its chunk-0 tiles (all, if it has fewer).
__host__ __device__ inline int xcd_splits(int64_t NS, int per, int x) {
    const int ns = xcd_share(NS, x);
    return ns < per ? ns : per;
}

// Workgroups are dealt round-robin over the 8 XCDs (workgroup g runs on XCD g % 8, as
// the (g / 8)-th of that XCD), and each XCD hands its workgroups to its CUs in order.
// The query tiles are two classes: those of chunks c >= 1, whose softmax window includes
// the To overlap frames, and the shorter ones of chunk 0.  Every XCD takes an equal
// contiguous share of each class, longer class first, so that its last workgroups are the
// short ones (a shorter tail) and the tiles of one chunk share an XCD's L2.  With tail
// splitting, the last split_per_xcd chunk-0 tiles of an XCD come as pairs of workgroups,
// one per half of the window.  A streaming launch is one class (its chunk's tiles); it
// splits only on the first chunk, the same tiles as the chunk-parallel grid.  Returns
// false for the padding workgroups of the grid.
template <class T, int D, bool STREAM>
__device__ inline bool decode_window(const AttnArgs& a, Window<T>& w) {
    const int x = blockIdx.x % 8, p = blockIdx.x / 8;
    const int tpc = a.tiles_per_chunk, cl = a.nchunks - 1;  // chunks of the longer class
    const int NL = cl * a.BH * tpc, NS = a.BH * tpc;
    const int l0 = (int)((int64_t)NL * x / 8), nl = (int)((int64_t)NL * (x + 1) / 8) - l0;
    const int s0 = (int)((int64_t)NS * x / 8), ns = (int)((int64_t)NS * (x + 1) / 8) - s0;
    const int ks = xcd_splits(NS, a.split_per_xcd, x);
    w.split = -1;
    w.half = 0;
    if (p < nl) {
        const int idx = l0 + p, ch = idx / tpc;
        w.qt = idx % tpc;
        w.c = 1 + ch % cl;
        w.bh = ch / cl;
    } else if (p < nl + ns + ks) {
        const int r = p - nl;  // whole chunk-0 tiles, then the split pairs
        int idx = s0 + r;
        if (r >= ns - ks) {
            const int pr = r - (ns - ks);
            int base = 0;
            for (int y = 0; y < x; ++y) base += xcd_splits(NS, a.split_per_xcd, y);
            idx = s0 + ns - ks + pr / 2;
            w.half = pr % 2;
            w.split = base + pr / 2;
        }
        w.qt = idx % tpc;
        w.c = 0;
        w.bh = idx / tpc;
    } else {
        return false;
    }
    w.hh = w.bh % a.H;
    const T* kb1 = reinterpret_cast<const T*>(a.k1) + (int64_t)w.bh * a.kv1_bh_stride;
    const T* vb1 = reinterpret_cast<const T*>(a.v1) + (int64_t)w.bh * a.kv1_bh_stride;
    if constexpr (!STREAM) {
        // chunk c = frames [f0, f1); softmax window [max(0, f0 - To), f1); linear [0, ws)
        const int f0 = w.c * a.Tc;
        const int f1 = min(f0 + a.Tc, a.T);
        const int ws = a.linear_only ? f1 : max(0, f0 - a.To);
        w.q0 = f0 * a.n;
        w.Lq = (f1 - f0) * a.n;
        w.Lk = (f1 - ws) * a.n;
        w.ls = ws;
        w.src.k1 = kb1 + (int64_t)ws * a.n * D;
        w.src.v1 = vb1 + (int64_t)ws * a.n * D;
        w.src.k2 = w.src.k1;
        w.src.v2 = w.src.v1;
        w.src.len1 = 1 << 30;
        w.img_slot = w.bh * a.img_slots + w.c;
    } else {
        // one streaming chunk: window = [held overlap frames | this chunk]
        w.q0 = 0;
        w.Lq = a.s_frames * a.n;
        w.Lk = a.linear_only ? 0 : (a.s_held + a.s_frames) * a.n;
        w.ls = a.s_ls;
        w.src.k1 = kb1;
        w.src.v1 = vb1;
        // the first s_pad chunk rows are read from their copy in the first segment
        w.src.k2 = reinterpret_cast<const T*>(a.k2) + (int64_t)w.bh * a.kv2_bh_stride + (int64_t)a.s_pad * D;
        w.src.v2 = reinterpret_cast<const T*>(a.v2) + (int64_t)w.bh * a.kv2_bh_stride + (int64_t)a.s_pad * D;
        w.src.len1 = a.s_held * a.n + a.s_pad;
        w.img_slot = w.bh;
    }
    return true;
}

// LDS needed by the epilogue: W_q [Dphi][D + VEC] and one power of the state image
// [D][Dphi + VEC].
template <class T, int D>
__host__ __device__ inline size_t epilogue_lds_bytes(int Dphi) {
    constexpr int VEC = 16 / sizeof(T);
    return ((size_t)Dphi * (D + VEC) + (size_t)D * (Dphi + VEC)) * sizeof(T);
}

// Merge and store one query row of a wave's query block qb (ReHyAt blog,
// maplevalley.com.cn, 2.3): out = (2^m O + y) / (2^m l + z), both scaled by 2^-max(m, 0);
// aux outputs if requested.  The row's values live in lane (row % 32, h) of the C layout.
template <class T, class OT, int D, int QB>
__device__ inline void merge_store_block(const AttnArgs& a, const Window<T>& w, int row, bool has_soft, bool has_lin,
                                         const f32x16 (&oacc)[D / 32][QB], int qb, const f32x16 (&yacc)[D / 32],
                                         float m_run, float l_tot, float zq, bool store_out = true) {
    constexpr int NDB = D / 32;
    const int lane = threadIdx.x % 64, h = lane / 32;
    OT* outs = reinterpret_cast<OT*>(a.out) + (int64_t)w.bh * a.q_bh_stride + (int64_t)w.q0 * D;
    const int64_t arow0 = (int64_t)w.bh * a.aux_bh_stride + w.q0;
    if (row >= w.Lq) return;
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
    OT* orow = outs + (int64_t)row * D;
    if (store_out) {
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int d = db * 32 + g * 8 + h * 4;
                float vals[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) vals[i] = ca * oacc[db][qb][g * 4 + i] + cg * yacc[db][g * 4 + i];
                if constexpr (sizeof(OT) == 4) {
                    *reinterpret_cast<float4*>(orow + d) = make_float4(vals[0], vals[1], vals[2], vals[3]);
                } else {
                    bf16x4 o4;
#pragma unroll
                    for (int i = 0; i < 4; ++i) o4[i] = (bf16)vals[i];
                    *reinterpret_cast<bf16x4*>(orow + d) = o4;
                }
            }
    }
    if (a.aux_o_soft || a.aux_y) {
        const float il = has_soft ? 1.f / l_tot : 0.f;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int d = db * 32 + g * 8 + h * 4;
                float4 so, yo;
                so.x = oacc[db][qb][g * 4 + 0] * il; so.y = oacc[db][qb][g * 4 + 1] * il;
                so.z = oacc[db][qb][g * 4 + 2] * il; so.w = oacc[db][qb][g * 4 + 3] * il;
                yo.x = yacc[db][g * 4 + 0]; yo.y = yacc[db][g * 4 + 1];
                yo.z = yacc[db][g * 4 + 2]; yo.w = yacc[db][g * 4 + 3];
                if (a.aux_o_soft) *reinterpret_cast<float4*>(a.aux_o_soft + (arow0 + row) * D + d) = so;
                if (a.aux_y) *reinterpret_cast<float4*>(a.aux_y + (arow0 + row) * D + d) = yo;
            }
    }
    if (h == 0) {
        if (a.aux_lse) a.aux_lse[arow0 + row] = has_soft ? m_run * 0.6931471805599453f + logf(l_tot) : -INFINITY;
        if (a.aux_z) a.aux_z[arow0 + row] = zq;
    }
}

// Epilogue of the attention kernels, one 32-query block of the wave at a time, so only one
// block's linear-part registers are live next to the softmax accumulators.
//
// Linear part (ReHyAt blog, maplevalley.com.cn, 2.2.2): u = W_q q on MFMA from the Q
// operand registers, phi = per-part powers of softplus(u + b); per power the chunk's state
// image is staged in LDS, y += S_c^T phi on MFMA (phi taken straight from the u registers)
// and z += phi . Z_c.  Merge (2.3): out = (2^m O + y) / (2^m l + z), both scaled by
// 2^-max(m, 0); aux outputs if requested.  Starts with a barrier: the caller's K/V tiles may
// still be read.
template <class T, class OT, int D, int QB, int NT>
__device__ inline void linear_and_merge(const AttnArgs& a, const Window<T>& w, unsigned char* smem, int qw,
                                        bool has_soft, bool has_lin,
                                        const typename Mfma<T>::frag (&qf)[QB][D / Mfma<T>::KS],
                                        const f32x16 (&oacc)[D / 32][QB], const float (&m_run)[QB],
                                        const float (&l_tot)[QB]) {
    using M = Mfma<T>;
    constexpr int KS = M::KS, EPL = M::EPL, NS = D / KS, NDB = D / 32, TPB = 16 / EPL;
    constexpr int VEC = 16 / sizeof(T);
    const int tid = threadIdx.x, lane = tid % 64, col = lane % 32, h = lane / 32;
    const int Dphi = a.Dphi, P = a.P, NJB = Dphi / 32;
    constexpr int WLD = D + VEC;  // W_q row stride in LDS
    const int SLD = Dphi + VEC;   // state-image row stride in LDS
    T* Ws = reinterpret_cast<T*>(smem);
    T* Ss = Ws + Dphi * WLD;
    const T* wq = reinterpret_cast<const T*>(a.wq) + (int64_t)w.hh * Dphi * D;
    const T* img = reinterpret_cast<const T*>(a.simg) + (int64_t)w.img_slot * P * D * Dphi;
    const float* zimg = a.zimg + (int64_t)w.img_slot * P * Dphi;
    const float* bq = a.bq ? a.bq + (int64_t)w.hh * Dphi : nullptr;

    if (has_lin) {
        __syncthreads();  // every wave is done with the K/V tiles
        for (int i = tid; i < Dphi * (D / VEC); i += NT) {
            const int j = i / (D / VEC), ch = i % (D / VEC);
            *reinterpret_cast<uint4*>(Ws + j * WLD + ch * VEC) = *reinterpret_cast<const uint4*>(wq + (int64_t)j * D + ch * VEC);
        }
    }
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        f32x16 yacc[NDB];
#pragma unroll
        for (int db = 0; db < NDB; ++db) yacc[db] = zero16();
        float zq = 0.f;
        if (has_lin) {
            __syncthreads();  // W_q staged / previous block done with the image
            constexpr int JBMAX = 4;  // Dphi <= 128
            float uu[JBMAX][16];
#pragma unroll
            for (int jb = 0; jb < JBMAX; ++jb) {
                if (jb >= NJB) break;
                f32x16 u = M::mma(M::load(Ws + (jb * 32 + col) * WLD + h * EPL), qf[qb][0], zero16());
#pragma unroll
                for (int s = 1; s < NS; ++s) u = M::mma(M::load(Ws + (jb * 32 + col) * WLD + s * KS + h * EPL), qf[qb][s], u);
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float x = u[r] + (bq ? bq[jb * 32 + crow(r, h)] : 0.f);
                    uu[jb][r] = softplus_fast<T>(x);
                }
            }
            for (int pw = 1; pw <= P; ++pw) {
                if (pw > 1) __syncthreads();  // previous power no longer read
                const T* ip = img + (int64_t)(pw - 1) * D * Dphi;
                for (int i = tid; i < D * (Dphi / VEC); i += NT) {
                    const int d = i / (Dphi / VEC), ch = i % (Dphi / VEC);
                    *reinterpret_cast<uint4*>(Ss + d * SLD + ch * VEC) = *reinterpret_cast<const uint4*>(ip + (int64_t)d * Dphi + ch * VEC);
                }
                __syncthreads();
                const float* zp = zimg + (pw - 1) * Dphi;
#pragma unroll
                for (int jb = 0; jb < JBMAX; ++jb) {
                    if (jb >= NJB) break;
                    float ph[16];
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        float v = uu[jb][r];
                        for (int e = 1; e < pw; ++e) v *= uu[jb][r];
                        ph[r] = v;
                        zq += v * zp[jb * 32 + crow(r, h)];
                    }
#pragma unroll
                    for (int t = 0; t < TPB; ++t) {
                        const typename M::frag bfr = M::pack(ph + t * EPL);
#pragma unroll
                        for (int db = 0; db < NDB; ++db) {
                            const typename M::frag sf = M::load(Ss + (db * 32 + col) * SLD + jb * 32 + t * 2 * EPL + h * EPL);
                            yacc[db] = M::mma(sf, bfr, yacc[db]);
                        }
                    }
                }
            }
            zq += other_half(zq);
        }

        merge_store_block<T, OT, D>(a, w, qw + qb * 32 + col, has_soft, has_lin, oacc, qb, yacc, m_run[qb], l_tot[qb],
                                    zq);
    }
}

// Launch bookkeeping common to the attention kernels: workgroups per XCD (a share of each
// class plus the second halves of its split tiles, see decode_window).  Returns the number
// of split tiles.
inline int attn_grid(AttnArgs& b, int BQ) {
    // query rows of the longest chunk: Tc frames, or all T when one chunk covers the clip
    const int qlen = (b.stream ? b.s_frames : (b.Tc < b.T ? b.Tc : b.T)) * b.n;
    b.tiles_per_chunk = (qlen + BQ - 1) / BQ;
    b.total_tiles = b.tiles_per_chunk * b.nchunks * b.BH;
    const int64_t NL = (int64_t)(b.nchunks - 1) * b.BH * b.tiles_per_chunk, NS = (int64_t)b.BH * b.tiles_per_chunk;
    int most = 0, splits = 0;
    for (int x = 0; x < 8; ++x) {
        const int ks = xcd_splits(NS, b.split_per_xcd, x);
        const int cnt = xcd_share(NL, x) + xcd_share(NS, x) + ks;
        most = cnt > most ? cnt : most;
        splits += ks;
    }
    b.per_xcd = most;
    return splits;
}

// Raise the dynamic LDS limit of a kernel once per device (idempotent, so a race between
// host threads only repeats the call).
inline hipError_t ensure_lds(const void* fn, size_t lds, size_t (&done)[64]) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
    if (lds > done[dev]) {
        hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
        done[dev] = lds;
    }
    return hipSuccess;
}

}  // namespace rehyat
