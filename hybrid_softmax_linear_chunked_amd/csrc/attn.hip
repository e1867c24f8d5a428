// attn.hip -- windowed softmax tile kernel with the linear part and the shared
// normalisation fused into its epilogue (ReHyAt blog, maplevalley.com.cn, 2.2.1-2.3).
//
// One workgroup = 4 waves x 32 queries of one chunk of one (batch, head); two workgroups
// share a CU (each wave stays under 256 VGPRs), so the softmax arithmetic of one
// workgroup overlaps the matrix-core work of the other -- they meet at no common barrier.
// The chunk's softmax window (its own frames plus To preceding frames, bidirectional) is
// streamed through LDS in 64-token tiles, double-buffered through registers.  Per tile
// and wave:
//   S^T (keys x queries) = K . Q^T  on MFMA, so every lane owns one query column and the
//      statistics of that query live in one lane pair (lane, lane^32);
//   online softmax in the log2 domain: p = exp2(s*log2(e)/sqrt(D) - m); the running max m
//      is only moved when a tile raises it by more than 2^8 (the accumulators are then
//      rescaled); otherwise the stale m is kept, which is exact because the final
//      normalisation uses the same m;
//   O^T (d x queries) += V^T . P^T on MFMA, with P^T taken directly from the S^T
//      registers (contraction slots follow the C layout, V^T is staged in that order).
// Only the last tile of a window can be ragged; it runs a separate masked copy of the
// tile step, so full tiles carry no bounds arithmetic.
// Epilogue (chunks with a linear region): W_q is staged in LDS and u = W_q q computed on
// MFMA from the Q operand registers; phi = per-part powers of softplus(u + b).  For each
// power the chunk's state image (S_c rows for that power, written by the scan kernel in
// the operand order used here) is staged in LDS, y += S_c^T phi on MFMA and
// z += phi . Z_c; finally out = (2^m O + y) / (2^m l + z), scaled by 2^-max(m,0).
#include <type_traits>

#include "tiles.hpp"
#include "kernels.hpp"

namespace rehyat {

static constexpr float kRescaleThreshold = 8.0f;  // log2 units

template <class T, int D, int NT>
struct AttnLds {
    using Tile = KVTile<T, D, NT>;
    static constexpr int VEC = Tile::VEC;
    static constexpr size_t kv_bytes = 2 * (size_t)(Tile::K_ELEMS + Tile::V_ELEMS) * sizeof(T);
    // epilogue: W_q [Dphi][D + VEC] and one power of the state image [D][Dphi + VEC]
    static size_t epi_bytes(int Dphi) {
        return ((size_t)Dphi * (D + VEC) + (size_t)D * (Dphi + VEC)) * sizeof(T);
    }
    static size_t bytes(int Dphi) { return kv_bytes > epi_bytes(Dphi) ? kv_bytes : epi_bytes(Dphi); }
};

template <class T, class OT, int D, int QB, int NW, bool STREAM>
__global__ __launch_bounds__(NW * 64, 2) void attn_kernel(const AttnArgs a) {
    using M = Mfma<T>;
    constexpr int NT = NW * 64;
    using Tile = KVTile<T, D, NT>;
    constexpr int KS = M::KS, EPL = M::EPL, NS = D / KS, NDB = D / 32;
    constexpr int BQ = NW * QB * 32;
    constexpr int TPB = 16 / EPL;  // MFMA steps per 32-token block of the value product
    constexpr int VEC = Tile::VEC;

    extern __shared__ __align__(16) unsigned char smem[];
    T* Ks0 = reinterpret_cast<T*>(smem);
    T* Vs0 = Ks0 + Tile::K_ELEMS;
    T* Ks1 = Vs0 + Tile::V_ELEMS;
    T* Vs1 = Ks1 + Tile::K_ELEMS;

    // ---- which (batch-head, chunk, query tile): consecutive logical ids share a chunk and
    // are placed on one XCD (workgroups are dealt round-robin over the 8 XCDs) ----
    const int wgid = blockIdx.x;
    const int L = (wgid % 8) * a.per_xcd + wgid / 8;
    if (L >= a.total_tiles) return;
    const int qt = L % a.tiles_per_chunk;
    const int rest = L / a.tiles_per_chunk;
    const int c = rest % a.nchunks;
    const int bh = rest / a.nchunks;
    const int hh = bh % a.H;

    int q0, Lq, Lk, ls;
    KeySrc<T> src;
    const T* kb1 = reinterpret_cast<const T*>(a.k1) + (int64_t)bh * a.kv1_bh_stride;
    const T* vb1 = reinterpret_cast<const T*>(a.v1) + (int64_t)bh * a.kv1_bh_stride;
    int img_slot;
    if constexpr (!STREAM) {
        const int f0 = c * a.Tc;
        const int f1 = min(f0 + a.Tc, a.T);
        const int ws = a.linear_only ? f1 : max(0, f0 - a.To);
        q0 = f0 * a.n;
        Lq = (f1 - f0) * a.n;
        Lk = (f1 - ws) * a.n;
        ls = ws;
        src.k1 = kb1 + (int64_t)ws * a.n * D;
        src.v1 = vb1 + (int64_t)ws * a.n * D;
        src.k2 = src.k1;
        src.v2 = src.v1;
        src.len1 = 1 << 30;
        img_slot = bh * a.img_slots + c;
    } else {
        q0 = 0;
        Lq = a.s_frames * a.n;
        Lk = a.linear_only ? 0 : (a.s_held + a.s_frames) * a.n;
        ls = a.s_ls;
        src.k1 = kb1;
        src.v1 = vb1;
        src.k2 = reinterpret_cast<const T*>(a.k2) + (int64_t)bh * a.kv2_bh_stride;
        src.v2 = reinterpret_cast<const T*>(a.v2) + (int64_t)bh * a.kv2_bh_stride;
        src.len1 = a.s_held * a.n;
        img_slot = bh;
    }
    if (qt * BQ >= Lq) return;
    const bool has_lin = ls > 0;
    const bool has_soft = Lk > 0;

    const int tid = threadIdx.x;
    const int wave = tid / 64, lane = tid % 64, col = lane % 32, h = lane / 32;
    const int qw = qt * BQ + wave * QB * 32;  // first query (chunk-local) of this wave
    const T* qs = reinterpret_cast<const T*>(a.q) + (int64_t)bh * a.q_bh_stride + (int64_t)q0 * D;

    // ---- Q^T operand registers (B operand of S^T = K Q^T and of u^T = W Q^T) ----
    typename M::frag qf[QB][NS];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const int row = qw + qb * 32 + col;
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            if (row < Lq) {
                qf[qb][s] = M::load(qs + (int64_t)row * D + s * KS + h * EPL);
            } else {
                float zz[EPL];
#pragma unroll
                for (int e = 0; e < EPL; ++e) zz[e] = 0.f;
                qf[qb][s] = M::pack(zz);
            }
        }
    }

    f32x16 oacc[NDB][QB];
    float m_run[QB], l_run[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        m_run[qb] = -INFINITY;
        l_run[qb] = 0.f;
#pragma unroll
        for (int db = 0; db < NDB; ++db) oacc[db][qb] = zero16();
    }

    const float sc = a.scale_log2;
    const int ntiles = (Lk + Tile::BK - 1) / Tile::BK;
    const bool ragged = Lk % Tile::BK != 0;
    Tile tile;

    // one 64-token tile: S^T, online softmax, O^T update
    auto tile_step = [&](const T* Ks, const T* Vs, int t0, auto mask_tag) {
        constexpr bool MASK = decltype(mask_tag)::value;
        f32x16 sacc[2][QB];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            const typename M::frag af = Tile::kfrag(Ks, kb, 0, col, h);
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) sacc[kb][qb] = M::mma(af, qf[qb][0], zero16());
        }
#pragma unroll
        for (int s = 1; s < NS; ++s) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const typename M::frag af = Tile::kfrag(Ks, kb, s, col, h);
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) sacc[kb][qb] = M::mma(af, qf[qb][s], sacc[kb][qb]);
            }
        }
        if constexpr (MASK) {  // keys beyond the window get -inf
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    if (t0 + kb * 32 + crow(r, h) >= Lk)
#pragma unroll
                        for (int qb = 0; qb < QB; ++qb) sacc[kb][qb][r] = -INFINITY;
        }

        typename M::frag pf[2][TPB][QB];
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            float mx = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][qb][r]);
            mx = fmaxf(mx, other_half(mx));
            const float mnew = mx * sc;
            if (__ballot(mnew > m_run[qb] + kRescaleThreshold) != 0ull) {
                const float mnext = fmaxf(m_run[qb], mnew);
                const float alpha = __builtin_amdgcn_exp2f(m_run[qb] - mnext);
                m_run[qb] = mnext;
                l_run[qb] *= alpha;
#pragma unroll
                for (int db = 0; db < NDB; ++db)
#pragma unroll
                    for (int r = 0; r < 16; ++r) oacc[db][qb][r] *= alpha;
            }
            const float mneg = -m_run[qb];
            float lsum = 0.f;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                float pv[16];
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    pv[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][qb][r], sc, mneg));
                    lsum += pv[r];
                }
#pragma unroll
                for (int t = 0; t < TPB; ++t) pf[kb][t][qb] = M::pack(pv + t * EPL);
            }
            l_run[qb] += lsum;
        }

#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int t = 0; t < TPB; ++t)
#pragma unroll
                for (int db = 0; db < NDB; ++db) {
                    const typename M::frag vf = Tile::vfrag(Vs, db * 32 + col, kb, t, h);
#pragma unroll
                    for (int qb = 0; qb < QB; ++qb) oacc[db][qb] = M::mma(vf, pf[kb][t][qb], oacc[db][qb]);
                }
    };

    // full tiles in the loop; a ragged last tile is peeled off after it
    const int nfull = ragged ? ntiles - 1 : ntiles;
    if (ntiles > 0) {
        if (nfull == 0) tile.template load<true, STREAM>(src, 0, Lk, tid);
        else tile.template load<false, STREAM>(src, 0, Lk, tid);
        tile.store(Ks0, Vs0, tid);
    }
    __syncthreads();
    for (int it = 0; it < nfull; ++it) {
        const T* Ks = (it & 1) ? Ks1 : Ks0;
        const T* Vs = (it & 1) ? Vs1 : Vs0;
        const int t0 = it * Tile::BK;
        const bool more = it + 1 < ntiles;
        if (more) {
            if (it + 1 == nfull) tile.template load<true, STREAM>(src, t0 + Tile::BK, Lk, tid);
            else tile.template load<false, STREAM>(src, t0 + Tile::BK, Lk, tid);
        }
        tile_step(Ks, Vs, t0, std::false_type{});
        if (more) tile.store((it & 1) ? Ks0 : Ks1, (it & 1) ? Vs0 : Vs1, tid);
        __syncthreads();
    }
    if (ragged) tile_step((nfull & 1) ? Ks1 : Ks0, (nfull & 1) ? Vs1 : Vs0, nfull * Tile::BK, std::true_type{});

    float l_tot[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) l_tot[qb] = l_run[qb] + other_half(l_run[qb]);

    // ---- linear part: phi_q(q) S_c and phi_q(q) . Z_c ----
    f32x16 yacc[NDB][QB];
    float zq[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        zq[qb] = 0.f;
#pragma unroll
        for (int db = 0; db < NDB; ++db) yacc[db][qb] = zero16();
    }
    if (has_lin) {
        const int Dphi = a.Dphi, P = a.P, NJB = Dphi / 32;
        constexpr int WLD = D + VEC;        // W_q row stride in LDS
        const int SLD = Dphi + VEC;         // state-image row stride in LDS
        T* Ws = reinterpret_cast<T*>(smem);
        T* Ss = Ws + Dphi * WLD;
        const T* wq = reinterpret_cast<const T*>(a.wq) + (int64_t)hh * Dphi * D;
        const T* img = reinterpret_cast<const T*>(a.simg) + (int64_t)img_slot * P * D * Dphi;
        const float* zimg = a.zimg + (int64_t)img_slot * P * Dphi;
        const float* bq = a.bq ? a.bq + (int64_t)hh * Dphi : nullptr;

        __syncthreads();  // every wave is done with the K/V tiles (the peeled tile included)
        // stage W_q [Dphi][D] (16-byte chunks)
        for (int i = tid; i < Dphi * (D / VEC); i += NT) {
            const int j = i / (D / VEC), ch = i % (D / VEC);
            *reinterpret_cast<uint4*>(Ws + j * WLD + ch * VEC) = *reinterpret_cast<const uint4*>(wq + (int64_t)j * D + ch * VEC);
        }
        __syncthreads();
        // u = softplus(W_q q + b) for every block of 32 phi rows (lane: one query, 16 rows)
        constexpr int JBMAX = 4;  // Dphi <= 128
        float uu[JBMAX][QB][16];
#pragma unroll
        for (int jb = 0; jb < JBMAX; ++jb) {
            if (jb >= NJB) break;
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
                f32x16 u = M::mma(M::load(Ws + (jb * 32 + col) * WLD + h * EPL), qf[qb][0], zero16());
#pragma unroll
                for (int s = 1; s < NS; ++s) u = M::mma(M::load(Ws + (jb * 32 + col) * WLD + s * KS + h * EPL), qf[qb][s], u);
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float x = u[r] + (bq ? bq[jb * 32 + crow(r, h)] : 0.f);
                    uu[jb][qb][r] = softplus_fast<T>(x);
                }
            }
        }
        for (int pw = 1; pw <= P; ++pw) {
            __syncthreads();  // W_q / previous power no longer read
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
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) {
                    float ph[16];
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        float v = uu[jb][qb][r];
                        for (int e = 1; e < pw; ++e) v *= uu[jb][qb][r];
                        ph[r] = v;
                        zq[qb] += v * zp[jb * 32 + crow(r, h)];
                    }
#pragma unroll
                    for (int t = 0; t < TPB; ++t) {
                        const typename M::frag bfr = M::pack(ph + t * EPL);
#pragma unroll
                        for (int db = 0; db < NDB; ++db) {
                            const typename M::frag sf = M::load(Ss + (db * 32 + col) * SLD + jb * 32 + t * 2 * EPL + h * EPL);
                            yacc[db][qb] = M::mma(sf, bfr, yacc[db][qb]);
                        }
                    }
                }
            }
        }
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) zq[qb] += other_half(zq[qb]);
    }

    // ---- merge and write ----
    OT* outs = reinterpret_cast<OT*>(a.out) + (int64_t)bh * a.q_bh_stride + (int64_t)q0 * D;
    const int64_t arow0 = (int64_t)bh * a.aux_bh_stride + q0;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const int row = qw + qb * 32 + col;
        if (row >= Lq) continue;
        float ca, cg;
        if (has_soft && has_lin) {
            const float M2 = fmaxf(m_run[qb], 0.f);
            const float ea = __builtin_amdgcn_exp2f(m_run[qb] - M2);
            const float eg = __builtin_amdgcn_exp2f(-M2);
            const float inv = 1.f / (ea * l_tot[qb] + eg * zq[qb]);
            ca = ea * inv;
            cg = eg * inv;
        } else if (has_soft) {
            ca = 1.f / l_tot[qb];
            cg = 0.f;
        } else {
            ca = 0.f;
            cg = 1.f / zq[qb];
        }
        OT* orow = outs + (int64_t)row * D;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int d = db * 32 + g * 8 + h * 4;
                float vals[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) vals[i] = ca * oacc[db][qb][g * 4 + i] + cg * yacc[db][qb][g * 4 + i];
                if constexpr (sizeof(OT) == 4) {
                    *reinterpret_cast<float4*>(orow + d) = make_float4(vals[0], vals[1], vals[2], vals[3]);
                } else {
                    bf16x4 o4;
#pragma unroll
                    for (int i = 0; i < 4; ++i) o4[i] = (bf16)vals[i];
                    *reinterpret_cast<bf16x4*>(orow + d) = o4;
                }
            }
        if (a.aux_o_soft || a.aux_y) {
            const float il = has_soft ? 1.f / l_tot[qb] : 0.f;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int d = db * 32 + g * 8 + h * 4;
                    float4 so, yo;
                    so.x = oacc[db][qb][g * 4 + 0] * il; so.y = oacc[db][qb][g * 4 + 1] * il;
                    so.z = oacc[db][qb][g * 4 + 2] * il; so.w = oacc[db][qb][g * 4 + 3] * il;
                    yo.x = yacc[db][qb][g * 4 + 0]; yo.y = yacc[db][qb][g * 4 + 1];
                    yo.z = yacc[db][qb][g * 4 + 2]; yo.w = yacc[db][qb][g * 4 + 3];
                    if (a.aux_o_soft) *reinterpret_cast<float4*>(a.aux_o_soft + (arow0 + row) * D + d) = so;
                    if (a.aux_y) *reinterpret_cast<float4*>(a.aux_y + (arow0 + row) * D + d) = yo;
                }
        }
        if (h == 0) {
            if (a.aux_lse) a.aux_lse[arow0 + row] = has_soft ? m_run[qb] * 0.6931471805599453f + logf(l_tot[qb]) : -INFINITY;
            if (a.aux_z) a.aux_z[arow0 + row] = zq[qb];
        }
    }
}

template <class T, class OT, int D, bool STREAM>
static hipError_t launch_one(const AttnArgs& a, hipStream_t stream) {
    constexpr int QB = 1, NW = 4;
    using LDS = AttnLds<T, D, NW * 64>;
    const size_t lds = LDS::bytes(a.Dphi);
    auto fn = attn_kernel<T, OT, D, QB, NW, STREAM>;
    // raise the dynamic LDS limit of this instantiation once per device (idempotent, so a
    // race between host threads only repeats the call)
    static size_t lds_set[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
    if (lds > lds_set[dev]) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(fn), hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
        lds_set[dev] = lds;
    }
    AttnArgs b = a;
    constexpr int BQ = NW * QB * 32;
    const int qlen = a.stream ? a.s_frames * a.n : a.Tc * a.n;
    b.tiles_per_chunk = (qlen + BQ - 1) / BQ;
    b.total_tiles = b.tiles_per_chunk * b.nchunks * b.BH;
    b.per_xcd = (b.total_tiles + 7) / 8;
    hipLaunchKernelGGL(fn, dim3(8 * b.per_xcd), dim3(NW * 64), lds, stream, b);
    return hipGetLastError();
}

template <class T, class OT, bool STREAM>
static hipError_t launch_d(const AttnArgs& a, hipStream_t stream) {
    switch (a.D) {
        case 32: return launch_one<T, OT, 32, STREAM>(a, stream);
        case 64: return launch_one<T, OT, 64, STREAM>(a, stream);
        case 128: return launch_one<T, OT, 128, STREAM>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

template <class T, class OT>
static hipError_t launch_dt(const AttnArgs& a, hipStream_t stream) {
    return a.stream ? launch_d<T, OT, true>(a, stream) : launch_d<T, OT, false>(a, stream);
}

hipError_t launch_attn(const AttnArgs& a, int in_dtype, int out_dtype, hipStream_t stream) {
    if (in_dtype == 1) {
        return out_dtype == 1 ? launch_dt<bf16, bf16>(a, stream) : launch_dt<bf16, float>(a, stream);
    }
    return out_dtype == 1 ? launch_dt<float, bf16>(a, stream) : launch_dt<float, float>(a, stream);
}

}  // namespace rehyat
