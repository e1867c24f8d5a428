// attn.hip -- windowed softmax tile kernel with the linear part and the shared
// normalisation fused into its epilogue (ReHyAt blog, maplevalley.com.cn, 2.2.1-2.3).
//
// One workgroup = NW waves = BQ = NW*QB*32 queries of one chunk of one (batch, head).
// The chunk's softmax window (its own frames plus To preceding frames, bidirectional) is
// streamed through LDS in 64-token tiles, double-buffered through registers.  Per tile
// and wave:
//   S^T (keys x queries) = K . Q^T  on MFMA, so every lane owns one query column and the
//      row statistics of that query live in one lane pair (lane, lane^32);
//   online softmax in the log2 domain: p = exp2(s*log2(e)/sqrt(D) - m); the running max m
//      is only moved when a tile raises it by more than 2^8 (the accumulators are then
//      rescaled); otherwise the stale m is kept, which is exact because the final
//      normalisation uses the same m;
//   O^T (d x queries) += V^T . P^T on MFMA, with P^T taken directly from the S^T
//      registers (contraction slots follow the C layout, V^T is staged in that order).
// Epilogue (chunks with a linear region): u = W_q q (MFMA, reusing the Q operand
// registers), phi = per-part powers of softplus(u + b), y = phi S_c and z = phi . Z_c
// (S_c staged in LDS), then out = (2^m O + y) / (2^m l + z), scaled by 2^-max(m,0).
#include "tiles.hpp"
#include "kernels.hpp"

#ifndef REHYAT_ATTN_QB
#define REHYAT_ATTN_QB 2
#endif

namespace rehyat {

static constexpr float kRescaleThreshold = 8.0f;  // log2 units

template <class T, class OT, int D, int QB, int NW>
__global__ __launch_bounds__(NW * 64) void attn_kernel(const AttnArgs a) {
    using M = Mfma<T>;
    using Tile = KVTile<T, D, NW * 64>;
    constexpr int KS = M::KS, EPL = M::EPL, NS = D / KS, NDB = D / 32;
    constexpr int BQ = NW * QB * 32;
    constexpr int NT = NW * 64;
    constexpr int TPB = 16 / EPL;  // MFMA steps per 32-token block of the value product

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
    int64_t s_off, z_off;
    if (!a.stream) {
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
        src.len1 = Lk;
        s_off = (int64_t)bh * a.S_bh_stride + (int64_t)max(ls - 1, 0) * a.S_frame_stride;
        z_off = (int64_t)bh * a.Z_bh_stride + (int64_t)max(ls - 1, 0) * a.Z_frame_stride;
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
        s_off = (int64_t)bh * a.S_bh_stride;
        z_off = (int64_t)bh * a.Z_bh_stride;
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
    Tile tile;
    if (ntiles > 0) {
        tile.load(src, 0, Lk, tid);
        tile.store(Ks0, Vs0, tid);
    }
    __syncthreads();

    for (int it = 0; it < ntiles; ++it) {
        T* Ks = (it & 1) ? Ks1 : Ks0;
        T* Vs = (it & 1) ? Vs1 : Vs0;
        const int t0 = it * Tile::BK;
        const bool more = it + 1 < ntiles;
        if (more) tile.load(src, t0 + Tile::BK, Lk, tid);

        // S^T = K Q^T for 2 key blocks x QB query blocks
        f32x16 sacc[2][QB];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) sacc[kb][qb] = zero16();
#pragma unroll
        for (int s = 0; s < NS; ++s) {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                const typename M::frag af = Tile::kfrag(Ks, kb, s, col, h);
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) sacc[kb][qb] = M::mma(af, qf[qb][s], sacc[kb][qb]);
            }
        }
        if (t0 + Tile::BK > Lk) {  // ragged last tile: keys beyond the window get -inf
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

        // O^T += V^T P^T
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

        if (more) tile.store((it & 1) ? Ks0 : Ks1, (it & 1) ? Vs0 : Vs1, tid);
        __syncthreads();
    }

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
        const int Dphi = a.Dphi, P = a.P, F = Dphi * P, NJB = Dphi / 32;
        const int SLD = F + Tile::VEC;
        T* Ss = reinterpret_cast<T*>(smem);
        float* Zs = reinterpret_cast<float*>(smem + (size_t)D * SLD * sizeof(T));
        const float* Sg = a.S + s_off;
        const float* Zg = a.Z + z_off;
        // stage S_c^T in LDS as Ss[d][(pw-1)*Dphi + 32-block slot order of j], Z_c as Zs[(pw-1)*Dphi + j]
        if (a.s_lds) {
            const int items = (Dphi / 4) * P * (D / 8);
            for (int it = tid; it < items; it += NT) {
                const int dc = it % (D / 8);
                const int jq = (it / (D / 8)) % (Dphi / 4);
                const int pw = it / ((D / 8) * (Dphi / 4)) + 1;
                const int j0 = jq * 4;
                float v[4][8];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float* srow = Sg + (int64_t)feat_index(j0 + i, pw, Dphi, P) * D + dc * 8;
                    const float4 lo = *reinterpret_cast<const float4*>(srow);
                    const float4 hi = *reinterpret_cast<const float4*>(srow + 4);
                    v[i][0] = lo.x; v[i][1] = lo.y; v[i][2] = lo.z; v[i][3] = lo.w;
                    v[i][4] = hi.x; v[i][5] = hi.y; v[i][6] = hi.z; v[i][7] = hi.w;
                }
#pragma unroll
                for (int jj = 0; jj < 8; ++jj) {
                    const int d = dc * 8 + jj;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int j = j0 + i;
                        Ss[d * SLD + (pw - 1) * Dphi + (j / 32) * 32 + slot_pos<EPL>(j % 32)] = from_float<T>(v[i][jj]);
                    }
                }
            }
            for (int it = tid; it < F; it += NT) {
                const int j = it % Dphi, pw = it / Dphi + 1;
                Zs[it] = Zg[feat_index(j, pw, Dphi, P)];
            }
            __syncthreads();
        }

        const T* wq = reinterpret_cast<const T*>(a.wq) + (int64_t)hh * Dphi * D;
        const float* bq = a.bq ? a.bq + (int64_t)hh * Dphi : nullptr;
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            float zpart = 0.f;
            for (int jb = 0; jb < NJB; ++jb) {
                f32x16 u = zero16();
#pragma unroll
                for (int s = 0; s < NS; ++s) {
                    const typename M::frag wf = M::load(wq + (int64_t)(jb * 32 + col) * D + s * KS + h * EPL);
                    u = M::mma(wf, qf[qb][s], u);
                }
                float uu[16], ph[16];
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float x = u[r] + (bq ? bq[jb * 32 + crow(r, h)] : 0.f);
                    uu[r] = softplus(x);
                    ph[r] = uu[r];
                }
                for (int pw = 1; pw <= P; ++pw) {
                    if (pw > 1) {
#pragma unroll
                        for (int r = 0; r < 16; ++r) ph[r] *= uu[r];
                    }
                    const int blk = (pw - 1) * NJB + jb;
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int jr = jb * 32 + crow(r, h);
                        zpart += ph[r] * (a.s_lds ? Zs[(pw - 1) * Dphi + jr] : Zg[feat_index(jr, pw, Dphi, P)]);
                    }
#pragma unroll
                    for (int t = 0; t < TPB; ++t) {
                        const typename M::frag bfr = M::pack(ph + t * EPL);
#pragma unroll
                        for (int db = 0; db < NDB; ++db) {
                            const int d = db * 32 + col;
                            typename M::frag sf;
                            if (a.s_lds) {
                                sf = M::load(Ss + d * SLD + blk * 32 + t * 2 * EPL + h * EPL);
                            } else {  // operand gathered from the fp32 state in memory
                                float sv[EPL];
#pragma unroll
                                for (int e = 0; e < EPL; ++e)
                                    sv[e] = Sg[(int64_t)feat_index(jb * 32 + crow(t * EPL + e, h), pw, Dphi, P) * D + d];
                                sf = M::pack(sv);
                            }
                            yacc[db][qb] = M::mma(sf, bfr, yacc[db][qb]);
                        }
                    }
                }
            }
            zq[qb] = zpart + other_half(zpart);
        }
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

template <class T, class OT, int D, int QB, int NW>
static hipError_t launch_one(const AttnArgs& a, hipStream_t stream) {
    using Tile = KVTile<T, D, NW * 64>;
    const size_t kv = 2 * (size_t)(Tile::K_ELEMS + Tile::V_ELEMS) * sizeof(T);
    const size_t st = (size_t)D * (a.Dphi * a.P + Tile::VEC) * sizeof(T) + (size_t)a.Dphi * a.P * sizeof(float);
    const size_t lds_max = 160 * 1024;
    const bool s_lds = st <= lds_max;
    const size_t lds = (s_lds && st > kv) ? st : kv;
    auto fn = attn_kernel<T, OT, D, QB, NW>;
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
    b.s_lds = s_lds ? 1 : 0;
    constexpr int BQ = NW * QB * 32;
    const int qlen = a.stream ? a.s_frames * a.n : a.Tc * a.n;
    b.tiles_per_chunk = (qlen + BQ - 1) / BQ;
    b.total_tiles = b.tiles_per_chunk * b.nchunks * b.BH;
    b.per_xcd = (b.total_tiles + 7) / 8;
    hipLaunchKernelGGL(fn, dim3(8 * b.per_xcd), dim3(NW * 64), lds, stream, b);
    return hipGetLastError();
}

template <class T, class OT>
static hipError_t launch_dt(const AttnArgs& a, hipStream_t stream) {
    constexpr int QB = sizeof(T) == 2 ? REHYAT_ATTN_QB : 1;
    switch (a.D) {
        case 32: return launch_one<T, OT, 32, QB, 4>(a, stream);
        case 64: return launch_one<T, OT, 64, QB, 4>(a, stream);
        case 128: return launch_one<T, OT, 128, QB, 4>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_attn(const AttnArgs& a, int in_dtype, int out_dtype, hipStream_t stream) {
    if (in_dtype == 1) {
        return out_dtype == 1 ? launch_dt<bf16, bf16>(a, stream) : launch_dt<bf16, float>(a, stream);
    }
    return out_dtype == 1 ? launch_dt<float, bf16>(a, stream) : launch_dt<float, float>(a, stream);
}

}  // namespace rehyat
