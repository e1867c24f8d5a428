// attn.hip -- windowed softmax tile kernel with the linear part and the shared
// normalisation fused into its epilogue (ReHyAt blog, maplevalley.com.cn, 2.2.1-2.3).
//
// One workgroup = 4 waves x 32 queries of one chunk of one (batch, head).  The chunk's
// softmax window (its own frames plus To preceding frames, bidirectional) is streamed
// through LDS in 64-token tiles, double-buffered through registers.  Per tile and wave:
//   S^T (keys x queries) = K . Q^T  on MFMA, so every lane owns one query column and the
//      statistics of that query live in one lane pair (lane, lane^32);
//   online softmax in the log2 domain: p = exp2(s*log2(e)/sqrt(D) - m); the running max m
//      is only moved when a tile raises it by more than 2^8 (the accumulators are then
//      rescaled); otherwise the stale m is kept, which is exact because the final
//      normalisation uses the same m;
//   O^T (d x queries) += V^T . P^T on MFMA, with P^T taken directly from the S^T
//      registers (contraction slots follow the C layout, V^T is staged in that order).
// Only the last tile of a window can be ragged; it runs a separate masked copy of the
// tile step after the loop, so full tiles carry no bounds arithmetic.
#include <type_traits>

#include "attn_common.hpp"

namespace rehyat {

static constexpr float kRescaleThreshold = 8.0f;  // log2 units

template <class T, class OT, int D, int QB, int NW, bool STREAM>
__global__ __launch_bounds__(NW * 64, 2) void attn_kernel(const AttnArgs a) {
    using M = Mfma<T>;
    constexpr int NT = NW * 64;
    using Tile = KVTile<T, D, NT>;
    constexpr int KS = M::KS, EPL = M::EPL, NS = D / KS, NDB = D / 32;
    constexpr int BQ = NW * QB * 32;
    constexpr int TPB = 16 / EPL;  // MFMA steps per 32-token block of the value product

    extern __shared__ __align__(16) unsigned char smem[];
    T* Ks0 = reinterpret_cast<T*>(smem);
    T* Vs0 = Ks0 + Tile::K_ELEMS;
    T* Ks1 = Vs0 + Tile::V_ELEMS;
    T* Vs1 = Ks1 + Tile::K_ELEMS;

    Window<T> w;
    if (!decode_window<T, D, STREAM>(a, w)) return;
    if (w.qt * BQ >= w.Lq) return;
    const int Lk = w.Lk;
    const bool has_lin = w.ls > 0;
    const bool has_soft = Lk > 0;

    const int tid = threadIdx.x;
    const int wave = tid / 64, lane = tid % 64, col = lane % 32, h = lane / 32;
    const int qw = w.qt * BQ + wave * QB * 32;  // first query (chunk-local) of this wave
    const bool wave_live = qw < w.Lq;            // waves past the chunk end only stage tiles
    const T* qs = reinterpret_cast<const T*>(a.q) + (int64_t)w.bh * a.q_bh_stride + (int64_t)w.q0 * D;

    // ---- Q^T operand registers (B operand of S^T = K Q^T and of u^T = W Q^T) ----
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
        // S^T = K Q^T.  Scheduling hint: four K operand reads in flight ahead of the matrix
        // core, then one read per MFMA, so LDS latency hides behind the products.
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);  // 4 LDS reads
#pragma unroll
        for (int i = 0; i < 2 * NS * QB; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // 1 MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // 1 LDS read
        }
        f32x16 sacc[2][QB];
        typename M::frag ka[2], kn[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) ka[kb] = Tile::kfrag(Ks, kb, 0, col, h);
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            if (s + 1 < NS) {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) kn[kb] = Tile::kfrag(Ks, kb, s + 1, col, h);
            }
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int qb = 0; qb < QB; ++qb)
                    sacc[kb][qb] = M::mma(ka[kb], qf[qb][s], s == 0 ? zero16() : sacc[kb][qb]);
            if (s + 1 < NS) {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) ka[kb] = kn[kb];
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
            mx = pair_max(mx);
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

        // O^T += V^T P^T; the V operands of the next step are read while this one runs
        constexpr int NV = 2 * TPB * NDB;
        typename M::frag va = Tile::vfrag(Vs, col, 0, 0, h), vn;
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int db = i % NDB, t = (i / NDB) % TPB, kb = i / (NDB * TPB);
            if (i + 1 < NV) {
                const int db1 = (i + 1) % NDB, t1 = ((i + 1) / NDB) % TPB, kb1 = (i + 1) / (NDB * TPB);
                vn = Tile::vfrag(Vs, db1 * 32 + col, kb1, t1, h);
            }
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) oacc[db][qb] = M::mma(va, pf[kb][t][qb], oacc[db][qb]);
            if (i + 1 < NV) va = vn;
        }
    };

    // full tiles in the loop; a ragged last tile is peeled off after it
    const int nfull = ragged ? ntiles - 1 : ntiles;
    if (ntiles > 0) {
        if (nfull == 0) tile.template load<true, STREAM>(w.src, 0, Lk, tid);
        else tile.template load<false, STREAM>(w.src, 0, Lk, tid);
        tile.store(Ks0, Vs0, tid);
    }
    __syncthreads();
    for (int it = 0; it < nfull; ++it) {
        const T* Ks = (it & 1) ? Ks1 : Ks0;
        const T* Vs = (it & 1) ? Vs1 : Vs0;
        const int t0 = it * Tile::BK;
        const bool more = it + 1 < ntiles;
        if (more) {
            if (it + 1 == nfull) tile.template load<true, STREAM>(w.src, t0 + Tile::BK, Lk, tid);
            else tile.template load<false, STREAM>(w.src, t0 + Tile::BK, Lk, tid);
        }
        if (wave_live) tile_step(Ks, Vs, t0, std::false_type{});
        if (more) tile.store((it & 1) ? Ks0 : Ks1, (it & 1) ? Vs0 : Vs1, tid);
        __syncthreads();
    }
    if (ragged && wave_live) tile_step((nfull & 1) ? Ks1 : Ks0, (nfull & 1) ? Vs1 : Vs0, nfull * Tile::BK, std::true_type{});

    float l_tot[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) l_tot[qb] = l_run[qb] + other_half(l_run[qb]);

    linear_and_merge<T, OT, D, QB, NT>(a, w, smem, qw, has_soft, has_lin, qf, oacc, m_run, l_tot);
}

template <class T, class OT, int D, bool STREAM>
static hipError_t launch_one(const AttnArgs& a, hipStream_t stream) {
    constexpr int QB = 1, NW = 4;
    using Tile = KVTile<T, D, NW * 64>;
    const size_t kv = 2 * (size_t)(Tile::K_ELEMS + Tile::V_ELEMS) * sizeof(T);
    const size_t epi = epilogue_lds_bytes<T, D>(a.Dphi);
    const size_t lds = kv > epi ? kv : epi;
    auto fn = attn_kernel<T, OT, D, QB, NW, STREAM>;
    static size_t lds_set[64] = {};
    hipError_t e = ensure_lds(reinterpret_cast<const void*>(fn), lds, lds_set);
    if (e != hipSuccess) return e;
    AttnArgs b = a;
    b.split_per_xcd = 0;  // no tail split in this kernel
    attn_grid(b, NW * QB * 32);
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

hipError_t launch_attn(const AttnArgs& a, int in_dtype, int out_dtype, hipStream_t stream) {
    if (in_dtype == 1) return launch_attn_wide(a, out_dtype, stream);
    if (out_dtype == 1) return a.stream ? launch_d<float, bf16, true>(a, stream) : launch_d<float, bf16, false>(a, stream);
    return a.stream ? launch_d<float, float, true>(a, stream) : launch_d<float, float, false>(a, stream);
}

}  // namespace rehyat
