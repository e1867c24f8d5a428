// state.hip -- linear-attention state of ReHyAt (blog, maplevalley.com.cn, section 2.3:
// S = sum phi_k(K)^T V, Z = sum phi_k(K), updated by the frames that leave the softmax
// window).
//
// state_kernel: one workgroup per (batch-head, frame) computes the frame's partial
//   Delta_f = phi_k(K_f)^T V_f  (F x D)  and  sum_tokens phi_k(K_f)  (F),
//   with phi computed on the fly: u = K W_k^T on MFMA (tokens x Dphi), softplus, powers,
//   then Delta += phi^T V on MFMA with phi taken straight from the u registers (the C
//   tile's rows are the tokens, which is the contraction of the second product).  Two
//   forms: state16_kernel (bf16 inputs: 16x16x32 products, each wave owning 16 phi rows
//   over whole tiles, K/V moved by LDS-DMA) and state_kernel (float32 inputs: 32x32x2
//   products, wave (jb, ts) owning the 32 phi rows of block jb and the 32-token half ts
//   of every 64-token tile, the two halves summed through LDS in a fixed order).
// scan_kernel: running sum over frame partials in frame order, either in place (prefix
//   over the clip, chunk-parallel form) or added to a carried state (streaming form).
//   Both forms add the same partials in the same order, so they agree bit for bit.
// copy_kernel: keeps the last To frames of the window as the streaming overlap.
#include <type_traits>

#include "dma.hpp"
#include "kernels.hpp"
#include "tiles.hpp"

namespace rehyat {

// Waves: wave = jb * TS + ts.  With P <= 2 the 64-token tile is split between two waves
// (TS = 2, eight waves for Dphi = 128); with larger P one wave takes the whole tile so the
// P x D/32 accumulator tiles still fit in its registers.
template <int P>
struct StateShape {
    static constexpr int TS = P <= 2 ? 2 : 1;
    static constexpr int NW = 4 * TS;  // Dphi <= 128: at most 4 blocks of 32 phi rows
};

template <class T, int D, int P>
__global__ __launch_bounds__(StateShape<P>::NW * 64) void state_kernel(const StateArgs a) {
    using M = Mfma<T>;
    constexpr int TS = StateShape<P>::TS;
    constexpr int NT = StateShape<P>::NW * 64;
    using Tile = KVTile<T, D, NT>;
    constexpr int KS = M::KS, EPL = M::EPL, NS = D / KS, NDB = D / 32, TPB = 16 / EPL;

    extern __shared__ __align__(16) unsigned char smem[];
    T* Ks0 = reinterpret_cast<T*>(smem);
    T* Vs0 = Ks0 + Tile::K_ELEMS;
    T* Ks1 = Vs0 + Tile::V_ELEMS;
    T* Vs1 = Ks1 + Tile::K_ELEMS;

    const int gi = blockIdx.x % a.G;
    const int bh = blockIdx.x / a.G;
    const int hh = bh % a.H;
    const int g = a.g0 + gi;
    const int n = a.n, Dphi = a.Dphi, F = Dphi * P, NJB = Dphi / 32;

    KeySrc<T> src;
    if (g < a.nf1) {
        src.k1 = reinterpret_cast<const T*>(a.k1) + (int64_t)bh * a.kv1_bh_stride + (int64_t)g * n * D;
        src.v1 = reinterpret_cast<const T*>(a.v1) + (int64_t)bh * a.kv1_bh_stride + (int64_t)g * n * D;
    } else {
        src.k1 = reinterpret_cast<const T*>(a.k2) + (int64_t)bh * a.kv2_bh_stride + (int64_t)(g - a.nf1) * n * D;
        src.v1 = reinterpret_cast<const T*>(a.v2) + (int64_t)bh * a.kv2_bh_stride + (int64_t)(g - a.nf1) * n * D;
    }
    src.k2 = src.k1;
    src.v2 = src.v1;
    src.len1 = n;

    const int tid = threadIdx.x;
    const int wave = tid / 64, lane = tid % 64, col = lane % 32, h = lane / 32;
    const bool active = wave < TS * NJB;
    const int jb = wave / TS, ts = wave % TS;
    const int j = jb * 32 + col;  // this lane's phi row

    // W_k^T operand (B of u = K W^T): column j, contraction over d
    typename M::frag wf[NS];
    float bias = 0.f;
    if (active) {
        const T* wk = reinterpret_cast<const T*>(a.wk) + ((int64_t)hh * Dphi + j) * D;
#pragma unroll
        for (int s = 0; s < NS; ++s) wf[s] = M::load(wk + s * KS + h * EPL);
        if (a.bk) bias = a.bk[(int64_t)hh * Dphi + j];
    }

    f32x16 acc[P][NDB];
    float zacc[P];
#pragma unroll
    for (int pw = 0; pw < P; ++pw) {
        zacc[pw] = 0.f;
#pragma unroll
        for (int db = 0; db < NDB; ++db) acc[pw][db] = zero16();
    }

    const int ntiles = (n + Tile::BK - 1) / Tile::BK;
    Tile tile;
    tile.template load<true, false>(src, 0, n, tid);
    tile.store(Ks0, Vs0, tid);
    __syncthreads();
    for (int it = 0; it < ntiles; ++it) {
        const T* Ks = (it & 1) ? Ks1 : Ks0;
        const T* Vs = (it & 1) ? Vs1 : Vs0;
        const int t0 = it * Tile::BK;
        const bool more = it + 1 < ntiles;
        if (more) tile.template load<true, false>(src, t0 + Tile::BK, n, tid);
        if (active) {
#pragma unroll
            for (int sub = ts; sub < 2; sub += TS) {
                f32x16 u = zero16();
#pragma unroll
                for (int s = 0; s < NS; ++s) u = M::mma(Tile::kfrag(Ks, sub, s, col, h), wf[s], u);
                float uu[16], ph[16];
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const bool valid = t0 + sub * 32 + crow(r, h) < n;
                    uu[r] = valid ? softplus_fast<T>(u[r] + bias) : 0.f;
                    ph[r] = uu[r];
                }
#pragma unroll
                for (int pw = 0; pw < P; ++pw) {
                    if (pw > 0) {
#pragma unroll
                        for (int r = 0; r < 16; ++r) ph[r] *= uu[r];
                    }
#pragma unroll
                    for (int r = 0; r < 16; ++r) zacc[pw] += ph[r];
#pragma unroll
                    for (int t = 0; t < TPB; ++t) {
                        const typename M::frag af = M::pack(ph + t * EPL);
#pragma unroll
                        for (int db = 0; db < NDB; ++db)
                            acc[pw][db] = M::mma(af, Tile::vfrag(Vs, db * 32 + col, sub, t, h), acc[pw][db]);
                    }
                }
            }
        }
        if (more) tile.store((it & 1) ? Ks0 : Ks1, (it & 1) ? Vs0 : Vs1, tid);
        __syncthreads();
    }

    // with TS = 2, the ts = 1 wave hands its tiles to ts = 0 through LDS; then store
    float* red = reinterpret_cast<float*>(smem);  // [NJB][16 regs][64 lanes]
    float* Sp = a.Sp + ((int64_t)bh * a.G + gi) * F * D;
    float* Zp = a.Zp + ((int64_t)bh * a.G + gi) * F;
#pragma unroll
    for (int pw = 0; pw < P; ++pw) {
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
            if (TS == 2) {
                if (active && ts == 1) {
#pragma unroll
                    for (int r = 0; r < 16; ++r) red[(jb * 16 + r) * 64 + lane] = acc[pw][db][r];
                }
                __syncthreads();
            }
            if (active && ts == 0) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const float v = acc[pw][db][r] + (TS == 2 ? red[(jb * 16 + r) * 64 + lane] : 0.f);
                    const int f = feat_index(jb * 32 + crow(r, h), pw + 1, Dphi, P);
                    Sp[(int64_t)f * D + db * 32 + col] = v;
                }
            }
            if (TS == 2) __syncthreads();
        }
        const float zt = zacc[pw] + other_half(zacc[pw]);
        if (TS == 2) {
            if (active && ts == 1 && h == 0) red[jb * 32 + col] = zt;
            __syncthreads();
        }
        if (active && ts == 0 && h == 0) Zp[feat_index(j, pw + 1, Dphi, P)] = zt + (TS == 2 ? red[jb * 32 + col] : 0.f);
        if (TS == 2) __syncthreads();
    }
}

// bf16 form of state_kernel: the same per-(batch-head, frame) partials on 16x16x32 bf16
// products (v_mfma_f32_16x16x32_bf16; lane l = 16 g + a holds row a and contraction slots
// 8 g .. 8 g + 7 of the A operand, column a and the same slots of B, and column a, rows
// 4 g .. 4 g + 3 of C).  Wave w owns the 16 phi rows 16 w .. 16 w + 15 and takes every
// token of a 64-token tile:
//   u = K W_k^T: four C tiles of 16 tokens x 16 phi rows, lane (a, g) holding phi row a of
//     tokens 16 tb + 4 g + i (i = 0..3); A = K rows from LDS, B = W_k rows in registers;
//   Delta += phi^T V: the eight values of C tiles 2 c and 2 c + 1 in a lane are, as they
//     stand, the A operand of contraction block c (tokens 32 c + 4 g + i in slots i and
//     32 c + 16 + 4 g + i in slots 4 + i), and the V operand is read in the same slot
//     order with two transposing LDS reads; one accumulator tile per (power, 16 d).
// So the P x D/16 accumulator tiles of a wave hold 2 P D registers (P = 4 at D = 128: 128)
// and no partial is exchanged between waves.  K/V tiles move to LDS by LDS-DMA three
// tiles ahead (ring of four); V rows are D + 16 elements long, so the eight rows a
// transposing read spans fall in eight different 32-byte bank groups.  The frame's ragged
// last tile is processed first, with the padded tokens given phi = 0, so full tiles carry
// no bounds arithmetic.  Sums run in a fixed order, so the result does not depend on
// timing.
constexpr int kState16Waves = 8;  // Dphi <= 128: 16 phi rows per wave
constexpr int kState16Ring = 4;

template <int D>
using State16Tiles = DmaTiles<D, kState16Waves, D + 16>;

__device__ inline f32x4 mma16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

template <int D, int P>
__global__ __launch_bounds__(kState16Waves * 64) void state16_kernel(const StateArgs a) {
    using T = bf16;
    using Tile = State16Tiles<D>;
    constexpr int NW = kState16Waves, R = kState16Ring, BK = Tile::BK;
    constexpr int NS = D / 32;   // contraction steps of u
    constexpr int ND = D / 16;   // 16-column blocks of Delta
    constexpr int KLD = Tile::KLD, VLD = Tile::VLD;
    static_assert(BK == 64, "four 16-token C tiles per tile");

    extern __shared__ __align__(16) unsigned char smem[];
    T* const kring = reinterpret_cast<T*>(smem);
    T* const vring = kring + R * Tile::K_ELEMS;

    const int gi = blockIdx.x % a.G;
    const int bh = blockIdx.x / a.G;
    const int hh = bh % a.H;
    const int g = a.g0 + gi;
    const int n = a.n, Dphi = a.Dphi, F = Dphi * P;

    KeySrc<T> src;
    if (g < a.nf1) {
        src.k1 = reinterpret_cast<const T*>(a.k1) + (int64_t)bh * a.kv1_bh_stride + (int64_t)g * n * D;
        src.v1 = reinterpret_cast<const T*>(a.v1) + (int64_t)bh * a.kv1_bh_stride + (int64_t)g * n * D;
    } else {
        src.k1 = reinterpret_cast<const T*>(a.k2) + (int64_t)bh * a.kv2_bh_stride + (int64_t)(g - a.nf1) * n * D;
        src.v1 = reinterpret_cast<const T*>(a.v2) + (int64_t)bh * a.kv2_bh_stride + (int64_t)(g - a.nf1) * n * D;
    }
    src.k2 = src.k1;
    src.v2 = src.v1;
    src.len1 = n;

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid / 64);  // wave-uniform
    __builtin_assume(wave >= 0 && wave < NW);
    const int lane = tid % 64, la = lane % 16, lg = lane / 16;
    const bool active = wave * 16 < Dphi;
    const int j = wave * 16 + la;  // this lane's phi row

    bf16x8 wf[NS];  // B operand of u: W_k row j, d = 32 s + 8 lg .. + 7
    float bias = 0.f;
    if (active) {
        const T* wk = reinterpret_cast<const T*>(a.wk) + ((int64_t)hh * Dphi + j) * D + 8 * lg;
#pragma unroll
        for (int s = 0; s < NS; ++s) wf[s] = *reinterpret_cast<const bf16x8*>(wk + 32 * s);
        if (a.bk) bias = a.bk[(int64_t)hh * Dphi + j];
    }

    f32x4 acc[P][ND];
    float zacc[P];
#pragma unroll
    for (int pw = 0; pw < P; ++pw) {
        zacc[pw] = 0.f;
#pragma unroll
        for (int dc = 0; dc < ND; ++dc) acc[pw][dc] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    Tile tile;
    tile.init(wave, lane);
    // A operand of u: token 16 tb + la, d = 32 s + 8 lg; V operand: token 4 lg + la / 4 of
    // the contraction block, d = 4 (la % 4) of the 16-column block
    const int ka = la * KLD + 8 * lg;
    const int va = (4 * lg + la / 4) * VLD + 4 * (la % 4);
    const int nt = (n + BK - 1) / BK;
    const int last_len = n - (nt - 1) * BK;
    const bool ragged = last_len < BK;
    auto tile_of = [&](int i) { return i == 0 ? nt - 1 : i - 1; };  // ragged tile first
    auto kslot = [&](int i) { return kring + (i % R) * Tile::K_ELEMS; };
    auto vslot = [&](int i) { return vring + (i % R) * Tile::V_ELEMS; };
    auto dma = [&](int i) {
        const int t0 = tile_of(i) * BK;
        if (ragged && i == 0) {
            tile.template issue_k<true, false>(src, t0, n, kslot(i), wave);
            tile.template issue_v<true, false>(src, t0, n, vslot(i), wave);
        } else {
            tile.template issue_k<false, false>(src, t0, n, kslot(i), wave);
            tile.template issue_v<false, false>(src, t0, n, vslot(i), wave);
        }
    };
    // wait until the copy of tile i + 1 is complete in every wave: vector memory completes
    // in issue order, so each wave lets at most the batches of the later tiles it has
    // issued be outstanding, counted for the wave with the fewest DMA instructions (a
    // wave with more waits a little longer); lgkmcnt(0) retires this wave's reads of the
    // slot that the next copy overwrites
    constexpr int NMIN = Tile::NIK / NW + Tile::NIV / NW;
    static_assert(2 * NMIN <= 15, "vmcnt immediate range");
    auto tile_sync = [&](int later) {
        if (later >= 2) __builtin_amdgcn_s_waitcnt(0x0070 | (2 * NMIN));
        else if (later == 1) __builtin_amdgcn_s_waitcnt(0x0070 | NMIN);
        else __builtin_amdgcn_s_waitcnt(0x0070);
        asm volatile("s_barrier" ::: "memory");
    };

    // one 64-token tile; kl = valid tokens (64 unless the tile is ragged).  One body for
    // both kinds of tile (two copies in the loop would not fit in the registers together)
    auto process = [&](const T* Ks, const T* Vs, int kl) {
        // operands are read one step ahead of their products, and the scheduler is kept
        // from hoisting more reads (all of them in flight at once would not fit beside
        // the accumulators)
        auto kread = [&](int s, bf16x8 (&kf)[4]) {
#pragma unroll
            for (int tb = 0; tb < 4; ++tb) kf[tb] = *reinterpret_cast<const bf16x8*>(Ks + ka + tb * 16 * KLD + 32 * s);
        };
        f32x4 u[4];
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) u[tb] = f32x4{0.f, 0.f, 0.f, 0.f};
        bf16x8 kf[4], kn[4];
        kread(0, kf);
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            if (s + 1 < NS) kread(s + 1, kn);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int tb = 0; tb < 4; ++tb) u[tb] = mma16(kf[tb], wf[s], u[tb]);
            if (s + 1 < NS) {
#pragma unroll
                for (int tb = 0; tb < 4; ++tb) kf[tb] = kn[tb];
            }
        }
        float uu[16], ph[16];  // value i of C tile tb at 4 tb + i
#pragma unroll
        for (int tb = 0; tb < 4; ++tb) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                uu[4 * tb + i] = softplus_fast<T>(u[tb][i] + bias);
            }
        }
        if (kl < BK) {
#pragma unroll
            for (int r = 0; r < 16; ++r)
                if (16 * (r / 4) + 4 * lg + r % 4 >= kl) uu[r] = 0.f;
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) ph[r] = uu[r];
        bf16x8 af[P][2];
#pragma unroll
        for (int pw = 0; pw < P; ++pw) {
            if (pw > 0) {
#pragma unroll
                for (int r = 0; r < 16; ++r) ph[r] *= uu[r];
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) zacc[pw] += ph[r];
#pragma unroll
            for (int c = 0; c < 2; ++c) {
#pragma unroll
                for (int e = 0; e < 8; ++e) af[pw][c][e] = (bf16)ph[8 * c + e];
            }
        }
        auto vread = [&](int idx) {  // idx = c * ND + dc
            typedef short v4i16 __attribute__((ext_vector_type(4)));
            typedef short v8i16 __attribute__((ext_vector_type(8)));
            const T* p = Vs + va + 32 * (idx / ND) * VLD + 16 * (idx % ND);
            const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)(p));
            const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)(p + 16 * VLD));
            return __builtin_bit_cast(bf16x8, (v8i16)__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        };
        bf16x8 vf = vread(0);
#pragma unroll
        for (int idx = 0; idx < 2 * ND; ++idx) {
            const bf16x8 vn = idx + 1 < 2 * ND ? vread(idx + 1) : vf;
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int pw = 0; pw < P; ++pw) acc[pw][idx % ND] = mma16(af[pw][idx / ND], vf, acc[pw][idx % ND]);
            vf = vn;
        }
    };

    // prologue: copies of tiles 0 .. R-2, all complete (together with the W_k operands
    // above, so that no wait for those is left inside the loop)
    dma(0);
    if (nt > 1) dma(1);
    if (nt > 2) dma(2);
    tile_sync(0);
    for (int i = 0; i < nt; ++i) {
        if (i + R - 1 < nt) dma(i + R - 1);  // into the slot tile i - 1 used
        if (active) process(kslot(i), vslot(i), i == 0 ? last_len : BK);
        tile_sync(min(nt - 2 - i, 2));
    }

    if (active) {
        float* Sp = a.Sp + ((int64_t)bh * a.G + gi) * F * D;
        float* Zp = a.Zp + ((int64_t)bh * a.G + gi) * F;
#pragma unroll
        for (int pw = 0; pw < P; ++pw) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int f = feat_index(wave * 16 + 4 * lg + i, pw + 1, Dphi, P);
#pragma unroll
                for (int dc = 0; dc < ND; ++dc) Sp[(int64_t)f * D + 16 * dc + la] = acc[pw][dc][i];
            }
            // phi row j's column sum: the four lane groups, in a fixed order
            float z = zacc[pw] + __shfl_xor(zacc[pw], 16);
            z += __shfl_xor(z, 32);
            if (lg == 0) Zp[feat_index(j, pw + 1, Dphi, P)] = z;
        }
    }
}

// One workgroup per (batch-head, power, 32-feature block, 32-d block) of S, plus one per
// batch-head for Z.  Each thread carries four running sums; partials are read along d
// (coalesced) and every emitted image block goes through a 32 x 32 LDS tile so that it is
// written as whole 64-byte (bf16) rows of the image, features in slot order.
template <class T>
__global__ __launch_bounds__(256) void scan_kernel(const ScanArgs a) {
    constexpr int EPL = Mfma<T>::EPL;
    constexpr int EPC = 16 / sizeof(T);      // elements per 16-byte chunk
    constexpr int CPR = 32 * sizeof(T) / 16;  // 16-byte chunks per 32-element image row
    const int Dphi = a.Dphi, P = a.P, D = a.D, F = Dphi * P, NJB = Dphi / 32, NDB = D / 32;
    const int bh = blockIdx.y, tid = threadIdx.x;
    if (a.zero_cnt && blockIdx.x == 0 && bh == 0)
        for (int i = tid; i < a.nzero; i += 256) a.zero_cnt[i] = 0u;
    T* img = reinterpret_cast<T*>(a.simg) + (int64_t)bh * a.slots * F * D;
    float* zimg = a.zimg + (int64_t)bh * a.slots * F;
    const int nc = (a.T + a.Tc - 1) / a.Tc;
    auto ls_of = [&](int cc) {
        const int f0 = cc * a.Tc, f1 = min(f0 + a.Tc, a.T);
        return a.linear_only ? f1 : max(0, f0 - a.To);
    };

    if ((int)blockIdx.x < P * NJB * NDB) {
        __shared__ __align__(16) T tile[32][32 + EPC];  // [d][feature, slot order]
        const int blk = blockIdx.x;
        const int db = blk % NDB, jb = (blk / NDB) % NJB, pw = blk / (NDB * NJB) + 1;
        const int dl = tid % 32, jr = tid / 32;  // this thread: d = db*32 + dl, j = jb*32 + jr + 8k
        int64_t off[4];
        float acc[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            off[k] = (int64_t)feat_index(jb * 32 + jr + 8 * k, pw, Dphi, P) * D + db * 32 + dl;
            acc[k] = 0.f;
        }
        const float* base = a.Sp + (int64_t)bh * a.G * F * D;
        const int64_t stride = (int64_t)F * D;
        auto emit = [&](int slot) {
            __syncthreads();  // the previous block left the tile
#pragma unroll
            for (int k = 0; k < 4; ++k) tile[dl][slot_pos<EPL>(jr + 8 * k)] = from_float<T>(acc[k]);
            __syncthreads();
            if (tid < 32 * CPR) {
                const int row = tid / CPR, c = tid % CPR;
                T* dst = img + (int64_t)slot * F * D + ((int64_t)(pw - 1) * D + db * 32 + row) * Dphi + jb * 32 + c * EPC;
                *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(&tile[row][c * EPC]);
            }
        };
        if (a.S_state) {  // streaming: carried state + this step's frames, in frame order
            float* st = a.S_state + (int64_t)bh * F * D;
#pragma unroll
            for (int k = 0; k < 4; ++k) acc[k] = st[off[k]];
            for (int g = 0; g < a.G; ++g)
#pragma unroll
                for (int k = 0; k < 4; ++k) acc[k] += base[g * stride + off[k]];
#pragma unroll
            for (int k = 0; k < 4; ++k) st[off[k]] = acc[k];
            emit(0);
            return;
        }
        // chunk-parallel: prefix over frames; chunk c reads the prefix through frame ls(c) - 1
        int c = 0;
        while (c < nc && ls_of(c) == 0) ++c;
        for (int g = 0; g < a.G && c < nc; ++g) {
#pragma unroll
            for (int k = 0; k < 4; ++k) acc[k] += base[g * stride + off[k]];
            while (c < nc && ls_of(c) == g + 1) {
                emit(c);
                ++c;
            }
        }
        return;
    }

    // Z: [F] running sums per batch-head, image [P][Dphi] in plain feature order
    const float* zb = a.Zp + (int64_t)bh * a.G * F;
    for (int f = tid; f < F; f += 256) {
        int j, pw;
        feat_split(f, Dphi, P, j, pw);
        const int zo = (pw - 1) * Dphi + j;
        if (a.Z_state) {
            float* st = a.Z_state + (int64_t)bh * F + f;
            float acc = *st;
            for (int g = 0; g < a.G; ++g) acc += zb[(int64_t)g * F + f];
            *st = acc;
            zimg[zo] = acc;
            continue;
        }
        int c = 0;
        while (c < nc && ls_of(c) == 0) ++c;
        float acc = 0.f;
        for (int g = 0; g < a.G && c < nc; ++g) {
            acc += zb[(int64_t)g * F + f];
            while (c < nc && ls_of(c) == g + 1) {
                zimg[(int64_t)c * F + zo] = acc;
                ++c;
            }
        }
    }
}

__global__ __launch_bounds__(256) void copy_kernel(const CopyArgs a) {
    const int64_t frame_bytes = (int64_t)a.n * a.D * a.elem_bytes;
    const int64_t chunks = frame_bytes / 16;  // 16-byte pieces per frame
    const int64_t total = chunks * a.cnt;
    const int bh = blockIdx.y;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total; i += (int64_t)gridDim.x * 256) {
        const int fl = (int)(i / chunks);
        const int64_t off = (i % chunks) * 16;
        const int fs = a.f0 + fl;
        const char* sk;
        const char* sv;
        if (fs < a.nf1) {
            sk = reinterpret_cast<const char*>(a.s1k) + (bh * a.s1_bh_stride + (int64_t)fs * a.n * a.D) * a.elem_bytes;
            sv = reinterpret_cast<const char*>(a.s1v) + (bh * a.s1_bh_stride + (int64_t)fs * a.n * a.D) * a.elem_bytes;
        } else {
            sk = reinterpret_cast<const char*>(a.s2k) + (bh * a.s2_bh_stride + (int64_t)(fs - a.nf1) * a.n * a.D) * a.elem_bytes;
            sv = reinterpret_cast<const char*>(a.s2v) + (bh * a.s2_bh_stride + (int64_t)(fs - a.nf1) * a.n * a.D) * a.elem_bytes;
        }
        char* dk = reinterpret_cast<char*>(a.dk) + (bh * a.d_bh_stride + (int64_t)fl * a.n * a.D) * a.elem_bytes;
        char* dv = reinterpret_cast<char*>(a.dv) + (bh * a.d_bh_stride + (int64_t)fl * a.n * a.D) * a.elem_bytes;
        *reinterpret_cast<uint4*>(dk + off) = *reinterpret_cast<const uint4*>(sk + off);
        *reinterpret_cast<uint4*>(dv + off) = *reinterpret_cast<const uint4*>(sv + off);
    }
}

template <class T, int D, int P>
static hipError_t launch_state_t(const StateArgs& a, hipStream_t stream) {
    // bf16 takes the 16x16x32 LDS-DMA kernel, float32 the register-staged one
    constexpr bool kBf16 = sizeof(T) == 2;
    size_t lds;
    const void* fn;
    if constexpr (kBf16) {
        using Tile = State16Tiles<D>;
        lds = kState16Ring * (size_t)(Tile::K_ELEMS + Tile::V_ELEMS) * sizeof(T);
        fn = reinterpret_cast<const void*>(state16_kernel<D, P>);
    } else {
        using Tile = KVTile<T, D, StateShape<P>::NW * 64>;
        const size_t kv = 2 * (size_t)(Tile::K_ELEMS + Tile::V_ELEMS) * sizeof(T);
        const size_t red = (size_t)(a.Dphi / 32) * 16 * 64 * sizeof(float);
        lds = kv > red ? kv : red;
        fn = reinterpret_cast<const void*>(state_kernel<T, D, P>);
    }
    // raise the dynamic LDS limit of this instantiation once per device (idempotent, so a
    // race between host threads only repeats the call)
    static size_t lds_set[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
    if (lds > lds_set[dev]) {
        hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
        lds_set[dev] = lds;
    }
    if constexpr (kBf16) {
        auto kfn = state16_kernel<D, P>;
        hipLaunchKernelGGL(kfn, dim3(a.BH * a.G), dim3(kState16Waves * 64), lds, stream, a);
    } else {
        auto kfn = state_kernel<T, D, P>;
        hipLaunchKernelGGL(kfn, dim3(a.BH * a.G), dim3(StateShape<P>::NW * 64), lds, stream, a);
    }
    return hipGetLastError();
}

template <class T, int D>
static hipError_t launch_state_p(const StateArgs& a, hipStream_t stream) {
    switch (a.P) {
        case 1: return launch_state_t<T, D, 1>(a, stream);
        case 2: return launch_state_t<T, D, 2>(a, stream);
        case 3: return launch_state_t<T, D, 3>(a, stream);
        case 4: return launch_state_t<T, D, 4>(a, stream);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_state(const StateArgs& a, int in_dtype, hipStream_t stream) {
    if (a.G <= 0) return hipSuccess;
    if (in_dtype == 1) {
        switch (a.D) {
            case 32: return launch_state_p<bf16, 32>(a, stream);
            case 64: return launch_state_p<bf16, 64>(a, stream);
            case 128: return launch_state_p<bf16, 128>(a, stream);
        }
    } else {
        switch (a.D) {
            case 32: return launch_state_p<float, 32>(a, stream);
            case 64: return launch_state_p<float, 64>(a, stream);
            case 128: return launch_state_p<float, 128>(a, stream);
        }
    }
    return hipErrorInvalidValue;
}

hipError_t launch_scan(const ScanArgs& a, int in_dtype, hipStream_t stream) {
    if (a.G <= 0) return hipSuccess;
    const dim3 grid((unsigned)(a.P * (a.Dphi / 32) * (a.D / 32) + 1), a.BH);
    if (in_dtype == 1) hipLaunchKernelGGL(scan_kernel<bf16>, grid, dim3(256), 0, stream, a);
    else hipLaunchKernelGGL(scan_kernel<float>, grid, dim3(256), 0, stream, a);
    return hipGetLastError();
}

__global__ __launch_bounds__(256) void zero_kernel(float* p, int64_t count) {
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < count; i += (int64_t)gridDim.x * 256) p[i] = 0.f;
}

// Clearing with a kernel rather than a memset keeps the call safe inside captured graphs.
hipError_t launch_zero(float* p, int64_t count, hipStream_t stream) {
    if (count <= 0) return hipSuccess;
    int64_t blocks = (count + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(zero_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, p, count);
    return hipGetLastError();
}

hipError_t launch_copy(const CopyArgs& a, hipStream_t stream) {
    if (a.cnt <= 0) return hipSuccess;
    const int64_t total = (int64_t)a.n * a.D * a.elem_bytes / 16 * a.cnt;
    int64_t blocks = (total + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(copy_kernel, dim3((unsigned)blocks, a.BH), dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace rehyat
