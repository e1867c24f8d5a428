// state16.hpp -- per-frame partials of the linear-attention state (ReHyAt blog,
// maplevalley.com.cn, section 2.3: Delta_f = phi_k(K_f)^T V_f and sum_tokens phi_k(K_f) of
// the frames that leave the softmax window) for bf16 inputs, as a workgroup body shared by
// the stand-alone state kernel and the streaming attention launch (which runs it in
// workgroups of its own beside the attention tiles).
#pragma once

#include "dma.hpp"
#include "kernels.hpp"
#include "tiles.hpp"

namespace rehyat {

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

// LDS bytes of the K/V ring
template <int D>
constexpr size_t state16_lds_bytes() {
    return kState16Ring * (size_t)(State16Tiles<D>::K_ELEMS + State16Tiles<D>::V_ELEMS) * sizeof(bf16);
}

// The work of workgroup blk (= bh * G + frame index) of a launch of kState16Waves waves,
// with state16_lds_bytes<D>() bytes of LDS at smem.
template <int D, int P>
__device__ __forceinline__ void state16_body(const StateArgs& a, int blk, unsigned char* smem) {
    using T = bf16;
    using Tile = State16Tiles<D>;
    constexpr int NW = kState16Waves, R = kState16Ring, BK = Tile::BK;
    constexpr int NS = D / 32;   // contraction steps of u
    constexpr int ND = D / 16;   // 16-column blocks of Delta
    constexpr int KLD = Tile::KLD, VLD = Tile::VLD;
    static_assert(BK == 64, "four 16-token C tiles per tile");

    T* const kring = reinterpret_cast<T*>(smem);
    T* const vring = kring + R * Tile::K_ELEMS;

    const int gi = blk % a.G;
    const int bh = blk / a.G;
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

template <int D>
__device__ __forceinline__ void state16_any_p(const StateArgs& a, int blk, unsigned char* smem) {
    switch (a.P) {
        case 1: state16_body<D, 1>(a, blk, smem); break;
        case 2: state16_body<D, 2>(a, blk, smem); break;
        case 3: state16_body<D, 3>(a, blk, smem); break;
        case 4: state16_body<D, 4>(a, blk, smem); break;
    }
}

}  // namespace rehyat
