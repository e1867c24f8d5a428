// tiles.hpp -- staging of key/value tiles (64 tokens) from HBM into LDS.
//
// K is stored row-major (token, d) and V transposed (d, token), because the value product
// contracts over tokens; the tokens of each 32-block of V^T are kept in slot order (see
// common.hpp) so one lane reads its EPL operand elements contiguously.  Both get one
// 16-byte chunk of padding per row: the MFMA operand reads (8 rows x 16 bytes per LDS
// cycle) then hit distinct banks, and every operand address is a per-lane base plus a
// compile-time offset.  The transposing V^T writes are arranged so that the 16 lanes of
// one LDS cycle write the 16 token quads of one d-row: one full, conflict-free row.
#pragma once

#include "common.hpp"

namespace rehyat {

// Key/value source for a window of tokens made of two contiguous segments: tokens
// [0, len1) come from (k1, v1), tokens [len1, ..) from (k2, v2).  Pointers are already
// offset to the batch-head slab and the window start.
template <class T>
struct KeySrc {
    const T* k1;
    const T* v1;
    const T* k2;
    const T* v2;
    int len1;
    __device__ inline const T* krow(int g, int D) const { return g < len1 ? k1 + (int64_t)g * D : k2 + (int64_t)(g - len1) * D; }
    __device__ inline const T* vrow(int g, int D) const { return g < len1 ? v1 + (int64_t)g * D : v2 + (int64_t)(g - len1) * D; }
};

template <class T, int D, int NT>
struct KVTile {
    static constexpr int BK = 64;                  // tokens per tile
    static constexpr int VEC = 16 / sizeof(T);     // elements per 16-byte chunk
    static constexpr int CPR = D / VEC;            // chunks per K row
    static constexpr int KLD = D + VEC;            // padded K row, elements
    static constexpr int VLD = BK + VEC;           // padded V^T row, elements
    static constexpr int K_ELEMS = BK * KLD;
    static constexpr int V_ELEMS = D * VLD;
    static constexpr int KCH = BK * CPR;           // K chunks per tile
    static constexpr int KPT = (KCH + NT - 1) / NT;
    static constexpr int VUN = (BK / 4) * CPR;     // V units: 4 tokens x one 16-byte chunk
    static constexpr int VPT = (VUN + NT - 1) / NT;
    static_assert(CPR >= 4 && CPR % 4 == 0, "head dim too small for the V staging layout");

    uint4 kr[KPT];
    uint4 vr[VPT][4];

    // unit u -> (token quad a, d-chunk b): 16 consecutive units are the 16 quads of a tile
    __device__ static inline void vunit(int u, int& a, int& b) {
        a = u % 16;
        b = u / 16;
    }

    // Issue the global loads of tile tokens [t0, t0+64).  CHECK: tokens >= Lk read as zeros
    // (only the last, ragged tile of a window needs it).  TWO: the window spans two
    // segments (streaming: held overlap frames, then the current chunk).
    template <bool CHECK, bool TWO>
    __device__ inline void load(const KeySrc<T>& src, int t0, int Lk, int tid) {
        load_k<CHECK, TWO>(src, t0, Lk, tid);
        load_v<CHECK, TWO>(src, t0, Lk, tid);
    }

    template <bool CHECK, bool TWO>
    __device__ inline void load_k(const KeySrc<T>& src, int t0, int Lk, int tid) {
#pragma unroll
        for (int i = 0; i < KPT; ++i) {
            const int c = tid + i * NT;
            if (CHECK || KCH % NT != 0) kr[i] = make_uint4(0, 0, 0, 0);
            if (KCH % NT == 0 || c < KCH) {
                const int row = c / CPR, ch = c % CPR;
                const int g = t0 + row;
                if (!CHECK || g < Lk) {
                    const T* p = TWO ? src.krow(g, D) : src.k1 + (int64_t)g * D;
                    kr[i] = *reinterpret_cast<const uint4*>(p + ch * VEC);
                }
            }
        }
    }
    template <bool CHECK, bool TWO>
    __device__ inline void load_v(const KeySrc<T>& src, int t0, int Lk, int tid) {
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            const int u = tid + i * NT;
            if (CHECK || VUN % NT != 0) {
#pragma unroll
                for (int ii = 0; ii < 4; ++ii) vr[i][ii] = make_uint4(0, 0, 0, 0);
            }
            if (VUN % NT == 0 || u < VUN) {
                int a, b;
                vunit(u, a, b);
#pragma unroll
                for (int ii = 0; ii < 4; ++ii) {
                    const int g = t0 + 4 * a + ii;
                    if (!CHECK || g < Lk) {
                        const T* p = TWO ? src.vrow(g, D) : src.v1 + (int64_t)g * D;
                        vr[i][ii] = *reinterpret_cast<const uint4*>(p + b * VEC);
                    }
                }
            }
        }
    }

    __device__ inline void store(T* Ks, T* Vs, int tid) const {
        store_k(Ks, tid);
        store_v(Vs, tid);
    }

    __device__ inline void store_k(T* Ks, int tid) const {
#pragma unroll
        for (int i = 0; i < KPT; ++i) {
            const int c = tid + i * NT;
            if (c < KCH) {
                const int row = c / CPR, ch = c % CPR;
                *reinterpret_cast<uint4*>(Ks + row * KLD + ch * VEC) = kr[i];
            }
        }
    }

    __device__ inline void store_v(T* Vs, int tid) const {
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            const int u = tid + i * NT;
            if (u >= VUN) continue;
            int a, b;
            vunit(u, a, b);
            const int kb = (4 * a) / 32, kk0 = (4 * a) % 32;
            if constexpr (sizeof(T) == 2) {
                // bf16: the 4 tokens of a quad stay adjacent in slot order
                const int pos = kb * 32 + slot_pos<8>(kk0);
                const int lc = pos / 8, half = (pos % 8) / 4;
                const uint32_t* w0 = reinterpret_cast<const uint32_t*>(&vr[i][0]);
                const uint32_t* w1 = reinterpret_cast<const uint32_t*>(&vr[i][1]);
                const uint32_t* w2 = reinterpret_cast<const uint32_t*>(&vr[i][2]);
                const uint32_t* w3 = reinterpret_cast<const uint32_t*>(&vr[i][3]);
#pragma unroll
                for (int jj = 0; jj < 8; ++jj) {
                    const int d = b * 8 + jj;
                    const int sh = (jj % 2) * 16;
                    const uint32_t e0 = (w0[jj / 2] >> sh) & 0xFFFFu, e1 = (w1[jj / 2] >> sh) & 0xFFFFu;
                    const uint32_t e2 = (w2[jj / 2] >> sh) & 0xFFFFu, e3 = (w3[jj / 2] >> sh) & 0xFFFFu;
                    uint2 val = make_uint2(e0 | (e1 << 16), e2 | (e3 << 16));
                    *reinterpret_cast<uint2*>(Vs + d * VLD + lc * 8 + half * 4) = val;
                }
            } else {
#pragma unroll
                for (int ii = 0; ii < 4; ++ii) {
                    const int pos = kb * 32 + slot_pos<1>(kk0 + ii);
                    const int lc = pos / VEC, e = pos % VEC;
                    const float* src = reinterpret_cast<const float*>(&vr[i][ii]);
#pragma unroll
                    for (int jj = 0; jj < VEC; ++jj) {
                        const int d = b * VEC + jj;
                        Vs[d * VLD + lc * VEC + e] = src[jj];
                    }
                }
            }
        }
    }

    // A operand of (keys x d) products: keys kb*32 + col, contraction step s over d.
    __device__ static inline typename Mfma<T>::frag kfrag(const T* Ks, int kb, int s, int col, int h) {
        return Mfma<T>::load(Ks + (kb * 32 + col) * KLD + s * Mfma<T>::KS + h * Mfma<T>::EPL);
    }
    // Operand holding V^T[d][tokens in slot order]: d = dbase + col, token block kb, step t.
    __device__ static inline typename Mfma<T>::frag vfrag(const T* Vs, int d, int kb, int t, int h) {
        constexpr int EPL = Mfma<T>::EPL;
        const int pos = kb * 32 + t * 2 * EPL + h * EPL;
        return Mfma<T>::load(Vs + d * VLD + pos);
    }
};

}  // namespace rehyat
