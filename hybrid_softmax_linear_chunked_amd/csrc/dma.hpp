// dma.hpp -- moving 64-token K/V tiles (and other row blocks) from HBM to LDS with the
// gfx950 LDS-DMA path, and reading MFMA operands out of them.
#pragma once

#include "common.hpp"
#include "tiles.hpp"

namespace rehyat {

// Byte address within the workgroup's LDS of a pointer into it.
__device__ inline uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// One LDS-DMA instruction (global_load_lds_dwordx4): lane l copies 16 bytes from its HBM
// address to LDS bytes [lds + 16 l, +16).  Issued from assembly so that the compiler does
// not take every later LDS read for a possible reader of the copy (it would wait for the
// copy in flight before the first such read and serialise the tile pipeline); completion is
// tracked by the explicit vmcnt waits of the pipeline instead.  The instruction has no
// register result and reads its address operands and M0 (the LDS base, one wait state
// after it is written) at issue; M0 is saved and restored around it.
// The base and the LDS address are wave-uniform; readfirstlane states it to the compiler,
// which may otherwise hold them in vector registers where they merge over branches.
__device__ inline const void* uniform_ptr(const void* p) {
    const uint64_t v = (uint64_t)(uintptr_t)p;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v), hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return (const void*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}
__device__ inline void dma16_s(const void* gbase, uint32_t voff, uint32_t lds) {  // uniform base + lane byte offset
    gbase = uniform_ptr(gbase);
    lds = __builtin_amdgcn_readfirstlane(lds);
    uint32_t keep;
    asm volatile(
        "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %3\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2\n\ts_mov_b32 m0, %0"
        : "=&s"(keep)
        : "v"(voff), "s"(gbase), "s"(lds)
        : "memory");
}

// The same, issued only where `issue` holds (wave-uniform) without a branch: the copy runs
// under an EXEC mask of the current lanes or of none (an instruction with no active lane
// moves nothing), restored before the block ends.  Keeps a basic block whole, so the
// scheduler can interleave the products around it.
__device__ inline void dma16_s_if(const void* gbase, uint32_t voff, uint32_t lds, bool issue) {
    // arithmetic, not a select: a select of the EXEC value becomes a branch
    gbase = uniform_ptr(gbase);
    lds = __builtin_amdgcn_readfirstlane(lds);
    const uint32_t on = __builtin_amdgcn_readfirstlane((uint32_t)issue);
    const uint64_t mask = __builtin_amdgcn_read_exec() & (0ull - (uint64_t)on);
    uint32_t keep;
    uint64_t keep_exec;
    asm volatile(
        "s_mov_b64 %1, exec\n\ts_mov_b64 exec, %5\n\ts_mov_b32 %0, m0\n\ts_mov_b32 m0, %4\n\ts_nop 0\n\t"
        "global_load_lds_dwordx4 %2, %3\n\ts_mov_b32 m0, %0\n\ts_mov_b64 exec, %1"
        : "=&s"(keep), "=&s"(keep_exec)
        : "v"(voff), "s"(gbase), "s"(lds), "s"(mask)
        : "memory");
}

// K/V tiles of 64 tokens moved HBM -> LDS by the LDS-DMA path (global_load_lds_dwordx4):
// no registers, no LDS write instructions, and the copy of tile t+2 runs while tile t is
// computed.  One DMA instruction fills 1 KB of LDS, lane l writing bytes [16l, 16l+16), so
// a tile is a sequence of 16-byte chunks and each lane picks the HBM chunk for its slot.
//   K: rows of D + 8 elements (one chunk of padding), read as MFMA A operands with one
//      ds_read_b128 per operand at compile-time offsets, conflict-free.
//   V: row-major rows of VLD elements, VLD chosen so that four consecutive rows start in
//      four different 64-byte bank groups; the value product reads V^T operands with
//      ds_read_b64_tr_b16, which hands lane i of each 16-lane group element i%4 of the
//      chunks addressed by lanes i/4 + 4r (r = 0..3): lanes pointing at a 4-token x 16-d
//      block receive it transposed, one d column of four tokens per lane.
// Padding chunks are filled with a copy of the row's first chunk, so every lane of every
// DMA instruction is active and the per-tile work is a uniform base plus fixed lane
// offsets.  Tokens past the end (ragged last tile) are clamped to the last token: the
// consumer masks their contributions, so only finite values are needed there.
// VLD_ overrides the V row length for readers with another access pattern (0: the
// default above).
template <int D, int NW, int VLD_ = 0>
struct DmaTiles {
    using T = bf16;
    static constexpr int BK = 64;
    static constexpr int KLD = D + 8;
    static constexpr int VLD = VLD_ ? VLD_ : D == 128 ? 160 : D == 64 ? 96 : 32;
    static constexpr int CPK = KLD / 8, CPV = VLD / 8;  // 16-byte chunks per row
    static constexpr int NIK = BK * CPK / 64, NIV = BK * CPV / 64;  // DMA instructions per tile
    static constexpr int PWK = (NIK + NW - 1) / NW, PWV = (NIV + NW - 1) / NW;
    static constexpr int K_ELEMS = BK * KLD, V_ELEMS = BK * VLD;
    static_assert(BK * CPK % 64 == 0 && BK * CPV % 64 == 0, "tile is not a whole number of DMA instructions");

    uint32_t koff[PWK], voff[PWV];  // element offset of this lane's chunk within a tile

    __device__ static inline uint32_t chunk_off(int q, int cpr, int dchunks) {
        const int row = q / cpr, c = q % cpr;
        return (uint32_t)(row * D + (c < dchunks ? c : 0) * 8);
    }
    __device__ inline void init(int wave, int lane) {
        // a wave's missing last instruction keeps offset 0 (it moves nothing)
#pragma unroll
        for (int i = 0; i < PWK; ++i) koff[i] = wave + i * NW < NIK ? chunk_off((wave + i * NW) * 64 + lane, CPK, D / 8) : 0u;
#pragma unroll
        for (int i = 0; i < PWV; ++i) voff[i] = wave + i * NW < NIV ? chunk_off((wave + i * NW) * 64 + lane, CPV, D / 8) : 0u;
    }
    // The i-th DMA instruction of this wave for the tile of tokens from t0 (none where the
    // wave has fewer): each lane copies its chunk; CHECK clamps tokens to the window, TWO
    // picks the segment of the two-segment (streaming) window
    template <bool CHECK, bool TWO, int NI, int PW>
    __device__ static inline void issue_one(int i, const T* b1, const T* b2, int len1, int t0, int Lk, T* dst,
                                            int wave, const uint32_t (&off)[PW]) {
        const int j = wave + i * NW;  // only the last instruction can be missing (wave < NW)
        const bool may_miss = NI % NW != 0 && i == PW - 1;
        if (!CHECK && !TWO) {
            // the missing instruction is issued under an empty EXEC mask, to a valid address
            if (may_miss) dma16_s_if(b1 + (int64_t)t0 * D, off[i] * (uint32_t)sizeof(T), lds_addr(dst + min(j, NI - 1) * 512), j < NI);
            else dma16_s(b1 + (int64_t)t0 * D, off[i] * (uint32_t)sizeof(T), lds_addr(dst + j * 512));
            return;
        }
        if (may_miss && j >= NI) return;
        const uint32_t lds = lds_addr(dst + j * 512);
        // token of this lane's chunk (clamped to the window) and its segment; each
        // segment is a uniform base, the lanes of the other one sit out (exec mask).  The
        // offset is opaque here, so these few instructions run where the copy is issued
        // instead of being hoisted and held in registers across the whole sweep.
        uint32_t o = off[i];
        asm volatile("" : "+v"(o));
        int g = t0 + (int)(o / D);
        if (CHECK) g = min(g, Lk - 1);
        const uint32_t col = o % D;
        if (TWO && g >= len1) dma16_s(b2, ((uint32_t)(g - len1) * D + col) * (uint32_t)sizeof(T), lds);
        else dma16_s(b1, ((uint32_t)g * D + col) * (uint32_t)sizeof(T), lds);
    }
    // all of this wave's DMA instructions for a tile
    template <bool CHECK, bool TWO, int NI, int PW>
    __device__ static inline void issue(const T* b1, const T* b2, int len1, int t0, int Lk, T* dst, int wave,
                                        const uint32_t (&off)[PW]) {
#pragma unroll
        for (int i = 0; i < PW; ++i) issue_one<CHECK, TWO, NI, PW>(i, b1, b2, len1, t0, Lk, dst, wave, off);
    }
    template <bool CHECK, bool TWO>
    __device__ inline void issue_k(const KeySrc<T>& src, int t0, int Lk, T* Ks, int wave) const {
        issue<CHECK, TWO, NIK, PWK>(src.k1, src.k2, src.len1, t0, Lk, Ks, wave, koff);
    }
    template <bool CHECK, bool TWO>
    __device__ inline void issue_v(const KeySrc<T>& src, int t0, int Lk, T* Vs, int wave) const {
        issue<CHECK, TWO, NIV, PWV>(src.v1, src.v2, src.len1, t0, Lk, Vs, wave, voff);
    }
    // single instructions (i < PWK, PWV) of the copy of a whole tile that starts at `tile`
    // (64 contiguous rows), for spreading the copy over the products of a sub-step
    __device__ inline void issue_k_at(int i, const T* tile, T* Ks, int wave) const {
        issue_one<false, false, NIK, PWK>(i, tile, tile, 0, 0, 0, Ks, wave, koff);
    }
    __device__ inline void issue_v_at(int i, const T* tile, T* Vs, int wave) const {
        issue_one<false, false, NIV, PWV>(i, tile, tile, 0, 0, 0, Vs, wave, voff);
    }

    // A operand of (keys x d) products: keys kb*32 + col, contraction step s over d
    __device__ static inline bf16x8 kfrag(const T* Ks, int kb, int s, int col, int h) {
        return *reinterpret_cast<const bf16x8*>(Ks + (kb * 32 + col) * KLD + s * 16 + h * 8);
    }
    // per-lane part of the V^T operand address: token 4h + a/4, d 16*(g%2) + 4*(a%4) for
    // lane = 16g + a
    __device__ static inline int vlane(int lane) {
        const int g = lane / 16, a = lane % 16;
        return (4 * (g / 2) + a / 4) * VLD + 16 * (g % 2) + 4 * (a % 4);
    }
    // V^T operand (d = db*32 + lane%32; tokens kb*32 + 16t + {4h..4h+3} and the same + 8:
    // the contraction slots of the C-layout P operand of step t)
    __device__ static inline bf16x8 vfrag(const T* Vs, int vl, int db, int kb, int t) {
        typedef short v4i16 __attribute__((ext_vector_type(4)));
        const T* p = Vs + vl + (kb * 32 + 16 * t) * VLD + db * 32;
        const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)(p));
        const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)(p + 8 * VLD));
        const v4i16 both_lo = lo, both_hi = hi;
        typedef short v8i16 __attribute__((ext_vector_type(8)));
        const v8i16 all = __builtin_shufflevector(both_lo, both_hi, 0, 1, 2, 3, 4, 5, 6, 7);
        return __builtin_bit_cast(bf16x8, all);
    }
};

}  // namespace rehyat
