// bwd.hip -- softmax branch of the ReHyAt backward, flash style, for bf16 inputs (ReHyAt blog,
// maplevalley.com.cn, 2.2.1 for the windowed softmax part; 3.1.1 for what the gradients
// serve).  With the saved per-query statistics lden_i = log(den_i) (den_i = the softmax sum
// of query i plus its linear normaliser) and delta_i = dout_i . o_i, the weights and score
// gradients of the softmax window are recomputed tile by tile,
//     P_ij  = exp(q_i . k_j / sqrt(D) - lden_i),
//     dS_ij = P_ij (dout_i . v_j - delta_i) / sqrt(D),
// and never stored:
//   bwd_dkv_kernel (key-stationary): each wave keeps dK_j and dV_j of its 32 keys in
//     registers and sweeps the query blocks of every chunk whose window holds them, in chunk
//     order: dV_j += sum_i P_ij dout_i, dK_j += sum_i dS_ij q_i;
//   bwd_dq_kernel (query-stationary): each wave keeps dQ_i of its 32 queries in registers
//     and sweeps the key tiles of its chunk's window: dQ_i += sum_j dS_ij k_j.
// Every sum runs in a fixed order and every output element is owned by one lane, which
// adds its total to the gradient buffer (the linear branch's share is already there), so
// the result is bitwise reproducible.  The only workspace is O(tokens): the statistics.
//
// Products are 16x16x32 bf16 MFMAs with fp32 accumulation; P and dS are rounded to bf16 as
// operands (the forward's P precision).  Tiles of 32 rows move to LDS by LDS-DMA several tiles
// ahead (a ring of four or five slots), in one layout that serves both the row operands (ds_read_b128) and
// the transposed ones (ds_read_b64_tr_b16, see dma.hpp).  Workgroups are dealt to the XCDs
// in contiguous runs, so the ones that read the same tiles share an L2.
#include "dma.hpp"
#include "grad.hpp"

namespace rehyat {

namespace {

constexpr float kLog2e = 1.4426950408889634f;

// s_waitcnt vmcnt(N) lgkmcnt(0) (expcnt untouched); N up to 63 in the split vmcnt field
template <int N>
__device__ inline void wait_vm_lds() {
    static_assert(N >= 0 && N <= 63, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4));
}

// The same for a wave-uniform run-time N (0 .. 16; larger N waits for everything, which is
// never wrong, only early).
__device__ inline void wait_vm_lds_n(int n) {
    switch (n) {
        case 1: wait_vm_lds<1>(); break;
        case 2: wait_vm_lds<2>(); break;
        case 3: wait_vm_lds<3>(); break;
        case 4: wait_vm_lds<4>(); break;
        case 5: wait_vm_lds<5>(); break;
        case 6: wait_vm_lds<6>(); break;
        case 7: wait_vm_lds<7>(); break;
        case 8: wait_vm_lds<8>(); break;
        case 9: wait_vm_lds<9>(); break;
        case 10: wait_vm_lds<10>(); break;
        case 11: wait_vm_lds<11>(); break;
        case 12: wait_vm_lds<12>(); break;
        case 13: wait_vm_lds<13>(); break;
        case 14: wait_vm_lds<14>(); break;
        case 15: wait_vm_lds<15>(); break;
        case 16: wait_vm_lds<16>(); break;
        default: wait_vm_lds<0>(); break;
    }
}

// One LDS-DMA instruction of 4-byte pieces: lane l copies the dword at gbase + voff to LDS
// bytes [lds + 4 l, +4).  Same conventions as dma16_s.
__device__ inline void dma4_s(const void* gbase, uint32_t voff, uint32_t lds) {
    gbase = uniform_ptr(gbase);
    lds = __builtin_amdgcn_readfirstlane(lds);
    uint32_t keep;
    asm volatile(
        "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %3\n\ts_nop 0\n\tglobal_load_lds_dword %1, %2\n\ts_mov_b32 m0, %0"
        : "=&s"(keep)
        : "v"(voff), "s"(gbase), "s"(lds)
        : "memory");
}

// 32 rows [r0, r0 + 32) of a row-major bf16 [rows][D] matrix (rows past rlast read row rlast)
// into an LDS tile of rows of LD elements.  16-byte chunk q of the tile is row q / (LD / 8),
// chunk q % (LD / 8) of it; padding chunks copy the row's first chunk.  The tile fills whole
// 1 KB blocks, one DMA instruction each, dealt round-robin over the NW waves.
template <int D, int LD, int NW>
struct Rows32 {
    static constexpr int CPR = LD / 8, CH = 32 * CPR, NI = (CH + 63) / 64, BYTES = NI * 1024;
    static constexpr int PW = (NI + NW - 1) / NW, NMIN = NI / NW;
    __device__ static inline void issue(const bf16* base, int r0, int rlast, unsigned char* dst, int wave, int lane) {
#pragma unroll
        for (int i = 0; i < PW; ++i) {
            const int j = wave + i * NW;
            if (j < NI) {
                const int qc = j * 64 + lane;
                const int row = qc < CH ? qc / CPR : 31, c = qc < CH ? qc % CPR : 0;
                const int gr = min(r0 + row, rlast);
                const uint32_t off = (uint32_t)(gr * D + (c < D / 8 ? c : 0) * 8) * 2u;
                dma16_s(base, off, lds_addr(dst + j * 1024));
            }
        }
    }
};

__device__ inline bf16x8 pack8(const float* x) {
    bf16x8 f;
#pragma unroll
    for (int e = 0; e < 8; ++e) f[e] = (bf16)x[e];
    return f;
}

// chunk c of the schedule: query rows [q0, q1), window key rows [k0, k1)
__device__ inline void chunk_span(const BwdArgs& a, int c, int& q0, int& q1, int& k0, int& k1) {
    const int f0 = c * a.Tc, f1 = min(f0 + a.Tc, a.T);
    const int ws = a.linear_only ? f1 : max(0, f0 - a.To);
    q0 = f0 * a.n;
    q1 = f1 * a.n;
    k0 = ws * a.n;
    k1 = f1 * a.n;
}

// Rows of D + 8 elements: row operands (ds_read_b128) conflict-free, transposed reads
// (ds_read_b64_tr_b16) two-way at most; one layout serves both, so each tile is copied once.
// Tile rows of D + 16 elements: the eight rows of a transposing read fall in eight different
// 32-byte bank groups, and the row reads of the 16x16x32 operands stay conflict-free too.
// waves (of 16 keys) per key-stationary workgroup: one workgroup per CU, three waves per
// SIMD, all sharing one ring of query tiles
constexpr int kDkvWaves = 12;

template <int D>
struct BwdTiles {
    static constexpr int LD16 = D + 16;
};

__device__ inline f32x4 mma16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Work item of this workgroup: workgroup g runs on XCD g % 8, and each XCD takes a
// contiguous run of the items, so that the workgroups sharing a chunk's tiles share an L2.
// -1 for the padding workgroups of the grid.
__device__ inline int xcd_item(int items) {
    const int per = (items + 7) / 8;
    const int it = (int)(blockIdx.x % 8) * per + (int)(blockIdx.x / 8);
    return it < items ? it : -1;
}

}  // namespace

// Both passes run on 16x16x32 products (lane l = 16 g + a holds row a and contraction slots
// 8 g .. 8 g + 7 of A, column a and the same slots of B, and column a, rows 4 g .. 4 g + 3 of
// C).  A score tile's C values are, as they stand, the operand of the next product over the
// same 32 rows, with slot i <-> row 4 g + i and slot 4 + i <-> row 16 + 4 g + i of the 32;
// the other operand of that product is read with two transposing LDS reads that deliver the
// same rows.

// row operand of a 16x16x32 product: row 16 r16 + a, columns 32 s + 8 g of a tile with rows of
// ld elements; ra = a * ld + 8 g
__device__ inline bf16x8 rd_row(const bf16* t, int ra, int ld, int r16, int s) {
    return *reinterpret_cast<const bf16x8*>(t + ra + 16 * r16 * ld + 32 * s);
}
// transposed operand: column 16 dc + a of rows 4 g + {0..3} and 16 + 4 g + {0..3};
// ta = (4 g + a / 4) * ld + 4 (a % 4)
__device__ inline bf16x8 rd_tr(const bf16* t, int ta, int ld, int dc) {
    typedef short v4i16 __attribute__((ext_vector_type(4)));
    typedef short v8i16 __attribute__((ext_vector_type(8)));
    const bf16* p = t + ta + 16 * dc;
    const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)(p));
    const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)(p + 16 * ld));
    return __builtin_bit_cast(bf16x8, (v8i16)__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Query-stationary pass: dQ of 256 queries of one chunk (8 waves x 32, two per SIMD).  Per
// 32-key half and wave: S^T = K Q^T and dP^T = V G^T as 2 x 2 C tiles (keys 16 kh + 4 g + i,
// this lane's query 16 qh + a), dS^T from them, dQ += dS K (A = dS^T values, B = K
// transposed).  Accumulators: 2 x D / 16 tiles of 4 registers.  Software-pipelined: the
// score products of key half i + 1 are issued before the softmax arithmetic of half i (the
// matrix core works while the vector ALU does).  A ring slot holds 64 keys (two halves of 32)
// and the workgroup meets at one barrier per slot; slot t + 1 must have landed before slot t
// is swept (its first half's scores are read at the end of slot t), and the ring holds four
// slots, the copy of slot t + 3 issued as slot t starts.
template <int D>
__global__ __launch_bounds__(512, 1) void bwd_dq_kernel(const BwdArgs a) {
    constexpr int NW = 8, NK = D / 32, ND = D / 16, R = 4;
    constexpr int LD = BwdTiles<D>::LD16;
    using Tl = Rows32<D, LD, NW>;
    constexpr int HALF = 2 * Tl::BYTES;  // K, then V, of 32 keys
    constexpr int SLOT = 2 * HALF;       // a ring slot holds 64 keys: one barrier per 64
    constexpr int NMIN = 4 * Tl::NMIN;   // copy instructions per slot of the wave with the fewest
    extern __shared__ __align__(16) unsigned char smem[];

    const int blk = xcd_item(a.BH * a.nc * a.qtiles);
    if (blk < 0) return;
    const int qt = blk % a.qtiles, c = (blk / a.qtiles) % a.nc, bh = blk / (a.qtiles * a.nc);
    int q0, q1, k0, k1;
    chunk_span(a, c, q0, q1, k0, k1);
    const int Lk = k1 - k0;
    const int qbase = q0 + qt * NW * 32;
    if (Lk <= 0 || qbase >= q1) return;

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
    const int lane = tid % 64, la = lane % 16, lg = lane / 16;
    const int64_t slab = (int64_t)bh * a.N;
    const bf16* qs = static_cast<const bf16*>(a.q) + slab * D;
    const bf16* ks = static_cast<const bf16*>(a.k) + slab * D;
    const bf16* vs = static_cast<const bf16*>(a.v) + slab * D;
    const bf16* gs = static_cast<const bf16*>(a.g) + slab * D;

    // this lane's queries (columns of the transposed score tiles) and their operands
    bf16x8 qf[2][NK], gf[2][NK];
    float l2[2], dl[2];
#pragma unroll
    for (int qh = 0; qh < 2; ++qh) {
        const int qrow = qbase + wave * 32 + 16 * qh + la;
        const bool ok = qrow < q1;
#pragma unroll
        for (int s = 0; s < NK; ++s) {
            qf[qh][s] = ok ? *reinterpret_cast<const bf16x8*>(qs + (int64_t)qrow * D + 32 * s + 8 * lg) : bf16x8{};
            gf[qh][s] = ok ? *reinterpret_cast<const bf16x8*>(gs + (int64_t)qrow * D + 32 * s + 8 * lg) : bf16x8{};
        }
        l2[qh] = ok ? a.stats[slab + qrow] * kLog2e : INFINITY;
        dl[qh] = ok ? a.stats[a.stat_stride + slab + qrow] : 0.f;
    }
    const float sl = a.scale_log2, sc = a.scale;

    f32x4 acc[2][ND];
#pragma unroll
    for (int qh = 0; qh < 2; ++qh)
#pragma unroll
        for (int dc = 0; dc < ND; ++dc) acc[qh][dc] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int nkt = (Lk + 31) / 32;   // 32-key halves
    const int nst = (nkt + 1) / 2;    // 64-key ring slots
    // half i of the window: keys k0 + 32 i .. + 31, in half i % 2 of slot i / 2
    auto slot = [&](int i) { return smem + ((i / 2) % R) * SLOT + (i % 2) * HALF; };
    // both halves of slot tile t (a half past the window copies its last rows, never used: every
    // slot issues the same number of copies, which the waits count)
    auto dma = [&](int t) {
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
            unsigned char* s0 = smem + (t % R) * SLOT + hf * HALF;
            const int r0 = min(k0 + 64 * t + 32 * hf, k1 - 1);
            Tl::issue(ks, r0, k1 - 1, s0, wave, lane);
            Tl::issue(vs, r0, k1 - 1, s0 + Tl::BYTES, wave, lane);
        }
    };
    // wait until at most `later` slots of copies are in flight, then the workgroup barrier
    auto sync = [&](int later) {
        if (later >= 1) wait_vm_lds<NMIN>();
        else wait_vm_lds<0>();
        asm volatile("s_barrier" ::: "memory");
    };
    const int ra = la * LD + 8 * lg;
    const int ta = (4 * lg + la / 4) * LD + 4 * (la % 4);
    // S^T and dP^T of tile i: [kh][qh]
    auto scores = [&](int i, f32x4 (&S)[2][2], f32x4 (&P)[2][2]) {
        const bf16* Kt = reinterpret_cast<const bf16*>(slot(i));
        const bf16* Vt = reinterpret_cast<const bf16*>(slot(i) + Tl::BYTES);
#pragma unroll
        for (int kh = 0; kh < 2; ++kh)
#pragma unroll
            for (int qh = 0; qh < 2; ++qh) {
                S[kh][qh] = f32x4{0.f, 0.f, 0.f, 0.f};
                P[kh][qh] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
#pragma unroll
        for (int s = 0; s < NK; ++s)
#pragma unroll
            for (int kh = 0; kh < 2; ++kh) {
                const bf16x8 kr = rd_row(Kt, ra, LD, kh, s), vr = rd_row(Vt, ra, LD, kh, s);
#pragma unroll
                for (int qh = 0; qh < 2; ++qh) {
                    S[kh][qh] = mma16(kr, qf[qh][s], S[kh][qh]);
                    P[kh][qh] = mma16(vr, gf[qh][s], P[kh][qh]);
                }
            }
    };
    // dS^T of tile i from its scores, then dQ += dS K
    auto products = [&](int i, const f32x4 (&S)[2][2], const f32x4 (&P)[2][2]) {
        const bf16* Kt = reinterpret_cast<const bf16*>(slot(i));
        const int klim = Lk - 32 * i;  // keys of this tile inside the window
        bf16x8 af[2];
#pragma unroll
        for (int qh = 0; qh < 2; ++qh) {
            float ds[8];
#pragma unroll
            for (int kh = 0; kh < 2; ++kh)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    float p = __builtin_amdgcn_exp2f(S[kh][qh][e] * sl - l2[qh]);
                    if (klim < 32 && 16 * kh + 4 * lg + e >= klim) p = 0.f;
                    ds[4 * kh + e] = p * (P[kh][qh][e] - dl[qh]) * sc;
                }
            af[qh] = pack8(ds);
        }
#pragma unroll
        for (int dc = 0; dc < ND; ++dc) {
            const bf16x8 kt = rd_tr(Kt, ta, LD, dc);
#pragma unroll
            for (int qh = 0; qh < 2; ++qh) acc[qh][dc] = mma16(af[qh], kt, acc[qh][dc]);
        }
    };

    // the operand loads above complete before the first copy is issued: the compiler does
    // not count the copies, and a wait for those loads inside the loop would drain them
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    for (int t = 0; t < R - 1 && t < nst; ++t) dma(t);
    sync(min(nst - 2, 1));  // slots 0 and 1 landed
    f32x4 SA[2][2], PA[2][2], SB[2][2], PB[2][2];
    scores(0, SA, PA);
    // slot tile t: halves 2t and 2t + 1, each with the score products of the next half (which
    // may lie in slot t + 1) ahead of its own dS and dQ products
    for (int t = 0; t < nst; ++t) {
        if (t + R - 1 < nst) dma(t + R - 1);  // into the slot tile t - 1 used
        const int i = 2 * t;
        if (i + 1 < nkt) scores(i + 1, SB, PB);
        products(i, SA, PA);
        if (i + 1 < nkt) {
            if (i + 2 < nkt) scores(i + 2, SA, PA);
            products(i + 1, SB, PB);
        }
        sync(min(nst - 3 - t, 1));  // slot t + 2 landed; every wave is done with slot t
    }
    // acc[qh][dc]: column d = 16 dc + a, rows = queries 16 qh + 4 g + {0..3} of this wave
    float* dq = a.dq + slab * D;
#pragma unroll
    for (int qh = 0; qh < 2; ++qh)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int qr = qbase + wave * 32 + 16 * qh + 4 * lg + e;
            if (qr < q1) {
#pragma unroll
                for (int dc = 0; dc < ND; ++dc) dq[(int64_t)qr * D + 16 * dc + la] += acc[qh][dc][e];
            }
        }
}

// Key-stationary pass: dK and dV of 16 NW keys (NW waves x 16; with NW = 12 one workgroup per
// CU and three waves per SIMD, so that one wave's arithmetic overlaps the others' products and
// the ring of query tiles is shared by all twelve), on 16x16x32
// products (lane l = 16 g + a holds row a and contraction slots 8 g .. 8 g + 7 of A, column a
// and the same slots of B, and column a, rows 4 g .. 4 g + 3 of C).  A ring slot holds 64
// queries (two halves of 32, one workgroup barrier per slot).  Per 32-query half and wave:
//   S = Q K^T, dP = G V^T: two C tiles each (queries 16 qh + 4 g + i, this lane's key a);
//   P, dS from them; as they stand, the eight values of a lane are the B operand (queries x
//     keys) with slot i <-> query 4 g + i and slot 4 + i <-> query 16 + 4 g + i;
//   dV^T += G^T P, dK^T += Q^T dS: A = G or Q transposed, read with two transposing LDS
//     reads that deliver the same queries for column 16 dc + a.
// The accumulators of a wave are 2 D / 16 tiles of 4 registers (64 at D = 128).
template <int D, int NW>
__global__ __launch_bounds__(NW * 64, NW >= 8 ? 1 : 2) void bwd_dkv_kernel(const BwdArgs a) {
    constexpr int KW = 16, NK = D / 32, ND = D / 16, R = 4;
    constexpr int LD = BwdTiles<D>::LD16;
    using Tl = Rows32<D, LD, NW>;
    constexpr int STAT = 256;  // lden of the 32 queries, then delta
    constexpr int HALF = 2 * Tl::BYTES + STAT;  // Q, G, statistics of 32 queries
    constexpr int SLOT = 2 * HALF;              // a slot holds 64 queries: one barrier per 64
    extern __shared__ __align__(16) unsigned char smem[];

    const int item = xcd_item(a.BH * a.kblocks);
    if (item < 0) return;
    const int kb = item % a.kblocks, bh = item / a.kblocks;
    const int key0 = kb * NW * KW;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
    const int lane = tid % 64, la = lane % 16, lg = lane / 16;
    const int64_t slab = (int64_t)bh * a.N;
    const bf16* qs = static_cast<const bf16*>(a.q) + slab * D;
    const bf16* ks = static_cast<const bf16*>(a.k) + slab * D;
    const bf16* vs = static_cast<const bf16*>(a.v) + slab * D;
    const bf16* gs = static_cast<const bf16*>(a.g) + slab * D;

    // chunks whose softmax window meets the block's keys: a contiguous range
    int c_lo = a.nc, c_hi = -1;
    for (int c = 0; c < a.nc; ++c) {
        int q0, q1, k0, k1;
        chunk_span(a, c, q0, q1, k0, k1);
        if (k1 > k0 && k0 < key0 + NW * KW && k1 > key0) {
            c_lo = min(c_lo, c);
            c_hi = c;
        }
    }
    if (c_hi < 0) return;
    // query blocks of 64 (two halves of 32), chunk after chunk
    auto nqb = [&](int c) {
        int q0, q1, k0, k1;
        chunk_span(a, c, q0, q1, k0, k1);
        return (q1 - q0 + 63) / 64;
    };
    int ntiles = 0;
    for (int c = c_lo; c <= c_hi; ++c) ntiles += nqb(c);
    // tile index -> (chunk, first query row); chunks are few, so a short walk
    auto tile_at = [&](int i, int& c, int& qb0) {
        c = c_lo;
        int nb = nqb(c);
        while (i >= nb) {
            i -= nb;
            ++c;
            nb = nqb(c);
        }
        qb0 = c * a.Tc * a.n + 64 * i;
    };

    const int kw = key0 + wave * KW + la;  // this lane's key
    const bool kok = kw < a.N;
    bf16x8 kf[NK], vf[NK];  // B operands: K / V row kw, d = 32 s + 8 lg .. + 7
#pragma unroll
    for (int s = 0; s < NK; ++s) {
        if (kok) {
            kf[s] = *reinterpret_cast<const bf16x8*>(ks + (int64_t)kw * D + 32 * s + 8 * lg);
            vf[s] = *reinterpret_cast<const bf16x8*>(vs + (int64_t)kw * D + 32 * s + 8 * lg);
        } else {
            kf[s] = bf16x8{};
            vf[s] = bf16x8{};
        }
    }
    const float sl = a.scale_log2, sc = a.scale;
    f32x4 dk[ND], dv[ND];
#pragma unroll
    for (int dc = 0; dc < ND; ++dc) {
        dk[dc] = f32x4{0.f, 0.f, 0.f, 0.f};
        dv[dc] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    auto slot = [&](int i) { return smem + (i % R) * SLOT; };
    auto dma = [&](int i) {
        int c, qb0;
        tile_at(i, c, qb0);
        const int qend = min((c * a.Tc + a.Tc), a.T) * a.n;
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
            // a half past the chunk's end copies its last rows (never used): every tile issues
            // the same number of copies, which the waits count
            const int qh0 = min(qb0 + 32 * hf, qend - 1);
            unsigned char* s0 = slot(i) + hf * HALF;
            Tl::issue(qs, qh0, qend - 1, s0, wave, lane);
            Tl::issue(gs, qh0, qend - 1, s0 + Tl::BYTES, wave, lane);
            // statistics: lanes 0..31 lden, 32..63 delta (rows past the chunk are masked; each
            // array carries 32 spare values, so reads past the last slab stay inside it)
            if (wave == 0) {
                const uint32_t off = (uint32_t)(((lane >= 32 ? a.stat_stride : 0) + slab + qh0 + lane % 32) * 4);
                dma4_s(a.stats, off, lds_addr(s0 + 2 * Tl::BYTES));
            }
        }
    };
    // this wave's copy instructions per tile: its share of the Q and G blocks, and the
    // statistics (wave 0), for both halves; waiting for all but `later` tiles' worth leaves
    // those in flight
    const int per_tile = 2 * (2 * (wave < Tl::NI ? (Tl::NI - 1 - wave) / NW + 1 : 0) + (wave == 0 ? 1 : 0));
    auto sync = [&](int later) {
        wait_vm_lds_n(per_tile * later);
        asm volatile("s_barrier" ::: "memory");
    };
    // row operand: row 16 qh + la, d = 32 s + 8 lg; transposed: rows 4 lg + la / 4 (+ 16),
    // d = 16 dc + 4 (la % 4)
    const int ra = la * LD + 8 * lg;
    const int ta = (4 * lg + la / 4) * LD + 4 * (la % 4);
    auto tread = [&](const bf16* t, int dc) {
        typedef short v4i16 __attribute__((ext_vector_type(4)));
        typedef short v8i16 __attribute__((ext_vector_type(8)));
        const bf16* p = t + ta + 16 * dc;
        const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)(p));
        const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4i16*)(p + 16 * LD));
        return __builtin_bit_cast(bf16x8, (v8i16)__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    };

    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the operand loads, before the first copy
    dma(0);
    if (ntiles > 1) dma(1);
    if (ntiles > 2) dma(2);
    sync(min(ntiles - 1, 2));
    for (int i = 0; i < ntiles; ++i) {
        if (i + 3 < ntiles) dma(i + 3);
        int c, qb0;
        tile_at(i, c, qb0);
        int q0, q1, k0, k1;
        chunk_span(a, c, q0, q1, k0, k1);
        const bool kin = kok && kw >= k0 && kw < k1;  // key inside this chunk's window
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
        const int qlim = q1 - (qb0 + 32 * hf);  // queries of this half inside the chunk
        if (qlim <= 0) break;
        const unsigned char* s0 = slot(i) + hf * HALF;
        const bf16* Qt_ = reinterpret_cast<const bf16*>(s0);
        const bf16* Gt_ = reinterpret_cast<const bf16*>(s0 + Tl::BYTES);
        const float* st = reinterpret_cast<const float*>(s0 + 2 * Tl::BYTES);
        f32x4 S[2], dP[2];
#pragma unroll
        for (int qh = 0; qh < 2; ++qh) {
            S[qh] = f32x4{0.f, 0.f, 0.f, 0.f};
            dP[qh] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < NK; ++s) {
                S[qh] = mma16(*reinterpret_cast<const bf16x8*>(Qt_ + ra + 16 * qh * LD + 32 * s), kf[s], S[qh]);
                dP[qh] = mma16(*reinterpret_cast<const bf16x8*>(Gt_ + ra + 16 * qh * LD + 32 * s), vf[s], dP[qh]);
            }
        }
        float p[8], ds[8];  // slot 4 qh + i <-> query 16 qh + 4 lg + i
#pragma unroll
        for (int qh = 0; qh < 2; ++qh) {
            const float4 l4 = *reinterpret_cast<const float4*>(st + 16 * qh + 4 * lg);
            const float4 d4 = *reinterpret_cast<const float4*>(st + 32 + 16 * qh + 4 * lg);
            const float lv[4] = {l4.x, l4.y, l4.z, l4.w}, dv4[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float pr = __builtin_amdgcn_exp2f(S[qh][e] * sl - lv[e] * kLog2e);
                if (!kin || (qlim < 32 && 16 * qh + 4 * lg + e >= qlim)) pr = 0.f;
                p[4 * qh + e] = pr;
                ds[4 * qh + e] = pr * (dP[qh][e] - dv4[e]) * sc;
            }
        }
        const bf16x8 pf = pack8(p), sf = pack8(ds);
#pragma unroll
        for (int dc = 0; dc < ND; ++dc) {
            dv[dc] = mma16(tread(Gt_, dc), pf, dv[dc]);
            dk[dc] = mma16(tread(Qt_, dc), sf, dk[dc]);
        }
        }
        sync(min(ntiles - 2 - i, 2));
    }
    if (!kok) return;
    // dk[dc], dv[dc]: column = this lane's key, rows d = 16 dc + 4 lg + {0..3}
    float* dkr = a.dk + (slab + kw) * D;
    float* dvr = a.dv + (slab + kw) * D;
#pragma unroll
    for (int dc = 0; dc < ND; ++dc) {
        const int d = 16 * dc + 4 * lg;
        float4 x = *reinterpret_cast<float4*>(dkr + d);
        x.x += dk[dc][0];
        x.y += dk[dc][1];
        x.z += dk[dc][2];
        x.w += dk[dc][3];
        *reinterpret_cast<float4*>(dkr + d) = x;
        float4 y = *reinterpret_cast<float4*>(dvr + d);
        y.x += dv[dc][0];
        y.y += dv[dc][1];
        y.z += dv[dc][2];
        y.w += dv[dc][3];
        *reinterpret_cast<float4*>(dvr + d) = y;
    }
}

namespace {

// raise the dynamic LDS limit of a kernel once per device
hipError_t lds_limit(const void* fn, size_t lds, size_t (&done)[64]) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
    if (lds > done[dev]) {
        hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
        done[dev] = lds;
    }
    return hipSuccess;
}

template <int D>
hipError_t launch_bwd_d(const BwdArgs& a, hipStream_t stream) {
    const size_t lds_q = 4 * 2 * (size_t)(2 * Rows32<D, BwdTiles<D>::LD16, 8>::BYTES);
    const size_t lds_k = 4 * 2 * (size_t)(2 * Rows32<D, BwdTiles<D>::LD16, kDkvWaves>::BYTES + 256);
    static size_t set_q[64] = {}, set_k[64] = {};
    hipError_t e = lds_limit(reinterpret_cast<const void*>(bwd_dkv_kernel<D, kDkvWaves>), lds_k, set_k);
    if (e != hipSuccess) return e;
    e = lds_limit(reinterpret_cast<const void*>(bwd_dq_kernel<D>), lds_q, set_q);
    if (e != hipSuccess) return e;
    const int nk = a.BH * a.kblocks, nq = a.BH * a.nc * a.qtiles;
    hipLaunchKernelGGL((bwd_dkv_kernel<D, kDkvWaves>), dim3((unsigned)((nk + 7) / 8 * 8)), dim3(kDkvWaves * 64), lds_k,
                       stream, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(bwd_dq_kernel<D>, dim3((unsigned)((nq + 7) / 8 * 8)), dim3(512), lds_q, stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_softmax(BwdArgs a, int D, hipStream_t stream) {
    a.qtiles = (a.Tc * a.n + 255) / 256;
    a.kblocks = (a.N + kDkvWaves * 16 - 1) / (kDkvWaves * 16);
    switch (D) {
        case 32: return launch_bwd_d<32>(a, stream);
        case 64: return launch_bwd_d<64>(a, stream);
        case 128: return launch_bwd_d<128>(a, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace rehyat
