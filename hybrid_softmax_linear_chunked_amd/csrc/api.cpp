// api.cpp -- C ABI of the ReHyAt hybrid-attention library (declared in include/rehyat.h).
//
// Host responsibilities only: argument validation (always before the first HIP call),
// the chunk schedule of the ReHyAt blog (maplevalley.com.cn) sections 2.2.1 and 2.3,
// workspace / state sizing, and the launch sequence on the caller's stream.  Every step
// of the computation runs in the HIP kernels of attn.hip, state.hip and phi.hip.
#include <cmath>
#include <algorithm>
#include <cstring>

#include "../../include/rehyat.h"
#include "kernels.hpp"
#include "grad.hpp"

using namespace rehyat;

namespace {

constexpr int32_t kStreamMagic = 0x52485954;  // "RHYT"

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

size_t elem_bytes(int32_t dt) { return dt == REHYAT_BF16 ? 2 : 4; }

rehyat_status check_params(const rehyat_params* p, bool need_T) {
    if (!p) return REHYAT_EINVAL;
    if (p->B < 1 || p->H < 1 || p->frame_tokens < 1 || p->Tc < 1 || p->To < 0) return REHYAT_EINVAL;
    if (need_T && p->T < 1) return REHYAT_EINVAL;
    if (p->linear_only != 0 && p->linear_only != 1) return REHYAT_EINVAL;
    if (p->in_dtype != REHYAT_FP32 && p->in_dtype != REHYAT_BF16) return REHYAT_EINVAL;
    if (p->out_dtype != REHYAT_FP32 && p->out_dtype != REHYAT_BF16) return REHYAT_EINVAL;
    if (p->D != 32 && p->D != 64 && p->D != 128) return REHYAT_ESHAPE;
    if (p->Dphi < 32 || p->Dphi > 128 || p->Dphi % 32 != 0) return REHYAT_ESHAPE;
    if (p->P < 1 || p->P > 4) return REHYAT_ESHAPE;
    // sizes must keep every slab index inside 32-bit token counts and 64-bit offsets
    const int64_t N = (int64_t)(need_T ? p->T : p->Tc) * p->frame_tokens;
    if (N > (int64_t)1 << 30 || (int64_t)p->Tc * p->frame_tokens > (int64_t)1 << 28) return REHYAT_EINVAL;
    if ((int64_t)p->B * p->H > (int64_t)1 << 24) return REHYAT_EINVAL;
    return REHYAT_OK;
}

bool aligned16(const void* ptr) { return ptr && (reinterpret_cast<uintptr_t>(ptr) % 16 == 0); }
bool aligned4_or_null(const void* ptr) { return !ptr || (reinterpret_cast<uintptr_t>(ptr) % 4 == 0); }

int num_chunks(const rehyat_params* p) { return (p->T + p->Tc - 1) / p->Tc; }

// Frames whose state enters some chunk: the last chunk's linear region [0, ls(nc-1)).
int state_frames(const rehyat_params* p) {
    const int nc = num_chunks(p);
    const int f0 = (nc - 1) * p->Tc;
    const int f1 = f0 + p->Tc < p->T ? f0 + p->Tc : p->T;
    if (p->linear_only) return f1;
    return f0 - p->To > 0 ? f0 - p->To : 0;
}

size_t partial_bytes(const rehyat_params* p, int frames) {
    const size_t F = (size_t)p->P * p->Dphi;
    const size_t BH = (size_t)p->B * p->H;
    return align256(BH * frames * F * p->D * sizeof(float)) + align256(BH * frames * F * sizeof(float));
}

// Chunk-parallel workspace: per-frame partials [BH, G, F, D] + [BH, G, F], then the
// state images of every chunk [BH, nc, ...].
struct ParallelLayout {
    size_t sp, zp, img, zimg, total;
};

ParallelLayout parallel_layout(const rehyat_params* p, int G) {
    const size_t F = (size_t)p->P * p->Dphi;
    const size_t BH = (size_t)p->B * p->H;
    const int nc = num_chunks(p);
    ParallelLayout L;
    size_t off = 0;
    L.sp = off; off += align256(BH * G * F * p->D * sizeof(float));
    L.zp = off; off += align256(BH * G * F * sizeof(float));
    L.img = off; off += align256(BH * nc * F * p->D * elem_bytes(p->in_dtype));
    L.zimg = off; off += align256(BH * nc * F * sizeof(float));
    L.total = off;
    return L;
}

// Streaming state: S, Z (float, carried sums), the image of the current state, and two
// overlap buffers of K and V with To frames per batch-head and 64 rows to spare: each step
// copies the first rows of its chunk after the held frames, up to the next multiple of 64,
// so that no 64-token key tile of the window spans both buffers.
constexpr int kOverlapSpareRows = 64;

int64_t overlap_rows(const rehyat_params* p) { return (int64_t)p->To * p->frame_tokens + kOverlapSpareRows; }

struct StateLayout {
    size_t S, Z, img, zimg, ovk[2], ovv[2], total;
};

StateLayout state_layout(const rehyat_params* p) {
    const size_t F = (size_t)p->P * p->Dphi;
    const size_t BH = (size_t)p->B * p->H;
    const size_t ov = BH * (size_t)overlap_rows(p) * p->D * elem_bytes(p->in_dtype);
    StateLayout L;
    size_t off = 0;
    L.S = off; off += align256(BH * F * p->D * sizeof(float));
    L.Z = off; off += align256(BH * F * sizeof(float));
    L.img = off; off += align256(BH * F * p->D * elem_bytes(p->in_dtype));
    L.zimg = off; off += align256(BH * F * sizeof(float));
    for (int i = 0; i < 2; ++i) { L.ovk[i] = off; off += align256(ov); }
    for (int i = 0; i < 2; ++i) { L.ovv[i] = off; off += align256(ov); }
    L.total = off;
    return L;
}

float scale_log2(int D) { return (float)(1.4426950408889634 / std::sqrt((double)D)); }

AttnArgs attn_common(const rehyat_params* p, const void* wq, const float* bq) {
    AttnArgs a;
    std::memset(&a, 0, sizeof(a));
    a.wq = wq;
    a.bq = bq;
    a.H = p->H;
    a.BH = p->B * p->H;
    a.D = p->D;
    a.n = p->frame_tokens;
    a.T = p->T;
    a.Tc = p->Tc;
    a.To = p->To;
    a.linear_only = p->linear_only;
    a.Dphi = p->Dphi;
    a.P = p->P;
    a.scale_log2 = scale_log2(p->D);
    return a;
}

StateArgs state_common(const rehyat_params* p, const void* wk, const float* bk) {
    StateArgs s;
    std::memset(&s, 0, sizeof(s));
    s.wk = wk;
    s.bk = bk;
    s.H = p->H;
    s.BH = p->B * p->H;
    s.D = p->D;
    s.n = p->frame_tokens;
    s.Dphi = p->Dphi;
    s.P = p->P;
    return s;
}

rehyat_status hip_status(hipError_t e) { return e == hipSuccess ? REHYAT_OK : REHYAT_EHIP; }

}  // namespace

extern "C" {

const char* rehyat_status_string(rehyat_status s) {
    switch (s) {
        case REHYAT_OK: return "ok";
        case REHYAT_EINVAL: return "invalid parameter value";
        case REHYAT_ESHAPE: return "unsupported shape";
        case REHYAT_EALIGN: return "null or misaligned pointer";
        case REHYAT_EWORKSPACE: return "workspace missing or too small";
        case REHYAT_ESTATE: return "invalid streaming state or call";
        case REHYAT_EHIP: return "HIP launch error";
        case REHYAT_ESCRATCH: return "workspace exceeds the static scratch area (64 MiB per GPU)";
    }
    return "unknown status";
}

int32_t rehyat_features(const rehyat_params* p) {
    if (check_params(p, false) != REHYAT_OK) return -1;
    return p->P * p->Dphi;
}

rehyat_status rehyat_phi(const rehyat_params* p, const void* x, const void* w, const float* bias,
                         void* feat, hipStream_t stream) {
    rehyat_status st = check_params(p, true);
    if (st != REHYAT_OK) return st;
    if (!aligned16(x) || !aligned16(w) || !aligned16(feat) || !aligned4_or_null(bias)) return REHYAT_EALIGN;
    PhiArgs a;
    a.x = x;
    a.w = w;
    a.bias = bias;
    a.feat = feat;
    a.N = (int64_t)p->T * p->frame_tokens;
    a.H = p->H;
    a.BH = p->B * p->H;
    a.D = p->D;
    a.Dphi = p->Dphi;
    a.P = p->P;
    return hip_status(launch_phi(a, p->in_dtype, stream));
}

// Tail-split scratch of a bf16 attention launch, placed at `base` of a workspace: one arrival
// counter per split tile, then the partials of both halves (none for float32 inputs or
// where the plan splits nothing).
struct SplitWs {
    int splits, split_per_xcd;
    size_t cnt, part, total;
};

static SplitWs split_ws(const rehyat_params* p, AttnArgs a, size_t base) {
    SplitWs L;
    L.splits = p->in_dtype == REHYAT_BF16 ? wide_split_plan(a) : 0;
    L.split_per_xcd = L.splits > 0 ? a.split_per_xcd : 0;
    L.cnt = base;
    L.part = L.cnt + (L.splits > 0 ? align256((size_t)L.splits * sizeof(unsigned)) : 0);
    L.total = L.part + (size_t)L.splits * wide_split_part_bytes(p->D);
    return L;
}

// Workspace of the chunk-parallel form: the per-frame partials and chunk state images, then
// the attention stage's tail-split scratch.
static SplitWs parallel_ws(const rehyat_params* p) {
    const int G = state_frames(p);
    AttnArgs a = attn_common(p, nullptr, nullptr);
    a.nchunks = num_chunks(p);
    return split_ws(p, a, G > 0 ? parallel_layout(p, G).total : 0);
}

static size_t parallel_ws_bytes(const rehyat_params* p) { return parallel_ws(p).total; }

// Workspace of a streaming chunk step: the per-frame partials of up to Tc frames, then the
// tail-split scratch of the first chunk's attention launch, which splits the same tiles as
// the chunk-parallel grid (sized for a whole first chunk; counters zeroed by the first step).
static SplitWs stream_ws(const rehyat_params* p) {
    AttnArgs a = attn_common(p, nullptr, nullptr);
    a.stream = 1;
    a.s_frames = p->Tc;
    a.nchunks = 1;
    a.split_per_xcd = 1;  // asked for; the plan decides
    return split_ws(p, a, partial_bytes(p, p->Tc));
}

size_t rehyat_workspace_bytes(const rehyat_params* p) {
    if (check_params(p, true) != REHYAT_OK) return 0;
    return parallel_ws_bytes(p);
}

rehyat_status rehyat_parallel_states(const rehyat_params* p, const void* k, const void* v,
                                     const void* wk, const float* bk, void* ws, size_t ws_bytes,
                                     hipStream_t stream) {
    rehyat_status st = check_params(p, true);
    if (st != REHYAT_OK) return st;
    if (!aligned16(k) || !aligned16(v) || !aligned16(wk) || !aligned4_or_null(bk)) return REHYAT_EALIGN;
    const int G = state_frames(p);
    const SplitWs WL = parallel_ws(p);
    const size_t need = WL.total;
    if (need > 0 && (!ws || ws_bytes < need || reinterpret_cast<uintptr_t>(ws) % 256 != 0)) return REHYAT_EWORKSPACE;
    // the attention stage's tail-split counters start at zero (each split's second arrival
    // sets its counter back, so they stay zero between attention calls)
    unsigned* const cnt = WL.splits > 0 ? reinterpret_cast<unsigned*>(reinterpret_cast<char*>(ws) + WL.cnt) : nullptr;
    if (G == 0) return cnt ? hip_status(launch_zero(reinterpret_cast<float*>(cnt), WL.splits, stream)) : REHYAT_OK;

    const int64_t N = (int64_t)p->T * p->frame_tokens;
    const int BH = p->B * p->H;
    const ParallelLayout PL = parallel_layout(p, G);
    char* w = reinterpret_cast<char*>(ws);
    float* Sp = reinterpret_cast<float*>(w + PL.sp);
    float* Zp = reinterpret_cast<float*>(w + PL.zp);
    StateArgs s = state_common(p, wk, bk);
    s.k1 = k;
    s.v1 = v;
    s.kv1_bh_stride = N * p->D;
    s.nf1 = p->T;
    s.k2 = k;
    s.v2 = v;
    s.kv2_bh_stride = N * p->D;
    s.g0 = 0;
    s.G = G;
    s.Sp = Sp;
    s.Zp = Zp;
    st = hip_status(launch_state(s, p->in_dtype, stream));
    if (st != REHYAT_OK) return st;
    ScanArgs sc;
    std::memset(&sc, 0, sizeof(sc));
    sc.Sp = Sp;
    sc.Zp = Zp;
    sc.G = G;
    sc.simg = w + PL.img;
    sc.zimg = reinterpret_cast<float*>(w + PL.zimg);
    sc.slots = num_chunks(p);
    sc.BH = BH;
    sc.D = p->D;
    sc.Dphi = p->Dphi;
    sc.P = p->P;
    sc.T = p->T;
    sc.Tc = p->Tc;
    sc.To = p->To;
    sc.linear_only = p->linear_only;
    sc.zero_cnt = cnt;
    sc.nzero = WL.splits;
    return hip_status(launch_scan(sc, p->in_dtype, stream));
}

rehyat_status rehyat_parallel_attend(const rehyat_params* p, const void* q, const void* k,
                                     const void* v, const void* wq, const float* bq, void* out,
                                     const rehyat_aux* aux, void* ws, size_t ws_bytes,
                                     hipStream_t stream) {
    rehyat_status st = check_params(p, true);
    if (st != REHYAT_OK) return st;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(wq) || !aligned16(out) ||
        !aligned4_or_null(bq))
        return REHYAT_EALIGN;
    if (aux) {
        if ((aux->o_soft && !aligned16(aux->o_soft)) || (aux->y && !aligned16(aux->y)) ||
            !aligned4_or_null(aux->lse) || !aligned4_or_null(aux->z))
            return REHYAT_EALIGN;
    }
    const int G = state_frames(p);
    const SplitWs WL = parallel_ws(p);
    const size_t need = WL.total;
    if (need > 0 && (!ws || ws_bytes < need || reinterpret_cast<uintptr_t>(ws) % 256 != 0)) return REHYAT_EWORKSPACE;

    const int64_t N = (int64_t)p->T * p->frame_tokens;
    char* w = reinterpret_cast<char*>(ws);
    AttnArgs a = attn_common(p, wq, bq);
    a.q = q;
    a.out = out;
    a.q_bh_stride = N * p->D;
    a.k1 = k;
    a.v1 = v;
    a.kv1_bh_stride = N * p->D;
    a.k2 = k;
    a.v2 = v;
    a.kv2_bh_stride = N * p->D;
    if (G > 0) {
        const ParallelLayout PL = parallel_layout(p, G);
        a.simg = w + PL.img;
        a.zimg = reinterpret_cast<const float*>(w + PL.zimg);
    }
    a.img_slots = num_chunks(p);
    if (aux) {
        a.aux_o_soft = aux->o_soft;
        a.aux_lse = aux->lse;
        a.aux_y = aux->y;
        a.aux_z = aux->z;
    }
    a.aux_bh_stride = N;
    a.stream = 0;
    a.nchunks = num_chunks(p);
    a.split_per_xcd = WL.split_per_xcd;
    if (WL.splits > 0) {
        // arrival counters: zeroed by rehyat_parallel_states, left zero by every call
        a.split_cnt = reinterpret_cast<unsigned*>(w + WL.cnt);
        a.split_part = reinterpret_cast<float*>(w + WL.part);
    }
    return hip_status(launch_attn(a, p->in_dtype, p->out_dtype, stream));
}

rehyat_status rehyat_forward_parallel_aux(const rehyat_params* p, const void* q, const void* k,
                                          const void* v, const void* wq, const void* wk,
                                          const float* bq, const float* bk, void* out,
                                          const rehyat_aux* aux, void* ws, size_t ws_bytes,
                                          hipStream_t stream) {
    // validate every argument before the first launch
    rehyat_status st = check_params(p, true);
    if (st != REHYAT_OK) return st;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(wq) || !aligned16(wk) ||
        !aligned16(out) || !aligned4_or_null(bq) || !aligned4_or_null(bk))
        return REHYAT_EALIGN;
    if (aux) {
        if ((aux->o_soft && !aligned16(aux->o_soft)) || (aux->y && !aligned16(aux->y)) ||
            !aligned4_or_null(aux->lse) || !aligned4_or_null(aux->z))
            return REHYAT_EALIGN;
    }
    const size_t need = parallel_ws_bytes(p);
    if (need > 0 && (!ws || ws_bytes < need || reinterpret_cast<uintptr_t>(ws) % 256 != 0)) return REHYAT_EWORKSPACE;
    st = rehyat_parallel_states(p, k, v, wk, bk, ws, ws_bytes, stream);
    if (st != REHYAT_OK) return st;
    return rehyat_parallel_attend(p, q, k, v, wq, bq, out, aux, ws, ws_bytes, stream);
}

rehyat_status rehyat_forward_parallel(const rehyat_params* p, const void* q, const void* k,
                                      const void* v, const void* wq, const void* wk,
                                      const float* bq, const float* bk, void* out, void* ws,
                                      size_t ws_bytes, hipStream_t stream) {
    return rehyat_forward_parallel_aux(p, q, k, v, wq, wk, bq, bk, out, nullptr, ws, ws_bytes, stream);
}

size_t rehyat_state_bytes(const rehyat_params* p) {
    if (check_params(p, false) != REHYAT_OK) return 0;
    return state_layout(p).total;
}

size_t rehyat_stream_workspace_bytes(const rehyat_params* p) {
    if (check_params(p, false) != REHYAT_OK) return 0;
    return stream_ws(p).total;
}

rehyat_status rehyat_state_init(const rehyat_params* p, void* state, rehyat_stream* st,
                                hipStream_t stream) {
    rehyat_status s = check_params(p, false);
    if (s != REHYAT_OK) return s;
    if (!st) return REHYAT_ESTATE;
    if (!state || reinterpret_cast<uintptr_t>(state) % 256 != 0) return REHYAT_EALIGN;
    const StateLayout L = state_layout(p);
    // S and Z are adjacent at the start of the state; the overlap buffers need no clearing
    // because only the frames written by earlier steps are ever read.
    hipError_t e = launch_zero(reinterpret_cast<float*>(state), (int64_t)(L.ovk[0] / sizeof(float)), stream);
    if (e != hipSuccess) return REHYAT_EHIP;
    st->frames_seen = 0;
    st->frames_absorbed = 0;
    st->closed = 0;
    st->overlap_slot = 0;
    st->magic = kStreamMagic;
    st->reserved = 0;
    return REHYAT_OK;
}

rehyat_status rehyat_chunk_step(const rehyat_params* p, void* state, rehyat_stream* st,
                                const void* q, const void* k, const void* v, int32_t frames,
                                const void* wq, const void* wk, const float* bq, const float* bk,
                                void* out, void* ws, size_t ws_bytes, hipStream_t stream) {
    rehyat_status s = check_params(p, false);
    if (s != REHYAT_OK) return s;
    if (!st || st->magic != kStreamMagic || st->closed) return REHYAT_ESTATE;
    if (frames < 1 || frames > p->Tc) return REHYAT_ESTATE;
    if (st->frames_seen + frames > ((int64_t)1 << 30) / p->frame_tokens) return REHYAT_ESTATE;
    if (!state || reinterpret_cast<uintptr_t>(state) % 256 != 0) return REHYAT_EALIGN;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(wq) || !aligned16(wk) ||
        !aligned16(out) || !aligned4_or_null(bq) || !aligned4_or_null(bk))
        return REHYAT_EALIGN;
    const SplitWs WS = stream_ws(p);
    const size_t need = WS.total;
    if (!ws || ws_bytes < need || reinterpret_cast<uintptr_t>(ws) % 256 != 0) return REHYAT_EWORKSPACE;

    const StateLayout L = state_layout(p);
    char* base = reinterpret_cast<char*>(state);
    float* S = reinterpret_cast<float*>(base + L.S);
    float* Z = reinterpret_cast<float*>(base + L.Z);
    void* simg = base + L.img;
    float* zimg = reinterpret_cast<float*>(base + L.zimg);
    const int slot = st->overlap_slot;
    void* ovk = base + L.ovk[slot];
    void* ovv = base + L.ovv[slot];
    void* nvk = base + L.ovk[slot ^ 1];
    void* nvv = base + L.ovv[slot ^ 1];

    const int n = p->frame_tokens;
    const int64_t f0 = st->frames_seen, f1 = f0 + frames;
    const int64_t absorbed = st->frames_absorbed;
    const int held = (int)(f0 - absorbed);  // overlap frames held: [absorbed, f0)
    const int64_t ws_frame = p->linear_only ? f1 : (f0 - p->To > 0 ? f0 - p->To : 0);
    const int64_t ls = ws_frame;  // linear region of this chunk: frames [0, ls)
    const int64_t next_abs = p->linear_only ? f1 : (f1 - p->To > 0 ? f1 - p->To : 0);
    const int F = p->P * p->Dphi;
    const int BH = p->B * p->H;
    const int64_t ov_bh = overlap_rows(p) * p->D;
    const int64_t ch_bh = (int64_t)frames * n * p->D;
    float* Sp = reinterpret_cast<float*>(ws);
    float* Zp = reinterpret_cast<float*>(reinterpret_cast<char*>(ws) + align256((size_t)BH * p->Tc * F * p->D * sizeof(float)));

    // Fold the window frames [from, to) (global frame numbers) into S, Z: per-frame
    // partials, then added to the state in frame order.  With `partials_done` the partials
    // are already in the workspace (computed inside the attention launch) and only the
    // scan runs.
    auto state_args = [&](int64_t from, int64_t to) {
        StateArgs sa = state_common(p, wk, bk);
        sa.k1 = ovk;
        sa.v1 = ovv;
        sa.kv1_bh_stride = ov_bh;
        sa.nf1 = held;
        sa.k2 = k;
        sa.v2 = v;
        sa.kv2_bh_stride = ch_bh;
        sa.g0 = (int)(from - absorbed);
        sa.G = (int)(to - from);
        sa.Sp = Sp;
        sa.Zp = Zp;
        return sa;
    };
    auto absorb = [&](int64_t from, int64_t to, bool partials_done, const CopyArgs* with) -> rehyat_status {
        if (to <= from) return with ? hip_status(launch_copy(*with, stream)) : REHYAT_OK;
        const StateArgs sa = state_args(from, to);
        if (!partials_done) {
            rehyat_status r = hip_status(launch_state(sa, p->in_dtype, stream));
            if (r != REHYAT_OK) return r;
        }
        ScanArgs sc;
        std::memset(&sc, 0, sizeof(sc));
        sc.Sp = Sp;
        sc.Zp = Zp;
        sc.G = sa.G;
        sc.S_state = S;
        sc.Z_state = Z;
        sc.simg = simg;
        sc.zimg = zimg;
        sc.slots = 1;
        sc.BH = BH;
        sc.D = p->D;
        sc.Dphi = p->Dphi;
        sc.P = p->P;
        if (with) {
            sc.copy = *with;
            sc.copy_blocks = copy_blocks(*with);
        }
        return hip_status(launch_scan(sc, p->in_dtype, stream));
    };

    // 1. frames that belong to this chunk's linear region but are not yet in the state
    //    (only with an empty softmax window, where the chunk itself is linear)
    s = absorb(absorbed, ls, false, nullptr);
    if (s != REHYAT_OK) return s;

    // 2. softmax over [held overlap | chunk], linear part from the state.  The first rows
    //    of the chunk are copied after the held frames, up to a multiple of 64 rows, and
    //    read from there: every key tile but the last then lies in one buffer.
    const int held_rows = p->linear_only ? 0 : held * n;
    const int pad = held_rows % 64 == 0 ? 0 : std::min(64 - held_rows % 64, frames * n);
    if (pad > 0) {
        const int eb = (int)elem_bytes(p->in_dtype);
        CopyArgs c;
        c.s1k = k;  // source "frames" of one row each, all from the chunk
        c.s1v = v;
        c.s1_bh_stride = ch_bh;
        c.nf1 = pad;
        c.s2k = k;
        c.s2v = v;
        c.s2_bh_stride = ch_bh;
        c.dk = reinterpret_cast<char*>(ovk) + (int64_t)held_rows * p->D * eb;
        c.dv = reinterpret_cast<char*>(ovv) + (int64_t)held_rows * p->D * eb;
        c.d_bh_stride = ov_bh;
        c.f0 = 0;
        c.cnt = pad;
        c.BH = BH;
        c.n = 1;
        c.D = p->D;
        c.elem_bytes = eb;
        s = hip_status(launch_copy(c, stream));
        if (s != REHYAT_OK) return s;
    }
    AttnArgs a = attn_common(p, wq, bq);
    a.q = q;
    a.out = out;
    a.q_bh_stride = ch_bh;
    a.k1 = ovk;
    a.v1 = ovv;
    a.kv1_bh_stride = ov_bh;
    a.k2 = k;
    a.v2 = v;
    a.kv2_bh_stride = ch_bh;
    a.simg = simg;
    a.zimg = zimg;
    a.img_slots = 1;
    a.aux_bh_stride = (int64_t)frames * n;
    a.stream = 1;
    a.s_frames = frames;
    a.s_held = p->linear_only ? 0 : held;
    a.s_ls = (int)ls;
    a.s_pad = pad;
    a.nchunks = 1;
    if (f0 == 0 && WS.splits > 0) {
        // the first chunk splits the tiles the chunk-parallel grid splits (a first chunk
        // shorter than Tc, the whole clip, at most as many as a full one); its counters
        // start at zero here and every second arrival sets its counter back
        a.split_per_xcd = 1;  // asked for; the plan decides
        const int splits = wide_split_plan(a);
        if (splits > 0) {
            char* const wsb = reinterpret_cast<char*>(ws);
            a.split_cnt = reinterpret_cast<unsigned*>(wsb + WS.cnt);
            a.split_part = reinterpret_cast<float*>(wsb + WS.part);
            s = hip_status(launch_zero(reinterpret_cast<float*>(a.split_cnt), splits, stream));
            if (s != REHYAT_OK) return s;
        }
    }
    // 3. frames leaving the window before the next chunk.  Their partials read only K/V
    //    of the held frames and of the chunk, so for bf16 inputs they run inside the
    //    attention launch, in workgroups after the tiles; the scan into S, Z follows it
    //    (the attention reads the state image the scan rewrites).
    const int64_t from = ls > absorbed ? ls : absorbed;
    const bool side = p->in_dtype == REHYAT_BF16 && next_abs > from;
    if (side) {
        a.side = state_args(from, next_abs);
        a.side_blocks = a.side.BH * a.side.G;
    }
    s = hip_status(launch_attn(a, p->in_dtype, p->out_dtype, stream));
    if (s != REHYAT_OK) return s;

    // 4. keep frames [next_abs, f1) as the next overlap (into the other buffer); the copy
    //    runs in the scan's launch (it reads the held frames and the chunk, writes the
    //    buffer nothing else in this step reads)
    CopyArgs c;
    std::memset(&c, 0, sizeof(c));
    const bool keep = !p->linear_only && f1 > next_abs;
    if (keep) {
        c.s1k = ovk;
        c.s1v = ovv;
        c.s1_bh_stride = ov_bh;
        c.nf1 = held;
        c.s2k = k;
        c.s2v = v;
        c.s2_bh_stride = ch_bh;
        c.dk = nvk;
        c.dv = nvv;
        c.d_bh_stride = ov_bh;
        c.f0 = (int)(next_abs - absorbed);
        c.cnt = (int)(f1 - next_abs);
        c.BH = BH;
        c.n = n;
        c.D = p->D;
        c.elem_bytes = (int)elem_bytes(p->in_dtype);
    }
    s = absorb(from, next_abs, side, keep ? &c : nullptr);
    if (s != REHYAT_OK) return s;
    if (keep) st->overlap_slot = slot ^ 1;
    st->frames_seen = f1;
    st->frames_absorbed = next_abs;
    if (frames < p->Tc) st->closed = 1;
    return REHYAT_OK;
}

}  // extern "C"

// Distillation workspace: student output, teacher output (float32 [BH, N, D] each), the
// per-segment partial sums, then the forward workspace the two forwards share in turn.
namespace {

struct DistillLayout {
    size_t stu, tea, part, fwd, total;
    int nseg;
};

rehyat_params distill_student(const rehyat_params* p) {
    rehyat_params s = *p;
    s.out_dtype = REHYAT_FP32;
    return s;
}

rehyat_params distill_teacher(const rehyat_params* p) {
    rehyat_params t = *p;
    t.Tc = p->T;
    t.To = 0;
    t.linear_only = 0;
    t.out_dtype = REHYAT_FP32;
    return t;
}

DistillLayout distill_layout(const rehyat_params* p) {
    const rehyat_params ps = distill_student(p), pt = distill_teacher(p);
    const int64_t len = (int64_t)p->T * p->frame_tokens * p->D;
    const size_t out_bytes = align256((size_t)p->B * p->H * len * sizeof(float));
    DistillLayout L;
    L.nseg = sqdist_segments(len);
    L.stu = 0;
    L.tea = out_bytes;
    L.part = 2 * out_bytes;
    L.fwd = L.part + align256((size_t)p->B * p->H * L.nseg * sizeof(float));
    L.total = L.fwd + std::max(parallel_ws_bytes(&ps), parallel_ws_bytes(&pt));
    return L;
}

}  // namespace

extern "C" {

size_t rehyat_distill_workspace_bytes(const rehyat_params* p) {
    if (check_params(p, true) != REHYAT_OK) return 0;
    const rehyat_params pt = distill_teacher(p);
    if (check_params(&pt, true) != REHYAT_OK) return 0;
    return distill_layout(p).total;
}

rehyat_status rehyat_distill_loss(const rehyat_params* p, const void* q, const void* k,
                                  const void* v, const void* wq, const void* wk,
                                  const float* bq, const float* bk, float* loss, void* ws,
                                  size_t ws_bytes, hipStream_t stream) {
    rehyat_status st = check_params(p, true);
    if (st != REHYAT_OK) return st;
    const rehyat_params ps = distill_student(p), pt = distill_teacher(p);
    st = check_params(&pt, true);
    if (st != REHYAT_OK) return st;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(wq) || !aligned16(wk) ||
        !aligned4_or_null(bq) || !aligned4_or_null(bk) || !loss || !aligned4_or_null(loss))
        return REHYAT_EALIGN;
    const DistillLayout L = distill_layout(p);
    if ((int64_t)L.nseg * p->B * p->H >= ((int64_t)1 << 31)) return REHYAT_EINVAL;
    if (!ws || ws_bytes < L.total || reinterpret_cast<uintptr_t>(ws) % 256 != 0) return REHYAT_EWORKSPACE;
    char* w = reinterpret_cast<char*>(ws);
    st = rehyat_forward_parallel(&ps, q, k, v, wq, wk, bq, bk, w + L.stu, w + L.fwd, ws_bytes - L.fwd, stream);
    if (st != REHYAT_OK) return st;
    st = rehyat_forward_parallel(&pt, q, k, v, wq, wk, bq, bk, w + L.tea, w + L.fwd, ws_bytes - L.fwd, stream);
    if (st != REHYAT_OK) return st;
    const int64_t len = (int64_t)p->T * p->frame_tokens * p->D;
    return hip_status(launch_sqdist(reinterpret_cast<const float*>(w + L.stu), reinterpret_cast<const float*>(w + L.tea),
                                    len, p->B * p->H, reinterpret_cast<float*>(w + L.part), loss, stream));
}

}  // extern "C"

// Gradient workspace.  Distillation: the two outputs, the student's per-part outputs lse and
// z, the loss partials, separate forward workspaces for the student (whose per-frame state
// partials the gradient reads) and the teacher, then the linear-branch buffers.  Backward
// (upstream gradient given): no teacher; adds delta and log den per query, transposed
// weights and chunk sums, and the per-chunk softmax-branch buffers (P and dS of one chunk
// window for every slab, the transposed window keys, partial sums over query segments).
namespace {

constexpr int kGradSegRows = 2048;    // token rows per dW partial
constexpr int kColsumSegRows = 256;   // token rows per bias-gradient partial
constexpr int kSoftSegRows = 2048;    // query rows per dK / dV partial of a window

struct GradLayout {
    size_t stu, tea, lse, z, sqd, fwd_s, fwd_t, ah, u, phi, dphi, sz, rp, r, wp, bp;
    size_t delta, lden, wt, rt, sbuf, dpbuf, kt, pp, g16, total;
    int64_t stat_stride;  // floats from lden to delta
    int nseg_sq, nseg_w, nseg_b, lq_max, lk_max, ldp, nseg_s;
};

GradArgs grad_args(const rehyat_params* p) {
    GradArgs s;
    s.H = p->H;
    s.BH = p->B * p->H;
    s.n = p->frame_tokens;
    s.N = p->T * p->frame_tokens;
    s.D = p->D;
    s.Dphi = p->Dphi;
    s.P = p->P;
    s.F = p->P * p->Dphi;
    s.T = p->T;
    s.Tc = p->Tc;
    s.To = p->To;
    s.linear_only = p->linear_only;
    s.nc = num_chunks(p);
    s.G = state_frames(p);
    return s;
}

// chunk c: query rows [r0, r1), window key rows [k0, k1)
void chunk_rows(const rehyat_params* p, int c, int& r0, int& r1, int& k0, int& k1) {
    const int n = p->frame_tokens;
    const int f0 = c * p->Tc, f1 = std::min(f0 + p->Tc, p->T);
    const int ws = p->linear_only ? f1 : std::max(0, f0 - p->To);
    r0 = f0 * n;
    r1 = f1 * n;
    k0 = ws * n;
    k1 = f1 * n;
}

GradLayout grad_layout(const rehyat_params* p, bool backward) {
    const rehyat_params ps = distill_student(p), pt = distill_teacher(p);
    const GradArgs s = grad_args(p);
    const size_t BH = s.BH, N = s.N, f4 = sizeof(float), LD = s.D + 32;
    GradLayout L;
    L.nseg_sq = sqdist_segments((int64_t)N * s.D);
    L.nseg_w = (int)((N + kGradSegRows - 1) / kGradSegRows);
    L.nseg_b = (int)((N + kColsumSegRows - 1) / kColsumSegRows);
    L.lq_max = L.lk_max = 0;
    for (int c = 0; c < s.nc; ++c) {
        int r0, r1, k0, k1;
        chunk_rows(p, c, r0, r1, k0, k1);
        L.lq_max = std::max(L.lq_max, r1 - r0);
        L.lk_max = std::max(L.lk_max, k1 - k0);
    }
    L.ldp = (L.lk_max + 31) / 32 * 32;
    L.nseg_s = (L.lq_max + kSoftSegRows - 1) / kSoftSegRows;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t at = off;
        off += align256(bytes);
        return at;
    };
    L.stu = take(BH * N * s.D * f4);
    L.tea = take(backward ? 0 : BH * N * s.D * f4);
    L.lse = take(BH * N * f4);
    L.z = take(BH * N * f4);
    L.sqd = take(backward ? 0 : BH * L.nseg_sq * f4);
    L.fwd_s = take(parallel_ws_bytes(&ps));
    L.fwd_t = take(backward ? 0 : parallel_ws_bytes(&pt));
    L.ah = take(BH * N * LD * f4);
    L.u = take(BH * N * s.Dphi * f4);
    L.phi = take(BH * N * s.F * f4);
    // dphi only where the feature map's backward is a pass of its own (the fused feature
    // gradients of bf16 inputs write dpre over u)
    L.dphi = take(p->in_dtype == REHYAT_BF16 && ntf16_fusable(s) ? 0 : BH * N * s.F * f4);
    L.sz = take(BH * s.nc * s.F * LD * f4);
    L.rp = take(BH * s.nc * s.Tc * s.F * LD * f4);
    L.r = take(BH * s.nc * s.F * LD * f4);
    L.wp = take(BH * L.nseg_w * s.Dphi * s.D * f4);
    L.bp = take(BH * L.nseg_b * s.Dphi * f4);
    const size_t bw = backward ? 1 : 0;
    // per-query statistics of the backward: lden, then delta, each with 32 spare values (the
    // flash kernels read whole 32-query blocks)
    L.stat_stride = (int64_t)((BH * N + 32 + 63) / 64 * 64);
    L.lden = take(bw * 2 * (size_t)L.stat_stride * f4);
    L.delta = L.lden + (size_t)L.stat_stride * f4;
    L.wt = take(bw * p->H * s.D * s.Dphi * f4);
    L.rt = take(bw * BH * s.nc * s.D * s.F * f4);
    // score-sized buffers of the float32 path only (bf16 inputs take the flash kernels)
    const size_t sw = backward && p->in_dtype != REHYAT_BF16 ? 1 : 0;
    L.sbuf = take(sw * BH * L.lq_max * L.ldp * f4);
    L.dpbuf = take(sw * BH * L.lq_max * L.ldp * f4);
    L.kt = take(sw * BH * s.D * L.ldp * f4);
    L.pp = take(sw * BH * L.nseg_s * (size_t)L.lk_max * s.D * f4);
    L.g16 = take(backward && p->in_dtype == REHYAT_BF16 ? BH * N * s.D * 2 : 0);
    L.total = off;
    return L;
}

int tiles32(int rows) { return (rows + 31) / 32; }

// grid y / z extents of the gradient launches
bool grad_grid_ok(const GradArgs& s, const GradLayout& L) {
    return s.BH <= 65535 && tiles32(s.N) <= 65535 && (int64_t)s.T * tiles32(s.n) <= 65535 &&
           (int64_t)s.nc * tiles32(s.Tc * s.n) <= 65535 && (int64_t)s.BH * s.nc <= 65535 &&
           (int64_t)s.nc * s.Tc <= 65535 && L.lq_max <= 65535 && (int64_t)L.nseg_s <= 65535;
}

#define GRAD_TRY(expr)                              \
    do {                                            \
        rehyat_status st_ = hip_status(expr);       \
        if (st_ != REHYAT_OK) return st_;           \
    } while (0)

// Linear branch of the backward (chunk states of blog 2.3, feature map of blog 2.2.2): with
// AH = [a | h | 0] per query in place, the gradients of W_q, W_k (b_q, b_k when non-null)
// and, when dq is non-null, the linear branch's share of dq, dk, dv written to them (its
// products are the first to reach them; the softmax branch adds to them afterwards).
rehyat_status linear_branch(const rehyat_params* p, const GradArgs& s, const GradLayout& L, char* w,
                            const void* q, const void* k, const void* v, const void* wq, const void* wk,
                            const float* bq, const float* bk, float* dwq, float* dwk, float* dbq, float* dbk,
                            float* dq, float* dk, float* dv, hipStream_t stream) {
    auto F32 = [&](size_t off) { return reinterpret_cast<float*>(w + off); };
    const bool bf = p->in_dtype == REHYAT_BF16;
    const int LD = s.D + 32;
    const int64_t N = s.N;
    const rehyat_params ps = distill_student(p);
    const ParallelLayout PL = parallel_layout(&ps, s.G);
    GRAD_TRY(launch_grad_state_sz(s, F32(L.fwd_s + PL.sp), F32(L.fwd_s + PL.zp), F32(L.sz), stream));

    auto nt_base = [&]() {
        NtArgs a;
        std::memset(&a, 0, sizeof(a));
        a.sub_col = -1;
        a.rows = s.N;
        return a;
    };
    // u = softplus(W x + b) into L.u and, when phi_out, its powers (blog 2.2.2) into L.phi
    auto pre = [&](const void* x, const void* wmat, const float* bias, bool phi_out) {
        NtArgs a = nt_base();
        a.x = x;
        a.x_bt_stride = N * s.D;
        a.ldx = s.D;
        a.y = wmat;
        a.y_mat_stride = (int64_t)s.Dphi * s.D;
        a.ldy = s.D;
        a.nmat = p->H;
        a.mode = 0;
        a.K = s.D;
        a.ncols = s.Dphi;
        a.colbias = bias;
        a.colbias_head_stride = s.Dphi;
        a.c = F32(L.u);
        a.c_bt_stride = N * s.Dphi;
        a.ldc = s.Dphi;
        a.group_rows = s.N;
        a.ngroups = 1;
        a.softplus = 1;
        a.phi = phi_out ? F32(L.phi) : nullptr;
        a.phi_bt_stride = N * s.F;
        return launch_nt(a, s, bf, bf, stream, bf);
    };
    auto dw = [&](const void* x, float* dwout, float* dbout) -> hipError_t {
        TnArgs t;
        std::memset(&t, 0, sizeof(t));
        t.x = F32(L.u);
        t.x_bt_stride = N * s.Dphi;
        t.ldx = s.Dphi;
        t.y = x;
        t.y_bt_stride = N * s.D;
        t.ldy = s.D;
        t.mrows = s.Dphi;
        t.ncols = s.D;
        t.part = F32(L.wp);
        t.rows = s.N;
        t.group_rows = s.N;
        t.ngroups = 1;
        t.seg_rows = kGradSegRows;
        t.nseg = L.nseg_w;
        hipError_t e = launch_tn(t, s.BH, bf, stream, bf);
        if (e == hipSuccess) e = launch_grad_reduce(F32(L.wp), dwout, p->B, p->H, L.nseg_w, (int64_t)s.Dphi * s.D, stream);
        if (e == hipSuccess && dbout) {
            e = launch_grad_colsum(F32(L.u), s.BH, N, s.Dphi, kColsumSegRows, F32(L.bp), stream);
            if (e == hipSuccess) e = launch_grad_reduce(F32(L.bp), dbout, p->B, p->H, L.nseg_b, s.Dphi, stream);
        }
        return e;
    };
    // dx = dpre W (contraction over Dphi) with W transposed into L.wt
    auto dx = [&](const void* wmat, float* dxout) -> hipError_t {
        hipError_t e = launch_transpose(wmat, bf, (int64_t)s.Dphi * s.D, s.D, F32(L.wt), (int64_t)s.D * s.Dphi, s.Dphi,
                                        s.Dphi, s.D, p->H, stream);
        if (e != hipSuccess) return e;
        NtArgs a = nt_base();
        a.x = F32(L.u);
        a.x_bt_stride = N * s.Dphi;
        a.ldx = s.Dphi;
        a.y = F32(L.wt);
        a.y_mat_stride = (int64_t)s.D * s.Dphi;
        a.ldy = s.Dphi;
        a.nmat = p->H;
        a.mode = 0;
        a.K = s.Dphi;
        a.ncols = s.D;
        a.c = dxout;
        a.c_bt_stride = N * s.D;
        a.ldc = s.D;
        a.group_rows = s.N;
        a.ngroups = 1;
        return launch_nt(a, s, false, false, stream, bf);
    };

    // bf16 inputs with whole-block parts: the feature gradients write dpre over u directly
    const bool fuse = bf && ntf16_fusable(s);

    // query side: phi_q, dphi_q = [S_c | -Z_c] [a | h], R per chunk, dpre_q, dW_q, db_q
    GRAD_TRY(pre(q, wq, bq, true));
    {
        NtArgs a = nt_base();
        a.x = F32(L.ah);
        a.x_bt_stride = N * LD;
        a.ldx = LD;
        a.y = F32(L.sz);
        a.y_mat_stride = (int64_t)s.F * LD;
        a.ldy = LD;
        a.nmat = s.nc;
        a.mode = 1;
        a.K = LD;
        a.ncols = s.F;
        a.c = F32(L.dphi);
        a.c_bt_stride = N * s.F;
        a.ldc = s.F;
        a.group_rows = s.Tc * s.n;
        a.ngroups = s.nc;
        if (fuse) {
            a.c = F32(L.u);
            a.c_bt_stride = N * s.Dphi;
            a.ldc = s.Dphi;
            GRAD_TRY(launch_ntf16(a, s, false, stream));
        } else {
            GRAD_TRY(launch_nt(a, s, false, false, stream, bf));
        }
    }
    {
        TnArgs t;
        std::memset(&t, 0, sizeof(t));
        t.x = F32(L.phi);
        t.x_bt_stride = N * s.F;
        t.ldx = s.F;
        t.y = F32(L.ah);
        t.y_bt_stride = N * LD;
        t.ldy = LD;
        t.mrows = s.F;
        t.ncols = LD;
        t.part = F32(L.rp);
        t.rows = s.N;
        t.group_rows = s.Tc * s.n;
        t.ngroups = s.nc;
        t.seg_rows = s.n;
        t.nseg = s.Tc;
        GRAD_TRY(launch_tn(t, s.BH, false, stream, bf, bf));  // phi in bf16 for bf16 inputs
        const int64_t E = (int64_t)s.F * LD;
        GRAD_TRY(launch_grad_reduce(F32(L.rp), F32(L.r), 1, s.BH * s.nc, s.Tc, E, stream));
        GRAD_TRY(launch_grad_suffix(F32(L.r), s.BH, s.nc, E, stream));
    }
    if (!fuse) GRAD_TRY(launch_grad_phi_bwd(s, F32(L.u), F32(L.dphi), stream));
    GRAD_TRY(dw(q, dwq, dbq));
    if (dq) GRAD_TRY(dx(wq, dq));

    // key side: u_k (phi_k only for dv += R^T phi_k), dphi_k = R v - r per key frame, dpre_k,
    // dW_k, db_k
    GRAD_TRY(pre(k, wk, bk, dv != nullptr));
    if (dv) {
        GRAD_TRY(launch_transpose(F32(L.r), false, (int64_t)s.F * LD, LD, F32(L.rt), (int64_t)s.D * s.F, s.F, s.F, s.D,
                                  s.BH * s.nc, stream));
        NtArgs a = nt_base();
        a.x = F32(L.phi);
        a.x_bt_stride = N * s.F;
        a.ldx = s.F;
        a.y = F32(L.rt);
        a.y_mat_stride = (int64_t)s.D * s.F;
        a.ldy = s.F;
        a.nmat = s.nc;
        a.mode = 2;
        a.K = s.F;
        a.ncols = s.D;
        a.c = dv;  // rows of key frames no chunk's state holds get zeros
        a.c_bt_stride = N * s.D;
        a.ldc = s.D;
        a.group_rows = s.n;
        a.ngroups = s.T;
        GRAD_TRY(launch_nt(a, s, bf, false, stream, bf));  // phi in bf16 for bf16 inputs
    }
    {
        NtArgs a = nt_base();
        a.x = v;
        a.x_bt_stride = N * s.D;
        a.ldx = s.D;
        a.y = F32(L.r);
        a.y_mat_stride = (int64_t)s.F * LD;
        a.ldy = LD;
        a.nmat = s.nc;
        a.mode = 2;
        a.K = s.D;
        a.ncols = s.F;
        a.sub_col = s.D;
        a.c = F32(L.dphi);
        a.c_bt_stride = N * s.F;
        a.ldc = s.F;
        a.group_rows = s.n;
        a.ngroups = s.T;
        if (fuse) {
            a.c = F32(L.u);
            a.c_bt_stride = N * s.Dphi;
            a.ldc = s.Dphi;
            GRAD_TRY(launch_ntf16(a, s, true, stream));
        } else {
            GRAD_TRY(launch_nt(a, s, bf, false, stream, bf));
        }
    }
    if (!fuse) GRAD_TRY(launch_grad_phi_bwd(s, F32(L.u), F32(L.dphi), stream));
    GRAD_TRY(dw(k, dwk, dbk));
    if (dk) GRAD_TRY(dx(wk, dk));
    return REHYAT_OK;
}

rehyat_status zero_param_grads(const rehyat_params* p, const GradArgs& s, float* dwq, float* dwk, float* dbq,
                               float* dbk, hipStream_t stream) {
    const int64_t HW = (int64_t)p->H * s.Dphi * s.D;
    GRAD_TRY(launch_zero(dwq, HW, stream));
    GRAD_TRY(launch_zero(dwk, HW, stream));
    if (dbq) GRAD_TRY(launch_zero(dbq, (int64_t)p->H * s.Dphi, stream));
    if (dbk) GRAD_TRY(launch_zero(dbk, (int64_t)p->H * s.Dphi, stream));
    return REHYAT_OK;
}

bool grad_ptrs_ok(const void* q, const void* k, const void* v, const void* wq, const void* wk, const float* bq,
                  const float* bk, const float* dwq, const float* dwk, const float* dbq, const float* dbk) {
    return aligned16(q) && aligned16(k) && aligned16(v) && aligned16(wq) && aligned16(wk) && aligned4_or_null(bq) &&
           aligned4_or_null(bk) && dwq && aligned4_or_null(dwq) && dwk && aligned4_or_null(dwk) &&
           aligned4_or_null(dbq) && aligned4_or_null(dbk);
}

}  // namespace

extern "C" {

size_t rehyat_distill_grad_workspace_bytes(const rehyat_params* p) {
    if (check_params(p, true) != REHYAT_OK) return 0;
    const rehyat_params pt = distill_teacher(p);
    if (check_params(&pt, true) != REHYAT_OK) return 0;
    return grad_layout(p, false).total;
}

rehyat_status rehyat_distill_grad(const rehyat_params* p, const void* q, const void* k, const void* v,
                                  const void* wq, const void* wk, const float* bq, const float* bk, float* loss,
                                  float* dwq, float* dwk, float* dbq, float* dbk, void* ws, size_t ws_bytes,
                                  hipStream_t stream) {
    rehyat_status st = check_params(p, true);
    if (st != REHYAT_OK) return st;
    const rehyat_params ps = distill_student(p), pt = distill_teacher(p);
    st = check_params(&pt, true);
    if (st != REHYAT_OK) return st;
    if (!grad_ptrs_ok(q, k, v, wq, wk, bq, bk, dwq, dwk, dbq, dbk) || !loss || !aligned4_or_null(loss))
        return REHYAT_EALIGN;
    const GradArgs s = grad_args(p);
    const GradLayout L = grad_layout(p, false);
    if ((int64_t)L.nseg_sq * s.BH >= ((int64_t)1 << 31) || (int64_t)s.N * (s.D + 32) >= ((int64_t)1 << 31) ||
        (int64_t)s.N * s.F >= ((int64_t)1 << 31) || !grad_grid_ok(s, L))
        return REHYAT_EINVAL;
    if (!ws || ws_bytes < L.total || reinterpret_cast<uintptr_t>(ws) % 256 != 0) return REHYAT_EWORKSPACE;
    char* w = reinterpret_cast<char*>(ws);
    auto F32 = [&](size_t off) { return reinterpret_cast<float*>(w + off); };

    // forward: student (float output and per-part outputs), teacher, loss
    rehyat_aux aux;
    std::memset(&aux, 0, sizeof(aux));
    aux.lse = F32(L.lse);
    aux.z = F32(L.z);
    st = rehyat_forward_parallel_aux(&ps, q, k, v, wq, wk, bq, bk, w + L.stu, &aux, w + L.fwd_s, L.fwd_t - L.fwd_s,
                                     stream);
    if (st != REHYAT_OK) return st;
    st = rehyat_forward_parallel(&pt, q, k, v, wq, wk, bq, bk, w + L.tea, w + L.fwd_t, L.ah - L.fwd_t, stream);
    if (st != REHYAT_OK) return st;
    const int64_t len = (int64_t)s.N * s.D;
    GRAD_TRY(launch_sqdist(F32(L.stu), F32(L.tea), len, s.BH, F32(L.sqd), loss, stream));
    if (s.G == 0) return zero_param_grads(p, s, dwq, dwk, dbq, dbk, stream);  // the loss does not depend on phi
    GRAD_TRY(launch_grad_rows(s, F32(L.stu), F32(L.tea), nullptr, F32(L.lse), F32(L.z), F32(L.ah), nullptr, nullptr,
                              nullptr, stream));
    return linear_branch(p, s, L, w, q, k, v, wq, wk, bq, bk, dwq, dwk, dbq, dbk, nullptr, nullptr, nullptr, stream);
}

size_t rehyat_backward_workspace_bytes(const rehyat_params* p) {
    if (check_params(p, true) != REHYAT_OK) return 0;
    return grad_layout(p, true).total;
}

rehyat_status rehyat_backward(const rehyat_params* p, const void* q, const void* k, const void* v, const void* wq,
                              const void* wk, const float* bq, const float* bk, const float* dout, float* dq,
                              float* dk, float* dv, float* dwq, float* dwk, float* dbq, float* dbk, void* ws,
                              size_t ws_bytes, hipStream_t stream) {
    rehyat_status st = check_params(p, true);
    if (st != REHYAT_OK) return st;
    if (!grad_ptrs_ok(q, k, v, wq, wk, bq, bk, dwq, dwk, dbq, dbk) || !aligned16(dout) || !aligned16(dq) ||
        !aligned16(dk) || !aligned16(dv))
        return REHYAT_EALIGN;
    const rehyat_params ps = distill_student(p);
    const GradArgs s = grad_args(p);
    const GradLayout L = grad_layout(p, true);
    if ((int64_t)s.N * (s.D + 32) >= ((int64_t)1 << 31) || (int64_t)s.N * s.F >= ((int64_t)1 << 31) ||
        (int64_t)L.lq_max * L.ldp >= ((int64_t)1 << 31) || !grad_grid_ok(s, L))
        return REHYAT_EINVAL;
    if (!ws || ws_bytes < L.total || reinterpret_cast<uintptr_t>(ws) % 256 != 0) return REHYAT_EWORKSPACE;
    char* w = reinterpret_cast<char*>(ws);
    auto F32 = [&](size_t off) { return reinterpret_cast<float*>(w + off); };
    const bool bf = p->in_dtype == REHYAT_BF16;
    const int64_t N = s.N, ND = N * s.D;

    // recompute the forward with float output and the per-part outputs lse, z
    rehyat_aux aux;
    std::memset(&aux, 0, sizeof(aux));
    aux.lse = F32(L.lse);
    aux.z = F32(L.z);
    st = rehyat_forward_parallel_aux(&ps, q, k, v, wq, wk, bq, bk, w + L.stu, &aux, w + L.fwd_s, L.fwd_t - L.fwd_s,
                                     stream);
    if (st != REHYAT_OK) return st;
    // bf16 inputs: the upstream gradient also rounded to bf16 once (the flash products' operand precision)
    GRAD_TRY(launch_grad_rows(s, F32(L.stu), nullptr, dout, F32(L.lse), F32(L.z), F32(L.ah), F32(L.delta),
                              F32(L.lden), bf ? (void*)(w + L.g16) : nullptr, stream));
    if (s.G > 0) {
        // writes dq, dk, dv first
        st = linear_branch(p, s, L, w, q, k, v, wq, wk, bq, bk, dwq, dwk, dbq, dbk, dq, dk, dv, stream);
        if (st != REHYAT_OK) return st;
    } else {
        GRAD_TRY(launch_zero(dq, (int64_t)s.BH * ND, stream));
        GRAD_TRY(launch_zero(dk, (int64_t)s.BH * ND, stream));
        GRAD_TRY(launch_zero(dv, (int64_t)s.BH * ND, stream));
        st = zero_param_grads(p, s, dwq, dwk, dbq, dbk, stream);
        if (st != REHYAT_OK) return st;
    }

    const float scale = (float)(1.0 / std::sqrt((double)s.D));
    if (bf) {
        // softmax branch, flash style (blog 2.2.1 window, scores q.k / sqrt(D)): P and dS
        // recomputed tile by tile from lden and delta, dK / dV and dQ in two passes
        BwdArgs b;
        std::memset(&b, 0, sizeof(b));
        b.q = q;
        b.k = k;
        b.v = v;
        b.g = w + L.g16;
        b.stats = F32(L.lden);
        b.stat_stride = L.stat_stride;
        b.dq = dq;
        b.dk = dk;
        b.dv = dv;
        b.BH = s.BH;
        b.N = (int)N;
        b.n = s.n;
        b.T = s.T;
        b.Tc = s.Tc;
        b.To = s.To;
        b.linear_only = s.linear_only;
        b.nc = s.nc;
        b.scale = scale;
        b.scale_log2 = scale * 1.4426950408889634f;
        GRAD_TRY(launch_bwd_softmax(b, s.D, stream));
        return REHYAT_OK;
    }
    // float32 inputs: one chunk window at a time through score-sized buffers (products on the
    // fp32 matrix core)
    const int64_t pbt = (int64_t)L.lq_max * L.ldp;
    for (int c = 0; c < s.nc; ++c) {
        int r0, r1, k0, k1;
        chunk_rows(p, c, r0, r1, k0, k1);
        const int Lq = r1 - r0, Lk = k1 - k0;
        if (Lk == 0) continue;
        const float* qc = reinterpret_cast<const float*>(q) + (size_t)r0 * s.D;
        const float* kw = reinterpret_cast<const float*>(k) + (size_t)k0 * s.D;
        const float* vw = reinterpret_cast<const float*>(v) + (size_t)k0 * s.D;
        auto nt = [&](const float* x, int64_t xbs, int ldx, const float* y, int64_t ybs, int ldy, int K, int ncols,
                      float* c_, int64_t cbs, int ldc, int acc) {
            NtArgs a;
            std::memset(&a, 0, sizeof(a));
            a.x = x;
            a.x_bt_stride = xbs;
            a.ldx = ldx;
            a.y = y;
            a.y_mat_stride = ybs;
            a.ldy = ldy;
            a.nmat = s.BH;
            a.mode = 3;
            a.K = K;
            a.ncols = ncols;
            a.sub_col = -1;
            a.c = c_;
            a.c_bt_stride = cbs;
            a.ldc = ldc;
            a.rows = Lq;
            a.group_rows = Lq;
            a.ngroups = 1;
            a.accumulate = acc;
            return launch_nt(a, s, false, false, stream);
        };
        // S = Q_c K_w^T and dP = G_c V_w^T, then P and dS in place
        GRAD_TRY(nt(qc, ND, s.D, kw, ND, s.D, s.D, Lk, F32(L.sbuf), pbt, L.ldp, 0));
        GRAD_TRY(nt(dout + (size_t)r0 * s.D, ND, s.D, vw, ND, s.D, s.D, Lk, F32(L.dpbuf), pbt, L.ldp, 0));
        GRAD_TRY(launch_softmax_bwd(F32(L.sbuf), F32(L.dpbuf), F32(L.lden) + r0, F32(L.delta) + r0, N, s.BH, Lq, Lk,
                                    L.ldp, pbt, scale, stream));
        // dV_w += P^T G_c and dK_w += dS^T Q_c: partial sums over query segments, then added
        auto tn_add = [&](const float* X, const float* Y, float* out) -> hipError_t {
            TnArgs t;
            std::memset(&t, 0, sizeof(t));
            t.x = X;
            t.x_bt_stride = pbt;
            t.ldx = L.ldp;
            t.y = Y;
            t.y_bt_stride = ND;
            t.ldy = s.D;
            t.mrows = Lk;
            t.ncols = s.D;
            t.part = F32(L.pp);
            t.rows = Lq;
            t.group_rows = Lq;
            t.ngroups = 1;
            t.seg_rows = kSoftSegRows;
            t.nseg = (Lq + kSoftSegRows - 1) / kSoftSegRows;
            hipError_t e = launch_tn(t, s.BH, false, stream);
            if (e == hipSuccess)
                e = launch_grad_reduce(F32(L.pp), out + (size_t)k0 * s.D, 1, s.BH, t.nseg, (int64_t)Lk * s.D, stream,
                                       ND, true);
            return e;
        };
        GRAD_TRY(tn_add(F32(L.sbuf), dout + (size_t)r0 * s.D, dv));
        GRAD_TRY(tn_add(F32(L.dpbuf), qc, dk));
        // dQ_c += dS K_w with K_w transposed (zero past Lk)
        GRAD_TRY(launch_transpose(kw, false, ND, s.D, F32(L.kt), (int64_t)s.D * L.ldp, L.ldp, Lk, s.D, s.BH, stream));
        GRAD_TRY(nt(F32(L.dpbuf), pbt, L.ldp, F32(L.kt), (int64_t)s.D * L.ldp, L.ldp, Lk, s.D, dq + (size_t)r0 * s.D,
                    ND, s.D, 1));
    }
    return REHYAT_OK;
}

}  // extern "C"
