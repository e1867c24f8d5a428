/*
 * rehyat.h -- C ABI of the MI355X (gfx950) library for ReHyAt chunk-wise recurrent
 * hybrid attention (forward pass).
 *
 * The operation (ReHyAt blog, maplevalley.com.cn, sections 2.2.1, 2.2.2 and 2.3):
 * tokens are T latent frames of `frame_tokens` (n) tokens each, token index = frame*n + s.
 * Frames are grouped into chunks of Tc frames (the last chunk may be shorter).  A query
 * in chunk [f0, f1) attends
 *   - with softmax weights exp(q.k / sqrt(D)) to every key of frames [max(0, f0-To), f1)
 *     (its own chunk plus To overlapping preceding frames; bidirectional inside), and
 *   - with polynomial-kernel weights phi_q(q) . phi_k(k) to every key of the earlier
 *     frames [0, max(0, f0-To)), carried as the states S = sum phi_k(k) v^T and
 *     Z = sum phi_k(k);
 * and the output is (softmax numerator + phi_q(q) S) / (softmax denominator + phi_q(q) Z).
 * phi (blog section 2.2.2): u = softplus(W x + b) with one Dphi x D map per head
 * (a grouped 1x1 linear), u split into P contiguous parts (the first Dphi mod P parts
 * one entry longer), each part raised elementwise to the powers 1..P, all concatenated:
 * F = P*Dphi features in the order [part0^1 | part0^2 | .. | part0^P | part1^1 | ..].
 * Queries and keys have separate maps (W_q, W_k).  With linear_only = 1 the softmax
 * window is empty and the linear region of chunk [f0, f1) is frames [0, f1).
 *
 * Conventions for every entry point:
 *   - Layout: q, k, v, out are dense row-major [B, H, tokens, D]; weights [H, Dphi, D]
 *     in the input dtype; biases [H, Dphi] float32 or NULL.
 *   - Ownership: the caller allocates every device buffer (inputs, outputs, state,
 *     workspace).  The library never allocates, frees or synchronises.
 *   - Pointers are device pointers, 16-byte aligned (biases 4-byte aligned).
 *   - Asynchrony: all work is enqueued on the caller's stream; the return value reports
 *     validation (checked before any HIP call) and launch errors.  Device faults appear
 *     at the caller's next synchronisation.
 *   - Determinism: repeated calls on the same inputs give identical bits.  Atomics appear
 *     only in the bf16 attention kernel's tail split (the last chunk-0 query tiles of each
 *     XCD run as two workgroups over the two halves of the window): each half stores its
 *     partial with agent-scope atomic stores and counts its arrival with one atomic add;
 *     the second to arrive reads the other's partial with agent-scope atomic loads and
 *     merges both in half order, so the result does not depend on which arrives first.
 *   - Thread safety: no shared mutable state beyond a per-device cache of kernel LDS limits
 *     (idempotent); one in-flight call per streaming state.
 */
#ifndef REHYAT_H
#define REHYAT_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    REHYAT_OK = 0,
    REHYAT_EINVAL = 1,     /* a parameter value is out of range */
    REHYAT_ESHAPE = 2,     /* unsupported shape: D not in {32,64,128}, Dphi not in {32,64,96,128}, P not in 1..4 */
    REHYAT_EALIGN = 3,     /* a required pointer is NULL or not 16-byte aligned */
    REHYAT_EWORKSPACE = 4, /* workspace pointer NULL or ws_bytes below the required size */
    REHYAT_ESTATE = 5,     /* streaming misuse: frames out of range, stream closed, bad handle */
    REHYAT_EHIP = 6,       /* a kernel launch failed */
    REHYAT_ESCRATCH = 7    /* rehyat_forward_parallel_noalloc: the call needs more workspace than
                              the library's static scratch area (64 MiB per GPU) */
} rehyat_status;

typedef enum { REHYAT_FP32 = 0, REHYAT_BF16 = 1 } rehyat_dtype;

typedef struct {
    int32_t B, H;          /* batch, heads */
    int32_t D;             /* head dim (value dim = D): 32, 64 or 128 */
    int32_t T;             /* latent frames (ignored by the streaming entry points) */
    int32_t frame_tokens;  /* n = tokens per latent frame (H x W of the latent grid) */
    int32_t Tc, To;        /* chunk frames (>= 1), overlap frames (>= 0) */
    int32_t Dphi, P;       /* phi width (32, 64, 96 or 128), parts = max power (1..4) */
    int32_t linear_only;   /* 1: empty softmax window (normalised chunk-causal linear attention) */
    int32_t in_dtype;      /* rehyat_dtype of q, k, v, weights (and features / overlap state) */
    int32_t out_dtype;     /* rehyat_dtype of out */
} rehyat_params;

/* Host-side handle of a streaming state; caller-owned, filled by rehyat_state_init. */
typedef struct {
    int64_t frames_seen;      /* frames consumed so far */
    int64_t frames_absorbed;  /* frames already folded into S, Z */
    int32_t closed;           /* 1 after a final chunk shorter than Tc */
    int32_t overlap_slot;     /* which of the two overlap buffers holds the held frames */
    int32_t magic;            /* set by rehyat_state_init */
    int32_t reserved;
} rehyat_stream;

/* Optional per-part outputs of rehyat_forward_parallel_aux (any member may be NULL).
 * All float32, tokens in the same [B, H, tokens] order as out. */
typedef struct {
    float* o_soft;  /* [B,H,N,D] softmax part normalised by its own sum (0 when the window is empty) */
    float* lse;     /* [B,H,N] log of the softmax denominator sum_j exp(q.k_j/sqrt(D)) (-inf if empty) */
    float* y;       /* [B,H,N,D] phi_q(q) S  (0 when the linear region is empty) */
    float* z;       /* [B,H,N]   phi_q(q) Z  (0 when the linear region is empty) */
} rehyat_aux;

/* Human-readable name of a status code (static string). */
const char* rehyat_status_string(rehyat_status s);

/* Number of phi features F = P * Dphi, or -1 if the parameters are invalid. */
int32_t rehyat_features(const rehyat_params* p);

/* phi feature map (blog 2.2.2) of x [B,H,N,D] with w [H,Dphi,D] (+ bias [H,Dphi]) into
 * feat [B,H,N,F] in in_dtype, N = T * frame_tokens.  Test and API entry point; the
 * attention entry points compute phi internally and never write features to memory. */
rehyat_status rehyat_phi(const rehyat_params* p, const void* x, const void* w, const float* bias,
                         void* feat, hipStream_t stream);

/* Workspace bytes needed by rehyat_forward_parallel(_aux): per-frame state partials,
 * float32 [B,H,G,F,D] + [B,H,G,F] for the G frames that enter some chunk's linear region,
 * then one image of the state per chunk (S in in_dtype, Z float32); then, for bf16 inputs
 * whose first chunk is a whole chunk (Tc frames) with a window of at least four 64-token
 * tiles, the attention stage's tail-split scratch: one uint32 arrival counter per split
 * tile (up to 8 per XCD; zeroed by the states stage, left zero by every attend) and per
 * split 2 x 8 waves x 64 lanes x (D/2 + 2) float32 partials.  0 if none of these is needed. */
size_t rehyat_workspace_bytes(const rehyat_params* p);

/* Chunk-parallel forward (all chunks at once): per-frame partials of phi_k(K)^T [V|1],
 * inclusive prefix over frames, then the windowed softmax tile kernel with the linear
 * part and the shared normalisation fused into its epilogue.  With Tc >= T this is
 * plain softmax attention (the full-softmax comparator).
 * q, k, v, out: [B,H,T*n,D]; wq, wk: [H,Dphi,D]; bq, bk: [H,Dphi] float32 or NULL. */
rehyat_status rehyat_forward_parallel(const rehyat_params* p, const void* q, const void* k,
                                      const void* v, const void* wq, const void* wk,
                                      const float* bq, const float* bk, void* out, void* ws,
                                      size_t ws_bytes, hipStream_t stream);

/* rehyat_forward_parallel without a caller workspace, for callers that cannot allocate
 * device memory (code under graph capture, serving loops, harnesses that forbid allocation).
 * The workspace is a static area of the library, 64 MiB on every GPU it runs on, held until
 * the process ends; the call allocates nothing (its first call on a device looks the area up).
 * Same operation, arguments (without ws, ws_bytes), layouts and results as
 * rehyat_forward_parallel.  REHYAT_ESCRATCH when rehyat_workspace_bytes(p) exceeds 64 MiB
 * (for example the 20 s, B = 2 layer; the 5 s Wan2.1-1.3B layer needs about 56 MB), before
 * any launch.  Every call on a GPU uses the same area: calls that overlap on one GPU (other
 * streams, other host threads) race; calls in stream order do not. */
rehyat_status rehyat_forward_parallel_noalloc(const rehyat_params* p, const void* q, const void* k,
                                              const void* v, const void* wq, const void* wk,
                                              const float* bq, const float* bk, void* out,
                                              hipStream_t stream);

/* Same as rehyat_forward_parallel, also writing the per-part outputs that are non-NULL
 * in *aux (aux itself may be NULL). */
rehyat_status rehyat_forward_parallel_aux(const rehyat_params* p, const void* q, const void* k,
                                          const void* v, const void* wq, const void* wk,
                                          const float* bq, const float* bk, void* out,
                                          const rehyat_aux* aux, void* ws, size_t ws_bytes,
                                          hipStream_t stream);

/* The two stages of rehyat_forward_parallel_aux, for callers that reuse the states or time
 * the stages separately.  rehyat_parallel_states writes the per-frame partials of
 * phi_k(K)^T [V|1] and their inclusive prefix over frames into ws (blog 2.3 state sums)
 * and zeroes the tail-split counters; rehyat_parallel_attend runs the windowed softmax
 * tile kernel with the fused linear part, reading the states and using only the
 * tail-split scratch of ws, whose counters it leaves zero, so it may run any number of
 * times per states call.  Same arguments, layouts and status codes as above; ws must hold
 * the states of the same k, v, wk, bk when attend runs (stream order suffices; calls on
 * the same ws must not overlap). */
rehyat_status rehyat_parallel_states(const rehyat_params* p, const void* k, const void* v,
                                     const void* wk, const float* bk, void* ws, size_t ws_bytes,
                                     hipStream_t stream);
rehyat_status rehyat_parallel_attend(const rehyat_params* p, const void* q, const void* k,
                                     const void* v, const void* wq, const float* bq, void* out,
                                     const rehyat_aux* aux, void* ws, size_t ws_bytes,
                                     hipStream_t stream);

/* Streaming (ReHyAt blog 5.2, the streaming loop: the state is carried from chunk to
 * chunk, so memory does not grow with the clip).  Device state bytes: S float32 [B,H,F,D], Z float32 [B,H,F], the image of the state and
 * two overlap buffers of K and V [B,H,To*n+64,D] in in_dtype (the held frames, then up to
 * 63 rows of the current chunk).  Independent of the clip length. */
size_t rehyat_state_bytes(const rehyat_params* p);

/* Workspace bytes for rehyat_chunk_step: per-frame partials for up to Tc frames,
 * float32 [B,H,Tc,F,D] + [B,H,Tc,F], then for bf16 inputs the tail-split scratch of the
 * first chunk's attention launch (the same layout and split tiles as the chunk-parallel
 * form's; its counters are zeroed by the first chunk step).  Independent of the clip
 * length. */
size_t rehyat_stream_workspace_bytes(const rehyat_params* p);

/* Zero S and Z on `stream` and reset the host handle (frames_seen = 0). */
rehyat_status rehyat_state_init(const rehyat_params* p, void* state, rehyat_stream* st,
                                hipStream_t stream);

/* Process the next chunk of `frames` frames: q, k, v, out are [B,H,frames*n,D].
 * frames must equal Tc except on a final, shorter call, after which the stream is closed
 * (REHYAT_ESTATE on further calls).  Outputs equal those of rehyat_forward_parallel on
 * the concatenated clip bit for bit: the same kernels add the same partials in the same
 * order, sweep the same window tiles and, on the first chunk, split the same tiles.  The call reads S, Z and the held overlap frames,
 * then folds the frames that leave the softmax window into S, Z (for bf16 inputs their
 * partials run in the attention launch, on CUs its tiles leave free) and keeps the last
 * To frames. */
rehyat_status rehyat_chunk_step(const rehyat_params* p, void* state, rehyat_stream* st,
                                const void* q, const void* k, const void* v, int32_t frames,
                                const void* wq, const void* wk, const float* bq, const float* bk,
                                void* out, void* ws, size_t ws_bytes, hipStream_t stream);

/* Attention-distillation objective (blog 3.1.1: with the teacher frozen, only phi_q and
 * phi_k are trained so that the hybrid block's output approaches, in L2, the softmax
 * teacher's output on the same inputs).  Reading taken: the squared Euclidean distance
 * per (batch, head) slab,
 *     loss[b*H + h] = sum_{i < N, d < D} (o_hyb[b,h,i,d] - o_soft[b,h,i,d])^2,
 * where o_hyb is rehyat_forward_parallel with *p and float32 output, and o_soft is full
 * softmax attention exp(q.k/sqrt(D)) over all N tokens of the clip (the same tile kernel
 * with one window, Tc = T, no linear part).  Both outputs stay float32 in ws; the sum runs
 * in a fixed order, so repeated calls give identical bits.  p->out_dtype is ignored.
 * loss: device float32 [B*H] (4-byte aligned).  q, k, v, wq, wk, bq, bk as for
 * rehyat_forward_parallel.  REHYAT_EINVAL when the teacher's single window would exceed
 * 2^28 tokens; REHYAT_EWORKSPACE when ws is smaller than rehyat_distill_workspace_bytes or
 * not 256-byte aligned.  The two outputs are left in ws (student first, then teacher,
 * float32 [B,H,N,D] each, at offset 0 and at the student's size rounded up to 256 bytes). */
size_t rehyat_distill_workspace_bytes(const rehyat_params* p);
rehyat_status rehyat_distill_loss(const rehyat_params* p, const void* q, const void* k,
                                  const void* v, const void* wq, const void* wk,
                                  const float* bq, const float* bk, float* loss, void* ws,
                                  size_t ws_bytes, hipStream_t stream);

/* Gradients of the summed distillation objective L = sum_{b,h} loss[b*H + h] (as
 * rehyat_distill_loss) with respect to the feature-map parameters, the only parameters the
 * distillation stage trains (blog 3.1.1).  By the chain rule through the joint
 * normalisation (blog 2.2.1), the recurrent states (blog 2.3) and the feature map (blog
 * 2.2.2): with g_i = 2 (o_i - t_i), a_i = g_i / den_i and h_i = (g_i . o_i) / den_i,
 *   dL/dphi_q(q_i) = S_c a_i - h_i Z_c for the state S_c, Z_c of the query's chunk,
 *   dL/dphi_k(k_j) = R v_j - r with R, r the sums of phi_q a^T and phi_q h over the
 *                    queries of every chunk whose linear region holds k_j,
 *   dL/dpre = sigmoid(pre) sum_p p u^(p-1) dL/dphi_(j,p) with u = softplus(pre), and
 *   dL/dW = sum over tokens (and batches) of dL/dpre x^T, dL/db = sum of dL/dpre.
 * Outputs (device float32, 4-byte aligned): loss [B*H] as rehyat_distill_loss, dwq and dwk
 * [H,Dphi,D], dbq and dbk [H,Dphi] (each of the two may be NULL).  All sums run in a fixed
 * order (bitwise reproducible).  Inputs as for rehyat_forward_parallel; p->out_dtype is
 * ignored.  Status: as rehyat_distill_loss, plus REHYAT_EINVAL when a launch grid would
 * exceed 65,535 row tiles (about 2M tokens) or B*H*chunks exceeds 65,535.  The workspace
 * holds the student and teacher outputs and float32 [B,H,N,*] gradient buffers (about
 * 1.4 GB for bf16 inputs, 1.8 GB for float32 inputs, at a 12-head, 32,760-token layer). */
size_t rehyat_distill_grad_workspace_bytes(const rehyat_params* p);
rehyat_status rehyat_distill_grad(const rehyat_params* p, const void* q, const void* k,
                                  const void* v, const void* wq, const void* wk,
                                  const float* bq, const float* bk, float* loss, float* dwq,
                                  float* dwk, float* dbq, float* dbk, void* ws, size_t ws_bytes,
                                  hipStream_t stream);

/* Backward of the chunk-parallel forward for an upstream gradient dout = dL/dout (float32
 * [B,H,N,D]): dq, dk, dv (float32 [B,H,N,D]), dwq, dwk (float32 [H,Dphi,D]) and dbq, dbk
 * (float32 [H,Dphi], each may be NULL).  The forward is recomputed (float output and the
 * per-part outputs lse, z); with w_ij the weight of key j in query i (exp(q.k/sqrt(D)) in
 * the softmax window, kappa_ij in the linear region, blog 2.2.1), a_i = dout_i / den_i and
 * h_i = (dout_i . o_i) / den_i:
 *   dv_j  = sum_i w_ij a_i;
 *   softmax window: dS_ij = (w_ij / den_i) (dout_i . v_j - dout_i . o_i) / sqrt(D),
 *                   dq_i += sum_j dS_ij k_j, dk_j += sum_i dS_ij q_i (per chunk window);
 *   linear region: as rehyat_distill_grad through the chunk states (blog 2.3), plus
 *                  dq += dpre_q W_q and dk += dpre_k W_k through the feature map.
 * Every sum runs in a fixed order (bitwise reproducible).  bf16 inputs: the softmax branch
 * runs flash style (P and dS recomputed tile by tile from the saved log-denominator and
 * delta, dK / dV in a key-stationary pass and dQ in a query-stationary one), so beyond the
 * gradient buffers of rehyat_distill_grad the workspace holds only per-token statistics and
 * the upstream gradient in bf16: it grows with the clip, not with the window.  float32
 * inputs take the softmax branch one chunk window at a time through two float32
 * [B*H, Tc*n, (Tc+To)*n] score-sized buffers.  Inputs as for rehyat_forward_parallel;
 * p->out_dtype is ignored.  Status: REHYAT_EALIGN for null or misaligned pointers (dout,
 * dq, dk, dv 16-byte aligned), REHYAT_EWORKSPACE, REHYAT_EINVAL as for rehyat_distill_grad. */
size_t rehyat_backward_workspace_bytes(const rehyat_params* p);
rehyat_status rehyat_backward(const rehyat_params* p, const void* q, const void* k, const void* v,
                              const void* wq, const void* wk, const float* bq, const float* bk,
                              const float* dout, float* dq, float* dk, float* dv, float* dwq,
                              float* dwk, float* dbq, float* dbk, void* ws, size_t ws_bytes,
                              hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* REHYAT_H */
