/*
 * muonclip.h — C ABI of the MI355X (gfx950) MuonClip optimizer-step library.
 *
 * One MuonClip step (Kimi K2 report, "MuonClip" paragraphs; the K2 report
 * translation, section 2.1 "MuonClip: stable training by weight clipping")
 * is, for every 2-D parameter W with gradient G and momentum M:
 *
 *   M  <- mu M + G                                  (Notes on Moonlight, "Background")
 *   O  <- NewtonSchulz5(M)                          (Notes on Muon blog, "Newton-Schulz",
 *                                                    "Algorithm": X0 = M/(||M||_F + eps),
 *                                                    iterate on X^T when rows > cols,
 *                                                    X <- aX + (bA + cA^2)X, A = X X^T)
 *   W  <- W - lr (rms_scale sqrt(max(rows, cols)) O + weight_decay W)
 *                                                   (Notes on Moonlight, "Scaling up Muon")
 *   then, for the query/key projections of an attention layer, the post-update
 *   per-head QK-Clip (Kimi K2 essay, section on Muon and attention logits):
 *   gamma_h = min(1, tau / S_max^h), S_max^h = (1/sqrt(d)) max_{X in batch}
 *   max_{i,j} Q_i^h . K_j^h from this step's forward; MHA scales the head's
 *   rows of W_q and W_k by sqrt(gamma_h); MLA (essay, MLA table) scales q^C
 *   and k^C rows by sqrt(gamma_h), q^R rows by gamma_h and leaves the shared
 *   k^R untouched.
 *
 * Conventions for every entry point:
 *   - Pointers are device pointers (HBM of the current HIP device) unless the
 *     comment says (host).
 *   - Matrices are row-major: element (r, c) at base + r*ld + c, ld in elements.
 *   - `stream` is a hipStream_t (NULL = the default stream). Calls only enqueue
 *     work on it and return; nothing is synchronised, no device->host copy is
 *     made, and no device memory is allocated: the caller owns every buffer,
 *     including the workspace. The only state kept between calls is, per
 *     device, one auxiliary stream and two events (created on first use,
 *     kept until the process ends) that muonclip_step forks from and joins
 *     back into `stream` to run two independent chains at once.
 *   - Every argument is validated before the first launch; on an error status
 *     nothing has been enqueued and nothing is modified. mc_last_error()
 *     returns a text for the last non-OK status of the calling thread.
 *   - HIP launch failures return MC_ERR_HIP. Device faults surface at the
 *     caller's next synchronisation. NaN/Inf in G, M or W propagate unchecked.
 *   - Two calls that share output buffers or a workspace must be ordered by
 *     the caller (same stream or events).
 */
#ifndef MUONCLIP_H
#define MUONCLIP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t mc_status;
enum {
  MC_OK = 0,
  MC_ERR_NULL = 1,       /* a required pointer is NULL */
  MC_ERR_SHAPE = 2,      /* sizes, strides or clip layout inconsistent */
  MC_ERR_DTYPE = 3,      /* unsupported dtype code */
  MC_ERR_WORKSPACE = 4,  /* workspace NULL, misaligned or too small */
  MC_ERR_HPARAM = 5,     /* hyper-parameter out of range */
  MC_ERR_HIP = 6,        /* a HIP runtime call or launch failed */
  MC_ERR_ALIGN = 7       /* pointer alignment below what the dtype needs */
};

enum { MC_F32 = 0, MC_BF16 = 1 };

/* One row segment of a head's block of rows: rows [h*period + offset,
 * h*period + offset + length) of head h are scaled by gamma_h ** expo.
 * expo 0.5 = sqrt(gamma) (MHA W_q/W_k, MLA q^C and k^C), 1.0 = gamma (MLA q^R). */
typedef struct {
  int32_t offset;
  int32_t length;
  float expo;
} mc_segment;

/* One 2-D Muon parameter. W, G and M share rows, cols and ld. rows and cols
 * are at most 2^20 and, each rounded up to 64, multiply to less than 2^31
 * elements (else MC_ERR_SHAPE).
 *   w        param, w_dtype (MC_F32 or MC_BF16), updated in place
 *   g        gradient, g_dtype (MC_F32 or MC_BF16), read only
 *   m        fp32 momentum, updated in place (M_0 = 0 is a zero buffer)
 *   o_out    optional bf16 [rows][cols] contiguous buffer that receives the
 *            Newton-Schulz output O of this step (NULL = not written)
 *   clip_slot  attention layer index: row `clip_slot` of s_max[slots][heads];
 *            -1 = the matrix is never clipped
 *   period, nseg, seg  head h owns rows [h*period, (h+1)*period); requires
 *            rows % period == 0 and rows/period <= heads. MHA W_q/W_k: period
 *            d_head, one segment {0, d_head, 0.5}. MLA q_b (rows per head
 *            [q^C 128 | q^R 64]): period 192, {0,128,0.5},{128,64,1.0}. MLA
 *            kv_b (rows per head [k^C 128 | v 128]): period 256, {0,128,0.5}.
 *            kv_a (holding k^R) and every other matrix: clip_slot -1.        */
typedef struct {
  void *w;
  const void *g;
  float *m;
  void *o_out;
  int64_t rows, cols, ld;
  int32_t w_dtype, g_dtype;
  int32_t clip_slot;
  int32_t period;
  int32_t nseg;
  mc_segment seg[2];
} mc_matrix;

/* Hyper-parameters (fp32). Defaults from mc_default_hparams: lr 2e-4,
 * mu 0.95, weight_decay 0.1, rms_scale 0.2, tau 100, Newton-Schulz
 * (a, b, c) = (3.4445, -4.7750, 2.0315), eps 1e-7, 5 steps, plain momentum,
 * per-head clip.
 *   nesterov     0: Newton-Schulz orthogonalises the momentum M_t (Notes on
 *                Moonlight, "Background"); 1: it orthogonalises the look-ahead
 *                G_t + mu M_t (Nesterov-style momentum, Notes on Muon blog,
 *                "Analysis"). The stored momentum is M_t either way.
 *   clip_global  0: per-head gamma_h = min(1, tau / S_max^h) (K2 report 2.1);
 *                1: the report's naive variant, one gamma = min(1, tau / max_h
 *                S_max^h) for every head of a layer (slot); the segment
 *                exponents then carry the balance alpha (W_q alpha, W_k
 *                1 - alpha; alpha = 0.5 gives 0.5 on both). gamma_out receives
 *                that gamma for every head. NaN heads are ignored by the max. */
typedef struct {
  float lr, mu, weight_decay, rms_scale, tau;
  float ns_a, ns_b, ns_c, ns_eps;
  int32_t ns_steps;   /* 1..16 */
  int32_t nesterov;   /* 0 or 1 */
  int32_t clip_global;/* 0 or 1 */
} mc_hparams;

/* (host) Fill *hp with the defaults above. */
void mc_default_hparams(mc_hparams *hp);

/* (host) Workspace bytes muonclip_step needs to run every shape group of
 * `mats` with up to 64 matrices in flight at once, twice over when the step
 * has more than one shape group, so that two groups can run concurrently
 * (larger buffers are not used; smaller ones down to mc_workspace_min_size
 * work in more waves, on one stream).
 * Returns 0 on invalid arguments (see mc_last_error). */
size_t mc_workspace_size(const mc_matrix *mats /* host, n */, int32_t n, const mc_hparams *hp /* host */);
/* (host) The smallest workspace muonclip_step accepts for these matrices
 * (one matrix of the largest shape group in flight). */
size_t mc_workspace_min_size(const mc_matrix *mats /* host, n */, int32_t n, const mc_hparams *hp /* host */);

/* One MuonClip step over n matrices (host array `mats`): Algorithm 1 of the
 * K2 report (only its caption survives in the report translation, section 2.1
 * "MuonClip: stable training by weight clipping"), assembled from the Muon
 * update paragraph of the K2 report (the 0.2 sqrt(max(rows, cols)) RMS
 * factor), Notes on Moonlight "Background" (M <- mu M + G) and "Scaling up
 * Muon" (decoupled decay W <- W - lr (U + weight_decay W)), Notes on Muon blog
 * "Algorithm" (five quintic Newton-Schulz steps) and the essay's per-head
 * clip applied to the updated weights.
 *   s_max      fp32 [slots][heads] per-head max logits of this step's forward
 *              (max_logits_per_head); NULL = no QK-Clip this step
 *   gamma_out  optional fp32 [slots][heads] receiving gamma = min(1, tau/S)
 *              (1 where S is not > 0); NULL = not written
 *   workspace  device buffer of workspace_bytes >= mc_workspace_min_size,
 *              256-byte aligned; its contents need no initialisation
 * Matrices are processed in groups of equal (min, max) shape; within a group
 * the momentum kernel, five Newton-Schulz iterations (bf16 MFMA, fp32
 * accumulation) and the fused update/decay/clip kernel run per wave of
 * matrices that fit the workspace. For groups with max >= 2 min the first
 * three iterations are formed in the min x min Gram space (A_{j+1} = P_j A_j
 * P_j, then one product with X0), which gives the same iterate in exact
 * arithmetic with fewer max-sized products; results therefore match the
 * iteration to bf16 rounding, not bit for bit. Waves are independent chains: with at
 * least two shape groups and a workspace that holds a wave of each twice
 * over, the chains are split between `stream` and the library's auxiliary
 * stream, which is forked after the work already on `stream` and joined back
 * before the call's work counts as done on `stream`. Results are identical
 * either way. */
mc_status muonclip_step(const mc_matrix *mats /* host, n */, int32_t n, const mc_hparams *hp /* host */,
                        const float *s_max, int32_t slots, int32_t heads, float *gamma_out,
                        void *workspace, size_t workspace_bytes, void *stream);

/* muonclip_step with S_max still being computed on another stream (the step
 * of Kimi K2 report 2.1 needs S_max only for the QK-Clip that follows the
 * update, so the S_max pass can run beside momentum and Newton-Schulz).
 *   s_max_ready  a hipEvent_t the caller recorded, before this call, after the
 *                launch that writes s_max (e.g. max_logits_per_head on a
 *                second stream); NULL = exactly muonclip_step
 * Every launch of the step that reads s_max (the update, or the last
 * Newton-Schulz product when the update rides on it, and the gamma launch
 * when n == 0) first makes its stream wait on the event; the launches before
 * it do not. Arguments, errors and results are those of muonclip_step, bit
 * for bit. The event is not recorded, reset or destroyed here. */
mc_status muonclip_step_overlapped(const mc_matrix *mats /* host, n */, int32_t n, const mc_hparams *hp /* host */,
                                   const float *s_max, int32_t slots, int32_t heads, float *gamma_out,
                                   void *workspace, size_t workspace_bytes, void *stream, void *s_max_ready);

/* muonclip_step for callers that cannot allocate (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * arguments without the workspace, which is a static device array of
 * MC_NOALLOC_SCRATCH_BYTES inside the library instead (one per device, held
 * until the process ends). The call allocates nothing and creates nothing:
 * all work runs on `stream` (no auxiliary lane). Matrices whose smallest
 * workspace (mc_workspace_min_size) exceeds the scratch are rejected with
 * MC_ERR_WORKSPACE before anything is enqueued; within it, waves are as
 * large as the scratch allows. Results equal muonclip_step's with a
 * workspace of MC_NOALLOC_SCRATCH_BYTES on one stream. Every call on a
 * device shares that device's scratch: two calls that overlap on one device
 * (different streams, no ordering) race and give undefined results. */
#define MC_NOALLOC_SCRATCH_BYTES (256u << 20)
mc_status muonclip_step_noalloc(const mc_matrix *mats /* host, n */, int32_t n, const mc_hparams *hp /* host */,
                                const float *s_max, int32_t slots, int32_t heads, float *gamma_out, void *stream);

/* Per-head max attention logit of one attention layer's forward (the essay's
 * S_max^h equation, section on Muon and attention logits: the largest
 * Q_i^h . K_j^h / sqrt(d) over the batch and over token pairs; the report
 * translation, section 2.1, defines the same quantity per head):
 *   s_max_out[h] = scale * max over b < B, i < T, j < T (j <= i if causal) of
 *     q[b,i,h,0:d_k] . k[b,j,h,:] + q[b,i,h,d_k:d_q] . k_shared[b,j,:]
 * q: [B,T,H,d_q] with element strides q_stride = {b, t, h} (last dim
 * contiguous); k: [B,T,H,d_k] with k_stride {b, t, h}; k_shared: [B,T,d_shared]
 * with ks_stride {b, t}, NULL when d_shared == 0 (MHA). Requires d_q ==
 * d_k + d_shared. dtype MC_BF16 or MC_F32 for all three. scale is normally
 * 1/sqrt(d_q) (MHA: d_head; MLA: 128 + 64). NaN logits are ignored; a head
 * with no pair gets -inf. s_max_out (fp32 [H]) is overwritten; it is also
 * used as the reduction buffer while the call runs. The MFMA kernel serves
 * bf16 with (d_k, d_shared) in {(128,0), (128,64), (64,0)}, 16-byte aligned
 * rows and strides that are multiples of 8; other inputs run a generic
 * fp32-dot kernel. */
mc_status max_logits_per_head(const void *q, const void *k, const void *k_shared, int32_t dtype,
                              int32_t B, int32_t T, int32_t H,
                              int32_t d_q, int32_t d_k, int32_t d_shared,
                              const int64_t *q_stride /* host [3] */, const int64_t *k_stride /* host [3] */,
                              const int64_t *ks_stride /* host [2], or NULL */,
                              int32_t causal, float scale, float *s_max_out, void *stream);

/* Softmax attention forward of one layer with S_max observed on the way
 * (Kimi K2 report, "Taming Muon with QK-Clip": O^h = softmax(Q^h K^h^T /
 * sqrt(d)) V^h, and S_max^h is the largest softmax input of that same
 * forward; K2 report 2.1 in translation, the same equations). For every
 * sample b, head h and query i:
 *   o[b,i,h,:] = sum_j w_j v[b,j,h,:],  w = softmax_j(scale * logit(b,i,j,h))
 * over keys j < T (j <= i if causal), logit as in max_logits_per_head (q, k
 * and k_shared have the same shapes and strides as there). bf16 in and out,
 * fp32 arithmetic (probabilities rounded to bf16 for the value product).
 *   v: [B,T,H,d_v] with v_stride {b, t, h}; o: [B,T,H,d_v] with o_stride,
 *      written; it must not overlap any input
 *   lse: optional fp32 [B][H][T] (contiguous), the natural log of the row's
 *      sum of exp(scale * logit); NULL = not written
 *   s_max_out: optional fp32 [H], overwritten with the value
 *      max_logits_per_head gives for the same q, k, k_shared, taken from the
 *      softmax's running row maxima (no second Q K^T pass); -inf for every
 *      head when B or T is 0; NULL = not computed
 * Covers (d_k, d_shared, d_v) in {(128, 0, 128), (128, 64, 128)} with d_q =
 * d_k + d_shared (MHA d = 128; MLA [q^C | q^R] against [k^C_h | k^R]).
 * q, k, k_shared, v, o 16-byte aligned, every stride a multiple of 8 elements
 * and t strides of k, k_shared, v below 2^23 elements; otherwise MC_ERR_SHAPE
 * or MC_ERR_ALIGN before anything is enqueued. scale finite and > 0. One
 * launch (plus two tiny ones for s_max_out) on `stream`; allocates nothing. */
mc_status attention_forward(const void *q, const void *k, const void *k_shared, const void *v, void *o,
                            float *lse, float *s_max_out,
                            int32_t B, int32_t T, int32_t H, int32_t d_q, int32_t d_k, int32_t d_shared,
                            int32_t d_v, const int64_t *q_stride /* host [3] */,
                            const int64_t *k_stride /* host [3] */, const int64_t *ks_stride /* host [2], or NULL */,
                            const int64_t *v_stride /* host [3] */, const int64_t *o_stride /* host [3] */,
                            int32_t causal, float scale, void *stream);

/* QK-Clip alone on existing weights (the clip part of muonclip_step without
 * the Muon update). gamma_h = min(1, tau / S_max^h) as in the essay's gamma
 * equation, with the guard of its MHA code sample (1 when S_max^h is not
 * positive); MHA rows of W_q and W_k scale by sqrt(gamma_h) (the essay's MHA
 * equations), MLA q^C and k^C rows by sqrt(gamma_h), q^R rows by gamma_h and
 * the shared k^R not at all (the essay's MLA table; report translation 2.1).
 * For every matrix with clip_slot >= 0, rows in its
 * segments are scaled by gamma_h ** expo, gamma from s_max[slots][heads] and
 * tau (per head; the all-head variant is muonclip_step's clip_global); rows
 * whose factor is exactly 1 are not touched (bit-identical). Uses w, w_dtype,
 * rows, cols, ld and the clip fields of each matrix.
 * gamma_out: optional fp32 [slots][heads]. */
mc_status qk_clip_apply(const mc_matrix *mats /* host, n */, int32_t n, const float *s_max,
                        int32_t slots, int32_t heads, float tau, float *gamma_out, void *stream);

/* ---- AdamW for the parameters Muon does not cover (Notes on Muon blog,
 * "Limitation": Muon is for 2-D parameters, the rest keep AdamW; Notes on
 * Moonlight, "Scaling up Muon": the two share lr and weight decay). The pages
 * give no AdamW formula; the textbook form with bias correction is used:
 *   m <- b1 m + (1 - b1) g,   v <- b2 v + (1 - b2) g^2,
 *   p <- p - lr ( m / (1 - b1^t) / (sqrt(v / (1 - b2^t)) + eps) + weight_decay p ).
 * One contiguous parameter vector (norm weights, biases, embeddings flattened):
 *   p  param, p_dtype (MC_F32 or MC_BF16), updated in place
 *   g  gradient, g_dtype (MC_F32 or MC_BF16), read only
 *   m, v  fp32 first and second moments, updated in place (zero at t = 1)
 *   n  elements (0 allowed: nothing is touched)                              */
typedef struct {
  void *p;
  const void *g;
  float *m, *v;
  int64_t n;
  int32_t p_dtype, g_dtype;
} mc_vector;

/* lr, weight_decay as for Muon (defaults 2e-4, 0.1); beta1 0.9, beta2 0.95,
 * eps 1e-8 by default (not on the pages); step t >= 1 (1-based). */
typedef struct {
  float lr, beta1, beta2, eps, weight_decay;
  int32_t step;
} mc_adamw_hparams;

/* (host) Fill *hp with the defaults above (step 1). */
void mc_default_adamw_hparams(mc_adamw_hparams *hp);

/* One AdamW step over n vectors (host array). Validates everything before
 * the first launch (NULL pointers, dtypes, alignment of each pointer to its
 * element size, 0 <= beta < 1, eps >= 0, finite values, step >= 1); enqueues
 * one launch per 16 vectors on `stream`; allocates nothing. Vectors must not
 * overlap each other. */
mc_status adamw_step(const mc_vector *vecs /* host, n */, int32_t n, const mc_adamw_hparams *hp /* host */,
                     void *stream);

/* (host) Text of the last non-OK status returned on this thread. */
const char *mc_last_error(void);

/* (host) Library version string. */
const char *mc_version(void);

/* ---- kernel timing (host). While enabled, every launch the library makes is
 * bracketed by a pair of hipEvents on the launch stream, and durations are
 * summed per kernel family; muonclip_step then runs all its chains on the
 * caller's stream (no auxiliary lane), so no two timed launches overlap.
 * Enabling creates events (hipEventCreate) as needed; it is meant for
 * measurement runs, not for capture. */
typedef struct {
  char name[32];
  int32_t launches;
  double ms;        /* summed event time */
  double flops;     /* algorithmic FLOPs of those launches (0 if not a contraction) */
  double bytes;     /* algorithmic HBM bytes of those launches */
} mc_profile_entry;

/* on != 0: start recording (clears previous records); 0: stop. */
mc_status mc_profile_enable(int32_t on);
/* Synchronises the recorded events and writes up to cap entries (one per
 * kernel family); returns the number of families, or -1 on error. */
int32_t mc_profile_read(mc_profile_entry *out /* host, cap */, int32_t cap);

#ifdef __cplusplus
}
#endif

#endif /* MUONCLIP_H */
