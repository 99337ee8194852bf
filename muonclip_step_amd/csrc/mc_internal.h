// Internal declarations shared by the HIP kernels and the host dispatcher of
// the MuonClip library. Not installed; the public surface is include/muonclip.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mc {

// Compute units of the current HIP device (cached per device; 256 when no
// device answers). Tile sizes, split-K counts and the wave layout of the
// Newton-Schulz products are planned against it.
int device_cus();

// ---------------------------------------------------------------- bf16 bits

// fp32 -> bf16 with round-to-nearest-even: gfx950's v_cvt_pk_bf16_f32 (NaN
// stays a quiet NaN). Device code only.
typedef __bf16 mc_bf16x2_t __attribute__((ext_vector_type(2)));
typedef float mc_f32x2_t __attribute__((ext_vector_type(2)));
__device__ inline uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}
// two values packed into one dword, a in the low half
__device__ inline uint32_t f32x2_to_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((mc_f32x2_t){a, b}, mc_bf16x2_t));
}
__host__ __device__ inline float bf16_to_f32(uint16_t h) {
  return __builtin_bit_cast(float, (uint32_t)h << 16);
}

// ---------------------------------------------------------------- NS GEMM

// One K segment of C = sum_s A_s B_s: A bf16 row-major [M][K]; B bf16 either
// [N][K] ("NT", the Gram and Poly products) or [K][N] (the apply).
constexpr int kGemmBK = 64;   // k per pipeline stage of the NS GEMM

struct GemmSeg {
  const uint16_t* a;
  const uint16_t* b;
  int32_t ktiles;       // K_s / kGemmBK
};

// Epilogue: v = alpha * scale[b]^pow * acc + beta * (cin_hi + cin_lo)[i][j]
// + diag * (i==j), then any of: bf16 store (hi), bf16 residual store
// (lo = v - hi). cin is a bf16 hi + lo pair (about 16 significant bits), or
// cin_hi alone when cin_lo is NULL. Every pointer is the batch-0 base; bs_* are the
// per-batch strides in elements.
struct GemmEpi {
  float alpha;
  int32_t scale_pow;
  const float* scale;
  float beta;
  const uint16_t* cin_hi; const uint16_t* cin_lo; int32_t ld_cin; int64_t bs_cin;
  float diag;
  uint16_t* out_hi; int32_t ld_hi; int64_t bs_hi;
  uint16_t* out_lo; int32_t ld_lo; int64_t bs_lo;
  // bf16(v), rounded as the out_hi store rounds it, in MFMA fragment order,
  // for a later epilogue whose tiles cover the same 32x32 blocks: register
  // r = 4g+q of lane l of block (bi, bj) of batch b sits at
  // (((bi * frag_nb + bj) * 2 + r / 8) * 64 + l) * 8 + r % 8 + b * bs_frag,
  // so each 16-byte access of a wave covers 1 KB. frag_out: written (the
  // Gram); frag_in: read as the beta term instead of cin (the Poly).
  uint16_t* frag_out; const uint16_t* frag_in; int32_t frag_nb; int64_t bs_frag;
  // unsplit apply only: out = bf16(bf16(v) + xadd_coef * scale * xadd[i][j]),
  // xadd a bf16 matrix laid out like the output (the identity part of the
  // Gram-space head's Q, added to R X0 at full precision)
  const uint16_t* xadd; int32_t ld_xadd; int64_t bs_xadd; float xadd_coef;
};

struct GemmArgs {
  int32_t M, N, batch;
  int32_t lda, ldb;
  int64_t bsa, bsb;
  int32_t nseg;
  GemmSeg seg[3];
  int32_t ktiles;        // total over segments
  int32_t splits;        // split-K count (>= 1)
  int32_t kt_per_split;
  float* partial;        // [splits][batch][M][N] fp32 when splits > 1
  int32_t tiles_m, tiles_n;
  GemmEpi epi;
};

enum GemmTile { TILE_256 = 0, TILE_128 = 1, TILE_64 = 2 };
// which Newton-Schulz product a launch computes; fixes the epilogue:
//   GRAM  A = s^2 X X^T      -> bf16 A_hi + A_lo           (symmetric tiles)
//         (also L R of two symmetric m x m matrices, R read by rows, to bf16
//         C alone or to C_hi + its bf16 fragment-order copy)
//   POLY  P = a I + b A + c A A -> bf16 P_hi (+ P_lo)        (symmetric tiles)
//   APPLY X' = s P X          -> bf16 X' (B = X read as [k][n])
enum GemmKind { GEMM_GRAM = 0, GEMM_POLY = 1, GEMM_APPLY = 2 };
int gemm_tile_dim(GemmTile t);
// workgroups per matrix and split (symmetric products count upper tiles only)
int gemm_tile_count(const GemmArgs& a, GemmKind kind);
// split_pair: the product's result is also stored as a residual bf16 (lo) part
struct FusedUpd;
// upd (Apply only, may be NULL): the product is the step's last X' = O and
// the epilogue applies the update to the weights instead of storing O
hipError_t launch_ns_gemm(GemmTile tile, GemmKind kind, bool split_pair, const GemmArgs& a, hipStream_t s,
                          const FusedUpd* upd = nullptr);
hipError_t launch_splitk_reduce(const GemmArgs& a, hipStream_t s);

// ---------------------------------------------------------------- elementwise

constexpr int kMaxBatchMats = 8;   // matrices per separate update launch (its tables carry clip rules)

// momentum update + sum of squares + bf16 copy in one orientation
struct MomMat {
  const void* g; float* m;
  int64_t ld;
  int32_t rows, cols, g_bf16, vec;
  uint16_t* x_orig; int32_t ld_orig;   // [rp][cp], the stored orientation, or NULL
  uint16_t* x_tr;   int32_t ld_tr;     // [cp][rp], or NULL
  int32_t rp, cp;                      // padded extents, multiples of 64
  int32_t tiles_c;                     // cp / 64
  int32_t block_start;
  float* partial;                      // one fp32 per block of this matrix
};
// nesterov: the norm and the bf16 copies are of G + mu M_t instead of M_t
// matrices per momentum launch: 32 tables of ~96 bytes stay well inside the
// kernel-argument limit, and fewer, larger launches stream HBM better (1155
// experts: 41.1 -> 39.7 ms per step over 8-matrix launches)
constexpr int kMaxMomMats = 32;
struct MomArgs { int32_t nmat; float mu; int32_t nesterov; int32_t total_blocks; MomMat mat[kMaxMomMats]; };
hipError_t launch_momentum(const MomArgs& a, hipStream_t s);

// sum of per-block partials -> scale = 1 / (sqrt(sum) + eps), one matrix per block
hipError_t launch_norm_finalize(const float* partial, int32_t parts_per_mat, int64_t partial_stride,
                                float* scale, int32_t nmat, float eps, hipStream_t s);

struct ClipRule {
  int32_t slot, period, nseg;
  int32_t off[2], len[2];
  float expo[2];
};

// QK-Clip factors (device): gamma_h = min(1, tau / S_max^h), 1 when S_max^h
// is not > 0 (S <= 0 or NaN); a row's scale is gamma of its head raised to
// the exponent of the segment holding the row (1 outside every segment).
__device__ inline float gamma_of(float s, float tau) {
  // 1 when S is not > 0 (covers S <= 0 and NaN); tau/inf = 0 zeroes the head
  return s > 0.0f ? fminf(1.0f, tau / s) : 1.0f;
}

// S_max that sets head h's gamma: its own, or with clip_global the largest
// of its layer's heads (fmaxf ignores NaN heads; all NaN gives -inf -> gamma 1)
__device__ inline float layer_s(const float* s_max, int slot, int h, int heads, int clip_global) {
  if (!clip_global) return s_max[slot * heads + h];
  float m = -INFINITY;
  for (int k = 0; k < heads; ++k) m = fmaxf(m, s_max[slot * heads + k]);
  return m;
}

__device__ inline float row_clip_scale(const ClipRule& c, int row, const float* s_max, int heads, float tau,
                                       int clip_global) {
  if (c.slot < 0 || !s_max || c.nseg == 0) return 1.0f;
  const int h = row / c.period, o = row - h * c.period;
  float expo = 0.0f;
  if (c.nseg > 0 && o >= c.off[0] && o < c.off[0] + c.len[0]) expo = c.expo[0];
  else if (c.nseg > 1 && o >= c.off[1] && o < c.off[1] + c.len[1]) expo = c.expo[1];
  if (expo == 0.0f) return 1.0f;
  const float g = gamma_of(layer_s(s_max, c.slot, h, heads, clip_global), tau);
  if (expo == 0.5f) return sqrtf(g);
  if (expo == 1.0f) return g;
  return powf(g, expo);
}

// W <- clip_row * ((1 - lr wd) W - lr * rms * O)
struct UpdMat {
  void* w; int32_t w_bf16, vec;
  int32_t vec8;                        // bf16 W, O and o_out rows of 16-byte aligned 8-element vectors
  int64_t ld;
  int32_t rows, cols;
  const uint16_t* o; int32_t ld_o;
  int32_t o_trans;                     // O is stored transposed: element (r, c) at o[c * ld_o + r]
  uint16_t* o_out;                     // optional copy of O, [rows][cols] contiguous
  float lr_rms;
  ClipRule clip;
  int32_t tiles_c, block_start;
};
// The update fused into the last Newton-Schulz apply: batch entry b is the
// weight W_b (bf16, row-major, ld[b]) whose O is that entry's product,
// stored as W's shape (trans = 0: O is [m][n] = [rows][cols]) or transposed
// (trans = 1: O is [m][n] = [cols][rows]). m, n are the unpadded extents; W's
// columns are a multiple of 8 and its rows 16-byte aligned. Entries below
// nclip carry their clip rule, the rest are never clipped. Block 0 also
// writes gamma [gamma_slots][heads] when gamma_out is set.
constexpr int kMaxFusedMats = 64, kMaxFusedClip = 8;
struct FusedUpd {
  int32_t n;                           // batch entries (0: not fused)
  int32_t m, nn;                       // unpadded NS extents
  float decay, lr_rms;
  const float* s_max; int32_t heads; float tau; int32_t clip_global;
  float* gamma_out; int32_t gamma_slots;
  int32_t nclip;
  ClipRule clip[kMaxFusedClip];
  int32_t ld[kMaxFusedMats];
  int32_t trans[kMaxFusedMats];
  void* w[kMaxFusedMats];
};

// clip_global: gamma of a layer from the largest S_max of its heads
struct UpdArgs {
  int32_t nmat; int32_t total_blocks;
  float decay;
  const float* s_max; int32_t heads; float tau; int32_t clip_global;
  float* gamma_out; int32_t gamma_slots;   // block 0 also writes gamma [slots][heads] when set
  UpdMat mat[kMaxBatchMats];
};
hipError_t launch_update(const UpdArgs& a, hipStream_t s);

// gamma for [slots][heads]; clip_global: one value per slot from its largest S_max
hipError_t launch_gamma(const float* s_max, float* gamma, int32_t slots, int32_t heads, float tau,
                        int32_t clip_global, hipStream_t s);

struct ClipApplyArgs {
  void* w; int32_t w_bf16;
  int64_t ld;
  int32_t rows, cols;
  ClipRule clip;
  const float* s_max; int32_t heads; float tau;
};
// one matrix, whatever its alignment (element accesses when it has to)
hipError_t launch_clip_apply(const ClipApplyArgs& a, hipStream_t s);
// Up to kMaxClipBatch matrices whose rows are whole 16-byte vectors (cols a
// multiple of 8 bf16 / 4 fp32, 16-byte aligned base and row stride) in one
// launch: their rows are numbered one matrix after another.
constexpr int kMaxClipBatch = 8;
struct ClipVecMat {
  char* w; int64_t ld_bytes;
  int32_t w_bf16, vpr;                 // 16-byte vectors per row
  int32_t rows;
  int64_t row_start;                   // first row of this matrix in the joint numbering
  ClipRule clip;
};
struct ClipVecArgs {
  int32_t nmat; int64_t total_rows;
  const float* s_max; int32_t heads; float tau;
  ClipVecMat mat[kMaxClipBatch];
};
bool clip_apply_vectorizable(const ClipApplyArgs& a);
hipError_t launch_clip_apply_vec(const ClipVecArgs& a, hipStream_t s);

// ---------------------------------------------------------------- AdamW

constexpr int kMaxBatchVecs = 16;
struct AdamVec {
  void* p; const void* g; float* m; float* v;
  int64_t n;
  int32_t p_bf16, g_bf16, vec;         // vec: 16-byte fp32 / 8-byte bf16 accesses allowed
  int32_t block_start;
};
// decay = 1 - lr wd, c1 = 1 / (1 - beta1^t), c2 = 1 / (1 - beta2^t)
struct AdamArgs {
  int32_t nvec, total_blocks;
  float lr, beta1, beta2, one_m_beta1, one_m_beta2, eps, decay, c1, c2;
  AdamVec vec[kMaxBatchVecs];
};
int64_t adamw_blocks(int64_t n);   // blocks one vector of n elements needs
hipError_t launch_adamw(const AdamArgs& a, hipStream_t s);

// ---------------------------------------------------------------- max logits

struct MaxLogitArgs {
  const void* q; const void* k; const void* ks;
  int64_t qs_b, qs_t, qs_h;
  int64_t ks_b, ks_t, ks_h;
  int64_t kss_b, kss_t;
  int32_t B, T, H, d_q, d_k, d_s;
  int32_t causal, bf16;
  float* out;            // [H] running max of the scaled logits (set to -inf first)
  float scale;           // applied to each block's max before it is merged
};
// true when the MFMA kernel covers this shape (bf16, d_k and d_s supported,
// 16-byte aligned rows); otherwise the generic kernel runs.
bool max_logits_mfma_supported(const MaxLogitArgs& a);
hipError_t launch_max_logits_init(float* out, int32_t H, hipStream_t s);   // out[h] = -inf
hipError_t launch_max_logits(const MaxLogitArgs& a, hipStream_t s, bool* used_mfma);

// Running maximum of floats in global memory by one integer atomic: a
// non-negative float orders like its bits as a signed integer, a negative
// one inversely to its bits as an unsigned integer, so atomicMax on the
// first and atomicMin on the second keep the larger float whatever the
// current value (initially -inf). NaN is ignored; -0 counts as +0.
__device__ inline void atomic_max_f32(float* p, float v) {
  if (v != v) return;
  if (v == 0.0f) v = 0.0f;
  if (v > 0.0f || __float_as_uint(v) == 0u) atomicMax((int*)p, __float_as_int(v));
  else atomicMin((unsigned int*)p, __float_as_uint(v));
}

// ---------------------------------------------------------------- attention forward

// Softmax attention of one layer (bf16 in and out), with the per-head max
// logit taken from the same pass when smax is set. Element strides; the
// last dimension of every tensor is contiguous.
struct AttnArgs {
  const void* q; const void* k; const void* ks; const void* v;
  void* o;
  float* lse;            // [B][H][T] natural-log sum of exp(scaled logits), or NULL
  float* smax;           // [H] running max of the scaled logits (-inf first), or NULL
  int64_t qs_b, qs_t, qs_h;
  int64_t ks_b, ks_t, ks_h;
  int64_t kss_b, kss_t;
  int64_t vs_b, vs_t, vs_h;
  int64_t os_b, os_t, os_h;
  int32_t B, T, H, d_k, d_s, d_v;
  int32_t causal;
  float scale;           // softmax scale (1/sqrt(d) normally)
};
// true when the kernel covers (d_k, d_s, d_v) and the alignments
bool attention_supported(const AttnArgs& a);
hipError_t launch_attention(const AttnArgs& a, hipStream_t s);
// S_max alone through the attention kernel's logit pass (d_k 128, d_s 64;
// v, o and lse unused; q, k, ks 16-byte aligned rows)
hipError_t launch_attention_smax_only(const AttnArgs& a, hipStream_t s);

}  // namespace mc
