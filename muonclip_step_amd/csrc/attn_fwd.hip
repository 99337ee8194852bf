// Softmax attention forward with the per-head max logit observed on the way.
//
// O^h = softmax(scale Q^h K^h^T) V^h per (sample, head) (K2 report, "Taming
// Muon with QK-Clip"; K2 report 2.1 in translation): the max logit S_max^h
// that QK-Clip needs is the largest softmax input of this same forward, so
// the kernel takes it from the running row maxima the online softmax keeps
// anyway, instead of a second Q K^T pass. Causal masking keeps j <= i. MLA
// keys are [k^C_h | k^R] with the rotary key shared by every head; the value
// width is 128.
//
// Layout of the work. A block owns 256 query rows of one (sample, head) in
// eight waves of 32 rows (two waves per SIMD; the logit pass alone: four
// waves of 64 rows, two blocks per CU). Each wave keeps its rows in
// registers as an MFMA B-fragment for the whole kernel and walks the key axis
// in tiles of 64 keys, which pass through a double-buffered LDS ring (K rows
// XOR-swizzled
// for 16-byte fragment reads, V rows swizzled for transposing reads). Both
// products run transposed, with v_mfma_f32_32x32x16_bf16:
//   S^T = K Q^T   (A = K from LDS, B = Q from registers)
//   O^T += V^T P^T (A = V^T via ds_read_b64_tr_b16, B = P^T from registers)
// so that every lane holds one query's logits, probabilities and output
// column: the row max and row sum stay inside a lane pair (lanes l, l^32),
// the rescale is a per-lane scalar, and P^T is the S^T accumulator itself
// converted to bf16 (the MFMA's k order is permuted to match it on both
// operands). The running max used for the exponentials moves only when a
// tile's max exceeds it by more than 96 binary orders (and then moves 32
// orders past the tile max), so the output
// accumulators are rescaled rarely; the exact running max is kept beside it
// for S_max. Blocks are issued heaviest causal row first; the q-tiles of one
// (sample, head) are HB apart in launch order, which keeps them on one XCD
// (and its L2) whenever HB is a multiple of 8.
#include <math.h>

#include <type_traits>
#include <utility>

#include "mc_internal.h"

namespace mc {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16_t lds_v4i16_t;
typedef __attribute__((address_space(3))) void lds_void_t;

// s_waitcnt on the vector-memory counter alone (the direct-to-LDS loads are
// the only vector loads in flight inside the loop)
#define FA_WAIT_DMA() __builtin_amdgcn_s_waitcnt(0x70 | 0xF00)

constexpr int kBQ = 256, kBKV = 64, kDV = 128;

// V rows (256 bytes): a transposing read's 16-lane group covers four
// consecutive rows at the same columns; chunk ^ 4 (r & 3) puts them on
// distinct banks.
__device__ __forceinline__ int v_swz(int r) { return 4 * (r & 3); }

// f(integral_constant<int, I>) for I = 0 .. N-1, unrolled at compile time
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// inline LDS reads with an immediate offset, and waits that name the
// registers they complete (see the kernel)
template <int OFF>
__device__ __forceinline__ void lds_read_b128(u32x4_t& dst, uint32_t addr) {
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(dst) : "v"(addr), "i"(OFF));
}
template <int OFF>
__device__ __forceinline__ void lds_read_tr(v4i16_t& dst, uint32_t addr) {
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(dst) : "v"(addr), "i"(OFF));
}
template <int N>
__device__ __forceinline__ void lgkm_wait(u32x4_t& r) {
  asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(r) : "i"(N));
}
template <int N>
__device__ __forceinline__ void lgkm_wait(v4i16_t (&l)[4], v4i16_t (&h)[4]) {
  asm volatile("s_waitcnt lgkmcnt(%8)"
               : "+v"(l[0]), "+v"(l[1]), "+v"(l[2]), "+v"(l[3]), "+v"(h[0]), "+v"(h[1]), "+v"(h[2]), "+v"(h[3])
               : "i"(N));
}

// S^T = K Q^T k-step as inline MFMAs writing VGPRs (the softmax reads the
// logits with VALU instructions; the compiler's own MFMAs accumulate the
// output). Hazards the compiler cannot see: a VALU write of an operand needs two wait states
// before the MFMA reads it (the leading s_nop 1), and VALU reads of the
// result wait for s_wait_logits below.
__device__ __forceinline__ void mfma_s_first(f32x16_t& acc, const u32x4_t& a, const bf16x8_t& b) {
  asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_s(f32x16_t& acc, const u32x4_t& a, const bf16x8_t& b) {
  asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}
// 24 wait states between the last logit MFMA and the first VALU read of its
// result (more than the 8-pass MFMA's requirement)
__device__ __forceinline__ void s_wait_logits(f32x16_t& a) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(a));
}
// the same after two fragments' chains (the second one's MFMA issues last)
__device__ __forceinline__ void s_wait_logits(f32x16_t& a, f32x16_t& b) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(a), "+v"(b));
}

// max of three numbers ignoring quiet NaNs (IEEE maxNum, as fmaxf), in one
// v_max3_f32 and without the quieting copies the compiler puts before fmaxf
// on MFMA results (the logits are read after s_wait_logits)
__device__ __forceinline__ float max3_nan_ignoring(float a, float b, float c) {
  float r;
  asm volatile("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

__device__ __forceinline__ float wave_max(float x) {
  for (int off = 32; off > 0; off >>= 1) x = fmaxf(x, __shfl_xor(x, off));
  return x;
}

// Eight waves of 32 query rows (one MFMA fragment, NF = 1), two waves per
// SIMD, which hide each other's softmax arithmetic and LDS latency behind
// their MFMAs (the LDS delivers about 200 bytes per clock per CU to two waves
// per SIMD, enough for the fragment traffic). The whole state fits 256
// VGPRs: every MFMA writes VGPRs and the rescale is plain VALU arithmetic.
// OUT = false: the logits and S_max only (no values, softmax or output),
// which serves max_logits_per_head for head width 128 and the MLA head
// shape. It runs four waves of 64 query rows (two fragments, so each K
// fragment read from LDS feeds two MFMAs and a wave has two independent
// accumulation chains) and two blocks per CU, again two waves per SIMD.
template <int DK, int DS, bool SMAX, bool OUT = true>
__global__ void __launch_bounds__(OUT ? 512 : 256, OUT ? 1 : 2) __attribute__((amdgpu_waves_per_eu(2, 2)))
attn_fwd_kernel(const AttnArgs a) {
  static_assert(OUT || SMAX, "a pass with neither output nor S_max");
  static_assert(DK == 128 && (DS == 0 || DS == 64), "head widths");
  constexpr int NF = OUT ? 1 : 2;            // query fragments per wave
  constexpr int NW = OUT ? 8 : 4, WR = 32 * NF;   // waves per block, query rows per wave
  // MLA (192-wide queries): to fit 256 registers a half's K fragments go
  // through a ring of KSL = KS / 2 slots (the second half of the reads is
  // issued under the first half's MFMAs) and the two value k-steps share one
  // fragment buffer (the second is read after the first one's MFMAs issued).
  constexpr bool kLean = DS > 0;
  constexpr int D = DK + DS, KS = D / 16;
  constexpr int KSL = kLean ? KS / 2 : KS, NVB = kLean ? 1 : 2;   // K slots, value buffers
  // one LDS stage: K content rows [64][256 B], rotary rows [64][128 B], V rows [64][256 B]
  // (the logit pass keeps no values: two blocks of four waves share a CU)
  constexpr int KC_BYTES = kBKV * 256, KR_BYTES = kBKV * DS * 2, VT_BYTES = OUT ? kBKV * kDV * 2 : 0;
  constexpr int STAGE = KC_BYTES + KR_BYTES + VT_BYTES;
  // LDS ring stages: each tile's loads go out while the previous tile is
  // computed (a third stage, loading two tiles ahead, measured 3 % slower)
  constexpr int NSTG = 2;
  __shared__ __attribute__((aligned(16))) char lds[NSTG * STAGE];
  __shared__ float red[NW];

  const int HB = a.H * a.B;
  const int nqt = (a.T + kBQ - 1) / kBQ;
  const int hb = blockIdx.x % HB;
  const int qt = nqt - 1 - (int)(blockIdx.x / HB);   // heaviest causal rows first
  const int h = hb % a.H, b = hb / a.H;
  const int q0 = qt * kBQ;
  const int tid = threadIdx.x, lane = tid & 63, hl = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int wq0 = q0 + wave * WR;

  const uint16_t* Q = (const uint16_t*)a.q + (int64_t)b * a.qs_b + (int64_t)h * a.qs_h;
  const char* K = (const char*)((const uint16_t*)a.k + (int64_t)b * a.ks_b + (int64_t)h * a.ks_h);
  const char* KR = DS > 0 ? (const char*)((const uint16_t*)a.ks + (int64_t)b * a.kss_b) : nullptr;
  const char* V = (const char*)((const uint16_t*)a.v + (int64_t)b * a.vs_b + (int64_t)h * a.vs_h);

  // the wave's WR query rows as B fragments: lane l holds query l % 32 of
  // fragment f, dimensions 16 s + 8 (l / 32) .. +7. Rows past T re-read row
  // T - 1: they see exactly row T - 1's keys, so they change no maximum, and
  // their outputs are not stored.
  bf16x8_t qf[NF][KS];
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    const int row = wq0 + 32 * f + (lane & 31);
    const int rr = row < a.T ? row : a.T - 1;
    const uint16_t* base = Q + (int64_t)rr * a.qs_t + 8 * hl;
#pragma unroll
    for (int s = 0; s < KS; ++s) qf[f][s] = __builtin_bit_cast(bf16x8_t, *(const u32x4_t*)(base + 16 * s));
  }

  const int kend = a.causal ? min(a.T, q0 + kBQ) : a.T;
  const int nkv = (kend + kBKV - 1) / kBKV;
  const float c2 = a.scale * 1.4426950408889634f;   // scale * log2(e)
  // lazy-rescale slack in raw logit units: probabilities stay below 2^96,
  // so row sums and output accumulators stay below 2^96 T max|v| (below the
  // fp32 / bf16 limit of 2^128 for T max|v| < 2^32), with the same relative
  // precision
  const float thr = 96.0f / c2;
  // a new reference sits this far above the tile max (the max element's
  // probability is then 2^-32), so the next rescale needs 128 orders of growth
  const float head = 32.0f / c2;

  f32x16_t oacc[NF][4];
#pragma unroll
  for (int f = 0; f < NF; ++f)
#pragma unroll
    for (int n = 0; n < 4; ++n) oacc[f][n] = f32x16_t{};
  float m_use[NF], m_all[NF], lsum[NF];   // reference max, exact running max (S_max), half row sum
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    m_use[f] = -INFINITY;
    m_all[f] = -INFINITY;
    lsum[f] = 0.0f;
  }

  // Tiles reach LDS through direct-to-LDS loads (global_load_lds_dwordx4:
  // 64 lanes fill 1 KB of consecutive LDS, so each swizzle is applied on the
  // source side: the lane filling physical chunk pc of row r fetches logical
  // chunk pc ^ swz(r)). Per wave: 4 instructions of K content rows, 2 of
  // rotary rows (MLA), 4 of V rows; lane offsets are relative to the tile's
  // first key, whose address is the only per-tile arithmetic. Keys past T
  // (only in the tile holding key T - 1) re-read key T - 1 and are masked.
  constexpr int IC = 16 / NW, IR = DS > 0 ? 8 / NW : 0, IV = 16 / NW;
  int crow[IC], coff[IC], vrow[IV], voffs[IV];
  int rrow[IR > 0 ? IR : 1], roff[IR > 0 ? IR : 1];
#pragma unroll
  for (int i = 0; i < IC; ++i) {
    const int idx = 64 * (IC * wave + i) + lane, r = idx >> 4, c = (idx & 15) ^ (r & 15);
    crow[i] = r;
    coff[i] = r * (int)a.ks_t * 2 + c * 16;
  }
#pragma unroll
  for (int i = 0; i < IR; ++i) {
    const int idx = 64 * (IR * wave + i) + lane, r = idx >> 3, c = (idx & 7) ^ ((r >> 1) & 7);
    rrow[i] = r;
    roff[i] = r * (int)a.kss_t * 2 + c * 16;
  }
#pragma unroll
  for (int i = 0; i < IV; ++i) {
    const int idx = 64 * (IV * wave + i) + lane, r = idx >> 4, c = (idx & 15) ^ v_swz(r);
    vrow[i] = r;
    voffs[i] = r * (int)a.vs_t * 2 + c * 16;
  }
  auto dma = [&](const int it, const int buf) {
    const int kv0 = it * kBKV;
    char* st = lds + buf * STAGE;
    const char* kb = K + (int64_t)kv0 * a.ks_t * 2;
    const char* rb = DS > 0 ? KR + (int64_t)kv0 * a.kss_t * 2 : nullptr;
    const char* vb = V + (int64_t)kv0 * a.vs_t * 2;
    if (kv0 + kBKV <= a.T) {
#pragma unroll
      for (int i = 0; i < IC; ++i)
        __builtin_amdgcn_global_load_lds((const void*)(kb + coff[i]), (lds_void_t*)(st + 1024 * (IC * wave + i)), 16, 0, 0);
#pragma unroll
      for (int i = 0; i < IR; ++i)
        __builtin_amdgcn_global_load_lds((const void*)(rb + roff[i]),
                                         (lds_void_t*)(st + KC_BYTES + 1024 * (IR * wave + i)), 16, 0, 0);
#pragma unroll
      for (int i = 0; i < (OUT ? IV : 0); ++i)
        __builtin_amdgcn_global_load_lds((const void*)(vb + voffs[i]),
                                         (lds_void_t*)(st + KC_BYTES + KR_BYTES + 1024 * (IV * wave + i)), 16, 0, 0);
    } else {
      const int last = a.T - 1 - kv0;   // rows past it re-read this one
#pragma unroll
      for (int i = 0; i < IC; ++i) {
        const int d = (min(crow[i], last) - crow[i]) * (int)a.ks_t * 2;
        __builtin_amdgcn_global_load_lds((const void*)(kb + coff[i] + d), (lds_void_t*)(st + 1024 * (IC * wave + i)), 16, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < IR; ++i) {
        const int d = (min(rrow[i], last) - rrow[i]) * (int)a.kss_t * 2;
        __builtin_amdgcn_global_load_lds((const void*)(rb + roff[i] + d),
                                         (lds_void_t*)(st + KC_BYTES + 1024 * (IR * wave + i)), 16, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < (OUT ? IV : 0); ++i) {
        const int d = (min(vrow[i], last) - vrow[i]) * (int)a.vs_t * 2;
        __builtin_amdgcn_global_load_lds((const void*)(vb + voffs[i] + d),
                                         (lds_void_t*)(st + KC_BYTES + KR_BYTES + 1024 * (IV * wave + i)), 16, 0, 0);
      }
    }
  };

  // LDS fragment reads are inline ds_read instructions, issued ahead of
  // their MFMAs and waited for with explicit counts: the compiler does not
  // see them, so it neither waits for every outstanding read before each use
  // nor (taking them for aliases of the direct-to-LDS loads) for the next
  // tile's loads. LDS operations complete in issue order, so a count that
  // also covers a compiler-issued operation (the lane-pair shuffles) only
  // waits longer. Each wait names the registers it completes, so nothing
  // reads or moves them earlier. Immediate offsets carry the buffer, the key
  // half and the k-step; the per-lane parts are computed once.
  //
  // K fragment reads (A operand of S^T): lane l reads key row 32 g + l % 32,
  // chunk 2 s + l / 32 (content dims, 256-byte rows, chunk ^ (r & 15)) or
  // 2 (s - 8) + l / 32 (rotary dims, 128-byte rows, chunk ^ ((r >> 1) & 7));
  // row r and r + 32 share the swizzle, so g is an immediate.
  const uint32_t lds0 = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) char*)lds);
  uint32_t kq[KS];
  {
    const int r = lane & 31;
#pragma unroll
    for (int s = 0; s < KS; ++s)
      kq[s] = lds0 + (s < 8 ? r * 256 + (((2 * s + hl) ^ (r & 15)) << 4)
                            : KC_BYTES + r * 128 + (((2 * (s - 8) + hl) ^ ((r >> 1) & 7)) << 4));
  }
  // V^T fragment reads: lane 4 q + a of 16-lane group G points at key row
  // 4 (G / 2) + q, columns 16 (G % 2) + 4 a of 32-column block n; the
  // transposing read returns to lane t of the group rows 4 (G / 2) .. +3 of
  // column 16 (G % 2) + t, and a second read 8 rows lower gives the other
  // four keys of the MFMA's k order.
  uint32_t vq[4];
  {
    const int G = lane >> 4, qq = (lane & 15) >> 2, a2 = lane & 3;
    const int r = 4 * (G >> 1) + qq;
#pragma unroll
    for (int n = 0; n < 4; ++n) {
      const int c = (32 * n + 16 * (G & 1) + 4 * a2) >> 3;
      vq[n] = lds0 + KC_BYTES + KR_BYTES + r * (kDV * 2) + ((c ^ v_swz(r)) << 4) + (a2 & 1) * 8;
    }
  }

  // One key tile of 64 in two halves of 32 keys (g): S^T = K Q^T, online
  // softmax, O^T += V^T P^T. MASK applies the causal and ragged-end masks
  // (only the wave's diagonal tile and the tile holding key T - 1 need it).
  // kq and vq point into the tile's LDS stage (next_stage moves them on).
  auto tile = [&](const int kv0, auto mask_tag) {
    constexpr bool MASK = decltype(mask_tag)::value;
    u32x4_t kf[KSL];
    v4i16_t vl[NVB][4], vh[NVB][4];
    // K fragment s of half g into ring slot s % KSL
    auto read_k1 = [&](auto g_, auto s_) {
      constexpr int g = decltype(g_)::value, s = decltype(s_)::value;
      constexpr int off = g * (s < 8 ? 32 * 256 : 32 * 128);
      lds_read_b128<off>(kf[s % KSL], kq[s]);
    };
    auto read_k = [&](auto g_) {   // the first KSL fragments of half g
      static_for<KSL>([&](auto s_) { read_k1(g_, s_); });
    };
    auto read_v = [&](auto g_, auto p_) {
      constexpr int g = decltype(g_)::value, p = decltype(p_)::value;
      static_for<4>([&](auto n_) {
        constexpr int n = decltype(n_)::value;
        constexpr int off = (32 * g + 16 * p) * (kDV * 2);
        lds_read_tr<off>(vl[p % NVB][n], vq[n]);
        lds_read_tr<off + 8 * kDV * 2>(vh[p % NVB][n], vq[n]);
      });
    };
    read_k(std::integral_constant<int, 0>{});
    static_for<2>([&](auto g_) {
      constexpr int g = decltype(g_)::value;
      // sacc[f] register e of lane l: key kv0 + 32 g + 8 (e / 4) + 4 (l / 32)
      // + e % 4, query wq0 + 32 f + l % 32
      f32x16_t sacc[NF];
      // outstanding before the first wait: the KSL K reads of this half
      // (issued last), nothing else; fragment s + KSL is read into the slot
      // fragment s leaves, right after its MFMAs issue (they take their
      // operands at issue). Reads issued after fragment s's when it is
      // waited for: KSL + min(s, KS - KSL) - s - 1.
      static_for<KS>([&](auto s_) {
        constexpr int s = decltype(s_)::value;
        lgkm_wait<KSL + (s < KS - KSL ? s : KS - KSL) - s - 1>(kf[s % KSL]);
#pragma unroll
        for (int f = 0; f < NF; ++f) {
          if (s == 0) mfma_s_first(sacc[f], kf[s % KSL], qf[f][s]);
          else mfma_s(sacc[f], kf[s % KSL], qf[f][s]);
        }
        if constexpr (s + KSL < KS) read_k1(g_, std::integral_constant<int, s + KSL>{});
      });
      // S_max pass: the next half's first K reads go out before this half's
      // fold (every ring slot is free once the last MFMA issued)
      if constexpr (!OUT) { if (g == 0) read_k(std::integral_constant<int, 1>{}); }
      if constexpr (NF == 2) s_wait_logits(sacc[0], sacc[1]);
      else s_wait_logits(sacc[0]);
      if constexpr (OUT) read_v(g_, std::integral_constant<int, 0>{});
      if (MASK) {
#pragma unroll
        for (int f = 0; f < NF; ++f) {
          const int i = wq0 + 32 * f + (lane & 31);
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int j = kv0 + 32 * g + 8 * (e >> 2) + 4 * hl + (e & 3);
            if (j >= a.T || (a.causal && j > i)) sacc[f][e] = -INFINITY;
          }
        }
      }
      if constexpr (!OUT) {
        // S_max alone needs no per-row maximum: the half's logits fold into
        // per-lane running maxima, which meet across lanes once, after the
        // last tile (no lane-pair exchange through LDS on every half)
#pragma unroll
        for (int f = 0; f < NF; ++f) {
          float x = max3_nan_ignoring(m_all[f], sacc[f][0], sacc[f][1]);
#pragma unroll
          for (int e = 2; e < 16; e += 2) x = max3_nan_ignoring(x, sacc[f][e], sacc[f][e + 1]);
          m_all[f] = x;
        }
        return;
      }
      // row max over the 32 keys (the lane pair l, l ^ 32 holds one query)
      float bm[NF];
      bool grow = false;
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        float x = max3_nan_ignoring(sacc[f][0], sacc[f][1], sacc[f][2]);
#pragma unroll
        for (int e = 3; e < 15; e += 2) x = max3_nan_ignoring(x, sacc[f][e], sacc[f][e + 1]);
        x = max3_nan_ignoring(x, sacc[f][15], sacc[f][15]);
        x = fmaxf(x, __shfl_xor(x, 32));
        bm[f] = x;
        if (SMAX) m_all[f] = fmaxf(m_all[f], x);
        grow = grow || (x > m_use[f] + thr);
      }
      if (__any(grow)) {
#pragma unroll
        for (int f = 0; f < NF; ++f) {
          const float mn = fmaxf(m_use[f], bm[f] + head);
          const float alpha = __builtin_amdgcn_exp2f((m_use[f] - mn) * c2);
          m_use[f] = mn;
          lsum[f] *= alpha;
#pragma unroll
          for (int n = 0; n < 4; ++n) oacc[f][n] *= alpha;
        }
      }
      // P^T = exp2(c2 (S^T - m)) in bf16; k-step p takes registers 8 p .. 8 p + 7
      bf16x8_t pb[2][NF];   // [p][f]
      auto probs = [&](const int p) {
#pragma unroll
        for (int f = 0; f < NF; ++f) {
          const float nm = -m_use[f] * c2;
          float ls = 0.0f;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float pv = __builtin_amdgcn_exp2f(fmaf(sacc[f][8 * p + e], c2, nm));
            ls += pv;
            pb[p][f][e] = (__bf16)pv;
          }
          lsum[f] += ls;
        }
      };
      auto pv_step = [&](const int p) {
#pragma unroll
        for (int n = 0; n < 4; ++n) {
          const bf16x8_t vf =
              __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(vl[p % NVB][n], vh[p % NVB][n], 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
          for (int f = 0; f < NF; ++f)
            oacc[f][n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pb[p][f], oacc[f][n], 0, 0, 0);
        }
      };
      probs(0);
      if constexpr (NVB == 2) {
        read_v(g_, std::integral_constant<int, 1>{});
        // outstanding: the 8 reads of p = 1 (those of p = 0 are older)
        lgkm_wait<8>(vl[0], vh[0]);
        pv_step(0);
      } else {
        lgkm_wait<0>(vl[0], vh[0]);
        pv_step(0);
        read_v(g_, std::integral_constant<int, 1>{});   // into the buffer p = 0 just used
      }
      probs(1);
      if (g == 0) read_k(std::integral_constant<int, 1>{});
      // outstanding: (the next half's KSL K reads, issued after) the reads of p = 1
      lgkm_wait<g == 0 ? KSL : 0>(vl[1 % NVB], vh[1 % NVB]);
      pv_step(1);
    });
  };

  // Tiles this wave computes: all of them without a causal mask; with one,
  // those starting at or before its last query. The leading ones that need
  // no mask (wholly below the diagonal and inside T) run without it. Every
  // wave takes part in every tile's loads and barrier.
  // (tile t is mask-free for the wave when its last key 64 t + 63 <= wq0)
  const int n_w = wq0 >= a.T ? 0 : (a.causal ? min(nkv, (wq0 + WR - 1) / kBKV + 1) : nkv);
  const int n_full = min(n_w, a.causal ? min(a.T >> 6, (wq0 + 1) >> 6) : (a.T >> 6));
  // Tile it lives in stage it % 2; its loads go out while tile it - 1 is
  // computed, into the stage tile it - 2 left (every wave passed the barrier
  // after finishing it). The stage is a runtime base carried in kq and vq, so
  // the tile code exists once per mask state.
  auto wait_next = [&]() __attribute__((always_inline)) {
    FA_WAIT_DMA();   // this wave's loads of the next tile have landed
    __syncthreads();
  };
  int stg = 0;   // stage of the current tile
  auto next_stage = [&]() __attribute__((always_inline)) {
    const uint32_t d = stg == NSTG - 1 ? (uint32_t)(-(NSTG - 1) * STAGE) : (uint32_t)STAGE;
#pragma unroll
    for (int s = 0; s < KS; ++s) kq[s] += d;
#pragma unroll
    for (int n = 0; n < 4; ++n) vq[n] += d;
    stg = stg == NSTG - 1 ? 0 : stg + 1;
  };
  if (nkv > 0) {
    dma(0, 0);
    wait_next();
  }
  int it = 0;
  for (; it < n_full; ++it) {
    if (it + 1 < nkv) dma(it + 1, (it + 1) & 1);
    tile(it * kBKV, std::false_type{});
    wait_next();
    next_stage();
  }
  for (; it < n_w; ++it) {
    if (it + 1 < nkv) dma(it + 1, (it + 1) & 1);
    tile(it * kBKV, std::true_type{});
    wait_next();
    next_stage();
  }
  for (; it < nkv; ++it) {
    if (it + 1 < nkv) dma(it + 1, (it + 1) & 1);
    wait_next();
  }

  if constexpr (OUT) {
  // normalise and store: oacc[f][n] register e of lane l is column
  // 32 n + 8 (e / 4) + 4 (l / 32) + e % 4 of query wq0 + 32 f + l % 32. The
  // wave's 32 output rows go through its 8 KB of the (now idle) LDS ring,
  // rows of 256 bytes with the 16-byte chunks XOR-swizzled by row, so that
  // each global store instruction writes four whole rows.
  static_assert(NF == 1 && (!OUT || NW * 32 * kDV * 2 <= NSTG * STAGE), "output staging");
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    const float lt = lsum[f] + __shfl_xor(lsum[f], 32);
    const int r = lane & 31, i = wq0 + 32 * f + r;
    const float inv = 1.0f / lt;
    char* ow = lds + wave * (32 * kDV * 2);
#pragma unroll
    for (int n = 0; n < 4; ++n)
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        uint2 w;
        w.x = f32x2_to_bf16x2(oacc[f][n][4 * t] * inv, oacc[f][n][4 * t + 1] * inv);
        w.y = f32x2_to_bf16x2(oacc[f][n][4 * t + 2] * inv, oacc[f][n][4 * t + 3] * inv);
        *(uint2*)(ow + r * 256 + (((4 * n + t) ^ (r & 15)) << 4) + 8 * hl) = w;
      }
    if (a.lse && hl == 0 && i < a.T) a.lse[((int64_t)b * a.H + h) * a.T + i] = a.scale * m_use[f] + logf(lt);
    // (each wave reads back only what it wrote: no barrier, LDS operations
    // of one wave complete in order)
    const int c = lane & 15;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int rr = 4 * k + (lane >> 4), ii = wq0 + 32 * f + rr;
      const u32x4_t v = *(const u32x4_t*)(ow + rr * 256 + ((c ^ (rr & 15)) << 4));
      if (ii < a.T)
        *(u32x4_t*)((uint16_t*)a.o + (int64_t)b * a.os_b + (int64_t)ii * a.os_t + (int64_t)h * a.os_h + 8 * c) = v;
    }
  }
  }   // OUT
  if (SMAX) {
    float mx = m_all[0];
#pragma unroll
    for (int f = 1; f < NF; ++f) mx = fmaxf(mx, m_all[f]);
    mx = wave_max(mx);
    if (lane == 0) red[wave] = mx;
    __syncthreads();
    if (tid == 0) {
      mx = red[0];
      for (int w = 1; w < NW; ++w) mx = fmaxf(mx, red[w]);
      atomic_max_f32(a.smax + h, mx * a.scale);
    }
  }
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

}  // namespace

hipError_t launch_attention_smax_only(const AttnArgs& a, hipStream_t s) {
  if (a.B <= 0 || a.T <= 0 || a.H <= 0) return hipSuccess;
  if (a.d_k != 128 || (a.d_s != 64 && a.d_s != 0) || !a.smax) return hipErrorInvalidValue;
  const int grid = (a.T + kBQ - 1) / kBQ * a.H * a.B;
  if (a.d_s == 64) attn_fwd_kernel<128, 64, true, false><<<grid, 256, 0, s>>>(a);
  else attn_fwd_kernel<128, 0, true, false><<<grid, 256, 0, s>>>(a);
  return hipGetLastError();
}

bool attention_supported(const AttnArgs& a) {
  const bool shape = a.d_k == 128 && (a.d_s == 0 || a.d_s == 64) && a.d_v == kDV;
  if (!shape) return false;
  if (!aligned16(a.q) || !aligned16(a.k) || !aligned16(a.v) || !aligned16(a.o) || (a.d_s && !aligned16(a.ks)))
    return false;
  if ((a.qs_b | a.qs_t | a.qs_h | a.ks_b | a.ks_t | a.ks_h | a.vs_b | a.vs_t | a.vs_h | a.os_b | a.os_t | a.os_h) & 7)
    return false;
  if (a.d_s && ((a.kss_b | a.kss_t) & 7)) return false;
  return true;
}

hipError_t launch_attention(const AttnArgs& a, hipStream_t s) {
  if (a.B <= 0 || a.T <= 0 || a.H <= 0) return hipSuccess;
  const int grid = (a.T + kBQ - 1) / kBQ * a.H * a.B;
  const bool sm = a.smax != nullptr;
  if (a.d_s == 64) {
    if (sm) attn_fwd_kernel<128, 64, true><<<grid, 512, 0, s>>>(a);
    else attn_fwd_kernel<128, 64, false><<<grid, 512, 0, s>>>(a);
  } else {
    if (sm) attn_fwd_kernel<128, 0, true><<<grid, 512, 0, s>>>(a);
    else attn_fwd_kernel<128, 0, false><<<grid, 512, 0, s>>>(a);
  }
  return hipGetLastError();
}

}  // namespace mc
