// Per-head max attention logit S_max^h = (1/sqrt(d)) max over the batch and
// over query/key pairs of Q_i^h . K_j^h (Kimi K2 essay, section on Muon and
// attention logits, S_max equation; K2 report 2.1). The logits are never
// written to memory.
//
// MFMA kernels (bf16). For d_k = 128 (MHA, and MLA with the 64-wide shared
// rotary key) the logit pass of the attention kernel (attn_fwd.hip) runs; the
// tile kernel below serves d = 64. Tile kernel: a 256-thread block owns
// 256 query rows of one (head, sample); waves keep their query rows as MFMA
// A-fragments in registers for the whole kernel and stream tiles of K
// through XOR-swizzled LDS; each 32x32 logit fragment is folded straight into
// per-lane running maxima; only tiles on the causal diagonal or the ragged
// end apply a mask, and a wave skips key tiles lying wholly above its causal
// diagonal. Blocks are issued heaviest causal row first. The block max, times
// the scale, is merged by one integer atomic (atomic_max_f32), so the result
// does not depend on scheduling and needs no finishing pass. MLA keys are [k^C_h | k^R]:
// the shared rotary key supplies the last d_s dimensions of every head's key
// (K2 report, per-head MLA clipping). The attention kernel's logit pass
// applies the same masking and merge.
//
// The generic kernel (fp32 inputs, or shapes the MFMA kernel does not cover)
// computes the same definition with one fp32 dot product per pair.
#include <math.h>

#include "mc_internal.h"

namespace mc {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__device__ inline void block_max_commit(float mx, float* out, float scale, float* red) {
  for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[wave] = mx;
  __syncthreads();
  if (threadIdx.x == 0) {
    float m = red[0];
    for (int w = 1; w < (int)(blockDim.x >> 6); ++w) m = fmaxf(m, red[w]);
    atomic_max_f32(out, m * scale);
  }
}

typedef __attribute__((address_space(3))) void ml_lds_void_t;


// XOR swizzle of the 16-byte chunks of an LDS key row of CPR chunks: a
// ds_read_b128 pass serves 16 lanes that read one logical chunk of 16
// consecutive rows, and the swizzle puts them on 16 distinct 4-bank groups.
// Rows of 256 bytes: chunk ^ (r & 15). Rows of 128 or 384 bytes, whose odd
// rows start half a bank cycle later: chunk ^ ((r >> 1) & 7). The XOR stays
// inside the chunk's aligned group of 8 or 16, so it never leaves the row.
template <int CPR>
__device__ __forceinline__ int ml_swz(int r) {
  static_assert(CPR == 8 || CPR == 16 || CPR == 24, "key row width");
  return CPR == 16 ? (r & 15) : ((r >> 1) & 7);
}

// Inline LDS fragment read and a counted wait that names the register it
// completes (the compiler neither tracks the read nor, taking it for an alias
// of the direct-to-LDS loads, waits for those before it).
__device__ __forceinline__ void ml_lds_read(u32x4_t& dst, uint32_t addr) {
  asm volatile("ds_read_b128 %0, %1" : "=v"(dst) : "v"(addr));
}
template <int N>
__device__ __forceinline__ void ml_lgkm_wait(u32x4_t& r) {
  asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(r) : "i"(N));
}
// Running max of a 32x32 logit fragment pair. v_max3_f32 returns the larger
// of two numbers when one is a quiet NaN (IEEE maxNum), as fmaxf does; the
// inline form skips the quieting copies the compiler otherwise puts before
// every fmaxf on an MFMA result. The MFMA results are read only after
// ml_wait_mfma's 24 wait states (more than an 8-pass MFMA's requirement).
__device__ __forceinline__ void ml_wait_mfma(f32x16_t& a0, f32x16_t& a1) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(a0), "+v"(a1));
}
__device__ __forceinline__ float ml_max3(float m, float x, float y) {
  float r;
  asm volatile("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(m), "v"(x), "v"(y));
  return r;
}
// s_waitcnt on the vector-memory counter alone
template <int N>
__device__ __forceinline__ void ml_vm_wait() {
  __builtin_amdgcn_s_waitcnt((N & 15) | 0x70 | 0xF00 | ((N >> 4) << 14));
}

// Key-tile kernel for per-head keys (written for d = 64 and 128; d = 128 now
// takes the attention kernel's logit pass): a 256-thread block owns
// 256 query rows, each wave keeps 64 of them as A fragments, and 64-key tiles
// of K arrive in a three-stage LDS ring through direct-to-LDS loads issued
// two tiles ahead (the XOR swizzle is applied on the source side: the lane
// filling physical chunk pc of row r fetches chunk pc ^ swz(r)). A wave
// reads the eight fragments of a 32-key half with inline reads and consumes
// them under counted waits. At most 168 registers and 48 KB of LDS, so three
// blocks share a CU and hide each other's start-up, fragment waits and
// per-tile barrier (two blocks of up to 256 registers measured 2 % slower).
template <int DK>
__global__ void __launch_bounds__(256, 3) max_logits_tile_kernel(const MaxLogitArgs a) {
  constexpr int D = DK, DC = D / 8, KS = D / 16, RB = 2 * D;
  constexpr int BQ = 256, BKV = 64, NST = 3;
  constexpr int TILE = BKV * RB;                  // bytes per stage
  constexpr int PW = BKV * DC / 64 / 4;           // direct-to-LDS instructions per wave per tile
  static_assert(PW * 256 == BKV * DC && KS <= 8, "tile shape");
  __shared__ __attribute__((aligned(16))) char kt[NST * TILE];
  __shared__ float red[4];

  const int HB = a.H * a.B;
  const int nqt = (a.T + BQ - 1) / BQ;
  const int hb = blockIdx.x % HB;
  const int qt = nqt - 1 - (int)(blockIdx.x / HB);   // heaviest causal rows first
  const int h = hb % a.H, b = hb / a.H;
  const int q0 = qt * BQ;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int wr0 = q0 + wave * 64;

  const uint16_t* Q = (const uint16_t*)a.q + (int64_t)b * a.qs_b + (int64_t)h * a.qs_h;
  const char* K = (const char*)((const uint16_t*)a.k + (int64_t)b * a.ks_b + (int64_t)h * a.ks_h);

  // this wave's query rows as A-fragments: lane l holds row l%32, k-chunk l/32.
  // Rows and keys past T re-read the last valid one; every logit they touch
  // is masked before the max.
  bf16x8_t qf[2][KS];
#pragma unroll
  for (int f = 0; f < 2; ++f) {
    const int row = wr0 + 32 * f + (lane & 31);
    const int rr = row < a.T ? row : a.T - 1;
    const uint16_t* base = Q + (int64_t)rr * a.qs_t + 8 * (lane >> 5);
#pragma unroll
    for (int s = 0; s < KS; ++s) qf[f][s] = __builtin_bit_cast(bf16x8_t, *(const u32x4_t*)(base + 16 * s));
  }

  const int kend = a.causal ? min(a.T, q0 + BQ) : a.T;
  const int nkv = (kend + BKV - 1) / BKV;
  float mx = -INFINITY;

  // direct-to-LDS loads: instruction i of wave w fills LDS chunks
  // 64 (PW w + i) .. +63 of the stage; lane offsets relative to the tile's
  // first key
  int lrow[PW], loff[PW];
#pragma unroll
  for (int i = 0; i < PW; ++i) {
    const int q = 64 * (PW * wave + i) + lane, r = q / DC, c = (q % DC) ^ ml_swz<DC>(r);
    lrow[i] = r;
    loff[i] = r * (int)a.ks_t * 2 + c * 16;
  }
  auto dma = [&](const int it) __attribute__((always_inline)) {
    const int kv0 = it * BKV;
    char* st = kt + (it % NST) * TILE;
    const char* kb = K + (int64_t)kv0 * a.ks_t * 2;
    const int last = a.T - 1 - kv0;   // rows past it re-read this one
#pragma unroll
    for (int i = 0; i < PW; ++i) {
      const int d = lrow[i] > last ? (last - lrow[i]) * (int)a.ks_t * 2 : 0;
      __builtin_amdgcn_global_load_lds((const void*)(kb + loff[i] + d),
                                       (ml_lds_void_t*)(st + 1024 * (PW * wave + i)), 16, 0, 0);
    }
  };
  // per-lane LDS offsets of the fragment reads: key row fk * 32 + l % 32,
  // chunk 2 s + l / 32
  const uint32_t kt0 = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) char*)kt);
  uint32_t fo[KS];
  {
    const int r = lane & 31;
#pragma unroll
    for (int s = 0; s < KS; ++s) fo[s] = kt0 + r * RB + (((2 * s + (lane >> 5)) ^ ml_swz<DC>(r)) << 4);
  }

  if (nkv > 0) dma(0);
  if (nkv > 1) dma(1);
  if (nkv > 1) ml_vm_wait<PW>();   // tile 0 landed (tile 1 may be in flight)
  else ml_vm_wait<0>();
  __syncthreads();
  for (int it = 0; it < nkv; ++it) {
    // the stage of tile it + 2 held tile it - 1, which every wave finished
    // before the last barrier
    if (it + 2 < nkv) dma(it + 2);
    const int kv0 = it * BKV;
    const uint32_t sb = (uint32_t)((it % NST) * TILE);
    if (!(a.causal && kv0 > wr0 + 63) && wr0 < a.T) {
      const bool need_mask = (a.causal && kv0 + BKV - 1 > wr0) || (kv0 + BKV > a.T) || (wr0 + 63 >= a.T);
#pragma unroll
      for (int fk = 0; fk < 2; ++fk) {
        u32x4_t kf[KS];
#pragma unroll
        for (int s = 0; s < KS; ++s) ml_lds_read(kf[s], fo[s] + sb + fk * 32 * RB);
        f32x16_t acc0 = f32x16_t{}, acc1 = f32x16_t{};
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          switch (KS - 1 - s) {   // reads complete in issue order
            case 7: ml_lgkm_wait<7>(kf[s]); break;
            case 6: ml_lgkm_wait<6>(kf[s]); break;
            case 5: ml_lgkm_wait<5>(kf[s]); break;
            case 4: ml_lgkm_wait<4>(kf[s]); break;
            case 3: ml_lgkm_wait<3>(kf[s]); break;
            case 2: ml_lgkm_wait<2>(kf[s]); break;
            case 1: ml_lgkm_wait<1>(kf[s]); break;
            default: ml_lgkm_wait<0>(kf[s]); break;
          }
          const bf16x8_t k8 = __builtin_bit_cast(bf16x8_t, kf[s]);
          acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf[0][s], k8, acc0, 0, 0, 0);
          acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf[1][s], k8, acc1, 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);   // keep each wait next to its MFMAs
        }
        if (!need_mask) {
          ml_wait_mfma(acc0, acc1);
#pragma unroll
          for (int e = 0; e < 16; ++e) mx = ml_max3(mx, acc0[e], acc1[e]);
        } else {
          // register e of lane l: query row 8*(e/4) + 4*(l/32) + e%4, key column l%32
          const int j = kv0 + fk * 32 + (lane & 31);
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int i0 = wr0 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
            const int i1 = i0 + 32;
            const bool ok0 = i0 < a.T && j < a.T && (!a.causal || j <= i0);
            const bool ok1 = i1 < a.T && j < a.T && (!a.causal || j <= i1);
            if (ok0) mx = fmaxf(mx, acc0[e]);
            if (ok1) mx = fmaxf(mx, acc1[e]);
          }
        }
      }
    }
    // tile it + 1 landed for this wave (tile it + 2 may be in flight), then
    // for every wave
    if (it + 2 < nkv) ml_vm_wait<PW>();
    else ml_vm_wait<0>();
    __syncthreads();
  }
  block_max_commit(mx, a.out + h, a.scale, red);
}

template <bool BF16>
__global__ void __launch_bounds__(256) max_logits_generic_kernel(const MaxLogitArgs a) {
  __shared__ float red[4];
  const int h = blockIdx.x % a.H, b = blockIdx.x / a.H;
  float mx = -INFINITY;
  const int64_t pairs = (int64_t)a.T * a.T;
  for (int64_t p = threadIdx.x; p < pairs; p += 256) {
    const int i = (int)(p / a.T), j = (int)(p - (int64_t)i * a.T);
    if (a.causal && j > i) continue;
    const int64_t qo = (int64_t)b * a.qs_b + (int64_t)i * a.qs_t + (int64_t)h * a.qs_h;
    const int64_t ko = (int64_t)b * a.ks_b + (int64_t)j * a.ks_t + (int64_t)h * a.ks_h;
    const int64_t so = (int64_t)b * a.kss_b + (int64_t)j * a.kss_t;
    float dot = 0.0f;
    if (BF16) {
      const uint16_t* q = (const uint16_t*)a.q;
      const uint16_t* k = (const uint16_t*)a.k;
      const uint16_t* ks = (const uint16_t*)a.ks;
      for (int f = 0; f < a.d_k; ++f) dot = fmaf(bf16_to_f32(q[qo + f]), bf16_to_f32(k[ko + f]), dot);
      for (int f = 0; f < a.d_s; ++f) dot = fmaf(bf16_to_f32(q[qo + a.d_k + f]), bf16_to_f32(ks[so + f]), dot);
    } else {
      const float* q = (const float*)a.q;
      const float* k = (const float*)a.k;
      const float* ks = (const float*)a.ks;
      for (int f = 0; f < a.d_k; ++f) dot = fmaf(q[qo + f], k[ko + f], dot);
      for (int f = 0; f < a.d_s; ++f) dot = fmaf(q[qo + a.d_k + f], ks[so + f], dot);
    }
    mx = fmaxf(mx, dot);
  }
  block_max_commit(mx, a.out + h, a.scale, red);
}

__global__ void max_logits_init_kernel(float* out, int H) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < H) out[i] = -INFINITY;
}

static bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

bool max_logits_mfma_supported(const MaxLogitArgs& a) {
  if (!a.bf16) return false;
  const bool shape = (a.d_k == 128 && (a.d_s == 0 || a.d_s == 64)) || (a.d_k == 64 && a.d_s == 0);
  if (!shape) return false;
  if (!aligned16(a.q) || !aligned16(a.k) || (a.d_s && !aligned16(a.ks))) return false;
  if ((a.qs_b | a.qs_t | a.qs_h | a.ks_b | a.ks_t | a.ks_h) & 7) return false;
  if (a.d_s && ((a.kss_b | a.kss_t) & 7)) return false;
  // the key tiles' lane offsets (64 rows of the t stride) are 32-bit
  const int64_t kLimit = (int64_t)1 << 23;
  if (a.ks_t >= kLimit || (a.d_s && a.kss_t >= kLimit)) return false;
  return true;
}

hipError_t launch_max_logits_init(float* out, int32_t H, hipStream_t s) {
  if (H <= 0) return hipSuccess;
  max_logits_init_kernel<<<(H + 255) / 256, 256, 0, s>>>(out, H);
  return hipGetLastError();
}

hipError_t launch_max_logits(const MaxLogitArgs& a, hipStream_t s, bool* used_mfma) {
  *used_mfma = false;
  if (a.B <= 0 || a.T <= 0 || a.H <= 0) return hipSuccess;
  if (max_logits_mfma_supported(a)) {
    *used_mfma = true;
    const int nqt = (a.T + 255) / 256;             // 256 query rows per block
    const int grid = nqt * a.H * a.B;
    if (a.d_k == 128) {
      // d_k = 128 with or without the MLA rotary part: the attention kernel's
      // logit pass (eight waves of 32 rows, two per SIMD). MLA layer: 472 us
      // against 562 us for a four-wave kernel of 64 rows per wave and 128-key
      // tiles; MHA layer: 140 us against 142 us for the tile kernel below.
      AttnArgs t{};
      t.q = a.q; t.k = a.k; t.ks = a.ks; t.v = a.k;
      t.smax = a.out;
      t.qs_b = a.qs_b; t.qs_t = a.qs_t; t.qs_h = a.qs_h;
      t.ks_b = a.ks_b; t.ks_t = a.ks_t; t.ks_h = a.ks_h;
      t.kss_b = a.kss_b; t.kss_t = a.kss_t;
      t.vs_b = a.ks_b; t.vs_t = a.ks_t; t.vs_h = a.ks_h;
      t.B = a.B; t.T = a.T; t.H = a.H; t.d_k = a.d_k; t.d_s = a.d_s; t.d_v = 128;
      t.causal = a.causal; t.scale = a.scale;
      return launch_attention_smax_only(t, s);
    }
    else max_logits_tile_kernel<64><<<grid, 256, 0, s>>>(a);
  } else if (a.bf16) {
    max_logits_generic_kernel<true><<<a.H * a.B, 256, 0, s>>>(a);
  } else {
    max_logits_generic_kernel<false><<<a.H * a.B, 256, 0, s>>>(a);
  }
  return hipGetLastError();
}


}  // namespace mc
