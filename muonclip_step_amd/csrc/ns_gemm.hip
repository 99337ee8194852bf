// bf16 MFMA GEMM for the Newton-Schulz chains of the MuonClip step.
//
// Every product of the quintic iteration (Notes on Muon blog, "Newton-Schulz"
// and "Algorithm": A = X X^T, A A, and the P X apply) is written in the "NT"
// form C[i][j] = sum_k A[i][k] B[j][k] with both operands row-major and the
// contraction index contiguous: X X^T reads X twice, A A reads the symmetric
// A twice, and P X reads P and the transposed copy X^T that the previous
// apply wrote. One kernel therefore serves all three, batched over the
// matrices of one shape group (grid = tiles x splits x batch, mapped
// XCD-major so the tiles of one matrix share an XCD's L2).
//
// gfx950 design: v_mfma_f32_32x32x16_bf16 with fp32 accumulation; a block of
// 2x2 waves owns a BMxBN tile, each wave a (BM/2)x(BN/2) sub-tile; BK = 64 k
// per stage; A and B stages are double-buffered in LDS (128 KB at 256x256)
// with an XOR swizzle of the 16-byte chunks so both the coalesced stores and
// the MFMA-fragment reads are bank-conflict free; the next stage's global
// loads are in flight while the current stage runs on the matrix cores.
#include "mc_internal.h"

namespace mc {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

int gemm_tile_dim(GemmTile t) { return t == TILE_256 ? 256 : (t == TILE_128 ? 128 : 64); }

// Bijective remap of the linear workgroup id so that consecutive ids of the
// logical order land on one XCD (hardware deals workgroups round-robin over 8).
__device__ inline int xcd_remap(int L, int total) {
  const int q = total >> 3, r = total & 7;
  const int xcd = L & 7, idx = L >> 3;
  return (xcd < r ? xcd * (q + 1) : r * (q + 1) + (xcd - r) * q) + idx;
}

__device__ __attribute__((always_inline)) inline void epilogue_store(const GemmEpi& e, int b, int i, int j, float acc, float sc) {
  float v = e.alpha * sc * acc;
  if (e.cin) v += e.beta * e.cin[(int64_t)b * e.bs_cin + (int64_t)i * e.ld_cin + j];
  if (i == j) v += e.diag;
  if (e.out_f32) e.out_f32[(int64_t)b * e.bs_f32 + (int64_t)i * e.ld_f32 + j] = v;
  if (e.out_hi || e.out_lo || e.out_t) {
    const uint16_t h = f32_to_bf16(v);
    if (e.out_hi) e.out_hi[(int64_t)b * e.bs_hi + (int64_t)i * e.ld_hi + j] = h;
    if (e.out_lo) e.out_lo[(int64_t)b * e.bs_lo + (int64_t)i * e.ld_lo + j] = f32_to_bf16(v - bf16_to_f32(h));
    if (e.out_t) e.out_t[(int64_t)b * e.bs_t + (int64_t)j * e.ld_t + i] = h;
  }
}

__device__ __attribute__((always_inline)) inline float batch_scale(const GemmEpi& e, int b) {
  if (e.scale_pow == 0 || !e.scale) return 1.0f;
  const float s = e.scale[b];
  return e.scale_pow == 1 ? s : s * s;
}

template <int BM, int BN>
__global__ void __launch_bounds__(256, 1) ns_gemm_kernel(const GemmArgs p) {
  constexpr int NT = 256, BK = 64;
  constexpr int WTM = BM / 2, WTN = BN / 2;       // 2 x 2 waves
  constexpr int FM = WTM / 32, FN = WTN / 32;     // 32x32 fragments per wave
  constexpr int CA = BM * BK / 8, CB = BN * BK / 8;   // 16-byte chunks per stage
  constexpr int PT = (CA + CB) / NT;
  constexpr int PA = CA / NT;
  static_assert((CA % NT) == 0 && (CB % NT) == 0, "tile/thread mismatch");
  __shared__ u32x4_t lds[2][CA + CB];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  const int tiles = p.tiles_m * p.tiles_n;
  const int total = tiles * p.splits * p.batch;
  const int L = xcd_remap(blockIdx.x, total);
  const int b = L / (tiles * p.splits);
  const int rem = L - b * tiles * p.splits;
  const int split = rem / tiles;
  const int t = rem - split * tiles;
  const int m0 = (t / p.tiles_n) * BM;
  const int n0 = (t % p.tiles_n) * BN;

  const int kt_begin = split * p.kt_per_split;
  const int kt_end = min(p.ktiles, kt_begin + p.kt_per_split);
  const int nk = kt_end - kt_begin;

  f32x16_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x16_t{};

  u32x4_t st[PT];
  const u32x4_t zero = {0u, 0u, 0u, 0u};

  // global -> registers for k-tile kt (chunk q of a stage: row q/8, 16-byte
  // column chunk q%8; rows past M or N load zeros)
#define MC_GLOAD(kt_)                                                                    \
  {                                                                                      \
    int s_ = 0, kl_ = (kt_);                                                             \
    if (p.nseg > 1 && kl_ >= p.seg[0].ktiles) {                                          \
      kl_ -= p.seg[0].ktiles; s_ = 1;                                                    \
      if (p.nseg > 2 && kl_ >= p.seg[1].ktiles) { kl_ -= p.seg[1].ktiles; s_ = 2; }      \
    }                                                                                    \
    const uint16_t* A_ = (s_ == 0 ? p.seg[0].a : (s_ == 1 ? p.seg[1].a : p.seg[2].a)) +  \
                         (int64_t)b * p.bsa;                                             \
    const uint16_t* B_ = (s_ == 0 ? p.seg[0].b : (s_ == 1 ? p.seg[1].b : p.seg[2].b)) +  \
                         (int64_t)b * p.bsb;                                             \
    const int k0_ = kl_ * BK;                                                            \
    _Pragma("unroll") for (int i = 0; i < PT; ++i) {                                     \
      if (i < PA) {                                                                      \
        const int q = tid + i * NT, r = q >> 3, c = q & 7, gr = m0 + r;                  \
        const int rr = gr < p.M ? gr : p.M - 1;                                          \
        u32x4_t v_ = *(const u32x4_t*)(A_ + (int64_t)rr * p.lda + k0_ + c * 8);              \
        st[i] = gr < p.M ? v_ : zero;                                                    \
      } else {                                                                           \
        const int q = tid + (i - PA) * NT, r = q >> 3, c = q & 7, gr = n0 + r;           \
        const int rr = gr < p.N ? gr : p.N - 1;                                          \
        u32x4_t v_ = *(const u32x4_t*)(B_ + (int64_t)rr * p.ldb + k0_ + c * 8);              \
        st[i] = gr < p.N ? v_ : zero;                                                    \
      }                                                                                  \
    }                                                                                    \
  }
  // registers -> LDS stage buf, 16-byte chunk c of row r stored at chunk c ^ (r & 7)
#define MC_LSTORE(buf_)                                                                  \
  {                                                                                      \
    _Pragma("unroll") for (int i = 0; i < PT; ++i) {                                     \
      if (i < PA) {                                                                      \
        const int q = tid + i * NT, r = q >> 3, c = q & 7;                               \
        lds[(buf_)][r * 8 + (c ^ (r & 7))] = st[i];                                      \
      } else {                                                                           \
        const int q = tid + (i - PA) * NT, r = q >> 3, c = q & 7;                        \
        lds[(buf_)][CA + r * 8 + (c ^ (r & 7))] = st[i];                                 \
      }                                                                                  \
    }                                                                                    \
  }

  if (nk > 0) {
    MC_GLOAD(kt_begin);
    MC_LSTORE(0);
    __syncthreads();
    for (int it = 0; it < nk; ++it) {
      const int cur = it & 1;
      if (it + 1 < nk) MC_GLOAD(kt_begin + it + 1);
      const u32x4_t* La = lds[cur];
      const u32x4_t* Lb = lds[cur] + CA;
#pragma unroll
      for (int kk = 0; kk < BK / 16; ++kk) {
        bf16x8_t af[FM], bfr[FN];
        const int c = kk * 2 + (lane >> 5);
#pragma unroll
        for (int i = 0; i < FM; ++i) {
          const int r = wm * WTM + i * 32 + (lane & 31);
          af[i] = __builtin_bit_cast(bf16x8_t, La[r * 8 + (c ^ (r & 7))]);
        }
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int r = wn * WTN + j * 32 + (lane & 31);
          bfr[j] = __builtin_bit_cast(bf16x8_t, Lb[r * 8 + (c ^ (r & 7))]);
        }
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
      }
      if (it + 1 < nk) MC_LSTORE(cur ^ 1);
      __syncthreads();
    }
  }
#undef MC_GLOAD
#undef MC_LSTORE

  // Epilogue, one 32-row fragment band of every wave at a time, staged through
  // LDS (free after the last barrier) so that every store is coalesced: the
  // accumulator layout of the 32x32 MFMA puts row 8*(r/4) + 4*(l/32) + r%4,
  // column l%32 of a fragment in register r of lane l.
  constexpr int RLD = WTN + 4;                       // padded row of a wave's band
  float* band = reinterpret_cast<float*>(&lds[0][0]) + wave * (32 * RLD);
  const float sc = batch_scale(p.epi, b);
  float* part = p.splits > 1 ? p.partial + ((int64_t)split * p.batch + b) * (int64_t)p.M * p.N : nullptr;
#pragma unroll
  for (int i = 0; i < FM; ++i) {
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        band[(8 * (r >> 2) + 4 * (lane >> 5) + (r & 3)) * RLD + j * 32 + (lane & 31)] = acc[i][j][r];
    __syncthreads();
    const int gi0 = m0 + wm * WTM + i * 32;
    const int gj0 = n0 + wn * WTN;
    // row-major pass: consecutive lanes take consecutive columns
    for (int e = lane; e < 32 * WTN; e += 64) {
      const int rr = e / WTN, cc = e - rr * WTN;
      const int gi = gi0 + rr, gj = gj0 + cc;
      if (gi >= p.M || gj >= p.N) continue;
      const float a = band[rr * RLD + cc];
      if (part) { part[(int64_t)gi * p.N + gj] = a; continue; }
      const GemmEpi& E = p.epi;
      float v = E.alpha * sc * a;
      if (E.cin) v += E.beta * E.cin[(int64_t)b * E.bs_cin + (int64_t)gi * E.ld_cin + gj];
      if (gi == gj) v += E.diag;
      if (E.out_f32) E.out_f32[(int64_t)b * E.bs_f32 + (int64_t)gi * E.ld_f32 + gj] = v;
      if (E.out_hi || E.out_lo) {
        const uint16_t h = f32_to_bf16(v);
        if (E.out_hi) E.out_hi[(int64_t)b * E.bs_hi + (int64_t)gi * E.ld_hi + gj] = h;
        if (E.out_lo) E.out_lo[(int64_t)b * E.bs_lo + (int64_t)gi * E.ld_lo + gj] = f32_to_bf16(v - bf16_to_f32(h));
      }
    }
    // transposed pass: consecutive lanes take consecutive rows of the band
    if (!part && p.epi.out_t) {
      const GemmEpi& E = p.epi;
      for (int e = lane; e < 32 * WTN; e += 64) {
        const int cc = e >> 5, rr = e & 31;
        const int gi = gi0 + rr, gj = gj0 + cc;
        if (gi >= p.M || gj >= p.N) continue;
        float v = E.alpha * sc * band[rr * RLD + cc];
        if (E.cin) v += E.beta * E.cin[(int64_t)b * E.bs_cin + (int64_t)gi * E.ld_cin + gj];
        if (gi == gj) v += E.diag;
        E.out_t[(int64_t)b * E.bs_t + (int64_t)gj * E.ld_t + gi] = f32_to_bf16(v);
      }
    }
    __syncthreads();
  }
}

// Deterministic split-K finish: fixed-order sum of the partial tiles, then the
// same epilogue as the unsplit kernel.
__global__ void __launch_bounds__(256) splitk_reduce_kernel(const GemmArgs p) {
  const int64_t mn = (int64_t)p.M * p.N;
  const int64_t total = mn * p.batch;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int b = (int)(idx / mn);
    const int64_t e = idx - (int64_t)b * mn;
    const int i = (int)(e / p.N), j = (int)(e - (int64_t)i * p.N);
    float acc = 0.0f;
    for (int s = 0; s < p.splits; ++s) acc += p.partial[((int64_t)s * p.batch + b) * mn + e];
    epilogue_store(p.epi, b, i, j, acc, batch_scale(p.epi, b));
  }
}

hipError_t launch_ns_gemm(GemmTile tile, const GemmArgs& a, hipStream_t s) {
  const int total = a.tiles_m * a.tiles_n * a.splits * a.batch;
  if (total <= 0) return hipSuccess;
  switch (tile) {
    case TILE_256: ns_gemm_kernel<256, 256><<<total, 256, 0, s>>>(a); break;
    case TILE_128: ns_gemm_kernel<128, 128><<<total, 256, 0, s>>>(a); break;
    default:       ns_gemm_kernel<64, 64><<<total, 256, 0, s>>>(a); break;
  }
  return hipGetLastError();
}

hipError_t launch_splitk_reduce(const GemmArgs& a, hipStream_t s) {
  const int64_t total = (int64_t)a.M * a.N * a.batch;
  int blocks = (int)((total + 255) / 256);
  if (blocks > 65536) blocks = 65536;
  if (blocks <= 0) return hipSuccess;
  splitk_reduce_kernel<<<blocks, 256, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace mc
