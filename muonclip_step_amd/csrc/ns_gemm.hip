// bf16 MFMA GEMM for the Newton-Schulz chains of the MuonClip step.
//
// Every product of the quintic iteration (Notes on Muon blog, "Newton-Schulz"
// and "Algorithm": A = X X^T, A A, and the P X apply) is C[i][j] = sum_k
// A[i][k] B[k][j] with A row-major and k contiguous. X X^T and the symmetric
// A A read their B operand as rows of the same row-major matrix ("NT" form:
// B[k][j] = X[j][k]); the apply P X reads B = X in its own row-major [k][n]
// layout and forms the MFMA B fragments with gfx950's transposing LDS read,
// so no transposed copy of X is ever written. One kernel serves all of them
// and the Gram-space head's m x m products, batched over the matrices of one
// shape group (grid = tiles x splits x batch, mapped XCD-major so the tiles
// of one matrix share an XCD's L2). The symmetric products (X X^T, A A,
// and the products of two commuting symmetric m x m matrices that run the
// first iterations in Gram space) compute only the tiles on and above the
// diagonal and store each off-diagonal tile a second time, transposed.
//
// gfx950 design: v_mfma_f32_32x32x16_bf16 with fp32 accumulation; a block of
// 2x2 waves (or 2x4) owns a BMxBN tile, each wave a (BM/2)x(BN/2) (or
// (BM/2)x(BN/4)) sub-tile. K advances in 64-wide stages held in a two-slot
// LDS ring that direct-to-LDS loads (global_load_lds_dwordx4) fill, so no
// register staging is needed. One barrier per stage retires a slot; the
// loads of the stage after next go out in two halves, under the last k-step
// of one stage and the first k-step of the next, each load placed between two
// MFMAs, and every memory instruction of the steady-state loop is
// unconditional (the last stage is peeled). The MFMA fragments of each 16-k
// step are read from LDS while the previous step's MFMAs run. The epilogue is
// specialised at compile time per use and stages each wave's results through
// LDS for 16-byte stores.
#include "mc_internal.h"

namespace mc {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint16_t u16x4_t __attribute__((ext_vector_type(4)));

int gemm_tile_dim(GemmTile t) { return t == TILE_256 ? 256 : (t == TILE_128 ? 128 : 64); }

// Tile order of the non-symmetric products: consecutive tiles walk down
// kGroupRows tile rows before moving one tile column right, so the 32
// workgroups an XCD runs at once cover a 4 x 8 block of tiles and share their
// operand rows in that XCD's L2 (a row-major order would share only one A
// block across 32 different B blocks).
constexpr int kGroupRows = 4;

// Bijective remap of the linear workgroup id so that consecutive ids of the
// logical order land on one XCD (hardware deals workgroups round-robin over 8).
__device__ inline int xcd_remap(int L, int total) {
  const int q = total >> 3, r = total & 7;
  const int xcd = L & 7, idx = L >> 3;
  return (xcd < r ? xcd * (q + 1) : r * (q + 1) + (xcd - r) * q) + idx;
}

// The epilogue of eight consecutive columns j0 .. j0+7 of row i (the split-K
// finish): v = alpha scale acc + beta (cin_hi + cin_lo) + diag (i == j)
// (cin_lo optional),
// bf16 v to out_hi and bf16 (v - hi) to out_lo, in 16-byte accesses (row
// starts and strides are multiples of 8 elements).
typedef uint16_t u16x8_t __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
__device__ __attribute__((always_inline)) inline void epilogue_store8(const GemmEpi& e, int b, int i, int j0,
                                                                      const float (&acc)[8], float sc) {
  float v[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) v[k] = e.alpha * sc * acc[k];
  if (e.cin_hi) {
    const int64_t o = (int64_t)b * e.bs_cin + (int64_t)i * e.ld_cin + j0;
    const u16x8_t h = *(const u16x8_t*)(e.cin_hi + o);
    const u16x8_t l = e.cin_lo ? *(const u16x8_t*)(e.cin_lo + o) : u16x8_t{0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] += e.beta * (bf16_to_f32(h[k]) + bf16_to_f32(l[k]));
  }
#pragma unroll
  for (int k = 0; k < 8; ++k)
    if (i == j0 + k) v[k] += e.diag;
  u16x8_t hi, lo;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    hi[k] = f32_to_bf16(v[k]);
    lo[k] = f32_to_bf16(v[k] - bf16_to_f32(hi[k]));
  }
  if (e.out_hi) *(u16x8_t*)(e.out_hi + (int64_t)b * e.bs_hi + (int64_t)i * e.ld_hi + j0) = hi;
  if (e.out_lo) *(u16x8_t*)(e.out_lo + (int64_t)b * e.bs_lo + (int64_t)i * e.ld_lo + j0) = lo;
}

__device__ __attribute__((always_inline)) inline float batch_scale(const GemmEpi& e, int b) {
  if (e.scale_pow == 0 || !e.scale) return 1.0f;
  const float s = e.scale[b];
  return e.scale_pow == 1 ? s : s * s;
}

// Chunk swizzle of a 128-byte LDS row (eight 16-byte chunks): row r stores
// logical chunk c at c ^ swz(r). Chosen from the SQ_LDS_BANK_CONFLICT counter
// of this kernel's fragment reads on gfx950 (which the swizzle drives to zero).
#ifndef MC_SWZ128
#define MC_SWZ128(r) (((r) >> 1) & 7)
#endif
__device__ __forceinline__ int swz(int r) { return MC_SWZ128(r); }

// Calls f(acc[I / FN][I % FN], I / FN, I % FN) for I = I0 .. N-1 with every
// index a compile-time constant (keeps the accumulators in registers).
template <int I0, int N, int FN>
struct FragVisit {
  template <typename A, typename F>
  __device__ __forceinline__ static void run(A& acc, F& f) {
    f(acc[I0 / FN][I0 % FN], I0 / FN, I0 % FN);
    FragVisit<I0 + 1, N, FN>::run(acc, f);
  }
};
template <int N, int FN>
struct FragVisit<N, N, FN> {
  template <typename A, typename F>
  __device__ __forceinline__ static void run(A&, F&) {}
};

// compile-time epilogue selection
enum : int {
  E_HI = 2,       // bf16 store of v
  E_LO = 4,       // bf16 store of v - bf16(v)
  E_CIN = 16,     // v += beta * (cin_hi + cin_lo)[i][j]
  E_DIAG = 32,    // v += diag on i == j
  E_PART = 64,    // split-K: raw fp32 partial, no epilogue
  E_SYM = 128,    // upper tiles only; off-diagonal tiles also stored mirrored
  E_UPD = 512,    // last apply: the weight update with v as O, no store of v
  E_FOUT = 1024,  // also store bf16(v) in fragment order (frag_out)
  E_FIN = 2048,   // v += beta * frag_in (bf16, fragment order) instead of cin
  E_XADD = 4096,  // store pass adds xadd_coef * scale * xadd[i][j] to bf16 v (apply)
  E_CIN1 = 8192,  // with E_CIN: cin_hi alone (v += beta * cin_hi[i][j])
};

typedef __attribute__((address_space(3))) void lds_void_t;

// wait for every outstanding LDS operation of this wave
#define MC_WAIT_LGKM_ALL() asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory")
// s_waitcnt with only vmcnt constrained (expcnt and lgkmcnt left at max)
#define MC_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | 0x70 | 0xF00 | (((n) >> 4) << 14))

template <int BM, int BN, int NSTAGE, int EPI, int NNB = 0, int NW = 4>
__global__ void __launch_bounds__(64 * NW, 1) __attribute__((amdgpu_waves_per_eu(NW / 4, NW / 4)))
ns_gemm_kernel(const GemmArgs p, const FusedUpd u) {
  // NNB: the B operand is stored [k][n] (n contiguous) and staged in LDS the
  // same way, BN columns per k-row; its fragments are read with
  // ds_read_b64_tr_b16, whose 16-lane groups read four k-rows of 32 bytes.
  // The 16-byte chunks of k-row r are XOR-swizzled so those four rows land on
  // distinct banks: ^ 4 (r & 3) for rows of 16 or more chunks, ^ 2 ((r >> 1) & 1)
  // for 128-byte rows (odd rows start half a bank cycle later).
  constexpr int PB = BN * 2;                      // bytes per LDS row of the [k][n] B tile
  constexpr int LPR = BN / 8, RPB = 64 / LPR;     // lanes per B row, B rows per DMA instruction
  auto swzB = [](int r) { return LPR >= 16 ? 4 * (r & 3) : 2 * ((r >> 1) & 1); };
  constexpr int BK = kGemmBK;                     // 64: one 128-byte row segment per operand row
  constexpr int KK = BK / 16;                     // MFMA k-steps per stage
  static_assert(NW == 4 || NW == 8, "2 x 2 or 2 x 4 waves");
  constexpr int NWN = NW / 2;                     // waves along n
  constexpr int WTM = BM / 2, WTN = BN / NWN;     // wave sub-tile
  constexpr int FM = WTM / 32, FN = WTN / 32;     // 32x32 fragments per wave
  constexpr int ROWB = BK * 2;                    // bytes per LDS row (128)
  constexpr int CPR = ROWB / 16;                  // 16-byte chunks per row (8)
  constexpr int RPI = 64 / CPR;                   // rows per DMA instruction (8)
  constexpr int STAGE = (BM + BN) * ROWB;         // bytes per stage
  constexpr int IA = BM / NW / RPI, IB = BN / NW / RPI;   // DMA instructions per wave per stage
  static_assert(IA >= 1 && IB >= 1 && IA * NW * RPI == BM && IB * NW * RPI == BN, "DMA split");
  constexpr int TP = WTM * 2 + 16;                // epilogue staging: bytes per T row
  constexpr int LDS_BYTES = STAGE * NSTAGE > NW * WTN * TP ? STAGE * NSTAGE : NW * WTN * TP;
  static_assert(LDS_BYTES <= 160 * 1024, "LDS");
  static_assert((KK % 2) == 0, "two fragment slots");
  __shared__ __attribute__((aligned(1024))) char lds[LDS_BYTES];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform: LDS targets stay scalar
  const int wm = wave / NWN, wn = wave % NWN;

  const int tiles = (EPI & E_SYM) ? p.tiles_m * (p.tiles_m + 1) / 2 : p.tiles_m * p.tiles_n;
  const int total = tiles * p.splits * p.batch;
  const int L = xcd_remap(blockIdx.x, total);
  const int b = L / (tiles * p.splits);
  const int rem = L - b * tiles * p.splits;
  const int split = rem / tiles;
  int t = rem - split * tiles;
  int tm, tn;
  if (EPI & E_SYM) {            // t-th tile of the upper triangle, row by row
    tm = 0;
    while (t >= p.tiles_m - tm) { t -= p.tiles_m - tm; ++tm; }
    tn = tm + t;
  } else {                      // groups of kGroupRows tile rows, column by column inside a group
    const int grp = t / (kGroupRows * p.tiles_n);
    const int rows = min(kGroupRows, p.tiles_m - grp * kGroupRows);
    const int local = t - grp * kGroupRows * p.tiles_n;
    tn = local / rows;
    tm = grp * kGroupRows + (local - tn * rows);
  }
  const int m0 = tm * BM;
  const int n0 = tn * BN;

  const int kt_begin = split * p.kt_per_split;
  const int kt_end = min(p.ktiles, kt_begin + p.kt_per_split);
  const int nk = kt_end - kt_begin;

  // Per-lane DMA source offsets (elements, without k): DMA instruction i of
  // this wave fills tile rows RPI*(wave*IA + i) .. +RPI-1; lane l lands at LDS
  // slot l of that 1 KB block = row l/CPR, physical chunk l%CPR, so it fetches
  // logical chunk (l%CPR) ^ swz(row). Rows past M / N re-read the last row;
  // they only feed outputs that are never stored.
  // (32-bit: a row offset is below rows * ld < 2^31 for every matrix this
  // library accepts; batch offsets are applied to the base pointers)
  int offA[IA], offB[IB];
#pragma unroll
  for (int i = 0; i < IA; ++i) {
    const int r = RPI * (wave * IA + i) + lane / CPR;
    const int gr = min(m0 + r, p.M - 1);
    offA[i] = gr * p.lda + (((lane % CPR) ^ swz(r)) * 8);
  }
#pragma unroll
  for (int i = 0; i < IB; ++i) {
    if (NNB) {   // k-row r of the stage, 16-byte chunk (lane % LPR) ^ swzB(r) of columns n0..
      const int r = RPB * (wave * IB + i) + lane / LPR;
      const int c = (lane % LPR) ^ swzB(r);
      offB[i] = r * p.ldb + min(n0 + c * 8, p.N - 8);
    } else {
      const int r = RPI * (wave * IB + i) + lane / CPR;
      const int gr = min(n0 + r, p.N - 1);
      offB[i] = gr * p.ldb + (((lane % CPR) ^ swz(r)) * 8);
    }
  }

  // segment bases and boundaries, read from the kernel arguments once so the
  // loop issues no scalar loads (they would force full LDS-counter waits)
  const int nseg = p.nseg;
  const int kb0 = p.seg[0].ktiles, kb1 = p.seg[0].ktiles + (nseg > 1 ? p.seg[1].ktiles : 0);
  const uint16_t* A0 = p.seg[0].a + (int64_t)b * p.bsa;
  const uint16_t* B0 = p.seg[0].b + (int64_t)b * p.bsb;
  const uint16_t* A1 = nseg > 1 ? p.seg[1].a + (int64_t)b * p.bsa : A0;
  const uint16_t* B1 = nseg > 1 ? p.seg[1].b + (int64_t)b * p.bsb : B0;
  const uint16_t* A2 = nseg > 2 ? p.seg[2].a + (int64_t)b * p.bsa : A1;
  const uint16_t* B2 = nseg > 2 ? p.seg[2].b + (int64_t)b * p.bsb : B1;

  // Source pointers of k-stage st_ (relative to kt_begin): the segment that
  // holds it and the k offset inside that segment.
#define MC_STAGE_SRC(st_, dA_, dB_)                                                      \
  const uint16_t* dA_ = A0;                                                              \
  const uint16_t* dB_ = B0;                                                              \
  {                                                                                      \
    const int kg_ = kt_begin + (st_);                                                    \
    int kl_ = kg_;                                                                       \
    if (kg_ >= kb1) { dA_ = A2; dB_ = B2; kl_ = kg_ - kb1; }                             \
    else if (kg_ >= kb0) { dA_ = A1; dB_ = B1; kl_ = kg_ - kb0; }                        \
    dA_ += kl_ * BK;                                                                     \
    dB_ += kl_ * BK * (NNB ? p.ldb : 1);                                                 \
  }
  // DMA instruction j_ (compile-time) of a stage: j_ < IA fill A rows, the
  // rest B rows; db_ is the stage's LDS slot
#define MC_DMA(j_, dA_, dB_, db_)                                                        \
  {                                                                                      \
    if ((j_) < IA) {                                                                     \
      __builtin_amdgcn_global_load_lds((const void*)(dA_ + offA[(j_) < IA ? (j_) : 0]),  \
          (lds_void_t*)(db_ + (RPI * (wave * IA + (j_))) * ROWB), 16, 0, 0);             \
    } else {                                                                             \
      const int i_ = (j_) - IA >= 0 && (j_) - IA < IB ? (j_) - IA : 0;                   \
      __builtin_amdgcn_global_load_lds((const void*)(dB_ + offB[i_]),                    \
          (lds_void_t*)(db_ + BM * ROWB + (RPI * (wave * IB + i_)) * ROWB), 16, 0, 0);   \
    }                                                                                    \
  }

  f32x16_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x16_t{};
  bf16x8_t af[2][FM], bfr[2][FN];
  typedef short v4i16_t __attribute__((ext_vector_type(4)));
  v4i16_t bl[2][FN], bh[2][FN];          // NNB: B fragments as two transposing 8-byte reads
  // NNB per-lane byte offsets of fragment j inside a B stage at k-step 0. A
  // ds_read_b64_tr_b16 gives lane t of a 16-lane group element b of the lanes
  // 4q + t/4 (q = 0..3): with lane 4q + a of group G pointing at k-row
  // 8 (G/2) + q, columns 16 (G%2) + 4a of the fragment, lane t receives rows
  // 8 (G/2) .. +3 of column 16 (G%2) + t, and a second read four rows lower
  // completes the eight k values of the MFMA B operand.
  uint32_t fragB[FN];
  {
    const int G = lane >> 4, q = (lane & 15) >> 2, a2 = lane & 3;
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int r = 8 * (G >> 1) + q;
      const int c = (wn * WTN + 32 * j + 16 * (G & 1) + 4 * a2) >> 3;
      fragB[j] = r * PB + ((c ^ swzB(r)) << 4) + (a2 & 1) * 8;
    }
  }

  // Fragment reads of k-step kk_ (16 k) of stage kt_ into register slot sl_.
  // They are issued as inline ds_read_b128 so the compiler does not track
  // them: its LDS-counter analysis is conservative across the loop back-edge
  // and would wait for every outstanding read before each MFMA block. The
  // compiler therefore also takes their destination registers as written
  // when the asm issues: every k-step ends with an explicit wait
  // (MC_WAIT_LGKM(0)) for the reads it issued, so no read is in flight at a
  // block boundary, where register allocation may copy those registers.
  // No other LDS-counter operation is in flight inside the loop.
  const uint32_t lds_base = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) char*)lds);
#define MC_FRAG(kt_, kk_, sl_)                                                           \
  {                                                                                      \
    const uint32_t base_ = lds_base + ((kt_) % NSTAGE) * STAGE;                          \
    const int c_ = (kk_) * 2 + (lane >> 5);                                              \
    _Pragma("unroll") for (int i = 0; i < FM; ++i) {                                     \
      const int r_ = wm * WTM + i * 32 + (lane & 31);                                    \
      const uint32_t ad_ = base_ + r_ * ROWB + ((c_ ^ swz(r_)) << 4);                    \
      asm volatile("ds_read_b128 %0, %1" : "=v"(af[(sl_)][i]) : "v"(ad_));              \
    }                                                                                    \
    _Pragma("unroll") for (int j = 0; j < FN; ++j) {                                     \
      if (NNB) {                                                                         \
        const uint32_t ad_ = base_ + BM * ROWB + (kk_) * 16 * PB + fragB[j];             \
        asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(bl[(sl_)][j]) : "v"(ad_));       \
        asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(bh[(sl_)][j]) : "v"(ad_), "i"(4 * PB)); \
      } else {                                                                           \
        const int r_ = wn * WTN + j * 32 + (lane & 31);                                  \
        const uint32_t ad_ = base_ + BM * ROWB + r_ * ROWB + ((c_ ^ swz(r_)) << 4);      \
        asm volatile("ds_read_b128 %0, %1" : "=v"(bfr[(sl_)][j]) : "v"(ad_));           \
      }                                                                                  \
    }                                                                                    \
  }
  // wait until at most n_ fragment reads are outstanding
#define MC_WAIT_LGKM(n_) asm volatile("s_waitcnt lgkmcnt(%0)" ::"i"(n_))
  // One k-step, interleaved: MFMA m of register slot sl_, then fragment read
  // m of the next k-step (stage rkt_, k-step rkk_, into slot rsl_; if rd_),
  // then, spaced evenly over the MFMAs, DMA instructions d0_ .. d1_-1 of
  // stage dsrc_ into the ring slot of stage dkt_ (if dma_). Spreading the
  // memory instructions between MFMAs keeps the in-order issue from stalling
  // the matrix core behind a burst of loads. Every flag and count is a
  // compile-time constant at each use, so no branch enters the MFMA stream.
  constexpr int NRD = FM + (NNB ? 2 : 1) * FN;    // fragment reads per k-step
  constexpr int NSTEP = (FM * FN > NRD ? FM * FN : NRD) > IA + IB ? (FM * FN > NRD ? FM * FN : NRD) : IA + IB;
#define MC_STEP(sl_, rd_, rkt_, rkk_, rsl_, dma_, dsrc_, dkt_, d0_, d1_)                 \
  {                                                                                      \
    const uint32_t rb_ = lds_base + ((rkt_) % NSTAGE) * STAGE;                           \
    const int rc_ = (rkk_) * 2 + (lane >> 5);                                            \
    MC_STAGE_SRC(dsrc_, dA_, dB_)                                                        \
    char* db_ = lds + ((dkt_) % NSTAGE) * STAGE;                                         \
    const int dn_ = (d1_) - (d0_);                                                       \
    const int ds_ = NSTEP / (dn_ > 0 ? dn_ : 1) > 0 ? NSTEP / (dn_ > 0 ? dn_ : 1) : 1;     \
    _Pragma("unroll") for (int m = 0; m < NSTEP; ++m) {                                  \
      if (m < FM * FN)                                                                   \
        acc[m / FN][m % FN] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(                   \
            af[(sl_)][m / FN], NNB ? __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(  \
            bl[(sl_)][m % FN], bh[(sl_)][m % FN], 0, 1, 2, 3, 4, 5, 6, 7)) : bfr[(sl_)][m % FN], \
            acc[m / FN][m % FN], 0, 0, 0);                                               \
      __builtin_amdgcn_sched_barrier(0);                                                 \
      if ((rd_) && m < FM) {                                                             \
        const int r_ = wm * WTM + m * 32 + (lane & 31);                                  \
        const uint32_t ad_ = rb_ + r_ * ROWB + ((rc_ ^ swz(r_)) << 4);                   \
        asm volatile("ds_read_b128 %0, %1" : "=v"(af[(rsl_)][m < FM ? m : 0]) : "v"(ad_)); \
      } else if ((rd_) && !NNB && m < FM + FN) {                                         \
        const int j_ = m - FM;                                                           \
        const int r_ = wn * WTN + j_ * 32 + (lane & 31);                                 \
        const uint32_t ad_ = rb_ + BM * ROWB + r_ * ROWB + ((rc_ ^ swz(r_)) << 4);       \
        asm volatile("ds_read_b128 %0, %1" : "=v"(bfr[(rsl_)][j_ < FN ? j_ : 0]) : "v"(ad_)); \
      } else if ((rd_) && NNB && m < FM + 2 * FN) {                                      \
        const int j_ = (m - FM) >> 1;                                                    \
        const uint32_t ad_ = rb_ + BM * ROWB + (rkk_) * 16 * PB + fragB[j_ < FN ? j_ : 0];  \
        if (((m - FM) & 1) == 0)                                                         \
          asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(bl[(rsl_)][j_ < FN ? j_ : 0]) : "v"(ad_)); \
        else                                                                             \
          asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(bh[(rsl_)][j_ < FN ? j_ : 0]) \
                       : "v"(ad_), "i"(4 * PB));                                          \
      }                                                                                  \
      if ((dma_) && dn_ > 0 && m % ds_ == 0 && (d0_) + m / ds_ < (d1_))                  \
        MC_DMA((d0_) + m / ds_, dA_, dB_, db_);                                          \
      __builtin_amdgcn_sched_barrier(0);                                                 \
    }                                                                                    \
  }

  // Pipeline over the two-slot ring; stage s lives in slot s % 2. Its loads
  // go out in two halves: [0, DH) under the last k-step of stage s-2, right
  // after the barrier that frees slot s % 2, and [DH, ND) under the first
  // k-step of stage s-1. Before the last k-step of stage kt every wave holds
  // all of stage kt's fragments in registers; the block then waits for
  // stage kt+1 to land, synchronises once (publishing stage kt+1 and
  // retiring slot kt % 2), and reads the first fragments of stage kt+1 under
  // the last k-step's MFMAs.
  static_assert(NSTAGE == 2, "the issue schedule assumes a two-slot ring");
  constexpr int ND = IA + IB, DH = ND / 2;
  if (nk > 0) {
    {   // prologue: all of stage 0, the first half of stage 1
      MC_STAGE_SRC(0, sA_, sB_)
#pragma unroll
      for (int j = 0; j < ND; ++j) MC_DMA(j, sA_, sB_, lds);
    }
    if (nk > 1) {
      MC_STAGE_SRC(1, sA_, sB_)
#pragma unroll
      for (int j = 0; j < DH; ++j) MC_DMA(j, sA_, sB_, lds + STAGE);
      MC_WAIT_VMCNT(DH);                // stage 0 landed
    } else {
      MC_WAIT_VMCNT(0);
    }
    __builtin_amdgcn_s_barrier();
    MC_FRAG(0, 0, 0);
    MC_WAIT_LGKM(0);
    // stages 0 .. nk-2. After the barrier that retires stage kt, the first
    // half of stage kt+2 goes into the freed slot; for kt+2 == nk it
    // re-reads stage nk-1 into that slot, which is never read again.
    for (int kt = 0; kt < nk - 1; ++kt) {
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        if (kk == 0) {
          MC_STEP(kk & 1, true, kt, kk + 1, (kk + 1) & 1, true, kt + 1, kt + 1, DH, ND);
        } else if (kk + 1 < KK) {
          MC_STEP(kk & 1, true, kt, kk + 1, (kk + 1) & 1, false, kt, kt, 0, 0);
        } else {
          MC_WAIT_VMCNT(0);             // stage kt+1 landed (this wave's part)
          __builtin_amdgcn_s_barrier();
          __builtin_amdgcn_sched_barrier(0);
          const int src = min(kt + 2, nk - 1);
          MC_STEP(kk & 1, true, kt + 1, 0, 0, true, src, kt + 2, 0, DH);
        }
        MC_WAIT_LGKM(0);                // the next k-step's fragments landed
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    {   // last stage: no loads, no barrier
      const int kt = nk - 1;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        if (kk + 1 < KK) {
          MC_STEP(kk & 1, true, kt, kk + 1, (kk + 1) & 1, false, kt, kt, 0, 0);
        } else {
          MC_STEP(kk & 1, false, kt, 0, 0, false, kt, kt, 0, 0);
        }
        MC_WAIT_LGKM(0);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
  MC_WAIT_VMCNT(0);
#undef MC_FRAG
#undef MC_STAGE_SRC
#undef MC_DMA
#undef MC_WAIT_LGKM
#undef MC_STEP

  // Epilogue. Register 4g+q of lane l holds row 8g + 4(l/32) + q, column
  // l%32 of its 32x32 fragment: runs of four consecutive rows at one column.
  // bf16 results are staged through LDS so that every global store moves 16
  // bytes per lane: each wave writes its sub-tile transposed (T[j][i], the
  // four rows as one 8-byte write) into a private region of the freed ring,
  // then reads T rows (8 consecutive i at one j) for the transposed or
  // mirrored store, and reads T with the gfx950 transposing LDS read
  // (ds_read_b64_tr_b16: lane t of a 16-lane group receives element b of
  // the lanes 4q + t/4, q = 0..3) to get 8 consecutive j at one i for the
  // row-major store. M and N are multiples of 32; stores test bounds per lane.
  const float sc = (EPI & E_PART) ? 1.0f : batch_scale(p.epi, b);
  const float alpha = p.epi.alpha * sc, beta = p.epi.beta, diag = p.epi.diag;
  static_assert(!(EPI & E_CIN) || (EPI & E_SYM), "cin is read transposed: symmetric products only");
  const bool mirror = (EPI & E_SYM) && tm != tn;
  const int wi0 = m0 + wm * WTM, wj0 = n0 + wn * WTN;          // wave sub-tile origin
  const int li = 4 * (lane >> 5), lj = lane & 31;

  if (EPI & E_PART) {   // split-K: raw fp32 partials, row-major
    float* part = p.partial + ((int64_t)split * p.batch + b) * ((int64_t)p.M * p.N);
    const uint32_t r0 = (uint32_t)((wi0 + li) * p.N + wj0 + lj);
    auto frag_part = [&](const f32x16_t& a, int fi, int fj) __attribute__((always_inline)) {
      if (wi0 + fi * 32 >= p.M || wj0 + fj * 32 >= p.N) return;
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int q = 0; q < 4; ++q) part[r0 + (uint32_t)((fi * 32 + 8 * g + q) * p.N + fj * 32)] = a[4 * g + q];
    };
    FragVisit<0, FM * FN, FN>::run(acc, frag_part);
    return;
  }

  const int ld_hi = (EPI & E_HI) ? p.epi.ld_hi : 0, ld_lo = (EPI & E_LO) ? p.epi.ld_lo : 0;
  const int ld_cin = (EPI & E_CIN) ? p.epi.ld_cin : 0;
  const uint16_t* cin_hi = (EPI & E_CIN) ? p.epi.cin_hi + (int64_t)b * p.epi.bs_cin : nullptr;
  const uint16_t* cin_lo = (EPI & E_CIN) ? p.epi.cin_lo + (int64_t)b * p.epi.bs_cin : nullptr;
  uint16_t* ohi = (EPI & E_HI) ? p.epi.out_hi + (int64_t)b * p.epi.bs_hi : nullptr;
  uint16_t* olo = (EPI & E_LO) ? p.epi.out_lo + (int64_t)b * p.epi.bs_lo : nullptr;
  const uint32_t t_cin = (uint32_t)((wj0 + lj) * ld_cin + wi0 + li);
  // this lane's registers 0 .. 7 of fragment (fi, fj) in the bf16
  // fragment-order copy (registers 8 .. 15 are 512 elements further)
  auto frag_ptr = [&](auto* base, int fi, int fj) __attribute__((always_inline)) {
    const int bi = (wi0 + fi * 32) >> 5, bj = (wj0 + fj * 32) >> 5;
    return base + (int64_t)b * p.epi.bs_frag + (int64_t)(bi * p.epi.frag_nb + bj) * 1024 + lane * 8;
  };
  if (EPI & E_FOUT) {   // straight from the accumulators, rounded as the bf16 store below rounds them
    auto frag_out = [&](const f32x16_t& a, int fi, int fj) __attribute__((always_inline)) {
      if (wi0 + fi * 32 >= p.M || wj0 + fj * 32 >= p.N) return;
      uint16_t* d = frag_ptr(p.epi.frag_out, fi, fj);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        uint32_t w[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) w[k] = f32x2_to_bf16x2(a[8 * h + 2 * k] * alpha, a[8 * h + 2 * k + 1] * alpha);
        *(u32x4_t*)(d + 512 * h) = u32x4_t{w[0], w[1], w[2], w[3]};
      }
    };
    FragVisit<0, FM * FN, FN>::run(acc, frag_out);
  }

  // private staging region of this wave: T[WTN][WTM] bf16, row pitch TP
  // bytes (16 bytes of padding keep the 8-byte writes of 16 lanes on
  // distinct banks)
  char* tw = lds + wave * (WTN * TP);
  __builtin_amdgcn_s_barrier();          // every wave is done with the ring

  // write pass: v (or its bf16 residual when lo_pass) into T
  // The bf16 A of the Poly's b A term (E_FIN) is read for a group of
  // fragments before they are staged, so its latency is paid once per group.
  constexpr int kFinGrp = 8;   // eight fragments' bf16 A: 64 registers (the fp32 copy allowed four with eight waves)
  constexpr int NFR = FM * FN, FGRP = (EPI & E_FIN) ? (NFR < kFinGrp ? NFR : kFinGrp) : 1;
  auto load_fin = [&](int fi, int fj, u32x4_t (&c_f)[2]) __attribute__((always_inline)) {
    // (fragments past M or N are never stored and read nothing)
    const bool in = wi0 + fi * 32 < p.M && wj0 + fj * 32 < p.N;
    const uint16_t* src = frag_ptr(p.epi.frag_in, in ? fi : 0, in ? fj : 0);
#pragma unroll
    for (int h = 0; h < 2; ++h) c_f[h] = in ? *(const u32x4_t*)(src + 512 * h) : u32x4_t{};
  };
  auto stage = [&](bool lo_pass) __attribute__((always_inline)) {
    auto frag_stage = [&](const f32x16_t& a, int fi, int fj, const u32x4_t (&c_f)[2]) __attribute__((always_inline)) {
      uint2 c_hi[4], c_lo[4];
      if (EPI & E_CIN) {   // rows r..r+3 at column c of the symmetric A, read as row c
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const uint32_t o = t_cin + (uint32_t)(fj * 32 * ld_cin + fi * 32 + 8 * g);
          c_hi[g] = *(const uint2*)(cin_hi + o);
          if (!(EPI & E_CIN1)) c_lo[g] = *(const uint2*)(cin_lo + o);
        }
      }
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int ur = fi * 32 + 8 * g + li;           // wave-local row of q = 0
        const int uc = fj * 32 + lj;                   // wave-local column
        float v[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          v[q] = a[4 * g + q] * alpha;
          if (EPI & E_FIN) {   // register 4g + q: half g / 2, element 4 (g % 2) + q
            const uint32_t wf = c_f[g >> 1][2 * (g & 1) + (q >> 1)];
            v[q] += beta * bf16_to_f32((uint16_t)((q & 1) ? wf >> 16 : wf));
          }
          if (EPI & E_CIN) {
            const uint32_t wh = q < 2 ? c_hi[g].x : c_hi[g].y;
            const float ch = bf16_to_f32((uint16_t)((q & 1) ? wh >> 16 : wh));
            if (EPI & E_CIN1) {
              v[q] += beta * ch;
            } else {
              const uint32_t wl = q < 2 ? c_lo[g].x : c_lo[g].y;
              v[q] += beta * (ch + bf16_to_f32((uint16_t)((q & 1) ? wl >> 16 : wl)));
            }
          }
          if ((EPI & E_DIAG) && wi0 + ur + q == wj0 + uc) v[q] += diag;
        }
        uint32_t w01 = f32x2_to_bf16x2(v[0], v[1]), w23 = f32x2_to_bf16x2(v[2], v[3]);
        if (lo_pass) {
          w01 = f32x2_to_bf16x2(v[0] - bf16_to_f32((uint16_t)w01), v[1] - bf16_to_f32((uint16_t)(w01 >> 16)));
          w23 = f32x2_to_bf16x2(v[2] - bf16_to_f32((uint16_t)w23), v[3] - bf16_to_f32((uint16_t)(w23 >> 16)));
        }
        *(uint2*)(tw + uc * TP + ur * 2) = make_uint2(w01, w23);
      }
    };
#pragma unroll
    for (int I0 = 0; I0 < NFR; I0 += FGRP) {
      u32x4_t cf[FGRP][2];
      if (EPI & E_FIN) {
#pragma unroll
        for (int k = 0; k < FGRP; ++k) load_fin((I0 + k) / FN, (I0 + k) % FN, cf[k]);
      }
#pragma unroll
      for (int k = 0; k < FGRP; ++k) frag_stage(acc[(I0 + k) / FN][(I0 + k) % FN], (I0 + k) / FN, (I0 + k) % FN, cf[k]);
    }
  };
  // row-major store of T^T: lane t of group gr reads rows i0+t, columns
  // j0..j0+7 (two transposing reads) and stores them as one 16-byte vector
  auto store_direct = [&](uint16_t* dst, int ld) __attribute__((always_inline)) {
    const int t = lane & 15, gr = lane >> 4;
    const int sq = t >> 2, sa = t & 3;               // this lane's source row / column block
#pragma unroll
    for (int jb = 0; jb < WTN / 32; ++jb)
#pragma unroll
      for (int ib = 0; ib < WTM / 16; ++ib) {
        const int i0 = ib * 16, j0 = jb * 32 + gr * 8;
        typedef short v4i16 __attribute__((ext_vector_type(4)));
        typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
        const v4i16 x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_v4i16*)(tw + (j0 + sq) * TP + (i0 + 4 * sa) * 2));
        const v4i16 x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_v4i16*)(tw + (j0 + 4 + sq) * TP + (i0 + 4 * sa) * 2));
        const int gi = wi0 + i0 + t, gj = wj0 + j0;
        if (gi < p.M && gj < p.N) {
          uint4 o;
          o.x = (uint32_t)(uint16_t)x0[0] | ((uint32_t)(uint16_t)x0[1] << 16);
          o.y = (uint32_t)(uint16_t)x0[2] | ((uint32_t)(uint16_t)x0[3] << 16);
          o.z = (uint32_t)(uint16_t)x1[0] | ((uint32_t)(uint16_t)x1[1] << 16);
          o.w = (uint32_t)(uint16_t)x1[2] | ((uint32_t)(uint16_t)x1[3] << 16);
          *(uint4*)(dst + (uint32_t)(gi * ld + gj)) = o;
        }
      }
  };
  // transposed store: T rows (8 consecutive i at one j) as 16-byte vectors
  auto store_trans = [&](uint16_t* dst, int ld) __attribute__((always_inline)) {
    constexpr int CH = WTM / 8, RPS = 64 / CH;       // chunks per T row, T rows per pass
    const int ch = lane % CH, rr = lane / CH;
#pragma unroll
    for (int it = 0; it < WTN / RPS; ++it) {
      const int jr = it * RPS + rr;
      const uint4 o = *(const uint4*)(tw + jr * TP + ch * 16);
      const int gj = wj0 + jr, gi = wi0 + ch * 8;
      if (gj < p.N && gi < p.M) *(uint4*)(dst + (uint32_t)(gj * ld + gi)) = o;
    }
  };

  // Store pass with a bf16 matrix added at the output's own positions:
  // out = bf16(v + c s X[i][j]), v the bf16 value staged in T, X read in
  // 16-byte vectors, each group's loads issued before its first store.
  auto store_xadd = [&]() __attribute__((always_inline)) {
    typedef uint16_t u16x8_t __attribute__((ext_vector_type(8)));
    const uint16_t* xs = p.epi.xadd + (int64_t)b * p.epi.bs_xadd;
    const int ldx = p.epi.ld_xadd;
    const float cx = p.epi.xadd_coef * sc;
    const int t = lane & 15, gr = lane >> 4;
    const int sq = t >> 2, sa = t & 3;
    constexpr int NIB = WTM / 16, NV = (WTN / 32) * NIB, CHK = NV < 8 ? NV : 8;
#pragma unroll
    for (int c0 = 0; c0 < NV; c0 += CHK) {
      u16x8_t xv[CHK];
#pragma unroll
      for (int q = 0; q < CHK; ++q) {
        const int jb = (c0 + q) / NIB, ib = (c0 + q) % NIB;
        const int gi = wi0 + ib * 16 + t, gj = wj0 + jb * 32 + gr * 8;
        if (gi < p.M && gj < p.N) xv[q] = *(const u16x8_t*)(xs + (int64_t)gi * ldx + gj);
      }
#pragma unroll
      for (int q = 0; q < CHK; ++q) {
        const int jb = (c0 + q) / NIB, ib = (c0 + q) % NIB;
        const int i0 = ib * 16, j0 = jb * 32 + gr * 8;
        typedef short v4i16 __attribute__((ext_vector_type(4)));
        typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
        const v4i16 x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_v4i16*)(tw + (j0 + sq) * TP + (i0 + 4 * sa) * 2));
        const v4i16 x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_v4i16*)(tw + (j0 + 4 + sq) * TP + (i0 + 4 * sa) * 2));
        const int gi = wi0 + i0 + t, gj = wj0 + j0;
        if (gi < p.M && gj < p.N) {
          const u16x8_t o = {(uint16_t)x0[0], (uint16_t)x0[1], (uint16_t)x0[2], (uint16_t)x0[3],
                             (uint16_t)x1[0], (uint16_t)x1[1], (uint16_t)x1[2], (uint16_t)x1[3]};
          u16x8_t r;
#pragma unroll
          for (int e = 0; e < 8; ++e) r[e] = f32_to_bf16(fmaf(cx, bf16_to_f32(xv[q][e]), bf16_to_f32(o[e])));
          *(u16x8_t*)(ohi + (uint32_t)(gi * ld_hi + gj)) = r;
        }
      }
    }
  };

  // Fused update: W <- clip_row ((1 - lr wd) W - lr rms O), O the bf16 value
  // staged in T, in the same arithmetic as the update kernel. W is row-major;
  // its rows are the product's rows (trans = 0: read T as store_direct does,
  // 8 consecutive columns of one row per lane) or its columns (trans = 1: T
  // rows as store_trans reads them). Each group of up to 8 vectors issues all
  // its W loads before the first store.
  constexpr int kUpdChunk = 8;   // (4 and 16 measured the same)
  auto store_update = [&]() __attribute__((always_inline)) {
    typedef uint16_t u16x8_t __attribute__((ext_vector_type(8)));
    uint16_t* W = (uint16_t*)u.w[b];
    const int ldw = u.ld[b];
    const ClipRule cr = b < u.nclip ? u.clip[b] : ClipRule{-1, 1, 0, {0, 0}, {0, 0}, {0.0f, 0.0f}};
    auto upd8 = [&](const u16x8_t& o, const u16x8_t& w, float sc) __attribute__((always_inline)) {
      u16x8_t r;
#pragma unroll
      for (int e = 0; e < 8; ++e) r[e] = f32_to_bf16(fmaf(-u.lr_rms, bf16_to_f32(o[e]), bf16_to_f32(w[e]) * u.decay) * sc);
      return r;
    };
    if (!u.trans[b]) {   // W is [m][nn]: row gi, columns gj .. gj + 7
      const int t = lane & 15, gr = lane >> 4;
      const int sq = t >> 2, sa = t & 3;
      constexpr int NIB = WTM / 16, NV = (WTN / 32) * NIB, CHK = NV < kUpdChunk ? NV : kUpdChunk;
#pragma unroll
      for (int c0 = 0; c0 < NV; c0 += CHK) {
        u16x8_t wv[CHK];
#pragma unroll
        for (int q = 0; q < CHK; ++q) {
          const int jb = (c0 + q) / NIB, ib = (c0 + q) % NIB;
          const int gi = wi0 + ib * 16 + t, gj = wj0 + jb * 32 + gr * 8;
          if (gi < u.m && gj < u.nn) wv[q] = *(const u16x8_t*)(W + (int64_t)gi * ldw + gj);
        }
#pragma unroll
        for (int q = 0; q < CHK; ++q) {
          const int jb = (c0 + q) / NIB, ib = (c0 + q) % NIB;
          const int i0 = ib * 16, j0 = jb * 32 + gr * 8;
          typedef short v4i16 __attribute__((ext_vector_type(4)));
          typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
          const v4i16 x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_v4i16*)(tw + (j0 + sq) * TP + (i0 + 4 * sa) * 2));
          const v4i16 x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (lds_v4i16*)(tw + (j0 + 4 + sq) * TP + (i0 + 4 * sa) * 2));
          const int gi = wi0 + i0 + t, gj = wj0 + j0;
          if (gi < u.m && gj < u.nn) {
            const u16x8_t o = {(uint16_t)x0[0], (uint16_t)x0[1], (uint16_t)x0[2], (uint16_t)x0[3],
                               (uint16_t)x1[0], (uint16_t)x1[1], (uint16_t)x1[2], (uint16_t)x1[3]};
            const float sc = row_clip_scale(cr, gi, u.s_max, u.heads, u.tau, u.clip_global);
            *(u16x8_t*)(W + (int64_t)gi * ldw + gj) = upd8(o, wv[q], sc);
          }
        }
      }
    } else {             // W is [nn][m]: row gj, columns gi .. gi + 7
      constexpr int CH = WTM / 8, RPS = 64 / CH, NV = WTN / RPS, CHK = NV < kUpdChunk ? NV : kUpdChunk;
      const int ch = lane % CH, rr = lane / CH;
      const int gi = wi0 + ch * 8;
#pragma unroll
      for (int c0 = 0; c0 < NV; c0 += CHK) {
        u16x8_t wv[CHK];
#pragma unroll
        for (int q = 0; q < CHK; ++q) {
          const int gj = wj0 + (c0 + q) * RPS + rr;
          if (gj < u.nn && gi < u.m) wv[q] = *(const u16x8_t*)(W + (int64_t)gj * ldw + gi);
        }
#pragma unroll
        for (int q = 0; q < CHK; ++q) {
          const int jr = (c0 + q) * RPS + rr, gj = wj0 + jr;
          if (gj < u.nn && gi < u.m) {
            const u16x8_t o = *(const u16x8_t*)(tw + jr * TP + ch * 16);
            const float sc = row_clip_scale(cr, gj, u.s_max, u.heads, u.tau, u.clip_global);
            *(u16x8_t*)(W + (int64_t)gj * ldw + gi) = upd8(o, wv[q], sc);
          }
        }
      }
    }
  };

  stage(false);
  if (EPI & E_UPD) {
    if (u.gamma_out && blockIdx.x == 0)   // the step's gamma output, from the same s_max
      for (int i = tid; i < u.gamma_slots * u.heads; i += 64 * NW)
        u.gamma_out[i] = gamma_of(layer_s(u.s_max, i / u.heads, i % u.heads, u.heads, u.clip_global), u.tau);
    MC_WAIT_LGKM_ALL();
    store_update();
    return;
  }
  if (EPI & E_XADD) {
    static_assert(!(EPI & E_XADD) || !(EPI & (E_SYM | E_LO)), "xadd: non-symmetric products, hi only");
    store_xadd();
    return;
  }
  if (EPI & E_HI) store_direct(ohi, ld_hi);
  if ((EPI & E_HI) && mirror) store_trans(ohi, ld_hi);
  if (EPI & E_LO) {
    MC_WAIT_LGKM_ALL();
    stage(true);
    store_direct(olo, ld_lo);
    if (mirror) store_trans(olo, ld_lo);
  }
}

// Deterministic split-K finish: fixed-order sum of the partial tiles, then the
// same epilogue as the unsplit kernel.
// Each thread finishes eight consecutive elements of a row; the partials are
// added in split order, as the tiles would have accumulated them.
__global__ void __launch_bounds__(256) splitk_reduce_kernel(const GemmArgs p) {
  const int64_t mn = (int64_t)p.M * p.N;
  const int n8 = p.N >> 3;
  const int64_t per_b = (int64_t)p.M * n8, total = per_b * p.batch;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int b = (int)(idx / per_b);
    const int64_t r = idx - (int64_t)b * per_b;
    const int i = (int)(r / n8), j0 = (int)(r - (int64_t)i * n8) * 8;
    const int64_t e = (int64_t)i * p.N + j0;
    float acc[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
    for (int s = 0; s < p.splits; ++s) {
      const f32x4_t* src = (const f32x4_t*)(p.partial + ((int64_t)s * p.batch + b) * mn + e);
      const f32x4_t x0 = src[0], x1 = src[1];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        acc[k] += x0[k];
        acc[4 + k] += x1[k];
      }
    }
    epilogue_store8(p.epi, b, i, j0, acc, batch_scale(p.epi, b));
  }
}

// A 256x256 launch runs eight waves (2 x 4, two per SIMD, which hide each
// other's LDS waits, barriers and epilogue) when it has at most one workgroup
// per CU, or when it is a symmetric m x m product (K = m: few k-stages per
// tile, so the epilogue weighs more); other launches keep four waves, whose
// 128x128 sub-tiles need fewer fragment reads per MFMA (measured: eight waves
// 2.4 % faster on the 4 x 2048^2 chains, 1.2 % slower over all launches of
// the 1155 expert matrices, 7 % faster on their Poly launches).
template <int EPI, int NNB = 0>
static void launch_epi(GemmTile tile, const GemmArgs& a, int total, hipStream_t s, const FusedUpd& u) {
  const bool square = (EPI & E_SYM) && a.ktiles * kGemmBK <= a.M;
  switch (tile) {
    case TILE_256:
      if (total <= device_cus() || square) ns_gemm_kernel<256, 256, 2, EPI, NNB, 8><<<total, 512, 0, s>>>(a, u);
      else ns_gemm_kernel<256, 256, 2, EPI, NNB, 4><<<total, 256, 0, s>>>(a, u);
      break;
    case TILE_128: ns_gemm_kernel<128, 128, 2, EPI, NNB><<<total, 256, 0, s>>>(a, u); break;
    default:       ns_gemm_kernel<64, 64, 2, EPI, NNB><<<total, 256, 0, s>>>(a, u); break;
  }
}

int gemm_tile_count(const GemmArgs& a, GemmKind kind) {
  const bool sym = a.splits == 1 && (kind == GEMM_GRAM || kind == GEMM_POLY);
  return sym ? a.tiles_m * (a.tiles_m + 1) / 2 : a.tiles_m * a.tiles_n;
}

hipError_t launch_ns_gemm(GemmTile tile, GemmKind kind, bool split_pair, const GemmArgs& a, hipStream_t s,
                          const FusedUpd* upd) {
  const int total = gemm_tile_count(a, kind) * a.splits * a.batch;
  if (total <= 0) return hipSuccess;
  static const FusedUpd none{};
  const bool fused = upd && upd->n > 0;
  // the fused update covers the whole batch, unsplit, of an apply
  if (fused && (kind != GEMM_APPLY || a.splits > 1 || upd->n != a.batch || a.batch > kMaxFusedMats))
    return hipErrorInvalidValue;
  const FusedUpd& u = fused ? *upd : none;
  // the epilogue works on 32x32 fragments and moves 16-byte vectors:
  // extents must be multiples of 32; leading dimensions and batch strides
  // multiples of 8 elements and bases 16-byte aligned
  const GemmEpi& e = a.epi;
  auto bad = [](const void* ptr, int64_t ld, int64_t bs) {
    return ptr && ((ld & 7) || (bs & 7) || ((uintptr_t)ptr & 15));
  };
  if ((a.M & 31) || (a.N & 31) || bad(e.cin_hi, e.ld_cin, e.bs_cin) || bad(e.cin_lo, e.ld_cin, e.bs_cin) ||
      bad(e.out_hi, e.ld_hi, e.bs_hi) || bad(e.out_lo, e.ld_lo, e.bs_lo) || bad(e.xadd, e.ld_xadd, e.bs_xadd))
    return hipErrorInvalidValue;
  // the added matrix rides on an unsplit, unfused apply that stores only hi
  if (e.xadd && (kind != GEMM_APPLY || a.splits > 1 || fused || !e.out_hi || e.out_lo)) return hipErrorInvalidValue;
  // a Gram-kind C input is hi only, on a product without operand pairs or fragment copy
  if (kind == GEMM_GRAM && e.cin_hi && (e.cin_lo || split_pair || e.frag_out || e.out_lo))
    return hipErrorInvalidValue;
  // a residual (lo) store needs operand pairs, which a Poly without them does not read
  if ((e.out_lo && !split_pair) || (kind == GEMM_POLY && e.cin_lo && !split_pair)) return hipErrorInvalidValue;
  const bool frag = (kind == GEMM_GRAM && e.frag_out) || (kind == GEMM_POLY && e.frag_in);
  if (frag && (a.splits > 1 || split_pair || ((uintptr_t)(kind == GEMM_GRAM ? (const void*)e.frag_out : e.frag_in) & 15) ||
               e.frag_nb * 32 < a.M || e.frag_nb * 32 < a.N || (e.bs_frag & 7)))
    return hipErrorInvalidValue;
  if (a.splits > 1) {
    launch_epi<E_PART>(tile, a, total, s, u);
  } else if (kind == GEMM_GRAM) {
    // without operand pairs the Poly epilogue reads A_hi from the bf16 copy
    // in fragment order (with them, A_lo is an operand too)
    if (split_pair) launch_epi<E_SYM | E_HI | E_LO>(tile, a, total, s, u);
    else if (frag) launch_epi<E_SYM | E_HI | E_FOUT>(tile, a, total, s, u);
    // bf16 products of two symmetric matrices (Gram-space head), plus diag on
    // the diagonal and beta times a third symmetric matrix
    else if (e.cin_hi) launch_epi<E_SYM | E_CIN | E_CIN1 | E_DIAG | E_HI>(tile, a, total, s, u);
    else if (e.diag != 0.0f) launch_epi<E_SYM | E_DIAG | E_HI>(tile, a, total, s, u);
    else launch_epi<E_SYM | E_HI>(tile, a, total, s, u);
  } else if (kind == GEMM_POLY) {
    if (split_pair) launch_epi<E_SYM | E_CIN | E_DIAG | E_HI | E_LO>(tile, a, total, s, u);
    else if (frag) launch_epi<E_SYM | E_FIN | E_DIAG | E_HI>(tile, a, total, s, u);
    else launch_epi<E_SYM | E_CIN | E_CIN1 | E_DIAG | E_HI>(tile, a, total, s, u);   // b A_hi
  } else if (fused) {
    launch_epi<E_UPD, 1>(tile, a, total, s, u);   // last apply with the weight update
  } else if (e.xadd) {
    launch_epi<E_HI | E_XADD, 1>(tile, a, total, s, u);   // apply ending the Gram-space head
  } else {
    launch_epi<E_HI, 1>(tile, a, total, s, u);   // apply: B = X stored [k][n]
  }
  return hipGetLastError();
}

hipError_t launch_splitk_reduce(const GemmArgs& a, hipStream_t s) {
  if ((a.N & 7) || (a.epi.out_hi && (a.epi.ld_hi & 7)) || (a.epi.out_lo && (a.epi.ld_lo & 7)) ||
      (a.epi.cin_hi && (a.epi.ld_cin & 7)))
    return hipErrorInvalidValue;
  const int64_t total = (int64_t)a.M * (a.N / 8) * a.batch;
  int blocks = (int)((total + 255) / 256);
  if (blocks > 65536) blocks = 65536;
  if (blocks <= 0) return hipSuccess;
  splitk_reduce_kernel<<<blocks, 256, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace mc
