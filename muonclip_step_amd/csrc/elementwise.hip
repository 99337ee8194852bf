// HBM-bound kernels of the MuonClip step (gfx950).
//
//  momentum_kernel   M <- mu M + G (Notes on Moonlight, "Background"), the
//                    per-block sum of squares of the new M (or of the Nesterov
//                    look-ahead G + mu M, Notes on Muon blog, "Analysis") for
//                    its Frobenius norm, and its bf16 copy in the [min][max]
//                    orientation the Newton-Schulz GEMMs read (Notes on Muon
//                    blog, "Algorithm": bf16 copy, normalisation, transpose
//                    when rows > cols; a 64x64 LDS tile transposes). The
//                    1/(||M||+eps) scale is not applied here; the first GEMM
//                    epilogues fold it in.
//  norm_finalize     fixed-order fp64 sum of the partials -> scale per matrix.
//  update_kernel     W <- s_row ((1 - lr wd) W - lr 0.2 sqrt(max(r,c)) O): the
//                    RMS-matched, decoupled-decay update (Notes on Moonlight,
//                    "Scaling up Muon"), with the post-update QK-Clip row scale
//                    s_row = gamma_h^expo (Kimi K2 essay, MHA equations and the
//                    MLA table; gamma_h = min(1, tau / S_max^h)) fused in.
//                    The step normally applies it in the last Newton-Schulz
//                    apply's epilogue; this kernel serves the waves that
//                    cannot fuse it (fp32 W, an O copy, unaligned rows).
//  gamma_kernel      gamma_h for every (layer, head); with clip_global one
//                    gamma per layer from its largest S_max (K2 report 2.1).
//  clip_apply_kernel the QK-Clip rescale alone on an existing weight.
//
// Tiles are 64x64 elements per 256-thread block; each thread moves 4
// consecutive elements per row (128-bit fp32 / 64-bit bf16 accesses) when the
// row stride and base allow, scalar accesses otherwise.
#include <algorithm>

#include "mc_internal.h"

namespace mc {

typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint16_t u16x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

template <typename M>
__device__ inline int find_mat(const M* mats, int nmat, int blk) {
  int j = 0;
  for (int t = 1; t < nmat; ++t)
    if (blk >= mats[t].block_start) j = t;
  return j;
}

// ---------------------------------------------------------------- momentum

__global__ void __launch_bounds__(256) momentum_kernel(const MomArgs a) {
  __shared__ uint16_t tile[64][66];
  __shared__ float red[4];
  const int j = find_mat(a.mat, a.nmat, blockIdx.x);
  const MomMat& mm = a.mat[j];
  const int local = blockIdx.x - mm.block_start;
  const int tr = local / mm.tiles_c, tc = local - tr * mm.tiles_c;
  const int tid = threadIdx.x, cx = tid & 15, ry = tid >> 4;
  const int col = tc * 64 + cx * 4;
  float ss = 0.0f;
  // vector path: every load of the thread's four rows goes out before the
  // first store (M is read and written in place and G is another buffer,
  // but the compiler cannot know the rows do not overlap and would
  // serialise them)
  f32x4_t mvs[4], gvs[4];
  if (mm.vec && col < mm.cols) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int row = tr * 64 + ry + 16 * k;
      if (row < mm.rows) {
        const int64_t base = (int64_t)row * mm.ld + col;
        // G and M are streamed once per step: non-temporal accesses
        mvs[k] = __builtin_nontemporal_load((const f32x4_t*)(mm.m + base));
        if (mm.g_bf16) {
          const u16x4_t gb = __builtin_nontemporal_load((const u16x4_t*)((const uint16_t*)mm.g + base));
          gvs[k] = f32x4_t{bf16_to_f32(gb[0]), bf16_to_f32(gb[1]), bf16_to_f32(gb[2]), bf16_to_f32(gb[3])};
        } else {
          gvs[k] = __builtin_nontemporal_load((const f32x4_t*)((const float*)mm.g + base));
        }
      }
    }
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int lr = ry + 16 * k, row = tr * 64 + lr;
    float v[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    if (row < mm.rows) {
      const int64_t base = (int64_t)row * mm.ld + col;
      if (mm.vec && col < mm.cols) {
        const f32x4_t mv = mvs[k], gv = gvs[k];
        f32x4_t nv;
        nv[0] = fmaf(a.mu, mv[0], gv[0]); nv[1] = fmaf(a.mu, mv[1], gv[1]);
        nv[2] = fmaf(a.mu, mv[2], gv[2]); nv[3] = fmaf(a.mu, mv[3], gv[3]);
        __builtin_nontemporal_store(nv, (f32x4_t*)(mm.m + base));
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = a.nesterov ? fmaf(a.mu, nv[e], gv[e]) : nv[e];
      } else if (!mm.vec) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (col + e < mm.cols) {
            const float g = mm.g_bf16 ? bf16_to_f32(((const uint16_t*)mm.g)[base + e]) : ((const float*)mm.g)[base + e];
            const float n = fmaf(a.mu, mm.m[base + e], g);
            mm.m[base + e] = n;
            v[e] = a.nesterov ? fmaf(a.mu, n, g) : n;
          }
        }
      }
    }
    u16x4_t h;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      ss = fmaf(v[e], v[e], ss);
      h[e] = f32_to_bf16(v[e]);
      tile[lr][cx * 4 + e] = h[e];
    }
    // stored orientation (zeros in the padding)
    if (mm.x_orig) *(u16x4_t*)(mm.x_orig + (int64_t)row * mm.ld_orig + col) = h;
  }
  // block sum of squares (fixed order)
  for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off);
  if ((tid & 63) == 0) red[tid >> 6] = ss;
  __syncthreads();
  if (tid == 0) mm.partial[local] = (red[0] + red[1]) + (red[2] + red[3]);
  if (!mm.x_tr) return;
  // transposed orientation: output row tc*64 + jj, 16 consecutive elements
  const int jj = tid >> 2, i0 = (tid & 3) * 16;
  uint16_t o[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) o[e] = tile[i0 + e][jj];
  u32x4_t w0, w1;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    w0[e] = (uint32_t)o[2 * e] | ((uint32_t)o[2 * e + 1] << 16);
    w1[e] = (uint32_t)o[8 + 2 * e] | ((uint32_t)o[8 + 2 * e + 1] << 16);
  }
  uint16_t* dst = mm.x_tr + (int64_t)(tc * 64 + jj) * mm.ld_tr + tr * 64 + i0;
  *(u32x4_t*)dst = w0;
  *(u32x4_t*)(dst + 8) = w1;
}

hipError_t launch_momentum(const MomArgs& a, hipStream_t s) {
  if (a.total_blocks <= 0) return hipSuccess;
  momentum_kernel<<<a.total_blocks, 256, 0, s>>>(a);
  return hipGetLastError();
}

__global__ void __launch_bounds__(256) norm_finalize_kernel(const float* partial, int parts, int64_t stride,
                                                            float* scale, float eps) {
  __shared__ double red[256];
  const float* p = partial + (int64_t)blockIdx.x * stride;
  double acc = 0.0;
  // thread t adds elements t, t + 256, ... in that order; eight loads go out
  // before their adds so the latency is paid once per eight
  int i = threadIdx.x;
  for (; i + 7 * 256 < parts; i += 8 * 256) {
    float v[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) v[k] = p[i + k * 256];
#pragma unroll
    for (int k = 0; k < 8; ++k) acc += (double)v[k];
  }
  for (; i < parts; i += 256) acc += (double)p[i];
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) scale[blockIdx.x] = (float)(1.0 / (sqrt(red[0]) + (double)eps));
}

hipError_t launch_norm_finalize(const float* partial, int32_t parts, int64_t stride, float* scale,
                                int32_t nmat, float eps, hipStream_t s) {
  if (nmat <= 0) return hipSuccess;
  norm_finalize_kernel<<<nmat, 256, 0, s>>>(partial, parts, stride, scale, eps);
  return hipGetLastError();
}

typedef uint16_t u16x8_t __attribute__((ext_vector_type(8)));

// ---------------------------------------------------------------- update

__global__ void __launch_bounds__(256) update_kernel(const UpdArgs a) {
  __shared__ uint16_t ot[64][66];
  if (a.gamma_out && blockIdx.x == 0)   // the step's gamma output, from the same s_max
    for (int i = threadIdx.x; i < a.gamma_slots * a.heads; i += blockDim.x)
      a.gamma_out[i] = gamma_of(layer_s(a.s_max, i / a.heads, i % a.heads, a.heads, a.clip_global), a.tau);
  const int j = find_mat(a.mat, a.nmat, blockIdx.x);
  const UpdMat& u = a.mat[j];
  const int local = blockIdx.x - u.block_start;
  const int tr = local / u.tiles_c, tc = local - tr * u.tiles_c;
  const int tid = threadIdx.x, cx = tid & 15, ry = tid >> 4;
  const int col = tc * 64 + cx * 4;
  if (u.o_trans) {
    // O is stored [cols][rows] (a tall matrix iterates on its transpose):
    // stage the 64x64 tile through LDS. The buffer is padded to multiples of
    // 64 in both directions, so the whole tile is in bounds.
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int oc = tc * 64 + ry + 16 * k;        // W column = O row
      const u16x4_t v = *(const u16x4_t*)(u.o + (int64_t)oc * u.ld_o + tr * 64 + cx * 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) ot[ry + 16 * k][cx * 4 + e] = v[e];
    }
    __syncthreads();
  }
  if (u.vec8 && !u.o_trans) {
    // 8-element (16-byte) vectors: the 64x64 tile as 32 rows x 8 vectors,
    // two rows per thread, every load before the first store (W and O never
    // alias, but the compiler cannot know that and would serialise the rows)
    const int c8 = tc * 64 + (tid & 7) * 8, r8 = tr * 64 + (tid >> 3);
    if (c8 >= u.cols) return;
    u16x8_t ov[2], wv[2];
    bool in[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int row = r8 + 32 * k;
      in[k] = row < u.rows;
      if (in[k]) {
        ov[k] = *(const u16x8_t*)(u.o + (int64_t)row * u.ld_o + c8);
        wv[k] = *(const u16x8_t*)((const uint16_t*)u.w + (int64_t)row * u.ld + c8);
      }
    }
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      if (!in[k]) break;
      const int row = r8 + 32 * k;
      const float sc = row_clip_scale(u.clip, row, a.s_max, a.heads, a.tau, a.clip_global);
      if (u.o_out) *(u16x8_t*)(u.o_out + (int64_t)row * u.cols + c8) = ov[k];
      u16x8_t r;
#pragma unroll
      for (int e = 0; e < 8; ++e)
        r[e] = f32_to_bf16(fmaf(-u.lr_rms, bf16_to_f32(ov[k][e]), bf16_to_f32(wv[k][e]) * a.decay) * sc);
      *(u16x8_t*)((uint16_t*)u.w + (int64_t)row * u.ld + c8) = r;
    }
    return;
  }
  if (col >= u.cols) return;
  if (u.vec && !u.o_trans && u.w_bf16) {
    // the common case, with every load of the thread's four rows issued
    // before the first store (W and O never alias, but the compiler cannot
    // know that and would otherwise serialise the rows)
    u16x4_t ov[4], wv[4];
    bool in[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int row = tr * 64 + ry + 16 * k;
      in[k] = row < u.rows;
      if (in[k]) {
        ov[k] = *(const u16x4_t*)(u.o + (int64_t)row * u.ld_o + col);
        wv[k] = *(const u16x4_t*)((const uint16_t*)u.w + (int64_t)row * u.ld + col);
      }
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if (!in[k]) break;
      const int row = tr * 64 + ry + 16 * k;
      const float sc = row_clip_scale(u.clip, row, a.s_max, a.heads, a.tau, a.clip_global);
      if (u.o_out) *(u16x4_t*)(u.o_out + (int64_t)row * u.cols + col) = ov[k];
      u16x4_t r;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        r[e] = f32_to_bf16(fmaf(-u.lr_rms, bf16_to_f32(ov[k][e]), bf16_to_f32(wv[k][e]) * a.decay) * sc);
      *(u16x4_t*)((uint16_t*)u.w + (int64_t)row * u.ld + col) = r;
    }
    return;
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int row = tr * 64 + ry + 16 * k;
    if (row >= u.rows) break;
    const float sc = row_clip_scale(u.clip, row, a.s_max, a.heads, a.tau, a.clip_global);
    const int64_t wb = (int64_t)row * u.ld + col;
    const uint16_t* op = u.o + (int64_t)row * u.ld_o + col;
    u16x4_t ov;
    if (u.o_trans) {
#pragma unroll
      for (int e = 0; e < 4; ++e) ov[e] = ot[cx * 4 + e][ry + 16 * k];
    } else if (u.vec) {
      ov = *(const u16x4_t*)op;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) ov[e] = col + e < u.cols ? op[e] : (uint16_t)0;
    }
    if (u.vec) {
      float o[4] = {bf16_to_f32(ov[0]), bf16_to_f32(ov[1]), bf16_to_f32(ov[2]), bf16_to_f32(ov[3])};
      if (u.o_out) *(u16x4_t*)(u.o_out + (int64_t)row * u.cols + col) = ov;
      if (u.w_bf16) {
        uint16_t* wp = (uint16_t*)u.w + wb;
        const u16x4_t wv = *(const u16x4_t*)wp;
        u16x4_t r;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          r[e] = f32_to_bf16(fmaf(-u.lr_rms, o[e], bf16_to_f32(wv[e]) * a.decay) * sc);
        *(u16x4_t*)wp = r;
      } else {
        float* wp = (float*)u.w + wb;
        const f32x4_t wv = *(const f32x4_t*)wp;
        f32x4_t r;
#pragma unroll
        for (int e = 0; e < 4; ++e) r[e] = fmaf(-u.lr_rms, o[e], wv[e] * a.decay) * sc;
        *(f32x4_t*)wp = r;
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (col + e >= u.cols) break;
        const uint16_t ob = ov[e];
        const float o = bf16_to_f32(ob);
        if (u.o_out) u.o_out[(int64_t)row * u.cols + col + e] = ob;
        if (u.w_bf16) {
          uint16_t* wp = (uint16_t*)u.w + wb + e;
          *wp = f32_to_bf16(fmaf(-u.lr_rms, o, bf16_to_f32(*wp) * a.decay) * sc);
        } else {
          float* wp = (float*)u.w + wb + e;
          *wp = fmaf(-u.lr_rms, o, *wp * a.decay) * sc;
        }
      }
    }
  }
}

hipError_t launch_update(const UpdArgs& a, hipStream_t s) {
  if (a.total_blocks <= 0) return hipSuccess;
  update_kernel<<<a.total_blocks, 256, 0, s>>>(a);
  return hipGetLastError();
}

// ---------------------------------------------------------------- gamma / clip

__global__ void gamma_kernel(const float* s_max, float* gamma, int slots, int heads, float tau, int clip_global) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < slots * heads) gamma[i] = gamma_of(layer_s(s_max, i / heads, i % heads, heads, clip_global), tau);
}

hipError_t launch_gamma(const float* s_max, float* gamma, int32_t slots, int32_t heads, float tau,
                        int32_t clip_global, hipStream_t s) {
  const int n = slots * heads;
  if (n <= 0) return hipSuccess;
  gamma_kernel<<<(n + 255) / 256, 256, 0, s>>>(s_max, gamma, slots, heads, tau, clip_global);
  return hipGetLastError();
}

// Rows padded, unaligned or with a ragged width: grid.x 1024-column chunks,
// grid.y strides over rows, one element per access. Rows whose scale is
// exactly 1 are skipped before touching memory, so gamma = 1 heads stay
// bit-identical.
__global__ void __launch_bounds__(256) clip_apply_kernel(const ClipApplyArgs a) {
  for (int row = blockIdx.y; row < a.rows; row += gridDim.y) {
    const float sc = row_clip_scale(a.clip, row, a.s_max, a.heads, a.tau, 0);
    if (sc == 1.0f) continue;
    const int c0 = blockIdx.x * 1024 + threadIdx.x;
    for (int e = 0; e < 4; ++e) {
      const int col = c0 + e * 256;
      if (col >= a.cols) break;
      const int64_t i = (int64_t)row * a.ld + col;
      if (a.w_bf16) {
        uint16_t* w = (uint16_t*)a.w;
        w[i] = f32_to_bf16(bf16_to_f32(w[i]) * sc);
      } else {
        float* w = (float*)a.w;
        w[i] = w[i] * sc;
      }
    }
  }
}

// Rows of whole 16-byte vectors (8 bf16 or 4 fp32; 16-byte aligned base and
// row stride) of up to kMaxClipBatch matrices, numbered one matrix after the
// other. Each wave owns one row at a time (a grid-stride loop over rows), so
// the row's head, segment and factor are computed once, in scalar registers;
// a row whose factor is exactly 1 is neither read nor written. The row's
// vectors go 64 lanes wide, four per lane, every load before the first store.
constexpr int kClipVPL = 4;
__global__ void __launch_bounds__(256) clip_apply_vec_kernel(const ClipVecArgs a) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = (int64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t nwaves = (int64_t)gridDim.x * 4;
  for (int64_t r = wave; r < a.total_rows; r += nwaves) {
    int j = 0;
    for (int t = 1; t < a.nmat; ++t)
      if (r >= a.mat[t].row_start) j = t;
    const ClipVecMat& m = a.mat[j];
    const int row = (int)(r - m.row_start);
    const float sc = row_clip_scale(m.clip, row, a.s_max, a.heads, a.tau, 0);
    if (sc == 1.0f) continue;
    char* base = m.w + row * m.ld_bytes;
    for (int c0 = 0; c0 < m.vpr; c0 += 64 * kClipVPL) {
      u32x4_t v[kClipVPL];
#pragma unroll
      for (int k = 0; k < kClipVPL; ++k) {
        const int c = c0 + k * 64 + lane;
        if (c < m.vpr) v[k] = *(const u32x4_t*)(base + (int64_t)c * 16);
      }
#pragma unroll
      for (int k = 0; k < kClipVPL; ++k) {
        const int c = c0 + k * 64 + lane;
        if (c >= m.vpr) break;
        u32x4_t out;
        if (m.w_bf16) {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            out[e] = f32x2_to_bf16x2(bf16_to_f32((uint16_t)v[k][e]) * sc, bf16_to_f32((uint16_t)(v[k][e] >> 16)) * sc);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) out[e] = __float_as_uint(__uint_as_float(v[k][e]) * sc);
        }
        *(u32x4_t*)(base + (int64_t)c * 16) = out;
      }
    }
  }
}

bool clip_apply_vectorizable(const ClipApplyArgs& a) {
  const int es = a.w_bf16 ? 2 : 4, epv = 16 / es;
  return a.rows > 0 && a.cols > 0 && a.cols % epv == 0 && (a.ld * es) % 16 == 0 && ((uintptr_t)a.w & 15) == 0;
}

hipError_t launch_clip_apply_vec(const ClipVecArgs& a, hipStream_t s) {
  if (a.nmat <= 0 || a.total_rows <= 0) return hipSuccess;
  // one row per wave up to 32 waves per CU of the device; more rows loop
  const int64_t cap = (int64_t)device_cus() * 8;
  const int64_t blocks = std::min<int64_t>((a.total_rows + 3) / 4, cap);
  clip_apply_vec_kernel<<<(unsigned)blocks, 256, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_clip_apply(const ClipApplyArgs& a, hipStream_t s) {
  if (a.rows <= 0 || a.cols <= 0) return hipSuccess;
  dim3 grid((a.cols + 1023) / 1024, a.rows < 32768 ? a.rows : 32768);
  clip_apply_kernel<<<grid, 256, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace mc
