// AdamW for the parameters Muon does not cover (Notes on Muon blog,
// "Limitation": Muon optimises 2-D parameters only, the rest still need
// AdamW; Notes on Moonlight, "Scaling up Muon": the RMS-matched Muon update
// lets Muon and AdamW share the learning rate and the weight decay). The
// pages give no AdamW formula; this is the textbook form with bias
// correction and the same decoupled decay as the Muon update:
//   m <- b1 m + (1 - b1) g,  v <- b2 v + (1 - b2) g^2
//   p <- p (1 - lr wd) - lr (m c1) / (sqrt(v c2) + eps),  c_i = 1 / (1 - b_i^t)
//
// HBM-bound: one pass reads p, g, m, v and writes p, m, v (24 bytes per
// element for a bf16 parameter with fp32 gradient). A block covers 4096
// consecutive elements of one vector; each thread moves four consecutive
// elements per access (16-byte fp32, 8-byte bf16) when the vector's pointers
// allow, element by element otherwise and at a vector's ragged end. Whole
// blocks of vector accesses issue all their loads before the first store and
// stream non-temporally (each element is touched once per step).
#include <math.h>

#include "mc_internal.h"

namespace mc {

typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint16_t u16x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kAdamBlockElems = 4096;

__device__ __forceinline__ void adam_one(float& p, float g, float& m, float& v, const AdamArgs& a) {
  m = fmaf(a.beta1, m, a.one_m_beta1 * g);
  v = fmaf(a.beta2, v, a.one_m_beta2 * g * g);
  const float upd = (m * a.c1) / (sqrtf(v * a.c2) + a.eps);
  p = fmaf(-a.lr, upd, p * a.decay);
}

__global__ void __launch_bounds__(256) adamw_kernel(const AdamArgs a) {
  int j = 0;
  for (int t = 1; t < a.nvec; ++t)
    if ((int)blockIdx.x >= a.vec[t].block_start) j = t;
  const AdamVec& d = a.vec[j];
  const int64_t e0 = (int64_t)(blockIdx.x - d.block_start) * kAdamBlockElems;
  constexpr int KC = kAdamBlockElems / 1024;   // 1024-element chunks per block
  if (d.vec && e0 + kAdamBlockElems <= d.n) {
    // a whole block of vector accesses: every load of the four chunks goes
    // out before the first store (the buffers never alias, but the compiler
    // cannot know that), and each element is streamed once, non-temporally
    f32x4_t g4[KC], m4[KC], v4[KC], p4[KC];
#pragma unroll
    for (int k = 0; k < KC; ++k) {
      const int64_t e = e0 + k * 1024 + threadIdx.x * 4;
      if (d.g_bf16) {
        const u16x4_t gb = __builtin_nontemporal_load((const u16x4_t*)((const uint16_t*)d.g + e));
        g4[k] = f32x4_t{bf16_to_f32(gb[0]), bf16_to_f32(gb[1]), bf16_to_f32(gb[2]), bf16_to_f32(gb[3])};
      } else {
        g4[k] = __builtin_nontemporal_load((const f32x4_t*)((const float*)d.g + e));
      }
      m4[k] = __builtin_nontemporal_load((const f32x4_t*)(d.m + e));
      v4[k] = __builtin_nontemporal_load((const f32x4_t*)(d.v + e));
      if (d.p_bf16) {
        const u16x4_t pb = __builtin_nontemporal_load((const u16x4_t*)((const uint16_t*)d.p + e));
        p4[k] = f32x4_t{bf16_to_f32(pb[0]), bf16_to_f32(pb[1]), bf16_to_f32(pb[2]), bf16_to_f32(pb[3])};
      } else {
        p4[k] = __builtin_nontemporal_load((const f32x4_t*)((const float*)d.p + e));
      }
    }
#pragma unroll
    for (int k = 0; k < KC; ++k) {
      const int64_t e = e0 + k * 1024 + threadIdx.x * 4;
      float p[4] = {p4[k][0], p4[k][1], p4[k][2], p4[k][3]};
      float m[4] = {m4[k][0], m4[k][1], m4[k][2], m4[k][3]}, v[4] = {v4[k][0], v4[k][1], v4[k][2], v4[k][3]};
#pragma unroll
      for (int q = 0; q < 4; ++q) adam_one(p[q], g4[k][q], m[q], v[q], a);
      if (d.p_bf16) {
        const uint32_t lo = f32x2_to_bf16x2(p[0], p[1]), hi = f32x2_to_bf16x2(p[2], p[3]);
        __builtin_nontemporal_store(u32x2_t{lo, hi}, (u32x2_t*)((uint16_t*)d.p + e));
      } else {
        __builtin_nontemporal_store(f32x4_t{p[0], p[1], p[2], p[3]}, (f32x4_t*)((float*)d.p + e));
      }
      __builtin_nontemporal_store(f32x4_t{m[0], m[1], m[2], m[3]}, (f32x4_t*)(d.m + e));
      __builtin_nontemporal_store(f32x4_t{v[0], v[1], v[2], v[3]}, (f32x4_t*)(d.v + e));
    }
    return;
  }
#pragma unroll
  for (int k = 0; k < KC; ++k) {
    const int64_t e = e0 + k * 1024 + threadIdx.x * 4;
    if (e >= d.n) break;
    if (d.vec && e + 4 <= d.n) {
      f32x4_t g4;
      if (d.g_bf16) {
        const u16x4_t gb = *(const u16x4_t*)((const uint16_t*)d.g + e);
        g4 = f32x4_t{bf16_to_f32(gb[0]), bf16_to_f32(gb[1]), bf16_to_f32(gb[2]), bf16_to_f32(gb[3])};
      } else {
        g4 = *(const f32x4_t*)((const float*)d.g + e);
      }
      const f32x4_t m4i = *(const f32x4_t*)(d.m + e), v4i = *(const f32x4_t*)(d.v + e);
      float m[4] = {m4i[0], m4i[1], m4i[2], m4i[3]}, v[4] = {v4i[0], v4i[1], v4i[2], v4i[3]};
      if (d.p_bf16) {
        uint16_t* pp = (uint16_t*)d.p + e;
        const u16x4_t pb = *(const u16x4_t*)pp;
        float p[4] = {bf16_to_f32(pb[0]), bf16_to_f32(pb[1]), bf16_to_f32(pb[2]), bf16_to_f32(pb[3])};
#pragma unroll
        for (int q = 0; q < 4; ++q) adam_one(p[q], g4[q], m[q], v[q], a);
        const uint32_t lo = f32x2_to_bf16x2(p[0], p[1]), hi = f32x2_to_bf16x2(p[2], p[3]);
        *(uint2*)pp = make_uint2(lo, hi);
      } else {
        float* pp = (float*)d.p + e;
        const f32x4_t p4 = *(const f32x4_t*)pp;
        float p[4] = {p4[0], p4[1], p4[2], p4[3]};
#pragma unroll
        for (int q = 0; q < 4; ++q) adam_one(p[q], g4[q], m[q], v[q], a);
        *(f32x4_t*)pp = f32x4_t{p[0], p[1], p[2], p[3]};
      }
      *(f32x4_t*)(d.m + e) = f32x4_t{m[0], m[1], m[2], m[3]};
      *(f32x4_t*)(d.v + e) = f32x4_t{v[0], v[1], v[2], v[3]};
    } else {
      for (int q = 0; q < 4 && e + q < d.n; ++q) {
        const int64_t i = e + q;
        const float g = d.g_bf16 ? bf16_to_f32(((const uint16_t*)d.g)[i]) : ((const float*)d.g)[i];
        float m = d.m[i], v = d.v[i];
        float p = d.p_bf16 ? bf16_to_f32(((const uint16_t*)d.p)[i]) : ((const float*)d.p)[i];
        adam_one(p, g, m, v, a);
        if (d.p_bf16) ((uint16_t*)d.p)[i] = f32_to_bf16(p);
        else ((float*)d.p)[i] = p;
        d.m[i] = m;
        d.v[i] = v;
      }
    }
  }
}

int64_t adamw_blocks(int64_t n) { return (n + kAdamBlockElems - 1) / kAdamBlockElems; }

hipError_t launch_adamw(const AdamArgs& a, hipStream_t s) {
  if (a.total_blocks <= 0) return hipSuccess;
  adamw_kernel<<<a.total_blocks, 256, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace mc
