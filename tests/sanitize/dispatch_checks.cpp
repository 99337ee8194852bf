// Host-only checks of the library's argument validation and workspace
// planning, linked against a dispatcher built with AddressSanitizer and
// UndefinedBehaviorSanitizer (host code only). Every call here either fails
// validation before any HIP call or is a pure host query, so the fake device
// addresses below are never dereferenced and no kernel is launched.
// Exit status: 0 when every call returned the expected status.
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <vector>

#include "muonclip.h"

static int g_fail = 0;

static void expect(const char* what, int got, int want) {
  if (got != want) {
    fprintf(stderr, "FAIL %s: status %d, expected %d (%s)\n", what, got, want, mc_last_error());
    ++g_fail;
  }
}

static mc_matrix fake(int64_t rows, int64_t cols, int32_t w_dtype = MC_BF16) {
  mc_matrix m;
  memset(&m, 0, sizeof m);
  m.w = (void*)0x10000000;
  m.g = (const void*)0x20000000;
  m.m = (float*)0x30000000;
  m.rows = rows; m.cols = cols; m.ld = cols;
  m.w_dtype = w_dtype; m.g_dtype = MC_F32;
  m.clip_slot = -1;
  return m;
}

static mc_matrix clipped(int64_t rows, int64_t cols, int32_t period, int nseg, mc_segment s0, mc_segment s1) {
  mc_matrix m = fake(rows, cols);
  m.clip_slot = 0; m.period = period; m.nseg = nseg; m.seg[0] = s0; m.seg[1] = s1;
  return m;
}

int main() {
  mc_hparams hp;
  mc_default_hparams(&hp);
  const float* smax = (const float*)0x40000000;
  float* gamma = (float*)0x50000000;
  void* ws = (void*)0x60000000;

  // ---- planning: workspace queries over the configurations' shape sets
  {
    std::vector<mc_matrix> mats;
    for (int e = 0; e < 385; ++e) {
      mats.push_back(fake(7168, 2048));
      mats.push_back(fake(7168, 2048));
      mats.push_back(fake(2048, 7168));
    }
    const int64_t mla[5][2] = {{1536, 7168}, {12288, 1536}, {576, 7168}, {16384, 512}, {7168, 8192}};
    for (auto& s : mla) mats.push_back(fake(s[0], s[1]));
    mats.push_back(fake(7168, 18432)); mats.push_back(fake(7168, 18432)); mats.push_back(fake(18432, 7168));
    mats.push_back(fake(1, 7)); mats.push_back(fake(7, 1)); mats.push_back(fake(100, 37));
    mats.push_back(fake(256, 512, MC_F32)); mats.push_back(fake(64, 64, MC_F32));
    const size_t full = mc_workspace_size(mats.data(), (int32_t)mats.size(), &hp);
    const size_t minimal = mc_workspace_min_size(mats.data(), (int32_t)mats.size(), &hp);
    if (!(full > 0 && minimal > 0 && minimal <= full)) {
      fprintf(stderr, "FAIL workspace sizes %zu / %zu\n", full, minimal);
      ++g_fail;
    }
    for (size_t i = 0; i < mats.size(); i += 97) {
      const size_t one = mc_workspace_size(&mats[i], 1, &hp);
      if (one == 0 || one > full) { fprintf(stderr, "FAIL single workspace %zu\n", one); ++g_fail; }
    }
    expect("noalloc beyond scratch", muonclip_step_noalloc(mats.data(), (int32_t)mats.size(), &hp, nullptr, 0, 0,
                                                           nullptr, nullptr), MC_ERR_WORKSPACE);
    if (mc_workspace_size(nullptr, 1, &hp) != 0) { fprintf(stderr, "FAIL workspace of NULL mats\n"); ++g_fail; }
  }

  // ---- muonclip_step validation
  mc_matrix ok = fake(256, 512);
  expect("NULL mats", muonclip_step(nullptr, 1, &hp, nullptr, 0, 0, nullptr, ws, 1 << 30, nullptr), MC_ERR_NULL);
  expect("n < 0", muonclip_step(&ok, -1, &hp, nullptr, 0, 0, nullptr, ws, 1 << 30, nullptr), MC_ERR_SHAPE);
  expect("NULL hparams", muonclip_step(&ok, 1, nullptr, nullptr, 0, 0, nullptr, ws, 1 << 30, nullptr), MC_ERR_NULL);
  {
    mc_hparams h = hp; h.lr = NAN;
    expect("NaN lr", muonclip_step(&ok, 1, &h, nullptr, 0, 0, nullptr, ws, 1 << 30, nullptr), MC_ERR_HPARAM);
    h = hp; h.ns_steps = 0;
    expect("ns_steps 0", muonclip_step(&ok, 1, &h, nullptr, 0, 0, nullptr, ws, 1 << 30, nullptr), MC_ERR_HPARAM);
    h = hp; h.ns_steps = 17;
    expect("ns_steps 17", muonclip_step(&ok, 1, &h, nullptr, 0, 0, nullptr, ws, 1 << 30, nullptr), MC_ERR_HPARAM);
    h = hp; h.tau = 0.0f;
    expect("tau 0", muonclip_step(&ok, 1, &h, nullptr, 0, 0, nullptr, ws, 1 << 30, nullptr), MC_ERR_HPARAM);
    h = hp; h.ns_eps = -1.0f;
    expect("eps < 0", muonclip_step(&ok, 1, &h, nullptr, 0, 0, nullptr, ws, 1 << 30, nullptr), MC_ERR_HPARAM);
    h = hp; h.nesterov = 2;
    expect("nesterov 2", muonclip_step(&ok, 1, &h, nullptr, 0, 0, nullptr, ws, 1 << 30, nullptr), MC_ERR_HPARAM);
    h = hp; h.clip_global = -1;
    expect("clip_global -1", muonclip_step(&ok, 1, &h, nullptr, 0, 0, nullptr, ws, 1 << 30, nullptr), MC_ERR_HPARAM);
  }
  {
    mc_matrix m = ok; m.w = nullptr;
    expect("NULL w", muonclip_step(&m, 1, &hp, nullptr, 0, 0, nullptr, ws, 1 << 30, nullptr), MC_ERR_NULL);
    m = ok; m.g = nullptr;
    expect("NULL g", muonclip_step(&m, 1, &hp, nullptr, 0, 0, nullptr, ws, 1 << 30, nullptr), MC_ERR_NULL);
    m = ok; m.rows = 0;
    expect("rows 0", muonclip_step(&m, 1, &hp, nullptr, 0, 0, nullptr, ws, 1 << 30, nullptr), MC_ERR_SHAPE);
    m = ok; m.cols = ((int64_t)1 << 20) + 1; m.ld = m.cols;
    expect("cols > 2^20", muonclip_step(&m, 1, &hp, nullptr, 0, 0, nullptr, ws, 1 << 30, nullptr), MC_ERR_SHAPE);
    m = fake(65536, 65536);
    expect("2^32 elements", muonclip_step(&m, 1, &hp, nullptr, 0, 0, nullptr, ws, 1 << 30, nullptr), MC_ERR_SHAPE);
    m = ok; m.ld = 100;
    expect("ld < cols", muonclip_step(&m, 1, &hp, nullptr, 0, 0, nullptr, ws, 1 << 30, nullptr), MC_ERR_SHAPE);
    m = ok; m.w_dtype = 7;
    expect("bad w dtype", muonclip_step(&m, 1, &hp, nullptr, 0, 0, nullptr, ws, 1 << 30, nullptr), MC_ERR_DTYPE);
    m = ok; m.g_dtype = 9;
    expect("bad g dtype", muonclip_step(&m, 1, &hp, nullptr, 0, 0, nullptr, ws, 1 << 30, nullptr), MC_ERR_DTYPE);
    m = ok; m.w = (void*)0x10000001;
    expect("misaligned w", muonclip_step(&m, 1, &hp, nullptr, 0, 0, nullptr, ws, 1 << 30, nullptr), MC_ERR_ALIGN);
    m = ok; m.m = (float*)0x30000002;
    expect("misaligned m", muonclip_step(&m, 1, &hp, nullptr, 0, 0, nullptr, ws, 1 << 30, nullptr), MC_ERR_ALIGN);
  }
  {
    const mc_segment s_all = {0, 16, 0.5f}, none = {0, 0, 0.0f};
    mc_matrix m = clipped(64, 64, 16, 1, s_all, none);
    expect("s_max with 0 slots", muonclip_step(&m, 1, &hp, smax, 0, 4, nullptr, ws, 1 << 30, nullptr), MC_ERR_SHAPE);
    mc_matrix m1 = m; m1.clip_slot = 1;
    expect("clip_slot >= slots", muonclip_step(&m1, 1, &hp, smax, 1, 4, gamma, ws, 1 << 30, nullptr), MC_ERR_SHAPE);
    expect("more head blocks than heads", muonclip_step(&m, 1, &hp, smax, 1, 2, nullptr, ws, 1 << 30, nullptr),
           MC_ERR_SHAPE);
    expect("gamma without s_max", muonclip_step(&m, 1, &hp, nullptr, 1, 4, gamma, ws, 1 << 30, nullptr), MC_ERR_NULL);
    m = clipped(64, 64, 24, 1, s_all, none);
    expect("rows % period", muonclip_step(&m, 1, &hp, smax, 1, 4, nullptr, ws, 1 << 30, nullptr), MC_ERR_SHAPE);
    m = clipped(64, 64, 16, 1, mc_segment{8, 16, 0.5f}, none);
    expect("segment past period", muonclip_step(&m, 1, &hp, smax, 1, 4, nullptr, ws, 1 << 30, nullptr), MC_ERR_SHAPE);
    m = clipped(64, 64, 16, 2, mc_segment{0, 10, 0.5f}, mc_segment{8, 8, 1.0f});
    expect("overlapping segments", muonclip_step(&m, 1, &hp, smax, 1, 4, nullptr, ws, 1 << 30, nullptr), MC_ERR_SHAPE);
    m = clipped(64, 64, 16, 1, mc_segment{0, 16, 0.0f}, none);
    expect("expo 0", muonclip_step(&m, 1, &hp, smax, 1, 4, nullptr, ws, 1 << 30, nullptr), MC_ERR_HPARAM);
    m = clipped(64, 64, 16, 3, s_all, none);
    expect("nseg 3", muonclip_step(&m, 1, &hp, smax, 1, 4, nullptr, ws, 1 << 30, nullptr), MC_ERR_SHAPE);
  }
  expect("NULL workspace", muonclip_step(&ok, 1, &hp, nullptr, 0, 0, nullptr, nullptr, 1 << 30, nullptr),
         MC_ERR_WORKSPACE);
  expect("misaligned workspace", muonclip_step(&ok, 1, &hp, nullptr, 0, 0, nullptr, (void*)0x60000010, 1 << 30,
                                               nullptr), MC_ERR_WORKSPACE);
  expect("small workspace", muonclip_step(&ok, 1, &hp, nullptr, 0, 0, nullptr, ws, 4096, nullptr), MC_ERR_WORKSPACE);
  expect("overlapped: bad hparams", muonclip_step_overlapped(&ok, 1, nullptr, nullptr, 0, 0, nullptr, ws, 1 << 30,
                                                             nullptr, nullptr), MC_ERR_NULL);

  // ---- max_logits_per_head / attention_forward / qk_clip_apply / adamw_step
  const int64_t st3[3] = {4096 * 16 * 128, 16 * 128, 128}, st2[2] = {4096 * 64, 64};
  const void* q = (const void*)0x70000000;
  float* out = (float*)0x80000000;
  expect("max_logits NULL out", max_logits_per_head(q, q, nullptr, MC_BF16, 1, 4096, 16, 128, 128, 0, st3, st3,
                                                    nullptr, 1, 0.088f, nullptr, nullptr), MC_ERR_NULL);
  expect("max_logits d_q mismatch", max_logits_per_head(q, q, nullptr, MC_BF16, 1, 4096, 16, 192, 128, 0, st3, st3,
                                                        nullptr, 1, 0.07f, out, nullptr), MC_ERR_SHAPE);
  expect("max_logits bad scale", max_logits_per_head(q, q, nullptr, MC_BF16, 1, 4096, 16, 128, 128, 0, st3, st3,
                                                     nullptr, 1, -1.0f, out, nullptr), MC_ERR_HPARAM);
  expect("max_logits shared NULL", max_logits_per_head(q, q, nullptr, MC_BF16, 1, 4096, 16, 192, 128, 64, st3, st3,
                                                       st2, 1, 0.07f, out, nullptr), MC_ERR_NULL);
  expect("max_logits dtype", max_logits_per_head(q, q, nullptr, 5, 1, 4096, 16, 128, 128, 0, st3, st3, nullptr, 1,
                                                 0.088f, out, nullptr), MC_ERR_DTYPE);
  expect("attention d_v", attention_forward(q, q, nullptr, q, (void*)q, nullptr, nullptr, 1, 4096, 16, 128, 128, 0,
                                            64, st3, st3, nullptr, st3, st3, 1, 0.088f, nullptr), MC_ERR_SHAPE);
  expect("attention NULL o", attention_forward(q, q, nullptr, q, nullptr, nullptr, nullptr, 1, 4096, 16, 128, 128, 0,
                                               128, st3, st3, nullptr, st3, st3, 1, 0.088f, nullptr), MC_ERR_NULL);
  {
    const mc_segment s_all = {0, 16, 0.5f}, none = {0, 0, 0.0f};
    mc_matrix m = clipped(64, 64, 16, 1, s_all, none);
    expect("clip NULL s_max", qk_clip_apply(&m, 1, nullptr, 1, 4, 100.0f, nullptr, nullptr), MC_ERR_NULL);
    expect("clip tau inf", qk_clip_apply(&m, 1, smax, 1, 4, INFINITY, nullptr, nullptr), MC_ERR_HPARAM);
    expect("clip heads 0", qk_clip_apply(&m, 1, smax, 1, 0, 100.0f, nullptr, nullptr), MC_ERR_SHAPE);
    expect("clip slot out of range", qk_clip_apply(&m, 1, smax, 0, 4, 100.0f, nullptr, nullptr), MC_ERR_SHAPE);
  }
  {
    mc_adamw_hparams ah;
    mc_default_adamw_hparams(&ah);
    mc_vector v;
    memset(&v, 0, sizeof v);
    v.p = (void*)0x90000000; v.g = (const void*)0xA0000000; v.m = (float*)0xB0000000; v.v = (float*)0xC0000000;
    v.n = 1000; v.p_dtype = MC_BF16; v.g_dtype = MC_F32;
    mc_adamw_hparams bad = ah; bad.beta1 = 1.0f;
    expect("adamw beta1 1", adamw_step(&v, 1, &bad, nullptr), MC_ERR_HPARAM);
    bad = ah; bad.step = 0;
    expect("adamw step 0", adamw_step(&v, 1, &bad, nullptr), MC_ERR_HPARAM);
    mc_vector w = v; w.m = nullptr;
    expect("adamw NULL m", adamw_step(&w, 1, &ah, nullptr), MC_ERR_NULL);
    w = v; w.p = (void*)0x90000001;
    expect("adamw misaligned", adamw_step(&w, 1, &ah, nullptr), MC_ERR_ALIGN);
    w = v; w.n = -1;
    expect("adamw n < 0", adamw_step(&w, 1, &ah, nullptr), MC_ERR_SHAPE);
  }
  expect("profile read with nothing recorded", mc_profile_read(nullptr, 0), 0);
  if (g_fail) {
    fprintf(stderr, "%d checks failed\n", g_fail);
    return 1;
  }
  printf("dispatch checks ok\n");
  return 0;
}
