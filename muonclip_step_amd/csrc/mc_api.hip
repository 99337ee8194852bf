// Host dispatcher and C ABI of the MuonClip library (see include/muonclip.h).
//
// muonclip_step: matrices are grouped by (m, n) = (min, max) of their shape;
// each group runs in waves of as many matrices as the workspace holds. Per
// wave, on the caller's stream:
//   momentum_kernel   M <- mu M + G, norm partials, bf16 X0 ([m][n]: M or M^T)
//   norm_finalize     s = 1 / (||M||_F + eps)
//   5 x { Gram  A = s0^2 X X^T          -> bf16 A_hi (+ A_lo if m < 1024)
//         Poly  P = a I + b A + c A A   -> P_hi (+ P_lo if m < 1024)
//         Apply X' = s0 P X             -> X' (ping-pong; last step: O) }
//   W <- clip_row ((1 - lr wd) W - lr rms sqrt(max) O): in the last Apply's
//   epilogue, or by update_kernel for waves that cannot fuse it
// (s0 = s on the first step, 1 after). The apply is the quintic step of the
// Notes on Muon blog, "Newton-Schulz", written as X' = (aI + bA + cA^2) X.
// Groups with n >= 2m (m >= 1024) run the first kGramHead iterations on
// m x m products instead (the Gram-space head, gram_head and run_wave).
// Operands are bf16, accumulation and every epilogue fp32. The Poly
// evaluates the polynomial at the matrix its product reads: P = a I +
// b A_hi + c A_hi A_hi in fp32 with A_hi the bf16 Gram, so P is an exact
// polynomial of one matrix (with b A taken from the fp32 Gram instead, the
// two terms see different matrices, and a CPU emulation of the iteration
// gave 1.2-2.5x larger errors against the fp64 iteration on full-rank
// inputs). For m < 1024 the Gram matrix and the polynomial enter their
// products as hi + lo bf16 pairs (3 and 2 MFMA passes; the b A term then
// reads the pair too), which keeps those small-m shapes well inside the
// 2e-2 relative Frobenius bound.
#include <math.h>
#include <cmath>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/muonclip.h"
#include "mc_internal.h"

using namespace mc;

namespace mc {

// Compute units of the current device, read once per device; 256 (MI355X)
// when the runtime cannot tell (no device: host-only workspace queries).
int device_cus() {
  static std::mutex mu;
  static std::map<int, int> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) { (void)hipGetLastError(); return 256; }
  std::lock_guard<std::mutex> lk(mu);
  auto it = cache.find(dev);
  if (it != cache.end()) return it->second;
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) {
    (void)hipGetLastError();
    cus = 256;
  }
  cache[dev] = cus;
  return cus;
}

}  // namespace mc

namespace {

thread_local std::string g_err;

mc_status fail(mc_status code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

constexpr size_t kAlign = 256;
inline size_t align_up(size_t x) { return (x + kAlign - 1) & ~(kAlign - 1); }
inline int64_t round64(int64_t x) { return (x + 63) / 64 * 64; }
constexpr int kWaveCap = 64;
constexpr int kSplitThreshold = 1024;   // m below this: hi/lo operand pairs

// ---------------------------------------------------------------- profiling

enum Family {
  F_MOMENTUM = 0, F_NORM, F_GEMM, F_SPLITK, F_UPDATE, F_GAMMA, F_CLIP,
  F_ML_INIT, F_ML, F_ADAMW, F_ATTN, F_COUNT
};
const char* kFamilyNames[F_COUNT] = {"momentum_norm", "norm_finalize", "ns_gemm", "splitk_reduce",
                                     "update_clip", "gamma", "clip_apply", "max_logits_init",
                                     "max_logits", "adamw", "attention"};

struct ProfRec { int fam; hipEvent_t a, b; double flops, bytes; };
std::mutex g_prof_mu;
std::atomic<bool> g_prof{false};   // written under g_prof_mu, read without it
std::vector<ProfRec> g_recs;
std::vector<hipEvent_t> g_pool;
size_t g_pool_used = 0;

bool profiling_on() { return g_prof.load(); }

hipEvent_t pool_event() {
  if (g_pool_used == g_pool.size()) {
    hipEvent_t e;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    g_pool.push_back(e);
  }
  return g_pool[g_pool_used++];
}

struct Prof {
  int fam; hipStream_t s; double flops, bytes; hipEvent_t a = nullptr, b = nullptr;
  Prof(int f, hipStream_t st, double fl, double by) : fam(f), s(st), flops(fl), bytes(by) {
    if (!g_prof) return;
    std::lock_guard<std::mutex> lk(g_prof_mu);
    a = pool_event(); b = pool_event();
    if (a) (void)hipEventRecord(a, s);
  }
  ~Prof() {
    if (!a || !b) return;
    (void)hipEventRecord(b, s);
    std::lock_guard<std::mutex> lk(g_prof_mu);
    g_recs.push_back({fam, a, b, flops, bytes});
  }
};

// ---------------------------------------------------------------- validation

bool dtype_ok(int32_t d) { return d == MC_F32 || d == MC_BF16; }
size_t dtype_size(int32_t d) { return d == MC_F32 ? 4 : 2; }
bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

mc_status check_hparams(const mc_hparams* hp) {
  if (!hp) return fail(MC_ERR_NULL, "hparams is NULL");
  const float v[] = {hp->lr, hp->mu, hp->weight_decay, hp->rms_scale, hp->tau,
                     hp->ns_a, hp->ns_b, hp->ns_c, hp->ns_eps};
  for (float x : v)
    if (!isfinite(x)) return fail(MC_ERR_HPARAM, "hyper-parameters must be finite");
  if (hp->ns_steps < 1 || hp->ns_steps > 16) return fail(MC_ERR_HPARAM, "ns_steps must be in 1..16 (got %d)", hp->ns_steps);
  if (hp->ns_eps < 0.0f) return fail(MC_ERR_HPARAM, "ns_eps must be >= 0");
  if (hp->tau <= 0.0f) return fail(MC_ERR_HPARAM, "tau must be > 0");
  if (hp->nesterov != 0 && hp->nesterov != 1) return fail(MC_ERR_HPARAM, "nesterov must be 0 or 1");
  if (hp->clip_global != 0 && hp->clip_global != 1) return fail(MC_ERR_HPARAM, "clip_global must be 0 or 1");
  return MC_OK;
}

mc_status check_clip(const mc_matrix& m, int i, int32_t slots, int32_t heads, bool need_slots) {
  if (m.clip_slot < 0) return MC_OK;
  if (need_slots && m.clip_slot >= slots)
    return fail(MC_ERR_SHAPE, "matrix %d: clip_slot %d >= slots %d", i, m.clip_slot, slots);
  if (m.period <= 0 || m.rows % m.period != 0)
    return fail(MC_ERR_SHAPE, "matrix %d: rows %lld not a multiple of period %d", i, (long long)m.rows, m.period);
  if (need_slots && m.rows / m.period > heads)
    return fail(MC_ERR_SHAPE, "matrix %d: %lld head blocks > heads %d", i, (long long)(m.rows / m.period), heads);
  if (m.nseg < 0 || m.nseg > 2) return fail(MC_ERR_SHAPE, "matrix %d: nseg must be 0..2", i);
  for (int s = 0; s < m.nseg; ++s) {
    const mc_segment& g = m.seg[s];
    if (g.offset < 0 || g.length <= 0 || g.offset + g.length > m.period)
      return fail(MC_ERR_SHAPE, "matrix %d: segment %d outside the head period", i, s);
    if (!(g.expo > 0.0f) || !isfinite(g.expo)) return fail(MC_ERR_HPARAM, "matrix %d: segment expo must be > 0", i);
  }
  if (m.nseg == 2) {
    const mc_segment &a = m.seg[0], &b = m.seg[1];
    if (a.offset < b.offset + b.length && b.offset < a.offset + a.length)
      return fail(MC_ERR_SHAPE, "matrix %d: segments overlap", i);
  }
  return MC_OK;
}

mc_status check_matrix_common(const mc_matrix& m, int i) {
  if (!m.w) return fail(MC_ERR_NULL, "matrix %d: w is NULL", i);
  if (m.rows <= 0 || m.cols <= 0) return fail(MC_ERR_SHAPE, "matrix %d: rows and cols must be >= 1", i);
  if (m.rows > (1 << 20) || m.cols > (1 << 20)) return fail(MC_ERR_SHAPE, "matrix %d: dimension above 2^20", i);
  // the Newton-Schulz buffers (rows and cols padded to 64) are addressed
  // with 32-bit element offsets inside one matrix
  if (((m.rows + 63) / 64 * 64) * ((m.cols + 63) / 64 * 64) >= ((int64_t)1 << 31))
    return fail(MC_ERR_SHAPE, "matrix %d: %lld x %lld exceeds 2^31 elements", i, (long long)m.rows, (long long)m.cols);
  if (m.ld < m.cols) return fail(MC_ERR_SHAPE, "matrix %d: ld %lld < cols %lld", i, (long long)m.ld, (long long)m.cols);
  if (!dtype_ok(m.w_dtype)) return fail(MC_ERR_DTYPE, "matrix %d: w_dtype %d", i, m.w_dtype);
  if (!aligned(m.w, dtype_size(m.w_dtype))) return fail(MC_ERR_ALIGN, "matrix %d: w misaligned", i);
  return MC_OK;
}

mc_status check_matrices_step(const mc_matrix* mats, int32_t n, int32_t slots, int32_t heads, bool have_smax) {
  if (n < 0) return fail(MC_ERR_SHAPE, "n < 0");
  if (n > 0 && !mats) return fail(MC_ERR_NULL, "mats is NULL");
  for (int i = 0; i < n; ++i) {
    const mc_matrix& m = mats[i];
    mc_status st = check_matrix_common(m, i);
    if (st) return st;
    if (!m.g || !m.m) return fail(MC_ERR_NULL, "matrix %d: g or m is NULL", i);
    if (!dtype_ok(m.g_dtype)) return fail(MC_ERR_DTYPE, "matrix %d: g_dtype %d", i, m.g_dtype);
    if (!aligned(m.g, dtype_size(m.g_dtype)) || !aligned(m.m, 4)) return fail(MC_ERR_ALIGN, "matrix %d: g or m misaligned", i);
    if (m.o_out && !aligned(m.o_out, 2)) return fail(MC_ERR_ALIGN, "matrix %d: o_out misaligned", i);
    if (have_smax) { st = check_clip(m, i, slots, heads, true); if (st) return st; }
    else if (m.clip_slot >= 0) { st = check_clip(m, i, 0, 0, false); if (st) return st; }
  }
  return MC_OK;
}

// ---------------------------------------------------------------- planning

struct Group {
  int64_t m, n, mp, np;
  bool split;
  std::vector<int> idx;
};

std::vector<Group> make_groups(const mc_matrix* mats, int32_t n) {
  std::vector<Group> gs;
  std::map<std::pair<int64_t, int64_t>, size_t> where;
  for (int i = 0; i < n; ++i) {
    const int64_t m = std::min(mats[i].rows, mats[i].cols), nn = std::max(mats[i].rows, mats[i].cols);
    auto key = std::make_pair(m, nn);
    auto it = where.find(key);
    if (it == where.end()) {
      Group g;
      g.m = m; g.n = nn; g.mp = round64(m); g.np = round64(nn);
      g.split = m < kSplitThreshold;
      where[key] = gs.size();
      gs.push_back(g);
      it = where.find(key);
    }
    gs[it->second].idx.push_back(i);
  }
  return gs;
}

struct GemmPlan { GemmTile tile; int tiles_m, tiles_n, splits, kt_per_split; size_t partial_bytes; };

// Tile size and split-K for one batched product. 256x256 tiles when they
// cover at least half the CUs, else 128x128 (64x64 below 128 rows);
// K is split only when the tiles alone cannot fill the chip, keeping every
// split at least 8 k-stages long. Symmetric products count upper tiles only.
GemmPlan plan_gemm(int cus, int64_t M, int64_t N, int ktiles, int batch, bool sym, bool reads_cin = false,
                   bool pair_out = false) {
  GemmPlan p{};
  auto count = [&](int d) {
    const int tm = (int)((M + d - 1) / d), tn = (int)((N + d - 1) / d);
    return (sym ? tm * (tm + 1) / 2 : tm * tn) * batch;
  };
  // 256 tiles run ~15-25% faster per tile than 128 (half the load bytes per
  // flop) and win as soon as they cover half the CUs, the Poly step (whose
  // epilogue also reads A) included since launches of at most one tile per
  // CU run eight waves per tile (measured against 128 tiles: 4 x 2048^2
  // chains 2.5 % faster, MLA layer step 5 % faster)
  const int need256 = cus / 2;
  // (the 256 tile of the Poly step with a hi/lo output pair needs more
  // registers than a wave has, so that case stays on 128 tiles)
  if (M >= 256 && N >= 256 && count(256) >= need256 && !(reads_cin && pair_out)) p.tile = TILE_256;
  else if (M >= 128 && N >= 128) p.tile = TILE_128;
  else p.tile = TILE_64;
  const int d = gemm_tile_dim(p.tile);
  p.tiles_m = (int)((M + d - 1) / d);
  p.tiles_n = (int)((N + d - 1) / d);
  const int tiles = count(d);
  int splits = 1;
  if (tiles < cus / 2 && ktiles >= 16) {
    // split-K runs the full (non-symmetric) tile set
    const int full = p.tiles_m * p.tiles_n * batch;
    // one wave of work items: a second wave of smaller splits measured
    // slower, its extra fp32 partials costing the finish more than the
    // better balance gained (MLA layer 9.29 -> 9.23 ms)
    splits = std::min((cus + full - 1) / full, ktiles / 8);
    splits = std::max(splits, 1);
  }
  p.kt_per_split = (ktiles + splits - 1) / splits;
  p.splits = (ktiles + p.kt_per_split - 1) / p.kt_per_split;
  p.partial_bytes = p.splits > 1 ? (size_t)p.splits * batch * M * N * 4 : 0;
  return p;
}

struct WavePlan {
  int nb;
  size_t off_x0, off_x1, off_ahi, off_alo, off_phi, off_plo, off_part, off_scale, off_splitk;
  size_t bytes;
  int64_t mom_blocks;          // momentum blocks per matrix
  GemmPlan gram, poly, apply;
  int kt_gram, kt_poly, kt_apply;
  // the Gram hands A_hi to the Poly epilogue a second time, in fragment
  // order (off_alo), which the epilogue reads in 1 KB runs: groups without
  // operand pairs whose two symmetric products run unsplit on the same tiles
  // (other groups without pairs read A_hi itself, at the transposed position)
  bool frag;
};

WavePlan plan_wave(const Group& g, int nb, int cus) {
  WavePlan w{};
  w.nb = nb;
  const size_t mp = (size_t)g.mp, np = (size_t)g.np;
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t o = off; off += align_up(bytes); return o; };
  w.kt_gram = (int)(np / kGemmBK);
  w.kt_poly = (int)(mp / kGemmBK) * (g.split ? 3 : 1);
  w.kt_apply = (int)(mp / kGemmBK) * (g.split ? 2 : 1);
  w.gram = plan_gemm(cus, g.mp, g.mp, w.kt_gram, nb, true);
  w.poly = plan_gemm(cus, g.mp, g.mp, w.kt_poly, nb, true, true, g.split);
  w.apply = plan_gemm(cus, g.mp, g.np, w.kt_apply, nb, false);
  w.frag = !g.split && w.gram.tile == w.poly.tile && w.gram.splits == 1 && w.poly.splits == 1;
  w.off_x0 = take(nb * mp * np * 2);
  w.off_x1 = take(nb * mp * np * 2);
  w.off_ahi = take(nb * mp * mp * 2);
  w.off_alo = take(nb * mp * mp * 2);
  w.off_phi = take(nb * mp * mp * 2);
  w.off_plo = g.split ? take(nb * mp * mp * 2) : 0;
  w.mom_blocks = (int64_t)(mp / 64) * (int64_t)(np / 64);
  w.off_part = take(nb * (size_t)w.mom_blocks * 4);
  w.off_scale = take(nb * 4);
  const size_t sk = std::max(w.gram.partial_bytes, std::max(w.poly.partial_bytes, w.apply.partial_bytes));
  w.off_splitk = sk ? take(sk) : 0;
  w.bytes = off;
  return w;
}

// Whether a wave runs its first kGramHead Newton-Schulz iterations in Gram
// space (each iteration after the first trades a Gram and an apply, both
// n-sized, for three m x m products): for groups with n >= 2 m, where the
// n-sized products saved outweigh the m x m products added, without hi/lo
// operand pairs (A reaches the Poly as A_hi, through the fragment-order copy
// or, when the symmetric products are split or tiled differently, as
// itself), and with an unsplit apply (whose epilogue adds the identity
// part of the accumulated product). At least one iteration follows it, so
// the fused update stays on an ordinary apply.
constexpr int kGramHead = 3;   // at least 2
bool gram_head(const Group& g, const WavePlan& w, int ns_steps) {
  return !g.split && w.apply.splits == 1 && ns_steps > kGramHead && g.np >= 2 * g.mp;
}

// Dense-GEMM flops of one wave's Newton-Schulz products (2 m n k each,
// symmetric products counted in full).
double wave_flops(const Group& g, const WavePlan& w, int ns_steps) {
  const double m = (double)g.m, n = (double)g.n;
  const double mmn = 2.0 * m * m * n, mmm = 2.0 * m * m * m;
  // head: Gram, P_0 .. P_{k-1}, two products per A_j and one per R_j, the apply
  const int k = kGramHead;
  if (gram_head(g, w, ns_steps)) return ((ns_steps - k + 1) * 2.0 * mmn + (ns_steps + 3 * (k - 1)) * mmm) * w.nb;
  return ns_steps * (2.0 * mmn + mmm) * w.nb;
}

// flops and bytes are what the profile records for the launch: its dense
// flops and its algorithmic bytes (bf16 operands read once, the bf16 output
// written once, plus the weight traffic of a fused update).
mc_status launch_gemm_planned(const GemmPlan& gp, GemmKind kind, bool split_pair, GemmArgs a, hipStream_t s,
                              void* ws_base, size_t off_splitk, double flops, double bytes,
                              const FusedUpd* upd = nullptr) {
  a.tiles_m = gp.tiles_m; a.tiles_n = gp.tiles_n;
  a.splits = gp.splits; a.kt_per_split = gp.kt_per_split;
  a.partial = gp.splits > 1 ? (float*)((char*)ws_base + off_splitk) : nullptr;
  {
    Prof pr(F_GEMM, s, flops, bytes);
    hipError_t e = launch_ns_gemm(gp.tile, kind, split_pair, a, s, upd);
    if (e != hipSuccess) return fail(MC_ERR_HIP, "ns_gemm launch: %s", hipGetErrorString(e));
  }
  if (gp.splits > 1) {
    Prof pr(F_SPLITK, s, 0.0, (double)gp.partial_bytes);
    hipError_t e = launch_splitk_reduce(a, s);
    if (e != hipSuccess) return fail(MC_ERR_HIP, "splitk_reduce launch: %s", hipGetErrorString(e));
  }
  return MC_OK;
}

ClipRule clip_rule(const mc_matrix& m, bool clip_on) {
  ClipRule c{};
  c.slot = clip_on ? m.clip_slot : -1;
  c.period = m.period > 0 ? m.period : 1;
  c.nseg = clip_on && m.clip_slot >= 0 ? m.nseg : 0;
  for (int s = 0; s < 2; ++s) {
    c.off[s] = s < m.nseg ? m.seg[s].offset : 0;
    c.len[s] = s < m.nseg ? m.seg[s].length : 0;
    c.expo[s] = s < m.nseg ? m.seg[s].expo : 0.0f;
  }
  return c;
}

// Launches that read s_max first make their stream wait for the caller's
// event (recorded after the launch that writes s_max); momentum and the
// Newton-Schulz products before them do not wait.
mc_status wait_smax(hipEvent_t ev, const float* s_max, hipStream_t s) {
  if (!ev || !s_max) return MC_OK;
  hipError_t e = hipStreamWaitEvent(s, ev, 0);
  return e == hipSuccess ? MC_OK : fail(MC_ERR_HIP, "wait on s_max_ready: %s", hipGetErrorString(e));
}

// gamma_once: when it points at a non-NULL gamma output, the first update
// launch of this wave also writes gamma [slots][heads] and the pointer is
// cleared, so exactly one launch of the step writes it.
mc_status run_wave(const mc_matrix* mats, const Group& g, const int* ids, int nb, const mc_hparams& hp,
                   const float* s_max, int32_t heads, char* ws, hipStream_t s, float** gamma_once,
                   int32_t slots, hipEvent_t smax_ready) {
  const int cus = device_cus();
  const WavePlan w = plan_wave(g, nb, cus);
  const int64_t mp = g.mp, np = g.np;
  // X ping-pong: iteration it reads X[it % 2] and writes X[(it + 1) % 2]
  uint16_t* X[2] = {(uint16_t*)(ws + w.off_x0), (uint16_t*)(ws + w.off_x1)};
  uint16_t* Ahi = (uint16_t*)(ws + w.off_ahi);
  uint16_t* Alo = (uint16_t*)(ws + w.off_alo);
  uint16_t* Phi = (uint16_t*)(ws + w.off_phi);
  uint16_t* Plo = g.split ? (uint16_t*)(ws + w.off_plo) : nullptr;
  float* part = (float*)(ws + w.off_part);
  float* scale = (float*)(ws + w.off_scale);

  // 1. momentum + norm partials + bf16 X0 = M (wide) or M^T (tall), [mp][np]
  for (int b0 = 0; b0 < nb; b0 += kMaxMomMats) {
    MomArgs a{};
    a.mu = hp.mu; a.nesterov = hp.nesterov;
    int blocks = 0;
    double bytes = 0;
    for (int j = 0; j < kMaxMomMats && b0 + j < nb; ++j) {
      const int slot = b0 + j;
      const mc_matrix& m = mats[ids[slot]];
      const bool wide = m.rows <= m.cols;
      MomMat& mm = a.mat[a.nmat++];
      mm.g = m.g; mm.m = m.m; mm.ld = m.ld;
      mm.rows = (int32_t)m.rows; mm.cols = (int32_t)m.cols;
      mm.g_bf16 = m.g_dtype == MC_BF16;
      mm.vec = (m.cols % 4 == 0) && (m.ld % 4 == 0) && aligned(m.m, 16) && aligned(m.g, 4 * dtype_size(m.g_dtype));
      uint16_t* xs = X[0] + (size_t)slot * mp * np;
      mm.x_orig = wide ? xs : nullptr; mm.ld_orig = (int32_t)np;
      mm.x_tr = wide ? nullptr : xs;   mm.ld_tr = (int32_t)np;
      mm.rp = (int32_t)(wide ? mp : np); mm.cp = (int32_t)(wide ? np : mp);
      mm.tiles_c = mm.cp / 64;
      mm.block_start = blocks;
      mm.partial = part + (size_t)slot * w.mom_blocks;
      blocks += (mm.rp / 64) * mm.tiles_c;
      // read G and M, write M and the bf16 copy of M that Newton-Schulz reads
      bytes += (double)m.rows * m.cols * (dtype_size(m.g_dtype) + 10);
    }
    a.total_blocks = blocks;
    Prof pr(F_MOMENTUM, s, 0.0, bytes);
    hipError_t e = launch_momentum(a, s);
    if (e != hipSuccess) return fail(MC_ERR_HIP, "momentum launch: %s", hipGetErrorString(e));
  }
  {
    Prof pr(F_NORM, s, 0.0, 0.0);
    hipError_t e = launch_norm_finalize(part, (int32_t)w.mom_blocks, w.mom_blocks, scale, nb, hp.ns_eps, s);
    if (e != hipSuccess) return fail(MC_ERR_HIP, "norm_finalize launch: %s", hipGetErrorString(e));
  }

  // The update rides on the last apply's epilogue (no O round trip through
  // HBM, no separate launch) when every matrix of the wave allows it: a bf16
  // weight with 8-element-aligned rows, no copy of O requested, an unsplit
  // apply, and clip rules only on the first kMaxFusedClip matrices.
  const float decay = (float)(1.0 - (double)hp.lr * (double)hp.weight_decay);
  FusedUpd fu{};
  double fu_bytes = 0.0;
  {
    bool fuse = hp.ns_steps >= 1 && w.apply.splits == 1 && nb <= kMaxFusedMats;
    for (int slot = 0; slot < nb && fuse; ++slot) {
      const mc_matrix& m = mats[ids[slot]];
      const ClipRule c = clip_rule(m, s_max != nullptr);
      fuse = m.w_dtype == MC_BF16 && !m.o_out && m.cols % 8 == 0 && m.ld % 8 == 0 && m.ld <= INT32_MAX &&
             aligned(m.w, 16) && (slot < kMaxFusedClip || c.slot < 0 || c.nseg == 0);
    }
    if (fuse) {
      fu.n = nb; fu.m = (int32_t)g.m; fu.nn = (int32_t)g.n;
      fu.decay = decay;
      fu.lr_rms = (float)((double)hp.lr * (double)hp.rms_scale * sqrt((double)g.n));
      fu.s_max = s_max; fu.heads = heads; fu.tau = hp.tau; fu.clip_global = hp.clip_global;
      fu.nclip = std::min(nb, kMaxFusedClip);
      for (int slot = 0; slot < nb; ++slot) {
        const mc_matrix& m = mats[ids[slot]];
        if (slot < kMaxFusedClip) fu.clip[slot] = clip_rule(m, s_max != nullptr);
        fu.ld[slot] = (int32_t)m.ld;
        fu.trans[slot] = m.rows <= m.cols ? 0 : 1;
        fu.w[slot] = m.w;
        fu_bytes += (double)m.rows * m.cols * 4.0;   // read and write W
      }
    }
  }

  // 2. Newton-Schulz iterations
  const double mm_ = (double)g.m, nn_ = (double)g.n;
  const int kt_sq = (int)(mp / kGemmBK);
  // Gram: A = s0^2 X X^T (s0 on the first iteration only), stored as a bf16
  // pair A_hi + A_lo (operand pairs), or as A_hi and, where the Poly tiles
  // match, its fragment-order copy
  auto gram = [&](const uint16_t* x, bool first) -> mc_status {
    GemmArgs a{};
    a.M = (int32_t)mp; a.N = (int32_t)mp; a.batch = nb;
    a.lda = (int32_t)np; a.ldb = (int32_t)np; a.bsa = mp * np; a.bsb = mp * np;
    a.nseg = 1; a.seg[0] = {x, x, w.kt_gram}; a.ktiles = w.kt_gram;
    a.epi.alpha = 1.0f; a.epi.scale_pow = first ? 2 : 0; a.epi.scale = scale;
    a.epi.out_hi = Ahi; a.epi.ld_hi = (int32_t)mp; a.epi.bs_hi = mp * mp;
    if (w.frag) {
      a.epi.frag_out = Alo; a.epi.frag_nb = (int32_t)(mp / 32); a.epi.bs_frag = mp * mp;
    } else if (g.split) {
      a.epi.out_lo = Alo; a.epi.ld_lo = (int32_t)mp; a.epi.bs_lo = mp * mp;
    }
    return launch_gemm_planned(w.gram, GEMM_GRAM, g.split, a, s, ws, w.off_splitk, 2.0 * mm_ * mm_ * nn_ * nb,
                               (2.0 * mm_ * nn_ + 2.0 * mm_ * mm_) * nb);
  };
  // Poly: P = a I + b A + c A A, to out_hi (+ P_lo with operand pairs)
  auto poly = [&](uint16_t* out_hi) -> mc_status {
    GemmArgs a{};
    a.M = (int32_t)mp; a.N = (int32_t)mp; a.batch = nb;
    a.lda = (int32_t)mp; a.ldb = (int32_t)mp; a.bsa = mp * mp; a.bsb = mp * mp;
    if (g.split) {
      a.nseg = 3;
      a.seg[0] = {Ahi, Ahi, kt_sq}; a.seg[1] = {Ahi, Alo, kt_sq}; a.seg[2] = {Alo, Ahi, kt_sq};
    } else {
      a.nseg = 1; a.seg[0] = {Ahi, Ahi, kt_sq};
    }
    a.ktiles = w.kt_poly;
    a.epi.alpha = hp.ns_c; a.epi.beta = hp.ns_b; a.epi.diag = hp.ns_a;
    if (w.frag) {
      a.epi.frag_in = Alo; a.epi.frag_nb = (int32_t)(mp / 32); a.epi.bs_frag = mp * mp;
    } else {
      a.epi.cin_hi = Ahi; a.epi.cin_lo = g.split ? Alo : nullptr; a.epi.ld_cin = (int32_t)mp; a.epi.bs_cin = mp * mp;
    }
    a.epi.out_hi = out_hi; a.epi.ld_hi = (int32_t)mp; a.epi.bs_hi = mp * mp;
    if (Plo) { a.epi.out_lo = Plo; a.epi.ld_lo = (int32_t)mp; a.epi.bs_lo = mp * mp; }
    return launch_gemm_planned(w.poly, GEMM_POLY, g.split, a, s, ws, w.off_splitk, 2.0 * mm_ * mm_ * mm_ * nb,
                               4.0 * mm_ * mm_ * nb);
  };
  // C = L R + diag I of two exactly symmetric m x m matrices (the Gram-space
  // head): R is read by rows, which are its columns; C is symmetric up to
  // rounding (L and R are polynomials in one matrix, so they commute) and only
  // its upper tiles are computed, then mirrored. to_a: C is the next A, so
  // its fragment-order copy is also written where the Poly reads one.
  auto sym_product = [&](const uint16_t* l, const uint16_t* r, uint16_t* out, bool to_a, float diag = 0.0f,
                         const uint16_t* c = nullptr, float beta = 0.0f) -> mc_status {
    GemmArgs a{};
    a.M = (int32_t)mp; a.N = (int32_t)mp; a.batch = nb;
    a.lda = (int32_t)mp; a.ldb = (int32_t)mp; a.bsa = mp * mp; a.bsb = mp * mp;
    a.nseg = 1; a.seg[0] = {l, r, kt_sq}; a.ktiles = kt_sq;
    a.epi.alpha = 1.0f; a.epi.diag = diag;
    if (c) { a.epi.cin_hi = c; a.epi.beta = beta; a.epi.ld_cin = (int32_t)mp; a.epi.bs_cin = mp * mp; }
    a.epi.out_hi = out; a.epi.ld_hi = (int32_t)mp; a.epi.bs_hi = mp * mp;
    if (to_a && w.frag) {
      a.epi.frag_out = Alo; a.epi.frag_nb = (int32_t)(mp / 32); a.epi.bs_frag = mp * mp;
    }
    return launch_gemm_planned(w.poly, GEMM_GRAM, false, a, s, ws, w.off_splitk, 2.0 * mm_ * mm_ * mm_ * nb,
                               (c ? 8.0 : 6.0) * mm_ * mm_ * nb);
  };
  // Apply: X' = s0 P X (s0 on the first product of X0 only), C[i][j] =
  // sum_k P[i][k] X[k][j] with X read as [k][n]; the last one carries the
  // update when it is fused. x_coef != 0: X' = s0 (P X + x_coef X), the
  // second term added in fp32 to the rounded product.
  auto apply = [&](const uint16_t* p_hi, const uint16_t* p_lo, const uint16_t* x_in, uint16_t* x_out,
                   bool first, bool last, float x_coef = 0.0f) -> mc_status {
    GemmArgs a{};
    a.M = (int32_t)mp; a.N = (int32_t)np; a.batch = nb;
    a.lda = (int32_t)mp; a.ldb = (int32_t)np; a.bsa = mp * mp; a.bsb = mp * np;
    if (p_lo) { a.nseg = 2; a.seg[0] = {p_hi, x_in, kt_sq}; a.seg[1] = {p_lo, x_in, kt_sq}; }
    else { a.nseg = 1; a.seg[0] = {p_hi, x_in, kt_sq}; }
    a.ktiles = w.kt_apply;
    a.epi.alpha = 1.0f; a.epi.scale_pow = first ? 1 : 0; a.epi.scale = scale;
    a.epi.out_hi = x_out; a.epi.ld_hi = (int32_t)np; a.epi.bs_hi = mp * np;
    if (x_coef != 0.0f) {
      a.epi.xadd = x_in; a.epi.ld_xadd = (int32_t)np; a.epi.bs_xadd = mp * np; a.epi.xadd_coef = x_coef;
    }
    const bool upd = last && fu.n > 0;
    if (upd) {
      if (mc_status ws_ = wait_smax(smax_ready, s_max, s)) return ws_;
      if (gamma_once && *gamma_once) {
        fu.gamma_out = *gamma_once; fu.gamma_slots = slots;
        *gamma_once = nullptr;
      }
    }
    // operands P and X (read once, also when the epilogue adds it); X' is
    // written unless the update consumes it
    const double bytes = (2.0 * mm_ * mm_ + 2.0 * mm_ * nn_ + (upd ? 0.0 : 2.0 * mm_ * nn_)) * nb;
    return launch_gemm_planned(w.apply, GEMM_APPLY, false, a, s, ws, w.off_splitk, 2.0 * mm_ * mm_ * nn_ * nb,
                               bytes + (upd ? fu_bytes : 0.0), upd ? &fu : nullptr);
  };

  int cur = 0, it0 = 0;   // X[cur] holds iterate X_it0
  if (gram_head(g, w, hp.ns_steps)) {
    // The first kGramHead iterations in Gram space. With A0 = s0^2 X0 X0^T and
    // P_j = p(A_j), X_{j+1} = P_j X_j gives A_{j+1} = P_j A_j P_j, so every
    // A_j and P_j follows from m x m products alone and X_k = (P_{k-1} ..
    // P_0) X0 takes one n-sized product. The accumulated product Q_j =
    // P_j .. P_0 is about a^{j+1} I plus a smaller part (a the quintic's
    // linear coefficient), so it is kept as R_j = Q_j - a^{j+1} I, whose bf16
    // rounding is much finer than Q_j's: R_1 = P_1 P_0 - a^2 I, R_j = P_j
    // R_{j-1} + a^j P_j - a^{j+1} I, and the apply adds a^k X0 back in fp32.
    // m x m scratch: T0 and T1 in X[1] (n >= 2 m columns), which X_k
    // overwrites last. The last R goes to A_hi (its A has been read by the
    // last Poly), so the R the apply reads is never in X[1]; earlier R_j
    // alternate between T1 and the buffer P0 leaves.
    static_assert(kGramHead >= 2, "a head of one is an ordinary iteration");
    uint16_t* T0 = X[1];
    uint16_t* T1 = X[1] + (size_t)nb * mp * mp;
    const double a_ = hp.ns_a;
    uint16_t* r_buf = kGramHead == 2 ? Ahi : T1;
    mc_status st = gram(X[0], true);
    if (!st) st = poly(Phi);                          // P0
    if (!st) st = sym_product(Ahi, Phi, T0, false);   // A0 P0
    if (!st) st = sym_product(Phi, T0, Ahi, true);    // A1 = P0 (A0 P0)
    if (!st) st = poly(T0);                           // P1
    if (!st) st = sym_product(T0, Phi, r_buf, false, (float)(-a_ * a_));   // R1 = P1 P0 - a^2 I
    // P_{j-1} in T0, R_{j-1} in r_buf, A_{j-1} in A_hi (+ its copy); spare
    // is free (P0's buffer once R1 is formed)
    uint16_t* spare = Phi;
    for (int j = 2; j < kGramHead && !st; ++j) {
      const double aj = std::pow(a_, j);
      const bool last = j + 1 == kGramHead;
      st = sym_product(Ahi, T0, spare, false);                // A_{j-1} P_{j-1}
      if (!st) st = sym_product(T0, spare, Ahi, true);        // A_j
      if (!st) st = poly(T0);                                 // P_j
      uint16_t* out = last ? Ahi : spare;
      if (!st) st = sym_product(T0, r_buf, out, false, (float)(-aj * a_), T0, (float)aj);   // R_j
      if (last) r_buf = out;
      else std::swap(r_buf, spare);
    }
    if (!st) st = apply(r_buf, nullptr, X[0], X[1], true, false, (float)std::pow(a_, kGramHead));   // X_k
    if (st) return st;
    cur = 1; it0 = kGramHead;
  }
  for (int it = it0; it < hp.ns_steps; ++it) {
    mc_status st = gram(X[cur], it == 0);
    if (!st) st = poly(Phi);
    if (!st) st = apply(Phi, Plo, X[cur], X[cur ^ 1], it == 0, it + 1 == hp.ns_steps);
    if (st) return st;
    cur ^= 1;
  }
  if (fu.n > 0) return MC_OK;

  // 3. update + decay + QK-Clip rows
  if (mc_status ws_ = wait_smax(smax_ready, s_max, s)) return ws_;
  uint16_t* x_final = X[cur];   // O in [m][n]: W itself (wide) or W^T (tall)
  for (int b0 = 0; b0 < nb; b0 += kMaxBatchMats) {
    UpdArgs a{};
    a.decay = decay; a.s_max = s_max; a.heads = heads; a.tau = hp.tau; a.clip_global = hp.clip_global;
    if (gamma_once && *gamma_once) {
      a.gamma_out = *gamma_once; a.gamma_slots = slots;
      *gamma_once = nullptr;
    }
    int blocks = 0;
    double bytes = 0;
    for (int j = 0; j < kMaxBatchMats && b0 + j < nb; ++j) {
      const int slot = b0 + j;
      const mc_matrix& m = mats[ids[slot]];
      const bool wide = m.rows <= m.cols;
      UpdMat& u = a.mat[a.nmat++];
      u.w = m.w; u.w_bf16 = m.w_dtype == MC_BF16; u.ld = m.ld;
      u.rows = (int32_t)m.rows; u.cols = (int32_t)m.cols;
      u.vec = (m.cols % 4 == 0) && (m.ld % 4 == 0) && aligned(m.w, 4 * dtype_size(m.w_dtype)) &&
              (!m.o_out || aligned(m.o_out, 8));
      u.o = x_final + (size_t)slot * mp * np;
      u.ld_o = (int32_t)np;
      u.vec8 = u.vec && u.w_bf16 && m.cols % 8 == 0 && m.ld % 8 == 0 && aligned(m.w, 16) &&
               (!m.o_out || aligned(m.o_out, 16)) && np % 8 == 0 && aligned(u.o, 16);
      u.o_trans = wide ? 0 : 1;
      u.o_out = (uint16_t*)m.o_out;
      u.lr_rms = (float)((double)hp.lr * (double)hp.rms_scale * sqrt((double)std::max(m.rows, m.cols)));
      u.clip = clip_rule(m, s_max != nullptr);
      u.tiles_c = (int32_t)((m.cols + 63) / 64);
      u.block_start = blocks;
      blocks += (int)((m.rows + 63) / 64) * u.tiles_c;
      bytes += (double)m.rows * m.cols * 2.0 * dtype_size(m.w_dtype);
    }
    a.total_blocks = blocks;
    Prof pr(F_UPDATE, s, 0.0, bytes);
    hipError_t e = launch_update(a, s);
    if (e != hipSuccess) return fail(MC_ERR_HIP, "update launch: %s", hipGetErrorString(e));
  }
  return MC_OK;
}

int largest_wave(const Group& g, int limit, size_t ws_bytes) {
  int best = 0;
  const int cus = device_cus();
  for (int nb = 1; nb <= limit; ++nb)
    if (plan_wave(g, nb, cus).bytes <= ws_bytes) best = nb;
  return best;
}

// A chain is one wave of one shape group: momentum, Newton-Schulz and update
// of nb matrices, independent of every other chain.
struct Chain { int gi, b0, nb; double flops; };

// Relative time of one wave's Newton-Schulz products: every launch runs in
// rounds of one tile per CU, so a round that only part of the chip has
// tiles for costs as much as a full one. A round costs its k-stages times
// the tile's share of a 256x256 tile's work (128 and 64 tiles run at about
// 0.8 of that rate per flop), split-K launches their partial k range.
double wave_cost(const Group& g, int nb, int cus, int ns_steps) {
  const WavePlan w = plan_wave(g, nb, cus);
  auto launch = [&](const GemmPlan& gp, bool sym) {
    const int d = gemm_tile_dim(gp.tile);
    const int64_t per = (sym && gp.splits == 1) ? (int64_t)gp.tiles_m * (gp.tiles_m + 1) / 2
                                                : (int64_t)gp.tiles_m * gp.tiles_n;
    const int64_t items = per * gp.splits * nb;
    const double rounds = (double)((items + cus - 1) / cus);
    const double share = (double)d * d / (256.0 * 256.0) / (d == 256 ? 1.0 : 0.8);
    return rounds * gp.kt_per_split * share + 2.0;   // + launch and drain, about two k-stages
  };
  const double gram = launch(w.gram, true), sq = launch(w.poly, true), apply = launch(w.apply, false);
  // each head iteration after the first trades a Gram and an apply for three m x m products
  const int k = kGramHead;
  if (gram_head(g, w, ns_steps)) return (ns_steps - k + 1) * (gram + apply) + (ns_steps + 3 * (k - 1)) * sq;
  return ns_steps * (gram + sq + apply);
}

// Waves of at most cap[gi] matrices per group. A group larger than one wave
// is cut into waves of one size s plus a remainder, s chosen between the
// even split and the cap to minimise the summed wave_cost (1155 expert
// matrices: 18 waves of 64 and one of 3, whose launches fill every round,
// instead of 19 waves of about 61 that leave most launches a partial round).
std::vector<Chain> plan_chains(const std::vector<Group>& groups, const std::vector<int>& cap, int ns_steps) {
  std::vector<Chain> out;
  const int cus = device_cus();
  for (size_t gi = 0; gi < groups.size(); ++gi) {
    const Group& g = groups[gi];
    const int count = (int)g.idx.size();
    const int waves = (count + cap[gi] - 1) / cap[gi];
    std::vector<int> sizes;
    for (int w = 0; w < waves; ++w) sizes.push_back(count / waves + (w < count % waves ? 1 : 0));
    if (waves > 1) {
      std::map<int, double> memo;
      auto cost_of = [&](int nb) {
        auto it = memo.find(nb);
        if (it != memo.end()) return it->second;
        return memo[nb] = wave_cost(g, nb, cus, ns_steps);
      };
      double best = 0.0;
      for (int nb : sizes) best += cost_of(nb);
      for (int sz = (count + waves - 1) / waves + 1; sz <= cap[gi]; ++sz) {
        const int full = count / sz, rest = count - full * sz;
        const double c = full * cost_of(sz) + (rest ? cost_of(rest) : 0.0);
        if (c < best * 0.999) {
          best = c;
          sizes.assign(full, sz);
          if (rest) sizes.push_back(rest);
        }
      }
    }
    for (int b0 = 0, w = 0; w < (int)sizes.size(); ++w) {
      const int nb = sizes[w];
      const double f = wave_flops(g, plan_wave(g, nb, cus), ns_steps);
      out.push_back({(int)gi, b0, nb, f});
      b0 += nb;
    }
  }
  return out;
}

// One auxiliary stream and a fork / join event pair per device, created on
// first use and kept for the life of the process. Two chains in flight let
// one chain's bandwidth-bound momentum and update kernels, and its launches
// that cannot fill the chip, overlap another chain's matrix-core work.
struct AuxLane { hipStream_t s = nullptr; hipEvent_t fork = nullptr, join = nullptr; };
std::mutex g_aux_mu;
std::map<int, AuxLane> g_aux;

// Under g_aux_mu. Returns nullptr when the device's lane cannot be created.
AuxLane* aux_lane() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return nullptr;
  auto it = g_aux.find(dev);
  if (it != g_aux.end()) return it->second.s ? &it->second : nullptr;
  AuxLane l;
  if (hipStreamCreateWithFlags(&l.s, hipStreamNonBlocking) != hipSuccess ||
      hipEventCreateWithFlags(&l.fork, hipEventDisableTiming) != hipSuccess ||
      hipEventCreateWithFlags(&l.join, hipEventDisableTiming) != hipSuccess) {
    (void)hipGetLastError();
    l = AuxLane{};
  }
  g_aux[dev] = l;
  return l.s ? &g_aux[dev] : nullptr;
}

}  // namespace

// ================================================================ C ABI

extern "C" {

void mc_default_hparams(mc_hparams* hp) {
  if (!hp) return;
  hp->lr = 2e-4f; hp->mu = 0.95f; hp->weight_decay = 0.1f; hp->rms_scale = 0.2f; hp->tau = 100.0f;
  hp->ns_a = 3.4445f; hp->ns_b = -4.7750f; hp->ns_c = 2.0315f; hp->ns_eps = 1e-7f; hp->ns_steps = 5;
  hp->nesterov = 0; hp->clip_global = 0;
}

const char* mc_last_error(void) { return g_err.c_str(); }
const char* mc_version(void) { return "muonclip-gfx950 0.1"; }

static size_t workspace_for(const mc_matrix* mats, int32_t n, const mc_hparams* hp, bool minimal) {
  if (check_hparams(hp) != MC_OK) return 0;
  if (check_matrices_step(mats, n, 0, 0, false) != MC_OK) return 0;
  size_t best = 0;
  const std::vector<Group> groups = make_groups(mats, n);
  std::vector<int> cap;
  for (const Group& g : groups) {
    const int nb = minimal ? 1 : std::min<int>((int)g.idx.size(), kWaveCap);
    cap.push_back(nb);
    best = std::max(best, plan_wave(g, nb, device_cus()).bytes);
  }
  // room for two chains in flight when the step has more than one shape group
  if (!minimal && groups.size() >= 2) best = 2 * align_up(best);
  return best;
}

size_t mc_workspace_size(const mc_matrix* mats, int32_t n, const mc_hparams* hp) {
  return workspace_for(mats, n, hp, false);
}
size_t mc_workspace_min_size(const mc_matrix* mats, int32_t n, const mc_hparams* hp) {
  return workspace_for(mats, n, hp, true);
}

// muonclip_step with an optional event that the launches reading s_max wait on.
static mc_status step_impl(const mc_matrix* mats, int32_t n, const mc_hparams* hp, const float* s_max,
                           int32_t slots, int32_t heads, float* gamma_out, void* workspace, size_t workspace_bytes,
                           void* stream, hipEvent_t smax_ready, bool one_lane = false) {
  mc_status st = check_hparams(hp);
  if (st) return st;
  const bool have_smax = s_max != nullptr;
  if (have_smax && (slots <= 0 || heads <= 0)) return fail(MC_ERR_SHAPE, "slots and heads must be >= 1 with s_max");
  if (gamma_out && !have_smax) return fail(MC_ERR_NULL, "gamma_out given without s_max");
  if ((have_smax && !aligned(s_max, 4)) || (gamma_out && !aligned(gamma_out, 4)))
    return fail(MC_ERR_ALIGN, "s_max / gamma_out misaligned");
  st = check_matrices_step(mats, n, slots, heads, have_smax);
  if (st) return st;
  if (n == 0) {   // nothing to update; gamma is still an output
    if (gamma_out) {
      if ((st = wait_smax(smax_ready, s_max, (hipStream_t)stream))) return st;
      Prof pr(F_GAMMA, (hipStream_t)stream, 0.0, 0.0);
      hipError_t e = launch_gamma(s_max, gamma_out, slots, heads, hp->tau, hp->clip_global, (hipStream_t)stream);
      if (e != hipSuccess) return fail(MC_ERR_HIP, "gamma launch: %s", hipGetErrorString(e));
    }
    return MC_OK;
  }
  if (!workspace) return fail(MC_ERR_WORKSPACE, "workspace is NULL");
  if (!aligned(workspace, kAlign)) return fail(MC_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  const std::vector<Group> groups = make_groups(mats, n);
  std::vector<int> wave_cap(groups.size());
  for (size_t gi = 0; gi < groups.size(); ++gi) {
    const Group& g = groups[gi];
    wave_cap[gi] = largest_wave(g, std::min<int>((int)g.idx.size(), kWaveCap), workspace_bytes);
    if (wave_cap[gi] == 0)
      return fail(MC_ERR_WORKSPACE, "workspace %zu bytes < %zu needed for one %lldx%lld matrix", workspace_bytes,
                  plan_wave(g, 1, device_cus()).bytes, (long long)g.m, (long long)g.n);
  }
  // Two lanes (the caller's stream and the library's auxiliary stream, each
  // with half the workspace) when there are at least two shape groups and
  // every group fits a half; which chain runs on which lane is decided below.
  // A single wave is never split to fill a second lane (on the MHA layer two
  // half-waves measured slower than one wave). While kernel timing is on
  // (mc_profile_enable), every chain runs on the caller's stream, so that no
  // two timed launches overlap.
  const size_t half = (workspace_bytes / 2) & ~(kAlign - 1);
  std::vector<Chain> chains = plan_chains(groups, wave_cap, hp->ns_steps);
  bool two = groups.size() >= 2 && chains.size() >= 2 && !one_lane && !profiling_on();
  std::vector<int> cap2(groups.size());
  for (size_t gi = 0; gi < groups.size() && two; ++gi) {
    cap2[gi] = largest_wave(groups[gi], std::min<int>((int)groups[gi].idx.size(), kWaveCap), half);
    two = cap2[gi] > 0;
  }
  if (two) chains = plan_chains(groups, cap2, hp->ns_steps);
  // Lanes. A chain whose Gram launch runs unsplit with a tile for every CU
  // ("large") runs on `stream`, after the other large ones: two large chains
  // side by side only interleave their workgroups (each takes whole CUs) and
  // break up the launches' full rounds (full K2 layer: 525-527 ms this way,
  // 530-532 ms with every chain balanced over the two lanes). The small
  // chains (split-K, or fewer tiles than CUs: launches that leave CUs idle)
  // go to the auxiliary stream beside them (MLA layer: 8.5 ms either way,
  // 10.2 ms on one lane). Without large chains, the chains are balanced over
  // both lanes, largest first; without small ones, one lane with the whole
  // workspace runs them all.
  const int cus = device_cus();
  std::vector<char> small(chains.size());
  bool any_large = false, any_small = false;
  for (size_t i = 0; i < chains.size() && two; ++i) {
    const GemmPlan gp = plan_wave(groups[chains[i].gi], chains[i].nb, cus).gram;
    small[i] = gp.splits > 1 || (int64_t)gp.tiles_m * (gp.tiles_m + 1) / 2 * chains[i].nb < cus;
    any_large = any_large || !small[i];
    any_small = any_small || small[i];
  }
  if (two && !any_small) {
    two = false;
    chains = plan_chains(groups, wave_cap, hp->ns_steps);
  }

  hipStream_t s = (hipStream_t)stream;
  float* gamma_once = gamma_out;   // written by the first update launch
  std::unique_lock<std::mutex> lk(g_aux_mu, std::defer_lock);
  AuxLane* aux = nullptr;
  if (two) {
    lk.lock();
    aux = aux_lane();
    if (!aux) {   // no auxiliary stream: everything on `stream`
      lk.unlock();
      two = false;
      chains = plan_chains(groups, wave_cap, hp->ns_steps);
    }
  }
  if (!two) {
    for (const Chain& c : chains) {
      st = run_wave(mats, groups[c.gi], groups[c.gi].idx.data() + c.b0, c.nb, *hp, s_max, heads, (char*)workspace, s,
                    &gamma_once, slots, smax_ready);
      if (st) return st;
    }
    return MC_OK;
  }
  // fork: the auxiliary stream starts after everything enqueued on `stream`
  if (hipEventRecord(aux->fork, s) != hipSuccess || hipStreamWaitEvent(aux->s, aux->fork, 0) != hipSuccess)
    return fail(MC_ERR_HIP, "stream fork failed");
  std::vector<int> order(chains.size());
  for (size_t i = 0; i < order.size(); ++i) order[i] = (int)i;
  std::stable_sort(order.begin(), order.end(), [&](int x, int y) { return chains[x].flops > chains[y].flops; });
  double load[2] = {0.0, 0.0};
  for (int i : order) {
    const Chain& c = chains[i];
    const int lane = any_large ? (small[i] ? 1 : 0) : (load[1] < load[0] ? 1 : 0);
    load[lane] += c.flops;
    st = run_wave(mats, groups[c.gi], groups[c.gi].idx.data() + c.b0, c.nb, *hp, s_max, heads,
                  (char*)workspace + lane * half, lane ? aux->s : s, &gamma_once, slots, smax_ready);
    if (st) break;
  }
  // join: `stream` continues only after the auxiliary stream's work (also
  // after an error, so the caller's stream stays ordered)
  if (hipEventRecord(aux->join, aux->s) != hipSuccess || hipStreamWaitEvent(s, aux->join, 0) != hipSuccess)
    return st ? st : fail(MC_ERR_HIP, "stream join failed");
  return st;
}

mc_status muonclip_step(const mc_matrix* mats, int32_t n, const mc_hparams* hp, const float* s_max,
                        int32_t slots, int32_t heads, float* gamma_out, void* workspace, size_t workspace_bytes,
                        void* stream) {
  return step_impl(mats, n, hp, s_max, slots, heads, gamma_out, workspace, workspace_bytes, stream, nullptr);
}

mc_status muonclip_step_overlapped(const mc_matrix* mats, int32_t n, const mc_hparams* hp, const float* s_max,
                                   int32_t slots, int32_t heads, float* gamma_out, void* workspace,
                                   size_t workspace_bytes, void* stream, void* s_max_ready) {
  return step_impl(mats, n, hp, s_max, slots, heads, gamma_out, workspace, workspace_bytes, stream,
                   (hipEvent_t)s_max_ready);
}

}  // extern "C"

// ---------------------------------------------------------------- allocation-free step

// The workspace of muonclip_step_noalloc: one copy per device, held from the
// library's load until the process ends. In host code `scratch` names a host
// stand-in; kernels get the device address that hipGetSymbolAddress returns
// for the current device, looked up once per device.
static __device__ __align__(256) char scratch[MC_NOALLOC_SCRATCH_BYTES];

namespace {
std::mutex g_scr_mu;
std::map<int, void*> g_scr;

mc_status scratch_ptr(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(MC_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  std::lock_guard<std::mutex> lk(g_scr_mu);
  auto it = g_scr.find(dev);
  if (it != g_scr.end()) { *out = it->second; return MC_OK; }
  void* p = nullptr;
  e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (e != hipSuccess || !p) return fail(MC_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
  g_scr[dev] = p;
  *out = p;
  return MC_OK;
}
}  // namespace

extern "C" {

mc_status muonclip_step_noalloc(const mc_matrix* mats, int32_t n, const mc_hparams* hp, const float* s_max,
                                int32_t slots, int32_t heads, float* gamma_out, void* stream) {
  mc_status st = check_hparams(hp);
  if (st) return st;
  st = check_matrices_step(mats, n, 0, 0, false);
  if (st) return st;
  if (n > 0) {
    const size_t need = workspace_for(mats, n, hp, true);
    if (need > (size_t)MC_NOALLOC_SCRATCH_BYTES)
      return fail(MC_ERR_WORKSPACE, "muonclip_step_noalloc: these matrices need %zu bytes of workspace; the "
                  "static scratch holds %zu (use muonclip_step with a caller workspace)", need,
                  (size_t)MC_NOALLOC_SCRATCH_BYTES);
  }
  void* ws = nullptr;
  if ((st = scratch_ptr(&ws))) return st;
  return step_impl(mats, n, hp, s_max, slots, heads, gamma_out, ws, (size_t)MC_NOALLOC_SCRATCH_BYTES, stream,
                   nullptr, true);
}

mc_status max_logits_per_head(const void* q, const void* k, const void* k_shared, int32_t dtype, int32_t B, int32_t T,
                              int32_t H, int32_t d_q, int32_t d_k, int32_t d_shared, const int64_t* q_stride,
                              const int64_t* k_stride, const int64_t* ks_stride, int32_t causal, float scale,
                              float* s_max_out, void* stream) {
  if (!s_max_out) return fail(MC_ERR_NULL, "s_max_out is NULL");
  if (!dtype_ok(dtype)) return fail(MC_ERR_DTYPE, "dtype %d", dtype);
  if (B < 0 || T < 0 || H <= 0) return fail(MC_ERR_SHAPE, "B, T must be >= 0 and H >= 1");
  if (d_k <= 0 || d_shared < 0 || d_q != d_k + d_shared)
    return fail(MC_ERR_SHAPE, "need d_q == d_k + d_shared with d_k >= 1 (got %d, %d, %d)", d_q, d_k, d_shared);
  if (!q_stride || !k_stride) return fail(MC_ERR_NULL, "q_stride / k_stride is NULL");
  if (!isfinite(scale) || scale <= 0.0f) return fail(MC_ERR_HPARAM, "scale must be finite and > 0");
  if (!aligned(s_max_out, 4)) return fail(MC_ERR_ALIGN, "s_max_out misaligned");
  const bool empty = B == 0 || T == 0;
  if (!empty) {
    if (!q || !k) return fail(MC_ERR_NULL, "q or k is NULL");
    if (d_shared > 0 && (!k_shared || !ks_stride)) return fail(MC_ERR_NULL, "k_shared / ks_stride is NULL");
    const size_t es = dtype_size(dtype);
    if (!aligned(q, es) || !aligned(k, es) || (d_shared > 0 && !aligned(k_shared, es)))
      return fail(MC_ERR_ALIGN, "q / k / k_shared misaligned");
    for (int i = 0; i < 3; ++i)
      if (q_stride[i] < 0 || k_stride[i] < 0) return fail(MC_ERR_SHAPE, "negative stride");
    if ((T > 1 && q_stride[1] < d_q) || (T > 1 && k_stride[1] < d_k))
      return fail(MC_ERR_SHAPE, "t stride smaller than the head dimension");
  }
  MaxLogitArgs a{};
  a.q = q; a.k = k; a.ks = d_shared > 0 ? k_shared : nullptr;
  a.qs_b = q_stride[0]; a.qs_t = q_stride[1]; a.qs_h = q_stride[2];
  a.ks_b = k_stride[0]; a.ks_t = k_stride[1]; a.ks_h = k_stride[2];
  a.kss_b = d_shared > 0 ? ks_stride[0] : 0; a.kss_t = d_shared > 0 ? ks_stride[1] : 0;
  a.B = B; a.T = T; a.H = H; a.d_q = d_q; a.d_k = d_k; a.d_s = d_shared;
  a.causal = causal ? 1 : 0; a.bf16 = dtype == MC_BF16;
  a.out = s_max_out; a.scale = scale;
  hipStream_t s = (hipStream_t)stream;
  {
    Prof pr(F_ML_INIT, s, 0.0, 0.0);
    hipError_t e = launch_max_logits_init(a.out, H, s);
    if (e != hipSuccess) return fail(MC_ERR_HIP, "max_logits init: %s", hipGetErrorString(e));
  }
  {
    const double pairs = causal ? (double)T * (T + 1) / 2.0 : (double)T * T;
    Prof pr(F_ML, s, 2.0 * d_q * pairs * B * H, 0.0);
    bool mfma = false;
    hipError_t e = launch_max_logits(a, s, &mfma);
    if (e != hipSuccess) return fail(MC_ERR_HIP, "max_logits launch: %s", hipGetErrorString(e));
  }
  return MC_OK;
}

mc_status attention_forward(const void* q, const void* k, const void* k_shared, const void* v, void* o, float* lse,
                            float* s_max_out, int32_t B, int32_t T, int32_t H, int32_t d_q, int32_t d_k,
                            int32_t d_shared, int32_t d_v, const int64_t* q_stride, const int64_t* k_stride,
                            const int64_t* ks_stride, const int64_t* v_stride, const int64_t* o_stride,
                            int32_t causal, float scale, void* stream) {
  if (B < 0 || T < 0 || H <= 0) return fail(MC_ERR_SHAPE, "B, T must be >= 0 and H >= 1");
  if (d_q != d_k + d_shared || d_k != 128 || !(d_shared == 0 || d_shared == 64) || d_v != 128)
    return fail(MC_ERR_SHAPE, "attention_forward covers (d_k, d_shared, d_v) = (128, 0 or 64, 128) with "
                "d_q = d_k + d_shared (got %d, %d, %d, %d)", d_q, d_k, d_shared, d_v);
  if (!isfinite(scale) || scale <= 0.0f) return fail(MC_ERR_HPARAM, "scale must be finite and > 0");
  if ((lse && !aligned(lse, 4)) || (s_max_out && !aligned(s_max_out, 4)))
    return fail(MC_ERR_ALIGN, "lse / s_max_out misaligned");
  const bool empty = B == 0 || T == 0;
  AttnArgs a{};
  if (!empty) {
    if (!q || !k || !v || !o) return fail(MC_ERR_NULL, "q, k, v or o is NULL");
    if (!q_stride || !k_stride || !v_stride || !o_stride) return fail(MC_ERR_NULL, "a stride array is NULL");
    if (d_shared > 0 && (!k_shared || !ks_stride)) return fail(MC_ERR_NULL, "k_shared / ks_stride is NULL");
    for (int i = 0; i < 3; ++i)
      if (q_stride[i] < 0 || k_stride[i] < 0 || v_stride[i] < 0 || o_stride[i] < 0)
        return fail(MC_ERR_SHAPE, "negative stride");
    if (d_shared > 0 && (ks_stride[0] < 0 || ks_stride[1] < 0)) return fail(MC_ERR_SHAPE, "negative stride");
    // the tile loads keep 64 rows of offsets in 32 bits
    const int64_t kLimit = (int64_t)1 << 23;
    if (k_stride[1] >= kLimit || v_stride[1] >= kLimit || (d_shared > 0 && ks_stride[1] >= kLimit))
      return fail(MC_ERR_SHAPE, "t stride of k, k_shared or v must be < 2^23 elements");
    a.q = q; a.k = k; a.ks = d_shared > 0 ? k_shared : nullptr; a.v = v; a.o = o;
    a.qs_b = q_stride[0]; a.qs_t = q_stride[1]; a.qs_h = q_stride[2];
    a.ks_b = k_stride[0]; a.ks_t = k_stride[1]; a.ks_h = k_stride[2];
    a.kss_b = d_shared > 0 ? ks_stride[0] : 0; a.kss_t = d_shared > 0 ? ks_stride[1] : 0;
    a.vs_b = v_stride[0]; a.vs_t = v_stride[1]; a.vs_h = v_stride[2];
    a.os_b = o_stride[0]; a.os_t = o_stride[1]; a.os_h = o_stride[2];
  }
  a.B = B; a.T = T; a.H = H; a.d_k = d_k; a.d_s = d_shared; a.d_v = d_v;
  a.causal = causal ? 1 : 0; a.scale = scale;
  a.lse = lse; a.smax = s_max_out;
  if (!empty && !attention_supported(a))
    return fail(MC_ERR_ALIGN, "attention_forward needs 16-byte aligned q, k, k_shared, v, o and strides that "
                "are multiples of 8 elements");
  hipStream_t s = (hipStream_t)stream;
  if (s_max_out) {
    Prof pr(F_ML_INIT, s, 0.0, 0.0);
    hipError_t e = launch_max_logits_init(a.smax, H, s);
    if (e != hipSuccess) return fail(MC_ERR_HIP, "s_max init: %s", hipGetErrorString(e));
  }
  if (!empty) {
    const double pairs = causal ? (double)T * (T + 1) / 2.0 : (double)T * T;
    Prof pr(F_ATTN, s, 2.0 * (d_q + d_v) * pairs * B * H, 0.0);
    hipError_t e = launch_attention(a, s);
    if (e != hipSuccess) return fail(MC_ERR_HIP, "attention launch: %s", hipGetErrorString(e));
  }
  return MC_OK;
}

mc_status qk_clip_apply(const mc_matrix* mats, int32_t n, const float* s_max, int32_t slots, int32_t heads,
                        float tau, float* gamma_out, void* stream) {
  if (!s_max) return fail(MC_ERR_NULL, "s_max is NULL");
  if (n < 0) return fail(MC_ERR_SHAPE, "n < 0");
  if (n > 0 && !mats) return fail(MC_ERR_NULL, "mats is NULL");
  if (slots <= 0 || heads <= 0) return fail(MC_ERR_SHAPE, "slots and heads must be >= 1");
  if (!isfinite(tau) || tau <= 0.0f) return fail(MC_ERR_HPARAM, "tau must be finite and > 0");
  if (!aligned(s_max, 4) || (gamma_out && !aligned(gamma_out, 4))) return fail(MC_ERR_ALIGN, "s_max / gamma_out misaligned");
  for (int i = 0; i < n; ++i) {
    mc_status st = check_matrix_common(mats[i], i);
    if (st) return st;
    st = check_clip(mats[i], i, slots, heads, true);
    if (st) return st;
  }
  hipStream_t s = (hipStream_t)stream;
  if (gamma_out) {
    Prof pr(F_GAMMA, s, 0.0, 0.0);
    hipError_t e = launch_gamma(s_max, gamma_out, slots, heads, tau, 0, s);
    if (e != hipSuccess) return fail(MC_ERR_HIP, "gamma launch: %s", hipGetErrorString(e));
  }
  // matrices of whole 16-byte row vectors go kMaxClipBatch to a launch; the
  // rest one launch each with element accesses
  ClipVecArgs va{};
  va.s_max = s_max; va.heads = heads; va.tau = tau;
  auto flush = [&]() -> mc_status {
    if (va.nmat == 0) return MC_OK;
    Prof pr(F_CLIP, s, 0.0, 0.0);
    hipError_t e = launch_clip_apply_vec(va, s);
    va.nmat = 0; va.total_rows = 0;
    return e == hipSuccess ? MC_OK : fail(MC_ERR_HIP, "clip_apply launch: %s", hipGetErrorString(e));
  };
  for (int i = 0; i < n; ++i) {
    const mc_matrix& m = mats[i];
    if (m.clip_slot < 0 || m.nseg == 0) continue;
    ClipApplyArgs a{};
    a.w = m.w; a.w_bf16 = m.w_dtype == MC_BF16; a.ld = m.ld;
    a.rows = (int32_t)m.rows; a.cols = (int32_t)m.cols;
    a.clip = clip_rule(m, true);
    a.s_max = s_max; a.heads = heads; a.tau = tau;
    if (clip_apply_vectorizable(a)) {
      ClipVecMat& v = va.mat[va.nmat++];
      const int es = a.w_bf16 ? 2 : 4;
      v.w = (char*)m.w; v.ld_bytes = m.ld * es; v.w_bf16 = a.w_bf16; v.vpr = a.cols * es / 16;
      v.rows = a.rows; v.row_start = va.total_rows; v.clip = a.clip;
      va.total_rows += a.rows;
      if (va.nmat == kMaxClipBatch) {
        if (mc_status st = flush()) return st;
      }
      continue;
    }
    Prof pr(F_CLIP, s, 0.0, 0.0);
    hipError_t e = launch_clip_apply(a, s);
    if (e != hipSuccess) return fail(MC_ERR_HIP, "clip_apply launch: %s", hipGetErrorString(e));
  }
  return flush();
}

void mc_default_adamw_hparams(mc_adamw_hparams* hp) {
  if (!hp) return;
  hp->lr = 2e-4f; hp->beta1 = 0.9f; hp->beta2 = 0.95f; hp->eps = 1e-8f; hp->weight_decay = 0.1f; hp->step = 1;
}

mc_status adamw_step(const mc_vector* vecs, int32_t n, const mc_adamw_hparams* hp, void* stream) {
  if (!hp) return fail(MC_ERR_NULL, "hparams is NULL");
  const float v[] = {hp->lr, hp->beta1, hp->beta2, hp->eps, hp->weight_decay};
  for (float x : v)
    if (!isfinite(x)) return fail(MC_ERR_HPARAM, "AdamW hyper-parameters must be finite");
  if (!(hp->beta1 >= 0.0f && hp->beta1 < 1.0f) || !(hp->beta2 >= 0.0f && hp->beta2 < 1.0f))
    return fail(MC_ERR_HPARAM, "beta1 and beta2 must be in [0, 1)");
  if (hp->eps < 0.0f) return fail(MC_ERR_HPARAM, "eps must be >= 0");
  if (hp->step < 1) return fail(MC_ERR_HPARAM, "step must be >= 1 (got %d)", hp->step);
  if (n < 0) return fail(MC_ERR_SHAPE, "n < 0");
  if (n > 0 && !vecs) return fail(MC_ERR_NULL, "vecs is NULL");
  for (int i = 0; i < n; ++i) {
    const mc_vector& d = vecs[i];
    if (d.n < 0) return fail(MC_ERR_SHAPE, "vector %d: n < 0", i);
    if (d.n == 0) continue;
    if (d.n > ((int64_t)1 << 40)) return fail(MC_ERR_SHAPE, "vector %d: n above 2^40", i);
    if (!d.p || !d.g || !d.m || !d.v) return fail(MC_ERR_NULL, "vector %d: p, g, m or v is NULL", i);
    if (!dtype_ok(d.p_dtype) || !dtype_ok(d.g_dtype)) return fail(MC_ERR_DTYPE, "vector %d: dtype", i);
    if (!aligned(d.p, dtype_size(d.p_dtype)) || !aligned(d.g, dtype_size(d.g_dtype)) || !aligned(d.m, 4) ||
        !aligned(d.v, 4))
      return fail(MC_ERR_ALIGN, "vector %d: misaligned pointer", i);
  }
  // bias corrections in double, then fp32 like every other hyper-parameter
  const double c1 = 1.0 / (1.0 - pow((double)hp->beta1, (double)hp->step));
  const double c2 = 1.0 / (1.0 - pow((double)hp->beta2, (double)hp->step));
  hipStream_t s = (hipStream_t)stream;
  AdamArgs a{};
  auto flush = [&]() -> mc_status {
    if (a.nvec == 0) return MC_OK;
    double bytes = 0;
    for (int k = 0; k < a.nvec; ++k)
      bytes += (double)a.vec[k].n * (2.0 * (a.vec[k].p_bf16 ? 2 : 4) + (a.vec[k].g_bf16 ? 2 : 4) + 16.0);
    Prof pr(F_ADAMW, s, 0.0, bytes);
    hipError_t e = launch_adamw(a, s);
    if (e != hipSuccess) return fail(MC_ERR_HIP, "adamw launch: %s", hipGetErrorString(e));
    a.nvec = 0; a.total_blocks = 0;
    return MC_OK;
  };
  a.lr = hp->lr; a.beta1 = hp->beta1; a.beta2 = hp->beta2;
  a.one_m_beta1 = 1.0f - hp->beta1; a.one_m_beta2 = 1.0f - hp->beta2; a.eps = hp->eps;
  a.decay = (float)(1.0 - (double)hp->lr * (double)hp->weight_decay);
  a.c1 = (float)c1; a.c2 = (float)c2;
  for (int i = 0; i < n; ++i) {
    const mc_vector& d = vecs[i];
    if (d.n == 0) continue;
    // a vector whose blocks would overflow one launch's grid index is split
    for (int64_t off = 0; off < d.n;) {
      const int64_t room = ((int64_t)1 << 30) - a.total_blocks;
      const int64_t chunk = std::min<int64_t>(d.n - off, room * 4096);
      if (a.nvec == kMaxBatchVecs || chunk <= 0) {
        mc_status st = flush();
        if (st) return st;
        continue;
      }
      AdamVec& v2 = a.vec[a.nvec++];
      const size_t pe = dtype_size(d.p_dtype), ge = dtype_size(d.g_dtype);
      v2.p = (char*)d.p + off * pe; v2.g = (const char*)d.g + off * ge;
      v2.m = d.m + off; v2.v = d.v + off; v2.n = chunk;
      v2.p_bf16 = d.p_dtype == MC_BF16; v2.g_bf16 = d.g_dtype == MC_BF16;
      v2.vec = aligned(v2.p, 4 * pe) && aligned(v2.g, 4 * ge) && aligned(v2.m, 16) && aligned(v2.v, 16);
      v2.block_start = a.total_blocks;
      a.total_blocks += (int32_t)adamw_blocks(chunk);
      off += chunk;
    }
  }
  return flush();
}

mc_status mc_profile_enable(int32_t on) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  if (on) { g_recs.clear(); g_pool_used = 0; }
  g_prof = on != 0;
  return MC_OK;
}

int32_t mc_profile_read(mc_profile_entry* out, int32_t cap) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  mc_profile_entry agg[F_COUNT];
  memset(agg, 0, sizeof agg);
  for (int f = 0; f < F_COUNT; ++f) snprintf(agg[f].name, sizeof agg[f].name, "%s", kFamilyNames[f]);
  for (const ProfRec& r : g_recs) {
    if (hipEventSynchronize(r.b) != hipSuccess) return fail(MC_ERR_HIP, "event sync failed"), -1;
    float ms = 0.0f;
    if (hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess) return fail(MC_ERR_HIP, "event elapsed failed"), -1;
    agg[r.fam].launches += 1;
    agg[r.fam].ms += ms;
    agg[r.fam].flops += r.flops;
    agg[r.fam].bytes += r.bytes;
  }
  int k = 0;
  for (int f = 0; f < F_COUNT; ++f) {
    if (agg[f].launches == 0) continue;
    if (out && k < cap) out[k] = agg[f];
    ++k;
  }
  return k;
}

}  // extern "C"
