// C ABI of the LaCT fast-weight layer: host-side validation, workspace
// layout and the chunk sequence driver.  Every entry point checks all of its
// arguments before it enqueues anything and allocates no device memory; only
// lact_check_finite and lact_prof_end wait for the device.
#include <hip/hip_runtime.h>

#include <stdint.h>
#include <string.h>

#include <mutex>
#include <set>
#include <utility>
#include <vector>

#include "../../include/lact.h"
#include "lact_internal.hpp"

namespace lact {

hipError_t allow_dynamic_lds(const void* kernel, int bytes) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  static std::mutex mu;
  static std::set<std::pair<const void*, int>> done;
  std::lock_guard<std::mutex> lock(mu);
  if (done.count({kernel, dev}) != 0) return hipSuccess;
  e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess) done.insert({kernel, dev});
  return e;
}

static thread_local int g_last_hip_error = 0;

static lact_status hip_fail(hipError_t e) {
  g_last_hip_error = (int)e;
  return LACT_ERR_HIP;
}

// ------------------------------------------------------------ profiling --
struct Prof {
  int kind = 0;
  int cap = 0;
  int n = 0;
  std::vector<hipEvent_t> ev;
};
static Prof g_prof;

struct ProfScope {
  bool on;
  hipStream_t s;
  ProfScope(int kind, hipStream_t st) : on(g_prof.kind == kind && g_prof.n < g_prof.cap), s(st) {
    if (on) hipEventRecord(g_prof.ev[2 * g_prof.n], s);
  }
  ~ProfScope() {
    if (on) {
      hipEventRecord(g_prof.ev[2 * g_prof.n + 1], s);
      ++g_prof.n;
    }
  }
};

Shadow make_shadow(void* base, int d, int dh) {
  Shadow s;
  s.base = base;
  const int64_t m = (int64_t)d * dh;
  s.per_head = 4 * m;
  s.off_w1 = 0;
  s.off_w3 = m;
  s.off_w2 = 2 * m;
  s.off_w2t = 3 * m;
  return s;
}

static int elem_size(int dtype) { return dtype == LACT_BF16 ? 2 : 4; }

static bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// any_f32_d: fp32 activations at every d (the backward, whose kernels are
// generic); otherwise fp32 activations need d <= 128.
static lact_status check_shape(const lact_shape* sh, bool any_f32_d = false) {
  if (sh == nullptr) return LACT_ERR_INVALID_ARG;
  if (sh->bh < 1 || sh->d < 1 || sh->dh < 1) return LACT_ERR_INVALID_ARG;
  if (sh->dtype != LACT_F32 && sh->dtype != LACT_BF16) return LACT_ERR_INVALID_ARG;
  if (sh->d != 64 && sh->d != 128 && sh->d != 256) return LACT_ERR_UNSUPPORTED;
  if (sh->dh % 64 != 0 || sh->dh < sh->d || sh->dh > 4096) return LACT_ERR_UNSUPPORTED;
  if (sh->dtype == LACT_F32 && sh->d > 128 && !any_f32_d) return LACT_ERR_UNSUPPORTED;
  return LACT_OK;
}

static lact_status check_state(const lact_shape* sh, const lact_state* st, bool need_m) {
  if (st == nullptr) return LACT_ERR_INVALID_ARG;
  const void* req[] = {st->w1, st->w3, st->w2, st->n1, st->n3, st->n2, st->shadow};
  for (const void* p : req) {
    if (p == nullptr) return LACT_ERR_INVALID_ARG;
    if (!aligned16(p)) return LACT_ERR_ALIGNMENT;
  }
  if (need_m) {
    const void* m[] = {st->m1, st->m3, st->m2};
    for (const void* p : m) {
      if (p == nullptr) return LACT_ERR_INVALID_ARG;
      if (!aligned16(p)) return LACT_ERR_ALIGNMENT;
    }
  }
  (void)sh;
  return LACT_OK;
}

static lact_status check_act(const lact_shape* sh, const void* p, lact_layout l, int64_t n_tok) {
  if (n_tok == 0) return LACT_OK;
  if (p == nullptr) return LACT_ERR_INVALID_ARG;
  if (l.stride_tok < sh->d || l.stride_bh < 0) return LACT_ERR_INVALID_ARG;
  const int es = elem_size(sh->dtype);
  if (!aligned16(p) || (l.stride_tok * es) % 16 != 0 || (l.stride_bh * es) % 16 != 0)
    return LACT_ERR_ALIGNMENT;
  return LACT_OK;
}

static lact_status check_opts(const lact_update_opts* o) {
  if (o == nullptr) return LACT_ERR_INVALID_ARG;
  if (!(o->renorm_eps >= 0.f) || !(o->ns_eps >= 0.f)) return LACT_ERR_INVALID_ARG;
  if (o->renorm < 0 || o->renorm > 2) return LACT_ERR_INVALID_ARG;
  if (o->ns_prec != LACT_NS_BF16_SHIFTED && o->ns_prec != LACT_NS_BF16 && o->ns_prec != LACT_NS_F32)
    return LACT_ERR_INVALID_ARG;
  if (o->nonfinite != nullptr && ((uintptr_t)o->nonfinite & 3u) != 0) return LACT_ERR_ALIGNMENT;
  if (o->eta_per_channel != 0 && o->eta_per_channel != 1) return LACT_ERR_INVALID_ARG;
  return LACT_OK;
}

// ------------------------------------------------------------ workspace --
static int64_t align256(int64_t x) { return (x + 255) & ~(int64_t)255; }

// Token splits of the gradient launch.  Its bf16 workgroups run one per
// compute unit, in rounds of 256; a split costs its 32-token tiles in every
// round and one more partial set (written, then read by the reduction).
// The split count minimises
//     rounds * tiles per split * t_tile + splits * t_partial
// with t_tile = 12 d hpb flop per token x 32 tokens at ~2.8 TFLOP/s per CU and
// t_partial = 2 x 3 d dh bh x 4 bytes at ~5 TB/s, over at most two rounds
// (so the workspace bound below holds for every token count).
static int nsplit_bound(const lact_shape* sh, int64_t n_tok) {
  const int hpb = grad_hidden_per_block(sh->dtype, sh->d, false);
  const int64_t base = (int64_t)sh->bh * ((sh->dh + hpb - 1) / hpb);
  int64_t ns = (512 + base - 1) / base;
  const int64_t tiles = (n_tok + 31) / 32;
  if (ns > tiles) ns = tiles;
  if (ns > 64) ns = 64;
  return ns < 1 ? 1 : (int)ns;
}

// generic: the gradient runs on the generic kernel (fp32 shapes, per-channel
// learning rates).
static int choose_nsplit(const lact_shape* sh, int64_t n_tok, bool generic) {
  const int hpb = grad_hidden_per_block(sh->dtype, sh->d, generic);
  const int64_t base = (int64_t)sh->bh * ((sh->dh + hpb - 1) / hpb);
  if (generic) {
    // several workgroups per CU; at least 256 tokens per split
    int64_t ns = (256 + base - 1) / base;
    const int64_t cap = (n_tok + 255) / 256;
    if (ns > cap) ns = cap;
    if (ns > 64) ns = 64;
    return ns < 1 ? 1 : (int)ns;
  }
  const int lim = nsplit_bound(sh, n_tok);
  const int64_t tiles = (n_tok + 31) / 32;
  const double t_tile = 32.0 * 12.0 * sh->d * hpb / 2.8e12;
  const double t_part = 2.0 * 3.0 * sh->d * sh->dh * (double)sh->bh * 4.0 / 5e12;
  int best = 1;
  double best_t = 0.0;
  for (int ns = 1; ns <= lim; ++ns) {
    const int64_t rounds = (base * ns + 255) / 256;
    const int64_t per = (tiles + ns - 1) / ns;
    const double t = (double)(rounds * per) * t_tile + (ns > 1 ? ns * t_part : 0.0);
    if (ns == 1 || t < best_t) { best = ns; best_t = t; }
  }
  return best;
}

struct Workspace {
  float* partial;
  float* beta;    // [bh] momentum coefficient of the write
  float* g;       // 3 wide matrices per head: [3][bh][d][dh]
  float* xa;      // Newton-Schulz buffers
  float* xb;
  float* xh;
  float* amat;    // [3 bh][d][d]
  float* bmat;
  float* ssp;     // Newton-Schulz tile sums of squares, 2 x [3 bh][tiles]
  void* shadow2;  // second operand copy of the weights (ns_step_fused shapes)
  int64_t bytes;
};

// Shapes whose Newton-Schulz workgroups also take the weight step (and can
// share their launch with a read, which then needs a second shadow).
static bool ns_step_fused(const lact_shape* sh, const lact_update_opts* op) {
  return op != nullptr && op->use_muon && op->ns_prec != LACT_NS_F32 && sh->dtype == LACT_BF16 &&
         !op->eta_per_channel && sh->d == 128 && (sh->dh == 256 || sh->dh == 512);
}

// The write's gradient runs on the generic kernel.
static bool generic_grad(const lact_shape* sh, const lact_update_opts* op) {
  return sh->dtype != LACT_BF16 || (op != nullptr && op->eta_per_channel);
}

// Precision of a write's Newton-Schulz products: fp32 shapes always use fp32
// operands.
static int ns_prec_of(const lact_shape* sh, const lact_update_opts* op) {
  return sh->dtype == LACT_F32 ? (int)LACT_NS_F32 : op->ns_prec;
}

// First shifted step (lact_ns_prec): the last three of the five.
static int ns_shift_from(int prec) { return prec == LACT_NS_BF16_SHIFTED ? 2 : 5; }

// fused: the shape's Newton-Schulz workgroups sum the split partials and take
// the step themselves (ns_step_fused), so the write needs the second operand
// copy but neither the reduced gradient nor the batched Newton-Schulz buffers.
static Workspace layout_ws(const lact_shape* sh, int nsplit, bool muon, char* base,
                           bool fused = false) {
  Workspace w;
  const int64_t msz = (int64_t)sh->d * sh->dh;
  int64_t off = 0;
  auto take = [&](int64_t nfloat) {
    float* p = base ? reinterpret_cast<float*>(base + off) : nullptr;
    off += align256(nfloat * 4);
    return p;
  };
  // first, so that its place does not depend on the split count: operand
  // copies, 4 d dh bf16 per head
  w.shadow2 = fused ? take((int64_t)sh->bh * 2 * msz) : nullptr;
  w.partial = take((int64_t)nsplit * sh->bh * 3 * msz);
  w.beta = take(sh->bh);
  w.g = fused ? nullptr : take((int64_t)3 * sh->bh * msz);
  if (muon && !fused) {
    w.xa = take((int64_t)3 * sh->bh * msz);
    w.xb = take((int64_t)3 * sh->bh * msz);
    w.xh = take((int64_t)3 * sh->bh * msz);
    w.amat = take((int64_t)3 * sh->bh * sh->d * sh->d);
    w.bmat = take((int64_t)3 * sh->bh * sh->d * sh->d);
    w.ssp = take((int64_t)2 * 3 * sh->bh * (sh->d / 64) * (sh->dh / 64));
  } else {
    w.xa = w.xb = w.xh = w.amat = w.bmat = w.ssp = nullptr;
  }
  w.bytes = off;
  return w;
}

// ------------------------------------------------------- Newton-Schulz --
static const float kNS[5][3] = {
    {4.0848f, -6.8946f, 2.9270f}, {3.9505f, -6.3029f, 2.6377f}, {3.7418f, -5.5913f, 2.3037f},
    {2.8769f, -3.1427f, 1.2046f}, {2.8366f, -3.0525f, 1.2012f}};

// Newton-Schulz workspace: X fp32 twice, the bf16 copies of X (two, in one
// fp32-sized region), A / B bf16 (one region), A fp32, and the tile sums of
// squares of X (the shifted steps' mu).
static int64_t ns_ws_bytes(int count, int rows, int cols) {
  const int64_t m = (int64_t)rows * cols;
  const int64_t tiles = (int64_t)(rows / 64) * (cols / 64);
  return 3 * align256((int64_t)count * m * 4) + 2 * align256((int64_t)count * rows * rows * 4) +
         align256(2 * (int64_t)count * tiles * 4);
}

// pre_np > 0: bm already holds pre_np partial sums of squares per matrix of
// the input (the split sum wrote them), for the normalisation of the
// batched-GEMM path.
// u_tall: NULL, or the number of leading matrices whose result may be
// written transposed ([cols][rows]); set to the number actually written so
// (the batched-GEMM path honours it, the one-workgroup kernels do not).
static hipError_t run_ns(int prec, int count, int rows, int cols, NsIn g, float* u,
                         float eps, float* xa, float* xb, float* xh, float* am, float* bm,
                         float* ssp, hipStream_t s, int pre_np = 0, int* u_tall = nullptr) {
  const int want_tall = u_tall != nullptr ? *u_tall : 0;
  if (u_tall != nullptr) *u_tall = 0;
  const int64_t m = (int64_t)rows * cols;
  const int shift_from = ns_shift_from(prec);
  hipError_t e = hipErrorNotSupported;
  if (prec != LACT_NS_F32) e = launch_ns_fused(count, rows, cols, g, u, eps, shift_from, s);
  if (e != hipErrorNotSupported) return e;
  if (prec != LACT_NS_F32) {
    // X fp32 in xa / xb, its bf16 copy in the two halves of xh; A fp32 in bm,
    // A and B bf16 in am; ssp: the tile sums of squares of X_k in half k % 2
    typedef __bf16 bf16;
    bf16* xh0 = reinterpret_cast<bf16*>(xh);
    bf16* xh1 = xh0 + (int64_t)count * m;
    bf16* ah = reinterpret_cast<bf16*>(am);
    bf16* bh = ah + (int64_t)count * rows * rows;
    const int64_t rr = (int64_t)rows * rows;
    const int tiles = (rows / 64) * (cols / 64);
    if ((e = launch_nsn(g, bm, xa, xh0, count, m, eps, s, pre_np)) != hipSuccess) return e;
    float* x = xa;
    float* y = xb;
    bf16* xc = xh0;
    bf16* yc = xh1;
    for (int it = 0; it < 5; ++it) {
      const float ca = kNS[it][0], cb = kNS[it][1], cc = kNS[it][2];
      // shifted step (mu = ||X||_F^2 / rows = trace(A) / rows from the tile
      // sums the previous step left): A_s = A - mu I, B_s = c A_s A_s +
      // (b + 2 c mu) A_s = B - (b mu + c mu^2) I, X' = B_s X + (a + b mu +
      // c mu^2) X - the same step in exact arithmetic
      const bool shf = it >= shift_from;
      const float* mp = shf ? ssp + (int64_t)(it & 1) * count * tiles : nullptr;
      // A = X X^T (fp32 for the b A term, bf16 operand)
      NsGemmArgs ga{xc, m, cols, xc, m, cols, nullptr, 0, bm, ah, rr, rows, rows, cols, 1.f, 0.f,
                    mp, tiles, (float)rows, 0.f, 0.f, -1.f, nullptr, 1};
      if ((e = launch_nsgemm(false, ga, count, s)) != hipSuccess) return e;
      // B = c A A + b A (A symmetric: its rows are the B operand)
      NsGemmArgs gb{ah, rr, rows, ah, rr, rows, bm, rr, nullptr, bh, rr, rows, rows, rows, cc, cb,
                    mp, tiles, (float)rows, 2.f * cc, 0.f, 0.f, nullptr, 1};
      if ((e = launch_nsgemm(false, gb, count, s)) != hipSuccess) return e;
      // X' = B X + a X (and its tile sums of squares for a shifted next step)
      const bool last = it == 4;
      NsGemmArgs gx{bh, rr, rows, xc, m, cols, x, m, last ? u : y, last ? nullptr : yc, m,
                    rows, cols, rows, 1.f, ca, mp, tiles, (float)rows, cb, cc, 0.f,
                    (!last && it + 1 >= shift_from) ? ssp + (int64_t)((it + 1) & 1) * count * tiles
                                                    : nullptr, 0, last ? want_tall : 0};
      if ((e = launch_nsgemm(true, gx, count, s)) != hipSuccess) return e;
      std::swap(x, y);
      std::swap(xc, yc);
    }
    if (u_tall != nullptr) *u_tall = want_tall;
    return hipSuccess;
  }
  NsNormArgs na{g, xa, count, m, eps};
  e = launch_ns_norm(na, s);
  if (e != hipSuccess) return e;
  float* x = xa;
  float* y = xb;
  for (int it = 0; it < 5; ++it) {
    const float ca = kNS[it][0], cb = kNS[it][1], cc = kNS[it][2];
    // A = X X^T
    GemmArgs ga{x, m, x, m, 0, nullptr, 0, am, (int64_t)rows * rows, rows, rows, cols, count, 1.f, 0.f};
    if ((e = launch_gemm(LACT_F32, ga, s)) != hipSuccess) return e;
    // B = c A A + b A
    GemmArgs gb{am, (int64_t)rows * rows, am, (int64_t)rows * rows, 1, am, (int64_t)rows * rows,
                bm, (int64_t)rows * rows, rows, rows, rows, count, cc, cb};
    if ((e = launch_gemm(LACT_F32, gb, s)) != hipSuccess) return e;
    // X' = B X + a X
    float* out = (it == 4) ? u : y;
    GemmArgs gx{bm, (int64_t)rows * rows, x, m, 1, x, m, out, m, rows, cols, rows, count, 1.f, ca};
    if ((e = launch_gemm(LACT_F32, gx, s)) != hipSuccess) return e;
    float* t = x;
    x = y;
    y = t;
  }
  return hipSuccess;
}

// -------------------------------------------------------------- pieces --
// A read (apply) that the drivers may hand to the next write: within one
// chunk step the read and the write gradient both use the current weights and
// only the step kernel replaces them, so the read can share the
// Newton-Schulz launch (which alone leaves most compute units idle).
struct ApplyJob {
  const void* q;
  lact_layout ql;
  void* o;
  lact_layout ol;
  int64_t n_tok;
};

static ApplyArgs apply_args(const lact_shape* sh, const lact_state* st, const void* q,
                            lact_layout ql, void* o, lact_layout ol, int64_t n_tok) {
  ApplyArgs a;
  a.q = q; a.q_sbh = ql.stride_bh; a.q_st = ql.stride_tok;
  a.o = o; a.o_sbh = ol.stride_bh; a.o_st = ol.stride_tok;
  a.sh = make_shadow(st->shadow, sh->d, sh->dh);
  a.bh = sh->bh; a.d = sh->d; a.dh = sh->dh; a.n_tok = n_tok;
  return a;
}

static lact_status do_apply(const lact_shape* sh, const lact_state* st, const void* q,
                            lact_layout ql, void* o, lact_layout ol, int64_t n_tok,
                            hipStream_t s, int max_blocks = 0) {
  if (n_tok == 0) return LACT_OK;
  const ApplyArgs a = apply_args(sh, st, q, ql, o, ol, n_tok);
  hipError_t e;
  {
    ProfScope p(LACT_PROF_APPLY, s);
    e = launch_apply(sh->dtype, a, s, max_blocks);
  }
  return e == hipSuccess ? LACT_OK : hip_fail(e);
}


// ------------------------------------------- the read on a second stream --
// With d = 256 and Muon, a write's Newton-Schulz is 17 small launches that
// leave most compute units idle, while the read of the chunk (which needs
// only the weights this write replaces) is a long MFMA launch.  The read
// then runs on a library-owned stream: forked from the caller's stream
// after the gradient launch (before the split sum), on three quarters of
// the compute units (its workgroups loop over the tiles, so the rest stay
// free for Newton-Schulz), and joined back before the step.  One stream and
// two events per device, created on first use (never while the caller's
// stream is being captured: the write then stays on one stream) and kept
// until the process ends.
struct SideStream {
  hipStream_t s = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
  int read_blocks = 0;
  // held from the fork's record to the join's wait: the events are shared
  // by every caller on the device, and a wait must see its own record
  mutable std::mutex mu;
};

static const SideStream* side_stream(hipStream_t caller) {
  static std::mutex mu;
  static SideStream sides[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  SideStream& sd = sides[dev];
  if (sd.s != nullptr) return &sd;
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(caller, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone) return nullptr;
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 8)
    return nullptr;
  hipStream_t st = nullptr;
  hipEvent_t f = nullptr, j = nullptr;
  if (hipStreamCreateWithFlags(&st, hipStreamNonBlocking) != hipSuccess) return nullptr;
  // (same-device ordering only: no system-scope fence)
  const unsigned fl = hipEventDisableTiming | hipEventDisableSystemFence;
  if (hipEventCreateWithFlags(&f, fl) != hipSuccess || hipEventCreateWithFlags(&j, fl) != hipSuccess) {
    if (f != nullptr) hipEventDestroy(f);
    hipStreamDestroy(st);
    return nullptr;
  }
  sd.fork = f;
  sd.join = j;
  sd.read_blocks = cus * 3 / 4;
  sd.s = st;
  return &sd;
}

// The shapes whose writes fork their read (the large-matrix Newton-Schulz).
static bool forks_read(const lact_shape* sh, const lact_update_opts* op) {
  return sh->dtype == LACT_BF16 && sh->d == 256 && op->use_muon != 0;
}

// The read of `job` on the second stream, after everything enqueued on s so
// far; the caller holds side->mu until it has made s wait for side->join.
static lact_status fork_read(const SideStream* side, const lact_shape* sh, const lact_state* st,
                             const ApplyJob* job, hipStream_t s) {
  hipError_t e = hipEventRecord(side->fork, s);
  if (e == hipSuccess) e = hipStreamWaitEvent(side->s, side->fork, 0);
  if (e != hipSuccess) return hip_fail(e);
  const lact_status r = do_apply(sh, st, job->q, job->ql, job->o, job->ol, job->n_tok, side->s,
                                 side->read_blocks);
  if (r != LACT_OK) return r;
  e = hipEventRecord(side->join, side->s);
  return e == hipSuccess ? LACT_OK : hip_fail(e);
}

static lact_status do_grad(const lact_shape* sh, const lact_state* st, const void* k,
                           lact_layout kl, const void* v, lact_layout vl, const float* e1,
                           const float* e3, const float* e2, int64_t esbh, int64_t n_tok,
                           const Workspace& w, int nsplit, float* o1, float* o3, float* o2,
                           float* m1, float* m3, float* m2, const float* mom, hipStream_t s,
                           bool reduce = true, int eta_per_channel = 0,
                           const SideStream* side = nullptr, const ApplyJob* job = nullptr,
                           float* ss_part = nullptr) {
  GradArgs a;
  a.k = k; a.k_sbh = kl.stride_bh; a.k_st = kl.stride_tok;
  a.v = v; a.v_sbh = vl.stride_bh; a.v_st = vl.stride_tok;
  a.eta1 = e1; a.eta3 = e3; a.eta2 = e2; a.eta_sbh = esbh;
  a.eta_per_channel = eta_per_channel;
  a.sh = make_shadow(st->shadow, sh->d, sh->dh);
  a.bh = sh->bh; a.d = sh->d; a.dh = sh->dh; a.n_tok = n_tok;
  a.nsplit = nsplit;
  int64_t sl = (n_tok + nsplit - 1) / nsplit;
  sl = (sl + 31) / 32 * 32;
  a.split_len = sl > 0 ? sl : 32;
  a.partial = w.partial;
  a.mom = mom; a.mom_sbh = esbh; a.beta = w.beta;
  // without the reduction launch, its consumer finishes the sum: the
  // momentum is folded into split 0 here
  a.mo1 = reduce ? nullptr : m1;
  a.mo3 = reduce ? nullptr : m3;
  a.mo2 = reduce ? nullptr : m2;
  hipError_t e;
  {
    ProfScope p(LACT_PROF_GRAD, s);
    e = launch_grad(sh->dtype, a, s);
  }
  if (e != hipSuccess) return hip_fail(e);
  if (side != nullptr) {
    // the gradient launch is the last one on s that the read must follow
    // (it uses the weights the write replaces), so the read leaves here
    const lact_status rr = fork_read(side, sh, st, job, s);
    if (rr != LACT_OK) return rr;
  }
  if (!reduce) return LACT_OK;  // the consumer sums the partials itself
  ReduceArgs r{w.partial, nsplit, sh->bh, sh->d, sh->dh, o1, o3, o2, m1, m3, m2, w.beta, ss_part};
  {
    ProfScope p(LACT_PROF_REDUCE, s);
    e = launch_reduce(r, s);
  }
  return e == hipSuccess ? LACT_OK : hip_fail(e);
}

static lact_status do_step(const lact_shape* sh, const lact_state* st, const float* u1,
                           const float* u3, const float* u2, int renorm, float eps,
                           int* nonfinite, void* shadow_out, hipStream_t s, int u13_tall = 0) {
  StepArgs a;
  memset(&a, 0, sizeof(a));
  a.w1 = st->w1; a.w3 = st->w3; a.w2 = st->w2;
  a.u1 = u1; a.u3 = u3; a.u2 = u2;
  a.u13_tall = u13_tall;
  a.n1 = st->n1; a.n3 = st->n3; a.n2 = st->n2;
  a.sh = make_shadow(shadow_out, sh->d, sh->dh);
  a.bh = sh->bh; a.d = sh->d; a.dh = sh->dh;
  a.renorm = renorm; a.eps = eps;
  a.nonfinite = nonfinite;
  hipError_t e;
  {
    ProfScope p(LACT_PROF_STEP, s);
    e = launch_step(sh->dtype, a, s);
  }
  return e == hipSuccess ? LACT_OK : hip_fail(e);
}

// One write.  The weights are read through st->shadow and their new operand
// copies go to shadow_out (NULL: st->shadow, in place).  job: a read with the
// weights this write replaces; it shares the Newton-Schulz launch where that
// kernel supports it and shadow_out is another buffer, else it runs first.
static lact_status do_update(const lact_shape* sh, const lact_state* st, const void* k,
                             lact_layout kl, const void* v, lact_layout vl, const float* e1,
                             const float* e3, const float* e2, const float* mom, int64_t esbh,
                             int64_t n_tok, const lact_update_opts* op, void* ws,
                             hipStream_t s, const ApplyJob* job = nullptr,
                             void* shadow_out = nullptr, const SideStream* side = nullptr) {
  if (shadow_out == nullptr) shadow_out = st->shadow;
  const bool nsstep = ns_step_fused(sh, op);
  const bool fuse = nsstep && job != nullptr && job->n_tok > 0 && shadow_out != st->shadow;
  const bool fork = side != nullptr && job != nullptr && job->n_tok > 0 && !fuse && !nsstep &&
                    forks_read(sh, op);
  if (job != nullptr && !fuse && !fork) {
    lact_status r = do_apply(sh, st, job->q, job->ql, job->o, job->ol, job->n_tok, s);
    if (r != LACT_OK) return r;
  }
  const int nsplit = choose_nsplit(sh, n_tok, generic_grad(sh, op));
  Workspace w = layout_ws(sh, nsplit, op->use_muon != 0, reinterpret_cast<char*>(ws), nsstep);
  const int64_t msz = (int64_t)sh->d * sh->dh;
  const int64_t mall = (int64_t)sh->bh * msz;
  // the reduced gradient (not laid out when the Newton-Schulz workgroups sum
  // the partials themselves)
  float* g1 = w.g;
  float* g3 = w.g ? w.g + mall : nullptr;
  float* g2 = w.g ? w.g + 2 * mall : nullptr;
  // with momentum the reduced gradient lives in M only (M <- G + beta M)
  const bool mo = op->use_momentum != 0;
  // with a forked read, side->mu is held from the fork to the join's wait:
  // the events are shared by every caller on the device
  std::unique_lock<std::mutex> side_lock;
  if (fork) side_lock = std::unique_lock<std::mutex>(side->mu);
  // with Newton-Schulz after the split sum, the sum also takes the first
  // pass of its Frobenius normalisation (per-tile sums of squares)
  const bool pre_norm = op->use_muon && !nsstep;
  int tall = 0;  // leading matrices of the Newton-Schulz output in W's layout
  lact_status r = do_grad(sh, st, k, kl, v, vl, e1, e3, e2, esbh, n_tok, w, nsplit,
                          mo ? nullptr : g1, mo ? nullptr : g3, mo ? nullptr : g2,
                          mo ? st->m1 : nullptr, mo ? st->m3 : nullptr, mo ? st->m2 : nullptr,
                          mo ? mom : nullptr, s, !nsstep, op->eta_per_channel,
                          fork ? side : nullptr, fork ? job : nullptr, pre_norm ? w.bmat : nullptr);
  if (r != LACT_OK) return r;
  const float* u1 = mo ? st->m1 : g1;
  const float* u3 = mo ? st->m3 : g3;
  const float* u2 = mo ? st->m2 : g2;
  if (op->use_muon) {
    ProfScope p(LACT_PROF_NS, s);
    const NsIn in{{u1, u3, u2}, sh->bh};
    hipError_t e;
    if (nsstep) {
      // Newton-Schulz workgroups sum the split partials (+ momentum) and take
      // the step; the read (if fused) fills the other compute units
      ApplyArgs aa;
      if (fuse) {
        aa = apply_args(sh, st, job->q, job->ql, job->o, job->ol, job->n_tok);
      } else {
        memset(&aa, 0, sizeof(aa));
        aa.n_tok = 0;
      }
      const NsStep ns{st->w1, st->w3, st->w2, st->n1, st->n3, st->n2,
                      make_shadow(shadow_out, sh->d, sh->dh), sh->bh, op->renorm,
                      op->renorm_eps, op->nonfinite};
      const NsGrad gr{w.partial, nsplit, sh->bh,
                      {mo ? st->m1 : nullptr, mo ? st->m3 : nullptr, mo ? st->m2 : nullptr}};
      e = launch_ns_step_apply(3 * sh->bh, sh->d, sh->dh, gr, op->ns_eps,
                               ns_shift_from(ns_prec_of(sh, op)), ns, aa, s);
      return e == hipSuccess ? LACT_OK : hip_fail(e);
    }
    // the W1 and W3 updates (the first 2 bh matrices) written in the layout
    // of W1 and W3 when the path allows it: the step then reads them as rows
    tall = 2 * sh->bh;
    e = run_ns(ns_prec_of(sh, op), 3 * sh->bh, sh->d, sh->dh, in, w.g, op->ns_eps, w.xa, w.xb,
               w.xh, w.amat, w.bmat, w.ssp, s, (sh->d / 64) * (sh->dh / 64), &tall);
    if (e != hipSuccess) return hip_fail(e);
    u1 = g1; u3 = g3; u2 = g2;
  }
  if (fork) {
    // the step rewrites the operand copies the read uses: join first
    const hipError_t e = hipStreamWaitEvent(s, side->join, 0);
    if (e != hipSuccess) return hip_fail(e);
  }
  return do_step(sh, st, u1, u3, u2, op->renorm, op->renorm_eps, op->nonfinite, shadow_out,
                 s, tall > 0 ? 1 : 0);
}

static lact_status check_update_args(const lact_shape* sh, const lact_state* st, const void* k,
                                     lact_layout kl, const void* v, lact_layout vl,
                                     const float* e1, const float* e3, const float* e2,
                                     const float* mom, int64_t esbh, int64_t n_tok,
                                     const lact_update_opts* op, const void* ws,
                                     size_t ws_bytes) {
  lact_status r;
  if ((r = check_shape(sh)) != LACT_OK) return r;
  if ((r = check_opts(op)) != LACT_OK) return r;
  if (op->eta_per_channel && sh->d > 128) return LACT_ERR_UNSUPPORTED;
  if ((r = check_state(sh, st, op->use_momentum != 0)) != LACT_OK) return r;
  if (n_tok < 0) return LACT_ERR_INVALID_ARG;
  if ((r = check_act(sh, k, kl, n_tok)) != LACT_OK) return r;
  if ((r = check_act(sh, v, vl, n_tok)) != LACT_OK) return r;
  if (n_tok > 0 && (e1 == nullptr || e3 == nullptr || e2 == nullptr)) return LACT_ERR_INVALID_ARG;
  if (op->use_momentum && n_tok > 0 && mom == nullptr) return LACT_ERR_INVALID_ARG;
  if (esbh < 0) return LACT_ERR_INVALID_ARG;
  const size_t need = lact_workspace_bytes(sh, n_tok, op);
  if (ws == nullptr || ws_bytes < need) return LACT_ERR_WORKSPACE;
  if (!aligned16(ws)) return LACT_ERR_ALIGNMENT;
  return LACT_OK;
}

// The workspace's second shadow (NULL when the shape does not use one).
static void* second_shadow(const lact_shape* sh, const lact_update_opts* op, void* ws) {
  if (!ns_step_fused(sh, op)) return nullptr;
  return layout_ws(sh, 1, op->use_muon != 0, reinterpret_cast<char*>(ws), true).shadow2;
}

}  // namespace lact

using namespace lact;

extern "C" {

size_t lact_shadow_bytes(const lact_shape* sh) {
  if (check_shape(sh) != LACT_OK) return 0;
  return (size_t)sh->bh * 4 * (size_t)sh->d * sh->dh * elem_size(sh->dtype);
}

size_t lact_workspace_bytes(const lact_shape* sh, int64_t max_update_tokens,
                            const lact_update_opts* opts) {
  if (check_shape(sh) != LACT_OK || max_update_tokens < 0) return 0;
  const bool muon = opts != nullptr && opts->use_muon != 0;
  const int ns = generic_grad(sh, opts) ? choose_nsplit(sh, max_update_tokens, true)
                                        : nsplit_bound(sh, max_update_tokens);
  return (size_t)layout_ws(sh, ns, muon, nullptr, ns_step_fused(sh, opts)).bytes;
}

size_t lact_ns_workspace_bytes(int32_t count, int32_t rows, int32_t cols) {
  if (count < 1 || rows < 1 || cols < 1) return 0;
  return (size_t)ns_ws_bytes(count, rows, cols);
}

lact_status lact_init_state(const lact_shape* sh, const lact_state* st, void* stream) {
  lact_status r;
  if ((r = check_shape(sh)) != LACT_OK) return r;
  if ((r = check_state(sh, st, false)) != LACT_OK) return r;
  for (float* m : {st->m1, st->m3, st->m2})
    if (m != nullptr && !aligned16(m)) return LACT_ERR_ALIGNMENT;
  hipStream_t s = (hipStream_t)stream;
  // one launch: row norms, operand copies, momentum buffers zeroed
  StepArgs a;
  memset(&a, 0, sizeof(a));
  a.w1 = st->w1; a.w3 = st->w3; a.w2 = st->w2;
  a.n1 = st->n1; a.n3 = st->n3; a.n2 = st->n2;
  a.sh = make_shadow(st->shadow, sh->d, sh->dh);
  a.bh = sh->bh; a.d = sh->d; a.dh = sh->dh;
  a.renorm = 0;
  a.init = 1;
  a.mz1 = st->m1; a.mz3 = st->m3; a.mz2 = st->m2;
  const hipError_t e = launch_step(sh->dtype, a, s);
  return e == hipSuccess ? LACT_OK : hip_fail(e);
}

lact_status lact_apply(const lact_shape* sh, const lact_state* st, const void* q,
                       lact_layout ql, void* o, lact_layout ol, int64_t n_tok, void* stream) {
  lact_status r;
  if ((r = check_shape(sh)) != LACT_OK) return r;
  if ((r = check_state(sh, st, false)) != LACT_OK) return r;
  if (n_tok < 0) return LACT_ERR_INVALID_ARG;
  if ((r = check_act(sh, q, ql, n_tok)) != LACT_OK) return r;
  if ((r = check_act(sh, o, ol, n_tok)) != LACT_OK) return r;
  if (n_tok > 0 && q == o) return LACT_ERR_INVALID_ARG;
  return do_apply(sh, st, q, ql, o, ol, n_tok, (hipStream_t)stream);
}

size_t lact_decode_workspace_bytes(const lact_shape* sh, int64_t n_tok) {
  if (check_shape(sh) != LACT_OK || n_tok < 1 || n_tok > LACT_DECODE_MAX_TOKENS) return 0;
  const int nb = decode_blocks(sh->dtype, sh->bh, sh->d, sh->dh);
  return (size_t)align256((int64_t)sh->bh * nb * n_tok * sh->d * 4);
}

lact_status lact_decode_apply(const lact_shape* sh, const lact_state* st, const void* q,
                              lact_layout ql, void* o, lact_layout ol, int64_t n_tok, void* ws,
                              size_t ws_bytes, void* stream) {
  lact_status r;
  if ((r = check_shape(sh)) != LACT_OK) return r;
  if ((r = check_state(sh, st, false)) != LACT_OK) return r;
  if (n_tok < 0 || n_tok > LACT_DECODE_MAX_TOKENS) return LACT_ERR_INVALID_ARG;
  if ((r = check_act(sh, q, ql, n_tok)) != LACT_OK) return r;
  if ((r = check_act(sh, o, ol, n_tok)) != LACT_OK) return r;
  if (n_tok == 0) return LACT_OK;
  if (q == o) return LACT_ERR_INVALID_ARG;
  if (ws == nullptr || ws_bytes < lact_decode_workspace_bytes(sh, n_tok)) return LACT_ERR_WORKSPACE;
  if (!aligned16(ws)) return LACT_ERR_ALIGNMENT;
  DecodeArgs a;
  a.q = q; a.q_sbh = ql.stride_bh; a.q_st = ql.stride_tok;
  a.o = o; a.o_sbh = ol.stride_bh; a.o_st = ol.stride_tok;
  a.sh = make_shadow(st->shadow, sh->d, sh->dh);
  a.bh = sh->bh; a.d = sh->d; a.dh = sh->dh; a.n = (int)n_tok;
  a.nblk = decode_blocks(sh->dtype, sh->bh, sh->d, sh->dh);
  a.part = reinterpret_cast<float*>(ws);
  const hipError_t e = launch_decode(sh->dtype, a, (hipStream_t)stream);
  return e == hipSuccess ? LACT_OK : hip_fail(e);
}

lact_status lact_gradient(const lact_shape* sh, const lact_state* st, const void* k,
                          lact_layout kl, const void* v, lact_layout vl, const float* e1,
                          const float* e3, const float* e2, int64_t esbh, int64_t n_tok,
                          float* g1, float* g3, float* g2, void* ws, size_t ws_bytes,
                          void* stream) {
  lact_update_opts op;
  memset(&op, 0, sizeof(op));
  lact_status r = check_update_args(sh, st, k, kl, v, vl, e1, e3, e2, nullptr, esbh, n_tok, &op,
                                    ws, ws_bytes);
  if (r != LACT_OK) return r;
  for (float* gp : {g1, g3, g2}) {
    if (gp == nullptr) return LACT_ERR_INVALID_ARG;
    if (!aligned16(gp)) return LACT_ERR_ALIGNMENT;
  }
  const int nsplit = choose_nsplit(sh, n_tok, generic_grad(sh, &op));
  Workspace w = layout_ws(sh, nsplit, false, reinterpret_cast<char*>(ws));
  return do_grad(sh, st, k, kl, v, vl, e1, e3, e2, esbh, n_tok, w, nsplit, g1, g3, g2, nullptr,
                 nullptr, nullptr, nullptr, (hipStream_t)stream);
}

lact_status lact_newton_schulz(int32_t count, int32_t rows, int32_t cols, int32_t prec,
                               const float* g, float* u, float eps, void* ws, size_t ws_bytes,
                               void* stream) {
  if (count < 1 || rows < 1 || cols < 1 || g == nullptr || u == nullptr) return LACT_ERR_INVALID_ARG;
  if (prec != LACT_NS_BF16_SHIFTED && prec != LACT_NS_BF16 && prec != LACT_NS_F32)
    return LACT_ERR_INVALID_ARG;
  if (!(eps >= 0.f)) return LACT_ERR_INVALID_ARG;
  if (rows % 64 != 0 || cols % 64 != 0 || rows > cols) return LACT_ERR_UNSUPPORTED;
  if (!aligned16(g) || !aligned16(u)) return LACT_ERR_ALIGNMENT;
  if (ws == nullptr || ws_bytes < (size_t)ns_ws_bytes(count, rows, cols)) return LACT_ERR_WORKSPACE;
  if (!aligned16(ws)) return LACT_ERR_ALIGNMENT;
  char* b = reinterpret_cast<char*>(ws);
  const int64_t xm = align256((int64_t)count * rows * cols * 4);
  const int64_t am = align256((int64_t)count * rows * rows * 4);
  float* xa = reinterpret_cast<float*>(b);
  float* xb = reinterpret_cast<float*>(b + xm);
  float* xh = reinterpret_cast<float*>(b + 2 * xm);
  float* a_ = reinterpret_cast<float*>(b + 3 * xm);
  float* b_ = reinterpret_cast<float*>(b + 3 * xm + am);
  float* ssp = reinterpret_cast<float*>(b + 3 * xm + 2 * am);
  const NsIn in{{g, g, g}, count};
  hipError_t e = run_ns(prec, count, rows, cols, in, u, eps, xa, xb, xh, a_, b_, ssp,
                        (hipStream_t)stream);
  return e == hipSuccess ? LACT_OK : hip_fail(e);
}

lact_status lact_step_renorm(const lact_shape* sh, const lact_state* st, const float* u1,
                             const float* u3, const float* u2, const lact_update_opts* op,
                             void* ws, size_t ws_bytes, void* stream) {
  lact_status r;
  if ((r = check_shape(sh)) != LACT_OK) return r;
  if ((r = check_opts(op)) != LACT_OK) return r;
  if ((r = check_state(sh, st, false)) != LACT_OK) return r;
  for (const float* up : {u1, u3, u2}) {
    if (up == nullptr) return LACT_ERR_INVALID_ARG;
    if (!aligned16(up)) return LACT_ERR_ALIGNMENT;
  }
  if (ws == nullptr || ws_bytes < lact_workspace_bytes(sh, 0, op)) return LACT_ERR_WORKSPACE;
  if (!aligned16(ws)) return LACT_ERR_ALIGNMENT;
  return do_step(sh, st, u1, u3, u2, op->renorm, op->renorm_eps, op->nonfinite, st->shadow,
                 (hipStream_t)stream);
}

lact_status lact_update(const lact_shape* sh, const lact_state* st, const void* k,
                        lact_layout kl, const void* v, lact_layout vl, const float* e1,
                        const float* e3, const float* e2, const float* mom, int64_t esbh,
                        int64_t n_tok, const lact_update_opts* op, void* ws, size_t ws_bytes,
                        void* stream) {
  lact_status r = check_update_args(sh, st, k, kl, v, vl, e1, e3, e2, mom, esbh, n_tok, op, ws,
                                    ws_bytes);
  if (r != LACT_OK) return r;
  if (n_tok == 0) return LACT_OK;
  return do_update(sh, st, k, kl, v, vl, e1, e3, e2, mom, esbh, n_tok, op, ws,
                   (hipStream_t)stream);
}

lact_status lact_chunk_step(const lact_shape* sh, const lact_state* st, const void* q,
                            lact_layout ql, const void* k, lact_layout kl, const void* v,
                            lact_layout vl, void* o, lact_layout ol, const float* e1,
                            const float* e3, const float* e2, const float* mom, int64_t esbh,
                            int64_t n_tok, const lact_update_opts* op, void* ws,
                            size_t ws_bytes, void* stream) {
  lact_status r = check_update_args(sh, st, k, kl, v, vl, e1, e3, e2, mom, esbh, n_tok, op, ws,
                                    ws_bytes);
  if (r != LACT_OK) return r;
  if ((r = check_act(sh, q, ql, n_tok)) != LACT_OK) return r;
  if ((r = check_act(sh, o, ol, n_tok)) != LACT_OK) return r;
  if (n_tok > 0 && q == o) return LACT_ERR_INVALID_ARG;
  hipStream_t s = (hipStream_t)stream;
  if (n_tok == 0) return LACT_OK;
  const ApplyJob job{q, ql, o, ol, n_tok};
  // with the read in the Newton-Schulz launch, the new operand copies go to
  // the workspace shadow and are copied back
  void* alt = second_shadow(sh, op, ws);
  const SideStream* side = forks_read(sh, op) ? side_stream(s) : nullptr;
  r = do_update(sh, st, k, kl, v, vl, e1, e3, e2, mom, esbh, n_tok, op, ws, s, &job, alt, side);
  if (r != LACT_OK || alt == nullptr) return r;
  const hipError_t e = launch_copy16(st->shadow, alt, (int64_t)lact_shadow_bytes(sh), s);
  return e == hipSuccess ? LACT_OK : hip_fail(e);
}

}  // extern "C"

namespace lact {

#define LACT_SEQ_PARAMS                                                                       \
  const lact_shape *sh, const lact_state *st, const void *q, lact_layout ql, const void *k, \
      lact_layout kl, const void *v, lact_layout vl, void *o, lact_layout ol, const float *e1, \
      const float *e3, const float *e2, const float *mom, int64_t esbh, int64_t T,             \
      int64_t chunk, int32_t order, int64_t sub_off, int64_t sub_len, int32_t update_last,     \
      const lact_update_opts *op
#define LACT_SEQ_ARGS                                                                          \
  sh, st, q, ql, k, kl, v, vl, o, ol, e1, e3, e2, mom, esbh, T, chunk, order, sub_off, sub_len, \
      update_last, op

// Every argument check of lact_sequence (ws, ws_bytes: the workspace offered).
static lact_status check_sequence(LACT_SEQ_PARAMS, const void* ws, size_t ws_bytes) {
  if (T < 0 || chunk < 1) return LACT_ERR_INVALID_ARG;
  if (order != LACT_APPLY_THEN_UPDATE && order != LACT_UPDATE_THEN_APPLY) return LACT_ERR_INVALID_ARG;
  if (sub_len >= 0 && (sub_off < 0 || sub_off >= chunk)) return LACT_ERR_INVALID_ARG;
  int64_t max_upd = chunk < T ? chunk : T;
  if (sub_len >= 0) {
    const int64_t room = chunk - sub_off;
    max_upd = sub_len < room ? sub_len : room;
    if (max_upd > T) max_upd = T;
  }
  lact_status r = check_update_args(sh, st, k, kl, v, vl, e1, e3, e2, mom, esbh, max_upd, op, ws,
                                    ws_bytes);
  if (r != LACT_OK) return r;
  if ((r = check_act(sh, q, ql, T)) != LACT_OK) return r;
  if ((r = check_act(sh, o, ol, T)) != LACT_OK) return r;
  if (T > 0 && q == o) return LACT_ERR_INVALID_ARG;
  if (T > 0 && (e1 == nullptr || e3 == nullptr || e2 == nullptr)) return LACT_ERR_INVALID_ARG;
  if (op->use_momentum && T > 0 && mom == nullptr) return LACT_ERR_INVALID_ARG;
  return LACT_OK;
}

// The sequence driver proper (arguments already checked).  allow_side: the
// read of a d = 256 Muon write may run on the library's second stream.
static lact_status run_sequence(LACT_SEQ_PARAMS, void* ws, hipStream_t s, bool allow_side) {
  lact_status r = LACT_OK;
  const SideStream* side = allow_side && forks_read(sh, op) ? side_stream(s) : nullptr;
  const int es = elem_size(sh->dtype);
  auto at = [&](const void* base, lact_layout l, int64_t t) {
    return reinterpret_cast<const char*>(base) + t * l.stride_tok * es;
  };
  ApplyJob pending{};
  bool have_pending = false;
  // Operand copies: a write whose read shares its Newton-Schulz launch puts
  // the new copies in the other of (state shadow, workspace shadow); cs reads
  // from the current one.  The state's own shadow holds them at the end.
  lact_state cs = *st;
  void* const alt = second_shadow(sh, op, ws);
  auto write = [&](const void* kp, const void* vp, int64_t a0, int64_t n, const ApplyJob* job) {
    void* out = cs.shadow;
    if (alt != nullptr && job != nullptr && job->n_tok > 0) out = cs.shadow == st->shadow ? alt : st->shadow;
    // learning rates: one per token, or (per channel) d or dh per token
    const int64_t c13 = op->eta_per_channel ? sh->d : 1, c2 = op->eta_per_channel ? sh->dh : 1;
    const lact_status rr = do_update(sh, &cs, kp, kl, vp, vl, e1 + a0 * c13, e3 + a0 * c13, e2 + a0 * c2,
                                     mom ? mom + a0 : nullptr, esbh, n, op, ws, s, job, out, side);
    if (rr == LACT_OK) cs.shadow = out;
    return rr;
  };
  for (int64_t s0 = 0; s0 < T; s0 += chunk) {
    const int64_t e0 = s0 + chunk < T ? s0 + chunk : T;
    const bool last = e0 == T;
    int64_t a0 = s0, a1 = e0;
    if (sub_len >= 0) {
      a0 = s0 + sub_off;
      a1 = a0 + sub_len < e0 ? a0 + sub_len : e0;
    }
    const bool do_write = ((order == LACT_UPDATE_THEN_APPLY) || !last || update_last) && a1 > a0;
    const ApplyJob job{at(q, ql, s0), ql, const_cast<char*>(at(o, ol, s0)), ol, e0 - s0};
    // the read of a chunk goes with the next write after the weights it uses
    // (this chunk's write when reading first, the next chunk's otherwise)
    if (order == LACT_APPLY_THEN_UPDATE) {
      if (do_write)
        r = write(at(k, kl, a0), at(v, vl, a0), a0, a1 - a0, &job);
      else
        r = do_apply(sh, &cs, job.q, job.ql, job.o, job.ol, job.n_tok, s);
      if (r != LACT_OK) return r;
    } else {
      if (do_write)
        r = write(at(k, kl, a0), at(v, vl, a0), a0, a1 - a0, have_pending ? &pending : nullptr);
      else if (have_pending)
        r = do_apply(sh, &cs, pending.q, pending.ql, pending.o, pending.ol, pending.n_tok, s);
      if (r != LACT_OK) return r;
      pending = job;
      have_pending = true;
    }
  }
  if (have_pending) {
    r = do_apply(sh, &cs, pending.q, pending.ql, pending.o, pending.ol, pending.n_tok, s);
    if (r != LACT_OK) return r;
  }
  if (cs.shadow != st->shadow) {
    const hipError_t e = launch_copy16(st->shadow, cs.shadow, (int64_t)lact_shadow_bytes(sh), s);
    if (e != hipSuccess) return hip_fail(e);
  }
  return LACT_OK;
}

// Scratch of lact_sequence_noalloc: one array per device the library runs
// on, held until the process ends.  Host code never uses the array's name
// as an address: each device's address comes from hipGetSymbolAddress,
// taken once per device with that device current.
static __device__ __align__(256) unsigned char scratch[LACT_NOALLOC_SCRATCH_BYTES];

static lact_status scratch_on_current_device(void** out) {
  static std::mutex mu;
  static void* addr[64] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e);
  if (dev < 0 || dev >= 64) return LACT_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e);
    if (p == nullptr) return LACT_ERR_HIP;
    addr[dev] = p;
  }
  *out = addr[dev];
  return LACT_OK;
}

}  // namespace lact

extern "C" {

lact_status lact_sequence(LACT_SEQ_PARAMS, void* ws, size_t ws_bytes, void* stream) {
  const lact_status r = check_sequence(LACT_SEQ_ARGS, ws, ws_bytes);
  if (r != LACT_OK) return r;
  return run_sequence(LACT_SEQ_ARGS, ws, (hipStream_t)stream, true);
}

lact_status lact_sequence_noalloc(LACT_SEQ_PARAMS, void* stream) {
  // checked against the scratch's size (the address only has to pass the
  // null and alignment checks here; the real one is looked up below)
  static const unsigned char* const kAnyAligned = reinterpret_cast<const unsigned char*>(256);
  lact_status r = check_sequence(LACT_SEQ_ARGS, kAnyAligned, (size_t)LACT_NOALLOC_SCRATCH_BYTES);
  if (r != LACT_OK) return r;
  void* ws = nullptr;
  if ((r = scratch_on_current_device(&ws)) != LACT_OK) return r;
  // one stream only: the second stream and its events are created on first
  // use, which this entry point's callers may not allow
  return run_sequence(LACT_SEQ_ARGS, ws, (hipStream_t)stream, false);
}

// ------------------------------------------------- linear variant --
size_t lact_linear_shadow_bytes(const lact_shape* sh) {
  if (check_shape(sh) != LACT_OK || sh->dh != sh->d) return 0;
  return (size_t)sh->bh * sh->d * sh->d * elem_size(sh->dtype);
}

size_t lact_linear_workspace_bytes(const lact_shape* sh, const lact_update_opts* opts) {
  if (check_shape(sh) != LACT_OK || sh->dh != sh->d) return 0;
  const int64_t g = align256((int64_t)sh->bh * sh->d * sh->d * 4);
  const bool muon = opts != nullptr && opts->use_muon;
  return (size_t)(g + (muon ? ns_ws_bytes(sh->bh, sh->d, sh->d) : 0));
}

static lact_status check_linear(const lact_shape* sh, const lact_linear_state* st, bool need_m) {
  lact_status r;
  if ((r = check_shape(sh)) != LACT_OK) return r;
  if (sh->dh != sh->d) return LACT_ERR_UNSUPPORTED;
  if (st == nullptr || st->w == nullptr || st->n == nullptr || st->shadow == nullptr) return LACT_ERR_INVALID_ARG;
  if (!aligned16(st->w) || !aligned16(st->n) || !aligned16(st->shadow)) return LACT_ERR_ALIGNMENT;
  if (need_m && st->m == nullptr) return LACT_ERR_INVALID_ARG;
  if (st->m != nullptr && !aligned16(st->m)) return LACT_ERR_ALIGNMENT;
  return LACT_OK;
}

static LinArgs lin_args(const lact_shape* sh, const lact_linear_state* st) {
  LinArgs a;
  memset(&a, 0, sizeof(a));
  a.w = st->w; a.n = st->n; a.m = st->m; a.shadow = st->shadow;
  a.bh = sh->bh; a.d = sh->d;
  return a;
}

lact_status lact_linear_init_state(const lact_shape* sh, const lact_linear_state* st, void* stream) {
  lact_status r;
  if ((r = check_linear(sh, st, false)) != LACT_OK) return r;
  const LinArgs a = lin_args(sh, st);
  const hipError_t e = launch_linear(sh->dtype, 3, a, nullptr, (hipStream_t)stream);
  return e == hipSuccess ? LACT_OK : hip_fail(e);
}

lact_status lact_linear_sequence(const lact_shape* sh, const lact_linear_state* st, const void* q,
                                 lact_layout ql, const void* k, lact_layout kl, const void* v,
                                 lact_layout vl, void* o, lact_layout ol, const float* eta,
                                 const float* mom, int64_t esbh, int64_t T, int64_t chunk,
                                 int32_t order, int64_t sub_off, int64_t sub_len, int32_t update_last,
                                 const lact_update_opts* op, void* ws, size_t ws_bytes, void* stream) {
  lact_status r;
  if ((r = check_opts(op)) != LACT_OK) return r;
  if (op->eta_per_channel) return LACT_ERR_UNSUPPORTED;
  if ((r = check_linear(sh, st, op->use_momentum != 0)) != LACT_OK) return r;
  if (T < 0 || chunk < 1 || esbh < 0) return LACT_ERR_INVALID_ARG;
  if (order != LACT_APPLY_THEN_UPDATE && order != LACT_UPDATE_THEN_APPLY) return LACT_ERR_INVALID_ARG;
  if (sub_len >= 0 && (sub_off < 0 || sub_off >= chunk)) return LACT_ERR_INVALID_ARG;
  if ((r = check_act(sh, q, ql, T)) != LACT_OK) return r;
  if ((r = check_act(sh, o, ol, T)) != LACT_OK) return r;
  if ((r = check_act(sh, k, kl, T)) != LACT_OK) return r;
  if ((r = check_act(sh, v, vl, T)) != LACT_OK) return r;
  if (T > 0 && (q == o || eta == nullptr)) return LACT_ERR_INVALID_ARG;
  if (op->use_momentum && T > 0 && mom == nullptr) return LACT_ERR_INVALID_ARG;
  if (ws == nullptr || ws_bytes < lact_linear_workspace_bytes(sh, op)) return LACT_ERR_WORKSPACE;
  if (!aligned16(ws)) return LACT_ERR_ALIGNMENT;
  hipStream_t s = (hipStream_t)stream;
  const int es = elem_size(sh->dtype);
  LinArgs a = lin_args(sh, st);
  a.renorm = op->renorm; a.eps = op->renorm_eps; a.nonfinite = op->nonfinite;
  a.eta_sbh = esbh; a.mom_sbh = esbh;
  if (!op->use_momentum) a.m = nullptr;
  char* wsb = reinterpret_cast<char*>(ws);
  a.g = reinterpret_cast<float*>(wsb);
  const int64_t gsz = align256((int64_t)sh->bh * sh->d * sh->d * 4);
  auto read = [&](int64_t s0, int64_t n) {
    LinArgs x = a;
    x.q = reinterpret_cast<const char*>(q) + s0 * ql.stride_tok * es; x.q_sbh = ql.stride_bh; x.q_st = ql.stride_tok;
    x.o = reinterpret_cast<char*>(o) + s0 * ol.stride_tok * es; x.o_sbh = ol.stride_bh; x.o_st = ol.stride_tok;
    x.n_tok = n;
    const hipError_t e = launch_linear(sh->dtype, 0, x, nullptr, s);
    return e == hipSuccess ? LACT_OK : hip_fail(e);
  };
  auto write = [&](int64_t a0, int64_t n) {
    LinArgs x = a;
    x.k = reinterpret_cast<const char*>(k) + a0 * kl.stride_tok * es; x.k_sbh = kl.stride_bh; x.k_st = kl.stride_tok;
    x.v = reinterpret_cast<const char*>(v) + a0 * vl.stride_tok * es; x.v_sbh = vl.stride_bh; x.v_st = vl.stride_tok;
    x.eta = eta + a0;
    x.mom = mom != nullptr ? mom + a0 : nullptr;
    x.n_tok = n;
    hipError_t e = launch_linear(sh->dtype, 1, x, nullptr, s);
    if (e != hipSuccess) return hip_fail(e);
    if (op->use_muon) {
      const int prec = ns_prec_of(sh, op);
      float* nb = reinterpret_cast<float*>(wsb + gsz);
      const int64_t xm = align256((int64_t)sh->bh * sh->d * sh->d * 4);
      const int64_t am = align256((int64_t)sh->bh * sh->d * sh->d * 4);
      char* b = reinterpret_cast<char*>(nb);
      const NsIn in{{a.g, a.g, a.g}, sh->bh};
      e = run_ns(prec, sh->bh, sh->d, sh->d, in, a.g, op->ns_eps, reinterpret_cast<float*>(b),
                 reinterpret_cast<float*>(b + xm), reinterpret_cast<float*>(b + 2 * xm),
                 reinterpret_cast<float*>(b + 3 * xm), reinterpret_cast<float*>(b + 3 * xm + am),
                 reinterpret_cast<float*>(b + 3 * xm + 2 * am), s);
      if (e != hipSuccess) return hip_fail(e);
    }
    e = launch_linear(sh->dtype, 2, x, a.g, s);
    return e == hipSuccess ? LACT_OK : hip_fail(e);
  };
  for (int64_t s0 = 0; s0 < T; s0 += chunk) {
    const int64_t e0 = s0 + chunk < T ? s0 + chunk : T;
    const bool last = e0 == T;
    int64_t a0 = s0, a1 = e0;
    if (sub_len >= 0) {
      a0 = s0 + sub_off;
      a1 = a0 + sub_len < e0 ? a0 + sub_len : e0;
    }
    const bool do_write = ((order == LACT_UPDATE_THEN_APPLY) || !last || update_last) && a1 > a0;
    if (order == LACT_APPLY_THEN_UPDATE && (r = read(s0, e0 - s0)) != LACT_OK) return r;
    if (do_write && (r = write(a0, a1 - a0)) != LACT_OK) return r;
    if (order == LACT_UPDATE_THEN_APPLY && (r = read(s0, e0 - s0)) != LACT_OK) return r;
  }
  return LACT_OK;
}

lact_status lact_prof_begin(int32_t kind, int32_t max_launches) {
  if (kind < LACT_PROF_APPLY || kind > LACT_PROF_STEP || max_launches < 1) return LACT_ERR_INVALID_ARG;
  if (g_prof.kind != 0) return LACT_ERR_INVALID_ARG;
  g_prof.ev.assign(2 * (size_t)max_launches, nullptr);
  for (auto& e : g_prof.ev) {
    // timing only: no system-scope fence (no cache writeback between the
    // bracketed launch and its neighbours)
    hipError_t r = hipEventCreateWithFlags(&e, hipEventDisableSystemFence);
    if (r != hipSuccess) {
      for (auto& x : g_prof.ev)
        if (x) hipEventDestroy(x);
      g_prof.ev.clear();
      return hip_fail(r);
    }
  }
  g_prof.kind = kind;
  g_prof.cap = max_launches;
  g_prof.n = 0;
  return LACT_OK;
}

lact_status lact_prof_end(int32_t* launches, float* total_ms, float* min_ms, float* max_ms) {
  if (g_prof.kind == 0) return LACT_ERR_INVALID_ARG;
  float tot = 0.f, mn = 0.f, mx = 0.f;
  lact_status st = LACT_OK;
  for (int i = 0; i < g_prof.n; ++i) {
    hipError_t r = hipEventSynchronize(g_prof.ev[2 * i + 1]);
    float ms = 0.f;
    if (r == hipSuccess) r = hipEventElapsedTime(&ms, g_prof.ev[2 * i], g_prof.ev[2 * i + 1]);
    if (r != hipSuccess) {
      st = hip_fail(r);
      break;
    }
    tot += ms;
    mn = (i == 0 || ms < mn) ? ms : mn;
    mx = (i == 0 || ms > mx) ? ms : mx;
  }
  if (launches) *launches = g_prof.n;
  if (total_ms) *total_ms = tot;
  if (min_ms) *min_ms = mn;
  if (max_ms) *max_ms = mx;
  for (auto& e : g_prof.ev) hipEventDestroy(e);
  g_prof.ev.clear();
  g_prof.kind = 0;
  g_prof.n = g_prof.cap = 0;
  return st;
}

const char* lact_status_string(lact_status st) {
  switch (st) {
    case LACT_OK: return "ok";
    case LACT_ERR_INVALID_ARG: return "invalid argument";
    case LACT_ERR_UNSUPPORTED: return "unsupported shape";
    case LACT_ERR_ALIGNMENT: return "pointer or stride not 16-byte aligned";
    case LACT_ERR_WORKSPACE: return "workspace missing or too small";
    case LACT_ERR_HIP: return "HIP error";
    case LACT_ERR_NONFINITE: return "a write produced non-finite weights";
  }
  return "unknown status";
}

int lact_last_hip_error(void) { return g_last_hip_error; }

lact_status lact_check_finite(const int32_t* flag, void* stream) {
  if (flag == nullptr) return LACT_ERR_INVALID_ARG;
  if (((uintptr_t)flag & 3u) != 0) return LACT_ERR_ALIGNMENT;
  int32_t h = 0;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = hipMemcpyAsync(&h, flag, sizeof(h), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e);
  return h != 0 ? LACT_ERR_NONFINITE : LACT_OK;
}

}  // extern "C"

// ------------------------------------------------ outer-loop backward --
// The vector-Jacobian product of lact_sequence (outputs o) with respect to
// q, k, v, the learning rates, the momentum coefficients and W0, given the
// cotangent dO: the forward is recomputed in fp32 chunk by chunk (the state
// before every chunk kept in the workspace), then the chunks are walked
// backwards through the chain rule of each step (read, chunk gradient,
// momentum, Newton-Schulz, step + renorm; see k_backward.hip).
namespace lact {

namespace {

// element (b, i, j) = p[b bs + i s0 + j s1] (bf: bf16 elements)
struct Mat {
  const void* p;
  int bf;
  int64_t bs, s0, s1;
};

struct Bw {
  // shape
  int bh, d, dh, cmax, nch;
  bool mom;
  int64_t msz;  // d dh
  // buffers (fp32)
  float *states, *n0, *dst, *dold, *dn0;
  float *xa, *xb, *xo, *dx;            // [bh][cmax][d]
  float *ag, *au, *ae, *o1, *o3, *o2, *r1, *r3, *r2;  // [bh][cmax][dh]
  float *G, *U, *dR;                   // [3][bh][d dh], natural orientation
  float *Xs;                           // [6][3 bh][d][dh]: Newton-Schulz iterates
  float *Am, *Bm, *dAm, *dBm, *Sm;     // [3 bh][d][d]
  float *dXw, *dXn;                    // [3 bh][d][dh]
  float *beta, *ss, *dot, *c1, *c2, *dbeta;  // scalars
  float* part;                         // split-K partial sums
  int64_t part_floats;
  int64_t bytes;
  int nstate() const { return mom ? 6 : 3; }
  float* state(int c) const { return states + (int64_t)c * nstate() * bh * msz; }
  // matrix j (0 W1, 1 W3, 2 W2; 3.. the momentum) of a state block
  static float* mat(float* base, int j, int bh, int64_t msz) { return base + (int64_t)j * bh * msz; }
};

Bw bw_layout(const lact_shape* sh, int64_t T, int64_t chunk, bool mom, char* base) {
  Bw w;
  memset(&w, 0, sizeof(w));
  w.bh = sh->bh; w.d = sh->d; w.dh = sh->dh;
  w.cmax = (int)(chunk < T ? chunk : T);
  if (w.cmax < 1) w.cmax = 1;
  w.nch = (int)((T + chunk - 1) / chunk);
  w.mom = mom;
  w.msz = (int64_t)sh->d * sh->dh;
  int64_t off = 0;
  auto take = [&](int64_t floats) {
    float* p = base ? reinterpret_cast<float*>(base + off) : nullptr;
    off += align256(floats * 4);
    return p;
  };
  const int64_t bh = w.bh, m3 = 3 * bh * w.msz;
  w.states = take((int64_t)(w.nch + 1) * w.nstate() * bh * w.msz);
  w.n0 = take(bh * (2 * w.dh + w.d));
  w.dst = take(2 * m3);
  w.dold = take(2 * m3);
  w.dn0 = take(bh * (2 * w.dh + w.d));
  const int64_t act_d = bh * w.cmax * w.d, act_h = bh * w.cmax * w.dh;
  w.xa = take(act_d); w.xb = take(act_d); w.xo = take(act_d); w.dx = take(act_d);
  w.ag = take(act_h); w.au = take(act_h); w.ae = take(act_h);
  w.o1 = take(act_h); w.o3 = take(act_h); w.o2 = take(act_h);
  w.r1 = take(act_h); w.r3 = take(act_h); w.r2 = take(act_h);
  w.G = take(m3); w.U = take(m3); w.dR = take(m3);
  w.Xs = take(6 * m3);
  const int64_t sq = 3 * bh * (int64_t)w.d * w.d;
  w.Am = take(sq); w.Bm = take(sq); w.dAm = take(sq); w.dBm = take(sq); w.Sm = take(sq);
  w.dXw = take(m3); w.dXn = take(m3);
  w.beta = take(bh); w.ss = take(3 * bh); w.dot = take(3 * bh);
  w.c1 = take(3 * bh); w.c2 = take(3 * bh); w.dbeta = take(3 * bh);
  w.part_floats = 16 * bh * w.msz;
  w.part = take(w.part_floats);
  w.bytes = off;
  return w;
}

// The GEMMs of the backward; the workspace's partial buffer lets the long
// token contractions split K.
hipError_t mm(const Bw& w, Mat A, Mat B, const float* D, int64_t dbs, int64_t dsm, float* C, int64_t cbs,
              int64_t csm, int M, int N, int K, int batch, float alpha, float beta, hipStream_t s) {
  BGemm g;
  g.A = A.p; g.a_bf16 = A.bf; g.a_bs = A.bs; g.a_sm = A.s0; g.a_sk = A.s1;
  g.B = B.p; g.b_bf16 = B.bf; g.b_bs = B.bs; g.b_sk = B.s0; g.b_sn = B.s1;
  g.D = D; g.d_bs = dbs; g.d_sm = dsm;
  g.C = C; g.c_bs = cbs; g.c_sm = csm;
  g.M = M; g.N = N; g.K = K; g.batch = batch;
  g.alpha = alpha; g.beta = beta;
  return launch_bgemm(g, s, w.part, w.part_floats);
}

// Rows of the three matrices: (pointer offset of block j, rows, row length).
inline int64_t rows_of(const Bw& w, int j) { return (int64_t)w.bh * (j < 2 ? w.dh : w.d); }
inline int len_of(const Bw& w, int j) { return j < 2 ? w.d : w.dh; }
inline float* n0_of(const Bw& w, float* base, int j) {
  return base + (j == 0 ? 0 : (j == 1 ? (int64_t)w.bh * w.dh : 2 * (int64_t)w.bh * w.dh));
}

#define BW_TRY(x)                                   \
  do {                                              \
    const hipError_t e_ = (x);                      \
    if (e_ != hipSuccess) return e_;                \
  } while (0)

// g = X W1^T, u = X W3^T into ag, au and (E: V W2, else skip) e into ae, for
// n rows of X ([bh][n][d], fp32) with the state W.
hipError_t bw_products(const Bw& w, const float* W, const float* X, const float* V, int n, hipStream_t s) {
  const int64_t msz = w.msz;
  const Mat x{X, 0, (int64_t)n * w.d, w.d, 1};
  const float* W1 = W;
  const float* W3 = W + w.bh * msz;
  const float* W2 = W + 2 * w.bh * msz;
  BW_TRY(mm(w, x, Mat{W1, 0, msz, 1, w.d}, nullptr, 0, 0, w.ag, (int64_t)n * w.dh, w.dh, n, w.dh, w.d, w.bh, 1.f, 0.f, s));
  BW_TRY(mm(w, x, Mat{W3, 0, msz, 1, w.d}, nullptr, 0, 0, w.au, (int64_t)n * w.dh, w.dh, n, w.dh, w.d, w.bh, 1.f, 0.f, s));
  if (V != nullptr)
    BW_TRY(mm(w, Mat{V, 0, (int64_t)n * w.d, w.d, 1}, Mat{W2, 0, msz, w.dh, 1}, nullptr, 0, 0, w.ae,
              (int64_t)n * w.dh, w.dh, n, w.dh, w.d, w.bh, 1.f, 0.f, s));
  return hipSuccess;
}

// The write's raw gradient G (natural orientation, into w.G) from the state
// W and the gathered keys / values (xa, xb: n rows); leaves g, u, e in ag,
// au, ae and the scaled factors in o1, o3, o2.
hipError_t bw_gradient(const Bw& w, const float* W, int n, const float* e1, const float* e3, const float* e2,
                       int64_t esbh, int64_t t0, hipStream_t s) {
  BW_TRY(bw_products(w, W, w.xa, w.xb, n, s));
  BW_TRY(bw_grad_fwd(w.ag, w.au, w.ae, w.o1, w.o3, w.o2, e1, e3, e2, esbh, t0, n, w.dh, w.bh, s));
  const int64_t msz = w.msz, nh = (int64_t)n * w.dh, nd = (int64_t)n * w.d;
  // G1 = o1^T K, G3 = o3^T K  [dh][d];  G2 = V^T o2  [d][dh]
  BW_TRY(mm(w, Mat{w.o1, 0, nh, 1, w.dh}, Mat{w.xa, 0, nd, w.d, 1}, nullptr, 0, 0, w.G, msz, w.d, w.dh, w.d, n,
            w.bh, 1.f, 0.f, s));
  BW_TRY(mm(w, Mat{w.o3, 0, nh, 1, w.dh}, Mat{w.xa, 0, nd, w.d, 1}, nullptr, 0, 0, w.G + w.bh * msz, msz, w.d,
            w.dh, w.d, n, w.bh, 1.f, 0.f, s));
  BW_TRY(mm(w, Mat{w.xb, 0, nd, 1, w.d}, Mat{w.o2, 0, nh, w.dh, 1}, nullptr, 0, 0, w.G + 2 * w.bh * msz, msz,
            w.dh, w.d, w.dh, n, w.bh, 1.f, 0.f, s));
  return hipSuccess;
}

// Natural (G1, G3 [dh][d], G2 [d][dh]) <-> wide ([d][dh]) orientation.
hipError_t bw_to_wide(const Bw& w, const float* nat, float* wide, hipStream_t s) {
  BW_TRY(bw_transpose(nat, wide, w.dh, w.d, 2 * w.bh, s));
  return bw_axpby(wide + 2 * w.bh * w.msz, nat + 2 * w.bh * w.msz, nullptr, nullptr, 1.f, nullptr, 0.f, w.msz,
                  w.bh, s);
}
hipError_t bw_from_wide(const Bw& w, const float* wide, float* nat, hipStream_t s) {
  BW_TRY(bw_transpose(wide, nat, w.d, w.dh, 2 * w.bh, s));
  return bw_axpby(nat + 2 * w.bh * w.msz, wide + 2 * w.bh * w.msz, nullptr, nullptr, 1.f, nullptr, 0.f, w.msz,
                  w.bh, s);
}

// A = X X^T, B = b A + c A A for the 3 bh wide matrices X.
hipError_t bw_ns_ab(const Bw& w, const float* X, float b, float c, hipStream_t s) {
  const int cnt = 3 * w.bh, d = w.d, dh = w.dh;
  const int64_t dd = (int64_t)d * d;
  BW_TRY(mm(w, Mat{X, 0, w.msz, dh, 1}, Mat{X, 0, w.msz, 1, dh}, nullptr, 0, 0, w.Am, dd, d, d, d, dh, cnt, 1.f, 0.f, s));
  return mm(w, Mat{w.Am, 0, dd, d, 1}, Mat{w.Am, 0, dd, d, 1}, w.Am, dd, d, w.Bm, dd, d, d, d, d, cnt, c, b, s);
}

// Newton-Schulz of the wide matrices in Xs[0] (normalised here), iterates
// X_1 .. X_5 into Xs[1 .. 5] (the rebuttal page's quintic coefficients).
hipError_t bw_ns_forward(const Bw& w, float eps, hipStream_t s) {
  const int cnt = 3 * w.bh, d = w.d, dh = w.dh;
  const int64_t m3 = (int64_t)cnt * w.msz, dd = (int64_t)d * d;
  BW_TRY(bw_dot(w.Xs, nullptr, w.ss, w.msz, cnt, s));
  BW_TRY(bw_nscoef(w.ss, nullptr, w.c1, nullptr, cnt, eps, s));
  // keep G (wide) in dXn for the normalisation's VJP
  BW_TRY(bw_axpby(w.dXn, w.Xs, nullptr, nullptr, 1.f, nullptr, 0.f, m3, 1, s));
  BW_TRY(bw_axpby(w.Xs, w.dXn, nullptr, w.c1, 0.f, nullptr, 0.f, w.msz, cnt, s));
  for (int it = 0; it < 5; ++it) {
    const float a = kNS[it][0], b = kNS[it][1], c = kNS[it][2];
    const float* X = w.Xs + it * m3;
    BW_TRY(bw_ns_ab(w, X, b, c, s));
    // X' = B X + a X
    BW_TRY(mm(w, Mat{w.Bm, 0, dd, d, 1}, Mat{X, 0, w.msz, dh, 1}, X, w.msz, dh, w.Xs + (it + 1) * m3, w.msz, dh,
              d, dh, d, cnt, 1.f, a, s));
  }
  return hipSuccess;
}

// VJP of Newton-Schulz: dXw holds dU (wide) on entry, dG (wide) on exit;
// dXn holds G (wide) from bw_ns_forward.
hipError_t bw_ns_vjp(const Bw& w, float eps, hipStream_t s) {
  const int cnt = 3 * w.bh, d = w.d, dh = w.dh;
  const int64_t m3 = (int64_t)cnt * w.msz, dd = (int64_t)d * d;
  float* dX = w.dXw;
  float* G = w.dXn;
  // a separate buffer for the new dX: the U buffer is free here (wide size)
  float* dY = w.dR;
  for (int it = 4; it >= 0; --it) {
    const float a = kNS[it][0], b = kNS[it][1], c = kNS[it][2];
    const float* X = w.Xs + it * m3;
    BW_TRY(bw_ns_ab(w, X, b, c, s));
    // dB = dX X^T
    BW_TRY(mm(w, Mat{dX, 0, w.msz, dh, 1}, Mat{X, 0, w.msz, 1, dh}, nullptr, 0, 0, w.dBm, dd, d, d, d, dh, cnt, 1.f,
              0.f, s));
    // dY = B dX + a dX   (B symmetric)
    BW_TRY(mm(w, Mat{w.Bm, 0, dd, d, 1}, Mat{dX, 0, w.msz, dh, 1}, dX, w.msz, dh, dY, w.msz, dh, d, dh, d, cnt, 1.f,
              a, s));
    // dA = b dB + c (dB A + A dB)   (A symmetric)
    BW_TRY(mm(w, Mat{w.dBm, 0, dd, d, 1}, Mat{w.Am, 0, dd, d, 1}, w.dBm, dd, d, w.dAm, dd, d, d, d, d, cnt, c, b, s));
    BW_TRY(mm(w, Mat{w.Am, 0, dd, d, 1}, Mat{w.dBm, 0, dd, d, 1}, w.dAm, dd, d, w.dAm, dd, d, d, d, d, cnt, c, 1.f, s));
    // dY += (dA + dA^T) X
    BW_TRY(bw_symm(w.dAm, w.Sm, d, cnt, s));
    BW_TRY(mm(w, Mat{w.Sm, 0, dd, d, 1}, Mat{X, 0, w.msz, dh, 1}, dY, w.msz, dh, dY, w.msz, dh, d, dh, d, cnt, 1.f,
              1.f, s));
    BW_TRY(bw_axpby(dX, dY, nullptr, nullptr, 1.f, nullptr, 0.f, m3, 1, s));
  }
  // X0 = G / (||G|| + eps):  dG = c1 dX + c2 G
  BW_TRY(bw_dot(dX, G, w.dot, w.msz, cnt, s));
  BW_TRY(bw_nscoef(w.ss, w.dot, w.c1, w.c2, cnt, eps, s));
  return bw_axpby(dX, dX, G, w.c1, 0.f, w.c2, 0.f, w.msz, cnt, s);
}

}  // namespace
}  // namespace lact

extern "C" {

size_t lact_backward_workspace_bytes(const lact_shape* sh, int64_t T, int64_t chunk,
                                     const lact_update_opts* opts) {
  if (check_shape(sh, true) != LACT_OK || T < 0 || chunk < 1 || opts == nullptr) return 0;
  return (size_t)bw_layout(sh, T, chunk, opts->use_momentum != 0, nullptr).bytes;
}

lact_status lact_sequence_backward(const lact_shape* sh, const float* w1, const float* w3, const float* w2,
                                   const void* q, lact_layout ql, const void* k, lact_layout kl,
                                   const void* v, lact_layout vl, const float* dout, const float* e1,
                                   const float* e3, const float* e2, const float* mom, int64_t esbh,
                                   int64_t T, int64_t chunk, int32_t order, int64_t sub_off,
                                   int64_t sub_len, int32_t update_last, const lact_update_opts* op,
                                   const lact_grads* gr, void* ws, size_t ws_bytes, void* stream) {
  lact_status r;
  if ((r = check_shape(sh, true)) != LACT_OK) return r;
  if ((r = check_opts(op)) != LACT_OK) return r;
  if (op->renorm == 2 || op->eta_per_channel) return LACT_ERR_UNSUPPORTED;
  if (T < 0 || chunk < 1) return LACT_ERR_INVALID_ARG;
  if (order != LACT_APPLY_THEN_UPDATE && order != LACT_UPDATE_THEN_APPLY) return LACT_ERR_INVALID_ARG;
  if (sub_len >= 0 && (sub_off < 0 || sub_off >= chunk)) return LACT_ERR_INVALID_ARG;
  if (gr == nullptr || esbh < T) return LACT_ERR_INVALID_ARG;
  if ((r = check_act(sh, q, ql, T)) != LACT_OK) return r;
  if ((r = check_act(sh, k, kl, T)) != LACT_OK) return r;
  if ((r = check_act(sh, v, vl, T)) != LACT_OK) return r;
  const bool mo = op->use_momentum != 0;
  for (const void* p : {(const void*)w1, (const void*)w3, (const void*)w2, (const void*)gr->dw1,
                        (const void*)gr->dw3, (const void*)gr->dw2}) {
    if (p == nullptr) return LACT_ERR_INVALID_ARG;
    if (!aligned16(p)) return LACT_ERR_ALIGNMENT;
  }
  if (T > 0) {
    for (const void* p : {(const void*)dout, (const void*)e1, (const void*)e3, (const void*)e2,
                          (const void*)gr->dq, (const void*)gr->dk, (const void*)gr->dv,
                          (const void*)gr->deta1, (const void*)gr->deta3, (const void*)gr->deta2}) {
      if (p == nullptr) return LACT_ERR_INVALID_ARG;
      if (!aligned16(p)) return LACT_ERR_ALIGNMENT;
    }
    if (mo && (mom == nullptr || gr->dmom == nullptr)) return LACT_ERR_INVALID_ARG;
    if (mo && (!aligned16(mom) || !aligned16(gr->dmom))) return LACT_ERR_ALIGNMENT;
  }
  Bw w = bw_layout(sh, T, chunk, mo, reinterpret_cast<char*>(ws));
  if (ws == nullptr || ws_bytes < (size_t)w.bytes) return LACT_ERR_WORKSPACE;
  if (!aligned16(ws)) return LACT_ERR_ALIGNMENT;
  hipStream_t s = (hipStream_t)stream;
  const int bh = sh->bh, d = sh->d, dh = sh->dh, bf = sh->dtype == LACT_BF16 ? 1 : 0;
  const int64_t msz = w.msz, m3 = 3 * (int64_t)bh * msz;
  const int64_t nd_all = (int64_t)bh * T * d;
  hipError_t e = hipSuccess;
#define BW_CALL(x)                         \
  do {                                     \
    e = (x);                               \
    if (e != hipSuccess) return hip_fail(e); \
  } while (0)
  // outputs start at zero
  BW_CALL(bw_fill(gr->dq, 0.f, nd_all, s));
  BW_CALL(bw_fill(gr->dk, 0.f, nd_all, s));
  BW_CALL(bw_fill(gr->dv, 0.f, nd_all, s));
  BW_CALL(bw_fill(gr->deta1, 0.f, (int64_t)bh * esbh, s));
  if (gr->deta3 != gr->deta1) BW_CALL(bw_fill(gr->deta3, 0.f, (int64_t)bh * esbh, s));
  if (gr->deta2 != gr->deta1 && gr->deta2 != gr->deta3) BW_CALL(bw_fill(gr->deta2, 0.f, (int64_t)bh * esbh, s));
  if (mo) BW_CALL(bw_fill(gr->dmom, 0.f, (int64_t)bh * esbh, s));
  // state 0: W0 (fp32, natural orientation), momentum zero; n0 = row norms
  float* S0 = w.state(0);
  BW_CALL(bw_axpby(S0, w1, nullptr, nullptr, 1.f, nullptr, 0.f, msz, bh, s));
  BW_CALL(bw_axpby(S0 + bh * msz, w3, nullptr, nullptr, 1.f, nullptr, 0.f, msz, bh, s));
  BW_CALL(bw_axpby(S0 + 2 * bh * msz, w2, nullptr, nullptr, 1.f, nullptr, 0.f, msz, bh, s));
  if (mo) BW_CALL(bw_fill(S0 + m3, 0.f, m3, s));
  for (int j = 0; j < 3; ++j)
    BW_CALL(bw_rownorm(S0 + j * bh * msz, n0_of(w, w.n0, j), rows_of(w, j), len_of(w, j), s));
  BW_CALL(bw_fill(w.dst, 0.f, 2 * m3, s));
  BW_CALL(bw_fill(w.dn0, 0.f, (int64_t)bh * (2 * dh + d), s));
  // chunk plan (the drivers' rule)
  struct Ch { int64_t s0, e0, a0, a1; bool write; };
  std::vector<Ch> plan;
  for (int64_t s0 = 0; s0 < T; s0 += chunk) {
    const int64_t e0 = s0 + chunk < T ? s0 + chunk : T;
    const bool last = e0 == T;
    int64_t a0 = s0, a1 = e0;
    if (sub_len >= 0) {
      a0 = s0 + sub_off;
      a1 = a0 + sub_len < e0 ? a0 + sub_len : e0;
    }
    const bool wr = ((order == LACT_UPDATE_THEN_APPLY) || !last || update_last) && a1 > a0;
    plan.push_back(Ch{s0, e0, a0, a1, wr});
  }
  // one write from state `in` to state `out` (fp32 recompute); leaves G~ in
  // w.G (natural) and, with Muon, the iterates in w.Xs
  auto write_forward = [&](const Ch& c, const float* in, float* out, bool keep_ns) -> hipError_t {
    const int n = (int)(c.a1 - c.a0);
    BW_TRY(bw_gather(k, bf, kl.stride_bh, kl.stride_tok, c.a0, n, d, bh, w.xa, s));
    BW_TRY(bw_gather(v, bf, vl.stride_bh, vl.stride_tok, c.a0, n, d, bh, w.xb, s));
    BW_TRY(bw_gradient(w, in, n, e1, e3, e2, esbh, c.a0, s));
    if (mo) {
      BW_TRY(bw_beta(mom, esbh, c.a0, n, w.beta, bh, s));
      for (int j = 0; j < 3; ++j)
        BW_TRY(bw_axpby(w.G + j * bh * msz, w.G + j * bh * msz, in + (3 + j) * bh * msz, nullptr, 1.f, w.beta,
                        0.f, msz, bh, s));
      BW_TRY(bw_axpby(out + m3, w.G, nullptr, nullptr, 1.f, nullptr, 0.f, m3, 1, s));  // M <- G~
    }
    if (op->use_muon) {
      BW_TRY(bw_to_wide(w, w.G, w.Xs, s));
      BW_TRY(bw_ns_forward(w, op->ns_eps, s));
      BW_TRY(bw_from_wide(w, w.Xs + 5 * m3, w.U, s));
    } else {
      BW_TRY(bw_axpby(w.U, w.G, nullptr, nullptr, 1.f, nullptr, 0.f, m3, 1, s));
    }
    (void)keep_ns;
    BW_TRY(bw_axpby(out, in, nullptr, nullptr, 1.f, nullptr, 0.f, m3, 1, s));
    for (int j = 0; j < 3; ++j)
      BW_TRY(bw_step(out + j * bh * msz, w.U + j * bh * msz, n0_of(w, w.n0, j), rows_of(w, j), len_of(w, j),
                     op->renorm, op->renorm_eps, s));
    return hipSuccess;
  };
  // forward: the state before every chunk (state nch = the final state)
  for (size_t ci = 0; ci < plan.size(); ++ci) {
    float* in = w.state((int)ci);
    float* out = w.state((int)ci + 1);
    if (plan[ci].write) {
      BW_CALL(write_forward(plan[ci], in, out, false));
    } else {
      BW_CALL(bw_axpby(out, in, nullptr, nullptr, 1.f, nullptr, 0.f, (int64_t)w.nstate() * bh * msz, 1, s));
    }
  }
  // read VJP of chunk c with state W: dq += dX, dstate W += dW
  auto read_vjp = [&](const Ch& c, const float* W) -> hipError_t {
    const int n = (int)(c.e0 - c.s0);
    const int64_t nd = (int64_t)n * d, nh = (int64_t)n * dh;
    BW_TRY(bw_gather(q, bf, ql.stride_bh, ql.stride_tok, c.s0, n, d, bh, w.xo, s));
    BW_TRY(bw_gather(dout, 0, (int64_t)T * d, d, c.s0, n, d, bh, w.dx, s));
    // g, u into ag, au; dh = dO W2 into ae
    BW_TRY(bw_products(w, W, w.xo, nullptr, n, s));
    BW_TRY(mm(w, Mat{w.dx, 0, nd, d, 1}, Mat{W + 2 * bh * msz, 0, msz, dh, 1}, nullptr, 0, 0, w.ae, nh, dh, n, dh, d,
              bh, 1.f, 0.f, s));
    BW_TRY(bw_read(w.ag, w.au, w.ae, (int64_t)bh * nh, s));  // ag = dg, au = du, ae = h
    float* dW1 = w.dst;
    float* dW3 = w.dst + bh * msz;
    float* dW2 = w.dst + 2 * bh * msz;
    // dW2 += dO^T h, dW1 += dg^T x, dW3 += du^T x
    BW_TRY(mm(w, Mat{w.dx, 0, nd, 1, d}, Mat{w.ae, 0, nh, dh, 1}, dW2, msz, dh, dW2, msz, dh, d, dh, n, bh, 1.f, 1.f, s));
    BW_TRY(mm(w, Mat{w.ag, 0, nh, 1, dh}, Mat{w.xo, 0, nd, d, 1}, dW1, msz, d, dW1, msz, d, dh, d, n, bh, 1.f, 1.f, s));
    BW_TRY(mm(w, Mat{w.au, 0, nh, 1, dh}, Mat{w.xo, 0, nd, d, 1}, dW3, msz, d, dW3, msz, d, dh, d, n, bh, 1.f, 1.f, s));
    // dx = dg W1 + du W3
    BW_TRY(mm(w, Mat{w.ag, 0, nh, dh, 1}, Mat{W, 0, msz, d, 1}, nullptr, 0, 0, w.xa, nd, d, n, d, dh, bh, 1.f, 0.f, s));
    BW_TRY(mm(w, Mat{w.au, 0, nh, dh, 1}, Mat{W + bh * msz, 0, msz, d, 1}, w.xa, nd, d, w.xa, nd, d, n, d, dh, bh, 1.f,
              1.f, s));
    return bw_scatter_add(w.xa, (int64_t)T * d, d, c.s0, n, d, bh, gr->dq, s);
  };
  // write VJP of chunk c from state `in` (the state before the write): the
  // cotangent of the new state is in w.dst, that of `in` replaces it
  auto write_vjp = [&](const Ch& c, const float* in) -> hipError_t {
    const int n = (int)(c.a1 - c.a0);
    const int64_t nd = (int64_t)n * d, nh = (int64_t)n * dh;
    // recompute G~ (w.G), the iterates, U
    float* scratch_out = w.dold;  // (overwritten below; only the G~ / U side products matter)
    BW_TRY(write_forward(c, in, scratch_out, true));
    // step + renorm VJP: dR (cotangent of W_in and of U)
    for (int j = 0; j < 3; ++j)
      BW_TRY(bw_step_vjp(in + j * bh * msz, w.U + j * bh * msz, n0_of(w, w.n0, j), w.dst + j * bh * msz,
                         w.dR + j * bh * msz, n0_of(w, w.dn0, j), rows_of(w, j), len_of(w, j), op->renorm,
                         op->renorm_eps, s));
    // dold W = dR
    BW_TRY(bw_axpby(w.dold, w.dR, nullptr, nullptr, 1.f, nullptr, 0.f, m3, 1, s));
    // dG~ (natural) into w.U
    if (op->use_muon) {
      BW_TRY(bw_to_wide(w, w.dR, w.dXw, s));
      // dXn must hold G~ (wide) for the normalisation VJP: bw_ns_forward
      // left it there
      BW_TRY(bw_ns_vjp(w, op->ns_eps, s));
      BW_TRY(bw_from_wide(w, w.dXw, w.U, s));
    } else {
      BW_TRY(bw_axpby(w.U, w.dR, nullptr, nullptr, 1.f, nullptr, 0.f, m3, 1, s));
    }
    if (mo) {
      // M_new = G~: its cotangent joins dG~; dbeta = sum dG~ . M_old; dM_old = beta dG~
      BW_TRY(bw_axpby(w.U, w.U, w.dst + m3, nullptr, 1.f, nullptr, 1.f, m3, 1, s));
      BW_TRY(bw_dot(w.U, in + m3, w.dbeta, msz, 3 * bh, s));
      for (int j = 0; j < 3; ++j)
        BW_TRY(bw_axpby(w.dold + m3 + j * bh * msz, w.U + j * bh * msz, nullptr, w.beta, 0.f, nullptr, 0.f, msz,
                        bh, s));
      BW_TRY(bw_dmom(w.dbeta, gr->dmom, esbh, c.a0, n, bh, s));
    }
    // chunk gradient VJP with dG = w.U (natural): p1 = k dG1^T, p3 = k dG3^T, p2 = v dG2
    const float* dG1 = w.U;
    const float* dG3 = w.U + bh * msz;
    const float* dG2 = w.U + 2 * bh * msz;
    BW_TRY(bw_products(w, in, w.xa, w.xb, n, s));  // g, u, e (unscaled)
    BW_TRY(mm(w, Mat{w.xa, 0, nd, d, 1}, Mat{dG1, 0, msz, 1, d}, nullptr, 0, 0, w.o1, nh, dh, n, dh, d, bh, 1.f, 0.f, s));
    BW_TRY(mm(w, Mat{w.xa, 0, nd, d, 1}, Mat{dG3, 0, msz, 1, d}, nullptr, 0, 0, w.o3, nh, dh, n, dh, d, bh, 1.f, 0.f, s));
    BW_TRY(mm(w, Mat{w.xb, 0, nd, d, 1}, Mat{dG2, 0, msz, dh, 1}, nullptr, 0, 0, w.o2, nh, dh, n, dh, d, bh, 1.f, 0.f, s));
    BW_TRY(bw_grad_bwd(w.ag, w.au, w.ae, w.o1, w.o3, w.o2, w.r1, w.r3, w.r2, e1, e3, e2, esbh, c.a0, n, dh, bh, s));
    BW_TRY(bw_rowsum(w.r1, gr->deta1, esbh, c.a0, n, dh, bh, s));
    BW_TRY(bw_rowsum(w.r3, gr->deta3, esbh, c.a0, n, dh, bh, s));
    BW_TRY(bw_rowsum(w.r2, gr->deta2, esbh, c.a0, n, dh, bh, s));
    // dV = (eta2 h) dG2^T + dE W2^T
    const float* Win2 = in + 2 * bh * msz;
    BW_TRY(mm(w, Mat{w.o2, 0, nh, dh, 1}, Mat{dG2, 0, msz, 1, dh}, nullptr, 0, 0, w.xo, nd, d, n, d, dh, bh, 1.f, 0.f, s));
    BW_TRY(mm(w, Mat{w.ae, 0, nh, dh, 1}, Mat{Win2, 0, msz, 1, dh}, w.xo, nd, d, w.xo, nd, d, n, d, dh, bh, 1.f, 1.f, s));
    BW_TRY(bw_scatter_add(w.xo, (int64_t)T * d, d, c.a0, n, d, bh, gr->dv, s));
    // dK = (eta3 a) dG3 + (eta1 b) dG1 + dg W1 + du W3
    BW_TRY(mm(w, Mat{w.o3, 0, nh, dh, 1}, Mat{dG3, 0, msz, d, 1}, nullptr, 0, 0, w.dx, nd, d, n, d, dh, bh, 1.f, 0.f, s));
    BW_TRY(mm(w, Mat{w.o1, 0, nh, dh, 1}, Mat{dG1, 0, msz, d, 1}, w.dx, nd, d, w.dx, nd, d, n, d, dh, bh, 1.f, 1.f, s));
    BW_TRY(mm(w, Mat{w.ag, 0, nh, dh, 1}, Mat{in, 0, msz, d, 1}, w.dx, nd, d, w.dx, nd, d, n, d, dh, bh, 1.f, 1.f, s));
    BW_TRY(mm(w, Mat{w.au, 0, nh, dh, 1}, Mat{in + bh * msz, 0, msz, d, 1}, w.dx, nd, d, w.dx, nd, d, n, d, dh, bh, 1.f,
              1.f, s));
    BW_TRY(bw_scatter_add(w.dx, (int64_t)T * d, d, c.a0, n, d, bh, gr->dk, s));
    // dW1 += dg^T k, dW3 += du^T k, dW2 += v^T dE (into dold)
    float* dW1 = w.dold;
    float* dW3 = w.dold + bh * msz;
    float* dW2 = w.dold + 2 * bh * msz;
    BW_TRY(mm(w, Mat{w.ag, 0, nh, 1, dh}, Mat{w.xa, 0, nd, d, 1}, dW1, msz, d, dW1, msz, d, dh, d, n, bh, 1.f, 1.f, s));
    BW_TRY(mm(w, Mat{w.au, 0, nh, 1, dh}, Mat{w.xa, 0, nd, d, 1}, dW3, msz, d, dW3, msz, d, dh, d, n, bh, 1.f, 1.f, s));
    BW_TRY(mm(w, Mat{w.xb, 0, nd, 1, d}, Mat{w.ae, 0, nh, dh, 1}, dW2, msz, dh, dW2, msz, dh, d, dh, n, bh, 1.f, 1.f, s));
    // the cotangent of the state before the write
    if (!mo) BW_TRY(bw_fill(w.dold + m3, 0.f, m3, s));
    return bw_axpby(w.dst, w.dold, nullptr, nullptr, 1.f, nullptr, 0.f, 2 * m3, 1, s);
  };
  for (int ci = (int)plan.size() - 1; ci >= 0; --ci) {
    const Ch& c = plan[ci];
    const float* before = w.state(ci);
    const float* after = w.state(ci + 1);
    if (order == LACT_UPDATE_THEN_APPLY) BW_CALL(read_vjp(c, after));
    if (c.write) BW_CALL(write_vjp(c, before));
    if (order == LACT_APPLY_THEN_UPDATE) BW_CALL(read_vjp(c, before));
  }
  // W0: its own cotangent plus the renorm targets (n0 = row norms of W0)
  const float* w0s[3] = {w1, w3, w2};
  float* outs[3] = {gr->dw1, gr->dw3, gr->dw2};
  for (int j = 0; j < 3; ++j) {
    if (op->renorm)
      BW_CALL(bw_w0(w0s[j], w.dst + j * bh * msz, n0_of(w, w.dn0, j), outs[j], rows_of(w, j), len_of(w, j), s));
    else
      BW_CALL(bw_axpby(outs[j], w.dst + j * bh * msz, nullptr, nullptr, 1.f, nullptr, 0.f, msz, bh, s));
  }
#undef BW_CALL
  return LACT_OK;
}

}  // extern "C"
