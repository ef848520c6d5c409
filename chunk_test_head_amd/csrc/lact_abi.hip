// C ABI of the LaCT fast-weight layer: host-side validation, workspace
// layout and the chunk sequence driver.  Every entry point checks all of its
// arguments before it enqueues anything, allocates nothing and never
// synchronises.
#include <hip/hip_runtime.h>

#include <stdint.h>
#include <string.h>

#include <vector>

#include "../../include/lact.h"
#include "lact_internal.hpp"
#include <utility>

namespace lact {

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

static lact_status check_shape(const lact_shape* sh) {
  if (sh == nullptr) return LACT_ERR_INVALID_ARG;
  if (sh->bh < 1 || sh->d < 1 || sh->dh < 1) return LACT_ERR_INVALID_ARG;
  if (sh->dtype != LACT_F32 && sh->dtype != LACT_BF16) return LACT_ERR_INVALID_ARG;
  if (sh->d != 64 && sh->d != 128 && sh->d != 256) return LACT_ERR_UNSUPPORTED;
  if (sh->dh % 64 != 0 || sh->dh < sh->d || sh->dh > 4096) return LACT_ERR_UNSUPPORTED;
  if (sh->dtype == LACT_F32 && sh->d > 128) return LACT_ERR_UNSUPPORTED;
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
  if (o->ns_fp32 != 0 && o->ns_fp32 != 1) return LACT_ERR_INVALID_ARG;
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
  const int hpb = grad_hidden_per_block(sh->dtype, sh->d);
  const int64_t base = (int64_t)sh->bh * ((sh->dh + hpb - 1) / hpb);
  int64_t ns = (512 + base - 1) / base;
  const int64_t tiles = (n_tok + 31) / 32;
  if (ns > tiles) ns = tiles;
  if (ns > 64) ns = 64;
  return ns < 1 ? 1 : (int)ns;
}

static int choose_nsplit(const lact_shape* sh, int64_t n_tok) {
  const int hpb = grad_hidden_per_block(sh->dtype, sh->d);
  const int64_t base = (int64_t)sh->bh * ((sh->dh + hpb - 1) / hpb);
  if (sh->dtype != LACT_BF16) {
    // fp32: several workgroups per CU; at least 256 tokens per split
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
  void* shadow2;  // second operand copy of the weights (ns_step_fused shapes)
  int64_t bytes;
};

// Shapes whose Newton-Schulz workgroups also take the weight step (and can
// share their launch with a read, which then needs a second shadow).
static bool ns_step_fused(const lact_shape* sh, const lact_update_opts* op) {
  return op != nullptr && op->use_muon && !op->ns_fp32 && sh->dtype == LACT_BF16 && sh->d == 128 &&
         (sh->dh == 256 || sh->dh == 512);
}

static Workspace layout_ws(const lact_shape* sh, int nsplit, bool muon, char* base,
                           bool shadow2 = false) {
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
  w.shadow2 = shadow2 ? take((int64_t)sh->bh * 2 * msz) : nullptr;
  w.partial = take((int64_t)nsplit * sh->bh * 3 * msz);
  w.beta = take(sh->bh);
  w.g = take((int64_t)3 * sh->bh * msz);
  if (muon) {
    w.xa = take((int64_t)3 * sh->bh * msz);
    w.xb = take((int64_t)3 * sh->bh * msz);
    w.xh = take((int64_t)3 * sh->bh * msz);
    w.amat = take((int64_t)3 * sh->bh * sh->d * sh->d);
    w.bmat = take((int64_t)3 * sh->bh * sh->d * sh->d);
  } else {
    w.xa = w.xb = w.xh = w.amat = w.bmat = nullptr;
  }
  w.bytes = off;
  return w;
}

// ------------------------------------------------------- Newton-Schulz --
static const float kNS[5][3] = {
    {4.0848f, -6.8946f, 2.9270f}, {3.9505f, -6.3029f, 2.6377f}, {3.7418f, -5.5913f, 2.3037f},
    {2.8769f, -3.1427f, 1.2046f}, {2.8366f, -3.0525f, 1.2012f}};

// Newton-Schulz workspace: X fp32 twice, the bf16 copies of X (two, in one
// fp32-sized region), A / B bf16 (one region) and A fp32.
static int64_t ns_ws_bytes(int count, int rows, int cols) {
  const int64_t m = (int64_t)rows * cols;
  return 3 * align256((int64_t)count * m * 4) + 2 * align256((int64_t)count * rows * rows * 4);
}

static hipError_t run_ns(int dtype, int count, int rows, int cols, NsIn g, float* u,
                         float eps, float* xa, float* xb, float* xh, float* am, float* bm,
                         hipStream_t s) {
  const int64_t m = (int64_t)rows * cols;
  hipError_t e = launch_ns_fused(dtype, count, rows, cols, g, u, eps, s);
  if (e != hipErrorNotSupported) return e;
  if (dtype == LACT_BF16) {
    // X fp32 in xa / xb, its bf16 copy in the two halves of xh; A fp32 in bm,
    // A and B bf16 in am
    typedef __bf16 bf16;
    bf16* xh0 = reinterpret_cast<bf16*>(xh);
    bf16* xh1 = xh0 + (int64_t)count * m;
    bf16* ah = reinterpret_cast<bf16*>(am);
    bf16* bh = ah + (int64_t)count * rows * rows;
    const int64_t rr = (int64_t)rows * rows;
    if ((e = launch_nsn(g, bm, xa, xh0, count, m, eps, s)) != hipSuccess) return e;
    float* x = xa;
    float* y = xb;
    bf16* xc = xh0;
    bf16* yc = xh1;
    for (int it = 0; it < 5; ++it) {
      const float ca = kNS[it][0], cb = kNS[it][1], cc = kNS[it][2];
      // A = X X^T (fp32 for the b A term, bf16 operand)
      NsGemmArgs ga{xc, m, cols, xc, m, cols, nullptr, 0, bm, ah, rr, rows, rows, cols, 1.f, 0.f};
      if ((e = launch_nsgemm(false, ga, count, s)) != hipSuccess) return e;
      // B = c A A + b A (A symmetric: its rows are the B operand)
      NsGemmArgs gb{ah, rr, rows, ah, rr, rows, bm, rr, nullptr, bh, rr, rows, rows, rows, cc, cb};
      if ((e = launch_nsgemm(false, gb, count, s)) != hipSuccess) return e;
      // X' = B X + a X
      const bool last = it == 4;
      NsGemmArgs gx{bh, rr, rows, xc, m, cols, x, m, last ? u : y, last ? nullptr : yc, m,
                    rows, cols, rows, 1.f, ca};
      if ((e = launch_nsgemm(true, gx, count, s)) != hipSuccess) return e;
      std::swap(x, y);
      std::swap(xc, yc);
    }
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
    if ((e = launch_gemm(dtype, ga, s)) != hipSuccess) return e;
    // B = c A A + b A
    GemmArgs gb{am, (int64_t)rows * rows, am, (int64_t)rows * rows, 1, am, (int64_t)rows * rows,
                bm, (int64_t)rows * rows, rows, rows, rows, count, cc, cb};
    if ((e = launch_gemm(dtype, gb, s)) != hipSuccess) return e;
    // X' = B X + a X
    float* out = (it == 4) ? u : y;
    GemmArgs gx{bm, (int64_t)rows * rows, x, m, 1, x, m, out, m, rows, cols, rows, count, 1.f, ca};
    if ((e = launch_gemm(dtype, gx, s)) != hipSuccess) return e;
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
                            hipStream_t s) {
  if (n_tok == 0) return LACT_OK;
  const ApplyArgs a = apply_args(sh, st, q, ql, o, ol, n_tok);
  hipError_t e;
  {
    ProfScope p(LACT_PROF_APPLY, s);
    e = launch_apply(sh->dtype, a, s);
  }
  return e == hipSuccess ? LACT_OK : hip_fail(e);
}

static lact_status do_grad(const lact_shape* sh, const lact_state* st, const void* k,
                           lact_layout kl, const void* v, lact_layout vl, const float* e1,
                           const float* e3, const float* e2, int64_t esbh, int64_t n_tok,
                           const Workspace& w, int nsplit, float* o1, float* o3, float* o2,
                           float* m1, float* m3, float* m2, const float* mom, hipStream_t s,
                           bool reduce = true) {
  GradArgs a;
  a.k = k; a.k_sbh = kl.stride_bh; a.k_st = kl.stride_tok;
  a.v = v; a.v_sbh = vl.stride_bh; a.v_st = vl.stride_tok;
  a.eta1 = e1; a.eta3 = e3; a.eta2 = e2; a.eta_sbh = esbh;
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
  if (!reduce) return LACT_OK;  // the consumer sums the partials itself
  ReduceArgs r{w.partial, nsplit, sh->bh, sh->d, sh->dh, o1, o3, o2, m1, m3, m2, w.beta};
  {
    ProfScope p(LACT_PROF_REDUCE, s);
    e = launch_reduce(r, s);
  }
  return e == hipSuccess ? LACT_OK : hip_fail(e);
}

static lact_status do_step(const lact_shape* sh, const lact_state* st, const float* u1,
                           const float* u3, const float* u2, int renorm, float eps,
                           void* shadow_out, hipStream_t s) {
  StepArgs a;
  memset(&a, 0, sizeof(a));
  a.w1 = st->w1; a.w3 = st->w3; a.w2 = st->w2;
  a.u1 = u1; a.u3 = u3; a.u2 = u2;
  a.n1 = st->n1; a.n3 = st->n3; a.n2 = st->n2;
  a.sh = make_shadow(shadow_out, sh->d, sh->dh);
  a.bh = sh->bh; a.d = sh->d; a.dh = sh->dh;
  a.renorm = renorm; a.eps = eps;
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
                             void* shadow_out = nullptr) {
  if (shadow_out == nullptr) shadow_out = st->shadow;
  const bool nsstep = ns_step_fused(sh, op);
  const bool fuse = nsstep && job != nullptr && job->n_tok > 0 && shadow_out != st->shadow;
  if (job != nullptr && !fuse) {
    lact_status r = do_apply(sh, st, job->q, job->ql, job->o, job->ol, job->n_tok, s);
    if (r != LACT_OK) return r;
  }
  const int nsplit = choose_nsplit(sh, n_tok);
  Workspace w = layout_ws(sh, nsplit, op->use_muon != 0, reinterpret_cast<char*>(ws), nsstep);
  const int64_t msz = (int64_t)sh->d * sh->dh;
  const int64_t mall = (int64_t)sh->bh * msz;
  float* g1 = w.g;
  float* g3 = w.g + mall;
  float* g2 = w.g + 2 * mall;
  // with momentum the reduced gradient lives in M only (M <- G + beta M)
  const bool mo = op->use_momentum != 0;
  lact_status r = do_grad(sh, st, k, kl, v, vl, e1, e3, e2, esbh, n_tok, w, nsplit,
                          mo ? nullptr : g1, mo ? nullptr : g3, mo ? nullptr : g2,
                          mo ? st->m1 : nullptr, mo ? st->m3 : nullptr, mo ? st->m2 : nullptr,
                          mo ? mom : nullptr, s, !nsstep);
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
                      make_shadow(shadow_out, sh->d, sh->dh), sh->bh, op->renorm ? 1 : 0,
                      op->renorm_eps};
      const NsGrad gr{w.partial, nsplit, sh->bh,
                      {mo ? st->m1 : nullptr, mo ? st->m3 : nullptr, mo ? st->m2 : nullptr}};
      e = launch_ns_step_apply(3 * sh->bh, sh->d, sh->dh, gr, op->ns_eps, ns, aa, s);
      return e == hipSuccess ? LACT_OK : hip_fail(e);
    }
    e = run_ns(op->ns_fp32 ? LACT_F32 : sh->dtype, 3 * sh->bh, sh->d, sh->dh, in, w.g,
               op->ns_eps, w.xa, w.xb, w.xh, w.amat, w.bmat, s);
    if (e != hipSuccess) return hip_fail(e);
    u1 = g1; u3 = g3; u2 = g2;
  }
  return do_step(sh, st, u1, u3, u2, op->renorm ? 1 : 0, op->renorm_eps, shadow_out, s);
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
  const int ns = sh->dtype == LACT_BF16 ? nsplit_bound(sh, max_update_tokens)
                                         : choose_nsplit(sh, max_update_tokens);
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
  const int nsplit = choose_nsplit(sh, n_tok);
  Workspace w = layout_ws(sh, nsplit, false, reinterpret_cast<char*>(ws));
  return do_grad(sh, st, k, kl, v, vl, e1, e3, e2, esbh, n_tok, w, nsplit, g1, g3, g2, nullptr,
                 nullptr, nullptr, nullptr, (hipStream_t)stream);
}

lact_status lact_newton_schulz(int32_t count, int32_t rows, int32_t cols, int32_t dtype,
                               const float* g, float* u, float eps, void* ws, size_t ws_bytes,
                               void* stream) {
  if (count < 1 || rows < 1 || cols < 1 || g == nullptr || u == nullptr) return LACT_ERR_INVALID_ARG;
  if (dtype != LACT_F32 && dtype != LACT_BF16) return LACT_ERR_INVALID_ARG;
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
  const NsIn in{{g, g, g}, count};
  hipError_t e = run_ns(dtype, count, rows, cols, in, u, eps, xa, xb, xh, a_, b_, (hipStream_t)stream);
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
  return do_step(sh, st, u1, u3, u2, op->renorm ? 1 : 0, op->renorm_eps, st->shadow,
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
  r = do_update(sh, st, k, kl, v, vl, e1, e3, e2, mom, esbh, n_tok, op, ws, s, &job, alt);
  if (r != LACT_OK || alt == nullptr) return r;
  const hipError_t e = launch_copy16(st->shadow, alt, (int64_t)lact_shadow_bytes(sh), s);
  return e == hipSuccess ? LACT_OK : hip_fail(e);
}

lact_status lact_sequence(const lact_shape* sh, const lact_state* st, const void* q,
                          lact_layout ql, const void* k, lact_layout kl, const void* v,
                          lact_layout vl, void* o, lact_layout ol, const float* e1,
                          const float* e3, const float* e2, const float* mom, int64_t esbh,
                          int64_t T, int64_t chunk, int32_t order, int64_t sub_off,
                          int64_t sub_len, int32_t update_last, const lact_update_opts* op,
                          void* ws, size_t ws_bytes, void* stream) {
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
  hipStream_t s = (hipStream_t)stream;
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
    const lact_status rr = do_update(sh, &cs, kp, kl, vp, vl, e1 + a0, e3 + a0, e2 + a0,
                                     mom ? mom + a0 : nullptr, esbh, n, op, ws, s, job, out);
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
  }
  return "unknown status";
}

int lact_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"
