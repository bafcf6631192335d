// C ABI of libfwmem: argument checks, buffer layout and dispatch to the launchers.
// Every check runs on the host before anything is enqueued; the functions keep no
// state between calls.
#include "fwmem.h"

#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstring>

#include "fwmem_backward.h"
#include "fwmem_internal.h"

namespace {

using fwmem::kChunk;

constexpr uint32_t kKnownFlags =
    FWMEM_PHI_ELU1 | FWMEM_LAMBDA_PER_CHANNEL | FWMEM_OUT_BF16 | FWMEM_QK_L2NORM | FWMEM_QK_RMSNORM |
    FWMEM_BETA_SIGMOID | FWMEM_BETA_SIGMOID2 | FWMEM_LAMBDA_PREACT | FWMEM_ZNORM |
    FWMEM_LAMBDA_SCALED;

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Half-open byte ranges [a, a+na) and [b, b+nb) intersect (empty ranges never do).
bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  if (a == nullptr || b == nullptr || na == 0 || nb == 0) return false;
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

struct Sizes {
  size_t BH, nS, nX, nH;  // element counts of the state parts
  size_t state_bytes;
};

Sizes sizes_of(const fwmem_shape* s) {
  Sizes z;
  z.BH = (size_t)s->B * (size_t)s->H;
  z.nS = z.BH * (size_t)s->dk * (size_t)s->dv;
  z.nX = z.BH * (size_t)s->dk;
  z.nH = z.BH;
  z.state_bytes = align256(4 * (z.nS + z.nX + z.nH));
  return z;
}

fwmem_status check_shape(const fwmem_shape* s, bool need_T) {
  if (s == nullptr) return FWMEM_EINVAL;
  if (s->B < 0 || s->H < 0 || s->dk <= 0 || s->dv <= 0) return FWMEM_EINVAL;
  if (need_T && s->T < 0) return FWMEM_EINVAL;
  if (s->dtype != FWMEM_F32 && s->dtype != FWMEM_BF16) return FWMEM_EINVAL;
  return FWMEM_OK;
}

fwmem_status check_mode(const fwmem_mode* m) {
  if (m == nullptr) return FWMEM_EINVAL;
  if (m->rule != FWMEM_RULE_DELTA && m->rule != FWMEM_RULE_ADDITIVE && m->rule != FWMEM_RULE_INNER &&
      m->rule != FWMEM_RULE_DELTA_PV)
    return FWMEM_EINVAL;
  // one step size per value channel, with a scalar ridge
  if (m->rule == FWMEM_RULE_DELTA_PV && (m->flags & FWMEM_LAMBDA_PER_CHANNEL)) return FWMEM_EUNSUPPORTED;
  if ((m->flags & ~kKnownFlags) != 0) return FWMEM_EINVAL;
  // one normalisation at a time, and only of the raw q and k (identity feature map)
  if ((m->flags & FWMEM_QK_L2NORM) && (m->flags & FWMEM_QK_RMSNORM)) return FWMEM_EINVAL;
  if ((m->flags & FWMEM_BETA_SIGMOID) && (m->flags & FWMEM_BETA_SIGMOID2)) return FWMEM_EINVAL;
  if ((m->flags & (FWMEM_QK_L2NORM | FWMEM_QK_RMSNORM)) && (m->flags & FWMEM_PHI_ELU1))
    return FWMEM_EUNSUPPORTED;
  // the normaliser accumulates the additive rule's writes
  if ((m->flags & FWMEM_ZNORM) && m->rule != FWMEM_RULE_ADDITIVE) return FWMEM_EUNSUPPORTED;
  // the additive rule's lambda is a retention, not a ridge
  if ((m->flags & FWMEM_LAMBDA_SCALED) && m->rule == FWMEM_RULE_ADDITIVE) return FWMEM_EUNSUPPORTED;
  if (!std::isfinite(m->eps) || m->eps < 0.f) return FWMEM_EINVAL;
  if (m->chunk != 0 && m->chunk != kChunk) return FWMEM_EUNSUPPORTED;
  return FWMEM_OK;
}

// Scans divide their float32 outputs in place and keep one normaliser per key channel
// only for a scalar decay; they couple the ridge to the key energy for a scalar lambda.
fwmem_status check_scan_mode(const fwmem_mode* m) {
  const fwmem_status st = check_mode(m);
  if (st != FWMEM_OK) return st;
  if ((m->flags & FWMEM_ZNORM) && (m->flags & (FWMEM_LAMBDA_PER_CHANNEL | FWMEM_OUT_BF16)))
    return FWMEM_EUNSUPPORTED;
  if ((m->flags & FWMEM_LAMBDA_SCALED) && (m->flags & FWMEM_LAMBDA_PER_CHANNEL))
    return FWMEM_EUNSUPPORTED;
  return FWMEM_OK;
}

// Pointers into a state buffer.
struct StatePtrs {
  float* S;
  float* x;
  int32_t* h;
};

// Workspace of a scan: the (head, chunk) records, and for a segmented scan (P > 1 segments
// per head, see SegParams) the virtual state buffers and each segment's decay; with
// FWMEM_ZNORM the normaliser's chunk terms (ZRec) and its value at every chunk entry.
struct WsLayout {
  int P;
  size_t rec, A0, B0, A1, B1, z, zr, zc, total;
};

size_t record_bytes(int bf16, int dk, const fwmem_mode* m) {
  if (fwmem::scan_add_path(bf16, m->rule, m->flags)) return 0;  // the fused kernel keeps no records
  return m->rule == FWMEM_RULE_DELTA_PV ? fwmem::scan_pv_record_bytes()
                                        : fwmem::scan_record_bytes(bf16, dk, m->flags);
}

WsLayout ws_layout(const fwmem_shape* s, const fwmem_mode* m) {
  WsLayout w{};
  const size_t BH = (size_t)s->B * (size_t)s->H, T = (size_t)s->T;
  const size_t nchunks = (T + kChunk - 1) / kChunk;
  const int bf16 = s->dtype == FWMEM_BF16 ? 1 : 0;
  const bool pv = m->rule == FWMEM_RULE_DELTA_PV;
  w.P = (T > 0 && !pv) ? fwmem::scan_segments(BH, T, s->dk, s->dv, bf16, m->rule, m->flags) : 1;
  size_t off = align256(BH * nchunks * record_bytes(bf16, s->dk, m));
  w.rec = 0;
  if (w.P > 1) {
    const size_t VH = BH * (size_t)w.P, dk = (size_t)s->dk, dv = (size_t)s->dv;
    // diagonal transitions need no transition states; gam [BH*P] holds each segment's
    // decay; the combine writes the segments' start states into B0 in both cases
    const bool diag = fwmem::seg_diagonal(m->rule, m->flags);
    const size_t sa = diag ? 0 : align256(4 * (VH * dk * dk + VH * dk + VH));
    const size_t sb = align256(4 * (VH * dk * dv + VH * dk + VH));
    w.A0 = off;
    w.A1 = w.A0 + sa;
    w.B0 = w.A1 + sa;
    w.B1 = w.B0 + sb;
    off = w.B1 + sb;
    w.z = off;
    off += align256(4 * VH);
  }
  // the normaliser's chunk terms and chunk-entry values (the fused additive kernel carries
  // the normaliser itself)
  if ((m->flags & FWMEM_ZNORM) && !fwmem::scan_add_path(bf16, m->rule, m->flags)) {
    w.zr = off;
    off += align256(4 * BH * nchunks * fwmem::zrec_floats(s->dk));
    w.zc = off;
    off += align256(4 * BH * nchunks * (size_t)s->dk);
  }
  w.total = T > 0 ? off : 0;
  return w;
}

StatePtrs state_ptrs(const void* base, const Sizes& z) {
  char* b = static_cast<char*>(const_cast<void*>(base));
  if (b == nullptr) return {nullptr, nullptr, nullptr};
  return {reinterpret_cast<float*>(b), reinterpret_cast<float*>(b + 4 * z.nS),
          reinterpret_cast<int32_t*>(b + 4 * (z.nS + z.nX))};
}

size_t esize(int dtype) { return dtype == FWMEM_BF16 ? 2 : 4; }

}  // namespace

namespace fwmem {
void wait_config(int* polls, int* bias) {
  *polls = 1 << 22;
  *bias = 0;
  const char* e = std::getenv("FWMEM_TEST_WAIT_TIMEOUT");
  if (e != nullptr) {
    const long n = std::strtol(e, nullptr, 10);
    if (n > 0 && n < (1 << 22)) {
      *polls = (int)n;
      *bias = 1 << 30;
    }
  }
}
}  // namespace fwmem

extern "C" {

const char* fwmem_version(void) { return "0.2.0"; }

fwmem_status fwmem_check_device(fwmem_stream stream) {
  int v = 0;
  if (fwmem::read_wait_status(reinterpret_cast<hipStream_t>(stream), &v) != hipSuccess)
    return FWMEM_ELAUNCH;
  return v != 0 ? FWMEM_EWAIT : FWMEM_OK;
}

const char* fwmem_strerror(fwmem_status st) {
  switch (st) {
    case FWMEM_OK: return "ok";
    case FWMEM_EINVAL: return "invalid argument";
    case FWMEM_EUNSUPPORTED: return "unsupported size or chunk length";
    case FWMEM_EALIGN: return "misaligned pointer";
    case FWMEM_EOVERLAP: return "overlapping buffers";
    case FWMEM_ELAUNCH: return "kernel launch failed";
    case FWMEM_EWORKSPACE: return "workspace missing or too small";
    case FWMEM_ESCRATCH: return "the call needs more workspace than the fixed device scratch holds";
    case FWMEM_EWAIT: return "a kernel's bounded wait gave up: results since the last check are wrong";
    case FWMEM_STATUS_MAX_ENUM: break;
  }
  return "unknown status";
}

fwmem_status fwmem_state_bytes(const fwmem_shape* shape, size_t* bytes) {
  if (bytes == nullptr) return FWMEM_EINVAL;
  const fwmem_status st = check_shape(shape, false);
  if (st != FWMEM_OK) return st;
  *bytes = sizes_of(shape).state_bytes;
  return FWMEM_OK;
}

fwmem_status fwmem_scan_workspace_bytes(const fwmem_shape* shape, const fwmem_mode* mode,
                                        size_t* bytes) {
  if (bytes == nullptr) return FWMEM_EINVAL;
  fwmem_status st = check_shape(shape, true);
  if (st != FWMEM_OK) return st;
  st = check_scan_mode(mode);
  if (st != FWMEM_OK) return st;
  if (!fwmem::scan_supported(shape->dk, shape->dv)) return FWMEM_EUNSUPPORTED;
  *bytes = ws_layout(shape, mode).total;
  return FWMEM_OK;
}

}  // extern "C"

namespace {

fwmem_status scan_impl(const fwmem_shape* shape, const void* q, const void* k, const void* v,
                       const float* beta, const float* lambda, const fwmem_mode* mode,
                       const void* S_in, void* out, void* S_out, void* workspace, size_t ws_bytes,
                       fwmem_stream stream, int phases) {
  fwmem_status st = check_shape(shape, true);
  if (st != FWMEM_OK) return st;
  st = check_scan_mode(mode);
  if (st != FWMEM_OK) return st;
  if (!fwmem::scan_supported(shape->dk, shape->dv)) return FWMEM_EUNSUPPORTED;

  const Sizes z = sizes_of(shape);
  if (z.BH == 0) return FWMEM_OK;
  // the delta and inner-product rules take beta as their step size
  const bool needs_beta = mode->rule != FWMEM_RULE_ADDITIVE;
  const bool pc = (mode->flags & FWMEM_LAMBDA_PER_CHANNEL) != 0;
  const size_t T = (size_t)shape->T;
  const size_t es = esize(shape->dtype);

  if (T > 0) {
    if (q == nullptr || k == nullptr || v == nullptr || out == nullptr) return FWMEM_EINVAL;
    if (needs_beta && beta == nullptr) return FWMEM_EINVAL;
  }
  // alignment
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) ||
      !aligned(S_in, 16) || !aligned(S_out, 16) || !aligned(workspace, 16) ||
      !aligned(beta, mode->rule == FWMEM_RULE_DELTA_PV ? 16 : 4) || !aligned(lambda, pc ? 16 : 4))
    return FWMEM_EALIGN;

  // overlap
  const size_t nq = z.BH * T * shape->dk * es, nv = z.BH * T * shape->dv * es;
  const bool rule_pv = mode->rule == FWMEM_RULE_DELTA_PV;
  const size_t nb = z.BH * T * 4 * (rule_pv ? shape->dv : 1), nl = z.BH * T * 4 * (pc ? shape->dk : 1);
  const size_t no = z.BH * T * shape->dv * ((mode->flags & FWMEM_OUT_BF16) ? 2 : 4);
  size_t need = 0;
  st = fwmem_scan_workspace_bytes(shape, mode, &need);
  if (st != FWMEM_OK) return st;
  if (S_in != nullptr && S_out != nullptr && S_in != S_out &&
      overlap(S_in, z.state_bytes, S_out, z.state_bytes))
    return FWMEM_EOVERLAP;
  const void* ins[] = {q, k, v, beta, lambda, S_in, S_out, workspace};
  const size_t nins[] = {nq, nq, nv, nb, nl, z.state_bytes, z.state_bytes, need};
  for (int i = 0; i < 8; ++i)
    if (overlap(out, no, ins[i], nins[i])) return FWMEM_EOVERLAP;
  for (int i = 0; i < 7; ++i)
    if (overlap(workspace, need, ins[i], nins[i])) return FWMEM_EOVERLAP;
  if (S_out != nullptr)
    for (int i = 0; i < 5; ++i)
      if (overlap(S_out, z.state_bytes, ins[i], nins[i])) return FWMEM_EOVERLAP;

  const StatePtrs si = state_ptrs(S_in, z), so = state_ptrs(S_out, z);
  hipStream_t hs = reinterpret_cast<hipStream_t>(stream);

  if (T == 0) {
    if (S_out == nullptr || S_out == S_in || (phases & 2) == 0) return FWMEM_OK;
    const hipError_t e = fwmem::launch_state_copy(si.S, si.x, si.h, so.S, so.x, so.h, z.nS, z.nX,
                                                  z.nH, hs);
    return e == hipSuccess ? FWMEM_OK : FWMEM_ELAUNCH;
  }
  if (ws_bytes < need || (need > 0 && workspace == nullptr)) return FWMEM_EWORKSPACE;

  fwmem::ScanParams p;
  std::memset(&p, 0, sizeof(p));
  p.q = q;
  p.k = k;
  p.v = v;
  p.beta = beta;
  p.lam = lambda;
  p.S_in = si.S;
  p.xprev_in = si.x;
  p.has_in = si.h;
  p.out = out;
  p.S_out = so.S;
  p.xprev_out = so.x;
  p.has_out = so.h;
  p.ws = static_cast<char*>(workspace);
  p.BH = (int)z.BH;
  p.T = (int)T;
  p.dk = shape->dk;
  p.dv = shape->dv;
  p.nchunks = (int)((T + kChunk - 1) / kChunk);
  p.rule = mode->rule;
  p.bf16 = shape->dtype == FWMEM_BF16 ? 1 : 0;
  p.flags = mode->flags;
  p.eps = mode->eps;
  fwmem::wait_config(&p.wait_polls, &p.wait_bias);
  if (z.BH > 0x7fffffff / 8 || (size_t)p.nchunks * z.BH > 0x7fffffffu) return FWMEM_EUNSUPPORTED;
  // per-head byte offsets of every buffer (inputs, outputs, records) stay below 2^31
  const size_t dmax = (size_t)(shape->dk > shape->dv ? shape->dk : shape->dv);
  if (T * dmax * 4 > 0x7fffffffu ||
      (size_t)p.nchunks * record_bytes(p.bf16, shape->dk, mode) > 0x7fffffffu)
    return FWMEM_EUNSUPPORTED;

  const WsLayout wl = ws_layout(shape, mode);
  if (rule_pv) {
    const hipError_t e = fwmem::launch_scan_pv(p, hs, phases);
    return e == hipSuccess ? FWMEM_OK : FWMEM_ELAUNCH;
  }
  // Normalised linear attention: prep writes the chunk terms of z, and after the
  // propagate kernels z is chained over the chunks of each head and divides the outputs.
  // Records of virtual heads (segments) are those of the real heads' chunks in order, so
  // the chain always runs over the real heads. The fused additive kernel (elu + 1 on bf16)
  // carries z as one more column itself and needs none of this.
  fwmem::ZParams zp;
  std::memset(&zp, 0, sizeof(zp));
  const bool zkern = (mode->flags & FWMEM_ZNORM) && !fwmem::scan_add_path(p.bf16, mode->rule, mode->flags);
  if (zkern) {
    char* ws = static_cast<char*>(workspace);
    p.zrec = reinterpret_cast<float*>(ws + wl.zr);
    zp.zrec = p.zrec;
    zp.zc = reinterpret_cast<float*>(ws + wl.zc);
    zp.z_in = si.x;
    zp.z_out = so.x;
    zp.has_out = so.h;
    zp.q = q;
    zp.out = static_cast<float*>(out);
    zp.BH = p.BH;
    zp.T = p.T;
    zp.nchunks = p.nchunks;
    zp.dk = p.dk;
    zp.dv = p.dv;
    zp.bf16 = p.bf16;
    zp.flags = p.flags;
    zp.eps = p.eps;
  }
  auto znorm = [&](hipError_t e) {
    if (e == hipSuccess && zkern && (phases & 2)) e = fwmem::launch_znorm(zp, hs);
    return e;
  };
  if (wl.P == 1) {
    const hipError_t e = znorm(fwmem::launch_scan(p, hs, phases));
    return e == hipSuccess ? FWMEM_OK : FWMEM_ELAUNCH;
  }

  // Segmented scan: P segments of each head run as virtual heads (SegParams). The prep
  // phase sets up the virtual states and builds every record. The propagate phase forms
  // each segment's own state change (with diagonal transitions directly; otherwise by a
  // local and a transition pass that compute states only), chains the segments, and runs
  // one pass from the true start states that writes the outputs.
  char* ws = static_cast<char*>(workspace);
  const size_t VH = z.BH * (size_t)wl.P, dk = (size_t)shape->dk, dv = (size_t)shape->dv;
  fwmem::SegParams sp;
  std::memset(&sp, 0, sizeof(sp));
  sp.k = k;
  sp.S_in = si.S;
  sp.xprev_in = si.x;
  sp.has_in = si.h;
  sp.S_out = so.S;
  sp.xprev_out = so.x;
  sp.has_out = so.h;
  // a virtual state buffer at byte offset o with n value columns: S, x_prev, has_prev
  auto vstate = [&](size_t o, size_t n, float*& S, float*& x, int32_t*& h) {
    S = reinterpret_cast<float*>(ws + o);
    x = S + VH * dk * n;
    h = reinterpret_cast<int32_t*>(x + VH * dk);
  };
  float *A1_x, *B1_x_unused;
  int32_t *A1_h, *B1_h;
  vstate(wl.A0, dk, sp.A0_S, sp.A0_x, sp.A0_h);
  vstate(wl.B0, dv, sp.B0_S, sp.B0_x, sp.B0_h);
  vstate(wl.A1, dk, sp.A1_S, A1_x, A1_h);
  vstate(wl.B1, dv, sp.B1_S, sp.B1_x, B1_h);
  (void)B1_x_unused;
  sp.out = static_cast<float*>(out);
  sp.BH = (int)z.BH;
  sp.P = wl.P;
  sp.L = (int)(T / (size_t)wl.P);
  sp.dk = shape->dk;
  sp.dv = shape->dv;
  sp.bf16 = p.bf16;
  sp.flags = p.flags;
  sp.diag = fwmem::seg_diagonal(mode->rule, mode->flags) ? 1 : 0;
  sp.zfused = (mode->flags & FWMEM_ZNORM) && fwmem::scan_add_path(p.bf16, mode->rule, mode->flags) ? 1 : 0;
  sp.q = q;
  sp.v = v;
  sp.beta = beta;
  sp.lam = lambda;
  sp.gam = reinterpret_cast<float*>(ws + wl.z);
  // the combine writes the start states where the output pass starts
  sp.S_start = sp.B0_S;

  fwmem::ScanParams pv = p;  // the output pass over the virtual heads, from the start states in B0
  pv.BH = (int)VH;
  pv.T = sp.L;
  pv.nchunks = sp.L / kChunk;
  pv.S_in = sp.B0_S;
  pv.xprev_in = sp.B0_x;
  pv.has_in = sp.B0_h;
  pv.S_out = sp.B1_S;
  pv.xprev_out = sp.B1_x;
  pv.has_out = B1_h;
  fwmem::ScanParams pl = pv;  // the local pass: each segment's own state from zero, no outputs
  pl.out = nullptr;
  pl.S_in = nullptr;
  fwmem::ScanParams pa = pv;  // the transition pass: identity start, zero values, no outputs
  pa.v = nullptr;
  pa.dv = shape->dk;
  pa.out = nullptr;
  pa.S_in = sp.A0_S;
  pa.xprev_in = sp.A0_x;
  pa.has_in = sp.A0_h;
  pa.S_out = sp.A1_S;
  pa.xprev_out = A1_x;
  pa.has_out = A1_h;

  hipError_t e = hipSuccess;
  if (phases & 1) {
    e = fwmem::launch_seg_init(sp, hs);
    if (e == hipSuccess) e = fwmem::launch_scan(pv, hs, 1);
  }
  if (e == hipSuccess && (phases & 2)) {
    if (sp.diag) {
      e = fwmem::launch_seg_state(sp, hs);
      if (e == hipSuccess) e = fwmem::launch_seg_combine(sp, hs);
      if (e == hipSuccess) e = fwmem::launch_scan(pv, hs, 2);
      if (e == hipSuccess) e = fwmem::launch_seg_extras(sp, hs);
    } else {
      e = fwmem::launch_scan(pl, hs, 2);
      if (e == hipSuccess) e = fwmem::launch_scan(pa, hs, 2);
      if (e == hipSuccess) e = fwmem::launch_seg_combine(sp, hs);
      if (e == hipSuccess) e = fwmem::launch_scan(pv, hs, 2);
    }
  }
  e = znorm(e);
  return e == hipSuccess ? FWMEM_OK : FWMEM_ELAUNCH;
}

}  // namespace

extern "C" {

fwmem_status fwmem_scan_fwd(const fwmem_shape* shape, const void* q, const void* k, const void* v,
                            const float* beta, const float* lambda, const fwmem_mode* mode,
                            const void* S_in, void* out, void* S_out, void* workspace,
                            size_t ws_bytes, fwmem_stream stream) {
  return scan_impl(shape, q, k, v, beta, lambda, mode, S_in, out, S_out, workspace, ws_bytes,
                   stream, 3);
}

fwmem_status fwmem_scan_chunk_prep(const fwmem_shape* shape, const void* q, const void* k,
                                   const void* v, const float* beta, const float* lambda,
                                   const fwmem_mode* mode, const void* S_in, void* out,
                                   void* S_out, void* workspace, size_t ws_bytes,
                                   fwmem_stream stream) {
  return scan_impl(shape, q, k, v, beta, lambda, mode, S_in, out, S_out, workspace, ws_bytes,
                   stream, 1);
}

fwmem_status fwmem_scan_chunk_propagate(const fwmem_shape* shape, const void* q, const void* k,
                                        const void* v, const float* beta, const float* lambda,
                                        const fwmem_mode* mode, const void* S_in, void* out,
                                        void* S_out, void* workspace, size_t ws_bytes,
                                        fwmem_stream stream) {
  return scan_impl(shape, q, k, v, beta, lambda, mode, S_in, out, S_out, workspace, ws_bytes,
                   stream, 2);
}

fwmem_status fwmem_step(const fwmem_shape* shape, const void* q, const void* k, const void* v,
                        const float* beta, const float* lambda, const fwmem_mode* mode,
                        const void* S_in, void* out, void* S_out, fwmem_stream stream) {
  fwmem_status st = check_shape(shape, false);
  if (st != FWMEM_OK) return st;
  st = check_mode(mode);
  if (st != FWMEM_OK) return st;
  if (!fwmem::step_supported(shape->dk, shape->dv)) return FWMEM_EUNSUPPORTED;
  const Sizes z = sizes_of(shape);
  if (z.BH == 0) return FWMEM_OK;
  // the delta and inner-product rules take beta as their step size
  const bool needs_beta = mode->rule != FWMEM_RULE_ADDITIVE;
  const bool pc = (mode->flags & FWMEM_LAMBDA_PER_CHANNEL) != 0;
  if (q == nullptr || k == nullptr || v == nullptr || out == nullptr || S_out == nullptr)
    return FWMEM_EINVAL;
  if (needs_beta && beta == nullptr) return FWMEM_EINVAL;
  const size_t es = esize(shape->dtype);
  if (!aligned(q, es) || !aligned(k, es) || !aligned(v, es) || !aligned(out, 16) ||
      !aligned(S_in, 16) || !aligned(S_out, 16) || !aligned(beta, 4) || !aligned(lambda, 4))
    return FWMEM_EALIGN;
  const size_t nq = z.BH * shape->dk * es, nv = z.BH * shape->dv * es;
  const size_t nb = z.BH * 4 * (mode->rule == FWMEM_RULE_DELTA_PV ? shape->dv : 1);
  const size_t nl = z.BH * 4 * (pc ? shape->dk : 1);
  const size_t no = z.BH * shape->dv * ((mode->flags & FWMEM_OUT_BF16) ? 2 : 4);
  if (S_in != nullptr && S_in != S_out && overlap(S_in, z.state_bytes, S_out, z.state_bytes))
    return FWMEM_EOVERLAP;
  const void* ins[] = {q, k, v, beta, lambda, S_in, S_out};
  const size_t nins[] = {nq, nq, nv, nb, nl, z.state_bytes, z.state_bytes};
  for (int i = 0; i < 7; ++i)
    if (overlap(out, no, ins[i], nins[i])) return FWMEM_EOVERLAP;
  for (int i = 0; i < 5; ++i)
    if (overlap(S_out, z.state_bytes, ins[i], nins[i])) return FWMEM_EOVERLAP;

  const StatePtrs si = state_ptrs(S_in, z), so = state_ptrs(S_out, z);
  fwmem::StepParams p;
  std::memset(&p, 0, sizeof(p));
  p.q = q;
  p.k = k;
  p.v = v;
  p.beta = beta;
  p.lam = lambda;
  p.S_in = si.S;
  p.xprev_in = si.x;
  p.has_in = si.h;
  p.out = out;
  p.S_out = so.S;
  p.xprev_out = so.x;
  p.has_out = so.h;
  p.BH = (int)z.BH;
  p.dk = shape->dk;
  p.dv = shape->dv;
  p.rule = mode->rule;
  p.bf16 = shape->dtype == FWMEM_BF16 ? 1 : 0;
  p.flags = mode->flags;
  p.eps = mode->eps;
  if (z.BH > 0x7fffffffu) return FWMEM_EUNSUPPORTED;
  const hipError_t e = fwmem::launch_step(p, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? FWMEM_OK : FWMEM_ELAUNCH;
}

}  // extern "C"

// ---- backward pass

namespace {

fwmem_status check_bwd(const fwmem_shape* shape, const fwmem_mode* mode) {
  fwmem_status st = check_shape(shape, true);
  if (st != FWMEM_OK) return st;
  st = check_scan_mode(mode);
  if (st != FWMEM_OK) return st;
  if ((mode->flags & ~(uint32_t)(FWMEM_PHI_ELU1 | FWMEM_LAMBDA_PER_CHANNEL | FWMEM_BETA_SIGMOID |
                                 FWMEM_BETA_SIGMOID2 | FWMEM_LAMBDA_PREACT | FWMEM_QK_L2NORM |
                                 FWMEM_QK_RMSNORM | FWMEM_LAMBDA_SCALED | FWMEM_ZNORM)) != 0)
    return FWMEM_EUNSUPPORTED;
  if (!fwmem::bwd_supported(shape->dk, shape->dv)) return FWMEM_EUNSUPPORTED;
  return FWMEM_OK;
}

size_t bwd_ws_bytes(const fwmem_shape* shape, const fwmem_mode* mode) {
  const size_t BH = (size_t)shape->B * (size_t)shape->H;
  if (fwmem::bwd_chunked(mode->rule, mode->flags, shape->T))
    return align256(4 * BH * fwmem::bwd_chunk_floats_per_head(shape->T, shape->dk, shape->dv));
  const bool zn = (mode->flags & FWMEM_ZNORM) != 0;
  const bool small = (mode->flags & FWMEM_LAMBDA_PER_CHANNEL) != 0 || mode->rule == FWMEM_RULE_DELTA_PV || zn;
  return align256(4 * BH * fwmem::bwd_floats_per_head(shape->T, shape->dk, shape->dv, small, zn));
}

}  // namespace

extern "C" {

fwmem_status fwmem_scan_bwd_workspace_bytes(const fwmem_shape* shape, const fwmem_mode* mode,
                                            size_t* bytes) {
  if (bytes == nullptr) return FWMEM_EINVAL;
  const fwmem_status st = check_bwd(shape, mode);
  if (st != FWMEM_OK) return st;
  *bytes = bwd_ws_bytes(shape, mode);
  return FWMEM_OK;
}

fwmem_status fwmem_scan_bwd(const fwmem_shape* shape, const void* q, const void* k,
                            const void* v, const float* beta, const float* lambda,
                            const fwmem_mode* mode, const void* S_in, const float* grad_out,
                            const void* grad_S_out, float* grad_q, float* grad_k,
                            float* grad_v, float* grad_beta, float* grad_lambda,
                            void* grad_S_in, void* workspace, size_t ws_bytes,
                            fwmem_stream stream) {
  fwmem_status st = check_bwd(shape, mode);
  if (st != FWMEM_OK) return st;
  const Sizes z = sizes_of(shape);
  const size_t T = (size_t)shape->T;
  if (z.BH == 0) return FWMEM_OK;
  const bool needs_beta = mode->rule != FWMEM_RULE_ADDITIVE;
  if (T > 0 && needs_beta && beta == nullptr) return FWMEM_EINVAL;
  if (T > 0 && (q == nullptr || k == nullptr || v == nullptr || grad_out == nullptr ||
                grad_q == nullptr || grad_k == nullptr || grad_v == nullptr))
    return FWMEM_EINVAL;
  if (T == 0 && grad_S_in == nullptr) return FWMEM_OK;
  const size_t need = bwd_ws_bytes(shape, mode);
  if (ws_bytes < need || (need > 0 && workspace == nullptr)) return FWMEM_EWORKSPACE;
  const size_t es = esize(shape->dtype);
  if (!aligned(q, es) || !aligned(k, es) || !aligned(v, es) || !aligned(beta, 4) ||
      !aligned(lambda, 4) || !aligned(grad_out, 4) || !aligned(grad_q, 4) ||
      (mode->rule == FWMEM_RULE_DELTA_PV && !aligned(grad_beta, 16)) ||
      !aligned(grad_k, 4) || !aligned(grad_beta, 4) || !aligned(grad_lambda, 4) ||
      !aligned(grad_v, 16) || !aligned(S_in, 16) || !aligned(grad_S_out, 16) ||
      !aligned(grad_S_in, 16) || !aligned(workspace, 16))
    return FWMEM_EALIGN;
  if (z.BH * T > 0x7fffffffu || z.BH > 0x7fffffffu) return FWMEM_EUNSUPPORTED;
  const size_t nq = z.BH * T * shape->dk * es, nv = z.BH * T * shape->dv * es;
  const size_t ns = z.BH * T * 4, nsb = z.state_bytes;
  const size_t nl = ns * ((mode->flags & FWMEM_LAMBDA_PER_CHANNEL) ? (size_t)shape->dk : 1);
  const bool rule_pv = mode->rule == FWMEM_RULE_DELTA_PV;
  const size_t nb = ns * (rule_pv ? (size_t)shape->dv : 1);  // beta: per value channel
  const size_t ngq = z.BH * T * shape->dk * 4, ngv = z.BH * T * shape->dv * 4;
  const void* ins[] = {q, k, v, beta, lambda, S_in, grad_out, grad_S_out};
  const size_t nins[] = {nq, nq, nv, nb, nl, nsb, ngv, nsb};
  const void* outs[] = {grad_q, grad_k, grad_v, grad_beta, grad_lambda, grad_S_in, workspace};
  const size_t nouts[] = {ngq, ngq, ngv, nb, nl, nsb, need};
  for (int i = 0; i < 7; ++i) {
    for (int j = 0; j < 8; ++j)
      if (overlap(outs[i], nouts[i], ins[j], nins[j])) return FWMEM_EOVERLAP;
    for (int j = i + 1; j < 7; ++j)
      if (overlap(outs[i], nouts[i], outs[j], nouts[j])) return FWMEM_EOVERLAP;
  }

  const StatePtrs si = state_ptrs(S_in, z), gso = state_ptrs(grad_S_out, z),
                  gsi = state_ptrs(grad_S_in, z);
  fwmem::BwdParams p;
  std::memset(&p, 0, sizeof(p));
  p.q = q;
  p.k = k;
  p.v = v;
  p.beta = beta;
  p.lam = lambda;
  p.S_in = si.S;
  p.xprev_in = si.x;
  p.has_in = si.h;
  p.dout = grad_out;
  p.dS_out = gso.S;
  p.dz_out = (mode->flags & FWMEM_ZNORM) ? gso.x : nullptr;
  p.gq = grad_q;
  p.gk = grad_k;
  p.gv = grad_v;
  p.gbeta = grad_beta;
  p.glam = grad_lambda;
  p.gS0 = gsi.S;
  p.gx0 = gsi.x;
  p.gh0 = gsi.h;
  p.ws = static_cast<float*>(workspace);
  p.BH = (int)z.BH;
  p.T = (int)T;
  p.dk = shape->dk;
  p.dv = shape->dv;
  const int ck = fwmem::bwd_chunk((mode->flags & (FWMEM_LAMBDA_PER_CHANNEL | FWMEM_ZNORM)) != 0 || rule_pv);
  p.nchunks = (int)((T + ck - 1) / ck);
  p.rule = mode->rule;
  p.bf16 = shape->dtype == FWMEM_BF16 ? 1 : 0;
  p.flags = mode->flags;
  p.eps = mode->eps;
  const hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  const hipError_t e = fwmem::bwd_chunked(p.rule, p.flags, p.T) ? fwmem::launch_bwd_chunked(p, hs)
                                                                : fwmem::launch_bwd(p, hs);
  return e == hipSuccess ? FWMEM_OK : FWMEM_ELAUNCH;
}

}  // extern "C"
