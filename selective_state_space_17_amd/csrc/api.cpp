// C-ABI front end of libmssm: argument checks, planning, dispatch.
// Every check runs on the host before anything is enqueued.
#include "../../include/mssm.h"

#include <cmath>
#include <cstring>
#include <limits>

#include "internal.h"

namespace {

thread_local char g_err[256] = "";

void set_err(hipError_t e) {
  const char* s = hipGetErrorString(e);
  std::strncpy(g_err, s ? s : "unknown HIP error", sizeof(g_err) - 1);
  g_err[sizeof(g_err) - 1] = '\0';
}

constexpr int64_t kSimds = 256 * 4;   // MI355X: 256 CUs x 4 SIMDs

bool mul_ok(int64_t a, int64_t b, int64_t* r) {
  if (a < 0 || b < 0) return false;
  if (a != 0 && b > std::numeric_limits<int64_t>::max() / a) return false;
  *r = a * b;
  return true;
}

bool aligned(const void* p, size_t a) { return p == nullptr || (reinterpret_cast<uintptr_t>(p) % a) == 0; }

struct Range {
  uintptr_t lo, hi;
};
Range rng(const void* p, int64_t bytes) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  return {a, a + static_cast<uintptr_t>(bytes)};
}
bool overlap(const void* p, int64_t pb, const void* q, int64_t qb) {
  if (p == nullptr || q == nullptr || pb <= 0 || qb <= 0) return false;
  const Range a = rng(p, pb), b = rng(q, qb);
  return a.lo < b.hi && b.lo < a.hi;
}

// --------------------------------------------------------------------------
// Mamba-1 planning
// --------------------------------------------------------------------------
int states_per_lane(int G, int64_t N) {
  const int64_t need = (N + G - 1) / G;
  return need <= 4 ? 4 : (need <= 8 ? 8 : 16);
}

int ilog2(int v) {
  int r = 0;
  while ((1 << (r + 1)) <= v) ++r;
  return r;
}

// Estimated kernel time in VALU issue slots per lane (smaller is better).
double scan_cost(const mssm_scan_desc& d, int G, int K) {
  const int npl = states_per_lane(G, d.dstate);
  const int64_t cpb = 256 / G;                               // channels per 4-wave block
  const int64_t groups = d.batch * ((d.dim + cpb - 1) / cpb) * 4;   // waves per chunk
  // 6 slots per state update + per-step epilogue; with 16 lanes per channel and
  // dstate 16 (one state per lane) the readout sum is a 16-step LDS transpose
  // and the per-(t, c) staging is spread over 16 lanes: about 11 slots per step
  const double slots_step = (G == 16 && d.dstate == 16) ? 11.0 : npl * 6.0 + ilog2(G) + 14.0;
  const int64_t chunk = (d.seqlen + K - 1) / K;
  // pass 2 rescans until the carried-in state has decayed (about 800 steps for
  // softplus-distributed deltas and |A| >= 1); bounded by the chunk length
  const double steps = static_cast<double>(chunk) + (K > 1 ? std::min<double>(chunk, 800.0) : 0.0);
  const int64_t waves = groups * K;
  if (G == 1 && d.dstate == 16 && d.io_dtype == MSSM_BF16) {
    // the one-channel-per-lane kernel: workgroups of eight waves, one per CU, two waves on every SIMD of
    // it (2048 resident over the chip), and its rescan stops once the carried-in part is below the
    // states' rounding (about 250 steps for those deltas)
    const double lane_steps = static_cast<double>(chunk) + (K > 1 ? std::min<double>(chunk, 250.0) : 0.0);
    const int64_t rounds = (waves + 2 * kSimds - 1) / (2 * kSimds);
    return static_cast<double>(rounds) * lane_steps * slots_step * 2.0 / 0.93 + (K > 1 ? 2e4 : 0.0);
  }
  const int64_t per_simd = (waves + kSimds - 1) / kSimds;
  const double eff = per_simd <= 1 ? 0.85 : (per_simd == 2 ? 0.93 : 0.97);
  return steps * slots_step * static_cast<double>(per_simd) / eff + (K > 1 ? 2e4 : 0.0);
}

int validate_scan_desc(const mssm_scan_desc* d) {
  if (d == nullptr) return MSSM_ERR_INVALID_ARG;
  if (d->batch < 0 || d->seqlen < 0 || d->dim <= 0 || d->dstate <= 0) return MSSM_ERR_INVALID_ARG;
  if (d->flags != 0) return MSSM_ERR_INVALID_ARG;
  if (d->io_dtype != MSSM_F32 && d->io_dtype != MSSM_BF16) return MSSM_ERR_UNSUPPORTED;
  if (d->dstate > 256) return MSSM_ERR_UNSUPPORTED;
  if (d->split_seq < 0 || d->split_seq > 4096) return MSSM_ERR_INVALID_ARG;
  if (d->split_state != 0 && !mssm::scan_supported_G(d->split_state, d->dstate)) return MSSM_ERR_UNSUPPORTED;
  const int64_t es = d->io_dtype == MSSM_BF16 ? 2 : 4;
  int64_t t = 0;
  if (!mul_ok(d->batch, d->seqlen, &t) || !mul_ok(t, d->dim, &t) || !mul_ok(t, es, &t)) return MSSM_ERR_INVALID_ARG;
  if (!mul_ok(d->batch, d->seqlen, &t) || !mul_ok(t, d->dstate, &t) || !mul_ok(t, es, &t)) return MSSM_ERR_INVALID_ARG;
  if (!mul_ok(d->batch, d->dim, &t) || !mul_ok(t, d->dstate, &t) || !mul_ok(t, 4 * 4096, &t)) return MSSM_ERR_INVALID_ARG;
  return MSSM_OK;
}

// Whether the launches of a plan fit a 1-D grid, whose size in work-items is a 32-bit count:
// batch * K * channel-groups blocks of 256 threads (256 / G channels per block; the one-channel-per-lane
// kernel's 64-thread blocks of 64 channels come to no more), and with a split the carry's one wave per
// (b, c, n), four waves per block.
bool plan_fits(const mssm_scan_desc& d, int G, int K) {
  constexpr int64_t kMaxItems = std::numeric_limits<uint32_t>::max();
  const int64_t cpb = 256 / G;
  const int64_t groups = (d.dim + cpb - 1) / cpb;
  if (d.batch > kMaxItems / 256 / K || groups > kMaxItems / 256 / K / std::max<int64_t>(d.batch, 1)) return false;
  if (K > 1 && (d.batch * d.dim * d.dstate + 3) / 4 > kMaxItems / 256) return false;
  return true;
}

int plan_scan(const mssm_scan_desc& d, int* K_out, int* G_out) {
  int bestK = 1, bestG = 0;
  double best = std::numeric_limits<double>::infinity();
  const int Gs[] = {1, 2, 4, 8, 16};
  for (int G : Gs) {
    if (!mssm::scan_supported_G(G, d.dstate)) continue;
    if (d.split_state != 0 && G != d.split_state) continue;
    if (d.split_seq != 0) {
      const int K = static_cast<int>(std::min<int64_t>(d.split_seq, std::max<int64_t>(d.seqlen, 1)));
      const double c = scan_cost(d, G, K);
      if (c < best && plan_fits(d, G, K)) { best = c; bestK = K; bestG = G; }
      continue;
    }
    // powers of two, and the chunk count that fills the chip's resident waves exactly
    const int64_t cpb = 256 / G;
    const int64_t per_chunk = std::max<int64_t>(1, d.batch * ((d.dim + cpb - 1) / cpb) * 4);
    const int fill = static_cast<int>(std::max<int64_t>(1, std::min<int64_t>(4096, 2 * kSimds / per_chunk)));
    for (int K = 1; K <= 4096; K *= 2) {
      for (int Kc : {K, K == 1 ? fill : 0}) {
        if (Kc == 0 || (Kc > 1 && d.seqlen / Kc < 256)) continue;
        const double c = scan_cost(d, G, Kc);
        if (c < best && plan_fits(d, G, Kc)) { best = c; bestK = Kc; bestG = G; }
      }
      if (K > 1 && d.seqlen / K < 256) break;
    }
  }
  if (bestG == 0) return MSSM_ERR_UNSUPPORTED;
  *K_out = bestK;
  *G_out = bestG;
  return MSSM_OK;
}

}  // namespace

extern "C" {

int mssm_abi_version(void) { return MSSM_ABI_VERSION; }

const char* mssm_status_string(int status) {
  switch (status) {
    case MSSM_OK: return "ok";
    case MSSM_ERR_INVALID_ARG: return "invalid argument";
    case MSSM_ERR_UNSUPPORTED: return "unsupported problem";
    case MSSM_ERR_MISALIGNED: return "misaligned pointer";
    case MSSM_ERR_WORKSPACE: return "workspace missing or too small";
    case MSSM_ERR_HIP: return "HIP launch failed";
    default: return "unknown status";
  }
}

const char* mssm_last_error_detail(void) { return g_err; }

int mssm_selective_scan_plan(const mssm_scan_desc* desc, int32_t* split_seq, int32_t* split_state) {
  const int v = validate_scan_desc(desc);
  if (v != MSSM_OK) return v;
  if (split_seq == nullptr || split_state == nullptr) return MSSM_ERR_INVALID_ARG;
  int K = 1, G = 1;
  const int r = plan_scan(*desc, &K, &G);
  if (r != MSSM_OK) return r;
  *split_seq = K;
  *split_state = G;
  return MSSM_OK;
}

size_t mssm_selective_scan_workspace_size(const mssm_scan_desc* desc) {
  if (validate_scan_desc(desc) != MSSM_OK) return 0;
  int K = 1, G = 1;
  if (plan_scan(*desc, &K, &G) != MSSM_OK) return 0;
  return mssm::scan_workspace_bytes(desc->batch, desc->dim, desc->dstate, K);
}

}  // extern "C"

namespace {
// The forward behind both entry points.  use_scratch: the workspace is the device's fixed scratch,
// looked up after every argument check has passed (workspace/workspace_bytes are then ignored).
int scan_fwd_impl(const mssm_scan_desc* desc, const void* x, const void* delta, const float* A, const void* B,
                  const void* C, const float* D, const void* z, const float* h0, void* out, float* final_state,
                  void* workspace, size_t workspace_bytes, bool use_scratch, void* stream) {
  const int v = validate_scan_desc(desc);
  if (v != MSSM_OK) return v;
  const mssm_scan_desc& d = *desc;
  if (d.batch == 0) return MSSM_OK;
  const int64_t es = d.io_dtype == MSSM_BF16 ? 2 : 4;
  const int64_t n_bld = d.batch * d.seqlen * d.dim;
  const int64_t n_bln = d.batch * d.seqlen * d.dstate;
  const bool has_steps = n_bld > 0;
  if (A == nullptr) return MSSM_ERR_INVALID_ARG;
  if (has_steps && (x == nullptr || delta == nullptr || B == nullptr || C == nullptr || out == nullptr))
    return MSSM_ERR_INVALID_ARG;
  if (!aligned(x, es) || !aligned(delta, es) || !aligned(B, es) || !aligned(C, es) || !aligned(z, es) ||
      !aligned(out, es) || !aligned(A, 4) || !aligned(D, 4) || !aligned(h0, 4) || !aligned(final_state, 4))
    return MSSM_ERR_MISALIGNED;
  // outputs must not alias inputs or each other
  const int64_t b_io = n_bld * es, b_bc = n_bln * es;
  const int64_t b_st = d.batch * d.dim * d.dstate * 4;
  const void* ins[] = {x, delta, B, C, z, A, D, h0};
  const int64_t inb[] = {b_io, b_io, b_bc, b_bc, b_io, d.dim * d.dstate * 4, d.dim * 4, b_st};
  for (int i = 0; i < 8; ++i) {
    if (overlap(out, b_io, ins[i], inb[i])) return MSSM_ERR_INVALID_ARG;
    if (overlap(final_state, b_st, ins[i], inb[i])) return MSSM_ERR_INVALID_ARG;
  }
  if (overlap(out, b_io, final_state, b_st)) return MSSM_ERR_INVALID_ARG;

  int K = 1, G = 1;
  const int pr = plan_scan(d, &K, &G);
  if (pr != MSSM_OK) return pr;
  const size_t need = mssm::scan_workspace_bytes(d.batch, d.dim, d.dstate, K);
  if (use_scratch) {
    if (need > mssm::kScratchBytes) return MSSM_ERR_WORKSPACE;
    workspace = nullptr;
    if (need > 0) {
      const hipError_t e = mssm::scratch_address(static_cast<hipStream_t>(stream), &workspace);
      if (e != hipSuccess) {
        set_err(e);
        return MSSM_ERR_HIP;
      }
    }
  } else if (need > 0) {
    if (workspace == nullptr || workspace_bytes < need) return MSSM_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return MSSM_ERR_MISALIGNED;
    if (overlap(workspace, static_cast<int64_t>(need), out, b_io) ||
        overlap(workspace, static_cast<int64_t>(need), final_state, b_st))
      return MSSM_ERR_INVALID_ARG;
  }

  mssm::ScanArgs a{};
  a.x = x; a.delta = delta; a.A = A; a.B = B; a.C = C; a.D = D; a.z = z; a.h0 = h0;
  a.out = out; a.final_state = final_state; a.workspace = workspace;
  a.batch = d.batch; a.L = d.seqlen; a.dim = d.dim; a.N = d.dstate;
  a.io = d.io_dtype; a.K = K; a.G = G;
  const hipError_t e = mssm::scan_launch(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) {
    set_err(e);
    return MSSM_ERR_HIP;
  }
  return MSSM_OK;
}
}  // namespace

extern "C" {

int mssm_selective_scan_fwd(const mssm_scan_desc* desc, const void* x, const void* delta, const float* A,
                            const void* B, const void* C, const float* D, const void* z, const float* h0, void* out,
                            float* final_state, void* workspace, size_t workspace_bytes, void* stream) {
  return scan_fwd_impl(desc, x, delta, A, B, C, D, z, h0, out, final_state, workspace, workspace_bytes, false,
                       stream);
}

int mssm_selective_scan_fwd_noalloc(const mssm_scan_desc* desc, const void* x, const void* delta, const float* A,
                                    const void* B, const void* C, const float* D, const void* z, const float* h0,
                                    void* out, float* final_state, void* stream) {
  const int v = validate_scan_desc(desc);
  if (v != MSSM_OK) return v;
  mssm_scan_desc c = *desc;
  if (c.batch > 0 && c.split_seq == 0) {
    // the library's own plan, with fewer chunks (down to an unsplit scan, which needs no workspace)
    // where its workspace would not fit in the scratch; a forced split_seq is kept, and refused by
    // the forward below if it does not fit
    int K = 1, G = 1;
    const int pr = plan_scan(c, &K, &G);
    if (pr != MSSM_OK) return pr;
    if (mssm::scan_workspace_bytes(c.batch, c.dim, c.dstate, K) > mssm::kScratchBytes) {
      while (K > 1 && mssm::scan_workspace_bytes(c.batch, c.dim, c.dstate, K) > mssm::kScratchBytes) K /= 2;
      c.split_seq = K;
    }
  }
  return scan_fwd_impl(&c, x, delta, A, B, C, D, z, h0, out, final_state, nullptr, 0, true, stream);
}

// --------------------------------------------------------------------------
// Mamba-2 scalar-A multi-head form
// --------------------------------------------------------------------------
// *matrix: the shape and dtype the matrix-core block kernel takes (bf16 I/O, headdim a multiple of 8,
// dstate a multiple of 16 up to 256 -- above 128 with one input per channel --, rank 1, 2, 4, 8 or 16);
// any other valid problem runs through the recurrent update kernel.  R: inputs and outputs per channel (MIMO; 1 otherwise), 1..64.
constexpr int64_t kMaxRank = 64;
static int validate_ssd_desc(const mssm_ssd_desc* d, int64_t R, int64_t* Q, bool* matrix) {
  if (d == nullptr) return MSSM_ERR_INVALID_ARG;
  if (d->batch < 0 || d->seqlen < 0 || d->nheads <= 0 || d->headdim <= 0 || d->dstate <= 0 || d->ngroups <= 0)
    return MSSM_ERR_INVALID_ARG;
  if (d->flags != 0) return MSSM_ERR_INVALID_ARG;
  if (R < 1) return MSSM_ERR_INVALID_ARG;
  if (R > kMaxRank) return MSSM_ERR_UNSUPPORTED;
  if (d->io_dtype != MSSM_BF16 && d->io_dtype != MSSM_F32) return MSSM_ERR_UNSUPPORTED;
  if (d->nheads % d->ngroups != 0 || d->dstate > 256) return MSSM_ERR_UNSUPPORTED;
  const int64_t q = d->chunk == 0 ? 64 : d->chunk;
  if (q != 64 && q != 128 && q != 256) return MSSM_ERR_UNSUPPORTED;
  const int64_t es = d->io_dtype == MSSM_BF16 ? 2 : 4;
  int64_t t = 0;
  if (!mul_ok(d->batch, d->seqlen, &t) || !mul_ok(t, d->nheads, &t) || !mul_ok(t, R, &t) ||
      !mul_ok(t, d->headdim, &t) || !mul_ok(t, es, &t))
    return MSSM_ERR_INVALID_ARG;
  if (!mul_ok(d->batch, d->seqlen, &t) || !mul_ok(t, d->ngroups, &t) || !mul_ok(t, R, &t) ||
      !mul_ok(t, d->dstate, &t) || !mul_ok(t, es, &t))
    return MSSM_ERR_INVALID_ARG;
  if (!mul_ok(d->batch, d->nheads, &t) || !mul_ok(t, d->headdim, &t) || !mul_ok(t, d->dstate, &t) ||
      !mul_ok(t, 4, &t))
    return MSSM_ERR_INVALID_ARG;
  // the block kernel's grid: one workgroup per (batch, head, 64-wide headdim slice) at most
  // (more than 128 states: one input per channel only, as two shares of the states)
  *matrix = d->io_dtype == MSSM_BF16 && mssm::ssd_supported(d->headdim, d->dstate) && mssm::ssd_rank_supported(R) &&
            (d->dstate <= 128 || R == 1) &&
            d->batch * d->nheads * ((d->headdim + 63) / 64) <= std::numeric_limits<int32_t>::max();
  *Q = q;
  return MSSM_OK;
}

// --------------------------------------------------------------------------
// Token-by-token state update
// --------------------------------------------------------------------------
int mssm_selective_state_update(const mssm_scan_desc* desc, float* state, const void* x, const void* delta,
                                const float* A, const void* B, const void* C, const float* D, const void* z,
                                void* out, void* stream) {
  const int v = validate_scan_desc(desc);
  if (v != MSSM_OK) return v;
  const mssm_scan_desc& d = *desc;
  if (d.batch == 0 || d.seqlen == 0) return MSSM_OK;
  const int64_t es = d.io_dtype == MSSM_BF16 ? 2 : 4;
  if (state == nullptr || A == nullptr || x == nullptr || delta == nullptr || B == nullptr || C == nullptr ||
      out == nullptr)
    return MSSM_ERR_INVALID_ARG;
  if (!aligned(x, es) || !aligned(delta, es) || !aligned(B, es) || !aligned(C, es) || !aligned(z, es) ||
      !aligned(out, es) || !aligned(A, 4) || !aligned(D, 4) || !aligned(state, 4))
    return MSSM_ERR_MISALIGNED;
  const int64_t b_io = d.batch * d.seqlen * d.dim * es, b_bc = d.batch * d.seqlen * d.dstate * es;
  const int64_t b_st = d.batch * d.dim * d.dstate * 4;
  const void* ins[] = {x, delta, B, C, z, A, D};
  const int64_t inb[] = {b_io, b_io, b_bc, b_bc, b_io, d.dim * d.dstate * 4, d.dim * 4};
  for (int i = 0; i < 7; ++i) {
    if (overlap(out, b_io, ins[i], inb[i])) return MSSM_ERR_INVALID_ARG;
    if (overlap(state, b_st, ins[i], inb[i])) return MSSM_ERR_INVALID_ARG;
  }
  if (overlap(out, b_io, state, b_st)) return MSSM_ERR_INVALID_ARG;
  if (mssm::update_grid_blocks(d.batch * d.dim, d.dstate) > std::numeric_limits<int32_t>::max())
    return MSSM_ERR_UNSUPPORTED;
  mssm::UpdateArgs a{};
  a.state = state; a.x = x; a.delta = delta; a.A = A; a.B = B; a.C = C; a.D = D; a.z = z; a.out = out;
  a.batch = d.batch; a.L = d.seqlen; a.N = d.dstate; a.dim = d.dim; a.io = d.io_dtype;
  const hipError_t e = mssm::scan_update_launch(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) {
    set_err(e);
    return MSSM_ERR_HIP;
  }
  return MSSM_OK;
}

int mssm_selective_state_update_conv(const mssm_scan_desc* desc, int32_t conv_width, float* state, void* conv_state,
                                     const void* xin, const float* conv_w, const float* conv_b, const void* delta,
                                     const float* A, const void* B, const void* C, const float* D, const void* z,
                                     void* out, void* stream) {
  const int v = validate_scan_desc(desc);
  if (v != MSSM_OK) return v;
  const mssm_scan_desc& d = *desc;
  if (conv_width < 1 || conv_width > 4) return MSSM_ERR_UNSUPPORTED;
  if (d.batch == 0 || d.seqlen == 0) return MSSM_OK;
  const int64_t es = d.io_dtype == MSSM_BF16 ? 2 : 4;
  if (state == nullptr || A == nullptr || xin == nullptr || delta == nullptr || B == nullptr || C == nullptr ||
      out == nullptr || conv_w == nullptr || (conv_width > 1 && conv_state == nullptr))
    return MSSM_ERR_INVALID_ARG;
  if (!aligned(xin, es) || !aligned(delta, es) || !aligned(B, es) || !aligned(C, es) || !aligned(z, es) ||
      !aligned(out, es) || !aligned(conv_state, es) || !aligned(A, 4) || !aligned(D, 4) || !aligned(state, 4) ||
      !aligned(conv_w, 4) || !aligned(conv_b, 4))
    return MSSM_ERR_MISALIGNED;
  const int64_t b_io = d.batch * d.seqlen * d.dim * es, b_bc = d.batch * d.seqlen * d.dstate * es;
  const int64_t b_st = d.batch * d.dim * d.dstate * 4;
  const int64_t b_cs = conv_width > 1 ? d.batch * (conv_width - 1) * d.dim * es : 0;
  const void* ins[] = {xin, delta, B, C, z, A, D, conv_w, conv_b};
  const int64_t inb[] = {b_io, b_io, b_bc, b_bc, b_io, d.dim * d.dstate * 4, d.dim * 4, d.dim * conv_width * 4,
                         d.dim * 4};
  for (int i = 0; i < 9; ++i) {
    if (overlap(out, b_io, ins[i], inb[i])) return MSSM_ERR_INVALID_ARG;
    if (overlap(state, b_st, ins[i], inb[i])) return MSSM_ERR_INVALID_ARG;
    if (overlap(conv_state, b_cs, ins[i], inb[i])) return MSSM_ERR_INVALID_ARG;
  }
  if (overlap(out, b_io, state, b_st) || overlap(out, b_io, conv_state, b_cs) || overlap(state, b_st, conv_state, b_cs))
    return MSSM_ERR_INVALID_ARG;
  if (mssm::update_grid_blocks(d.batch * d.dim, d.dstate) > std::numeric_limits<int32_t>::max())
    return MSSM_ERR_UNSUPPORTED;
  mssm::UpdateArgs a{};
  a.state = state; a.x = xin; a.delta = delta; a.A = A; a.B = B; a.C = C; a.D = D; a.z = z; a.out = out;
  a.batch = d.batch; a.L = d.seqlen; a.N = d.dstate; a.dim = d.dim; a.io = d.io_dtype;
  a.conv_w = conv_w; a.conv_b = conv_b; a.conv_state = conv_width > 1 ? conv_state : nullptr; a.conv_width = conv_width;
  const hipError_t e = mssm::scan_update_launch(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) {
    set_err(e);
    return MSSM_ERR_HIP;
  }
  return MSSM_OK;
}

}  // extern "C"

namespace {
// every multi-head decode rule: lam == nullptr (want_lam false) is the Mamba-2 rule; R > 1 is MIMO
int ssd_update_impl(const mssm_ssd_desc* desc, int64_t R, float* state, const void* x_prev, const void* B_prev,
                    const void* x, const void* delta, const void* lam, bool want_lam, const float* A,
                    const float* omega, bool want_omega, const void* B, const void* C, const float* D,
                    const void* z, void* out, void* stream) {
  const mssm_ssd_desc* d = desc;
  if (d == nullptr) return MSSM_ERR_INVALID_ARG;
  if (d->batch < 0 || d->seqlen < 0 || d->nheads <= 0 || d->headdim <= 0 || d->dstate <= 0 || d->ngroups <= 0)
    return MSSM_ERR_INVALID_ARG;
  if (d->flags != 0) return MSSM_ERR_INVALID_ARG;
  if (R < 1) return MSSM_ERR_INVALID_ARG;
  if (R > kMaxRank) return MSSM_ERR_UNSUPPORTED;
  if (d->io_dtype != MSSM_BF16 && d->io_dtype != MSSM_F32) return MSSM_ERR_UNSUPPORTED;
  if (d->nheads % d->ngroups != 0 || d->dstate > 256) return MSSM_ERR_UNSUPPORTED;
  if (want_omega && d->dstate % 2 != 0) return MSSM_ERR_UNSUPPORTED;   // complex state: whole pairs
  const int64_t es = d->io_dtype == MSSM_BF16 ? 2 : 4;
  int64_t n_x = 0, n_bc = 0, n_st = 0, n_d = 0, t = 0;
  if (!mul_ok(d->batch, d->seqlen, &t) || !mul_ok(t, d->nheads, &n_d) || !mul_ok(n_d, R, &t) ||
      !mul_ok(t, d->headdim, &n_x) || !mul_ok(n_x, es, &t))
    return MSSM_ERR_INVALID_ARG;
  if (!mul_ok(d->batch, d->seqlen, &t) || !mul_ok(t, d->ngroups, &t) || !mul_ok(t, R, &t) ||
      !mul_ok(t, d->dstate, &n_bc) || !mul_ok(n_bc, es, &t))
    return MSSM_ERR_INVALID_ARG;
  if (!mul_ok(d->batch, d->nheads, &t) || !mul_ok(t, d->headdim, &t) || !mul_ok(t, d->dstate, &n_st) ||
      !mul_ok(n_st, 4 * 64, &t))
    return MSSM_ERR_INVALID_ARG;
  if (d->batch == 0 || d->seqlen == 0) return MSSM_OK;
  if (state == nullptr || A == nullptr || x == nullptr || delta == nullptr || B == nullptr || C == nullptr ||
      out == nullptr)
    return MSSM_ERR_INVALID_ARG;
  if (want_lam && lam == nullptr) return MSSM_ERR_INVALID_ARG;
  if (want_omega && omega == nullptr) return MSSM_ERR_INVALID_ARG;
  if (!aligned(x, es) || !aligned(delta, es) || !aligned(B, es) || !aligned(C, es) || !aligned(z, es) ||
      !aligned(out, es) || !aligned(A, 4) || !aligned(D, 4) || !aligned(state, 4) || !aligned(lam, es) ||
      !aligned(x_prev, es) || !aligned(B_prev, es) || !aligned(omega, 4))
    return MSSM_ERR_MISALIGNED;
  const int64_t b_io = n_x * es, b_st = n_st * 4;
  const int64_t b_xp = d->batch * d->nheads * R * d->headdim * es, b_bp = d->batch * d->ngroups * R * d->dstate * es;
  const void* ins[] = {x, delta, B, C, z, A, D, lam, x_prev, B_prev, omega};
  const int64_t inb[] = {b_io, n_d * es, n_bc * es, n_bc * es, b_io, d->nheads * 4, d->nheads * 4, n_d * es,
                         b_xp, b_bp, d->nheads * (d->dstate / 2) * 4};
  for (int i = 0; i < 11; ++i) {
    if (overlap(out, b_io, ins[i], inb[i])) return MSSM_ERR_INVALID_ARG;
    if (overlap(state, b_st, ins[i], inb[i])) return MSSM_ERR_INVALID_ARG;
  }
  if (overlap(out, b_io, state, b_st)) return MSSM_ERR_INVALID_ARG;
  if (mssm::update_grid_blocks(d->batch * d->nheads * d->headdim, d->dstate) > std::numeric_limits<int32_t>::max())
    return MSSM_ERR_UNSUPPORTED;
  mssm::UpdateArgs a{};
  a.state = state; a.x = x; a.delta = delta; a.A = A; a.B = B; a.C = C; a.D = D; a.z = z; a.out = out;
  a.batch = d->batch; a.L = d->seqlen; a.N = d->dstate;
  a.H = d->nheads; a.P = d->headdim; a.G = d->ngroups; a.io = d->io_dtype; a.rank = R;
  if (want_lam) {
    a.lam = lam; a.x_prev = x_prev; a.B_prev = B_prev;
    if (want_omega) a.omega = omega;
  }
  const hipError_t e = mssm::ssd_update_launch(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) {
    set_err(e);
    return MSSM_ERR_HIP;
  }
  return MSSM_OK;
}
}  // namespace

extern "C" {

int mssm_ssd_state_update(const mssm_ssd_desc* desc, float* state, const void* x, const void* delta,
                          const float* A, const void* B, const void* C, const float* D, const void* z, void* out,
                          void* stream) {
  return ssd_update_impl(desc, 1, state, nullptr, nullptr, x, delta, nullptr, false, A, nullptr, false, B, C, D, z,
                         out, stream);
}

int mssm_ssd_trapezoidal_state_update(const mssm_ssd_desc* desc, float* state, const void* x_prev,
                                      const void* B_prev, const void* x, const void* delta, const void* lam,
                                      const float* A, const void* B, const void* C, const float* D, const void* z,
                                      void* out, void* stream) {
  return ssd_update_impl(desc, 1, state, x_prev, B_prev, x, delta, lam, true, A, nullptr, false, B, C, D, z, out,
                         stream);
}

int mssm_mamba3_siso_update(const mssm_ssd_desc* desc, float* state, const void* x_prev, const void* B_prev,
                            const void* x, const void* delta, const void* lam, const float* A, const float* omega,
                            const void* B, const void* C, const float* D, const void* z, void* out, void* stream) {
  return ssd_update_impl(desc, 1, state, x_prev, B_prev, x, delta, lam, true, A, omega, true, B, C, D, z, out,
                         stream);
}

int mssm_ssd_mimo_state_update(const mssm_ssd_desc* desc, int32_t rank, float* state, const void* x_prev,
                               const void* B_prev, const void* x, const void* delta, const void* lam,
                               const float* A, const void* B, const void* C, const float* D, const void* z,
                               void* out, void* stream) {
  return ssd_update_impl(desc, rank, state, x_prev, B_prev, x, delta, lam, lam != nullptr, A, nullptr, false, B, C,
                         D, z, out, stream);
}

// --------------------------------------------------------------------------
// Training-mode forward: also stores the state entering every 16-step tile
// --------------------------------------------------------------------------
size_t mssm_selective_scan_checkpoint_size(const mssm_scan_desc* desc) {
  if (validate_scan_desc(desc) != MSSM_OK || desc->dstate != 16) return 0;
  return mssm::scan_checkpoint_bytes(desc->batch, desc->seqlen, desc->dim);
}

int mssm_selective_scan_fwd_ckpt(const mssm_scan_desc* desc, const void* x, const void* delta, const float* A,
                                 const void* B, const void* C, const float* D, const void* z, const float* h0,
                                 void* out, float* final_state, float* checkpoints, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  const int v = validate_scan_desc(desc);
  if (v != MSSM_OK) return v;
  const mssm_scan_desc& d = *desc;
  if (d.dstate != 16 || (d.split_state != 0 && d.split_state != 16)) return MSSM_ERR_UNSUPPORTED;
  const int64_t es = d.io_dtype == MSSM_BF16 ? 2 : 4;
  if ((d.dim * es) % 16 != 0) return MSSM_ERR_UNSUPPORTED;
  if (A == nullptr) return MSSM_ERR_INVALID_ARG;
  if (d.batch == 0) return MSSM_OK;
  const int64_t n_bld = d.batch * d.seqlen * d.dim;
  const int64_t n_bln = d.batch * d.seqlen * d.dstate;
  if (n_bld > 0 && (x == nullptr || delta == nullptr || B == nullptr || C == nullptr || out == nullptr ||
                    checkpoints == nullptr))
    return MSSM_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(delta, 16) || !aligned(B, 16) || !aligned(C, 16) || !aligned(z, 16) ||
      !aligned(out, 16) || !aligned(A, 4) || !aligned(D, 4) || !aligned(h0, 4) || !aligned(final_state, 4) ||
      !aligned(checkpoints, 4))
    return MSSM_ERR_MISALIGNED;
  const int64_t b_io = n_bld * es, b_bc = n_bln * es;
  const int64_t b_st = d.batch * d.dim * d.dstate * 4;
  const int64_t b_ck = static_cast<int64_t>(mssm::scan_checkpoint_bytes(d.batch, d.seqlen, d.dim));
  const void* ins[] = {x, delta, B, C, z, A, D, h0};
  const int64_t inb[] = {b_io, b_io, b_bc, b_bc, b_io, d.dim * d.dstate * 4, d.dim * 4, b_st};
  for (int i = 0; i < 8; ++i) {
    if (overlap(out, b_io, ins[i], inb[i])) return MSSM_ERR_INVALID_ARG;
    if (overlap(final_state, b_st, ins[i], inb[i])) return MSSM_ERR_INVALID_ARG;
    if (overlap(checkpoints, b_ck, ins[i], inb[i])) return MSSM_ERR_INVALID_ARG;
  }
  if (overlap(out, b_io, final_state, b_st) || overlap(out, b_io, checkpoints, b_ck) ||
      overlap(final_state, b_st, checkpoints, b_ck))
    return MSSM_ERR_INVALID_ARG;

  mssm_scan_desc c = d;
  c.split_state = 16;
  int K = 1, G = 16;
  const int pr = plan_scan(c, &K, &G);
  if (pr != MSSM_OK) return pr;
  const size_t need = mssm::scan_workspace_bytes(d.batch, d.dim, d.dstate, K);
  if (need > 0) {
    if (workspace == nullptr || workspace_bytes < need) return MSSM_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return MSSM_ERR_MISALIGNED;
    if (overlap(workspace, static_cast<int64_t>(need), out, b_io) ||
        overlap(workspace, static_cast<int64_t>(need), final_state, b_st) ||
        overlap(workspace, static_cast<int64_t>(need), checkpoints, b_ck))
      return MSSM_ERR_INVALID_ARG;
  }
  if (n_bld == 0 && final_state == nullptr) return MSSM_OK;

  mssm::ScanArgs a{};
  a.x = x; a.delta = delta; a.A = A; a.B = B; a.C = C; a.D = D; a.z = z; a.h0 = h0;
  a.out = out; a.final_state = final_state; a.workspace = workspace; a.ckpt = checkpoints;
  a.batch = d.batch; a.L = d.seqlen; a.dim = d.dim; a.N = d.dstate;
  a.io = d.io_dtype; a.K = K; a.G = G;
  const hipError_t e = mssm::scan_launch(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) {
    set_err(e);
    return MSSM_ERR_HIP;
  }
  return MSSM_OK;
}

size_t mssm_selective_scan_fwd_ckpt_workspace_size(const mssm_scan_desc* desc) {
  if (validate_scan_desc(desc) != MSSM_OK || desc->dstate != 16) return 0;
  if (desc->split_state != 0 && desc->split_state != 16) return 0;
  mssm_scan_desc c = *desc;
  c.split_state = 16;
  int K = 1, G = 16;
  if (plan_scan(c, &K, &G) != MSSM_OK) return 0;
  return mssm::scan_workspace_bytes(c.batch, c.dim, c.dstate, K);
}

// --------------------------------------------------------------------------
// Short causal convolution + SiLU fused in front of the scan
// --------------------------------------------------------------------------
namespace {
// the convolution front end runs in the one-state-per-lane kernel: 16 lanes per channel
mssm_scan_desc conv_plan_desc(const mssm_scan_desc& d) {
  mssm_scan_desc c = d;
  c.split_state = 16;
  return c;
}
}  // namespace

size_t mssm_selective_scan_conv_workspace_size(const mssm_scan_desc* desc) {
  if (validate_scan_desc(desc) != MSSM_OK || desc->dstate != 16) return 0;
  if (desc->split_state != 0 && desc->split_state != 16) return 0;
  const mssm_scan_desc c = conv_plan_desc(*desc);
  int K = 1, G = 16;
  if (plan_scan(c, &K, &G) != MSSM_OK) return 0;
  return mssm::scan_workspace_bytes(c.batch, c.dim, c.dstate, K);
}

// The convolution and scan over a whole sequence through the recurrent update kernel, for the problems the
// fused block kernel does not take: the window starts from conv_init (or zero inputs) and is not written
// back, the state starts from h0 (or zero) and goes to final_state (if given).
static int conv_fwd_recurrent(const mssm_scan_desc& d, int32_t conv_width, const void* xin, const float* conv_w,
                              const float* conv_b, const void* conv_init, const void* delta, const float* A,
                              const void* B, const void* C, const float* D, const void* z, const float* h0,
                              void* out, float* final_state, void* stream) {
  const int64_t es = d.io_dtype == MSSM_BF16 ? 2 : 4;
  const int64_t n_bld = d.batch * d.seqlen * d.dim;
  const int64_t n_bln = d.batch * d.seqlen * d.dstate;
  if (n_bld > 0 && (xin == nullptr || delta == nullptr || B == nullptr || C == nullptr || out == nullptr))
    return MSSM_ERR_INVALID_ARG;
  if (!aligned(xin, es) || !aligned(delta, es) || !aligned(B, es) || !aligned(C, es) || !aligned(z, es) ||
      !aligned(out, es) || !aligned(conv_init, es) || !aligned(A, 4) || !aligned(D, 4) || !aligned(h0, 4) ||
      !aligned(final_state, 4) || !aligned(conv_w, 4) || !aligned(conv_b, 4))
    return MSSM_ERR_MISALIGNED;
  const int64_t b_io = n_bld * es, b_bc = n_bln * es;
  const int64_t b_st = d.batch * d.dim * d.dstate * 4;
  const int64_t b_init = d.batch * (conv_width - 1) * d.dim * es;
  const void* ins[] = {xin, delta, B, C, z, A, D, h0, conv_w, conv_b, conv_init};
  const int64_t inb[] = {b_io, b_io, b_bc, b_bc, b_io, d.dim * d.dstate * 4, d.dim * 4, b_st,
                         d.dim * conv_width * 4, d.dim * 4, b_init};
  for (int i = 0; i < 11; ++i) {
    if (overlap(out, b_io, ins[i], inb[i])) return MSSM_ERR_INVALID_ARG;
    if (overlap(final_state, b_st, ins[i], inb[i])) return MSSM_ERR_INVALID_ARG;
  }
  if (overlap(out, b_io, final_state, b_st)) return MSSM_ERR_INVALID_ARG;
  if (n_bld == 0 && final_state == nullptr) return MSSM_OK;
  if (mssm::update_grid_blocks(d.batch * d.dim, d.dstate) > std::numeric_limits<int32_t>::max())
    return MSSM_ERR_UNSUPPORTED;
  mssm::UpdateArgs a{};
  a.state = nullptr; a.state_in = h0; a.state_out = final_state;
  a.x = xin; a.delta = delta; a.A = A; a.B = B; a.C = C; a.D = D; a.z = z; a.out = out;
  a.conv_w = conv_w; a.conv_b = conv_b; a.conv_width = conv_width;
  a.conv_state = nullptr; a.conv_in = conv_init; a.conv_out = nullptr;
  a.batch = d.batch; a.L = d.seqlen; a.N = d.dstate; a.dim = d.dim; a.io = d.io_dtype;
  const hipError_t e = mssm::scan_update_launch(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) {
    set_err(e);
    return MSSM_ERR_HIP;
  }
  return MSSM_OK;
}

int mssm_selective_scan_conv_fwd(const mssm_scan_desc* desc, int32_t conv_width, const void* xin,
                                 const float* conv_w, const float* conv_b, const void* conv_init,
                                 const void* delta, const float* A, const void* B, const void* C, const float* D,
                                 const void* z, const float* h0, void* out, float* final_state, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  const int v = validate_scan_desc(desc);
  if (v != MSSM_OK) return v;
  const mssm_scan_desc& d = *desc;
  if (conv_width < 1 || conv_width > 4) return MSSM_ERR_UNSUPPORTED;
  const int64_t es = d.io_dtype == MSSM_BF16 ? 2 : 4;
  if (A == nullptr || conv_w == nullptr) return MSSM_ERR_INVALID_ARG;
  if (d.batch == 0) return MSSM_OK;
  // the fused block kernel: one state per lane (dstate 16) and 16-byte pieces of every io tensor
  const bool fused = d.dstate == 16 && (d.split_state == 0 || d.split_state == 16) && (d.dim * es) % 16 == 0 &&
                     aligned(xin, 16) && aligned(delta, 16) && aligned(B, 16) && aligned(C, 16) && aligned(z, 16) &&
                     aligned(out, 16) && aligned(conv_init, 16);
  if (!fused)
    return conv_fwd_recurrent(d, conv_width, xin, conv_w, conv_b, conv_init, delta, A, B, C, D, z, h0, out,
                              final_state, stream);
  const int64_t n_bld = d.batch * d.seqlen * d.dim;
  const int64_t n_bln = d.batch * d.seqlen * d.dstate;
  if (n_bld > 0 && (xin == nullptr || delta == nullptr || B == nullptr || C == nullptr || out == nullptr))
    return MSSM_ERR_INVALID_ARG;
  // the fused kernel moves 16-byte pieces of every io tensor
  if (!aligned(xin, 16) || !aligned(delta, 16) || !aligned(B, 16) || !aligned(C, 16) || !aligned(z, 16) ||
      !aligned(out, 16) || !aligned(conv_init, 16) || !aligned(A, 4) || !aligned(D, 4) || !aligned(h0, 4) ||
      !aligned(final_state, 4) || !aligned(conv_w, 4) || !aligned(conv_b, 4))
    return MSSM_ERR_MISALIGNED;
  const int64_t b_io = n_bld * es, b_bc = n_bln * es;
  const int64_t b_st = d.batch * d.dim * d.dstate * 4;
  const int64_t b_init = d.batch * (conv_width - 1) * d.dim * es;
  const void* ins[] = {xin, delta, B, C, z, A, D, h0, conv_w, conv_b, conv_init};
  const int64_t inb[] = {b_io, b_io, b_bc, b_bc, b_io, d.dim * d.dstate * 4, d.dim * 4, b_st,
                         d.dim * conv_width * 4, d.dim * 4, b_init};
  for (int i = 0; i < 11; ++i) {
    if (overlap(out, b_io, ins[i], inb[i])) return MSSM_ERR_INVALID_ARG;
    if (overlap(final_state, b_st, ins[i], inb[i])) return MSSM_ERR_INVALID_ARG;
  }
  if (overlap(out, b_io, final_state, b_st)) return MSSM_ERR_INVALID_ARG;

  const mssm_scan_desc c = conv_plan_desc(d);
  int K = 1, G = 16;
  const int pr = plan_scan(c, &K, &G);
  if (pr != MSSM_OK) return pr;
  const size_t need = mssm::scan_workspace_bytes(d.batch, d.dim, d.dstate, K);
  if (need > 0) {
    if (workspace == nullptr || workspace_bytes < need) return MSSM_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return MSSM_ERR_MISALIGNED;
    if (overlap(workspace, static_cast<int64_t>(need), out, b_io) ||
        overlap(workspace, static_cast<int64_t>(need), final_state, b_st))
      return MSSM_ERR_INVALID_ARG;
  }
  if (n_bld == 0 && final_state == nullptr) return MSSM_OK;

  mssm::ScanArgs a{};
  a.x = xin; a.delta = delta; a.A = A; a.B = B; a.C = C; a.D = D; a.z = z; a.h0 = h0;
  a.out = out; a.final_state = final_state; a.workspace = workspace;
  a.batch = d.batch; a.L = d.seqlen; a.dim = d.dim; a.N = d.dstate;
  a.io = d.io_dtype; a.K = K; a.G = G;
  a.conv_w = conv_w; a.conv_b = conv_b; a.conv_init = conv_init; a.conv_width = conv_width;
  const hipError_t e = mssm::scan_launch(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) {
    set_err(e);
    return MSSM_ERR_HIP;
  }
  return MSSM_OK;
}

// --------------------------------------------------------------------------
// Gradients of the Mamba-1 selective scan
// --------------------------------------------------------------------------
size_t mssm_selective_scan_bwd_workspace_size(const mssm_scan_desc* desc) {
  if (validate_scan_desc(desc) != MSSM_OK) return 0;
  return mssm::scan_bwd_workspace_bytes(desc->batch, desc->seqlen, desc->dim, desc->dstate);
}

int mssm_selective_scan_bwd(const mssm_scan_desc* desc, const void* x, const void* delta, const float* A,
                            const void* B, const void* C, const float* D, const void* z, const float* h0,
                            const void* dout, const float* dfinal, void* dx, void* ddelta, float* dA, float* dB,
                            float* dC, float* dD, void* dz, float* dh0, const float* checkpoints, void* workspace,
                            size_t workspace_bytes, void* stream) {
  const int v = validate_scan_desc(desc);
  if (v != MSSM_OK) return v;
  const mssm_scan_desc& d = *desc;
  const int64_t es = d.io_dtype == MSSM_BF16 ? 2 : 4;
  const int64_t n_bld = d.batch * d.seqlen * d.dim;
  const bool has_steps = n_bld > 0;
  if (A == nullptr || dA == nullptr) return MSSM_ERR_INVALID_ARG;
  if (D != nullptr && dD == nullptr) return MSSM_ERR_INVALID_ARG;
  if (has_steps && (x == nullptr || delta == nullptr || B == nullptr || C == nullptr || dout == nullptr ||
                    dx == nullptr || ddelta == nullptr || dB == nullptr || dC == nullptr ||
                    (z != nullptr && dz == nullptr)))
    return MSSM_ERR_INVALID_ARG;
  if (!aligned(x, es) || !aligned(delta, es) || !aligned(B, es) || !aligned(C, es) || !aligned(z, es) ||
      !aligned(dout, es) || !aligned(dx, es) || !aligned(ddelta, es) || !aligned(dz, es) || !aligned(A, 4) ||
      !aligned(D, 4) || !aligned(h0, 4) || !aligned(dfinal, 4) || !aligned(dA, 4) || !aligned(dB, 4) ||
      !aligned(dC, 4) || !aligned(dD, 4) || !aligned(dh0, 4) || !aligned(checkpoints, 4))
    return MSSM_ERR_MISALIGNED;
  if (checkpoints != nullptr && d.dstate != 16) return MSSM_ERR_UNSUPPORTED;   // written by the dstate-16 forward
  // launch grids count their work-items in 32 bits: the gradient kernel's blocks of 256 threads, the dB/dC
  // sums over (b, t, 4 states), and with more than 16 states the element-wise finish over (b, t, c)
  constexpr int64_t kMaxItems = std::numeric_limits<uint32_t>::max();
  if ((d.seqlen + 15) / 16 > std::numeric_limits<int32_t>::max() ||
      mssm::scan_bwd_grid_blocks(d.batch, d.dim, d.dstate) > kMaxItems / 256 ||
      d.batch * d.seqlen * ((d.dstate + 15) / 16 * 4) > kMaxItems - 255 ||
      (d.dstate > 16 && n_bld > kMaxItems - 255))
    return MSSM_ERR_UNSUPPORTED;
  const size_t need = mssm::scan_bwd_workspace_bytes(d.batch, d.seqlen, d.dim, d.dstate);
  if (need > 0) {
    if (workspace == nullptr || workspace_bytes < need) return MSSM_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return MSSM_ERR_MISALIGNED;
  }
  // outputs (and the workspace) must not alias the inputs or each other
  const int64_t b_io = n_bld * es, b_bc = d.batch * d.seqlen * d.dstate * es;
  const int64_t b_bc32 = d.batch * d.seqlen * d.dstate * 4, b_st = d.batch * d.dim * d.dstate * 4;
  const int64_t b_a = d.dim * d.dstate * 4, b_d = d.dim * 4;
  const bool with_z = z != nullptr, with_d = D != nullptr;
  const int64_t b_ck = static_cast<int64_t>(mssm::scan_checkpoint_bytes(d.batch, d.seqlen, d.dim));
  const void* ins[] = {x, delta, B, C, z, A, D, h0, dout, dfinal, checkpoints};
  const int64_t inb[] = {b_io, b_io, b_bc, b_bc, b_io, b_a, b_d, b_st, b_io, b_st, b_ck};
  const void* outs[] = {dx, ddelta, dA, dB, dC, with_d ? dD : nullptr, with_z ? dz : nullptr, dh0, workspace};
  const int64_t outb[] = {b_io, b_io, b_a, b_bc32, b_bc32, b_d, b_io, b_st, static_cast<int64_t>(need)};
  for (int i = 0; i < 9; ++i) {
    for (int j = 0; j < 11; ++j)
      if (overlap(outs[i], outb[i], ins[j], inb[j])) return MSSM_ERR_INVALID_ARG;
    for (int j = i + 1; j < 9; ++j)
      if (overlap(outs[i], outb[i], outs[j], outb[j])) return MSSM_ERR_INVALID_ARG;
  }

  mssm::ScanBwdArgs a{};
  a.x = x; a.delta = delta; a.A = A; a.B = B; a.C = C; a.D = D; a.z = z; a.h0 = h0;
  a.dout = dout; a.dfinal = dfinal;
  a.dx = dx; a.ddelta = ddelta; a.dA = dA; a.dB = dB; a.dC = dC; a.dD = with_d ? dD : nullptr;
  a.dz = with_z ? dz : nullptr; a.dh0 = dh0; a.ckpt_in = checkpoints; a.workspace = workspace;
  a.batch = d.batch; a.L = d.seqlen; a.dim = d.dim; a.N = d.dstate; a.io = d.io_dtype;
  const hipError_t e = mssm::scan_bwd_launch(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) {
    set_err(e);
    return MSSM_ERR_HIP;
  }
  return MSSM_OK;
}

int mssm_ssd_plan(const mssm_ssd_desc* desc, int32_t* route) { return mssm_ssd_mimo_plan(desc, 1, route); }

int mssm_ssd_mimo_plan(const mssm_ssd_desc* desc, int32_t rank, int32_t* route) {
  int64_t Q = 0;
  bool matrix = false;
  const int v = validate_ssd_desc(desc, rank, &Q, &matrix);
  if (v != MSSM_OK) return v;
  if (route == nullptr) return MSSM_ERR_INVALID_ARG;
  *route = matrix ? MSSM_SSD_ROUTE_BLOCK : MSSM_SSD_ROUTE_RECURRENT;
  return MSSM_OK;
}

size_t mssm_ssd_workspace_size(const mssm_ssd_desc* desc) {
  int64_t Q = 0;
  bool matrix = false;
  if (validate_ssd_desc(desc, 1, &Q, &matrix) != MSSM_OK || !matrix) return 0;
  return mssm::ssd_workspace_bytes(desc->batch, desc->seqlen, desc->nheads, desc->headdim, desc->dstate,
                                   desc->ngroups, Q);
}

}  // extern "C"

namespace {
// A whole sequence through the recurrent update kernel, for the problems the block kernel does not take:
// the state starts from h0 (or zero) and is written to final_state (if given); no previous token.
int ssd_fwd_recurrent(const mssm_ssd_desc& d, int64_t R, const void* x, const void* delta, const void* lam,
                      bool want_lam, const float* A, const void* B, const void* C, const float* D, const void* z,
                      const float* h0, void* out, float* final_state, void* stream) {
  const int64_t es = d.io_dtype == MSSM_BF16 ? 2 : 4;
  const int64_t n_d = d.batch * d.seqlen * d.nheads;
  const int64_t n_x = n_d * R * d.headdim;
  const int64_t n_bc = d.batch * d.seqlen * d.ngroups * R * d.dstate;
  // the descriptor check bounds batch * nheads * headdim * dstate * 4; the update kernel's lane count
  // is up to 64 times that many bytes' worth of states
  const int64_t n_st = d.batch * d.nheads * d.headdim * d.dstate;
  int64_t t = 0;
  if (!mul_ok(n_st, 4 * 64, &t)) return MSSM_ERR_INVALID_ARG;
  const int64_t b_st = n_st * 4;
  const bool has_steps = n_x > 0;
  if (A == nullptr) return MSSM_ERR_INVALID_ARG;
  if (has_steps && (x == nullptr || delta == nullptr || B == nullptr || C == nullptr || out == nullptr))
    return MSSM_ERR_INVALID_ARG;
  if (want_lam && has_steps && lam == nullptr) return MSSM_ERR_INVALID_ARG;
  if (!aligned(x, es) || !aligned(delta, es) || !aligned(B, es) || !aligned(C, es) || !aligned(z, es) ||
      !aligned(out, es) || !aligned(lam, es) || !aligned(A, 4) || !aligned(D, 4) || !aligned(h0, 4) ||
      !aligned(final_state, 4))
    return MSSM_ERR_MISALIGNED;
  const int64_t b_io = n_x * es, b_d = n_d * es;
  const void* ins[] = {x, delta, B, C, z, A, D, h0, lam};
  const int64_t inb[] = {b_io, b_d, n_bc * es, n_bc * es, b_io, d.nheads * 4, d.nheads * 4, b_st, b_d};
  for (int i = 0; i < 9; ++i) {
    if (overlap(out, b_io, ins[i], inb[i])) return MSSM_ERR_INVALID_ARG;
    if (overlap(final_state, b_st, ins[i], inb[i])) return MSSM_ERR_INVALID_ARG;
  }
  if (overlap(out, b_io, final_state, b_st)) return MSSM_ERR_INVALID_ARG;
  if (!has_steps && final_state == nullptr) return MSSM_OK;   // nothing to compute or store
  if (mssm::update_grid_blocks(d.batch * d.nheads * d.headdim, d.dstate) > std::numeric_limits<int32_t>::max())
    return MSSM_ERR_UNSUPPORTED;
  mssm::UpdateArgs a{};
  a.state = nullptr; a.state_in = h0; a.state_out = final_state;
  a.x = x; a.delta = delta; a.A = A; a.B = B; a.C = C; a.D = D; a.z = z; a.out = out;
  a.lam = want_lam ? lam : nullptr;
  a.batch = d.batch; a.L = d.seqlen; a.N = d.dstate; a.H = d.nheads; a.P = d.headdim; a.G = d.ngroups;
  a.io = d.io_dtype; a.rank = R;
  const hipError_t e = mssm::ssd_update_launch(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) {
    set_err(e);
    return MSSM_ERR_HIP;
  }
  return MSSM_OK;
}

// every multi-head sequence form: lam == nullptr (want_lam false) is the Mamba-2 rule, else lam is
// required; R > 1 is MIMO
int ssd_fwd_impl(const mssm_ssd_desc* desc, int64_t R, const void* x, const void* delta, const void* lam,
                 bool want_lam, const float* A, const void* B, const void* C, const float* D, const void* z,
                 const float* h0, void* out, float* final_state, void* workspace, size_t workspace_bytes,
                 void* stream) {
  int64_t Q = 0;
  bool matrix = false;
  const int v = validate_ssd_desc(desc, R, &Q, &matrix);
  if (v != MSSM_OK) return v;
  const mssm_ssd_desc& d = *desc;
  if (d.batch == 0) return MSSM_OK;
  if (!matrix)
    return ssd_fwd_recurrent(d, R, x, delta, want_lam ? lam : nullptr, want_lam, A, B, C, D, z, h0, out,
                             final_state, stream);
  const int64_t n_x = d.batch * d.seqlen * d.nheads * R * d.headdim;
  const int64_t n_d = d.batch * d.seqlen * d.nheads;
  const int64_t n_bc = d.batch * d.seqlen * d.ngroups * R * d.dstate;
  const int64_t b_st = d.batch * d.nheads * d.headdim * d.dstate * 4;
  const bool has_steps = n_x > 0;
  if (A == nullptr) return MSSM_ERR_INVALID_ARG;
  if (has_steps && (x == nullptr || delta == nullptr || B == nullptr || C == nullptr || out == nullptr))
    return MSSM_ERR_INVALID_ARG;
  if (want_lam && has_steps && lam == nullptr) return MSSM_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(z, 16) || !aligned(out, 16) || !aligned(B, 16) || !aligned(C, 16) ||
      !aligned(delta, 2) || !aligned(lam, 2) || !aligned(A, 4) || !aligned(D, 4) || !aligned(h0, 16) ||
      !aligned(final_state, 16))
    return MSSM_ERR_MISALIGNED;
  const void* ins[] = {x, delta, B, C, z, A, D, h0, lam};
  const int64_t inb[] = {n_x * 2, n_d * 2, n_bc * 2, n_bc * 2, n_x * 2, d.nheads * 4, d.nheads * 4, b_st, n_d * 2};
  for (int i = 0; i < 9; ++i) {
    if (overlap(out, n_x * 2, ins[i], inb[i])) return MSSM_ERR_INVALID_ARG;
    if (overlap(final_state, b_st, ins[i], inb[i])) return MSSM_ERR_INVALID_ARG;
  }
  if (overlap(out, n_x * 2, final_state, b_st)) return MSSM_ERR_INVALID_ARG;
  const size_t need = mssm::ssd_workspace_bytes(d.batch, d.seqlen, d.nheads, d.headdim, d.dstate, d.ngroups, Q);
  if (need > 0) {
    if (workspace == nullptr || workspace_bytes < need) return MSSM_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return MSSM_ERR_MISALIGNED;
    for (int i = 0; i < 9; ++i)
      if (overlap(workspace, static_cast<int64_t>(need), ins[i], inb[i])) return MSSM_ERR_INVALID_ARG;
    if (overlap(workspace, static_cast<int64_t>(need), out, n_x * 2) ||
        overlap(workspace, static_cast<int64_t>(need), final_state, b_st))
      return MSSM_ERR_INVALID_ARG;
    // the elementwise kernel adding the two shares: four columns per work-item
    if (n_x / 4 > static_cast<int64_t>(std::numeric_limits<uint32_t>::max()) - 255) return MSSM_ERR_UNSUPPORTED;
  }
  mssm::SSDArgs a{};
  a.x = x; a.delta = delta; a.lam = want_lam ? lam : nullptr; a.A = A; a.B = B; a.C = C; a.D = D; a.z = z;
  a.h0 = h0; a.out = out; a.final_state = final_state; a.workspace = workspace;
  a.batch = d.batch; a.L = d.seqlen; a.H = d.nheads; a.P = d.headdim; a.N = d.dstate; a.G = d.ngroups; a.Q = Q;
  a.R = R;
  const hipError_t e = mssm::ssd_launch(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) {
    set_err(e);
    return MSSM_ERR_HIP;
  }
  return MSSM_OK;
}
}  // namespace

extern "C" {

int mssm_ssd_fwd(const mssm_ssd_desc* desc, const void* x, const void* delta, const float* A, const void* B,
                 const void* C, const float* D, const void* z, const float* h0, void* out, float* final_state,
                 void* workspace, size_t workspace_bytes, void* stream) {
  return ssd_fwd_impl(desc, 1, x, delta, nullptr, false, A, B, C, D, z, h0, out, final_state, workspace,
                      workspace_bytes, stream);
}

int mssm_ssd_trapezoidal_fwd(const mssm_ssd_desc* desc, const void* x, const void* delta, const void* lam,
                             const float* A, const void* B, const void* C, const float* D, const void* z,
                             const float* h0, void* out, float* final_state, void* workspace,
                             size_t workspace_bytes, void* stream) {
  return ssd_fwd_impl(desc, 1, x, delta, lam, true, A, B, C, D, z, h0, out, final_state, workspace,
                      workspace_bytes, stream);
}

int mssm_ssd_mimo_fwd(const mssm_ssd_desc* desc, int32_t rank, const void* x, const void* delta, const void* lam,
                      const float* A, const void* B, const void* C, const float* D, const void* z, const float* h0,
                      void* out, float* final_state, void* workspace, size_t workspace_bytes, void* stream) {
  return ssd_fwd_impl(desc, rank, x, delta, lam, lam != nullptr, A, B, C, D, z, h0, out, final_state, workspace,
                      workspace_bytes, stream);
}

}  // extern "C"
