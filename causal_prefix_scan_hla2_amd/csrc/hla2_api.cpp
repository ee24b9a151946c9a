// hla2_api.cpp -- the C ABI of include/hla2.h: argument validation, the
// segment plan, workspace layout and kernel launches.  Validation runs on the
// host before any HIP call, so every error path is testable without a GPU.
#include <math.h>
#include <stdint.h>

#include "hla2.h"
#include "hla2_internal.h"

namespace {

struct Plan {
  int DK, DV, CP;  // padded head dims and chunk tile of the kernel instantiation
  int kc;          // tokens per chunk the walker steps by
  int cps;         // chunks per segment (segment 0: cps0; the last may be shorter)
  int cps0;        // chunks of segment 0
  int nseg;        // segments per (b, h)
  bool lead;       // lead plan: segment 0's output walk runs beside the summary walks and
                   // leaves the prefix of segment 1 (bf16 forward without state export)
  long BH;
};

// The output pass aims for one full round of workgroups on a 256-CU part.
constexpr long kComputeUnits = 256;
constexpr int kMaxSegments = 64;
constexpr long kMinChunksPerSegment = 4;
// Lead plans at d = 64 with this many summaries to fold (three segments) fold it in the output
// walk's prologue instead of launching the scan; the walker folds exactly one.  A fold step there
// is latency-bound (about 2 us: the summary's loads, then two barriers), so the launch is worth
// saving for one step only (decay workload: 0.2472 -> 0.2443 ms); at six steps (normalised 2k
// workload) a fold loop took 13 us of the output walk against 9.7 us for the scan launch.
constexpr int kMaxPrologueFolds = 1;
static_assert(kMaxPrologueFolds == 1, "the output walker folds exactly one summary in its prologue");
// Lead plans: segment 0 holds about lead_ratio(DK) times the chunks of the others, so that
// its output walk (the slower walk per chunk) ends with the summary walks it shares the launch
// with.  Measured per chunk, one workgroup per CU: d = 64, dv = 128: output 3.3 us, summary
// 2.3 us; d = dv = 128: output 5.4 us, summary 4.5 us.
double lead_ratio(int DK) { return DK > 64 ? 0.83 : 0.7; }

bool is_pow2_chunk(int c) { return c == 16 || c == 32 || c == 64 || c == 128; }

int check_shape(int B, int H, int n, int d, int dv, int chunk, int dtype) {
  if (B <= 0 || H <= 0 || n <= 0 || d <= 0 || dv <= 0 || chunk <= 0) return HLA2_ERR_INVALID;
  if (dtype != HLA2_F32 && dtype != HLA2_BF16) return HLA2_ERR_INVALID;
  if (d % 16 || dv % 16 || d > 128 || dv > 128 || !is_pow2_chunk(chunk)) return HLA2_ERR_UNSUPPORTED;
  if (dtype == HLA2_F32 && (d > 64 || dv > 64)) return HLA2_ERR_UNSUPPORTED;
  const long BH = (long)B * H;
  if (BH > (1L << 24) || (long)n > (1L << 30) || BH * (long)n > (1L << 40)) return HLA2_ERR_UNSUPPORTED;
  // one head's rows (padded by up to 16 columns) are addressed with 32-bit byte offsets
  if ((long)n * ((d > dv ? d : dv) + 16) * 4 > 0x7fffff00L) return HLA2_ERR_UNSUPPORTED;
  return HLA2_OK;
}

Plan make_plan(int B, int H, int n, int d, int dv, int chunk, int dtype, int segments = 0, long groups_per_cu = 0,
               bool lead = false, double lead_rho = 0.0) {
  Plan p;
  p.BH = (long)B * H;
  long gpc;  // workgroups of the output walker per CU
  if (dtype == HLA2_BF16) {
    // the bf16 walker always steps by 64-token chunks; `chunk` only changes rounding
    p.DK = d <= 64 ? 64 : 128;
    p.DV = dv <= 64 ? 64 : 128;
    p.CP = p.kc = 64;
    gpc = hla2::walk8_groups_per_cu();
  } else {
    const int m = d > dv ? d : dv;
    p.DK = p.DV = m <= 16 ? 16 : 64;
    p.CP = chunk <= 16 ? 16 : (chunk <= 64 ? 64 : 128);
    p.kc = chunk;
    gpc = hla2::walk_groups_per_cu(4, p.DK, p.DV, p.CP, true);
  }
  if (groups_per_cu > 0) gpc = groups_per_cu;
  p.lead = lead && dtype == HLA2_BF16;
  const long nc = ((long)n + p.kc - 1) / p.kc;
  const long target = kComputeUnits * gpc;
  long r;
  if (segments > 0) {
    r = segments;
  } else if (p.lead) {
    // the output walk of segments 1 .. r-1 (and the lead launch) put one workgroup on each
    // CU: without a summary of segment 0, fewer and longer segments save more summary work
    // than a second workgroup per CU gains (measured on the 8 x 16 x 8192, d = 64 workload:
    // 3 segments 276 us, 5 segments 292 us)
    r = p.BH >= kComputeUnits ? 1 : kComputeUnits / p.BH + 1;
  } else {
    r = (target + p.BH - 1) / p.BH;
  }
  // automatic plans keep at least kMinChunksPerSegment chunks per segment: shorter
  // segments add scan steps faster than they shorten the walks
  if (segments == 0 && r > nc / kMinChunksPerSegment) r = nc / kMinChunksPerSegment;
  if (r > nc) r = nc;
  if (r > kMaxSegments) r = kMaxSegments;
  if (r < 1) r = 1;
  if (p.lead && segments == 0 && r > 1) {
    // segment 0 about rho times the others (at least that, when the chunks do not
    // divide evenly: the last segment is then the shorter one)
    const double rho = lead_rho > 0.0 ? lead_rho : lead_ratio(p.DK);
    long cps = (long)ceil((double)nc / ((double)(r - 1) + rho));
    long cps0 = nc - (r - 1) * cps;
    const long lo = (long)ceil(rho * (double)cps);
    if (cps0 < lo) cps0 = lo;
    // a share above 1 makes segment 0 the longer one (for walkers whose summary walk costs more per
    // chunk than their output walk); otherwise segment 0 is never the longest
    if (cps0 > cps && rho <= 1.0) cps0 = cps;
    if (cps0 > nc - 1) cps0 = nc - 1;
    // spread the chunks after segment 0 evenly (never below segment 0's length), so that the
    // last segment is not the only short one
    const long even = (nc - cps0 + r - 2) / (r - 1);
    if (even >= cps0 && even < cps) cps = even;
    p.cps = (int)cps;
    p.cps0 = (int)cps0;
    p.nseg = 1 + (int)((nc - cps0 + cps - 1) / cps);
  } else {
    p.cps = p.cps0 = (int)((nc + r - 1) / r);
    p.nseg = (int)((nc + p.cps - 1) / p.cps);
  }
  if (p.nseg < 2) p.lead = false;
  return p;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// A launch of `groups` workgroups of `threads` work-items along one grid dimension must stay
// below 2^32 work-items; shapes whose grids would not fit are rejected before any launch.
bool grid_fits(long groups, long threads) { return groups > 0 && groups * threads <= 0xFFFFFFFFL; }
// every forward launch of a plan: walkers (up to 512 threads, one workgroup per head and
// segment), the scan (one column of up to 512 threads per head) and the state export
bool forward_grids_fit(const Plan &p) { return grid_fits(p.BH * p.nseg, 512) && grid_fits(p.BH, 512); }

// summary blocks per (b, h): segments 0 .. nseg-2 for the scan; every segment when the final
// state is exported
int nsum(const Plan &p, bool state) { return state ? p.nseg : p.nseg - 1; }
size_t sums_bytes(const Plan &p, bool state) {
  return (size_t)p.BH * nsum(p, state) * hla2::sum_block_floats(p.DK, p.DV) * sizeof(float);
}
size_t prefix_bytes(const Plan &p) {
  return p.nseg > 1 ? (size_t)p.BH * p.nseg * hla2::prefix_block_floats(p.DK, p.DV) * sizeof(float) : 0;
}
size_t workspace_bytes(const Plan &p, bool state = false) {
  if (p.nseg == 1 && !state) return 0;
  return align256(sums_bytes(p, state)) + prefix_bytes(p);
}

// Backward pass: the forward's segment plan (its summary walk and scan give each segment's
// incoming state), walked again in chunks of BC tokens.  The backward walkers hold one
// workgroup per CU.
struct BwdPlan {
  Plan p;
  int BC, DVP, nbc;
  bool norm;
  // Split prefix (bf16, two segments): the incoming state of segment 1 is formed from the
  // summaries of segment 0's two halves, walked by two workgroups per head, so that the
  // summary walk fills every CU instead of half of them.
  bool split;
  int half0, half1;  // chunks of the two halves
  size_t off_fsum, off_prefix, off_cst, off_rsum, off_suffix, off_gprep, total;
};
BwdPlan make_bwd_plan(int B, int H, int n, int d, int dv, int dtype, int normalize, int segments) {
  BwdPlan b;
  const int chunk = dtype == HLA2_BF16 ? 64 : 32;
  b.p = make_plan(B, H, n, d, dv, chunk, dtype, segments, 1);
  b.norm = normalize != 0;
  b.DVP = hla2::lds_walk_dvp(dtype == HLA2_F32, b.p.DV, b.norm);
  b.BC = hla2::lds_bwd_chunk(dtype == HLA2_F32, b.p.DK, b.DVP);
  b.nbc = (n + b.BC - 1) / b.BC;
  const size_t es = dtype == HLA2_F32 ? 4 : 2, BH = (size_t)b.p.BH, R = (size_t)b.p.nseg;
  const size_t DK = (size_t)b.p.DK, DVP = (size_t)b.DVP, adj = (DK * DVP + DK * DK) * 4;
  b.split = dtype == HLA2_BF16 && R == 2 && b.p.cps >= 2;
  b.half1 = b.p.cps / 2;
  b.half0 = b.p.cps - b.half1;
  size_t o = 0;
  b.off_fsum = o;
  o += align256(BH * (b.split ? 2 : R - 1) * (size_t)hla2::sum_block_floats(b.p.DK, b.p.DV) * 4);
  b.off_prefix = o;
  o += R > 1 ? align256(BH * R * (size_t)hla2::prefix_block_floats(b.p.DK, b.p.DV) * 4) : 0;
  b.off_cst = o;
  o += align256(BH * (size_t)b.nbc * (DK * DK + DK * DVP) * es);
  b.off_rsum = o;
  o += align256(BH * R * adj);
  b.off_suffix = o;
  o += align256(BH * R * adj);
  b.off_gprep = o;
  o += b.norm ? align256(BH * (size_t)n * DVP * es) : 0;
  b.total = o;
  return b;
}

int run_forward(const void *q, const void *k, const void *v, void *out, int B, int H, int n, int d, int dv,
                float decay, int normalize, int chunk, hla2_dtype_t dtype, float *den_out, float *state_out,
                void *workspace, size_t workspace_bytes_given, int segments, hipEvent_t const *events,
                hipStream_t stream) {
  return hla2::forward_run(q, k, v, out, B, H, n, d, dv, decay, normalize, chunk, (int)dtype, den_out, state_out,
                           workspace, workspace_bytes_given, segments, events, stream);
}

bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

}  // namespace

extern "C" {

const char *hla2_strerror(int code) {
  switch (code) {
    case HLA2_OK: return "ok";
    case HLA2_ERR_INVALID: return "invalid argument";
    case HLA2_ERR_UNSUPPORTED: return "unsupported shape, chunk or dtype";
    case HLA2_ERR_WORKSPACE: return "workspace missing or too small";
    case HLA2_ERR_LAUNCH: return "kernel launch failed";
    default: return "unknown error code";
  }
}

int hla2_abi_version(void) { return 1; }

long hla2_state_floats(int d, int dv) {
  if (d <= 0 || dv <= 0) return HLA2_ERR_INVALID;
  return (long)d * d + 2L * d * dv + 2L * d;
}

static size_t forward_workspace(int B, int H, int n, int d, int dv, int chunk, int segments, bool state) {
  // the plan does not depend on dtype beyond padding; size for the larger padding
  if (segments < 0 || check_shape(B, H, n, d, dv, chunk, HLA2_BF16) != HLA2_OK) return 0;
  Plan pb = make_plan(B, H, n, d, dv, chunk, HLA2_BF16, segments, 0, !state);
  size_t wb = workspace_bytes(pb, state);
  if (d <= 64 && dv <= 64) {
    Plan pf = make_plan(B, H, n, d, dv, chunk, HLA2_F32, segments);
    size_t wf = workspace_bytes(pf, state);
    if (wf > wb) wb = wf;
  }
  return wb;
}

size_t hla2_forward_ex_workspace_bytes(int B, int H, int n, int d, int dv, int chunk, int segments) {
  return forward_workspace(B, H, n, d, dv, chunk, segments, false);
}

size_t hla2_forward_state_workspace_bytes(int B, int H, int n, int d, int dv, int chunk, int segments) {
  return forward_workspace(B, H, n, d, dv, chunk, segments, true);
}

size_t hla2_forward_workspace_bytes(int B, int H, int n, int d, int dv, int chunk) {
  return hla2_forward_ex_workspace_bytes(B, H, n, d, dv, chunk, 0);
}

int hla2_forward_ex_segments(int B, int H, int n, int d, int dv, int chunk, int segments) {
  if (segments < 0) return HLA2_ERR_INVALID;
  int rc = check_shape(B, H, n, d, dv, chunk, HLA2_BF16);
  if (rc != HLA2_OK) return rc;
  return make_plan(B, H, n, d, dv, chunk, HLA2_BF16, segments, 0, true).nseg;
}

int hla2_forward_ex_plan(int B, int H, int n, int d, int dv, int chunk, int segments, int *nseg, int *lead_chunks,
                         int *seg_chunks) {
  if (segments < 0 || !nseg || !lead_chunks || !seg_chunks) return HLA2_ERR_INVALID;
  int rc = check_shape(B, H, n, d, dv, chunk, HLA2_BF16);
  if (rc != HLA2_OK) return rc;
  const Plan p = make_plan(B, H, n, d, dv, chunk, HLA2_BF16, segments, 0, true);
  *nseg = p.nseg;
  *lead_chunks = p.cps0;
  *seg_chunks = p.cps;
  return p.lead ? 1 : 0;
}

int hla2_forward_segments(int B, int H, int n, int d, int dv, int chunk) {
  return hla2_forward_ex_segments(B, H, n, d, dv, chunk, 0);
}

int hla2_forward(const void *q, const void *k, const void *v, void *out, int B, int H, int n, int d,
                 int dv, float decay, int normalize, int chunk, hla2_dtype_t dtype, float *den_out,
                 void *workspace, size_t workspace_bytes_given, hipStream_t stream) {
  return hla2_forward_ex(q, k, v, out, B, H, n, d, dv, decay, normalize, chunk, dtype, den_out, workspace,
                         workspace_bytes_given, 0, stream);
}

int hla2_forward_ex(const void *q, const void *k, const void *v, void *out, int B, int H, int n, int d,
                    int dv, float decay, int normalize, int chunk, hla2_dtype_t dtype, float *den_out,
                    void *workspace, size_t workspace_bytes_given, int segments, hipStream_t stream) {
  return hla2_forward_timed(q, k, v, out, B, H, n, d, dv, decay, normalize, chunk, dtype, den_out, workspace,
                            workspace_bytes_given, segments, nullptr, stream);
}

int hla2_forward_timed(const void *q, const void *k, const void *v, void *out, int B, int H, int n, int d,
                       int dv, float decay, int normalize, int chunk, hla2_dtype_t dtype, float *den_out,
                       void *workspace, size_t workspace_bytes_given, int segments, hipEvent_t const *events,
                       hipStream_t stream) {
  return run_forward(q, k, v, out, B, H, n, d, dv, decay, normalize, chunk, dtype, den_out, nullptr, workspace,
                     workspace_bytes_given, segments, events, stream);
}

int hla2_forward_state(const void *q, const void *k, const void *v, void *out, int B, int H, int n, int d,
                       int dv, float decay, int normalize, int chunk, hla2_dtype_t dtype, float *den_out,
                       float *state_out, void *workspace, size_t workspace_bytes_given, int segments,
                       hipStream_t stream) {
  if (!state_out) return HLA2_ERR_INVALID;
  return run_forward(q, k, v, out, B, H, n, d, dv, decay, normalize, chunk, dtype, den_out, state_out, workspace,
                     workspace_bytes_given, segments, nullptr, stream);
}

size_t hla2_backward_workspace_bytes(int B, int H, int n, int d, int dv, int normalize, hla2_dtype_t dtype,
                                     int segments) {
  if (segments < 0 || (normalize != 0 && normalize != 1)) return 0;
  const int chunk = dtype == HLA2_BF16 ? 64 : 32;
  if (check_shape(B, H, n, d, dv, chunk, (int)dtype) != HLA2_OK) return 0;
  return make_bwd_plan(B, H, n, d, dv, (int)dtype, normalize, segments).total;
}

int hla2_backward(const void *q, const void *k, const void *v, const void *out, const float *den, const void *dout,
                  void *grad_q, void *grad_k, void *grad_v, int B, int H, int n, int d, int dv, float decay,
                  int normalize, hla2_dtype_t dtype, void *workspace, size_t workspace_bytes_given, int segments,
                  hipStream_t stream) {
  if (!q || !k || !v || !dout || !grad_q || !grad_k || !grad_v) return HLA2_ERR_INVALID;
  if (normalize != 0 && normalize != 1) return HLA2_ERR_INVALID;
  if (normalize && (!out || !den)) return HLA2_ERR_INVALID;
  if (segments < 0) return HLA2_ERR_INVALID;
  if (!(decay > 0.0f && decay <= 1.0f)) return HLA2_ERR_INVALID;
  if (dtype != HLA2_F32 && dtype != HLA2_BF16) return HLA2_ERR_INVALID;
  const int chunk = dtype == HLA2_BF16 ? 64 : 32;
  int rc = check_shape(B, H, n, d, dv, chunk, (int)dtype);
  if (rc != HLA2_OK) return rc;
  const void *tens[] = {q, k, v, dout, grad_q, grad_k, grad_v};
  for (const void *t : tens)
    if (!aligned(t, 16)) return HLA2_ERR_INVALID;
  if (normalize && (!aligned(out, 16) || !aligned(den, 4))) return HLA2_ERR_INVALID;
  const BwdPlan b = make_bwd_plan(B, H, n, d, dv, (int)dtype, normalize, segments);
  // the pre-walk runs two roles per segment; the ratio's preparation one thread per 4 values
  if (!forward_grids_fit(b.p) || !grid_fits(2 * b.p.BH * b.p.nseg, 512) ||
      (b.norm && !grid_fits((b.p.BH * n + 3) / 4, 256)))
    return HLA2_ERR_UNSUPPORTED;
  if (!workspace || workspace_bytes_given < b.total || !aligned(workspace, 256)) return HLA2_ERR_WORKSPACE;
  const Plan &p = b.p;
  const int dt = dtype == HLA2_F32 ? 0 : 1;
  char *ws = (char *)workspace;
  float *fsum = (float *)(ws + b.off_fsum), *prefix = p.nseg > 1 ? (float *)(ws + b.off_prefix) : nullptr;
  const float log2g = decay < 1.0f ? log2f(decay) : 0.0f;
  hipError_t e;

  hla2::BwdPrepArgs pa;
  pa.dout = dout;
  pa.out = out;
  pa.den = den;
  pa.gprep = ws + b.off_gprep;
  pa.rows = p.BH * n;
  pa.dv = dv;
  if (b.norm) {
    e = hla2::launch_bwd(dt, p.DK, p.DV, true, hla2::BWD_PREP, (int)p.BH, hla2::BwdArgs{}, pa, 1.f, stream);
    if (e != hipSuccess) return HLA2_ERR_LAUNCH;
  }
  // incoming forward state of every segment: the forward's summary walk and scan (with a split
  // prefix: the two halves of segment 0 summarised and folded, only segment 1's prefix kept)
  if (p.nseg > 1) {
    hla2::WalkArgs a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.out = nullptr;
    a.den_out = nullptr;
    a.prefix = nullptr;
    a.sums = fsum;
    a.n = n;
    a.d = d;
    a.dv = dv;
    a.chunk = p.kc;
    a.cps = p.cps;
    a.nseg = p.nseg;
    a.log2g = log2g;
    a.decay_on = decay < 1.0f ? 1 : 0;
    a.normalize = normalize;
    a.need_den = normalize;
    a.sum_all = 0;
    if (b.split) {  // segments 0 | 1 | 2 of the walk: the two halves, then the whole segment 1
      a.nseg = 3;
      a.cps0 = b.half0;
      a.cps = b.half1;
    }
    e = hla2::launch_walk(dt, p.DK, p.DV, p.CP, false, dim3((unsigned)(p.BH * (a.nseg - 1))), a, stream);
    if (e != hipSuccess) return HLA2_ERR_LAUNCH;
    hla2::ScanArgs sa;
    sa.sums = fsum;
    sa.nsum = a.nseg - 1;
    sa.prefix = prefix;
    sa.nseg = a.nseg;
    // the fold of the first summary starts from zero, so only the later segments' length counts
    sa.gamma_seg = decay < 1.0f ? (float)pow((double)decay, (double)a.cps * p.kc) : 1.0f;
    if (b.split) {  // keep the prefix after both halves, as block 1 of the two-segment layout
      sa.pnseg = 2;
      sa.pmin = 2;
      sa.pshift = 1;
    }
    e = hla2::launch_scan(dt, p.DK, p.DV, (int)p.BH, sa, stream);
    if (e != hipSuccess) return HLA2_ERR_LAUNCH;
  }
  hla2::BwdArgs ba;
  ba.q = q;
  ba.k = k;
  ba.v = v;
  ba.g = b.norm ? (const void *)(ws + b.off_gprep) : dout;
  ba.dq_out = grad_q;
  ba.dk_out = grad_k;
  ba.dv_out = grad_v;
  ba.prefix = prefix;
  ba.fsum = fsum;
  ba.cstate = ws + b.off_cst;
  ba.rsum = (float *)(ws + b.off_rsum);
  ba.suffix = (float *)(ws + b.off_suffix);
  ba.n = n;
  ba.d = d;
  ba.dv = dv;
  ba.gld = b.norm ? b.DVP : dv;
  ba.nseg = p.nseg;
  ba.cps = p.cps;
  ba.kc = p.kc;
  ba.nbc = b.nbc;
  ba.nbh = (int)p.BH;
  ba.log2g = log2g;
  // With 64-token backward chunks at d <= 64, segment 0's forward-state walk runs in two halves, the
  // second from the first's summary: the pre-walk then has four workgroups per head, two per CU, and
  // every CU gets one long walk and one short one instead of half the CUs getting both long ones
  // (decay workload: 0.967 -> 0.889 ms per backward call; with the ratio at dv = 128, whose chunks
  // are 32 tokens, it measured 0.6% slower and is not split).
  ba.half0 = (b.split && p.DK <= 64 && b.BC == 64) ? b.half0 : 0;
  const float gL = decay < 1.0f ? (float)pow((double)decay, (double)p.cps * p.kc) : 1.0f;
  const int phases[] = {hla2::BWD_PRE, hla2::BWD_RSCAN, hla2::BWD_WALK};
  for (int ph : phases) {
    e = hla2::launch_bwd(dt, p.DK, p.DV, b.norm, ph, (int)p.BH, ba, pa, gL, stream);
    if (e != hipSuccess) return HLA2_ERR_LAUNCH;
  }
  return HLA2_OK;
}

static size_t ahla_workspace(const Plan &p, int dtype) {
  const size_t DK = (size_t)p.DK, DVP = (size_t)hla2::lds_walk_dvp(dtype == HLA2_F32, p.DV, true);
  const size_t BH = (size_t)p.BH, R = (size_t)p.nseg;
  if (R == 1) return 0;
  return align256(BH * (R - 1) * (2 * DK * DVP + DK * DK) * 4) + BH * R * 2 * DK * DVP * 4;
}

// AHLA and third order: one workgroup per CU; bf16 runs a lead plan.  Segment 0's share is
// about the ratio of a summary chunk to an output chunk of the walker (tile walkers, d = 64,
// dv = 128, one workgroup per CU: AHLA 2.75 against 3.8 us, third order 4.5 against 5.1 us).
// At d <= 64, dv > 64 the calls without den run on the register-resident walkers, for which
// the share was measured directly at the decay workload's shape (AHLA: 0.72, 0.84, 0.95 gave
// 218-228, 215-222, 214-217 us; third order: 0.75, 0.88, 1.0 gave 334-344, 327-338, 325-329 us,
// and once its output walk skipped the masked tiles, 1.05 against 1.0 gave 304-323 against 316-330
// us: its summary walk then costs more per chunk than its output walk, so segment 0 is the longest).
// The share depends only on the shape, so that the workspace query, which does not know
// whether den is carried, sizes the same plan.
static bool variant_register_walker(int d, int dv, int dtype) { return dtype == HLA2_BF16 && d <= 64 && dv > 64; }
static Plan ahla_plan(int B, int H, int n, int d, int dv, int dtype, int segments, double rho = 0.0) {
  if (rho <= 0.0) rho = variant_register_walker(d, dv, dtype) ? 0.95 : 0.72;
  return make_plan(B, H, n, d, dv, dtype == HLA2_BF16 ? 64 : 32, dtype, segments, 1, true, rho);
}
static Plan ho3_plan(int B, int H, int n, int d, int dv, int dtype, int segments) {
  return ahla_plan(B, H, n, d, dv, dtype, segments, variant_register_walker(d, dv, dtype) ? 1.05 : 0.88);
}

size_t hla2_ahla_forward_workspace_bytes(int B, int H, int n, int d, int dv, hla2_dtype_t dtype, int segments) {
  if (segments < 0 || (dtype != HLA2_F32 && dtype != HLA2_BF16)) return 0;
  if (check_shape(B, H, n, d, dv, dtype == HLA2_BF16 ? 64 : 32, (int)dtype) != HLA2_OK) return 0;
  return ahla_workspace(ahla_plan(B, H, n, d, dv, (int)dtype, segments), (int)dtype);
}

int hla2_ahla_forward(const void *q, const void *k, const void *v, void *out, int B, int H, int n, int d, int dv,
                      float decay, int normalize, hla2_dtype_t dtype, float *den_out, void *workspace,
                      size_t workspace_bytes_given, int segments, hipStream_t stream) {
  if (!q || !k || !v || !out) return HLA2_ERR_INVALID;
  if (normalize != 0 && normalize != 1) return HLA2_ERR_INVALID;
  if (segments < 0) return HLA2_ERR_INVALID;
  if (!(decay > 0.0f && decay <= 1.0f)) return HLA2_ERR_INVALID;
  if (dtype != HLA2_F32 && dtype != HLA2_BF16) return HLA2_ERR_INVALID;
  int rc = check_shape(B, H, n, d, dv, dtype == HLA2_BF16 ? 64 : 32, (int)dtype);
  if (rc != HLA2_OK) return rc;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16)) return HLA2_ERR_INVALID;
  if (den_out && !aligned(den_out, 4)) return HLA2_ERR_INVALID;
  const Plan p = ahla_plan(B, H, n, d, dv, (int)dtype, segments);
  if (!forward_grids_fit(p)) return HLA2_ERR_UNSUPPORTED;
  const size_t need = ahla_workspace(p, (int)dtype);
  if (need > 0 && (!workspace || workspace_bytes_given < need || !aligned(workspace, 256))) return HLA2_ERR_WORKSPACE;
  const int dt = dtype == HLA2_F32 ? 0 : 1;
  const bool norm = normalize || den_out;
  const size_t DK = (size_t)p.DK, DVP = (size_t)hla2::lds_walk_dvp(dt == 0, p.DV, norm);
  hla2::AhlaArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.out = out;
  a.den_out = den_out;
  a.sums = need ? (float *)workspace : nullptr;
  a.prefix = need ? (float *)((char *)workspace + align256((size_t)p.BH * (p.nseg - 1) * (2 * DK * DVP + DK * DK) * 4))
                  : nullptr;
  a.n = n;
  a.d = d;
  a.dv = dv;
  a.nseg = p.nseg;
  a.cps = p.cps;
  a.kc = p.kc;
  a.log2g = decay < 1.0f ? log2f(decay) : 0.0f;
  a.normalize = normalize;
  a.cps0 = p.cps0;
  a.nbh = (int)p.BH;
  const float gseg = decay < 1.0f ? (float)pow((double)decay, (double)p.cps * p.kc) : 1.0f;
  hipError_t e;
  if (p.lead) {
    // segment 0's outputs beside the summaries of segments 1 .. nseg-2; the scan from the
    // prefix segment 0 leaves; the outputs of segments 1 .. nseg-1
    e = hla2::launch_ahla(dt, p.DK, p.DV, norm, hla2::AHLA_LEAD, (int)p.BH, a, gseg, stream);
    if (e != hipSuccess) return HLA2_ERR_LAUNCH;
    if (p.nseg == 3 && p.DK == 64) {
      // one summary to fold: segment 2's output workgroups fold it in their prologue
      a.pfold = 1;
      a.gseg = gseg;
    } else if (p.nseg > 2) {
      a.first = 1;
      e = hla2::launch_ahla(dt, p.DK, p.DV, norm, hla2::AHLA_SCAN, (int)p.BH, a, gseg, stream);
      if (e != hipSuccess) return HLA2_ERR_LAUNCH;
    }
    a.seg_lo = 1;
  } else if (p.nseg > 1) {
    e = hla2::launch_ahla(dt, p.DK, p.DV, norm, hla2::AHLA_SUMMARY, (int)p.BH, a, gseg, stream);
    if (e != hipSuccess) return HLA2_ERR_LAUNCH;
    e = hla2::launch_ahla(dt, p.DK, p.DV, norm, hla2::AHLA_SCAN, (int)p.BH, a, gseg, stream);
    if (e != hipSuccess) return HLA2_ERR_LAUNCH;
  }
  e = hla2::launch_ahla(dt, p.DK, p.DV, norm, hla2::AHLA_OUTPUT, (int)p.BH, a, gseg, stream);
  return e == hipSuccess ? HLA2_OK : HLA2_ERR_LAUNCH;
}

static size_t ho3_sums_bytes(const Plan &p, int dt, bool norm) {
  const size_t DK = (size_t)p.DK, DVP = (size_t)hla2::lds_walk_dvp(dt == 0, p.DV, norm);
  return (size_t)p.BH * (p.nseg - 1) * (DK * DK + 2 * DK * DVP + 2 * DK * DK + DK * DVP) * 4;
}
static size_t ho3_workspace(const Plan &p, int dtype) {
  if (p.nseg == 1) return 0;
  const int dt = dtype == HLA2_F32 ? 0 : 1;
  const size_t DK = (size_t)p.DK, DVP = (size_t)hla2::lds_walk_dvp(dt == 0, p.DV, true);
  return align256(ho3_sums_bytes(p, dt, true)) + (size_t)p.BH * p.nseg * (DK * DK + 2 * DK * DVP) * 4;
}
static int ho3_check(int B, int H, int n, int d, int dv, int dtype) {
  int rc = check_shape(B, H, n, d, dv, dtype == HLA2_BF16 ? 64 : 32, dtype);
  if (rc != HLA2_OK) return rc;
  return d > 64 ? HLA2_ERR_UNSUPPORTED : HLA2_OK;  // the third-order state (d x d twice) is held for d <= 64
}

size_t hla2_ho3_forward_workspace_bytes(int B, int H, int n, int d, int dv, hla2_dtype_t dtype, int segments) {
  if (segments < 0 || (dtype != HLA2_F32 && dtype != HLA2_BF16)) return 0;
  if (ho3_check(B, H, n, d, dv, (int)dtype) != HLA2_OK) return 0;
  return ho3_workspace(ho3_plan(B, H, n, d, dv, (int)dtype, segments), (int)dtype);
}

int hla2_ho3_forward(const void *q, const void *k, const void *v, void *out, int B, int H, int n, int d, int dv,
                     float decay, int normalize, hla2_dtype_t dtype, float *den_out, void *workspace,
                     size_t workspace_bytes_given, int segments, hipStream_t stream) {
  if (!q || !k || !v || !out) return HLA2_ERR_INVALID;
  if (normalize != 0 && normalize != 1) return HLA2_ERR_INVALID;
  if (segments < 0) return HLA2_ERR_INVALID;
  if (!(decay > 0.0f && decay <= 1.0f)) return HLA2_ERR_INVALID;
  if (dtype != HLA2_F32 && dtype != HLA2_BF16) return HLA2_ERR_INVALID;
  int rc = ho3_check(B, H, n, d, dv, (int)dtype);
  if (rc != HLA2_OK) return rc;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16)) return HLA2_ERR_INVALID;
  if (den_out && !aligned(den_out, 4)) return HLA2_ERR_INVALID;
  const Plan p = ho3_plan(B, H, n, d, dv, (int)dtype, segments);
  if (!forward_grids_fit(p)) return HLA2_ERR_UNSUPPORTED;
  const size_t need = ho3_workspace(p, (int)dtype);
  if (need > 0 && (!workspace || workspace_bytes_given < need || !aligned(workspace, 256))) return HLA2_ERR_WORKSPACE;
  const int dt = dtype == HLA2_F32 ? 0 : 1;
  const bool norm = normalize || den_out;
  hla2::Ho3Args a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.out = out;
  a.den_out = den_out;
  a.sums = need ? (float *)workspace : nullptr;
  a.prefix = need ? (float *)((char *)workspace + align256(ho3_sums_bytes(p, dt, norm))) : nullptr;
  a.n = n;
  a.d = d;
  a.dv = dv;
  a.nseg = p.nseg;
  a.cps = p.cps;
  a.kc = p.kc;
  a.log2g = decay < 1.0f ? log2f(decay) : 0.0f;
  a.normalize = normalize;
  a.cps0 = p.cps0;
  a.nbh = (int)p.BH;
  const float gseg = decay < 1.0f ? (float)pow((double)decay, (double)p.cps * p.kc) : 1.0f;
  hipError_t e;
  if (p.lead) {
    // as for AHLA: segment 0's outputs beside the summaries, the scan from its prefix, the rest
    e = hla2::launch_ho3(dt, p.DK, p.DV, norm, hla2::HO3_LEAD, (int)p.BH, a, gseg, stream);
    if (e != hipSuccess) return HLA2_ERR_LAUNCH;
    if (p.nseg == 3 && !(norm && p.DV > 64)) {
      // one summary to fold: segment 2's output workgroups fold it in their prologue (the walkers of
      // the ratio at dv = 128 step by 32-token chunks, whose slots cannot stage the d x d operands)
      a.pfold = 1;
      a.gseg = gseg;
    } else if (p.nseg > 2) {
      a.first = 1;
      e = hla2::launch_ho3(dt, p.DK, p.DV, norm, hla2::HO3_SCAN, (int)p.BH, a, gseg, stream);
      if (e != hipSuccess) return HLA2_ERR_LAUNCH;
    }
    a.seg_lo = 1;
  } else if (p.nseg > 1) {
    e = hla2::launch_ho3(dt, p.DK, p.DV, norm, hla2::HO3_SUMMARY, (int)p.BH, a, gseg, stream);
    if (e != hipSuccess) return HLA2_ERR_LAUNCH;
    e = hla2::launch_ho3(dt, p.DK, p.DV, norm, hla2::HO3_SCAN, (int)p.BH, a, gseg, stream);
    if (e != hipSuccess) return HLA2_ERR_LAUNCH;
  }
  e = hla2::launch_ho3(dt, p.DK, p.DV, norm, hla2::HO3_OUTPUT, (int)p.BH, a, gseg, stream);
  return e == hipSuccess ? HLA2_OK : HLA2_ERR_LAUNCH;
}

int hla2_decode_step(float *state, const void *q, const void *k, const void *v, void *out, int N, int H,
                     int d, int dv, float decay, int normalize, hla2_dtype_t dtype, hipStream_t stream) {
  if (!state || !q || !k || !v || !out) return HLA2_ERR_INVALID;
  if (N <= 0 || H <= 0 || d <= 0 || dv <= 0) return HLA2_ERR_INVALID;
  if (!(decay > 0.0f && decay <= 1.0f)) return HLA2_ERR_INVALID;
  if (normalize != 0 && normalize != 1) return HLA2_ERR_INVALID;
  if (dtype != HLA2_F32 && dtype != HLA2_BF16) return HLA2_ERR_INVALID;
  auto ok = [](int x) { return x == 16 || x == 32 || x == 64 || x == 128; };
  if (!ok(d) || !ok(dv)) return HLA2_ERR_UNSUPPORTED;
  const long NH = (long)N * H;
  if (!grid_fits(NH, 256)) return HLA2_ERR_UNSUPPORTED;  // one 256-thread workgroup per (sequence, head)
  if (!aligned(state, 16)) return HLA2_ERR_INVALID;
  const size_t esz = dtype == HLA2_F32 ? 4 : 2;
  if (!aligned(q, esz) || !aligned(k, esz) || !aligned(v, esz) || !aligned(out, esz)) return HLA2_ERR_INVALID;
  hla2::DecodeArgs a;
  a.state = state;
  a.q = q;
  a.k = k;
  a.v = v;
  a.out = out;
  a.NH = (int)NH;
  a.d = d;
  a.dv = dv;
  a.gamma = decay;
  a.normalize = normalize;
  hipError_t e = hla2::launch_decode(dtype == HLA2_F32 ? 0 : 1, a, stream);
  return e == hipSuccess ? HLA2_OK : HLA2_ERR_LAUNCH;
}

}  // extern "C"

namespace hla2 {

int forward_check(const void *q, const void *k, const void *v, const void *out, int B, int H, int n, int d, int dv,
                  float decay, int normalize, int chunk, int dtype, const float *den_out, const float *state_out,
                  int segments, size_t *need_out) {
  if (!q || !k || !v || !out) return HLA2_ERR_INVALID;
  if (segments < 0) return HLA2_ERR_INVALID;
  if (!(decay > 0.0f && decay <= 1.0f)) return HLA2_ERR_INVALID;  // also rejects NaN
  if (normalize != 0 && normalize != 1) return HLA2_ERR_INVALID;
  int rc = check_shape(B, H, n, d, dv, chunk, dtype);
  if (rc != HLA2_OK) return rc;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16)) return HLA2_ERR_INVALID;
  if (den_out && !aligned(den_out, 4)) return HLA2_ERR_INVALID;
  if (state_out && !aligned(state_out, 4)) return HLA2_ERR_INVALID;
  const bool state = state_out != nullptr;
  const Plan p = make_plan(B, H, n, d, dv, chunk, dtype, segments, 0, !state);
  if (!forward_grids_fit(p)) return HLA2_ERR_UNSUPPORTED;
  // callers are held to the size the workspace query reports (the larger of the bf16 and
  // fp32 plans), whichever dtype this call uses
  const size_t need = workspace_bytes(p, state), need_doc = forward_workspace(B, H, n, d, dv, chunk, segments, state);
  *need_out = need > need_doc ? need : need_doc;
  return HLA2_OK;
}

int forward_run(const void *q, const void *k, const void *v, void *out, int B, int H, int n, int d, int dv,
                float decay, int normalize, int chunk, int dtype_i, float *den_out, float *state_out,
                void *workspace, size_t workspace_bytes_given, int segments, hipEvent_t const *events,
                hipStream_t stream) {
  const hla2_dtype_t dtype = (hla2_dtype_t)dtype_i;
  size_t need_all = 0;
  int rc = forward_check(q, k, v, out, B, H, n, d, dv, decay, normalize, chunk, dtype_i, den_out, state_out,
                         segments, &need_all);
  if (rc != HLA2_OK) return rc;
  const bool state = state_out != nullptr;
  const Plan p = make_plan(B, H, n, d, dv, chunk, (int)dtype, segments, 0, !state);
  const size_t need = workspace_bytes(p, state);
  if (need_all > 0) {
    if (!workspace || workspace_bytes_given < need_all || !aligned(workspace, 256)) return HLA2_ERR_WORKSPACE;
  }

  hla2::WalkArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.out = out;
  a.den_out = den_out;
  a.n = n;
  a.d = d;
  a.dv = dv;
  a.chunk = p.kc;
  a.cps = p.cps;
  a.cps0 = p.cps0;
  a.nseg = p.nseg;
  a.nbh = (int)p.BH;
  a.log2g = decay < 1.0f ? log2f(decay) : 0.0f;
  a.decay_on = decay < 1.0f ? 1 : 0;
  a.normalize = normalize;
  a.need_den = (normalize || den_out || state) ? 1 : 0;
  a.sum_all = state ? 1 : 0;
  float *sums = nullptr, *prefix = nullptr;
  if (need > 0) {
    sums = (float *)workspace;
    prefix = p.nseg > 1 ? (float *)((char *)workspace + align256(sums_bytes(p, state))) : nullptr;
  }
  a.sums = sums;
  a.prefix = prefix;
  a.prefix_out = prefix;
  const int dt = dtype == HLA2_F32 ? 0 : 1;
  const int ns = nsum(p, state);

  // Plain plan: summary walk of segments 0 .. ns-1, scan from the zero state, output walk of
  // every segment.  Lead plan: segment 0's output walk (leaving the prefix of segment 1) in
  // one launch with the summary walks of segments 1 .. ns-1, the scan from that prefix, then
  // the output walk of segments 1 .. nseg-1.
  auto mark = [&](int i) { return (events && events[i]) ? hipEventRecord(events[i], stream) : hipSuccess; };
  hipError_t e = mark(0);
  if (e != hipSuccess) return HLA2_ERR_LAUNCH;
  // with the final state of a sequence shorter than one chunk there is no full chunk to summarise:
  // the state kernel absorbs every token itself
  const bool all_tail = state && p.nseg == 1 && n < p.kc;
  if (p.lead) {
    e = hla2::launch_walk_lead(p.DK, p.DV, dim3((unsigned)(p.BH * ns)), a, stream);
    if (e != hipSuccess) return HLA2_ERR_LAUNCH;
  } else if (ns > 0 && !all_tail) {
    e = hla2::launch_walk(dt, p.DK, p.DV, p.CP, false, dim3((unsigned)(p.BH * ns)), a, stream);
    if (e != hipSuccess) return HLA2_ERR_LAUNCH;
  }
  if (mark(1) != hipSuccess) return HLA2_ERR_LAUNCH;
  // a three-segment lead plan at d = 64 folds segment 1's summary in the prologue of segment 2's
  // output walk instead of launching the scan
  const float gseg = decay < 1.0f ? (float)pow((double)decay, (double)p.cps * p.kc) : 1.0f;
  const bool pfold = p.lead && dt == 1 && p.DK == 64 && p.nseg > 2 && p.nseg - 2 <= kMaxPrologueFolds;
  if (p.nseg > (p.lead ? 2 : 1) && !pfold) {
    hla2::ScanArgs s;
    s.sums = sums;
    s.nsum = ns;
    s.prefix = prefix;
    s.nseg = p.nseg;
    s.gamma_seg = gseg;
    s.first = p.lead ? 1 : 0;
    e = hla2::launch_scan(dt, p.DK, p.DV, (int)p.BH, s, stream);
    if (e != hipSuccess) return HLA2_ERR_LAUNCH;
  }
  if (mark(2) != hipSuccess) return HLA2_ERR_LAUNCH;
  a.seg_lo = p.lead ? 1 : 0;
  a.pfold = pfold ? 1 : 0;
  a.gamma_seg = gseg;
  e = hla2::launch_walk(dt, p.DK, p.DV, p.CP, true, dim3((unsigned)(p.BH * (p.nseg - a.seg_lo))), a, stream);
  if (e != hipSuccess) return HLA2_ERR_LAUNCH;
  if (mark(3) != hipSuccess) return HLA2_ERR_LAUNCH;
  if (state) {
    hla2::StateArgs st;
    st.sums = all_tail ? nullptr : sums;
    st.prefix = prefix;
    st.q = q;
    st.k = k;
    st.v = v;
    st.state_out = state_out;
    st.n = n;
    st.d = d;
    st.dv = dv;
    st.nseg = p.nseg;
    st.cps = p.cps;
    st.kc = p.kc;
    st.log2g = a.log2g;
    st.decay_on = a.decay_on;
    e = hla2::launch_state(dt, p.DK, p.DV, (int)p.BH, st, stream);
    if (e != hipSuccess) return HLA2_ERR_LAUNCH;
  }
  return HLA2_OK;
}

}  // namespace hla2
