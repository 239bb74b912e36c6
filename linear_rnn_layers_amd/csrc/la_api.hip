// la_api.hip -- the C ABI of include/la.h: argument validation, sequence
// planning, workspace layout, kernel dispatch and timing hooks.
//
// Nothing here allocates device memory or synchronises the stream (except
// la_forward_wait_status, a documented blocking query), and nothing keeps
// mutable state between calls: every choice a call depends on comes from its
// arguments (la_options).  The only process-wide data are immutable caches of
// device properties (compute units, kernel occupancy), filled on first use.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <atomic>
#include <functional>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/la.h"
#include "la_decay.h"
#include "la_bwd2.h"
#include "la_wide.h"

// la_forward_causal_noalloc takes the workspace of the causal forward from
// this file-scope array instead of from the caller: for callers that cannot
// allocate.  Each GPU holds its own copy (allocated when the code object is
// loaded on it, kept until the process ends); host code reaches it only
// through the device address that hipGetSymbolAddress returns with that
// device current (scratch_ptr), never through the array's name.  Every call
// on one GPU shares it: calls that overlap on one GPU race.  The forward
// clears what must start at zero (the one-launch form's flags and status
// word) itself, with a kernel.
constexpr size_t kScratchBytes = LA_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

thread_local std::string g_err;

int fail(int status, const std::string& msg) {
  g_err = msg;
  return status;
}

// ------------------------------------------------------------------ plan
// The sequence of each head is cut into segments of L tokens, a multiple of
// 64, so that about 512 or 1024 workgroups exist (two to four per compute
// unit) even when B*H is small: the aggregate, forward and reverse-aggregate kernels keep
// several workgroups resident per compute unit to hide their memory and LDS
// latency.  Segment boundaries are the checkpoint entries.  The backward,
// whose workgroup fills most of a compute unit's LDS, walks coarser segments
// of kb consecutive segments (chosen at launch from its occupancy).  The
// segment plan depends on the sizes only.
struct Plan {
  long BH = 0;  // heads the segment kernels see: B*H, or B*H*ns feature slices of a wide head
  long N = 0;
  int L = 0;
  int nseg = 0;
  int SV = 0;  // floats per state vector: D*M + D (D = 64 for a slice)
  int M = 0;
  int ns = 1;  // feature slices per value head (wide feature vectors), else 1
  long BHv() const { return BH / ns; }
};

constexpr long kFineTarget = 1024;  // workgroups of the segment-parallel kernels: finer plan
// About half as many, longer segments: fewer aggregates to sum or scan and
// less set-up per token.  The non-causal ops (no running state between
// segments, only totals that every workgroup needs) and the decayed
// recurrence (no grouping of segments in its backward) always plan this way
// (measured: 800-frame speech encoder 26.7 -> 28.9 M tokens/s, gated 2^16
// sequence 72.0 -> 75.9 M tokens/s), and so do the causal ops except on short
// sequences of small states (measured per step: 16-layer 3072-token stack
// 927 -> 889 us, 2^16-token sequence 709 -> 691 us, 784-token layer with 64
// features 186 -> 180 us; the 784-token layer at D = M = 32 keeps the finer
// plan, 96 against 101 us, its aggregate kernels running four to five
// workgroups per compute unit over only a few segments per head).
constexpr long kFineTargetNC = 512;

// The causal ops' target; never below the other ops', so la_checkpoint_size
// bounds the decayed recurrence's checkpoint too.
long causal_target(long nchunks, int D, int M) {
  return nchunks <= 16 && (long)D * M <= 1024 ? kFineTarget : kFineTargetNC;
}

int opt_chunks(const la_options* o) { return o && o->segment_chunks > 0 ? o->segment_chunks : 0; }

// target 0: the causal ops' rule; forced > 0: segments of that many chunks
Plan make_plan(int B, int H, int N, int D, int M, long target, int forced) {
  Plan p;
  p.BH = (long)B * H;
  p.N = N;
  p.SV = D * M + D;
  p.M = M;
  const long nchunks = ((long)N + la::CH - 1) / la::CH;
  if (target <= 0) target = causal_target(nchunks, D, M);
  if (N <= 0) {
    p.L = la::CH;
    p.nseg = 0;
    return p;
  }
  long segs = (target + p.BH - 1) / p.BH;
  if (segs > nchunks) segs = nchunks;
  if (segs < 1) segs = 1;
  long cps = (nchunks + segs - 1) / segs;
  if (forced > 0) cps = forced < nchunks ? forced : nchunks;
  p.L = (int)(cps * la::CH);
  p.nseg = (int)(((long)N + p.L - 1) / p.L);
  return p;
}

// Wide feature vectors (D > 64, a multiple of 64): the plan of the D / 64
// feature slices of every head, each a 64-feature head of its own.
bool is_wide(int D) { return D > 64; }

Plan plan_for(int B, int H, int N, int D, int M, long target, int forced) {
  if (!is_wide(D)) return make_plan(B, H, N, D, M, target, forced);
  Plan p = make_plan(B, H * (D / 64), N, 64, M, target, forced);
  p.ns = D / 64;
  return p;
}

// The consumers of segment aggregates need prefix (or suffix) sums over
// them.  When the aggregates are small, every consumer workgroup sums the
// ones it needs (reading on average nseg / 2 of them, all of its threads
// with many loads in flight); beyond about 64 KiB per workgroup a separate
// scan kernel forms all prefix sums once.
bool use_scan(const Plan& p) { return (size_t)p.nseg * p.SV * sizeof(float) / 2 > (64u << 10); }

// Compute units of the current device (cached per device; 256 on MI355X).
long device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
  std::atomic<int>& c = cache[dev < 64 ? dev : 63];
  int n = c.load(std::memory_order_relaxed);
  if (n <= 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    c.store(n, std::memory_order_relaxed);
  }
  return n;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

size_t state_bytes(const Plan& p, long entries) { return align256((size_t)p.BH * entries * p.SV * sizeof(float)); }

// Workspace regions (bytes) per operation.
struct WsLayout {
  size_t agg = 0, ckpt = 0, ragg = 0, rpref = 0, dlam = 0, gc = 0, xseg = 0, sync = 0;
  size_t pn = 0, pd = 0;  // wide feature vectors: the slices' shares
  size_t bytes() const { return agg + ckpt + ragg + rpref + dlam + gc + xseg + sync + pn + pd; }
};

// Wide feature vectors, per slice head: the share of the numerators ([N][M];
// in the backward, of dV), and of the denominators ([N]; in the backward, the
// pair of shares that forms (1/den, O.dO), [N] float2).
size_t wide_pn(const Plan& p) { return align256((size_t)p.BH * p.N * p.M * sizeof(float)); }
size_t wide_pd(const Plan& p, size_t per) { return align256((size_t)p.BH * p.N * per); }

// fwd causal: aggregates and prefix states when there is more than one
//   segment (the prefix states go to the caller's checkpoint when given and
//   are only formed by the scan kernel), and the one-pass forward's error
//   word and flags;
// fwd non-causal: aggregates and their scan (its last entry is the total);
// bwd non-causal: both for the key side and for the reverse side;
// bwd: aggregates and prefix states to recompute a missing checkpoint, the
//   reverse aggregates (scanned in place) when there is more than one
//   segment, and the per-token pair (1/den, O.dO) passed from the query
//   pass to the key pass.
// Wide feature vectors add the slices' shares of the forward's numerators and
// denominators, and in the backward those of dV and of the pair (1/den,
// O.dO).
WsLayout ws_layout(int op, const Plan& p) {
  WsLayout w;
  if (p.nseg == 0) return w;
  const bool wide = p.ns > 1;
  switch (op) {
    case LA_OP_FWD_CAUSAL:
      if (p.nseg > 1) {
        w.agg = state_bytes(p, p.nseg);
        w.ckpt = state_bytes(p, p.nseg + 1);
        if (!wide) w.sync = align256((size_t)(1 + p.BH * p.nseg) * sizeof(unsigned));
      }
      if (wide) {
        w.pn = wide_pn(p);
        w.pd = wide_pd(p, sizeof(float));
      }
      break;
    case LA_OP_FWD_NONCAUSAL:
      w.agg = state_bytes(p, p.nseg);
      w.ckpt = state_bytes(p, p.nseg + 1);
      if (wide) {
        w.pn = wide_pn(p);
        w.pd = wide_pd(p, sizeof(float));
      }
      break;
    case LA_OP_BWD_CAUSAL:
      w.agg = state_bytes(p, p.nseg);       // checkpoint recomputation only
      w.ckpt = state_bytes(p, p.nseg + 1);  // checkpoint recomputation only
      if (p.nseg > 1) w.ragg = state_bytes(p, p.nseg);
      w.gc = align256((size_t)p.BHv() * p.N * 2 * sizeof(float));  // (1/den, O.dO) per token
      if (wide) {
        w.pn = wide_pn(p);                     // dV shares
        w.pd = wide_pd(p, 2 * sizeof(float));  // shares of (num . dO, den)
      }
      break;
    case LA_OP_BWD_NONCAUSAL:  // key aggregates and their scan; reverse aggregates and their scan
      w.agg = state_bytes(p, p.nseg);
      w.ckpt = state_bytes(p, p.nseg + 1);
      w.ragg = state_bytes(p, p.nseg);
      w.rpref = state_bytes(p, p.nseg + 1);
      if (wide) {
        w.gc = align256((size_t)p.BHv() * p.N * 2 * sizeof(float));  // (1/den, O.dO) per token
        w.pn = wide_pn(p);                                            // dV shares
        w.pd = wide_pd(p, 2 * sizeof(float));                         // shares of (num . dO, den)
      }
      break;
    case LA_OP_FWD_DECAY:  // aggregates, per-segment log-decay sums and the prefix states
      if (p.nseg > 1) {
        w.agg = state_bytes(p, p.nseg);
        w.ckpt = state_bytes(p, p.nseg + 1);
        w.dlam = align256((size_t)p.BH * p.nseg * sizeof(float));
      }
      break;
    case LA_OP_BWD_DECAY:  // checkpoint recomputation, log-decay sums, reverse aggregates, (1/den, c) per
                           // token, per-segment totals of the dlogA terms
      w.agg = state_bytes(p, p.nseg);
      w.ckpt = state_bytes(p, p.nseg + 1);
      w.dlam = align256((size_t)p.BH * p.nseg * sizeof(float));
      w.ragg = state_bytes(p, p.nseg);
      w.gc = align256((size_t)p.BH * p.N * 2 * sizeof(float));
      w.xseg = align256((size_t)p.BH * p.nseg * sizeof(float));
      break;
    default:
      break;
  }
  return w;
}

// -------------------------------------------------------------- validation
bool dims_ok(int D, int M) { return (D == 32 || D == 64) && (M == 32 || M == 64); }
bool wide_ok(int C) { return C > 64 && C <= la::kWideMax && C % 64 == 0; }

int check_sizes(int B, int H, int N, int D, int M, int dtype) {
  if (dtype != LA_F32 && dtype != LA_BF16) return fail(LA_ERR_DTYPE, "dtype must be LA_F32 (0) or LA_BF16 (1)");
  if (B < 1 || H < 1 || N < 0) return fail(LA_ERR_SHAPE, "need B >= 1, H >= 1, N >= 0");
  if (!dims_ok(D, M) && !(wide_ok(D) && (M == 32 || M == 64)))
    return fail(LA_ERR_UNSUPPORTED, "D must be 32, 64 or a multiple of 64 up to 4096 (wide feature vectors) and M "
                                    "32 or 64");
  const double elems = (double)B * H * (double)N * (D > M ? D : M);
  if (elems > 4.0e18 || (double)B * H * (N > 0 ? N : 1) > 2.0e9) return fail(LA_ERR_SHAPE, "sizes overflow");
  return LA_OK;
}

// Wide feature vectors come from a feature map: they are used as they are
// (LA_FEATURE_IDENTITY), without a decay.
int check_wide(int D, int feature, const float* logA) {
  if (!is_wide(D)) return LA_OK;
  if (feature != LA_FEATURE_IDENTITY)
    return fail(LA_ERR_UNSUPPORTED, "D > 64 (wide feature vectors) needs feature = LA_FEATURE_IDENTITY");
  if (logA) return fail(LA_ERR_UNSUPPORTED, "D > 64 (wide feature vectors) has no decayed form");
  return LA_OK;
}

int check_opts(const la_options* o) {
  if (!o) return LA_OK;
  if (o->segment_chunks < 0) return fail(LA_ERR_ARG, "opts->segment_chunks must be >= 0");
  if (o->forward_form < LA_FORM_AUTO || o->forward_form > LA_FORM_ONE_LAUNCH)
    return fail(LA_ERR_ARG, "opts->forward_form must be LA_FORM_AUTO, LA_FORM_TWO_LAUNCH or LA_FORM_ONE_LAUNCH");
  if (o->timed_kernel && (!o->events || !o->events_used || o->event_pairs < 0))
    return fail(LA_ERR_ARG, "opts->timed_kernel needs events, event_pairs >= 0 and events_used");
  if (o->status && reinterpret_cast<uintptr_t>(o->status) % 4)
    return fail(LA_ERR_ALIGN, "opts->status is not 4-byte aligned");
  return LA_OK;
}

struct Range {
  const char* name;
  uintptr_t lo, hi;  // [lo, hi)
  bool output;
};

int check_ptrs(const std::vector<Range>& rs) {
  for (const Range& r : rs) {
    if (r.lo == 0) continue;
    if (r.lo % 16) return fail(LA_ERR_ALIGN, std::string(r.name) + " is not 16-byte aligned");
  }
  for (size_t a = 0; a < rs.size(); ++a) {
    if (!rs[a].output || rs[a].lo == 0 || rs[a].hi <= rs[a].lo) continue;
    for (size_t b = 0; b < rs.size(); ++b) {
      if (a == b || rs[b].lo == 0 || rs[b].hi <= rs[b].lo) continue;
      if (rs[a].lo < rs[b].hi && rs[b].lo < rs[a].hi)
        return fail(LA_ERR_ALIAS, std::string(rs[a].name) + " overlaps " + rs[b].name);
    }
  }
  return LA_OK;
}

Range rng(const char* name, const void* p, size_t bytes, bool out) {
  const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
  return Range{name, lo, lo ? lo + bytes : 0, out};
}

// ------------------------------------------------------------ launching
// What a launch needs besides its arguments: the stream and the caller's
// options (timing events among them).
struct Call {
  hipStream_t s;
  const la_options* o;
};

bool timed(const Call& c, const char* name) {
  const la_options* o = c.o;
  return o && o->timed_kernel && o->events && o->events_used && *o->events_used >= 0 &&
         *o->events_used < o->event_pairs && std::strcmp(o->timed_kernel, name) == 0;
}

template <typename Kern, typename... Args>
int launch(const char* name, Kern kern, dim3 grid, dim3 block, const Call& c, Args... args) {
  if (grid.x == 0 || grid.y == 0 || grid.z == 0) return LA_OK;
  const bool ev = timed(c, name);
  hipEvent_t* pair = ev ? reinterpret_cast<hipEvent_t*>(c.o->events) + 2 * (*c.o->events_used) : nullptr;
  if (ev && hipEventRecord(pair[0], c.s) != hipSuccess) return fail(LA_ERR_HIP, std::string(name) + ": event record");
  hipLaunchKernelGGL(kern, grid, block, 0, c.s, args...);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(LA_ERR_HIP, std::string(name) + ": " + hipGetErrorString(e));
  if (ev) {
    if (hipEventRecord(pair[1], c.s) != hipSuccess) return fail(LA_ERR_HIP, std::string(name) + ": event record");
    ++*c.o->events_used;
  }
  return LA_OK;
}

// ------------------------------------------------------------- dispatch
#define LA_DISPATCH(dtype, D, M, FN, ...)                                                        \
  do {                                                                                           \
    if ((dtype) == LA_F32) {                                                                     \
      if ((D) == 32 && (M) == 32) return FN<float, 32, 32>(__VA_ARGS__);                         \
      if ((D) == 32 && (M) == 64) return FN<float, 32, 64>(__VA_ARGS__);                         \
      if ((D) == 64 && (M) == 32) return FN<float, 64, 32>(__VA_ARGS__);                         \
      return FN<float, 64, 64>(__VA_ARGS__);                                                     \
    } else {                                                                                     \
      if ((D) == 32 && (M) == 32) return FN<la::bf16_t, 32, 32>(__VA_ARGS__);                    \
      if ((D) == 32 && (M) == 64) return FN<la::bf16_t, 32, 64>(__VA_ARGS__);                    \
      if ((D) == 64 && (M) == 32) return FN<la::bf16_t, 64, 32>(__VA_ARGS__);                    \
      return FN<la::bf16_t, 64, 64>(__VA_ARGS__);                                                \
    }                                                                                            \
  } while (0)

char* region(void* ws, size_t off) { return static_cast<char*>(ws) + off; }

dim3 scan_grid(const Plan& p) { return dim3((unsigned)p.BH, (unsigned)((p.SV + la::NT - 1) / la::NT)); }

template <typename T, int D, int M>
int seg_aggregates(const Plan& p, const void* K, const void* V, float* agg, int N, int fm, const Call& s) {
  return launch("seg_state", la::k_seg_state<T, D, M>, dim3((unsigned)(p.BH * p.nseg)), dim3(la::NT), s,
                (const T*)K, (const T*)V, agg, N, p.L, p.nseg, fm, p.ns);
}

template <int D, int M>
int scan_prefix(const Plan& p, const float* agg, const float* S0, const float* Z0, float* pref, const Call& s,
                int last_only = 0) {
  return launch("scan_states", la::k_scan_states<D, M>, scan_grid(p), dim3(la::NT), s, agg, S0, Z0, pref, p.nseg,
                last_only);
}

// The one-pass forward (k_fwd_lb) can serve segments of at most four chunks
// whose aggregates every workgroup sums itself.  It saves the aggregate pass
// but adds a launch that clears its flags and, at the end of every
// workgroup, the round trips of publishing and reading aggregates between
// XCDs; it is chosen for states of D*M >= 2048, where the aggregate pass
// costs more than that (measured per 784-token layer of 16x8 heads, float32:
// D = 64, M = 32: 48.0 -> 40.6 us; D = M = 32: 33.4 -> 37.4 us, and 21.2 ->
// 25.6 us per 3072-token bf16 layer of 4x8 heads, so those keep two launches).
// The automatic rule also requires the whole grid to be resident at once, so
// that no wait depends on the order in which workgroups are dispatched.
// la_options::forward_form: LA_FORM_AUTO by this rule (the default),
// LA_FORM_TWO_LAUNCH never, LA_FORM_ONE_LAUNCH wherever the segments allow.
// Polls of a one-launch forward's wait for an earlier segment's flag before
// it gives up (each poll waits for a device-scope load of about a
// microsecond, so 2^22 polls are a few seconds): la_options::wait_polls.
constexpr int kDefaultPolls = 1 << 22;
int opt_polls(const la_options* o) { return !o || o->wait_polls == 0 ? kDefaultPolls : o->wait_polls < 0 ? 0 : o->wait_polls; }

// workgroups of the one-launch forward resident per compute unit
template <typename T, int D, int M, int NC>
int onepass_resident() {
  static const int n = [] {
    int r = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&r, la::k_fwd_lb<T, D, M, NC>, la::NT, 0) != hipSuccess)
      r = 0;
    return r;
  }();
  return n;
}

template <typename T, int D, int M>
bool use_onepass(const Plan& p, const la_options* o) {
  const int mode = o ? o->forward_form : LA_FORM_AUTO;
  if (mode == LA_FORM_TWO_LAUNCH || p.nseg <= 1 || p.L > 4 * la::CH || use_scan(p)) return false;
  if (mode == LA_FORM_ONE_LAUNCH) return true;
  const int resident = p.L <= 2 * la::CH ? onepass_resident<T, D, M, 2>() : onepass_resident<T, D, M, 4>();
  return D * M >= 2048 && p.BH * p.nseg <= (long)resident * device_cus();
}

template <typename T, int D, int M, int NC>
int fwd_onepass(const Plan& p, const void* Q, const void* K, const void* V, void* O, float* den, const float* S0,
                const float* Z0, float* S_out, float* Z_out, float* ckpt, int N, void* ws, int fm, const Call& s) {
  const WsLayout wl = ws_layout(LA_OP_FWD_CAUSAL, p);
  float* agg = reinterpret_cast<float*>(region(ws, 0));
  unsigned* sync = reinterpret_cast<unsigned*>(region(ws, wl.agg + wl.ckpt));
  const int nsync = (int)(1 + p.BH * p.nseg);
  int st = launch("sync_clear", la::k_sync_clear, dim3((unsigned)std::min(64, (nsync + la::NT - 1) / la::NT)),
                  dim3(la::NT), s, sync, nsync);
  if (st) return st;
  return launch("fwd_causal", la::k_fwd_lb<T, D, M, NC>, dim3((unsigned)(p.BH * p.nseg)), dim3(la::NT), s,
                (const T*)Q, (const T*)K, (const T*)V, (T*)O, den, S0, Z0, agg, sync, ckpt, S_out, Z_out, N, p.L,
                p.nseg, fm, opt_polls(s.o), s.o ? s.o->status : (unsigned*)nullptr);
}

template <typename T, int D, int M>
int fwd_causal_impl(const Plan& p, const void* Q, const void* K, const void* V, void* O, float* den, const float* S0,
                    const float* Z0, float* S_out, float* Z_out, float* ckpt, int N, void* ws, int fm, const Call& s) {
  if (p.nseg == 0)
    return launch("state_copy", la::k_state_copy<D, M>, dim3((unsigned)p.BH), dim3(la::NT), s, S0, Z0, ckpt, S_out,
                  Z_out);
  if (use_onepass<T, D, M>(p, s.o)) {
    if (p.L <= 2 * la::CH)
      return fwd_onepass<T, D, M, 2>(p, Q, K, V, O, den, S0, Z0, S_out, Z_out, ckpt, N, ws, fm, s);
    return fwd_onepass<T, D, M, 4>(p, Q, K, V, O, den, S0, Z0, S_out, Z_out, ckpt, N, ws, fm, s);
  }
  const float* pref = nullptr;
  float* agg = nullptr;
  float* ckw = ckpt;  // checkpoint written by the forward itself unless the scan forms it
  if (p.nseg > 1) {
    const WsLayout wl = ws_layout(LA_OP_FWD_CAUSAL, p);
    agg = reinterpret_cast<float*>(region(ws, 0));
    int st = seg_aggregates<T, D, M>(p, K, V, agg, N, fm, s);
    if (st) return st;
    if (use_scan(p)) {
      float* pr = ckpt ? ckpt : reinterpret_cast<float*>(region(ws, wl.agg));
      st = scan_prefix<D, M>(p, agg, S0, Z0, pr, s);
      if (st) return st;
      pref = pr;
      ckw = nullptr;
    }
  }
  return launch("fwd_causal", la::k_fwd<T, D, M, true>, dim3((unsigned)(p.BH * p.nseg)), dim3(la::NT), s,
                (const T*)Q, (const T*)K, (const T*)V, (T*)O, den, pref, (const float*)agg, S0, Z0, ckw, S_out,
                Z_out, N, p.L, p.nseg, fm, 1, (float*)nullptr);
}

template <typename T, int D, int M>
int fwd_noncausal_impl(const Plan& p, const void* Q, const void* K, const void* V, void* O, float* S_out,
                       float* Z_out, int N, void* ws,
                       int fm, const Call& s) {
  if (p.nseg == 0)  // empty sequence: zero totals
    return S_out ? launch("state_copy", la::k_state_copy<D, M>, dim3((unsigned)p.BH), dim3(la::NT), s,
                          (const float*)nullptr, (const float*)nullptr, (float*)nullptr, S_out, Z_out)
                 : LA_OK;
  const WsLayout wl = ws_layout(LA_OP_FWD_NONCAUSAL, p);
  float* agg = reinterpret_cast<float*>(region(ws, 0));
  int st = seg_aggregates<T, D, M>(p, K, V, agg, N, fm, s);
  if (st) return st;
  const float* pref = nullptr;
  if (use_scan(p)) {  // the total once per head (else every workgroup sums the aggregates)
    float* pr = reinterpret_cast<float*>(region(ws, wl.agg));
    st = scan_prefix<D, M>(p, agg, nullptr, nullptr, pr, s, 1);
    if (st) return st;
    pref = pr;
  }
  return launch("fwd_noncausal", la::k_fwd<T, D, M, false>, dim3((unsigned)(p.BH * p.nseg)), dim3(la::NT), s,
                (const T*)Q, (const T*)K, (const T*)V, (T*)O, (float*)nullptr, pref, (const float*)agg,
                (const float*)nullptr, (const float*)nullptr, (float*)nullptr, S_out, Z_out, N,
                p.L, p.nseg, fm, 1, (float*)nullptr);
}

template <typename T, int D, int M>
int bwd_causal_impl(const Plan& p, const void* Q, const void* K, const void* V, const void* O, const float* den,
                    const void* dO, const float* S0, const float* Z0, const float* ckpt, const float* dSN,
                    const float* dZN, void* dQ, void* dK, void* dV, float* dS0, float* dZ0, int N, void* ws,
                    int fm, const Call& s) {
  (void)O;  // the query pass recomputes den and O.dO from the forward states (see la_bwd2.h)
  (void)den;
  if (p.nseg == 0)  // empty sequence: the initial state is the final state
    return dS0 ? launch("state_copy", la::k_state_copy<D, M>, dim3((unsigned)p.BH), dim3(la::NT), s, dSN, dZN,
                        (float*)nullptr, dS0, dZ0)
               : LA_OK;
  const WsLayout wl = ws_layout(LA_OP_BWD_CAUSAL, p);
  int st = LA_OK;
  const float* ck = ckpt;
  if (!ck) {  // recompute the checkpoint: aggregates, then their scan
    float* agg = reinterpret_cast<float*>(region(ws, 0));
    float* ckw = reinterpret_cast<float*>(region(ws, wl.agg));
    st = seg_aggregates<T, D, M>(p, K, V, agg, N, fm, s);
    if (st) return st;
    st = scan_prefix<D, M>(p, agg, S0, Z0, ckw, s);
    if (st) return st;
    ck = ckw;
  }
  float* ragg = p.nseg > 1 ? reinterpret_cast<float*>(region(ws, wl.agg + wl.ckpt)) : nullptr;
  float2* gc = reinterpret_cast<float2*>(region(ws, wl.agg + wl.ckpt + wl.ragg));
  const dim3 grid((unsigned)(p.BH * p.nseg));
  st = launch("bwd_query", la::k_bq<T, D, M>, grid, dim3(la::NT), s, (const T*)Q, (const T*)K, (const T*)V,
              (const T*)dO, ck, (T*)dQ, gc, ragg, N, p.L, p.nseg, fm, 1);
  if (st) return st;
  const int scanned = p.nseg > 1 && use_scan(p) ? 1 : 0;
  if (scanned) {
    st = launch("scan_rev", la::k_scan_rev<D, M>, scan_grid(p), dim3(la::NT), s, ragg, p.nseg);
    if (st) return st;
  }
  return launch("bwd_kv", la::k_bkv<T, D, M>, grid, dim3(la::NT), s, (const T*)Q, (const T*)K, (const T*)V,
                (const T*)dO, (const float2*)gc, (const float*)ragg, dSN, dZN, (T*)dK, (T*)dV, dS0, dZ0, N, p.L,
                p.nseg, scanned, fm, 1, (float*)nullptr);
}

template <typename T, int D, int M>
int bwd_noncausal_impl(const Plan& p, const void* Q, const void* K, const void* V, const void* dO,
                       const float* St, const float* Zt, void* dQ, void* dK, void* dV, int N, void* ws, int fm, const Call& s) {
  if (p.nseg == 0) return LA_OK;
  const WsLayout wl = ws_layout(LA_OP_BWD_NONCAUSAL, p);
  float* agg = reinterpret_cast<float*>(region(ws, 0));
  float* pref = reinterpret_cast<float*>(region(ws, wl.agg));
  float* ragg = reinterpret_cast<float*>(region(ws, wl.agg + wl.ckpt));
  float* rpref = reinterpret_cast<float*>(region(ws, wl.agg + wl.ckpt + wl.ragg));
  const bool scan = use_scan(p);  // the totals once per head (else every workgroup sums the aggregates)
  int st = LA_OK;
  if (!St) {  // key totals: the forward's when given, else recomputed
    st = seg_aggregates<T, D, M>(p, K, V, agg, N, fm, s);
    if (st) return st;
    if (scan) {
      st = scan_prefix<D, M>(p, agg, nullptr, nullptr, pref, s, 1);
      if (st) return st;
    }
  }
  const dim3 grid((unsigned)(p.BH * p.nseg));
  st = launch("nc_qr", la::k_nc_qr<T, D, M>, grid, dim3(la::NT), s, (const T*)Q, (const T*)dO, St, Zt,
              (const float*)(St ? nullptr : agg), (const float*)(scan && !St ? pref : nullptr), (T*)dQ, ragg, N, p.L,
              p.nseg, fm, 1, (float2*)nullptr);
  if (st) return st;
  if (scan) {
    st = scan_prefix<D, M>(p, ragg, nullptr, nullptr, rpref, s, 1);
    if (st) return st;
  }
  return launch("nc_kv", la::k_nc_kv<T, D, M>, grid, dim3(la::NT), s, (const T*)K, (const T*)V, (const float*)ragg,
                (const float*)(scan ? rpref : nullptr), (T*)dK, (T*)dV, N, p.L, p.nseg, fm, 1, (float*)nullptr);
}

// ----------------------------------------------------- decayed recurrence
template <typename T, int D, int M>
int fwd_decay_impl(const Plan& p, const void* Q, const void* K, const void* V, const float* logA, void* O,
                   float* den, const float* S0, const float* Z0, float* S_out, float* Z_out, float* ckpt, int N,
                   void* ws, int fm, const Call& s) {
  if (p.nseg == 0)
    return launch("state_copy", la::k_state_copy<D, M>, dim3((unsigned)p.BH), dim3(la::NT), s, S0, Z0, ckpt, S_out,
                  Z_out);
  const float* pref = nullptr;
  if (p.nseg > 1) {  // segment aggregates and their decayed prefix states (into the checkpoint when given)
    const WsLayout wl = ws_layout(LA_OP_FWD_DECAY, p);
    float* agg = reinterpret_cast<float*>(region(ws, 0));
    float* dlam = reinterpret_cast<float*>(region(ws, wl.agg + wl.ckpt));
    int st = launch("dseg_state", la::k_dseg_state<T, D, M>, dim3((unsigned)(p.BH * p.nseg)), dim3(la::NT), s,
                    (const T*)K, (const T*)V, logA, agg, dlam, N, p.L, p.nseg, fm);
    if (st) return st;
    float* pr = ckpt ? ckpt : reinterpret_cast<float*>(region(ws, wl.agg));
    st = launch("dscan_states", la::k_dscan_states<D, M>, scan_grid(p), dim3(la::NT), s, (const float*)agg,
                (const float*)dlam, S0, Z0, pr, p.nseg);
    if (st) return st;
    pref = pr;
  }
  return launch("dfwd", la::k_dfwd<T, D, M>, dim3((unsigned)(p.BH * p.nseg)), dim3(la::NT), s, (const T*)Q,
                (const T*)K, (const T*)V, logA, (T*)O, den, pref, S0, Z0, pref ? (float*)nullptr : ckpt, S_out, Z_out,
                N, p.L, p.nseg, fm);
}

template <typename T, int D, int M>
int bwd_decay_impl(const Plan& p, const void* Q, const void* K, const void* V, const float* logA, const void* dO,
                   const float* S0, const float* Z0, const float* ckpt, const float* dSN, const float* dZN, void* dQ,
                   void* dK, void* dV, float* dlogA, float* dS0, float* dZ0, int N, void* ws, int fm, const Call& s) {
  if (p.nseg == 0)
    return dS0 ? launch("state_copy", la::k_state_copy<D, M>, dim3((unsigned)p.BH), dim3(la::NT), s, dSN, dZN,
                        (float*)nullptr, dS0, dZ0)
               : LA_OK;
  const WsLayout wl = ws_layout(LA_OP_BWD_DECAY, p);
  float* agg = reinterpret_cast<float*>(region(ws, 0));
  float* ckw = reinterpret_cast<float*>(region(ws, wl.agg));
  float* dlam = reinterpret_cast<float*>(region(ws, wl.agg + wl.ckpt));
  float* ragg = reinterpret_cast<float*>(region(ws, wl.agg + wl.ckpt + wl.dlam));
  float2* gc = reinterpret_cast<float2*>(region(ws, wl.agg + wl.ckpt + wl.dlam + wl.ragg));
  float* xseg = reinterpret_cast<float*>(region(ws, wl.agg + wl.ckpt + wl.dlam + wl.ragg + wl.gc));
  const dim3 grid((unsigned)(p.BH * p.nseg));
  int st = LA_OK;
  const float* ck = ckpt;
  if (!ck) {  // recompute the checkpoint
    st = launch("dseg_state", la::k_dseg_state<T, D, M>, grid, dim3(la::NT), s, (const T*)K, (const T*)V, logA, agg,
                dlam, N, p.L, p.nseg, fm);
    if (st) return st;
    st = launch("dscan_states", la::k_dscan_states<D, M>, scan_grid(p), dim3(la::NT), s, (const float*)agg,
                (const float*)dlam, S0, Z0, ckw, p.nseg);
    if (st) return st;
    ck = ckw;
  }
  st = launch("dbq", la::k_dbq<T, D, M>, grid, dim3(2 * la::NT), s, (const T*)Q, (const T*)K, (const T*)V, (const T*)dO,
              logA, ck, (T*)dQ, gc, ragg, dlam, N, p.L, p.nseg, fm);
  if (st) return st;
  st = launch("dscan_rev", la::k_dscan_rev<D, M>, scan_grid(p), dim3(la::NT), s, ragg, (const float*)dlam, dSN, dZN,
              dS0, dZ0, p.nseg);
  if (st) return st;
  st = launch("dbkv", la::k_dbkv<T, D, M>, grid, dim3(2 * la::NT), s, (const T*)Q, (const T*)K, (const T*)V,
              (const T*)dO, logA, (const float2*)gc, (const float*)ragg, ck, dSN, dZN, (T*)dK, (T*)dV, dlogA, xseg, N,
              p.L, p.nseg, fm);
  if (st) return st;
  if (p.nseg == 1) return LA_OK;
  return launch("dla_fix", la::k_dla_fix, grid, dim3(la::NT), s, dlogA, (const float*)xseg, N, p.L, p.nseg);
}

template <typename T, int D, int M>
int decode_impl(long BH, const void* q, const void* k, const void* v, const float* logA, float* S, float* Z, void* y,
                int fm, const Call& s) {
  return launch("decode", la::k_decode<T, D, M>, dim3((unsigned)((BH + 3) / 4)), dim3(la::NT), s, (const T*)q,
                (const T*)k, (const T*)v, logA, S, Z, (T*)y, (int)BH, fm);
}

// ------------------------------------------------- wide feature vectors
// Feature slices run as 64-feature heads of the chunked kernels (la_wide.h);
// the sums over slices follow.  The checkpoint of a wide forward is the
// slices' states (S [B,H,D,M] is the same memory as [B H ns, 64, M]).
size_t ckpt_bytes(const Plan& p) { return (size_t)p.BH * (p.nseg + 1) * p.SV * sizeof(float); }

template <int M>
dim3 token_grid(long rows) { return dim3((unsigned)((rows * (M / 4) + la::NT - 1) / la::NT)); }

template <typename T, int M>
int fwd_wide_impl(const Plan& p, bool causal, const void* Q, const void* K, const void* V, void* O, float* den,
                  const float* S0, const float* Z0, float* S_out, float* Z_out, float* ckpt, int N, void* ws, int fm,
                  const Call& s) {
  if (p.nseg == 0) {
    if (!causal)
      return S_out ? launch("state_copy", la::k_state_copy<64, M>, dim3((unsigned)p.BH), dim3(la::NT), s,
                            (const float*)nullptr, (const float*)nullptr, (float*)nullptr, S_out, Z_out)
                   : LA_OK;
    return launch("state_copy", la::k_state_copy<64, M>, dim3((unsigned)p.BH), dim3(la::NT), s, S0, Z0, ckpt, S_out,
                  Z_out);
  }
  const WsLayout wl = ws_layout(causal ? LA_OP_FWD_CAUSAL : LA_OP_FWD_NONCAUSAL, p);
  float* agg = nullptr;
  const float* pref = nullptr;
  float* ckw = causal ? ckpt : nullptr;
  int st = LA_OK;
  if (p.nseg > 1 || !causal) {
    agg = reinterpret_cast<float*>(region(ws, 0));
    st = seg_aggregates<T, 64, M>(p, K, V, agg, N, fm, s);
    if (st) return st;
    if (use_scan(p)) {
      float* pr = causal && ckpt ? ckpt : reinterpret_cast<float*>(region(ws, wl.agg));
      st = scan_prefix<64, M>(p, agg, causal ? S0 : nullptr, causal ? Z0 : nullptr, pr, s, causal ? 0 : 1);
      if (st) return st;
      pref = pr;
      ckw = nullptr;
    }
  }
  float* pnum = reinterpret_cast<float*>(region(ws, wl.agg + wl.ckpt + wl.sync));
  float* pden = reinterpret_cast<float*>(region(ws, wl.agg + wl.ckpt + wl.sync + wl.pn));
  const dim3 grid((unsigned)(p.BH * p.nseg));
  if (causal)
    st = launch("fwd_causal", la::k_fwd<T, 64, M, true, true>, grid, dim3(la::NT), s, (const T*)Q, (const T*)K,
                (const T*)V, (T*)nullptr, pden, pref, (const float*)agg, S0, Z0, ckw, S_out, Z_out, N, p.L, p.nseg, fm,
                p.ns, pnum);
  else
    st = launch("fwd_noncausal", la::k_fwd<T, 64, M, false, true>, grid, dim3(la::NT), s, (const T*)Q, (const T*)K,
                (const T*)V, (T*)nullptr, pden, pref, (const float*)agg, (const float*)nullptr,
                (const float*)nullptr, (float*)nullptr, S_out, Z_out, N, p.L, p.nseg, fm, p.ns, pnum);
  if (st) return st;
  const long rows = p.BHv() * N;
  return launch("wide_combine", la::k_wide_combine<T, M>, token_grid<M>(rows), dim3(la::NT), s, (const float*)pnum,
                (const float*)pden, (T*)O, den, rows, N, p.ns);
}

template <typename T, int M>
int bwd_wide_impl(const Plan& p, const void* Q, const void* K, const void* V, const void* dO, const float* S0,
                  const float* Z0, const float* ckpt, const float* dSN, const float* dZN, void* dQ, void* dK, void* dV,
                  float* dS0, float* dZ0, int N, void* ws, int fm, const Call& s) {
  if (p.nseg == 0)
    return dS0 ? launch("state_copy", la::k_state_copy<64, M>, dim3((unsigned)p.BH), dim3(la::NT), s, dSN, dZN,
                        (float*)nullptr, dS0, dZ0)
               : LA_OK;
  const WsLayout wl = ws_layout(LA_OP_BWD_CAUSAL, p);
  float* ragg = p.nseg > 1 ? reinterpret_cast<float*>(region(ws, wl.agg + wl.ckpt)) : nullptr;
  float2* gc = reinterpret_cast<float2*>(region(ws, wl.agg + wl.ckpt + wl.ragg));
  float* pn = reinterpret_cast<float*>(region(ws, wl.agg + wl.ckpt + wl.ragg + wl.gc));
  float2* sh = reinterpret_cast<float2*>(region(ws, wl.agg + wl.ckpt + wl.ragg + wl.gc + wl.pn));
  const long rows = p.BHv() * N;
  const dim3 grid((unsigned)(p.BH * p.nseg));
  int st = LA_OK;
  const float* ck = ckpt;
  if (!ck) {  // recompute the checkpoint: the slices' aggregates, then their scan
    float* agg = reinterpret_cast<float*>(region(ws, 0));
    float* ckw = reinterpret_cast<float*>(region(ws, wl.agg));
    st = seg_aggregates<T, 64, M>(p, K, V, agg, N, fm, s);
    if (st) return st;
    st = scan_prefix<64, M>(p, agg, S0, Z0, ckw, s);
    if (st) return st;
    ck = ckw;
  }
  // every slice's shares of (num . dO, den), their sums per token, then the query pass proper
  st = launch("bwd_query_shares", la::k_bq<T, 64, M, la::kBqShares>, grid, dim3(la::NT), s, (const T*)Q,
              (const T*)K, (const T*)V, (const T*)dO, ck, (T*)nullptr, sh, (float*)nullptr, N, p.L, p.nseg, fm, p.ns);
  if (st) return st;
  st = launch("wide_pairs", la::k_wide_pairs, dim3((unsigned)((rows + la::NT - 1) / la::NT)), dim3(la::NT), s,
              (const float2*)sh, gc, rows, N, p.ns);
  if (st) return st;
  st = launch("bwd_query", la::k_bq<T, 64, M, la::kBqGiven>, grid, dim3(la::NT), s, (const T*)Q, (const T*)K,
              (const T*)V, (const T*)dO, ck, (T*)dQ, gc, ragg, N, p.L, p.nseg, fm, p.ns);
  if (st) return st;
  const int scanned = p.nseg > 1 && use_scan(p) ? 1 : 0;
  if (scanned) {
    st = launch("scan_rev", la::k_scan_rev<64, M>, scan_grid(p), dim3(la::NT), s, ragg, p.nseg);
    if (st) return st;
  }
  st = launch("bwd_kv", la::k_bkv<T, 64, M, true>, grid, dim3(la::NT), s, (const T*)Q, (const T*)K, (const T*)V,
              (const T*)dO, (const float2*)gc, (const float*)ragg, dSN, dZN, (T*)dK, (T*)nullptr, dS0, dZ0, N, p.L,
              p.nseg, scanned, fm, p.ns, pn);
  if (st) return st;
  return launch("wide_sum", la::k_wide_sum<T, M>, token_grid<M>(rows), dim3(la::NT), s, (const float*)pn, (T*)dV,
                rows, N, p.ns);
}

template <typename T, int M>
int bwd_noncausal_wide_impl(const Plan& p, const void* Q, const void* K, const void* V, const void* dO,
                            const float* St, const float* Zt, void* dQ, void* dK, void* dV, int N, void* ws, int fm,
                            const Call& s) {
  if (p.nseg == 0) return LA_OK;
  const WsLayout wl = ws_layout(LA_OP_BWD_NONCAUSAL, p);
  float* agg = reinterpret_cast<float*>(region(ws, 0));
  float* pref = reinterpret_cast<float*>(region(ws, wl.agg));
  float* ragg = reinterpret_cast<float*>(region(ws, wl.agg + wl.ckpt));
  float* rpref = reinterpret_cast<float*>(region(ws, wl.agg + wl.ckpt + wl.ragg));
  float2* gc = reinterpret_cast<float2*>(region(ws, wl.agg + wl.ckpt + wl.ragg + wl.rpref));
  float* pn = reinterpret_cast<float*>(region(ws, wl.agg + wl.ckpt + wl.ragg + wl.rpref + wl.gc));
  float2* sh = reinterpret_cast<float2*>(region(ws, wl.agg + wl.ckpt + wl.ragg + wl.rpref + wl.gc + wl.pn));
  const bool scan = use_scan(p);
  const long rows = p.BHv() * N;
  int st = LA_OK;
  if (!St) {  // key totals of every slice: the forward's when given, else formed here
    st = seg_aggregates<T, 64, M>(p, K, V, agg, N, fm, s);
    if (st) return st;
    if (scan) {
      st = scan_prefix<64, M>(p, agg, nullptr, nullptr, pref, s, 1);
      if (st) return st;
    }
  }
  const dim3 grid((unsigned)(p.BH * p.nseg));
  const float* ag = St ? nullptr : agg;
  const float* pr = scan && !St ? pref : nullptr;
  // every slice's shares of (num . dO, den), their sums per token, then the query pass proper
  st = launch("nc_qr_shares", la::k_nc_qr<T, 64, M, la::kNcShares>, grid, dim3(la::NT), s, (const T*)Q,
              (const T*)dO, St, Zt, ag, pr, (T*)nullptr, (float*)nullptr, N, p.L, p.nseg, fm, p.ns, sh);
  if (st) return st;
  st = launch("wide_pairs", la::k_wide_pairs, dim3((unsigned)((rows + la::NT - 1) / la::NT)), dim3(la::NT), s,
              (const float2*)sh, gc, rows, N, p.ns);
  if (st) return st;
  st = launch("nc_qr", la::k_nc_qr<T, 64, M, la::kNcGiven>, grid, dim3(la::NT), s, (const T*)Q, (const T*)dO, St, Zt,
              ag, pr, (T*)dQ, ragg, N, p.L, p.nseg, fm, p.ns, gc);
  if (st) return st;
  if (scan) {
    st = scan_prefix<64, M>(p, ragg, nullptr, nullptr, rpref, s, 1);
    if (st) return st;
  }
  st = launch("nc_kv", la::k_nc_kv<T, 64, M, true>, grid, dim3(la::NT), s, (const T*)K, (const T*)V,
              (const float*)ragg, (const float*)(scan ? rpref : nullptr), (T*)dK, (T*)nullptr, N, p.L, p.nseg, fm,
              p.ns, pn);
  if (st) return st;
  return launch("wide_sum", la::k_wide_sum<T, M>, token_grid<M>(rows), dim3(la::NT), s, (const float*)pn, (T*)dV,
                rows, N, p.ns);
}

template <typename T, int M>
int decode_wide_impl(long BH, int C, const void* q, const void* k, const void* v, float* S, float* Z, void* y, int fm,
                     const Call& s) {
  return launch("decode_wide", la::k_decode_wide<T, M>, dim3((unsigned)BH), dim3(la::NT), s, (const T*)q,
                (const T*)k, (const T*)v, S, Z, (T*)y, C, fm);
}

#define LA_WIDE_DISPATCH(dtype, M, FN, ...)                                  \
  do {                                                                       \
    if ((dtype) == LA_F32) {                                                 \
      if ((M) == 32) return FN<float, 32>(__VA_ARGS__);                      \
      return FN<float, 64>(__VA_ARGS__);                                     \
    }                                                                        \
    if ((M) == 32) return FN<la::bf16_t, 32>(__VA_ARGS__);                   \
    return FN<la::bf16_t, 64>(__VA_ARGS__);                                  \
  } while (0)

size_t esize(int dtype) { return dtype == LA_BF16 ? 2 : 4; }

// ----------------------------------------------------------- feature maps
#define LA_FEAT_DISPATCH(dtype, DIN, C, FN, ...)                                                    \
  do {                                                                                             \
    if ((dtype) == LA_F32) {                                                                       \
      if ((DIN) == 32 && (C) == 32) return FN<float, 32, 32>(__VA_ARGS__);                         \
      if ((DIN) == 32 && (C) == 64) return FN<float, 32, 64>(__VA_ARGS__);                         \
      if ((DIN) == 64 && (C) == 32) return FN<float, 64, 32>(__VA_ARGS__);                         \
      return FN<float, 64, 64>(__VA_ARGS__);                                                       \
    } else {                                                                                       \
      if ((DIN) == 32 && (C) == 32) return FN<la::bf16_t, 32, 32>(__VA_ARGS__);                    \
      if ((DIN) == 32 && (C) == 64) return FN<la::bf16_t, 32, 64>(__VA_ARGS__);                    \
      if ((DIN) == 64 && (C) == 32) return FN<la::bf16_t, 64, 32>(__VA_ARGS__);                    \
      return FN<la::bf16_t, 64, 64>(__VA_ARGS__);                                                  \
    }                                                                                              \
  } while (0)

// A random-feature workgroup stages its head's projection once and walks cpw
// consecutive chunks, cpw chosen so that about 1024 workgroups exist (the
// projection is as large as a chunk of X, so one chunk per workgroup would
// stage twice the data it maps).
template <typename T, int DIN, int C>
int feat_rf_impl(long BH, int H, int N, const void* X, const float* W, const void* dPhi, void* out, const Call& s) {
  const long nch = (N + la::CH - 1) / la::CH;
  long cpw = (BH * nch + 1023) / 1024;
  cpw = cpw < 1 ? 1 : cpw > nch ? nch : cpw;
  const dim3 grid((unsigned)(BH * ((nch + cpw - 1) / cpw)));
  if (dPhi)
    return launch("feat_rf_vjp", la::k_feat_rf_vjp<T, DIN, C>, grid, dim3(la::NT), s, (const T*)X, W,
                  (const T*)dPhi, (T*)out, N, H, (int)cpw);
  return launch("feat_rf", la::k_feat_rf<T, DIN, C>, grid, dim3(la::NT), s, (const T*)X, W, (T*)out, N, H, (int)cpw,
                1, (float)(1.0 / std::sqrt((double)C)));
}

// Wide random features (C = 64 ns, feature-sliced output): the forward runs
// one workgroup per slice and group of chunks; the vector-Jacobian product,
// which sums over every feature, walks the slices inside each workgroup.
template <typename T, int DIN>
int feat_rf_wide_impl(long BH, int H, int N, int C, const void* X, const float* W, const void* dPhi, void* out,
                      const Call& s) {
  const int ns = C / 64;
  const float sc = (float)(1.0 / std::sqrt((double)C));
  const long nch = (N + la::CH - 1) / la::CH;
  if (dPhi) {
    constexpr int CPW = sizeof(T) == 2 ? 4 : 2;  // chunks of X resident per workgroup (LDS)
    const dim3 grid((unsigned)(BH * ((nch + CPW - 1) / CPW)));
    return launch("feat_rf_vjp_wide", la::k_feat_rf_vjp_wide<T, DIN, CPW>, grid, dim3(la::NT), s, (const T*)X, W,
                  (const T*)dPhi, (T*)out, N, H, ns, sc);
  }
  long cpw = (BH * ns * nch + 1023) / 1024;
  cpw = cpw < 1 ? 1 : cpw > nch ? nch : cpw;
  const dim3 grid((unsigned)(BH * ns * ((nch + cpw - 1) / cpw)));
  return launch("feat_rf", la::k_feat_rf<T, DIN, 64>, grid, dim3(la::NT), s, (const T*)X, W, (T*)out, N, H, (int)cpw,
                ns, sc);
}

// Wide polynomial features (C = 64 ns, feature-sliced): a workgroup per 64
// tokens of a head writes every slice; the vector-Jacobian product stages
// each token's feature gradient in LDS (as many tokens per workgroup as fit
// 64 KiB, at most 32).
template <typename T>
int feat_poly2_wide_impl(long BH, int N, int din, int C, const void* X, const void* dPhi, void* out, const Call& s) {
  const int ns = C / 64;
  if (dPhi) {
    const long rows = BH * N;
    const int tpw = std::min(32, (int)(la::kPolyVjpLds / ((size_t)C * sizeof(T))));  // tokens per workgroup
    const dim3 grid((unsigned)((rows + tpw - 1) / tpw));
    if (din <= 32)
      return launch("feat_poly2_vjp_wide", la::k_feat_poly2_vjp_wide<T, 32>, grid, dim3(la::NT), s, (const T*)X,
                    (const T*)dPhi, (T*)out, rows, N, din, ns, tpw);
    return launch("feat_poly2_vjp_wide", la::k_feat_poly2_vjp_wide<T, 64>, grid, dim3(la::NT), s, (const T*)X,
                  (const T*)dPhi, (T*)out, rows, N, din, ns, tpw);
  }
  const long ntb = (N + la::CH - 1) / la::CH;
  return launch("feat_poly2_wide", la::k_feat_poly2_wide<T>, dim3((unsigned)(BH * ntb)), dim3(la::NT), s,
                (const T*)X, (T*)out, N, din, ns);
}

template <typename T, int C>
int feat_poly2_impl(long rows, int din, const void* X, const void* dPhi, void* out, const Call& s) {
  const dim3 grid((unsigned)((rows + la::NT - 1) / la::NT));
  if (dPhi)
    return launch("feat_poly2_vjp", la::k_feat_poly2_vjp<T, C>, grid, dim3(la::NT), s, (const T*)X,
                  (const T*)dPhi, (T*)out, rows, din);
  return launch("feat_poly2", la::k_feat_poly2<T, C>, grid, dim3(la::NT), s, (const T*)X, (T*)out, rows, din);
}

int feature_random(const void* X, const float* W, const void* dPhi, void* out, int B, int H, int N, int Din, int C,
                   int dtype, void* stream) {
  g_err.clear();
  int st = check_sizes(B, H, N, 32, 32, dtype);
  if (st) return st;
  if ((Din != 32 && Din != 64) || (C != 32 && C != 64 && !wide_ok(C)))
    return fail(LA_ERR_UNSUPPORTED, "Din must be 32 or 64 and C 32, 64 or a multiple of 64 up to 4096");
  if (N == 0) return LA_OK;
  if (!X || !W || !out) return fail(LA_ERR_NULL, "X, W and the output are required");
  const size_t es = esize(dtype), bh = (size_t)B * H;
  st = check_ptrs({rng("X", X, bh * N * Din * es, false), rng("W", W, (size_t)H * C * Din * 4, false),
                   rng("dPhi", dPhi, bh * N * C * es, false),
                   rng(dPhi ? "dX" : "Phi", out, bh * N * (dPhi ? Din : C) * es, true)});
  if (st) return st;
  const Call call{(hipStream_t)stream, nullptr};
  if (wide_ok(C)) {
    if (dtype == LA_F32)
      return Din == 32 ? feat_rf_wide_impl<float, 32>((long)bh, H, N, C, X, W, dPhi, out, call)
                       : feat_rf_wide_impl<float, 64>((long)bh, H, N, C, X, W, dPhi, out, call);
    return Din == 32 ? feat_rf_wide_impl<la::bf16_t, 32>((long)bh, H, N, C, X, W, dPhi, out, call)
                     : feat_rf_wide_impl<la::bf16_t, 64>((long)bh, H, N, C, X, W, dPhi, out, call);
  }
  LA_FEAT_DISPATCH(dtype, Din, C, feat_rf_impl, (long)bh, H, N, X, W, dPhi, out, call);
}

int feature_poly2(const void* X, const void* dPhi, void* out, int B, int H, int N, int Din, int C, int dtype,
                  void* stream) {
  g_err.clear();
  int st = check_sizes(B, H, N, 32, 32, dtype);
  if (st) return st;
  if (C != 32 && C != 64 && !wide_ok(C))
    return fail(LA_ERR_UNSUPPORTED, "C must be 32, 64 or a multiple of 64 up to 4096");
  if (Din < 1 || Din > 64 || 1 + Din + Din * Din > C)
    return fail(LA_ERR_UNSUPPORTED, "degree-2 features need 1 <= Din <= 64 and 1 + Din + Din^2 <= C");
  if (N == 0) return LA_OK;
  if (!X || !out) return fail(LA_ERR_NULL, "X and the output are required");
  const size_t es = esize(dtype), bh = (size_t)B * H;
  st = check_ptrs({rng("X", X, bh * N * Din * es, false), rng("dPhi", dPhi, bh * N * C * es, false),
                   rng(dPhi ? "dX" : "Phi", out, bh * N * (dPhi ? Din : C) * es, true)});
  if (st) return st;
  const long rows = (long)bh * N;
  if (wide_ok(C)) {
    if (dtype == LA_F32)
      return feat_poly2_wide_impl<float>((long)bh, N, Din, C, X, dPhi, out, Call{(hipStream_t)stream, nullptr});
    return feat_poly2_wide_impl<la::bf16_t>((long)bh, N, Din, C, X, dPhi, out, Call{(hipStream_t)stream, nullptr});
  }
  if (dtype == LA_F32) {
    if (C == 32) return feat_poly2_impl<float, 32>(rows, Din, X, dPhi, out, Call{(hipStream_t)stream, nullptr});
    return feat_poly2_impl<float, 64>(rows, Din, X, dPhi, out, Call{(hipStream_t)stream, nullptr});
  }
  if (C == 32) return feat_poly2_impl<la::bf16_t, 32>(rows, Din, X, dPhi, out, Call{(hipStream_t)stream, nullptr});
  return feat_poly2_impl<la::bf16_t, 64>(rows, Din, X, dPhi, out, Call{(hipStream_t)stream, nullptr});
}

// ------------------------------------------------------- static scratch
// Device address of `scratch` (top of this file) on the current device,
// looked up once per device with that device current.
int scratch_ptr(void** out) {
  constexpr int kMaxDev = 64;
  static std::once_flag once[kMaxDev];
  static void* ptrs[kMaxDev];
  static hipError_t errs[kMaxDev];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev)
    return fail(LA_ERR_HIP, "la_forward_causal_noalloc: no current device");
  std::call_once(once[dev], [dev] { errs[dev] = hipGetSymbolAddress(&ptrs[dev], HIP_SYMBOL(scratch)); });
  if (errs[dev] != hipSuccess || !ptrs[dev])
    return fail(LA_ERR_HIP, std::string("la_forward_causal_noalloc: hipGetSymbolAddress(scratch): ") +
                                hipGetErrorString(errs[dev]));
  *out = ptrs[dev];
  return LA_OK;
}

int forward_causal_entry(const void* Q, const void* K, const void* V, const float* logA, void* O, float* den,
                         const float* S0, const float* Z0, float* S_out, float* Z_out, float* ckpt, int B, int H,
                         int N, int D, int M, int dtype, int feature, void* ws, size_t ws_bytes, void* stream,
                         const la_options* opts, bool use_scratch);

}  // namespace

#pragma GCC visibility push(default)
extern "C" {

int la_version(void) { return 200; }

const char* la_status_string(int status) {
  switch (status) {
    case LA_OK: return "LA_OK";
    case LA_ERR_NULL: return "LA_ERR_NULL";
    case LA_ERR_SHAPE: return "LA_ERR_SHAPE";
    case LA_ERR_DTYPE: return "LA_ERR_DTYPE";
    case LA_ERR_ALIGN: return "LA_ERR_ALIGN";
    case LA_ERR_ALIAS: return "LA_ERR_ALIAS";
    case LA_ERR_WORKSPACE: return "LA_ERR_WORKSPACE";
    case LA_ERR_UNSUPPORTED: return "LA_ERR_UNSUPPORTED";
    case LA_ERR_HIP: return "LA_ERR_HIP";
    case LA_ERR_ARG: return "LA_ERR_ARG";
    case LA_ERR_WAIT: return "LA_ERR_WAIT";
    default: return "LA_ERR_UNKNOWN";
  }
}

const char* la_last_error(void) { return g_err.c_str(); }

const char* la_kernel_names(void) {
  return "seg_state,fwd_causal,fwd_noncausal,bwd_query,bwd_kv,nc_qr,nc_kv,decode,scan_states,scan_rev,"
         "state_copy,dseg_state,dscan_states,dfwd,dbq,dscan_rev,dbkv,dla_fix,feat_rf,feat_rf_vjp,feat_poly2,"
         "feat_poly2_vjp,sync_clear,wide_combine,bwd_query_shares,nc_qr_shares,wide_pairs,wide_sum,decode_wide,feat_rf_vjp_wide,"
         "feat_poly2_wide,feat_poly2_vjp_wide";
}

size_t la_workspace_size(int op, int B, int H, int N, int D, int M, int dtype, const la_options* opts) {
  if (check_sizes(B, H, N, D, M, dtype) != LA_OK) return 0;
  if (op < LA_OP_FWD_CAUSAL || op > LA_OP_BWD_DECAY) return 0;
  const bool nc = op == LA_OP_FWD_NONCAUSAL || op == LA_OP_BWD_NONCAUSAL || op == LA_OP_FWD_DECAY ||
                  op == LA_OP_BWD_DECAY;
  if (is_wide(D) && (op == LA_OP_DECODE || op == LA_OP_FWD_DECAY || op == LA_OP_BWD_DECAY)) return 0;
  return ws_layout(op, plan_for(B, H, N, D, M, nc ? kFineTargetNC : 0, opt_chunks(opts))).bytes();
}

size_t la_checkpoint_size(int B, int H, int N, int D, int M, const la_options* opts) {
  if (check_sizes(B, H, N, D, M, LA_F32) != LA_OK) return 0;
  return ckpt_bytes(plan_for(B, H, N, D, M, 0, opt_chunks(opts)));
}

int la_segment_length(int B, int H, int N, int D, int M, const la_options* opts) {
  if (check_sizes(B, H, N, D, M, LA_F32) != LA_OK) return 0;
  return plan_for(B, H, N, D, M, 0, opt_chunks(opts)).L;
}

int la_forward_wait_status(const void* ws, size_t ws_bytes, int B, int H, int N, int D, int M, int dtype,
                           void* stream, const la_options* opts) {
  g_err.clear();
  int st = check_sizes(B, H, N, D, M, dtype);
  if (st) return st;
  st = check_opts(opts);
  if (st) return st;
  const Plan p = plan_for(B, H, N, D, M, 0, opt_chunks(opts));
  const WsLayout wl = ws_layout(LA_OP_FWD_CAUSAL, p);
  if (wl.sync == 0) return LA_OK;  // no flags: never the one-launch form
  if (!ws || ws_bytes < wl.bytes())
    return fail(LA_ERR_WORKSPACE, "workspace of " + std::to_string(wl.bytes()) + " bytes required");
  unsigned word = 0;
  const hipStream_t s = (hipStream_t)stream;
  if (hipMemcpyAsync(&word, region(const_cast<void*>(ws), wl.agg + wl.ckpt), sizeof(word), hipMemcpyDeviceToHost,
                     s) != hipSuccess ||
      hipStreamSynchronize(s) != hipSuccess)
    return fail(LA_ERR_HIP, std::string("reading the status word: ") + hipGetErrorString(hipGetLastError()));
  return word ? fail(LA_ERR_WAIT, "a one-launch forward workgroup gave up waiting for an earlier segment") : LA_OK;
}

int la_forward_causal(const void* Q, const void* K, const void* V, const float* logA, void* O, float* den,
                      const float* S0, const float* Z0, float* S_out, float* Z_out, float* ckpt, int B, int H, int N,
                      int D, int M, int dtype, int feature, void* ws, size_t ws_bytes, void* stream,
                      const la_options* opts) {
  return forward_causal_entry(Q, K, V, logA, O, den, S0, Z0, S_out, Z_out, ckpt, B, H, N, D, M, dtype, feature, ws,
                              ws_bytes, stream, opts, false);
}

int la_forward_causal_noalloc(const void* Q, const void* K, const void* V, const float* logA, void* O, float* den,
                              const float* S0, const float* Z0, float* S_out, float* Z_out, float* ckpt, int B, int H,
                              int N, int D, int M, int dtype, int feature, void* stream, const la_options* opts) {
  return forward_causal_entry(Q, K, V, logA, O, den, S0, Z0, S_out, Z_out, ckpt, B, H, N, D, M, dtype, feature,
                              nullptr, 0, stream, opts, true);
}

}  // extern "C"
#pragma GCC visibility pop

namespace {

int forward_causal_entry(const void* Q, const void* K, const void* V, const float* logA, void* O, float* den,
                         const float* S0, const float* Z0, float* S_out, float* Z_out, float* ckpt, int B, int H,
                         int N, int D, int M, int dtype, int feature, void* ws, size_t ws_bytes, void* stream,
                         const la_options* opts, bool use_scratch) {
  g_err.clear();
  if (feature != LA_FEATURE_ELU1 && feature != LA_FEATURE_IDENTITY)
    return fail(LA_ERR_ARG, "feature must be LA_FEATURE_ELU1 (0) or LA_FEATURE_IDENTITY (1)");
  const int fm = feature;
  int st = check_sizes(B, H, N, D, M, dtype);
  if (st) return st;
  st = check_opts(opts);
  if (st) return st;
  st = check_wide(D, feature, logA);
  if (st) return st;
  if ((S0 == nullptr) != (Z0 == nullptr)) return fail(LA_ERR_ARG, "S0 and Z0 must be given together");
  if ((S_out == nullptr) != (Z_out == nullptr)) return fail(LA_ERR_ARG, "S_out and Z_out must be given together");
  if (N > 0 && (!Q || !K || !V || !O)) return fail(LA_ERR_NULL, "Q, K, V and O are required");
  const Plan p = plan_for(B, H, N, D, M, logA ? kFineTargetNC : 0, opt_chunks(opts));
  const size_t es = esize(dtype), bh = (size_t)p.BHv();
  const size_t need = ws_layout(logA ? LA_OP_FWD_DECAY : LA_OP_FWD_CAUSAL, p).bytes();
  const bool uses_ws = need > 0;
  if (use_scratch && uses_ws) {  // the library's static scratch of this device in place of a workspace
    if (need > kScratchBytes)
      return fail(LA_ERR_WORKSPACE, "these sizes need " + std::to_string(need) + " bytes of scratch; the static "
                  "scratch of la_forward_causal_noalloc holds " + std::to_string(kScratchBytes) +
                  " (use la_forward_causal with a workspace)");
    st = scratch_ptr(&ws);
    if (st) return st;
    ws_bytes = kScratchBytes;
  }
  if (uses_ws && (ws == nullptr || ws_bytes < need))
    return fail(LA_ERR_WORKSPACE, "workspace of " + std::to_string(need) + " bytes required");
  st = check_ptrs({rng("Q", Q, bh * N * D * es, false), rng("K", K, bh * N * D * es, false),
                   rng("V", V, bh * N * M * es, false), rng("logA", logA, bh * N * 4, false),
                   rng("S0", S0, bh * D * M * 4, false),
                   rng("Z0", Z0, bh * D * 4, false), rng("O", O, bh * N * M * es, true),
                   rng("den", den, bh * N * 4, true), rng("S_out", S_out, bh * D * M * 4, true),
                   rng("Z_out", Z_out, bh * D * 4, true),
                   rng("ckpt", ckpt, la_checkpoint_size(B, H, N, D, M, opts), true),
                   rng("ws", uses_ws ? ws : nullptr, need, true)});
  if (st) return st;
  if (N == 0 && !S_out && !ckpt) return LA_OK;
  if (p.ns > 1)
    LA_WIDE_DISPATCH(dtype, M, fwd_wide_impl, p, true, Q, K, V, O, den, S0, Z0, S_out, Z_out, ckpt, N, ws, fm,
                     Call{(hipStream_t)stream, opts});
  if (logA)
    LA_DISPATCH(dtype, D, M, fwd_decay_impl, p, Q, K, V, logA, O, den, S0, Z0, S_out, Z_out, ckpt, N, ws,
                fm, Call{(hipStream_t)stream, opts});
  LA_DISPATCH(dtype, D, M, fwd_causal_impl, p, Q, K, V, O, den, S0, Z0, S_out, Z_out, ckpt, N, ws,
              fm, Call{(hipStream_t)stream, opts});
}

}  // namespace

#pragma GCC visibility push(default)
extern "C" {

int la_forward_noncausal(const void* Q, const void* K, const void* V, void* O, float* S_out, float* Z_out, int B,
                         int H, int N, int D, int M, int dtype, int feature, void* ws, size_t ws_bytes,
                         void* stream, const la_options* opts) {
  g_err.clear();
  if (feature != LA_FEATURE_ELU1 && feature != LA_FEATURE_IDENTITY)
    return fail(LA_ERR_ARG, "feature must be LA_FEATURE_ELU1 (0) or LA_FEATURE_IDENTITY (1)");
  const int fm = feature;
  int st = check_sizes(B, H, N, D, M, dtype);
  if (st) return st;
  st = check_opts(opts);
  if (st) return st;
  st = check_wide(D, feature, nullptr);
  if (st) return st;
  if ((S_out == nullptr) != (Z_out == nullptr)) return fail(LA_ERR_ARG, "S_out and Z_out must be given together");
  if (N == 0 && !S_out) return LA_OK;
  if (N > 0 && (!Q || !K || !V || !O)) return fail(LA_ERR_NULL, "Q, K, V and O are required");
  const Plan p = plan_for(B, H, N, D, M, kFineTargetNC, opt_chunks(opts));
  const size_t es = esize(dtype), bh = (size_t)p.BHv();
  const size_t need = ws_layout(LA_OP_FWD_NONCAUSAL, p).bytes();
  if (need > 0 && (ws == nullptr || ws_bytes < need))
    return fail(LA_ERR_WORKSPACE, "workspace of " + std::to_string(need) + " bytes required");
  st = check_ptrs({rng("Q", Q, bh * N * D * es, false), rng("K", K, bh * N * D * es, false),
                   rng("V", V, bh * N * M * es, false), rng("O", O, bh * N * M * es, true),
                   rng("S_out", S_out, bh * D * M * 4, true), rng("Z_out", Z_out, bh * D * 4, true),
                   rng("ws", need > 0 ? ws : nullptr, need, true)});
  if (st) return st;
  if (p.ns > 1)
    LA_WIDE_DISPATCH(dtype, M, fwd_wide_impl, p, false, Q, K, V, O, (float*)nullptr, (const float*)nullptr,
                     (const float*)nullptr, S_out, Z_out, (float*)nullptr, N, ws, fm, Call{(hipStream_t)stream, opts});
  LA_DISPATCH(dtype, D, M, fwd_noncausal_impl, p, Q, K, V, O, S_out, Z_out, N, ws, fm, Call{(hipStream_t)stream, opts});
}

int la_backward_causal(const void* Q, const void* K, const void* V, const float* logA, const void* O,
                       const float* den, const void* dO, const float* S0, const float* Z0, const float* ckpt,
                       const float* dS_N, const float* dZ_N, void* dQ, void* dK, void* dV, float* dlogA, float* dS0,
                       float* dZ0, int B, int H, int N, int D, int M, int dtype, int feature, void* ws, size_t ws_bytes,
                       void* stream, const la_options* opts) {
  g_err.clear();
  if (feature != LA_FEATURE_ELU1 && feature != LA_FEATURE_IDENTITY)
    return fail(LA_ERR_ARG, "feature must be LA_FEATURE_ELU1 (0) or LA_FEATURE_IDENTITY (1)");
  const int fm = feature;
  int st = check_sizes(B, H, N, D, M, dtype);
  if (st) return st;
  st = check_opts(opts);
  if (st) return st;
  st = check_wide(D, feature, logA);
  if (st) return st;
  if ((logA == nullptr) != (dlogA == nullptr)) return fail(LA_ERR_ARG, "logA and dlogA must be given together");
  if ((S0 == nullptr) != (Z0 == nullptr)) return fail(LA_ERR_ARG, "S0 and Z0 must be given together");
  if ((dS_N == nullptr) != (dZ_N == nullptr)) return fail(LA_ERR_ARG, "dS_N and dZ_N must be given together");
  if ((dS0 == nullptr) != (dZ0 == nullptr)) return fail(LA_ERR_ARG, "dS0 and dZ0 must be given together");
  const size_t bh = (size_t)B * H;
  if (N == 0) {
    if (!dS0) return LA_OK;
    st = check_ptrs({rng("dS_N", dS_N, bh * D * M * 4, false), rng("dZ_N", dZ_N, bh * D * 4, false),
                     rng("dS0", dS0, bh * D * M * 4, true), rng("dZ0", dZ0, bh * D * 4, true)});
    if (st) return st;
    const Plan p = plan_for(B, H, N, D, M, logA ? kFineTargetNC : 0, opt_chunks(opts));
    if (p.ns > 1)
      LA_WIDE_DISPATCH(dtype, M, bwd_wide_impl, p, Q, K, V, dO, S0, Z0, ckpt, dS_N, dZ_N, dQ, dK, dV, dS0, dZ0, N,
                       ws, fm, Call{(hipStream_t)stream, opts});
    LA_DISPATCH(dtype, D, M, bwd_causal_impl, p, Q, K, V, O, den, dO, S0, Z0, ckpt, dS_N, dZ_N, dQ, dK, dV, dS0,
                dZ0, N, ws, fm, Call{(hipStream_t)stream, opts});
  }
  if (!Q || !K || !V || !O || !den || !dO || !dQ || !dK || !dV)
    return fail(LA_ERR_NULL, "Q, K, V, O, den, dO, dQ, dK and dV are required");
  const Plan p = plan_for(B, H, N, D, M, logA ? kFineTargetNC : 0, opt_chunks(opts));
  const size_t es = esize(dtype);
  const size_t need = ws_layout(logA ? LA_OP_BWD_DECAY : LA_OP_BWD_CAUSAL, p).bytes();
  const bool uses_ws = need > 0;
  if (uses_ws && (ws == nullptr || ws_bytes < need))
    return fail(LA_ERR_WORKSPACE, "workspace of " + std::to_string(need) + " bytes required");
  st = check_ptrs({rng("Q", Q, bh * N * D * es, false), rng("K", K, bh * N * D * es, false),
                   rng("V", V, bh * N * M * es, false), rng("logA", logA, bh * N * 4, false),
                   rng("O", O, bh * N * M * es, false), rng("den", den, bh * N * 4, false),
                   rng("dO", dO, bh * N * M * es, false), rng("S0", S0, bh * D * M * 4, false),
                   rng("Z0", Z0, bh * D * 4, false), rng("ckpt", ckpt, la_checkpoint_size(B, H, N, D, M, opts), false),
                   rng("dS_N", dS_N, bh * D * M * 4, false), rng("dZ_N", dZ_N, bh * D * 4, false),
                   rng("dQ", dQ, bh * N * D * es, true), rng("dK", dK, bh * N * D * es, true),
                   rng("dV", dV, bh * N * M * es, true), rng("dlogA", dlogA, bh * N * 4, true),
                   rng("dS0", dS0, bh * D * M * 4, true), rng("dZ0", dZ0, bh * D * 4, true),
                   rng("ws", uses_ws ? ws : nullptr, need, true)});
  if (st) return st;
  if (p.ns > 1)
    LA_WIDE_DISPATCH(dtype, M, bwd_wide_impl, p, Q, K, V, dO, S0, Z0, ckpt, dS_N, dZ_N, dQ, dK, dV, dS0, dZ0, N, ws,
                     fm, Call{(hipStream_t)stream, opts});
  if (logA)
    LA_DISPATCH(dtype, D, M, bwd_decay_impl, p, Q, K, V, logA, dO, S0, Z0, ckpt, dS_N, dZ_N, dQ, dK, dV, dlogA, dS0,
                dZ0, N, ws, fm, Call{(hipStream_t)stream, opts});
  LA_DISPATCH(dtype, D, M, bwd_causal_impl, p, Q, K, V, O, den, dO, S0, Z0, ckpt, dS_N, dZ_N, dQ, dK, dV, dS0, dZ0,
              N, ws, fm, Call{(hipStream_t)stream, opts});
}

int la_backward_noncausal(const void* Q, const void* K, const void* V, const void* dO, const float* S_tot,
                          const float* Z_tot, void* dQ, void* dK, void* dV, int B, int H, int N, int D, int M,
                          int dtype, int feature, void* ws, size_t ws_bytes, void* stream,
                          const la_options* opts) {
  g_err.clear();
  if (feature != LA_FEATURE_ELU1 && feature != LA_FEATURE_IDENTITY)
    return fail(LA_ERR_ARG, "feature must be LA_FEATURE_ELU1 (0) or LA_FEATURE_IDENTITY (1)");
  const int fm = feature;
  int st = check_sizes(B, H, N, D, M, dtype);
  if (st) return st;
  st = check_opts(opts);
  if (st) return st;
  st = check_wide(D, feature, nullptr);
  if (st) return st;
  if (N == 0) return LA_OK;
  if (!Q || !K || !V || !dO || !dQ || !dK || !dV) return fail(LA_ERR_NULL, "Q, K, V, dO, dQ, dK and dV are required");
  if ((S_tot == nullptr) != (Z_tot == nullptr)) return fail(LA_ERR_ARG, "S_tot and Z_tot must be given together");
  const Plan p = plan_for(B, H, N, D, M, kFineTargetNC, opt_chunks(opts));
  const size_t es = esize(dtype), bh = (size_t)p.BHv();
  const size_t need = ws_layout(LA_OP_BWD_NONCAUSAL, p).bytes();
  if (ws == nullptr || ws_bytes < need)
    return fail(LA_ERR_WORKSPACE, "workspace of " + std::to_string(need) + " bytes required");
  st = check_ptrs({rng("Q", Q, bh * N * D * es, false), rng("K", K, bh * N * D * es, false),
                   rng("V", V, bh * N * M * es, false), rng("dO", dO, bh * N * M * es, false),
                   rng("S_tot", S_tot, bh * D * M * 4, false), rng("Z_tot", Z_tot, bh * D * 4, false),
                   rng("dQ", dQ, bh * N * D * es, true), rng("dK", dK, bh * N * D * es, true),
                   rng("dV", dV, bh * N * M * es, true), rng("ws", ws, need, true)});
  if (st) return st;
  if (p.ns > 1)
    LA_WIDE_DISPATCH(dtype, M, bwd_noncausal_wide_impl, p, Q, K, V, dO, S_tot, Z_tot, dQ, dK, dV, N, ws, fm,
                     Call{(hipStream_t)stream, opts});
  LA_DISPATCH(dtype, D, M, bwd_noncausal_impl, p, Q, K, V, dO, S_tot, Z_tot, dQ, dK, dV, N, ws, fm,
              Call{(hipStream_t)stream, opts});
}

int la_decode_step(const void* q, const void* k, const void* v, const float* logA, float* S, float* Z, void* y,
                   int B, int H, int D, int M, int dtype, int feature, void* stream, const la_options* opts) {
  g_err.clear();
  if (feature != LA_FEATURE_ELU1 && feature != LA_FEATURE_IDENTITY)
    return fail(LA_ERR_ARG, "feature must be LA_FEATURE_ELU1 (0) or LA_FEATURE_IDENTITY (1)");
  const int fm = feature;
  int st = check_sizes(B, H, 1, D, M, dtype);
  if (st) return st;
  st = check_opts(opts);
  if (st) return st;
  st = check_wide(D, feature, logA);
  if (st) return st;
  if (!q || !k || !v || !S || !Z || !y) return fail(LA_ERR_NULL, "q, k, v, S, Z and y are required");
  const size_t es = esize(dtype), bh = (size_t)B * H;
  st = check_ptrs({rng("q", q, bh * D * es, false), rng("k", k, bh * D * es, false), rng("v", v, bh * M * es, false),
                   rng("logA", logA, bh * 4, false), rng("S", S, bh * D * M * 4, true),
                   rng("Z", Z, bh * D * 4, true), rng("y", y, bh * M * es, true)});
  if (st) return st;
  if (is_wide(D))
    LA_WIDE_DISPATCH(dtype, M, decode_wide_impl, (long)bh, D, q, k, v, S, Z, y, fm, Call{(hipStream_t)stream, opts});
  LA_DISPATCH(dtype, D, M, decode_impl, (long)bh, q, k, v, logA, S, Z, y, fm, Call{(hipStream_t)stream, opts});
}

int la_feature_random(const void* X, const float* W, void* Phi, int B, int H, int N, int Din, int C, int dtype,
                      void* stream) {
  return feature_random(X, W, nullptr, Phi, B, H, N, Din, C, dtype, stream);
}

int la_feature_random_vjp(const void* X, const float* W, const void* dPhi, void* dX, int B, int H, int N, int Din,
                          int C, int dtype, void* stream) {
  if (!dPhi) {
    g_err.clear();
    return fail(LA_ERR_NULL, "dPhi is required");
  }
  return feature_random(X, W, dPhi, dX, B, H, N, Din, C, dtype, stream);
}

int la_feature_poly2(const void* X, void* Phi, int B, int H, int N, int Din, int C, int dtype, void* stream) {
  return feature_poly2(X, nullptr, Phi, B, H, N, Din, C, dtype, stream);
}

int la_feature_poly2_vjp(const void* X, const void* dPhi, void* dX, int B, int H, int N, int Din, int C, int dtype,
                         void* stream) {
  if (!dPhi) {
    g_err.clear();
    return fail(LA_ERR_NULL, "dPhi is required");
  }
  return feature_poly2(X, dPhi, dX, B, H, N, Din, C, dtype, stream);
}

}  // extern "C"
#pragma GCC visibility pop
