// C ABI of libgdr: host-side validation, the chunk planner, the workspace
// layout and the launch sequence of each call.  See include/gdr.h for the
// contract of every entry point.
#include "gdr.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>
#include <mutex>
#include <numeric>
#include <string>
#include <vector>

#include "gdr_kernels.h"

// Workspace of gdr_kda_ckpt_noalloc: one copy per device, held from the
// library's load on that device until the process ends.  Host code never uses
// this name as an address; it uses the pointer hipGetSymbolAddress returns for
// the current device (scratch_of_device below).
static __device__ __align__(256) unsigned char scratch[GDR_NOALLOC_SCRATCH_BYTES];

namespace gdr {
hipError_t set_dynamic_lds_once(const void *kernel, int bytes) {
  struct Entry {
    int dev;
    const void *fn;
    int bytes;
  };
  static std::mutex mu;
  static std::vector<Entry> done;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(mu);
  for (const Entry &x : done)
    if (x.dev == dev && x.fn == kernel && x.bytes >= bytes) return hipSuccess;
  e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess) done.push_back(Entry{dev, kernel, bytes});
  return e;
}
}  // namespace gdr

namespace {

thread_local std::string g_last_error;

int32_t fail(int32_t code, const std::string &msg) {
  g_last_error = msg;
  return code;
}

constexpr int64_t kAlign = 256;
constexpr int64_t kChunk = 64;
constexpr int64_t kHD = 128;

int64_t round_up(int64_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Per (chunk, value head) unit bytes of each workspace region.
constexpr int64_t kFrag64x128 = 16 * 64 * 16;  // 16 fragment tiles of 1 KB
constexpr int64_t kFrag64x64 = 8 * 64 * 16;
constexpr int64_t kAcc64x128 = kChunk * kHD * 2;
constexpr int64_t kGamma = kHD * 4;
constexpr int64_t kState = kHD * kHD * 2;
constexpr int64_t kRows = kChunk * kHD * 2;

// Walk segments per document: more than one only when the chains (documents x
// value heads, 8 wavefronts each) would leave the compute units underfilled and
// some document spans two chunks.  This is the equal plan's count and the
// balanced plan's average (its budget is N times it).
int walk_segments(int64_t N, int64_t Hv, int64_t NC) {
  const int64_t waves = 8 * N * Hv;
  if (waves == 0 || waves >= 512 || NC <= N) return 1;
  return (int)std::min<int64_t>(4, std::max<int64_t>(1, 512 / waves));
}
// Most segments one document can get: the balanced plan may give a long document
// up to twice the average (at most 8).
int walk_segment_cap(int64_t N, int64_t Hv, int64_t NC) {
  const int P = walk_segments(N, Hv, NC);
  return P > 1 && N > 1 ? std::min(8, 2 * P) : P;
}

struct Layout {
  int64_t carry;                          // segment carries (segmented walks only)
  int64_t WfN, KbT, Pf, Oacc, Uacc, gam;  // forward walk operands
  int64_t QGT, MTs, Tt, Et, S, Vn;        // tapes kept for the backward
  int64_t qk_rstd;                           // q/k inverse norms (per token and Q/K head)
  int64_t fwd_bytes, full_bytes;
};

// The backward's scratch tapes overlay forward-walk operands, which are dead once
// the forward walk has run: dS (32 KB per unit) the adjacent Pf|Oacc, dVnT (16 KB)
// Uacc.  WfN and KbT stay: the adjoint walk reads them transposed.  KbT and QGT are
// per (chunk, Q/K head).
Layout make_layout(int64_t units, int64_t N, int64_t Hv, int64_t T, int64_t Hqk) {
  Layout L{};
  int64_t off = 0;
  auto take = [&](int64_t per_unit) {
    const int64_t at = off;
    off += round_up(per_unit * units);
    return at;
  };
  // per (chunk, Q/K head): the K fragments a Q/K head's value heads share
  const int64_t qk_units = Hv > 0 ? units / Hv * Hqk : 0;
  auto take_qk = [&](int64_t per_unit) {
    const int64_t at = off;
    off += round_up(per_unit * qk_units);
    return at;
  };
  L.carry = off;
  off += round_up((int64_t)(walk_segment_cap(N, Hv, units / Hv) - 1) * N * Hv * 2 * kHD * kHD * 4);
  L.WfN = take(kFrag64x128);
  L.KbT = take_qk(kFrag64x128);
  L.Pf = take(kFrag64x128);
  L.Oacc = take(kAcc64x128);  // right after Pf: the two carry the dS tape
  L.Uacc = take(kAcc64x128);
  L.gam = take(kGamma);
  L.fwd_bytes = off;
  L.QGT = take_qk(kFrag64x128);
  L.MTs = take(kFrag64x64);
  L.Tt = take(kFrag64x64);
  L.Et = take(kFrag64x64);
  L.S = take(kState);
  L.Vn = take(kRows);
  L.qk_rstd = off;
  off += round_up(T * Hqk * 2 * 4);
  L.full_bytes = off;
  return L;
}

gdr::Workspace bind(const Layout &L, void *base) {
  char *b = static_cast<char *>(base);
  gdr::Workspace w{};
  w.WfN = reinterpret_cast<uint4 *>(b + L.WfN);
  w.Pf = reinterpret_cast<uint4 *>(b + L.Pf);
  w.KbT = reinterpret_cast<uint4 *>(b + L.KbT);
  w.Uacc = reinterpret_cast<uint16_t *>(b + L.Uacc);
  w.Oacc = reinterpret_cast<uint16_t *>(b + L.Oacc);
  w.gam = reinterpret_cast<float *>(b + L.gam);
  w.QGT = reinterpret_cast<uint4 *>(b + L.QGT);
  w.MTs = reinterpret_cast<uint4 *>(b + L.MTs);
  w.Tt = reinterpret_cast<uint4 *>(b + L.Tt);
  w.Et = reinterpret_cast<uint4 *>(b + L.Et);
  w.S = reinterpret_cast<uint16_t *>(b + L.S);
  w.Vn = reinterpret_cast<uint16_t *>(b + L.Vn);
  w.dS = reinterpret_cast<uint16_t *>(b + L.Pf);    // over Pf|Oacc
  w.dVnT = reinterpret_cast<uint16_t *>(b + L.Uacc);// over Uacc
  w.carry = reinterpret_cast<float *>(b + L.carry);
  w.qk_rstd = reinterpret_cast<float *>(b + L.qk_rstd);
  return w;
}

int32_t check_sizes(int32_t variant, int64_t T, int64_t N, int64_t NC, int64_t Hqk, int64_t Hv, int64_t K,
                    int64_t V) {
  if (variant != GDR_KDA && variant != GDR_GDN) return fail(GDR_ERR_INVALID_ARG, "unknown variant");
  if (T < 0 || N < 0 || NC < 0) return fail(GDR_ERR_INVALID_ARG, "T, N and n_chunks must be >= 0");
  if (Hqk <= 0 || Hv <= 0) return fail(GDR_ERR_INVALID_ARG, "head counts must be positive");
  if (K != kHD || V != kHD) return fail(GDR_ERR_UNSUPPORTED, "only K = V = 128 is implemented");
  if (variant == GDR_KDA && Hqk != Hv) return fail(GDR_ERR_UNSUPPORTED, "KDA needs H_qk == H_v");
  if (variant == GDR_GDN && Hv % Hqk != 0) return fail(GDR_ERR_UNSUPPORTED, "GDN needs H_v to be a multiple of H_qk");
  if (T > 0 && N == 0) return fail(GDR_ERR_INVALID_ARG, "tokens without documents");
  // every chunk holds 1..64 tokens of one document, and each document adds at
  // most one partial chunk
  if (NC > T || NC < (T + kChunk - 1) / kChunk || NC > (T + kChunk - 1) / kChunk + N)
    return fail(GDR_ERR_INVALID_ARG, "n_chunks is inconsistent with T and N");
  // grid sizes are 32-bit: chunk grids use NC * H_v blocks, walk grids 8 * N * H_v
  if (N * Hv > (int64_t(1) << 27) || NC * Hv > (int64_t(1) << 31) - 1)
    return fail(GDR_ERR_UNSUPPORTED, "problem too large");
  // the walks address one chunk's rows of o / dout through buffer resources
  // with a 32-bit byte range: 64 rows of H_v * 128 bf16
  if (Hv > 65536) return fail(GDR_ERR_UNSUPPORTED, "H_v above 65536");
  return GDR_OK;
}

struct DeviceCache {
  std::mutex mu;
  std::vector<int> state;  // 0 unknown, 1 gfx950, 2 other
};
DeviceCache &device_cache() {
  static DeviceCache c;
  return c;
}

int32_t check_device_impl() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(GDR_ERR_HIP, "hipGetDevice failed");
  DeviceCache &c = device_cache();
  std::lock_guard<std::mutex> lk(c.mu);
  if ((int)c.state.size() <= dev) c.state.resize(dev + 1, 0);
  if (c.state[dev] == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return fail(GDR_ERR_HIP, "hipGetDeviceProperties failed");
    c.state[dev] = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
  }
  if (c.state[dev] != 1) return fail(GDR_ERR_ARCH, "the current device is not gfx950");
  return GDR_OK;
}

int32_t check_problem(int32_t variant, const gdr_problem *p) {
  if (!p) return fail(GDR_ERR_INVALID_ARG, "problem is NULL");
  int32_t rc = check_sizes(variant, p->T, p->N, p->n_chunks, p->H_qk, p->H_v, p->K, p->V);
  if (rc) return rc;
  if (p->T > 0 && (!p->q || !p->k || !p->v || !p->g || !p->beta))
    return fail(GDR_ERR_INVALID_ARG, "q, k, v, g and beta must be non-NULL");
  if (p->N > 0 && (!p->cu_seqlens || !p->chunk_table))
    return fail(GDR_ERR_INVALID_ARG, "cu_seqlens and chunk_table must be non-NULL");
  if (!(p->scale == p->scale)) return fail(GDR_ERR_INVALID_ARG, "scale is NaN");
  if (p->input_flags & ~(GDR_IN_QK_L2NORM | GDR_IN_BETA_SIGMOID))
    return fail(GDR_ERR_INVALID_ARG, "unknown input flag");
  if (p->walk_segments < 0) return fail(GDR_ERR_INVALID_ARG, "walk_segments < 0");
  if (p->max_doc_chunks < 0 || p->max_doc_chunks > p->n_chunks)
    return fail(GDR_ERR_INVALID_ARG, "max_doc_chunks outside [0, n_chunks]");
  if (p->walk_layout != GDR_WALK_AUTO && p->walk_layout != GDR_WALK_SLICES && p->walk_layout != GDR_WALK_RINGS)
    return fail(GDR_ERR_INVALID_ARG, "unknown walk_layout");
  if (p->walk_plan != GDR_PLAN_BALANCED && p->walk_plan != GDR_PLAN_EQUAL)
    return fail(GDR_ERR_INVALID_ARG, "unknown walk_plan");
  return GDR_OK;
}

int32_t check_workspace(const gdr_problem *p, void *ws, int64_t ws_bytes, bool full, Layout &L) {
  L = make_layout((int64_t)p->n_chunks * p->H_v, p->N, p->H_v, p->T, p->H_qk);
  const int64_t need = full ? L.full_bytes : L.fwd_bytes;
  if (need > 0 && !ws) return fail(GDR_ERR_WORKSPACE, "workspace is NULL");
  if (reinterpret_cast<uintptr_t>(ws) % kAlign) return fail(GDR_ERR_WORKSPACE, "workspace is not 256-byte aligned");
  if (ws_bytes < need)
    return fail(GDR_ERR_WORKSPACE, "workspace too small: need " + std::to_string(need) + " bytes, got " +
                                       std::to_string(ws_bytes));
  return GDR_OK;
}

gdr::Problem to_internal(const gdr_problem *p) {
  gdr::Problem q{};
  q.T = p->T;
  q.N = p->N;
  q.Hqk = p->H_qk;
  q.Hv = p->H_v;
  q.NC = p->n_chunks;
  q.q = p->q;
  q.k = p->k;
  q.v = p->v;
  q.g = p->g;
  q.beta = p->beta;
  q.cu = p->cu_seqlens;
  q.table = p->chunk_table;
  q.h0 = p->h0;
  q.scale = p->scale;
  q.inflags = (int)p->input_flags;
  int P = walk_segments(p->N, p->H_v, p->n_chunks);  // the equal plan's count per document
  if (p->walk_segments > 0 && p->walk_segments < P) P = p->walk_segments;
  if (p->walk_plan == GDR_PLAN_BALANCED && P > 1 && p->N > 1) {
    // per-document cap: twice the average, within the carry slots the workspace holds
    q.P = std::min(2 * P, walk_segment_cap(p->N, p->H_v, p->n_chunks));
    q.B = P * p->N;  // as many segments in all as the equal plan
  } else {
    q.P = P;
    q.B = 0;
  }
  q.L = p->max_doc_chunks > 0 ? p->max_doc_chunks : p->n_chunks;
  q.layout = p->walk_layout;
  return q;
}

// ---- optional per-kernel timing with events on the call's stream ----
struct Timing {
  std::mutex mu;
  bool on = false;
  struct Pending {
    int kernel;
    hipEvent_t a, b;
  };
  std::vector<Pending> pending;
  std::vector<hipEvent_t> pool;
  double total_ms[4] = {0, 0, 0, 0};
  int64_t launches[4] = {0, 0, 0, 0};
};
const char *const kKernelNames[4] = {"fwd_prep", "fwd_walk", "bwd_walk", "bwd_grad"};
Timing &timing() {
  static Timing t;
  return t;
}
hipEvent_t take_event(Timing &t) {
  if (!t.pool.empty()) {
    hipEvent_t e = t.pool.back();
    t.pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// Runs `launch` (which enqueues one kernel on st), bracketed by events when timing is on.
template <class F>
hipError_t timed(int kernel, hipStream_t st, F launch) {
  Timing &t = timing();
  if (!t.on) return launch();
  std::lock_guard<std::mutex> lk(t.mu);
  hipEvent_t a = take_event(t), b = take_event(t);
  if (!a || !b) return hipErrorOutOfMemory;
  hipError_t e = hipEventRecord(a, st);
  if (e == hipSuccess) e = launch();
  if (e == hipSuccess) e = hipEventRecord(b, st);
  if (e != hipSuccess) {
    t.pool.push_back(a);
    t.pool.push_back(b);
    return e;
  }
  t.pending.push_back({kernel, a, b});
  return hipSuccess;
}

int32_t hip_status(hipError_t e, const char *what) {
  if (e == hipSuccess) return GDR_OK;
  return fail(GDR_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

int32_t fwd_impl(int32_t variant, const gdr_problem *p, uint16_t *o, float *ht, void *ws, int64_t ws_bytes,
                 uint32_t flags, void *stream) {
  int32_t rc = check_problem(variant, p);
  if (rc) return rc;
  if (flags & ~(GDR_FWD_SAVE | GDR_FWD_SKIP_OUTPUT)) return fail(GDR_ERR_INVALID_ARG, "unknown forward flag");
  const bool save = (flags & GDR_FWD_SAVE) != 0, out = (flags & GDR_FWD_SKIP_OUTPUT) == 0;
  if (p->T > 0 && out && !o) return fail(GDR_ERR_INVALID_ARG, "o is NULL");
  Layout L;
  if ((rc = check_workspace(p, ws, ws_bytes, save, L))) return rc;
  if ((rc = check_device_impl())) return rc;
  const gdr::Problem q = to_internal(p);
  const gdr::Workspace w = bind(L, ws);
  hipStream_t st = static_cast<hipStream_t>(stream);
  if ((rc = hip_status(timed(0, st, [&] { return gdr::launch_fwd_prep(variant == GDR_GDN, q, w, save, out, st); }),
                       "prep launch")))
    return rc;
  if ((rc = hip_status(timed(1, st, [&] { return gdr::launch_fwd_walk(variant == GDR_GDN, q, w, out ? o : nullptr, ht, save, out, st); }), "walk launch")))
    return rc;
  g_last_error.clear();
  return GDR_OK;
}

int32_t bwd_impl(int32_t variant, const gdr_problem *p, const uint16_t *dout, const float *dht, uint16_t *dq,
                 uint16_t *dk, uint16_t *dv, float *dg, void *dbeta, float *dh0, void *ws, int64_t ws_bytes,
                 void *stream) {
  int32_t rc = check_problem(variant, p);
  if (rc) return rc;
  if (p->T > 0 && (!dout || !dq || !dk || !dv || !dg || !dbeta))
    return fail(GDR_ERR_INVALID_ARG, "dout, dq, dk, dv, dg and dbeta must be non-NULL");
  Layout L;
  if ((rc = check_workspace(p, ws, ws_bytes, true, L))) return rc;
  if ((rc = check_device_impl())) return rc;
  const gdr::Problem q = to_internal(p);
  const gdr::Workspace w = bind(L, ws);
  hipStream_t st = static_cast<hipStream_t>(stream);
  if ((rc = hip_status(timed(2, st, [&] { return gdr::launch_bwd_walk(variant == GDR_GDN, q, w, dout, dht, dh0, st); }),
                       "adjoint walk launch")))
    return rc;
  if ((rc = hip_status(
           timed(3, st, [&] { return gdr::launch_bwd_grad(variant == GDR_GDN, q, w, dout, dq, dk, dv, dg, dbeta, st); }),
           "gradient launch")))
    return rc;
  g_last_error.clear();
  return GDR_OK;
}

int32_t ckpt_impl(int32_t variant, const gdr_problem *p, uint16_t *o, float *ht, const uint16_t *dout,
                  const float *dht, uint16_t *dq, uint16_t *dk, uint16_t *dv, float *dg, void *dbeta, float *dh0,
                  void *ws, int64_t ws_bytes, void *stream) {
  // validate everything the three phases need before enqueueing any of them
  int32_t rc = check_problem(variant, p);
  if (rc) return rc;
  if (p->T > 0 && (!o || !dout || !dq || !dk || !dv || !dg || !dbeta))
    return fail(GDR_ERR_INVALID_ARG, "o, dout, dq, dk, dv, dg and dbeta must be non-NULL");
  Layout L;
  if ((rc = check_workspace(p, ws, ws_bytes, true, L))) return rc;
  if ((rc = fwd_impl(variant, p, o, ht, ws, ws_bytes, 0, stream))) return rc;
  // the recompute writes the tapes only: o is already there
  if ((rc = fwd_impl(variant, p, nullptr, nullptr, ws, ws_bytes, GDR_FWD_SAVE | GDR_FWD_SKIP_OUTPUT, stream)))
    return rc;
  return bwd_impl(variant, p, dout, dht, dq, dk, dv, dg, dbeta, dh0, ws, ws_bytes, stream);
}

// Device address of `scratch` on the current device, looked up once per device
// with that device current and kept in a fixed table (no allocation).
constexpr int kMaxDevices = 64;
int32_t scratch_of_device(void **out) {
  static std::mutex mu;
  static void *addr[kMaxDevices] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(GDR_ERR_HIP, "hipGetDevice failed");
  if (dev < 0 || dev >= kMaxDevices) return fail(GDR_ERR_UNSUPPORTED, "device index above 63");
  std::lock_guard<std::mutex> lk(mu);
  if (!addr[dev]) {
    void *p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(GDR_ERR_HIP, std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e));
    addr[dev] = p;
  }
  *out = addr[dev];
  return GDR_OK;
}

int32_t ckpt_noalloc_impl(const gdr_problem *p, uint16_t *o, float *ht, const uint16_t *dout, const float *dht,
                          uint16_t *dq, uint16_t *dk, uint16_t *dv, float *dg, void *dbeta, float *dh0, void *stream) {
  int32_t rc = check_problem(GDR_KDA, p);
  if (rc) return rc;
  const Layout L = make_layout((int64_t)p->n_chunks * p->H_v, p->N, p->H_v, p->T, p->H_qk);
  if (L.full_bytes > GDR_NOALLOC_SCRATCH_BYTES)
    return fail(GDR_ERR_WORKSPACE, "problem needs " + std::to_string(L.full_bytes) +
                                       " bytes of workspace; the static scratch holds " +
                                       std::to_string((int64_t)GDR_NOALLOC_SCRATCH_BYTES));
  if ((rc = check_device_impl())) return rc;
  void *ws = nullptr;
  if ((rc = scratch_of_device(&ws))) return rc;
  return ckpt_impl(GDR_KDA, p, o, ht, dout, dht, dq, dk, dv, dg, dbeta, dh0, ws, GDR_NOALLOC_SCRATCH_BYTES, stream);
}

}  // namespace

extern "C" {

int32_t gdr_plan_chunks(const int32_t *cu, int32_t N, int32_t *table, int64_t capacity, int32_t *n_chunks_out,
                        int64_t *table_len_out) {
  if (N < 0) return fail(GDR_ERR_INVALID_ARG, "N must be >= 0");
  if (!cu) return fail(GDR_ERR_INVALID_ARG, "cu_seqlens is NULL");
  if (cu[0] != 0) return fail(GDR_ERR_INVALID_ARG, "cu_seqlens[0] must be 0");
  int64_t nc = 0;
  for (int32_t n = 0; n < N; ++n) {
    const int64_t len = (int64_t)cu[n + 1] - cu[n];
    if (len < 0) return fail(GDR_ERR_INVALID_ARG, "cu_seqlens must be non-decreasing");
    nc += (len + kChunk - 1) / kChunk;
  }
  if (nc > INT32_MAX / 4) return fail(GDR_ERR_UNSUPPORTED, "too many chunks");
  const int64_t tlen = 3 * nc + 2 * (int64_t)N + 1;
  if (n_chunks_out) *n_chunks_out = (int32_t)nc;
  if (table_len_out) *table_len_out = tlen;
  if (!table) {
    g_last_error.clear();
    return GDR_OK;
  }
  if (capacity < tlen) return fail(GDR_ERR_INVALID_ARG, "table capacity too small");
  int32_t *start = table, *clen = table + nc, *doc = table + 2 * nc, *ptr = table + 3 * nc;
  int32_t *order = ptr + N + 1;
  int64_t c = 0;
  for (int32_t n = 0; n < N; ++n) {
    ptr[n] = (int32_t)c;
    for (int64_t t = cu[n]; t < cu[n + 1]; t += kChunk) {
      start[c] = (int32_t)t;
      clen[c] = (int32_t)std::min<int64_t>(kChunk, cu[n + 1] - t);
      doc[c] = n;
      ++c;
    }
  }
  ptr[N] = (int32_t)c;
  std::vector<int32_t> idx(N);
  std::iota(idx.begin(), idx.end(), 0);
  std::stable_sort(idx.begin(), idx.end(),
                   [&](int32_t a, int32_t b) { return ptr[a + 1] - ptr[a] > ptr[b + 1] - ptr[b]; });
  std::copy(idx.begin(), idx.end(), order);
  g_last_error.clear();
  return GDR_OK;
}

int64_t gdr_workspace_bytes(int32_t variant, int32_t T, int32_t N, int32_t n_chunks, int32_t H_qk, int32_t H_v,
                            int32_t K, int32_t V, uint32_t flags) {
  const int32_t rc = check_sizes(variant, T, N, n_chunks, H_qk, H_v, K, V);
  if (rc) return -(int64_t)rc;
  if (flags & ~(GDR_FWD_SAVE | GDR_FWD_SKIP_OUTPUT)) return -(int64_t)fail(GDR_ERR_INVALID_ARG, "unknown flag");
  const Layout L = make_layout((int64_t)n_chunks * H_v, N, H_v, T, H_qk);
  return (flags & GDR_FWD_SAVE) ? L.full_bytes : L.fwd_bytes;
}

int32_t gdr_kda_fwd(const gdr_problem *p, uint16_t *o, float *ht, void *ws, int64_t ws_bytes, uint32_t flags,
                    void *stream) {
  return fwd_impl(GDR_KDA, p, o, ht, ws, ws_bytes, flags, stream);
}
int32_t gdr_gdn_fwd(const gdr_problem *p, uint16_t *o, float *ht, void *ws, int64_t ws_bytes, uint32_t flags,
                    void *stream) {
  return fwd_impl(GDR_GDN, p, o, ht, ws, ws_bytes, flags, stream);
}
int32_t gdr_kda_bwd(const gdr_problem *p, const uint16_t *dout, const float *dht, uint16_t *dq, uint16_t *dk,
                    uint16_t *dv, float *dg, void *dbeta, float *dh0, void *ws, int64_t ws_bytes, void *stream) {
  return bwd_impl(GDR_KDA, p, dout, dht, dq, dk, dv, dg, dbeta, dh0, ws, ws_bytes, stream);
}
int32_t gdr_gdn_bwd(const gdr_problem *p, const uint16_t *dout, const float *dht, uint16_t *dq, uint16_t *dk,
                    uint16_t *dv, float *dg, void *dbeta, float *dh0, void *ws, int64_t ws_bytes, void *stream) {
  return bwd_impl(GDR_GDN, p, dout, dht, dq, dk, dv, dg, dbeta, dh0, ws, ws_bytes, stream);
}
int32_t gdr_kda_ckpt(const gdr_problem *p, uint16_t *o, float *ht, const uint16_t *dout, const float *dht,
                     uint16_t *dq, uint16_t *dk, uint16_t *dv, float *dg, void *dbeta, float *dh0, void *ws,
                     int64_t ws_bytes, void *stream) {
  return ckpt_impl(GDR_KDA, p, o, ht, dout, dht, dq, dk, dv, dg, dbeta, dh0, ws, ws_bytes, stream);
}
int32_t gdr_gdn_ckpt(const gdr_problem *p, uint16_t *o, float *ht, const uint16_t *dout, const float *dht,
                     uint16_t *dq, uint16_t *dk, uint16_t *dv, float *dg, void *dbeta, float *dh0, void *ws,
                     int64_t ws_bytes, void *stream) {
  return ckpt_impl(GDR_GDN, p, o, ht, dout, dht, dq, dk, dv, dg, dbeta, dh0, ws, ws_bytes, stream);
}

int32_t gdr_kda_ckpt_noalloc(const gdr_problem *p, uint16_t *o, float *ht, const uint16_t *dout, const float *dht,
                             uint16_t *dq, uint16_t *dk, uint16_t *dv, float *dg, void *dbeta, float *dh0,
                             void *stream) {
  return ckpt_noalloc_impl(p, o, ht, dout, dht, dq, dk, dv, dg, dbeta, dh0, stream);
}

int32_t gdr_walk_layout_chosen(int32_t variant, const gdr_problem *p, int32_t compute_units, int32_t *layout) {
  int32_t rc = check_problem(variant, p);
  if (rc) return rc;
  if (!layout) return fail(GDR_ERR_INVALID_ARG, "layout is NULL");
  if (compute_units < 0) return fail(GDR_ERR_INVALID_ARG, "compute_units < 0");
  const gdr::Problem q = to_internal(p);
  *layout = gdr::walk_uses_rings(q, compute_units > 0 ? compute_units : gdr::compute_units()) ? GDR_WALK_RINGS
                                                                                              : GDR_WALK_SLICES;
  return GDR_OK;
}

int32_t gdr_check_device(void) { return check_device_impl(); }

int32_t gdr_timing_enable(int32_t on) {
  Timing &t = timing();
  std::lock_guard<std::mutex> lk(t.mu);
  t.on = on != 0;
  return GDR_OK;
}

int32_t gdr_timing_read(const char **names, double *total_ms, int64_t *launches, int32_t capacity, int32_t *count,
                        int32_t reset) {
  Timing &t = timing();
  std::lock_guard<std::mutex> lk(t.mu);
  int32_t rc = GDR_OK;
  for (const auto &pd : t.pending) {
    float ms = 0.f;
    hipError_t e = hipEventSynchronize(pd.b);
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, pd.a, pd.b);
    if (e != hipSuccess && rc == GDR_OK) rc = fail(GDR_ERR_HIP, std::string("timing: ") + hipGetErrorString(e));
    t.total_ms[pd.kernel] += ms;
    t.launches[pd.kernel] += 1;
    t.pool.push_back(pd.a);
    t.pool.push_back(pd.b);
  }
  t.pending.clear();
  const int32_t n = std::min<int32_t>(capacity, 4);
  for (int32_t i = 0; i < n; ++i) {
    if (names) names[i] = kKernelNames[i];
    if (total_ms) total_ms[i] = t.total_ms[i];
    if (launches) launches[i] = t.launches[i];
  }
  if (count) *count = n;
  if (reset)
    for (int i = 0; i < 4; ++i) {
      t.total_ms[i] = 0;
      t.launches[i] = 0;
    }
  return rc;
}

const char *gdr_status_string(int32_t s) {
  switch (s) {
    case GDR_OK: return "ok";
    case GDR_ERR_INVALID_ARG: return "invalid argument";
    case GDR_ERR_UNSUPPORTED: return "unsupported problem";
    case GDR_ERR_WORKSPACE: return "workspace too small or misaligned";
    case GDR_ERR_HIP: return "HIP runtime error";
    case GDR_ERR_ARCH: return "device is not gfx950";
    default: return "unknown status";
  }
}

const char *gdr_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
