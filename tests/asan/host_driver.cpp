// Drives libgdr's host code (chunk planner, workspace sizer, argument and
// workspace validation of every entry point, layout query) under
// AddressSanitizer and UndefinedBehaviorSanitizer, on a machine without a GPU.
// The kernel launchers are replaced by stubs that count calls: no path here may
// reach a launch (invalid arguments are refused before, and a valid problem
// stops at the device check).  The chunk tables of thousands of random packs are
// checked entry by entry against every index the kernels take from them.
// Exit status 0 when every check holds.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdio>
#include <cstring>
#include <random>
#include <vector>

#include "gdr.h"
#include "gdr_kernels.h"

static int g_launches = 0;
namespace gdr {
int compute_units() { return 256; }
hipError_t launch_fwd_prep(bool, const Problem &, const Workspace &, bool, bool, hipStream_t) { ++g_launches; return hipErrorUnknown; }
hipError_t launch_fwd_walk(bool, const Problem &, const Workspace &, uint16_t *, float *, bool, bool, hipStream_t) { ++g_launches; return hipErrorUnknown; }
hipError_t launch_bwd_walk(bool, const Problem &, const Workspace &, const uint16_t *, const float *, float *, hipStream_t) { ++g_launches; return hipErrorUnknown; }
hipError_t launch_bwd_grad(bool, const Problem &, const Workspace &, const uint16_t *, uint16_t *, uint16_t *, uint16_t *, float *, void *, hipStream_t) { ++g_launches; return hipErrorUnknown; }
}  // namespace gdr

static int g_fail = 0;
#define CHECK(c)                                                   \
  do {                                                             \
    if (!(c)) {                                                    \
      std::fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__); \
      ++g_fail;                                                    \
    }                                                              \
  } while (0)

// Every index a kernel takes from the table lies in range and the table
// describes exactly the documents of cu.
static void check_table(const std::vector<int32_t> &cu, const std::vector<int32_t> &t, int NC) {
  const int N = (int)cu.size() - 1, T = cu[N];
  const int32_t *start = t.data(), *len = start + NC, *doc = len + NC, *ptr = doc + NC, *order = ptr + N + 1;
  for (int c = 0; c < NC; ++c) {
    CHECK(doc[c] >= 0 && doc[c] < N);
    CHECK(len[c] >= 1 && len[c] <= 64);
    CHECK(start[c] >= 0 && start[c] + len[c] <= T);
    if (doc[c] >= 0 && doc[c] < N) {
      CHECK(start[c] >= cu[doc[c]] && start[c] + len[c] <= cu[doc[c] + 1]);
      CHECK((start[c] - cu[doc[c]]) % 64 == 0);
      CHECK(c >= ptr[doc[c]] && c < ptr[doc[c] + 1]);
    }
  }
  CHECK(ptr[0] == 0 && ptr[N] == NC);
  for (int n = 0; n < N; ++n) {
    CHECK(ptr[n] <= ptr[n + 1]);
    CHECK(ptr[n + 1] - ptr[n] == (cu[n + 1] - cu[n] + 63) / 64);
  }
  std::vector<int> seen(N, 0);
  for (int r = 0; r < N; ++r) {
    CHECK(order[r] >= 0 && order[r] < N);
    if (order[r] < 0 || order[r] >= N) continue;
    ++seen[order[r]];
    if (r > 0) {
      const int a = order[r - 1], b = order[r], ca = ptr[a + 1] - ptr[a], cb = ptr[b + 1] - ptr[b];
      CHECK(ca > cb || (ca == cb && a < b));
    }
  }
  for (int n = 0; n < N; ++n) CHECK(seen[n] == 1);
}

static gdr_problem valid_problem(const std::vector<int32_t> &table, int T, int N, int NC, int Hqk, int Hv, void *buf) {
  gdr_problem p;
  std::memset(&p, 0, sizeof p);
  p.T = T; p.N = N; p.H_qk = Hqk; p.H_v = Hv; p.K = 128; p.V = 128;
  const uint16_t *d = static_cast<const uint16_t *>(buf);  // never dereferenced: no launch happens here
  p.q = d; p.k = d; p.v = d; p.g = static_cast<const float *>(buf); p.beta = buf;
  p.cu_seqlens = static_cast<const int32_t *>(buf);
  p.chunk_table = table.data();
  p.n_chunks = NC;
  p.scale = 0.088388f;
  return p;
}

int main() {
  std::mt19937 rng(1234);
  // ---- planner ----
  for (int trial = 0; trial < 3000; ++trial) {
    const int N = trial % 50 == 0 ? 0 : (int)(rng() % 40) + 1;
    std::vector<int32_t> cu(N + 1, 0);
    for (int n = 0; n < N; ++n) {
      const unsigned r = rng() % 10;
      const int len = r == 0 ? 0 : (r == 1 ? 1 : (r == 2 ? 64 * (int)(1 + rng() % 5) : (int)(rng() % 400)));
      cu[n + 1] = cu[n] + len;
    }
    int32_t nc = -1;
    int64_t tl = -1;
    CHECK(gdr_plan_chunks(cu.data(), N, nullptr, 0, &nc, &tl) == GDR_OK);
    CHECK(tl == 3 * (int64_t)nc + 2 * N + 1);
    std::vector<int32_t> table(tl + 8, -77);  // sentinel past the end
    if (tl > 0) CHECK(gdr_plan_chunks(cu.data(), N, table.data(), tl - 1, nullptr, nullptr) == GDR_ERR_INVALID_ARG);
    CHECK(gdr_plan_chunks(cu.data(), N, table.data(), tl, &nc, &tl) == GDR_OK);
    for (int i = 0; i < 8; ++i) CHECK(table[tl + i] == -77);
    table.resize(tl);
    check_table(cu, table, nc);
  }
  {
    const int32_t bad0[2] = {1, 5}, bad1[3] = {0, 5, 3};
    int32_t nc;
    int64_t tl;
    CHECK(gdr_plan_chunks(bad0, 1, nullptr, 0, &nc, &tl) == GDR_ERR_INVALID_ARG);
    CHECK(gdr_plan_chunks(bad1, 2, nullptr, 0, &nc, &tl) == GDR_ERR_INVALID_ARG);
    CHECK(gdr_plan_chunks(nullptr, 1, nullptr, 0, &nc, &tl) == GDR_ERR_INVALID_ARG);
    CHECK(gdr_plan_chunks(bad0, -1, nullptr, 0, &nc, &tl) == GDR_ERR_INVALID_ARG);
    CHECK(std::strlen(gdr_last_error()) > 0);
  }
  // ---- workspace sizer ----
  for (int trial = 0; trial < 2000; ++trial) {
    const int variant = (int)(rng() % 2), N = 1 + (int)(rng() % 20), Hqk = 1 + (int)(rng() % 8);
    const int Hv = variant ? Hqk * (1 + (int)(rng() % 4)) : Hqk, NCmin = 1 + (int)(rng() % 300);
    const int T = 64 * (NCmin - 1) + 1 + (int)(rng() % 64), NC = (T + 63) / 64 + (int)(rng() % (N + 1));
    for (uint32_t flags : {0u, (uint32_t)GDR_FWD_SAVE}) {
      const int64_t b = gdr_workspace_bytes(variant, T, N, NC, Hqk, Hv, 128, 128, flags);
      // every chunk holds 1..64 tokens of one document: ceil(T/64) <= NC <= min(T, ceil(T/64) + N)
      if (NC > (T + 63) / 64 + N || NC > T) CHECK(b == -GDR_ERR_INVALID_ARG);
      else CHECK(b > 0 && b % 256 == 0);
    }
  }
  CHECK(gdr_workspace_bytes(GDR_KDA, 64, 1, 1, 1, 1, 64, 128, 0) == -GDR_ERR_UNSUPPORTED);
  CHECK(gdr_workspace_bytes(GDR_KDA, 64, 1, 1, 2, 1, 128, 128, 0) == -GDR_ERR_UNSUPPORTED);
  CHECK(gdr_workspace_bytes(7, 64, 1, 1, 1, 1, 128, 128, 0) == -GDR_ERR_INVALID_ARG);
  CHECK(gdr_workspace_bytes(GDR_KDA, 64, 1, 1, 1, 1, 128, 128, 8u) == -GDR_ERR_INVALID_ARG);
  // ---- validation of the entry points (nothing may be launched) ----
  {
    const std::vector<int32_t> cu = {0, 100, 100, 357};
    int32_t nc;
    int64_t tl;
    CHECK(gdr_plan_chunks(cu.data(), 3, nullptr, 0, &nc, &tl) == GDR_OK);
    std::vector<int32_t> table(tl);
    CHECK(gdr_plan_chunks(cu.data(), 3, table.data(), tl, &nc, &tl) == GDR_OK);
    alignas(256) static unsigned char buf[1 << 16];
    uint16_t *o = reinterpret_cast<uint16_t *>(buf);
    float *f = reinterpret_cast<float *>(buf);
    for (int variant : {GDR_KDA, GDR_GDN}) {
      const int Hqk = 2, Hv = variant == GDR_KDA ? 2 : 6;
      gdr_problem p = valid_problem(table, 357, 3, nc, Hqk, Hv, buf);
      const int64_t need = gdr_workspace_bytes(variant, 357, 3, nc, Hqk, Hv, 128, 128, GDR_FWD_SAVE);
      auto fwd = variant == GDR_KDA ? gdr_kda_fwd : gdr_gdn_fwd;
      auto bwd = variant == GDR_KDA ? gdr_kda_bwd : gdr_gdn_bwd;
      auto ckpt = variant == GDR_KDA ? gdr_kda_ckpt : gdr_gdn_ckpt;
      CHECK(fwd(nullptr, o, f, buf, need, 0, nullptr) == GDR_ERR_INVALID_ARG);
      CHECK(fwd(&p, o, f, buf, need - 256, GDR_FWD_SAVE, nullptr) == GDR_ERR_WORKSPACE);
      CHECK(fwd(&p, o, f, buf + 16, need, 0, nullptr) == GDR_ERR_WORKSPACE);
      CHECK(fwd(&p, o, f, buf, need, 4u, nullptr) == GDR_ERR_INVALID_ARG);
      CHECK(fwd(&p, nullptr, f, buf, need, 0, nullptr) == GDR_ERR_INVALID_ARG);
      CHECK(bwd(&p, o, f, nullptr, o, o, f, buf, f, buf, need, nullptr) == GDR_ERR_INVALID_ARG);
      CHECK(ckpt(&p, o, f, o, f, o, o, o, f, buf, f, buf, need - 1, nullptr) == GDR_ERR_WORKSPACE);
      gdr_problem q = p;
      q.K = 64;
      CHECK(fwd(&q, o, f, buf, need, 0, nullptr) == GDR_ERR_UNSUPPORTED);
      q = p; q.q = nullptr;
      CHECK(fwd(&q, o, f, buf, need, 0, nullptr) == GDR_ERR_INVALID_ARG);
      q = p; q.n_chunks = nc + 5;
      CHECK(fwd(&q, o, f, buf, need, 0, nullptr) == GDR_ERR_INVALID_ARG);
      q = p; q.walk_segments = -1;
      CHECK(fwd(&q, o, f, buf, need, 0, nullptr) == GDR_ERR_INVALID_ARG);
      q = p; q.walk_layout = 3;
      CHECK(fwd(&q, o, f, buf, need, 0, nullptr) == GDR_ERR_INVALID_ARG);
      q = p; q.walk_plan = 2;
      CHECK(fwd(&q, o, f, buf, need, 0, nullptr) == GDR_ERR_INVALID_ARG);
      q = p; q.input_flags = 4;
      CHECK(fwd(&q, o, f, buf, need, 0, nullptr) == GDR_ERR_INVALID_ARG);
      q = p; q.max_doc_chunks = nc + 1;
      CHECK(fwd(&q, o, f, buf, need, 0, nullptr) == GDR_ERR_INVALID_ARG);
      q = p; q.scale = __builtin_nanf("");
      CHECK(fwd(&q, o, f, buf, need, 0, nullptr) == GDR_ERR_INVALID_ARG);
      // a valid call stops at the device check (no GPU here)
      const int32_t rc = fwd(&p, o, f, buf, need, GDR_FWD_SAVE, nullptr);
      CHECK(rc == GDR_ERR_HIP || rc == GDR_ERR_ARCH);
      int32_t layout = -1;
      CHECK(gdr_walk_layout_chosen(variant, &p, 256, &layout) == GDR_OK);
      CHECK(layout == GDR_WALK_SLICES || layout == GDR_WALK_RINGS);
      CHECK(gdr_walk_layout_chosen(variant, &p, -1, &layout) == GDR_ERR_INVALID_ARG);
    }
    gdr_problem p = valid_problem(table, 357, 3, nc, 2, 2, buf);
    const int32_t rc = gdr_kda_ckpt_noalloc(&p, o, f, o, f, o, o, o, f, buf, f, nullptr);
    CHECK(rc == GDR_ERR_HIP || rc == GDR_ERR_ARCH);
  }
  for (int s = 0; s <= 6; ++s) CHECK(gdr_status_string(s) != nullptr);
  CHECK(g_launches == 0);
  std::printf("host driver: %d failures, %d launches\n", g_fail, g_launches);
  return g_fail != 0;
}
