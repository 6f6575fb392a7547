// Test driver for the library's host-only code (csrc/dah_host.cpp: argument
// validation, the split planner, status strings and the per-thread last
// error), built as plain host C++ so that it can run under AddressSanitizer
// and UndefinedBehaviorSanitizer.  Every case states the status it expects;
// the driver prints one line per failure and "checks N failures F" at the end
// and exits non-zero on any failure.  No pointer passed here is ever
// dereferenced: validation rejects or accepts addresses without reading them.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <thread>

#include "dah.h"
#include "dah_host.h"

namespace {

int g_checks = 0, g_failures = 0;

void expect(int got, int want, const char* what, int line) {
  ++g_checks;
  if (got != want) {
    ++g_failures;
    printf("FAIL line %d: %s returned %d, expected %d (last error: %s)\n", line, what, got, want,
           dah_last_error());
  }
}

#define EXPECT(call, want) expect((call), (want), #call, __LINE__)

// Fake, aligned addresses (never dereferenced).
const void* const A = reinterpret_cast<const void*>(uintptr_t{0x100000});
const void* at(uintptr_t off) { return reinterpret_cast<const void*>(uintptr_t{0x100000} + off); }

struct Dec {
  const void *q = A, *k = A, *v = A, *bt = A, *sl = A, *o = A;
  int dt = DAH_BF16, mpps = 4, B = 2, heads = 16, max_len = 64, ns = 0;
  int64_t num_pages = 16;
  int run() const {
    return dah::validate_decode(q, k, v, dt, num_pages, bt, mpps, sl, B, heads, max_len, ns, o);
  }
};

struct App {
  const void *q = A, *kn = A, *vn = A, *qg = A, *kg = A, *k = A, *v = A, *bt = A, *sl = A,
             *qo = A;
  float eps = 1e-6f, theta = 1e6f;
  int dt = DAH_BF16, mpps = 4, B = 2, heads = 16;
  int64_t num_pages = 16;
  int run() const {
    return dah::validate_append(q, kn, vn, qg, kg, eps, theta, k, v, dt, num_pages, bt, mpps, sl,
                                B, heads, qo);
  }
};

void decode_cases() {
  EXPECT(Dec{}.run(), DAH_OK);
  { Dec d; d.q = nullptr; EXPECT(d.run(), DAH_ERR_NULL); }
  { Dec d; d.k = nullptr; EXPECT(d.run(), DAH_ERR_NULL); }
  { Dec d; d.v = nullptr; EXPECT(d.run(), DAH_ERR_NULL); }
  { Dec d; d.bt = nullptr; EXPECT(d.run(), DAH_ERR_NULL); }
  { Dec d; d.sl = nullptr; EXPECT(d.run(), DAH_ERR_NULL); }
  { Dec d; d.o = nullptr; EXPECT(d.run(), DAH_ERR_NULL); }
  { Dec d; d.dt = 2; EXPECT(d.run(), DAH_ERR_DTYPE); }
  { Dec d; d.dt = -1; EXPECT(d.run(), DAH_ERR_DTYPE); }
  { Dec d; d.B = 0; EXPECT(d.run(), DAH_ERR_SHAPE); }
  { Dec d; d.B = -5; EXPECT(d.run(), DAH_ERR_SHAPE); }
  { Dec d; d.num_pages = 0; EXPECT(d.run(), DAH_ERR_SHAPE); }
  { Dec d; d.num_pages = int64_t{1} << 31; EXPECT(d.run(), DAH_ERR_SHAPE); }
  { Dec d; d.mpps = 0; EXPECT(d.run(), DAH_ERR_SHAPE); }
  { Dec d; d.max_len = 0; EXPECT(d.run(), DAH_ERR_SHAPE); }
  { Dec d; d.max_len = 65; EXPECT(d.run(), DAH_ERR_SHAPE); }
  { Dec d; d.mpps = 1 << 30; d.max_len = 1 << 30; EXPECT(d.run(), DAH_OK); }  // no overflow
  { Dec d; d.ns = -1; EXPECT(d.run(), DAH_ERR_SHAPE); }
  { Dec d; d.heads = 24; EXPECT(d.run(), DAH_ERR_SHAPE); }
  { Dec d; d.q = at(4); EXPECT(d.run(), DAH_ERR_ALIGN); }
  { Dec d; d.o = at(8); EXPECT(d.run(), DAH_ERR_ALIGN); }
  { Dec d; d.k = at(2); EXPECT(d.run(), DAH_ERR_ALIGN); }
  { Dec d; d.bt = at(2); EXPECT(d.run(), DAH_ERR_ALIGN); }
  for (int h : {16, 32, 40, 64}) { Dec d; d.heads = h; EXPECT(d.run(), DAH_OK); }
}

void append_cases() {
  EXPECT(App{}.run(), DAH_OK);
  const void* App::*ptrs[] = {&App::q, &App::kn, &App::vn, &App::qg, &App::kg,
                              &App::k, &App::v,  &App::bt, &App::sl, &App::qo};
  for (auto m : ptrs) { App a; a.*m = nullptr; EXPECT(a.run(), DAH_ERR_NULL); }
  { App a; a.dt = 7; EXPECT(a.run(), DAH_ERR_DTYPE); }
  { App a; a.B = 0; EXPECT(a.run(), DAH_ERR_SHAPE); }
  { App a; a.num_pages = 0; EXPECT(a.run(), DAH_ERR_SHAPE); }
  { App a; a.mpps = 0; EXPECT(a.run(), DAH_ERR_SHAPE); }
  { App a; a.eps = -1.0f; EXPECT(a.run(), DAH_ERR_SHAPE); }
  { App a; a.eps = __builtin_nanf(""); EXPECT(a.run(), DAH_ERR_SHAPE); }
  { App a; a.theta = 0.0f; EXPECT(a.run(), DAH_ERR_SHAPE); }
  { App a; a.q = at(4); EXPECT(a.run(), DAH_ERR_ALIGN); }
  { App a; a.qo = at(4); EXPECT(a.run(), DAH_ERR_ALIGN); }
  { App a; a.kn = at(8); EXPECT(a.run(), DAH_ERR_ALIGN); }
  { App a; a.v = at(2); EXPECT(a.run(), DAH_ERR_ALIGN); }
  { App a; a.sl = at(1); EXPECT(a.run(), DAH_ERR_ALIGN); }
  { App a; a.heads = 65; EXPECT(a.run(), DAH_ERR_SHAPE); }
}

void chunk_cases() {
  auto chunk = [](const void* cu, int total, int max_chunk, int max_len, const void* o, int B) {
    return dah::validate_chunk(A, A, A, A, A, 1e-6f, 1e6f, A, A, DAH_BF16, 16, A, 4, A, cu, B,
                               total, max_chunk, max_len, 16, A, o);
  };
  EXPECT(chunk(A, 8, 4, 64, A, 2), DAH_OK);
  EXPECT(chunk(nullptr, 8, 4, 64, A, 2), DAH_ERR_NULL);
  EXPECT(chunk(A, 8, 4, 64, nullptr, 2), DAH_ERR_NULL);
  EXPECT(chunk(A, 0, 1, 64, A, 2), DAH_ERR_SHAPE);
  EXPECT(chunk(A, 8, 0, 64, A, 2), DAH_ERR_SHAPE);
  EXPECT(chunk(A, 8, 9, 64, A, 2), DAH_ERR_SHAPE);
  EXPECT(chunk(A, 8, 4, 65, A, 2), DAH_ERR_SHAPE);
  EXPECT(chunk(A, 8, 4, 0, A, 2), DAH_ERR_SHAPE);
  EXPECT(chunk(at(2), 8, 4, 64, A, 2), DAH_ERR_ALIGN);
  EXPECT(chunk(A, 8, 4, 64, at(4), 2), DAH_ERR_ALIGN);
  EXPECT(chunk(A, 1 << 30, 1 << 30, 64, A, 1 << 20), DAH_ERR_SHAPE);  // B * max_chunk overflows
}

void linear_cases() {
  EXPECT(dah::validate_linear(A, A, 256, 4096, 1024, A), DAH_OK);
  EXPECT(dah::validate_linear(nullptr, A, 1, 64, 256, A), DAH_ERR_NULL);
  EXPECT(dah::validate_linear(A, nullptr, 1, 64, 256, A), DAH_ERR_NULL);
  EXPECT(dah::validate_linear(A, A, 1, 64, 256, nullptr), DAH_ERR_NULL);
  EXPECT(dah::validate_linear(A, A, 0, 64, 256, A), DAH_ERR_SHAPE);
  EXPECT(dah::validate_linear(A, A, 1, 96, 256, A), DAH_ERR_SHAPE);
  EXPECT(dah::validate_linear(A, A, 1, 0, 256, A), DAH_ERR_SHAPE);
  EXPECT(dah::validate_linear(A, A, 1, 64, 300, A), DAH_ERR_SHAPE);
  EXPECT(dah::validate_linear(A, A, 1 << 30, 64, 1 << 20, A), DAH_ERR_SHAPE);  // T*K too large
  EXPECT(dah::validate_linear(at(4), A, 1, 64, 256, A), DAH_ERR_ALIGN);
  EXPECT(dah::validate_linear(A, A, 1, 64, 256, at(8)), DAH_ERR_ALIGN);
}

// Every plan is consistent with its inputs over a grid of shapes, including
// ones whose page and workgroup counts approach the int range.
void planner_cases() {
  const int shapes[][2] = {{1, 1},       {2, 12},     {32, 4096},  {256, 2048}, {4, 40960},
                           {128, 16384}, {256, 40960}, {1, 17},     {7, 999},    {4096, 64},
                           {5000, 2048}, {1, 1 << 30}, {4096, 1 << 30}, {1 << 20, 40960}};
  const int splits[] = {0, 1, 2, 3, 7, 16, 1000, 1 << 30};
  for (auto& sh : shapes)
    for (int n : splits)
      for (int h : {16, 64})
        for (int dt : {DAH_F32, DAH_BF16}) {
          dah::Plan p;
          const int st = dah::plan_decode(sh[0], h, dt, sh[1], n, 256, &p);
          if (st != DAH_OK) {
            // only a grid too large for int may be refused
            EXPECT(st, DAH_ERR_SHAPE);
            continue;
          }
          ++g_checks;
          const long long pages = (sh[1] + 15LL) / 16;
          bool ok = p.workgroups >= 1 && p.mode >= 0 && p.mode <= 2;
          if (p.mode == DAH_PLAN_SPLIT)
            ok = ok && p.splits > 1 && p.grid_splits % 8 == 0 && p.grid_splits >= p.splits &&
                 (long long)p.splits * p.pages_per_split >= pages &&
                 (long long)(p.splits - 1) * p.pages_per_split < pages && p.workspace > 0;
          if (p.mode == DAH_PLAN_PER_SEQUENCE) ok = ok && p.workgroups == sh[0] && p.workspace == 0;
          if (p.mode == DAH_PLAN_BALANCED) ok = ok && sh[0] <= dah::kMaxBalancedBatch;
          if (p.mfma) ok = ok && dt == DAH_BF16;
          if (!ok) {
            ++g_failures;
            printf("FAIL plan B=%d L=%d n=%d H=%d dt=%d: mode %d splits %d pps %d wg %d\n", sh[0],
                   sh[1], n, h, dt, p.mode, p.splits, p.pages_per_split, p.workgroups);
          }
        }
  dah::Plan p;
  EXPECT(dah::plan_decode(0, 16, DAH_BF16, 10, 0, 256, &p), DAH_ERR_SHAPE);
  EXPECT(dah::plan_decode(1, 16, DAH_BF16, 0, 0, 256, &p), DAH_ERR_SHAPE);
  EXPECT(dah::plan_decode(1, 16, DAH_BF16, 10, -1, 256, &p), DAH_ERR_SHAPE);
  EXPECT(dah::plan_decode(1, 16, DAH_BF16, 10, 0, 0, &p), DAH_ERR_SHAPE);
  EXPECT(dah::plan_decode(1, 12, DAH_BF16, 10, 0, 256, &p), DAH_ERR_SHAPE);
  EXPECT(dah::plan_decode(1, 16, DAH_BF16, 10, 0, 256, nullptr), DAH_ERR_NULL);
  dah_decode_plan cp;
  EXPECT(dah_plan_decode_ex(8, 32, 2, 64, 0, 256, &cp), DAH_ERR_DTYPE);
  EXPECT(dah_plan_decode_ex(8, 32, DAH_BF16, 64, 0, 256, nullptr), DAH_ERR_NULL);
  EXPECT(dah_plan_decode(256, 2048, 0, 256, &cp), DAH_OK);
  EXPECT(cp.mode, DAH_PLAN_PER_SEQUENCE);
  EXPECT(dah_workspace_bytes_for(0, 64, 0, 256) == 0, 1);
}

void status_cases() {
  const char* names[] = {"DAH_OK",           "DAH_ERR_NULL",  "DAH_ERR_SHAPE", "DAH_ERR_DTYPE",
                         "DAH_ERR_ALIGN",    "DAH_ERR_WORKSPACE", "DAH_ERR_HIP"};
  for (int i = 0; i < 7; ++i) EXPECT(strcmp(dah_status_string(i), names[i]), 0);
  EXPECT(strcmp(dah_status_string(99), "unknown status"), 0);
  EXPECT(strcmp(dah_status_string(-1), "unknown status"), 0);
  // a message longer than the buffer is truncated, never overrun
  char big[2048];
  memset(big, 'x', sizeof(big) - 1);
  big[sizeof(big) - 1] = '\0';
  EXPECT(dah::set_error(DAH_ERR_SHAPE, "%s", big), DAH_ERR_SHAPE);
  EXPECT(strlen(dah_last_error()) < sizeof(big) - 1, 1);
  dah::clear_error();
  EXPECT((int)strlen(dah_last_error()), 0);
  // the last error is per thread
  Dec bad;
  bad.B = 0;
  EXPECT(bad.run(), DAH_ERR_SHAPE);
  int other_len = -1;
  std::thread t([&] { other_len = (int)strlen(dah_last_error()); });
  t.join();
  EXPECT(other_len, 0);
  EXPECT(strlen(dah_last_error()) > 0, 1);
}

}  // namespace

int main() {
  decode_cases();
  append_cases();
  chunk_cases();
  linear_cases();
  planner_cases();
  status_cases();
  printf("checks %d failures %d\n", g_checks, g_failures);
  return g_failures == 0 ? 0 : 1;
}
