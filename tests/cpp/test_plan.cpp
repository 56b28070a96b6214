// Host-only unit tests of the planner and argument checks (no HIP).
// Built by tests/test_abi.py with g++ -fsanitize=address,undefined.
#include <cassert>
#include <cstdint>
#include <cstdio>
#include <string>
#include <vector>

#include "plan.h"

using namespace muon;

static int failures = 0;
#define CHECK(c)                                                         \
  do {                                                                   \
    if (!(c)) { std::printf("FAIL %s:%d %s\n", __FILE__, __LINE__, #c); ++failures; } \
  } while (0)

int main() {
  std::string err;
  // MoE bank: 256 x 2048x1408 (tall) + 256 x 1408x2048 -> one group, 3 batches.
  {
    std::vector<int> r, c;
    for (int i = 0; i < 256; ++i) { r.push_back(2048); c.push_back(1408); }
    for (int i = 0; i < 256; ++i) { r.push_back(1408); c.push_back(2048); }
    Plan p;
    CHECK(build_plan(r.data(), c.data(), 512, MUON_BF16, 0, 0, p, err) == MUON_OK);
    CHECK(p.batches.size() == 3);
    CHECK(p.batches[0].count == 171 && p.batches[1].count == 171 && p.batches[2].count == 170);
    for (auto& b : p.batches) {
      CHECK(b.m == 1408 && b.n == 2048 && b.m_pad == 1408 && b.n_pad == 2048);  // m: 128-granular
      CHECK((size_t)b.count * 1408 * 2048 <= MUON_DEFAULT_BATCH_CAP);
    }
    CHECK(p.transposed[0] == 1 && p.transposed[300] == 0);
    CHECK(p.order.size() == 512 && p.order[0] == 0 && p.order[511] == 511);
    Layout L = batch_layout(171, 1408, 2048, MUON_BF16);
    CHECK(L.x0 % 512 == 0 && L.x1 % 512 == 0 && L.a % 512 == 0 && L.b % 512 == 0);
    CHECK(L.partials % 512 == 0 && L.scales % 512 == 0);
    CHECK(L.ew_blocks == 22 * 32);
    CHECK(L.total >= (size_t)171 * (2 * 1408 * 2048 + 2 * 1408 * 1408) * 2);
    CHECK(p.workspace_bytes == L.total);
  }
  // MoE bank fitted to 256 compute units: 4 x 128 (tiles 18 and 44 per
  // matrix fill whole rounds: 2304 = 9 * 256, 5632 = 22 * 256) instead of
  // 171/171/170 (3078 tiles = 12 rounds + 6). fp32 is never refitted.
  {
    std::vector<int> r, c;
    for (int i = 0; i < 256; ++i) { r.push_back(2048); c.push_back(1408); }
    for (int i = 0; i < 256; ++i) { r.push_back(1408); c.push_back(2048); }
    Plan p, q;
    CHECK(build_plan(r.data(), c.data(), 512, MUON_BF16, 0, 256, p, err) == MUON_OK);
    CHECK(p.batches.size() == 4);
    for (auto& b : p.batches) CHECK(b.count == 128 && (size_t)b.count * 1408 * 2048 <= MUON_DEFAULT_BATCH_CAP);
    CHECK(build_plan(r.data(), c.data(), 512, MUON_F32, 0, 256, q, err) == MUON_OK);
    CHECK(q.batches.size() == 3);
  }
  // Mixed stack: groups in descending element count, balanced batches.
  {
    std::vector<int> r, c;
    for (int i = 0; i < 4; ++i) { r.push_back(7168); c.push_back(7168); }
    for (int i = 0; i < 2; ++i) { r.push_back(7168); c.push_back(18432); }
    for (int i = 0; i < 128; ++i) { r.push_back(7168); c.push_back(2048); }
    Plan p;
    CHECK(build_plan(r.data(), c.data(), (int)r.size(), MUON_BF16, 0, 0, p, err) == MUON_OK);
    CHECK(p.batches.size() == 1 + 1 + 4);
    CHECK(p.batches[0].m == 7168 && p.batches[0].n == 18432 && p.batches[0].count == 2);
    CHECK(p.batches[1].m == 7168 && p.batches[1].n == 7168 && p.batches[1].count == 4);
    for (int k = 2; k < 6; ++k) CHECK(p.batches[k].m == 2048 && p.batches[k].n == 7168 && p.batches[k].count == 32);
    CHECK(p.order[0] == 4 && p.order[1] == 5 && p.order[2] == 0);
  }
  // Ragged shapes pad to the dtype granularity; a matrix above the cap runs alone.
  {
    int r[3] = {5, 300, 3}, c[3] = {3, 130, 5};
    Plan p;
    CHECK(build_plan(r, c, 3, MUON_BF16, 0, 0, p, err) == MUON_OK);
    CHECK(p.batches.size() == 2);
    CHECK(p.batches[0].m == 130 && p.batches[0].n == 300 && p.batches[0].m_pad == 256 && p.batches[0].n_pad == 512);
    CHECK(p.batches[1].m_pad == 128 && p.batches[1].n_pad == 256);
    CHECK(p.batches[1].m == 3 && p.batches[1].n == 5 && p.batches[1].count == 2);
    CHECK(p.order[1] == 0 && p.order[2] == 2);
    Plan q;
    CHECK(build_plan(r, c, 3, MUON_F32, 100, 0, q, err) == MUON_OK);
    CHECK(q.batches.size() == 2);  // 15 elements fit two per batch under cap 100
    CHECK(q.batches[0].count == 1 && q.batches[0].m_pad == 192 && q.batches[0].n_pad == 320);
    Plan s;
    CHECK(build_plan(r, c, 3, MUON_F32, 10, 0, s, err) == MUON_OK);
    CHECK(s.batches.size() == 3);  // cap below one matrix: one per batch
  }
  // Errors.
  {
    int r[2] = {4, 0}, c[2] = {4, 4};
    Plan p;
    CHECK(build_plan(r, c, 2, MUON_BF16, 0, 0, p, err) == MUON_ERR_INVALID_ARGUMENT);
    CHECK(err.find("matrix 1") != std::string::npos);
    CHECK(build_plan(r, c, -1, MUON_BF16, 0, 0, p, err) == MUON_ERR_INVALID_ARGUMENT);
    CHECK(build_plan(r, c, 1, (muon_dtype)7, 0, 0, p, err) == MUON_ERR_INVALID_ARGUMENT);
    CHECK(build_plan(nullptr, nullptr, 0, MUON_BF16, 0, 0, p, err) == MUON_OK && p.batches.empty());
    CHECK(check_scalars(0.1f, 0.9f, 65, MUON_BF16, err) == MUON_ERR_INVALID_ARGUMENT);
    CHECK(check_scalars(0.1f, 0.9f, 5, MUON_BF16, err) == MUON_OK);
    CHECK(check_ptr(reinterpret_cast<void*>(uintptr_t(0x1008)), "params", 3, err) == MUON_ERR_MISALIGNED);
    CHECK(err == "params[3] is not 16-byte aligned");
    std::vector<Range> rg = {{0, 100, "params", 0}, {100, 200, "grads", 0}, {150, 160, "momentum", 1}};
    CHECK(check_no_overlap(rg, err) == MUON_ERR_INVALID_ARGUMENT);
    std::vector<Range> ok = {{0, 100, "params", 0}, {100, 200, "grads", 0}};
    CHECK(check_no_overlap(ok, err) == MUON_OK);
    muon_options o;
    default_options(o);
    CHECK(check_options(o, 5, err) == MUON_OK);
    o.scale_rule = 3;
    CHECK(check_options(o, 5, err) == MUON_ERR_INVALID_ARGUMENT);
  }
  std::printf(failures ? "planner tests: %d failures\n" : "planner tests: ok\n", failures);
  return failures ? 1 : 0;
}
