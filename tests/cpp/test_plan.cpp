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
    CHECK(o.ns_dtype == -1);
    o.scale_rule = 3;
    CHECK(check_options(o, 5, err) == MUON_ERR_INVALID_ARGUMENT);
    default_options(o);
    o.ns_dtype = 2;
    CHECK(check_options(o, 5, err) == MUON_ERR_INVALID_ARGUMENT);
    o.ns_dtype = MUON_BF16;
    CHECK(check_options(o, 5, err) == MUON_OK);
  }
  // Coefficient sets: a shape group splits by set, sets in ascending order
  // after the element-count order; a bad index is an error.
  {
    std::vector<int> r = {256, 384, 256, 100, 384}, c = {384, 256, 384, 60, 256}, set = {1, 0, 0, 1, 1};
    Plan p;
    CHECK(build_plan(r.data(), c.data(), 5, MUON_BF16, 0, 0, p, err, set.data(), 2) == MUON_OK);
    CHECK(p.batches.size() == 3);
    CHECK(p.batches[0].m == 256 && p.batches[0].n == 384 && p.batches[0].set == 0 && p.batches[0].count == 2);
    CHECK(p.batches[1].m == 256 && p.batches[1].n == 384 && p.batches[1].set == 1 && p.batches[1].count == 2);
    CHECK(p.batches[2].m == 60 && p.batches[2].set == 1 && p.batches[2].count == 1);
    CHECK(p.order[0] == 1 && p.order[1] == 2 && p.order[2] == 0 && p.order[3] == 4 && p.order[4] == 3);
    Plan q;
    CHECK(build_plan(r.data(), c.data(), 5, MUON_BF16, 0, 0, q, err) == MUON_OK);
    CHECK(q.batches.size() == 2 && q.batches[0].count == 4 && q.batches[0].set == 0);
    set[3] = 2;
    CHECK(build_plan(r.data(), c.data(), 5, MUON_BF16, 0, 0, p, err, set.data(), 2) == MUON_ERR_INVALID_ARGUMENT);
    CHECK(err.find("matrix 3") != std::string::npos);
    set[3] = -1;
    CHECK(build_plan(r.data(), c.data(), 5, MUON_BF16, 0, 0, p, err, set.data(), 2) == MUON_ERR_INVALID_ARGUMENT);
    CHECK(build_plan(r.data(), c.data(), 5, MUON_BF16, 0, 0, p, err, set.data(), 0) == MUON_ERR_INVALID_ARGUMENT);
    muon_options o;
    default_options(o);
    CHECK(o.poly_form == MUON_POLY_SQUARE && o.num_coeff_sets == 0);
    o.poly_form = MUON_POLY_FOLDED;
    CHECK(check_options(o, 5, err) == MUON_OK);
    o.poly_form = 3;
    CHECK(check_options(o, 5, err) == MUON_ERR_INVALID_ARGUMENT);
    default_options(o);
    o.num_coeff_sets = 1;
    CHECK(check_options(o, 5, err) == MUON_ERR_INVALID_ARGUMENT);   // tables missing
    float tab[15] = {3, -3, 1, 3, -3, 1, 3, -3, 1, 3, -3, 1, 3, -3, 1};
    int of[1] = {0};
    o.coeff_sets = tab;
    o.coeff_set_of = of;
    CHECK(check_options(o, 5, err) == MUON_OK);
    o.coeffs = tab;
    CHECK(check_options(o, 5, err) == MUON_ERR_INVALID_ARGUMENT);   // coeffs and sets together
    o.coeffs = nullptr;
    tab[7] = 1.0f / 0.0f;
    CHECK(check_options(o, 5, err) == MUON_ERR_INVALID_ARGUMENT);
  }
  // Workspace bound: batches hold as many matrices as fit in max_ws bytes;
  // a matrix that alone needs more is an error naming it.
  {
    std::vector<int> r(40, 1408), c(40, 2048);
    const size_t one = batch_layout(1, 1408, 2048, MUON_BF16).total;
    const size_t lim = batch_layout(7, 1408, 2048, MUON_BF16).total;
    Plan p;
    CHECK(build_plan(r.data(), c.data(), 40, MUON_BF16, 0, 0, p, err, nullptr, 0, lim) == MUON_OK);
    CHECK(p.batches.size() == 6);   // 40 = 7+7+7+7+6+6 in balanced batches of at most 7
    for (auto& b : p.batches) CHECK(b.count <= 7 && b.count >= 6);
    CHECK(p.workspace_bytes <= lim);
    CHECK(build_plan(r.data(), c.data(), 40, MUON_BF16, 0, 256, p, err, nullptr, 0, lim) == MUON_OK);
    CHECK(p.workspace_bytes <= lim);   // no refit beyond the bound
    CHECK(build_plan(r.data(), c.data(), 40, MUON_BF16, 0, 0, p, err, nullptr, 0, one - 1) == MUON_ERR_INVALID_ARGUMENT);
    CHECK(err.find("matrix 0 (1408 x 2048)") != std::string::npos);
  }
  // Strided views of one parameter (bytes; a 4 x 64-byte parameter at 0x1000).
  {
    const auto at = [](unsigned long long a) { return reinterpret_cast<const void*>(uintptr_t(a)); };
    // Interleaved rows (even / odd rows, stride 128): disjoint.
    std::vector<Range> il = {strided_range(at(0x1000), 2, 64, 128, "params", 0),
                             strided_range(at(0x1040), 2, 64, 128, "params", 1)};
    CHECK(check_no_overlap(il, err) == MUON_OK);
    // Column halves (32 bytes each of 64-byte rows): disjoint; a third view
    // covering bytes 16..48 of every row meets both.
    std::vector<Range> ch = {strided_range(at(0x1000), 4, 32, 64, "params", 0),
                             strided_range(at(0x1020), 4, 32, 64, "params", 1)};
    CHECK(check_no_overlap(ch, err) == MUON_OK);
    ch.push_back(strided_range(at(0x1010), 4, 32, 64, "params", 2));
    CHECK(check_no_overlap(ch, err) == MUON_ERR_INVALID_ARGUMENT);
    // A view whose rows wrap into the next row of the other: row 0 of b
    // covers bytes 48..80, i.e. byte 0..16 of a's row 1.
    std::vector<Range> wr = {strided_range(at(0x1000), 2, 16, 64, "params", 0),
                             strided_range(at(0x1030), 1, 32, 64, "grads", 0)};
    CHECK(check_no_overlap(wr, err) == MUON_ERR_INVALID_ARGUMENT);
    std::vector<Range> wr_ok = {strided_range(at(0x1000), 1, 16, 64, "params", 0),
                                strided_range(at(0x1030), 1, 32, 64, "grads", 0)};
    CHECK(check_no_overlap(wr_ok, err) == MUON_OK);
    // Row blocks below one another: disjoint; one row more and they meet.
    std::vector<Range> rb = {strided_range(at(0x1000), 2, 64, 64, "params", 0),
                             strided_range(at(0x1080), 2, 64, 64, "params", 1)};
    CHECK(check_no_overlap(rb, err) == MUON_OK);
    rb[0] = strided_range(at(0x1000), 3, 64, 64, "params", 0);
    CHECK(check_no_overlap(rb, err) == MUON_ERR_INVALID_ARGUMENT);
    // Different strides with intersecting spans count as overlapping.
    std::vector<Range> ds = {strided_range(at(0x1000), 2, 32, 128, "params", 0),
                             strided_range(at(0x1040), 2, 32, 64, "params", 1)};
    CHECK(check_no_overlap(ds, err) == MUON_ERR_INVALID_ARGUMENT);
    // A long block that meets a block two places after it in address order.
    std::vector<Range> far = {strided_range(at(0x1000), 4, 16, 64, "params", 0),
                              strided_range(at(0x1010), 1, 16, 64, "params", 1),
                              strided_range(at(0x1020), 1, 16, 64, "params", 2),
                              strided_range(at(0x10c0), 1, 16, 64, "params", 3)};
    CHECK(check_no_overlap(far, err) == MUON_ERR_INVALID_ARGUMENT);
    CHECK(err == "params[0] overlaps params[3]");
  }
  std::printf(failures ? "planner tests: %d failures\n" : "planner tests: ok\n", failures);
  return failures ? 1 : 0;
}
