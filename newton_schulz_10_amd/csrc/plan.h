// Host-side planning for the batched Muon step: shape grouping, batch
// splitting, execution order and workspace layout. No HIP dependency, so
// the planner builds and is tested on a host without a GPU.
//
// Source: arXiv:2609.21594 (HyperParallel-FSDP), section 6.6 (matrices are
// grouped by core shape and fused along a batch axis; tall matrices are
// transposed first; the NS workspace is allocated once per batched
// invocation; batches are capped at 2^29 elements) and section 6.7
// (batches are issued largest matrices first).
#pragma once

#include <cstddef>
#include <string>
#include <vector>

#include "muon.h"

namespace muon {

// Element tile of the momentum/apply passes (wide orientation).
constexpr int kEwTile = 64;
// bf16 GEMM tile scheduler words per batch: 8 per-XCD tile counters, one
// completion counter, padding to 16, then one broadcast slot per workgroup
// (at most kSchedSlots workgroups use the dynamic schedule).
constexpr int kSchedSlots = 1024;
constexpr int kSchedWords = 16 + kSchedSlots;

// One fused batch; m <= n is the group's wide shape.
struct Batch {
  int group;
  int m, n;
  int m_pad, n_pad;
  int first;   // offset into Plan::order
  int count;
  int set;     // coefficient set of every matrix of the batch (0 without sets)
};

struct Plan {
  std::vector<Batch> batches;             // execution order
  std::vector<int> order;                 // matrix indices, execution order
  std::vector<unsigned char> transposed;  // per input matrix: rows > cols
  size_t workspace_bytes = 0;
};

// Byte offsets of one batch's workspace regions (each 512-byte aligned).
struct Layout {
  size_t x0 = 0, x1 = 0, a = 0, b = 0, partials = 0, nonzero = 0, scales = 0, live = 0, live_list = 0,
         nlive = 0, ptab = 0, sched = 0, total = 0;
  size_t mat_x = 0;     // elements per padded m_pad x n_pad matrix
  size_t mat_a = 0;     // elements per padded m_pad x m_pad matrix
  int ew_blocks = 0;    // elementwise tiles per matrix
};

// Padding granularity of the GEMM kernels for a dtype: the wide matrix's
// rows (m) and columns (n) are rounded up to these (bf16: m to 128, with
// half-height tiles covering an odd multiple; n to 256). The padding holds
// zeros, which the NS iteration keeps at zero.
int pad_granularity_m(muon_dtype dtype);
int pad_granularity_n(muon_dtype dtype);
size_t dtype_size(muon_dtype dtype);

Layout batch_layout(int count, int m_pad, int n_pad, muon_dtype dtype);

// Groups matrices by {min, max} and, when `set_of` is given, by their
// coefficient set set_of[i] in [0, num_sets); orders groups by descending
// rows*cols (then set); splits each group into balanced batches of at most
// `cap` elements and, when max_ws > 0, of at most max_ws workspace bytes.
// With cus > 0 (bf16), the number of batches is the one, among the fewest
// and a few more, whose GEMM tiles best fill whole rounds of `cus` compute
// units. Returns MUON_OK, or MUON_ERR_INVALID_ARGUMENT with `err` set (a
// bad shape or set index, or one matrix whose workspace exceeds max_ws).
int build_plan(const int* rows, const int* cols, int num, muon_dtype dtype, size_t cap, int cus,
               Plan& out, std::string& err, const int* set_of = nullptr, int num_sets = 0,
               size_t max_ws = 0);

// Option defaults and validation.
void default_options(muon_options& o);
int check_options(const muon_options& o, int ns_steps, std::string& err);

// Argument checks shared by the entry points (no device access).
int check_scalars(float lr, float beta, int ns_steps, muon_dtype dtype, std::string& err);
int check_shape(int m, int n, std::string& err, int index = -1);
int check_ptr(const void* p, const char* what, int index, std::string& err);

// The matrices (params, grads, momentum of all matrices) must not share
// any byte. Each is a strided block: `rows` rows of `row_bytes` bytes,
// `ld_bytes` apart, from `lo`; a contiguous matrix is the case ld_bytes ==
// row_bytes. Blocks whose spans [lo, hi) intersect are compared exactly
// when their strides are equal (interleaved views of one parameter) and
// count as overlapping otherwise.
struct Range {
  unsigned long long lo, hi;   // span: hi = lo + (rows-1)*ld_bytes + row_bytes
  const char* what;
  int index;
  unsigned long long rows, row_bytes, ld_bytes;
};
Range strided_range(const void* p, unsigned long long rows, unsigned long long row_bytes,
                    unsigned long long ld_bytes, const char* what, int index);
int check_no_overlap(std::vector<Range>& ranges, std::string& err);

}  // namespace muon
