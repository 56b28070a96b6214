// HBM-bound passes of the batched Muon step: momentum (+ transpose to the
// wide orientation, cast, Frobenius partial sums), the norm finalize, and
// the parameter update apply (+ transpose back).
//
// Paper: arXiv:2609.21594 section 6.2 (a step updates the momentum, runs
// the batched NS iteration and applies the update locally), section 6.4
// step 4 (the update and weight decay are applied by fused elementwise
// kernels), section 6.6 (transpose first when rows exceed columns),
// section 7.4 (FP32 optimizer state).
//
// Every pass works on 64x64 tiles of the wide (m <= n) orientation. A
// 256-thread block covers one tile: 16 threads per row, 4 consecutive
// elements per thread, 4 row passes. Tall matrices go through an LDS tile
// so that both the original-orientation access and the wide-orientation
// access are coalesced. Partial sums are per tile, in a fixed order, so
// the norm does not depend on how matrices are batched.
#include "device_common.h"
#include "kernels.h"
#include "plan.h"

namespace muon {

namespace {

constexpr int T = kEwTile;  // 64

// Workgroups of the momentum and apply passes resident on the chip at once:
// 256 compute units x 8 (four waves each, one per SIMD, within the LDS and
// register budget). A tall matrix with more tiles than this takes its tiles
// along the stored rows (see tile_coords).
constexpr int kEwResident = 256 * 8;

// Wide tile (ti, tj) of workgroup index b. Wide matrices (and tall ones that
// fit in the resident window) run the wide tile rows in order. A tall
// matrix larger than the window runs the wide tile columns in order, so
// consecutive workgroups read consecutive bands of the stored rows: in the
// row-major wide order the resident workgroups would read 64-column strips
// from every stored row at once, which measured 27% slower on MI355X for
// 14336x4096 and 3% slower for 7168x2048; for 2048x1408 (704 tiles, all
// resident either way) the wide order measured 3.5% faster.
__device__ __forceinline__ void tile_coords(int b, int tiles_m, int tiles_n, bool tall, int& ti, int& tj) {
  if (tall && tiles_m * tiles_n > kEwResident) { tj = b / tiles_m; ti = b % tiles_m; }
  else { ti = b / tiles_n; tj = b % tiles_n; }
}

// The matrix table travels in the kernel argument block; keep it (with the
// largest per-launch arguments) within 4 KiB.
static_assert(sizeof(EwMats) + sizeof(MomentumArgs) <= 4096, "elementwise kernel arguments exceed 4 KiB");

template <typename ST>
__device__ __forceinline__ void load4(const ST* p, int valid, float v[4]) {
  // valid: number of in-range elements starting at p (0..4)
  if (valid == 4 && (reinterpret_cast<uintptr_t>(p) % (4 * sizeof(ST)) == 0)) {
    if constexpr (sizeof(ST) == 4) {
      float4 q = *reinterpret_cast<const float4*>(p);
      v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
    } else {
      uint2 q = *reinterpret_cast<const uint2*>(p);
      v[0] = bf16_to_f32(q.x & 0xffffu); v[1] = bf16_to_f32(q.x >> 16);
      v[2] = bf16_to_f32(q.y & 0xffffu); v[3] = bf16_to_f32(q.y >> 16);
    }
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = e < valid ? Elem<ST>::load(p + e) : 0.0f;
  }
}

// 4 whole elements at a 4-element-aligned address (interior tiles).
// Non-temporal: every
// byte of these passes is touched once (the workspace of a batch is far
// larger than the L2), and streaming hints measured 4% faster for the
// momentum pass.
typedef float nt_f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned nt_u32x2 __attribute__((ext_vector_type(2)));
template <typename ST>
__device__ __forceinline__ void load4a(const ST* p, float v[4]) {
  if constexpr (sizeof(ST) == 4) {
    const nt_f32x4 q = __builtin_nontemporal_load(reinterpret_cast<const nt_f32x4*>(p));
    v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
  } else {
    const nt_u32x2 q = __builtin_nontemporal_load(reinterpret_cast<const nt_u32x2*>(p));
    v[0] = bf16_to_f32(q.x & 0xffffu); v[1] = bf16_to_f32(q.x >> 16);
    v[2] = bf16_to_f32(q.y & 0xffffu); v[3] = bf16_to_f32(q.y >> 16);
  }
}
template <typename ST>
__device__ __forceinline__ void store4a(ST* p, const float v[4]) {
  if constexpr (sizeof(ST) == 4) {
    __builtin_nontemporal_store(nt_f32x4{v[0], v[1], v[2], v[3]}, reinterpret_cast<nt_f32x4*>(p));
  } else {
    nt_u32x2 q;
    q.x = f32x2_to_bf16x2(v[0], v[1]);
    q.y = f32x2_to_bf16x2(v[2], v[3]);
    __builtin_nontemporal_store(q, reinterpret_cast<nt_u32x2*>(p));
  }
}

template <typename ST>
__device__ __forceinline__ void store4(ST* p, int valid, const float v[4]) {
  if (valid == 4 && (reinterpret_cast<uintptr_t>(p) % (4 * sizeof(ST)) == 0)) {
    if constexpr (sizeof(ST) == 4) {
      *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
    } else {
      uint2 q;
      q.x = f32x2_to_bf16x2(v[0], v[1]);
      q.y = f32x2_to_bf16x2(v[2], v[3]);
      *reinterpret_cast<uint2*>(p) = q;
    }
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (e < valid) Elem<ST>::store(p + e, v[e]);
  }
}

__device__ __forceinline__ int clamp4(int v) { return v < 0 ? 0 : (v > 4 ? 4 : v); }

// One momentum element: returns the NS input u and updates *b.
__device__ __forceinline__ float momentum_elem(float g, float& b, const MomentumArgs& a) {
  if (!a.has_buf) return g;
  const float nb = fmaf(a.beta, b, a.kg * g);
  b = nb;
  return a.nesterov ? fmaf(a.beta, nb, a.kg * g) : nb;
}

template <typename GT, typename XT>
__global__ __launch_bounds__(256) void momentum_kernel(EwMats mats, MomentumArgs a) {
  __shared__ float tile[T][T + 1];
  __shared__ float red[4];
  const int mi = blockIdx.y;
  const int tiles_n = a.n_pad / T;
  // The tile's partial keeps its wide row-major index in either tile order.
  int ti, tj;
  tile_coords(blockIdx.x, a.m_pad / T, tiles_n, mats.tr[mi], ti, tj);
  const int tile_id = ti * tiles_n + tj;
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  const GT* g = static_cast<const GT*>(mats.src[mi]);
  float* buf = mats.buf[mi];
  XT* x0 = static_cast<XT*>(a.x0) + (size_t)(a.first + mi) * a.mat_x;
  float ss = 0.0f;
  int nz = 0;   // any u of the tile not exactly 0 (NaN != 0 counts)
  const size_t ld = (size_t)mats.ld[mi];   // row stride of g and buf as stored
  if (a.ptab && blockIdx.x == 0 && threadIdx.x == 0)
    a.ptab[a.first + mi] = ApplyEntry{mats.dst[mi], mats.tr[mi], mats.ld[mi]};

  // Interior tiles (all 64 x 64 elements in range, row stride a multiple
  // of 4, so every 4-element access is whole and aligned) issue all their
  // loads before any arithmetic or store: four passes of loads in flight
  // per thread instead of one. Edge tiles take the general path below.
  const bool interior = (ld % 4 == 0) && (ti + 1) * T <= a.m && (tj + 1) * T <= a.n;
  if (interior && !mats.tr[mi]) {
    float gv[4][4], bv[4][4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const size_t off = (size_t)(ti * T + ty + 16 * p) * ld + tj * T + tx * 4;
      load4a<GT>(g + off, gv[p]);
      if (a.has_buf) load4a<float>(buf + off, bv[p]);
    }
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int i = ti * T + ty + 16 * p;
      const size_t off = (size_t)i * ld + tj * T + tx * 4;
      float u[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        u[e] = momentum_elem(gv[p][e], bv[p][e], a);
        ss = fmaf(u[e], u[e], ss);
        nz |= u[e] != 0.0f;
      }
      if (a.has_buf) store4a<float>(buf + off, bv[p]);
      store4a<XT>(x0 + (size_t)i * a.n_pad + tj * T + tx * 4, u);
    }
  } else if (interior) {
    float gv[4][4], bv[4][4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const size_t off = (size_t)(tj * T + ty + 16 * p) * ld + ti * T + tx * 4;
      load4a<GT>(g + off, gv[p]);
      if (a.has_buf) load4a<float>(buf + off, bv[p]);
    }
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const size_t off = (size_t)(tj * T + ty + 16 * p) * ld + ti * T + tx * 4;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float u = momentum_elem(gv[p][e], bv[p][e], a);
        ss = fmaf(u, u, ss);
        nz |= u != 0.0f;
        tile[ty + 16 * p][tx * 4 + e] = u;
      }
      if (a.has_buf) store4a<float>(buf + off, bv[p]);
    }
    __syncthreads();
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int il = ty + 16 * p, jl = tx * 4;
      float v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = tile[jl + e][il];
      store4a<XT>(x0 + (size_t)(ti * T + il) * a.n_pad + tj * T + jl, v);
    }
  } else if (!mats.tr[mi]) {
    // Stored wide: element (i, j) of the m x n matrix is X0[i][j].
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int i = ti * T + ty + 16 * p;
      const int j = tj * T + tx * 4;
      float u[4] = {0.f, 0.f, 0.f, 0.f};
      if (i < a.m) {
        const int valid = clamp4(a.n - j);
        float gv[4], bv[4] = {0.f, 0.f, 0.f, 0.f};
        load4<GT>(g + (size_t)i * ld + j, valid, gv);
        if (a.has_buf) load4<float>(buf + (size_t)i * ld + j, valid, bv);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (e < valid) {
            u[e] = momentum_elem(gv[e], bv[e], a);
            ss = fmaf(u[e], u[e], ss);
            nz |= u[e] != 0.0f;
          }
        }
        if (a.has_buf) store4<float>(buf + (size_t)i * ld + j, valid, bv);
      }
      store4<XT>(x0 + (size_t)i * a.n_pad + j, 4, u);
    }
  } else {
    // Stored tall: the original is n x m (rows = wide n, cols = wide m) and
    // X0[i][j] = u[j][i]. Read a 64x64 original tile coalesced and write X0
    // through the LDS tile.
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int r = tj * T + ty + 16 * p;   // original row  = wide column
      const int c = ti * T + tx * 4;        // original col  = wide row
      float u[4] = {0.f, 0.f, 0.f, 0.f};
      if (r < a.n) {
        const int valid = clamp4(a.m - c);
        float gv[4], bv[4] = {0.f, 0.f, 0.f, 0.f};
        load4<GT>(g + (size_t)r * ld + c, valid, gv);
        if (a.has_buf) load4<float>(buf + (size_t)r * ld + c, valid, bv);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (e < valid) {
            u[e] = momentum_elem(gv[e], bv[e], a);
            ss = fmaf(u[e], u[e], ss);
            nz |= u[e] != 0.0f;
          }
        }
        if (a.has_buf) store4<float>(buf + (size_t)r * ld + c, valid, bv);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) tile[ty + 16 * p][tx * 4 + e] = u[e];
    }
    __syncthreads();
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int il = ty + 16 * p, jl = tx * 4;
      float v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = tile[jl + e][il];
      store4<XT>(x0 + (size_t)(ti * T + il) * a.n_pad + tj * T + jl, 4, v);
    }
  }
  const float tot = block_sum_256(ss, red);
  const int any = __syncthreads_or(nz);
  if (threadIdx.x == 0) {
    a.partials[(size_t)(a.first + mi) * a.ew_blocks + tile_id] = tot;
    a.nonzero[(size_t)(a.first + mi) * a.ew_blocks + tile_id] = any ? 1 : 0;
  }
}

__global__ __launch_bounds__(256) void finalize_kernel(FinalizeArgs a) {
  __shared__ float red[4];
  const int mi = blockIdx.x;
  const float* p = a.partials + (size_t)mi * a.ew_blocks;
  float s = 0.0f;
  int nz = 0;
  for (int k = threadIdx.x; k < a.ew_blocks; k += 256) {
    s += p[k];
    nz |= a.nonzero[(size_t)mi * a.ew_blocks + k];
  }
  const float tot = block_sum_256(s, red);
  const int any = __syncthreads_or(nz);
  if (threadIdx.x == 0) {
    a.scales[mi] = 1.0f / (sqrtf(tot) + a.eps);
    a.live[mi] = any ? 1 : 0;
  }
}

template <typename PT, typename XT>
__global__ __launch_bounds__(256) void apply_kernel(EwMats mats, ApplyArgs a) {
  __shared__ float tile[T][T + 1];
  const int mi = blockIdx.y;
  const int tr = mats.tr[mi];
  int ti, tj;
  tile_coords(blockIdx.x, (a.m + T - 1) / T, a.n_pad / T, tr, ti, tj);
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  const XT* x = static_cast<const XT*>(a.x) + (size_t)(a.first + mi) * a.mat_x;
  const float os = a.use_scale ? a.scales[a.first + mi] : 1.0f;
  const float gamma = a.gamma[tr];
  // A matrix whose NS input was exactly zero has O = 0 exactly (its iterate
  // was not stored); with dead_only, live matrices are someone else's.
  const bool zo = a.live != nullptr && a.live[a.first + mi] == 0;
  if (a.dead_only && !zo) return;
  PT* dst = static_cast<PT*>(mats.dst[mi]);
  const PT* src = static_cast<const PT*>(mats.src[mi]);
  const size_t ld = (size_t)mats.ld[mi];   // row stride of src and dst as stored

  // Interior tiles: all loads first (see momentum_kernel).
  const bool interior = (ld % 4 == 0) && (ti + 1) * T <= a.m && (tj + 1) * T <= a.n;
  if (interior && !tr) {
    float o[4][4], pv[4][4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int i = ti * T + ty + 16 * p, j = tj * T + tx * 4;
      load4a<XT>(x + (size_t)i * a.n_pad + j, o[p]);
      if (zo) o[p][0] = o[p][1] = o[p][2] = o[p][3] = 0.0f;
      if (a.mode == 0) load4a<PT>(src + (size_t)i * ld + j, pv[p]);
    }
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int i = ti * T + ty + 16 * p, j = tj * T + tx * 4;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float oe = o[p][e] * os;
        pv[p][e] = a.mode == 0 ? fmaf(-gamma, oe, a.alpha * pv[p][e]) : oe;
      }
      store4a<PT>(dst + (size_t)i * ld + j, pv[p]);
    }
    return;
  }
  if (interior) {
    float o[4][4], pv[4][4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      load4a<XT>(x + (size_t)(ti * T + ty + 16 * p) * a.n_pad + tj * T + tx * 4, o[p]);
      if (zo) o[p][0] = o[p][1] = o[p][2] = o[p][3] = 0.0f;
      if (a.mode == 0) load4a<PT>(src + (size_t)(tj * T + ty + 16 * p) * ld + ti * T + tx * 4, pv[p]);
    }
#pragma unroll
    for (int p = 0; p < 4; ++p)
#pragma unroll
      for (int e = 0; e < 4; ++e) tile[ty + 16 * p][tx * 4 + e] = o[p][e];
    __syncthreads();
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int r = tj * T + ty + 16 * p, c = ti * T + tx * 4;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float oe = tile[tx * 4 + e][ty + 16 * p] * os;
        pv[p][e] = a.mode == 0 ? fmaf(-gamma, oe, a.alpha * pv[p][e]) : oe;
      }
      store4a<PT>(dst + (size_t)r * ld + c, pv[p]);
    }
    return;
  }

  if (!tr) {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int i = ti * T + ty + 16 * p;
      const int j = tj * T + tx * 4;
      if (i >= a.m) continue;
      const int valid = clamp4(a.n - j);
      if (valid == 0) continue;
      float o[4], pv[4] = {0.f, 0.f, 0.f, 0.f};
      load4<XT>(x + (size_t)i * a.n_pad + j, 4, o);
      if (zo) o[0] = o[1] = o[2] = o[3] = 0.0f;
      if (a.mode == 0) load4<PT>(src + (size_t)i * ld + j, valid, pv);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float oe = o[e] * os;
        pv[e] = a.mode == 0 ? fmaf(-gamma, oe, a.alpha * pv[e]) : oe;
      }
      store4<PT>(dst + (size_t)i * ld + j, valid, pv);
    }
  } else {
    // Original is n x m; element (r, c) takes O[c][r].
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int il = ty + 16 * p;
      float o[4];
      load4<XT>(x + (size_t)(ti * T + il) * a.n_pad + tj * T + tx * 4, 4, o);
      if (zo) o[0] = o[1] = o[2] = o[3] = 0.0f;
#pragma unroll
      for (int e = 0; e < 4; ++e) tile[il][tx * 4 + e] = o[e];
    }
    __syncthreads();
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int r = tj * T + ty + 16 * p;  // original row
      const int c = ti * T + tx * 4;       // original col
      if (r >= a.n) continue;
      const int valid = clamp4(a.m - c);
      if (valid == 0) continue;
      float pv[4] = {0.f, 0.f, 0.f, 0.f};
      if (a.mode == 0) load4<PT>(src + (size_t)r * ld + c, valid, pv);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float oe = tile[tx * 4 + e][ty + 16 * p] * os;
        pv[e] = a.mode == 0 ? fmaf(-gamma, oe, a.alpha * pv[e]) : oe;
      }
      store4<PT>(dst + (size_t)r * ld + c, valid, pv);
    }
  }
}

// One workgroup: the live flags of a batch -> the ascending list of live
// matrices and its length (a block-wide scan of per-thread counts).
__global__ __launch_bounds__(256) void compact_kernel(const int* live, int count, int* list, int* nlive,
                                                     int* sched) {
  __shared__ int sums[256];
  const int t = threadIdx.x;
  if (sched && t < 16) sched[t] = 0;
  const int per = (count + 255) / 256;
  const int lo = t * per, hi = min(count, lo + per);
  int c = 0;
  for (int i = lo; i < hi; ++i) c += live[i] != 0;
  sums[t] = c;
  __syncthreads();
  for (int off = 1; off < 256; off <<= 1) {
    const int v = t >= off ? sums[t - off] : 0;
    __syncthreads();
    sums[t] += v;
    __syncthreads();
  }
  int pos = sums[t] - c;
  for (int i = lo; i < hi; ++i)
    if (live[i] != 0) list[pos++] = i;
  if (t == 255) *nlive = sums[255];
}

}  // namespace

hipError_t launch_compact(const int* live, int count, int* live_list, int* nlive, int* sched, hipStream_t s) {
  if (count <= 0) return hipSuccess;
  hipLaunchKernelGGL(compact_kernel, dim3(1), dim3(256), 0, s, live, count, live_list, nlive, sched);
  return hipGetLastError();
}

hipError_t launch_momentum(const EwMats& mats, const MomentumArgs& a, int src_bf16, int ws_bf16,
                           hipStream_t s) {
  if (a.count <= 0) return hipSuccess;
  // The kernel reads its matrices from the table's kEwChunk slots and maps
  // workgroups onto the padded shape's 64 x 64 tiles.
  if (a.count > kEwChunk || a.m_pad % T || a.n_pad % T || a.m > a.m_pad || a.n > a.n_pad ||
      a.ew_blocks != (a.m_pad / T) * (a.n_pad / T))
    return hipErrorInvalidValue;
  dim3 grid(a.ew_blocks, a.count), block(256);
  if (src_bf16 && ws_bf16) hipLaunchKernelGGL((momentum_kernel<bf16_t, bf16_t>), grid, block, 0, s, mats, a);
  else if (!src_bf16 && ws_bf16) hipLaunchKernelGGL((momentum_kernel<float, bf16_t>), grid, block, 0, s, mats, a);
  else if (src_bf16 && !ws_bf16) hipLaunchKernelGGL((momentum_kernel<bf16_t, float>), grid, block, 0, s, mats, a);
  else hipLaunchKernelGGL((momentum_kernel<float, float>), grid, block, 0, s, mats, a);
  return hipGetLastError();
}

hipError_t launch_finalize(const FinalizeArgs& a, hipStream_t s) {
  if (a.count <= 0) return hipSuccess;
  hipLaunchKernelGGL(finalize_kernel, dim3(a.count), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_apply(const EwMats& mats, const ApplyArgs& a, int p_bf16, int ws_bf16,
                        hipStream_t s) {
  if (a.count <= 0) return hipSuccess;
  if (a.count > kEwChunk || a.n_pad % T || a.n > a.n_pad) return hipErrorInvalidValue;
  const int m_pad = (a.m + T - 1) / T * T;
  dim3 grid((m_pad / T) * (a.n_pad / T), a.count), block(256);
  if (p_bf16 && ws_bf16) hipLaunchKernelGGL((apply_kernel<bf16_t, bf16_t>), grid, block, 0, s, mats, a);
  else if (!p_bf16 && ws_bf16) hipLaunchKernelGGL((apply_kernel<float, bf16_t>), grid, block, 0, s, mats, a);
  else if (p_bf16 && !ws_bf16) hipLaunchKernelGGL((apply_kernel<bf16_t, float>), grid, block, 0, s, mats, a);
  else hipLaunchKernelGGL((apply_kernel<float, float>), grid, block, 0, s, mats, a);
  return hipGetLastError();
}

}  // namespace muon
