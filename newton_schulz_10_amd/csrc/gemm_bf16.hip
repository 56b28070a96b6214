// Batched bf16 GEMMs of the quintic Newton-Schulz iteration on CDNA4 MFMA.
//
// Paper: arXiv:2609.21594 section 6.6 -- same-shaped matrices are
// concatenated along a batch axis and orthogonalized by one batched NS
// iteration, a single sequence of batched matmuls, in bf16 arithmetic.
// Per NS step and matrix (X is m x n, m <= n, padded with zeros):
//   Gram   : A  = sc * X X^T        symmetric: upper tiles only, mirrored
//   Poly   : B  = b*A + c*(A A)     A symmetric, so A A = A A^T; B symmetric
//   Update : X' = sc * (a*X + B X)
// sc is the first step's Frobenius scale (s^2 for Gram, s for Update) and 1
// afterwards. Accumulation is fp32 on v_mfma_f32_32x32x16_bf16; every
// epilogue is formed in fp32 and rounded once to bf16.
//
// Design (gfx950):
//  * Block: 256 threads = 4 waves (2 x 2); output tile 256 x 256; each wave
//    owns 128 x 128 = 4 x 4 MFMA 32x32 blocks (256 fp32 accumulators/lane).
//  * K-slabs of 64 staged in LDS by direct global->LDS loads
//    (global_load_lds_dwordx4, 16 B per lane), two stages of 64 KiB.
//  * Operands whose K is contiguous in memory (rows of X for Gram, rows of A
//    for Poly, rows of B for Update) are stored [row][64 k], 128 B rows,
//    with the 16 B chunk index XOR-swizzled by (row & 7): the MFMA fragment
//    reads (ds_read_b128, 32 rows per half-wave) are bank-conflict free.
//  * Update's X operand is N-contiguous; it is stored [k][256 n] as loaded
//    and read with ds_read_b64_tr_b16, which hands each lane 4 consecutive
//    k of one column, i.e. the MFMA operand layout, so no transpose pass or
//    transposed copy of X is needed. Its chunk swizzle keeps those reads
//    conflict free.
//  * The column operand goes in the MFMA's first slot, so each lane ends
//    with 4 consecutive output columns of one row: epilogue loads and
//    stores are 8-byte row chunks; the symmetric mirror stores are
//    coalesced across lanes.
//  * One grid covers every tile of every matrix of the batch; block ids are
//    remapped so each XCD works on whole matrices (L2 reuse).
#include "device_common.h"
#include "kernels.h"

namespace muon {

namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;

constexpr int TILE = 256;            // output tile edge
constexpr int BK = 64;               // K per LDS stage
constexpr int kThreads = 256;
constexpr int kStageElems = TILE * BK;   // elements per operand per stage (16 Ki)

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

__device__ __forceinline__ void upper_tile(int t, int nt, int& I, int& J) {
  int i = 0, rowlen = nt;
  while (t >= rowlen) { t -= rowlen; ++i; --rowlen; }
  I = i; J = i + t;
}

// Swizzle of Update's [k][n] X stage: 16 B chunk index XOR f(k). Rows
// k..k+3 (k % 4 == 0) land in distinct bank groups for the transpose reads.
__device__ __forceinline__ int xswz(int k) { return 4 * (k & 3) + 2 * ((k >> 1) & 1); }

// Direct global->LDS load of 16 B per lane: lane l's bytes land at
// lds_dst + 16*l. Issued as inline asm so that the compiler does not
// track it: its conservative LDS-DMA alias tracking would otherwise wait
// for the prefetch of the next slab before any LDS read. Completion is
// awaited with explicit vmcnt waits. `lds_dst` must be wave-uniform.
__device__ __forceinline__ void dma16(const void* g, const bf16_t* lds_dst) {
  const unsigned a = static_cast<unsigned>(reinterpret_cast<uintptr_t>(
      (const __attribute__((address_space(3))) char*)(lds_dst)));
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off"
               :: "s"(__builtin_amdgcn_readfirstlane(a)), "v"(g) : "memory", "m0");
}

// Workgroup barrier without the release/acquire fence of __syncthreads():
// the fence would wait for every outstanding global->LDS load, including
// the next slab's prefetch. LDS readiness is established by the explicit
// waits placed before each call; the memory clobber keeps the compiler
// from moving LDS accesses across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_barrier" ::: "memory"); }

template <int ROLE>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void ns_gemm_bf16(GemmArgs g) {
  // [stage][operand 0 = row operand, 1 = column operand][TILE * BK]
  __shared__ __attribute__((aligned(1024))) bf16_t lds[2][2][kStageElems];

  constexpr bool kSym = (ROLE != kUpdate);
  const int tiles_m = g.m_pad / TILE;
  const int tiles_n = kSym ? tiles_m : g.n_pad / TILE;
  const int per_mat = kSym ? tiles_m * (tiles_m + 1) / 2 : tiles_m * tiles_n;
  const int total = per_mat * g.count;
  const int logical = xcd_remap(blockIdx.x, total);
  const int mat = logical / per_mat;
  int I, J;
  if (kSym) upper_tile(logical % per_mat, tiles_m, I, J);
  else { I = (logical % per_mat) / tiles_n; J = (logical % per_mat) % tiles_n; }

  const int K = (ROLE == kGram) ? g.n_pad : g.m_pad;
  const bf16_t* rowop;   // output rows i: K contiguous
  const bf16_t* colop;   // output cols j: K contiguous (Gram/Poly) or X[k][j] (Update)
  int ldr, ldc_op;
  if (ROLE == kGram) {
    rowop = static_cast<const bf16_t*>(g.x) + (size_t)mat * g.mat_x; ldr = g.n_pad;
    colop = rowop; ldc_op = g.n_pad;
  } else if (ROLE == kPoly) {
    rowop = static_cast<const bf16_t*>(g.a) + (size_t)mat * g.mat_a; ldr = g.m_pad;
    colop = rowop; ldc_op = g.m_pad;
  } else {
    rowop = static_cast<const bf16_t*>(g.b) + (size_t)mat * g.mat_a; ldr = g.m_pad;
    colop = static_cast<const bf16_t*>(g.x) + (size_t)mat * g.mat_x; ldc_op = g.n_pad;
  }
  rowop += (size_t)(I * TILE) * ldr;
  if (ROLE == kUpdate) colop += (size_t)J * TILE;
  else colop += (size_t)(J * TILE) * ldc_op;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;   // wave's 128-row / 128-col block

  // Issue one K-slab into `stage`: each wave moves 64 rows of the row
  // operand and its share of the column operand (8 + 8 loads of 1 KiB).
  auto issue = [&](int kt, int stage) {
    const int k0 = kt * BK;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const int rb = wave * 64 + q * 8;
      const int r = rb + (lane >> 3);
      const int ch = (lane & 7) ^ (r & 7);
      dma16(rowop + (size_t)r * ldr + k0 + ch * 8, &lds[stage][0][rb * BK]);
    }
    if (ROLE == kUpdate) {
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int kb = wave * 16 + q * 2;
        const int k = kb + (lane >> 5);
        const int ch = (lane & 31) ^ xswz(k);
        dma16(colop + (size_t)(k0 + k) * ldc_op + ch * 8, &lds[stage][1][kb * TILE]);
      }
    } else {
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int rb = wave * 64 + q * 8;
        const int r = rb + (lane >> 3);
        const int ch = (lane & 7) ^ (r & 7);
        dma16(colop + (size_t)r * ldc_op + k0 + ch * 8, &lds[stage][1][rb * BK]);
      }
    }
  };

  f32x16 acc[4][4];  // [column block][row block]
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[a][b][v] = 0.0f;

  const int nk = K / BK;
  issue(0, 0);
  if (nk > 1) issue(1, 1);
  for (int kt = 0; kt < nk; ++kt) {
    const int stage = kt & 1;
    // Wait until this wave's loads of slab kt have landed (the 16 loads of
    // slab kt+1 may stay in flight), then until every wave's have.
    if (kt + 1 < nk) __builtin_amdgcn_s_waitcnt(0x4F70);  // vmcnt(16)
    else __builtin_amdgcn_s_waitcnt(0x0F70);              // vmcnt(0)
    lds_barrier();
    const bf16_t* As = lds[stage][0];
    const bf16_t* Bs = lds[stage][1];
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      bf16x8 rf[4], cf[4];
      const int ch = 2 * ks + (lane >> 5);
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int r = wm * 128 + b * 32 + (lane & 31);
        rf[b] = *reinterpret_cast<const bf16x8*>(As + r * BK + ((ch ^ (r & 7)) * 8));
      }
      if (ROLE == kUpdate) {
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          // 16-lane group: 4 k rows x 16 columns; two reads give 8 k.
          const int grp = lane >> 4, jj = lane & 15;
          const int n = wn * 128 + a * 32 + 16 * (grp & 1) + 4 * (jj & 3);
          s16x4 h[2];
#pragma unroll
          for (int half = 0; half < 2; ++half) {
            const int k = ks * 16 + 8 * (grp >> 1) + 4 * half + (jj >> 2);
            const int off = k * TILE + (((n >> 3) ^ xswz(k)) << 3) + (n & 7);
            h[half] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(Bs + off));
          }
          cf[a] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(h[0], h[1], 0, 1, 2, 3, 4, 5, 6, 7));
        }
      } else {
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const int r = wn * 128 + a * 32 + (lane & 31);
          cf[a] = *reinterpret_cast<const bf16x8*>(Bs + r * BK + ((ch ^ (r & 7)) * 8));
        }
      }
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cf[a], rf[b], acc[a][b], 0, 0, 0);
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's LDS reads are done
    lds_barrier();                       // ... and every wave's, before `stage` is refilled
    if (kt + 2 < nk) issue(kt + 2, stage);
  }

  // Epilogue. acc[a][b] element v: output row i = row block b, lane % 32;
  // output columns j .. j+3 with j = col block a, 8*(v/4) + 4*(lane/32).
  float sc = 1.0f;
  if (g.scales) {
    const float s = g.scales[mat];
    sc = (ROLE == kGram) ? s * s : s;
  }
  bf16_t* out = static_cast<bf16_t*>(g.out);
  const int ldo = (ROLE == kUpdate) ? g.n_pad : g.m_pad;
  out += (size_t)mat * ((ROLE == kUpdate) ? g.mat_x : g.mat_a);
  const bf16_t* ep = nullptr;
  if (ROLE == kPoly) ep = static_cast<const bf16_t*>(g.a) + (size_t)mat * g.mat_a;
  if (ROLE == kUpdate) ep = static_cast<const bf16_t*>(g.x) + (size_t)mat * g.mat_x;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const int gi = I * TILE + wm * 128 + b * 32 + (lane & 31);
#pragma unroll
    for (int a = 0; a < 4; ++a) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int gj = J * TILE + wn * 128 + a * 32 + 8 * q + 4 * (lane >> 5);
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = acc[a][b][4 * q + e];
        if (ROLE == kPoly || ROLE == kUpdate) {
          const uint2 w = *reinterpret_cast<const uint2*>(ep + (size_t)gi * ldo + gj);
          const float x[4] = {bf16_to_f32(w.x & 0xffffu), bf16_to_f32(w.x >> 16),
                              bf16_to_f32(w.y & 0xffffu), bf16_to_f32(w.y >> 16)};
#pragma unroll
          for (int e = 0; e < 4; ++e)
            v[e] = (ROLE == kPoly) ? fmaf(g.cb, x[e], g.cc * v[e]) : sc * fmaf(g.ca, x[e], v[e]);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] *= sc;
        }
        bf16_t h[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) h[e] = f32_to_bf16(v[e]);
        if (!kSym || I != J) {
          uint2 w;
          w.x = h[0] | (static_cast<unsigned>(h[1]) << 16);
          w.y = h[2] | (static_cast<unsigned>(h[3]) << 16);
          *reinterpret_cast<uint2*>(out + (size_t)gi * ldo + gj) = w;
          if (kSym) {
#pragma unroll
            for (int e = 0; e < 4; ++e) out[(size_t)(gj + e) * ldo + gi] = h[e];
          }
        } else {
          // Diagonal tile: keep i <= j, mirror the strict upper part.
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            if (gi <= gj + e) {
              out[(size_t)gi * ldo + gj + e] = h[e];
              out[(size_t)(gj + e) * ldo + gi] = h[e];
            }
          }
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_gemm_bf16(GemmRole role, const GemmArgs& g, hipStream_t s) {
  if (g.count <= 0) return hipSuccess;
  if (g.m_pad % TILE || g.n_pad % TILE) return hipErrorInvalidValue;
  const int tm = g.m_pad / TILE, tn = g.n_pad / TILE;
  const long long per = (role == kUpdate) ? (long long)tm * tn : (long long)tm * (tm + 1) / 2;
  const long long total = per * g.count;
  if (total <= 0 || total > 0x7fffffffLL) return hipErrorInvalidValue;
  dim3 grid((unsigned)total), block(kThreads);
  switch (role) {
    case kGram: hipLaunchKernelGGL(ns_gemm_bf16<kGram>, grid, block, 0, s, g); break;
    case kPoly: hipLaunchKernelGGL(ns_gemm_bf16<kPoly>, grid, block, 0, s, g); break;
    case kUpdate: hipLaunchKernelGGL(ns_gemm_bf16<kUpdate>, grid, block, 0, s, g); break;
  }
  return hipGetLastError();
}

double gemm_flops(GemmRole role, const GemmArgs& g) {
  const double m = g.m, n = g.n;
  const double per = (role == kPoly) ? 2.0 * m * m * m : 2.0 * m * m * n;
  return per * g.count;
}

}  // namespace muon
