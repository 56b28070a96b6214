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
// Block: 256 threads (4 waves as 2x2), output tile 128x128, K-slab 32. Each
// wave owns a 64x64 sub-tile = 2x2 MFMA 32x32 blocks. Operands are staged in
// LDS with K contiguous ([row][k], padded rows), double buffered, the next
// slab prefetched into registers while the current one is multiplied.
// Gram and Poly read both operands along K-contiguous rows; Update's second
// operand X is N-contiguous and is transposed on its way into LDS.
// One grid covers every tile of every matrix of the batch; block ids are
// remapped so each XCD works on whole matrices.
#include "device_common.h"
#include "kernels.h"

namespace muon {

namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;

constexpr int BM = 128, BN = 128, BK = 32;
constexpr int LDK = BK + 8;  // padded LDS row (elements)
constexpr int kThreads = 256;

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

// Upper-triangle tile decode: t -> (I, J), I <= J, row-major over I.
__device__ __forceinline__ void upper_tile(int t, int nt, int& I, int& J) {
  int i = 0, rowlen = nt;
  while (t >= rowlen) { t -= rowlen; ++i; --rowlen; }
  I = i; J = i + t;
}

template <int ROLE>
__global__ __launch_bounds__(kThreads) void ns_gemm_bf16(GemmArgs g) {
  __shared__ __attribute__((aligned(16))) bf16_t As[2][BM * LDK];
  __shared__ __attribute__((aligned(16))) bf16_t Bs[2][BN * LDK];

  constexpr bool kSym = (ROLE != kUpdate);
  const int tiles_m = g.m_pad / BM;
  const int tiles_n = kSym ? tiles_m : g.n_pad / BN;
  const int per_mat = kSym ? tiles_m * (tiles_m + 1) / 2 : tiles_m * tiles_n;
  const int total = per_mat * g.count;
  const int logical = xcd_remap(blockIdx.x, total);
  const int mat = logical / per_mat;
  int I, J;
  if (kSym) upper_tile(logical % per_mat, tiles_m, I, J);
  else { I = (logical % per_mat) / tiles_n; J = (logical % per_mat) % tiles_n; }

  const int K = (ROLE == kGram) ? g.n_pad : g.m_pad;
  const bf16_t* Aop;  // rows i, K contiguous, leading dim lda
  const bf16_t* Bop;  // Gram/Poly: rows j, K contiguous; Update: X[k][j]
  int lda, ldb;
  if (ROLE == kGram) {
    Aop = static_cast<const bf16_t*>(g.x) + (size_t)mat * g.mat_x; lda = g.n_pad;
    Bop = Aop; ldb = g.n_pad;
  } else if (ROLE == kPoly) {
    Aop = static_cast<const bf16_t*>(g.a) + (size_t)mat * g.mat_a; lda = g.m_pad;
    Bop = Aop; ldb = g.m_pad;
  } else {
    Aop = static_cast<const bf16_t*>(g.b) + (size_t)mat * g.mat_a; lda = g.m_pad;
    Bop = static_cast<const bf16_t*>(g.x) + (size_t)mat * g.mat_x; ldb = g.n_pad;
  }
  Aop += (size_t)(I * BM) * lda;
  if (ROLE == kUpdate) Bop += (size_t)J * BN;          // column offset in X
  else Bop += (size_t)(J * BN) * ldb;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // Register staging of one K-slab: 2 x 16B of A and 2 x 16B of B per thread.
  uint4 ra[2], rb[2];
  auto load_slab = [&](int k0) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int c = tid + q * kThreads;
      const int row = c >> 2, kq = (c & 3) * 8;
      ra[q] = *reinterpret_cast<const uint4*>(Aop + (size_t)row * lda + k0 + kq);
      if (ROLE == kUpdate) {
        const int kr = c >> 4, jq = (c & 15) * 8;
        rb[q] = *reinterpret_cast<const uint4*>(Bop + (size_t)(k0 + kr) * ldb + jq);
      } else {
        rb[q] = *reinterpret_cast<const uint4*>(Bop + (size_t)row * ldb + k0 + kq);
      }
    }
  };
  auto store_slab = [&](int buf) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int c = tid + q * kThreads;
      const int row = c >> 2, kq = (c & 3) * 8;
      *reinterpret_cast<uint4*>(&As[buf][row * LDK + kq]) = ra[q];
      if (ROLE == kUpdate) {
        const int kr = c >> 4, jq = (c & 15) * 8;
        const unsigned w[4] = {rb[q].x, rb[q].y, rb[q].z, rb[q].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          Bs[buf][(jq + 2 * e) * LDK + kr] = static_cast<bf16_t>(w[e] & 0xffffu);
          Bs[buf][(jq + 2 * e + 1) * LDK + kr] = static_cast<bf16_t>(w[e] >> 16);
        }
      } else {
        *reinterpret_cast<uint4*>(&Bs[buf][row * LDK + kq]) = rb[q];
      }
    }
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  const int nk = K / BK;
  load_slab(0);
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    store_slab(buf);
    __syncthreads();
    if (kt + 1 < nk) load_slab((kt + 1) * BK);
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      const int kofs = ks * 16 + (lane >> 5) * 8;
      bf16x8 af[2], bfr[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int r = wm * 64 + i * 32 + (lane & 31);
        af[i] = as_bf16x8(*reinterpret_cast<const uint4*>(&As[buf][r * LDK + kofs]));
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int r = wn * 64 + j * 32 + (lane & 31);
        bfr[j] = as_bf16x8(*reinterpret_cast<const uint4*>(&Bs[buf][r * LDK + kofs]));
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
  }

  // Epilogue. Accumulator element v of a 32x32 block sits at row
  // 8*(v/4) + 4*(lane/32) + v%4 and column lane%32.
  float sc = 1.0f;
  if (g.scales) {
    const float s = g.scales[mat];
    sc = (ROLE == kGram) ? s * s : s;
  }
  bf16_t* out = static_cast<bf16_t*>(g.out);
  const int ldc = (ROLE == kUpdate) ? g.n_pad : g.m_pad;
  out += (size_t)mat * ((ROLE == kUpdate) ? g.mat_x : g.mat_a);
  const bf16_t* ep = nullptr;
  if (ROLE == kPoly) ep = static_cast<const bf16_t*>(g.a) + (size_t)mat * g.mat_a;
  if (ROLE == kUpdate) ep = static_cast<const bf16_t*>(g.x) + (size_t)mat * g.mat_x;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int gi = I * BM + wm * 64 + i * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        const int gj = J * BN + wn * 64 + j * 32 + (lane & 31);
        const float a = acc[i][j][v];
        float val;
        if (ROLE == kGram) val = sc * a;
        else if (ROLE == kPoly) val = fmaf(g.cb, bf16_to_f32(ep[(size_t)gi * ldc + gj]), g.cc * a);
        else val = sc * fmaf(g.ca, bf16_to_f32(ep[(size_t)gi * ldc + gj]), a);
        const bf16_t h = f32_to_bf16(val);
        if (kSym) {
          if (gi <= gj) {
            out[(size_t)gi * ldc + gj] = h;
            out[(size_t)gj * ldc + gi] = h;
          }
        } else {
          out[(size_t)gi * ldc + gj] = h;
        }
      }
}

}  // namespace

hipError_t launch_gemm_bf16(GemmRole role, const GemmArgs& g, hipStream_t s) {
  if (g.count <= 0) return hipSuccess;
  if (g.m_pad % BM || g.n_pad % BN) return hipErrorInvalidValue;
  const int tm = g.m_pad / BM, tn = g.n_pad / BN;
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
