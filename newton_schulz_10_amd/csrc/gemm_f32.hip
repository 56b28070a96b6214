// Batched fp32 GEMMs of the quintic Newton-Schulz iteration (float32 path).
//
// Same three roles and epilogues as the bf16 path (see gemm_bf16.hip), in
// the direct form:
//   Gram   : A  = sc * X X^T        (upper tiles, mirrored)
//   Poly   : B  = b*A + c*(A A)     (A symmetric; upper tiles, mirrored)
//   Update : X' = sc * (a*X + B X)
// on the fp32 matrix cores (v_mfma_f32_32x32x2_f32): 64 x 64 output tiles,
// 256 threads = 4 waves of 32 x 32 (one MFMA block of 16 fp32 accumulators
// per lane). K-slabs of 16 staged K-major in LDS ([k][row]: a fragment
// read is 32 consecutive floats per half-wave), double buffered: the next
// slab's global loads are in flight while the current one is multiplied,
// one barrier per slab. Small tiles and registers keep several workgroups
// on a CU, which hide the load latency.
#include "device_common.h"
#include "kernels.h"

namespace muon {

namespace {

constexpr int TM = 64, TK = 16, TP = TM + 4;   // tile edge, K-slab, padded LDS row
typedef __attribute__((ext_vector_type(16))) float f32x16;

__device__ __forceinline__ void upper_tile(int t, int nt, int& I, int& J) {
  int i = 0, rowlen = nt;
  while (t >= rowlen) { t -= rowlen; ++i; --rowlen; }
  I = i; J = i + t;
}

template <int ROLE>
__global__ __launch_bounds__(256) void ns_gemm_f32(GemmArgs g) {
  __shared__ __attribute__((aligned(16))) float As[2][TK][TP];
  __shared__ __attribute__((aligned(16))) float Bs[2][TK][TP];   // rows of 272 B: float4 stores stay aligned
  constexpr bool kSym = (ROLE != kUpdate);
  const int tiles_m = g.m_pad / TM;
  const int tiles_n = kSym ? tiles_m : g.n_pad / TM;
  const int per_mat = kSym ? tiles_m * (tiles_m + 1) / 2 : tiles_m * tiles_n;
  const int total = per_mat * g.count;
  const int logical = xcd_remap(blockIdx.x, total);
  const int mat = logical / per_mat;
  int I, J;
  if (kSym) upper_tile(logical % per_mat, tiles_m, I, J);
  else { I = (logical % per_mat) / tiles_n; J = (logical % per_mat) % tiles_n; }

  const int K = (ROLE == kGram) ? g.n_pad : g.m_pad;
  const float* Aop;
  const float* Bop;
  int lda, ldb;
  if (ROLE == kGram) {
    Aop = static_cast<const float*>(g.x) + (size_t)mat * g.mat_x; lda = g.n_pad; Bop = Aop; ldb = lda;
  } else if (ROLE == kPoly) {
    Aop = static_cast<const float*>(g.a) + (size_t)mat * g.mat_a; lda = g.m_pad; Bop = Aop; ldb = lda;
  } else {
    Aop = static_cast<const float*>(g.b) + (size_t)mat * g.mat_a; lda = g.m_pad;
    Bop = static_cast<const float*>(g.x) + (size_t)mat * g.mat_x; ldb = g.n_pad;
  }
  Aop += (size_t)(I * TM) * lda;
  if (ROLE == kUpdate) Bop += (size_t)J * TM;
  else Bop += (size_t)(J * TM) * ldb;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r0 = (wave >> 1) * 32, c0 = (wave & 1) * 32;   // the wave's 32 x 32 block
  // Slab loads (one float4 of A and one of B per thread): A rows (and the
  // rows of Q for Gram/Poly) as 16 k of a row; Update's B as 64 columns of
  // one of 16 k rows of X.
  const int lrow = tid >> 2, lkq = (tid & 3) * 4;
  const int bkr = tid >> 4, bjq = (tid & 15) * 4;
  float4 ra, rb;
  auto load = [&](int k0) {
    ra = *reinterpret_cast<const float4*>(Aop + (size_t)lrow * lda + k0 + lkq);
    if (ROLE == kUpdate) rb = *reinterpret_cast<const float4*>(Bop + (size_t)(k0 + bkr) * ldb + bjq);
    else rb = *reinterpret_cast<const float4*>(Bop + (size_t)lrow * ldb + k0 + lkq);
  };
  auto stash = [&](int buf) {
    As[buf][lkq + 0][lrow] = ra.x; As[buf][lkq + 1][lrow] = ra.y;
    As[buf][lkq + 2][lrow] = ra.z; As[buf][lkq + 3][lrow] = ra.w;
    if (ROLE == kUpdate) {
      *reinterpret_cast<float4*>(&Bs[buf][bkr][bjq]) = rb;
    } else {
      Bs[buf][lkq + 0][lrow] = rb.x; Bs[buf][lkq + 1][lrow] = rb.y;
      Bs[buf][lkq + 2][lrow] = rb.z; Bs[buf][lkq + 3][lrow] = rb.w;
    }
  };

  // MFMA operands: lane l supplies A[r0 + l%32][k + l/32] and
  // B[k + l/32][c0 + l%32]; accumulator element v of lane l is output
  // (r0 + 8*(v/4) + 4*(l/32) + v%4, c0 + l%32).
  f32x16 acc = {};
  const int nk = K / TK;
  load(0);
  stash(0);
  __syncthreads();
  for (int s = 0; s < nk; ++s) {
    const int buf = s & 1;
    if (s + 1 < nk) load((s + 1) * TK);
#pragma unroll
    for (int kk = 0; kk < TK; kk += 2) {
      const float av = As[buf][kk + (lane >> 5)][r0 + (lane & 31)];
      const float bv = Bs[buf][kk + (lane >> 5)][c0 + (lane & 31)];
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(av, bv, acc, 0, 0, 0);
    }
    if (s + 1 < nk) stash(buf ^ 1);
    __syncthreads();
  }

  float sc = 1.0f;
  if (g.scales) {
    const float sv = g.scales[mat];
    sc = (ROLE == kGram) ? sv * sv : sv;
  }
  float* out = static_cast<float*>(g.out);
  const int ldc = (ROLE == kUpdate) ? g.n_pad : g.m_pad;
  out += (size_t)mat * ((ROLE == kUpdate) ? g.mat_x : g.mat_a);
  const float* ep = nullptr;
  if (ROLE == kPoly) ep = static_cast<const float*>(g.a) + (size_t)mat * g.mat_a;
  if (ROLE == kUpdate) ep = static_cast<const float*>(g.x) + (size_t)mat * g.mat_x;
  const int gj = J * TM + c0 + (lane & 31);
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int gi = I * TM + r0 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
    const float a = acc[v];
    float val;
    if (ROLE == kGram) val = sc * a;
    else if (ROLE == kPoly) val = fmaf(g.cb, ep[(size_t)gi * ldc + gj], g.cc * a);
    else val = sc * fmaf(g.ca, ep[(size_t)gi * ldc + gj], a);
    if (kSym) {
      if (gi <= gj) { out[(size_t)gi * ldc + gj] = val; out[(size_t)gj * ldc + gi] = val; }
    } else {
      out[(size_t)gi * ldc + gj] = val;
    }
  }
}

}  // namespace

hipError_t launch_gemm_f32(GemmRole role, const GemmArgs& g, hipStream_t s) {
  if (g.count <= 0) return hipSuccess;
  if (g.m_pad % TM || g.n_pad % TM) return hipErrorInvalidValue;
  const int tm = g.m_pad / TM, tn = g.n_pad / TM;
  const long long per = (role == kUpdate) ? (long long)tm * tn : (long long)tm * (tm + 1) / 2;
  const long long total = per * g.count;
  if (total <= 0 || total > 0x7fffffffLL) return hipErrorInvalidValue;
  dim3 grid((unsigned)total), block(256);
  switch (role) {
    case kGram: hipLaunchKernelGGL(ns_gemm_f32<kGram>, grid, block, 0, s, g); break;
    case kPoly: hipLaunchKernelGGL(ns_gemm_f32<kPoly>, grid, block, 0, s, g); break;
    case kUpdate: hipLaunchKernelGGL(ns_gemm_f32<kUpdate>, grid, block, 0, s, g); break;
  }
  return hipGetLastError();
}

}  // namespace muon
