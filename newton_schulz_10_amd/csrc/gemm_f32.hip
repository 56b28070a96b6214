// Batched fp32 GEMMs of the quintic Newton-Schulz iteration (float32 path).
//
// Same three roles and epilogues as the bf16 path (see gemm_bf16.hip):
//   Gram   : A  = sc * X X^T        (upper tiles, mirrored)
//   Poly   : B  = b*A + c*(A A)     (A symmetric; upper tiles, mirrored)
//   Update : X' = sc * (a*X + B X)
// computed with fp32 FMA on the vector ALUs: 64x64 output tiles, 256
// threads with 4x4 outputs each, K-slabs of 16 staged in LDS (K-major so
// that the inner product reads are broadcasts / contiguous). The float32
// path serves small groups where bf16 is not wanted; it is not tuned.
#include "device_common.h"
#include "kernels.h"

namespace muon {

namespace {

constexpr int TM = 64, TK = 16;

__device__ __forceinline__ void upper_tile(int t, int nt, int& I, int& J) {
  int i = 0, rowlen = nt;
  while (t >= rowlen) { t -= rowlen; ++i; --rowlen; }
  I = i; J = i + t;
}

template <int ROLE>
__global__ __launch_bounds__(256) void ns_gemm_f32(GemmArgs g) {
  __shared__ float As[TK][TM + 4];
  __shared__ float Bs[TK][TM + 4];
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

  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  float acc[4][4];
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[r][c] = 0.0f;

  for (int k0 = 0; k0 < K; k0 += TK) {
    {
      const int row = tid >> 2, kq = (tid & 3) * 4;
      const float4 va = *reinterpret_cast<const float4*>(Aop + (size_t)row * lda + k0 + kq);
      As[kq + 0][row] = va.x; As[kq + 1][row] = va.y; As[kq + 2][row] = va.z; As[kq + 3][row] = va.w;
      if (ROLE == kUpdate) {
        const int kr = tid >> 4, jq = (tid & 15) * 4;
        const float4 vb = *reinterpret_cast<const float4*>(Bop + (size_t)(k0 + kr) * ldb + jq);
        Bs[kr][jq + 0] = vb.x; Bs[kr][jq + 1] = vb.y; Bs[kr][jq + 2] = vb.z; Bs[kr][jq + 3] = vb.w;
      } else {
        const float4 vb = *reinterpret_cast<const float4*>(Bop + (size_t)row * ldb + k0 + kq);
        Bs[kq + 0][row] = vb.x; Bs[kq + 1][row] = vb.y; Bs[kq + 2][row] = vb.z; Bs[kq + 3][row] = vb.w;
      }
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < TK; ++k) {
      float av[4], bv[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) av[r] = As[k][ty + 16 * r];
#pragma unroll
      for (int c = 0; c < 4; ++c) bv[c] = Bs[k][tx + 16 * c];
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[r][c] = fmaf(av[r], bv[c], acc[r][c]);
    }
    __syncthreads();
  }

  float sc = 1.0f;
  if (g.scales) {
    const float s = g.scales[mat];
    sc = (ROLE == kGram) ? s * s : s;
  }
  float* out = static_cast<float*>(g.out);
  const int ldc = (ROLE == kUpdate) ? g.n_pad : g.m_pad;
  out += (size_t)mat * ((ROLE == kUpdate) ? g.mat_x : g.mat_a);
  const float* ep = nullptr;
  if (ROLE == kPoly) ep = static_cast<const float*>(g.a) + (size_t)mat * g.mat_a;
  if (ROLE == kUpdate) ep = static_cast<const float*>(g.x) + (size_t)mat * g.mat_x;
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int gi = I * TM + ty + 16 * r, gj = J * TM + tx + 16 * c;
      const float a = acc[r][c];
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
