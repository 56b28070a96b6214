// Internal interface between the C ABI layer (muon_api.cpp) and the HIP
// kernels (elementwise.hip, gemm_bf16.hip, gemm_f32.hip). Not installed.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

namespace muon {

// Matrices per elementwise launch: their pointers travel by value in the
// kernel argument block (no device pointer table, nothing to upload).
constexpr int kEwChunk = 128;

// Per-chunk matrix table for the momentum / apply passes.
struct EwMats {
  const void* src[kEwChunk];  // momentum pass: grad (or NS input); apply: param
  float* buf[kEwChunk];       // momentum pass: momentum buffer (may be unused)
  void* dst[kEwChunk];        // apply: param or output matrix
  int ld[kEwChunk];            // row stride (elements) of src, buf and dst as stored
  unsigned char tr[kEwChunk]; // 1 when the matrix is stored tall (rows > cols)
};

// Where the parameter update of one matrix goes, for the apply fused into
// the last Update GEMM: written per matrix by the momentum pass (whose
// kernel arguments carry the pointers), read per tile by the GEMM.
struct ApplyEntry {
  void* dst;   // param, updated in place (step), or the output (orthogonalize)
  int tr;      // 1 when the matrix is stored tall (rows > cols)
  int ld;      // row stride of dst (elements), a multiple of 8
};

// Momentum pass: reads each matrix's source (and momentum buffer), writes
// the buffer, the wide zero-padded NS input X0 = u (rounded to the
// workspace type), and per 64x64 tile one fp32 partial sum of u^2 and a
// flag telling whether any u of the tile is nonzero.
struct MomentumArgs {
  int count;                // matrices in this chunk
  int m, n;                 // wide shape (m <= n)
  int m_pad, n_pad;
  int ew_blocks;            // tiles per matrix
  int first;                // index of the chunk's first matrix in the batch
  void* x0;                 // workspace X0 of the batch
  size_t mat_x;             // elements per padded matrix
  float* partials;          // [batch matrices][ew_blocks]
  int* nonzero;             // [batch matrices][ew_blocks]: 1 if any u of the tile is
                            // not exactly 0 (NaN included), else 0
  int has_buf;              // 0: NS input is src itself (orthogonalize)
  float beta;               // buf' = beta*buf + kg*g
  float kg;                 // 1-beta (EMA) or 1 (heavy ball)
  int nesterov;             // u = kg*g + beta*buf' if 1, else buf'
  ApplyEntry* ptab;         // [batch matrices] entries to fill (dst, tr), or nullptr
};

// Compaction of the per-matrix live flags of a batch into the list of live
// matrices (ascending) and its length, by one workgroup.
// It also zeroes the batch's GEMM tile scheduler counters (sched[0..15]).
hipError_t launch_compact(const int* live, int count, int* live_list, int* nlive, int* sched, hipStream_t s);

// Norm finalize: scales[i] = 1 / (sqrt(sum_k partials[i][k]) + eps), and
// live[i] from the tile flags.
struct FinalizeArgs {
  int count;
  int ew_blocks;
  const float* partials;
  float* scales;
  float eps;
  const int* nonzero;       // per-tile flags of the momentum pass
  int* live;                // per matrix: 1 unless every u is exactly 0
};

// Apply pass: mode 0: p' = alpha*p - gamma[tr]*O; mode 1: out = O.
// O is the wide workspace matrix, times scales[i] when use_scale.
struct ApplyArgs {
  // live (per batch matrix) or nullptr: O is taken as exactly 0 where
  // live[i] == 0 (the NS iterate of those matrices is not stored);
  // dead_only: matrices with live[i] != 0 are left alone (their apply runs
  // inside the last Update GEMM).
  const int* live;
  int dead_only;
  int count;
  int m, n, n_pad;
  int first;
  const void* x;            // workspace holding O
  size_t mat_x;
  const float* scales;
  int use_scale;
  int mode;
  float alpha;              // 1 - lr*wd
  float gamma[2];           // lr*scale for wide [0] and tall [1] members
};

// Batched NS GEMM roles. All operate on padded wide matrices of a batch,
// element strides per matrix given below. Symmetric roles compute only the
// tiles on one side of the diagonal and mirror them.
//   fp32 kernels: Poly writes B = b*A + c*(A A), Update X' = sc*(a*X + B X).
//   bf16 kernels, by muon_options.poly_form:
//     MUON_POLY_SQUARE: with c != 0, Gram writes A' = A + (b/2c) I, Poly
//                 B' = c A'A' + (a - b^2/4c) I = a I + b A + c A A and
//                 Update X' = sc (B' X), so no epilogue reads an operand
//                 tile; with c = 0, Poly writes B' = a I + b A + c A A with
//                 the A tile and Update X' = sc (B' X).
//     MUON_POLY_DIRECT: as the fp32 kernels (A, then b A + c A A with the A
//                 tile, then sc (a X + B X) with the X tile), each rounded
//                 once to bf16.
enum GemmRole {
  kGram = 0,    // A   = sc * X X^T                (sc = s_i^2 or 1)
  kPoly = 1,    // B   (A symmetric)
  kUpdate = 2   // X'                              (sc = s_i or 1)
};

struct GemmArgs {
  const void* x;      // X (Gram and Update operand)
  const void* a;      // A (Poly operand and epilogue)
  const void* b;      // B (Update operand)
  void* out;          // output matrices
  size_t mat_x;       // elements per padded X (m_pad * n_pad)
  size_t mat_a;       // elements per padded A or B (m_pad * m_pad)
  int count;          // matrices in the batch
  int m, n;           // true wide shape (for flop accounting)
  int m_pad, n_pad;
  const float* scales;  // per-matrix s (first iteration) or nullptr
  float ca, cb, cc;     // quintic coefficients of this step
  // bf16 kernels only: the value added on the global diagonal by Gram (A'
  // = A + diag_add I) and Poly, whether Poly reads the A tile in its
  // epilogue (b A + c A A + diag_add I) or not (c A'A' + diag_add I), and
  // whether Update reads the X tile in its epilogue (sc (a X + B X)) or
  // not (sc B' X).
  float diag_add;
  int poly_operand;
  int update_operand;
  // bf16 Update only: when ptab is set, the tile is not stored as X' but
  // applied: p' = alpha*p - gamma[tr]*O (apply_mode 0) or out = O (1), O
  // being X' rounded to bf16, in the matrix's original orientation.
  const ApplyEntry* ptab;
  // bf16 only: the matrices to compute, when not all of the batch: indices
  // of the matrices whose NS input is not exactly zero (idle experts are
  // left out: their iterate stays zero, so no product is needed), and
  // their number (both in device memory). nullptr: every matrix.
  const int* live_list;
  const int* nlive;
  // bf16 only: tile scheduler words (see kSchedWords), or nullptr for the
  // static schedule. sched[x], x < 8, counts the tiles claimed from XCD
  // x's range, sched[8] the workgroups done; both are zero at launch (the
  // last workgroup to finish zeroes them again); sched[16 + b] carries
  // workgroup b's claimed tile to its waves.
  int* sched;
  float alpha;
  float gamma[2];
  int apply_mode;
};

hipError_t launch_momentum(const EwMats& mats, const MomentumArgs& a, int src_bf16, int ws_bf16,
                           hipStream_t s);
hipError_t launch_finalize(const FinalizeArgs& a, hipStream_t s);
hipError_t launch_apply(const EwMats& mats, const ApplyArgs& a, int p_bf16, int ws_bf16,
                        hipStream_t s);
hipError_t launch_gemm_bf16(GemmRole role, const GemmArgs& g, hipStream_t s);
hipError_t launch_gemm_f32(GemmRole role, const GemmArgs& g, hipStream_t s);

// Device address and size of the calling thread's current device's static
// workspace (scratch.hip), resolved on the first call per device.
hipError_t static_workspace(void** ptr, size_t* bytes);

// Algorithmic flops of one launch (nominal: a dense product counts
// 2*M*N*K even where symmetry halves the executed work).
double gemm_flops(GemmRole role, const GemmArgs& g);

}  // namespace muon
