// Internal interface between the host library and the patch-builder kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kamera {

constexpr int kBuildMaxRank = 64;       // top-m factors kept, m <= 64
constexpr int kBuildMaxSubspace = 80;   // iterated subspace p = min(80, width, T)
constexpr int kBuildMaxPairs = 256;     // d_rot <= 512
constexpr int kBuildMaxSweeps = 40;     // Jacobi sweeps (quadratic convergence: ~6-10 needed)
constexpr double kBuildJacobiTol = 2.220446049250313e-16;
constexpr int kBuildMaxOrbit = 32;      // orderings averaged by an orbit patch

struct BuildArgs {
  const void* x_cond[kBuildMaxOrbit];     // per ordering: [T][F] storage dtype
  int64_t delta_k[kBuildMaxOrbit];        // per ordering: the relocation offset
  int norbit;                             // orderings averaged (1: a single deficit)
  const void* x_canon;  // [T][F]
  void* u_out;          // [T][m]
  void* v_out;          // [W][m]
  double* sigma;        // [m] or null
  double* delta;        // workspace: [T][W]
  double* gram;         // [W][W]
  double* q;            // [p][W]
  double* z;            // [p][W]
  double* h;            // [p][p]
  double* evec;         // [p][p]
  double* lam;          // [p]
  double* vm;           // [W][m]
  double* bz;           // [p][p]  Gram of the block being orthonormalised
  double* lf;           // [p][p]  its Cholesky factor (lower)
  double* zpart;        // [ksplit][p][W] partial products of Z = Q G (ksplit > 1)
  int ksplit;           // slices of the sum over j in Z = Q G
  int* flag;            // 1: Cholesky QR rejected the block, the CGS2 fallback runs
  double base;          // RoPE base
  int T, F, W, col0, m, p, iters;
  int dtype;            // 0 fp32, 1 bf16
  int rotate;           // the tensor carries rotary bands
  int band0, band_stride, nbands, d_rot, pairing;
};

// Workspace layout: fp64 arrays in the order of BuildArgs, each 256-byte aligned.
size_t build_workspace_bytes(int64_t T, int64_t W, int64_t m);
void build_workspace_carve(BuildArgs& a, void* ws);

hipError_t launch_builder(const BuildArgs& a, hipStream_t stream);

}  // namespace kamera
