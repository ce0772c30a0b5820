// Patch builder (the compile step) for gfx950: top-m factors of the deficit
//     Delta = KV(B|A) - R(delta) . KV(B|empty)
// Kamera preprint, §2 Eq. 2 (the deficit) and App. A (compile step: conditioned
// rows minus the relocated canonical, truncated SVD stored as U*Sigma and V), or of
// the mean deficit over a set of orderings (§5, reorder: the orbit patch).
//
// Method: randomized subspace iteration with a Rayleigh-Ritz step (Halko,
// Martinsson & Tropp, SIAM Review 2011, §4.5 and §5.3) on the Gram matrix
// G = Delta^T Delta, everything in fp64:
//   delta_k   Delta [T][W] for the patched columns [col0, col0 + W)
//   gram_k    G [W][W] (upper 32 x 32 tiles, mirrored)
//             (gram_wide_k for wide rows: one wave per tile, 4 x 4 outputs per lane)
//   start_k   a deterministic pseudo-random start block Z0 [p][W]
//   orthonormalisation of the block Z (p x W) into Q, once for the range
//   finder and once per power step: shifted CholeskyQR (Fukaya, Kannan,
//   Nakatsukasa, Yamamoto & Yanagisawa, SIAM J. Sci. Comput. 2020), a Cholesky
//   QR pass on Z Z^T + sI; the last one, whose Q enters the Rayleigh-Ritz step,
//   adds two plain passes (shifted CholeskyQR3) for orthonormality to working
//   precision, while the earlier ones only carry the span to the next product;
//   each pass is B = X X^T (dots_k), B = L L^T (chol_k, one workgroup, LDS) and
//   X <- L^-1 X (trsm_k).
//   A block whose pivots collapse anyway (rank-deficient Z, e.g. Delta = 0)
//   sets a flag and is orthonormalised by CGS2 instead (by the first workgroup of
//   the orthonormalisation's last trsm_k)
//   zt_k      Z = Q G (rows of Q times the symmetric G)
//   dots_k    H = Q Z^T = Q G Q^T (p x p)
//   jacobi_k  eigenpairs of H: parallel cyclic Jacobi (Brent & Luk 1985
//             round-robin ordering) in one workgroup's LDS, sorted descending
//   finish_k  V_m = Q^T E[:, :m], sigma = sqrt(lambda)
//   usig_k    U*Sigma = Delta V_m
// U*Sigma and V are rounded once from fp64 to the storage dtype.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kamera_builder.h"

namespace kamera {

namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ double load_x(const void* p, int dtype, int64_t i) {
  if (dtype == 1) return (double)__uint_as_float((uint32_t)((const uint16_t*)p)[i] << 16);
  return (double)((const float*)p)[i];
}

// fp64 -> bf16, round to nearest even, without double rounding: round to odd
// into fp32 first (an exact sticky bit, 16 spare bits), then to nearest even.
__device__ __forceinline__ uint16_t bf16_from_f64(double v) {
  float f = (float)v;
  if ((double)f != v && f == f && !__builtin_isinf(f)) {
    if (fabs((double)f) > fabs(v)) f = __uint_as_float(__float_as_uint(f) - 1u);  // toward zero
    f = __uint_as_float(__float_as_uint(f) | 1u);                                // sticky
  }
  uint32_t b = __float_as_uint(f);
  if ((b & 0x7f800000u) == 0x7f800000u) return (uint16_t)((b >> 16) | ((b & 0xffffu) ? 0x40u : 0u));
  b += 0x7fffu + ((b >> 16) & 1u);
  return (uint16_t)(b >> 16);
}

__device__ __forceinline__ void store_x(void* p, int dtype, int64_t i, double v) {
  if (dtype == 1)
    ((uint16_t*)p)[i] = bf16_from_f64(v);
  else
    ((float*)p)[i] = (float)v;
}

__device__ __forceinline__ double wave_sum(double v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Sum over the workgroup; every thread gets the result. `red` holds one slot per wave.
__device__ double block_sum(double v, double* red) {
  v = wave_sum(v);
  const int w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  double s = 0.0;
  for (int i = 0; i < nw; ++i) s += red[i];
  return s;
}

// Counter-based hash (the splitmix64 finaliser) -> uniform in [-1, 1).
__device__ __forceinline__ double hash_uniform(uint64_t x) {
  x = x * 0x9E3779B97F4A7C15ull + 0x2545F4914F6CDD1Dull;
  x ^= x >> 30;
  x *= 0xBF58476D1CE4E5B9ull;
  x ^= x >> 27;
  x *= 0x94D049BB133111EBull;
  x ^= x >> 31;
  return (double)(x >> 11) * (2.0 / 9007199254740992.0) - 1.0;
}

// Delta[t][w] = mean_k x_cond_k[t][c] - (Rbar x_canon)[t][c], c = col0 + w, in fp64,
// where Rbar = mean_k R(delta_k) acts on each rotary pair as [[cbar, -sbar], [sbar, cbar]]
// (cbar, sbar the means of cos and sin of delta_k theta_i). By linearity this is the
// mean of the per-ordering deficits x_cond_k - R(delta_k) x_canon (one ordering: the
// plain deficit). Rotation as in the relocation operator: theta_i = base^(-2i/d_rot),
// NeoX pairs (i, i + d_rot/2) or GPT-J pairs (2i, 2i + 1) per band.
__global__ __launch_bounds__(kThreads) void delta_k(BuildArgs a) {
  __shared__ double cs_tab[kBuildMaxPairs], sn_tab[kBuildMaxPairs];
  const int npairs = a.d_rot / 2;
  const double inv_k = 1.0 / (double)a.norbit;
  if (a.rotate)
    for (int i = threadIdx.x; i < npairs; i += blockDim.x) {
      const double th = pow(a.base, (-2.0 * (double)i) / (double)a.d_rot);
      double cm = 0.0, sm = 0.0;
      for (int k = 0; k < a.norbit; ++k) {
        double s, c;
        sincos((double)a.delta_k[k] * th, &s, &c);
        cm += c;
        sm += s;
      }
      cs_tab[i] = cm * inv_k;
      sn_tab[i] = sm * inv_k;
    }
  __syncthreads();
  const int64_t n = (int64_t)a.T * a.W;
  const int64_t band_end = a.band0 + (int64_t)a.nbands * a.band_stride;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < n; e += (int64_t)gridDim.x * blockDim.x) {
    const int t = (int)(e / a.W), w = (int)(e % a.W);
    const int c = a.col0 + w;
    const int64_t row = (int64_t)t * a.F;
    double solo = load_x(a.x_canon, a.dtype, row + c);
    if (a.rotate && c >= a.band0 && c < band_end) {
      const int o = a.band0 + ((c - a.band0) / a.band_stride) * a.band_stride;
      const int i = c - o;
      if (i < a.d_rot) {
        int pi, partner;
        bool first;
        if (a.pairing == 1) {
          pi = i >> 1;
          first = (i & 1) == 0;
          partner = o + (first ? i + 1 : i - 1);
        } else {
          first = i < npairs;
          pi = first ? i : i - npairs;
          partner = o + (first ? i + npairs : i - npairs);
        }
        const double other = load_x(a.x_canon, a.dtype, row + partner);
        const double cv = cs_tab[pi], sv = sn_tab[pi];
        solo = first ? solo * cv - other * sv : other * sv + solo * cv;
      }
    }
    double cond = 0.0;
    for (int k = 0; k < a.norbit; ++k) cond += load_x(a.x_cond[k], a.dtype, row + c);
    a.delta[e] = cond * inv_k - solo;
  }
}

// G = Delta^T Delta. One 32 x 32 tile (bi <= bj) per workgroup; the mirror tile is
// written from the same sums, so G is exactly symmetric.
static_assert(32 * 32 % kThreads == 0, "gram_k's staging covers a 32 x 32 tile exactly");
__global__ __launch_bounds__(kThreads) void gram_k(BuildArgs a) {
  __shared__ double ti[32][33], tj[32][33];
  const int tiles = (a.W + 31) / 32;
  int bi = 0, rem = blockIdx.x;  // blockIdx.x enumerates the upper triangle row by row
  while (rem >= tiles - bi) {
    rem -= tiles - bi;
    ++bi;
  }
  const int bj = bi + rem;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;  // ty in [0, 8): rows 4ty..4ty+3
  double acc[4] = {0.0, 0.0, 0.0, 0.0};
  // The next 32 rows' loads are issued before the current ones are multiplied, all of
  // them together: entries outside Delta read element 0 instead (in bounds) and are
  // replaced by zeros when stored.
  constexpr int kGL = 32 * 32 / kThreads;
  double vi[kGL], vj[kGL];
  auto fetch = [&](int t0) {
#pragma unroll
    for (int q = 0; q < kGL; ++q) {
      const int k = threadIdx.x + q * kThreads, r = k >> 5, col = k & 31, t = t0 + r;
      const int ci = bi * 32 + col, cj = bj * 32 + col;
      vi[q] = a.delta[(t < a.T && ci < a.W) ? (int64_t)t * a.W + ci : 0];
      vj[q] = a.delta[(t < a.T && cj < a.W) ? (int64_t)t * a.W + cj : 0];
    }
  };
  fetch(0);
  for (int t0 = 0; t0 < a.T; t0 += 32) {
#pragma unroll
    for (int q = 0; q < kGL; ++q) {
      const int k = threadIdx.x + q * kThreads, r = k >> 5, col = k & 31, t = t0 + r;
      const int ci = bi * 32 + col, cj = bj * 32 + col;
      ti[r][col] = (t < a.T && ci < a.W) ? vi[q] : 0.0;
      tj[r][col] = (t < a.T && cj < a.W) ? vj[q] : 0.0;
    }
    __syncthreads();
    if (t0 + 32 < a.T) fetch(t0 + 32);  // uniform
    for (int r = 0; r < 32; ++r) {
      const double vj = tj[r][tx];
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[q] = fma(ti[r][ty * 4 + q], vj, acc[q]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int i = bi * 32 + ty * 4 + q, j = bj * 32 + tx;
    if (i < a.W && j < a.W) {
      a.gram[(int64_t)i * a.W + j] = acc[q];
      a.gram[(int64_t)j * a.W + i] = acc[q];
    }
  }
}

// G for wide rows (many tiles, so one wave per tile still fills the chip): one wave per 32 x 32
// tile of the upper triangle, lane (ty, tx) of an 8 x 8 grid accumulating rows 4 ty .. 4 ty + 3
// and columns 4 tx .. 4 tx + 3 of the tile, which reads 8 LDS values per 16 fmas (gram_k: 5 per
// 4). Each output is the same sum over t, in the same order, as in gram_k.
constexpr int kGramWideTiles = 2048;  // upper-triangle tiles from which this kernel is used
__global__ __launch_bounds__(64) void gram_wide_k(BuildArgs a) {
  __shared__ __align__(16) double ti[32][36], tj[32][36];  // rows of 288 B: 16-byte aligned pairs
  const int tiles = (a.W + 31) / 32;
  int bi = 0, rem = blockIdx.x;  // blockIdx.x enumerates the upper triangle row by row
  while (rem >= tiles - bi) {
    rem -= tiles - bi;
    ++bi;
  }
  const int bj = bi + rem;
  const int lane = threadIdx.x, ty = lane >> 3, tx = lane & 7;
  double acc[4][4];
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int v = 0; v < 4; ++v) acc[u][v] = 0.0;
  for (int t0 = 0; t0 < a.T; t0 += 32) {
    // all 32 loads of the chunk in flight together; entries outside Delta read element 0
    // (in bounds) and are stored as zeros
    double vi[16], vj[16];
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int k = lane + 64 * q, r = k >> 5, col = k & 31, t = t0 + r;
      const int ci = bi * 32 + col, cj = bj * 32 + col;
      vi[q] = a.delta[(t < a.T && ci < a.W) ? (int64_t)t * a.W + ci : 0];
      vj[q] = a.delta[(t < a.T && cj < a.W) ? (int64_t)t * a.W + cj : 0];
    }
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int k = lane + 64 * q, r = k >> 5, col = k & 31, t = t0 + r;
      const int ci = bi * 32 + col, cj = bj * 32 + col;
      ti[r][col] = (t < a.T && ci < a.W) ? vi[q] : 0.0;
      tj[r][col] = (t < a.T && cj < a.W) ? vj[q] : 0.0;
    }
    __syncthreads();
#pragma unroll 4
    for (int r = 0; r < 32; ++r) {
      const double2 x01 = *(const double2*)&ti[r][4 * ty], x23 = *(const double2*)&ti[r][4 * ty + 2];
      const double2 y01 = *(const double2*)&tj[r][4 * tx], y23 = *(const double2*)&tj[r][4 * tx + 2];
      const double x[4] = {x01.x, x01.y, x23.x, x23.y}, y[4] = {y01.x, y01.y, y23.x, y23.y};
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[u][v] = fma(x[u], y[v], acc[u][v]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int i = bi * 32 + 4 * ty + u, j = bj * 32 + 4 * tx + v;
      if (i < a.W && j < a.W) {
        a.gram[(int64_t)i * a.W + j] = acc[u][v];
        a.gram[(int64_t)j * a.W + i] = acc[u][v];
      }
    }
}

__global__ __launch_bounds__(kThreads) void start_k(BuildArgs a) {
  const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e < (int64_t)a.p * a.W) a.z[e] = hash_uniform((uint64_t)e);
}

// Z[k][i] = sum_j Q[k][j] G[j][i] (Q: p x W, p <= 80; G: W x W). A workgroup computes all p rows
// of 64 columns over one slice of the sum (workgroup (cb, s): columns 64 cb + [0, 64), j in
// slice s of zt_split(W)), staging 32-wide chunks of Q and G in LDS; thread (tr, tc) of a 16 x 16
// grid accumulates rows tr + 16 r (r < 5) and columns tc + 16 c (c < 4), so its LDS reads and the
// final writes have unit stride across the wave. Each G element is read once per slice and used
// for 80 rows. With more than one slice the partial products go to zpart and zred_k adds them
// in slice order (deterministic).
constexpr int kZCols = 64, kZChunk = 32;
static_assert(kBuildMaxSubspace * kZChunk % kThreads == 0 && kZChunk * kZCols % kThreads == 0,
              "the staging loops cover the LDS chunks exactly");
__global__ __launch_bounds__(kThreads) void zt_k(BuildArgs a) {
  __shared__ double qs[kBuildMaxSubspace][kZChunk + 1];
  __shared__ double gs[kZChunk][kZCols + 1];
  const int tid = threadIdx.x, tr = tid >> 4, tc = tid & 15;
  const int c0 = blockIdx.x * kZCols;
  const int kl = (a.W + a.ksplit - 1) / a.ksplit;
  const int j0 = blockIdx.y * kl, j1 = min(a.W, j0 + kl);
  double acc[5][4];
#pragma unroll
  for (int r = 0; r < 5; ++r)
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[r][c] = 0.0;
  for (int jc = j0; jc < j1; jc += kZChunk) {
    const int kn = min(kZChunk, j1 - jc);
    // Every load of the chunk is issued before the first is waited for: entries outside
    // Q or G read element 0 instead (in bounds) and are replaced by zeros afterwards.
    constexpr int kQL = kBuildMaxSubspace * kZChunk / kThreads, kGL = kZChunk * kZCols / kThreads;
    double qv[kQL], gv[kGL];
#pragma unroll
    for (int t = 0; t < kQL; ++t) {
      const int e = tid + t * kThreads, r = e / kZChunk, k = e % kZChunk;
      qv[t] = a.q[(r < a.p && k < kn) ? (int64_t)r * a.W + jc + k : 0];
    }
#pragma unroll
    for (int t = 0; t < kGL; ++t) {
      const int e = tid + t * kThreads, k = e / kZCols, c = e % kZCols;
      gv[t] = a.gram[(k < kn && c0 + c < a.W) ? (int64_t)(jc + k) * a.W + c0 + c : 0];
    }
#pragma unroll
    for (int t = 0; t < kQL; ++t) {
      const int e = tid + t * kThreads, r = e / kZChunk, k = e % kZChunk;
      qs[r][k] = (r < a.p && k < kn) ? qv[t] : 0.0;
    }
#pragma unroll
    for (int t = 0; t < kGL; ++t) {
      const int e = tid + t * kThreads, k = e / kZCols, c = e % kZCols;
      gs[k][c] = (k < kn && c0 + c < a.W) ? gv[t] : 0.0;
    }
    __syncthreads();
#pragma unroll 4
    for (int k = 0; k < kZChunk; ++k) {  // entries past kn are zero and add nothing
      double qv[5], gv[4];
#pragma unroll
      for (int r = 0; r < 5; ++r) qv[r] = qs[tr + 16 * r][k];
#pragma unroll
      for (int c = 0; c < 4; ++c) gv[c] = gs[k][tc + 16 * c];
#pragma unroll
      for (int r = 0; r < 5; ++r)
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[r][c] = fma(qv[r], gv[c], acc[r][c]);
    }
    __syncthreads();
  }
  double* out = a.ksplit > 1 ? a.zpart + (int64_t)blockIdx.y * a.p * a.W : a.z;
#pragma unroll
  for (int r = 0; r < 5; ++r)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int row = tr + 16 * r, col = c0 + tc + 16 * c;
      if (row < a.p && col < a.W) out[(int64_t)row * a.W + col] = acc[r][c];
    }
}

// Z = the sum of the slices' partial products, added in slice order.
__global__ __launch_bounds__(kThreads) void zred_k(BuildArgs a) {
  const int64_t e = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const int64_t n = (int64_t)a.p * a.W;
  if (e >= n) return;
  double v = 0.0;
#pragma unroll 8
  for (int s = 0; s < a.ksplit; ++s) v += a.zpart[(int64_t)s * n + e];  // unrolled: the loads overlap, the sum keeps its order
  a.z[e] = v;
}

// Q = rows of Z orthonormalised by classical Gram-Schmidt with one
// re-orthogonalisation pass (CGS2). A row that is numerically in the span of
// the previous ones (rank-deficient Delta, or Delta = 0) is replaced by a fresh
// pseudo-random row and orthonormalised again. Run by one whole workgroup.
__device__ void cgs2_block(const BuildArgs& a, double* red, double* coef) {
  const int W = a.W, p = a.p;
  const int waves = blockDim.x >> 6, wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  for (int j = 0; j < p; ++j) {
    double* qj = a.q + (int64_t)j * W;
    for (int attempt = 0; attempt < 4; ++attempt) {
      double n0 = 0.0;
      for (int i = threadIdx.x; i < W; i += blockDim.x) {
        const double v = attempt == 0
                             ? a.z[(int64_t)j * W + i]
                             : hash_uniform(((uint64_t)(attempt * kBuildMaxSubspace + j) << 32) + (uint64_t)i);
        qj[i] = v;
        n0 += v * v;
      }
      n0 = block_sum(n0, red);  // its barriers also publish the row written above
      for (int pass = 0; pass < 2; ++pass) {
        for (int k = wave; k < j; k += waves) {
          const double* qk = a.q + (int64_t)k * W;
          double d = 0.0;
          for (int i = lane; i < W; i += 64) d = fma(qk[i], qj[i], d);
          d = wave_sum(d);
          if (lane == 0) coef[k] = d;
        }
        __syncthreads();
        for (int i = threadIdx.x; i < W; i += blockDim.x) {
          double v = qj[i];
          for (int k = 0; k < j; ++k) v = fma(-coef[k], a.q[(int64_t)k * W + i], v);
          qj[i] = v;
        }
        __syncthreads();
      }
      double nn = 0.0;
      for (int i = threadIdx.x; i < W; i += blockDim.x) nn += qj[i] * qj[i];
      nn = block_sum(nn, red);
      if (n0 > 0.0 && nn > 1e-24 * n0 && nn > 1e-280) {
        const double inv = 1.0 / sqrt(nn);
        for (int i = threadIdx.x; i < W; i += blockDim.x) qj[i] *= inv;
        __syncthreads();
        break;
      }
    }
  }
}

// out[r][c] = sum_i X[r][i] Y[c][i] for p x W blocks X, Y: one wave per entry.
__global__ __launch_bounds__(kThreads) void dots_k(BuildArgs a, const double* x, const double* y, double* out) {
  const int e = blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (e >= a.p * a.p) return;
  const int r = e / a.p, c = e % a.p;
  // X X^T: entries (r, c) and (c, r) take the same products in the same order, so the
  // wave of the upper one writes both and the other returns
  const bool gram = x == y;
  if (gram && c < r) return;  // uniform over the wave
  const double* xr = x + (int64_t)r * a.W;
  const double* yc = y + (int64_t)c * a.W;
  double s = 0.0;
#pragma unroll 8
  for (int i = lane; i < a.W; i += 64) s = fma(xr[i], yc[i], s);  // unrolled: the loads overlap
  s = wave_sum(s);
  if (lane == 0) {
    out[e] = s;
    if (gram) out[c * a.p + r] = s;
  }
}

// Cholesky factor B = L L^T of the p x p Gram of a block (right-looking, in LDS).
// pass 0 factors B + sI with s = 11 (W p + p (p + 1)) u trace(B), u = 2^-53 (the
// shift of shifted CholeskyQR, which keeps the factorisation alive up to a
// condition number of 1/u); passes 1 and 2 factor B itself and reject a pivot
// below 1e-14 (pass 1) or 1e-6 (pass 2) of its column's squared norm, which
// CholeskyQR2 could not bring back to orthogonality. A rejection sets the flag
// (pass 0 sets it, later passes can only add to it) and the CGS2 fallback runs.
//
// Blocked by 16 columns: wave 0 factors the diagonal block in registers (lane i holds
// row i of the block; the pivot and the entries of column k are read with v_readlane,
// so a pivot step costs no LDS round trip and no workgroup barrier) and carries up to 48
// rows below it through the same eliminations (the panel; rows past the wave's 64 are
// solved one per thread), then the workgroup updates the trailing triangle: two
// barriers per block instead of two per pivot. Every pivot is still
// the fully updated diagonal entry, so the breakdown test sees the values the
// unblocked order would (up to rounding order). A pivot step is a chain of dependent
// fp64 operations, so it is kept short: 1/sqrt(d) from v_rsq_f64 and two Newton steps
// (relative error ~1 ulp; L[k][k] = d / sqrt(d), the column scaled by the product; a
// pivot below 2^-1000, far under any useful scale, counts as a breakdown, which keeps the
// estimate away from subnormal inputs), and no lane predication in the update (a lane's
// entries above the diagonal take garbage and are never stored).
constexpr int kCholThreads = 1024;
constexpr int kCholB = 16;
__device__ __forceinline__ double readlane_f64(double v, int l) {
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, l);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), l);
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

__global__ __launch_bounds__(kCholThreads) void chol_k(BuildArgs a, int pass) {
  __shared__ double Ls[kBuildMaxSubspace][kBuildMaxSubspace + 1];
  __shared__ double dg[kBuildMaxSubspace];
  __shared__ double dinv[kCholB];
  __shared__ double red[kCholThreads / 64];
  __shared__ int bad_s;
  const int p = a.p;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  double tr = 0.0;
  for (int i = threadIdx.x; i < p; i += blockDim.x) tr += a.bz[i * p + i];
  tr = block_sum(tr, red);
  const double shift = pass == 0 ? 11.0 * ((double)a.W * p + (double)p * (p + 1)) * 0x1p-53 * tr : 0.0;
  const double ratio = pass == 0 ? 0.0 : (pass == 1 ? 1e-14 : 1e-6);
  // lower triangle only; 32 x 32 thread grid, loads unrolled so they overlap
#pragma unroll
  for (int r0 = 0; r0 < kBuildMaxSubspace; r0 += kCholThreads / 32) {
    const int r = r0 + (threadIdx.x >> 5);
#pragma unroll
    for (int cc = 0; cc < kBuildMaxSubspace; cc += 32) {
      const int c = cc + (threadIdx.x & 31);
      if (r < p && c <= r) {
        const double v = 0.5 * (a.bz[r * p + c] + a.bz[c * p + r]) + (r == c ? shift : 0.0);
        Ls[r][c] = v;
        if (r == c) dg[r] = v;
      }
    }
  }
  if (threadIdx.x == 0) bad_s = !(tr > 0.0) || !(tr < 1e300);
  __syncthreads();
  for (int k0 = 0; k0 < p; k0 += kCholB) {
    const int kb = min(kCholB, p - k0), k1 = k0 + kb;
    if (wave == 0) {  // ---- columns [k0, k1) of rows k0 .. k0 + 63 in registers
      // lane i holds row k0 + i: the diagonal block's rows (i < kb, lower part) and below
      // them up to 48 panel rows, which the same eliminations turn into L[row][k0 .. k1)
      double r[kCholB];
      const int row = k0 + lane;
#pragma unroll
      for (int j = 0; j < kCholB; ++j) r[j] = (row < p && j < kb && (lane >= kb || j <= lane)) ? Ls[row][k0 + j] : 0.0;
      // Fully unrolled (register indices must be constants): steps past the block or
      // after a rejected pivot are skipped by uniform conditions, never by a break.
      int bad = bad_s;
      const double dgl = lane < kb ? dg[k0 + lane] : 0.0;      // the block's original diagonal
      // A rejected pivot only raises the flag (the block is discarded); the arithmetic goes
      // on with a harmless value, so no step branches on it. What a lane computes above its
      // own diagonal or in columns at and past kb is never stored (rows past p hold zeros),
      // so the updates need no guard.
      auto pivot = [&](int k) {
        const double d0 = readlane_f64(r[k], k);                // the pivot
        const bool ok = d0 > ratio * readlane_f64(dgl, k) && d0 > 0x1p-1000 && d0 < 1e300;
        bad |= !ok;
        const double d = ok ? d0 : 1.0;
        double y = __builtin_amdgcn_rsq(d);                     // 1/sqrt(d), refined twice
        y = y * fma(-0.5 * d * y, y, 1.5);
        y = y * fma(-0.5 * d * y, y, 1.5);
        const double lik = r[k] * y;                            // L[i][k] for the lanes below the pivot
        r[k] = lane == k ? d * y : lik;
#pragma unroll
        for (int j = k + 1; j < kCholB; ++j) r[j] = fma(-lik, readlane_f64(r[k], j), r[j]);
      };
      if (kb == kCholB) {  // uniform: a full block runs as one straight line, so the compiler
                           // can start each pivot while the previous one's updates issue
#pragma unroll
        for (int k = 0; k < kCholB; ++k) pivot(k);
      } else {
#pragma unroll
        for (int k = 0; k < kCholB; ++k)
          if (k < kb) pivot(k);                                 // uniform
      }
      if (!bad) {
#pragma unroll
        for (int j = 0; j < kCholB; ++j)
          if (row < p && j < kb && (lane >= kb || j <= lane)) Ls[row][k0 + j] = r[j];
        if (lane < kb) {
          double djj = 0.0;
#pragma unroll
          for (int j = 0; j < kCholB; ++j) djj = j == lane ? r[j] : djj;
          dinv[lane] = 1.0 / djj;
        }
      }
      if (lane == 0) bad_s = bad;
    }
    __syncthreads();
    if (bad_s) break;  // uniform
    // ---- panel rows past wave 0's 64 (only with p > k0 + 64): L[i][K] = B[i][K] L_KK^-T, row by row
    if (k0 + 64 < p) {  // uniform
    for (int i = k0 + 64 + threadIdx.x; i < p; i += blockDim.x) {
      double x[kCholB];
#pragma unroll
      for (int j = 0; j < kCholB; ++j) {
        if (j < kb) {  // uniform
          double v = Ls[i][k0 + j];
#pragma unroll
          for (int l = 0; l < j; ++l) v = fma(-x[l], Ls[k0 + j][k0 + l], v);
          x[j] = v * dinv[j];
          Ls[i][k0 + j] = x[j];
        }
      }
    }
    __syncthreads();
    }
    // ---- trailing triangle k1 <= j <= i < p: B[i][j] -= L[i][K] . L[j][K]
    for (int i = k1 + (threadIdx.x >> 5); i < p; i += kCholThreads / 32) {
#pragma unroll
      for (int jj = 0; jj < kBuildMaxSubspace; jj += 32) {
        const int j = k1 + jj + (threadIdx.x & 31);
        if (j <= i) {  // the block's 16 products unrolled: their loads are independent
          double v = Ls[i][j];
#pragma unroll
          for (int l = 0; l < kCholB; ++l)
            if (l < kb) v = fma(-Ls[i][k0 + l], Ls[j][k0 + l], v);
          Ls[i][j] = v;
        }
      }
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) *a.flag = pass == 0 ? bad_s : (*a.flag | bad_s);
  for (int r0 = 0; r0 < p; r0 += kCholThreads / 32) {  // lower triangle; the upper part is never read
    const int r = r0 + (threadIdx.x >> 5);
#pragma unroll
    for (int cc = 0; cc < kBuildMaxSubspace; cc += 32) {
      const int c = cc + (threadIdx.x & 31);
      if (r < p && c <= r) a.lf[r * p + c] = Ls[r][c];
    }
  }
}

// Q = L^-1 Z by forward substitution, one wave per column i of the block: lane l
// holds rows l and l + 64. Step k takes the finished entry q_k from its lane
// (v_readlane at a uniform index) and removes its contribution from the rows below;
// L is kept transposed in LDS so the lanes read a contiguous row of it. The LDS copy
// holds only the strictly lower part (the diagonal enters through its reciprocals) and
// zeros elsewhere, also past p, so the steps need no lane conditions and the loop is
// unrolled over the largest p: the Lt reads are issued ahead of the dependency chain.
// All of a column is read before any of it is written, so src == dst is allowed.
constexpr int kTrsmWaves = 8;

// With `fallback` set (the last solve of an orthonormalisation) and the flag raised, the
// first workgroup orthonormalises Z by CGS2 instead and the others return.
__global__ __launch_bounds__(kTrsmWaves * 64) void trsm_k(BuildArgs a, const double* src, double* dst,
                                                        int fallback) {
  __shared__ double Lt[kBuildMaxSubspace][kBuildMaxSubspace + 1];  // Lt[k][r] = L[r][k], r > k
  __shared__ double inv[kBuildMaxSubspace];
  __shared__ double red[kTrsmWaves];
  const int p = a.p, W = a.W;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  // The flag, L and this wave's column are requested together (one memory round trip,
  // not three); the flag is only tested once they are in flight.
  const int flagged = *a.flag;
  const int i = blockIdx.x * kTrsmWaves + wave;
  const int r0 = lane, r1 = lane + 64, r1c = min(r1, kBuildMaxSubspace);
  const bool col = i < W;  // uniform over the wave
  double acc0 = col && r0 < p ? src[(int64_t)r0 * W + i] : 0.0;
  double acc1 = col && r1 < p ? src[(int64_t)r1 * W + i] : 0.0;
  // compile-time trip counts: all of a thread's loads are in flight together (a runtime
  // loop would wait for each load before the next)
#pragma unroll
  for (int rr = 0; rr < kBuildMaxSubspace; rr += kTrsmWaves) {
    const int r = rr + wave;
#pragma unroll
    for (int kk = 0; kk < kBuildMaxSubspace + 64 - 1; kk += 64) {
      const int k = kk + lane;
      if (k < kBuildMaxSubspace) Lt[k][r] = (r < p && k < r) ? a.lf[r * p + k] : 0.0;
    }
  }
  for (int r = threadIdx.x; r < kBuildMaxSubspace; r += blockDim.x) {
    inv[r] = r < p ? 1.0 / a.lf[r * p + r] : 0.0;
    Lt[r][kBuildMaxSubspace] = 0.0;  // the padding column: what lanes past the last row read
  }
  if (flagged) {  // uniform over the workgroup
    if (fallback && blockIdx.x == 0) cgs2_block(a, red, inv);  // inv: scratch for the CGS2 coefficients
    return;
  }
  __syncthreads();
  if (!col) return;     // uniform over the wave
#pragma unroll
  for (int k = 0; k < kBuildMaxSubspace; ++k) {  // past p: q_k = 0 and the rows stay as they are
    const double qk = readlane_f64(k < 64 ? acc0 : acc1, k & 63) * inv[k];
    acc0 = fma(-Lt[k][r0], qk, acc0);
    acc1 = fma(-Lt[k][r1c], qk, acc1);
  }
  if (r0 < p) dst[(int64_t)r0 * W + i] = acc0 * inv[r0];
  if (r1 < p) dst[(int64_t)r1 * W + i] = acc1 * inv[r1];
}

// Eigenpairs of the symmetric p x p matrix H by parallel cyclic Jacobi: each
// round applies p/2 disjoint plane rotations chosen by the round-robin
// tournament (player n-1 fixed, the rest rotating); a rotation is skipped when
// its off-diagonal entry is negligible against the geometric mean of the two
// diagonal entries or against 1e-17 ||H||_F, and the sweeps stop once a whole
// sweep skips every pair.
constexpr int kJacobiThreads = 1024;
constexpr int kJacobiPairs = kBuildMaxSubspace / 2;
constexpr int kJacobiStride = kBuildMaxSubspace + 1;
constexpr int kJacobiRows = 4;  // rows of E per work item
static_assert(kJacobiPairs * (kJacobiPairs + 1) / 2 <= kJacobiThreads, "one block of A per thread");
static_assert(kBuildMaxSubspace % kJacobiRows == 0 &&
              64 + kBuildMaxSubspace / kJacobiRows * kJacobiPairs <= kJacobiThreads, "one item of E per thread");

// The two players of slot k in round r of the round-robin tournament of n players (n
// even): slot 0 pits player n-1 against player r, slot k > 0 players r + k and r - k
// modulo n - 1.
__device__ __forceinline__ void tourney_pair(int n, int r, int k, int& lo, int& hi) {
  int x = n - 1, y = r;
  if (k != 0) {
    x = r + k;
    y = r + n - 1 - k;
    if (x >= n - 1) x -= n - 1;  // both sums lie below 2 (n - 1)
    if (y >= n - 1) y -= n - 1;
  }
  lo = min(x, y);
  hi = max(x, y);
}

__global__ __launch_bounds__(kJacobiThreads) void jacobi_k(BuildArgs a) {
  // H is symmetric and so is every J^T H J: only the upper triangle of A (row <= column)
  // is kept, entry (i, j) at (min(i, j), max(i, j)). Rows and columns past p (the bye, when
  // p is odd, and the rows of E that fill the last item) hold zeros, which every rotation
  // maps to zeros, so the items need no bounds tests.
  __shared__ double A[kBuildMaxSubspace * kJacobiStride];
  __shared__ double E[kBuildMaxSubspace * kJacobiStride];
  __shared__ double2 rot[2][kJacobiPairs];  // (cos, sin) of each slot, for rounds of either parity
  __shared__ int2 slot_pq[2][kJacobiPairs];  // the slot's two players (lo, hi)
  __shared__ int order[kBuildMaxSubspace];
  __shared__ int rotated, rot_stamp;
  __shared__ double red[kJacobiThreads / 64];
  const int p = a.p;
  const int n = p + (p & 1);  // an even number of players; index p is a bye when p is odd
  auto at = [](int i, int j) { return min(i, j) * kJacobiStride + max(i, j); };
  double ss = 0.0;
  for (int e = threadIdx.x; e < kBuildMaxSubspace * kJacobiStride; e += blockDim.x) {
    const int r = e / kJacobiStride, c = e % kJacobiStride;
    double v = 0.0;
    if (r < p && c < p) v = 0.5 * (a.h[r * p + c] + a.h[c * p + r]);
    A[e] = v;
    E[e] = (r == c && r < p) ? 1.0 : 0.0;
    ss += v * v;
  }
  // entries below 1e-17 ||H||_F are left alone: rounding noise of that size
  // reappears with every rotation, so chasing it would never end
  const double floor_abs = fmax(1e-17 * sqrt(block_sum(ss, red)), 1e-300);
  // Round g: wave 0 derives the rotations of the round's n/2 disjoint slots while the other
  // waves apply round g - 1's rotations to E (E <- E J; the rotations only read A); then
  // one flat pass applies A <- J^T A J. The slots split the rows and the columns alike, so
  // the 2 x 2 blocks (row slot k, column slot l) partition A; a block's new values depend
  // only on its own four entries and the two rotations, and block (l, k) is the transpose
  // of block (k, l), so thread w < n/2 (n/2 + 1) / 2 takes block (k, l) with k <= l and
  // w = l (l + 1) / 2 + k. Thread 64 + v, v < (rows / 4) n/2, takes rows 4 (v / (n/2)) to
  // 4 (v / (n/2)) + 3 of E for slot v % (n/2). No entry is touched by two threads and every
  // item runs without branches, so its LDS reads issue together. Two barriers per round.
  const int np2 = n / 2, nblk = np2 * (np2 + 1) / 2;
  const int nitem = (p + kJacobiRows - 1) / kJacobiRows * np2;
  const int w = threadIdx.x, v = threadIdx.x - 64;
  int bk = 0, bl = 0;  // this thread's block of A
  if (w < nblk) {      // the float root is off by at most one
    int l = (int)((sqrtf((float)(8 * w + 1)) - 1.0f) * 0.5f);
    if ((l + 1) * (l + 2) / 2 <= w) ++l;
    if (l * (l + 1) / 2 > w) --l;
    bk = w - l * (l + 1) / 2;
    bl = l;
  }
  const bool has_e = v >= 0 && v < nitem;
  const int erow = max(v, 0) / max(np2, 1) * kJacobiRows, eslot = max(v, 0) % max(np2, 1);  // its item of E
  auto update_e = [&](int b) {  // E <- E J with the rotations recorded in buffer b
    const double2 r = rot[b][eslot];
    const int lo = slot_pq[b][eslot].x, hi = slot_pq[b][eslot].y;
    double u[kJacobiRows], x[kJacobiRows];
#pragma unroll
    for (int i = 0; i < kJacobiRows; ++i) {
      u[i] = E[(erow + i) * kJacobiStride + lo];
      x[i] = E[(erow + i) * kJacobiStride + hi];
    }
#pragma unroll
    for (int i = 0; i < kJacobiRows; ++i) {
      E[(erow + i) * kJacobiStride + lo] = r.x * u[i] - r.y * x[i];
      E[(erow + i) * kJacobiStride + hi] = r.y * u[i] + r.x * x[i];
    }
  };
  bool pending = false;  // uniform: the last round turned, and E has yet to follow
  int g = 0;             // rounds so far; the rotation buffers alternate with its parity
  if (threadIdx.x == 0) rot_stamp = 0;  // published by the first sweep's barriers
  for (int sweep = 0; sweep < kBuildMaxSweeps; ++sweep) {
    __syncthreads();
    if (threadIdx.x == 0) rotated = 0;
    __syncthreads();
    for (int round = 0; round < n - 1; ++round, ++g) {
      const int b = g & 1;
      // A round that turns no pair skips its pass. The rotating pairs write the round's own
      // stamp: a later round can overwrite it only after every thread has read it (a round
      // that turns something has a second barrier), and in a round that turns nothing any
      // value seen differs from the round's stamp, so no reset (and no race on one) is needed.
      const int stamp = sweep * n + round + 1;
      if (pending && has_e) update_e(b ^ 1);
      for (int k = threadIdx.x; k < np2; k += blockDim.x) {  // k < n/2 <= 40: wave 0 only
        int lo, hi;
        tourney_pair(n, round, k, lo, hi);
        // the bye's row and column are zeros: apq = 0 never turns
        const double apq = A[at(lo, hi)], app = A[at(lo, lo)], aqq = A[at(hi, hi)];
        const bool turn = fabs(apq) > floor_abs && fabs(apq) > kBuildJacobiTol * sqrt(fabs(app * aqq));
        // The rotation that zeroes apq, by two reciprocal square roots (v_rsq_f64 and two
        // Newton steps each) in place of a square root and a division: with
        // 1/r = 1/sqrt(da^2 + db^2), cos 2th = |da|/r and sin 2th = sign(da) db/r, so
        // cos th = sqrt(h) with h = (1 + cos 2th)/2, and sin th = sin 2th/(2 cos th); the
        // smaller angle, |th| <= pi/4. Computed without a branch (the test above runs
        // beside it) and discarded when apq is below the thresholds. The entries are Gram
        // sums of bounded data, so da^2 + db^2 neither overflows nor, when apq passes the
        // floor, vanishes.
        const double da = aqq - app, db = 2.0 * apq;
        const double u = fma(da, da, db * db);
        double r = __builtin_amdgcn_rsq(u);
        r = r * fma(-0.5 * u * r, r, 1.5);
        r = r * fma(-0.5 * u * r, r, 1.5);
        const double h = fma(0.5 * fabs(da), r, 0.5);
        double y = __builtin_amdgcn_rsq(h);
        y = y * fma(-0.5 * h * y, y, 1.5);
        y = y * fma(-0.5 * h * y, y, 1.5);
        const double c = turn ? h * y : 1.0;
        const double s = turn ? copysign(0.5, da) * db * r * y : 0.0;
        if (turn) {
          rotated = 1;
          rot_stamp = stamp;
        }
        rot[b][k] = make_double2(c, s);
        slot_pq[b][k] = make_int2(lo, hi);
      }
      __syncthreads();
      // Buffer b ^ 1, read by the E items before this barrier, is next written in round
      // g + 1, after it. A round that turns nothing skips its pass and its second barrier:
      // a wave that reads the stamp late may then see round g + 1's, which differs from
      // this round's as well.
      pending = rot_stamp == stamp;
      if (!pending) continue;
      if (w < nblk) {
        // (a diagonal block, k == l, reads and writes its off-diagonal entry twice, as
        // (pk, qk) and as (qk, pk); the second write holds the same value up to rounding)
        const double2 rk = rot[b][bk], rl = rot[b][bl];
        const int2 sk = slot_pq[b][bk], sl = slot_pq[b][bl];
        const int pk = sk.x, qk = sk.y, pl = sl.x, ql = sl.y;
        const int o00 = at(pk, pl), o01 = at(pk, ql), o10 = at(qk, pl), o11 = at(qk, ql);
        const double x00 = A[o00], x01 = A[o01], x10 = A[o10], x11 = A[o11];
        const double r00 = rk.x * x00 - rk.y * x10, r10 = rk.y * x00 + rk.x * x10;   // rows (pk, qk)
        const double r01 = rk.x * x01 - rk.y * x11, r11 = rk.y * x01 + rk.x * x11;
        A[o00] = rl.x * r00 - rl.y * r01;                                            // columns (pl, ql)
        A[o01] = rl.y * r00 + rl.x * r01;
        A[o10] = rl.x * r10 - rl.y * r11;
        A[o11] = rl.y * r10 + rl.x * r11;
      }
      __syncthreads();
    }
    if (!rotated) break;
  }
  if (pending && has_e) update_e((g - 1) & 1);  // the last round's rotations
  __syncthreads();
  for (int i = threadIdx.x; i < p; i += blockDim.x) {  // rank by eigenvalue, descending; ties by index
    int rank = 0;
    for (int j = 0; j < p; ++j)
      if (A[at(j, j)] > A[at(i, i)] || (A[at(j, j)] == A[at(i, i)] && j < i)) ++rank;
    order[rank] = i;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < p * p; e += blockDim.x) {
    const int r = e / p, k = e % p;
    a.evec[r * p + k] = E[r * kJacobiStride + order[k]];
  }
  for (int k = threadIdx.x; k < p; k += blockDim.x) a.lam[k] = A[at(order[k], order[k])];
}

// V_m[i][k] = sum_j Q[j][i] E[j][k]; sigma_k = sqrt(max(lambda_k, 0)).
__global__ __launch_bounds__(kThreads) void finish_k(BuildArgs a) {
  const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e < a.m && a.sigma) a.sigma[e] = sqrt(fmax(a.lam[e], 0.0));
  if (e >= (int64_t)a.W * a.m) return;
  const int i = (int)(e / a.m), k = (int)(e % a.m);
  double s = 0.0;
#pragma unroll 8
  for (int j = 0; j < a.p; ++j) s = fma(a.q[(int64_t)j * a.W + i], a.evec[j * a.p + k], s);  // loads overlap
  a.vm[e] = s;
  store_x(a.v_out, a.dtype, e, s);
}

// (U Sigma)[t][k] = sum_w Delta[t][w] V_m[w][k].
__global__ __launch_bounds__(kThreads) void usig_k(BuildArgs a) {
  const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= (int64_t)a.T * a.m) return;
  const int t = (int)(e / a.m), k = (int)(e % a.m);
  const double* d = a.delta + (int64_t)t * a.W;
  double s = 0.0;
#pragma unroll 8
  for (int w = 0; w < a.W; ++w) s = fma(d[w], a.vm[(int64_t)w * a.m + k], s);  // loads overlap, order kept
  store_x(a.u_out, a.dtype, e, s);
}

unsigned blocks_for(int64_t n, int per) { return (unsigned)((n + per - 1) / per); }

size_t align256(size_t v) { return (v + 255) / 256 * 256; }

}  // namespace

// Slices of the sum in Z = Q G: enough workgroups to fill the chip (about 512 with 64-column
// blocks), each slice at least 16 terms long.
int zt_split(int64_t W) {
  const int64_t blocks = (W + kZCols - 1) / kZCols;
  int64_t ks = (512 + blocks - 1) / blocks;
  ks = std::min<int64_t>(ks, std::max<int64_t>(W / 16, 1));
  return (int)std::max<int64_t>(ks, 1);
}

size_t build_workspace_bytes(int64_t T, int64_t W, int64_t m) {
  const int64_t p = std::min<int64_t>(kBuildMaxSubspace, std::min(W, T));
  const int64_t ks = zt_split(W);
  const size_t d = sizeof(double);
  return align256(T * W * d) + align256(W * W * d) + 2 * align256(p * W * d) + 4 * align256(p * p * d) +
         align256(p * d) + align256(W * m * d) + (ks > 1 ? align256(ks * p * W * d) : 0) + 256;
}

void build_workspace_carve(BuildArgs& a, void* ws) {
  char* c = (char*)ws;
  const size_t d = sizeof(double);
  auto take = [&](int64_t count) {
    double* r = (double*)c;
    c += align256((size_t)count * d);
    return r;
  };
  a.delta = take((int64_t)a.T * a.W);
  a.gram = take((int64_t)a.W * a.W);
  a.q = take((int64_t)a.p * a.W);
  a.z = take((int64_t)a.p * a.W);
  a.h = take((int64_t)a.p * a.p);
  a.evec = take((int64_t)a.p * a.p);
  a.lam = take(a.p);
  a.vm = take((int64_t)a.W * a.m);
  a.bz = take((int64_t)a.p * a.p);
  a.lf = take((int64_t)a.p * a.p);
  a.ksplit = zt_split(a.W);
  a.zpart = a.ksplit > 1 ? take((int64_t)a.ksplit * a.p * a.W) : nullptr;
  a.flag = (int*)c;
}

hipError_t launch_builder(const BuildArgs& a, hipStream_t st) {
  const dim3 blk(kThreads);
  const int64_t tw = (int64_t)a.T * a.W;
  hipLaunchKernelGGL(delta_k, dim3(std::min<unsigned>(blocks_for(tw, kThreads), 8192u)), blk, 0, st, a);
  const int tiles = (a.W + 31) / 32;
  const int gtiles = tiles * (tiles + 1) / 2;
  if (gtiles >= kGramWideTiles) hipLaunchKernelGGL(gram_wide_k, dim3(gtiles), dim3(64), 0, st, a);
  else hipLaunchKernelGGL(gram_k, dim3(gtiles), blk, 0, st, a);
  hipLaunchKernelGGL(start_k, dim3(blocks_for((int64_t)a.p * a.W, kThreads)), blk, 0, st, a);
  const dim3 dgrid(blocks_for((int64_t)a.p * a.p, kThreads / 64));
  const dim3 tgrid(blocks_for(a.W, kTrsmWaves));
  // a.z -> a.q. Only the last orthonormalisation feeds the Rayleigh-Ritz step, which needs Q
  // orthonormal to working precision: it takes all three passes. The earlier ones only carry
  // the iterates' span (the same for any basis of it) to the next product and must keep that
  // basis well conditioned, which the shifted pass alone does; they stop after it.
  auto orthonormalise = [&](bool last) {
    hipLaunchKernelGGL(dots_k, dgrid, blk, 0, st, a, (const double*)a.z, (const double*)a.z, a.bz);
    hipLaunchKernelGGL(chol_k, dim3(1), dim3(kCholThreads), 0, st, a, 0);
    hipLaunchKernelGGL(trsm_k, tgrid, dim3(kTrsmWaves * 64), 0, st, a, (const double*)a.z, a.q, last ? 0 : 1);
    for (int pass = 1; last && pass <= 2; ++pass) {
      hipLaunchKernelGGL(dots_k, dgrid, blk, 0, st, a, (const double*)a.q, (const double*)a.q, a.bz);
      hipLaunchKernelGGL(chol_k, dim3(1), dim3(kCholThreads), 0, st, a, pass);
      hipLaunchKernelGGL(trsm_k, tgrid, dim3(kTrsmWaves * 64), 0, st, a, (const double*)a.q, a.q,
                         pass == 2 ? 1 : 0);
    }
  };
  orthonormalise(false);
  const dim3 zgrid(blocks_for(a.W, kZCols), a.ksplit);
  const dim3 rgrid(blocks_for((int64_t)a.p * a.W, kThreads));
  auto product = [&]() {  // a.z = a.q G
    hipLaunchKernelGGL(zt_k, zgrid, blk, 0, st, a);
    if (a.ksplit > 1) hipLaunchKernelGGL(zred_k, rgrid, blk, 0, st, a);
  };
  for (int it = 0; it <= a.iters; ++it) {  // the range finder's product, then `iters` power steps
    product();
    orthonormalise(it == a.iters);
  }
  product();
  hipLaunchKernelGGL(dots_k, dgrid, blk, 0, st, a, (const double*)a.q, (const double*)a.z, a.h);
  hipLaunchKernelGGL(jacobi_k, dim3(1), dim3(kJacobiThreads), 0, st, a);
  hipLaunchKernelGGL(finish_k, dim3(blocks_for((int64_t)a.W * a.m, kThreads)), blk, 0, st, a);
  hipLaunchKernelGGL(usig_k, dim3(blocks_for((int64_t)a.T * a.m, kThreads)), blk, 0, st, a);
  return hipGetLastError();
}

}  // namespace kamera
