// HIP kernels (gfx950) of the Kamera reuse operator:
//     Y = R(delta) . X + sum_f U_f V_f^T        (Kamera preprint, Eq. 1 in §1)
// R(delta) re-rotates the rope band of keys by delta (preprint §3 "Relocate");
// the patch U_f V_f^T is added after the rotation and is not rotated (preprint
// App. A serve listing). Results are written to dense rows or scattered into a
// paged KV pool (preprint §6).
//
// Two kernels read the same packed batch (kamera_desc.h):
//   rehydrate_mfma<V>  bf16, head_dim 64/128 or MLA with a 64-wide rope band.
//     One wave = 16 tokens x one column group (a 128-column head = 2 slabs, or
//     one 64-column slab) of one tensor, looping over a block of token tiles.
//     The patch contraction (16 tokens x m) . (m x 16 columns) runs on
//     v_mfma_f32_16x16x32_bf16 with the rotated rows as the accumulator input.
//   rehydrate_generic  any dtype/shape; plain fp32 VALU, one workgroup per
//     (chunk, tensor, layer, token block).
//
// Lane layout of the MFMA path (lane = 16*lg + c, c = token in the tile):
//   per 64-column slab s a lane holds columns 64s + 8lg + [0,8) (run 0) and
//   64s + 32 + 8lg + [0,8) (run 1), loaded as two 16-byte reads, so a wave
//   instruction reads 16 rows x 64 contiguous bytes. NeoX partners of a 128-wide
//   head (i, i+64) are the same lane/position in slabs 0 and 1; NeoX partners of
//   a 64-wide band (i, i+32) are runs 0 and 1 of one lane; GPT-J partners are
//   neighbours inside a run.
//   The MFMA result layout gives lane (lg, c) rows M = 4lg + [0,4) of column c.
//   Tile q of slab s maps row M to column 64s + 32(q>>1) + 8(M>>2) + 4(q&1) + (M&3),
//   so the 4 tiles x 4 values of a lane are exactly its two loaded runs. The
//   V^T operand is loaded once per task with that same column map.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kamera_desc.h"

namespace kamera {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

enum { ROT_NONE = 0, ROT_NEOX_SLABS = 1, ROT_NEOX_RUNS = 2, ROT_GPTJ = 3 };

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  bf16x2 r;
  r.x = (__bf16)a;  // v_cvt_pk_bf16_f32: round to nearest even
  r.y = (__bf16)b;
  return __builtin_bit_cast(uint32_t, r);
}
__device__ __forceinline__ float bf_to_f(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }
__device__ __forceinline__ uint16_t f_to_bf(float f) {
  __bf16 b = (__bf16)f;
  return __builtin_bit_cast(uint16_t, b);
}

// cos/sin of delta * theta_i, theta_i = base^(-2i/d_rot), angle formed and
// evaluated in fp64, then rounded once to fp32.
__device__ __forceinline__ void phase_fp64(double base, int d_rot, int64_t delta, int i, float& c,
                                           float& s) {
  const double th = pow(base, (-2.0 * (double)i) / (double)d_rot);
  const double phi = (double)delta * th;
  double sd, cd;
  sincos(phi, &sd, &cd);
  c = (float)cd;
  s = (float)sd;
}

__device__ __forceinline__ int find_chunk(const DevChunk* __restrict__ chunks, int n, int64_t task) {
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (chunks[mid].task0 <= task) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Element offset of token t's row inside one layer of a tensor.
__device__ __forceinline__ int64_t row_offset(const int32_t* __restrict__ pages, int slot0, int P, int F,
                                              int t) {
  if (pages == nullptr) return (int64_t)t * F;
  const int s = slot0 + t;
  const int pg = pages[s / P];
  return ((int64_t)pg * P + (s % P)) * F;
}

// ============================================================================
// MFMA path
// ============================================================================
struct TaskCtx {
  const uint16_t* src;   // layer base of the source tensor
  uint16_t* dst;         // layer base of the destination tensor
  const int32_t* pages;
  int slot0, P, F, T;
  int colbase;           // first column of the group
  int tok0, ntiles;
  bool in_place, paged;
};

template <int NSLAB, int NK>
__device__ __forceinline__ void mfma_task(const DevHeader& hd, const DevChunk& ch, const TaskCtx& tc,
                                          int layer, int tensor, int rot, const int* kfac,
                                          const int* kstep, int lane) {
  const int lg = lane >> 4;
  const int c = lane & 15;

  // ---- rotation coefficients for the pairs this lane holds
  float cs[NSLAB * 8], sn[NSLAB * 8];
  if (rot != ROT_NONE) {
    float cl = 1.f, sl = 0.f;
    const int npairs = hd.d_rot >> 1;
    if (lane < npairs) phase_fp64(hd.rope_base, hd.d_rot, ch.delta, lane, cl, sl);
#pragma unroll
    for (int j = 0; j < NSLAB * 8; ++j) {
      int p;
      if (rot == ROT_NEOX_SLABS) {          // j in [0,16): slab 0 element j
        p = 32 * (j >> 3) + 8 * lg + (j & 7);
      } else if (rot == ROT_NEOX_RUNS) {    // j in [0,8): run 0 element j
        p = 8 * lg + j;
      } else {                              // GPT-J: element pair (2j, 2j+1)
        const int e2 = 2 * j;               // element index inside the lane's 16*NSLAB
        const int s = e2 >> 4, r = (e2 >> 3) & 1, e = e2 & 7;
        p = (64 * s + 32 * r + 8 * lg + e) >> 1;
      }
      cs[j] = __shfl(cl, p, 64);
      sn[j] = __shfl(sl, p, 64);
    }
  }

  // ---- V^T operands: A[M][k] = Vt[k][col(M)] for every slab, tile and k-step
  bf16x8 av[NK > 0 ? NSLAB * 4 * NK : 1];
  bool uvec[NK > 0 ? NK : 1];
  const uint16_t* ubase[NK > 0 ? NK : 1];
  int urank[NK > 0 ? NK : 1];
#pragma unroll
  for (int j = 0; j < NK; ++j) {
    const DevFactor& f = ch.fac[kfac[j]];
    const int lrel = layer - f.layer0;
    const uint16_t* vt = (const uint16_t*)f.vt + (int64_t)lrel * f.rank * f.width;
    ubase[j] = (const uint16_t*)f.u + (int64_t)lrel * ch.T * f.rank + 32 * kstep[j] + 8 * lg;
    urank[j] = f.rank - 32 * kstep[j] - 8 * lg;   // valid k entries from this lane's offset
    uvec[j] = f.pad[0] != 0;
    const int mrow = lane & 15;
    const int kg = lane >> 4;
#pragma unroll
    for (int s = 0; s < NSLAB; ++s) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int col = tc.colbase + 64 * s + 32 * (q >> 1) + 8 * (mrow >> 2) + 4 * (q & 1) + (mrow & 3);
        const int rel = col - f.col0;
        const bool in = rel >= 0 && rel < f.width;
        bf16x8 a;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int k = 32 * kstep[j] + 8 * kg + e;
          const uint16_t h = (in && k < f.rank) ? vt[(int64_t)k * f.width + rel] : (uint16_t)0;
          a[e] = __builtin_bit_cast(__bf16, h);
        }
        av[(s * 4 + q) * NK + j] = a;
      }
    }
  }

  const bool compute = (rot != ROT_NONE) || (NK > 0);

  auto src_row = [&](int t) -> const uint16_t* {
    return tc.src + row_offset(tc.in_place ? tc.pages : nullptr, tc.slot0, tc.P, tc.F, t);
  };
  auto dst_row = [&](int t) -> uint16_t* {
    return tc.dst + row_offset(tc.pages, tc.slot0, tc.P, tc.F, t);
  };

  u32x4 cur[NSLAB][2], nxt[NSLAB][2];
  bf16x8 ucur[NK > 0 ? NK : 1], unxt[NK > 0 ? NK : 1];

  auto load_tile = [&](int tile, u32x4 (&raw)[NSLAB][2], bf16x8 (&ub)[NK > 0 ? NK : 1]) {
    const int t = tc.tok0 + tile * kTileTokens + c;
    const bool valid = t < tc.T;
    const uint16_t* row = valid ? src_row(t) : nullptr;
#pragma unroll
    for (int s = 0; s < NSLAB; ++s)
#pragma unroll
      for (int r = 0; r < 2; ++r)
        raw[s][r] = valid ? *(const u32x4*)(row + tc.colbase + 64 * s + 32 * r + 8 * lg) : u32x4{0, 0, 0, 0};
#pragma unroll
    for (int j = 0; j < NK; ++j) {
      bf16x8 b;
      if (valid && uvec[j] && urank[j] >= 8) {
        b = *(const bf16x8*)(ubase[j] + (int64_t)t * (ch.fac[kfac[j]].rank));
      } else {
        const int rk = ch.fac[kfac[j]].rank;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint16_t h = (valid && e < urank[j]) ? ubase[j][(int64_t)t * rk + e] : (uint16_t)0;
          b[e] = __builtin_bit_cast(__bf16, h);
        }
      }
      ub[j] = b;
    }
  };

  load_tile(0, cur, ucur);
  for (int tile = 0; tile < tc.ntiles; ++tile) {
    if (tile + 1 < tc.ntiles) load_tile(tile + 1, nxt, unxt);
    const int t = tc.tok0 + tile * kTileTokens + c;
    const bool valid = t < tc.T;

    u32x4 out[NSLAB][2];
    if (!compute) {
#pragma unroll
      for (int s = 0; s < NSLAB; ++s)
#pragma unroll
        for (int r = 0; r < 2; ++r) out[s][r] = cur[s][r];
    } else {
      float x[NSLAB * 16];
#pragma unroll
      for (int s = 0; s < NSLAB; ++s)
#pragma unroll
        for (int r = 0; r < 2; ++r)
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            x[16 * s + 8 * r + 2 * w] = bf_lo(cur[s][r][w]);
            x[16 * s + 8 * r + 2 * w + 1] = bf_hi(cur[s][r][w]);
          }
      if (rot == ROT_NEOX_SLABS) {
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const float a = x[j], b = x[16 + (j & 15)];
          x[j] = fmaf(a, cs[j], -(b * sn[j]));
          x[16 + (j & 15)] = fmaf(a, sn[j], b * cs[j]);
        }
      } else if (rot == ROT_NEOX_RUNS) {
#pragma unroll
        for (int s = 0; s < NSLAB; ++s)
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const float a = x[16 * s + j], b = x[16 * s + 8 + j];
            x[16 * s + j] = fmaf(a, cs[j], -(b * sn[j]));
            x[16 * s + 8 + j] = fmaf(a, sn[j], b * cs[j]);
          }
      } else if (rot == ROT_GPTJ) {
#pragma unroll
        for (int j = 0; j < NSLAB * 8; ++j) {
          const float a = x[2 * j], b = x[2 * j + 1];
          x[2 * j] = fmaf(a, cs[j], -(b * sn[j]));
          x[2 * j + 1] = fmaf(a, sn[j], b * cs[j]);
        }
      }
      if constexpr (NK > 0) {
#pragma unroll
        for (int s = 0; s < NSLAB; ++s)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            f32x4 acc = {x[16 * s + 4 * q], x[16 * s + 4 * q + 1], x[16 * s + 4 * q + 2], x[16 * s + 4 * q + 3]};
#pragma unroll
            for (int j = 0; j < NK; ++j)
              acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[(s * 4 + q) * NK + j], ucur[j], acc, 0, 0, 0);
            x[16 * s + 4 * q] = acc[0];
            x[16 * s + 4 * q + 1] = acc[1];
            x[16 * s + 4 * q + 2] = acc[2];
            x[16 * s + 4 * q + 3] = acc[3];
          }
      }
#pragma unroll
      for (int s = 0; s < NSLAB; ++s)
#pragma unroll
        for (int r = 0; r < 2; ++r)
#pragma unroll
          for (int w = 0; w < 4; ++w)
            out[s][r][w] = pack2(x[16 * s + 8 * r + 2 * w], x[16 * s + 8 * r + 2 * w + 1]);
    }
    if (valid) {
      uint16_t* row = dst_row(t);
#pragma unroll
      for (int s = 0; s < NSLAB; ++s)
#pragma unroll
        for (int r = 0; r < 2; ++r)
          *(u32x4*)(row + tc.colbase + 64 * s + 32 * r + 8 * lg) = out[s][r];
    }
    if (tile + 1 < tc.ntiles) {
#pragma unroll
      for (int s = 0; s < NSLAB; ++s)
#pragma unroll
        for (int r = 0; r < 2; ++r) cur[s][r] = nxt[s][r];
#pragma unroll
      for (int j = 0; j < NK; ++j) ucur[j] = unxt[j];
    }
  }
}

template <int NSLAB, int BUDGET>
__device__ __forceinline__ void mfma_dispatch_nk(int nk, const DevHeader& hd, const DevChunk& ch,
                                                 const TaskCtx& tc, int layer, int tensor, int rot,
                                                 const int* kfac, const int* kstep, int lane) {
  // NK must satisfy NSLAB * NK <= BUDGET; the host guarantees it.
  switch (nk) {
    case 0: mfma_task<NSLAB, 0>(hd, ch, tc, layer, tensor, rot, kfac, kstep, lane); break;
    case 1: if constexpr (NSLAB * 1 <= BUDGET) mfma_task<NSLAB, 1>(hd, ch, tc, layer, tensor, rot, kfac, kstep, lane); break;
    case 2: if constexpr (NSLAB * 2 <= BUDGET) mfma_task<NSLAB, 2>(hd, ch, tc, layer, tensor, rot, kfac, kstep, lane); break;
    case 3: if constexpr (NSLAB * 3 <= BUDGET) mfma_task<NSLAB, 3>(hd, ch, tc, layer, tensor, rot, kfac, kstep, lane); break;
    case 4: if constexpr (NSLAB * 4 <= BUDGET) mfma_task<NSLAB, 4>(hd, ch, tc, layer, tensor, rot, kfac, kstep, lane); break;
    case 5: if constexpr (NSLAB * 5 <= BUDGET) mfma_task<NSLAB, 5>(hd, ch, tc, layer, tensor, rot, kfac, kstep, lane); break;
    case 6: if constexpr (NSLAB * 6 <= BUDGET) mfma_task<NSLAB, 6>(hd, ch, tc, layer, tensor, rot, kfac, kstep, lane); break;
    case 7: if constexpr (NSLAB * 7 <= BUDGET) mfma_task<NSLAB, 7>(hd, ch, tc, layer, tensor, rot, kfac, kstep, lane); break;
    case 8: if constexpr (NSLAB * 8 <= BUDGET) mfma_task<NSLAB, 8>(hd, ch, tc, layer, tensor, rot, kfac, kstep, lane); break;
    default: break;
  }
}

template <int BUDGET>
__global__ __launch_bounds__(kBlockThreads) void rehydrate_mfma(const DevHeader* __restrict__ hdr,
                                                                const DevChunk* __restrict__ chunks) {
  const int lane = threadIdx.x & (kWaveSize - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const DevHeader& hd = *hdr;
  const int64_t task = (int64_t)blockIdx.x * kWavesPerBlock + wave;
  if (task >= hd.total_tasks) return;
  const DevChunk& ch = chunks[find_chunk(chunks, hd.nchunks, task)];

  int64_t r = task - ch.task0;
  const int g = ch.group0 + (int)(r % ch.ngroups);
  r /= ch.ngroups;
  const int tb = (int)(r % ch.ntb);
  r /= ch.ntb;
  const int layer = (int)(r % hd.L);
  const int stream = (int)(r / hd.L);
  const int tensor = ch.stream_tensor[stream];

  TaskCtx tc;
  tc.in_place = (ch.flags & 2u) != 0;
  tc.pages = ch.pages;
  tc.paged = ch.pages != nullptr;
  tc.slot0 = ch.slot0;
  tc.P = hd.page_size;
  tc.F = hd.F;
  tc.T = ch.T;
  tc.colbase = g * hd.group_cols;
  tc.tok0 = tb * ch.tb_tokens;
  const int ntok = min(ch.tb_tokens, ch.T - tc.tok0);
  tc.ntiles = (ntok + kTileTokens - 1) / kTileTokens;
  tc.src = (const uint16_t*)ch.src[tensor] + (int64_t)layer * ch.src_ls;
  tc.dst = (uint16_t*)ch.dst[tensor] + (int64_t)layer * ch.dst_ls;

  const int nslab = hd.group_cols / kSlab;
  // Does this task rotate? K (GQA) or the rope group (MLA), and only for delta != 0.
  int rot = ROT_NONE;
  const bool band = hd.family == 0 ? (tensor == 0) : (g == hd.rope_group);
  if (band && ch.delta != 0) {
    if (hd.pairing == 1) rot = ROT_GPTJ;
    else rot = (hd.d_rot == 128) ? ROT_NEOX_SLABS : ROT_NEOX_RUNS;
  }
  // k-steps of the factors covering this group's columns
  int kfac[8], kstep[8];
  int nk = 0;
  if (ch.flags & 1u) {
    for (int f = 0; f < ch.nfac; ++f) {
      const DevFactor& fa = ch.fac[f];
      if (fa.tensor != tensor || fa.rank <= 0 || layer < fa.layer0) continue;
      if (fa.col0 >= tc.colbase + hd.group_cols || fa.col0 + fa.width <= tc.colbase) continue;
      for (int k = 0; k * 32 < fa.rank && nk < 8; ++k) {
        kfac[nk] = f;
        kstep[nk] = k;
        ++nk;
      }
    }
  }
  // In place, a group with nothing to do is left untouched.
  if (tc.in_place && rot == ROT_NONE && nk == 0) return;

  if (nslab == 2) mfma_dispatch_nk<2, BUDGET>(nk, hd, ch, tc, layer, tensor, rot, kfac, kstep, lane);
  else mfma_dispatch_nk<1, BUDGET>(nk, hd, ch, tc, layer, tensor, rot, kfac, kstep, lane);
}

// ============================================================================
// Generic path (fp32 or bf16, any even rotary width, any rank)
// ============================================================================
template <typename T>
__device__ __forceinline__ float ld(const void* p, int64_t i);
template <>
__device__ __forceinline__ float ld<float>(const void* p, int64_t i) { return ((const float*)p)[i]; }
template <>
__device__ __forceinline__ float ld<uint16_t>(const void* p, int64_t i) { return bf_to_f(((const uint16_t*)p)[i]); }
template <typename T>
__device__ __forceinline__ void st(void* p, int64_t i, float v);
template <>
__device__ __forceinline__ void st<float>(void* p, int64_t i, float v) { ((float*)p)[i] = v; }
template <>
__device__ __forceinline__ void st<uint16_t>(void* p, int64_t i, float v) { ((uint16_t*)p)[i] = f_to_bf(v); }

template <typename T>
__device__ __forceinline__ float add_patch(const DevChunk& ch, int layer, int tensor, int t, int col, float acc) {
  for (int fi = 0; fi < ch.nfac; ++fi) {
    const DevFactor& f = ch.fac[fi];
    if (f.tensor != tensor || layer < f.layer0 || col < f.col0 || col >= f.col0 + f.width) continue;
    const int64_t lrel = layer - f.layer0;
    const int64_t ub = lrel * ch.T * f.rank + (int64_t)t * f.rank;
    const int64_t vb = lrel * f.rank * f.width + (col - f.col0);
    for (int j = 0; j < f.rank; ++j) acc = fmaf(ld<T>(f.u, ub + j), ld<T>(f.vt, vb + (int64_t)j * f.width), acc);
  }
  return acc;
}

template <typename T>
__global__ __launch_bounds__(kBlockThreads) void rehydrate_generic(const DevHeader* __restrict__ hdr,
                                                                   const DevChunk* __restrict__ chunks) {
  __shared__ float2 tab[256];
  const DevHeader& hd = *hdr;
  const int64_t task = blockIdx.x;
  if (task >= hd.total_tasks) return;  // uniform over the block
  const DevChunk& ch = chunks[find_chunk(chunks, hd.nchunks, task)];
  int64_t r = task - ch.task0;
  const int tb = (int)(r % ch.ntb);
  r /= ch.ntb;
  const int layer = (int)(r % hd.L);
  const int stream = (int)(r / hd.L);
  const int tensor = ch.stream_tensor[stream];
  const bool in_place = (ch.flags & 2u) != 0;
  const bool patch = (ch.flags & 1u) != 0;
  const bool rotate = tensor == 0 && ch.delta != 0;
  const int npairs = hd.d_rot >> 1;
  if (rotate)
    for (int p = threadIdx.x; p < npairs; p += blockDim.x) {
      float c, s;
      phase_fp64(hd.rope_base, hd.d_rot, ch.delta, p, c, s);
      tab[p] = make_float2(c, s);
    }
  __syncthreads();

  const int nbands = hd.family == 0 ? hd.H : 1;
  const int band_stride = hd.family == 0 ? hd.head_dim : 0;
  const int band0 = hd.family == 0 ? 0 : hd.latent_dim;
  const int n_pair_items = (tensor == 0) ? nbands * npairs : 0;   // rotary pairs (rotated or not)
  const int n_single = hd.F - 2 * n_pair_items;
  // In place without a patch only the rotary pairs change.
  const int first_item = (in_place && !patch) ? n_single : 0;
  const int nitems = n_single + n_pair_items - first_item;
  const int tok0 = tb * ch.tb_tokens;
  const int ntok = min(ch.tb_tokens, ch.T - tok0);
  const size_t es = sizeof(T);
  const char* src = (const char*)ch.src[tensor] + (int64_t)layer * ch.src_ls * es;
  char* dst = (char*)ch.dst[tensor] + (int64_t)layer * ch.dst_ls * es;

  for (int idx = threadIdx.x; idx < ntok * nitems; idx += blockDim.x) {
    const int t = tok0 + idx / nitems;
    const int item = first_item + idx % nitems;
    const int64_t so = row_offset(in_place ? ch.pages : nullptr, ch.slot0, hd.page_size, hd.F, t);
    const int64_t dof = row_offset(ch.pages, ch.slot0, hd.page_size, hd.F, t);
    if (item < n_single) {
      const int col = item;
      const bool touched = patch;
      if (!touched) {  // byte-exact copy
        if (!in_place) {
          if (es == 2) ((uint16_t*)dst)[dof + col] = ((const uint16_t*)src)[so + col];
          else ((uint32_t*)dst)[dof + col] = ((const uint32_t*)src)[so + col];
        }
        continue;
      }
      float v = ld<T>(src, so + col);
      v = add_patch<T>(ch, layer, tensor, t, col, v);
      st<T>(dst, dof + col, v);
    } else {
      const int k = item - n_single;
      const int b = k / npairs, i = k % npairs;
      const int p = hd.pairing == 1 ? 2 * i : i;
      const int q = hd.pairing == 1 ? 2 * i + 1 : i + npairs;
      const int cp = band0 + b * band_stride + p, cq = band0 + b * band_stride + q;
      if (!rotate && !patch) {
        if (!in_place) {
          if (es == 2) {
            ((uint16_t*)dst)[dof + cp] = ((const uint16_t*)src)[so + cp];
            ((uint16_t*)dst)[dof + cq] = ((const uint16_t*)src)[so + cq];
          } else {
            ((uint32_t*)dst)[dof + cp] = ((const uint32_t*)src)[so + cp];
            ((uint32_t*)dst)[dof + cq] = ((const uint32_t*)src)[so + cq];
          }
        }
        continue;
      }
      float a = ld<T>(src, so + cp), bb = ld<T>(src, so + cq);
      if (rotate) {
        const float2 cs = tab[i];
        const float na = fmaf(a, cs.x, -(bb * cs.y));
        const float nb = fmaf(a, cs.y, bb * cs.x);
        a = na;
        bb = nb;
      }
      if (patch) {
        a = add_patch<T>(ch, layer, tensor, t, cp, a);
        bb = add_patch<T>(ch, layer, tensor, t, cq, bb);
      }
      st<T>(dst, dof + cp, a);
      st<T>(dst, dof + cq, bb);
    }
  }
}

// ============================================================================
// Launchers
// ============================================================================
hipError_t launch_mfma(int variant, const DevHeader* hdr, const DevChunk* chunks, int64_t tasks,
                       hipStream_t stream) {
  const int64_t blocks = (tasks + kWavesPerBlock - 1) / kWavesPerBlock;
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  const dim3 grid((unsigned)blocks), block(kBlockThreads);
  switch (variant) {
    case 0: hipLaunchKernelGGL(rehydrate_mfma<2>, grid, block, 0, stream, hdr, chunks); break;
    case 1: hipLaunchKernelGGL(rehydrate_mfma<4>, grid, block, 0, stream, hdr, chunks); break;
    case 2: hipLaunchKernelGGL(rehydrate_mfma<8>, grid, block, 0, stream, hdr, chunks); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_generic(int dtype, const DevHeader* hdr, const DevChunk* chunks, int64_t tasks,
                          hipStream_t stream) {
  if (tasks <= 0) return hipSuccess;
  if (tasks > 0x7fffffffLL) return hipErrorInvalidValue;
  const dim3 grid((unsigned)tasks), block(kBlockThreads);
  if (dtype == 0) hipLaunchKernelGGL(rehydrate_generic<float>, grid, block, 0, stream, hdr, chunks);
  else hipLaunchKernelGGL(rehydrate_generic<uint16_t>, grid, block, 0, stream, hdr, chunks);
  return hipGetLastError();
}

}  // namespace kamera
