// HIP kernels (gfx950) of the Kamera reuse operator:
//     Y = R(delta) . X + sum_f U_f V_f^T        (Kamera preprint, Eq. 1 in §1)
// R(delta) re-rotates the rope band of keys by delta (preprint §3 "Relocate");
// the patch U_f V_f^T is added after the rotation and is not rotated (preprint
// App. A serve listing). Results are written to dense rows or scattered into a
// paged KV pool (preprint §6).
//
// Two kernels read the same packed batch (kamera_desc.h):
//   rehydrate_mfma<S,K>  bf16, head_dim 64/128 or MLA with a 64-wide rope band.
//     One wave = one column group (a 128-column head = 2 slabs, or one
//     64-column slab) of one tensor over a block of 16-token tiles. The patch
//     contraction (16 tokens x m) . (m x 16 columns) runs on
//     v_mfma_f32_16x16x32_bf16 with the rotated rows as the accumulator input.
//     Rows stream through HBM in whole-line order with nontemporal loads and
//     stores and are transposed to and from the MFMA layout in a per-wave LDS
//     tile.
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
//   V operand (one 16-byte read of a V row per tile and k-step) is loaded once
//   per task with that same column map.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <utility>

#include "kamera_desc.h"

namespace kamera {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Every buffer the kernels read or write lives in device global memory, but a pointer
// read out of the packed batch is a generic pointer, and accesses through it compile to
// FLAT instructions. Those count in the LDS counter as well as the vector-memory one, so
// each wait for an LDS result of the transposes would also wait for the row stores still
// in flight (a tile's four stores would go out one at a time). Cast once to the global
// address space, the accesses compile to global_* instructions, which only the
// vector-memory counter tracks (measured: 28-layer GQA batch 172.6 -> 171.1 us, 32-layer
// MHA reorder batch 8137 -> 8097 us).
#define KGLOBAL __attribute__((address_space(1)))
template <typename T>
__device__ __forceinline__ KGLOBAL T* as_global(T* p) {
  return (KGLOBAL T*)p;
}

// 16 zero bytes in global memory: operand reads of lanes with no data point here.
static __device__ __align__(16) const uint32_t kZeroBlock[4] = {0u, 0u, 0u, 0u};
__device__ __forceinline__ const KGLOBAL uint16_t* zero_block() { return (const KGLOBAL uint16_t*)kZeroBlock; }

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

// theta_i = base^(-2i/d_rot) in fp64.
__device__ __forceinline__ double theta_fp64(double base, int d_rot, int i) {
  return pow(base, (-2.0 * (double)i) / (double)d_rot);
}

// cos/sin of p * theta, the angle formed and evaluated in fp64, then rounded once to fp32.
__device__ __forceinline__ void phase_at(double th, int64_t p, float& c, float& s) {
  const double phi = (double)p * th;
  double sd, cd;
  sincos(phi, &sd, &cd);
  c = (float)cd;
  s = (float)sd;
}

// cos/sin of delta * theta_i (the per-chunk phase).
__device__ __forceinline__ void phase_fp64(double base, int d_rot, int64_t delta, int i, float& c,
                                           float& s) {
  phase_at(theta_fp64(base, d_rot, i), delta, c, s);
}

// Rotary pair (index into the band's d_rot/2 pairs) of coefficient slot j of a lane
// (lg = lane >> 4) in the MFMA layout; slots 2k and 2k+1 are always neighbouring pairs.
__device__ __forceinline__ int lane_pair(int rot, int j, int lg) {
  if (rot == ROT_NEOX_SLABS) return 32 * (j >> 3) + 8 * lg + (j & 7);   // slab-0 element j
  if (rot == ROT_NEOX_RUNS) return 8 * lg + (j & 7);                    // run-0 element j
  const int e2 = 2 * j, s = e2 >> 4, r = (e2 >> 3) & 1, e = e2 & 7;     // GPT-J pair (2j, 2j+1)
  return (64 * s + 32 * r + 8 * lg + e) >> 1;
}

// Rotation mode of a layout's rotary band in the MFMA path.
__device__ __forceinline__ int band_rot(const DevHeader& hd) {
  return hd.pairing == 1 ? ROT_GPTJ : (hd.d_rot == 128 ? ROT_NEOX_SLABS : ROT_NEOX_RUNS);
}

// Float offset of (cos, sin) of pair i of token t in a chunk's per-token table.
// Bands of 64 or 128 columns (every MFMA layout) store the table tile-major in the
// MFMA lane order: tile t/16 is a block of 16 * d_rot floats holding, for each
// coefficient step k (two neighbouring pairs, lane_pair(2k)) and lane group lg, the
// 16 tokens' (cos, sin, cos, sin) as 16 bytes each, so the wave instruction that
// loads step k of a tile reads 1 KB of consecutive bytes. Other widths (generic
// kernel only) store [token][pair].
__device__ __forceinline__ int64_t phase_offset(const DevHeader& hd, int64_t t, int i) {
  if (hd.d_rot != 64 && hd.d_rot != 128) return (t * (hd.d_rot >> 1) + i) * 2;
  int k, lg;
  const int rot = band_rot(hd);
  if (rot == ROT_NEOX_SLABS) {        // i = 32 (k >> 2) + 8 lg + 2 (k & 3) + half
    lg = (i >> 3) & 3;
    k = 4 * (i >> 5) + ((i & 7) >> 1);
  } else if (rot == ROT_NEOX_RUNS) {  // i = 8 lg + 2 k + half
    lg = i >> 3;
    k = (i & 7) >> 1;
  } else {                            // i = 32 (k >> 2) + 16 ((k >> 1) & 1) + 4 lg + 2 (k & 1) + half
    lg = (i >> 2) & 3;
    k = 4 * (i >> 5) + 2 * ((i >> 4) & 1) + ((i >> 1) & 1);
  }
  return (t >> 4) * 16 * hd.d_rot + ((k * 4 + lg) * 16 + (t & 15)) * 4 + 2 * (i & 1);
}

template <typename C>  // the chunk record: DevChunk, or DevChunkInline for batches passed by value
__device__ __forceinline__ int find_chunk(const C* __restrict__ chunks, int n, int64_t task) {
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (chunks[mid].task0 <= task) lo = mid; else hi = mid - 1;
  }
  return lo;
}

struct TaskCoord {
  int chunk, layer, stream, tb, g;
};

// (chunk, layer, stream, token block, group) of a task:
//   chunk-major:  task = task0 + ((stream * L + layer) * ntb + tb) * ngroups + g
//   layer-major:  task = layer * layer_tasks + task0 + (stream * ntb + tb) * ngroups + g
template <typename C>
__device__ __forceinline__ TaskCoord decode_task(const DevHeader& hd, const C* __restrict__ chunks, int64_t task) {
  TaskCoord tc;
  int64_t r;
  if (hd.layer_tasks > 0) {
    tc.layer = (int)(task / hd.layer_tasks);
    const int64_t in_layer = task - (int64_t)tc.layer * hd.layer_tasks;
    tc.chunk = find_chunk(chunks, hd.nchunks, in_layer);
    const C& ch = chunks[tc.chunk];
    r = in_layer - ch.task0;
    tc.g = ch.group0 + (int)(r % ch.ngroups);
    r /= ch.ngroups;
    tc.tb = (int)(r % ch.ntb);
    tc.stream = (int)(r / ch.ntb);
    return tc;
  }
  tc.chunk = find_chunk(chunks, hd.nchunks, task);
  const C& ch = chunks[tc.chunk];
  r = task - ch.task0;
  tc.g = ch.group0 + (int)(r % ch.ngroups);
  r /= ch.ngroups;
  tc.tb = (int)(r % ch.ntb);
  r /= ch.ntb;
  tc.layer = (int)(r % hd.L);
  tc.stream = (int)(r / hd.L);
  return tc;
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
// A wave task is (chunk, tensor, layer, token block, column group). Rows move
// between HBM and registers in "line" layout: a load or store instruction covers
// whole rows of the group (4 rows x 256 B for a 128-column group), so every
// 128-byte line is touched by one instruction and the stream can bypass the
// caches (nontemporal). A per-wave LDS tile (rows padded by 16 B so both
// layouts are bank-conflict free) turns line layout into the MFMA layout and
// back. V operands and cos/sin stay in registers for the whole task.

__device__ __forceinline__ void wave_lds_fence() {
  // LDS traffic of one wave is processed in order; this only stops the compiler
  // from moving LDS accesses across the hand-off between the two layouts.
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int NSLAB>
struct Geo {
  static constexpr int GC = 64 * NSLAB;        // columns per group
  static constexpr int CPR = GC / 8;           // 16-byte chunks per row
  static constexpr int RPI = 64 / CPR;         // rows per line-layout instruction
  static constexpr int NI = 16 / RPI;          // line-layout instructions per tile (= 2 * NSLAB)
  static constexpr int RS = 2 * GC + 16;       // LDS row stride in bytes
  static constexpr int LDS = 16 * RS;          // bytes per wave
};

// VALU form of the patch (the alternative to the MFMA contraction, for 128-wide heads): lane
// (lg, c) holds token c's 16 * NSLAB columns x[k] (the MFMA layout), its own U pairs uw[jp] =
// U[c][2jp, 2jp+1], and for each of its columns the V pair of rank pair c, vv[k] = V[col][2c,
// 2c+1] as bf16x2. A row broadcast (DPP row_newbcast:jp) hands every lane of the row lane jp's
// V pair, and v_dot2c_f32_bf16 adds both products to the fp32 value: 2 instructions per pair
// and column, 1024 per tile at rank 32.
template <int NSLAB, int JP>
__device__ __forceinline__ void valu_pair(float* x, const uint32_t* vv, uint32_t u2) {
  const bf16x2 u = __builtin_bit_cast(bf16x2, u2);
#pragma unroll
  for (int k = 0; k < NSLAB * 16; ++k) {
    const int b = __builtin_amdgcn_mov_dpp((int)vv[k], 0x150 + JP, 0xf, 0xf, true);
    x[k] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, b), u, x[k], false);
  }
}
template <int NSLAB, int... JP>
__device__ __forceinline__ void valu_patch(float* x, const uint32_t* vv, const uint32_t* uw, int npairs,
                                           std::integer_sequence<int, JP...>) {
  ((JP < npairs ? valu_pair<NSLAB, JP>(x, vv, uw[JP]) : void()), ...);
}

template <int NSLAB, int NK, bool POS, bool VALU, typename C>
__device__ __forceinline__ void mfma_task(const DevHeader& hd, const C& ch, int layer, int tensor,
                                          int colbase, int tok0, int ntiles, int rot, const int* kfac,
                                          const int* kstep, int lane, unsigned char* lds) {
  using G = Geo<NSLAB>;
  const int lg = lane >> 4;
  const int c = lane & 15;
  const int lrow = lane / G::CPR;   // line layout: row inside an instruction's rows
  const int lchunk = lane % G::CPR; // line layout: 16-byte chunk of the row
  const bool in_place = (ch.flags & 2u) != 0;
  const int P = hd.page_size, F = hd.F, T = ch.T;
  const KGLOBAL int32_t* pages = as_global(ch.pages);
  const KGLOBAL uint16_t* src =
      as_global((const uint16_t*)ch.src[tensor]) + (int64_t)layer * ch.src_ls + colbase + 8 * lchunk;
  KGLOBAL uint16_t* dst = as_global((uint16_t*)ch.dst[tensor]) + (int64_t)layer * ch.dst_ls + colbase + 8 * lchunk;

  // Pool pages. The task's page ids (at most 64) are read once, lane i holding the
  // i-th; with pages of >= 16 slots a 16-token tile spans at most two of them, which
  // v_readlane extracts at a uniform index, so no memory read sits on the row
  // address path. Other page sizes read the table once per row.
  const int pshift = hd.page_shift;
  int pg_base = 0, pg_last = 0, pg_reg = 0;
  bool two_pages = false;
  if (pages != nullptr) {
    const int s_first = ch.slot0 + tok0, s_end = ch.slot0 + min(tok0 + ch.tb_tokens, T) - 1;
    pg_base = pshift >= 0 ? s_first >> pshift : s_first / P;
    pg_last = pshift >= 0 ? s_end >> pshift : s_end / P;
    two_pages = P >= kTileTokens && pg_last - pg_base < 64;
    if (two_pages && lane <= pg_last - pg_base) pg_reg = pages[pg_base + lane];
  }
  auto page_row = [&](int tt, int t) -> int64_t {  // element offset of token t's row (tile starting at tt)
    const int s = ch.slot0 + t;
    const int pi = pshift >= 0 ? s >> pshift : s / P;
    const int off = pshift >= 0 ? s & (P - 1) : s - pi * P;
    int pg;
    if (two_pages) {
      const int s0 = ch.slot0 + tt;
      const int pi0 = pshift >= 0 ? s0 >> pshift : s0 / P;
      const int pg0 = __builtin_amdgcn_readlane(pg_reg, pi0 - pg_base);
      const int pg1 = __builtin_amdgcn_readlane(pg_reg, min(pi0 + 1, pg_last) - pg_base);
      pg = pi == pi0 ? pg0 : pg1;
    } else {
      pg = pages[pi];
    }
    return ((int64_t)pg * P + off) * F;
  };
  // A tile whose 16 rows sit in one page (or in dense rows) is addressed from one
  // uniform base, like dense rows; only tiles that straddle pages take page_row.
  auto tile_base = [&](bool paged, int tt, int64_t& base) -> bool {
    if (!paged) {
      base = (int64_t)tt * F;
      return true;
    }
    if (!two_pages) return false;
    const int s0 = ch.slot0 + tt;
    const int pi0 = pshift >= 0 ? s0 >> pshift : s0 / P;
    const int off0 = s0 - pi0 * P;
    if (off0 + kTileTokens > P) return false;
    base = ((int64_t)__builtin_amdgcn_readlane(pg_reg, pi0 - pg_base) * P + off0) * F;
    return true;
  };

  // The first tile's rows are requested before the per-task set-up (phase, V operands),
  // so the set-up runs while they are in flight (tasks without prefetch, below, excepted).
  u32x4 cur[G::NI], nxt[G::NI], nxt2[G::NI];
  // Tasks without k-steps (rotation or copy only, e.g. sliding-window survivors) hold no V
  // operands or U rows, so they keep a second tile in flight ahead of the current one
  // without raising the kernel's register peak (survivors +1.4% measured).
  constexpr bool kDeep = NK == 0;
  // One-slab tasks with two k-steps (the MLA rope band under the row factor and the band
  // factor) request each tile's rows and U rows at the top of that tile, not one tile ahead:
  // the 16 registers saved put the whole instantiation at <= 128 VGPRs, 4 waves per SIMD
  // for every task of the batch instead of 3 (27-layer MLA batch 195.5 -> 194.8 us; with
  // per-token offsets 201.1 -> 199.9 us).
  constexpr bool kNoPf = NSLAB == 1 && NK == 2;
  auto load_rows = [&](int tile, u32x4 (&raw)[G::NI]) {
    // Rows past the chunk end load the last row instead (computed, never stored), so
    // no loaded value is merged with a default and the loads stay in flight.
    const int tt = tok0 + tile * kTileTokens;
    int64_t base;
    if (tile_base(in_place && pages, tt, base)) {
#pragma unroll
      for (int i = 0; i < G::NI; ++i) {
        const int t = min(tt + i * G::RPI + lrow, T - 1);
        raw[i] = __builtin_nontemporal_load((const KGLOBAL u32x4*)(src + base + (int64_t)(t - tt) * F));
      }
    } else {
#pragma unroll
      for (int i = 0; i < G::NI; ++i) {
        const int t = min(tt + i * G::RPI + lrow, T - 1);
        raw[i] = __builtin_nontemporal_load((const KGLOBAL u32x4*)(src + page_row(tt, t)));
      }
    }
  };
  if (!kNoPf) load_rows(0, cur);
  if (kDeep && ntiles > 1) load_rows(1, nxt);

  // ---- rotation coefficients for the pairs this lane holds (MFMA layout): one set per
  // chunk (delta), or, for chunks with per-token offsets, the set of this lane's token,
  // read from the batch's cos/sin table for every tile. Where the next tile's rows are
  // prefetched and registers allow (one slab, or one k-step) the next tile's set is loaded
  // with them; otherwise at the top of its own tile.
  const bool tok_phase = POS && rot != ROT_NONE && (ch.flags & 4u) != 0;
  constexpr bool kPrefetchPhase = !kNoPf && (NSLAB == 1 || NK <= 1);
  float cs[NSLAB * 8], sn[NSLAB * 8], pcs[NSLAB * 8], psn[NSLAB * 8];
  auto load_phase = [&](int tile, float (&c_)[NSLAB * 8], float (&s_)[NSLAB * 8]) {
    if constexpr (POS) {  // tile-major table (phase_offset): step k of the tile is 1 KB
      const KGLOBAL float* blk = as_global(ch.phase) + (int64_t)((tok0 >> 4) + tile) * 16 * hd.d_rot + 4 * lane;
#pragma unroll
      for (int k = 0; k < NSLAB * 4; ++k) {
        const f32x4 v = *(const KGLOBAL f32x4*)(blk + 256 * k);
        c_[2 * k] = v[0];
        s_[2 * k] = v[1];
        c_[2 * k + 1] = v[2];
        s_[2 * k + 1] = v[3];
      }
    }
  };
  if (tok_phase) {
    load_phase(0, cs, sn);
  } else if (rot != ROT_NONE) {
    float cl = 1.f, sl = 0.f;
    if (lane < (hd.d_rot >> 1)) phase_fp64(hd.rope_base, hd.d_rot, ch.delta, lane, cl, sl);
#pragma unroll
    for (int j = 0; j < NSLAB * 8; ++j) {
      const int p = lane_pair(rot, j, lg);
      cs[j] = __shfl(cl, p, 64);
      sn[j] = __shfl(sl, p, 64);
    }
  }

  // ---- V operands: A[M][k] = V[col(M)][k] for every slab, tile and k-step
  bf16x8 av[(NK > 0 && !VALU) ? NSLAB * 4 * NK : 1];
  const KGLOBAL uint16_t* ubase[NK > 0 ? NK : 1];
  int urank[NK > 0 ? NK : 1], ustride[NK > 0 ? NK : 1];
  bool uvec[NK > 0 ? NK : 1];
  // VALU form: V pairs, U rows of 32 coefficients per k-step, and the pairs inside the rank
  uint32_t vv[(VALU && NK > 0) ? NK * NSLAB * 16 : 1];
  const KGLOBAL uint16_t* uvbase[(VALU && NK > 0) ? NK : 1];
  int uvrem[(VALU && NK > 0) ? NK : 1], vpairs[(VALU && NK > 0) ? NK : 1];
  if constexpr (VALU) {
#pragma unroll
    for (int j = 0; j < NK; ++j) {
      const DevFactor& f = ch.fac[kfac[j]];
      const int64_t lrel = layer - f.layer0;
      const KGLOBAL uint16_t* vf = as_global((const uint16_t*)f.v) + lrel * f.width * f.rank;
      uvec[j] = f.uvec != 0;
      uvrem[j] = f.rank - 32 * kstep[j];
      vpairs[j] = min(16, (uvrem[j] + 1) >> 1);
      uvbase[j] = as_global((const uint16_t*)f.u) + lrel * T * f.rank + 32 * kstep[j];
      ustride[j] = f.rank;
      const int k0 = 32 * kstep[j] + 2 * c;   // this lane's rank pair
#pragma unroll
      for (int s = 0; s < NSLAB; ++s)
#pragma unroll
        for (int r = 0; r < 2; ++r)
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int rel = colbase + 64 * s + 32 * r + 8 * lg + e - f.col0;
            const bool in = rel >= 0 && rel < f.width && k0 < f.rank;
            uint32_t w = 0;
            if (in) {
              const KGLOBAL uint16_t* p = vf + (int64_t)rel * f.rank + k0;
              if (f.vvec) w = *(const KGLOBAL uint32_t*)p;   // rank % 8 == 0: the pair is whole and aligned
              else w = (uint32_t)p[0] | (k0 + 1 < f.rank ? (uint32_t)p[1] << 16 : 0u);
            }
            vv[j * NSLAB * 16 + 16 * s + 8 * r + e] = w;
          }
    }
  }
#pragma unroll
  for (int j = 0; j < (VALU ? 0 : NK); ++j) {
    const DevFactor& f = ch.fac[kfac[j]];
    const int64_t lrel = layer - f.layer0;
    const KGLOBAL uint16_t* vf = as_global((const uint16_t*)f.v) + lrel * f.width * f.rank;
    uvec[j] = f.uvec != 0;
    urank[j] = f.rank - 32 * kstep[j] - 8 * lg;
    // Vector mode (rank a multiple of 8): every lane reads a whole 16-byte slice;
    // lanes past the rank read the header's zero block (stride 0).
    const bool upast = uvec[j] && urank[j] <= 0;
    ustride[j] = upast ? 0 : f.rank;
    ubase[j] = upast ? zero_block() : as_global((const uint16_t*)f.u) + lrel * T * f.rank + 32 * kstep[j] + 8 * lg;
    const int mrow = lane & 15, kg = lane >> 4;
    const int k0 = 32 * kstep[j] + 8 * kg;   // first k of this lane's 8
#pragma unroll
    for (int s = 0; s < NSLAB; ++s)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int col = colbase + 64 * s + 32 * (q >> 1) + 8 * (mrow >> 2) + 4 * (q & 1) + (mrow & 3);
        const int rel = col - f.col0;
        const bool in = rel >= 0 && rel < f.width;
        bf16x8 a;
        if (f.vvec) {  // uniform: whole slices, or the zero block outside the factor
          a = *(const KGLOBAL bf16x8*)((in && k0 < f.rank) ? vf + (int64_t)rel * f.rank + k0 : zero_block());
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const uint16_t h = (in && k0 + e < f.rank) ? vf[(int64_t)rel * f.rank + k0 + e] : (uint16_t)0;
            a[e] = __builtin_bit_cast(__bf16, h);
          }
        }
        av[(s * 4 + q) * NK + j] = a;
      }
  }

  const bool compute = (rot != ROT_NONE) || (NK > 0);

  bf16x8 ucur[NK > 0 ? NK : 1], unxt[NK > 0 ? NK : 1];
  auto load_u = [&](int tile, bf16x8 (&ub)[NK > 0 ? NK : 1]) {  // U rows of the tile's tokens
    const int tt = tok0 + tile * kTileTokens;
    const int t = min(tt + c, T - 1);
#pragma unroll
    for (int j = 0; j < NK; ++j) {
      bf16x8 b;
      if (uvec[j]) {
        b = *(const KGLOBAL bf16x8*)(ubase[j] + (int64_t)t * ustride[j]);
      } else {  // ranks that are not a multiple of 8: element reads, zero past the rank
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint16_t h = e < urank[j] ? ubase[j][(int64_t)t * ustride[j] + e] : (uint16_t)0;
          b[e] = __builtin_bit_cast(__bf16, h);
        }
      }
      ub[j] = b;
    }
  };


  // VALU form: token c's 32 coefficients of each k-step as 16 bf16x2 words, zero past the rank
  uint32_t uw[(VALU && NK > 0) ? NK * 16 : 1];
  auto load_uw = [&](int tile) {
    const int t = min(tok0 + tile * kTileTokens + c, T - 1);
#pragma unroll
    for (int j = 0; j < NK; ++j) {
      const KGLOBAL uint16_t* p = uvbase[j] + (int64_t)t * ustride[j];
      if (uvec[j]) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const u32x4 w = 8 * q < uvrem[j] ? *(const KGLOBAL u32x4*)(p + 8 * q) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
          for (int i = 0; i < 4; ++i) uw[j * 16 + 4 * q + i] = w[i];
        }
      } else {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const uint32_t lo = 2 * e < uvrem[j] ? (uint32_t)p[2 * e] : 0u;
          const uint32_t hi = 2 * e + 1 < uvrem[j] ? (uint32_t)p[2 * e + 1] << 16 : 0u;
          uw[j * 16 + e] = lo | hi;
        }
      }
    }
  };

  if (!kNoPf && !VALU) load_u(0, ucur);
  for (int tile = 0; tile < ntiles; ++tile) {
    if constexpr (VALU) load_uw(tile);
    if (kNoPf) {
      load_rows(tile, cur);
      load_u(tile, ucur);
    } else if (kDeep) {
      if (tile + 2 < ntiles) load_rows(tile + 2, nxt2);
      if (kPrefetchPhase && tok_phase && tile + 1 < ntiles) load_phase(tile + 1, pcs, psn);
    } else if (tile + 1 < ntiles) {
      load_rows(tile + 1, nxt);
      if constexpr (!VALU) load_u(tile + 1, unxt);
      if (kPrefetchPhase && tok_phase) load_phase(tile + 1, pcs, psn);
    }
    if (!kPrefetchPhase && tok_phase && tile > 0) load_phase(tile, cs, sn);
    const int tt = tok0 + tile * kTileTokens;
    u32x4 out[G::NI];
    if (!compute) {
#pragma unroll
      for (int i = 0; i < G::NI; ++i) out[i] = cur[i];  // line layout in, line layout out
    } else {
      // line layout -> LDS -> MFMA layout (lane (lg, c): row c, chunks 8s + 4r + lg)
#pragma unroll
      for (int i = 0; i < G::NI; ++i)
        *(u32x4*)(lds + (i * G::RPI + lrow) * G::RS + 16 * lchunk) = cur[i];
      wave_lds_fence();
      u32x4 m[NSLAB][2];
#pragma unroll
      for (int s = 0; s < NSLAB; ++s)
#pragma unroll
        for (int r = 0; r < 2; ++r) m[s][r] = *(const u32x4*)(lds + c * G::RS + 16 * (8 * s + 4 * r + lg));
      float x[NSLAB * 16];
#pragma unroll
      for (int s = 0; s < NSLAB; ++s)
#pragma unroll
        for (int r = 0; r < 2; ++r)
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            x[16 * s + 8 * r + 2 * w] = bf_lo(m[s][r][w]);
            x[16 * s + 8 * r + 2 * w + 1] = bf_hi(m[s][r][w]);
          }
      if (NSLAB == 2 && rot == ROT_NEOX_SLABS) {  // pair (i, i + 64): slabs 0 and 1, same position
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const float a = x[j], b = x[(NSLAB - 1) * 16 + j];
          x[j] = fmaf(a, cs[j], -(b * sn[j]));
          x[(NSLAB - 1) * 16 + j] = fmaf(a, sn[j], b * cs[j]);
        }
      } else if (rot == ROT_NEOX_RUNS) {          // pair (i, i + 32): runs 0 and 1 of slab 0
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float a = x[j], b = x[8 + j];
          x[j] = fmaf(a, cs[j], -(b * sn[j]));
          x[8 + j] = fmaf(a, sn[j], b * cs[j]);
        }
      } else if (rot == ROT_GPTJ) {               // pair (2i, 2i + 1): neighbours in a run
#pragma unroll
        for (int j = 0; j < NSLAB * 8; ++j) {
          const float a = x[2 * j], b = x[2 * j + 1];
          x[2 * j] = fmaf(a, cs[j], -(b * sn[j]));
          x[2 * j + 1] = fmaf(a, sn[j], b * cs[j]);
        }
      }
      if constexpr (NK > 0 && VALU) {
#pragma unroll
        for (int j = 0; j < NK; ++j)
          valu_patch<NSLAB>(x, vv + j * NSLAB * 16, uw + j * 16, vpairs[j], std::make_integer_sequence<int, 16>{});
      } else if constexpr (NK > 0) {
#pragma unroll
        for (int set = 0; set < NSLAB * 4; ++set) {
          f32x4 acc = {x[4 * set], x[4 * set + 1], x[4 * set + 2], x[4 * set + 3]};
#pragma unroll
          for (int j = 0; j < NK; ++j)
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[set * NK + j], ucur[j], acc, 0, 0, 0);
          x[4 * set] = acc[0];
          x[4 * set + 1] = acc[1];
          x[4 * set + 2] = acc[2];
          x[4 * set + 3] = acc[3];
        }
      }
      // MFMA layout -> LDS -> line layout
#pragma unroll
      for (int s = 0; s < NSLAB; ++s)
#pragma unroll
        for (int r = 0; r < 2; ++r) {
          u32x4 o;
#pragma unroll
          for (int w = 0; w < 4; ++w) o[w] = pack2(x[16 * s + 8 * r + 2 * w], x[16 * s + 8 * r + 2 * w + 1]);
          *(u32x4*)(lds + c * G::RS + 16 * (8 * s + 4 * r + lg)) = o;
        }
      wave_lds_fence();
#pragma unroll
      for (int i = 0; i < G::NI; ++i) out[i] = *(const u32x4*)(lds + (i * G::RPI + lrow) * G::RS + 16 * lchunk);
      wave_lds_fence();
    }
    int64_t obase;
    if (tile_base(pages != nullptr, tt, obase)) {
#pragma unroll
      for (int i = 0; i < G::NI; ++i) {
        const int t = tt + i * G::RPI + lrow;
        if (t < T) __builtin_nontemporal_store(out[i], (KGLOBAL u32x4*)(dst + obase + (int64_t)(t - tt) * F));
      }
    } else {
#pragma unroll
      for (int i = 0; i < G::NI; ++i) {
        const int t = tt + i * G::RPI + lrow;
        if (t < T) __builtin_nontemporal_store(out[i], (KGLOBAL u32x4*)(dst + page_row(tt, t)));
      }
    }
    if (!kNoPf && tile + 1 < ntiles) {
#pragma unroll
      for (int i = 0; i < G::NI; ++i) cur[i] = nxt[i];
      if (kDeep) {
#pragma unroll
        for (int i = 0; i < G::NI; ++i) nxt[i] = nxt2[i];
      }
      if constexpr (!VALU) {
#pragma unroll
        for (int j = 0; j < NK; ++j) ucur[j] = unxt[j];
      }
      if (kPrefetchPhase && tok_phase) {
#pragma unroll
        for (int j = 0; j < NSLAB * 8; ++j) {
          cs[j] = pcs[j];
          sn[j] = psn[j];
        }
      }
    }
  }
}

template <int NSLAB, int NKMAX, bool POS, bool VALU, typename C>
__device__ __forceinline__ void mfma_dispatch(int nk, const DevHeader& hd, const C& ch, int layer,
                                              int tensor, int colbase, int tok0, int ntiles, int rot,
                                              const int* kfac, const int* kstep, int lane, unsigned char* lds) {
#define KAMERA_NK_CASE(N)                                                                                      \
  case N:                                                                                                     \
    if constexpr (N <= NKMAX)                                                                                 \
      mfma_task<NSLAB, N, POS, VALU, C>(hd, ch, layer, tensor, colbase, tok0, ntiles, rot, kfac, kstep, lane, \
                                        lds);                                                                 \
    break;
  switch (nk) {
    KAMERA_NK_CASE(0)
    KAMERA_NK_CASE(1)
    KAMERA_NK_CASE(2)
    KAMERA_NK_CASE(3)
    KAMERA_NK_CASE(4)
    KAMERA_NK_CASE(5)
    KAMERA_NK_CASE(6)
    KAMERA_NK_CASE(7)
    KAMERA_NK_CASE(8)
    default: break;
  }
#undef KAMERA_NK_CASE
}

template <int NSLAB, int NKMAX, bool POS, bool VALU, typename C>
__device__ __forceinline__ void rehydrate_mfma_body(const DevHeader* __restrict__ hdr, const C* __restrict__ chunks,
                                                    unsigned char* lds_all) {
  constexpr int kWaves = mfma_waves_per_block(NSLAB, NKMAX);
  const int lane = threadIdx.x & (kWaveSize - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const DevHeader& hd = *hdr;
  // Workgroups are dispatched to the 8 XCDs in turn (workgroup b to XCD b % 8).
  // For rows wider than one workgroup's heads, windows of 8*W workgroups are
  // remapped so that XCD x runs W consecutive logical workgroups: whole rows of a
  // token block, and the V operands they share, stay in one XCD's L2. Narrow rows
  // keep the plain order (W = 1), where neighbouring workgroups already stream
  // neighbouring rows. The map is a bijection; a partial last window is unchanged.
  int64_t blk = blockIdx.x;
  if (hd.xcd_window_log2 > 0) {
    const int wl = hd.xcd_window_log2;
    const int64_t win = (int64_t)8 << wl;
    const int64_t nfull = ((int64_t)gridDim.x >> (3 + wl)) << (3 + wl);
    if (blk < nfull) {
      const int64_t x = blk & 7, j = blk >> 3;
      blk = (j >> wl) * win + (x << wl) + (j & ((1 << wl) - 1));
    }
  }
  const int64_t task = blk * kWaves + wave;
  if (task >= hd.total_tasks) return;  // no workgroup barrier follows: waves are independent
  const TaskCoord tcd = decode_task(hd, chunks, task);
  const C& ch = chunks[tcd.chunk];
  const int g = tcd.g, tb = tcd.tb, layer = tcd.layer;
  const int tensor = ch.stream_tensor[tcd.stream];
  const int colbase = g * hd.group_cols;
  const int tok0 = tb * ch.tb_tokens;
  const int ntiles = (min(ch.tb_tokens, ch.T - tok0) + kTileTokens - 1) / kTileTokens;

  int rot = ROT_NONE;
  const bool band = hd.family == 0 ? (tensor == 0) : (g == hd.rope_group);
  const bool turns = ch.delta != 0 || (POS && (ch.flags & 4u) != 0);
  if (band && turns) rot = band_rot(hd);

  // 32-wide k-steps of the factors covering this group's columns
  int kfac[kMaxKSteps], kstep[kMaxKSteps];
  int nk = 0;
  if (ch.flags & 1u) {
    for (int f = 0; f < ch.nfac; ++f) {
      const DevFactor& fa = ch.fac[f];
      if (fa.tensor != tensor || fa.rank <= 0 || layer < fa.layer0) continue;
      if (fa.col0 >= colbase + hd.group_cols || fa.col0 + fa.width <= colbase) continue;
      for (int k = 0; k * 32 < fa.rank && nk < kMaxKSteps; ++k) {
        kfac[nk] = f;
        kstep[nk] = k;
        ++nk;
      }
    }
  }
  if ((ch.flags & 2u) && rot == ROT_NONE && nk == 0) return;  // in place and nothing changes
  mfma_dispatch<NSLAB, NKMAX, POS, VALU, C>(nk, hd, ch, layer, tensor, colbase, tok0, ntiles, rot, kfac, kstep, lane,
                              lds_all + wave * Geo<NSLAB>::LDS);
}

// The batch description read from the workspace (plans; paged or re-anchored batches;
// batches of more than kInlineChunks chunks or with chunks of more than two factors) ...
// VALU: the patch on the VALU (dot2 + row broadcasts) instead of the MFMA; 128-wide heads only.
template <int NSLAB, int NKMAX, bool POS, bool VALU>
__global__ __launch_bounds__((kWaveSize * mfma_waves_per_block(NSLAB, NKMAX))) void rehydrate_mfma(
    const DevHeader* __restrict__ hdr, const DevChunk* __restrict__ chunks) {
  __shared__ __attribute__((aligned(16))) unsigned char lds_all[mfma_waves_per_block(NSLAB, NKMAX) * Geo<NSLAB>::LDS];
  rehydrate_mfma_body<NSLAB, NKMAX, POS, VALU, DevChunk>(hdr, chunks, lds_all);
}

// ... or carried by the dispatch as the kernel's argument (small dense batches).
template <int NSLAB, int NKMAX, bool POS, bool VALU>
__global__ __launch_bounds__((kWaveSize * mfma_waves_per_block(NSLAB, NKMAX))) void rehydrate_mfma_inline(
    const InlineBatch batch) {
  __shared__ __attribute__((aligned(16))) unsigned char lds_all[mfma_waves_per_block(NSLAB, NKMAX) * Geo<NSLAB>::LDS];
  rehydrate_mfma_body<NSLAB, NKMAX, POS, VALU, DevChunkInline>(&batch.hd, batch.ch, lds_all);
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

template <typename T, typename C>
__device__ __forceinline__ float add_patch(const C& ch, int layer, int tensor, int t, int col, float acc) {
  for (int fi = 0; fi < ch.nfac; ++fi) {
    const DevFactor& f = ch.fac[fi];
    if (f.tensor != tensor || layer < f.layer0 || col < f.col0 || col >= f.col0 + f.width) continue;
    const int64_t lrel = layer - f.layer0;
    const int64_t ub = lrel * ch.T * f.rank + (int64_t)t * f.rank;
    const int64_t vb = lrel * f.width * f.rank + (int64_t)(col - f.col0) * f.rank;
    for (int j = 0; j < f.rank; ++j) acc = fmaf(ld<T>(f.u, ub + j), ld<T>(f.v, vb + j), acc);
  }
  return acc;
}

template <typename T, typename C>
__device__ __forceinline__ void rehydrate_generic_body(const DevHeader* __restrict__ hdr, const C* __restrict__ chunks,
                                                       float2* tab) {
  const DevHeader& hd = *hdr;
  const int64_t task = blockIdx.x;
  if (task >= hd.total_tasks) return;  // uniform over the block
  const TaskCoord tcd = decode_task(hd, chunks, task);
  const C& ch = chunks[tcd.chunk];
  const int tb = tcd.tb, layer = tcd.layer;
  const int tensor = ch.stream_tensor[tcd.stream];
  const bool in_place = (ch.flags & 2u) != 0;
  const bool patch = (ch.flags & 1u) != 0;
  const bool tok_phase = tensor == 0 && (ch.flags & 4u) != 0;  // per-token offsets: cos/sin table
  const bool rotate = tensor == 0 && (ch.delta != 0 || tok_phase);
  const int npairs = hd.d_rot >> 1;
  if (rotate && !tok_phase)
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
        const float2 cs = tok_phase ? *(const float2*)(ch.phase + phase_offset(hd, t, i)) : tab[i];
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

template <typename T>
__global__ __launch_bounds__(kBlockThreads) void rehydrate_generic(const DevHeader* __restrict__ hdr,
                                                                   const DevChunk* __restrict__ chunks) {
  __shared__ float2 tab[256];
  rehydrate_generic_body<T>(hdr, chunks, tab);
}

template <typename T>
__global__ __launch_bounds__(kBlockThreads) void rehydrate_generic_inline(const InlineBatch batch) {
  __shared__ float2 tab[256];
  rehydrate_generic_body<T>(&batch.hd, batch.ch, tab);
}

// ============================================================================
// Per-token cos/sin table of chunks with position offsets (QV-PIC Eq. 2: M-RoPE
// applied with each token's own (t, h, w) position). Entry (t, i) of a chunk's
// table holds cos/sin of positions[t][section(i)] * theta_i, the angle formed and
// evaluated in fp64 like the per-chunk phase, rounded once to fp32. Pairs are
// assigned to the t, h, w components in blocks of mrope[0], mrope[1], mrope[2]
// pairs; all zero means every pair follows component t (1-D RoPE).
// ============================================================================
template <typename C>
__device__ __forceinline__ void phase_table_body(const DevHeader* __restrict__ hdr, const C* __restrict__ chunks,
                                                 double* theta) {
  const DevHeader& hd = *hdr;
  const int blocks_per_chunk = hd.phase_blocks;
  // workgroup b covers entries [256 (b % blocks_per_chunk), ...) of chunk b / blocks_per_chunk
  const C& ch = chunks[blockIdx.x / blocks_per_chunk];
  const int np = hd.d_rot >> 1;
  const int64_t n_entries = ch.phase ? (int64_t)((ch.T + kTileTokens - 1) / kTileTokens) * kTileTokens * np : 0;
  const int64_t e = (int64_t)(blockIdx.x % blocks_per_chunk) * kBlockThreads + threadIdx.x;
  if (e - threadIdx.x >= n_entries) return;  // uniform over the workgroup, before its barrier
  for (int i = threadIdx.x; i < np; i += kBlockThreads) theta[i] = theta_fp64(hd.rope_base, hd.d_rot, i);
  __syncthreads();
  if (e >= n_entries) return;
  const int64_t t = e / np;             // token of the padded tile range; past T: a copy of T-1
  const int i = (int)(e - t * np);
  int comp = 0;
  if (hd.mrope[0] | hd.mrope[1] | hd.mrope[2]) comp = i < hd.mrope[0] ? 0 : (i < hd.mrope[0] + hd.mrope[1] ? 1 : 2);
  float c, s;
  phase_at(theta[i], (int64_t)ch.positions[min(t, (int64_t)ch.T - 1) * 3 + comp], c, s);
  *(float2*)(ch.phase + phase_offset(hd, t, i)) = make_float2(c, s);
}

__global__ __launch_bounds__(kBlockThreads) void phase_table(const DevHeader* __restrict__ hdr,
                                                             const DevChunk* __restrict__ chunks) {
  __shared__ double theta[256];   // theta_i of the band's d_rot/2 <= 256 pairs, once per workgroup
  phase_table_body(hdr, chunks, theta);
}

__global__ __launch_bounds__(kBlockThreads) void phase_table_inline(const InlineBatch batch) {
  __shared__ double theta[256];
  phase_table_body(&batch.hd, batch.ch, theta);
}

// ============================================================================
// Descriptor copy-in: packed batch from mapped pinned host memory to the workspace
// ============================================================================
__global__ __launch_bounds__(kBlockThreads) void copy_in(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                         int64_t n16) {
  const int64_t i = (int64_t)blockIdx.x * kBlockThreads + threadIdx.x;
  if (i < n16) dst[i] = src[i];
}

// ============================================================================
// Scratch of the allocation-free entry point (kamera_rehydrate_batched_noalloc)
// ============================================================================
// Stands in for the caller's workspace: packed batch (header, chunk records, block
// tables) and the per-token cos/sin tables of re-anchored chunks. Each GPU the library
// runs on holds its own copy until the process ends. Every call on a device uses it from
// offset 0, so calls that overlap in time on one device race; calls on one stream are
// ordered. Nothing in it has to start at zero: a call writes every byte the kernels read
// (the whole packed region, and every entry of every table it reads).
static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

// Device address of this device's copy of `scratch`, looked up once per device with that
// device current. (In host code the array's own name is a host-side stand-in, never a
// device address: only this address may reach a kernel or a copy.)
constexpr int kScratchDevices = 64;
hipError_t scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kScratchDevices) return hipErrorInvalidDevice;
  static std::mutex mu;
  static void* addr[kScratchDevices];
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *out = addr[dev];
  return hipSuccess;
}

// Host bytes moved into device memory by the launch itself: the kernel's argument carries
// up to kFill16 16-byte words and one thread stores each, so no staging buffer, host
// allocation or copy engine is involved.
constexpr int kFill16 = 232;
struct FillArg {
  u32x4 data[kFill16];
  u32x4* dst;
  uint32_t n16;
  uint32_t pad;
};
static_assert(sizeof(FillArg) + 256 <= 4096, "kernel arguments are limited to 4 KB");
static_assert(kFill16 <= kBlockThreads, "one thread per word");

__global__ __launch_bounds__(kBlockThreads) void fill_by_argument(const FillArg a) {
  if (threadIdx.x < a.n16) a.dst[threadIdx.x] = a.data[threadIdx.x];
}

// `bytes` a multiple of 16; src host memory (read during the call), dst device memory
hipError_t launch_fill_by_argument(void* dst, const void* src, size_t bytes, hipStream_t stream) {
  FillArg a;
  memset(&a, 0, sizeof(a));
  for (size_t off = 0; off < bytes; off += (size_t)kFill16 * 16) {
    const size_t n = std::min(bytes - off, (size_t)kFill16 * 16);
    memcpy(a.data, (const unsigned char*)src + off, n);
    a.dst = (u32x4*)((unsigned char*)dst + off);
    a.n16 = (uint32_t)(n / 16);
    hipLaunchKernelGGL(fill_by_argument, dim3(1), dim3(kBlockThreads), 0, stream, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// ============================================================================
// Launchers
// ============================================================================
hipError_t launch_copy_in(void* dst, const void* src, size_t bytes, hipStream_t stream) {
  const int64_t n16 = (int64_t)(bytes / 16);  // packed batches are multiples of 256 bytes
  if (n16 <= 0) return hipSuccess;
  const int64_t blocks = (n16 + kBlockThreads - 1) / kBlockThreads;
  hipLaunchKernelGGL(copy_in, dim3((unsigned)blocks), dim3(kBlockThreads), 0, stream, (const u32x4*)src,
                     (u32x4*)dst, n16);
  return hipGetLastError();
}

// per_chunk: the header's phase_blocks (workgroups per chunk), set by the host
hipError_t launch_phase_table(const DevHeader* hdr, const DevChunk* chunks, int nchunks, int64_t per_chunk,
                              hipStream_t stream, const InlineBatch* inl) {
  if (per_chunk <= 0 || nchunks <= 0) return hipSuccess;
  if (per_chunk * nchunks > 0x7fffffffLL) return hipErrorInvalidValue;
  if (inl != nullptr)
    hipLaunchKernelGGL(phase_table_inline, dim3((unsigned)(per_chunk * nchunks)), dim3(kBlockThreads), 0, stream,
                       *inl);
  else
    hipLaunchKernelGGL(phase_table, dim3((unsigned)(per_chunk * nchunks)), dim3(kBlockThreads), 0, stream, hdr,
                       chunks);
  return hipGetLastError();
}

// `inl` non-null: the batch travels as the kernel argument (hdr and chunks unused)
template <int NSLAB, int NKMAX, bool POS = false, bool VALU = false>
static hipError_t launch_one(int64_t tasks, hipStream_t stream, const DevHeader* hdr, const DevChunk* chunks,
                             const InlineBatch* inl) {
  constexpr int w = mfma_waves_per_block(NSLAB, NKMAX);
  const int64_t blocks = (tasks + w - 1) / w;
  if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
  if (inl == nullptr) {
    hipLaunchKernelGGL((rehydrate_mfma<NSLAB, NKMAX, POS, VALU>), dim3((unsigned)blocks), dim3(kWaveSize * w), 0,
                       stream, hdr, chunks);
  } else {
    hipLaunchKernelGGL((rehydrate_mfma_inline<NSLAB, NKMAX, POS, VALU>), dim3((unsigned)blocks), dim3(kWaveSize * w),
                       0, stream, *inl);
  }
  return hipGetLastError();
}

hipError_t launch_mfma(int variant, const DevHeader* hdr, const DevChunk* chunks, int64_t tasks,
                       hipStream_t stream, const InlineBatch* inl) {
  if (tasks <= 0) return hipSuccess;
  switch (variant) {  // variant = (nslab - 1) * 4 + log2(nk_max)
    case 0: return launch_one<1, 1>(tasks, stream, hdr, chunks, inl);
    case 1: return launch_one<1, 2>(tasks, stream, hdr, chunks, inl);
    case 2: return launch_one<1, 4>(tasks, stream, hdr, chunks, inl);
    case 3: return launch_one<1, 8>(tasks, stream, hdr, chunks, inl);
    case 4: return launch_one<2, 1>(tasks, stream, hdr, chunks, inl);
    case 5: return launch_one<2, 2>(tasks, stream, hdr, chunks, inl);
    case 6: return launch_one<2, 4>(tasks, stream, hdr, chunks, inl);
    // batches with per-token offsets (kVariantPositions + the variant above)
    case 8: return launch_one<1, 1, true>(tasks, stream, hdr, chunks, inl);
    case 9: return launch_one<1, 2, true>(tasks, stream, hdr, chunks, inl);
    case 10: return launch_one<1, 4, true>(tasks, stream, hdr, chunks, inl);
    case 12: return launch_one<2, 1, true>(tasks, stream, hdr, chunks, inl);
    case 13: return launch_one<2, 2, true>(tasks, stream, hdr, chunks, inl);
    // the patch on the VALU (kVariantValu + the variant above; 128-wide heads, no per-token offsets)
    case 20: return launch_one<2, 1, false, true>(tasks, stream, hdr, chunks, inl);
    case 21: return launch_one<2, 2, false, true>(tasks, stream, hdr, chunks, inl);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_generic(int dtype, const DevHeader* hdr, const DevChunk* chunks, int64_t tasks,
                          hipStream_t stream, const InlineBatch* inl) {
  if (tasks <= 0) return hipSuccess;
  if (tasks > 0x7fffffffLL) return hipErrorInvalidValue;
  const dim3 grid((unsigned)tasks), block(kBlockThreads);
  if (inl != nullptr) {
    if (dtype == 0) hipLaunchKernelGGL(rehydrate_generic_inline<float>, grid, block, 0, stream, *inl);
    else hipLaunchKernelGGL(rehydrate_generic_inline<uint16_t>, grid, block, 0, stream, *inl);
  } else {
    if (dtype == 0) hipLaunchKernelGGL(rehydrate_generic<float>, grid, block, 0, stream, hdr, chunks);
    else hipLaunchKernelGGL(rehydrate_generic<uint16_t>, grid, block, 0, stream, hdr, chunks);
  }
  return hipGetLastError();
}

}  // namespace kamera
