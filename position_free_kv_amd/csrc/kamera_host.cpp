// Host side of the Kamera C ABI (include/kamera.h): argument validation, batch
// packing, the stream-ordered descriptor upload and kernel selection/launch.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "kamera.h"
#include "kamera_builder.h"
#include "kamera_desc.h"

namespace kamera {
hipError_t launch_mfma(int variant, const DevHeader* hdr, const DevChunk* chunks, int64_t tasks,
                       hipStream_t stream, const InlineBatch* inl);
hipError_t launch_generic(int dtype, const DevHeader* hdr, const DevChunk* chunks, int64_t tasks,
                          hipStream_t stream, const InlineBatch* inl);
hipError_t launch_copy_in(void* dst, const void* src, size_t bytes, hipStream_t stream);
hipError_t launch_phase_table(const DevHeader* hdr, const DevChunk* chunks, int nchunks, int64_t per_chunk,
                              hipStream_t stream, const InlineBatch* inl);
hipError_t scratch_address(void** out);
hipError_t launch_stream_probe(int kind, const void* src, void* dst, int64_t n16, uint32_t value, hipStream_t stream);
hipError_t launch_fill_by_argument(void* dst, const void* src, size_t bytes, hipStream_t stream);
}  // namespace kamera

using namespace kamera;

namespace {

thread_local std::string g_last_error;

kamera_status fail(kamera_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

constexpr size_t kAlign = 256;
size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Workspace: header | chunk records | block tables | per-token cos/sin tables. The
// first three are packed on the host and copied in; the tables are computed on the
// device from the chunks' position offsets when the batch is uploaded.
size_t ws_bytes(int64_t nchunks, int64_t pages) {
  return round_up(sizeof(DevHeader), kAlign) + round_up((size_t)nchunks * sizeof(DevChunk), kAlign) +
         round_up((size_t)pages * sizeof(int32_t), kAlign);
}

// cos/sin table of one chunk with per-token offsets: (cos, sin) fp32 of every rotary
// pair of every token, the token count padded to whole 16-token tiles
int64_t phase_tokens(int64_t T) { return (T + kTileTokens - 1) / kTileTokens * kTileTokens; }
size_t phase_bytes(int64_t T, int d_rot) {
  return round_up((size_t)phase_tokens(T) * (d_rot / 2) * 2 * sizeof(float), kAlign);
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// ------------------------------------------------------------------ staging ring
// Pinned, device-mapped host buffers holding packed batches. A small copy-in
// kernel on the caller's stream moves a batch into the device workspace (a
// copy-engine transfer would add a cross-engine handoff to every call). A slot
// is reused only after the copy-in that last read it has completed.
struct Slot {
  void* host = nullptr;
  void* dev = nullptr;  // device view of `host`
  size_t cap = 0;
  hipEvent_t done = nullptr;
  bool pending = false;
};
constexpr int kSlots = 8;
constexpr int kMaxDevices = 64;
struct Ring {
  std::mutex mu;
  Slot slot[kSlots];
  int next = 0;
};
Ring g_ring[kMaxDevices];

kamera_status upload(const void* src, size_t bytes, void* dst, hipStream_t stream) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return fail(KAMERA_E_HIP, "hipGetDevice failed");
  Ring& ring = g_ring[dev];
  std::lock_guard<std::mutex> lock(ring.mu);
  Slot& s = ring.slot[ring.next];
  ring.next = (ring.next + 1) % kSlots;
  if (s.pending) {
    if (hipEventSynchronize(s.done) != hipSuccess) return fail(KAMERA_E_HIP, "hipEventSynchronize failed");
    s.pending = false;
  }
  if (s.cap < bytes) {
    if (s.host) (void)hipHostFree(s.host);
    s.host = s.dev = nullptr;
    s.cap = 0;
    const size_t cap = std::max(round_up(bytes, 64 * 1024), (size_t)64 * 1024);
    if (hipHostMalloc(&s.host, cap, hipHostMallocMapped) != hipSuccess)
      return fail(KAMERA_E_HIP, "hipHostMalloc(%zu) failed", cap);
    if (hipHostGetDevicePointer(&s.dev, s.host, 0) != hipSuccess) {
      (void)hipHostFree(s.host);
      s.host = nullptr;
      return fail(KAMERA_E_HIP, "hipHostGetDevicePointer failed");
    }
    s.cap = cap;
  }
  if (!s.done && hipEventCreateWithFlags(&s.done, hipEventDisableTiming) != hipSuccess)
    return fail(KAMERA_E_HIP, "hipEventCreate failed");
  std::memcpy(s.host, src, bytes);
  const hipError_t e = launch_copy_in(dst, s.dev, bytes, stream);
  if (e != hipSuccess) return fail(KAMERA_E_HIP, "descriptor copy-in launch failed: %s", hipGetErrorString(e));
  if (hipEventRecord(s.done, stream) != hipSuccess) return fail(KAMERA_E_HIP, "hipEventRecord failed");
  s.pending = true;
  return KAMERA_OK;
}

// ------------------------------------------------------------------ validation
kamera_status check_layout(const kamera_layout* L) {
  if (!L) return fail(KAMERA_E_NULL, "layout is NULL");
  if (L->family != KAMERA_GQA && L->family != KAMERA_MLA)
    return fail(KAMERA_E_UNSUPPORTED, "unknown family %d", L->family);
  if (L->dtype != KAMERA_BF16 && L->dtype != KAMERA_F32) return fail(KAMERA_E_DTYPE, "unknown dtype %d", L->dtype);
  if (L->num_layers < 1) return fail(KAMERA_E_SHAPE, "num_layers must be >= 1 (got %d)", L->num_layers);
  if (L->pairing != KAMERA_NEOX && L->pairing != KAMERA_GPTJ)
    return fail(KAMERA_E_UNSUPPORTED, "unknown pairing %d", L->pairing);
  if (L->page_size < 1) return fail(KAMERA_E_SHAPE, "page_size must be >= 1 (got %d)", L->page_size);
  if (L->patch_unit < KAMERA_PATCH_UNIT_AUTO || L->patch_unit > KAMERA_PATCH_UNIT_VALU)
    return fail(KAMERA_E_UNSUPPORTED, "unknown patch_unit %d", L->patch_unit);
  if (!(L->rope_base > 0.0) || !std::isfinite(L->rope_base))
    return fail(KAMERA_E_SHAPE, "rope_base must be positive and finite");
  if (L->reserved2 != 0) return fail(KAMERA_E_SHAPE, "layout.reserved2 must be 0");
  if (L->family == KAMERA_GQA) {
    if (L->num_kv_heads < 1) return fail(KAMERA_E_SHAPE, "num_kv_heads must be >= 1");
    if (L->head_dim < 2 || L->head_dim % 2 || L->head_dim > 512)
      return fail(KAMERA_E_SHAPE, "head_dim must be even in [2, 512] (got %d)", L->head_dim);
    if ((int64_t)L->num_kv_heads * L->head_dim > (1 << 20)) return fail(KAMERA_E_SHAPE, "row too wide");
  } else {
    if (L->latent_dim < 0) return fail(KAMERA_E_SHAPE, "latent_dim must be >= 0");
    if (L->rope_dim < 2 || L->rope_dim % 2 || L->rope_dim > 512)
      return fail(KAMERA_E_SHAPE, "rope_dim must be even in [2, 512] (got %d)", L->rope_dim);
    if ((int64_t)L->latent_dim + L->rope_dim > (1 << 20)) return fail(KAMERA_E_SHAPE, "row too wide");
  }
  const int s0 = L->mrope_section[0], s1 = L->mrope_section[1], s2 = L->mrope_section[2];
  if (s0 < 0 || s1 < 0 || s2 < 0) return fail(KAMERA_E_SHAPE, "mrope_section entries must be >= 0");
  const int npairs = (L->family == KAMERA_GQA ? L->head_dim : L->rope_dim) / 2;
  if ((s0 || s1 || s2) && (int64_t)s0 + s1 + s2 != npairs)
    return fail(KAMERA_E_SHAPE, "mrope_section must add up to d_rot / 2 = %d (got %d + %d + %d)", npairs, s0, s1, s2);
  return KAMERA_OK;
}

int row_width(const kamera_layout* L) {
  return L->family == KAMERA_GQA ? L->num_kv_heads * L->head_dim : L->latent_dim + L->rope_dim;
}

struct Packed {
  std::vector<unsigned char>& blob;  // header | chunks | pages (thread-local, reused across calls)
  std::vector<int64_t>& page_off;    // per chunk: offset (entries) of its page table, -1 if dense
  std::vector<int64_t>& phase_off;   // per chunk: byte offset of its cos/sin table, -1 if none
  size_t upload_bytes = 0;           // header | chunks | pages
  size_t bytes = 0;                  // the whole workspace (tables included)
  int64_t phase_entries = 0;         // table entries (padded token, pair) of the batch
  int64_t phase_max = 0;             // the most entries of one chunk's table
  int64_t phase_blocks = 0;          // table kernel: workgroups per chunk
  bool positions = false;
  bool paged = false;                // a chunk writes through a block table
  int64_t tasks = 0;
  int kernel = 0;   // 0 none, 1 mfma, 2 generic
  int variant = 0;
};

// Task order of batches with paged destinations (see the kernel's decode_task):
// layer-major keeps the workgroups in flight inside one layer's slice of the pool
// (a pool layer is ~180 MB at 36-layer deque sizes); measured 1.5% faster on the
// 16-token random-page deque than chunk-major.
constexpr bool kLayerMajorPaged = true;

// Is the bf16 MFMA kernel able to run this layout at all?
bool mfma_layout_ok(const kamera_layout* L) {
  if (L->dtype != KAMERA_BF16) return false;
  if (L->family == KAMERA_GQA) return L->head_dim == 64 || L->head_dim == 128;
  return L->latent_dim % kSlab == 0 && L->rope_dim == kSlab;
}

kamera_status pack_batch(const kamera_layout* L, const kamera_chunk* chunks, int32_t n, const kamera_pool* pool,
                         Packed& out) {
  kamera_status st = check_layout(L);
  if (st != KAMERA_OK) return st;
  if (n < 0) return fail(KAMERA_E_SHAPE, "num_chunks must be >= 0");
  if (n > 0 && !chunks) return fail(KAMERA_E_NULL, "chunks is NULL");
  const int F = row_width(L);
  const int P = L->page_size;
  const size_t es = L->dtype == KAMERA_BF16 ? 2 : 4;
  const int ntensors = L->family == KAMERA_GQA ? 2 : 1;
  const int d_rot = L->family == KAMERA_GQA ? L->head_dim : L->rope_dim;

  bool any_paged = false;
  int64_t total_pages = 0;
  for (int i = 0; i < n; ++i)
    if (chunks[i].block_table && chunks[i].num_tokens > 0) {
      any_paged = true;
      total_pages += (chunks[i].slot0 + (int64_t)chunks[i].num_tokens + P - 1) / P;
    }
  if (any_paged) {
    if (!pool) return fail(KAMERA_E_NULL, "a chunk has a block table but pool is NULL");
    if (pool->num_pages < 1) return fail(KAMERA_E_SHAPE, "pool.num_pages must be >= 1");
    if (pool->reserved != 0) return fail(KAMERA_E_SHAPE, "pool.reserved must be 0");
    if (!pool->k_pool) return fail(KAMERA_E_NULL, "pool.k_pool is NULL");
    if (!aligned(pool->k_pool, es) || (pool->v_pool && !aligned(pool->v_pool, es)))
      return fail(KAMERA_E_ALIGN, "pool pointers must be aligned to %zu bytes", es);
    if (pool->layer_stride < 0) return fail(KAMERA_E_SHAPE, "pool.layer_stride must be >= 0");
    const int64_t min_ls = (int64_t)pool->num_pages * P * F;
    if (pool->layer_stride != 0 && pool->layer_stride < min_ls)
      return fail(KAMERA_E_SHAPE, "pool.layer_stride %lld smaller than one layer (%lld)",
                  (long long)pool->layer_stride, (long long)min_ls);
  }

  // -------------------------------------------------------------- per-chunk checks
  bool mfma = mfma_layout_ok(L);
  int need_ksteps = 0;  // MFMA path: most 32-wide k-steps covering any column group
  // Pool slots written by this batch: the slot range [lo, hi) each chunk covers in each of
  // its pages, sorted by page, so the overlap check costs O(B log B) in the batch's B page
  // entries, whatever the pool's size.
  struct SlotRange {
    int32_t page, lo, hi, chunk;
  };
  thread_local std::vector<SlotRange> ranges;
  ranges.clear();

  for (int i = 0; i < n; ++i) {
    const kamera_chunk& c = chunks[i];
    if (c.num_tokens < 0) return fail(KAMERA_E_SHAPE, "chunk %d: num_tokens < 0", i);
    if (c.flags & ~(uint32_t)(KAMERA_PATCH | KAMERA_IN_PLACE | KAMERA_POSITIONS))
      return fail(KAMERA_E_UNSUPPORTED, "chunk %d: unknown flag bits 0x%x", i, c.flags);
    if ((c.flags & KAMERA_POSITIONS) && c.num_tokens > 0) {
      if (!c.positions) return fail(KAMERA_E_NULL, "chunk %d: KAMERA_POSITIONS without positions", i);
      if (!aligned(c.positions, sizeof(int32_t)))
        return fail(KAMERA_E_ALIGN, "chunk %d: positions must be 4-byte aligned", i);
    }
    if (c.delta <= -(int64_t(1) << 31) || c.delta >= (int64_t(1) << 31))
      return fail(KAMERA_E_DELTA, "chunk %d: |delta| must be < 2^31", i);
    if (c.num_factors < 0 || c.num_factors > KAMERA_MAX_FACTORS)
      return fail(KAMERA_E_SHAPE, "chunk %d: num_factors must be in [0, %d]", i, KAMERA_MAX_FACTORS);
    if (c.num_tokens == 0) continue;
    const bool in_place = c.flags & KAMERA_IN_PLACE;
    const bool patch = c.flags & KAMERA_PATCH;
    const bool paged = c.block_table != nullptr;
    const int64_t T = c.num_tokens;
    // sources
    if (!in_place) {
      if (!c.k_src || (ntensors == 2 && !c.v_src)) return fail(KAMERA_E_NULL, "chunk %d: source pointer is NULL", i);
      if (!aligned(c.k_src, es) || (c.v_src && !aligned(c.v_src, es)))
        return fail(KAMERA_E_ALIGN, "chunk %d: source pointers must be aligned to %zu bytes", i, es);
      if (c.src_layer_stride < 0 || (c.src_layer_stride != 0 && c.src_layer_stride < T * F))
        return fail(KAMERA_E_SHAPE, "chunk %d: src_layer_stride smaller than T*F", i);
      if (mfma && (!aligned(c.k_src, 16) || (c.v_src && !aligned(c.v_src, 16)) || c.src_layer_stride % 8))
        mfma = false;
    }
    // destination
    // V is touched out of place always, in place only by a patch with a V factor (the
    // packing below streams the same tensors)
    bool v_factor = false;
    for (int f = 0; patch && f < c.num_factors; ++f)
      if (c.factors[f].tensor == 1 && c.factors[f].rank > 0) v_factor = true;
    const bool touches_v = ntensors == 2 && (!in_place || v_factor);
    if (paged) {
      if (touches_v && !pool->v_pool) return fail(KAMERA_E_NULL, "chunk %d: pool.v_pool is NULL", i);
      if (c.slot0 < 0 || c.slot0 >= P) return fail(KAMERA_E_PAGE, "chunk %d: slot0 must be in [0, page_size)", i);
      const int64_t np = (c.slot0 + T + P - 1) / P;
      for (int64_t k = 0; k < np; ++k) {
        const int32_t pg = c.block_table[k];
        if (pg < 0 || pg >= pool->num_pages)
          return fail(KAMERA_E_PAGE, "chunk %d: block_table[%lld] = %d outside [0, %d)", i, (long long)k, pg,
                      pool->num_pages);
      }
      for (int64_t k = 0; k < np; ++k) {
        const int64_t lo = std::max<int64_t>(c.slot0 - k * P, 0);
        const int64_t hi = std::min<int64_t>(c.slot0 + T - k * P, P);
        ranges.push_back(SlotRange{c.block_table[k], (int32_t)lo, (int32_t)hi, i});
      }
      if (mfma && (!aligned(pool->k_pool, 16) || (pool->v_pool && !aligned(pool->v_pool, 16)) ||
                   pool->layer_stride % 8))
        mfma = false;
    } else {
      if (!c.k_dst || (touches_v && !c.v_dst))
        return fail(KAMERA_E_NULL, "chunk %d: destination pointer is NULL", i);
      if (!aligned(c.k_dst, es) || (c.v_dst && !aligned(c.v_dst, es)))
        return fail(KAMERA_E_ALIGN, "chunk %d: destination pointers must be aligned to %zu bytes", i, es);
      if (c.dst_layer_stride < 0 || (c.dst_layer_stride != 0 && c.dst_layer_stride < T * F))
        return fail(KAMERA_E_SHAPE, "chunk %d: dst_layer_stride smaller than T*F", i);
      if (mfma && (!aligned(c.k_dst, 16) || (c.v_dst && !aligned(c.v_dst, 16)) || c.dst_layer_stride % 8))
        mfma = false;
    }
    // factors
    if (patch) {
      for (int f = 0; f < c.num_factors; ++f) {
        const kamera_factor& fa = c.factors[f];
        if (fa.reserved != 0) return fail(KAMERA_E_SHAPE, "chunk %d factor %d: reserved must be 0", i, f);
        if (fa.tensor < 0 || fa.tensor >= ntensors)
          return fail(KAMERA_E_SHAPE, "chunk %d factor %d: tensor %d invalid for this family", i, f, fa.tensor);
        if (fa.rank < 0 || fa.rank > KAMERA_MAX_RANK)
          return fail(KAMERA_E_RANK, "chunk %d factor %d: rank %d outside [0, %d]", i, f, fa.rank, KAMERA_MAX_RANK);
        if (fa.rank == 0) continue;
        if (fa.col0 < 0 || fa.width < 1 || (int64_t)fa.col0 + fa.width > F)
          return fail(KAMERA_E_SHAPE, "chunk %d factor %d: columns [%d, %d) outside the row of %d", i, f, fa.col0,
                      fa.col0 + fa.width, F);
        if (fa.layer0 < 0 || fa.layer0 >= L->num_layers)
          return fail(KAMERA_E_SHAPE, "chunk %d factor %d: layer0 outside [0, L)", i, f);
        if (!fa.u || !fa.v) return fail(KAMERA_E_NULL, "chunk %d factor %d: u or v is NULL", i, f);
        if (!aligned(fa.u, es) || !aligned(fa.v, es))
          return fail(KAMERA_E_ALIGN, "chunk %d factor %d: factor pointers must be aligned to %zu bytes", i, f, es);
      }
      // MFMA path: k-steps of the factors covering each column group
      if (mfma) {
        const int gcols = L->family == KAMERA_GQA ? L->head_dim : kSlab;
        const int ngroups = F / gcols;
        for (int t = 0; t < ntensors; ++t)
          for (int g = 0; g < ngroups; ++g) {
            int ks = 0;
            for (int f = 0; f < c.num_factors; ++f) {
              const kamera_factor& fa = c.factors[f];
              if (fa.rank == 0 || fa.tensor != t || fa.col0 >= (g + 1) * gcols || fa.col0 + fa.width <= g * gcols)
                continue;
              ks += (fa.rank + 31) / 32;
            }
            need_ksteps = std::max(need_ksteps, ks);
          }
      }
    }
  }
  if (ranges.size() > 1) {
    std::sort(ranges.begin(), ranges.end(), [](const SlotRange& a, const SlotRange& b) {
      return a.page != b.page ? a.page < b.page : a.lo < b.lo;
    });
    size_t open = 0;  // the entry of the current page reaching furthest
    for (size_t j = 1; j < ranges.size(); ++j) {
      if (ranges[j].page != ranges[open].page) {
        open = j;
        continue;
      }
      if (ranges[j].lo < ranges[open].hi) {
        const int c0 = std::min(ranges[open].chunk, ranges[j].chunk), c1 = std::max(ranges[open].chunk, ranges[j].chunk);
        if (c0 == c1)
          return fail(KAMERA_E_OVERLAP, "chunk %d writes slot %d of pool page %d twice (its block table repeats the page)",
                      c0, ranges[j].lo, ranges[j].page);
        return fail(KAMERA_E_OVERLAP, "chunks %d and %d both write slot %d of pool page %d", c0, c1, ranges[j].lo,
                    ranges[j].page);
      }
      if (ranges[j].hi > ranges[open].hi) open = j;
    }
  }
  // 128-wide groups keep at most 4 k-steps of V operands in registers; with per-token
  // offsets (a cos/sin set per tile in registers as well) 2 k-steps, 64-wide groups 4
  bool any_positions = false;
  for (int i = 0; i < n; ++i)
    if ((chunks[i].flags & KAMERA_POSITIONS) && chunks[i].num_tokens > 0) any_positions = true;
  const bool wide = L->family == KAMERA_GQA && L->head_dim == 128;
  if (mfma && need_ksteps > (wide ? kMaxKSteps / 2 : kMaxKSteps)) mfma = false;
  if (mfma && any_positions && need_ksteps > (wide ? 2 : 4)) mfma = false;
  if (L->patch_unit == KAMERA_PATCH_UNIT_MFMA && !mfma)
    return fail(KAMERA_E_UNSUPPORTED, "patch_unit MFMA: this batch cannot run on the bf16 matrix-core kernel "
                                      "(dtype, head width, alignment or more k-steps than it holds)");
  const bool valu = L->patch_unit == KAMERA_PATCH_UNIT_VALU;
  if (valu && !(mfma && wide && !any_positions && need_ksteps <= 2))
    return fail(KAMERA_E_UNSUPPORTED, "patch_unit VALU is built for bf16 GQA/MHA with 128-wide heads, at most 64 "
                                      "ranks per column group and no KAMERA_POSITIONS chunk");

  // -------------------------------------------------------------- pack
  out.upload_bytes = ws_bytes(n, total_pages);
  out.bytes = out.upload_bytes;
  out.phase_off.assign((size_t)n, -1);
  out.phase_entries = 0;
  out.phase_max = 0;
  out.positions = false;
  out.paged = any_paged;
  for (int i = 0; i < n; ++i)
    if ((chunks[i].flags & KAMERA_POSITIONS) && chunks[i].num_tokens > 0) {
      out.phase_off[(size_t)i] = (int64_t)out.bytes;
      out.bytes += phase_bytes(chunks[i].num_tokens, d_rot);
      out.positions = true;
    }
  out.blob.assign(out.upload_bytes, 0);
  DevHeader* hd = reinterpret_cast<DevHeader*>(out.blob.data());
  DevChunk* dc = reinterpret_cast<DevChunk*>(out.blob.data() + round_up(sizeof(DevHeader), kAlign));
  int32_t* pg = reinterpret_cast<int32_t*>(out.blob.data() + round_up(sizeof(DevHeader), kAlign) +
                                           round_up((size_t)n * sizeof(DevChunk), kAlign));
  hd->nchunks = n;
  hd->family = L->family;
  hd->dtype = L->dtype;
  hd->L = L->num_layers;
  hd->F = F;
  hd->H = L->family == KAMERA_GQA ? L->num_kv_heads : 0;
  hd->head_dim = L->head_dim;
  hd->latent_dim = L->latent_dim;
  hd->rope_dim = L->rope_dim;
  hd->d_rot = d_rot;
  hd->pairing = L->pairing;
  hd->page_size = P;
  hd->page_shift = (P & (P - 1)) == 0 ? __builtin_ctz((unsigned)P) : -1;
  hd->rope_base = L->rope_base;
  for (int k = 0; k < 3; ++k) hd->mrope[k] = L->mrope_section[k];
  hd->group_cols = mfma ? (L->family == KAMERA_GQA ? L->head_dim : kSlab) : F;
  hd->rope_group = (mfma && L->family == KAMERA_MLA) ? L->latent_dim / kSlab : -1;
  // XCD window (measured on MI355X): rows of more than 8 column groups (e.g. 32 heads x
  // 128) span several workgroups and gain 19% from keeping a row's workgroups on one
  // XCD (W = 16); rows of exactly 8 groups gain ~1% with W = 4; narrower rows, where a
  // workgroup already covers whole rows, are fastest in plain order.
  if (mfma) {
    const int ngroups = F / hd->group_cols;
    hd->xcd_window_log2 = ngroups > kWavesPerBlock ? 4 : (ngroups == kWavesPerBlock ? 2 : 0);
  }

  // Generic kernel: one workgroup per 16 tokens, or per 4 tokens when the batch is too
  // small to fill the chip that way (fewer than 1024 workgroups of 16 tokens): each
  // thread then has about one element to compute instead of waiting out several memory
  // round trips in turn (a single-layer 256-token fp32 chunk: 14.8 -> 6.3 us).
  int64_t generic_rows = 0;
  for (int i = 0; i < n; ++i) generic_rows += (int64_t)chunks[i].num_tokens * L->num_layers * ntensors;
  const int tb_tokens = mfma ? kMfmaRangeTokens : (generic_rows >= 16 * 1024 ? 16 : 4);
  const bool layer_major = kLayerMajorPaged && mfma && any_paged;
  int64_t task = 0;
  int64_t page_cursor = 0;
  out.page_off.assign((size_t)n, -1);
  const int64_t pool_ls = (any_paged && pool->layer_stride == 0) ? (int64_t)pool->num_pages * P * F
                                                                 : (pool ? pool->layer_stride : 0);
  for (int i = 0; i < n; ++i) {
    const kamera_chunk& c = chunks[i];
    DevChunk& d = dc[i];
    d.task0 = task;
    d.T = c.num_tokens;
    d.flags = c.flags;
    d.delta = c.delta;
    d.slot0 = c.slot0;
    if (out.phase_off[(size_t)i] >= 0) {
      d.positions = c.positions;
      const int64_t ne = phase_tokens(c.num_tokens) * (d_rot / 2);
      out.phase_entries += ne;
      out.phase_max = std::max(out.phase_max, ne);
    }
    if (c.num_tokens == 0) continue;
    const bool in_place = c.flags & KAMERA_IN_PLACE;
    const bool patch = c.flags & KAMERA_PATCH;
    const bool paged = c.block_table != nullptr;
    const int64_t T = c.num_tokens;
    if (paged) {
      const int64_t np = (c.slot0 + T + P - 1) / P;
      std::memcpy(pg + page_cursor, c.block_table, (size_t)np * sizeof(int32_t));
      out.page_off[(size_t)i] = page_cursor;  // turned into a device address once the workspace is known
      page_cursor += np;
      d.dst[0] = pool->k_pool;
      d.dst[1] = pool->v_pool;
      d.dst_ls = pool_ls;
    } else {
      d.pages = nullptr;
      d.dst[0] = c.k_dst;
      d.dst[1] = c.v_dst;
      d.dst_ls = c.dst_layer_stride ? c.dst_layer_stride : T * F;
    }
    if (in_place) {
      d.src[0] = d.dst[0];
      d.src[1] = d.dst[1];
      d.src_ls = d.dst_ls;
    } else {
      d.src[0] = c.k_src;
      d.src[1] = c.v_src;
      d.src_ls = c.src_layer_stride ? c.src_layer_stride : T * F;
    }
    d.nfac = patch ? c.num_factors : 0;
    bool v_factor = false;
    for (int f = 0; f < d.nfac; ++f) {
      const kamera_factor& fa = c.factors[f];
      DevFactor& df = d.fac[f];
      df.u = fa.u;
      df.v = fa.v;
      df.tensor = fa.tensor;
      df.col0 = fa.col0;
      df.width = fa.width;
      df.rank = fa.rank;
      df.layer0 = fa.layer0;
      df.uvec = (fa.rank % 8 == 0 && aligned(fa.u, 16)) ? 1 : 0;
      df.vvec = (fa.rank % 8 == 0 && aligned(fa.v, 16)) ? 1 : 0;
      if (fa.tensor == 1 && fa.rank > 0) v_factor = true;
    }
    // streams: tensors this chunk touches
    if (L->family == KAMERA_GQA) {
      d.stream_tensor[0] = 0;
      d.stream_tensor[1] = 1;
      d.nstreams = (in_place && !(patch && v_factor)) ? 1 : 2;
    } else {
      d.stream_tensor[0] = 0;
      d.stream_tensor[1] = 0;
      d.nstreams = 1;
    }
    d.tb_tokens = tb_tokens;
    d.ntb = (int32_t)((T + tb_tokens - 1) / tb_tokens);
    if (mfma) {
      const int ngroups = F / hd->group_cols;
      if (L->family == KAMERA_MLA && in_place && !patch) {
        d.group0 = hd->rope_group;
        d.ngroups = 1;
      } else {
        d.group0 = 0;
        d.ngroups = ngroups;
      }
    } else {
      d.group0 = 0;
      d.ngroups = 1;
    }
    task += (int64_t)d.nstreams * (layer_major ? 1 : L->num_layers) * d.ntb * d.ngroups;
  }
  if (layer_major) {
    hd->layer_tasks = task;
    task *= L->num_layers;
  }
  hd->total_tasks = task;
  out.phase_blocks = (out.phase_max + kBlockThreads - 1) / kBlockThreads;
  hd->phase_blocks = (int32_t)std::min<int64_t>(out.phase_blocks, 0x7fffffff);  // the launcher rejects larger
  out.tasks = task;
  out.kernel = task == 0 ? 0 : (mfma ? 1 : 2);
  out.variant = 0;
  if (mfma) {
    int cap_log2 = 0;
    while ((1 << cap_log2) < need_ksteps) ++cap_log2;
    out.variant = (hd->group_cols / kSlab - 1) * 4 + cap_log2 + (out.positions ? kVariantPositions : 0) +
                  (valu ? kVariantValu : 0);
  }
  return KAMERA_OK;
}

// The packed batch's block-table and cos/sin-table offsets turned into device addresses
// inside the workspace `ws` it will be copied to.
void bind_workspace(Packed& pk, int n, void* ws) {
  const size_t pages_off = round_up(sizeof(DevHeader), kAlign) + round_up((size_t)n * sizeof(DevChunk), kAlign);
  DevChunk* dc = reinterpret_cast<DevChunk*>(pk.blob.data() + round_up(sizeof(DevHeader), kAlign));
  for (int i = 0; i < n; ++i)
    dc[i].pages = pk.page_off[(size_t)i] < 0
                      ? nullptr
                      : reinterpret_cast<const int32_t*>((char*)ws + pages_off +
                                                         (size_t)pk.page_off[(size_t)i] * sizeof(int32_t));
  for (int i = 0; i < n; ++i)
    dc[i].phase = pk.phase_off[(size_t)i] < 0 ? nullptr
                                              : reinterpret_cast<const float*>((char*)ws + pk.phase_off[(size_t)i]);
}

const DevHeader* ws_header(const void* ws) { return reinterpret_cast<const DevHeader*>(ws); }
const DevChunk* ws_chunks(const void* ws) {
  return reinterpret_cast<const DevChunk*>((const char*)ws + round_up(sizeof(DevHeader), kAlign));
}

// After the packed batch has reached the workspace: the per-token cos/sin tables (when the
// batch has re-anchored chunks) are computed there, on the same stream.
kamera_status launch_phase_tables(const Packed& pk, int n, void* ws, void* stream) {
  if (pk.phase_entries <= 0) return KAMERA_OK;
  const hipError_t e = launch_phase_table(ws_header(ws), ws_chunks(ws), n, pk.phase_blocks, (hipStream_t)stream,
                                          nullptr);
  if (e != hipSuccess) return fail(KAMERA_E_HIP, "phase table launch failed: %s", hipGetErrorString(e));
  return KAMERA_OK;
}

kamera_status launch_main(int kernel, int variant, int dtype, int64_t tasks, const void* ws, void* stream) {
  if (tasks <= 0 || kernel == 0) return KAMERA_OK;
  hipError_t e;
  if (kernel == 1) e = launch_mfma(variant, ws_header(ws), ws_chunks(ws), tasks, (hipStream_t)stream, nullptr);
  else if (kernel == 2) e = launch_generic(dtype, ws_header(ws), ws_chunks(ws), tasks, (hipStream_t)stream, nullptr);
  else return fail(KAMERA_E_UNSUPPORTED, "plan names unknown kernel %d", kernel);
  if (e != hipSuccess) return fail(KAMERA_E_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return KAMERA_OK;
}

kamera_status upload_plan(const kamera_layout* L, const kamera_chunk* chunks, int32_t n, const kamera_pool* pool,
                          void* ws, size_t ws_size, void* stream, kamera_plan* plan) {
  thread_local std::vector<unsigned char> blob;
  thread_local std::vector<int64_t> page_off;
  thread_local std::vector<int64_t> phase_off;
  Packed pk{blob, page_off, phase_off};
  kamera_status st = pack_batch(L, chunks, n, pool, pk);
  if (st != KAMERA_OK) return st;
  if (!ws) return fail(KAMERA_E_WORKSPACE, "workspace is NULL");
  if (!aligned(ws, kAlign)) return fail(KAMERA_E_ALIGN, "workspace must be %zu-byte aligned", kAlign);
  if (ws_size < pk.bytes) return fail(KAMERA_E_WORKSPACE, "workspace has %zu bytes, %zu needed", ws_size, pk.bytes);
  bind_workspace(pk, n, ws);
  if (pk.tasks > 0) {
    st = upload(pk.blob.data(), pk.upload_bytes, ws, (hipStream_t)stream);
    if (st != KAMERA_OK) return st;
    st = launch_phase_tables(pk, n, ws, stream);  // computed once per upload
    if (st != KAMERA_OK) return st;
  }
  std::memset(plan, 0, sizeof(*plan));
  plan->workspace = ws;
  plan->num_tasks = pk.tasks;
  plan->kernel = pk.kernel;
  plan->variant = pk.variant;
  plan->num_chunks = n;
  plan->reserved[0] = L->dtype;
  return KAMERA_OK;
}

// Small dense batches (at most kInlineChunks chunks, no block tables, at most
// kInlineFactors factors each): validated and packed as usual, then handed to the kernels
// as their argument, so nothing is staged or copied in (re-anchored chunks' cos/sin tables
// are still computed into the workspace). Returns false when the batch does not qualify (the caller
// then uploads it); otherwise the call's status is in *st.
bool launch_inline(const kamera_layout* L, const kamera_chunk* chunks, int32_t n, const kamera_pool* pool,
                   void* ws, size_t ws_size, void* stream, kamera_status* st_out) {
  if (n < 1 || n > kInlineChunks || !chunks) return false;
  for (int i = 0; i < n; ++i) {
    const kamera_chunk& c = chunks[i];
    if (c.block_table) return false;
    if ((c.flags & KAMERA_PATCH) && c.num_factors > kInlineFactors) return false;
  }
  kamera_status& st_ret = *st_out;
  thread_local std::vector<unsigned char> blob;
  thread_local std::vector<int64_t> page_off;
  thread_local std::vector<int64_t> phase_off;
  Packed pk{blob, page_off, phase_off};
  st_ret = pack_batch(L, chunks, n, pool, pk);
  if (st_ret != KAMERA_OK) return true;
  if (pk.paged) return false;
  // the workspace is not used on this path, but the call's contract is the same on both
  if (!ws) {
    st_ret = fail(KAMERA_E_WORKSPACE, "workspace is NULL");
  } else if (!aligned(ws, kAlign)) {
    st_ret = fail(KAMERA_E_ALIGN, "workspace must be %zu-byte aligned", kAlign);
  } else if (ws_size < pk.bytes) {
    st_ret = fail(KAMERA_E_WORKSPACE, "workspace has %zu bytes, %zu needed", ws_size, pk.bytes);
  }
  if (st_ret != KAMERA_OK || pk.tasks == 0) return true;
  InlineBatch b;
  std::memset(&b, 0, sizeof(b));
  std::memcpy(&b.hd, pk.blob.data(), sizeof(DevHeader));
  const DevChunk* dc = reinterpret_cast<const DevChunk*>(pk.blob.data() + round_up(sizeof(DevHeader), kAlign));
  for (int i = 0; i < n; ++i) {  // the compact records: the fields the dense path reads
    const DevChunk& d = dc[i];
    DevChunkInline& e = b.ch[i];
    for (int t = 0; t < 2; ++t) {
      e.src[t] = d.src[t];
      e.dst[t] = d.dst[t];
      e.stream_tensor[t] = (int16_t)d.stream_tensor[t];
    }
    e.src_ls = d.src_ls;
    e.dst_ls = d.dst_ls;
    e.delta = d.delta;
    e.task0 = d.task0;
    e.T = d.T;
    e.flags = d.flags;
    e.slot0 = d.slot0;
    e.nfac = (int16_t)d.nfac;              // <= kInlineFactors
    e.ntb = d.ntb;
    e.tb_tokens = d.tb_tokens;
    e.nstreams = (int16_t)d.nstreams;      // 1 or 2
    e.ngroups = (int16_t)d.ngroups;        // <= 2^20 / 64 (the row-width check)
    e.group0 = (int16_t)d.group0;
    e.pages = nullptr;
    e.positions = d.positions;
    e.phase = pk.phase_off[(size_t)i] < 0 ? nullptr
                                         : reinterpret_cast<const float*>((char*)ws + pk.phase_off[(size_t)i]);
    for (int f = 0; f < d.nfac; ++f) e.fac[f] = d.fac[f];  // nfac <= kInlineFactors (checked above)
  }
  hipError_t e = hipSuccess;
  if (pk.phase_entries > 0)  // per-token cos/sin tables into the workspace, from the same argument
    e = launch_phase_table(nullptr, nullptr, n, pk.phase_blocks, (hipStream_t)stream, &b);
  if (e != hipSuccess) {
    st_ret = fail(KAMERA_E_HIP, "phase table launch failed: %s", hipGetErrorString(e));
    return true;
  }
  if (pk.kernel == 1) e = launch_mfma(pk.variant, nullptr, nullptr, pk.tasks, (hipStream_t)stream, &b);
  else e = launch_generic(L->dtype, nullptr, nullptr, pk.tasks, (hipStream_t)stream, &b);
  if (e != hipSuccess) st_ret = fail(KAMERA_E_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return true;
}

}  // namespace

extern "C" {

size_t kamera_workspace_bytes(int32_t num_chunks, int64_t total_block_table_entries) {
  if (num_chunks < 0 || total_block_table_entries < 0) return 0;
  return ws_bytes(num_chunks, total_block_table_entries);
}

size_t kamera_batch_workspace_bytes(const kamera_layout* layout, const kamera_chunk* chunks, int32_t num_chunks) {
  if (!layout || num_chunks < 0 || (num_chunks > 0 && !chunks) || layout->page_size < 1) return 0;
  const int d_rot = layout->family == KAMERA_GQA ? layout->head_dim : layout->rope_dim;
  const int P = layout->page_size;
  int64_t pages = 0;
  size_t tables = 0;
  for (int i = 0; i < num_chunks; ++i) {
    const kamera_chunk& c = chunks[i];
    if (c.num_tokens < 0 || c.slot0 < 0) return 0;
    if (c.num_tokens == 0) continue;
    if (c.block_table) pages += (c.slot0 + (int64_t)c.num_tokens + P - 1) / P;
    if (c.flags & KAMERA_POSITIONS) tables += phase_bytes(c.num_tokens, d_rot);
  }
  return ws_bytes(num_chunks, pages) + tables;
}

kamera_status kamera_plan_upload(const kamera_layout* layout, const kamera_chunk* chunks, int32_t num_chunks,
                                 const kamera_pool* pool, void* workspace, size_t workspace_bytes, void* stream,
                                 kamera_plan* plan) {
  g_last_error.clear();
  if (!plan) return fail(KAMERA_E_NULL, "plan is NULL");
  return upload_plan(layout, chunks, num_chunks, pool, workspace, workspace_bytes, stream, plan);
}

kamera_status kamera_plan_launch(const kamera_plan* plan, void* stream) {
  g_last_error.clear();
  if (!plan) return fail(KAMERA_E_NULL, "plan is NULL");
  if (plan->num_tasks <= 0 || plan->kernel == 0) return KAMERA_OK;
  if (!plan->workspace) return fail(KAMERA_E_WORKSPACE, "plan has no workspace");
  return launch_main(plan->kernel, plan->variant, plan->reserved[0], plan->num_tasks, plan->workspace, stream);
}

kamera_status kamera_rehydrate_batched(const kamera_layout* layout, const kamera_chunk* chunks, int32_t num_chunks,
                                       const kamera_pool* pool, void* workspace, size_t workspace_bytes,
                                       void* stream) {
  g_last_error.clear();
  kamera_status st0 = KAMERA_OK;
  if (launch_inline(layout, chunks, num_chunks, pool, workspace, workspace_bytes, stream, &st0)) return st0;
  kamera_plan plan;
  kamera_status st = kamera_plan_upload(layout, chunks, num_chunks, pool, workspace, workspace_bytes, stream, &plan);
  if (st != KAMERA_OK) return st;
  return kamera_plan_launch(&plan, stream);
}

static_assert(KAMERA_NOALLOC_SCRATCH_BYTES == kNoallocScratchBytes, "scratch limit of the ABI and the library");

kamera_status kamera_rehydrate_batched_noalloc(const kamera_layout* layout, const kamera_chunk* chunks,
                                               int32_t num_chunks, const kamera_pool* pool, void* stream) {
  g_last_error.clear();
  thread_local std::vector<unsigned char> blob;
  thread_local std::vector<int64_t> page_off;
  thread_local std::vector<int64_t> phase_off;
  Packed pk{blob, page_off, phase_off};
  kamera_status st = pack_batch(layout, chunks, num_chunks, pool, pk);
  if (st != KAMERA_OK) return st;
  if (pk.bytes > kNoallocScratchBytes)
    return fail(KAMERA_E_WORKSPACE,
                "the batch needs %zu bytes of scratch (packed chunks, block tables, cos/sin tables); "
                "kamera_rehydrate_batched_noalloc holds at most %zu: split the batch, or pass a workspace to "
                "kamera_rehydrate_batched",
                pk.bytes, kNoallocScratchBytes);
  if (pk.tasks == 0) return KAMERA_OK;
  void* ws = nullptr;
  const hipError_t e = scratch_address(&ws);
  if (e != hipSuccess) return fail(KAMERA_E_HIP, "device address of the scratch array: %s", hipGetErrorString(e));
  // a small dense batch goes as the kernels' argument (only cos/sin tables use the scratch)
  kamera_status st0 = KAMERA_OK;
  if (launch_inline(layout, chunks, num_chunks, pool, ws, kNoallocScratchBytes, stream, &st0)) return st0;
  bind_workspace(pk, num_chunks, ws);
  const hipError_t ef = launch_fill_by_argument(ws, pk.blob.data(), pk.upload_bytes, (hipStream_t)stream);
  if (ef != hipSuccess) return fail(KAMERA_E_HIP, "scratch fill launch failed: %s", hipGetErrorString(ef));
  st = launch_phase_tables(pk, num_chunks, ws, stream);
  if (st != KAMERA_OK) return st;
  return launch_main(pk.kernel, pk.variant, layout->dtype, pk.tasks, ws, stream);
}

kamera_status kamera_rehydrate(const kamera_layout* layout, const kamera_chunk* chunk, const kamera_pool* pool,
                               void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  if (!chunk) return fail(KAMERA_E_NULL, "chunk is NULL");
  return kamera_rehydrate_batched(layout, chunk, 1, pool, workspace, workspace_bytes, stream);
}

kamera_status kamera_relocate(const kamera_layout* layout, const kamera_pool* pool, const int32_t* block_table,
                              int32_t slot0, int32_t num_tokens, int64_t delta, void* workspace,
                              size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  kamera_status st = check_layout(layout);
  if (st != KAMERA_OK) return st;
  if (!pool) return fail(KAMERA_E_NULL, "pool is NULL");
  if (num_tokens < 0) return fail(KAMERA_E_SHAPE, "num_tokens < 0");
  const int P = layout->page_size;
  std::vector<int32_t> ident;
  if (!block_table && num_tokens > 0) {
    if (slot0 < 0) return fail(KAMERA_E_PAGE, "slot0 < 0");
    const int64_t np = ((int64_t)slot0 % P + num_tokens + P - 1) / P;
    const int64_t first = slot0 / P;
    // range first, so that an oversized request fails before the identity table is built
    if (first + np > (int64_t)pool->num_pages)
      return fail(KAMERA_E_PAGE, "rows [%d, %lld) outside the pool's %lld rows", slot0, (long long)slot0 + num_tokens,
                  (long long)pool->num_pages * P);
    ident.resize((size_t)np);
    for (int64_t k = 0; k < np; ++k) ident[(size_t)k] = (int32_t)(first + k);
    block_table = ident.data();
    slot0 = slot0 % P;
  }
  kamera_chunk c;
  std::memset(&c, 0, sizeof(c));
  c.num_tokens = num_tokens;
  c.flags = KAMERA_IN_PLACE;
  c.delta = delta;
  c.block_table = block_table;
  c.slot0 = slot0;
  return kamera_rehydrate_batched(layout, &c, 1, pool, workspace, workspace_bytes, stream);
}

size_t kamera_build_workspace_bytes(int64_t num_tokens, int32_t width, int32_t rank) {
  if (num_tokens < 1 || width < 1 || rank < 1) return 0;
  return build_workspace_bytes(num_tokens, width, rank);
}

}  // extern "C"

namespace {

static_assert(KAMERA_BUILD_MAX_ORBIT == kBuildMaxOrbit, "orbit limit of the ABI and the builder");
static_assert(KAMERA_BUILD_MAX_RANK == kBuildMaxRank, "rank limit of the ABI and the builder");
static_assert(KAMERA_BUILD_MAX_SUBSPACE == kBuildMaxSubspace, "subspace size of the ABI and the builder");

kamera_status build_impl(const kamera_layout* layout, int32_t tensor, int32_t norbit, const void* const* x_conds,
                         const int64_t* deltas, const void* x_canon, int64_t num_tokens, int32_t col0,
                         int32_t width, int32_t rank, int32_t iterations, void* u_out, void* v_out,
                         double* sigma_out, void* workspace, size_t workspace_bytes, void* stream) {
  kamera_status st = check_layout(layout);
  if (st != KAMERA_OK) return st;
  const bool gqa = layout->family == KAMERA_GQA;
  if (tensor < 0 || tensor > (gqa ? 1 : 0))
    return fail(KAMERA_E_SHAPE, "tensor %d invalid for this family", tensor);
  if (norbit < 1 || norbit > KAMERA_BUILD_MAX_ORBIT)
    return fail(KAMERA_E_SHAPE, "num_orderings must be in [1, %d] (got %d)", KAMERA_BUILD_MAX_ORBIT, norbit);
  if (!x_conds || !deltas) return fail(KAMERA_E_NULL, "x_conds or deltas is NULL");
  const size_t es = layout->dtype == KAMERA_BF16 ? 2 : 4;
  for (int k = 0; k < norbit; ++k) {
    if (!x_conds[k]) return fail(KAMERA_E_NULL, "x_cond of ordering %d is NULL", k);
    if (!aligned(x_conds[k], es)) return fail(KAMERA_E_ALIGN, "x_cond of ordering %d must be aligned to %zu bytes", k, es);
    if (deltas[k] <= -(int64_t(1) << 31) || deltas[k] >= (int64_t(1) << 31))
      return fail(KAMERA_E_DELTA, "ordering %d: |delta| must be < 2^31", k);
  }
  if (!x_canon) return fail(KAMERA_E_NULL, "x_canon is NULL");
  if (!u_out || !v_out) return fail(KAMERA_E_NULL, "u_out or v_out is NULL");
  if (!aligned(x_canon, es) || !aligned(u_out, es) || !aligned(v_out, es))
    return fail(KAMERA_E_ALIGN, "row and factor pointers must be aligned to %zu bytes", es);
  if (sigma_out && !aligned(sigma_out, sizeof(double))) return fail(KAMERA_E_ALIGN, "sigma_out must be 8-byte aligned");
  if (num_tokens < 1 || num_tokens > (1 << 24)) return fail(KAMERA_E_SHAPE, "num_tokens must be in [1, 2^24]");
  const int F = row_width(layout);
  if (col0 < 0 || width < 1 || (int64_t)col0 + width > F)
    return fail(KAMERA_E_SHAPE, "columns [%d, %lld) outside the row of %d", col0, (long long)col0 + width, F);
  const int64_t max_rank = std::min<int64_t>(KAMERA_BUILD_MAX_RANK, std::min<int64_t>(width, num_tokens));
  if (rank < 1 || rank > max_rank) return fail(KAMERA_E_RANK, "rank %d outside [1, %lld]", rank, (long long)max_rank);
  if (iterations < 0 || iterations > 64) return fail(KAMERA_E_SHAPE, "iterations must be in [0, 64]");
  if ((int64_t)num_tokens * width > (int64_t(1) << 31))
    return fail(KAMERA_E_SHAPE, "num_tokens * width must be <= 2^31");
  const size_t need = build_workspace_bytes(num_tokens, width, rank);
  if (!workspace) return fail(KAMERA_E_WORKSPACE, "workspace is NULL");
  if (!aligned(workspace, kAlign)) return fail(KAMERA_E_ALIGN, "workspace must be %zu-byte aligned", kAlign);
  if (workspace_bytes < need) return fail(KAMERA_E_WORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes, need);

  BuildArgs a;
  std::memset(&a, 0, sizeof(a));
  for (int k = 0; k < norbit; ++k) {
    a.x_cond[k] = x_conds[k];
    a.delta_k[k] = deltas[k];
  }
  a.norbit = norbit;
  a.x_canon = x_canon;
  a.u_out = u_out;
  a.v_out = v_out;
  a.sigma = sigma_out;
  a.base = layout->rope_base;
  a.T = (int)num_tokens;
  a.F = F;
  a.W = width;
  a.col0 = col0;
  a.m = rank;
  a.p = (int)std::min<int64_t>(kBuildMaxSubspace, std::min<int64_t>(width, num_tokens));
  a.iters = iterations;
  a.dtype = layout->dtype == KAMERA_BF16 ? 1 : 0;
  a.rotate = tensor == 0;
  a.pairing = layout->pairing;
  if (gqa) {
    a.band0 = 0;
    a.band_stride = layout->head_dim;
    a.nbands = layout->num_kv_heads;
    a.d_rot = layout->head_dim;
  } else {
    a.band0 = layout->latent_dim;
    a.band_stride = layout->rope_dim;
    a.nbands = 1;
    a.d_rot = layout->rope_dim;
  }
  build_workspace_carve(a, workspace);
  const hipError_t e = launch_builder(a, (hipStream_t)stream);
  if (e != hipSuccess) return fail(KAMERA_E_HIP, "builder launch failed: %s", hipGetErrorString(e));
  return KAMERA_OK;
}

}  // namespace

extern "C" {

kamera_status kamera_build_patch(const kamera_layout* layout, int32_t tensor, const void* x_cond,
                                 const void* x_canon, int64_t num_tokens, int64_t delta, int32_t col0,
                                 int32_t width, int32_t rank, int32_t iterations, void* u_out, void* v_out,
                                 double* sigma_out, void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  if (!x_cond) return fail(KAMERA_E_NULL, "x_cond is NULL");
  const void* conds[1] = {x_cond};
  const int64_t deltas[1] = {delta};
  return build_impl(layout, tensor, 1, conds, deltas, x_canon, num_tokens, col0, width, rank, iterations, u_out,
                    v_out, sigma_out, workspace, workspace_bytes, stream);
}

kamera_status kamera_build_orbit_patch(const kamera_layout* layout, int32_t tensor, int32_t num_orderings,
                                       const void* const* x_conds, const int64_t* deltas, const void* x_canon,
                                       int64_t num_tokens, int32_t col0, int32_t width, int32_t rank,
                                       int32_t iterations, void* u_out, void* v_out, double* sigma_out,
                                       void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  return build_impl(layout, tensor, num_orderings, x_conds, deltas, x_canon, num_tokens, col0, width, rank,
                    iterations, u_out, v_out, sigma_out, workspace, workspace_bytes, stream);
}

kamera_status kamera_stream_probe(int32_t kind, const void* src, void* dst, size_t bytes, uint32_t value,
                                  void* stream) {
  g_last_error.clear();
  if (kind < KAMERA_PROBE_COPY || kind > KAMERA_PROBE_WRITE) return fail(KAMERA_E_UNSUPPORTED, "unknown probe kind %d", kind);
  if (bytes % 16) return fail(KAMERA_E_SHAPE, "bytes must be a multiple of 16 (got %zu)", bytes);
  if (bytes == 0) return KAMERA_OK;
  if ((kind != KAMERA_PROBE_WRITE && !src) || !dst) return fail(KAMERA_E_NULL, "src or dst is NULL");
  if ((src && !aligned(src, 16)) || !aligned(dst, 16)) return fail(KAMERA_E_ALIGN, "src and dst must be 16-byte aligned");
  const hipError_t e = launch_stream_probe(kind, src, dst, (int64_t)(bytes / 16), value, (hipStream_t)stream);
  if (e != hipSuccess) return fail(KAMERA_E_HIP, "probe launch failed: %s", hipGetErrorString(e));
  return KAMERA_OK;
}

const char* kamera_status_string(kamera_status s) {
  switch (s) {
    case KAMERA_OK: return "KAMERA_OK";
    case KAMERA_E_NULL: return "KAMERA_E_NULL";
    case KAMERA_E_SHAPE: return "KAMERA_E_SHAPE";
    case KAMERA_E_DTYPE: return "KAMERA_E_DTYPE";
    case KAMERA_E_RANK: return "KAMERA_E_RANK";
    case KAMERA_E_DELTA: return "KAMERA_E_DELTA";
    case KAMERA_E_PAGE: return "KAMERA_E_PAGE";
    case KAMERA_E_OVERLAP: return "KAMERA_E_OVERLAP";
    case KAMERA_E_ALIGN: return "KAMERA_E_ALIGN";
    case KAMERA_E_WORKSPACE: return "KAMERA_E_WORKSPACE";
    case KAMERA_E_UNSUPPORTED: return "KAMERA_E_UNSUPPORTED";
    case KAMERA_E_HIP: return "KAMERA_E_HIP";
  }
  return "KAMERA_E_UNKNOWN";
}

const char* kamera_last_error(void) { return g_last_error.c_str(); }

const char* kamera_version(void) { return "kamera-gfx950 0.1.0"; }

}  // extern "C"
