// Internal packed batch description shared by the host packer and the kernels.
// Not part of the public ABI (include/kamera.h is).
#pragma once

#include <stdint.h>

namespace kamera {

constexpr int kWaveSize = 64;
constexpr int kBlockThreads = 256;           // generic and copy-in kernels
// MFMA path: 8 waves per workgroup. Consecutive wave tasks are the heads of one
// token block and the next block, so a workgroup's waves share U rows (4 heads)
// and V rows (2 blocks) through the CU's caches; measured faster than 4 or 16.
constexpr int kWavesPerBlock = 8;
// One-slab variants with at most 2 k-steps (MLA rows, 64-wide heads) stay within 128
// VGPRs, 4 waves per SIMD; 4-wave workgroups let 4 of them share a CU (16 waves, against
// 8 with 8-wave workgroups): measured 9% faster on the 27-layer MLA batch.
constexpr int kWavesPerBlockNarrow = 4;
constexpr int mfma_waves_per_block(int nslab, int nkmax) {
  return (nslab == 1 && nkmax <= 2) ? kWavesPerBlockNarrow : kWavesPerBlock;
}
constexpr int kSlab = 64;          // columns per slab of the MFMA path
constexpr int kTileTokens = 16;    // tokens per MFMA tile (the N dimension)
constexpr int kMaxFactors = 4;

// MFMA path: a wave task covers a column group of 1 or 2 slabs and holds up to
// kMaxKSteps 32-wide k-steps of V operands in registers. Kernel variant
// v = (slabs - 1) * 4 + log2(k-step capacity), capacity in {1, 2, 4, 8}.
constexpr int kMaxKSteps = 8;
constexpr int kVariantPositions = 8;   // added to the variant: batches with per-token offsets
constexpr int kVariantValu = 16;       // added to the variant: the patch on the VALU instead of the MFMA
constexpr int kMfmaRangeTokens = 128;  // tokens per wave task (8 tiles)

struct alignas(16) DevFactor {
  const void* u;        // [L - layer0][T][rank]
  const void* v;        // [L - layer0][width][rank]
  int32_t tensor;
  int32_t col0;
  int32_t width;
  int32_t rank;
  int32_t layer0;
  int32_t uvec;         // rank % 8 == 0 and u 16-byte aligned: 16-byte loads of U rows
  int32_t vvec;         // rank % 8 == 0 and v 16-byte aligned: 16-byte loads of V rows
  int32_t pad;
};
static_assert(sizeof(DevFactor) == 48, "DevFactor layout");

// Per-chunk record. Task space of a chunk (MFMA path: one task = one wave; generic: one workgroup):
//   chunk-major:  task = task0 + ((stream * L + layer) * ntb + tb) * ngroups + g
//   layer-major:  task = layer * layer_tasks + task0 + (stream * ntb + tb) * ngroups + g
// stream indexes the tensors this chunk touches (stream_tensor[]), tb the token
// block, g the column group (MFMA path: head or slab; generic path: unused = 1).
struct alignas(16) DevChunk {
  const void* src[2];   // per tensor: first source row of layer 0 (in place: == dst)
  void* dst[2];         // per tensor: dense destination, or pool base (paged)
  int64_t src_ls;       // elements between layers (source)
  int64_t dst_ls;       // elements between layers (destination / pool)
  int64_t delta;
  const int32_t* pages; // device copy of the block table (NULL: dense destination)
  const int32_t* positions;  // per-token offsets [T][3] (KAMERA_POSITIONS), caller's device memory
  const float* phase;   // per-token cos/sin table in the workspace (positions chunks; see phase_offset)
  int64_t task0;        // first task id of this chunk
  int32_t T;
  uint32_t flags;
  int32_t slot0;
  int32_t nfac;
  int32_t ntb;          // token blocks
  int32_t tb_tokens;    // tokens per block
  int32_t nstreams;     // tensors touched (1 or 2)
  int32_t ngroups;      // column groups per tensor (MFMA path)
  int32_t group0;       // first group id (MLA in-place rotation touches only the rope group)
  int32_t stream_tensor[2];
  int32_t pad;
  DevFactor fac[kMaxFactors];
};

struct alignas(16) DevHeader {
  uint32_t reserved[4];  // zero
  int64_t total_tasks;
  int32_t nchunks;
  int32_t family;
  int32_t dtype;
  int32_t L;
  int32_t F;            // row width
  int32_t H;            // GQA heads
  int32_t head_dim;
  int32_t latent_dim;
  int32_t rope_dim;
  int32_t d_rot;        // rotary band width
  int32_t pairing;
  int32_t page_size;
  int32_t group_cols;   // MFMA path: columns per group (64 or 128)
  int32_t rope_group;   // MFMA path, MLA: group id of the rope band (-1 for GQA)
  double rope_base;
  int32_t page_shift;   // log2(page_size) when it is a power of two, else -1
  int32_t xcd_window_log2;  // MFMA path: log2 of the workgroups an XCD takes in a row (0: plain order)
  int64_t layer_tasks;  // > 0: layer-major task order, this many tasks per layer (task0 within a layer)
  int32_t mrope[3];     // rotary pairs following the t, h, w offsets (all 0: every pair follows t)
  int32_t phase_blocks; // per-token cos/sin table kernel: workgroups per chunk
};

// A small dense batch travels as a kernel argument instead: the dispatch carries the header
// and up to kInlineChunks compact chunk records, so the call needs neither the staging copy
// nor the copy-in kernel. Compact records hold what a dense chunk uses (no block table: that
// pointer is NULL; per-token cos/sin tables still live in the workspace) and at most
// kInlineFactors factors; other batches use the workspace.
constexpr int kInlineFactors = 2;
struct DevChunkInline {
  const void* src[2];
  void* dst[2];
  int64_t src_ls;
  int64_t dst_ls;
  int64_t delta;
  int64_t task0;
  int32_t T;
  uint32_t flags;
  int32_t slot0;
  int32_t ntb;
  int32_t tb_tokens;
  // small counts in 16 bits (column groups <= 2^20 / 64 by the layout checks)
  int16_t nstreams;
  int16_t ngroups;
  int16_t group0;
  int16_t stream_tensor[2];
  int16_t nfac;
  const int32_t* pages;      // always NULL here (dense destinations)
  const int32_t* positions;  // per-token offsets (KAMERA_POSITIONS), caller's device memory
  const float* phase;        // their cos/sin table in the workspace, or NULL
  DevFactor fac[kInlineFactors];
};
static_assert(sizeof(DevChunkInline) == 224, "compact chunk record layout");
constexpr int kInlineChunks = 16;
struct InlineBatch {
  DevHeader hd;
  DevChunkInline ch[kInlineChunks];
};
// kernel arguments, with the runtime's 256 bytes of implicit ones, stay within 4 KB
static_assert(sizeof(InlineBatch) + 256 <= 4096, "kernel arguments are limited to 4 KB");

// Scratch array of the allocation-free entry point (one per device, in kamera_kernels.hip):
// it stands in for the caller's workspace, so it holds at most this many bytes of packed
// batch, block tables and per-token cos/sin tables.
constexpr size_t kNoallocScratchBytes = size_t(4) << 20;

}  // namespace kamera
