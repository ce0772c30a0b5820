/*
 * kamera.h - C ABI of the Kamera position-free KV reuse operator on AMD gfx950.
 *
 * The operator (Kamera preprint, "Kamera: Unified Position-Invariant Multimodal
 * KV Cache for Training-Free Reuse", Eq. 1 in §1; stated cleanly as Eq. 1 in §2
 * of the page's Dutch summary) rebuilds a cached chunk's KV at a new position:
 *
 *     KV^(B|A) = R(delta) . KV(B|empty) + U_m V_m^T
 *
 *   R(delta)   exact RoPE phase re-rotation of the stored keys' rotary band by
 *              delta = p1 - p0 (preprint §3 "Relocate"); V and the MLA latent
 *              c_KV are never rotated.
 *   U_m V_m^T  rank-m conditioning patch, stored as the two tall factors
 *              U*Sigma [T][m] and V [width][m] (preprint App. A: the compile
 *              listing keeps U[:, :m]*S[:m] and the top-m right singular
 *              vectors; the serve listing applies U @ V^T), added after the
 *              rotation (preprint App. A serve listing).
 *
 * Layout families (preprint §3, Fig. 2):
 *   KAMERA_GQA  rows of K and of V, F = num_kv_heads * head_dim; every key head
 *               is one rotary band of head_dim columns (MHA = GQA with one KV
 *               head per query head). K and V may each carry factors.
 *   KAMERA_MLA  one row per token, F = latent_dim + rope_dim: the latent c_KV
 *               followed by the decoupled k_rope band, the only rotated part.
 *               Factors may cover any column range of that row (the preprint
 *               patches the latent and adds a small k_rope-band patch).
 *
 * Rotary convention: theta_i = rope_base^(-2i/d_rot), phi_i = delta * theta_i
 * formed in fp64; a pair (a, b) becomes (a cos phi - b sin phi,
 * a sin phi + b cos phi). NEOX pairs column i with i + d_rot/2 of the band,
 * GPTJ pairs 2i with 2i+1. Arithmetic is fp32 (cos/sin rounded once from fp64,
 * patch products accumulated in fp32); each output is rounded once to the
 * storage dtype (bf16: round-to-nearest-even).
 *
 * Memory and ownership
 *   - All tensor pointers are DEVICE pointers owned by the caller; element
 *     type is the layout dtype; rows are contiguous (row stride F elements).
 *   - Block tables and descriptor arrays are HOST memory, read only during the
 *     call; they may be freed or reused as soon as the call returns.
 *   - The caller supplies a device workspace of at least
 *     kamera_workspace_bytes(...) bytes; the library copies the packed batch
 *     description there (stream-ordered). Calls on the same stream may reuse
 *     one workspace (each call's copy-in runs after the previous call's work);
 *     a call on another stream must not use it until the work enqueued on
 *     `stream` has finished.
 *   - `stream` is a hipStream_t (NULL: the null stream). Work is enqueued
 *     asynchronously and the device is never synchronised, with one bound on
 *     how far the host runs ahead: a call that stages its batch (below) takes
 *     the next of 8 staging slots per device, and if that slot's previous
 *     copy-in (8 staged calls earlier, on any stream) has not yet run on the
 *     GPU, the call blocks the calling thread until it has.
 *   - The library never allocates device memory. It keeps a ring of 8 pinned,
 *     device-mapped host staging buffers per device (allocated with
 *     hipHostMalloc on first use, grown when a batch does not fit, kept until
 *     the process ends); a small copy-in kernel on `stream` moves each packed
 *     batch into the workspace. A one-shot
 *     kamera_rehydrate_batched / kamera_rehydrate call on a small dense batch (at
 *     most 16 chunks, none with a block table or with more than two factors under
 *     KAMERA_PATCH) instead passes the packed batch as the kernels' argument; the
 *     workspace then receives only the cos/sin tables of KAMERA_POSITIONS chunks
 *     (it is still validated, so both routes accept the same arguments). Such a
 *     call makes no HIP call besides its kernel launches, so it may itself be
 *     recorded in a captured graph; a call that stages its batch may not (a
 *     replay would read a staging buffer that later calls reuse): record
 *     kamera_plan_launch instead.
 *
 * Errors
 *   Every entry point returns a kamera_status. Arguments are validated on the
 *   host before anything is enqueued; on a validation error nothing is
 *   enqueued, and kamera_last_error() (thread-local) describes the first
 *   problem found. KAMERA_E_HIP reports a failed HIP call (staging, launch);
 *   a call makes up to three launches in order (copy-in, cos/sin tables,
 *   operator), so KAMERA_E_HIP can follow the successful enqueue of the
 *   earlier ones, which then run on the stream. Faults inside a kernel surface
 *   on the stream like any other HIP error.
 */
#ifndef KAMERA_H_
#define KAMERA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum kamera_status {
  KAMERA_OK = 0,
  KAMERA_E_NULL = 1,        /* a required pointer is NULL                               */
  KAMERA_E_SHAPE = 2,       /* a dimension, count or stride is out of range              */
  KAMERA_E_DTYPE = 3,       /* unknown dtype                                             */
  KAMERA_E_RANK = 4,        /* patch rank out of range for this layout                   */
  KAMERA_E_DELTA = 5,       /* |delta| >= 2^31                                           */
  KAMERA_E_PAGE = 6,        /* page id outside [0, num_pages) or slot0 outside the page  */
  KAMERA_E_OVERLAP = 7,     /* two chunks of one batch write the same pool slot          */
  KAMERA_E_ALIGN = 8,       /* a pointer is not aligned to its element size              */
  KAMERA_E_WORKSPACE = 9,   /* workspace NULL or smaller than kamera_workspace_bytes()   */
  KAMERA_E_UNSUPPORTED = 10,/* unknown family/pairing/flag, or a layout not supported    */
  KAMERA_E_HIP = 11         /* a HIP runtime call failed                                 */
} kamera_status;

enum { KAMERA_GQA = 0, KAMERA_MLA = 1 };
enum { KAMERA_F32 = 0, KAMERA_BF16 = 1 };
enum { KAMERA_NEOX = 0, KAMERA_GPTJ = 1 };

/* chunk flags */
enum {
  KAMERA_PATCH = 1u,     /* add the chunk's factors (else rotation only; V, c_KV copied as stored) */
  KAMERA_IN_PLACE = 2u,  /* read the rows from the destination itself and write them back       */
  KAMERA_POSITIONS = 4u  /* rotate token t by its own offsets positions[t] (per-token re-anchoring,
                            QV-PIC Eq. 2) instead of the chunk-wide delta                        */
};

enum { KAMERA_MAX_FACTORS = 4, KAMERA_MAX_RANK = 256 };

/* Unit that adds the rank-m patch in the bf16 kernel (64- or 128-wide heads, or MLA rows
 * with a 64-wide rope band); every other layout runs a plain fp32 FMA kernel.
 *   AUTO  the library's choice: the matrix cores (v_mfma_f32_16x16x32_bf16), measured as
 *         fast or faster than the VALU form at every rank (1 to 64) on the 28-layer
 *         4 x 128 GQA batch;
 *   MFMA  the matrix cores; KAMERA_E_UNSUPPORTED if the batch cannot run on that kernel;
 *   VALU  vector ALU dot products (v_dot2c_f32_bf16 with row broadcasts of the V factor),
 *         built for bf16 GQA/MHA with 128-wide heads, at most 64 ranks per column group and
 *         no KAMERA_POSITIONS chunk; else KAMERA_E_UNSUPPORTED.
 * The two units accumulate in a different order; both meet the same tolerance. */
enum { KAMERA_PATCH_UNIT_AUTO = 0, KAMERA_PATCH_UNIT_MFMA = 1, KAMERA_PATCH_UNIT_VALU = 2 };

typedef struct kamera_layout {
  int32_t family;        /* KAMERA_GQA or KAMERA_MLA                                      */
  int32_t dtype;         /* KAMERA_BF16 or KAMERA_F32 (all tensors of a call share it)    */
  int32_t num_layers;    /* L >= 1                                                        */
  int32_t num_kv_heads;  /* GQA: H_kv >= 1                                                */
  int32_t head_dim;      /* GQA: even, in [2, 512]; the rotary band is the whole head     */
  int32_t latent_dim;    /* MLA: c_KV width >= 0                                          */
  int32_t rope_dim;      /* MLA: k_rope width, even, in [2, 512]                          */
  int32_t pairing;       /* KAMERA_NEOX or KAMERA_GPTJ                                    */
  int32_t page_size;     /* tokens per pool page (>= 1); used by paged destinations       */
  int32_t patch_unit;    /* KAMERA_PATCH_UNIT_*: which unit adds the patch (see below)     */
  double rope_base;      /* RoPE base (> 0, finite), e.g. 1e4 or 1e6                      */
  int32_t mrope_section[3];  /* KAMERA_POSITIONS chunks: rotary pairs driven by the t, h and w
                                offsets, blocked in that order (sum = d_rot / 2, e.g. 16, 24, 24
                                for a 128-wide head); all 0: every pair follows t (1-D RoPE)    */
  int32_t reserved2;     /* must be 0                                                     */
} kamera_layout;

/* One stored factor pair of a chunk (preprint App. A: U[:, :m]*S[:m] and V_m; the
 * patch added to the rows is U V^T). Both factors keep a row's m coefficients
 * contiguous: V is the transpose of the V^T [m][width] of Fig. 2(d). */
typedef struct kamera_factor {
  const void* u;         /* device [L - layer0][T][rank]: U*Sigma, row-major               */
  const void* v;         /* device [L - layer0][width][rank]: V, row-major                 */
  int32_t tensor;        /* 0: K (GQA) or the MLA row; 1: V (GQA only)                     */
  int32_t col0;          /* first patched column of that tensor's row                     */
  int32_t width;         /* patched columns [col0, col0 + width), within the row          */
  int32_t rank;          /* m, 0 <= m <= KAMERA_MAX_RANK (0: no-op)                        */
  int32_t layer0;        /* layers below layer0 carry no factor (layer-sparse patches)    */
  int32_t reserved;      /* must be 0                                                     */
} kamera_factor;

/* One chunk to relocate/rehydrate across all L layers. */
typedef struct kamera_chunk {
  int32_t num_tokens;          /* T >= 0 (0: nothing to do)                                   */
  uint32_t flags;              /* KAMERA_PATCH | KAMERA_IN_PLACE | KAMERA_POSITIONS            */
  int64_t delta;               /* signed position shift p1 - p0, |delta| < 2^31 (not used by
                                  KAMERA_POSITIONS chunks, which turn each token by its own
                                  offsets)                                                    */
  const void* k_src;           /* device [L][T][F] canonical K (MLA: the row); unused in place */
  const void* v_src;           /* device [L][T][F] canonical V (GQA); unused for MLA/in place */
  int64_t src_layer_stride;    /* elements between layers of k_src/v_src; 0 means T*F          */
  void* k_dst;                 /* dense destination [L][T][F] when block_table == NULL         */
  void* v_dst;                 /* (GQA only)                                                   */
  int64_t dst_layer_stride;    /* elements between layers of k_dst/v_dst; 0 means T*F          */
  const int32_t* block_table;  /* HOST page ids; token t lives at slot s = slot0 + t, page
                                  block_table[s / page_size], offset s % page_size of the pool;
                                  NULL selects the dense destination                          */
  const int32_t* positions;    /* KAMERA_POSITIONS: DEVICE [T][3] int32 offsets (t, h, w) of each
                                  token, |offset| < 2^31; read on `stream` (stream-ordered, like
                                  every device input) by the upload of the batch, which turns
                                  them into a cos/sin table in the workspace; a plan relaunched
                                  later does not read them again. Pair i of token t turns by
                                  positions[t][section(i)] * theta_i. Ignored without the flag */
  int32_t slot0;               /* 0 <= slot0 < page_size                                       */
  int32_t num_factors;         /* 0 .. KAMERA_MAX_FACTORS                                      */
  kamera_factor factors[KAMERA_MAX_FACTORS];
} kamera_chunk;

/* Paged KV pool (preprint §6: the rebuilt KV is written into the engine's pool). */
typedef struct kamera_pool {
  void* k_pool;            /* device [L][num_pages][page_size][F] (MLA: the rows)          */
  void* v_pool;            /* device, same shape (GQA only)                                 */
  int32_t num_pages;       /* pages per layer                                              */
  int32_t reserved;        /* must be 0                                                    */
  int64_t layer_stride;    /* elements between layers; 0 means num_pages*page_size*F       */
} kamera_pool;

/* Launch summary produced by kamera_plan_upload and consumed by kamera_plan_launch. */
typedef struct kamera_plan {
  void* workspace;         /* device workspace holding the packed batch                    */
  int64_t num_tasks;       /* wave tasks of the main kernel (0: nothing to launch)         */
  int32_t kernel;          /* 0 none, 1 MFMA bf16 path, 2 generic VALU path                */
  int32_t variant;         /* register-budget instantiation of the chosen kernel           */
  int32_t num_chunks;
  int32_t reserved[9];
} kamera_plan;

/* Bytes of device workspace needed for a batch of `num_chunks` chunks whose block
 * tables hold `total_block_table_entries` page ids in total and none of which has
 * KAMERA_POSITIONS (those also need a cos/sin table; use kamera_batch_workspace_bytes). */
size_t kamera_workspace_bytes(int32_t num_chunks, int64_t total_block_table_entries);

/* Bytes of device workspace needed for exactly this batch (block tables and the per-token
 * cos/sin tables of KAMERA_POSITIONS chunks included; a table holds (cos, sin) in fp32 for
 * every rotary pair of every token, tokens rounded up to a multiple of 16); 0 if the
 * arguments are invalid. */
size_t kamera_batch_workspace_bytes(const kamera_layout* layout, const kamera_chunk* chunks,
                                    int32_t num_chunks);

/* Rotation-only relocation in place (preprint §5: sliding-window survivors need only
 * R(delta)): rotates the K rotary bands (GQA) or the k_rope band (MLA) of tokens
 * [0, num_tokens) stored in `pool`; V and c_KV are neither read nor written.
 * block_table (HOST) maps slots as in kamera_chunk; NULL maps slot s to pool row s
 * (page s / page_size, offset s % page_size), i.e. the pool as dense rows. Either way the
 * workspace needs kamera_workspace_bytes(1, pages spanned by slots [slot0, slot0 +
 * num_tokens)) bytes. */
kamera_status kamera_relocate(const kamera_layout* layout, const kamera_pool* pool,
                              const int32_t* block_table, int32_t slot0, int32_t num_tokens,
                              int64_t delta, void* workspace, size_t workspace_bytes, void* stream);

/* Eq. 1 for one chunk across all layers (preprint App. A serve listing). */
kamera_status kamera_rehydrate(const kamera_layout* layout, const kamera_chunk* chunk,
                               const kamera_pool* pool, void* workspace, size_t workspace_bytes,
                               void* stream);

/* Eq. 1 for a batch of chunks in one launch: each chunk has its own delta, patch flag,
 * factors and destination (dense rows, or pages of `pool`). Pool slots written by two
 * chunks of one batch are rejected (KAMERA_E_OVERLAP); dense destinations are the
 * caller's to keep disjoint, and so is every source row of an out-of-place chunk from
 * every row the batch writes (only KAMERA_IN_PLACE reads and writes the same rows: each
 * element is read, then written, by one lane). `pool` may be NULL when no chunk uses a
 * block table. */
kamera_status kamera_rehydrate_batched(const kamera_layout* layout, const kamera_chunk* chunks,
                                       int32_t num_chunks, const kamera_pool* pool,
                                       void* workspace, size_t workspace_bytes, void* stream);

/* Split form of kamera_rehydrate_batched: validate and upload the batch once, then
 * launch it any number of times (for example from a captured graph). The plan stays
 * valid while the workspace and every pointer it references are untouched. */
kamera_status kamera_plan_upload(const kamera_layout* layout, const kamera_chunk* chunks,
                                 int32_t num_chunks, const kamera_pool* pool, void* workspace,
                                 size_t workspace_bytes, void* stream, kamera_plan* plan);
kamera_status kamera_plan_launch(const kamera_plan* plan, void* stream);

/* Allocation-free form of kamera_rehydrate_batched, for callers that cannot allocate
 * device memory or pass a workspace: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation. Arguments, validation, semantics and results are
 * those of kamera_rehydrate_batched (the same kernels run), but the workspace is a
 * device array inside the library, one per GPU, of KAMERA_NOALLOC_SCRATCH_BYTES bytes,
 * held from the first call on that GPU until the process ends. The packed batch travels
 * to it as kernel arguments (small launches on `stream`), so the call allocates nothing
 * (no hipMalloc, no pinned staging, no copy engine) and never blocks the host.
 *   - A batch whose packed chunks, block tables and per-token cos/sin tables need more
 *     than KAMERA_NOALLOC_SCRATCH_BYTES (kamera_batch_workspace_bytes tells) is rejected
 *     with KAMERA_E_WORKSPACE before anything is enqueued.
 *   - Every call on one GPU reuses the same array: calls enqueued on one stream are
 *     ordered and safe; calls whose work may overlap in time on one GPU (other streams,
 *     other threads) race and must not be issued.
 *   - KAMERA_E_HIP after a successful validation can follow partly enqueued work (an
 *     earlier launch of the same call). */
enum { KAMERA_NOALLOC_SCRATCH_BYTES = 4194304 };
kamera_status kamera_rehydrate_batched_noalloc(const kamera_layout* layout, const kamera_chunk* chunks,
                                               int32_t num_chunks, const kamera_pool* pool, void* stream);

/* Patch builder (the compile step; preprint §2 Eq. 2 and App. A): forms the deficit
 *     Delta = x_cond - R(delta) x_canon
 * on columns [col0, col0 + width) of one layer's rows of one tensor and returns its
 * top-`rank` truncated SVD as the factors a kamera_factor takes: u_out = U[:, :m] Sigma
 * [num_tokens][rank] and v_out = V[:, :m] [width][rank], both in layout->dtype, and
 * sigma_out[rank] (fp64; may be NULL). The rotation is the operator's R(delta): the K
 * heads' bands (GQA, tensor 0) or the k_rope band (MLA); tensor 1 (GQA V) is not
 * rotated. x_cond and x_canon are [num_tokens][F] rows (F the layout's row width).
 * Everything is computed in fp64 on the device: Delta, G = Delta^T Delta, a
 * randomized range finder for G on a block of p = min(KAMERA_BUILD_MAX_SUBSPACE,
 * width, num_tokens) vectors followed by `iterations` power (subspace-iteration)
 * steps, and a Rayleigh-Ritz step. The result is the exact truncated SVD when
 * p = min(width, num_tokens); otherwise its residual approaches the Eckart-Young
 * optimum at a rate set by the gap sigma_{p+1}/sigma_m (16 is a good default). rank in [1, min(KAMERA_BUILD_MAX_RANK, width, num_tokens)], iterations in
 * [0, 64]. The workspace (256-byte aligned, kamera_build_workspace_bytes bytes) and the
 * outputs must not overlap the inputs. The call is stream-ordered and does not
 * synchronise; the library allocates nothing. */
enum { KAMERA_BUILD_MAX_RANK = 64, KAMERA_BUILD_MAX_SUBSPACE = 80, KAMERA_BUILD_MAX_ORBIT = 32 };
size_t kamera_build_workspace_bytes(int64_t num_tokens, int32_t width, int32_t rank);
kamera_status kamera_build_patch(const kamera_layout* layout, int32_t tensor, const void* x_cond,
                                 const void* x_canon, int64_t num_tokens, int64_t delta, int32_t col0,
                                 int32_t width, int32_t rank, int32_t iterations, void* u_out,
                                 void* v_out, double* sigma_out, void* workspace,
                                 size_t workspace_bytes, void* stream);

/* Orbit patch (preprint §5, reorder): one patch for every ordering of a cached set. The
 * chunk sat at offset deltas[k] in ordering k and x_conds[k] holds its conditioned rows
 * there; the factors are those of the mean deficit
 *     (1/K) sum_k (x_conds[k] - R(deltas[k]) x_canon)
 * (the ordering held out for evaluation is simply not passed). x_conds and deltas are
 * HOST arrays of num_orderings entries in [1, KAMERA_BUILD_MAX_ORBIT], read during the
 * call; each x_conds[k] is a device pointer laid out like x_canon. Everything else is
 * as kamera_build_patch (which is this call with one ordering). */
kamera_status kamera_build_orbit_patch(const kamera_layout* layout, int32_t tensor, int32_t num_orderings,
                                       const void* const* x_conds, const int64_t* deltas,
                                       const void* x_canon, int64_t num_tokens, int32_t col0,
                                       int32_t width, int32_t rank, int32_t iterations, void* u_out,
                                       void* v_out, double* sigma_out, void* workspace,
                                       size_t workspace_bytes, void* stream);

/* Streaming probes (measurement only, not part of the operator): nontemporal 16-byte
 * accesses, each workgroup over a contiguous 16 KB block. KAMERA_PROBE_COPY copies `bytes`
 * from src to dst; KAMERA_PROBE_READ reads `bytes` of src (dst: a device sink of at least
 * 4 KB, stored to only when the XOR of the words one thread read equals a fixed 16-byte value,
 * which keeps the loads from being dropped); KAMERA_PROBE_WRITE
 * fills `bytes` of dst with the 32-bit `value` (src unused). Timing them beside the operator
 * gives the HBM's practical rates for the access kinds the operator mixes. `bytes` a
 * multiple of 16, pointers 16-byte aligned; stream-ordered like every call. */
enum { KAMERA_PROBE_COPY = 0, KAMERA_PROBE_READ = 1, KAMERA_PROBE_WRITE = 2 };
kamera_status kamera_stream_probe(int32_t kind, const void* src, void* dst, size_t bytes, uint32_t value,
                                  void* stream);

/* Human-readable name of a status code (static storage). */
const char* kamera_status_string(kamera_status status);
/* Detail of the last error on the calling thread ("" if none). */
const char* kamera_last_error(void);
/* Library version string. */
const char* kamera_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KAMERA_H_ */
