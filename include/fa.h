/*
 * libfa - exact attention (FlashAttention forward and recompute backward)
 * for AMD Instinct MI355X (gfx950).
 *
 * What is computed, per batch b and head h, for query row i:
 *   S_ij  = scale * <Q_i, K_j>                       (scores; "Foundations",
 *            sections 4 and 9: query-key dot products scaled by 1/sqrt(d_k))
 *   S_ij  = -inf where key j is hidden                ("Worked examples", Cell D)
 *   O_i   = sum_j softmax(S_i)_j V_j                  ("Foundations", sections 7-8)
 *   lse_i = m_i + ln(sum_j exp(S_ij - m_i)),  m_i = max_j S_ij
 * computed by streaming K/V in blocks with the online max / normaliser
 * recurrence and one division at the end (the interactive explainer on
 * "The Flash Attention"; "Exercises", the block merges). Neither S nor the
 * probabilities P = softmax(S) are ever written to device memory.
 * A row with no visible key returns O_i = 0 and lse_i = -inf ("Worked
 * examples", Cell D2, the guard).
 *
 * Shapes: B batches, H query heads of Nq rows each, Hkv key/value heads of
 * Nk rows each, head dimension d. H must be a multiple of Hkv; query head h
 * attends to K/V head h / (H / Hkv) (Hkv = H: multi-head; 1 < Hkv < H:
 * grouped K/V heads; Hkv = 1: one K/V head shared by all). Attention runs per
 * query head exactly as for one head ("Question bank": the method is applied
 * per head unchanged inside multi-head attention). The plain entry points
 * (fa_fwd, fa_fwd_f32, fa_bwd) are the case Hkv = H, Nq = Nk = N.
 *
 * Visibility: key j is visible to query i iff j < kv_len_b and
 *   FA_MASK_CAUSAL:         j <= i + (Nk - Nq)
 *   FA_MASK_CAUSAL_STRICT:  j <  i + (Nk - Nq)
 * where kv_len_b = kv_lens[b] clamped to [0, Nk] (kv_lens == NULL means Nk).
 * With Nq = Nk this is the usual j <= i (j < i); with Nq < Nk the queries are
 * the last Nq of the Nk positions (a continuation after a cached prefix:
 * Nq = 1 sees every key). With Nq > Nk the first Nq - Nk queries see no key.
 * Padding hides keys only; every query row is computed.
 *
 * Layout: q, o (and dout, dq) are contiguous [B, H, Nq, d]; k, v (and dk, dv)
 * contiguous [B, Hkv, Nk, d] (d innermost); lse is contiguous [B, H, Nq]
 * float32. Pointers are device pointers allocated by the caller (the library
 * allocates and frees no device memory; fa_fwd_ex_noalloc's scratch is a
 * device array reserved when the library's code is loaded onto a GPU. On the
 * host it keeps a bounded cache of work plans and per-device occupancy,
 * guarded by mutexes). Tensor and workspace base pointers must be 16-byte
 * aligned.
 *
 * Asynchrony: each call validates its arguments on the host, enqueues its
 * kernels on `stream` (a hipStream_t; NULL = the null stream) and returns.
 * Faults inside a kernel surface at the caller's next synchronisation.
 *
 * Errors are returned before anything is enqueued:
 *   FA_ERR_INVALID_ARG  null tensor pointer, B/H/Hkv/Nq/Nk <= 0, H not a
 *                       multiple of Hkv, scale not finite or not > 0,
 *                       unknown mask_kind, an output overlapping an input;
 *   FA_ERR_UNSUPPORTED  d not supported (32, 64, 96, 128 and 256 are), a tensor pointer
 *                       not 16-byte aligned, sizes whose element count does
 *                       not fit the kernels' 32-bit row indices;
 *   FA_ERR_HIP          the launch itself failed (hipGetLastError).
 * kv_lens values outside [0, Nk] are clamped by the kernels.
 */
#ifndef LIBFA_FA_H
#define LIBFA_FA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* HIP's stream handle. hip_runtime_api.h defines hipStream_t as a pointer to
 * the opaque struct ihipStream_t; this header repeats that definition when
 * HIP's own header has not been included yet, so it builds without the HIP
 * headers and a hipStream_t passes to every call unchanged (NULL = the null
 * stream). Identical typedefs may be repeated (C11, C++). */
#ifndef HIP_INCLUDE_HIP_HIP_RUNTIME_API_H
struct ihipStream_t;
typedef struct ihipStream_t* hipStream_t;
#endif

#define FA_ABI_VERSION 12

typedef enum {
  FA_OK = 0,
  FA_ERR_INVALID_ARG = -1,
  FA_ERR_UNSUPPORTED = -2,
  FA_ERR_HIP = -3
} fa_status;

/* Element type of q, k, v, o (and dout, dq, dk, dv) in the _ex entry points. */
typedef enum {
  FA_DTYPE_BF16 = 0,  /* bfloat16; matrix products on bf16 MFMA, fp32 accumulation */
  FA_DTYPE_F16 = 1,   /* IEEE half; fp16 MFMA, fp32 accumulation */
  FA_DTYPE_F32 = 2    /* float32 throughout (forward only, no split) */
} fa_dtype;

typedef enum {
  FA_MASK_NONE = 0,          /* every key visible (subject to kv_lens) */
  FA_MASK_CAUSAL = 1,        /* key j visible to query i iff j <= i
                                (+ Nk - Nq) */
  FA_MASK_CAUSAL_STRICT = 2  /* key j visible to query i iff j < i (+ Nk - Nq):
                                the variant of "Worked examples", Cell D2,
                                whose first row sees no key (O = 0,
                                lse = -inf) */
} fa_mask_kind;

/*
 * Forward pass, bfloat16 inputs and output, float32 logsumexp.
 *   q, k, v : [B, H, N, d] bfloat16 (read)
 *   o       : [B, H, N, d] bfloat16 (written; round-to-nearest-even)
 *   lse     : [B, H, N] float32 (written; natural log; -inf for empty rows);
 *             may be NULL when the caller does not need it
 *   scale   : multiplies Q K^T; normally 1/sqrt(d)
 *   kv_lens : device int32 [B] valid key counts, or NULL
 *   stream  : the HIP stream the kernels are enqueued on (NULL = null stream)
 * Products Q K^T and P V run on bf16 matrix cores with float32 accumulation;
 * P is rounded to bfloat16 before the P V product. One workgroup computes
 * each block of 128 query rows over all of its visible keys; under the
 * causal mask with long key rows one workgroup computes two such blocks
 * (fa_fwd_tile_order).
 */
int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           int B, int H, int N, int d, float scale, int mask_kind,
           const int32_t* kv_lens, hipStream_t stream);

/*
 * Bytes of workspace fa_fwd_ex needs for these sizes on the current device
 * to split key ranges; 0 when its plan does not split any tile (then no
 * workspace is needed), for FA_DTYPE_F32, or for invalid arguments.
 */
size_t fa_fwd_ex_workspace_bytes(int B, int H, int Hkv, int Nq, int Nk, int d, int dtype,
                                 int mask_kind);

/*
 * fa_fwd for any element type (dtype: FA_DTYPE_BF16, FA_DTYPE_F16 or
 * FA_DTYPE_F32), grouped K/V heads (Hkv) and Nq != Nk (see the shapes and
 * visibility above), with optional split-KV: given a workspace, the key range
 * of the heaviest query tiles is split over several workgroups; each part
 * streams its share of the keys, stores its partial softmax state (row max,
 * both row sums, unnormalised output; fp32) in the workspace, and the last
 * part of a tile to finish merges all parts with the exact block merge
 * ("Exercises" of the interactive explainer "The Flash Attention", the block
 * merges) in part order. For grids too small to fill the GPU (few heads,
 * long rows, short decode queries over long caches) this spreads a tile over
 * several compute units. Same results as without the split up to rounding;
 * bitwise reproducible for a given device and shape.
 *   q, o      : [B, H, Nq, d];  k, v : [B, Hkv, Nk, d]; all of type dtype
 *   lse       : [B, H, Nq] float32 or NULL
 *   kv_lens   : device int32 [B] valid key counts (clamped to [0, Nk]), or NULL
 *   workspace : device memory, or NULL with workspace_bytes = 0 (no split).
 *               With fewer than fa_fwd_ex_workspace_bytes(...) bytes no tile
 *               is split. Its first 64 KiB hold arrival counters that must be
 *               zero before the first use; every completed call leaves them
 *               zero, for any later shape (the rest is scratch). Calls
 *               sharing a workspace must be ordered (same stream, or
 *               synchronised). It must not overlap any tensor argument.
 *               Not used with FA_DTYPE_F32.
 * With FA_DTYPE_F16 the probabilities are rounded to fp16 (not bf16) before
 * the P V product and O is written in fp16 (round-to-nearest-even).
 * Decode with grouped heads (Nq = 1, H > Hkv, no mask or the causal one;
 * 16-bit types): the H / Hkv query heads of a K/V head are launched as rows
 * of one query tile, so each K/V head is streamed once; the results are
 * those of the per-head launch up to the rounding of a different key split,
 * and fa_fwd_ex_workspace_bytes sizes the workspace for this launch.
 * Errors as fa_fwd, and FA_ERR_INVALID_ARG for an unknown dtype or for
 * workspace_bytes > 0 with a NULL workspace, FA_ERR_UNSUPPORTED for a
 * workspace not 16-byte aligned.
 */
int fa_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse,
              int B, int H, int Hkv, int Nq, int Nk, int d, int dtype, float scale,
              int mask_kind, const int32_t* kv_lens, void* workspace,
              size_t workspace_bytes, hipStream_t stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): fa_fwd_ex
 * with its split-KV workspace taken from a scratch array that the library
 * holds on each device instead of a caller-provided one. Same arguments,
 * results and plans as fa_fwd_ex given a large enough workspace (bitwise the
 * same outputs); no device memory is allocated or freed.
 * The scratch is FA_NOALLOC_SCRATCH_BYTES per GPU, reserved when the
 * library's device code is loaded onto that GPU and held until the process
 * ends. Every call on a GPU shares it and it keeps the last call's contents:
 * each call that splits first clears the arrival counters it uses (a small
 * kernel on `stream`, never a memset). Calls that overlap on one GPU race
 * for the scratch and give wrong results: order them (one stream, or
 * synchronised).
 * Errors as fa_fwd_ex; FA_ERR_UNSUPPORTED when the split plan for these
 * sizes needs more than FA_NOALLOC_SCRATCH_BYTES of workspace
 * (fa_fwd_ex_workspace_bytes tells), FA_ERR_HIP when the scratch's device
 * address cannot be obtained or a launch fails.
 */
#define FA_NOALLOC_SCRATCH_BYTES (64u << 20)
int fa_fwd_ex_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                      int B, int H, int Hkv, int Nq, int Nk, int d, int dtype, float scale,
                      int mask_kind, const int32_t* kv_lens, hipStream_t stream);

/*
 * The same contract with float32 q, k, v, o (float32 arithmetic throughout).
 */
int fa_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse,
               int B, int H, int N, int d, float scale, int mask_kind,
               const int32_t* kv_lens, hipStream_t stream);

/*
 * Bytes of device workspace fa_bwd needs for these sizes (caller-allocated,
 * at least 256-byte aligned; contents need not be initialised). For
 * fa_bwd_ex pass the query rows: fa_bwd_workspace_bytes(B, H, Nq, d).
 */
size_t fa_bwd_workspace_bytes(int B, int H, int N, int d);

/*
 * Backward pass of fa_fwd: given dO = dL/dO, returns dQ, dK, dV.
 * P is recomputed from Q, K and the saved lse (the "Question bank" answers:
 * S and P are recomputed rather than stored); the formulas are the standard
 * softmax derivative:
 *   P = exp(S - lse) (0 where hidden or lse = -inf),  D_i = sum_c dO_ic O_ic,
 *   dV = P^T dO,  dS = P * (dO V^T - D),  dQ = scale dS K,  dK = scale dS^T Q.
 *   q, k, v, o, dout : [B, H, N, d] bfloat16 (read); o is fa_fwd's output
 *   lse              : [B, H, N] float32 from fa_fwd (read)
 *   dq, dk, dv       : [B, H, N, d] bfloat16 (written)
 *   workspace        : fa_bwd_workspace_bytes(B, H, N, d) bytes of device memory
 */
int fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
           const void* dout, void* dq, void* dk, void* dv, void* workspace,
           int B, int H, int N, int d, float scale, int mask_kind,
           const int32_t* kv_lens, hipStream_t stream);

/*
 * fa_bwd for bf16 or fp16 tensors (dtype FA_DTYPE_BF16 or FA_DTYPE_F16;
 * FA_DTYPE_F32 returns FA_ERR_UNSUPPORTED), grouped K/V heads and Nq != Nk
 * (shapes as fa_fwd_ex):
 *   q, o, dout, dq : [B, H, Nq, d];  k, v, dk, dv : [B, Hkv, Nk, d]
 *   lse            : [B, H, Nq] float32 from fa_fwd / fa_fwd_ex
 *   workspace      : fa_bwd_workspace_bytes(B, H, Nq, d) bytes
 * dK and dV of a K/V head are the sums over the H / Hkv query heads that
 * share it (each such head uses the same K, V rows, so their gradient
 * contributions add).
 */
int fa_bwd_ex(const void* q, const void* k, const void* v, const void* o, const float* lse,
              const void* dout, void* dq, void* dk, void* dv, void* workspace,
              int B, int H, int Hkv, int Nq, int Nk, int d, int dtype, float scale,
              int mask_kind, const int32_t* kv_lens, hipStream_t stream);

/*
 * Host-only view of fa_fwd_ex's work plan (no device call): for Nq query
 * rows and Nk keys, BH = B*H query heads, head dimension d, mask_kind, `cus`
 * compute units and `occ` resident workgroups per compute unit, returns the
 * number of work items (0 = one item per query tile, no split) and copies up
 * to max_items of them to `items`, each
 *   tile | part << 9 | (nparts - 1) << 15 | slot_base << 21
 * (a plan has at most 512 items; a tile is split into at most 16 parts, or
 * 64 when the query rows are a single tile), in dispatch order; *nslots
 * receives the partial-state slots per head.
 * Query tiles are 128 rows; a tile's keys stream in blocks of 64 keys;
 * part p of n covers blocks [p * nb / n, (p + 1) * nb / n) of the tile's nb
 * blocks.
 * Returns FA_ERR_INVALID_ARG for invalid arguments.
 */
int fa_fwd_schedule(int Nq, int Nk, int BH, int d, int mask_kind, int cus, int occ,
                    uint32_t* items, int max_items, int* nslots);

/* Assignment of query tiles (128 rows) to workgroups; fa_fwd_tile_order. */
typedef enum {
  FA_FWD_ORDER_HEAVY_FIRST = 0,  /* one tile per workgroup, the tiles that see
                                    the most keys dispatched first; keys
                                    stream in ascending order */
  FA_FWD_ORDER_PAIRED = 1,       /* causal: workgroup r takes tile
                                    ntiles-1-r (keys ascending) and then tile
                                    r (keys descending), so every workgroup
                                    streams about ntiles+1 tiles' worth of
                                    key blocks and those of one head read the
                                    same two key blocks at a time */
  FA_FWD_ORDER_HEAD_SEQUENTIAL = 2 /* one tile per workgroup; each XCD (the
                                    workgroups of one residue of the id mod 8)
                                    runs its heads one after another, the
                                    heaviest tile of a head first */
} fa_fwd_order;

/*
 * Host-side view of the tile order fa_fwd and fa_fwd_ex use for Nq query
 * rows against Nk keys, BH = B*H query heads, head dimension d, dtype
 * (FA_DTYPE_BF16 or FA_DTYPE_F16) and mask_kind, on `cus` compute units with
 * `occ` resident workgroups per compute unit (cus = occ = 0: those of the
 * current device, which makes a device query; otherwise no device call).
 * When fa_fwd_ex splits key ranges (a workspace and fa_fwd_schedule > 0),
 * the split plan is used instead. Pairs are used under a causal mask when
 * one head's K and V (2 * Nk * d elements of 2 bytes) are at least 4 MB,
 * the L2 cache of one XCD, and BH * ceil(Nq / 128) / 2 workgroups still fill
 * every resident slot: streaming every tile from key 0 then fetches K and V
 * again from memory in proportion to Nq, while pairs keep the fetched bytes
 * a constant multiple of the inputs. Otherwise the heads run one after
 * another on each XCD when BH is a multiple of 8 and the BH * ceil(Nq / 128)
 * workgroups are at least 16 rounds of the cus * occ resident slots, so that
 * few heads' K and V share an XCD's L2 at a time; on smaller grids the tiles
 * go out item-major (all heads' heaviest tiles first), which balances the
 * last rounds. Outputs are bitwise the same in every order.
 * Returns an fa_fwd_order value, FA_ERR_INVALID_ARG for invalid arguments,
 * or FA_ERR_UNSUPPORTED for FA_DTYPE_F32.
 */
int fa_fwd_tile_order(int Nq, int Nk, int BH, int d, int dtype, int mask_kind, int cus, int occ);

/* Work order of the backward's gradient kernels; fa_bwd_tile_order. */
#define FA_BWD_DQ_HEAD_SEQUENTIAL 1    /* the dQ kernel runs each XCD's heads one after another */
#define FA_BWD_DKDV_HEAD_SEQUENTIAL 2  /* the dK/dV kernel does */

/*
 * Host-side view of the work order fa_bwd / fa_bwd_ex use for these sizes
 * (shapes as fa_bwd_ex) on `cus` compute units with `occ` resident
 * workgroups per compute unit (cus = occ = 0: the current device's compute
 * units and the kernels' own occupancy, two workgroups per compute unit, one
 * at d = 256). Each gradient kernel takes its tiles tile-major (every XCD
 * starts with the heaviest tiles of all its heads) unless its grid is at
 * least 16 rounds of the resident slots and its head count (B*H for dQ,
 * B*Hkv for dK/dV) a multiple of 8; then each XCD runs its heads one after
 * another, so that few heads' streamed operands share its L2 at a time. The
 * gradients are bitwise the same either way.
 * Returns a combination of FA_BWD_DQ_HEAD_SEQUENTIAL and
 * FA_BWD_DKDV_HEAD_SEQUENTIAL, or FA_ERR_INVALID_ARG / FA_ERR_UNSUPPORTED.
 */
int fa_bwd_tile_order(int B, int H, int Hkv, int Nq, int Nk, int d, int cus, int occ);

/*
 * Keys per streamed block that fa_fwd / fa_fwd_ex use for these sizes on the
 * current device (16-bit types; currently 64 for every supported shape), or
 * FA_ERR_INVALID_ARG / FA_ERR_UNSUPPORTED.
 */
int fa_fwd_block_keys(int B, int H, int Nq, int Nk, int d, int mask_kind);

/* Human-readable name of a status code (static storage). */
const char* fa_status_string(int status);

/* FA_ABI_VERSION of the library that was loaded. */
int fa_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LIBFA_FA_H */
