/*
 * libmoe -- routed-expert MoE layer forward behind an expert-slot cache, for AMD
 * Instinct MI355X (gfx950).  Plain C ABI: raw pointers, sizes and status codes.
 *
 * What the layer is (the pages describe an offloaded-MoE runtime; citations
 * name the page and its section):
 *   - a router picks a few experts per token (FreeToken linux guide, "MoE memory
 *     handling": DeepSeek-V4-Flash activates 6 of 256 routed experts per layer);
 *   - GPU memory holds expert slots, the whole routed pool stays in host RAM, and
 *     one LRU over those slots is shared by all MoE layers (same section, memory
 *     tier table and mechanism table; FreeToken GGUF page, "MoE backends",
 *     offload backend);
 *   - a missed expert is copied to GPU memory over PCIe and kept for reuse (same
 *     places); prefill streams the next layer's experts while the current layer
 *     runs (FreeToken linux guide, mechanism table, full-layer double buffering;
 *     FreeToken RTX 5090 page, memory-hierarchy paragraph).
 * Router form, expert form and the combine are not given on the pages; the
 * plain readings used are stated at each call.
 *
 * Conventions for every call:
 *   - OWNERSHIP: the caller owns every buffer passed in (device or host); the
 *     library allocates no device memory.  It owns only cache objects, their HIP
 *     events, pinned blocks returned by moe_pinned_alloc, and profiling events.
 *   - ERRORS: arguments are checked on the host before anything is enqueued; a
 *     call that returns non-OK has enqueued nothing.  moe_last_error() gives a
 *     thread-local message for the last non-OK status.  Asynchronous device
 *     faults surface at the caller's next synchronisation, as in HIP.
 *   - STREAMS: moe_stream is a hipStream_t (NULL = the null stream).  Kernel
 *     calls are asynchronous on their stream and run on the current device.
 *   - T == 0 is a valid no-op that returns MOE_OK.
 *   - DETERMINISM: identical inputs give bitwise identical outputs; no atomics
 *     decide positions or the order of any floating-point sum.
 *   - DTYPES: activations MOE_F32 or MOE_BF16 (bfloat16 bit patterns, uint16);
 *     weights MOE_F32, MOE_BF16 or MOE_INT4_G128.
 */
#ifndef MOE_H_
#define MOE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_API __attribute__((visibility("default")))

typedef int32_t moe_status;
enum {
    MOE_OK = 0,
    MOE_EINVAL = -1,    /* bad pointer, range or flag */
    MOE_ESHAPE = -2,    /* shape outside the supported set */
    MOE_EDTYPE = -3,    /* dtype combination not supported */
    MOE_ENOMEM = -4,    /* workspace too small or host allocation failed */
    MOE_EHIP = -5,      /* a HIP runtime call failed; text in moe_last_error() */
    MOE_ECAPACITY = -6, /* request set larger than the slot cache */
    MOE_ESTATE = -7     /* call out of order, or an eviction would hit an unread slot */
};

/* element type codes (an integer, so that any value a caller passes is well defined; values other
 * than these are rejected with MOE_EDTYPE) */
typedef int32_t moe_dtype;
enum { MOE_F32 = 0, MOE_BF16 = 1, MOE_INT4_G128 = 2 };
typedef void* moe_stream;

MOE_API const char* moe_last_error(void);
MOE_API const char* moe_version(void);

/* ------------------------------------------------------------------------------------------
 * Expert slots.  One slot holds one SwiGLU expert (W_g, W_u: [f, d]; W_d: [d, f]; rows are
 * outputs) in the kernel-ready layout below; the pinned host pool stores experts in the same
 * layout so that a cache fill is one contiguous copy per expert (the pages' FTW format keeps
 * expert banks in runtime layout for the same reason: FreeToken linux guide, setup section,
 * model-weight preparation).
 *
 * Layout: matrices are cut into blocks of 16 rows.  Gate/up blocks alternate (gate rows
 * 16b..16b+15, then up rows 16b..16b+15, for b = 0 .. f/16-1), followed by the W_d blocks.
 *   F32/BF16: a 16-row block is K/32 consecutive fragments of 16 rows x 32 inputs; inside a
 *     fragment, lane l (0..63) owns row l%16, inputs 8*(l/16) .. 8*(l/16)+7, stored as 8
 *     consecutive elements at element offset 8*l.
 *   INT4_G128: a 16-row block is K/128 fragments of 16 rows x 128 inputs (1024 bytes), then
 *     the block's scales as bf16 [16 rows][K/128].  In a fragment lane l owns 16 bytes at
 *     offset 16*l: row l%16, word s (0..3) holds inputs 32s + 8*(l/16) + (0..7); input pair
 *     (2p, 2p+1) of a word sits in bits [4p, 4p+4) and [16+4p, 20+4p).  A stored nibble u is
 *     the integer u - 8 in [-7, 7]; weight = (u - 8) * scale of its row and 128-group.
 * ------------------------------------------------------------------------------------------ */

/* Bytes of one packed expert (a multiple of 256).  0 if the shape/dtype is unsupported:
 * d, f multiples of 32 (F32/BF16) or of 128 (INT4_G128), 64 <= d, f <= 16384. */
MOE_API size_t moe_slot_bytes(int d, int f, moe_dtype w);

/* Pack one expert from the canonical row-major layout into a slot image (host memory).
 * F32/BF16: wg, wu [f][d], wd [d][f] in the weight dtype; sg, su, sd must be NULL.
 * INT4_G128: wg, wu [f][d/2], wd [d][f/2] bytes (element 2i low nibble of byte i, offset
 * binary); sg, su [f][d/128], sd [d][f/128] bf16 scale bits.  slot_out: moe_slot_bytes bytes. */
MOE_API moe_status moe_pack_expert(moe_dtype w, int d, int f, const void* wg, const void* wu,
                                   const void* wd, const void* sg, const void* su, const void* sd,
                                   void* slot_out);

/* ------------------------------------------------------------------------------------------
 * moe_route -- router scores, top-k and gates (FreeToken linux guide, "MoE memory handling":
 * the router activates a subset of experts per token).
 *   logits[t,e] = x[t,:] . w_router[e,:] (+ bias[e]) in binary32, in one fixed order: row
 *     elements are split into 64 contiguous segments of d/64; each segment is summed from +0
 *     in ascending index with every product and sum rounded to nearest even (no fused
 *     multiply-add for F32 inputs; for BF16 inputs products are exact); the 64 segment sums
 *     are joined pairwise, neighbours first (a tree of 6 levels); the bias is added last.
 *   topk_idx[t,:]  the k largest logits, largest first, equal logits -> lower expert id first.
 *   topk_w[t,j]    softmax over all E logits renormalised over the selected k, i.e.
 *                  exp(l_j - l_max) / sum_{i in S} exp(l_i - l_max), formed in binary64 and
 *                  rounded once to binary32.
 * With forced_idx (a device [T,k] int32 array of distinct ids in [0,E), e.g. a replayed
 * routing trace), the selection is skipped: topk_idx = forced_idx and the gates are computed
 * at those ids in the given order.  Out-of-range forced ids give unspecified gates.
 *   x [T,d] act dtype; w_router [E,d] act dtype; bias [E] f32 or NULL (device pointers).
 *   logits [T,E] f32 (device, required: it is the selection's input as well as an output).
 * Shapes: 1 <= k <= E <= 1024, d a multiple of 64, d <= 16384. */
MOE_API moe_status moe_route(const void* x, moe_dtype act, int T, int d, const void* w_router,
                             const float* bias, int E, int k, const int32_t* forced_idx,
                             int32_t* topk_idx, float* topk_w, float* logits, moe_stream s);

/* ------------------------------------------------------------------------------------------
 * moe_permute -- group the T*k (token, choice) pairs by expert (pages silent; the plain
 * reading is a stable counting sort of the flat ids t*k + j):
 *   counts[e] pairs routed to e; offsets[0..E] exclusive prefix sum (offsets[E] = T*k);
 *   perm[p] flat pair index at sorted position p (stable: ascending flat index within an
 *   expert); inv_perm[i] sorted position of flat pair i.  All int32, device.
 * topk_idx must hold ids in [0, E).  T*k <= 2^24.  ws: device scratch of moe_permute_workspace_bytes
 * bytes (4-byte aligned) or NULL/0, see below. */
MOE_API moe_status moe_permute(const int32_t* topk_idx, int T, int k, int E, int32_t* counts,
                               int32_t* offsets, int32_t* perm, int32_t* inv_perm, void* ws,
                               size_t ws_bytes, moe_stream s);
/* Device scratch moe_permute (and moe_route_permute) can use for T*k pairs over E experts: the
 * per-workgroup counts of a sort split over several workgroups, used when T*k is large (more than
 * 8192 pairs).  0 when one workgroup sorts.  With a smaller or NULL ws the call still works (one
 * workgroup sorts); the results are the same bits either way. */
MOE_API size_t moe_permute_workspace_bytes(int T, int k, int E);

/* ------------------------------------------------------------------------------------------
 * moe_route_permute -- moe_route followed by moe_permute on its topk_idx, as one call
 * (FreeToken linux guide, "MoE memory handling": per layer the router picks the experts and
 * the runtime gathers each expert's tokens).  Every output is bitwise what the two calls give
 * for the same arguments: logits, topk_idx, topk_w as moe_route; counts, offsets, perm,
 * inv_perm as moe_permute.  For T = 1 one block selects, gates and places the k pairs by expert,
 * one launch fewer than the two calls; other shapes run the two calls' kernels (ws and ws_bytes
 * go to moe_permute).  Arguments, shapes, ownership and errors are those of the two calls; a
 * non-OK status means nothing was enqueued.
 * With T = 0 only counts and offsets are written (zeros). */
MOE_API moe_status moe_route_permute(const void* x, moe_dtype act, int T, int d, const void* w_router,
                                     const float* bias, int E, int k, const int32_t* forced_idx,
                                     int32_t* topk_idx, float* topk_w, float* logits, int32_t* counts,
                                     int32_t* offsets, int32_t* perm, int32_t* inv_perm, void* ws,
                                     size_t ws_bytes, moe_stream s);

/* ------------------------------------------------------------------------------------------
 * moe_expert_ffn_grouped -- every expert with n_e > 0 runs once on its n_e rows (SwiGLU, the
 * plain reading of the expert form: h = silu(x W_g^T) * (x W_u^T), y = h W_d^T, no biases).
 * Expert e's weights are read from the slot slot_of_expert[e] of slot_pool (FreeToken GGUF
 * page, offload backend: expert slots on the GPU), i.e. at slot_pool + slot * slot_stride.
 *   x [T,d] act; perm, offsets, counts from moe_permute (offsets must be the exclusive prefix
 *   sums of counts, as moe_permute writes them: an expert's first row may be taken from either);
 *   slot_of_expert [E] int32 (a device
 *   row of the slot table; MOE_SLOT_ELSEWHERE (-2) means the expert's rows of y_perm are
 *   produced elsewhere, e.g. on the host (hybrid miss handling), and are left untouched; any
 *   other slot outside [0, n_slots) sets the workspace status word to 1 and that expert's rows
 *   to 0 -- it never reads outside the pool).
 *   shared_w: an always-on shared expert packed like a slot (or NULL); it runs on all T tokens.
 *   y_perm [T*k (+T if shared_w), d] of type y_dtype: row p = expert output of sorted pair p; rows
 *   T*k+t hold the shared expert's output for token t.  y_dtype F32 keeps the binary32 sums;
 *   BF16 (only with act BF16) rounds each output once to bf16 (nearest even), which halves the
 *   bytes the grouped call writes and the combine reads: the prefill reading, where the
 *   intermediate rows may be bf16 like h.  Any other value: MOE_EDTYPE.
 *   ws: device workspace of at least moe_workspace_bytes(...) bytes, zero-filled before its
 *   first use.  Its first 4 bytes are a sticky int32 status word (0 = no error).
 * Intermediate h is rounded to bf16 when act is BF16 (binary32 when act is F32). */
#define MOE_SLOT_ELSEWHERE (-2)
/* Above 64 tokens (prefill) the experts run on the matrix-core grouped GEMM, which feeds int4
 * weights to the matrix cores as bf16(q * s).  Experts holding at most moe_prefill_gemv_tokens(w)
 * tokens instead run on the decode kernels (their weights are streamed once and no 128-token tile
 * is left mostly empty); those take exact q * s products.  For bf16 weights this applies only to
 * calls with T*k <= 64*E.  The shared expert always holds T tokens.  0 = every expert on the GEMM. */
MOE_API int moe_prefill_gemv_tokens(moe_dtype w);
MOE_API size_t moe_workspace_bytes(int T, int d, int f, int E, int k, int has_shared,
                                   moe_dtype act, moe_dtype w);
MOE_API moe_status moe_expert_ffn_grouped(const void* x, moe_dtype act, int T, int d, int f, int E,
                                          int k, const int32_t* perm, const int32_t* offsets,
                                          const int32_t* counts, const int32_t* slot_of_expert,
                                          int n_slots, const void* slot_pool, size_t slot_stride,
                                          moe_dtype w, const void* shared_w, void* y_perm,
                                          moe_dtype y_dtype, void* ws, size_t ws_bytes, moe_stream s);

/* moe_expert_ffn_grouped for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same kernels, with the
 * workspace replaced by a scratch array the library holds per GPU (MOE_NOALLOC_SCRATCH_BYTES, on
 * each GPU it runs on, until the process ends).  The call allocates nothing.
 *   status: device int32, the sticky status word of the workspace (the caller zero-fills it before
 *   its first use), or NULL: an absent slot then still gives zero rows but is not reported.
 *   A call whose moe_workspace_bytes(...) exceeds MOE_NOALLOC_SCRATCH_BYTES returns MOE_ENOMEM with
 *   nothing enqueued.  Every call on one GPU uses that GPU's one array: calls that may run at the
 *   same time on one GPU (streams not ordered with each other) race and give undefined outputs.
 * Other arguments, outputs and errors as moe_expert_ffn_grouped. */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
MOE_API moe_status moe_expert_ffn_grouped_noalloc(const void* x, moe_dtype act, int T, int d, int f, int E,
                                                  int k, const int32_t* perm, const int32_t* offsets,
                                                  const int32_t* counts, const int32_t* slot_of_expert,
                                                  int n_slots, const void* slot_pool, size_t slot_stride,
                                                  moe_dtype w, const void* shared_w, void* y_perm,
                                                  moe_dtype y_dtype, int32_t* status, moe_stream s);

/* ------------------------------------------------------------------------------------------
 * moe_combine -- gate-weighted sum (pages silent on the form; plain reading):
 *   y[t,:] = sum_{j=0..k-1} topk_w[t,j] * y_perm[inv_perm[t*k+j], :]  (+ y_perm[T*k+t, :] if
 *   has_shared), j ascending, binary32 accumulation, one final rounding to out (F32 or BF16,
 *   round to nearest even).  y_perm holds y_dtype elements (F32, or BF16 as
 *   moe_expert_ffn_grouped writes them with y_dtype BF16; widened exactly before the products). */
MOE_API moe_status moe_combine(const void* y_perm, moe_dtype y_dtype, const float* topk_w,
                               const int32_t* inv_perm, int T, int k, int d, int has_shared, void* y,
                               moe_dtype out, moe_stream s);

/* ------------------------------------------------------------------------------------------
 * Expert-slot cache shared by all MoE layers (FreeToken linux guide, "MoE memory handling":
 * one LRU over GPU expert slots across the MoE layers, full pool in host RAM; a missed expert
 * is copied over PCIe from pinned memory and kept -- FreeToken GGUF page, offload backend;
 * prefill double-buffers the next layer -- mechanism table).
 * Keys are (layer, expert).  A request set S is processed as: resident members are hits and
 * become most recent in ascending id; then each other member, ascending, is a miss that takes
 * the lowest-numbered free slot, else evicts the least recently used entry and reuses its slot.
 * |S| > n_slots -> MOE_ECAPACITY.  Slots handed out by a lookup/prefetch of layer l stay pinned
 * until moe_cache_mark_read(l); evicting a pinned slot is refused with MOE_ESTATE (it never
 * happens when n_slots >= 2E with the prefill order prefetch(l+1) -> mark_read(l)).
 * Policy-only mode: slot_pool == NULL (then slot_table and host_expert must be NULL) keeps the
 * bookkeeping and statistics and makes no HIP call at all (simulations, CPU tests).
 * The cache object is not thread-safe; mark_read events must come from one compute stream. */
typedef struct moe_cache moe_cache;

/* slot_pool: device, n_slots * slot_stride bytes.  slot_table: device int32 [L*E]; this call
 * sets it to -1 (synchronously) and the cache keeps it equal to its own table.
 * host_expert: [L*E] host pointers to pinned slot images of slot_stride bytes (layer-major).
 * The arrays pointed to must stay valid until moe_cache_destroy. */
MOE_API moe_status moe_cache_create(int L, int E, int n_slots, size_t slot_stride, void* slot_pool,
                                    int32_t* slot_table, const void* const* host_expert,
                                    moe_cache** out);
/* Decode lookup of layer `layer`: ids (host, n distinct ids in [0,E)).  slots_out[i] (host) is
 * the slot of ids[i] once pending fills are done; *n_miss_out the number of misses.  Host only:
 * the caller has the ids on the host (copy topk_idx back and synchronise first). */
MOE_API moe_status moe_cache_lookup(moe_cache* c, int layer, const int32_t* ids, int n,
                                    int32_t* slots_out, int32_t* n_miss_out);
/* Enqueue the copies of all pending misses on `copy` (each waits for the last recorded read of
 * the slot it overwrites), then the slot-table update; `compute` waits for them.  A failed copy
 * enqueue leaves the failed entries non-resident (-1) and returns MOE_EHIP. */
MOE_API moe_status moe_cache_fill(moe_cache* c, moe_stream copy, moe_stream compute);
/* moe_cache_fill for hybrid miss handling (FreeToken linux guide, mechanism table: a miss is
 * streamed, run on the CPU, or both): the pending misses of the last request whose expert ids are
 * in `later` are copied after the others, and `compute` waits only for the others (those experts
 * run elsewhere for this request, e.g. moe_cpu_expert_ffn).  The next fill, prefetch or resize
 * makes `compute` wait for the deferred copies before anything else reads the slots. */
MOE_API moe_status moe_cache_fill_split(moe_cache* c, const int32_t* later, int n_later, moe_stream copy,
                                        moe_stream compute);
/* Prefill: request all E experts of `layer` (prefill statistics) and fill on `copy`; `compute`
 * waits for the copies (enqueue the current layer's kernels on `compute` first, then prefetch
 * the next layer, so that the copies overlap the current layer). */
MOE_API moe_status moe_cache_prefetch_layer(moe_cache* c, int layer, moe_stream copy,
                                            moe_stream compute);
/* Record on `compute` the point after which layer `layer`'s pinned slots are no longer read
 * (call after enqueueing the layer's kernels); unpins them. */
MOE_API moe_status moe_cache_mark_read(moe_cache* c, int layer, moe_stream compute);
/* Elastic capacity (FreeToken linux guide, mechanism table: the cache is resized at scheduler
 * safe points; FreeToken RTX 5090 page, reconfiguration).  Allowed only at a safe point: every
 * layer marked read and no fill pending (else MOE_ESTATE).  Growing adds free slots C..n-1 (the
 * slot pool given at creation must hold n slots).  Shrinking keeps the n most recently used
 * entries: LRU entries are evicted, oldest first; each kept entry in a slot >= n is copied
 * device-to-device to the lowest free slot below n (kept entries taken in ascending old-slot
 * order) on `copy`, after the last recorded read of its new slot; then the slot table is
 * updated and `compute` waits.  A slot removed by a shrink and added back later is refilled only
 * after every read recorded before the shrink.  Moves appear in moe_cache_copy_log with the
 * third field = -2 - source slot.  Outputs never depend on the capacity. */
MOE_API moe_status moe_cache_resize(moe_cache* c, int n_slots, moe_stream copy, moe_stream compute);
/* out[0..5] = decode accesses, decode hits, decode misses, prefill accesses, prefill misses,
 * bytes copied host -> device. */
MOE_API moe_status moe_cache_stats(const moe_cache* c, int64_t out[6]);
/* Hit (1) / miss (0) flag of every access so far, in request order, ascending id within a
 * request; writes min(cap, total) flags and sets *n to the total. */
MOE_API moe_status moe_cache_trace(const moe_cache* c, uint8_t* hitmiss, int64_t cap, int64_t* n);
/* Host view of the slot table: *slot = slot of (layer, expert) or -1. */
MOE_API moe_status moe_cache_slot_of(const moe_cache* c, int layer, int expert, int32_t* slot);
/* Copy plan so far (test and tracing aid): for the i-th expert copy enqueued (or, in
 * policy-only mode, simulated) out[3i..3i+2] = slot, key (layer*E + expert), and the read
 * sequence number the copy waited for (-1 = none; sequence numbers count mark_read calls from 1).
 * Writes min(cap, total) triples and sets *n to the total. */
MOE_API moe_status moe_cache_copy_log(const moe_cache* c, int64_t* out, int64_t cap, int64_t* n);
/* Fault injection for tests of the failure path: the next n expert copies are treated as failed
 * enqueues (no HIP call is made for them), which leaves those entries non-resident. */
MOE_API moe_status moe_cache_inject_copy_failures(moe_cache* c, int n);
/* Waits for outstanding copies, releases events; the caller's buffers are untouched. */
MOE_API void moe_cache_destroy(moe_cache* c);

/* ------------------------------------------------------------------------------------------
 * moe_decode_step -- one decode step of an offloaded stack, every layer in one call (FreeToken
 * linux guide, "MoE memory handling"; FreeToken GGUF page, offload backend).  For each layer,
 * in order, on `compute`: moe_route_permute (forced_idx may be NULL) into the given buffers;
 * moe_expert_ffn_grouped through slot_table row `layer` (the cache's slot table, device [L*E]) and
 * moe_combine into y (act dtype), enqueued before the host has the ids; the ids reach host_idx
 * (pinned, T*k int32) -- at one token the route kernel also stores them into coherent host memory
 * of the library, which the host polls, otherwise topk_idx is copied and the host waits for the
 * copy; the distinct ids, ascending, to moe_cache_lookup(layer); moe_cache_fill(copy, compute);
 * when the layer has misses, the missed experts once more after their copies (a slot-table row of
 * the library with every other expert marked MOE_SLOT_ELSEWHERE) and moe_combine again;
 * moe_cache_mark_read(layer).  A resident expert's rows from the first launch are final; a missed
 * expert's (its slot absent or being refilled) are recomputed.  Outputs, cache decisions and
 * statistics are those of the same calls made one by one (route, lookup, fill, experts, combine,
 * mark_read).  The first launch flags absent slots in a word of the library, not in the workspace's
 * status word, which only the final launches set.  The library holds, per host thread and device,
 * a 4 KB coherent host buffer, a 4 KB pinned host row and a 4.25 KB device buffer, allocated on
 * first use until the process ends; when they cannot be allocated the step runs the calls in that
 * order instead.  Buffers as in those calls;
 * y_perm [T*k (+T), d] f32; ws: moe_workspace_bytes(T, ...) bytes.  Every layer's x, w_router and
 * y are checked (MOE_EINVAL) before anything is enqueued; later errors return at once, the layers
 * before them enqueued.  Returns the first error. */
typedef struct {
    const void* x;             /* [T, d] act: this layer's input (device) */
    const void* w_router;      /* [E, d] act */
    const float* bias;         /* [E] or NULL */
    const int32_t* forced_idx; /* [T, k] or NULL */
    const void* shared_w;      /* shared expert slot image or NULL */
    void* y;                   /* [T, d] act: output (device) */
    int32_t layer;             /* cache layer index */
    int32_t reserved;          /* 0 */
} moe_decode_layer;
MOE_API moe_status moe_decode_step(moe_cache* cache, int n_layers, const moe_decode_layer* layers, int T, int d,
                                   int f, int E, int k, moe_dtype act, moe_dtype w, const void* slot_pool,
                                   int n_slots, size_t slot_stride, const int32_t* slot_table, int32_t* topk_idx,
                                   float* topk_w, float* logits, int32_t* counts, int32_t* offsets, int32_t* perm,
                                   int32_t* inv_perm, float* y_perm, void* ws, size_t ws_bytes, int32_t* host_idx,
                                   moe_stream compute, moe_stream copy);

/* moe_decode_step with split launches (the hit/miss overlap of the pages' decode: FreeToken linux
 * guide, mechanism table, resident experts used while misses stream in).  A layer without misses
 * runs as in moe_decode_step.  A layer with misses stages two table rows in host_tables (pinned,
 * 2*E int32) and copies them to dev_tables (device, 2*E int32): row 0 holds the resident experts'
 * slots with the missed ones MOE_SLOT_ELSEWHERE, row 1 the missed experts' new slots with the
 * resident ones MOE_SLOT_ELSEWHERE; the resident experts (and the shared expert) are enqueued with
 * row 0 before moe_cache_fill, so they run while the copies do, then the missed experts with row 1,
 * then moe_combine and mark_read.  Outputs and cache decisions are bitwise those of
 * moe_decode_step.  Other arguments as moe_decode_step. */
MOE_API moe_status moe_decode_step_split(moe_cache* cache, int n_layers, const moe_decode_layer* layers, int T, int d,
                                         int f, int E, int k, moe_dtype act, moe_dtype w, const void* slot_pool,
                                         int n_slots, size_t slot_stride, const int32_t* slot_table,
                                         int32_t* topk_idx, float* topk_w, float* logits, int32_t* counts,
                                         int32_t* offsets, int32_t* perm, int32_t* inv_perm, float* y_perm, void* ws,
                                         size_t ws_bytes, int32_t* host_idx, int32_t* host_tables,
                                         int32_t* dev_tables, moe_stream compute, moe_stream copy);

/* The hybrid miss split (FreeToken RTX 5090 page, miss split: a miss is copied over PCIe, run on the
 * CPU where its weights live, or both, split by the host and PCIe bandwidths measured on the
 * machine; stork.ai article, miss policy).  Of a layer's m misses the host takes *n_host, the n
 * minimising t(n): t(0) = m / pcie_rate; t(n) = max((m - n) / pcie_rate, host_fixed_s + n / cpu_rate)
 * for n >= 1, ties to the smaller n.  Rates are expert images per second (cpu_rate 0 = no host
 * path); host_fixed_s is the per-layer host-path cost that does not grow with n (activation row to
 * the host, thread wake-up, output rows back), in seconds.  Host only.  MOE_EINVAL for m < 0,
 * pcie_rate <= 0, cpu_rate < 0, host_fixed_s < 0 or n_host NULL. */
MOE_API moe_status moe_hybrid_split(int m, double cpu_rate, double pcie_rate, double host_fixed_s, int32_t* n_host);

/* moe_decode_step with hybrid miss handling (FreeToken RTX 5090 page, miss split; stork.ai
 * article, miss policy), one token per step (T = 1, bf16 activations).  Per layer, as in
 * moe_decode_step, the experts and the combine are first enqueued through the slot-table row as it
 * stands; after the ids reach the host (host_idx: k int32, pinned): the layer's m misses are split
 * by moe_hybrid_split (cpu_rate, pcie_rate, host_fixed_s), the host taking the n highest-numbered
 * ones.  A layer with n = 0 continues as moe_decode_step (lookup, fill, the missed experts again).
 * Otherwise x is copied to host_x (d bf16, pinned), and the other ids (all of them with copy_too,
 * whose host experts are then also inserted, their copies deferred through moe_cache_fill_split)
 * go to moe_cache_lookup and a fill; a table row with only the GPU's missed experts in their slots
 * (every other expert MOE_SLOT_ELSEWHERE) is staged in host_table (pinned, E int32) and copied to
 * dev_table (device, E int32), and those experts are enqueued again; each host expert runs
 * moe_cpu_expert_ffn on its pinned image (cpu_threads, 0 = all) into host_y (pinned, k*d f32) and
 * its row is copied into y_perm; then moe_combine and mark_read.  Outputs and cache decisions are
 * those of the same calls made one by one.  *n_cpu_out (if not NULL) is increased by the number of
 * host-run experts.  Other arguments, and the library's per-thread buffers, as moe_decode_step. */
MOE_API moe_status moe_decode_step_hybrid(moe_cache* cache, int n_layers, const moe_decode_layer* layers, int d,
                                          int f, int E, int k, moe_dtype act, moe_dtype w, const void* slot_pool,
                                          int n_slots, size_t slot_stride, const int32_t* slot_table,
                                          int32_t* topk_idx, float* topk_w, float* logits, int32_t* counts,
                                          int32_t* offsets, int32_t* perm, int32_t* inv_perm, float* y_perm,
                                          void* ws, size_t ws_bytes, int32_t* host_idx, void* host_x, float* host_y,
                                          int32_t* host_table, int32_t* dev_table, double cpu_rate,
                                          double pcie_rate, double host_fixed_s, int copy_too, int cpu_threads,
                                          int64_t* n_cpu_out, moe_stream compute, moe_stream copy);

/* Host execution of one routed expert, the CPU side of hybrid miss handling (FreeToken RTX 5090
 * page, miss split: a miss runs on the GPU after a PCIe copy or on the CPU, split by the measured
 * host and PCIe bandwidths).  slot_image: host, the expert's packed slot (moe_pack_expert layout,
 * w = MOE_BF16 or MOE_INT4_G128); x: host bf16 [n, d] (1 <= n <= 256); y: host binary32 [n, d],
 * written.  y = W_d (silu(W_g x) * (W_u x)) with binary32 sums and h rounded to bf16, as on the GPU
 * path.  threads: host threads to use (0 = all of the library's pool; MOE_CPU_THREADS sets the
 * pool size, default the hardware concurrency).  Synchronous; no HIP call. */
MOE_API moe_status moe_cpu_expert_ffn(const void* slot_image, moe_dtype w, int d, int f, const void* x, int n,
                                      float* y, int threads);

/* Page-locked host memory for the expert pool (hipHostMalloc). */
MOE_API moe_status moe_pinned_alloc(size_t bytes, void** out);
MOE_API void moe_pinned_free(void* p);

/* ------------------------------------------------------------------------------------------
 * Kernel timing.  While enabled, each kernel launch of the calls above is bracketed by two
 * HIP events recorded on the launch stream; moe_profile_collect() waits for them and adds the
 * elapsed times per kernel name.  moe_profile_get(i, ...) reads entry i (MOE_EINVAL past the
 * end).  Adds event overhead: for measurement runs only. */
MOE_API void moe_profile_enable(int on);
MOE_API moe_status moe_profile_collect(void);
MOE_API moe_status moe_profile_get(int i, char* name, int name_cap, double* total_ms,
                                   int64_t* launches);
MOE_API void moe_profile_reset(void);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H_ */
