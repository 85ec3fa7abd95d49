/*
 * pagedweight.h -- C ABI of libpagedweight, a fused mixed-precision
 * Mixture-of-Experts expert layer for AMD Instinct MI355X (gfx950).
 *
 * What it computes.  "Technical summary: PagedWeight" (gist.science, paper
 * 2607.16184), Core components 1 (Paged Weight representation): every expert
 * linear block -- (layer, expert, gate_up | down) -- is stored as Any-Precision
 * overlaid bit planes with per-row lookup tables, and a Weight Page Table holds
 * the committed bitwidth q_i of each block.  Core components 3 (second bullet,
 * fused mixed-precision kernel): one fused operation reads the planes and the
 * tables directly and computes each block at its own q_i.  The layer is a routed
 * SwiGLU FFN:
 *     gate, up = rows [0, I) and [I, 2I) of  W_gate_up(e) x_t      (W: [2I][H])
 *     h        = SiLU(gate) * up,  SiLU(z) = z / (1 + exp(-z))
 *     o        = W_down(e) h                                       (W: [H][I])
 *     y_t      = sum_{j < k} w[t][j] * o_{ids[t][j]}(x_t)
 * with W[n][c] = LUT_{q}[n][code_q(n, c)] and code_q the value of the first q
 * planes (plane 0 = most significant bit).
 *
 * Storage of one block with N rows and K columns (K % 32 == 0, N % 16 == 0).
 * Canonical planes (what pw_pack_planes takes): uint32 [8][N][K/32],
 * plane-major; bit j (LSB = 0) of word [p][n][c] is plane p of weight
 * (n, 32c + j).  The forward and pw_dequant_block read the DEVICE layout that
 * pw_pack_planes writes from them:
 *   planes : device layout, pw_planes_bytes(N, K, nplanes) bytes.  Planes stay
 *            outermost and each takes N * K / 8 bytes, so a block committed at
 *            q needs only its first q planes resident (a shorter allocation is
 *            fine).  Inside a plane the words sit in tiles of 16 rows by 16
 *            words, tile-row-major; inside a tile the 16 rows follow each
 *            other, each holding the tile's words (16, or (K/32) mod 16 in the
 *            last column tile).  Rows of a gate_up block are interleaved: tile
 *            t holds gate rows 8t..8t+7, then up rows I+8t..I+8t+7.
 *   lut_all: fp16 bits [504 * N], the per-row tables for b = 3..8 laid one
 *            after another in canonical row order; the table of bitwidth b
 *            starts at element N * (2^b - 8) and is [N][2^b].  Only the table
 *            of q is read.
 *
 * Conventions of every entry point.
 *   - Pointers are DEVICE pointers unless the comment says host.  The caller
 *     owns every device buffer; the library allocates no device memory.  Its
 *     only state is the host-side bookkeeping of pager objects (weight pager
 *     section below); every other entry point is stateless.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Calls enqueue work and return; results are ready when the stream reaches
 *     that point.  Inputs (including the q table) must not change before that:
 *     a q write ordered on the stream after a forward never affects it, which
 *     is the "commit only at a safe boundary" rule (Core components 3, first
 *     bullet).
 *   - Host-detectable errors return a negative pw_status before anything is
 *     enqueued.  Device-only errors (expert id outside [0, E), committed
 *     bitwidth outside 3..8) make the offending slot / block contribute zero and
 *     set a bit in the workspace status word, read by pw_get_device_status.
 *   - No C++ exception crosses this interface.
 */
#ifndef PAGEDWEIGHT_H
#define PAGEDWEIGHT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PW_ABI_VERSION 4

typedef int32_t pw_status;
#define PW_OK                     0
#define PW_ERR_INVALID_ARG       -1  /* null pointer, negative size, bad enum  */
#define PW_ERR_UNSUPPORTED_SHAPE -2  /* H, I not multiples of 32, E > 256, k > E,
                                        2*I*H > 2^31 - 1, or T*k > 2^29 - 1      */
#define PW_ERR_BITWIDTH          -3  /* host-side bitwidth outside 3..8        */
#define PW_ERR_WORKSPACE         -4  /* workspace too small                    */
#define PW_ERR_ALIGNMENT         -5  /* pointer not 16-byte aligned            */
#define PW_ERR_HIP               -6  /* a HIP runtime call failed              */
#define PW_ERR_UNSUPPORTED       -7  /* option the library does not support     */
#define PW_ERR_OUT_OF_MEMORY     -8  /* pager: no free arena range large enough */

/* device status bits (pw_get_device_status) */
#define PW_DEV_BAD_EXPERT_ID  0x1u   /* some ids[t][j] outside [0, E)          */
#define PW_DEV_BAD_BITWIDTH   0x2u   /* some routed block has q outside 3..8   */

/* Layer shape: H = hidden size, I = expert intermediate size, E = number of
 * routed experts (1..256), k = experts per token (1..E). */
typedef struct {
  int32_t hidden;
  int32_t inter;
  int32_t num_experts;
  int32_t top_k;
} pw_moe_shape;

/* One Weight Page Table entry: where one block's planes and tables live.
 * The table is device memory [E][2] (index 2e + m, m = 0 gate_up, 1 down),
 * both pointers 16-byte aligned.  Moving a block means rewriting its entry. */
typedef struct {
  const uint32_t* planes;
  const uint16_t* lut_all;
} pw_block_desc;

/* Kernel family for the expert products. */
#define PW_PATH_AUTO  0  /* one family per call by the mean routed slots per
                            routed expert m = T*top_k / min(E, T*top_k): GEMV
                            for m < 1.6, matrix-core GEMV for 1.6 <= m <= 64,
                            MFMA above, where an expert's tokens past its last
                            whole 512-token tile take the matrix-core GEMV when
                            there are at most 96 of them (pw_path_info's
                            mfma_tail).  If either *_min_tokens option is > 0
                            and m >= 1.6, per expert by its token count n
                            instead: GEMV below mgemv_min_tokens (default 1),
                            matrix-core GEMV below mfma_min_tokens (default
                            256), MFMA from there; with m < 1.6 the GEMV still
                            takes every expert below mfma_min_tokens */
#define PW_PATH_GEMV  1  /* every expert on the bit-plane GEMV kernels            */
#define PW_PATH_MFMA  2  /* every expert on the dequant-to-LDS MFMA kernels       */
#define PW_PATH_MGEMV 3  /* every expert on the matrix-core GEMV kernels          */

/* Stage boundaries at which optional events are recorded. */
#define PW_STAGE_ROUTE   0
#define PW_STAGE_GATE_UP 1
#define PW_STAGE_DOWN    2
#define PW_STAGE_COMBINE 3
#define PW_NUM_STAGES    4

/* What the optional events of pw_moe_options record. */
#define PW_EVENTS_STAGES  0  /* stage_events[s] recorded on the stream right
                                before stage s, stage_events[PW_NUM_STAGES]
                                after the last stage (kernel time plus the
                                launch gaps between them)                      */
#define PW_EVENTS_KERNELS 1  /* stage_events[0] / [1]: start / stop of the
                                gate_up product's kernel(s), [2] / [3]: start /
                                stop of the down product's kernel(s), taken by
                                the launches themselves (the kernels' own
                                execution, no launch gap); [4] unused.  A NULL
                                entry is not recorded                          */

typedef struct {
  int32_t path;              /* PW_PATH_*                                     */
  int32_t mfma_min_tokens;   /* AUTO bands: MFMA from this many tokens per
                                expert; <= 0: per-call rule or default 256    */
  /* Optional hipEvent_t handles (as void*), used if stage_events[0] is
   * non-NULL; what they record is set by event_mode. */
  void* stage_events[PW_NUM_STAGES + 1];
  int32_t mgemv_min_tokens;  /* AUTO bands: matrix-core GEMV from this many
                                tokens per expert (below mfma_min_tokens);
                                <= 0: per-call rule or default 1              */
  int32_t event_mode;        /* PW_EVENTS_* (other values: PW_ERR_INVALID_ARG) */
} pw_moe_options;

/* ABI version of the loaded library (PW_ABI_VERSION). */
int32_t pw_abi_version(void);

/* Static, never-NULL text for a status code. */
const char* pw_status_str(pw_status status);

/* Element counts of one block's canonical storage (see the storage format above). */
size_t pw_plane_words(int32_t N, int32_t K);   /* 8 * N * K / 32, 0 if invalid */
size_t pw_lut_elems(int32_t N);                /* 504 * N                      */
size_t pw_lut_offset(int32_t N, int32_t b);    /* N * (2^b - 8)                */

/* Host-only shape check for a forward of T tokens (no device access). */
pw_status pw_check_shape(const pw_moe_shape* shape /* host */, int32_t T);

/* Workspace bytes a forward of up to T_max tokens needs (0 on a bad shape). */
size_t pw_workspace_bytes(const pw_moe_shape* shape /* host */, int32_t T_max);

/* Clear the workspace status word.  Call once on a fresh workspace before its
 * first forward (the status word is otherwise sticky; see
 * pw_get_device_status).  Enqueues one small kernel. */
pw_status pw_workspace_init(void* workspace, size_t workspace_bytes, void* stream);

/* The fused mixed-precision MoE layer (Core components 3, fused kernel).
 *   shape   host; T >= 0 tokens (T == 0 returns PW_OK and enqueues nothing)
 *   x       fp16 [T][H]                         ids  int32 [T][k]
 *   w       fp32 [T][k] routing weights, used as given (no renormalisation)
 *   blocks  device pw_block_desc [E][2]         q    device uint8 [E][2]
 *   y       fp16 [T][H], overwritten (round to nearest even from fp32)
 *   workspace, workspace_bytes: device scratch of at least
 *           pw_workspace_bytes(shape, T) bytes, 256-byte aligned; its first
 *           bytes hold the status word.  Concurrent calls need distinct
 *           workspaces.
 *   opts    host, may be NULL (AUTO path, per-call rule, no events).
 * Accumulation is fp32; h is rounded to fp16 before the down product.
 * Results are deterministic: the same inputs give the same bits. */
pw_status pw_moe_forward(const pw_moe_shape* shape, int32_t T,
                         const uint16_t* x, const int32_t* ids, const float* w,
                         const pw_block_desc* blocks, const uint8_t* q,
                         uint16_t* y, void* workspace, size_t workspace_bytes,
                         const pw_moe_options* opts, void* stream);

/* Allocation-free variant of pw_moe_forward, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same computation, kernels and results
 * as pw_moe_forward; the scratch the workspace would hold lives in a static
 * device array of PW_NOALLOC_SCRATCH_BYTES per GPU, kept until the process
 * ends.  The call allocates nothing.
 *   shape, T, x, ids, w, blocks, q, y, opts, stream: as for pw_moe_forward
 *   status  device uint32, may be NULL: device errors (PW_DEV_* bits) are OR-ed
 *           into it; the caller clears and reads it.  With NULL they are not
 *           reported.
 * Errors: those of pw_moe_forward; PW_ERR_WORKSPACE if the call needs more
 * than PW_NOALLOC_SCRATCH_BYTES (pw_workspace_bytes(shape, T) bytes);
 * PW_ERR_HIP if the scratch address cannot be found.  All calls on one GPU
 * share its scratch array: calls that overlap in time on one GPU race.  Each
 * call overwrites what it reads, so nothing needs clearing between calls. */
#define PW_NOALLOC_SCRATCH_BYTES (64u << 20)
pw_status pw_moe_forward_noalloc(const pw_moe_shape* shape, int32_t T, const uint16_t* x, const int32_t* ids,
                                 const float* w, const pw_block_desc* blocks, const uint8_t* q, uint16_t* y,
                                 uint32_t* status, const pw_moe_options* opts, void* stream);

/* The kernel families a pw_moe_forward call with this shape, T and options
 * runs (the fused kernel's dispatch between its decode, moderate-batch and
 * prefill forms, Core components 3), without touching the GPU.  Host only;
 * the result does not depend on the routing itself. */
typedef struct {
  int32_t gemv;          /* 1: the bit-plane GEMV kernels run                 */
  int32_t mgemv;         /* 1: the matrix-core GEMV kernels run (for their
                            band, or only for the MFMA experts' tails)        */
  int32_t mfma;          /* 1: the dequant-to-LDS MFMA kernels run            */
  int32_t mgemv_from;    /* experts with at least this many tokens (and below
                            mfma_from, if MFMA runs) take the matrix-core GEMV;
                            0 if it has no band                                */
  int32_t mfma_from;     /* experts with at least this many tokens take MFMA;
                            0 if it does not run                               */
  int32_t inline_route;  /* 1: no separate routing kernel (GEMV alone, at most
                            64 slots: the gate_up kernel routes)               */
  int32_t down_kparts;   /* parts of the K range of the GEMV down product    */
  int32_t launches;      /* kernels the call enqueues (T > 0)                 */
  int32_t mfma_tail;     /* an MFMA expert's tokens past its last whole
                            512-token tile, when at most this many, take the
                            matrix-core GEMV instead (the AUTO rule's prefill
                            form; the kernels of both families run); 0: never */
} pw_path_info;

/*   shape, opts  host, as for pw_moe_forward (opts may be NULL)
 *   info         host, overwritten (all zero for T == 0)
 * Errors: those pw_moe_forward reports for the shape, T and options. */
pw_status pw_moe_path_info(const pw_moe_shape* shape, int32_t T, const pw_moe_options* opts,
                           pw_path_info* info);

/* Bytes of `nplanes` planes (1..8) of an N x K block in the device layout:
 * nplanes * N * K / 8 (0 if N % 16, K % 32 or nplanes is invalid).  The
 * bitplane packing layout of Core components 1 ("Technical summary:
 * PagedWeight": overlaid Any-Precision bit planes with lookup tables). */
size_t pw_planes_bytes(int32_t N, int32_t K, int32_t nplanes);

/* Write planes 0..nplanes-1 of one block in the device layout the kernels read
 * (see the storage format above): a lossless permutation of the words of the
 * canonical planes.  module 0 (gate_up, N = 2I) interleaves gate and up rows
 * per 16-row tile, module 1 (down) keeps the row order.
 *   canon       device uint32 [nplanes][N][K/32] (4-byte aligned), not modified
 *   dev_layout  device, pw_planes_bytes(N, K, nplanes) bytes, 16-byte aligned,
 *               distinct from canon (no in-place packing); overwritten
 * Errors: PW_ERR_INVALID_ARG (null, nplanes outside 1..8, module not 0/1,
 * in place), PW_ERR_UNSUPPORTED_SHAPE (N % 16, K % 32), PW_ERR_ALIGNMENT.
 * Enqueued on `stream`; one kernel. */
pw_status pw_pack_planes(const uint32_t* canon, int32_t N, int32_t K, int32_t nplanes, int32_t module,
                         uint32_t* dev_layout, void* stream);

/* Dequantize one block at bitwidth q (host value, 3..8): w_out fp16 bits
 * [N][K] in canonical row order, = LUT_q[n][code_q(n, c)].  planes in the
 * device layout (pw_pack_planes, same module), at least q planes.  The same
 * device decode the forward uses; bit-exact by definition (a table copy).
 * Core components 1.  Errors as pw_pack_planes, PW_ERR_BITWIDTH for q. */
pw_status pw_dequant_block(const uint32_t* planes, const uint16_t* lut_all,
                           int32_t N, int32_t K, int32_t q, int32_t module,
                           uint16_t* w_out, void* stream);

/* Wait for `stream`, copy the workspace status word to *flags (host), then
 * clear it.  Returns PW_ERR_HIP if the copy or the wait fails. */
pw_status pw_get_device_status(void* workspace, uint32_t* flags /* host */, void* stream);

/* Router and online routing statistics ("Technical summary: PagedWeight",
 * Core components 2, second bullet: each expert's routing mass -- how often it
 * is selected and with what weight -- is tracked online).  The router is the
 * top-k softmax router of a routed MoE layer:
 *     logits[t][e] = sum_h x[t][h] * router_w[e][h]   (fp16 inputs, fp32 sums)
 *     ids[t][0..k)  = the k largest logits, descending; lower id first on ties
 *     w[t][j]       = exp(l_j - l_0) / sum_i exp(l_i - l_0) over the selected
 * and, if stat_count / stat_mass are non-NULL, for every slot
 *     stat_count[ids[t][j]] += 1,  stat_mass[ids[t][j]] += w[t][j]
 * (device uint32 [E] and fp32 [E], accumulated across calls; the caller
 * zeroes them to start a window; mass is an fp32 atomic sum, so its last bits
 * depend on the order the slots arrive in).
 *   x fp16 [T][H], router_w fp16 [E][H] (both 16-byte aligned);
 *   ids int32 [T][k], w fp32 [T][k] outputs; k <= 64 (else
 *   PW_ERR_UNSUPPORTED_SHAPE); workspace as for pw_moe_forward (not used by
 *   the router itself).  T == 0 returns PW_OK and enqueues nothing.  One
 *   launch. */
pw_status pw_router_topk(const pw_moe_shape* shape /* host */, int32_t T, const uint16_t* x,
                         const uint16_t* router_w, int32_t* ids, float* w, uint32_t* stat_count,
                         float* stat_mass, void* workspace, size_t workspace_bytes, void* stream);

/* Router + fused mixed-precision layer in one call: pw_router_topk into the
 * workspace (ids and weights are not returned), then pw_moe_forward on them.
 * Arguments as for those two calls. */
pw_status pw_moe_forward_routed(const pw_moe_shape* shape /* host */, int32_t T, const uint16_t* x,
                                const uint16_t* router_w, const pw_block_desc* blocks, const uint8_t* q,
                                uint16_t* y, uint32_t* stat_count, float* stat_mass, void* workspace,
                                size_t workspace_bytes, const pw_moe_options* opts, void* stream);

/* L chained layers of one decode step: layer l routes its input with its own
 * top-k softmax router (as pw_router_topk), runs the fused mixed-precision
 * layer on its own page table (as pw_moe_forward), and its output is layer
 * l + 1's input; y receives the last layer's output.  "Technical summary:
 * PagedWeight", Core components 3 (the fused kernel, which reduces overhead;
 * committed bitwidths read on the device, so a pager commit between two calls,
 * or two replays of a captured graph of one call, takes effect without new
 * launch arguments) and Core components 2 (routing statistics per layer).
 * Each layer's weighted combine is computed inside the next layer's router
 * kernel, so a layer takes the router and the expert products (three launches
 * for decode batches) and only the last layer launches a combine.  Results are
 * bit-identical to L chained pw_moe_forward_routed calls.
 *   shape        host, the same for every layer; k <= 64, H <= 16384
 *   x            fp16 [T][H], layer 0's input;  y  fp16 [T][H], overwritten
 *   router_w     host array [L] of device fp16 [E][H] router matrices
 *   blocks, q    host arrays [L] of device page tables [E][2] and bitwidths [E][2]
 *   stat_count, stat_mass  device uint32 / fp32 [L][E] or NULL: routing
 *                statistics accumulated per layer, as pw_router_topk
 *   workspace    as for pw_moe_forward with the same T (intermediate layer
 *                inputs live in it)
 *   opts         as for pw_moe_forward; events are not supported
 *                (PW_ERR_UNSUPPORTED)
 * Errors: those of pw_moe_forward and pw_router_topk; PW_ERR_INVALID_ARG for
 * L < 1 or a NULL entry. */
pw_status pw_moe_forward_layers(const pw_moe_shape* shape /* host */, int32_t L, int32_t T, const uint16_t* x,
                                const uint16_t* const* router_w /* host [L] */,
                                const pw_block_desc* const* blocks /* host [L] */,
                                const uint8_t* const* q /* host [L] */, uint16_t* y, uint32_t* stat_count,
                                float* stat_mass, void* workspace, size_t workspace_bytes,
                                const pw_moe_options* opts, void* stream);

/* ------------------------------------------------------------------------
 * Quality-aware bitwidth planner (host code; "Technical summary: PagedWeight",
 * Core components 2: offline sensitivity per block, online routing statistics
 * with hot experts protected by higher floors and damage multipliers, a
 * prompt-specific correction, and a greedy choice of the reductions with the
 * least damage per byte saved until a memory target is met).
 *
 *   D_b(q) = mu_b * (S_b(q) + R_b(q))   damage of block b at bitwidth q
 *   mu_b   = hot_multiplier for blocks of hot experts, else 1
 *   hot    = the ceil(hot_fraction * E) experts with the largest positive
 *            routing mass (equal masses: lower expert id)
 *   floor  = floor_hot for blocks of hot experts, else floor_cold; a block
 *            below its floor is raised to it first
 * If the resident plane bytes sum_b q_b * plane_bytes[b] exceed the budget,
 * one-bit reductions are taken in increasing (D_b(q-1) - D_b(q)) /
 * plane_bytes[b] (equal: lower b) until they fit or every block sits on its
 * floor.  Otherwise one-bit restorations are taken in decreasing
 * (D_b(q) - D_b(q+1)) / plane_bytes[b] (equal: lower b) among the steps that
 * still fit, up to 8 bits.  Costs are evaluated in fp64 exactly as written.
 * The result feeds pw_pager_request.
 * ---------------------------------------------------------------------- */
typedef struct {
  int32_t num_blocks;          /* B                                                  */
  int32_t num_experts;         /* E                                                  */
  const int32_t* expert_of;    /* host [B]: expert of block b, in [0, E)             */
  const int64_t* plane_bytes;  /* host [B]: bytes of one bit plane of block b (> 0)  */
  const float* sensitivity;    /* host [B][6]: offline score S_b(q), column q - 3    */
  const float* correction;     /* host [B][6]: prompt correction R_b(q); NULL = 0    */
  const float* routing_mass;   /* host [E]; NULL = no expert is hot                  */
  double hot_fraction;
  int32_t floor_cold;          /* 3..8 */
  int32_t floor_hot;           /* 3..8 */
  float hot_multiplier;
  int32_t reserved;
} pw_plan_problem;

/* Plan bitwidths for a plane-byte budget.  q_cur (host [B], 3..8): current
 * desired bitwidths; q_out (host [B]) receives the plan; *plane_bytes_out
 * (may be NULL) the resident plane bytes of the plan; *fits (may be NULL) 1 if
 * they fit the budget, 0 if the floors alone exceed it (the plan then holds
 * every block at its floor).  Pure host computation; no device access. */
pw_status pw_plan_bitwidths(const pw_plan_problem* problem /* host */, const int32_t* q_cur /* host */,
                            int64_t budget_bytes, int32_t* q_out /* host */, int64_t* plane_bytes_out /* host */,
                            int32_t* fits /* host */);

/* ------------------------------------------------------------------------
 * Weight pager: the Weight Page Table kept on the host, asynchronous page
 * movement and safe-boundary commits ("Technical summary: PagedWeight",
 * Core components 1, third bullet: desired bitwidth d_i, committed bitwidth
 * q_i, pages GPU-resident, CPU-resident or in transfer; Core components 3,
 * first bullet: pages offloaded to CPU memory and reloaded asynchronously,
 * bitwidth commits only at safe boundaries).
 *
 * A page is one bit plane of one block.  The host holds all eight planes of
 * every block in pinned memory (caller-owned, never written by the library);
 * the GPU holds planes 0..q-1 of each block as one extent of a caller-owned
 * device arena.  The pager owns the device page table the forward reads
 * (`blocks` [B] and `q` [B], caller-allocated device memory, q zeroed by the
 * caller before the first commit; for a layer B = 2E and block 2e + m).
 *
 * Use:  pw_pager_request(b, d) for the blocks of a plan (host only), then
 * pw_pager_execute(copy_stream) enqueues the page movement (host-to-device
 * copies of planes the GPU lacks, device-to-device moves when an extent cannot
 * grow in place), then pw_pager_commit(stream) at a safe boundary (between
 * forwards on `stream`) enqueues one kernel that rewrites the page-table
 * entries and q bytes of every staged block together.  Forwards enqueued on
 * `stream` before the commit use the old bitwidths and storage, forwards after
 * it the new ones.  Every forward that reads the page table must run on the
 * commit stream or be ordered with it.  Arena ranges that a commit frees (a
 * lowered block's plane suffix, a moved block's old extent) are reused only
 * after `stream` has passed the commit.  The pager object is host state
 * (malloc'd bookkeeping, HIP events); it allocates no device memory.  One
 * pager is not thread-safe: calls on it must not overlap.
 * ---------------------------------------------------------------------- */
typedef struct pw_pager pw_pager;

#define PW_PAGE_CPU          0   /* no plane of the block on the GPU           */
#define PW_PAGE_GPU          1   /* planes 0..committed-1 on the GPU           */
#define PW_PAGE_IN_TRANSFER  2   /* planes for a staged increase still copying */

typedef struct {
  int32_t desired;        /* d_i (0 = never requested)                          */
  int32_t committed;      /* q_i in the device page table (0 = not committed)   */
  int32_t resident;       /* planes of the committed extent on the GPU          */
  int32_t pending;        /* bitwidth staged for the next commit, 0 if none     */
  int32_t state;          /* PW_PAGE_*                                          */
  int32_t reserved;
  uint64_t arena_offset;  /* byte offset of the committed extent, UINT64_MAX if none */
} pw_page_info;

/* Create a pager for `num_blocks` blocks of rows[b] x cols[b] weights (host
 * arrays; cols % 32 == 0).  `arena` (device, 256-byte aligned, arena_bytes
 * long) is where resident planes live.  *out receives the handle. */
pw_status pw_pager_create(int32_t num_blocks, const int32_t* rows /* host */, const int32_t* cols /* host */,
                          void* arena, size_t arena_bytes, pw_block_desc* blocks, uint8_t* q,
                          pw_pager** out /* host */);

/* Wait for the pager's outstanding copies and commits, then free it. */
pw_status pw_pager_destroy(pw_pager* pager);

/* Register block b's storage before its first commit: host_planes is pinned
 * host memory holding all 8 planes in the device layout (pw_pack_planes of the
 * block's module, pw_planes_bytes(N, K, 8) bytes; plane p starts at byte
 * p * N * K / 8, which is what the pager copies); lut_all is the device table
 * block [504 N] (fp16 bits, 16-byte aligned), which stays resident. */
pw_status pw_pager_set_block(pw_pager* pager, int32_t b, const uint32_t* host_planes /* pinned host */,
                             const uint16_t* lut_all);

/* Set the desired bitwidth d_i (3..8) of block b.  Host bookkeeping only. */
pw_status pw_pager_request(pw_pager* pager, int32_t b, int32_t desired);

/* Stage every block whose desired bitwidth differs from its committed one:
 * enqueue on copy_stream the copies of the planes it lacks.  Blocks staged
 * earlier and not yet committed are left alone.  PW_ERR_OUT_OF_MEMORY when the
 * arena has no room, PW_ERR_HIP when a copy cannot be enqueued: the blocks
 * staged before that stay staged, the rest keep their committed state
 * (commit lowered blocks first to free their planes). */
pw_status pw_pager_execute(pw_pager* pager, void* copy_stream);

/* Safe boundary: commit every staged block in one step.  If copies are still
 * in flight: with wait == 0 nothing is committed (*committed = 0); with
 * wait != 0 `stream` is made to wait for them on the device (the host does not
 * block).  *committed (host, may be NULL) receives the number of blocks whose
 * entries the enqueued commit rewrites. */
pw_status pw_pager_commit(pw_pager* pager, void* stream, int32_t wait, int32_t* committed /* host */);

/* Host view of block b's page-table entry. */
pw_status pw_pager_info(const pw_pager* pager, int32_t b, pw_page_info* info /* host */);

/* Arena bytes held by extents, including ranges freed by a commit that the
 * compute stream has not passed yet (as of the last execute/commit call). */
size_t pw_pager_arena_used(const pw_pager* pager);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDWEIGHT_H */
