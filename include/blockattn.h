/*
 * libblockattn: block-wise video-DiT attention on AMD MI355X (gfx950).
 *
 * The per-GPU hot path of block-wise long-video denoising as described in
 * "Minute-Long Videos with Dual Parallelisms" (arXiv 2505.21070, Abstract):
 * frames are denoised in temporal blocks, each at its own noise level, and a
 * per-GPU feature cache keeps the K/V a block produced so the neighbouring
 * block reuses them as attention context instead of recomputing them.
 *
 *   ba_cache_append     write one block's K/V into the HBM ring (the cache)
 *   ba_block_attention  queries of each queued block attend over
 *                       [cached segments ... | text] in one launch
 *   ba_block_update     per-block denoising step, each block at its own t
 *
 * Conventions for every call:
 *   - Pointers are device pointers owned by the caller unless marked (host).
 *     The library allocates no device memory and keeps no pointer after it
 *     returns.  Device buffers must be 16-byte aligned; a ring base 256-byte.
 *   - All argument checks run on the host before anything is enqueued.  On a
 *     non-BA_OK return nothing was enqueued and no ring descriptor changed;
 *     ba_last_error() then describes the failure (thread-local string).
 *   - Work is enqueued asynchronously on `stream` (NULL = the default stream);
 *     device faults surface at the caller's next synchronisation.  A failed
 *     launch returns BA_ERR_HIP.
 *   - Calls that touch the same ring must be ordered on one stream (or by the
 *     caller's events): an append into a slot that an attention call still
 *     reads is a race the library cannot see.
 *   - The library holds no global state besides the thread-local error text.
 */
#ifndef BLOCKATTN_H
#define BLOCKATTN_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  BA_OK = 0,
  BA_ERR_INVALID_ARG = 1,   /* null/misaligned pointer, inconsistent sizes */
  BA_ERR_UNSUPPORTED = 2,   /* head_dim or dtype the kernels do not cover  */
  BA_ERR_OUT_OF_RANGE = 3,  /* slot, length or timestep outside its range  */
  BA_ERR_HIP = 4            /* the HIP runtime refused a launch            */
} ba_status;

typedef enum { BA_BF16 = 0, BA_F32 = 1 } ba_dtype;

#define BA_TOKEN_ALIGN 64   /* slot token stride is a multiple of this      */
#define BA_MAX_SEGS 8       /* cache segments per block (text comes extra)  */

/*
 * K/V ring buffer: the per-GPU feature cache (Abstract of the DualParal page;
 * the pith.science verdict on it, pith_extraction.core_discovery: the cache
 * holds the self-attention K/V of the neighbouring, already processed block).
 * FIFO use follows the block queue of that verdict (key_machinery): the next
 * slot written is `appended mod n_slots`.
 *
 * Layout of the device buffer at `base` (dtype elements, e = 2 or 4 bytes):
 *   T_pad = slot_stride_tokens = slot_tokens rounded up to BA_TOKEN_ALIGN
 *   K[s][h][t][d] at element ((s*2 + 0)*heads + h)*T_pad*head_dim + t*head_dim + d
 *   V[s][h][t][d] at element ((s*2 + 1)*heads + h)*T_pad*head_dim + d*T_pad + t
 * Per (slot, head) K is token-major [T_pad][head_dim] and V is stored
 * transposed, dim-major [head_dim][T_pad], so the attention kernel streams
 * both operands of its two matrix products with contiguous 16-byte loads.
 * An append of n tokens writes tokens [0, n) and zeroes [n, T_pad) of the slot.
 *
 * The struct is plain data on the host, owned by the caller.
 */
typedef struct {
  void*   base;               /* device buffer of ba_ring_bytes(...) bytes   */
  int32_t n_slots;
  int32_t slot_tokens;        /* capacity of one slot, in tokens             */
  int32_t heads;
  int32_t head_dim;           /* 64 or 128                                   */
  int32_t dtype;              /* ba_dtype                                    */
  int32_t slot_stride_tokens; /* T_pad, set by ba_ring_init                  */
  int64_t appended;           /* FIFO appends so far                         */
} ba_ring;

/* Bytes a ring needs (0 if an argument is out of range). */
size_t ba_ring_bytes(int32_t n_slots, int32_t slot_tokens, int32_t heads,
                     int32_t head_dim, int32_t dtype);

/* Fill in `ring` for the buffer `base` (>= ba_ring_bytes bytes, 256-byte
 * aligned) and enqueue a zero fill of the whole buffer on `stream`, so that
 * slots never appended read as zeros.  appended = 0. */
ba_status ba_ring_init(ba_ring* ring, void* base, size_t bytes, int32_t n_slots,
                       int32_t slot_tokens, int32_t heads, int32_t head_dim,
                       int32_t dtype, hipStream_t stream);

/*
 * Write one block's K/V into the next FIFO slot (appended mod n_slots), store
 * that slot in *slot_out (host, may be NULL) and advance ring->appended.
 * k, v: [n_tokens][heads][head_dim] in the ring's dtype (token-major, as a
 * QKV projection emits them); 1 <= n_tokens <= slot_tokens.
 * Pure data movement: the slot afterwards holds the exact bits of k and v.
 */
ba_status ba_cache_append(ba_ring* ring, const void* k, const void* v,
                          int32_t n_tokens, int32_t* slot_out, hipStream_t stream);

/*
 * Batched form for a queue of blocks: block i of k, v ([n_blocks][n_tokens]
 * [heads][head_dim]) goes to slots[i] (host array, distinct slots).  Leaves
 * ring->appended unchanged.  One launch.
 */
ba_status ba_cache_append_batched(const ba_ring* ring, const void* k, const void* v,
                                  int32_t n_tokens, const int32_t* slots,
                                  int32_t n_blocks, hipStream_t stream);

/* Tokens [0, len) of ring slot `slot` form one segment of a block's keys. */
typedef struct {
  int32_t slot;
  int32_t len;
} ba_seg;

/*
 * Key set of one queued block: its cache segments in key order (normally the
 * neighbouring block's cached K/V, then the block's own K/V), followed by
 * tokens [0, text_len) of slot `text_slot` of the text ring.  Segments of
 * length 0 are skipped.  There is no other mask: every listed key is visible
 * to every query of the block (video DiT attention is bidirectional).
 */
typedef struct {
  int32_t q_len;              /* queries of this block, 0..q_stride          */
  int32_t n_segs;             /* 0..BA_MAX_SEGS                              */
  ba_seg  seg[BA_MAX_SEGS];
  int32_t text_slot;
  int32_t text_len;           /* 0..text->slot_tokens                        */
} ba_block_meta;

/*
 * Block attention for n_blocks queued blocks in one call:
 *   out[b][i][h][:] = sum_j p_ij V_j,  p_ij = softmax_j(scale * <q_bih, K_j>)
 * over the keys K_j / values V_j of meta[b] (head h), for i < meta[b].q_len.
 * This is scaled dot-product attention ("Attention Is All You Need", listed
 * among the works the DualParal page builds on) with the key set the feature
 * cache defines (DualParal Abstract; pith.science verdict, core_discovery).
 *
 * q, out:  [n_blocks][q_stride][heads][head_dim], the ring's dtype.  Rows
 *          i >= q_len of a block are neither read nor written.  out may be q.
 * cache:   the K/V ring; text: a ring with the text K/V (same heads,
 *          head_dim, dtype), or NULL when every text_len is 0.  The text
 *          K/V is passed as a ring (filled once per prompt with
 *          ba_cache_append, or from [heads][text_cap][head_dim] arrays with
 *          ba_text_ring_set; meta[b].text_slot picks the slot) rather than
 *          as plain arrays (ba_block_attention_text_arrays takes those and
 *          fills a ring in its workspace first): a ring matrix stores V
 *          transposed ([head_dim][T_pad] per head), which is the layout the
 *          PV product streams from, so the text keys take the same path
 *          through the kernel as the cached segments, with no per-call
 *          transpose.
 * meta:    (host) n_blocks entries.  Every block with q_len > 0 needs >= 1 key.
 * scale:   > 0, or <= 0 for 1/sqrt(head_dim).
 * lse:     optional [n_blocks][heads][q_stride] fp32 log-sum-exp (natural
 *          log) of the scaled scores per query, or NULL.
 * workspace: optional device buffer (256-byte aligned) of workspace_bytes,
 *          see ba_attention_workspace_bytes (bf16 only).  With it, the tasks
 *          that would form a last, partly filled wave of workgroups are split
 *          evenly over the workgroups the device holds at once; the pieces of
 *          a cut task are written there and folded by a second kernel on the
 *          same stream.  Without it (NULL) each query tile is one workgroup.
 *          The split is skipped when the pieces would be short (fewer than
 *          24 key tiles of 64 per tail workgroup, e.g. a text-only key set)
 *          and when whole query tiles would leave less than a quarter of an
 *          XCD's workgroup slots idle in their last round;
 *          ba_attention_plan tells which schedule a call takes.  A launch
 *          of the resident shape (see ba_attention_query_tile) uses none.
 *          Results agree to rounding either way and are deterministic.  Its
 *          contents need no initialisation; calls that share a workspace must
 *          be ordered on one stream.
 * bf16: products of bf16 inputs accumulate in fp32; the weights are rounded
 * to bf16 (nearest even) for the second product and the output to bf16.
 * The weight sums are taken in fp32 of the rounded weights at head_dim 64
 * (on the matrix cores) and of the unrounded ones at head_dim 128.
 * fp32: all arithmetic in fp32 (the workspace is not used).
 */
ba_status ba_block_attention(const void* q, int32_t q_stride, const ba_ring* cache,
                             const ba_ring* text, const ba_block_meta* meta,
                             int32_t n_blocks, float scale, void* out, float* lse,
                             void* workspace, size_t workspace_bytes,
                             hipStream_t stream);

/*
 * ba_block_attention for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same arguments and results, without a workspace argument.
 * The split schedule's partial results go to a device array the library
 * holds itself (72 MiB on each GPU it runs on, kept until the process
 * ends); the call allocates nothing.  Calls on one GPU share that array:
 * calls that overlap on one GPU (other streams, other threads) race and must
 * be ordered by the caller.  BA_ERR_OUT_OF_RANGE when the device would need
 * more than 72 MiB of partial results (more workgroup slots than 256 CUs
 * hold); fp32 rings use no scratch.
 */
ba_status ba_block_attention_static(const void* q, int32_t q_stride, const ba_ring* cache,
                                    const ba_ring* text, const ba_block_meta* meta,
                                    int32_t n_blocks, float scale, void* out, float* lse,
                                    hipStream_t stream);

/* Workspace bytes for ba_block_attention on the current device (0: none is
 * used, e.g. fp32, or no device): two partial results per workgroup the
 * device holds at once.  A smaller buffer still works, with fewer workgroups
 * sharing the split. */
size_t ba_attention_workspace_bytes(int32_t head_dim, int32_t dtype, int32_t n_blocks,
                                    int32_t q_stride, int32_t heads);

/*
 * The text part of the key set (the text K/V every block of a call attends
 * to besides its cache segments; DualParal Abstract, pith.science verdict,
 * core_discovery) given as plain arrays: text_k, text_v are
 * [heads][text_cap][head_dim] in the ring's dtype, head-major, 16-byte
 * aligned.  Tokens [0, text_len) go into slot `slot` of the ring `text`
 * (K rows as they are, V transposed to the ring's layout) and tokens
 * [text_len, T_pad) of that slot become zeros; text->appended is unchanged.
 * 1 <= text_len <= min(text_cap, text->slot_tokens).  One launch; pure data
 * movement (the slot holds the exact bits afterwards).
 */
ba_status ba_text_ring_set(const ba_ring* text, int32_t slot, const void* text_k,
                           const void* text_v, int32_t text_cap, int32_t text_len,
                           hipStream_t stream);

/*
 * ba_block_attention with the text K/V as plain arrays (as for
 * ba_text_ring_set; NULL allowed when every text_len is 0) instead of a text
 * ring: every meta[b].text_slot must be 0 and text_len <= text_cap.  The
 * call writes the text (the longest text_len of the call) into a one-slot
 * ring at the start of `workspace`, then runs ba_block_attention on it with
 * the rest of the workspace for the split schedule's partial results.  The
 * workspace (256-byte aligned, caller-owned, no initialisation needed) must
 * hold the ring when any text_len > 0: ba_attention_text_arrays_workspace_bytes
 * gives the ring plus a full ba_attention_workspace_bytes; any size from the
 * ring's up works, with fewer tail workgroups.  Every check of both steps
 * runs before either launch.  Results are those of ba_block_attention on a
 * ring filled with the same text.  Callers that keep one prompt for many
 * calls save the per-call text copy by filling a text ring once
 * (ba_text_ring_set) and calling ba_block_attention.
 */
ba_status ba_block_attention_text_arrays(const void* q, int32_t q_stride, const ba_ring* cache,
                                         const void* text_k, const void* text_v,
                                         int32_t text_cap, const ba_block_meta* meta,
                                         int32_t n_blocks, float scale, void* out, float* lse,
                                         void* workspace, size_t workspace_bytes,
                                         hipStream_t stream);

/* Workspace bytes for ba_block_attention_text_arrays on the current device:
 * the one-slot text ring of text_cap tokens (rounded up to 256 bytes), then
 * ba_attention_workspace_bytes.  0 for a bad shape. */
size_t ba_attention_text_arrays_workspace_bytes(int32_t head_dim, int32_t dtype, int32_t n_blocks,
                                                int32_t q_stride, int32_t heads, int32_t text_cap);

/* Queries of one head that one workgroup of ba_block_attention takes (its
 * query tile) in a launch whose longest key set (cache segments + text) has
 * max_keys keys: a block of q_len queries is heads * ceil(q_len / tile)
 * tasks.  bf16, head_dim 64: 32 up to 512 keys (the resident shape: each
 * workgroup holds one head's whole key set in LDS and its waves take units
 * of 32 queries), 128 up to 3072 keys (short key sets, several workgroups
 * per CU), else 384; head_dim 128: 256; fp32: 64.  A launch with key sets of
 * at most 512 keys takes the resident shape only when every key set spans at
 * most 8 tiles of 64 keys (tiles do not cross segments) and it has at least
 * as many 32-query units as the device has wave slots for it (12 per CU);
 * else it takes the 128-query shape.  A call covers its blocks in launches of
 * up to 16.  0 for a head_dim / dtype pair the call does not support or
 * max_keys < 0.  Needs no device. */
int32_t ba_attention_query_tile(int32_t head_dim, int32_t dtype, int32_t max_keys);

/* The schedule ba_block_attention would take for these arguments and a
 * workspace of workspace_bytes (0: none), without launching anything:
 * *tail_workgroups = tail workgroups per XCD sharing the split (the largest
 * over the call's launches of 16 blocks), 0 when every workgroup runs whole
 * query tiles.  Same argument checks as ba_block_attention; with a workspace
 * and a bf16 ring it queries the current device. */
ba_status ba_attention_plan(int32_t q_stride, const ba_ring* cache, const ba_ring* text,
                            const ba_block_meta* meta, int32_t n_blocks, size_t workspace_bytes,
                            int32_t* tail_workgroups);

/*
 * Fused K/V producer: the QKV projection of one block, written where it is
 * consumed.  The feature cache (DualParal Abstract) holds the self-attention
 * K/V a block produced; this call produces them with the block's projection
 * and stores K and V straight into ring slot `slot` (the layout of
 * ba_cache_append, tokens [n_tokens, T_pad) zeroed), and Q into q:
 *   Y = X W^T;  q | k | v = Y[:, 0:HD] | Y[:, HD:2HD] | Y[:, 2HD:3HD]  (HD = heads * head_dim)
 * then, if rope is given, every adjacent pair (y[2p], y[2p+1]) of q and k is
 * rotated by the table's (c, s) for its token and pair: (y0 c - y1 s,
 * y0 s + y1 c), the same for every head.
 * x:    [n_tokens][dim] bf16, 1 <= n_tokens <= cache->slot_tokens, dim a
 *       multiple of 64 (n_tokens * dim < 2^30).
 * w:    [3 * heads * head_dim][dim] bf16 (a linear layer's weight: output
 *       rows q, then k, then v, each head-major).
 * q:    [n_tokens][heads][head_dim] bf16, or NULL to skip the q rows.
 * cache: bf16 ring; heads and head_dim (64 or 128) give the shapes.
 * rope: [head_dim / 2][n_tokens][2] fp32 (cos, sin) of pair p at token t at
 *       element 2 (p n_tokens + t): pair-major, so that consecutive tokens
 *       read one run; 8-byte aligned, or NULL.
 * Products accumulate in fp32 on the matrix cores; the rotation is fp32;
 * every output is rounded once to bf16 (nearest even).  Does not change
 * cache->appended.
 */
ba_status ba_qkv_project(const void* x, int32_t n_tokens, int32_t dim, const void* w, void* q,
                         const ba_ring* cache, int32_t slot, const float* rope, hipStream_t stream);

/* The same for n_blocks blocks of n_tokens tokens in one launch (the queued
 * blocks of one step): x [n_blocks][n_tokens][dim], q [n_blocks][n_tokens]
 * [heads][head_dim] or NULL, block b's K/V into ring slot slots[b] (host
 * array; 1 <= n_blocks <= 64, slots distinct).  rope: NULL, or block b's
 * pair-major table at rope + b * rope_block_stride floats (stride 0: one
 * table for every block, else >= n_tokens * head_dim).  Each block's outputs
 * are bit-identical to a ba_qkv_project call on that block alone. */
ba_status ba_qkv_project_batched(const void* x, int32_t n_blocks, int32_t n_tokens, int32_t dim, const void* w,
                                 void* q, const ba_ring* cache, const int32_t* slots, const float* rope,
                                 int64_t rope_block_stride, hipStream_t stream);

/*
 * Noise schedule of the per-block update.  NULL selects the default
 * {T = 1000, stride = 20, beta_start = 1e-4, beta_end = 0.02, BA_SCHED_DDIM}.
 *
 * BA_SCHED_DDIM: eps-prediction DDIM (eta = 0) on the DDPM linear beta
 *   schedule, see ba_block_update.
 * BA_SCHED_FLOW: velocity-prediction flow matching (rectified flow, the
 *   family of the Wan2.1 generator the DualParal page evaluates on, named on
 *   the pages only through flow-matching titles): noise level
 *   sigma(t) = shift * u / (1 + (shift - 1) * u), u = t / T (shift = 1: linear),
 *   and one Euler step x' = x + (sigma(t') - sigma(t)) * v, i.e. c1 = 1,
 *   c2 = sigma(t') - sigma(t); the second input of ba_block_update is the
 *   predicted velocity v.  beta_start / beta_end are not used.
 */
typedef enum { BA_SCHED_DDIM = 0, BA_SCHED_FLOW = 1 } ba_schedule_kind;

typedef struct {
  int32_t T;                  /* number of training timesteps (>= 2)         */
  int32_t stride;             /* t' = max(t - stride, 0), stride >= 0        */
  double  beta_start, beta_end; /* DDIM: 0 < beta_start <= beta_end < 1      */
  int32_t kind;               /* ba_schedule_kind                            */
  double  shift;              /* FLOW: sigma shift, 0 < shift <= 1e6         */
} ba_schedule;

/*
 * Per-block denoising update, in place on x (bf16):
 *   x'[b][e] = c1(t_b) * x[b][e] + c2(t_b) * eps[b][e]
 * the deterministic DDIM step (eta = 0) from t_b to t_b' = max(t_b - stride, 0)
 * on the DDPM linear beta schedule (abar_t = prod_{s<=t}(1 - beta_s),
 * abar_0 = 1): c1 = sqrt(abar_t'/abar_t),
 * c2 = sqrt(1 - abar_t') - sqrt(abar_t') sqrt(1 - abar_t) / sqrt(abar_t).
 * Each queued block sits at its own timestep (DualParal Abstract: blocks at
 * progressively decreasing noise levels; pith.science verdict, key_machinery).
 * x, eps: [n_blocks][elems_per_block] bf16 (elems_per_block <= 2^40);
 * t_per_block: (host) n_blocks
 * integers in [0, T].  Coefficients are computed on the host in fp64 and
 * applied as fp32 FMAs; the result is rounded to bf16 (nearest even).
 */
ba_status ba_block_update(void* x, const void* eps, int64_t elems_per_block,
                          const int32_t* t_per_block, int32_t n_blocks,
                          const ba_schedule* sched, hipStream_t stream);

/* Host only: the fp32 (c1, c2) pairs ba_block_update would apply (either
 * schedule kind). */
ba_status ba_schedule_coefficients(const ba_schedule* sched, const int32_t* t,
                                   int32_t n, float* c1, float* c2);

/*
 * Single-GPU FIFO block queue: host bookkeeping only (no device memory, no
 * launch).  Block-wise denoising as the pith.science verdict on the DualParal
 * page describes it (pith_extraction.key_machinery): the queued blocks sit at
 * monotonically decreasing noise levels from tail to head, and every step
 * appends a new noisy block at the tail and pops a clean one at the head.
 *
 * Here the queue holds n_queue blocks.  Before a step, queue position i
 * (0 = head) sits at timestep t_i = (i + 1) * T / n_queue (T divisible by
 * n_queue); the step moves every block down one rung (stride T / n_queue), so
 * the head reaches t = 0 and leaves, and a block of pure noise (t = T) enters
 * at the tail.  Blocks carry absolute ids k (the head has the smallest);
 * the caller keeps block k's latents in latent slot k mod n_queue, so the
 * entering block takes the leaving block's slot.
 *
 * Feature cache (DualParal Abstract: the prior block's features are stored
 * and reused as context): at step g block k writes its K/V into ring slot
 *   2 * (k mod n_queue) + (g mod 2)
 * and reads, besides its own K/V and the text, the K/V its neighbour toward
 * the head (block k - 1) wrote at step g - 1, one step old as in the
 * pipelined original, from slot 2 * ((k - 1) mod n_queue) + ((g - 1) mod 2):
 * the slots a step reads and the slots it writes differ in parity, so no
 * write of a step overwrites what the step reads (the block that leaves after
 * step g - 1 is still read as the head's context at step g).  At step 0
 * there is no such context.  The ring needs 2 n_queue slots of block_tokens
 * each; the text sits in slot 0 of a text ring.
 */
typedef struct {
  int32_t n_queue;            /* blocks in the queue, 1..BA_QUEUE_MAX          */
  int32_t T;                  /* noise levels, a multiple of n_queue           */
  int32_t block_tokens;       /* tokens (keys and queries) per block           */
  int32_t text_len;           /* text keys, 0.. (slot 0 of the text ring)      */
  int64_t step;               /* steps taken so far (g of the next step)       */
  int64_t head_id;            /* absolute id of the head block                 */
} ba_queue;

#define BA_QUEUE_MAX 4096

/* Fill in *q: step = 0, head_id = 0. */
ba_status ba_queue_init(ba_queue* q, int32_t n_queue, int32_t T, int32_t block_tokens, int32_t text_len);

/* Ring slots the queue's feature cache needs: 2 n_queue, or 0 if n_queue is
 * out of range. */
int32_t ba_queue_ring_slots(int32_t n_queue);

/*
 * The next step's plan, indexed by latent slot m = 0..n_queue-1 (host arrays
 * of n_queue entries, owned by the caller): the ring slot the block in latent
 * slot m writes its K/V to (write_slots[m], for ba_cache_append_batched), its
 * key set (meta[m], for ba_block_attention: [neighbour's K/V of the previous
 * step | own K/V | text]) and its timestep (t[m], for ba_block_update);
 * *stride receives T / n_queue (the schedule stride of the update).
 */
ba_status ba_queue_plan(const ba_queue* q, int32_t* write_slots, ba_block_meta* meta, int32_t* t,
                        int32_t* stride);

/* After the step: the head (now at t = 0, latent slot head_id mod n_queue)
 * has left and the new tail block takes its latent slot; head_id and step
 * advance by one. */
ba_status ba_queue_advance(ba_queue* q);

/*
 * Coordinated noise initialisation.  Every GPU holds the same noise pool
 * (DualParal Abstract: initial noise patterns shared across GPUs at no extra
 * cost) and each new block takes its latent frames from the whole pool by a
 * shuffled assignment that leaves out the pool's last few latents (the
 * pith.science verdict on it, pith_inferences), so that concatenated blocks
 * do not repeat one noise pattern.  The pool is the caller's (for instance
 * N(0, 1) noise of the model's native clip length drawn from one seed).
 */
#define BA_NOISE_MAX_FRAMES 64

/* (host only) The pool frames block `block_id` takes, in its frame order:
 * block_frames distinct frames of [0, pool_frames - n_exclude), the first
 * block_frames entries of a uniformly random permutation of those candidates
 * (partial Fisher-Yates from the front: position i swaps with a uniform
 * position in [i, m), m = pool_frames - n_exclude).  Random words come from
 * SplitMix64 (Steele, Lea, Flood 2014: state += 0x9E3779B97F4A7C15, output
 * the state through z ^= z >> 30, z *= 0xBF58476D1CE4E5B9, z ^= z >> 27,
 * z *= 0x94D049BB133111EB, z ^= z >> 31); block b's generator is seeded with
 * output b (0-based) of the generator seeded with `seed`, so each GPU computes
 * any block's frames alone.  A uniform draw below n rejects words under
 * 2^64 mod n and takes the rest mod n.  frames: block_frames int32 (host).
 * Requires 0 <= n_exclude < pool_frames, 1 <= block_frames <=
 * min(pool_frames - n_exclude, BA_NOISE_MAX_FRAMES), block_id >= 0. */
ba_status ba_noise_assign(uint64_t seed, int64_t block_id, int32_t pool_frames, int32_t n_exclude,
                          int32_t block_frames, int32_t* frames);

/* The block's noise: out[c][f][:] = pool[c][frames[f]][:] for c < channels,
 * f < block_frames (pool: [channels][pool_frames][frame_bytes] bytes, out:
 * [channels][block_frames][frame_bytes]; any element type).  frames (host):
 * block_frames entries in [0, pool_frames), e.g. from ba_noise_assign.
 * pool and out 16-byte aligned, frame_bytes a positive multiple of 16,
 * channels * block_frames <= 65535, block_frames <= BA_NOISE_MAX_FRAMES; out
 * must not overlap the pool.  Enqueued on `stream`. */
ba_status ba_noise_block(const void* pool, int32_t channels, int32_t pool_frames, int64_t frame_bytes,
                         const int32_t* frames, int32_t block_frames, void* out, hipStream_t stream);

const char* ba_status_string(ba_status status);
const char* ba_last_error(void);
int32_t     ba_version(void);   /* major*10000 + minor*100 + patch */

#ifdef __cplusplus
}
#endif

#endif /* BLOCKATTN_H */
