/*
 * hsa.h - C ABI of the heterogeneous sparse-attention KV cache (MI355X, gfx950).
 *
 * The library keeps the two pools of the DeepSeek-V4 heterogeneous KV layout on
 * one GPU and runs the decode step over them:
 *
 *   State Cache  one fixed-size block per request: the SWA ring of the last
 *                n_win tokens' exact K/V and the in-flight tail of the open
 *                128-token block (its indexer keys; its K/V are the newest
 *                ring slots).
 *   Block Cache  sealed, immutable, refcounted blocks of lcm(4, 128) = 128
 *                tokens, each holding 32 CSA (C4) entries, 1 HCA entry and the
 *                128 tokens' indexer keys.
 *
 * Options at create time: a stack of layers of four types over one State quota
 * and one Block Cache (HSA_LAYER_*), FP8 C4 entries (HSA_ENTRY_FP8), MXFP4 indexer
 * keys (HSA_INDEX_MXFP4) and eager C4 entries of the open block (HSA_C4_EAGER).
 * Prefix hits under the pages' three SWA policies are built from hsa_block_ref,
 * hsa_prefix_attach, hsa_state_write and State checkpoints.
 *
 * Pages cited (by title and section):
 *   [Q&A]    "V4 为何要分池？块对齐与尾缓冲怎么配合？" (deepseek-tech-notes)
 *   [Layout] "V4 KV Layout：Classical + State 双池" (deepseek-tech-notes)
 *   [Ch12]   "Ch 12 · 推理框架 — KV 的异构调度" (DeepSeek-V4-book)
 *   [Disk]   "V4 磁盘 Prefix Cache" (deepseek-tech-notes)
 *
 * Conventions for every call:
 *   - Shapes are fixed: 16 heads x 128 bf16 for K/V/Q, 4 heads x 64 fp32 for
 *     indexer keys/queries, m = 4, m' = 128 (other values: HSA_ERR_INVALID).
 *   - "dev" pointers are device memory owned by the caller, alive until the
 *     work enqueued on `stream` has run; "host" arrays are read during the
 *     call only. `stream` is a hipStream_t passed as void* (NULL = default).
 *   - Host metadata (lengths, block tables, refcounts) changes at call time;
 *     device work is enqueued on `stream` and never waited for, except by the
 *     introspection calls, which synchronise `stream`.
 *   - Every argument and capacity check runs before any metadata changes or
 *     any work is enqueued: a call that returns an error changed nothing.
 *     HSA_ERR_DEVICE (a HIP runtime failure) leaves the context unusable
 *     except for hsa_destroy.
 *   - A context is not thread safe, and its calls must be issued on one stream
 *     at a time (calls share scratch memory).
 */
#ifndef HSA_H
#define HSA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t hsa_status;
#define HSA_OK 0
#define HSA_ERR_INVALID (-1)     /* bad argument, shape, id or unallocated state   */
#define HSA_ERR_OOM_BLOCKS (-2)  /* Block Cache or a state's block table is full   */
#define HSA_ERR_OOM_STATES (-3)  /* no free State slot                             */
#define HSA_ERR_STATE (-4)       /* lifecycle: share into a non-empty state, append
                                    to a full deferred tail, deferred append past
                                    one block                                      */
#define HSA_ERR_DEVICE (-5)      /* HIP runtime error                              */

#define HSA_APPEND_DEFER_SEAL 1u

#define HSA_MAX_TOPK 4096        /* largest k accepted by indexer_topk / attend     */

#define HSA_TOPK_SORTED 1u       /* top-k rows by (score desc, ordinal asc)         */

typedef struct hsa_ctx hsa_ctx;

typedef struct hsa_config {
  int32_t n_heads;              /* 16                                               */
  int32_t head_dim;             /* 128                                              */
  int32_t m_csa;                /* 4   ([Q&A] §1.2: CSA compresses 4 tokens)        */
  int32_t m_hca;                /* 128 ([Q&A] §1.2: HCA compresses 128 tokens)      */
  int32_t n_win;                /* SWA tokens; multiple of 128 ([Ch12] 公式白话翻译:
                                   the window is an integer number of blocks)       */
  int32_t idx_heads;            /* 4                                                */
  int32_t idx_dim;              /* 64                                               */
  int32_t max_states;           /* State slots                                      */
  int64_t max_blocks;           /* physical blocks in the Block Cache               */
  int64_t max_blocks_per_state; /* block-table row length; 0 = max_blocks           */
  const float* gate_csa;        /* host [n_layers][n_heads][head_dim] compressor gates,
                                   copied (one [n_heads][head_dim] row set per layer) */
  const float* gate_hca;        /* host [n_layers][n_heads][head_dim], copied       */
  int32_t entry_format;         /* storage of C4 entries: HSA_ENTRY_BF16 or
                                   HSA_ENTRY_FP8 ([Ch12] §2.2 accounts entries in FP8) */
  int32_t index_format;         /* storage of sealed indexer keys: HSA_INDEX_F32 or
                                   HSA_INDEX_MXFP4 ([Ch12] §2.2 stores them as FP4) */
  int32_t n_layers;             /* attention layers sharing the State quota and the
                                   Block Cache; 0 means 1                           */
  const int32_t* layer_types;   /* host [n_layers] HSA_LAYER_*, copied; NULL: every
                                   layer HSA_LAYER_MIXED                            */
  int32_t c4_mode;              /* HSA_C4_SEALED or HSA_C4_EAGER                    */
  uint32_t create_flags;        /* 0 or HSA_CREATE_POISON                           */
  int32_t kv_format;            /* storage of SWA ring tokens and HCA entries: HSA_KV_BF16
                                   or HSA_KV_FP8 ([Ch12] §1 accounts them in FP8)     */
  int32_t reserved;             /* 0                                                */
} hsa_config;

/* SWA ring and HCA entry storage. BF16: K and V rows of 16 x 128 bf16. FP8: each
 * token's K and V (as it enters the State: append, replay, fork, restore) and each
 * HCA entry (at its seal) are stored per head as E4M3 codes and a float32 scale, by
 * the HSA_ENTRY_FP8 rule; the State keeps no other copy of a token, so the seal pools
 * the stored values of a block's tokens and attention reads them. Indexer keys are
 * not affected. Not with HSA_C4_EAGER. */
#define HSA_KV_BF16 0
#define HSA_KV_FP8 1

/* Create flag: fill every pool and every scratch buffer with 0xFF bytes when it is
 * allocated (bf16, fp32 and E4M3 NaN, E8M0 NaN scales, table entries -1), so that a
 * read of a slot that was never written shows as NaN in the results. A debugging and
 * test aid; it costs one device fill per allocation. */
#define HSA_CREATE_POISON 1u

/* When C4 entries exist. SEALED: a block's 32 entries are written when its 128 tokens
 * are complete ([Q&A] §3.1 block-level sealing). EAGER: each complete group of 4
 * tokens of the open block (L mod 4 = 0, the CSA tail of [Q&A] §3.1) has its entry
 * at once, pooled as the seal pools it (bit-identical), kept in the State; the
 * open block's g = (L mod 128) / 4 entries (32 with a deferred full tail) are top-k
 * candidates with ordinals 32 nb .. 32 nb + g - 1, scored from the indexer tail, and
 * attention keys when selected. EAGER takes bf16 entries and fp32 indexer keys. */
#define HSA_C4_SEALED 0
#define HSA_C4_EAGER 1

/* Layer types ([Ch12] Figure 12-1: per request one State quota over all layers - SWA
 * layers, CSA state, HCA state - and per block the layers' compressed KV - CSA
 * indexer keys, CSA main KV, HCA KV). Every type keeps an SWA window of n_win tokens.
 *   MIXED  32 C4 + 1 HCA + 128 indexer keys per block; attention over SWA, every HCA
 *          entry and the top-k C4 entries in one softmax (the single-layer path).
 *   SWA    nothing in the Block Cache; attention over the SWA only.
 *   CSA    32 C4 + 128 indexer keys per block; attention over SWA and the top-k C4.
 *   HCA    1 HCA entry per block; attention over SWA and every HCA entry.
 * A top-k row of a layer without C4 entries is all -1.
 *
 * Layers: data calls act on the current layer (hsa_set_layer; 0 after create). An
 * append (hsa_append_kv, hsa_compress_flush, hsa_decode_step) is made at layer 0,
 * which checks it and commits it to the shared State lengths and block tables; the
 * same call (same states, token counts, flags) must then be made at layers 1 .. n-1
 * in order, each with its own layer's K/V (and indexer keys, queries), before any
 * other call that changes states or blocks (those return HSA_ERR_STATE meanwhile).
 * Reads, exports, hsa_state_write, checkpoints and restores act on the current layer
 * at any time. */
#define HSA_LAYER_MIXED 0
#define HSA_LAYER_SWA 1
#define HSA_LAYER_CSA 2
#define HSA_LAYER_HCA 3

/* C4 entry storage. BF16: K and V rows of 16 x 128 bf16. FP8: per head, 128 OCP
 * FP8 E4M3 codes and one float32 scale s = amax / 448, amax = max |x| over the
 * head's 128 values (s = 1 where amax / 448 is not a normal float32: an all-zero
 * head, or amax below 448 * 2^-126); code = E4M3(x / s), round to nearest, ties to
 * even, with x, s and the quotient float32 and each division correctly rounded;
 * the entry reads as code value * s. The pages give no scale scheme: this
 * per-head scale is the reading used. HCA entries are always bf16. */
#define HSA_ENTRY_BF16 0
#define HSA_ENTRY_FP8 1

/* Sealed indexer key storage. F32: [128][4][64] float32 per block. MXFP4 (OCP
 * Microscaling): each key's 256 values form 8 blocks of 32 (block 2h + j = head h,
 * dims 32j .. 32j + 31) with one E8M0 scale byte E + 127, E = floor(log2 max |x|)
 * - 2, at least -127 (-127 for an all-zero block), and E2M1 codes of x / 2^E
 * (nearest of 0, .5, 1, 1.5, 2, 3, 4, 6, ties to the even code, saturating at 6,
 * sign bit for x < 0); value 2i in the low nibble of byte i. The key reads as code
 * value * 2^E. The open block's keys (the State's indexer tail) stay float32 until
 * the block seals; queries are float32. The pages give no scale scheme: the OCP
 * block scaling is the reading used. */
#define HSA_INDEX_F32 0
#define HSA_INDEX_MXFP4 1

typedef struct hsa_state_info {
  int64_t len;          /* L, tokens appended so far                                 */
  int64_t n_blocks;     /* sealed blocks in the state's block table                  */
  int32_t csa_tail;     /* L mod 4                                                   */
  int32_t hca_tail;     /* tokens in the open block: L - 128 * n_blocks (<= 128)     */
  int32_t swa_len;      /* min(L, n_win)                                             */
  int32_t pending_seal; /* 1 if a deferred full tail awaits hsa_compress_flush       */
} hsa_state_info;

/* Create a context on `device`: validates `cfg`, allocates every pool in device
 * memory (owned by the context until hsa_destroy) and copies the gates.
 * Pools: SWA ring K and V [max_states][n_win][16][128] bf16, indexer tail
 * [max_states][128][4][64] fp32, C4 K and V [max_blocks][32][16][128] bf16 (FP8
 * entries: codes [max_blocks][32][K, V][16][128] u8 and scales
 * [max_blocks][32][K, V][16] fp32), HCA K and V [max_blocks][16][128] bf16, indexer
 * keys [max_blocks][128][4][64] fp32, block table [max_states][max_blocks_per_state]
 * int32.
 * ([Q&A] §1.1: two pools with different lifetimes; [Ch12] §2.1, §2.2.) */
hsa_status hsa_create(const hsa_config* cfg, int device, hsa_ctx** out);
hsa_status hsa_destroy(hsa_ctx* ctx);

/* Take the lowest free State slot; its length is 0 and its table empty.
 * ([Ch12] §2.1: one State block per request for its whole life.) */
hsa_status hsa_state_alloc(hsa_ctx* ctx, int32_t* state_out);

/* Release a State slot: drop one reference from each of its blocks; a block
 * whose count reaches 0 returns to the free list. No device work.
 * ([Ch12] §2.1: the block is freed whole at request end; §2.2: refcounts.) */
hsa_status hsa_state_free(hsa_ctx* ctx, int32_t state);

/* Append tokens to n_req distinct states ([Q&A] §4 steps 1-3; §3.1).
 *   states    host [n_req]
 *   cu_tokens host [n_req+1], cu_tokens[0] = 0, nondecreasing: request i owns
 *             rows cu_tokens[i] .. cu_tokens[i+1]-1 of the packed inputs
 *   k, v      dev bf16 [T][16][128], T = cu_tokens[n_req]
 *   idx_k     dev fp32 [T][4][64] (indexer keys)
 * Token at position p goes to SWA ring slot p mod n_win and indexer-tail slot
 * p mod 128. Without flags, each time a state's open block reaches 128 tokens
 * it is sealed: a block id is taken (lowest free id; requests in call order,
 * blocks in token order), its 32 C4 entries (tokens 4j..4j+3) and its HCA
 * entry (all 128 tokens) are computed by gated pooling and stored as bf16,
 * and the 128 indexer keys are copied in. With HSA_APPEND_DEFER_SEAL the open
 * block may fill to exactly 128 tokens and waits for hsa_compress_flush;
 * going past 128 is HSA_ERR_STATE, as is any append to a state whose full
 * tail awaits a flush. Errors: INVALID, OOM_BLOCKS, STATE. */
hsa_status hsa_append_kv(hsa_ctx* ctx, int32_t n_req, const int32_t* states,
                         const int64_t* cu_tokens, const void* k, const void* v,
                         const float* idx_k, uint32_t flags, void* stream);

/* Seal every listed state whose open block holds 128 tokens (deferred seals);
 * others are left as they are. ([Q&A] §3.1: full block -> compress -> append
 * to the Classical pool.) Errors: INVALID, OOM_BLOCKS. */
hsa_status hsa_compress_flush(hsa_ctx* ctx, int32_t n_req, const int32_t* states,
                              void* stream);

/* Make `dst` (allocated, L = 0) a fork of `src`: dst's table references every
 * sealed block of src (refcount + 1 each) and src's State (SWA ring, indexer
 * tail, L) is copied into dst's slot on `stream`. ([Ch12] §2.2: requests with
 * the same prefix reference the same block, refcounted.) Errors: INVALID
 * (bad ids, src == dst), STATE (dst not empty, src has a pending seal). */
hsa_status hsa_block_table_share(hsa_ctx* ctx, int32_t src, int32_t dst, void* stream);

/* ---- prefix hits under the three SWA policies ([Ch12] §3.1; [Disk] SWA
 * policies: Full / Periodic Checkpointing / Zero).
 * A prefix entry holds the prefix's sealed blocks by reference (hsa_block_ref) and,
 * by policy, State checkpoints. A hit makes a fresh state from it:
 *   Zero      hsa_prefix_attach, then hsa_state_write of the prefix's tokens
 *             [max(0, len - n_win), len) (raw K, V, indexer keys);
 *   Periodic  hsa_prefix_attach, hsa_state_restore of the latest checkpoint c <= len,
 *             then hsa_state_write of the tokens [c, len);
 *   Full      hsa_prefix_attach, then hsa_state_restore of the checkpoint at len.
 * (hsa_state_restore_batch restores a whole batch of hits in one launch.)
 * Each gives the state, slot for slot, that hsa_block_table_share of a live request
 * at len gives; the shared blocks are never sealed again. Until its window is
 * filled that way, an attached state must not be read or appended to (the library
 * cannot tell). */

/* Add delta (+1 or -1) to the refcount of each listed block (host [n]; a block may
 * repeat), so that a prefix entry can hold blocks with no state. +1 needs each block
 * in use; -1 may not release more than is held; a block reaching 0 is freed. Checked
 * as a whole: on error nothing changes. No device work. Errors: INVALID. */
hsa_status hsa_block_ref(hsa_ctx* ctx, const int32_t* blocks, int64_t n, int32_t delta);

/* Each of n_req distinct states (allocated, L = 0) takes len[i] and, as its sealed
 * blocks, blocks[block_off[i] .. block_off[i] + len[i] / 128) of a host list of
 * n_blocks ids (each used one in use; requests of one prefix may point at the same
 * range), refcount + 1 per reference. The table rows are written on `stream` (one
 * launch); the SWA rings and indexer tails are left as they are (fill them as
 * above). len, block_off: host [n_req]. Checked as a whole. Errors: INVALID (bad ids,
 * lengths or offsets), STATE (a state not empty). */
hsa_status hsa_prefix_attach(hsa_ctx* ctx, int32_t n_req, const int32_t* states, const int64_t* len,
                             const int32_t* blocks, int64_t n_blocks, const int64_t* block_off,
                             void* stream);

/* Replay raw tokens into states without sealing. Request i writes input rows
 * [cu_tokens[i], cu_tokens[i+1]) as positions pos0[i] .. pos0[i] + n_i - 1, which must
 * lie in [0, L) of states[i] (distinct states). A position in the window
 * [L - n_win, L) goes to ring slot p mod n_win, one of the open block also to indexer
 * tail slot p mod 128; older positions are skipped. L and the block table do not
 * change. k, v: device bf16 [T][16][128]; idx: device fp32 [T][4][64]; cu_tokens,
 * pos0: host [n_req + 1], [n_req]. Errors: INVALID. */
hsa_status hsa_state_write(hsa_ctx* ctx, int32_t n_req, const int32_t* states,
                           const int64_t* cu_tokens, const int64_t* pos0, const void* k,
                           const void* v, const float* idx, void* stream);

/* Bytes of one State checkpoint: SWA ring K and V (n_win x 4 KiB each; with FP8 KV
 * the ring's codes, n_win x 4 KiB, and scales, n_win x 128 B), then the indexer tail
 * (128 x 1 KiB). */
hsa_status hsa_checkpoint_bytes(hsa_ctx* ctx, int64_t* bytes);

/* Copy a state's SWA ring and indexer tail into `buf` (device or pinned host memory,
 * hsa_checkpoint_bytes long, owned by the caller) on `stream`; *len_out = its L, the
 * checkpoint's position. Errors: INVALID, STATE (pending seal). */
hsa_status hsa_state_checkpoint(hsa_ctx* ctx, int32_t state, void* buf, int64_t* len_out,
                                void* stream);

/* Copy a checkpoint taken at ckpt_len (<= the state's L, from the same prefix) into
 * the state's ring and tail slots on `stream`. Positions [ckpt_len, L) keep whatever
 * their slots hold until replayed with hsa_state_write, so restore first. Errors:
 * INVALID. */
hsa_status hsa_state_restore(hsa_ctx* ctx, int32_t state, const void* buf, int64_t ckpt_len,
                             void* stream);

/* hsa_state_restore of n distinct states in one copy launch (the Full and Periodic
 * policies restore a whole batch of hits at once; same source as hsa_state_restore):
 * state states[i] takes the checkpoint in bufs[i], taken at ckpt_lens[i]. states,
 * bufs and ckpt_lens are host arrays of n; each bufs[i] is a checkpoint
 * (hsa_checkpoint_bytes long, 16-byte aligned, owned by the caller) in device
 * memory or in pinned host memory the device can read. Every argument is checked
 * before anything is copied. Errors: INVALID (bad or repeated state, a length past
 * the state's L, a NULL, misaligned or pageable host buffer). */
hsa_status hsa_state_restore_batch(hsa_ctx* ctx, int32_t n, const int32_t* states,
                                   const void* const* bufs, const int64_t* ckpt_lens, void* stream);

/* Indexer top-k over each state's sealed C4 entries ([Ch12] 名词速通: the
 * indexer's K-only keys serve top-k selection; [Layout] Classical KV cache:
 * CSA entries are read sparsely through top-k).
 *   q_idx     dev fp32 [n_req][4][64]
 *   idx_out   dev int32 [n_req][k]: C4 ordinals j (block j/32, slot j%32 of
 *             the state's table) of the kk = min(k, 32 * n_blocks) entries that
 *             come first by score descending, ties to the lowest ordinal; they
 *             are written in ascending ordinal order, or in that selection order
 *             with HSA_TOPK_SORTED; -1 after kk
 *   score_out dev fp32 [n_req][k] or NULL: their scores, -inf after kk
 * Score of token t: sum over 4 heads x 64 dims of q_idx * idx_key_t; score of
 * C4 entry j = mean of its 4 tokens' scores. 1 <= k <= HSA_MAX_TOPK. */
hsa_status hsa_indexer_topk(hsa_ctx* ctx, int32_t n_req, const int32_t* states,
                            const float* q_idx, int32_t k, uint32_t flags, int32_t* idx_out,
                            float* score_out, void* stream);

/* Heterogeneous decode attention ([Q&A] §4 step 4: sparse/dense reads of the
 * compressed entries plus exact reads of the State): per request and head, one
 * softmax over the SWA tokens (min(L, n_win), the open tail included), the HCA
 * entries of every sealed block and the C4 entries named in the first
 * min(k, 32 * n_blocks) slots of its topk row (-1 and ordinals outside
 * [0, 32 * n_blocks) are skipped); scores are q.k / sqrt(128).
 *   q    dev bf16 [n_req][16][128]
 *   topk dev int32 [n_req][k] (NULL when k == 0)
 *   out  dev fp32 [n_req][16][128]
 * Every state must hold at least one token. 0 <= k <= HSA_MAX_TOPK. */
hsa_status hsa_decode_attend(hsa_ctx* ctx, int32_t n_req, const int32_t* states,
                             const void* q, const int32_t* topk, int32_t k,
                             float* out, void* stream);

/* One decode step ([Q&A] §4): append one token per request (k_new, v_new dev
 * bf16 [n_req][16][128], idx_new dev fp32 [n_req][4][64]) sealing full blocks,
 * then hsa_indexer_topk(q_idx, k, flags, topk_out, score_out), then
 * hsa_decode_attend(q, topk_out, k, out). Same argument rules as those calls;
 * k >= 1. */
hsa_status hsa_decode_step(hsa_ctx* ctx, int32_t n_req, const int32_t* states,
                           const void* k_new, const void* v_new, const float* idx_new,
                           const void* q, const float* q_idx, int32_t k, uint32_t flags,
                           int32_t* topk_out, float* score_out, float* out, void* stream);

/* hsa_decode_step for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc). Same
 * arguments, results and errors as hsa_decode_step, and the same kernels; every
 * kernel's scratch (score rows, attention partials, selected rows, top-k candidates,
 * seal partials) comes from one fixed device buffer of hsa_noalloc_scratch_bytes
 * bytes (32 MiB) that the library holds on each GPU until the process ends, so the
 * call allocates no device memory and never synchronises the device (it makes
 * no timing records either). A step whose largest batch of 64 requests needs more
 * scratch than the buffer holds returns HSA_ERR_INVALID before anything changes
 * (the need grows with the batch's longest score row: 128 B per sealed block of it
 * for each of the batch's requests, up to 64). Every context on a GPU shares that
 * GPU's buffer, which keeps the last call's contents (nothing in it needs to start
 * at zero): calls that overlap on one GPU - on different streams, or from different
 * contexts - race, so issue them in one stream order. */
hsa_status hsa_decode_step_noalloc(hsa_ctx* ctx, int32_t n_req, const int32_t* states,
                                   const void* k_new, const void* v_new, const float* idx_new,
                                   const void* q, const float* q_idx, int32_t k, uint32_t flags,
                                   int32_t* topk_out, float* score_out, float* out, void* stream);
/* Size in bytes of the fixed scratch buffer of hsa_decode_step_noalloc. */
hsa_status hsa_noalloc_scratch_bytes(int64_t* bytes);

/* Select the layer that data calls act on (0 <= layer < n_layers). Errors: INVALID. */
hsa_status hsa_set_layer(hsa_ctx* ctx, int32_t layer);

/* ---- introspection (host side; the export calls synchronise `stream`) ---- */
hsa_status hsa_state_query(hsa_ctx* ctx, int32_t state, hsa_state_info* out);
/* Copy up to `cap` ids of the state's block table to host `ids`; *n = count. */
hsa_status hsa_block_table_get(hsa_ctx* ctx, int32_t state, int32_t* ids, int64_t cap,
                               int64_t* n);
hsa_status hsa_block_refcount(hsa_ctx* ctx, int32_t block, int32_t* rc);
/* Copy one block to host buffers (any may be NULL): csa_k, csa_v bf16
 * [32][16][128] (must be NULL with FP8 entries: see hsa_export_c4_fp8); hca_k,
 * hca_v bf16 [16][128] (must be NULL with FP8 KV: see hsa_export_hca_fp8); idx_k
 * fp32 [128][4][64] (must be NULL with MXFP4 indexer keys: see
 * hsa_export_idx_mxfp4). */
hsa_status hsa_export_block(hsa_ctx* ctx, int32_t block, void* csa_k, void* csa_v,
                            void* hca_k, void* hca_v, float* idx_k, void* stream);
/* FP8 entries only: copy one block's C4 entries to host buffers (any may be NULL):
 * codes_k, codes_v u8 [32][16][128] E4M3 codes; scale_k, scale_v fp32 [32][16]
 * per-head scales. HSA_ERR_INVALID with bf16 entries. */
hsa_status hsa_export_c4_fp8(hsa_ctx* ctx, int32_t block, uint8_t* codes_k, uint8_t* codes_v,
                             float* scale_k, float* scale_v, void* stream);

/* The FP8 entry quantisation on its own (the one the seal applies to each head of a
 * C4 entry): for each of n_rows rows of 128 float32 values (device x
 * [n_rows][128]), writes device codes u8 [n_rows][128] and scales fp32 [n_rows].
 * Needs no context; n_rows >= 0. */
hsa_status hsa_fp8_quantize_rows(const float* x, int64_t n_rows, uint8_t* codes, float* scales,
                                 void* stream);

/* MXFP4 indexer keys only: copy one block's 128 sealed keys to host buffers (either
 * may be NULL): codes u8 [128][128] (E2M1 code pairs), scales u8 [128][8] (E8M0
 * bytes). HSA_ERR_INVALID with fp32 keys. */
hsa_status hsa_export_idx_mxfp4(hsa_ctx* ctx, int32_t block, uint8_t* codes, uint8_t* scales,
                                void* stream);

/* The MXFP4 key quantisation on its own (the one the seal applies to each indexer
 * key): for each of n_rows keys of 256 float32 values (device x [n_rows][256]),
 * writes device codes u8 [n_rows][128] and scale bytes u8 [n_rows][8]. Needs no
 * context; 0 <= n_rows <= 2^32. */
hsa_status hsa_mxfp4_quantize_rows(const float* x, int64_t n_rows, uint8_t* codes, uint8_t* scales,
                                   void* stream);

/* Copy one State block to host buffers (any may be NULL): swa_k, swa_v bf16
 * [n_win][16][128] in ring-slot order (token p sits in slot p mod n_win; must be
 * NULL with FP8 KV: see hsa_export_state_fp8); idx_tail fp32 [128][4][64] (token p in
 * slot p mod 128). */
hsa_status hsa_export_state(hsa_ctx* ctx, int32_t state, void* swa_k, void* swa_v,
                            float* idx_tail, void* stream);
/* FP8 KV only: copy one State's ring to host buffers (either may be NULL): codes u8
 * [n_win][K, V][16][128] E4M3 in ring-slot order, scales fp32 [n_win][K, V][16] per
 * head. HSA_ERR_INVALID with bf16 KV. */
hsa_status hsa_export_state_fp8(hsa_ctx* ctx, int32_t state, uint8_t* codes, float* scales,
                                void* stream);
/* FP8 KV only: copy one block's HCA entry to host buffers (either may be NULL): codes
 * u8 [K, V][16][128], scales fp32 [K, V][16]. HSA_ERR_INVALID with bf16 KV or in a
 * layer without HCA entries. */
hsa_status hsa_export_hca_fp8(hsa_ctx* ctx, int32_t block, uint8_t* codes, float* scales,
                              void* stream);

/* Per-kernel timing with HIP events recorded on the launch stream around each
 * launch of the kernels in `mask` (bit i = kernel id i below); 0 disables.
 * hsa_timing_read waits for the recorded events, returns total milliseconds
 * and launch counts per kernel id (arrays of HSA_KERNEL_COUNT) and clears. */
#define HSA_KERNEL_APPEND 0   /* decode append + fused seal            */
#define HSA_KERNEL_SEAL 1     /* bulk seal, or decode-seal HCA merge   */
#define HSA_KERNEL_WRITE 2    /* bulk ring / indexer-tail write        */
#define HSA_KERNEL_SCORE 3    /* indexer scores                        */
#define HSA_KERNEL_SELECT 4   /* top-k select                          */
#define HSA_KERNEL_ATTEND 5   /* split-KV attention partials           */
#define HSA_KERNEL_MERGE 6    /* attention partial merge               */
#define HSA_KERNEL_STEP1 7    /* decode step: append, seal, scores     */
#define HSA_KERNEL_STEP2 8    /* decode step: top-k select, HCA merge,
                                 attention over SWA + earlier HCA      */
#define HSA_KERNEL_STEP3 9    /* decode step: attention over selected
                                 C4 + the new HCA                      */
#define HSA_KERNEL_STEP4 10   /* decode step: partial merge            */
#define HSA_KERNEL_STEP2B 11  /* decode step: second top-k round over
                                 the candidates of sliced long rows    */
#define HSA_KERNEL_COUNT 12
hsa_status hsa_timing_enable(hsa_ctx* ctx, uint32_t mask);
hsa_status hsa_timing_read(hsa_ctx* ctx, double* ms, int64_t* launches);

const char* hsa_status_str(hsa_status s);
/* Text of the last error raised in this thread (argument or HIP failure). */
const char* hsa_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* HSA_H */
