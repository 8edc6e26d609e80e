/*
 * mtgr.h -- C ABI of libmtgr.so: forward pass of the MTGR HSTU encoder on one MI355X (gfx950),
 * the backward pass of one block, and the embedding front end (hash embedding store, key dedup).
 *
 * Page keys used in the citations below:
 *   [P1]/[P2] chenhuiyu blog post "MTGR" (Chinese / English)
 *   [P3] marovi.ai "MTGR: Industrial-Scale Generative Recommendation Framework in Meituan/zh"
 *   [P5] fun-rec mdbook section 7.3 "MTGR: Hybrid Paradigm Modeling"
 *
 * What the library computes (one HSTU block, [P3] section 方法, the two update equations):
 *   X~ = GroupLN1(X)                                   per-token statistics, per-group gamma/beta
 *   [Q|K|V|U] = X~ W_qkvu^T + b_qkvu                   four d-wide affine projections
 *   V~_h = (silu(Q_h K_h^T) / N  (.)  M) V_h           per head h; N = the user's token count;
 *                                                      M = three-rule dynamic mask ([P5] 7.3.4)
 *   X <- W2 silu(W1 GroupLN2(V~ (.) U) + b1) + b2 + X  residual MLP
 * and, after L blocks, CTR/CTCVR logits at candidate tokens ([P1]/[P2] token section; [P5] 7.3.1):
 *   logits = W_h2 silu(W_h1 x + b_h1) + b_h2.
 *
 * Batch format ([P3] 方法, equation for D; [P1]/[P2] sequence packing): users are packed back to
 * back; user b owns tokens offsets[b] .. offsets[b+1]-1, in group order U, S, R, C
 * (group id 0 = static user feature, 1 = long-term history, 2 = real-time event, 3 = candidate).
 * Tokens of different users never attend to each other.
 *
 * Mask ([P5] 7.3.4 Rules 1-3, [P3] 方法): key j is visible to query i of the same user iff
 * j is a U or S token, or j == i, or (j is an R token, i is an R or C token, t_j < t_i).
 * Timestamps are float32 seconds; U/S timestamps are never read.
 *
 * Conventions
 *   - Every buffer is owned by the caller.  "device" pointers are HIP device memory of the
 *     current device; "host" pointers are ordinary host memory read during the call only.
 *   - The library never allocates device memory: scratch space is a caller-provided workspace
 *     whose size the *_workspace_size functions report.  It keeps no state between calls.  The one
 *     exception is mtgr_attention_fwd_noalloc, whose scratch is a fixed array of the library.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and the call returns
 *     after enqueueing.  Faults inside kernels surface at the caller's next synchronisation.
 *   - Argument and shape errors are found on the host before anything is enqueued and are
 *     returned as a status; MTGR_ERR_HIP reports a failed launch (hipGetLastError).
 *   - Weights use the torch Linear layout [out][in], row-major.  Row block order in W_qkvu is
 *     Q, K, V, U; head h owns rows h*d_h .. (h+1)*d_h-1 of each block.
 *   - Storage dtype MTGR_BF16 means bf16 weights and bf16 intermediate activations with fp32
 *     accumulation; the residual stream x is always fp32.  MTGR_F32 keeps everything fp32.
 *   - Supported shapes: d % H == 0; d_h = d/H in {32, 64, 128} (bf16: {64, 128});
 *     d, h multiples of 64 and >= 128 (bf16) or multiples of 8 (fp32); d <= 1024; h <= 8192;
 *     head hidden a multiple of 32 (bf16) or 8 (fp32).
 */
#ifndef MTGR_H
#define MTGR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MTGR_ABI_VERSION 5

typedef enum {
  MTGR_OK = 0,
  MTGR_ERR_NULL_ARG = 1,     /* a required pointer is NULL */
  MTGR_ERR_BAD_SHAPE = 2,    /* d, H, h, M, N, K out of the supported set; also, in bf16, a user
                                whose QKVU rows span 2^31 bytes or more (8 d bytes per token) */
  MTGR_ERR_BAD_BATCH = 3,    /* offsets not monotone, T or C inconsistent, bad group order */
  MTGR_ERR_UNSUPPORTED = 4,  /* dtype / epilogue / option not implemented */
  MTGR_ERR_WORKSPACE = 5,    /* workspace NULL or smaller than the reported size */
  MTGR_ERR_HIP = 6,          /* a HIP launch or copy failed */
  MTGR_ERR_SCRATCH_LIMIT = 7 /* mtgr_attention_fwd_noalloc: the batch's prep tables exceed the
                                library's fixed scratch (4 MiB per device) */
} mtgr_status;

typedef enum { MTGR_F32 = 0, MTGR_BF16 = 1 } mtgr_dtype;

enum { MTGR_G_U = 0, MTGR_G_S = 1, MTGR_G_R = 2, MTGR_G_C = 3, MTGR_NUM_GROUPS = 4 };

/* Attention masks.  MTGR_MASK_DYNAMIC is the method's three-rule mask.  The other two are the
 * baselines of the ablation without the dynamic mask ([P1]/[P2] experiments; [P3] 结果):
 * MTGR_MASK_CAUSAL, key j visible to query i iff j <= i in the user's token order (the plain
 * causal mask the dynamic rules replace, [P3] 方法 and [P5] 7.3.4), and MTGR_MASK_FULL, every
 * key of the user visible. */
enum { MTGR_MASK_DYNAMIC = 0, MTGR_MASK_CAUSAL = 1, MTGR_MASK_FULL = 2 };

/* Normalisation.  MTGR_NORM_GROUP is GroupLN; MTGR_NORM_SHARED is the ablation without GroupLN
 * ([P1]/[P2] experiments; [P3] 方法, GLN paragraph): one LayerNorm whose gamma/beta are row 0
 * of the [4][d] parameter arrays, for every token. */
enum { MTGR_NORM_GROUP = 0, MTGR_NORM_SHARED = 1 };

/* GEMM epilogues of mtgr_linear_fwd */
enum {
  MTGR_EPI_STORE = 0,        /* out(dtype)  = a W^T + bias              */
  MTGR_EPI_SILU = 1,         /* out(dtype)  = silu(a W^T + bias)        */
  MTGR_EPI_RESIDUAL_F32 = 2  /* out(float)  = a W^T + bias + resid(float); out may alias resid */
};

/* Packed jagged batch.  All device arrays are read-only for the library. */
typedef struct mtgr_batch {
  int32_t num_users;              /* B >= 0 */
  int64_t num_tokens;             /* T == offsets[B] */
  int64_t num_candidates;         /* C == number of tokens with group id 3 */
  const int64_t* offsets_host;    /* host   [B+1], offsets_host[0] == 0, non-decreasing */
  const int64_t* offsets;         /* device [B+1], same values */
  const uint8_t* group_ids;       /* device [T], 0..3, non-decreasing within each user */
  const float* timestamps;        /* device [T], seconds; R and C entries must not be NaN */
} mtgr_batch;

/* One HSTU block.  All pointers are device pointers in `dtype`; biases may be NULL (= 0). */
typedef struct mtgr_block_params {
  int32_t d_model;                /* d */
  int32_t num_heads;              /* H */
  int32_t mlp_hidden;             /* h */
  int32_t dtype;                  /* mtgr_dtype */
  float ln_eps;                   /* GroupLN epsilon (1e-5 in the workloads) */
  const void* gln1_gamma;         /* [4][d] */
  const void* gln1_beta;          /* [4][d] */
  const void* w_qkvu;             /* [4d][d] */
  const void* b_qkvu;             /* [4d] or NULL */
  const void* gln2_gamma;         /* [4][d] */
  const void* gln2_beta;          /* [4][d] */
  const void* w_mlp1;             /* [h][d] */
  const void* b_mlp1;             /* [h] or NULL */
  const void* w_mlp2;             /* [d][h] */
  const void* b_mlp2;             /* [d] or NULL */
  int32_t mask_mode;              /* MTGR_MASK_*; 0 (a zeroed struct) = the dynamic mask */
  int32_t norm_mode;              /* MTGR_NORM_*; 0 = GroupLN */
} mtgr_block_params;

/* Parameter gradients of one block (mtgr_block_bwd): device float pointers shaped like the
 * parameters of mtgr_block_params (gamma/beta gradients always [4][d]; with MTGR_NORM_SHARED rows
 * 1..3 come out zero).  They are overwritten, not accumulated.  A NULL bias-gradient pointer skips
 * that gradient; every other pointer is required. */
typedef struct mtgr_block_grads {
  float* gln1_gamma;              /* [4][d] */
  float* gln1_beta;               /* [4][d] */
  float* w_qkvu;                  /* [4d][d] */
  float* b_qkvu;                  /* [4d] or NULL */
  float* gln2_gamma;              /* [4][d] */
  float* gln2_beta;               /* [4][d] */
  float* w_mlp1;                  /* [h][d] */
  float* b_mlp1;                  /* [h] or NULL */
  float* w_mlp2;                  /* [d][h] */
  float* b_mlp2;                  /* [d] or NULL */
} mtgr_block_grads;

/* L blocks plus the candidate head.  `layers` is a host array of L block descriptions that
 * must all share d, H, dtype. */
typedef struct mtgr_encoder_params {
  int32_t num_layers;             /* L >= 1 */
  const mtgr_block_params* layers;/* host [L] */
  int32_t head_hidden;            /* hh (d/2 in the workloads) */
  const void* w_head1;            /* device [hh][d]  */
  const void* b_head1;            /* device [hh] or NULL */
  const void* w_head2;            /* device [2][hh]  */
  const void* b_head2;            /* device [2] or NULL */
} mtgr_encoder_params;

/* ---- version and messages -------------------------------------------------------------- */
int32_t mtgr_abi_version(void);
const char* mtgr_status_str(int32_t status);

/* ---- workspace sizes (host only, no HIP call) ------------------------------------------- */
mtgr_status mtgr_encoder_workspace_size(const mtgr_encoder_params* p, const mtgr_batch* b,
                                        size_t* bytes);
mtgr_status mtgr_block_workspace_size(const mtgr_block_params* p, const mtgr_batch* b,
                                      size_t* bytes);
mtgr_status mtgr_attention_workspace_size(const mtgr_batch* b, int32_t d, int32_t num_heads,
                                          size_t* bytes);
mtgr_status mtgr_block_bwd_workspace_size(const mtgr_block_params* p, const mtgr_batch* b,
                                          size_t* bytes);
mtgr_status mtgr_attention_bwd_workspace_size(const mtgr_batch* b, int32_t d, int32_t num_heads,
                                              int32_t dtype, size_t* bytes);

/* ---- the hot path ----------------------------------------------------------------------- */
/* Full encoder: L blocks over x_in (device float [T][d]) then the head at candidate tokens.
 * hidden_out (device float [T][d], may be NULL) receives the final hidden states and may alias
 * x_in; logits (device float [C][2]) receive (CTR, CTCVR) logits in packed candidate order
 * (user-major, then token order within the user).  No sigmoid is applied.
 * Follows [P3] 方法 (the stack of HSTU blocks over the packed sample D) and [P1]/[P2] token
 * section with [P5] 7.3.1 (multi-task CTR/CTCVR scores read at the candidate tokens). */
mtgr_status mtgr_encoder_fwd(const mtgr_encoder_params* p, const mtgr_batch* b, const float* x_in,
                             float* hidden_out, float* logits, void* ws, size_t ws_bytes,
                             void* stream);

/* One block: x_out = block(x_in), both device float [T][d]; x_out may alias x_in.
 * The HSTU block of [P3] 方法, its two update equations (attention update, then the residual
 * MLP), with GroupLN before each ([P5] 7.3.3) and the mask of mask_mode ([P5] 7.3.4). */
mtgr_status mtgr_block_fwd(const mtgr_block_params* p, const mtgr_batch* b, const float* x_in,
                           float* x_out, void* ws, size_t ws_bytes, void* stream);

/* Backward pass of one block ([P3] 方法, the two update equations, differentiated by the chain
 * rule; the pages train the model end to end, [P1]/[P2] training-system section).  Given x_in
 * (device float [T][d], the block's input) and dx_out = dLoss/dx_out (device float [T][d]), writes
 * dx_in = dLoss/dx_in (device float [T][d]; may alias dx_out) and the parameter gradients summed
 * over every token of the batch into *g.  The forward activations are recomputed into the
 * workspace (mtgr_block_bwd_workspace_size); in MTGR_BF16 they and the activation gradients are
 * stored in bf16 with fp32 accumulation, the parameter gradients are fp32 sums of fp32 split
 * partials.  Every reduction has a fixed order: repeated calls give identical bits. */
mtgr_status mtgr_block_bwd(const mtgr_block_params* p, const mtgr_batch* b, const float* x_in,
                           const float* dx_out, float* dx_in, const mtgr_block_grads* g, void* ws,
                           size_t ws_bytes, void* stream);

/* ---- kernel-level entries (the same kernels the block uses) ------------------------------ */
/* GroupLN over T rows of width d: y = (x - mean) / sqrt(var + eps) * gamma[g] + beta[g].
 * x in `in_dtype`, y in `out_dtype`, gamma/beta [4][d] in `param_dtype` ([1][d] suffices with
 * MTGR_NORM_SHARED, which uses g = 0 for every row).
 * Supported (in, out): (F32, F32), (F32, BF16), (BF16, BF16).
 * The GLN equation of [P5] 7.3.3 (LayerNorm statistics per token, affine parameters per token
 * group; [P3] 方法, GLN paragraph); the variance is the biased one (1/d). */
mtgr_status mtgr_groupln_fwd(const mtgr_batch* b, int32_t d, int32_t in_dtype, int32_t out_dtype,
                             int32_t param_dtype, int32_t norm_mode, const void* gamma,
                             const void* beta, float eps, const void* x, void* y, void* stream);

/* out = epilogue(a[M][K] W[N][K]^T + bias[N]); a, W, bias in `dtype`; see MTGR_EPI_*.
 * bf16: K a multiple of 64 and >= 128, N a multiple of 8.  fp32: K a multiple of 4.
 * The affine maps of the block ([P3] 方法: the Q/K/V/U projection of the first update
 * equation, the two MLP layers with SiLU and the residual add of the second). */
mtgr_status mtgr_linear_fwd(int64_t M, int32_t N, int32_t K, int32_t dtype, int32_t epilogue,
                            const void* a, const void* w, const void* bias, const float* resid,
                            void* out, void* stream);

/* Masked SiLU attention with the U gate for every user and head, under mask `mask_mode`
 * (MTGR_MASK_*): qkvu device [T][4d] in `dtype` -> y_gated device [T][d] in `dtype` (V~ (.) U).
 * The normaliser is the user's token count N in every mode.
 * The V~ update equation of [P3] 方法 (silu(Q K^T) / N masked by M, times V, per head) with the
 * U gate of the second update, under the rules of [P5] 7.3.4; users never attend to each other
 * ([P1]/[P2] training-system section, sequence packing). */
mtgr_status mtgr_attention_fwd(const mtgr_batch* b, int32_t d, int32_t num_heads, int32_t dtype,
                               int32_t mask_mode, const void* qkvu, void* y_gated, void* ws,
                               size_t ws_bytes, void* stream);

/* mtgr_attention_fwd without a workspace, for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation).  The batch-prep tables
 * live in a fixed scratch array of 4 MiB that the library holds on every device it runs on until the
 * process ends: about 32 bytes per user plus 8 bytes per (user, head) group and 8 per XCD (e.g. up to
 * 26,000 users at 16 heads, 52,000 at 6).  A batch that needs more returns MTGR_ERR_SCRATCH_LIMIT before anything is
 * enqueued.  Every call on one device writes that device's scratch: calls that overlap on one GPU (two
 * streams, or two host threads) race and must be serialised by the caller.  Results equal
 * mtgr_attention_fwd's bit for bit.  No device or host heap memory is allocated. */
mtgr_status mtgr_attention_fwd_noalloc(const mtgr_batch* b, int32_t d, int32_t num_heads, int32_t dtype,
                                       int32_t mask_mode, const void* qkvu, void* y_gated, void* stream);

/* Backward of mtgr_attention_fwd: qkvu device [T][4d], v_tilde device [T][d] (the ungated
 * V~ = (silu(Q K^T) / N (.) M) V of the forward), dy_gated device [T][d] (dLoss/d(V~ (.) U)), all
 * in `dtype` -> dqkvu device [T][4d] in `dtype` (dQ, dK, dV, dU).  Every element of dqkvu is
 * written.  bf16 runs MFMA kernels (P and dS rounded to bf16 as MFMA operands, fp32 accumulation,
 * no atomics); fp32 runs one thread per (row, head).  The chain rule of the V~ update equation
 * ([P3] 方法) under the same mask rules as the forward. */
mtgr_status mtgr_attention_bwd(const mtgr_batch* b, int32_t d, int32_t num_heads, int32_t dtype,
                               int32_t mask_mode, const void* qkvu, const void* v_tilde,
                               const void* dy_gated, void* dqkvu, void* ws, size_t ws_bytes,
                               void* stream);

/* ---- hash embedding store ----------------------------------------------------------------- */
/* The pages' decoupled embedding table ([P3] 方法, training-framework paragraph; [P1]/[P2]
 * training-system section): a compact index from int64 key to a row of a separate value arena, so
 * keys are inserted and evicted in real time and the index can be rebuilt larger while the values
 * stay in place.  The caller owns both device buffers; the library keeps no state.  Keys are
 * >= 0 (negative keys are never stored; inserting one fails, looking one up misses).
 *   index_mem: mtgr_hash_index_bytes(index_cap) bytes, index_cap a power of two in [8, 2^40]
 *              (slots; keep the live count below ~3/4 of it for short probes)
 *   arena_mem: mtgr_hash_arena_bytes(rows, dim, dtype) bytes: free-row stack, last-use steps and
 *              the values [rows][dim] in dtype (dim * element size a multiple of 16 bytes)
 * Calls that modify the store must not overlap on the device (one stream, or ordered streams).
 * Within one call, a key occurring several times is handled once. */
typedef struct mtgr_hash_table {
  void* index_mem;
  int64_t index_cap;
  void* arena_mem;
  int32_t rows;
  int32_t dim;
  int32_t dtype;                  /* MTGR_F32 or MTGR_BF16 */
} mtgr_hash_table;

typedef struct mtgr_hash_stats {
  int64_t live;                   /* keys in the index */
  int64_t tombstones;             /* evicted slots not yet reclaimed by a rebuild */
  int64_t dropped;                /* entries the rebuild that produced this index could not place */
  int32_t free_rows;              /* arena rows on the free stack */
  int32_t failed_inserts;         /* insert occurrences since mtgr_hash_init that got no row */
} mtgr_hash_stats;

mtgr_status mtgr_hash_index_bytes(int64_t index_cap, size_t* bytes);
mtgr_status mtgr_hash_arena_bytes(int32_t rows, int32_t dim, int32_t dtype, size_t* bytes);
/* Empty index, every arena row free, counters zero. */
mtgr_status mtgr_hash_init(const mtgr_hash_table* t, void* stream);
mtgr_status mtgr_hash_insert_workspace_size(int64_t n, size_t* bytes);
/* Insert keys[n] (device int64).  A key already present keeps its row and value; a new key takes
 * a free row, initialised from init_values (device [n][dim] in dtype, row i for keys[i]; for a key
 * repeated in the call, one of its rows) or zeros when init_values is NULL.  Every occurrence's
 * row (or -1: arena full, index full, negative key) goes to rows_out (device int32 [n], may be
 * NULL); failures are counted per occurrence.  Rows of the keys touched record `step`. */
mtgr_status mtgr_hash_insert(const mtgr_hash_table* t, int64_t n, const int64_t* keys,
                             const void* init_values, int32_t step, int32_t* rows_out, void* ws,
                             size_t ws_bytes, void* stream);
/* Values of keys[n] into values_out (device [n][dim] in dtype, zeros for a missing key; may be
 * NULL) and their rows into rows_out (-1 missing; may be NULL).  step >= 0 records the use. */
mtgr_status mtgr_hash_lookup(const mtgr_hash_table* t, int64_t n, const int64_t* keys, int32_t step,
                             void* values_out, int32_t* rows_out, void* stream);
/* Remove keys[n] (missing keys are ignored); their rows return to the free stack. */
mtgr_status mtgr_hash_evict(const mtgr_hash_table* t, int64_t n, const int64_t* keys, void* stream);
/* Remove every key whose row was last used before step_threshold. */
mtgr_status mtgr_hash_evict_older(const mtgr_hash_table* t, int32_t step_threshold, void* stream);
/* Re-index the live keys of src into a fresh index at dst_index_mem (dst_index_cap slots, a
 * different buffer): no tombstones, same arena rows.  Use {dst_index_mem, dst_index_cap, same
 * arena} afterwards.  Keys that do not fit are dropped and counted (stats.dropped of dst). */
mtgr_status mtgr_hash_rebuild(const mtgr_hash_table* src, void* dst_index_mem, int64_t dst_index_cap,
                              void* stream);
/* Counters of the store.  Synchronises `stream`. */
mtgr_status mtgr_hash_get_stats(const mtgr_hash_table* t, mtgr_hash_stats* out, void* stream);

/* Batch key dedup ([P3] 方法: IDs are deduplicated before the embedding lookup): the distinct
 * values of keys[n] (device int64, >= 0) into unique_out[0 .. u-1] in an unspecified order, u into
 * *num_unique_out (device int64), and for every i the position of keys[i] in unique_out into
 * inverse_out[i] (device int64; -1 for a negative key).  The workspace holds a scratch index. */
mtgr_status mtgr_dedup_workspace_size(int64_t n, size_t* bytes);
mtgr_status mtgr_dedup(int64_t n, const int64_t* keys, int64_t* unique_out, int64_t* inverse_out,
                       int64_t* num_unique_out, void* ws, size_t ws_bytes, void* stream);

/* ---- tokenizer front end ----------------------------------------------------------------- */
/* Field IDs -> encoder input.  A token of group g (U, S, R, C = 0..3) has num_fields[g] fields;
 * field f reads table field_table[g][f] of the bf16 store at key (table << 40) | id (tables of one
 * width merged into one store, [P3] 方法, training-framework paragraph).  The token's input is
 *   x = W2_g silu(W1_g concat_f(emb_f) + b1_g) + b2_g
 * (a domain-specific MLP over the concatenated field embeddings, [P1]/[P2] "Converting
 * heterogeneous features into tokens"; the candidate token MLP(Concat(Emb(Item), Emb(Cross))),
 * [P5] 7.3.2).  The batch's keys are deduplicated and each distinct key is read from the store
 * once.  An id outside [0, 2^40) or a key absent from the store embeds to zeros.
 * W1_g: device bf16 [d][num_fields[g] * dim] (num_fields[g] * dim a multiple of 64, >= 128);
 * W2_g: device bf16 [d][d]; biases device bf16 [d] or NULL; d a multiple of 64 in [128, 4096]. */
#define MTGR_TOK_MAX_FIELDS 8
typedef struct mtgr_tokenizer_params {
  int32_t d_model;
  int32_t max_fields;                                  /* columns of field_ids, 1..8 */
  int32_t num_fields[4];                               /* 1..max_fields */
  int32_t field_table[4][MTGR_TOK_MAX_FIELDS];         /* 0 .. 2^23 - 1 */
  const void* w1[4];
  const void* b1[4];
  const void* w2[4];
  const void* b2[4];
} mtgr_tokenizer_params;

/* group_counts (host [4]): tokens of each group in the batch; must sum to num_tokens, with
 * group_counts[3] == num_candidates.  field_ids: device int64 [T][max_fields] (columns past a
 * token's num_fields are ignored).  store: dim = the embedding width, dtype MTGR_BF16.  step >= 0
 * records the use of every key read.  x_out: device float [T][d].  flags_out (device int32, may be
 * NULL) gets bit 0 set when the device's own group counts disagree with group_counts (such tokens
 * get x = 0; nothing is accessed out of range). */
mtgr_status mtgr_tokenize_workspace_size(const mtgr_tokenizer_params* p, const mtgr_batch* b,
                                         const mtgr_hash_table* store, const int64_t group_counts[4],
                                         size_t* bytes);
mtgr_status mtgr_tokenize(const mtgr_tokenizer_params* p, const mtgr_batch* b,
                          const int64_t group_counts[4], const int64_t* field_ids,
                          const mtgr_hash_table* store, int32_t step, float* x_out, int32_t* flags_out,
                          void* ws, size_t ws_bytes, void* stream);

/* ---- test / debug ------------------------------------------------------------------------ */
/* Device-side checks of a batch (group ids in 0..3 and non-decreasing within each user, no NaN
 * R/C timestamp, candidate count == num_candidates).  Synchronises `stream`.  *flags_out gets
 * a bit set per failed check (1 group range, 2 group order, 4 NaN time, 8 candidate count). */
mtgr_status mtgr_validate_batch(const mtgr_batch* b, void* ws, size_t ws_bytes, void* stream,
                                int32_t* flags_out);

/* Writes the mask `mask_mode` (MTGR_MASK_*) of user `user` as uint8 [n_b][n_b] (rows = queries)
 * into mask_dev, using the same visibility predicate as the attention kernels. */
mtgr_status mtgr_debug_mask(const mtgr_batch* b, int32_t user, int32_t mask_mode,
                            uint8_t* mask_dev, void* ws, size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MTGR_H */
