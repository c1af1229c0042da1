/*
 * attn.h -- C ABI of the gfx950 (MI355X) tiled attention forward library (libattn.so).
 *
 * The library computes scaled-dot-product attention O = softmax(tau * Q K^T) V,
 * tau = 1/sqrt(d) by default, with the streaming (online) softmax: a running row
 * maximum m, a running denominator l and an un-normalised output o are carried
 * across 64-key tiles, each tile rescales the old state by alpha = e^(m_old - m_new),
 * and O = o / l at the end, so the S_q x S_k score matrix is never stored
 * (page "gfx942 unified attention, from the math up", sections 1-3).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Pointers named q, k, v, o, lse, block_table, seqlens_k, partial_*, workspace
 *    are DEVICE pointers owned by the caller (for instance torch tensors). The
 *    library allocates no memory and keeps no pointer after a call returns.
 *  - 16-bit tensors (fp16 / bf16) must be 16-byte aligned and contiguous in the
 *    stated layout; the head dimension d is the innermost, contiguous axis.
 *  - `stream` is a hipStream_t (NULL = the default stream). Work is enqueued
 *    asynchronously on it; nothing synchronises inside the library.
 *  - Every call returns an attn_status_t; no C++ exception crosses the ABI.
 *    Arguments are validated on the host before any HIP call, so invalid
 *    arguments are reported even on a machine without a GPU. A non-OK status
 *    leaves a message readable with attn_last_error() (thread-local).
 *  - Values stored in the device buffers are not validated (that would need a
 *    synchronising copy): the 64 keys of a page whose id is outside
 *    [0, num_blocks) are left out of the softmax, and key lengths are clamped to
 *    their stated host-side bounds, so a bad table gives wrong numbers, never an
 *    out-of-bounds access.
 *  - Outputs in fp16 / bf16 are rounded to nearest, ties to even, unless the call's
 *    o_round field selects another mode for a bf16 output (attn_round_t).
 */
#ifndef ATTN_H
#define ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ATTN_ABI_VERSION 5
#define ATTN_PAGE_SIZE 64      /* tokens per KV page (block_size); equal to the KV tile width */
#define ATTN_MAX_SPLITS 64     /* upper bound of num_splits for the split-KV decode */
#define ATTN_MAX_SEQLEN (1 << 30)  /* upper bound of seqlen_q, seqlen_k and max_seqlen_k */
#define ATTN_NOALLOC_SCRATCH_BYTES (32u << 20)  /* scratch of attn_decode_fwd_noalloc: 32 MiB */

typedef enum {
  ATTN_OK = 0,
  ATTN_ERR_INVALID_ARG = 1,   /* an argument is out of its documented domain */
  ATTN_ERR_UNSUPPORTED = 2,   /* a valid combination the library does not implement */
  ATTN_ERR_LAUNCH = 3,        /* the HIP runtime refused the launch */
  ATTN_ERR_NO_DEVICE = 4      /* no usable HIP device */
} attn_status_t;

typedef enum { ATTN_F16 = 0, ATTN_BF16 = 1, ATTN_F32 = 2 } attn_dtype_t;

/* Rounding of the fp32 result to a bf16 output (page 7minutos.es / MoonMath, section
 * "Punto de referencia", which measures all three): RTNE = to nearest, ties to even;
 * RTNA = to nearest, ties away from zero; RTZ = toward zero (truncation). NaN stays
 * NaN in every mode. fp16 outputs support RTNE only (ATTN_ERR_UNSUPPORTED otherwise);
 * fp32 outputs are not rounded and accept any value of the field. */
typedef enum { ATTN_ROUND_RTNE = 0, ATTN_ROUND_RTNA = 1, ATTN_ROUND_RTZ = 2 } attn_round_t;

/* BSHD = [batch, seq, heads, d]; BHSD = [batch, heads, seq, d]. Both are accepted
 * as-is, without a transposition (page 7minutos.es / MoonMath, section
 * "Entendiendo el nucleo"). */
typedef enum { ATTN_BSHD = 0, ATTN_BHSD = 1 } attn_layout_t;

/*
 * Prefill (S_q >= 1 queries per sequence).
 *
 * Operation: for every sequence b, query head h and query row i (0 <= i < S_q),
 *   O[b,h,i] = sum_j a_j V_b[j],  a_j = exp(s_j - m) / sum_j' exp(s_j' - m),
 *   s_j = scale * <Q[b,h,i], K_b[j]>, m = max of the visible s_j,
 * over the visible keys j (page "gfx942 unified attention, from the math up",
 * sections 1-2). Key j is visible iff j < L_b and, when causal, j <= i + (L_b - S_q):
 * the causal mask is aligned to the bottom-right corner (same page, section 4),
 * and key tiles entirely in a query tile's future are skipped. Query head h reads
 * KV head floor(h / G), G = num_heads_q / num_heads_kv (GQA; same page, section 5).
 * A row with no visible key gets O = 0 and lse = -inf. Q and the visible K/V rows must
 * be finite (NaN or infinity there gives unspecified values, not necessarily NaN); key
 * rows that are not visible, such as the unused tail of a sequence's last page, may
 * hold anything and are never read into the arithmetic.
 *
 * Fields:
 *  q        [B, S_q, Hq, d] (BSHD) or [B, Hq, S_q, d] (BHSD), qkv_dtype.
 *  k, v     paged (block_table != NULL): caches [num_blocks, 64, Hkv, d]; logical
 *           key j of sequence b is row j % 64 of page block_table[b*max_blocks_per_seq
 *           + j / 64] (same page, section 5).
 *           dense (block_table == NULL): [B, S_k, Hkv, d] (BSHD) or [B, Hkv, S_k, d]
 *           (BHSD), S_k = seqlen_k, same layout as q.
 *  o        output, layout of q, o_dtype (F16, BF16 or F32).
 *  lse      optional (NULL to skip) fp32 [B, Hq, S_q]: natural-log log-sum-exp of the
 *           scaled visible scores of each row.
 *  block_table  int32 [B, max_blocks_per_seq], or NULL for dense K/V.
 *  seqlens_k    int32 [B] per-sequence key lengths L_b (clamped to seqlen_k), or NULL
 *           for L_b = seqlen_k. Required when block_table != NULL.
 *  seqlen_k upper bound of the key lengths (dense: the K/V row count).
 *  head_dim d in {64, 128, 256}. num_heads_q % num_heads_kv == 0, and
 *           num_heads_q / num_heads_kv <= 128.
 *  causal   0 or 1. precise: 0 or 1; 1 keeps the probabilities P at ~fp32 precision
 *           in the P.V product (two fp16/bf16 MFMA terms, hi + lo), for an fp32 O.
 *  scale    softmax scale; 0 selects 1/sqrt(d).
 *  o_round  attn_round_t for a bf16 output.
 *
 * Packed queries (cu_seqlens_q != NULL, BSHD only): sequences of different query
 * counts share one buffer. q and o are [total_q, Hq, d]; int32 cu_seqlens_q [B + 1]
 * (device) holds the first row of every sequence, cu_seqlens_q[B] = total_q, so
 * sequence b has S_q,b = cu_seqlens_q[b + 1] - cu_seqlens_q[b] queries (clamped to
 * [0, seqlen_q]; seqlen_q is then the host-side maximum). The operation above holds
 * per sequence with S_q,b in place of S_q, including the bottom-right causal offset
 * L_b - S_q,b (a batch of chunked-prefill steps of different lengths). lse, when
 * given, is fp32 [Hq, total_q]. The caller sizes q, o and lse for total_q; the
 * library reads cu_seqlens_q only on the device.
 * Tail split (the key-split of the last round of work, merged with a log-sum-exp
 * combine: page "gfx942 unified attention, from the math up", section 8, and the
 * 7minutos.es article on MoonMath AI's HIP attention kernel, paragraph "Punto de
 * referencia"). The launch cuts the query rows into work items (256 or 128 rows of one
 * sequence and KV head); when the last round of items on the device's CUs would leave
 * CUs idle, the library can give the key tiles of each of those last items to several
 * workgroups, which write fp32 partial outputs into the workspace, and merge the
 * partials afterwards exactly as attn_splitkv_combine does. This is done for
 * non-causal launches with precise = 0 (the items of such a launch all have the same
 * key range), and for causal launches with precise = 0 whose items are so few that at
 * most half of the CUs would have one: then every item is split (chunked prefill of a
 * few short chunks against long keys). A split row's O is the same attention up to fp32 rounding
 * and the fp16/bf16 rounding of P against a different running maximum: within the
 * tolerances of the unsplit result, not bit-identical to it.
 *  kv_splits  0: the library splits when the items of the last round would leave at
 *             least half of the CUs idle and the items have at least 2048 keys (3072
 *             for the causal case; up to 16 parts); 1: never split;
 *             2..ATTN_MAX_SPLITS: split into that many parts whenever the launch
 *             qualifies (non-causal: the last round is not full, and every item is in
 *             it when the launch has fewer items than one round; causal: few items as
 *             above).
 *  workspace, workspace_bytes  device scratch for the partials, 256-byte aligned, at
 *             least attn_prefill_workspace_bytes(args) bytes; caller-owned and only
 *             used in stream order by this call, so calls that may overlap need
 *             separate workspaces. NULL (with workspace_bytes 0) turns the tail split
 *             off when kv_splits = 0.
 * Errors: INVALID_ARG for null required pointers, misalignment, non-positive
 * sizes (B or S_q of 0 is a no-op returning OK), d not in {64,128,256}, a head
 * count that is not a multiple, a paged cache whose table cannot hold seqlen_k
 * keys (64*max_blocks_per_seq < seqlen_k), bad enum values, packed queries with the
 * BHSD layout or a misaligned cu_seqlens_q, kv_splits outside [0, ATTN_MAX_SPLITS],
 * seqlen_q or seqlen_k above ATTN_MAX_SEQLEN (UNSUPPORTED: positions are 32-bit in the
 * kernels),
 * a split (kv_splits >= 2) without a workspace, or a workspace that is misaligned or
 * smaller than attn_prefill_workspace_bytes(args).
 */
typedef struct {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  const int32_t* block_table;
  const int32_t* seqlens_k;
  const int32_t* cu_seqlens_q; /* NULL, or packed queries: see "Packed queries" */
  int32_t batch;
  int32_t num_heads_q;
  int32_t num_heads_kv;
  int32_t seqlen_q;
  int32_t seqlen_k;
  int32_t head_dim;
  int32_t num_blocks;          /* paged: pages in the cache */
  int32_t max_blocks_per_seq;  /* paged: columns of block_table */
  int32_t qkv_dtype;           /* attn_dtype_t: F16 or BF16 */
  int32_t o_dtype;             /* attn_dtype_t: F16, BF16 or F32 */
  int32_t layout;              /* attn_layout_t */
  int32_t causal;
  int32_t precise;
  float scale;
  int32_t o_round;             /* attn_round_t for a bf16 output (0 = RTNE) */
  int32_t kv_splits;           /* tail split: 0 = library's choice, 1 = never, n = n parts */
  void* workspace;             /* tail split partials, or NULL */
  size_t workspace_bytes;
} attn_prefill_args_t;

attn_status_t attn_prefill_fwd(const attn_prefill_args_t* args, void* stream);

/* Bytes of workspace the call attn_prefill_fwd(args) uses for its tail split on the
 * current device (0 when it does not split, including for arguments it would reject;
 * the pointer fields of args are not read). Layout, each part 256-byte aligned: fp32
 * partial outputs [rows, parts, d], fp32 partial lse [rows, parts], int64 output
 * offsets [rows], int64 lse indices [rows], rows = tail items x rows per item. */
size_t attn_prefill_workspace_bytes(const attn_prefill_args_t* args);

/*
 * Split-KV decode (one query per sequence), split kernel + log-sum-exp combine.
 *
 * Operation: the attention of attn_prefill_fwd at S_q = 1, non-causal (one query
 * attends to every key; identical to the bottom-right causal mask at S_q = 1:
 * page "gfx942 unified attention, from the math up", sections 4 and 8). The keys
 * of each (sequence, KV head) are split into at most num_splits partitions of whole
 * 64-key pages; each partition yields a partial (O_s normalised, lse_s) for the G
 * query heads of the group in the workspace, and the combine merges them (see
 * attn_splitkv_combine). The result does not depend on the partition plan beyond
 * rounding. With num_splits >= 2 the library chooses the partitions: a small plan
 * kernel divides every KV head's pages into equal ranges, one per workgroup (about
 * one workgroup per compute unit in total), and a range boundary inside a sequence
 * starts a new partition. With num_splits = 1 each sequence is one partition. All
 * kernels run on `stream` in order.
 *
 * Fields:
 *  q          [B, Hq, d] (the BSHD and BHSD layouts coincide at S_q = 1), qkv_dtype.
 *  k_cache, v_cache  [num_blocks, 64, Hkv, d], qkv_dtype.
 *  block_table int32 [B, max_blocks_per_seq]; seqlens_k int32 [B] (clamped to
 *             max_seqlen_k, which must be <= 64*max_blocks_per_seq and
 *             <= ATTN_MAX_SEQLEN).
 *  o          [B, Hq, d], o_dtype. lse: optional fp32 [B, Hq].
 *  workspace  device buffer of at least attn_decode_workspace_bytes(B, Hq,
 *             num_splits, d) bytes, 256-byte aligned; caller-owned scratch, reused
 *             freely between calls on the same stream.
 *  num_splits 1..ATTN_MAX_SPLITS. num_heads_q / num_heads_kv <= 16.
 * Errors: as for prefill (max_seqlen_k above ATTN_MAX_SEQLEN: UNSUPPORTED), plus
 * INVALID_ARG for a too-small or misaligned workspace.
 */
typedef struct {
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_table;
  const int32_t* seqlens_k;
  void* o;
  float* lse;
  void* workspace;
  size_t workspace_bytes;
  int32_t batch;
  int32_t num_heads_q;
  int32_t num_heads_kv;
  int32_t head_dim;
  int32_t num_blocks;
  int32_t max_blocks_per_seq;
  int32_t max_seqlen_k;
  int32_t num_splits;
  int32_t qkv_dtype;
  int32_t o_dtype;
  float scale;
  int32_t o_round;             /* attn_round_t for a bf16 output (0 = RTNE) */
} attn_decode_args_t;

attn_status_t attn_decode_fwd(const attn_decode_args_t* args, void* stream);

/*
 * Split-KV decode for callers that cannot allocate device memory: code under HIP graph
 * capture, serving loops and harnesses that forbid hipMalloc. Same operation, fields
 * and kernels as attn_decode_fwd, except that args->workspace must be NULL and
 * args->workspace_bytes 0: the split partials and the partition plan go to a static
 * device buffer of ATTN_NOALLOC_SCRATCH_BYTES that the library holds on every device it
 * runs on until the process ends. The call allocates and frees nothing; the caller
 * passes the inputs and the output (and lse) as for attn_decode_fwd.
 * Every call on one device shares that device's buffer, which keeps the last call's
 * contents (nothing in it has to start at zero: each call writes every word it reads).
 * Calls that overlap in time on one device (on different streams, or from host threads
 * not ordered with each other) race on the buffer and give wrong results; calls ordered
 * on one stream are safe.
 * Errors: as attn_decode_fwd, plus INVALID_ARG when a workspace is passed or when
 * attn_decode_workspace_bytes(B, Hq, num_splits, d) exceeds ATTN_NOALLOC_SCRATCH_BYTES
 * (for instance B * Hq * num_splits * d above about 8.3 million at d = 128).
 */
attn_status_t attn_decode_fwd_noalloc(const attn_decode_args_t* args, void* stream);

/* Bytes of decode workspace: fp32 partial outputs [B, Hq, num_splits, d], then (at
 * 256-byte aligned offsets) fp32 partial lse [B, Hq, num_splits] and the partition
 * plan (int32, about 4*(B + 1) + 4 KiB). Slots of unused partitions hold lse = -inf
 * and an undefined O_s. Returns 0 for invalid sizes. */
size_t attn_decode_workspace_bytes(int32_t batch, int32_t num_heads_q, int32_t num_splits,
                                   int32_t head_dim);

/*
 * Log-sum-exp combine of split partial results (page "gfx942 unified attention,
 * from the math up", section 8: partial softmax-weighted outputs of the KV splits
 * are combined). For each (b, h):
 *   M = max_s lse_s,  w_s = exp(lse_s - M),  O = sum_s w_s O_s / sum_s w_s,
 *   lse = M + ln(sum_s w_s).
 * A split with lse_s = -inf (no key) has weight 0 and its O_s is not read; if every
 * split is empty, O = 0 and lse = -inf.
 *
 * Fields: partial_o fp32 [B, H, num_splits, d] (each O_s already normalised);
 * partial_lse fp32 [B, H, num_splits] (natural log); o [B, H, d] in o_dtype;
 * lse optional fp32 [B, H]; num_splits 1..ATTN_MAX_SPLITS; d in {64, 128, 256}.
 * Errors: INVALID_ARG for null pointers, sizes or dtype out of range.
 */
typedef struct {
  const float* partial_o;
  const float* partial_lse;
  void* o;
  float* lse;
  int32_t batch;
  int32_t num_heads;
  int32_t num_splits;
  int32_t head_dim;
  int32_t o_dtype;
  int32_t o_round;             /* attn_round_t for a bf16 output (0 = RTNE) */
} attn_combine_args_t;

attn_status_t attn_splitkv_combine(const attn_combine_args_t* args, void* stream);

/* Message of the last non-OK status on this thread ("" if none). */
const char* attn_last_error(void);

/* ATTN_ABI_VERSION of the loaded library. */
int32_t attn_abi_version(void);

/* Number of visible HIP devices (0 when none or when the runtime is unavailable). */
int32_t attn_device_count(void);

/* Facts of one HIP device, read from hipDeviceProp_t and the runtime, so that measured
 * throughput can be stated against peaks derived from the device itself (matrix-core
 * peak = compute units x engine clock x flops per clock and CU). Strings are
 * NUL-terminated and truncated to their buffers. */
typedef struct {
  char name[256];              /* marketing name */
  char arch[256];              /* gcnArchName, e.g. "gfx950:sramecc+:xnack-" */
  int64_t total_memory;        /* bytes of device memory */
  int32_t compute_units;       /* multiProcessorCount */
  int32_t clock_khz;           /* clockRate: peak engine clock */
  int32_t memory_clock_khz;    /* memoryClockRate */
  int32_t memory_bus_bits;     /* memoryBusWidth */
  int32_t lds_per_cu;          /* maxSharedMemoryPerMultiProcessor, bytes */
  int32_t l2_bytes;            /* l2CacheSize */
  int32_t runtime_version;     /* hipRuntimeGetVersion */
  int32_t driver_version;      /* hipDriverGetVersion */
} attn_device_info_t;

/* Fill *info for HIP device `device`. Errors: INVALID_ARG for a NULL info or a device
 * index outside [0, attn_device_count()), NO_DEVICE when no device is visible, LAUNCH
 * when the runtime refuses the query. */
attn_status_t attn_device_info(int32_t device, attn_device_info_t* info);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_H */
