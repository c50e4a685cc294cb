/*
 * pkv.h -- C ABI of the MI355X (gfx950) paged-KV split-KV decode attention
 * library (libpkv.so).
 *
 * The operation (AstrAI commit d565d44, "csrc/kernels/attn_paged_decode.cu",
 * commit notes on the scalar and MMA split-KV paged decode kernels and their
 * bindings): for every sequence b, query token i < q_len and query head h,
 *
 *     out[b,i,h,:] = sum_j softmax_j(s_j) * V[b, j, g(h), :]
 *     s_j          = scale * <q[b,i,h,:], K[b, j, g(h), :]> + mask[b,(i,)j]
 *
 * over the keys j the row may see: j < kv_lens[b], and j <= c + i when a
 * causal offset c >= 0 applies ("unified causal_offset: -1 = off, >= 0 = first
 * Q position").  K and V live in fixed-size physical pages; logical key j of
 * sequence b is slot j % page_size of physical page block_table[b, j /
 * page_size].  GQA: query head h reads kv head g(h) = h / (Hq / Hkv).  A row
 * that sees no finite score gets 0.  The work is split along the keys
 * ("split-KV"); each split leaves a normalised partial output and its
 * (max, sum) pair, merged with the log-sum-exp rule; in pkv_paged_decode the
 * workgroup that finishes last among the splits of a (sequence, kv-head
 * group, row block) unit does that merge, so one kernel launch covers the
 * whole path.
 *
 * Conventions shared by every entry point:
 *  - All tensor pointers are caller-owned DEVICE memory of the current HIP
 *    device, read or written asynchronously on `stream`.  The library keeps
 *    no pointer after a call returns.
 *  - No entry point allocates, frees, copies, sets memory through the
 *    runtime or synchronises; the entry points taking a stream only launch
 *    kernels on it, so they may be captured into a hipGraph.  Kernel arguments depend only on
 *    host values, so device data (kv_lens, block_table, q, K/V, mask) may
 *    change between graph replays.
 *  - Every host-side check runs before any launch (the only other HIP calls
 *    are queries: the current device, its compute-unit count and, for
 *    pkv_paged_decode_noalloc, the address of its static workspace); a failed
 *    check returns its status with nothing enqueued.  There are no
 *    exceptions, aborts or prints.  The library is stateless apart from a
 *    per-device cache of the compute-unit count and the static workspace of
 *    pkv_paged_decode_noalloc, and is thread-safe.
 *  - Caller contract (not checkable without a device sync): block-table
 *    entries for the pages that hold keys j < kv_lens[b] are in
 *    [0, num_pages); 0 <= kv_lens[b] <= max_kv_len; causal_offsets[b] >= -1.
 *    Entries past ceil(kv_lens[b] / page_size) may hold any value: they may
 *    be read, but are never used to address memory.  Page slots at or past
 *    kv_lens[b] are never read.
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes (distinct per failure kind, in the spirit of the structured
 * unsupported-feature errors in the ejkernel v0.0.55 release notes and the
 * binding validation in the AstrAI commit notes). */
enum {
  PKV_OK = 0,
  PKV_ERR_NULL = 1,        /* a required pointer is NULL */
  PKV_ERR_SHAPE = 2,       /* bad dimension, Hq % Hkv != 0, Hkv % heads_per_block != 0, Hkv * D > 2^24, max_kv_len too big, bad stride */
  PKV_ERR_UNSUPPORTED = 3, /* head_dim not in {32,64,128,256}, page_size not a power of two in [1, 4096], splits > PKV_MAX_SPLITS, heads_per_block not in {0, 1, 2, 4, 8} (8: head_dim <= 64) */
  PKV_ERR_WORKSPACE = 4,   /* o_part / ml_part missing or smaller than pkv_workspace_bytes */
  PKV_ERR_ALIGN = 5,       /* a pointer is not aligned as documented */
  PKV_ERR_LAUNCH = 6,      /* the HIP runtime rejected a kernel launch */
  PKV_ERR_DEVICE = 7,      /* querying the current device failed */
  PKV_ERR_SCRATCH = 8      /* pkv_paged_decode_noalloc: the split workspace exceeds PKV_NOALLOC_SCRATCH_BYTES */
};

#define PKV_MAX_SPLITS 256

/* causal_offset value: the query tokens of each sequence are its last keys,
 * token i of a sequence with n query tokens sits at position kv_lens[b] - n + i
 * (the chunked-prefill / decode convention; requires kv_lens[b] >= n). */
#define PKV_CAUSAL_LAST (-2)

/* Head of the pkv_paged_decode ml_part workspace holding the per-unit arrival
 * counters of the in-kernel merge (one int32 per (sequence, kv-head group,
 * row block) unit, see pkv_plan), and the largest unit count merged
 * in-kernel; problems with more units and several splits use a separate
 * combine launch instead. */
#define PKV_COUNTER_BYTES 16384
#define PKV_MAX_FUSED_UNITS (PKV_COUNTER_BYTES / 4)

/* Problem description (host memory; read during the call only).
 * Sizes follow the statement of the paged decode problem: q[B, q_len, Hq, D],
 * k_cache / v_cache[num_pages, page_size, Hkv, D], block_table[B,
 * max_pages_per_seq], kv_lens[B]; the split count follows ejkernel's
 * PageAttentionConfig (operations.configs docs: num_splits, 0 = auto). */
typedef struct pkv_problem {
  int32_t batch;             /* B >= 0 (0: nothing to do) */
  int32_t q_len;             /* query tokens per sequence, >= 1 */
  int32_t num_q_heads;       /* Hq >= 1 */
  int32_t num_kv_heads;      /* Hkv >= 1, Hq % Hkv == 0 */
  int32_t head_dim;          /* D in {32, 64, 128, 256} */
  int32_t page_size;         /* power of two in [1, 4096] */
  int32_t num_pages;         /* physical pages in the pool, >= 0 */
  int32_t max_pages_per_seq; /* block_table row stride, >= 1 */
  int32_t max_kv_len;        /* host-known bound on kv_lens; 0 => max_pages_per_seq * page_size */
  float scale;               /* finite score scale, usually 1/sqrt(D) */
  int32_t causal_offset;     /* -1 off; >= 0 position of query token 0 (all sequences);
                                PKV_CAUSAL_LAST: each sequence's query tokens are its last keys */
  int32_t num_splits;        /* 0 heuristic; 1..PKV_MAX_SPLITS forced */
  int64_t mask_stride_b;     /* mask element stride between sequences (>= 0) */
  int64_t mask_stride_q;     /* mask element stride between query tokens; 0 => 2D [B, kv] mask */
  int32_t heads_per_block;   /* kv heads per split workgroup: 0 heuristic; 1, 2, 4 or 8 forced
                                (must divide num_kv_heads; 8 needs head_dim <= 64); a
                                launch-shape choice only, the results do not depend on it
                                beyond rounding order */
} pkv_problem;

/* Number of splits pkv_paged_decode uses for this problem on a device with
 * `num_cus` compute units (num_cus <= 0: the current device's count).  A
 * forced p->num_splits is returned unchanged.  Pure host arithmetic once the
 * CU count is known.  (The split-count heuristic of the AstrAI commit notes,
 * "compute_num_splits"; 0 = automatic as in ejkernel's PageAttentionConfig.) */
int pkv_num_splits(const pkv_problem *p, int num_cus, int *splits_out);

/* The launch plan pkv_paged_decode follows for this problem on a device with
 * `num_cus` compute units (num_cus <= 0: the current device's count).  Pure
 * host arithmetic once the CU count is known; forced num_splits and
 * heads_per_block are reported unchanged. */
typedef struct pkv_plan_info {
  int32_t splits;           /* key splits per sequence */
  int32_t heads_per_block;  /* kv heads per split workgroup (1, 2, 4 or 8) */
  int32_t rows_per_block;   /* packed query rows (G * q_len) per kv head per workgroup:
                               1 or 2 (vector kernel; 4 at head_dim 256 with 3 or 4
                               rows), 16 or 32 (matrix-core kernel),
                               128 (prefill-shaped matrix-core kernel: from 128 rows on at
                               D <= 128 with one kv head per workgroup, four waves of 32
                               rows sharing each K/V tile) */
  int32_t matrix_core;      /* 1: a matrix-core split kernel; 0: the vector one */
  int64_t units;            /* (sequence, kv-head group, row block) units */
  int64_t workgroups;       /* split-kernel workgroups: units * splits */
  int32_t merge_in_kernel;  /* 1: the split kernel merges the splits itself */
  int32_t kernels;          /* kernel launches per pkv_paged_decode call (0 when batch == 0) */
  int32_t kernel;           /* the split kernel: PKV_KERNEL_* below */
  int32_t paired_heads;     /* 1: head pairing.  At head_dim 32 (an even number of kv heads,
                               at most 8 packed rows per kv head, heads_per_block 0, paged
                               or [B, L, Hkv, D] K/V) kv heads 2g and 2g + 1, adjacent in
                               every key row, are read as one head of 64 columns, so each
                               load fetches whole 128-byte lines; a row's q fills its own
                               head's half (zero in the other) and its output is that half.
                               heads_per_block then counts kv heads (two per pair),
                               rows_per_block and units those of the paired launch (2 * G
                               query heads per pair).  Results stay within the same bounds;
                               their bits differ from an unpaired plan's.  Forced groupings
                               are never paired; pkv_contiguous_decode in the [B, Hkv, L, D]
                               layout (whose head slices are not adjacent) runs the same
                               split count unpaired, one kv head per workgroup, so the split
                               count and workspace of a problem never depend on its layout. */
} pkv_plan_info;

/* pkv_plan_info.kernel: the vector kernel (1 or 2 rows per kv head, up to 4
 * at head_dim 256); the
 * one-head matrix-core kernel (16 or 32 rows of one kv head per wave, each
 * wave its own key tiles); the shared-tile matrix-core kernel (a workgroup
 * of 4 or 8 kv heads whose waves share each K/V tile of the whole head group,
 * read as contiguous runs of the page slots, through LDS: 8 kv heads per
 * workgroup, or 4 from 3 rows per kv head on at head_dim <= 128); the
 * prefill-shaped matrix-core kernel (128 rows of one kv head). */
#define PKV_KERNEL_VECTOR 0
#define PKV_KERNEL_MATRIX 1
#define PKV_KERNEL_SHARED_TILE 2
#define PKV_KERNEL_PREFILL 3

int pkv_plan(const pkv_problem *p, int num_cus, pkv_plan_info *info);

/* Workspace pkv_paged_decode needs with `splits` splits (the caller-owned,
 * pre-allocated split partials of the AstrAI commit notes, which replace
 * cached static buffers so a decode step allocates nothing and can be
 * captured into a graph):
 *   o_part : fp32 [B, q_len, Hq, splits, D]      (normalised partial outputs)
 *   ml_part: PKV_COUNTER_BYTES of int32 arrival counters, then
 *            fp32 [B, q_len, Hq, splits, 2]      (m, l) per partial,
 * m = max scaled+masked score in natural-log units, l = sum exp(s - m).
 * Both are 0 when splits == 1 (the split kernel then writes `out` itself).
 * The counter head must read zero when a call starts: clear a new workspace
 * once (pkv_workspace_clear, or any zero fill, ordered before the first call
 * on the call's stream); every call returns the counters it used to zero
 * before its kernel ends, so a workspace stays ready across calls of any
 * shape.  Calls sharing one workspace must be ordered (one stream, or
 * synchronised streams).  A head that does not read zero is not detected: a
 * unit whose counter starts at k < n (n its splits with keys) merges before
 * its last k partials land and leaves k behind; a counter at n or more never
 * merges, leaving that unit's output unwritten.  For hipGraph capture, clear
 * the head before capturing, or capture pkv_workspace_clear ahead of the
 * call (a fill kernel, safe to replay). */
int pkv_workspace_bytes(const pkv_problem *p, int splits, size_t *o_part_bytes,
                        size_t *ml_part_bytes);

/* Zero `bytes` (a multiple of 4) of device memory at `ptr` (4-byte aligned)
 * -- the workspace preparation that the AstrAI commit notes' graph-capture
 * work does outside the captured step --
 * with a fill kernel on `stream` (not a runtime memset, so it may be
 * captured into a hipGraph).  Meant for a newly allocated ml_part workspace.
 * bytes == 0 is a no-op. */
int pkv_workspace_clear(void *ptr, size_t bytes, hipStream_t stream);

/* Paged decode attention: the whole split-KV path of the AstrAI commit notes
 * (the scalar and MMA split-KV paged decode kernels with GQA head packing,
 * the page table resolved per tile, the unified causal offset, 2D/3D
 * additive masks and the LSE combine of the split partials) in one call.
 *   q            bf16 [B, q_len, Hq, D], contiguous, 16-byte aligned
 *   k_cache      bf16 [num_pages, page_size, Hkv, D], contiguous, 16-byte aligned
 *   v_cache      bf16 [num_pages, page_size, Hkv, D], contiguous, 16-byte aligned
 *   block_table  int32 [B, max_pages_per_seq]
 *   kv_lens      int32 [B]
 *   causal_offsets  NULL, or int32 [B]: per-sequence causal offset that
 *                replaces p->causal_offset (-1 turns causality off for b)
 *   mask         NULL, or fp32 additive mask; element (b, i, j) at
 *                mask[b * mask_stride_b + i * mask_stride_q + j]; -inf removes
 *                a key; entries at j >= kv_lens[b] are never read
 *   o_part, ml_part  workspace of at least pkv_workspace_bytes for the split
 *                count in use (16- and 8-byte aligned, ml_part's counter
 *                head zero as described there); may be NULL when that count
 *                is 1.  Contents on return: the counter head zero, the split
 *                partials of the splits that saw at least one key (l > 0;
 *                an empty split writes only (m, l) = (-inf, 0)).
 *   out_bf16     bf16 [B, q_len, Hq, D], 16-byte aligned; round-to-nearest-even
 *                of the fp32 result
 *   out_f32      NULL, or fp32 [B, q_len, Hq, D] (the value before rounding)
 * Returns PKV_OK after enqueueing one kernel on `stream` (two, the split
 * kernel and the combine kernel, when several splits are used and the
 * problem has more than PKV_MAX_FUSED_UNITS units). */
int pkv_paged_decode(const pkv_problem *p, const void *q, const void *k_cache,
                     const void *v_cache, const int32_t *block_table,
                     const int32_t *kv_lens, const int32_t *causal_offsets,
                     const float *mask, float *o_part, size_t o_part_bytes,
                     float *ml_part, size_t ml_part_bytes, void *out_bf16,
                     float *out_f32, hipStream_t stream);

/* Size of the static split workspace of pkv_paged_decode_noalloc: one array
 * of this many bytes per GPU the library runs on, held until the process
 * ends. */
#define PKV_NOALLOC_SCRATCH_BYTES (64u << 20)

/* pkv_paged_decode without a workspace argument, for callers that cannot
 * allocate device memory: code under hipGraph capture, tight serving loops,
 * harnesses that forbid allocation.  The split partials and merge counters
 * live in a static device array of PKV_NOALLOC_SCRATCH_BYTES bytes per GPU
 * (its address looked up once per device, on the first call with that device
 * current); the call allocates nothing, and the caller passes only inputs and
 * outputs.  The plan, kernels and results are those of pkv_paged_decode on
 * the same problem, bit for bit.
 *  - Size limit: with S > 1 splits (pkv_plan), pkv_workspace_bytes(p, S)'s
 *    ml_part bytes rounded up to 256 plus its o_part bytes must not exceed
 *    PKV_NOALLOC_SCRATCH_BYTES, else PKV_ERR_SCRATCH with nothing enqueued
 *    (one split needs no workspace and has no limit).
 *  - Shared state: every call on one GPU uses that GPU's one array, which
 *    keeps the last call's contents.  The first call on a device clears the
 *    merge counters with a fill kernel on its stream; every call leaves them
 *    zero.  Calls that overlap on one GPU (unordered streams, threads) race
 *    on the array and give undefined results: order them.
 * Arguments and other statuses as for pkv_paged_decode. */
int pkv_paged_decode_noalloc(const pkv_problem *p, const void *q, const void *k_cache,
                             const void *v_cache, const int32_t *block_table,
                             const int32_t *kv_lens, const int32_t *causal_offsets,
                             const float *mask, void *out_bf16, float *out_f32,
                             hipStream_t stream);

/* The launch plan of pkv_paged_decode_varlen for a batch of total_tokens
 * query tokens (0 .. B * q_len, else PKV_ERR_SHAPE): as pkv_plan, with the
 * split count and heads per workgroup sized for the rows the tokens fill
 * rather than for q_len tokens in every sequence.  The workspace of a call is
 * pkv_workspace_bytes(p, info->splits). */
int pkv_plan_varlen(const pkv_problem *p, int64_t total_tokens, int num_cus, pkv_plan_info *info);

/* Decode over a batch whose sequences have different numbers of query
 * tokens ("varlen": chunked prefill and single-token decode in one call, as
 * in the AstrAI paged-decode commit notes on prefill and decode kernels over
 * the same paged cache).  Sequence b has n_b = cu_q_lens[b+1] - cu_q_lens[b]
 * query tokens, 0 <= n_b <= p->q_len (the bound the launch is sized for).
 *   cu_q_lens    device int32 [B + 1], cu_q_lens[0] = 0, non-decreasing,
 *                cu_q_lens[B] = total_tokens (4-byte aligned)
 *   total_tokens 0 .. B * q_len (else PKV_ERR_SHAPE); host copy of cu_q_lens[B]
 *   q, out_bf16, out_f32   [total_tokens, Hq, D], token t of sequence b at
 *                cu_q_lens[b] + t
 *   mask         element (b, t, j) at mask[b * mask_stride_b + t * mask_stride_q + j]
 *   causal       p->causal_offset PKV_CAUSAL_LAST (the usual choice), -1, a
 *                position >= 0, or causal_offsets[B] as for pkv_paged_decode
 * The workspace is the one pkv_workspace_bytes gives for p (B * q_len * Hq
 * rows bound the token rows); other arguments and statuses as for
 * pkv_paged_decode.  The offsets in cu_q_lens are device data the host cannot
 * check: the kernels clamp each sequence's count to 0 .. q_len but trust the
 * offsets to stay within total_tokens.  With every count equal to q_len the
 * results are bit for bit those of pkv_paged_decode on the same problem. */
int pkv_paged_decode_varlen(const pkv_problem *p, const int32_t *cu_q_lens, int64_t total_tokens,
                            const void *q, const void *k_cache, const void *v_cache,
                            const int32_t *block_table, const int32_t *kv_lens,
                            const int32_t *causal_offsets, const float *mask, float *o_part,
                            size_t o_part_bytes, float *ml_part, size_t ml_part_bytes,
                            void *out_bf16, float *out_f32, hipStream_t stream);

/* K/V layouts of pkv_contiguous_decode, and the largest key capacity per
 * sequence it takes. */
#define PKV_KV_BLHD 1                    /* k_cache, v_cache bf16 [B, kv_capacity, Hkv, D] */
#define PKV_KV_BHLD 2                    /* k_cache, v_cache bf16 [B, Hkv, kv_capacity, D] */
#define PKV_MAX_CONTIGUOUS_KEYS (1 << 30)

/* Decode attention over contiguous (non-paged) K/V: the same operation and
 * kernels as pkv_paged_decode, with key j of sequence b at row j of sequence
 * b's own region of the cache instead of a page-table lookup (AstrAI
 * paged-decode commit notes: one set of decode kernels over a contiguous and
 * a paged K/V addressing policy, and stride-based addressing with a
 * "bhld"/"blhd" layout switch).
 *   kv_layout    PKV_KV_BLHD or PKV_KV_BHLD (else PKV_ERR_UNSUPPORTED)
 *   kv_capacity  keys per sequence in the cache, 1 .. PKV_MAX_CONTIGUOUS_KEYS
 *                (else PKV_ERR_SHAPE); p->max_kv_len <= kv_capacity (0 means
 *                kv_capacity)
 *   k_cache, v_cache  bf16 in the chosen layout, contiguous, 16-byte aligned;
 *                rows at or past kv_lens[b] are never read
 * p->page_size, p->num_pages and p->max_pages_per_seq are ignored; every other
 * field, argument, the workspace (pkv_workspace_bytes, pkv_plan with
 * p->max_kv_len set) and the status codes are as for pkv_paged_decode. */
int pkv_contiguous_decode(const pkv_problem *p, int kv_layout, int64_t kv_capacity,
                          const void *q, const void *k_cache, const void *v_cache,
                          const int32_t *kv_lens, const int32_t *causal_offsets,
                          const float *mask, float *o_part, size_t o_part_bytes,
                          float *ml_part, size_t ml_part_bytes, void *out_bf16,
                          float *out_f32, hipStream_t stream);

/* The split step alone (the split-KV kernels of the AstrAI commit notes,
 * without their combine): the same split kernel as pkv_paged_decode, always
 * writing the split partials and never launching the combine.  For callers
 * that merge partials themselves, e.g. after gathering the partials of key
 * shards held by several devices, with pkv_combine.  o_part (fp32 [B, q_len,
 * Hq, splits, D], 16-byte aligned) and ml_part (fp32 [B, q_len, Hq, splits,
 * 2], 8-byte aligned, no counter head) are required for every split count,
 * including 1: rows * splits * D * 4 and rows * splits * 8 bytes.  Splits
 * that see no key write only (m, l) = (-inf, 0) and leave their o_part rows
 * untouched.  Other arguments as for pkv_paged_decode. */
int pkv_paged_decode_partials(const pkv_problem *p, const void *q,
                              const void *k_cache, const void *v_cache,
                              const int32_t *block_table,
                              const int32_t *kv_lens,
                              const int32_t *causal_offsets, const float *mask,
                              float *o_part, size_t o_part_bytes,
                              float *ml_part, size_t ml_part_bytes,
                              hipStream_t stream);

/* The combine step alone (the single combine kernel of the AstrAI commit
 * notes, merging split partials by their log-sum-exp): merges `splits`
 * partials per row with the
 * log-sum-exp rule  M = max_{l_s>0} m_s,  w_s = l_s exp(m_s - M),
 * out = sum_s w_s o_s / sum_s w_s  (0 when no partial has l_s > 0); the
 * o_part rows of partials with l_s = 0 are never read; a row with exactly one
 * partial of l_s > 0 gets that o_s unchanged.
 *   o_part   fp32 [rows, splits, head_dim]   (16-byte aligned)
 *   ml_part  fp32 [rows, splits, 2]          (m, l), 8-byte aligned
 *   out_bf16 bf16 [rows, head_dim] (16-byte aligned), out_f32 NULL or fp32 [rows, head_dim]
 * head_dim in {32, 64, 128, 256}; 1 <= splits <= PKV_MAX_SPLITS; rows >= 0. */
int pkv_combine(int64_t rows, int splits, int head_dim, const float *o_part,
                const float *ml_part, void *out_bf16, float *out_f32,
                hipStream_t stream);

/* Compute units of the current device (queried once per device, then cached). */
int pkv_device_cus(int *num_cus);

/* Static text for a status code. */
const char *pkv_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */
