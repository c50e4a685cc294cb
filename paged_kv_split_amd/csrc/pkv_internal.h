// pkv_internal.h -- launch plan shared by the host entry points and the HIP
// kernels of libpkv.so (not part of the public ABI).
#pragma once

#include <stdint.h>
#include <hip/hip_runtime_api.h>

namespace pkv {

// Everything a split-decode launch needs, fixed on the host from host values
// only (so a captured graph stays valid when device data changes).
struct DecodeArgs {
  const uint16_t *q;
  const uint16_t *k;
  const uint16_t *v;
  const int32_t *block_table;
  const int32_t *kv_lens;
  const int32_t *causal_offsets;  // nullable
  const int32_t *cu_q;            // nullable: [B + 1] token starts of a varlen batch (q, out packed by token)
  const float *mask;              // nullable
  float *o_part;                  // [rows, S, D]   (S > 1)
  float *ml_part;                 // [rows, S, 2]   (S > 1)
  uint16_t *out;                  // bf16 [rows, D] (S == 1)
  float *out_f32;                 // nullable       (S == 1)
  int64_t mask_sb, mask_sq;
  int64_t page_stride;            // elements per physical page: P * Hkv * D (contiguous K/V: one sequence)
  int64_t head_stride;            // elements between kv heads: D (paged, blhd) or capacity * D (bhld)
  int32_t row_stride;             // elements between consecutive keys: Hkv * D (paged, blhd) or D (bhld)
  int32_t contig;                 // 1: contiguous K/V, sequence b is page b (no block table)
  int32_t B, q_len, Hq, Hkv, G, R;  // R = G * q_len rows per kv head
  int32_t page_shift;             // log2(page_size); 30 for contiguous K/V
  int32_t max_pages;              // block_table row stride
  int32_t S;                      // splits
  int32_t chunk;                  // keys per split (multiple of the tile)
  int32_t nrb;                    // row blocks per kv head
  int32_t hpb, lhpb;              // kv heads per workgroup (1, 2 or 4) and its log2
  int32_t causal_offset;          // -1 off, kCausalLast, >= 0 (overridden by causal_offsets)
  float scale_log2;               // scale * log2(e)
  int32_t outer;                  // B * S pairs (sequence, split); exact schedule: a bound on the items
  int32_t inner;                  // (Hkv / hpb) * nrb unit slots (kv-head group, row block) per pair;
                                  // exact schedule: Hkv / hpb kv-head groups per item
  int32_t exact;                  // 1: exact schedule (B <= 64 * kExactPerLane)
  int32_t lpt;                    // 1: the exact schedule deals its items longest first
  int32_t rp;                     // packed rows per row block (a power of two)
  int32_t partials;               // 1: write o_part/ml_part even when S == 1
  int32_t fused;                  // 1: the last block of a unit merges the partials (S > 1)
  int32_t wide_part;              // 1: o_part under 2^31 bytes (16-byte partial stores, store_part4)
  int32_t pair;                   // 1: head pairing -- kv heads 2g, 2g + 1 of 32 columns read as one
                                  // head g of 64 (the fields above describe that problem: Hkv / 2
                                  // heads, G = 2 * G_real); q, out and the partials keep 32 columns
  int32_t *counters;              // [units] arrival counters (fused), zero between calls
  int64_t rows;                   // output rows: tokens * Hq
};

struct CombineArgs {
  const float *o_part;
  const float *ml_part;
  uint16_t *out;
  float *out_f32;
  int64_t rows;
  int32_t S;
};

// Which split kernel serves a problem.  R = G * q_len rows share a kv head.
// Up to 2 rows run on the VALU kernel (rows padded to RP in {1, 2}); from 3
// rows on, the matrix-core kernel (16-row tiles, one or two per workgroup)
// was measured as fast or faster on gfx950 even with most of a tile padded
// (R = 3, 4, 6, 8), so it takes over there -- except at head_dim 256, where
// the matrix-core kernel keeps one register tile per wave and one workgroup
// per CU (more spill) and the VALU kernel (RP = 4) stays ahead up to 4 rows.
// Measured on MI355X, Hkv = 8, bench protocol, matrix-core -> VALU: B = 16 x
// 4096 keys with 32 query heads 93.8 -> 92.5 us, with 24 query heads
// 93.5 -> 91.4 us, 16 query heads x 2 tokens 94.3 -> 92.1 us; B = 16 x 8192
// keys 176.8 -> 172.2 us, x 1024 keys 31.5 -> 30.3 us (at 8 rows the VALU
// kernel is slower everywhere).
inline bool use_mfma(int R, int head_dim) { return head_dim == 256 ? R > 4 : R > 2; }
// The prefill-shaped matrix-core kernel: four waves of 32 rows each share
// every K/V tile (128 rows per workgroup), so a key is read once per 128 rows
// rather than once per 32.  Taken at D <= 128 with one kv head per workgroup
// from 128 rows on (a chunk of 128 / G tokens).  Measured on MI355X against
// the 32-row kernel (Hq = 32, Hkv = 8, D = 128, causal at the sequence end;
// B x tokens over keys): 4 x 512 over 4096 369 -> 243 us, 1 x 2048 over 2048
// 134 -> 101 us, 8 x 128 over 8192 384 -> 271 us, 1 x 512 over 8192
// 187 -> 157 us, 64 x 32 over 1024 138 -> 74 us, 16 x 64 over 4096
// 217 -> 166 us, 8 x 32 over 8192 136 -> 109 us; a varlen batch of 32
// sequences of which a quarter hold prefill chunks of up to 64 tokens (256
// rows) 115 us either way.
constexpr int kPrefillRows = 128;      // rows per prefill-shaped workgroup
constexpr int kPrefillMinRows = 128;   // packed rows per kv head from which it is taken
inline bool use_prefill(int R, int head_dim, int hpb) {
  return R >= kPrefillMinRows && head_dim <= 128 && hpb <= 1;
}
// The split kernels (pkv_plan_info.kernel): the vector kernel (one or two
// rows per kv head), the one-head matrix-core kernel (each wave its own
// 16-key tiles of one kv head), the shared-tile matrix-core kernel (a
// workgroup of 4 or 8 kv heads whose waves share whole head-group K/V tiles
// in LDS: with 8 heads always, with 4 heads from 3 rows on at D <= 128) and
// the prefill-shaped kernel.  hpb: the kv heads per workgroup of the plan (0
// or 1 for one).
enum { kKernelValu = 0, kKernelMfma = 1, kKernelGroup = 2, kKernelPrefill = 3 };
inline int kernel_kind(int R, int head_dim, int hpb) {
  if (use_prefill(R, head_dim, hpb)) return kKernelPrefill;
  if (hpb == 8 || (hpb == 4 && R > 2 && head_dim <= 128)) return kKernelGroup;
  return use_mfma(R, head_dim) ? kKernelMfma : kKernelValu;
}
// rows per workgroup and kv head: RP (vector kernel, 1, 2 or 4), 16/32
// (matrix-core kernels) or 128 (prefill-shaped)
int rows_per_block(int R, int head_dim, int hpb);
int tile_keys(int head_dim);       // keys per VALU wave tile T (a multiple of 16)
constexpr int kWavesPerBlock = 4;  // waves per split workgroup
constexpr int kCausalLast = -2;    // causal_offset: the query tokens are the sequence's last keys
constexpr int kMaxHeadsPerBlock = 4;  // kv heads a one-head-per-wave workgroup may cover (one wave or more each)
constexpr int kMaxGroupHeads = 8;     // kv heads a shared-tile workgroup may cover (HW = hpb / 4 per wave)

// Blocks of a split-kernel grid: 8 XCD queues of equal length holding every
// (pair, unit slot), or (exact schedule) the item bound times the groups.
inline int64_t split_grid(const DecodeArgs &a) {
  if (a.outer < 8 && !a.exact) return ((int64_t)a.outer * a.inner + 7) / 8 * 8;
  return ((int64_t)a.outer + 7) / 8 * 8 * a.inner;
}

// Launchers (return a hipError_t value).
int launch_split(const DecodeArgs &a, int head_dim, int rp, bool causal,
                 bool has_mask, hipStream_t stream);
int launch_split_mfma(const DecodeArgs &a, int head_dim, int nrb16, bool causal, bool has_mask,
                      hipStream_t stream);
int launch_split_prefill(const DecodeArgs &a, int head_dim, bool causal, bool has_mask, hipStream_t stream);
int launch_split_group(const DecodeArgs &a, int head_dim, int nrb16, bool causal, bool has_mask,
                       hipStream_t stream);
int launch_combine(const CombineArgs &a, int head_dim, hipStream_t stream);
int launch_zero(void *p, int64_t words, hipStream_t stream);

// The static split workspace of pkv_paged_decode_noalloc (pkv_noalloc.hip):
// the current device's copy of the scratch array (looked up once per device)
// and whether its counter head has been zeroed yet; returns a PKV status.
int noalloc_scratch(void **ptr, bool *cleared);
void noalloc_mark_cleared();

}  // namespace pkv
