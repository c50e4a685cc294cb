// pkv_host.cpp -- host side of the C ABI: argument checks, split heuristic,
// workspace sizing and launch of the split kernels (which merge their splits
// themselves up to PKV_MAX_FUSED_UNITS units) and of the combine kernel.
//
// Every check runs before the first HIP call, so a rejected call enqueues
// nothing; the HIP calls made are kernel launches on the caller's stream,
// hipGetLastError after them, and (once per device, for the split heuristic)
// a compute-unit query.
#include <math.h>
#include <stddef.h>
#include <stdint.h>

#include <atomic>

#include <hip/hip_runtime_api.h>

#include "pkv.h"
#include "pkv_internal.h"

namespace {

constexpr int kMaxDevices = 64;
std::atomic<int> g_cus[kMaxDevices];  // 0 = not queried yet

// A launch's work-items (blocks x 256 threads) must fit 32 bits.
constexpr int64_t kMaxBlocks = (int64_t)0xFFFFFFFF / 256;

bool is_pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }

int ilog2(int x) {
  int s = 0;
  while ((1 << s) < x) ++s;
  return s;
}

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

bool supported_dim(int d) { return d == 32 || d == 64 || d == 128 || d == 256; }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Shape checks common to every entry point taking a pkv_problem.
int check_problem(const pkv_problem *p) {
  if (!p) return PKV_ERR_NULL;
  if (p->batch < 0 || p->q_len < 1 || p->num_q_heads < 1 || p->num_kv_heads < 1)
    return PKV_ERR_SHAPE;
  if (p->num_q_heads % p->num_kv_heads) return PKV_ERR_SHAPE;
  if (!supported_dim(p->head_dim)) return PKV_ERR_UNSUPPORTED;
  // a key row of all kv heads (Hkv * D elements) times a tile of keys must fit 32 bits
  if ((int64_t)p->num_kv_heads * p->head_dim > (1 << 24)) return PKV_ERR_SHAPE;
  if (!is_pow2(p->page_size) || p->page_size > 4096) return PKV_ERR_UNSUPPORTED;
  if (p->num_pages < 0 || p->max_pages_per_seq < 1) return PKV_ERR_SHAPE;
  if (p->max_kv_len < 0) return PKV_ERR_SHAPE;
  const int64_t cap = (int64_t)p->max_pages_per_seq * p->page_size;
  if (cap > INT32_MAX) return PKV_ERR_SHAPE;
  if ((int64_t)p->max_kv_len > cap) return PKV_ERR_SHAPE;
  if (!isfinite(p->scale)) return PKV_ERR_SHAPE;
  if (p->causal_offset < PKV_CAUSAL_LAST) return PKV_ERR_SHAPE;
  if (p->num_splits < 0) return PKV_ERR_SHAPE;
  if (p->num_splits > PKV_MAX_SPLITS) return PKV_ERR_UNSUPPORTED;
  if (p->heads_per_block < 0) return PKV_ERR_SHAPE;
  if (p->heads_per_block > 0) {
    if (!is_pow2(p->heads_per_block) || p->heads_per_block > pkv::kMaxGroupHeads) return PKV_ERR_UNSUPPORTED;
    // eight kv heads per workgroup: the shared-tile kernel, built for D <= 64
    if (p->heads_per_block == 8 && p->head_dim > 64) return PKV_ERR_UNSUPPORTED;
    if (p->num_kv_heads % p->heads_per_block) return PKV_ERR_SHAPE;
  }
  if (p->mask_stride_b < 0 || p->mask_stride_q < 0) return PKV_ERR_SHAPE;
  // rows * D and pool sizes must fit the 64-bit element arithmetic used on device
  const int64_t rows = (int64_t)p->batch * p->q_len * p->num_q_heads;
  if (rows > (int64_t)1 << 40) return PKV_ERR_SHAPE;
  return PKV_OK;
}

// Host-known bound on the keys of any sequence.
int max_len_of(const pkv_problem *p) {
  return p->max_kv_len > 0 ? p->max_kv_len : p->max_pages_per_seq * p->page_size;
}

int query_cus(int *out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return PKV_ERR_DEVICE;
  if (dev < kMaxDevices) {
    int c = g_cus[dev].load(std::memory_order_relaxed);
    if (c > 0) { *out = c; return PKV_OK; }
  }
  int c = 0;
  if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c <= 0)
    return PKV_ERR_DEVICE;
  if (dev < kMaxDevices) g_cus[dev].store(c, std::memory_order_relaxed);
  *out = c;
  return PKV_OK;
}

// Split heuristic (keys only along the sequence axis, in the spirit of the
// pages' compute_num_splits and ejkernel's num_splits = 0 "auto").  Few
// units: split each sequence so that the grid has about blocks_per_cu()
// workgroups per CU, never below kMinTilesPerWave tiles per wave and never
// above 64 splits.  Units that fill the chip by themselves: cap the keys of
// one workgroup at split_cap_keys(), so that in a ragged batch the longest
// sequences do not run alone at the end of the launch (splits past a
// sequence's end exit at once; a sequence that fits one split writes its
// output directly).
constexpr int kMinTilesPerWave = 2;

// Keys per workgroup in a batch that fills the chip: at least 1024, and at
// least 64 per packed row, so that the partials of a split sequence (rows * D
// fp32 per split, written and read back) stay within 2 / 64 of its K/V bytes.
// Measured on MI355X for B = 256 lognormal lengths (median 1024, clipped to
// [32, 8192], 32 rows per kv head, D = 128): 4 splits of 2048 keys in place
// of one take a call from 425 to 377 us (8 splits of 1024: 403 us).
int split_cap_keys(int rows) {
  const int cap = 64 * rows;
  return cap > 1024 ? cap : 1024;
}

// Workgroups per CU to aim at, measured on MI355X over the decode shapes:
// one where a workgroup keeps enough K/V bytes in flight to cover memory
// latency (VALU kernel: 8-16 KB tiles per wave; matrix-core kernel at
// D = 128) or sits at the register limit (matrix-core kernel at D = 256:
// 16 sequences x 1024 / 4096 / 8192 keys, 32 query heads, 2 splits against 4:
// 31.6 / 93.3 / 176.0 against 32.6 / 96.3 / 181.3 us), two where it keeps
// fewer (matrix-core 16-key tiles of 2-4 KB at D <= 64).
// The prefill-shaped kernel: one, its 128-row workgroups being compute-heavy
// (4 x 64 tokens over 2048 keys: 4 splits 52 us, 8 splits 68 us; 8 x 32 over
// 8192: 109 against 123 us).
// The shared-tile kernel (two workgroups of at most 80 KB of LDS per CU): two.
int blocks_per_cu(const pkv_problem *p, int hpb) {
  const int R = (p->num_q_heads / p->num_kv_heads) * p->q_len;
  switch (pkv::kernel_kind(R, p->head_dim, hpb)) {
    case pkv::kKernelPrefill: return 1;
    case pkv::kKernelGroup: return 2;
    case pkv::kKernelMfma: return p->head_dim >= 128 ? 1 : 2;
    default: return 1;
  }
}

// The kernel serving the problem with hpb kv heads per workgroup.
int kernel_of(const pkv_problem *p, int hpb) {
  const int R = (p->num_q_heads / p->num_kv_heads) * p->q_len;
  return pkv::kernel_kind(R, p->head_dim, hpb);
}

// Packed rows per workgroup and kv head (the kernel family follows from it).
int rows_per_block_of(const pkv_problem *p, int hpb) {
  const int R = (p->num_q_heads / p->num_kv_heads) * p->q_len;
  return pkv::rows_per_block(R, p->head_dim, hpb);
}

// Row blocks per kv head.
int64_t row_blocks(const pkv_problem *p, int hpb) {
  const int R = (p->num_q_heads / p->num_kv_heads) * p->q_len;
  return ceil_div(R, rows_per_block_of(p, hpb));
}

// (sequence, kv-head group, row block) units with hpb kv heads per group:
// the workgroups of one unit differ only in their split.
int64_t units_of(const pkv_problem *p, int hpb) {
  return (int64_t)p->batch * (p->num_kv_heads / hpb) * row_blocks(p, hpb);
}

// Varlen batches up to this size take the exact schedule (every workgroup
// counts the work items of the whole batch, each lane a run of up to 4
// sequences, which keeps the kernels' register counts unchanged); other
// calls get one block per (sequence, split, row block).  Measured on MI355X:
// a batch of 32 sequences, a quarter with prefill chunks of up to 64 tokens,
// 240 -> 110 us.  Fixed-length batches keep the per-block split-major order:
// there the exact schedule won only on the B = 256, q_len = 4 lognormal batch
// at 4 splits (2-5%) and lost elsewhere (the same batch at 8 splits 8-13%,
// other ragged shapes 1-3%, the 1B decode shape 10.0 -> 11.0 us).
constexpr int kExactMaxBatch = 64 * 4;
// Fixed-length batches from this many sequences on also take the exact
// schedule, dealt longest first (their lengths may differ widely; the
// workgroups of the longest splits then start first).
constexpr int kLptMinBatch = 32;

// Row-block slots the grid holds: B * ceil(R / rp); a varlen batch of
// `tokens` tokens under the exact schedule at most floor(tokens * G / rp) + B
// (sequence b has ceil(n_b * G / rp) <= floor(n_b * G / rp) + 1 row blocks).
int64_t row_block_slots(const pkv_problem *p, int64_t tokens, int hpb) {
  const int64_t all = (int64_t)p->batch * row_blocks(p, hpb);
  if (tokens < 0 || p->batch > kExactMaxBatch) return all;
  const int G = p->num_q_heads / p->num_kv_heads;
  const int rp = rows_per_block_of(p, hpb);
  const int64_t nv = tokens * G / rp + p->batch;
  return nv < all ? nv : all;
}

// Units of the grid: (sequence, kv-head group, row block) slots.
int64_t grid_units(const pkv_problem *p, int hpb, int64_t tokens) {
  return row_block_slots(p, tokens, hpb) * (p->num_kv_heads / hpb);
}

// The work the split heuristic sizes the grid for: (sequence, kv-head group,
// row block) units that hold rows, and packed rows per such unit.  A batch
// of q_len tokens per sequence (or a varlen batch that has them all): every
// unit, R rows.  A varlen batch of `tokens` tokens: its row blocks number at most
// ceil(tokens * G / rp) + B (each sequence may end in a partial block), and
// the rows spread over them; the other units of the grid exit at once.
struct Load {
  int64_t units;
  int rows;
};

Load load_of(const pkv_problem *p, int hpb, int64_t tokens) {
  const int G = p->num_q_heads / p->num_kv_heads;
  const int R = G * p->q_len;
  if (tokens < 0 || tokens >= (int64_t)p->batch * p->q_len) return Load{units_of(p, hpb), R};
  int64_t rb = ceil_div(tokens * G, rows_per_block_of(p, hpb)) + p->batch;
  const int64_t all = (int64_t)p->batch * row_blocks(p, hpb);
  if (rb > all) rb = all;
  int64_t rows = ceil_div(tokens * G, rb);
  if (rows < 1) rows = 1;
  return Load{rb * (p->num_kv_heads / hpb), (int)(rows < R ? rows : R)};
}

int heuristic_splits(const pkv_problem *p, int cus, int hpb, int64_t tokens) {
  const Load ld = load_of(p, hpb, tokens);
  const int64_t units = ld.units;
  if (units <= 0 || tokens == 0) return 1;
  const int64_t target = (int64_t)cus * blocks_per_cu(p, hpb);
  if (units >= target) {
    const int64_t s = ceil_div(max_len_of(p), split_cap_keys(ld.rows));
    return (int)(s < 1 ? 1 : (s > 64 ? 64 : s));
  }
  // at least kMinTilesPerWave tiles per wave (the shared-tile kernel's waves
  // all see every tile of the split)
  const int T = pkv::tile_keys(p->head_dim);
  const int wpt = kernel_of(p, hpb) == pkv::kKernelGroup || hpb >= pkv::kWavesPerBlock
                      ? 1 : pkv::kWavesPerBlock / hpb;
  const int64_t min_keys = (int64_t)T * wpt * kMinTilesPerWave;
  const int64_t max_by_len = ceil_div(max_len_of(p), min_keys);
  int64_t s = target / units;
  if (s > max_by_len) s = max_by_len;
  // a varlen batch mixes sequences of few rows (decode tokens) with long
  // key ranges: cap the keys per workgroup as for a full chip
  if (tokens >= 0) {
    const int64_t sc = ceil_div(max_len_of(p), split_cap_keys(ld.rows));
    if (sc > s) s = sc;
  }
  if (s > 64) s = 64;
  if (s < 1) s = 1;
  return (int)s;
}

// Kv heads per workgroup.  Grouping the heads of a page slot in one
// workgroup (one or two waves per head) makes it read longer runs of each
// slot, which HBM serves faster than separate D * 2-byte head slices.
// Measured on MI355X (B = 16, 4096 keys, Hkv = 8): the VALU kernel gains 13%
// at D = 64 and 5% at D = 128 with four heads, nothing at D = 256; the
// matrix-core kernel gains 2-3% with two heads at D = 64 and 128 and loses
// with four (its 16-key tiles keep fewer bytes in flight per wave) and at
// D = 32 and 256; in batches that fill the chip the VALU kernel gains up to
// 13% with four heads (B = 64 and 256).  Grouping is taken only while the
// split count stays in [2, kMaxGroupedSplits]: at one split a workgroup would
// hold hpb whole sequences, which ragged lengths unbalance (B = 256 lognormal
// lengths: 1.65x slower), and more splits cost more partial traffic; and only
// while a split holds at most kMaxGroupedChunk keys: grouping halves the
// units, and a grid of few long splits leaves the chip idle behind the
// longest sequences (B = 32 lognormal lengths up to 8192 keys, D = 128:
// two heads at 2 splits 108 us, one head at 8 splits 61 us).
constexpr int kMaxGroupedSplits = 8;
constexpr int64_t kMaxGroupedChunk = 2048;

int max_heads_per_block(const pkv_problem *p) {
  const int R = (p->num_q_heads / p->num_kv_heads) * p->q_len;
  if (pkv::use_prefill(R, p->head_dim, 1)) return 1;
  if (pkv::use_mfma(R, p->head_dim)) return (p->head_dim == 64 || p->head_dim == 128) ? 2 : 1;
  return p->head_dim <= 128 ? pkv::kMaxHeadsPerBlock : 1;
}

int heuristic_hpb(const pkv_problem *p, int cus, int64_t tokens) {
  for (int hpb = max_heads_per_block(p); hpb > 1; hpb /= 2) {
    if (p->num_kv_heads % hpb) continue;
    const int s = p->num_splits > 0 ? p->num_splits : heuristic_splits(p, cus, hpb, tokens);
    if (s >= 2 && s <= kMaxGroupedSplits && ceil_div(max_len_of(p), s) <= kMaxGroupedChunk) return hpb;
  }
  return 1;
}

// The launch plan of a problem on a device with `cus` compute units.
struct Plan {
  int S;          // splits
  int hpb;        // kv heads per workgroup
  int64_t units;  // (sequence, kv-head group, row block) units
  bool fused;     // pkv_paged_decode merges the splits inside the split kernel
};

// tokens: -1 for q_len tokens per sequence, else a varlen batch's total.  A
// varlen batch that holds every token (B * q_len) is planned as the
// fixed-length batch, so both entry points give it the same splits and
// grouping, hence the same bits.
Plan make_plan(const pkv_problem *p, int cus, int64_t tokens = -1) {
  if (tokens >= (int64_t)p->batch * p->q_len) tokens = -1;
  Plan pl;
  pl.hpb = p->heads_per_block > 0 ? p->heads_per_block : heuristic_hpb(p, cus, tokens);
  pl.S = p->num_splits > 0 ? p->num_splits : heuristic_splits(p, cus, pl.hpb, tokens);
  pl.units = grid_units(p, pl.hpb, tokens);
  // In-kernel merge (a counter for every unit) whenever the counters fit the
  // workspace head.  Splits past a sequence's end exit at once and a unit
  // with one split holding keys writes its output directly, so only units
  // split for real merge, each as soon as its last split ends; on MI355X this
  // matched or beat a separate combine launch from 24 to 8192 workgroups
  // (B = 256 ragged: 377 against 403 us).
  pl.fused = pl.S > 1 && pl.units <= PKV_MAX_FUSED_UNITS;
  return pl;
}

// Head pairing.  At head_dim 32 one kv head's slice of a key row is 64
// bytes, half of a 128-byte cache line whose other half is the next head's;
// requests for half lines leave memory concurrency unused (the L2 held about
// half the reads in flight that it holds at head_dim 64 and up).  Two
// adjacent kv heads 2g, 2g + 1 are then read as one head g of 64 columns --
// in the paged and [B, L, Hkv, D] layouts their slices are adjacent in every
// key row (in [B, Hkv, L, D] they are not: that layout runs the paired
// problem's split count, one kv head per workgroup, so that a problem's split
// count and workspace do not depend on its layout) -- whose packed rows are
// the query heads of both: a row's q fills
// its own head's half and is zero in the other, so its scores are those of
// its own head, and its output is its half of the 64 columns.  The paired
// problem (Hkv / 2 heads of 64 columns, 2G query heads per kv head) is planned
// and launched like any other, on the vector kernel (one query head per kv
// head: two rows) or the matrix-core kernel (up to 16 rows).  Measured on
// MI355X, B = 16, 4096 keys, Hkv = 8, with 64-column heads standing in for the
// pairs: 8 query heads 19.8 -> 17.9 us, 32 query heads 20.9 -> 18.2 us, 64
// query heads 21.0 -> 18.9 us.  Not with forced kv heads per workgroup (they
// count real heads).
bool pair_eligible(const pkv_problem *p) {
  if (p->head_dim != 32 || (p->num_kv_heads & 1) || p->heads_per_block != 0) return false;
  const int R = (p->num_q_heads / p->num_kv_heads) * p->q_len;
  return 2 * R <= 16;
}

bool pair_heads(const pkv_problem *p, int layout) { return layout != PKV_KV_BHLD && pair_eligible(p); }

pkv_problem paired_problem(const pkv_problem *p) {
  pkv_problem v = *p;
  v.head_dim = 2 * p->head_dim;
  v.num_kv_heads = p->num_kv_heads / 2;
  return v;
}

// The plan of a problem whose K/V sit in `layout` (0: paged): with head
// pairing, that of the paired problem (its kv heads per workgroup count
// pairs).
Plan plan_of(const pkv_problem *p, int layout, int cus, int64_t tokens = -1) {
  if (!pair_eligible(p)) return make_plan(p, cus, tokens);
  const pkv_problem v = paired_problem(p);
  const Plan pl = make_plan(&v, cus, tokens);
  if (pair_heads(p, layout)) return pl;
  pkv_problem u = *p;   // [B, Hkv, L, D]: the paired split count, one kv head per workgroup
  u.num_splits = pl.S;
  u.heads_per_block = 1;
  return make_plan(&u, cus, tokens);
}

// ml_part bytes of pkv_paged_decode with S >= 2 splits: counter head + (m, l).
size_t ml_bytes_split(const pkv_problem *p, int S) {
  const size_t rows = (size_t)p->batch * p->q_len * p->num_q_heads;
  return (size_t)PKV_COUNTER_BYTES + rows * (size_t)S * 2 * sizeof(float);
}

}  // namespace

extern "C" {

const char *pkv_status_string(int status) {
  switch (status) {
    case PKV_OK: return "ok";
    case PKV_ERR_NULL: return "a required pointer is NULL";
    case PKV_ERR_SHAPE: return "invalid problem shape or stride";
    case PKV_ERR_UNSUPPORTED: return "unsupported head_dim, page_size or split count";
    case PKV_ERR_WORKSPACE: return "split workspace missing or too small";
    case PKV_ERR_ALIGN: return "pointer misaligned";
    case PKV_ERR_LAUNCH: return "kernel launch failed";
    case PKV_ERR_DEVICE: return "device query failed";
    case PKV_ERR_SCRATCH: return "split workspace exceeds the static scratch buffer";
    default: return "unknown status";
  }
}

int pkv_device_cus(int *num_cus) {
  if (!num_cus) return PKV_ERR_NULL;
  return query_cus(num_cus);
}

int pkv_num_splits(const pkv_problem *p, int num_cus, int *splits_out) {
  if (!splits_out) return PKV_ERR_NULL;
  int rc = check_problem(p);
  if (rc) return rc;
  if (p->num_splits > 0) { *splits_out = p->num_splits; return PKV_OK; }
  if (num_cus <= 0) {
    rc = query_cus(&num_cus);
    if (rc) return rc;
  }
  *splits_out = plan_of(p, 0, num_cus).S;
  return PKV_OK;
}

namespace {

int plan_query(const pkv_problem *p, int64_t tokens, int num_cus, pkv_plan_info *info) {
  if (!info) return PKV_ERR_NULL;
  int rc = check_problem(p);
  if (rc) return rc;
  if (tokens > (int64_t)p->batch * p->q_len) return PKV_ERR_SHAPE;
  if (num_cus <= 0) {
    rc = query_cus(&num_cus);
    if (rc) return rc;
  }
  const Plan pl = plan_of(p, 0, num_cus, tokens);
  const bool pair = pair_heads(p, 0);
  const pkv_problem pv = pair ? paired_problem(p) : *p;
  *info = pkv_plan_info{};
  info->splits = pl.S;
  info->heads_per_block = pair ? 2 * pl.hpb : pl.hpb;
  info->rows_per_block = rows_per_block_of(&pv, pl.hpb);
  info->kernel = kernel_of(&pv, pl.hpb);
  info->paired_heads = pair ? 1 : 0;
  info->matrix_core = info->kernel == pkv::kKernelValu ? 0 : 1;
  info->units = pl.units;
  info->workgroups = pl.units * pl.S;
  info->merge_in_kernel = pl.fused ? 1 : 0;
  info->kernels = (pl.S > 1 && !pl.fused && p->batch > 0) ? 2 : (p->batch > 0 ? 1 : 0);
  return PKV_OK;
}

}  // namespace

int pkv_plan(const pkv_problem *p, int num_cus, pkv_plan_info *info) {
  return plan_query(p, -1, num_cus, info);
}

int pkv_plan_varlen(const pkv_problem *p, int64_t total_tokens, int num_cus, pkv_plan_info *info) {
  if (total_tokens < 0) return PKV_ERR_SHAPE;
  return plan_query(p, total_tokens, num_cus, info);
}

int pkv_workspace_bytes(const pkv_problem *p, int splits, size_t *o_part_bytes,
                        size_t *ml_part_bytes) {
  if (!o_part_bytes || !ml_part_bytes) return PKV_ERR_NULL;
  int rc = check_problem(p);
  if (rc) return rc;
  if (splits < 1) return PKV_ERR_SHAPE;
  if (splits > PKV_MAX_SPLITS) return PKV_ERR_UNSUPPORTED;
  if (splits == 1) { *o_part_bytes = 0; *ml_part_bytes = 0; return PKV_OK; }
  const size_t rows = (size_t)p->batch * p->q_len * p->num_q_heads;
  *o_part_bytes = rows * (size_t)splits * (size_t)p->head_dim * sizeof(float);
  *ml_part_bytes = ml_bytes_split(p, splits);
  return PKV_OK;
}

int pkv_workspace_clear(void *ptr, size_t bytes, hipStream_t stream) {
  if (bytes == 0) return PKV_OK;
  if (!ptr) return PKV_ERR_NULL;
  if (!aligned(ptr, 4) || (bytes & 3)) return PKV_ERR_ALIGN;
  (void)hipGetLastError();
  return pkv::launch_zero(ptr, (int64_t)(bytes / 4), stream) == hipSuccess ? PKV_OK : PKV_ERR_LAUNCH;
}

}  // extern "C"

namespace {

// Checks and launch plan shared by pkv_paged_decode (partials_only = false)
// and pkv_paged_decode_partials (true).  Returns a status; on PKV_OK `a`
// holds the split-kernel arguments (a->S is the split count).
// Where the keys live: paged (block table) or contiguous per sequence.
struct KvSource {
  const void *k, *v;
  const int32_t *block_table;  // paged only
  int layout;                  // 0 paged, PKV_KV_BLHD or PKV_KV_BHLD
  int64_t capacity;            // contiguous: keys per sequence in the cache
};

// Query tokens: q_len per sequence, or (cu_q) a varlen batch of
// total_tokens tokens packed by sequence, at most q_len each.
struct QSource {
  const int32_t *cu_q;
  int64_t total_tokens;
};

int plan_decode(const pkv_problem *p, const void *q, const QSource &qs, const KvSource &src,
                const int32_t *kv_lens, const int32_t *causal_offsets, const float *mask, float *o_part,
                size_t o_part_bytes, float *ml_part, size_t ml_part_bytes, void *out_bf16, float *out_f32,
                bool partials_only, pkv::DecodeArgs *a) {
  const bool paged = src.layout == 0;
  const int32_t *block_table = src.block_table;
  if (!q || !src.k || !src.v || (paged && !block_table) || !kv_lens) return PKV_ERR_NULL;
  if (!partials_only && !out_bf16) return PKV_ERR_NULL;
  if (!aligned(q, 16) || !aligned(src.k, 16) || !aligned(src.v, 16) ||
      (out_bf16 && !aligned(out_bf16, 16)) || (paged && !aligned(block_table, 4)) || !aligned(kv_lens, 4) ||
      (causal_offsets && !aligned(causal_offsets, 4)) || (mask && !aligned(mask, 4)) ||
      (out_f32 && !aligned(out_f32, 16)))
    return PKV_ERR_ALIGN;

  // split count: forced, or the heuristic (needs the device's CU count)
  int cus = 0;
  int S = p->num_splits;
  if (S == 0) {
    const int rc = query_cus(&cus);
    if (rc) return rc;
    S = plan_of(p, src.layout, cus, qs.cu_q ? qs.total_tokens : -1).S;
  }
  // pkv_paged_decode with several splits: ml_part = counter head + (m, l)
  const bool split_ws = S > 1 && !partials_only;
  if (S > 1 || partials_only) {
    const size_t rows = (size_t)p->batch * p->q_len * p->num_q_heads;
    const size_t need_o = rows * (size_t)S * (size_t)p->head_dim * sizeof(float);
    const size_t need_ml = split_ws ? ml_bytes_split(p, S) : rows * (size_t)S * 2 * sizeof(float);
    if (!o_part || !ml_part || o_part_bytes < need_o || ml_part_bytes < need_ml) return PKV_ERR_WORKSPACE;
    if (!aligned(o_part, 16) || !aligned(ml_part, split_ws ? 16 : 8)) return PKV_ERR_ALIGN;
  }

  // heads per workgroup and merge path (the CU count is needed unless both
  // are fixed: one forced split and forced heads per workgroup)
  Plan pl{S, p->heads_per_block, 0, false};
  if (S > 1 || p->heads_per_block == 0) {
    if (cus == 0) {
      const int rc = query_cus(&cus);
      if (rc) return rc;
    }
    pl = plan_of(p, src.layout, cus, qs.cu_q ? qs.total_tokens : -1);
  }
  const int64_t tokens = qs.cu_q ? qs.total_tokens : -1;
  const bool exact = p->batch <= kExactMaxBatch && (tokens >= 0 || p->batch >= kLptMinBatch);
  // the launch's problem: with head pairing, Hkv / 2 heads of 64 columns
  const bool pair = pair_heads(p, src.layout);
  const pkv_problem pv = pair ? paired_problem(p) : *p;
  pl.units = grid_units(&pv, pl.hpb, tokens);

  const int G = pv.num_q_heads / pv.num_kv_heads;
  const int R = G * pv.q_len;
  const int rp = rows_per_block_of(&pv, pl.hpb);
  const int T = pkv::tile_keys(pv.head_dim);
  const int64_t L = max_len_of(p);
  int64_t chunk = ceil_div(ceil_div(L, S), T) * T;
  if (chunk < T) chunk = T;
  if (chunk > INT32_MAX) return PKV_ERR_SHAPE;

  *a = pkv::DecodeArgs{};
  a->q = static_cast<const uint16_t *>(q);
  a->k = static_cast<const uint16_t *>(src.k);
  a->v = static_cast<const uint16_t *>(src.v);
  a->block_table = paged ? block_table : nullptr;
  a->cu_q = qs.cu_q;
  a->rows = qs.total_tokens * p->num_q_heads;
  a->kv_lens = kv_lens;
  a->causal_offsets = causal_offsets;
  a->mask = mask;
  a->o_part = (S > 1 || partials_only) ? o_part : nullptr;
  a->ml_part = split_ws ? ml_part + PKV_COUNTER_BYTES / sizeof(float)
                        : ((S > 1 || partials_only) ? ml_part : nullptr);
  a->out = static_cast<uint16_t *>(out_bf16);
  a->out_f32 = out_f32;
  a->mask_sb = p->mask_stride_b;
  a->mask_sq = p->mask_stride_q;
  if (paged) {
    a->page_stride = (int64_t)p->page_size * p->num_kv_heads * p->head_dim;
    a->row_stride = p->num_kv_heads * p->head_dim;
    a->head_stride = pv.head_dim;   // paired: head g of the launch starts at kv head 2g
    a->page_shift = ilog2(p->page_size);
    a->max_pages = p->max_pages_per_seq;
  } else {  // one page of 2^30 key slots per sequence, addressed with the cache's strides
    a->page_stride = src.capacity * p->num_kv_heads * p->head_dim;
    a->row_stride = src.layout == PKV_KV_BLHD ? p->num_kv_heads * p->head_dim : p->head_dim;
    a->head_stride = src.layout == PKV_KV_BLHD ? (int64_t)pv.head_dim : src.capacity * p->head_dim;
    a->page_shift = 30;
    a->max_pages = 1;
    a->contig = 1;
  }
  a->B = p->batch;
  a->q_len = p->q_len;
  a->Hq = p->num_q_heads;
  a->Hkv = pv.num_kv_heads;
  a->G = G;
  a->R = R;
  a->S = S;
  a->chunk = (int32_t)chunk;
  a->nrb = (R + rp - 1) / rp;
  a->hpb = pl.hpb;
  a->lhpb = ilog2(pl.hpb);
  a->causal_offset = p->causal_offset;
  a->scale_log2 = p->scale * 1.4426950408889634f;
  a->exact = exact ? 1 : 0;
  a->rp = rp;
  const int64_t outer = (exact ? row_block_slots(&pv, tokens, pl.hpb) : (int64_t)p->batch) * S;
  const int64_t inner = (int64_t)(pv.num_kv_heads / pl.hpb) * (exact ? 1 : a->nrb);
  if (outer > INT32_MAX / 8 || inner * ceil_div(outer, 8) * 8 > kMaxBlocks) return PKV_ERR_SHAPE;
  // the combine kernel's grid (several splits without the in-kernel merge)
  const int64_t rows_all = (int64_t)p->batch * p->q_len * p->num_q_heads;
  if (ceil_div(rows_all, 2) > kMaxBlocks) return PKV_ERR_SHAPE;
  a->outer = (int32_t)outer;
  a->inner = (int32_t)inner;
  a->partials = (S > 1 || partials_only) ? 1 : 0;
  a->fused = split_ws && pl.fused ? 1 : 0;
  a->wide_part = a->o_part && o_part_bytes <= (size_t)INT32_MAX ? 1 : 0;
  a->pair = pair ? 1 : 0;
  a->counters = a->fused ? reinterpret_cast<int32_t *>(ml_part) : nullptr;
  // longest first where every split past a sequence's keys is trimmed
  a->lpt = exact && (a->fused || S == 1) ? 1 : 0;
  return PKV_OK;
}

int launch_plan(const pkv::DecodeArgs &a, const pkv_problem *p, hipStream_t stream) {
  const bool causal = a.causal_offsets != nullptr || p->causal_offset >= 0 || p->causal_offset == PKV_CAUSAL_LAST;
  (void)hipGetLastError();
  const int rows = a.rp;
  const bool mask = a.mask != nullptr;
  const int hd = a.pair ? 2 * p->head_dim : p->head_dim;   // the launch's head width
  int err;
  switch (pkv::kernel_kind(a.R, hd, a.hpb)) {
    case pkv::kKernelPrefill: err = pkv::launch_split_prefill(a, hd, causal, mask, stream); break;
    case pkv::kKernelGroup: err = pkv::launch_split_group(a, hd, rows / 16, causal, mask, stream); break;
    case pkv::kKernelMfma: err = pkv::launch_split_mfma(a, hd, rows / 16, causal, mask, stream); break;
    default: err = pkv::launch_split(a, hd, rows, causal, mask, stream); break;
  }
  return err == hipSuccess ? PKV_OK : PKV_ERR_LAUNCH;
}

// The split kernel, then (several splits without the in-kernel merge) the
// combine kernel.
int launch_all(const pkv::DecodeArgs &a, const pkv_problem *p, float *o_part, void *out_bf16, float *out_f32,
               hipStream_t stream) {
  int rc = launch_plan(a, p, stream);
  if (rc) return rc;
  if (a.S > 1 && !a.fused) {
    pkv::CombineArgs c = {};
    c.o_part = o_part;
    c.ml_part = a.ml_part;
    c.out = static_cast<uint16_t *>(out_bf16);
    c.out_f32 = out_f32;
    c.rows = a.rows;
    c.S = a.S;
    if (pkv::launch_combine(c, p->head_dim, stream) != hipSuccess) return PKV_ERR_LAUNCH;
  }
  return PKV_OK;
}

}  // namespace

extern "C" {

int pkv_paged_decode(const pkv_problem *p, const void *q, const void *k_cache,
                     const void *v_cache, const int32_t *block_table,
                     const int32_t *kv_lens, const int32_t *causal_offsets,
                     const float *mask, float *o_part, size_t o_part_bytes,
                     float *ml_part, size_t ml_part_bytes, void *out_bf16,
                     float *out_f32, hipStream_t stream) {
  int rc = check_problem(p);
  if (rc) return rc;
  if (p->batch == 0) return PKV_OK;
  pkv::DecodeArgs a;
  rc = plan_decode(p, q, QSource{nullptr, (int64_t)p->batch * p->q_len}, KvSource{k_cache, v_cache, block_table, 0, 0},
                   kv_lens, causal_offsets, mask, o_part, o_part_bytes, ml_part, ml_part_bytes, out_bf16, out_f32,
                   false, &a);
  if (rc) return rc;
  return launch_all(a, p, o_part, out_bf16, out_f32, stream);
}

int pkv_paged_decode_noalloc(const pkv_problem *p, const void *q, const void *k_cache, const void *v_cache,
                             const int32_t *block_table, const int32_t *kv_lens, const int32_t *causal_offsets,
                             const float *mask, void *out_bf16, float *out_f32, hipStream_t stream) {
  int rc = check_problem(p);
  if (rc) return rc;
  if (p->batch == 0) return PKV_OK;
  // the split count (the workspace size follows from it)
  int S = p->num_splits;
  if (S == 0) {
    int cus = 0;
    rc = query_cus(&cus);
    if (rc) return rc;
    S = plan_of(p, 0, cus).S;
  }
  // the static workspace: ml_part (counter head + (m, l)) first, then o_part
  size_t ob = 0, mb = 0, mb_al = 0;
  if (S > 1) {
    const size_t rows = (size_t)p->batch * p->q_len * p->num_q_heads;
    ob = rows * (size_t)S * (size_t)p->head_dim * sizeof(float);
    mb = ml_bytes_split(p, S);
    mb_al = (mb + 255) & ~(size_t)255;
    if (mb_al > PKV_NOALLOC_SCRATCH_BYTES || ob > PKV_NOALLOC_SCRATCH_BYTES - mb_al) return PKV_ERR_SCRATCH;
  }
  // plan_decode plans from the caller's problem as pkv_paged_decode does (it
  // finds the same split count); forcing S here would change the heads-per-
  // workgroup choice, which depends on whether the split count was forced
  const QSource qs{nullptr, (int64_t)p->batch * p->q_len};
  const KvSource src{k_cache, v_cache, block_table, 0, 0};
  pkv::DecodeArgs a;
  // every argument check first, on a placeholder workspace address (256-byte
  // aligned, never dereferenced): the static array is looked up only for a
  // call that will launch
  char *const placeholder = reinterpret_cast<char *>((uintptr_t)1 << 20);
  float *o_part = S > 1 ? reinterpret_cast<float *>(placeholder + mb_al) : nullptr;
  float *ml_part = S > 1 ? reinterpret_cast<float *>(placeholder) : nullptr;
  rc = plan_decode(p, q, qs, src, kv_lens, causal_offsets, mask, o_part, ob, ml_part, mb, out_bf16, out_f32, false,
                   &a);
  if (rc) return rc;
  bool cleared = true;
  if (S > 1) {
    void *base = nullptr;
    rc = pkv::noalloc_scratch(&base, &cleared);
    if (rc) return rc;
    ml_part = static_cast<float *>(base);
    o_part = reinterpret_cast<float *>(static_cast<char *>(base) + mb_al);
    rc = plan_decode(p, q, qs, src, kv_lens, causal_offsets, mask, o_part, ob, ml_part, mb, out_bf16, out_f32,
                     false, &a);
    if (rc) return rc;
  }
  if (!cleared) {  // first use on this device: zero the merge counters ahead of the kernel
    (void)hipGetLastError();
    if (pkv::launch_zero(ml_part, PKV_COUNTER_BYTES / 4, stream) != hipSuccess) return PKV_ERR_LAUNCH;
    pkv::noalloc_mark_cleared();
  }
  return launch_all(a, p, o_part, out_bf16, out_f32, stream);
}

int pkv_paged_decode_varlen(const pkv_problem *p, const int32_t *cu_q_lens, int64_t total_tokens, const void *q,
                            const void *k_cache, const void *v_cache, const int32_t *block_table,
                            const int32_t *kv_lens, const int32_t *causal_offsets, const float *mask,
                            float *o_part, size_t o_part_bytes, float *ml_part, size_t ml_part_bytes,
                            void *out_bf16, float *out_f32, hipStream_t stream) {
  int rc = check_problem(p);
  if (rc) return rc;
  if (total_tokens < 0 || total_tokens > (int64_t)p->batch * p->q_len) return PKV_ERR_SHAPE;
  if (p->batch == 0 || total_tokens == 0) return PKV_OK;
  if (!cu_q_lens) return PKV_ERR_NULL;
  if (!aligned(cu_q_lens, 4)) return PKV_ERR_ALIGN;
  pkv::DecodeArgs a;
  rc = plan_decode(p, q, QSource{cu_q_lens, total_tokens}, KvSource{k_cache, v_cache, block_table, 0, 0}, kv_lens,
                   causal_offsets, mask, o_part, o_part_bytes, ml_part, ml_part_bytes, out_bf16, out_f32, false,
                   &a);
  if (rc) return rc;
  return launch_all(a, p, o_part, out_bf16, out_f32, stream);
}

int pkv_contiguous_decode(const pkv_problem *p, int kv_layout, int64_t kv_capacity, const void *q,
                          const void *k_cache, const void *v_cache, const int32_t *kv_lens,
                          const int32_t *causal_offsets, const float *mask, float *o_part,
                          size_t o_part_bytes, float *ml_part, size_t ml_part_bytes, void *out_bf16,
                          float *out_f32, hipStream_t stream) {
  if (!p) return PKV_ERR_NULL;
  if (kv_layout != PKV_KV_BLHD && kv_layout != PKV_KV_BHLD) return PKV_ERR_UNSUPPORTED;
  if (kv_capacity < 1 || kv_capacity > PKV_MAX_CONTIGUOUS_KEYS) return PKV_ERR_SHAPE;
  // the paged fields do not apply: check the rest as a problem whose single
  // page per sequence holds kv_capacity keys
  pkv_problem pc = *p;
  pc.page_size = 1;
  pc.num_pages = 0;
  pc.max_pages_per_seq = (int32_t)kv_capacity;
  int rc = check_problem(&pc);
  if (rc) return rc;
  if (pc.batch == 0) return PKV_OK;
  if (pc.max_kv_len == 0) pc.max_kv_len = (int32_t)kv_capacity;
  // K/V element offsets must fit the 64-bit arithmetic of the kernels
  if ((double)pc.batch * (double)kv_capacity * pc.num_kv_heads * pc.head_dim > 9.0e18) return PKV_ERR_SHAPE;
  pkv::DecodeArgs a;
  rc = plan_decode(&pc, q, QSource{nullptr, (int64_t)pc.batch * pc.q_len},
                   KvSource{k_cache, v_cache, nullptr, kv_layout, kv_capacity}, kv_lens, causal_offsets, mask, o_part,
                   o_part_bytes, ml_part, ml_part_bytes, out_bf16, out_f32, false, &a);
  if (rc) return rc;
  return launch_all(a, &pc, o_part, out_bf16, out_f32, stream);
}

int pkv_paged_decode_partials(const pkv_problem *p, const void *q, const void *k_cache,
                              const void *v_cache, const int32_t *block_table,
                              const int32_t *kv_lens, const int32_t *causal_offsets,
                              const float *mask, float *o_part, size_t o_part_bytes,
                              float *ml_part, size_t ml_part_bytes, hipStream_t stream) {
  int rc = check_problem(p);
  if (rc) return rc;
  if (p->batch == 0) return PKV_OK;
  pkv::DecodeArgs a;
  rc = plan_decode(p, q, QSource{nullptr, (int64_t)p->batch * p->q_len}, KvSource{k_cache, v_cache, block_table, 0, 0},
                   kv_lens, causal_offsets, mask, o_part, o_part_bytes, ml_part, ml_part_bytes, nullptr, nullptr, true,
                   &a);
  if (rc) return rc;
  return launch_plan(a, p, stream);
}

int pkv_combine(int64_t rows, int splits, int head_dim, const float *o_part,
                const float *ml_part, void *out_bf16, float *out_f32,
                hipStream_t stream) {
  if (rows < 0 || splits < 1) return PKV_ERR_SHAPE;
  if (splits > PKV_MAX_SPLITS || !supported_dim(head_dim)) return PKV_ERR_UNSUPPORTED;
  if (rows == 0) return PKV_OK;
  if (!o_part || !ml_part || !out_bf16) return PKV_ERR_NULL;
  if (!aligned(o_part, 16) || !aligned(ml_part, 8) || !aligned(out_bf16, 16) ||
      (out_f32 && !aligned(out_f32, 16)))
    return PKV_ERR_ALIGN;
  if (ceil_div(rows, 2) > kMaxBlocks) return PKV_ERR_SHAPE;  // combine: >= 2 rows per block
  pkv::CombineArgs c = {};
  c.o_part = o_part;
  c.ml_part = ml_part;
  c.out = static_cast<uint16_t *>(out_bf16);
  c.out_f32 = out_f32;
  c.rows = rows;
  c.S = splits;
  (void)hipGetLastError();
  int err = pkv::launch_combine(c, head_dim, stream);
  return err == hipSuccess ? PKV_OK : PKV_ERR_LAUNCH;
}

}  // extern "C"
